// Chunked prefill of the KDA mixer on gfx950: the chunkwise (WY/UT) form of
// the gated delta rule over variable-length sequences.
//
// Source: the KDA prefill kernel and its varlen chunk-index glue ("Kimi K3
// NVFP4 on Rubin (SM107): Modeling V2 target and the runtime it needs",
// section 3); FP32 recurrence with FP32 or BF16 state storage, the state
// stored once at the end ("Extend NVIDIA/TensorRT-LLM#19991 with isolated
// NVFP4 Kimi K3 targets", Description).
//
// Within a chunk of L <= 64 tokens with start state S0, let G_t be the sum of
// log alpha over tokens 0..t of the chunk (per key channel).  The write
// vectors u_t of the token-by-token recurrence satisfy
//     (I + A) U = diag(beta) (V - K_G S0),
//     A_ti = beta_t sum_c kh_tc kh_ic exp(G_tc - G_ic)   (i < t),
// so U = Ut - W S0 with T = (I + A)^-1, Ut = T diag(beta) V and
// W = T diag(beta) (exp(G) * K).  Then
//     O   = (exp(G) * Q) S0 + (P (.) causal) U,
//           P_ti = sum_c qh_tc kh_ic exp(G_tc - G_ic)   (i <= t),
//     S_L = Diag(exp(G_last)) S0 + (exp(G_last - G) * K)^T U.
//
// Three kernels:
//   chunk  (parallel over chunk x head): conv, L2 norms, decay sums, A, P,
//          T, W, Ut and the scaled Q / K, written to the workspace;
//   state  (per sequence x head x 64 value columns, sequential over the
//          sequence's chunks): U, O and the next state on the matrix cores,
//          the state slice held in registers; O is written unnormalised;
//   finish (per token x head): the gated RMSNorm of O, and the ring update
//          with the last three raw tokens of each sequence.
//
// Decay factors.  Every exponential is taken of a sum of log alpha over a
// token range, so its argument is <= 0 and nothing can overflow for any
// alpha in (0, 1].  The sums come from block-local prefix sums over 16-token
// blocks plus whole-block totals, never from the difference of two long
// prefix sums.  Pairs inside one 16-token block are formed elementwise;
// pairs across blocks factor through the first token n of the row block,
//     exp(G_t - G_i) = exp(G_t - G_n) * exp(G_n - G_i)    (i < n <= t),
// both factors <= 1, so those tiles are products on the matrix cores.
// log alpha is clamped at -80 (alpha below 1.8e-35 acts as 1.8e-35; the
// state it scales changes by at most that fraction).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {

constexpr int PC = 64;             // chunk length
constexpr int PB = 16;             // sub-block for the decay factors
constexpr int NB = PC / PB;        // sub-blocks per chunk
constexpr int PD = 128;            // dk = dv handled by the prefill kernels
constexpr int LR = PD + 4;         // padded LDS row of a [PC][PD] tile (floats)
constexpr int LS = PC + 4;         // padded LDS row of a [PC][PC] tile
constexpr float kLogAlphaMin = -80.0f;

// Workspace per (chunk slot, head), in floats.
constexpr int WS_W = 0;                    // W      [PC][PD]
constexpr int WS_U = WS_W + PC * PD;       // Ut     [PC][PD]
constexpr int WS_QG = WS_U + PC * PD;      // exp(G) * qh            [PC][PD]
constexpr int WS_KC = WS_QG + PC * PD;     // exp(G_last - G) * kh   [PC][PD]
constexpr int WS_P = WS_KC + PC * PD;      // P (causal, incl. diagonal) [PC][PC]
constexpr int WS_GAMMA = WS_P + PC * PC;   // exp(G_last)            [PD]
constexpr int WS_PER = WS_GAMMA + PD;

// Chunk slot of chunk c of sequence s: floor(lo / 64) + s + c.  Distinct for
// all (s, c) of monotone cu_seqlens and below ceil(total / 64) + num_seqs.
__device__ __forceinline__ int64_t chunk_slot(int lo, int s, int c) {
    return (int64_t)(lo / PC) + s + c;
}

size_t prefill_workspace_bytes(const kda_shape& sh, int32_t num_seqs, int64_t total_tokens) {
    if (sh.head_k != PD || sh.head_v != PD) return 0;
    const int64_t slots = (total_tokens + PC - 1) / PC + num_seqs;
    return (size_t)slots * sh.num_heads * WS_PER * sizeof(float);
}

struct SeqView {
    int lo, len, slot, pos;
};

// Validates sequence s.  Returns false when it must be skipped; `report`
// selects the one thread in the grid that ORs the status bits.
__device__ __forceinline__ bool seq_view(const PrefillArgs& a, int s, bool report, SeqView& v) {
    const int lo = a.cu_seqlens[s], hi = a.cu_seqlens[s + 1];
    if (!(lo >= 0 && lo <= hi && hi <= a.total_tokens && hi - lo <= a.max_seqlen)) {
        if (report && a.status) atomicOr(a.status, KDA_STATUS_BAD_SEQLENS);
        return false;
    }
    const int slot = a.slot_ids[s];
    if (slot < 0) return false;
    if (slot >= a.num_slots) {
        if (report && a.status) atomicOr(a.status, KDA_STATUS_BAD_SLOT);
        return false;
    }
    const int pos = a.positions[s];
    if (pos < 0) {
        if (report && a.status) atomicOr(a.status, KDA_STATUS_BAD_POSITION);
        return false;
    }
    v = SeqView{lo, hi - lo, slot, pos};
    return true;
}

// Raw activation of history token `lt` (local index within the sequence,
// may be negative) for channel `ch` of the q|k|v layout: the packed input for
// lt >= 0, the ring for earlier positions >= 0, else zero.
template <int ACT>
__device__ __forceinline__ float hist_raw(const PrefillArgs& a, const SeqView& v, int h,
                                          int lt, const void* src, int src_dim, int src_ch,
                                          int ring_ch) {
    constexpr int C = 3 * PD;
    if (lt >= 0) return ld_act<ACT>(src, ((int64_t)(v.lo + lt) * a.H + h) * src_dim + src_ch);
    const int p = v.pos + lt;
    if (p < 0) return 0.f;
    return ld_act<ACT>(a.ring,
                       (((int64_t)v.slot * kConvW + (p & (kConvW - 1))) * a.H + h) * C + ring_ch);
}

// ---------------------------------------------------------------- chunk

template <int ACT>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(PrefillArgs a, int cps) {
    __shared__ float Qn[PC][LR];       // normalised q, later the conv of v
    __shared__ float Kn[PC][LR];       // normalised k
    __shared__ float Gb[PC][LR];       // block-local prefix sums of log alpha
    __shared__ float Am[PC][LS];       // beta_t * (K K^T decayed), strictly lower
    __shared__ float Pm[PC][LS];       // (Q K^T decayed), lower incl. diagonal
    __shared__ float Tm[PC][LS];       // (I + A)^-1
    __shared__ float Bt[NB][PD];       // block totals of log alpha
    __shared__ float bet[PC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int H = a.H;
    const int h = blockIdx.y;
    const int s = blockIdx.x / cps, cc = blockIdx.x % cps;
    SeqView v;
    if (!seq_view(a, s, cc == 0 && h == 0 && tid == 0, v)) return;
    const int t0 = cc * PC;
    if (t0 >= v.len) return;
    const int L = min(PC, v.len - t0);
    float* ws = static_cast<float*>(a.workspace) +
                ((size_t)chunk_slot(v.lo, s, cc) * H + h) * WS_PER;

    // zero A, P (upper parts and unused tiles stay zero)
    for (int e = tid; e < PC * LS; e += 256) {
        (&Am[0][0])[e] = 0.f;
        (&Pm[0][0])[e] = 0.f;
    }

    // ---- 1. conv of q (threads 0..127) and k (128..255), one channel each
    {
        const int ch = tid & (PD - 1);
        const bool isk = tid >= PD;
        const void* src = isk ? a.k : a.q;
        const float4 w4 = *reinterpret_cast<const float4*>(
            (isk ? a.wk : a.wq) + ((size_t)h * PD + ch) * kConvW);
        const int ring_ch = (isk ? PD : 0) + ch;
        float x0 = hist_raw<ACT>(a, v, h, t0 - 3, src, PD, ch, ring_ch);
        float x1 = hist_raw<ACT>(a, v, h, t0 - 2, src, PD, ch, ring_ch);
        float x2 = hist_raw<ACT>(a, v, h, t0 - 1, src, PD, ch, ring_ch);
        float (*dst)[LR] = isk ? Kn : Qn;
#pragma unroll 16
        for (int t = 0; t < PC; ++t) {
            const float x3 =
                t < L ? ld_act<ACT>(src, ((int64_t)(v.lo + t0 + t) * H + h) * PD + ch) : 0.f;
            float c = w4.x * x0;
            c = fmaf(w4.y, x1, c);
            c = fmaf(w4.z, x2, c);
            c = fmaf(w4.w, x3, c);
            dst[t][ch] = t < L ? c : 0.f;
            x0 = x1;
            x1 = x2;
            x2 = x3;
        }
    }
    // ---- decay sums (threads 0..127) and beta (threads 128..191)
    if (tid < PD) {
        const int ch = tid;
        float run = 0.f;
        for (int t = 0; t < PC; ++t) {
            if ((t % PB) == 0) run = 0.f;
            float lg = 0.f;
            if (t < L) {
                const float al = ld_act<ACT>(a.alpha, ((int64_t)(v.lo + t0 + t) * H + h) * PD + ch);
                lg = fmaxf(logf(al), kLogAlphaMin);
            }
            run += lg;
            Gb[t][ch] = run;
            if ((t % PB) == PB - 1) Bt[t / PB][ch] = run;
        }
    } else if (tid < PD + PC) {
        const int t = tid - PD;
        bet[t] = t < L ? ld_act<ACT>(a.beta, (int64_t)(v.lo + t0 + t) * H + h) : 0.f;
    }
    __syncthreads();

    // ---- 2. L2 norms: wave w normalises tokens 16w..16w+15
    for (int tl = 0; tl < PB; ++tl) {
        const int t = wave * PB + tl;
        const float q0 = Qn[t][lane], q1 = Qn[t][lane + 64];
        const float k0 = Kn[t][lane], k1 = Kn[t][lane + 64];
        const float sq = wave_sum(q0 * q0 + q1 * q1);
        const float sk = wave_sum(k0 * k0 + k1 * k1);
        const float rq = a.q_scale / sqrtf(sq + a.l2_eps);
        const float rk = 1.0f / sqrtf(sk + a.l2_eps);
        Qn[t][lane] = q0 * rq;
        Qn[t][lane + 64] = q1 * rq;
        Kn[t][lane] = k0 * rk;
        Kn[t][lane + 64] = k1 * rk;
    }
    __syncthreads();

    // ---- 3. scaled q and k for the state pass, and exp(G_last)
    for (int e = tid; e < PC * PD; e += 256) {
        const int t = e / PD, c = e % PD, bt = t / PB;
        float before = 0.f, after = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < bt) before += Bt[b][c];
            if (b > bt) after += Bt[b][c];
        }
        const float gpre = before + Gb[t][c];                 // G_t
        const float gsuf = (Bt[bt][c] - Gb[t][c]) + after;    // G_last - G_t
        ws[WS_QG + e] = Qn[t][c] * expf(gpre);
        ws[WS_KC + e] = Kn[t][c] * expf(gsuf);
    }
    if (tid < PD) {
        float tot = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) tot += Bt[b][tid];
        ws[WS_GAMMA + tid] = expf(tot);
    }

    // ---- 4a. diagonal 16-token blocks, elementwise: wave w owns block w
    {
        const int base = wave * PB;
        for (int p = lane; p < PB * (PB + 1) / 2; p += 64) {
            int tl = 0;
            while ((tl + 1) * (tl + 2) / 2 <= p) ++tl;
            const int il = p - tl * (tl + 1) / 2;
            const int t = base + tl, i = base + il;
            float sa = 0.f, sp = 0.f;
            for (int c = 0; c < PD; ++c) {
                const float e = expf(Gb[t][c] - Gb[i][c]);
                const float ki = Kn[i][c] * e;
                sa = fmaf(Kn[t][c], ki, sa);
                sp = fmaf(Qn[t][c], ki, sp);
            }
            Am[t][i] = il < tl ? bet[t] * sa : 0.f;
            Pm[t][i] = sp;
        }
    }
    // ---- 4b. tiles below the diagonal on the matrix cores: wave w owns row
    // block w; reference n0 = 16w (first token of the row block)
    if (wave > 0) {
        const int n0 = wave * PB;
        const int t = n0 + n;                     // A-operand row of this lane
        SplitOp kl[4], ql[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float xk[8], xq[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int c = 32 * kb + 8 * g + q;
                const float e = expf(Gb[t][c] - Gb[n0][c]);
                xk[q] = Kn[t][c] * e;
                xq[q] = Qn[t][c] * e;
            }
            kl[kb] = split_op(xk);
            ql[kb] = split_op(xq);
        }
        for (int bi = 0; bi < wave; ++bi) {
            const int i = bi * PB + n;            // B-operand column of this lane
            f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accP = accA;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float xr[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int c = 32 * kb + 8 * g + q;
                    float r = Bt[bi][c] - Gb[i][c];
                    for (int b = bi + 1; b < wave; ++b) r += Bt[b][c];
                    r += Gb[n0][c];
                    xr[q] = Kn[i][c] * expf(r);
                }
                const SplitOp kr = split_op(xr);
                accA = mma3(kl[kb], kr, accA);
                accP = mma3(ql[kb], kr, accP);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = n0 + 4 * g + r;
                Am[tr][bi * PB + n] = bet[tr] * accA[r];
                Pm[tr][bi * PB + n] = accP[r];
            }
        }
    }
    __syncthreads();

    // ---- 5. wave 0: T = (I + A)^-1, lane i owns column i (forward
    // substitution); waves 1..3: conv of v into Qn, and P to the workspace
    if (wave == 0) {
        const int i = lane;
        float x[PC];
#pragma unroll
        for (int t = 0; t < PC; ++t) x[t] = 0.f;
#pragma unroll
        for (int t = 0; t < PC; ++t) {
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int s4 = 0; s4 < t; s4 += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(&Am[t][s4]);
                a0 = fmaf(a4.x, x[s4], a0);
                a1 = fmaf(a4.y, x[s4 + 1], a1);
                a2 = fmaf(a4.z, x[s4 + 2], a2);
                a3 = fmaf(a4.w, x[s4 + 3], a3);
            }
            const float acc = (a0 + a1) + (a2 + a3);
            x[t] = t < i ? 0.f : (t == i ? 1.f : -acc);
        }
#pragma unroll
        for (int t = 0; t < PC; ++t) Tm[t][i] = x[t];
    } else {
        const int ch = tid - 64;                  // 0..191
        if (ch < PD) {
            const float4 w4 =
                *reinterpret_cast<const float4*>(a.wv + ((size_t)h * PD + ch) * kConvW);
            const int ring_ch = 2 * PD + ch;
            float x0 = hist_raw<ACT>(a, v, h, t0 - 3, a.v, PD, ch, ring_ch);
            float x1 = hist_raw<ACT>(a, v, h, t0 - 2, a.v, PD, ch, ring_ch);
            float x2 = hist_raw<ACT>(a, v, h, t0 - 1, a.v, PD, ch, ring_ch);
#pragma unroll 16
            for (int t = 0; t < PC; ++t) {
                const float x3 =
                    t < L ? ld_act<ACT>(a.v, ((int64_t)(v.lo + t0 + t) * H + h) * PD + ch) : 0.f;
                float c = w4.x * x0;
                c = fmaf(w4.y, x1, c);
                c = fmaf(w4.z, x2, c);
                c = fmaf(w4.w, x3, c);
                Qn[t][ch] = t < L ? c : 0.f;
                x0 = x1;
                x1 = x2;
                x2 = x3;
            }
        }
        for (int e = tid - 64; e < PC * PC; e += 192) {
            const int t = e / PC, i = e % PC;
            ws[WS_P + e] = Pm[t][i];
        }
    }
    __syncthreads();

    // ---- 6. W = T diag(beta) (exp(G) * K) and Ut = T diag(beta) V on the
    // matrix cores: wave w owns value/key columns 32w..32w+31
    {
        SplitOp ta[4][2];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float x[8];
                const int t = 16 * tt + n;
#pragma unroll
                for (int q = 0; q < 8; ++q) x[q] = Tm[t][32 * kb + 8 * g + q];
                ta[tt][kb] = split_op(x);
            }
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            const int c = 32 * wave + 16 * cl + n;   // B-operand column of this lane
            f32x4_t accW[4], accU[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                accW[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                accU[tt] = accW[tt];
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float xw[8], xu[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int i = 32 * kb + 8 * g + q, bi = i / PB;
                    float gpre = Gb[i][c];
                    for (int b = 0; b < bi; ++b) gpre += Bt[b][c];
                    xw[q] = bet[i] * Kn[i][c] * expf(gpre);
                    xu[q] = bet[i] * Qn[i][c];
                }
                const SplitOp bw = split_op(xw), bu = split_op(xu);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    if (32 * kb > 16 * tt + 15) continue;   // T is lower triangular
                    accW[tt] = mma3(ta[tt][kb], bw, accW[tt]);
                    accU[tt] = mma3(ta[tt][kb], bu, accU[tt]);
                }
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tt + 4 * g + r;
                    ws[WS_W + t * PD + c] = accW[tt][r];
                    ws[WS_U + t * PD + c] = accU[tt][r];
                }
        }
    }
}

// ---------------------------------------------------------------- state

template <int ST>
__global__ __launch_bounds__(256) void prefill_state_kernel(PrefillArgs a) {
    __shared__ float Ws[PC][LR];
    __shared__ float Qs[PC][LR];
    __shared__ float Ks[PC][LR];
    __shared__ float Ps[PC][LS];
    __shared__ float gam[PD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int H = a.H;
    const int half = blockIdx.x & 1;
    const int sh = blockIdx.x >> 1;
    const int h = sh % H, s = sh / H;
    SeqView v;
    if (!seq_view(a, s, false, v)) return;
    if (v.len == 0) return;
    const int j0 = 64 * half + 16 * wave;          // this wave's value columns
    const size_t head_off = ((size_t)v.slot * H + h) * PD * PD;

    // state slice S[c][j0 + n], c = 16 ct + 4 g + r, in the D-tile layout
    f32x4_t S[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x = 0.f;
            if (v.pos > 0) {
                const size_t e = head_off + (size_t)(16 * ct + 4 * g + r) * PD + j0 + n;
                x = ST == kF32 ? static_cast<const float*>(a.pool)[e]
                               : bf16_to_f32(static_cast<const uint16_t*>(a.pool)[e]);
            }
            S[ct][r] = x;
        }

    // The next chunk's operands are loaded into registers while the current
    // chunk computes, then written to LDS after the step's barrier: one
    // memory round trip per chunk, hidden behind the previous chunk's work.
    constexpr int NF4 = PC * PD / 4 / 256;        // float4 per thread per [PC][PD] tile
    constexpr int NP4 = PC * PC / 4 / 256;        // float4 per thread for P
    float4 fw[NF4], fq[NF4], fk[NF4], fp[NP4];
    float fu[16], fg = 0.f;
    auto fetch = [&](int cc) {
        const float* ws = static_cast<const float*>(a.workspace) +
                          ((size_t)chunk_slot(v.lo, s, cc) * H + h) * WS_PER;
#pragma unroll
        for (int k = 0; k < NF4; ++k) {
            const int e4 = tid + 256 * k;
            const int t = e4 / (PD / 4), c = 4 * (e4 % (PD / 4));
            fw[k] = *reinterpret_cast<const float4*>(ws + WS_W + t * PD + c);
            fq[k] = *reinterpret_cast<const float4*>(ws + WS_QG + t * PD + c);
            fk[k] = *reinterpret_cast<const float4*>(ws + WS_KC + t * PD + c);
        }
#pragma unroll
        for (int k = 0; k < NP4; ++k) {
            const int e4 = tid + 256 * k;
            const int t = e4 / (PC / 4), i = 4 * (e4 % (PC / 4));
            fp[k] = *reinterpret_cast<const float4*>(ws + WS_P + t * PC + i);
        }
        if (tid < PD) fg = ws[WS_GAMMA + tid];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                fu[4 * tt + r] = ws[WS_U + (16 * tt + 4 * g + r) * PD + j0 + n];
    };

    const int nch = (v.len + PC - 1) / PC;
    fetch(0);
    for (int cc = 0; cc < nch; ++cc) {
        const int L = min(PC, v.len - cc * PC);
        __syncthreads();                           // the previous chunk's LDS reads are done
#pragma unroll
        for (int k = 0; k < NF4; ++k) {
            const int e4 = tid + 256 * k;
            const int t = e4 / (PD / 4), c = 4 * (e4 % (PD / 4));
            *reinterpret_cast<float4*>(&Ws[t][c]) = fw[k];
            *reinterpret_cast<float4*>(&Qs[t][c]) = fq[k];
            *reinterpret_cast<float4*>(&Ks[t][c]) = fk[k];
        }
#pragma unroll
        for (int k = 0; k < NP4; ++k) {
            const int e4 = tid + 256 * k;
            const int t = e4 / (PC / 4), i = 4 * (e4 % (PC / 4));
            *reinterpret_cast<float4*>(&Ps[t][i]) = fp[k];
        }
        if (tid < PD) gam[tid] = fg;
        f32x4_t U[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) U[tt][r] = fu[4 * tt + r];
        if (cc + 1 < nch) fetch(cc + 1);
        __syncthreads();

        // S as the B operand (k = key channel), stacked D-tile pairing
        SplitOp sb[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float x[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[q] = S[2 * kb][q];
                x[4 + q] = S[2 * kb + 1][q];
            }
            sb[kb] = split_op(x);
        }
        // U = Ut - W S
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 16 * tt + n;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const float4 lo4 = *reinterpret_cast<const float4*>(&Ws[t][32 * kb + 4 * g]);
                const float4 hi4 = *reinterpret_cast<const float4*>(&Ws[t][32 * kb + 16 + 4 * g]);
                float x[8] = {-lo4.x, -lo4.y, -lo4.z, -lo4.w, -hi4.x, -hi4.y, -hi4.z, -hi4.w};
                U[tt] = mma3(split_op(x), sb[kb], U[tt]);
            }
        }
        // U as the B operand (k = token), stacked D-tile pairing
        SplitOp ub[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float x[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[q] = U[2 * kb][q];
                x[4 + q] = U[2 * kb + 1][q];
            }
            ub[kb] = split_op(x);
        }
        // O = (exp(G) * Q) S + P U, written unnormalised into y
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 16 * tt + n;
            f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const float4 lo4 = *reinterpret_cast<const float4*>(&Qs[t][32 * kb + 4 * g]);
                const float4 hi4 = *reinterpret_cast<const float4*>(&Qs[t][32 * kb + 16 + 4 * g]);
                float x[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
                o = mma3(split_op(x), sb[kb], o);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb > 16 * tt + 15) continue;       // P is causal
                const float4 lo4 = *reinterpret_cast<const float4*>(&Ps[t][32 * kb + 4 * g]);
                const float4 hi4 = *reinterpret_cast<const float4*>(&Ps[t][32 * kb + 16 + 4 * g]);
                float x[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
                o = mma3(split_op(x), ub[kb], o);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * tt + 4 * g + r;
                if (tr < L)
                    a.y[((int64_t)(v.lo + cc * PC + tr) * H + h) * PD + j0 + n] = o[r];
            }
        }
        // S <- Diag(exp(G_last)) S + (exp(G_last - G) * K)^T U
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            f32x4_t acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gam[16 * ct + 4 * g + r] * S[ct][r];
            const int c = 16 * ct + n;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float x[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) x[q] = Ks[32 * kb + kslot(g, q)][c];
                acc = mma3(split_op(x), ub[kb], acc);
            }
            S[ct] = acc;
        }
    }

    // typed store of the final state, once
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t e = head_off + (size_t)(16 * ct + 4 * g + r) * PD + j0 + n;
            if (ST == kF32)
                static_cast<float*>(a.pool)[e] = S[ct][r];
            else
                static_cast<uint16_t*>(a.pool)[e] = (uint16_t)f32_to_bf16_rne(S[ct][r]);
        }
}

// ---------------------------------------------------------------- finish

// Gated RMSNorm of O (one wave per token and head), and in the first
// workgroup of each (sequence, head) the ring update with the sequence's
// last min(3, len) raw tokens.
template <int ACT>
__global__ __launch_bounds__(256) void prefill_finish_kernel(PrefillArgs a, int tpb) {
    constexpr int C = 3 * PD;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H;
    const int h = blockIdx.y;
    const int s = blockIdx.x / tpb, blk = blockIdx.x % tpb;
    SeqView v;
    if (!seq_view(a, s, false, v)) return;
    if (blk == 0) {
        const int pend = v.pos + v.len;
        const int pfirst = max(v.pos, pend - (kConvW - 1));
        for (int p = pfirst; p < pend; ++p) {
            const int64_t row = v.lo + (p - v.pos);
            const int64_t dst = (((int64_t)v.slot * kConvW + (p & (kConvW - 1))) * H + h) * C;
            for (int ch = tid; ch < C; ch += 256) {
                const void* src = ch < PD ? a.q : (ch < 2 * PD ? a.k : a.v);
                const int sc = ch % PD;
                st_act_bits<ACT>(a.ring, dst + ch, ld_act_bits<ACT>(src, (row * H + h) * PD + sc));
            }
        }
    }
    const int t = blk * 4 + wave;
    if (t >= v.len) return;
    const int64_t row = v.lo + t;
    float* y = a.y + (row * H + h) * PD;
    const float o0 = y[lane], o1 = y[lane + 64];
    const float ms = wave_sum(o0 * o0 + o1 * o1);
    const float rr = 1.0f / sqrtf(ms / (float)PD + a.norm_eps);
    const float w0 = a.norm_w ? a.norm_w[lane] : 1.0f;
    const float w1 = a.norm_w ? a.norm_w[lane + 64] : 1.0f;
    const float g0 = ld_act<ACT>(a.g, (row * H + h) * PD + lane);
    const float g1 = ld_act<ACT>(a.g, (row * H + h) * PD + lane + 64);
    y[lane] = w0 * (o0 * rr) * gate_fn(a.gate, g0);
    y[lane + 64] = w1 * (o1 * rr) * gate_fn(a.gate, g1);
}

template <int ACT, int ST>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    const int cps = (a.max_seqlen + PC - 1) / PC;
    const int tpb = (a.max_seqlen + 3) / 4;
    hipLaunchKernelGGL((prefill_chunk_kernel<ACT>), dim3((unsigned)a.num_seqs * cps, a.H),
                       dim3(256), 0, stream, a, cps);
    hipLaunchKernelGGL((prefill_state_kernel<ST>), dim3((unsigned)a.num_seqs * a.H * 2),
                       dim3(256), 0, stream, a);
    hipLaunchKernelGGL((prefill_finish_kernel<ACT>), dim3((unsigned)a.num_seqs * tpb, a.H),
                       dim3(256), 0, stream, a, tpb);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int launch_prefill(const kda_shape& s, const PrefillArgs& a, hipStream_t stream) {
    if (s.head_k != PD || s.head_v != PD) return KDA_ERR_UNSUPPORTED;
    if (s.act_dtype == kF32 && s.state_dtype == kF32) return launch_prefill_t<kF32, kF32>(a, stream);
    if (s.act_dtype == kF32 && s.state_dtype == kBF16) return launch_prefill_t<kF32, kBF16>(a, stream);
    if (s.act_dtype == kBF16 && s.state_dtype == kF32) return launch_prefill_t<kBF16, kF32>(a, stream);
    return launch_prefill_t<kBF16, kBF16>(a, stream);
}

}  // namespace kda
