// KDA decode and speculative verify on gfx950: one per-token kernel.
//
// One workgroup owns one (row, head) and its whole dk x dv state.  The state
// streams in once with 128-bit loads, stays in VGPRs across every token of
// the call, and streams out once (decode: the typed pool store; verify: one
// FP32 record per draft token).  Sources: the one-token KDA decode kernel
// and the speculative verify kernels with per-token verify states ("Kimi K3
// on modeling_v2: stateful catalog entries, ...", sections 5 and 6 and the
// manual 16-rank runs); FP32 recurrence, FP32 draft records under either
// storage dtype, explicit FP32 loads and typed state stores ("Extend
// NVIDIA/TensorRT-LLM#19991 with isolated NVFP4 Kimi K3 targets",
// Description).
//
// Per token, with S the state before the token (rows = key channels i):
//   c        = causal conv of the raw q | k | v channels (4 taps)
//   qh, kh   = L2-normalised c_q (times q_scale), c_k;   vt = c_v
//   u        = S^T (alpha * kh)            = (Diag(alpha) S)^T kh
//   o'       = S^T (alpha * qh)
//   delta    = beta (vt - u)
//   S'       = Diag(alpha) S + kh delta^T  = (I - beta kh kh^T) Diag(alpha) S
//                                            + beta kh vt^T
//   o        = S'^T qh = o' + (kh . qh) delta
//   y        = norm_w * o / sqrt(mean(o^2) + eps) * gate(g)
// so a single pass over S serves both dk-reductions.
//
// Thread map: the physical state of a head is [dv][dk] (dk contiguous).  A
// thread owns VEC consecutive dk entries (16 bytes of storage) of PASSES
// rows j = r + ROWS * p.  LANES = dk / VEC lanes cover one row, and the two
// dk-reductions of all PASSES rows (2 * PASSES == LANES values per lane) are
// finished with one recursive-halving shuffle pass per lane group, which
// leaves lane i of the group holding reduced value i.  Workgroup size is
// 2 * dv threads, so every reduction, load and store is fixed in order and
// the result is bitwise reproducible.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV, int VEC>
struct TileMap {
    static constexpr int LANES = DK / VEC;      // lanes per state row
    static constexpr int NT = 2 * DV;           // threads per workgroup
    static constexpr int ROWS = NT / LANES;     // rows per pass
    static constexpr int PASSES = DV / ROWS;    // rows per thread
    static_assert(2 * PASSES == LANES, "reduction needs 2*PASSES == LANES");
    static_assert(kWave % LANES == 0, "lane groups must tile a wave");
    static_assert(NT >= DK + DV, "conv needs one thread per q/k and v channel");
};

// Load the thread's state slice as raw 128-bit words (issued early).
template <int ST, int DK, int PASSES, int ROWS, int VEC>
__device__ __forceinline__ void load_state_raw(const void* head_base, int r,
                                               int l, uint4 (&raw)[PASSES]) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int j = r + ROWS * p;
        if constexpr (ST == kF32) {
            raw[p] = *reinterpret_cast<const uint4*>(
                static_cast<const float*>(head_base) + j * DK + l * VEC);
        } else {
            raw[p] = *reinterpret_cast<const uint4*>(
                static_cast<const uint16_t*>(head_base) + j * DK + l * VEC);
        }
    }
}

template <int ST, int PASSES, int VEC>
__device__ __forceinline__ void unpack_state(const uint4 (&raw)[PASSES],
                                             float (&s)[PASSES][VEC]) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const uint32_t w[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
        if constexpr (ST == kF32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[p][e] = __uint_as_float(w[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[p][2 * e] = bf16_to_f32(w[e] & 0xffffu);
                s[p][2 * e + 1] = bf16_to_f32(w[e] >> 16);
            }
        }
    }
}

// Typed store of the thread's state slice into [dv][dk] storage.
template <int ST, int DK, int PASSES, int ROWS, int VEC>
__device__ __forceinline__ void store_state(void* head_base, int r, int l,
                                            const float (&s)[PASSES][VEC]) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int j = r + ROWS * p;
        if constexpr (ST == kF32) {
            float4 x = make_float4(s[p][0], s[p][1], s[p][2], s[p][3]);
            *reinterpret_cast<float4*>(static_cast<float*>(head_base) + j * DK +
                                       l * VEC) = x;
        } else {
            uint4 x;
            x.x = f32_to_bf16_rne(s[p][0]) | (f32_to_bf16_rne(s[p][1]) << 16);
            x.y = f32_to_bf16_rne(s[p][2]) | (f32_to_bf16_rne(s[p][3]) << 16);
            x.z = f32_to_bf16_rne(s[p][4]) | (f32_to_bf16_rne(s[p][5]) << 16);
            x.w = f32_to_bf16_rne(s[p][6]) | (f32_to_bf16_rne(s[p][7]) << 16);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(head_base) + j * DK +
                                      l * VEC) = x;
        }
    }
}

// FP32 record store, [dv][dk] like the pool.
template <int DK, int PASSES, int ROWS, int VEC>
__device__ __forceinline__ void store_record(float* rec, int r, int l,
                                             const float (&s)[PASSES][VEC]) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int j = r + ROWS * p;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            *reinterpret_cast<float4*>(rec + j * DK + l * VEC + e) =
                make_float4(s[p][e], s[p][e + 1], s[p][e + 2], s[p][e + 3]);
        }
    }
}

// Phase A of a token: the causal conv of this thread's channels (t < DK: q
// and k channel t; DK <= t < DK + DV: v channel t - DK) into conv_s, and the
// raw token copied to the ring (decode, entry pos mod 4) or to draft_conv
// (verify).  Conv taps 0..2 read the three previous raw tokens (earlier
// drafts, else the ring, else zero before position 0), tap 3 the current.
template <int DK, int DV, int ACT, bool VERIFY>
__device__ __forceinline__ void conv_token(const TokenArgs& a, int b, int h, int t, int n,
                                       int slot, int pos, float4 wq4, float4 wk4,
                                       float4 wv4, float* conv_s, float (*red_s)[4],
                                       float& cq, float& ck) {
    constexpr int C = 2 * DK + DV;
    const int tid = threadIdx.x;
    const int H = a.H;
    const bool has_qk = tid < DK;
    const bool has_v = tid >= DK && tid < DK + DV;
    const size_t ring_slot = (size_t)slot * kConvW;  // ring [slot][4][H][C]
    const int64_t tok = (int64_t)b * n + t;
    const int wave = tid / kWave;
    float cv = 0.f;
    cq = 0.f;
    ck = 0.f;
    if (has_qk || has_v) {
        const int ch_q = tid, ch_k = DK + tid, ch_v = 2 * DK + (tid - DK);
        float hq[kConvW], hk[kConvW], hv[kConvW];
#pragma unroll
        for (int j = 0; j < kConvW; ++j) {
            const int rel = t - (kConvW - 1) + j;   // draft-token index
            float xq = 0.f, xk = 0.f, xv = 0.f;
            if (rel >= 0) {
                if (has_qk) {
                    xq = ld_act<ACT>(a.q, ((int64_t)b * n + rel) * H * DK + h * DK + tid);
                    xk = ld_act<ACT>(a.k, ((int64_t)b * n + rel) * H * DK + h * DK + tid);
                } else {
                    xv = ld_act<ACT>(a.v, ((int64_t)b * n + rel) * H * DV + h * DV + (tid - DK));
                }
            } else if (pos + rel >= 0) {
                const size_t e = ring_slot + ((pos + rel) & (kConvW - 1));
                const int64_t base = ((int64_t)e * H + h) * C;
                if (has_qk) {
                    xq = ld_act<ACT>(a.ring, base + ch_q);
                    xk = ld_act<ACT>(a.ring, base + ch_k);
                } else {
                    xv = ld_act<ACT>(a.ring, base + ch_v);
                }
            }
            hq[j] = xq; hk[j] = xk; hv[j] = xv;
        }
        if (has_qk) {
            cq = wq4.x * hq[0]; cq = fmaf(wq4.y, hq[1], cq);
            cq = fmaf(wq4.z, hq[2], cq); cq = fmaf(wq4.w, hq[3], cq);
            ck = wk4.x * hk[0]; ck = fmaf(wk4.y, hk[1], ck);
            ck = fmaf(wk4.z, hk[2], ck); ck = fmaf(wk4.w, hk[3], ck);
            conv_s[ch_q] = cq;
            conv_s[ch_k] = ck;
        } else {
            cv = wv4.x * hv[0]; cv = fmaf(wv4.y, hv[1], cv);
            cv = fmaf(wv4.z, hv[2], cv); cv = fmaf(wv4.w, hv[3], cv);
            conv_s[ch_v] = cv;
        }
        // keep the raw token: decode -> ring entry pos mod 4,
        // verify -> draft_conv[b, t, h, :]
        if constexpr (!VERIFY) {
            const int64_t base = ((int64_t)(ring_slot + (pos & (kConvW - 1))) * H + h) * C;
            if (has_qk) {
                cp_act<ACT>(a.ring, base + ch_q, a.q, tok * H * DK + h * DK + tid);
                cp_act<ACT>(a.ring, base + ch_k, a.k, tok * H * DK + h * DK + tid);
            } else {
                cp_act<ACT>(a.ring, base + ch_v, a.v, tok * H * DV + h * DV + (tid - DK));
            }
        } else {
            const int64_t base = (tok * H + h) * C;
            if (has_qk) {
                cp_act<ACT>(a.draft_conv, base + ch_q, a.q, tok * H * DK + h * DK + tid);
                cp_act<ACT>(a.draft_conv, base + ch_k, a.k, tok * H * DK + h * DK + tid);
            } else {
                cp_act<ACT>(a.draft_conv, base + ch_v, a.v, tok * H * DV + h * DV + (tid - DK));
            }
        }
    }
    {
        float sq = cq * cq, sk = ck * ck, sqk = cq * ck;
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        sqk = wave_sum(sqk);
        if ((tid % kWave) == 0) {
            red_s[wave][0] = sq;
            red_s[wave][1] = sk;
            red_s[wave][2] = sqk;
        }
    }
}

template <int DK, int DV, int ACT, int ST, bool VERIFY>
__global__ __launch_bounds__(2 * DV) void token_kernel(TokenArgs a) {
    constexpr int VEC = (ST == kF32) ? 4 : 8;
    using M = TileMap<DK, DV, VEC>;
    constexpr int LANES = M::LANES, ROWS = M::ROWS, PASSES = M::PASSES;
    constexpr int NT = M::NT;
    constexpr int C = 2 * DK + DV;
    constexpr int NW = NT / kWave;

    __shared__ float conv_s[C];      // conv outputs of the token
    __shared__ float delta_s[DV];
    __shared__ float orow_s[DV];     // o' = S^T (alpha * qh)
    __shared__ float red_s[NW][4];

    const int tid = threadIdx.x;
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int b = blockIdx.x / H;
    const int slot = a.slot_ids[b];
    if (slot < 0) return;
    if (slot >= a.num_slots) {
        if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_SLOT);
        return;
    }
    const int pos = a.positions[b];
    if (pos < 0) {
        if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_POSITION);
        return;
    }
    const int n = a.n;
    const int l = tid % LANES;
    const int r = tid / LANES;
    const int wave = tid / kWave;

    // ---- state in: issued first, consumed after the conv ----------------
    const size_t head_elems = (size_t)DV * DK;
    const size_t head_off = ((size_t)slot * H + h) * head_elems;
    uint4 raw[PASSES];
    if (pos > 0) {
        const void* base = (ST == kF32)
            ? static_cast<const void*>(static_cast<const float*>(a.pool) + head_off)
            : static_cast<const void*>(static_cast<const uint16_t*>(a.pool) + head_off);
        load_state_raw<ST, DK, PASSES, ROWS, VEC>(base, r, l, raw);
    } else {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) raw[p] = make_uint4(0, 0, 0, 0);
    }

    // ---- conv taps of this thread's channels
    const bool has_qk = tid < DK;
    const bool has_v = tid >= DK && tid < DK + DV;
    float4 wq4 = make_float4(0, 0, 0, 0), wk4 = wq4, wv4 = wq4;
    if (has_qk) {
        wq4 = *reinterpret_cast<const float4*>(a.wq + ((size_t)h * DK + tid) * kConvW);
        wk4 = *reinterpret_cast<const float4*>(a.wk + ((size_t)h * DK + tid) * kConvW);
    } else if (has_v) {
        wv4 = *reinterpret_cast<const float4*>(a.wv + ((size_t)h * DV + tid - DK) * kConvW);
    }
    const float norm_w = (tid < DV) ? (a.norm_w ? a.norm_w[tid] : 1.0f) : 0.0f;

    float s[PASSES][VEC];
    float cq = 0.f, ck = 0.f;
    // ---------------- A. conv, raw copy, norm partial sums ---------------
    conv_token<DK, DV, ACT, VERIFY>(a, b, h, 0, n, slot, pos, wq4, wk4, wv4, conv_s, red_s,
                                    cq, ck);
    unpack_state<ST, PASSES, VEC>(raw, s);

    for (int t = 0; t < n; ++t) {
        const int64_t tok = (int64_t)b * n + t;     // row of the inputs
        if (t > 0)
            conv_token<DK, DV, ACT, VERIFY>(a, b, h, t, n, slot, pos, wq4, wk4, wv4, conv_s,
                                            red_s, cq, ck);
        // per-thread decay factors for its dk slice (independent of LDS)
        float al[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            al[e] = ld_act<ACT>(a.alpha, tok * H * DK + h * DK + l * VEC + e);
        const float beta = ld_act<ACT>(a.beta, tok * H + h);
        __syncthreads();

        // ---------------- B. normalise, partial dots, reduction ----------
        float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
        for (int w = 0; w < DK / kWave; ++w) {   // q/k channels live in waves 0..DK/64-1
            sq += red_s[w][0];
            sk += red_s[w][1];
            sqk += red_s[w][2];
        }
        const float rq = a.q_scale / sqrtf(sq + a.l2_eps);
        const float rk = 1.0f / sqrtf(sk + a.l2_eps);
        const float kq = sqk * rq * rk;          // kh . qh
        float kh[VEC], akh[VEC], aqh[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int i = l * VEC + e;
            kh[e] = conv_s[DK + i] * rk;
            akh[e] = al[e] * kh[e];
            aqh[e] = al[e] * (conv_s[i] * rq);
        }
        float vals[LANES];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            float u = 0.f, o = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                u = fmaf(s[p][e], akh[e], u);
                o = fmaf(s[p][e], aqh[e], o);
            }
            vals[p] = u;
            vals[PASSES + p] = o;
        }
        const float red = group_transpose_sum<LANES>(vals, l);
        if (l < PASSES) {
            const int j = r + ROWS * l;
            delta_s[j] = beta * (conv_s[2 * DK + j] - red);
        } else {
            const int j = r + ROWS * (l - PASSES);
            orow_s[j] = red;
        }
        __syncthreads();

        // ---------------- C. state update, store, read-out ----------------
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const float d = delta_s[r + ROWS * p];
#pragma unroll
            for (int e = 0; e < VEC; ++e) s[p][e] = fmaf(kh[e], d, s[p][e] * al[e]);
        }
        if constexpr (VERIFY) {
            float* rec = a.records + ((size_t)tok * H + h) * head_elems;
            store_record<DK, PASSES, ROWS, VEC>(rec, r, l, s);
        }
        float o = 0.f;
        if (tid < DV) o = fmaf(kq, delta_s[tid], orow_s[tid]);
        {
            const float ms = wave_sum(o * o);
            if ((tid % kWave) == 0) red_s[wave][3] = ms;
        }
        __syncthreads();

        // ---------------- D. gated RMSNorm -------------------------------
        if (tid < DV) {
            float ms = 0.f;
#pragma unroll
            for (int w = 0; w < DV / kWave; ++w) ms += red_s[w][3];
            const float rr = 1.0f / sqrtf(ms / (float)DV + a.norm_eps);
            const float gv = ld_act<ACT>(a.g, tok * H * DV + h * DV + tid);
            a.y[(tok * H + h) * DV + tid] = norm_w * (o * rr) * gate_fn(a.gate, gv);
        }
        // The next token's first writes (conv_s, red_s[.][0..2]) touch only
        // LDS that every thread finished reading before the second barrier.
    }

    if constexpr (!VERIFY) {
        void* base = (ST == kF32)
            ? static_cast<void*>(static_cast<float*>(a.pool) + head_off)
            : static_cast<void*>(static_cast<uint16_t*>(a.pool) + head_off);
        store_state<ST, DK, PASSES, ROWS, VEC>(base, r, l, s);
    }
}

// Commit: per (row, head), m = accepted[row] in [0, n]; record m-1 -> pool
// (typed store), raw drafts of the last min(m, 4) accepted tokens -> ring.
template <int DK, int DV, int ACT, int ST>
__global__ __launch_bounds__(256) void commit_kernel(CommitArgs a) {
    constexpr int C = 2 * DK + DV;
    const int tid = threadIdx.x;
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int b = blockIdx.x / H;
    const int slot = a.slot_ids[b];
    if (slot < 0) return;
    if (slot >= a.num_slots) {
        if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_SLOT);
        return;
    }
    const int pos = a.positions[b];
    if (pos < 0) {
        if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_POSITION);
        return;
    }
    const int m = a.accepted[b];
    if (m < 0 || m > a.n) {
        if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_ACCEPTED);
        return;
    }
    if (m == 0) return;
    const size_t head_elems = (size_t)DV * DK;
    const float* rec = a.records + (((size_t)b * a.n + (m - 1)) * H + h) * head_elems;
    const size_t head_off = ((size_t)slot * H + h) * head_elems;
    if constexpr (ST == kF32) {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.pool) + head_off);
        const float4* src = reinterpret_cast<const float4*>(rec);
        for (int i = tid; i < (int)(head_elems / 4); i += blockDim.x) dst[i] = src[i];
    } else {
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.pool) + head_off);
        const float4* src = reinterpret_cast<const float4*>(rec);
        for (int i = tid; i < (int)(head_elems / 8); i += blockDim.x) {
            const float4 x0 = src[2 * i], x1 = src[2 * i + 1];
            uint4 o;
            o.x = f32_to_bf16_rne(x0.x) | (f32_to_bf16_rne(x0.y) << 16);
            o.y = f32_to_bf16_rne(x0.z) | (f32_to_bf16_rne(x0.w) << 16);
            o.z = f32_to_bf16_rne(x1.x) | (f32_to_bf16_rne(x1.y) << 16);
            o.w = f32_to_bf16_rne(x1.z) | (f32_to_bf16_rne(x1.w) << 16);
            dst[i] = o;
        }
    }
    const int first = m > kConvW ? m - kConvW : 0;
    for (int t = first; t < m; ++t) {
        const int64_t src = (((int64_t)b * a.n + t) * H + h) * C;
        const int64_t dst = (((int64_t)slot * kConvW + ((pos + t) & (kConvW - 1))) * H + h) * C;
        for (int c = tid; c < C; c += blockDim.x)
            st_act_bits<ACT>(a.ring, dst + c, ld_act_bits<ACT>(a.draft_conv, src + c));
    }
}

template <int DK, int DV, int ACT, int ST>
static int launch_token_t(const TokenArgs& a, int32_t batch, bool verify,
                          hipStream_t stream) {
    const dim3 grid((unsigned)batch * (unsigned)a.H), block(2 * DV);
    if (verify)
        hipLaunchKernelGGL((token_kernel<DK, DV, ACT, ST, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((token_kernel<DK, DV, ACT, ST, false>), grid, block, 0, stream, a);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

template <int DK, int DV>
static int dispatch_token(const kda_shape& s, const TokenArgs& a, int32_t batch,
                          bool verify, hipStream_t stream) {
    if (s.act_dtype == kF32 && s.state_dtype == kF32)
        return launch_token_t<DK, DV, kF32, kF32>(a, batch, verify, stream);
    if (s.act_dtype == kF32 && s.state_dtype == kBF16)
        return launch_token_t<DK, DV, kF32, kBF16>(a, batch, verify, stream);
    if (s.act_dtype == kBF16 && s.state_dtype == kF32)
        return launch_token_t<DK, DV, kBF16, kF32>(a, batch, verify, stream);
    return launch_token_t<DK, DV, kBF16, kBF16>(a, batch, verify, stream);
}

int launch_token(const kda_shape& s, const TokenArgs& a, int32_t batch,
                 bool verify, hipStream_t stream) {
    if (s.head_k == 128 && s.head_v == 128)
        return dispatch_token<128, 128>(s, a, batch, verify, stream);
    if (s.head_k == 64 && s.head_v == 64)
        return dispatch_token<64, 64>(s, a, batch, verify, stream);
    return KDA_ERR_UNSUPPORTED;
}

template <int DK, int DV, int ACT, int ST>
static int launch_commit_t(const CommitArgs& a, int32_t batch, hipStream_t stream) {
    hipLaunchKernelGGL((commit_kernel<DK, DV, ACT, ST>), dim3((unsigned)batch * a.H),
                       dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

template <int DK, int DV>
static int dispatch_commit(const kda_shape& s, const CommitArgs& a, int32_t batch,
                           hipStream_t stream) {
    if (s.act_dtype == kF32 && s.state_dtype == kF32)
        return launch_commit_t<DK, DV, kF32, kF32>(a, batch, stream);
    if (s.act_dtype == kF32 && s.state_dtype == kBF16)
        return launch_commit_t<DK, DV, kF32, kBF16>(a, batch, stream);
    if (s.act_dtype == kBF16 && s.state_dtype == kF32)
        return launch_commit_t<DK, DV, kBF16, kF32>(a, batch, stream);
    return launch_commit_t<DK, DV, kBF16, kBF16>(a, batch, stream);
}

int launch_commit(const kda_shape& s, const CommitArgs& a, int32_t batch,
                  hipStream_t stream) {
    if (s.head_k == 128 && s.head_v == 128)
        return dispatch_commit<128, 128>(s, a, batch, stream);
    if (s.head_k == 64 && s.head_v == 64)
        return dispatch_commit<64, 64>(s, a, batch, stream);
    return KDA_ERR_UNSUPPORTED;
}

}  // namespace kda
