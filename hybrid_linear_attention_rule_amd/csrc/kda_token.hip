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
// Thread map: the state of a head is stored [dk][dv] (dv contiguous).  A
// thread owns VEC consecutive dv entries (16 bytes of storage) of RPT
// consecutive key rows; LJ = dv / VEC lanes span a row and RG = 2 * VEC row
// groups span dk.  The dk-reductions run in-thread over the thread's RPT
// rows, then over the RG row groups through LDS in a fixed order, so every
// result is bitwise reproducible.  Workgroup size is 2 * dv threads.
#include "kda_device.h"
#include "kda_internal.h"

#include <hip/hip_bf16.h>

namespace kda {

template <int DK, int DV, int VEC>
struct TileMap {
    static constexpr int NT = 2 * DV;          // threads per workgroup
    static constexpr int LJ = DV / VEC;        // lanes along one dv row
    static constexpr int RG = NT / LJ;         // row groups (= 2 * VEC)
    static constexpr int RPT = DK / RG;        // consecutive rows per thread
    static_assert(kWave % LJ == 0, "a dv row must tile a wave");
    static_assert(RPT >= 4 && DK % RG == 0 && RPT % 4 == 0, "rows per thread");
    static_assert(NT >= DK + DV, "conv needs one thread per q/k and v channel");
};

// Raw 128-bit words of the thread's state slice (issued early).
template <int ST, int DV, int RPT, int VEC>
__device__ __forceinline__ void load_state_raw(const void* head_base, int r, int c,
                                               uint4 (&raw)[RPT]) {
    const size_t esz = (ST == kF32) ? 4 : 2;
    const char* base = static_cast<const char*>(head_base) +
                       ((size_t)(r * RPT) * DV + (size_t)c * VEC) * esz;
#pragma unroll
    for (int p = 0; p < RPT; ++p)
        raw[p] = *reinterpret_cast<const uint4*>(base + (size_t)p * DV * esz);
}

template <int ST, int RPT, int VEC>
__device__ __forceinline__ void unpack_state(const uint4 (&raw)[RPT],
                                             float (&s)[RPT][VEC]) {
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
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

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __hip_bfloat162 p = __float22bfloat162_rn(make_float2(lo, hi));
    return *reinterpret_cast<uint32_t*>(&p);
}

// Typed store of the thread's state slice into [dk][dv] storage.
template <int ST, int DV, int RPT, int VEC>
__device__ __forceinline__ void store_state(void* head_base, int r, int c,
                                            const float (&s)[RPT][VEC]) {
    const size_t esz = (ST == kF32) ? 4 : 2;
    char* base = static_cast<char*>(head_base) +
                 ((size_t)(r * RPT) * DV + (size_t)c * VEC) * esz;
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        uint4 x;
        if constexpr (ST == kF32) {
            x = make_uint4(__float_as_uint(s[p][0]), __float_as_uint(s[p][1]),
                           __float_as_uint(s[p][2]), __float_as_uint(s[p][3]));
        } else {
            x = make_uint4(pack_bf16x2(s[p][0], s[p][1]), pack_bf16x2(s[p][2], s[p][3]),
                           pack_bf16x2(s[p][4], s[p][5]), pack_bf16x2(s[p][6], s[p][7]));
        }
        *reinterpret_cast<uint4*>(base + (size_t)p * DV * esz) = x;
    }
}

// FP32 record store, [dk][dv] like the pool.
template <int DV, int RPT, int VEC>
__device__ __forceinline__ void store_record(float* rec, int r, int c,
                                             const float (&s)[RPT][VEC]) {
    float* base = rec + (size_t)(r * RPT) * DV + c * VEC;
#pragma unroll
    for (int p = 0; p < RPT; ++p)
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
            *reinterpret_cast<float4*>(base + p * DV + e) =
                make_float4(s[p][e], s[p][e + 1], s[p][e + 2], s[p][e + 3]);
}

// Phase A of a token: the causal conv of this thread's channels (t < DK: q
// and k channel t; DK <= t < DK + DV: v channel t - DK), and the raw token
// copied to the ring (decode: entry pos mod 4) or to draft_conv (verify).
// Conv taps 0..2 read the three previous raw tokens (earlier drafts, else
// the ring, else zero before position 0), tap 3 the current one.
template <int DK, int DV, int ACT, bool VERIFY>
__device__ __forceinline__ void conv_token(const TokenArgs& a, int b, int h, int t, int n,
                                           int slot, int pos, float4 w4a, float4 w4b,
                                           float& ca, float& cb) {
    constexpr int C = 2 * DK + DV;
    const int tid = threadIdx.x;
    const int H = a.H;
    const bool has_qk = tid < DK;
    const bool has_v = tid >= DK && tid < DK + DV;
    ca = 0.f;
    cb = 0.f;
    if (!has_qk && !has_v) return;
    const int64_t tok = (int64_t)b * n + t;
    const size_t ring_slot = (size_t)slot * kConvW;   // ring [slot][4][H][C]
    const int vch = tid - DK;
    float xa[kConvW], xb[kConvW];
#pragma unroll
    for (int j = 0; j < kConvW; ++j) {
        const int rel = t - (kConvW - 1) + j;          // draft-token index
        float va = 0.f, vb = 0.f;
        if (rel >= 0) {
            const int64_t row = (int64_t)b * n + rel;
            if (has_qk) {
                va = ld_act<ACT>(a.q, (row * H + h) * DK + tid);
                vb = ld_act<ACT>(a.k, (row * H + h) * DK + tid);
            } else {
                va = ld_act<ACT>(a.v, (row * H + h) * DV + vch);
            }
        } else if (pos + rel >= 0) {
            const int64_t base = ((int64_t)(ring_slot + ((pos + rel) & (kConvW - 1))) * H + h) * C;
            if (has_qk) {
                va = ld_act<ACT>(a.ring, base + tid);
                vb = ld_act<ACT>(a.ring, base + DK + tid);
            } else {
                va = ld_act<ACT>(a.ring, base + 2 * DK + vch);
            }
        }
        xa[j] = va;
        xb[j] = vb;
    }
    ca = w4a.x * xa[0];
    ca = fmaf(w4a.y, xa[1], ca);
    ca = fmaf(w4a.z, xa[2], ca);
    ca = fmaf(w4a.w, xa[3], ca);
    if (has_qk) {
        cb = w4b.x * xb[0];
        cb = fmaf(w4b.y, xb[1], cb);
        cb = fmaf(w4b.z, xb[2], cb);
        cb = fmaf(w4b.w, xb[3], cb);
    }
    // keep the raw token: decode -> ring entry pos mod 4, verify -> draft_conv
    void* dst = VERIFY ? a.draft_conv : a.ring;
    const int64_t dbase = VERIFY ? (tok * H + h) * C
                                 : ((int64_t)(ring_slot + (pos & (kConvW - 1))) * H + h) * C;
    if (has_qk) {
        cp_act<ACT>(dst, dbase + tid, a.q, (tok * H + h) * DK + tid);
        cp_act<ACT>(dst, dbase + DK + tid, a.k, (tok * H + h) * DK + tid);
    } else {
        cp_act<ACT>(dst, dbase + 2 * DK + vch, a.v, (tok * H + h) * DV + vch);
    }
}

// Phase A of a token: conv, the decay factor of this thread's key channel,
// beta and the gate input, the conv of v into LDS, and the per-wave partial
// sums of |c_q|^2, |c_k|^2 and c_q . c_k.
template <int DK, int DV, int ACT, bool VERIFY>
__device__ __forceinline__ void phase_a(const TokenArgs& a, int b, int h, int t, int n,
                                        int slot, int pos, float4 w4a, float4 w4b,
                                        float* vt_s, float (*red_s)[4], float& ca,
                                        float& cb, float& al, float& beta, float& gv) {
    const int tid = threadIdx.x;
    const int H = a.H;
    const int64_t tok = (int64_t)b * n + t;
    const bool has_qk = tid < DK;
    const bool has_v = tid >= DK && tid < DK + DV;
    conv_token<DK, DV, ACT, VERIFY>(a, b, h, t, n, slot, pos, w4a, w4b, ca, cb);
    al = has_qk ? ld_act<ACT>(a.alpha, (tok * H + h) * DK + tid) : 0.f;
    beta = ld_act<ACT>(a.beta, tok * H + h);
    gv = (tid < DV) ? ld_act<ACT>(a.g, (tok * H + h) * DV + tid) : 0.f;
    if (has_v) vt_s[tid - DK] = ca;
    const float cq = has_qk ? ca : 0.f, ck = cb;
    const float sq = wave_sum(cq * cq), sk = wave_sum(ck * ck), sqk = wave_sum(cq * ck);
    if ((tid % kWave) == 0) {
        const int wave = tid / kWave;
        red_s[wave][0] = sq;
        red_s[wave][1] = sk;
        red_s[wave][2] = sqk;
    }
}

template <int DK, int DV, int ACT, int ST, bool VERIFY>
__global__ __launch_bounds__(2 * DV) void token_kernel(TokenArgs a) {
    constexpr int VEC = (ST == kF32) ? 4 : 8;
    using M = TileMap<DK, DV, VEC>;
    constexpr int LJ = M::LJ, RG = M::RG, RPT = M::RPT;
    constexpr int NW = M::NT / kWave;
    constexpr int PAD = 4;

    __shared__ float vt_s[DV];                   // conv of v
    __shared__ float ak_s[DK], aq_s[DK];         // alpha*kh, alpha*qh
    __shared__ float al_s[DK], kh_s[DK];         // alpha, kh
    __shared__ float delta_s[DV];
    __shared__ float part_s[2][RG][DV + PAD];    // dk-reduction partials
    __shared__ float red_s[NW][4];

    const int tid = threadIdx.x;
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int b = blockIdx.x / H;
    const int wave = tid / kWave;
    const int c = tid % LJ;                      // dv chunk: j = c*VEC + e
    const int r = tid / LJ;                      // row group: i = r*RPT + p
    const int n = a.n;
    const bool has_qk = tid < DK;
    const bool has_v = tid >= DK && tid < DK + DV;

    // slot-independent loads first: conv taps and the norm weight
    float4 w4a = make_float4(0, 0, 0, 0), w4b = w4a;
    if (has_qk) {
        w4a = *reinterpret_cast<const float4*>(a.wq + ((size_t)h * DK + tid) * kConvW);
        w4b = *reinterpret_cast<const float4*>(a.wk + ((size_t)h * DK + tid) * kConvW);
    } else if (has_v) {
        w4a = *reinterpret_cast<const float4*>(a.wv + ((size_t)h * DV + tid - DK) * kConvW);
    }
    const float norm_w = (tid < DV) ? (a.norm_w ? a.norm_w[tid] : 1.0f) : 0.0f;

    const int slot = a.slot_ids[b];
    const int pos = a.positions[b];
    if (slot < 0) return;
    if (slot >= a.num_slots) {
        if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_SLOT);
        return;
    }
    if (pos < 0) {
        if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_POSITION);
        return;
    }

    // ---- state in: issued first, consumed after the conv ----------------
    const size_t head_elems = (size_t)DK * DV;
    const size_t head_off = ((size_t)slot * H + h) * head_elems;
    const void* pool_head = static_cast<const char*>(a.pool) +
                            head_off * (ST == kF32 ? 4 : 2);
    uint4 raw[RPT];
    if (pos > 0) {
        load_state_raw<ST, DV, RPT, VEC>(pool_head, r, c, raw);
    } else {
#pragma unroll
        for (int p = 0; p < RPT; ++p) raw[p] = make_uint4(0, 0, 0, 0);
    }

    // token 0's phase A overlaps the state loads; the unpack then waits for them
    float ca, cb, al, beta, gv;
    phase_a<DK, DV, ACT, VERIFY>(a, b, h, 0, n, slot, pos, w4a, w4b, vt_s, red_s, ca, cb, al,
                                 beta, gv);
    float s[RPT][VEC];
    unpack_state<ST, RPT, VEC>(raw, s);

    for (int t = 0; t < n; ++t) {
        const int64_t tok = (int64_t)b * n + t;     // row of the inputs
        // ---------------- A. conv, raw copy, norm partial sums -----------
        if (t > 0)
            phase_a<DK, DV, ACT, VERIFY>(a, b, h, t, n, slot, pos, w4a, w4b, vt_s, red_s, ca, cb,
                                         al, beta, gv);
        __syncthreads();

        // ---------------- B. normalised keys and queries ----------------
        float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
        for (int w = 0; w < DK / kWave; ++w) {       // q/k live in waves 0..DK/64-1
            sq += red_s[w][0];
            sk += red_s[w][1];
            sqk += red_s[w][2];
        }
        const float rq = a.q_scale / sqrtf(sq + a.l2_eps);
        const float rk = 1.0f / sqrtf(sk + a.l2_eps);
        const float kq = sqk * rq * rk;              // kh . qh
        if (has_qk) {
            const float kh = cb * rk, qh = ca * rq;
            ak_s[tid] = al * kh;
            aq_s[tid] = al * qh;
            al_s[tid] = al;
            kh_s[tid] = kh;
        }
        __syncthreads();

        // ---------------- C. in-thread dk partials -----------------------
        {
            float u[VEC], o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) u[e] = o[e] = 0.f;
#pragma unroll
            for (int p4 = 0; p4 < RPT; p4 += 4) {
                const float4 ak4 = *reinterpret_cast<const float4*>(&ak_s[r * RPT + p4]);
                const float4 aq4 = *reinterpret_cast<const float4*>(&aq_s[r * RPT + p4]);
                const float akv[4] = {ak4.x, ak4.y, ak4.z, ak4.w};
                const float aqv[4] = {aq4.x, aq4.y, aq4.z, aq4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        u[e] = fmaf(s[p4 + q][e], akv[q], u[e]);
                        o[e] = fmaf(s[p4 + q][e], aqv[q], o[e]);
                    }
            }
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                *reinterpret_cast<float4*>(&part_s[0][r][c * VEC + e]) =
                    make_float4(u[e], u[e + 1], u[e + 2], u[e + 3]);
                *reinterpret_cast<float4*>(&part_s[1][r][c * VEC + e]) =
                    make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
            }
        }
        __syncthreads();

        // ---------------- D. finish the reductions, delta, read-out --------
        float o = 0.f;
        if (tid < DV) {
            float u = 0.f, op = 0.f;
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                u += part_s[0][g][tid];
                op += part_s[1][g][tid];
            }
            const float d = beta * (vt_s[tid] - u);
            delta_s[tid] = d;
            o = fmaf(kq, d, op);
        }
        {
            const float ms = wave_sum(o * o);
            if ((tid % kWave) == 0) red_s[wave][3] = ms;
        }
        __syncthreads();

        // ---------------- E. state update, store, gated RMSNorm ----------
        {
            float d[VEC];
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const float4 d4 = *reinterpret_cast<const float4*>(&delta_s[c * VEC + e]);
                d[e] = d4.x; d[e + 1] = d4.y; d[e + 2] = d4.z; d[e + 3] = d4.w;
            }
#pragma unroll
            for (int p4 = 0; p4 < RPT; p4 += 4) {
                const float4 al4 = *reinterpret_cast<const float4*>(&al_s[r * RPT + p4]);
                const float4 kh4 = *reinterpret_cast<const float4*>(&kh_s[r * RPT + p4]);
                const float alv[4] = {al4.x, al4.y, al4.z, al4.w};
                const float khv[4] = {kh4.x, kh4.y, kh4.z, kh4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        s[p4 + q][e] = fmaf(khv[q], d[e], s[p4 + q][e] * alv[q]);
            }
        }
        if constexpr (VERIFY) {
            store_record<DV, RPT, VEC>(a.records + ((size_t)tok * H + h) * head_elems, r, c, s);
        }
        if (tid < DV) {
            float ms = 0.f;
#pragma unroll
            for (int w = 0; w < DV / kWave; ++w) ms += red_s[w][3];
            const float rr = 1.0f / sqrtf(ms / (float)DV + a.norm_eps);
            a.y[(tok * H + h) * DV + tid] = norm_w * (o * rr) * gate_fn(a.gate, gv);
        }
        // The next token's LDS writes (vt_s, red_s[.][0..2], then ak_s..kh_s
        // after its first barrier) touch only what every thread finished
        // reading before this token's last barrier or in its own phase E.
    }

    if constexpr (!VERIFY) {
        store_state<ST, DV, RPT, VEC>(const_cast<void*>(pool_head), r, c, s);
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
