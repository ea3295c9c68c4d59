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
// consecutive key rows; LJ = dv / VEC lanes span a row and RG row groups
// span dk (EPT = 32 state elements per thread: 512 threads for
// dk = dv = 128; a one-token decode of a BF16 head takes EPT = 64, 256
// threads).  The dk-reductions run in-thread over the thread's RPT
// rows, then over the RG row groups through LDS in a fixed order, so every
// result is bitwise reproducible.
#include "kda_device.h"
#include "kda_internal.h"

#include <hip/hip_bf16.h>

namespace kda {

// What one launch does per row.
//   kModeDecode:    one token; state and ring stored.
//   kModeVerify:    n draft tokens, state in registers; optional FP32 record
//                   per token and raw drafts; pool and ring read only.
//   kModeRecompute: the first m = accepted[row] of n draft tokens again from
//                   the stored state (commit without records); state stored
//                   once, ring entries of the m tokens written, no output.
constexpr int kModeDecode = 0, kModeVerify = 1, kModeRecompute = 2;

template <int DK, int DV, int VEC, int EPT>
struct TileMap {
    static constexpr int NT = DK * DV / EPT;   // threads per workgroup: EPT state
                                               // elements per thread
    static constexpr int LJ = DV / VEC;        // lanes along one dv row
    static constexpr int RG = NT / LJ;         // row groups
    static constexpr int RPT = DK / RG;        // consecutive rows per thread
    static_assert(kWave % LJ == 0, "a dv row must tile a wave");
    static_assert(RPT >= 4 && DK % RG == 0 && RPT % 4 == 0, "rows per thread");
    static_assert(NT >= DK + DV, "conv needs one thread per q/k and v channel");
    static_assert(NT % kWave == 0 && NT <= 1024, "workgroup size");
};

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

// Streaming 128-bit accesses: each state byte is touched once per call and
// not again until the next call, so loads and stores bypass cache retention
// (nontemporal hint).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
    const v4u32 v = __builtin_nontemporal_load(static_cast<const v4u32*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, uint4 x) {
    const v4u32 v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, static_cast<v4u32*>(p));
}

// Raw 128-bit words of the thread's state slice (issued early).
template <int ST, int DV, int RPT, int VEC>
__device__ __forceinline__ void load_state_raw(const void* head_base, int r, int c,
                                               uint4 (&raw)[RPT]) {
    const size_t esz = (ST == kF32) ? 4 : 2;
    const char* base = static_cast<const char*>(head_base) +
                       ((size_t)(r * RPT) * DV + (size_t)c * VEC) * esz;
#pragma unroll
    for (int p = 0; p < RPT; ++p) raw[p] = ld_stream(base + (size_t)p * DV * esz);
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
        st_stream(base + (size_t)p * DV * esz, x);
    }
}

// Store of the thread's state slice kept packed (BF16 storage, decode).
template <int DV, int RPT, int VEC>
__device__ __forceinline__ void store_packed(void* head_base, int r, int c,
                                             const uint4 (&raw)[RPT]) {
    char* base = static_cast<char*>(head_base) + ((size_t)(r * RPT) * DV + (size_t)c * VEC) * 2;
#pragma unroll
    for (int p = 0; p < RPT; ++p) st_stream(base + (size_t)p * DV * 2, raw[p]);
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
            st_stream(base + p * DV + e,
                      make_uint4(__float_as_uint(s[p][e]), __float_as_uint(s[p][e + 1]),
                                 __float_as_uint(s[p][e + 2]), __float_as_uint(s[p][e + 3])));
}

// Phase A of a token.  Conv roles, one per wave (dk and dv are multiples of
// the wave size): waves covering threads t < DK convolve q channel t (A) and
// k channel t (B); waves covering DK <= t < DK + DV convolve v channel t - DK
// (A); the remaining waves only load their inputs.  Conv taps 0..2 read the
// three previous raw tokens (earlier drafts of this call, else the ring, else
// zero before position 0), tap 3 the current token.  Every row address is
// wave-uniform (a scalar base plus a 32-bit lane offset), and every load is
// issued before any loaded value is used, so no wait for one tap stalls the
// others or the state stream; taps before position 0 are zeroed afterwards.
// The raw token is copied to the ring (decode and recompute: entry
// (pos + t) mod 4) or to draft_conv (verify; skipped when draft_conv is
// NULL).  Also loads alpha, beta and g (forming them from their logits when
// asked), writes the conv of v to LDS and the per-wave partial sums of
// |c_q|^2, |c_k|^2 and c_q . c_k.  `n` is the number of input rows per batch
// row (1 for decode, the draft count otherwise).
template <int DK, int DV, int ACT, int MODE, bool STRIDED, class Issue>
__device__ __forceinline__ void phase_a(const TokenArgs& a, int b, int h, int t, int n,
                                        int slot, int pos, float4 w4a, float4 w4b,
                                        float* vt_s, float (*red_s)[4], float& ca,
                                        float& cb, float& al, float& beta, float& gv,
                                        Issue&& issue_more) {
    constexpr int C = 2 * DK + DV;
    constexpr size_t ESZ = kActSize<ACT>;                  // q, k, v, ring, drafts
    constexpr int GACT = kGateAct<ACT>;
    constexpr size_t GESZ = kActSize<GACT>;                // alpha, beta, g
    const int tid = threadIdx.x;
    const int H = a.H;
    const int64_t tok = (int64_t)b * n + t;
    const int wfirst = __builtin_amdgcn_readfirstlane(tid);
    const bool qk = wfirst < DK;                         // wave-uniform role
    const bool isv = !qk && wfirst < DK + DV;
    const int lc = qk ? tid : (isv ? tid - DK : 0);     // channel within q|k or v

    const char* qb = static_cast<const char*>(a.q);
    const char* kb = static_cast<const char*>(a.k);
    const char* vb = static_cast<const char*>(a.v);
    const char* ringb = static_cast<const char*>(a.ring);

    // unconditional loads from valid lane offsets; lanes that do not own a
    // channel discard the value
    const float al_ld = ld_act<GACT>(static_cast<const char*>(a.alpha) +
                                         (size_t)(tok * H + h) * DK * GESZ, qk ? tid : 0);
    // token rows of q, k, v and g: contiguous [rows, H, d], or (STRIDED)
    // a.qkv_rs / a.g_rs elements apart
    const size_t g_off = STRIDED ? (size_t)(tok * a.g_rs + h * DV) : (size_t)(tok * H + h) * DV;
    const float g_ld = ld_act<GACT>(static_cast<const char*>(a.g) + g_off * GESZ,
                                    tid < DV ? tid : 0);
    beta = ld_act<GACT>(a.beta, tok * H + h);
    al = qk ? al_ld : 0.f;
    if (a.gate_logits) {
        beta = write_from_logit(beta);
        al = qk ? decay_from_logit(al_ld) : 0.f;
    }
    gv = (tid < DV) ? g_ld : 0.f;

    ca = 0.f;
    cb = 0.f;
    const size_t ring_slot = (size_t)slot * kConvW;       // ring [slot][4][H][C]
    uint32_t bA[kConvW], bB[kConvW];
    if (qk || isv) {
#pragma unroll
        for (int j = 0; j < kConvW; ++j) {
            const int rel = t - (kConvW - 1) + j;          // draft-token index
            const char* pa;
            const char* pb;
            if (rel >= 0) {
                const int64_t row = (int64_t)b * n + rel;
                if constexpr (STRIDED) {
                    pa = qk ? qb + (size_t)(row * a.qkv_rs + h * DK) * ESZ
                            : vb + (size_t)(row * a.qkv_rs + h * DV) * ESZ;
                    pb = kb + (size_t)(row * a.qkv_rs + h * DK) * ESZ;
                } else {
                    pa = qk ? qb + (size_t)(row * H + h) * DK * ESZ
                            : vb + (size_t)(row * H + h) * DV * ESZ;
                    pb = kb + (size_t)(row * H + h) * DK * ESZ;
                }
            } else {
                const char* e = ringb +
                    ((size_t)(ring_slot + ((pos + rel) & (kConvW - 1))) * H + h) * C * ESZ;
                pa = e + (qk ? 0 : 2 * DK) * ESZ;
                pb = e + DK * ESZ;
            }
            bA[j] = ld_act_bits<ACT>(pa, lc);
            bB[j] = ld_act_bits<ACT>(pb, lc);
        }
    }
    // further loads (the state stream on a call's first token) go out behind
    // the conv taps, so the conv below waits only for the taps
    issue_more();
    if (qk || isv) {
        float xa[kConvW], xb[kConvW];
#pragma unroll
        for (int j = 0; j < kConvW; ++j) {
            const int rel = t - (kConvW - 1) + j;
            const bool live = rel >= 0 || pos + rel >= 0;
            xa[j] = live ? act_from_bits<ACT>(bA[j]) : 0.f;
            xb[j] = live ? act_from_bits<ACT>(bB[j]) : 0.f;
        }
        ca = w4a.x * xa[0];
        ca = fmaf(w4a.y, xa[1], ca);
        ca = fmaf(w4a.z, xa[2], ca);
        ca = fmaf(w4a.w, xa[3], ca);
        if (qk) {
            cb = w4b.x * xb[0];
            cb = fmaf(w4b.y, xb[1], cb);
            cb = fmaf(w4b.z, xb[2], cb);
            cb = fmaf(w4b.w, xb[3], cb);
        }
        if constexpr (ACT == kFP8) {
            // per-tensor dequantisation, taken out of the conv sum
            ca *= qk ? a.scale_q : a.scale_v;
            cb *= a.scale_k;
        }
        // keep the raw token: decode and recompute -> ring entry (pos + t)
        // mod 4, verify -> draft_conv (when kept)
        if (MODE != kModeVerify || a.draft_conv) {
            char* dst = MODE == kModeVerify
                ? static_cast<char*>(a.draft_conv) + (size_t)(tok * H + h) * C * ESZ
                : static_cast<char*>(a.ring) +
                      ((size_t)(ring_slot + ((pos + t) & (kConvW - 1))) * H + h) * C * ESZ;
            st_act_bits<ACT>(dst + (qk ? 0 : 2 * DK) * ESZ, lc, bA[kConvW - 1]);
            if (qk) st_act_bits<ACT>(dst + DK * ESZ, lc, bB[kConvW - 1]);
        }
    }
    if (isv) vt_s[lc] = ca;
    const float cq = qk ? ca : 0.f, ck = cb;
    const float sq = wave_sum(cq * cq), sk = wave_sum(ck * ck), sqk = wave_sum(cq * ck);
    if ((tid % kWave) == 0) {
        const int wave = tid / kWave;
        red_s[wave][0] = sq;
        red_s[wave][1] = sk;
        red_s[wave][2] = sqk;
    }
}

template <int DK, int DV, int ACT, int ST, int MODE, bool STRIDED, int EPT>
__global__ __launch_bounds__(DK * DV / EPT) void token_kernel(TokenArgs a) {
    constexpr int VEC = (ST == kF32) ? 4 : 8;
    using M = TileMap<DK, DV, VEC, EPT>;
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
    constexpr bool VERIFY = MODE == kModeVerify;
    constexpr bool RECOMP = MODE == kModeRecompute;
    const int stride = MODE == kModeDecode ? 1 : a.n;   // input rows per batch row
    int n = VERIFY ? a.n : 1;                   // tokens to run (decode: one)
    const bool qk_lane = tid < DK;
    const bool v_lane = tid >= DK && tid < DK + DV;

    // slot-independent loads first: conv taps (q|v and k channel of this
    // thread's conv role; idle lanes read a valid row they do not use) and
    // the norm weight
    const float* wA = qk_lane ? a.wq + ((size_t)h * DK + tid) * kConvW
                              : a.wv + ((size_t)h * DV + (v_lane ? tid - DK : 0)) * kConvW;
    const float* wB = a.wk + ((size_t)h * DK + (qk_lane ? tid : 0)) * kConvW;
    const float4 w4a = *reinterpret_cast<const float4*>(wA);
    const float4 w4b = *reinterpret_cast<const float4*>(wB);
    const float norm_w = (tid < DV) ? (a.norm_w ? a.norm_w[tid] : 1.0f) : 0.0f;

    // both row parameters are tested before any store can happen, so they
    // stay scalar loads and nothing waits on vector memory before the state
    // stream is issued
    const int slot = a.slot_ids[b];
    const int pos = a.positions[b];
    if (slot < 0) return;
    if (slot >= a.num_slots || pos < 0) {
        if (tid == 0 && a.status)
            atomicOr(a.status, slot >= a.num_slots ? KDA_STATUS_BAD_SLOT : KDA_STATUS_BAD_POSITION);
        return;
    }
    if constexpr (RECOMP) {
        const int m = a.accepted[b];
        if (m < 0 || m > a.n) {
            if (tid == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_ACCEPTED);
            return;
        }
        if (m == 0) return;
        n = m;
    }

    // ---- state in: issued as soon as the slot is known (a fresh sequence,
    // position 0, discards what it loaded), consumed after the conv --------
    const size_t head_elems = (size_t)DK * DV;
    const size_t head_off = ((size_t)slot * H + h) * head_elems;
    const void* pool_head = static_cast<const char*>(a.pool) +
                            head_off * (ST == kF32 ? 4 : 2);
    // token 0: conv taps first, then the state stream; phase A's math and
    // phase B overlap the state loads, and the unpack waits for them
    uint4 raw[RPT];
    float ca, cb, al, beta, gv;
    phase_a<DK, DV, ACT, MODE, STRIDED>(a, b, h, 0, stride, slot, pos, w4a, w4b, vt_s, red_s, ca, cb, al,
                                 beta, gv,
                                 [&] { load_state_raw<ST, DV, RPT, VEC>(pool_head, r, c, raw); });
    // A decode call with BF16 storage keeps the state packed as loaded and
    // widens one row at a time where it is used: the FP32 values are exact
    // and the update rounds once on the way out, as with a widened copy,
    // but 16 fewer registers stay live.  Verify, recompute (several tokens,
    // rounded once at the end) and FP32 storage hold the FP32 state.
    constexpr bool PACKED = MODE == kModeDecode && ST == kBF16;
    float s[PACKED ? 1 : RPT][VEC];
    if constexpr (PACKED) {
        if (pos == 0) {
#pragma unroll
            for (int p = 0; p < RPT; ++p) raw[p] = make_uint4(0u, 0u, 0u, 0u);
        }
    } else {
        unpack_state<ST, RPT, VEC>(raw, s);
        if (pos == 0) {
#pragma unroll
            for (int p = 0; p < RPT; ++p)
#pragma unroll
                for (int e = 0; e < VEC; ++e) s[p][e] = 0.f;
        }
    }
    auto srow = [&](int p, float (&sv)[VEC]) {
        if constexpr (PACKED) {
            const uint32_t w[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sv[2 * e] = bf16_to_f32(w[e] & 0xffffu);
                sv[2 * e + 1] = bf16_to_f32(w[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) sv[e] = s[p][e];
        }
    };

#pragma unroll 1
    for (int t = 0; t < n; ++t) {
        const int64_t tok = (int64_t)b * stride + t;   // row of the inputs
        // ---------------- A. conv, raw copy, norm partial sums -----------
        if (t > 0)
            phase_a<DK, DV, ACT, MODE, STRIDED>(a, b, h, t, stride, slot, pos, w4a, w4b, vt_s, red_s, ca, cb,
                                         al, beta, gv, [] {});
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
        if (qk_lane) {
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
                for (int q = 0; q < 4; ++q) {
                    float sv[VEC];
                    srow(p4 + q, sv);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        u[e] = fmaf(sv[e], akv[q], u[e]);
                        o[e] = fmaf(sv[e], aqv[q], o[e]);
                    }
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
                for (int q = 0; q < 4; ++q) {
                    float sv[VEC];
                    srow(p4 + q, sv);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) sv[e] = fmaf(khv[q], d[e], sv[e] * alv[q]);
                    if constexpr (PACKED) {
                        raw[p4 + q] = make_uint4(pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                                                 pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7]));
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) s[p4 + q][e] = sv[e];
                    }
                }
            }
        }
        if constexpr (VERIFY) {
            if (a.records)
                store_record<DV, RPT, VEC>(a.records + ((size_t)tok * H + h) * head_elems, r, c, s);
        }
        if (!RECOMP && tid < DV) {
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

    if constexpr (PACKED) {
        store_packed<DV, RPT, VEC>(const_cast<void*>(pool_head), r, c, raw);
    } else if constexpr (!VERIFY) {
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
    // every 16-byte word of the thread's share of the record is requested
    // before any is stored (the record and the pool are distinct buffers),
    // so the copy streams instead of waiting once per word
    constexpr int kThreads = 256;
    if constexpr (ST == kF32) {
        constexpr int kWords = DK * DV / 4 / kThreads;
        char* dst = static_cast<char*>(a.pool) + head_off * 4;
        const char* src = reinterpret_cast<const char*>(rec);
        uint4 w[kWords];
#pragma unroll
        for (int q = 0; q < kWords; ++q) w[q] = ld_stream(src + (size_t)(tid + q * kThreads) * 16);
#pragma unroll
        for (int q = 0; q < kWords; ++q) st_stream(dst + (size_t)(tid + q * kThreads) * 16, w[q]);
    } else {
        constexpr int kWords = DK * DV / 8 / kThreads;     // bf16 words out, two FP32 words in
        char* dst = static_cast<char*>(a.pool) + head_off * 2;
        const char* src = reinterpret_cast<const char*>(rec);
        uint4 x[2 * kWords];
#pragma unroll
        for (int q = 0; q < kWords; ++q) {
            x[2 * q] = ld_stream(src + (size_t)(tid + q * kThreads) * 32);
            x[2 * q + 1] = ld_stream(src + (size_t)(tid + q * kThreads) * 32 + 16);
        }
#pragma unroll
        for (int q = 0; q < kWords; ++q) {
            const uint4 x0 = x[2 * q], x1 = x[2 * q + 1];
            uint4 o;
            o.x = pack_bf16x2(__uint_as_float(x0.x), __uint_as_float(x0.y));
            o.y = pack_bf16x2(__uint_as_float(x0.z), __uint_as_float(x0.w));
            o.z = pack_bf16x2(__uint_as_float(x1.x), __uint_as_float(x1.y));
            o.w = pack_bf16x2(__uint_as_float(x1.z), __uint_as_float(x1.w));
            st_stream(dst + (size_t)(tid + q * kThreads) * 16, o);
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

// State elements per thread of a one-token decode: a 32 KiB BF16 head
// (dk = dv = 128) is streamed by 256 threads with 128 bytes each (measured
// 0.3% faster than 512 threads with 64 bytes on the 256-row BF16-state
// workload, same session, ABBA), every other case by DK * DV / 32 threads.
template <int DK, int ST>
constexpr int kDecodeEpt = (ST == kBF16 && DK == 128) ? 64 : 32;

template <int DK, int DV, int ACT, int ST, bool STRIDED>
static void launch_token_s(const TokenArgs& a, int32_t batch, int mode, hipStream_t stream) {
    const dim3 grid((unsigned)batch * (unsigned)a.H), block(DK * DV / 32);
    if (mode == kModeVerify) {
        hipLaunchKernelGGL((token_kernel<DK, DV, ACT, ST, kModeVerify, STRIDED, 32>), grid, block,
                           0, stream, a);
    } else if (mode == kModeRecompute) {
        hipLaunchKernelGGL((token_kernel<DK, DV, ACT, ST, kModeRecompute, STRIDED, 32>), grid,
                           block, 0, stream, a);
    } else {
        constexpr int EPT = kDecodeEpt<DK, ST>;
        hipLaunchKernelGGL((token_kernel<DK, DV, ACT, ST, kModeDecode, STRIDED, EPT>), grid,
                           dim3(DK * DV / EPT), 0, stream, a);
    }
}

// Contiguous inputs take the instantiation whose addressing has no row
// strides; inputs with a row stride other than the contiguous one take the
// strided one.
template <int DK, int DV, int ACT, int ST>
static int launch_token_t(const TokenArgs& a, int32_t batch, int mode, hipStream_t stream) {
    const int64_t w = (int64_t)a.H * DK;
    if (a.qkv_rs == w && a.g_rs == w)
        launch_token_s<DK, DV, ACT, ST, false>(a, batch, mode, stream);
    else
        launch_token_s<DK, DV, ACT, ST, true>(a, batch, mode, stream);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

template <int DK, int DV>
static int dispatch_token(const kda_shape& s, const TokenArgs& a, int32_t batch, int mode,
                          hipStream_t stream) {
    if (s.act_dtype == kF32 && s.state_dtype == kF32)
        return launch_token_t<DK, DV, kF32, kF32>(a, batch, mode, stream);
    if (s.act_dtype == kF32 && s.state_dtype == kBF16)
        return launch_token_t<DK, DV, kF32, kBF16>(a, batch, mode, stream);
    if (s.act_dtype == kBF16 && s.state_dtype == kF32)
        return launch_token_t<DK, DV, kBF16, kF32>(a, batch, mode, stream);
    if (s.act_dtype == kFP8 && s.state_dtype == kF32)
        return launch_token_t<DK, DV, kFP8, kF32>(a, batch, mode, stream);
    if (s.act_dtype == kFP8)
        return launch_token_t<DK, DV, kFP8, kBF16>(a, batch, mode, stream);
    return launch_token_t<DK, DV, kBF16, kBF16>(a, batch, mode, stream);
}

int launch_token(const kda_shape& s, const TokenArgs& a, int32_t batch, TokenMode mode,
                 hipStream_t stream) {
    const int m = mode == TokenMode::Verify ? kModeVerify
                : mode == TokenMode::Recompute ? kModeRecompute : kModeDecode;
    if (s.head_k == 128 && s.head_v == 128)
        return dispatch_token<128, 128>(s, a, batch, m, stream);
    if (s.head_k == 64 && s.head_v == 64)
        return dispatch_token<64, 64>(s, a, batch, m, stream);
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
    if (s.act_dtype == kFP8 && s.state_dtype == kF32)
        return launch_commit_t<DK, DV, kFP8, kF32>(a, batch, stream);
    if (s.act_dtype == kFP8)
        return launch_commit_t<DK, DV, kFP8, kBF16>(a, batch, stream);
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
