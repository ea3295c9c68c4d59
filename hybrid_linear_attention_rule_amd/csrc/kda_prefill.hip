// Chunked prefill of the KDA mixer on gfx950: the chunkwise (WY/UT) form of
// the gated delta rule over variable-length sequences.
//
// Source: the KDA prefill kernel and its varlen chunk-index glue ("Kimi K3
// NVFP4 on Rubin (SM107): Modeling V2 target and the runtime it needs",
// section 3); FP32 recurrence with FP32 or BF16 state storage, the state
// stored once at the end ("Extend NVIDIA/TensorRT-LLM#19991 with isolated
// NVFP4 Kimi K3 targets", Description).
//
// Within a chunk of L <= 64 tokens with start state S0, let e(t, i) be the
// product of alpha over tokens i+1..t (per key channel; 1 when i = t).  The
// write vectors u_t of the token-by-token recurrence satisfy
//     (I + A) U = diag(beta) (V - K_G S0),
//     A_ti = beta_t sum_c kh_tc kh_ic e_c(t, i)    (i < t),
// with K_G = kh scaled by e(t, -1), the decay from the chunk start.  So
// U = Ut - W S0, where [W | Ut] solves (I + A) X = diag(beta) [K_G | V].
// Then
//     O   = (e(t,-1) * Q) S0 + (P (.) causal) U,
//           P_ti = sum_c qh_tc kh_ic e_c(t, i)   (i <= t),
//     S_L = Diag(e(last,-1)) S0 + (e(last, t) * K)^T U.
//
// Decay factors are products of alpha, never exponentials of differences of
// prefix sums, so nothing can overflow or lose range for any alpha in
// (0, 1].  Tokens are grouped in 4-token sub-blocks.  For a pair (t, i) in
// different sub-blocks, e(t, i) factors through any sub-block boundary J
// between them: (alpha over J..t) * (alpha over i+1..J-1), both factors in
// [0, 1], so those entries are matrix-core products of scaled keys and
// queries.  Pairs inside one sub-block are formed elementwise in registers.
//
// Three kernels:
//   chunk  (persistent, one eight-wave workgroup per compute unit, items
//          chunk x head): conv, L2 norms, decay products, A and P, the
//          diagonal 16x16 inverses of (I + A), the blocked forward
//          substitution for [W | Ut]; writes W (negated), decay-scaled Q and
//          K and P as pre-split fp16 pairs in matrix-core fragment order, Ut
//          in FP32, and the chunk's total decay;
//   state  (four workgroups per sequence x head, 32 value columns each,
//          sequential over the sequence's chunks, one barrier per chunk):
//          U, O and the next state on the matrix cores; two loader waves
//          stream each chunk's chain operands into LDS by direct
//          global-to-LDS loads, a chunk ahead, double-buffered; two U/S
//          waves, one per 16-column tile, form U and update the state tile
//          they hold in registers, independently of each other; two O waves
//          form O; O is written unnormalised; the final state is stored
//          once and the ring gets the sequence's last raw tokens;
//   finish (per token x head): the gated RMSNorm of O.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace kda {

constexpr int PC = 64;             // chunk length
constexpr int PD = 128;            // dk = dv handled by the prefill kernels
constexpr int LR = PD + 4;         // padded LDS row of a [PC][PD] tile (floats)
constexpr int LS = PC + 4;         // padded LDS row of a [PC][PC] tile
constexpr int NSB = PC / 4;        // 4-token sub-blocks per chunk

// Operand scaling for the split-fp16 products.  The split of x into fp16
// hi + lo keeps 2^-22 of |x| only while |x| < 65504 and |x| >= 2^-3; below
// that lo falls into fp16 subnormals (about 3e-8 absolute per element).
//   - Key-side operands bounded by 1 (normalised keys and queries times decay
//     factors, A and P) are multiplied by 2^12 before the split, T_bb and W
//     by 2^8.  |W| <= 1: row t of W is beta_t times the product of the
//     earlier tokens' (I - beta k k^T) Diag(alpha) factors applied to k_t,
//     each factor of norm at most 1.
//   - Value-side operands (V, Ut, U and the state S) have no bound: v and
//     the stored state may have any magnitude.  Every value column j carries
//     a power-of-two scale 2^-e_j per chunk, with e_j the exponent of the
//     column's largest magnitude (pow2_scale), so the split always sees values
//     of order 1.  Every product on the value side is linear in each value
//     column and never mixes columns, so a column's scale passes through it
//     unchanged and is removed exactly afterwards.
// Products are scaled back by exact powers of two.  The query scale is not
// folded into any operand: O is linear in the normalised queries, so it
// multiplies O once before the gated norm.
constexpr float kSc = 4096.f, kInvSc = 1.f / 4096.f, kInvSc2 = 1.f / 16777216.f;
constexpr float kScW = 256.f, kInvScW = 1.f / 256.f;

// Power-of-two scale for a value column whose largest magnitude is m:
// s = 2^-e with e the exponent of m, so m * s lies in [1, 2); is = 1 / s.
// The exponent is clamped so that both stay normal FP32 numbers (m = 0 gives
// s = 2^126, harmless on a zero column).
__device__ __forceinline__ void pow2_scale(float m, float& s, float& is) {
    const uint32_t ef = min(max((__float_as_uint(m) >> 23) & 0xffu, 1u), 253u);
    s = __uint_as_float((254u - ef) << 23);
    is = __uint_as_float(ef << 23);
}

// Largest value over the four lanes n, n + 16, n + 32, n + 48 (one matrix
// column); every one of them gets the result.  The lane swaps of gfx950
// (v_permlane16_swap, v_permlane32_swap) pair each lane with lane ^ 16 and
// then lane ^ 32 in the vector unit, without a round trip through LDS.
__device__ __forceinline__ float col_max4(float m) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Workspace per (chunk slot, head), in bytes.  A fragment is one 16x16x32
// MFMA operand for a wave: 64 lanes x 8 fp16 hi values, then 64 x 8 lo.
// Half h of a chunk (tokens 32h..32h+31 for the token-indexed operands)
// holds, in this order: -W tiles (2 x 4), scaled-Q tiles (2 x 4), scaled-K
// tiles for that half of the tokens (8), and the P tiles of its rows (2 in
// half 0, 4 in half 1); half 0's slot 26 holds the chunk's total decay
// (FP32 [PD]) and then the largest |Ut| of each value column over the
// chunk (FP32 [PD]).  Ut follows in FP32, in the state kernel's D-tile order.
constexpr int FRAG_B = 2048;
constexpr int HALF_FRAGS = 28;
constexpr int HALF_B = HALF_FRAGS * FRAG_B;
constexpr int GAM_OFF = 26 * FRAG_B;           // in half 0
constexpr int UTMAX_OFF = GAM_OFF + PD * 4;    // in half 0
constexpr int UT_OFF = 2 * HALF_B;
constexpr int WS_B = UT_OFF + PC * PD * 4;

__device__ __forceinline__ int frag_w(int u, int kb) { return 4 * u + kb; }
__device__ __forceinline__ int frag_q(int u, int kb) { return 8 + 4 * u + kb; }
__device__ __forceinline__ int frag_k(int ct) { return 16 + ct; }
__device__ __forceinline__ int frag_p(int hh, int u, int kb) { return 24 + u * (hh + 1) + kb; }

// Chunk slot of chunk c of sequence s: floor(lo / 64) + s + c.  Distinct for
// all (s, c) of monotone cu_seqlens and below ceil(total / 64) + num_seqs.
__device__ __forceinline__ int64_t chunk_slot(int lo, int s, int c) {
    return (int64_t)(lo / PC) + s + c;
}

size_t prefill_workspace_bytes(const kda_shape& sh, int32_t num_seqs, int64_t total_tokens) {
    if (sh.head_k != PD || sh.head_v != PD) return 0;
    const int64_t slots = (total_tokens + PC - 1) / PC + num_seqs;
    return (size_t)slots * sh.num_heads * WS_B;
}

struct SeqView {
    int lo, len, slot, pos;
};

// Checks a sequence's bounds, slot and position.  Returns false when it must
// be skipped; `bits` gets the status bits to report (0 for an inactive slot).
__device__ __forceinline__ bool seq_ok(const PrefillArgs& a, int lo, int hi, int slot, int pos,
                                       int& bits) {
    bits = 0;
    if (!(lo >= 0 && lo <= hi && hi <= a.total_tokens && hi - lo <= a.max_seqlen))
        bits = KDA_STATUS_BAD_SEQLENS;
    else if (slot < 0)
        return false;                            // inactive: skipped, not an error
    else if (slot >= a.num_slots)
        bits = KDA_STATUS_BAD_SLOT;
    else if (pos < 0)
        bits = KDA_STATUS_BAD_POSITION;
    return bits == 0;
}

// Validates sequence s.  Returns false when it must be skipped; `report`
// selects the threads that OR the status bits.  All four values are read
// before the status update can happen, so that for a uniform s they stay
// scalar loads.
__device__ __forceinline__ bool seq_view(const PrefillArgs& a, int s, bool report, SeqView& v) {
    const int lo = a.cu_seqlens[s], hi = a.cu_seqlens[s + 1];
    const int slot = a.slot_ids[s], pos = a.positions[s];
    int bits;
    const bool ok = seq_ok(a, lo, hi, slot, pos, bits);
    if (bits != 0 && report && a.status) atomicOr(a.status, bits);
    if (!ok) return false;
    v = SeqView{lo, hi - lo, slot, pos};
    return true;
}

// A 32-bit read through the scalar data cache, waited for at once, of a
// value the kernel never writes.  For uniform reads inside a loop that also
// stores to global memory, where the compiler would make a vector load
// (assuming a store may alias it) and wait behind every outstanding vector
// access, stores included.
// Every caller passes a uniform address; it is read through readfirstlane so
// that it sits in scalar registers even where the compiler keeps it in
// vector ones.
__device__ __forceinline__ int32_t sload_i32(const int32_t* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    const int32_t* q = reinterpret_cast<const int32_t*>(lo | (hi << 32));
    int32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q));
    return v;
}

// Four consecutive activations of one token, as loaded (aligned to their
// size: 16 bytes FP32, 8 bytes BF16, 4 bytes FP8).
template <int ACT>
struct Raw4;
template <>
struct Raw4<kF32> {
    float4 a;
};
template <>
struct Raw4<kBF16> {
    uint2 u;
};
template <>
struct Raw4<kFP8> {
    uint32_t u;                       // four E4M3 bytes
};

template <int ACT>
__device__ __forceinline__ Raw4<ACT> ld_raw4(const void* base, int64_t idx) {
    Raw4<ACT> r;
    if constexpr (ACT == kF32)
        r.a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    else if constexpr (ACT == kBF16)
        r.u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    else
        r.u = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(base) + idx);
    return r;
}

// The same at byte offset `off` from `base`.
template <int ACT>
__device__ __forceinline__ Raw4<ACT> ld_raw4_at(const char* base, uint32_t off) {
    Raw4<ACT> r;
    if constexpr (ACT == kF32)
        r.a = *reinterpret_cast<const float4*>(base + off);
    else if constexpr (ACT == kBF16)
        r.u = *reinterpret_cast<const uint2*>(base + off);
    else
        r.u = *reinterpret_cast<const uint32_t*>(base + off);
    return r;
}

// Zero unless ok, selected on the raw words.
template <int ACT>
__device__ __forceinline__ Raw4<ACT> keep_if(const Raw4<ACT>& r, bool ok) {
    Raw4<ACT> o;
    if constexpr (ACT == kF32)
        o.a = make_float4(ok ? r.a.x : 0.f, ok ? r.a.y : 0.f, ok ? r.a.z : 0.f, ok ? r.a.w : 0.f);
    else if constexpr (ACT == kBF16)
        o.u = make_uint2(ok ? r.u.x : 0u, ok ? r.u.y : 0u);
    else
        o.u = ok ? r.u : 0u;
    return o;
}

// Widens to FP32.
template <int ACT>
__device__ __forceinline__ void unpack4(const Raw4<ACT>& r, float (&x)[4]) {
    if constexpr (ACT == kF32) {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    } else if constexpr (ACT == kBF16) {
        x[0] = __uint_as_float(r.u.x << 16); x[1] = __uint_as_float(r.u.x & 0xffff0000u);
        x[2] = __uint_as_float(r.u.y << 16); x[3] = __uint_as_float(r.u.y & 0xffff0000u);
    } else {
        e4m3x4_to_f32(r.u, x);
    }
}

// Raw channels [ch0, ch0 + 4) of one of q|k|v for local chunk token lt
// (-3 <= lt < 64): the packed input inside the sequence, the ring for
// earlier positions >= 0; `ok` is false before position 0 and past the
// chunk's end, where the value must count as zero.  Branch-free: the load
// always goes to a valid address (the chunk's first token where `ok` is
// false), so all of a lane's loads are in flight together.
template <int ACT>
__device__ __forceinline__ Raw4<ACT> raw4(const PrefillArgs& a, const SeqView& v, int h, int t0,
                                          int L, int lt, const void* src, int ch0, int ring_ch0,
                                          bool& ok) {
    const int gt = t0 + lt;
    const int p = v.pos + gt;
    const bool in_seq = gt >= 0;
    ok = lt < L && (in_seq || p >= 0);
    const bool use_ring = ok && !in_seq;
    const int64_t idx_in = (int64_t)(v.lo + (ok && in_seq ? gt : t0)) * a.qkv_rs + h * PD + ch0;
    const int64_t idx_ring =
        (((int64_t)v.slot * kConvW + (p & (kConvW - 1))) * a.H + h) * (3 * PD) + ring_ch0;
    return ld_raw4<ACT>(use_ring ? a.ring : src, use_ring ? idx_ring : idx_in);
}

// Conv of one of q|k|v for this lane's four tokens (tb..tb+3) and channels
// [c0, c0 + 4), from the seven raw tokens tb-3..tb+3 and the channels' four
// taps; zero for tokens at or past L.  FP8 activations: times the tensor's
// dequantisation scale `sc`, taken out of the sum.  Only the three raw
// tokens before tb can lie before position 0 and must read as zero (`ok`);
// a later raw token past the chunk's end feeds only outputs at or past L,
// which are zeroed here whatever it holds.
template <int ACT>
__device__ __forceinline__ void conv4x4(const Raw4<ACT> (&r)[7], const bool (&ok)[3],
                                        const float4 (&wt)[4], int tb, int L, float sc,
                                        float (&c)[4][4]) {
    float x[7][4];
#pragma unroll
    for (int m = 0; m < 7; ++m) unpack4<ACT>(m < 3 ? keep_if<ACT>(r[m], ok[m]) : r[m], x[m]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 w4 = wt[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = w4.x * x[e][q];
            acc = fmaf(w4.y, x[e + 1][q], acc);
            acc = fmaf(w4.z, x[e + 2][q], acc);
            acc = fmaf(w4.w, x[e + 3][q], acc);
            if constexpr (ACT == kFP8) acc *= sc;
            c[e][q] = tb + e < L ? acc : 0.f;
        }
    }
}

// Index of (channel c, token t) in a [PD][PC] transposed tile whose 4-token
// chunks are permuted by channel bits 0-3 and 4-7, so that both the 16 lanes
// of a matrix-core lane group reading 4 consecutive tokens of 16 consecutive
// channels and the 16 lanes writing 4 tokens of channels 8 apart hit
// distinct LDS banks.
__device__ __forceinline__ int swz(int c, int t) {
    return c * PC + ((((t >> 2) ^ (c & 15) ^ ((c >> 4) & 15)) << 2) | (t & 3));
}

// Sum over each row of 16 lanes; every lane of the row gets the same value.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0x128>(x);   // row_ror:8
    x += dpp_mov<0x124>(x);   // row_ror:4
    x += dpp_mov<0x122>(x);   // row_ror:2
    x += dpp_mov<0x121>(x);   // row_ror:1
    return x;
}

// Sum over each half-wave of 32 lanes; every lane of the half gets the same
// value (the two rows' sums meet through a swizzle of lane ^ 16).
__device__ __forceinline__ float row32_sum(float x) {
    x = row16_sum(x);
    return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

__device__ __forceinline__ void ld4x2(const float* p0, const float* p1, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p0);
    const float4 b = *reinterpret_cast<const float4*>(p1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void st_frag(char* dst, int lane, const SplitOp& sp) {
    *reinterpret_cast<f16x8_t*>(dst + lane * 16) = sp.hi;
    *reinterpret_cast<f16x8_t*>(dst + 1024 + lane * 16) = sp.lo;
}

// ---------------------------------------------------------------- chunk

// Workgroup barrier for LDS data only: each wave waits for its own LDS
// accesses, not for its global loads and stores (no wave of the chunk kernel
// reads global memory another wave wrote), so stores to the workspace drain
// while the next step runs.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One (chunk, head) work item of the chunk kernel.  Chunk c of sequence s
// owns workspace slot floor(lo / 64) + s + c; item i is head i % H of slot
// n_slots - 1 - i / H, so later slots come first, and the few slots that no
// chunk owns (at most one per sequence) are the only items without work.
struct ChunkItem {
    int64_t idx;                     // -1: none left
    int cc, s, h, t0, L;
    SeqView v;
};

// The first item at index i, i + step, ... that has work.  The owner of a
// slot is the last sequence whose first slot is not above it (first slots
// grow with s when cu_seqlens is monotone); its bounds are then checked.
// `prev` (a checked item, or idx < 0) answers slots of its own sequence
// without any load.
// Workgroup-uniform values, stated as such: the direct-to-LDS loads' inline
// assembly elsewhere in the chunk kernel otherwise leads the compiler to keep
// the item search in vector registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni(int64_t x) {
    const uint64_t lo = (uint32_t)uni((int)(uint32_t)x), hi = (uint32_t)uni((int)(uint32_t)((uint64_t)x >> 32));
    return (int64_t)(lo | (hi << 32));
}
__device__ __forceinline__ ChunkItem uni(const ChunkItem& it) {
    return ChunkItem{uni(it.idx), uni(it.cc), uni(it.s), uni(it.h), uni(it.t0), uni(it.L),
                     SeqView{uni(it.v.lo), uni(it.v.len), uni(it.v.slot), uni(it.v.pos)}};
}

__device__ __forceinline__ ChunkItem next_item(const PrefillArgs& a, int n_slots, int64_t i,
                                               int64_t step, const ChunkItem& prev) {
    const int64_t total = (int64_t)n_slots * a.H;
    ChunkItem it;
    it.idx = -1;
    for (i = uni(i); i < total; i = uni(i + step)) {
        const int slot = n_slots - 1 - (int)(i / a.H);
        const int h = (int)(i % a.H);
        if (prev.idx >= 0) {
            const int cc = slot - (prev.v.lo / PC + prev.s);
            if (cc >= 0 && cc * PC < prev.v.len) {
                it = ChunkItem{i, cc, prev.s, h, cc * PC, min(PC, prev.v.len - cc * PC), prev.v};
                break;
            }
        }
        int lo = 0, hi = a.num_seqs - 1, s = -1;
        while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            if (sload_i32(a.cu_seqlens + mid) / PC + mid <= slot) {
                s = mid;
                lo = mid + 1;
            } else {
                hi = mid - 1;
            }
        }
        if (s < 0) continue;
        const int lo_t = sload_i32(a.cu_seqlens + s), hi_t = sload_i32(a.cu_seqlens + s + 1);
        const int slot_s = sload_i32(a.slot_ids + s), pos = sload_i32(a.positions + s);
        int bits;
        if (!seq_ok(a, lo_t, hi_t, slot_s, pos, bits)) continue;
        const SeqView v{lo_t, hi_t - lo_t, slot_s, pos};
        const int cc = slot - (v.lo / PC + s);
        if (cc < 0 || cc * PC >= v.len) continue;
        it = ChunkItem{i, cc, s, h, cc * PC, min(PC, v.len - cc * PC), v};
        break;
    }
    return it;
}

// A lane's raw inputs for one item: q, k, v for its seven conv tokens, alpha
// and beta (in the gate dtype) for its four tokens.
template <int ACT>
struct ChunkIn {
    Raw4<ACT> rq[7], rk[7], rv[7];
    Raw4<kGateAct<ACT>> ra[4];
    uint32_t rb[4];                  // bits, widened where used (no wait here)
    bool okm[3];                     // raw tokens tb-3..tb-1: false where they count as zero
};

// Part PART of a lane's raw inputs: 0 q, 1 k, 2 v with alpha and beta.  The
// three parts go out before three different steps, so that the loads pass
// the address units in turn, and only part of the next item's inputs
// occupies registers during step 2b, where the current item's products
// need the most; `okm` is set by part 0.
template <int ACT, int PART>
__device__ __forceinline__ void load_chunk_part(const PrefillArgs& a, const ChunkItem& it, int tb,
                                                int c0, ChunkIn<ACT>& in) {
    const int h = it.h, t0 = it.t0, L = it.L;
    Raw4<ACT>* dst = PART == 0 ? in.rq : (PART == 1 ? in.rk : in.rv);
    const void* src = PART == 0 ? a.q : (PART == 1 ? a.k : a.v);
    if (it.cc >= 1 && L == PC) {
        // Interior chunk: every conv token lies inside the sequence.  Each
        // load is a uniform row base plus one per-lane byte offset (lane's
        // first token, head and channels), so the addressing is scalar.
        constexpr int GACT = kGateAct<ACT>;
        constexpr size_t ESZ = kActSize<ACT>, GESZ = kActSize<GACT>;
        const size_t row_b = (size_t)a.qkv_rs * ESZ;             // bytes per q|k|v token row
        const int64_t row0 = (int64_t)it.v.lo + t0 - 3;          // token of conv tap 0, lane 0
        const uint32_t off = (uint32_t)((size_t)tb * row_b + ((size_t)h * PD + c0) * ESZ);
        const char* xb = static_cast<const char*>(src) + row0 * row_b;
#pragma unroll
        for (int m = 0; m < 7; ++m) dst[m] = ld_raw4_at<ACT>(xb + m * row_b, off);
        if constexpr (PART == 0) {
#pragma unroll
            for (int m = 0; m < 3; ++m) in.okm[m] = true;
        }
        if constexpr (PART == 2) {
            const size_t rowa_b = (size_t)a.H * PD * GESZ;       // bytes per alpha token row
            const uint32_t offa = (uint32_t)((size_t)tb * rowa_b + ((size_t)h * PD + c0) * GESZ);
            const char* ab = static_cast<const char*>(a.alpha) + (row0 + 3) * rowa_b;
            const char* bb = static_cast<const char*>(a.beta) + (row0 + 3) * (int64_t)a.H * GESZ;
            const uint32_t offb = (uint32_t)(((size_t)tb * a.H + h) * GESZ);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                in.ra[e] = ld_raw4_at<GACT>(ab + e * rowa_b, offa);
                in.rb[e] = GACT == kF32
                    ? *reinterpret_cast<const uint32_t*>(bb + e * a.H * GESZ + offb)
                    : *reinterpret_cast<const uint16_t*>(bb + e * a.H * GESZ + offb);
            }
        }
        return;
    }
#pragma unroll
    for (int m = 0; m < 7; ++m) {
        bool ok;
        dst[m] = raw4<ACT>(a, it.v, h, t0, L, tb - 3 + m, src, c0, PART * PD + c0, ok);
        if (PART == 0 && m < 3) in.okm[m] = ok;
    }
    if constexpr (PART == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // past the chunk's end: alpha = 1, beta = 0 (loads clamped to a valid token)
            const int64_t row = (int64_t)(it.v.lo + t0 + min(tb + e, L - 1)) * a.H + h;
            in.ra[e] = ld_raw4<kGateAct<ACT>>(a.alpha, row * PD + c0);
            in.rb[e] = ld_act_bits<kGateAct<ACT>>(a.beta, row);
        }
    }
}

template <int ACT>
__device__ __forceinline__ void load_chunk_in(const PrefillArgs& a, const ChunkItem& it, int tb,
                                              int c0, ChunkIn<ACT>& in) {
    load_chunk_part<ACT, 0>(a, it, tb, c0, in);
    load_chunk_part<ACT, 1>(a, it, tb, c0, in);
    load_chunk_part<ACT, 2>(a, it, tb, c0, in);
}

typedef __attribute__((address_space(3))) char lds_char_t;

// The conv taps of head h (q, k and v, 128 channels of four FP32 taps each:
// 6 KB) into LDS at dst as [tensor][channel] float4.  Waves 0-5 move 1 KB
// each, lane l 16 bytes, straight from global memory to LDS (M0 holds the
// wave's LDS destination); the caller waits for them (s_waitcnt vmcnt(0))
// before a barrier publishes them.
__device__ __forceinline__ void dma_taps(const PrefillArgs& a, int h, char* dst, int wave,
                                         int lane) {
    if (wave < 6) {
        const float* w = wave < 2 ? a.wq : (wave < 4 ? a.wk : a.wv);
        const char* src = reinterpret_cast<const char*>(w + ((size_t)h * PD + 64 * (wave & 1)) * kConvW);
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src + lane * 16), "{m0}"((lds_char_t*)(dst + 1024 * wave))
                     : "memory");
    }
}

// Threads of a chunk workgroup: eight waves, two per SIMD, so that one
// wave's LDS, matrix-core and memory latencies hide behind the other's
// vector work.
constexpr int kChunkThreads = 512;

template <int ACT>
__global__ __launch_bounds__(kChunkThreads) void prefill_chunk_kernel(PrefillArgs a, int n_slots) {
    // LDS regions (bytes), reused as the steps go:
    //   RA  kh * D4 [PC][LR]                    -> -W [PC][LR] (step 4)
    //   RB  qh * D4 [PC][LR]                    -> beta K_G transposed (step X)
    //   RC  kh * E4 [PC][LR]                    -> beta V transposed (step X)
    //   RD  A [PC][LS], T_bb on its diagonal blocks after step 3b
    //   RE  P [PC][LS]
    //   (RA, RB, RC and RE hold their values times 2^12, the matrix-core
    //   operand scale, which step 1 puts into the norm factors of q and k)
    //   RF  alpha product over each sub-block [NSB][PD]
    //   RG  step 2: per-wave suffix tables; from step 3a: prefix | suffix
    //       products over whole sub-blocks [2 NSB][PD]; from step X to the
    //       next item's step 1: that item's conv taps [3][PD] float4
    //   RH  beta [PC]
    // D4 = alpha over the sub-block start..t, E4 = alpha over t+1..sub-block end.
    constexpr int RA = 0, RB = RA + PC * LR * 4, RC = RB + PC * LR * 4;
    constexpr int RD = RC + PC * LR * 4, RE = RD + PC * LS * 4, RF = RE + PC * LS * 4;
    constexpr int RG = RF + NSB * PD * 4, RH = RG + 2 * NSB * PD * 4, LDS_B = RH + PC * 4;
    __shared__ __attribute__((aligned(16))) char lds[LDS_B];
    float (*KD)[LR] = reinterpret_cast<float (*)[LR]>(lds + RA);
    float (*QD)[LR] = reinterpret_cast<float (*)[LR]>(lds + RB);
    float (*KE)[LR] = reinterpret_cast<float (*)[LR]>(lds + RC);
    float (*Am)[LS] = reinterpret_cast<float (*)[LS]>(lds + RD);
    float (*Pm)[LS] = reinterpret_cast<float (*)[LS]>(lds + RE);
    float (*T4)[PD] = reinterpret_cast<float (*)[PD]>(lds + RF);
    float (*AUX)[PD] = reinterpret_cast<float (*)[PD]>(lds + RG);
    float* bet = reinterpret_cast<float*>(lds + RH);
    float (*Wn)[LR] = reinterpret_cast<float (*)[LR]>(lds + RA);
    float* RWt = reinterpret_cast<float*>(lds + RB);
    float* VT = reinterpret_cast<float*>(lds + RC);

    const int H = a.H;

    // Persistent: the workgroup takes items blockIdx.x, + gridDim.x, ...
    // The next item's inputs are requested in three parts (before steps 2b,
    // X and 4), after the current item's convolutions have consumed theirs,
    // and arrive by the next item's step 1.  Lane l of wave w handles tokens 4 (2w + l / 32) ..
    // + 3 and channels 4 (l % 32) .. + 3 in step 1.
    // The conv taps of an item go into RG by direct loads after the previous
    // item's step X (for the first item, here) and are read in step 1.
    ChunkItem it;
    ChunkIn<ACT> in;
    {
        const int tid = threadIdx.x, lane = tid & 63;
        // workgroup 0 validates every sequence once and reports the bad ones
        if (blockIdx.x == 0)
            for (int sq = tid; sq < a.num_seqs; sq += kChunkThreads) {
                SeqView sv;
                seq_view(a, sq, true, sv);
            }
        ChunkItem none;
        none.idx = -1;
        it = uni(next_item(a, n_slots, blockIdx.x, gridDim.x, none));
        if (it.idx < 0) return;
        load_chunk_in<ACT>(a, it, 4 * (tid >> 5), 4 * (lane & 31), in);
        dma_taps(a, it.h, lds + RG, __builtin_amdgcn_readfirstlane(tid >> 6), lane);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_sync();
    }
    for (;;) {
    // The thread index is passed through an empty assembly statement on each
    // item, so that the index arithmetic of every step is redone per item
    // instead of being hoisted out of the loop and held in registers.
    int tid_v = threadIdx.x;
    asm volatile("" : "+v"(tid_v));
    const int tid = tid_v, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int tb = 4 * (tid >> 5);             // this lane's sub-block (step 1): tokens tb..tb+3
    const int c0 = 4 * (lane & 31);            // and channels c0..c0+3
    const int h = it.h, L = it.L;
    const SeqView v = it.v;
    char* ws = static_cast<char*>(a.workspace) + ((size_t)chunk_slot(v.lo, it.s, it.cc) * H + h) * WS_B;
    ChunkItem nx;

    // ---- 1. per lane: sub-block tb / 4 (tokens tb..tb+3; half-wave h32 of
    // wave w holds sub-block 2w + h32), channels c0..c0+3: conv, L2 norms,
    // decay products, in-sub-block pairs
    float cv[4][4], bt[4];
    {
        float4 wtq[4], wtk[4], wtv[4];           // conv taps of the lane's channels
        {
            const float4* tp = reinterpret_cast<const float4*>(lds + RG);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wtq[q] = tp[c0 + q];
                wtk[q] = tp[PD + c0 + q];
                wtv[q] = tp[2 * PD + c0 + q];
            }
        }
        float qh[4][4], kh[4][4], al[4][4];
        conv4x4<ACT>(in.rq, in.okm, wtq, tb, L, a.scale_q, qh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float sq = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) sq = fmaf(qh[e][q], qh[e][q], sq);
            const float r = kSc * __builtin_amdgcn_rsqf(row32_sum(sq) + a.l2_eps);
#pragma unroll
            for (int q = 0; q < 4; ++q) qh[e][q] *= r;
        }
        conv4x4<ACT>(in.rk, in.okm, wtk, tb, L, a.scale_k, kh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float sk = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) sk = fmaf(kh[e][q], kh[e][q], sk);
            const float r = kSc * __builtin_amdgcn_rsqf(row32_sum(sk) + a.l2_eps);
#pragma unroll
            for (int q = 0; q < 4; ++q) kh[e][q] *= r;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool live = tb + e < L;
            unpack4<kGateAct<ACT>>(in.ra[e], al[e]);
            float bv = act_from_bits<kGateAct<ACT>>(in.rb[e]);
            if (a.gate_logits) {
#pragma unroll
                for (int q = 0; q < 4; ++q) al[e][q] = decay_from_logit(al[e][q]);
                bv = write_from_logit(bv);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) al[e][q] = live ? al[e][q] : 1.f;
            bt[e] = live ? bv : 0.f;
        }
        conv4x4<ACT>(in.rv, in.okm, wtv, tb, L, a.scale_v, cv);

        // every input of this item is consumed: find the next item (its
        // inputs are requested in three parts, from step 2b on)
        nx = uni(next_item(a, n_slots, it.idx + gridDim.x, gridDim.x, it));

        // pairs inside the sub-block: e(t, i) = alpha over i+1..t
        float pp[10], pa[6];
        {
            int ip = 0, ia = 0;
#pragma unroll
            for (int ei = 0; ei < 4; ++ei) {
                float d[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) d[q] = 1.f;
#pragma unroll
                for (int et = ei; et < 4; ++et) {
                    if (et > ei) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) d[q] *= al[et][q];
                    }
                    float sp = 0.f, sa = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float kd = kh[ei][q] * d[q];
                        sp = fmaf(qh[et][q], kd, sp);
                        sa = fmaf(kh[et][q], kd, sa);
                    }
                    pp[ip++] = row32_sum(sp);
                    if (et > ei) pa[ia++] = row32_sum(sa);
                }
            }
        }
        if ((lane & 31) == 0) {
            // 4x4 sub-tiles on the diagonal, zeros above
            int ip = 0, ia = 0;
            float P4[4][4], A4[4][4];
#pragma unroll
            for (int ei = 0; ei < 4; ++ei)
#pragma unroll
                for (int et = 0; et < 4; ++et) {
                    P4[et][ei] = 0.f;
                    A4[et][ei] = 0.f;
                }
#pragma unroll
            for (int ei = 0; ei < 4; ++ei)
#pragma unroll
                for (int et = ei; et < 4; ++et) {
                    P4[et][ei] = pp[ip++] * kInvSc;
                    if (et > ei) A4[et][ei] = bt[et] * (pa[ia++] * kInvSc2);
                }
#pragma unroll
            for (int et = 0; et < 4; ++et) {
                *reinterpret_cast<float4*>(&Pm[tb + et][tb]) =
                    make_float4(P4[et][0], P4[et][1], P4[et][2], P4[et][3]);
                *reinterpret_cast<float4*>(&Am[tb + et][tb]) =
                    make_float4(A4[et][0], A4[et][1], A4[et][2], A4[et][3]);
                bet[tb + et] = bt[et];
            }
        }

        // decay products inside the sub-block
        float D4[4][4], E4[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            D4[0][q] = al[0][q];
            E4[3][q] = 1.f;
        }
#pragma unroll
        for (int e = 1; e < 4; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q) D4[e][q] = D4[e - 1][q] * al[e][q];
#pragma unroll
        for (int e = 2; e >= 0; --e)
#pragma unroll
            for (int q = 0; q < 4; ++q) E4[e][q] = E4[e + 1][q] * al[e + 1][q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<float4*>(&KD[tb + e][c0]) = make_float4(
                kh[e][0] * D4[e][0], kh[e][1] * D4[e][1], kh[e][2] * D4[e][2], kh[e][3] * D4[e][3]);
            *reinterpret_cast<float4*>(&QD[tb + e][c0]) = make_float4(
                qh[e][0] * D4[e][0], qh[e][1] * D4[e][1], qh[e][2] * D4[e][2], qh[e][3] * D4[e][3]);
            *reinterpret_cast<float4*>(&KE[tb + e][c0]) = make_float4(
                kh[e][0] * E4[e][0], kh[e][1] * E4[e][1], kh[e][2] * E4[e][2], kh[e][3] * E4[e][3]);
        }
        *reinterpret_cast<float4*>(&T4[tb >> 2][c0]) =
            make_float4(D4[3][0], D4[3][1], D4[3][2], D4[3][3]);
    }
    lds_sync();

    // ---- 2a. suffix tables of row blocks rb = 1..3: AUX[2 rb (rb - 1) + j]
    // = alpha over sub-blocks j+1 .. 4 rb - 1, for j < 4 rb (the column
    // factors of the tiles left of the diagonal block).  Waves 1..6 take
    // row block 1 + (w - 1) / 2, channel half (w - 1) % 2.
    if (wave >= 1 && wave <= 6) {
        const int rbk = 1 + ((wave - 1) >> 1);
        const int aux_o = 2 * rbk * (rbk - 1), nj = 4 * rbk;
        const int c = lane + 64 * ((wave - 1) & 1);
        float t4v[12];
#pragma unroll
        for (int jj = 0; jj < 12; ++jj) t4v[jj] = T4[jj][c];   // all reads in flight at once
        float run = 1.f;
#pragma unroll
        for (int jj = 11; jj >= 0; --jj) {
            if (jj < nj) {
                AUX[aux_o + jj][c] = run;
                run *= t4v[jj];
            }
        }
    }
    lds_sync();

    // The next item's inputs go out in three parts: q here, k before step X,
    // v, alpha and beta before step 4.  The first is requested here rather
    // than right after the convolutions: by now the previous item's
    // workspace stores have drained, and the loads still have steps 2b-5 to
    // arrive.
    if (nx.idx >= 0) load_chunk_part<ACT, 0>(a, nx, tb, c0, in);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2b. cross-sub-block entries of A and P on the matrix cores.
    // Waves 0-3: the diagonal 16x16 block of row block w.  Adjacent
    // sub-blocks go through their common boundary ("adj"), sub-blocks two or
    // three apart through the boundary before local sub-block 2 ("J2").
    // Waves 4-7: the tiles left of the diagonal, through the row block's
    // first boundary: wave 4 takes (2,0) and (2,1), wave 5 (3,0) and (3,1),
    // wave 6 (3,2), wave 7 (1,0).
    if (wave < 4) {
        const int t = 16 * wave + n;              // A-operand row of this lane
        const int i = 16 * wave + n;              // B-operand column of this lane
        f32x4_t aA1 = {0.f, 0.f, 0.f, 0.f}, aP1 = aA1, aA2 = aA1, aP2 = aA1;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int cb = 32 * kb + 8 * g;
            float rk[8], rq[8], ck[8], f3[8], f1[8];
            ld4x2(&KD[t][cb], &KD[t][cb + 4], rk);
            ld4x2(&QD[t][cb], &QD[t][cb + 4], rq);
            ld4x2(&KE[i][cb], &KE[i][cb + 4], ck);
            ld4x2(&T4[4 * wave + 2][cb], &T4[4 * wave + 2][cb + 4], f3);
            ld4x2(&T4[4 * wave + 1][cb], &T4[4 * wave + 1][cb + 4], f1);
            float rk2[8], rq2[8], ck2[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float fr = n >= 12 ? f3[q] : 1.f;
                const float fc = n < 4 ? f1[q] : 1.f;
                rk2[q] = rk[q] * fr;
                rq2[q] = rq[q] * fr;
                ck2[q] = ck[q] * fc;
            }
            const SplitOp sck = split_op(ck), sck2 = split_op(ck2);
            aA1 = mma3(split_op(rk), sck, aA1);
            aP1 = mma3(split_op(rq), sck, aP1);
            aA2 = mma3(split_op(rk2), sck2, aA2);
            aP2 = mma3(split_op(rq2), sck2, aP2);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tl = 4 * g + r, jtl = g, jil = n >> 2;
            if (jil < jtl) {
                const bool adj = jtl - jil == 1;
                Am[16 * wave + tl][16 * wave + n] =
                    bet[16 * wave + tl] * ((adj ? aA1[r] : aA2[r]) * kInvSc2);
                Pm[16 * wave + tl][16 * wave + n] = (adj ? aP1[r] : aP2[r]) * kInvSc;
            } else if (jil > jtl) {
                Am[16 * wave + tl][16 * wave + n] = 0.f;
                Pm[16 * wave + tl][16 * wave + n] = 0.f;
            }
        }
        // tiles right of the diagonal block are zero
        for (int bi = wave + 1; bi < 4; ++bi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Am[16 * wave + 4 * g + r][16 * bi + n] = 0.f;
                Pm[16 * wave + 4 * g + r][16 * bi + n] = 0.f;
            }
        __builtin_amdgcn_sched_barrier(0);
    } else {
        const int rb = wave == 4 ? 2 : (wave == 7 ? 1 : 3);     // row block
        const int bi0 = wave == 6 ? 2 : 0;
        const int bi1 = wave <= 5 ? 2 : (wave == 6 ? 3 : 1);    // exclusive
        {
            // row operand: scaled to the row block's first token
            const int tr0 = 16 * rb + n;
            const int jtl = n >> 2;
            const int aux_rb = 2 * rb * (rb - 1);              // row block rb's suffix table
            SplitOp xk[4], xq[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int cb = 32 * kb + 8 * g;
                float rk[8], rq[8], t0f[8], t1f[8], t2f[8];
                ld4x2(&KD[tr0][cb], &KD[tr0][cb + 4], rk);
                ld4x2(&QD[tr0][cb], &QD[tr0][cb + 4], rq);
                ld4x2(&T4[4 * rb][cb], &T4[4 * rb][cb + 4], t0f);
                ld4x2(&T4[4 * rb + 1][cb], &T4[4 * rb + 1][cb + 4], t1f);
                ld4x2(&T4[4 * rb + 2][cb], &T4[4 * rb + 2][cb + 4], t2f);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    float f = jtl >= 1 ? t0f[q] : 1.f;
                    f *= jtl >= 2 ? t1f[q] : 1.f;
                    f *= jtl >= 3 ? t2f[q] : 1.f;
                    rk[q] *= f;
                    rq[q] *= f;
                }
                xk[kb] = split_op(rk);
                xq[kb] = split_op(rq);
            }
            __builtin_amdgcn_sched_barrier(0);
            for (int bi = bi0; bi < bi1; ++bi) {
                const int ic = 16 * bi + n;
                const int ji = ic >> 2;
                f32x4_t A = {0.f, 0.f, 0.f, 0.f}, P = A;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int cb = 32 * kb + 8 * g;
                    float ck[8], sf[8];
                    ld4x2(&KE[ic][cb], &KE[ic][cb + 4], ck);
                    ld4x2(&AUX[aux_rb + ji][cb], &AUX[aux_rb + ji][cb + 4], sf);
#pragma unroll
                    for (int q = 0; q < 8; ++q) ck[q] *= sf[q];
                    const SplitOp sck = split_op(ck);
                    A = mma3(xk[kb], sck, A);
                    P = mma3(xq[kb], sck, P);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 16 * rb + 4 * g + r;
                    Am[tr][ic] = bet[tr] * (A[r] * kInvSc2);
                    Pm[tr][ic] = P[r] * kInvSc;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();

    // ---- 3a. prefix / suffix products over whole sub-blocks, and the
    // chunk's total decay
    if (tid < PD) {
        float run = 1.f;
#pragma unroll
        for (int jj = 0; jj < NSB; ++jj) {
            AUX[jj][tid] = run;
            run *= T4[jj][tid];
        }
        reinterpret_cast<float*>(ws + GAM_OFF)[tid] = run;
    } else if (tid < 2 * PD) {
        const int c = tid - PD;
        float run = 1.f;
#pragma unroll
        for (int jj = NSB - 1; jj >= 0; --jj) {
            AUX[NSB + jj][c] = run;
            run *= T4[jj][c];
        }
    }
    lds_sync();

    // ---- 3b. wave 0: T_bb = (I + A_bb)^-1 for the four diagonal blocks,
    // in place (lane = block * 16 + column).  Waves 1..7: the scaled-Q,
    // scaled-K and P fragments to the workspace, five or six each.
    // (e(t,-1) * qh) rows, A operand
    auto q_frag = [&](int f) {
        const int tt = f >> 2, kb = f & 3;
        const int t = 16 * tt + n, cb = 32 * kb + 4 * g;
        float qd[8], pr[8], x[8];
        ld4x2(&QD[t][cb], &QD[t][cb + 16], qd);
        ld4x2(&AUX[t >> 2][cb], &AUX[t >> 2][cb + 16], pr);
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = qd[q] * pr[q];
        st_frag(ws + (tt >> 1) * HALF_B + frag_q(tt & 1, kb) * FRAG_B, lane, split_op(x));
    };
    // (e(last,t) * kh)^T, A operand
    auto k_frag = [&](int f) {
        const int ct = f & 7, kb = f >> 3;
        const int c = 16 * ct + n;
        float x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int ts = 32 * kb + kslot(g, q);
            x[q] = KE[ts][c] * AUX[NSB + (ts >> 2)][c];
        }
        st_frag(ws + kb * HALF_B + frag_k(ct) * FRAG_B, lane, split_op(x));
    };
    // P rows, A operand: the two tiles of half 0 and the four of half 1
    auto p_frag = [&](int p) {
        const int hh = p >= 2, u = hh ? (p - 2) >> 1 : p, kb = hh ? (p & 1) : 0;
        const int tt = 2 * hh + u, t = 16 * tt + n, cb = 32 * kb + 4 * g;
        float xp[8];
        ld4x2(&Pm[t][cb], &Pm[t][cb + 16], xp);
        st_frag(ws + hh * HALF_B + frag_p(hh, u, kb) * FRAG_B, lane, split_op(xp));
    };
    if (wave == 0) {
        const int b = lane >> 4, ic = lane & 15;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = 0.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int s4 = 0; s4 < t; s4 += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(&Am[16 * b + t][16 * b + s4]);
                acc = fmaf(a4.x, x[s4], acc);
                acc = fmaf(a4.y, x[s4 + 1], acc);
                acc = fmaf(a4.z, x[s4 + 2], acc);
                acc = fmaf(a4.w, x[s4 + 3], acc);
            }
            x[t] = t < ic ? 0.f : (t == ic ? 1.f : -acc);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) Am[16 * b + t][16 * b + ic] = x[t];
    } else {
        // Wave w takes scaled-Q fragments w-1, w+6, w+13, scaled-K fragments
        // (w+1) mod 7 + 0, 7, 14 (those below 16), and waves 3-5 two P
        // fragments each: 5 or 6 fragments per wave.  The guards are
        // uniform, and the first two of each kind are unconditional so that
        // their LDS reads overlap.
        const int wq = wave - 1, wk = (wave + 1) % 7;
        q_frag(wq);
        q_frag(wq + 7);
        if (wq + 14 < 16) q_frag(wq + 14);
        k_frag(wk);
        k_frag(wk + 7);
        if (wk + 14 < 16) k_frag(wk + 14);
        if (wave >= 3 && wave <= 5) {
            p_frag(2 * (wave - 3));
            p_frag(2 * (wave - 3) + 1);
        }
    }
    lds_sync();

    // The next item's k inputs (its q inputs went out before step 2b, its
    // v, alpha and beta go out before step 4): requested outside step 2b's
    // register peak.
    if (nx.idx >= 0) load_chunk_part<ACT, 1>(a, nx, tb, c0, in);
    // ---- X. beta_t K_G = beta_t kh_t e(t,-1) and beta_t V, transposed to
    // [channel][token] (swizzled) so that the solve reads 4 tokens at once
    {
        const int c = tid & (PD - 1), th = tid >> 7;   // tokens 16 th .. 16 th + 15
        float kd[4][4], bq[4][4], pre[4];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int t = 16 * th + 4 * t4;
            pre[t4] = AUX[t >> 2][c];
            const float4 b4 = *reinterpret_cast<const float4*>(&bet[t]);
            bq[t4][0] = b4.x; bq[t4][1] = b4.y; bq[t4][2] = b4.z; bq[t4][3] = b4.w;
#pragma unroll
            for (int e = 0; e < 4; ++e) kd[t4][e] = KD[t + e][c];
        }
        // every read above is issued before the first write below (the
        // compiler cannot tell the written region from the ones read, and
        // would otherwise wait for each read before the next write)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int t = 16 * th + 4 * t4;
            *reinterpret_cast<float4*>(&RWt[swz(c, t)]) =
                make_float4(bq[t4][0] * kd[t4][0] * pre[t4], bq[t4][1] * kd[t4][1] * pre[t4],
                            bq[t4][2] * kd[t4][2] * pre[t4], bq[t4][3] * kd[t4][3] * pre[t4]);
        }
        float bs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bs[e] = bt[e] * kSc;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(&VT[swz(c0 + q, tb)]) =
                make_float4(bs[0] * cv[0][q], bs[1] * cv[1][q], bs[2] * cv[2][q], bs[3] * cv[3][q]);
    }
    lds_sync();

    // the next item's conv taps into RG (free until the next item's step
    // 2a); waited for in step 4, before its stores
    if (nx.idx >= 0) dma_taps(a, nx.h, lds + RG, wave, lane);

    // the next item's v, alpha and beta inputs
    if (nx.idx >= 0) load_chunk_part<ACT, 2>(a, nx, tb, c0, in);
    // ---- 4. [W | Ut] = T (diag(beta) [K_G | V]) by block forward
    // substitution: X_b = T_bb (R_b - sum_{a<b} A_ba X_a).  Wave w owns one
    // column tile of each: u = 0 the W tile of key channels 16w..16w+15, u = 1
    // the Ut tile of value channels 16w..16w+15, so the two waves of a SIMD
    // carry the same work.
    {
        constexpr int NU = 2;
        const int cw = 16 * wave + n;             // the lane's column in both tiles
        // Value columns: the solve runs on R scaled by the column's power-of-
        // two scale (largest |beta v| over the chunk in [1, 2)); X comes out
        // scaled by the same factor and is unscaled on its way out.
        float sgv, isgv;
        {
            float m = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const f32x4_t r4 = *reinterpret_cast<const f32x4_t*>(&VT[swz(cw, 16 * b + 4 * g)]);
                m = fmaxf(m, fmaxf(fmaxf(fabsf(r4[0]), fabsf(r4[1])),
                                   fmaxf(fabsf(r4[2]), fabsf(r4[3]))));
            }
            pow2_scale(col_max4(m) * kInvSc, sgv, isgv);
        }
        f32x4_t X[4][NU];
        SplitOp4 Xs[3][NU];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x4_t acc[NU];
            acc[0] = *reinterpret_cast<const f32x4_t*>(&RWt[swz(cw, 16 * b + 4 * g)]);
            acc[1] = *reinterpret_cast<const f32x4_t*>(&VT[swz(cw, 16 * b + 4 * g)]) * sgv;
            if (b == 1) {
                const float4 a4 = *reinterpret_cast<const float4*>(&Am[16 + n][4 * g]);
                const float av[4] = {-a4.x * kSc, -a4.y * kSc, -a4.z * kSc, -a4.w * kSc};
                const SplitOp4 sa = split_op4(av);
#pragma unroll
                for (int u = 0; u < NU; ++u) acc[u] = mma3(sa, Xs[0][u], acc[u]);
            } else if (b >= 2) {
                float av[8];
                ld4x2(&Am[16 * b + n][4 * g], &Am[16 * b + n][16 + 4 * g], av);
#pragma unroll
                for (int q = 0; q < 8; ++q) av[q] = -av[q] * kSc;
                const SplitOp sa = split_op(av);
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    SplitOp xb;
                    xb.hi = __builtin_shufflevector(Xs[0][u].hi, Xs[1][u].hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    xb.lo = __builtin_shufflevector(Xs[0][u].lo, Xs[1][u].lo, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[u] = mma3(sa, xb, acc[u]);
                }
                if (b == 3) {
                    const float4 a4 = *reinterpret_cast<const float4*>(&Am[48 + n][32 + 4 * g]);
                    const float a3[4] = {-a4.x * kSc, -a4.y * kSc, -a4.z * kSc, -a4.w * kSc};
                    const SplitOp4 sa3 = split_op4(a3);
#pragma unroll
                    for (int u = 0; u < NU; ++u) acc[u] = mma3(sa3, Xs[2][u], acc[u]);
                }
            }
            const float4 t4 = *reinterpret_cast<const float4*>(&Am[16 * b + n][16 * b + 4 * g]);
            const float tv[4] = {t4.x * kScW, t4.y * kScW, t4.z * kScW, t4.w * kScW};
            const SplitOp4 st = split_op4(tv);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                X[b][u] = mma3(st, split_op4(acc[u] * kInvSc), f32x4_t{0.f, 0.f, 0.f, 0.f}) * kInvScW;
                if (b < 3) Xs[b][u] = split_op4(X[b][u]);
            }
        }
        // the W tile to LDS (negated), the Ut tile to the workspace.  First
        // the wait for the taps' direct loads, issued before this step, so
        // that it never waits behind this step's stores; the loop's last
        // barrier then publishes them.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) Wn[16 * b + 4 * g + r][cw] = -X[b][0][r];
        float m = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int hh = b >> 1, uu = b & 1;
            const f32x4_t x = X[b][1] * isgv;
            *reinterpret_cast<f32x4_t*>(ws + UT_OFF +
                                        ((((hh * 8 + wave) * 2 + uu) * 64 + lane) * 16)) = x;
            m = fmaxf(m, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
        }
        // the column's largest |Ut| over the chunk, for the state pass's scale
        m = col_max4(m);
        if (g == 0) reinterpret_cast<float*>(ws + UTMAX_OFF)[cw] = m;
    }
    lds_sync();

    // ---- 5. -W fragments (A operand, k = key channel in pairing order)
#pragma unroll
    for (int k4 = 0; k4 < 2; ++k4) {
        const int f = wave + 8 * k4;
        const int tt = f >> 2, kb = f & 3;
        const int t = 16 * tt + n, cb = 32 * kb + 4 * g;
        float x[8];
        ld4x2(&Wn[t][cb], &Wn[t][cb + 16], x);
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] *= kScW;
        st_frag(ws + (tt >> 1) * HALF_B + frag_w(tt & 1, kb) * FRAG_B, lane, split_op(x));
    }
    if (nx.idx < 0) break;
    lds_sync();                                // step 5's reads before the next step 1's writes
    it = nx;
    }
}

// ---------------------------------------------------------------- state

__device__ __forceinline__ SplitOp ld_frag(const char* buf, int f, int lane) {
    SplitOp o;
    o.hi = *reinterpret_cast<const f16x8_t*>(buf + f * FRAG_B + lane * 16);
    o.lo = *reinterpret_cast<const f16x8_t*>(buf + f * FRAG_B + 1024 + lane * 16);
    return o;
}

// body(P) for the three passes P = 0, 1, 2 of a split product.
template <class F>
__device__ __forceinline__ void three_passes(F&& body) {
    body(std::integral_constant<int, 0>{});
    body(std::integral_constant<int, 1>{});
    body(std::integral_constant<int, 2>{});
}

__device__ __forceinline__ void put_split(f16x8_t* hi, f16x8_t* lo, int lane, const SplitOp& x) {
    hi[lane] = x.hi;
    lo[lane] = x.lo;
}
__device__ __forceinline__ SplitOp get_split(const f16x8_t* hi, const f16x8_t* lo, int lane) {
    return SplitOp{hi[lane], lo[lane]};
}

// One-way hand-offs between the state pass's waves through LDS flags: a U/S
// wave publishes a chunk's split U and the O waves poll before reading it;
// an O wave publishes once it has read the chunk's split state, and the U/S
// waves poll before overwriting it.  The writer writes, waits for those
// writes, then stores the chunk's number plus one (never 0) in its flag.
// Each wait is for work its own workgroup does in the same chunk, between
// the same two barriers, so no hand-off can block.  The poll is bounded all
// the same: await_half returns false when the flag never arrived, and the
// kernel then reports KDA_STATUS_STALLED.
// The flag is accessed through an LDS-typed pointer: through a generic one
// the volatile access becomes a flat store, which also counts as a vector
// memory operation and makes the compiler wait for every outstanding load.
typedef __attribute__((address_space(3))) volatile int lds_vint_t;
__device__ __forceinline__ void publish_half(int* flag, int epoch) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    *(lds_vint_t*)flag = epoch;
}
__device__ __forceinline__ bool await_half(int* flag, int epoch) {
    bool ok = false;
    for (int spin = 0; spin < (1 << 22); ++spin) {
        const int f = __builtin_amdgcn_readfirstlane(*(lds_vint_t*)flag);
        if (f == epoch) {
            ok = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    return ok;
}

// A fragment straight from the workspace (same layout as in LDS).
__device__ __forceinline__ SplitOp ld_frag_g(const char* half, int f, int lane) {
    SplitOp o;
    o.hi = *reinterpret_cast<const f16x8_t*>(half + f * FRAG_B + lane * 16);
    o.lo = *reinterpret_cast<const f16x8_t*>(half + f * FRAG_B + 1024 + lane * 16);
    return o;
}

// A chunk's operands of the state chain in LDS: the -W and scaled-K
// fragments of both halves and the chunk's total decay and largest |Ut|,
// 65 pieces of 1 KB.  Layout: [half h][-W (16 KB) | scaled K (16 KB)] for
// h = 0, 1, then the 1 KB of decay and |Ut| maxima.
constexpr int CB_PIECES = 65;
constexpr int CB_B = CB_PIECES * 1024;
constexpr int CB_G = 64 * 1024;                   // decay [PD] FP32, then |Ut| maxima [PD]
__device__ __forceinline__ int cb_w(int h) { return h * 32768; }
__device__ __forceinline__ int cb_k(int h) { return h * 32768 + 16384; }

// Workspace byte offset of LDS piece p of a chunk (see the layout above):
// -W is fragments 0-7 of a half, scaled K fragments 16-23, and the decay and
// maxima sit at GAM_OFF of half 0.
__device__ __forceinline__ int cb_src(int p) {
    if (p == 64) return GAM_OFF;
    const int h = p >> 5, q = p & 31;
    return h * HALF_B + (q < 16 ? q * 1024 : 32768 + (q - 16) * 1024);
}

// One chunk's chain operands into an LDS buffer, loader wave lw (0, 1)
// taking every other piece; lane l moves 16 bytes straight from global
// memory to LDS.  Issued as inline assembly: the compiler would otherwise
// wait for these loads before every LDS read of the other buffer.  The
// loaders wait for them with counted s_waitcnt vmcnt before the barrier
// that publishes the buffer.
__device__ __forceinline__ void dma_chunk(const char* ws, char* dst, int lw, int lane) {
#pragma unroll
    for (int q = 0; q < (CB_PIECES + 1) / 2; ++q) {
        const int piece = lw + 2 * q;
        if (piece < CB_PIECES)
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                         :
                         : "v"(ws + cb_src(piece) + lane * 16),
                           "{m0}"((lds_char_t*)(dst + piece * 1024))
                         : "memory");
    }
}
// Loads issued by loader wave lw in dma_chunk: 33 for lw = 0, 32 for lw = 1.

// Pulls a later chunk into the L2: one 4-byte load per 128-byte line of its
// fragments (both halves, 896 lines) and of the workgroup's 8 KB of Ut (64
// lines), eight loads per lane of the two loader waves, aimed at a small LDS
// sink whose contents are never read.  The DMA of the chain operands and
// the O waves' and U/S waves' direct loads then find their lines in the L2.
// ut is the workgroup's Ut of half 0 (4 KB); half 1's lies 16 KB further.
constexpr int kPrefetchLoads = 8;
__device__ __forceinline__ void prefetch_chunk_lines(const char* ws, const char* ut, char* sink,
                                                     int lw, int lane) {
#pragma unroll
    for (int q = 0; q < kPrefetchLoads; ++q) {
        const int line = lw * 64 + lane + 128 * q;               // 0..1023
        const int fl = 2 * HALF_B / 128;                          // 896 fragment lines
        const int ul = min(line - fl, 63);                        // Ut lines: 32 per half
        const char* src = line < fl ? ws + line * 128 : ut + (ul >> 5) * 16384 + (ul & 31) * 128;
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off"
                     :
                     : "v"(src), "{m0}"((lds_char_t*)(sink + lw * 256))
                     : "memory");
    }
}

// acc[j] += sum over the four 32-deep k blocks of fa[kb] * b[j][kb] for two
// column tiles j, one accumulator per (pass, tile): six independent chains.
// The hi*hi pass starts from acc.
__device__ __forceinline__ void prod4x2(const SplitOp (&fa)[4], const SplitOp (&b)[2][4],
                                        f32x4_t (&acc)[2]) {
    f32x4_t pa[3][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        pa[0][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        pa[1][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        pa[2][j] = acc[j];
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        three_passes([&](auto P) {
            constexpr int pp = decltype(P)::value;
#pragma unroll
            for (int j = 0; j < 2; ++j) pa[pp][j] = mma_pass<pp>(fa[kb], b[j][kb], pa[pp][j]);
        });
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = pa[2][j] + pa[1][j] + pa[0][j];
}

// Split operands the state pass's waves share through LDS, for the
// workgroup's two 16-column tiles: the chunk's start state as the B operand
// (k = key channel, four 32-deep blocks) and both halves' U (k = token).
struct StateX {
    f16x8_t sb_hi[2][4][64], sb_lo[2][4][64];     // [column tile][k block]
    f16x8_t ub_hi[2][2][64], ub_lo[2][2][64];     // [half][column tile]
};

constexpr int kStateThreads = 384;

// State pass.  Four workgroups per (sequence, head), 32 value columns (two
// 16-column tiles) each, six waves: two U/S waves, two O waves and two
// loader waves, one barrier per chunk.
//
// The loader waves stream each chunk's chain operands (-W and scaled K of
// both halves, the decay, the |Ut| maxima) into one of two LDS buffers by
// direct loads, a chunk ahead of its use, and pull the chunk after that into
// the L2.  The O waves and U/S waves read their other operands (scaled Q and
// P fragments, Ut) straight from the workspace, where those prefetches have
// put them in the L2.
//
// U/S wave j (0, 1) holds value-column tile j of the state for all 128 key
// channels and updates it once per chunk: U = Ut - W S for all 64 tokens of
// the chunk from the chunk's start state, then S <- Diag(gamma) S + Kc^T U.
// The MFMA output layout of a half's two U row tiles is, lane for lane and
// in order, the B operand the update takes (the scaled-K fragments are
// stored in that pairing order), so U stays in registers and the two U/S
// waves exchange nothing.  Each U/S wave leaves its split U in LDS for the
// O waves and sets its flag.
//
// O wave r computes row tile r of both halves' O = Qg S + P U for both
// column tiles and stores it, one chunk late.  It publishes a flag once it
// has read the chunk's split start state and scales, and the U/S waves wait
// for it before they overwrite them with the next chunk's.
//
// Value columns carry power-of-two scales (pow2_scale).  Each U/S wave
// splits the chunk's start state scaled by its column maxima, and leaves
// those maxima in LDS beside the split blocks.  U and O are accumulated at
// the chunk's column scale (the larger of the state's maxima and the
// chunk's largest |Ut|), the state products brought to it by an exact power
// of two.  S is held unscaled between chunks.
template <int ACT, int ST>
__global__ __launch_bounds__(kStateThreads) void prefill_state_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) char cbuf[2][CB_B];
    __shared__ StateX X;
    __shared__ int xflag[2];                      // per U/S wave: last chunk whose U is published
    __shared__ int oflag[2];                      // per O wave: last chunk whose split state is read
    __shared__ float xmax[2][16];                 // [column tile][column]: largest |S|
    __shared__ __attribute__((aligned(16))) char pf_sink[2 * 256];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: role branches are scalar
    const int n = lane & 15, g = lane >> 4;
    const int r = wave & 1;                       // U/S column tile; O row tile; loader index
    const int H = a.H;
    if (tid < 2) xflag[tid] = 0;
    if (tid >= 2 && tid < 4) oflag[tid - 2] = 0;
    lds_sync();                                   // the flags before any wave uses them
    // The chunk buffers are filled only by assembly loads; this store, which
    // never runs (num_seqs >= 1), keeps the compiler from treating them as
    // never written.
    if (a.num_seqs < 0) cbuf[0][tid] = cbuf[1][tid] = 0;
    // the column groups of one (sequence, head) sit eight workgroups apart,
    // so they land on the same XCD and share its L2
    const int G = a.num_seqs * H;
    const int rr = (int)(blockIdx.x % 32);
    const int grp = rr >> 3;
    const int p = (int)(blockIdx.x / 32) * 8 + (rr & 7);
    if (p >= G) return;
    const int s = p / H, h = p % H;
    SeqView v;
    if (!seq_view(a, s, false, v)) return;
    if (v.len == 0) return;
    int jc[2];                                    // the lane's value column in each tile
    jc[0] = 32 * grp + n;
    jc[1] = 32 * grp + 16 + n;
    const size_t head_off = ((size_t)v.slot * H + h) * PD * PD;
    const int nch = (v.len + PC - 1) / PC;

    auto cws = [&](int c) -> const char* {
        return static_cast<const char*>(a.workspace) +
               ((size_t)chunk_slot(v.lo, s, c) * H + h) * WS_B;
    };
    // this workgroup's Ut of chunk c: half hh, column tile j, row tile rt
    auto ut_tile = [&](int c, int hh, int j, int rt) -> const char* {
        return cws(c) + UT_OFF + ((((hh * 8 + 2 * grp + j) * 2 + rt) * 64) * 16);
    };

    if (wave >= 4) {
        // ---------------------------------------------------------- loaders
        const int lw = r;
        dma_chunk(cws(0), cbuf[0], lw, lane);
        int npf = 0;                              // prefetch loads issued after the last DMA
        if (nch > 1) {
            prefetch_chunk_lines(cws(1), ut_tile(1, 0, 0, 0), pf_sink, lw, lane);
            npf = kPrefetchLoads;
        }
        for (int cc = 0; cc < nch; ++cc) {
            // the DMA of chunk cc has landed; prefetches issued after it
            // (loads complete in order) may stay in flight
            if (npf == kPrefetchLoads)
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_sync();                           // chunk cc may be read
            if (cc + 1 < nch) dma_chunk(cws(cc + 1), cbuf[(cc + 1) & 1], lw, lane);
            npf = 0;
            if (cc + 2 < nch) {
                prefetch_chunk_lines(cws(cc + 2), ut_tile(cc + 2, 0, 0, 0), pf_sink, lw, lane);
                npf = kPrefetchLoads;
            }
        }
    } else if (wave < 2) {
        // ---------------------------------------------------------- U/S wave
        // U/S wave jw owns value-column tile jw (the lane's column jc[jw]) of
        // the state over all 128 key channels: S[i] is channel tile i
        // (channels 16 i + 4 g + e).  Its U of both row tiles of a half lands
        // in the lanes and order the update's B operand takes, so the two
        // U/S waves exchange nothing.
        const int jw = r;
        f32x4_t S[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (v.pos > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t el = head_off + (size_t)(16 * i + 4 * g + e) * PD + jc[jw];
                    S[i][e] = ST == kF32 ? static_cast<const float*>(a.pool)[el]
                                         : bf16_to_f32(static_cast<const uint16_t*>(a.pool)[el]);
                }
        }
        bool stalled = false;
        // the split scale: the largest |S| of each value column, left in LDS
        // for the O waves
        float xo, so, iso;
        auto own_scale = [&]() {
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) x = fmaxf(x, fabsf(S[i][e]));
            x = col_max4(x);
            xo = x;
            if (g == 0) xmax[jw][n] = x;
            pow2_scale(x, so, iso);
        };
        // the B operands of the U products (k block kb: channel tiles 2 kb,
        // 2 kb + 1), also left in LDS for the O waves
        SplitOp sb[4];
        auto make_own = [&]() {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                sb[kb] = split_pair(S[2 * kb] * so, S[2 * kb + 1] * so);
                put_split(X.sb_hi[jw][kb], X.sb_lo[jw][kb], lane, sb[kb]);
            }
        };
        own_scale();
        make_own();
        // the chunk's column scale sg (the largest of |S| and the chunk's
        // |Ut|) and the factor that brings the state products to it (a power
        // of two, at most 1)
        float sg, isg, rown;
        auto set_scale = [&](const char* buf) {
            const float* utm = reinterpret_cast<const float*>(buf + CB_G) + PD;
            pow2_scale(fmaxf(xo, utm[jc[jw]]), sg, isg);
            rown = sg * iso;
        };
        // the chunk's Ut of this column tile: [half][row tile], loaded a
        // chunk ahead
        f32x4_t ut[2][2], utn[2][2];
        auto ld_ut = [&](int c, f32x4_t (&u)[2][2]) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    u[hh][rt] = *reinterpret_cast<const f32x4_t*>(ut_tile(c, hh, jw, rt) + lane * 16);
        };
        ld_ut(0, ut);
        // One chunk of the chain: U of both halves (accumulated at 2^8 times
        // the column scale) from the chunk's start state, split (the update's
        // B operand, and in LDS for the O waves), then S += Kc^T U over both
        // halves and all 128 channels (at 2^12; Sn holds the decayed start
        // state).  Both halves' U products are issued before either half is
        // finished, and the first half's update before the second half's U
        // is finished, so that vector work runs under matrix instructions.
        auto chain = [&](const char* buf, f32x4_t (&Sn)[8], int epoch) {
            f32x4_t pa[2][3][2];                  // [half][pass][row tile]
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                SplitOp w[2][4];
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) w[u][kb] = ld_frag(buf + cb_w(hh), frag_w(u, kb), lane);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    pa[hh][0][u] = pa[hh][1][u] = pa[hh][2][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    three_passes([&](auto P) {
                        constexpr int pp = decltype(P)::value;
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            pa[hh][pp][u] = mma_pass<pp>(w[u][kb], sb[kb], pa[hh][pp][u]);
                    });
            }
            SplitOp ub[2];
            auto finish_u = [&](int hh) {
                f32x4_t uu[2];
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    uu[u] = (ut[hh][u] * (kScW * sg) +
                             (pa[hh][2][u] + pa[hh][1][u] + pa[hh][0][u]) * rown) * kInvScW;
                ub[hh] = split_pair(uu[0], uu[1]);
                put_split(X.ub_hi[hh][jw], X.ub_lo[hh][jw], lane, ub[hh]);
            };
            auto update = [&](int hh) {
                SplitOp kf[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) kf[i] = ld_frag(buf + cb_k(hh), frag_k(i) - 16, lane);
                three_passes([&](auto P) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) Sn[i] = mma_pass<decltype(P)::value>(kf[i], ub[hh], Sn[i]);
                });
            };
            finish_u(0);
            update(0);
            finish_u(1);
            publish_half(&xflag[jw], epoch);
            update(1);
        };
        for (int cc = 0; cc < nch; ++cc) {
            const char* buf = cbuf[cc & 1];
            lds_sync();                                            // chunk cc's operands
            if (cc + 1 < nch) ld_ut(cc + 1, utn);                 // used next chunk
            set_scale(buf);
            f32x4_t Sn[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4_t gm =
                    *reinterpret_cast<const f32x4_t*>(buf + CB_G + (16 * i + 4 * g) * 4) * kSc;
                Sn[i] = gm * (S[i] * sg);
            }
            chain(buf, Sn, cc + 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) S[i] = Sn[i] * (kInvSc * isg);
            if (cc + 1 < nch) {                           // the next chunk's split state
                // the O waves have read this chunk's split state and scales
                stalled |= !await_half(&oflag[0], cc + 1);
                stalled |= !await_half(&oflag[1], cc + 1);
                own_scale();
                make_own();
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) ut[hh][rt] = utn[hh][rt];
            }
        }
        if (stalled && lane == 0 && a.status) atomicOr(a.status, KDA_STATUS_STALLED);
        // typed store of the final state, once
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const size_t el = head_off + (size_t)(16 * i + 4 * g + e) * PD + jc[jw];
                if (ST == kF32)
                    static_cast<float*>(a.pool)[el] = S[i][e];
                else
                    static_cast<uint16_t*>(a.pool)[el] = (uint16_t)f32_to_bf16_rne(S[i][e]);
            }
    } else {
        // ---------------------------------------------------------- O wave
        // row tile r of O of the previous chunk's two halves, stored after the
        // next chunk's barrier
        f32x4_t Oprev[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}},
                               {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
        int orow0 = -1;
        bool stalled = false;
        auto store_o = [&]() {
            if (orow0 < 0) return;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tl = orow0 + 32 * hh + 16 * r + 4 * g + e;
                    if (tl < v.len) {
                        float* yrow = a.y + ((int64_t)(v.lo + tl) * H + h) * PD;
                        yrow[jc[0]] = Oprev[hh][0][e];
                        yrow[jc[1]] = Oprev[hh][1][e];
                    }
                }
        };
        SplitOp sb[2][4];
        for (int cc = 0; cc < nch; ++cc) {
            const char* buf = cbuf[cc & 1];
            const char* ws = cws(cc);
            lds_sync();                                            // chunk cc's operands
            // this chunk's scaled-Q and P fragments of row tile r, straight
            // from the workspace (in the L2 by the loaders' prefetch)
            SplitOp fq[2][4], fp[3];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) fq[hh][kb] = ld_frag_g(ws + hh * HALF_B, frag_q(r, kb), lane);
            fp[0] = ld_frag_g(ws, frag_p(0, r, 0), lane);
            fp[1] = ld_frag_g(ws + HALF_B, frag_p(1, r, 0), lane);
            fp[2] = ld_frag_g(ws + HALF_B, frag_p(1, r, 1), lane);
            // O comes out at 2^12 times the chunk's column scales; the query
            // scale multiplies it here.  The split state carries its own
            // column scale (the largest |S|), which rs brings to the chunk's.
            float osc[2], rs[2];
            {
                const float* utm = reinterpret_cast<const float*>(buf + CB_G) + PD;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float m = xmax[j][n];
                    float ss, iss, su, isu;
                    pow2_scale(m, ss, iss);
                    pow2_scale(fmaxf(m, utm[jc[j]]), su, isu);
                    osc[j] = a.q_scale * (kInvSc * isu);
                    rs[j] = su * iss;
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    sb[j][kb] = get_split(X.sb_hi[j][kb], X.sb_lo[j][kb], lane);
            publish_half(&oflag[r], cc + 1);              // split state and scales read
            store_o();
            // O = (e(t,-1) q) S for both halves, brought to the chunk's
            // column scale
            f32x4_t O[2][2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f32x4_t o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                prod4x2(fq[hh], sb, o);
#pragma unroll
                for (int j = 0; j < 2; ++j) O[hh][j] = o[j] * rs[j];
            }
            stalled |= !await_half(&xflag[0], cc + 1);
            stalled |= !await_half(&xflag[1], cc + 1);
            SplitOp ub0[2], ub1[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                ub0[j] = get_split(X.ub_hi[0][j], X.ub_lo[0][j], lane);
                ub1[j] = get_split(X.ub_hi[1][j], X.ub_lo[1][j], lane);
            }
            three_passes([&](auto P) {
                constexpr int pp = decltype(P)::value;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    O[0][j] = mma_pass<pp>(fp[0], ub0[j], O[0][j]);
                    O[1][j] = mma_pass<pp>(fp[1], ub0[j], O[1][j]);
                    O[1][j] = mma_pass<pp>(fp[2], ub1[j], O[1][j]);
                }
            });
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int j = 0; j < 2; ++j) Oprev[hh][j] = O[hh][j] * osc[j];
            orow0 = cc * PC;
        }
        store_o();
        if (stalled && lane == 0 && a.status) atomicOr(a.status, KDA_STATUS_STALLED);
    }

    // ring: the sequence's last min(3, len) raw tokens (the chunk kernel,
    // which read the old entries, has finished)
    if (grp == 0) {
        constexpr int C = 3 * PD;
        const int pend = v.pos + v.len;
        const int pfirst = max(v.pos, pend - (kConvW - 1));
        for (int pp = pfirst; pp < pend; ++pp) {
            const int64_t row = v.lo + (pp - v.pos);
            const int64_t dst = (((int64_t)v.slot * kConvW + (pp & (kConvW - 1))) * H + h) * C;
            for (int ch = tid; ch < C; ch += kStateThreads) {
                const void* src = ch < PD ? a.q : (ch < 2 * PD ? a.k : a.v);
                st_act_bits<ACT>(a.ring, dst + ch,
                                 ld_act_bits<ACT>(src, row * a.qkv_rs + h * PD + (ch % PD)));
            }
        }
    }
}

// ---------------------------------------------------------------- finish

// Gated RMSNorm of O in place: one workgroup per (token, 8 heads), 32 lanes
// per head row, four values per lane.  Rows of sequences that are skipped
// are left untouched.  The rows' O, gates and weights are requested first;
// the sequence lookup (uniform over the workgroup, so scalar loads) that
// decides whether they are written overlaps those loads.
template <int ACT>
__global__ __launch_bounds__(256) void prefill_finish_kernel(PrefillArgs a) {
    const int tid = threadIdx.x, l32 = tid & 31;
    const int64_t token = blockIdx.x;
    const int h_raw = 8 * (int)blockIdx.y + (tid >> 5);
    const bool in = h_raw < a.H;
    const int h = in ? h_raw : a.H - 1;
    const int64_t row = token * a.H + h;
    const int64_t grow = token * a.g_rs + (int64_t)h * PD;      // g of (token, head)
    float* y = a.y + row * PD + 4 * l32;
    const float4 o = *reinterpret_cast<const float4*>(y);
    float gv[4];
    if constexpr (kGateAct<ACT> == kF32) {
        const float4 g4 =
            *reinterpret_cast<const float4*>(static_cast<const float*>(a.g) + grow + 4 * l32);
        gv[0] = g4.x; gv[1] = g4.y; gv[2] = g4.z; gv[3] = g4.w;
    } else {
        const uint2 g2 =
            *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.g) + grow + 4 * l32);
        gv[0] = __uint_as_float(g2.x << 16); gv[1] = __uint_as_float(g2.x & 0xffff0000u);
        gv[2] = __uint_as_float(g2.y << 16); gv[3] = __uint_as_float(g2.y & 0xffff0000u);
    }
    const float4 w = a.norm_w ? *reinterpret_cast<const float4*>(a.norm_w + 4 * l32)
                              : make_float4(1.f, 1.f, 1.f, 1.f);
    // the sequence holding the token (cu_seqlens is monotone for valid input)
    int lo_s = 0, hi_s = a.num_seqs;
    while (hi_s - lo_s > 1) {
        const int mid = (lo_s + hi_s) >> 1;
        if (a.cu_seqlens[mid] <= token) lo_s = mid; else hi_s = mid;
    }
    SeqView v;
    const bool ok = in && seq_view(a, lo_s, false, v) && token >= v.lo && token < v.lo + v.len;
    float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
    ss = row16_sum(ss);
    ss += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ss), 0x401F));  // lane ^ 16
    if (!ok) return;
    const float rr = 1.0f / sqrtf(ss / (float)PD + a.norm_eps);
    *reinterpret_cast<float4*>(y) =
        make_float4(w.x * (o.x * rr) * gate_fn(a.gate, gv[0]), w.y * (o.y * rr) * gate_fn(a.gate, gv[1]),
                    w.z * (o.z * rr) * gate_fn(a.gate, gv[2]), w.w * (o.w * rr) * gate_fn(a.gate, gv[3]));
}

static bool is_prime(int64_t x) {
    if (x < 2) return false;
    for (int64_t d = 2; d * d <= x; ++d)
        if (x % d == 0) return false;
    return true;
}


// One chunk workgroup per compute unit of the current device (the kernel's
// LDS allows no more), looked up once per device.
static int chunk_grid() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int ACT, int ST>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    const int64_t n_slots = (a.total_tokens + PC - 1) / PC + a.num_seqs;
    const int64_t nchunk = n_slots * a.H;
    const int64_t G = (int64_t)a.num_seqs * a.H;
    const int64_t sgrid = (G + 7) / 8 * 8 * 4;    // four 32-column workgroups each
    const int hgroups = (a.H + 7) / 8;
    if (nchunk > 0) {
        // Workgroup b takes items b, b + grid, ...  A prime grid keeps the
        // items without work (periodic for regular batches) from piling up
        // on some workgroups.
        int64_t grid = std::min<int64_t>(nchunk, chunk_grid());
        while (grid > 2 && !is_prime(grid)) --grid;
        hipLaunchKernelGGL((prefill_chunk_kernel<ACT>), dim3((unsigned)grid), dim3(kChunkThreads), 0,
                           stream, a, (int)n_slots);
    }
    if (sgrid > 0)
        hipLaunchKernelGGL((prefill_state_kernel<ACT, ST>), dim3((unsigned)sgrid),
                           dim3(kStateThreads), 0, stream, a);
    if (a.total_tokens > 0)
        hipLaunchKernelGGL((prefill_finish_kernel<ACT>), dim3((unsigned)a.total_tokens, hgroups),
                           dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// The fixed workspace of kda_prefill_noalloc: one array per GPU the library
// runs on, placed when the code object loads and held until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels and copies take the address prefill_scratch() resolves.
static __device__ __align__(256) char scratch[KDA_PREFILL_SCRATCH_BYTES];

void* prefill_scratch() {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> ptrs[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = ptrs[dev].load(std::memory_order_acquire);
    if (p) return p;
    // once per device (a concurrent first call resolves the same address)
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();              // leave no error behind for the next call
        return nullptr;
    }
    ptrs[dev].store(p, std::memory_order_release);
    return p;
}

int launch_prefill(const kda_shape& s, const PrefillArgs& a, hipStream_t stream) {
    if (s.head_k != PD || s.head_v != PD) return KDA_ERR_UNSUPPORTED;
    if (s.act_dtype == kF32 && s.state_dtype == kF32) return launch_prefill_t<kF32, kF32>(a, stream);
    if (s.act_dtype == kF32 && s.state_dtype == kBF16) return launch_prefill_t<kF32, kBF16>(a, stream);
    if (s.act_dtype == kBF16 && s.state_dtype == kF32) return launch_prefill_t<kBF16, kF32>(a, stream);
    if (s.act_dtype == kBF16 && s.state_dtype == kBF16) return launch_prefill_t<kBF16, kBF16>(a, stream);
    if (s.act_dtype == kFP8 && s.state_dtype == kF32) return launch_prefill_t<kFP8, kF32>(a, stream);
    if (s.act_dtype == kFP8 && s.state_dtype == kBF16) return launch_prefill_t<kFP8, kBF16>(a, stream);
    return KDA_ERR_UNSUPPORTED;
}

}  // namespace kda
