// Split-fp16 matrix-core products for gfx950 (v_mfma_f32_16x16x32_f16 and
// v_mfma_f32_16x16x16_f16).
//
// An FP32 operand x is carried as a pair of fp16 values, hi = fp16(x) and
// lo = fp16(x - hi) (both rounded to nearest even), so that hi + lo equals x
// to 2^-22 relative, or to 2^-25 absolute for |x| below the fp16 normal range.
// A product takes three MFMA passes, a_lo*b_hi + a_hi*b_lo + a_hi*b_hi,
// accumulated in FP32 (each fp16 x fp16 product is exact in FP32); the
// dropped a_lo*b_lo term and the two splits leave about 2^-21 relative error
// per product.  That keeps FP32-level parity at the 16-bit matrix rate: three
// passes of 16 cycles against 32 cycles per four-deep FP32 MFMA step.  A
// bf16 pair (8 + 8 significant bits) was measured to leave ~2e-5 relative
// error in the read-outs, too close to the FP32 parity bar.
// Domain: |x| < 65504 for every (scaled) operand.  Values whose lo part
// would fall below the fp16 normal range (|x| < 2^-3) lose precision, so
// callers scale bounded operands up by a power of two first.
//
// Lane layout of one 16x16x32 MFMA (wave64), checked on gfx950 for bf16;
// the f16 form has the same layout:
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + s], s = 0..7
//   B (32 x 16): lane l holds B[8 * (l / 16) + s][l % 16], s = 0..7
//   D (16 x 16): lane l holds D[4 * (l / 16) + r][l % 16], r = 0..3
// The 16x16x16 form is the same with four k-slots per lane:
//   A: lane l holds A[l % 16][4 * (l / 16) + s], B: B[4 * (l / 16) + s][l % 16],
// so a D tile (rows 4g..4g+3 in lane group g) is directly a 16-deep B operand.
// The order of the 32 k-indices inside one product is free as long as A and
// B agree, so the kernels pair each lane's eight k-slots with the rows that
// lane already holds in two stacked D tiles: slot s < 4 is row 4g + s of the
// first tile and slot s >= 4 is row 16 + 4g + (s - 4) (g = l / 16).  A D tile
// pair can then feed the next product's B operand without any shuffle.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

struct SplitOp {
    f16x8_t hi;
    f16x8_t lo;
};

struct SplitOp4 {
    f16x4_t hi;
    f16x4_t lo;
};

// Splits two FP32 values.  The pair is pinned in registers first by an empty
// non-volatile asm that the compiler cannot see through but may still
// schedule freely: otherwise FP contraction may fold the multiply that
// produced x into the conversion (a fused multiply-convert for hi in one
// place and a separately rounded product in another), and hi + lo would then
// miss x by one fp16 ulp.  hi is one packed RNE conversion; x - hi is exact
// in FP32 and is formed by one mixed-precision FMA that reads hi's fp16
// halves directly; lo is one more packed conversion.
__device__ __forceinline__ void split2(float x0, float x1, f16x2_t& hi, f16x2_t& lo) {
    f32x2_t xv = {x0, x1};
    asm("" : "+v"(xv));
    hi = __builtin_convertvector(xv, f16x2_t);
    float r0, r1;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r0) : "v"(hi), "v"(xv[0]));
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r1) : "v"(hi), "v"(xv[1]));
    const f32x2_t rv = {r0, r1};
    lo = __builtin_convertvector(rv, f16x2_t);
}

__device__ __forceinline__ SplitOp split_op(const float (&x)[8]) {
    SplitOp o;
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
        f16x2_t h, l;
        split2(x[s], x[s + 1], h, l);
        o.hi[s] = h[0];
        o.hi[s + 1] = h[1];
        o.lo[s] = l[0];
        o.lo[s + 1] = l[1];
    }
    return o;
}

__device__ __forceinline__ SplitOp4 split_op4(const float (&x)[4]) {
    SplitOp4 o;
#pragma unroll
    for (int s = 0; s < 4; s += 2) {
        f16x2_t h, l;
        split2(x[s], x[s + 1], h, l);
        o.hi[s] = h[0];
        o.hi[s + 1] = h[1];
        o.lo[s] = l[0];
        o.lo[s + 1] = l[1];
    }
    return o;
}

__device__ __forceinline__ SplitOp4 split_op4(f32x4_t x) {
    const float v[4] = {x[0], x[1], x[2], x[3]};
    return split_op4(v);
}

// Eight k-slots from two stacked D tiles (the pairing described above).
__device__ __forceinline__ SplitOp split_pair(f32x4_t lo_tile, f32x4_t hi_tile) {
    const float v[8] = {lo_tile[0], lo_tile[1], lo_tile[2], lo_tile[3],
                        hi_tile[0], hi_tile[1], hi_tile[2], hi_tile[3]};
    return split_op(v);
}

// acc += a * b over one 32-deep k block.
__device__ __forceinline__ f32x4_t mma3(const SplitOp& a, const SplitOp& b, f32x4_t acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.hi, acc, 0, 0, 0);
    return acc;
}

// One of the three passes of a split product (0: lo*hi, 1: hi*lo, 2: hi*hi).
// Issuing pass p for several independent accumulators before pass p + 1
// keeps the matrix pipe busy instead of waiting on one accumulator chain.
template <int P>
__device__ __forceinline__ f32x4_t mma_pass(const SplitOp& a, const SplitOp& b, f32x4_t acc) {
    if constexpr (P == 0) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, b.hi, acc, 0, 0, 0);
    else if constexpr (P == 1) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.lo, acc, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.hi, acc, 0, 0, 0);
}

// acc += a * b over one 16-deep k block.
__device__ __forceinline__ f32x4_t mma3(const SplitOp4& a, const SplitOp4& b, f32x4_t acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a.hi, b.hi, acc, 0, 0, 0);
    return acc;
}

// k index (0..31 within a 32-deep block) carried by slot s of lane group g
// under the stacked-D-tile pairing described above.
__device__ __forceinline__ int kslot(int g, int s) {
    return s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
}

}  // namespace kda
