// Split-fp16 matrix-core products for gfx950 (v_mfma_f32_16x16x32_f16).
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
// Domain: |x| < 65504 for every operand (normalised keys and queries, decay
// factors <= 1, bounded states and values all satisfy it).
//
// Lane layout of one 16x16x32 MFMA (wave64), checked on gfx950 for bf16;
// the f16 form has the same layout:
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + s], s = 0..7
//   B (32 x 16): lane l holds B[8 * (l / 16) + s][l % 16], s = 0..7
//   D (16 x 16): lane l holds D[4 * (l / 16) + r][l % 16], r = 0..3
// The order of the 32 k-indices inside one product is free as long as A and
// B agree, so the kernels pair each lane's eight k-slots with the rows that
// lane already holds in two stacked D tiles: slot s < 4 is row 4g + s of the
// first tile and slot s >= 4 is row 16 + 4g + (s - 4) (g = l / 16).  A D tile
// pair can then feed the next product's B operand without any shuffle.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct SplitOp {
    f16x8_t hi;
    f16x8_t lo;
};

// The FP32 value is pinned in a register before it is split: otherwise FP
// contraction may fold the multiply that produced x into the split (a fused
// multiply-convert for hi in one place and a separately rounded product in
// another), and hi + lo would then miss x by one fp16 ulp.
__device__ __forceinline__ SplitOp split_op(const float (&x)[8]) {
    SplitOp o;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        float xv = x[s];
        asm volatile("" : "+v"(xv));
        const _Float16 h = (_Float16)xv;
        o.hi[s] = h;
        o.lo[s] = (_Float16)(xv - (float)h);   // xv - h is exact in FP32
    }
    return o;
}

// acc += a * b over one 32-deep k block.
__device__ __forceinline__ f32x4_t mma3(const SplitOp& a, const SplitOp& b, f32x4_t acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.hi, acc, 0, 0, 0);
    return acc;
}

// k index (0..31 within a 32-deep block) carried by slot s of lane group g
// under the stacked-D-tile pairing described above.
__device__ __forceinline__ int kslot(int g, int s) {
    return s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
}

}  // namespace kda
