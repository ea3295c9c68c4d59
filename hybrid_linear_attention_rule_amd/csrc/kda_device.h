// Device helpers shared by the KDA kernels (gfx950, wave64).
//
// Typed loads widen activations and states to FP32 exactly; the typed store
// of a BF16 state rounds to nearest, ties to even, once per store (the FP32
// recurrence with FP32 or BF16 state storage of "Extend
// NVIDIA/TensorRT-LLM#19991 with isolated NVFP4 Kimi K3 targets",
// Description).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// FP8 activations carry q, k, v (and the raw tokens kept in the ring and
// the draft buffer) as OCP E4M3 bytes times a per-tensor scale; alpha, beta
// and g then stay BF16.  kGateAct is the dtype of alpha, beta and g.
template <int ACT>
constexpr int kGateAct = ACT == kFP8 ? kBF16 : ACT;
template <int ACT>
constexpr size_t kActSize = ACT == kF32 ? 4 : (ACT == kBF16 ? 2 : 1);
enum : int { kGateSigmoid = 0, kGateSilu = 1 };

constexpr int kWave = 64;
constexpr int kConvW = 4;  // conv taps; the ring holds kConvW entries

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// OCP FP8 E4M3 (bias 7, three mantissa bits, no infinities, largest finite
// 448) to FP32, exactly, by the matrix-core generation's conversion
// instruction (v_cvt_f32_fp8 on byte 0).  On gfx950 it reads the OCP
// encoding: for every finite code it gives 2^(e-7) * (1 + m/8) for an
// exponent field e > 0 and m * 2^-9 for e = 0, and NaN for the NaN codes.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
    return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Four E4M3 bytes of a word to FP32 (bytes 0..3 in order), two per
// v_cvt_pk_f32_fp8.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t word, float (&x)[4]) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    const f2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
    const f2v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
    x[0] = lo.x; x[1] = lo.y; x[2] = hi.x; x[3] = hi.y;
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Activation bits to FP32 (exact; an FP8 value before its tensor scale).
template <int ACT>
__device__ __forceinline__ float act_from_bits(uint32_t bits) {
    if constexpr (ACT == kF32) return __uint_as_float(bits);
    else if constexpr (ACT == kBF16) return bf16_to_f32(bits);
    else return e4m3_to_f32(bits);
}

// Scalar activation load, widened to FP32.
template <int ACT>
__device__ __forceinline__ float ld_act(const void* base, int64_t idx) {
    if constexpr (ACT == kF32) {
        return static_cast<const float*>(base)[idx];
    } else if constexpr (ACT == kBF16) {
        return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    } else {
        return e4m3_to_f32(static_cast<const uint8_t*>(base)[idx]);
    }
}

template <int ACT>
__device__ __forceinline__ void st_act_bits(void* dst, int64_t di, uint32_t bits) {
    if constexpr (ACT == kF32) {
        static_cast<uint32_t*>(dst)[di] = bits;
    } else if constexpr (ACT == kBF16) {
        static_cast<uint16_t*>(dst)[di] = static_cast<uint16_t>(bits);
    } else {
        static_cast<uint8_t*>(dst)[di] = static_cast<uint8_t>(bits);
    }
}

template <int ACT>
__device__ __forceinline__ uint32_t ld_act_bits(const void* src, int64_t si) {
    if constexpr (ACT == kF32) {
        return static_cast<const uint32_t*>(src)[si];
    } else if constexpr (ACT == kBF16) {
        return static_cast<const uint16_t*>(src)[si];
    } else {
        return static_cast<const uint8_t*>(src)[si];
    }
}

// Decay and write strengths from their logits: alpha = exp(-softplus(a)),
// which equals 1 / (1 + e^a), and beta = sigmoid(b) = 1 / (1 + e^-b).
__device__ __forceinline__ float decay_from_logit(float a) { return 1.0f / (1.0f + expf(a)); }
__device__ __forceinline__ float write_from_logit(float b) { return 1.0f / (1.0f + expf(-b)); }

__device__ __forceinline__ float gate_fn(int gate, float x) {
    const float sig = 1.0f / (1.0f + expf(-x));
    return gate == kGateSilu ? x * sig : sig;
}

// DPP move of a float within rows of 16 lanes (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over a whole wavefront; the result is uniform.  Fixed order: pairs,
// quads, halves and rows of 16 by DPP, then the four row sums in lane order.
// Must be called with every lane of the wave active.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm(1,0,3,2): lane ^ 1
    x += dpp_mov<0x4E>(x);    // quad_perm(2,3,0,1): lane ^ 2
    x += dpp_mov<0x141>(x);   // row_half_mirror: lane i <-> 7 - i
    x += dpp_mov<0x140>(x);   // row_mirror: lane i <-> 15 - i
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return ((r0 + r1) + r2) + r3;
}

}  // namespace kda
