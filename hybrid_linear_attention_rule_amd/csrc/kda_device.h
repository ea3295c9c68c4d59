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

enum : int { kF32 = 0, kBF16 = 1 };
enum : int { kGateSigmoid = 0, kGateSilu = 1 };

constexpr int kWave = 64;
constexpr int kConvW = 4;  // conv taps; the ring holds kConvW entries

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Scalar activation load, widened to FP32.
template <int ACT>
__device__ __forceinline__ float ld_act(const void* base, int64_t idx) {
    if constexpr (ACT == kF32) {
        return static_cast<const float*>(base)[idx];
    } else {
        return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    }
}

// Raw copy of one activation element (bit exact).
template <int ACT>
__device__ __forceinline__ void cp_act(void* dst, int64_t di, const void* src,
                                       int64_t si) {
    if constexpr (ACT == kF32) {
        static_cast<float*>(dst)[di] = static_cast<const float*>(src)[si];
    } else {
        static_cast<uint16_t*>(dst)[di] = static_cast<const uint16_t*>(src)[si];
    }
}

template <int ACT>
__device__ __forceinline__ void st_act_bits(void* dst, int64_t di, uint32_t bits) {
    if constexpr (ACT == kF32) {
        static_cast<uint32_t*>(dst)[di] = bits;
    } else {
        static_cast<uint16_t*>(dst)[di] = static_cast<uint16_t>(bits);
    }
}

template <int ACT>
__device__ __forceinline__ uint32_t ld_act_bits(const void* src, int64_t si) {
    if constexpr (ACT == kF32) {
        return static_cast<const uint32_t*>(src)[si];
    } else {
        return static_cast<const uint16_t*>(src)[si];
    }
}

__device__ __forceinline__ float gate_fn(int gate, float x) {
    const float sig = 1.0f / (1.0f + expf(-x));
    return gate == kGateSilu ? x * sig : sig;
}

// Sum over a whole wavefront; every lane gets the total.  Fixed order.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) x += __shfl_xor(x, d, kWave);
    return x;
}

// Recursive-halving reduction over groups of G consecutive lanes, for
// N == G values per lane.  On return lane (lane % G) == i of the group holds
// the group's sum of value i.  N - 1 shuffles per lane, fixed order.
//
// At each level the upper lane of a pair first swaps the two halves of its
// values, so that every lane keeps v[0..half) and sends v[half..2*half).
// The swap reads each element twice, which keeps the selects on values: a
// select between two element addresses would turn the register array into a
// dynamically indexed one (compare-and-select chains).
template <int G>
__device__ __forceinline__ float group_transpose_sum(float (&v)[G], int lane_in_group) {
#pragma unroll
    for (int half = G / 2; half >= 1; half >>= 1) {
        const bool upper = (lane_in_group & half) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float a = v[i], b = v[i + half];
            v[i] = upper ? b : a;
            v[i + half] = upper ? a : b;
        }
#pragma unroll
        for (int i = 0; i < half; ++i) v[i] += __shfl_xor(v[i + half], half, kWave);
    }
    return v[0];
}

}  // namespace kda
