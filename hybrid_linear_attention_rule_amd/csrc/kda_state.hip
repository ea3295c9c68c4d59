// Typed state store and conv-history import/export: the logical FP32
// checkpoint format of the KDA state pool and conv ring.  FP32 loads widen
// exactly; BF16 stores round to nearest even ("Extend
// NVIDIA/TensorRT-LLM#19991 with isolated NVFP4 Kimi K3 targets",
// Description: explicit FP32 loads and typed state stores).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// One workgroup per (row, head); the pool stores each head's state in the
// logical [dk][dv] order, so import/export is a typed copy.
template <int ST>
__global__ __launch_bounds__(256) void state_io_kernel(StateIoArgs a, int DK, int DV) {
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int b = blockIdx.x / H;
    const int slot = a.slot_ids[b];
    if (slot < 0) return;
    if (slot >= a.num_slots) {
        if (threadIdx.x == 0 && a.status) atomicOr(a.status, KDA_STATUS_BAD_SLOT);
        return;
    }
    const size_t elems = (size_t)DK * DV;
    const size_t phys0 = ((size_t)slot * H + h) * elems;
    float* logical = a.logical + ((size_t)b * H + h) * elems;
    for (int e = threadIdx.x; e < (int)elems; e += blockDim.x) {
        if (a.write) {
            const float x = logical[e];
            if constexpr (ST == kF32)
                static_cast<float*>(a.pool)[phys0 + e] = x;
            else
                static_cast<uint16_t*>(a.pool)[phys0 + e] = (uint16_t)f32_to_bf16_rne(x);
        } else {
            float x;
            if constexpr (ST == kF32)
                x = static_cast<const float*>(a.pool)[phys0 + e];
            else
                x = bf16_to_f32(static_cast<const uint16_t*>(a.pool)[phys0 + e]);
            logical[e] = x;
        }
    }
}

// One workgroup per (row, history entry, head): window [n][3][H][C] <->
// ring [slot][4][H][C], entry (p - 3 + j) mod 4 for positions p - 3 + j >= 0.
template <int ACT>
__global__ __launch_bounds__(256) void conv_io_kernel(StateIoArgs a, int C) {
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int j = (blockIdx.x / H) % (kConvW - 1);
    const int b = blockIdx.x / (H * (kConvW - 1));
    const int slot = a.slot_ids[b];
    if (slot < 0) return;
    if (slot >= a.num_slots) {
        if (threadIdx.x == 0 && j == 0 && h == 0 && a.status)
            atomicOr(a.status, KDA_STATUS_BAD_SLOT);
        return;
    }
    const int pos = a.positions[b];
    if (pos < 0) {
        if (threadIdx.x == 0 && j == 0 && h == 0 && a.status)
            atomicOr(a.status, KDA_STATUS_BAD_POSITION);
        return;
    }
    const int pp = pos - (kConvW - 1) + j;
    const int64_t w0 = (((int64_t)b * (kConvW - 1) + j) * H + h) * C;
    if (pp < 0) {
        if (!a.write)
            for (int c = threadIdx.x; c < C; c += blockDim.x) st_act_bits<ACT>(a.window, w0 + c, 0u);
        return;
    }
    const int64_t r0 = (((int64_t)slot * kConvW + (pp & (kConvW - 1))) * H + h) * C;
    for (int c = threadIdx.x; c < C; c += blockDim.x) {
        if (a.write)
            st_act_bits<ACT>(a.pool, r0 + c, ld_act_bits<ACT>(a.window, w0 + c));
        else
            st_act_bits<ACT>(a.window, w0 + c, ld_act_bits<ACT>(a.pool, r0 + c));
    }
}

int launch_state_io(const kda_shape& s, const StateIoArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.n * (unsigned)a.H), block(256);
    if (s.state_dtype == kF32)
        hipLaunchKernelGGL(state_io_kernel<kF32>, grid, block, 0, stream, a, s.head_k, s.head_v);
    else
        hipLaunchKernelGGL(state_io_kernel<kBF16>, grid, block, 0, stream, a, s.head_k, s.head_v);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int launch_conv_io(const kda_shape& s, const StateIoArgs& a, hipStream_t stream) {
    const int C = 2 * s.head_k + s.head_v;
    const dim3 grid((unsigned)a.n * (kConvW - 1) * (unsigned)a.H), block(256);
    if (s.act_dtype == kF32)
        hipLaunchKernelGGL(conv_io_kernel<kF32>, grid, block, 0, stream, a, C);
    else if (s.act_dtype == kFP8)
        hipLaunchKernelGGL(conv_io_kernel<kFP8>, grid, block, 0, stream, a, C);
    else
        hipLaunchKernelGGL(conv_io_kernel<kBF16>, grid, block, 0, stream, a, C);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace kda
