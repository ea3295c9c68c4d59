// Internal launcher interface between the C-ABI layer (kda_api.cpp) and
// the kernels.  Host code only; no torch types.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Decode (n == 1, stores state and ring), verify (n draft tokens, writes
// records and raw drafts when given) and recompute (the first accepted[row]
// of n draft tokens from the stored state; stores state and ring) share one
// per-token kernel.
struct TokenArgs {
    const int32_t* slot_ids;
    const int32_t* positions;
    const void* q;
    const void* k;
    const void* v;
    const void* alpha;
    const void* beta;
    const void* g;
    const float* wq;
    const float* wk;
    const float* wv;
    const float* norm_w;
    void* pool;          // decode: read + written; verify: read only
    void* ring;          // decode: read + written; verify: read only
    float* records;      // verify only; NULL: no records
    void* draft_conv;    // verify only; NULL: raw drafts not kept
    const int32_t* accepted;  // recompute only: tokens to run per row
    float* y;
    int32_t* status;
    int64_t num_slots;
    int32_t H;
    int32_t n;           // input rows per batch row (1 for decode)
    float q_scale;
    float l2_eps;
    float norm_eps;
    int32_t gate;
    int32_t gate_logits;  // alpha, beta hold logits a, b
    float scale_q, scale_k, scale_v;  // FP8 activations: dequantisation scales
    int64_t qkv_rs, g_rs;             // elements between token rows of q|k|v and of g
};

struct CommitArgs {
    const int32_t* slot_ids;
    const int32_t* positions;
    const int32_t* accepted;
    const float* records;
    const void* draft_conv;
    void* pool;
    void* ring;
    int32_t* status;
    int64_t num_slots;
    int32_t H;
    int32_t n;
};

struct StateIoArgs {
    void* pool;
    const int32_t* slot_ids;
    const int32_t* positions;  // conv io only
    float* logical;            // [n, H, dk, dv] FP32 (state io)
    void* window;              // [n, 3, H, C] act (conv io)
    int32_t* status;
    int64_t num_slots;
    int32_t H;
    int32_t n;
    int32_t write;             // 1: logical -> pool, 0: pool -> logical
};

struct PrefillArgs {
    const int32_t* cu_seqlens;
    const int32_t* slot_ids;
    const int32_t* positions;
    const void* q;
    const void* k;
    const void* v;
    const void* alpha;
    const void* beta;
    const void* g;
    const float* wq;
    const float* wk;
    const float* wv;
    const float* norm_w;
    void* pool;
    void* ring;
    float* y;
    void* workspace;
    int32_t* status;
    int64_t total_tokens;
    int64_t num_slots;
    int32_t num_seqs;
    int32_t max_seqlen;
    int32_t H;
    float q_scale;
    float l2_eps;
    float norm_eps;
    int32_t gate;
    int32_t gate_logits;  // alpha, beta hold logits a, b
    float scale_q, scale_k, scale_v;  // FP8 activations: dequantisation scales
    int64_t qkv_rs, g_rs;             // elements between token rows of q|k|v and of g
};

enum class TokenMode { Decode, Verify, Recompute };

// Each returns KDA_OK, KDA_ERR_UNSUPPORTED (no instantiation) or KDA_ERR_HIP.
int launch_token(const kda_shape& s, const TokenArgs& a, int32_t batch, TokenMode mode,
                 hipStream_t stream);
int launch_commit(const kda_shape& s, const CommitArgs& a, int32_t batch,
                  hipStream_t stream);
int launch_state_io(const kda_shape& s, const StateIoArgs& a,
                    hipStream_t stream);
int launch_conv_io(const kda_shape& s, const StateIoArgs& a,
                   hipStream_t stream);
size_t prefill_workspace_bytes(const kda_shape& s, int32_t num_seqs,
                               int64_t total_tokens);
int launch_prefill(const kda_shape& s, const PrefillArgs& a,
                   hipStream_t stream);
// Device address of the current device's fixed prefill scratch array
// (KDA_PREFILL_SCRATCH_BYTES), resolved once per device; NULL on a HIP error.
void* prefill_scratch();

}  // namespace kda
