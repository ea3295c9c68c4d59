// The C-ABI of the KDA mixer library: argument validation, size queries and
// dispatch.  Every host-detectable error returns before any launch, so a
// failed call writes nothing and leaves the next call unaffected (the
// stateful-op conventions of "Kimi K3 on modeling_v2: stateful catalog
// entries, ...", section 1).  Nothing here allocates, synchronises the host
// or reads the environment.
#include <hip/hip_runtime_api.h>
#include <math.h>

#include <algorithm>

#include "kda.h"
#include "kda_internal.h"

namespace {

constexpr int kConvW = 4;
constexpr int kMaxDraft = 16;

// A launch may hold fewer than 2^32 work-items.  The per-token kernels run
// batch * H workgroups of at most dk * dv / 32 threads, the commit kernel
// batch * H workgroups of 256.
bool token_grid_ok(const kda_shape* s, int32_t batch) {
    const int64_t threads = std::max<int64_t>((int64_t)s->head_k * s->head_v / 32, 256);
    return (int64_t)batch * s->num_heads * threads < (1LL << 32);
}

bool dtype_ok(int d) { return d == KDA_F32 || d == KDA_BF16; }

size_t act_size(const kda_shape* s) {
    return s->act_dtype == KDA_F32 ? 4 : (s->act_dtype == KDA_BF16 ? 2 : 1);
}
size_t state_size(const kda_shape* s) { return s->state_dtype == KDA_BF16 ? 2 : 4; }

// Shape check shared by every entry point.  Returns KDA_OK or an error.
int check_shape(const kda_shape* s) {
    if (!s) return KDA_ERR_NULL;
    if (!(dtype_ok(s->act_dtype) || s->act_dtype == KDA_FP8_E4M3) || !dtype_ok(s->state_dtype))
        return KDA_ERR_DTYPE;
    if (s->gate != KDA_GATE_SIGMOID && s->gate != KDA_GATE_SILU) return KDA_ERR_DTYPE;
    if (s->gate_inputs != KDA_GATES_VALUES && s->gate_inputs != KDA_GATES_LOGITS)
        return KDA_ERR_DTYPE;
    if (s->num_heads < 1 || s->head_k < 1 || s->head_v < 1) return KDA_ERR_SHAPE;
    if (s->conv_width != kConvW) return KDA_ERR_UNSUPPORTED;
    if (!(s->l2_eps >= 0.0f) || !(s->norm_eps >= 0.0f)) return KDA_ERR_SHAPE;
    if (!(fabsf(s->q_scale) < INFINITY)) return KDA_ERR_SHAPE;   // NaN or infinite
    if (!((s->head_k == 64 && s->head_v == 64) || (s->head_k == 128 && s->head_v == 128)))
        return KDA_ERR_UNSUPPORTED;
    const int64_t w = (int64_t)s->num_heads * s->head_k;      // == H * head_v
    for (int32_t rs : {s->qkv_row_stride, s->g_row_stride})
        if (rs != 0 && (rs < w || rs % 8 != 0)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

// Checks the parameters a call with shape s uses (s already checked).
int check_params(const kda_params* p, const kda_shape* s) {
    if (!p || !p->conv_w_q || !p->conv_w_k || !p->conv_w_v) return KDA_ERR_NULL;
    if (s->act_dtype == KDA_FP8_E4M3)
        for (int i = 0; i < 3; ++i)
            if (!(p->qkv_scale[i] > 0.0f) || !(p->qkv_scale[i] < INFINITY)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

// Elements between token rows of q, k, v and of g.
void set_row_strides(const kda_shape* s, int64_t& qkv, int64_t& g) {
    const int64_t w = (int64_t)s->num_heads * s->head_k;
    qkv = s->qkv_row_stride ? s->qkv_row_stride : w;
    g = s->g_row_stride ? s->g_row_stride : w;
}

// Dequantisation scales of q, k and v (1 unless the activations are FP8).
void set_scales(const kda_params* p, const kda_shape* s, float& sq, float& sk, float& sv) {
    const bool fp8 = s->act_dtype == KDA_FP8_E4M3;
    sq = fp8 ? p->qkv_scale[0] : 1.0f;
    sk = fp8 ? p->qkv_scale[1] : 1.0f;
    sv = fp8 ? p->qkv_scale[2] : 1.0f;
}

}  // namespace

extern "C" {

const char* kda_status_str(int code) {
    switch (code) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "a size or count is out of range";
        case KDA_ERR_DTYPE: return "unknown dtype or gate code";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_UNSUPPORTED: return "no kernel for these sizes";
        case KDA_ERR_HIP: return "HIP launch error";
        case KDA_ERR_TOO_LARGE:
            return "the call needs more scratch than the no-allocation prefill holds";
        case KDA_STATUS_BAD_SLOT: return "device status: a slot id is >= num_slots";
        case KDA_STATUS_BAD_POSITION: return "device status: a position is negative";
        case KDA_STATUS_BAD_ACCEPTED: return "device status: an accepted length is outside [0, n_draft]";
        case KDA_STATUS_BAD_SEQLENS: return "device status: cu_seqlens is not monotone or runs past the end";
        case KDA_STATUS_STALLED:
            return "device status: a prefill hand-off between waves timed out; the call's outputs are not valid";
        default:
            return code > 0 && code < 32 ? "device status: several bits set" : "unknown status code";
    }
}

size_t kda_state_bytes(const kda_shape* s, int64_t num_slots) {
    if (check_shape(s) != KDA_OK || num_slots < 0) return 0;
    return (size_t)num_slots * s->num_heads * s->head_v * s->head_k * state_size(s);
}

size_t kda_conv_bytes(const kda_shape* s, int64_t num_slots) {
    if (check_shape(s) != KDA_OK || num_slots < 0) return 0;
    return (size_t)num_slots * kConvW * s->num_heads * (2 * s->head_k + s->head_v) *
           act_size(s);
}

size_t kda_draft_state_bytes(const kda_shape* s, int32_t batch, int32_t n_draft) {
    if (check_shape(s) != KDA_OK || batch < 0 || n_draft < 0) return 0;
    return (size_t)batch * n_draft * s->num_heads * s->head_v * s->head_k * sizeof(float);
}

size_t kda_draft_conv_bytes(const kda_shape* s, int32_t batch, int32_t n_draft) {
    if (check_shape(s) != KDA_OK || batch < 0 || n_draft < 0) return 0;
    return (size_t)batch * n_draft * s->num_heads * (2 * s->head_k + s->head_v) *
           act_size(s);
}

size_t kda_prefill_workspace_bytes(const kda_shape* s, int32_t num_seqs,
                                   int64_t total_tokens) {
    if (check_shape(s) != KDA_OK || num_seqs < 0 || total_tokens < 0) return 0;
    return kda::prefill_workspace_bytes(*s, num_seqs, total_tokens);
}

int kda_state_write(const kda_shape* s, void* pool, int64_t num_slots,
                    const int32_t* slot_ids, int32_t n, const float* src,
                    int32_t* status, hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if (n < 0 || num_slots < 0) return KDA_ERR_SHAPE;
    if (n == 0) return KDA_OK;
    if (!pool || !slot_ids || !src) return KDA_ERR_NULL;
    kda::StateIoArgs a{};
    a.pool = pool;
    a.slot_ids = slot_ids;
    a.logical = const_cast<float*>(src);
    a.status = status;
    a.num_slots = num_slots;
    a.H = s->num_heads;
    a.n = n;
    a.write = 1;
    return kda::launch_state_io(*s, a, stream);
}

int kda_state_read(const kda_shape* s, const void* pool, int64_t num_slots,
                   const int32_t* slot_ids, int32_t n, float* dst,
                   int32_t* status, hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if (n < 0 || num_slots < 0) return KDA_ERR_SHAPE;
    if (n == 0) return KDA_OK;
    if (!pool || !slot_ids || !dst) return KDA_ERR_NULL;
    kda::StateIoArgs a{};
    a.pool = const_cast<void*>(pool);
    a.slot_ids = slot_ids;
    a.logical = dst;
    a.status = status;
    a.num_slots = num_slots;
    a.H = s->num_heads;
    a.n = n;
    a.write = 0;
    return kda::launch_state_io(*s, a, stream);
}

int kda_conv_write(const kda_shape* s, void* ring, int64_t num_slots,
                   const int32_t* slot_ids, const int32_t* positions, int32_t n,
                   const void* window, int32_t* status, hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if (n < 0 || num_slots < 0) return KDA_ERR_SHAPE;
    if (n == 0) return KDA_OK;
    if (!ring || !slot_ids || !positions || !window) return KDA_ERR_NULL;
    kda::StateIoArgs a{};
    a.pool = ring;
    a.slot_ids = slot_ids;
    a.positions = positions;
    a.window = const_cast<void*>(window);
    a.status = status;
    a.num_slots = num_slots;
    a.H = s->num_heads;
    a.n = n;
    a.write = 1;
    return kda::launch_conv_io(*s, a, stream);
}

int kda_conv_read(const kda_shape* s, const void* ring, int64_t num_slots,
                  const int32_t* slot_ids, const int32_t* positions, int32_t n,
                  void* window, int32_t* status, hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if (n < 0 || num_slots < 0) return KDA_ERR_SHAPE;
    if (n == 0) return KDA_OK;
    if (!ring || !slot_ids || !positions || !window) return KDA_ERR_NULL;
    kda::StateIoArgs a{};
    a.pool = const_cast<void*>(ring);
    a.slot_ids = slot_ids;
    a.positions = positions;
    a.window = window;
    a.status = status;
    a.num_slots = num_slots;
    a.H = s->num_heads;
    a.n = n;
    a.write = 0;
    return kda::launch_conv_io(*s, a, stream);
}

static kda::TokenArgs token_args(const kda_shape* s, const kda_params* p,
                                 int64_t num_slots, const int32_t* slot_ids,
                                 const int32_t* positions, const void* q,
                                 const void* k, const void* v, const void* alpha,
                                 const void* beta, const void* g, float* y,
                                 int32_t* status, int32_t n) {
    kda::TokenArgs a{};
    a.slot_ids = slot_ids;
    a.positions = positions;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.g = g;
    a.wq = p->conv_w_q;
    a.wk = p->conv_w_k;
    a.wv = p->conv_w_v;
    a.norm_w = p->norm_w;
    a.y = y;
    a.status = status;
    a.num_slots = num_slots;
    a.H = s->num_heads;
    a.n = n;
    a.q_scale = s->q_scale;
    a.l2_eps = s->l2_eps;
    a.norm_eps = s->norm_eps;
    a.gate = s->gate;
    a.gate_logits = s->gate_inputs == KDA_GATES_LOGITS;
    set_scales(p, s, a.scale_q, a.scale_k, a.scale_v);
    set_row_strides(s, a.qkv_rs, a.g_rs);
    return a;
}

int kda_decode(const kda_shape* s, const kda_params* p, int32_t batch,
               int64_t num_slots, const int32_t* slot_ids, const int32_t* positions,
               const void* q, const void* k, const void* v, const void* alpha,
               const void* beta, const void* g, void* pool, void* ring, float* y,
               int32_t* status, hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if ((rc = check_params(p, s)) != KDA_OK) return rc;
    if (batch < 0 || num_slots < 0) return KDA_ERR_SHAPE;
    if (batch == 0) return KDA_OK;
    if (!token_grid_ok(s, batch)) return KDA_ERR_SHAPE;
    if (!slot_ids || !positions || !q || !k || !v || !alpha || !beta || !g || !pool ||
        !ring || !y)
        return KDA_ERR_NULL;
    kda::TokenArgs a = token_args(s, p, num_slots, slot_ids, positions, q, k, v, alpha,
                                  beta, g, y, status, 1);
    a.pool = pool;
    a.ring = ring;
    return kda::launch_token(*s, a, batch, kda::TokenMode::Decode, stream);
}

int kda_verify(const kda_shape* s, const kda_params* p, int32_t batch,
               int32_t n_draft, int64_t num_slots, const int32_t* slot_ids,
               const int32_t* positions, const void* q, const void* k, const void* v,
               const void* alpha, const void* beta, const void* g, const void* pool,
               const void* ring, float* draft_states, void* draft_conv, float* y,
               int32_t* status, hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if ((rc = check_params(p, s)) != KDA_OK) return rc;
    if (batch < 0 || num_slots < 0 || n_draft < 1 || n_draft > kMaxDraft)
        return KDA_ERR_SHAPE;
    if (batch == 0) return KDA_OK;
    if (!token_grid_ok(s, batch)) return KDA_ERR_SHAPE;
    if (!slot_ids || !positions || !q || !k || !v || !alpha || !beta || !g || !pool ||
        !ring || !y)
        return KDA_ERR_NULL;
    kda::TokenArgs a = token_args(s, p, num_slots, slot_ids, positions, q, k, v, alpha,
                                  beta, g, y, status, n_draft);
    a.pool = const_cast<void*>(pool);
    a.ring = const_cast<void*>(ring);
    a.records = draft_states;
    a.draft_conv = draft_conv;
    return kda::launch_token(*s, a, batch, kda::TokenMode::Verify, stream);
}

int kda_commit_recompute(const kda_shape* s, const kda_params* p, int32_t batch,
                         int32_t n_draft, int64_t num_slots, const int32_t* slot_ids,
                         const int32_t* positions, const int32_t* accepted, const void* q,
                         const void* k, const void* v, const void* alpha, const void* beta,
                         const void* g, void* pool, void* ring, int32_t* status,
                         hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if ((rc = check_params(p, s)) != KDA_OK) return rc;
    if (batch < 0 || num_slots < 0 || n_draft < 1 || n_draft > kMaxDraft)
        return KDA_ERR_SHAPE;
    if (batch == 0) return KDA_OK;
    if (!token_grid_ok(s, batch)) return KDA_ERR_SHAPE;
    if (!slot_ids || !positions || !accepted || !q || !k || !v || !alpha || !beta || !g ||
        !pool || !ring)
        return KDA_ERR_NULL;
    kda::TokenArgs a = token_args(s, p, num_slots, slot_ids, positions, q, k, v, alpha,
                                  beta, g, nullptr, status, n_draft);
    a.pool = pool;
    a.ring = ring;
    a.accepted = accepted;
    return kda::launch_token(*s, a, batch, kda::TokenMode::Recompute, stream);
}

int kda_commit_accepted(const kda_shape* s, int32_t batch, int32_t n_draft,
                        int64_t num_slots, const int32_t* slot_ids,
                        const int32_t* positions, const int32_t* accepted,
                        const float* draft_states, const void* draft_conv, void* pool,
                        void* ring, int32_t* status, hipStream_t stream) {
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if (batch < 0 || num_slots < 0 || n_draft < 1 || n_draft > kMaxDraft)
        return KDA_ERR_SHAPE;
    if (batch == 0) return KDA_OK;
    if (!token_grid_ok(s, batch)) return KDA_ERR_SHAPE;
    if (!slot_ids || !positions || !accepted || !draft_states || !draft_conv || !pool ||
        !ring)
        return KDA_ERR_NULL;
    kda::CommitArgs a{};
    a.slot_ids = slot_ids;
    a.positions = positions;
    a.accepted = accepted;
    a.records = draft_states;
    a.draft_conv = draft_conv;
    a.pool = pool;
    a.ring = ring;
    a.status = status;
    a.num_slots = num_slots;
    a.H = s->num_heads;
    a.n = n_draft;
    return kda::launch_commit(*s, a, batch, stream);
}

// Validation shared by both prefill entry points, before any launch.
static int check_prefill(const kda_shape* s, const kda_params* p, int32_t num_seqs,
                         const int32_t* cu_seqlens, int64_t total_tokens, int32_t max_seqlen,
                         int64_t num_slots, const int32_t* slot_ids, const int32_t* positions,
                         const void* q, const void* k, const void* v, const void* alpha,
                         const void* beta, const void* g, void* pool, void* ring, float* y,
                         bool& nothing_to_do) {
    nothing_to_do = false;
    int rc = check_shape(s);
    if (rc != KDA_OK) return rc;
    if ((rc = check_params(p, s)) != KDA_OK) return rc;
    if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0 || num_slots < 0)
        return KDA_ERR_SHAPE;
    if (num_seqs == 0 || total_tokens == 0 || max_seqlen == 0) {
        nothing_to_do = true;
        return KDA_OK;
    }
    // the finish kernel runs one 256-thread workgroup per token (grid x)
    if (total_tokens > 0x7fffffffLL || total_tokens * 256 >= (1LL << 32)) return KDA_ERR_SHAPE;
    if (!cu_seqlens || !slot_ids || !positions || !q || !k || !v || !alpha || !beta ||
        !g || !pool || !ring || !y)
        return KDA_ERR_NULL;
    return KDA_OK;
}

static int run_prefill(const kda_shape* s, const kda_params* p, int32_t num_seqs,
                       const int32_t* cu_seqlens, int64_t total_tokens, int32_t max_seqlen,
                       int64_t num_slots, const int32_t* slot_ids, const int32_t* positions,
                       const void* q, const void* k, const void* v, const void* alpha,
                       const void* beta, const void* g, void* pool, void* ring, float* y,
                       void* workspace, int32_t* status, hipStream_t stream) {
    kda::PrefillArgs a{};
    a.cu_seqlens = cu_seqlens;
    a.slot_ids = slot_ids;
    a.positions = positions;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.g = g;
    a.wq = p->conv_w_q;
    a.wk = p->conv_w_k;
    a.wv = p->conv_w_v;
    a.norm_w = p->norm_w;
    a.pool = pool;
    a.ring = ring;
    a.y = y;
    a.workspace = workspace;
    a.status = status;
    a.total_tokens = total_tokens;
    a.num_slots = num_slots;
    a.num_seqs = num_seqs;
    a.max_seqlen = max_seqlen;
    a.H = s->num_heads;
    a.q_scale = s->q_scale;
    a.l2_eps = s->l2_eps;
    a.norm_eps = s->norm_eps;
    a.gate = s->gate;
    a.gate_logits = s->gate_inputs == KDA_GATES_LOGITS;
    set_scales(p, s, a.scale_q, a.scale_k, a.scale_v);
    set_row_strides(s, a.qkv_rs, a.g_rs);
    return kda::launch_prefill(*s, a, stream);
}

int kda_prefill(const kda_shape* s, const kda_params* p, int32_t num_seqs,
                const int32_t* cu_seqlens, int64_t total_tokens, int32_t max_seqlen,
                int64_t num_slots, const int32_t* slot_ids, const int32_t* positions,
                const void* q, const void* k, const void* v, const void* alpha,
                const void* beta, const void* g, void* pool, void* ring, float* y,
                void* workspace, size_t workspace_bytes, int32_t* status,
                hipStream_t stream) {
    bool none;
    int rc = check_prefill(s, p, num_seqs, cu_seqlens, total_tokens, max_seqlen, num_slots,
                           slot_ids, positions, q, k, v, alpha, beta, g, pool, ring, y, none);
    if (rc != KDA_OK || none) return rc;
    if (s->head_k != 128 || s->head_v != 128) return KDA_ERR_UNSUPPORTED;
    const size_t need = kda::prefill_workspace_bytes(*s, num_seqs, total_tokens);
    if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
    return run_prefill(s, p, num_seqs, cu_seqlens, total_tokens, max_seqlen, num_slots,
                       slot_ids, positions, q, k, v, alpha, beta, g, pool, ring, y, workspace,
                       status, stream);
}

int kda_prefill_noalloc(const kda_shape* s, const kda_params* p, int32_t num_seqs,
                        const int32_t* cu_seqlens, int64_t total_tokens, int32_t max_seqlen,
                        int64_t num_slots, const int32_t* slot_ids, const int32_t* positions,
                        const void* q, const void* k, const void* v, const void* alpha,
                        const void* beta, const void* g, void* pool, void* ring, float* y,
                        int32_t* status, hipStream_t stream) {
    bool none;
    int rc = check_prefill(s, p, num_seqs, cu_seqlens, total_tokens, max_seqlen, num_slots,
                           slot_ids, positions, q, k, v, alpha, beta, g, pool, ring, y, none);
    if (rc != KDA_OK || none) return rc;
    if (s->head_k != 128 || s->head_v != 128) return KDA_ERR_UNSUPPORTED;
    if (kda::prefill_workspace_bytes(*s, num_seqs, total_tokens) > KDA_PREFILL_SCRATCH_BYTES)
        return KDA_ERR_TOO_LARGE;
    void* scratch = kda::prefill_scratch();
    if (!scratch) return KDA_ERR_HIP;
    return run_prefill(s, p, num_seqs, cu_seqlens, total_tokens, max_seqlen, num_slots,
                       slot_ids, positions, q, k, v, alpha, beta, g, pool, ring, y, scratch,
                       status, stream);
}

}  // extern "C"
