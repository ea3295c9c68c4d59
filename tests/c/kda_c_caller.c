/*
 * A plain C caller of the KDA C-ABI (include/kda.h, libkda.so): no Python.
 *
 *   kda_c_caller host            host-side checks only (no GPU needed):
 *                                size queries, status strings and errors
 *                                returned before any launch; exit 0 if all hold
 *   kda_c_caller decode DIR      one decode call on the GPU: reads the inputs
 *                                DIR/{meta.txt, *.f32} written by the test,
 *                                writes DIR/y.f32 and DIR/state.f32
 *   kda_c_caller verify DIR      kda_verify over n draft tokens, then
 *                                kda_commit_accepted with DIR/accepted.i32;
 *                                writes DIR/y.f32, DIR/records.f32 and
 *                                DIR/state.f32 (the committed states)
 *   kda_c_caller prefill DIR     kda_prefill of the packed sequences of
 *                                DIR/cu_seqlens.i32 (workspace allocated here,
 *                                by the caller); writes DIR/y.f32 and
 *                                DIR/state.f32
 *
 * Shapes: batch (or sequences) B, heads H, dk = dv = d (64 or 128; 128 for
 * prefill), FP32 activations and FP32 state, slots 0..B-1, positions 0
 * (fresh sequences: zero state and empty history).  meta.txt holds
 * "B H d" (decode, prefill) or "B H d n" (verify).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

static int fails = 0;
#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++fails;                                                     \
        }                                                                \
    } while (0)

static kda_shape make_shape(int H, int d) {
    kda_shape s;
    memset(&s, 0, sizeof(s));
    s.num_heads = H;
    s.head_k = d;
    s.head_v = d;
    s.conv_width = 4;
    s.act_dtype = KDA_F32;
    s.state_dtype = KDA_F32;
    s.gate = KDA_GATE_SIGMOID;
    s.q_scale = 1.0f;
    s.l2_eps = 1e-6f;
    s.norm_eps = 1e-6f;
    s.gate_inputs = KDA_GATES_VALUES;
    return s;
}

static int host_checks(void) {
    kda_shape s = make_shape(32, 128);
    CHECK(kda_state_bytes(&s, 64) == (size_t)64 * 32 * 128 * 128 * 4);
    CHECK(kda_conv_bytes(&s, 2) == (size_t)2 * 4 * 32 * 384 * 4);
    CHECK(kda_draft_state_bytes(&s, 16, 4) == (size_t)16 * 4 * 32 * 128 * 128 * 4);
    CHECK(kda_status_str(KDA_OK) != NULL && kda_status_str(KDA_ERR_NULL) != NULL);
    /* errors before any launch: nothing here is ever dereferenced */
    void* bogus = (void*)0x1000;
    kda_params p;
    memset(&p, 0, sizeof(p));
    p.conv_w_q = p.conv_w_k = p.conv_w_v = (const float*)bogus;
    CHECK(kda_decode(NULL, &p, 4, 8, bogus, bogus, bogus, bogus, bogus, bogus, bogus, bogus,
                     bogus, bogus, bogus, NULL, NULL) == KDA_ERR_NULL);
    kda_shape bad = s;
    bad.head_k = bad.head_v = 96;
    CHECK(kda_decode(&bad, &p, 4, 8, bogus, bogus, bogus, bogus, bogus, bogus, bogus, bogus,
                     bogus, bogus, bogus, NULL, NULL) == KDA_ERR_UNSUPPORTED);
    bad = s;
    bad.act_dtype = 9;
    CHECK(kda_decode(&bad, &p, 4, 8, bogus, bogus, bogus, bogus, bogus, bogus, bogus, bogus,
                     bogus, bogus, bogus, NULL, NULL) == KDA_ERR_DTYPE);
    CHECK(kda_decode(&s, &p, 4, 8, bogus, bogus, NULL, bogus, bogus, bogus, bogus, bogus,
                     bogus, bogus, bogus, NULL, NULL) == KDA_ERR_NULL);
    CHECK(kda_decode(&s, &p, 0, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                     NULL, NULL, NULL) == KDA_OK);
    return fails;
}

static float* read_f32(const char* dir, const char* name, size_t n) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/%s.f32", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    float* x = (float*)malloc(n * sizeof(float));
    size_t got = x ? fread(x, sizeof(float), n, f) : 0;
    fclose(f);
    if (got != n) {
        free(x);
        return NULL;
    }
    return x;
}

static int write_f32(const char* dir, const char* name, const float* x, size_t n) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/%s.f32", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return -1;
    size_t put = fwrite(x, sizeof(float), n, f);
    fclose(f);
    return put == n ? 0 : -1;
}

/* device copy of a host array; NULL on failure */
static void* to_device(const void* h, size_t bytes) {
    void* d = NULL;
    if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
    if (hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return d;
}

static int32_t* read_i32(const char* dir, const char* name, size_t n) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/%s.i32", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    int32_t* x = (int32_t*)malloc(n * sizeof(int32_t));
    size_t got = x ? fread(x, sizeof(int32_t), n, f) : 0;
    fclose(f);
    if (got != n) {
        free(x);
        return NULL;
    }
    return x;
}

/* device buffer of `bytes` zero bytes; NULL on failure */
static void* device_zeros(size_t bytes) {
    void* d = NULL;
    if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
    if (hipMemset(d, 0, bytes) != hipSuccess) return NULL;
    return d;
}

static int copy_out(const char* dir, const char* name, const void* dev, size_t nfloats) {
    float* h = (float*)malloc(nfloats * sizeof(float));
    if (!h || hipMemcpy(h, dev, nfloats * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
        return -1;
    int rc = write_f32(dir, name, h, nfloats);
    free(h);
    return rc;
}

/* the layer's conv taps from DIR/w{q,k,v}.f32; 0 on success */
static int load_params(const char* dir, int H, int d, kda_params* p) {
    float* wq = read_f32(dir, "wq", (size_t)H * d * 4);
    float* wk = read_f32(dir, "wk", (size_t)H * d * 4);
    float* wv = read_f32(dir, "wv", (size_t)H * d * 4);
    if (!wq || !wk || !wv) return -1;
    memset(p, 0, sizeof(*p));
    p->conv_w_q = (const float*)to_device(wq, (size_t)H * d * 4 * 4);
    p->conv_w_k = (const float*)to_device(wk, (size_t)H * d * 4 * 4);
    p->conv_w_v = (const float*)to_device(wv, (size_t)H * d * 4 * 4);
    free(wq);
    free(wk);
    free(wv);
    return (p->conv_w_q && p->conv_w_k && p->conv_w_v) ? 0 : -1;
}

/* device copies of DIR/{q,k,v,alpha,beta,g}.f32 for `rows` token rows */
static int load_tokens(const char* dir, size_t rows, int H, int d, void* dev[6]) {
    static const char* names[6] = {"q", "k", "v", "alpha", "beta", "g"};
    for (int i = 0; i < 6; ++i) {
        const size_t n = rows * H * (i == 4 ? 1 : (size_t)d);
        float* h = read_f32(dir, names[i], n);
        if (!h) return -1;
        dev[i] = to_device(h, n * 4);
        free(h);
        if (!dev[i]) return -1;
    }
    return 0;
}

static int verify_from_files(const char* dir) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/meta.txt", dir);
    FILE* f = fopen(path, "r");
    int B = 0, H = 0, d = 0, n = 0;
    if (!f || fscanf(f, "%d %d %d %d", &B, &H, &d, &n) != 4) return 2;
    fclose(f);
    kda_shape s = make_shape(H, d);
    kda_params p;
    void* tok[6];
    if (load_params(dir, H, d, &p) != 0 || load_tokens(dir, (size_t)B * n, H, d, tok) != 0)
        return 3;
    int32_t* acc = read_i32(dir, "accepted", B);
    int32_t* slots = (int32_t*)malloc(B * sizeof(int32_t));
    int32_t* pos = (int32_t*)calloc(B, sizeof(int32_t));
    if (!acc || !slots || !pos) return 3;
    for (int b = 0; b < B; ++b) slots[b] = b;
    void *dslots = to_device(slots, B * 4), *dpos = to_device(pos, B * 4);
    void *dacc = to_device(acc, B * 4);
    const size_t pool_b = kda_state_bytes(&s, B), ring_b = kda_conv_bytes(&s, B);
    const size_t rec_b = kda_draft_state_bytes(&s, B, n), dconv_b = kda_draft_conv_bytes(&s, B, n);
    const size_t y_n = (size_t)B * n * H * d;
    void *pool = device_zeros(pool_b), *ring = device_zeros(ring_b);
    void *rec = device_zeros(rec_b), *dconv = device_zeros(dconv_b);
    void *y = device_zeros(y_n * 4), *status = device_zeros(4);
    if (!dslots || !dpos || !dacc || !pool || !ring || !rec || !dconv || !y || !status) return 4;
    int rc = kda_verify(&s, &p, B, n, B, (const int32_t*)dslots, (const int32_t*)dpos, tok[0],
                        tok[1], tok[2], tok[3], tok[4], tok[5], pool, ring, (float*)rec, dconv,
                        (float*)y, (int32_t*)status, NULL);
    if (rc != KDA_OK) {
        fprintf(stderr, "kda_verify: %s\n", kda_status_str(rc));
        return 5;
    }
    rc = kda_commit_accepted(&s, B, n, B, (const int32_t*)dslots, (const int32_t*)dpos,
                             (const int32_t*)dacc, (const float*)rec, dconv, pool, ring,
                             (int32_t*)status, NULL);
    if (rc != KDA_OK) {
        fprintf(stderr, "kda_commit_accepted: %s\n", kda_status_str(rc));
        return 5;
    }
    if (hipDeviceSynchronize() != hipSuccess) return 6;
    int32_t hstatus = -1;
    if (hipMemcpy(&hstatus, status, 4, hipMemcpyDeviceToHost) != hipSuccess) return 7;
    if (hstatus != 0) return 8;
    if (copy_out(dir, "y", y, y_n) != 0 || copy_out(dir, "records", rec, rec_b / 4) != 0 ||
        copy_out(dir, "state", pool, pool_b / 4) != 0)
        return 9;
    printf("verify + commit ok: B=%d H=%d d=%d n=%d\n", B, H, d, n);
    return 0;
}

static int prefill_from_files(const char* dir) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/meta.txt", dir);
    FILE* f = fopen(path, "r");
    int B = 0, H = 0, d = 0;
    if (!f || fscanf(f, "%d %d %d", &B, &H, &d) != 3) return 2;
    fclose(f);
    kda_shape s = make_shape(H, d);
    int32_t* cu = read_i32(dir, "cu_seqlens", (size_t)B + 1);
    if (!cu) return 3;
    const int64_t T = cu[B];
    int32_t max_len = 0;
    for (int b = 0; b < B; ++b)
        if (cu[b + 1] - cu[b] > max_len) max_len = cu[b + 1] - cu[b];
    kda_params p;
    void* tok[6];
    if (load_params(dir, H, d, &p) != 0 || load_tokens(dir, (size_t)T, H, d, tok) != 0) return 3;
    int32_t* slots = (int32_t*)malloc(B * sizeof(int32_t));
    int32_t* pos = (int32_t*)calloc(B, sizeof(int32_t));
    if (!slots || !pos) return 3;
    for (int b = 0; b < B; ++b) slots[b] = b;
    void *dslots = to_device(slots, B * 4), *dpos = to_device(pos, B * 4);
    void* dcu = to_device(cu, ((size_t)B + 1) * 4);
    const size_t pool_b = kda_state_bytes(&s, B), ring_b = kda_conv_bytes(&s, B);
    const size_t ws_b = kda_prefill_workspace_bytes(&s, B, T), y_n = (size_t)T * H * d;
    void *pool = device_zeros(pool_b), *ring = device_zeros(ring_b), *ws = device_zeros(ws_b);
    void *y = device_zeros(y_n * 4), *status = device_zeros(4);
    if (!dslots || !dpos || !dcu || !pool || !ring || !ws || !y || !status) return 4;
    int rc = kda_prefill(&s, &p, B, (const int32_t*)dcu, T, max_len, B, (const int32_t*)dslots,
                         (const int32_t*)dpos, tok[0], tok[1], tok[2], tok[3], tok[4], tok[5],
                         pool, ring, (float*)y, ws, ws_b, (int32_t*)status, NULL);
    if (rc != KDA_OK) {
        fprintf(stderr, "kda_prefill: %s\n", kda_status_str(rc));
        return 5;
    }
    if (hipDeviceSynchronize() != hipSuccess) return 6;
    int32_t hstatus = -1;
    if (hipMemcpy(&hstatus, status, 4, hipMemcpyDeviceToHost) != hipSuccess) return 7;
    if (hstatus != 0) return 8;
    if (copy_out(dir, "y", y, y_n) != 0 || copy_out(dir, "state", pool, pool_b / 4) != 0)
        return 9;
    printf("prefill ok: B=%d H=%d d=%d tokens=%lld\n", B, H, d, (long long)T);
    return 0;
}

static int decode_from_files(const char* dir) {
    char path[1024];
    snprintf(path, sizeof(path), "%s/meta.txt", dir);
    FILE* f = fopen(path, "r");
    int B = 0, H = 0, d = 0;
    if (!f || fscanf(f, "%d %d %d", &B, &H, &d) != 3) return 2;
    fclose(f);
    const size_t C = 3 * (size_t)d, BH = (size_t)B * H;
    kda_shape s = make_shape(H, d);
    float* q = read_f32(dir, "q", BH * d);
    float* k = read_f32(dir, "k", BH * d);
    float* v = read_f32(dir, "v", BH * d);
    float* al = read_f32(dir, "alpha", BH * d);
    float* be = read_f32(dir, "beta", BH);
    float* g = read_f32(dir, "g", BH * d);
    float* wq = read_f32(dir, "wq", (size_t)H * d * 4);
    float* wk = read_f32(dir, "wk", (size_t)H * d * 4);
    float* wv = read_f32(dir, "wv", (size_t)H * d * 4);
    if (!q || !k || !v || !al || !be || !g || !wq || !wk || !wv) return 3;
    int32_t* slots = (int32_t*)malloc(B * sizeof(int32_t));
    int32_t* pos = (int32_t*)calloc(B, sizeof(int32_t));
    for (int b = 0; b < B; ++b) slots[b] = b;
    kda_params p;
    memset(&p, 0, sizeof(p));
    p.conv_w_q = (const float*)to_device(wq, (size_t)H * d * 4 * 4);
    p.conv_w_k = (const float*)to_device(wk, (size_t)H * d * 4 * 4);
    p.conv_w_v = (const float*)to_device(wv, (size_t)H * d * 4 * 4);
    void *dq = to_device(q, BH * d * 4), *dk = to_device(k, BH * d * 4);
    void *dv = to_device(v, BH * d * 4), *dal = to_device(al, BH * d * 4);
    void *dbe = to_device(be, BH * 4), *dg = to_device(g, BH * d * 4);
    void *dslots = to_device(slots, B * 4), *dpos = to_device(pos, B * 4);
    void *pool = NULL, *ring = NULL, *y = NULL, *status = NULL;
    const size_t pool_b = kda_state_bytes(&s, B), ring_b = kda_conv_bytes(&s, B);
    if (hipMalloc(&pool, pool_b) != hipSuccess || hipMalloc(&ring, ring_b) != hipSuccess ||
        hipMalloc(&y, BH * d * 4) != hipSuccess || hipMalloc(&status, 4) != hipSuccess)
        return 4;
    if (hipMemset(status, 0, 4) != hipSuccess) return 4;
    int rc = kda_decode(&s, &p, B, B, (const int32_t*)dslots, (const int32_t*)dpos, dq, dk, dv,
                        dal, dbe, dg, pool, ring, (float*)y, (int32_t*)status, NULL);
    if (rc != KDA_OK) {
        fprintf(stderr, "kda_decode: %s\n", kda_status_str(rc));
        return 5;
    }
    if (hipDeviceSynchronize() != hipSuccess) return 6;
    float* hy = (float*)malloc(BH * d * 4);
    float* hs = (float*)malloc(pool_b);
    int32_t hstatus = -1;
    if (hipMemcpy(hy, y, BH * d * 4, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(hs, pool, pool_b, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(&hstatus, status, 4, hipMemcpyDeviceToHost) != hipSuccess)
        return 7;
    if (hstatus != 0) return 8;
    if (write_f32(dir, "y", hy, BH * d) != 0 || write_f32(dir, "state", hs, pool_b / 4) != 0)
        return 9;
    (void)C;
    printf("decode ok: B=%d H=%d d=%d\n", B, H, d);
    return 0;
}

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) {
        int f = host_checks();
        printf("host checks: %d failed\n", f);
        return f ? 1 : 0;
    }
    if (argc >= 3 && strcmp(argv[1], "decode") == 0) return decode_from_files(argv[2]);
    if (argc >= 3 && strcmp(argv[1], "verify") == 0) return verify_from_files(argv[2]);
    if (argc >= 3 && strcmp(argv[1], "prefill") == 0) return prefill_from_files(argv[2]);
    fprintf(stderr, "usage: %s host | decode DIR | verify DIR | prefill DIR\n", argv[0]);
    return 2;
}
