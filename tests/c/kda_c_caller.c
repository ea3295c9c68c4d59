/*
 * A plain C caller of the KDA C-ABI (include/kda.h, libkda.so): no Python.
 *
 *   kda_c_caller host            host-side checks only (no GPU needed):
 *                                size queries, status strings and errors
 *                                returned before any launch; exit 0 if all hold
 *   kda_c_caller decode DIR      one decode call on the GPU: reads the inputs
 *                                DIR/{meta.txt, *.f32} written by the test,
 *                                writes DIR/y.f32 and DIR/state.f32
 *
 * Shapes for "decode": batch B, heads H, dk = dv = d (64 or 128), FP32
 * activations and FP32 state, slots 0..B-1, positions 0 (fresh sequences).
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
    fprintf(stderr, "usage: %s host | decode DIR\n", argv[0]);
    return 2;
}
