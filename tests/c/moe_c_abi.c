/*
 * moe_c_abi.c -- the library driven from plain C through include/moe.h, with no Python or
 * torch: device memory and streams from the HIP runtime API, every call of the decode path and
 * of the replicated-token prefill path on a small problem, and every output checked against the
 * CPU oracle (oracle/oracle.h, test infrastructure) on the same inputs.
 *
 *   moe_c_abi            run on GPU 0; exit 0 and print "ok" when everything matches
 *   moe_c_abi --host     host-only checks (sizes, validation), no GPU needed
 *
 * Bars: indices, counts, offsets, positions, metadata and payload bytes bit-exact; router
 * weights within 1 fp32 ulp; combine outputs within 1 bf16 ulp of the oracle's fp64 sums.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moe.h"
#include "../../oracle/oracle.h"

static int failures = 0;

#define CHECK(cond, ...)                        \
    do {                                        \
        if (!(cond)) {                          \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");              \
            ++failures;                         \
        }                                       \
    } while (0)

#define HIP(x)                                                                    \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

#define MOE(x)                                                                    \
    do {                                                                          \
        int r_ = (x);                                                             \
        if (r_ != MOE_OK) {                                                       \
            fprintf(stderr, "%s failed: %d (%s)\n", #x, r_, moe_strerror(r_));    \
            exit(3);                                                              \
        }                                                                         \
    } while (0)

/* xorshift64* -- deterministic inputs */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 2685821657736338717ull;
}
static float rnd_uniform(float lo, float hi) { return lo + (hi - lo) * (float)((rnd() >> 40) * (1.0 / 16777216.0)); }

static uint16_t bf16_trunc(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void* dalloc(int64_t bytes) {
    void* p = NULL;
    HIP(hipMalloc(&p, bytes > 0 ? (size_t)bytes : 16));
    return p;
}
static void* halloc(int64_t bytes) {
    void* p = calloc(1, bytes > 0 ? (size_t)bytes : 16);
    if (!p) exit(4);
    return p;
}
static void h2d(void* d, const void* h, int64_t n) { HIP(hipMemcpy(d, h, (size_t)n, hipMemcpyHostToDevice)); }
static void d2h(void* h, const void* d, int64_t n) { HIP(hipMemcpy(h, d, (size_t)n, hipMemcpyDeviceToHost)); }

static int32_t key16(uint16_t b) { return (b & 0x8000) ? -(int32_t)(b & 0x7FFF) : (int32_t)(b & 0x7FFF); }
static int64_t f32_ulps(float a, float b) {
    int32_t ia, ib;
    memcpy(&ia, &a, 4);
    memcpy(&ib, &b, 4);
    return llabs((int64_t)ia - (int64_t)ib);
}

/* ---------------------------------------------------------------- host-only checks */

static void host_checks(void) {
    moe_shape sh;
    moe_sizes_t sz;
    memset(&sh, 0, sizeof sh);
    sh.N = 32; sh.T = 128; sh.H = 7168; sh.E = 256; sh.R = 8; sh.dtype = MOE_BF16;
    MOE(moe_sizes(&sh, &sz));
    CHECK(sz.capacity == 32 * 128 * 8, "capacity %lld", (long long)sz.capacity);
    CHECK(sz.row_bytes == 2 * 7168, "row bytes");
    sh.dtype = MOE_FP8_E4M3;
    MOE(moe_sizes(&sh, &sz));
    CHECK(sz.row_bytes == 7168 + 4 * 56, "fp8 row bytes");
    sh.E = 255;  /* not a multiple of N */
    CHECK(moe_sizes(&sh, &sz) == MOE_EINVAL, "E %% N != 0 accepted");
    sh.E = 256; sh.layout = MOE_LAYOUT_PREFILL; sh.dtype = MOE_BF16;
    MOE(moe_sizes(&sh, &sz));
    CHECK(sz.capacity == 128 * 8 && sz.partial == 32LL * 128 * 7168 * 4, "prefill sizes");
    CHECK(moe_abi_version() == MOE_ABI_VERSION, "abi version %d", moe_abi_version());
    CHECK(moe_route(NULL, NULL, NULL, NULL, NULL, NULL) == MOE_EINVAL, "null shape accepted");
    /* the no-allocation send refuses, before any device work, a call whose histograms exceed the
     * library's static array (1024 ranks and experts, 1600 slots per rank) */
    void* good = (void*)(uintptr_t)(1 << 20);
    memset(&sh, 0, sizeof sh);
    sh.N = 1024; sh.T = 200; sh.H = 64; sh.E = 1024; sh.R = 8; sh.dtype = MOE_BF16;
    MOE(moe_sizes(&sh, &sz));
    CHECK(sz.workspace > (int64_t)MOE_STATIC_SCRATCH_BYTES, "workspace %lld", (long long)sz.workspace);
    CHECK(moe_dispatch_send_noalloc(&sh, good, NULL, good, good, good, good, good, good, NULL) == MOE_ENOSCRATCH,
          "oversized no-allocation send accepted");
    CHECK(moe_stream_copy(good, (char*)good + 32, 64, NULL) == MOE_EINVAL, "overlapping copy accepted");
    CHECK(moe_stream_copy(good, (char*)good + 4096, 24, NULL) == MOE_EINVAL, "ragged copy accepted");
}

/* ---------------------------------------------------------------- no-allocation send, stream copy */

/* moe_dispatch_send_noalloc on a shape whose ranks span several count chunks (the static
 * histograms in use), against the oracle's dispatch send; then moe_stream_copy of its send buffer */
static void noalloc_and_copy(void) {
    const int N = 2, T = 700, H = 64, E = 32, R = 8;
    moe_shape sh;
    memset(&sh, 0, sizeof sh);
    sh.N = N; sh.T = T; sh.H = H; sh.E = E; sh.R = R; sh.dtype = MOE_BF16;
    moe_sizes_t sz;
    MOE(moe_sizes(&sh, &sz));
    CHECK(sz.workspace > 0, "this shape should need histograms");
    const int64_t P = sz.row_bytes, TR = (int64_t)T * R;
    float* logits = halloc(sz.logits);
    uint16_t* x = halloc(sz.x);
    for (int64_t i = 0; i < (int64_t)N * T * E; ++i) logits[i] = rnd_uniform(-3.0f, 3.0f);
    for (int64_t i = 0; i < (int64_t)N * T * H; ++i) x[i] = bf16_trunc(rnd_uniform(-2.0f, 2.0f));
    int32_t* status = dalloc(4);
    HIP(hipMemset(status, 0, 4));
    sh.status = status;
    void *d_logits = dalloc(sz.logits), *d_x = dalloc(sz.x), *d_idx = dalloc(sz.topk_idx), *d_w = dalloc(sz.topk_w),
         *d_counts = dalloc(sz.counts), *d_soff = dalloc(sz.send_off), *d_spos = dalloc(sz.send_pos),
         *d_sbuf = dalloc(sz.send_buf), *d_smeta = dalloc(sz.send_meta), *d_copy = dalloc(sz.send_buf);
    h2d(d_logits, logits, sz.logits);
    h2d(d_x, x, sz.x);
    MOE(moe_route(&sh, d_logits, NULL, d_idx, d_w, NULL));
    MOE(moe_dispatch_send_noalloc(&sh, d_x, NULL, d_idx, d_counts, d_soff, d_spos, d_sbuf, d_smeta, NULL));
    MOE(moe_stream_copy(d_sbuf, d_copy, sz.send_buf, NULL));
    HIP(hipDeviceSynchronize());
    int32_t* g_idx = halloc(sz.topk_idx); int32_t* g_counts = halloc(sz.counts);
    int32_t* g_soff = halloc(sz.send_off); int32_t* g_spos = halloc(sz.send_pos);
    uint8_t* g_sbuf = halloc(sz.send_buf); int32_t* g_smeta = halloc(sz.send_meta);
    uint8_t* g_copy = halloc(sz.send_buf);
    int32_t g_status = -99;
    d2h(g_idx, d_idx, sz.topk_idx); d2h(g_counts, d_counts, sz.counts); d2h(g_soff, d_soff, sz.send_off);
    d2h(g_spos, d_spos, sz.send_pos); d2h(g_sbuf, d_sbuf, sz.send_buf); d2h(g_smeta, d_smeta, sz.send_meta);
    d2h(g_copy, d_copy, sz.send_buf); d2h(&g_status, status, 4);
    oracle_shape osh = {N, T, H, E, R, 0, sz.capacity, NULL, NULL};
    int32_t* o_counts = halloc(sz.counts); int32_t* o_soff = halloc(sz.send_off);
    int32_t* o_spos = halloc(sz.send_pos); uint8_t* o_sbuf = halloc(sz.send_buf);
    int32_t* o_smeta = halloc(sz.send_meta);
    oracle_dispatch_send(&osh, (const uint8_t*)x, NULL, g_idx, o_counts, o_soff, o_spos, o_sbuf, o_smeta);
    CHECK(g_status == 0, "status word %d", g_status);
    CHECK(!memcmp(g_counts, o_counts, sz.counts), "no-allocation send: counts");
    CHECK(!memcmp(g_soff, o_soff, sz.send_off), "no-allocation send: send_off");
    CHECK(!memcmp(g_spos, o_spos, sz.send_pos), "no-allocation send: send_pos");
    for (int s = 0; s < N; ++s) {
        const int64_t n = o_soff[s * (N + 1) + N];
        CHECK(!memcmp(g_sbuf + s * TR * P, o_sbuf + s * TR * P, n * P), "no-allocation send: send_buf rank %d", s);
        CHECK(!memcmp(g_smeta + 2 * s * TR, o_smeta + 2 * s * TR, n * 8), "no-allocation send: send_meta rank %d", s);
    }
    CHECK(!memcmp(g_copy, g_sbuf, sz.send_buf), "stream copy differs from its source");
    printf("no-allocation send: N%d T%d H%d E%d R%d equal to the oracle; stream copy of %lld bytes exact\n",
           N, T, H, E, R, (long long)sz.send_buf);
}

/* ---------------------------------------------------------------- decode path */

static void decode_path(void) {
    const int N = 3, T = 37, H = 264, E = 9, R = 3, L = E / N;
    moe_shape sh;
    memset(&sh, 0, sizeof sh);
    sh.N = N; sh.T = T; sh.H = H; sh.E = E; sh.R = R; sh.dtype = MOE_BF16;
    moe_sizes_t sz;
    MOE(moe_sizes(&sh, &sz));
    const int64_t B = sz.capacity, P = sz.row_bytes, TR = (int64_t)T * R;

    float* logits = halloc(sz.logits);
    uint16_t* x = halloc(sz.x);
    for (int64_t i = 0; i < (int64_t)N * T * E; ++i) logits[i] = rnd_uniform(-3.0f, 3.0f);
    for (int64_t i = 0; i < (int64_t)N * T * H; ++i) x[i] = bf16_trunc(rnd_uniform(-2.0f, 2.0f));

    /* device buffers */
    int32_t* status = dalloc(4);
    HIP(hipMemset(status, 0, 4));
    sh.status = status;
    void *d_logits = dalloc(sz.logits), *d_x = dalloc(sz.x), *d_idx = dalloc(sz.topk_idx),
         *d_w = dalloc(sz.topk_w), *d_counts = dalloc(sz.counts), *d_soff = dalloc(sz.send_off),
         *d_spos = dalloc(sz.send_pos), *d_sbuf = dalloc(sz.send_buf), *d_smeta = dalloc(sz.send_meta),
         *d_rbuf = dalloc(sz.recv_buf), *d_rmeta = dalloc(sz.recv_meta), *d_roff = dalloc(sz.recv_off),
         *d_ex = dalloc(sz.expert_x), *d_ecnt = dalloc(sz.expert_cnt), *d_eoff = dalloc(sz.expert_off),
         *d_esrc = dalloc(sz.expert_src), *d_erpos = dalloc(sz.expert_rpos), *d_ey = dalloc(sz.expert_y),
         *d_cs = dalloc(sz.cs_buf), *d_cr = dalloc(sz.cr_buf), *d_out = dalloc(sz.out),
         *d_ws = dalloc(sz.workspace);
    h2d(d_logits, logits, sz.logits);
    h2d(d_x, x, sz.x);
    hipStream_t st;
    HIP(hipStreamCreate(&st));
    MOE(moe_route(&sh, d_logits, NULL, d_idx, d_w, st));
    MOE(moe_dispatch_send(&sh, d_x, NULL, d_idx, d_counts, d_soff, d_spos, d_sbuf, d_smeta, d_ws, st));
    MOE(moe_net_dispatch(&sh, d_soff, d_sbuf, d_smeta, d_rbuf, d_rmeta, d_roff, st));
    MOE(moe_dispatch_recv(&sh, d_counts, d_roff, d_rbuf, d_rmeta, d_ex, NULL, d_ecnt, d_eoff, d_esrc,
                          d_erpos, st));
    MOE(moe_expert_stub(&sh, 1, d_ex, NULL, d_eoff, d_ey, st));
    MOE(moe_combine_send(&sh, d_ey, d_erpos, d_roff, d_soff, d_cs, d_cr, st));
    MOE(moe_combine_recv(&sh, d_cr, d_spos, d_w, d_out, st));
    HIP(hipStreamSynchronize(st));

    /* host copies */
    int32_t* g_idx = halloc(sz.topk_idx); float* g_w = halloc(sz.topk_w);
    int32_t* g_counts = halloc(sz.counts); int32_t* g_soff = halloc(sz.send_off);
    int32_t* g_spos = halloc(sz.send_pos); uint8_t* g_sbuf = halloc(sz.send_buf);
    int32_t* g_smeta = halloc(sz.send_meta); uint8_t* g_rbuf = halloc(sz.recv_buf);
    int32_t* g_roff = halloc(sz.recv_off); uint16_t* g_ex = halloc(sz.expert_x);
    int32_t* g_ecnt = halloc(sz.expert_cnt); int32_t* g_eoff = halloc(sz.expert_off);
    int32_t* g_esrc = halloc(sz.expert_src); int32_t* g_erpos = halloc(sz.expert_rpos);
    uint16_t* g_ey = halloc(sz.expert_y); uint16_t* g_out = halloc(sz.out);
    int32_t g_status = -99;
    d2h(g_idx, d_idx, sz.topk_idx); d2h(g_w, d_w, sz.topk_w); d2h(g_counts, d_counts, sz.counts);
    d2h(g_soff, d_soff, sz.send_off); d2h(g_spos, d_spos, sz.send_pos); d2h(g_sbuf, d_sbuf, sz.send_buf);
    d2h(g_smeta, d_smeta, sz.send_meta); d2h(g_rbuf, d_rbuf, sz.recv_buf); d2h(g_roff, d_roff, sz.recv_off);
    d2h(g_ex, d_ex, sz.expert_x); d2h(g_ecnt, d_ecnt, sz.expert_cnt); d2h(g_eoff, d_eoff, sz.expert_off);
    d2h(g_esrc, d_esrc, sz.expert_src); d2h(g_erpos, d_erpos, sz.expert_rpos); d2h(g_ey, d_ey, sz.expert_y);
    d2h(g_out, d_out, sz.out); d2h(&g_status, status, 4);

    /* the oracle on the same inputs (same receive stride B) */
    oracle_shape osh = {N, T, H, E, R, 0, B, NULL, NULL};
    int32_t* o_idx = halloc(sz.topk_idx); float* o_w = halloc(sz.topk_w);
    int32_t* o_counts = halloc(sz.counts); int32_t* o_soff = halloc(sz.send_off);
    int32_t* o_spos = halloc(sz.send_pos); uint8_t* o_sbuf = halloc(sz.send_buf);
    int32_t* o_smeta = halloc(sz.send_meta); uint8_t* o_rbuf = halloc(sz.recv_buf);
    int32_t* o_rmeta = halloc(sz.recv_meta); int32_t* o_roff = halloc(sz.recv_off);
    uint16_t* o_ex = halloc(sz.expert_x); int32_t* o_ecnt = halloc(sz.expert_cnt);
    int32_t* o_eoff = halloc(sz.expert_off); int32_t* o_esrc = halloc(sz.expert_src);
    int32_t* o_erpos = halloc(sz.expert_rpos); uint16_t* o_ey = halloc(sz.expert_y);
    uint16_t* o_cs = halloc(sz.cs_buf); uint16_t* o_cr = halloc(sz.cr_buf); uint16_t* o_out = halloc(sz.out);
    oracle_route(N * T, E, R, logits, NULL, o_idx, o_w);
    oracle_dispatch_send(&osh, (const uint8_t*)x, NULL, o_idx, o_counts, o_soff, o_spos, o_sbuf, o_smeta);
    oracle_net_dispatch(&osh, o_soff, o_sbuf, o_smeta, o_rbuf, o_rmeta, o_roff);
    oracle_dispatch_recv(&osh, o_counts, o_roff, o_rbuf, o_rmeta, (uint8_t*)o_ex, NULL, o_ecnt, o_eoff,
                         o_esrc, o_erpos);
    oracle_expert(&osh, 1, (const uint8_t*)o_ex, NULL, o_eoff, o_ey);
    oracle_combine(&osh, 0, o_ey, o_erpos, o_roff, o_soff, o_spos, o_w, o_cs, o_cr, o_out);

    CHECK(g_status == 0, "status word %d", g_status);
    CHECK(!memcmp(g_idx, o_idx, sz.topk_idx), "topk_idx");
    for (int64_t i = 0; i < (int64_t)N * T * R; ++i) CHECK(f32_ulps(g_w[i], o_w[i]) <= 1, "topk_w[%lld]", (long long)i);
    CHECK(!memcmp(g_counts, o_counts, sz.counts), "counts");
    CHECK(!memcmp(g_soff, o_soff, sz.send_off), "send_off");
    CHECK(!memcmp(g_spos, o_spos, sz.send_pos), "send_pos");
    CHECK(!memcmp(g_roff, o_roff, sz.recv_off), "recv_off");
    CHECK(!memcmp(g_ecnt, o_ecnt, sz.expert_cnt), "expert_cnt");
    CHECK(!memcmp(g_eoff, o_eoff, sz.expert_off), "expert_off");
    for (int s = 0; s < N; ++s) {
        const int64_t n = o_soff[s * (N + 1) + N];
        CHECK(!memcmp(g_sbuf + s * TR * P, o_sbuf + s * TR * P, n * P), "send_buf rank %d", s);
        CHECK(!memcmp(g_smeta + 2 * s * TR, o_smeta + 2 * s * TR, n * 8), "send_meta rank %d", s);
    }
    for (int d = 0; d < N; ++d) {
        const int64_t n = o_roff[d * (N + 1) + N];
        CHECK(!memcmp(g_rbuf + d * B * P, o_rbuf + d * B * P, n * P), "recv_buf rank %d", d);
        CHECK(!memcmp(g_ex + d * B * H, o_ex + d * B * H, n * 2 * H), "expert_x rank %d", d);
        CHECK(!memcmp(g_esrc + d * B, o_esrc + d * B, n * 4), "expert_src rank %d", d);
        CHECK(!memcmp(g_erpos + d * B, o_erpos + d * B, n * 4), "expert_rpos rank %d", d);
        CHECK(!memcmp(g_ey + d * B * H, o_ey + d * B * H, n * 2 * H), "expert_y rank %d", d);
    }
    int worst = 0;
    for (int64_t i = 0; i < (int64_t)N * T * H; ++i) {
        const int dd = abs(key16(g_out[i]) - key16(o_out[i]));
        if (dd > worst) worst = dd;
    }
    CHECK(worst <= 1, "combine out differs by %d bf16 ulp", worst);

    /* the combine with the sum on the sending side, on the same dispatched buffers: bit for bit
     * against the oracle's fp32 steps for every token whose router weights are identical */
    MOE(moe_combine_acc(&sh, d_ey, d_rmeta, d_counts, d_roff, d_eoff, d_soff, d_w, d_idx, d_spos, d_cs,
                        d_cr, d_out, st));
    HIP(hipStreamSynchronize(st));
    d2h(g_out, d_out, sz.out);
    d2h(&g_status, status, 4);
    CHECK(g_status == 0, "status word after the send-side sum %d", g_status);
    oracle_combine_acc(&osh, 1, o_ey, o_esrc, o_erpos, o_roff, o_soff, o_idx, o_spos, o_w, o_cs, o_cr, o_out);
    int64_t acc_tokens = 0;
    for (int64_t tok = 0; tok < (int64_t)N * T; ++tok) {
        if (memcmp(g_w + tok * R, o_w + tok * R, 4 * R)) continue;
        CHECK(!memcmp(g_out + tok * H, o_out + tok * H, 2 * H), "send-side sum, token %lld", (long long)tok);
        ++acc_tokens;
    }
    (void)L;
    printf("decode path: N%d T%d H%d E%d R%d checked (max %d bf16 ulp); send-side sum bit-exact on %lld tokens\n",
           N, T, H, E, R, worst, (long long)acc_tokens);
    HIP(hipStreamDestroy(st));
}

/* ---------------------------------------------------------------- prefill path */

static void prefill_path(void) {
    const int N = 4, T = 300, H = 512, E = 16, R = 4;
    moe_shape sh;
    memset(&sh, 0, sizeof sh);
    sh.N = N; sh.T = T; sh.H = H; sh.E = E; sh.R = R; sh.dtype = MOE_BF16; sh.layout = MOE_LAYOUT_PREFILL;
    moe_sizes_t sz;
    MOE(moe_sizes(&sh, &sz));
    const int64_t B = sz.capacity;
    float* logits = halloc(sz.logits);
    uint16_t* x = halloc(sz.x);
    for (int64_t i = 0; i < (int64_t)T * E; ++i) logits[i] = rnd_uniform(-3.0f, 3.0f);
    for (int64_t i = 0; i < (int64_t)T * H; ++i) x[i] = bf16_trunc(rnd_uniform(-2.0f, 2.0f));
    int32_t* status = dalloc(4);
    HIP(hipMemset(status, 0, 4));
    sh.status = status;
    void *d_logits = dalloc(sz.logits), *d_x = dalloc(sz.x), *d_idx = dalloc(sz.topk_idx),
         *d_w = dalloc(sz.topk_w), *d_pos = dalloc(sz.slot_pos), *d_ex = dalloc(sz.expert_x),
         *d_ecnt = dalloc(sz.expert_cnt), *d_eoff = dalloc(sz.expert_off), *d_esrc = dalloc(sz.expert_src),
         *d_ey = dalloc(sz.expert_y), *d_part = dalloc(sz.partial), *d_out = dalloc(sz.out),
         *d_ws = dalloc(sz.workspace);
    h2d(d_logits, logits, sz.logits);
    h2d(d_x, x, sz.x);
    MOE(moe_route(&sh, d_logits, NULL, d_idx, d_w, NULL));
    MOE(moe_prefill_dispatch(&sh, d_x, NULL, d_idx, d_pos, d_ex, NULL, d_ecnt, d_eoff, d_esrc, d_ws, NULL));
    MOE(moe_expert_stub(&sh, 1, d_ex, NULL, d_eoff, d_ey, NULL));
    MOE(moe_prefill_combine(&sh, d_ey, d_idx, d_pos, d_w, d_part, d_out, NULL));
    HIP(hipDeviceSynchronize());
    int32_t* g_pos = halloc(sz.slot_pos); uint16_t* g_ex = halloc(sz.expert_x);
    int32_t* g_eoff = halloc(sz.expert_off); int32_t* g_esrc = halloc(sz.expert_src);
    float* g_part = halloc(sz.partial); uint16_t* g_out = halloc(sz.out);
    int32_t g_status = -99;
    d2h(g_pos, d_pos, sz.slot_pos); d2h(g_ex, d_ex, sz.expert_x); d2h(g_eoff, d_eoff, sz.expert_off);
    d2h(g_esrc, d_esrc, sz.expert_src); d2h(g_part, d_part, sz.partial); d2h(g_out, d_out, sz.out);
    d2h(&g_status, status, 4);

    oracle_shape osh = {N, T, H, E, R, 0, B, NULL, NULL};
    int32_t* o_idx = halloc(sz.topk_idx); float* o_w = halloc(sz.topk_w);
    int32_t* o_pos = halloc(sz.slot_pos); uint16_t* o_ex = halloc(sz.expert_x);
    int32_t* o_ecnt = halloc(sz.expert_cnt); int32_t* o_eoff = halloc(sz.expert_off);
    int32_t* o_esrc = halloc(sz.expert_src); uint16_t* o_ey = halloc(sz.expert_y);
    float* o_part = halloc(sz.partial); uint16_t* o_out = halloc(sz.out);
    oracle_route(T, E, R, logits, NULL, o_idx, o_w);
    oracle_prefill_dispatch(&osh, (const uint8_t*)x, NULL, o_idx, o_pos, (uint8_t*)o_ex, NULL, o_ecnt,
                            o_eoff, o_esrc);
    oracle_expert(&osh, 1, (const uint8_t*)o_ex, NULL, o_eoff, o_ey);
    oracle_prefill_combine(&osh, 0, o_ey, o_pos, o_idx, o_w, o_part, o_out);

    CHECK(g_status == 0, "prefill status word %d", g_status);
    CHECK(!memcmp(g_pos, o_pos, sz.slot_pos), "slot_pos");
    CHECK(!memcmp(g_eoff, o_eoff, sz.expert_off), "prefill expert_off");
    for (int d = 0; d < N; ++d) {
        const int64_t n = o_eoff[d * (E / N + 1) + E / N];
        CHECK(!memcmp(g_ex + d * B * H, o_ex + d * B * H, n * 2 * H), "prefill expert_x rank %d", d);
        CHECK(!memcmp(g_esrc + d * B, o_esrc + d * B, n * 4), "prefill expert_src rank %d", d);
    }
    int worst = 0;
    for (int64_t i = 0; i < (int64_t)T * H; ++i) {
        const int dd = abs(key16(g_out[i]) - key16(o_out[i]));
        if (dd > worst) worst = dd;
    }
    CHECK(worst <= 1, "prefill out differs by %d bf16 ulp", worst);
    printf("prefill path: N%d T%d H%d E%d R%d checked (max %d bf16 ulp)\n", N, T, H, E, R, worst);
}

int main(int argc, char** argv) {
    host_checks();
    if (!(argc > 1 && !strcmp(argv[1], "--host"))) {
        int n = 0;
        HIP(hipGetDeviceCount(&n));
        if (n < 1) {
            fprintf(stderr, "no GPU\n");
            return 2;
        }
        HIP(hipSetDevice(0));
        decode_path();
        prefill_path();
        noalloc_and_copy();
    }
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
