/*
 * oracle_sanitize.c -- drives every function of the CPU oracle (oracle/oracle.h) through small
 * seeded shapes, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitize.py compiles and runs it).  Every buffer is allocated at exactly the
 * size the oracle's contract gives, so an access outside it is reported.  A few invariants are
 * checked so that the run provably went through the whole path:
 *   - the per-expert counts of every rank add up to its valid slots;
 *   - every rank receives what the others send to it and at most its B rows;
 *   - with identity experts, bf16 payloads and every slot present, the fp64-mode combine returns
 *     bf16(x * sum of the token's weights) within one bf16 ulp.
 * Exit status 0 on success; a sanitizer report or a failed check ends the program otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t rng_state;
static uint32_t next_u32(void) {  /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 2685821657736338717ULL) >> 32);
}
static float uniform(float lo, float hi) { return lo + (hi - lo) * (next_u32() / 4294967296.0f); }

static void* xalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    memset(p, 0, n ? n : 1);
    return p;
}

static void check(int ok, const char* what, int c) {
    if (!ok) { fprintf(stderr, "case %d: check failed: %s\n", c, what); exit(1); }
}

static uint16_t bf16_bits(float f) {  /* round to nearest even, finite inputs */
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void run_case(int c, int N, int L, int R, int T, int H, int fp8, int ragged) {
    const int E = N * L, TR = T * R;
    const long B = (long)N * T * (R > L ? R : L);
    int32_t* tokens = NULL;
    if (ragged) {
        tokens = xalloc(sizeof(int32_t) * N);
        for (int s = 0; s < N; ++s) tokens[s] = (s * 7 + c) % (T + 1);
    }
    oracle_shape sh = {N, T, H, E, R, fp8, B, NULL, tokens};
    const long P = oracle_row_bytes(&sh), NT = (long)N * T, M = NT * R, nsc = H / 128;

    float* logits = xalloc(sizeof(float) * NT * E);
    float* bias = xalloc(sizeof(float) * E);
    for (long i = 0; i < NT * E; ++i) logits[i] = uniform(-2.0f, 2.0f);
    for (int e = 0; e < E; ++e) bias[e] = (c & 1) ? -logf(1.0f + (float)e) : 0.0f;
    uint16_t* xb = xalloc(sizeof(uint16_t) * NT * H);
    for (long i = 0; i < NT * H; ++i) xb[i] = bf16_bits(uniform(-3.0f, 3.0f));

    int32_t* idx = xalloc(sizeof(int32_t) * M);
    float* w = xalloc(sizeof(float) * M);
    oracle_route((int)NT, E, R, logits, (c & 1) ? bias : NULL, idx, w);

    const uint8_t* x = (const uint8_t*)xb;
    uint8_t* q = NULL;
    float* xs = NULL;
    if (fp8) {
        q = xalloc(NT * H);
        xs = xalloc(sizeof(float) * NT * nsc);
        oracle_quantize_e4m3(NT, H, xb, q, xs);
        x = q;
    }

    int32_t* counts = xalloc(sizeof(int32_t) * N * E);
    int32_t* send_off = xalloc(sizeof(int32_t) * N * (N + 1));
    int32_t* send_pos = xalloc(sizeof(int32_t) * M);
    uint8_t* send_buf = xalloc(M * P);
    int32_t* send_meta = xalloc(sizeof(int32_t) * 2 * M);
    oracle_dispatch_send(&sh, x, xs, idx, counts, send_off, send_pos, send_buf, send_meta);
    for (int s = 0; s < N; ++s) {
        long sum = 0;
        for (int e = 0; e < E; ++e) sum += counts[(long)s * E + e];
        const long valid = (long)(tokens ? tokens[s] : T) * R;
        check(sum == valid, "counts add up to the valid slots", c);
        check(send_off[(long)s * (N + 1) + N] == sum, "send offsets end at the row count", c);
    }

    uint8_t* recv_buf = xalloc(N * B * P);
    int32_t* recv_meta = xalloc(sizeof(int32_t) * 2 * N * B);
    int32_t* recv_off = xalloc(sizeof(int32_t) * N * (N + 1));
    oracle_net_dispatch(&sh, send_off, send_buf, send_meta, recv_buf, recv_meta, recv_off);
    for (int d = 0; d < N; ++d) {
        long in = 0;
        for (int s = 0; s < N; ++s)
            in += send_off[(long)s * (N + 1) + d + 1] - send_off[(long)s * (N + 1) + d];
        check(recv_off[(long)d * (N + 1) + N] == in, "a rank receives what is sent to it", c);
        check(in <= B, "receive count within the bound", c);
    }

    const long xw = fp8 ? 1 : 2;
    uint8_t* expert_x = xalloc(N * B * H * xw);
    float* expert_scale = fp8 ? xalloc(sizeof(float) * N * B * nsc) : NULL;
    int32_t* expert_cnt = xalloc(sizeof(int32_t) * N * L);
    int32_t* expert_off = xalloc(sizeof(int32_t) * N * (L + 1));
    int32_t* expert_src = xalloc(sizeof(int32_t) * N * B);
    int32_t* expert_rpos = xalloc(sizeof(int32_t) * N * B);
    oracle_dispatch_recv(&sh, counts, recv_off, recv_buf, recv_meta, expert_x, expert_scale,
                         expert_cnt, expert_off, expert_src, expert_rpos);

    uint16_t* y = xalloc(sizeof(uint16_t) * N * B * H);
    uint16_t* cs = xalloc(sizeof(uint16_t) * N * B * H);
    uint16_t* cr = xalloc(sizeof(uint16_t) * M * H);
    uint16_t* out = xalloc(sizeof(uint16_t) * NT * H);
    for (int mode = 1; mode >= 0; --mode) {
        oracle_expert(&sh, mode, expert_x, expert_scale, expert_off, y);
        for (int cm = 0; cm < 2; ++cm) {
            oracle_combine(&sh, cm, y, expert_rpos, recv_off, send_off, send_pos, w, cs, cr, out);
            oracle_combine_acc(&sh, cm, y, expert_src, expert_rpos, recv_off, send_off, idx,
                               send_pos, w, cs, cr, out);
        }
    }
    if (!fp8 && !ragged) {  /* identity experts: out = bf16(x * sum w), fp64 mode */
        oracle_combine(&sh, 0, y, expert_rpos, recv_off, send_off, send_pos, w, cs, cr, out);
        for (long t = 0; t < NT; ++t) {
            double sw = 0.0;
            for (int k = 0; k < R; ++k) sw += w[t * R + k];
            for (int h = 0; h < H; ++h) {
                const double want = oracle_bf16_to_double(xb[t * H + h]) * sw;
                const double got = oracle_bf16_to_double(out[t * H + h]);
                check(fabs(got - want) <= fabs(want) * 0x1p-7 + 1e-30, "identity round trip", c);
            }
        }
    }

    /* prefill with replicated tokens: rank 0's token set stands in for the shared one */
    oracle_shape pf = {N, T, H, E, R, fp8, (long)T * (R > L ? R : L), NULL, NULL};
    int32_t* slot_pos = xalloc(sizeof(int32_t) * TR);
    uint8_t* pf_x = xalloc(N * pf.B * H * xw);
    float* pf_scale = fp8 ? xalloc(sizeof(float) * N * pf.B * nsc) : NULL;
    int32_t* pf_src = xalloc(sizeof(int32_t) * N * pf.B);
    oracle_prefill_dispatch(&pf, x, xs, idx, slot_pos, pf_x, pf_scale, expert_cnt, expert_off, pf_src);
    uint16_t* pf_y = xalloc(sizeof(uint16_t) * N * pf.B * H);
    float* partial = xalloc(sizeof(float) * N * T * H);
    oracle_expert(&pf, 0, pf_x, pf_scale, expert_off, pf_y);
    for (int cm = 0; cm < 2; ++cm)
        oracle_prefill_combine(&pf, cm, pf_y, slot_pos, idx, w, partial, out);

    free(logits); free(bias); free(xb); free(idx); free(w); free(q); free(xs); free(counts);
    free(send_off); free(send_pos); free(send_buf); free(send_meta); free(recv_buf); free(recv_meta);
    free(recv_off); free(expert_x); free(expert_scale); free(expert_cnt); free(expert_off);
    free(expert_src); free(expert_rpos); free(y); free(cs); free(cr); free(out); free(slot_pos);
    free(pf_x); free(pf_scale); free(pf_src); free(pf_y); free(partial); free(tokens);
}

int main(void) {
    int c = 0;
    static const int Ns[] = {1, 2, 3, 4}, Ls[] = {1, 2, 3}, Ts[] = {1, 5, 17};
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 3; ++b)
            for (int t = 0; t < 3; ++t) {
                const int N = Ns[a], L = Ls[b], T = Ts[t], E = N * L;
                const int R = 1 + (a + b + t) % (E < 4 ? E : 4);
                rng_state = 0x9E3779B97F4A7C15ULL ^ (uint64_t)(c + 1);
                run_case(c, N, L, R, T, 128 * (1 + (c % 2)), (c % 3) == 1, (c % 4) == 3);
                ++c;
            }
    printf("oracle sanitize: %d cases passed\n", c);
    return 0;
}
