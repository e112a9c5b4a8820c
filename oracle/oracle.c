/*
 * oracle.c -- plain, slow CPU oracle for MoE expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and the benchmark's CPU-baseline
 * leg, never by the product.  Plain loops in the order the pages describe the method; no
 * blocking, fusion or reordering.  Floating point the method computes is done in fp64 and
 * rounded once.  Build with -ffp-contract=off and without fast-math so that every fp32
 * operation written here is exactly one IEEE operation.
 *
 * Pages cited: [EFA] "Enabling trillion-parameter models on AWS EFA";
 * [PORT] "Efficient and portable mixture-of-experts communication";
 * [DSK] "Lower latency and higher throughput with multi-node DeepSeek deployment";
 * [QWEN] "Hosting Qwen on Blackwell".
 *
 * Readings of the pages taken here (the pages leave these steps open):
 *  - expert e lives on rank e / L, L = E / N (contiguous blocks; [DSK] Expert Parallelism only
 *    says each GPU holds E / EP experts);
 *  - one row per (token, slot), i.e. one copy per routed expert ([PORT] Dispatch: the same
 *    buffer is sent once to each expert);
 *  - slot order is descending (logit + bias), ties to the lower expert id; the weights are the
 *    softmax of the selected R values; combine does not renormalise;
 *  - inside a send segment rows keep the (token, slot) order; the receive buffer therefore
 *    holds rows in (source, token, slot) order and the expert-major tensor in
 *    (local expert, source, token, slot) order.
 */
#include "oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* First receive-side row of rank d, and how many rows rank d has room for. */
static long rrow0(const oracle_shape* sh, int d) { return sh->rbase ? sh->rbase[d] : (long)d * sh->B; }
static long rcap(const oracle_shape* sh, int d) {
    return sh->rbase ? sh->rbase[d + 1] - sh->rbase[d] : sh->B;
}

/* Tokens rank s dispatches. */
static int ntok(const oracle_shape* sh, int s) {
    if (!sh->tokens) return sh->T;
    assert(sh->tokens[s] >= 0 && sh->tokens[s] <= sh->T);
    return sh->tokens[s];
}

long oracle_row_bytes(const oracle_shape* sh) {
    if (!sh->fp8) return 2L * sh->H;
    return (long)sh->H + 4L * (sh->H / 128);
}

/* ---------------------------------------------------------------- scalar formats */

/* bf16 = the upper half of an IEEE binary32: 1 sign, 8 exponent, 7 fraction bits.  Round a
 * double to the nearest bf16 value, ties to even, by scaling it so that one bf16 ulp becomes
 * 1.0 (an exact power-of-two scaling), rounding to an integer with nearbyint (the default
 * rounding mode is to-nearest-even) and scaling back. */
uint16_t oracle_bf16_from_double(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int ex;
    frexp(a, &ex);                     /* a = m * 2^ex, 0.5 <= m < 1 */
    int ulp_exp = ex - 8;              /* 8 significant bits */
    if (ulp_exp < -133) ulp_exp = -133; /* subnormal spacing 2^-126 * 2^-7 */
    double q = nearbyint(ldexp(a, -ulp_exp));
    double r = ldexp(q, ulp_exp);
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (r > bf16_max) return sign | 0x7F80;
    float f = (float)r;                /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; S.1111.111 is
 * NaN; exponent field 0 holds subnormals m/8 * 2^-6. */
double oracle_e4m3_to_double(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Nearest e4m3 value to v, ties to the even code, magnitudes above 448 clamped to 448.  The
 * spacing of e4m3 values at |v| is 2^(floor(log2|v|) - 3) for |v| >= 2^-6 (three mantissa bits)
 * and 2^-9 below (subnormals); v / spacing is exact (a power-of-two scaling) and nearbyint
 * rounds it to the nearest integer, ties to even, whose parity is the code's last bit. */
uint8_t oracle_e4m3_from_float_sat(float v) {
    assert(isfinite(v));
    const uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    int ex;
    frexp(a, &ex);                       /* a = m * 2^ex, 0.5 <= m < 1, so floor(log2 a) = ex - 1 */
    int sp = (a >= ldexp(1.0, -6)) ? ex - 1 - 3 : -9;
    double r = ldexp(nearbyint(ldexp(a, -sp)), sp);
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    uint8_t code;
    if (r < ldexp(1.0, -6)) {
        code = (uint8_t)ldexp(r, 9);     /* subnormal: r = m * 2^-9, m = 1..7 */
    } else {
        frexp(r, &ex);                   /* rounding may have carried into the next binade */
        int e = ex - 1;                  /* r = (8 + m) / 8 * 2^e */
        int m = (int)ldexp(r, 3 - e) - 8;
        code = (uint8_t)(((e + 7) << 3) | m);
    }
    return sign | code;
}

/* [DSK] Implementation, Quantization and the activation-kernel paragraph after it: activations
 * are quantised on the fly with one scaling factor per 128-element vector, found from the
 * block's largest absolute value.  The fp8 format (OCP E4M3, largest finite 448) and
 * scale = amax / 448 are readings; both divisions are single fp32 operations. */
void oracle_quantize_e4m3(long n_rows, int H, const uint16_t* x, uint8_t* q, float* scale) {
    assert(H % 128 == 0);
    const int nb = H / 128;
    for (long n = 0; n < n_rows; ++n) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t* xb = x + n * H + b * 128;
            float amax = 0.0f;
            for (int i = 0; i < 128; ++i) {
                float a = fabsf((float)oracle_bf16_to_double(xb[i]));
                if (a > amax) amax = a;
            }
            float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
            scale[n * nb + b] = sc;
            for (int i = 0; i < 128; ++i)
                q[n * H + b * 128 + i] =
                    oracle_e4m3_from_float_sat((float)oracle_bf16_to_double(xb[i]) / sc);
        }
    }
}

/* ---------------------------------------------------------------- routing */

/* [DSK] Expert Parallelism: each token goes to 8 of the 256 routed experts and the expert
 * results are summed with weights.  [DSK] MoE Router: the router sorts the scores while
 * tracking the indices of the sorted elements.  [PORT] introduction: weights come from the
 * router's probability distribution and the output is a weighted average.
 * Selection: R passes, each taking the best unselected expert under (v desc, e asc). */
void oracle_route_tokens(int t0, int t1, int E, int R, const float* logits, const float* bias,
                         int32_t* topk_idx, float* topk_w) {
    assert(E >= 1 && R >= 1 && R <= E && 0 <= t0 && t0 <= t1);
    float* v = (float*)malloc(sizeof(float) * E);
    char* taken = (char*)malloc(E);
    double* z = (double*)malloc(sizeof(double) * R);
    for (int n = t0; n < t1; ++n) {
        for (int e = 0; e < E; ++e) {
            float l = logits[(long)n * E + e];
            assert(isfinite(l));
            v[e] = bias ? l + bias[e] : l; /* one fp32 addition */
            taken[e] = 0;
        }
        for (int k = 0; k < R; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || v[e] > v[best]) best = e; /* strict '>' keeps the lower id on ties */
            }
            taken[best] = 1;
            topk_idx[(long)n * R + k] = best;
        }
        /* softmax over the selected values, in fp64, shifted by the largest (slot 0) */
        double v0 = (double)v[topk_idx[(long)n * R]];
        double sum = 0.0;
        for (int k = 0; k < R; ++k) {
            z[k] = exp((double)v[topk_idx[(long)n * R + k]] - v0);
            sum += z[k];
        }
        for (int k = 0; k < R; ++k) topk_w[(long)n * R + k] = (float)(z[k] / sum);
    }
    free(v);
    free(taken);
    free(z);
}

void oracle_route(int n_tokens, int E, int R, const float* logits, const float* bias,
                  int32_t* topk_idx, float* topk_w) {
    oracle_route_tokens(0, n_tokens, E, R, logits, bias, topk_idx, topk_w);
}

/* ---------------------------------------------------------------- dispatch */

/* [EFA] dispatch timing paragraph: the send kernel counts tokens per expert, takes a cumulative
 * sum of the counts to find the offsets that pack tokens into send buffers contiguous per peer,
 * and packs them.  [EFA] send-buffer paragraph: senders must lay out their writes contiguously.
 * [PORT] Dispatch: activations, block scales and the token's index travel together.
 * Row metadata: meta[0] = e*T*R + t*R + k (expert and source slot), meta[1] = how many earlier
 * slots of the same source chose the same expert. */
void oracle_dispatch_send_ranks(const oracle_shape* sh, int r0, int r1, const uint8_t* x,
                                const float* x_scale, const int32_t* topk_idx, int32_t* counts,
                                int32_t* send_off, int32_t* send_pos, uint8_t* send_buf,
                                int32_t* send_meta) {
    const int N = sh->N, T = sh->T, H = sh->H, E = sh->E, R = sh->R;
    assert(N >= 1 && E % N == 0 && 0 <= r0 && r0 <= r1 && r1 <= N);
    const int L = E / N;
    const long P = oracle_row_bytes(sh);
    const long TR = (long)T * R;
    const long xrow = sh->fp8 ? H : 2L * H; /* payload bytes of one token */
    const int nsc = H / 128;               /* fp8 block scales per token */
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * N);
    int32_t* seen = (int32_t*)malloc(sizeof(int32_t) * E);
    for (int s = r0; s < r1; ++s) {
        const int32_t* idx = topk_idx + s * TR;
        int32_t* cnt = counts + (long)s * E;
        int32_t* off = send_off + (long)s * (N + 1);
        const int Ts = ntok(sh, s);
        /* per-expert token counts */
        for (int e = 0; e < E; ++e) cnt[e] = 0;
        for (long i = (long)Ts * R; i < TR; ++i) send_pos[s * TR + i] = -1; /* absent tokens */
        for (long i = 0; i < (long)Ts * R; ++i) {
            int e = idx[i];
            assert(e >= 0 && e < E);
            cnt[e] += 1;
        }
        /* per-destination sizes, exclusive scan */
        off[0] = 0;
        for (int d = 0; d < N; ++d) {
            int n = 0;
            for (int e = d * L; e < (d + 1) * L; ++e) n += cnt[e];
            off[d + 1] = off[d] + n;
        }
        /* pack in (token, slot) order */
        for (int d = 0; d < N; ++d) fill[d] = 0;
        for (int e = 0; e < E; ++e) seen[e] = 0;
        for (int t = 0; t < Ts; ++t) {
            for (int k = 0; k < R; ++k) {
                long i = (long)t * R + k;
                int e = idx[i];
                for (int kk = 0; kk < k; ++kk) assert(idx[(long)t * R + kk] != e); /* distinct */
                int d = e / L;
                long pos = off[d] + fill[d];
                fill[d] += 1;
                send_pos[s * TR + i] = (int32_t)pos;
                uint8_t* row = send_buf + ((long)s * TR + pos) * P;
                memcpy(row, x + ((long)s * T + t) * xrow, xrow);
                if (sh->fp8)
                    memcpy(row + xrow, x_scale + ((long)s * T + t) * nsc, 4L * nsc);
                int32_t* meta = send_meta + 2 * ((long)s * TR + pos);
                meta[0] = (int32_t)((long)e * TR + i);
                meta[1] = seen[e];
                seen[e] += 1;
            }
        }
    }
    free(fill);
    free(seen);
}

void oracle_dispatch_send(const oracle_shape* sh, const uint8_t* x, const float* x_scale,
                          const int32_t* topk_idx, int32_t* counts, int32_t* send_off,
                          int32_t* send_pos, uint8_t* send_buf, int32_t* send_meta) {
    oracle_dispatch_send_ranks(sh, 0, sh->N, x, x_scale, topk_idx, counts, send_off, send_pos,
                               send_buf, send_meta);
}

/* [EFA] send-buffer paragraph: once the per-expert counts are exchanged every rank knows where
 * its writes land and at which offset each source's tokens arrive; the bulk then moves as one
 * write per peer.  recv_off[d][s] = sum over s' < s of what s' sends to d. */
void oracle_net_dispatch_ranks(const oracle_shape* sh, int r0, int r1, const int32_t* send_off,
                               const uint8_t* send_buf, const int32_t* send_meta, uint8_t* recv_buf,
                               int32_t* recv_meta, int32_t* recv_off) {
    const int N = sh->N;
    const long P = oracle_row_bytes(sh);
    const long TR = (long)sh->T * sh->R;
    assert(0 <= r0 && r0 <= r1 && r1 <= N);
    for (int d = r0; d < r1; ++d) {
        int32_t* roff = recv_off + (long)d * (N + 1);
        roff[0] = 0;
        for (int s = 0; s < N; ++s) {
            const int32_t* soff = send_off + (long)s * (N + 1);
            roff[s + 1] = roff[s] + (soff[d + 1] - soff[d]);
        }
        assert(roff[N] <= rcap(sh, d));
        for (int s = 0; s < N; ++s) {
            const int32_t* soff = send_off + (long)s * (N + 1);
            long n = soff[d + 1] - soff[d];
            long src = (long)s * TR + soff[d];
            long dst = rrow0(sh, d) + roff[s];
            memcpy(recv_buf + dst * P, send_buf + src * P, n * P);
            memcpy(recv_meta + 2 * dst, send_meta + 2 * src, 8 * n);
        }
    }
}

void oracle_net_dispatch(const oracle_shape* sh, const int32_t* send_off, const uint8_t* send_buf,
                         const int32_t* send_meta, uint8_t* recv_buf, int32_t* recv_meta,
                         int32_t* recv_off) {
    oracle_net_dispatch_ranks(sh, 0, sh->N, send_off, send_buf, send_meta, recv_buf, recv_meta,
                              recv_off);
}

/* [PORT] Dispatch: the receiver copies tokens into contiguous buffers that feed the grouped
 * GEMM, grouping tokens of one expert together, and stores source rank, expert index and token
 * index for combine.  Expert-major order: walking the receive rows in order and appending each
 * to its local expert's group keeps (source, token, slot) order inside the group. */
void oracle_dispatch_recv_ranks(const oracle_shape* sh, int r0, int r1, const int32_t* counts,
                                const int32_t* recv_off, const uint8_t* recv_buf,
                                const int32_t* recv_meta, uint8_t* expert_x, float* expert_scale,
                                int32_t* expert_cnt, int32_t* expert_off, int32_t* expert_src,
                                int32_t* expert_rpos) {
    const int N = sh->N, H = sh->H, E = sh->E;
    assert(0 <= r0 && r0 <= r1 && r1 <= N);
    const int L = E / N;
    const long P = oracle_row_bytes(sh);
    const long TR = (long)sh->T * sh->R;
    const long xrow = sh->fp8 ? H : 2L * H;
    const int nsc = H / 128;
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * L);
    for (int d = r0; d < r1; ++d) {
        int32_t* ecnt = expert_cnt + (long)d * L;
        int32_t* eoff = expert_off + (long)d * (L + 1);
        const int32_t* roff = recv_off + (long)d * (N + 1);
        eoff[0] = 0;
        for (int j = 0; j < L; ++j) {
            int c = 0;
            for (int s = 0; s < N; ++s) c += counts[(long)s * E + d * L + j];
            ecnt[j] = c;
            eoff[j + 1] = eoff[j] + c;
        }
        assert(eoff[L] == roff[N]);
        for (int j = 0; j < L; ++j) fill[j] = 0;
        int s = 0;
        for (long r = 0; r < roff[N]; ++r) {
            while (r >= roff[s + 1]) ++s; /* source rank of receive row r */
            const int32_t* meta = recv_meta + 2 * (rrow0(sh, d) + r);
            int e = (int)(meta[0] / TR);
            long i = meta[0] % TR;
            assert(e / L == d);
            int j = e - d * L;
            long q = eoff[j] + fill[j];
            fill[j] += 1;
            const uint8_t* row = recv_buf + (rrow0(sh, d) + r) * P;
            memcpy(expert_x + (rrow0(sh, d) + q) * xrow, row, xrow);
            if (sh->fp8)
                memcpy(expert_scale + (rrow0(sh, d) + q) * nsc, row + xrow, 4L * nsc);
            expert_src[rrow0(sh, d) + q] = (int32_t)((long)s * TR + i);
            expert_rpos[rrow0(sh, d) + q] = (int32_t)r;
        }
    }
    free(fill);
}

void oracle_dispatch_recv(const oracle_shape* sh, const int32_t* counts, const int32_t* recv_off,
                          const uint8_t* recv_buf, const int32_t* recv_meta, uint8_t* expert_x,
                          float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                          int32_t* expert_src, int32_t* expert_rpos) {
    oracle_dispatch_recv_ranks(sh, 0, sh->N, counts, recv_off, recv_buf, recv_meta, expert_x,
                               expert_scale, expert_cnt, expert_off, expert_src, expert_rpos);
}

/* Stand-in for the grouped GEMM ([EFA] dispatch/combine overview: the grouped GEMM multiplies
 * tokens by expert weights between dispatch and combine).  Identity: y = the dispatched value
 * (bf16 as is; fp8 decoded and multiplied by its block scale, rounded once to bf16).  Tagged:
 * y = bf16(identity * (64 + e % 64) / 64), which makes every expert's output distinct. */
void oracle_expert(const oracle_shape* sh, int mode, const uint8_t* expert_x,
                   const float* expert_scale, const int32_t* expert_off, uint16_t* expert_y) {
    const int N = sh->N, H = sh->H, L = sh->E / sh->N;
    const int nsc = H / 128;
    for (int d = 0; d < N; ++d) {
        const int32_t* eoff = expert_off + (long)d * (L + 1);
        for (int j = 0; j < L; ++j) {
            int e = d * L + j;
            double tag = (mode == 1) ? (double)(64 + e % 64) / 64.0 : 1.0;
            for (long q = eoff[j]; q < eoff[j + 1]; ++q) {
                long row = rrow0(sh, d) + q;
                for (int h = 0; h < H; ++h) {
                    double v;
                    if (sh->fp8) {
                        v = oracle_e4m3_to_double(expert_x[row * H + h]) *
                            (double)expert_scale[row * nsc + h / 128];
                    } else {
                        uint16_t b;
                        memcpy(&b, expert_x + (row * H + h) * 2, 2);
                        v = oracle_bf16_to_double(b);
                    }
                    expert_y[row * H + h] = oracle_bf16_from_double(v * tag);
                }
            }
        }
    }
}

/* ---------------------------------------------------------------- combine */

/* [EFA] combine paragraphs: the routing metadata is already known from dispatch, so combine
 * shuffles the expert outputs, copies them back with one write per peer, and the receiver then
 * reads its receive buffer and accumulates the weighted average into the output tensor.
 * [PORT] Combine: senders copy unquantized 16-bit activations; the receiver computes the
 * weighted average of all expert contributions locally.
 * cs[d] is rank d's combine send buffer in its receive order; cr[s] is rank s's combine receive
 * buffer laid out like its dispatch send buffer. */
/* shuffle of ranks d in [r0, r1): expert-major row q goes back to receive position rpos[q] */
void oracle_combine_pack_ranks(const oracle_shape* sh, int r0, int r1, const uint16_t* expert_y,
                               const int32_t* expert_rpos, const int32_t* recv_off, uint16_t* cs_buf) {
    const int N = sh->N, H = sh->H;
    assert(0 <= r0 && r0 <= r1 && r1 <= N);
    for (int d = r0; d < r1; ++d) {
        long total = recv_off[(long)d * (N + 1) + N];
        for (long q = 0; q < total; ++q) {
            long r = expert_rpos[rrow0(sh, d) + q];
            memcpy(cs_buf + (rrow0(sh, d) + r) * H, expert_y + (rrow0(sh, d) + q) * H, 2L * H);
        }
    }
}

/* network back to ranks s in [r0, r1): segment (d -> s) lands where s's dispatch segment for d
 * sat */
void oracle_combine_net_ranks(const oracle_shape* sh, int r0, int r1, const int32_t* recv_off,
                              const int32_t* send_off, const uint16_t* cs_buf, uint16_t* cr_buf) {
    const int N = sh->N, H = sh->H;
    const long TR = (long)sh->T * sh->R;
    assert(0 <= r0 && r0 <= r1 && r1 <= N);
    for (int s = r0; s < r1; ++s) {
        const int32_t* soff = send_off + (long)s * (N + 1);
        for (int d = 0; d < N; ++d) {
            long n = soff[d + 1] - soff[d];
            long src = rrow0(sh, d) + recv_off[(long)d * (N + 1) + s];
            long dst = (long)s * TR + soff[d];
            memcpy(cr_buf + dst * H, cs_buf + src * H, 2L * n * H);
        }
    }
}

/* weighted sum over the token's R slots, for the tokens of ranks s in [r0, r1) */
void oracle_combine_sum_ranks(const oracle_shape* sh, int r0, int r1, int mode, const int32_t* send_pos,
                              const float* topk_w, const uint16_t* cr_buf, uint16_t* out) {
    const int N = sh->N, T = sh->T, H = sh->H, R = sh->R;
    const long TR = (long)T * R;
    assert(0 <= r0 && r0 <= r1 && r1 <= N);
    (void)N;
    for (int s = r0; s < r1; ++s) {
        for (int t = 0; t < ntok(sh, s); ++t) {
            const long base = (long)s * TR + (long)t * R;
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                float accf = 0.0f;
                for (int k = 0; k < R; ++k) {
                    long row = (long)s * TR + send_pos[base + k];
                    uint16_t yb = cr_buf[row * H + h];
                    double y = oracle_bf16_to_double(yb);
                    if (mode == 0) acc += (double)topk_w[base + k] * y;
                    else accf = fmaf(topk_w[base + k], (float)y, accf);
                }
                out[((long)s * T + t) * H + h] =
                    oracle_bf16_from_double(mode == 0 ? acc : (double)accf);
            }
        }
    }
}

void oracle_combine(const oracle_shape* sh, int mode, const uint16_t* expert_y,
                    const int32_t* expert_rpos, const int32_t* recv_off, const int32_t* send_off,
                    const int32_t* send_pos, const float* topk_w, uint16_t* cs_buf, uint16_t* cr_buf,
                    uint16_t* out) {
    oracle_combine_pack_ranks(sh, 0, sh->N, expert_y, expert_rpos, recv_off, cs_buf);
    oracle_combine_net_ranks(sh, 0, sh->N, recv_off, send_off, cs_buf, cr_buf);
    oracle_combine_sum_ranks(sh, 0, sh->N, mode, send_pos, topk_w, cr_buf, out);
}

/* Combine with the sum taken on the sending side ([EFA] results for the EP64 prefill latency
 * figure: another library sums a token's expert contributions on the expert side before sending,
 * which cuts the bytes moved at some cost in accuracy; the decode kernels of the page sum on the
 * receiving side only).  Rank d turns the rows it received for one token (s, t) -- consecutive in
 * its receive order, in slot order -- into one partial row
 *     p[d][s][t] = bf16( sum over those rows of w[s][t][k] * y ),
 * stored at the receive position of the token's first row (cs_buf) and sent back to the send
 * position of the token's first slot owned by d (cr_buf); the other rows are not sent.  Rank s
 * then adds the partials of each token in the order of their first slots:
 *     out[s][t] = bf16( sum over owners of p ).
 * The bf16 rounding of each partial is the transmitted precision (the accuracy cost).
 * mode 0: both sums in fp64, each rounded once to bf16.
 * mode 1: the partial as an fp32 fused-multiply-add chain in slot order, the final sum as fp32
 *         additions in first-slot order, each rounded once to bf16. */
void oracle_combine_acc(const oracle_shape* sh, int mode, const uint16_t* expert_y,
                        const int32_t* expert_src, const int32_t* expert_rpos,
                        const int32_t* recv_off, const int32_t* send_off, const int32_t* topk_idx,
                        const int32_t* send_pos, const float* topk_w, uint16_t* cs_buf,
                        uint16_t* cr_buf, uint16_t* out) {
    const int N = sh->N, T = sh->T, H = sh->H, R = sh->R, L = sh->E / sh->N;
    const long TR = (long)T * R;
    /* first[d][r]: receive row r of rank d is its token's first row there */
    char** first = calloc(N, sizeof(char*));
    assert(first);
    /* expert side */
    for (int d = 0; d < N; ++d) {
        const long total = recv_off[(long)d * (N + 1) + N];
        long* qof = malloc(sizeof(long) * (total > 0 ? total : 1));  /* receive row -> expert-major row */
        first[d] = calloc(total > 0 ? total : 1, 1);
        assert(qof && first[d]);
        for (long q = 0; q < total; ++q) qof[expert_rpos[rrow0(sh, d) + q]] = q;
        long r = 0;
        while (r < total) {
            const long tok = expert_src[rrow0(sh, d) + qof[r]] / R;  /* s * T + t */
            long c = 1;  /* the token's rows at rank d: r .. r + c - 1 */
            while (r + c < total && expert_src[rrow0(sh, d) + qof[r + c]] / R == tok) ++c;
            first[d][r] = 1;
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                float accf = 0.0f;
                for (long i = 0; i < c; ++i) {
                    const long q = qof[r + i];
                    const long si = expert_src[rrow0(sh, d) + q];  /* s * T * R + t * R + k */
                    const double y = oracle_bf16_to_double(expert_y[(rrow0(sh, d) + q) * H + h]);
                    if (mode == 0) acc += (double)topk_w[si] * y;
                    else accf = fmaf(topk_w[si], (float)y, accf);
                }
                cs_buf[(rrow0(sh, d) + r) * H + h] = oracle_bf16_from_double(mode == 0 ? acc : (double)accf);
            }
            r += c;
        }
        free(qof);
    }
    /* network back: the partial rows only; segment (d -> s) row i lands where s's dispatch
     * segment for d held row i, i.e. at the send position of the token's first slot owned by d */
    for (int s = 0; s < N; ++s) {
        const int32_t* soff = send_off + (long)s * (N + 1);
        for (int d = 0; d < N; ++d) {
            const long r0 = recv_off[(long)d * (N + 1) + s];
            for (long i = 0; i < soff[d + 1] - soff[d]; ++i) {
                if (!first[d][r0 + i]) continue;
                memcpy(cr_buf + ((long)s * TR + soff[d] + i) * H, cs_buf + (rrow0(sh, d) + r0 + i) * H,
                       2L * H);
            }
        }
    }
    for (int d = 0; d < N; ++d) free(first[d]);
    free(first);
    /* the source's sum over the token's owners, in the order of their first slots */
    for (int s = 0; s < N; ++s) {
        for (int t = 0; t < ntok(sh, s); ++t) {
            const long base = (long)s * TR + (long)t * R;
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                float accf = 0.0f;
                for (int k = 0; k < R; ++k) {
                    if (send_pos[base + k] < 0) continue;  /* dropped slot */
                    const int d = topk_idx[base + k] / L;
                    int is_first = 1;
                    for (int kk = 0; kk < k; ++kk)
                        if (send_pos[base + kk] >= 0 && topk_idx[base + kk] / L == d) is_first = 0;
                    if (!is_first) continue;
                    const double p = oracle_bf16_to_double(cr_buf[((long)s * TR + send_pos[base + k]) * H + h]);
                    if (mode == 0) acc += p;
                    else accf = accf + (float)p;
                }
                out[((long)s * T + t) * H + h] = oracle_bf16_from_double(mode == 0 ? acc : (double)accf);
            }
        }
    }
}

/* ---------------------------------------------------------------- prefill (replicated inputs) */

/* [QWEN] MoE dispatch-combine, Expert parallel: the prefill kernel's inputs are the same on every
 * rank, so each rank's dispatch only picks the tokens routed to its own experts and stages them
 * as grouped-GEMM inputs.  Rank d walks its local experts j in order and, for each, every
 * (token, slot) in order: the rows of one expert are contiguous, in (t, k) order. */
void oracle_prefill_dispatch(const oracle_shape* sh, const uint8_t* x, const float* x_scale,
                             const int32_t* topk_idx, int32_t* slot_pos, uint8_t* expert_x,
                             float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                             int32_t* expert_src) {
    const int N = sh->N, T = sh->T, H = sh->H, E = sh->E, R = sh->R;
    assert(N >= 1 && E % N == 0);
    const int L = E / N;
    const long xrow = sh->fp8 ? H : 2L * H;
    const int nsc = H / 128;
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < R; ++k) {
            const int e = topk_idx[(long)t * R + k];
            assert(e >= 0 && e < E);
            for (int kk = 0; kk < k; ++kk) assert(topk_idx[(long)t * R + kk] != e); /* distinct */
        }
    for (int d = 0; d < N; ++d) {
        int32_t* ecnt = expert_cnt + (long)d * L;
        int32_t* eoff = expert_off + (long)d * (L + 1);
        long q = 0;
        eoff[0] = 0;
        for (int j = 0; j < L; ++j) {
            const int e = d * L + j;
            for (int t = 0; t < T; ++t) {
                for (int k = 0; k < R; ++k) {
                    if (topk_idx[(long)t * R + k] != e) continue;
                    assert(q < sh->B);
                    const long row = (long)d * sh->B + q;
                    memcpy(expert_x + row * xrow, x + (long)t * xrow, xrow);
                    if (sh->fp8) memcpy(expert_scale + row * nsc, x_scale + (long)t * nsc, 4L * nsc);
                    expert_src[row] = t * R + k;
                    slot_pos[(long)t * R + k] = (int32_t)q;
                    q += 1;
                }
            }
            eoff[j + 1] = (int32_t)q;
            ecnt[j] = eoff[j + 1] - eoff[j];
        }
    }
}

/* [QWEN] MoE dispatch-combine, Expert parallel: the combine kernel first accumulates, locally,
 * the contributions of the tokens' slots routed to this rank's experts, then all-reduces across
 * the ranks.  Every rank writes a partial for every token (zero where it owns none of the
 * token's experts); the all-reduce sums them. */
void oracle_prefill_combine(const oracle_shape* sh, int mode, const uint16_t* expert_y,
                            const int32_t* slot_pos, const int32_t* topk_idx, const float* topk_w,
                            float* partial, uint16_t* out) {
    const int N = sh->N, T = sh->T, H = sh->H, R = sh->R;
    const int L = sh->E / N;
    for (int d = 0; d < N; ++d) {
        for (int t = 0; t < T; ++t) {
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                float accf = 0.0f;
                for (int k = 0; k < R; ++k) {
                    const long i = (long)t * R + k;
                    if (topk_idx[i] / L != d) continue;
                    const double y =
                        oracle_bf16_to_double(expert_y[((long)d * sh->B + slot_pos[i]) * H + h]);
                    if (mode == 0) acc += (double)topk_w[i] * y;
                    else accf = fmaf(topk_w[i], (float)y, accf);
                }
                partial[((long)d * T + t) * H + h] = mode == 0 ? (float)acc : accf;
            }
        }
    }
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            if (mode == 0) {
                double acc = 0.0;
                for (int k = 0; k < R; ++k) {
                    const long i = (long)t * R + k;
                    const int d = topk_idx[i] / L;
                    acc += (double)topk_w[i] *
                           oracle_bf16_to_double(expert_y[((long)d * sh->B + slot_pos[i]) * H + h]);
                }
                out[(long)t * H + h] = oracle_bf16_from_double(acc);
            } else {
                float s = 0.0f;
                for (int d = 0; d < N; ++d) s = s + partial[((long)d * T + t) * H + h];
                out[(long)t * H + h] = oracle_bf16_from_double((double)s);
            }
        }
    }
}
