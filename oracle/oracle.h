/*
 * oracle.h -- plain, slow CPU oracle for MoE expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product (the HIP library and its Python binding)
 * never calls it and shares no code, header or constant with it.
 *
 * Pages cited (by title; sections named in each function's comment):
 *   [EFA]  "Enabling trillion-parameter models on AWS EFA"
 *   [PORT] "Efficient and portable mixture-of-experts communication"
 *   [DSK]  "Lower latency and higher throughput with multi-node DeepSeek deployment"
 *   [QWEN] "Hosting Qwen on Blackwell"
 *
 * Problem statement ([EFA], send-buffer design paragraph): N ranks, each dispatching T tokens,
 * every token routed to R of E experts; expert e lives on rank e / L with L = E / N.
 *
 * All arrays are dense, row-major and rank-major ([N][...]).  Every function asserts its
 * contract (valid indices, capacity) and aborts on violation: the oracle defines results
 * for valid inputs only.
 *
 * Parity pins: every function here is pinned by CPU tests against brute force, closed forms
 * and invariants (tests/test_oracle_pins.py).  Nothing here is "parity unpinned".
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

typedef struct {
    int N, T, H, E, R;
    int fp8;   /* 0: bf16 payload (2H bytes per row); 1: e4m3 payload + fp32 scale per 128 */
    long B;    /* receive-side rows per rank (row stride of every [N][B][...] array) */
    const long* rbase; /* optional: rank d's receive-side rows start at row rbase[d] and it has
                          rbase[d+1] - rbase[d] of them (N+1 entries); NULL means d * B and B */
    const int32_t* tokens; /* optional: rank s dispatches only its first tokens[s] <= T tokens
                              (N entries); NULL means T for every rank */
} oracle_shape;

/* Bytes of one dispatched row: the payload, then (fp8 only) its block scales. */
long oracle_row_bytes(const oracle_shape* sh);

/* Scalar conversions, written from the IEEE-754 binary16-brain-float and OCP E4M3 definitions. */
uint16_t oracle_bf16_from_double(double x);  /* round to nearest, ties to even */
double oracle_bf16_to_double(uint16_t b);
double oracle_e4m3_to_double(uint8_t b);
uint8_t oracle_e4m3_from_float_sat(float v); /* nearest, ties to even, clamped to +-448 */

/* Block quantisation of bf16 activations to e4m3 with one fp32 scale per 128 values:
 * scale = amax / 448 (1 when amax = 0), code = e4m3(x / scale).  x: bf16 bits [n_rows][H];
 * q: [n_rows][H]; scale: [n_rows][H / 128]. */
void oracle_quantize_e4m3(long n_rows, int H, const uint16_t* x, uint8_t* q, float* scale);

/* Router: top-R experts of fp32 (logits + bias) and softmax weights over the selected R. */
void oracle_route(int n_tokens, int E, int R, const float* logits, const float* bias,
                  int32_t* topk_idx, float* topk_w);

/* Dispatch send: counts, exclusive-scan offsets, positions, packed send rows and metadata.
 * Slots of tokens t >= tokens[s] take no part: their send_pos is -1. */
void oracle_dispatch_send(const oracle_shape* sh, const uint8_t* x, const float* x_scale,
                          const int32_t* topk_idx, int32_t* counts, int32_t* send_off,
                          int32_t* send_pos, uint8_t* send_buf, int32_t* send_meta);

/* The network: one contiguous copy per (source, destination) segment. */
void oracle_net_dispatch(const oracle_shape* sh, const int32_t* send_off, const uint8_t* send_buf,
                         const int32_t* send_meta, uint8_t* recv_buf, int32_t* recv_meta,
                         int32_t* recv_off);

/* Dispatch receive: shuffle received rows into expert-major order for the grouped GEMM. */
void oracle_dispatch_recv(const oracle_shape* sh, const int32_t* counts, const int32_t* recv_off,
                          const uint8_t* recv_buf, const int32_t* recv_meta, uint8_t* expert_x,
                          float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                          int32_t* expert_src, int32_t* expert_rpos);

/* Stand-in expert (not part of the method): mode 0 identity, mode 1 tagged (y * (64 + e%64)/64). */
void oracle_expert(const oracle_shape* sh, int mode, const uint8_t* expert_x,
                   const float* expert_scale, const int32_t* expert_off, uint16_t* expert_y);

/* Combine: rows back to their source slots, then the router-weighted sum.
 * mode 0: the sum in fp64, rounded once to bf16.
 * mode 1: an fp32 fused-multiply-add chain in slot order 0..R-1, then rounded to bf16.
 * Output rows of tokens t >= tokens[s] are not written. */
void oracle_combine(const oracle_shape* sh, int mode, const uint16_t* expert_y,
                    const int32_t* expert_rpos, const int32_t* recv_off, const int32_t* send_off,
                    const int32_t* send_pos, const float* topk_w, uint16_t* cs_buf, uint16_t* cr_buf,
                    uint16_t* out);

/* Combine with the sum taken on the sending side: rank d sends one bf16 partial row per token
 * it holds rows for (the weighted sum of those rows), and the source adds the partials.
 * expert_src/expert_rpos as dispatch receive wrote them; topk_idx [N][T][R] (the owner of each
 * slot).  cs_buf holds a partial at the receive position of each token's first row at rank d,
 * cr_buf at the send position of each token's first slot per owner rank; no other rows are
 * written.
 * mode 0: partial and final sums in fp64, each rounded once to bf16.
 * mode 1: the partial as an fp32 fused-multiply-add chain in slot order, the final sum as fp32
 *         additions in first-slot order, each rounded once to bf16. */
void oracle_combine_acc(const oracle_shape* sh, int mode, const uint16_t* expert_y,
                        const int32_t* expert_src, const int32_t* expert_rpos,
                        const int32_t* recv_off, const int32_t* send_off, const int32_t* topk_idx,
                        const int32_t* send_pos, const float* topk_w, uint16_t* cs_buf,
                        uint16_t* cr_buf, uint16_t* out);

/* Prefill expert parallelism with replicated inputs ([QWEN] "Hosting Qwen on Blackwell", MoE
 * dispatch-combine, Expert parallel): every rank holds the same T tokens (sh->T), so dispatch
 * only selects, on each rank, the slots routed to its own experts, and combine accumulates each
 * rank's contributions locally and then all-reduces over the ranks.  sh->B is the per-rank row
 * stride of the receive-side arrays; rank d has expert_off[d][L] rows.
 *   x [T][H] (bf16 bits or e4m3 codes), x_scale [T][H/128] (fp8), topk_idx [T][R]
 *   slot_pos [T][R] (out): row of slot (t, k) in its owner rank's expert-major arrays
 *   expert_x [N][B][H], expert_scale [N][B][H/128], expert_cnt [N][L], expert_off [N][L+1],
 *   expert_src [N][B] = t*R + k.  Rows are in (local expert, token, slot) order. */
void oracle_prefill_dispatch(const oracle_shape* sh, const uint8_t* x, const float* x_scale,
                             const int32_t* topk_idx, int32_t* slot_pos, uint8_t* expert_x,
                             float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                             int32_t* expert_src);

/* Prefill combine.  partial [N][T][H] fp32 (out), out [T][H] bf16 (out).
 * mode 0: partial[d][t] = sum over d's slots of w * y in fp64 (stored rounded to fp32);
 *         out = bf16 of the fp64 sum over every slot (the definition).
 * mode 1: partial[d][t] = fp32 fused-multiply-add chain over d's slots in slot order;
 *         out = bf16 of the fp32 sum of the partials in rank order 0..N-1. */
void oracle_prefill_combine(const oracle_shape* sh, int mode, const uint16_t* expert_y,
                            const int32_t* slot_pos, const int32_t* topk_idx, const float* topk_w,
                            float* partial, uint16_t* out);


/* Rank-range (token-range) forms of the steps above: the same loops restricted to the ranks
 * [r0, r1) (route: tokens [t0, t1)); arrays stay full-size and global-indexed.  Ranges of one step
 * touch disjoint outputs, so several may run at once on different threads; a step may start only
 * once every range of the step before it has finished.  The network step handles destinations
 * (each computes its receive offsets and copies its N incoming segments); the combine splits into
 * the shuffle (by destination), the network back (by source) and the weighted sum (by source).
 * The single calls above are these over the full range. */
void oracle_route_tokens(int t0, int t1, int E, int R, const float* logits, const float* bias,
                         int32_t* topk_idx, float* topk_w);
void oracle_dispatch_send_ranks(const oracle_shape* sh, int r0, int r1, const uint8_t* x,
                                const float* x_scale, const int32_t* topk_idx, int32_t* counts,
                                int32_t* send_off, int32_t* send_pos, uint8_t* send_buf,
                                int32_t* send_meta);
void oracle_net_dispatch_ranks(const oracle_shape* sh, int r0, int r1, const int32_t* send_off,
                               const uint8_t* send_buf, const int32_t* send_meta, uint8_t* recv_buf,
                               int32_t* recv_meta, int32_t* recv_off);
void oracle_dispatch_recv_ranks(const oracle_shape* sh, int r0, int r1, const int32_t* counts,
                                const int32_t* recv_off, const uint8_t* recv_buf,
                                const int32_t* recv_meta, uint8_t* expert_x, float* expert_scale,
                                int32_t* expert_cnt, int32_t* expert_off, int32_t* expert_src,
                                int32_t* expert_rpos);
void oracle_combine_pack_ranks(const oracle_shape* sh, int r0, int r1, const uint16_t* expert_y,
                               const int32_t* expert_rpos, const int32_t* recv_off, uint16_t* cs_buf);
void oracle_combine_net_ranks(const oracle_shape* sh, int r0, int r1, const int32_t* recv_off,
                              const int32_t* send_off, const uint16_t* cs_buf, uint16_t* cr_buf);
void oracle_combine_sum_ranks(const oracle_shape* sh, int r0, int r1, int mode, const int32_t* send_pos,
                              const float* topk_w, const uint16_t* cr_buf, uint16_t* out);

#endif
