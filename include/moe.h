/*
 * moe.h -- C ABI of libmoe: MoE expert-parallel token dispatch and combine on one MI355X.
 *
 * Pages cited by title:
 *   [EFA]  "Enabling trillion-parameter models on AWS EFA"
 *   [PORT] "Efficient and portable mixture-of-experts communication"
 *   [DSK]  "Lower latency and higher throughput with multi-node DeepSeek deployment"
 *   [QWEN] "Hosting Qwen on Blackwell"
 *
 * The problem ([EFA], send-buffer design paragraph): N ranks each dispatch T tokens of hidden
 * size H; every token goes to R of E experts; expert e lives on rank e / L, L = E / N.  Here all
 * N ranks live in one GPU's memory: every array below is rank-major ([N][...]) and a device copy
 * kernel stands in for the network between the send and receive halves.
 *
 * Conventions for every call:
 *  - Every pointer is a device pointer owned by the caller.  The library never allocates, frees
 *    or synchronises; each call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    legacy default stream) and returns.  Outputs are valid once the stream reaches that point.
 *  - Return value: MOE_OK, or a negative moe_status after host-side validation (nothing is
 *    enqueued then), or MOE_EHIP if a launch failed.  Launches are checked with hipGetLastError(),
 *    which also returns (and clears) an error an earlier HIP call on the same thread left unread;
 *    such an error is reported as MOE_EHIP by the next call.
 *  - Payload buffers (x, x_scale, send_buf, recv_buf, expert_x, expert_scale, expert_y,
 *    cs_buf, cr_buf, out) must be 16-byte aligned; metadata 8-byte; everything else 4-byte.
 *  - Index types are int32.  Rows are addressed as [rank][row] with the row strides given by
 *    moe_sizes().  Every buffer must be the full size moe_sizes() gives, also for a call on a
 *    rank range: the row-copy kernels may read the first row of their source buffer (for lanes
 *    that have no row to move) and never write outside the call's rows.
 *  - Device-detected errors (an expert id outside [0, E), or the same expert twice in one
 *    token's R slots) set *shape->status to MOE_EBADIDX if it is still 0 (sticky) and drop the
 *    offending slot: it is not counted, not sent, gets send_pos = -1 and adds nothing to the
 *    combine.  The caller reads the status word after its own synchronisation.
 *  - Calls are reentrant; the library keeps no state, except the static per-GPU histogram array
 *    of moe_dispatch_send_noalloc (calls of it that overlap in time on one GPU race on it).  Two
 *    calls that overlap in time must not share output buffers or a workspace.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 6

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad shape, null or misaligned pointer; (device status word) a
                               token count outside [0, T] */
    MOE_EUNSUPPORTED = -2,  /* valid but outside what these kernels implement */
    MOE_EHIP = -3,          /* a HIP launch failed */
    MOE_EBADIDX = -5,       /* (device status word) bad expert id in topk_idx */
    MOE_ENOSCRATCH = -6     /* moe_dispatch_send_noalloc: the call needs more than the library's
                               static scratch (MOE_STATIC_SCRATCH_BYTES) */
} moe_status;

/* Bytes of device scratch the library holds per GPU for moe_dispatch_send_noalloc. */
#define MOE_STATIC_SCRATCH_BYTES (4u << 20)

typedef enum {
    MOE_BF16 = 0,       /* dispatch payload: H bf16 values per row */
    MOE_FP8_E4M3 = 1,   /* OCP e4m3 codes, H per row, plus one fp32 scale per 128 of them */
    MOE_BF16_TO_FP8 = 2 /* tokens arrive as bf16 and moe_dispatch_send quantises them into the
                           e4m3 rows of MOE_FP8_E4M3 ([DSK] Implementation, Quantization: one
                           scale per 128-value vector found from its largest magnitude):
                           scale = amax / 448 (1.0 for an all-zero block), code = the e4m3 value
                           nearest to x / scale (fp32 division), ties to even, clamped to
                           +-448.  Everything after the send pack is the MOE_FP8_E4M3 path. */
} moe_dtype;

typedef enum {
    MOE_LAYOUT_DECODE = 0,  /* every rank dispatches its own T tokens (the send/network/receive path) */
    MOE_LAYOUT_PREFILL = 1  /* every rank holds the same T tokens ([QWEN] MoE dispatch-combine, Expert
                               parallel): moe_prefill_dispatch / moe_prefill_combine(_local) /
                               moe_prefill_allreduce; x, topk_idx, topk_w and out are [T][...] */
} moe_layout;

typedef struct {
    int32_t N;          /* ranks (expert-parallel size), 1..1024 */
    int32_t T;          /* tokens per rank (decode: each rank's own; prefill: the one set every
                           rank holds) */
    int32_t H;          /* hidden size; multiple of 8 (bf16) or 512 (fp8) */
    int32_t E;          /* experts, multiple of N, at most 1024 */
    int32_t R;          /* experts per token, 1..min(E, 64) */
    int32_t dtype;      /* moe_dtype of the dispatch payload; combine is always bf16 */
    int32_t rank_begin; /* the ranks whose work this call does: [rank_begin, rank_begin + rank_count); */
    int32_t rank_count; /*   0, 0 = all N.  A rank owns its tokens (route, dispatch send, weighted
                             sum), the pushes of its own rows to every peer (both network steps) and
                             its receive side (dispatch receive, combine shuffle, stand-in expert).
                             Running every rank's calls, each step for all ranks before the next,
                             gives exactly the all-ranks result.  Arrays stay full-size [N][...]. */
    int64_t capacity;   /* receive-side rows per rank; 0 = S*T*max(R, E/N), the [EFA] bound, with
                           S = N token sets (decode) or 1 (prefill).  Must be at least
                           S*T*min(R, E/N), the most any rank can receive. */
    int32_t* status;    /* device int32 sticky error word, or NULL */
    const int32_t* tokens; /* device int32[N], or NULL: rank s dispatches only its first
                              tokens[s] (0..T) tokens ([PORT] Portable kernels: T is the most any
                              rank may dispatch; [DSK] Cuda Graph: ranks run different batch sizes
                              without padding).  The others take no part: moe_route does not
                              write their rows, their slots get send_pos = -1 and are not counted
                              or sent, and moe_combine(_recv) does not write their output rows.
                              The counts stay on the device; a count outside [0, T] sets
                              MOE_EINVAL in the status word and counts as 0.  Decode layout
                              only (NULL for prefill). */
    int32_t layout;     /* moe_layout; the calls of the other layout return MOE_EINVAL */
} moe_shape;

/* Byte sizes of every buffer for a shape.  rows: capacity = B (receive-side rows per rank),
 * row_bytes = P (one dispatched row: the payload, then for fp8 its H/128 fp32 scales). */
typedef struct {
    int64_t capacity, row_bytes;
    int64_t logits, bias, topk_idx, topk_w;
    int64_t x, x_scale;
    int64_t counts, send_off, send_pos, send_buf, send_meta;
    int64_t recv_buf, recv_meta, recv_off;
    int64_t expert_x, expert_scale, expert_cnt, expert_off, expert_src, expert_rpos;
    int64_t expert_y, cs_buf, cr_buf, out;
    int64_t workspace;
    int64_t slot_pos, partial;  /* prefill only (0 for decode); decode-only buffers are 0 for prefill */
} moe_sizes_t;

/* Host only; no GPU needed.  Fills *out for a valid shape, else returns MOE_EINVAL or
 * MOE_EUNSUPPORTED. */
int moe_sizes(const moe_shape* shape, moe_sizes_t* out);

/* Router.  [DSK] Expert Parallelism and MoE Router: each token takes R experts from a sort of
 * the router scores that tracks indices, and the expert outputs are summed with weights;
 * [PORT] introduction: the weights come from the router's probability distribution.
 *   logits   f32[N*T][E]        router scores ([T][E] for MOE_LAYOUT_PREFILL: the replicated
 *                                tokens are routed once, whatever the rank range)
 *   bias     f32[E] or NULL     added to every token's scores before selection (one fp32 add)
 *   topk_idx i32[N*T][R] (out)  experts by descending (score + bias), ties to the lower id
 *   topk_w   f32[N*T][R] (out)  softmax over the R selected values, computed in fp64 and
 *                                rounded to fp32 */
int moe_route(const moe_shape* shape, const float* logits, const float* bias,
              int32_t* topk_idx, float* topk_w, void* stream);

/* Dispatch, send half.  [EFA] dispatch timing paragraph: count tokens per expert, take the
 * cumulative sum of the counts as offsets into a send buffer contiguous per destination rank,
 * pack the tokens; [PORT] Dispatch: activations, block scales and index travel together.
 *   x         bf16[N][T][H] (MOE_BF16, MOE_BF16_TO_FP8) or e4m3 u8[N][T][H]   tokens
 *   x_scale   f32[N][T][H/128] (MOE_FP8_E4M3), else NULL                     block scales
 *   topk_idx  i32[N][T*R]                          experts per (token, slot)
 *   counts    i32[N][E] (out)       counts[s][e] = slots of rank s that chose expert e
 *   send_off  i32[N][N+1] (out)     exclusive scan over destinations of rows s sends to d
 *   send_pos  i32[N][T*R] (out)     row of slot (t, k) in s's send buffer, -1 if dropped
 *   send_buf  u8[N][T*R][P] (out)   rows grouped by destination rank, (token, slot) order
 *                                    inside each group; row = payload bytes, then scales
 *   send_meta i32[N][T*R][2] (out)  per send row: {e*T*R + t*R + k, number of earlier slots of
 *                                    rank s that chose the same expert e}
 *   workspace device scratch of moe_sizes().workspace bytes (may be NULL if that is 0) */
int moe_dispatch_send(const moe_shape* shape, const void* x, const float* x_scale,
                      const int32_t* topk_idx, int32_t* counts, int32_t* send_off,
                      int32_t* send_pos, void* send_buf, int32_t* send_meta, void* workspace,
                      void* stream);

/* moe_dispatch_send for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): no workspace argument.  The
 * per-chunk histograms it needs when a rank's T*R slots span several chunks of 1024 (the workspace
 * of moe_dispatch_send) live in a static device array of MOE_STATIC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends; its address is looked up on the first call
 * on each device.  The call allocates and frees nothing.
 *   arguments, outputs and results as for moe_dispatch_send
 *   MOE_ENOSCRATCH  the call's histograms (rank_count * chunks * E int32) exceed the array
 * Every call on one GPU shares that array: calls that overlap in time on one GPU (two streams
 * without an ordering between them) race on it and give undefined results.  Each call writes every
 * histogram it reads before reading it, so the contents left by an earlier call do not matter. */
int moe_dispatch_send_noalloc(const moe_shape* shape, const void* x, const float* x_scale,
                              const int32_t* topk_idx, int32_t* counts, int32_t* send_off,
                              int32_t* send_pos, void* send_buf, int32_t* send_meta, void* stream);

/* The network stand-in.  [EFA] send-buffer paragraph: after the per-expert counts are
 * exchanged every rank knows where its writes go and where each source's tokens land, and the
 * bulk moves with one write per peer.
 *   send_off  i32[N][N+1]          from moe_dispatch_send (every source's: the exchanged table)
 *   send_buf, send_meta            from moe_dispatch_send
 *   recv_buf  u8[N][B][P] (out)    rank d receives segment (s -> d) at row recv_off[d][s]
 *   recv_meta i32[N][B][2] (out)   the rows' metadata, moved with them
 *   recv_off  i32[N][N+1] (out)    exclusive scan over sources of rows d receives; the total
 *                                   recv_off[d][N] <= N*T*min(R, E/N) <= B */
int moe_net_dispatch(const moe_shape* shape, const int32_t* send_off, const void* send_buf,
                     const int32_t* send_meta, void* recv_buf, int32_t* recv_meta,
                     int32_t* recv_off, void* stream);

/* Dispatch, receive half.  [PORT] Dispatch: the receiver copies tokens into contiguous buffers
 * that feed the grouped GEMM, tokens of one expert together, and keeps source rank, expert and
 * token index for combine; [DSK] Cuda Graph: tokens per expert stay on the device.
 *   counts, recv_off, recv_buf, recv_meta   from the calls above
 *   expert_x     bf16[N][B][H] or u8[N][B][H] (out)  rows in (local expert, source, token,
 *                                                     slot) order
 *   expert_scale f32[N][B][H/128] (out, fp8) or NULL
 *   expert_cnt   i32[N][L] (out)    rows per local expert
 *   expert_off   i32[N][L+1] (out)  exclusive scan of expert_cnt
 *   expert_src   i32[N][B] (out)    s*T*R + t*R + k of each expert-major row
 *   expert_rpos  i32[N][B] (out)    the row's index in recv_buf (its receive position) */
int moe_dispatch_recv(const moe_shape* shape, const int32_t* counts, const int32_t* recv_off,
                      const void* recv_buf, const int32_t* recv_meta, void* expert_x,
                      float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                      int32_t* expert_src, int32_t* expert_rpos, void* stream);

/* Combine.  [EFA] combine paragraphs: with the metadata known from dispatch, shuffle the expert
 * outputs, copy them back with one write per peer, and accumulate the weighted average from the
 * receive buffer into the output; [PORT] Combine: 16-bit activations, the weighted average is
 * computed by the receiver into an externally allocated tensor.
 *   expert_y   bf16[N][B][H]        expert outputs in expert-major order
 *   expert_rpos, recv_off           from dispatch (receive side)
 *   send_off, send_pos, topk_w      from dispatch (send side) and the router
 *   cs_buf     bf16[N][B][H] (out)  combine send buffer: cs[d][expert_rpos[q]] = y[d][q]
 *   cr_buf     bf16[N][T*R][H] (out) combine receive buffer, laid out like send_buf
 *   out        bf16[N][T][H] (out)  bf16(sum over k = 0..R-1 of w[t][k] * cr[send_pos[t][k]]),
 *                                    accumulated in fp32 with fused multiply-adds in slot order */
int moe_combine(const moe_shape* shape, const uint16_t* expert_y, const int32_t* expert_rpos,
                const int32_t* recv_off, const int32_t* send_off, const int32_t* send_pos,
                const float* topk_w, uint16_t* cs_buf, uint16_t* cr_buf, uint16_t* out,
                void* stream);  /* = moe_combine_send then moe_combine_recv.  All ranks only:
                                   rank_count must be 0 or N (MOE_EINVAL otherwise), since the
                                   weighted sum reads rows that every rank's send half writes. */

/* Combine, send half: the shuffle and the network back (the first two steps of moe_combine).
 * [PORT] Portable kernels: send halves only issue writes, so other work (the shared expert,
 * attention) can run while the transfer is in flight; [EFA] combine paragraphs.
 *   expert_y, expert_rpos, recv_off, send_off, cs_buf, cr_buf   as for moe_combine */
int moe_combine_send(const moe_shape* shape, const uint16_t* expert_y, const int32_t* expert_rpos,
                     const int32_t* recv_off, const int32_t* send_off, uint16_t* cs_buf,
                     uint16_t* cr_buf, void* stream);

/* Combine, receive half: the router-weighted sum from the combine receive buffer (the last step
 * of moe_combine).  [PORT] Combine: the receiver computes the weighted average of all expert
 * contributions into an externally allocated tensor.
 *   cr_buf, send_pos, topk_w, out   as for moe_combine */
int moe_combine_recv(const moe_shape* shape, const uint16_t* cr_buf, const int32_t* send_pos,
                     const float* topk_w, uint16_t* out, void* stream);

/* Combine with the sum taken on the sending side ([EFA] results under the EP64 prefill latency
 * figure: summing a token's expert contributions on the expert side before sending cuts the data
 * moved, at some cost in accuracy; moe_combine sums on the receiving side only).  Decode layout.
 * Rank d forms, for every token (s, t) it received rows for, one partial row
 *     p = bf16(sum over those rows, in slot order, of w[s][t][k] * y)   (fp32 fused multiply-adds)
 * and only the partials are sent back; rank s then sums the partials of each token:
 *     out[s][t] = bf16(sum over the token's owner ranks, in the order of their first slots, of p)
 * (fp32 additions).  Each partial is rounded to bf16 once more than in moe_combine: the results
 * differ from moe_combine by up to about one bf16 ulp per owner rank of a token.
 *   expert_y, recv_meta, counts, recv_off, expert_off   from dispatch and the grouped GEMM
 *   send_off, topk_w     from dispatch (send side) and the router (the weight of a received row is
 *                        read from its source's topk_w: in a deployment it travels with the row)
 *   topk_idx, send_pos   from the router and dispatch (send side)
 *   cs_buf  bf16[N][B][H] (out)   the partial of token (s, t) at the receive position of its first
 *                                  row at rank d; other rows not written
 *   cr_buf  bf16[N][T*R][H] (out) the partial from rank d at the send position of the token's
 *                                  first slot owned by d; other rows not written
 *   out     bf16[N][T][H] (out)
 * Errors: as moe_combine; rows whose metadata or tables are inconsistent set MOE_EINVAL in the
 * status word and are skipped. */
int moe_combine_acc(const moe_shape* shape, const uint16_t* expert_y, const int32_t* recv_meta,
                    const int32_t* counts, const int32_t* recv_off, const int32_t* expert_off,
                    const int32_t* send_off, const float* topk_w, const int32_t* topk_idx,
                    const int32_t* send_pos, uint16_t* cs_buf, uint16_t* cr_buf, uint16_t* out,
                    void* stream);  /* = moe_combine_acc_send then moe_combine_acc_recv.  All
                                       ranks only: rank_count must be 0 or N (MOE_EINVAL
                                       otherwise), as for moe_combine. */

/* Send half of moe_combine_acc: the partial rows and their network step back.
 *   arguments as for moe_combine_acc */
int moe_combine_acc_send(const moe_shape* shape, const uint16_t* expert_y, const int32_t* recv_meta,
                         const int32_t* counts, const int32_t* recv_off, const int32_t* expert_off,
                         const int32_t* send_off, const float* topk_w, uint16_t* cs_buf,
                         uint16_t* cr_buf, void* stream);

/* Receive half of moe_combine_acc: the source's sum of the partials.
 *   arguments as for moe_combine_acc */
int moe_combine_acc_recv(const moe_shape* shape, const uint16_t* cr_buf, const int32_t* topk_idx,
                         const int32_t* send_pos, uint16_t* out, void* stream);

/* Stand-in for the grouped GEMM between dispatch and combine (not part of dispatch/combine;
 * [EFA] overview: the grouped GEMM multiplies tokens by expert weights in between).
 *   mode 0 (identity): y = the dispatched value (bf16 as is; e4m3 decoded times its block
 *          scale, rounded once to bf16)
 *   mode 1 (tagged):   y = bf16(that value * (64 + e % 64) / 64) for the row's expert e
 *   expert_x, expert_scale, expert_off  from moe_dispatch_recv or moe_prefill_dispatch;
 *   expert_y bf16[N][B][H] (out).  Both layouts. */
int moe_expert_stub(const moe_shape* shape, int32_t mode, const void* expert_x,
                    const float* expert_scale, const int32_t* expert_off, uint16_t* expert_y,
                    void* stream);

/* Prefill dispatch (MOE_LAYOUT_PREFILL).  [QWEN] MoE dispatch-combine, Expert parallel: the
 * inputs are replicated on every rank, so each rank's dispatch only selects the tokens routed to
 * its own experts and stages them for the grouped GEMM.  No network step: nothing moves between
 * ranks until the combine's all-reduce.
 *   x            bf16[T][H] or e4m3 u8[T][H]       the replicated tokens
 *   x_scale      f32[T][H/128] (e4m3) or NULL
 *   topk_idx     i32[T][R]                          from moe_route on the same shape (routes T tokens)
 *   slot_pos     i32[T][R] (out)    row of slot (t, k) in its owner rank's expert-major arrays; -1
 *                                    for a dropped slot (bad id, flagged as MOE_EBADIDX)
 *   expert_x     [N][B][H] (out), expert_scale f32[N][B][H/128] (out, e4m3), expert_cnt i32[N][L]
 *   (out), expert_off i32[N][L+1] (out), expert_src i32[N][B] (out) = t*R + k: rank d's rows in
 *   (local expert, token, slot) order, as moe_dispatch_recv lays them out for one source
 *   workspace    device scratch of moe_sizes().workspace bytes (NULL if 0)
 * With a rank range, only the range's rows and tables are written; slot_pos covers every slot. */
int moe_prefill_dispatch(const moe_shape* shape, const void* x, const float* x_scale,
                         const int32_t* topk_idx, int32_t* slot_pos, void* expert_x,
                         float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                         int32_t* expert_src, void* workspace, void* stream);

/* Prefill combine, local step: [QWEN] MoE dispatch-combine, Expert parallel: each rank first
 * accumulates the contributions of its own experts.
 *   expert_y   bf16[N][B][H]       expert outputs in the dispatch's expert-major order
 *   topk_idx, slot_pos, topk_w    [T][R] from moe_route and moe_prefill_dispatch
 *   partial    f32[N][T][H] (out)  for each of the call's ranks d and every token t: the fp32
 *                                   fused-multiply-add chain over t's slots owned by d in slot
 *                                   order 0..R-1 (0 where d owns none) */
int moe_prefill_combine_local(const moe_shape* shape, const uint16_t* expert_y,
                              const int32_t* topk_idx, const int32_t* slot_pos, const float* topk_w,
                              float* partial, void* stream);

/* Prefill combine, all-reduce (the collective's stand-in): out[t] = bf16 of the fp32 sum of
 * partial[0][t] .. partial[N-1][t] in rank order, rounded once (nearest even).  Reads every
 * rank's partial whatever the rank range (each must have been written); out is bf16[T][H]. */
int moe_prefill_allreduce(const moe_shape* shape, const float* partial, uint16_t* out, void* stream);

/* = moe_prefill_combine_local then moe_prefill_allreduce (all arguments validated first).  All
 * ranks only: rank_count must be 0 or N (MOE_EINVAL otherwise), since the all-reduce reads every
 * rank's partial. */
int moe_prefill_combine(const moe_shape* shape, const uint16_t* expert_y, const int32_t* topk_idx,
                        const int32_t* slot_pos, const float* topk_w, float* partial, uint16_t* out,
                        void* stream);

/* Static string for a status code. */
const char* moe_strerror(int status);

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* A measurement aid, not a step of the path: copies `bytes` (a multiple of 16) from src to dst
 * (device pointers, 16-byte aligned, not overlapping) with the row-streaming engine the copy
 * kernels use, on the simplest row map (contiguous rows of 256 threads' chunks, one per block,
 * nontemporal), so its rate is the practical copy ceiling the row-copy kernels are measured
 * against.  Returns MOE_EINVAL for a bad size, alignment or overlap. */
int moe_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif
