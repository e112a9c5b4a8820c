// api.hip -- the extern "C" entry points of libmoe (declared in include/moe.h): host-side
// validation, buffer sizes, and the kernel launches of each step.  No allocation, no
// synchronisation: every call enqueues on the caller's stream and returns.
#include <limits.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {
hipError_t launch_route(const Dims&, const float*, const float*, int32_t*, float*, hipStream_t);
size_t send_workspace_bytes(const Dims&);
size_t send_workspace_bytes_used(const Dims&);
hipError_t scratch_address(void**);
hipError_t launch_dispatch_send(const Dims&, const void*, const float*, const int32_t*, int32_t*,
                                int32_t*, int32_t*, void*, int32_t*, void*, hipStream_t);
hipError_t launch_net_dispatch(const Dims&, const int32_t*, const void*, const int32_t*, void*,
                               int32_t*, int32_t*, hipStream_t);
hipError_t launch_dispatch_recv(const Dims&, const int32_t*, const int32_t*, const void*,
                                const int32_t*, void*, float*, int32_t*, int32_t*, int32_t*,
                                int32_t*, hipStream_t);
hipError_t launch_expert_stub(const Dims&, int, const void*, const float*, const int32_t*,
                              uint16_t*, hipStream_t);
hipError_t launch_combine_send(const Dims&, const uint16_t*, const int32_t*, const int32_t*,
                               const int32_t*, uint16_t*, uint16_t*, hipStream_t);
hipError_t launch_combine_recv(const Dims&, const uint16_t*, const int32_t*, const float*, uint16_t*,
                               hipStream_t);
hipError_t launch_combine_acc_send(const Dims&, const uint16_t*, const int32_t*, const int32_t*, const int32_t*,
                                   const int32_t*, const int32_t*, const float*, uint16_t*, uint16_t*,
                                   hipStream_t);
hipError_t launch_combine_acc_recv(const Dims&, const uint16_t*, const int32_t*, const int32_t*, uint16_t*,
                                   hipStream_t);
size_t prefill_workspace_bytes(const Dims&);
hipError_t launch_prefill_dispatch(const Dims&, const void*, const float*, const int32_t*, int32_t*, void*,
                                   float*, int32_t*, int32_t*, int32_t*, void*, hipStream_t);
hipError_t launch_prefill_local(const Dims&, const uint16_t*, const int32_t*, const int32_t*, const float*,
                                float*, hipStream_t);
hipError_t launch_prefill_allreduce(const Dims&, const float*, uint16_t*, hipStream_t);
hipError_t launch_stream_copy(const void*, void*, long, hipStream_t);
}  // namespace moe

using moe::Dims;

namespace {

constexpr int kMaxN = 1024;
constexpr int kMaxE = 1024;
constexpr int kMaxR = 64;

// Validate a shape and derive the kernels' view of it.  Returns MOE_OK or an error code.
int make_dims(const moe_shape* sh, Dims* D) {
    if (!sh) return MOE_EINVAL;
    const long long N = sh->N, T = sh->T, H = sh->H, E = sh->E, R = sh->R;
    if (N < 1 || T < 1 || H < 1 || E < 1 || R < 1) return MOE_EINVAL;
    if (E % N != 0 || R > E) return MOE_EINVAL;
    if (sh->dtype != MOE_BF16 && sh->dtype != MOE_FP8_E4M3 && sh->dtype != MOE_BF16_TO_FP8)
        return MOE_EINVAL;
    if (sh->layout != MOE_LAYOUT_DECODE && sh->layout != MOE_LAYOUT_PREFILL) return MOE_EINVAL;
    const bool prefill = sh->layout == MOE_LAYOUT_PREFILL;
    if (prefill && sh->tokens) return MOE_EINVAL;                        // one replicated token set
    if (prefill && sh->dtype == MOE_BF16_TO_FP8) return MOE_EUNSUPPORTED;
    if (N > kMaxN || E > kMaxE || R > kMaxR) return MOE_EUNSUPPORTED;
    const bool fp8 = sh->dtype != MOE_BF16;  // e4m3 rows, given or made by the send pack
    if (!fp8 && H % 8 != 0) return MOE_EUNSUPPORTED;   // 16-byte rows
    if (fp8 && H % 512 != 0) return MOE_EUNSUPPORTED;  // 16-byte rows of codes and of scales
    const long long L = E / N;
    const long long TR = T * R;
    if (N * TR > INT_MAX || E * TR > INT_MAX) return MOE_EUNSUPPORTED;  // int32 indices, meta
    const long long S = prefill ? 1 : N;  // token sets: one per rank, or one replicated set
    const long long tight = S * T * (R < L ? R : L);
    const long long bound = S * T * (R > L ? R : L);
    const long long B = sh->capacity == 0 ? bound : sh->capacity;
    if (B < tight) return MOE_EINVAL;
    if (B > INT_MAX) return MOE_EUNSUPPORTED;
    if (H > (1 << 20)) return MOE_EUNSUPPORTED;
    D->N = (int)N;
    D->T = (int)T;
    D->H = (int)H;
    D->E = (int)E;
    D->R = (int)R;
    D->L = (int)L;
    D->fp8 = fp8;
    D->quant = sh->dtype == MOE_BF16_TO_FP8;
    D->prefill = prefill;
    if (sh->tokens && reinterpret_cast<uintptr_t>(sh->tokens) % 4 != 0) return MOE_EINVAL;
    D->tok = sh->tokens;
    D->TR = (int)TR;
    D->B = B;
    D->P = fp8 ? (int)(H + H / 32) : (int)(2 * H);
    D->P16 = D->P / 16;
    D->X16 = fp8 ? (int)(H / 16) : (int)(2 * H / 16);
    D->nsc = (int)(H / 128);
    D->Y16 = (int)(2 * H / 16);
    if (sh->rank_begin < 0 || sh->rank_count < 0) return MOE_EINVAL;
    if (sh->rank_count == 0 && sh->rank_begin != 0) return MOE_EINVAL;
    if ((long long)sh->rank_begin + sh->rank_count > N) return MOE_EINVAL;
    D->rb = sh->rank_begin;
    D->rc = sh->rank_count == 0 ? (int)N : sh->rank_count;
    D->status = sh->status;
    return MOE_OK;
}

bool aligned(const void* p, uintptr_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0 || bytes / 16 > (int64_t)1 << 40) return MOE_EINVAL;
    if (bytes == 0) return MOE_OK;
    if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_EINVAL;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + (uintptr_t)bytes && d < s + (uintptr_t)bytes) return MOE_EINVAL;  // overlapping
    return hip_status(moe::launch_stream_copy(src, dst, (long)bytes, (hipStream_t)stream));
}

const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument (shape, null or misaligned pointer, inconsistent tables)";
        case MOE_EUNSUPPORTED: return "unsupported shape for these kernels";
        case MOE_EHIP: return "HIP launch error";
        case MOE_EBADIDX: return "expert id out of range or repeated within a token";
        case MOE_ENOSCRATCH: return "the call needs more scratch than the library's static array holds";
        default: return "unknown status";
    }
}

int moe_sizes(const moe_shape* shape, moe_sizes_t* out) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (!out) return MOE_EINVAL;
    const int64_t N = D.N, T = D.T, H = D.H, E = D.E, R = D.R, L = D.L, B = D.B, P = D.P;
    const int64_t S = D.prefill ? 1 : N;  // token sets
    const int64_t NT = S * T, M = S * T * R;
    const int64_t xb = D.fp8 ? 1 : 2;  // bytes per value of expert_x
    out->capacity = B;
    out->row_bytes = P;
    out->logits = NT * E * 4;
    out->bias = E * 4;
    out->topk_idx = M * 4;
    out->topk_w = M * 4;
    out->x = NT * H * (D.quant ? 2 : xb);
    out->x_scale = D.fp8 && !D.quant ? NT * (H / 128) * 4 : 0;
    const bool dec = !D.prefill;  // the decode path's send/receive staging
    out->counts = dec ? N * E * 4 : 0;
    out->send_off = dec ? N * (N + 1) * 4 : 0;
    out->send_pos = dec ? M * 4 : 0;
    out->send_buf = dec ? M * P : 0;
    out->send_meta = dec ? M * 8 : 0;
    out->recv_buf = dec ? N * B * P : 0;
    out->recv_meta = dec ? N * B * 8 : 0;
    out->recv_off = dec ? N * (N + 1) * 4 : 0;
    out->expert_x = N * B * H * xb;
    out->expert_scale = D.fp8 ? N * B * (H / 128) * 4 : 0;
    out->expert_cnt = N * L * 4;
    out->expert_off = N * (L + 1) * 4;
    out->expert_src = N * B * 4;
    out->expert_rpos = dec ? N * B * 4 : 0;
    out->expert_y = N * B * H * 2;
    out->cs_buf = dec ? N * B * H * 2 : 0;
    out->cr_buf = dec ? M * H * 2 : 0;
    out->out = NT * H * 2;
    out->slot_pos = D.prefill ? M * 4 : 0;
    out->partial = D.prefill ? N * T * H * 4 : 0;
    if (D.prefill) {
        out->workspace = (int64_t)moe::prefill_workspace_bytes(D);
    } else {
        out->workspace = (int64_t)moe::send_workspace_bytes(D);
    }
    return MOE_OK;
}

int moe_route(const moe_shape* shape, const float* logits, const float* bias, int32_t* topk_idx,
              float* topk_w, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_EINVAL;
    if (bias && !aligned(bias, 4)) return MOE_EINVAL;
    return hip_status(moe::launch_route(D, logits, bias, topk_idx, topk_w, (hipStream_t)stream));
}

int moe_dispatch_send(const moe_shape* shape, const void* x, const float* x_scale,
                      const int32_t* topk_idx, int32_t* counts, int32_t* send_off, int32_t* send_pos,
                      void* send_buf, int32_t* send_meta, void* workspace, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!aligned(x, 16) || !aligned(send_buf, 16) || !aligned(send_meta, 8)) return MOE_EINVAL;
    if (D.fp8 && !D.quant && !aligned(x_scale, 16)) return MOE_EINVAL;
    if (D.quant && x_scale) return MOE_EINVAL;  // the scales are made here
    if (!aligned(topk_idx, 4) || !aligned(counts, 4) || !aligned(send_off, 4) || !aligned(send_pos, 4))
        return MOE_EINVAL;
    if (moe::send_workspace_bytes(D) > 0 && !aligned(workspace, 4)) return MOE_EINVAL;
    return hip_status(moe::launch_dispatch_send(D, x, x_scale, topk_idx, counts, send_off, send_pos,
                                                send_buf, send_meta, workspace, (hipStream_t)stream));
}

int moe_dispatch_send_noalloc(const moe_shape* shape, const void* x, const float* x_scale,
                              const int32_t* topk_idx, int32_t* counts, int32_t* send_off,
                              int32_t* send_pos, void* send_buf, int32_t* send_meta, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!aligned(x, 16) || !aligned(send_buf, 16) || !aligned(send_meta, 8)) return MOE_EINVAL;
    if (D.fp8 && !D.quant && !aligned(x_scale, 16)) return MOE_EINVAL;
    if (D.quant && x_scale) return MOE_EINVAL;  // the scales are made here
    if (!aligned(topk_idx, 4) || !aligned(counts, 4) || !aligned(send_off, 4) || !aligned(send_pos, 4))
        return MOE_EINVAL;
    if (moe::send_workspace_bytes_used(D) > MOE_STATIC_SCRATCH_BYTES) return MOE_ENOSCRATCH;
    // every histogram the kernels read is written earlier in the same call: nothing to clear
    void* ws = nullptr;
    if (moe::scratch_address(&ws) != hipSuccess) return MOE_EHIP;
    return hip_status(moe::launch_dispatch_send(D, x, x_scale, topk_idx, counts, send_off, send_pos,
                                                send_buf, send_meta, ws, (hipStream_t)stream));
}

int moe_net_dispatch(const moe_shape* shape, const int32_t* send_off, const void* send_buf,
                     const int32_t* send_meta, void* recv_buf, int32_t* recv_meta, int32_t* recv_off,
                     void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!aligned(send_off, 4) || !aligned(send_buf, 16) || !aligned(send_meta, 8) ||
        !aligned(recv_buf, 16) || !aligned(recv_meta, 8) || !aligned(recv_off, 4))
        return MOE_EINVAL;
    return hip_status(moe::launch_net_dispatch(D, send_off, send_buf, send_meta, recv_buf, recv_meta,
                                               recv_off, (hipStream_t)stream));
}

int moe_dispatch_recv(const moe_shape* shape, const int32_t* counts, const int32_t* recv_off,
                      const void* recv_buf, const int32_t* recv_meta, void* expert_x,
                      float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                      int32_t* expert_src, int32_t* expert_rpos, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!aligned(counts, 4) || !aligned(recv_off, 4) || !aligned(recv_buf, 16) ||
        !aligned(recv_meta, 8) || !aligned(expert_x, 16) || !aligned(expert_cnt, 4) ||
        !aligned(expert_off, 4) || !aligned(expert_src, 4) || !aligned(expert_rpos, 4))
        return MOE_EINVAL;
    if (D.fp8 && !aligned(expert_scale, 16)) return MOE_EINVAL;
    return hip_status(moe::launch_dispatch_recv(D, counts, recv_off, recv_buf, recv_meta, expert_x,
                                                expert_scale, expert_cnt, expert_off, expert_src,
                                                expert_rpos, (hipStream_t)stream));
}

int moe_combine_send(const moe_shape* shape, const uint16_t* expert_y, const int32_t* expert_rpos,
                     const int32_t* recv_off, const int32_t* send_off, uint16_t* cs_buf,
                     uint16_t* cr_buf, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!aligned(expert_y, 16) || !aligned(expert_rpos, 4) || !aligned(recv_off, 4) ||
        !aligned(send_off, 4) || !aligned(cs_buf, 16) || !aligned(cr_buf, 16))
        return MOE_EINVAL;
    return hip_status(moe::launch_combine_send(D, expert_y, expert_rpos, recv_off, send_off, cs_buf,
                                               cr_buf, (hipStream_t)stream));
}

int moe_combine_recv(const moe_shape* shape, const uint16_t* cr_buf, const int32_t* send_pos,
                     const float* topk_w, uint16_t* out, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!aligned(cr_buf, 16) || !aligned(send_pos, 4) || !aligned(topk_w, 4) || !aligned(out, 16))
        return MOE_EINVAL;
    return hip_status(moe::launch_combine_recv(D, cr_buf, send_pos, topk_w, out, (hipStream_t)stream));
}

int moe_combine(const moe_shape* shape, const uint16_t* expert_y, const int32_t* expert_rpos,
                const int32_t* recv_off, const int32_t* send_off, const int32_t* send_pos,
                const float* topk_w, uint16_t* cs_buf, uint16_t* cr_buf, uint16_t* out, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (D.rc != D.N) return MOE_EINVAL;  // its second half reads what every rank's first half wrote
    // validate both halves before launching either
    if (!aligned(expert_y, 16) || !aligned(expert_rpos, 4) || !aligned(recv_off, 4) ||
        !aligned(send_off, 4) || !aligned(send_pos, 4) || !aligned(topk_w, 4) ||
        !aligned(cs_buf, 16) || !aligned(cr_buf, 16) || !aligned(out, 16))
        return MOE_EINVAL;
    rc = hip_status(moe::launch_combine_send(D, expert_y, expert_rpos, recv_off, send_off, cs_buf,
                                             cr_buf, (hipStream_t)stream));
    if (rc) return rc;
    return hip_status(moe::launch_combine_recv(D, cr_buf, send_pos, topk_w, out, (hipStream_t)stream));
}

static bool acc_send_aligned(const uint16_t* expert_y, const int32_t* recv_meta, const int32_t* counts,
                             const int32_t* recv_off, const int32_t* expert_off, const int32_t* send_off,
                             const float* topk_w, const uint16_t* cs_buf, const uint16_t* cr_buf) {
    return aligned(expert_y, 16) && aligned(recv_meta, 8) && aligned(counts, 4) && aligned(recv_off, 4) &&
           aligned(expert_off, 4) && aligned(send_off, 4) && aligned(topk_w, 4) && aligned(cs_buf, 16) &&
           aligned(cr_buf, 16);
}

int moe_combine_acc_send(const moe_shape* shape, const uint16_t* expert_y, const int32_t* recv_meta,
                         const int32_t* counts, const int32_t* recv_off, const int32_t* expert_off,
                         const int32_t* send_off, const float* topk_w, uint16_t* cs_buf,
                         uint16_t* cr_buf, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!acc_send_aligned(expert_y, recv_meta, counts, recv_off, expert_off, send_off, topk_w, cs_buf, cr_buf))
        return MOE_EINVAL;
    return hip_status(moe::launch_combine_acc_send(D, expert_y, recv_meta, counts, recv_off, expert_off,
                                                   send_off, topk_w, cs_buf, cr_buf, (hipStream_t)stream));
}

int moe_combine_acc_recv(const moe_shape* shape, const uint16_t* cr_buf, const int32_t* topk_idx,
                         const int32_t* send_pos, uint16_t* out, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (!aligned(cr_buf, 16) || !aligned(topk_idx, 4) || !aligned(send_pos, 4) || !aligned(out, 16))
        return MOE_EINVAL;
    return hip_status(moe::launch_combine_acc_recv(D, cr_buf, send_pos, topk_idx, out, (hipStream_t)stream));
}

int moe_combine_acc(const moe_shape* shape, const uint16_t* expert_y, const int32_t* recv_meta,
                    const int32_t* counts, const int32_t* recv_off, const int32_t* expert_off,
                    const int32_t* send_off, const float* topk_w, const int32_t* topk_idx,
                    const int32_t* send_pos, uint16_t* cs_buf, uint16_t* cr_buf, uint16_t* out,
                    void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (D.prefill) return MOE_EINVAL;  // the decode layout only
    if (D.rc != D.N) return MOE_EINVAL;  // its second half reads what every rank's first half wrote
    // validate both halves before launching either
    if (!acc_send_aligned(expert_y, recv_meta, counts, recv_off, expert_off, send_off, topk_w, cs_buf, cr_buf) ||
        !aligned(topk_idx, 4) || !aligned(send_pos, 4) || !aligned(out, 16))
        return MOE_EINVAL;
    rc = hip_status(moe::launch_combine_acc_send(D, expert_y, recv_meta, counts, recv_off, expert_off, send_off,
                                                 topk_w, cs_buf, cr_buf, (hipStream_t)stream));
    if (rc) return rc;
    return hip_status(moe::launch_combine_acc_recv(D, cr_buf, send_pos, topk_idx, out, (hipStream_t)stream));
}

int moe_expert_stub(const moe_shape* shape, int32_t mode, const void* expert_x,
                    const float* expert_scale, const int32_t* expert_off, uint16_t* expert_y,
                    void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (mode != 0 && mode != 1) return MOE_EINVAL;
    if (!aligned(expert_x, 16) || !aligned(expert_off, 4) || !aligned(expert_y, 16)) return MOE_EINVAL;
    if (D.fp8 && !aligned(expert_scale, 4)) return MOE_EINVAL;
    return hip_status(moe::launch_expert_stub(D, mode, expert_x, expert_scale, expert_off, expert_y,
                                              (hipStream_t)stream));
}

}  // extern "C"

extern "C" {

int moe_prefill_dispatch(const moe_shape* shape, const void* x, const float* x_scale,
                         const int32_t* topk_idx, int32_t* slot_pos, void* expert_x,
                         float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                         int32_t* expert_src, void* workspace, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (!D.prefill) return MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(topk_idx, 4) || !aligned(slot_pos, 4) || !aligned(expert_x, 16) ||
        !aligned(expert_cnt, 4) || !aligned(expert_off, 4) || !aligned(expert_src, 4))
        return MOE_EINVAL;
    if (D.fp8 && (!aligned(x_scale, 16) || !aligned(expert_scale, 16))) return MOE_EINVAL;
    if (moe::prefill_workspace_bytes(D) > 0 && !aligned(workspace, 4)) return MOE_EINVAL;
    return hip_status(moe::launch_prefill_dispatch(D, x, x_scale, topk_idx, slot_pos, expert_x,
                                                   expert_scale, expert_cnt, expert_off, expert_src,
                                                   workspace, (hipStream_t)stream));
}

int moe_prefill_combine_local(const moe_shape* shape, const uint16_t* expert_y,
                              const int32_t* topk_idx, const int32_t* slot_pos, const float* topk_w,
                              float* partial, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (!D.prefill) return MOE_EINVAL;
    if (!aligned(expert_y, 16) || !aligned(topk_idx, 4) || !aligned(slot_pos, 4) ||
        !aligned(topk_w, 4) || !aligned(partial, 16))
        return MOE_EINVAL;
    return hip_status(moe::launch_prefill_local(D, expert_y, topk_idx, slot_pos, topk_w, partial,
                                                (hipStream_t)stream));
}

int moe_prefill_allreduce(const moe_shape* shape, const float* partial, uint16_t* out, void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (!D.prefill) return MOE_EINVAL;
    if (!aligned(partial, 16) || !aligned(out, 16)) return MOE_EINVAL;
    return hip_status(moe::launch_prefill_allreduce(D, partial, out, (hipStream_t)stream));
}

int moe_prefill_combine(const moe_shape* shape, const uint16_t* expert_y, const int32_t* topk_idx,
                        const int32_t* slot_pos, const float* topk_w, float* partial, uint16_t* out,
                        void* stream) {
    Dims D;
    int rc = make_dims(shape, &D);
    if (rc) return rc;
    if (!D.prefill) return MOE_EINVAL;
    if (D.rc != D.N) return MOE_EINVAL;  // the all-reduce reads every rank's partial
    // validate both steps before launching either
    if (!aligned(expert_y, 16) || !aligned(topk_idx, 4) || !aligned(slot_pos, 4) ||
        !aligned(topk_w, 4) || !aligned(partial, 16) || !aligned(out, 16))
        return MOE_EINVAL;
    rc = hip_status(moe::launch_prefill_local(D, expert_y, topk_idx, slot_pos, topk_w, partial,
                                              (hipStream_t)stream));
    if (rc) return rc;
    return hip_status(moe::launch_prefill_allreduce(D, partial, out, (hipStream_t)stream));
}

}  // extern "C"
