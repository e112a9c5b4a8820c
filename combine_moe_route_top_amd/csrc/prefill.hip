// prefill.hip -- expert parallelism for prefill with replicated tokens.
//
// [QWEN] = "Hosting Qwen on Blackwell", section MoE dispatch-combine, Expert parallel: the
// prefill kernel's inputs are the same on every rank, so dispatch only has to pick, on each
// rank, the tokens routed to that rank's experts and stage them as grouped-GEMM inputs; combine
// first accumulates locally the contributions of the rank's experts and then all-reduces across
// the ranks.  Here the N ranks live in one GPU's memory: the receive-side arrays are [N][B][...]
// as in the decode path, the partial sums are [N][T][H] fp32, and the all-reduce is a kernel
// that sums the N partials in rank order.
//
// Dispatch:  k_send_hist (per-chunk expert counts, only when the T*R slots span several chunks),
//            k_pf_rank (slot positions in expert-major order, per-rank expert tables),
//            k_pf_pack (a wave per token: the row read once, written to each local slot's row).
// Combine:   k_pf_local (per rank and token: fp32 fused multiply-adds over the rank's slots in
//            slot order), k_pf_allreduce (fp32 sum over ranks 0..N-1, one rounding to bf16).
#include <algorithm>

#include "common.hpp"
#include "slots.hpp"

// Launch-shape constants, overridable at build time for experiments: the most waves per (rank,
// token) in the local accumulation, and the waves the pack aims for.
#ifndef MOE_PF_LOCAL_WAVES
#define MOE_PF_LOCAL_WAVES 16
#endif
#ifndef MOE_PF_PACK_MIN_WAVES
#define MOE_PF_PACK_MIN_WAVES 4096
#endif

namespace moe {

hipError_t launch_slot_hist(const Dims& D, const int32_t* topk_idx, int32_t* chunk_cnt, int C, int CH,
                            int ranks, hipStream_t st);

// ------------------------------------------------------------------ dispatch

// Slot positions and the per-rank expert tables.  One block per chunk of CH = blockDim of the
// T*R slots.  A slot's position in its owner rank's expert-major rows is (rows of the rank's
// earlier experts) + (earlier slots with the same expert): the latter from the chunk bases of
// earlier chunks, the per-wave starting ranks and the rank inside the wave.
// LDS: wcnt[W][E] (per-wave key counts, scanned in place into starting ranks), tot[E],
// ebase[E], chunk[CH].
__global__ __launch_bounds__(1024) void k_pf_rank(Dims D, const int32_t* __restrict__ topk_idx,
                                                  const int32_t* __restrict__ chunk_cnt, int C,
                                                  int32_t* __restrict__ slot_pos,
                                                  int32_t* __restrict__ expert_cnt,
                                                  int32_t* __restrict__ expert_off) {
    extern __shared__ int lds[];
    const int c = blockIdx.x;
    const int E = D.E, L = D.L, TR = D.TR;
    const int W = blockDim.x / kWave;
    const int w = wave_id();
    int* wcnt = lds;
    int* tot = wcnt + W * E;
    int* ebase = tot + E;
    int* chunk = ebase + E;
    for (int i = threadIdx.x; i < W * E; i += blockDim.x) wcnt[i] = 0;
    const long c0 = (long)c * blockDim.x;
    const long n = stage_chunk(topk_idx, chunk, c0, TR);  // also orders the zeroing above
    const long i = c0 + threadIdx.x;
    int e = -1;
    bool valid = false;
    if (i < TR) {
        valid = slot_valid(topk_idx, chunk, c0, n, i, D.R, E, e);
        if (!valid) set_status(D.status, MOE_EBADIDX);
    }
    const int re = wave_key_rank(valid, e, key_bits(E), wcnt + w * E);
    __syncthreads();
    for (int key = threadIdx.x; key < E; key += blockDim.x) {
        int before = 0, after = 0;
        const int nc = C > 1 ? C : 0;  // one chunk: no histograms (the workspace may be absent)
#pragma unroll 8
        for (int cc = 0; cc < nc; ++cc) {  // independent loads, several in flight
            const int v = chunk_cnt[(long)cc * E + key];
            before += cc < c ? v : 0;
            after += cc > c ? v : 0;
        }
        tot[key] = column_excl_scan(wcnt + key, E, W, before) + after;
    }
    __syncthreads();
    // rows of each rank's earlier experts: a scan over its L experts
    for (int d = threadIdx.x; d < D.N; d += blockDim.x) {
        int run = 0;
        for (int j = 0; j < L; ++j) {
            ebase[d * L + j] = run;
            run += tot[d * L + j];
        }
    }
    __syncthreads();
    if (i < TR) slot_pos[i] = valid ? ebase[e] + wcnt[w * E + e] + re : -1;
    if (c == 0) {  // the tables of the call's ranks
        for (int f = threadIdx.x; f < D.rc * L; f += blockDim.x) {
            const int d = D.rb + f / L, j = f % L;
            expert_cnt[(long)d * L + j] = tot[d * L + j];
            expert_off[(long)d * (L + 1) + j] = ebase[d * L + j];
        }
        for (int dl = threadIdx.x; dl < D.rc; dl += blockDim.x) {
            const int d = D.rb + dl;
            expert_off[(long)d * (L + 1) + L] = ebase[d * L + L - 1] + tot[d * L + L - 1];
        }
    }
}

// WPT waves per token: the token's payload (and fp8 scales) is read once and written to the
// expert-major row of each of its slots owned by one of the call's ranks; wave `part` owns the
// chunk groups part, part + WPT, ... of 64 chunks.  Payload chunks go to expert_x, scale chunks
// to expert_scale.  The first wave of the token also writes expert_src of those rows.  Ordinary
// (cached) stores: the grouped GEMM (here its stand-in) reads the rows next.  Part of their
// write-back then happens while the stand-in runs: nontemporal stores made this call 16 us slower
// and the stand-in 14 us faster, and with the stand-in counted the cached stores are still
// ahead (323 against 331 us for the Qwen3-shaped layer, same process and buffers).
template <int U>
__global__ __launch_bounds__(kBlock) void k_pf_pack(Dims D, int WPT, const uint8_t* __restrict__ x,
                                                    const float* __restrict__ x_scale,
                                                    const int32_t* __restrict__ topk_idx,
                                                    const int32_t* __restrict__ slot_pos,
                                                    uint8_t* __restrict__ expert_x,
                                                    float* __restrict__ expert_scale,
                                                    int32_t* __restrict__ expert_src) {
    const long gw = (long)blockIdx.x * kWavesPerBlock + wave_id();
    const long t = gw / WPT;
    const int part = (int)(gw - t * WPT);
    if (t >= D.T) return;
    const int lane = lane_id();
    const int R = D.R;
    const int pos = lane < R ? slot_pos[t * R + lane] : -1;
    const int d = pos >= 0 ? topk_idx[t * R + lane] / D.L : -1;
    const bool mine = pos >= 0 && pos < D.B && d >= D.rb && d < D.rb + D.rc;
    const uint64_t slots = ballot(mine);
    if (slots == 0) return;  // no slot of this token lands on the call's ranks
    if (part == 0 && mine) expert_src[(size_t)d * D.B + pos] = (int32_t)(t * R + lane);
    const long xrow = D.fp8 ? D.H : 2L * D.H;
    const u32x4* src_a = reinterpret_cast<const u32x4*>(x + t * xrow);
    const u32x4* src_b = D.fp8 ? reinterpret_cast<const u32x4*>(x_scale + t * D.nsc) : src_a;
    const int n16 = D.P16, split = D.X16;
    const int stride = kWave * WPT;
    for (int c0 = part * kWave; c0 < n16; c0 += stride * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * stride + lane;
            if (c < n16) v[u] = c < split ? src_a[c] : src_b[c - split];
        }
        for (int k = 0; k < R; ++k) {
            if (!((slots >> k) & 1)) continue;
            const size_t row = (size_t)readlane(d, k) * D.B + readlane(pos, k);
            u32x4* dst_a = reinterpret_cast<u32x4*>(expert_x + row * xrow);
            u32x4* dst_b = D.fp8 ? reinterpret_cast<u32x4*>(expert_scale + row * D.nsc) : dst_a;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * stride + lane;
                if (c < n16) {
                    if (c < split) dst_a[c] = v[u];
                    else dst_b[c - split] = v[u];
                }
            }
        }
    }
}

// ------------------------------------------------------------------ combine

// partial[d][t] = the fp32 fused-multiply-add chain, in slot order, of w[t][k] * y[d][pos(t, k)]
// over the token's slots k owned by rank d (zero when there are none).  LW waves per (rank,
// token), each owning every LW-th group of 64 chunks of 8 hidden values (the launcher picks LW
// so that a lane has one chunk where it can); a lane keeps one chunk (8 fp32 sums) and loads
// every owned slot's chunk before the multiply-adds.  The partials are stored with ordinary
// (cached) stores: the all-reduce reads them next and writes an eighth as much, so the
// memory-side cache holds most of them for it and their write-back overlaps light writes.  Same
// process, same buffers, Qwen3-shaped prefill: this kernel 110 -> 95 us, the all-reduce 54 -> 52 us,
// the layer 252 -> 232 us back to back (the next layer's calls unchanged).
__global__ __launch_bounds__(kBlock) void k_pf_local(Dims D, int LW, const uint16_t* __restrict__ expert_y,
                                                     const int32_t* __restrict__ topk_idx,
                                                     const int32_t* __restrict__ slot_pos,
                                                     const float* __restrict__ topk_w,
                                                     float* __restrict__ partial) {
    const long gw = (long)blockIdx.x * kWavesPerBlock + wave_id();
    const long item = gw / LW;  // (rank in the call, token)
    const int part = (int)(gw - item * LW);
    if (item >= (long)D.rc * D.T) return;
    const int lane = lane_id();
    const int R = D.R;
    const int d = D.rb + (int)(item / D.T);
    const long t = item % D.T;
    const int pos = lane < R ? slot_pos[t * R + lane] : -1;
    const bool mine = pos >= 0 && pos < D.B && topk_idx[t * R + lane] / D.L == d;
    const float wl = lane < R ? topk_w[t * R + lane] : 0.0f;
    const uint64_t slots = ballot(mine);
    const u32x4* yrows = reinterpret_cast<const u32x4*>(expert_y + (size_t)d * D.B * D.H);
    u32x4* prow = reinterpret_cast<u32x4*>(partial + ((size_t)d * D.T + t) * D.H);
    const int n16 = D.Y16;
    for (int c = part * kWave + lane; c < n16; c += kWave * LW) {
        float acc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
        for (int k0 = 0; k0 < R; k0 += 8) {
            u32x4 v[8];
            float wk[8];
            bool ok[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int k = k0 + kk;
                ok[kk] = k < R && ((slots >> k) & 1);
                wk[kk] = k < R ? readlane_f(wl, k) : 0.0f;
                const int p = k < R ? readlane(pos, k) : 0;
                if (ok[kk]) v[kk] = ld_nt(yrows + (size_t)p * n16 + c);
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (!ok[kk]) continue;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float y = bf16_to_f32((v[kk][u >> 1] >> (16 * (u & 1))) & 0xFFFFu);
                    acc[u] = __builtin_fmaf(wk[kk], y, acc[u]);
                }
            }
        }
        u32x4 o0 = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                    __float_as_uint(acc[3])};
        u32x4 o1 = {__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]),
                    __float_as_uint(acc[7])};
        prow[2 * c] = o0;
        prow[2 * c + 1] = o1;
    }
}

// out[t] = bf16(partial[0][t] + partial[1][t] + ... + partial[N-1][t]): fp32 additions in rank
// order, one rounding.  One thread per 8 hidden values (32 bytes of each partial, 16 of out).
__global__ __launch_bounds__(kBlock) void k_pf_allreduce(Dims D, const float* __restrict__ partial,
                                                         uint16_t* __restrict__ out) {
    const long g = (long)blockIdx.x * kBlock + threadIdx.x;  // a chunk of 8 values of out
    const long n8 = (long)D.T * D.Y16;
    if (g >= n8) return;
    const u32x4* p = reinterpret_cast<const u32x4*>(partial);
    const long plane = (long)D.T * D.Y16 * 2;  // u32x4 per rank's partial
    float s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] = 0.0f;
    // four ranks' chunks in flight at a time, added in rank order
    int d = 0;
    for (; d + 4 <= D.N; d += 4) {
        u32x4 a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = ld_nt(p + (d + j) * plane + 2 * g);
            b[j] = ld_nt(p + (d + j) * plane + 2 * g + 1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                s[u] = s[u] + __uint_as_float(a[j][u]);
                s[4 + u] = s[4 + u] + __uint_as_float(b[j][u]);
            }
    }
    for (; d < D.N; ++d) {
        const u32x4 a = ld_nt(p + d * plane + 2 * g);
        const u32x4 b = ld_nt(p + d * plane + 2 * g + 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s[u] = s[u] + __uint_as_float(a[u]);
            s[4 + u] = s[4 + u] + __uint_as_float(b[u]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = f32_to_bf16(s[2 * u]) | (f32_to_bf16(s[2 * u + 1]) << 16);
    st_nt(reinterpret_cast<u32x4*>(out) + g, o);
}

// ------------------------------------------------------------------ launchers

static size_t pf_rank_lds(const Dims& D, int CH) { return ((size_t)(CH / kWave) * D.E + 2 * D.E + CH) * 4; }

static int pf_chunk(const Dims& D) { return pf_rank_lds(D, 1024) <= 64 * 1024 ? 1024 : 256; }

size_t prefill_workspace_bytes(const Dims& D) {
    const int CH = pf_chunk(D);
    const long C = (D.TR + CH - 1) / CH;
    return C > 1 ? (size_t)C * D.E * 4 : 0;
}

hipError_t launch_prefill_dispatch(const Dims& D, const void* x, const float* x_scale,
                                   const int32_t* topk_idx, int32_t* slot_pos, void* expert_x,
                                   float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                                   int32_t* expert_src, void* workspace, hipStream_t st) {
    const int CH = pf_chunk(D);
    const int C = (D.TR + CH - 1) / CH;
    int32_t* chunk_cnt = static_cast<int32_t*>(workspace);
    if (C > 1) {
        hipError_t e = launch_slot_hist(D, topk_idx, chunk_cnt, C, CH, 1, st);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_pf_rank, dim3(C), dim3(CH), pf_rank_lds(D, CH), st, D, topk_idx,
                       (const int32_t*)chunk_cnt, C, slot_pos, expert_cnt, expert_off);
    const long ntok = D.T;
    int wpt = 1;
    while (wpt < 8 && ntok * wpt < MOE_PF_PACK_MIN_WAVES && (long)kWave * wpt * 2 <= D.P16) wpt *= 2;
    const long waves = ntok * wpt;
    hipLaunchKernelGGL(k_pf_pack<8>, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0,
                       st, D, wpt, (const uint8_t*)x, x_scale, topk_idx, (const int32_t*)slot_pos,
                       (uint8_t*)expert_x, expert_scale, expert_src);
    return hipGetLastError();
}

hipError_t launch_prefill_local(const Dims& D, const uint16_t* expert_y, const int32_t* topk_idx,
                                const int32_t* slot_pos, const float* topk_w, float* partial,
                                hipStream_t st) {
    const int LW = (int)std::min<long>(MOE_PF_LOCAL_WAVES, std::max<long>(1, (D.Y16 + kWave - 1) / kWave));
    const long waves = (long)D.rc * D.T * LW;
    hipLaunchKernelGGL(k_pf_local, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0,
                       st, D, LW, expert_y, topk_idx, slot_pos, topk_w, partial);
    return hipGetLastError();
}

hipError_t launch_prefill_allreduce(const Dims& D, const float* partial, uint16_t* out, hipStream_t st) {
    const long n8 = (long)D.T * D.Y16;
    hipLaunchKernelGGL(k_pf_allreduce, dim3((n8 + kBlock - 1) / kBlock), dim3(kBlock), 0, st, D,
                       partial, out);
    return hipGetLastError();
}

}  // namespace moe
