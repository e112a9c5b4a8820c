// dispatch.hip -- MoE dispatch: per-expert counts and exclusive-scan offsets, the pack into
// send buffers contiguous per destination rank (optionally quantising bf16 tokens to e4m3 rows
// on the way), the network stand-in, and the unpack into expert-major order.  Ranks may
// dispatch fewer than T tokens (per-rank counts on the device); absent tokens take no part.
//
// Pages: [EFA] = "Enabling trillion-parameter models on AWS EFA" (send-buffer design paragraph;
// dispatch timing paragraph), [PORT] = "Efficient and portable mixture-of-experts
// communication" (sections Portable kernels and Dispatch), [DSK] = "Lower latency and higher
// throughput with multi-node DeepSeek deployment" (Implementation: Quantization, Cuda Graph).
//
// Orders (all stable, so every output has exactly one correct value):
//  - send buffer of rank s: rows grouped by destination rank d = e / L, (token, slot) order
//    inside a group;
//  - receive buffer of rank d: the groups (s -> d) one after another by s;
//  - expert-major tensor of rank d: by local expert j, then (source, token, slot).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "slots.hpp"

// Waves the send packs aim for (the grid is one token per wave when there are at least this many
// tokens); overridable at build time for launch-shape experiments.
#ifndef MOE_PACK_MIN_WAVES
#define MOE_PACK_MIN_WAVES 4096
#endif
#ifndef MOE_QPACK_MIN_WAVES
#define MOE_QPACK_MIN_WAVES 32768
#endif

namespace moe {

// ------------------------------------------------------------------ count and scan

// Per-chunk expert histogram (only when a rank's T*R slots span several chunks): the counts of
// earlier chunks give each chunk's starting ranks.  Grid (C, N), one slot per thread.
__global__ __launch_bounds__(1024) void k_send_hist(Dims D, const int32_t* __restrict__ topk_idx,
                                                    int32_t* __restrict__ chunk_cnt, int C) {
    extern __shared__ int lds_h[];
    int* hist = lds_h;              // [E]
    int* chunk = lds_h + D.E;       // [blockDim]
    const int s = blockIdx.y, c = blockIdx.x;
    for (int e = threadIdx.x; e < D.E; e += blockDim.x) hist[e] = 0;
    const int32_t* idx_s = topk_idx + (long)s * D.TR;
    const long c0 = (long)c * blockDim.x;
    const long n = stage_chunk(idx_s, chunk, c0, D.TR);
    const long i = c0 + threadIdx.x;
    if (i < (long)rank_tokens(D, D.rb + s) * D.R) {  // slots of present tokens
        int e;
        if (slot_valid(idx_s, chunk, c0, n, i, D.R, D.E, e)) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < D.E; e += blockDim.x)
        chunk_cnt[((long)s * C + c) * D.E + e] = hist[e];
}

// Counts, offsets, positions and metadata.  Grid (C, N); block = chunk of CH = blockDim slots.
// LDS: wcnt[W][E+N] per-wave key counts (scanned in place into per-wave starting ranks),
// base[E+N], tot[E+N], soff[N+1].
__global__ __launch_bounds__(1024) void k_send_rank(Dims D, const int32_t* __restrict__ topk_idx,
                                                    const int32_t* __restrict__ chunk_cnt, int C,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ send_off,
                                                    int32_t* __restrict__ send_pos,
                                                    int32_t* __restrict__ send_meta) {
    extern __shared__ int lds[];
    const int s = blockIdx.y, c = blockIdx.x;
    const int E = D.E, N = D.N, L = D.L, TR = D.TR;
    const int K = E + N;
    const int W = blockDim.x / kWave;
    const int w = wave_id();
    int* wcnt = lds;
    int* base = wcnt + W * K;
    int* tot = base + K;
    int* soff = tot + K;
    int* chunk = soff + N + 1;  // [blockDim]
    for (int i = threadIdx.x; i < W * K; i += blockDim.x) wcnt[i] = 0;

    const int32_t* idx_s = topk_idx + (long)s * TR;
    const long c0 = (long)c * blockDim.x;
    const long n = stage_chunk(idx_s, chunk, c0, TR);  // also orders the zeroing above
    const long i = c0 + threadIdx.x;
    int e = -1;
    bool valid = false;
    if (i < (long)rank_tokens(D, D.rb + s) * D.R) {  // slots of absent tokens stay invalid
        valid = slot_valid(idx_s, chunk, c0, n, i, D.R, E, e);
        if (!valid) set_status(D.status, MOE_EBADIDX);
    }
    const int d = valid ? e / L : 0;
    const int re = wave_key_rank(valid, e, key_bits(E), wcnt + w * K);
    const int rd = wave_key_rank(valid, d, key_bits(N), wcnt + w * K + E);
    __syncthreads();

    // experts: rank base from earlier chunks, per-wave starting ranks, rank totals
    for (int key = threadIdx.x; key < E; key += blockDim.x) {
        int before = 0, after = 0;
        const int nc = C > 1 ? C : 0;  // one chunk: no histograms (the workspace may be absent)
#pragma unroll 8
        for (int cc = 0; cc < nc; ++cc) {  // independent loads, several in flight
            const int v = chunk_cnt[((long)s * C + cc) * E + key];
            before += cc < c ? v : 0;
            after += cc > c ? v : 0;
        }
        base[key] = before;
        tot[key] = column_excl_scan(wcnt + key, K, W, before) + after;
    }
    __syncthreads();
    // destinations: the same from the experts they own
    for (int dd = threadIdx.x; dd < N; dd += blockDim.x) {
        int b = 0, n = 0;
        for (int ee = dd * L; ee < (dd + 1) * L; ++ee) {
            b += base[ee];
            n += tot[ee];
        }
        column_excl_scan(wcnt + E + dd, K, W, b);
        tot[E + dd] = n;
    }
    __syncthreads();
    if (w == 0) wave_excl_scan_array(tot + E, soff, N);
    __syncthreads();

    if (i < TR) {
        int pos = -1;
        if (valid) {
            const int rank_e = wcnt[w * K + e] + re;
            pos = soff[d] + wcnt[w * K + E + d] + rd;
            int2 m;
            m.x = e * TR + (int)i;
            m.y = rank_e;
            reinterpret_cast<int2*>(send_meta)[(long)s * TR + pos] = m;
        }
        send_pos[(long)s * TR + i] = pos;
    }
    if (c == 0) {
        for (int ee = threadIdx.x; ee < E; ee += blockDim.x) counts[(long)s * E + ee] = tot[ee];
        for (int dd = threadIdx.x; dd <= N; dd += blockDim.x)
            send_off[(long)s * (N + 1) + dd] = soff[dd];
    }
}

// ------------------------------------------------------------------ pack

// WPT waves per token (WPT > 1 only when the call has few tokens): the token's payload (and fp8
// scales) is read once and written to each of its R send rows; wave `part` of a token owns the
// chunk groups part, part + WPT, ... of 64 chunks.
template <int U>
__global__ __launch_bounds__(kBlock) void k_send_pack(Dims D, int WPT, const uint8_t* __restrict__ x,
                                                      const float* __restrict__ x_scale,
                                                      const int32_t* __restrict__ send_pos,
                                                      uint8_t* __restrict__ send_buf) {
    const long gw = (long)blockIdx.x * kWavesPerBlock + wave_id();
    const long tok = gw / WPT;  // within the call's ranks
    const int part = (int)(gw - tok * WPT);
    if (tok >= (long)D.rc * D.T) return;
    const int lane = lane_id();
    const long s = tok / D.T;
    if (tok - s * D.T >= rank_tokens(D, D.rb + s)) return;  // absent token
    const int R = D.R;
    const int mypos = lane < R ? send_pos[tok * R + lane] : -1;
    const long xrow = D.fp8 ? D.H : 2L * D.H;
    const u32x4* src_a = reinterpret_cast<const u32x4*>(x + tok * xrow);
    const u32x4* src_b = D.fp8 ? reinterpret_cast<const u32x4*>(x_scale + tok * D.nsc) : src_a;
    uint8_t* rank_base = send_buf + (size_t)s * D.TR * D.P;
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
            const int pos = readlane(mypos, k);
            if (pos < 0 || pos >= D.TR) continue;
            u32x4* dst = reinterpret_cast<u32x4*>(rank_base + (size_t)pos * D.P);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * stride + lane;
                if (c < n16) dst[c] = v[u];
            }
        }
    }
}

// Nearest OCP e4m3 code (exponent bias 7, 3 mantissa bits, largest finite 448) to v, ties to
// the even code, magnitudes above 448 clamped to 448.  Below 2^-6 the codes are multiples of
// 2^-9 (v * 512 is exact; rint rounds half to even).  Above, the fp32 mantissa is rounded to
// 3 bits in place (adding 0x7FFFF plus the kept last bit carries exactly when the dropped bits
// exceed half, or equal half with an odd kept bit) and the exponent rebased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fminf(fabsf(v), 448.0f);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        uint32_t b = __float_as_uint(a);
        b += 0x7FFFFu + ((b >> 20) & 1u);
        code = (b >> 20) - (120u << 3);
    }
    return sign | code;
}

// Send pack with on-the-fly block quantisation ([DSK] Implementation, Quantization: activation
// scales are found per 128-value vector from its largest magnitude): bf16 tokens become e4m3
// codes and one fp32 scale per 128 values, scale = amax / 448 (1 for an all-zero block),
// code = e4m3(x / scale) with an IEEE fp32 division.  WPT waves per token; a wave takes 1024
// values per pass, 16 per lane (8 lanes per 128-value block, whose amax is reduced over them),
// writes 16 code bytes per lane and, from lanes 0 and 1, the pass's 8 scales (32 bytes) into
// each of the token's send rows.
__global__ __launch_bounds__(kBlock) void k_send_pack_q(Dims D, int WPT, const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ send_pos,
                                                        uint8_t* __restrict__ send_buf) {
    const long gw = (long)blockIdx.x * kWavesPerBlock + wave_id();
    const long tok = gw / WPT;  // within the call's ranks
    const int part = (int)(gw - tok * WPT);
    if (tok >= (long)D.rc * D.T) return;
    const long s = tok / D.T;
    if (tok - s * D.T >= rank_tokens(D, D.rb + s)) return;  // absent token
    const int lane = lane_id();
    const int R = D.R, H = D.H;
    const int mypos = lane < R ? send_pos[tok * R + lane] : -1;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + tok * H);
    uint8_t* rank_base = send_buf + (size_t)s * D.TR * D.P;
    for (int v0 = part * 1024; v0 < H; v0 += WPT * 1024) {
        const int v = v0 + lane * 16;  // this lane's first value
        const bool in = v < H;
        u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
        if (in) {
            a = src[v / 8];
            b = src[v / 8 + 1];
        }
        float f[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_to_f32(a[i] & 0xFFFFu);
            f[2 * i + 1] = bf16_to_f32(a[i] >> 16);
            f[8 + 2 * i] = bf16_to_f32(b[i] & 0xFFFFu);
            f[8 + 2 * i + 1] = bf16_to_f32(b[i] >> 16);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = e4m3_rne_sat(f[4 * i] / sc) | (e4m3_rne_sat(f[4 * i + 1] / sc) << 8) |
                   (e4m3_rne_sat(f[4 * i + 2] / sc) << 16) | (e4m3_rne_sat(f[4 * i + 3] / sc) << 24);
        // lane 0 gathers the scales of blocks 0..3 of this pass, lane 1 those of blocks 4..7
        u32x4 sv;
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[j] = __float_as_uint(__shfl(sc, 8 * (4 * (lane & 1) + j), kWave));
        const bool sc_lane = lane < 2 && v0 + 512 * lane < H;
        for (int k = 0; k < R; ++k) {
            const int pos = readlane(mypos, k);
            if (pos < 0 || pos >= D.TR) continue;
            uint8_t* row = rank_base + (size_t)pos * D.P;
            if (in) *reinterpret_cast<u32x4*>(row + v) = q;
            if (sc_lane) *reinterpret_cast<u32x4*>(row + H + 4 * (v0 / 128 + 4 * lane)) = sv;
        }
    }
}

// ------------------------------------------------------------------ network stand-in

// recv_off[d][s] = rows the sources s' < s send to rank d, from the exchanged table (every
// source's send_off): a wave sum over s'.
__device__ __forceinline__ int recv_offset(const int32_t* __restrict__ send_off, int N, int d, int s) {
    int v = 0;
    for (int b = 0; b < s; b += kWave) {
        const int sp = b + lane_id();
        if (sp < s) v += send_off[(long)sp * (N + 1) + d + 1] - send_off[(long)sp * (N + 1) + d];
    }
    return wave_sum(v);
}

// RPB consecutive send rows (s, i) per block, one resolved per wave: its segment d is
// found by a ballot over send_off[s] and it lands at recv_off[d][s] + (i - send_off[s][d]) in
// rank d's receive buffer, metadata alongside; then the block streams the rows.  Blocks 0..N-1
// also write row d = blockIdx of the recv_off output (a wave scan over sources).
template <int RPB, int U, bool CACHED>
__global__ __launch_bounds__(kBlock) void k_net_dispatch(Dims D, const int32_t* __restrict__ send_off,
                                                         const uint8_t* __restrict__ send_buf,
                                                         const int32_t* __restrict__ send_meta,
                                                         uint8_t* __restrict__ recv_buf,
                                                         int32_t* __restrict__ recv_meta,
                                                         int32_t* __restrict__ recv_off) {
    static_assert(RPB <= kWavesPerBlock, "one row per wave");
    __shared__ RowDesc rows[RPB];
    __shared__ u32x4 stage[stage_len(U)];
    const int N = D.N;
    if (blockIdx.x < (unsigned)D.rc && wave_id() == kWavesPerBlock - 1) {
        const int d = D.rb + blockIdx.x;
        int carry = 0;
        for (int b = 0; b < N; b += kWave) {
            const int sp = b + lane_id();
            const int n = sp < N ? send_off[(long)sp * (N + 1) + d + 1] - send_off[(long)sp * (N + 1) + d] : 0;
            const int inc = wave_incl_scan(n);
            if (sp < N) recv_off[(long)d * (N + 1) + sp] = carry + inc - n;
            carry += readlane(inc, kWave - 1);
        }
        if (lane_id() == 0) recv_off[(long)d * (N + 1) + N] = carry;
    }
    const long g = (long)blockIdx.x * RPB + wave_id();  // a send row of the call's ranks
    RowDesc rd = {0, 0, 0, 0};
    if (wave_id() < RPB && g < (long)D.rc * D.TR) {
        const int s = D.rb + (int)(g / D.TR);
        const int i = (int)(g - (long)(s - D.rb) * D.TR);
        const int32_t* so = send_off + (long)s * (N + 1);
        if (i < so[N]) {  // dropped slots leave the tail of the send buffer unused
            const int d = wave_count_le(so, N, i) - 1;
            const long r = d >= 0 ? recv_offset(send_off, N, d, s) + (i - so[d]) : -1;
            if (r >= 0 && r < D.B) {
                const size_t src_row = (size_t)s * D.TR + i, dst_row = (size_t)d * D.B + r;
                if (lane_id() == 0)
                    reinterpret_cast<int2*>(recv_meta)[dst_row] =
                        reinterpret_cast<const int2*>(send_meta)[src_row];
                rd.src_a = rd.src_b = (uint64_t)(send_buf + src_row * D.P);
                rd.dst_a = rd.dst_b = (uint64_t)(recv_buf + dst_row * D.P);
            } else {
                set_status(D.status, MOE_EINVAL);
            }
        }
    }
    if (wave_id() < RPB && lane_id() == 0) rows[wave_id()] = rd;
    __syncthreads();
    // rows past their rank's send total (ranks that send fewer than T tokens) are dead; a block
    // with no live row has nothing to stream (the same test in every thread: block-uniform)
    bool live = false;
#pragma unroll
    for (int w = 0; w < RPB; ++w) live |= rows[w].dst_a != 0;
    if (!live) return;
    block_stream_rows<U, true, !CACHED>(rows, RPB, D.P16, D.P16, D.P16, send_buf, stage);
}

// ------------------------------------------------------------------ receive side

// Where the rows of source s for local expert j start in rank d's expert-major order:
// (rows of experts d*L + j' < d*L + j from every source) + (rows of expert d*L + j from sources
// s' < s).  A wave sum over sources; every lane gets the result.
__device__ __forceinline__ long expert_base(const int32_t* __restrict__ counts, int N, int E, int L, int d,
                                            int s, int j) {
    const int W = j + 1;  // columns d*L .. d*L + j of every source's counts
    const int total = N * W;
    int v = 0;
#pragma unroll 4
    for (int f = lane_id(); f < total; f += kWave) {
        const int sp = f / W, jj = f - sp * W;
        const int c = counts[(long)sp * E + d * L + jj];
        if (jj < j || sp < s) v += c;
    }
    return wave_sum(v);
}

// RPB received rows per block (a global index over all ranks), one resolved per wave:
// its expert-major position is expert_base(d, s, j) + the per-expert rank carried in its
// metadata.  The rows are those received by the call's ranks; block b < rank_count also writes
// the expert_cnt and expert_off of rank rank_begin + b.  STRIDE: blocks stride over the rows
// (a capped grid, for calls on a subset of ranks); otherwise the grid covers every row once, a
// shape that keeps fewer registers live.
template <int RPB, int U, bool STRIDE, bool CACHED>
__global__ __launch_bounds__(kBlock) void k_unpack(Dims D, const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ recv_off,
                                                   const uint8_t* __restrict__ recv_buf,
                                                   const int32_t* __restrict__ recv_meta,
                                                   uint8_t* __restrict__ expert_x,
                                                   float* __restrict__ expert_scale,
                                                   int32_t* __restrict__ expert_cnt,
                                                   int32_t* __restrict__ expert_off,
                                                   int32_t* __restrict__ expert_src,
                                                   int32_t* __restrict__ expert_rpos) {
    extern __shared__ int gb[];  // [rank_count + 1]
    __shared__ RowDesc rows[RPB];
    __shared__ u32x4 stage[stage_len(U)];
    const int N = D.N, L = D.L, E = D.E;
    rank_bases(recv_off + (long)D.rb * (N + 1), N + 1, N, D.rc, gb);
    if (blockIdx.x < (unsigned)D.rc && wave_id() == kWavesPerBlock - 1) {
        const int d = D.rb + blockIdx.x;
        int carry = 0;
        for (int b = 0; b < L; b += kWave) {
            const int j = b + lane_id();
            int c = 0;
            if (j < L) {
#pragma unroll 8
                for (int sp = 0; sp < N; ++sp) c += counts[(long)sp * E + d * L + j];
            }
            const int inc = wave_incl_scan(c);
            if (j < L) {
                expert_cnt[(long)d * L + j] = c;
                expert_off[(long)d * (L + 1) + j] = carry + inc - c;
            }
            carry += readlane(inc, kWave - 1);
        }
        if (lane_id() == 0) expert_off[(long)d * (L + 1) + L] = carry;
    }
    __syncthreads();
    const long total = gb[D.rc];
    auto pass = [&](long base) {
        if (base >= total) return;  // the block's rows all lie past the call's rows (block-uniform)
        const long G = base + wave_id();
        RowDesc rd = {0, 0, 0, 0};
        if (wave_id() < RPB && G < total) {
            const int dl = wave_count_le(gb + 1, D.rc, G);  // ranks whose rows all lie before G
            const int d = D.rb + dl;
            const long r = G - gb[dl];
            const int32_t* ro = recv_off + (long)d * (N + 1);
            const int s = wave_count_le(ro, N, r) - 1;
            const size_t rrow = (size_t)d * D.B + r;
            const int2 m = reinterpret_cast<const int2*>(recv_meta)[rrow];
            const int e = m.x / D.TR;
            const int i = m.x - e * D.TR;
            const int j = e - d * L;
            const long q = (j >= 0 && j < L && s >= 0) ? expert_base(counts, N, E, L, d, s, j) + m.y : -1;
            if (q >= 0 && q < D.B) {
                const size_t qrow = (size_t)d * D.B + q;
                if (lane_id() == 0) {
                    expert_src[qrow] = s * D.TR + i;
                    expert_rpos[qrow] = (int32_t)r;
                }
                const long xrow = D.fp8 ? D.H : 2L * D.H;
                rd.src_a = rd.src_b = (uint64_t)(recv_buf + rrow * D.P);
                rd.dst_a = (uint64_t)(expert_x + qrow * xrow);
                rd.dst_b = D.fp8 ? (uint64_t)(expert_scale + qrow * D.nsc) : rd.dst_a;
            } else {
                set_status(D.status, MOE_EINVAL);
            }
        }
        if (wave_id() < RPB && lane_id() == 0) rows[wave_id()] = rd;
        __syncthreads();
        block_stream_rows<U, !CACHED, true>(rows, RPB, D.P16, D.P16, D.X16, recv_buf, stage);
    };
    if constexpr (STRIDE) {
        for (long base = (long)blockIdx.x * RPB; base < total; base += (long)gridDim.x * RPB) {
            pass(base);
            if (base + (long)gridDim.x * RPB < total) __syncthreads();  // rows[] is rewritten
        }
    } else {
        pass((long)blockIdx.x * RPB);
    }
}

// ------------------------------------------------------------------ launchers

static size_t send_rank_lds(const Dims& D, int CH) {
    const size_t K = (size_t)D.E + D.N;
    return ((CH / kWave) * K + 2 * K + D.N + 1 + CH) * 4;
}

static int send_chunk(const Dims& D) {
    // 16 waves per chunk when the per-wave key table fits in 64 KB of LDS, else 4 (E, N <= 1024
    // keeps the 4-wave table under 64 KB)
    return send_rank_lds(D, 1024) <= 64 * 1024 ? 1024 : 256;
}

hipError_t launch_slot_hist(const Dims& D, const int32_t* topk_idx, int32_t* chunk_cnt, int C, int CH,
                            int ranks, hipStream_t st) {
    hipLaunchKernelGGL(k_send_hist, dim3(C, ranks), dim3(CH), (D.E + CH) * 4, st, D, topk_idx, chunk_cnt, C);
    return hipGetLastError();
}

size_t send_workspace_bytes(const Dims& D) {
    const int CH = send_chunk(D);
    const long C = (D.TR + CH - 1) / CH;
    return C > 1 ? (size_t)D.N * C * D.E * 4 : 0;
}

// Bytes of the workspace one call uses: the histograms of its own ranks.
size_t send_workspace_bytes_used(const Dims& D) {
    const int CH = send_chunk(D);
    const long C = (D.TR + CH - 1) / CH;
    return C > 1 ? (size_t)D.rc * C * D.E * 4 : 0;
}

// ------------------------------------------------------------------ static scratch

// Device memory the library owns, for the dispatch send of callers that cannot allocate: the
// per-chunk expert histograms ([rank][chunk][expert] int32) that k_send_hist writes and
// k_send_rank reads, otherwise kept in the caller's workspace.  Each GPU holds its own copy at its
// own address until the process ends.  On the host this name is a stand-in, not a device
// address: host code passes the address scratch_address() looked up, never `scratch` itself.
static __device__ __align__(256) int32_t scratch[MOE_STATIC_SCRATCH_BYTES / sizeof(int32_t)];

constexpr int kMaxDevices = 64;

// The current device's address of `scratch`, looked up once per device (with that device
// current) and kept.
hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_dispatch_send(const Dims& D, const void* x, const float* x_scale,
                                const int32_t* topk_idx, int32_t* counts, int32_t* send_off,
                                int32_t* send_pos, void* send_buf, int32_t* send_meta,
                                void* workspace, hipStream_t st) {
    const int CH = send_chunk(D);
    const int C = (D.TR + CH - 1) / CH;
    int32_t* chunk_cnt = static_cast<int32_t*>(workspace);
    // the call's ranks [rb, rb + rc): per-rank arrays start at rank rb
    const long rb = D.rb;
    const long xrow = D.fp8 && !D.quant ? D.H : 2L * D.H;  // bytes of one input token
    x = static_cast<const uint8_t*>(x) + rb * D.T * xrow;
    if (x_scale) x_scale += rb * D.T * D.nsc;
    topk_idx += rb * D.TR;
    counts += rb * D.E;
    send_off += rb * (D.N + 1);
    send_pos += rb * D.TR;
    send_buf = static_cast<uint8_t*>(send_buf) + rb * D.TR * D.P;
    send_meta += rb * D.TR * 2;
    if (C > 1) {
        hipLaunchKernelGGL(k_send_hist, dim3(C, D.rc), dim3(CH), (D.E + CH) * 4, st, D, topk_idx, chunk_cnt, C);
    }
    const size_t lds = send_rank_lds(D, CH);
    hipLaunchKernelGGL(k_send_rank, dim3(C, D.rc), dim3(CH), lds, st, D, topk_idx,
                       (const int32_t*)chunk_cnt, C, counts, send_off, send_pos, send_meta);
    const long ntok = (long)D.rc * D.T;
    if (D.quant) {
        // waves per token: enough for MOE_QPACK_MIN_WAVES waves in all, at most one per pass
        const long passes = (D.H + 1023) / 1024;
        const long want = (MOE_QPACK_MIN_WAVES + ntok - 1) / ntok;
        const int wpt = (int)std::max(1L, std::min(passes, want));
        const long waves = ntok * wpt;
        hipLaunchKernelGGL(k_send_pack_q, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock),
                           0, st, D, wpt, (const uint16_t*)x, (const int32_t*)send_pos, (uint8_t*)send_buf);
        return hipGetLastError();
    }
    // up to 8 waves per token when there are fewer than MOE_PACK_MIN_WAVES tokens
    int wpt = 1;
    while (wpt < 8 && ntok * wpt < MOE_PACK_MIN_WAVES && (long)kWave * wpt * 2 <= D.P16) wpt *= 2;
    const long waves = ntok * wpt;
    hipLaunchKernelGGL(k_send_pack<8>, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0,
                       st, D, wpt, (const uint8_t*)x, x_scale, (const int32_t*)send_pos, (uint8_t*)send_buf);
    return hipGetLastError();
}

hipError_t launch_net_dispatch(const Dims& D, const int32_t* send_off, const void* send_buf,
                               const int32_t* send_meta, void* recv_buf, int32_t* recv_meta,
                               int32_t* recv_off, hipStream_t st) {
    const long rows = (long)D.rc * D.TR;  // the send rows of the call's ranks
    const StreamShape sh = stream_shape(D.P16, MOE_NET_MIN_CHUNKS);
    const long blocks = std::max<long>((rows + sh.rpb - 1) / sh.rpb, D.rc);
    const bool cached = exchange_fits_mall(D);
#define MOE_LAUNCH_C(R_, U_, C_)                                                                    \
    hipLaunchKernelGGL((k_net_dispatch<R_, U_, C_>), dim3(blocks), dim3(kBlock), 0, st, D, send_off, \
                       (const uint8_t*)send_buf, send_meta, (uint8_t*)recv_buf, recv_meta, recv_off);
#define MOE_LAUNCH(R_, U_)                                                                          \
    if (sh.rpb == R_ && sh.u == U_) {                                                               \
        if (cached) MOE_LAUNCH_C(R_, U_, true) else MOE_LAUNCH_C(R_, U_, false)                     \
    }
    MOE_STREAM_SHAPES(MOE_LAUNCH)
#undef MOE_LAUNCH
#undef MOE_LAUNCH_C
    return hipGetLastError();
}

hipError_t launch_dispatch_recv(const Dims& D, const int32_t* counts, const int32_t* recv_off,
                                const void* recv_buf, const int32_t* recv_meta, void* expert_x,
                                float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                                int32_t* expert_src, int32_t* expert_rpos, hipStream_t st) {
    const long rows = recv_rows_bound(D);
    const StreamShape sh = stream_shape(D.P16, MOE_UNPACK_MIN_CHUNKS);
    const long blocks = row_blocks(D, rows, sh.rpb);
    const bool stride = blocks * sh.rpb < rows;
    const bool cached = exchange_fits_mall(D);  // the network kernel left the rows in the cache
#define MOE_LAUNCH_S(R_, U_, S_, C_)                                                                \
    hipLaunchKernelGGL((k_unpack<R_, U_, S_, C_>), dim3(blocks), dim3(kBlock), (D.rc + 1) * 4, st, D, counts, \
                       recv_off, (const uint8_t*)recv_buf, recv_meta, (uint8_t*)expert_x, expert_scale,  \
                       expert_cnt, expert_off, expert_src, expert_rpos);
#define MOE_LAUNCH(R_, U_)                                                                          \
    if (sh.rpb == R_ && sh.u == U_) {                                                               \
        if (stride) {                                                                               \
            if (cached) MOE_LAUNCH_S(R_, U_, true, true) else MOE_LAUNCH_S(R_, U_, true, false)     \
        } else {                                                                                    \
            if (cached) MOE_LAUNCH_S(R_, U_, false, true) else MOE_LAUNCH_S(R_, U_, false, false)   \
        }                                                                                           \
    }
    MOE_STREAM_SHAPES(MOE_LAUNCH)
#undef MOE_LAUNCH
#undef MOE_LAUNCH_S
    return hipGetLastError();
}

}  // namespace moe
