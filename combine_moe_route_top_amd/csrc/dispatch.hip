// dispatch.hip -- MoE dispatch: per-expert counts and exclusive-scan offsets, the pack into
// send buffers contiguous per destination rank, the network stand-in, and the unpack into
// expert-major order.
//
// Pages: [EFA] = "Enabling trillion-parameter models on AWS EFA" (send-buffer design paragraph;
// dispatch timing paragraph), [PORT] = "Efficient and portable mixture-of-experts
// communication" (sections Portable kernels and Dispatch).
//
// Orders (all stable, so every output has exactly one correct value):
//  - send buffer of rank s: rows grouped by destination rank d = e / L, (token, slot) order
//    inside a group;
//  - receive buffer of rank d: the groups (s -> d) one after another by s;
//  - expert-major tensor of rank d: by local expert j, then (source, token, slot).
#include "common.cuh"

namespace moe {

// ------------------------------------------------------------------ count and scan

// Slot (t, k) of rank s is valid if its expert id is in range and differs from the ids of the
// token's earlier slots.  Invalid slots are dropped and flagged in the status word.
__device__ __forceinline__ bool slot_valid(const int32_t* __restrict__ idx_s, long i, int R, int E,
                                           int& e) {
    e = idx_s[i];
    if (e < 0 || e >= E) return false;
    const long t0 = (i / R) * R;
    for (long j = t0; j < i; ++j)
        if (idx_s[j] == e) return false;
    return true;
}

// Stable rank of this lane's key among the active lanes of the wave with the same key (lower
// lanes first); the leader of each key group also stores the group's size in cnt_row[key].
__device__ __forceinline__ int wave_match_rank(bool active, int key, int* cnt_row) {
    uint64_t pending = ballot(active);
    int rank = 0;
    while (pending) {
        const int leader = __ffsll((unsigned long long)pending) - 1;
        const int lkey = readlane(key, leader);
        const bool mine = active && key == lkey;
        const uint64_t m = ballot(mine);
        if (mine) rank = __popcll(m & lanemask_lt());
        if (lane_id() == leader) cnt_row[lkey] = __popcll(m);
        pending &= ~m;
    }
    return rank;
}

// Per-chunk expert histogram (only when a rank's T*R slots span several chunks): the counts of
// earlier chunks give each chunk's starting ranks.  Grid (C, N), one slot per thread.
__global__ __launch_bounds__(1024) void k_send_hist(Dims D, const int32_t* __restrict__ topk_idx,
                                                    int32_t* __restrict__ chunk_cnt, int C) {
    extern __shared__ int hist[];
    const int s = blockIdx.y, c = blockIdx.x;
    for (int e = threadIdx.x; e < D.E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const long i = (long)c * blockDim.x + threadIdx.x;
    if (i < D.TR) {
        int e;
        if (slot_valid(topk_idx + (long)s * D.TR, i, D.R, D.E, e)) atomicAdd(&hist[e], 1);
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
    for (int i = threadIdx.x; i < W * K; i += blockDim.x) wcnt[i] = 0;
    __syncthreads();

    const int32_t* idx_s = topk_idx + (long)s * TR;
    const long i = (long)c * blockDim.x + threadIdx.x;
    int e = -1;
    bool valid = false;
    if (i < TR) {
        valid = slot_valid(idx_s, i, D.R, E, e);
        if (!valid) set_status(D.status, MOE_EBADIDX);
    }
    const int d = valid ? e / L : 0;
    const int re = wave_match_rank(valid, e, wcnt + w * K);
    const int rd = wave_match_rank(valid, E + d, wcnt + w * K);
    __syncthreads();

    // experts: rank base from earlier chunks, per-wave starting ranks, rank totals
    for (int key = threadIdx.x; key < E; key += blockDim.x) {
        int before = 0, after = 0;
        for (int cc = 0; cc < C; ++cc) {
            if (cc == c) continue;
            const int v = chunk_cnt[((long)s * C + cc) * E + key];
            if (cc < c) before += v;
            else after += v;
        }
        int run = before;
        for (int ww = 0; ww < W; ++ww) {
            const int x = wcnt[ww * K + key];
            wcnt[ww * K + key] = run;
            run += x;
        }
        base[key] = before;
        tot[key] = run + after;
    }
    __syncthreads();
    // destinations: the same from the experts they own
    for (int dd = threadIdx.x; dd < N; dd += blockDim.x) {
        int b = 0, n = 0;
        for (int ee = dd * L; ee < (dd + 1) * L; ++ee) {
            b += base[ee];
            n += tot[ee];
        }
        int run = b;
        for (int ww = 0; ww < W; ++ww) {
            const int x = wcnt[ww * K + E + dd];
            wcnt[ww * K + E + dd] = run;
            run += x;
        }
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

// One wave per token: its payload (and fp8 scales) is read once and written to each of the
// token's R send rows.
template <int U>
__global__ __launch_bounds__(kBlock) void k_send_pack(Dims D, const uint8_t* __restrict__ x,
                                                      const float* __restrict__ x_scale,
                                                      const int32_t* __restrict__ send_pos,
                                                      uint8_t* __restrict__ send_buf) {
    const long tok = (long)blockIdx.x * kWavesPerBlock + wave_id();
    if (tok >= (long)D.N * D.T) return;
    const int lane = lane_id();
    const long s = tok / D.T;
    const int R = D.R;
    const int mypos = lane < R ? send_pos[tok * R + lane] : -1;
    const long xrow = D.fp8 ? D.H : 2L * D.H;
    const u32x4* src_a = reinterpret_cast<const u32x4*>(x + tok * xrow);
    const u32x4* src_b = D.fp8 ? reinterpret_cast<const u32x4*>(x_scale + tok * D.nsc) : src_a;
    uint8_t* rank_base = send_buf + (size_t)s * D.TR * D.P;
    const int n16 = D.P16, split = D.X16;
    for (int c0 = 0; c0 < n16; c0 += kWave * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave + lane;
            if (c < n16) v[u] = c < split ? src_a[c] : src_b[c - split];
        }
        for (int k = 0; k < R; ++k) {
            const int pos = readlane(mypos, k);
            if (pos < 0 || pos >= D.TR) continue;
            u32x4* dst = reinterpret_cast<u32x4*>(rank_base + (size_t)pos * D.P);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave + lane;
                if (c < n16) dst[c] = v[u];
            }
        }
    }
}

// ------------------------------------------------------------------ network stand-in

// recv_off[d][s] = rows sources s' < s send to d.  One wave per destination d.
__global__ __launch_bounds__(kBlock) void k_net_prep(Dims D, const int32_t* __restrict__ send_off,
                                                     int32_t* __restrict__ recv_off) {
    const int d = blockIdx.x * kWavesPerBlock + wave_id();
    if (d >= D.N) return;
    const int N = D.N;
    int carry = 0;
    for (int base = 0; base < N; base += kWave) {
        const int s = base + lane_id();
        int n = 0;
        if (s < N) n = send_off[(long)s * (N + 1) + d + 1] - send_off[(long)s * (N + 1) + d];
        const int inc = wave_incl_scan(n);
        if (s < N) recv_off[(long)d * (N + 1) + s] = carry + inc - n;
        carry += readlane(inc, kWave - 1);
    }
    if (lane_id() == 0) recv_off[(long)d * (N + 1) + N] = carry;
}

// kRowsPerBlock consecutive send rows (s, i) per block, one resolved per wave: its segment d is
// found by a ballot over send_off[s] and it lands at recv_off[d][s] + (i - send_off[s][d]) in
// rank d's receive buffer, metadata alongside; then the block streams the rows.
__global__ __launch_bounds__(kBlock) void k_net_dispatch(Dims D, const int32_t* __restrict__ send_off,
                                                         const uint8_t* __restrict__ send_buf,
                                                         const int32_t* __restrict__ send_meta,
                                                         const int32_t* __restrict__ recv_off,
                                                         uint8_t* __restrict__ recv_buf,
                                                         int32_t* __restrict__ recv_meta) {
    static_assert(kRowsPerBlock == kWavesPerBlock, "one row per wave");
    __shared__ RowDesc rows[kRowsPerBlock];
    const int N = D.N;
    const long g = (long)blockIdx.x * kRowsPerBlock + wave_id();
    RowDesc rd = {0, 0, 0, 0};
    if (g < (long)N * D.TR) {
        const long s = g / D.TR;
        const int i = (int)(g - s * D.TR);
        const int32_t* so = send_off + s * (N + 1);
        if (i < so[N]) {  // dropped slots leave the tail of the send buffer unused
            const int d = wave_count_le(so, N, i) - 1;
            const long r = recv_off[(long)d * (N + 1) + s] + (i - so[d]);
            if (d >= 0 && d < N && r >= 0 && r < D.B) {
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
    if (lane_id() == 0) rows[wave_id()] = rd;
    __syncthreads();
    block_stream_rows(rows, kRowsPerBlock, D.P16, D.P16, D.P16);
}

// ------------------------------------------------------------------ receive side

// Per destination rank d: expert_cnt/expert_off, and base[d][s][j] = expert_off[d][j] + rows of
// local expert j from sources s' < s (the start of source s's run inside expert j's group).
// One block per rank; LDS tab[N][L] of counts, scanned over s by one wave per local expert.
__global__ __launch_bounds__(kBlock) void k_recv_prep(Dims D, const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ expert_cnt,
                                                      int32_t* __restrict__ expert_off,
                                                      int32_t* __restrict__ base_tab) {
    extern __shared__ int lds[];
    const int d = blockIdx.x;
    const int N = D.N, L = D.L, E = D.E;
    int* tab = lds;            // [N][L]
    int* cnt = tab + N * L;    // [L]
    int* off = cnt + L;        // [L + 1]
    for (int idx = threadIdx.x; idx < N * L; idx += blockDim.x) {
        const int s = idx / L, j = idx - s * L;
        tab[idx] = counts[(long)s * E + d * L + j];
    }
    __syncthreads();
    for (int j = wave_id(); j < L; j += kWavesPerBlock) {  // exclusive scan over s of column j
        int carry = 0;
        for (int b = 0; b < N; b += kWave) {
            const int s = b + lane_id();
            const int v = s < N ? tab[s * L + j] : 0;
            const int inc = wave_incl_scan(v);
            if (s < N) tab[s * L + j] = carry + inc - v;
            carry += readlane(inc, kWave - 1);
        }
        if (lane_id() == 0) cnt[j] = carry;
    }
    __syncthreads();
    if (wave_id() == 0) wave_excl_scan_array(cnt, off, L);
    __syncthreads();
    for (int j = threadIdx.x; j < L; j += blockDim.x) expert_cnt[(long)d * L + j] = cnt[j];
    for (int j = threadIdx.x; j <= L; j += blockDim.x) expert_off[(long)d * (L + 1) + j] = off[j];
    for (int idx = threadIdx.x; idx < N * L; idx += blockDim.x)
        base_tab[(long)d * N * L + idx] = tab[idx] + off[idx % L];
}

// kRowsPerBlock received rows per block (a global index over all ranks), one resolved per wave:
// its expert-major position is base[d][s][j] + the per-expert rank carried in its metadata.
__global__ __launch_bounds__(kBlock) void k_unpack(Dims D, const int32_t* __restrict__ recv_off,
                                                   const uint8_t* __restrict__ recv_buf,
                                                   const int32_t* __restrict__ recv_meta,
                                                   const int32_t* __restrict__ base_tab,
                                                   uint8_t* __restrict__ expert_x,
                                                   float* __restrict__ expert_scale,
                                                   int32_t* __restrict__ expert_src,
                                                   int32_t* __restrict__ expert_rpos) {
    extern __shared__ int gb[];  // [N + 1]
    __shared__ RowDesc rows[kRowsPerBlock];
    const int N = D.N;
    rank_bases(recv_off, N + 1, N, N, gb);
    __syncthreads();
    const long G = (long)blockIdx.x * kRowsPerBlock + wave_id();
    RowDesc rd = {0, 0, 0, 0};
    if (G < gb[N]) {
        const int d = wave_count_le(gb + 1, N, G);  // ranks whose rows all lie before G
        const long r = G - gb[d];
        const int32_t* ro = recv_off + (long)d * (N + 1);
        const int s = wave_count_le(ro, N, r) - 1;
        const size_t rrow = (size_t)d * D.B + r;
        const int2 m = reinterpret_cast<const int2*>(recv_meta)[rrow];
        const int e = m.x / D.TR;
        const int i = m.x - e * D.TR;
        const int j = e - d * D.L;
        const long q = (j >= 0 && j < D.L && s >= 0)
                           ? (long)base_tab[((long)d * N + s) * D.L + j] + m.y : -1;
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
    if (lane_id() == 0) rows[wave_id()] = rd;
    __syncthreads();
    block_stream_rows(rows, kRowsPerBlock, D.P16, D.P16, D.X16);
}

// ------------------------------------------------------------------ launchers

static size_t send_rank_lds(const Dims& D, int CH) {
    const size_t K = (size_t)D.E + D.N;
    return ((CH / kWave) * K + 2 * K + D.N + 1) * 4;
}

static int send_chunk(const Dims& D) {
    // 16 waves per chunk when the per-wave key table fits in 64 KB of LDS, else 4 (E, N <= 1024
    // keeps the 4-wave table under 64 KB)
    return send_rank_lds(D, 1024) <= 64 * 1024 ? 1024 : 256;
}

size_t send_workspace_bytes(const Dims& D) {
    const int CH = send_chunk(D);
    const long C = (D.TR + CH - 1) / CH;
    return C > 1 ? (size_t)D.N * C * D.E * 4 : 0;
}

hipError_t launch_dispatch_send(const Dims& D, const void* x, const float* x_scale,
                                const int32_t* topk_idx, int32_t* counts, int32_t* send_off,
                                int32_t* send_pos, void* send_buf, int32_t* send_meta,
                                void* workspace, hipStream_t st) {
    const int CH = send_chunk(D);
    const int C = (D.TR + CH - 1) / CH;
    int32_t* chunk_cnt = static_cast<int32_t*>(workspace);
    if (C > 1) {
        hipLaunchKernelGGL(k_send_hist, dim3(C, D.N), dim3(CH), D.E * 4, st, D, topk_idx, chunk_cnt, C);
    }
    const size_t lds = send_rank_lds(D, CH);
    hipLaunchKernelGGL(k_send_rank, dim3(C, D.N), dim3(CH), lds, st, D, topk_idx,
                       (const int32_t*)chunk_cnt, C, counts, send_off, send_pos, send_meta);
    const long ntok = (long)D.N * D.T;
    hipLaunchKernelGGL(k_send_pack<8>, dim3((ntok + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0,
                       st, D, (const uint8_t*)x, x_scale, (const int32_t*)send_pos, (uint8_t*)send_buf);
    return hipGetLastError();
}

hipError_t launch_net_dispatch(const Dims& D, const int32_t* send_off, const void* send_buf,
                               const int32_t* send_meta, void* recv_buf, int32_t* recv_meta,
                               int32_t* recv_off, hipStream_t st) {
    hipLaunchKernelGGL(k_net_prep, dim3((D.N + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0, st,
                       D, send_off, recv_off);
    const long rows = (long)D.N * D.TR;
    hipLaunchKernelGGL(k_net_dispatch, dim3((rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(kBlock),
                       0, st, D, send_off, (const uint8_t*)send_buf, send_meta,
                       (const int32_t*)recv_off, (uint8_t*)recv_buf, recv_meta);
    return hipGetLastError();
}

size_t recv_workspace_bytes(const Dims& D) { return (size_t)D.N * D.E * 4; }

hipError_t launch_dispatch_recv(const Dims& D, const int32_t* counts, const int32_t* recv_off,
                                const void* recv_buf, const int32_t* recv_meta, void* expert_x,
                                float* expert_scale, int32_t* expert_cnt, int32_t* expert_off,
                                int32_t* expert_src, int32_t* expert_rpos, void* workspace,
                                hipStream_t st) {
    int32_t* base_tab = static_cast<int32_t*>(workspace);
    const size_t lds = ((size_t)D.N * D.L + 2 * D.L + 1) * 4;
    hipLaunchKernelGGL(k_recv_prep, dim3(D.N), dim3(kBlock), lds, st, D, counts, expert_cnt, expert_off,
                       base_tab);
    const long rows = (long)D.N * D.TR;  // every received row, over all ranks, is one of these
    hipLaunchKernelGGL(k_unpack, dim3((rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(kBlock),
                       (D.N + 1) * 4, st, D, recv_off, (const uint8_t*)recv_buf, recv_meta,
                       (const int32_t*)base_tab, (uint8_t*)expert_x, expert_scale, expert_src,
                       expert_rpos);
    return hipGetLastError();
}

}  // namespace moe
