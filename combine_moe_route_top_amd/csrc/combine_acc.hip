// combine_acc.hip -- combine with the sum taken on the sending side: the expert rank forms one
// bf16 partial row per token it holds rows for (the router-weighted sum of those rows), sends
// only the partials back, and the source adds them.  Fewer rows cross the network; each partial
// is rounded to bf16 once more than in the receive-side combine (the accuracy cost).
//
// Pages: [EFA] = "Enabling trillion-parameter models on AWS EFA" (results under the EP64 prefill
// latency figure: another library accumulates on the sending side to cut the data moved, which
// can cost accuracy; the page's own decode kernels accumulate on the receiving side only).
//
// Layout (no new tables): rank d's rows of one token (s, t) are consecutive in its receive order
// (segment s, then (token, slot)).  The partial takes the receive position of the token's first
// row at d in the combine send buffer and, through the network, the send position of the token's
// first slot owned by d in the combine receive buffer; the other rows are not written.  The
// weights of a row come from the source's topk_w (in a deployment they travel with the
// dispatched row: 4 bytes).
#include <algorithm>

#include "common.hpp"
#include "slots.hpp"

namespace moe {

// The token (t) of a receive row from its metadata (e * T*R + t*R + k).
__device__ __forceinline__ int meta_token(int2 m, int TR, int R) { return (m.x % TR) / R; }

// Launch constants, overridable at build time for experiments: the partial kernel's blocks at most
// (blocks step over the receive rows), and the receive rows the network kernel's blocks resolve
// (several per block: many rows move nothing).
#ifndef MOE_ACC_PARTIAL_BLOCKS
#define MOE_ACC_PARTIAL_BLOCKS 1048576
#endif
// Four rows per block (same-process A/B of 2, 4, 8 and 16, and of 512-thread blocks): Kimi-K2's
// combine send 402 -> 381 us; DeepSeek-V3's, where nine in ten rows hold a partial and four rows
// take two streaming passes, 329 -> 338 us.
#ifndef MOE_ACC_NET_ROWS
#define MOE_ACC_NET_ROWS 4
#endif

// What a block needs to form one partial: where it goes, how many rows, their expert-major
// positions and weights (c = 0: the row holds no partial).
struct PartialDesc {
    uint64_t src, dst;  // rank d's expert outputs; the partial's row in the combine send buffer
    int c;
    int q[64];
    float w[64];
};

// Resolve receive row G (a global index over the call's ranks) into a PartialDesc, one wave.  The
// row holds a partial if it is its token's first row at its rank d; lane j < c then takes the
// token's j-th row there (consecutive rows, c <= min(R, L)): its expert-major position
//   expert_off[d][e - d*L] + (rows of expert e from sources s' < s) + rank_e (metadata)
// (the middle term: lanes hold sources, 8 rows' counts loaded together, one wave sum per row) and
// its weight.
__device__ __forceinline__ void resolve_partial(const Dims& D, long G, const int* gb,
                                                const int32_t* __restrict__ recv_meta,
                                                const int32_t* __restrict__ counts,
                                                const int32_t* __restrict__ recv_off,
                                                const int32_t* __restrict__ expert_off,
                                                const float* __restrict__ topk_w,
                                                const uint16_t* __restrict__ expert_y,
                                                uint16_t* __restrict__ cs_buf, PartialDesc* pd) {
    const int N = D.N, L = D.L, E = D.E, TR = D.TR, R = D.R;
    const int lane = lane_id();
    if (lane == 0) pd->c = 0;
    const int dl = wave_count_le(gb + 1, D.rc, G);
    const int d = D.rb + dl;
    const long r = G - gb[dl];
    const int32_t* ro = recv_off + (long)d * (N + 1);
    const int s = wave_count_le(ro, N, r) - 1;
    if (s < 0 || r >= D.B) {
        set_status(D.status, MOE_EINVAL);
        return;
    }
    const long seg0 = ro[s], seg1 = ro[s + 1];
    const int2* meta = reinterpret_cast<const int2*>(recv_meta) + (size_t)d * D.B;
    // the metadata of row r - 1 (every lane) and of rows r + lane, loaded together
    const int2 mprev = r > seg0 ? meta[r - 1] : make_int2(-1, 0);
    const bool in = lane < R && r + lane < seg1;
    int2 mj = {0, 0};
    if (in) mj = meta[r + lane];
    const int t = meta_token(make_int2(readlane(mj.x, 0), 0), TR, R);  // lane 0 holds row r
    if (r > seg0 && meta_token(mprev, TR, R) == t) return;  // not the token's first row here
    const bool mine = in && meta_token(mj, TR, R) == t;
    const int c = __popcll(ballot(mine));  // lanes 0 .. c-1: the token's rows are consecutive
    // row j's expert, its offset, weight and rank, issued before the counts' wave sums
    const int e = mine ? mj.x / TR : 0;
    const int jl = e - d * L, i = mj.x - e * TR;  // local expert; slot t*R + k of the source
    const bool e_ok = !mine || (jl >= 0 && jl < L && i >= 0);
    const int eoff = mine && e_ok ? expert_off[(long)d * (L + 1) + jl] : 0;
    const float wj = mine && e_ok ? topk_w[(size_t)s * TR + i] : 0.0f;
    const int ec = (e >= 0 && e < E) ? e : 0;  // counts are read in range whatever the metadata
    int before = 0;
    for (int j0 = 0; j0 < c; j0 += 8) {
        int ej[8], cnt[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            ej[jj] = j0 + jj < c ? readlane(ec, j0 + jj) : 0;
            cnt[jj] = 0;
        }
        for (int sp0 = 0; sp0 < s; sp0 += kWave) {
            const int sp = sp0 + lane;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                if (sp < s && j0 + jj < c) cnt[jj] += counts[(long)sp * E + ej[jj]];
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            if (j0 + jj >= c) break;
            const int b = wave_sum(cnt[jj]);
            if (lane == j0 + jj) before = b;
        }
    }
    const long qq = (long)eoff + before + mj.y;
    const int q = mine && e_ok && qq >= 0 && qq < D.B ? (int)qq : -1;
    if (ballot(mine && q < 0)) {
        set_status(D.status, MOE_EINVAL);
        return;
    }
    if (mine) {
        pd->q[lane] = q;
        pd->w[lane] = wj;
    }
    if (lane == 0) {
        pd->src = (uint64_t)(expert_y + (size_t)d * D.B * D.H);
        pd->dst = (uint64_t)(cs_buf + ((size_t)d * D.B + r) * D.H);
        pd->c = c;
    }
}

// The block's threads form the partial row: UE chunks per thread per step, every load of a step
// (UE * c <= 8, or the rows in groups of 8 when UE == 1) issued at once, each chunk's rows summed
// in slot order with fp32 fused multiply-adds and rounded once to bf16.
template <int UE>
__device__ __forceinline__ void partial_stream(const PartialDesc* pd, int c, const u32x4* __restrict__ yrank,
                                               int n16) {
    u32x4* orow = reinterpret_cast<u32x4*>(pd->dst);
    for (int cb = threadIdx.x; cb < n16; cb += kBlock * UE) {
        if constexpr (UE > 1) {
            u32x4 v[8];
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const int j = n / UE, ch = cb + (n % UE) * kBlock;
                if (j < c && ch < n16) v[n] = ld_nt(yrank + (size_t)pd->q[j] * n16 + ch);
            }
#pragma unroll
            for (int u = 0; u < UE; ++u) {
                const int ch = cb + u * kBlock;
                float acc[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
#pragma unroll
                for (int j = 0; j < 8 / UE; ++j) {
                    if (j >= c) break;
                    const float w = pd->w[j];
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        acc[k] = __builtin_fmaf(w, bf16_to_f32((v[j * UE + u][k >> 1] >> (16 * (k & 1))) & 0xFFFF),
                                                acc[k]);
                }
                if (ch < n16) {
                    u32x4 o;
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = f32_to_bf16(acc[2 * k]) | (f32_to_bf16(acc[2 * k + 1]) << 16);
                    st_nt(orow + ch, o);
                }
            }
        } else {
            const int ch = cb;
            float acc[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
            for (int j0 = 0; j0 < c; j0 += 8) {
                u32x4 v[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    if (j0 + jj < c) v[jj] = ld_nt(yrank + (size_t)pd->q[j0 + jj] * n16 + ch);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    if (j0 + jj >= c) break;
                    const float w = pd->w[j0 + jj];
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        acc[k] = __builtin_fmaf(w, bf16_to_f32((v[jj][k >> 1] >> (16 * (k & 1))) & 0xFFFF), acc[k]);
                }
            }
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = f32_to_bf16(acc[2 * k]) | (f32_to_bf16(acc[2 * k + 1]) << 16);
            st_nt(orow + ch, o);
        }
    }
}

// Partial rows: rpb receive rows per block and step (blocks step over the rows of the call's
// ranks); wave w < rpb resolves one row, then the whole block streams the partials among them in
// turn.  Four rows per step hide the resolve latency when every block has several rows to do; one
// row per step keeps a small call (one rank's few rows) short.  The choice follows the device-side
// row count, the same for every block.
__global__ __launch_bounds__(kBlock) void k_acc_partial(Dims D, const uint16_t* __restrict__ expert_y,
                                                        const int32_t* __restrict__ recv_meta,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ recv_off,
                                                        const int32_t* __restrict__ expert_off,
                                                        const float* __restrict__ topk_w,
                                                        uint16_t* __restrict__ cs_buf) {
    extern __shared__ int gb[];
    __shared__ PartialDesc pd[kWavesPerBlock];
    rank_bases(recv_off + (long)D.rb * (D.N + 1), D.N + 1, D.N, D.rc, gb);
    __syncthreads();
    const long total = gb[D.rc];
    const int rpb = total >= (long)gridDim.x * kWavesPerBlock ? kWavesPerBlock : 1;
    for (long G0 = (long)blockIdx.x * rpb; G0 < total; G0 += (long)gridDim.x * rpb) {
        if (wave_id() < rpb) {
            PartialDesc* mine = &pd[wave_id()];
            if (G0 + wave_id() < total)
                resolve_partial(D, G0 + wave_id(), gb, recv_meta, counts, recv_off, expert_off, topk_w, expert_y,
                                cs_buf, mine);
            else if (lane_id() == 0)
                mine->c = 0;
        }
        __syncthreads();
        for (int w = 0; w < rpb; ++w) {
            const int c = pd[w].c;  // block-uniform
            const u32x4* yrank = reinterpret_cast<const u32x4*>(pd[w].src);
            if (c == 1 || c == 2) partial_stream<4>(&pd[w], c, yrank, D.Y16);
            else if (c == 3 || c == 4) partial_stream<2>(&pd[w], c, yrank, D.Y16);
            else if (c > 4) partial_stream<1>(&pd[w], c, yrank, D.Y16);
        }
        __syncthreads();  // pd is rewritten by the next step
    }
}

// Network back for the partials: as the receive-side combine's network step (row r of segment
// (s -> d) to send_off[s][d] + (r - recv_off[d][s]) in rank s's combine receive buffer), but a
// row moves only if it is its token's first row at d.  W receive rows per block (a global index
// over the call's ranks) are resolved by wave 0, one per lane; the rows that hold a partial are
// gathered at the front of the block's row list (a ballot) and only they are streamed, so the
// rows that move nothing (most of them where a token's rows crowd onto one rank) cost a resolve
// lane, not a block.  STRIDE: blocks stride over a capped grid.  Cached stores, as in the
// receive-side network back: the source's sum reads these rows next (same process, cache flushed
// between layers: the send half 338 -> 304 us on DeepSeek-V3, 379 -> 361 us on Kimi-K2, the sum
// within 4 us).
// Threads per block of the partial network kernel (512 let four rows stream in one pass but lost
// the Kimi-K2 gain: 406 us).
#ifndef MOE_ACC_NET_THREADS
#define MOE_ACC_NET_THREADS 256
#endif
template <int W, int U, bool STRIDE>
__global__ __launch_bounds__(MOE_ACC_NET_THREADS) void k_acc_net(Dims D, const uint16_t* __restrict__ cs_buf,
                                                    const int32_t* __restrict__ recv_meta,
                                                    const int32_t* __restrict__ recv_off,
                                                    const int32_t* __restrict__ send_off,
                                                    uint16_t* __restrict__ cr_buf) {
    static_assert(W <= kWave, "one row per lane of wave 0");
    extern __shared__ int lds_an[];  // gb[rank_count + 1], then ro[N + 1] of the block's first rank
    __shared__ RowDesc rows[W];
    __shared__ u32x4 stage[stage_len(U, MOE_ACC_NET_THREADS)];
    __shared__ int nlive;
    const int N = D.N;
    int* gb = lds_an;
    int* sro = lds_an + D.rc + 1;
    rank_bases(recv_off + (long)D.rb * (N + 1), N + 1, N, D.rc, gb);
    __syncthreads();
    const long total = gb[D.rc];
    auto pass = [&](long base) {
        if (wave_id() == 0) {
            const int lane = lane_id();
            const long G = base + lane;
            const bool in = lane < W && G < total;
            // rank of each row: gb[lo] <= G < gb[lo + 1]
            int lo = 0;
            if (in) {
                int hi = D.rc;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (gb[mid] <= G) lo = mid;
                    else hi = mid;
                }
            }
            // the receive offsets of the rank of the block's first row, staged in LDS
            const int l0 = readlane(lo, 0);
            const int32_t* ro0 = recv_off + (long)(D.rb + l0) * (N + 1);
            for (int k = lane; k <= N; k += kWave) sro[k] = ro0[k];
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            RowDesc rd = {0, 0, 0, 0};
            bool live = false;
            if (in) {
                const int d = D.rb + lo;
                const long r = G - gb[lo];  // < recv_off[d][N]
                const int32_t* ro = recv_off + (long)d * (N + 1);
                const bool staged = lo == l0;
                // source: ro[s] <= r < ro[s + 1]
                int s = 0, hi = N;
                while (hi - s > 1) {
                    const int mid = (s + hi) >> 1;
                    if ((staged ? sro[mid] : ro[mid]) <= r) s = mid;
                    else hi = mid;
                }
                const long seg0 = staged ? sro[s] : ro[s];
                const long i = send_off[(long)s * (N + 1) + d] + (r - seg0);
                if (i >= 0 && i < D.TR && r < D.B) {
                    const int2* meta = reinterpret_cast<const int2*>(recv_meta) + (size_t)d * D.B;
                    live = r == seg0 || meta_token(meta[r - 1], D.TR, D.R) != meta_token(meta[r], D.TR, D.R);
                    if (live) {
                        rd.src_a = rd.src_b = (uint64_t)(cs_buf + ((size_t)d * D.B + r) * D.H);
                        rd.dst_a = rd.dst_b = (uint64_t)(cr_buf + ((size_t)s * D.TR + i) * D.H);
                    }
                } else {
                    set_status(D.status, MOE_EINVAL);
                }
            }
            const uint64_t m = ballot(live);
            if (live) rows[__popcll(m & lanemask_lt())] = rd;
            if (lane == 0) nlive = __popcll(m);
        }
        __syncthreads();
        block_stream_rows<U, true, false>(rows, nlive, D.Y16, D.Y16, D.Y16, cs_buf, stage);
    };
    if constexpr (STRIDE) {
        for (long base = (long)blockIdx.x * W; base < total; base += (long)gridDim.x * W) {
            pass(base);
            if (base + (long)gridDim.x * W < total) __syncthreads();  // rows[], nlive, sro are rewritten
        }
    } else {
        pass((long)blockIdx.x * W);
    }
}

// The source's sum: out[s][t] = bf16(fp32 sum of the token's partials in the order of their first
// slots).  Slot k holds a partial if it is valid and no earlier valid slot of the token has the
// same owner rank (one ballot per owner bit finds the lower lanes with the same owner).  The
// partial slots (a ballot, in slot order) are taken GP at a time: every load of a group is issued
// before its adds, a group's unused entries add a zero chunk (exact: the sums start at +0.0 and so
// are never -0.0), and a lane past the row's end reads the row's last chunk and drops it.  WW waves
// per token and CU chunks per lane, chosen as in the receive-side weighted sum; walking only the
// partials (about three of a Kimi-K2 token's eight slots) instead of every slot holds GP * CU
// chunks per lane instead of 8 * CU: 133 instead of 220 registers in the four-chunk shape, and
// Kimi-K2's sum 111 -> 81 us (groups of 8: 102 us).
#ifndef MOE_ACC_SUM_GROUP
#define MOE_ACC_SUM_GROUP 4
#endif
template <int CU, int GP>
__global__ __launch_bounds__(kBlock) void k_acc_sum(Dims D, int WW, const uint16_t* __restrict__ cr_buf,
                                                    const int32_t* __restrict__ send_pos,
                                                    const int32_t* __restrict__ topk_idx,
                                                    uint16_t* __restrict__ out) {
    const long gw = (long)blockIdx.x * kWavesPerBlock + wave_id();
    const long tok = gw / WW;  // within the call's ranks
    const int part = (int)(gw - tok * WW);
    if (tok >= (long)D.rc * D.T) return;
    const int lane = lane_id();
    const int R = D.R;
    const long s = tok / D.T;
    if (tok - s * D.T >= rank_tokens(D, D.rb + s)) return;  // absent token: its row is not written
    const int pos = lane < R ? send_pos[tok * R + lane] : -1;
    const bool valid = pos >= 0 && pos < D.TR;
    const int owner = valid ? topk_idx[tok * R + lane] / D.L : 0;
    const uint64_t same = same_key_lanes(valid, owner, key_bits(D.N));
    const uint64_t pm = ballot(valid && (same & lanemask_lt()) == 0);  // slots holding a partial
    const int np = __popcll(pm);
    const u32x4* rank_rows = reinterpret_cast<const u32x4*>(cr_buf + (size_t)s * D.TR * D.H);
    u32x4* orow = reinterpret_cast<u32x4*>(out + (size_t)tok * D.H);
    const int n16 = D.Y16;
    for (int c0 = part * kWave + lane; c0 < n16; c0 += kWave * WW * CU) {
        float acc[CU][8];
#pragma unroll
        for (int cu = 0; cu < CU; ++cu)
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[cu][u] = 0.0f;
        uint64_t m = pm;
        for (int j0 = 0; j0 < np; j0 += GP) {
            u32x4 v[CU][GP];
#pragma unroll
            for (int jj = 0; jj < GP; ++jj) {
                int p = -1;
                if (m) {
                    p = readlane(pos, (int)__builtin_ctzll(m));
                    m &= m - 1;
                }
#pragma unroll
                for (int cu = 0; cu < CU; ++cu) {
                    const int c = min(c0 + cu * kWave * WW, n16 - 1);
                    v[cu][jj] = u32x4{0u, 0u, 0u, 0u};
                    if (p >= 0) v[cu][jj] = ld_nt(rank_rows + (size_t)p * n16 + c);
                }
            }
#pragma unroll
            for (int jj = 0; jj < GP; ++jj) {
#pragma unroll
                for (int cu = 0; cu < CU; ++cu)
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        acc[cu][u] += bf16_to_f32((v[cu][jj][u >> 1] >> (16 * (u & 1))) & 0xFFFF);
            }
        }
#pragma unroll
        for (int cu = 0; cu < CU; ++cu) {
            const int c = c0 + cu * kWave * WW;
            if (c < n16) {
                u32x4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    o[u] = f32_to_bf16(acc[cu][2 * u]) | (f32_to_bf16(acc[cu][2 * u + 1]) << 16);
                st_nt(orow + c, o);
            }
        }
    }
}

// ------------------------------------------------------------------ launchers

// Waves per token for the source's sum: the fewest (at most max_ww) that cover a row with cu
// 8-value chunks per lane.
static int acc_waves(const Dims& D, int cu, int max_ww) {
    return (int)std::min<long>(max_ww, std::max<long>(1, (D.Y16 + cu * kWave - 1) / (cu * kWave)));
}
// Calls with at least this many waves in the four-chunk shape take it (as the weighted sum does).
#ifndef MOE_ACC_SUM_WIDE_MIN_WAVES
#define MOE_ACC_SUM_WIDE_MIN_WAVES 4096
#endif

hipError_t launch_combine_acc_send(const Dims& D, const uint16_t* expert_y, const int32_t* recv_meta,
                                   const int32_t* counts, const int32_t* recv_off,
                                   const int32_t* expert_off, const int32_t* send_off,
                                   const float* topk_w, uint16_t* cs_buf, uint16_t* cr_buf,
                                   hipStream_t st) {
    const long rows = recv_rows_bound(D);  // rows the call's ranks received
    const long blocks = std::min<long>(MOE_ACC_PARTIAL_BLOCKS, row_blocks(D, rows, kWavesPerBlock));
    hipLaunchKernelGGL(k_acc_partial, dim3((unsigned)blocks), dim3(kBlock), (D.rc + 1) * 4, st, D, expert_y,
                       recv_meta, counts, recv_off, expert_off, topk_w, cs_buf);
    // W receive rows per block, at most 8 chunks per thread per pass
    const int u = (int)std::min<long>(8, std::max<long>(1, (long)D.Y16 * MOE_ACC_NET_ROWS / MOE_ACC_NET_THREADS));
    const int u2 = u <= 1 ? 1 : u <= 2 ? 2 : u <= 4 ? 4 : 8;
    const long nb = row_blocks(D, rows, MOE_ACC_NET_ROWS);
    const bool stride = nb * MOE_ACC_NET_ROWS < rows;
    const size_t lds = (size_t)(D.rc + 1 + D.N + 1) * 4;
#define MOE_LAUNCH_S(U_, S_)                                                                         \
    hipLaunchKernelGGL((k_acc_net<MOE_ACC_NET_ROWS, U_, S_>), dim3(nb), dim3(MOE_ACC_NET_THREADS), lds, st, D, \
                       (const uint16_t*)cs_buf, recv_meta, recv_off, send_off, cr_buf);
#define MOE_LAUNCH(U_)                                                                              \
    if (u2 == U_) {                                                                                 \
        if (stride) MOE_LAUNCH_S(U_, true)                                                          \
        else MOE_LAUNCH_S(U_, false)                                                                \
    }
    MOE_LAUNCH(1) MOE_LAUNCH(2) MOE_LAUNCH(4) MOE_LAUNCH(8)
#undef MOE_LAUNCH
#undef MOE_LAUNCH_S
    return hipGetLastError();
}

hipError_t launch_combine_acc_recv(const Dims& D, const uint16_t* cr_buf, const int32_t* send_pos,
                                   const int32_t* topk_idx, uint16_t* out, hipStream_t st) {
    // the tokens of ranks [rb, rb + rc)
    const long rb = D.rb;
    cr_buf += rb * D.TR * D.H;
    send_pos += rb * D.TR;
    topk_idx += rb * D.TR;
    out += rb * D.T * D.H;
    const long ntok = (long)D.rc * D.T;
    const int ww4 = acc_waves(D, 4, 4);
    if (ntok * ww4 >= MOE_ACC_SUM_WIDE_MIN_WAVES) {
        const long waves = ntok * ww4;
        hipLaunchKernelGGL((k_acc_sum<4, MOE_ACC_SUM_GROUP>), dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                           dim3(kBlock), 0, st, D, ww4, cr_buf, send_pos, topk_idx, out);
    } else {
        const int ww1 = acc_waves(D, 1, 16);
        const long waves = ntok * ww1;
        hipLaunchKernelGGL((k_acc_sum<1, MOE_ACC_SUM_GROUP>), dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                           dim3(kBlock), 0, st, D, ww1, cr_buf, send_pos, topk_idx, out);
    }
    return hipGetLastError();
}

}  // namespace moe
