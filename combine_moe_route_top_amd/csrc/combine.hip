// combine.hip -- MoE combine: shuffle the expert outputs back into receive order, move them
// back with one contiguous write per (rank, peer) segment, and take the router-weighted sum.
// Also the stand-in expert between dispatch and combine.
//
// Pages: [EFA] = "Enabling trillion-parameter models on AWS EFA" (combine paragraphs: the
// metadata is known from dispatch, tokens are shuffled, sent back with one write per peer and
// accumulated from the receive buffer into the output); [PORT] = "Efficient and portable
// mixture-of-experts communication" (section Combine: 16-bit activations, the receiver forms
// the weighted average of all expert contributions into an externally allocated tensor).
#include <algorithm>

#include "common.hpp"

namespace moe {

// ------------------------------------------------------------------ stand-in expert

// e4m3 (OCP: bias 7, 3 mantissa bits, S.1111.111 = NaN) to double, exactly.
__device__ __forceinline__ double e4m3_to_f64(uint32_t b) {
    const int e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) v = __longlong_as_double(0x7FF8000000000000ll);
    else if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return (b & 0x80) ? -v : v;
}

// Round a double to bf16 (nearest even) without double rounding: first to fp32 rounding to odd
// (sticky low bit), which keeps enough bits for the second, nearest-even, rounding to be exact.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
    float f = (float)x;
    if ((double)f != x && !isnan(x) && !isinf(f)) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(x)) u -= 1;  // step back toward zero: the truncated value
        u |= 1;
        f = __uint_as_float(u);
    }
    return f32_to_bf16(f);
}

// The stand-in expert for one expert-major row G (a global index over the call's ranks).
__device__ __forceinline__ void stub_row(Dims D, int mode, const uint8_t* __restrict__ expert_x,
                                         const float* __restrict__ expert_scale,
                                         const int32_t* __restrict__ expert_off,
                                         uint16_t* __restrict__ expert_y, const int* gb, long G) {
    const int L = D.L;
    const int dl = wave_count_le(gb + 1, D.rc, G);
    const int d = D.rb + dl;
    const long q = G - gb[dl];
    const int j = wave_count_le(expert_off + (long)d * (L + 1) + 1, L, q);
    const int e = d * L + j;
    const double tag = mode == 1 ? (double)(64 + e % 64) / 64.0 : 1.0;
    const size_t row = (size_t)d * D.B + q;
    const int H = D.H;
    uint16_t* y = expert_y + row * H;
    // 8 outputs per lane per step: one 16-byte store
    for (int h0 = lane_id() * 8; h0 < H; h0 += kWave * 8) {
        uint32_t o[8];
        if (D.fp8) {
            const uint8_t* xq = expert_x + row * H;
            const float sc = expert_scale[row * D.nsc + h0 / 128];
            const uint2 codes = *reinterpret_cast<const uint2*>(xq + h0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t b = ((u < 4 ? codes.x : codes.y) >> (8 * (u & 3))) & 0xFF;
                o[u] = f64_to_bf16(e4m3_to_f64(b) * (double)sc * tag);
            }
        } else {
            const uint16_t* xb = reinterpret_cast<const uint16_t*>(expert_x) + row * H;
            const u32x4 v = *reinterpret_cast<const u32x4*>(xb + h0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t b = (v[u >> 1] >> (16 * (u & 1))) & 0xFFFF;
                o[u] = f64_to_bf16((double)bf16_to_f32(b) * tag);
            }
        }
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = o[2 * u] | (o[2 * u + 1] << 16);
        *reinterpret_cast<u32x4*>(y + h0) = w;
    }
}

// One wave per expert-major row (a global index over the call's ranks; waves stride over the
// rows).  mode 0: identity; mode 1: times (64 + e % 64) / 64.  The product is formed exactly in
// fp64 and rounded once to bf16.
__global__ __launch_bounds__(kBlock) void k_expert_stub(Dims D, int mode, const uint8_t* __restrict__ expert_x,
                                                        const float* __restrict__ expert_scale,
                                                        const int32_t* __restrict__ expert_off,
                                                        uint16_t* __restrict__ expert_y) {
    extern __shared__ int gb[];
    const int L = D.L;
    rank_bases(expert_off + (long)D.rb * (L + 1), L + 1, L, D.rc, gb);
    __syncthreads();
    for (long G = (long)blockIdx.x * kWavesPerBlock + wave_id(); G < gb[D.rc];
         G += (long)gridDim.x * kWavesPerBlock)
        stub_row(D, mode, expert_x, expert_scale, expert_off, expert_y, gb, G);
}

// ------------------------------------------------------------------ combine

// Shuffle: cs[d][expert_rpos[q]] = y[d][q].  RPB expert-major rows per block (a global
// index over all ranks), one resolved per wave, then streamed.  STRIDE: blocks stride over the
// rows of a capped grid (calls on a subset of ranks); otherwise one pass covers every row.
template <int RPB, int U, bool STRIDE>
__global__ __launch_bounds__(kBlock) void k_combine_pack(Dims D, const uint16_t* __restrict__ expert_y,
                                                         const int32_t* __restrict__ expert_rpos,
                                                         const int32_t* __restrict__ recv_off,
                                                         uint16_t* __restrict__ cs_buf) {
    extern __shared__ int gb[];
    __shared__ RowDesc rows[RPB];
    __shared__ u32x4 stage[stage_len(U)];
    const int N = D.N;
    rank_bases(recv_off + (long)D.rb * (N + 1), N + 1, N, D.rc, gb);
    __syncthreads();
    const long total = gb[D.rc];
    auto pass = [&](long base) {
        if (base >= total) return;  // the block's rows all lie past the call's rows (block-uniform)
        const long G = base + wave_id();
        RowDesc rd = {0, 0, 0, 0};
        if (wave_id() < RPB && G < total) {
            const int dl = wave_count_le(gb + 1, D.rc, G);
            const int d = D.rb + dl;
            const long q = G - gb[dl];
            const long r = expert_rpos[(size_t)d * D.B + q];
            if (r >= 0 && r < D.B) {
                rd.src_a = rd.src_b = (uint64_t)(expert_y + ((size_t)d * D.B + q) * D.H);
                rd.dst_a = rd.dst_b = (uint64_t)(cs_buf + ((size_t)d * D.B + r) * D.H);
            } else {
                set_status(D.status, MOE_EINVAL);
            }
        }
        if (wave_id() < RPB && lane_id() == 0) rows[wave_id()] = rd;
        __syncthreads();
        block_stream_rows<U>(rows, RPB, D.Y16, D.Y16, D.Y16, expert_y, stage);
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

// Network back: the call's ranks d push their combine send buffers, read in order (a global
// index over those ranks); row r of segment (s -> d) lands at send_off[s][d] + (r - recv_off[d][s])
// in rank s's combine receive buffer, where s's dispatch send buffer had it.  STRIDE as for the
// shuffle.  Nontemporal loads, cached stores: the weighted sum reads these rows next and writes
// only one row per token, so it finds part of them in the memory-side cache and the write-back of
// the rest overlaps a kernel whose own writes are light.  In one process on the same buffers,
// layers run back to back with nothing between them (so no write-back could fall outside the
// timed calls), DeepSeek-V3 bf16 went 885 -> 860 us and e4m3 659 -> 629 us, the weighted sum
// unchanged; Kimi-K2, whose 940 MB exchange is far larger than the cache, was unchanged.
template <int RPB, int U, bool STRIDE>
__global__ __launch_bounds__(kBlock) void k_combine_net(Dims D, const uint16_t* __restrict__ cs_buf,
                                                        const int32_t* __restrict__ recv_off,
                                                        const int32_t* __restrict__ send_off,
                                                        uint16_t* __restrict__ cr_buf) {
    extern __shared__ int gb[];
    __shared__ RowDesc rows[RPB];
    __shared__ u32x4 stage[stage_len(U)];
    const int N = D.N;
    rank_bases(recv_off + (long)D.rb * (N + 1), N + 1, N, D.rc, gb);
    __syncthreads();
    const long total = gb[D.rc];
    auto pass = [&](long base) {
        if (base >= total) return;  // the block's rows all lie past the call's rows (block-uniform)
        const long G = base + wave_id();
        RowDesc rd = {0, 0, 0, 0};
        if (wave_id() < RPB && G < total) {
            const int dl = wave_count_le(gb + 1, D.rc, G);
            const int d = D.rb + dl;
            const long r = G - gb[dl];
            const int32_t* ro = recv_off + (long)d * (N + 1);
            const int s = wave_count_le(ro, N, r) - 1;
            const long i = s >= 0 ? send_off[(long)s * (N + 1) + d] + (r - ro[s]) : -1;
            if (i >= 0 && i < D.TR) {
                rd.src_a = rd.src_b = (uint64_t)(cs_buf + ((size_t)d * D.B + r) * D.H);
                rd.dst_a = rd.dst_b = (uint64_t)(cr_buf + ((size_t)s * D.TR + i) * D.H);
            } else {
                set_status(D.status, MOE_EINVAL);
            }
        }
        if (wave_id() < RPB && lane_id() == 0) rows[wave_id()] = rd;
        __syncthreads();
        block_stream_rows<U, true, false>(rows, RPB, D.Y16, D.Y16, D.Y16, cs_buf, stage);
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

// Weighted sum: out[s][t] = bf16(sum_k w[k] * cr[s][send_pos[k]]), fp32 fused multiply-adds in
// slot order k = 0..R-1; dropped slots (send_pos < 0) add nothing.  WW waves per token, each
// owning every WW-th group of 64 chunks; a lane keeps CU chunks (8 hidden values each) and, for
// each, up to 8 slots' loads in flight.  The launcher picks CU by the size of the call and then
// the fewest waves that cover the row in one pass (at most 16 waves at one chunk per lane, at
// most 4 at four), so that short rows leave no wave idle.  Four chunks per lane over four waves
// (a 7168-wide row in one pass) beat one chunk per lane over fourteen waves by 10-12% on the
// full-size decode layers with the memory-side cache flushed before each call (equal without):
// fewer, longer-lived waves pay the per-token table loads once for four chunks, at the same
// loads in flight per SIMD (179 VGPRs, two waves per SIMD).  A call on one rank's 128 tokens has
// too few of those waves to fill the GPU (8.0 against 11.3 us), so calls that would launch fewer
// than MOE_WSUM_WIDE_MIN_WAVES waves in the four-chunk shape keep one chunk per lane.
#ifndef MOE_WSUM_WIDE_MIN_WAVES
#define MOE_WSUM_WIDE_MIN_WAVES 4096
#endif

template <int CU>
__global__ __launch_bounds__(kBlock) void k_wsum(Dims D, int WW, const uint16_t* __restrict__ cr_buf,
                                                 const int32_t* __restrict__ send_pos,
                                                 const float* __restrict__ topk_w,
                                                 uint16_t* __restrict__ out) {
    const long gw = (long)blockIdx.x * kWavesPerBlock + wave_id();
    const long tok = gw / WW;  // within the call's ranks
    const int part = (int)(gw - tok * WW);
    if (tok >= (long)D.rc * D.T) return;
    const int lane = lane_id();
    const int R = D.R;
    const long s = tok / D.T;
    if (tok - s * D.T >= rank_tokens(D, D.rb + s)) return;  // absent token: its row is not written
    const int my_pos = lane < R ? send_pos[tok * R + lane] : -1;
    const float my_w = lane < R ? topk_w[tok * R + lane] : 0.0f;
    const u32x4* rank_rows = reinterpret_cast<const u32x4*>(cr_buf + (size_t)s * D.TR * D.H);
    u32x4* orow = reinterpret_cast<u32x4*>(out + (size_t)tok * D.H);
    const int n16 = D.Y16;
    for (int c0 = part * kWave + lane; c0 < n16; c0 += kWave * WW * CU) {
        float acc[CU][8];
#pragma unroll
        for (int cu = 0; cu < CU; ++cu)
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[cu][u] = 0.0f;
        for (int k0 = 0; k0 < R; k0 += 8) {
            u32x4 v[CU][8];
            float wk[8];
            bool ok[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int k = k0 + kk;
                const int pos = k < R ? readlane(my_pos, k) : -1;
                ok[kk] = pos >= 0 && pos < D.TR;
                wk[kk] = k < R ? readlane_f(my_w, k) : 0.0f;
#pragma unroll
                for (int cu = 0; cu < CU; ++cu) {
                    const int c = c0 + cu * kWave * WW;
                    if (ok[kk] && c < n16) v[cu][kk] = ld_nt(rank_rows + (size_t)pos * n16 + c);
                }
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (!ok[kk]) continue;
#pragma unroll
                for (int cu = 0; cu < CU; ++cu)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float y = bf16_to_f32((v[cu][kk][u >> 1] >> (16 * (u & 1))) & 0xFFFF);
                        acc[cu][u] = __builtin_fmaf(wk[kk], y, acc[cu][u]);
                    }
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

// ------------------------------------------------------------------ copy ceiling

// A contiguous copy through the row-streaming engine: the buffer cut into rows of 256 * U chunks,
// one row per block, U chunks per thread in one pass, nontemporal loads and stores.  Not a step of
// the path: the same engine on the simplest row map, the practical ceiling the row-copy kernels are
// measured against.
template <int U>
__global__ __launch_bounds__(kBlock) void k_stream_copy(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                        long n16) {
    __shared__ RowDesc rows[1];
    __shared__ u32x4 stage[stage_len(U)];
    constexpr int ch = kBlock * U;
    const long c0 = (long)blockIdx.x * ch;
    const int n = (int)(n16 - c0 < ch ? n16 - c0 : ch);
    if (threadIdx.x == 0) {
        rows[0].src_a = rows[0].src_b = (uint64_t)(src + c0 * 16);
        rows[0].dst_a = rows[0].dst_b = (uint64_t)(dst + c0 * 16);
    }
    __syncthreads();
    // dummy: the block's own source row (n chunks), which every lane may read
    block_stream_rows<U>(rows, 1, n, n, n, src + c0 * 16, stage);
}

hipError_t launch_stream_copy(const void* src, void* dst, long bytes, hipStream_t st) {
    const long n16 = bytes / 16;
    constexpr int U = MOE_STREAM_MAX_U;
    const long blocks = (n16 + kBlock * U - 1) / (kBlock * U);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_stream_copy<U>), dim3(blocks), dim3(kBlock), 0, st, (const uint8_t*)src, (uint8_t*)dst,
                       n16);
    return hipGetLastError();
}

// ------------------------------------------------------------------ launchers

hipError_t launch_expert_stub(const Dims& D, int mode, const void* expert_x, const float* expert_scale,
                              const int32_t* expert_off, uint16_t* expert_y, hipStream_t st) {
    const long rows = recv_rows_bound(D);
    hipLaunchKernelGGL(k_expert_stub, dim3(row_blocks(D, rows, kWavesPerBlock)), dim3(kBlock),
                       (D.rc + 1) * 4, st, D, mode, (const uint8_t*)expert_x, expert_scale, expert_off,
                       expert_y);
    return hipGetLastError();
}

hipError_t launch_combine_send(const Dims& D, const uint16_t* expert_y, const int32_t* expert_rpos,
                               const int32_t* recv_off, const int32_t* send_off, uint16_t* cs_buf,
                               uint16_t* cr_buf, hipStream_t st) {
    const long rows = recv_rows_bound(D);  // rows the call's ranks received
    const StreamShape sp = stream_shape(D.Y16, MOE_CPACK_MIN_CHUNKS);
    const StreamShape sn = stream_shape(D.Y16, MOE_CNET_MIN_CHUNKS);
    // blocks stride over the rows only when the grid was capped (calls on a subset of ranks)
#define MOE_LAUNCH_S(K_, R_, U_, S_, ...)                                                            \
    hipLaunchKernelGGL((K_<R_, U_, S_>), dim3(row_blocks(D, rows, R_)), dim3(kBlock), (D.rc + 1) * 4, \
                       st, D, __VA_ARGS__);
#define MOE_LAUNCH(R_, U_)                                                                          \
    if (sp.rpb == R_ && sp.u == U_) {                                                               \
        if (row_blocks(D, rows, R_) * R_ < rows)                                                    \
            MOE_LAUNCH_S(k_combine_pack, R_, U_, true, expert_y, expert_rpos, recv_off, cs_buf)     \
        else                                                                                        \
            MOE_LAUNCH_S(k_combine_pack, R_, U_, false, expert_y, expert_rpos, recv_off, cs_buf)    \
    }
    MOE_STREAM_SHAPES(MOE_LAUNCH)
#undef MOE_LAUNCH
#define MOE_LAUNCH(R_, U_)                                                                          \
    if (sn.rpb == R_ && sn.u == U_) {                                                               \
        if (row_blocks(D, rows, R_) * R_ < rows)                                                    \
            MOE_LAUNCH_S(k_combine_net, R_, U_, true, (const uint16_t*)cs_buf, recv_off, send_off, cr_buf) \
        else                                                                                        \
            MOE_LAUNCH_S(k_combine_net, R_, U_, false, (const uint16_t*)cs_buf, recv_off, send_off, cr_buf) \
    }
    MOE_STREAM_SHAPES(MOE_LAUNCH)
#undef MOE_LAUNCH
#undef MOE_LAUNCH_S
    return hipGetLastError();
}

hipError_t launch_combine_recv(const Dims& D, const uint16_t* cr_buf, const int32_t* send_pos,
                               const float* topk_w, uint16_t* out, hipStream_t st) {
    // the tokens of ranks [rb, rb + rc)
    const long rb = D.rb;
    cr_buf += rb * D.TR * D.H;
    send_pos += rb * D.TR;
    topk_w += rb * D.T * D.R;
    out += rb * D.T * D.H;
    // waves per token covering the row in one pass at cu chunks per lane, at most max_ww
    auto waves_per_token = [&](int cu, int max_ww) {
        return (int)std::min<long>(max_ww, std::max<long>(1, (D.Y16 + cu * kWave - 1) / (cu * kWave)));
    };
    const long ntok = (long)D.rc * D.T;
    const int ww4 = waves_per_token(4, 4);
    if (ntok * ww4 >= MOE_WSUM_WIDE_MIN_WAVES) {
        const long waves = ntok * ww4;
        hipLaunchKernelGGL(k_wsum<4>, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0, st,
                           D, ww4, cr_buf, send_pos, topk_w, out);
    } else {
        const int ww1 = waves_per_token(1, 16);
        const long waves = ntok * ww1;
        hipLaunchKernelGGL(k_wsum<1>, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0, st,
                           D, ww1, cr_buf, send_pos, topk_w, out);
    }
    return hipGetLastError();
}

}  // namespace moe
