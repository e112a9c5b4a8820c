// common.hpp -- shared device helpers for the libmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 256;               // 4 waves per workgroup for the row kernels
constexpr int kWavesPerBlock = kBlock / kWave;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Everything a kernel needs to know about the problem, passed by value.
struct Dims {
    int N, T, H, E, R, L;
    int fp8;           // e4m3 payload rows (codes, then fp32 block scales)
    int quant;         // the send pack makes those rows from bf16 tokens
    const int32_t* tok;  // device int32[N]: tokens each rank dispatches, or NULL (T for all)
    int prefill;       // replicated tokens: the same T tokens on every rank
    int TR;            // T * R: rows each rank sends
    long long B;       // receive-side rows per rank
    int P;             // bytes of one dispatched row
    int P16;           // P / 16
    int X16;           // payload part of a row in 16-byte chunks (2H/16 or H/16)
    int nsc;           // fp8 scales per token (H / 128)
    int Y16;           // a bf16 combine row in 16-byte chunks (2H / 16)
    int rb, rc;        // ranks this call works for: [rb, rb + rc)
    int32_t* status;
};

// ------------------------------------------------------------------ wave primitives

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int readlane(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
    int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off, kWave);
        if (l >= off) v += o;
    }
    return v;
}

__device__ __forceinline__ void set_status(int32_t* status, int code) {
    if (status) atomicCAS(status, 0, code);
}

// Tokens rank s (a global rank) dispatches: T, or the caller's per-rank count; a count outside
// [0, T] flags MOE_EINVAL and counts as 0.
__device__ __forceinline__ int rank_tokens(const Dims& D, long s) {
    if (!D.tok) return D.T;
    const int v = D.tok[s];
    if (v < 0 || v > D.T) {
        set_status(D.status, MOE_EINVAL);
        return 0;
    }
    return v;
}

// Exclusive scan of n ints (n <= a few thousand) done by one wave, in place from `in` to
// `out[0..n]` (out[n] = total).  Both may live in LDS or global memory.  Only wave `w` of the
// block executes it; the caller synchronises afterwards.
__device__ __forceinline__ void wave_excl_scan_array(const int* in, int* out, int n) {
    int carry = 0;
    for (int base = 0; base < n; base += kWave) {
        int i = base + lane_id();
        int v = i < n ? in[i] : 0;
        int inc = wave_incl_scan(v);
        if (i < n) out[i] = carry + inc - v;
        carry += readlane(inc, kWave - 1);
    }
    if (lane_id() == 0) out[n] = carry;
}

// Number of entries of the non-decreasing array a[0..n) that are <= x (a wave-wide count,
// uniform across the wave).  Used to find which segment of an offset table a row falls in.
__device__ __forceinline__ int wave_count_le(const int* a, int n, long long x) {
    int c = 0;
    for (int base = 0; base < n; base += kWave) {
        int i = base + lane_id();
        bool p = i < n && (long long)a[i] <= x;
        c += __popcll(ballot(p));
    }
    return c;
}

// Sum of an int over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// At most how many rows the call's ranks receive in total: every rank receives at most
// S*T*min(R, L) rows (one per routed slot, distinct experts per token) from the S token sets
// (N sources; one replicated set for prefill), and all ranks together exactly the S*T*R routed
// rows.
inline long recv_rows_bound(const Dims& D) {
    const long S = D.prefill ? 1 : D.N;
    const long per_rank = S * D.T * (D.R < D.L ? D.R : D.L);
    const long all = S * D.TR;
    const long b = (long)D.rc * per_rank;
    return b < all ? b : all;
}

// Blocks for a row kernel whose rows are only known on the device: one block per RPB rows of
// the bound when the call covers all ranks, at most kSubrangeBlocks when it covers a subset (most
// of the bound is usually empty; blocks then stride over the rows).  With per-rank token counts
// part of an all-rank bound is empty too; the blocks past the call's rows return before they
// resolve or stream anything, which leaves them only their launch (letting them stream their dead
// rows' dummy loads cost the ragged DeepSeek-V3 mix, tokens uniform on 1..T, 96 against 84 us in
// the unpack and 228 against 206 us in the combine).  Halving the grid for calls with token counts
// gained 8 us more there but cost calls whose ranks all send T tokens as much, so the grid stays.
#ifndef MOE_SUBRANGE_BLOCKS
#define MOE_SUBRANGE_BLOCKS 4096
#endif
constexpr long kSubrangeBlocks = MOE_SUBRANGE_BLOCKS;
inline long row_blocks(const Dims& D, long rows_bound, int rpb) {
    long b = (rows_bound + rpb - 1) / rpb;
    if (D.rc < D.N && b > kSubrangeBlocks) b = kSubrangeBlocks;
    return b > D.rc ? b : D.rc;
}

// The routed rows of a whole exchange (N token sets of T*R rows) fit in the 256 MB memory-side
// cache: the network kernel then stores them cached and the unpack reads them cached, so they need
// not travel to HBM and back between the two (e4m3 DeepSeek-V3 rows: 242 MB).
constexpr long kMallBytes = 256L << 20;
inline bool exchange_fits_mall(const Dims& D) { return (long)D.N * D.TR * D.P <= kMallBytes; }

// ------------------------------------------------------------------ block row streaming

// Nontemporal 16-byte accesses: streamed data does not stay in the caches, and the stores do not
// leave dirty lines in the 256 MB memory-side cache for the next kernel to write back.
__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// The same through global-address-space pointers: the compiler then emits global_ (not flat_)
// instructions, which it does not also count against the LDS counter.
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
__device__ __forceinline__ const g_u32x4* as_global(const void* p) { return (const g_u32x4*)p; }
__device__ __forceinline__ g_u32x4* as_global(void* p) { return (g_u32x4*)p; }
template <bool NT>
__device__ __forceinline__ u32x4 ld_g(const g_u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st_g(g_u32x4* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// A row-copy kernel block (256 threads) handles RPB consecutive rows of its source: one row is
// resolved per wave (its source and destination found), then all 256 threads stream the rows'
// 16-byte chunks, U per thread per pass.  Launchers pick (RPB, U) from the row size.

// A resolved row: the source is src_a (its first split_src chunks) then src_b; the destination
// dst_a (first split_dst chunks) then dst_b.  dst_a == 0 marks "no row".
struct RowDesc {
    uint64_t src_a, src_b, dst_a, dst_b;
};

// 1: row chunks pass through LDS: each load is a gfx950 direct-to-LDS load
// (global_load_lds_dwordx4: 16 bytes per lane from memory into LDS without a register round trip),
// then each thread reads its own chunks back and stores them.  0 (the default): every load goes
// into registers, then the stores.  Timed in one process on the same buffers, the LDS path made the
// dispatch network kernel alone 13% faster on bf16 rows (4 chunks per thread, two passes) but left
// every kernel of a whole layer within a few microseconds of the register path, so the register
// path stays; the LDS path is kept as a build option (MOE_STREAM_LDS=1 MOE_STREAM_MAX_U=4).
#ifndef MOE_STREAM_LDS
#define MOE_STREAM_LDS 0
#endif
// Most chunks per thread per pass (the LDS path holds U * 4 KB of LDS per block).
#ifndef MOE_STREAM_MAX_U
#define MOE_STREAM_MAX_U 8
#endif

// LDS a streaming block of `threads` threads declares for U chunks per thread:
// __shared__ u32x4 stage[stage_len(U, threads)].
constexpr int stage_len(int U, int threads = kBlock) { return MOE_STREAM_LDS ? U * threads : 1; }

typedef __attribute__((address_space(3))) void lds_void;

// Stream nrows resolved rows of n16 chunks each, flat over (row, chunk).  NTLD / NTST: nontemporal
// loads / stores (the default); cached ones where the rows should stay in the memory-side cache
// for the next kernel.  `dummy` points at n16 readable chunks (the first row of the source
// buffer): a lane past the block's chunks, or on a row that did not resolve (dst_a == 0), loads
// from there and stores nothing, so that every load is unconditional.  With loads under the
// per-lane test instead, the compiler could not tell which loads were still in flight and waited
// for each load before issuing the next.  `stage`: stage_len(U, blockDim.x) chunks of LDS.  In the
// LDS path lane l of wave w lands chunk u of a pass at stage[u * blockDim.x + w * 64 + l], the slot
// its own thread reads back, so no barrier is needed; a pass reads every chunk back before the next
// pass loads over them.
template <int U, bool NTLD = true, bool NTST = true>
__device__ __forceinline__ void block_stream_rows(const RowDesc* rows, int nrows, int n16, int split_src,
                                                  int split_dst, const void* dummy, u32x4* stage) {
    const int total = nrows * n16;
    const float inv = 1.0f / (float)n16;
    for (int k0 = threadIdx.x; k0 < total; k0 += blockDim.x * U) {
        u32x4 v[U];
        int rr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + u * blockDim.x;
            const int kc = k < total ? k : total - 1;
            int r = (int)((float)kc * inv);  // kc / n16, corrected below (kc < 2^24)
            if (r * n16 > kc) --r;
            else if ((r + 1) * n16 <= kc) ++r;
            rr[u] = r;
            const int c = kc - r * n16;
            const bool live = k < total && rows[r].dst_a;
            const g_u32x4* src = !live ? as_global(dummy) + c
                                 : c < split_src ? as_global((const void*)rows[r].src_a) + c
                                                 : as_global((const void*)rows[r].src_b) + (c - split_src);
            if constexpr (MOE_STREAM_LDS)
                __builtin_amdgcn_global_load_lds((const void*)src,
                                                 (lds_void*)(stage + u * blockDim.x + wave_id() * kWave), 16, 0,
                                                 NTLD ? 2 : 0);  // 2: nontemporal
            else
                v[u] = ld_g<NTLD>(src);
        }
        if constexpr (MOE_STREAM_LDS) {
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = stage[u * blockDim.x + threadIdx.x];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + u * blockDim.x;
            const int r = rr[u];
            if (k < total && rows[r].dst_a) {
                const int c = k - r * n16;
                g_u32x4* dst = c < split_dst ? as_global((void*)rows[r].dst_a) + c
                                             : as_global((void*)rows[r].dst_b) + (c - split_dst);
                st_g<NTST>(dst, v[u]);
            }
        }
    }
}

// (rows per block, chunks per thread per pass) for rows of n16 chunks: the fewest rows (1, 2 or 4)
// whose chunks reach min_chunks -- enough bytes per block to hide the row-resolve latency -- and
// the fewest chunks per thread (at most MOE_STREAM_MAX_U) that cover them in one pass; rows
// longer than that take several passes.
struct StreamShape {
    int rpb, u;
};
inline StreamShape stream_shape(int n16, int min_chunks) {
    int rpb = 1;
    while (rpb < kWavesPerBlock && rpb * n16 < min_chunks) rpb *= 2;
    const int per_thread = (rpb * n16 + kBlock - 1) / kBlock;
    int u = 1;
    while (u < per_thread && u < MOE_STREAM_MAX_U) u *= 2;
    return {rpb, u};
}

// Minimum chunks per block, per kernel (a row-resolve costs 2-4 dependent memory round trips;
// the unpack's, with its expert-base reduction, is the heaviest).
#ifndef MOE_NET_MIN_CHUNKS
#define MOE_NET_MIN_CHUNKS 1792
#endif
#ifndef MOE_UNPACK_MIN_CHUNKS
#define MOE_UNPACK_MIN_CHUNKS 1792
#endif
#ifndef MOE_CPACK_MIN_CHUNKS
#define MOE_CPACK_MIN_CHUNKS 896
#endif
#ifndef MOE_CNET_MIN_CHUNKS
#define MOE_CNET_MIN_CHUNKS 896
#endif

// The (RPB, U) instances a launcher may pick.
#define MOE_STREAM_SHAPES(X) \
    X(1, 1) X(1, 2) X(1, 4) X(1, 8) X(2, 1) X(2, 2) X(2, 4) X(2, 8) X(4, 1) X(4, 2) X(4, 4) X(4, 8)

// Global row bases over ranks, gb[d] = sum over d' < d of table[d' * stride + col], gb[N] = the
// total; computed by wave 0 into LDS (the caller synchronises).
__device__ __forceinline__ void rank_bases(const int32_t* table, int stride, int col, int N, int* gb) {
    if (wave_id() != 0) return;
    int carry = 0;
    for (int b = 0; b < N; b += kWave) {
        const int dd = b + lane_id();
        const int v = dd < N ? table[(long)dd * stride + col] : 0;
        const int inc = wave_incl_scan(v);
        if (dd < N) gb[dd] = carry + inc - v;
        carry += readlane(inc, kWave - 1);
    }
    if (lane_id() == 0) gb[N] = carry;
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

}  // namespace moe
