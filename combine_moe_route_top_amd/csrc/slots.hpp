// slots.hpp -- per-slot helpers shared by the count kernels of the decode and prefill
// dispatches: slot validity, staging a chunk of expert ids in LDS, and stable per-key ranks
// inside a wave.
#pragma once
#include "common.hpp"

namespace moe {

// Slot (t, k) of rank s is valid if its expert id is in range and differs from the ids of the
// token's earlier slots.  Invalid slots are dropped and flagged in the status word.  `chunk`
// holds the ids of slots c0 .. c0 + n - 1 in LDS; earlier slots come from global memory.
__device__ __forceinline__ bool slot_valid(const int32_t* __restrict__ idx_s, const int* chunk,
                                           long c0, long n, long i, int R, int E, int& e) {
    e = chunk[i - c0];
    if (e < 0 || e >= E) return false;
    const long t0 = (i / R) * R;
    for (long j = t0; j < i; ++j) {
        const int o = (j >= c0 && j < c0 + n) ? chunk[j - c0] : idx_s[j];
        if (o == e) return false;
    }
    return true;
}

// Stage the ids of slots c0 .. c0 + blockDim - 1 (those below TR) into LDS; returns how many.
__device__ __forceinline__ long stage_chunk(const int32_t* __restrict__ idx_s, int* chunk, long c0, long TR) {
    const long n = min((long)blockDim.x, TR - c0);
    if ((long)threadIdx.x < n) chunk[threadIdx.x] = idx_s[c0 + threadIdx.x];
    __syncthreads();
    return n;
}

// Bits needed to hold the keys 0 .. n-1.
__device__ __forceinline__ int key_bits(int n) { return n > 1 ? 32 - __clz(n - 1) : 0; }

// The active lanes of the wave whose key equals this lane's (keys in [0, 2^nbits)), found in
// constant time with one ballot per key bit (the ballot form of a multisplit): a lane keeps the
// lanes that agree with it on every bit.
__device__ __forceinline__ uint64_t same_key_lanes(bool active, int key, int nbits) {
    uint64_t same = ballot(active);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = ballot(bit);
        same &= bit ? ones : ~ones;
    }
    return same;
}

// Stable rank of this lane's key among the active lanes of the wave with the same key (lower
// lanes first); the lowest lane of each key group also stores the group's size in cnt_row[key].
__device__ __forceinline__ int wave_key_rank(bool active, int key, int nbits, int* cnt_row) {
    const uint64_t same = same_key_lanes(active, key, nbits);
    const uint64_t lower = same & lanemask_lt();
    if (active && lower == 0) cnt_row[key] = __popcll(same);
    return __popcll(lower);
}

// Exclusive running sums down a column of W <= 16 LDS entries col[0], col[stride], ...,
// starting at `start`, written in place; returns start plus the column's total.  Every load is
// issued before the first store.
__device__ __forceinline__ int column_excl_scan(int* col, int stride, int W, int start) {
    int x[16];
#pragma unroll
    for (int ww = 0; ww < 16; ++ww) x[ww] = ww < W ? col[ww * stride] : 0;
    int run = start;
#pragma unroll
    for (int ww = 0; ww < 16; ++ww) {
        if (ww < W) col[ww * stride] = run;
        run += x[ww];
    }
    return run;
}

}  // namespace moe
