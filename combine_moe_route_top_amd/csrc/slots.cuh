// slots.cuh -- per-slot helpers shared by the count kernels of the decode and prefill
// dispatches: slot validity, staging a chunk of expert ids in LDS, and stable per-key ranks
// inside a wave.
#pragma once
#include "common.cuh"

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

}  // namespace moe
