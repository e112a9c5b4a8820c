// common.cuh -- shared device helpers for the libmoe kernels (gfx950, wave64).
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
    int fp8;
    int TR;            // T * R: rows each rank sends
    long long B;       // receive-side rows per rank
    int P;             // bytes of one dispatched row
    int P16;           // P / 16
    int X16;           // payload part of a row in 16-byte chunks (2H/16 or H/16)
    int nsc;           // fp8 scales per token (H / 128)
    int Y16;           // a bf16 combine row in 16-byte chunks (2H / 16)
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

// ------------------------------------------------------------------ 16-byte row copies

// Copy n16 chunks of 16 bytes from a row made of two parts (src_a: the first split_src chunks,
// src_b: the rest) to a row made of two parts (dst_a: first split_dst chunks, dst_b: the rest).
// One wave; each lane moves chunks lane, lane+64, ...; U loads are issued before their stores.
template <int U>
__device__ __forceinline__ void wave_copy_row(const u32x4* __restrict__ src_a,
                                              const u32x4* __restrict__ src_b, int split_src,
                                              u32x4* __restrict__ dst_a, u32x4* __restrict__ dst_b,
                                              int split_dst, int n16) {
    const int l = lane_id();
    for (int c0 = 0; c0 < n16; c0 += kWave * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = c0 + u * kWave + l;
            if (c < n16) v[u] = c < split_src ? src_a[c] : src_b[c - split_src];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = c0 + u * kWave + l;
            if (c < n16) {
                if (c < split_dst) dst_a[c] = v[u];
                else dst_b[c - split_dst] = v[u];
            }
        }
    }
}

template <int U>
__device__ __forceinline__ void wave_copy_row(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                              int n16) {
    const int l = lane_id();
    for (int c0 = 0; c0 < n16; c0 += kWave * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = c0 + u * kWave + l;
            if (c < n16) v[u] = src[c];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = c0 + u * kWave + l;
            if (c < n16) dst[c] = v[u];
        }
    }
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
