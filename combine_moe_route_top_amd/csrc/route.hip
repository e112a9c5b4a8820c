// route.hip -- top-R expert selection and softmax weights, one lane group per token.
//
// [DSK] = "Lower latency and higher throughput with multi-node DeepSeek deployment",
// sections Expert Parallelism and MoE Router: each token is sent to R routed experts picked by a
// sort of the router scores that tracks the indices, and the expert outputs are summed with
// weights.  [PORT] = "Efficient and portable mixture-of-experts communication", introduction:
// the weights come from the router's probability distribution.
//
// Selection order: descending fp32 (logit + bias), ties to the lower expert id (-0 == +0).
// A group of G lanes (16, 32 or 64; 64/G tokens per wave) holds a token's experts
// gl, gl+G, ... as order-preserving score bits.  Each of the R rounds takes the lane's best
// (score, lowest id) as a 64-bit key (score bits, ~expert id), then a group max: DPP row
// rotations by 1, 2, 4, 8 inside each 16-lane row (plain VALU moves, no LDS crossbar), and for
// G > 16 one or two lane swaps across rows.  Weights: softmax over the R selected values in fp64, summed in slot order, rounded
// once to fp32.
#include "common.hpp"

// Waves below which the launcher gives each token a wider lane group; overridable at build time
// for launch-shape experiments.
#ifndef MOE_ROUTE_MIN_WAVES
#define MOE_ROUTE_MIN_WAVES 1024
#endif

namespace moe {

// Order-preserving map of a float to uint32 (after -0 is folded into +0).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// DPP row_ror:n (rotate inside each 16-lane row), n = 1..15: control 0x120 + n.
template <int N>
__device__ __forceinline__ uint64_t row_ror_u64(uint64_t x) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, 0x120 + N, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), 0x120 + N, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = __shfl_xor((uint32_t)x, m, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// Max over each group of G consecutive lanes; every lane of the group gets it.
template <int G>
__device__ __forceinline__ uint64_t group_max(uint64_t x) {
    x = umax64(x, row_ror_u64<1>(x));
    x = umax64(x, row_ror_u64<2>(x));
    x = umax64(x, row_ror_u64<4>(x));
    x = umax64(x, row_ror_u64<8>(x));
    if constexpr (G >= 32) x = umax64(x, shfl_xor_u64(x, 16));
    if constexpr (G >= 64) x = umax64(x, shfl_xor_u64(x, 32));
    return x;
}

template <int G, int VPL>
__global__ __launch_bounds__(kBlock) void k_route(const float* __restrict__ logits,
                                                  const float* __restrict__ bias,
                                                  int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ topk_w, Dims D) {
    constexpr int TPW = kWave / G;  // tokens per wave
    const int E = D.E, R = D.R;
    const int lane = lane_id();
    const int grp = lane / G, gl = lane % G;
    const long tok = ((long)blockIdx.x * kWavesPerBlock + wave_id()) * TPW + grp;  // call's ranks
    const long s = tok / D.T;
    // tokens past their rank's count take no part
    const bool active = tok < (long)D.rc * D.T && tok - s * D.T < rank_tokens(D, D.rb + s);
    // a wave with no token leaves; otherwise every lane takes part in the DPP rotations and
    // lane swaps
    if (ballot(active) == 0) return;
    const float* row = logits + (active ? tok : 0) * E;

    // ordered scores; 0 marks "taken" or "no expert" (every finite score maps above 0).  Within a
    // lane the expert id grows with m, so a strict '>' scan keeps the lower id on ties.
    // Loads are unconditional (indices clamped into the row) so that they all issue together.
    float lv[VPL];
#pragma unroll
    for (int m = 0; m < VPL; ++m) lv[m] = row[min(gl + G * m, E - 1)];
    if (bias) {
#pragma unroll
        for (int m = 0; m < VPL; ++m) lv[m] += bias[min(gl + G * m, E - 1)];
    }
    uint32_t sc[VPL];
#pragma unroll
    for (int m = 0; m < VPL; ++m) sc[m] = (active && gl + G * m < E) ? ordered_bits(lv[m]) : 0u;

    int my_e = 0;
    float my_v = 0.0f;
#pragma unroll 1
    for (int k = 0; k < R; ++k) {
        uint32_t bs = 0;
        int bm = 0;
#pragma unroll
        for (int m = 0; m < VPL; ++m)
            if (sc[m] > bs) {
                bs = sc[m];
                bm = m;
            }
        uint64_t best = bs ? (((uint64_t)bs << 32) | (uint32_t)(~(uint32_t)(gl + G * bm))) : 0;
        best = group_max<G>(best);
        const int e = (int)(~(uint32_t)best);
        const float v = from_ordered_bits((uint32_t)(best >> 32));
#pragma unroll
        for (int m = 0; m < VPL; ++m)
            if (gl + G * m == e) sc[m] = 0;  // taken
        if (gl == k) {
            my_e = e;
            my_v = v;
        }
    }

    // softmax over the group's R selected values, shifted by the largest (slot 0), in fp64: lane
    // k of the group forms slot k's term, and every lane sums the terms in slot order
    const int base = grp * G;
    const double v0 = (double)__shfl(my_v, base, kWave);
    const double z = exp((double)my_v - v0);
    double sum = 0.0;
    for (int j = 0; j < R; ++j) sum += __shfl(z, base + j, kWave);
    if (active && gl < R) {
        topk_idx[tok * R + gl] = my_e;
        topk_w[tok * R + gl] = (float)(z / sum);
    }
}

template <int G>
static void launch_g(int vpl, dim3 grid, hipStream_t st, const float* logits, const float* bias,
                     int32_t* topk_idx, float* topk_w, const Dims& D) {
    if (vpl <= 1)
        hipLaunchKernelGGL((k_route<G, 1>), grid, dim3(kBlock), 0, st, logits, bias, topk_idx, topk_w, D);
    else if (vpl <= 2)
        hipLaunchKernelGGL((k_route<G, 2>), grid, dim3(kBlock), 0, st, logits, bias, topk_idx, topk_w, D);
    else if (vpl <= 4)
        hipLaunchKernelGGL((k_route<G, 4>), grid, dim3(kBlock), 0, st, logits, bias, topk_idx, topk_w, D);
    else if (vpl <= 8)
        hipLaunchKernelGGL((k_route<G, 8>), grid, dim3(kBlock), 0, st, logits, bias, topk_idx, topk_w, D);
    else
        hipLaunchKernelGGL((k_route<G, 16>), grid, dim3(kBlock), 0, st, logits, bias, topk_idx, topk_w, D);
}

hipError_t launch_route(const Dims& D0, const float* logits, const float* bias, int32_t* topk_idx,
                        float* topk_w, hipStream_t st) {
    // replicated tokens (prefill): one token set of T, routed once whatever the rank range
    Dims D = D0;
    if (D.prefill) {
        D.rb = 0;
        D.rc = 1;
    }
    // the tokens of ranks [rb, rb + rc)
    const long t0 = (long)D.rb * D.T;
    const int ntok = D.rc * D.T;
    logits += t0 * D.E;
    topk_idx += t0 * D.R;
    topk_w += t0 * D.R;
    // the smallest group with at most 16 experts per lane and at least R lanes, widened while
    // the call has fewer than MOE_ROUTE_MIN_WAVES waves (fewer experts per lane, shorter rounds)
    int G = 16;
    while (G < 64 && (D.E > 16 * G || D.R > G)) G *= 2;
    while (G < 64 && (long)ntok * G < (long)MOE_ROUTE_MIN_WAVES * kWave) G *= 2;
    const int vpl = (D.E + G - 1) / G;
    const long waves = ((long)ntok * G + kWave - 1) / kWave;
    const dim3 grid((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    if (G == 16) launch_g<16>(vpl, grid, st, logits, bias, topk_idx, topk_w, D);
    else if (G == 32) launch_g<32>(vpl, grid, st, logits, bias, topk_idx, topk_w, D);
    else launch_g<64>(vpl, grid, st, logits, bias, topk_idx, topk_w, D);
    return hipGetLastError();
}

}  // namespace moe
