// route.hip -- top-R expert selection and softmax weights, one wave per token.
//
// [DSK] = "Lower latency and higher throughput with multi-node DeepSeek deployment",
// sections Expert Parallelism and MoE Router: each token is sent to R routed experts picked by a
// sort of the router scores that tracks the indices, and the expert outputs are summed with
// weights.  [PORT] = "Efficient and portable mixture-of-experts communication", introduction:
// the weights come from the router's probability distribution.
//
// Selection order: descending fp32 (logit + bias), ties to the lower expert id (-0 == +0).
// Each lane holds experts lane, lane+64, ... as 64-bit keys (ordered score, ~expert); R rounds
// of a wave max pick the winners.  Weights: softmax over the R selected values in fp64,
// summed in slot order and rounded once to fp32.
#include "common.cuh"

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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)x, off, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        x = o > x ? o : x;
    }
    return x;
}

template <int VPL>
__global__ __launch_bounds__(kBlock) void k_route(const float* __restrict__ logits,
                                                  const float* __restrict__ bias,
                                                  int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ topk_w, int ntok, int E,
                                                  int R) {
    const int lane = lane_id();
    const long tok = (long)blockIdx.x * kWavesPerBlock + wave_id();
    if (tok >= ntok) return;
    const float* row = logits + tok * E;

    uint64_t key[VPL];
#pragma unroll
    for (int m = 0; m < VPL; ++m) {
        int e = lane + kWave * m;
        key[m] = 0;
        if (e < E) {
            float v = bias ? row[e] + bias[e] : row[e];
            key[m] = ((uint64_t)ordered_bits(v) << 32) | (uint32_t)(~(uint32_t)e);
        }
    }

    int my_e = 0;
    float my_v = 0.0f;
    for (int k = 0; k < R; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int m = 0; m < VPL; ++m) best = key[m] > best ? key[m] : best;
        best = wave_max_u64(best);
        const int e = (int)(~(uint32_t)best);
        const float v = from_ordered_bits((uint32_t)(best >> 32));
#pragma unroll
        for (int m = 0; m < VPL; ++m)
            if (lane + kWave * m == e) key[m] = 0;  // taken
        if (lane == k) {
            my_e = e;
            my_v = v;
        }
    }

    // softmax over the selected values, shifted by the largest (slot 0), in fp64
    const double v0 = (double)readlane_f(my_v, 0);
    const double z = exp((double)my_v - v0);
    double sum = 0.0;
    for (int k = 0; k < R; ++k) {
        int lo = __builtin_amdgcn_readlane((int)(uint32_t)__double_as_longlong(z), k);
        int hi = __builtin_amdgcn_readlane((int)(uint32_t)(__double_as_longlong(z) >> 32), k);
        sum += __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
    }
    if (lane < R) {
        topk_idx[tok * R + lane] = my_e;
        topk_w[tok * R + lane] = (float)(z / sum);
    }
}

hipError_t launch_route(const Dims& D, const float* logits, const float* bias, int32_t* topk_idx,
                        float* topk_w, hipStream_t st) {
    const int ntok = D.N * D.T;
    dim3 grid((ntok + kWavesPerBlock - 1) / kWavesPerBlock), block(kBlock);
    const int vpl = (D.E + kWave - 1) / kWave;
    if (vpl <= 1)
        hipLaunchKernelGGL(k_route<1>, grid, block, 0, st, logits, bias, topk_idx, topk_w, ntok, D.E, D.R);
    else if (vpl <= 2)
        hipLaunchKernelGGL(k_route<2>, grid, block, 0, st, logits, bias, topk_idx, topk_w, ntok, D.E, D.R);
    else if (vpl <= 4)
        hipLaunchKernelGGL(k_route<4>, grid, block, 0, st, logits, bias, topk_idx, topk_w, ntok, D.E, D.R);
    else if (vpl <= 8)
        hipLaunchKernelGGL(k_route<8>, grid, block, 0, st, logits, bias, topk_idx, topk_w, ntok, D.E, D.R);
    else
        hipLaunchKernelGGL(k_route<16>, grid, block, 0, st, logits, bias, topk_idx, topk_w, ntok, D.E, D.R);
    return hipGetLastError();
}

}  // namespace moe
