// Router step before the layer: per token, the top_k experts of largest
// softmax probability (descending, ties to the lower expert id) and their
// probabilities renormalised over the k.  None of the MoE-LoRA pages describes
// a router: the layer configurations this library is measured on define it as
// softmax over the experts, top-k, renormalised; the tie rule and the
// descending order are this library's reading.
//
// Softmax is strictly increasing in the logit, so the ranking is taken on the
// logits themselves (exact fp32 input values), and in the renormalised weight
// the softmax normaliser cancels:
//   w_j = exp(l_j - m) / sum_{i in top-k} exp(l_i - m),  m = the largest logit.
//
// One wave per token.  Lane c holds the experts c, c + 64, c + 128, ... of the
// row (in registers when E <= 64 V).  The order "larger logit, or equal logit
// and lower id" is total, so the k winners come out of k rounds of a wave-wide
// arg-best: every lane offers its best expert not yet taken, a butterfly of
// shuffles picks the best offer, and only the lane that gave it looks for its
// next one.  A lane's experts leave in its own rank order, so its next offer
// is its best expert ranking after the one just taken: no taken-set is kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace moelora {

static constexpr int kRouteMaxK = 16;
static constexpr int kRouteWaves = 4;   // waves (tokens in flight) per workgroup

// (v1, i1) ranks before (v2, i2): larger logit, or equal logit and lower id
__device__ __forceinline__ bool ranks_before(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// V: logits per lane kept in registers (E <= 64 V); V = 0 re-reads the row
// from memory on every scan (any E)
template <int V>
__global__ void __launch_bounds__(64 * kRouteWaves)
route_kernel(int32_t T, int32_t E, int32_t k, const float* __restrict__ logits,
             int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights) {
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kRouteWaves;
  const int nper = E > lane ? (E - lane + 63) / 64 : 0;   // experts of this lane
  for (int64_t t = wave0; t < T; t += nwaves) {
    const float* row = logits + t * E;
    float cache[V > 0 ? V : 1];
    if constexpr (V > 0) {
#pragma unroll
      for (int i = 0; i < V; ++i) cache[i] = i < nper ? row[lane + 64 * i] : 0.0f;
    }
    auto logit = [&](int i) -> float {
      if constexpr (V > 0) return cache[i];
      else return row[lane + 64 * i];
    };
    // best expert of this lane ranking after (tv, ti) (after nothing when
    // ti < 0); none: (-inf, INT32_MAX), which every real expert ranks before
    auto lane_best = [&](float tv, int ti, float& bv, int& bi) {
      bv = -INFINITY;
      bi = INT32_MAX;
      auto consider = [&](int i) {
        const float x = logit(i);
        const int id = lane + 64 * i;
        if (ti >= 0 && !ranks_before(tv, ti, x, id)) return;
        if (ranks_before(x, id, bv, bi)) {
          bv = x;
          bi = id;
        }
      };
      if constexpr (V > 0) {
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (i < nper) consider(i);
      } else {
        for (int i = 0; i < nper; ++i) consider(i);
      }
    };
    float bv;
    int bi;
    lane_best(0.0f, -1, bv, bi);
    float my_v = -INFINITY;   // lane j < k: the j-th winner
    int my_i = INT32_MAX;
    for (int j = 0; j < k; ++j) {
      float wv = bv;
      int wi = bi;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(wv, off, 64);
        const int oi = __shfl_xor(wi, off, 64);
        if (ranks_before(ov, oi, wv, wi)) {
          wv = ov;
          wi = oi;
        }
      }
      if (lane == j) {
        my_v = wv;
        my_i = wi;
      }
      if (wi != INT32_MAX && (wi & 63) == lane) lane_best(wv, wi, bv, bi);
    }
    const float m = __shfl(my_v, 0, 64);
    const float ex = lane < k ? expf(my_v - m) : 0.0f;
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __shfl(ex, j, 64);   // in rank order
    if (lane < k) {
      topk_ids[t * k + lane] = my_i;
      topk_weights[t * k + lane] = ex * (1.0f / sum);
    }
  }
}

int route_max_k() { return kRouteMaxK; }

hipError_t launch_route(int32_t T, int32_t E, int32_t k, const float* logits, int32_t* topk_ids,
                        float* topk_weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(((int64_t)T + kRouteWaves - 1) / kRouteWaves, 256 * 16);
  const dim3 grid((unsigned)blocks), block(64 * kRouteWaves);
  if (E <= 64)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, stream, T, E, k, logits, topk_ids, topk_weights);
  else if (E <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, stream, T, E, k, logits, topk_ids, topk_weights);
  else if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, stream, T, E, k, logits, topk_ids, topk_weights);
  else if (E <= 1024)
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, stream, T, E, k, logits, topk_ids, topk_weights);
  else
    hipLaunchKernelGGL(route_kernel<0>, grid, block, 0, stream, T, E, k, logits, topk_ids, topk_weights);
  return hipGetLastError();
}

}  // namespace moelora
