// Router step before the layer: per token, the top_k experts of largest
// softmax probability (descending, ties to the lower expert id) and their
// probabilities renormalised over the k.  The layer configs of the pages'
// workloads define the router as softmax, top-k, renormalised; the tie rule
// and the descending order are this library's reading.
//
// One thread per token.  Softmax is strictly increasing in the logit, so the
// ranking is taken on the logits themselves (exact fp32 input values), and in
// the renormalised weight the softmax normaliser cancels:
//   w_j = exp(l_j - m) / sum_{i in top-k} exp(l_i - m),  m = the largest logit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace moelora {

static constexpr int kRouteMaxK = 16;

// (v1, i1) ranks before (v2, i2): larger logit, or equal logit and lower id
__device__ __forceinline__ bool ranks_before(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__global__ void __launch_bounds__(256)
route_kernel(int32_t T, int32_t E, int32_t k, const float* __restrict__ logits,
             int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  // the k best so far, sorted by ranks_before; unused entries rank last
  float tv[kRouteMaxK];
  int ti[kRouteMaxK];
#pragma unroll
  for (int j = 0; j < kRouteMaxK; ++j) {
    tv[j] = -INFINITY;
    ti[j] = INT32_MAX;
  }
  const float* row = logits + t * E;
  for (int e = 0; e < E; ++e) {
    float v = row[e];
    int id = e;
    // insertion by one bubbling pass over the (compile-time sized) list:
    // the candidate swaps with every entry it ranks before, so the entries
    // it passes move down one place and the last one falls off
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j) {
      if (j < k && ranks_before(v, id, tv[j], ti[j])) {
        const float sv = tv[j];
        const int si = ti[j];
        tv[j] = v;
        ti[j] = id;
        v = sv;
        id = si;
      }
    }
  }
  const float m = tv[0];
  float ex[kRouteMaxK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kRouteMaxK; ++j) {
    ex[j] = j < k ? expf(tv[j] - m) : 0.0f;
    sum += ex[j];
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int j = 0; j < kRouteMaxK; ++j) {
    if (j < k) {
      topk_ids[t * k + j] = ti[j];
      topk_weights[t * k + j] = ex[j] * inv;
    }
  }
}

int route_max_k() { return kRouteMaxK; }

hipError_t launch_route(int32_t T, int32_t E, int32_t k, const float* logits, int32_t* topk_ids,
                        float* topk_weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream, T, E,
                     k, logits, topk_ids, topk_weights);
  return hipGetLastError();
}

}  // namespace moelora
