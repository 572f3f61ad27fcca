// Per-batch MoE-LoRA metadata (SGLang PR #24160 page, on sharing the MoE LoRA
// batch info, section 实现拆解 items 1-3): token_lora_mapping expands each request's
// slot over its segment; adapter_enabled marks slots named by some request whose
// rank is > 0 (-1 entries are masked before the scatter, as the page's review
// section asks).
//
// One launch, token-parallel: each thread binary-searches seg_indptr for the
// request that owns its token, so coverage never depends on a max-length hint.
// Workgroup 0 additionally builds adapter_enabled through an LDS flag array.
#include "common.hpp"
#include "kernels.hpp"

namespace moelora {

static constexpr int kInfoThreads = 256;
static constexpr int kInfoFlagSlots = 8192;  // slots handled per LDS pass

__global__ void __launch_bounds__(kInfoThreads)
info_kernel(int32_t num_tokens, int32_t num_reqs, int32_t num_loras,
            const int32_t* __restrict__ seg_indptr, const int32_t* __restrict__ weight_indices,
            const int32_t* __restrict__ lora_ranks, int32_t* __restrict__ adapter_enabled,
            int32_t* __restrict__ token_lora_mapping) {
  const int t = blockIdx.x * kInfoThreads + threadIdx.x;
  if (t < num_tokens) {
    // last b with seg_indptr[b] <= t (empty segments are skipped naturally)
    int lo = 0, hi = num_reqs;  // answer in [lo, hi)
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (seg_indptr[mid] <= t) lo = mid; else hi = mid;
    }
    token_lora_mapping[t] = weight_indices[lo];
  }

  if (blockIdx.x != 0) return;
  __shared__ int32_t used[kInfoFlagSlots];
  for (int base = 0; base < num_loras; base += kInfoFlagSlots) {
    const int n = min(kInfoFlagSlots, num_loras - base);
    for (int i = threadIdx.x; i < n; i += kInfoThreads) used[i] = 0;
    __syncthreads();
    for (int b = threadIdx.x; b < num_reqs; b += kInfoThreads) {
      int slot = weight_indices[b] - base;
      if (slot >= 0 && slot < n) used[slot] = 1;   // benign same-value race
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kInfoThreads)
      adapter_enabled[base + i] = (used[i] && lora_ranks[base + i] > 0) ? 1 : 0;
    __syncthreads();
  }
}

hipError_t launch_info(int32_t num_tokens, int32_t num_reqs, int32_t num_loras,
                       const int32_t* seg_indptr, const int32_t* weight_indices,
                       const int32_t* lora_ranks, int32_t* adapter_enabled,
                       int32_t* token_lora_mapping, hipStream_t stream) {
  int blocks = (int)ceil_div(num_tokens > 0 ? num_tokens : 1, kInfoThreads);
  hipLaunchKernelGGL(info_kernel, dim3(blocks), dim3(kInfoThreads), 0, stream, num_tokens,
                     num_reqs, num_loras, seg_indptr, weight_indices, lora_ranks,
                     adapter_enabled, token_lora_mapping);
  return hipGetLastError();
}

}  // namespace moelora
