// Per-batch MoE-LoRA metadata (SGLang PR #24160 page, on sharing the MoE LoRA
// batch info, section 实现拆解 items 1-3): token_lora_mapping expands each request's
// slot over its segment; adapter_enabled marks slots named by some request whose
// rank is > 0 (-1 entries are masked before the scatter, as the page's review
// section asks).
//
// One launch, token-parallel: each thread binary-searches seg_indptr for the
// request that owns its token, so coverage never depends on a max-length hint.
// Workgroup 0 additionally builds adapter_enabled through an LDS flag array.
#include "moe_lora.h"
#include "common.hpp"
#include "kernels.hpp"

namespace moelora {

static constexpr int kInfoThreads = 256;
static constexpr int kInfoFlagSlots = 8192;  // slots handled per LDS pass

__global__ void __launch_bounds__(kInfoThreads)
info_kernel(int32_t num_tokens, int32_t num_reqs, int32_t num_loras,
            const int32_t* __restrict__ seg_indptr, const int32_t* __restrict__ weight_indices,
            const int32_t* __restrict__ lora_ranks, int32_t* __restrict__ adapter_enabled,
            int32_t* __restrict__ token_lora_mapping, uint32_t* __restrict__ dbg) {
  const int t = blockIdx.x * kInfoThreads + threadIdx.x;
#ifdef MOE_LORA_DEBUG
  // preconditions: seg_indptr starts at 0, is nondecreasing and ends at
  // num_tokens; weight_indices in [-1, num_loras); lora_ranks >= 0
  for (int64_t i = t; i <= (int64_t)max(num_reqs, num_loras); i += (int64_t)gridDim.x * kInfoThreads) {
    if (i < num_reqs) {
      const int32_t a = seg_indptr[i], b = seg_indptr[i + 1];
      if (b < a || (i == 0 && a != 0) || (i == num_reqs - 1 && b != num_tokens))
        debug_flag(dbg, MOE_LORA_DEBUG_SEG_INDPTR);
      const int32_t wi = weight_indices[i];
      if (wi < -1 || wi >= num_loras) debug_flag(dbg, MOE_LORA_DEBUG_WEIGHT_INDEX);
    }
    if (i == 0 && num_reqs == 0 && (seg_indptr[0] != 0 || num_tokens != 0))
      debug_flag(dbg, MOE_LORA_DEBUG_SEG_INDPTR);
    if (i < num_loras && lora_ranks[i] < 0) debug_flag(dbg, MOE_LORA_DEBUG_RANK);
  }
#endif
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
                       int32_t* token_lora_mapping, uint32_t* debug_word, hipStream_t stream) {
  int blocks = (int)ceil_div(num_tokens > 0 ? num_tokens : 1, kInfoThreads);
  hipLaunchKernelGGL(info_kernel, dim3(blocks), dim3(kInfoThreads), 0, stream, num_tokens,
                     num_reqs, num_loras, seg_indptr, weight_indices, lora_ranks,
                     adapter_enabled, token_lora_mapping, debug_word);
  return hipGetLastError();
}

#ifdef MOE_LORA_DEBUG
// the precondition flag word of debug builds (one per device)
__device__ uint32_t g_debug_flags;

uint32_t* debug_word() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_flags)) != hipSuccess) return nullptr;
  return static_cast<uint32_t*>(p);
}

hipError_t debug_word_read(uint32_t* flags, bool clear, hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_debug_flags), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &zero, sizeof(uint32_t), 0, hipMemcpyHostToDevice);
}
#else
uint32_t* debug_word() { return nullptr; }
hipError_t debug_word_read(uint32_t* flags, bool, hipStream_t) {
  *flags = 0;
  return hipErrorNotSupported;
}
#endif

}  // namespace moelora
