// C ABI of the MoE-LoRA library: host-side validation (host scalars only) and
// dispatch to the HIP launchers.  See include/moe_lora.h for the contract.
#include <cstddef>
#include "moe_lora.h"

#include <hip/hip_runtime.h>

#include "kernels.hpp"

using namespace moelora;

namespace {

constexpr int64_t kMaxKeys = 32768;  // E * (L + 1) supported by the align kernels
constexpr int64_t kMaxRank = 64;
// x [T, H] and one expert's (or the dense projection's) weight matrix must each
// stay below 4 GiB: the GEMMs address them with 32-bit byte offsets
constexpr int64_t kMaxOffsetBytes = int64_t(1) << 32;

bool bad_block_m(int32_t bm) { return bm < 16 || bm > 256 || (bm % 16) != 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_LORA_OK : MOE_LORA_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_lora_status_str(int status) {
  switch (status) {
    case MOE_LORA_OK: return "ok";
    case MOE_LORA_ERR_INVALID: return "invalid argument";
    case MOE_LORA_ERR_UNDERCOVER: return "launch under-covers tokens (num_reqs * max_seg_len < num_tokens)";
    case MOE_LORA_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case MOE_LORA_ERR_HIP: return "HIP runtime error";
    case MOE_LORA_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int moe_lora_route(int32_t num_tokens, int32_t num_experts, int32_t top_k, const float* logits,
                   int32_t* topk_ids, float* topk_weights, void* stream) {
  if (num_tokens < 0 || num_experts <= 0 || top_k <= 0 || top_k > num_experts)
    return MOE_LORA_ERR_INVALID;
  if (top_k > route_max_k()) return MOE_LORA_ERR_UNSUPPORTED;
  if (num_tokens > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_LORA_ERR_INVALID;
  return hip_status(launch_route(num_tokens, num_experts, top_k, logits, topk_ids, topk_weights,
                                 static_cast<hipStream_t>(stream)));
}

int moe_lora_info(int32_t num_tokens, int32_t num_reqs, int32_t num_loras, int32_t max_seg_len,
                  const int32_t* seg_indptr, const int32_t* weight_indices,
                  const int32_t* lora_ranks, int32_t* adapter_enabled,
                  int32_t* token_lora_mapping, void* stream) {
  if (num_tokens < 0 || num_reqs < 0 || num_loras < 0 || max_seg_len < 0) return MOE_LORA_ERR_INVALID;
  if (num_tokens > 0 && num_reqs == 0) return MOE_LORA_ERR_INVALID;
  if (max_seg_len > 0 && (int64_t)num_reqs * max_seg_len < num_tokens) return MOE_LORA_ERR_UNDERCOVER;
  if (!seg_indptr) return MOE_LORA_ERR_INVALID;
  if (num_reqs > 0 && !weight_indices) return MOE_LORA_ERR_INVALID;
  if (num_loras > 0 && (!lora_ranks || !adapter_enabled)) return MOE_LORA_ERR_INVALID;
  if (num_tokens > 0 && !token_lora_mapping) return MOE_LORA_ERR_INVALID;
  if (num_tokens == 0 && num_loras == 0) return MOE_LORA_OK;
  return hip_status(launch_info(num_tokens, num_reqs, num_loras, seg_indptr, weight_indices,
                                lora_ranks, adapter_enabled, token_lora_mapping, debug_word(),
                                static_cast<hipStream_t>(stream)));
}

int64_t moe_lora_align_capacity_rows(int32_t num_tokens, int32_t top_k, int32_t num_experts,
                                     int32_t num_loras, int32_t block_m) {
  if (num_tokens < 0 || top_k <= 0 || num_experts <= 0 || num_loras < 0 || bad_block_m(block_m))
    return -1;
  // sizes align refuses have no capacity (and P, E*(L+1) bounded here keep the
  // arithmetic below 2^40)
  const int64_t P = (int64_t)num_tokens * top_k;
  if (P > INT32_MAX / 2 || (int64_t)num_experts * ((int64_t)num_loras + 1) > kMaxKeys) return -1;
  return align_capacity(P, num_experts, num_loras, block_m);
}

size_t moe_lora_align_workspace_bytes(int32_t num_tokens, int32_t top_k, int32_t num_experts,
                                      int32_t num_loras, int32_t block_m) {
  if (moe_lora_align_capacity_rows(num_tokens, top_k, num_experts, num_loras, block_m) < 0) return 0;
  return align_ws_layout((int64_t)num_tokens * top_k, (int64_t)num_experts * ((int64_t)num_loras + 1)).bytes;
}

int moe_lora_align(int32_t num_tokens, int32_t top_k, int32_t num_experts, int32_t num_loras,
                   int32_t block_m, const int32_t* topk_ids, const int32_t* token_lora_mapping,
                   const int32_t* adapter_enabled, int32_t* sorted_pair_ids, int32_t* tile_expert,
                   int32_t* tile_lora, int32_t* expert_tile_offsets, int32_t* num_rows_padded,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (num_tokens < 0 || top_k <= 0 || num_experts <= 0 || num_loras < 0 || bad_block_m(block_m))
    return MOE_LORA_ERR_INVALID;
  if (top_k > num_experts) return MOE_LORA_ERR_INVALID;
  const int64_t P = (int64_t)num_tokens * top_k;
  if (P > INT32_MAX / 2) return MOE_LORA_ERR_UNSUPPORTED;
  if ((int64_t)num_experts * ((int64_t)num_loras + 1) > kMaxKeys) return MOE_LORA_ERR_UNSUPPORTED;
  if (!expert_tile_offsets || !num_rows_padded) return MOE_LORA_ERR_INVALID;
  if (P > 0 && (!topk_ids || !token_lora_mapping || !sorted_pair_ids || !tile_expert || !tile_lora))
    return MOE_LORA_ERR_INVALID;
  if (num_loras > 0 && !adapter_enabled) return MOE_LORA_ERR_INVALID;
  const size_t need = moe_lora_align_workspace_bytes(num_tokens, top_k, num_experts, num_loras, block_m);
  if (!workspace || workspace_bytes < need) return MOE_LORA_ERR_WORKSPACE;
  return hip_status(launch_align(num_tokens, top_k, num_experts, num_loras, block_m, topk_ids,
                                 token_lora_mapping, adapter_enabled, sorted_pair_ids, tile_expert,
                                 tile_lora, expert_tile_offsets, num_rows_padded, workspace,
                                 debug_word(), static_cast<hipStream_t>(stream)));
}

int moe_lora_debug_flags(uint32_t* flags, int32_t clear, void* stream) {
  if (!flags) return MOE_LORA_ERR_INVALID;
  *flags = 0;
  if (!debug_word()) return MOE_LORA_ERR_UNSUPPORTED;   // a release build: no checks
  return hip_status(debug_word_read(flags, clear != 0, static_cast<hipStream_t>(stream)));
}

// the kernels move activations, weights, pools and outputs in 16-byte units
static bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }

static int to_problem(const moe_lora_forward_args* a, ForwardProblem* p, bool check_ptrs) {
  // the fields up to out_dtype are required; the fp8 weight fields are read
  // when struct_size covers them
  constexpr size_t kBaseSize = offsetof(moe_lora_forward_args, out_dtype) + sizeof(int32_t);
  if (!a || a->struct_size < kBaseSize) return MOE_LORA_ERR_INVALID;
  const bool has_w = a->struct_size >= sizeof(moe_lora_forward_args);
  const int32_t wdt = has_w && a->weight_dtype != 0 ? a->weight_dtype : a->dtype;
  if (a->dtype != MOE_LORA_F32 && a->dtype != MOE_LORA_BF16) return MOE_LORA_ERR_UNSUPPORTED;
  if (a->num_tokens < 0 || a->hidden <= 0 || a->inter <= 0 || a->num_experts <= 0 ||
      a->top_k <= 0 || a->num_loras < 0 || a->max_rank < 0 || bad_block_m(a->block_m))
    return MOE_LORA_ERR_INVALID;
  if (a->top_k > a->num_experts) return MOE_LORA_ERR_INVALID;
  if (a->hidden % 64 || a->inter % 64) return MOE_LORA_ERR_UNSUPPORTED;
  if (a->max_rank > kMaxRank) return MOE_LORA_ERR_UNSUPPORTED;
  if ((int64_t)a->num_tokens * a->top_k > INT32_MAX / 2) return MOE_LORA_ERR_UNSUPPORTED;
  if (a->num_loras > 0 && a->max_rank <= 0) return MOE_LORA_ERR_INVALID;
  {
    // the GEMMs address gathered x rows and one expert's weight matrix with
    // 32-bit byte offsets from 64-bit bases
    const int64_t esz = a->dtype == MOE_LORA_BF16 ? 2 : 4;
    const int64_t wsz = (has_w && a->weight_dtype == MOE_LORA_FP8_E4M3) ? 1 : esz;
    if ((int64_t)a->num_tokens * a->hidden * esz >= kMaxOffsetBytes ||
        2 * (int64_t)a->inter * a->hidden * wsz >= kMaxOffsetBytes)
      return MOE_LORA_ERR_UNSUPPORTED;
  }
  if (check_ptrs && a->num_tokens > 0) {
    if (!a->x || !a->topk_weights || !a->w_gate_up || !a->w_down || !a->sorted_pair_ids ||
        !a->tile_expert || !a->tile_lora || !a->expert_tile_offsets || !a->num_rows_padded || !a->y)
      return MOE_LORA_ERR_INVALID;
    if (a->num_loras > 0 && (!a->a_gate || !a->a_up || !a->b_gate || !a->b_up || !a->a_down ||
                             !a->b_down || !a->lora_ranks || !a->scaling))
      return MOE_LORA_ERR_INVALID;
    if (misaligned(a->x) || misaligned(a->w_gate_up) || misaligned(a->w_down) || misaligned(a->y) ||
        misaligned(a->workspace))
      return MOE_LORA_ERR_INVALID;
    if (a->num_loras > 0 && (misaligned(a->a_gate) || misaligned(a->a_up) || misaligned(a->b_gate) ||
                             misaligned(a->b_up) || misaligned(a->a_down) || misaligned(a->b_down)))
      return MOE_LORA_ERR_INVALID;
  }
  p->dtype = a->dtype;
  p->T = a->num_tokens; p->H = a->hidden; p->I = a->inter; p->E = a->num_experts;
  p->k = a->top_k; p->L = a->num_loras; p->R = a->num_loras > 0 ? a->max_rank : 0; p->BM = a->block_m;
  p->x = a->x; p->topk_weights = a->topk_weights;
  p->w_gate_up = a->w_gate_up; p->w_down = a->w_down;
  p->a_gate = a->a_gate; p->a_up = a->a_up; p->b_gate = a->b_gate; p->b_up = a->b_up;
  p->a_down = a->a_down; p->b_down = a->b_down;
  p->lora_ranks = a->lora_ranks; p->scaling = a->scaling;
  p->sorted_ids = a->sorted_pair_ids; p->tile_expert = a->tile_expert; p->tile_lora = a->tile_lora;
  p->expert_tile_offsets = a->expert_tile_offsets; p->num_rows_padded = a->num_rows_padded;
  p->y = a->y;
  if (a->out_dtype != a->dtype && a->out_dtype != MOE_LORA_F32) return MOE_LORA_ERR_UNSUPPORTED;
  p->out_f32 = (a->out_dtype == MOE_LORA_F32) && a->dtype != MOE_LORA_F32;
  p->wdtype = 0;
  if (wdt != a->dtype) {
    if (wdt != MOE_LORA_FP8_E4M3 || a->dtype != MOE_LORA_BF16) return MOE_LORA_ERR_UNSUPPORTED;
    if (a->hidden % 128 || a->inter % 128 || a->hidden > 16384 || a->inter > 16384)
      return MOE_LORA_ERR_UNSUPPORTED;
    if (check_ptrs && a->num_tokens > 0 && (!a->w_gate_up_scale || !a->w_down_scale))
      return MOE_LORA_ERR_INVALID;
    p->wdtype = kWeightFp8;
    p->w_gate_up_scale = a->w_gate_up_scale;
    p->w_down_scale = a->w_down_scale;
  }
  return MOE_LORA_OK;
}

size_t moe_lora_forward_workspace_bytes(const moe_lora_forward_args* args) {
  ForwardProblem p;
  if (to_problem(args, &p, false) != MOE_LORA_OK) return 0;
  return forward_ws_layout(p).bytes;
}

static int forward_impl(const moe_lora_forward_args* args, void* stream, void* const* events) {
  ForwardProblem p;
  int st = to_problem(args, &p, true);
  if (st != MOE_LORA_OK) return st;
  if (p.T == 0) return MOE_LORA_OK;
  const size_t need = forward_ws_layout(p).bytes;
  if (!args->workspace || args->workspace_bytes < need) return MOE_LORA_ERR_WORKSPACE;
  hipEvent_t ev[2 * kNumStages];
  if (events)
    for (int i = 0; i < 2 * kNumStages; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  return hip_status(launch_forward(p, args->workspace, static_cast<hipStream_t>(stream),
                                   events ? ev : nullptr));
}

int moe_lora_forward(const moe_lora_forward_args* args, void* stream) {
  return forward_impl(args, stream, nullptr);
}

int moe_lora_forward_events(const moe_lora_forward_args* args, void* stream,
                            void* const* events) {
  if (!events) return MOE_LORA_ERR_INVALID;
  return forward_impl(args, stream, events);
}

int moe_lora_forward_noalloc(const moe_lora_forward_args* args, void* stream) {
  ForwardProblem p;
  // the workspace fields are not used: validate as if a workspace were given
  int st = to_problem(args, &p, false);
  if (st != MOE_LORA_OK) return st;
  if (p.T == 0) return MOE_LORA_OK;
  moe_lora_forward_args chk = *args;
  chk.workspace = reinterpret_cast<void*>(uintptr_t(256));
  st = to_problem(&chk, &p, true);
  if (st != MOE_LORA_OK) return st;
  if (forward_ws_layout(p).bytes > kNoAllocScratchBytes) return MOE_LORA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess || !ws) return MOE_LORA_ERR_HIP;
  return hip_status(launch_forward(p, ws, static_cast<hipStream_t>(stream), nullptr));
}

size_t moe_lora_forward_noalloc_max_workspace_bytes(void) { return kNoAllocScratchBytes; }

static int to_dense(const moe_lora_dense_args* a, DenseProblem* p, bool check_ptrs) {
  if (!a || a->struct_size < sizeof(moe_lora_dense_args)) return MOE_LORA_ERR_INVALID;
  if (a->dtype != MOE_LORA_F32 && a->dtype != MOE_LORA_BF16) return MOE_LORA_ERR_UNSUPPORTED;
  if (a->num_tokens < 0 || a->hidden <= 0 || a->out0 <= 0 || a->out1 < 0 || a->num_loras < 0 ||
      a->max_rank < 0 || bad_block_m(a->block_m))
    return MOE_LORA_ERR_INVALID;
  if (a->hidden % 64 || a->out0 % 64 || a->out1 % 64) return MOE_LORA_ERR_UNSUPPORTED;
  if (a->max_rank > kMaxRank) return MOE_LORA_ERR_UNSUPPORTED;
  if (a->num_loras > 0 && a->max_rank <= 0) return MOE_LORA_ERR_INVALID;
  if ((int64_t)a->num_loras + 1 > kMaxKeys) return MOE_LORA_ERR_UNSUPPORTED;
  {
    const int64_t esz = a->dtype == MOE_LORA_BF16 ? 2 : 4;
    if ((int64_t)a->num_tokens * a->hidden * esz >= kMaxOffsetBytes ||
        ((int64_t)a->out0 + a->out1) * a->hidden * esz >= kMaxOffsetBytes)
      return MOE_LORA_ERR_UNSUPPORTED;
  }
  if (a->out_dtype != a->dtype && a->out_dtype != MOE_LORA_F32) return MOE_LORA_ERR_UNSUPPORTED;
  if (check_ptrs && a->num_tokens > 0) {
    if (!a->x || !a->w || !a->sorted_pair_ids || !a->tile_expert || !a->tile_lora ||
        !a->expert_tile_offsets || !a->num_rows_padded || !a->y)
      return MOE_LORA_ERR_INVALID;
    if (a->num_loras > 0 && (!a->a0 || !a->b0 || !a->lora_ranks || !a->scaling ||
                             (a->out1 > 0 && (!a->a1 || !a->b1))))
      return MOE_LORA_ERR_INVALID;
    if (misaligned(a->x) || misaligned(a->w) || misaligned(a->y) || misaligned(a->workspace) ||
        (a->num_loras > 0 && (misaligned(a->a0) || misaligned(a->b0) || misaligned(a->a1) ||
                              misaligned(a->b1))))
      return MOE_LORA_ERR_INVALID;
  }
  p->dtype = a->dtype;
  p->T = a->num_tokens; p->H = a->hidden; p->N0 = a->out0; p->N1 = a->out1;
  p->L = a->num_loras; p->R = a->num_loras > 0 ? a->max_rank : 0; p->BM = a->block_m;
  p->x = a->x; p->w = a->w;
  p->a0 = a->a0; p->a1 = a->a1; p->b0 = a->b0; p->b1 = a->b1;
  p->lora_ranks = a->lora_ranks; p->scaling = a->scaling;
  p->sorted_ids = a->sorted_pair_ids; p->tile_expert = a->tile_expert; p->tile_lora = a->tile_lora;
  p->expert_tile_offsets = a->expert_tile_offsets; p->num_rows_padded = a->num_rows_padded;
  p->y = a->y;
  p->out_f32 = (a->out_dtype == MOE_LORA_F32) && a->dtype != MOE_LORA_F32;
  return MOE_LORA_OK;
}

size_t moe_lora_dense_workspace_bytes(const moe_lora_dense_args* args) {
  DenseProblem p;
  if (to_dense(args, &p, false) != MOE_LORA_OK) return 0;
  return dense_ws_layout(p).bytes;
}

static int dense_impl(const moe_lora_dense_args* args, void* stream, void* const* events) {
  DenseProblem p;
  int st = to_dense(args, &p, true);
  if (st != MOE_LORA_OK) return st;
  if (p.T == 0) return MOE_LORA_OK;
  if (!args->workspace || args->workspace_bytes < dense_ws_layout(p).bytes) return MOE_LORA_ERR_WORKSPACE;
  hipEvent_t ev[2 * kDenseNumStages];
  if (events)
    for (int i = 0; i < 2 * kDenseNumStages; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  return hip_status(launch_dense(p, args->workspace, static_cast<hipStream_t>(stream),
                                 events ? ev : nullptr));
}

int moe_lora_dense_forward(const moe_lora_dense_args* args, void* stream) {
  return dense_impl(args, stream, nullptr);
}

int moe_lora_dense_forward_events(const moe_lora_dense_args* args, void* stream,
                                  void* const* events) {
  if (!events) return MOE_LORA_ERR_INVALID;
  return dense_impl(args, stream, events);
}

}  // extern "C"
