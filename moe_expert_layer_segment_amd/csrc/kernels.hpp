// Host-side launchers of the gfx950 MoE-LoRA kernels (internal to the library;
// the public surface is the C ABI in include/moe_lora.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moelora {

// ---- align -----------------------------------------------------------------
struct AlignWs {
  int64_t nchunks;
  size_t rank_off, cnt_off, bstart_off, btotal_off, bytes;
};
AlignWs align_ws_layout(int64_t num_pairs, int64_t num_keys);
int64_t align_chunk_pairs(int64_t num_pairs, int64_t num_keys);

// rows of the align outputs: P + min(P, E*(L+1)) * (BM - 1), rounded up to BM
inline int64_t align_capacity(int64_t P, int64_t E, int64_t L, int64_t BM) {
  int64_t K = E * (L + 1);
  int64_t nb = P < K ? P : K;
  int64_t rows = P + nb * (BM - 1);
  return (rows + BM - 1) / BM * BM;
}

// debug_word: the device flag word of MOE_LORA_DEBUG builds (null: no checks)
hipError_t launch_info(int32_t num_tokens, int32_t num_reqs, int32_t num_loras,
                       const int32_t* seg_indptr, const int32_t* weight_indices,
                       const int32_t* lora_ranks, int32_t* adapter_enabled,
                       int32_t* token_lora_mapping, uint32_t* debug_word, hipStream_t stream);

// The device flag word of this build on the current device (null in release
// builds), and reading / clearing it after a stream synchronisation.
uint32_t* debug_word();
hipError_t debug_word_read(uint32_t* flags, bool clear, hipStream_t stream);

int route_max_k();
hipError_t launch_route(int32_t T, int32_t E, int32_t k, const float* logits, int32_t* topk_ids,
                        float* topk_weights, hipStream_t stream);

hipError_t launch_align(int32_t T, int32_t k, int32_t E, int32_t L, int32_t BM,
                        const int32_t* topk_ids, const int32_t* mapping, const int32_t* enabled,
                        int32_t* sorted_ids, int32_t* tile_expert, int32_t* tile_lora,
                        int32_t* expert_tile_offsets, int32_t* num_rows_padded, void* workspace,
                        uint32_t* debug_word, hipStream_t stream);

// ---- forward ---------------------------------------------------------------
// expert weights as fp8 e4m3 codes with 128 x 128 block scales (dtype bf16)
constexpr int kWeightFp8 = 2;

struct ForwardProblem {
  int dtype;  // 0 = fp32, 1 = bf16
  int wdtype = 0;  // dtype of the expert weights: dtype, or kWeightFp8
  const float* w_gate_up_scale = nullptr;   // fp8: [E, 2I/128, H/128]
  const float* w_down_scale = nullptr;      // fp8: [E, H/128, I/128]
  int64_t T, H, I, E, k, L, R, BM;
  const void* x;
  const float* topk_weights;
  const void *w_gate_up, *w_down;
  const void *a_gate, *a_up, *b_gate, *b_up, *a_down, *b_down;
  const int32_t* lora_ranks;
  const float* scaling;
  const int32_t *sorted_ids, *tile_expert, *tile_lora, *expert_tile_offsets, *num_rows_padded;
  void* y;
  int out_f32;  // y in fp32 instead of dtype
};

struct ForwardWs {
  int64_t cap, max_items, RP;
  int64_t n_tiles_gu = 0, n_tiles_dn = 0;   // column tiles (x K splits) of the two GEMMs
  size_t items_off, count_off, tab_gu_off, tab_dn_off, slot_rank_off, hgu_off, act_off, hd_off, z_off,
      part_off = 0, bytes;
  int64_t grid_gu = 0;             // workgroups of the general gate_up GEMM (0: tail split unused)
  int split_gu = 1, split_d = 1;   // K splits of the two shrinks
  bool shrink4 = false;            // shrinks share pool rows across 4 row groups
  int split_down_k = 1;            // K splits of the down GEMM (planes of z)
  bool big = false;                // the large-tile bf16 GEMMs (256-row items)
  int rows_per_item = 0;           // rows of a GEMM work item
};
ForwardWs forward_ws_layout(const ForwardProblem& p);
// stages of the forward, in launch order (index into the optional event pairs)
enum { kStagePlan = 0, kStageShrinkX, kStageGateUp, kStageShrinkA, kStageDown, kStageCombine,
       kNumStages };
hipError_t launch_forward(const ForwardProblem& p, void* workspace, hipStream_t stream,
                          hipEvent_t* events);

// The allocation-free forward's workspace: a static device array of this many
// bytes, one per device; noalloc_scratch returns the current device's address.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

// A dense projection with per-request LoRA whose output is two column slices
// [0, N0) and [N0, N0 + N1), each with its own LoRA factors (N1 may be 0).
struct DenseProblem {
  int dtype;  // 0 = fp32, 1 = bf16
  int64_t T, H, N0, N1, L, R, BM;
  const void* x;                       // [T, H]
  const void* w;                       // [N0 + N1, H]
  const void *a0, *a1, *b0, *b1;       // [L, R, H] x2, [L, R, N0], [L, R, N1]
  const int32_t* lora_ranks;
  const float* scaling;
  const int32_t *sorted_ids, *tile_expert, *tile_lora, *expert_tile_offsets, *num_rows_padded;
  void* y;                             // [T, N0 + N1]
  int out_f32;
};
struct DenseWs {
  int64_t cap, max_items, RP;
  int npool = 1, split = 1, ksplit = 1;   // shrink pools / shrink K splits / GEMM K splits
  int64_t n_tiles = 0;                    // GEMM column tiles x K splits
  size_t items_off, count_off, tab_off, slot_rank_off, h_off, z_off, bytes;
};
DenseWs dense_ws_layout(const DenseProblem& p);
enum { kDenseStagePlan = 0, kDenseStageShrink, kDenseStageGemm, kDenseStageCombine, kDenseNumStages };
hipError_t launch_dense(const DenseProblem& p, void* workspace, hipStream_t stream, hipEvent_t* events);

}  // namespace moelora
