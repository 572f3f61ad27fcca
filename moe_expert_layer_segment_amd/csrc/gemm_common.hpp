// Shared pieces of the grouped GEMM kernels: the argument block, the
// global -> LDS DMA helper and the wait-then-barrier of the LDS rings.
#pragma once

#include "common.hpp"

namespace moelora {

template <typename T>
struct GemmArgs {
  const int4* items;
  const int32_t* item_count;
  int max_items, n_tiles;      // n_tiles: column tiles x K splits
  int n_cols, ksplit;           // column tiles; K splits (down only, else 1)
  // A operand
  const T* a_src;             // x [T, K] (gate_up, gathered) or act [cap, K] (down)
  const int32_t* sorted_ids;
  int top_k, P;
  int64_t K;
  // B operand: weights [E, w_rows, K], in T or as fp8 e4m3 codes
  const void* w;
  const float* w_scale;       // fp8 weights: [E, w_rows/128, K/128] block scales, else null
  int64_t n_out;              // output columns (I for gate_up, H for down)
  int64_t w_rows;             // rows per expert of w (2I or H)
  // LoRA
  const int32_t* tile_lora;
  const int32_t* expert_tile_offsets;   // [E+1], in align blocks of BM_tile rows
  int BM_tile;
  const int32_t* lora_ranks;
  const float* h;             // [cap, HS] scaled shrink result: fp32 (fp32 T) or split bf16 halves (store_h_split)
  int HS, RP, R, L, E;
  const T* b_pool0;           // [L, E, R, n_out] (gate or down)
  const T* b_pool1;           // [L, E, R, n_out] (up) or null
  // outputs
  T* act;                     // gate_up: [cap, n_out]
  void* z;                    // down: [ksplit, P, n_out] weighted rows, one plane per K split:
                              // fp24 (fp24_pack4) for bf16 T, fp32 for fp32 T and dense mode
  const float* topk_weights;
  int64_t cap;                // rows of sorted_ids / act / h
  int32_t* tile_ctr;          // [8] per-XCD tile counters, zero at launch
  const int4* tile_tab;       // [item count x n_tiles] logical tile records (tile_table_kernel)
  const int32_t* slot_rank;   // [cap / BM_tile] slot | rank << 16 per align block, or -1
  int64_t n_split;            // dense mode: output columns [0, n_split) use b_pool0 and h[:, :RP],
                              // the rest b_pool1 and h[:, RP:2RP] (a multiple of 32)
  float* part;                // gate_up: partial sums of tail-tile K pieces, [gridDim.x][BM * BN]
                              // (null: no tail split)
};



// Issue one 16-byte-per-lane global -> LDS load: lane i of the wave writes the
// 16 bytes at gbase + goff to LDS byte address lds_addr + 16 * i.  The LDS base
// goes through M0 (saved and restored around the load, so the compiler's view
// of M0 is unchanged).  The compiler does not track these loads: callers wait
// for them with an explicit s_waitcnt vmcnt before a barrier.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t goff, uint32_t lds_addr) {
  // base and LDS address are wave-uniform: move them to SGPRs explicitly
  const uint64_t g = (uint64_t)(uintptr_t)gbase;
  const uint32_t glo = __builtin_amdgcn_readfirstlane((uint32_t)g);
  const uint32_t ghi = __builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
  const uint64_t gs = ((uint64_t)ghi << 32) | glo;
  const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[la]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[go], %[gb]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [la] "s"(la), [go] "v"(goff), [gb] "s"(gs)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  // all of this wave's LDS loads except the newest N have landed, then every
  // wave of the workgroup has got that far
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace moelora

namespace moelora {

// The large-tile bf16 GEMM (gemm_big.hip): tile rows, tile output columns and
// K tile depth, and its launch (gate_up or down form; the event pair, when
// given, is recorded by the dispatch itself).
int big_tile_rows();
int big_tile_cols(bool gate_up);
int big_tile_k();
void launch_gemm_big(bool gate_up, const GemmArgs<bf16_t>& a, int64_t nblk, hipStream_t stream,
                     hipEvent_t ev0, hipEvent_t ev1);

}  // namespace moelora
