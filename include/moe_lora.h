/*
 * moe_lora.h -- C ABI of the MI355X (gfx950) MoE expert layer with per-request
 * LoRA deltas.
 *
 * The layer (SGLang PR #14105 page, on LoRA for MoE expert layers, section
 * 实现拆解, the layer formula) computes, for every token t with top-k experts
 * e_j and router weights w_j, and the token's adapter slot l:
 *
 *   y_t = sum_j w_j * (W_down[e] + s_l B_d A_d)
 *                     [ SiLU((W_gate[e] + s_l B_g A_g) x_t) * ((W_up[e] + s_l B_u A_u) x_t) ]
 *
 * with LoRA factors taken from 4-D pools [num_loras, num_experts, rank, dim]
 * (same page, same section) and the slot picked per token from request
 * segments (SGLang PR #24160 page, on sharing the MoE LoRA batch info, sections
 * 实现拆解 and 关键源码片段).
 *
 * Three calls, plus the router step before them:
 *   moe_lora_route   -- per layer, optional: top-k experts and weights from router logits.
 *   moe_lora_info    -- once per batch: token_lora_mapping and adapter_enabled.
 *   moe_lora_align   -- per layer: bucket (token, expert) pairs by (expert, adapter),
 *                       padded to block_m rows.
 *   moe_lora_forward -- per layer: grouped gate_up GEMM with fused LoRA expand and
 *                       SiLU*mul, grouped down GEMM with fused LoRA expand and the
 *                       router weight, then the top-k combine.
 *
 * Conventions shared by every call:
 *   - Every array argument is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or retains memory.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) with no host synchronisation.
 *   - Validation reads host scalars only; device contents are never read on the
 *     host.  Calls on disjoint buffers may run concurrently.
 *   - Integer metadata is int32; router weights and scaling are float32.
 *   - Return value: MOE_LORA_OK or one of the negative codes below.
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_LORA_OK = 0,
  MOE_LORA_ERR_INVALID = -1,     /* null pointer, bad dimension or inconsistent sizes */
  MOE_LORA_ERR_UNDERCOVER = -2,  /* num_reqs * max_seg_len < num_tokens (info only)   */
  MOE_LORA_ERR_UNSUPPORTED = -3, /* dtype or size outside what the kernels support     */
  MOE_LORA_ERR_HIP = -4,         /* a HIP launch / runtime error                        */
  MOE_LORA_ERR_WORKSPACE = -5    /* workspace missing or too small                      */
};

typedef enum { MOE_LORA_F32 = 0, MOE_LORA_BF16 = 1, MOE_LORA_FP8_E4M3 = 2 } moe_lora_dtype;

/* Human-readable text of a status code (static storage, never NULL). */
const char* moe_lora_status_str(int status);

/*
 * moe_lora_route -- the router step before the layer.  None of the MoE-LoRA
 * pages describes a router; the layer configurations this library is measured
 * on define it as softmax over the experts, top-k, renormalised.  The order and
 * the tie rule are this library's reading.
 *
 *   logits        [num_tokens, num_experts] fp32, row-major, finite values.
 *   topk_ids      [num_tokens, top_k] out  int32: the top_k experts of largest
 *                                 probability (equivalently logit), in descending
 *                                 order, ties to the lower expert id.  Bit-exact.
 *   topk_weights  [num_tokens, top_k] out  fp32: their softmax probabilities
 *                                 renormalised over the top_k (sum to 1).
 *
 * 1 <= top_k <= num_experts, top_k <= 16 (else MOE_LORA_ERR_UNSUPPORTED).
 * num_tokens == 0 enqueues nothing.  The outputs feed moe_lora_align and
 * moe_lora_forward directly.
 */
int moe_lora_route(int32_t num_tokens, int32_t num_experts, int32_t top_k, const float* logits,
                   int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * moe_lora_info -- per-batch MoE-LoRA metadata (SGLang PR #24160 page,
 * section 实现拆解 items 1-3; its unit test in section 关键源码片段).
 *
 *   seg_indptr      [num_reqs + 1]  request segments: request b owns tokens
 *                                   [seg_indptr[b], seg_indptr[b+1]); must start at
 *                                   0, be nondecreasing and end at num_tokens.
 *   weight_indices  [num_reqs]      slot of each request (req_to_lora), -1 = none.
 *   lora_ranks      [num_loras]     rank of each slot, >= 0.
 *   adapter_enabled [num_loras] out 1 iff some request names the slot and its rank
 *                                   is > 0, else 0.  Every entry is written.
 *   token_lora_mapping [>= num_tokens] out  weight_indices repeated over each
 *                                   segment (-1 kept).  Entries past num_tokens are
 *                                   left untouched.
 *   max_seg_len     host hint of the longest segment; when > 0 and
 *                   num_reqs * max_seg_len < num_tokens the call returns
 *                   MOE_LORA_ERR_UNDERCOVER ("under-covers tokens") and launches
 *                   nothing.  0 skips the check.  The kernel itself covers every
 *                   token whatever the hint.
 * num_tokens == 0 is valid (only adapter_enabled is written).  num_loras == 0 is
 * valid.  Out-of-range device values (weight_indices outside [-1, num_loras)) are
 * ignored for adapter_enabled and copied through to the mapping.
 */
int moe_lora_info(int32_t num_tokens, int32_t num_reqs, int32_t num_loras, int32_t max_seg_len,
                  const int32_t* seg_indptr, const int32_t* weight_indices,
                  const int32_t* lora_ranks, int32_t* adapter_enabled,
                  int32_t* token_lora_mapping, void* stream);

/*
 * Capacity (rows) of the align outputs: P + min(P, E*(L+1)) * (block_m - 1)
 * rounded up to block_m, with P = num_tokens * top_k.  sorted_pair_ids needs
 * this many entries; tile_expert / tile_lora need capacity / block_m.
 * Returns -1 for invalid arguments and for sizes moe_lora_align does not
 * support (P > INT32_MAX / 2 or num_experts * (num_loras + 1) > 32768).
 */
int64_t moe_lora_align_capacity_rows(int32_t num_tokens, int32_t top_k, int32_t num_experts,
                                     int32_t num_loras, int32_t block_m);

/* Workspace bytes moe_lora_align needs for these sizes (0 on invalid arguments). */
size_t moe_lora_align_workspace_bytes(int32_t num_tokens, int32_t top_k, int32_t num_experts,
                                      int32_t num_loras, int32_t block_m);

/*
 * moe_lora_align -- bucket (token, expert) pairs by expert and adapter (SGLang
 * PR #14105 page, section 实现拆解: tokens sorted by LoRA adapter and expert id).
 *
 * Pair p = t * top_k + j has expert e = topk_ids[t * top_k + j] and effective
 * slot a = token_lora_mapping[t] if that is >= 0 and adapter_enabled[it] == 1,
 * else -1 (so rank-0 and unused slots fall into the no-LoRA bucket).  Buckets are
 * ordered by key e * (num_loras + 1) + (a + 1) (expert-major, no-LoRA first);
 * inside a bucket pairs keep ascending p.  Each bucket is padded with the
 * sentinel P = num_tokens * top_k up to a multiple of block_m rows; every
 * block_m rows form one tile.
 *
 *   topk_ids            [num_tokens, top_k]   expert ids in [0, num_experts).
 *   token_lora_mapping  [num_tokens]          from moe_lora_info.
 *   adapter_enabled     [num_loras]           from moe_lora_info (may be NULL iff
 *                                              num_loras == 0).
 *   sorted_pair_ids     [capacity]      out   pair ids in bucket order; P for pads
 *                                              and for the unused tail.
 *   tile_expert         [capacity/block_m] out expert of each tile, -1 past the end.
 *   tile_lora           [capacity/block_m] out effective slot of each tile (-1 = no
 *                                              LoRA, and past the end).
 *   expert_tile_offsets [num_experts + 1] out  first tile of each expert (experts
 *                                              with no pairs repeat the next
 *                                              offset); [num_experts] = tile count.
 *   num_rows_padded     [1]             out   tiles * block_m.
 *   workspace           >= moe_lora_align_workspace_bytes(...) bytes of device memory.
 * block_m must be a multiple of 16 in [16, 256].  Supports
 * num_experts * (num_loras + 1) <= 32768.  Expert ids outside [0, num_experts)
 * are undefined input; they never cause out-of-bounds writes.
 * Every output word up to the capacity is written, so results are fully defined.
 */
int moe_lora_align(int32_t num_tokens, int32_t top_k, int32_t num_experts, int32_t num_loras,
                   int32_t block_m, const int32_t* topk_ids, const int32_t* token_lora_mapping,
                   const int32_t* adapter_enabled, int32_t* sorted_pair_ids, int32_t* tile_expert,
                   int32_t* tile_lora, int32_t* expert_tile_offsets, int32_t* num_rows_padded,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device-side precondition checks (MOE_LORA_DEBUG builds, libmoe_lora_debug.so).
 *
 * Release builds never read device data on the host and treat device-side
 * precondition violations as undefined input (they never cause out-of-bounds
 * accesses: align drops pairs whose expert id is out of range, info ignores
 * out-of-range slots for adapter_enabled).  A library built with
 * MOE_LORA_DEBUG defined additionally checks, inside its kernels:
 *   MOE_LORA_DEBUG_SEG_INDPTR    (info)  seg_indptr[0] == 0, nondecreasing,
 *                                        seg_indptr[num_reqs] == num_tokens
 *   MOE_LORA_DEBUG_WEIGHT_INDEX  (info)  -1 <= weight_indices[b] < num_loras
 *   MOE_LORA_DEBUG_RANK          (info)  lora_ranks[i] >= 0
 *   MOE_LORA_DEBUG_EXPERT_ID     (align) 0 <= topk_ids[p] < num_experts
 *   MOE_LORA_DEBUG_MAPPING       (align) -1 <= token_lora_mapping[t] < num_loras
 * and ORs the bit of each violated check into a device word of the library
 * (one per device, shared by every call on it; the page on sharing the MoE
 * LoRA batch info, section 评论区精华, is about such a -1 index reaching a
 * scatter).  The results of the calls are those of the release build.
 *
 * moe_lora_debug_flags synchronises `stream`, writes the word to *flags and,
 * when `clear` is nonzero, resets it to 0.  A release build writes 0 and
 * returns MOE_LORA_ERR_UNSUPPORTED.  flags NULL is MOE_LORA_ERR_INVALID.
 */
enum {
  MOE_LORA_DEBUG_SEG_INDPTR = 1,
  MOE_LORA_DEBUG_WEIGHT_INDEX = 2,
  MOE_LORA_DEBUG_RANK = 4,
  MOE_LORA_DEBUG_EXPERT_ID = 8,
  MOE_LORA_DEBUG_MAPPING = 16
};
int moe_lora_debug_flags(uint32_t* flags, int32_t clear, void* stream);

/*
 * Arguments of moe_lora_forward.  All tensors are row-major and contiguous.
 * `dtype` applies to x, the expert weights, the six pools and y.
 *
 *   x            [T, H]           hidden states.
 *   topk_ids     [T, k] int32     (only used through the align outputs; may be NULL).
 *   topk_weights [T, k] float32   router weights, applied to each expert output.
 *   w_gate_up    [E, 2I, H]       rows [0, I) = gate, rows [I, 2I) = up (nn.Linear
 *                                  [out, in] layout stacked over experts).
 *   w_down       [E, H, I]
 *   a_gate, a_up [L, E, R, H]     LoRA A of gate / up, rank-major.
 *   b_gate, b_up [L, E, R, I]     LoRA B of gate / up stored transposed (rank-major).
 *   a_down       [L, E, R, I]
 *   b_down       [L, E, R, H]     LoRA B of down, transposed.
 *   lora_ranks   [L] int32        rows >= lora_ranks[l] of slot l's pools are never read.
 *   scaling      [L] float32      s_l = alpha / r of each slot.
 *   sorted_pair_ids, tile_expert, tile_lora, expert_tile_offsets, num_rows_padded:
 *                the outputs of moe_lora_align for the same topk_ids, mapping,
 *                block_m.  Any layout with the same structure works (every pair
 *                exactly once, tiles uniform in (expert, slot), each expert's tiles
 *                contiguous and listed by expert_tile_offsets).
 *   workspace    >= moe_lora_forward_workspace_bytes(args) bytes of device memory.
 *   y            [T, H] out       overwritten, in out_dtype.
 *   out_dtype    dtype of y: `dtype` (the default layout) or MOE_LORA_F32 (the fp32
 *                combine result without the final rounding to bf16).
 * num_loras == 0 (pools NULL) runs the plain MoE layer.  H and I must be
 * multiples of 64, R <= 64, top_k <= num_experts.  Size limits (else
 * MOE_LORA_ERR_UNSUPPORTED): T * H elements of x and 2I * H elements of one
 * expert's gate_up matrix must each take less than 4 GiB (the GEMMs address
 * them with 32-bit offsets from 64-bit bases); T * top_k < 2^30.
 * x, the expert weights, the six pools, y and the workspace must be 16-byte
 * aligned (the kernels read and write them in 16-byte units); a misaligned
 * pointer is MOE_LORA_ERR_INVALID.
 *
 * FP8 expert weights (the fields after out_dtype; a caller whose struct_size
 * ends at out_dtype gets weights in `dtype`):
 *   weight_dtype     `dtype` (0 is read as `dtype` too) or MOE_LORA_FP8_E4M3:
 *                    w_gate_up and w_down then hold one-byte OCP e4m3 codes
 *                    (bias 7, no infinities, S.1111.111 = NaN) in the same
 *                    [E, 2I, H] / [E, H, I] layouts.  Requires dtype BF16 (x,
 *                    pools and y stay bf16), H and I multiples of 128 and at
 *                    most 16384.
 *   w_gate_up_scale  [E, 2I/128, H/128] float32: weight (e, n, k) is
 *                    code(e, n, k) * scale[e, n/128, k/128] (block-scaled
 *                    quantization over 128 x 128 blocks of each expert's
 *                    [rows, K] matrix).
 *   w_down_scale     [E, H/128, I/128] float32, likewise.
 * The kernels convert each code exactly and round code * scale to bf16 (exact
 * for a power-of-two scale) before the bf16 matrix cores; accumulation is fp32.
 * Errors: MOE_LORA_ERR_UNSUPPORTED for another weight dtype or shape,
 * MOE_LORA_ERR_INVALID for a missing scale pointer.
 */
typedef struct moe_lora_forward_args {
  size_t struct_size; /* sizeof(moe_lora_forward_args) */
  int32_t dtype;      /* moe_lora_dtype */
  int32_t num_tokens, hidden, inter, num_experts, top_k, num_loras, max_rank, block_m;
  const void* x;
  const int32_t* topk_ids;
  const float* topk_weights;
  const void* w_gate_up;
  const void* w_down;
  const void* a_gate;
  const void* a_up;
  const void* b_gate;
  const void* b_up;
  const void* a_down;
  const void* b_down;
  const int32_t* lora_ranks;
  const float* scaling;
  const int32_t* sorted_pair_ids;
  const int32_t* tile_expert;
  const int32_t* tile_lora;
  const int32_t* expert_tile_offsets;
  const int32_t* num_rows_padded;
  void* workspace;
  size_t workspace_bytes;
  void* y;
  int32_t out_dtype; /* moe_lora_dtype of y */
  int32_t weight_dtype;           /* moe_lora_dtype of w_gate_up / w_down */
  const float* w_gate_up_scale;   /* FP8_E4M3 weights: [E, 2I/128, H/128] */
  const float* w_down_scale;      /* FP8_E4M3 weights: [E, H/128, I/128] */
} moe_lora_forward_args;

/* Workspace bytes moe_lora_forward needs for the sizes in `args` (0 if invalid). */
size_t moe_lora_forward_workspace_bytes(const moe_lora_forward_args* args);

/*
 * moe_lora_forward -- the layer (SGLang PR #14105 page, section 实现拆解): gate/up
 * projections with LoRA, SiLU(gate) * up, down projection with LoRA, router
 * weight, and the sum over the top-k experts (in slot order j = 0..k-1, fp32).
 */
int moe_lora_forward(const moe_lora_forward_args* args, void* stream);

/*
 * Number of kernel stages of moe_lora_forward, in launch order: 0 plan (work
 * items and tile tables), 1 gate/up LoRA shrink, 2 gate_up GEMM (+LoRA expand, SiLU*mul),
 * 3 down LoRA shrink, 4 down GEMM (+LoRA expand, router weight), 5 top-k combine.
 */
#define MOE_LORA_FORWARD_STAGES 6

/*
 * moe_lora_forward_events -- moe_lora_forward for measurement: additionally
 * records the caller's hipEvent_t handles on `stream`, events[2s] before and
 * events[2s+1] after stage s (s < MOE_LORA_FORWARD_STAGES; NULL entries are
 * skipped; a stage that launches nothing gets two adjacent records).  The two
 * GEMM stages (2 and 4), one kernel each, hand their pair to the kernel launch
 * itself (hipExtLaunchKernel: the dispatch records the kernel's start and end),
 * so timing them puts no marker between kernels; the other stages' events are
 * recorded with hipEventRecord.  Adds no synchronisation; results are
 * identical to moe_lora_forward.  The caller owns
 * the events and reads them with hipEventElapsedTime after synchronising.
 */
int moe_lora_forward_events(const moe_lora_forward_args* args, void* stream,
                            void* const* events);

/*
 * moe_lora_forward_noalloc -- moe_lora_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, with the
 * workspace taken from a static device array of the library instead of
 * args->workspace (workspace and workspace_bytes are ignored).  The call itself
 * allocates nothing.
 *   - The array holds moe_lora_forward_noalloc_max_workspace_bytes() bytes
 *     (64 MiB), one per device, from the library's load until the process
 *     ends.  A problem whose moe_lora_forward_workspace_bytes exceeds it
 *     returns MOE_LORA_ERR_WORKSPACE and launches nothing.
 *   - Every call on a device shares that device's array: calls that overlap
 *     on one device (two streams, or host threads) race; serialise them.  The
 *     kernels initialise everything they read, so the previous call's
 *     contents never matter.
 *   - Its device address is looked up on the first call on each device
 *     (hipGetSymbolAddress, with that device current); MOE_LORA_ERR_HIP if
 *     that fails.  Other errors as for moe_lora_forward.
 */
int moe_lora_forward_noalloc(const moe_lora_forward_args* args, void* stream);
size_t moe_lora_forward_noalloc_max_workspace_bytes(void);

/*
 * Dense projection with per-request LoRA and a two-slice output (LoRA on a
 * fused projection with outputs of unequal sizes: the SGLang PR #22323
 * page, sections 功能与动机 and 实现拆解 item 2 -- the fused q_a_proj +
 * kv_a_proj_with_mqa projection of MLA, whose LoRA B is split in two and
 * applied per output part).  For token t in a request using slot l:
 *
 *   y[t, 0:N0)        = x_t W[0:N0)^T     + on * s_l (x_t A0_l^T) B0_l^T
 *   y[t, N0:N0+N1)    = x_t W[N0:N0+N1)^T + on * s_l (x_t A1_l^T) B1_l^T
 *
 * with on = (l >= 0 && adapter_enabled[l] && lora_ranks[l] > 0), exactly the
 * masking of the MoE layer.  The batch metadata comes from moe_lora_info and
 * moe_lora_align called with num_experts = 1, top_k = 1 and topk_ids all 0
 * (align then buckets the tokens by slot).
 *
 *   x            [T, H]            activations (dtype).
 *   w            [N0 + N1, H]      the fused weight, rows [0, N0) slice 0.
 *   a0, a1       [L, R, H]         LoRA A of slice 0 / 1, rank-major.
 *   b0           [L, R, N0]        LoRA B of slice 0, stored transposed.
 *   b1           [L, R, N1]        LoRA B of slice 1 (a1, b1 may be NULL when N1 == 0).
 *   lora_ranks   [L] int32, scaling [L] float32: as for the MoE layer.
 *   the align outputs, workspace (>= moe_lora_dense_workspace_bytes) and
 *   y            [T, N0 + N1] out  overwritten, in out_dtype (dtype or F32).
 * H, N0 and N1 must be multiples of 64 (N0 > 0, N1 >= 0), R <= 64; x and w
 * must each take less than 4 GiB (else MOE_LORA_ERR_UNSUPPORTED).  x, w, the
 * four pools, y and the workspace must be 16-byte aligned.  Errors and
 * ownership as for moe_lora_forward.
 */
typedef struct moe_lora_dense_args {
  size_t struct_size; /* sizeof(moe_lora_dense_args) */
  int32_t dtype;      /* MOE_LORA_F32 or MOE_LORA_BF16 */
  int32_t num_tokens, hidden, out0, out1, num_loras, max_rank, block_m;
  const void* x;
  const void* w;
  const void* a0;
  const void* a1;
  const void* b0;
  const void* b1;
  const int32_t* lora_ranks;
  const float* scaling;
  const int32_t* sorted_pair_ids;
  const int32_t* tile_expert;
  const int32_t* tile_lora;
  const int32_t* expert_tile_offsets;
  const int32_t* num_rows_padded;
  void* workspace;
  size_t workspace_bytes;
  void* y;
  int32_t out_dtype;
} moe_lora_dense_args;

/* Workspace bytes moe_lora_dense_forward needs for the sizes in `args` (0 if invalid). */
size_t moe_lora_dense_workspace_bytes(const moe_lora_dense_args* args);

int moe_lora_dense_forward(const moe_lora_dense_args* args, void* stream);

/* moe_lora_dense_forward plus caller-owned HIP events recorded around its four
 * kernel stages (plan, shrink, GEMM, combine): events[2s] before and
 * events[2s+1] after stage s; NULL entries are skipped; the GEMM stage's pair
 * is recorded by its kernel launch, as in moe_lora_forward_events.
 * Measurement only. */
int moe_lora_dense_forward_events(const moe_lora_dense_args* args, void* stream,
                                  void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LORA_H */
