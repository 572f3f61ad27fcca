// The MoE-LoRA layer forward on gfx950 (SGLang PR #14105 page, on LoRA for MoE
// expert layers, section 实现拆解: y = (W_down + s B_d A_d)[SiLU((W_gate + s B_g A_g)x)
// * ((W_up + s B_u A_u)x)], summed over the top-k experts with the router weights).
//
// Launch sequence on one stream, no host synchronisation:
//   plan     -- one workgroup turns expert_tile_offsets into GEMM work items
//               (row ranges of one expert, at most kBM rows each).
//   shrink_x -- per 16-row group with an adapter: h_gu = s * [x A_g^T | x A_u^T]
//               (rank columns beyond the slot rank are zero; a bf16 layer stores h
//               as its bf16 high and low halves, store_h_split).
//   gate_up  -- grouped MFMA GEMM over the work items: x rows gathered by pair id
//               times W_gate / W_up rows; LoRA expand h_g B_g, h_u B_u added to the
//               accumulators of each 16-row group; SiLU(gate) * up epilogue -> act.
//   shrink_a -- h_d = s * act A_d^T per 16-row group.
//   down     -- grouped MFMA GEMM act * W_down^T + h_d B_d, times the router weight,
//               written to z in pair order (fp32 layers: fp32; bf16 layers: the
//               top 24 bits of the fp32 value, fp24_pack4).
//   combine  -- y[t] = sum_j z[t*k + j] for j = 0..k-1 in order, summed in fp32,
//               cast to the output dtype.
#include <hip/hip_ext.h>

#include <mutex>

#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moelora {

// --------------------------------------------------------------------------
// plan: GEMM work items
// --------------------------------------------------------------------------
static constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(int E, int BM, int rows_per_item, const int32_t* __restrict__ expert_tile_offsets,
            int4* __restrict__ items, int32_t* __restrict__ item_count, int max_items) {
  __shared__ int lds_waves[kPlanThreads / 64 + 1];
  const int ept = (E + kPlanThreads - 1) / kPlanThreads;
  const int e0 = min(E, (int)threadIdx.x * ept), e1 = min(E, e0 + ept);
  int mine = 0;
  for (int e = e0; e < e1; ++e) {
    int rows = (expert_tile_offsets[e + 1] - expert_tile_offsets[e]) * BM;
    mine += (rows + rows_per_item - 1) / rows_per_item;
  }
  // exclusive scan over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      int c = lds_waves[w];
      lds_waves[w] = run;
      run += c;
    }
    lds_waves[kPlanThreads / 64] = run;
  }
  __syncthreads();
  int start = lds_waves[wave] + x - mine;
  for (int e = e0; e < e1; ++e) {
    int row0 = expert_tile_offsets[e] * BM;
    int rows = (expert_tile_offsets[e + 1] - expert_tile_offsets[e]) * BM;
    const int first = start;   // the expert's first item: the GEMMs order tiles by expert
    for (int r = 0; r < rows; r += rows_per_item) {
      if (start < max_items) items[start] = make_int4(row0 + r, min(rows_per_item, rows - r), e, first);
      ++start;
    }
  }
  if (threadIdx.x == 0) item_count[0] = min(lds_waves[kPlanThreads / 64], max_items);
  // the two GEMMs' per-XCD tile counters follow the item count
  if (threadIdx.x < 16) item_count[4 + threadIdx.x] = 0;
}

// --------------------------------------------------------------------------
// tile tables: the persistent GEMMs' logical tile order, one record per tile,
// so a workgroup finds its tile with one load instead of a chain of dependent
// ones; and each align block's LoRA slot with its rank in one word
// --------------------------------------------------------------------------
// Logical tiles are ordered expert by expert.  An expert's n_e work items are
// cut into round(n_e / 8) near-equal groups, and a group's tiles are
// column-major with its items fastest, so a weight column tile is fetched
// once per group and shared by its items.  (About 8 items per group balances
// the x rows and the weight columns that a window of 32 resident tiles
// fetches: a 128-row x tile is half a 256-row weight tile.)  Record:
// {first row, rows, expert, column tile x K split}; rows = 0 marks a tile
// past the item count.
#ifndef MOELORA_GROUP_ITEMS
#define MOELORA_GROUP_ITEMS 8   // work items per tile group of 128-row items (see above)
#endif
// 256-row items against 256-row weight tiles (measured on the 16384-token
// prefill batch, gate_up GEMM: 4 items 7.87 ms, 6 7.79, 8 7.66, 12 7.52)
#ifndef MOELORA_GROUP_ITEMS_BIG
#define MOELORA_GROUP_ITEMS_BIG 12
#endif
__device__ inline int4 gemm_tile_of(const int4* items, int count, int n_tiles, const int32_t* eto,
                                    int BM_tile, int E, int rows_per_item, int logical,
                                    int group_items) {
  const int4 skip = make_int4(0, 0, 0, -1);
  // the expert group of logical tile `logical` spans its items' range times
  // n_tiles, so item logical / n_tiles belongs to it
  const int4 in_group = items[logical / n_tiles];
  const int first = in_group.w, eg = in_group.z;
  if (eg < 0 || eg >= E || first < 0 || first > logical / n_tiles) return skip;
  const int rows_e = (eto[eg + 1] - eto[eg]) * BM_tile;
  const int n_e = (rows_e + rows_per_item - 1) / rows_per_item;   // the expert's items
  if (n_e <= 0) return skip;
  const int ng = max(1, (n_e + group_items / 2) / group_items);
  const int gbase = n_e / ng, grem = n_e % ng;   // groups 0..grem-1 have gbase+1 items
  const int li = logical / n_tiles - first;      // an item index inside the group
  const int gj = li < grem * (gbase + 1) ? li / (gbase + 1) : grem + (li - grem * (gbase + 1)) / gbase;
  const int g_off = gj * gbase + min(gj, grem);  // the group's first item
  const int g_n = gbase + (gj < grem ? 1 : 0);
  const int local = logical - (first + g_off) * n_tiles;
  const int item_idx = first + g_off + local % g_n;
  const int col_t = local / g_n;                 // column tile x K split
  if (item_idx >= count || col_t >= n_tiles) return skip;
  const int4 item = items[item_idx];
  if (item.z != eg) return skip;
  return make_int4(item.x, item.y, item.z, col_t);
}

// slot_rank[b] = slot | rank << 16 of align block b (rank = min(r_l, R)), or
// -1 when the block has no LoRA (slot -1, outside [0, L), or rank 0)
__global__ void __launch_bounds__(256)
tile_table_kernel(const int4* __restrict__ items, const int32_t* __restrict__ item_count, int max_items,
                  const int32_t* __restrict__ expert_tile_offsets, int BM_tile, int E, int rows_per_item,
                  int n_tiles0, int4* __restrict__ tab0, int n_tiles1, int4* __restrict__ tab1,
                  const int32_t* __restrict__ tile_lora, const int32_t* __restrict__ lora_ranks, int L,
                  int R, int n_blocks, int32_t* __restrict__ slot_rank, int group_items) {
  const int count = min(item_count[0], max_items);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n0 = (int64_t)count * n_tiles0, n1 = tab1 ? (int64_t)count * n_tiles1 : 0;
  const int64_t n = max(max(n0, n1), (int64_t)(slot_rank ? n_blocks : 0));
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (i < n0)
      tab0[i] = gemm_tile_of(items, count, n_tiles0, expert_tile_offsets, BM_tile, E, rows_per_item, (int)i,
                             group_items);
    if (i < n1)
      tab1[i] = gemm_tile_of(items, count, n_tiles1, expert_tile_offsets, BM_tile, E, rows_per_item, (int)i,
                             group_items);
    if (slot_rank && i < n_blocks) {
      const int l = tile_lora[i];
      const int r = (l >= 0 && l < L) ? min(lora_ranks[l], R) : 0;
      slot_rank[i] = r > 0 ? (l | (r << 16)) : -1;
    }
  }
}

// --------------------------------------------------------------------------
// shrink: h[row, pool*RP + q] = s_l * sum_k a_src[row, k] * A_pool[l, e, q, k]
// for q < r_l (zero for r_l <= q < RP).  One workgroup per (16-row group, K
// split); with more than one split, split c writes its partial sums to its
// own buffer and shrink_reduce adds them, in split order, into split 0.
// --------------------------------------------------------------------------
template <typename T>
struct ShrinkArgs {
  const T* src;               // x [T, K] (gathered) or act [cap, K] (direct)
  const int32_t* sorted_ids;  // gathered mode: pair id of each row
  int gathered, top_k, P;
  int64_t K;                  // contraction length (H or I)
  int64_t kchunk;             // K elements per split (multiple of 128)
  int64_t split_stride;       // floats between the splits' h buffers
  const T* pool0;             // [L, E, R, K]
  const T* pool1;             // second pool or null
  int R, RP, L, E, BM;
  const int32_t* tile_expert;
  const int32_t* tile_lora;
  const int32_t* num_rows_padded;
  const int32_t* lora_ranks;
  const float* scaling;
  float* h;                   // [cap, npools * RP]: fp32, or for bf16 T the final h split (store_h_split)
  int64_t cap;                // rows of h / act / sorted_ids
};

// The final h of a bf16 layer is stored split for the GEMM's expand, which
// multiplies h = hi + lo on bf16 matrix cores: per row, each group of 8
// consecutive columns takes the 32 bytes of 8 fp32 values as the 8 bf16 high
// parts hi = bf16(v), then the 8 low parts lo = bf16(v - hi) (both round to
// nearest even; v - hi is exact, so hi + lo keeps about 16 bits of v).
// Partial sums of a K-split shrink stay fp32 until shrink_reduce adds them.
__device__ inline void store_h_split(float* hrow, int c, float v) {
  bf16_t* g = reinterpret_cast<bf16_t*>(hrow + (c & ~7));
  const bf16_t hi = (bf16_t)v;
  g[c & 7] = hi;
  g[8 + (c & 7)] = (bf16_t)(v - (float)hi);
}

template <typename T, int NPOOL>
__global__ void __launch_bounds__(256) shrink_kernel(ShrinkArgs<T> a) {
  // one workgroup per 16-row group; its 4 waves take interleaved 32-deep K
  // steps and their partial sums are added in LDS
  typedef Elt<T> E_;
  typedef typename E_::frag frag;
  constexpr int NQB = 4;  // up to 64 rank columns per pool = 4 blocks of 16
  __shared__ floatx4 part[3][NPOOL * NQB][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  if (row0 >= a.num_rows_padded[0] || row0 + 16 > a.cap) return;
  const int64_t k_begin = (int64_t)blockIdx.y * a.kchunk;
  const int64_t k_end = min(a.K, k_begin + a.kchunk);
  const int tile = (int)(row0 / a.BM);
  const int l = a.tile_lora[tile];
  if (l < 0 || l >= a.L) return;
  const int e = a.tile_expert[tile];
  if (e < 0 || e >= a.E) return;
  const int r = min(a.lora_ranks[l], a.R);
  const float s = a.scaling[l];
  const int HS = NPOOL * a.RP;
  float* hrow_base = a.h + (int64_t)blockIdx.y * a.split_stride + row0 * HS;
  // a bf16 layer without a K split writes its final h, split (else fp32 partials)
  const bool split_h = sizeof(T) == 2 && gridDim.y == 1;
  if (r <= 0) {
    // rank-0 slots are folded into the no-LoRA bucket by align; keep h defined anyway
    for (int i = threadIdx.x; i < 16 * HS; i += 256) hrow_base[i] = 0.0f;
    return;
  }
  // A operand row of this lane
  const int my_row = lane & 15;
  const int kq = (lane >> 4) * 8;
  const T* arow = nullptr;
  {
    int64_t row = row0 + my_row;
    if (a.gathered) {
      int p = a.sorted_ids[row];
      if (p < a.P) arow = a.src + (int64_t)(p / a.top_k) * a.K;
    } else {
      arow = a.src + row * a.K;
    }
  }
  const T* prow[NPOOL][NQB];
  const int nqb = (r + 15) / 16;
#pragma unroll
  for (int pi = 0; pi < NPOOL; ++pi) {
    const T* pool = pi == 0 ? a.pool0 : a.pool1;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      int q = qb * 16 + my_row;
      prow[pi][qb] = (q < r) ? pool + (((int64_t)l * a.E + e) * a.R + q) * a.K : nullptr;
    }
  }
  floatx4 acc[NPOOL][NQB];
#pragma unroll
  for (int pi = 0; pi < NPOOL; ++pi)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc[pi][qb] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 2
  for (int64_t k0 = k_begin + wave * 32; k0 < k_end; k0 += 128) {
    frag av = arow ? load_frag_global<T>(arow + k0 + kq) : E_::zero();
#pragma unroll
    for (int pi = 0; pi < NPOOL; ++pi)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        if (qb < nqb) {
          frag bv = prow[pi][qb] ? load_frag_global<T>(prow[pi][qb] + k0 + kq) : E_::zero();
          acc[pi][qb] = E_::mma(av, bv, acc[pi][qb]);
        }
      }
  }
  if (wave > 0) {
#pragma unroll
    for (int pi = 0; pi < NPOOL; ++pi)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) part[wave - 1][pi * NQB + qb][lane] = acc[pi][qb];
  }
  __syncthreads();
  if (wave != 0) return;
  // C layout: lane holds rows 4*(lane/16)+i, column lane%16 of each 16x16 block
#pragma unroll
  for (int pi = 0; pi < NPOOL; ++pi)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int col = qb * 16 + (lane & 15);
      if (col >= a.RP) continue;
      floatx4 t = acc[pi][qb];
#pragma unroll
      for (int w = 0; w < 3; ++w) t += part[w][pi * NQB + qb][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = (lane >> 4) * 4 + i;
        float v = (qb < nqb && col < r) ? s * t[i] : 0.0f;
        if (split_h)
          store_h_split(hrow_base + (int64_t)rr * HS, pi * a.RP + col, v);
        else
          hrow_base[(int64_t)rr * HS + pi * a.RP + col] = v;
      }
    }
}

// The same shrink with the pool rows shared through LDS: a workgroup takes
// NW consecutive 16-row groups (one per wave) of one K split; when they belong
// to one (expert, slot) bucket -- the common case -- the bucket's pool rows
// are loaded once per 128-deep K chunk into LDS by the whole workgroup
// (double-buffered, register-staged) and each wave multiplies its own rows
// against them.  A wave whose group has another slot reads its pool rows from
// global memory instead.  Pool rows past the slot's rank are never read.
template <typename T, int NPOOL, int NW>
__global__ void __launch_bounds__(64 * NW) shrink4_kernel(ShrinkArgs<T> a) {
  typedef Elt<T> E_;
  typedef typename E_::frag frag;
  constexpr int NQB = 4;                            // up to 64 rank columns per pool
  constexpr int KC = 256 / (int)sizeof(T);          // K elements per LDS chunk (256 B a row)
  constexpr int CPQ = KC * (int)sizeof(T) / 16;     // 16-byte chunks per pool row and chunk
  constexpr int ROWEL = KC;                         // elements per LDS pool row
  // two buffers of NPOOL * RP rows of ROWEL elements (dynamic LDS, sized by the launch)
  extern __shared__ __attribute__((aligned(16))) unsigned char shrink4_lds[];
  T* const pool_lds = reinterpret_cast<T*>(shrink4_lds);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t nrp = a.num_rows_padded[0];
  const int64_t g0 = (int64_t)blockIdx.x * NW;      // the workgroup's first group
  if (g0 * 16 >= nrp) return;
  const int64_t k_begin = (int64_t)blockIdx.y * a.kchunk;
  const int64_t k_end = min(a.K, k_begin + a.kchunk);
  const int HS = NPOOL * a.RP;

  // slot, expert and rank of group g0 + w; false when the group has no rows
  // or no slot (its h rows are not written, as in shrink_kernel)
  auto group_key = [&](int w, int& l, int& e, int& r) -> bool {
    const int64_t row0 = (g0 + w) * 16;
    l = -1; e = -1; r = 0;
    if (row0 >= nrp || row0 + 16 > a.cap) return false;
    const int tile = (int)(row0 / a.BM);
    l = a.tile_lora[tile];
    e = a.tile_expert[tile];
    if (l < 0 || l >= a.L || e < 0 || e >= a.E) return false;
    r = min(a.lora_ranks[l], a.R);
    return true;
  };
  // the shared bucket: the first group's with a positive rank
  int sl = -1, se = -1, sr = 0;
  for (int w = 0; w < NW; ++w) {
    int l, e, r;
    if (group_key(w, l, e, r) && r > 0) { sl = l; se = e; sr = r; break; }
  }
  int l, e, r;
  const bool live = group_key(wave, l, e, r);
  const int64_t row0 = (g0 + wave) * 16;
  if (live && r <= 0) {
    // rank-0 slots are folded into the no-LoRA bucket by align; keep h defined anyway
    float* hz = a.h + (int64_t)blockIdx.y * a.split_stride + row0 * HS;
    for (int i = lane; i < 16 * HS; i += 64) hz[i] = 0.0f;
  }
  if (sl < 0) return;                               // no positive rank in these groups (uniform)
  const bool active = live && r > 0;
  const bool shared = active && l == sl && e == se;

  const int my_row = lane & 15;
  const int kq = (lane >> 4) * 8;
  const T* arow = nullptr;
  if (active) {
    const int64_t row = row0 + my_row;
    if (a.gathered) {
      const int pid = a.sorted_ids[row];
      if (pid < a.P) arow = a.src + (int64_t)(pid / a.top_k) * a.K;
    } else {
      arow = a.src + row * a.K;
    }
  }
  // this wave's own pool rows (used when its slot is not the shared one)
  const T* prow[NPOOL][NQB];
#pragma unroll
  for (int pi = 0; pi < NPOOL; ++pi) {
    const T* pool = pi == 0 ? a.pool0 : a.pool1;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int q = qb * 16 + my_row;
      prow[pi][qb] = (active && q < r) ? pool + (((int64_t)l * a.E + e) * a.R + q) * a.K : nullptr;
    }
  }
  const int nqb = (r + 15) / 16;
  floatx4 acc[NPOOL][NQB];
#pragma unroll
  for (int pi = 0; pi < NPOOL; ++pi)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc[pi][qb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // cooperative load of the shared pool rows q < sr of one K chunk: 16-byte
  // pieces, LDS row q of pool pi with piece c stored at piece c ^ (q % CPQ)
  // (16 consecutive rows read at one piece hit distinct banks)
  const int RPL = a.RP;                             // LDS rows per pool
  const int64_t buf_elems = (int64_t)NPOOL * RPL * ROWEL;
  const int PIECES = NPOOL * RPL * CPQ;
  constexpr int NT = 64 * NW;                        // threads
  constexpr int PER_THREAD = (NPOOL * 64 * CPQ + NT - 1) / NT;  // RP <= 64
  int4v stage[PER_THREAD];
  auto load_chunk = [&](int64_t kc0, int valid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = threadIdx.x + i * NT;
      const int pi = c / (RPL * CPQ), q = (c / CPQ) % RPL, pc = c % CPQ;
      const bool ok = c < PIECES && q < sr && pc * (16 / (int)sizeof(T)) < valid;
      const T* pool = pi == 0 ? a.pool0 : a.pool1;
      stage[i] = ok ? *reinterpret_cast<const int4v*>(
                          pool + (((int64_t)sl * a.E + se) * a.R + q) * a.K + kc0 + pc * (16 / (int)sizeof(T)))
                    : int4v{0, 0, 0, 0};
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c >= PIECES) continue;
      const int pi = c / (RPL * CPQ), q = (c / CPQ) % RPL, pc = c % CPQ;
      *reinterpret_cast<int4v*>(&pool_lds[buf * buf_elems + (pi * RPL + q) * ROWEL +
                                          ((pc ^ (q % CPQ)) * 16 / (int)sizeof(T))]) = stage[i];
    }
  };
  // one frag (8 K elements from kel) of LDS pool row q
  auto lds_frag = [&](int buf, int pi, int q, int kel) -> frag {
    constexpr int EPP = 16 / (int)sizeof(T);       // elements per piece
    frag f;
    if constexpr (sizeof(T) == 2) {
      const int pc = kel / EPP;
      f = *reinterpret_cast<const frag*>(&pool_lds[buf * buf_elems + (pi * RPL + q) * ROWEL + ((pc ^ (q % CPQ)) * EPP)]);
    } else {
      const int pc = kel / EPP;
      const T* rowp = &pool_lds[buf * buf_elems + (pi * RPL + q) * ROWEL];
      const floatx4 lo = *reinterpret_cast<const floatx4*>(rowp + ((pc ^ (q % CPQ)) * EPP));
      const floatx4 hi = *reinterpret_cast<const floatx4*>(rowp + (((pc + 1) ^ (q % CPQ)) * EPP));
      f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
      f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    }
    return f;
  };

  const int nchunks = (int)ceil_div(k_end - k_begin, KC);
  if (nchunks > 0) {
    load_chunk(k_begin, (int)min<int64_t>(KC, k_end - k_begin));
    store_chunk(0);
  }
  for (int c = 0; c < nchunks; ++c) {
    const int64_t kc0 = k_begin + (int64_t)c * KC;
    const int valid = (int)min<int64_t>(KC, k_end - kc0);
    __syncthreads();   // chunk c is in LDS; everyone is done with chunk c-1
    const bool more = c + 1 < nchunks;
    // this chunk's A rows are requested before the next pool chunk, so that
    // waiting for them does not wait for the prefetch
    frag avs[KC / 32];
#pragma unroll
    for (int j = 0; j < KC / 32; ++j)
      avs[j] = (active && arow && j * 32 < valid) ? load_frag_global<T>(arow + kc0 + j * 32 + kq) : E_::zero();
    if (more) load_chunk(kc0 + KC, (int)min<int64_t>(KC, k_end - kc0 - KC));
    if (active) {
#pragma unroll
      for (int j = 0; j < KC / 32; ++j) {
        if (j * 32 >= valid) break;
        const int ks = j * 32;
        const frag av = avs[j];
#pragma unroll
        for (int pi = 0; pi < NPOOL; ++pi)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            if (qb >= nqb) continue;
            const int q = qb * 16 + my_row;
            frag bv;
            if (shared)
              bv = q < r ? lds_frag(c & 1, pi, q, ks + kq) : E_::zero();
            else
              bv = prow[pi][qb] ? load_frag_global<T>(prow[pi][qb] + kc0 + ks + kq) : E_::zero();
            acc[pi][qb] = E_::mma(av, bv, acc[pi][qb]);
          }
      }
    }
    if (more) store_chunk((c + 1) & 1);
  }
  if (!active) return;
  const float sc = a.scaling[l];
  float* hrow_base = a.h + (int64_t)blockIdx.y * a.split_stride + row0 * HS;
  // C layout: lane holds rows 4*(lane/16)+i, column lane%16 of each 16x16 block
#pragma unroll
  for (int pi = 0; pi < NPOOL; ++pi)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int col = qb * 16 + (lane & 15);
      if (col >= a.RP) continue;
      const floatx4 t = acc[pi][qb];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = (lane >> 4) * 4 + i;
        const float v = (qb < nqb && col < r) ? sc * t[i] : 0.0f;
        if (sizeof(T) == 2 && gridDim.y == 1)   // the final h of a bf16 layer: split (store_h_split)
          store_h_split(hrow_base + (int64_t)rr * HS, pi * a.RP + col, v);
        else
          hrow_base[(int64_t)rr * HS + pi * a.RP + col] = v;
      }
    }
}

// h[0] += h[1] + ... + h[S-1] over the padded rows, in split order; with
// split_h (a bf16 layer) the sum is stored split (store_h_split).  A thread
// takes one group of 8 columns.
__global__ void __launch_bounds__(256)
shrink_reduce_kernel(float* __restrict__ h, int64_t split_stride, int splits,
                     const int32_t* __restrict__ num_rows_padded, int HS, int split_h) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= (int64_t)num_rows_padded[0] * HS) return;
  floatx4 v0 = *reinterpret_cast<const floatx4*>(h + i);
  floatx4 v1 = *reinterpret_cast<const floatx4*>(h + i + 4);
  for (int sp = 1; sp < splits; ++sp) {
    v0 += *reinterpret_cast<const floatx4*>(h + sp * split_stride + i);
    v1 += *reinterpret_cast<const floatx4*>(h + sp * split_stride + i + 4);
  }
  if (split_h) {
    bf16x8 hi, lo;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float v = u < 4 ? v0[u] : v1[u - 4];
      hi[u] = (bf16_t)v;
      lo[u] = (bf16_t)(v - (float)hi[u]);
    }
    *reinterpret_cast<bf16x8*>(h + i) = hi;
    *reinterpret_cast<bf16x8*>(h + i + 4) = lo;
  } else {
    *reinterpret_cast<floatx4*>(h + i) = v0;
    *reinterpret_cast<floatx4*>(h + i + 4) = v1;
  }
}

// --------------------------------------------------------------------------
// grouped GEMM with fused LoRA expand
// --------------------------------------------------------------------------
// Output-block traits.  bf16 uses v_mfma_f32_32x32x16_bf16 (32x32 blocks; on
// gfx950 it runs at twice the rate of the 16x16x32 form); fp32 uses eight
// v_mfma_f32_16x16x4_f32 per 32-deep step on 16x16 blocks.  In both, lane l
// feeds row / column (l % BS) with the 8 consecutive K elements starting at
// 8 * (l / BS) of the current KF-deep step.
template <typename T> struct Blk;
template <> struct Blk<bf16_t> {
  static constexpr int BS = 32, KF = 16, ACC = 16;
  typedef floatx16 acc_t;
  __device__ static inline acc_t mma(const bf16x8& a, const bf16x8& b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // row (inside the 32x32 block) of accumulator element v of lane `lane`
  __device__ static inline int row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
};
template <> struct Blk<float> {
  static constexpr int BS = 16, KF = 32, ACC = 4;
  typedef floatx4 acc_t;
  __device__ static inline acc_t mma(const floatx8& a, const floatx8& b, acc_t c) {
    return Elt<float>::mma(a, b, c);
  }
  __device__ static inline int row(int v, int lane) { return 4 * (lane >> 4) + v; }
};

// 16 fp8 e4m3 codes (4 dwords, element 4w+b = byte b of dword w) times a
// block scale, as two bf16x8 fragments: elements 0..7 and 8..15.  The code
// itself converts exactly (every e4m3 value is a bf16 value); the product
// with the scale is rounded to nearest-even bf16.  A positive normal
// power-of-two scale (pow2, wave-uniform) makes the product exact: then the
// scaled conversion instruction, which applies only the scale's exponent,
// gives the same bits at one instruction per two codes.
__device__ __forceinline__ void fp8x16_to_bf16(int4v raw, float sc, bool pow2, bf16x8& lo, bf16x8& hi) {
  typedef float float2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  if (pow2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[w], sc, false);
      const bf16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[w], sc, true);
      bf16x8& d = w < 2 ? lo : hi;
      const int o = 4 * (w & 1);
      d[o + 0] = p0[0]; d[o + 1] = p0[1]; d[o + 2] = p1[0]; d[o + 3] = p1[1];
    }
    return;
  }
  float f[16];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2v p0 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[w], false);
    const float2v p1 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[w], true);
    f[4 * w + 0] = p0[0]; f[4 * w + 1] = p0[1];
    f[4 * w + 2] = p1[0]; f[4 * w + 3] = p1[1];
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    lo[v] = (bf16_t)(f[v] * sc);
    hi[v] = (bf16_t)(f[8 + v] * sc);
  }
}


// Tail split of the gate_up GEMM's persistent schedule.  An XCD's range of n_x
// tiles runs on wx workgroups in q = n_x / wx full rounds and a last round of
// r = n_x % wx tiles; when that round would leave at least 3/4 of the XCD's
// workgroups idle for a whole tile (the 128-token decode batch
// over 256 experts of H = 7168: 34 tiles for 32 workgroups),
// each of its r tiles is handed out instead as S pieces of about nk / S K tiles
// (S r <= wx, at least 2 K tiles a piece).  A piece leaves its partial sums in
// a buffer and gate_up_fixup_kernel adds the S pieces of a tile in order and
// finishes it (SiLU(g) * u).  S = 1: no split.
struct TailSplit {
  int q, r, S;
};
__host__ __device__ inline TailSplit tail_split(int n_x, int wx, int nk) {
  TailSplit t{0, 0, 1};
  if (wx <= 0 || n_x <= 0) return t;
  t.q = n_x / wx;
  t.r = n_x - t.q * wx;
  if (t.r > 0 && 4 * t.r <= wx) t.S = min(wx / t.r, nk / 2);
  if (t.S < 2) t.S = 1;
  return t;
}

// W: weight element, T (bf16 / fp32 weights) or uint8_t (fp8 e4m3 codes with
// 128 x 128 block scales; T = bf16).
// GATE_UP: x rows gathered by pair, gate / up columns paired, SiLU(g) * u to act.
// Otherwise the down form: A rows in sorted order, weighted rows scattered to z;
// DENSE (with !GATE_UP): A rows gathered like gate_up, unit weights, and the
// LoRA expand switches pools at column n_split (a projection whose output is
// two slices with their own LoRA factors).
template <typename T, typename W, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int ROWB, bool GATE_UP,
          bool DENSE = false>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N) gemm_kernel(GemmArgs<T> a) {
  static_assert(!(GATE_UP && DENSE), "dense mode is a form of the down GEMM");
  constexpr bool GATHER = GATE_UP || DENSE;       // A rows are x rows of the rows' pairs
  typedef Elt<T> E_;
  typedef Blk<T> B_;
  typedef typename E_::frag frag;
  typedef typename B_::acc_t acc_t;
  constexpr int BS = B_::BS, KF = B_::KF;
  // ROWB: bytes per LDS tile row = one K tile of one row (64 or 128)
  constexpr int BK = ROWB / sizeof(T);            // K elements per tile
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  constexpr int RPS = 1024 / ROWB;                // rows per 1 KB DMA segment
  static_assert(ROWB == 64 || ROWB == 128 || ROWB == 256, "row size");
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr bool WF8 = sizeof(W) == 1;            // fp8 weights: B rows hold BK one-byte codes
  static_assert(!WF8 || (sizeof(T) == 2 && ROWB >= 128), "fp8 weights with bf16 activations");
  constexpr int ROWB_B = WF8 ? ROWB / 2 : ROWB;   // bytes per LDS row of B
  constexpr int CPR_B = ROWB_B / 16, RPS_B = 1024 / ROWB_B;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB_B;
  constexpr int A_SEGS = A_BYTES / 1024;          // stage: A rows, then B rows
  constexpr int SEGS = (A_BYTES + B_BYTES) / 1024;  // 1 KB segments per stage
  constexpr int SEG_PER_WAVE = SEGS / NWAVES;     // DMA instructions per wave per stage
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // wave tile
  constexpr int MB = WM / BS, NB = WN / BS;
  constexpr int KSUB = BK / KF;
  static_assert(SEGS % NWAVES == 0 && MB >= 1 && NB >= 1, "tile / wave split");
  static_assert(!GATE_UP || (NB % 2) == 0, "gate/up blocks come in pairs");
  static_assert(STAGES >= 2, "ring depth");

  __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];
  __shared__ int ep_pid[BM];      // down epilogue: pair id of each tile row
  __shared__ float ep_w[BM];      // and its router weight
  // fp8 weights: each wave's block scales for the tile's K range, [wave][j][K/128]
  constexpr int MAXKB = 128;      // K / 128 per tile (K <= 16384)
  __shared__ float sc_lds[WF8 ? NWAVES * NB * MAXKB : 1];

  // Persistent tile loop over the logical tile order of tile_table_kernel
  // (expert by expert; inside an expert, groups of about 8 work items whose
  // tiles are column-major, items fastest).  Workgroups are dealt round-robin
  // over the 8 XCDs; each XCD owns a contiguous range of logical tiles, handed
  // out in order by a per-XCD counter, so the tiles resident on one XCD at any
  // time are a sliding window of neighbours sharing x rows and weight columns
  // in its L2.  A workgroup claims its next tile when it starts the current
  // one and loads the next tile's record before the current epilogue.
  const int count = min(a.item_count[0], a.max_items);
  const int total = count * a.n_tiles;
  const int xcd = blockIdx.x % 8;
  const int per_xcd = (total + 7) / 8;
  const int t_begin = xcd * per_xcd, t_end = min(total, t_begin + per_xcd);
  // claims: n_main whole tiles, then (tail split) S K pieces of each tail tile
  constexpr bool TAILS = GATE_UP;
  const int wx = (int)gridDim.x / 8;
  TailSplit ts{0, 0, 1};
  if (TAILS && a.part) ts = tail_split(t_end - t_begin, wx, (int)(a.K / BK));
  const int n_main = ts.S > 1 ? ts.q * wx : max(t_end - t_begin, 0);
  const int n_claims = n_main + (ts.S > 1 ? ts.r * ts.S : 0);
  auto tile_of = [&](int j) -> int {   // logical tile of claim j, clamped to a valid index
    const int t = t_begin + (j < n_main ? j : n_main + (j - n_main) / ts.S);
    return max(min(t, t_end - 1), 0);
  };
  __shared__ int claimed;
  if (threadIdx.x == 0) claimed = atomicAdd(&a.tile_ctr[xcd], 1);
  __syncthreads();
  int jc = __builtin_amdgcn_readfirstlane(claimed);   // this workgroup's claim
  int4 desc = a.tile_tab[tile_of(jc)];
  while (jc < n_claims) {
  int next_claim = 0;
  if (threadIdx.x == 0) next_claim = atomicAdd(&a.tile_ctr[xcd], 1);
  bool published = false;   // the next claim was written to LDS inside the tile
  bool have_next = false;   // next_desc holds the next tile's record
  int4 next_desc;
  [&]() {
  const int col_t = desc.w;
  const int64_t row0 = desc.x;
  const int nrows = desc.y;
  const int e = desc.z;
  if (col_t < 0 || col_t >= a.n_tiles || row0 < 0 || nrows <= 0 || nrows > BM || (nrows & 15) ||
      (row0 & 15) || row0 + nrows > a.cap || e < 0 || e >= a.E)
    return;
  const int split = col_t / a.n_cols;            // K split (split-major: a window shares its x rows)
  const int ntile = col_t - split * a.n_cols;
  const int64_t kper = a.K / a.ksplit;           // K elements per split, a multiple of BK
  // K tiles [kt0, kt0 + nk) of this tile: its split, or one piece of a tail tile
  const int piece = jc >= n_main ? (jc - n_main) % ts.S : -1;
  int kt_lo = 0, nk = (int)(kper / BK);
  if (TAILS && piece >= 0) {
    kt_lo = piece * nk / ts.S;
    nk = (piece + 1) * nk / ts.S - kt_lo;
  }
  const int kt0 = split * (int)(kper / BK) + kt_lo;
  const bool lora_here = a.h != nullptr && split == 0 && piece <= 0;   // the expand is added once
  __syncthreads();  // the previous tile's last LDS reads are done

  // wave index in an SGPR: every wave-level test below is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // lane-derived values are recomputed per tile: the empty asm keeps the
  // compiler from hoisting them out of the persistent loop, where they would
  // stay live (and spill) across the main loop
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane % BS;                     // row / column this lane feeds
  const int lk = 8 * (lane / BS);                 // K offset of its 8 elements

  const int64_t n0 = GATE_UP ? (int64_t)ntile * (BN / 2) : (int64_t)ntile * BN;

  // ---- DMA source offsets --------------------------------------------------
  // Stage layout: LDS row r < BM holds A row r, row BM + n holds B row n, 128
  // bytes (one K tile) each, its eight 16-byte chunks permuted by
  // slot = chunk ^ swz(row) so fragment reads of 16 / 32 consecutive rows hit
  // distinct banks.  Wave w fills segments w*SEG_PER_WAVE.. (8 rows each);
  // lane l of a segment writes row 8*seg + l/8, slot l%8, i.e. global chunk
  // (l%8) ^ swz(row).  Rows outside the tile (pads, rows past nrows, columns
  // past n_out) load a valid row instead: MFMA rows / columns are
  // independent and those results are never stored.
  // 16 lanes read 16 consecutive rows at one chunk: with 256-byte rows every
  // row starts at the same bank, with 128-byte rows rows 2 apart share banks,
  // with 64-byte rows rows 4 apart
  auto swz = [](int row) -> int {
    return ROWB == 256 ? (row & 15) : ROWB == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
  };
  // B rows: 64-byte rows (fp8) swizzle like 64-byte A rows would
  auto swzb = [](int n) -> int {
    return ROWB_B == 128 ? ((n >> 1) & 7) : ((n >> 2) & 3);
  };
  // 64-bit bases; the per-lane DMA offsets below are 32-bit.  A non-gathered
  // A operand (act) starts at the tile's first row, so its offsets stay below
  // BM * K elements whatever the batch; gathered x rows and one expert's
  // weights are kept under 4 GiB by the host checks.
  const T* a_base = GATHER ? a.a_src : a.a_src + row0 * a.K;
  const W* b_base = static_cast<const W*>(a.w) + (int64_t)e * a.w_rows * a.K;
  // global row (of a_base for row < BM, of b_base otherwise) behind LDS row `row`
  auto grow_of = [&](int row, int pid_in) -> int64_t {
    if (row < BM) {
      const int r = row;
      if (GATHER) {
        const int pid = r < nrows ? pid_in : a.P;
        return pid < a.P ? pid / a.top_k : 0;
      }
      return r < nrows ? r : 0;   // relative to the tile's first row
    }
    const int n = row - BM;
    if (GATE_UP) {
      const int64_t col = n0 + (n % (BN / 2));
      return col < a.n_out ? ((n < BN / 2) ? col : a.n_out + col) : 0;
    }
    return n0 + n < a.n_out ? n0 + n : 0;
  };
  uint32_t src_off[SEG_PER_WAVE];   // byte offsets from a_base / b_base
  int pidv[SEG_PER_WAVE];
  if (GATHER) {
    // pair ids of the gathered A rows: clamped, unconditional loads, issued together
#pragma unroll
    for (int i = 0; i < SEG_PER_WAVE; ++i) {
      const int row = (wave * SEG_PER_WAVE + i) * RPS + lane / CPR;
      pidv[i] = a.sorted_ids[row0 + min(min(row, BM - 1), nrows - 1)];
    }
  }
  // LoRA slot table of this wave's row blocks, loaded with the pair ids and
  // resolved before the first DMA, so the expand (ahead of the K loop) waits
  // for its operands together with the ring's first stages: lg[i][g] = slot
  // of 16-row group g of block i (-1: none or rank 0), rg[i][g] its rank;
  // p0[i] = slot of the block's first pass (its first served group), r0[i]
  // its rank.
  constexpr int NG = BS / 16;
  int lg[MB][NG], rg[MB][NG], p0[MB], r0[MB];
  if (lora_here) {
    // row numbers fit in 32 bits: a 32-bit divide each, and all the loads go
    // out before the first is used (a 64-bit divide's branches kept each load
    // behind the previous one's wait: one round trip per group)
    int srv[MB][NG];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int r16 = max(min(wm * WM + i * BS + 16 * g, nrows - 16), 0);   // clamped: loads stay unconditional
        srv[i][g] = a.slot_rank[((uint32_t)row0 + (uint32_t)r16) / (uint32_t)a.BM_tile];
      }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int rb = wm * WM + i * BS;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int sr = srv[i][g];
        const bool on = rb + 16 * g < nrows && sr >= 0;
        lg[i][g] = on ? (sr & 0xFFFF) : -1;
        rg[i][g] = on ? (sr >> 16) : 0;
      }
      int l = -1, r = 0;
#pragma unroll
      for (int g = NG - 1; g >= 0; --g)
        if (lg[i][g] >= 0) { l = lg[i][g]; r = rg[i][g]; }
      p0[i] = l;
      r0[i] = r;
    }
  }
#pragma unroll
  for (int i = 0; i < SEG_PER_WAVE; ++i) {
    const int seg = wave * SEG_PER_WAVE + i;
    if (seg < A_SEGS) {
      const int row = seg * RPS + lane / CPR;
      const int kc = (lane % CPR) ^ swz(row);
      src_off[i] = (uint32_t)((grow_of(row, pidv[i]) * a.K + kc * E_::kChunk) * sizeof(T));
    } else {
      // B row n of the stage (LDS row BM + n; swz(BM + n) == swzb(n) as BM % 16 == 0)
      const int n = (seg - A_SEGS) * RPS_B + lane / CPR_B;
      const int kc = (lane % CPR_B) ^ swzb(n);
      src_off[i] = (uint32_t)(grow_of(BM + n, 0) * a.K * (int64_t)sizeof(W) + kc * 16);
    }
  }
  // Publish the next claim now: every wave read the current one before the
  // barrier above, and the K loop's barriers make this write visible before
  // the end of the tile.  (The claim's load has completed: the pair-id loads
  // issued after it were just waited for.)
  if (threadIdx.x == 0) claimed = next_claim;
  published = true;
  if (lora_here) {
    // the slot table is needed by the expand's loads: wait for it here, not
    // after the DMA below (the counter would then take the DMA along)
#pragma unroll
    for (int i = 0; i < MB; ++i) asm volatile("" ::"v"(p0[i]), "v"(r0[i]));
  }

  const uint32_t lds_u32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  // this wave's DMA instructions [I0, I1) of one stage
  auto issue_part = [&](auto i0_c, auto i1_c, int stage_k, int buf) {
    constexpr int I0 = decltype(i0_c)::value, I1 = decltype(i1_c)::value;
    const uint32_t ktile = (uint32_t)(kt0 + stage_k);
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int seg = wave * SEG_PER_WAVE + i;
      const bool is_a = seg < A_SEGS;
      const void* base = is_a ? (const void*)a_base : (const void*)b_base;
      dma16(base, src_off[i] + ktile * (is_a ? ROWB : ROWB_B), lds_u32 + buf * STAGE_BYTES + seg * 1024);
    }
  };
  auto issue_stage = [&](int stage_k, int buf) {
    issue_part(std::integral_constant<int, 0>{}, std::integral_constant<int, SEG_PER_WAVE>{},
               stage_k, buf);
  };
  // one frag (8 K elements starting at kel) of LDS row `row`
  auto lfrag = [&](const char* base, int row, int kel) -> frag {
    if constexpr (sizeof(T) == 2) {
      const int kc = kel >> 3;
      return *reinterpret_cast<const frag*>(base + row * ROWB + ((kc ^ swz(row)) * 16));
    } else {
      const int kc = kel >> 2;
      floatx4 lo = *reinterpret_cast<const floatx4*>(base + row * ROWB + ((kc ^ swz(row)) * 16));
      floatx4 hi = *reinterpret_cast<const floatx4*>(base + row * ROWB + (((kc + 1) ^ swz(row)) * 16));
      frag f;
      f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
      f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
      return f;
    }
  };
  // wave-local column block j -> first output column (act column for gate_up)
  auto col_of = [&](int j) -> int64_t {
    if (GATE_UP) return n0 + wn * (WN / 2) + (j % (NB / 2)) * BS;
    return n0 + wn * WN + j * BS;
  };
  // fp8 weights: this wave's block scales of the K split's range into sc_lds
  // (the wave reads only its own entries, so no barrier is needed); a piece
  // of a tail tile reads them from its first K tile kt_lo on
  auto fill_scales = [&]() {
    const int nkb = (int)(kper / 128);
    const int64_t kbs = a.K / 128, rows128 = a.w_rows / 128;
    for (int idx = lane; idx < NB * nkb; idx += 64) {
      const int j = idx / nkb, kb = idx - j * nkb;
      const int64_t col = col_of(j);
      int64_t wrow = (GATE_UP && j >= NB / 2) ? a.n_out + col : col;
      wrow = min(wrow, a.w_rows - 1);
      sc_lds[(wave * NB + j) * MAXKB + kb] =
          a.w_scale[((int64_t)e * rows128 + wrow / 128) * kbs + (int64_t)split * nkb + kb];
    }
  };
  // LDS row of B for this lane in column block j
  auto b_row_of = [&](int j) -> int {
    if (GATE_UP) {
      const int n = wn * (WN / 2) + (j % (NB / 2)) * BS + lrow;
      return BM + ((j < NB / 2) ? n : BN / 2 + n);
    }
    return BM + wn * WN + j * BS + lrow;
  };

  acc_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < B_::ACC; ++v) acc[i][j][v] = 0.0f;

  // Fragments are double-buffered in registers: the LDS reads of sub-step
  // ks+1 are issued before the MFMAs of sub-step ks.
  frag fa[2][MB], fb[2][NB];
  // fp8 weights: a lane's 8 K elements of sub-step ks are K offsets
  // 32*(ks/2) + 16*h + 8*(ks%2) (h = lane half), the same for A and B, so one
  // 16-byte read of a B row serves sub-steps ks and ks+1.  fbq[pair][half][j]
  // holds the converted fragments; sck[j] the K tile's block scales.
  frag fbq[2][2][NB];
  float sck[NB];
  bool sc_pow2[NB];
  auto load_frags = [&](const char* base, int ks, int set) {
    const int kel = WF8 ? 32 * (ks >> 1) + 2 * lk + 8 * (ks & 1) : ks * KF + lk;
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[set][i] = lfrag(base, wm * WM + i * BS + lrow, kel);
    if constexpr (!WF8) {
#pragma unroll
      for (int j = 0; j < NB; ++j) fb[set][j] = lfrag(base, b_row_of(j), kel);
    } else {
      if ((ks & 1) == 0) {
        const int kc = 2 * (ks >> 1) + (lk >> 3);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int n = b_row_of(j) - BM;
          const int4v raw = *reinterpret_cast<const int4v*>(base + A_BYTES + n * ROWB_B + ((kc ^ swzb(n)) * 16));
          fp8x16_to_bf16(raw, sck[j], sc_pow2[j], fbq[(ks >> 1) & 1][0][j], fbq[(ks >> 1) & 1][1][j]);
        }
      }
    }
  };
  // ---- main loop: STAGES-deep LDS ring fed by DMA, one barrier per K tile --
  // Step s: wait for this wave's loads of tile s, barrier (everyone's tile s
  // has landed and everyone is done with tile s-1), refill the slot of tile
  // s-1 with tile s+STAGES-1, multiply tile s.
  //
  // The loop is instantiated twice: with every row block of the wave live
  // (no test near the MFMAs, so the compiler interleaves them freely with
  // the LDS reads), and for a short last item of an expert, where row blocks
  // wholly past nrows skip their MFMAs (a scalar test: the wave index is
  // uniform).
  auto main_loop = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    auto mma_frags = [&](int ks) {
      const int set = ks & 1;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (!FULL && wm * WM + i * BS >= nrows) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = B_::mma(fa[set][i], WF8 ? fbq[(ks >> 1) & 1][ks & 1][j] : fb[set][j], acc[i][j]);
      }
    };
    // Multiply the stage in ring slot buf; when next_k >= 0 also issue the
    // DMA of K tile next_k into slot next_buf, spread over the sub-steps.
    // Instruction order is pinned with scheduling barriers: the fragment
    // reads of sub-step ks+1 and a share of the DMA go out before the MFMAs
    // of sub-step ks, so LDS latency and DMA issue hide behind MFMA work.
    auto compute = [&](int buf, int next_k, int next_buf, int kt) {
      const char* base = lds + buf * STAGE_BYTES;
      if constexpr (WF8) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          // one scale per wave (its columns share a 128-row block): a scalar
          const uint32_t bits = __builtin_amdgcn_readfirstlane(
              __builtin_bit_cast(uint32_t, sc_lds[(wave * NB + j) * MAXKB + ((kt_lo + kt) * BK) / 128]));
          sck[j] = __builtin_bit_cast(float, bits);
          const uint32_t ex = (bits >> 23) & 0xFF;
          sc_pow2[j] = (bits & 0x807FFFFFu) == 0 && ex != 0 && ex != 0xFF;
        }
      }
      load_frags(base, 0, 0);
      static_for<KSUB>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        constexpr int d0 = ks * SEG_PER_WAVE / KSUB, d1 = (ks + 1) * SEG_PER_WAVE / KSUB;
        __builtin_amdgcn_sched_barrier(0);
        if (next_k >= 0)
          issue_part(std::integral_constant<int, d0>{}, std::integral_constant<int, d1>{},
                     next_k, next_buf);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ks + 1 < KSUB) load_frags(base, ks + 1, (ks + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_frags(ks);
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    int s = 0;
    // steady state: STAGES-1 tiles are in flight at each wait
    for (; s + STAGES - 1 < nk; ++s) {
      wait_vm_barrier<(STAGES - 2) * SEG_PER_WAVE>();
      compute(s % STAGES, s + STAGES - 1, (s + STAGES - 1) % STAGES, s);
    }
    // drain: no more loads to issue
    for (; s < nk; ++s) {
      wait_vm_barrier<0>();
      compute(s % STAGES, -1, 0, s);
    }
  };
  // the ring's first STAGES-1 stages: all but the last before the expand, the
  // last right after it (the expand waits for every load issued before its
  // own, the inline-asm DMA included, so that stage then stays in flight
  // into the K loop)
  constexpr int PRE = STAGES > 2 ? STAGES - 2 : 1;
  // every load issued so far has been used and the previous tile's stores
  // have been waited for by now; a wait the compiler sees keeps it from
  // placing one after these DMAs (it does not count them, and a wait there
  // drains them before the expand's loads go out)
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#pragma unroll
  for (int st = 0; st < PRE; ++st)
    if (st < nk) issue_stage(st, st);
  if constexpr (WF8) fill_scales();

  // ---- LoRA expand: acc = h[rows, q] * Bpool[l, e, q, cols], before the K loop --
  // Its operand loads go out right after the ring's first stages, so both
  // latencies overlap, and its MFMAs start the accumulators.
  // Each 16-row group has its own slot; a BS-row block holds BS/16 groups, so
  // every distinct slot of the block gets its own pass with the rows of the
  // other slots masked to zero.
  if constexpr (sizeof(T) == 2) {
    // bf16: one pass per distinct slot of the wave's 16-row groups (first-seen
    // order; usually one).  Per pass and 16-deep rank step the wave loads the
    // B tile once for all its row blocks -- 16 rank rows x 32 columns per
    // column block, one 16-byte load per lane -- and turns it into MFMA
    // fragments through a wave-private scratch in the ring slot that the
    // prologue leaves idle (the K loop refills it only after its first
    // barrier).  Rank rows >= r and columns >= n_out are zero, never read.
    if (lora_here) {
      static_assert(BS == 32 && KF == 16, "bf16 expand layout");
      constexpr int NSLOT = MB * NG;
      constexpr int BTS = 24;   // elements per column of the scratch: 16 rank rows + pad (48 B)
      static_assert(NWAVES * NB * 32 * BTS * (int)sizeof(T) <= STAGE_BYTES, "B scratch fits a ring slot");
      T* bt = reinterpret_cast<T*>(lds + (STAGES - 1) * STAGE_BYTES) + wave * (NB * 32 * BTS);
      // column block j: second pool (up columns; dense: the second output slice)?
      auto second_of = [&](int j) -> bool {
        return GATE_UP ? j >= NB / 2 : (DENSE && a.n_split < a.n_out && col_of(j) >= a.n_split);
      };
      const bool two_h = GATE_UP || (DENSE && a.HS > a.RP);   // h has a second half
      const int qq = lane >> 2, ch = lane & 3;                 // B tile load: rank row, 8-column chunk
      static_for<NSLOT>([&](auto C) {
        constexpr int c = decltype(C)::value;
        const int l = lg[c / NG][c % NG];
        bool first = l >= 0;
#pragma unroll
        for (int c2 = 0; c2 < c; ++c2) first = first && lg[c2 / NG][c2 % NG] != l;
        if (!first) return;
        const int r = rg[c / NG][c % NG];
        const int nks = (r + KF - 1) / KF;
        // blocks holding slot l
        bool has[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          has[i] = false;
#pragma unroll
          for (int g = 0; g < NG; ++g) has[i] = has[i] || lg[i][g] == l;
        }
        // loads of rank step ks: B tile rows ks*16 .. ks*16+15 of slot l (this
        // lane's 8 columns of each block), and h of this lane's row in every
        // block holding slot l (other rows: the block's first row, zeroed later)
        auto load_ks = [&](int ks, int4v* braw, floatx8* hg, floatx8* hu) {
          const int q = ks * KF + qq;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const bool sec = second_of(j);
            const T* pool = sec ? a.b_pool1 : a.b_pool0;
            const int64_t c0 = DENSE && sec ? a.n_split : 0;
            const int64_t width = DENSE ? (sec ? a.n_out - a.n_split : a.n_split) : a.n_out;
            const int64_t col = col_of(j) + 8 * ch;
            braw[j] = int4v{0, 0, 0, 0};
            if (q < r && col < a.n_out)
              braw[j] = *reinterpret_cast<const int4v*>(pool + (((int64_t)l * a.E + e) * a.R + q) * width + (col - c0));
          }
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            const int rb = wm * WM + i * BS;
            const bool mine = lg[i][lrow / 16] == l;
            const float* hrow = a.h + (row0 + min(rb + (mine ? lrow : 0), nrows - 1)) * a.HS;
            const int q0 = ks * KF + lk;
            if (has[i]) {
              hg[i] = *reinterpret_cast<const floatx8*>(hrow + q0);
              hu[i] = two_h ? *reinterpret_cast<const floatx8*>(hrow + a.RP + q0) : hg[i];
            }
          }
        };
        auto proc_ks = [&](const int4v* braw, const floatx8* hg, const floatx8* hu) {
          // transpose through the scratch: (rank row, column n of block j) at bt[(j*32 + n)*BTS + row]
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, braw[j]);
#pragma unroll
            for (int t = 0; t < 8; ++t) bt[(j * 32 + 8 * ch + t) * BTS + qq] = v[t];
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          frag bfr[NB];
#pragma unroll
          for (int j = 0; j < NB; ++j) bfr[j] = *reinterpret_cast<const frag*>(bt + (j * 32 + lrow) * BTS + lk);
          static_for<MB>([&](auto I) {
            constexpr int i = decltype(I)::value;
            if (!has[i]) return;
            const bool mine = lg[i][lrow / 16] == l;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              // h arrives split (store_h_split): the 32 bytes of this lane's 8
              // ranks are their 8 bf16 high parts, then the 8 low parts; rows
              // of another slot contribute zero
              const floatx8 hv = second_of(j) ? hu[i] : hg[i];
              const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
              const floatx4 h0 = {hv[0], hv[1], hv[2], hv[3]}, h1 = {hv[4], hv[5], hv[6], hv[7]};
              const frag hi = __builtin_bit_cast(frag, mine ? h0 : z4);
              const frag lo = __builtin_bit_cast(frag, mine ? h1 : z4);
              acc[i][j] = B_::mma(hi, bfr[j], acc[i][j]);
              acc[i][j] = B_::mma(lo, bfr[j], acc[i][j]);
            }
          });
        };
        // two rank steps per round, their loads issued together (one in the
        // dense form, whose gathered rows leave no registers for a second set)
        constexpr int PER_ROUND = DENSE ? 1 : 2;
        for (int ks = 0; ks < nks; ks += PER_ROUND) {
          int4v b0[NB], b1[NB];
          floatx8 hg0[MB], hu0[MB], hg1[MB], hu1[MB];
          load_ks(ks, b0, hg0, hu0);
          const bool two = PER_ROUND == 2 && ks + 1 < nks;
          if (two) load_ks(ks + 1, b1, hg1, hu1);
          proc_ks(b0, hg0, hu0);
          if (two) proc_ks(b1, hg1, hu1);
        }
      });
    }
  } else if (lora_here) {
    constexpr int MAXKS = 64 / KF;   // RP <= 64
    // dense mode: column block j belongs to the second output slice
    auto dense_second = [&](int j) -> bool {
      return DENSE && a.n_split < a.n_out && col_of(j) >= a.n_split;
    };
    // rank step ks of the pass serving slot l in block i: h of this lane's
    // row (the block's first row, zeroed later, if its group is not served)
    // and the B^T values of its column (rows q >= r never read: q clamped)
    auto load_step = [&](int i, int l, int r, int ks, floatx8& hg, floatx8& hu, frag* bfv) {
      const int rb = wm * WM + i * BS;
      const int q0 = ks * KF + lk;
      const bool mine = lg[i][lrow / 16] == l;
      const float* hrow = a.h + (row0 + min(rb + (mine ? lrow : 0), nrows - 1)) * a.HS;
      hg = *reinterpret_cast<const floatx8*>(hrow + q0);
      // the second h half exists for gate_up and for a dense output with two slices
      hu = (GATE_UP || (DENSE && a.HS > a.RP)) ? *reinterpret_cast<const floatx8*>(hrow + a.RP + q0) : hg;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        // second pool: the up columns, or (dense, when the second slice is not
        // empty) the columns past n_split; blocks past n_out (never stored)
        // clamp into the last slice that exists
        const bool up = GATE_UP ? j >= NB / 2 : dense_second(j);
        const T* pool = up ? a.b_pool1 : a.b_pool0;
        const int64_t c0 = DENSE && up ? a.n_split : 0;           // the pool's first column
        const int64_t width = DENSE ? (up ? a.n_out - a.n_split : a.n_split) : a.n_out;
        const int64_t col = min(col_of(j) + lrow, a.n_out - 1) - c0;
        const T* pb = pool + (((int64_t)max(l, 0) * a.E + e) * a.R) * width + col;
#pragma unroll
        for (int v = 0; v < 8; ++v) bfv[j][v] = pb[(int64_t)min(q0 + v, max(r, 1) - 1) * width];
      }
    };
    auto mma_step = [&](auto I, int l, int r, int ks, floatx8 hg, floatx8 hu, frag* bfv) {
      constexpr int i = decltype(I)::value;
      const int q0 = ks * KF + lk;
      const bool mine = lg[i][lrow / 16] == l;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        if (!mine) { hg[v] = 0.0f; hu[v] = 0.0f; }
#pragma unroll
        for (int j = 0; j < NB; ++j)
          if (q0 + v >= r || col_of(j) + lrow >= a.n_out) bfv[j][v] = E_::from_float(0.0f);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const bool up = GATE_UP ? j >= NB / 2 : dense_second(j);
        const floatx8& hv = up ? hu : hg;
        acc[i][j] = B_::mma(hv, bfv[j], acc[i][j]);   // fp32 layers: h in fp32
      }
    };
    // one pass: rank steps from ks0 on (ks0 = 1: step 0 already done)
    auto pass_rest = [&](auto I, int l, int rk, int ks0) {
      constexpr int i = decltype(I)::value;
      const int r = rk;
      const int nks = (r + KF - 1) / KF;
#pragma unroll
      for (int ks = 1; ks < MAXKS; ++ks) {
        if (ks < ks0 || ks >= nks) continue;
        floatx8 hg, hu;
        frag bfv[NB];
        load_step(i, l, r, ks, hg, hu, bfv);
        mma_step(I, l, r, ks, hg, hu, bfv);
      }
    };
    floatx8 hg0[MB], hu0[MB];
    frag bf0[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) load_step(i, p0[i], r0[i], 0, hg0[i], hu0[i], bf0[i]);
    static_for<MB>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if (p0[i] < 0) return;
      mma_step(I, p0[i], r0[i], 0, hg0[i], hu0[i], bf0[i]);
      pass_rest(I, p0[i], r0[i], 1);
    });
    // further passes: groups whose slot differs from every earlier group's
    static_for<MB>([&](auto I) {
      constexpr int i = decltype(I)::value;
#pragma unroll
      for (int g = 1; g < NG; ++g) {
        const int l = lg[i][g];
        bool seen = l < 0 || l == p0[i];
#pragma unroll
        for (int g2 = 0; g2 < g; ++g2) seen = seen || lg[i][g2] == l;
        if (seen) continue;
        const int r = rg[i][g];
        floatx8 hg, hu;
        frag bfv[NB];
        load_step(i, l, r, 0, hg, hu, bfv);
        mma_step(I, l, r, 0, hg, hu, bfv);
        pass_rest(I, l, r, 1);
      }
    });
  }

#pragma unroll
  for (int st = PRE; st < STAGES - 1; ++st)
    if (st < nk) issue_stage(st, st);
  if (wm * WM + WM <= nrows)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});
  __builtin_amdgcn_s_barrier();   // everyone is done reading the ring

  // the next tile's record, loaded now so that it has arrived when the
  // epilogue's stores are done (the claim was published before the K loop,
  // whose barriers made it visible)
  next_desc = a.tile_tab[tile_of(__builtin_amdgcn_readfirstlane(claimed))];
  have_next = true;

  // a piece of a tail tile: its partial sums go out as they sit in the
  // registers (for each register, the wave's 64 lanes write 256 contiguous
  // bytes); gate_up_fixup_kernel adds the pieces in order and finishes the tile
  if constexpr (TAILS) {
    if (piece >= 0) {
      float* dst = a.part + (size_t)(xcd * wx + (jc - n_main)) * (BM * BN) +
                   (size_t)wave * (MB * NB * B_::ACC * 64) + lane;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int v = 0; v < B_::ACC; ++v) dst[((i * NB + j) * B_::ACC + v) * 64] = acc[i][j][v];
      return;
    }
  }

  // ---- epilogue -------------------------------------------------------------
  // Results go through this wave's own LDS region (the ring is idle after the
  // barrier that ended the K loop) so that every lane stores 16 contiguous
  // bytes: a lane's accumulators hold one column of several rows.
  constexpr int CH = 16 / (GATE_UP ? (int)sizeof(T) : 4);   // elements per 16-byte chunk (of fp32 for z)
  // z of a bf16 layer in 24-bit form (fp24_pack4); fp32 layers and the dense
  // projection (whose z is its output) keep fp32
  constexpr bool Z24 = sizeof(T) == 2 && !DENSE;
  if (GATE_UP) {
    // act = SiLU(gate) * up, [WM rows][WN/2 cols] of T per wave
    constexpr int EW = WN / 2;
    static_assert(NWAVES * WM * EW * sizeof(T) <= STAGES * STAGE_BYTES, "epilogue staging fits");
    T* ep = reinterpret_cast<T*>(lds) + wave * (WM * EW);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB / 2; ++j)
#pragma unroll
        for (int v = 0; v < B_::ACC; ++v) {
          const float g = acc[i][j][v], u = acc[i][j + NB / 2][v];
          ep[(i * BS + B_::row(v, lane)) * EW + j * BS + lrow] = E_::from_float(silu_f(g) * u);
        }
    constexpr int CPRW = EW / CH;   // chunks per row
#pragma unroll
    for (int c = lane; c < WM * CPRW; c += 64) {
      const int r = c / CPRW, cc = c % CPRW;
      const int rloc = wm * WM + r;
      const int64_t col = n0 + wn * EW + cc * CH;
      if (rloc >= nrows || col >= a.n_out) continue;
      const int4v vv = *reinterpret_cast<const int4v*>(ep + r * EW + cc * CH);
      *reinterpret_cast<int4v*>(a.act + (row0 + rloc) * a.n_out + col) = vv;
    }
  } else {
    // pair ids and router weights of the tile's rows, staged once in LDS
    for (int r = threadIdx.x; r < BM; r += 64 * NWAVES) {
      const int pid = a.sorted_ids[row0 + min(r, nrows - 1)];
      ep_pid[r] = r < nrows ? pid : a.P;
      ep_w[r] = DENSE ? 1.0f : a.topk_weights[min(pid, a.P - 1)];
    }
    // the unweighted results, [WM rows][WN cols] fp32 per wave
    static_assert(NWAVES * WM * WN * 4 <= STAGES * STAGE_BYTES, "epilogue staging fits");
    float* ep = reinterpret_cast<float*>(lds) + wave * (WM * WN);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < B_::ACC; ++v)
          ep[(i * BS + B_::row(v, lane)) * WN + j * BS + lrow] = acc[i][j][v];
    __syncthreads();   // ep_pid / ep_w are written by other waves
    constexpr int CPRW = WN / CH;
#pragma unroll 4
    for (int c = lane; c < WM * CPRW; c += 64) {
      const int r = c / CPRW, cc = c % CPRW;
      const int rloc = wm * WM + r;
      const int64_t col = n0 + wn * WN + cc * CH;
      if (rloc >= nrows || col >= a.n_out) continue;
      const int pid = ep_pid[rloc];
      if (pid >= a.P) continue;
      const float wgt = ep_w[rloc];
      floatx4 vv = *reinterpret_cast<const floatx4*>(ep + r * WN + cc * CH);
#pragma unroll
      for (int q = 0; q < 4; ++q) vv[q] = wgt * vv[q];
      const int64_t zi = ((int64_t)split * a.P + pid) * a.n_out + col;
      if constexpr (Z24)   // 4 values in 12 bytes
        *reinterpret_cast<u32x3*>(static_cast<char*>(a.z) + zi * 3) = fp24_pack4(vv);
      else
        *reinterpret_cast<floatx4*>(static_cast<float*>(a.z) + zi) = vv;
    }
  }
  }();
  if (!published) {   // a skipped tile: publish here
    __syncthreads();   // everyone has read the current claim
    if (threadIdx.x == 0) claimed = next_claim;
    __syncthreads();
  }
  jc = __builtin_amdgcn_readfirstlane(claimed);
  if (!have_next) next_desc = a.tile_tab[tile_of(jc)];
  desc = next_desc;
  }  // persistent tile loop
}

// Finish the tail tiles that gemm_kernel<..., GATE_UP> split into K pieces.
// blockIdx.y = xcd * max(wx / 4, 1) + u names the u-th tail tile of that XCD
// (wx = gemm_grid / 8, the GEMM's workgroups per XCD); each thread takes one
// (gate, up) pair of registers of the GEMM's layout, adds its partial sums over
// the pieces in piece order (the result does not depend on which piece ended
// last) and writes SiLU(gate) * up to act.
template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int ROWB>
__global__ void __launch_bounds__(256) gate_up_fixup_kernel(GemmArgs<T> a, int gemm_grid) {
  typedef Elt<T> E_;
  typedef Blk<T> B_;
  constexpr int BS = B_::BS, ACC = B_::ACC;
  constexpr int BK = ROWB / sizeof(T);
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MB = WM / BS, NB = WN / BS;
  const int wx = gemm_grid / 8;
  const int maxr = max(wx / 4, 1);
  const int xcd = blockIdx.y / maxr, u = blockIdx.y % maxr;
  const int t = blockIdx.x * 256 + threadIdx.x;   // register pair of the tile
  if (xcd >= 8 || !a.part || t >= BM * BN / 2) return;
  const int count = min(a.item_count[0], a.max_items);
  const int total = count * a.n_tiles;
  const int per_xcd = (total + 7) / 8;
  const int t_begin = xcd * per_xcd, t_end = min(total, t_begin + per_xcd);
  const TailSplit ts = tail_split(t_end - t_begin, wx, (int)(a.K / BK));
  if (ts.S < 2 || u >= ts.r) return;
  const int4 desc = a.tile_tab[t_begin + ts.q * wx + u];
  const int col_t = desc.w;
  const int64_t row0 = desc.x;
  const int nrows = desc.y;
  const int e = desc.z;
  // the GEMM skipped such records (no pieces were written)
  if (col_t < 0 || col_t >= a.n_tiles || row0 < 0 || nrows <= 0 || nrows > BM || (nrows & 15) ||
      (row0 & 15) || row0 + nrows > a.cap || e < 0 || e >= a.E)
    return;
  // t = (((wave * MB + i) * NB/2 + j) * ACC + v) * 64 + lane, j < NB/2 (gate);
  // its up partner is column block j + NB/2
  const int lane = t % 64;
  int rest = t / 64;
  const int v = rest % ACC;
  rest /= ACC;
  const int j = rest % (NB / 2);
  rest /= NB / 2;
  const int i = rest % MB, wave = rest / MB;
  const size_t og = ((((size_t)wave * MB + i) * NB + j) * ACC + v) * 64 + lane;
  const size_t ou = og + (size_t)(NB / 2) * ACC * 64;
  const float* src = a.part + (size_t)(xcd * wx + u * ts.S) * (BM * BN);
  float g = 0.0f, up = 0.0f;
#pragma unroll 8
  for (int s = 0; s < ts.S; ++s) {
    g += src[(size_t)s * (BM * BN) + og];
    up += src[(size_t)s * (BM * BN) + ou];
  }
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int r = wm * WM + i * BS + B_::row(v, lane);
  const int64_t col = (int64_t)col_t * (BN / 2) + wn * (WN / 2) + j * BS + lane % BS;
  if (r < nrows && col < a.n_out) a.act[(row0 + r) * a.n_out + col] = E_::from_float(silu_f(g) * up);
}

// --------------------------------------------------------------------------
// combine: y[t, c] = sum_j sum_q z[q, t*k + j, c]  (j, then the down GEMM's
// K splits q, in order, fp32).  z in fp32, or (Z24) in the 24-bit form of a
// bf16 layer, 4 columns in 12 bytes; a thread takes 4 columns.
// --------------------------------------------------------------------------
template <bool Z24, typename OutT>
__global__ void __launch_bounds__(256)
combine_kernel(const void* __restrict__ z, OutT* __restrict__ y, int64_t T_, int k, int64_t H,
               int nsplit, int64_t split_stride) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= T_ * H) return;
  const int64_t t = i / H, c = i % H;
  floatx4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j)
    for (int q = 0; q < nsplit; ++q) {   // pair j's K splits, in order
      const int64_t zi = q * split_stride + (t * k + j) * H + c;
      if constexpr (Z24)
        s += fp24_unpack4(*reinterpret_cast<const u32x3*>(static_cast<const char*>(z) + zi * 3));
      else
        s += *reinterpret_cast<const floatx4*>(static_cast<const float*>(z) + zi);
    }
#pragma unroll
  for (int q = 0; q < 4; ++q) y[i + q] = Elt<OutT>::from_float(s[q]);
}

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------
template <typename T> struct TileCfg;
#ifndef MOELORA_BF16_BM
#define MOELORA_BF16_BM 128
#endif
#ifndef MOELORA_BF16_BN
#define MOELORA_BF16_BN 256
#endif
// 4 x 2 waves (32 rows x 128 columns each): a wave's rows span two 16-row
// align blocks, so the LoRA expand makes at most two passes (one per slot)
// instead of four; measured against 2 x 4 on decode and fine-grained batches:
// GEMM stages 0.5-3% faster, from fewer expand passes
#ifndef MOELORA_BF16_WM
#define MOELORA_BF16_WM 4
#endif
#ifndef MOELORA_BF16_WN
#define MOELORA_BF16_WN 2
#endif
#ifndef MOELORA_BF16_STAGES
#define MOELORA_BF16_STAGES 3
#endif
#ifndef MOELORA_BF16_ROWB
#define MOELORA_BF16_ROWB 128
#endif
#ifndef MOELORA_BF16_BN_DOWN
#define MOELORA_BF16_BN_DOWN MOELORA_BF16_BN
#endif
#ifndef MOELORA_BF16_STAGES_DOWN
#define MOELORA_BF16_STAGES_DOWN MOELORA_BF16_STAGES
#endif
template <> struct TileCfg<bf16_t> {
  static constexpr int BM = MOELORA_BF16_BM, BN = MOELORA_BF16_BN, WM = MOELORA_BF16_WM,
                       WN = MOELORA_BF16_WN, STAGES = MOELORA_BF16_STAGES,
                       ROWB = MOELORA_BF16_ROWB, PER_CU = 1;
  static constexpr int BN_DOWN = MOELORA_BF16_BN_DOWN, STAGES_DOWN = MOELORA_BF16_STAGES_DOWN;
};
// fp8 e4m3 weights (bf16 activations), the same 128 x 256 tile.  Batches
// with many pairs per expert (prefill) take 128-deep K tiles, so a weight row
// is fetched 128 bytes at a time (256-byte x rows), in two 64 KB stages;
// decode-sized batches take 64-deep K tiles in a 4-deep ring of 32 KB stages,
// which starts each short tile sooner.  Either ring is 128 KB, which also
// holds the down epilogue's fp32 staging.
struct Fp8Cfg {
  static constexpr int BM = 128, BN = 256, WM = 2, WN = 4, STAGES = 2, ROWB = 256, PER_CU = 1;
};
struct Fp8DecodeCfg {
  static constexpr int BM = 128, BN = 256, WM = 2, WN = 4, STAGES = 4, ROWB = 128, PER_CU = 1;
};
#ifndef MOELORA_FP8_DEEP_K_MIN_PAIRS_PER_EXPERT
#define MOELORA_FP8_DEEP_K_MIN_PAIRS_PER_EXPERT 64
#endif
static_assert(Fp8Cfg::BM == TileCfg<bf16_t>::BM && Fp8Cfg::BN == TileCfg<bf16_t>::BN &&
                  Fp8Cfg::BN == TileCfg<bf16_t>::BN_DOWN && Fp8DecodeCfg::BM == Fp8Cfg::BM &&
                  Fp8DecodeCfg::BN == Fp8Cfg::BN && Fp8Cfg::PER_CU == TileCfg<bf16_t>::PER_CU &&
                  Fp8DecodeCfg::PER_CU == Fp8Cfg::PER_CU,
              "fp8 tiles share the work items, column tiles, grid and partial tiles of the bf16 path");
// fp8 weights take 128-deep K tiles when a batch routes at least
// MOELORA_FP8_DEEP_K_MIN_PAIRS_PER_EXPERT pairs per expert, else 64-deep ones
static bool fp8_deep_k_tiles(int64_t P, int64_t E) {
  return P >= (int64_t)MOELORA_FP8_DEEP_K_MIN_PAIRS_PER_EXPERT * E;
}
template <> struct TileCfg<float> {
  static constexpr int BM = 64, BN = 64, WM = 2, WN = 2, STAGES = 3, ROWB = 128, PER_CU = 2;
  static constexpr int BN_DOWN = 64, STAGES_DOWN = 3;
};

// persistent GEMM grid: PER_CU workgroups on each of the 256 CUs, a multiple
// of the 8 XCDs
static int64_t gemm_grid(int64_t tiles, int per_cu) {
  const int64_t full = 256 * per_cu;
  return tiles >= full ? full : round_up(tiles > 0 ? tiles : 1, 8);
}

// K splits of the down GEMM.  With few, long tiles (a long I and fewer than 8
// tiles per workgroup) the last round of the persistent grid leaves part of
// the GPU idle for a whole tile; two K halves double the tile count and halve
// that loss.  The tile count is estimated from P, E and the tile shape only
// (one item per BM pairs plus a partial one per expert), so the choice, and
// with it the rounding of y, does not depend on the align block size.
template <typename T>
static int down_ksplit(int64_t P, int64_t E, int64_t H, int64_t I, bool fp8) {
  constexpr int BM = TileCfg<T>::BM, BN = TileCfg<T>::BN_DOWN, BK = TileCfg<T>::ROWB / (int)sizeof(T);
  const int64_t items = ceil_div(P, BM) + std::min(P, E);
  const int64_t tiles = items * ceil_div(H, BN);
  const int64_t slots = 256 * (int64_t)TileCfg<T>::PER_CU;
  const int64_t kalign = fp8 ? 128 : BK;   // a split holds whole K tiles (and whole scale blocks)
  if (P <= 0 || I % (2 * kalign) != 0 || I / 2 < 4096 || tiles >= 8 * slots) return 1;
  return 2;
}

static int rows_per_item(int dtype) { return dtype == 1 ? TileCfg<bf16_t>::BM : TileCfg<float>::BM; }

// The large-tile bf16 GEMMs serve batches with at least this many pairs per
// expert on average (prefill) on layers with a hidden size of at least
// MOELORA_BIG_MIN_HIDDEN.  Their 256-row items would be mostly padding for
// decode-sized batches, and a short last item wastes more rows than the
// general kernel's: on the 128-expert layer (hidden 2048, intermediate 768,
// 8192 tokens, 512 pairs per expert with skewed routing) they measured
// slower (1.49 against 1.35 ms per layer), on the 256-expert layer (hidden
// 7168, 512 pairs per expert) faster (13.8 against 14.5 ms), on the 8-expert
// layer (hidden 4096, 1024 pairs per expert) even.
#ifndef MOELORA_BIG_MIN_PAIRS_PER_EXPERT
#define MOELORA_BIG_MIN_PAIRS_PER_EXPERT 256
#endif
#ifndef MOELORA_BIG_MIN_HIDDEN
#define MOELORA_BIG_MIN_HIDDEN 4096
#endif
static bool use_big(const ForwardProblem& p) {
  return p.dtype == 1 && p.wdtype != kWeightFp8 && p.H >= MOELORA_BIG_MIN_HIDDEN &&
         p.T * p.k >= (int64_t)MOELORA_BIG_MIN_PAIRS_PER_EXPERT * p.E;
}

// K splits of the large-tile down GEMM: as for the general kernel, two K
// halves when a long I leaves fewer than 8 tiles per workgroup
static int down_ksplit_big(int64_t P, int64_t E, int64_t H, int64_t I) {
  const int64_t items = ceil_div(P, big_tile_rows()) + std::min(P, E);
  const int64_t tiles = items * ceil_div(H, big_tile_cols(false));
  if (P <= 0 || I % (2 * big_tile_k()) != 0 || I / 2 < 4096 || tiles >= 8 * 256) return 1;
  return 2;
}

// K splits of a shrink: enough workgroups to fill the GPU when the batch has
// few rows (decode), each split at least 512 deep and a multiple of 128 (the
// four waves' interleaved 32-deep steps).
// The shrink shares pool rows across the row groups of a workgroup on large
// batches whose (expert, slot) buckets hold at least 64 pairs on average.
// Smaller buckets leave little to share; on smaller batches the narrower grid
// and its per-chunk barriers cost more than the pool re-reads.
#ifndef MOELORA_SHRINK4_MIN_ROWS
#define MOELORA_SHRINK4_MIN_ROWS 64
#endif
#ifndef MOELORA_SHRINK4_MIN_P
#define MOELORA_SHRINK4_MIN_P 65536
#endif

// waves (16-row groups) per workgroup of the LDS-shared shrink: 8 halves the
// pool-row traffic of 4 (each 256-byte pool chunk serves 128 rows), and with
// the deeper K split below took c4p's gate_up shrink from 0.86 to 0.65 ms
// (down shrink 0.19 -> 0.18; 16 waves: 0.78 ms)
#ifndef MOELORA_SHRINK_SHARED_WAVES
#define MOELORA_SHRINK_SHARED_WAVES 8
#endif
static constexpr int kShrinkSharedWaves = MOELORA_SHRINK_SHARED_WAVES;

static bool use_shrink4(int64_t P, int64_t E, int64_t L) {
  return L > 0 && P >= (int64_t)MOELORA_SHRINK4_MIN_P && P >= (int64_t)MOELORA_SHRINK4_MIN_ROWS * E * L;
}

template <typename T, int NPOOL>
static void launch_shrink(const ShrinkArgs<T>& s, int64_t groups, int splits, bool shared,
                          hipStream_t stream) {
  if (shared)  // two LDS buffers of NPOOL * RP pool rows of 256 bytes
    hipLaunchKernelGGL((shrink4_kernel<T, NPOOL, kShrinkSharedWaves>),
                       dim3((unsigned)ceil_div(groups, kShrinkSharedWaves), (unsigned)splits),
                       dim3(64 * kShrinkSharedWaves), (size_t)2 * NPOOL * s.RP * 256, stream, s);
  else
    hipLaunchKernelGGL((shrink_kernel<T, NPOOL>), dim3((unsigned)groups, (unsigned)splits),
                       dim3(256), 0, stream, s);
}

// K elements per split: enough splits for about MOELORA_SHRINK_WGS workgroups
// of 4 waves, each split at least npool * MOELORA_SHRINK_MIN_K deep (a split
// of the layer's two-pool gate/up shrink carries twice the pool rows per K
// element, and measured faster at twice the depth; the one-pool down shrink
// and the dense projection's shrink are kept at the single depth)
#ifndef MOELORA_SHRINK_WGS
#define MOELORA_SHRINK_WGS 1024
#endif
// the LDS-shared shrink's own target: K splits until about this many
// workgroups (c4p gate_up: 4 splits of 1792; 1024 (one split) 0.86 ms with 4
// waves, 2048 0.70, 4096 0.65)
#ifndef MOELORA_SHRINK4_WGS
#define MOELORA_SHRINK4_WGS 4096
#endif
#ifndef MOELORA_SHRINK_MIN_K
#define MOELORA_SHRINK_MIN_K 512
#endif
static int64_t shrink_kchunk(int64_t P, int64_t K, bool shared, int npool) {
  const int64_t groups = P / 16 + 1;
  const int64_t wgs = shared ? ceil_div(groups, kShrinkSharedWaves) : groups;
  const int64_t target = shared ? MOELORA_SHRINK4_WGS : MOELORA_SHRINK_WGS;
  int64_t s = std::min<int64_t>(16, std::max<int64_t>(1, ceil_div(target, wgs)));
  s = std::min<int64_t>(s, std::max<int64_t>(1, K / ((int64_t)npool * MOELORA_SHRINK_MIN_K)));
  return round_up(ceil_div(K, s), 128);
}
static int shrink_splits(int64_t P, int64_t K, bool shared, int npool) {
  return (int)ceil_div(K, shrink_kchunk(P, K, shared, npool));
}

// A GEMM launch.  With timing events the launch itself takes them (the
// dispatch records the kernel's start and end: no marker packets between
// kernels); without, a plain launch, as ordinary callers and stream capture
// get it.
template <typename... Args>
static void launch_timed(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t stream,
                         hipEvent_t ev0, hipEvent_t ev1, Args... args) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev0, ev1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

// The general gate_up GEMM, then, when it splits tail tiles into K pieces
// (a.part set), the kernel that adds the pieces and finishes those tiles.
template <typename T, typename W, typename F>
static void launch_gate_up(const GemmArgs<T>& a, int64_t nblk, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1) {
  const bool tails = a.part != nullptr;
  launch_timed((gemm_kernel<T, W, F::BM, F::BN, F::WM, F::WN, F::STAGES, F::ROWB, true>),
               dim3((unsigned)nblk), dim3(64 * F::WM * F::WN), stream, ev0, tails ? nullptr : ev1, a);
  if (tails)
    launch_timed((gate_up_fixup_kernel<T, F::BM, F::BN, F::WM, F::WN, F::ROWB>),
                 dim3((unsigned)ceil_div(F::BM * F::BN / 2, 256), (unsigned)(8 * std::max<int64_t>(nblk / 8 / 4, 1))),
                 dim3(256), stream, nullptr, ev1, a, (int)nblk);
}

ForwardWs forward_ws_layout(const ForwardProblem& p) {
  ForwardWs w;
  const int64_t P = p.T * p.k;
  const size_t esz = p.dtype == 1 ? 2 : 4;
  w.cap = align_capacity(P, p.E, p.L, p.BM);
  w.big = use_big(p);
  const int rpi = w.big ? big_tile_rows() : rows_per_item(p.dtype);
  w.rows_per_item = rpi;
  w.max_items = ceil_div(w.cap, rpi) + (P < p.E ? P : p.E);
  if (w.max_items < 1) w.max_items = 1;
  w.RP = p.L > 0 ? round_up(p.R > 0 ? p.R : 1, 32) : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += round_up((int64_t)bytes, 256); return o; };
  w.items_off = take(sizeof(int4) * (size_t)w.max_items);
  w.count_off = take(sizeof(int32_t) * 20);   // item count, then 2 x 8 tile counters
  w.shrink4 = use_shrink4(P, p.E, p.L);
  w.split_gu = shrink_splits(P, p.H, w.shrink4, 2);
  w.split_d = shrink_splits(P, p.I, w.shrink4, 1);
  w.split_down_k = w.big ? down_ksplit_big(P, p.E, p.H, p.I)
                 : p.dtype == 1 ? down_ksplit<bf16_t>(P, p.E, p.H, p.I, p.wdtype == kWeightFp8)
                                : down_ksplit<float>(P, p.E, p.H, p.I, false);
  if (w.big) {
    w.n_tiles_gu = ceil_div(p.I, big_tile_cols(true));
    w.n_tiles_dn = ceil_div(p.H, big_tile_cols(false)) * w.split_down_k;
  } else if (p.dtype == 1) {
    w.n_tiles_gu = ceil_div(p.I, TileCfg<bf16_t>::BN / 2);
    w.n_tiles_dn = ceil_div(p.H, TileCfg<bf16_t>::BN_DOWN) * w.split_down_k;
  } else {
    w.n_tiles_gu = ceil_div(p.I, TileCfg<float>::BN / 2);
    w.n_tiles_dn = ceil_div(p.H, TileCfg<float>::BN_DOWN) * w.split_down_k;
  }
  w.tab_gu_off = take(sizeof(int4) * (size_t)w.max_items * w.n_tiles_gu);
  w.tab_dn_off = take(sizeof(int4) * (size_t)w.max_items * w.n_tiles_dn);
  w.slot_rank_off = take(sizeof(int32_t) * (size_t)(w.cap / p.BM + 1));
  w.hgu_off = take(p.L > 0 ? sizeof(float) * (size_t)w.split_gu * w.cap * 2 * w.RP : 0);
  w.act_off = take(esz * (size_t)w.cap * p.I);
  w.hd_off = take(p.L > 0 ? sizeof(float) * (size_t)w.split_d * w.cap * w.RP : 0);
  w.z_off = take((p.dtype == 1 ? 3 : 4) * (size_t)w.split_down_k * P * p.H);   // 24-bit z for bf16 layers
  // the general gate_up GEMM may split tail tiles into K pieces (one partial
  // tile per workgroup of its grid) when its tiles are long: with fewer than
  // 64 K tiles a split saves less than the extra launch that finishes the
  // pieces costs (measured on the decode batches)
  const bool fp8w = p.dtype == 1 && p.wdtype == kWeightFp8;
  const int64_t bk_gu = !fp8w ? (p.dtype == 1 ? TileCfg<bf16_t>::ROWB / 2 : TileCfg<float>::ROWB / 4)
                        : fp8_deep_k_tiles(P, p.E) ? Fp8Cfg::ROWB / 2 : Fp8DecodeCfg::ROWB / 2;
  if (!w.big && p.H >= 64 * bk_gu) {
    const int per_cu = p.dtype == 1 ? TileCfg<bf16_t>::PER_CU : TileCfg<float>::PER_CU;
    const int64_t tile_elems = p.dtype == 1 ? (int64_t)TileCfg<bf16_t>::BM * TileCfg<bf16_t>::BN
                                            : (int64_t)TileCfg<float>::BM * TileCfg<float>::BN;
    w.grid_gu = gemm_grid(w.n_tiles_gu * w.max_items, per_cu);
    w.part_off = take(sizeof(float) * (size_t)(w.grid_gu * tile_elems));
  }
  w.bytes = off;
  return w;
}

template <typename T>
static hipError_t run_forward(const ForwardProblem& p, void* workspace, hipStream_t stream,
                             hipEvent_t* events) {
  // optional measurement: events[2s] / events[2s+1] bracket stage s; the
  // single-kernel GEMM stages hand theirs to the launch itself (the dispatch
  // records them: no marker packets, which idle the GPU between kernels)
  auto mark = [&](int idx) {
    if (events && events[idx]) (void)hipEventRecord(events[idx], stream);
  };
  const ForwardWs w = forward_ws_layout(p);
  char* ws = static_cast<char*>(workspace);
  int4* items = reinterpret_cast<int4*>(ws + w.items_off);
  int32_t* count = reinterpret_cast<int32_t*>(ws + w.count_off);
  float* hgu = reinterpret_cast<float*>(ws + w.hgu_off);
  T* act = reinterpret_cast<T*>(ws + w.act_off);
  float* hd = reinterpret_cast<float*>(ws + w.hd_off);
  void* z = ws + w.z_off;
  const int64_t P = p.T * p.k;
  const bool lora = p.L > 0;
  const int BM = w.rows_per_item;   // rows of a work item
  constexpr int BN = TileCfg<T>::BN;
  constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  const bool fp8w = kBf16 && p.wdtype == kWeightFp8;
  const bool fp8_deep_k = fp8_deep_k_tiles(P, p.E);

  mark(2 * kStagePlan);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, (int)p.E, (int)p.BM, BM,
                     p.expert_tile_offsets, items, count, (int)w.max_items);
  int4* tab_gu = reinterpret_cast<int4*>(ws + w.tab_gu_off);
  int4* tab_dn = reinterpret_cast<int4*>(ws + w.tab_dn_off);
  int32_t* slot_rank = reinterpret_cast<int32_t*>(ws + w.slot_rank_off);
  {
    const int64_t n = std::max<int64_t>(w.max_items * std::max(w.n_tiles_gu, w.n_tiles_dn), w.cap / p.BM);
    hipLaunchKernelGGL(tile_table_kernel, dim3((unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(n, 256)))),
                       dim3(256), 0, stream, items, count, (int)w.max_items, p.expert_tile_offsets,
                       (int)p.BM, (int)p.E, BM, (int)w.n_tiles_gu, tab_gu, (int)w.n_tiles_dn, tab_dn,
                       p.tile_lora, p.lora_ranks, (int)p.L, (int)p.R, (int)(w.cap / p.BM),
                       lora ? slot_rank : nullptr, w.big ? MOELORA_GROUP_ITEMS_BIG : MOELORA_GROUP_ITEMS);
  }
  mark(2 * kStagePlan + 1);

  const int64_t groups = w.cap / 16;
  mark(2 * kStageShrinkX);
  if (lora && groups > 0) {
    ShrinkArgs<T> s{};
    s.src = static_cast<const T*>(p.x);
    s.sorted_ids = p.sorted_ids;
    s.gathered = 1;
    s.top_k = (int)p.k;
    s.P = (int)P;
    s.K = p.H;
    s.pool0 = static_cast<const T*>(p.a_gate);
    s.pool1 = static_cast<const T*>(p.a_up);
    s.R = (int)p.R; s.RP = (int)w.RP; s.L = (int)p.L; s.E = (int)p.E; s.BM = (int)p.BM;
    s.tile_expert = p.tile_expert;
    s.tile_lora = p.tile_lora;
    s.num_rows_padded = p.num_rows_padded;
    s.lora_ranks = p.lora_ranks;
    s.scaling = p.scaling;
    s.h = hgu;
    s.cap = w.cap;
    s.kchunk = shrink_kchunk(P, p.H, w.shrink4, 2);
    s.split_stride = w.cap * 2 * w.RP;
    launch_shrink<T, 2>(s, groups, w.split_gu, w.shrink4, stream);
    if (w.split_gu > 1)
      hipLaunchKernelGGL(shrink_reduce_kernel, dim3((unsigned)ceil_div(w.cap * 2 * w.RP / 8, 256)),
                         dim3(256), 0, stream, hgu, (int64_t)s.split_stride, w.split_gu,
                         p.num_rows_padded, (int)(2 * w.RP), kBf16 ? 1 : 0);
  }
  mark(2 * kStageShrinkX + 1);

  GemmArgs<T> g{};
  g.items = items;
  g.item_count = count;
  g.max_items = (int)w.max_items;
  g.top_k = (int)p.k;
  g.P = (int)P;
  g.sorted_ids = p.sorted_ids;
  g.tile_lora = p.tile_lora;
  g.expert_tile_offsets = p.expert_tile_offsets;
  g.BM_tile = (int)p.BM;
  g.lora_ranks = p.lora_ranks;
  g.RP = (int)w.RP; g.R = (int)p.R; g.L = (int)p.L; g.E = (int)p.E;
  g.topk_weights = p.topk_weights;
  g.cap = w.cap;
  g.slot_rank = slot_rank;

  // gate_up
  {
    GemmArgs<T> a = g;
    a.a_src = static_cast<const T*>(p.x);
    a.K = p.H;
    a.w = p.w_gate_up;
    a.w_scale = fp8w ? p.w_gate_up_scale : nullptr;
    a.n_out = p.I;
    a.w_rows = 2 * p.I;
    a.n_cols = (int)w.n_tiles_gu;
    a.ksplit = 1;
    a.n_tiles = a.n_cols;
    a.tile_tab = tab_gu;
    a.h = lora ? hgu : nullptr;
    a.HS = 2 * (int)w.RP;
    a.b_pool0 = static_cast<const T*>(p.b_gate);
    a.b_pool1 = static_cast<const T*>(p.b_up);
    a.act = act;
    a.tile_ctr = count + 4;
    int64_t nblk = gemm_grid((int64_t)a.n_tiles * w.max_items, TileCfg<T>::PER_CU);
    hipEvent_t ev0 = events ? events[2 * kStageGateUp] : nullptr, ev1 = events ? events[2 * kStageGateUp + 1] : nullptr;
    if (w.grid_gu > 0) {
      if (nblk != w.grid_gu) return hipErrorInvalidValue;   // the partial buffer is sized for this grid
      a.part = reinterpret_cast<float*>(ws + w.part_off);
    }
    if constexpr (kBf16) {
      if (w.big)
        launch_gemm_big(true, a, nblk, stream, ev0, ev1);
      else if (fp8w && fp8_deep_k)
        launch_gate_up<T, uint8_t, Fp8Cfg>(a, nblk, stream, ev0, ev1);
      else if (fp8w)
        launch_gate_up<T, uint8_t, Fp8DecodeCfg>(a, nblk, stream, ev0, ev1);
    }
    if (!fp8w && !w.big) launch_gate_up<T, T, TileCfg<T>>(a, nblk, stream, ev0, ev1);
  }
  mark(2 * kStageShrinkA);
  if (lora && groups > 0) {
    ShrinkArgs<T> s{};
    s.src = act;
    s.sorted_ids = p.sorted_ids;
    s.gathered = 0;
    s.top_k = (int)p.k;
    s.P = (int)P;
    s.K = p.I;
    s.pool0 = static_cast<const T*>(p.a_down);
    s.pool1 = nullptr;
    s.R = (int)p.R; s.RP = (int)w.RP; s.L = (int)p.L; s.E = (int)p.E; s.BM = (int)p.BM;
    s.tile_expert = p.tile_expert;
    s.tile_lora = p.tile_lora;
    s.num_rows_padded = p.num_rows_padded;
    s.lora_ranks = p.lora_ranks;
    s.scaling = p.scaling;
    s.h = hd;
    s.cap = w.cap;
    s.kchunk = shrink_kchunk(P, p.I, w.shrink4, 1);
    s.split_stride = w.cap * w.RP;
    launch_shrink<T, 1>(s, groups, w.split_d, w.shrink4, stream);
    if (w.split_d > 1)
      hipLaunchKernelGGL(shrink_reduce_kernel, dim3((unsigned)ceil_div(w.cap * w.RP / 8, 256)),
                         dim3(256), 0, stream, hd, (int64_t)s.split_stride, w.split_d,
                         p.num_rows_padded, (int)w.RP, kBf16 ? 1 : 0);
  }
  mark(2 * kStageShrinkA + 1);
  // down
  {
    GemmArgs<T> a = g;
    a.a_src = act;
    a.K = p.I;
    a.w = p.w_down;
    a.w_scale = fp8w ? p.w_down_scale : nullptr;
    a.n_out = p.H;
    a.w_rows = p.H;
    constexpr int SD = TileCfg<T>::STAGES_DOWN;
    a.n_cols = (int)(w.n_tiles_dn / w.split_down_k);
    a.ksplit = w.split_down_k;
    a.n_tiles = a.n_cols * a.ksplit;
    a.tile_tab = tab_dn;
    a.h = lora ? hd : nullptr;
    a.HS = (int)w.RP;
    a.b_pool0 = static_cast<const T*>(p.b_down);
    a.b_pool1 = nullptr;
    a.z = z;
    a.tile_ctr = count + 12;
    int64_t nblk = gemm_grid((int64_t)a.n_tiles * w.max_items, TileCfg<T>::PER_CU);
    hipEvent_t ev0 = events ? events[2 * kStageDown] : nullptr, ev1 = events ? events[2 * kStageDown + 1] : nullptr;
    if constexpr (kBf16) {
      if (w.big) {
        launch_gemm_big(false, a, nblk, stream, ev0, ev1);
      } else if (fp8w && fp8_deep_k) {
        typedef Fp8Cfg F;
        launch_timed((gemm_kernel<T, uint8_t, F::BM, F::BN, F::WM, F::WN, F::STAGES, F::ROWB, false>),
                           dim3((unsigned)nblk), dim3(64 * F::WM * F::WN), stream, ev0, ev1, a);
      } else if (fp8w) {
        typedef Fp8DecodeCfg F;
        launch_timed((gemm_kernel<T, uint8_t, F::BM, F::BN, F::WM, F::WN, F::STAGES, F::ROWB, false>),
                           dim3((unsigned)nblk), dim3(64 * F::WM * F::WN), stream, ev0, ev1, a);
      }
    }
    if (!fp8w && !w.big)
      launch_timed((gemm_kernel<T, T, TileCfg<T>::BM, TileCfg<T>::BN_DOWN, TileCfg<T>::WM, TileCfg<T>::WN, SD, TileCfg<T>::ROWB, false>),
                            dim3((unsigned)nblk), dim3(64 * TileCfg<T>::WM * TileCfg<T>::WN), stream, ev0, ev1, a);
  }
  mark(2 * kStageCombine);
  if (P > 0) {
    const int64_t n4 = p.T * p.H / 4;
    const dim3 cg((unsigned)ceil_div(n4, 256));
    if (p.out_f32)
      hipLaunchKernelGGL((combine_kernel<kBf16, float>), cg, dim3(256), 0, stream, (const void*)z,
                         static_cast<float*>(p.y), p.T, (int)p.k, p.H, w.split_down_k, P * p.H);
    else
      hipLaunchKernelGGL((combine_kernel<kBf16, T>), cg, dim3(256), 0, stream, (const void*)z,
                         static_cast<T*>(p.y), p.T, (int)p.k, p.H, w.split_down_k, P * p.H);
  }
  mark(2 * kStageCombine + 1);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// dense projection with two LoRA output slices
// --------------------------------------------------------------------------
// K splits of the dense GEMM: a decode-sized batch has a handful of tiles
// (one or two items times the column tiles), far fewer than the 256 CUs; each
// K split is a tile of its own (one fp32 plane of z each, added in order by the
// combine), up to 8, each at least 512 deep and a whole number of K tiles
template <typename T>
static int dense_ksplit(int64_t P, int64_t K, int64_t N) {
  constexpr int BM = TileCfg<T>::BM, BN = TileCfg<T>::BN_DOWN, BK = TileCfg<T>::ROWB / (int)sizeof(T);
  const int64_t tiles = (ceil_div(P, BM) + 1) * ceil_div(N, BN);
  const int64_t slots = 256 * (int64_t)TileCfg<T>::PER_CU;
  if (P <= 0 || tiles >= slots / 2) return 1;
  int s = (int)std::min<int64_t>(8, ceil_div(slots, tiles));
  while (s > 1 && (K % (s * BK) != 0 || K / s < 512)) --s;
  return s;
}

DenseWs dense_ws_layout(const DenseProblem& p) {
  DenseWs w;
  const int64_t P = p.T;   // one pair per token (E = 1, k = 1)
  w.cap = align_capacity(P, 1, p.L, p.BM);
  w.max_items = ceil_div(w.cap, rows_per_item(p.dtype)) + (P < 1 ? P : 1);
  if (w.max_items < 1) w.max_items = 1;
  w.RP = p.L > 0 ? round_up(p.R > 0 ? p.R : 1, 32) : 0;
  w.npool = p.N1 > 0 ? 2 : 1;
  w.split = shrink_splits(P, p.H, false, 1);   // (deeper two-pool splits measured slower here)
  w.ksplit = p.dtype == 1 ? dense_ksplit<bf16_t>(P, p.H, p.N0 + p.N1) : dense_ksplit<float>(P, p.H, p.N0 + p.N1);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += round_up((int64_t)bytes, 256); return o; };
  w.n_tiles = ceil_div(p.N0 + p.N1, p.dtype == 1 ? TileCfg<bf16_t>::BN_DOWN : TileCfg<float>::BN_DOWN) * w.ksplit;
  w.items_off = take(sizeof(int4) * (size_t)w.max_items);
  w.count_off = take(sizeof(int32_t) * 36);
  w.tab_off = take(sizeof(int4) * (size_t)w.max_items * w.n_tiles);
  w.slot_rank_off = take(sizeof(int32_t) * (size_t)(w.cap / p.BM + 1));
  w.h_off = take(p.L > 0 ? sizeof(float) * (size_t)w.split * w.cap * w.npool * w.RP : 0);
  w.z_off = take(sizeof(float) * (size_t)w.ksplit * P * (p.N0 + p.N1));
  w.bytes = off;
  return w;
}

template <typename T>
static hipError_t run_dense(const DenseProblem& p, void* workspace, hipStream_t stream,
                            hipEvent_t* events) {
  auto mark = [&](int idx) {
    if (events && events[idx]) (void)hipEventRecord(events[idx], stream);
  };
  const DenseWs w = dense_ws_layout(p);
  char* ws = static_cast<char*>(workspace);
  int4* items = reinterpret_cast<int4*>(ws + w.items_off);
  int32_t* count = reinterpret_cast<int32_t*>(ws + w.count_off);
  float* h = reinterpret_cast<float*>(ws + w.h_off);
  float* z = reinterpret_cast<float*>(ws + w.z_off);
  const int64_t P = p.T, N = p.N0 + p.N1;
  const bool lora = p.L > 0;
  constexpr int BM = TileCfg<T>::BM, BND = TileCfg<T>::BN_DOWN, SD = TileCfg<T>::STAGES_DOWN;

  mark(2 * kDenseStagePlan);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, 1, (int)p.BM, BM,
                     p.expert_tile_offsets, items, count, (int)w.max_items);
  int4* tab = reinterpret_cast<int4*>(ws + w.tab_off);
  int32_t* slot_rank = reinterpret_cast<int32_t*>(ws + w.slot_rank_off);
  {
    const int64_t n = std::max<int64_t>(w.max_items * w.n_tiles, w.cap / p.BM);
    hipLaunchKernelGGL(tile_table_kernel, dim3((unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(n, 256)))),
                       dim3(256), 0, stream, items, count, (int)w.max_items, p.expert_tile_offsets,
                       (int)p.BM, 1, BM, (int)w.n_tiles, tab, 0, (int4*)nullptr, p.tile_lora,
                       p.lora_ranks, (int)p.L, (int)p.R, (int)(w.cap / p.BM), lora ? slot_rank : nullptr,
                       MOELORA_GROUP_ITEMS);
  }
  mark(2 * kDenseStagePlan + 1);

  const int64_t groups = w.cap / 16;
  mark(2 * kDenseStageShrink);
  if (lora && groups > 0 && P > 0) {
    // h[:, :RP] = s x A0^T, h[:, RP:] = s x A1^T over the tokens' rows
    ShrinkArgs<T> s{};
    s.src = static_cast<const T*>(p.x);
    s.sorted_ids = p.sorted_ids;
    s.gathered = 1;
    s.top_k = 1;
    s.P = (int)P;
    s.K = p.H;
    s.pool0 = static_cast<const T*>(p.a0);
    s.pool1 = static_cast<const T*>(p.a1);
    s.R = (int)p.R; s.RP = (int)w.RP; s.L = (int)p.L; s.E = 1; s.BM = (int)p.BM;
    s.tile_expert = p.tile_expert;
    s.tile_lora = p.tile_lora;
    s.num_rows_padded = p.num_rows_padded;
    s.lora_ranks = p.lora_ranks;
    s.scaling = p.scaling;
    s.h = h;
    s.cap = w.cap;
    s.kchunk = shrink_kchunk(P, p.H, false, 1);
    s.split_stride = w.cap * w.npool * w.RP;
    if (w.npool == 2)
      launch_shrink<T, 2>(s, groups, w.split, false, stream);
    else
      launch_shrink<T, 1>(s, groups, w.split, false, stream);
    if (w.split > 1)
      hipLaunchKernelGGL(shrink_reduce_kernel, dim3((unsigned)ceil_div(w.cap * w.npool * w.RP / 8, 256)),
                         dim3(256), 0, stream, h, (int64_t)s.split_stride, w.split,
                         p.num_rows_padded, (int)(w.npool * w.RP), std::is_same<T, bf16_t>::value ? 1 : 0);
  }
  mark(2 * kDenseStageShrink + 1);

  if (P == 0) mark(2 * kDenseStageGemm);
  if (P > 0) {
    GemmArgs<T> a{};
    a.items = items;
    a.item_count = count;
    a.max_items = (int)w.max_items;
    a.top_k = 1;
    a.P = (int)P;
    a.sorted_ids = p.sorted_ids;
    a.tile_lora = p.tile_lora;
    a.expert_tile_offsets = p.expert_tile_offsets;
    a.BM_tile = (int)p.BM;
    a.lora_ranks = p.lora_ranks;
    a.RP = (int)w.RP; a.R = (int)p.R; a.L = (int)p.L; a.E = 1;
    a.topk_weights = nullptr;
    a.cap = w.cap;
    a.a_src = static_cast<const T*>(p.x);
    a.K = p.H;
    a.w = p.w;
    a.n_out = N;
    a.w_rows = N;
    a.n_cols = (int)ceil_div(N, BND);
    a.ksplit = w.ksplit;
    a.n_tiles = a.n_cols * a.ksplit;
    if (a.n_tiles != w.n_tiles) return hipErrorInvalidValue;   // the table's tile count
    a.tile_tab = tab;
    a.slot_rank = slot_rank;
    a.h = lora ? h : nullptr;
    a.HS = w.npool * (int)w.RP;
    a.b_pool0 = static_cast<const T*>(p.b0);
    a.b_pool1 = static_cast<const T*>(p.b1);
    a.n_split = p.N0;
    a.z = z;
    a.tile_ctr = count + 4;
    const int64_t nblk = gemm_grid((int64_t)a.n_tiles * w.max_items, TileCfg<T>::PER_CU);
    // the stage's events, when given, are taken by the launch itself
    hipEvent_t ev0 = events ? events[2 * kDenseStageGemm] : nullptr;
    hipEvent_t ev1 = events ? events[2 * kDenseStageGemm + 1] : nullptr;
    launch_timed((gemm_kernel<T, T, BM, BND, TileCfg<T>::WM, TileCfg<T>::WN, SD, TileCfg<T>::ROWB, false, true>),
                          dim3((unsigned)nblk), dim3(64 * TileCfg<T>::WM * TileCfg<T>::WN), stream, ev0, ev1, a);
  }
  if (P == 0) mark(2 * kDenseStageGemm + 1);

  mark(2 * kDenseStageCombine);
  if (P > 0) {
    const int64_t n4 = P * N / 4;
    if (p.out_f32)
      hipLaunchKernelGGL((combine_kernel<false, float>), dim3((unsigned)ceil_div(n4, 256)), dim3(256), 0,
                         stream, (const void*)z, static_cast<float*>(p.y), P, 1, N, w.ksplit, P * N);
    else
      hipLaunchKernelGGL((combine_kernel<false, T>), dim3((unsigned)ceil_div(n4, 256)), dim3(256), 0,
                         stream, (const void*)z, static_cast<T*>(p.y), P, 1, N, w.ksplit, P * N);
  }
  mark(2 * kDenseStageCombine + 1);
  return hipGetLastError();
}

hipError_t launch_dense(const DenseProblem& p, void* workspace, hipStream_t stream,
                        hipEvent_t* events) {
  if (p.dtype == 1) return run_dense<bf16_t>(p, workspace, stream, events);
  return run_dense<float>(p, workspace, stream, events);
}

hipError_t launch_forward(const ForwardProblem& p, void* workspace, hipStream_t stream,
                          hipEvent_t* events) {
  if (p.dtype == 1) return run_forward<bf16_t>(p, workspace, stream, events);
  return run_forward<float>(p, workspace, stream, events);
}

// --------------------------------------------------------------------------
// the static workspace of the allocation-free forward entry point
// --------------------------------------------------------------------------
// One array per device, held from the library's load until the process ends.
// Host code never passes the array's name to a kernel (in host code it is only
// a stand-in for the device symbol): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moelora
