// Bucketing of (token, expert) pairs by (expert, adapter) -- the align step of
// the MoE-LoRA layer (SGLang PR #14105 page, section 实现拆解: tokens are sorted
// by LoRA adapter and expert id before the grouped GEMMs).
//
// A stable counting sort over keys e * (L + 1) + (a_eff + 1) in three launches:
//   1. count   -- each workgroup takes a chunk of pairs; each of its waves ranks
//                 its pairs among equal keys with a bitwise ballot match (one
//                 ballot per key bit, no loop over distinct keys) and an LDS
//                 histogram, so the rank is the pair's order inside the chunk.
//   2. scan    -- one workgroup: per key, prefix over chunks; bucket sizes padded
//                 to block_m; exclusive scan over keys; tile counts per expert.
//   3. scatter -- one thread per output row and per pair: pairs go to
//                 bucket offset + chunk prefix + rank; pads, tile tables and the
//                 unused tail are filled by binary search over bucket starts.
// Every output word up to the capacity is written.
#include "moe_lora.h"
#include "common.hpp"
#include "kernels.hpp"

namespace moelora {

// at most this many 64-pair steps per wave in the count kernel: fewer, longer
// chunks shorten the one-workgroup scan (chunks x keys) more than they lengthen
// the count (align on c4p 95 -> 67 us, c2 58 -> 48 us against 8 steps; 32 steps
// lose on c2 and c3)
static constexpr int kAlignSteps = 16;
static constexpr int kScanThreads = 1024;
static constexpr int kScatterThreads = 256;

int align_waves_for_keys(int64_t K) {
  if (K <= 8192) return 4;
  if (K <= 16384) return 2;
  return 1;
}

// 64-pair steps per wave: as many as keep the chunk count near 16, so a
// small batch spreads over several workgroups instead of walking its pairs
// step by step in one (the scan's cost grows with chunks x keys: targets of
// 32, 64 and 128 chunks measured align on c2 at 42, 58 and 91 us against 38)
int align_steps(int64_t P, int64_t K) {
  const int64_t per_step = (int64_t)align_waves_for_keys(K) * 64;
  return (int)std::min<int64_t>(kAlignSteps, std::max<int64_t>(1, ceil_div(P, per_step * 16)));
}

int64_t align_chunk_pairs(int64_t P, int64_t K) {
  return (int64_t)align_waves_for_keys(K) * align_steps(P, K) * 64;
}

AlignWs align_ws_layout(int64_t P, int64_t K) {
  AlignWs w;
  int64_t ch = align_chunk_pairs(P, K);
  w.nchunks = P > 0 ? ceil_div(P, ch) : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += round_up((int64_t)bytes, 256); return o; };
  w.rank_off = take(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
  w.cnt_off = take(sizeof(int32_t) * (size_t)(w.nchunks * K));
  w.bstart_off = take(sizeof(int32_t) * (size_t)(K + 1));
  w.btotal_off = take(sizeof(int32_t) * (size_t)K);
  w.bytes = off;
  return w;
}

// key of pair p, or -1 when its expert id is out of range
__device__ inline int pair_key(int p, int k, int E, int L, const int32_t* __restrict__ topk_ids,
                               const int32_t* __restrict__ mapping,
                               const int32_t* __restrict__ enabled) {
  int e = topk_ids[p];
  if (e < 0 || e >= E) return -1;
  int a = mapping[p / k];
  int a_eff = (a >= 0 && a < L && enabled[a] == 1) ? a : -1;
  return e * (L + 1) + (a_eff + 1);
}

__global__ void __launch_bounds__(256)
align_count_kernel(int P, int k, int E, int L, int K, int key_bits, int waves, int steps,
                   const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ mapping,
                   const int32_t* __restrict__ enabled, int32_t* __restrict__ ws_rank,
                   int32_t* __restrict__ ws_cnt, uint32_t* __restrict__ dbg) {
  extern __shared__ uint16_t hist[];  // [waves][K]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* h = hist + (size_t)wave * K;
  for (int i = lane; i < K; i += 64) h[i] = 0;

  const int chunk = blockIdx.x;
  const int64_t chunk_pairs = (int64_t)waves * steps * 64;
  const int64_t wbase = chunk * chunk_pairs + (int64_t)wave * steps * 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));

  int keys[kAlignSteps], ranks[kAlignSteps];
#pragma unroll
  for (int s = 0; s < kAlignSteps; ++s) {
    const int64_t p = wbase + s * 64 + lane;
    int key = -1;
    if (s < steps && p < P) {
      key = pair_key((int)p, k, E, L, topk_ids, mapping, enabled);
#ifdef MOE_LORA_DEBUG
      // preconditions: expert ids in [0, E), the token's slot in [-1, L)
      const int32_t e = topk_ids[p];
      if (e < 0 || e >= E) debug_flag(dbg, MOE_LORA_DEBUG_EXPERT_ID);
      const int32_t a = mapping[p / k];
      if (p % k == 0 && (a < -1 || a >= L)) debug_flag(dbg, MOE_LORA_DEBUG_MAPPING);
#endif
    }
    const bool valid = key >= 0;
    // lanes holding the same key: AND of per-bit ballots
    uint64_t m = __ballot(valid);
    for (int b = 0; b < key_bits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int r = 0;
    if (valid) {
      const int before = __popcll(m & lt_mask);
      const int old = h[key];
      r = old + before;
      if (before == 0) h[key] = (uint16_t)(old + __popcll(m));
    }
    keys[s] = key;
    ranks[s] = r;
  }
  __syncthreads();
  // exclusive prefix over waves for each key; chunk totals to global
  for (int key = threadIdx.x; key < K; key += blockDim.x) {
    int sum = 0;
    for (int w = 0; w < waves; ++w) {
      int c = hist[(size_t)w * K + key];
      hist[(size_t)w * K + key] = (uint16_t)sum;
      sum += c;
    }
    ws_cnt[(int64_t)chunk * K + key] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kAlignSteps; ++s) {
    const int64_t p = wbase + s * 64 + lane;
    if (s < steps && p < P && keys[s] >= 0) ws_rank[p] = ranks[s] + h[keys[s]];
  }
}

// exclusive scan of one int per thread over a kScanThreads workgroup
__device__ inline int block_exclusive_scan(int v, int* lds_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      int c = lds_waves[w];
      lds_waves[w] = run;
      run += c;
    }
    lds_waves[kScanThreads / 64] = run;
  }
  __syncthreads();
  int res = lds_waves[wave] + x - v;
  *total = lds_waves[kScanThreads / 64];
  __syncthreads();
  return res;
}

__global__ void __launch_bounds__(kScanThreads)
align_scan_kernel(int nchunks, int K, int E, int L, int BM, int32_t* __restrict__ ws_cnt,
                  int32_t* __restrict__ ws_bstart, int32_t* __restrict__ ws_btotal,
                  int32_t* __restrict__ expert_tile_offsets, int32_t* __restrict__ num_rows_padded) {
  __shared__ int lds_waves[kScanThreads / 64 + 1];
  const int kpt = (K + kScanThreads - 1) / kScanThreads;
  const int k0 = min(K, (int)threadIdx.x * kpt), k1 = min(K, k0 + kpt);
  // A thread's keys k0..k1-1 are scanned over the chunks in place (each
  // chunk's count becomes the key's count in the chunks before it), KB keys
  // and CB chunks at a time: the block's loads all go out before the first
  // use, one memory round trip per block (a key-by-key, chunk-by-chunk loop
  // waits for each load: its next load cannot pass the store before it).
  // The key's first row is added by the scatter, not here.
  constexpr int KB = 4, CB = 8;
  int tot[KB] = {0, 0, 0, 0};   // the totals of the first KB keys (all of them when kpt <= KB)
  int mine = 0;
  for (int kb = k0; kb < k1; kb += KB) {
    int run[KB];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) run[kk] = 0;
    for (int c0 = 0; c0 < nchunks; c0 += CB) {
      int v[KB][CB];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int c = 0; c < CB; ++c)
          v[kk][c] = (kb + kk < k1 && c0 + c < nchunks) ? ws_cnt[(int64_t)(c0 + c) * K + kb + kk] : 0;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          const int x = v[kk][c];
          v[kk][c] = run[kk];
          run[kk] += x;
        }
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int c = 0; c < CB; ++c)
          if (kb + kk < k1 && c0 + c < nchunks) ws_cnt[(int64_t)(c0 + c) * K + kb + kk] = v[kk][c];
    }
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      if (kb + kk >= k1) continue;
      ws_btotal[kb + kk] = run[kk];
      mine += (int)round_up(run[kk], BM);
      if (kb == k0) tot[kk] = run[kk];
    }
  }
  int total = 0;
  int start = block_exclusive_scan(mine, lds_waves, &total);
  // the first KB keys' totals are in registers, further ones (kpt > KB) are read back
  auto place = [&](int key, int key_total) {
    ws_bstart[key] = start;
    if (key % (L + 1) == 0) expert_tile_offsets[key / (L + 1)] = start / BM;   // the expert's first key
    start += (int)round_up(key_total, BM);
  };
#pragma unroll
  for (int kk = 0; kk < KB; ++kk)
    if (k0 + kk < k1) place(k0 + kk, tot[kk]);
  for (int key = k0 + KB; key < k1; ++key) place(key, ws_btotal[key]);
  if (threadIdx.x == 0) {
    ws_bstart[K] = total;
    num_rows_padded[0] = total;
    expert_tile_offsets[E] = total / BM;
  }
}

__global__ void __launch_bounds__(kScatterThreads)
align_scatter_kernel(int P, int k, int E, int L, int K, int BM, int64_t cap, int64_t chunk_pairs,
                     const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ mapping,
                     const int32_t* __restrict__ enabled, const int32_t* __restrict__ ws_rank,
                     const int32_t* __restrict__ ws_off, const int32_t* __restrict__ ws_bstart,
                     const int32_t* __restrict__ ws_btotal, int32_t* __restrict__ sorted_ids,
                     int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_lora) {
  const int64_t i = (int64_t)blockIdx.x * kScatterThreads + threadIdx.x;
  if (i < P) {
    int key = pair_key((int)i, k, E, L, topk_ids, mapping, enabled);
    if (key >= 0) {
      // the key's first row + the key's pairs in earlier chunks + the rank in this chunk
      int64_t pos = (int64_t)ws_bstart[key] + ws_off[(i / chunk_pairs) * K + key] + ws_rank[i];
      if (pos >= 0 && pos < cap) sorted_ids[pos] = (int32_t)i;
    }
  }
  if (i < cap) {
    const int rows = ws_bstart[K];
    if (i >= rows) {
      sorted_ids[i] = P;
      if (i % BM == 0) {
        tile_expert[i / BM] = -1;
        tile_lora[i / BM] = -1;
      }
    } else {
      int lo = 0, hi = K;  // largest key with bstart[key] <= i
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (ws_bstart[mid] <= i) lo = mid; else hi = mid;
      }
      if (i - ws_bstart[lo] >= ws_btotal[lo]) sorted_ids[i] = P;
      if (i % BM == 0) {
        tile_expert[i / BM] = lo / (L + 1);
        tile_lora[i / BM] = lo % (L + 1) - 1;
      }
    }
  }
}

hipError_t launch_align(int32_t T, int32_t k, int32_t E, int32_t L, int32_t BM,
                        const int32_t* topk_ids, const int32_t* mapping, const int32_t* enabled,
                        int32_t* sorted_ids, int32_t* tile_expert, int32_t* tile_lora,
                        int32_t* expert_tile_offsets, int32_t* num_rows_padded, void* workspace,
                        uint32_t* debug_word, hipStream_t stream) {
  const int64_t P = (int64_t)T * k;
  const int64_t K = (int64_t)E * (L + 1);
  const AlignWs w = align_ws_layout(P, K);
  char* ws = static_cast<char*>(workspace);
  int32_t* ws_rank = reinterpret_cast<int32_t*>(ws + w.rank_off);
  int32_t* ws_cnt = reinterpret_cast<int32_t*>(ws + w.cnt_off);
  int32_t* ws_bstart = reinterpret_cast<int32_t*>(ws + w.bstart_off);
  int32_t* ws_btotal = reinterpret_cast<int32_t*>(ws + w.btotal_off);
  const int waves = align_waves_for_keys(K);
  int key_bits = 0;
  while ((int64_t(1) << key_bits) < K) ++key_bits;
  const size_t lds = (size_t)waves * K * sizeof(uint16_t);

  hipLaunchKernelGGL(align_count_kernel, dim3((unsigned)w.nchunks), dim3(64 * waves), lds, stream,
                     (int)P, k, E, L, (int)K, key_bits, waves, align_steps(P, K), topk_ids, mapping,
                     enabled, ws_rank, ws_cnt, debug_word);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, (int)w.nchunks,
                     (int)K, E, L, BM, ws_cnt, ws_bstart, ws_btotal, expert_tile_offsets,
                     num_rows_padded);
  const int64_t cap = align_capacity(P, E, L, BM);
  const int64_t n = cap > P ? cap : P;
  if (n > 0) {
    hipLaunchKernelGGL(align_scatter_kernel, dim3((unsigned)ceil_div(n, kScatterThreads)),
                       dim3(kScatterThreads), 0, stream, (int)P, k, E, L, (int)K, BM, cap,
                       align_chunk_pairs(P, K), topk_ids, mapping, enabled, ws_rank, ws_cnt,
                       ws_bstart, ws_btotal, sorted_ids, tile_expert, tile_lora);
  }
  return hipGetLastError();
}

}  // namespace moelora
