// Large-tile grouped GEMM of the MoE-LoRA layer for prefill-sized batches
// (bf16): the gate_up and down projections of the layer formula on the SGLang
// PR #14105 page (LoRA for MoE expert layers), section 实现拆解, with the LoRA
// expand added ahead of the K loop, SiLU(gate) * up formed in the gate_up
// epilogue and the router weight applied in the down epilogue.
//
// Tile: 256 rows (pairs of one expert) x 256 weight rows (gate_up: 128 gate
// rows and the matching 128 up rows), 8 waves as 2 x 4, each wave 128 x 64 in
// 16 x 16 blocks of v_mfma_f32_16x16x32_bf16.  K tiles of 64 (128-byte LDS
// rows, 16-byte chunks XOR-swizzled by (row >> 1) & 7) stream through a
// two-slot ring filled by global -> LDS DMA.  The loop is software pipelined
// across its one barrier per K tile: after the barrier that admits tile s+1
// a wave first issues the DMA of tile s+2 into the slot tile s has vacated,
// then requests tile s+1's first fragments, then issues the MFMAs of tile s's
// second sub-step (fragments already in registers) -- the LDS latency of the
// new tile hides behind MFMA work and the DMA has two sub-steps of lead (the
// most a two-slot ring allows).  Against the
// 128 x 256 tile of the general kernel this moves 2/3 of the bytes per flop
// from L2 into LDS and reads 3/4 of the LDS bytes per flop.
//
// The persistent schedule (per-XCD tile ranges, a claim counter per XCD, one
// record per logical tile from the tile table) is the general kernel's; work
// items are at most 256 rows of one expert.  The waves of a short last item
// whose rows all lie past its end skip their MFMAs.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moelora {

namespace big {
constexpr int BM = 256;              // tile rows
constexpr int BN = 256;              // tile weight rows
constexpr int ROWB = 128;            // bytes of one LDS row: one K tile of 64 bf16
constexpr int BK = 64;
constexpr int NW = 8, WAVES_N = 4;   // 2 x 4 waves
constexpr int WM = 128, WN = 64;     // wave tile
constexpr int MB = WM / 16, NB = WN / 16;
constexpr int STAGE = (BM + BN) * ROWB;     // 64 KB
constexpr int SPW = STAGE / 1024 / NW;      // DMA instructions per wave per stage (1 KB each)
constexpr int A_WAVES = BM * ROWB / 1024 / SPW;   // waves 0..3 load A rows, 4..7 weight rows
constexpr int EXP_LD = 40;           // expand scratch: elements per column (32 ranks + pad)
constexpr int EP_GU_LD = 40;         // gate_up epilogue staging: row stride in bf16
#ifndef MOELORA_BIG_Z_ROWS
#define MOELORA_BIG_Z_ROWS 32
#endif
constexpr int Z_ROWS = MOELORA_BIG_Z_ROWS;   // down epilogue staging: rows per pass and wave
constexpr int EP_Z_LD = 68;          // and its row stride in fp32
constexpr int LDS_BYTES = 2 * STAGE;
static_assert(NW * 64 * EXP_LD * 2 <= STAGE, "expand scratch fits the second ring slot");
static_assert(NW * WM * EP_GU_LD * 2 <= LDS_BYTES, "gate_up staging fits");
constexpr int LDS_DOWN = NW * Z_ROWS * EP_Z_LD * 4 > LDS_BYTES ? NW * Z_ROWS * EP_Z_LD * 4 : LDS_BYTES;
static_assert(LDS_DOWN + 4096 <= 160 * 1024 && WM % Z_ROWS == 0 && Z_ROWS % 16 == 0, "down staging fits");
}  // namespace big

template <bool GATE_UP>
__global__ void __launch_bounds__(512) gemm_big_kernel(GemmArgs<bf16_t> a) {
  using namespace big;
  typedef bf16_t T;
  __shared__ __attribute__((aligned(1024))) char lds[GATE_UP ? LDS_BYTES : LDS_DOWN];
  __shared__ int ep_pid[BM];     // down epilogue: pair id of each tile row
  __shared__ float ep_w[BM];     // and its router weight
  __shared__ int claimed;

  const int count = min(a.item_count[0], a.max_items);
  const int total = count * a.n_tiles;
  const int xcd = blockIdx.x % 8;
  const int per_xcd = (total + 7) / 8;
  const int t_begin = xcd * per_xcd, t_end = min(total, t_begin + per_xcd);
  if (threadIdx.x == 0) claimed = atomicAdd(&a.tile_ctr[xcd], 1);
  __syncthreads();
  int logical = t_begin + __builtin_amdgcn_readfirstlane(claimed);
  int4 desc = a.tile_tab[max(min(logical, t_end - 1), 0)];
  while (logical < t_end) {
  int next_claim = 0;
  if (threadIdx.x == 0) next_claim = atomicAdd(&a.tile_ctr[xcd], 1);
  bool published = false;
  bool have_next = false;
  int4 next_desc;
  [&]() {
  // the record is wave-uniform: keep it in scalar registers so that every
  // test on it below is a scalar branch
  const int col_t = __builtin_amdgcn_readfirstlane(desc.w);
  const int64_t row0 = __builtin_amdgcn_readfirstlane(desc.x);
  const int nrows = __builtin_amdgcn_readfirstlane(desc.y);
  const int e = __builtin_amdgcn_readfirstlane(desc.z);
  if (col_t < 0 || col_t >= a.n_tiles || row0 < 0 || nrows <= 0 || nrows > BM || (nrows & 15) ||
      (row0 & 15) || row0 + nrows > a.cap || e < 0 || e >= a.E)
    return;
  const int split = col_t / a.n_cols;            // K split (split-major)
  const int ntile = col_t - split * a.n_cols;
  const int nk = (int)(a.K / a.ksplit / BK);     // K tiles of this split
  const int64_t kt0 = (int64_t)split * nk;
  const bool lora_here = a.h != nullptr && split == 0;
  __syncthreads();  // the previous tile's LDS use is over

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));   // recomputed per tile: not kept live across it
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane & 15, lk = 8 * (lane >> 4);
  const int64_t n0 = GATE_UP ? (int64_t)ntile * (BN / 2) : (int64_t)ntile * BN;
  auto swz = [](int row) -> int { return (row >> 1) & 7; };

  // the slot words of this wave's 16-row blocks, loaded first so that they
  // arrive with the pair ids below (one round trip).  Row numbers fit in 32
  // bits: a 32-bit divide each (a 64-bit divide's branches kept each load
  // behind the previous one's wait: eight round trips per tile start)
  int srv[MB];
  if (lora_here) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const uint32_t row = (uint32_t)row0 + (uint32_t)min(wm * WM + i * 16, nrows - 16);
      srv[i] = a.slot_rank[row / (uint32_t)a.BM_tile];
    }
  }
  // gate_up A rows are gathered: the pair id of each row this lane loads
  int pidv[SPW];
  if (GATE_UP && wave < A_WAVES) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int row = (wave * SPW + i) * 8 + lane / 8;
      pidv[i] = a.sorted_ids[row0 + min(row, nrows - 1)];
    }
  }
  // both groups of loads are out before either is used (left to itself the
  // compiler moves the slot words' first use ahead of the pair-id loads)
  if (GATE_UP && lora_here) {
    asm volatile("" ::"v"(srv[0]), "v"(srv[1]), "v"(srv[2]), "v"(srv[3]), "v"(srv[4]), "v"(srv[5]),
                 "v"(srv[6]), "v"(srv[7]));
    static_assert(MB == 8, "one operand per row block");
  }

  // 64-bit bases, 32-bit per-lane DMA offsets: the down A operand (act) is
  // addressed from the tile's first row; x and one expert's weights stay
  // under 4 GiB (host checks)
  const T* a_base = GATE_UP ? a.a_src : a.a_src + row0 * a.K;
  const T* b_base = static_cast<const T*>(a.w) + (int64_t)e * a.w_rows * a.K;
  uint32_t src_off[SPW];
  if (wave < A_WAVES) {
    // A rows: lane l of segment s fills LDS row 8 s + l / 8, slot l % 8 with
    // global chunk (l % 8) ^ swz(row); rows past nrows load the tile's first
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int row = (wave * SPW + i) * 8 + lane / 8;
      const int kc = (lane % 8) ^ swz(row);
      int64_t grow;
      if (GATE_UP) {
        const int pid = row < nrows ? pidv[i] : a.P;
        grow = pid < a.P ? pid / a.top_k : 0;
      } else {
        grow = row < nrows ? row : 0;
      }
      src_off[i] = (uint32_t)((grow * a.K + kc * 8) * 2);
    }
  } else {
    // weight rows n of the tile (LDS row BM + n; swz(BM + n) == swz(n));
    // columns past n_out load row 0 (never stored)
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int n = ((wave - A_WAVES) * SPW + i) * 8 + lane / 8;
      const int kc = (lane % 8) ^ swz(n);
      int64_t wrow;
      if (GATE_UP) {
        const int64_t col = n0 + (n % (BN / 2));
        wrow = col < a.n_out ? (n < BN / 2 ? col : a.n_out + col) : 0;
      } else {
        wrow = n0 + n < a.n_out ? n0 + n : 0;
      }
      src_off[i] = (uint32_t)((wrow * a.K + kc * 8) * 2);
    }
  }
  // LoRA slot and rank of each of this wave's 16-row blocks (one align block
  // or a part of one: a single slot each), -1 / 0 without LoRA
  // (packed as slot | rank << 16, -1 without LoRA, in scalar registers)
  int sr[MB];
  if (lora_here) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int v = __builtin_amdgcn_readfirstlane(srv[i]);
      sr[i] = wm * WM + i * 16 < nrows ? v : -1;
    }
    // resolved before the first DMA: the compiler does not count the
    // inline-asm DMA, so a wait placed after it would drain the DMA too
#pragma unroll
    for (int i = 0; i < MB; ++i) asm volatile("" ::"s"(sr[i]));
  }
  auto slot_of = [&](int i) -> int { return sr[i] >= 0 ? (sr[i] & 0xFFFF) : -1; };
  // every wave read the current claim before the barrier above
  if (threadIdx.x == 0) claimed = next_claim;
  published = true;

  const uint32_t lds_u32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int seg = wave * SPW + i;
      const void* base = wave < A_WAVES ? (const void*)a_base : (const void*)b_base;
      dma16(base, src_off[i] + (uint32_t)((kt0 + kt) * ROWB), lds_u32 + buf * STAGE + seg * 1024);
    }
  };

  floatx4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // every load issued so far has been used and every store of the previous
  // tile has been waited for by now; saying so with a wait the compiler sees
  // keeps it from placing one after the first stage's DMA (it does not count
  // the asm DMA, and a wait there drains it before the expand's loads go out)
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  issue(0, 0);

  // ---- LoRA expand: acc += h[rows, q] * Bpool[l, e, q, cols], ahead of the K loop
  // One pass per distinct slot of the wave's row blocks (first-seen order),
  // one step per 32 ranks.  Per step the wave loads its 32 rank rows x 64
  // columns of B (gate_up: 32 gate and the matching 32 up columns) with one
  // 16-byte load per lane and chunk, turns them into MFMA fragments through a
  // wave-private scratch in the second ring slot (filled by DMA only after
  // the barrier below), and multiplies the rows of each block holding the
  // slot: h = hi + lo, both bf16, stored split by the shrink (about 16 bits
  // of h survive).
  // Rank rows >= r and columns >= n_out are zero, never read.
  if (lora_here) {
    T* bt = reinterpret_cast<T*>(lds + STAGE) + wave * (64 * EXP_LD);
    // operand addresses as a wave-uniform base (scalar registers) plus one
    // 32-bit byte offset per lane: per-lane 64-bit addresses for every block
    // were spilled and reloaded behind the first stage's DMA
    // h: the lane's row in the wave's first block, at its K offset
    const char* hbase = reinterpret_cast<const char*>(a.h + (row0 + wm * WM) * a.HS);
    const uint32_t hoff = (uint32_t)((lrow * a.HS + lk) * 4);
    // blocks still to serve (wave-uniform bit mask); a pass serves every
    // block holding the slot of the lowest remaining one
    uint32_t todo = 0;
#pragma unroll
    for (int i = 0; i < MB; ++i) todo |= (sr[i] >= 0 ? 1u : 0u) << i;
    todo = __builtin_amdgcn_readfirstlane(todo);
    while (todo) {
      const int c = __builtin_ctz(todo);
      int v = -1;
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (i == c) v = sr[i];
      v = __builtin_amdgcn_readfirstlane(v);
      const int l = v & 0xFFFF, r = v >> 16;
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (slot_of(i) == l) todo &= ~(1u << i);
      for (int ks = 0; ks * 32 < r; ++ks) {
        int4v braw[4];
        const int64_t col0 = n0 + (GATE_UP ? wn * 32 : wn * 64);   // the wave's first column
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int ci = lane + 64 * t;
          const int pi = GATE_UP ? t >> 1 : 0;   // == ci >> 7: the pool is uniform per t
          const int rem = GATE_UP ? ci & 127 : ci;
          const int q = GATE_UP ? rem >> 2 : rem >> 3;
          const int cc = GATE_UP ? rem & 3 : rem & 7;
          const T* pool = pi ? a.b_pool1 : a.b_pool0;
          const char* pbase =
              reinterpret_cast<const char*>(pool + (((int64_t)l * a.E + e) * a.R + ks * 32) * a.n_out + col0);
          braw[t] = int4v{0, 0, 0, 0};
          if (ks * 32 + q < r && col0 + cc * 8 < a.n_out)
            braw[t] = *reinterpret_cast<const int4v*>(pbase + (uint32_t)((q * a.n_out + cc * 8) * 2));
        }
        // transpose through the scratch: (column n, rank q) at bt[n * EXP_LD + q]
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int ci = lane + 64 * t;
          const int pi = GATE_UP ? ci >> 7 : 0;
          const int rem = GATE_UP ? ci & 127 : ci;
          const int q = GATE_UP ? rem >> 2 : rem >> 3;
          const int cc = GATE_UP ? rem & 3 : rem & 7;
          const int nb = (GATE_UP ? pi * 32 : 0) + cc * 8;
          const bf16x8 v = __builtin_bit_cast(bf16x8, braw[t]);
#pragma unroll
          for (int u = 0; u < 8; ++u) bt[(nb + u) * EXP_LD + q] = v[u];
        }
        bf16x8 bfr[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(bt + (j * 16 + lrow) * EXP_LD + lk);
        // h of this lane's row in the blocks holding slot l, HB blocks at a
        // time (their loads go out together)
        constexpr int HB = GATE_UP ? 2 : 4;
        static_for<MB / HB>([&](auto G) {
          constexpr int g0 = decltype(G)::value * HB;
          floatx8 hg[HB], hu[HB];
          static_for<HB>([&](auto II) {
            constexpr int ii = decltype(II)::value, i = g0 + ii;
            hg[ii] = floatx8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            hu[ii] = hg[ii];
            if (slot_of(i) != l) return;
            // a block holding a slot lies inside nrows
            const char* hb = hbase + (((int64_t)i * 16) * a.HS + ks * 32) * 4;
            hg[ii] = *reinterpret_cast<const floatx8*>(hb + hoff);
            if (GATE_UP) hu[ii] = *reinterpret_cast<const floatx8*>(hb + (int64_t)a.RP * 4 + hoff);
          });
          static_for<HB>([&](auto II) {
            constexpr int ii = decltype(II)::value, i = g0 + ii;
            if (slot_of(i) != l) return;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              // h arrives split: the 32 bytes of the lane's 8 ranks hold their
              // 8 bf16 high parts, then the 8 low parts
              const int4v* hw = reinterpret_cast<const int4v*>((GATE_UP && j >= NB / 2) ? &hu[ii] : &hg[ii]);
              const bf16x8 hi = __builtin_bit_cast(bf16x8, hw[0]);
              const bf16x8 lo = __builtin_bit_cast(bf16x8, hw[1]);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bfr[j], acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bfr[j], acc[i][j], 0, 0, 0);
            }
          });
        });
      }
    }
  }

  // tile 0 has landed everywhere and every wave is done with its scratch
  wait_vm_barrier<0>();
  if (nk > 1) issue(1, 1);

  // ---- main loop ------------------------------------------------------------
  auto lfrag = [&](const char* base, int row, int ks) -> bf16x8 {
    const int kc = ks * 4 + (lane >> 4);
    return *reinterpret_cast<const bf16x8*>(base + row * ROWB + ((kc ^ swz(row)) * 16));
  };
  auto b_row = [&](int j) -> int {
    if (GATE_UP) return BM + (j < NB / 2 ? 0 : BN / 2) + wn * (WN / 2) + (j % (NB / 2)) * 16 + lrow;
    return BM + wn * WN + j * 16 + lrow;
  };
  // A fragments: one set, each block's reloaded for the next sub-step right
  // after its MFMAs (used again 7 blocks later); B fragments double-buffered
  bf16x8 fa[MB], fb[2][NB];
  auto load_b = [&](const char* base, int ks, int set) {
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[set][j] = lfrag(base, b_row(j), ks);
  };
  // LIVE: the wave has rows below nrows (all its MFMAs run; rows past nrows
  // compute values that are never stored).  A wave wholly past nrows (a short
  // last item) only takes its part in the DMA and the barriers.  (A test per
  // row block inside the loop costs more than the wasted rows.)
  auto main_loop = [&](auto live_c) {
    constexpr bool LIVE = decltype(live_c)::value;
    // one sub-step on B set `set`, each block's A fragment then replaced by
    // the one of sub-step ks_next of the tile in `nbase`
    auto step = [&](int set, const char* nbase, int ks_next) {
      if constexpr (LIVE) {
        static_for<MB>([&](auto I) {
          constexpr int i = decltype(I)::value;
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[set][j], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          fa[i] = lfrag(nbase, wm * WM + i * 16 + lrow, ks_next);
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto lb = [&](const char* base, int ks, int set) {
      if constexpr (LIVE) load_b(base, ks, set);
    };
    if constexpr (LIVE) {
#pragma unroll
      for (int i = 0; i < MB; ++i) fa[i] = lfrag(lds, wm * WM + i * 16 + lrow, 0);
    }
    lb(lds, 0, 0);
    for (int s = 0; s + 1 < nk; ++s) {
      const char* base = lds + (s & 1) * STAGE;
      const char* nxt = lds + ((s + 1) & 1) * STAGE;
      __builtin_amdgcn_sched_barrier(0);
      lb(base, 1, 1);
      step(0, base, 1);
      // tile s+1 has landed everywhere; every wave's reads of tile s are done
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // tile s's slot is free now: its refill goes out at once, so it has two
      // sub-steps (the rest of tile s and the first of tile s+1) to land
      // before the next barrier (issued after the second sub-step it had one:
      // c4p gate_up 7.38 -> 7.14 ms)
      if (s + 2 < nk) issue(s + 2, s & 1);
      __builtin_amdgcn_sched_barrier(0);
      lb(nxt, 0, 0);
      step(1, nxt, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    const char* last = lds + ((nk - 1) & 1) * STAGE;
    lb(last, 1, 1);
    step(0, last, 1);
    step(1, last, 1);   // (its reloads are dead: harmless reads of the last tile)
  };
  if (wm * WM < nrows)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();   // everyone is done reading the ring

  // the next tile's record, loaded now so that it has arrived when the
  // epilogue's stores are done (the claim was published before the K loop)
  next_desc = a.tile_tab[max(min(t_begin + __builtin_amdgcn_readfirstlane(claimed), t_end - 1), 0)];
  have_next = true;

  // ---- epilogue: through this wave's LDS region, so that every lane stores
  // 16 contiguous bytes of act (gate_up) or 12 of z (down): a lane's
  // accumulators hold one column of 4 rows
  if (GATE_UP) {
    T* ep = reinterpret_cast<T*>(lds) + wave * (WM * EP_GU_LD);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB / 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = acc[i][j][v], u = acc[i][j + NB / 2][v];
          ep[(i * 16 + 4 * (lane >> 4) + v) * EP_GU_LD + j * 16 + lrow] = (T)(silu_f(g) * u);
        }
    constexpr int CPR = (WN / 2) / 8;   // 16-byte chunks per staged row
#pragma unroll 4
    for (int c = lane; c < WM * CPR; c += 64) {
      const int r = c / CPR, cc = c % CPR;
      const int rloc = wm * WM + r;
      const int64_t col = n0 + wn * (WN / 2) + cc * 8;
      if (rloc >= nrows || col >= a.n_out) continue;
      *reinterpret_cast<int4v*>(a.act + (row0 + rloc) * a.n_out + col) =
          *reinterpret_cast<const int4v*>(ep + r * EP_GU_LD + cc * 8);
    }
  } else {
    for (int r = threadIdx.x; r < BM; r += 64 * NW) {
      const int pid = a.sorted_ids[row0 + min(r, nrows - 1)];
      ep_pid[r] = r < nrows ? pid : a.P;
      ep_w[r] = a.topk_weights[min(pid, a.P - 1)];
    }
    __syncthreads();   // ep_pid / ep_w are written by other waves
    // z rows in the 24-bit form (fp24_pack4), through this wave's LDS region
    // in passes of Z_ROWS rows: the lanes stage their accumulators (a lane holds one
    // column of 4 rows per block), then each takes 4 consecutive columns of
    // one row, weights them and stores 12 bytes (16 lanes: one row's 64
    // columns, 192 contiguous bytes)
    char* zb = static_cast<char*>(a.z);
    float* ep = reinterpret_cast<float*>(lds) + wave * (Z_ROWS * EP_Z_LD);
    constexpr int BPP = Z_ROWS / 16;   // row blocks per pass
#pragma unroll
    for (int ps = 0; ps < MB / BPP; ++ps) {
#pragma unroll
      for (int ii = 0; ii < BPP; ++ii)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            ep[(ii * 16 + 4 * (lane >> 4) + v) * EP_Z_LD + j * 16 + lrow] = acc[BPP * ps + ii][j][v];
      __builtin_amdgcn_wave_barrier();   // the wave's staging writes before its reads
#pragma unroll
      for (int c = lane; c < Z_ROWS * (WN / 4); c += 64) {
        const int r = c / (WN / 4), cc = c % (WN / 4);
        const int rloc = wm * WM + ps * Z_ROWS + r;
        const int64_t col = n0 + wn * WN + cc * 4;
        const int pid = ep_pid[rloc];
        if (rloc >= nrows || pid >= a.P || col >= a.n_out) continue;
        const float wgt = ep_w[rloc];
        floatx4 vv = *reinterpret_cast<const floatx4*>(ep + r * EP_Z_LD + cc * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) vv[q] = wgt * vv[q];
        *reinterpret_cast<u32x3*>(zb + (((int64_t)split * a.P + pid) * a.n_out + col) * 3) = fp24_pack4(vv);
      }
      __builtin_amdgcn_wave_barrier();   // and its reads before the next pass's writes
    }
  }
  }();
  if (!published) {   // a skipped tile: publish here
    __syncthreads();
    if (threadIdx.x == 0) claimed = next_claim;
    __syncthreads();
  }
  logical = t_begin + __builtin_amdgcn_readfirstlane(claimed);
  if (!have_next) next_desc = a.tile_tab[max(min(logical, t_end - 1), 0)];
  desc = next_desc;
  }  // persistent tile loop
}

int big_tile_rows() { return big::BM; }
int big_tile_cols(bool gate_up) { return gate_up ? big::BN / 2 : big::BN; }
int big_tile_k() { return big::BK; }

void launch_gemm_big(bool gate_up, const GemmArgs<bf16_t>& a, int64_t nblk, hipStream_t stream,
                     hipEvent_t ev0, hipEvent_t ev1) {
  void (*k)(GemmArgs<bf16_t>) = gate_up ? gemm_big_kernel<true> : gemm_big_kernel<false>;
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(64 * big::NW), 0, stream, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(64 * big::NW), 0, stream, a);
}

}  // namespace moelora
