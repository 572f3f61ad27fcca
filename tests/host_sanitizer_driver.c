/*
 * Host-side checks of the C ABI for the AddressSanitizer / UndefinedBehavior-
 * Sanitizer build of the library (tests/test_host_sanitizer.py).  Every call
 * here returns before any kernel launch: invalid arguments, refused sizes,
 * a missing workspace, size queries.  The pointers are stand-ins that the host
 * code checks for NULL and alignment but never dereferences.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_lora.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void* fake(uintptr_t i) { return (void*)(uintptr_t)(4096 * (i + 1)); }

static moe_lora_forward_args fwd_args(int32_t dtype, int32_t T, int32_t H, int32_t I, int32_t E,
                                      int32_t k, int32_t L, int32_t R, int32_t bm) {
  moe_lora_forward_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.dtype = dtype;
  a.num_tokens = T; a.hidden = H; a.inter = I; a.num_experts = E; a.top_k = k;
  a.num_loras = L; a.max_rank = R; a.block_m = bm;
  a.x = fake(0); a.topk_weights = (const float*)fake(1); a.w_gate_up = fake(2); a.w_down = fake(3);
  if (L > 0) {
    a.a_gate = fake(4); a.a_up = fake(5); a.b_gate = fake(6); a.b_up = fake(7);
    a.a_down = fake(8); a.b_down = fake(9);
    a.lora_ranks = (const int32_t*)fake(10); a.scaling = (const float*)fake(11);
  }
  a.sorted_pair_ids = (const int32_t*)fake(12); a.tile_expert = (const int32_t*)fake(13);
  a.tile_lora = (const int32_t*)fake(14); a.expert_tile_offsets = (const int32_t*)fake(15);
  a.num_rows_padded = (const int32_t*)fake(16);
  a.y = fake(17);
  a.out_dtype = dtype;
  a.weight_dtype = dtype;
  return a;
}

static moe_lora_dense_args dense_args(int32_t dtype, int32_t T, int32_t H, int32_t N0, int32_t N1,
                                      int32_t L, int32_t R, int32_t bm) {
  moe_lora_dense_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.dtype = dtype;
  a.num_tokens = T; a.hidden = H; a.out0 = N0; a.out1 = N1; a.num_loras = L; a.max_rank = R;
  a.block_m = bm;
  a.x = fake(0); a.w = fake(1);
  if (L > 0) {
    a.a0 = fake(2); a.b0 = fake(3); a.a1 = fake(4); a.b1 = fake(5);
    a.lora_ranks = (const int32_t*)fake(6); a.scaling = (const float*)fake(7);
  }
  a.sorted_pair_ids = (const int32_t*)fake(8); a.tile_expert = (const int32_t*)fake(9);
  a.tile_lora = (const int32_t*)fake(10); a.expert_tile_offsets = (const int32_t*)fake(11);
  a.num_rows_padded = (const int32_t*)fake(12);
  a.y = fake(13);
  a.out_dtype = dtype;
  return a;
}

static void check_status_strings(void) {
  for (int s = -8; s <= 2; ++s) EXPECT(moe_lora_status_str(s) != NULL);
  EXPECT(strstr(moe_lora_status_str(MOE_LORA_ERR_UNDERCOVER), "under-covers tokens") != NULL);
}

static void check_capacity(void) {
  /* P + min(P, E(L+1)) (BM - 1), rounded up to BM */
  EXPECT(moe_lora_align_capacity_rows(16384, 8, 256, 8, 16) == 165632);
  EXPECT(moe_lora_align_capacity_rows(0, 8, 256, 8, 16) == 0);
  EXPECT(moe_lora_align_capacity_rows(1, 1, 1, 0, 256) == 256);
  EXPECT(moe_lora_align_capacity_rows(4, 2, 8, 2, 17) == -1);
  EXPECT(moe_lora_align_capacity_rows(-1, 2, 8, 2, 16) == -1);
  /* sizes align refuses have no capacity; none of these may overflow */
  const int32_t big[] = {0, 1, 2, 255, 65535, 1 << 20, (1 << 30) - 1, INT32_MAX};
  for (int a = 0; a < 8; ++a)
    for (int b = 1; b < 8; ++b)
      for (int c = 1; c < 8; ++c)
        for (int d = 0; d < 8; ++d) {
          int64_t cap = moe_lora_align_capacity_rows(big[a], big[b], big[c], big[d], 256);
          int64_t P = (int64_t)big[a] * big[b];
          if (P > INT32_MAX / 2 || (int64_t)big[c] * ((int64_t)big[d] + 1) > 32768)
            EXPECT(cap == -1);
          else
            EXPECT(cap >= P && cap % 256 == 0);
          size_t ws = moe_lora_align_workspace_bytes(big[a], big[b], big[c], big[d], 256);
          EXPECT((cap < 0) == (ws == 0));
        }
}

static void check_route_info_align(void) {
  int32_t* p = (int32_t*)fake(20);
  float* f = (float*)fake(21);
  EXPECT(moe_lora_route(-1, 8, 2, f, p, f, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_route(4, 8, 9, f, p, f, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_route(4, 8, 0, f, p, f, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_route(4, 8, 2, NULL, p, f, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_route(4, 4096, 4096, f, p, f, NULL) == MOE_LORA_ERR_UNSUPPORTED);

  EXPECT(moe_lora_info(-1, 1, 0, 0, p, p, NULL, NULL, p, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_info(4, 0, 0, 0, p, p, NULL, NULL, p, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_info(9, 2, 2, 4, p, p, p, p, p, NULL) == MOE_LORA_ERR_UNDERCOVER);
  EXPECT(moe_lora_info(INT32_MAX, 2, 2, INT32_MAX / 2, p, p, p, p, p, NULL) ==
         MOE_LORA_ERR_UNDERCOVER);
  EXPECT(moe_lora_info(4, 1, 2, 0, p, p, NULL, p, p, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_info(4, 1, 0, 0, NULL, p, NULL, NULL, p, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_info(0, 0, 0, 0, p, NULL, NULL, NULL, NULL, NULL) == MOE_LORA_OK);

  EXPECT(moe_lora_align(4, 2, 8, 2, 8, p, p, p, p, p, p, p, p, fake(22), 1 << 20, NULL) ==
         MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_align(4, 9, 8, 2, 16, p, p, p, p, p, p, p, p, fake(22), 1 << 20, NULL) ==
         MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_align(1 << 28, 8, 256, 8, 16, p, p, p, p, p, p, p, p, fake(22), 1 << 20, NULL) ==
         MOE_LORA_ERR_UNSUPPORTED);
  EXPECT(moe_lora_align(4, 2, 4096, 8, 16, p, p, p, p, p, p, p, p, fake(22), 1 << 20, NULL) ==
         MOE_LORA_ERR_UNSUPPORTED);
  EXPECT(moe_lora_align(4, 2, 8, 2, 16, p, p, NULL, p, p, p, p, p, fake(22), 1 << 20, NULL) ==
         MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_align(4, 2, 8, 2, 16, p, p, p, p, p, p, p, p, NULL, 1 << 20, NULL) ==
         MOE_LORA_ERR_WORKSPACE);
  EXPECT(moe_lora_align(4, 2, 8, 2, 16, p, p, p, p, p, p, p, p, fake(22), 1, NULL) ==
         MOE_LORA_ERR_WORKSPACE);
  {
    uint32_t flags = 7;
    EXPECT(moe_lora_debug_flags(NULL, 0, NULL) == MOE_LORA_ERR_INVALID);
    EXPECT(moe_lora_debug_flags(&flags, 0, NULL) == MOE_LORA_ERR_UNSUPPORTED && flags == 0);
  }
}

static void check_forward(void) {
  /* the layer shapes of the workloads, bf16 / fp32 / fp8, up to the size limits */
  const int32_t shapes[][8] = {
      /* T, H, I, E, k, L, R, bm */
      {8, 256, 512, 4, 2, 4, 16, 16},        {4096, 4096, 14336, 8, 2, 8, 64, 16},
      {16384, 2048, 768, 128, 8, 16, 32, 16}, {64, 2048, 768, 128, 8, 32, 32, 16},
      {16384, 7168, 2048, 256, 8, 8, 32, 16}, {128, 7168, 2048, 256, 8, 8, 32, 64},
      {1, 64, 64, 1, 1, 0, 0, 16},            {(1 << 30) / 8 - 1, 64, 64, 256, 8, 8, 64, 256},
      {262143, 8192, 8192, 256, 8, 8, 64, 256}, {1, 16384, 16384, 4096, 8, 7, 64, 16},
  };
  const int nshape = (int)(sizeof(shapes) / sizeof(shapes[0]));
  for (int i = 0; i < nshape; ++i)
    for (int dt = 0; dt < 3; ++dt) {
      const int32_t* s = shapes[i];
      const int32_t dtype = dt == 0 ? MOE_LORA_F32 : MOE_LORA_BF16;
      moe_lora_forward_args a = fwd_args(dtype, s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]);
      if (dt == 2) {
        a.weight_dtype = MOE_LORA_FP8_E4M3;
        a.w_gate_up_scale = (const float*)fake(30);
        a.w_down_scale = (const float*)fake(31);
      }
      const size_t need = moe_lora_forward_workspace_bytes(&a);
      const int64_t esz = dtype == MOE_LORA_BF16 ? 2 : 4;
      const int64_t wsz = dt == 2 ? 1 : esz;
      const int fp8_bad = dt == 2 && (s[1] % 128 || s[2] % 128);
      const int too_big = (int64_t)s[0] * s[1] * esz >= ((int64_t)1 << 32) ||
                          2 * (int64_t)s[2] * s[1] * wsz >= ((int64_t)1 << 32);
      const int ok = !fp8_bad && !too_big;
      EXPECT(ok ? need > 0 : need == 0);
      /* no workspace: refused after every other check, before any launch */
      const int st = moe_lora_forward(&a, NULL);
      EXPECT(st == (ok ? MOE_LORA_ERR_WORKSPACE : MOE_LORA_ERR_UNSUPPORTED));
      a.workspace = fake(40);
      a.workspace_bytes = need ? need - 1 : 0;
      if (ok) EXPECT(moe_lora_forward(&a, NULL) == MOE_LORA_ERR_WORKSPACE);
      if (ok && need > moe_lora_forward_noalloc_max_workspace_bytes())
        EXPECT(moe_lora_forward_noalloc(&a, NULL) == MOE_LORA_ERR_WORKSPACE);
    }

  moe_lora_forward_args a = fwd_args(MOE_LORA_BF16, 64, 2048, 768, 128, 8, 32, 32, 16);
  moe_lora_forward_args b;
  b = a; b.hidden = 2056; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_UNSUPPORTED);
  b = a; b.max_rank = 65; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_UNSUPPORTED);
  b = a; b.top_k = 129; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_INVALID);
  b = a; b.block_m = 24; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_INVALID);
  b = a; b.dtype = 7; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_UNSUPPORTED);
  b = a; b.out_dtype = 5; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_UNSUPPORTED);
  b = a; b.struct_size = 8; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_INVALID);
  b = a; b.a_up = NULL; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_INVALID);
  b = a; b.x = (const char*)a.x + 2; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_INVALID);
  b = a; b.weight_dtype = MOE_LORA_FP8_E4M3;
  EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_INVALID);       /* no block scales */
  b.inter = 832;
  EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_ERR_UNSUPPORTED);   /* I no multiple of 128 */
  EXPECT(moe_lora_forward(NULL, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_forward_events(&a, NULL, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_forward_workspace_bytes(NULL) == 0);
  b = a; b.num_tokens = 0; EXPECT(moe_lora_forward(&b, NULL) == MOE_LORA_OK);
}

static void check_dense(void) {
  const int32_t shapes[][7] = {
      /* T, H, N0, N1, L, R, bm */
      {4096, 7168, 1536, 576, 8, 16, 16}, {64, 7168, 1536, 576, 32, 32, 16},
      {1, 64, 64, 0, 0, 0, 16},           {(1 << 30) - 1, 64, 64, 64, 4, 64, 256},
      {262143, 8192, 8192, 8192, 8, 64, 16},
  };
  for (int i = 0; i < 5; ++i)
    for (int dt = 0; dt < 2; ++dt) {
      const int32_t* s = shapes[i];
      const int32_t dtype = dt ? MOE_LORA_BF16 : MOE_LORA_F32;
      moe_lora_dense_args a = dense_args(dtype, s[0], s[1], s[2], s[3], s[4], s[5], s[6]);
      const int64_t esz = dt ? 2 : 4;
      const int ok = (int64_t)s[0] * s[1] * esz < ((int64_t)1 << 32) &&
                     ((int64_t)s[2] + s[3]) * s[1] * esz < ((int64_t)1 << 32);
      const size_t need = moe_lora_dense_workspace_bytes(&a);
      EXPECT(ok ? need > 0 : need == 0);
      EXPECT(moe_lora_dense_forward(&a, NULL) ==
             (ok ? MOE_LORA_ERR_WORKSPACE : MOE_LORA_ERR_UNSUPPORTED));
    }
  moe_lora_dense_args a = dense_args(MOE_LORA_BF16, 64, 7168, 1536, 576, 32, 32, 16);
  moe_lora_dense_args b;
  b = a; b.out1 = 100; EXPECT(moe_lora_dense_forward(&b, NULL) == MOE_LORA_ERR_UNSUPPORTED);
  b = a; b.b1 = NULL; EXPECT(moe_lora_dense_forward(&b, NULL) == MOE_LORA_ERR_INVALID);
  b = a; b.struct_size = 16; EXPECT(moe_lora_dense_forward(&b, NULL) == MOE_LORA_ERR_INVALID);
  EXPECT(moe_lora_dense_forward_events(&a, NULL, NULL) == MOE_LORA_ERR_INVALID);
}

int main(void) {
  check_status_strings();
  check_capacity();
  check_route_info_align();
  check_forward();
  check_dense();
  if (failures) {
    fprintf(stderr, "%d host checks failed\n", failures);
    return 1;
  }
  printf("all host checks passed\n");
  return 0;
}
