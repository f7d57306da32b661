/*
 * Drives the host half of the C ABI (include/txl.h) without a GPU, for a build
 * whose txl_api.cpp is compiled with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host side: the size queries, the status
 * strings and every argument check that returns before a launch.  Device
 * addresses are fake; no call here reaches the GPU.  Exits non-zero if a call
 * returns something other than the documented error.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/txl.h"

static int fails = 0;
#define EXPECT(cond)                                             \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "line %d: expectation failed\n", __LINE__); \
      ++fails;                                                   \
    }                                                            \
  } while (0)

static void* fake(uintptr_t gib) { return (void*)(gib << 30); }

int main(void) {
  for (int s = -5; s <= 1; ++s) EXPECT(strlen(txl_status_string(s)) > 0);
  txl_layer_dims dm = {22, 512, 512, 8, 64, 1e-5f};
  EXPECT(txl_layer_workspace_bytes(&dm, 512, TXL_BF16) > 0);
  EXPECT(txl_layer_workspace_bytes(&dm, 512, 7) == 0);
  EXPECT(txl_layer_bwd_workspace_bytes(&dm, 512, TXL_BF16) > 0);
  EXPECT(txl_layer_saved_bytes(&dm, 512, TXL_BF16) > 0);
  EXPECT(txl_layer_kv_workspace_bytes(&dm, 512, TXL_BF16) > 0);
  EXPECT(txl_kv_ring_bytes(&dm, 1024, TXL_BF16) == (size_t)22 * 8 * 1024 * 64 * 2);
  EXPECT(txl_pos_ff_workspace_bytes(11264, 512, 2048, TXL_BF16) > 0);
  EXPECT(txl_rel_attn_workspace_bytes(TXL_BF16, 1, 16, 128, 1600, 64) > 0);
  EXPECT(txl_rel_attn_bwd_workspace_bytes(TXL_BF16, 1, 16, 128, 1600, 64) > 0);
  EXPECT(txl_rel_attn_noalloc_max_scratch_bytes() == (size_t)16 << 20);
  txl_workspace_map map;
  EXPECT(txl_layer_workspace_map(&dm, 512, TXL_BF16, &map) == TXL_OK && map.d_pad == 64);
  txl_layer_dims bad = dm;
  bad.d_head = 200;
  EXPECT(txl_layer_workspace_map(&bad, 512, TXL_BF16, &map) == TXL_EUNSUPPORTED);
  bad = dm;
  bad.B = 0;
  EXPECT(txl_layer_workspace_bytes(&bad, 512, TXL_BF16) == 0);

  /* attention: NULL tensors, unsupported sizes, out overlapping q, too few r rows */
  const int64_t B = 2, H = 4, L = 64, M = 32, d = 64, T = M + L;
  void *q = fake(1), *k = fake(2), *v = fake(3), *r = fake(4), *u = fake(5), *vb = fake(6),
       *out = fake(7);
  EXPECT(txl_rel_attn_fwd(NULL, TXL_BF16, B, H, L, M, d, NULL, L * H * d, H * d, d, k, v,
                          T * H * d, H * d, d, r, H * d, d, T, u, vb, 0.125f, out, L * H * d,
                          H * d, d, NULL, NULL, 0) == TXL_EINVAL);
  EXPECT(txl_rel_attn_fwd(NULL, TXL_BF16, B, H, L, M, 129, q, L * H * 129, H * 129, 129, k, v,
                          T * H * 129, H * 129, 129, r, H * 129, 129, T, u, vb, 0.125f, out,
                          L * H * 129, H * 129, 129, NULL, NULL, 0) == TXL_EUNSUPPORTED);
  EXPECT(txl_rel_attn_fwd(NULL, TXL_BF16, B, H, L, M, d, q, L * H * d, H * d, d, k, v,
                          T * H * d, H * d, d, r, H * d, d, T, u, vb, 0.125f, q, L * H * d,
                          H * d, d, NULL, NULL, 0) == TXL_EINVAL);
  EXPECT(txl_rel_attn_fwd(NULL, TXL_BF16, B, H, L, M, d, q, L * H * d, H * d, d, k, v,
                          T * H * d, H * d, d, r, H * d, d, T - 1, u, vb, 0.125f, out,
                          L * H * d, H * d, d, NULL, NULL, 0) == TXL_EINVAL);
  /* the split of a 1 x 16 x 1600 x 1600 block needs more than the static scratch */
  EXPECT(txl_rel_attn_fwd_noalloc(NULL, TXL_BF16, 1, 16, 1600, 1600, 64, fake(1), 16 * 1600 * 64,
                                  64, 1600 * 64, fake(2), fake(3), 16 * 3200 * 64, 64, 3200 * 64,
                                  fake(4), 64, 3200 * 64, 3200, fake(5), fake(6), 0.125f,
                                  fake(7), 1600 * 16 * 64, 16 * 64, 64, NULL) == TXL_EWORKSPACE);

  /* memory update: ring state checks leave the ring untouched */
  txl_ring ring = {fake(8), 16, 3, 17};
  EXPECT(txl_mem_update(NULL, TXL_BF16, &ring, 2, 64, fake(9), 8) == TXL_EINVAL);
  EXPECT(ring.start == 3 && ring.len == 17);
  ring.len = 4;
  EXPECT(txl_mem_update(NULL, TXL_BF16, &ring, 2, 64, NULL, 8) == TXL_EINVAL);

  /* layer step: workspace too small, h_out aliasing h_in, unaligned workspace */
  txl_layer_weights w = {fake(10), fake(11), fake(12), fake(13), fake(14), fake(15), fake(16)};
  txl_ring mem = {fake(17), 512, 0, 512};
  const size_t need = txl_layer_workspace_bytes(&dm, 512, TXL_BF16);
  EXPECT(txl_layer_step(NULL, TXL_BF16, &dm, fake(18), &mem, &w, u, vb, fake(19), 1024, fake(20),
                        fake(21), need - 256) == TXL_EWORKSPACE);
  EXPECT(txl_layer_step(NULL, TXL_BF16, &dm, fake(18), &mem, &w, u, vb, fake(19), 1024, fake(18),
                        fake(21), need) == TXL_EINVAL);
  EXPECT(txl_layer_step(NULL, TXL_BF16, &dm, fake(18), &mem, &w, u, vb, fake(19), 1024, fake(20),
                        (char*)fake(21) + 16, need) == TXL_EINVAL);
  EXPECT(txl_layer_step(NULL, TXL_BF16, &dm, fake(18), &mem, &w, u, vb, fake(19), 1000, fake(20),
                        fake(21), need) == TXL_EINVAL);

  /* the backward with a saved state taken at another ring position */
  txl_layer_saved sv;
  memset(&sv, 0, sizeof(sv));
  sv.data = fake(22);
  sv.bytes = txl_layer_saved_bytes(&dm, 512, TXL_BF16);
  sv.mem_data = mem.data;
  sv.mem_capacity = 512;
  sv.mem_start = 100;
  sv.mem_len = 512;
  sv.h_in = fake(18);
  sv.B = dm.B; sv.L = dm.L; sv.d_model = dm.d_model; sv.n_head = dm.n_head;
  sv.d_head = dm.d_head;
  sv.dtype = TXL_BF16;
  txl_layer_grads g = {(float*)fake(30), (float*)fake(31), (float*)fake(32), (float*)fake(33),
                       (float*)fake(34), (float*)fake(35), (float*)fake(36), (float*)fake(37),
                       (float*)fake(38), (float*)fake(39)};
  EXPECT(txl_layer_step_bwd_saved(NULL, TXL_BF16, &dm, fake(18), &mem, &w, u, vb, fake(19), 1024,
                                  fake(23), &sv, &g, fake(40),
                                  txl_layer_bwd_workspace_bytes(&dm, 512, TXL_BF16)) ==
         TXL_EINVAL);
  EXPECT(strstr(txl_status_string(TXL_EINVAL), "memory differs") != NULL);

  /* evaluation cache: capacity below mem_max + L */
  txl_kv_ring kv = {fake(24), fake(25), 600, 0, 0, 512};
  EXPECT(txl_layer_step_kv(NULL, TXL_BF16, &dm, fake(18), &kv, &w, u, vb, fake(26), 1024,
                           fake(20), fake(21), txl_layer_kv_workspace_bytes(&dm, 512, TXL_BF16)) ==
         TXL_EINVAL);
  printf("abi driver done, %d failed expectations\n", fails);
  return fails ? 1 : 0;
}
