/* Plain-C consumer of include/routed_moe.h: compiled with gcc against the header and the
 * shared library, it calls only host-side entry points (sizes, layouts, status strings)
 * and argument validation that returns before any HIP call, so it runs without a GPU.
 * Prints "ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "routed_moe.h"

static int failures = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);     \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

int main(void) {
  moe_dims_t d = {3584, 384, 896, 16};
  size_t ws16 = 0, ws16k = 0, prep = 0, route = 0;
  CHECK(moe_workspace_size(d, 16, MOE_QUANT_NVFP4_G16, &ws16) == MOE_OK);
  CHECK(moe_workspace_size(d, MOE_MAX_TOKENS, MOE_QUANT_NVFP4_G16, &ws16k) == MOE_OK);
  CHECK(ws16 > 0 && ws16 <= ws16k);
  CHECK(moe_prepared_weights_size(d, &prep) == MOE_OK);
  /* FC1 codes + scales and FC2 codes + scales of 896 experts */
  CHECK(prep == (size_t)896 * (768 * 1792 + 768 * 224 + 3584 * 192 + 3584 * 24));
  moe_workspace_layout_t lay;
  CHECK(moe_workspace_layout(d, 16, &lay) == MOE_OK);
  CHECK(lay.total == ws16 && lay.x_codes < lay.total && lay.o_rows < lay.total);
  CHECK(moe_route_workspace_size(8192, 8, 256, &route) == MOE_OK && route > 0);
  /* the routing-only workload's dims: moe_route ignores inter */
  moe_dims_t rd = {7168, 0, 256, 8};
  size_t rws = 0, rws_fp4 = 0;
  CHECK(moe_workspace_size(rd, 8192, MOE_QUANT_INT8_ROW_DYNAMIC, &rws) == MOE_OK && rws == route);
  CHECK(moe_workspace_size(rd, 8192, MOE_QUANT_NVFP4_G16, &rws_fp4) == MOE_ERR_INVALID_ARG);
  CHECK(moe_route(rd, 8192, (const uint16_t*)0x1000, (const int32_t*)0x2000, MOE_QUANT_NVFP4_G16,
                  NULL, NULL, NULL, (int32_t*)0x3000, (int32_t*)0x4000, (void*)0x5000,
                  (void*)0x6000, (void*)0x7000, route, 0) == MOE_ERR_INVALID_ARG); /* no qx */
  moe_ring_layout_t rl;
  CHECK(moe_ring_layout(d, 2, 64, &rl) == MOE_OK && rl.total > rl.counters);

  /* validation errors come back as codes, before any device work */
  moe_dims_t bad = {3584, 384, 896, 0};
  CHECK(moe_workspace_size(bad, 16, MOE_QUANT_NVFP4_G16, &ws16) == MOE_ERR_INVALID_ARG);
  moe_dims_t odd = {3500, 384, 896, 16};
  CHECK(moe_workspace_size(odd, 16, MOE_QUANT_NVFP4_G16, &ws16) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_forward(d, 16, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                    0, NULL, 0) == MOE_ERR_INVALID_ARG);
  CHECK(moe_topk_softmax(16, 896, 17 * 60, (const float*)0x1000, (int32_t*)0x2000,
                         (uint16_t*)0x3000, 0) == MOE_ERR_INVALID_ARG);
  moe_route_options_t o;
  memset(&o, 0, sizeof(o));
  o.quant_mode = 5;
  CHECK(moe_route_v2(64, 256, 32, 8, (const uint16_t*)0x1000, (const int32_t*)0x2000, NULL, NULL,
                     &o, (void*)0x3000, (int32_t*)0x4000, NULL, NULL, NULL, (void*)0x5000,
                     route, 0) == MOE_ERR_INVALID_ARG);
  /* layouts and sizes over many batch sizes and expert counts (host arithmetic only) */
  for (int T = 1; T <= MOE_MAX_TOKENS; T += 997) {
    size_t n = 0;
    moe_workspace_layout_t l;
    CHECK(moe_workspace_size(d, T, MOE_QUANT_NVFP4_G16, &n) == MOE_OK);
    CHECK(moe_workspace_layout(d, T, &l) == MOE_OK && l.total <= n && l.o_exp < l.total);
  }
  size_t sealed = 0;
  CHECK(moe_sealed_workspace_size(d, 16384, &sealed) == MOE_OK && sealed > 0);
  for (int E = 1; E <= 10240; E = 2 * E + 1)
    CHECK(moe_route_workspace_size(4096, 8, E, &route) == MOE_OK && route > 0);
  CHECK(moe_route_workspace_size(4096, 8, 10241, &route) != MOE_OK);
  /* the allocation-free entry point rejects batches beyond its fixed array up front */
  CHECK(moe_forward_noalloc(d, 263, (const uint16_t*)0x1000, (const int32_t*)0x2000,
                            (const uint16_t*)0x3000, (const void*)0x4000, (const float*)0x5000,
                            (const float*)0x6000, (const float*)0x7000, (const float*)0x8000,
                            NULL, NULL, (uint16_t*)0x9000, 0) == MOE_ERR_UNSUPPORTED);
  CHECK(strcmp(moe_status_string(MOE_OK), "ok") == 0);
  CHECK(moe_status_string((moe_status_t)12345) != NULL);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
