/*
 * Host-only driver of the C ABI for the sanitizer build (AddressSanitizer +
 * UndefinedBehaviorSanitizer on the host code of nc.cpp): every entry point's
 * host-side validation, sizing and layout paths, with no GPU work.  Prints
 * "ok" and exits 0 when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "../include/nc.h"

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

static nc_config cfg(int depth, int vocab, int seq, int batch, int dtype) {
  nc_config c;
  memset(&c, 0, sizeof(c));
  c.depth = depth;
  c.vocab = vocab;
  c.seq_len = seq;
  c.max_batch = batch;
  c.dtype = dtype;
  return c;
}

int main(void) {
  for (int code = -1; code <= 9; ++code) CHECK(nc_strerror(code) != NULL);

  nc_ctx* ctx = NULL;
  nc_config c = cfg(20, 65536, 2048, 32, NC_BF16);
  CHECK(nc_init(NULL, NULL, &ctx) == NC_ERR_NULL);
  CHECK(nc_init(&c, NULL, NULL) == NC_ERR_NULL);
  CHECK(nc_init(&c, NULL, &ctx) == NC_OK && ctx != NULL);
  nc_config out;
  CHECK(nc_get_config(ctx, &out) == NC_OK);
  CHECK(out.d_model == 1280 && out.n_heads == 10 && out.head_dim == 128 && out.d_ff == 5120);
  CHECK(nc_param_count(ctx) == 560988160ull);
  CHECK(nc_param_layout(ctx, NULL, 0) == 82);
  nc_tensor_desc d[82];
  CHECK(nc_param_layout(ctx, d, 3) == 82);
  CHECK(nc_param_layout(ctx, d, 82) == 82);
  CHECK(strcmp(d[0].name, "E") == 0 && strcmp(d[81].name, "W_lm") == 0);
  CHECK(d[81].offset + (uint64_t)d[81].rows * d[81].cols == nc_param_count(ctx));
  CHECK(nc_workspace_bytes(ctx, 0) == 0);
  CHECK(nc_workspace_bytes(ctx, 33) == 0);
  CHECK(nc_workspace_bytes(ctx, 1) > 0 && nc_workspace_bytes(ctx, 32) > nc_workspace_bytes(ctx, 1));
  CHECK(nc_kv_cache_bytes(ctx, 1, 0) == 0 && nc_kv_cache_bytes(ctx, 2, 1024) > 0);
  CHECK(nc_decode_workspace_bytes(ctx, 4, 4096) > 0);
  CHECK(nc_optim_state_bytes(ctx) > 0 && nc_optim_workspace_bytes(ctx) > 0);
  CHECK(nc_optim_state_bytes(NULL) == 0);
  /* every compute entry point rejects bad arguments on the host */
  float f = 0.f;
  int32_t ids[4] = {0, 1, 2, 3};
  CHECK(nc_forward_backward(NULL, &f, ids, ids, 1, &f, &f, 0) == NC_ERR_NULL);
  CHECK(nc_forward_backward(ctx, NULL, ids, ids, 1, &f, &f, 0) == NC_ERR_NULL);
  CHECK(nc_forward_backward(ctx, &f, ids, ids, 0, &f, &f, 0) == NC_ERR_ARG);
  CHECK(nc_forward_backward(ctx, &f, ids, ids, 1, &f, &f, 2) == NC_ERR_ARG);
  CHECK(nc_forward_backward(ctx, &f, ids, ids, 1, &f, &f, 0) == NC_ERR_WORKSPACE);
  CHECK(nc_forward_backward_accum(ctx, &f, ids, ids, 0, 1, &f, &f) == NC_ERR_ARG);
  CHECK(nc_forward_logits(ctx, &f, ids, 1, NULL) == NC_ERR_NULL);
  CHECK(nc_forward_logits(ctx, &f, ids, 1, &f) == NC_ERR_WORKSPACE);
  CHECK(nc_set_workspace(ctx, (void*)0x1001, 1 << 20) == NC_ERR_ARG);
  CHECK(nc_check(ctx) == NC_ERR_WORKSPACE);
  CHECK(nc_prefill(ctx, &f, ids, 1, 0, &f, 1, 64, 0, &f) == NC_ERR_ARG);
  CHECK(nc_decode(ctx, &f, ids, ids, 0, &f, 64, &f, 0, &f) == NC_ERR_ARG);
  CHECK(nc_decode(ctx, &f, ids, ids, 1, &f, 64, (void*)0x1001, 1 << 20, &f) == NC_ERR_ARG);
  CHECK(nc_decode_static(ctx, &f, ids, ids, 1, &f, 64, &f, NULL) == NC_ERR_NULL);
  CHECK(nc_decode_static(ctx, &f, ids, ids, 0, &f, 64, &f, ids) == NC_ERR_ARG);
  CHECK(nc_decode_static(ctx, &f, ids, ids, 64, &f, 65536, &f, ids) == NC_ERR_WORKSPACE);
  CHECK(nc_debug_poison_workspace(ctx, 2) == NC_ERR_ARG);
  CHECK(nc_debug_poison_workspace(ctx, 1) == NC_OK && nc_debug_poison_workspace(ctx, 0) == NC_OK);
  CHECK(nc_set_residual_fp32(NULL, 1) == NC_ERR_NULL && nc_set_residual_fp32(ctx, 2) == NC_ERR_ARG);
  CHECK(nc_set_residual_fp32(ctx, 1) == NC_OK && nc_set_residual_fp32(ctx, 0) == NC_OK);
  CHECK(nc_profile_enable(NULL, 1) == NC_ERR_NULL);
  nc_optim_config oc;
  memset(&oc, 0, sizeof(oc));
  CHECK(nc_optim_step(ctx, &oc, 0, &f, &f, &f, &f, 0, NULL) == NC_ERR_ARG);
  nc_destroy(ctx);

  /* op entry points: sizes and host-side validation */
  CHECK(nc_attention_workspace_bytes(16, 10, 2048, 128, NC_BF16) > 0);
  CHECK(nc_attention_workspace_bytes(1, 1, 1, 24, NC_BF16) == 0);
  CHECK(nc_attention_fwd_bwd(&f, &f, &f, &f, &f, &f, &f, &f, 1, 1, 40000, 128, 10000.f, 1e-6f, NC_BF16, &f, 0,
                             NULL) == NC_ERR_UNSUPPORTED);
  CHECK(nc_lmhead_ce_workspace_bytes(32768, 1280, 65536, NC_BF16) > 0);
  CHECK(nc_lmhead_ce_fwd_bwd(&f, &f, ids, 3, 7, 64, &f, &f, &f, NC_BF16, &f, 0, NULL) == NC_ERR_ARG);
  CHECK(nc_gemm_workspace_bytes(256, 264, 8200, NC_BF16) > 0);
  CHECK(nc_gemm(&f, 8, 1, &f, 8, 1, &f, 8, 8, 6, 8, 0, NC_BF16, NULL, 0, NULL) == NC_ERR_ARG);
  CHECK(nc_embedding_bwd_workspace_bytes(5000, 64, 65536) > 0);
  CHECK(nc_rmsnorm_fwd(&f, &f, &f, 4, 6, 1e-6f, NC_BF16, NULL) == NC_ERR_ARG);

  /* other configurations: grouped-query, fp32, bad ones */
  c = cfg(4, 1024, 128, 2, NC_BF16);
  c.n_kv_heads = 2;
  c.d_model = 512;
  CHECK(nc_init(&c, NULL, &ctx) == NC_OK);
  CHECK(nc_param_layout(ctx, NULL, 0) == 18);
  nc_destroy(ctx);
  c = cfg(2, 512, 64, 2, NC_FP32);
  c.d_model = 128; c.n_heads = 4; c.head_dim = 32;
  CHECK(nc_init(&c, NULL, &ctx) == NC_OK);
  nc_destroy(ctx);
  c = cfg(2, 500, 64, 2, NC_BF16);
  ctx = NULL;
  CHECK(nc_init(&c, NULL, &ctx) == NC_ERR_CONFIG && ctx == NULL);
  c = cfg(2, 512, 40000, 1, NC_BF16);
  CHECK(nc_init(&c, NULL, &ctx) == NC_ERR_UNSUPPORTED);

  if (fails) return 1;
  printf("ok\n");
  return 0;
}
