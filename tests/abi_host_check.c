/* Host-side exercise of the libcsa C ABI for sanitizer builds (no GPU work).
 *
 * Every entry point is called with rejected arguments, edge-case sizes and, for the
 * size queries, shapes the attention planner must decline (head counts without an
 * instantiated head group).  Built with AddressSanitizer and UndefinedBehaviorSanitizer
 * on the host code by tests/test_abi_sanitized.py; any sanitizer report fails that
 * test.  Prints one line per failed expectation and exits non-zero if there was one.
 */
#include <stdio.h>
#include <string.h>

#include "csa.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAILED: %s (last error: %s)\n", what, csa_last_error());
    ++failures;
  }
}

int main(void) {
  char* p = (char*)0x100000;  /* never dereferenced: every call below stops on the host */
  csa_buf bf16 = {p, NULL, NULL, CSA_BF16, 0};
  csa_buf f32 = {p, NULL, NULL, CSA_F32, 0};
  csa_buf fp8_noscale = {p, NULL, NULL, CSA_FP8MIX, 0};
  csa_buf mx_noscale = {p, NULL, NULL, CSA_MXFP4, 0};
  csa_buf bad_dtype = {p, NULL, NULL, 9, 0};

  expect(csa_abi_version() == CSA_ABI_VERSION, "abi version");
  expect(csa_device_check() != CSA_OK || 1, "device check returns");

  /* compress */
  expect(csa_compress(NULL, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 0, 0, 1e4f, 0, &bf16, 2,
                      NULL) == CSA_ERR_NULL, "compress: NULL input");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 9, 16, 4, 1, 0, 0, 1e4f, 0, &bf16, 3,
                      NULL) == CSA_ERR_SHAPE, "compress: ragged T");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 0, 3, 1e4f, 0, &bf16, 2,
                      NULL) == CSA_ERR_SHAPE, "compress: odd rope dims");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 512, 4, 1, 0, 256, 1e4f, 0, &bf16, 2,
                      NULL) == CSA_ERR_UNSUPPORTED, "compress: 256 rope dims");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 4, 0, 1e4f, 0, &bf16, 3,
                      NULL) == CSA_ERR_NULL, "compress: t0 > 0 without the previous block");
  expect(csa_compress(p, p, p, p, CSA_FP8MIX, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 0, 0, 1e4f, 0, &bf16, 2,
                      NULL) == CSA_ERR_DTYPE, "compress: input dtype");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 0, 0, 1e4f, 0, &mx_noscale, 2,
                      NULL) == CSA_ERR_NULL, "compress: MXFP4 without a scale plane");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 0, 0, 1e4f, 0, &bad_dtype, 2,
                      NULL) == CSA_ERR_DTYPE, "compress: unknown output dtype");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 0, 1, 0, 0, 1e4f, 0, &bf16, 2,
                      NULL) == CSA_ERR_SHAPE, "compress: ratio 0");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, -1, 8, 16, 4, 1, 0, 0, 1e4f, 0, &bf16, 2,
                      NULL) == CSA_ERR_SHAPE, "compress: negative B");
  expect(csa_compress(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 0, 0, 1e4f, 0, &bf16, 1,
                      NULL) == CSA_ERR_SHAPE, "compress: too few output rows");

  /* quantize */
  expect(csa_quantize(NULL, 4, 128, 0, &bf16, NULL) == CSA_ERR_NULL, "quantize: NULL input");
  expect(csa_quantize((const float*)p, 4, 128, 0, &f32, NULL) == CSA_ERR_DTYPE, "quantize: F32 target");
  expect(csa_quantize((const float*)p, 4, 100, 0, &bf16, NULL) == CSA_ERR_SHAPE, "quantize: D % 8");

  /* index scores */
  expect(csa_index_scores(&bf16, (const float*)p, &f32, (const int64_t*)p, 1, 1, 4, 32, 8, 8, 4, (float*)p, NULL) ==
         CSA_ERR_DTYPE, "index: dtype mismatch");
  expect(csa_index_scores(&bf16, (const float*)p, &bf16, (const int64_t*)p, 1, 1, 4, 30, 8, 8, 4, (float*)p, NULL) ==
         CSA_ERR_SHAPE, "index: DI % 8");
  expect(csa_index_scores(&bf16, (const float*)p, &bf16, (const int64_t*)p, 1, 1, 200, 32, 8, 8, 4, (float*)p,
                          NULL) == CSA_ERR_SHAPE, "index: HI > 128");
  expect(csa_index_scores(&bf16, NULL, &bf16, (const int64_t*)p, 1, 1, 4, 32, 8, 8, 4, (float*)p, NULL) ==
         CSA_ERR_NULL, "index: NULL weights");

  /* top-k */
  expect(csa_topk(NULL, 1, 10, 4, (int32_t*)p, NULL, NULL, 0, NULL) == CSA_ERR_NULL, "topk: NULL scores");
  expect(csa_topk((const float*)p, 1, 10, 0, (int32_t*)p, NULL, NULL, 0, NULL) == CSA_ERR_SHAPE, "topk: k = 0");
  expect(csa_topk((const float*)p, 1, 10, 5000, (int32_t*)p, NULL, NULL, 0, NULL) == CSA_ERR_SHAPE, "topk: k > 4096");
  expect(csa_topk((const float*)p, 2048, 262144, 1024, (int32_t*)p, NULL, NULL, 16, NULL) == CSA_ERR_WORKSPACE,
         "topk: small workspace");
  (void)csa_topk_workspace_size(0, 0, 1);
  (void)csa_topk_workspace_size(1 << 20, 1 << 20, 4096);

  /* fused indexer + top-k */
  expect(csa_index_topk(&bf16, (const float*)p, &f32, (const int64_t*)p, 1, 1, 16, 128, 64, 64, 4, 8, 0, (int32_t*)p,
                        NULL, NULL, NULL, 0, NULL) == CSA_ERR_DTYPE, "index_topk: dtype mismatch");
  expect(csa_index_topk(&bf16, (const float*)p, &bf16, (const int64_t*)p, 1, 1, 16, 128, 64, 64, 4, 0, 0, (int32_t*)p,
                        NULL, NULL, NULL, 0, NULL) == CSA_ERR_SHAPE, "index_topk: k = 0");
  expect(csa_index_topk(&bf16, (const float*)p, &bf16, (const int64_t*)p, 1, 1, 16, 128, 64, 64, 4, 8, 6, (int32_t*)p,
                        NULL, NULL, NULL, 0, NULL) == CSA_ERR_SHAPE, "index_topk: unknown flag");
  expect(csa_index_topk(&bf16, (const float*)p, &bf16, (const int64_t*)p, 16, 1, 64, 128, 32768, 32768, 4, 1024, 0,
                        (int32_t*)p, NULL, NULL, NULL, 0, NULL) == CSA_ERR_WORKSPACE, "index_topk: no workspace");
  (void)csa_index_topk_workspace_size(16, 1, 64, 128, 32768, 1024, CSA_BF16, 0);
  (void)csa_index_topk_workspace_size(1, 2048, 64, 128, 262144, 1024, CSA_BF16, CSA_FLAG_BF16_SCORES);
  (void)csa_index_topk_workspace_size(8, 1, 64, 128, 262144, 1024, CSA_MXFP4, 0);

  /* attention size queries over many shapes, including head counts with no MFMA head group */
  {
    const int Hs[] = {1, 8, 16, 17, 32, 48, 64, 72, 80, 112, 128, 144, 176, 200, 240, 256};
    const int Ds[] = {8, 64, 128, 256, 512, 1024};
    for (unsigned i = 0; i < sizeof Hs / sizeof Hs[0]; ++i)
      for (unsigned j = 0; j < sizeof Ds / sizeof Ds[0]; ++j) {
        (void)csa_sparse_mqa_workspace_size(16, 1, Hs[i], Ds[j], 1024, 128);
        (void)csa_sparse_mqa_workspace_size(1, 2048, Hs[i], Ds[j], 1024, 128);
        (void)hca_dense_attn_workspace_size(32, 1, Hs[i], Ds[j], 8192, 128);
        (void)hca_dense_attn_workspace_size(0, 0, Hs[i], Ds[j], 0, 1);
      }
  }
  expect(csa_sparse_mqa(&bf16, (const int64_t*)p, &bf16, 10, (const int32_t*)p, 4, &bf16, (const int64_t*)p, 16,
                        (const float*)p, 1.f, 64, 1e4f, 0, 1, 1, 16, 128, 10, 0, &bf16, NULL, 0, NULL) ==
         CSA_ERR_SHAPE, "mqa: n_win 0");
  expect(csa_sparse_mqa(&bf16, (const int64_t*)p, &fp8_noscale, 10, (const int32_t*)p, 4, &bf16, (const int64_t*)p,
                        16, (const float*)p, 1.f, 64, 1e4f, 0, 1, 1, 16, 128, 10, 8, &bf16, NULL, 0, NULL) ==
         CSA_ERR_NULL, "mqa: FP8MIX without a scale");
  expect(csa_sparse_mqa_noalloc(&bf16, (const int64_t*)p, &bf16, 10, (const int32_t*)p, 4, &bf16, (const int64_t*)p,
                                16, (const float*)p, 1.f, 64, 1e4f, 0, 1, 1, 16, 128, 10, 0, &bf16, NULL) ==
         CSA_ERR_SHAPE, "mqa noalloc: n_win 0");
  expect(csa_sparse_mqa_noalloc(&bf16, (const int64_t*)p, &bf16, 64, (const int32_t*)p, 1024, &bf16, (const int64_t*)p,
                                128, (const float*)p, 1.f, 64, 1e4f, 0, 64, 4, 128, 512, 64, 128, &bf16, NULL) ==
         CSA_ERR_UNSUPPORTED, "mqa noalloc: above the scratch limit");
  expect(csa_sparse_mqa_noalloc_limit() == ((size_t)32 << 20), "mqa noalloc: limit");
  expect(hca_dense_attn(&bf16, (const int64_t*)p, &bf16, 10, 0, &bf16, (const int64_t*)p, 16, (const float*)p, 1.f,
                        64, 1e4f, 0, 1, 1, 16, 128, 10, 8, &bf16, NULL, 0, NULL) == CSA_ERR_SHAPE, "hca: ratio 0");

  /* RMSNorm, compress with a norm, grouped output projection */
  {
    const float* w = (const float*)p;
    expect(csa_rmsnorm(&bf16, 4, 512, NULL, 1e-6f, &bf16, NULL) == CSA_ERR_NULL, "rmsnorm: no weight");
    expect(csa_rmsnorm(&bf16, 4, 500, w, 1e-6f, &bf16, NULL) == CSA_ERR_SHAPE, "rmsnorm: D % 8");
    expect(csa_rmsnorm(&bf16, 4, 512, w, 1e-6f, &f32, NULL) == CSA_ERR_DTYPE, "rmsnorm: mixed dtypes");
    expect(csa_rmsnorm(&bf16, -1, 512, w, 1e-6f, &bf16, NULL) == CSA_ERR_SHAPE, "rmsnorm: negative rows");
    expect(csa_compress_norm(p, p, p, p, CSA_BF16, NULL, NULL, NULL, NULL, 1, 8, 16, 4, 1, 0, 0, 1e4f, 0,
                             (const float*)(p + 4), 1e-6f, &bf16, 2, NULL) == CSA_ERR_SHAPE,
           "compress_norm: misaligned weight");
    expect(csa_grouped_out_proj(&bf16, p, p, 16, 128, 512, 12, 1024, 7168, &bf16, p, (size_t)1 << 30, NULL) ==
           CSA_ERR_SHAPE, "proj: g does not divide n_h");
    expect(csa_grouped_out_proj(&f32, p, p, 16, 128, 512, 16, 1024, 7168, &bf16, p, (size_t)1 << 30, NULL) ==
           CSA_ERR_DTYPE, "proj: f32 input");
    expect(csa_grouped_out_proj(&bf16, p, p, 16, 128, 512, 16, 1024, 7168, &bf16, NULL, 0, NULL) == CSA_ERR_WORKSPACE,
           "proj: no workspace");
    expect(csa_grouped_out_proj_workspace_size(0, 128, 512, 16, 1024, 7168) == 0, "proj: size at T = 0");
    const int64_t Ts[] = {1, 16, 32, 33, 2048, (int64_t)1 << 22};
    for (unsigned i = 0; i < sizeof Ts / sizeof Ts[0]; ++i)
      expect(csa_grouped_out_proj_workspace_size(Ts[i], 128, 512, 16, 1024, 7168) >= (size_t)Ts[i] * 16 * 1024 * 2,
             "proj: size holds mid");
  }

  /* forward descriptors */
  {
    csa_layer_desc d;
    csa_forward_io io;
    memset(&d, 0, sizeof d);
    memset(&io, 0, sizeof io);
    expect(csa_forward(&d, &io, NULL, 0, NULL) == CSA_ERR_SHAPE, "forward: struct_size");
    expect(csa_forward_workspace_size(&d) == 0, "forward: size of a bad descriptor");
    expect(csa_forward(NULL, &io, NULL, 0, NULL) == CSA_ERR_NULL, "forward: NULL descriptor");
    d.struct_size = (int32_t)sizeof d;
    const int Hs[] = {16, 80, 128, 144};
    for (int mode = 0; mode < 2; ++mode)
      for (unsigned i = 0; i < sizeof Hs / sizeof Hs[0]; ++i) {
        d.mode = mode;
        d.B = 16;
        d.T = 4;
        d.t0 = 131068;
        d.Tq = 1;
        d.cache_rows = 32768;
        d.Tw = 128;
        d.D = 512;
        d.H = Hs[i];
        d.HI = 64;
        d.DI = 128;
        d.ratio = mode == 0 ? 4 : 128;
        d.t0 = mode == 0 ? 131068 : 131072 - 128;
        d.T = d.ratio;
        d.topk = 1024;
        d.n_win = 128;
        d.rope_dims = 64;
        d.rope_base = 1e4f;
        d.softmax_scale = 1.f;
        d.stream_dtype = CSA_BF16;
        d.flags = 0;
        (void)csa_forward_workspace_size(&d);
        expect(csa_forward(&d, &io, NULL, 0, NULL) != CSA_OK, "forward: empty io is rejected");
        d.flags = CSA_FLAG_QKV_NORM;
        d.norm_eps = 1e-6f;
        expect(csa_forward_workspace_size(&d) > 0, "forward: size with norms");
        expect(csa_forward(&d, &io, NULL, 0, NULL) != CSA_OK, "forward: norms without weights are rejected");
        d.flags = 0;
      }
  }
  /* decode step descriptors */
  {
    csa_decode_desc d;
    csa_decode_io io;
    memset(&d, 0, sizeof d);
    memset(&io, 0, sizeof io);
    expect(csa_decode_step(&d, &io, NULL, 0, NULL) == CSA_ERR_SHAPE, "decode: struct_size");
    expect(csa_decode_step(NULL, &io, NULL, 0, NULL) == CSA_ERR_NULL, "decode: NULL descriptor");
    d.struct_size = (int32_t)sizeof d;
    d.B = 16;
    d.slots = 16;
    d.pages = 1100;
    d.max_pages = 64;
    d.page_tokens = 2048;
    d.D = 512;
    d.H = 128;
    d.HI = 64;
    d.DI = 128;
    d.ratio = 4;
    d.topk = 1024;
    d.n_win = 128;
    d.rope_dims = 64;
    d.rope_base = 1e4f;
    d.softmax_scale = 1.f;
    d.stream_dtype = CSA_BF16;
    expect(csa_decode_step_workspace_size(&d) > 0, "decode: size");
    expect(csa_decode_step(&d, &io, NULL, 0, NULL) == CSA_ERR_NULL, "decode: empty io");
    const int32_t pts[] = {1024, 3072, 2, 1 << 30};
    for (unsigned i = 0; i < sizeof pts / sizeof pts[0]; ++i) {
      d.page_tokens = pts[i];
      expect(csa_decode_step_workspace_size(&d) == 0, "decode: bad page size");
    }
    d.page_tokens = 2048;
    d.mode = CSA_MODE_HCA;
    d.ratio = 128;
    d.page_tokens = 4096;
    d.max_pages = 256;
    expect(csa_decode_step_workspace_size(&d) > 0, "decode: HCA size");
    d.flags = CSA_FLAG_QKV_NORM;
    d.norm_eps = 1e-6f;
    expect(csa_decode_step_workspace_size(&d) > 0, "decode: HCA size with norms");
  }
  if (failures == 0) printf("abi host check: ok\n");
  return failures == 0 ? 0 : 1;
}
