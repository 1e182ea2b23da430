/*
 * csa.h -- C ABI of the MI355X (gfx950) CSA / HCA attention library (libcsa.so).
 *
 * The library computes one forward pass of the DeepSeek-V4 hybrid attention layer
 * as the report defines it (cited by page title and section):
 *
 *   [V4-CN]  "DeepSeek-V4中文翻译（翻译模型：Opus4.7）" (blog.uika.cn), report §2.3.1-§2.3.4,
 *            §3.4, §3.6.1;
 *   [NOTES]  "DeepSeek-V4：把百万 token 上下文从额度变成架构问题"
 *            (awesome.papernotes.org), "关键设计 1" and "关键设计 2".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a DEVICE pointer owned by the caller: dense,
 *   row-major, last dimension contiguous, in the shape written beside it.  The
 *   library never allocates device memory; scratch comes from a caller workspace
 *   whose size the matching *_workspace_size() query returns.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call only ENQUEUES work on it and returns; results are valid after the stream
 *   is synchronised.  Calls are re-entrant; two calls that share output or
 *   workspace buffers must be ordered by the caller (same stream).
 * - Errors: all arguments are validated on the host before anything is launched.
 *   On error the call returns a non-zero csa_status, launches nothing and leaves
 *   outputs untouched; csa_last_error() then returns a message (thread-local,
 *   valid until the next call on that thread).  No C++ exception crosses the ABI.
 *   CSA_ERR_DEVICE means no gfx950 device is current or a launch failed.
 * - Device-resident data (indices, positions) is NOT validated: entry indices must
 *   lie in [0, N) or be -1, positions must be >= 0, and the raw window buffer must
 *   cover every window position a query needs.  Violations are undefined.
 * - Positions are absolute token indices from the start of the sequence.  A
 *   compressed entry i covers tokens [ratio*i, ratio*(i+1)) and carries RoPE
 *   position ratio*i.  `pos_offset` is added to every RoPE position and to nothing
 *   else (block visibility and windows use the plain positions).
 * - RoPE ([V4-CN] §2.3.3) rotates the last `rope_dims` dims in adjacent pairs
 *   (D-R+2j, D-R+2j+1) by angle pos * rope_base^(-2j/R); rope_dims is even,
 *   D - rope_dims is even and rope_dims <= 128 (else CSA_ERR_UNSUPPORTED).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 4

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  CSA_ERR_SHAPE = 2,       /* sizes inconsistent or out of the supported range  */
  CSA_ERR_DTYPE = 3,       /* dtype (combination) not supported by this call    */
  CSA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required        */
  CSA_ERR_DEVICE = 5,      /* no gfx950 device current, or a launch failed      */
  CSA_ERR_UNSUPPORTED = 6  /* valid request the library does not implement      */
} csa_status;

/*
 * Storage formats of a csa_buf ([V4-CN] §2.3.4 and §3.4):
 *   CSA_F32    data = float [rows, D]
 *   CSA_BF16   data = bf16  [rows, D]  (raw 16-bit patterns)
 *   CSA_FP8MIX data  = uint8 e4m3 (OCP, max 448) [rows, D-R]  -- the non-RoPE dims
 *              rope  = bf16 [rows, R]                         -- the RoPE dims
 *              scale = float [rows]; value = e4m3(code) * scale for the first D-R dims
 *   CSA_MXFP4  data  = uint8 [rows, D/2], two e2m1 codes per byte, element 2j in
 *                      the low nibble; D % 32 == 0
 *              scale = uint8 e8m0 [rows, D/32]; value = e2m1 * 2^(code-127) per 32
 *                      contiguous elements
 */
typedef enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8MIX = 2, CSA_MXFP4 = 3 } csa_dtype;

/*
 * CSA_FLAG_BF16_SCORES: index scores are rounded to bf16 (nearest-even) before the
 * top-k selection, as the report stores them to speed the selector up ([V4-CN] §3.4:
 * FP32 -> BF16 index scores, 99.7% recall of the selected KV entries).  Equal bf16
 * scores are then taken in increasing entry order.  Off by default: the selection is
 * then exact on the fp32 scores.
 */
#define CSA_FLAG_BF16_SCORES 1
/*
 * CSA_FLAG_QKV_NORM (csa_forward only): RMSNorm the query heads and the KV before
 * core attention ([V4-CN] §2.3.3): every compressed KV entry is normalized with
 * io->kv_norm before its RoPE, every raw window row with io->kv_norm, every query
 * head with io->q_norm, all with desc->norm_eps.  The indexer path is unchanged.
 */
#define CSA_FLAG_QKV_NORM 2

typedef struct csa_buf {
  void* data;
  void* rope;   /* FP8MIX only */
  void* scale;  /* FP8MIX, MXFP4 */
  int32_t dtype;
  int32_t reserved;
} csa_buf;

int csa_abi_version(void);
const char* csa_last_error(void);
/* CSA_OK iff the current HIP device is a gfx950 GPU. */
csa_status csa_device_check(void);

/*
 * csa_compress -- softmax-weighted KV compression ([V4-CN] §2.3.1 compression
 * equations for CSA, §2.3.2 for HCA; [NOTES] "关键设计 1": weights are per channel).
 *
 * For every entry i with t0/ratio <= i < (t0+T)/ratio of every sequence b and every
 * channel d, the logits of the positions are
 *     overlap=1 (CSA):  Z^a[ratio*i + j, d] + bias_a[j, d]              j < ratio
 *                       Z^b[ratio*(i-1) + j, d] + bias_b[j, d]          j < ratio, i >= 1
 *     overlap=0 (HCA):  Z^a[ratio*i + j, d] + bias_a[j, d]              j < ratio
 * they are soft-maxed across the positions (per channel), and the entry is the
 * weighted sum of the matching C^a / C^b rows.  Entry 0 has no previous block.
 * The last rope_dims dims are then rotated to position pos_offset + ratio*i.
 *
 *   ca, za           [B, T, D]  rows of tokens t0 .. t0+T-1 (C^a, Z^a; for HCA: C, Z)
 *   cb, zb           [B, T, D]  b-branch rows (overlap=1 only; NULL for overlap=0)
 *   in_dtype         CSA_F32 or CSA_BF16 (all four streams and prev_* share it)
 *   bias_a, bias_b   float [ratio, D] or NULL (= 0)
 *   prev_cb, prev_zb [B, ratio, D] the b-branch rows of tokens t0-ratio .. t0-1;
 *                    required iff overlap=1 and t0 > 0, else ignored
 *   T                multiple of ratio (T = 0 is a no-op); t0 multiple of ratio
 *   out              [B, out_rows, D] in F32, BF16, FP8MIX (R = rope_dims) or
 *                    MXFP4 (D % 32 == 0); entry i is written to row i of its sequence,
 *                    so (t0+T)/ratio <= out_rows.  Other rows are untouched.
 * Limits: 1 <= ratio <= 1024, 2 <= D <= 2048, D % 8 == 0.
 */
csa_status csa_compress(const void* ca, const void* cb, const void* za, const void* zb,
                        int32_t in_dtype, const float* bias_a, const float* bias_b,
                        const void* prev_cb, const void* prev_zb, int64_t B, int64_t T,
                        int32_t D, int32_t ratio, int32_t overlap, int64_t t0,
                        int32_t rope_dims, float rope_base, int64_t pos_offset,
                        const csa_buf* out, int64_t out_rows, void* stream);

/*
 * csa_compress_norm -- csa_compress with an RMSNorm of every entry before its RoPE
 * ([V4-CN] §2.3.3: KV entries are normalized ahead of core attention):
 *     e <- e / sqrt(mean_d(e_d^2) + norm_eps) * norm_weight      (fp32)
 * norm_weight: float [D] (16-byte aligned) or NULL (then identical to csa_compress);
 * norm_eps finite, >= 0.  Other arguments and limits as csa_compress.
 */
csa_status csa_compress_norm(const void* ca, const void* cb, const void* za, const void* zb,
                             int32_t in_dtype, const float* bias_a, const float* bias_b,
                             const void* prev_cb, const void* prev_zb, int64_t B, int64_t T,
                             int32_t D, int32_t ratio, int32_t overlap, int64_t t0,
                             int32_t rope_dims, float rope_base, int64_t pos_offset,
                             const float* norm_weight, float norm_eps, const csa_buf* out,
                             int64_t out_rows, void* stream);

/*
 * csa_rmsnorm -- row-wise RMSNorm ([V4-CN] §2.3.3: query heads and KV entries are
 * normalized before core attention):
 *     out[r, d] = x[r, d] / sqrt(mean_j(x[r, j]^2) + eps) * weight[d]
 * computed in fp32 and stored in out's dtype.
 *   x, out   [rows, D], both F32 or both BF16, 16-byte aligned; may alias exactly
 *   weight   float [D]
 * Limits: 8 <= D <= 2048, D % 8 == 0; eps finite, >= 0.  rows = 0 is a no-op.
 */
csa_status csa_rmsnorm(const csa_buf* x, int64_t rows, int32_t D, const float* weight,
                       float eps, const csa_buf* out, void* stream);

/*
 * csa_grouped_out_proj -- grouped output projection ([V4-CN] §2.3.1 output
 * projection; g groups of intermediate width d_g, §4.2.1):
 *     mid[t, j*d_g + e] = sum_i o[t, j*(n_h/g)*c + i] * w_group[j, e, i]   j < g
 *     out[t, f]         = sum_e mid[t, e] * w_out[f, e]
 * bf16 operands, fp32 accumulation; mid is stored in bf16 (workspace) between the
 * two products.  With few rows the contraction is split across workgroups and the
 * fp32 partials are summed in a fixed order, so results are deterministic.
 *   o        bf16 [T, n_h, c] (the core-attention output of every head; 16-byte aligned)
 *   w_group  bf16 [g, d_g, (n_h/g)*c]   (each group's projection, [out, in])
 *   w_out    bf16 [d, g*d_g]            ([out, in])
 *   out      [T, d], BF16 or F32
 *   ws       csa_grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d) bytes, 16-byte
 *            aligned
 * Limits: g divides n_h; (n_h/g)*c and g*d_g multiples of 32; T <= 2^22.  T = 0 is a
 * no-op.
 */
size_t csa_grouped_out_proj_workspace_size(int64_t T, int32_t n_h, int32_t c, int32_t g,
                                           int32_t d_g, int32_t d);
csa_status csa_grouped_out_proj(const csa_buf* o, const void* w_group, const void* w_out,
                                int64_t T, int32_t n_h, int32_t c, int32_t g, int32_t d_g,
                                int32_t d, const csa_buf* out, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * csa_quantize -- store fp32 rows [rows, D] in another storage format
 * (CSA_BF16, CSA_FP8MIX with R = rope_dims, CSA_MXFP4).  Rounding: nearest-even;
 * fp8 saturates at +-448; FP8MIX scale = amax(|non-RoPE dims|)/448 in fp32 (1 for an
 * all-zero entry), codes = e4m3(x / scale); MXFP4 block exponent
 * X = floor(log2(amax)) - 2 (OCP MX), codes = e2m1(x / 2^X), saturating at 6.
 * ([V4-CN] §2.3.4 mixed FP8/BF16 KV storage; §3.4 FP4 indexer QK path.)
 */
csa_status csa_quantize(const float* x, int64_t rows, int32_t D, int32_t rope_dims,
                        const csa_buf* out, void* stream);

/*
 * csa_index_scores -- lightning indexer ([V4-CN] §2.3.1 index-score equation):
 *     scores[b,t,s] = sum_h wI[b,t,h] * max(0, qI[b,t,h,:] . kI[b,s,:])
 * for s < floor(q_pos[b,t] / ratio) (a query sees only earlier compressed blocks,
 * [V4-CN] §2.3.3), and -inf for the other s < N.
 *
 *   qI      [B, Tq, HI, DI]  F32, BF16 or MXFP4 (same dtype as kI)
 *   wI      float [B, Tq, HI]
 *   kI      [B, kI_rows, DI] compressed indexer keys; the first N rows are used
 *   q_pos   int64 [B, Tq]
 *   scores  float [B, Tq, N]
 * Limits: HI <= 128, DI <= 512, DI % 8 == 0 (MXFP4: DI % 32 == 0).
 */
csa_status csa_index_scores(const csa_buf* qI, const float* wI, const csa_buf* kI,
                            const int64_t* q_pos, int64_t B, int64_t Tq, int32_t HI,
                            int32_t DI, int64_t N, int64_t kI_rows, int32_t ratio,
                            float* scores, void* stream);

/*
 * csa_topk -- top-k selector ([V4-CN] §2.3.1; [NOTES] C_t = TopK_k(I_t,:)).
 * For each row of scores [rows, N] selects the min(k, #finite) largest finite
 * scores; equal scores are taken in increasing index order; -inf / NaN are never
 * selected.  idx [rows, k] receives the selected indices in ascending order,
 * padded with -1; count [rows] (optional, may be NULL) the number selected.
 * Limits: 1 <= k <= 4096, N < 2^31.
 * ws (device, caller-owned, at least csa_topk_workspace_size bytes, 0 for rows of
 * at most 32768 scores when rows <= 64) holds the candidate lists between selection
 * levels and, for many long rows, a sampled per-row estimate of the k-th score; the
 * result is exact whatever the estimate (rows it misjudges are recomputed).
 */
size_t csa_topk_workspace_size(int64_t rows, int64_t N, int32_t k);
csa_status csa_topk(const float* scores, int64_t rows, int64_t N, int32_t k, int32_t* idx,
                    int32_t* count, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_topk -- lightning indexer and top-k selector in one call ([V4-CN] §2.3.1:
 * index scores, then C_t = TopK_k(I_t,:); §3.4 for the BF16-score option).
 * idx [B*Tq, k] and count [B*Tq] (optional) are exactly those of csa_index_scores
 * followed by csa_topk on the same scores (with CSA_FLAG_BF16_SCORES in flags: on the
 * scores rounded to bf16).  Few queries per sequence with bf16 operands and rows much
 * longer than the candidates they keep (the decode shape: Tq < 16, HI % 16 == 0, DI in
 * {32, 64, 128}, 8 * ceil(N / 2048) * k <= N) take a fused path: every workgroup keeps
 * its 2048-entry slice's top-k while it scores, so the score row is not written, and
 * one merge selects each row's top-k from those candidates.  Other shapes run the two
 * stages.
 *   scores  optional float [B, Tq, N]: when not NULL it also receives the scores
 *   ws      device workspace of at least csa_index_topk_workspace_size(...) bytes
 *           (candidate lists, or the score rows and top-k levels)
 * Arguments and limits as csa_index_scores and csa_topk; flags: CSA_FLAG_* bits.
 */
size_t csa_index_topk_workspace_size(int64_t B, int64_t Tq, int32_t HI, int32_t DI, int64_t N, int32_t k,
                                     int32_t qI_dtype, int32_t flags);
csa_status csa_index_topk(const csa_buf* qI, const float* wI, const csa_buf* kI, const int64_t* q_pos,
                          int64_t B, int64_t Tq, int32_t HI, int32_t DI, int64_t N, int64_t kI_rows,
                          int32_t ratio, int32_t k, int32_t flags, int32_t* idx, int32_t* count,
                          float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_sparse_mqa -- shared-KV multi-query attention over the selected compressed
 * entries plus the raw sliding window ([V4-CN] §2.3.1 shared-KV MQA: each entry is
 * both key and value for all heads; §2.3.3 window branch, attention sink, partial
 * and inverse RoPE; [NOTES] csa() sketch: one attention over concat(selected, window)).
 *
 * For query t of sequence b (position p = q_pos[b,t]) the keys are
 *     kv[b, idx[b,t,j]]                     for the K slots with idx >= 0
 *     RoPE(win[b, r - win_pos0[b]], r)      for r = max(0, p-n_win+1) .. p
 * and for every head h
 *     z_j   = softmax_scale * RoPE(q[b,t,h], p) . key_j
 *     o     = sum_j exp(z_j) key_j / (sum_j exp(z_j) + exp(sink[h]))
 *     out   = RoPE(o, -p)
 * (sink = -inf removes the sink term; +inf gives 0).
 *
 *   q       [B, Tq, H, D]  F32 or BF16, not roped;  out: same shape and dtype
 *   kv      [B, kv_rows, D] compressed entries (already roped), F32/BF16/FP8MIX
 *   idx     int32 [B, Tq, K]
 *   win     [B, Tw, D] raw (un-roped) entries of positions win_pos0[b] ..; same
 *           dtype as kv
 *   sink    float [H]
 * Limits: D <= 1024; H <= 256; K + n_win <= 2^20.  The MFMA path needs a BF16 or
 * FP8MIX cache, BF16 q, H % 16 == 0 and D % 32 == 0; other combinations run a
 * slower SIMT kernel.
 *
 * FP8MIX queries ([V4-CN] §2.3.4: the attention arithmetic in FP8): q may be an FP8MIX
 * buffer laid out like a cache row per (token, head) -- e4m3 codes [B, Tq, H, D - R],
 * bf16 RoPE dims [B, Tq, H, R] (not roped), f32 scale [B, Tq, H] -- as csa_quantize
 * writes it.  The QK products of the D - R coded dims then run on fp8 MFMA over the
 * codes of query and key (exact products, fp32 sums, times both scales); the RoPE
 * dims and the probability-weighted sum of values stay bf16.  The result is the
 * attention of the dequantized query.  Needs an FP8MIX cache, D = 512, R = 64,
 * H in {64, 128, 256} and a BF16 out; anything else returns CSA_ERR_UNSUPPORTED (or
 * CSA_ERR_DTYPE for another out dtype) and launches nothing.  csa_forward and
 * csa_decode_step take FP8MIX queries the same way (without CSA_FLAG_QKV_NORM).
 */
size_t csa_sparse_mqa_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t D, int32_t K,
                                     int32_t n_win);
csa_status csa_sparse_mqa(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv,
                          int64_t kv_rows, const int32_t* idx, int32_t K, const csa_buf* win,
                          const int64_t* win_pos0, int64_t Tw, const float* sink,
                          float softmax_scale, int32_t rope_dims, float rope_base,
                          int64_t pos_offset, int64_t B, int64_t Tq, int32_t H, int32_t D,
                          int64_t N, int32_t n_win, const csa_buf* out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * csa_sparse_mqa_noalloc -- csa_sparse_mqa without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * csa_sparse_mqa minus ws / ws_bytes.  The split partials live in a static device
 * array of csa_sparse_mqa_noalloc_limit() bytes (32 MiB) that each GPU holds for the
 * life of the process; a call needing more (csa_sparse_mqa_workspace_size larger than
 * the limit) returns CSA_ERR_UNSUPPORTED and launches nothing.  No call allocates or
 * frees memory.  Calls that overlap on one GPU share the array and race: order them
 * (same stream) or use csa_sparse_mqa.
 */
csa_status csa_sparse_mqa_noalloc(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv,
                                  int64_t kv_rows, const int32_t* idx, int32_t K, const csa_buf* win,
                                  const int64_t* win_pos0, int64_t Tw, const float* sink,
                                  float softmax_scale, int32_t rope_dims, float rope_base,
                                  int64_t pos_offset, int64_t B, int64_t Tq, int32_t H, int32_t D,
                                  int64_t N, int32_t n_win, const csa_buf* out, void* stream);
size_t csa_sparse_mqa_noalloc_limit(void);

/*
 * hca_dense_attn -- HCA core attention ([V4-CN] §2.3.2; [NOTES] hca() sketch):
 * as csa_sparse_mqa, with the compressed keys being every entry i < min(N,
 * floor(p / ratio)) instead of an index list.
 */
size_t hca_dense_attn_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t D, int64_t N,
                                     int32_t n_win);
csa_status hca_dense_attn(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv,
                          int64_t kv_rows, int32_t ratio, const csa_buf* win,
                          const int64_t* win_pos0, int64_t Tw, const float* sink,
                          float softmax_scale, int32_t rope_dims, float rope_base,
                          int64_t pos_offset, int64_t B, int64_t Tq, int32_t H, int32_t D,
                          int64_t N, int32_t n_win, const csa_buf* out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * csa_forward -- one layer forward (prefill chunk or decode step):
 *   mode CSA: compress the T new tokens of the KV streams and of the indexer-key
 *             streams into the caches (entries t0/m .. (t0+T)/m - 1), score every
 *             query against the N = (t0+T)/m entries, select top-k, attend;
 *   mode HCA: compress with ratio m', attend densely.
 * ([NOTES] csa()/hca() sketches; [V4-CN] §2.3.1-§2.3.3.)
 */
typedef enum csa_mode { CSA_MODE_CSA = 0, CSA_MODE_HCA = 1 } csa_mode;

typedef struct csa_layer_desc {
  int32_t struct_size;   /* sizeof(csa_layer_desc) */
  int32_t mode;          /* csa_mode */
  int64_t B;             /* sequences */
  int64_t T;             /* new tokens to compress (multiple of ratio, may be 0) */
  int64_t t0;            /* absolute index of the first new token (multiple of ratio) */
  int64_t Tq;            /* query tokens per sequence */
  int64_t cache_rows;    /* rows of kv_cache / ik_cache per sequence */
  int64_t Tw;            /* rows of the raw window buffer per sequence */
  int32_t D;             /* KV / head dim */
  int32_t H;             /* query heads */
  int32_t HI, DI;        /* indexer heads and dim (CSA) */
  int32_t ratio;         /* m (CSA) or m' (HCA) */
  int32_t topk;          /* k (CSA) */
  int32_t n_win;         /* sliding window */
  int32_t rope_dims;
  float rope_base;
  float softmax_scale;
  int64_t pos_offset;
  int32_t stream_dtype;  /* C/Z streams: F32 or BF16 */
  int32_t flags;         /* CSA_FLAG_* (0 = the exact default) */
  float norm_eps;        /* RMSNorm epsilon (CSA_FLAG_QKV_NORM) */
  int32_t reserved;      /* 0 */
} csa_layer_desc;

typedef struct csa_forward_io {
  /* KV streams of the new tokens [B, T, D] (HCA: ca = C, za = Z; cb, zb unused) */
  const void *ca, *cb, *za, *zb;
  const float *bias_a, *bias_b;          /* [ratio, D] or NULL */
  const void *prev_cb, *prev_zb;         /* [B, ratio, D], CSA with t0 > 0 */
  /* indexer-key streams of the new tokens [B, T, DI] (CSA) */
  const void *ica, *icb, *iza, *izb;
  const float *ibias_a, *ibias_b;
  const void *iprev_cb, *iprev_zb;
  csa_buf kv_cache;                      /* [B, cache_rows, D]  in/out */
  csa_buf ik_cache;                      /* [B, cache_rows, DI] in/out (CSA) */
  csa_buf q;                             /* [B, Tq, H, D]: F32, BF16 or FP8MIX (see csa_sparse_mqa) */
  const int64_t* q_pos;                  /* [B, Tq] */
  csa_buf qI;                            /* [B, Tq, HI, DI] (CSA) */
  const float* wI;                       /* [B, Tq, HI] (CSA) */
  csa_buf win;                           /* [B, Tw, D] raw */
  const int64_t* win_pos0;               /* [B] */
  const float* sink;                     /* [H] */
  csa_buf out;                           /* [B, Tq, H, D] */
  float* scores_out;                     /* optional [B, Tq, N] copy of the index scores */
  int32_t* idx_out;                      /* optional [B, Tq, topk] selected entries */
  const float* q_norm;                   /* [D] query-head RMSNorm weight (CSA_FLAG_QKV_NORM) */
  const float* kv_norm;                  /* [D] KV RMSNorm weight (CSA_FLAG_QKV_NORM) */
} csa_forward_io;

size_t csa_forward_workspace_size(const csa_layer_desc* L);
csa_status csa_forward(const csa_layer_desc* L, const csa_forward_io* io, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * csa_decode_step -- one decode token per sequence, with a state cache and paged
 * compressed caches ([V4-CN] §3.6.1: the sliding window and the compression branch's
 * uncompressed tail are a fixed-size per-sequence state taken from a preallocated pool;
 * the compressed caches are blocks of page_tokens raw tokens, which may be any multiple
 * of lcm(m, m'), so one block table serves CSA and HCA layers).
 *
 * For batch row b, slot s = slot[b], position p = length[s]:
 *   1. the token's stream rows enter the slot's tail ring and its raw KV row the window;
 *      when p + 1 is a multiple of ratio, the block's entry (CSA: and its indexer key)
 *      is compressed exactly as csa_compress_norm would, into the paged cache at entry
 *      p / ratio;
 *   2. CSA: the query at position p is scored against the entries it may see
 *      (e < p / ratio) and the top-k kept (as csa_index_topk); HCA: every entry it may
 *      see is used;
 *   3. core attention over those entries and the raw window positions
 *      max(0, p - n_win + 1) .. p, with the sink (as csa_sparse_mqa / hca_dense_attn);
 *   4. length[s] = p + 1.
 * Every slot has its own length (ragged batches).  A sequence's result does not depend
 * on the other sequences of the batch: no step reduces across sequences, and the split
 * of a query's keys over workgroups depends only on the layer shape.
 *
 * State pool (caller-owned device memory):
 *   length     int64 [slots]
 *   tail       CSA: [slots, 2 ratio, 4, D], the C^a, C^b, Z^a, Z^b rows of position q at
 *              ring row q mod 2 ratio; HCA: [slots, ratio, 2, D], the C, Z rows at ring
 *              row q mod ratio; in stream_dtype.  Precondition: the rows of positions
 *              ratio * (floor(length / ratio) - 1) .. length - 1 (those >= 0) (HCA: of
 *              the current block) are in the ring.
 *   itail      CSA: [slots, 2 ratio, 4, DI], the indexer streams, same rule
 *   win        [slots, 2 n_win, D] raw KV rows, F32, BF16 or FP8MIX: row j holds position
 *              win_pos0[s] + j.  Precondition: positions max(0, length - n_win + 1) ..
 *              length - 1 are present, and length - win_pos0[s] <= 2 n_win.  A row that
 *              would fall past the buffer first moves the last n_win - 1 rows to the front
 *              (win_pos0 advances).
 *   win_pos0   int64 [slots]
 * Paged caches, P = page_tokens / ratio entries per page:
 *   kv_pages   [pages, P, D], the format of win (F32, BF16 or FP8MIX)
 *   ik_pages   [pages, P, DI] (CSA), the dtype of qI (F32, BF16 or MXFP4)
 *   block_table int32 [slots, max_pages]: page holding entries j P .. (j + 1) P - 1 of the
 *              slot.  Precondition: assigned for every block holding an entry
 *              < (length + 1) / ratio.
 * Step tensors: ca, cb, za, zb [B, D] (HCA: ca = C, za = Z) and ica, icb, iza, izb
 *   [B, DI] (CSA): the new token's streams, in stream_dtype; biases as csa_compress;
 *   kv_raw [B, D] in win's format; q [B, H, D] and out (q's dtype); qI [B, HI, DI] and wI
 *   [B, HI] (CSA); sink [H]; q_norm / kv_norm [D] with CSA_FLAG_QKV_NORM.
 *   idx_out (optional, CSA) int32 [B, topk]: the selected entries' pool rows (page * P +
 *   offset), in increasing entry order, -1 padded.  scores_out (optional, CSA) float
 *   [B, max_pages * P].
 * Limits: page_tokens a power of two and a multiple of ratio; CSA: P >= 512 (an indexer
 *   key range stays inside one page) and roundup(D / 8, 64) + DI / 8 <= 256 (one thread
 *   per 8 channels); D <= 1024; distinct slots within a batch; max_pages * P < 2^31;
 *   FP8MIX: (D - rope_dims) % 16 == 0, rope_dims % 8 == 0, no CSA_FLAG_QKV_NORM.
 */
typedef struct csa_decode_desc {
  int32_t struct_size;   /* sizeof(csa_decode_desc) */
  int32_t mode;          /* csa_mode */
  int64_t B;             /* sequences in this step */
  int64_t slots;         /* state-pool slots */
  int64_t pages;         /* pages of each cache pool */
  int32_t max_pages;     /* block-table row length */
  int32_t page_tokens;   /* raw tokens per page */
  int32_t D, H, HI, DI;
  int32_t ratio, topk, n_win, rope_dims;
  float rope_base, softmax_scale;
  int64_t pos_offset;
  int32_t stream_dtype;  /* F32 or BF16 */
  int32_t flags;         /* CSA_FLAG_BF16_SCORES, CSA_FLAG_QKV_NORM */
  float norm_eps;
  int32_t reserved;      /* 0 */
} csa_decode_desc;

typedef struct csa_decode_io {
  const int32_t* slot;                   /* [B] */
  int64_t* length;                       /* [slots] in/out */
  const void *ca, *cb, *za, *zb;         /* [B, D] */
  const float *bias_a, *bias_b;          /* [ratio, D] or NULL */
  const void *ica, *icb, *iza, *izb;     /* [B, DI] (CSA) */
  const float *ibias_a, *ibias_b;
  csa_buf kv_raw;                        /* [B, D], in win's format */
  void* tail;                            /* state pool, in/out */
  void* itail;
  csa_buf win;
  int64_t* win_pos0;
  csa_buf kv_pages;                      /* paged caches, in/out */
  csa_buf ik_pages;
  const int32_t* block_table;
  csa_buf q;                             /* [B, H, D]: F32, BF16 or FP8MIX (see csa_sparse_mqa) */
  csa_buf qI;                            /* [B, HI, DI] (CSA) */
  const float* wI;                       /* [B, HI] (CSA) */
  const float* sink;                     /* [H] */
  csa_buf out;                           /* [B, H, D] */
  const float *q_norm, *kv_norm;         /* [D] (CSA_FLAG_QKV_NORM) */
  int32_t* idx_out;                      /* optional [B, topk] (CSA) */
  float* scores_out;                     /* optional [B, max_pages * P] (CSA) */
} csa_decode_io;

size_t csa_decode_step_workspace_size(const csa_decode_desc* L);
csa_status csa_decode_step(const csa_decode_desc* L, const csa_decode_io* io, void* ws,
                           size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
