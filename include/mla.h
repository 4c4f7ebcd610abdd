/*
 * mla.h — C ABI of the MI355X (gfx950) Multi-head Latent Attention library (libmla.so).
 *
 * The operation is the MLA layer of DeepSeek-V2 as written out on the page
 * "DeepSeek-V2 paper summary" (7shi.hateblo.jp), App. C "Full Formulas of MLA",
 * with the definitions of section 2.1.2 (joint KV compression) and section 2.1.3
 * (decoupled RoPE: per-head rope query, one rope key shared by all heads):
 *
 *   c^q_t  = W_DQ h_t                      (c^q_t := h_t when d_cq == 0: App. B.1, V2-Lite)
 *   q^C_t  = W_UQ c^q_t,   q^R_t = RoPE_t(W_QR c^q_t)      (head i = rows i*d_h.., i*d_hr..)
 *   c^KV_t = W_DKV h_t,    k^R_t = RoPE_t(W_KR h_t)        (the cached vectors)
 *   k^C_{t,i} = W_UK_i c^KV_t,   v_{t,i} = W_UV_i c^KV_t
 *   o_{t,i} = sum_{j<=t} softmax_j(scale * ([q^C;q^R]_{t,i} . [k^C_{j,i};k^R_j])) v_{j,i}
 *   u_t    = W_O [o_{t,1}; ...; o_{t,n_h}]
 *
 * RoPE rotates interleaved pairs (x_2k, x_2k+1) by angle pos * theta_k, theta_k =
 * rope_base^(-2k/d_hr), pos = the token's 0-based index in its sequence.  The page only names
 * "the RoPE matrix"; this is the RoFormer rotation it cites.  With YaRN (section 3.1.4, a layer
 * with rope_scale s > 1) each pair rotates by (1 - g_k) theta_k / s + g_k theta_k instead, where
 * g_k ramps linearly from 0 to 1 as the pair's number of turns over the original context,
 * r_k = rope_orig_ctx * theta_k / (2 pi), goes from yarn_alpha to yarn_beta (the YaRN paper's
 * "NTK-by-parts" frequencies, which the page cites), and the default scale is multiplied by
 * t = (yarn_mscale ln s + 1)^2 (the page gives sqrt(t) = 0.0707 ln s + 1).
 *
 * Conventions for every entry point
 *   - Weights are row-major [out][in] (y = W x), in dims->dtype, device memory, 16-byte aligned.
 *   - The cache pool is [num_blocks][block_size][d_c + d_hr] in dims->dtype (bytes of e4m3 codes
 *     when dims->cache_dtype is MLA_FP8_E4M3, with per-token scales beside it); each token's
 *     entry is [c^KV | k^R] (d_c + d_hr = 576 values at DeepSeek-V2 sizes).  block_table[b][k] is the
 *     physical block holding logical block k of sequence b (int32, device).
 *   - Every pointer argument is a device pointer unless marked "host".
 *   - The caller owns all memory (weights, cache, tables, inputs, outputs, workspace).  The
 *     library never allocates or frees device memory and keeps no state between calls; calls on
 *     different streams are independent as long as their output and workspace buffers differ.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued asynchronously; the
 *     call returns without synchronising.
 *   - Host-side validation runs before anything is enqueued and returns a negative mla_status;
 *     on error nothing has been launched.  Device-side preconditions (block ids < num_blocks,
 *     ctx_lens[b] <= max_ctx_len, positions inside the block table) are the caller's duty; the
 *     MLA_DEBUG build of the library (libmla_debug.so) checks them too, by reading the tables
 *     back before launching (MLA_ERR_INVALID_ARG, with a message on stderr), and synchronises
 *     the device after every launch group (a failing kernel: MLA_ERR_HIP from its own call).
 *   - Accumulation is always fp32.  In MLA_BF16 mode the intermediates handed between kernels
 *     (c^q, q^C, the absorbed query, attention outputs) are stored as bf16.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* NULL pointer, non-positive or inconsistent size */
  MLA_ERR_UNSUPPORTED = -2, /* valid MLA sizes the library has no kernel for */
  MLA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than mla_workspace_size() */
  MLA_ERR_HIP = -4          /* a HIP call or kernel launch failed */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype;

typedef enum { MLA_OP_CACHE_APPEND = 0, MLA_OP_PREFILL = 1, MLA_OP_DECODE = 2, MLA_OP_PREFILL_CHUNK = 3 } mla_op;

/* Layer sizes, in the pages' notation (section 3.1.2; App. B.1). */
typedef struct {
  int32_t d_model;     /* d: hidden size */
  int32_t n_h;         /* attention heads */
  int32_t d_h;         /* per-head content dimension (query/key/value) */
  int32_t d_c;         /* KV compression dimension (latent width) */
  int32_t d_cq;        /* query compression dimension d'_q; 0 = no query compression */
  int32_t d_hr;        /* per-head decoupled rope dimension d_e (d_h^R); even */
  float softmax_scale; /* 0 => 1/sqrt(d_h + d_hr) (App. C), times YaRN's t when it is on */
  float rope_base;     /* RoPE frequency base (10000 for DeepSeek-V2) */
  int32_t dtype;       /* mla_dtype: storage of weights, h, cache, u */
  int32_t cache_dtype; /* element type of the cache pool: 0 = dtype, or MLA_FP8_E4M3 (with
                          dtype MLA_BF16, d_c 512, d_hr 64): the low-bit cache of the serving
                          section (section 3.2.3, "about 6 bits per element"), read here as
                          OCP e4m3 codes with one fp32 scale per token for each of the two
                          parts [c^KV] and [k^R]: s = amax(|part|) / 448 (448 = the largest e4m3
                          value), code = e4m3(x / s), rounded to nearest even, saturating; an
                          all-zero part has s = 0.  The quantised entry is the bf16 entry the
                          bf16 path would store.  Attention reads value(code) * s. */
  /* YaRN context extension (section 3.1.4; off when rope_scale <= 1, e.g. all zero): */
  float rope_scale;      /* s (40 for DeepSeek-V2); finite, >= 0 */
  int32_t rope_orig_ctx; /* original context length the turns are counted over (4096); > 0 when on */
  float yarn_alpha;      /* ramp start in turns (1); >= 0 when on */
  float yarn_beta;       /* ramp end in turns (32); > yarn_alpha when on */
  float yarn_mscale;     /* c in sqrt(t) = c ln s + 1 (0.0707); finite, >= 0 when on; applies to the
                            default scale only (softmax_scale == 0) */
  float rms_eps;         /* epsilon of the latent RMSNorms (see mla_weights); 0 => 1e-6 */
} mla_dims;

/* Device pointers, row-major [out][in].  W_DQ is NULL iff d_cq == 0. */
typedef struct {
  const void *W_DQ;  /* [d_cq][d_model] */
  const void *W_UQ;  /* [n_h*d_h][q_in], q_in = d_cq or d_model */
  const void *W_QR;  /* [n_h*d_hr][q_in] */
  const void *W_DKV; /* [d_c][d_model] */
  const void *W_KR;  /* [d_hr][d_model] */
  const void *W_UK;  /* [n_h*d_h][d_c] */
  const void *W_UV;  /* [n_h*d_h][d_c] */
  const void *W_O;   /* [d_model][n_h*d_h] */
  /* RMSNorm after the compressed latents (section 3.1.2), each optional (NULL = no norm):
   * x <- g * x / sqrt(mean(x^2) + rms_eps) over the d_cq values of c^q (before W_UQ and W_QR;
   * requires d_cq > 0) and over the d_c values of c^KV (before it is cached; the rope key is not
   * normalised).  The page's unspecified bottleneck scaling factors fold into the gains. */
  const void *g_cq;  /* [d_cq] */
  const void *g_ckv; /* [d_c] */
} mla_weights;

/* Paged latent cache (the App. C cached vectors, in pages of block_size tokens). */
typedef struct {
  void *pool;                 /* [num_blocks][block_size][d_c + d_hr], dims->dtype */
  int32_t num_blocks;
  int32_t block_size;         /* tokens per block (64 at DeepSeek-V2 sizes); >= 1 */
  int32_t max_blocks_per_seq; /* columns of block_table */
  const int32_t *block_table; /* [batch][max_blocks_per_seq] */
  float *scales;              /* fp8 cache: [num_blocks][block_size][2] fp32 (s_c, s_r) per token,
                                 written with the codes; else ignored (may be NULL) */
} mla_paged_cache;

/*
 * Bytes of workspace that `op` needs for the given sizes (written to *bytes, host).
 *   MLA_OP_CACHE_APPEND: batch ignored, max_tokens = n (tokens appended in one call).
 *   MLA_OP_PREFILL:      batch sequences of max_tokens tokens each.
 *   MLA_OP_DECODE:       batch sequences, max_ctx_len = largest ctx_lens[b] the call may see,
 *                        num_splits = the value that will be passed to mla_decode (0 = auto).
 *   MLA_OP_PREFILL_CHUNK: batch sequences, chunks of max_tokens tokens, max_ctx_len = the
 *                        largest start position (tokens already cached) a call may see.
 * The size is an upper bound for every call whose sizes (batch, tokens, context) do not exceed
 * these, with the same num_splits.  Returns MLA_OK or MLA_ERR_INVALID_ARG/UNSUPPORTED.
 */
int mla_workspace_size(const mla_dims *dims, int op, int32_t batch, int32_t max_tokens,
                       int32_t max_ctx_len, int32_t num_splits, size_t *bytes);

/*
 * The fp8 cache quantiser alone (the cache_dtype reading above), for tests and for callers that
 * form entries themselves: for each of n dense bf16 entries [c^KV | k^R] (entry = d_c + d_hr
 * values), codes[r][:] = its e4m3 codes and scales[r][0..1] = (s_c, s_r).
 *   entries [n][entry] bf16; codes [n][entry] uint8; scales [n][2] fp32 (all device)
 * Requires dims->cache_dtype == MLA_FP8_E4M3 (else MLA_ERR_INVALID_ARG).
 */
int mla_quantize_entries(const mla_dims *dims, const void *entries, int32_t n, uint8_t *codes,
                         float *scales, void *stream);

/*
 * Cache writer (section 2.1.2 compression, section 2.1.3 shared rope key, App. C cached
 * vectors): for each of n tokens r, entry = [W_DKV h_r | RoPE_{pos[r]}(W_KR h_r)] is stored at
 * pool[block_table[seq_idx[r]][pos[r] / block_size]][pos[r] % block_size][:].
 *   h        [n][d_model], dims->dtype
 *   seq_idx  [n] int32 (row of block_table), pos [n] int32 (0-based position in that sequence)
 * Tokens with the same (seq_idx, pos) write the same slot (last writer unspecified).
 */
int mla_cache_append(const mla_dims *dims, const mla_weights *w, const mla_paged_cache *cache,
                     const void *h, int32_t n, const int32_t *seq_idx, const int32_t *pos,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * Causal prefill (App. C, o_t sums over j = 1..t) of `batch` sequences of T tokens each,
 * starting at position 0.  Writes every token's cache entry (as mla_cache_append, sequence b =
 * block_table row b) and u.  Attention uses the un-absorbed form: per-head keys
 * [W_UK_i c^KV | k^R] and values W_UV_i c^KV are built in the workspace.
 *   h  [batch][T][d_model], u [batch][T][d_model] (dims->dtype)
 *   o_heads: NULL, or fp32 [batch][T][n_h][d_h] receiving the per-head attention outputs o_{t,i}.
 */
int mla_prefill(const mla_dims *dims, const mla_weights *w, const mla_paged_cache *cache,
                const void *h, int32_t batch, int32_t T, void *u, float *o_heads,
                void *workspace, size_t ws_bytes, void *stream);

/*
 * Chunked prefill: the next T tokens of each of `batch` sequences whose first start_pos[b]
 * tokens are already in the cache (App. C's causal sum over j = 1..t with t = start_pos[b] + i:
 * every new token attends to the whole cached prefix and to the new tokens up to itself).
 * mla_prefill is the case start_pos == 0.  Writes the new tokens' cache entries at positions
 * start_pos[b] .. start_pos[b] + T - 1 (sequence b = block_table row b) and u.  Attention uses
 * the un-absorbed form over the prefix read back from the cache (dequantised to bf16 for the fp8
 * cache) and the chunk's own entries as computed (as mla_prefill does), with per-head keys and
 * values built in the workspace.
 *   h  [batch][T][d_model], u [batch][T][d_model] (dims->dtype)
 *   start_pos [batch] int32 (device): tokens already cached in each sequence.
 *   max_start (host) >= every start_pos[b]; sizes the key buffers.  Requires
 *             max_start + T <= max_blocks_per_seq * block_size.
 *   o_heads: NULL, or fp32 [batch][T][n_h][d_h].
 * The workspace is MLA_OP_PREFILL_CHUNK's for (batch, T, max_start).
 */
int mla_prefill_chunk(const mla_dims *dims, const mla_weights *w, const mla_paged_cache *cache,
                      const void *h, int32_t batch, int32_t T, const int32_t *start_pos, int32_t max_start,
                      void *u, float *o_heads, void *workspace, size_t ws_bytes, void *stream);

/*
 * One decode step for `batch` sequences (App. C with the absorption that the page derives
 * from associativity: W_UK_i folds into the query, q_hat_i = W_UK_i^T q^C_i, and W_UV_i is
 * applied after the softmax, o_i = W_UV_i sum_j p_ij c^KV_j, so attention reads only the
 * cached [c^KV | k^R] entries, shared by all heads).
 *   h         [batch][d_model] hidden state of the new token of each sequence
 *   ctx_lens  [batch] int32: tokens already cached before this step.  The new token's entry is
 *             written at position ctx_lens[b] and the token attends over ctx_lens[b] + 1 entries.
 *             The library does not modify ctx_lens.
 *   max_ctx_len (host) >= every ctx_lens[b]; sizes the grid.  Requires
 *             max_ctx_len + 1 <= max_blocks_per_seq * block_size.
 *   num_splits (host): KV partitions per sequence (split-KV, combined by a log-sum-exp
 *             reduction); 0 = chosen from the sizes and the device's compute-unit count.
 *             With 0 and fewer than 16 (sequence, 128-head group) units, the bf16 and fp8
 *             paged kernels size their partitions on the device from ctx_lens (up to twice
 *             the automatic count per sequence), so that ragged contexts load the compute
 *             units evenly; otherwise each partition covers a fixed token range.
 *   u         [batch][d_model] output
 *   o_heads   NULL, or fp32 [batch][n_h][d_h] receiving o_{t,i}.
 */
int mla_decode(const mla_dims *dims, const mla_weights *w, const mla_paged_cache *cache,
               const void *h, int32_t batch, const int32_t *ctx_lens, int32_t max_ctx_len,
               int32_t num_splits, void *u, float *o_heads, void *workspace, size_t ws_bytes,
               void *stream);

/*
 * Allocation-free variant of mla_decode, for callers that cannot allocate device memory or hand
 * over a workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and validation as mla_decode, without the workspace.
 *   - Scratch: the library's own device array of MLA_NOALLOC_SCRATCH_BYTES on each device,
 *     reserved when the library's code object loads on that device and held until the process
 *     ends; its address is looked up once per device, on the first call there.  Nothing in it
 *     needs to start at zero.
 *   - Calls whose sizes need more, i.e. mla_workspace_size(MLA_OP_DECODE, batch, 0, max_ctx_len,
 *     num_splits) > MLA_NOALLOC_SCRATCH_BYTES, return MLA_ERR_WORKSPACE and launch nothing.
 *     (DeepSeek-V2 sizes: batch 64 at any context up to 131072 fits.)
 *   - Every call on one device uses that device's one array: calls that overlap in time on one
 *     device (on different streams, or from threads without ordering) race and their results are
 *     undefined.  Calls on one stream are ordered and safe.
 *   - Allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
int mla_decode_noalloc(const mla_dims *dims, const mla_weights *w, const mla_paged_cache *cache,
                       const void *h, int32_t batch, const int32_t *ctx_lens, int32_t max_ctx_len,
                       int32_t num_splits, void *u, float *o_heads, void *stream);

/*
 * Decode attention core only (the split-KV latent attention and its reduction), for timing and
 * kernel-level tests.  Inputs are the absorbed queries already formed:
 *   q        [batch][n_h][d_c + d_hr], dims->dtype: [q_hat_i | RoPE'd q^R_i] per head
 *   kv_lens  [batch] int32: entries to attend over (positions 0..kv_lens[b]-1 of the cache)
 *   max_kv_len (host) >= every kv_lens[b]
 *   o_hat    [batch][n_h][d_c] output, dims->dtype: sum_j softmax_j(scale * q . entry_j) c^KV_j
 *   lse      NULL or fp32 [batch][n_h]: natural-log log-sum-exp of the scaled scores
 * Workspace: mla_workspace_size(MLA_OP_DECODE, batch, 0, max_kv_len - 1, num_splits).
 */
int mla_decode_attention(const mla_dims *dims, const mla_paged_cache *cache, const void *q,
                         int32_t batch, const int32_t *kv_lens, int32_t max_kv_len,
                         int32_t num_splits, void *o_hat, float *lse, void *workspace,
                         size_t ws_bytes, void *stream);

/*
 * The decode attention core without the reduction of its KV partitions: the attention kernel that
 * mla_decode runs, with each partition's result left in caller buffers.  For callers that reduce
 * the partitions themselves (e.g. GPUs that hold different page ranges of one sequence, each
 * contributing its partitions to one log-sum-exp reduction), and for timing the kernel alone.
 *   q, kv_lens, max_kv_len: as mla_decode_attention.
 *   num_splits (host) >= 1: the partition length is ceil(ceil(max_kv_len / 64) / num_splits) * 64
 *             tokens; partition p of sequence b covers its tokens [p * length, (p + 1) * length).
 *   *splits_out (host): P, the number of partitions (<= num_splits); the buffers below hold
 *             batch * P rows of n_h heads.
 *   part_m    [batch][P][n_h] fp32: a reference for the partition's scores x_j = scale * log2(e) *
 *             (q . entry_j), within 64 of their maximum: max_j x_j - 64 <= part_m <= max_j x_j
 *             (-inf for a partition with no tokens);
 *   part_l    [batch][P][n_h] fp32: sum_j 2^(x_j - part_m);
 *   part_o    [batch][P][n_h][d_c] bf16: sum_j 2^(x_j - part_m) c^KV_j / part_l (the partition's
 *             normalised output; not written for a partition with no tokens).
 *   The combined result is o_hat = sum_p w_p part_o_p / sum_p w_p with w_p = 2^(part_m_p - M)
 *   part_l_p, M = max_p part_m_p.
 * Requires dims->dtype MLA_BF16, d_c 512, d_hr 64 and block_size a multiple of 32 (else
 * MLA_ERR_UNSUPPORTED).  Needs no workspace.
 */
int mla_decode_attention_partials(const mla_dims *dims, const mla_paged_cache *cache, const void *q,
                                  int32_t batch, const int32_t *kv_lens, int32_t max_kv_len,
                                  int32_t num_splits, float *part_m, float *part_l, void *part_o,
                                  int32_t *splits_out, void *stream);

/* The split count mla_decode uses for num_splits == 0 with fixed partitions (host query; -1 on
 * invalid sizes).  Small batches with num_splits == 0 use up to twice as many partition slots,
 * balanced over the actual context lengths (see mla_decode). */
int32_t mla_decode_auto_splits(const mla_dims *dims, int32_t batch, int32_t max_ctx_len);

/* Static text for a status code. */
const char *mla_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
