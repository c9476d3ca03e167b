/*
 * libmla -- Multi-head Latent Attention (DeepSeek-V2) decode over a compressed
 * latent KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method (DeepSeek-V2 reading card, ai-papers.xuzou.cn, "Bottlenecks" and
 * "Method adaptation"; discosf explainer, "long-context bottleneck" and
 * "decoupled RoPE and YaRN" sections): each cached token holds only a latent
 * c_KV of width d_c = 512 and one decoupled RoPE key k_pe of width d_R = 64
 * that all heads share, 576 elements per token per layer. Keys and values of
 * head h are c_KV up-projected by W_UK[h] and W_UV[h]; because W_UK folds into
 * the query side and W_UV into the output side, attention runs directly on the
 * 576-wide latent rows and K/V are never materialised.
 *
 * Conventions shared by every call
 *  - Pointers marked (device) are device memory on the current HIP device;
 *    pointers marked (host) are host memory. Every call only enqueues work on
 *    `stream` (a hipStream_t; NULL is the legacy default stream) and returns
 *    without synchronising (MLA_DEBUG below aside). The library allocates no
 *    device memory and keeps no state between calls (mla_decode_noalloc's
 *    per-device array aside), and may run concurrently on several streams
 *    when each call has its own workspace and outputs.
 *  - The caller owns every buffer. Inputs are only read; outputs and the
 *    workspace are overwritten.
 *  - Host-side validation happens before any HIP call. A call that returns
 *    an error enqueued nothing. MLA_ERR_HIP reports a launch failure.
 *  - Device-resident values outside the contract (lengths outside
 *    [1, capacity], appended tokens with a sequence outside [0, B) or a
 *    position outside [0, capacity)) are clamped or skipped as each call
 *    documents. With MLA_DEBUG=1 in the environment, mla_decode and its
 *    stages, mla_append and mla_append_absorb first copy those arrays (and
 *    seq_start/seq_capacity, whose rows must lie inside the cache) to the
 *    host on `stream`, synchronise it, and return MLA_ERR_INVALID_ARGUMENT
 *    without running anything if one is violated (MLA_ERR_HIP if a copy
 *    fails). This is the only case in which a call synchronises.
 *  - Kernel choice switches read from the environment at each decode call:
 *    MLA_FP8_MFMA=1 runs the value contraction over an fp8 cache (32 heads
 *    or more) on fp8 MFMA with e4m3 value weights (output error about 2e-2
 *    relative instead of about 3e-3); MLA_H32=1 selects the 128-head
 *    one-wave-per-SIMD kernel for a bf16 cache. Results stay within the
 *    decode tolerances either way.
 *  - All tensors are dense and row-major with the shapes given.
 */
#ifndef LIBMLA_H
#define LIBMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1
#define MLA_D_C 512          /* latent width d_c */
#define MLA_D_R 64           /* decoupled RoPE key width d_R */
#define MLA_D_ROW 576        /* d_c + d_R elements per cached token */
#define MLA_D_NOPE 128       /* per-head non-RoPE query/key width */
#define MLA_D_V 128          /* per-head value width */

/* Status codes and dtype codes are plain 32-bit integers (the named values
 * below), so that any value a caller passes, valid or not, is well defined
 * to receive and is rejected by validation rather than being undefined. */
typedef int32_t mla_status_t;
enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size or shape */
  MLA_ERR_UNSUPPORTED = 2,        /* valid but unsupported dtype combination / head count */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
};

typedef int32_t mla_dtype_t;
enum {
  MLA_DTYPE_F32 = 0,
  MLA_DTYPE_BF16 = 1,
  MLA_DTYPE_FP8_E4M3 = 2,         /* OCP e4m3fn codes (max 448, no infinities) */
  MLA_DTYPE_FP6_E2M3_MX = 3       /* 6-bit e2m3 codes in blocks of 32 with e8m0 scales */
};

/*
 * Ragged per-sequence latent cache (the MLA cache of one layer). The struct
 * itself is host memory; the arrays it points to are device memory.
 *
 * Sequence b owns rows [seq_start[b], seq_start[b] + seq_capacity[b]) of
 * `rows`. Row r is c_KV (elements 0..511) followed by k_pe (512..575), stored
 * in `dtype`. For MLA_DTYPE_FP8_E4M3 the value of element i of row r is
 * e4m3(rows[r][i]) * row_scale[r]; one fp32 scale covers the whole row.
 * MLA_DTYPE_FP6_E2M3_MX is the ~6-bit cache (the pages quantise the deployed
 * cache to about 6 bits per element on average without naming a format:
 * DeepSeek-V2 reading card, "Method adaptation"): OCP microscaling FP6. A
 * row is 464 bytes: bytes 0..431 hold the 576 six-bit e2m3 codes (sign,
 * 2-bit exponent with bias 1, 3-bit mantissa; largest 7.5) packed
 * little-endian, element i in bits 6i .. 6i+5; bytes 432..449 the 18 e8m0
 * scale codes of the blocks of 32 elements; bytes 450..463 padding (written
 * as zero by mla_append). Element i's value is e2m3(code_i) *
 * 2^(scale[i / 32] - 127); row_scale must be NULL. Row ranges of different
 * sequences must not overlap.
 */
typedef struct {
  mla_dtype_t dtype;             /* element type of rows: F32, BF16, FP8_E4M3 or FP6_E2M3_MX */
  int32_t d_c;                   /* must be 512 */
  int32_t d_r;                   /* must be 64 */
  int32_t num_seqs;              /* B >= 1 */
  int64_t total_rows;            /* rows allocated in `rows` (>= 1) */
  void* rows;                    /* (device) [total_rows][576] elements (FP6: [total_rows][464] bytes) */
  float* row_scale;              /* (device) [total_rows] for FP8_E4M3, else NULL */
  const int64_t* seq_start;      /* (device) [B] first row of sequence b */
  const int32_t* seq_capacity;   /* (device) [B] rows reserved for sequence b */
} mla_cache_t;

/*
 * Paged latent cache: the same rows in a pool of pages of `page_tokens` rows
 * each, found through a per-sequence block table (the layout behind the
 * PagedAttention of the serving engines the mlqm.cn deployment guide names,
 * sections 3.2 "software environment" and 8.2 "deployment optimisation").
 * Token t (0 <= t < max_pages * page_tokens) of sequence b is row
 *   block_table[b][t / page_tokens] * page_tokens + t % page_tokens
 * of `rows`; rows and row scales are stored as in mla_cache_t. page_tokens is
 * a positive multiple of 32 (a 32-token tile never spans two pages). Entries
 * a call uses (blocks below ceil(len / page_tokens) for decode, the block of
 * each appended position for append) must lie in [0, total_pages): decode
 * reads page 0 instead of an entry outside the pool, append skips such a
 * token, and MLA_DEBUG=1 reports either as MLA_ERR_INVALID_ARGUMENT. Pages of
 * different sequences must not overlap where rows are written.
 */
typedef struct {
  mla_dtype_t dtype;             /* element type of rows: F32, BF16, FP8_E4M3 or FP6_E2M3_MX */
  int32_t d_c;                   /* must be 512 */
  int32_t d_r;                   /* must be 64 */
  int32_t num_seqs;              /* B >= 1 */
  int32_t page_tokens;           /* rows per page: a positive multiple of 32 */
  int32_t max_pages;             /* block-table columns (pages per sequence) >= 1 */
  int64_t total_pages;           /* pages in `rows` >= 1 */
  void* rows;                    /* (device) [total_pages * page_tokens][576] (FP6: [..][464] bytes) */
  float* row_scale;              /* (device) [total_pages * page_tokens] for FP8_E4M3, else NULL */
  const int32_t* block_table;    /* (device) [B][max_pages] page of each block */
} mla_paged_cache_t;

/*
 * mla_append -- compress hidden states into latent cache rows.
 *
 * For each token n (discosf explainer, "long-context bottleneck" and
 * "decoupled RoPE" sections; DeepSeek-V2 reading card, "Method adaptation"):
 *   c      = W_DKV h[n]                  (512 values)
 *   k      = W_KR  h[n]                  (64 values)
 *   k_pe   = RoPE(k, pos)                pairs (2i, 2i+1), i = 0..31, rotated by
 *                                        pos * rope_base^(-2i/64); the angle is
 *                                        formed and reduced to [-pi, pi] in fp64,
 *                                        its sine and cosine taken in fp32 (BF16
 *                                        cache) or fp64 (F32, FP8_E4M3, FP6)
 *   row    = c || k_pe, stored at row seq_start[s] + pos of the cache, where
 *            s = tok_seq[n] and pos = tok_pos[n] (pos is both the slot and the
 *            RoPE position, 0-based within the sequence).
 * Storage: F32 as computed; BF16 rounded to nearest even; FP8_E4M3 with
 * row_scale = max|row| / 448 (1 for an all-zero row) and codes rounded to
 * nearest even with saturation at +-448; FP6_E2M3_MX per block of 32
 * elements with scale 2^X, X = floor(log2(max|block|)) - 2 (scale code 0 for
 * an all-zero block), codes rounded to nearest even with saturation at
 * +-7.5.
 * Arithmetic: products in `act_dtype`, fp32 accumulation.
 *
 *   h        (device) [n_tok][d_model] in act_dtype
 *   w_dkv    (device) [512][d_model] in act_dtype
 *   w_kr     (device) [64][d_model] in act_dtype
 *   tok_seq  (device) [n_tok] sequence of each token
 *   tok_pos  (device) [n_tok] slot/position of each token
 * act_dtype must be F32 (with an F32 cache) or BF16 (with a BF16, FP8 or
 * FP6 cache); d_model must be a positive multiple of 64. A token whose sequence
 * is outside [0, B) or whose position is outside [0, seq_capacity) is not
 * written. Two tokens naming the same slot race. n_tok == 0 is a no-op.
 * The call does not change any length: the caller passes lengths to decode.
 */
mla_status_t mla_append(const mla_cache_t* cache,
                        const void* h, int32_t n_tok, int32_t d_model,
                        const void* w_dkv, const void* w_kr, mla_dtype_t act_dtype,
                        const int32_t* tok_seq, const int32_t* tok_pos,
                        float rope_base, void* stream);

/*
 * YaRN parameters of the decoupled RoPE key (discosf explainer, "decoupled
 * RoPE and YaRN" section: YaRN with scale 40, alpha 1, beta 32 extends the
 * context to 160K; the formula is the published YaRN method's). For pair i,
 * theta_i = base^(-2i/64) turns orig_context * theta_i / (2 pi) times over the
 * original context; with gamma = clamp((turns - alpha) / (beta - alpha), 0, 1)
 * the pair rotates at theta'_i = (1 - gamma) * theta_i / scale + gamma * theta_i
 * (computed in fp64 on the host). DeepSeek-V2's values: base 10000, scale 40,
 * alpha 1, beta 32, orig_context 4096 (160K / 40).
 */
typedef struct {
  float base;                    /* > 0 */
  float scale;                   /* >= 1 (1 gives plain RoPE) */
  float alpha;                   /* >= 0 */
  float beta;                    /* > alpha */
  int32_t orig_context;          /* >= 1 */
} mla_yarn_t;

/*
 * mla_append_yarn -- mla_append with the RoPE key rotated at the YaRN
 * frequencies theta'_i of `rope` (host) instead of base^(-2i/64); everything
 * else (arguments, storage, rules) as mla_append. A NULL or out-of-range
 * `rope` returns MLA_ERR_INVALID_ARGUMENT.
 */
mla_status_t mla_append_yarn(const mla_cache_t* cache,
                             const void* h, int32_t n_tok, int32_t d_model,
                             const void* w_dkv, const void* w_kr, mla_dtype_t act_dtype,
                             const int32_t* tok_seq, const int32_t* tok_pos,
                             const mla_yarn_t* rope, void* stream);

/*
 * mla_yarn_softmax_factor -- the factor YaRN's attention temperature puts on
 * the softmax scale: (0.1 ln scale + 1)^2 for scale > 1, else 1. A decode over
 * rows appended with mla_append_yarn passes softmax_scale times this factor.
 */
float mla_yarn_softmax_factor(float scale);

/*
 * mla_decode_workspace_size -- bytes of device workspace mla_decode needs for
 * `num_seqs` sequences and `n_heads` heads with the given dtypes. The result
 * does not depend on the sequence lengths. Writes *bytes (host).
 */
mla_status_t mla_decode_workspace_size(int32_t num_seqs, int32_t n_heads,
                                       mla_dtype_t cache_dtype, mla_dtype_t act_dtype,
                                       size_t* bytes);

/*
 * mla_decode -- one decode step of MLA attention for B sequences.
 *
 * For sequence b with L = seq_len[b] cached rows (c_t, k_pe_t), t < L, and
 * head h (discosf explainer, "long-context bottleneck": the new token attends
 * to all previous tokens; W_UK folds into the query, W_UV into the output):
 *   q_lat   = W_UK[h]^T q_nope[b,h]                         (512)
 *   s_t     = softmax_scale * (q_lat . c_t + q_pe[b,h] . k_pe_t)
 *   p       = softmax(s)    over t = 0..L-1 (no mask)
 *   out[b,h]= W_UV[h]^T (sum_t p_t c_t)                       (128)
 *   lse[b,h]= ln sum_t exp(s_t)                               (if lse != NULL)
 * which equals attention with keys K_t = W_UK[h] c_t ++ k_pe_t and values
 * V_t = W_UV[h]^T c_t. q_pe arrives already rotated; decode applies no RoPE.
 *
 *   seq_len  (device) [B], 1 <= seq_len[b] <= seq_capacity[b]. Values outside
 *            are clamped to [0, seq_capacity[b]], so no row outside the
 *            sequence is read; a sequence of length 0 yields out = 0 and
 *            lse = -inf.
 *   q_nope   (device) [B][H][128] in act_dtype
 *   q_pe     (device) [B][H][64]  in act_dtype
 *   w_uk     (device) [H][128][512] in act_dtype   (k = W_UK[h] c)
 *   w_uv     (device) [H][512][128] in act_dtype   (v = W_UV[h]^T c)
 *   out      (device) [B][H][128] in act_dtype
 *   lse      (device) [B][H] fp32, natural log, or NULL
 *   workspace(device) at least mla_decode_workspace_size(...) bytes, 256-byte
 *            aligned; contents on entry are ignored.
 * Supported (cache dtype, act_dtype): (F32, F32), (BF16, BF16),
 * (FP8_E4M3, BF16), (FP6_E2M3_MX, BF16). n_heads must be a positive multiple
 * of 16. FP6 rows are widened exactly to bf16 (block scales applied) once per
 * tile in LDS. Arithmetic:
 * bf16 (or fp32 for F32) matrix products with fp32 accumulation; softmax in
 * fp32. The result is deterministic: no floating-point atomics.
 */
mla_status_t mla_decode(const mla_cache_t* cache, const int32_t* seq_len,
                        const void* q_nope, const void* q_pe,
                        const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                        int32_t n_heads, float softmax_scale,
                        void* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_append_paged / mla_decode_paged -- mla_append and mla_decode over a
 * paged cache: same arguments, rules and results, with each sequence's
 * capacity max_pages * page_tokens and its rows found through the block
 * table. mla_decode_paged takes the workspace of mla_decode_workspace_size and
 * equals mla_decode over the same rows laid out contiguously, bit for bit.
 */
mla_status_t mla_append_paged(const mla_paged_cache_t* cache,
                              const void* h, int32_t n_tok, int32_t d_model,
                              const void* w_dkv, const void* w_kr, mla_dtype_t act_dtype,
                              const int32_t* tok_seq, const int32_t* tok_pos,
                              float rope_base, void* stream);
mla_status_t mla_decode_paged(const mla_paged_cache_t* cache, const int32_t* seq_len,
                              const void* q_nope, const void* q_pe,
                              const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                              int32_t n_heads, float softmax_scale,
                              void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_append_yarn_paged -- mla_append_yarn into a paged cache: the rows of
 * mla_append_paged with the RoPE key at the YaRN frequencies of `rope`.
 */
mla_status_t mla_append_yarn_paged(const mla_paged_cache_t* cache,
                                   const void* h, int32_t n_tok, int32_t d_model,
                                   const void* w_dkv, const void* w_kr, mla_dtype_t act_dtype,
                                   const int32_t* tok_seq, const int32_t* tok_pos,
                                   const mla_yarn_t* rope, void* stream);

/*
 * The three stages mla_decode runs, exposed so a caller can time or
 * interleave them. Same arguments and rules as mla_decode; calling
 * absorb, attend and combine in this order on one stream with the same
 * workspace equals one mla_decode call. attend and combine trust the work
 * plan absorb left in the workspace: calling them on a workspace that absorb
 * (or mla_append_absorb) has not prepared with the same cache, lengths and
 * head count is undefined, and can read and write outside the buffers. The workspace carries the
 * intermediate results between the stages:
 *   absorb  -- q_lat = W_UK[h]^T q_nope for every (b, h), and the work plan
 *              (tile counts of the clamped lengths, each worker's tile range)
 *              that partitions the attention (discosf explainer, "long-context
 *              bottleneck": W_UK folds into the query);
 *   attend  -- streams the latent rows once and writes, per tile range and
 *              sequence, the running max, sum and normalised sum_t p_t c_t / l
 *              (split-K);
 *   combine -- merges the ranges of each sequence and applies W_UV (W_UV folds
 *              into the output), writing out and lse.
 */
mla_status_t mla_decode_absorb(const mla_cache_t* cache, const int32_t* seq_len,
                               const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                               int32_t n_heads, float softmax_scale,
                               void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);
mla_status_t mla_decode_attend(const mla_cache_t* cache, const int32_t* seq_len,
                               const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                               int32_t n_heads, float softmax_scale,
                               void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);
mla_status_t mla_decode_combine(const mla_cache_t* cache, const int32_t* seq_len,
                                const void* q_nope, const void* q_pe,
                                const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                                int32_t n_heads, float softmax_scale,
                                void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);
/* attend then combine in one call (stages 2 and 3): what completes a decode
 * step after mla_decode_absorb or mla_append_absorb, with one host call. */
mla_status_t mla_decode_attend_combine(const mla_cache_t* cache, const int32_t* seq_len,
                                       const void* q_nope, const void* q_pe,
                                       const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                                       int32_t n_heads, float softmax_scale,
                                       void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_append_absorb -- mla_append followed by mla_decode_absorb, in one launch
 * where it applies (BF16 cache and activations, and a grid that fits the GPU
 * at once); otherwise the two run one after the other. The absorb product and
 * the work plan read queries, W_UK and lengths, never cache rows, so the two
 * do not depend on each other. Arguments: mla_append's (cache, h ... rope_base)
 * then mla_decode's (seq_len ... stream), with the same meaning, ownership and
 * rules; both argument sets are validated before anything runs. Calling
 * mla_decode_attend and mla_decode_combine (or mla_decode_attend_combine)
 * afterwards with the same decode arguments and workspace completes the
 * decode step: the result equals mla_append then mla_decode, bit for bit.
 * For callers that run a decode step right after appending its token.
 */
mla_status_t mla_append_absorb(const mla_cache_t* cache,
                               const void* h, int32_t n_tok, int32_t d_model,
                               const void* w_dkv, const void* w_kr,
                               const int32_t* tok_seq, const int32_t* tok_pos, float rope_base,
                               const int32_t* seq_len, const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                               int32_t n_heads, float softmax_scale,
                               void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_noalloc -- mla_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops or harnesses that forbid hipMalloc). Same arguments, rules and result
 * as mla_decode (bit for bit with the same inputs); the workspace is a
 * library-owned device array of MLA_NOALLOC_WORKSPACE_BYTES per device,
 * reserved when the library's device code loads on that device and held until
 * the process ends. The call allocates nothing and needs no clearing of that
 * array. It returns MLA_ERR_WORKSPACE_TOO_SMALL, having enqueued nothing,
 * when mla_decode_workspace_size for (num_seqs, n_heads, dtypes) exceeds
 * MLA_NOALLOC_WORKSPACE_BYTES (about 100 sequences at 128 heads over a bf16
 * cache), and MLA_ERR_HIP if the array's device address cannot be found.
 * All calls on one device share its array: calls that overlap in time on one
 * device (different streams, or host threads, without ordering between them)
 * race and give undefined results. Calls on one stream are ordered and safe.
 */
#define MLA_NOALLOC_WORKSPACE_BYTES (64u << 20)
mla_status_t mla_decode_noalloc(const mla_cache_t* cache, const int32_t* seq_len,
                                const void* q_nope, const void* q_pe,
                                const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                                int32_t n_heads, float softmax_scale,
                                void* out, float* lse, void* stream);

/*
 * mla_prefill -- causal multi-query (prefill) attention over the latent cache.
 * The pages report prompt processing beside generation (DeepSeek-V2 reading
 * card, "Evidence": over 100K prompt tokens/s on one 8-GPU node) but give no
 * prefill formula; this call takes the plain reading. The queries of
 * sequence b are query rows q_start[b] .. q_start[b+1]-1, its LAST
 * n_b = q_start[b+1] - q_start[b] positions: query row q_start[b] + i sits at
 * position p = seq_len[b] - n_b + i and attends cache rows 0..p of b (their
 * rows must already be in the cache, e.g. from mla_append). Score, softmax
 * and output are mla_decode's for a sequence of length p + 1 (discosf
 * explainer, "long-context bottleneck"): o = sum_t softmax_t(s) (W_UV[h]^T c_t),
 * s_t = softmax_scale * (q_nope . W_UK[h] c_t + q_pe . k_pe,t); it is computed
 * in the unabsorbed form (each cached row up-projected once to per-head K and
 * V, rounded to bf16 in the workspace).
 *   cache          contiguous cache, BF16, FP8_E4M3 or FP6_E2M3_MX (F32:
 *                  MLA_ERR_UNSUPPORTED).
 *   seq_len        device int32 [num_seqs], in [0, capacity].
 *   q_start        device int32 [num_seqs + 1], non-decreasing from 0 to n_q,
 *                  with n_b <= seq_len[b].
 *   n_q            query rows (0: nothing runs).
 *   max_kv_rows    host bound >= sum of seq_len; sizes the workspace.
 *   q_nope, q_pe   device BF16 [n_q][n_heads][128], [n_q][n_heads][64].
 *   w_uk, w_uv     device BF16 [n_heads][128][512], [n_heads][512][128].
 *   act_dtype      MLA_DTYPE_BF16 (others: MLA_ERR_UNSUPPORTED).
 *   n_heads        1..1024, any count.
 *   out            device BF16 [n_q][n_heads][128]; lse device F32
 *                  [n_q][n_heads] (natural log) or NULL.
 *   workspace      device, 256-byte aligned, at least
 *                  mla_prefill_workspace_size(num_seqs, n_heads, n_q,
 *                  max_kv_rows) bytes (about 64 KB per cached row at 128
 *                  heads); caller-owned, overwritten.
 * Contract values on the device are clamped: lengths into [0, capacity],
 * q_start into [0, n_q]; a query whose position would be negative gets o = 0
 * and lse = -inf, and so do the queries of every sequence from the first
 * whose rows pass max_kv_rows. MLA_DEBUG=1 reports those cases as
 * MLA_ERR_INVALID_ARGUMENT. Errors: MLA_ERR_INVALID_ARGUMENT (null pointer,
 * bad count or scale, misaligned workspace), MLA_ERR_UNSUPPORTED (dtypes,
 * sizes past the limits), MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP.
 */
mla_status_t mla_prefill_workspace_size(int32_t num_seqs, int32_t n_heads, int64_t n_q,
                                        int64_t max_kv_rows, size_t* bytes);
mla_status_t mla_prefill(const mla_cache_t* cache, const int32_t* seq_len, const int32_t* q_start,
                         int64_t n_q, int64_t max_kv_rows, const void* q_nope, const void* q_pe,
                         const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                         int32_t n_heads, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_prefill_paged -- mla_prefill over a paged cache (the layout of
 * mla_decode_paged: each sequence's capacity max_pages * page_tokens, its rows
 * found through the block table): same arguments, rules and workspace, and
 * the same result as mla_prefill over those rows laid out contiguously, bit
 * for bit. A table entry outside the page pool reads page 0 of the pool (as
 * the paged decode does); MLA_DEBUG=1 rejects such entries instead.
 */
mla_status_t mla_prefill_paged(const mla_paged_cache_t* cache, const int32_t* seq_len,
                               const int32_t* q_start, int64_t n_q, int64_t max_kv_rows,
                               const void* q_nope, const void* q_pe, const void* w_uk,
                               const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                               float softmax_scale, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Static English text for a status code (host); "unknown status" for any
 * other value. */
const char* mla_status_string(mla_status_t status);

/* MLA_ABI_VERSION of the loaded library. */
int mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_H */
