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
 *    device memory, keeps no state between calls, and may run concurrently
 *    on several streams when each call has its own workspace and outputs.
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

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size or shape */
  MLA_ERR_UNSUPPORTED = 2,        /* valid but unsupported dtype combination / head count */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} mla_status_t;

typedef enum {
  MLA_DTYPE_F32 = 0,
  MLA_DTYPE_BF16 = 1,
  MLA_DTYPE_FP8_E4M3 = 2          /* OCP e4m3fn codes (max 448, no infinities) */
} mla_dtype_t;

/*
 * Ragged per-sequence latent cache (the MLA cache of one layer). The struct
 * itself is host memory; the arrays it points to are device memory.
 *
 * Sequence b owns rows [seq_start[b], seq_start[b] + seq_capacity[b]) of
 * `rows`. Row r is c_KV (elements 0..511) followed by k_pe (512..575), stored
 * in `dtype`. For MLA_DTYPE_FP8_E4M3 the value of element i of row r is
 * e4m3(rows[r][i]) * row_scale[r]; one fp32 scale covers the whole row. Row
 * ranges of different sequences must not overlap.
 */
typedef struct {
  mla_dtype_t dtype;             /* element type of rows: F32, BF16 or FP8_E4M3 */
  int32_t d_c;                   /* must be 512 */
  int32_t d_r;                   /* must be 64 */
  int32_t num_seqs;              /* B >= 1 */
  int64_t total_rows;            /* rows allocated in `rows` (>= 1) */
  void* rows;                    /* (device) [total_rows][576] */
  float* row_scale;              /* (device) [total_rows] for FP8_E4M3, else NULL */
  const int64_t* seq_start;      /* (device) [B] first row of sequence b */
  const int32_t* seq_capacity;   /* (device) [B] rows reserved for sequence b */
} mla_cache_t;

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
 *                                        cache) or fp64 (F32, FP8_E4M3)
 *   row    = c || k_pe, stored at row seq_start[s] + pos of the cache, where
 *            s = tok_seq[n] and pos = tok_pos[n] (pos is both the slot and the
 *            RoPE position, 0-based within the sequence).
 * Storage: F32 as computed; BF16 rounded to nearest even; FP8_E4M3 with
 * row_scale = max|row| / 448 (1 for an all-zero row) and codes rounded to
 * nearest even with saturation at +-448.
 * Arithmetic: products in `act_dtype`, fp32 accumulation.
 *
 *   h        (device) [n_tok][d_model] in act_dtype
 *   w_dkv    (device) [512][d_model] in act_dtype
 *   w_kr     (device) [64][d_model] in act_dtype
 *   tok_seq  (device) [n_tok] sequence of each token
 *   tok_pos  (device) [n_tok] slot/position of each token
 * act_dtype must be F32 (with an F32 cache) or BF16 (with a BF16 or FP8
 * cache); d_model must be a positive multiple of 64. A token whose sequence
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
 * (FP8_E4M3, BF16). n_heads must be a positive multiple of 16. Arithmetic:
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
 * The three stages mla_decode runs, exposed so a caller can time or
 * interleave them. Same arguments and rules as mla_decode; calling
 * absorb, attend and combine in this order on one stream with the same
 * workspace equals one mla_decode call. The workspace carries the
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

/* Static English text for a status code (host). */
const char* mla_status_string(mla_status_t status);

/* MLA_ABI_VERSION of the loaded library. */
int mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_H */
