// C ABI of libmla: argument validation, launch planning, workspace layout
// and launch sequencing on the caller's stream. No call here allocates,
// synchronises or keeps state; every check runs before the first HIP call.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "../../include/libmla.h"
#include "internal.h"

#include <mutex>
#include <vector>

namespace mla {

static constexpr int kMaxHeads = 1024;
static constexpr int kMaxSeqs = 1 << 20;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// An environment switch read at planning time (experiments only).
static bool getenv_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] == '1' && v[1] == 0;
}

DecodePlan make_plan(int ct, int B, int H) {
  DecodePlan p{};
  if (ct == kBF16 && H % 128 == 0 && getenv_flag("MLA_H32")) {
    // 128-head groups over a bf16 cache: four waves of 32 heads, one per
    // SIMD, a four-stage ring (opt-in while it is slower than the pair kernel)
    p.h32 = true;
    p.nstage = 4;
    p.head_groups = H / 128;
  } else if ((ct == kBF16 || ct == kFP8 || ct == kFP6) && H % 32 == 0) {
    // pair kernels: up to 128 heads (8 waves) per workgroup; the ring depth
    // is what fits in LDS beside the exchange buffers (and, for fp6, two
    // widened bf16 tiles)
    p.pair = true;
    p.np = (H % 128 == 0) ? 4 : (H % 64 == 0) ? 2 : 1;
    p.nstage = (ct == kFP8 || (ct == kBF16 && p.np == 1)) ? 4 : 3;
    p.head_groups = H / (32 * p.np);
    p.f8 = ct == kFP8 && getenv_flag("MLA_FP8_MFMA");
  } else if (ct == kBF16) {
    // 16-head blocks over a bf16 cache: the streaming kernel
    p.stream = true;
    p.nstage = 3;
    p.head_groups = H / 16;
  } else {
    p.hb = 1;
    p.ds = 4;
    p.nstage = (ct == kF32) ? 2 : 4;
    p.head_groups = H / 16;
  }
  p.tile = (ct == kF32) ? 16 : 32;
  // what a segment start costs in tiles of work: queries in and a partial
  // out; the pair kernel moves 147 KB of queries and 128 KB of partial per
  // segment and drains its copy queue (measured best: 1 for the streaming
  // kernel against 0..6, 5 for the pair kernel against 1..6)
  p.seg_tiles = p.h32 ? 3 : (p.pair ? 5 : 1);
  int w = kTargetCUs / p.head_groups;
  w = w < 8 ? 8 : (w / 8) * 8;                 // a multiple of the 8 XCDs
  p.workers = w;
  p.nslot = (int64_t)w + B;
  (void)B;
  return p;
}

WorkspaceLayout workspace_layout(int ct, int B, int H) {
  const DecodePlan p = make_plan(ct, B, H);
  WorkspaceLayout l{};
  size_t off = 0;
  l.seqinfo = off; off = align256(off + sizeof(SeqInfo) * (size_t)B);
  l.starts = off;  off = align256(off + sizeof(int64_t) * ((size_t)p.workers + 1));
  l.wseq = off;    off = align256(off + sizeof(int32_t) * (size_t)p.workers);
  l.winfo = off;   off = align256(off + sizeof(WorkerInfo) * (size_t)p.workers);
  l.wfirst = off;  off = align256(off + sizeof(int32_t) * (size_t)B);
  l.wlast = off;   off = align256(off + sizeof(int32_t) * (size_t)B);
  l.q_lat = off;   off = align256(off + (size_t)B * H * MLA_D_C * (ct == kF32 ? 4 : 2));
  l.part_o = off;  off = align256(off + (size_t)p.nslot * H * MLA_D_C * (ct == kF32 ? 4 : 2));
  l.part_ml = off; off = align256(off + (size_t)p.nslot * H * 2 * 4);
  l.total = off;
  return l;
}

PrefillLayout prefill_layout(int B, int H, int64_t max_kv_rows) {
  PrefillLayout l{};
  l.kv_rows = (int64_t)kPfRows * ((max_kv_rows + kPfRows - 1) / kPfRows + B);
  size_t off = 0;
  l.kv_row0 = off;  off = align256(off + sizeof(int64_t) * ((size_t)B + 1));
  l.qb_start = off; off = align256(off + sizeof(int32_t) * ((size_t)B + 1));
  l.lenc = off;     off = align256(off + sizeof(int32_t) * (size_t)B);
  l.nq = off;       off = align256(off + sizeof(int32_t) * (size_t)B);
  l.k = off;        off = align256(off + (size_t)H * l.kv_rows * (128 + MLA_D_R) * 2);
  l.v = off;        off = align256(off + (size_t)H * l.kv_rows * 128 * 2);
  l.total = off;
  return l;
}

}  // namespace mla

using namespace mla;

static bool valid_dtype(int d) {
  return d == MLA_DTYPE_F32 || d == MLA_DTYPE_BF16 || d == MLA_DTYPE_FP8_E4M3 ||
         d == MLA_DTYPE_FP6_E2M3_MX;
}

// supported (cache, activation) dtype pairs
static bool supported_pair(int cache, int act) {
  return (cache == MLA_DTYPE_F32 && act == MLA_DTYPE_F32) ||
         (cache == MLA_DTYPE_BF16 && act == MLA_DTYPE_BF16) ||
         (cache == MLA_DTYPE_FP8_E4M3 && act == MLA_DTYPE_BF16) ||
         (cache == MLA_DTYPE_FP6_E2M3_MX && act == MLA_DTYPE_BF16);
}

static int cache_type(int dtype) {
  return dtype == MLA_DTYPE_F32 ? kF32 : dtype == MLA_DTYPE_BF16 ? kBF16
       : dtype == MLA_DTYPE_FP8_E4M3 ? kFP8 : kFP6;
}

// The cache as the launchers see it: contiguous per-sequence row ranges
// (seq_start, seq_cap) or a page pool with a block table.
struct CacheView {
  int32_t dtype;
  int32_t num_seqs;
  void* rows;
  float* row_scale;
  const int64_t* seq_start;      // contiguous
  const int32_t* seq_cap;        // contiguous
  int64_t total_rows;
  const int32_t* block_table;    // paged ([B][max_pages]), else null
  int32_t page_tokens;
  int32_t max_pages;
  int64_t total_pages;
};

static mla_status_t check_common(int32_t dtype, int32_t d_c, int32_t d_r, int32_t num_seqs,
                                 const void* rows, const float* row_scale) {
  if (!valid_dtype(dtype)) return MLA_ERR_INVALID_ARGUMENT;
  if (d_c != MLA_D_C || d_r != MLA_D_R) return MLA_ERR_INVALID_ARGUMENT;
  if (num_seqs < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (num_seqs > kMaxSeqs) return MLA_ERR_UNSUPPORTED;
  if (!rows) return MLA_ERR_INVALID_ARGUMENT;
  if (dtype == MLA_DTYPE_FP8_E4M3 && !row_scale) return MLA_ERR_INVALID_ARGUMENT;
  if (dtype == MLA_DTYPE_FP6_E2M3_MX && row_scale) return MLA_ERR_INVALID_ARGUMENT;  // scales are in the rows
  return MLA_OK;
}

static mla_status_t view_of(const mla_cache_t* c, CacheView& v) {
  if (!c) return MLA_ERR_INVALID_ARGUMENT;
  const mla_status_t st = check_common(c->dtype, c->d_c, c->d_r, c->num_seqs, c->rows, c->row_scale);
  if (st != MLA_OK) return st;
  if (c->total_rows < 1 || !c->seq_start || !c->seq_capacity) return MLA_ERR_INVALID_ARGUMENT;
  v = CacheView{};
  v.dtype = c->dtype;
  v.num_seqs = c->num_seqs;
  v.rows = c->rows;
  v.row_scale = c->row_scale;
  v.seq_start = c->seq_start;
  v.seq_cap = c->seq_capacity;
  v.total_rows = c->total_rows;
  return MLA_OK;
}

static mla_status_t view_of(const mla_paged_cache_t* c, CacheView& v) {
  if (!c) return MLA_ERR_INVALID_ARGUMENT;
  const mla_status_t st = check_common(c->dtype, c->d_c, c->d_r, c->num_seqs, c->rows, c->row_scale);
  if (st != MLA_OK) return st;
  if (!c->block_table || c->max_pages < 1 || c->total_pages < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (c->page_tokens < 32 || c->page_tokens % 32 != 0) return MLA_ERR_INVALID_ARGUMENT;
  // positions and lengths are int32: a sequence's capacity must fit
  if ((int64_t)c->max_pages * c->page_tokens > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (c->total_pages > INT64_MAX / c->page_tokens) return MLA_ERR_INVALID_ARGUMENT;
  v = CacheView{};
  v.dtype = c->dtype;
  v.num_seqs = c->num_seqs;
  v.rows = c->rows;
  v.row_scale = c->row_scale;
  v.total_rows = c->total_pages * c->page_tokens;
  v.block_table = c->block_table;
  v.page_tokens = c->page_tokens;
  v.max_pages = c->max_pages;
  v.total_pages = c->total_pages;
  return MLA_OK;
}

// ---------------------------------------------------------------- MLA_DEBUG
// With MLA_DEBUG=1 in the environment, the entry points also check the
// device-resident contract before launching: every length in [1, capacity],
// every appended token's sequence in [0, B) and position in [0, capacity),
// every sequence's rows inside the cache. The arrays come to the host on the
// caller's stream, which is synchronised (the only synchronisation the
// library ever does); a violation returns MLA_ERR_INVALID_ARGUMENT and
// nothing runs. Without it such values are clamped or skipped as documented.
static bool debug_mode() {
  const char* v = getenv("MLA_DEBUG");
  return v && v[0] == '1' && v[1] == 0;
}

template <typename T>
static bool to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t s) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s) != hipSuccess) return false;
  return hipStreamSynchronize(s) == hipSuccess;
}

// Each sequence's capacity (and, contiguous, its rows inside the cache;
// paged, every table entry a call can use inside the pool: all of them when
// `len` is null, else those of the first ceil(len / P) blocks).
static mla_status_t debug_capacity(const CacheView& c, const std::vector<int32_t>* len,
                                   std::vector<int32_t>& cap, hipStream_t s) {
  const int B = c.num_seqs;
  if (c.block_table) {
    std::vector<int32_t> tab;
    if (!to_host(tab, c.block_table, (size_t)B * c.max_pages, s)) return MLA_ERR_HIP;
    cap.assign(B, c.max_pages * c.page_tokens);
    for (int b = 0; b < B; ++b) {
      const int64_t used = len ? ((int64_t)(*len)[b] + c.page_tokens - 1) / c.page_tokens : c.max_pages;
      for (int64_t j = 0; j < used && j < c.max_pages; ++j) {
        const int32_t pg = tab[(size_t)b * c.max_pages + j];
        if (pg < 0 || pg >= c.total_pages) return MLA_ERR_INVALID_ARGUMENT;
      }
    }
    return MLA_OK;
  }
  std::vector<int64_t> start;
  if (!to_host(start, c.seq_start, B, s) || !to_host(cap, c.seq_cap, B, s)) return MLA_ERR_HIP;
  for (int b = 0; b < B; ++b)
    if (start[b] < 0 || cap[b] < 0 || start[b] + cap[b] > c.total_rows) return MLA_ERR_INVALID_ARGUMENT;
  return MLA_OK;
}

// the cache's rows and the lengths; MLA_ERR_HIP if a copy fails
static mla_status_t debug_check_decode(const CacheView& c, const int32_t* seq_len, hipStream_t s) {
  std::vector<int32_t> cap, len;
  if (!to_host(len, seq_len, c.num_seqs, s)) return MLA_ERR_HIP;
  for (int b = 0; b < c.num_seqs; ++b)
    if (len[b] < 1) return MLA_ERR_INVALID_ARGUMENT;
  const mla_status_t st = debug_capacity(c, &len, cap, s);
  if (st != MLA_OK) return st;
  for (int b = 0; b < c.num_seqs; ++b)
    if (len[b] > cap[b]) return MLA_ERR_INVALID_ARGUMENT;
  return MLA_OK;
}

static mla_status_t debug_check_append(const CacheView& c, const int32_t* tok_seq,
                                       const int32_t* tok_pos, int32_t n_tok, hipStream_t s) {
  std::vector<int32_t> cap, sq, ps;
  mla_status_t st = debug_capacity(c, nullptr, cap, s);
  if (st != MLA_OK) return st;
  if (!to_host(sq, tok_seq, n_tok, s) || !to_host(ps, tok_pos, n_tok, s)) return MLA_ERR_HIP;
  for (int n = 0; n < n_tok; ++n) {
    if (sq[n] < 0 || sq[n] >= c.num_seqs) return MLA_ERR_INVALID_ARGUMENT;
    if (ps[n] < 0 || ps[n] >= cap[sq[n]]) return MLA_ERR_INVALID_ARGUMENT;
  }
  return MLA_OK;
}

extern "C" {

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dtype combination or size";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime or launch error";
  }
  return "unknown status";
}

}  // extern "C"

// YaRN frequencies of the RoPE pairs (the published YaRN method's
// "NTK-by-parts" interpolation, with the constants the discosf explainer's
// "decoupled RoPE and YaRN" section gives): pair i turns
// orig_context * theta_i / (2 pi) times over the original context; pairs with
// at most `alpha` turns run `scale` times slower, pairs with at least `beta`
// keep theta_i, and a linear ramp in the number of turns mixes the two in
// between. fp64, like the plain table.
static void yarn_table(const mla_yarn_t& y, double* inv_freq) {
  const double two_pi = 6.283185307179586;
  for (int i = 0; i < MLA_D_R / 2; ++i) {
    const double theta = pow((double)y.base, -2.0 * i / (double)MLA_D_R);
    const double turns = (double)y.orig_context * theta / two_pi;
    double g = (turns - (double)y.alpha) / ((double)y.beta - (double)y.alpha);
    g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
    inv_freq[i] = (1.0 - g) * theta / (double)y.scale + g * theta;
  }
}

static bool valid_yarn(const mla_yarn_t* y) {
  if (!y) return false;
  auto fin = [](float v) { return isfinite(v) != 0; };
  return fin(y->base) && y->base > 0.f && fin(y->scale) && y->scale >= 1.f && fin(y->alpha) &&
         y->alpha >= 0.f && fin(y->beta) && y->beta > y->alpha && y->orig_context >= 1;
}

// Validate mla_append's arguments and fill `a` (n_tok == 0 is valid and
// leaves nothing to launch). `yarn` NULL: plain RoPE with `rope_base`; else
// YaRN frequencies (its base).
static mla_status_t append_args(const CacheView& cache, const void* h, int32_t n_tok,
                                int32_t d_model, const void* w_dkv, const void* w_kr,
                                mla_dtype_t act_dtype, const int32_t* tok_seq,
                                const int32_t* tok_pos, float rope_base, AppendArgs& a,
                                const mla_yarn_t* yarn = nullptr) {
  if (!valid_dtype(act_dtype)) return MLA_ERR_INVALID_ARGUMENT;
  if (n_tok < 0 || d_model <= 0 || d_model % 64 != 0) return MLA_ERR_INVALID_ARGUMENT;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return MLA_ERR_INVALID_ARGUMENT;
  if (!supported_pair(cache.dtype, act_dtype)) return MLA_ERR_UNSUPPORTED;
  if (n_tok > 0 && (!h || !w_dkv || !w_kr || !tok_seq || !tok_pos)) return MLA_ERR_INVALID_ARGUMENT;
  a = AppendArgs{};
  a.rows = cache.rows;
  a.row_scale = cache.row_scale;
  a.seq_start = cache.seq_start;
  a.seq_cap = cache.seq_cap;
  a.num_seqs = cache.num_seqs;
  a.block_table = cache.block_table;
  a.page_tokens = cache.page_tokens;
  a.max_pages = cache.max_pages;
  a.total_pages = cache.total_pages;
  a.h = h;
  a.w_dkv = w_dkv;
  a.w_kr = w_kr;
  a.tok_seq = tok_seq;
  a.tok_pos = tok_pos;
  a.n_tok = n_tok;
  a.d_model = d_model;
  if (yarn) {
    yarn_table(*yarn, a.inv_freq);
  } else {
    for (int i = 0; i < MLA_D_R / 2; ++i)
      a.inv_freq[i] = pow((double)rope_base, -2.0 * i / (double)MLA_D_R);
  }
  return MLA_OK;
}

// append through any cache view (YaRN table when `yarn` is given)
static mla_status_t append_impl(const CacheView& cv, const void* h, int32_t n_tok,
                                int32_t d_model, const void* w_dkv, const void* w_kr,
                                mla_dtype_t act_dtype, const int32_t* tok_seq,
                                const int32_t* tok_pos, float rope_base, const mla_yarn_t* yarn,
                                void* stream) {
  AppendArgs a;
  const mla_status_t st = append_args(cv, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq,
                                      tok_pos, rope_base, a, yarn);
  if (st != MLA_OK || n_tok == 0) return st;
  if (debug_mode()) {
    const mla_status_t ds = debug_check_append(cv, tok_seq, tok_pos, n_tok, (hipStream_t)stream);
    if (ds != MLA_OK) return ds;
  }
  hipError_t e = launch_append(cache_type(cv.dtype), a, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" {

mla_status_t mla_append(const mla_cache_t* cache, const void* h, int32_t n_tok, int32_t d_model,
                        const void* w_dkv, const void* w_kr, mla_dtype_t act_dtype,
                        const int32_t* tok_seq, const int32_t* tok_pos, float rope_base,
                        void* stream) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  return append_impl(cv, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq, tok_pos, rope_base,
                     nullptr, stream);
}

mla_status_t mla_append_yarn(const mla_cache_t* cache, const void* h, int32_t n_tok,
                             int32_t d_model, const void* w_dkv, const void* w_kr,
                             mla_dtype_t act_dtype, const int32_t* tok_seq,
                             const int32_t* tok_pos, const mla_yarn_t* rope, void* stream) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  if (!valid_yarn(rope)) return MLA_ERR_INVALID_ARGUMENT;
  return append_impl(cv, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq, tok_pos, rope->base,
                     rope, stream);
}

mla_status_t mla_append_paged(const mla_paged_cache_t* cache, const void* h, int32_t n_tok,
                              int32_t d_model, const void* w_dkv, const void* w_kr,
                              mla_dtype_t act_dtype, const int32_t* tok_seq,
                              const int32_t* tok_pos, float rope_base, void* stream) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  return append_impl(cv, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq, tok_pos, rope_base,
                     nullptr, stream);
}

mla_status_t mla_append_yarn_paged(const mla_paged_cache_t* cache, const void* h, int32_t n_tok,
                                   int32_t d_model, const void* w_dkv, const void* w_kr,
                                   mla_dtype_t act_dtype, const int32_t* tok_seq,
                                   const int32_t* tok_pos, const mla_yarn_t* rope, void* stream) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  if (!valid_yarn(rope)) return MLA_ERR_INVALID_ARGUMENT;
  return append_impl(cv, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq, tok_pos, rope->base,
                     rope, stream);
}

float mla_yarn_softmax_factor(float scale) {
  if (!(scale > 1.f) || !isfinite(scale)) return 1.f;
  const double m = 0.1 * log((double)scale) + 1.0;
  return (float)(m * m);
}

mla_status_t mla_decode_workspace_size(int32_t num_seqs, int32_t n_heads, mla_dtype_t cache_dtype,
                                       mla_dtype_t act_dtype, size_t* bytes) {
  if (!bytes) return MLA_ERR_INVALID_ARGUMENT;
  if (num_seqs < 1 || n_heads < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(cache_dtype) || !valid_dtype(act_dtype)) return MLA_ERR_INVALID_ARGUMENT;
  if (!supported_pair(cache_dtype, act_dtype)) return MLA_ERR_UNSUPPORTED;
  if (n_heads % 16 != 0 || n_heads > kMaxHeads || num_seqs > kMaxSeqs) return MLA_ERR_UNSUPPORTED;
  *bytes = workspace_layout(cache_type(cache_dtype), num_seqs, n_heads).total;
  return MLA_OK;
}

}  // extern "C"

// Validate mla_decode's arguments and fill `a` and the launch plan.
static mla_status_t decode_args(const CacheView& cache, const int32_t* seq_len,
                                const void* q_nope, const void* q_pe, const void* w_uk,
                                const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                                float softmax_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, DecodeArgs& a, DecodePlan& plan) {
  if (!valid_dtype(act_dtype)) return MLA_ERR_INVALID_ARGUMENT;
  if (!seq_len || !q_nope || !q_pe || !w_uk || !w_uv || !out || !workspace)
    return MLA_ERR_INVALID_ARGUMENT;
  if (n_heads < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)workspace & 255) != 0) return MLA_ERR_INVALID_ARGUMENT;
  if (!supported_pair(cache.dtype, act_dtype)) return MLA_ERR_UNSUPPORTED;
  if (n_heads % 16 != 0 || n_heads > kMaxHeads) return MLA_ERR_UNSUPPORTED;
  const int ct = cache_type(cache.dtype);
  const int B = cache.num_seqs;
  const WorkspaceLayout wl = workspace_layout(ct, B, n_heads);
  if (workspace_bytes < wl.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

  char* ws = (char*)workspace;
  a = DecodeArgs{};
  a.rows = cache.rows;
  a.row_scale = cache.row_scale;
  a.seq_start = cache.seq_start;
  a.seq_cap = cache.seq_cap;
  a.block_table = cache.block_table;
  a.page_tokens = cache.page_tokens;
  a.max_pages = cache.max_pages;
  a.total_pages = cache.total_pages;
  a.seq_len = seq_len;
  a.B = B;
  a.H = n_heads;
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.lse = lse;
  a.softmax_scale = softmax_scale;
  a.seqinfo = (SeqInfo*)(ws + wl.seqinfo);
  a.starts = (int64_t*)(ws + wl.starts);
  a.wseq = (int32_t*)(ws + wl.wseq);
  a.winfo = (WorkerInfo*)(ws + wl.winfo);
  a.wfirst = (int32_t*)(ws + wl.wfirst);
  a.wlast = (int32_t*)(ws + wl.wlast);
  a.q_lat = ws + wl.q_lat;
  a.part_o = (void*)(ws + wl.part_o);
  a.part_ml = (float*)(ws + wl.part_ml);
  plan = make_plan(ct, B, n_heads);
  return MLA_OK;
}

static mla_status_t decode_view(const CacheView& cv, const int32_t* seq_len, const void* q_nope,
                                const void* q_pe, const void* w_uk, const void* w_uv,
                                mla_dtype_t act_dtype, int32_t n_heads, float softmax_scale,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream, int stage) {
  DecodeArgs a;
  DecodePlan plan;
  const mla_status_t st = decode_args(cv, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads,
                                      softmax_scale, out, lse, workspace, workspace_bytes, a, plan);
  if (st != MLA_OK) return st;
  if (debug_mode()) {
    const mla_status_t ds = debug_check_decode(cv, seq_len, (hipStream_t)stream);
    if (ds != MLA_OK) return ds;
  }
  hipError_t e = launch_decode(cache_type(cv.dtype), plan, a, (hipStream_t)stream, stage);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

static mla_status_t decode_impl(const mla_cache_t* cache, const int32_t* seq_len,
                                const void* q_nope, const void* q_pe, const void* w_uk,
                                const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                                float softmax_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream, int stage) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  return decode_view(cv, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads, softmax_scale, out,
                     lse, workspace, workspace_bytes, stream, stage);
}

#define MLA_DECODE_ENTRY(NAME, STAGE)                                                        \
  mla_status_t NAME(const mla_cache_t* cache, const int32_t* seq_len, const void* q_nope,  \
                    const void* q_pe, const void* w_uk, const void* w_uv,                   \
                    mla_dtype_t act_dtype, int32_t n_heads, float softmax_scale, void* out, \
                    float* lse, void* workspace, size_t workspace_bytes, void* stream) {    \
    return decode_impl(cache, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads,        \
                       softmax_scale, out, lse, workspace, workspace_bytes, stream, STAGE); \
  }

extern "C" {

MLA_DECODE_ENTRY(mla_decode, 0)
MLA_DECODE_ENTRY(mla_decode_absorb, 1)
MLA_DECODE_ENTRY(mla_decode_attend, 2)
MLA_DECODE_ENTRY(mla_decode_combine, 3)
MLA_DECODE_ENTRY(mla_decode_attend_combine, 4)

mla_status_t mla_decode_paged(const mla_paged_cache_t* cache, const int32_t* seq_len,
                              const void* q_nope, const void* q_pe, const void* w_uk,
                              const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                              float softmax_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  return decode_view(cv, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads, softmax_scale, out,
                     lse, workspace, workspace_bytes, stream, 0);
}

mla_status_t mla_append_absorb(const mla_cache_t* cache, const void* h, int32_t n_tok,
                               int32_t d_model, const void* w_dkv, const void* w_kr,
                               const int32_t* tok_seq, const int32_t* tok_pos, float rope_base,
                               const int32_t* seq_len, const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                               int32_t n_heads, float softmax_scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  CacheView cv;
  mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  AppendArgs aa;
  st = append_args(cv, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq, tok_pos, rope_base, aa);
  if (st != MLA_OK) return st;
  DecodeArgs da;
  DecodePlan plan;
  st = decode_args(cv, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads, softmax_scale, out,
                   lse, workspace, workspace_bytes, da, plan);
  if (st != MLA_OK) return st;
  if (debug_mode()) {
    mla_status_t ds = n_tok > 0 ? debug_check_append(cv, tok_seq, tok_pos, n_tok, (hipStream_t)stream)
                                : MLA_OK;
    if (ds == MLA_OK) ds = debug_check_decode(cv, seq_len, (hipStream_t)stream);
    if (ds != MLA_OK) return ds;
  }
  const int ct = cache_type(cv.dtype);
  hipError_t e;
  if (n_tok > 0 && append_absorb_fits(ct, aa, da)) {
    e = launch_append_absorb(aa, plan, da, (hipStream_t)stream);
  } else {
    e = n_tok > 0 ? launch_append(ct, aa, (hipStream_t)stream) : hipSuccess;
    if (e == hipSuccess) e = launch_decode(ct, plan, da, (hipStream_t)stream, 1);
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------- prefill
// Largest workspace row bound and query count the launches can index.
static constexpr int64_t kMaxPrefillRows = (int64_t)1 << 31;

static mla_status_t prefill_shape(int32_t num_seqs, int32_t n_heads, int64_t n_q,
                                  int64_t max_kv_rows) {
  if (num_seqs < 1 || n_heads < 1 || n_q < 0 || max_kv_rows < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (num_seqs > kMaxSeqs || n_heads > kMaxHeads) return MLA_ERR_UNSUPPORTED;
  if (n_q > INT32_MAX || max_kv_rows > kMaxPrefillRows) return MLA_ERR_UNSUPPORTED;
  // attention grid: heads x (query blocks + sequences), rounded to 8
  const int64_t items = (int64_t)n_heads * ((n_q + kPfQ - 1) / kPfQ + num_seqs);
  if (items + 8 > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

extern "C" {

mla_status_t mla_prefill_workspace_size(int32_t num_seqs, int32_t n_heads, int64_t n_q,
                                        int64_t max_kv_rows, size_t* bytes) {
  if (!bytes) return MLA_ERR_INVALID_ARGUMENT;
  const mla_status_t st = prefill_shape(num_seqs, n_heads, n_q, max_kv_rows);
  if (st != MLA_OK) return st;
  *bytes = prefill_layout(num_seqs, n_heads, max_kv_rows).total;
  return MLA_OK;
}

}  // extern "C"

// MLA_DEBUG: lengths in [0, capacity], q_start non-decreasing from 0 to n_q,
// every sequence's queries at most its length, the padded rows within the
// bound, rows inside the cache
static mla_status_t debug_check_prefill(const CacheView& c, const int32_t* seq_len,
                                        const int32_t* q_start, int64_t n_q, int64_t max_kv_rows,
                                        hipStream_t s) {
  std::vector<int32_t> cap, len, qs;
  const mla_status_t st = debug_capacity(c, nullptr, cap, s);
  if (st != MLA_OK) return st;
  if (!to_host(len, seq_len, c.num_seqs, s) || !to_host(qs, q_start, (size_t)c.num_seqs + 1, s))
    return MLA_ERR_HIP;
  if (qs[0] != 0 || qs[c.num_seqs] != n_q) return MLA_ERR_INVALID_ARGUMENT;
  int64_t rows = 0;
  for (int b = 0; b < c.num_seqs; ++b) {
    if (len[b] < 0 || len[b] > cap[b]) return MLA_ERR_INVALID_ARGUMENT;
    if (qs[b + 1] < qs[b] || qs[b + 1] - qs[b] > len[b]) return MLA_ERR_INVALID_ARGUMENT;
    rows += len[b];
  }
  if (rows > max_kv_rows) return MLA_ERR_INVALID_ARGUMENT;
  return MLA_OK;
}

static mla_status_t prefill_view(const CacheView& cv, const int32_t* seq_len,
                                 const int32_t* q_start, int64_t n_q, int64_t max_kv_rows,
                                 const void* q_nope, const void* q_pe, const void* w_uk,
                                 const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                                 float softmax_scale, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!valid_dtype(act_dtype)) return MLA_ERR_INVALID_ARGUMENT;
  mla_status_t st = prefill_shape(cv.num_seqs, n_heads, n_q, max_kv_rows);
  if (st != MLA_OK) return st;
  if (!seq_len || !q_start || !q_nope || !q_pe || !w_uk || !w_uv || !out || !workspace)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)workspace & 255) != 0) return MLA_ERR_INVALID_ARGUMENT;
  if (act_dtype != MLA_DTYPE_BF16 ||
      (cv.dtype != MLA_DTYPE_BF16 && cv.dtype != MLA_DTYPE_FP8_E4M3 &&
       cv.dtype != MLA_DTYPE_FP6_E2M3_MX))
    return MLA_ERR_UNSUPPORTED;
  const PrefillLayout wl = prefill_layout(cv.num_seqs, n_heads, max_kv_rows);
  if (workspace_bytes < wl.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (debug_mode()) {
    const mla_status_t ds = debug_check_prefill(cv, seq_len, q_start, n_q, max_kv_rows,
                                                (hipStream_t)stream);
    if (ds != MLA_OK) return ds;
  }
  char* ws = (char*)workspace;
  PrefillArgs a{};
  a.rows = cv.rows;
  a.row_scale = cv.row_scale;
  a.seq_start = cv.seq_start;
  a.seq_cap = cv.seq_cap;
  a.block_table = cv.block_table;
  a.max_pages = cv.max_pages;
  a.page_tokens = cv.page_tokens;
  a.page_limit = (uint32_t)(cv.total_pages < (int64_t)1 << 31 ? cv.total_pages : (int64_t)1 << 31);
  a.seq_len = seq_len;
  a.q_start = q_start;
  a.n_q = n_q;
  a.kv_rows = wl.kv_rows;
  a.B = cv.num_seqs;
  a.H = n_heads;
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.lse = lse;
  a.softmax_scale = softmax_scale;
  a.kv_row0 = (int64_t*)(ws + wl.kv_row0);
  a.qb_start = (int32_t*)(ws + wl.qb_start);
  a.lenc = (int32_t*)(ws + wl.lenc);
  a.nq = (int32_t*)(ws + wl.nq);
  a.k = ws + wl.k;
  a.v = ws + wl.v;
  const hipError_t e = launch_prefill(cache_type(cv.dtype), a, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" {

mla_status_t mla_prefill(const mla_cache_t* cache, const int32_t* seq_len, const int32_t* q_start,
                         int64_t n_q, int64_t max_kv_rows, const void* q_nope, const void* q_pe,
                         const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                         int32_t n_heads, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  return prefill_view(cv, seq_len, q_start, n_q, max_kv_rows, q_nope, q_pe, w_uk, w_uv, act_dtype,
                      n_heads, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

mla_status_t mla_prefill_paged(const mla_paged_cache_t* cache, const int32_t* seq_len,
                               const int32_t* q_start, int64_t n_q, int64_t max_kv_rows,
                               const void* q_nope, const void* q_pe, const void* w_uk,
                               const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                               float softmax_scale, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  CacheView cv;
  const mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  return prefill_view(cv, seq_len, q_start, n_q, max_kv_rows, q_nope, q_pe, w_uk, w_uv, act_dtype,
                      n_heads, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// mla_decode_noalloc: mla_decode with the workspace in a file-scope device
// array instead of caller memory, for callers that cannot allocate.
//
// Each device the library runs on holds its own copy of `scratch` from module
// load until the process ends. In host code `scratch` names only a host-side
// stand-in: its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_WORKSPACE_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's `scratch` (nullptr on failure).
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

extern "C" {

mla_status_t mla_decode_noalloc(const mla_cache_t* cache, const int32_t* seq_len,
                                const void* q_nope, const void* q_pe, const void* w_uk,
                                const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                                float softmax_scale, void* out, float* lse, void* stream) {
  // every host-side check, the workspace size included, before any HIP call:
  // a fake non-null workspace stands in until the real address is known
  CacheView cv;
  mla_status_t st = view_of(cache, cv);
  if (st != MLA_OK) return st;
  DecodeArgs a;
  DecodePlan plan;
  st = decode_args(cv, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads,
                                softmax_scale, out, lse, (void*)(uintptr_t)256,
                                MLA_NOALLOC_WORKSPACE_BYTES, a, plan);
  if (st != MLA_OK) return st;
  void* ws = scratch_address();
  if (!ws) return MLA_ERR_HIP;
  // the workspace needs no clearing: absorb writes everything the later
  // stages read
  return decode_impl(cache, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads, softmax_scale,
                     out, lse, ws, MLA_NOALLOC_WORKSPACE_BYTES, stream, 0);
}

}  // extern "C"
