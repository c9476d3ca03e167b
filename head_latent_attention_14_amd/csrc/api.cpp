// C ABI of libmla: argument validation, launch planning, workspace layout
// and launch sequencing on the caller's stream. No call here allocates,
// synchronises or keeps state; every check runs before the first HIP call.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/libmla.h"
#include "internal.h"

#include <stdlib.h>
#include <vector>

namespace mla {

static constexpr int kMaxHeads = 1024;
static constexpr int kMaxSeqs = 1 << 20;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodePlan make_plan(int ct, int B, int H) {
  DecodePlan p{};
  if (ct != kF32 && H % 32 == 0) {
    // pair kernel: up to 128 heads (8 waves) per workgroup; the ring depth is
    // what fits in LDS beside the score-exchange buffer
    p.pair = true;
    p.np = (H % 128 == 0) ? 4 : (H % 64 == 0) ? 2 : 1;
    p.nstage = (ct == kFP8 || p.np == 1) ? 4 : 3;
    p.head_groups = H / (32 * p.np);
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
  p.seg_tiles = p.pair ? 5 : 1;
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

}  // namespace mla

using namespace mla;

static bool valid_dtype(int d) {
  return d == MLA_DTYPE_F32 || d == MLA_DTYPE_BF16 || d == MLA_DTYPE_FP8_E4M3;
}

// supported (cache, activation) dtype pairs
static bool supported_pair(int cache, int act) {
  return (cache == MLA_DTYPE_F32 && act == MLA_DTYPE_F32) ||
         (cache == MLA_DTYPE_BF16 && act == MLA_DTYPE_BF16) ||
         (cache == MLA_DTYPE_FP8_E4M3 && act == MLA_DTYPE_BF16);
}

static int cache_type(int dtype) {
  return dtype == MLA_DTYPE_F32 ? kF32 : (dtype == MLA_DTYPE_BF16 ? kBF16 : kFP8);
}

static mla_status_t check_cache(const mla_cache_t* c) {
  if (!c) return MLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(c->dtype)) return MLA_ERR_INVALID_ARGUMENT;
  if (c->d_c != MLA_D_C || c->d_r != MLA_D_R) return MLA_ERR_INVALID_ARGUMENT;
  if (c->num_seqs < 1 || c->total_rows < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (c->num_seqs > kMaxSeqs) return MLA_ERR_UNSUPPORTED;
  if (!c->rows || !c->seq_start || !c->seq_capacity) return MLA_ERR_INVALID_ARGUMENT;
  if (c->dtype == MLA_DTYPE_FP8_E4M3 && !c->row_scale) return MLA_ERR_INVALID_ARGUMENT;
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

// the cache's rows and, when given, the lengths; MLA_ERR_HIP if a copy fails
static mla_status_t debug_check_decode(const mla_cache_t* c, const int32_t* seq_len, hipStream_t s) {
  std::vector<int64_t> start;
  std::vector<int32_t> cap, len;
  if (!to_host(start, c->seq_start, c->num_seqs, s) || !to_host(cap, c->seq_capacity, c->num_seqs, s))
    return MLA_ERR_HIP;
  if (seq_len && !to_host(len, seq_len, c->num_seqs, s)) return MLA_ERR_HIP;
  for (int b = 0; b < c->num_seqs; ++b) {
    if (start[b] < 0 || cap[b] < 0 || start[b] + cap[b] > c->total_rows) return MLA_ERR_INVALID_ARGUMENT;
    if (seq_len && (len[b] < 1 || len[b] > cap[b])) return MLA_ERR_INVALID_ARGUMENT;
  }
  return MLA_OK;
}

static mla_status_t debug_check_append(const mla_cache_t* c, const int32_t* tok_seq,
                                       const int32_t* tok_pos, int32_t n_tok, hipStream_t s) {
  mla_status_t st = debug_check_decode(c, nullptr, s);
  if (st != MLA_OK) return st;
  std::vector<int32_t> cap, sq, ps;
  if (!to_host(cap, c->seq_capacity, c->num_seqs, s) || !to_host(sq, tok_seq, n_tok, s) ||
      !to_host(ps, tok_pos, n_tok, s))
    return MLA_ERR_HIP;
  for (int n = 0; n < n_tok; ++n) {
    if (sq[n] < 0 || sq[n] >= c->num_seqs) return MLA_ERR_INVALID_ARGUMENT;
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

// Validate mla_append's arguments and fill `a` (n_tok == 0 is valid and
// leaves nothing to launch).
static mla_status_t append_args(const mla_cache_t* cache, const void* h, int32_t n_tok,
                                int32_t d_model, const void* w_dkv, const void* w_kr,
                                mla_dtype_t act_dtype, const int32_t* tok_seq,
                                const int32_t* tok_pos, float rope_base, AppendArgs& a) {
  mla_status_t st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!valid_dtype(act_dtype)) return MLA_ERR_INVALID_ARGUMENT;
  if (n_tok < 0 || d_model <= 0 || d_model % 64 != 0) return MLA_ERR_INVALID_ARGUMENT;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return MLA_ERR_INVALID_ARGUMENT;
  if (!supported_pair(cache->dtype, act_dtype)) return MLA_ERR_UNSUPPORTED;
  if (n_tok > 0 && (!h || !w_dkv || !w_kr || !tok_seq || !tok_pos)) return MLA_ERR_INVALID_ARGUMENT;
  a = AppendArgs{};
  a.rows = cache->rows;
  a.row_scale = cache->row_scale;
  a.seq_start = cache->seq_start;
  a.seq_cap = cache->seq_capacity;
  a.num_seqs = cache->num_seqs;
  a.h = h;
  a.w_dkv = w_dkv;
  a.w_kr = w_kr;
  a.tok_seq = tok_seq;
  a.tok_pos = tok_pos;
  a.n_tok = n_tok;
  a.d_model = d_model;
  for (int i = 0; i < MLA_D_R / 2; ++i)
    a.inv_freq[i] = pow((double)rope_base, -2.0 * i / (double)MLA_D_R);
  return MLA_OK;
}

extern "C" {

mla_status_t mla_append(const mla_cache_t* cache, const void* h, int32_t n_tok, int32_t d_model,
                        const void* w_dkv, const void* w_kr, mla_dtype_t act_dtype,
                        const int32_t* tok_seq, const int32_t* tok_pos, float rope_base,
                        void* stream) {
  AppendArgs a;
  const mla_status_t st = append_args(cache, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq,
                                      tok_pos, rope_base, a);
  if (st != MLA_OK || n_tok == 0) return st;
  if (debug_mode()) {
    const mla_status_t ds = debug_check_append(cache, tok_seq, tok_pos, n_tok, (hipStream_t)stream);
    if (ds != MLA_OK) return ds;
  }
  hipError_t e = launch_append(cache_type(cache->dtype), a, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
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
static mla_status_t decode_args(const mla_cache_t* cache, const int32_t* seq_len,
                                const void* q_nope, const void* q_pe, const void* w_uk,
                                const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                                float softmax_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, DecodeArgs& a, DecodePlan& plan) {
  mla_status_t st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!valid_dtype(act_dtype)) return MLA_ERR_INVALID_ARGUMENT;
  if (!seq_len || !q_nope || !q_pe || !w_uk || !w_uv || !out || !workspace)
    return MLA_ERR_INVALID_ARGUMENT;
  if (n_heads < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)workspace & 255) != 0) return MLA_ERR_INVALID_ARGUMENT;
  if (!supported_pair(cache->dtype, act_dtype)) return MLA_ERR_UNSUPPORTED;
  if (n_heads % 16 != 0 || n_heads > kMaxHeads) return MLA_ERR_UNSUPPORTED;
  const int ct = cache_type(cache->dtype);
  const int B = cache->num_seqs;
  const WorkspaceLayout wl = workspace_layout(ct, B, n_heads);
  if (workspace_bytes < wl.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

  char* ws = (char*)workspace;
  a = DecodeArgs{};
  a.rows = cache->rows;
  a.row_scale = cache->row_scale;
  a.seq_start = cache->seq_start;
  a.seq_cap = cache->seq_capacity;
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

static mla_status_t decode_impl(const mla_cache_t* cache, const int32_t* seq_len,
                                const void* q_nope, const void* q_pe, const void* w_uk,
                                const void* w_uv, mla_dtype_t act_dtype, int32_t n_heads,
                                float softmax_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream, int stage) {
  DecodeArgs a;
  DecodePlan plan;
  const mla_status_t st = decode_args(cache, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads,
                                      softmax_scale, out, lse, workspace, workspace_bytes, a, plan);
  if (st != MLA_OK) return st;
  if (debug_mode()) {
    const mla_status_t ds = debug_check_decode(cache, seq_len, (hipStream_t)stream);
    if (ds != MLA_OK) return ds;
  }
  hipError_t e = launch_decode(cache_type(cache->dtype), plan, a, (hipStream_t)stream, stage);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
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

mla_status_t mla_append_absorb(const mla_cache_t* cache, const void* h, int32_t n_tok,
                               int32_t d_model, const void* w_dkv, const void* w_kr,
                               const int32_t* tok_seq, const int32_t* tok_pos, float rope_base,
                               const int32_t* seq_len, const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv, mla_dtype_t act_dtype,
                               int32_t n_heads, float softmax_scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  AppendArgs aa;
  mla_status_t st = append_args(cache, h, n_tok, d_model, w_dkv, w_kr, act_dtype, tok_seq, tok_pos,
                                rope_base, aa);
  if (st != MLA_OK) return st;
  DecodeArgs da;
  DecodePlan plan;
  st = decode_args(cache, seq_len, q_nope, q_pe, w_uk, w_uv, act_dtype, n_heads, softmax_scale, out,
                   lse, workspace, workspace_bytes, da, plan);
  if (st != MLA_OK) return st;
  if (debug_mode()) {
    mla_status_t ds = n_tok > 0 ? debug_check_append(cache, tok_seq, tok_pos, n_tok, (hipStream_t)stream)
                                : MLA_OK;
    if (ds == MLA_OK) ds = debug_check_decode(cache, seq_len, (hipStream_t)stream);
    if (ds != MLA_OK) return ds;
  }
  const int ct = cache_type(cache->dtype);
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
