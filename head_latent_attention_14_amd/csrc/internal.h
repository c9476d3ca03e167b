// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

enum CacheType : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kFP6 = 3 };

constexpr int kTargetCUs = 256;   // MI355X compute units

// ---------------------------------------------------------------- append
struct AppendArgs {
  void* rows;                 // [total_rows][576] cache storage
  float* row_scale;           // [total_rows] (fp8 only)
  const int64_t* seq_start;   // [B]
  const int32_t* seq_cap;     // [B]
  int32_t num_seqs;
  const void* h;              // [n_tok][d_model]
  const void* w_dkv;          // [512][d_model]
  const void* w_kr;           // [64][d_model]
  const int32_t* tok_seq;     // [n_tok]
  const int32_t* tok_pos;     // [n_tok]
  int32_t n_tok;
  int32_t d_model;
  double inv_freq[32];        // rope_base^(-2i/64), fp64
  // paged cache (block_table non-null): token t of sequence b is row
  // block_table[b][t / page_tokens] * page_tokens + t % page_tokens;
  // seq_start and seq_cap are unused
  const int32_t* block_table; // [B][max_pages]
  int32_t page_tokens;
  int32_t max_pages;
  int64_t total_pages;
};
hipError_t launch_append(int cache_type, const AppendArgs& a, hipStream_t s);

// ---------------------------------------------------------------- decode
// Per-sequence record of the work plan (written by the absorb launch, read by
// the attention kernels). Work is split in tiles: the sequences' tiles form
// one stream in which each non-empty sequence also counts one unit for the
// cost of starting it; sequence b's ceil(len / tile) real tiles, the last one
// possibly partial, are [tile0, tile1) of that stream.
struct SeqInfo {
  int64_t row0;     // cache row of the sequence's first token
  int32_t len;      // length clamped to [0, capacity]
  int32_t tile0;    // first real tile
  int32_t tile1;    // one past the last tile
  int32_t next;     // next sequence that has tiles (B: none)
  int32_t pad[2];
};
static_assert(sizeof(SeqInfo) == 32, "one 32-byte record per sequence");

// Per-worker record of the work plan: where worker w starts, so that a
// workgroup knows its first tile from one 32-byte load.
struct WorkerInfo {
  int64_t row0;     // cache row of the worker's first token
  int32_t b;        // its first sequence (-1: the worker has no tiles)
  int32_t t;        // first token, local to that sequence
  int32_t t_end;    // end of the first segment (local token)
  int32_t next;     // next sequence with tiles after b (B: none)
  int32_t r_hi;     // one past the worker's last tile
  int32_t pad;
};
static_assert(sizeof(WorkerInfo) == 32, "one 32-byte record per worker");

// Launch plan: fixed by (cache type, B, H) so that the workspace size can be
// computed on the host without seeing the device-resident lengths.
struct DecodePlan {
  bool pair;     // pair kernel (two waves per 32 heads) instead of the block kernel
  bool stream;   // streaming kernel (one copy wave + four compute waves per 16 heads)
  bool h32;      // 128-head kernel (four waves of 32 heads, one per SIMD)
  bool f8;       // pair kernel over an fp8 cache: fp8 MFMA for both contractions
  int np;        // pair kernel: 32-head pairs per workgroup
  int hb;        // block kernel: 16-head blocks per workgroup
  int ds;        // block kernel: value-dimension splits per head block
  int nstage;    // cache tiles in flight per workgroup (LDS ring depth)
  int tile;      // tokens per tile of the kernel (the unit of the work split)
  int seg_tiles; // tiles of work the split counts for starting a sequence segment
  int workers;   // W: tile ranges of the stream of all sequences' tiles
  int head_groups;  // workgroups sharing one token range (H / heads per workgroup)
  int64_t nslot;    // partial-result slots: W + B
};
DecodePlan make_plan(int cache_type, int B, int H);

struct WorkspaceLayout {
  size_t seqinfo;    // SeqInfo [B]
  size_t starts;     // int64 [W+1] first tile of each worker (and the tile count)
  size_t wseq;       // int32 [W] first sequence of each worker
  size_t winfo;      // WorkerInfo [W]
  size_t wfirst;     // int32 [B] first worker of each sequence
  size_t wlast;      // int32 [B] last worker of each sequence (-1 if empty)
  size_t q_lat;      // [B][H][512] bf16 (f32 for the f32 path)
  size_t part_o;     // [nslot][H][512] normalised partial outputs: f32 (f32 path) or bf16
  size_t part_ml;    // f32 [nslot][H][2] running max (log2 domain) and sum
  size_t total;
};
WorkspaceLayout workspace_layout(int cache_type, int B, int H);

struct DecodeArgs {
  // cache
  const void* rows;
  const float* row_scale;
  const int64_t* seq_start;
  const int32_t* seq_cap;
  const int32_t* seq_len;
  // paged cache (block_table non-null; seq_start/seq_cap unused), as in AppendArgs
  const int32_t* block_table;
  int32_t page_tokens;
  int32_t max_pages;
  int64_t total_pages;
  int32_t B;
  int32_t H;
  // activations / weights (bf16 or f32)
  const void* q_nope;
  const void* q_pe;
  const void* w_uk;
  const void* w_uv;
  void* out;
  float* lse;
  float softmax_scale;
  // workspace views
  SeqInfo* seqinfo;
  int64_t* starts;
  int32_t* wseq;
  WorkerInfo* winfo;
  int32_t* wfirst;
  int32_t* wlast;
  void* q_lat;
  void* part_o;
  float* part_ml;
};
// stage: 1 = absorb (+ work plan), 2 = attention, 3 = merge + W_UV,
// 4 = attention then merge + W_UV, 0 = all three
hipError_t launch_decode(int cache_type, const DecodePlan& plan, const DecodeArgs& a,
                         hipStream_t s, int stage);

// Append and the absorb stage of the following decode in one launch (bf16
// cache, and a grid that fits the CUs at once: append_absorb_fits).
bool append_absorb_fits(int cache_type, const AppendArgs& a, const DecodeArgs& d);
hipError_t launch_append_absorb(const AppendArgs& a, const DecodePlan& plan, const DecodeArgs& d,
                                hipStream_t s);

// ---------------------------------------------------------------- prefill
// Causal multi-query attention: the queries of sequence b are its last n_b
// positions. Three launches: a one-workgroup plan (prefix sums), the
// up-projection of every cached row to per-head K (128, followed by a copy of
// the row's 64-wide RoPE key) and V (128), and the attention over query blocks.
constexpr int kPfRows = 128;      // cached rows per up-projection workgroup (and K/V padding)
constexpr int kPfQ = 256;         // queries per attention workgroup (8 waves of 32)
constexpr int kPfKV = 64;         // cached rows per attention step

struct PrefillLayout {
  int64_t kv_rows;   // rows of the K/V buffers: kPfRows * (ceil(max_kv_rows / kPfRows) + B)
  size_t kv_row0;    // int64 [B+1] first packed K/V row of each sequence (multiples of kPfRows)
  size_t qb_start;   // int32 [B+1] first query block of each sequence
  size_t lenc;       // int32 [B] length clamped to [0, capacity] (0: not served)
  size_t nq;         // int32 [B] queries of each sequence (clamped to [0, length])
  size_t k;          // bf16 [H][kv_rows][192] K: 128 up-projected dims, then the RoPE key
  size_t v;          // bf16 [H][kv_rows][128]
  size_t total;
};
PrefillLayout prefill_layout(int B, int H, int64_t max_kv_rows);

struct PrefillArgs {
  const void* rows;           // cache storage (contiguous rows or the page pool)
  const float* row_scale;     // fp8 only
  const int64_t* seq_start;   // [B] (contiguous)
  const int32_t* seq_cap;     // [B] (contiguous)
  const int32_t* block_table; // [B][max_pages] (paged; null: contiguous)
  int32_t max_pages;
  int32_t page_tokens;
  uint32_t page_limit;        // pages in the pool, at most 2^31
  const int32_t* seq_len;     // [B]
  const int32_t* q_start;     // [B+1]
  int64_t n_q;
  int64_t kv_rows;            // PrefillLayout::kv_rows
  int32_t B;
  int32_t H;
  const void* q_nope;         // [n_q][H][128] bf16
  const void* q_pe;           // [n_q][H][64] bf16
  const void* w_uk;           // [H][128][512] bf16
  const void* w_uv;           // [H][512][128] bf16
  void* out;                  // [n_q][H][128] bf16
  float* lse;                 // [n_q][H] or null
  float softmax_scale;
  // workspace views
  int64_t* kv_row0;
  int32_t* qb_start;
  int32_t* lenc;
  int32_t* nq;
  void* k;
  void* v;
};
hipError_t launch_prefill(int cache_type, const PrefillArgs& a, hipStream_t s);

}  // namespace mla
