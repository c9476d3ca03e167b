// Pieces shared by the attention kernels: kernel parameters, the per-dtype
// tile geometry, the token-range cursor, the asynchronous tile copies and
// the transposing value-operand reads.
#pragma once

#include "common.h"
#include "internal.h"

namespace mla {

struct AttnParams {
  const char* rows;
  const float* row_scale;
  const SeqInfo* seqinfo;    // [B]
  const WorkerInfo* winfo;   // [W]
  const void* q_lat;         // [B][H][512]  bf16 (f32 for the f32 cache)
  const void* q_pe;          // [B][H][64]
  void* part_o;              // [nslot][H][512] o/l: fp32 (f32 cache) or bf16
  float* part_ml;            // [nslot][H][2]
  int32_t B;
  int32_t H;
  float scale_log2;          // softmax_scale * log2(e)
  // paged cache (block_table non-null): a tile never spans two pages
  // (page_tokens is a multiple of the tile); the cursor looks up the next
  // page when it crosses into it
  const int32_t* block_table;  // [B][max_pages]
  int32_t max_pages;
  int32_t page_tokens;
  int32_t page_tiles;          // page_tokens / tile
  uint32_t page_limit;         // min(pool pages, 2^31): a valid entry is below it
};

// Per cache dtype: bytes of a stored row, bytes of a padded LDS row, and
// tokens per tile. Rows in LDS are padded by 16 bytes so that the 16 rows one
// MFMA operand read touches start on different banks; every operand read is
// then a per-lane base plus a compile-time offset.
template <int CT> struct Tr;
template <> struct Tr<kBF16> { static constexpr int kRowBytes = 1152, kPad = 1168, kTile = 32; };
template <> struct Tr<kFP8> { static constexpr int kRowBytes = 576, kPad = 592, kTile = 32; };
template <> struct Tr<kF32> { static constexpr int kRowBytes = 2304, kPad = 2320, kTile = 16; };
// fp6 rows (464 bytes: packed codes, block scales, padding) are only read by
// the widening pass, which needs no padding
template <> struct Tr<kFP6> { static constexpr int kRowBytes = 464, kPad = 464, kTile = 32; };
constexpr int kConvPad = 1168;   // padded bf16 row of the widened fp8 tile
constexpr float kSlack = 8.f;    // lazy-rescale slack of the running max (log2 units)

__device__ __forceinline__ int seqinfo_word(const SeqInfo* si, int b, int lane) {
  return ((const int*)(si + b))[lane & 7];
}

// A worker's position in its tile range: the tile at token t of sequence b.
// The record of the next sequence with tiles is loaded one segment ahead, so
// moving into it needs no memory access on the way. The contiguous kernels
// hold it spread over the lanes (lane l holds its 32-bit word l % 8: one
// VGPR); the paged kernels hold it in scalar registers, loaded with scalar
// loads: there the register allocator moves the record between registers in
// the tile loop, and a move of a VGPR whose vector load may still be pending
// waits for every tile copy in flight, while a scalar load is counted apart
// from the copies.
struct Cursor {
  int b;            // sequence
  int64_t t;        // first token of the tile, local to the sequence
  int64_t t_end;    // end of this worker's segment of the sequence (local)
  int64_t row0;     // cache row of token t
  int nb;           // next sequence with tiles (B: none)
  int nx;           // contiguous kernels: this lane's word of seqinfo[nb]
  int nw[6];        // paged kernels: words 0..5 of seqinfo[nb]
  int page;         // paged cache: block of token t in the sequence's table
  int page_left;    // paged cache: tiles of that page from t on
};

// Load the record of sequence c.nb (which must be below B) into the cursor.
template <bool PAGED>
__device__ __forceinline__ void load_next(Cursor& c, const AttnParams& p, int lane) {
  if constexpr (PAGED) {
    const int* rec = (const int*)(p.seqinfo + c.nb);
#pragma unroll
    for (int k = 0; k < 6; ++k) c.nw[k] = ld_const(rec, k);
  } else {
    c.nx = seqinfo_word(p.seqinfo, c.nb, opaque(lane));
  }
}
// Word k of the loaded record (wave-uniform).
template <bool PAGED>
__device__ __forceinline__ int next_word(const Cursor& c, int k) {
  if constexpr (PAGED) return c.nw[k];
  else return __builtin_amdgcn_readlane(c.nx, k);
}

// Paged cache: the row of the first token of block `page` of sequence b (an
// entry outside the pool reads page 0 of it: a wrong page, never outside it).
// One unsigned 32-bit compare tests both bounds (a negative entry is 2^31 or
// more as unsigned), so the test stays on the scalar unit.
__device__ __forceinline__ int64_t page_row0(const AttnParams& p, int b, int page) {
  const int32_t pg = ld_const(p.block_table, (int64_t)b * p.max_pages + page);
  return (int64_t)((uint32_t)pg < p.page_limit ? pg : 0) * p.page_tokens;
}

// The first tile of worker w (c.b < 0: the worker has none); r_hi receives
// one past its last tile. PAGED: the cache is a page pool (AttnParams'
// block table); a compile-time switch, so that the contiguous kernels carry
// none of the page bookkeeping.
template <int TILE, bool PAGED>
__device__ __forceinline__ Cursor cursor_start(const AttnParams& p, int64_t w, int lane,
                                               int64_t& r_hi) {
  const WorkerInfo* wi = p.winfo + w;
  Cursor c;
  c.b = ld_const(&wi->b, 0);
  c.t = ld_const(&wi->t, 0);
  c.t_end = ld_const(&wi->t_end, 0);
  c.row0 = ld_const(&wi->row0, 0);
  c.nb = ld_const(&wi->next, 0);
  r_hi = ld_const(&wi->r_hi, 0);
  c.nx = 0;
#pragma unroll
  for (int k = 0; k < 6; ++k) c.nw[k] = 0;
  if (c.b >= 0 && c.nb < p.B) load_next<PAGED>(c, p, lane);
  c.page = 0;
  c.page_left = 0;
  if (PAGED && c.b >= 0) {
    const int t = (int)c.t;
    c.page = t / p.page_tokens;
    c.page_left = p.page_tiles - (t - c.page * p.page_tokens) / TILE;
  }
  return c;
}

// The sequence of the worker's next segment after the current one (-1: none).
template <bool PAGED>
__device__ __forceinline__ int next_segment_seq(const Cursor& c, const AttnParams& p, int64_t r_hi) {
  if (c.nb >= p.B) return -1;
  const int64_t t0 = next_word<PAGED>(c, 3);
  return t0 < r_hi ? c.nb : -1;
}

// Move to the next tile of the worker's range; false when done.
template <int TILE, bool PAGED>
__device__ __forceinline__ bool advance(Cursor& c, const AttnParams& p, int64_t r_hi, int lane) {
  c.t += TILE;
  c.row0 += TILE;
  if (c.t < c.t_end) {
    if constexpr (PAGED) {
      if (--c.page_left == 0) {                        // into the next page
        ++c.page;
        c.page_left = p.page_tiles;
        c.row0 = page_row0(p, c.b, c.page);
      }
    }
    return true;
  }
  if (c.nb >= p.B) return false;
  const int64_t t0 = next_word<PAGED>(c, 3);
  if (t0 >= r_hi) return false;
  const int64_t t1 = next_word<PAGED>(c, 4);
  const int64_t len = next_word<PAGED>(c, 2);
  const int64_t se = t1 < r_hi ? t1 : r_hi;
  c.b = c.nb;
  c.t = 0;
  c.t_end = (se - t0) * TILE < len ? (se - t0) * TILE : len;
  c.row0 = (int64_t)(((uint64_t)(uint32_t)next_word<PAGED>(c, 1) << 32) |
                     (uint32_t)next_word<PAGED>(c, 0));
  c.nb = next_word<PAGED>(c, 5);
  if (c.nb < p.B) load_next<PAGED>(c, p, lane);
  if constexpr (PAGED) {                                // the plan's row0 is page 0's
    c.page = 0;
    c.page_left = p.page_tiles;
  }
  return true;
}

// The asynchronous copies of one tile, split over the NW waves of a
// workgroup. Stage slot s = id*64 + lane (id = a 1 KB wave copy) holds
// padded-row s / SPR, 16-byte chunk s % SPR; the pad chunk and slots past
// the tile repeat valid data, so every copy is a full 64-lane copy. fp8
// tiles add one copy of the 32 row scales.
template <int CT, int NW>
struct TileCopy {
  static constexpr int TILE = Tr<CT>::kTile;
  static constexpr int RB = Tr<CT>::kRowBytes;
  static constexpr int RP = Tr<CT>::kPad;
  static constexpr int SPR = RP / 16;
  static constexpr int NCH = (TILE * RP + 1023) / 1024;
  static constexpr int STAGE_DATA = NCH * 1024;
  static constexpr int STAGE_BYTES = STAGE_DATA + (CT == kFP8 ? 256 : 0);
  static constexpr int NCOPY = NCH + (CT == kFP8 ? 1 : 0);
  static constexpr int CPW = (NCOPY + NW - 1) / NW;
  static_assert(NCOPY > NW, "a repeated copy needs an earlier copy of the same wave");

  int wave_;

  __device__ __forceinline__ void init(int wave, int /*lane*/) { wave_ = wave; }
  // this lane's index, recomputed at each use (two VALU operations) rather
  // than held in a register through the tile loop
  __device__ __forceinline__ static int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  }
  // wave-uniform copy index of this wave's i-th copy (a 1 KB block of the stage)
  __device__ __forceinline__ int id(int i) const {
    const int k = wave_ + i * NW;
    return k >= NCOPY ? k - NW : k;                      // repeat this wave's previous copy
  }
  // this lane's byte offset in a full tile for copy k (recomputed at every
  // issue rather than hoisted out of the tile loop into registers)
  __device__ __forceinline__ uint32_t off(int k) const {
    const int ln = lane_id();
    const int s = k * 64 + ln;
    int r = s / SPR, c = s - (s / SPR) * SPR;
    if (c >= RB / 16) c = RB / 16 - 1;
    if (r >= TILE) r = TILE - 1;
    return (uint32_t)(r * RB + c * 16);
  }

  // The same offset from the slot's row r = s / SPR written as the row of the
  // wave's first slot (a wave-uniform division) plus one for the lanes past
  // the next row boundary: two vector compares instead of a vector division.
  __device__ __forceinline__ uint32_t off_rows(int k) const {
    static_assert(SPR >= 64, "a wave's 64 slots cross at most one row boundary");
    const int ln = lane_id();
    const int s0 = uniform(k * 64);
    const int r0 = s0 / SPR;
    const int thr = SPR * (r0 + 1) - s0;               // first lane of row r0 + 1
    const int up = ln >= thr ? 1 : 0;
    int r = r0 + up;
    int c = ln + (s0 - SPR * r0) - SPR * up;
    if (c >= RB / 16) c = RB / 16 - 1;
    if (r >= TILE) r = TILE - 1;
    return (uint32_t)(r * RB + c * 16);
  }

  // One tile's copies, issued one at a time (so that a wave can spread them
  // over its compute instead of stalling on the memory pipeline at once).
  struct Pending {
    __amdgpu_buffer_rsrc_t rsrc, srsrc;
    char* sb;
    int nvalid;
  };
  __device__ __forceinline__ Pending prepare(const char* rows, const float* row_scale,
                                             const Cursor& c, char* sb) const {
    Pending q;
    const int64_t left = c.t_end - c.t;
    q.nvalid = left < TILE ? (int)left : TILE;
    q.rsrc = make_rsrc(rows + c.row0 * RB, (uint32_t)(TILE * RB));
    q.srsrc = make_rsrc(CT == kFP8 ? (const void*)(row_scale + c.row0) : (const void*)rows,
                        (uint32_t)(TILE * 4));
    q.sb = sb;
    return q;
  }
  template <bool ROWS = false>
  __device__ __forceinline__ void copy(const Pending& q, int i) const {
    const int k = id(i);
    if (CT == kFP8 && k == NCH) {
      const int ln = lane_id() & (TILE - 1);
      const int r = ln < q.nvalid ? ln : q.nvalid - 1;
      buffer_copy4(q.srsrc, (uint32_t)(r * 4), q.sb + STAGE_DATA);
      return;
    }
    uint32_t o;
    if constexpr (ROWS) o = off_rows(k);
    else o = off(k);
    if (q.nvalid < TILE) {
      const uint32_t r = o / RB;
      if (r >= (uint32_t)q.nvalid) o -= (r - (q.nvalid - 1)) * RB;
    }
    buffer_copy16(q.rsrc, o, q.sb + k * 1024);
  }

  // Copy the tile at cursor c into stage buffer sb. Rows past the end of the
  // segment repeat its last valid row.
  __device__ __forceinline__ void issue(const char* rows, const float* row_scale, const Cursor& c,
                                        char* sb, int lane) const {
    const int64_t left = c.t_end - c.t;
    const int nvalid = left < TILE ? (int)left : TILE;
    const auto rsrc = make_rsrc(rows + c.row0 * RB, (uint32_t)(TILE * RB));
    // exactly one copy instruction per i on every path, so that wait counts
    // the compiler derives for later loads hold on all of them
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int k = id(i);
      if (CT == kFP8 && k == NCH) {
        const auto srsrc = make_rsrc(row_scale + c.row0, (uint32_t)(TILE * 4));
        const int r = (lane & (TILE - 1)) < nvalid ? (lane & (TILE - 1)) : nvalid - 1;
        buffer_copy4(srsrc, (uint32_t)(r * 4), sb + STAGE_DATA);
      } else {
        uint32_t o = off(k);
        if (nvalid < TILE) {
          const uint32_t r = o / RB;
          if (r >= (uint32_t)nvalid) o -= (r - (nvalid - 1)) * RB;
        }
        buffer_copy16(rsrc, o, sb + k * 1024);
      }
    }
  }
};

// Widen a staged fp8 tile (codes at pitch RP) to bf16 rows at pitch
// kConvPad, all threads of the workgroup cooperating. Every e4m3fn value is
// exact in bf16.
template <int NT>
__device__ __forceinline__ void widen_fp8_tile(const char* stage, char* conv) {
  constexpr int RP = Tr<kFP8>::kPad;
  for (int i = threadIdx.x; i < 32 * 36; i += NT) {      // 16-code chunks
    const int r = i / 36;
    const int j = i - r * 36;
    const u32x4 v = *(const u32x4*)(stage + r * RP + j * 16);
    const uint2 c0 = fp8x4_to_bf16x4(v[0]), c1 = fp8x4_to_bf16x4(v[1]);
    const uint2 c2 = fp8x4_to_bf16x4(v[2]), c3 = fp8x4_to_bf16x4(v[3]);
    *(u32x4*)(conv + r * kConvPad + j * 32) = u32x4{c0.x, c0.y, c1.x, c1.y};
    *(u32x4*)(conv + r * kConvPad + j * 32 + 16) = u32x4{c2.x, c2.y, c3.x, c3.y};
  }
}

// Widen a staged fp6 tile (464-byte rows: 576 packed e2m3 codes, then the
// 18 e8m0 block scales) to bf16 rows at pitch kConvPad, all threads of the
// workgroup cooperating: one block of 32 codes (24 bytes) and its scale per
// conversion (v_cvt_scalef32_pk32_bf16_fp6: element i from bits 6i .. 6i+5,
// times the scale; an e2m3 value times a power of two is exact in bf16).
template <int NT>
__device__ __forceinline__ void widen_fp6_tile(const char* stage, char* conv) {
  typedef int i32x6 __attribute__((ext_vector_type(6)));
  typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));
  constexpr int RB = Tr<kFP6>::kRowBytes;
  for (int i = threadIdx.x; i < 32 * 18; i += NT) {
    const int r = i / 18;
    const int j = i - r * 18;
    const char* src = stage + r * RB + 24 * j;
    const uint2 w0 = *(const uint2*)src, w1 = *(const uint2*)(src + 8), w2 = *(const uint2*)(src + 16);
    const int e = (int)*(const uint8_t*)(stage + r * RB + 432 + j);
    const i32x6 codes = {(int)w0.x, (int)w0.y, (int)w1.x, (int)w1.y, (int)w2.x, (int)w2.y};
    const bf16x32 v = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(codes, __builtin_amdgcn_ldexpf(1.f, e - 127));
    const u32x4* vv = (const u32x4*)&v;
    char* dst = conv + r * kConvPad + 64 * j;
#pragma unroll
    for (int k = 0; k < 4; ++k) *(u32x4*)(dst + 16 * k) = vv[k];
  }
}

// The same widening for kernels whose stage buffers are filled by
// asynchronous copies: the staged codes and scales are read in asm blocks
// that wait inside, so the compiler does not make them wait for every copy in
// flight (the converted rows are ordinary LDS stores).
template <int NT>
__device__ __forceinline__ void widen_fp6_tile_async(const char* stage, char* conv) {
  typedef int i32x6 __attribute__((ext_vector_type(6)));
  typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  constexpr int RB = Tr<kFP6>::kRowBytes;
  for (int i = threadIdx.x; i < 32 * 18; i += NT) {
    const int r = i / 18;
    const int j = i - r * 18;
    const uint32_t a = (uint32_t)(size_t)(stage + r * RB + 24 * j);
    const uint32_t as = (uint32_t)(size_t)(stage + r * RB + 432 + j);
    u32x2 w0, w1, w2;
    uint32_t e;
    asm volatile(
        "ds_read_b64 %0, %4\n"
        "ds_read_b64 %1, %4 offset:8\n"
        "ds_read_b64 %2, %4 offset:16\n"
        "ds_read_u8 %3, %5\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(e)
        : "v"(a), "v"(as)
        : "memory");
    const unsigned x0 = w0[0], x1 = w0[1], x2 = w1[0], x3 = w1[1], x4 = w2[0], x5 = w2[1];
    const i32x6 codes = {(int)x0, (int)x1, (int)x2, (int)x3, (int)x4, (int)x5};
    const bf16x32 v = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(codes, __builtin_amdgcn_ldexpf(1.f, (int)e - 127));
    const u32x4* vv = (const u32x4*)&v;
    char* dst = conv + r * kConvPad + 64 * j;
#pragma unroll
    for (int k = 0; k < 4; ++k) *(u32x4*)(dst + 16 * k) = vv[k];
  }
}

// Value operands of four 16-dim blocks starting at block NB0: the low half
// covers tile rows 0..15, the high half rows 16..31 (row pitch TP bytes).
template <int TP, int NB0>
__device__ __forceinline__ void pv_read4(uint32_t addr, s16x4* lo, s16x4* hi) {
  lds_tr16_x8<NB0 * 32, 16 * TP + NB0 * 32, (NB0 + 1) * 32, 16 * TP + (NB0 + 1) * 32,
              (NB0 + 2) * 32, 16 * TP + (NB0 + 2) * 32, (NB0 + 3) * 32, 16 * TP + (NB0 + 3) * 32>(
      addr, lo[0], hi[0], lo[1], hi[1], lo[2], hi[2], lo[3], hi[3]);
}

// Store four consecutive values (dims d..d+3 of one head) of a segment's
// normalised partial output o / l: fp32 for the f32 cache, bf16 otherwise
// (the normalised partial is a convex combination of cached rows, so one bf16
// rounding of it is of the size of the rounding of the bf16 output itself).
template <int CT>
__device__ __forceinline__ void store_part4(void* part_o, int64_t elem, const f32x4& v, float inv_l) {
  const f32x4 x = v * inv_l;
  if constexpr (CT == kF32) {
    *(f32x4*)((float*)part_o + elem) = x;
  } else {
    uint2 u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    *(uint2*)((uint16_t*)part_o + elem) = u;
  }
}
// 1 / l for the normalisation (0 for an empty sum; NaN stays NaN)
__device__ __forceinline__ float inv_or_zero(float l) { return l != 0.f ? 1.f / l : 0.f; }

// Launcher of the streaming kernel (decode_attn_stream.hip).
hipError_t launch_attn_stream(const DecodePlan& plan, const AttnParams& prm, hipStream_t s);
// Launcher of the 128-head kernel (decode_attn_h32.hip).
hipError_t launch_attn_h32(const DecodePlan& plan, const AttnParams& prm, hipStream_t s);

}  // namespace mla
