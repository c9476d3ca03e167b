// The per-head GEMMs around the attention kernel and the work plan, shared
// by the decode launches (decode_gemm.hip) and the fused append + absorb
// launch (append.hip).
#pragma once

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace mla {

struct GemmParams {
  const void* x;              // absorb: q_nope [B][H][128]
  const void* w;              // [H][KD][ND]
  void* y;                    // absorb: q_lat [B][H][512]; project: out [B][H][128]
  float* lse;                 // project: [B][H] or null
  const void* part_o;         // merge: [nslot][H][512] o/l, f32 (f32 path) or bf16
  const float* part_ml;       // merge: [nslot][H][2] (m, l)
  SeqInfo* seqinfo;           // [B] (written by the plan block of absorb)
  int64_t* starts;            // [W+1]
  int32_t* wseq;              // [W]
  WorkerInfo* winfo;          // [W]
  int32_t* wfirst;            // [B]
  int32_t* wlast;             // [B]
  const int32_t* seq_len;     // absorb: [B]
  const int32_t* seq_cap;     // absorb: [B]
  const int64_t* seq_start;   // absorb: [B]
  const int32_t* block_table; // absorb, paged cache: [B][max_pages] (null: contiguous)
  int32_t page_tokens;
  int32_t max_pages;
  int64_t total_pages;
  int32_t B;
  int32_t H;
  int32_t workers;            // W of the attention launch
  int32_t tile;               // tokens per tile of the attention launch
  int32_t seg_tiles;          // tiles of work counted for starting a sequence segment
};

constexpr int kNT = 64;       // output columns per workgroup (one 16-wide block per wave)

// The work plan, built by one extra workgroup of the absorb launch so the
// attention and merge kernels need no divisions or searches. Sequence b has
// n_b = ceil(len_b / tile) tiles (len clamped to [0, capacity]). Starting a
// sequence segment costs a worker about a tile's time or more (its queries
// come in, a partial goes out), so a non-empty sequence counts seg_tiles
// more (a property of the attention kernel): v_b = n_b + seg_tiles, or 0. P_b is the prefix sum of v, NT = P_B, and the
// work of all sequences forms one stream in which sequence b holds
// [P_b, P_(b+1)), its real tiles being the last n_b of them:
//   seqinfo[b] = {first cache row, len_b, P_(b+1) - n_b, P_(b+1), next sequence with tiles}
//   starts[w]  = floor(w * NT / W): worker w takes [starts[w], starts[w+1])
//   wseq[w]    = the sequence holding starts[w] (non-empty workers)
//   wfirst[b], wlast[b] = first and last worker that touch a real tile of b
//                (wlast < wfirst for an empty sequence)
// Splitting whole tiles keeps every split inside a sequence on a tile
// boundary, so the only partial tile of a sequence is its last one. A worker
// whose range holds only counted-but-empty units has no tiles and lies
// outside every sequence's [wfirst, wlast].
// floor(w NT / W) >= P exactly when w >= ceil(P W / NT), so sequence b holds
// the starts of workers [ceil(P_b W/NT), ceil(P_(b+1) W/NT)), the worker
// holding unit R is ceil((R + 1) W / NT) - 1, so b's first worker is that of
// its first real tile R0 = P_(b+1) - n_b and its last ceil(P_(b+1) W / NT) - 1:
// every entry is a closed form of the prefix sums, which stay in LDS (`lds`,
// room for `lds_n` values) when they fit.
__device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ void build_plan(const GemmParams& p, int64_t* lds, int lds_n) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = p.B;
  const int64_t W = p.workers;
  const int TL = p.tile;
  // LDS (when it fits): P[0..B], then each sequence's first cache row and
  // clamped length, so the worker records need no second trip to memory
  const bool in_lds = 3 * (int64_t)B + 1 <= lds_n;
  int64_t* lrow = lds + B + 1;
  int64_t* llen = lds + 2 * B + 1;
  if (tid < 64) {
    int64_t carry = 0;
    if (lane == 0 && in_lds) lds[0] = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      // the three per-sequence loads go out together (one asm block that
      // waits at its end; left to itself the compiler waits for each load
      // before issuing the next)
      const int bc = b < B ? b : B - 1;
      int Lr, cap;
      int64_t row0;
      if (p.block_table) {
        // paged: the capacity is the table's, the first row that of page 0
        // (an entry outside the pool reads page 0: attention then reads a
        // wrong page, never outside the pool)
        Lr = p.seq_len[bc];
        cap = p.max_pages * p.page_tokens;
        bool ok;
        row0 = paged_row(p.block_table, p.max_pages, p.page_tokens, p.total_pages, bc, 0, ok);
      } else {
        asm volatile(
            "global_load_dword %0, %3, off\n"
            "global_load_dword %1, %4, off\n"
            "global_load_dwordx2 %2, %5, off\n"
            "s_waitcnt vmcnt(0)"
            : "=&v"(Lr), "=&v"(cap), "=&v"(row0)
            : "v"(p.seq_len + bc), "v"(p.seq_cap + bc), "v"(p.seq_start + bc)
            : "memory");
      }
      int L = 0;
      if (b < B) L = Lr < 0 ? 0 : (Lr > cap ? cap : Lr);
      const int64_t n = (L + TL - 1) / TL;
      int64_t v = n > 0 ? n + p.seg_tiles : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int src = lane - off;
        const int lo = __builtin_amdgcn_ds_bpermute((src < 0 ? lane : src) << 2, (int)(v & 0xffffffff));
        const int hi = __builtin_amdgcn_ds_bpermute((src < 0 ? lane : src) << 2, (int)(v >> 32));
        const int64_t u = ((int64_t)hi << 32) | (uint32_t)lo;
        if (src >= 0) v += u;
      }
      if (b < B) {
        SeqInfo si;
        si.row0 = row0;
        si.len = L;
        si.tile0 = (int32_t)(carry + v - n);
        si.tile1 = (int32_t)(carry + v);
        si.next = B;                                     // set below
        si.pad[0] = si.pad[1] = 0;
        p.seqinfo[b] = si;
        if (in_lds) {
          lds[b + 1] = carry + v;
          lrow[b] = si.row0;
          llen[b] = L;
        }
      }
      const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffff), 63);
      const int hi = __builtin_amdgcn_readlane((int)(v >> 32), 63);
      carry += ((int64_t)hi << 32) | (uint32_t)lo;
    }
    if (!in_lds && lane == 0) lds[0] = carry;            // NT for the other waves
  }
  // the records are read back only by this workgroup's threads (and by later
  // launches, which the kernel boundary orders), so workgroup scope suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const volatile int32_t* gtile1 = &p.seqinfo[0].tile1;
  const volatile int32_t* glen = &p.seqinfo[0].len;
  constexpr int SI = sizeof(SeqInfo) / 4;
  // P_b for b < B (P_B = NT): the end of the previous sequence's units
  auto prefix = [&](int b) -> int64_t {
    return in_lds ? lds[b] : (b == 0 ? 0 : (int64_t)gtile1[(int64_t)(b - 1) * SI]);
  };
  // real tiles of sequence b
  auto ntiles = [&](int b) -> int64_t {
    const int64_t len = in_lds ? llen[b] : (int64_t)glen[(int64_t)b * SI];
    return (len + TL - 1) / TL;
  };
  const int64_t NT = in_lds ? lds[B] : lds[0];
  // the sequence holding tile t < NT: the largest b in [lo, B) with P_b <= t
  auto owner = [&](int lo, int64_t t) {
    int hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix(mid) <= t) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  const int nthr = (int)blockDim.x;
  for (int64_t w = tid; w <= W; w += nthr) p.starts[w] = (w * NT) / W;
  if (NT == 0) {
    for (int64_t w = tid; w < W; w += nthr) p.wseq[w] = 0;
  }
  for (int b = tid; b < B; b += nthr) {
    const int64_t P0 = prefix(b), P1 = (b + 1 < B) ? prefix(b + 1) : NT;
    if (P1 > P0) {
      const int64_t wlo = ceil_div64(P0 * W, NT), whi = ceil_div64(P1 * W, NT);
      for (int64_t w = wlo; w < whi; ++w) p.wseq[w] = b;
      p.wfirst[b] = (int)(ceil_div64((P1 - ntiles(b) + 1) * W, NT) - 1);
      p.wlast[b] = (int)(whi - 1);
    } else {
      p.wfirst[b] = 0;
      p.wlast[b] = -1;
    }
    // next sequence with tiles: the one owning tile P_(b+1) (none when it is NT)
    p.seqinfo[b].next = (P1 < NT) ? owner(b + 1, P1) : B;
  }
  if (!in_lds) {                                         // the records come back from memory
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  // each worker's starting point
  for (int64_t w = tid; w < W; w += nthr) {
    const int64_t r_lo = (w * NT) / W, r_hi = ((w + 1) * NT) / W;
    WorkerInfo wi;
    wi.r_hi = (int32_t)r_hi;
    wi.pad = 0;
    wi.row0 = 0;
    wi.b = -1;
    wi.t = wi.t_end = 0;
    wi.next = B;
    if (r_lo < r_hi) {
      int b;
      int64_t t0, t1, len, row0;
      int nx;
      if (in_lds) {
        b = owner(0, r_lo);
        t1 = lds[b + 1];
        len = llen[b];
        t0 = t1 - (len + TL - 1) / TL;                   // first real tile of b
        row0 = lrow[b];
        nx = (t1 < NT) ? owner(b + 1, t1) : B;
      } else {
        b = ((const volatile int32_t*)p.wseq)[w];
        const volatile SeqInfo* si = p.seqinfo + b;
        t0 = si->tile0;
        t1 = si->tile1;
        len = si->len;
        row0 = si->row0;
        nx = si->next;
      }
      // a range that ends within b's counted-only units holds no tile (and
      // cannot reach the next sequence); otherwise it starts at its first
      // real tile of b
      if (r_hi > t0) {
        const int64_t first = r_lo > t0 ? r_lo : t0;
        const int64_t se = t1 < r_hi ? t1 : r_hi;
        wi.b = b;
        wi.t = (int32_t)((first - t0) * TL);
        wi.t_end = (int32_t)((se - t0) * TL < len ? (se - t0) * TL : len);
        if (p.block_table) {
          bool ok;
          wi.row0 = paged_row(p.block_table, p.max_pages, p.page_tokens, p.total_pages, b, wi.t, ok);
        } else {
          wi.row0 = row0 + wi.t;
        }
        wi.next = nx;
      }
    }
    p.winfo[w] = wi;
  }
}

// Y[b][h][:] = X[b][h][:] . W[h] for one head, 64 output columns from n0 and
// 16*NBT batch rows from b0. AT: kF32 or kBF16, the element type of x, w
// and y. The weight slice W[h][0:KD][n0:n0+64] is staged in LDS KC rows at a
// time. load() issues the X tile and the first weight chunk into registers
// (so a caller can put other work between the loads and their use); run()
// stages them in LDS (`lds`, LDS_BYTES), computes and stores Y. It runs on
// 256 threads: threads 256k..256k+255 of a larger workgroup form a group of
// their own (each with its own LDS), and run() takes 2*kChunks - 1 barriers.
template <int AT, int KD, int ND, int NBT, int KC>
struct HeadGemm {
  using E = typename std::conditional<AT == kF32, float, __bf16>::type;
  static constexpr int ES = sizeof(E);
  static constexpr int BT = 16 * NBT;                 // batch rows per workgroup
  static constexpr int WROW = kNT * ES + 16;          // LDS stride of a weight row
  static constexpr int XROW = KD * ES + 16;           // LDS stride of an X row
  static constexpr int XP = BT * KD * ES / 16;        // 16-byte pieces of the X tile
  static constexpr int WP = KC * kNT * ES / 16;       // 16-byte pieces of one weight chunk
  static constexpr int XPR = KD * ES / 16;            // 16-byte pieces per X row
  static constexpr int WPR = kNT * ES / 16;           // 16-byte pieces per weight row
  static constexpr int W_BYTES = KC * WROW;
  static constexpr int LDS_BYTES = KC * WROW + BT * XROW;
  static constexpr int kChunks = KD / KC;             // weight chunks staged by run()
  static_assert(XP % 256 == 0 && WP % 256 == 0, "whole rounds of 16-byte pieces");

  struct Regs {
    u32x4 xv[XP / 256];
    u32x4 wv[WP / 256];
  };

  __device__ static void load_w(const GemmParams& p, int h, int n0, int k0, u32x4* v) {
    const int tid = threadIdx.x & 255;
#pragma unroll
    for (int k = 0; k < WP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / WPR, c = i - r * WPR;
      v[k] = *(const u32x4*)((const char*)p.w + (((int64_t)h * KD + k0 + r) * ND + n0) * ES + c * 16);
    }
  }
  __device__ static void store_w(char* w_lds, const u32x4* v) {
    const int tid = threadIdx.x & 255;
#pragma unroll
    for (int k = 0; k < WP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / WPR, c = i - r * WPR;
      *(u32x4*)(w_lds + r * WROW + c * 16) = v[k];
    }
  }
  __device__ static void load(const GemmParams& p, int n0, int h, int b0, Regs& rg) {
    const int tid = threadIdx.x & 255;
#pragma unroll
    for (int k = 0; k < XP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / XPR, c = i - r * XPR;
      const int b = b0 + r;
      rg.xv[k] = u32x4{0u, 0u, 0u, 0u};
      if (b < p.B) rg.xv[k] = *(const u32x4*)((const char*)p.x + (((int64_t)b * p.H + h) * KD) * ES + c * 16);
    }
    load_w(p, h, n0, 0, rg.wv);
  }
  __device__ static void run(const GemmParams& p, int n0, int h, int b0, Regs& rg, char* lds) {
    const int tid = threadIdx.x & 255;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int g = lane >> 4;
    const int H = p.H, B = p.B;
    char* w_lds = lds;
    char* x_lds = lds + W_BYTES;
#pragma unroll
    for (int k = 0; k < XP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / XPR, c = i - r * XPR;
      *(u32x4*)(x_lds + r * XROW + c * 16) = rg.xv[k];
    }
    store_w(w_lds, rg.wv);

    f32x4 acc[NBT];
#pragma unroll
    for (int i = 0; i < NBT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < KD; k0 += KC) {
      if (k0) {
        u32x4 wv[WP / 256];
        load_w(p, h, n0, k0, wv);
        __syncthreads();                               // previous chunk consumed
        store_w(w_lds, wv);
      }
      __syncthreads();
      if constexpr (AT == kF32) {
#pragma unroll 4
        for (int kk = 0; kk < KC; kk += 4) {
          const float a = *(const float*)(w_lds + (kk + g) * WROW + (16 * wave + l16) * 4);
#pragma unroll
          for (int nb = 0; nb < NBT; ++nb) {
            const float bv = *(const float*)(x_lds + (16 * nb + l16) * XROW + (k0 + kk + g) * 4);
            acc[nb] = mfma_f32_k4(a, bv, acc[nb]);
          }
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KC; kk += 32) {
          // A = W^T block: lane (n, g) gets W[kk + 8g + 0..7][16*wave + n]
          const int rs = kk + 8 * g + (l16 >> 2);
          const int cb = (16 * wave + 4 * (l16 & 3)) * 2;
          const s16x4 lo = lds_read_tr16(w_lds, rs * WROW + cb);
          const s16x4 hi = lds_read_tr16(w_lds, (rs + 4) * WROW + cb);
          const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
          for (int nb = 0; nb < NBT; ++nb) {
            const bf16x8 bv = lds_read_b128(x_lds, (16 * nb + l16) * XROW + (k0 + kk + 8 * g) * 2);
            acc[nb] = mfma_bf16_k32(a, bv, acc[nb]);
          }
        }
      }
    }

    // ---------------- store: lane holds Y[b][n0 + 16w + 4g + r] ----------------
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb) {
      const int b = b0 + 16 * nb + l16;
      if (b >= B) continue;
      const int n = n0 + 16 * wave + 4 * g;
      char* dst = (char*)p.y + (((int64_t)b * H + h) * ND + n) * ES;
      if constexpr (AT == kF32) {
        *(f32x4*)dst = acc[nb];
      } else {
        uint2 v;
        v.x = pack_bf16x2(acc[nb][0], acc[nb][1]);
        v.y = pack_bf16x2(acc[nb][2], acc[nb][3]);
        *(uint2*)dst = v;
      }
    }
  }
};

// The absorb product as launched (bf16: 64 batch rows per workgroup)
using AbsorbBf16 = HeadGemm<kBF16, kDnope, kDc, 4, kDnope>;
using AbsorbF32 = HeadGemm<kF32, kDnope, kDc, 1, kDnope>;

// Parameters of the absorb launch (and its plan workgroup) for a decode call.
inline GemmParams absorb_params(const DecodePlan& plan, const DecodeArgs& a) {
  GemmParams g{};
  g.B = a.B;
  g.H = a.H;
  g.workers = plan.workers;
  g.seqinfo = a.seqinfo;
  g.winfo = a.winfo;
  g.starts = a.starts;
  g.seq_start = a.seq_start;
  g.tile = plan.tile;
  g.seg_tiles = plan.seg_tiles;
  g.wseq = a.wseq;
  g.wfirst = a.wfirst;
  g.wlast = a.wlast;
  g.seq_len = a.seq_len;
  g.seq_cap = a.seq_cap;
  g.block_table = a.block_table;
  g.page_tokens = a.page_tokens;
  g.max_pages = a.max_pages;
  g.total_pages = a.total_pages;
  g.x = a.q_nope;
  g.w = a.w_uk;
  g.y = a.q_lat;
  return g;
}

}  // namespace mla
