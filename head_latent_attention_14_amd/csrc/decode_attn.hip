// MLA decode attention over the latent cache (split-K partials).
//
// One workgroup streams a contiguous range of cached tokens (a share of the
// concatenation of all sequences, so every workgroup moves the same number of
// bytes) through an LDS ring filled by asynchronous global->LDS copies. Every
// 32-token tile of 576-wide latent rows is read from HBM once and used from
// LDS by all heads of the workgroup for both contractions (discosf explainer,
// "long-context bottleneck": W_UK folds into the query and W_UV into the
// output, so scores and values both come from the same latent rows):
//   scores  S^T[t][h] = c_t . q_lat[h] + k_pe_t . q_pe[h]  (MFMA, A = tile rows)
//   values  O^T[d][h] += sum_t c_t[d] p[t][h]              (MFMA, A = tile^T)
// with an online softmax per head in between. When a range ends or crosses a
// sequence boundary the unnormalised (m, l, o_lat) of that segment is written
// to a partial slot; the merge kernel combines the slots of each sequence.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace mla {

struct AttnParams {
  const char* rows;
  const float* row_scale;
  const int64_t* seq_start;
  const int64_t* prefix;     // [B+1]
  const void* q_lat;         // [B][H][512]  bf16 (f32 for the f32 cache)
  const void* q_pe;          // [B][H][64]
  float* part_o;             // [nslot][H][512]
  float* part_ml;            // [nslot][H][2]
  int32_t B;
  int32_t H;
  float scale_log2;          // softmax_scale * log2(e)
};

template <int CT> struct Tr;
template <> struct Tr<kBF16> { static constexpr int kRowBytes = 1152, kTile = 32; };
template <> struct Tr<kFP8> { static constexpr int kRowBytes = 576, kTile = 32; };
template <> struct Tr<kF32> { static constexpr int kRowBytes = 2304, kTile = 16; };

// XOR swizzle of the 16-byte chunk index inside an LDS row: rows 576, 1152
// or 2304 bytes apart start on the same bank, so chunk j of row r is stored
// at j ^ swz(r) to spread the 16 rows one MFMA operand read touches over the
// banks. The XOR stays inside aligned groups of 8 chunks (4 for the 36-chunk
// fp8 rows), so it never leaves the row.
template <int RB>
__device__ __forceinline__ int swz(int r) {
  return (RB % 128 == 0) ? ((r >> 1) & 7) : ((r >> 1) & 3);
}

template <int RB>
__device__ __forceinline__ uint32_t lds_off(int r, int chunk, int within = 0) {
  return (uint32_t)(r * RB + ((chunk ^ swz<RB>(r)) << 4) + within);
}

struct Cursor {
  int b;          // sequence
  int64_t t;      // first token of the tile, local to the sequence
  int64_t t_end;  // end of this worker's segment of the sequence (local)
};

// Move to the next tile of this worker's token range; false when done.
template <int TILE>
__device__ __forceinline__ bool advance(Cursor& c, const int64_t* prefix, int B, int64_t r_hi) {
  c.t += TILE;
  if (c.t < c.t_end) return true;
  int b = c.b + 1;
  while (b < B && ld_const(prefix, b + 1) == ld_const(prefix, b)) ++b;   // skip empty sequences
  b = uniform(b);
  if (b >= B || ld_const(prefix, b) >= r_hi) return false;
  c.b = b;
  c.t = 0;
  const int64_t pb = ld_const(prefix, b), pe = ld_const(prefix, b + 1);
  c.t_end = (pe < r_hi ? pe : r_hi) - pb;
  return true;
}

template <int CT, int HB, int DS, int NSTAGE>
__global__ void __launch_bounds__(64 * HB * DS)
mla_attn_kernel(AttnParams p) {
  constexpr int NW = HB * DS;
  constexpr int TILE = Tr<CT>::kTile;
  constexpr int RB = Tr<CT>::kRowBytes;
  constexpr int STAGE_DATA = TILE * RB;
  constexpr int STAGE_BYTES = STAGE_DATA + (CT == kFP8 ? 256 : 0);
  constexpr int NCH = STAGE_DATA / 1024;                 // 1 KB wave copies per tile
  constexpr int CPR = RB / 16;                           // 16-byte chunks per row
  constexpr int CONV_BYTES = (CT == kFP8) ? TILE * 1152 : 0;
  constexpr int DSLICE = kDc / DS;
  constexpr int NB = DSLICE / 16;
  static_assert(STAGE_DATA % 1024 == 0, "tile must be whole 1 KB copies");
  static_assert(NSTAGE >= 2, "ring needs two stages");

  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE_BYTES + CONV_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int hb = wave % HB;
  const int ds = wave / HB;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int H = p.H;
  const int B = p.B;
  const int h = (blockIdx.y * HB + hb) * 16 + l16;       // head of this lane
  const int64_t W = gridDim.x;
  const int64_t w = blockIdx.x;
  const int64_t T = ld_const(p.prefix, B);
  const int64_t r_lo = worker_start(w, W, T);
  const int64_t r_hi = worker_start(w + 1, W, T);
  if (r_lo >= r_hi) return;                              // whole workgroup

  // Every wave issues CPW asynchronous copies per tile (the fp8 row scales
  // are one extra copy; a wave with nothing left repeats its previous copy),
  // so the number of copies in flight per tile is a compile-time constant.
  constexpr int NCOPY = NCH + (CT == kFP8 ? 1 : 0);
  constexpr int CPW = (NCOPY + NW - 1) / NW;
  static_assert(NCOPY > NW, "a repeated copy needs an earlier copy of the same wave");

  Cursor c0;
  c0.b = uniform(find_seq(p.prefix, B, r_lo));
  {
    const int64_t pb = ld_const(p.prefix, c0.b), pe = ld_const(p.prefix, c0.b + 1);
    c0.t = r_lo - pb;
    c0.t_end = (pe < r_hi ? pe : r_hi) - pb;
  }

  auto issue = [&](const Cursor& c, int stage) {
    const int64_t row0 = ld_const(p.seq_start, c.b) + c.t;
    const int64_t left = c.t_end - c.t;
    const int nvalid = left < TILE ? (int)left : TILE;
    char* sb = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      int id = wave + i * NW;
      if (id >= NCOPY) id -= NW;                         // repeat this wave's previous copy
      if (id < NCH) {
        const int pos = id * 64 + lane;
        const int r = pos / CPR;
        const int jp = pos - r * CPR;
        const int j = jp ^ swz<RB>(r);
        const int rr = r < nvalid ? r : nvalid - 1;      // pad rows repeat a valid row
        async_copy16(p.rows + (row0 + rr) * RB + j * 16, sb + id * 1024);
      } else {
        const int r = lane & (TILE - 1);
        const int rr = r < nvalid ? r : nvalid - 1;
        async_copy4(p.row_scale + row0 + rr, sb + STAGE_DATA);
      }
    }
  };

  // ---- per-lane query fragments (B operand of the score MFMA) ----
  typedef typename std::conditional<CT == kF32, float, bf16x8>::type QFrag;
  constexpr int NQ = (CT == kF32) ? kDrow / 4 : kDrow / 32;
  QFrag q[NQ];
  auto load_q = [&](int b) {
    const int64_t base = ((int64_t)b * H + h);
    if constexpr (CT == kF32) {
      const float* ql = (const float*)p.q_lat + base * kDc;
      const float* qp = (const float*)p.q_pe + base * kDr;
#pragma unroll
      for (int ks = 0; ks < kDc / 4; ++ks) q[ks] = ql[4 * ks + g];
#pragma unroll
      for (int ks = 0; ks < kDr / 4; ++ks) q[kDc / 4 + ks] = qp[4 * ks + g];
    } else {
      const __bf16* ql = (const __bf16*)p.q_lat + base * kDc;
      const __bf16* qp = (const __bf16*)p.q_pe + base * kDr;
#pragma unroll
      for (int ks = 0; ks < kDc / 32; ++ks) q[ks] = *(const bf16x8*)(ql + 32 * ks + 8 * g);
      q[16] = *(const bf16x8*)(qp + 8 * g);
      q[17] = *(const bf16x8*)(qp + 32 + 8 * g);
    }
  };

  load_q(c0.b);
  wait_vmcnt<0>();

  // ---- prologue: fill NSTAGE-1 stages ----
  Cursor lc = c0;
  bool lvalid = true;
  int issued = 0;
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i) {
    if (lvalid) {
      issue(lc, i);
      ++issued;
      lvalid = advance<TILE>(lc, p.prefix, B, r_hi);
    }
  }

  // ---- softmax state ----
  float m_run = -INFINITY;   // running max of this lane's head (log2 domain)
  float l_run = 0.f;         // this lane's share of the running sum
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  Cursor cc = c0;
  int it = 0;
  while (true) {
    wait_tiles<CPW, NSTAGE - 2>(issued - 1 - it);       // this wave's copies of tile `it` landed
    barrier_lds();                                       // tile `it` visible; stage it-1 free
    if (lvalid) {
      issue(lc, issued % NSTAGE);
      ++issued;
      lvalid = advance<TILE>(lc, p.prefix, B, r_hi);
    }
    const char* stage = smem + (it % NSTAGE) * STAGE_BYTES;
    const int64_t left = cc.t_end - cc.t;
    const int nvalid = left < TILE ? (int)left : TILE;

    const char* tb = stage;                              // bf16/f32 rows of this tile
    if constexpr (CT == kFP8) {
      // widen the fp8 codes to bf16 once for all waves
      char* conv = smem + NSTAGE * STAGE_BYTES;
      for (int i = threadIdx.x; i < TILE * 36; i += 64 * NW) {   // 16-code chunks
        const int r = i / 36;
        const int j = i - r * 36;                        // fp8 chunk (16 codes)
        const u32x4 v = *(const u32x4*)(stage + lds_off<576>(r, j));
        const uint2 c0 = fp8x4_to_bf16x4(v[0]), c1 = fp8x4_to_bf16x4(v[1]);
        const uint2 c2 = fp8x4_to_bf16x4(v[2]), c3 = fp8x4_to_bf16x4(v[3]);
        const u32x4 lo = {c0.x, c0.y, c1.x, c1.y};
        const u32x4 hi = {c2.x, c2.y, c3.x, c3.y};
        *(u32x4*)(conv + lds_off<1152>(r, 2 * j)) = lo;
        *(u32x4*)(conv + lds_off<1152>(r, 2 * j + 1)) = hi;
      }
      barrier_lds();
      tb = conv;
    }

    if constexpr (CT != kF32) {
      // ---------------- scores: two 16-token blocks ----------------
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const int j = 4 * ks + g;
        const bf16x8 a0 = lds_read_b128(tb, lds_off<1152>(l16, j));
        const bf16x8 a1 = lds_read_b128(tb, lds_off<1152>(16 + l16, j));
        s0 = mfma_bf16_k32(a0, q[ks], s0);
        s1 = mfma_bf16_k32(a1, q[ks], s1);
      }
      float sc[8];
      float tsc[8];                                      // fp8 row scales (1 otherwise)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t0 = 4 * g + r, t1 = 16 + 4 * g + r;
        if constexpr (CT == kFP8) {
          const float* scl = (const float*)(stage + STAGE_DATA);
          tsc[r] = scl[t0];
          tsc[4 + r] = scl[t1];
        } else {
          tsc[r] = 1.f;
          tsc[4 + r] = 1.f;
        }
        sc[r] = t0 < nvalid ? s0[r] * (p.scale_log2 * tsc[r]) : -INFINITY;
        sc[4 + r] = t1 < nvalid ? s1[r] * (p.scale_log2 * tsc[4 + r]) : -INFINITY;
      }
      float tmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = __builtin_fmaxf(tmax, sc[i]);
      tmax = max_over_groups(tmax);
      const float m_new = __builtin_fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = exp2f(sc[i] - m_use);
        psum += e;
        pv[i] = e * tsc[i];                              // fp8: value scale folded into P
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb] *= alpha;
      }
      const bf16x8 pb = pack_bf16x8(pv);

      // ---------------- values: O^T += tile^T P^T ----------------
      // A operand (tile^T): lane (d, g) needs c_t[d] for t = 4g+q and 16+4g+q,
      // q = 0..3. Read as 16-bit values; the transposing LDS read would make
      // the compiler wait for every copy in flight.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int d = ds * DSLICE + nb * 16 + l16;
        const uint32_t cb = (uint32_t)((d >> 3) << 4) + (d & 7) * 2;
        s16x8 a8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = 4 * g + q, r1 = 16 + 4 * g + q;
          a8[q] = *(const short*)(tb + r0 * 1152 + (cb ^ (swz<1152>(r0) << 4)));
          a8[4 + q] = *(const short*)(tb + r1 * 1152 + (cb ^ (swz<1152>(r1) << 4)));
        }
        o[nb] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a8), pb, o[nb]);
      }
    } else {
      // ---------------- f32 cache: one 16-token block ----------------
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kDrow / 4; ++ks) {
        const int e = 4 * ks + g;
        const float a = *(const float*)(tb + lds_off<2304>(l16, e >> 2, (e & 3) * 4));
        s0 = mfma_f32_k4(a, q[ks], s0);
      }
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = (4 * g + r) < nvalid ? s0[r] * p.scale_log2 : -INFINITY;
      float tmax = __builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3]));
      tmax = max_over_groups(tmax);
      const float m_new = __builtin_fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float pv[4];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = exp2f(sc[r] - m_use);
        psum += pv[r];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int d = ds * DSLICE + nb * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = *(const float*)(tb + lds_off<2304>(4 * g + r, d >> 2, (d & 3) * 4));
          o[nb] = mfma_f32_k4(a, pv[r], o[nb]);
        }
      }
    }

    // ---------------- segment end: write the partial ----------------
    const bool seg_end = (cc.t + TILE >= cc.t_end);
    if (seg_end) {
      const float lsum = sum_over_groups(l_run);
      const int64_t slot = w + cc.b;
      float* po = p.part_o + (slot * H + h) * kDc + ds * DSLICE + 4 * g;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) *(f32x4*)(po + nb * 16) = o[nb];
      if (ds == 0 && g == 0) {
        p.part_ml[(slot * H + h) * 2 + 0] = m_run;
        p.part_ml[(slot * H + h) * 2 + 1] = lsum;
      }
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (!advance<TILE>(cc, p.prefix, B, r_hi)) break;
    if (seg_end) {
      load_q(cc.b);
      wait_vmcnt<0>();
    }
    ++it;
  }
}

// ------------------------------------------------------------------ launch
template <int CT, int HB, int DS, int NSTAGE>
static hipError_t launch_attn_t(const AttnParams& prm, int workers, int head_groups,
                                hipStream_t s) {
  dim3 grid(workers, head_groups);
  dim3 block(64 * HB * DS);
  hipLaunchKernelGGL((mla_attn_kernel<CT, HB, DS, NSTAGE>), grid, block, 0, s, prm);
  return hipGetLastError();
}

hipError_t launch_attn(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  AttnParams prm;
  prm.rows = (const char*)a.rows;
  prm.row_scale = a.row_scale;
  prm.seq_start = a.seq_start;
  prm.prefix = a.prefix;
  prm.q_lat = a.q_lat;
  prm.q_pe = a.q_pe;
  prm.part_o = a.part_o;
  prm.part_ml = a.part_ml;
  prm.B = a.B;
  prm.H = a.H;
  prm.scale_log2 = a.softmax_scale * kLog2e;
  const int W = plan.workers, G = plan.head_groups;
#define MLA_CASE(CT_, HB_, DS_, NS_)                                              \
  if (ct == CT_ && plan.hb == HB_ && plan.ds == DS_ && plan.nstage == NS_)        \
    return launch_attn_t<CT_, HB_, DS_, NS_>(prm, W, G, s);
  MLA_CASE(kF32, 1, 4, 2)
  MLA_CASE(kBF16, 1, 4, 4)
  MLA_CASE(kBF16, 2, 2, 4)
  MLA_CASE(kBF16, 4, 1, 3)
  MLA_CASE(kFP8, 1, 4, 4)
  MLA_CASE(kFP8, 2, 2, 4)
  MLA_CASE(kFP8, 4, 1, 3)
#undef MLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace mla
