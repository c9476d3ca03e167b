// MLA decode attention over the latent cache (split-K partials).
//
// One workgroup streams a contiguous range of the tiles of all sequences (a
// share of their concatenation, each sequence start counted as some tiles of
// work; see the work plan) through an LDS ring filled by asynchronous
// global->LDS copies. Every
// 32-token tile of 576-wide latent rows is read from HBM once and used from
// LDS by all heads of the workgroup for both contractions (discosf explainer,
// "long-context bottleneck": W_UK folds into the query and W_UV into the
// output, so scores and values both come from the same latent rows):
//   scores  S^T[t][h] = c_t . q_lat[h] + k_pe_t . q_pe[h]  (MFMA, A = tile rows)
//   values  O^T[d][h] += sum_t c_t[d] p[t][h]              (MFMA, A = tile^T)
// with an online softmax per head in between. When a range ends or crosses a
// sequence boundary the segment's (m, l, o_lat / l) is written to a partial
// slot; the merge + W_UV launch combines the slots of each sequence.
#include <type_traits>

#include "attn_tile.h"

namespace mla {

template <int CT, int HB, int DS, int NSTAGE, bool PAGED>
__global__ void __launch_bounds__(64 * HB * DS)
mla_attn_kernel(AttnParams p) {
  constexpr int NW = HB * DS;
  constexpr int TILE = Tr<CT>::kTile;
  constexpr int RB = Tr<CT>::kRowBytes;
  constexpr int RP = Tr<CT>::kPad;
  constexpr int STAGE_DATA = TileCopy<CT, NW>::STAGE_DATA;
  constexpr int STAGE_BYTES = TileCopy<CT, NW>::STAGE_BYTES;
  constexpr bool WIDEN = (CT == kFP8 || CT == kFP6);     // codes widened to bf16 in LDS
  constexpr int CONV_BYTES = WIDEN ? TILE * kConvPad : 0;
  constexpr int CPW = TileCopy<CT, NW>::CPW;             // copies per wave per tile
  constexpr int DSLICE = kDc / DS;
  constexpr int NB = DSLICE / 16;
  // Split scores: with one 16-head block shared by four waves, wave w
  // computes the scores of token block (w & 1) over half of the 576-wide
  // contraction (w >> 1) and the four fp32 partials meet in LDS, so each
  // score MFMA and each tile read for scores happens once per workgroup.
  constexpr bool SK = (CT != kF32) && HB == 1 && DS == 4;
  constexpr int SX_BYTES = SK ? 4096 : 0;
  static_assert(NSTAGE >= 2, "ring needs two stages");
  static_assert(CT == kF32 || SK, "bf16/fp8 caches: one 16-head block over four waves");

  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE_BYTES + CONV_BYTES + SX_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int hb = wave % HB;
  const int ds = wave / HB;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int H = p.H;
  const int B = p.B;
  const int h = (blockIdx.y * HB + hb) * 16 + l16;       // head of this lane
  const int64_t w = blockIdx.x;
  int64_t r_hi;
  const Cursor c0 = cursor_start<TILE, PAGED>(p, w, lane, r_hi);
  if (c0.b < 0) return;                                  // whole workgroup

  TileCopy<CT, NW> cp;
  cp.init(wave, lane);

  auto issue = [&](const Cursor& c, int stage) {
    cp.issue(p.rows, p.row_scale, c, smem + stage * STAGE_BYTES, lane);
  };

  // ---- per-lane query fragments (B operand of the score MFMA) ----
  typedef typename std::conditional<CT == kF32, float, bf16x8>::type QFrag;
  constexpr int NQ = (CT == kF32) ? kDrow / 4 : (SK ? 9 : kDrow / 32);
  const int k_first = SK ? 9 * (wave >> 1) : 0;          // first 32-wide k-step of this wave
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
      for (int i = 0; i < NQ; ++i) {
        const int ks = k_first + i;                      // k-steps 16, 17 are the RoPE part
        q[i] = ks < 16 ? *(const bf16x8*)(ql + 32 * ks + 8 * g)
                       : *(const bf16x8*)(qp + 32 * (ks - 16) + 8 * g);
      }
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
      lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
    }
  }

  // ---- softmax state ----
  float m_run = -INFINITY;   // running max of this lane's head (log2 domain)
  float l_run = 0.f;         // this lane's share of the running sum
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane operand bases (bytes from the tile start)
  constexpr int TP = WIDEN ? kConvPad : RP;              // row pitch of the tile computed on
  const uint32_t s_base = (uint32_t)(l16 * TP + g * 16);                   // score A rows
  const uint32_t v_base = (uint32_t)(4 * g * TP + (ds * DSLICE + l16) * (CT == kF32 ? 4 : 2));
  // transposing value reads: source lane (g, l16) points at row 4g + l16/4,
  // dims ds*DSLICE + 4*(l16%4) .. +3 of the tile computed on
  const uint32_t tr_lane = (uint32_t)((4 * g + (l16 >> 2)) * TP + 2 * ds * DSLICE + 8 * (l16 & 3));
  s16x4 vlo[8], vhi[8];

  Cursor cc = c0;
  int it = 0;
  while (true) {
    wait_tiles<CPW, NSTAGE - 2>(issued - 1 - it);       // this wave's copies of tile `it` landed
    barrier_lds();                                       // tile `it` visible; stage it-1 free
    // bf16/fp8: the next tile's copies are spread over the score steps so the
    // wave is not stalled on the memory pipeline by a burst of them
    const bool do_copy = lvalid;
    typename TileCopy<CT, NW>::Pending pend;
    if (lvalid) {
      if constexpr (CT == kF32)
        issue(lc, issued % NSTAGE);
      else
        pend = cp.prepare(p.rows, p.row_scale, lc, smem + (issued % NSTAGE) * STAGE_BYTES);
      ++issued;
      lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
    }
    const char* stage = smem + (it % NSTAGE) * STAGE_BYTES;
    const int64_t left = cc.t_end - cc.t;
    const int nvalid = left < TILE ? (int)left : TILE;

    const char* tb = stage;                              // bf16/f32 rows of this tile
    if constexpr (WIDEN) {
      // widen the codes to bf16 once for all waves (fp6: block scales applied)
      char* conv = smem + NSTAGE * STAGE_BYTES;
      if constexpr (CT == kFP8) widen_fp8_tile<64 * NW>(stage, conv);
      else widen_fp6_tile<64 * NW>(stage, conv);
      barrier_lds();
      tb = conv;
    }

    if constexpr (CT != kF32) {
      // ---------------- scores: two 16-token blocks ----------------
      const uint32_t tr_addr = (uint32_t)(size_t)tb + tr_lane;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const char* sa = tb + s_base;
      {
        // this wave: token block (wave & 1), k-steps [k_first, k_first + 9)
        const char* sk = sa + (wave & 1) * 16 * TP + k_first * 64;
        bf16x8 av[9];
#pragma unroll
        for (int j = 0; j < 9; ++j) av[j] = *(const bf16x8*)(sk + j * 64);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 pa = {0.f, 0.f, 0.f, 0.f}, pc = {0.f, 0.f, 0.f, 0.f};   // two independent chains
#pragma unroll
        for (int j = 0; j < 9; ++j) {
          if (j & 1) pc = mfma_bf16_k32(av[j], q[j], pc);
          else pa = mfma_bf16_k32(av[j], q[j], pa);
          if (do_copy) {
#pragma unroll
            for (int i = 0; i < CPW; ++i)
              if (i * 9 / CPW == j) cp.copy(pend, i);
          }
        }
        // value operands of this tile, read while the score MFMAs run
        pv_read4<TP, 0>(tr_addr, vlo, vhi);
        pv_read4<TP, 4>(tr_addr, vlo + 4, vhi + 4);
        const f32x4 part = pa + pc;
        char* sx = smem + NSTAGE * STAGE_BYTES + CONV_BYTES;
        *(f32x4*)(sx + wave * 1024 + lane * 16) = part;
        barrier_lds();
        const f32x4 p0 = *(const f32x4*)(sx + 0 * 1024 + lane * 16);
        const f32x4 p1 = *(const f32x4*)(sx + 1 * 1024 + lane * 16);
        const f32x4 p2 = *(const f32x4*)(sx + 2 * 1024 + lane * 16);
        const f32x4 p3 = *(const f32x4*)(sx + 3 * 1024 + lane * 16);
        s0 = p0 + p2;
        s1 = p1 + p3;
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
        sc[r] = s0[r] * (p.scale_log2 * tsc[r]);
        sc[4 + r] = s1[r] * (p.scale_log2 * tsc[4 + r]);
      }
      if (nvalid < TILE) {                               // tail tile: mask rows past the end
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (4 * g + r >= nvalid) sc[r] = -INFINITY;
          if (16 + 4 * g + r >= nvalid) sc[4 + r] = -INFINITY;
        }
      }
      float tmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = __builtin_fmaxf(tmax, sc[i]);
      tmax = max_over_groups(tmax);
      // Lazy rescaling: the reference max moves only when a score exceeds it
      // by more than 2^kSlack, so p = 2^(s - m_run) <= 2^kSlack stays finite
      // and the accumulators are rescaled rarely (the result is unchanged:
      // o and l always share the reference m_run).
      if (__any(tmax > m_run + kSlack)) {
        const float m_new = __builtin_fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(sc[i] - m_use);
        psum += e;
        pv[i] = e * tsc[i];                              // fp8: value scale folded into P
      }
      l_run += psum;
      const bf16x8 pb = pack_bf16x8(pv);

      // ---------------- values: O^T += tile^T P^T ----------------
      // A operand (tile^T): lane (d, g) holds c_t[d] for t = 4g+q (low half)
      // and 16+4g+q (high half), from transposing LDS reads.
      auto pv_mfma = [&](int nb, const s16x4& lo, const s16x4& hi) {
        const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[nb] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a8), pb, o[nb]);
      };
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) pv_mfma(nb, vlo[nb], vhi[nb]);
    } else {
      // ---------------- f32 cache: one 16-token block ----------------
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
      const char* sa = tb + (l16 * RP + g * 4);
#pragma unroll
      for (int ks = 0; ks < kDrow / 4; ++ks) s0 = mfma_f32_k4(*(const float*)(sa + ks * 16), q[ks], s0);
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
      const char* va = tb + v_base;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[nb] = mfma_f32_k4(*(const float*)(va + r * RP + nb * 64), pv[r], o[nb]);
    }

    // ---------------- segment end: write the partial ----------------
    const bool seg_end = (cc.t + TILE >= cc.t_end);
    if (seg_end) {
      const float lsum = sum_over_groups(l_run);
      const int64_t slot = w + cc.b;
      const float inv = inv_or_zero(lsum);
      const int64_t po = (slot * H + h) * kDc + ds * DSLICE + 4 * g;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) store_part4<CT>(p.part_o, po + nb * 16, o[nb], inv);
      if (ds == 0 && g == 0) {
        p.part_ml[(slot * H + h) * 2 + 0] = m_run;
        p.part_ml[(slot * H + h) * 2 + 1] = lsum;
      }
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (!advance<TILE, PAGED>(cc, p, r_hi, lane)) break;
    if (seg_end) {
      load_q(cc.b);
      wait_vmcnt<0>();
    }
    ++it;
  }
}

// Pair kernel, for head counts that are multiples of 32 over an fp8 cache
// (bf16 and fp6 caches run mla_attn_pair2_kernel below, which shares the
// softmax between the two waves of a pair).
// Two waves share 32 heads (two 16-head MFMA blocks): for the scores each
// wave contracts one half of the 576-wide rows (k-steps 0..8 or 9..17) and
// the two fp32 partials meet in LDS; for the values each wave accumulates
// one half of the 512 latent dims. Every tile operand a wave reads from LDS
// then feeds two MFMAs (one per head block), and the per-wave registers are
// 72 for the query half and 128 for the output half, so NP pairs (up to 128
// heads) run as 2*NP waves of one workgroup, two waves per SIMD at NP = 4,
// and each tile is fetched from HBM once for all of them.
//
// F8 (fp8 cache): the value contraction on fp8 MFMA (K = 32 tokens, the
// tile's codes straight from the transposing reads). The value weights
// p * scale_t become e4m3 codes, the one extra rounding of this variant
// (about 2% relative error in the output): they are multiplied by 2^G, G the
// segment's exponent that keeps scale_t * 2^G <= 2^kF8Lift for every row
// seen (lowered, with a power-of-two rescale of o, when a tile has a larger
// scale), and the lazy max keeps a slack of 2^(8 - kF8Lift), so that every
// weight is at most 256 and the largest near 2^kF8Lift or more, away from the
// format's subnormals; the output is divided by 2^G at the end.
template <int CT, int NP, int NSTAGE, bool PAGED, bool F8>
__global__ void __launch_bounds__(128 * NP)
mla_attn_pair_kernel(AttnParams p) {
  static_assert(CT == kFP8, "pair kernel: fp8 cache");
  constexpr int kF8Lift = 4;
  constexpr float kSlackP = F8 ? (float)(8 - kF8Lift) : kSlack;
  constexpr int NW = 2 * NP;
  constexpr int TILE = 32;
  constexpr int RP = Tr<CT>::kPad;
  constexpr int STAGE_DATA = TileCopy<CT, NW>::STAGE_DATA;
  constexpr int STAGE_BYTES = TileCopy<CT, NW>::STAGE_BYTES;
  constexpr int CPW = TileCopy<CT, NW>::CPW;
  constexpr int X_BYTES = NW * 4096;                     // one 32x32 fp32 partial per wave
  constexpr int TP = RP;                                 // row pitch of the staged tile
  static_assert(NSTAGE >= 2, "ring needs two stages");
  static_assert(Tr<CT>::kTile == TILE, "32-token tiles");

  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE_BYTES + X_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int half = wave & 1;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int H = p.H;
  const int B = p.B;
  const int hp = (blockIdx.y * NP + (wave >> 1)) * 32;  // first head of the pair
  const int64_t w = blockIdx.x;
  int64_t r_hi;
  const Cursor c0 = cursor_start<TILE, PAGED>(p, w, lane, r_hi);
  if (c0.b < 0) return;                                  // whole workgroup

  TileCopy<CT, NW> cp;
  cp.init(wave, lane);
  auto issue = [&](const Cursor& c, int stage) {
    cp.issue(p.rows, p.row_scale, c, smem + stage * STAGE_BYTES, lane);
  };

  // query fragments (B operand of the score MFMA): head block hb, k-step j of
  // this wave's half of the row (elements 288*half ..): k-steps 2m and 2m+1
  // (m < 4) hold elements 64m + 16g .. +7 and 64m + 16g + 8 .. +15 for lane
  // group g, so that one 16-byte read of the codes feeds both; k-step 8 is
  // 256 + 8g .. +7 (the contraction runs over the row's elements in another
  // order than mla_attn_pair2_kernel's, with the same result up to rounding)
  auto q_elem = [&](int j, int gg) {
    if (j < 8) return 288 * half + 64 * (j >> 1) + 16 * gg + 8 * (j & 1);
    return 288 * half + 32 * j + 8 * gg;
  };
  bf16x8 q[2][9];
  auto load_q = [&](int b) {
    const int ln = opaque(lane);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int64_t base = (int64_t)b * H + hp + 16 * hb + (ln & 15);
      const __bf16* ql = (const __bf16*)p.q_lat + base * kDc;
      const __bf16* qp = (const __bf16*)p.q_pe + base * kDr;
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int e = q_elem(j, ln >> 4);                // elements 512.. are the RoPE part
        const __bf16* src = e < kDc ? ql + e : qp + (e - kDc);
        q[hb][j] = *(const bf16x8*)src;
      }
    }
  };
  // After a wait that covers the query loads: an empty asm that reads and
  // rewrites every query register, so that no path the compiler cannot rule
  // out (it does not correlate the branches that issue copies and loads)
  // leaves a query load outstanding in its wait counting; otherwise every
  // tile's score MFMAs would wait for all copies issued before them.
  auto settle_q = [&]() {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 9; ++j) asm volatile("" : "+v"(q[hb][j]));
  };
  // the first tile's copies, the queries, then the other prologue tiles'
  // copies (the empty asm keeps the compiler from hoisting the query loads
  // above the first copies, whose address arithmetic it would then make wait
  // for them). A worker with fewer tiles than the prologue copies its first
  // tile again into the unused stages, so that every path issues the same
  // number of copies after the queries and one wait covers them: with a query
  // load outstanding on some path into the loop, the compiler's wait counting
  // would make every tile's score MFMAs wait for all copies issued before them
  Cursor lc = c0;
  issue(lc, 0);
  bool lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
  {
    int b0 = c0.b;
    asm volatile("" : "+s"(b0) :: "memory");
    load_q(b0);
  }
#pragma unroll
  for (int i = 1; i < NSTAGE - 1; ++i) {
    issue(lvalid ? lc : c0, i);
    if (lvalid) lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
  }
  int issued = NSTAGE - 1;
  // the queries and the first tile land here; later prologue tiles may stay
  // in flight
  wait_vmcnt<(NSTAGE - 2) * CPW>();
  settle_q();

  float m_run[2] = {-INFINITY, -INFINITY};   // running max per head block (log2 domain)
  float l_run[2] = {0.f, 0.f};               // this lane's share of the running sums
  f32x4 o[2][16];                            // O^T: dims 256*half + 16*nb + 4g + r, head l16
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // score A operand: tile row l16 (+16 for the second token block), k-step 9*half
  const uint32_t s_base = (uint32_t)(l16 * TP + half * 288);
  // transposing value reads: source lane (g, l16) points at row T(g, l16/2),
  // dims 256*half + 8*(l16%2) .. +7, with T(g, q) = 4g + q for q < 4 and
  // 16 + 4g + (q - 4) otherwise, so that lane (n, g) receives dim n of
  // tokens 4g..4g+3 and 16+4g..16+4g+3: the token order of the P operand
  const int tq = l16 >> 1;
  const uint32_t tr_lane =
      (uint32_t)(((tq < 4 ? 4 * g + tq : 16 + 4 * g + tq - 4)) * TP + 256 * half + 8 * (l16 & 1));
  char* xbuf = smem + NSTAGE * STAGE_BYTES;
  // F8: exponent G of the value weights (a large start: the first tile of a
  // segment lowers it)
  constexpr int kGStart = 127;
  int gexp = kGStart;

  // a segment change loads the next queries and then stores the partial
  // (at least kStoreOps stores); the stores may stay in flight into the next
  // tile
  constexpr int kStoreOps = 32;
  constexpr int kTileWait = (NSTAGE - 2) * CPW;
  constexpr int kSegExtra = kStoreOps < 63 - kTileWait ? kStoreOps : 63 - kTileWait;
  Cursor cc = c0;
  int it = 0;
  bool after_seg = false;
  while (true) {
    // this wave's copies of tile `it` landed
    if (after_seg) wait_tiles_extra<CPW, NSTAGE - 2, kSegExtra>(issued - 1 - it);
    else wait_tiles<CPW, NSTAGE - 2>(issued - 1 - it);
    barrier_lds();                                       // tile visible; stage it-1 and xbuf free
    // the next tile's copies go out after this wave's score MFMAs are issued
    const bool do_copy = lvalid;
    typename TileCopy<CT, NW>::Pending pend;
    if (do_copy) {
      pend = cp.prepare(p.rows, p.row_scale, lc, smem + (issued % NSTAGE) * STAGE_BYTES);
      ++issued;
      lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
    }
    const char* stage = smem + (it % NSTAGE) * STAGE_BYTES;
    const int64_t left = cc.t_end - cc.t;
    const int nvalid = left < TILE ? (int)left : TILE;
    const char* tb = stage;

    // ---------------- scores: this wave's half of the contraction ----------------
    f32x4 acc[2][2];                                     // [token block][head block]
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const char* sa = tb + s_base;
    // one batch of nine k-steps: the compiler places the 18 operand reads
    // among the 36 MFMAs as registers allow (measured: batches of two with a
    // scheduling barrier between them left the matrix unit idle longer)
    // fp8: 16-byte reads of the codes, two k-steps each (the last k-step an
    // 8-byte read), in small asm batches the compiler does not see (a visible
    // LDS read here would make it wait for every copy in flight), widened in
    // registers
    u32x4 c8[2][4];
    const uint32_t a16 = (uint32_t)(size_t)sa + 16 * g;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      bf16x8 a0, a1;
      {                                                  // codes widened in registers
        uint2 u0, u1;
        if (k < 8) {
          if (k == 0) lds_read_b128_x2<0, 16 * TP>(a16, c8[0][0], c8[1][0]);
          if (k == 2) lds_read_b128_x2<64, 16 * TP + 64>(a16, c8[0][1], c8[1][1]);
          if (k == 4) lds_read_b128_x2<128, 16 * TP + 128>(a16, c8[0][2], c8[1][2]);
          if (k == 6) lds_read_b128_x2<192, 16 * TP + 192>(a16, c8[0][3], c8[1][3]);
          const u32x4 v0 = c8[0][k >> 1], v1 = c8[1][k >> 1];
          u0 = (k & 1) ? uint2{v0[2], v0[3]} : uint2{v0[0], v0[1]};
          u1 = (k & 1) ? uint2{v1[2], v1[3]} : uint2{v1[0], v1[1]};
        } else {
          lds_read_b64_x2<0, 16 * TP>((uint32_t)(size_t)sa + 256 + 8 * g, u0, u1);
        }
        a0 = fp8x8_to_bf16x8(u0);
        a1 = fp8x8_to_bf16x8(u1);
      }
      acc[0][0] = mfma_bf16_k32(a0, q[0][k], acc[0][0]);
      acc[0][1] = mfma_bf16_k32(a0, q[1][k], acc[0][1]);
      acc[1][0] = mfma_bf16_k32(a1, q[0][k], acc[1][0]);
      acc[1][1] = mfma_bf16_k32(a1, q[1][k], acc[1][1]);
    }
    // the next tile's copies, after this wave's score work is issued
    if (do_copy) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) cp.copy(pend, i);
    }
    // exchange partials with the other wave of the pair (a + b == b + a, so
    // both waves hold bit-identical scores and take identical decisions)
    char* xw = xbuf + wave * 4096 + lane * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(f32x4*)(xw + i * 1024) = acc[i >> 1][i & 1];
    barrier_lds();
    const char* xp = xbuf + (wave ^ 1) * 4096 + lane * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i >> 1][i & 1] += *(const f32x4*)(xp + i * 1024);

    // ---------------- online softmax per head block ----------------
    // row scales of tokens 4g.. and 16 + 4g..
    u32x4 scl8[2];
    lds_read_b128_x2<0, 64>((uint32_t)(size_t)(stage + STAGE_DATA) + 16 * g, scl8[0], scl8[1]);
    float tsc[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // (the element goes through a plain variable: a bit cast of a vector
      // element expression read the vector's first element here)
      const unsigned int w0 = scl8[0][r], w1 = scl8[1][r];
      tsc[r] = __builtin_bit_cast(float, w0);
      tsc[4 + r] = __builtin_bit_cast(float, w1);
    }
    float sc[2][8];
    float tmax[2];
    bool grow = false;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[hb][r] = acc[0][hb][r] * (p.scale_log2 * tsc[r]);
        sc[hb][4 + r] = acc[1][hb][r] * (p.scale_log2 * tsc[4 + r]);
      }
      if (nvalid < TILE) {                               // tail tile: mask rows past the end
        const int g4 = 4 * (opaque(lane) >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (g4 >= nvalid - r) sc[hb][r] = -INFINITY;
          if (g4 >= nvalid - 16 - r) sc[hb][4 + r] = -INFINITY;
        }
      }
      float t = sc[hb][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) t = __builtin_fmaxf(t, sc[hb][i]);
      tmax[hb] = max_over_groups(t);
      grow = grow || (tmax[hb] > m_run[hb] + kSlackP);
    }
    // F8: a tile whose largest row scale exceeds 2^(kF8Lift - G) lowers G
    // (o follows)
    float gshift = 1.f;
    if constexpr (F8) {
      float tm = tsc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tm = __builtin_fmaxf(tm, tsc[i]);
      tm = max_over_groups(tm);                          // all 32 rows of the tile
      // tm < 2^e (e = frexp exponent), so tm * 2^(kF8Lift - e) < 2^kF8Lift
      const int gneed = kF8Lift - uniform(__builtin_amdgcn_frexp_expf(tm));
      if (gneed < gexp) {
        gshift = __builtin_amdgcn_ldexpf(1.f, gneed - gexp);
        gexp = gneed;
      }
    }
    // lazy rescale: the reference max moves only when a score exceeds it by
    // more than 2^kSlack (o and l always share the reference)
    if (__any(grow) || (F8 && gshift != 1.f)) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float m_new = __builtin_fmaxf(m_run[hb], tmax[hb]);
        float alpha = __builtin_amdgcn_exp2f(m_run[hb] - m_new);
        if (F8 && m_new == m_run[hb]) alpha = 1.f;       // (also when both are -inf)
        l_run[hb] *= alpha;
        const float ao = F8 ? alpha * gshift : alpha;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) o[hb][nb] *= ao;
        m_run[hb] = m_new;
      }
    }
    bf16x8 pb[2];
    uint2 p8[2];                                         // F8: e4m3 codes of the value weights
    if constexpr (F8) {
      const float g2 = __builtin_amdgcn_ldexpf(1.f, gexp);
#pragma unroll
      for (int i = 0; i < 8; ++i) tsc[i] *= g2;          // below 2^kF8Lift
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float m_use = (m_run[hb] == -INFINITY) ? 0.f : m_run[hb];
      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(sc[hb][i] - m_use);
        psum += e;
        pv[i] = e * tsc[i];                              // fp8: value scale folded into P
      }
      l_run[hb] += psum;
      if constexpr (F8)
        p8[hb] = uint2{f32x4_to_fp8x4(pv[0], pv[1], pv[2], pv[3]),
                       f32x4_to_fp8x4(pv[4], pv[5], pv[6], pv[7])};
      else
        pb[hb] = pack_bf16x8(pv);
    }

    // ---------------- values: O^T += tile^T P^T, this wave's 256 dims ----------------
    const uint32_t tr_addr = (uint32_t)(size_t)tb + tr_lane;
#pragma unroll
    for (int n0 = 0; n0 < 16; n0 += 4) {
      if constexpr (F8) {                                // codes straight into fp8 MFMA
        uint2 v[4];
        lds_tr8_x4<0, 16, 32, 48>(tr_addr + n0 * 16, v[0], v[1], v[2], v[3]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[0][n0 + k] = mfma_fp8_k32(v[k], p8[0], o[0][n0 + k]);
          o[1][n0 + k] = mfma_fp8_k32(v[k], p8[1], o[1][n0 + k]);
        }
        continue;
      }
      bf16x8 a[4];
      {
        uint2 v[4];
        lds_tr8_x4<0, 16, 32, 48>(tr_addr + n0 * 16, v[0], v[1], v[2], v[3]);
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = fp8x8_to_bf16x8(v[k]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[0][n0 + k] = mfma_bf16_k32(a[k], pb[0], o[0][n0 + k]);
        o[1][n0 + k] = mfma_bf16_k32(a[k], pb[1], o[1][n0 + k]);
      }
    }

    // ---------------- segment end: write the partial ----------------
    const bool seg_end = (cc.t + TILE >= cc.t_end);
    if (seg_end) {
      // the next segment's queries go out before the partial's stores, so
      // that the wait for them below leaves the stores in flight
      const int nseq = next_segment_seq<PAGED>(cc, p, r_hi);
      if (nseq >= 0) load_q(nseq);
      __builtin_amdgcn_sched_barrier(0);
      const int64_t slot = w + cc.b;
      const int ln = opaque(lane);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float lsum = sum_over_groups(l_run[hb]);
        const int h = hp + 16 * hb + (ln & 15);
        float inv = inv_or_zero(lsum);
        if constexpr (F8) inv *= __builtin_amdgcn_ldexpf(1.f, -gexp);
        const int64_t po = (slot * H + h) * kDc + 256 * half + 4 * (ln >> 4);
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) store_part4<CT>(p.part_o, po + nb * 16, o[hb][nb], inv);
        if (half == 0 && (ln >> 4) == 0) {
          p.part_ml[(slot * H + h) * 2 + 0] = m_run[hb];
          p.part_ml[(slot * H + h) * 2 + 1] = lsum;
        }
        m_run[hb] = -INFINITY;
        l_run[hb] = 0.f;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // the queries have landed (at least kStoreOps stores follow them);
      // the stores may stay in flight
      wait_vmcnt<kStoreOps>();
      settle_q();
      gexp = kGStart;
    }
    if (!advance<TILE, PAGED>(cc, p, r_hi, lane)) break;
    after_seg = seg_end;
    ++it;
  }
}

// Pair kernel with the softmax shared between the two waves of a pair and
// the value product one tile behind the scores. Same contractions and the
// same work split as mla_attn_pair_kernel; what changes:
//  * each wave runs the online softmax of one of the pair's two 16-head
//    blocks (wave half 0: heads 0..15 of the pair, half 1: heads 16..31):
//    the score partials cross in LDS only for the other wave's block, and
//    the probabilities (bf16), the rescale factor and the running sum of
//    each block go to the other wave through LDS;
//  * the values of tile t run after the barrier that opens tile t+1, so
//    that barrier also publishes tile t's probabilities (no extra barrier);
//    tile t's stage (and, for fp6, its widened copy) stays in LDS until
//    then, and the copies into that stage go out after the score exchange
//    of tile t+1, which every wave reaches only after its values of tile t;
//  * a segment's last tile loads the next segment's queries right after its
//    score MFMAs, so they arrive during the exchange and the softmax.
template <int CT, int NP, int NSTAGE, bool PAGED>
__global__ void __launch_bounds__(128 * NP)
mla_attn_pair2_kernel(AttnParams p) {
  static_assert(CT == kBF16 || CT == kFP6, "shared-softmax pair kernel: bf16 or fp6 cache");
  constexpr int CONV_BYTES = (CT == kFP6) ? 2 * 32 * kConvPad : 0;   // two widened tiles
  constexpr int NW = 2 * NP;
  constexpr int TILE = 32;
  constexpr int RP = Tr<CT>::kPad;
  constexpr int STAGE_BYTES = TileCopy<CT, NW>::STAGE_BYTES;
  constexpr int CPW = TileCopy<CT, NW>::CPW;
  constexpr int X_BYTES = NW * 2048;                     // the other block's 32x16 fp32 partial
  constexpr int P_BYTES = NW * 1536;                     // probabilities, alpha, running sum
  constexpr int TP = (CT == kFP6) ? kConvPad : RP;       // row pitch of the tile computed on
  static_assert(NSTAGE >= 3, "a tile stays until the next tile's exchange");
  static_assert(Tr<CT>::kTile == TILE, "32-token tiles");

  __shared__ __attribute__((aligned(1024)))
      char smem[NSTAGE * STAGE_BYTES + X_BYTES + P_BYTES + CONV_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int half = wave & 1;                             // also this wave's softmax head block
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int H = p.H;
  const int B = p.B;
  const int hp = (blockIdx.y * NP + (wave >> 1)) * 32;  // first head of the pair
  const int64_t w = blockIdx.x;
  int64_t r_hi;
  const Cursor c0 = cursor_start<TILE, PAGED>(p, w, lane, r_hi);
  if (c0.b < 0) return;                                  // whole workgroup

  TileCopy<CT, NW> cp;
  cp.init(wave, lane);
  auto issue = [&](const Cursor& c, int stage) {
    cp.issue(p.rows, p.row_scale, c, smem + stage * STAGE_BYTES, lane);
  };

  // query fragments (B operand of the score MFMA): head block hb, k-step j of
  // this wave's half of the row (elements 288*half ..): lane group g holds
  // elements 32j + 8g .. +7 of the half
  auto q_elem = [&](int j, int gg) { return 288 * half + 32 * j + 8 * gg; };
  bf16x8 q[2][9];
  auto load_q = [&](int b) {
    const int ln = opaque(lane);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int64_t base = (int64_t)b * H + hp + 16 * hb + (ln & 15);
      const __bf16* ql = (const __bf16*)p.q_lat + base * kDc;
      const __bf16* qp = (const __bf16*)p.q_pe + base * kDr;
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int e = q_elem(j, ln >> 4);
        const __bf16* src = e < kDc ? ql + e : qp + (e - kDc);
        q[hb][j] = *(const bf16x8*)src;
      }
    }
  };
  auto settle_q = [&]() {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 9; ++j) asm volatile("" : "+v"(q[hb][j]));
  };
  Cursor lc = c0;
  issue(lc, 0);
  bool lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
  {
    int b0 = c0.b;
    asm volatile("" : "+s"(b0) :: "memory");
    load_q(b0);
  }
#pragma unroll
  for (int i = 1; i < NSTAGE - 1; ++i) {
    issue(lvalid ? lc : c0, i);
    if (lvalid) lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
  }
  int issued = NSTAGE - 1;
  wait_vmcnt<(NSTAGE - 2) * CPW>();
  settle_q();

  float m_own = -INFINITY;     // running max of this wave's head block (log2 domain)
  float l_own = 0.f;           // this lane's share of its running sum
  f32x4 o[2][16];              // O^T: dims 256*half + 16*nb + 4g + r, head l16 of block hb
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // score A operand: tile row l16 (+16 for the second token block), k-step 9*half
  const uint32_t s_base = (uint32_t)(l16 * TP + g * 16 + half * 9 * 64);
  // transposing value reads: source lane (g, l16) points at row 4g + l16/4,
  // dims 256*half + 4*(l16%4) .. +3
  const uint32_t tr_lane = (uint32_t)((4 * g + (l16 >> 2)) * TP + 2 * 256 * half + 8 * (l16 & 3));
  char* xbuf = smem + NSTAGE * STAGE_BYTES;
  char* pbuf = xbuf + X_BYTES;
  char* conv = pbuf + P_BYTES;                           // fp6: two widened tiles
  (void)conv;
  // this wave's slots: partial for the other block, probabilities (16 B per
  // lane), alpha and running sum (4 B per lane each)
  char* xw = xbuf + wave * 2048 + lane * 16;
  const char* xp = xbuf + (wave ^ 1) * 2048 + lane * 16;
  char* pw = pbuf + wave * 1536;
  const char* pp = pbuf + (wave ^ 1) * 1536;

  // the previous tile, whose values are still to be added
  bool have_prev = false;
  const char* prev_tb = nullptr;
  bf16x8 pb_own = {};
  bool prev_seg_end = false;
  int prev_b = 0;

  // values of the previous tile (both head blocks of this wave's 256 dims),
  // then, at its segment's end, the partial
  auto finish_prev = [&]() {
    const bf16x8 pb_oth = *(const bf16x8*)(pp + lane * 16);
    const float a_oth = *(const float*)(pp + 1024 + lane * 4);
    const float l_oth = *(const float*)(pp + 1280 + lane * 4);
    if (__any(a_oth != 1.f)) {                           // the other block's max moved
      const float a0 = half ? a_oth : 1.f, a1 = half ? 1.f : a_oth;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) {
        o[0][nb] *= a0;
        o[1][nb] *= a1;
      }
    }
    const bf16x8 pb0 = half ? pb_oth : pb_own;
    const bf16x8 pb1 = half ? pb_own : pb_oth;
    const uint32_t tr_addr = (uint32_t)(size_t)prev_tb + tr_lane;
#pragma unroll
    for (int n0 = 0; n0 < 16; n0 += 4) {
      bf16x8 a[4];
      {
        s16x4 lo[4], hi[4];
        pv_read4<TP, 0>(tr_addr + n0 * 32, lo, hi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const s16x8 a8 = {lo[k][0], lo[k][1], lo[k][2], lo[k][3], hi[k][0], hi[k][1], hi[k][2], hi[k][3]};
          a[k] = __builtin_bit_cast(bf16x8, a8);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[0][n0 + k] = mfma_bf16_k32(a[k], pb0, o[0][n0 + k]);
        o[1][n0 + k] = mfma_bf16_k32(a[k], pb1, o[1][n0 + k]);
      }
    }
    if (prev_seg_end) {
      const int64_t slot = w + prev_b;
      const int ln = opaque(lane);
      const float ls_own = sum_over_groups(l_own);
      const float ls_oth = sum_over_groups(l_oth);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float lsum = (hb == half) ? ls_own : ls_oth;
        const int h = hp + 16 * hb + (ln & 15);
        const float inv = inv_or_zero(lsum);
        const int64_t po = (slot * H + h) * kDc + 256 * half + 4 * (ln >> 4);
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) store_part4<CT>(p.part_o, po + nb * 16, o[hb][nb], inv);
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if ((ln >> 4) == 0) {                              // the block's owner writes (m, l)
        const int h = hp + 16 * half + (ln & 15);
        p.part_ml[(slot * H + h) * 2 + 0] = m_own;
        p.part_ml[(slot * H + h) * 2 + 1] = ls_own;
      }
      m_own = -INFINITY;
      l_own = 0.f;
    }
  };

  Cursor cc = c0;
  int it = 0;
  while (true) {
    // this wave's copies of tile `it` landed
    wait_tiles<CPW, NSTAGE - 2>(issued - 1 - it);
    barrier_lds();            // tile `it` and the previous tile's probabilities visible
    const bool do_copy = lvalid;
    typename TileCopy<CT, NW>::Pending pend;
    if (do_copy) {
      pend = cp.prepare(p.rows, p.row_scale, lc, smem + (issued % NSTAGE) * STAGE_BYTES);
      ++issued;
      lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
    }
    const char* stage = smem + (it % NSTAGE) * STAGE_BYTES;
    const int64_t left = cc.t_end - cc.t;
    const int nvalid = left < TILE ? (int)left : TILE;
    const char* tb = stage;
    if constexpr (CT == kFP6) {
      char* cv = conv + (it & 1) * (32 * kConvPad);
      widen_fp6_tile_async<128 * NP>(stage, cv);
      barrier_lds();
      tb = cv;
    }
    if (have_prev) finish_prev();

    // ---------------- scores: this wave's half of the contraction ----------------
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const char* sa = tb + s_base;
    // one batch of nine k-steps; the compiler places the 18 operand reads
    // among the 36 MFMAs as registers allow
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const bf16x8 a0 = *(const bf16x8*)(sa + k * 64);
      const bf16x8 a1 = *(const bf16x8*)(sa + 16 * TP + k * 64);
      acc[0][0] = mfma_bf16_k32(a0, q[0][k], acc[0][0]);
      acc[0][1] = mfma_bf16_k32(a0, q[1][k], acc[0][1]);
      acc[1][0] = mfma_bf16_k32(a1, q[0][k], acc[1][0]);
      acc[1][1] = mfma_bf16_k32(a1, q[1][k], acc[1][1]);
    }
    // a segment's last tile: the next segment's queries go out now
    const bool seg_end = (cc.t + TILE >= cc.t_end);
    const int nseq = seg_end ? next_segment_seq<PAGED>(cc, p, r_hi) : -1;
    if (nseq >= 0) load_q(nseq);
    __builtin_amdgcn_sched_barrier(0);
    // the other block's partial to the other wave; its partial of this block back
    const f32x4 x0 = half ? acc[0][0] : acc[0][1];
    const f32x4 x1 = half ? acc[1][0] : acc[1][1];
    *(f32x4*)(xw) = x0;
    *(f32x4*)(xw + 1024) = x1;
    barrier_lds();            // every wave's values of the previous tile are done
    f32x4 s0 = half ? acc[0][1] : acc[0][0];
    f32x4 s1 = half ? acc[1][1] : acc[1][0];
    s0 += *(const f32x4*)(xp);
    s1 += *(const f32x4*)(xp + 1024);
    // the freed stage (the previous tile's) takes the next tile
    if (do_copy) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) cp.copy(pend, i);
    }

    // ---------------- online softmax of this wave's head block ----------------
    float sc[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = s0[r] * p.scale_log2;
      sc[4 + r] = s1[r] * p.scale_log2;
    }
    if (nvalid < TILE) {
      const int g4 = 4 * (opaque(lane) >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (g4 >= nvalid - r) sc[r] = -INFINITY;
        if (g4 >= nvalid - 16 - r) sc[4 + r] = -INFINITY;
      }
    }
    float t = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) t = __builtin_fmaxf(t, sc[i]);
    const float tmax = max_over_groups(t);
    float alpha = 1.f;
    if (__any(tmax > m_own + kSlack)) {                  // lazy rescale (see the pair kernel)
      const float m_new = __builtin_fmaxf(m_own, tmax);
      alpha = __builtin_amdgcn_exp2f(m_own - m_new);
      l_own *= alpha;
      const float a0 = half ? 1.f : alpha, a1 = half ? alpha : 1.f;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) {
        o[0][nb] *= a0;
        o[1][nb] *= a1;
      }
      m_own = m_new;
    }
    const float m_use = (m_own == -INFINITY) ? 0.f : m_own;
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __builtin_amdgcn_exp2f(sc[i] - m_use);
      psum += e;
      pv[i] = e;
    }
    l_own += psum;
    pb_own = pack_bf16x8(pv);
    *(bf16x8*)(pw + lane * 16) = pb_own;
    *(float*)(pw + 1024 + lane * 4) = alpha;
    *(float*)(pw + 1280 + lane * 4) = l_own;

    have_prev = true;
    prev_tb = tb;
    prev_seg_end = seg_end;
    prev_b = (int)cc.b;
    if (!advance<TILE, PAGED>(cc, p, r_hi, lane)) break;
    if (seg_end) {
      // the next segment's queries have landed (the copies just issued, if
      // any, may stay in flight)
      if (do_copy) wait_vmcnt<CPW>();
      else wait_vmcnt<0>();
      settle_q();
    }
    ++it;
  }
  barrier_lds();              // the last tile's probabilities visible
  finish_prev();
}

// ------------------------------------------------------------------ launch
template <int CT, int NP, int NSTAGE, bool F8>
static void launch_pair_f(const AttnParams& prm, dim3 grid, dim3 block, hipStream_t s) {
  if constexpr (!F8 && CT != kFP8) {                   // bf16, fp6: the shared-softmax kernel
    if (prm.block_table)
      hipLaunchKernelGGL((mla_attn_pair2_kernel<CT, NP, NSTAGE, true>), grid, block, 0, s, prm);
    else
      hipLaunchKernelGGL((mla_attn_pair2_kernel<CT, NP, NSTAGE, false>), grid, block, 0, s, prm);
  } else {                                               // fp8 (and its fp8-MFMA variant)
    if (prm.block_table)
      hipLaunchKernelGGL((mla_attn_pair_kernel<CT, NP, NSTAGE, true, F8>), grid, block, 0, s, prm);
    else
      hipLaunchKernelGGL((mla_attn_pair_kernel<CT, NP, NSTAGE, false, F8>), grid, block, 0, s, prm);
  }
}
template <int CT, int NP, int NSTAGE>
static hipError_t launch_pair_t(const AttnParams& prm, bool f8, int workers, int head_groups,
                                hipStream_t s) {
  dim3 grid(workers, head_groups);
  dim3 block(128 * NP);
  if constexpr (CT == kFP8) {
    if (f8) launch_pair_f<CT, NP, NSTAGE, true>(prm, grid, block, s);
    else launch_pair_f<CT, NP, NSTAGE, false>(prm, grid, block, s);
  } else {
    (void)f8;
    launch_pair_f<CT, NP, NSTAGE, false>(prm, grid, block, s);
  }
  return hipGetLastError();
}

template <int CT, int HB, int DS, int NSTAGE>
static hipError_t launch_attn_t(const AttnParams& prm, int workers, int head_groups,
                                hipStream_t s) {
  dim3 grid(workers, head_groups);
  dim3 block(64 * HB * DS);
  if (prm.block_table)
    hipLaunchKernelGGL((mla_attn_kernel<CT, HB, DS, NSTAGE, true>), grid, block, 0, s, prm);
  else
    hipLaunchKernelGGL((mla_attn_kernel<CT, HB, DS, NSTAGE, false>), grid, block, 0, s, prm);
  return hipGetLastError();
}

hipError_t launch_attn(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  AttnParams prm;
  prm.rows = (const char*)a.rows;
  prm.row_scale = a.row_scale;
  prm.seqinfo = a.seqinfo;
  prm.winfo = a.winfo;
  prm.q_lat = a.q_lat;
  prm.q_pe = a.q_pe;
  prm.part_o = a.part_o;
  prm.part_ml = a.part_ml;
  prm.B = a.B;
  prm.H = a.H;
  prm.scale_log2 = a.softmax_scale * kLog2e;
  prm.block_table = a.block_table;
  prm.max_pages = a.max_pages;
  prm.page_tokens = a.page_tokens;
  prm.page_tiles = a.block_table ? a.page_tokens / plan.tile : 0;
  prm.page_limit = (uint32_t)(a.total_pages < (int64_t)1 << 31 ? a.total_pages : (int64_t)1 << 31);
  const int W = plan.workers, G = plan.head_groups;
  if (plan.stream) return launch_attn_stream(plan, prm, s);
  if (plan.h32) return launch_attn_h32(plan, prm, s);
#define MLA_CASE(CT_, HB_, DS_, NS_)                                              \
  if (!plan.pair && ct == CT_ && plan.hb == HB_ && plan.ds == DS_ && plan.nstage == NS_) \
    return launch_attn_t<CT_, HB_, DS_, NS_>(prm, W, G, s);
#define MLA_PAIR(CT_, NP_, NS_)                                                   \
  if (plan.pair && ct == CT_ && plan.np == NP_ && plan.nstage == NS_)             \
    return launch_pair_t<CT_, NP_, NS_>(prm, plan.f8, W, G, s);
  MLA_CASE(kF32, 1, 4, 2)
  MLA_CASE(kBF16, 1, 4, 4)
  MLA_CASE(kFP8, 1, 4, 4)
  MLA_CASE(kFP6, 1, 4, 4)
  MLA_PAIR(kBF16, 4, 3)
  MLA_PAIR(kBF16, 2, 3)
  MLA_PAIR(kBF16, 1, 4)
  MLA_PAIR(kFP8, 4, 4)
  MLA_PAIR(kFP8, 2, 4)
  MLA_PAIR(kFP8, 1, 4)
  MLA_PAIR(kFP6, 4, 3)
  MLA_PAIR(kFP6, 2, 3)
  MLA_PAIR(kFP6, 1, 3)
#undef MLA_PAIR
#undef MLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace mla
