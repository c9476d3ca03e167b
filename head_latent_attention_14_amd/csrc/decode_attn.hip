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
  const int64_t* starts;     // [W+1]
  const int32_t* wseq;       // [W]
  const void* q_lat;         // [B][H][512]  bf16 (f32 for the f32 cache)
  const void* q_pe;          // [B][H][64]
  float* part_o;             // [nslot][H][512]
  float* part_ml;            // [nslot][H][2]
  int32_t B;
  int32_t H;
  float scale_log2;          // softmax_scale * log2(e)
};

// Per cache dtype: bytes of a stored row, bytes of a padded LDS row, and
// tokens per tile. Rows in LDS are padded by 16 bytes so that the 16 rows one
// MFMA operand read touches start on different banks; every operand read is
// then a per-lane base plus a compile-time offset.
template <int CT> struct Tr;
template <> struct Tr<kBF16> { static constexpr int kRowBytes = 1152, kPad = 1168, kTile = 32; };
template <> struct Tr<kFP8> { static constexpr int kRowBytes = 576, kPad = 592, kTile = 32; };
template <> struct Tr<kF32> { static constexpr int kRowBytes = 2304, kPad = 2320, kTile = 16; };
constexpr int kConvPad = 1168;   // padded bf16 row of the widened fp8 tile
constexpr float kSlack = 8.f;    // lazy-rescale slack of the running max (log2 units)

struct Cursor {
  int b;            // sequence
  int64_t t;        // first token of the tile, local to the sequence
  int64_t t_end;    // end of this worker's segment of the sequence (local)
  int64_t row0;     // cache row of token t
};

// Move to the next tile of this worker's token range; false when done.
template <int TILE>
__device__ __forceinline__ bool advance(Cursor& c, const int64_t* prefix, const int64_t* seq_start,
                                        int B, int64_t r_hi) {
  c.t += TILE;
  c.row0 += TILE;
  if (c.t < c.t_end) return true;
  int b = c.b + 1;
  while (b < B && ld_const(prefix, b + 1) == ld_const(prefix, b)) ++b;   // skip empty sequences
  b = uniform(b);
  if (b >= B || ld_const(prefix, b) >= r_hi) return false;
  c.b = b;
  c.t = 0;
  const int64_t pb = ld_const(prefix, b), pe = ld_const(prefix, b + 1);
  c.t_end = (pe < r_hi ? pe : r_hi) - pb;
  c.row0 = ld_const(seq_start, b);
  return true;
}

// Value operands of four 16-dim blocks starting at block NB0: the low half
// covers tile rows 0..15, the high half rows 16..31 (row pitch TP bytes).
template <int TP, int NB0>
__device__ __forceinline__ void pv_read4(uint32_t addr, s16x4* lo, s16x4* hi) {
  lds_tr16_x8<NB0 * 32, 16 * TP + NB0 * 32, (NB0 + 1) * 32, 16 * TP + (NB0 + 1) * 32,
              (NB0 + 2) * 32, 16 * TP + (NB0 + 2) * 32, (NB0 + 3) * 32, 16 * TP + (NB0 + 3) * 32>(
      addr, lo[0], hi[0], lo[1], hi[1], lo[2], hi[2], lo[3], hi[3]);
}

template <int CT, int HB, int DS, int NSTAGE>
__global__ void __launch_bounds__(64 * HB * DS)
mla_attn_kernel(AttnParams p) {
  constexpr int NW = HB * DS;
  constexpr int TILE = Tr<CT>::kTile;
  constexpr int RB = Tr<CT>::kRowBytes;
  constexpr int RP = Tr<CT>::kPad;
  constexpr int SPR = RP / 16;                           // 16-byte slots per padded row
  constexpr int NCH = (TILE * RP + 1023) / 1024;         // 1 KB wave copies per tile
  constexpr int STAGE_DATA = NCH * 1024;
  constexpr int STAGE_BYTES = STAGE_DATA + (CT == kFP8 ? 256 : 0);
  constexpr int CONV_BYTES = (CT == kFP8) ? TILE * kConvPad : 0;
  constexpr int NCOPY = NCH + (CT == kFP8 ? 1 : 0);      // fp8 adds the row-scale copy
  constexpr int CPW = (NCOPY + NW - 1) / NW;             // copies per wave per tile
  constexpr int DSLICE = kDc / DS;
  constexpr int NB = DSLICE / 16;
  // Split scores: with one 16-head block shared by four waves, wave w
  // computes the scores of token block (w & 1) over half of the 576-wide
  // contraction (w >> 1) and the four fp32 partials meet in LDS, so each
  // score MFMA and each tile read for scores happens once per workgroup.
  constexpr bool SK = (CT != kF32) && HB == 1 && DS == 4;
  constexpr int SX_BYTES = SK ? 4096 : 0;
  static_assert(NSTAGE >= 2, "ring needs two stages");
  static_assert(NCOPY > NW, "a repeated copy needs an earlier copy of the same wave");

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
  const int64_t r_lo = ld_const(p.starts, w);
  const int64_t r_hi = ld_const(p.starts, w + 1);
  if (r_lo >= r_hi) return;                              // whole workgroup

  // ---- this wave's copies: LDS slot -> (row, byte in row) of the tile ----
  // slot s = id*64 + lane of the padded stage holds row s / SPR, chunk
  // s % SPR; the pad chunk and slots past the tile repeat valid data.
  int cp_row[CPW], cp_col[CPW], cp_lds[CPW];
  uint32_t cp_off[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    int id = wave + i * NW;
    if (id >= NCOPY) id -= NW;                           // repeat this wave's previous copy
    cp_lds[i] = uniform(id);
    const int s = id * 64 + lane;
    int r = s / SPR, c = s - (s / SPR) * SPR;
    if (c >= RB / 16) c = RB / 16 - 1;
    if (r >= TILE) r = TILE - 1;
    cp_row[i] = r;
    cp_col[i] = c * 16;
    cp_off[i] = (uint32_t)(r * RB + c * 16);
  }

  Cursor c0;
  c0.b = ld_const(p.wseq, w);
  {
    const int64_t pb = ld_const(p.prefix, c0.b), pe = ld_const(p.prefix, c0.b + 1);
    c0.t = r_lo - pb;
    c0.t_end = (pe < r_hi ? pe : r_hi) - pb;
    c0.row0 = ld_const(p.seq_start, c0.b) + c0.t;
  }

  auto issue = [&](const Cursor& c, int stage) {
    const int64_t left = c.t_end - c.t;
    const int nvalid = left < TILE ? (int)left : TILE;
    const auto rsrc = make_rsrc(p.rows + c.row0 * RB, (uint32_t)(TILE * RB));
    char* sb = smem + stage * STAGE_BYTES;
    if (nvalid == TILE) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        if (NCOPY == NCH || cp_lds[i] < NCH) buffer_copy16(rsrc, cp_off[i], sb + cp_lds[i] * 1024);
      }
    } else {
      // last tile of a segment: rows past the end repeat the last valid row
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int r = cp_row[i] < nvalid ? cp_row[i] : nvalid - 1;
        if (NCOPY == NCH || cp_lds[i] < NCH)
          buffer_copy16(rsrc, (uint32_t)(r * RB + cp_col[i]), sb + cp_lds[i] * 1024);
      }
    }
    if constexpr (CT == kFP8) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        if (cp_lds[i] == NCH) {
          const auto srsrc = make_rsrc(p.row_scale + c.row0, (uint32_t)(TILE * 4));
          const int r = (lane & (TILE - 1)) < nvalid ? (lane & (TILE - 1)) : nvalid - 1;
          buffer_copy4(srsrc, (uint32_t)(r * 4), sb + STAGE_DATA);
        }
      }
    }
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
      lvalid = advance<TILE>(lc, p.prefix, p.seq_start, B, r_hi);
    }
  }

  // ---- softmax state ----
  float m_run = -INFINITY;   // running max of this lane's head (log2 domain)
  float l_run = 0.f;         // this lane's share of the running sum
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane operand bases (bytes from the tile start)
  constexpr int TP = (CT == kFP8) ? kConvPad : RP;       // row pitch of the tile computed on
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
    if (lvalid) {
      issue(lc, issued % NSTAGE);
      ++issued;
      lvalid = advance<TILE>(lc, p.prefix, p.seq_start, B, r_hi);
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
        const int j = i - r * 36;
        const u32x4 v = *(const u32x4*)(stage + r * RP + j * 16);
        const uint2 c0 = fp8x4_to_bf16x4(v[0]), c1 = fp8x4_to_bf16x4(v[1]);
        const uint2 c2 = fp8x4_to_bf16x4(v[2]), c3 = fp8x4_to_bf16x4(v[3]);
        *(u32x4*)(conv + r * kConvPad + j * 32) = u32x4{c0.x, c0.y, c1.x, c1.y};
        *(u32x4*)(conv + r * kConvPad + j * 32 + 16) = u32x4{c2.x, c2.y, c3.x, c3.y};
      }
      barrier_lds();
      tb = conv;
    }

    if constexpr (CT != kF32) {
      // ---------------- scores: two 16-token blocks ----------------
      const uint32_t tr_addr = (uint32_t)(size_t)tb + tr_lane;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const char* sa = tb + s_base;
      if constexpr (SK) {
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
        }
        // value operands of this tile, read while the score MFMAs run
        if constexpr (NB == 8) {
          pv_read4<TP, 0>(tr_addr, vlo, vhi);
          pv_read4<TP, 4>(tr_addr, vlo + 4, vhi + 4);
        }
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
      } else {
      // operands in three batches of 6 k-steps, double-buffered: the reads
      // of batch i+1 are in flight while batch i feeds the MFMAs
      constexpr int KB = 6;
      bf16x8 abuf[2][2 * KB];
      auto load_batch = [&](int buf, int kb) {
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          abuf[buf][2 * j] = *(const bf16x8*)(sa + (kb * KB + j) * 64);
          abuf[buf][2 * j + 1] = *(const bf16x8*)(sa + 16 * TP + (kb * KB + j) * 64);
        }
      };
      auto mfma_batch = [&](int buf, int kb) {
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          s0 = mfma_bf16_k32(abuf[buf][2 * j], q[kb * KB + j], s0);
          s1 = mfma_bf16_k32(abuf[buf][2 * j + 1], q[kb * KB + j], s1);
        }
      };
      load_batch(0, 0);
      load_batch(1, 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_batch(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_batch(0, 2);
      __builtin_amdgcn_sched_barrier(0);
      mfma_batch(1, 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_batch(0, 2);
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
      if constexpr (SK && NB == 8) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) pv_mfma(nb, vlo[nb], vhi[nb]);
      } else {
        static_assert(NB % 4 == 0, "value blocks come in groups of four");
#pragma unroll
        for (int n0 = 0; n0 < NB; n0 += 4) {
          s16x4 lo[4], hi[4];
          pv_read4<TP, 0>(tr_addr + n0 * 32, lo, hi);
#pragma unroll
          for (int k = 0; k < 4; ++k) pv_mfma(n0 + k, lo[k], hi[k]);
        }
      }
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
    if (!advance<TILE>(cc, p.prefix, p.seq_start, B, r_hi)) break;
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
  prm.starts = a.starts;
  prm.wseq = a.wseq;
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
