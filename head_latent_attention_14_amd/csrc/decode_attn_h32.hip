// MLA decode attention for head counts that are multiples of 128 (the
// DeepSeek-V2 shape) over a bf16 latent cache.
//
// Same contractions as decode_attn.hip (discosf explainer, "long-context
// bottleneck": W_UK folds into the query and W_UV into the output, so scores
// and values both come from the 576-wide latent rows):
//   scores  S[t][h] = c_t . q_lat[h] + k_pe_t . q_pe[h]
//   values  O^T[d][h] += sum_t c_t[d] p[t][h]
//
// One workgroup of four waves, one wave per SIMD, streams a range of 32-token
// tiles through an LDS ring; wave w owns 32 heads for both contractions, so
// no score partial crosses waves and each head's softmax runs once. With
// 32x32x16 MFMA tiles every 1 KB operand read from LDS feeds 32 heads, for
// the scores (A = tile rows, B = the wave's queries in registers) and for the
// values (A = tile^T through transposing reads, B = the wave's
// probabilities). A wave holds 256 fp32 accumulators for its 32 heads x 512
// latent dims and 144 registers of queries, so it runs alone on its SIMD:
// the value accumulators live in the 256 accumulation registers and
// everything else in the 256 ordinary ones.
//
// Two choices follow from how the compiler treats the gfx950 instructions:
//  * The score MFMAs are written in inline asm with an ordinary-register
//    accumulator. Through the builtin every MFMA of the kernel would take
//    the accumulation-register form, and the score tile would compete with
//    the value accumulators for those registers (spills).
//  * Every LDS read of a staged tile is inline asm that completes inside its
//    own block. A compiler-visible LDS read after an asynchronous global->LDS
//    copy makes the compiler wait for all copies in flight, which would
//    empty the prefetch ring on every tile.
// Hazards the compiler cannot see are covered inside the asm blocks: two
// wait states before the first MFMA of a block (a vector ALU write of an
// operand just before it), twenty after the last score MFMA of a tile
// (before vector ALU reads of the scores).
#include <type_traits>

#include "attn_tile.h"

namespace mla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Row i of the score tile (the MFMA's M index, i = 16j + 8v + 4u + e) reads
// token 16j + 4e + 2v + u of the staged tile. At the 1168-byte row pitch
// (36 banks modulo the 64 banks of the LDS) the sixteen rows one 256-byte
// score read serves then fall on disjoint banks, and so do the four rows one
// transposing value read serves (tokens 4 apart: 16 banks apart); the value
// product reads tokens in the order the score accumulator holds them (lane
// half u, register r: rows 8(r/4) + 4u + r%4).
__host__ __device__ constexpr int h32_token(int i) {
  return (i & 16) | ((i & 3) << 2) | (((i >> 3) & 1) << 1) | ((i >> 2) & 1);
}

// Four score MFMAs (k-steps K0 .. K0+3) on operands already in registers.
// With two accumulators (s for even k-steps, s2 for odd ones) consecutive
// MFMAs do not wait for each other's result. FIRST: the first MFMA of each
// accumulator starts it (C = 0). LAST: the block ends with the wait states a
// vector ALU read of the results needs.
template <int K0, bool FIRST, bool LAST, int NACC>
__device__ __forceinline__ void score_mfma4(f32x16& s, f32x16& s2, const bf16x8* a,
                                            const bf16x8* q) {
#define MLA_MF(d, c, qq) "v_mfma_f32_32x32x16_bf16 %[" d "], %[" c "], %[" qq "], %[" d "]\n"
#define MLA_MZ(d, c, qq) "v_mfma_f32_32x32x16_bf16 %[" d "], %[" c "], %[" qq "], 0\n"
#define MLA_IN                                                                    \
  [c0] "v"(a[0]), [c1] "v"(a[1]), [c2] "v"(a[2]), [c3] "v"(a[3]),                  \
  [q0] "v"(q[K0]), [q1] "v"(q[K0 + 1]), [q2] "v"(q[K0 + 2]), [q3] "v"(q[K0 + 3])
#define MLA_END "s_nop 7\n s_nop 7\n s_nop 3"
  if constexpr (NACC == 1) {
    if constexpr (FIRST) {
      asm volatile("s_nop 1\n" MLA_MZ("s", "c0", "q0") MLA_MF("s", "c1", "q1")
                   MLA_MF("s", "c2", "q2") MLA_MF("s", "c3", "q3")
                   : [s] "=&v"(s)
                   : MLA_IN);
    } else if constexpr (LAST) {
      asm volatile("s_nop 1\n" MLA_MF("s", "c0", "q0") MLA_MF("s", "c1", "q1")
                   MLA_MF("s", "c2", "q2") MLA_MF("s", "c3", "q3") MLA_END
                   : [s] "+v"(s)
                   : MLA_IN);
    } else {
      asm volatile("s_nop 1\n" MLA_MF("s", "c0", "q0") MLA_MF("s", "c1", "q1")
                   MLA_MF("s", "c2", "q2") MLA_MF("s", "c3", "q3")
                   : [s] "+v"(s)
                   : MLA_IN);
    }
  } else {
    if constexpr (FIRST) {
      asm volatile("s_nop 1\n" MLA_MZ("s", "c0", "q0") MLA_MZ("t", "c1", "q1")
                   MLA_MF("s", "c2", "q2") MLA_MF("t", "c3", "q3")
                   : [s] "=&v"(s), [t] "=&v"(s2)
                   : MLA_IN);
    } else if constexpr (LAST) {
      asm volatile("s_nop 1\n" MLA_MF("s", "c0", "q0") MLA_MF("t", "c1", "q1")
                   MLA_MF("s", "c2", "q2") MLA_MF("t", "c3", "q3") MLA_END
                   : [s] "+v"(s), [t] "+v"(s2)
                   : MLA_IN);
    } else {
      asm volatile("s_nop 1\n" MLA_MF("s", "c0", "q0") MLA_MF("t", "c1", "q1")
                   MLA_MF("s", "c2", "q2") MLA_MF("t", "c3", "q3")
                   : [s] "+v"(s), [t] "+v"(s2)
                   : MLA_IN);
    }
  }
#undef MLA_MF
#undef MLA_MZ
#undef MLA_IN
#undef MLA_END
}

// Value operands of dim blocks DB and DB+1 (32 dims each), both 16-token
// k-steps: a[2*(db-DB) + j] is the A operand (tile^T) of block db, k-step j.
// Source lane (g, e, a) of a 16-lane group points at token 4e + g/2 (+16j +
// 2v) and dims 32*DB + 16*(g%2) + 4a; instruction v supplies k-slots 4v..4v+3.
template <int RP, int DB>
__device__ __forceinline__ void value_read2(uint32_t addr, bf16x8* a) {
  s16x4 r[8];
  lds_tr16_x8<64 * DB, 2 * RP + 64 * DB, 16 * RP + 64 * DB, 18 * RP + 64 * DB,
              64 * DB + 64, 2 * RP + 64 * DB + 64, 16 * RP + 64 * DB + 64,
              18 * RP + 64 * DB + 64>(addr, r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const s16x4 lo = r[2 * i], hi = r[2 * i + 1];
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    a[i] = __builtin_bit_cast(bf16x8, v);
  }
}

// Four accumulators c*4 .. c*4+3 of a 32x32 block, read from the
// accumulation registers. Every vector ALU access to the value accumulators
// goes through these small asm blocks, four registers at a time: written as
// plain C++ the compiler moves all 256 accumulators through ordinary
// registers at once and spills the queries. FIRST adds the wait states
// between the last MFMA writing the block and the first read.
__device__ __forceinline__ f32x4 read_acc4(const f32x16& o, int c, bool first) {
  float t0, t1, t2, t3;
  if (first) asm volatile("s_nop 7\n s_nop 7\n s_nop 3" ::: "memory");
  asm volatile(
      "v_accvgpr_read_b32 %[t0], %[e0]\n v_accvgpr_read_b32 %[t1], %[e1]\n"
      "v_accvgpr_read_b32 %[t2], %[e2]\n v_accvgpr_read_b32 %[t3], %[e3]"
      : [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
      : [e0] "a"(o[4 * c]), [e1] "a"(o[4 * c + 1]), [e2] "a"(o[4 * c + 2]),
        [e3] "a"(o[4 * c + 3]));
  return f32x4{t0, t1, t2, t3};
}
// o[4c .. 4c+3] *= alpha in place (see read_acc4).
__device__ __forceinline__ void scale_acc4(f32x16& o, int c, float alpha, bool first) {
  float t0, t1, t2, t3;
  if (first) asm volatile("s_nop 7\n s_nop 7\n s_nop 3" ::: "memory");
  asm volatile(
      "v_accvgpr_read_b32 %[t0], %[e0]\n v_accvgpr_read_b32 %[t1], %[e1]\n"
      "v_accvgpr_read_b32 %[t2], %[e2]\n v_accvgpr_read_b32 %[t3], %[e3]\n"
      "v_mul_f32 %[t0], %[t0], %[al]\n v_mul_f32 %[t1], %[t1], %[al]\n"
      "v_mul_f32 %[t2], %[t2], %[al]\n v_mul_f32 %[t3], %[t3], %[al]\n"
      "v_accvgpr_write_b32 %[e0], %[t0]\n v_accvgpr_write_b32 %[e1], %[t1]\n"
      "v_accvgpr_write_b32 %[e2], %[t2]\n v_accvgpr_write_b32 %[e3], %[t3]"
      : [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3),
        [e0] "+a"(o[4 * c]), [e1] "+a"(o[4 * c + 1]), [e2] "+a"(o[4 * c + 2]),
        [e3] "+a"(o[4 * c + 3])
      : [al] "v"(alpha));
}

template <int CT, int NW, int NSTAGE, int NACC, bool PAGED>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_attn_h32_kernel(AttnParams p) {
  static_assert(CT == kBF16, "bf16 cache");
  constexpr int TILE = 32;
  constexpr int RP = Tr<CT>::kPad;
  using TC = TileCopy<CT, NW>;
  constexpr int STAGE_BYTES = TC::STAGE_BYTES;
  constexpr int CPW = TC::CPW;                           // copies per wave per tile
  static_assert(NSTAGE >= 2, "ring needs two stages");
  static_assert(CPW * (NSTAGE - 1) < 64, "outstanding copies fit the vmcnt counter");
  static_assert(Tr<CT>::kTile == TILE, "32-token tiles");

  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int H = p.H;
  const int hw = (blockIdx.y * NW + wave) * 32;          // this wave's first head
  const int64_t w = blockIdx.x;
  int64_t r_hi;
  const Cursor c0 = cursor_start<TILE, PAGED>(p, w, lane, r_hi);
  if (c0.b < 0) return;                                  // whole workgroup

  TC cp;
  cp.init(wave, lane);

  // queries, the B operand of the score MFMAs: k-step kk covers dims
  // 16kk..16kk+15 of the 576-wide row (kk >= 32: the RoPE part); lane l holds
  // head hw + l%32, dims 16kk + 8(l/32) .. +7
  bf16x8 q[36];
  auto load_q = [&](int b) {
    const int ln = opaque(lane);
    const int64_t base = (int64_t)b * H + hw + (ln & 31);
    const __bf16* ql = (const __bf16*)p.q_lat + base * kDc + 8 * (ln >> 5);
    const __bf16* qp = (const __bf16*)p.q_pe + base * kDr + 8 * (ln >> 5);
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) q[kk] = *(const bf16x8*)(ql + 16 * kk);
#pragma unroll
    for (int kk = 32; kk < 36; ++kk) q[kk] = *(const bf16x8*)(qp + 16 * (kk - 32));
  };

  // the first tiles' copies, then the queries; all of them land before the
  // loop, so the compiler knows of no load in flight inside it
  Cursor lc = c0;
  bool lvalid = true;
  int issued = 0;
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i) {
    if (lvalid) {
      cp.issue(p.rows, p.row_scale, lc, smem + i * STAGE_BYTES, lane);
      ++issued;
      lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
    }
  }
  {
    int b0 = c0.b;
    asm volatile("" : "+s"(b0) :: "memory");
    load_q(b0);
  }
  wait_vmcnt<0>();

  float m_run = -INFINITY;     // running max of this lane's head (log2 domain)
  float l_run = 0.f;           // this lane's share of the running sum
  bool fresh = true;           // the accumulators hold nothing of this segment yet
  f32x16 o[16];                // O^T: dims 32db + 8(r/4) + 4(l/32) + r%4, head hw + l%32
#pragma unroll
  for (int db = 0; db < 16; ++db) o[db] = f32x16{};

  // per-lane LDS offsets: score operand row h32_token(l%32), bytes 16(l/32);
  // value operand source lane (g, e, a): token 4e + g/2, bytes 32(g%2) + 8a
  const uint32_t s_lane = (uint32_t)(h32_token(lane & 31) * RP + 16 * (lane >> 5));
  const int tg = lane >> 4, te = (lane & 15) >> 2, ta = lane & 3;
  const uint32_t tr_lane = (uint32_t)((4 * te + (tg >> 1)) * RP + 32 * (tg & 1) + 8 * ta);

  Cursor cc = c0;
  int it = 0;
  while (true) {
    wait_tiles<CPW, NSTAGE - 2>(issued - 1 - it);       // this wave's copies of tile `it` landed
    barrier_lds();                                       // all copies visible; stage it-1 free
    const bool do_copy = lvalid;
    typename TC::Pending pend;
    if (do_copy) {
      pend = cp.prepare(p.rows, p.row_scale, lc, smem + (issued % NSTAGE) * STAGE_BYTES);
      ++issued;
      lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
    }
    const uint32_t tb = (uint32_t)(size_t)(smem + (it % NSTAGE) * STAGE_BYTES);
    const int64_t left = cc.t_end - cc.t;
    const int nvalid = left < TILE ? (int)left : TILE;

    // ---------------- scores: 36 k-steps in nine blocks of four ----------------
    // (operands read two blocks ahead; the compiler counts their waits)
    f32x16 s, s2;
    {
      const char* sa = smem + (it % NSTAGE) * STAGE_BYTES + s_lane;
      bf16x8 a[3][4];
      auto rd = [&](int blk) {
#pragma unroll
        for (int k = 0; k < 4; ++k) a[blk % 3][k] = *(const bf16x8*)(sa + 32 * (4 * blk + k));
      };
      rd(0);
      rd(1);
#define MLA_SB(BLK, FIRST, LAST)                                           \
  if constexpr (BLK + 2 <= 8) rd(BLK + 2);                                 \
  score_mfma4<4 * BLK, FIRST, LAST, NACC>(s, s2, a[BLK % 3], q);           \
  __builtin_amdgcn_sched_barrier(0);
      MLA_SB(0, true, false)
      MLA_SB(1, false, false)
      MLA_SB(2, false, false)
      MLA_SB(3, false, false)
      MLA_SB(4, false, false)
      MLA_SB(5, false, false)
      MLA_SB(6, false, false)
      MLA_SB(7, false, false)
      MLA_SB(8, false, true)
#undef MLA_SB
      if constexpr (NACC == 2) s += s2;
    }

    // ---------------- online softmax (this lane's head, 16 tokens) ----------------
    if (nvalid < TILE) {                                 // tail tile: mask tokens past the end
      const int u = opaque(lane) >> 5;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (h32_token(8 * (r >> 2) + (r & 3)) + u >= nvalid) s[r] = -INFINITY;
    }
    float tmax = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = __builtin_fmaxf(tmax, s[r]);
    {
      const auto x = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, tmax),
                                                      __builtin_bit_cast(unsigned, tmax), false, false);
      const unsigned x0 = x[0], x1 = x[1];
      tmax = __builtin_fmaxf(__builtin_bit_cast(float, x0), __builtin_bit_cast(float, x1));
    }
    const float mt = tmax * p.scale_log2;                // scale > 0: max commutes with it
    // lazy rescale: the reference max moves only when a score exceeds it by
    // more than 2^kSlack, so p <= 2^kSlack stays finite (o and l share it)
    if (__any(mt > m_run + kSlack)) {
      const float m_new = __builtin_fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      if (!fresh) {
#pragma unroll
        for (int db = 0; db < 16; ++db)
#pragma unroll
          for (int c = 0; c < 4; ++c) scale_acc4(o[db], c, alpha, db == 0 && c == 0);
        asm volatile("s_nop 4" ::: "memory");           // accumulator writes before the next MFMA
      }
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[16];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.scale_log2, -m_use));
      psum += pv[r];
    }
    l_run += psum;
    const bf16x8 pb0 = pack_bf16x8(pv), pb1 = pack_bf16x8(pv + 8);

    // ---------------- values: O^T += tile^T P^T over 16 dim blocks ----------------
    // (FRESH: the first tile of a segment starts the accumulators from zero)
    const uint32_t ta0 = tb + tr_lane;
    auto values = [&](auto fresh_c) {
      constexpr bool FRESH = decltype(fresh_c)::value;
      bf16x8 va[2][4];
      value_read2<RP, 0>(ta0, va[0]);
      auto step = [&](auto db_c, const bf16x8* a) {
        constexpr int DB = decltype(db_c)::value;
        if constexpr (FRESH) {
          o[DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], pb0, f32x16{}, 0, 0, 0);
          o[DB + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], pb0, f32x16{}, 0, 0, 0);
        } else {
          o[DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], pb0, o[DB], 0, 0, 0);
          o[DB + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], pb0, o[DB + 1], 0, 0, 0);
        }
        o[DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], pb1, o[DB], 0, 0, 0);
        o[DB + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], pb1, o[DB + 1], 0, 0, 0);
      };
      // the MFMAs of a pair of dim blocks go out, then the next pair's
      // operand reads (completing while those MFMAs run) and one copy
#define MLA_VSTEP(DB, CUR, NXT, COPY)                                              \
  step(std::integral_constant<int, DB>{}, va[CUR]);                                \
  __builtin_amdgcn_sched_barrier(0);                                               \
  if constexpr (DB + 2 < 16) value_read2<RP, DB + 2>(ta0, va[NXT]);                \
  if constexpr (COPY >= 0 && COPY < CPW) {                                         \
    if (do_copy) cp.template copy<true>(pend, COPY);                                              \
  }                                                                                \
  __builtin_amdgcn_sched_barrier(0);
      MLA_VSTEP(0, 0, 1, 0)
      MLA_VSTEP(2, 1, 0, 1)
      MLA_VSTEP(4, 0, 1, 2)
      MLA_VSTEP(6, 1, 0, 3)
      MLA_VSTEP(8, 0, 1, 4)
      MLA_VSTEP(10, 1, 0, 5)
      MLA_VSTEP(12, 0, 1, 6)
      MLA_VSTEP(14, 1, 0, 7)
      if constexpr (CPW > 8) {
        if (do_copy) {
#pragma unroll
          for (int k = 8; k < CPW; ++k) cp.template copy<true>(pend, k);
        }
      }
#undef MLA_VSTEP
    };
    if (fresh) values(std::true_type{});
    else values(std::false_type{});
    fresh = false;

    // ---------------- segment end: write the partial ----------------
    const bool seg_end = (cc.t + TILE >= cc.t_end);
    if (seg_end) {
      const int64_t slot = w + cc.b;
      const int ln = opaque(lane);
      const auto x = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, l_run),
                                                      __builtin_bit_cast(unsigned, l_run), false, false);
      const unsigned x0 = x[0], x1 = x[1];
      const float lsum = __builtin_bit_cast(float, x0) + __builtin_bit_cast(float, x1);
      const int h = hw + (ln & 31);
      const float inv = inv_or_zero(lsum);
      const int64_t po = (slot * H + h) * kDc + 4 * (ln >> 5);
#pragma unroll
      for (int db = 0; db < 16; ++db)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          store_part4<CT>(p.part_o, po + 32 * db + 8 * c, read_acc4(o[db], c, db == 0 && c == 0),
                          inv);
          __builtin_amdgcn_sched_barrier(0);
        }
      if (ln < 32) {
        p.part_ml[(slot * H + h) * 2 + 0] = m_run;
        p.part_ml[(slot * H + h) * 2 + 1] = lsum;
      }
      m_run = -INFINITY;
      l_run = 0.f;
      fresh = true;
    }
    if (!advance<TILE, PAGED>(cc, p, r_hi, lane)) break;
    if (seg_end) {
      load_q(cc.b);
      wait_vmcnt<0>();
    }
    ++it;
  }
}

hipError_t launch_attn_h32(const DecodePlan& plan, const AttnParams& prm, hipStream_t s) {
  dim3 grid(plan.workers, plan.head_groups);
  if (plan.nstage == 4) {
    if (prm.block_table)
      hipLaunchKernelGGL((mla_attn_h32_kernel<kBF16, 4, 4, 2, true>), grid, dim3(256), 0, s, prm);
    else
      hipLaunchKernelGGL((mla_attn_h32_kernel<kBF16, 4, 4, 2, false>), grid, dim3(256), 0, s, prm);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
