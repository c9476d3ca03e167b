// Streaming MLA decode attention for one 16-head block per workgroup (the
// DeepSeek-V2-Lite shape) over a bf16 latent cache.
//
// Same contractions as decode_attn.hip (discosf explainer, "long-context
// bottleneck": W_UK folds into the query, W_UV into the output, so both
// products read the 576-wide latent rows):
//   scores  S^T[t][h] = c_t . q_lat[h] + k_pe_t . q_pe[h]
//   values  O^T[d][h] += sum_t c_t[d] p[t][h]
//
// With 16 heads the arithmetic per cached byte is small and the kernel is
// bound by the stream of latent rows from HBM. An asynchronous global->LDS
// copy holds the issuing wave until the memory pipeline accepts it, so one
// wave of the workgroup issues every copy and four other waves only compute:
//   copy wave   waits for tile t, joins the barrier, issues tile t+NSTAGE-1
//               (and, on the last tile of a sequence segment, the next
//               sequence's queries into the other of two LDS query buffers)
//   compute q   its share of the 18 k-steps of the scores (5, 4, 5, 4), the
//               fp32 partial to LDS, a barrier, the sum of the four partials
//               in a fixed order (so the four waves hold bit-identical
//               scores), the online softmax, and the values for latent dims
//               128q..128q+127.
// A tile takes two barriers: the tile is visible (A), the score partials are
// (B). The copy wave issues a few copies of a later tile between them and the
// rest after B, so the compute waves rarely wait for it at B. Each wave
// writes its quarter of a segment's partial itself.
#include <type_traits>

#include "attn_tile.h"

namespace mla {

template <int NSTAGE, bool PAGED>
__global__ void __launch_bounds__(320)
mla_attn_stream_kernel(AttnParams p) {
  constexpr int CT = kBF16;
  constexpr int TILE = 32;
  constexpr int RB = Tr<CT>::kRowBytes;
  constexpr int TP = Tr<CT>::kPad;
  using TC = TileCopy<CT, 1>;                            // all copies from one wave
  constexpr int STAGE_BYTES = TC::STAGE_BYTES;
  constexpr int NCOPY = TC::NCOPY;                       // 37 one-kilobyte copies per tile
  // queries of a segment in LDS: 16 rows of q_lat at the padded row pitch
  // (one 1 KB copy each) and the 16 q_pe rows of 128 bytes (two 1 KB copies),
  // whose eight 16-byte chunks are stored XOR-swizzled by (row / 2) so the
  // sixteen rows one operand read touches fall on different banks
  constexpr int QLAT_BYTES = 16 * TP;
  constexpr int QBUF = QLAT_BYTES + 16 * 128;
  constexpr int NQCOPY = 16 + 2;
  static_assert(NCOPY * (NSTAGE - 2) < 64 && NCOPY + NQCOPY < 64,
                "outstanding copies must fit the vmcnt counter");
  static_assert(Tr<CT>::kTile == TILE, "32-token tiles");

  constexpr int XBUF = 4 * 2048;                         // score partials, 2 KB per compute wave
  constexpr int NEARLY = 8;                              // copies issued between barriers A and B
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE_BYTES + 2 * QBUF + XBUF];
  // per stage: the tile's sequence, valid rows, whether it ends its segment,
  // whether another tile follows, and the following segment's sequence
  struct TileMeta {
    int b, nvalid, seg_end, more, next_b;
  };
  __shared__ TileMeta meta[NSTAGE];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const bool copier = (wave == 4);
  const int dq = wave & 3;                               // latent quarter of a compute wave
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int H = p.H;
  const int B = p.B;
  const int64_t w = blockIdx.x;
  int64_t r_hi;
  const Cursor c0 = cursor_start<TILE, PAGED>(p, w, lane, r_hi);
  if (c0.b < 0) return;                                  // whole workgroup

  char* qlds = smem + NSTAGE * STAGE_BYTES;             // two query buffers (segment parity)
  char* xbuf = qlds + 2 * QBUF;

  // ---- copy wave: copy i moves stage slots 64i..64i+63; slot s holds
  // padded row s / SPR, 16-byte chunk s % SPR (the pad chunk repeats the
  // last one). The row and chunk of this lane advance by 64 slots per copy,
  // which wraps the chunk at most once since 64 < SPR. ----
  constexpr int SPR = TP / 16;
  static_assert(SPR > 64, "one wrap per copy");
  struct Copies {
    __amdgpu_buffer_rsrc_t rsrc;
    char* sb;
    int nvalid, row, chunk;
  };
  auto prepare = [&](const Cursor& c, int stage) {
    const int64_t left = c.t_end - c.t;
    Copies k;
    k.nvalid = left < TILE ? (int)left : TILE;
    k.rsrc = make_rsrc(p.rows + c.row0 * RB, (uint32_t)(TILE * RB));
    k.sb = smem + stage * STAGE_BYTES;
    k.row = 0;
    k.chunk = opaque(lane);                              // slot `lane` of copy 0
    return k;
  };
  // copies [I0, I1) of a tile
  auto copies = [&](Copies& k, auto i0c, auto i1c) {
    constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      int r = k.row < k.nvalid ? k.row : k.nvalid - 1;   // rows past the end repeat the last one
      r = r < TILE ? r : TILE - 1;
      const int ch = k.chunk < RB / 16 ? k.chunk : RB / 16 - 1;
      buffer_copy16(k.rsrc, (uint32_t)(r * RB + ch * 16), k.sb + i * 1024);
      k.chunk += 64;
      if (k.chunk >= SPR) {
        k.chunk -= SPR;
        ++k.row;
      }
    }
  };
  using I0_ = std::integral_constant<int, 0>;
  using IE_ = std::integral_constant<int, NEARLY>;
  using IN_ = std::integral_constant<int, NCOPY>;
  // the 16 heads' queries of sequence b into query buffer `buf`
  auto issue_q = [&](int b, int buf) {
    char* qb = qlds + buf * QBUF;
    const int64_t h0 = (int64_t)b * H + blockIdx.y * 16;
    const auto ql = make_rsrc((const char*)p.q_lat + h0 * kDc * 2, 16 * kDc * 2);
    const auto qp = make_rsrc((const char*)p.q_pe + h0 * kDr * 2, 16 * kDr * 2);
    const int ln = opaque(lane);
    const uint32_t lo = (uint32_t)ln * 16;
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) buffer_copy16(ql, hh * 1024 + lo, qb + hh * TP);
    // LDS chunk ln of copy k holds row 8k + ln/8, position ln%8, which stores
    // chunk (ln%8) ^ (row/2 % 8) of that row
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int row = 8 * k + (ln >> 3);
      const int src = (ln & 7) ^ ((row >> 1) & 7);
      buffer_copy16(qp, (uint32_t)(row * 128 + src * 16), qb + QLAT_BYTES + k * 1024);
    }
  };

  // this compute wave's k-steps of the scores: [ks_lo, ks_hi) of 18
  const int ks_lo = (dq * 9 + 1) / 2, ks_hi = (dq * 9 + 10) / 2;
  // score A operand: tile row l16 (+16 for the second token block), k-run 8g
  const uint32_t s_base = (uint32_t)(l16 * TP + g * 16 + ks_lo * 64);
  // value A operand (transposing reads): source lane (g, l16) points at row
  // 4g + l16/4, dims 128*dq + 4*(l16%4) .. +3; the low half of a read holds
  // c_t[128*dq + 16*nb + l16] for t = 4g + q, the high half t = 16 + 4g + q
  const uint32_t tr_lane = (uint32_t)((4 * g + (l16 >> 2)) * TP + 2 * 128 * dq + 8 * (l16 & 3));
  // query operand (B of the score MFMA): lane (h, g) takes head h's k-run
  // 8g..8g+7 of each k-step
  const uint32_t q_lat_lane = (uint32_t)(l16 * TP + 16 * g);
  const uint32_t q_pe_lane = (uint32_t)(QLAT_BYTES + l16 * 128);

  // The two roles run separate loops over the same tiles, so they meet at
  // the same barriers: two per tile. Only the copy wave walks the sequences
  // (its cursor runs NSTAGE-1 tiles ahead); it records each tile's place in
  // the stream next to the tile, so the compute waves read it from LDS, and
  // keeps its own copy of the flags it needs in registers.
  static_assert(NSTAGE == 3, "the copy wave's flag queue holds two tiles");
  if (copier) {
    Cursor lc = c0;
    bool lvalid = true;
    int issued = 0;
    // flags of an issued tile: segment end (bit 0), another tile follows
    // (bit 1), the sequence after it (bits 2..)
    auto finish_tile = [&](Copies& k, int stage) {
      copies(k, IE_{}, IN_{});
      const int b = lc.b;
      const bool seg_end = (lc.t + TILE >= lc.t_end);
      ++issued;
      lvalid = advance<TILE, PAGED>(lc, p, r_hi, lane);
      if (lane == 0) meta[stage] = TileMeta{b, k.nvalid, seg_end ? 1 : 0, lvalid ? 1 : 0, lc.b};
      return (seg_end ? 1 : 0) | (lvalid ? 2 : 0) | (lc.b << 2);
    };
    issue_q(c0.b, 0);
    int fq0 = 0, fq1 = 0;                                // flags of tiles `it` and `it`+1
    {
      Copies k = prepare(lc, 0);
      copies(k, I0_{}, IE_{});
      fq0 = finish_tile(k, 0);
      if (lvalid) {
        k = prepare(lc, 1);
        copies(k, I0_{}, IE_{});
        fq1 = finish_tile(k, 1);
      }
    }
    int it = 0;
    int qpar = 0;                                        // query buffer of the current segment
    while (true) {
      wait_tiles<NCOPY, NSTAGE - 2>(issued - 1 - it);
      barrier_lds();                                     // A: tile `it` (and its queries) visible
      const int m = fq0;
      const bool m_seg_end = (m & 1) != 0, m_more = (m & 2) != 0;
      // the next segment's queries go out before this round's tile copies,
      // so the wait before the next barrier A covers them
      if (m_seg_end && m_more) issue_q(m >> 2, qpar ^ 1);
      const bool go = lvalid;
      const int stage = issued % NSTAGE;
      Copies k;
      if (go) {
        k = prepare(lc, stage);
        copies(k, I0_{}, IE_{});
      }
      barrier_lds();                                     // B: score partials visible
      fq0 = fq1;
      if (go) fq1 = finish_tile(k, stage);
      if (!m_more) break;
      if (m_seg_end) qpar ^= 1;
      ++it;
    }
    return;
  }

  // ---------------- compute waves: one pass per sequence segment ----------------
  int it = 0;
  int qpar = 0;
  bool more = true;
  while (more) {
    // first tile of the segment: its queries are in LDS buffer qpar once the
    // barrier has passed; they stay in registers for the whole segment
    barrier_lds();
    bf16x8 q[5];                                         // k-steps ks_lo + j
    {
      const char* qb = qlds + qpar * QBUF;
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const int ks = ks_lo + j;
        if (ks < 16) {
          q[j] = *(const bf16x8*)(qb + q_lat_lane + ks * 64);
        } else if (ks < 18) {
          const int c = 4 * (ks - 16) + g;               // logical 16-byte chunk of the q_pe row
          q[j] = *(const bf16x8*)(qb + q_pe_lane + 16 * (c ^ ((l16 >> 1) & 7)));
        }
      }
    }
    float m_run = -INFINITY;   // running max of this lane's head (log2 domain)
    float l_run = 0.f;         // this lane's share of the running sum
    f32x4 o[8];                // O^T: dims 128*dq + 16*nb + 4g + r, head l16
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int seg_b = 0;
    bool seg_end = false;
    bool first = true;
    while (!seg_end) {
      if (!first) barrier_lds();                         // tile `it` visible
      first = false;
      const TileMeta m = meta[it % NSTAGE];
      const int nvalid = uniform(m.nvalid);
      seg_end = uniform(m.seg_end) != 0;
      more = uniform(m.more) != 0;
      seg_b = uniform(m.b);
      const char* tbase = smem + (it % NSTAGE) * STAGE_BYTES;
      // ---------------- scores of the 32 tokens: this wave's k-steps ----------------
      const char* sa = tbase + s_base;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      {
        bf16x8 a0[5], a1[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          if (ks_lo + j < ks_hi) {
            a0[j] = *(const bf16x8*)(sa + j * 64);
            a1[j] = *(const bf16x8*)(sa + 16 * TP + j * 64);
          }
        }
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          if (ks_lo + j < ks_hi) {
            s0 = mfma_bf16_k32(a0[j], q[j], s0);
            s1 = mfma_bf16_k32(a1[j], q[j], s1);
          }
        }
      }
      {
        char* xw = xbuf + dq * 2048 + lane * 16;
        *(f32x4*)xw = s0;
        *(f32x4*)(xw + 1024) = s1;
      }
      // value operands of this tile, read while the score MFMAs run
      s16x4 vlo[8], vhi[8];
      const uint32_t tr_addr = (uint32_t)(size_t)tbase + tr_lane;
      lds_tr16_x8<0, 16 * TP, 32, 16 * TP + 32, 64, 16 * TP + 64, 96, 16 * TP + 96>(
          tr_addr, vlo[0], vhi[0], vlo[1], vhi[1], vlo[2], vhi[2], vlo[3], vhi[3]);
      lds_tr16_x8<128, 16 * TP + 128, 160, 16 * TP + 160, 192, 16 * TP + 192, 224, 16 * TP + 224>(
          tr_addr, vlo[4], vhi[4], vlo[5], vhi[5], vlo[6], vhi[6], vlo[7], vhi[7]);

      barrier_lds();                                     // B: the four partials are in LDS
      {
        // the same order in every wave: ((p0 + p1) + p2) + p3
        f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const char* xr = xbuf + u * 2048 + lane * 16;
          const f32x4 u0 = (u == dq) ? s0 : *(const f32x4*)xr;
          const f32x4 u1 = (u == dq) ? s1 : *(const f32x4*)(xr + 1024);
          if (u == 0) {
            t0 = u0;
            t1 = u1;
          } else {
            t0 += u0;
            t1 += u1;
          }
        }
        s0 = t0;
        s1 = t1;
      }
      // ---------------- online softmax over the tile ----------------
      float sc[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = s0[r] * p.scale_log2;
        sc[4 + r] = s1[r] * p.scale_log2;
      }
      if (nvalid < TILE) {                               // tail tile: mask rows past the end
        const int t4 = 4 * (opaque(lane) >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (t4 >= nvalid - r) sc[r] = -INFINITY;
          if (t4 >= nvalid - 16 - r) sc[4 + r] = -INFINITY;
        }
      }
      float tmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = __builtin_fmaxf(tmax, sc[i]);
      tmax = max_over_groups(tmax);
      // lazy rescale: the reference max moves only when a score exceeds it by
      // more than 2^kSlack (o and l always share the reference)
      if (__any(tmax > m_run + kSlack)) {
        const float m_new = __builtin_fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[nb] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
        l_run += pv[i];
      }
      // B operand (32 tokens x 16 heads): lane (h, g) holds p for tokens
      // 4g..4g+3 and 16+4g..16+4g+3, the order of the value operand's halves
      const bf16x8 pb = pack_bf16x8(pv);

      // ---------------- values: O^T += tile^T P^T, this wave's 128 dims ----------------
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const s16x8 a8 = {vlo[nb][0], vlo[nb][1], vlo[nb][2], vlo[nb][3],
                          vhi[nb][0], vhi[nb][1], vhi[nb][2], vhi[nb][3]};
        o[nb] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a8), pb, o[nb]);
      }
      ++it;
    }
    // ---------------- segment end: this wave's quarter of the partial ----------------
    {
      const float lsum = sum_over_groups(l_run);
      const int64_t slot = w + seg_b;
      const int ln = opaque(lane);
      const int hh = blockIdx.y * 16 + (ln & 15);
      const float inv = inv_or_zero(lsum);
      const int64_t po = (slot * H + hh) * kDc + 128 * dq + 4 * (ln >> 4);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) store_part4<CT>(p.part_o, po + nb * 16, o[nb], inv);
      if (dq == 0 && (ln >> 4) == 0) {
        p.part_ml[(slot * H + hh) * 2 + 0] = m_run;
        p.part_ml[(slot * H + hh) * 2 + 1] = lsum;
      }
    }
    qpar ^= 1;
  }
}

hipError_t launch_attn_stream(const DecodePlan& plan, const AttnParams& prm, hipStream_t s) {
  if (plan.nstage != 3) return hipErrorInvalidValue;
  dim3 grid(plan.workers, plan.head_groups);
  if (prm.block_table)
    hipLaunchKernelGGL((mla_attn_stream_kernel<3, true>), grid, dim3(320), 0, s, prm);
  else
    hipLaunchKernelGGL((mla_attn_stream_kernel<3, false>), grid, dim3(320), 0, s, prm);
  return hipGetLastError();
}

}  // namespace mla
