// mla_append: compress hidden states into latent cache rows.
//
// row = (W_DKV h) || RoPE(W_KR h, pos), stored at seq_start[seq] + pos
// (discosf explainer, "long-context bottleneck": only the compressed latent
// c_KV is cached; "decoupled RoPE": a separate 64-wide key carries RoPE and is
// shared by all heads, adding d_R elements per token).
//
#include <math.h>

#include <type_traits>

#include "gemm_tile.h"

namespace mla {

constexpr int kColGroup = 16;                  // columns per group (one MFMA block)
constexpr int kNumGroups = kDrow / kColGroup;  // 36

// One workgroup computes 16 output columns (all 576 for the fp8 cache, whose
// per-row scale needs the whole row) for 16 tokens; its four waves split the
// d_model contraction into quarters and reduce through LDS.
struct Tr6 {
  static constexpr int kRowBytes = 464;                // fp6 row: 432 code bytes, 18 scales, padding
};

template <int CT>
__global__ void __launch_bounds__(256)
mla_append_kernel(AppendArgs a) {
  using E = typename std::conditional<CT == kF32, float, __bf16>::type;
  // fp8 (one scale per row) and fp6 (scales per block of 32) quantise whole
  // rows: one workgroup computes all 576 columns of its 16 tokens
  constexpr bool FP8 = (CT == kFP8 || CT == kFP6);
  constexpr int KPL = (CT == kF32) ? 1 : 8;        // k elements per lane per MFMA
  constexpr int KSTEP = 4 * KPL;                   // k per MFMA
  constexpr int U = 16;                            // MFMAs per load round
  __shared__ float red[4][16][16];                 // [wave][column][token]
  __shared__ float rowt[16][kDrow + 4];            // fp32 rows of the 16 tokens
  __shared__ int64_t trow[16];                     // cache row of each token (-1: skip)
  __shared__ int tpos[16];                         // RoPE position of each token

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int tok0 = blockIdx.x * 16;
  const int D = a.d_model;
  const int nks = D / KSTEP;                       // k-steps of the contraction

  // Slot of each of the 16 tokens (token -> sequence -> first row and
  // capacity): two batches of independent scalar loads, issued by wave 0
  // once its contraction loads are in flight, so the chain overlaps them.
  auto find_slots = [&]() {
    int sq[16], ps[16], cap[16];
    int64_t st[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tok = tok0 + t < a.n_tok ? tok0 + t : a.n_tok - 1;
      sq[t] = ld_const(a.tok_seq, tok);
      ps[t] = ld_const(a.tok_pos, tok);
    }
    if (a.block_table) {
      // paged: the row from the block table; a position past the table or a
      // table entry outside the page pool skips the token
      if (lane == 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          bool ok = sq[t] >= 0 && sq[t] < a.num_seqs;
          const int64_t r = ok ? paged_row(a.block_table, a.max_pages, a.page_tokens, a.total_pages,
                                           sq[t], ps[t], ok)
                               : 0;
          trow[t] = ok ? r : -1;
          tpos[t] = ps[t];
        }
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int sc = (sq[t] >= 0 && sq[t] < a.num_seqs) ? sq[t] : 0;
      cap[t] = ld_const(a.seq_cap, sc);
      st[t] = ld_const(a.seq_start, sc);
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const bool ok = sq[t] >= 0 && sq[t] < a.num_seqs && ps[t] >= 0 && ps[t] < cap[t];
        trow[t] = ok ? st[t] + ps[t] : -1;
        tpos[t] = ps[t];
      }
    }
  };

  const int tok_b = tok0 + l16 < a.n_tok ? tok0 + l16 : a.n_tok - 1;   // clamped B-operand token
  const E* hrow = (const E*)a.h + (int64_t)tok_b * D;

  const int cg_begin = FP8 ? 0 : blockIdx.y;
  const int cg_end = FP8 ? kNumGroups : blockIdx.y + 1;
  for (int cg = cg_begin; cg < cg_end; ++cg) {
    const int j = cg * kColGroup + l16;            // output column of this lane's A row
    const E* wrow = (j < kDc) ? (const E*)a.w_dkv + (int64_t)j * D
                              : (const E*)a.w_kr + (int64_t)(j - kDc) * D;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // wave w takes k-steps w, w+4, w+8, ...; one round issues the loads of U
    // of its k-steps, then their MFMAs
    for (int ks0 = wave; ks0 < nks; ks0 += 4 * U) {
      if constexpr (CT == kF32) {
        float av[U], bv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int ks = ks0 + 4 * u;
          const int k = ks * KSTEP + g;
          av[u] = ks < nks ? wrow[k] : 0.f;
          bv[u] = ks < nks ? hrow[k] : 0.f;
        }
        if (wave == 0 && cg == cg_begin && ks0 == 0) find_slots();
#pragma unroll
        for (int u = 0; u < U; ++u) acc = mfma_f32_k4(av[u], bv[u], acc);
      } else {
        bf16x8 av[U], bv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int ks = ks0 + 4 * u;
          const int k = ks * KSTEP + 8 * g;
          av[u] = ks < nks ? *(const bf16x8*)(wrow + k) : bf16x8{};
          bv[u] = ks < nks ? *(const bf16x8*)(hrow + k) : bf16x8{};
        }
        if (wave == 0 && cg == cg_begin && ks0 == 0) find_slots();
#pragma unroll
        for (int u = 0; u < U; ++u) acc = mfma_bf16_k32(av[u], bv[u], acc);
      }
    }
    // lane holds column cg*16 + 4g + r of token l16
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * g + r][l16] = acc[r];
    __syncthreads();
    {
      const int c = tid >> 4, t = tid & 15;
      rowt[t][cg * kColGroup + c] = red[0][c][t] + red[1][c][t] + red[2][c][t] + red[3][c][t];
    }
    __syncthreads();
  }

  // ---------------- RoPE on columns 512..575 (pairs 2i, 2i+1) ----------------
  const int c_lo = FP8 ? 0 : blockIdx.y * kColGroup;
  const int c_hi = FP8 ? kDrow : c_lo + kColGroup;
  if (c_hi > kDc) {
    for (int i = tid; i < 16 * 32; i += 256) {
      const int t = i >> 5, pr = i & 31;
      const int col = kDc + 2 * pr;
      const int tok = tok0 + t;
      if (col < c_lo || col >= c_hi || tok >= a.n_tok) continue;
      // angle in fp64, reduced to [-pi, pi] with a two-term 2*pi
      // (Cody-Waite) before the sine and cosine
      const double phi = (double)tpos[t] * a.inv_freq[pr];
      const double kq = rint(phi * 0.15915494309189535);          // 1 / (2 pi)
      double red_phi = fma(-kq, 6.283185307179586, phi);          // 2 pi, leading part
      red_phi = fma(-kq, 2.4492935982947064e-16, red_phi);        // 2 pi, trailing part
      double sn, cs;
      sincos(red_phi, &sn, &cs);
      const double x0 = rowt[t][col], x1 = rowt[t][col + 1];
      rowt[t][col] = (float)(x0 * cs - x1 * sn);
      rowt[t][col + 1] = (float)(x0 * sn + x1 * cs);
    }
    __syncthreads();
  }

  // ---------------- store ----------------
  if constexpr (!FP8) {
    {
      const int t = tid >> 4, c = c_lo + (tid & 15);
      const int tok = tok0 + t;
      if (tok < a.n_tok) {
        const int64_t row = trow[t];
        if (row >= 0) {
          if constexpr (CT == kF32)
            ((float*)a.rows)[row * kDrow + c] = rowt[t][c];
          else
            ((uint16_t*)a.rows)[row * kDrow + c] = f32_to_bf16_bits(rowt[t][c]);
        }
      }
    }
  } else if constexpr (CT == kFP6) {
    // one token per 16 lanes; lane sl quantises blocks sl and sl + 16 (< 18)
    // of 32 elements: shared exponent X = floor(log2(amax)) - 2 (0 for an
    // all-zero block: scale code 0), e2m3 codes rounded to nearest even with
    // saturation at 7.5, packed little-endian (element e at bits 6e .. 6e+5
    // of the block's 24 bytes), then the scale codes and zero padding
    const int t = tid >> 4, sl = tid & 15;
    const int tok = tok0 + t;
    const int64_t row = tok < a.n_tok ? trow[t] : -1;
    if (row >= 0) {
      uint8_t* dst = (uint8_t*)a.rows + row * Tr6::kRowBytes;
      for (int blk = sl; blk < 18; blk += 16) {
        const float* v = &rowt[t][32 * blk];
        float amax = 0.f;
        for (int e = 0; e < 32; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
        int x = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 2 : -127;   // amax = m 2^(x+3), m in [1, 2)
        x = x < -127 ? -127 : (x > 127 ? 127 : x);
        uint32_t w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
        for (int e = 0; e < 32; ++e) {
          const float q = __builtin_fabsf(__builtin_amdgcn_ldexpf(v[e], -x));   // exact
          float c;                                     // code magnitude, round to nearest even
          if (q < 2.f) c = __builtin_rintf(q * 8.f);                      // step 1/8: codes 0..16
          else if (q < 4.f) c = 16.f + __builtin_rintf((q - 2.f) * 4.f);  // step 1/4: codes 16..24
          else c = 24.f + __builtin_rintf((q - 4.f) * 2.f);               // step 1/2: codes 24..32
          uint32_t code = c > 31.f ? 31u : (uint32_t)c;                   // saturate at 7.5
          if (__builtin_signbit(v[e])) code |= 32u;
          const int bit = 6 * e;
          w[bit >> 5] |= code << (bit & 31);
          if ((bit & 31) > 26) w[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
        }
        uint32_t* d32 = (uint32_t*)(dst + 24 * blk);
        for (int k = 0; k < 6; ++k) d32[k] = w[k];
        dst[432 + blk] = (uint8_t)(x + 127);
      }
      if (sl == 0)
        for (int k = 450; k < Tr6::kRowBytes; ++k) dst[k] = 0;
    }
  } else {
    // one token per 16 lanes: amax, scale, then 36 codes per lane
    const int t = tid >> 4, sl = tid & 15;
    const int tok = tok0 + t;
    float amax = 0.f;
    for (int c = sl; c < kDrow; c += 16) amax = __builtin_fmaxf(amax, __builtin_fabsf(rowt[t][c]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, shfl_xor_f(amax, off));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    const int64_t row = tok < a.n_tok ? trow[t] : -1;
    if (row >= 0) {
      uint32_t* dst = (uint32_t*)((uint8_t*)a.rows + row * kDrow);
      for (int q4 = sl; q4 < kDrow / 4; q4 += 16) {
        const float* v = &rowt[t][4 * q4];
        dst[q4] = f32x4_to_fp8x4_sat(v[0] / scale, v[1] / scale, v[2] / scale, v[3] / scale);
      }
      if (sl == 0) a.row_scale[row] = scale;
    }
  }
}

// BF16 cache and activations: the same 16 columns x 16 tokens per workgroup,
// with both operands staged in LDS by asynchronous 1 KB copies. A wave copy
// covers 512 contiguous elements of one weight or hidden row, so every HBM
// request is a full contiguous kilobyte (loading MFMA operands straight from
// memory would touch 16 rows 2*d_model bytes apart per instruction). The
// contraction runs in stages of KC elements, two stages in LDS; rows are
// padded by 16 bytes so the 16 rows of an operand read fall on distinct banks.
struct AppendBf16Lds {
  static constexpr int KC = 1024;          // contraction elements per stage
  static constexpr int RS = KC * 2 + 16;   // padded LDS row (bytes)
  static constexpr int OPND = 16 * RS;     // 16 rows of one operand
  static constexpr int STAGE = 2 * OPND;   // weight rows, then hidden rows
  static constexpr int NST = 2;
  char stg[NST * STAGE];
  float red[8][16][17];                    // [wave][column][token] (up to 8 waves)
  float rowt[16][17];                      // [token][column]
  float2 rot[16][8];                       // (cos, sin) per token and pair (RoPE groups)
  int64_t trow[16];
  int tpos[16];
};

// One (16 tokens, 16 columns) block: token block tb, column group cg, run by
// NW waves (4 or 8), which share the copies and the contraction's k-steps.
template <int NW>
__device__ void append_bf16_block(const AppendArgs& a, int tb, int cg, AppendBf16Lds& L) {
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int KPW = 32 / NW;             // k-steps of a full stage per wave
  constexpr int KC = AppendBf16Lds::KC;
  constexpr int RS = AppendBf16Lds::RS;
  constexpr int OPND = AppendBf16Lds::OPND;
  constexpr int STAGE = AppendBf16Lds::STAGE;
  constexpr int NST = AppendBf16Lds::NST;
  char* stg = L.stg;
  auto& red = L.red;
  auto& rowt = L.rowt;
  auto& rot = L.rot;
  auto& trow = L.trow;
  auto& tpos = L.tpos;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int tok0 = tb * 16;
  const int j0 = cg * kColGroup;           // first output column
  const int D = a.d_model;
  const int nch = (D + KC - 1) / KC;

  const __bf16* wbase = (j0 < kDc) ? (const __bf16*)a.w_dkv + (int64_t)j0 * D
                                   : (const __bf16*)a.w_kr + (int64_t)(j0 - kDc) * D;
  const int nh = (a.n_tok - tok0 < 16) ? a.n_tok - tok0 : 16;
  // rows past the last token read as zeros (buffer range check)
  const auto rw = make_rsrc(wbase, (uint32_t)(16 * D * 2));
  const auto rh = make_rsrc((const __bf16*)a.h + (int64_t)tok0 * D, (uint32_t)(nh * D * 2));

  // stage c: copy i (wave-uniform) = operand i/32, row (i/2)%16, half i%2 of the KC slice
  auto issue = [&](int c) {
    const int k0 = c * KC;
    char* sb = stg + (c % NST) * STAGE;
#pragma unroll
    for (int u = 0; u < 64 / NW; ++u) {
      const int i = wave + NW * u;
      const int op = i >> 5, r = (i >> 1) & 15, pc = i & 1;
      if (k0 + pc * 512 >= D) continue;
      const uint32_t voff = (uint32_t)(((r * D) + k0 + pc * 512) * 2 + lane * 16);
      buffer_copy16(op ? rh : rw, voff, sb + op * OPND + r * RS + pc * 1024);
    }
  };
  issue(0);
  if (nch > 1) issue(1);

  // token slots (wave 0) and, for the RoPE columns, the rotation of every
  // (token, pair): angle in fp64, reduced to [-pi, pi] with a two-term 2*pi
  // (Cody-Waite), then sine and cosine of the reduced angle in fp32
  if (wave == 0) {
    const int t = (tok0 + l16 < a.n_tok) ? tok0 + l16 : a.n_tok - 1;
    const int sq = a.tok_seq[t];
    const int ps = a.tok_pos[t];
    const int sc = (sq >= 0 && sq < a.num_seqs) ? sq : 0;
    if (g == 0) {
      bool ok = sq >= 0 && sq < a.num_seqs;
      int64_t r = 0;
      if (a.block_table) {                 // paged: the row from the block table
        if (ok) r = paged_row(a.block_table, a.max_pages, a.page_tokens, a.total_pages, sq, ps, ok);
      } else {
        const int cap = a.seq_cap[sc];
        ok = ok && ps >= 0 && ps < cap;
        r = a.seq_start[sc] + ps;
      }
      trow[l16] = ok ? r : -1;
      tpos[l16] = ps;
    }
    if (j0 >= kDc) {
      const int i0 = (j0 - kDc) / 2;       // first pair of this column group
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int pr = g + 4 * pass;       // pairs g, g + 4 for the lanes of group g
        const double f0 = a.inv_freq[i0 + 4 * pass + 0], f1 = a.inv_freq[i0 + 4 * pass + 1];
        const double f2 = a.inv_freq[i0 + 4 * pass + 2], f3 = a.inv_freq[i0 + 4 * pass + 3];
        const double f = g == 0 ? f0 : g == 1 ? f1 : g == 2 ? f2 : f3;
        const double phi = (double)ps * f;
        const double kq = rint(phi * 0.15915494309189535);         // 1 / (2 pi)
        double rp = fma(-kq, 6.283185307179586, phi);              // 2 pi, leading part
        rp = fma(-kq, 2.4492935982947064e-16, rp);                 // 2 pi, trailing part
        float sn, cs;
        sincosf((float)rp, &sn, &cs);
        rot[l16][pr] = make_float2(cs, sn);
      }
    }
  }

  // ---------------- contraction ----------------
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    wait_vmcnt<0>();
    __syncthreads();                                   // stage c visible to all waves
    const int k0 = c * KC;
    const int nks = ((D - k0) < KC ? (D - k0) : KC) / 32;
    const char* sb = stg + (c % NST) * STAGE;
    const char* pa = sb + l16 * RS + g * 16;
    const char* pb = pa + OPND;
    // wave w takes k-steps KPW*w .. KPW*w + KPW-1
    if (nks == KC / 32) {                              // full stage: all reads, then the MFMAs
      bf16x8 av[KPW], bv[KPW];
#pragma unroll
      for (int u = 0; u < KPW; ++u) {
        av[u] = *(const bf16x8*)(pa + (KPW * wave + u) * 64);
        bv[u] = *(const bf16x8*)(pb + (KPW * wave + u) * 64);
      }
#pragma unroll
      for (int u = 0; u < KPW; ++u) acc = mfma_bf16_k32(av[u], bv[u], acc);
    } else {
#pragma unroll
      for (int u = 0; u < KPW; ++u) {
        const int ks = KPW * wave + u;
        if (ks < nks) acc = mfma_bf16_k32(*(const bf16x8*)(pa + ks * 64), *(const bf16x8*)(pb + ks * 64), acc);
      }
    }
    if (c + NST < nch) {
      __syncthreads();                                 // stage c consumed
      issue(c + NST);
    }
  }
  // lane holds column j0 + 4g + r of token l16
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * g + r][l16] = acc[r];
  __syncthreads();
  if (tid < 256) {
    const int cc = tid >> 4, t = tid & 15;
    float v = red[0][cc][t];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w][cc][t];
    rowt[t][cc] = v;
  }
  __syncthreads();
  if (j0 >= kDc && tid < 128) {                        // RoPE: pair pr of token t
    const int t = tid >> 3, pr = tid & 7;
    const float2 cs = rot[t][pr];
    const float x0 = rowt[t][2 * pr], x1 = rowt[t][2 * pr + 1];
    rowt[t][2 * pr] = x0 * cs.x - x1 * cs.y;
    rowt[t][2 * pr + 1] = x0 * cs.y + x1 * cs.x;
  }
  __syncthreads();
  if (tid < 256) {
    const int t = tid >> 4, cc = tid & 15;
    if (tok0 + t < a.n_tok && trow[t] >= 0)
      ((uint16_t*)a.rows)[trow[t] * kDrow + j0 + cc] = f32_to_bf16_bits(rowt[t][cc]);
  }
}

template <int NW>
__global__ void __launch_bounds__(64 * NW)
mla_append_bf16_kernel(AppendArgs a) {
  __shared__ __attribute__((aligned(1024))) AppendBf16Lds L;
  append_bf16_block<NW>(a, blockIdx.x, blockIdx.y, L);
}

// Append and the absorb launch of the following decode in one launch (bf16):
// neither reads what the other writes (the absorb product and the work plan
// read queries, weights and lengths, not cache rows). Workgroups of eight
// waves: [0, n_app) run one append block each; the next n_absw run absorb
// tiles j (waves 0-3) and, when it exists, j + n_absw (waves 4-7) side by
// side in their own LDS; the last one builds the plan. An append block
// moves 128 KB through its CU, and a wave issues its copies at a bounded
// rate, so the absorb tiles go to CUs of their own rather than queueing
// their loads ahead of an append block's.
__global__ void __launch_bounds__(512)
mla_append_absorb_kernel(AppendArgs a, GemmParams g, int n_app, int n_absw, int n_abs) {
  using G = AbsorbBf16;
  __shared__ __attribute__((aligned(1024))) AppendBf16Lds L;
  static_assert(2 * G::LDS_BYTES <= (int)sizeof(AppendBf16Lds::stg), "two absorb tiles fit the append stages");
  static_assert(G::kChunks == 1, "an absorb tile's run() takes one barrier");
  const int wg = blockIdx.x;
  if (wg == (int)gridDim.x - 1) {
    build_plan(g, (int64_t*)L.stg, (int)(sizeof(L.stg) / 8));
    return;
  }
  if (wg < n_app) {
    const int ntb = (a.n_tok + 15) / 16;
    append_bf16_block<8>(a, wg % ntb, wg / ntb, L);
    return;
  }
  // absorb tile t: 64 columns from n0 of head h for batch rows from b0
  const int nxb = kDc / kNT;                             // absorb tiles per (head, batch slice)
  const int half = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8);
  const int t = wg - n_app + half * n_absw;
  if (t < n_abs) {
    const int n0 = (t % nxb) * kNT;
    const int h = (t / nxb) % g.H;
    const int b0 = (t / nxb / g.H) * G::BT;
    typename G::Regs rg;
    G::load(g, n0, h, b0, rg);
    G::run(g, n0, h, b0, rg, L.stg + half * G::LDS_BYTES);
  } else {
    __syncthreads();                                     // the other half's run() barrier
  }
}

// The fused launch's workgroups: append blocks, absorb workgroups (one or
// two tiles each) and the plan workgroup, all in one round of CUs (the
// kernel's LDS allows one workgroup per CU); false when they do not fit.
struct FusedGrid {
  int n_app, n_absw, n_abs;
};
static bool fused_grid(const AppendArgs& a, const DecodeArgs& d, FusedGrid& f) {
  const int64_t n_app = (int64_t)((a.n_tok + 15) / 16) * kNumGroups;
  const int64_t n_abs = (int64_t)(kDc / kNT) * d.H * ((d.B + AbsorbBf16::BT - 1) / AbsorbBf16::BT);
  const int64_t room = kTargetCUs - 1 - n_app;
  if (room < 1 || n_abs > 2 * room) return false;
  f.n_app = (int)n_app;
  f.n_abs = (int)n_abs;
  f.n_absw = (int)(n_abs < room ? n_abs : room);
  return true;
}

hipError_t launch_append_absorb(const AppendArgs& a, const DecodePlan& plan, const DecodeArgs& d,
                                hipStream_t s) {
  FusedGrid f;
  if (!fused_grid(a, d, f)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_append_absorb_kernel, dim3(f.n_app + f.n_absw + 1), dim3(512), 0, s, a,
                     absorb_params(plan, d), f.n_app, f.n_absw, f.n_abs);
  return hipGetLastError();
}

// Whether the fused launch applies: bf16 cache and activations, and a grid
// that fits the CUs in one round.
bool append_absorb_fits(int cache_type, const AppendArgs& a, const DecodeArgs& d) {
  FusedGrid f;
  return cache_type == kBF16 && fused_grid(a, d, f);
}

hipError_t launch_append(int ct, const AppendArgs& a, hipStream_t s) {
  dim3 grid((a.n_tok + 15) / 16, (ct == kFP8 || ct == kFP6) ? 1 : kNumGroups);
  switch (ct) {
    case kF32: hipLaunchKernelGGL(mla_append_kernel<kF32>, grid, dim3(256), 0, s, a); break;
    case kBF16: hipLaunchKernelGGL(mla_append_bf16_kernel<8>, grid, dim3(512), 0, s, a); break;
    case kFP8: hipLaunchKernelGGL(mla_append_kernel<kFP8>, grid, dim3(256), 0, s, a); break;
    case kFP6: hipLaunchKernelGGL(mla_append_kernel<kFP6>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
