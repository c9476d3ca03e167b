// The two per-head products around the attention kernel (discosf explainer,
// "long-context bottleneck": W_UK is absorbed on the query side and W_UV on
// the output side, so neither K nor V is ever formed):
//   absorb   q_lat[b][h][:] = q_nope[b][h][:] . W_UK[h]          [1x128]x[128x512]
//   project  out[b][h][:]   = (merged o_lat[b][h][:] / l) . W_UV[h] [1x512]x[512x128]
// Both are one GEMM per head over the batch: Y[b][n] = sum_k X[b][k] W[h][k][n].
// The weight's contraction index is its row index, so weight tiles are staged
// in LDS and fed to the MFMA through transposing LDS reads.
//
// The absorb launch also builds the work plan that the attention and merge
// kernels split the sequences' tiles with.
#include "gemm_tile.h"

namespace mla {

// One head-GEMM tile per workgroup: 64 columns of one head for a batch slice
// of 16*NBT rows (the numbering below groups tiles by XCD). The absorb launch has
// one more workgroup, the first (dispatched before the CUs fill up), which
// builds the plan.
template <int AT, int KD, int ND, int NBT, int KC>
__global__ void __launch_bounds__(256)
mla_headgemm_kernel(GemmParams p) {
  using G = HeadGemm<AT, KD, ND, NBT, KC>;
  __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
  int i = blockIdx.x;
  if (p.seq_len) {                                       // workgroup 0 builds the plan
    if (i == 0) {
      build_plan(p, (int64_t*)lds, (int)(G::W_BYTES / 8));
      return;
    }
    --i;
  }
  constexpr int NXB = ND / kNT;
  // The column tiles of one (head, batch slice) read the same X rows, and
  // the batch slices of one head the same weight slices. Workgroups are
  // dispatched to the 8 XCDs in turn, each with its own L2: group (h, slice)
  // j runs on the XCD of workgroups j % 8 (mod 8), so that L2 serves the
  // repeats. A bijection as the group count H * slices is a multiple of 8.
  const int slot = i / 8;
  const int grp = i % 8 + 8 * (slot / NXB);
  typename G::Regs rg;
  const int n0 = (slot % NXB) * kNT, h = grp % p.H, b0 = (grp / p.H) * G::BT;
  G::load(p, n0, h, b0, rg);
  G::run(p, n0, h, b0, rg, lds);
}

// Log-sum-exp merge of the split partials of one (b, h) by one wave. Slot s
// holds the normalised output u_s = o_s / l_s of its segment with (m_s, l_s):
//   M = max_s m_s,  w_s = 2^(m_s - M) l_s,  l = sum_s w_s,
//   o_lat = sum_s w_s u_s / l,
//   lse = (M + log2 l) ln 2.
// merge_slots folds the slots wf+off, wf+off+step, ... (wf, wl: the first and
// last worker of sequence b) into the running state (mmax, lsum, acc), with
// acc the unnormalised sum over dims 8*lane .. 8*lane+7.
template <int AT, int RU>
__device__ __forceinline__ void merge_slots(const GemmParams& p, int b, int h, int lane, int off,
                                            int step, float* acc, float& mmax, float& lsum) {
  const int H = p.H;
  const int64_t wf = ld_const(p.wfirst, b) + off, wl = ld_const(p.wlast, b);
  // rounds of up to RU slots: every address of a round depends only on wf
  // and wl, so all its loads are in flight together; a slot counts only if
  // its worker's range is non-empty (an empty worker writes nothing),
  // which is applied by selection once the data is back
  for (int64_t w0 = wf; w0 <= wl; w0 += (int64_t)RU * step) {
    float m[RU], l[RU];
    int64_t st0[RU], st1[RU];
    f32x4 v0[RU], v1[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int64_t w = (w0 + (int64_t)u * step <= wl) ? w0 + (int64_t)u * step : wl;
      const int64_t s = (w + b) * H + h;
      st0[u] = ld_const(p.starts, w);
      st1[u] = ld_const(p.starts, w + 1);
      m[u] = ld_const(p.part_ml, s * 2);
      l[u] = ld_const(p.part_ml, s * 2 + 1);
      if constexpr (AT == kF32) {
        const float* po = (const float*)p.part_o + s * kDc + 8 * lane;
        v0[u] = *(const f32x4*)po;
        v1[u] = *(const f32x4*)(po + 4);
      } else {
        const u32x4 r = *(const u32x4*)((const uint16_t*)p.part_o + s * kDc + 8 * lane);
        const uint32_t r0 = r[0], r1 = r[1], r2 = r[2], r3 = r[3];
        v0[u] = f32x4{__builtin_bit_cast(float, r0 << 16), __builtin_bit_cast(float, r0 & 0xffff0000u),
                      __builtin_bit_cast(float, r1 << 16), __builtin_bit_cast(float, r1 & 0xffff0000u)};
        v1[u] = f32x4{__builtin_bit_cast(float, r2 << 16), __builtin_bit_cast(float, r2 & 0xffff0000u),
                      __builtin_bit_cast(float, r3 << 16), __builtin_bit_cast(float, r3 & 0xffff0000u)};
      }
    }
    bool ok[RU];
    float rmax = mmax;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      ok[u] = (w0 + (int64_t)u * step <= wl) && st0[u] != st1[u];
      if (ok[u]) rmax = __builtin_fmaxf(rmax, m[u]);
    }
    const float alpha = (mmax == -INFINITY) ? 0.f : exp2f(mmax - rmax);
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      if (ok[u]) {
        // a segment whose scores were all NaN keeps m = -inf and l = NaN:
        // weight 0 * NaN, which carries the NaN into the result
        const float e = ((m[u] == -INFINITY) ? 0.f : exp2f(m[u] - rmax)) * l[u];
        lsum += e;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += e * v0[u][i];
          acc[4 + i] += e * v1[u][i];
        }
      }
    }
    mmax = rmax;
  }
}

// The whole merge of one (b, h): lane l returns dims 8l..8l+7 of o_lat in
// `acc`, and the function returns lse. A sequence of length 0 gets o_lat = 0
// and lse = -inf.
template <int AT, int RU = 8>
__device__ __forceinline__ float merge_row(const GemmParams& p, int b, int h, int lane, float* acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float mmax = -INFINITY, lsum = 0.f;
  merge_slots<AT, RU>(p, b, h, lane, 0, 1, acc, mmax, lsum);
  if (ld_const(p.wlast, b) >= ld_const(p.wfirst, b)) {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv;
  }
  return (lsum > 0.f) ? (mmax + __log2f(lsum)) * kLn2 : -INFINITY;
}

// merge_slots over NR rows at once (bf16 partials): row j is sequence b[j]
// with slot workers wf[j], wf[j]+step, ... up to wl[j]; each round takes RU
// slots of every row, so all NR*RU slot loads of a round are in flight
// together. The per-slot bookkeeping (is the worker non-empty, m_s, l_s and
// the weight 2^(m_s - M) l_s) runs in lane k = j*RU + u of the wave, and the
// weights reach the data through readlane; the arithmetic and its order are
// those of merge_slots. A row with no slot left in a round loads slot 0 (a
// valid address) and ignores it: every load is unconditional, so none waits
// at a branch join.
template <int NR, int RU>
__device__ __forceinline__ void merge_rows(const GemmParams& p, const int* b, const int64_t* wf,
                                           const int64_t* wl, int h, int lane, int step,
                                           float (*acc)[8], float* mmax, float* lsum) {
  static_assert(NR * RU <= 64, "one bookkeeping lane per slot");
  const int H = p.H;
  int64_t n = 0;                                       // slot positions of the longest row
#pragma unroll
  for (int j = 0; j < NR; ++j) n = (wl[j] - wf[j] + 1 > n) ? wl[j] - wf[j] + 1 : n;
  // this lane's bookkeeping slot: row kj, position ku of the round
  const int kj = lane / RU, ku = lane - (lane / RU) * RU;
  int64_t kwf = wf[0], kwl = -1;
  int kb = b[0];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    if (kj == j) {
      kwf = wf[j];
      kwl = wl[j];
      kb = b[j];
    }
  }
  for (int64_t w0 = 0; w0 < n; w0 += (int64_t)RU * step) {
    u32x4 v[NR][RU];                                   // raw bf16 (unpacked at use)
#pragma unroll
    for (int j = 0; j < NR; ++j) {
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int64_t w = wf[j] + w0 + (int64_t)u * step;
        const int64_t s = (w <= wl[j]) ? (w + b[j]) * H + h : (int64_t)h;
        v[j][u] = *(const u32x4*)((const uint16_t*)p.part_o + s * kDc + 8 * lane);
      }
    }
    const int64_t kw = kwf + w0 + (int64_t)ku * step;
    const bool kin = lane < NR * RU && kw <= kwl;
    // all of a round's loads go out before any is used: a load under a
    // branch (a short-circuit test) would be followed by a wait for every
    // load before it
    const int64_t kwc = kin ? kw : 0;
    const int64_t ks = kin ? (kw + kb) * H + h : (int64_t)h;
    const int64_t kst0 = p.starts[kwc], kst1 = p.starts[kwc + 1];
    const float km = p.part_ml[ks * 2];
    const float kl = p.part_ml[ks * 2 + 1];
    const bool kok = kin & (kst0 != kst1);
    float ke = 0.f;                                    // this lane's slot weight
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      float rmax = mmax[j];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const bool oku = __builtin_amdgcn_readlane((int)kok, j * RU + u) != 0;
        if (oku) rmax = __builtin_fmaxf(rmax, __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                  __builtin_bit_cast(int, km), j * RU + u)));
      }
      if (kj == j) ke = kok ? ((km == -INFINITY) ? 0.f : exp2f(km - rmax)) * kl : 0.f;
      const float alpha = (mmax[j] == -INFINITY) ? 0.f : exp2f(mmax[j] - rmax);
      lsum[j] *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[j][i] *= alpha;
      mmax[j] = rmax;
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        if (__builtin_amdgcn_readlane((int)kok, j * RU + u) != 0) {
          // a segment whose scores were all NaN keeps m = -inf and l = NaN:
          // weight 0 * NaN, which carries the NaN into the result
          const float e = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ke), j * RU + u));
          lsum[j] += e;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t x = v[j][u][i];
            acc[j][2 * i] += e * __builtin_bit_cast(float, x << 16);
            acc[j][2 * i + 1] += e * __builtin_bit_cast(float, x & 0xffff0000u);
          }
        }
      }
    }
  }
}

// Merge one (b, h) per wave into o_lat (the q_lat buffer) and lse.
template <int AT>
__global__ void __launch_bounds__(256)
mla_merge_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int B = p.B, H = p.H;
  if (pair >= (int64_t)B * H) return;
  const int b = (int)(pair / H), h = (int)(pair - (int64_t)b * H);
  float acc[8];
  const float lse = merge_row<AT>(p, b, h, lane, acc);
  if (p.lse && lane == 0) p.lse[pair] = lse;
  char* dst = (char*)p.y + (pair * kDc + 8 * lane) * (AT == kF32 ? 4 : 2);
  if constexpr (AT == kF32) {
    *(f32x4*)dst = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(dst + 16) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    *(bf16x8*)dst = pack_bf16x8(acc);
  }
}

// Merge and W_UV in one launch (bf16), for batches whose rows have few
// partial slots: workgroup (64 output columns, head h, 16 batch rows) with
// sixteen waves. Each wave merges one row (all its slot loads in one round)
// while the weight slice is in flight, writes the merged row in bf16 to LDS,
// and four waves then multiply. The two column workgroups of a (head, rows)
// both merge the rows; the first writes lse.
__global__ void __launch_bounds__(1024)
mla_combine_kernel(GemmParams p) {
  using G = HeadGemm<kBF16, kDc, kDv, 1, kDc>;
  constexpr int TPW = 1024;                            // threads
  constexpr int WP = kDc * kNT * 2 / 16;               // 16-byte pieces of the weight slice
  __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
  char* w_lds = lds;
  char* x_lds = lds + G::W_BYTES;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n0 = blockIdx.x * kNT, h = blockIdx.y, b0 = blockIdx.z * 16;
  const int bw = b0 + wave;                            // this wave's row
  // the row's workers (scalar loads; unconditional, so nothing waits for
  // them at a branch join), and the weight slice while the merge runs
  const int bc = bw < p.B ? bw : p.B - 1;
  const int64_t wf[1] = {ld_const(p.wfirst, bc)};
  const int64_t wl[1] = {ld_const(p.wlast, bc)};
  u32x4 wv[WP / TPW];
#pragma unroll
  for (int k = 0; k < WP / TPW; ++k) {
    const int i = tid + TPW * k;
    const int r = i / G::WPR, c = i - r * G::WPR;
    wv[k] = *(const u32x4*)((const char*)p.w + (((int64_t)h * kDc + r) * kDv + n0) * 2 + c * 16);
  }
  {
    float acc[1][8] = {{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
    if (bw < p.B) {
      // one row, its slot bookkeeping in lanes (vector loads: sixteen waves
      // of scalar loads per CU queue at the scalar cache)
      const int bj[1] = {bw};
      float mmax = -INFINITY, lsum = 0.f;
      merge_rows<1, 8>(p, bj, wf, wl, h, lane, 1, acc, &mmax, &lsum);
      if (wl[0] >= wf[0]) {
        const float inv = 1.f / lsum;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[0][i] *= inv;
      }
      if (p.lse && blockIdx.x == 0 && lane == 0)
        p.lse[(int64_t)bw * p.H + h] = (lsum > 0.f) ? (mmax + __log2f(lsum)) * kLn2 : -INFINITY;
    }
    *(bf16x8*)(x_lds + wave * G::XROW + 16 * lane) = pack_bf16x8(acc[0]);
  }
#pragma unroll
  for (int k = 0; k < WP / TPW; ++k) {
    const int i = tid + TPW * k;
    const int r = i / G::WPR, c = i - r * G::WPR;
    *(u32x4*)(w_lds + r * G::WROW + c * 16) = wv[k];
  }
  __syncthreads();
  if (wave >= 4) return;
  const int l16 = lane & 15, g = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < kDc; kk += 32) {
    // A = W^T block: lane (n, g) gets W[kk + 8g + 0..7][16*wave + n]
    const int rs = kk + 8 * g + (l16 >> 2);
    const int cb = (16 * wave + 4 * (l16 & 3)) * 2;
    const s16x4 lo = lds_read_tr16(w_lds, rs * G::WROW + cb);
    const s16x4 hi = lds_read_tr16(w_lds, (rs + 4) * G::WROW + cb);
    const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const bf16x8 bv = lds_read_b128(x_lds, l16 * G::XROW + (kk + 8 * g) * 2);
    acc = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a8), bv, acc);
  }
  // lane holds Y[b0 + l16][n0 + 16*wave + 4g + r]
  const int b = b0 + l16;
  if (b < p.B) {
    const int n = n0 + 16 * wave + 4 * g;
    uint2 v;
    v.x = pack_bf16x2(acc[0], acc[1]);
    v.y = pack_bf16x2(acc[2], acc[3]);
    *(uint2*)((char*)p.y + (((int64_t)b * p.H + h) * kDv + n) * 2) = v;
  }
}

// Merge and W_UV in one launch (bf16) for many (b, h) rows: workgroup (head
// h, RB batch rows) with eight waves, numbered h + H * (row block) so that
// with H a multiple of the 8 XCDs all workgroups of one head share an L2 and
// W_UV[h] (128 KB) comes from HBM about once. The weight streams through LDS
// in four 128-row chunks (two buffers, the next chunk in registers) while the
// waves merge: with 8 or more rows each wave merges whole rows; with fewer,
// 8/R' waves share a row (R' = R rounded up to 1, 2 or 4), each folding every
// (8/R')-th slot, and their states meet in LDS. The merged rows are stored in
// LDS as bf16 (as the fused launch above does); wave w then produces
// output columns 16w..16w+15 of all RB rows.
template <int RB>
__global__ void __launch_bounds__(512)
mla_combine_wide_kernel(GemmParams p) {
  constexpr int NT = 512;
  constexpr int NRB = RB / 16;
  constexpr int KC = 128;                              // weight rows per chunk
  constexpr int NCH = kDc / KC;                        // chunks
  constexpr int WROW = kDv * 2 + 16;                   // LDS stride of a weight row
  constexpr int XROW = kDc * 2 + 16;                   // LDS stride of a merged row
  constexpr int WPR = kDv * 2 / 16;                    // 16-byte pieces per weight row
  constexpr int WPT = KC * WPR / NT;                   // pieces per thread per chunk
  constexpr int W_CHUNK = KC * WROW;
  constexpr int X_BYTES = RB * XROW;
  constexpr int S_ACC = 8 * 64 * 8 * 4;                // split-merge states: 8 x [64 lanes][8]
  static_assert(NRB >= 1 && RB % 16 == 0, "whole 16-row blocks");
  static_assert(KC * WPR % NT == 0, "whole rounds of weight pieces");
  __shared__ __attribute__((aligned(16))) char lds[2 * W_CHUNK + X_BYTES + S_ACC + 8 * 2 * 4];
  char* w_lds = lds;
  char* x_lds = lds + 2 * W_CHUNK;
  float* s_acc = (float*)(x_lds + X_BYTES);
  float* s_ml = s_acc + 8 * 64 * 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int H = p.H, B = p.B;
  const int h = (int)(blockIdx.x % (unsigned)H);
  const int b0 = (int)(blockIdx.x / (unsigned)H) * RB;
  const int R = (B - b0) < RB ? (B - b0) : RB;         // rows of this workgroup

  auto load_w = [&](int c, u32x4* v) {
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int i = tid + NT * k;
      const int r = i / WPR, cc = i - r * WPR;
      v[k] = *(const u32x4*)((const char*)p.w + (((int64_t)h * kDc + c * KC + r) * kDv) * 2 + cc * 16);
    }
  };
  auto store_w = [&](int buf, const u32x4* v) {
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int i = tid + NT * k;
      const int r = i / WPR, cc = i - r * WPR;
      *(u32x4*)(w_lds + buf * W_CHUNK + r * WROW + cc * 16) = v[k];
    }
  };
  u32x4 wv[2][WPT];
  load_w(0, wv[0]);
  load_w(1, wv[1]);

  // ---------------- merge the rows into x_lds ----------------
  if (R >= 8) {
    // rows wave, wave+8, ... in groups of NR, all their slot loads together
    constexpr int NR = RB / 8 < 4 ? RB / 8 : 4;
    for (int r0 = wave; r0 < R; r0 += 8 * NR) {
      int bj[NR];
      int64_t wf[NR], wl[NR];
      float acc[NR][8], mmax[NR], lsum[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int r = r0 + 8 * j;
        bj[j] = b0 + (r < R ? r : 0);
        wf[j] = ld_const(p.wfirst, bj[j]);
        wl[j] = r < R ? ld_const(p.wlast, bj[j]) : wf[j] - 1;
        mmax[j] = -INFINITY;
        lsum[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
      }
      merge_rows<NR, 4>(p, bj, wf, wl, h, lane, 1, acc, mmax, lsum);
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int r = r0 + 8 * j;
        if (r < R) {
          if (wl[j] >= wf[j]) {
            const float inv = 1.f / lsum[j];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] *= inv;
          }
          if (p.lse && lane == 0)
            p.lse[(int64_t)(b0 + r) * H + h] = (lsum[j] > 0.f) ? (mmax[j] + __log2f(lsum[j])) * kLn2 : -INFINITY;
          *(bf16x8*)(x_lds + r * XROW + 16 * lane) = pack_bf16x8(acc[j]);
        }
      }
    }
  } else {
    const int RP = R <= 1 ? 1 : (R <= 2 ? 2 : 4);      // R < 8 here
    const int P = 8 / RP;                              // waves per row (R = 5..7: RP = 4 is
    const int r = wave % RP, part = wave / RP;         //  too few rows: handled below)
    if (R <= 4) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float mmax = -INFINITY, lsum = 0.f;
      if (r < R) {
        const int bj[1] = {b0 + r};
        const int64_t wf[1] = {ld_const(p.wfirst, b0 + r) + part};
        const int64_t wl[1] = {ld_const(p.wlast, b0 + r)};
        float a1[1][8] = {{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
        merge_rows<1, 16>(p, bj, wf, wl, h, lane, P, a1, &mmax, &lsum);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = a1[0][i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) s_acc[(wave * 64 + lane) * 8 + i] = acc[i];
      if (lane == 0) {
        s_ml[wave * 2] = mmax;
        s_ml[wave * 2 + 1] = lsum;
      }
      __syncthreads();
      if (part == 0 && r < R) {
        float M = -INFINITY;
        for (int q = 0; q < P; ++q) M = __builtin_fmaxf(M, s_ml[(q * RP + r) * 2]);
        float l = 0.f;
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < P; ++q) {
          const int wq = q * RP + r;
          const float mq = s_ml[wq * 2];
          const float e = (mq == -INFINITY) ? 0.f : exp2f(mq - M);
          l += e * s_ml[wq * 2 + 1];
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] += e * s_acc[(wq * 64 + lane) * 8 + i];
        }
        const bool any = ld_const(p.wlast, b0 + r) >= ld_const(p.wfirst, b0 + r);
        if (any) {
          const float inv = 1.f / l;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] *= inv;
        }
        if (p.lse && lane == 0)
          p.lse[(int64_t)(b0 + r) * H + h] = (l > 0.f) ? (M + __log2f(l)) * kLn2 : -INFINITY;
        *(bf16x8*)(x_lds + r * XROW + 16 * lane) = pack_bf16x8(o);
      }
    } else {
      if (wave < R) {
        float acc[8];
        const float lse = merge_row<kBF16>(p, b0 + wave, h, lane, acc);
        if (p.lse && lane == 0) p.lse[(int64_t)(b0 + wave) * H + h] = lse;
        *(bf16x8*)(x_lds + wave * XROW + 16 * lane) = pack_bf16x8(acc);
      }
    }
  }
  store_w(0, wv[0]);
  __syncthreads();

  // ---------------- out rows = merged rows . W_UV[h] ----------------
  const int l16 = lane & 15, g = lane >> 4;
  const int nrb = (R + 15) >> 4;                       // row blocks holding rows
  f32x4 acc[NRB];
#pragma unroll
  for (int i = 0; i < NRB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) store_w((c + 1) & 1, wv[(c + 1) & 1]);   // its buffer's chunk c-1 is done
    if (c + 2 < NCH) load_w(c + 2, wv[c & 1]);
    const char* wb = w_lds + (c & 1) * W_CHUNK;
#pragma unroll
    for (int kk = 0; kk < KC; kk += 32) {
      // A = W^T block: lane (n, g) gets W[c*KC + kk + 8g + 0..7][16*wave + n]
      const int rs = kk + 8 * g + (l16 >> 2);
      const int cb = (16 * wave + 4 * (l16 & 3)) * 2;
      const s16x4 lo = lds_read_tr16(wb, rs * WROW + cb);
      const s16x4 hi = lds_read_tr16(wb, (rs + 4) * WROW + cb);
      const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if (rb < nrb) {
          const bf16x8 bv = lds_read_b128(x_lds, (16 * rb + l16) * XROW + (c * KC + kk + 8 * g) * 2);
          acc[rb] = mfma_bf16_k32(a, bv, acc[rb]);
        }
      }
    }
    __syncthreads();
  }
  // lane holds out[b0 + 16 rb + l16][16*wave + 4g + r]
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = 16 * rb + l16;
    if (row < R) {
      const int n = 16 * wave + 4 * g;
      uint2 v;
      v.x = pack_bf16x2(acc[rb][0], acc[rb][1]);
      v.y = pack_bf16x2(acc[rb][2], acc[rb][3]);
      *(uint2*)((char*)p.y + (((int64_t)(b0 + row) * H + h) * kDv + n) * 2) = v;
    }
  }
}

template <int AT, int KD, int ND, int NBT, int KC>
static hipError_t launch_gemm_t(const GemmParams& prm, hipStream_t s) {
  constexpr int BT = 16 * NBT;
  // absorb (seq_len given) gets one more workgroup, which builds the plan
  const int64_t n = (int64_t)(ND / kNT) * prm.H * ((prm.B + BT - 1) / BT) + (prm.seq_len ? 1 : 0);
  hipLaunchKernelGGL((mla_headgemm_kernel<AT, KD, ND, NBT, KC>), dim3((unsigned)n), dim3(256), 0, s,
                     prm);
  return hipGetLastError();
}

hipError_t launch_attn(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s);

hipError_t launch_decode(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s,
                         int stage) {
  const bool f32 = (ct == kF32);
  hipError_t e = hipSuccess;
  // 1. absorb W_UK into the query; build the work plan
  if (stage == 0 || stage == 1) {
    const GemmParams g = absorb_params(plan, a);
    // bf16: 64 batch rows per workgroup, 32 for batches of at most 32
    e = f32 ? launch_gemm_t<kF32, kDnope, kDc, 1, kDnope>(g, s)
            : (a.B <= 32 ? launch_gemm_t<kBF16, kDnope, kDc, 2, kDnope>(g, s)
                         : launch_gemm_t<kBF16, kDnope, kDc, 4, kDnope>(g, s));
    if (e != hipSuccess) return e;
  }
  // 2. attention over the latent rows -> split partials
  if (stage == 0 || stage == 2 || stage == 4) {
    e = launch_attn(ct, plan, a, s);
    if (e != hipSuccess) return e;
  }
  if (stage != 0 && stage != 3 && stage != 4) return e;
  // 3. merge the partials and apply W_UV. bf16: one launch, per (64 output
  //    columns, head, 16 rows) when the sequences have few slots each (one
  //    merge round per row, on average) and its workgroups fit the CUs at
  //    once, else per (head, row block). fp32: merge, then projection.
  const int64_t comb_wgs = (int64_t)(kDv / kNT) * a.H * ((a.B + 15) / 16);
  if (!f32 && plan.nslot <= 6 * (int64_t)a.B && comb_wgs <= kTargetCUs) {
    GemmParams c{};
    c.B = a.B;
    c.H = a.H;
    c.starts = a.starts;
    c.wfirst = a.wfirst;
    c.wlast = a.wlast;
    c.part_o = a.part_o;
    c.part_ml = a.part_ml;
    c.lse = a.lse;
    c.w = a.w_uv;
    c.y = a.out;
    hipLaunchKernelGGL(mla_combine_kernel, dim3(kDv / kNT, a.H, (a.B + 15) / 16), dim3(1024), 0, s,
                       c);
    return hipGetLastError();
  }
  if (!f32) {
    // many rows: merge + W_UV per (head, row block), the largest block that
    // still gives every CU a workgroup (16 rows when none does); H is a
    // multiple of 16, so the workgroups of one head share an XCD
    GemmParams c{};
    c.B = a.B;
    c.H = a.H;
    c.starts = a.starts;
    c.wfirst = a.wfirst;
    c.wlast = a.wlast;
    c.part_o = a.part_o;
    c.part_ml = a.part_ml;
    c.lse = a.lse;
    c.w = a.w_uv;
    c.y = a.out;
    auto wgs = [&](int rb) { return (int64_t)a.H * ((a.B + rb - 1) / rb); };
    if (wgs(64) >= kTargetCUs) {
      hipLaunchKernelGGL(mla_combine_wide_kernel<64>, dim3((unsigned)wgs(64)), dim3(512), 0, s, c);
    } else if (wgs(32) >= kTargetCUs) {
      hipLaunchKernelGGL(mla_combine_wide_kernel<32>, dim3((unsigned)wgs(32)), dim3(512), 0, s, c);
    } else {
      hipLaunchKernelGGL(mla_combine_wide_kernel<16>, dim3((unsigned)wgs(16)), dim3(512), 0, s, c);
    }
    return hipGetLastError();
  }
  // fp32: the merge (into the q_lat buffer, free once attention is done),
  // then the projection
  GemmParams m{};
  m.B = a.B;
  m.H = a.H;
  m.workers = plan.workers;
  m.seqinfo = a.seqinfo;
  m.starts = a.starts;
  m.wfirst = a.wfirst;
  m.wlast = a.wlast;
  m.y = a.q_lat;
  m.lse = a.lse;
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  const int64_t pairs = (int64_t)a.B * a.H;
  hipLaunchKernelGGL(mla_merge_kernel<kF32>, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, s, m);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmParams g{};
  g.B = a.B;
  g.H = a.H;
  g.x = a.q_lat;
  g.w = a.w_uv;
  g.y = a.out;
  return launch_gemm_t<kF32, kDc, kDv, 1, 128>(g, s);
}

}  // namespace mla
