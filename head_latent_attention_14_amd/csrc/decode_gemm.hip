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

// One head-GEMM tile per workgroup, numbered (64-column block, head, batch
// slice of 16*NBT rows) with the column block fastest. The absorb launch has
// one more workgroup, the last, which builds the plan.
template <int AT, int KD, int ND, int NBT, int KC>
__global__ void __launch_bounds__(256)
mla_headgemm_kernel(GemmParams p) {
  using G = HeadGemm<AT, KD, ND, NBT, KC>;
  __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
  const int i = blockIdx.x;
  if (p.seq_len && i == (int)gridDim.x - 1) {           // the extra plan workgroup
    build_plan(p, (int64_t*)lds, (int)(G::W_BYTES / 8));
    return;
  }
  constexpr int NXB = ND / kNT;
  typename G::Regs rg;
  const int n0 = (i % NXB) * kNT, h = (i / NXB) % p.H, b0 = (i / NXB / p.H) * G::BT;
  G::load(p, n0, h, b0, rg);
  G::run(p, n0, h, b0, rg, lds);
}

// Log-sum-exp merge of the split partials of one (b, h) by one wave. Slot s
// holds the normalised output u_s = o_s / l_s of its segment with (m_s, l_s):
//   M = max_s m_s,  w_s = 2^(m_s - M) l_s,  l = sum_s w_s,
//   o_lat = sum_s w_s u_s / l,
//   lse = (M + log2 l) ln 2.
// Lane l returns dims 8l..8l+7 of o_lat in `acc`. A sequence of length 0
// gets o_lat = 0 and lse = -inf.
template <int AT, int RU = 8>
__device__ __forceinline__ float merge_row(const GemmParams& p, int b, int h, int lane, float* acc) {
  const int H = p.H;
  const int64_t wf = ld_const(p.wfirst, b), wl = ld_const(p.wlast, b);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float mmax = -INFINITY, lsum = 0.f;
  if (wl >= wf) {
    // rounds of up to RU slots: every address of a round depends only on wf
    // and wl, so all its loads are in flight together; a slot counts only if
    // its worker's range is non-empty (an empty worker writes nothing),
    // which is applied by selection once the data is back
    for (int64_t w0 = wf; w0 <= wl; w0 += RU) {
      float m[RU], l[RU];
      int64_t st0[RU], st1[RU];
      f32x4 v0[RU], v1[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int64_t w = (w0 + u <= wl) ? w0 + u : wl;
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
        ok[u] = (w0 + u <= wl) && st0[u] != st1[u];
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
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv;
  }
  return (lsum > 0.f) ? (mmax + __log2f(lsum)) * kLn2 : -INFINITY;
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
// while the weight slice is in flight, writes the merged row in bf16 to LDS
// (the value the separate merge stores), and four waves then multiply. The
// two column workgroups of a (head, rows) both merge the rows; the first
// writes lse.
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
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * kNT, h = blockIdx.y, b0 = blockIdx.z * 16;
  u32x4 wv[WP / TPW];
#pragma unroll
  for (int k = 0; k < WP / TPW; ++k) {
    const int i = tid + TPW * k;
    const int r = i / G::WPR, c = i - r * G::WPR;
    wv[k] = *(const u32x4*)((const char*)p.w + (((int64_t)h * kDc + r) * kDv + n0) * 2 + c * 16);
  }
  {
    const int b = b0 + wave;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (b < p.B) {
      const float lse = merge_row<kBF16, 6>(p, b, h, lane, acc);
      if (p.lse && blockIdx.x == 0 && lane == 0) p.lse[(int64_t)b * p.H + h] = lse;
    }
    *(bf16x8*)(x_lds + wave * G::XROW + 16 * lane) = pack_bf16x8(acc);
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
  if (stage == 0 || stage == 2) {
    e = launch_attn(ct, plan, a, s);
    if (e != hipSuccess) return e;
  }
  if (stage != 0 && stage != 3) return e;
  // 3. merge the partials and apply W_UV: one fused launch (bf16) when the
  //    sequences have few slots each (one merge round per row, on average)
  //    and its workgroups fit the CUs at once, else the merge (into the q_lat
  //    buffer, free once attention is done) and the projection
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
  dim3 mgrid((unsigned)((pairs + 3) / 4));
  if (f32)
    hipLaunchKernelGGL(mla_merge_kernel<kF32>, mgrid, dim3(256), 0, s, m);
  else
    hipLaunchKernelGGL(mla_merge_kernel<kBF16>, mgrid, dim3(256), 0, s, m);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmParams g{};
  g.B = a.B;
  g.H = a.H;
  g.x = a.q_lat;
  g.w = a.w_uv;
  g.y = a.out;
  if (f32) return launch_gemm_t<kF32, kDc, kDv, 1, 128>(g, s);
  // 16, 32 or 64 batch rows per workgroup, whichever loads fewer bytes per CU:
  // each workgroup reads a 64 KB weight slice and 16 KB of merged output per
  // 16 rows, and every 256 workgroups share the CUs once more
  auto per_cu = [&](int nbt) {
    const int64_t wgs = (int64_t)(kDv / kNT) * a.H * ((a.B + 16 * nbt - 1) / (16 * nbt));
    const int64_t rounds = (wgs + kTargetCUs - 1) / kTargetCUs;
    return rounds * (64 + 16 * nbt);
  };
  const int64_t c1 = per_cu(1), c2 = per_cu(2), c4 = per_cu(4);
  if (c4 < c2 && c4 < c1) return launch_gemm_t<kBF16, kDc, kDv, 4, kDc>(g, s);
  return c2 < c1 ? launch_gemm_t<kBF16, kDc, kDv, 2, kDc>(g, s)
                 : launch_gemm_t<kBF16, kDc, kDv, 1, kDc>(g, s);
}

}  // namespace mla
