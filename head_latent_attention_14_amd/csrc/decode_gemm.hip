// The two per-head products around the attention kernel (discosf explainer,
// "long-context bottleneck": W_UK is absorbed on the query side and W_UV on
// the output side, so neither K nor V is ever formed):
//   absorb   q_lat[b][h][:] = q_nope[b][h][:] . W_UK[h]          [1x128]x[128x512]
//   project  out[b][h][:]   = (merged o_lat[b][h][:] / l) . W_UV[h] [1x512]x[512x128]
// Both are one GEMM per head over the batch: Y[b][n] = sum_k X[b][k] W[h][k][n].
// The weight's contraction index is its row index, so weight tiles are staged
// in LDS and fed to the MFMA through transposing LDS reads.
//
// The absorb launch also builds the prefix sums of the clamped sequence
// lengths that the attention and merge kernels partition work with.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace mla {

struct GemmParams {
  const void* x;              // absorb: q_nope [B][H][128]
  const void* w;              // [H][KD][ND]
  void* y;                    // absorb: q_lat [B][H][512]; project: out [B][H][128]
  float* lse;                 // project: [B][H] or null
  const float* part_o;        // project: [nslot][H][512]
  const float* part_ml;       // project: [nslot][H][2]
  int64_t* prefix;            // [B+1] (written by absorb, read by project)
  const int32_t* seq_len;     // absorb: [B]
  const int32_t* seq_cap;     // absorb: [B]
  int32_t B;
  int32_t H;
  int32_t workers;            // W of the attention launch
};

constexpr int kNT = 64;       // output columns per workgroup (one 16-wide block per wave)
constexpr int kKC = 128;      // weight rows staged per K chunk

// inclusive prefix of clamped lengths, written by one wave
__device__ void build_prefix(const GemmParams& p) {
  const int lane = threadIdx.x & 63;
  int64_t carry = 0;
  if (lane == 0) p.prefix[0] = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    int64_t v = 0;
    if (b < p.B) {
      int L = p.seq_len[b];
      const int cap = p.seq_cap[b];
      L = L < 0 ? 0 : (L > cap ? cap : L);
      v = L;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int src = lane - off;
      const int lo = __builtin_amdgcn_ds_bpermute((src < 0 ? lane : src) << 2, (int)(v & 0xffffffff));
      const int hi = __builtin_amdgcn_ds_bpermute((src < 0 ? lane : src) << 2, (int)(v >> 32));
      const int64_t u = ((int64_t)hi << 32) | (uint32_t)lo;
      if (src >= 0) v += u;
    }
    if (b < p.B) p.prefix[b + 1] = carry + v;
    const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffff), 63);
    const int hi = __builtin_amdgcn_readlane((int)(v >> 32), 63);
    carry += ((int64_t)hi << 32) | (uint32_t)lo;
  }
}

// AT: kF32 or kBF16 (element type of x, w, y); MODE 0 = absorb, 1 = project
template <int AT, int MODE, int KD, int ND, int NBT>
__global__ void __launch_bounds__(256)
mla_headgemm_kernel(GemmParams p) {
  using E = typename std::conditional<AT == kF32, float, __bf16>::type;
  constexpr int ES = sizeof(E);
  constexpr int BT = 16 * NBT;                        // batch rows per workgroup
  constexpr int WROW = kNT * ES + 16;                 // LDS stride of a weight row
  constexpr int XROW = KD * ES + 16;                  // LDS stride of an X row
  __shared__ __attribute__((aligned(16))) char w_lds[kKC * WROW];
  __shared__ __attribute__((aligned(16))) char x_lds[BT * XROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * kNT;
  const int h = blockIdx.y;
  const int b0 = blockIdx.z * BT;
  const int H = p.H, B = p.B;

  if constexpr (MODE == 0) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && wave == 0) build_prefix(p);
  }

  // ---------------- X tile -> LDS ----------------
  if constexpr (MODE == 0) {
    // q_nope rows: KD elements each, 16-byte pieces
    constexpr int PPR = KD * ES / 16;
    for (int i = tid; i < BT * PPR; i += 256) {
      const int r = i / PPR, c = i - r * PPR;
      const int b = b0 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (b < B) v = *(const u32x4*)((const char*)p.x + (((int64_t)b * H + h) * KD) * ES + c * 16);
      *(u32x4*)(x_lds + r * XROW + c * 16) = v;
    }
  } else {
    // merge the split partials of each (b, h) into the normalised o_lat row
    const int64_t T = p.prefix[B];
    const int64_t W = p.workers;
    for (int r = 0; r < BT; ++r) {
      const int b = b0 + r;
      float acc0 = 0.f, acc1 = 0.f;                   // elements 2*tid, 2*tid+1
      float mmax = -INFINITY, lsum = 0.f;
      if (b < B) {
        const int64_t P0 = p.prefix[b], P1 = p.prefix[b + 1];
        if (P1 > P0) {
          const int64_t wf = find_worker(P0, W, T), wl = find_worker(P1 - 1, W, T);
          for (int64_t w = wf; w <= wl; ++w) {
            if (worker_start(w, W, T) == worker_start(w + 1, W, T)) continue;
            mmax = __builtin_fmaxf(mmax, p.part_ml[((w + b) * H + h) * 2]);
          }
          for (int64_t w = wf; w <= wl; ++w) {
            if (worker_start(w, W, T) == worker_start(w + 1, W, T)) continue;
            const int64_t s = (w + b) * H + h;
            const float e = exp2f(p.part_ml[s * 2] - mmax);
            lsum += e * p.part_ml[s * 2 + 1];
            const float2 v = *(const float2*)(p.part_o + s * kDc + 2 * tid);
            acc0 += e * v.x;
            acc1 += e * v.y;
          }
          const float inv = 1.f / lsum;
          acc0 *= inv;
          acc1 *= inv;
        }
        if (p.lse && tid == 0 && blockIdx.x == 0)
          p.lse[(int64_t)b * H + h] = (lsum > 0.f) ? (mmax + __log2f(lsum)) * kLn2 : -INFINITY;
      }
      if constexpr (AT == kF32) {
        *(float2*)(x_lds + r * XROW + 8 * tid) = make_float2(acc0, acc1);
      } else {
        *(uint32_t*)(x_lds + r * XROW + 4 * tid) = pack_bf16x2(acc0, acc1);
      }
    }
  }

  // ---------------- GEMM over K chunks ----------------
  f32x4 acc[NBT];
#pragma unroll
  for (int i = 0; i < NBT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < KD; k0 += kKC) {
    __syncthreads();                                   // X ready / previous chunk consumed
    constexpr int PPR = kNT * ES / 16;                 // 16-byte pieces per weight row
    for (int i = tid; i < kKC * PPR; i += 256) {
      const int r = i / PPR, c = i - r * PPR;
      const u32x4 v = *(const u32x4*)((const char*)p.w +
                                       (((int64_t)h * KD + k0 + r) * ND + n0) * ES + c * 16);
      *(u32x4*)(w_lds + r * WROW + c * 16) = v;
    }
    __syncthreads();
    if constexpr (AT == kF32) {
#pragma unroll 4
      for (int kk = 0; kk < kKC; kk += 4) {
        const float a = *(const float*)(w_lds + (kk + g) * WROW + (16 * wave + l16) * 4);
#pragma unroll
        for (int nb = 0; nb < NBT; ++nb) {
          const float bv = *(const float*)(x_lds + (16 * nb + l16) * XROW + (k0 + kk + g) * 4);
          acc[nb] = mfma_f32_k4(a, bv, acc[nb]);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < kKC; kk += 32) {
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

template <int AT, int MODE, int KD, int ND, int NBT>
static hipError_t launch_gemm_t(const GemmParams& prm, hipStream_t s) {
  constexpr int BT = 16 * NBT;
  dim3 grid(ND / kNT, prm.H, (prm.B + BT - 1) / BT);
  hipLaunchKernelGGL((mla_headgemm_kernel<AT, MODE, KD, ND, NBT>), grid, dim3(256), 0, s, prm);
  return hipGetLastError();
}

hipError_t launch_attn(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s);

hipError_t launch_decode(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  GemmParams g{};
  g.B = a.B;
  g.H = a.H;
  g.workers = plan.workers;
  g.prefix = a.prefix;
  g.seq_len = a.seq_len;
  g.seq_cap = a.seq_cap;
  const bool f32 = (ct == kF32);
  // 1. absorb W_UK into the query; build the length prefix
  g.x = a.q_nope;
  g.w = a.w_uk;
  g.y = a.q_lat;
  hipError_t e = f32 ? launch_gemm_t<kF32, 0, kDnope, kDc, 1>(g, s)
                     : launch_gemm_t<kBF16, 0, kDnope, kDc, 4>(g, s);
  if (e != hipSuccess) return e;
  // 2. attention over the latent rows -> split partials
  e = launch_attn(ct, plan, a, s);
  if (e != hipSuccess) return e;
  // 3. merge the partials and apply W_UV
  GemmParams m{};
  m.B = a.B;
  m.H = a.H;
  m.workers = plan.workers;
  m.prefix = a.prefix;
  m.w = a.w_uv;
  m.y = a.out;
  m.lse = a.lse;
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  return f32 ? launch_gemm_t<kF32, 1, kDc, kDv, 1>(m, s)
             : launch_gemm_t<kBF16, 1, kDc, kDv, 2>(m, s);
}

}  // namespace mla
