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
  int32_t B;
  int32_t H;
  int32_t workers;            // W of the attention launch
  int32_t tile;               // tokens per tile of the attention launch
};

constexpr int kNT = 64;       // output columns per workgroup (one 16-wide block per wave)

// The work plan, built by one extra workgroup of the absorb launch so the
// attention and merge kernels need no divisions or searches. Sequence b has
// n_b = ceil(len_b / tile) tiles (len clamped to [0, capacity]); P_b is the
// prefix sum of n, NT = P_B, and the tiles of all sequences form one stream:
//   seqinfo[b] = {first cache row, len_b, P_b, P_(b+1), next sequence with tiles}
//   starts[w]  = floor(w * NT / W): worker w takes tiles [starts[w], starts[w+1])
//   wseq[w]    = the sequence holding tile starts[w] (non-empty workers)
//   wfirst[b], wlast[b] = first and last worker that touch sequence b
//                (wlast < wfirst for an empty sequence)
// Splitting whole tiles keeps every split inside a sequence on a tile
// boundary, so the only partial tile of a sequence is its last one.
// floor(w NT / W) >= P exactly when w >= ceil(P W / NT), so sequence b holds
// the starts of workers [ceil(P_b W/NT), ceil(P_(b+1) W/NT)), its first
// worker is ceil((P_b + 1) W / NT) - 1 and its last ceil(P_(b+1) W / NT) - 1:
// every entry is a closed form of the prefix sums, which stay in LDS (`lds`,
// room for `lds_n` values) when they fit.
__device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ void build_plan(const GemmParams& p, int64_t* lds, int lds_n) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = p.B;
  const int64_t W = p.workers;
  const int TL = p.tile;
  const bool in_lds = B + 1 <= lds_n;
  if (tid < 64) {
    int64_t carry = 0;
    if (lane == 0 && in_lds) lds[0] = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      int L = 0;
      if (b < B) {
        const int Lr = p.seq_len[b];
        const int cap = p.seq_cap[b];
        L = Lr < 0 ? 0 : (Lr > cap ? cap : Lr);
      }
      const int64_t n = (L + TL - 1) / TL;
      int64_t v = n;
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
        si.row0 = p.seq_start[b];
        si.len = L;
        si.tile0 = (int32_t)(carry + v - n);
        si.tile1 = (int32_t)(carry + v);
        si.next = B;                                     // set below
        si.pad[0] = si.pad[1] = 0;
        p.seqinfo[b] = si;
        if (in_lds) lds[b + 1] = carry + v;
      }
      const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffff), 63);
      const int hi = __builtin_amdgcn_readlane((int)(v >> 32), 63);
      carry += ((int64_t)hi << 32) | (uint32_t)lo;
    }
    if (!in_lds && lane == 0) lds[0] = carry;            // NT for the other waves
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const volatile int32_t* gtile0 = &p.seqinfo[0].tile0;
  // P_b for b < B (P_B = NT)
  auto prefix = [&](int b) -> int64_t {
    return in_lds ? lds[b] : (int64_t)gtile0[(int64_t)b * (sizeof(SeqInfo) / 4)];
  };
  const int64_t NT = in_lds ? lds[B] : lds[0];
  for (int64_t w = tid; w <= W; w += 256) p.starts[w] = (w * NT) / W;
  if (NT == 0) {
    for (int64_t w = tid; w < W; w += 256) p.wseq[w] = 0;
  }
  for (int b = tid; b < B; b += 256) {
    const int64_t P0 = prefix(b), P1 = (b + 1 < B) ? prefix(b + 1) : NT;
    if (P1 > P0) {
      const int64_t wlo = ceil_div64(P0 * W, NT), whi = ceil_div64(P1 * W, NT);
      for (int64_t w = wlo; w < whi; ++w) p.wseq[w] = b;
      p.wfirst[b] = (int)(ceil_div64((P0 + 1) * W, NT) - 1);
      p.wlast[b] = (int)(whi - 1);
    } else {
      p.wfirst[b] = 0;
      p.wlast[b] = -1;
    }
    // next sequence with tiles: the largest b' > b with P_b' <= P_(b+1), which
    // owns tile P_(b+1) (none when P_(b+1) = NT)
    int nx = B;
    if (P1 < NT) {
      int lo = b + 1, hi = B - 1;                        // P_lo <= P1 holds (P_(b+1) = P1)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix(mid) <= P1) lo = mid;
        else hi = mid - 1;
      }
      nx = lo;
    }
    p.seqinfo[b].next = nx;
  }
  // each worker's starting point, from the records above
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int64_t w = tid; w < W; w += 256) {
    const int64_t r_lo = (w * NT) / W, r_hi = ((w + 1) * NT) / W;
    WorkerInfo wi;
    wi.r_hi = (int32_t)r_hi;
    wi.pad = 0;
    if (r_lo >= r_hi) {
      wi.row0 = 0;
      wi.b = -1;
      wi.t = wi.t_end = 0;
      wi.next = B;
    } else {
      const int b = ((const volatile int32_t*)p.wseq)[w];
      const volatile SeqInfo* si = p.seqinfo + b;
      const int64_t t0 = si->tile0, t1 = si->tile1, len = si->len;
      const int64_t se = t1 < r_hi ? t1 : r_hi;
      wi.b = b;
      wi.t = (int32_t)((r_lo - t0) * TL);
      wi.t_end = (int32_t)((se - t0) * TL < len ? (se - t0) * TL : len);
      wi.row0 = si->row0 + wi.t;
      wi.next = si->next;
    }
    p.winfo[w] = wi;
  }
}

// Y[b][h][:] = X[b][h][:] . W[h] for one head (blockIdx.y), 64 output columns
// (blockIdx.x) and 16*NBT batch rows (blockIdx.z). AT: kF32 or kBF16, the
// element type of x, w and y. The weight slice W[h][0:KD][n0:n0+64] is
// staged in LDS KC rows at a time.
template <int AT, int KD, int ND, int NBT, int KC>
__global__ void __launch_bounds__(256)
mla_headgemm_kernel(GemmParams p) {
  using E = typename std::conditional<AT == kF32, float, __bf16>::type;
  constexpr int ES = sizeof(E);
  constexpr int BT = 16 * NBT;                        // batch rows per workgroup
  constexpr int WROW = kNT * ES + 16;                 // LDS stride of a weight row
  constexpr int XROW = KD * ES + 16;                  // LDS stride of an X row
  constexpr int XP = BT * KD * ES / 16;               // 16-byte pieces of the X tile
  constexpr int WP = KC * kNT * ES / 16;              // 16-byte pieces of one weight chunk
  static_assert(XP % 256 == 0 && WP % 256 == 0, "whole rounds of 16-byte pieces");
  __shared__ __attribute__((aligned(16))) char w_lds[KC * WROW];
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

  if (p.seq_len && blockIdx.z == gridDim.z - 1) {       // the extra plan workgroup
    if (blockIdx.x == 0 && blockIdx.y == 0)
      build_plan(p, (int64_t*)w_lds, (int)(sizeof(w_lds) / 8));
    return;
  }

  // ---------------- X tile and the first weight chunk -> LDS ----------------
  // (every load of both is issued before any store, so the two round trips
  // to memory overlap)
  constexpr int XPR = KD * ES / 16;                    // 16-byte pieces per X row
  constexpr int WPR = kNT * ES / 16;                   // 16-byte pieces per weight row
  auto load_w = [&](int k0, u32x4* v) {
#pragma unroll
    for (int k = 0; k < WP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / WPR, c = i - r * WPR;
      v[k] = *(const u32x4*)((const char*)p.w + (((int64_t)h * KD + k0 + r) * ND + n0) * ES + c * 16);
    }
  };
  auto store_w = [&](const u32x4* v) {
#pragma unroll
    for (int k = 0; k < WP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / WPR, c = i - r * WPR;
      *(u32x4*)(w_lds + r * WROW + c * 16) = v[k];
    }
  };
  {
    u32x4 xv[XP / 256], wv[WP / 256];
#pragma unroll
    for (int k = 0; k < XP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / XPR, c = i - r * XPR;
      const int b = b0 + r;
      xv[k] = u32x4{0u, 0u, 0u, 0u};
      if (b < B) xv[k] = *(const u32x4*)((const char*)p.x + (((int64_t)b * H + h) * KD) * ES + c * 16);
    }
    load_w(0, wv);
#pragma unroll
    for (int k = 0; k < XP / 256; ++k) {
      const int i = tid + 256 * k;
      const int r = i / XPR, c = i - r * XPR;
      *(u32x4*)(x_lds + r * XROW + c * 16) = xv[k];
    }
    store_w(wv);
  }

  f32x4 acc[NBT];
#pragma unroll
  for (int i = 0; i < NBT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < KD; k0 += KC) {
    if (k0) {
      u32x4 wv[WP / 256];
      load_w(k0, wv);
      __syncthreads();                                 // previous chunk consumed
      store_w(wv);
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

// Log-sum-exp merge of the split partials of one (b, h) by one wave. Slot s
// holds the normalised output u_s = o_s / l_s of its segment with (m_s, l_s):
//   M = max_s m_s,  w_s = 2^(m_s - M) l_s,  l = sum_s w_s,
//   o_lat = sum_s w_s u_s / l,
//   lse = (M + log2 l) ln 2.
// Lane l returns dims 8l..8l+7 of o_lat in `acc`. A sequence of length 0
// gets o_lat = 0 and lse = -inf.
template <int AT>
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
    constexpr int RU = 8;
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

template <int AT, int KD, int ND, int NBT, int KC>
static hipError_t launch_gemm_t(const GemmParams& prm, hipStream_t s) {
  constexpr int BT = 16 * NBT;
  // absorb (seq_len given) gets one more z slice whose first block builds the plan
  dim3 grid(ND / kNT, prm.H, (prm.B + BT - 1) / BT + (prm.seq_len ? 1 : 0));
  hipLaunchKernelGGL((mla_headgemm_kernel<AT, KD, ND, NBT, KC>), grid, dim3(256), 0, s, prm);
  return hipGetLastError();
}

hipError_t launch_attn(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s);

hipError_t launch_decode(int ct, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s,
                         int stage) {
  const bool f32 = (ct == kF32);
  hipError_t e = hipSuccess;
  // 1. absorb W_UK into the query; build the work plan
  if (stage == 0 || stage == 1) {
    GemmParams g{};
    g.B = a.B;
    g.H = a.H;
    g.workers = plan.workers;
    g.seqinfo = a.seqinfo;
    g.winfo = a.winfo;
    g.starts = a.starts;
    g.seq_start = a.seq_start;
    g.tile = plan.tile;
    g.wseq = a.wseq;
    g.wfirst = a.wfirst;
    g.wlast = a.wlast;
    g.seq_len = a.seq_len;
    g.seq_cap = a.seq_cap;
    g.x = a.q_nope;
    g.w = a.w_uk;
    g.y = a.q_lat;
    e = f32 ? launch_gemm_t<kF32, kDnope, kDc, 1, kDnope>(g, s)
            : launch_gemm_t<kBF16, kDnope, kDc, 4, kDnope>(g, s);
    if (e != hipSuccess) return e;
  }
  // 2. attention over the latent rows -> split partials
  if (stage == 0 || stage == 2) {
    e = launch_attn(ct, plan, a, s);
    if (e != hipSuccess) return e;
  }
  if (stage != 0 && stage != 3) return e;
  // 3. merge the partials (into the q_lat buffer, free once attention is
  //    done) and apply W_UV
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
