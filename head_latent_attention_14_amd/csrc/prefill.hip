// MLA prefill / multi-query attention over the latent cache: the queries of
// sequence b are its last n_b positions, and the query at position p attends
// rows 0..p of b (causal). The pages report prompt processing beside
// generation (DeepSeek-V2 reading card, "Evidence": over 100K prompt tokens/s
// on one 8-GPU node) without a prefill formula; the score, softmax and output
// are decode's.
//
// With many queries per sequence the unabsorbed form is the cheaper one: a
// (query, row) pair then costs 128 + 64 multiply-adds for the score and 128
// for the value per head, against 576 + 512 over the latent, and the
// up-projection K = W_UK c, V = W_UV^T c is paid once per row (discosf
// explainer, "long-context bottleneck": the latent is up-projected to K/V at
// attention time). Three launches:
//   plan   one workgroup: per-sequence prefix sums of the padded K/V rows and
//          of the query blocks;
//   kv     per (head, 128 cached rows): K[h] (128 dims, then a copy of the
//          row's RoPE key, so that a K row is one 384-byte run) and V[h] (128
//          dims) as bf16 into the workspace, on bf16 MFMA (fp8 caches: codes
//          widened exactly, scales applied to the fp32 products);
//   attn   per (head, 256 queries): 8 waves of 32 queries stream 64-row K/V
//          blocks through a two-stage LDS ring (asynchronous global->LDS
//          copies), S^T = K Q^T and O^T += V^T P^T on 16x16x32 bf16 MFMA with
//          an online softmax, the causal mask on the diagonal blocks only.
#include <type_traits>

#include "attn_tile.h"

namespace mla {

// ------------------------------------------------------------------ plan
__global__ void __launch_bounds__(256) mla_prefill_plan_kernel(PrefillArgs a) {
  __shared__ int64_t s_kv[256];
  __shared__ int32_t s_qb[256];
  const int tid = threadIdx.x;
  int64_t carry_kv = 0;
  int32_t carry_qb = 0;
  for (int base = 0; base < a.B; base += 256) {
    const int b = base + tid;
    int len = 0, n = 0;
    int64_t kvr = 0;
    int32_t qb = 0;
    if (b < a.B) {
      const int cap = a.block_table ? a.max_pages * a.page_tokens
                                    : (a.seq_cap[b] > 0 ? a.seq_cap[b] : 0);
      len = a.seq_len[b];
      len = len < 0 ? 0 : (len > cap ? cap : len);
      int64_t q0 = a.q_start[b], q1 = a.q_start[b + 1];
      q0 = q0 < 0 ? 0 : (q0 > a.n_q ? a.n_q : q0);
      q1 = q1 < q0 ? q0 : (q1 > a.n_q ? a.n_q : q1);
      n = (int)(q1 - q0);
      kvr = (int64_t)((len + kPfRows - 1) / kPfRows) * kPfRows;
      qb = (n + kPfQ - 1) / kPfQ;
    }
    s_kv[tid] = kvr;
    s_qb[tid] = qb;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {                // inclusive scans
      const int64_t xk = tid >= d ? s_kv[tid - d] : 0;
      const int32_t xq = tid >= d ? s_qb[tid - d] : 0;
      __syncthreads();
      s_kv[tid] += xk;
      s_qb[tid] += xq;
      __syncthreads();
    }
    if (b < a.B) {
      int64_t r0 = carry_kv + s_kv[tid] - kvr;
      // a sequence whose rows would pass the K/V buffers is not served
      // (its queries get o = 0, lse = -inf): the caller's row bound was short
      if (r0 + kvr > a.kv_rows) len = 0;
      a.kv_row0[b] = r0;
      a.qb_start[b] = carry_qb + s_qb[tid] - qb;
      a.lenc[b] = len;
      a.nq[b] = n;
    }
    carry_kv += s_kv[255];
    carry_qb += s_qb[255];
    __syncthreads();
  }
  if (tid == 0) {
    a.kv_row0[a.B] = carry_kv;
    a.qb_start[a.B] = carry_qb;
  }
}

// Largest b in [0, B) with arr[b] <= x (arr non-decreasing, arr[0] <= x),
// through scalar loads.
template <typename T>
__device__ __forceinline__ int search_seq(const T* arr, int B, int64_t x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)ld_const(arr, mid) <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ kv
// One workgroup per (128 packed rows = blockIdx.x, head h = blockIdx.y): the
// row tiles of one head run next to each other and share its weights in L2.
// D^T = W X^T with A = the weight rows (output dims, 16 per block) and B =
// the latent rows (16 per block), so a lane ends with four consecutive
// output dims of one row (one 8-byte store). Wave w computes output dims
// 64w .. 64w + 63 of [K (0..127) | V (128..255)] for all 128 rows. The
// latent is contracted in 8 chunks of 64, each staged in LDS (latent rows,
// W_UK rows, W_UV rows) from registers loaded one chunk ahead.
template <int CT>
__global__ void __launch_bounds__(256) mla_prefill_kv_kernel(PrefillArgs a) {
  constexpr int KC = 64;
  constexpr int XP = KC * 2 + 16;                      // LDS pitch of a latent row chunk (bf16)
  constexpr int WKP = KC * 2 + 16;                     // W_UK row chunk
  constexpr int WVP = 128 * 2 + 16;                    // W_UV row (one latent dim)
  constexpr int X_BYTES = kPfRows * XP;
  constexpr int WK_BYTES = 128 * WKP;
  constexpr int WV_BYTES = KC * WVP;
  __shared__ __attribute__((aligned(16))) char lds[X_BYTES + WK_BYTES + WV_BYTES];
  __shared__ float s_scale[kPfRows];
  char* xs = lds;
  char* wk = lds + X_BYTES;
  char* wv = wk + WK_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int h = blockIdx.y;
  const int H = a.H;
  const int64_t r0 = (int64_t)blockIdx.x * kPfRows;
  if (r0 >= ld_const(a.kv_row0, a.B)) return;
  const int b = search_seq(a.kv_row0, a.B, r0);
  const int L = ld_const(a.lenc, b);
  const int t0 = (int)(r0 - ld_const(a.kv_row0, b));
  // cache row of position t0 + r: contiguous, seq_start[b] + t0 + r; paged,
  // through the block table (an entry outside the pool reads page 0 of it,
  // as the decode kernels do: a wrong page, never outside the pool)
  const bool paged = a.block_table != nullptr;
  const int64_t crow0 = paged ? 0 : ld_const(a.seq_start, b) + t0;
  auto crow = [&](int r) -> int64_t {
    if (!paged) return crow0 + r;
    const int t = t0 + r;
    const int j = t / a.page_tokens;
    const int32_t pg = a.block_table[(int64_t)b * a.max_pages + j];
    return (int64_t)((uint32_t)pg < a.page_limit ? pg : 0) * a.page_tokens + (t - j * a.page_tokens);
  };
  constexpr int RB = (CT == kFP8) ? kDrow : (CT == kFP6) ? 464 : kDrow * 2;   // bytes of a cache row
  const char* rows = (const char*)a.rows;

  if constexpr (CT == kFP8) {
    if (tid < kPfRows) s_scale[tid] = (t0 + tid < L) ? a.row_scale[crow(tid)] : 0.f;
  }

  // ---- global loads of one chunk into registers ----
  constexpr int NX = (CT == kFP8) ? 2 : 4;             // 16-byte pieces of latent per thread
  struct Chunk {
    u32x4 x[NX];
    uint2 c6[3];                                       // fp6: one 32-element block's codes
    uint32_t e6;                                       //      and its scale code
    u32x4 k[4];
    u32x4 v[4];
  };
  auto load = [&](int k0, Chunk& c) {
    if constexpr (CT == kFP6) {                        // thread: row tid/2, block k0/32 + tid%2
      const int r = tid >> 1;
      const int j = (k0 >> 5) + (tid & 1);
      c.c6[0] = c.c6[1] = c.c6[2] = uint2{0u, 0u};
      c.e6 = 127u;
      if (t0 + r < L) {
        const char* rp = rows + crow(r) * RB;
#pragma unroll
        for (int m = 0; m < 3; ++m) c.c6[m] = *(const uint2*)(rp + 24 * j + 8 * m);
        c.e6 = *(const unsigned char*)(rp + 432 + j);
      }
    }
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      if constexpr (CT == kFP6) break;
      const int i = tid + 256 * j;
      const int r = (CT == kFP8) ? (i >> 2) : (i >> 3);
      const int p = (CT == kFP8) ? (i & 3) : (i & 7);
      c.x[j] = u32x4{0u, 0u, 0u, 0u};
      if (t0 + r < L)
        c.x[j] = *(const u32x4*)(rows + crow(r) * RB + (CT == kFP8 ? k0 : 2 * k0) + 16 * p);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int n = i >> 3, p = i & 7;                 // W_UK[h][n][k0 + 8p ..]
      c.k[j] = *(const u32x4*)((const char*)a.w_uk + (((int64_t)h * 128 + n) * kDc + k0) * 2 + 16 * p);
      const int kk = i >> 4, q = i & 15;               // W_UV[h][k0 + kk][8q ..]
      c.v[j] = *(const u32x4*)((const char*)a.w_uv + (((int64_t)h * kDc + k0 + kk) * 128) * 2 + 16 * q);
    }
  };
  auto store = [&](const Chunk& c) {
    if constexpr (CT == kFP6) {                        // 32 codes -> 32 exact bf16 values
      const int r = tid >> 1;
      const fp6x32_words codes = {(int)c.c6[0].x, (int)c.c6[0].y, (int)c.c6[1].x,
                                  (int)c.c6[1].y, (int)c.c6[2].x, (int)c.c6[2].y};
      const bf16x32 v = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(
          codes, __builtin_amdgcn_ldexpf(1.f, (int)c.e6 - 127));
      const u32x4* vv = (const u32x4*)&v;
      char* dst = xs + r * XP + 64 * (tid & 1);
#pragma unroll
      for (int m = 0; m < 4; ++m) *(u32x4*)(dst + 16 * m) = vv[m];
    }
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      if constexpr (CT == kFP6) break;
      const int i = tid + 256 * j;
      if constexpr (CT == kFP8) {                      // 16 codes -> 16 exact bf16 values
        const int r = i >> 2, p = i & 3;
        const u32x4 u = c.x[j];
        const uint2 e0 = fp8x4_to_bf16x4(u[0]), e1 = fp8x4_to_bf16x4(u[1]);
        const uint2 e2 = fp8x4_to_bf16x4(u[2]), e3 = fp8x4_to_bf16x4(u[3]);
        *(u32x4*)(xs + r * XP + 32 * p) = u32x4{e0.x, e0.y, e1.x, e1.y};
        *(u32x4*)(xs + r * XP + 32 * p + 16) = u32x4{e2.x, e2.y, e3.x, e3.y};
      } else {
        const int r = i >> 3, p = i & 7;
        *(u32x4*)(xs + r * XP + 16 * p) = c.x[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      *(u32x4*)(wk + (i >> 3) * WKP + 16 * (i & 7)) = c.k[j];
      *(u32x4*)(wv + (i >> 4) * WVP + 16 * (i & 15)) = c.v[j];
    }
  };

  f32x4 acc[4][8];                                     // [output block][row block]
#pragma unroll
  for (int ob = 0; ob < 4; ++ob)
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) acc[ob][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool is_k = wave < 2;
  const int nbase = 64 * (wave & 1);                   // first output dim of the wave in K or V
  Chunk cur;
  load(0, cur);
  for (int k0 = 0; k0 < kDc; k0 += KC) {
    __syncthreads();                                   // previous chunk consumed
    store(cur);
    __syncthreads();
    if (k0 + KC < kDc) load(k0 + KC, cur);             // next chunk in flight during the MFMAs
#pragma unroll
    for (int kk = 0; kk < KC; kk += 32) {
      bf16x8 w8[4];
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) {
        if (is_k) {                                    // lane (n, g): W_UK[h][n][kk + 8g ..]
          w8[ob] = *(const bf16x8*)(wk + (nbase + 16 * ob + l16) * WKP + (kk + 8 * g) * 2);
        } else {                                       // lane (n, g): W_UV[h][kk + 8g + 0..7][n]
          const int rs = kk + 8 * g + (l16 >> 2);
          const int cb = (nbase + 16 * ob + 4 * (l16 & 3)) * 2;
          const s16x4 lo = lds_read_tr16(wv, rs * WVP + cb);
          const s16x4 hi = lds_read_tr16(wv, (rs + 4) * WVP + cb);
          const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          w8[ob] = __builtin_bit_cast(bf16x8, a8);
        }
      }
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        const bf16x8 x8 = *(const bf16x8*)(xs + (16 * rb + l16) * XP + (kk + 8 * g) * 2);
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) acc[ob][rb] = mfma_bf16_k32(w8[ob], x8, acc[ob][rb]);
      }
    }
  }

  // ---- epilogue: lane holds D^T[dim 16 ob + 4g + r][row 16 rb + l16]; rows
  // past the sequence are written as zeros ----
  constexpr int KW = 128 + kDr;                        // K row width (elements)
  const int dst_w = is_k ? KW : 128;
  char* dst_base = (char*)(is_k ? a.k : a.v) + ((int64_t)h * a.kv_rows + r0) * dst_w * 2;
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    const int r = 16 * rb + l16;
    float sc = (t0 + r < L) ? 1.f : 0.f;
    if constexpr (CT == kFP8) sc = s_scale[r];        // 0 past the sequence
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      const f32x4 x = acc[ob][rb] * sc;
      uint2 u;
      u.x = pack_bf16x2(x[0], x[1]);
      u.y = pack_bf16x2(x[2], x[3]);
      *(uint2*)(dst_base + ((int64_t)r * dst_w + nbase + 16 * ob + 4 * g) * 2) = u;
    }
  }

  // ---- the RoPE key of the 128 rows after K[h]'s 128 dims (bf16; fp8 codes
  // times the row scale, rounded once) ----
  if constexpr (CT == kFP6) {                          // thread: row tid/2, block 16 + tid%2
    char* kpe = (char*)a.k + ((int64_t)h * a.kv_rows + r0) * KW * 2 + 128 * 2;
    const int r = tid >> 1;
    const int j = 16 + (tid & 1);
    u32x4 out[4] = {};
    if (t0 + r < L) {
      const char* rp = rows + crow(r) * RB;
      uint2 c[3];
#pragma unroll
      for (int m = 0; m < 3; ++m) c[m] = *(const uint2*)(rp + 24 * j + 8 * m);
      const unsigned e = *(const unsigned char*)(rp + 432 + j);
      const fp6x32_words codes = {(int)c[0].x, (int)c[0].y, (int)c[1].x, (int)c[1].y, (int)c[2].x, (int)c[2].y};
      const bf16x32 v = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(codes, __builtin_amdgcn_ldexpf(1.f, (int)e - 127));
      const u32x4* vv = (const u32x4*)&v;
#pragma unroll
      for (int m = 0; m < 4; ++m) out[m] = vv[m];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) *(u32x4*)(kpe + (r * KW + 32 * (tid & 1) + 8 * m) * 2) = out[m];
  } else {
    char* kpe = (char*)a.k + ((int64_t)h * a.kv_rows + r0) * KW * 2 + 128 * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;                     // 8-element piece i of the 128 x 64 block
      const int r = i >> 3, p = i & 7;
      u32x4 out = u32x4{0u, 0u, 0u, 0u};
      if (t0 + r < L) {
        if constexpr (CT == kFP8) {
          const uint2 c = *(const uint2*)(rows + crow(r) * RB + kDc + 8 * p);
          const float sc = s_scale[r];
          float f[8];
#pragma unroll
          for (int w2 = 0; w2 < 2; ++w2) {
            const uint32_t word = w2 ? c.y : c.x;
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
            const float v0 = lo[0], v1 = lo[1], v2 = hi[0], v3 = hi[1];
            f[4 * w2 + 0] = v0 * sc;
            f[4 * w2 + 1] = v1 * sc;
            f[4 * w2 + 2] = v2 * sc;
            f[4 * w2 + 3] = v3 * sc;
          }
          out = u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
        } else {
          out = *(const u32x4*)(rows + crow(r) * RB + kDc * 2 + 16 * p);
        }
      }
      *(u32x4*)(kpe + (r * KW + 8 * p) * 2) = out;
    }
  }
}

// ------------------------------------------------------------------ attention
// One workgroup per (head, block of 256 queries of one sequence). Work items
// are ordered by (head, sequence, query block, later blocks first) and dealt
// to the 8 XCDs in contiguous ranges, so the workgroups that read one
// (sequence, head)'s K/V run on one XCD close together and share its L2.
// LDS stages hold 64 K rows (128 + 64 dims, pitch 400 B: 16 rows of a
// 16-byte operand read start on distinct bank groups) and 64 V rows (pitch
// 272 B); stage slot s of a copy is K row s / 25, chunk s % 25 (chunks
// 0..15 from K[h], 16..23 from the RoPE key, 24 a repeat of 23) or V row
// s / 17, chunk s % 17 (16 a repeat of 15).
constexpr int kPfKP = 400;                             // K row pitch in LDS
constexpr int kPfVP = 272;                             // V row pitch in LDS
constexpr int kPfKSlots = kPfKP / 16;                  // 25
constexpr int kPfVSlots = kPfVP / 16;                  // 17
constexpr int kPfKCopies = kPfKV * kPfKSlots / 64;     // 25 one-kilobyte copies
constexpr int kPfVCopies = kPfKV * kPfVSlots / 64;     // 17
constexpr int kPfStage = (kPfKCopies + kPfVCopies) * 1024;
constexpr int kPfStages = 3;                           // LDS ring depth (129 KB)

__global__ void __launch_bounds__(512) mla_prefill_attn_kernel(PrefillArgs a) {
  static_assert(kPfKV * kPfKSlots % 64 == 0 && kPfKV * kPfVSlots % 64 == 0, "whole copies");
  constexpr int NS = kPfStages;
  __shared__ __attribute__((aligned(1024))) char smem[NS * kPfStage];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int H = a.H;
  const int B = a.B;

  // ---- work item ----
  const int per = gridDim.x / 8;
  const int64_t k = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  const int QB = ld_const(a.qb_start, B);
  if (QB == 0 || k >= (int64_t)H * QB) return;
  const int h = (int)(k / QB);
  const int qbg = (int)(k - (int64_t)h * QB);
  const int b = search_seq(a.qb_start, B, qbg);
  const int qb0 = ld_const(a.qb_start, b);
  const int nqb = ld_const(a.qb_start, b + 1) - qb0;
  const int j = nqb - 1 - (qbg - qb0);                 // later blocks (longer rows) first
  const int L = ld_const(a.lenc, b);
  const int n = ld_const(a.nq, b);
  int64_t qrow0 = ld_const(a.q_start, b);
  qrow0 = qrow0 < 0 ? 0 : (qrow0 > a.n_q ? a.n_q : qrow0);
  const int64_t kv0_row = ld_const(a.kv_row0, b);
  // positions: query i of the sequence sits at L - n + i
  const int i_blk = j * kPfQ;                          // first query of the block
  const int i_last = (i_blk + kPfQ < n ? i_blk + kPfQ : n) - 1;
  const int p_last = L - n + i_last;                   // the block's last position
  const int nblk = p_last >= 0 ? (p_last + kPfKV) / kPfKV : 0;
  const int i_w = i_blk + 32 * wave;                   // this wave's first query
  const int p_w0 = L - n + i_w;                        // its first position

  // ---- queries: B operand of the score MFMA, lane (query l16, k-run 8g) ----
  bf16x8 q[2][6];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int i = i_w + 16 * qb + l16;
    i = i < n ? i : n - 1;                             // rows past the sequence's queries: any valid one
    const int64_t qr = qrow0 + i;
    const __bf16* qn = (const __bf16*)a.q_nope + (qr * H + h) * kDnope;
    const __bf16* qp = (const __bf16*)a.q_pe + (qr * H + h) * kDr;
#pragma unroll
    for (int kk = 0; kk < 6; ++kk)
      q[qb][kk] = kk < 4 ? *(const bf16x8*)(qn + 32 * kk + 8 * g) : *(const bf16x8*)(qp + 32 * (kk - 4) + 8 * g);
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) asm volatile("" : "+v"(q[qb][kk]));

  // ---- copies of K/V block `blk` into stage `st`: copy c of the 42 goes to
  // wave c % 8; a lane's byte offset in the block's K rows (384 B) or V rows
  // (256 B) is fixed per copy, so it is computed once ----
  constexpr int kCopies = kPfKCopies + kPfVCopies;
  constexpr int kMaxPer = (kCopies + 7) / 8;
  uint32_t coff[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = wave + 8 * i;
    const int ln = lane;
    if (c < kPfKCopies) {
      const int sl = 64 * c + ln, r = sl / kPfKSlots;
      const int ch = sl - r * kPfKSlots;
      coff[i] = (uint32_t)(r * 384 + 16 * (ch < 23 ? ch : 23));
    } else {
      const int sl = 64 * (c - kPfKCopies) + ln, r = sl / kPfVSlots;
      const int ch = sl - r * kPfVSlots;
      coff[i] = (uint32_t)(r * 256 + 16 * (ch < 15 ? ch : 15));
    }
  }
  const char* kbase = (const char*)a.k + (int64_t)h * a.kv_rows * 384;
  const char* vbase = (const char*)a.v + (int64_t)h * a.kv_rows * 256;
  auto issue = [&](int blk, int st) {
    const int64_t row0 = kv0_row + (int64_t)blk * kPfKV;
    const auto rk = make_rsrc(kbase + row0 * 384, kPfKV * 384);
    const auto rv = make_rsrc(vbase + row0 * 256, kPfKV * 256);
    char* stage = smem + st * kPfStage;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int c = wave + 8 * i;
      if (c < kPfKCopies) buffer_copy16(rk, coff[i], stage + c * 1024);
      else if (c < kCopies) buffer_copy16(rv, coff[i], stage + c * 1024);
    }
  };

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 o[8][2];                                       // O^T: dims 16 db + 4g + r, query l16 of block qb
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db][0] = o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.softmax_scale * kLog2e;
  const uint32_t k_lane = (uint32_t)(l16 * kPfKP + 16 * g);
  const uint32_t v_lane = (uint32_t)((4 * g + (l16 >> 2)) * kPfVP + 8 * (l16 & 3));

  // this wave's copies per block: copies wave, wave + 8, ... of the 42
  const bool six = wave < kCopies % 8;                 // (kCopies + 7) / 8 copies, else one fewer
  for (int i = 0; i < NS - 1 && i < nblk; ++i) issue(i, i);
  for (int blk = 0; blk < nblk; ++blk) {
    // block blk's copies have landed: the ones of blocks blk+1 .. blk+NS-2
    // already issued may stay in flight
    const int younger = (nblk - 1 - blk < NS - 2) ? nblk - 1 - blk : NS - 2;
    if (six) wait_tiles<(kCopies + 7) / 8, NS - 2>(younger);
    else wait_tiles<kCopies / 8, NS - 2>(younger);
    barrier_lds();                                     // block blk visible; stage (blk - 1) % NS free
    if (blk + NS - 1 < nblk) issue(blk + NS - 1, (blk + NS - 1) % NS);
    const int kv0 = blk * kPfKV;
    if (kv0 > p_w0 + 31) continue;                     // every query of this wave is earlier
    const char* stage = smem + (blk % NS) * kPfStage;
    const uint32_t ks = (uint32_t)(size_t)stage + k_lane;
    const uint32_t vs = (uint32_t)(size_t)(stage + kPfKCopies * 1024) + v_lane;

    // scores S^T[row 16 kb + 4g + r][query 16 qb + l16]
    f32x4 acc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb][0] = acc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // two k-steps (eight 16-byte reads) per wait
#pragma unroll
    for (int k2 = 0; k2 < 3; ++k2) {
      u32x4 r8[8];
      constexpr int R = 16 * kPfKP;
      if (k2 == 0) lds_read_b128_x8<0, R, 2 * R, 3 * R, 64, R + 64, 2 * R + 64, 3 * R + 64>(ks, r8);
      if (k2 == 1) lds_read_b128_x8<128, R + 128, 2 * R + 128, 3 * R + 128, 192, R + 192, 2 * R + 192, 3 * R + 192>(ks, r8);
      if (k2 == 2) lds_read_b128_x8<256, R + 256, 2 * R + 256, 3 * R + 256, 320, R + 320, 2 * R + 320, 3 * R + 320>(ks, r8);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 a8 = __builtin_bit_cast(bf16x8, r8[4 * h2 + kb]);
          acc[kb][0] = mfma_bf16_k32(a8, q[0][2 * k2 + h2], acc[kb][0]);
          acc[kb][1] = mfma_bf16_k32(a8, q[1][2 * k2 + h2], acc[kb][1]);
        }
    }

    // online softmax per query (log2 domain, lazy rescale as in decode)
    const bool diag = kv0 + kPfKV - 1 > p_w0;           // some row is past some query's position
    bf16x8 pb[2][2];                                   // [query block][k-step of 32 rows]
    float sc[2][16];
    bool grow = false;
    float tmax[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[qb][4 * kb + r] = acc[kb][qb][r];   // unscaled: the scale enters the exponent
    }
    if (diag) {                                        // (a uniform branch: only diagonal blocks mask)
      const int lim = p_w0 + l16 - kv0 - 4 * g;        // row 16 kb + r is visible to query 16 qb + l16
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)                   //   when 16 kb + r <= lim + 16 qb
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + r > lim + 16 * qb) sc[qb][4 * kb + r] = -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float t = sc[qb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) t = __builtin_fmaxf(t, sc[qb][i]);
      tmax[qb] = max_over_groups(t) * sl2;             // (sl2 > 0: the max commutes)
      grow = grow || (tmax[qb] > m_run[qb] + kSlack);
    }
    if (__any(grow)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m_new = __builtin_fmaxf(m_run[qb], tmax[qb]);
        float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        if (m_new == m_run[qb]) alpha = 1.f;           // (also when both are -inf)
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
        m_run[qb] = m_new;
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float pv[16];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][i], sl2, -m_use));
        psum += pv[i];
      }
      l_run[qb] += psum;
      pb[qb][0] = pack_bf16x8(pv);                     // rows 4g.. (block 0) and 16 + 4g.. (block 1)
      pb[qb][1] = pack_bf16x8(pv + 8);                 // rows 32 + 4g.. and 48 + 4g..
    }

    // values: O^T[dim][query] += V^T P^T over two k-steps of 32 rows, all
    // eight dim blocks' operands (sixteen transposing reads) per wait
#pragma unroll
    for (int kstep = 0; kstep < 2; ++kstep) {
      s16x4 rr[16];                                    // [2 db]: rows 0..15, [2 db + 1]: rows 16..31
      if (kstep == 0) lds_tr16_x16<0, 32, 16 * kPfVP>(vs, rr);
      else lds_tr16_x16<32 * kPfVP, 32, 16 * kPfVP>(vs, rr);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const s16x4 lo = rr[2 * db], hi = rr[2 * db + 1];
        const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 av = __builtin_bit_cast(bf16x8, a8);
        o[db][0] = mfma_bf16_k32(av, pb[0][kstep], o[db][0]);
        o[db][1] = mfma_bf16_k32(av, pb[1][kstep], o[db][1]);
      }
    }
  }

  // ---- outputs of the wave's valid queries ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lsum = sum_over_groups(l_run[qb]);
    const int i = i_w + 16 * qb + l16;
    if (i >= n || i < 0) continue;
    const int64_t qr = qrow0 + i;
    const float inv = inv_or_zero(lsum);
    char* dst = (char*)a.out + ((qr * H + h) * kDv + 4 * g) * 2;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 x = o[db][qb] * inv;
      uint2 u;
      u.x = pack_bf16x2(x[0], x[1]);
      u.y = pack_bf16x2(x[2], x[3]);
      *(uint2*)(dst + 32 * db) = u;
    }
    if (a.lse && g == 0)
      a.lse[qr * H + h] = lsum > 0.f ? (m_run[qb] + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------ launch
hipError_t launch_prefill(int ct, const PrefillArgs& a, hipStream_t s) {
  if (a.B == 0 || a.n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_prefill_plan_kernel, dim3(1), dim3(256), 0, s, a);
  const int64_t tiles = a.kv_rows / kPfRows;
  if (ct == kFP8)
    hipLaunchKernelGGL(mla_prefill_kv_kernel<kFP8>, dim3((unsigned)tiles, a.H), dim3(256), 0, s, a);
  else if (ct == kFP6)
    hipLaunchKernelGGL(mla_prefill_kv_kernel<kFP6>, dim3((unsigned)tiles, a.H), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(mla_prefill_kv_kernel<kBF16>, dim3((unsigned)tiles, a.H), dim3(256), 0, s, a);
  const int64_t items = (int64_t)a.H * ((a.n_q + kPfQ - 1) / kPfQ + a.B);
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL(mla_prefill_attn_kernel, dim3((unsigned)grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
