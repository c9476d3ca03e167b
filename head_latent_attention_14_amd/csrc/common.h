// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// microscaling FP6: 32 packed e2m3 codes (element i in bits 6i..6i+5) and
// the 32 bf16 values the scaled hardware conversion makes of them
typedef int fp6x32_words __attribute__((ext_vector_type(6)));
typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDrow = 576;
constexpr int kDnope = 128;
constexpr int kDv = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// MFMA wrappers. Lane layout (checked on gfx950): for the 16x16 shapes lane l
// supplies row (A) / column (B) l%16 and a run of K elements chosen by l/16;
// the 4 results of lane l are D[4*(l/16) + r][l%16], r = 0..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// e4m3fn x e4m3fn, K = 128 (v_mfma_scale_f32_16x16x128_f8f6f4 with both block
// scales 2^0): lane l supplies 32 codes of row / column l%16; A and B take the
// same K order, so any assignment of elements to (l/16, byte) that A and B
// share contracts over the same elements.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_fp8_k128(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// e4m3fn x e4m3fn, K = 32 (v_mfma_f32_16x16x32_fp8_fp8): 8 codes per lane.
__device__ __forceinline__ f32x4 mfma_fp8_k32(uint2 a, uint2 b, const f32x4& c) {
  const long la = (long)(((uint64_t)a.y << 32) | a.x);
  const long lb = (long)(((uint64_t)b.y << 32) | b.x);
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(la, lb, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 per pair)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  u32x4 u;
  u[0] = pack_bf16x2(v[0], v[1]);
  u[1] = pack_bf16x2(v[2], v[3]);
  u[2] = pack_bf16x2(v[4], v[5]);
  u[3] = pack_bf16x2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// four e4m3fn codes (one dword) -> four exact bf16 values (two dwords).
// Every e4m3fn value is exactly representable in bf16, so truncating the
// fp32 value's low half is exact. (Vector elements are copied to scalars
// before __builtin_bit_cast: applied to an element expression such as a[1]
// the builtin reads element 0.)
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t codes) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
  const float a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
  uint2 r;
  r.x = (__builtin_bit_cast(uint32_t, a0) >> 16) | (__builtin_bit_cast(uint32_t, a1) & 0xffff0000u);
  r.y = (__builtin_bit_cast(uint32_t, b0) >> 16) | (__builtin_bit_cast(uint32_t, b1) & 0xffff0000u);
  return r;
}

// fp32 -> e4m3fn code, round to nearest even, saturating at +-448
// (the hardware conversion rounds to nearest even but does not saturate).
__device__ __forceinline__ uint32_t f32x4_to_fp8x4_sat(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.f), 448.f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.f), 448.f);
  c = __builtin_fminf(__builtin_fmaxf(c, -448.f), 448.f);
  d = __builtin_fminf(__builtin_fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// fp32 -> e4m3fn codes, round to nearest even, for values known to lie within
// +-448 (no clamp).
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// cross-lane
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  int lane = __lane_id();
  int src = lane ^ mask;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}
// Reductions over the four lanes l, l^16, l^32, l^48 that hold one MFMA
// column. v_permlane32_swap / v_permlane16_swap (gfx950) hand each lane the
// pair {x[l], x[l^32]} and {x[l], x[l^16]} (checked on gfx950), so each step
// is VALU work with no LDS round trip.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  const unsigned a0 = a[0], a1 = a[1];
  v = __builtin_fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return __builtin_fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  const unsigned a0 = a[0], a1 = a[1];
  v = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

// Eight transposing LDS reads (ds_read_b64_tr_b16, gfx950) at one per-lane
// address plus compile-time offsets, completed inside the same asm block:
// the compiler never sees a load in flight. (Through the builtin the
// compiler would wait for every asynchronous global->LDS copy first.)
// Within each group of 16 lanes, element q of lane j comes from the 16-bit
// value at addr(lane 4q + j/4) + 2*(j%4).
template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_tr16_x8(uint32_t addr, s16x4& r0, s16x4& r1, s16x4& r2,
                                            s16x4& r3, s16x4& r4, s16x4& r5, s16x4& r6,
                                            s16x4& r7) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%9\n"
      "ds_read_b64_tr_b16 %1, %8 offset:%10\n"
      "ds_read_b64_tr_b16 %2, %8 offset:%11\n"
      "ds_read_b64_tr_b16 %3, %8 offset:%12\n"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n"
      "ds_read_b64_tr_b16 %5, %8 offset:%14\n"
      "ds_read_b64_tr_b16 %6, %8 offset:%15\n"
      "ds_read_b64_tr_b16 %7, %8 offset:%16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3), "i"(O4), "i"(O5), "i"(O6), "i"(O7)
      : "memory");
}

// Four transposing 8-bit LDS reads (ds_read_b64_tr_b8, gfx950), completed
// inside the asm block like lds_tr16_x8. Within each group of 16 lanes,
// byte q of lane j is the byte at addr(lane 2q + j/8) + j%8 (checked on
// gfx950 with every lane pointing at its own 64-byte row).
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_tr8_x4(uint32_t addr, uint2& r0, uint2& r1, uint2& r2, uint2& r3) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %4 offset:%5\n"
      "ds_read_b64_tr_b8 %1, %4 offset:%6\n"
      "ds_read_b64_tr_b8 %2, %4 offset:%7\n"
      "ds_read_b64_tr_b8 %3, %4 offset:%8\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3)
      : "memory");
}

// 16- and 8-byte LDS reads at compile-time offsets from one per-lane
// address, completed inside the asm block. For reads the compiler must not see: a
// visible LDS read after asynchronous global->LDS copies can make it wait for
// every copy in flight.
template <int O0, int O1>
__device__ __forceinline__ void lds_read_b128_x2(uint32_t addr, u32x4& r0, u32x4& r1) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%3\n"
      "ds_read_b128 %1, %2 offset:%4\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(addr), "i"(O0), "i"(O1)
      : "memory");
}
template <int O0, int O1>
__device__ __forceinline__ void lds_read_b64_x2(uint32_t addr, uint2& r0, uint2& r1) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x2 a, b;
  asm volatile(
      "ds_read_b64 %0, %2 offset:%3\n"
      "ds_read_b64 %1, %2 offset:%4\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b)
      : "v"(addr), "i"(O0), "i"(O1)
      : "memory");
  r0 = uint2{a[0], a[1]};
  r1 = uint2{b[0], b[1]};
}
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read_b128_x4(uint32_t addr, u32x4& r0, u32x4& r1, u32x4& r2,
                                                 u32x4& r3) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n"
      "ds_read_b128 %1, %4 offset:%6\n"
      "ds_read_b128 %2, %4 offset:%7\n"
      "ds_read_b128 %3, %4 offset:%8\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3)
      : "memory");
}

// Eight 16-byte LDS reads at compile-time offsets from one per-lane address,
// completed inside the asm block (as lds_read_b128_x4).
template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_read_b128_x8(uint32_t addr, u32x4* r) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%9\n"
      "ds_read_b128 %1, %8 offset:%10\n"
      "ds_read_b128 %2, %8 offset:%11\n"
      "ds_read_b128 %3, %8 offset:%12\n"
      "ds_read_b128 %4, %8 offset:%13\n"
      "ds_read_b128 %5, %8 offset:%14\n"
      "ds_read_b128 %6, %8 offset:%15\n"
      "ds_read_b128 %7, %8 offset:%16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3), "i"(O4), "i"(O5), "i"(O6), "i"(O7)
      : "memory");
}

// Sixteen transposing reads (ds_read_b64_tr_b16) at offsets O(i) = A + B*(i/2)
// + C*(i%2) from one per-lane address, completed inside the asm block: r[2j]
// at A + B*j, r[2j+1] at A + B*j + C.
template <int A, int B, int C>
__device__ __forceinline__ void lds_tr16_x16(uint32_t addr, s16x4* r) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%17\n"
      "ds_read_b64_tr_b16 %1, %16 offset:%18\n"
      "ds_read_b64_tr_b16 %2, %16 offset:%19\n"
      "ds_read_b64_tr_b16 %3, %16 offset:%20\n"
      "ds_read_b64_tr_b16 %4, %16 offset:%21\n"
      "ds_read_b64_tr_b16 %5, %16 offset:%22\n"
      "ds_read_b64_tr_b16 %6, %16 offset:%23\n"
      "ds_read_b64_tr_b16 %7, %16 offset:%24\n"
      "ds_read_b64_tr_b16 %8, %16 offset:%25\n"
      "ds_read_b64_tr_b16 %9, %16 offset:%26\n"
      "ds_read_b64_tr_b16 %10, %16 offset:%27\n"
      "ds_read_b64_tr_b16 %11, %16 offset:%28\n"
      "ds_read_b64_tr_b16 %12, %16 offset:%29\n"
      "ds_read_b64_tr_b16 %13, %16 offset:%30\n"
      "ds_read_b64_tr_b16 %14, %16 offset:%31\n"
      "ds_read_b64_tr_b16 %15, %16 offset:%32\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(addr), "i"(A), "i"(A + C), "i"(A + B), "i"(A + B + C), "i"(A + 2 * B),
        "i"(A + 2 * B + C), "i"(A + 3 * B), "i"(A + 3 * B + C), "i"(A + 4 * B),
        "i"(A + 4 * B + C), "i"(A + 5 * B), "i"(A + 5 * B + C), "i"(A + 6 * B),
        "i"(A + 6 * B + C), "i"(A + 7 * B), "i"(A + 7 * B + C)
      : "memory");
}

// Eight e4m3fn codes (bytes 0..7 of v) as eight bf16 values, in order; every
// e4m3fn value is exact in bf16 and the unit scale leaves it unchanged.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint2 v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  const __bf16 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1], c0 = c[0], c1 = c[1], d0 = d[0], d1 = d[1];
  return bf16x8{a0, a1, b0, b1, c0, c1, d0, d1};
}

// ---------------------------------------------------------------------------
// LDS access
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 lds_read_b128(const char* lds_base, uint32_t byte_off) {
  return *reinterpret_cast<const bf16x8*>(lds_base + byte_off);
}
// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, result element q of lane j is the 16-bit value at
// addr(lane 4q + j/4) + 2*(j%4): each quad of source lanes supplies a 4x4
// block that arrives transposed.
__device__ __forceinline__ s16x4 lds_read_tr16(const char* lds_base, uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_base + byte_off));
}

// Asynchronous 16-byte-per-lane copy global -> LDS. Lane i's 16 bytes land at
// lds_wave_base + 16*i; lds_wave_base must be wave-uniform.
__device__ __forceinline__ void async_copy16(const void* gsrc, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void async_copy4(const void* gsrc, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_wave_base, 4, 0, 0);
}

// The same copies through a buffer resource: the 64-bit base sits in scalar
// registers and each lane only supplies a 32-bit byte offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ void buffer_copy16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_copy4(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                             char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 4, voff, 0, 0, 0);
}

// Cache row of token `pos` of sequence `seq` in a paged cache:
// block_table[seq][pos / P] * P + pos % P. `valid` is false (and the row 0)
// when pos is past the table or the table's entry lies outside the page pool.
__device__ __forceinline__ int64_t paged_row(const int32_t* table, int max_pages, int P,
                                             int64_t total_pages, int seq, int pos, bool& valid) {
  const int j = pos / P;
  valid = pos >= 0 && j < max_pages;
  const int64_t page = valid ? (int64_t)table[(int64_t)seq * max_pages + j] : 0;
  valid = valid && page >= 0 && page < total_pages;
  return valid ? page * P + (pos - j * P) : 0;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}
// Wait until at most K*PER copies are outstanding, K = min(younger, KMAX),
// choosing the immediate at run time from a wave-uniform `younger`.
template <int PER, int KMAX>
__device__ __forceinline__ void wait_tiles(int younger) {
  if constexpr (KMAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (younger >= KMAX) wait_vmcnt<KMAX * PER>();
    else wait_tiles<PER, KMAX - 1>(younger);
  }
}
// The same with EXTRA more operations issued after the younger copies (loads
// and stores of a segment change) allowed to stay outstanding.
template <int PER, int KMAX, int EXTRA>
__device__ __forceinline__ void wait_tiles_extra(int younger) {
  if constexpr (KMAX <= 0) {
    wait_vmcnt<EXTRA>();
  } else {
    if (younger >= KMAX) wait_vmcnt<KMAX * PER + EXTRA>();
    else wait_tiles_extra<PER, KMAX - 1, EXTRA>(younger);
  }
}

// Workgroup barrier that does not wait for outstanding global loads: LDS
// operations of this wave complete first (lgkmcnt(0)), vmcnt is left alone
// so asynchronous global->LDS copies of later tiles stay in flight. The empty
// asm keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Read a value that is constant for the whole launch through the constant
// address space, so a wave-uniform index becomes a scalar load (lgkmcnt)
// instead of a vector load that would be counted with the async copies.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A copy of v the compiler cannot see through: values derived from it are
// recomputed where they are used instead of being hoisted out of a loop into
// registers that stay live across it.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(v & 0xffffffff));
  const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return ((int64_t)hi << 32) | (uint32_t)lo;
}

}  // namespace mla
