// Matrix-core rate probe for gfx950: each wave runs ITER rounds of eight
// independent MFMAs of one kind (no memory traffic in the loop); the time of
// the whole launch over 1024 SIMDs gives the time per MFMA per SIMD.
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//          mfma_rate.hip -o mfma_rate
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); exit(1); } } while (0)
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int ITER = 2048;

template <int KIND>
__global__ void __launch_bounds__(256) probe(float* out, long long* cyc, int seed) {
  v4f c[8];
  for (int i = 0; i < 8; ++i) c[i] = v4f{0, 0, 0, 0};
  v8i a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (threadIdx.x * 7 + i + seed) & 0x3f3f3f3f; b[i] = (threadIdx.x * 3 + i * 5 + seed) & 0x3f3f3f3f; }
  long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < ITER; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0) {
        bf16x8 x = __builtin_bit_cast(bf16x8, v4f{__builtin_bit_cast(float, a[0]), __builtin_bit_cast(float, a[1]), __builtin_bit_cast(float, a[2]), __builtin_bit_cast(float, a[3])});
        bf16x8 y = __builtin_bit_cast(bf16x8, v4f{__builtin_bit_cast(float, b[0]), __builtin_bit_cast(float, b[1]), __builtin_bit_cast(float, b[2]), __builtin_bit_cast(float, b[3])});
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c[i], 0, 0, 0);
      } else if constexpr (KIND == 1) {
        long x = ((long)a[1] << 32) | (unsigned)a[0], y = ((long)b[1] << 32) | (unsigned)b[0];
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(x, y, c[i], 0, 0, 0);
      } else if constexpr (KIND == 2) {
        c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 0, 0, 0, 127, 0, 127);
      } else if constexpr (KIND == 3) {   // fp4 x fp4 (formats 4,4)
        c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 4, 4, 0, 127, 0, 127);
      } else if constexpr (KIND == 4) {   // fp6 e2m3 A x fp8 B
        c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 2, 0, 0, 127, 0, 127);
      }
    }
  }
  long long t1 = __builtin_readcyclecounter();
  float s = 0;
  for (int i = 0; i < 8; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * 4 + threadIdx.x / 64] = t1 - t0;
}

template <int KIND>
void run(const char* name, int blocks, float* out, long long* cyc) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  probe<KIND><<<blocks, 256>>>(out, cyc, 1);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0));
  probe<KIND><<<blocks, 256>>>(out, cyc, 2);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  long long h[4];
  CHECK(hipMemcpy(h, cyc, sizeof(h), hipMemcpyDeviceToHost));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  double n = (double)blocks * 4 * ITER * 8;   // MFMAs
  printf("%-22s blocks %5d: %.3f ms, %.2f ns per MFMA per SIMD, wave 0: %.1f timer ticks per MFMA\n",
         name, blocks, ms, ms * 1e6 / (n / 1024.0), (double)h[0] / (ITER * 8));
}

int main() {
  float* out; long long* cyc;
  CHECK(hipMalloc(&out, 4096 * 256 * sizeof(float)));
  CHECK(hipMalloc(&cyc, 4096 * 4 * sizeof(long long)));
  for (int blocks : {256, 512, 1024}) {
    run<0>("bf16 16x16x32", blocks, out, cyc);
    run<1>("fp8 16x16x32 (legacy)", blocks, out, cyc);
    run<2>("f8f6f4 16x16x128 fp8", blocks, out, cyc);
    run<3>("f8f6f4 16x16x128 fp4", blocks, out, cyc);
    run<4>("f8f6f4 16x16x128 fp6a", blocks, out, cyc);
  }
  return 0;
}
