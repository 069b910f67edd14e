// Calibration of the int8 matrix pipe: every SIMD issues independent
// v_mfma_i32_16x16x64_i8 (four accumulator chains per wave, no memory traffic
// but one store per lane at the end) for a fixed count, with one, two and four
// waves per SIMD.  Prints the throughput in int8 TOP/s and the cycles per
// instruction per SIMD at the nominal 2.4 GHz.  Run under a counter profile it
// also gives the busy cycles the MFMA counters charge per instruction, which
// is what the MFMA summaries of the linear kernels are read against.
//
//     mfma_peak [iterations per wave, default 20000]
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWorkgroups = 256;  // one per compute unit

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_mfma_peak(int* out, int iters) {
  const int t = threadIdx.x;
  const v4i a = {t, t + 1, t + 2, t + 3}, b = {3 * t, 5, 7, t};
  v4i c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, b, c3, 0, 0, 0);
  }
  out[blockIdx.x * WAVES * 64 + t] = c0[0] + c1[1] + c2[2] + c3[3];
}

template <int WAVES>
static bool run(int* out, int iters) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return false;
  hipLaunchKernelGGL(k_mfma_peak<WAVES>, dim3(kWorkgroups), dim3(WAVES * 64), 0, 0, out, 100);  // warm-up
  if (hipDeviceSynchronize() != hipSuccess) return false;
  (void)hipEventRecord(e0);
  hipLaunchKernelGGL(k_mfma_peak<WAVES>, dim3(kWorkgroups), dim3(WAVES * 64), 0, 0, out, iters);
  (void)hipEventRecord(e1);
  if (hipEventSynchronize(e1) != hipSuccess) return false;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  const double mfma = (double)kWorkgroups * WAVES * iters * 4.0;
  const double simds = kWorkgroups * 4.0;
  printf("waves per SIMD %d: %.3f ms, %.0f MFMA, %.1f TOP/s int8, %.2f cycles per MFMA per SIMD at 2.4 GHz\n",
         WAVES / 4, ms, mfma, mfma * 2.0 * 16 * 16 * 64 / (ms * 1e-3) / 1e12, ms * 1e-3 * 2.4e9 / (mfma / simds));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return true;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  if (iters < 1) return 2;
  int* out = nullptr;
  if (hipMalloc(&out, sizeof(int) * kWorkgroups * 16 * 64) != hipSuccess) return 1;
  const bool ok = run<4>(out, iters) && run<8>(out, iters) && run<16>(out, iters);
  (void)hipFree(out);
  return ok ? 0 : 1;
}
