// Sustained dense bf16 MFMA rate of this GPU under its own power and clock
// management: every wave of one 256-thread workgroup per CU issues
// independent v_mfma_f32_32x32x16_bf16 back to back from registers, with no
// memory traffic.  This is the ceiling any bf16 GEMM kernel can reach here;
// the published peak assumes the maximum engine clock, which a chip busy
// with matrix work does not hold.
//
// Prints one JSON line: {"tflops": .., "mhz": .., "cycles_per_mfma": ..}.
// "mhz" is shader-clock cycles (s_memtime) per microsecond of wall time.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 1) void k_mfma_rate(const bf16x8_t* __restrict__ a,
                                                      const bf16x8_t* __restrict__ b,
                                                      float* __restrict__ out,
                                                      unsigned long long* __restrict__ cycles,
                                                      int iters) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  bf16x8_t x = a[i & 4095];
  const bf16x8_t y = b[i & 4095];
  f32x16_t acc[16];
  for (int k = 0; k < 16; ++k)
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.0f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[k], 0, 0, 0);
    x[0] = x[0] + static_cast<__bf16>(1.0f);  // operands change every round
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.0f;
  for (int k = 0; k < 16; ++k)
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  out[i] = s;
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

int main() {
  int n_cu = 0;
  CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, 0));
  const int blocks = 4 * n_cu, iters = 1000;
  bf16x8_t *a = nullptr, *b = nullptr;
  float* out = nullptr;
  unsigned long long* cyc = nullptr;
  CHECK(hipMalloc(&a, 4096 * sizeof(bf16x8_t)));
  CHECK(hipMalloc(&b, 4096 * sizeof(bf16x8_t)));
  CHECK(hipMalloc(&out, sizeof(float) * blocks * 256));
  CHECK(hipMalloc(&cyc, sizeof(unsigned long long) * blocks));
  // operands: bf16 values in [0.5, 2) with random signs and mantissas
  std::vector<unsigned short> h(4096 * 8);
  unsigned s = 12345u;
  auto fill = [&](bf16x8_t* d) -> hipError_t {
    for (auto& v : h) {
      s = s * 1664525u + 1013904223u;
      v = static_cast<unsigned short>(((s >> 8) & 0x8000u) | (0x3f00u + ((s >> 16) & 0xffu)));
    }
    return hipMemcpy(d, h.data(), h.size() * 2, hipMemcpyHostToDevice);
  };
  CHECK(fill(a));
  CHECK(fill(b));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  double tflops = 0.0, mhz = 0.0, cpm = 0.0;
  for (int rep = 0; rep < 6; ++rep) {  // the first rounds let the clock settle
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(k_mfma_rate, dim3(blocks), dim3(256), 0, 0, a, b, out, cyc, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::vector<unsigned long long> c(blocks);
    CHECK(hipMemcpy(c.data(), cyc, sizeof(unsigned long long) * blocks, hipMemcpyDeviceToHost));
    double avg = 0.0;
    for (auto v : c) avg += static_cast<double>(v);
    avg /= blocks;
    const double mfma_per_wave = 16.0 * iters;
    tflops = blocks * 4.0 * mfma_per_wave * 32768.0 / (ms * 1e-3) / 1e12;
    // each CU runs blocks / n_cu workgroups one after another
    mhz = avg * (static_cast<double>(blocks) / n_cu) / (ms * 1e3);
    cpm = avg / mfma_per_wave;
  }
  std::printf("{\"tflops\": %.1f, \"mhz\": %.0f, \"cycles_per_mfma\": %.2f, \"cus\": %d}\n", tflops,
              mhz, cpm, n_cu);
  return 0;
}
