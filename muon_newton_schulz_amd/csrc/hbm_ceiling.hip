// Sustained HBM stream rates of this GPU: a plain read + write copy, a
// read-only pass and a write-only pass over buffers far larger than the
// 256 MiB last-level cache, each swept over grid sizes and loads in flight
// per thread.  The best copy rate is the practical ceiling of the
// optimizer's elementwise kernels, which read and write in about equal
// amounts (momentum 6 + 6 bytes, apply 4 + 2, AdamW 14 + 14 per parameter).
//
// Prints one JSON line:
//   {"copy_gbps": .., "read_gbps": .., "write_gbps": .., "bytes": ..,
//    "copy_best": "U<loads>/g<grid>", ...}
// Bytes moved: copy 2 x buffer (read + write), read and write 1 x buffer.
#include <hip/hip_runtime.h>

#include <cstdio>

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Thread t of block b handles vectors b*256*U + t + 256*u (u < U) of each
// grid-stride round; n is a multiple of 256*U, so every access is in range.
template <int U>
__global__ __launch_bounds__(256) void k_copy(const f32x4_t* __restrict__ a,
                                              f32x4_t* __restrict__ b, long n) {
  const long stride = static_cast<long>(gridDim.x) * 256 * U;
  for (long i = static_cast<long>(blockIdx.x) * 256 * U + threadIdx.x; i < n; i += stride) {
    f32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = a[i + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) b[i + 256 * u] = v[u];
  }
}

template <int U>
__global__ __launch_bounds__(256) void k_read(const f32x4_t* __restrict__ a,
                                              float* __restrict__ sink, long n) {
  const long stride = static_cast<long>(gridDim.x) * 256 * U;
  float s = 0.0f;
  for (long i = static_cast<long>(blockIdx.x) * 256 * U + threadIdx.x; i < n; i += stride) {
    f32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = a[i + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u][0] + v[u][1] + v[u][2] + v[u][3];
  }
  // the buffers hold zeros: the store never happens, but the sum is live
  if (s == 1.0f) sink[0] = s;
}

__global__ __launch_bounds__(256) void k_write(f32x4_t* __restrict__ b, long n) {
  const long stride = static_cast<long>(gridDim.x) * 256;
  const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
  for (long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) b[i] = z;
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
  const long bytes = 2L << 30;        // 2 GiB per buffer (8x the last-level cache)
  const long n = bytes / 16;          // float4 vectors: a multiple of 256 * 8
  f32x4_t *a = nullptr, *b = nullptr;
  float* sink = nullptr;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMalloc(&sink, 64));
  CHECK(hipMemset(a, 0, bytes));
  CHECK(hipMemset(b, 0, bytes));
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));

  // best rate over 10 back-to-back launches (after one untimed launch)
  auto rate = [&](double moved, auto launch) -> double {
    launch();
    if (hipDeviceSynchronize() != hipSuccess) return -1.0;
    if (hipEventRecord(e0) != hipSuccess) return -1.0;
    for (int r = 0; r < 10; ++r) launch();
    if (hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return -1.0;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.0f) return -1.0;
    return moved * 10.0 / (ms * 1e-3) / 1e9;
  };

  double best_copy = 0.0, best_read = 0.0, best_write = 0.0;
  int copy_u = 0, copy_g = 0, read_u = 0, read_g = 0, write_g = 0;
  const int grids[] = {1024, 2048, 4096, 8192, 16384};
  for (int g : grids) {
    const double c1 = rate(2.0 * bytes, [&] { hipLaunchKernelGGL(k_copy<1>, dim3(g), dim3(256), 0, 0, a, b, n); });
    const double c2 = rate(2.0 * bytes, [&] { hipLaunchKernelGGL(k_copy<2>, dim3(g), dim3(256), 0, 0, a, b, n); });
    const double c4 = rate(2.0 * bytes, [&] { hipLaunchKernelGGL(k_copy<4>, dim3(g), dim3(256), 0, 0, a, b, n); });
    const double c8 = rate(2.0 * bytes, [&] { hipLaunchKernelGGL(k_copy<8>, dim3(g), dim3(256), 0, 0, a, b, n); });
    const double r4 = rate(1.0 * bytes, [&] { hipLaunchKernelGGL(k_read<4>, dim3(g), dim3(256), 0, 0, a, sink, n); });
    const double r8 = rate(1.0 * bytes, [&] { hipLaunchKernelGGL(k_read<8>, dim3(g), dim3(256), 0, 0, a, sink, n); });
    const double w1 = rate(1.0 * bytes, [&] { hipLaunchKernelGGL(k_write, dim3(g), dim3(256), 0, 0, b, n); });
    CHECK(hipGetLastError());
    const double cs[] = {c1, c2, c4, c8};
    const int us[] = {1, 2, 4, 8};
    for (int k = 0; k < 4; ++k)
      if (cs[k] > best_copy) best_copy = cs[k], copy_u = us[k], copy_g = g;
    if (r4 > best_read) best_read = r4, read_u = 4, read_g = g;
    if (r8 > best_read) best_read = r8, read_u = 8, read_g = g;
    if (w1 > best_write) best_write = w1, write_g = g;
  }
  if (best_copy <= 0.0 || best_read <= 0.0 || best_write <= 0.0) {
    std::fprintf(stderr, "a timed launch failed\n");
    return 1;
  }
  std::printf("{\"copy_gbps\": %.1f, \"read_gbps\": %.1f, \"write_gbps\": %.1f, \"bytes\": %ld, "
              "\"copy_best\": \"U%d/g%d\", \"read_best\": \"U%d/g%d\", \"write_best\": \"U1/g%d\"}\n",
              best_copy, best_read, best_write, bytes, copy_u, copy_g, read_u, read_g, write_g);
  return 0;
}
