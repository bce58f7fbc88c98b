// Stand-alone measurement (not part of the library): what it costs to accumulate the query gradient dQ
// across key-stationary work items, the alternative to recomputing S and dP in a query-stationary pass.
//
// Layer: B = 4, H = 32, T = 4096, d = 64, per-head windows [512 x12, 2048 x4, 512 x12, 1024 x4] (heads in
// that order).  A key-stationary backward holds 128 keys of one head per workgroup; for every 32-query
// block its keys are seen by, the workgroup would add a 32 x 64 fp32 partial of dQ = dS K (its four
// waves' partials already summed in LDS).  This program issues exactly those additions, with nothing
// else, as device-scope fp32 atomics (mode 0) and, for reference, as plain stores of the same tiles
// (mode 1), and prints the time per launch.
//
// Build and run:  hipcc -O3 --offload-arch=gfx950 -munsafe-fp-atomics dq_atomics.hip -o dq_atomics
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                   \
  do {                                                                             \
    const hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                        \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

namespace {

constexpr int kKeys = 128;  // keys per work item
constexpr int kQB = 32;     // queries per block
constexpr int kD = 64;

// Grid (T / kKeys, B * H), 256 threads: thread t adds elements t, t + 256, ... of each 32 x 64 tile.
__global__ __launch_bounds__(256) void accumulate(float* dq, const int* win, int H, int T, int mode) {
  const int kt = blockIdx.x, bh = blockIdx.y;
  const int W = win[bh % H];
  const int k0 = kt * kKeys, k1 = k0 + kKeys - 1;
  const int qb0 = k0 / kQB, qb1 = min(T - 1, k1 + W - 1) / kQB;  // blocks holding a query that sees a key
  float* head = dq + static_cast<size_t>(bh) * T * kD;
  const float v = 1.0f + threadIdx.x * 1e-3f;
  for (int qb = qb0; qb <= qb1; ++qb) {
    float* tile = head + static_cast<size_t>(qb) * kQB * kD;
#pragma unroll
    for (int i = 0; i < kQB * kD / 256; ++i) {
      float* p = tile + i * 256 + threadIdx.x;
      if (mode == 0)
        atomicAdd(p, v);
      else
        *p = v;
    }
  }
}

}  // namespace

int main() {
  const int B = 4, H = 32, T = 4096;
  std::vector<int> w(H);
  for (int h = 0; h < H; ++h) w[h] = h < 12 ? 512 : h < 16 ? 2048 : h < 28 ? 512 : 1024;
  long tiles = 0;
  for (int bh = 0; bh < B * H; ++bh)
    for (int kt = 0; kt < T / kKeys; ++kt) {
      const int k0 = kt * kKeys, k1 = k0 + kKeys - 1;
      tiles += std::min(T - 1, k1 + w[bh % H] - 1) / kQB - k0 / kQB + 1;
    }
  const double bytes = static_cast<double>(tiles) * kQB * kD * 4;
  std::printf("32 x 64 tiles: %ld, fp32 additions: %.3g, tile bytes: %.3f GB\n", tiles, tiles * 2048.0, bytes / 1e9);

  int* dw;
  float* dq;
  const size_t n = static_cast<size_t>(B) * H * T * kD;
  CHECK(hipMalloc(&dw, H * sizeof(int)));
  CHECK(hipMemcpy(dw, w.data(), H * sizeof(int), hipMemcpyHostToDevice));
  CHECK(hipMalloc(&dq, n * sizeof(float)));
  CHECK(hipMemset(dq, 0, n * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const dim3 grid(T / kKeys, B * H);
  for (int mode = 0; mode < 2; ++mode) {
    for (int r = 0; r < 3; ++r) hipLaunchKernelGGL(accumulate, grid, dim3(256), 0, 0, dq, dw, H, T, mode);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    const int reps = 20;
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(accumulate, grid, dim3(256), 0, 0, dq, dw, H, T, mode);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double us = ms * 1e3 / reps;
    std::printf("%s: %.1f us per launch (%.2f TB/s of tile data)\n",
                mode == 0 ? "device-scope fp32 atomic add" : "plain stores of the same tiles", us,
                bytes / (us * 1e-6) / 1e12);
  }
  CHECK(hipFree(dq));
  CHECK(hipFree(dw));
  return 0;
}
