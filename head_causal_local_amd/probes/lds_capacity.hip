// Stand-alone measurement (not part of the library): how many 256-thread workgroups one CU holds at
// once for a given static LDS size.  Each workgroup records its start and end time (s_memrealtime) and
// its CU (HW_ID, XCC_ID); the program prints, per LDS size, the histogram over CUs of the largest number
// of workgroups that were resident on one CU at the same time.  The kernels use few registers, so LDS
// is the only limit besides the wave slots.
//
// Build and run:  hipcc -O3 --offload-arch=gfx950 lds_capacity.hip -o lds_capacity
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
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

template <int BYTES>
__global__ __launch_bounds__(256) void resident(unsigned* out, int spin) {
  __shared__ char buf[BYTES];
  const unsigned t0 = static_cast<unsigned>(__builtin_amdgcn_s_memrealtime());
  buf[threadIdx.x * 4] = static_cast<char>(threadIdx.x);
  float x = threadIdx.x;
  for (int i = 0; i < spin; ++i) x = x * 1.0000001f + 0.5f;  // about 20 us of work
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned hw, xcc;
    __asm__ volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    __asm__ volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const unsigned t1 = static_cast<unsigned>(__builtin_amdgcn_s_memrealtime());
    unsigned* o = out + 4 * blockIdx.x;
    o[0] = t0;
    o[1] = t1;
    o[2] = hw;
    o[3] = xcc + (buf[(threadIdx.x * 7) % 64] == 127 && x == 0.f ? 1u : 0u);  // keeps buf and x live
  }
}

template <int BYTES>
void measure(unsigned* d, int nblk) {
  hipLaunchKernelGGL(resident<BYTES>, dim3(nblk), dim3(256), 0, 0, d, 20000);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  std::vector<unsigned> h(4 * static_cast<size_t>(nblk));
  CHECK(hipMemcpy(h.data(), d, h.size() * sizeof(unsigned), hipMemcpyDeviceToHost));
  std::map<unsigned, std::vector<std::pair<long, int>>> ev;  // per CU: (time, +1 start / -1 end)
  for (int b = 0; b < nblk; ++b) {
    const unsigned hw = h[4 * b + 2], xcc = h[4 * b + 3];
    const unsigned cu = xcc * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 8) & 15);
    ev[cu].push_back({static_cast<long>(h[4 * b]), 1});
    ev[cu].push_back({static_cast<long>(h[4 * b + 1]), -1});
  }
  std::map<int, int> hist;
  for (auto& kv : ev) {
    auto& v = kv.second;
    std::sort(v.begin(), v.end(), [](const auto& a, const auto& b) {
      return a.first != b.first ? a.first < b.first : a.second < b.second;
    });
    int cur = 0, mx = 0;
    for (const auto& e : v) mx = std::max(mx, cur += e.second);
    hist[mx]++;
  }
  std::printf("LDS %6d B per workgroup: %zu CUs; most workgroups resident at once on a CU (CUs):", BYTES,
              ev.size());
  for (const auto& kv : hist) std::printf(" %d (%d)", kv.first, kv.second);
  std::printf("\n");
}

}  // namespace

int main() {
  int ncu = 0;
  CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
  const int nblk = ncu * 12;
  unsigned* d;
  CHECK(hipMalloc(&d, 4 * static_cast<size_t>(nblk) * sizeof(unsigned)));
  measure<16384>(d, nblk);
  measure<24576>(d, nblk);
  measure<26624>(d, nblk);
  measure<30720>(d, nblk);
  measure<31744>(d, nblk);
  measure<32256>(d, nblk);
  measure<32768>(d, nblk);
  measure<40960>(d, nblk);
  measure<49152>(d, nblk);
  measure<53248>(d, nblk);
  measure<65536>(d, nblk);
  measure<81920>(d, nblk);
  CHECK(hipFree(d));
  return 0;
}
