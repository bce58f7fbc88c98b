/*
 * A plain C99 caller of libaah_attn.so: it includes include/aah_attn.h as C, links the library, and uses
 * nothing but the header's calls, plain pointers and (for the device checks) the HIP runtime's C API.
 *
 * Without arguments: argument checks only (no device needed) -- the ABI version, a NULL tensor refused
 * before any HIP call, an empty problem accepted with NULL tensors, status strings.
 * With --device: closed forms of the windowed softmax ("Asymmetric Attention Heads", section 5.8: key j is
 * visible to query i iff i - W < j <= i), bf16 and fp32, on a stream the program creates:
 *   - a window of 1 sees only its own key, whose weight is 1: O = V (bitwise in bf16, where the weight is
 *     rounded to bf16; within 1e-6 in fp32), LSE = scale q_i . k_i, and in the backward dV = dO (within the
 *     gradient bounds of the parity tests: 3e-2 of max |dO| in bf16, 1e-4 in fp32, since the backward
 *     recomputes the weight from the saved LSE);
 *   - with every V row equal to one vector, any window's weights sum to 1: O = that vector (bitwise in bf16,
 *     within 1e-5 in fp32).
 * Prints "ok" and exits 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "aah_attn.h"

#define CHECK(cond, ...)                   \
  do {                                     \
    if (!(cond)) {                         \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");               \
      exit(1);                             \
    }                                      \
  } while (0)

static int host_checks(void) {
  const int32_t w[2] = {1, 64};
  CHECK(aah_abi_version() == AAH_ABI_VERSION, "ABI version %d, header %d", aah_abi_version(), AAH_ABI_VERSION);
  /* A NULL tensor is refused before any HIP call. */
  aah_status st = aah_attn_fwd(NULL, NULL, NULL, w, NULL, 1, 2, 2, 64, 64, AAH_BF16, 0.125f, NULL, NULL, NULL, 0,
                               NULL);
  CHECK(st == AAH_ERR_INVALID_ARG, "NULL q gave %s", aah_status_string(st));
  CHECK(strlen(aah_last_error_detail()) > 0, "no error detail");
  /* An empty problem (B = 0) computes nothing and touches no tensor. */
  st = aah_attn_fwd(NULL, NULL, NULL, w, NULL, 0, 2, 2, 64, 64, AAH_BF16, 0.125f, NULL, NULL, NULL, 0, NULL);
  CHECK(st == AAH_OK, "empty forward gave %s", aah_status_string(st));
  CHECK(strcmp(aah_status_string(AAH_ERR_UNSUPPORTED), "AAH_ERR_UNSUPPORTED") == 0, "status string");
  CHECK(aah_attn_workspace_size(4, 32, 4096, 64, AAH_BF16, 1) == (size_t)2 * 4 * 32 * 4096 * 4, "workspace size");
  return 0;
}

#include <hip/hip_runtime_api.h>

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    CHECK(e_ == hipSuccess, "%s: %s", #call, hipGetErrorString(e_));        \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) / 9007199254740992.0;
}

static uint16_t to_bf16(float x) { /* round to nearest even (finite inputs) */
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}

enum { B = 2, H = 2, T = 300, D = 64 };
#define N ((size_t)B * H * T * D)
#define NR ((size_t)B * H * T)

/* Values of tensor index i as floats (after rounding to the dtype), written into dev-ready host memory. */
static void fill(void* host, float* vals, aah_dtype dt, int constant_rows_head) {
  for (size_t i = 0; i < N; ++i) {
    const size_t row = i / D, col = i % D;
    const int h = (int)(row / T % H);
    float x = (float)(4.0 * uniform() - 2.0);
    if (h == constant_rows_head) x = (float)(0.25 * ((int)col % 7) - 0.75); /* every row of this head equal */
    if (dt == AAH_BF16) {
      ((uint16_t*)host)[i] = to_bf16(x);
      vals[i] = from_bf16(((uint16_t*)host)[i]);
    } else {
      ((float*)host)[i] = x;
      vals[i] = x;
    }
  }
}

static float value_at(const void* host, aah_dtype dt, size_t i) {
  return dt == AAH_BF16 ? from_bf16(((const uint16_t*)host)[i]) : ((const float*)host)[i];
}

static void device_checks(aah_dtype dt) {
  const size_t es = dt == AAH_BF16 ? 2 : 4;
  const int32_t windows[H] = {1, 1000}; /* head 0: one key; head 1: wider than T (full causal) */
  const float scale = 0.125f;
  float* qv = malloc(N * 4);
  float* kv = malloc(N * 4);
  float* vv = malloc(N * 4);
  float* gv = malloc(N * 4);
  void* hq = malloc(N * es);
  void* hk = malloc(N * es);
  void* hv = malloc(N * es);
  void* hg = malloc(N * es);
  void* ho = malloc(N * es);
  void* hdv = malloc(N * es);
  float* hl = malloc(NR * 4);
  fill(hq, qv, dt, -1);
  fill(hk, kv, dt, -1);
  fill(hv, vv, dt, 1); /* head 1: constant V rows */
  fill(hg, gv, dt, -1);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void *q, *k, *v, *o, *g, *dq, *dk, *dv, *ws;
  float* lse;
  HIP_OK(hipMalloc(&q, N * es));
  HIP_OK(hipMalloc(&k, N * es));
  HIP_OK(hipMalloc(&v, N * es));
  HIP_OK(hipMalloc(&o, N * es));
  HIP_OK(hipMalloc(&g, N * es));
  HIP_OK(hipMalloc(&dq, N * es));
  HIP_OK(hipMalloc(&dk, N * es));
  HIP_OK(hipMalloc(&dv, N * es));
  HIP_OK(hipMalloc((void**)&lse, NR * 4));
  const size_t ws_bytes = aah_attn_workspace_size(B, H, T, D, dt, 1);
  CHECK(ws_bytes > 0, "backward workspace size");
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemcpy(q, hq, N * es, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, N * es, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, N * es, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(g, hg, N * es, hipMemcpyHostToDevice));

  aah_status st = aah_attn_fwd(q, k, v, windows, NULL, B, H, H, T, D, dt, scale, o, lse, NULL, 0,
                               (aah_stream_t)stream);
  CHECK(st == AAH_OK, "forward: %s (%s)", aah_status_string(st), aah_last_error_detail());
  st = aah_attn_bwd(q, k, v, o, g, lse, windows, NULL, B, H, H, T, D, dt, scale, dq, dk, dv, ws, ws_bytes,
                    (aah_stream_t)stream);
  CHECK(st == AAH_OK, "backward: %s (%s)", aah_status_string(st), aah_last_error_detail());
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(ho, o, N * es, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl, lse, NR * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hdv, dv, N * es, hipMemcpyDeviceToHost));

  for (size_t r = 0; r < NR; ++r) {
    const int h = (int)(r / T % H);
    const float* vrow = vv + r * D;
    if (h == 0) { /* window 1 */
      double s = 0.0;
      for (int c = 0; c < D; ++c) s += (double)qv[r * D + c] * kv[r * D + c];
      CHECK(fabs(hl[r] - scale * s) <= 1e-4 * (1.0 + fabs(scale * s)), "LSE row %zu: %g vs %g", r, hl[r],
            scale * s);
      if (dt == AAH_BF16)
        CHECK(memcmp((const char*)ho + r * D * es, (const char*)hv + r * D * es, D * es) == 0,
              "window 1: O row %zu differs from V", r);
      for (int c = 0; c < D; ++c) {
        const float o_err = fabsf(value_at(ho, dt, r * D + c) - vrow[c]);
        CHECK(o_err <= 1e-6f * (1.0f + fabsf(vrow[c])), "window 1: O[%zu][%d] off by %g", r, c, o_err);
        const float dv_err = fabsf(value_at(hdv, dt, r * D + c) - gv[r * D + c]);
        /* bound relative to max |dO|, which is below 2 here */
        CHECK(dv_err <= (dt == AAH_BF16 ? 3e-2f : 1e-4f) * 2.0f, "window 1: dV[%zu][%d] off by %g", r, c, dv_err);
      }
    } else { /* constant V rows: O = that row for every window */
      for (int c = 0; c < D; ++c) {
        const float got = value_at(ho, dt, r * D + c);
        const float tol = dt == AAH_BF16 ? 0.0f : 1e-5f;
        CHECK(fabsf(got - vrow[c]) <= tol, "constant V: O[%zu][%d] = %g, expected %g", r, c, got, vrow[c]);
      }
    }
  }
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(o));
  HIP_OK(hipFree(g));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(lse));
  HIP_OK(hipFree(ws));
  HIP_OK(hipStreamDestroy(stream));
  free(qv), free(kv), free(vv), free(gv), free(hq), free(hk), free(hv), free(hg), free(ho), free(hdv), free(hl);
}

int main(int argc, char** argv) {
  host_checks();
  if (argc > 1 && strcmp(argv[1], "--device") == 0) {
    device_checks(AAH_BF16);
    device_checks(AAH_F32);
    aah_cache_clear();
  }
  puts("ok");
  return 0;
}
