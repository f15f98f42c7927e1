// Measurement probe (not part of the library): do the matrix cores and the
// vector ALU of one SIMD work at the same time when different waves feed
// them?  Every wave runs the same loop; per iteration it issues, depending on
// the mode, 16 v_mfma_f32_32x32x16_bf16 (two independent accumulator chains),
// 128 independent-chain v_med3_f32, or both.  Twelve waves per CU (three
// workgroups of four), 24 rounds of workgroups over the 256 CUs.  If the two
// units overlap, the time of "both" is near the larger of the two alone; if
// they do not, near their sum.
//
//   hipcc --offload-arch=gfx950 -O3 -o mfma_valu_overlap mfma_valu_overlap.hip
//   ./mfma_valu_overlap        (prints one JSON line)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define CHECK(x)                                                                     \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

constexpr int kThreads = 256;
constexpr int kValuPerIter = 128;

// mode bit 0: MFMA chains; bit 1: VALU chains
__global__ __launch_bounds__(kThreads) void probe(float* out, int iters, int mode, float seed) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (lane + e));
    b[e] = (__bf16)(seed * (lane - e));
  }
  f32x16 acc0 = {}, acc1 = {};
  float v0 = seed * lane, v1 = v0 + 1.f, v2 = v0 + 2.f, v3 = v0 + 3.f;
  for (int it = 0; it < iters; ++it) {
    if (mode & 1) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc1, 0, 0, 0);
      }
    }
    if (mode & 2) {
#pragma unroll
      for (int i = 0; i < kValuPerIter / 4; ++i) {
        v0 = __builtin_amdgcn_fmed3f(v0, v1, v2);
        v1 = __builtin_amdgcn_fmed3f(v1, v2, v3);
        v2 = __builtin_amdgcn_fmed3f(v2, v3, v0);
        v3 = __builtin_amdgcn_fmed3f(v3, v0, v1);
      }
    }
  }
  float s = v0 + v1 + v2 + v3;
  for (int r = 0; r < 16; ++r) s += acc0[r] + acc1[r];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;  // keeps both chains live
}

int main() {
  const int blocks = 256 * 3 * 8;
  const int iters = 256;
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)blocks * kThreads * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const char* names[3] = {"mfma_ms", "valu_ms", "both_ms"};
  float ms[3];
  for (int m = 1; m <= 3; ++m) {
    float best = 1e30f;
    for (int rep = 0; rep < 3; ++rep) {
      CHECK(hipEventRecord(e0));
      probe<<<blocks, kThreads>>>(out, iters, m, 1e-3f);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float t = 0.f;
      CHECK(hipEventElapsedTime(&t, e0, e1));
      best = t < best ? t : best;
    }
    ms[m - 1] = best;
  }
  const double flops = 16.0 * 32 * 32 * 16 * 2 * iters * 4.0 * blocks;  // 4 waves per workgroup
  std::printf("{\"%s\": %.4f, \"%s\": %.4f, \"%s\": %.4f, \"mfma_alone_tflops\": %.1f}\n", names[0], ms[0], names[1],
              ms[1], names[2], ms[2], flops / ms[0] / 1e9);
  CHECK(hipFree(out));
  return 0;
}
