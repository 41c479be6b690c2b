// Sustained bf16 MFMA throughput probe (a measurement tool, not part of the library).
//
// Every wave of 256 workgroups x 8 waves (two per SIMD) issues back-to-back
// v_mfma_f32_32x32x16_bf16 on four independent accumulators for ~3 s of
// consecutive launches, once with constant operands and once with operands of
// random bits (bf16 values in [0.5, 2) of either sign).  The chip's clock
// follows its power draw, and the draw of the matrix cores follows how many
// operand bits toggle, so the second figure is the MFMA rate real data can
// sustain.  Prints one JSON line.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kThreads = 512;
constexpr int kBlocks = 256;
constexpr int kIters = 65536;   // MFMA rounds per wave and launch (a multiple of 4)

__device__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <bool RANDOM>
__global__ __launch_bounds__(kThreads) void probe(float *out) {
  bf16x8 a[4], b[4];
  for (int j = 0; j < 4; ++j) {
    u32x4 ua, ub;
    for (int i = 0; i < 4; ++i) {
      const uint32_t r1 = mix(blockIdx.x * 7919u + threadIdx.x * 131u + j * 17u + i);
      const uint32_t r2 = mix(r1 + 7u);
      ua[i] = RANDOM ? ((r1 & 0x807f807fu) | 0x3f003f00u) : 0x3f803f80u;
      ub[i] = RANDOM ? ((r2 & 0x807f807fu) | 0x3f003f00u) : 0x3f803f80u;
    }
    a[j] = __builtin_bit_cast(bf16x8, ua);
    b[j] = __builtin_bit_cast(bf16x8, ub);
  }
  f32x16 c[4];
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 16; ++i) c[j][i] = 0.0f;
  for (int it = 0; it < kIters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + u) & 3], b[(j + 2 * u) & 3], c[j], 0, 0, 0);
  }
  float s = 0.0f;
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 16; ++i) s += c[j][i];
  if (s == 1234.5f) out[blockIdx.x] = s;   // keeps the products live
}

// Median TFLOP/s of the launches of the last second of a ~3 s run.
template <bool RANDOM>
double run(float *d) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.0;
  const double flops = (double)kBlocks * (kThreads / 64) * kIters * 4 * 32768.0;
  double total = 0.0, tail[512];
  int n = 0, nt = 0;
  while (total < 3000.0 && n < 1000) {
    (void)hipEventRecord(e0);
    hipLaunchKernelGGL(probe<RANDOM>, dim3(kBlocks), dim3(kThreads), 0, 0, d);
    (void)hipEventRecord(e1);
    if (hipEventSynchronize(e1) != hipSuccess) return -1.0;
    float ms = 0.0f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    total += ms;
    ++n;
    if (total > 2000.0 && nt < 512) tail[nt++] = flops / (ms * 1e-3) / 1e12;
  }
  for (int i = 1; i < nt; ++i)
    for (int j = i; j > 0 && tail[j - 1] > tail[j]; --j) {
      const double t = tail[j];
      tail[j] = tail[j - 1];
      tail[j - 1] = t;
    }
  return nt ? tail[nt / 2] : -1.0;
}

}  // namespace

int main() {
  float *d = nullptr;
  if (hipMalloc(&d, 4096) != hipSuccess) return 1;
  const double constant = run<false>(d);
  const double random = run<true>(d);
  if (hipGetLastError() != hipSuccess || constant < 0 || random < 0) return 2;
  printf("{\"mfma\": \"v_mfma_f32_32x32x16_bf16\", \"waves_per_simd\": 2, \"seconds_each\": 3, "
         "\"tflops_constant_operands\": %.1f, \"tflops_random_operands\": %.1f, \"nominal_peak\": 2516.6}\n",
         constant, random);
  (void)hipFree(d);
  return 0;
}
