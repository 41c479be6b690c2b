// Two memory-system probes behind design decisions of the attention kernels
// (measurement tools, not part of the attention path).
//
//   mem_probes atomic   fp32 atomic adds (no return) against plain stores and
//                       load-add-store, in the shape a dQ accumulation over
//                       key items would have: each step adds a 64-row x 128
//                       fp32 tile of one head into a [L][32][128] buffer.
//                       Prints one JSON line per run and an exactness check.
//   mem_probes lds      the two LDS operand read patterns of the kernels (16-
//                       byte direct reads of 16 rows at one column; 8-byte
//                       transposing reads of 4 rows x 64 bytes) over a 64-row
//                       block at several row strides; one kernel per pattern
//                       and stride, meant to run under rocprofv3 with the
//                       SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE counters.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

namespace libra {

constexpr int kL = 262144, kH = 32, kD = 128, kT = 512, kPer = 64 * kD / kT;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// MODE 0: atomicAdd; 1: store; 2: load + add + store.  Row block rb < kL / 64
// and head < kH, so every address is inside the kL * kH * kD buffer.
template <int MODE>
__global__ __launch_bounds__(kT) void atomic_probe(float *acc, int steps) {
  const int tid = threadIdx.x;
  const uint32_t base = mix32(blockIdx.x * 977u + 1u);
  for (int i = 0; i < steps; ++i) {
    const uint32_t h = mix32(base ^ (uint32_t)i * 2654435761u);
    const int rb = (int)(h % (uint32_t)(kL / 64));
    const int head = (int)((h >> 12) % (uint32_t)kH);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = tid + kT * j, row = e / kD, col = e % kD;
      float *p = acc + ((int64_t)(rb * 64 + row) * kH + head) * kD + col;
      const float v = 1.0f + (float)(j & 3);
      if (MODE == 0)
        atomicAdd(p, v);
      else if (MODE == 1)
        __builtin_nontemporal_store(v, p);
      else
        *p += v;
    }
  }
}

typedef short s16x4p __attribute__((ext_vector_type(4)));
typedef unsigned u32x4p __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int sigma16(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// PAT 0: direct reads (rows sigma(lane mod 32) + 32 t, 16-byte slabs s);
// PAT 1: transposing reads (rows 8 (g >> 1) + (j >> 2) + 16 t + 4 p + 32 kt,
// columns 16 (g & 1) + 4 (j & 3) + 32 dt).  Rows stay below 64 and columns
// below 128 <= RS, so every read is inside the 64 x RS block.
template <int PAT, int RS>
__global__ __launch_bounds__(256) void lds_probe(unsigned *out, int iters) {
  __shared__ __attribute__((aligned(16))) uint16_t blk[64 * RS];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < 64 * RS; i += 256) blk[i] = (uint16_t)((unsigned)i * 2654435761u >> 7);
  __syncthreads();
  const int dlo = sigma16(lane & 31) * RS + 8 * (lane >> 5);
  const int g = lane >> 4, j = lane & 15;
  const int tlo = (8 * (g >> 1) + (j >> 2)) * RS + 16 * (g & 1) + 4 * (j & 3);
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    if (PAT == 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const u32x4p v = *reinterpret_cast<const u32x4p *>(blk + dlo + 32 * t * RS + 16 * s);
          acc ^= v[0] + v[1] + v[2] + v[3];
        }
    } else {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const s16x4p v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4p *)(__attribute__((address_space(3))) void *)(
                      blk + tlo + (kt * 32 + 16 * t + 4 * p) * RS + dt * 32));
              acc ^= (unsigned)v[0] + (unsigned)v[1] * 3u + (unsigned)v[2] * 5u + (unsigned)v[3] * 7u;
            }
    }
    acc = acc * 1664525u + (unsigned)it;
  }
  out[blockIdx.x * 256 + tid] = acc;
}

}  // namespace libra

namespace {

bool ok(hipError_t e, const char *what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

int run_atomic() {
  using namespace libra;
  const size_t n = (size_t)kL * kH * kD;
  float *acc = nullptr;
  if (!ok(hipMalloc(&acc, n * sizeof(float)), "hipMalloc")) return 1;
  if (!ok(hipMemset(acc, 0, n * sizeof(float)), "hipMemset")) return 1;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return 1;
  const int grid = 768, steps = 600;
  const char *names[3] = {"atomic_add_f32", "store", "load_add_store"};
  for (int rep = 0; rep < 2; ++rep)
    for (int mode = 0; mode < 3; ++mode) {
      (void)hipEventRecord(a);
      if (mode == 0) atomic_probe<0><<<grid, kT>>>(acc, steps);
      if (mode == 1) atomic_probe<1><<<grid, kT>>>(acc, steps);
      if (mode == 2) atomic_probe<2><<<grid, kT>>>(acc, steps);
      (void)hipEventRecord(b);
      if (!ok(hipEventSynchronize(b), "kernel")) return 1;
      float ms = 0;
      (void)hipEventElapsedTime(&ms, a, b);
      const double bytes = (double)grid * steps * 64 * kD * 4;
      std::printf("{\"op\": \"%s\", \"rep\": %d, \"ms\": %.3f, \"payload_GBps\": %.1f}\n", names[mode], rep, ms,
                  bytes / ms / 1e6);
    }
  // exactness: one atomic launch into a zeroed buffer; small integers sum exactly
  if (!ok(hipMemset(acc, 0, n * sizeof(float)), "hipMemset")) return 1;
  atomic_probe<0><<<grid, kT>>>(acc, 50);
  std::vector<float> h(n);
  if (!ok(hipMemcpy(h.data(), acc, n * sizeof(float), hipMemcpyDeviceToHost), "copy")) return 1;
  double got = 0, expect = 0;
  for (size_t i = 0; i < n; ++i) got += h[i];
  for (int j = 0; j < kPer; ++j) expect += (1.0 + (j & 3)) * kT;
  expect *= (double)grid * 50;
  std::printf("{\"check\": \"atomic total\", \"got\": %.1f, \"expect\": %.1f, \"exact\": %s}\n", got, expect,
              got == expect ? "true" : "false");
  (void)hipFree(acc);
  return got == expect ? 0 : 2;
}

template <int PAT, int RS>
bool lds_one(unsigned *out) {
  libra::lds_probe<PAT, RS><<<1024, 256>>>(out, 400);
  if (!ok(hipDeviceSynchronize(), "lds probe")) return false;
  std::printf("{\"pattern\": \"%s\", \"row_stride\": %d}\n", PAT == 0 ? "direct_b128" : "transpose_b64", RS);
  return true;
}

template <int PAT>
bool lds_all(unsigned *out) {
  return lds_one<PAT, 128>(out) && lds_one<PAT, 136>(out) && lds_one<PAT, 144>(out) && lds_one<PAT, 152>(out) &&
         lds_one<PAT, 160>(out) && lds_one<PAT, 168>(out) && lds_one<PAT, 176>(out) && lds_one<PAT, 192>(out) &&
         lds_one<PAT, 224>(out);
}

int run_lds() {
  unsigned *out = nullptr;
  if (!ok(hipMalloc(&out, 1024 * 256 * sizeof(unsigned)), "hipMalloc")) return 1;
  const bool good = lds_all<0>(out) && lds_all<1>(out);
  (void)hipFree(out);
  return good ? 0 : 1;
}

}  // namespace

int main(int argc, char **argv) {
  if (argc == 2 && std::strcmp(argv[1], "atomic") == 0) return run_atomic();
  if (argc == 2 && std::strcmp(argv[1], "lds") == 0) return run_lds();
  std::fprintf(stderr, "usage: mem_probes atomic|lds\n");
  return 64;
}
