// Device-side building blocks for gfx950 (CDNA4) attention kernels.
//
// Matrix products use v_mfma_f32_32x32x16_bf16: A is 32x16, B is 16x32, both
// bf16; C/D is 32x32 fp32.  Per lane l (wave of 64):
//   A operand: row l % 32, eight reduction elements of group l / 32;
//   B operand: column l % 32, eight reduction elements of group l / 32;
//   C/D: column l % 32, rows 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15.
// The kernels only assume that A and B place the reduction index the same
// way, so every operand below is loaded with reduction element (l / 32, i) =
// index 8 * (l / 32) + i of a 16-wide slab.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libra.h"

namespace libra {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

// Two fp32 values rounded to bf16 (nearest even) and packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The two fp32 values a packed bf16 pair stands for.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a per-lane value with the same lane of the other 32-lane half.
__device__ __forceinline__ float halves_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// Plan arrays and cu_seqlens are never written while a kernel runs, so the
// kernels read them through the constant address space: wave-uniform reads
// then compile to scalar loads.  Those are counted apart from vector memory
// operations, so an item's set-up (descriptor, sample bounds) does not wait
// behind the vector memory queue that still holds the previous item's output
// stores, as vector loads would.
template <typename T>
using cptr = const __attribute__((address_space(4))) T *;
template <typename T>
__device__ __forceinline__ cptr<T> as_const(const T *p) { return (cptr<T>)p; }

// Work item it of a plan queue (wave-uniform it), read field by field through
// the constant address space.  The kernels do not use the placement fields
// (cost, pairs), which are left zero.
__device__ __forceinline__ libra_item load_item(const libra_item *items, int it) {
  static_assert(sizeof(libra_item) % 4 == 0, "32-bit fields");
  const cptr<int32_t> f = as_const(reinterpret_cast<const int32_t *>(items + it));
  libra_item r;
  r.row0 = f[offsetof(libra_item, row0) / 4];
  r.nrows = f[offsetof(libra_item, nrows) / 4];
  r.kv_head = f[offsetof(libra_item, kv_head) / 4];
  r.head0 = f[offsetof(libra_item, head0) / 4];
  r.nheads = f[offsetof(libra_item, nheads) / 4];
  r.tile_id = f[offsetof(libra_item, tile_id) / 4];
  r.id = f[offsetof(libra_item, id) / 4];
  r.flags = f[offsetof(libra_item, flags) / 4];
  r.cost = 0;
  r.pairs = 0;
  return r;
}

// Index of the sample that holds token t, for a wave-uniform t < cu[n]: the
// largest j < n with cu[j] <= t (so empty samples are passed over).  A binary
// search over cu_seqlens with scalar loads.
__device__ __forceinline__ int sample_index(cptr<int32_t> cu, int n, int t) {
  int lo = 0, hi = n;   // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Bounds [start, end) of the sample that holds this lane's token q, where the
// tokens of the wave lie in the wave-uniform range [t0, t1], t1 < cu[n].  The
// samples that begin inside the range are walked in order with scalar loads
// and each lane keeps the last one that starts at or before q; lanes whose q
// lies outside the range get meaningless bounds.
__device__ __forceinline__ void lane_sample(cptr<int32_t> cu, int n, int t0, int t1, int q,
                                            int &start, int &end) {
  int j = sample_index(cu, n, t0);
  int s = cu[j], e = cu[j + 1];
  start = s;
  end = e;
  while (e <= t1) {   // sample j + 1 begins inside the range; e <= t1 < cu[n] gives j + 1 < n
    ++j;
    s = e;
    e = cu[j + 1];
    if (q >= s) {
      start = s;
      end = e;
    }
  }
}

// Physical placement of the running wave, for per-CU busy records.
__device__ __forceinline__ uint32_t hw_id_reg() {
  return __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);    // HW_REG_HW_ID
}
__device__ __forceinline__ uint32_t xcc_id_reg() {
  return __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 20);   // HW_REG_XCC_ID
}

// Direct global -> LDS copy of 16 bytes per lane: lane i of the wave copies
// the 16 bytes at sbase + voff (sbase wave-uniform, in scalar registers; voff
// the lane's 32-bit byte offset) to lds_base + 16 * i (lds_base is made
// wave-uniform); lanes switched off by control flow copy nothing.  The copy
// is issued from inline assembly so the compiler does not track it: callers
// account for every copy themselves with wait_vmem (the vector-memory counter
// retires in issue order) and a barrier before another wave reads the data.
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// A pointer every lane holds the same value of, moved into scalar registers.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(((uint64_t)hi << 32) | lo);
}

// The same for 4 bytes per lane from a per-lane address: lane i copies the 4
// bytes at gsrc to lds_base + 4 * i.
__device__ __forceinline__ void lds_dma4(const void *gsrc, uint32_t lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(gsrc) : "memory", "m0");
}

// Byte address of a __shared__ object in the LDS aperture.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Index of the calling wave in its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until at most n (0..15, wave-uniform) vector-memory operations of this
// wave are outstanding.
__device__ __forceinline__ void wait_vmem_upto(int n) {
  switch (n) {
    case 0: wait_vmem<0>(); break;
    case 1: wait_vmem<1>(); break;
    case 2: wait_vmem<2>(); break;
    case 3: wait_vmem<3>(); break;
    case 4: wait_vmem<4>(); break;
    case 5: wait_vmem<5>(); break;
    case 6: wait_vmem<6>(); break;
    case 7: wait_vmem<7>(); break;
    case 8: wait_vmem<8>(); break;
    case 9: wait_vmem<9>(); break;
    case 10: wait_vmem<10>(); break;
    case 11: wait_vmem<11>(); break;
    case 12: wait_vmem<12>(); break;
    case 13: wait_vmem<13>(); break;
    case 14: wait_vmem<14>(); break;
    default: wait_vmem<15>(); break;
  }
}

// Wait until this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Both: no vector-memory operation (including LDS-DMA copies) and no LDS
// access of this wave is outstanding.
__device__ __forceinline__ void wait_vmem_lds() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Workgroup barrier that keeps the compiler from moving memory accesses across
// it but adds no memory-counter waits: the kernels wait explicitly (wait_vmem
// for their LDS-DMA copies, wait_lds before a buffer is refilled), so copies
// for the next block stay in flight across the barrier.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Rows of a block sit in LDS permuted within each group of 16: logical row x
// is stored at physical row lds_row(x), which swaps the two 2-bit fields of
// x mod 16 (an involution).  With a row stride of an odd number of 16-byte
// chunks, both operand read patterns are then free of bank conflicts:
//   - a 16-byte direct read serves 16 lanes reading 16 rows of one 16-row
//     group at one column: any permutation of the group keeps their chunks
//     on 16 distinct groups of four banks;
//   - a transposing read serves 32 lanes reading four consecutive logical
//     rows 4i .. 4i + 3 of a group, 64 bytes each: they are stored at rows
//     i, i + 4, i + 8, i + 12, whose starting banks lie 16 dwords apart for
//     every odd chunk stride, so the four 64-byte pieces cover the 64 banks.
// The copy into LDS fills physical row R with logical row lds_row(R); every
// read offset stays a per-lane constant plus a compile-time immediate.
__device__ __forceinline__ constexpr int lds_row(int x) {
  return (x & ~15) | ((x & 3) << 2) | ((x >> 2) & 3);
}

// Row m of a 32-row C tile produced from A rows loaded in the order sigma:
// sigma swaps bits 2 and 3, so C registers 8t..8t+7 of lane half h hold
// A rows 16t + 8h + 0..7 (contiguous), ready to be a B operand.
__device__ __forceinline__ int sigma_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j supplies the address of four consecutive 16-bit values M[j][0..3];
// lane 4a + b receives M[a][b], M[a + 4][b], M[a + 8][b], M[a + 12][b].
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(const __attribute__((address_space(3))) void *)p);
}

// Row-major bf16 blocks of D columns live in LDS with a padded row stride of
// an odd number of 16-byte chunks; with the row permutation lds_row, direct
// and transposing operand reads are then both free of bank conflicts.  The
// kernels pick among such strides so that the copies of a block pair divide
// evenly among their waves (PairCopy):
//   kStride       = 152 elements (19 chunks; D = 128) or 72 (9; D = 64);
//   kDirectStride = 136 (17 chunks; D = 128) or 72 (D = 64), the shortest
//                   (17 copy instructions per 64-row block instead of 19).
// Every operand address stays a per-lane base plus a compile-time offset.
template <int D>
struct PadRows {
  static_assert(D == 128 || D == 64, "head_dim 64 or 128");
  static constexpr int kStride = D == 128 ? 152 : 72;     // elements per row
  static constexpr int kDirectStride = D == 128 ? 136 : 72;
};

// Copy of two blocks of NR rows each (D elements per row, row r at src +
// r * stride), the first into LDS rows of RA elements and the second into
// rows of RB, as one list of NA + NB one-kilobyte LDS-DMA instructions:
// instruction g is issued by wave g mod NW.  When NW divides NA + NB, every
// wave issues exactly kPerWave copies per pair of blocks, so the count a
// wave waits for is a compile-time constant and no wave branches on whether
// it has a copy to issue.  A lane whose 16-byte slot is a row's padding
// copies that row's first chunk into the padding, which is never read, so no
// lane is switched off.  The lane's offsets are fixed per kernel.
template <int D, int NR, int NW, int RA, int RB>
struct PairCopy {
  static constexpr int NA = (NR * RA * 2 + 1023) / 1024;
  static constexpr int NB = (NR * RB * 2 + 1023) / 1024;
  static constexpr int NI = NA + NB;
  static constexpr int NJ = (NI + NW - 1) / NW;
  static constexpr bool kUniform = NI % NW == 0;
  static constexpr int kPerWave = NI / NW;
  static_assert(NA * 1024 == NR * RA * 2 && NB * 1024 == NR * RB * 2, "the blocks fill whole copy instructions");
  uint32_t voff[NJ];                         // byte offset of the lane's source: row * stride + col

  // Copy instructions a wave issues per pair of blocks.
  static __device__ __forceinline__ int count(int wave) { return wave < NI ? (NI - 1 - wave) / NW + 1 : 0; }

  __device__ __forceinline__ void init(int wave, int lane, int64_t stride) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int g = wave + j * NW;
      const bool in_a = g < NA;
      const int rs = in_a ? RA : RB;
      const int e = 512 * (in_a ? g : g - NA) + 8 * lane;   // element offset of the lane's slot
      const int row = e / rs, c = e - row * rs;             // physical row of the slot
      const int col = c < D ? c : 0;
      voff[j] = g < NI ? (uint32_t)(2 * ((int64_t)lds_row(row) * stride + col)) : 0u;
    }
  }
  // Rows r0 .. r0 + NR - 1 of both tensors; rows at or past `rows` (only in
  // the pack's last block) are replaced by row rows - 1, recovering the
  // lane's row and column from its offset behind an empty asm statement so
  // that none of it is hoisted out of the caller's loops.
  __device__ __forceinline__ void issue(uint32_t lds_a, uint32_t lds_b, int wave, const uint16_t *base_a,
                                        const uint16_t *base_b, int64_t stride, int r0, int rows) const {
    const void *ba = uniform_ptr(base_a + (int64_t)r0 * stride);
    const void *bb = uniform_ptr(base_b + (int64_t)r0 * stride);
    if (r0 + NR <= rows) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int g = wave + j * NW;
        if (kUniform || g < NI) {
          const bool in_a = g < NA;
          lds_dma16_s(in_a ? ba : bb, voff[j], in_a ? lds_a + 1024 * g : lds_b + 1024 * (g - NA));
        }
      }
    } else {
      const uint32_t st = (uint32_t)stride;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int g = wave + j * NW;
        if (kUniform || g < NI) {
          const bool in_a = g < NA;
          uint32_t vo = voff[j];
          asm volatile("" : "+v"(vo));
          const uint32_t e = vo >> 1;            // row * stride + col
          const uint32_t row = e / st, col = e - row * st;
          const uint32_t rr = (uint32_t)min(r0 + (int)row, rows - 1) - (uint32_t)r0;
          lds_dma16_s(in_a ? ba : bb, 2 * (rr * st + col), in_a ? lds_a + 1024 * g : lds_b + 1024 * (g - NA));
        }
      }
    }
  }
};

// Direct A operand: lane (col, half) reads logical row sigma_row(col) + 32 t
// of the block, reduction elements 16 s + 8 half .. + 7.  direct_lane_off is
// the lane's part (its physical row); slab (t, s) adds direct_off(t, s).
template <int RS>
__device__ __forceinline__ int direct_lane_off(int lane) {
  return lds_row(sigma_row(lane & 31)) * RS + 8 * (lane >> 5);
}
template <int RS>
constexpr int direct_off(int t, int s) { return 32 * t * RS + 16 * s; }

// MFMA A operand of Mat^T from a row-major padded block Mat [rows][D] in LDS:
// lane (col, half) receives Mat[k0 + 8 half + i][r0 + col], i = 0..7.  Lane j
// of 16-lane group g addresses logical row k0 + 8 (g >> 1) + 4 p + j / 4,
// columns r0 + 16 (g & 1) + 4 (j % 4) + 0..3, for the two reads p = 0, 1; by
// the rule of the transposing read the group's lane i then holds rows
// k0 + 8 (g >> 1) + 4 p + 0..3 of column r0 + 16 (g & 1) + i.  With k0 a
// multiple of 16 that logical row sits at physical row
// k0 + 4 (j / 4) + 2 (g >> 1) + p (lds_row); tr_lane_off is the lane's part,
// (k0, r0, p) add tr_off(k0, r0, p).
template <int RS>
__device__ __forceinline__ int tr_lane_off(int lane) {
  const int g = lane >> 4, j = lane & 15;
  return (4 * (j >> 2) + 2 * (g >> 1)) * RS + 16 * (g & 1) + 4 * (j & 3);
}
template <int RS>
constexpr int tr_off(int k0, int r0, int p) { return (k0 + p) * RS + r0; }

__device__ __forceinline__ bf16x8 lds_tr_operand(const uint16_t *lo_p, const uint16_t *hi_p) {
  const s16x4 lo = lds_read_tr16(lo_p), hi = lds_read_tr16(hi_p);
  const s16x4 v[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v);
}


}  // namespace libra
