// Backward of packed block-diagonal causal attention on gfx950: the row-dot
// phase D = rowsum(dO * O) and the query-major dQ pass (see attn_bwd.hip for
// the method).  These two kernels live apart from the dK/dV pass so that the
// build can give them their own instruction scheduling.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>

#include "bwd_common.h"

namespace libra {

namespace {

// D[h][t] = sum_d dO[t][h][d] * O[t][h][d], one row per D/8 lanes; also the
// forward's LSE in log2 units, lse2[h][t] = LSE[h][t] * log2(e).
template <int D>
__global__ __launch_bounds__(kThreads) void rowdot_kernel(const uint16_t *__restrict__ o,
                                                          const uint16_t *__restrict__ dout,
                                                          const float *__restrict__ lse,
                                                          float *__restrict__ dvec, float *__restrict__ lse2,
                                                          int L, int h_q) {
  constexpr int LPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  const int64_t rows = (int64_t)L * h_q;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(o + row * D + sub * 8);
    const u32x4 y = *reinterpret_cast<const u32x4 *>(dout + row * D + sub * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(x[i]) * bf16_lo(y[i]) + bf16_hi(x[i]) * bf16_hi(y[i]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (sub == 0 && row < rows) {
    const int64_t t = row / h_q, h = row % h_q;
    dvec[h * L + t] = acc;
    lse2[h * L + t] = lse[h * L + t] * kLog2e;
  }
}

// ----------------------------------------------------------------- dQ pass
// Eight waves of 32 query positions each cover the kDqItemColumns query
// columns of a dQ work item (two waves per SIMD: the kernel needs more than
// the 168 registers three would leave).  Per key block of kKB keys, LDS
// holds K and V (row-major: A operands of S^T and dP^T, and through
// transposing reads the K^T operand of dQ^T), in a ring of kStages buffers
// like the forward; all query heads of the item's KV head read the same copy.
constexpr int kDqWaves = kDqItemColumns / 32;

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kDqWaves * 64, kDqWaves * 64), amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = kDqWaves;
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int RS = PadRows<D>::kStride;          // K rows: direct and transposing reads
  // V rows, read only directly, take the conflict-free 168 (D = 128) or 120
  // (D = 64) elements, so that a K and a V block fill 19 + 21 = 40 (9 + 15 =
  // 24) copy instructions, the same number for each of the eight waves.
  constexpr int RV = D == 128 ? 168 : 120;
  constexpr int KBLK = kKB * RS, BUF = KBLK + kKB * RV;
  // kStages buffers of a K and a V block; block b uses buffer b mod kStages.
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[kStages * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int half = lane >> 5, col = lane & 31;
  const int w = blockIdx.x;
  const uint64_t t_start = wall_clock64();
  // A device plan that is not a copy of the host plan runs no item.
  const bool plan_ok = as_const(a.plan_sum_dev)[0] == a.plan_sum;
  const int beg = plan_ok ? as_const(a.cu_off)[w] : 0, end = plan_ok ? as_const(a.cu_off)[w + 1] : 0;
  const cptr<int32_t> cu = as_const(a.cu);
  const float c = a.scale_log2;
  const uint32_t kv_base = lds_addr(kv_lds);
  const int dlo = direct_lane_off<RS>(lane);       // K operand reads
  const int dlo_v = direct_lane_off<RV>(lane);     // V operand reads
  const int tlo = tr_lane_off<RS>(lane);           // K^T operand reads
  const int64_t kv_stride = (int64_t)a.h_kv * D;
  using KVCopy = PairCopy<D, kKB, NW, RS, RV>;
  static_assert(KVCopy::kUniform, "every wave issues the same number of copies");
  KVCopy kvcopy;
  kvcopy.init(wave, lane, kv_stride);

  // Operands of the wave's query of item itq: Q and dO rows, LSE * log2(e)
  // and D.  Each item's are loaded as soon as the previous item's last block
  // is done, before that item's dQ is stored, so their latency overlaps the
  // stores, the next item's set-up and the item-start barrier.
  float lse2, dd;
  bf16x8 qop[NS], dop[NS];
  auto load_rows = [&](int itq) {
    const libra_item nx = load_item(a.items, itq);
    const int nhx = nx.nheads, hx = nx.head0 + (wave % nhx);
    const int rx = (wave / nhx) * 32 + col;
    const bool okx = rx < nx.nrows;
    const int px = nx.row0 + rx;
    lse2 = okx ? a.lse2[(int64_t)hx * a.L + px] : 0.0f;
    dd = okx ? a.dvec[(int64_t)hx * a.L + px] : 0.0f;
    const int64_t base = ((int64_t)px * a.h_q + hx) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qop[s] = as_bf16x8(okx ? *reinterpret_cast<const u32x4 *>(a.q + base + 16 * s) : zero_u32x4());
      dop[s] = as_bf16x8(okx ? *reinterpret_cast<const u32x4 *>(a.dout + base + 16 * s) : zero_u32x4());
    }
  };

  for (int it = beg; it < end; ++it) {
    const libra_item item = load_item(a.items, it);
    if (it == beg) load_rows(it);
    const int row0 = item.row0, nrows = item.nrows, kvh = item.kv_head, nh = item.nheads;
    const int head = item.head0 + (wave % nh);
    const int sub = wave / nh;
    const int r = sub * 32 + col;
    const bool qok = r < nrows;
    const int qpos = row0 + r;
    // Sample start of each query of the wave (scalar loads only).
    int qss = 0;
    if (sub * 32 < nrows) {
      int st, en;
      lane_sample(cu, a.n_samples, row0 + sub * 32, row0 + min(nrows, sub * 32 + 32) - 1, qpos, st, en);
      if (qok) qss = st;
    }
    const int kstart = cu[sample_index(cu, a.n_samples, row0)] & ~(kKB - 1);
    const int kend = row0 + nrows;
    const int nkb = (kend - kstart + kKB - 1) / kKB;
    // Step b's key block: up from the sample start, or (LIBRA_ITEM_REVERSE,
    // the second item of a zigzag pair) down from the item's last block.
    const bool rev = (item.flags & LIBRA_ITEM_REVERSE) != 0;
    auto kblock = [&](int b) { return kstart + (rev ? nkb - 1 - b : b) * kKB; };

    f32x16 dqacc[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) dqacc[dt] = zero16();

    auto issue = [&](int k0, int buf) {   // rows past L are masked; clamped to row L - 1
      const uint32_t dst = kv_base + buf * 2 * BUF;   // bytes
      kvcopy.issue(dst, dst + 2 * KBLK, wave, a.k + kvh * D, a.v + kvh * D, kv_stride, k0, a.L);
    };

    auto block = [&](int b, int buf) {
      const uint16_t *bk = kv_lds + buf * BUF;
      const int k0 = kblock(b);
      // block b landed; block b + 1 may fly
      if (b + 1 < nkb) wait_vmem<KVCopy::kPerWave>(); else wait_vmem<0>();
      wait_lds();
      block_barrier();
      if (b + kStages - 1 < nkb) issue(kblock(b + kStages - 1), buf == 0 ? kStages - 1 : buf - 1);
      const bool touch = qok && (k0 <= qpos) && (k0 + kKB - 1 >= qss);
      const bool partial = qok && !((k0 >= qss) && (k0 + kKB - 1 <= qpos));
      if (wave_any(touch)) {
        const bool masked = wave_any(partial);
        const uint16_t *k_l = bk, *v_l = bk + KBLK;
        const int lo = qok ? qss : 1, hi = qok ? qpos : 0;
        // One 32-key tile at a time keeps S^T, dP^T and dS^T of a single tile live.
#pragma unroll
        for (int kt = 0; kt < kKB / 32; ++kt) {
          __builtin_amdgcn_sched_barrier(0);   // the groups below cover this tile's S^T and dP^T only
          f32x16 sacc = zero16(), pacc = zero16();   // S^T and dP^T (lane = query)
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4 *>(k_l + dlo + direct_off<RS>(kt, s)));
            const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4 *>(v_l + dlo_v + direct_off<RV>(kt, s)));
            sacc = mfma32x32x16(ka, qop[s], sacc);
            pacc = mfma32x32x16(va, dop[s], pacc);
          }
          // Two K / V operand reads first, then one read after each product:
          // every product finds its operand loaded while the next read flies.
          {
            constexpr int kReads = 2 * NS, kAhead = 2;
            __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
            for (int i = 0; i < kReads - kAhead; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
          }
          if (masked) {             // rare: blocks on a sample start or the diagonal
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int kk = k0 + kt * 32 + 16 * (rr >> 3) + 8 * half + (rr & 7);
              if (kk < lo || kk > hi) sacc[rr] = -__builtin_inff();
            }
          }
          u32x4 dsw[2];   // [16-key slab]: bf16 dS^T operands
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float ds2[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const int rr = 8 * t + 2 * i + e;
                const float pv = exp2_fast(fmaf(sacc[rr], c, -lse2));   // masked: 2^-inf = 0
                ds2[e] = pv * (pacc[rr] - dd);
              }
              dsw[t][i] = pack_bf16x2(ds2[0], ds2[1]);
            }
#pragma unroll
          for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int t = 0; t < 2; ++t) {   // K^T operand read transposed from the row-major K block
              const bf16x8 ka = lds_tr_operand(k_l + tlo + tr_off<RS>(kt * 32 + 16 * t, dt * 32, 0),
                                               k_l + tlo + tr_off<RS>(kt * 32 + 16 * t, dt * 32, 1));
              dqacc[dt] = mfma32x32x16(ka, as_bf16x8(dsw[t]), dqacc[dt]);
            }
        }
      }
    };

    wait_lds();
    block_barrier();                // the previous item's reads of every buffer are done
    // This item's operands and the previous item's dQ stores have been in
    // flight since the previous item's last block: one full wait for them
    // here, before the first copies, costs little and tells the compiler that
    // the operand registers are loaded (it cannot see that the per-block copy
    // waits cover them, and would otherwise wait for every copy at every block).
    wait_vmem<0>();
#pragma unroll
    for (int b = 0; b < kStages - 1; ++b)
      if (b < nkb) issue(kblock(b), b);
    for (int b = 0, buf = 0; b < nkb; ++b, buf = buf == kStages - 1 ? 0 : buf + 1) block(b, buf);
    if (it + 1 < end) load_rows(it + 1);

    if (qok) {
      uint16_t *op = a.dq + ((int64_t)qpos * a.h_q + head) * D;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          u32x2 pk;
          pk[0] = pack_bf16x2(dqacc[dt][4 * cc] * a.scale, dqacc[dt][4 * cc + 1] * a.scale);
          pk[1] = pack_bf16x2(dqacc[dt][4 * cc + 2] * a.scale, dqacc[dt][4 * cc + 3] * a.scale);
          *reinterpret_cast<u32x2 *>(op + dt * 32 + 8 * cc + 4 * half) = pk;
        }
    }
  }
  __syncthreads();
  if (a.records != nullptr && tid == 0) write_record(a, w, end - beg, t_start, plan_ok);
}

}  // namespace

libra_status launch_prepare(const libra_plan_info &h, const void *o, const void *dout, const float *lse,
                            void *ws, void *stream) {
  const libra_plan_params &p = h.params;
  const BwdLayout lay = bwd_layout(p);
  char *w = static_cast<char *>(ws);
  const int64_t rows = (int64_t)p.total_tokens * p.h_q;
  const int rows_per_block = kThreads / (p.head_dim / 8);
  const dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block));
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *dvec = reinterpret_cast<float *>(w + lay.dvec);
  float *lse2 = reinterpret_cast<float *>(w + lay.lse2);
  clear_hip_error();
  if (p.head_dim == 128)
    hipLaunchKernelGGL(rowdot_kernel<128>, grid, dim3(kThreads), 0, s, static_cast<const uint16_t *>(o),
                       static_cast<const uint16_t *>(dout), lse, dvec, lse2, p.total_tokens, p.h_q);
  else
    hipLaunchKernelGGL(rowdot_kernel<64>, grid, dim3(kThreads), 0, s, static_cast<const uint16_t *>(o),
                       static_cast<const uint16_t *>(dout), lse, dvec, lse2, p.total_tokens, p.h_q);
  return launch_status();
}

libra_status launch_dq(const libra_plan_info &h, BwdArgs a, const void *plan_dev, void *dq,
                       libra_cu_record *records, void *stream) {
  const char *pd = static_cast<const char *>(plan_dev);
  a.items = reinterpret_cast<const libra_item *>(pd + h.off_dq_items);
  a.cu_off = reinterpret_cast<const int32_t *>(pd + h.off_dq_cu_off);
  a.plan_sum_dev = reinterpret_cast<const uint64_t *>(pd + offsetof(libra_plan_info, checksum));
  a.plan_sum = h.checksum;
  a.dq = static_cast<uint16_t *>(dq);
  a.records = records;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_hip_error();
  if (h.params.head_dim == 128)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, dim3(h.num_cus), dim3(kDqWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, dim3(h.num_cus), dim3(kDqWaves * 64), 0, s, a);
  return launch_status();
}

}  // namespace libra
