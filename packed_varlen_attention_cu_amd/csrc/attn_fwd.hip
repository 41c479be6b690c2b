// Forward packed block-diagonal causal attention on gfx950 (CDNA4).
//
// One persistent workgroup per CU runs the queue of work items the host
// planner assigned to it (Libra technical review, section 5.4: placement is
// decided on the host, the device only executes it).  A work item is up to
// 384 query columns (positions x heads) of one KV head; each of the twelve
// waves owns 32 query positions of one query head (three waves per SIMD).
//
// Per item the workgroup walks key blocks of 64 from the start of the sample
// holding the item's first row to its last row (the second item of a zigzag
// pair walks them in reverse, so that items started together read the same
// block).  K and V blocks are copied
// straight from HBM into LDS (a ring of kStages buffers, copies running
// kStages - 1 blocks ahead) and read by every wave, so all query heads of a
// GQA group share one copy.  Each wave computes S^T = K Q^T
// with bf16 MFMA (its query columns land one per lane, so row statistics need
// no cross-lane reduction beyond the two 32-lane halves), applies the
// block-diagonal causal mask only on blocks that straddle a sample start or
// the diagonal, skips blocks that are wholly masked for it, and keeps an fp32
// online softmax with c = scale * log2(e):
//   m' = max(m, max_k s c),  P = 2^(s c - m'),  l = l 2^(m - m') + sum P,
//   O^T = O^T 2^(m - m') + V^T P^T.
// P is rounded to bf16 for the PV product and l sums the rounded values, so
// the weights applied to V sum to exactly l.  The epilogue writes O = O^T / l
// (bf16) and LSE = (m + log2 l) ln 2 (natural log, fp32).  The V^T operands
// are read from the row-major V block with transposing LDS reads.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstring>
#include <type_traits>

#include "device_common.h"
#include "libra.h"
#include "plan_layout.h"

namespace libra {

constexpr int kBN = 64;          // keys per block
constexpr int kStages = 4;       // LDS buffers: copies run kStages - 1 blocks ahead

struct FwdArgs {
  const libra_item *items;
  const int32_t *cu_off;
  const uint64_t *plan_sum_dev;   // checksum field of the device copy of the plan
  uint64_t plan_sum;              // checksum of the host plan the launch was made from
  const uint16_t *q, *k, *v;
  const int32_t *cu;
  uint16_t *o;
  float *lse;
  libra_cu_record *records;
  int n_samples, L, h_q, h_kv;
  float scale_log2;
};

// Workgroup shape of the forward kernel: kFwdWaves waves, each owning 32
// query positions of one head, so a workgroup covers the kFwdItemColumns query
// columns of one work item.  Twelve waves run three per SIMD: the kernel fits
// in the 168 registers that leaves, the softmax of some waves overlaps the
// matrix products of others, and each K/V block copied into LDS serves 384
// query columns.
constexpr int kFwdQT = 1;                          // 32-query tiles per wave
constexpr int kFwdWaves = kFwdItemColumns / 32;
static_assert(kFwdWaves % 4 == 0, "whole waves per SIMD");

// Exponent slack of the online softmax: the running maximum m (log2 units)
// is only raised when a block's maximum exceeds it by more than this, so O is
// rescaled rarely; in between, P = 2^(s c - m) stays below 2^kRescaleSlack.
constexpr float kRescaleSlack = 8.0f;

#ifdef LIBRA_COUNT_PAIRS
// Debug build only: the unmasked (query, key, head) triples the forward
// computed, summed over every launch since the last reset (eq. 8 counts
// exactly these).
__device__ unsigned long long g_unmasked_pairs;
#endif

template <int D, int QT, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(NW / 4, NW / 4)))
void attn_fwd_kernel(FwdArgs a) {
  constexpr int QW = 32 * QT;                   // query positions per wave
  constexpr int NS = D / 16;                    // reduction slabs of d
  constexpr int ND = D / 32;                    // 32-row tiles of d in O^T
  constexpr int RS = PadRows<D>::kDirectStride;   // K rows: direct operand reads only
  // V rows take the 152-element stride: the transposing reads then pay one
  // extra cycle in two, but the K and V blocks take 17 + 19 = 36 copy
  // instructions, three for each of the twelve waves, so every wave waits for
  // a fixed count and issues its copies without branches (3-5 % faster than
  // conflict-free 160-element V rows, 37 copies).
  constexpr int RV = PadRows<D>::kStride;
  // kStages buffers, each a K and a V block [kBN][D] in padded rows; block b
  // uses buffer b mod kStages and is copied kStages - 1 blocks ahead.  The V^T
  // operands of O^T = V^T P^T come from transposing reads of the V block.
  constexpr int KBLK = kBN * RS, BUF = KBLK + kBN * RV;
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[kStages * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int half = lane >> 5, col = lane & 31;
  const int w = blockIdx.x;
  const uint64_t t_start = wall_clock64();
  // A device plan that is not a copy of the host plan runs no item.
  const bool plan_ok = as_const(a.plan_sum_dev)[0] == a.plan_sum;
  const int beg = plan_ok ? as_const(a.cu_off)[w] : 0, end = plan_ok ? as_const(a.cu_off)[w + 1] : 0;
  const cptr<int32_t> cu = as_const(a.cu);
  const float sl2 = a.scale_log2;
  const uint32_t kv_base = lds_addr(kv_lds);
  const float NEG_INF = -__builtin_inff();
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  const int dlo = direct_lane_off<RS>(lane);    // K operand reads
  const int tlo = tr_lane_off<RV>(lane);        // V^T operand reads
  const int64_t kv_stride = (int64_t)a.h_kv * D;
  using KVCopy = PairCopy<D, kBN, NW, RS, RV>;
  KVCopy kvcopy;
  kvcopy.init(wave, lane, kv_stride);
  // this wave's copies per block
  const int copies = KVCopy::count(wave);
#ifdef LIBRA_COUNT_PAIRS
  uint32_t counted = 0;   // unmasked (query, key) slots this lane computed
#endif

  // Q operands of the wave's queries of item itq.  Each item's Q is loaded
  // as soon as the previous item's last block is done, before that item's
  // output is normalised and stored, so its latency overlaps the output
  // stores, the next item's set-up and the item-start barrier.
  bf16x8 qop[QT][NS];
  auto load_q = [&](int itq) {
    const libra_item nx = load_item(a.items, itq);
    const int nhx = nx.nheads, hx = nx.head0 + (wave % nhx), subx = wave / nhx;
    const int r0x = nx.row0 + subx * QW, nrx = min(QW, nx.nrows - subx * QW);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int r = qt * 32 + col;
      const bool ok = r < nrx;
      const uint16_t *qp = a.q + ((int64_t)(r0x + r) * a.h_q + hx) * D + 8 * half;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        qop[qt][s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4 *>(qp + 16 * s) : zero_u32x4());
    }
  };

  for (int it = beg; it < end; ++it) {
    const libra_item item = load_item(a.items, it);
    if (it == beg) load_q(it);
    const int row0 = item.row0, nrows = item.nrows, kvh = item.kv_head, nh = item.nheads;
    const int head = item.head0 + (wave % nh);
    const int sub = wave / nh;
    const int wrow0 = row0 + sub * QW;
    const int wrows = min(QW, nrows - sub * QW);

    // Sample start of each query of the wave (scalar loads only).
    int qpos[QT], qss[QT];
    bool qok[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int r = qt * 32 + col;
      qok[qt] = r < wrows;
      qpos[qt] = wrow0 + r;
      qss[qt] = 0;
      if (wrows > 0) {
        int st, en;
        lane_sample(cu, a.n_samples, wrow0, wrow0 + wrows - 1, qpos[qt], st, en);
        if (qok[qt]) qss[qt] = st;
      }
    }
    const int kstart = cu[sample_index(cu, a.n_samples, row0)] & ~(kBN - 1);
    const int kend = row0 + nrows;
    const int nblk = (kend - kstart + kBN - 1) / kBN;
    // Step b's key block: up from the sample start, or (LIBRA_ITEM_REVERSE,
    // the second item of a zigzag pair) down from the item's last block.
    const bool rev = (item.flags & LIBRA_ITEM_REVERSE) != 0;
    auto kblock = [&](int b) { return kstart + (rev ? nblk - 1 - b : b) * kBN; };

    f32x16 oacc[QT][ND];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) oacc[qt][dt] = zero16();
    float m_run[QT], l_run[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      m_run[qt] = NEG_INF;
      l_run[qt] = 0.0f;
    }

    // Queue the K and V blocks at key k0 into LDS buffer buf (no registers);
    // rows past L are masked, so their addresses are clamped to row L - 1.
    auto issue = [&](int k0, int buf) {
      const uint32_t dst = kv_base + buf * 2 * BUF;   // bytes
      kvcopy.issue(dst, dst + 2 * KBLK, wave, a.k + kvh * D, a.v + kvh * D, kv_stride, k0, a.L);
    };

    // One key block.  Once this wave's copies of block b have landed (those of
    // later blocks may still fly) and its reads of block b - 1 have completed,
    // one barrier makes both true for every wave; then block b + kStages - 1
    // is queued into the buffer block b - 1 used, and block b is computed.
    auto block = [&](int b, int buf) {
      const int k0 = kblock(b);
      // The copies of up to kStages - 2 later blocks may still fly.
      const int later = min(kStages - 2, nblk - 1 - b);
      if (KVCopy::kUniform) {
        static_assert((kStages - 2) * KVCopy::kPerWave < 64, "vmcnt range");
        if (kStages > 3 && later >= 2) wait_vmem<2 * KVCopy::kPerWave>();
        else if (later >= 1) wait_vmem<KVCopy::kPerWave>();
        else wait_vmem<0>();
      } else {
        wait_vmem_upto(later * copies);
      }
      wait_lds();
      block_barrier();
      if (b + kStages - 1 < nblk) issue(kblock(b + kStages - 1), buf == 0 ? kStages - 1 : buf - 1);
      const uint16_t *kb = kv_lds + buf * BUF;
      const uint16_t *vb = kb + KBLK;

      bool touch = false, partial = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (qok[qt]) {
          touch |= (k0 <= qpos[qt]) && (k0 + kBN - 1 >= qss[qt]);
          partial |= !((k0 >= qss[qt]) && (k0 + kBN - 1 <= qpos[qt]));
        }
      }
      if (wave_any(touch)) {
        const bool masked = wave_any(partial);
        f32x16 sacc[2][QT];   // [key tile][query tile]: S^T, one query column per lane
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) sacc[kt][qt] = zero16();
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4 *>(kb + dlo + direct_off<RS>(kt, s)));
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) sacc[kt][qt] = mfma32x32x16(ka, qop[qt][s], sacc[kt][qt]);
          }
        }
        // Scheduling groups for the S^T products: two K operand reads first,
        // then one read after each product, so that every product finds its
        // operand already loaded while the next read is in flight.  Left to
        // itself the scheduler issued each read right before its product and
        // waited for it there (2-3.5 % slower).
        {
          constexpr int kReads = 2 * NS, kAhead = 2;
          __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
          for (int i = 0; i < kReads - kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, QT, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, QT * kAhead, 0);
        }
        if (masked) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const int lo = qok[qt] ? qss[qt] : 1, hi = qok[qt] ? qpos[qt] : 0;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = k0 + kt * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
                if (key < lo || key > hi) sacc[kt][qt][r] = NEG_INF;
              }
          }
        }
#ifdef LIBRA_COUNT_PAIRS
        // Unmasked (query, key) slots of this lane's 32 keys of the block.
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if (!qok[qt]) continue;
          if (!masked) {
            counted += 32;
          } else {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int r = 0; r < 16; ++r) counted += sacc[kt][qt][r] != NEG_INF ? 1u : 0u;
          }
        }
#endif
        // Block maximum per query; raise the running maximum only when it is
        // exceeded by more than the slack (then rescale O and l).
        float mxs[QT];
        bool grow = false;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          float mx = NEG_INF;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][qt][r]);
          mxs[qt] = halves_max(mx) * sl2;
          grow |= mxs[qt] > m_run[qt] + kRescaleSlack;
        }
        if (wave_any(grow)) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const float m_new = fmaxf(m_run[qt], mxs[qt]);
            const float alpha = exp2_fast(m_run[qt] - (m_new == NEG_INF ? 0.0f : m_new));
            m_run[qt] = m_new;
            l_run[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[qt][dt][r] *= alpha;
          }
        }
        u32x4 pw[QT][2][2];   // [query tile][key tile][16-key slab]: bf16 P^T operands
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float m_use = m_run[qt] == NEG_INF ? 0.0f : m_run[qt];
          float psum = l_run[qt];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float p0 = exp2_fast(fmaf(sacc[kt][qt][8 * t + 2 * i], sl2, -m_use));
                const float p1 = exp2_fast(fmaf(sacc[kt][qt][8 * t + 2 * i + 1], sl2, -m_use));
                const uint32_t wv = pack_bf16x2(p0, p1);
                psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv), ones, psum, false);
                pw[qt][kt][t][i] = wv;
              }
          l_run[qt] = psum;
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const bf16x8 va = lds_tr_operand(vb + tlo + tr_off<RV>(kt * 32 + 16 * t, dt * 32, 0),
                                               vb + tlo + tr_off<RV>(kt * 32 + 16 * t, dt * 32, 1));
#pragma unroll
              for (int qt = 0; qt < QT; ++qt)
                oacc[qt][dt] = mfma32x32x16(va, as_bf16x8(pw[qt][kt][t]), oacc[qt][dt]);
            }
      }
    };

    wait_lds();
    block_barrier();                // the previous item's reads of every buffer are done
    // This item's Q and the previous item's output stores have been in flight
    // since the previous item's last block: one full wait for them here,
    // before the first copies, costs little and tells the compiler that the
    // Q registers are loaded (it cannot see that the per-block copy waits
    // cover them, and would otherwise wait for every copy at every block).
    wait_vmem<0>();
#pragma unroll
    for (int b = 0; b < kStages - 1; ++b)
      if (b < nblk) issue(kblock(b), b);
    for (int b = 0, buf = 0; b < nblk; ++b, buf = buf == kStages - 1 ? 0 : buf + 1) block(b, buf);
    if (it + 1 < end) load_q(it + 1);

#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float lt = halves_sum(l_run[qt]);
      const float inv = 1.0f / lt;
      if (qok[qt]) {
        uint16_t *op = a.o + ((int64_t)qpos[qt] * a.h_q + head) * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x2 pk;
            pk[0] = pack_bf16x2(oacc[qt][dt][4 * c] * inv, oacc[qt][dt][4 * c + 1] * inv);
            pk[1] = pack_bf16x2(oacc[qt][dt][4 * c + 2] * inv, oacc[qt][dt][4 * c + 3] * inv);
            *reinterpret_cast<u32x2 *>(op + dt * 32 + 8 * c + 4 * half) = pk;
          }
        if (half == 0) a.lse[(int64_t)head * a.L + qpos[qt]] = (m_run[qt] + __log2f(lt)) * kLn2;
      }
    }
  }

#ifdef LIBRA_COUNT_PAIRS
  {
    uint64_t wave_sum = counted;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wave_sum += __shfl_xor(wave_sum, off);
    if (lane == 0) atomicAdd(&g_unmasked_pairs, (unsigned long long)wave_sum);
  }
#endif
  __syncthreads();
  if (a.records != nullptr && tid == 0) {
    libra_cu_record rec;
    rec.hw_id = hw_id_reg();
    rec.xcc_id = xcc_id_reg();
    rec.n_items = (uint32_t)(end - beg);
    rec.flags = plan_ok ? 0u : LIBRA_RECORD_PLAN_MISMATCH;
    rec.t_start = t_start;
    rec.t_end = wall_clock64();
    a.records[w] = rec;
  }
}

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

namespace {
thread_local hipError_t g_last_hip_error = hipSuccess;
}

void clear_hip_error() { (void)hipGetLastError(); }

libra_status launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return LIBRA_OK;
  g_last_hip_error = e;
  return LIBRA_EHIP;
}

}  // namespace libra

using namespace libra;

namespace {

libra_status check_header(const void *plan, libra_plan_info *h) {
  if (plan_validate(plan, h) != LIBRA_OK) return LIBRA_EINVAL;
  if (h->params.head_dim != 64 && h->params.head_dim != 128) return LIBRA_EUNSUPPORTED;
  return LIBRA_OK;
}

libra_status check_fwd(const libra_plan_info &h, const void *plan_dev, const void *q, const void *k,
                       const void *v, const int32_t *cu_dev, const void *o, const float *lse, float scale,
                       const void *records) {
  const libra_plan_params &p = h.params;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return LIBRA_EINVAL;
  if (p.total_tokens == 0) return LIBRA_OK;
  if (!plan_dev || !q || !k || !v || !cu_dev || !o || !lse) return LIBRA_EINVAL;
  if (misaligned(plan_dev, 16) || misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) ||
      misaligned(o, 16) || misaligned(lse, 4) || misaligned(cu_dev, 4) || misaligned(records, 16))
    return LIBRA_EINVAL;
  return LIBRA_OK;
}

libra_status launch_fwd(const libra_plan_info &h, const void *plan_dev, const void *q, const void *k,
                        const void *v, const int32_t *cu_dev, void *o, float *lse, float scale,
                        libra_cu_record *records, void *stream) {
  const libra_plan_params &p = h.params;
  FwdArgs a;
  const char *pd = static_cast<const char *>(plan_dev);
  a.items = reinterpret_cast<const libra_item *>(pd + h.off_items);
  a.cu_off = reinterpret_cast<const int32_t *>(pd + h.off_cu_off);
  a.plan_sum_dev = reinterpret_cast<const uint64_t *>(pd + offsetof(libra_plan_info, checksum));
  a.plan_sum = h.checksum;
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.cu = cu_dev;
  a.o = static_cast<uint16_t *>(o);
  a.lse = lse;
  a.records = records;
  a.n_samples = p.num_samples;
  a.L = p.total_tokens;
  a.h_q = p.h_q;
  a.h_kv = p.h_kv;
  a.scale_log2 = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_hip_error();
  if (p.head_dim == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, kFwdQT, kFwdWaves>), dim3(h.num_cus), dim3(kFwdWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, kFwdQT, kFwdWaves>), dim3(h.num_cus), dim3(kFwdWaves * 64), 0, s, a);
  return launch_status();
}

}  // namespace

extern "C" libra_status libra_attn_fwd(const void *plan, const void *plan_dev, const void *q,
                                       const void *k, const void *v, const int32_t *cu_dev, void *o,
                                       float *lse, float softmax_scale, libra_cu_record *records,
                                       void *stream) {
  libra_plan_info h;
  libra_status st = check_header(plan, &h);
  if (st == LIBRA_OK) st = check_fwd(h, plan_dev, q, k, v, cu_dev, o, lse, softmax_scale, records);
  if (st != LIBRA_OK || h.params.total_tokens == 0) return st;
  return launch_fwd(h, plan_dev, q, k, v, cu_dev, o, lse, softmax_scale, records, stream);
}

extern "C" const char *libra_last_hip_error(void) {
  const hipError_t e = g_last_hip_error;
  return e == hipSuccess ? "" : hipGetErrorName(e);
}

extern "C" libra_status libra_device_clock_khz(int32_t *khz) {
  if (!khz) return LIBRA_EINVAL;
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LIBRA_EHIP;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return LIBRA_EHIP;
  *khz = v;
  return LIBRA_OK;
}

#ifdef LIBRA_COUNT_PAIRS
extern "C" libra_status libra_debug_unmasked_pairs(uint64_t *count) {
  if (!count) return LIBRA_EINVAL;
  unsigned long long v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_unmasked_pairs), sizeof v) != hipSuccess) return LIBRA_EHIP;
  *count = v;
  return LIBRA_OK;
}

extern "C" libra_status libra_debug_reset_unmasked_pairs(void) {
  const unsigned long long zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_unmasked_pairs), &zero, sizeof zero) != hipSuccess) return LIBRA_EHIP;
  return LIBRA_OK;
}
#endif
