// Backward packed block-diagonal causal attention on gfx950 (CDNA4).
//
// Gradients of O = softmax(scale Q K^T + mask) V for the block-diagonal
// causal mask (Libra technical review, section 1 "Sequence packing"; the
// pages leave the backward to the attention kernel and state only that it
// reuses the forward placement with reversed transfers, Libra paper section
// 4.3.3).  With P = exp(scale S - LSE) recomputed from the forward's LSE:
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Work is split into two deterministic persistent passes (no atomics):
//   * key-major dK/dV: an item is 192 keys of one KV head; pairs of waves own
//     32 keys each and walk every query block of every query head of the group
//     that can see them, accumulating dK^T and dV^T in registers (GQA heads
//     are summed in place);
//   * query-major dQ: items cut from the forward's SH-Tiles (256 query
//     columns each, the forward's are 384) and placed like them, each wave
//     owning 32 query positions of one head and walking its key blocks.
// Both passes avoid atomics: summing dQ over key items with fp32 atomic adds
// would move about 40 times the bytes of an fp32 dQ, at a quarter of the
// store rate.
// Both walk their blocks in the order the planner's zigzag pairs ask for
// (LIBRA_ITEM_REVERSE), so that items started together share L2 lines.
// This source holds the dK/dV pass and the C ABI of the backward; the row-dot
// phase and the dQ pass are compiled from attn_bwd_dq.hip.
// Operand blocks are copied straight from HBM into LDS; operands that need
// the transposed layout (Q^T, dO^T, K^T) come from transposing LDS reads of
// the row-major blocks.  A first phase computes D = rowsum(dO * O) (fp32)
// from the forward's bf16 O and the forward's LSE in log2 units.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "bwd_common.h"

namespace libra {

namespace {

// ----------------------------------------------------------------- dK / dV pass
// Twelve waves, three per SIMD.  The 192 keys of an item are split into six
// groups of 32; each group has a P wave (waves 0-5: S = Q K^T, P, dV^T +=
// dO^T P) and a dS wave (waves 6-11: dP = dO V^T, dS = P * (dP - D),
// dK^T += Q^T dS).  The P wave publishes its bf16 P through LDS tile by
// tile, with a flag its dS wave waits for (no workgroup barrier within a
// step), so the matrix products of some waves of a SIMD overlap the
// element-wise work of others.  Only the P wave applies the
// block-diagonal mask: masked P is 0, hence masked dS is 0 too.  Three waves
// per SIMD leave each 168 registers, which the kernel fits in; the larger
// item shares each Q and dO block among 192 keys instead of 128.
//
// Per query block of kQB rows and one head, LDS holds Q and dO (row-major:
// A operands of S and dP directly, and of dK^T and dV^T through transposing
// reads) and the block's LSE * log2(e) and D values.  kStages such buffers
// rotate: after one barrier the copies for the step kStages - 1 ahead are
// queued into the buffer the previous step used, and the current one is
// computed while they fly.  Blocks use padded rows (PadRows).
constexpr int kDkdvGroups = kKvItemKeys / 32;   // key groups of 32
constexpr int kDkdvWaves = 2 * kDkdvGroups;      // a P wave and a dS wave per group
// Bound of a dS wave's wait for its P wave's tile: polls 64 cycles apart,
// about 4M cycles in all, against a few thousand when nothing is wrong.
constexpr int kPWaitPolls = 1 << 16;
static_assert(kDkdvWaves % 4 == 0, "whole waves per SIMD");

// Q blocks take 152-element rows (D = 128; 72 at D = 64) and dO blocks 168
// (72): both are read directly and through transposing reads, and 168 has
// the same conflict profile as 152.  A Q and a dO block then fill 19 + 21 =
// 40 copy instructions; with the eight row-vector copies (LSE, D) that makes
// four per wave for each of the twelve waves at D = 128.
template <int D>
struct DkdvLds {
  static constexpr int kRQ = PadRows<D>::kStride;          // Q row stride (elements)
  static constexpr int kRO = D == 128 ? 168 : PadRows<D>::kStride;   // dO row stride
  static constexpr int kRowQ = kQB * kRQ, kRowO = kQB * kRO;   // elements of one padded block
  static constexpr int kBuf = kRowQ + kRowO + 2 * kQB * 2;  // Q, dO + LSE and D (fp32), in uint16 units
  static constexpr int kP = kDkdvGroups * 32 * kQB;       // bf16 P of every key group
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kDkdvWaves * 64, kDkdvWaves * 64),
                         amdgpu_waves_per_eu(kDkdvWaves / 4, kDkdvWaves / 4)))
void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = kDkdvWaves;
  constexpr int NS = D / 16, ND = D / 32;
  static_assert(2 * kQB <= NW * 16, "LSE and D copies: 16 values per wave");
  constexpr int RQ = DkdvLds<D>::kRQ, RO = DkdvLds<D>::kRO;
  constexpr int ROWQ = DkdvLds<D>::kRowQ, ROWO = DkdvLds<D>::kRowO;
  // kStages buffers of a step's Q, dO, LSE and D; step i uses buffer i mod kStages.
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kStages * DkdvLds<D>::kBuf];
  __shared__ __attribute__((aligned(16))) uint16_t p_lds[DkdvLds<D>::kP];
  // Step at which each key group's P of query tile t was last published, and
  // whether any wave's bounded wait for it ran out.
  __shared__ int p_ready[kDkdvGroups][2];
  __shared__ int wait_expired;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int half = lane >> 5, col = lane & 31;
  const int kg = wave % kDkdvGroups;               // key group
  const int w = blockIdx.x;
  const uint64_t t_start = wall_clock64();
  // A device plan that is not a copy of the host plan runs no item.
  const bool plan_ok = as_const(a.plan_sum_dev)[0] == a.plan_sum;
  const int beg = plan_ok ? as_const(a.cu_off)[w] : 0, end = plan_ok ? as_const(a.cu_off)[w + 1] : 0;
  const cptr<int32_t> cu = as_const(a.cu);
  const float c = a.scale_log2;
  const uint32_t q_base = lds_addr(q_lds);
  u32x4 *p_mine = reinterpret_cast<u32x4 *>(p_lds + kg * 32 * kQB) + lane;   // [4 slabs][64 lanes]
  const int64_t q_stride = (int64_t)a.h_q * D;
  using QOCopy = PairCopy<D, kQB, NW, RQ, RO>;
  QOCopy qocopy;
  qocopy.init(wave, lane, q_stride);
  // The last kRowVec waves copy 16 LSE / D values each; they are the waves
  // with one Q / dO copy fewer whenever kUniformStep holds.
  constexpr int kRowVec = 2 * kQB / 16;
  constexpr bool kUniformStep = QOCopy::NI % NW == NW - kRowVec;
  constexpr int kStepCopies = QOCopy::NI / NW + 1;
  const int rv = wave - (NW - kRowVec);            // row-vector copy of this wave, if >= 0
  const bool rowvec = rv >= 0;
  const int copies = QOCopy::count(wave) + (rowvec ? 1 : 0);   // this wave's copies per step

  if (tid < 2 * kDkdvGroups) (&p_ready[0][0])[tid] = -1;   // visible after the first item's barrier
  if (tid == 0) wait_expired = 0;
  int step_no = 0;   // steps run so far in this workgroup (the same count in every wave)
  bool expired = false;   // one of this wave's waits for its P wave ran out
  // The two roles are separate instantiations, so each allocates registers
  // for its own path only; both pass the same barriers.
  auto run = [&](auto role) {
    constexpr bool pwave = decltype(role)::value;
    // Direct reads: Q (P wave) or dO (dS wave); transposing reads: the other.
    constexpr int RA = pwave ? RQ : RO, RT = pwave ? RO : RQ;
    const int dlo = direct_lane_off<RA>(lane);
    const int tlo = tr_lane_off<RT>(lane);
    for (int it = beg; it < end; ++it) {
      const libra_item item = load_item(a.items, it);
      const int row0 = item.row0, nrows = item.nrows, kvh = item.kv_head;
      const int kloc = kg * 32 + col;
      const bool kok = kloc < nrows;
      const int key = row0 + kloc;
      // End of each key's sample, queries [key, kend) (scalar loads only).
      int kend = 0;
      if (kg * 32 < nrows) {
        int st, en;
        lane_sample(cu, a.n_samples, row0 + kg * 32, row0 + min(nrows, kg * 32 + 32) - 1, key, st, en);
        if (kok) kend = en;
      }
      // B operand of this wave's first product: K (P wave) or V (dS wave),
      // loaded once the previous item's buffers are free.
      bf16x8 bop[NS];
      const int qstart = row0 & ~(kQB - 1);
      const int qend = cu[sample_index(cu, a.n_samples, row0 + nrows - 1) + 1];
      const int nqb = (qend - qstart + kQB - 1) / kQB;
      const int nsteps = nqb * item.nheads;

      f32x16 acc[ND];   // dV^T (P wave) or dK^T (dS wave), one key column per lane
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] = zero16();

      // Queue the copies of the step at (head h, query block q0); rows past L
      // are masked, so their addresses are clamped to row L - 1.
      auto issue = [&](int h, int q0, int buf) {
        const uint32_t dst = q_base + buf * 2 * DkdvLds<D>::kBuf;   // bytes
        qocopy.issue(dst, dst + 2 * ROWQ, wave, a.q + h * D, a.dout + h * D, q_stride, q0, a.L);   // byte offsets
        // LSE * log2(e) then D of the block's queries: lanes 0..15 of the last
        // kRowVec waves copy 16 values each.
        if (rowvec && lane < 16) {
          const int e = rv * 16 + lane;               // 0 .. 2 kQB - 1
          const int qq = min(q0 + (e & (kQB - 1)), a.L - 1);
          const float *src = (e < kQB ? a.lse2 : a.dvec) + (int64_t)h * a.L + qq;
          lds_dma4(src, dst + 2 * (ROWQ + ROWO) + rv * 64);
        }
      };

      // Steps run over (query block, head), heads inner, query blocks from
      // the sample's last one down, or (LIBRA_ITEM_REVERSE) from the item's
      // first one up.  The planner pairs a chunk walking down with one
      // walking up so that items started together on one XCD read the same
      // Q / dO rows at every step.  (ch, cq0) is the step to compute next,
      // (nh, nq0) the next one to copy.
      const bool up = (item.flags & LIBRA_ITEM_REVERSE) != 0;
      const int qfirst = up ? qstart : qstart + (nqb - 1) * kQB;
      const int qstep = up ? kQB : -kQB;
      int ch = item.head0, cq0 = qfirst, nh = item.head0, nq0 = qfirst;
      auto advance = [&](int &hh, int &qq) {
        if (++hh == item.head0 + item.nheads) {
          hh = item.head0;
          qq += qstep;
        }
      };
      auto step = [&](int i, int buf) {
        const uint16_t *bq = q_lds + buf * DkdvLds<D>::kBuf;
        const int q0 = cq0;
        advance(ch, cq0);
        // step i landed; step i + 1 may fly
        if (kUniformStep) {
          if (i + 1 < nsteps) wait_vmem<kStepCopies>(); else wait_vmem<0>();
        } else {
          wait_vmem_upto(i + 1 < nsteps ? copies : 0);
        }
        wait_lds();                   // own LDS accesses of step i - 1 done
        block_barrier();
        if (i + kStages - 1 < nsteps) {
          issue(nh, nq0, buf == 0 ? kStages - 1 : buf - 1);
          advance(nh, nq0);
        }
        const bool touch = kok && (q0 + kQB - 1 >= key) && (q0 < kend);
        const bool full = !kok || ((key <= q0) && (q0 + kQB - 1 < kend));
        const bool act = wave_any(touch);     // identical for the two waves of a key group
        const bool masked = wave_any(!full);
        const uint16_t *q_l = bq, *do_l = bq + ROWQ;
        const float *lse_l = reinterpret_cast<const float *>(bq + ROWQ + ROWO);
        const float *dd_l = lse_l + kQB;

        // First product of query tile qt: S (P wave, A = Q) or dP (dS wave, A = dO).
        auto first = [&](int qt) {
          const uint16_t *a_l = (pwave ? q_l : do_l) + dlo;
          f32x16 out = zero16();
#pragma unroll
          for (int s = 0; s < NS; ++s)
            out = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4 *>(a_l + direct_off<RA>(qt, s))),
                               bop[s], out);
          return out;
        };
        // Second product of query tile qt: acc += (dO or Q)^T x w, transposed reads.
        auto second = [&](int qt, const u32x4 (&wv)[2]) {
          const uint16_t *t_l = (pwave ? do_l : q_l) + tlo;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
              const bf16x8 av = lds_tr_operand(t_l + tr_off<RT>(qt * 32 + 16 * t, dt * 32, 0),
                                               t_l + tr_off<RT>(qt * 32 + 16 * t, dt * 32, 1));
              acc[dt] = mfma32x32x16(av, as_bf16x8(wv[t]), acc[dt]);
            }
        };
        // P of query tile qt, published through LDS for the dS wave.
        auto p_tile = [&](int qt, u32x4 (&pw)[2]) {
          f32x16 sacc = first(qt);
          if (masked) {             // rare: blocks on a sample start or the diagonal
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qq = q0 + qt * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
              if (!(kok && key <= qq && qq < kend)) sacc[r] = -__builtin_inff();
            }
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int ql = qt * 32 + 16 * t + 8 * half;   // first of 8 consecutive queries
            const float4 l0 = *reinterpret_cast<const float4 *>(lse_l + ql);
            const float4 l1 = *reinterpret_cast<const float4 *>(lse_l + ql + 4);
            const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = exp2_fast(fmaf(sacc[8 * t + 2 * e], c, -lv[2 * e]));   // masked: 0
              const float p1 = exp2_fast(fmaf(sacc[8 * t + 2 * e + 1], c, -lv[2 * e + 1]));
              pw[t][e] = pack_bf16x2(p0, p1);
            }
            p_mine[(qt * 2 + t) * 64] = pw[t];
          }
        };
        // dS of query tile qt from this wave's dP and the P wave's P.
        auto ds_tile = [&](int qt, const f32x16 &pacc, u32x4 (&dsw)[2]) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int ql = qt * 32 + 16 * t + 8 * half;
            const float4 d0 = *reinterpret_cast<const float4 *>(dd_l + ql);
            const float4 d1 = *reinterpret_cast<const float4 *>(dd_l + ql + 4);
            const float dv8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            const u32x4 pv = p_mine[(qt * 2 + t) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float ds0 = bf16_lo(pv[e]) * (pacc[8 * t + 2 * e] - dv8[2 * e]);
              const float ds1 = bf16_hi(pv[e]) * (pacc[8 * t + 2 * e + 1] - dv8[2 * e + 1]);
              dsw[t][e] = pack_bf16x2(ds0, ds1);
            }
          }
        };

        // Within a step the dS wave of a key group waits only for its own P
        // wave, not for the workgroup: P of query tile t is published with a
        // flag in LDS (a release store after the P writes; an acquire load
        // before the P reads), so the twelve waves drift freely between the
        // step barriers:
        //   P wave:  S0 P0 (publish) S1 P1 (publish) dV0 dV1
        //   dS wave: dP0 dP1 (wait P0) dS0 dK0 (wait P1) dS1 dK1
        // Both waves of a group skip a step together (act is the same for
        // them).  The wait is bounded so that no defect can hang the
        // workgroup; running out is reported in the record.
        const int stamp = step_no;
        if constexpr (pwave) {
          u32x4 pw0[2], pw1[2];
          if (act) {
            p_tile(0, pw0);
            __hip_atomic_store(&p_ready[kg][0], stamp, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            p_tile(1, pw1);
            __hip_atomic_store(&p_ready[kg][1], stamp, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            second(0, pw0);
            second(1, pw1);
          }
        } else {
          auto wait_p = [&](int t) {
            int seen = -1;
            for (int n = 0; n < kPWaitPolls; ++n) {
              seen = __hip_atomic_load(&p_ready[kg][t], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
              if (seen >= stamp) break;
              __builtin_amdgcn_s_sleep(1);
            }
            expired |= seen < stamp;
          };
          if (act) {
            const f32x16 pacc0 = first(0), pacc1 = first(1);
            u32x4 dsw[2];
            wait_p(0);
            ds_tile(0, pacc0, dsw);
            second(0, dsw);
            wait_p(1);
            ds_tile(1, pacc1, dsw);
            second(1, dsw);
          }
        }
        ++step_no;
      };

      // The previous item's dK / dV stores may still fly while this item's
      // loads and first copies are issued; one wait then covers all of them
      // (and tells the compiler that the operand registers are loaded).
      wait_lds();
      block_barrier();              // the previous item's reads of every buffer and of P are done
      {
        const uint16_t *src = (pwave ? a.k : a.v) + ((int64_t)key * a.h_kv + kvh) * D + 8 * half;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          bop[s] = as_bf16x8(kok ? *reinterpret_cast<const u32x4 *>(src + 16 * s) : zero_u32x4());
      }
#pragma unroll
      for (int i = 0; i < kStages - 1; ++i)
        if (i < nsteps) {
          issue(nh, nq0, i);
          advance(nh, nq0);
        }
      wait_vmem<0>();
      for (int i = 0, buf = 0; i < nsteps; ++i, buf = buf == kStages - 1 ? 0 : buf + 1) step(i, buf);

      if (kok) {
        uint16_t *dst = (pwave ? a.dv : a.dk) + ((int64_t)key * a.h_kv + kvh) * D;
        const float sc = pwave ? 1.0f : a.scale;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            u32x2 pk;
            pk[0] = pack_bf16x2(acc[dt][4 * cc] * sc, acc[dt][4 * cc + 1] * sc);
            pk[1] = pack_bf16x2(acc[dt][4 * cc + 2] * sc, acc[dt][4 * cc + 3] * sc);
            *reinterpret_cast<u32x2 *>(dst + dt * 32 + 8 * cc + 4 * half) = pk;
          }
      }
    }
  };
  if (wave < kDkdvGroups) run(std::true_type{});
  else run(std::false_type{});
  if (expired) wait_expired = 1;
  __syncthreads();
  if (a.records != nullptr && tid == 0)
    write_record(a, w, end - beg, t_start, plan_ok, wait_expired ? LIBRA_RECORD_WAIT_EXPIRED : 0u);
}

libra_status check_header(const void *plan, libra_plan_info *h) {
  if (plan_validate(plan, h) != LIBRA_OK) return LIBRA_EINVAL;
  if (h->params.head_dim != 64 && h->params.head_dim != 128) return LIBRA_EUNSUPPORTED;
  return LIBRA_OK;
}

bool any_null(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (!p) return true;
  return false;
}

bool any_misaligned(std::initializer_list<const void *> ps, uintptr_t a) {
  for (const void *p : ps)
    if (misaligned(p, a)) return true;
  return false;
}

libra_status check_workspace(const libra_plan_info &h, const void *ws, size_t bytes) {
  if (!ws || misaligned(ws, 256)) return LIBRA_EINVAL;
  return bytes < bwd_layout(h.params).total ? LIBRA_ESIZE : LIBRA_OK;
}

libra_status check_prepare(const libra_plan_info &h, const void *o, const void *dout, const float *lse,
                           const void *ws, size_t bytes) {
  if (h.params.total_tokens == 0) return LIBRA_OK;
  if (any_null({o, dout, lse}) || any_misaligned({o, dout}, 16) || misaligned(lse, 4)) return LIBRA_EINVAL;
  return check_workspace(h, ws, bytes);
}

libra_status check_pass(const libra_plan_info &h, const void *plan_dev,
                        std::initializer_list<const void *> tensors, const float *lse,
                        const int32_t *cu_dev, float scale, const void *ws, size_t bytes,
                        const void *records) {
  if (!(scale > 0.0f) || !std::isfinite(scale)) return LIBRA_EINVAL;
  if (h.params.total_tokens == 0) return LIBRA_OK;
  if (!plan_dev || !lse || !cu_dev || any_null(tensors)) return LIBRA_EINVAL;
  if (misaligned(plan_dev, 16) || any_misaligned(tensors, 16) || misaligned(lse, 4) ||
      misaligned(cu_dev, 4) || misaligned(records, 16))
    return LIBRA_EINVAL;
  return check_workspace(h, ws, bytes);
}

BwdArgs make_args(const libra_plan_info &h, const void *q, const void *k, const void *v,
                  const void *dout, const float *lse, const int32_t *cu_dev, const void *ws,
                  float scale) {
  const libra_plan_params &p = h.params;
  const BwdLayout lay = bwd_layout(p);
  const char *w = static_cast<const char *>(ws);
  BwdArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.dout = static_cast<const uint16_t *>(dout);
  a.lse = lse;
  a.dvec = reinterpret_cast<const float *>(w + lay.dvec);
  a.lse2 = reinterpret_cast<const float *>(w + lay.lse2);
  a.cu = cu_dev;
  a.n_samples = p.num_samples;
  a.L = p.total_tokens;
  a.h_q = p.h_q;
  a.h_kv = p.h_kv;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  return a;
}

libra_status launch_dkdv(const libra_plan_info &h, BwdArgs a, const void *plan_dev, void *dk, void *dv,
                         libra_cu_record *records, void *stream) {
  const char *pd = static_cast<const char *>(plan_dev);
  a.items = reinterpret_cast<const libra_item *>(pd + h.off_kv_items);
  a.cu_off = reinterpret_cast<const int32_t *>(pd + h.off_kv_cu_off);
  a.plan_sum_dev = reinterpret_cast<const uint64_t *>(pd + offsetof(libra_plan_info, checksum));
  a.plan_sum = h.checksum;
  a.dk = static_cast<uint16_t *>(dk);
  a.dv = static_cast<uint16_t *>(dv);
  a.records = records;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_hip_error();
  if (h.params.head_dim == 128)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, dim3(h.num_cus), dim3(kDkdvWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, dim3(h.num_cus), dim3(kDkdvWaves * 64), 0, s, a);
  return launch_status();
}

}  // namespace
}  // namespace libra

using namespace libra;

extern "C" libra_status libra_attn_bwd_workspace(const void *plan, size_t *bytes) {
  libra_plan_info h;
  if (!bytes || plan_header(plan, &h) != LIBRA_OK) return LIBRA_EINVAL;
  *bytes = bwd_layout(h.params).total;
  return LIBRA_OK;
}

extern "C" libra_status libra_attn_bwd_prepare(const void *plan, const void *o, const void *dout,
                                               const float *lse, void *workspace, size_t workspace_bytes,
                                               void *stream) {
  libra_plan_info h;
  libra_status st = check_header(plan, &h);
  if (st == LIBRA_OK) st = check_prepare(h, o, dout, lse, workspace, workspace_bytes);
  if (st != LIBRA_OK || h.params.total_tokens == 0) return st;
  return launch_prepare(h, o, dout, lse, workspace, stream);
}

extern "C" libra_status libra_attn_bwd_dkdv(const void *plan, const void *plan_dev, const void *q,
                                            const void *k, const void *v, const void *dout,
                                            const float *lse, const int32_t *cu_dev, void *dk, void *dv,
                                            float softmax_scale, const void *workspace,
                                            size_t workspace_bytes, libra_cu_record *records,
                                            void *stream) {
  libra_plan_info h;
  libra_status st = check_header(plan, &h);
  if (st == LIBRA_OK)
    st = check_pass(h, plan_dev, {q, k, v, dout, dk, dv}, lse, cu_dev, softmax_scale, workspace,
                    workspace_bytes, records);
  if (st != LIBRA_OK || h.params.total_tokens == 0) return st;
  return launch_dkdv(h, make_args(h, q, k, v, dout, lse, cu_dev, workspace, softmax_scale), plan_dev,
                     dk, dv, records, stream);
}

extern "C" libra_status libra_attn_bwd_dq(const void *plan, const void *plan_dev, const void *q,
                                          const void *k, const void *v, const void *dout, const float *lse,
                                          const int32_t *cu_dev, void *dq, float softmax_scale,
                                          const void *workspace, size_t workspace_bytes,
                                          libra_cu_record *records, void *stream) {
  libra_plan_info h;
  libra_status st = check_header(plan, &h);
  if (st == LIBRA_OK)
    st = check_pass(h, plan_dev, {q, k, v, dout, dq}, lse, cu_dev, softmax_scale, workspace,
                    workspace_bytes, records);
  if (st != LIBRA_OK || h.params.total_tokens == 0) return st;
  return launch_dq(h, make_args(h, q, k, v, dout, lse, cu_dev, workspace, softmax_scale), plan_dev,
                   dq, records, stream);
}

extern "C" libra_status libra_attn_bwd(const void *plan, const void *plan_dev, const void *q,
                                       const void *k, const void *v, const void *o, const void *dout,
                                       const float *lse, const int32_t *cu_dev, void *dq, void *dk,
                                       void *dv, float softmax_scale, void *workspace,
                                       size_t workspace_bytes, libra_cu_record *records, void *stream) {
  libra_plan_info h;
  libra_status st = check_header(plan, &h);
  if (st == LIBRA_OK) st = check_prepare(h, o, dout, lse, workspace, workspace_bytes);
  if (st == LIBRA_OK)
    st = check_pass(h, plan_dev, {q, k, v, dout, dq, dk, dv}, lse, cu_dev, softmax_scale, workspace,
                    workspace_bytes, records);
  if (st != LIBRA_OK || h.params.total_tokens == 0) return st;
  if ((st = launch_prepare(h, o, dout, lse, workspace, stream)) != LIBRA_OK) return st;
  const BwdArgs a = make_args(h, q, k, v, dout, lse, cu_dev, workspace, softmax_scale);
  if ((st = launch_dkdv(h, a, plan_dev, dk, dv, records, stream)) != LIBRA_OK) return st;
  return launch_dq(h, a, plan_dev, dq, records ? records + h.num_cus : nullptr, stream);
}

// ----------------------------------------------------------------- backward without allocation
// The backward's only scratch memory is its workspace (D and LSE * log2(e),
// fp32 [h_q][L] each).  For callers that cannot allocate, it lives in this
// file-scope device array, one copy per GPU the library runs on, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device array: its device address comes from hipGetSymbolAddress, taken
// once per device (with that device current) and kept in scratch_dev.
namespace {

static __device__ __align__(256) unsigned char scratch[LIBRA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_dev[kMaxDevices];   // device address of `scratch` on each device, once taken

// The device address of the current device's copy of `scratch`.
libra_status scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LIBRA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return LIBRA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_dev[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return LIBRA_EHIP;
    }
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return LIBRA_OK;
}

}  // namespace

extern "C" libra_status libra_attn_bwd_noalloc(const void *plan, const void *plan_dev, const void *q,
                                               const void *k, const void *v, const void *o, const void *dout,
                                               const float *lse, const int32_t *cu_dev, void *dq, void *dk,
                                               void *dv, float softmax_scale, libra_cu_record *records,
                                               void *stream) {
  libra_plan_info h;
  libra_status st = check_header(plan, &h);
  if (st != LIBRA_OK) return st;
  const size_t need = bwd_layout(h.params).total;
  if (need > (size_t)LIBRA_NOALLOC_SCRATCH_BYTES) return LIBRA_ESIZE;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return LIBRA_EINVAL;
  if (h.params.total_tokens == 0) return LIBRA_OK;
  // The checks of libra_attn_bwd, with a stand-in workspace address (the
  // array's address is only taken once the arguments are known to be good).
  const void *probe = reinterpret_cast<const void *>(uintptr_t(256));
  st = check_prepare(h, o, dout, lse, probe, need);
  if (st == LIBRA_OK)
    st = check_pass(h, plan_dev, {q, k, v, dout, dq, dk, dv}, lse, cu_dev, softmax_scale, probe, need, records);
  if (st != LIBRA_OK) return st;
  void *ws = nullptr;
  if ((st = scratch_address(&ws)) != LIBRA_OK) return st;
  if ((st = launch_prepare(h, o, dout, lse, ws, stream)) != LIBRA_OK) return st;
  const BwdArgs a = make_args(h, q, k, v, dout, lse, cu_dev, ws, softmax_scale);
  if ((st = launch_dkdv(h, a, plan_dev, dk, dv, records, stream)) != LIBRA_OK) return st;
  return launch_dq(h, a, plan_dev, dq, records ? records + h.num_cus : nullptr, stream);
}
