// Declarations shared by the two backward sources: the pass arguments, the
// per-workgroup record, the workspace layout, and the host launchers of the
// row-dot and dQ kernels, which live in their own source so that they can be
// compiled with the instruction scheduling that suits them.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "libra.h"
#include "plan_layout.h"

namespace libra {

constexpr int kThreads = 256;   // row-dot kernel
constexpr int kQB = kKvQueryBlock;   // query rows per block in the dK/dV pass
constexpr int kStages = 3;   // LDS buffers: copies run kStages - 1 blocks ahead
constexpr int kKB = 64;      // key rows per block in the dQ pass

inline int64_t round_up64(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct BwdArgs {
  const libra_item *items;     // dK/dV: key-major queue; dQ: forward queue
  const int32_t *cu_off;
  const uint64_t *plan_sum_dev;   // checksum field of the device copy of the plan
  uint64_t plan_sum;              // checksum of the host plan the launch was made from
  const uint16_t *q, *k, *v, *dout;
  const float *lse, *dvec, *lse2;  // [h_q][L]: LSE, D = rowsum(dO * O), LSE * log2(e)
  const int32_t *cu;
  uint16_t *dq, *dk, *dv;
  libra_cu_record *records;
  int n_samples, L, h_q, h_kv;
  float scale, scale_log2;
};

__device__ __forceinline__ void write_record(const BwdArgs &a, int w, int n, uint64_t t0, bool plan_ok,
                                             uint32_t flags = 0u) {
  libra_cu_record rec;
  rec.hw_id = hw_id_reg();
  rec.xcc_id = xcc_id_reg();
  rec.n_items = (uint32_t)n;
  rec.flags = (plan_ok ? 0u : LIBRA_RECORD_PLAN_MISMATCH) | flags;
  rec.t_start = t0;
  rec.t_end = wall_clock64();
  a.records[w] = rec;
}

struct BwdLayout {
  size_t dvec, lse2, total;
};

inline BwdLayout bwd_layout(const libra_plan_params &p) {
  BwdLayout l;
  const size_t rows = (size_t)round_up64((int64_t)p.h_q * p.total_tokens * 4, 256);
  l.dvec = 0;
  l.lse2 = rows;
  l.total = 2 * rows;
  return l;
}

// Defined in attn_bwd_dq.hip.
libra_status launch_prepare(const libra_plan_info &h, const void *o, const void *dout, const float *lse,
                            void *ws, void *stream);
libra_status launch_dq(const libra_plan_info &h, BwdArgs a, const void *plan_dev, void *dq,
                       libra_cu_record *records, void *stream);

}  // namespace libra
