// Variance-reduced sequence placement (host).
//
// Libra technical review, section 4.2 (Algorithm 1), and Libra paper,
// section 4.2.  The rule: the packed sequences of one optimizer-step window
// are dealt out heaviest first (workload F = sum of squared sample lengths,
// eq. 1; equal workloads by sequence index), each to the pool with the least
// summed workload among the pools that still hold fewer than P sequences
// (equal loads by pool index), so that every pool ends with exactly P.
//
// Here the pools are the leaves of a tournament tree: every inner node holds
// the winner of its two children under (open, load, pool index), a full pool
// losing to any open one.  The root is the pool the rule asks for; after a
// sequence is added, only the path from that pool's leaf to the root is
// replayed.  Cost: one sort of the window and O(log K) per sequence.
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "libra.h"

extern "C" libra_status libra_pack_workload(const int32_t *cu_seqlens, int32_t num_samples, int64_t *workload) {
  if (cu_seqlens == nullptr || workload == nullptr || num_samples < 0 || cu_seqlens[0] != 0)
    return LIBRA_EINVAL;
  int64_t f = 0;
  for (int32_t j = 0; j < num_samples; ++j) {
    const int64_t len = (int64_t)cu_seqlens[j + 1] - cu_seqlens[j];
    if (len < 0) return LIBRA_EINVAL;
    f += len * len;
  }
  *workload = f;
  return LIBRA_OK;
}

namespace {

libra_status vrsp_impl(const int64_t *workload, int32_t num_seqs, int32_t pool_size, int32_t *pool_of,
                       int32_t *order, int64_t *pool_load) {
  if (workload == nullptr || pool_of == nullptr || order == nullptr || num_seqs <= 0 || pool_size <= 0 ||
      num_seqs % pool_size != 0)
    return LIBRA_EINVAL;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (workload[i] < 0) return LIBRA_EINVAL;
  const int32_t pools = num_seqs / pool_size;

  std::vector<int32_t> seq(num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) seq[i] = i;
  std::sort(seq.begin(), seq.end(), [&](int32_t x, int32_t y) {
    return workload[x] != workload[y] ? workload[x] > workload[y] : x < y;
  });

  // Tournament tree over the pools: leaves at [width, width + pools), node i
  // holds the better of nodes 2i and 2i + 1, or -1 when neither subtree has an
  // open pool; padding leaves are -1.
  int32_t width = 1;
  while (width < pools) width *= 2;
  std::vector<int32_t> count(pools, 0);
  std::vector<int64_t> load(pools, 0);
  std::vector<int32_t> node(2 * (size_t)width, -1);
  auto better = [&](int32_t x, int32_t y) {   // the winner of pools x and y (-1: none)
    if (x < 0) return y;
    if (y < 0) return x;
    return (load[x] < load[y] || (load[x] == load[y] && x < y)) ? x : y;
  };
  for (int32_t k = 0; k < pools; ++k) node[width + k] = k;
  for (int32_t i = width - 1; i >= 1; --i) node[i] = better(node[2 * i], node[2 * i + 1]);
  for (int32_t i : seq) {
    const int32_t k = node[1];                 // open pool of least (load, index)
    pool_of[i] = k;
    order[(int64_t)k * pool_size + count[k]] = i;
    load[k] += workload[i];
    if (++count[k] == pool_size) node[width + k] = -1;   // full: out of the contest
    for (int32_t j = (width + k) / 2; j >= 1; j /= 2) node[j] = better(node[2 * j], node[2 * j + 1]);
  }
  if (pool_load != nullptr)
    for (int32_t k = 0; k < pools; ++k) pool_load[k] = load[k];
  return LIBRA_OK;
}

}  // namespace

extern "C" libra_status libra_vrsp(const int64_t *workload, int32_t num_seqs, int32_t pool_size, int32_t *pool_of,
                                   int32_t *order, int64_t *pool_load) {
  try {
    return vrsp_impl(workload, num_seqs, pool_size, pool_of, order, pool_load);
  } catch (const std::bad_alloc &) {
    return LIBRA_EHOST;
  }
}
