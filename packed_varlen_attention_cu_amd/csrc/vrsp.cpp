// Variance-reduced sequence placement (host).
//
// Libra technical review, section 4.2, Algorithm 1, and Libra paper,
// section 4.2: the packed sequences of one optimizer-step window are placed
// heaviest first (workload F = sum of squared sample lengths, eq. 1), each on
// the least-loaded pool that still holds fewer than P sequences; full pools
// leave the candidate heap for good, which enforces the exact cardinality.
// Ties: equal workloads by sequence index, equal loads by pool index.
//
// Cost: one sort of the window and one heap operation per sequence,
// O(D log D) time and O(K) pool state.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <queue>
#include <utility>
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

extern "C" libra_status libra_vrsp(const int64_t *workload, int32_t num_seqs, int32_t pool_size, int32_t *pool_of,
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

  // Min-heap of (load, pool) over the pools that still have room.
  using Entry = std::pair<int64_t, int32_t>;
  std::vector<Entry> init;
  init.reserve(pools);
  for (int32_t k = 0; k < pools; ++k) init.emplace_back(0, k);
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap(std::greater<Entry>(), std::move(init));
  std::vector<int32_t> count(pools, 0);
  std::vector<int64_t> load(pools, 0);
  for (int32_t i : seq) {
    const int32_t k = heap.top().second;
    heap.pop();
    pool_of[i] = k;
    order[(int64_t)k * pool_size + count[k]] = i;
    load[k] += workload[i];
    if (++count[k] < pool_size) heap.emplace(load[k], k);
  }
  if (pool_load != nullptr)
    for (int32_t k = 0; k < pools; ++k) pool_load[k] = load[k];
  return LIBRA_OK;
}
