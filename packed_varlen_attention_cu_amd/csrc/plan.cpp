// Host SH-Tile planner and FLOPs-aware work placement.
//
// SH-Tiles follow the Libra technical review, section 5: the packed sequence
// is cut at global token positions into blocks of at most B tokens and the
// query heads into shards of W heads (eq. 6); a tile's KV groups are the
// samples its block intersects (eq. 7); its cost is the exact number of
// unmasked causal pairs, sum over those samples of sum_{q=a}^{e-1} (q + 1),
// times W (eq. 8).
//
// On one GPU the workers are the CUs.  A tile is cut into work items that one
// workgroup executes: forward items of at most 384 query columns (positions
// x heads), dQ items of at most 256, and key-major dK/dV items of 192 keys
// (see libra.h).  Items are costed by the work their kernel executes (or, on
// request, by eq. 8 pairs), grouped into zigzag pairs, and placed by
// Algorithm 2 (section 5.4): heaviest first, onto a worker within the soft
// target (1 + tau) x the even share that adds the least communication (eq.
// 9), else the least loaded one.  With no communication term the rule
// reduces to least-loaded placement, which runs as a binary heap keyed by
// (load, worker id); the L2 term of LIBRA_ASSIGN_PLACER_L2 (the XCD's L2
// standing in for the worker's memory) runs over one heap per XCD.
//
// Everything here is integer arithmetic (the soft-target test excepted, done
// in double precision in a fixed order) and bitwise deterministic.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <exception>
#include <functional>
#include <queue>
#include <thread>
#include <unordered_map>
#include <vector>

#include "libra.h"
#include "plan_layout.h"

namespace {

constexpr int kFwdItemColumns = libra::kFwdItemColumns;   // query columns per forward item
constexpr int kDqItemColumns = libra::kDqItemColumns;     // query columns per dQ item
constexpr int kKvChunk = libra::kKvItemKeys;   // keys per dK/dV item
constexpr int kDefaultCus = 256;
constexpr int kMaxCus = 1 << 16;

// sum_{q=a}^{e-1} (q + 1) for sample-local query positions a <= e.
inline int64_t triangle(int64_t a, int64_t e) { return (e * (e + 1) - a * (a + 1)) / 2; }

// Per-head causal pairs of query rows [lo, hi); `j` walks forward over samples.
int64_t query_pairs(const int32_t *cu, int n, int64_t lo, int64_t hi, int *j) {
  while (*j < n && cu[*j + 1] <= lo) ++*j;
  int64_t pairs = 0;
  for (int s = *j; s < n && cu[s] < hi; ++s) {
    int64_t a = std::max<int64_t>(lo, cu[s]), e = std::min<int64_t>(hi, cu[s + 1]);
    if (a < e) pairs += triangle(a - cu[s], e - cu[s]);
  }
  return pairs;
}

// Per-head pairs seen from keys [lo, hi): each key k pairs with queries k..end(k)-1.
int64_t key_pairs(const int32_t *cu, int n, int64_t lo, int64_t hi, int *j) {
  while (*j < n && cu[*j + 1] <= lo) ++*j;
  int64_t pairs = 0;
  for (int s = *j; s < n && cu[s] < hi; ++s) {
    int64_t a = std::max<int64_t>(lo, cu[s]), b = std::min<int64_t>(hi, cu[s + 1]);
    if (a < b) pairs += (b - a) * (int64_t)cu[s + 1] - (a + b - 1) * (b - a) / 2;
  }
  return pairs;
}

// End of the non-empty sample holding position pos; `j` walks forward over samples.
int64_t sample_end(const int32_t *cu, int n, int64_t pos, int *j) {
  while (*j < n && cu[*j + 1] <= pos) ++*j;
  return cu[*j + 1];
}

int head_group(int n) { return n % 4 == 0 ? 4 : (n % 2 == 0 ? 2 : 1); }

// Index of the sample holding position pos (pos < L): the last j with cu[j] <= pos.
int sample_of(const int32_t *cu, int n, int64_t pos) {
  return (int)(std::upper_bound(cu, cu + n + 1, (int32_t)pos) - cu) - 1;
}

// Query-key slots of the walk of a forward or dQ item of rows [row0, row0 +
// nrows) and nh heads: its workgroup steps through every 64-key block from the
// one holding the start of its first row's sample to the one holding its last
// row, and each step copies the block and synchronises all of its waves (32
// rows of one head each) whether or not their rows see a key there.
int64_t executed_slots(const int32_t *cu, int n, int64_t row0, int64_t nrows, int nh) {
  if (nrows <= 0) return 0;
  const int64_t first = cu[sample_of(cu, n, row0)] / libra::kKeyBlock;
  const int64_t blocks = (row0 + nrows - 1) / libra::kKeyBlock - first + 1;
  const int64_t waves = nh * ((nrows + libra::kQueryTile - 1) / libra::kQueryTile);
  return waves * blocks * libra::kQueryTile * libra::kKeyBlock;
}

libra_status validate(const int32_t *cu, const libra_plan_params *p) {
  if (!cu || !p) return LIBRA_EINVAL;
  if (p->total_tokens < 0 || p->num_samples < 0) return LIBRA_EINVAL;
  if (p->h_q <= 0 || p->h_kv <= 0 || p->h_q % p->h_kv) return LIBRA_EINVAL;
  if (p->tile_tokens <= 0 || p->tile_heads <= 0 || p->h_q % p->tile_heads) return LIBRA_EINVAL;
  if (p->num_cus < 0 || p->num_cus > kMaxCus) return LIBRA_EINVAL;
  if (!(p->tau >= 0.0f) || !std::isfinite(p->tau)) return LIBRA_EINVAL;
  if (p->assign != LIBRA_ASSIGN_PLACER && p->assign != LIBRA_ASSIGN_ROUND_ROBIN &&
      p->assign != LIBRA_ASSIGN_PLACER_L2)
    return LIBRA_EINVAL;
  if (p->cost != LIBRA_COST_EXECUTED && p->cost != LIBRA_COST_PAIRS) return LIBRA_EINVAL;
  if (p->reserved != 0) return LIBRA_EINVAL;
  if (p->item_overhead < 0) return LIBRA_EINVAL;
  if (cu[0] != 0) return LIBRA_EINVAL;
  for (int j = 0; j < p->num_samples; ++j)
    if (cu[j + 1] < cu[j]) return LIBRA_EINVAL;
  if (cu[p->num_samples] != p->total_tokens) return LIBRA_EINVAL;
  if (p->head_dim != 64 && p->head_dim != 128) return LIBRA_EUNSUPPORTED;
  return LIBRA_OK;
}

struct Queue {
  std::vector<libra_item> items;   // in CU order
  std::vector<int32_t> cu_off;
  int64_t load_max = 0, load_sum = 0;
};

// A worker's load and id; heaps of them are ordered by (load, worker id).
struct Load {
  int64_t load;
  int32_t worker;
};
inline bool lighter(const Load &x, const Load &y) {
  return x.load != y.load ? x.load < y.load : x.worker < y.worker;
}

// Give the root of a min-heap the load `top` and restore the heap order.
void sift_root(std::vector<Load> &h, Load top) {
  size_t i = 0;
  for (;;) {
    const size_t l = 2 * i + 1, r = l + 1;
    size_t m = i;
    const Load *best = &top;
    if (l < h.size() && lighter(h[l], *best)) { m = l; best = &h[l]; }
    if (r < h.size() && lighter(h[r], *best)) { m = r; best = &h[r]; }
    if (m == i) break;
    h[i] = h[m];
    i = m;
  }
  h[i] = top;
}

// Worker speeds of a plan: the eight class speeds, 0 read as 1000.
struct Speeds {
  int64_t s[8];
  bool uniform;
  explicit Speeds(const uint16_t *v) {
    for (int x = 0; x < 8; ++x) s[x] = v[x] ? v[x] : 1000;
    uniform = true;
    for (int x = 1; x < 8; ++x) uniform = uniform && s[x] == s[0];
  }
};

// The KV groups of every placement unit and their volumes, for the L2 term:
// unit u holds groups ids[off[u] .. off[u + 1]), group g has volume vol[g].
struct UnitGroups {
  std::vector<int64_t> off;
  std::vector<int32_t> ids;
  std::vector<int64_t> vol;
  int32_t n_groups = 0;
};

// Algorithm 2 over workers in eight speed classes (worker r in class r mod 8,
// the XCD that runs workgroup r), with the L2 communication term when
// `groups` is given and none otherwise.  Within a class every worker has the
// same speed and the same communication term, so the class's candidate is
// its least loaded worker (a heap top): a unit goes to the best of the eight
// tops under the key (within target, term, finish, id) / (beyond target,
// finish, term, id), finish = (load + cost) / speed compared exactly by
// cross-multiplication.  (load + cost) * speed < 2^47 * 2^11 fits int64.
void place_classes(const std::vector<int64_t> &costs_sorted, const std::vector<int32_t> &idx_sorted,
                   int workers, const Speeds &sp, float tau, const UnitGroups *groups,
                   std::vector<int32_t> &worker, std::vector<int64_t> &load) {
  std::vector<Load> heap[8];
  for (int32_t r = 0; r < workers; ++r) heap[r % 8].push_back({0, r});   // ascending ids: valid heaps
  double speed_sum = 0, cost_sum = 0;
  for (int32_t r = 0; r < workers; ++r) speed_sum += (double)sp.s[r % 8];
  int64_t total = 0;
  for (int64_t c : costs_sorted) total += c;
  cost_sum = (double)total;
  const double budget = (1.0 + (double)tau) * cost_sum;
  std::vector<uint8_t> held;                        // held[x * n_groups + g]: group g committed to XCD x
  if (groups) held.assign((size_t)8 * groups->n_groups, 0);
  for (size_t k = 0; k < costs_sorted.size(); ++k) {
    const int64_t c = costs_sorted[k];
    const int32_t u = idx_sorted[k];
    int best = -1;
    bool best_fits = false;
    int64_t best_term = 0;
    for (int x = 0; x < 8; ++x) {
      if (heap[x].empty()) continue;
      const Load &t = heap[x][0];
      const bool fits = (double)(t.load + c) * speed_sum <= budget * (double)sp.s[x];
      int64_t term = 0;
      if (groups) {
        for (int64_t i = groups->off[u]; i < groups->off[u + 1]; ++i) {
          const int32_t g = groups->ids[i];
          if (!held[(size_t)x * groups->n_groups + g]) term += groups->vol[g];
        }
      }
      bool better;
      if (best < 0) {
        better = true;
      } else {
        const Load &b = heap[best][0];
        const int64_t lhs = (t.load + c) * sp.s[best], rhs = (b.load + c) * sp.s[x];   // finish x vs best
        const int finish_cmp = lhs < rhs ? -1 : (lhs > rhs ? 1 : 0);
        if (fits != best_fits) better = fits;
        else if (fits && term != best_term) better = term < best_term;
        else if (finish_cmp != 0) better = finish_cmp < 0;
        else if (!fits && term != best_term) better = term < best_term;
        else better = t.worker < b.worker;
      }
      if (better) {
        best = x;
        best_fits = fits;
        best_term = term;
      }
    }
    std::vector<Load> &h = heap[best];
    Load top = h[0];
    worker[u] = top.worker;
    top.load += c;
    load[top.worker] = top.load;
    sift_root(h, top);
    if (groups)
      for (int64_t i = groups->off[u]; i < groups->off[u + 1]; ++i)
        held[(size_t)best * groups->n_groups + groups->ids[i]] = 1;
  }
}

// Place `units` (Algorithm 2, or round-robin) and emit per-worker queues as
// CSR.  Units are taken heaviest first, ties to the lower index.
Queue place(const std::vector<libra_item> &units, int workers, int mode, const Speeds &sp, float tau,
            const UnitGroups *groups) {
  Queue q;
  const size_t n = units.size();
  std::vector<int32_t> worker(n);
  std::vector<int32_t> order(n);
  std::vector<int64_t> load(workers, 0);
  if (mode == LIBRA_ASSIGN_ROUND_ROBIN) {
    for (size_t t = 0; t < n; ++t) {
      order[t] = (int32_t)t;
      worker[t] = (int32_t)(t % workers);
      load[worker[t]] += units[t].cost;
    }
  } else {
    int64_t cmax = 0;
    for (size_t i = 0; i < n; ++i) cmax = std::max(cmax, units[i].cost);
    if (cmax < (int64_t(1) << 43) && n < (size_t(1) << 20)) {
      // (cost descending, index ascending) as one ascending 64-bit key
      std::vector<uint64_t> packed(n);
      for (size_t i = 0; i < n; ++i)
        packed[i] = (uint64_t)((int64_t(1) << 43) - 1 - units[i].cost) << 20 | (uint64_t)i;
      std::sort(packed.begin(), packed.end());
      for (size_t k = 0; k < n; ++k) order[k] = (int32_t)(packed[k] & ((1u << 20) - 1));
    } else {
      for (size_t i = 0; i < n; ++i) order[i] = (int32_t)i;
      std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        return units[a].cost != units[b].cost ? units[a].cost > units[b].cost : a < b;
      });
    }
    std::vector<int64_t> cs(n);
    for (size_t k = 0; k < n; ++k) cs[k] = units[order[k]].cost;
    const UnitGroups *g = mode == LIBRA_ASSIGN_PLACER_L2 ? groups : nullptr;
    if (g || !sp.uniform) {
      place_classes(cs, order, workers, sp, tau, g, worker, load);
    } else {
      // No communication term, equal speeds: the least loaded worker (ties: lowest id), one heap.
      std::vector<Load> heap(workers);
      for (int32_t r = 0; r < workers; ++r) heap[r] = {0, r};   // ordered, hence a valid heap
      for (size_t k = 0; k < n; ++k) {
        Load top = heap[0];
        worker[order[k]] = top.worker;
        top.load += cs[k];
        load[top.worker] = top.load;
        sift_root(heap, top);
      }
    }
  }
  q.cu_off.assign(workers + 1, 0);
  for (size_t t = 0; t < n; ++t) q.cu_off[worker[t] + 1]++;
  for (int r = 0; r < workers; ++r) q.cu_off[r + 1] += q.cu_off[r];
  std::vector<int32_t> fill(q.cu_off.begin(), q.cu_off.end() - 1);
  q.items.resize(n);
  for (int32_t t : order) q.items[fill[worker[t]]++] = units[t];
  for (int r = 0; r < workers; ++r) {
    q.load_max = std::max(q.load_max, load[r]);
    q.load_sum += load[r];
  }
  return q;
}

// Largest finish time (load / speed) over the mean one; with equal speeds,
// the largest load over the mean load.
double finish_max_over_mean(const Queue &q, int workers, const Speeds &sp) {
  double mx = 0, sum = 0;
  for (int r = 0; r < workers; ++r) {
    int64_t l = 0;
    for (int32_t k = q.cu_off[r]; k < q.cu_off[r + 1]; ++k) l += q.items[k].cost;
    const double f = (double)l / (double)sp.s[r % 8];
    mx = std::max(mx, f);
    sum += f;
  }
  return sum > 0 ? mx * workers / sum : 1.0;
}

// Where the KV groups of the L2 term come from: the packing and the KV head count.
struct GroupSource {
  const int32_t *cu;
  int n, h_kv;
};

// Append the KV groups (sample j, KV head) of item `it` -- every non-empty
// sample its rows meet -- to `ids`, skipping those already listed from `from`.
void append_groups(const GroupSource &gs, const libra_item &it, size_t from, std::vector<int32_t> &ids) {
  const int64_t lo = it.row0, hi = (int64_t)it.row0 + it.nrows;
  for (int j = sample_of(gs.cu, gs.n, lo); j < gs.n && gs.cu[j] < hi; ++j) {
    if (gs.cu[j + 1] <= std::max<int64_t>(lo, gs.cu[j])) continue;
    const int32_t g = j * gs.h_kv + it.kv_head;
    if (std::find(ids.begin() + from, ids.end(), g) == ids.end()) ids.push_back(g);
  }
}

// Zigzag units.  Items sharing a group key (for the dK/dV items: the sample
// of the last key and the KV head; for forward and dQ items: the sample of
// the first row, the KV head and the first head) are taken in row order
// u_0 .. u_{m-1}; u_i pairs with u_{m-1-i} (the middle one of an odd group
// stands alone).  A pair is one placement unit of cost f(u_i) + f(u_{m-1-i}),
// numbered by its first item; its worker runs u_i in its kind's default walk
// order, then u_{m-1-i} in reverse (LIBRA_ITEM_REVERSE).  The walks of a
// pair then cover a fixed span, so pairs of a group cost the same and pairs
// that start together read the same K / V (or Q / dO) block at every step:
// the CUs sharing an L2 share the streamed rows.  Equal-cost pairs are
// coarser than single items: when one group holds most of the work they leave
// too few small units to level the workers, so the pairs are kept only if,
// placed by least finish time, their largest finish time is within 0.5 % of
// the mean one; otherwise the single items are placed, all in the default
// order.  The units are then placed in the plan's mode.
// Items arrive in id order (id = index) and rows ascend within a group.
Queue place_zigzag(const std::vector<libra_item> &items, const std::vector<int64_t> &group, int workers,
                   int mode, const Speeds &sp, float tau, const GroupSource &gs) {
  const size_t n = items.size();
  std::vector<int32_t> second(n, -2);   // -2: not a unit's first item, -1: alone
  {
    std::unordered_map<int64_t, std::vector<int32_t>> members;
    members.reserve(n / 4 + 1);
    for (size_t i = 0; i < n; ++i) members[group[i]].push_back((int32_t)i);
    for (auto &kv : members) {
      const std::vector<int32_t> &m = kv.second;
      for (size_t i = 0; i + i + 1 <= m.size(); ++i) {
        const size_t j = m.size() - 1 - i;
        second[m[i]] = i == j ? -1 : m[j];
      }
    }
  }
  std::vector<libra_item> units;   // each unit carries its first item, with the pair's cost
  units.reserve(n / 2 + 1);
  for (size_t i = 0; i < n; ++i)
    if (second[i] != -2) {
      libra_item u = items[i];
      if (second[i] >= 0) u.cost += items[second[i]].cost;
      units.push_back(u);
    }
  const int trial_mode = mode == LIBRA_ASSIGN_ROUND_ROBIN ? mode : LIBRA_ASSIGN_PLACER;
  Queue uq = place(units, workers, trial_mode, sp, tau, nullptr);
  if (finish_max_over_mean(uq, workers, sp) > 1.005) {   // pairs too coarse: single items
    units = items;
    std::fill(second.begin(), second.end(), -1);
    if (mode == trial_mode) uq = place(units, workers, mode, sp, tau, nullptr);
  }
  if (mode != trial_mode) {
    UnitGroups ug;
    ug.n_groups = gs.n * gs.h_kv;
    ug.vol.resize(ug.n_groups);
    for (int j = 0; j < gs.n; ++j)
      for (int kv = 0; kv < gs.h_kv; ++kv) ug.vol[(size_t)j * gs.h_kv + kv] = gs.cu[j + 1] - gs.cu[j];
    ug.off.reserve(units.size() + 1);
    ug.off.push_back(0);
    for (const libra_item &u : units) {
      const size_t from = ug.ids.size();
      append_groups(gs, items[u.id], from, ug.ids);
      if (second[u.id] >= 0) append_groups(gs, items[second[u.id]], from, ug.ids);
      ug.off.push_back((int64_t)ug.ids.size());
    }
    uq = place(units, workers, mode, sp, tau, &ug);
  }
  Queue q;
  q.load_max = uq.load_max;
  q.load_sum = uq.load_sum;
  q.cu_off.assign(workers + 1, 0);
  q.items.reserve(n);
  for (int r = 0; r < workers; ++r) {
    for (int32_t k = uq.cu_off[r]; k < uq.cu_off[r + 1]; ++k) {
      const int32_t a = uq.items[k].id;
      q.items.push_back(items[a]);
      if (second[a] >= 0) {
        q.items.push_back(items[second[a]]);
        q.items.back().flags = LIBRA_ITEM_REVERSE;
      }
    }
    q.cu_off[r + 1] = (int32_t)q.items.size();
  }
  return q;
}

size_t align64(size_t x) { return (x + 63) & ~size_t(63); }

// Byte offsets of the plan sections (written into hdr when it is not null)
// and the total size: header, tiles, items, cu_off, dQ items, dQ cu_off,
// kv items, kv cu_off.
size_t section_offsets(size_t n_tiles, size_t n_items, size_t n_dq, size_t n_kv, int workers,
                       libra_plan_info *hdr) {
  libra_plan_info tmp{};
  libra_plan_info &h = hdr ? *hdr : tmp;
  size_t off = align64(sizeof(libra_plan_info));
  h.off_tiles = off;
  off = align64(off + n_tiles * sizeof(libra_tile));
  h.off_items = off;
  off = align64(off + n_items * sizeof(libra_item));
  h.off_cu_off = off;
  off = align64(off + (workers + 1) * sizeof(int32_t));
  h.off_dq_items = off;
  off = align64(off + n_dq * sizeof(libra_item));
  h.off_dq_cu_off = off;
  off = align64(off + (workers + 1) * sizeof(int32_t));
  h.off_kv_items = off;
  off = align64(off + n_kv * sizeof(libra_item));
  h.off_kv_cu_off = off;
  off = align64(off + (workers + 1) * sizeof(int32_t));
  return off;
}

size_t plan_bytes(int64_t n_tiles, int64_t n_items, int64_t n_dq, int64_t n_kv, int workers) {
  return section_offsets((size_t)n_tiles, (size_t)n_items, (size_t)n_dq, (size_t)n_kv, workers, nullptr);
}

// FNV-1a over 64-bit words, run as four interleaved streams (words i mod 4)
// that are folded together at the end, so the multiplies overlap.
uint64_t fnv1a_words(const void *buf, size_t bytes) {
  const uint64_t *w = static_cast<const uint64_t *>(buf);
  const size_t n = bytes / 8;
  uint64_t h[4] = {0xcbf29ce484222325ull, 0xcbf29ce484222325ull ^ 1, 0xcbf29ce484222325ull ^ 2,
                   0xcbf29ce484222325ull ^ 3};
  size_t i = 0;
  for (; i + 4 <= n; i += 4)
    for (int s = 0; s < 4; ++s) {
      h[s] ^= w[i + s];
      h[s] *= 0x100000001b3ull;
    }
  for (; i < n; ++i) {
    h[0] ^= w[i];
    h[0] *= 0x100000001b3ull;
  }
  uint64_t r = h[0];
  for (int s = 1; s < 4; ++s) {
    r ^= h[s];
    r *= 0x100000001b3ull;
  }
  return r;
}

}  // namespace

namespace libra {

uint64_t plan_checksum(const void *plan, size_t bytes) {
  libra_plan_info hdr;
  std::memcpy(&hdr, plan, sizeof hdr);
  hdr.checksum = 0;
  uint64_t h = fnv1a_words(&hdr, sizeof hdr);
  const char *p = static_cast<const char *>(plan);
  uint64_t rest = fnv1a_words(p + sizeof hdr, bytes - sizeof hdr);
  return h ^ (rest * 0x9e3779b97f4a7c15ull);
}

libra_status plan_header(const void *plan, libra_plan_info *out) {
  if (!plan) return LIBRA_EINVAL;
  std::memcpy(out, plan, sizeof *out);
  if (out->magic != LIBRA_PLAN_MAGIC || out->version != LIBRA_PLAN_VERSION) return LIBRA_EINVAL;
  return LIBRA_OK;
}

libra_status plan_validate(const void *plan, libra_plan_info *out) {
  libra_plan_info h;
  if (plan_header(plan, &h) != LIBRA_OK) return LIBRA_EINVAL;
  if (h.bytes < sizeof h || h.bytes % 8 || h.num_cus <= 0 || h.num_cus > kMaxCus) return LIBRA_EINVAL;
  if (h.n_tiles < 0 || h.n_items < 0 || h.n_dq_items < 0 || h.n_kv_items < 0) return LIBRA_EINVAL;
  const uint64_t sections[][2] = {
      {h.off_tiles, (uint64_t)h.n_tiles * sizeof(libra_tile)},
      {h.off_items, (uint64_t)h.n_items * sizeof(libra_item)},
      {h.off_cu_off, (uint64_t)(h.num_cus + 1) * sizeof(int32_t)},
      {h.off_dq_items, (uint64_t)h.n_dq_items * sizeof(libra_item)},
      {h.off_dq_cu_off, (uint64_t)(h.num_cus + 1) * sizeof(int32_t)},
      {h.off_kv_items, (uint64_t)h.n_kv_items * sizeof(libra_item)},
      {h.off_kv_cu_off, (uint64_t)(h.num_cus + 1) * sizeof(int32_t)}};
  for (const auto &sec : sections)
    if (sec[0] % 64 || sec[0] < sizeof h || sec[0] > h.bytes || sec[1] > h.bytes - sec[0]) return LIBRA_EINVAL;
  if (plan_checksum(plan, h.bytes) != h.checksum) return LIBRA_EINVAL;
  *out = h;
  return LIBRA_OK;
}

}  // namespace libra

namespace {

// Joins its thread, if one was started, when it goes out of scope.
struct Joiner {
  std::thread t;
  ~Joiner() {
    if (t.joinable()) t.join();
  }
};

libra_status plan_impl(const int32_t *cu, const libra_plan_params *pp, void *buf, size_t *bytes) {
  if (!bytes) return LIBRA_EINVAL;
  libra_status st = validate(cu, pp);
  if (st != LIBRA_OK) return st;
  libra_plan_params p = *pp;
  const int workers = p.num_cus ? p.num_cus : kDefaultCus;
  const int n = p.num_samples;
  const int64_t L = p.total_tokens;
  const int g = p.h_q / p.h_kv;
  const int S = p.h_q / p.tile_heads;
  const int64_t nblocks = (L + p.tile_tokens - 1) / p.tile_tokens;

  // Work items a tile is cut into for a kernel whose workgroup covers
  // `columns` query columns (positions x heads).
  auto count_items = [&](int columns) {
    int64_t count = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
      const int64_t rows_in = std::min<int64_t>(L, (b + 1) * p.tile_tokens) - b * p.tile_tokens;
      for (int s = 0; s < S; ++s) {
        const int h_lo = s * p.tile_heads, h_hi = h_lo + p.tile_heads;
        for (int kv = h_lo / g; kv <= (h_hi - 1) / g; ++kv) {
          const int hn = std::min(h_hi, (kv + 1) * g) - std::max(h_lo, kv * g);
          const int nh = head_group(hn), rows = columns / nh;
          count += (int64_t)(hn / nh) * ((rows_in + rows - 1) / rows);
        }
      }
    }
    return count;
  };
  // The section lengths follow from the counts alone.
  const int64_t n_items = count_items(kFwdItemColumns), n_dq = count_items(kDqItemColumns);
  const int64_t n_kv = (L + kKvChunk - 1) / kKvChunk * p.h_kv;
  if (!buf) {   // size query
    *bytes = plan_bytes(nblocks * S, n_items, n_dq, n_kv, workers);
    return LIBRA_OK;
  }

  // Tiles (eq. 6-8), forward items and dQ items.
  std::vector<libra_tile> tiles;
  std::vector<libra_item> items, dq_items;
  tiles.reserve(nblocks * S);
  items.reserve(n_items);
  dq_items.reserve(n_dq);
  // Per-head pairs and per-head walk slots (executed_slots) of a block's row
  // chunks of one length, computed once per block and chunk length.
  struct ChunkWork {
    int64_t pairs, slots;
  };
  std::vector<std::pair<int, std::vector<ChunkWork>>> chunk_pairs;
  int jb = 0;
  // Cut tile t (rows [lo, hi) of block b, whose first sample is jb) into
  // items of at most `columns` query columns, appended to `out`; returns how
  // many.
  auto cut = [&](const libra_tile &t, int64_t lo, int64_t hi, int columns, std::vector<libra_item> &out) {
    const int h_lo = t.head_begin, h_hi = h_lo + t.head_count;
    int32_t made = 0;
    for (int kv = h_lo / g; kv <= (h_hi - 1) / g; ++kv) {
      const int a = std::max(h_lo, kv * g), e = std::min(h_hi, (kv + 1) * g);
      const int nh = head_group(e - a);
      const int rows = columns / nh;
      std::vector<ChunkWork> *cp = nullptr;
      for (auto &c : chunk_pairs)
        if (c.first == rows) cp = &c.second;
      if (!cp) {
        chunk_pairs.emplace_back(rows, std::vector<ChunkWork>());
        cp = &chunk_pairs.back().second;
        int ji = jb;
        for (int64_t r0 = lo; r0 < hi; r0 += rows) {
          const int64_t r1 = std::min<int64_t>(hi, r0 + rows);
          const int64_t pairs = query_pairs(cu, n, r0, r1, &ji);
          cp->push_back({pairs, p.cost == LIBRA_COST_PAIRS ? 0 : executed_slots(cu, n, r0, r1 - r0, 1)});
        }
      }
      for (int gi = 0; gi < (e - a) / nh; ++gi) {
        size_t ci = 0;
        for (int64_t r0 = lo; r0 < hi; r0 += rows, ++ci) {
          const int64_t r1 = std::min<int64_t>(hi, r0 + rows);
          libra_item it{};
          it.row0 = (int32_t)r0;
          it.nrows = (int32_t)(r1 - r0);
          it.kv_head = kv;
          it.head0 = a + gi * nh;
          it.nheads = nh;
          it.tile_id = t.tile_id;
          it.id = (int32_t)out.size();
          it.pairs = nh * (*cp)[ci].pairs;
          it.cost = (p.cost == LIBRA_COST_PAIRS ? it.pairs : nh * (*cp)[ci].slots) + p.item_overhead;
          out.push_back(it);
          ++made;
        }
      }
    }
    return made;
  };
  for (int64_t b = 0; b < nblocks; ++b) {
    const int64_t lo = b * p.tile_tokens, hi = std::min<int64_t>(L, lo + p.tile_tokens);
    chunk_pairs.clear();
    const int64_t per_head = query_pairs(cu, n, lo, hi, &jb);
    // K(t): the non-empty samples the block meets (all samples from jb end after lo).
    int first = -1, last = -1;
    for (int s = jb; s < n && cu[s] < hi; ++s) {
      if (cu[s + 1] == cu[s]) continue;
      if (first < 0) first = s;
      last = s;
    }
    for (int s = 0; s < S; ++s) {
      libra_tile t{};
      t.tile_id = (int32_t)(b * S + s);
      t.block = (int32_t)b;
      t.shard = s;
      t.tok_begin = (int32_t)lo;
      t.tok_end = (int32_t)hi;
      t.head_begin = s * p.tile_heads;
      t.head_count = p.tile_heads;
      t.sample_first = first;
      t.sample_last = last;
      t.pairs = per_head * p.tile_heads;
      t.n_items = cut(t, lo, hi, kFwdItemColumns, items);
      cut(t, lo, hi, kDqItemColumns, dq_items);
      tiles.push_back(t);
    }
  }

  // Key-major dK/dV items: chunks of kKvChunk keys, all g query heads of a KV
  // head.  Their cost is the work the dK/dV kernel executes, not the causal
  // pairs: every step runs a whole query block of kKvQueryBlock rows against
  // all of the item's keys, masked or not, and a step's time hardly depends
  // on how many of its pairs the mask keeps (per-CU busy time follows the
  // step count, not the pair count).
  std::vector<libra_item> kv_items;
  const int64_t nchunks = (L + kKvChunk - 1) / kKvChunk;
  kv_items.reserve(n_kv);
  int jk = 0, je = 0;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t lo = c * kKvChunk, hi = std::min<int64_t>(L, lo + kKvChunk);
    const int64_t per_head = key_pairs(cu, n, lo, hi, &jk);
    const int64_t qstart = lo / libra::kKvQueryBlock * libra::kKvQueryBlock;
    const int64_t qblocks = (sample_end(cu, n, hi - 1, &je) - qstart + libra::kKvQueryBlock - 1) /
                            libra::kKvQueryBlock;
    const int64_t executed = g * qblocks * libra::kKvQueryBlock * (hi - lo);
    for (int kv = 0; kv < p.h_kv; ++kv) {
      libra_item it{};
      it.row0 = (int32_t)lo;
      it.nrows = (int32_t)(hi - lo);
      it.kv_head = kv;
      it.head0 = kv * g;
      it.nheads = g;
      it.tile_id = -1;
      it.id = (int32_t)kv_items.size();
      it.pairs = g * per_head;
      it.cost = executed + p.item_overhead;
      kv_items.push_back(it);
    }
  }

  // The three queues are independent: place them on three host threads.
  Queue fq, dq, kq;
  // Zigzag group keys: (sample, KV head, first head) of each item, the sample
  // being that of the first row (forward, dQ) or of the last key (dK/dV).
  auto group_keys = [&](const std::vector<libra_item> &v, bool last_key) {
    std::vector<int64_t> key(v.size());
    for (size_t i = 0; i < v.size(); ++i) {
      const int64_t r = v[i].row0 + (last_key ? v[i].nrows - 1 : 0);
      const int64_t j = std::upper_bound(cu, cu + n + 1, (int32_t)r) - cu - 1;
      key[i] = j << 32 | (int64_t)v[i].kv_head << 16 | v[i].head0;
    }
    return key;
  };
  const Speeds sp(p.worker_speed);
  const GroupSource gs{cu, n, p.h_kv};
  {
    // An exception on a placement thread is carried to this one; the joiners
    // join every started thread on any exit from this block.
    std::exception_ptr err[2];
    Joiner t_dq, t_kv;
    t_dq.t = std::thread([&] {
      try {
        dq = place_zigzag(dq_items, group_keys(dq_items, false), workers, p.assign, sp, p.tau, gs);
      } catch (...) {
        err[0] = std::current_exception();
      }
    });
    t_kv.t = std::thread([&] {
      try {
        kq = place_zigzag(kv_items, group_keys(kv_items, true), workers, p.assign, sp, p.tau, gs);
      } catch (...) {
        err[1] = std::current_exception();
      }
    });
    fq = place_zigzag(items, group_keys(items, false), workers, p.assign, sp, p.tau, gs);
    t_dq.t.join();
    t_kv.t.join();
    for (const std::exception_ptr &e : err)
      if (e) std::rethrow_exception(e);
  }

  libra_plan_info hdr{};
  hdr.magic = LIBRA_PLAN_MAGIC;
  hdr.version = LIBRA_PLAN_VERSION;
  hdr.params = p;
  hdr.num_cus = workers;
  hdr.n_tiles = (int32_t)tiles.size();
  hdr.n_items = (int32_t)items.size();
  hdr.n_dq_items = (int32_t)dq_items.size();
  hdr.n_kv_items = (int32_t)kv_items.size();
  for (const auto &t : tiles) hdr.total_pairs += t.pairs;
  hdr.load_max = fq.load_max;
  hdr.load_sum = fq.load_sum;
  hdr.dq_load_max = dq.load_max;
  hdr.dq_load_sum = dq.load_sum;
  hdr.kv_load_max = kq.load_max;
  hdr.kv_load_sum = kq.load_sum;
  const size_t off = section_offsets(tiles.size(), fq.items.size(), dq.items.size(), kq.items.size(), workers, &hdr);
  hdr.bytes = off;

  if (*bytes < off || (reinterpret_cast<uintptr_t>(buf) & 7)) {
    *bytes = off;
    return (reinterpret_cast<uintptr_t>(buf) & 7) ? LIBRA_EINVAL : LIBRA_ESIZE;
  }
  char *out = static_cast<char *>(buf);
  std::memset(out, 0, off);
  std::memcpy(out + hdr.off_tiles, tiles.data(), tiles.size() * sizeof(libra_tile));
  std::memcpy(out + hdr.off_items, fq.items.data(), fq.items.size() * sizeof(libra_item));
  std::memcpy(out + hdr.off_cu_off, fq.cu_off.data(), fq.cu_off.size() * sizeof(int32_t));
  std::memcpy(out + hdr.off_dq_items, dq.items.data(), dq.items.size() * sizeof(libra_item));
  std::memcpy(out + hdr.off_dq_cu_off, dq.cu_off.data(), dq.cu_off.size() * sizeof(int32_t));
  std::memcpy(out + hdr.off_kv_items, kq.items.data(), kq.items.size() * sizeof(libra_item));
  std::memcpy(out + hdr.off_kv_cu_off, kq.cu_off.data(), kq.cu_off.size() * sizeof(int32_t));
  std::memcpy(out, &hdr, sizeof hdr);
  hdr.checksum = libra::plan_checksum(out, off);
  std::memcpy(out, &hdr, sizeof hdr);
  *bytes = off;
  return LIBRA_OK;
}

}  // namespace

extern "C" libra_status libra_plan(const int32_t *cu, const libra_plan_params *params, void *buf,
                                   size_t *bytes) {
  try {
    return plan_impl(cu, params, buf, bytes);
  } catch (...) {   // std::bad_alloc, std::system_error from std::thread
    return LIBRA_EHOST;
  }
}

extern "C" libra_status libra_plan_check(const void *plan, size_t bytes, libra_plan_info *info) {
  libra_plan_info hdr;
  if (!plan || bytes < sizeof hdr) return LIBRA_EINVAL;
  std::memcpy(&hdr, plan, sizeof hdr);
  if (hdr.bytes != bytes) return LIBRA_EINVAL;
  if (libra::plan_validate(plan, &hdr) != LIBRA_OK) return LIBRA_EINVAL;
  if (info) *info = hdr;
  return LIBRA_OK;
}

extern "C" libra_status libra_worker_speed(const void *plan_host, int32_t queue, const libra_cu_record *records,
                                           uint16_t speed_out[8]) {
  libra_plan_info h;
  if (!plan_host || !records || !speed_out) return LIBRA_EINVAL;
  if (libra::plan_header(plan_host, &h) != LIBRA_OK) return LIBRA_EINVAL;
  if (queue < LIBRA_QUEUE_FWD || queue > LIBRA_QUEUE_KV) return LIBRA_EINVAL;
  const uint8_t *base = static_cast<const uint8_t *>(plan_host);
  const uint64_t off_items[] = {h.off_items, h.off_dq_items, h.off_kv_items};
  const uint64_t off_cu[] = {h.off_cu_off, h.off_dq_cu_off, h.off_kv_cu_off};
  const libra_item *items = reinterpret_cast<const libra_item *>(base + off_items[queue]);
  const int32_t *cu_off = reinterpret_cast<const int32_t *>(base + off_cu[queue]);
  double load[8] = {0}, busy[8] = {0};
  for (int w = 0; w < h.num_cus; ++w) {
    int64_t l = 0;
    for (int32_t k = cu_off[w]; k < cu_off[w + 1]; ++k) l += items[k].cost;
    const uint64_t t0 = records[w].t_start, t1 = records[w].t_end;
    if (l <= 0 || t1 <= t0) continue;
    load[w % 8] += (double)l;
    busy[w % 8] += (double)(t1 - t0);
  }
  double rate[8], mean = 0;
  int classes = 0;
  for (int x = 0; x < 8; ++x) {
    rate[x] = busy[x] > 0 ? load[x] / busy[x] : 0.0;
    if (rate[x] > 0) {
      mean += rate[x];
      ++classes;
    }
  }
  if (classes) mean /= classes;
  for (int x = 0; x < 8; ++x) {
    const double v = rate[x] > 0 ? 1000.0 * rate[x] / mean : 1000.0;
    speed_out[x] = (uint16_t)std::lround(std::min(2000.0, std::max(500.0, v)));
  }
  return LIBRA_OK;
}

extern "C" const char *libra_status_str(libra_status s) {
  switch (s) {
    case LIBRA_OK: return "ok";
    case LIBRA_EINVAL: return "invalid argument";
    case LIBRA_ESIZE: return "buffer too small";
    case LIBRA_EUNSUPPORTED: return "unsupported configuration";
    case LIBRA_EHIP: return "HIP runtime error";
    case LIBRA_EHOST: return "host out of memory or threads";
  }
  return "unknown status";
}
