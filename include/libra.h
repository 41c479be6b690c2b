/*
 * libra.h -- C ABI of the MI355X (gfx950) packed variable-length causal
 * attention library: SH-Tile planner, FLOPs-aware tile-to-CU placement,
 * and persistent forward / backward attention kernels.
 *
 * Operation (Libra technical review, section 1 "Sequence packing" and
 * section 5.3 under eq. 8; Libra paper, section 2.3): samples are packed into
 * one sequence of L tokens described by cu_seqlens (n + 1 int32 prefix sums,
 * cu_seqlens[0] = 0, cu_seqlens[n] = L).  Query token i of sample j attends to
 * the keys of sample j at positions cu_seqlens[j] .. i (diagonal included),
 * never across samples.  Query head h reads KV head h / (h_q / h_kv).
 *
 *   O   = softmax(scale * Q K^T + mask) V          (bf16 out, fp32 accumulate)
 *   LSE = log(sum exp(scale * Q K^T + mask))        (natural log, fp32)
 *
 * Conventions shared by every entry point:
 *   - All tensors are contiguous and token-major:
 *       q, o, dout, dq : [L, h_q, head_dim] bf16
 *       k, v, dk, dv   : [L, h_kv, head_dim] bf16
 *       lse            : [h_q, L] fp32
 *     Device pointers must be 16-byte aligned.
 *   - The caller owns and allocates every buffer, host and device.  The
 *     library allocates no device memory (the host-only planner and VRSP use
 *     heap temporaries), keeps no state beyond the calling thread's last HIP
 *     error, never synchronises, and only enqueues work on the stream it is
 *     given (a hipStream_t passed as void*; NULL is the default stream).
 *   - Every argument is validated on the host before anything is enqueued;
 *     a failed check returns a negative libra_status and enqueues nothing.
 *     Launches verify the whole host plan (magic, version, section bounds,
 *     checksum over all its bytes; the plan's extent is the size its header
 *     records).  A launch error returns LIBRA_EHIP.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - A plan is a pure function of (cu_seqlens, libra_plan_params); one plan
 *     serves every layer with the same packing (Libra paper, section 4.1:
 *     the assignment is reused across layers with the same layout).  The
 *     device copy of a plan is a byte copy of the host buffer, uploaded by
 *     the caller, at least as long as the plan.  The kernels compare its
 *     checksum field with the host plan's before reading any queue; on a
 *     mismatch they run no item and set LIBRA_RECORD_PLAN_MISMATCH in their
 *     records (when records are given): the outputs are then left unwritten.
 */
#ifndef LIBRA_H
#define LIBRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LIBRA_OK = 0,
  LIBRA_EINVAL = -1,        /* malformed argument: pointer, cu_seqlens, shape, plan */
  LIBRA_ESIZE = -2,         /* a caller buffer is too small (required size returned) */
  LIBRA_EUNSUPPORTED = -3,  /* well formed but not supported (e.g. head_dim) */
  LIBRA_EHIP = -4,          /* the HIP runtime rejected a launch */
  LIBRA_EHOST = -5          /* the host ran out of memory or could not start a thread */
} libra_status;

/* Placement of the work items on the workers (libra_plan_params::assign).
 * Algorithm 2 (Libra technical review, section 5.4) sends units heaviest
 * first to a worker that stays within the soft target (1 + tau) x the even
 * share, preferring the smallest communication term of eq. 9, then the
 * least load, then the lowest id; if none stays within it, to the least
 * loaded worker.  On one GPU nothing is sent over a network:
 *   LIBRA_ASSIGN_PLACER     the communication term is 0, so the rule reduces
 *                           to least-loaded (earliest-finish) placement;
 *   LIBRA_ASSIGN_PLACER_L2  the term is eq. 9's KV part with the XCD's L2 in
 *                           the role of the worker's memory: worker w runs on
 *                           XCD w mod 8, a unit's KV groups are the (sample,
 *                           KV head) pairs its rows meet, and the term is the
 *                           token count of the groups not yet committed to
 *                           that XCD (a group joins the XCD's set once a unit
 *                           holding it is placed there);
 *   LIBRA_ASSIGN_ROUND_ROBIN unit i -> worker i mod num_cus (ablation). */
enum {
  LIBRA_ASSIGN_PLACER = 0,
  LIBRA_ASSIGN_ROUND_ROBIN = 1,
  LIBRA_ASSIGN_PLACER_L2 = 2
};

/* Cost of a forward or dQ work item (libra_plan_params::cost).  The pages
 * cost a tile by its unmasked causal pairs (eq. 8); a kernel that steps
 * through whole 64-key blocks spends more than that on blocks that straddle
 * a sample start or the diagonal, most of all on short samples.
 *   LIBRA_COST_EXECUTED  the query-key slots of the item's walk: for each of
 *                        its waves (32 query positions of one head), 32 x 64
 *                        per 64-key block from the one holding the start of
 *                        its first row's sample to the one holding its last
 *                        row (every step of the walk copies a block and
 *                        synchronises all waves, whether or not their rows
 *                        see a key in it);
 *   LIBRA_COST_PAIRS     the item's eq. 8 pairs.
 * Either way item_overhead is added.  dK/dV items are always costed by the
 * work their kernel executes (see libra_item). */
enum {
  LIBRA_COST_EXECUTED = 0,
  LIBRA_COST_PAIRS = 1
};

#define LIBRA_PLAN_MAGIC 0x4152424Cu   /* "LBRA" little-endian */
#define LIBRA_PLAN_VERSION 5u

/* Planner inputs.  SH-Tiles (Libra technical review, section 5.1, eq. 6)
 * are tile_tokens (B) tokens by tile_heads (W = h_q / H) query heads. */
typedef struct {
  int32_t total_tokens;   /* L >= 0 */
  int32_t num_samples;    /* n >= 0; cu_seqlens holds n + 1 entries */
  int32_t h_q;            /* query heads, a multiple of h_kv */
  int32_t h_kv;           /* key/value heads >= 1 */
  int32_t head_dim;       /* 64 or 128 */
  int32_t tile_tokens;    /* B >= 1: sequence block of an SH-Tile */
  int32_t tile_heads;     /* W >= 1, divides h_q: head shard width */
  int32_t num_cus;        /* workers = persistent workgroups; 0 means 256 */
  float tau;              /* soft-target slack of Algorithm 2 (0.03 on the pages) */
  int32_t assign;         /* LIBRA_ASSIGN_* */
  int64_t item_overhead;  /* cost added to every work item, in query-key slots */
  /* Relative speed of the workers of each class, worker w being of class
   * w mod 8 (on MI355X workgroup w runs on XCD w mod 8), in thousandths; 0
   * means 1000.  Algorithm 2 then sends each unit to the worker that would
   * finish it first, (load + cost) / speed, instead of the least loaded one;
   * equal speeds give exactly the unweighted placement.  libra_worker_speed
   * estimates the speeds from the records of a previous launch. */
  uint16_t worker_speed[8];
  int32_t cost;           /* LIBRA_COST_* for forward and dQ items */
  int32_t reserved;       /* 0 */
} libra_plan_params;

/* One SH-Tile t = (block, shard), tile_id = block * (h_q / W) + shard.
 * Samples sample_first..sample_last are its KV groups K(t) (section 5.2,
 * eq. 7); pairs is its eq. 8 count of unmasked (query, key, head) triples. */
typedef struct {
  int32_t tile_id, block, shard;
  int32_t tok_begin, tok_end;       /* tokens [tok_begin, tok_end) */
  int32_t head_begin, head_count;   /* query heads [head_begin, head_begin + head_count) */
  int32_t sample_first, sample_last;
  int32_t n_items;                  /* forward work items cut from the tile */
  int64_t pairs;
} libra_tile;

/* One unit of work for one persistent workgroup.
 * Forward and dQ items: query rows [row0, row0 + nrows) of heads
 *   [head0, head0 + nheads), all reading KV head kv_head; nheads is 1, 2 or 4
 *   and nrows * nheads <= 384 (forward) or 256 (dQ).
 * dK/dV items (tile_id == -1): key rows [row0, row0 + nrows) of kv_head,
 *   nrows <= 192, gathering the gradient of all h_q / h_kv query heads of
 *   that KV head.
 * Walk order.  A forward or dQ item walks the key blocks of its rows from
 *   the start of its first row's sample up to its last row; a dK/dV item
 *   walks the query blocks its keys see from the end of its last key's
 *   sample down to its first key.  With LIBRA_ITEM_REVERSE in flags the walk
 *   runs the other way.  The planner places items in zigzag pairs (item i
 *   and item m - 1 - i of the m items of one sample, KV head and first head,
 *   in row order) that run back to back, the second reversed: pairs then
 *   cost the same, and pairs started together read the same block at every
 *   step.  A queue whose pairs, placed by least finish time, would leave a
 *   CU more than 0.5 % above the mean load gets single items, none
 *   reversed. */
#define LIBRA_ITEM_REVERSE 1
typedef struct {
  int32_t row0, nrows;
  int32_t kv_head, head0, nheads;
  int32_t tile_id;
  int32_t id;                       /* position in the planner's enumeration */
  int32_t flags;                    /* LIBRA_ITEM_REVERSE or 0 */
  int64_t cost;                     /* placement key (query-key slots): forward and dQ items
                                       by libra_plan_params::cost; dK/dV items by the slots
                                       their kernel executes, g heads x 64-row query blocks
                                       from the first key (rounded down to 64) to the end of
                                       the last key's sample x 64 x nrows; + item_overhead */
  int64_t pairs;                    /* unmasked (query, key, head) triples */
} libra_item;

/* Header at offset 0 of every plan buffer.  Sections follow at the given
 * byte offsets: tiles[n_tiles]; the forward queue, items[n_items] grouped by
 * CU in placement order with cu_off[num_cus + 1] (CSR); the same for the dQ
 * queue and for the dK/dV queue. */
typedef struct {
  uint32_t magic, version;
  uint64_t bytes;
  libra_plan_params params;
  int32_t num_cus;                  /* resolved worker count */
  int32_t n_tiles, n_items, n_dq_items, n_kv_items, reserved;
  int64_t total_pairs;              /* sum of tile pairs = h_q * sum_j l_j (l_j + 1) / 2 */
  int64_t load_max, load_sum;       /* per-CU cost of the forward queue */
  int64_t dq_load_max, dq_load_sum; /* per-CU cost of the dQ queue */
  int64_t kv_load_max, kv_load_sum; /* per-CU cost of the dK/dV queue */
  uint64_t off_tiles, off_items, off_cu_off, off_dq_items, off_dq_cu_off, off_kv_items, off_kv_cu_off;
  uint64_t checksum;                /* FNV-1a over 64-bit words in four interleaved streams
                                       (word i feeds stream i mod 4), folded in order; this
                                       field taken as 0 */
} libra_plan_info;

/* Per-workgroup record of a persistent kernel (optional output).  hw_id and
 * xcc_id identify the physical CU; t_start / t_end are ticks of the
 * constant-rate device clock (libra_device_clock_khz).  flags holds
 * LIBRA_RECORD_PLAN_MISMATCH when the workgroup found that the device copy
 * of the plan is not a copy of the host plan it was launched with (its
 * checksum differs) and therefore ran no item.  In the dK/dV pass it holds
 * LIBRA_RECORD_WAIT_EXPIRED when a wave's bounded wait for the P tile of its
 * partner wave ran out (about 4M cycles); that is a defect, and the launch's
 * dK and dV are not to be trusted.  Zero otherwise. */
#define LIBRA_RECORD_PLAN_MISMATCH 1u
#define LIBRA_RECORD_WAIT_EXPIRED 2u
typedef struct {
  uint32_t hw_id, xcc_id, n_items, flags;
  uint64_t t_start, t_end;
} libra_cu_record;

/* Queues of a plan. */
enum { LIBRA_QUEUE_FWD = 0, LIBRA_QUEUE_DQ = 1, LIBRA_QUEUE_KV = 2 };

/* Speed of each worker class (worker mod 8), in thousandths of the mean,
 * from one completed launch of `queue` of this plan (host function, no device
 * work): class x's rate is the planned cost of its workers over their busy
 * ticks (t_end - t_start of records[w], w < num_cus), and speed_out[x] is
 * 1000 x rate_x / mean rate, clamped to [500, 2000]; classes that ran nothing
 * get 1000.  records: host copy of the launch's num_cus records.
 * LIBRA_EINVAL for a bad plan, queue or pointer. */
libra_status libra_worker_speed(const void *plan_host, int32_t queue, const libra_cu_record *records,
                                uint16_t speed_out[8]);

/* Build a plan on the host (pure function, thread-safe, no device work).
 * cu_seqlens: host int32[num_samples + 1].  buf == NULL: only *bytes is set to
 * the size needed.  Otherwise *bytes is the capacity of buf (8-byte aligned);
 * LIBRA_ESIZE if too small (with *bytes set to the size needed).
 * Tiles follow eq. 6-8 (Libra technical review, section 5); work items are
 * placed on CUs by Algorithm 2 (section 5.4) with no communication term, or
 * round-robin.  Errors: LIBRA_EINVAL for malformed cu_seqlens or parameters,
 * LIBRA_EUNSUPPORTED for head_dim other than 64 or 128. */
libra_status libra_plan(const int32_t *cu_seqlens, const libra_plan_params *params,
                        void *buf, size_t *bytes);

/* Validate a plan buffer of the given size (magic, version, size, section
 * bounds, checksum) and copy its header to *info (may be NULL). */
libra_status libra_plan_check(const void *plan, size_t bytes, libra_plan_info *info);

/* Forward pass.  plan: host plan buffer; plan_dev: its byte copy on the
 * device.  Writes o [L, h_q, d] bf16 and lse [h_q, L] fp32.  softmax_scale > 0
 * (commonly 1/sqrt(head_dim)).  records: NULL or device
 * libra_cu_record[num_cus].  Enqueues one persistent kernel of num_cus
 * workgroups that runs each CU's queue of work items (Libra technical review,
 * section 5.4: the placement decided on the host is only executed here). */
libra_status libra_attn_fwd(const void *plan, const void *plan_dev,
                            const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens_dev, void *o, float *lse,
                            float softmax_scale, libra_cu_record *records, void *stream);

/* Device workspace the backward needs (D = rowsum(dout * o) and LSE * log2(e),
 * fp32 [h_q, L] each), in bytes. */
libra_status libra_attn_bwd_workspace(const void *plan, size_t *bytes);

/* Backward pass: dq [L, h_q, d], dk and dv [L, h_kv, d] (bf16) from q, k, v,
 * the forward's o and lse, and dout.  Reuses the plan's forward assignment
 * for dQ and its key-major queue for dK/dV (Libra paper, section 4.3.3: the
 * backward reuses the forward placement).  records: NULL or device
 * libra_cu_record[2 * num_cus] (dK/dV kernel, then dQ kernel); a dK/dV
 * record with LIBRA_RECORD_WAIT_EXPIRED marks the launch's dk and dv as not
 * to be trusted (a defect, see libra_cu_record). */
libra_status libra_attn_bwd(const void *plan, const void *plan_dev,
                            const void *q, const void *k, const void *v,
                            const void *o, const void *dout, const float *lse,
                            const int32_t *cu_seqlens_dev,
                            void *dq, void *dk, void *dv, float softmax_scale,
                            void *workspace, size_t workspace_bytes,
                            libra_cu_record *records, void *stream);

/* The backward without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, results and errors as libra_attn_bwd,
 * but the workspace is a device array inside the library, one per GPU, of
 * LIBRA_NOALLOC_SCRATCH_BYTES (64 MiB: h_q x L up to 8M, e.g. 32 query heads
 * x 262144 tokens), held on every GPU the library's backward code is loaded
 * on until the process ends.
 * A plan needing more (libra_attn_bwd_workspace) gets LIBRA_ESIZE and nothing
 * is enqueued.  The call allocates nothing (no hipMalloc, no host or library
 * allocation) and synchronises nothing; nothing in the array needs to start
 * at zero, since each call's first phase writes all of it before the later
 * phases read it.  Every call on one GPU shares that GPU's array, so calls
 * whose work overlaps on one GPU (other streams, other threads) race: order
 * them on one stream or with events. */
#define LIBRA_NOALLOC_SCRATCH_BYTES (64u << 20)
libra_status libra_attn_bwd_noalloc(const void *plan, const void *plan_dev,
                                    const void *q, const void *k, const void *v,
                                    const void *o, const void *dout, const float *lse,
                                    const int32_t *cu_seqlens_dev,
                                    void *dq, void *dk, void *dv, float softmax_scale,
                                    libra_cu_record *records, void *stream);

/* The backward in three phases on the same stream (libra_attn_bwd enqueues
 * all three, in this order):
 *   _prepare: computes D = rowsum(dout * o) and LSE * log2(e) (fp32) into the
 *             workspace;
 *   _dkdv:    the key-major persistent kernel writing dk and dv
 *             (records: NULL or libra_cu_record[num_cus]);
 *   _dq:      the query-major persistent kernel writing dq
 *             (records: NULL or libra_cu_record[num_cus]).
 * _dkdv and _dq read the workspace a preceding _prepare filled from the same
 * tensors.  Arguments and errors as for libra_attn_bwd. */
libra_status libra_attn_bwd_prepare(const void *plan, const void *o, const void *dout,
                                    const float *lse, void *workspace, size_t workspace_bytes,
                                    void *stream);
libra_status libra_attn_bwd_dkdv(const void *plan, const void *plan_dev,
                                 const void *q, const void *k, const void *v,
                                 const void *dout, const float *lse,
                                 const int32_t *cu_seqlens_dev, void *dk, void *dv,
                                 float softmax_scale, const void *workspace,
                                 size_t workspace_bytes, libra_cu_record *records, void *stream);
libra_status libra_attn_bwd_dq(const void *plan, const void *plan_dev,
                               const void *q, const void *k, const void *v, const void *dout,
                               const float *lse, const int32_t *cu_seqlens_dev, void *dq,
                               float softmax_scale, const void *workspace,
                               size_t workspace_bytes, libra_cu_record *records, void *stream);

/* ---- Sequence pools (host only) ----------------------------------------
 *
 * Variance-reduced sequence placement, VRSP (Libra technical review,
 * section 4.2, Algorithm 1; Libra paper, section 4.2): the num_seqs packed
 * sequences of one optimizer-step window are split into
 * K = num_seqs / pool_size pools of exactly pool_size sequences each, so that
 * the pools' summed workloads are as even as the heuristic makes them.
 * Sequences are taken in order of decreasing workload (equal workloads by
 * increasing index) and each goes to the least-loaded pool that still has
 * room (equal loads by increasing pool index): the placement is a pure,
 * deterministic function of its inputs.
 */

/* Workload proxy of one packed sequence (Libra technical review, section 3.1,
 * eq. 1): *workload = sum over its samples of (sample length)^2.
 * cu_seqlens: host, num_samples + 1 non-decreasing int32 offsets starting at
 * 0 (empty samples allowed).  LIBRA_EINVAL on a NULL pointer, a negative
 * num_samples or malformed offsets. */
libra_status libra_pack_workload(const int32_t *cu_seqlens, int32_t num_samples, int64_t *workload);

/* VRSP over one window.
 *   workload   host, num_seqs values >= 0 (e.g. from libra_pack_workload);
 *   pool_size  P > 0 dividing num_seqs;
 *   pool_of    host out, num_seqs entries: the pool of sequence i;
 *   order      host out, num_seqs entries: the reordered window S', the
 *              pools in pool order (pool k fills order[k P .. k P + P - 1]),
 *              each pool's sequences in the order they were assigned;
 *   pool_load  host out, K entries, or NULL: each pool's summed workload.
 * All buffers are the caller's; the call allocates nothing on the heap
 * beyond temporaries and touches no device.  LIBRA_EINVAL on a NULL
 * required pointer, num_seqs <= 0, pool_size <= 0, num_seqs not a multiple
 * of pool_size or a negative workload; the outputs are then unspecified. */
libra_status libra_vrsp(const int64_t *workload, int32_t num_seqs, int32_t pool_size, int32_t *pool_of,
                        int32_t *order, int64_t *pool_load);

/* Frequency of the clock in libra_cu_record, for the current device. */
libra_status libra_device_clock_khz(int32_t *khz);

/* Name of the HIP error behind the calling thread's most recent LIBRA_EHIP
 * (e.g. "hipErrorInvalidDeviceFunction"), or "" if this thread has had none.
 * The string is static; the call never fails. */
const char *libra_last_hip_error(void);

/* Static description of a status code. */
const char *libra_status_str(libra_status status);

#ifdef __cplusplus
}
#endif

#endif /* LIBRA_H */
