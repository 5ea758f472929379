/*
 * ersj.h -- exact epsilon-distance similarity self-join on AMD Instinct
 * MI355X (gfx950).  C ABI of libersj.so.
 *
 * The operation ("RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
 * Similarity Searches", Sec. II-A, Problem Statement): for a dataset D of n
 * points in d dimensions and a search distance eps, the self-join result R
 * holds every ordered pair (i, j) of point ids whose Euclidean distance is at
 * most eps.  Self pairs (i, i) are included (the selectivity of Sec. V-B,
 * z = (|R| - |D|) / |D|, counts them in |R|), both (i, j) and (j, i) appear,
 * and each pair appears once.  Results are key-value pairs of two 32-bit ids
 * (Sec. II-A1).
 *
 * Exactness.  A pair belongs to R iff D64(x_i, x_j) <= fl64(eps * eps), where
 * D64 is the binary64 sum over the input's dimension order of
 * ((double)x_i[k] - (double)x_j[k])^2, each operation rounded to nearest, no
 * fused multiply-add.  The library classifies pairs in fp32 with a proven
 * error band and re-evaluates every pair inside the band with exactly that
 * binary64 sequence, so the returned set equals this definition bit for bit.
 *
 * Pipeline (search-then-refine, Sec. IV): build_index picks the three
 * highest-variance dimensions (Sec. IV-A), bins points into a uniform grid of
 * cell width >= eps on them, sorts points by the cells' Morton codes and
 * stores them contiguously per cell (Sec. IV-C); count_pass finds for every
 * cell the neighbouring cells that can hold a neighbour and so an upper
 * bound on every query's candidates (the first pass of the two-pass scheme,
 * Sec. IV-D); plan_batches cuts the queries into batches whose result masks
 * fit a memory budget (Sec. IV-D, window batching against free memory);
 * fill_pass refines one batch into a one-bit-per-candidate result mask
 * (Sec. IV-E, IV-F) and compacts the mask into pairs (Sec. IV-F1, Fig. 5).
 *
 * Conventions for every entry point:
 *  - d_* pointers are HIP device memory of the current device; h_* and
 *    plain scalar out-parameters are host memory.
 *  - stream is a hipStream_t (NULL = the default stream).  All device work
 *    of a call is ordered on that stream.  Calls that return host values
 *    synchronise the stream before returning.
 *  - Return value: ERSJ_OK or a negative ERSJ_ERR_* code; no C++ exception
 *    crosses the ABI.  After an error, ersj_last_error() returns a message
 *    (thread-local), and the outputs of that call are unspecified.
 *  - Arguments are validated before any HIP call is made.
 *  - A handle may be used from one host thread at a time.
 */
#ifndef ERSJ_H
#define ERSJ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ERSJ_OK = 0,
    ERSJ_ERR_INVALID_ARG = -1, /* bad pointer, size, eps, or non-finite input */
    ERSJ_ERR_STATE = -2,       /* call out of order (e.g. fill before plan) */
    ERSJ_ERR_HIP = -3,         /* HIP runtime error; message names it */
    ERSJ_ERR_OOM = -4,         /* device allocation failed or max_device_bytes hit */
    ERSJ_ERR_BUDGET = -5,      /* one row tile's mask exceeds the batch budget */
    ERSJ_ERR_CAPACITY = -6,    /* output buffer too small; *n_pairs = required */
    ERSJ_ERR_SCRATCH = -7,     /* ersj_fill_pass_noalloc: the batch does not fit the fixed scratch */
    ERSJ_ERR_INTERNAL = -8     /* an invariant of the library failed (message names it) */
};

typedef struct ersj_index ersj_index; /* opaque; owns all its device memory */

/* Refinement kernels (Sec. IV-E).  Both return identical pair sets. */
enum {
    ERSJ_REFINE_AUTO = 0,   /* library's choice: MFMA16 where admissible, else MFMA, else DIRECT */
    ERSJ_REFINE_DIRECT = 1, /* fp32 sum of squared differences on the vector ALUs */
    ERSJ_REFINE_MFMA = 2,   /* |q|^2 + |x|^2 - 2 q.x with the dot products on MFMA */
    ERSJ_REFINE_MFMA16 = 3  /* the same with each centred coordinate split into fp16 high and low
                               parts (hi.hi + hi.lo + lo.hi on fp16 MFMA, fp32 accumulation) and a
                               correspondingly wider band */
};

typedef struct ersj_options {
    uint32_t struct_size;       /* sizeof(ersj_options) of the caller */
    int32_t refine_kernel;      /* ERSJ_REFINE_* */
    double cell_width_scale;    /* grid cell width = eps * max(1, scale); default 1 */
    uint64_t max_device_bytes;  /* cap on library-owned device memory; 0 = none */
    uint64_t boundary_capacity; /* initial boundary-pair list entries over all 256 sub-lists (grown and
                                   the batch refined again on overflow); 0 = default */
    int32_t timing;             /* nonzero: record HIP events around each phase */
    int32_t grid_reach;         /* 0 or 1: cells of width >= eps and the 27-cell stencil; 2: cells of
                                   width >= eps/2 and a 5x5x5 stencil, fewer candidates (tighter
                                   pruning, more cells) with the same result */
    int32_t block_prune;        /* 0 or 1: a block of queries and a group of candidates (MFMA kernels:
                                   32 x 64, direct kernel: 8 x 256) whose bounding boxes over the
                                   first 8 dimensions of the variance order are farther apart than
                                   eps skip their distance computations and get zero mask bits;
                                   -1: off.  Same result. */
    int32_t cell_order;         /* order of the rows within a cell (Sec. IV-B groups points so that
                                   each group has a tight box): 1 = Morton order of 8 x 8 x 8
                                   sub-cells on the grid axes; 2 = the leaf order of a kd-tree over
                                   the cell's own box in the first 8 dimensions of the variance
                                   order, each of its 24 levels halving the widest remaining
                                   extent, which lets the MFMA kernels' block box test (and above
                                   64 dimensions the split form's partial test) settle more;
                                   3 = the leaf order of a balanced binary tree (the equal-count
                                   grouping of the Sec. IV-B kd-tree): each node splits at a
                                   multiple of 32 rows by the dimension, among the first 64 of the
                                   variance order, whose values vary most over the node's rows, so
                                   32-row blocks of clustered data in many dimensions hold few
                                   clusters; 0 = 3 above 64 dimensions and 2 up to 64 where an MFMA
                                   kernel refines, else 1.  Same result. */
    int32_t mfma_products;      /* split-fp16 form above 64 dimensions: 3 = the three products
                                   hi.hi + hi.lo + lo.hi of each 16-dimension slab; 1 = hi.hi alone,
                                   a third of the matrix work and half the operand traffic, with a
                                   band about 4.5 times as wide (more pairs re-checked in binary64);
                                   0 = 1.  Same result. */
    int32_t filter_bits;        /* operands of the 64-dimension filter above 64 dimensions: 8 = int8
                                   values of the centred, scaled coordinates (two int8 MFMAs of 32
                                   dimensions a 32 x 32 block, exact integer sums, a wider but
                                   rigorous bound); 16 = the fp16 high halves (four MFMAs a block);
                                   0 = 8 (16 where the coordinates' range is not finite).  Same
                                   result. */
} ersj_options;

typedef struct ersj_stats {
    int64_t n;                   /* points */
    int32_t d;                   /* dimensions */
    int32_t index_dims[3];       /* original ids of the grid dimensions (-1: unused) */
    int32_t grid[3];             /* cells per grid dimension */
    int32_t refine_kernel;       /* kernel used (ERSJ_REFINE_DIRECT or _MFMA) */
    int64_t cells;               /* non-empty grid cells */
    int64_t tiles;               /* row tiles (up to 128 query rows of one cell) */
    uint64_t total_candidates;   /* sum over queries of the candidate upper bound */
    uint64_t total_mask_words;   /* 64-bit mask words over all batches */
    int32_t n_batches;           /* from the last plan_batches */
    int32_t last_batch;          /* batch of the last fill_pass (-1: none) */
    uint64_t max_batch_words;    /* largest batch mask in 64-bit words */
    uint64_t last_batch_candidates; /* candidates refined by the last fill_pass */
    uint64_t last_batch_pairs;   /* pairs produced by the last fill_pass */
    uint64_t last_boundary_pairs;/* pairs in the fp32 band, re-checked in fp64 */
    uint64_t last_recheck_in;    /* of those, pairs found to be neighbours */
    uint64_t device_bytes;       /* device memory held by the handle */
    /* phase times in ms, accumulated since build (only with options.timing) */
    double build_ms, count_ms, plan_ms, refine_ms, recheck_ms, expand_ms;
    int64_t refine_launches;     /* refine kernel launches timed in refine_ms */
    uint64_t refined_candidates; /* candidates refined in those launches */
    int64_t n_queries;           /* query rows: n for the self-join, nq after ersj_set_queries */
    uint64_t last_skipped;       /* comparisons of the last fill_pass decided by the block box test */
    uint64_t skipped_candidates; /* the same, over the launches timed in refine_ms */
    int32_t mfma_products;       /* products per slab of the split-fp16 form (1 or 3; 0: other forms) */
    uint64_t last_partial;       /* comparisons of the last fill_pass decided "out" from the first 64
                                    dimensions alone (split form above 64 dimensions) */
    uint64_t partial_candidates; /* the same, over the launches timed in refine_ms */
    int32_t last_filtered;       /* 1: the last fill_pass refined with the 64-dimension filter and the
                                    block kernel (above 64 dimensions), 0: with one kernel */
    int32_t filter_bits;         /* operands of that filter: 8 (int8), 16 (fp16); 0: no filter */
} ersj_stats;

/* Fill *opt with the defaults (struct_size set). */
void ersj_default_options(ersj_options *opt);

/*
 * Build the grid index over d_x (Sec. IV-A to IV-C).
 *  d_x  : device, n rows of d floats, row r at d_x + r*ld; borrowed only for
 *         the duration of the call (the stream is synchronised on return).
 *  n    : 1 <= n <= 2^32 - 1;  d: 1 <= d <= 4096;  ld >= d.
 *  eps  : >= 0 (may be +inf; NaN rejected).
 *  opt  : NULL for defaults.
 *  out  : receives a new handle (freed by ersj_free).
 * Errors: INVALID_ARG (also for NaN/inf coordinates, detected on the device),
 *         HIP, OOM.
 */
int ersj_build_index(const float *d_x, int64_t n, int32_t d, int64_t ld, double eps,
                     const ersj_options *opt, void *stream, ersj_index **out);

/*
 * Semi-join (Sec. II-A: a query set Q distinct from the dataset D, the pair
 * (q_j, p_i) in the result iff dist(p_i, q_j) <= eps; Sec. IV-D, Fig. 3(d):
 * a query's candidates are the points of the index cells around it).  Bins
 * the nq query rows into the index's grid; count_pass, plan_batches and
 * fill_pass then work on these queries and fill_pass returns pairs (query
 * row id in d_q, point id).  Without this call the queries are the points
 * (the self-join).  Calling it again replaces the queries; either way the
 * previous count and plan are discarded.
 *  d_q : device, nq rows of d floats (d of the index), row r at d_q + r*ldq;
 *        borrowed for the duration of the call (the stream is synchronised).
 *  nq  : 1 <= nq <= 2^32 - 1;  ldq >= d.
 * Errors: INVALID_ARG (also non-finite coordinates, and an explicitly chosen
 *         MFMA kernel that the query coordinates make unusable), STATE (index
 *         not built), HIP, OOM.  On error the handle is back in the self-join
 *         state, built and not counted.
 */
int ersj_set_queries(ersj_index *h, const float *d_q, int64_t nq, int64_t ldq, void *stream);

/*
 * Count pass (Sec. IV-D, "First Intersection Test" and pass 1): for each
 * cell keep the neighbouring cells whose boxes can hold a neighbour; every
 * query's candidate count is the size of its cell's kept cells.
 *  total_candidates: host out, sum over all queries (may be NULL).
 * Errors: INVALID_ARG, STATE (index not built), HIP, OOM.
 */
int ersj_count_pass(ersj_index *h, uint64_t *total_candidates, void *stream);

/*
 * Cut the queries (in index order, whole row tiles) into batches whose
 * result masks (one bit per candidate, Sec. IV-F) fit budget_bytes
 * (Sec. IV-D: queries are accumulated while the total stays within the
 * budget).  budget_bytes = 0 uses 3/4 of the device's free memory.
 *  n_batches: host out.
 * Errors: INVALID_ARG, STATE (count_pass not run), BUDGET (a single row
 *         tile's mask exceeds the budget), HIP, OOM.
 */
int ersj_plan_batches(ersj_index *h, uint64_t budget_bytes, int32_t *n_batches, void *stream);

/*
 * Refine batch `batch` and write its result pairs (Sec. IV-E, IV-F).
 *  d_pairs : device, room for `capacity` pairs of two uint32 (query id,
 *            point id), original row ids, interleaved; may be NULL when
 *            capacity is 0.
 *  n_pairs : host out, the batch's pair count.
 * The union over all batches is R, each pair once.  Order within a batch is
 * index order of the query, then candidate order.
 * If capacity < pair count the call returns CAPACITY with *n_pairs set to the
 * pair count and writes nothing; calling again for the same batch with a
 * larger buffer only re-runs the final compaction.
 * Errors: INVALID_ARG, STATE (plan_batches not run), CAPACITY, HIP, OOM.
 */
int ersj_fill_pass(ersj_index *h, int32_t batch, uint32_t *d_pairs, uint64_t capacity,
                   uint64_t *n_pairs, void *stream);

/*
 * fill_pass with delivery to host memory (the pages' response time includes
 * the results' transfer to the host, Sec. IV-D and V): the batch is refined
 * and compacted on `stream` into one of two device staging buffers
 * (alternating by batch), and copied into host_pairs on a copy stream of the
 * handle's own, so the copy of batch b overlaps the refinement of batch b+1.
 * Returns once the copy is enqueued: host_pairs is complete only after
 * ersj_host_sync.  host_pairs should be pinned (hipHostMalloc, or a torch
 * tensor with pin_memory=True) for the copy to run asynchronously; pageable
 * memory works but copies synchronously.  The caller keeps host_pairs alive
 * until ersj_host_sync (or ersj_free) returns.  Pair layout, CAPACITY and the
 * other errors as for ersj_fill_pass; the staging buffers are allocated on
 * demand.
 */
int ersj_fill_pass_host(ersj_index *h, int32_t batch, uint32_t *host_pairs, uint64_t capacity,
                        uint64_t *n_pairs, void *stream);

/*
 * ersj_fill_pass for callers that cannot allocate device memory (code that
 * must not call hipMalloc, such as work prepared for stream capture, tight
 * serving loops, or harnesses that forbid allocation).  Same arguments,
 * result and errors as ersj_fill_pass, but the batch's working memory (its
 * result mask and unit flags, row counts and offsets, counters and band
 * list) comes from a fixed device array of ERSJ_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends; the call
 * allocates nothing.  The caller still provides d_pairs.
 *  - A batch whose working memory exceeds the scratch is rejected with
 *    ERSJ_ERR_SCRATCH before any device work: plan with
 *    budget_bytes <= ERSJ_NOALLOC_MASK_BUDGET (mask words cost 8.25 bytes,
 *    and the rows of a batch 20 bytes each on top).  A band list that
 *    outgrows what remains of the scratch is ERSJ_ERR_SCRATCH as well.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (each call clears what it needs): calls that overlap
 *    on one GPU, from any thread, handle or stream, race.
 *  - On CAPACITY a retry refines the batch again (nothing is kept between
 *    calls).  The handle's own buffers and ersj_fill_pass are untouched.
 */
#define ERSJ_NOALLOC_SCRATCH_BYTES ((uint64_t)64 << 20)
#define ERSJ_NOALLOC_MASK_BUDGET ((uint64_t)48 << 20)
int ersj_fill_pass_noalloc(ersj_index *h, int32_t batch, uint32_t *d_pairs, uint64_t capacity,
                           uint64_t *n_pairs, void *stream);

/* Wait until every copy started by ersj_fill_pass_host has landed in host
 * memory.  Errors: INVALID_ARG, HIP. */
int ersj_host_sync(ersj_index *h);

/*
 * Exact k nearest neighbours by growing similarity searches (Sec. VI: the
 * kNN problem recast as distance similarity searches whose radius grows until
 * k neighbours are found, which stays exact with three indexed dimensions).
 * The k nearest neighbours of a query are the k points with the smallest
 * D64 (the canonical binary64 squared distance of the join), ties broken by
 * the smaller point id.
 *  d_x, n, d, ld : the points, as for ersj_build_index.
 *  d_q, nq, ldq  : device query rows (row-major, d floats each); d_q = NULL
 *                  searches the points themselves (nq and ldq are ignored): a
 *                  point is then its own first neighbour unless an identical
 *                  point has a smaller id.  Query rows borrowed for the call.
 *  k             : 1 <= k <= min(n, 1024).
 *  eps0          : radius of the first round, > 0 (+inf: one round in which
 *                  every point is a candidate).
 *  growth        : > 1: each round multiplies the radius by it; 0: the next
 *                  radius is estimated from the queries still short of k
 *                  neighbours (their counts and, pooled, the maximum-likelihood
 *                  local dimension of Levina and Bickel, d when nothing can
 *                  be estimated): enough for 95% of them, held back so that
 *                  no more than 10% are predicted to exceed 1024 neighbours,
 *                  factor in [1.02, 4] ([2, 4] after 20 rounds).
 *  opt           : as for ersj_build_index (NULL: defaults).
 *  d_ids         : device [nq][k] uint32, row q = its neighbours' input row
 *                  numbers, nearest first.
 *  d_dist2       : device [nq][k] double, their D64 values, or NULL.
 *  info          : host out (may be NULL).
 * Round r searches only the queries that still lack k neighbours, as a
 * semi-join against the points with its own index; a query with c >= k
 * neighbours takes the k smallest keys among them (every closer point lies
 * within the radius).  After 40 rounds, or once the radius overflows, the
 * radius becomes +inf, where every query has all n points as neighbours, so
 * the search always ends.  No pair list is written: each round needs the
 * memory of a semi-join's index and result mask.
 * Errors: INVALID_ARG (also non-finite coordinates), HIP, OOM, BUDGET.
 */
#define ERSJ_KNN_MAX_ROUNDS 41
typedef struct ersj_knn_info {
    int32_t rounds;                             /* rounds run */
    int32_t refine_kernel;                      /* ERSJ_REFINE_* used (last round) */
    double eps[ERSJ_KNN_MAX_ROUNDS];            /* radius of round r */
    int64_t queries[ERSJ_KNN_MAX_ROUNDS];       /* queries searched in round r */
    uint64_t candidates[ERSJ_KNN_MAX_ROUNDS];   /* candidates refined in round r */
    double dim_estimate[ERSJ_KNN_MAX_ROUNDS];   /* local dimension estimated after round r (0: none) */
    uint64_t total_candidates;
    /* with options.timing (ms, summed over rounds; HIP events on the stream) */
    double index_ms;                            /* index builds, query binning, counts, plans */
    double refine_ms;                           /* refinement kernel launches */
    double recheck_ms;                          /* binary64 re-check and per-row counts */
    double select_ms;                           /* ranking kernel */
    int64_t refine_launches;
    uint64_t computed_candidates;               /* candidates refined minus those the box test decided */
} ersj_knn_info;

int ersj_knn(const float *d_x, int64_t n, int32_t d, int64_t ld, const float *d_q, int64_t nq,
             int64_t ldq, int32_t k, double eps0, double growth, const ersj_options *opt,
             uint32_t *d_ids, double *d_dist2, ersj_knn_info *info, void *stream);

/* Rows covered by a batch (index order) and its mask size.  Host outputs. */
int ersj_batch_info(const ersj_index *h, int32_t batch, uint64_t *first_row, uint64_t *n_rows,
                    uint64_t *mask_words);

/* Counters and phase times of the handle (host out). */
int ersj_get_stats(const ersj_index *h, ersj_stats *out);

/* Release the handle and all device memory it owns.  NULL is a no-op.  The
 * library keeps released blocks (per device, up to half of its memory) and
 * hands them out again to allocations of the same size; ersj_release_cached
 * returns them to the HIP runtime. */
void ersj_free(ersj_index *h);

/* Return the device memory that the library keeps for reuse on a device
 * (blocks released by ersj_free and by earlier passes) to the HIP runtime, so
 * that other allocators (torch's included) can use it.  Handles stay valid:
 * memory they own is not touched.
 *  device   : HIP device ordinal, or -1 for the calling thread's current one.
 *  released : host out (may be NULL): bytes freed.
 * Waits for the device to finish enqueued work first (a released block may
 * still be read by it).  Errors: ERSJ_ERR_INVALID_ARG for an ordinal that is
 * not a device, ERSJ_ERR_HIP if the device cannot be selected. */
int ersj_release_cached(int32_t device, uint64_t *released);

/* Message of the last failed call on this thread ("" if none). */
const char *ersj_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ERSJ_H */
