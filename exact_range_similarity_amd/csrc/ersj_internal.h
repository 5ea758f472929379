// Internal declarations of libersj: device data layout and kernel launchers.
//
// Device layout of an index (n points, d dims, nb = ceil(d/4) dim blocks):
//   xs      float4 [nb][n]   point i's permuted dims 4b..4b+3 at xs[b*n + i]
//                            (dims in descending-variance order, zero padded)
//   orig    u32 [n]          sorted position -> original row id
//   cell_*  per non-empty grid cell, in Morton order of the cell coordinates
//   rstart/rpref             per cell, the candidate ranges of its kept
//                            neighbour cells (merged when contiguous) and the
//                            prefix of their lengths: candidate position p of
//                            the cell maps to point rstart[g] + p - rpref[g]
//   tiles   Tile [T]         row tiles: up to kTileRows rows of one cell
//   toff    u64 [T+1]        first mask word of each tile (all batches)
//   coff    u64 [T+1]        candidates before each tile (sum of rows * U)
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ersj {

constexpr int kTileRows = 128;  // query rows per row tile
// Candidate ranges per cell: at most one per stencil cell, (2R+1)^3 for grid
// reach R <= 2 (cell width eps/R, stencil of 5x5x5 cells at R = 2).
constexpr int kMaxGridReach = 2;
constexpr int kMaxRanges = (2 * kMaxGridReach + 1) * (2 * kMaxGridReach + 1) * (2 * kMaxGridReach + 1);

// Range g holding candidate position p: the largest g < nr with pref[g] <= p
// (pref[0] = 0, ascending).
__device__ __forceinline__ int range_of(const uint32_t *pref, uint32_t nr, uint32_t p)
{
    int lo = 0, hi = (int)nr;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= p) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Block box test.  Rows within a cell follow a fine Morton order, so a few
// consecutive rows (queries, or candidates of a cell's list) are compact on
// the three grid axes, which are the first three dimensions of the layout.
// wave_box: lo = min, hi = max of (x, y, z) over the 64 lanes, in every lane.
__device__ __forceinline__ void wave_box(float4 &lo, float4 &hi)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        lo.x = fminf(lo.x, __shfl_xor(lo.x, o, 64));
        lo.y = fminf(lo.y, __shfl_xor(lo.y, o, 64));
        lo.z = fminf(lo.z, __shfl_xor(lo.z, o, 64));
        hi.x = fmaxf(hi.x, __shfl_xor(hi.x, o, 64));
        hi.y = fmaxf(hi.y, __shfl_xor(hi.y, o, 64));
        hi.z = fmaxf(hi.z, __shfl_xor(hi.z, o, 64));
    }
}

// fp32 sum of squared gaps between two boxes on the grid axes.  Compared
// with RefineArgs::tbox, which covers its rounding: above it no pair of
// points in the two boxes is within eps.
__device__ __forceinline__ float box_gap2(const float *alo, const float *ahi, float4 blo, float4 bhi)
{
    const float gx = fmaxf(0.f, fmaxf(blo.x - ahi[0], alo[0] - bhi.x));
    const float gy = fmaxf(0.f, fmaxf(blo.y - ahi[1], alo[1] - bhi.y));
    const float gz = fmaxf(0.f, fmaxf(blo.z - ahi[2], alo[2] - bhi.z));
    return gx * gx + gy * gy + gz * gz;
}

// Candidate-chunk boxes cover the first kBoxBlocks float4 blocks of the
// variance-ordered layout (dimensions 0-7; zero padding where d is
// smaller): chunk ch has lo, hi of block b at cbox[(ch * kBoxBlocks + b) * 2
// + 0, 1].  The refinement's box test sums the squared gaps of all 8
// dimensions: a term takes one rounded difference and one rounded square,
// (1 + u)^3, and at most 7 rounded additions follow it, so the fp32 sum is
// within (1 + u)^10 < 1 + 2^-20 of the exact one (u = 2^-24), plus less than
// 2^-146 where squares underflow; RefineArgs::tbox covers both.
constexpr int kBoxBlocks = 2;

__device__ __forceinline__ float gap4(float4 alo, float4 ahi, float4 blo, float4 bhi, float acc)
{
    const float gx = fmaxf(0.f, fmaxf(blo.x - ahi.x, alo.x - bhi.x));
    const float gy = fmaxf(0.f, fmaxf(blo.y - ahi.y, alo.y - bhi.y));
    const float gz = fmaxf(0.f, fmaxf(blo.z - ahi.z, alo.z - bhi.z));
    const float gw = fmaxf(0.f, fmaxf(blo.w - ahi.w, alo.w - bhi.w));
    return acc + gx * gx + gy * gy + gz * gz + gw * gw;
}

// lo = min, hi = max of all four components over the 64 lanes, in every lane
__device__ __forceinline__ void wave_box4(float4 &lo, float4 &hi)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        lo.x = fminf(lo.x, __shfl_xor(lo.x, o, 64));
        lo.y = fminf(lo.y, __shfl_xor(lo.y, o, 64));
        lo.z = fminf(lo.z, __shfl_xor(lo.z, o, 64));
        lo.w = fminf(lo.w, __shfl_xor(lo.w, o, 64));
        hi.x = fmaxf(hi.x, __shfl_xor(hi.x, o, 64));
        hi.y = fmaxf(hi.y, __shfl_xor(hi.y, o, 64));
        hi.z = fmaxf(hi.z, __shfl_xor(hi.z, o, 64));
        hi.w = fmaxf(hi.w, __shfl_xor(hi.w, o, 64));
    }
}
constexpr int kMaxDim = 4096;

struct Tile {
    uint32_t cell;
    uint32_t row0;
    uint32_t nrows;
    uint32_t words;  // row stride of the mask in 64-bit words: used, rounded up to kRowAlign
    uint32_t used;   // mask words that hold candidates = ceil(U / 64)
};

// Mask rows start on 64-byte boundaries, so the refinement's 64-byte row
// pieces are whole aligned segments.  Words past `used` are never read.
constexpr uint32_t kRowAlign = 8;

// A pair inside the fp32 uncertainty band, re-evaluated in binary64.
struct Boundary {
    uint32_t q;      // sorted row of the query
    uint32_t x;      // sorted row of the candidate
    uint64_t bit;    // bit address in the batch mask (word * 64 + bit)
};

struct GridParams {
    int32_t dim[3];   // original dimension ids of the grid axes
    double lo[3];
    double w[3];
    int32_t G[3];
    int32_t ndim;     // grid dimensions in use (min(d, 3))
    int32_t bits;     // Morton bits per dimension (coordinates 0 .. G + 1)
    int32_t reach;    // stencil reach R: cell width >= eps / R, offsets in [-R, R]^3
    int32_t sub;      // sub-cell bits per axis: rows within a cell ordered by a 2^sub-per-axis
                      // Morton key (bits + sub <= 21); the cell key is the row key >> 3*sub
};

// ---- index construction (k_index.hip) ----
hipError_t launch_stats(const float *x, int64_t n, int32_t d, int64_t ld, double *partial,
                        uint32_t *bad_partial, int64_t nthreads, double *out_stats,
                        unsigned long long *out_bad, hipStream_t s);
int64_t stats_threads(int64_t n, int32_t d);

// Morton keys of the cells; cell coordinates are stored plus one, so that a
// query of a semi-join one cell outside the points' grid (coordinate -1 or G)
// still has a key.  Points clamp to [0, G-1], queries (`queries` set) to
// [-1, G]: a query further out has no neighbour, and the clamp only adds
// candidates that refinement rejects.
hipError_t launch_keys(const float *x, int64_t n, int64_t ld, const GridParams &gp, bool queries,
                       uint64_t *keys, uint32_t *ids, hipStream_t s);

// LSD radix sort of (key, value) pairs on the low `bits` bits of the keys.
// Result ends in (k0, v0); k1/v1 are scratch of the same size; hist needs
// radix_hist_entries(n) u64 and scan_tmp scan_tmp_entries(radix_hist_entries(n)).
size_t radix_hist_entries(int64_t n);
hipError_t radix_sort(uint64_t *k0, uint32_t *v0, uint64_t *k1, uint32_t *v1, int64_t n, int bits,
                      uint64_t *hist, uint64_t *scan_tmp, hipStream_t s);

// rows orig[i] of x into the dimension-blocked layout xs (n rows per
// block, layout dimension k = input dimension perm[k]), blocks [0, nbw)
hipError_t launch_gather(const float *x, int64_t n, int32_t d, int64_t ld, const uint32_t *orig,
                         const int32_t *perm, int nbw, float4 *xs, hipStream_t s);

// Exclusive scan: out[i] = sum in[0..i), out[n] = total.  tmp needs
// scan_tmp_entries(n) u64.
size_t scan_tmp_entries(int64_t n);
hipError_t scan_u32(const uint32_t *in, uint64_t *out, int64_t n, uint64_t *tmp, hipStream_t s);
hipError_t scan_u64(const uint64_t *in, uint64_t *out, int64_t n, uint64_t *tmp, hipStream_t s);

hipError_t launch_cell_flags(const uint64_t *keys, int64_t n, int shift, uint32_t *flags, hipStream_t s);
hipError_t launch_cell_scatter(const uint64_t *keys, int shift, const uint32_t *flags, const uint64_t *cid,
                               int64_t n, uint32_t *cell_start, uint64_t *cell_key,
                               hipStream_t s);
hipError_t launch_cell_aabb(const float4 *xs, const uint64_t *cid, int64_t n, int64_t M,
                            uint32_t *lo_bits, uint32_t *hi_bits, hipStream_t s);

// Cells of the query rows (home: the points themselves for the self-join)
// against the cells of the points (target).
struct CellSet {
    const uint64_t *key;
    const uint32_t *start;
    const uint32_t *lo_bits, *hi_bits;
    int64_t M;
};
hipError_t launch_chunk_counts(const uint32_t *rpref, const uint32_t *nrng, int64_t M, uint32_t *cnt,
                               hipStream_t s);
// pbox: box of every 8 consecutive sorted points over the first kBoxBlocks
// blocks of xs (n points, nb blocks; ceil(n / 8) groups, layout as cbox);
// cbox: exact box of every 64-candidate chunk of every cell's candidate
// list, from the group boxes and the points of partial groups
// Order of the rows within each cell, from the rows gathered in cell order
// (xs, dimension-blocked): key (cell << 24) | the row's 24-bit code in its
// cell's box over the first kOrderDims layout dimensions, the bits in the
// order midpoint splits of the widest extent take them, value = the row's
// position (box_lo/box_hi/masks: [M][kOrderDims] temporaries; cid: the cell
// scan, cell of position i = cid[i + 1] - 1).  Sorting the keys gives perm;
// launch_permute_rows then moves every block of row perm[i] and its input id
// to position i.
constexpr int kOrderDims = 8;
hipError_t launch_cell_order_keys(const float4 *xs, int64_t n, int nb, const uint64_t *cid, int64_t M,
                                  uint32_t *box_lo, uint32_t *box_hi, uint32_t *masks, uint64_t *keys, uint32_t *vals,
                                  hipStream_t s);
// Balanced tree order of the rows within each cell (k_index.hip): the
// leaves of a binary tree whose nodes split at 32-row multiples by the
// dimension of largest sampled variance among the first kTreeDims layout
// dimensions.  launch_tree_roots makes a node per cell (nstart/nsize [M]),
// pos = 0..n-1 and *maxsz the largest cell; each launch_tree_level (while
// *maxsz > kTreeLeaf) sorts pos within the K nodes and writes the next
// level's nodes (ostart/osize; their count is off[K], off from the counts
// cnt[K]) and their largest size.  Node arrays hold up to n + 1 entries; k0,
// k1, v1, hist, stmp as for radix_sort over n rows.  pos ends as the
// permutation for launch_permute_rows.
constexpr int kTreeLeaf = 32;
constexpr int kTreeDims = 64;
hipError_t launch_tree_roots(const uint32_t *cell_start, int64_t M, uint32_t *nstart, uint32_t *nsize,
                             uint32_t *pos, int64_t n, uint32_t *maxsz, hipStream_t s);
hipError_t launch_tree_level(const float4 *xs, int64_t n, int nb, uint32_t *pos, const uint32_t *nstart,
                             const uint32_t *nsize, uint32_t K, uint32_t *ndim, uint64_t *k0, uint64_t *k1,
                             uint32_t *v1, uint64_t *hist, uint64_t *stmp, uint32_t *cnt, uint64_t *off,
                             uint32_t *ostart, uint32_t *osize, uint32_t *maxsz, hipStream_t s);
hipError_t launch_permute_rows(const float4 *src, const uint32_t *orig_src, const uint32_t *perm, int64_t n, int nb,
                               float4 *dst, uint32_t *orig_dst, hipStream_t s);
hipError_t launch_point_boxes(const float4 *xs, uint64_t n, int nb, float4 *pbox, hipStream_t s);
hipError_t launch_chunk_boxes(const uint64_t *base, int64_t M, uint64_t nchunks, const uint32_t *rstart,
                              const uint32_t *rpref, const uint32_t *nrng, const float4 *xs, uint64_t n, int nb,
                              const float4 *pbox, float4 *cbox, hipStream_t s);
hipError_t launch_stencil(const CellSet &home, const CellSet &target, const GridParams &gp,
                          double prune_e2, uint32_t *rstart, uint32_t *rpref, uint32_t *nrng,
                          uint32_t *tiles_per_cell, unsigned int *umax, hipStream_t s);

hipError_t launch_tiles(const uint64_t *tile_base, int64_t M, int64_t T,
                        const uint32_t *cell_start, const uint32_t *rpref, const uint32_t *nrng,
                        Tile *tiles, uint64_t *words, uint64_t *cands, hipStream_t s);

// Per row tile t: tref[t * nb + b] = per-dimension lower median of up to 32
// of the tile's query rows spread evenly over it (block b of the
// dimension-blocked layout xq, nq rows)
hipError_t launch_tile_ref(const Tile *tiles, int64_t T, const float4 *xq, uint64_t nq, int nb, float4 *tref,
                           hipStream_t s);

// result = {batches, max batch words, failing tile + 1 (0 = ok), max batch rows}
hipError_t launch_plan(const uint64_t *toff, const uint64_t *coff, const Tile *tiles, int64_t T,
                       int64_t n, uint64_t budget_words, uint32_t *bounds, uint64_t *row_bounds,
                       uint64_t *word_bounds, uint64_t *cand_bounds, uint64_t *result,
                       hipStream_t s);

hipError_t launch_order_keys(const Tile *tiles, const uint32_t *rpref, const uint32_t *nrng,
                             int64_t T, const uint32_t *bounds, int32_t nb, int ubits,
                             uint32_t umax, uint64_t *keys, uint32_t *vals, hipStream_t s);

hipError_t launch_fill_u64(uint64_t *p, uint64_t v, int64_t n, hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s);

// ---- refinement (k_refine.hip, k_refine_mfma.hip) ----

// Work item of refinement block b among ntiles * ncol: (tile rank, column),
// where a column is a (candidate segment, row sub-block) pair.
// Items come in groups of kGroupTiles consecutive tile ranks, segment-major
// inside a group, so consecutive items read the same candidate segment.
// Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8);
// the remap hands each XCD runs of kXcdRun consecutive items, so one
// segment is fetched into one XCD's L2 and reused by kGroupTiles tiles.
constexpr uint32_t kGroupTiles = 16;
constexpr uint32_t kXcdRun = 16;
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ void work_item(uint32_t b, uint32_t ntiles, uint32_t nseg, uint32_t *rank,
                                          uint32_t *seg)
{
    const uint64_t B = (uint64_t)ntiles * nseg;  // nseg here counts columns
    const uint64_t span = (uint64_t)kXcds * kXcdRun;
    const uint64_t full = B / span * span;
    uint64_t i = b;
    if (i < full) {
        const uint64_t x = i % kXcds, j = i / kXcds;
        i = (j / kXcdRun) * span + x * kXcdRun + (j % kXcdRun);
    }
    const uint64_t gsz = (uint64_t)kGroupTiles * nseg;
    const uint64_t g = i / gsz, within = i - g * gsz;
    const uint64_t r0 = g * kGroupTiles;
    const uint64_t rg = ntiles - r0 < kGroupTiles ? ntiles - r0 : kGroupTiles;
    *seg = (uint32_t)(within / rg);
    *rank = (uint32_t)(r0 + within % rg);
}

// Band pairs go to kBandLists sub-lists, picked by workgroup, each with its
// own counter on its own 128-byte line: one counter for the whole grid made
// the appends contend on a single address.  Workgroup b uses sub-list
// b % kBandLists, so each sub-list is served by one XCD's L2.
constexpr uint32_t kBandLists = 256;
constexpr uint32_t kBandStride = 16;  // u64 words between two counters
// The re-check's hits and the refinement's skipped comparisons are counted
// in kHitSlots counters each (workgroup b adds to slot b % kHitSlots,
// kBandStride words apart), summed on the host: one counter for the whole
// grid serialised c4's 1.6 M re-check additions.
constexpr uint32_t kHitSlots = 32;

__device__ __forceinline__ unsigned long long *band_counter(unsigned long long *bcount)
{
    return bcount + (uint64_t)(blockIdx.x % kBandLists) * kBandStride;
}
__device__ __forceinline__ Boundary *band_list(Boundary *blist, uint64_t lcap)
{
    return blist + (uint64_t)(blockIdx.x % kBandLists) * lcap;
}

struct RefineArgs {
    const float4 *xs;    // points (candidates), dimension-blocked
    uint64_t n;
    const float4 *xq;    // query rows, same layout (== xs for the self-join)
    uint64_t nqr;
    int32_t nb;
    const Tile *tiles;
    const uint32_t *order;
    uint32_t ord0;       // first entry of `order` for this batch
    uint32_t ntiles;     // tiles in this batch
    uint32_t nseg;       // candidate segments per tile
    uint32_t seg_len;    // candidates per segment (multiple of 512)
    uint32_t nsub;       // row sub-blocks per tile (one work item each)
    const uint32_t *rstart;
    const uint32_t *rpref;
    const uint32_t *nrng;
    const uint64_t *toff;
    uint64_t wbase;      // first mask word of the batch
    uint64_t *mask;
    float tlo, thi;      // fp32 classification thresholds
    float kp, km;        // 1 + K and 1 - K of the MFMA kernel's norm-proportional band
    float kmf;           // 1 - K of the d > 64 filter's partial test (high-half products alone)
    float s16;           // split-fp16 form: power-of-two scale of the centred coordinates
                         // (tlo, thi are then the scaled thresholds)
    float tabs;          // absolute widening of its thresholds (fp16 subnormal parts)
    Boundary *blist;              // kBandLists sub-lists of lcap entries each
    unsigned long long *bcount;   // sub-list c's counter at bcount[c * kBandStride]
    uint64_t lcap;                // entries per sub-list
    float tbox;                   // a query block and a candidate chunk whose boxes have an fp32
                                  // gap^2 sum > tbox hold no pair (inf: off)
    const float4 *cbox;           // MFMA kernels, tbox finite: box of each 64-candidate chunk of
                                  // each cell's candidate list (kBoxBlocks blocks, see above)
    const uint64_t *chunk_base;   // first chunk of each cell
    unsigned long long *skipped;  // comparisons decided by that box test alone (kHitSlots slots)
    uint8_t *gflag;               // per 4 mask words (aligned): 1 if any bit is set, else 0
    uint32_t *rowcnt;             // per query row of the batch: neighbours set in the mask (added)
    uint64_t row_base;            // first query row of the batch
    // split-fp16 operands prepared once per point (k_refine_g16): points and
    // query rows, [slabs][4 parts][rows] x 16 bytes, their norms and their
    // norms over the first kPartialDims dimensions of the layout
    const uint4 *p16, *p16q;
    uint64_t ps, psq;  // their part strides (uint4 elements, prep16_stride of n and nqr)
    const float *n16, *n16q;
    const float *np16, *np16q;
    const float *xb16;  // k_filter16's column bound of each point, n + 1 entries (the last NaN)
    // the filter's int8 form (k_prep8; all four set, or all null for the
    // fp16 form): points' and query rows' operands [4 parts][rows] x 16
    // bytes with part strides ps8, ps8q; column bounds (n + 1 entries, the
    // last INT_MAX) and row starts
    const uint4 *p8, *p8q;
    uint64_t ps8, ps8q;
    const int *xb8, *qs8;
    unsigned long long *partial;  // comparisons decided from those dimensions alone (kHitSlots slots)
    // k_filter16: 32 x 32 blocks still live after that test, handed to
    // k_refine_g16_blocks: kBandLists sub-lists of dcap entries {tile,
    // (candidate position / 32) << 2 | query block, point index of the
    // block's first candidate when its candidates are consecutive points
    // (else ~0), valid candidates of the block (1 .. 32)}, sub-list c counted
    // at dcount[c * kBandStride] (a
    // count past dcap means entries were lost and the batch must be refined
    // again by the tiled kernel)
    uint4 *dlist;
    unsigned long long *dcount;
    uint64_t dcap;
    const uint32_t *dorder;  // k_refine_g16_blocks: entries in this order (dtotal of them), or null
    uint64_t dtotal;
    // MFMA kernels that centre per row tile: reference of tile t at
    // tref[t * nb .. t * nb + nb - 1] (the first query row of the tile when NULL)
    const float4 *tref;
};
hipError_t launch_refine_direct(const RefineArgs &a, hipStream_t s);

// ---- exact kNN (k_knn.hip) ----
struct KnnArgs {
    const Tile *tiles;
    uint32_t t0;                 // first tile of the batch (index order)
    const uint64_t *toff;
    uint64_t wbase;              // first mask word of the batch
    uint64_t row_base;           // first query row of the batch
    const uint64_t *mask;
    const uint8_t *gflag;        // per 4 mask words: any bit set
    const uint32_t *rowcnt;      // neighbours per row of the batch
    const uint32_t *rpref, *rstart, *nrng;
    const uint32_t *orig;        // sorted point -> input row
    const uint32_t *qorig;       // index-order query row -> row of the round's query array
    const uint32_t *qmap;        // row of the round's query array -> query id of the search (NULL: identity)
    const float *xr;             // the points in sorted order, row-major, input dimension order
    const float *xqr;            // the round's queries likewise (sorted query order)
    int32_t ldr;                 // row stride of both: recheck_stride(d)
    int32_t d;
    uint32_t k;
    double e64;                  // the round's fl(eps^2)
    uint32_t *next;              // queries left for the next round
    uint32_t *next_count;
    uint32_t *next_nbrs;         // their neighbour count c at this radius, | (terms << 16)
    double *next_lsum;           // sum of log(eps / dist) over the neighbours at dist > 0 (terms)
    uint32_t *ids;               // [nq][k]
    double *dist;                // [nq][k] or NULL
};
int knn_max_k();
hipError_t launch_knn_select(const KnnArgs &a, uint32_t ntiles, hipStream_t s);
// out row i (stride ldo >= d; columns d .. ldo-1 zero) = q row idx[i]
hipError_t launch_gather_rows(const float *q, int64_t ldq, const uint32_t *idx, uint64_t m, int32_t d,
                              int32_t ldo, float *out, hipStream_t s);

// Fixed device scratch of the allocation-free fill pass (k_scratch.hip):
// kNoallocScratchBytes per device; *out = this device's address of it
// (looked up on the first call for the device, which must be current).
constexpr uint64_t kNoallocScratchBytes = (uint64_t)64 << 20;
hipError_t noalloc_scratch(int dev, void **out);

// row stride of the row-major copies read by the re-check: d rounded up to
// four floats, so that a row is read in 16-byte pieces
inline int32_t recheck_stride(int32_t d) { return (d + 3) & ~3; }

// k_refine_mfma.hip: query blocks of 32 rows per work item (4, 2 or 1)
int refine_mfma_qblocks(int nb);
size_t refine_mfma_lds_bytes(int nb);
hipError_t prepare_refine_mfma(int nb, bool f16);
hipError_t launch_refine_mfma(const RefineArgs &a, bool f16, hipStream_t s);

// k_refine_m16.hip: split-fp16 refinement for nb <= 16 (d <= 64), one row
// tile per work item (nsub = 1), seg_len a multiple of 512 and <= 8192
bool refine_m16_supported(int nb);
hipError_t prepare_refine_m16(int nb);
hipError_t launch_refine_m16(const RefineArgs &a, hipStream_t s);

// k_refine_g16.hip: split-fp16 refinement for nb > 16 on operands prepared by
// launch_prep16 (rows of xs centred by -nrs / s, scaled by s, split; N n
// floats; P needs g16_stages(nb, hh) * 4 * ps uint4, part k of row i at
// P[k * ps + i], ps = prep16_stride(n)); nsub = 1, seg_len a multiple of 512.  hh: high halves only (one product per slab, the wider
// band of the high-part form), for both calls alike.
// k_refine_g16 and k_filter16 test every 32 x 32 block after the first
// kPartialDims dimensions: the squared distance over a subset of the
// dimensions bounds the full one from below
constexpr int kPartialDims = 64;
// the run kernel's order: handed-on blocks grouped by the 2^kHandonGroupBits
// consecutive points holding their first candidate, then by query block
constexpr int kHandonGroupBits = 12;
inline int g16_stages(int nb, bool hh)
{
    const int ns = (nb + 3) / 4;
    return hh ? (ns + 1) / 2 : ns;
}
uint64_t prep16_stride(uint64_t n);
hipError_t launch_prep16(const float4 *xs, uint64_t n, int nb, const float4 *nrs, float s, bool hh, uint4 *P,
                         uint64_t ps, float *N, float *NP, hipStream_t st);
hipError_t prepare_refine_g16(bool hh);
hipError_t launch_refine_g16(const RefineArgs &a, bool hh, hipStream_t s);
// filter over the first kPartialDims dimensions: every 32 x 32 block settled
// there or handed on (a.dlist, required); the mask units of steps with a
// live block zeroed (the batch's unit flags must be clear before)
hipError_t prepare_filter16();
// xb[i] = the filter's column bound of point i (from its norm over the
// first kPartialDims dimensions and 1 - K), xb[n] = NaN
hipError_t launch_col_bounds16(const float *np16, uint64_t n, float kmf, float *xb, hipStream_t st);
// the filter's int8 form: mx = bits of max |x_i - ref_i| over the first
// kPartialDims dimensions (fp32; maxed into *mx, which starts at 0); the
// operands of a point set scaled by S (|x_i - ref_i| S <= 127 for all rows),
// row starts (start, may be null) and column bounds (bound, n + 1 entries,
// may be null) against squared radius E; P needs 4 * ps uint4, ps >= n
hipError_t launch_maxabs8(const float4 *xs, uint64_t n, const float4 *ref, unsigned int *mx, hipStream_t st);
hipError_t launch_prep8(const float4 *xs, uint64_t n, const float4 *ref, double S, double E, uint4 *P, uint64_t ps,
                        int *start, int *bound, hipStream_t st);
hipError_t launch_filter16(const RefineArgs &a, bool hh, hipStream_t s);
// sort keys of the total handed-on blocks (pref: device copy of the
// exclusive prefix of the sub-lists' kept counts, kBandLists + 1 entries):
// (first candidate point >> 10, gend for a block whose candidates are not
// consecutive points) << qbits | (tile << 2 | query block), qbits covering
// 4 x the tile count, with each entry's index in dlist (kBandLists * dcap
// must fit 32 bits)
hipError_t launch_handon_keys(const uint4 *dl, uint64_t dcap, const uint64_t *pref, uint64_t total, int qbits,
                              uint32_t gend, uint64_t *keys, uint32_t *vals, hipStream_t st);
// the blocks handed on (a.dlist), after the filter, on the same stream: in
// the order a.dorder (a.dtotal entries, indices into dlist) when given, else
// sub-list by sub-list
hipError_t launch_refine_g16_blocks(const RefineArgs &a, bool hh, hipStream_t s);

// ---- re-check and compaction (k_expand.hip) ----
// Band-list bookkeeping after a refinement launch: out[0] = entries kept
// (each sub-list's count, clipped to lcap), out[1] = the largest unclipped
// count, lpref[0..kBandLists] = exclusive prefix of the kept counts.
hipError_t launch_band_prefix(const unsigned long long *bcount, uint64_t lcap, uint64_t *lpref,
                              uint64_t *out, hipStream_t s);
// xr, xqr: points and query rows in sorted order, input dimension order,
// row-major, ldr = recheck_stride(d) floats per row, the floats past d zero.
hipError_t launch_recheck(const Boundary *bl, uint64_t lcap, const uint64_t *lpref, uint64_t cnt,
                          const float *xr, const float *xqr, int32_t d, int32_t ldr, double e64, uint64_t *mask,
                          uint8_t *gflag, unsigned long long *nin, uint32_t *rowcnt, uint64_t row_base,
                          hipStream_t s);


hipError_t launch_expand(const Tile *tiles, uint32_t t0, uint32_t ntiles, const uint64_t *toff,
                         uint64_t wbase, uint64_t row_base, const uint64_t *mask, const uint8_t *gflag,
                         const uint64_t *roff, const uint32_t *rstart, const uint32_t *rpref,
                         const uint32_t *nrng, const uint32_t *qorig, const uint32_t *orig,
                         uint32_t *pairs, hipStream_t s);

}  // namespace ersj
