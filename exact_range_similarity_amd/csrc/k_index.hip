// Index construction kernels for gfx950: per-dimension statistics, grid
// Morton keys, LSD radix sort, point gather into the dimension-blocked
// layout, cell boundaries and boxes, the 27-cell stencil with box pruning,
// row tiles, device-wide scans and the batch planner.
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches".  Sec. IV-A picks the indexing dimensions by variance;
// Sec. IV-B/IV-C group nearby points and store each group contiguously, the
// groups in Morton order; Sec. IV-D counts candidates per query in a first
// pass, builds a prefix sum over the counts and accumulates queries into
// batches whose storage fits the free memory.  Here the groups are the
// non-empty cells of a uniform grid over three dimensions (a grid index
// searches the 3^k neighbouring cells, Sec. II-B1) and the box lower bound
// used to drop neighbour cells is the one of "JZ-tree", Sec. III-B, eq. (15).
#include "ersj_internal.h"

#include <algorithm>
#include <cmath>
#include <cfloat>

namespace ersj {

namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ uint64_t spread3(uint64_t x)
{
    x &= 0x1fffffull;
    x = (x | (x << 32)) & 0x1f00000000ffffull;
    x = (x | (x << 16)) & 0x1f0000ff0000ffull;
    x = (x | (x << 8)) & 0x100f00f00f00f00full;
    x = (x | (x << 4)) & 0x10c30c30c30c30c3ull;
    x = (x | (x << 2)) & 0x1249249249249249ull;
    return x;
}

__device__ __forceinline__ uint64_t compact3(uint64_t x)
{
    x &= 0x1249249249249249ull;
    x = (x ^ (x >> 2)) & 0x10c30c30c30c30c3ull;
    x = (x ^ (x >> 4)) & 0x100f00f00f00f00full;
    x = (x ^ (x >> 8)) & 0x1f0000ff0000ffull;
    x = (x ^ (x >> 16)) & 0x1f00000000ffffull;
    x = (x ^ (x >> 32)) & 0x1fffffull;
    return x;
}

// Order-preserving map of a float's bits onto uint32 (for atomic min/max).
__device__ __forceinline__ uint32_t f2ord(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o)
{
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

inline unsigned grid_for(int64_t n, int block = kBlock)
{
    int64_t g = (n + block - 1) / block;
    return (unsigned)(g < 1 ? 1 : g);
}

// ---------------------------------------------------------------- stats --
// Thread g owns dimension g % d and rows g/d, g/d + step, ...; the thread
// count is d*step, so every thread sees a single dimension.
__global__ __launch_bounds__(kBlock) void k_stats_partial(const float *__restrict__ x, int64_t n,
                                                          int32_t d, int64_t ld, int64_t T,
                                                          double *__restrict__ part,
                                                          uint32_t *__restrict__ badp)
{
    int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= T) return;
    const int32_t k = (int32_t)(g % d);
    const int64_t step = T / d;
    const double shift = (double)x[k];
    double s = 0.0, s2 = 0.0;
    float mn = FLT_MAX, mx = -FLT_MAX;
    uint32_t bad = 0;
    for (int64_t r = g / d; r < n; r += step) {
        float v = x[r * ld + k];
        if (!isfinite(v)) {
            ++bad;
            continue;
        }
        double t = (double)v - shift;
        s += t;
        s2 += t * t;
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    part[g * 4 + 0] = s;
    part[g * 4 + 1] = s2;
    part[g * 4 + 2] = mn;
    part[g * 4 + 3] = mx;
    badp[g] = bad;
}

// One block per dimension: out[k*4 + {0,1,2,3}] = mean, variance, min, max.
__global__ __launch_bounds__(kBlock) void k_stats_final(const float *__restrict__ x, int64_t n,
                                                        int32_t d, int64_t T,
                                                        const double *__restrict__ part,
                                                        const uint32_t *__restrict__ badp,
                                                        double *__restrict__ out,
                                                        unsigned long long *__restrict__ bad_total)
{
    __shared__ double ss[kBlock], ss2[kBlock], smn[kBlock], smx[kBlock];
    __shared__ unsigned long long sb[kBlock];
    const int32_t k = blockIdx.x;
    const int64_t step = T / d;
    double s = 0.0, s2 = 0.0, mn = DBL_MAX, mx = -DBL_MAX;
    unsigned long long b = 0;
    for (int64_t j = threadIdx.x; j < step; j += blockDim.x) {
        int64_t g = j * d + k;
        s += part[g * 4 + 0];
        s2 += part[g * 4 + 1];
        mn = fmin(mn, part[g * 4 + 2]);
        mx = fmax(mx, part[g * 4 + 3]);
        b += badp[g];
    }
    ss[threadIdx.x] = s;
    ss2[threadIdx.x] = s2;
    smn[threadIdx.x] = mn;
    smx[threadIdx.x] = mx;
    sb[threadIdx.x] = b;
    __syncthreads();
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            ss[threadIdx.x] += ss[threadIdx.x + w];
            ss2[threadIdx.x] += ss2[threadIdx.x + w];
            smn[threadIdx.x] = fmin(smn[threadIdx.x], smn[threadIdx.x + w]);
            smx[threadIdx.x] = fmax(smx[threadIdx.x], smx[threadIdx.x + w]);
            sb[threadIdx.x] += sb[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double shift = (double)x[k];
        const double m = ss[0] / (double)n;
        out[k * 4 + 0] = shift + m;
        out[k * 4 + 1] = fmax(0.0, ss2[0] / (double)n - m * m);
        out[k * 4 + 2] = smn[0];
        out[k * 4 + 3] = smx[0];
        atomicAdd(bad_total, sb[0]);
    }
}

// ----------------------------------------------------------------- keys --
// Cell coordinate c = floor(t), t = (x - lo) / w in binary64, clamped to
// [0, G-1] for points and to [-1, G] for semi-join queries, stored as c + 1.
// With w >= eps * (1 + 2^-20) / R two coordinates of a neighbour pair land in
// cells at most R apart, so the (2R+1)^3 stencil is exhaustive.  The row key
// interleaves c + 1 followed by the sub-cell coordinate floor(t * 2^sub) -
// c * 2^sub (exact: scaling by a power of two), so rows sort by cell and,
// within a cell, along a finer Morton curve; a clamped coordinate takes the
// sub-cell at its clamped end.
__global__ __launch_bounds__(kBlock) void k_keys(const float *__restrict__ x, int64_t n, int64_t ld,
                                                 GridParams gp, int queries, uint64_t *__restrict__ keys,
                                                 uint32_t *__restrict__ ids)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t nsub = (int64_t)1 << gp.sub;
    uint64_t key = 0;
    for (int a = 0; a < gp.ndim; ++a) {
        const double v = (double)x[i * ld + gp.dim[a]];
        const double t = (v - gp.lo[a]) / gp.w[a];
        const double c = floor(t);
        const double cmin = queries ? -1.0 : 0.0;
        const double cmax = queries ? (double)gp.G[a] : (double)(gp.G[a] - 1);
        int64_t ci, si;
        if (!(c > cmin)) {  // also NaN-free: x is finite
            ci = (int64_t)cmin;
            si = c < cmin ? 0 : (int64_t)(floor(t * (double)nsub) - c * (double)nsub);
        } else if (c >= cmax) {
            ci = (int64_t)cmax;
            si = c > cmax ? nsub - 1 : (int64_t)(floor(t * (double)nsub) - c * (double)nsub);
        } else {
            ci = (int64_t)c;
            si = (int64_t)(floor(t * (double)nsub) - c * (double)nsub);
        }
        si = si < 0 ? 0 : (si >= nsub ? nsub - 1 : si);
        key |= spread3((uint64_t)(((ci + 1) << gp.sub) | si)) << a;
    }
    keys[i] = key;
    ids[i] = (uint32_t)i;
}

// ----------------------------------------------------------- radix sort --
constexpr int kRsItems = 16;
constexpr int kRsTile = kBlock * kRsItems;

__global__ __launch_bounds__(kBlock) void k_radix_hist(const uint64_t *__restrict__ keys, int64_t n,
                                                       int shift, int64_t nblk,
                                                       uint64_t *__restrict__ hist)
{
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRsTile;
    for (int r = 0; r < kRsItems; ++r) {
        int64_t i = base + r * kBlock + threadIdx.x;
        if (i < n) atomicAdd(&h[(keys[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter: within a block the items are ranked in input order, round
// by round (256 items per round), with wave ballots matching equal digits.
__global__ __launch_bounds__(kBlock) void k_radix_scatter(const uint64_t *__restrict__ kin,
                                                          const uint32_t *__restrict__ vin,
                                                          uint64_t *__restrict__ kout,
                                                          uint32_t *__restrict__ vout, int64_t n,
                                                          int shift, int64_t nblk,
                                                          const uint64_t *__restrict__ offs)
{
    __shared__ uint64_t s_off[256];
    __shared__ uint32_t s_wc[4][256];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    s_off[tid] = offs[(int64_t)tid * nblk + blockIdx.x];
    for (int w = 0; w < 4; ++w) s_wc[w][tid] = 0;
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t base = (int64_t)blockIdx.x * kRsTile;
    for (int r = 0; r < kRsItems; ++r) {
        const int64_t i = base + r * kBlock + tid;
        const bool valid = i < n;
        uint64_t k = 0;
        uint32_t v = 0;
        if (valid) {
            k = kin[i];
            v = vin[i];
        }
        const uint32_t dig = (uint32_t)(k >> shift) & 255u;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < 8; ++b) {
            const bool bit = (dig >> b) & 1u;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint32_t rank = __popcll(peers & lt);
        if (valid && rank == 0) s_wc[wave][dig] = __popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pre = 0;
            for (int w = 0; w < wave; ++w) pre += s_wc[w][dig];
            const uint64_t pos = s_off[dig] + pre + rank;
            kout[pos] = k;
            vout[pos] = v;
        }
        __syncthreads();
        s_off[tid] += (uint64_t)s_wc[0][tid] + s_wc[1][tid] + s_wc[2][tid] + s_wc[3][tid];
        for (int w = 0; w < 4; ++w) s_wc[w][tid] = 0;
        __syncthreads();
    }
}

// ----------------------------------------------------------------- scan --
constexpr int kScItems = 16;
constexpr int kScTile = kBlock * kScItems;

template <typename T>
__global__ __launch_bounds__(kBlock) void k_scan_reduce(const T *__restrict__ in, int64_t n,
                                                        uint64_t *__restrict__ bsum)
{
    __shared__ uint64_t sw[kBlock / 64];
    const int64_t base = (int64_t)blockIdx.x * kScTile;
    uint64_t v = 0;
    for (int r = 0; r < kScItems; ++r) {
        int64_t i = base + r * kBlock + threadIdx.x;
        if (i < n) v += (uint64_t)in[i];
    }
    for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
    if ((threadIdx.x & 63) == 0) sw[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) bsum[blockIdx.x] = sw[0] + sw[1] + sw[2] + sw[3];
}

// Block-wide exclusive scan of one value per thread; returns the prefix and
// sets *total.
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t v, uint64_t *sw, uint64_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t inc = v;
    for (int o = 1; o < 64; o <<= 1) {
        uint64_t t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) sw[wave] = inc;
    __syncthreads();
    uint64_t pre = 0, tot = 0;
    for (int w = 0; w < kBlock / 64; ++w) {
        if (w < wave) pre += sw[w];
        tot += sw[w];
    }
    __syncthreads();
    *total = tot;
    return pre + inc - v;
}

__global__ __launch_bounds__(kBlock) void k_scan_top(uint64_t *__restrict__ bsum, int64_t nb)
{
    __shared__ uint64_t sw[kBlock / 64];
    uint64_t carry = 0;
    for (int64_t s = 0; s < nb; s += kBlock) {
        int64_t i = s + threadIdx.x;
        uint64_t v = i < nb ? bsum[i] : 0, tot;
        uint64_t ex = block_excl_scan(v, sw, &tot);
        if (i < nb) bsum[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) bsum[nb] = carry;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_scan_down(const T *__restrict__ in, int64_t n,
                                                      const uint64_t *__restrict__ bsum, int64_t nb,
                                                      uint64_t *__restrict__ out)
{
    __shared__ uint64_t st[kScTile];
    __shared__ uint64_t sw[kBlock / 64];
    const int64_t base = (int64_t)blockIdx.x * kScTile;
    for (int r = 0; r < kScItems; ++r) {
        int64_t i = base + r * kBlock + threadIdx.x;
        st[r * kBlock + threadIdx.x] = i < n ? (uint64_t)in[i] : 0;
    }
    __syncthreads();
    uint64_t loc[kScItems];
    uint64_t s = 0;
    for (int j = 0; j < kScItems; ++j) {
        loc[j] = s;
        s += st[threadIdx.x * kScItems + j];
    }
    uint64_t tot;
    const uint64_t pre = block_excl_scan(s, sw, &tot) + bsum[blockIdx.x];
    for (int j = 0; j < kScItems; ++j) st[threadIdx.x * kScItems + j] = pre + loc[j];
    __syncthreads();
    for (int r = 0; r < kScItems; ++r) {
        int64_t i = base + r * kBlock + threadIdx.x;
        if (i < n) out[i] = st[r * kBlock + threadIdx.x];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) out[n] = bsum[nb];
}

template <typename T>
hipError_t scan_impl(const T *in, uint64_t *out, int64_t n, uint64_t *tmp, hipStream_t s)
{
    const int64_t nb = (n + kScTile - 1) / kScTile;
    if (nb == 0) return launch_fill_u64(out, 0, 1, s);
    hipLaunchKernelGGL(k_scan_reduce<T>, dim3((unsigned)nb), dim3(kBlock), 0, s, in, n, tmp);
    hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(kBlock), 0, s, tmp, nb);
    hipLaunchKernelGGL(k_scan_down<T>, dim3((unsigned)nb), dim3(kBlock), 0, s, in, n, tmp, nb, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------- gather --
// Rows orig[i] of x (row-major, stride ld) into the dimension-blocked,
// variance-ordered layout: block b of row i holds input dimensions
// perm[4b .. 4b + 3] (0 past d).
//
// Narrow rows (up to 64 dimensions): a thread per output row, its blocks
// in turn (the row's few cache lines serve all of them).
__global__ __launch_bounds__(kBlock) void k_gather_narrow(const float *__restrict__ x, int64_t n, int32_t d,
                                                          int64_t ld, const uint32_t *__restrict__ orig,
                                                          const int32_t *__restrict__ perm, int nbw,
                                                          float4 *__restrict__ xs)
{
    __shared__ int32_t sp[64];
    for (int k = threadIdx.x; k < 64; k += blockDim.x) sp[k] = k < d ? perm[k] : -1;
    __syncthreads();
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float *row = x + (int64_t)orig[i] * ld;
    for (int b = 0; b < nbw; ++b) {
        float4 v;
        v.x = sp[4 * b + 0] >= 0 ? row[sp[4 * b + 0]] : 0.0f;
        v.y = sp[4 * b + 1] >= 0 ? row[sp[4 * b + 1]] : 0.0f;
        v.z = sp[4 * b + 2] >= 0 ? row[sp[4 * b + 2]] : 0.0f;
        v.w = sp[4 * b + 3] >= 0 ? row[sp[4 * b + 3]] : 0.0f;
        xs[(int64_t)b * n + i] = v;
    }
}

// Wider rows: a workgroup takes gather_rows_per_group(d)
// consecutive output rows: their input rows are read whole into LDS (each
// row's floats by consecutive threads), then every block of the rows is
// written as consecutive float4 of the rows (LDS row stride d + 1 floats,
// odd, so that threads reading one dimension of consecutive rows hit
// distinct banks).  Only blocks [0, nbw) are written.
constexpr int kGatherLds = 12288;  // floats of LDS for the staged rows
__host__ __device__ inline int gather_rows_per_group(int32_t d)
{
    const int r = kGatherLds / (d + 1);
    return r > kBlock ? kBlock : (r < 1 ? 1 : r);
}

__global__ __launch_bounds__(kBlock) void k_gather(const float *__restrict__ x, int64_t n, int32_t d,
                                                   int64_t ld, const uint32_t *__restrict__ orig,
                                                   const int32_t *__restrict__ perm, int nbw,
                                                   float4 *__restrict__ xs)
{
    __shared__ float sx[kGatherLds];
    const int R = gather_rows_per_group(d), ldl = d + 1;
    const int64_t r0 = (int64_t)blockIdx.x * R;
    const int rows = (int)(n - r0 < R ? n - r0 : R);
    const int tid = threadIdx.x;
    if (d >= 128) {
        for (int r = 0; r < rows; ++r) {
            const float *row = x + (int64_t)orig[r0 + r] * ld;
            for (int k = tid; k < d; k += kBlock) sx[r * ldl + k] = row[k];
        }
    } else {
        // rows * d < 12288: element idx is dimension idx - r d of row r
        const float rd = 1.0f / (float)d;
        for (int idx = tid; idx < rows * d; idx += kBlock) {
            int r = (int)((float)idx * rd);
            r = r * d > idx ? r - 1 : r;
            r = (r + 1) * d <= idx ? r + 1 : r;
            const int k = idx - r * d;
            sx[r * ldl + k] = x[(int64_t)orig[r0 + r] * ld + k];
        }
    }
    __syncthreads();
    // thread tid: row tid % Rp of the group, blocks tid / Rp + j (256 / Rp)
    // (Rp: R rounded up to a power of two)
    int Rp = 1;
    while (Rp < R) Rp <<= 1;
    const int r = tid & (Rp - 1), bstep = kBlock / Rp;
    if (r >= rows) return;
    for (int b = tid / Rp; b < nbw; b += bstep) {
        float c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = 4 * b + q;
            c[q] = k < d ? sx[r * ldl + perm[k]] : 0.0f;
        }
        xs[(int64_t)b * n + r0 + r] = make_float4(c[0], c[1], c[2], c[3]);
    }
}

// ----------------------------------------------------------------- cells --
// cells are runs of equal row keys >> shift (the sub-cell bits dropped)
__global__ __launch_bounds__(kBlock) void k_cell_flags(const uint64_t *__restrict__ keys, int64_t n,
                                                       int shift, uint32_t *__restrict__ flags)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    flags[i] = (i == 0 || (keys[i] >> shift) != (keys[i - 1] >> shift)) ? 1u : 0u;
}

__global__ __launch_bounds__(kBlock) void k_cell_scatter(const uint64_t *__restrict__ keys, int shift,
                                                         const uint32_t *__restrict__ flags,
                                                         const uint64_t *__restrict__ cid, int64_t n,
                                                         uint32_t *__restrict__ cell_start,
                                                         uint64_t *__restrict__ cell_key)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (flags[i]) {
        cell_start[cid[i]] = (uint32_t)i;
        cell_key[cid[i]] = keys[i] >> shift;
    }
    if (i == n - 1) cell_start[cid[n]] = (uint32_t)n;
}

// ------------------------------------------------- order within a cell --
// Rows of a cell ordered as the leaves of a kd-tree with midpoint splits of
// the cell's own box in the first kOrderDims dimensions of the variance
// order (each split halves the widest remaining extent; 24 levels), so that
// runs of consecutive rows - the refinement's 32-row query blocks and
// 64-candidate chunks - are compact in those dimensions and not only on the
// grid axes.  The box test of the refinement covers the same dimensions.

// Box of each cell over the first kOrderDims layout dimensions (ordered
// float bits; box must hold 0xffffffff / 0 before), from the rows gathered in
// cell order (dimension-blocked, first two blocks): a wave per 64
// consecutive rows, reduced in the wave when they share a cell.
__global__ __launch_bounds__(kBlock) void k_cell_box8(const float4 *__restrict__ xs, int64_t n, int nb,
                                                      const uint64_t *__restrict__ cid,
                                                      uint32_t *__restrict__ lo_bits,
                                                      uint32_t *__restrict__ hi_bits)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    if (i - lane >= n) return;  // whole wave
    const bool valid = i < n;
    const int64_t cell = valid ? (int64_t)cid[i + 1] - 1 : -1;
    const int64_t c0 = __shfl(cell, 0, 64);
    const bool shared = __ballot(valid && cell != c0) == 0;  // lanes past n hold no row
    for (int b = 0; b < kOrderDims / 4; ++b) {
        const float4 v = valid && b < nb ? xs[(uint64_t)b * n + i] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float c[4] = {v.x, v.y, v.z, v.w};
        for (int k = 0; k < 4; ++k) {
            const int a = 4 * b + k;
            const uint32_t o = valid ? f2ord(c[k]) : 0u;
            if (shared) {
                uint32_t lo = valid ? o : 0xffffffffu, hi = o;
                for (int m = 1; m < 64; m <<= 1) {
                    lo = min(lo, (uint32_t)__shfl_xor((int)lo, m, 64));
                    hi = max(hi, (uint32_t)__shfl_xor((int)hi, m, 64));
                }
                if (lane == 0) {
                    atomicMin(&lo_bits[c0 * kOrderDims + a], lo);
                    atomicMax(&hi_bits[c0 * kOrderDims + a], hi);
                }
            } else if (valid) {
                atomicMin(&lo_bits[cell * kOrderDims + a], o);
                atomicMax(&hi_bits[cell * kOrderDims + a], o);
            }
        }
    }
}

// The order of the key bits of a cell's rows, as a kd-tree with midpoint
// splits would cut the cell's box: 24 times, the dimension whose current
// width (extent / 2^(bits already taken)) is largest takes the next bit
// (ties: the lower dimension).  masks[c][a] holds the key positions of
// dimension a's bits (bit 23 first).  A thread per cell.
__global__ __launch_bounds__(kBlock) void k_cell_split(const uint32_t *__restrict__ lo_bits,
                                                       const uint32_t *__restrict__ hi_bits, int64_t M,
                                                       uint32_t *__restrict__ masks)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= M) return;
    float ext[kOrderDims];
    uint32_t m[kOrderDims];
    int nbits[kOrderDims];
#pragma unroll
    for (int a = 0; a < kOrderDims; ++a) {
        const float e = ord2f(hi_bits[c * kOrderDims + a]) - ord2f(lo_bits[c * kOrderDims + a]);
        ext[a] = e > 0.f ? e : 0.f;  // inf stays inf (never split past it)
        m[a] = 0;
        nbits[a] = 0;
    }
    for (int t = 23; t >= 0; --t) {
        int best = 0;
        float bw = -1.f;
#pragma unroll
        for (int a = 0; a < kOrderDims; ++a) {
            const float w = ldexpf(ext[a], -nbits[a]);
            if (w > bw) {
                bw = w;
                best = a;
            }
        }
#pragma unroll
        for (int a = 0; a < kOrderDims; ++a) {
            if (a == best) {
                m[a] |= 1u << t;
                ++nbits[a];
            }
        }
    }
#pragma unroll
    for (int a = 0; a < kOrderDims; ++a) masks[c * kOrderDims + a] = m[a];
}

// key = (cell << 24) | the row's position in its cell's box, each dimension
// quantised to as many bits as k_cell_split gave it and its bits placed at
// that dimension's key positions; value = the row's position in cell order
__global__ __launch_bounds__(kBlock) void k_cell_order_keys(const float4 *__restrict__ xs, int64_t n, int nb,
                                                            const uint64_t *__restrict__ cid,
                                                            const uint32_t *__restrict__ lo_bits,
                                                            const uint32_t *__restrict__ hi_bits,
                                                            const uint32_t *__restrict__ masks,
                                                            uint64_t *__restrict__ keys,
                                                            uint32_t *__restrict__ vals)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t cell = cid[i + 1] - 1;
    uint32_t key = 0;
#pragma unroll
    for (int b = 0; b < kOrderDims / 4; ++b) {
        const float4 v4 = b < nb ? xs[(uint64_t)b * n + i] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float c[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int a = 4 * b + k;
            uint32_t pm = masks[cell * kOrderDims + a];
            const int nbits = __popc(pm);
            if (nbits == 0) continue;
            const float lo = ord2f(lo_bits[cell * kOrderDims + a]), hi = ord2f(hi_bits[cell * kOrderDims + a]);
            const float w = hi - lo;  // 0 (a one-point cell) or inf: every row takes 0
            const float t = w > 0.f && w < INFINITY ? (c[k] - lo) / w * (float)(1u << nbits) : 0.0f;
            const uint32_t top = (1u << nbits) - 1u;
            const uint32_t q = t >= (float)top ? top : (t > 0.0f ? (uint32_t)t : 0u);
            // deposit q's bits, most significant first, at the positions of pm
            for (int j = nbits - 1; j >= 0; --j) {
                const int pos = 31 - __clz(pm);
                key |= ((q >> j) & 1u) << pos;
                pm &= ~(1u << pos);
            }
        }
    }
    keys[i] = (cell << 24) | key;
    vals[i] = (uint32_t)i;
}

// Rows put in their final order: thread i takes cell-order row perm[i]
// (every dimension block, and its input row id).
__global__ __launch_bounds__(kBlock) void k_permute_rows(const float4 *__restrict__ src, const uint32_t *__restrict__ orig_src,
                                                         const uint32_t *__restrict__ perm, int64_t n, int nb,
                                                         float4 *__restrict__ dst, uint32_t *__restrict__ orig_dst)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t j = perm[i];
    orig_dst[i] = orig_src[j];
    for (int b = 0; b < nb; ++b) dst[(uint64_t)b * n + i] = src[(uint64_t)b * n + j];
}

// ------------------------------------------------- balanced tree order --
// Rows of a cell ordered as the leaves of a balanced binary tree, the
// equal-count grouping of the kd-tree of Sec. IV-B (about the same number of
// points per leaf).  A node is a run of consecutive rows.  A node of more
// than kTreeLeaf rows splits into a first child of 32 floor(size / 64) rows
// (size / 2 below 64) and a second child of the rest, by the rows' values
// in the node's split dimension: of the first kTreeDims layout dimensions,
// the one whose values vary most over up to 256 of the node's rows sampled
// at equal strides.  Children start on 32-row boundaries from the cell's
// first row, so the refinement's 32-row query blocks are leaves (or
// sub-runs of the last, smaller ones).  A level is built from a key per row,
// (node << 32) | the row's value as ordered bits (0 in a leaf), and a stable
// radix sort of the keys with the rows' cell-order positions.

// one workgroup per node: its split dimension, 0xffffffff for a leaf.
// Thread t sums dimension t % 64 over samples t / 64, t / 64 + 4, ...,
// shifted by the first sample's value.
__global__ __launch_bounds__(kBlock) void k_tree_dims(const float4 *__restrict__ xs, int64_t n, int nb,
                                                      const uint32_t *__restrict__ pos,
                                                      const uint32_t *__restrict__ nstart,
                                                      const uint32_t *__restrict__ nsize,
                                                      uint32_t *__restrict__ ndim)
{
    __shared__ float s1[4][64], s2[4][64];
    const uint32_t k = blockIdx.x, t = threadIdx.x;
    const uint32_t st = nstart[k], sz = nsize[k];
    if (sz <= (uint32_t)kTreeLeaf) {
        if (t == 0) ndim[k] = 0xffffffffu;
        return;
    }
    const int D = min(4 * nb, kTreeDims);
    const int a = (int)(t & 63u), g = (int)(t >> 6);
    const uint32_t m = min(sz, 256u);
    auto value = [&](uint32_t j) -> float {
        const uint32_t p = st + (uint32_t)((uint64_t)j * sz / m);
        const float4 v = xs[(uint64_t)(a >> 2) * (uint64_t)n + pos[p]];
        const int c = a & 3;
        return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
    };
    float a1 = 0.f, a2 = 0.f;
    if (a < D) {
        const float sh = value(0);
        for (uint32_t j = (uint32_t)g; j < m; j += 4) {
            const float y = value(j) - sh;
            a1 += y;
            a2 = fmaf(y, y, a2);
        }
    }
    s1[g][a] = a1;
    s2[g][a] = a2;
    __syncthreads();
    if (t < 64) {
        const float q1 = s1[0][t] + s1[1][t] + s1[2][t] + s1[3][t];
        const float q2 = s2[0][t] + s2[1][t] + s2[2][t] + s2[3][t];
        const float mu = q1 / (float)m;
        float var = (int)t < D ? q2 / (float)m - mu * mu : -1.0f;
        if (!(var >= 0.0f)) var = (int)t < D ? 0.0f : -1.0f;  // rounding below 0, or overflow
        uint32_t best = t;
        // largest variance, ties to the lower dimension
        for (int o = 1; o < 64; o <<= 1) {
            const float ov = __shfl_xor(var, o, 64);
            const uint32_t ob = (uint32_t)__shfl_xor((int)best, o, 64);
            if (ov > var || (ov == var && ob < best)) {
                var = ov;
                best = ob;
            }
        }
        if (t == 0) ndim[k] = best;
    }
}

// key of position p: node k (largest with nstart[k] <= p) in the high word,
// the row's value in k's split dimension as ordered bits in the low word
__global__ __launch_bounds__(kBlock) void k_tree_keys(const float4 *__restrict__ xs, int64_t n,
                                                      const uint32_t *__restrict__ pos,
                                                      const uint32_t *__restrict__ nstart, uint32_t K,
                                                      const uint32_t *__restrict__ ndim,
                                                      uint64_t *__restrict__ keys)
{
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n) return;
    uint32_t lo = 0, hi = K;  // nstart[lo] <= p < nstart[hi] (nstart[K] taken as n)
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if ((int64_t)nstart[mid] <= p) lo = mid;
        else hi = mid;
    }
    const uint32_t dm = ndim[lo];
    uint32_t v = 0;
    if (dm != 0xffffffffu) {
        const float4 x = xs[(uint64_t)(dm >> 2) * (uint64_t)n + pos[p]];
        const uint32_t c = dm & 3u;
        v = f2ord(c == 0 ? x.x : c == 1 ? x.y : c == 2 ? x.z : x.w);
    }
    keys[p] = ((uint64_t)lo << 32) | v;
}

__global__ __launch_bounds__(kBlock) void k_tree_counts(const uint32_t *__restrict__ nsize, uint32_t K,
                                                        uint32_t *__restrict__ cnt)
{
    const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < K) cnt[k] = nsize[k] > (uint32_t)kTreeLeaf ? 2u : 1u;
}

// the next level's nodes at off[k] (exclusive scan of the counts); the
// largest next-level size into *maxsz (must hold 0 before)
__global__ __launch_bounds__(kBlock) void k_tree_next(const uint32_t *__restrict__ nstart,
                                                      const uint32_t *__restrict__ nsize, uint32_t K,
                                                      const uint64_t *__restrict__ off,
                                                      uint32_t *__restrict__ ostart, uint32_t *__restrict__ osize,
                                                      uint32_t *__restrict__ maxsz)
{
    const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    const uint32_t st = nstart[k], sz = nsize[k];
    const uint64_t o = off[k];
    uint32_t big = sz;
    if (sz > (uint32_t)kTreeLeaf) {
        const uint32_t h = sz >= 64u ? sz / 64u * 32u : sz / 2u;
        ostart[o] = st;
        osize[o] = h;
        ostart[o + 1] = st + h;
        osize[o + 1] = sz - h;
        big = max(h, sz - h);
    } else {
        ostart[o] = st;
        osize[o] = sz;
    }
    atomicMax(maxsz, big);
}

// level 0: a node per cell; the largest cell size into *maxsz (0 before)
__global__ __launch_bounds__(kBlock) void k_tree_roots(const uint32_t *__restrict__ cell_start, int64_t M,
                                                       uint32_t *__restrict__ nstart, uint32_t *__restrict__ nsize,
                                                       uint32_t *__restrict__ pos_identity, int64_t n,
                                                       uint32_t *__restrict__ maxsz)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) pos_identity[i] = (uint32_t)i;
    if (i < M) {
        const uint32_t st = cell_start[i], sz = cell_start[i + 1] - st;
        nstart[i] = st;
        nsize[i] = sz;
        atomicMax(maxsz, sz);
    }
}

constexpr int kAabbSteps = 8;  // 64-point steps per wave

// A wave per 512 consecutive sorted points, 64 at a time (coalesced loads).
// While a step's 64 points share the running cell, each lane keeps its own
// bounds; when the cell changes the wave reduces them and one lane merges
// them into the cell's box by atomic min/max.  A step that straddles a cell
// boundary (a few per cell) merges every point on its own.
__global__ __launch_bounds__(kBlock) void k_cell_aabb(const float4 *__restrict__ xs,
                                                      const uint64_t *__restrict__ cid, int64_t n,
                                                      uint32_t *__restrict__ lo_bits,
                                                      uint32_t *__restrict__ hi_bits)
{
    const int lane = threadIdx.x & 63;
    const int64_t i0 = ((int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * (64 * kAabbSteps);
    if (i0 >= n) return;  // whole wave
    int64_t cur = -1;     // wave-uniform
    uint32_t lo[3], hi[3];
    auto reset = [&]() {
        for (int a = 0; a < 3; ++a) {
            lo[a] = 0xffffffffu;
            hi[a] = 0u;
        }
    };
    auto flush = [&]() {
        for (int a = 0; a < 3; ++a) {
            for (int o = 1; o < 64; o <<= 1) {
                lo[a] = min(lo[a], (uint32_t)__shfl_xor((int)lo[a], o, 64));
                hi[a] = max(hi[a], (uint32_t)__shfl_xor((int)hi[a], o, 64));
            }
        }
        if (lane == 0) {
            for (int a = 0; a < 3; ++a) {
                atomicMin(&lo_bits[cur * 3 + a], lo[a]);
                atomicMax(&hi_bits[cur * 3 + a], hi[a]);
            }
        }
    };
    reset();
    // every step's loads first, so that they are in flight together
    int64_t cellv[kAabbSteps];
    float4 xv[kAabbSteps];
#pragma unroll
    for (int j = 0; j < kAabbSteps; ++j) {
        const int64_t i = i0 + 64 * j + lane;
        cellv[j] = i < n ? (int64_t)cid[i + 1] - 1 : -1;
        xv[j] = i < n ? xs[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < kAabbSteps; ++j) {
        const int64_t i = i0 + 64 * j + lane;
        if (i0 + 64 * j >= n) break;  // uniform
        const bool valid = i < n;
        const int64_t cell = cellv[j];
        uint32_t o[3] = {0u, 0u, 0u};
        if (valid) {
            o[0] = f2ord(xv[j].x);
            o[1] = f2ord(xv[j].y);
            o[2] = f2ord(xv[j].z);
        }
        const int64_t c0 = __shfl(cell, 0, 64);
        const bool same = __ballot(valid && cell == c0) == __ballot(true);
        if (same && c0 == cur) {
            for (int a = 0; a < 3; ++a) {
                lo[a] = min(lo[a], o[a]);
                hi[a] = max(hi[a], o[a]);
            }
            continue;
        }
        if (cur >= 0) flush();
        reset();
        if (same) {
            cur = c0;
            for (int a = 0; a < 3; ++a) {
                lo[a] = o[a];
                hi[a] = o[a];
            }
        } else {
            cur = -1;
            if (valid) {
                for (int a = 0; a < 3; ++a) {
                    atomicMin(&lo_bits[cell * 3 + a], o[a]);
                    atomicMax(&hi_bits[cell * 3 + a], o[a]);
                }
            }
        }
    }
    if (cur >= 0) flush();
}

__global__ __launch_bounds__(kBlock) void k_fill_u32(uint32_t *__restrict__ p, uint32_t v, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ __launch_bounds__(kBlock) void k_fill_u64(uint64_t *__restrict__ p, uint64_t v, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// --------------------------------------------------------------- stencil --
__device__ __forceinline__ int64_t find_key(const uint64_t *__restrict__ k, int64_t M, uint64_t key)
{
    int64_t lo = 0, hi = M;
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (k[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    return (lo < M && k[lo] == key) ? lo : -1;
}

// Per home cell A (a cell of the query rows; of the points for the
// self-join): the target cells B (cells of the points) at offsets in
// [-R, R]^3 (R = 1: the 27-cell stencil) that exist and whose box lower distance to A's box (binary64,
// over the grid dimensions) does not exceed the pruning threshold.  Kept
// cells are sorted by index and runs of consecutive cells are merged into one
// contiguous candidate range.  A query cell with no kept cell gets one empty
// range (U = 0).
// A wave per home cell: lane s takes stencil offset s (and s + 64, ...), so
// the binary searches for the neighbour keys run side by side; the kept
// cells are listed in LDS and one lane sorts and merges them.
__global__ __launch_bounds__(256) void k_stencil(CellSet home, CellSet target, GridParams gp,
                                                 double prune_e2, uint32_t *__restrict__ rstart,
                                                 uint32_t *__restrict__ rpref,
                                                 uint32_t *__restrict__ nrng,
                                                 uint32_t *__restrict__ tiles_per_cell,
                                                 unsigned int *__restrict__ umax)
{
    __shared__ uint32_t s_kept[4][kMaxRanges];
    __shared__ uint32_t s_rs[4][kMaxRanges];
    __shared__ uint32_t s_rp[4][kMaxRanges + 1];
    __shared__ uint32_t s_nr[4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t A = (int64_t)blockIdx.x * 4 + wave;
    if (A >= home.M) return;  // whole wave; no workgroup barrier follows
    const uint64_t key = home.key[A];
    int64_t c[3];
    double alo[3], ahi[3];
    for (int a = 0; a < 3; ++a) {
        c[a] = (int64_t)compact3(key >> a);
        alo[a] = (double)ord2f(home.lo_bits[A * 3 + a]);
        ahi[a] = (double)ord2f(home.hi_bits[A * 3 + a]);
    }
    uint32_t *const kept = s_kept[wave];
    uint32_t nk = 0;
    const int R = gp.reach, span = 2 * gp.reach + 1;
    const int nst = span * span * span;
    for (int s0 = 0; s0 < nst; s0 += 64) {
        const int s = s0 + lane;
        bool keep = false;
        uint32_t Bk = 0;
        if (s < nst) {
            const int64_t dlt[3] = {s % span - R, (s / span) % span - R, s / (span * span) - R};
            uint64_t nkey = 0;
            bool ok = true;
            for (int a = 0; a < 3; ++a) {
                const int64_t v = c[a] + dlt[a];
                // stored coordinates run 0 .. G + 1 on a grid axis, 0 elsewhere
                const int64_t G = a < gp.ndim ? (int64_t)gp.G[a] + 2 : 1;
                if (v < 0 || v >= G) ok = false;
                else nkey |= spread3((uint64_t)v) << a;
            }
            const int64_t B = ok ? find_key(target.key, target.M, nkey) : -1;
            if (B >= 0) {
                double dl2 = 0.0;
                for (int a = 0; a < 3; ++a) {
                    const double blo = (double)ord2f(target.lo_bits[B * 3 + a]);
                    const double bhi = (double)ord2f(target.hi_bits[B * 3 + a]);
                    double gap = 0.0;
                    if (blo > ahi[a]) gap = blo - ahi[a];
                    else if (alo[a] > bhi) gap = alo[a] - bhi;
                    dl2 += gap * gap;
                }
                keep = !(dl2 > prune_e2);
                Bk = (uint32_t)B;
            }
        }
        const uint64_t bk = __ballot(keep);
        if (keep) kept[nk + __popcll(bk & ((1ull << lane) - 1ull))] = Bk;
        nk += __popcll(bk);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint32_t *const rs = s_rs[wave];
    uint32_t *const rp = s_rp[wave];
    if (lane == 0) {
        for (uint32_t i = 1; i < nk; ++i) {
            const uint32_t v = kept[i];
            int j = (int)i - 1;
            while (j >= 0 && kept[j] > v) {
                kept[j + 1] = kept[j];
                --j;
            }
            kept[j + 1] = v;
        }
        uint32_t nr = 0, U = 0;
        uint32_t cur_start = 0, cur_len = 0;
        for (uint32_t i = 0; i < nk; ++i) {
            const uint32_t st = target.start[kept[i]], len = target.start[kept[i] + 1] - st;
            if (i > 0 && kept[i] == kept[i - 1] + 1) {
                cur_len += len;
            } else {
                if (i > 0) {
                    rs[nr] = cur_start;
                    rp[nr] = U;
                    U += cur_len;
                    ++nr;
                }
                cur_start = st;
                cur_len = len;
            }
        }
        rs[nr] = cur_start;
        rp[nr] = U;
        U += cur_len;
        ++nr;
        rp[nr] = U;  // nr <= kMaxRanges
        s_nr[wave] = nr;
        nrng[A] = nr;
        const uint32_t sz = home.start[A + 1] - home.start[A];
        tiles_per_cell[A] = (sz + kTileRows - 1) / kTileRows;
        atomicMax(umax, U);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint32_t nr = s_nr[wave];
    const uint32_t U = rp[nr];
    for (int g = lane; g <= kMaxRanges; g += 64) {
        rpref[A * (kMaxRanges + 1) + g] = (uint32_t)g < nr ? rp[g] : U;
        if (g < kMaxRanges) rstart[A * kMaxRanges + g] = (uint32_t)g < nr ? rs[g] : 0u;
    }
}

// ----------------------------------------------------------------- tiles --
// ------------------------------------------------------- chunk boxes --
// Chunks of 64 consecutive positions of each cell's candidate list: counts
// per cell, then the box of each chunk's points over the first kBoxBlocks
// layout blocks, for the refinement's block box test.
__global__ __launch_bounds__(kBlock) void k_chunk_counts(const uint32_t *__restrict__ rpref,
                                                         const uint32_t *__restrict__ nrng, int64_t M,
                                                         uint32_t *__restrict__ cnt)
{
    const int64_t A = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (A >= M) return;
    const uint32_t U = rpref[(uint64_t)A * (kMaxRanges + 1) + nrng[A]];
    cnt[A] = (U + 63) / 64;
}

// Box of every 8 consecutive sorted points (the last group may be short)
// over the first kBoxBlocks layout blocks: a thread per group and block.
__global__ __launch_bounds__(256) void k_point_boxes(const float4 *__restrict__ xs, uint64_t n, int nb,
                                                     uint64_t ngroups, float4 *__restrict__ pbox)
{
    const uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t k = g / kBoxBlocks;
    const int b = (int)(g % kBoxBlocks);
    if (k >= ngroups) return;
    float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
    if (b < nb) {
        const float4 *x = xs + (uint64_t)b * n;
        const uint64_t e = min(n, k * 8 + 8);
        lo = x[k * 8];
        hi = lo;
        for (uint64_t j = k * 8 + 1; j < e; ++j) {
            const float4 v = x[j];
            lo = make_float4(fminf(lo.x, v.x), fminf(lo.y, v.y), fminf(lo.z, v.z), fminf(lo.w, v.w));
            hi = make_float4(fmaxf(hi.x, v.x), fmaxf(hi.y, v.y), fmaxf(hi.z, v.z), fmaxf(hi.w, v.w));
        }
    }
    pbox[(k * kBoxBlocks + b) * 2] = lo;
    pbox[(k * kBoxBlocks + b) * 2 + 1] = hi;
}

// Box of each 64-candidate chunk of each cell's candidate list, exact: a
// thread per chunk and layout block.  The chunk's cell is the last A with
// base[A] <= chunk (binary search over the per-cell chunk prefix); its
// candidates are pieces of the cell's point ranges, and each piece is
// covered by the boxes of the 8-point groups that lie wholly inside it plus
// the points of its partial groups at either end.
__global__ __launch_bounds__(256) void k_chunk_boxes(const uint64_t *__restrict__ base, int64_t M,
                                                     uint64_t nchunks, const uint32_t *__restrict__ rstart,
                                                     const uint32_t *__restrict__ rpref,
                                                     const uint32_t *__restrict__ nrng,
                                                     const float4 *__restrict__ xs, uint64_t n, int nb,
                                                     const float4 *__restrict__ pbox, float4 *__restrict__ cbox)
{
    const uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t ch = gid / kBoxBlocks;
    const int b = (int)(gid % kBoxBlocks);
    if (ch >= nchunks) return;
    float4 blo = make_float4(0.f, 0.f, 0.f, 0.f), bhi = blo;
    if (b < nb) {
        int64_t lo = 0, hi = M;  // the last A with base[A] <= ch
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) >> 1;
            if (base[mid] <= ch) lo = mid;
            else hi = mid;
        }
        const int64_t A = lo;
        const uint32_t *pref = rpref + (uint64_t)A * (kMaxRanges + 1);
        const uint32_t *start = rstart + (uint64_t)A * kMaxRanges;
        const uint32_t nr = nrng[A];
        const uint32_t U = pref[nr];
        const uint32_t p0 = (uint32_t)(ch - base[A]) * 64, p1 = min(U, p0 + 64);
        const float4 *x = xs + (uint64_t)b * n;
        blo = make_float4(INFINITY, INFINITY, INFINITY, INFINITY);
        bhi = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        auto add = [&](float4 l, float4 h) __attribute__((always_inline)) {
            blo = make_float4(fminf(blo.x, l.x), fminf(blo.y, l.y), fminf(blo.z, l.z), fminf(blo.w, l.w));
            bhi = make_float4(fmaxf(bhi.x, h.x), fmaxf(bhi.y, h.y), fmaxf(bhi.z, h.z), fmaxf(bhi.w, h.w));
        };
        for (int g = range_of(pref, nr, p0); g < (int)nr && pref[g] < p1; ++g) {
            uint32_t j = start[g] + (max(p0, pref[g]) - pref[g]);
            const uint32_t e = start[g] + (min(p1, pref[g + 1]) - pref[g]);  // exclusive, > j
            for (; j < e && (j & 7u); ++j) add(x[j], x[j]);
            for (; j + 8 <= e; j += 8)
                add(pbox[((uint64_t)(j >> 3) * kBoxBlocks + b) * 2], pbox[((uint64_t)(j >> 3) * kBoxBlocks + b) * 2 + 1]);
            for (; j < e; ++j) add(x[j], x[j]);
        }
    }
    cbox[(ch * kBoxBlocks + b) * 2] = blo;
    cbox[(ch * kBoxBlocks + b) * 2 + 1] = bhi;
}

__global__ __launch_bounds__(kBlock) void k_tiles(const uint64_t *__restrict__ tile_base, int64_t M,
                                                  int64_t T, const uint32_t *__restrict__ cell_start,
                                                  const uint32_t *__restrict__ rpref,
                                                  const uint32_t *__restrict__ nrng,
                                                  Tile *__restrict__ tiles,
                                                  uint64_t *__restrict__ words,
                                                  uint64_t *__restrict__ cands)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    int64_t lo = 0, hi = M;  // largest A with tile_base[A] <= t
    while (hi - lo > 1) {
        int64_t mid = (lo + hi) >> 1;
        if (tile_base[mid] <= (uint64_t)t) lo = mid;
        else hi = mid;
    }
    const int64_t A = lo;
    const uint32_t j = (uint32_t)(t - (int64_t)tile_base[A]);
    const uint32_t row0 = cell_start[A] + j * kTileRows;
    const uint32_t end = cell_start[A + 1];
    const uint32_t nrows = min((uint32_t)kTileRows, end - row0);
    const uint32_t U = rpref[A * (kMaxRanges + 1) + nrng[A]];
    const uint32_t used = (U + 63u) / 64u;
    const uint32_t W = (used + kRowAlign - 1) / kRowAlign * kRowAlign;
    Tile tl;
    tl.cell = (uint32_t)A;
    tl.row0 = row0;
    tl.nrows = nrows;
    tl.words = W;
    tl.used = used;
    tiles[t] = tl;
    words[t] = (uint64_t)nrows * W;
    cands[t] = (uint64_t)nrows * U;
}

// ------------------------------------------------------------------ plan --
// Greedy window batching over row tiles in index order: a batch grows while
// its mask words stay within the budget.  result = {batches, max words,
// failing tile + 1 (0 = ok)}.
// Reference point of each row tile for the MFMA refinement's centring: per
// dimension the lower median of up to 32 of the tile's rows, taken evenly
// spread over it (rows i m / 32).  Any fp32 point serves the error analysis;
// a median keeps the rows' norms about it small when most of the tile's rows
// lie in one cluster, whatever its first row is.  One workgroup per tile;
// each thread ranks one sampled row's value in one dimension among the
// samples (ties by sample index), eight dimensions per pass.
constexpr int kRefSamples = 32;

__global__ __launch_bounds__(256) void k_tile_ref(const Tile *__restrict__ tiles, const float4 *__restrict__ xq,
                                                  uint64_t nq, int nb, float4 *__restrict__ tref)
{
    __shared__ float vals[8][kRefSamples];
    const uint32_t t = blockIdx.x;
    const Tile tl = tiles[t];
    const int m = (int)min((uint32_t)kTileRows, tl.nrows);
    const int ms = min(m, kRefSamples);
    const int tid = threadIdx.x;
    const int i = tid & (kRefSamples - 1), dd = tid >> 5;  // sample, dimension of the pass
    const int med = (ms - 1) / 2;
    for (int b0 = 0; b0 < nb; b0 += 2) {
        const int b = b0 + (dd >> 2), c = dd & 3;
        __syncthreads();
        if (i < ms && b < nb) {
            const float4 v = xq[(uint64_t)b * nq + tl.row0 + (uint32_t)(i * m / ms)];
            vals[dd][i] = c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
        }
        __syncthreads();
        if (i < ms && b < nb) {
            const float v = vals[dd][i];
            int rank = 0;
            for (int j = 0; j < ms; ++j) {
                const float w = vals[dd][j];
                rank += (w < v) || (w == v && j < i);
            }
            if (rank == med) ((float *)&tref[(uint64_t)t * nb + b])[c] = v;
        }
    }
}

__global__ void k_plan(const uint64_t *__restrict__ toff, const uint64_t *__restrict__ coff,
                       const Tile *__restrict__ tiles, int64_t T, int64_t n, uint64_t budget,
                       uint32_t *__restrict__ bounds, uint64_t *__restrict__ row_bounds,
                       uint64_t *__restrict__ word_bounds, uint64_t *__restrict__ cand_bounds,
                       uint64_t *__restrict__ result)
{
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    int64_t t = 0, nb = 0;
    uint64_t maxw = 0, err = 0, maxrows = 0;
    bounds[0] = 0;
    row_bounds[0] = 0;
    word_bounds[0] = 0;
    cand_bounds[0] = 0;
    while (t < T) {
        const uint64_t base = toff[t];
        const uint64_t lim = base + budget < base ? ~0ull : base + budget;
        int64_t lo = t, hi = T;  // largest t2 in [t, T] with toff[t2] <= lim
        while (lo < hi) {
            int64_t mid = (lo + hi + 1) >> 1;
            if (toff[mid] <= lim) lo = mid;
            else hi = mid - 1;
        }
        if (lo == t) {
            err = (uint64_t)t + 1;
            break;
        }
        ++nb;
        bounds[nb] = (uint32_t)lo;
        row_bounds[nb] = lo < T ? tiles[lo].row0 : (uint64_t)n;
        word_bounds[nb] = toff[lo];
        cand_bounds[nb] = coff[lo];
        maxw = max(maxw, toff[lo] - base);
        maxrows = max(maxrows, row_bounds[nb] - row_bounds[nb - 1]);
        t = lo;
    }
    result[0] = (uint64_t)nb;
    result[1] = maxw;
    result[2] = err;
    result[3] = maxrows;
}

// Launch order: by batch, then heaviest cell first (Sec. IV-D: primitives
// with more intersections are processed first).
__global__ __launch_bounds__(kBlock) void k_order_keys(const Tile *__restrict__ tiles,
                                                       const uint32_t *__restrict__ rpref,
                                                       const uint32_t *__restrict__ nrng, int64_t T,
                                                       const uint32_t *__restrict__ bounds,
                                                       int32_t nb, int ubits, uint32_t umax,
                                                       uint64_t *__restrict__ keys,
                                                       uint32_t *__restrict__ vals)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    int lo = 0, hi = nb;  // largest b with bounds[b] <= t
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (bounds[mid] <= (uint32_t)t) lo = mid;
        else hi = mid;
    }
    const uint32_t A = tiles[t].cell;
    const uint32_t U = rpref[(uint64_t)A * (kMaxRanges + 1) + nrng[A]];
    keys[t] = ((uint64_t)lo << ubits) | (uint64_t)(umax - U);
    vals[t] = (uint32_t)t;
}

}  // namespace

// ============================================================ launchers ==
int64_t stats_threads(int64_t n, int32_t d)
{
    int64_t step = 131072 / d;
    if (step < 1) step = 1;
    if (step > n) step = n;
    return step * d;
}

hipError_t launch_stats(const float *x, int64_t n, int32_t d, int64_t ld, double *partial,
                        uint32_t *bad_partial, int64_t T, double *out_stats,
                        unsigned long long *out_bad, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_u64, dim3(1), dim3(kBlock), 0, s, (uint64_t *)out_bad, 0ull, 1);
    hipLaunchKernelGGL(k_stats_partial, dim3(grid_for(T)), dim3(kBlock), 0, s, x, n, d, ld, T,
                       partial, bad_partial);
    hipLaunchKernelGGL(k_stats_final, dim3((unsigned)d), dim3(kBlock), 0, s, x, n, d, T, partial,
                       bad_partial, out_stats, out_bad);
    return hipGetLastError();
}

hipError_t launch_keys(const float *x, int64_t n, int64_t ld, const GridParams &gp, bool queries,
                       uint64_t *keys, uint32_t *ids, hipStream_t s)
{
    hipLaunchKernelGGL(k_keys, dim3(grid_for(n)), dim3(kBlock), 0, s, x, n, ld, gp, (int)queries, keys,
                       ids);
    return hipGetLastError();
}

size_t radix_hist_entries(int64_t n)
{
    const int64_t nblk = (n + kRsTile - 1) / kRsTile;
    return (size_t)(2 * (256 * nblk + 1));  // counts, then their scan
}

size_t scan_tmp_entries(int64_t n)
{
    const int64_t nb = (n + kScTile - 1) / kScTile;
    return (size_t)(nb + 1);
}

hipError_t scan_u32(const uint32_t *in, uint64_t *out, int64_t n, uint64_t *tmp, hipStream_t s)
{
    return scan_impl<uint32_t>(in, out, n, tmp, s);
}

hipError_t scan_u64(const uint64_t *in, uint64_t *out, int64_t n, uint64_t *tmp, hipStream_t s)
{
    return scan_impl<uint64_t>(in, out, n, tmp, s);
}

hipError_t radix_sort(uint64_t *k0, uint32_t *v0, uint64_t *k1, uint32_t *v1, int64_t n, int bits,
                      uint64_t *hist, uint64_t *scan_tmp, hipStream_t s)
{
    const int passes = (bits + 7) / 8;
    const int64_t nblk = (n + kRsTile - 1) / kRsTile;
    uint64_t *hs = hist + 256 * nblk + 1;  // scanned offsets live after the counts
    uint64_t *ki = k0, *ko = k1;
    uint32_t *vi = v0, *vo = v1;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        hipLaunchKernelGGL(k_radix_hist, dim3((unsigned)nblk), dim3(kBlock), 0, s, ki, n, shift, nblk,
                           hist);
        hipError_t e = scan_u64(hist, hs, 256 * nblk, scan_tmp, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_radix_scatter, dim3((unsigned)nblk), dim3(kBlock), 0, s, ki, vi, ko, vo, n,
                           shift, nblk, hs);
        uint64_t *tk = ki; ki = ko; ko = tk;
        uint32_t *tv = vi; vi = vo; vo = tv;
    }
    if (ki != k0) {
        hipError_t e = hipMemcpyAsync(k0, ki, sizeof(uint64_t) * n, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return e;
        e = hipMemcpyAsync(v0, vi, sizeof(uint32_t) * n, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

hipError_t launch_cell_order_keys(const float4 *xs, int64_t n, int nb, const uint64_t *cid, int64_t M,
                                  uint32_t *box_lo, uint32_t *box_hi, uint32_t *masks, uint64_t *keys, uint32_t *vals,
                                  hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(kOrderDims * M)), dim3(kBlock), 0, s, box_lo, 0xffffffffu,
                       (int64_t)kOrderDims * M);
    hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(kOrderDims * M)), dim3(kBlock), 0, s, box_hi, 0u,
                       (int64_t)kOrderDims * M);
    hipLaunchKernelGGL(k_cell_box8, dim3(grid_for(n)), dim3(kBlock), 0, s, xs, n, nb, cid, box_lo, box_hi);
    hipLaunchKernelGGL(k_cell_split, dim3(grid_for(M)), dim3(kBlock), 0, s, box_lo, box_hi, M, masks);
    hipLaunchKernelGGL(k_cell_order_keys, dim3(grid_for(n)), dim3(kBlock), 0, s, xs, n, nb, cid, box_lo, box_hi,
                       masks, keys, vals);
    return hipGetLastError();
}

hipError_t launch_permute_rows(const float4 *src, const uint32_t *orig_src, const uint32_t *perm, int64_t n, int nb,
                               float4 *dst, uint32_t *orig_dst, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_permute_rows, dim3(grid_for(n)), dim3(kBlock), 0, s, src, orig_src, perm, n, nb, dst,
                       orig_dst);
    return hipGetLastError();
}

hipError_t launch_tree_roots(const uint32_t *cell_start, int64_t M, uint32_t *nstart, uint32_t *nsize,
                             uint32_t *pos, int64_t n, uint32_t *maxsz, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(kBlock), 0, s, maxsz, 0u, (int64_t)1);
    const int64_t m = std::max<int64_t>(n, M);
    if (m == 0) return hipSuccess;
    hipLaunchKernelGGL(k_tree_roots, dim3(grid_for(m)), dim3(kBlock), 0, s, cell_start, M, nstart, nsize, pos, n,
                       maxsz);
    return hipGetLastError();
}

hipError_t launch_tree_level(const float4 *xs, int64_t n, int nb, uint32_t *pos, const uint32_t *nstart,
                             const uint32_t *nsize, uint32_t K, uint32_t *ndim, uint64_t *k0, uint64_t *k1,
                             uint32_t *v1, uint64_t *hist, uint64_t *stmp, uint32_t *cnt, uint64_t *off,
                             uint32_t *ostart, uint32_t *osize, uint32_t *maxsz, hipStream_t s)
{
    if (n == 0 || K == 0) return hipSuccess;
    if (K > 0x7fffffffu || (uint64_t)K > (uint64_t)n) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_tree_dims, dim3(K), dim3(kBlock), 0, s, xs, n, nb, pos, nstart, nsize, ndim);
    hipLaunchKernelGGL(k_tree_keys, dim3(grid_for(n)), dim3(kBlock), 0, s, xs, n, pos, nstart, K, ndim, k0);
    int kb = 0;
    while (kb < 32 && (1ull << kb) < (uint64_t)K) ++kb;
    hipError_t e = radix_sort(k0, pos, k1, v1, n, 32 + kb, hist, stmp, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_tree_counts, dim3(grid_for(K)), dim3(kBlock), 0, s, nsize, K, cnt);
    e = scan_u32(cnt, off, K, stmp, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(kBlock), 0, s, maxsz, 0u, (int64_t)1);
    hipLaunchKernelGGL(k_tree_next, dim3(grid_for(K)), dim3(kBlock), 0, s, nstart, nsize, K, off, ostart, osize,
                       maxsz);
    return hipGetLastError();
}

hipError_t launch_gather(const float *x, int64_t n, int32_t d, int64_t ld, const uint32_t *orig,
                         const int32_t *perm, int nbw, float4 *xs, hipStream_t s)
{
    if (n == 0 || nbw <= 0) return hipSuccess;
    if (d < 1 || d > kMaxDim || nbw > (d + 3) / 4) return hipErrorInvalidValue;
    if (d <= 64) {
        hipLaunchKernelGGL(k_gather_narrow, dim3(grid_for(n)), dim3(kBlock), 0, s, x, n, d, ld, orig, perm, nbw, xs);
        return hipGetLastError();
    }
    const int R = gather_rows_per_group(d);
    const int64_t groups = (n + R - 1) / R;
    if (groups > 0x7fffffffll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_gather, dim3((unsigned)groups), dim3(kBlock), 0, s, x, n, d, ld, orig, perm, nbw, xs);
    return hipGetLastError();
}

hipError_t launch_cell_flags(const uint64_t *keys, int64_t n, int shift, uint32_t *flags, hipStream_t s)
{
    hipLaunchKernelGGL(k_cell_flags, dim3(grid_for(n)), dim3(kBlock), 0, s, keys, n, shift, flags);
    return hipGetLastError();
}

hipError_t launch_cell_scatter(const uint64_t *keys, int shift, const uint32_t *flags, const uint64_t *cid,
                               int64_t n, uint32_t *cell_start, uint64_t *cell_key, hipStream_t s)
{
    hipLaunchKernelGGL(k_cell_scatter, dim3(grid_for(n)), dim3(kBlock), 0, s, keys, shift, flags, cid, n,
                       cell_start, cell_key);
    return hipGetLastError();
}

hipError_t launch_cell_aabb(const float4 *xs, const uint64_t *cid, int64_t n, int64_t M,
                            uint32_t *lo_bits, uint32_t *hi_bits, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(3 * M)), dim3(kBlock), 0, s, lo_bits, 0xffffffffu,
                       3 * M);
    hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(3 * M)), dim3(kBlock), 0, s, hi_bits, 0u, 3 * M);
    const int64_t waves = (n + 64 * kAabbSteps - 1) / (64 * kAabbSteps);
    hipLaunchKernelGGL(k_cell_aabb, dim3(grid_for(waves, kBlock / 64)), dim3(kBlock), 0, s, xs, cid, n, lo_bits,
                       hi_bits);
    return hipGetLastError();
}

hipError_t launch_chunk_counts(const uint32_t *rpref, const uint32_t *nrng, int64_t M, uint32_t *cnt,
                               hipStream_t s)
{
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(k_chunk_counts, dim3(grid_for(M)), dim3(kBlock), 0, s, rpref, nrng, M, cnt);
    return hipGetLastError();
}

hipError_t launch_point_boxes(const float4 *xs, uint64_t n, int nb, float4 *pbox, hipStream_t s)
{
    const uint64_t ng = (n + 7) / 8;
    const uint64_t blocks = (ng * kBoxBlocks + 255) / 256;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_point_boxes, dim3((unsigned)blocks), dim3(256), 0, s, xs, n, nb, ng, pbox);
    return hipGetLastError();
}

hipError_t launch_chunk_boxes(const uint64_t *base, int64_t M, uint64_t nchunks, const uint32_t *rstart,
                              const uint32_t *rpref, const uint32_t *nrng, const float4 *xs, uint64_t n, int nb,
                              const float4 *pbox, float4 *cbox, hipStream_t s)
{
    const uint64_t blocks = (nchunks * kBoxBlocks + 255) / 256;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_chunk_boxes, dim3((unsigned)blocks), dim3(256), 0, s, base, M, nchunks, rstart, rpref,
                       nrng, xs, n, nb, pbox, cbox);
    return hipGetLastError();
}

hipError_t launch_stencil(const CellSet &home, const CellSet &target, const GridParams &gp,
                          double prune_e2, uint32_t *rstart, uint32_t *rpref, uint32_t *nrng,
                          uint32_t *tiles_per_cell, unsigned int *umax, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(kBlock), 0, s, umax, 0u, 1);
    if (home.M == 0) return hipGetLastError();
    if ((home.M + 3) / 4 > 0x7fffffffll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_stencil, dim3((unsigned)((home.M + 3) / 4)), dim3(256), 0, s, home, target, gp, prune_e2,
                       rstart, rpref, nrng, tiles_per_cell, umax);
    return hipGetLastError();
}

hipError_t launch_tiles(const uint64_t *tile_base, int64_t M, int64_t T, const uint32_t *cell_start,
                        const uint32_t *rpref, const uint32_t *nrng, Tile *tiles, uint64_t *words,
                        uint64_t *cands, hipStream_t s)
{
    hipLaunchKernelGGL(k_tiles, dim3(grid_for(T)), dim3(kBlock), 0, s, tile_base, M, T, cell_start,
                       rpref, nrng, tiles, words, cands);
    return hipGetLastError();
}

hipError_t launch_tile_ref(const Tile *tiles, int64_t T, const float4 *xq, uint64_t nq, int nb, float4 *tref,
                           hipStream_t s)
{
    if (T == 0) return hipSuccess;
    if (T > 0x7fffffffll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_tile_ref, dim3((unsigned)T), dim3(256), 0, s, tiles, xq, nq, nb, tref);
    return hipGetLastError();
}

hipError_t launch_plan(const uint64_t *toff, const uint64_t *coff, const Tile *tiles, int64_t T,
                       int64_t n, uint64_t budget_words, uint32_t *bounds, uint64_t *row_bounds,
                       uint64_t *word_bounds, uint64_t *cand_bounds, uint64_t *result,
                       hipStream_t s)
{
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(64), 0, s, toff, coff, tiles, T, n, budget_words, bounds,
                       row_bounds, word_bounds, cand_bounds, result);
    return hipGetLastError();
}

hipError_t launch_order_keys(const Tile *tiles, const uint32_t *rpref, const uint32_t *nrng,
                             int64_t T, const uint32_t *bounds, int32_t nb, int ubits, uint32_t umax,
                             uint64_t *keys, uint32_t *vals, hipStream_t s)
{
    hipLaunchKernelGGL(k_order_keys, dim3(grid_for(T)), dim3(kBlock), 0, s, tiles, rpref, nrng, T,
                       bounds, nb, ubits, umax, keys, vals);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n)), dim3(kBlock), 0, s, p, v, n);
    return hipGetLastError();
}

hipError_t launch_fill_u64(uint64_t *p, uint64_t v, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(n)), dim3(kBlock), 0, s, p, v, n);
    return hipGetLastError();
}

}  // namespace ersj
