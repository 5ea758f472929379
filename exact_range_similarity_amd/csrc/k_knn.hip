// Exact k nearest neighbours from a similarity-search round, for gfx950.
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. VI: the k-nearest-neighbours search becomes a
// sequence of distance similarity searches whose radius grows until every
// query has k neighbours; with the index on three dimensions this still
// gives the exact kNN.  After a round's batch is refined (its result mask
// final, Sec. IV-F), each query row with at least k neighbours holds its k
// nearest among them: every point closer than the k-th neighbour is within
// the round's radius.  Rows with fewer go to the next round.
//
// Ranking key of a neighbour: (D64, point id), D64 the canonical binary64
// squared distance (sum over the input's own dimension order of the squared
// differences, each operation rounded, no fused multiply-add).  D64 >= 0, so
// its bit pattern orders like its value, and the 96-bit key (D64 bits, id)
// is unique within a row.
//
// A row with fewer than k neighbours also reports its count and the sum of
// log(eps / dist) over its neighbours at a positive distance: with the
// counts, the maximum-likelihood estimate of the local dimension m of
// Levina and Bickel ("Maximum likelihood estimation of intrinsic
// dimension", 2004) is (number of terms) / (sum), from which the host sizes
// the next radius (a count growing like radius^m).
//
// Workgroup per row tile, wave per row.  A row with at most kCap neighbours
// gathers their keys into the wave's LDS area and sorts them (bitonic); with
// more than 2k of them, a histogram of D64 / E64 taken while they are
// gathered picks the bucket prefix holding the k smallest, and only that
// prefix is sorted.  A longer row first narrows the keys with a histogram of D64 / E64 (one or
// two counting passes, then a gathering pass of at most kCap keys); when
// ties crowd a bucket, or the radius is infinite, an exact radix select over
// 8-bit digits of the key (twelve passes) finds the k-th smallest key and
// the k keys at or below it are gathered.  Every pass recomputes the keys
// from the mask: no pair list is written to memory.
#include "ersj_internal.h"

namespace ersj {

namespace {

constexpr int kCap = 1024;  // keys a wave sorts in LDS (also the largest k)
constexpr int kWaves = 4;

struct KnnLds {
    uint64_t hi[kWaves][kCap];   // D64 bits
    uint32_t lo[kWaves][kCap];   // point id
    uint32_t hist[kWaves][256];
    uint64_t words[kWaves][64];  // staged mask words of the row
    uint32_t widx[kWaves][64];   // their word index in the row
    uint32_t before[kWaves][64]; // set bits in the earlier staged words
    uint32_t pref[kMaxRanges + 1];
    uint32_t start[kMaxRanges];
    // the tile's rows short of k neighbours, appended to the next round's
    // list with one counter update per workgroup
    uint32_t nshort;
    uint32_t soq[kTileRows], snb[kTileRows];
    double sls[kTileRows];
};

__device__ __forceinline__ bool key_less(uint64_t ah, uint32_t al, uint64_t bh, uint32_t bl)
{
    return ah < bh || (ah == bh && al < bl);
}

// digit p (0 = most significant) of the 96-bit key
__device__ __forceinline__ uint32_t key_digit(uint64_t h, uint32_t l, int p)
{
    return p < 8 ? (uint32_t)(h >> (56 - 8 * p)) & 255u : (l >> (24 - 8 * (p - 8))) & 255u;
}

// the digits above p of the key equal those of the prefix
__device__ __forceinline__ bool key_match(uint64_t h, uint32_t l, uint64_t ph, uint32_t pl, int p)
{
    if (p == 0) return true;
    if (p <= 8) return (h >> (64 - 8 * p)) == (ph >> (64 - 8 * p));
    return h == ph && (l >> (32 - 8 * (p - 8))) == (pl >> (32 - 8 * (p - 8)));
}

// sort hi/lo[0, S) ascending by key; S a power of two, one wave
__device__ void wave_bitonic(uint64_t *hi, uint32_t *lo, int S, int lane)
{
    for (int size = 2; size <= S; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = lane; i < (S >> 1); i += 64) {
                const int a = 2 * i - (i & (stride - 1));
                const int b = a + stride;
                const bool up = (a & size) == 0;
                const uint64_t ah = hi[a], bh = hi[b];
                const uint32_t al = lo[a], bl = lo[b];
                if (key_less(bh, bl, ah, al) == up) {
                    hi[a] = bh;
                    lo[a] = bl;
                    hi[b] = ah;
                    lo[b] = al;
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
    }
}

// Canonical D64 of two rows in the input's dimension order: each difference,
// square and sum rounded on its own (the pragma sits in this body because a
// lambda body does not take it from the enclosing function).  The rows are
// 16-byte aligned and zero-padded to a multiple of four floats; only the
// first d are summed.
__device__ __forceinline__ double canonical_d64(const float4 *__restrict__ q, const float4 *__restrict__ x, int d)
{
#pragma clang fp contract(off)
    double s = 0.0;
    for (int j4 = 0; 4 * j4 < d; ++j4) {
        const float4 qv = q[j4], xv = x[j4];
        const float qc[4] = {qv.x, qv.y, qv.z, qv.w}, xc[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (4 * j4 + c < d) {
                const double u = (double)qc[c] - (double)xc[c];
                const double uu = u * u;
                s = s + uu;
            }
        }
    }
    return s;
}

// position of the r-th (0-based) set bit of w; r < popcount(w)
__device__ __forceinline__ int nth_set_bit(uint64_t w, uint32_t r)
{
    int pos = 0;
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
        const uint64_t low = (1ull << sh) - 1ull;
        const uint32_t c = __popcll(w & low);
        if (r >= c) {
            r -= c;
            w >>= sh;
            pos += sh;
        } else {
            w &= low;
        }
    }
    return pos;
}

__device__ __forceinline__ uint32_t pow2_at_least(uint32_t v)
{
    uint32_t s = 1;
    while (s < v) s <<= 1;
    return s;
}

__global__ __launch_bounds__(256) void k_knn_select(KnnArgs a)
{
    __shared__ KnnLds L;
    const uint32_t t = a.t0 + blockIdx.x;
    const Tile tl = a.tiles[t];
    const uint32_t A = tl.cell;
    const uint32_t nr = a.nrng[A];
    if (threadIdx.x <= kMaxRanges)
        L.pref[threadIdx.x] = threadIdx.x <= nr ? a.rpref[(uint64_t)A * (kMaxRanges + 1) + threadIdx.x] : 0xffffffffu;
    if (threadIdx.x < kMaxRanges) L.start[threadIdx.x] = a.rstart[(uint64_t)A * kMaxRanges + threadIdx.x];
    if (threadIdx.x == 0) L.nshort = 0;
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    uint64_t *const ehi = L.hi[wave];
    uint32_t *const elo = L.lo[wave];
    uint32_t *const hist = L.hist[wave];
    uint64_t *const cw = L.words[wave];
    uint32_t *const ci = L.widx[wave];
    uint32_t *const cb = L.before[wave];
    const uint32_t k = a.k;
    const int32_t d = a.d;
    const uint64_t tbase = a.toff[t] - a.wbase;

    for (uint32_t r = wave; r < tl.nrows; r += kWaves) {
        const uint32_t q = tl.row0 + r;
        const uint32_t c = a.rowcnt[q - a.row_base];
        const uint32_t qid = a.qorig[q];                   // row of the round's query array
        const uint32_t oq = a.qmap ? a.qmap[qid] : qid;    // query id of the whole search
        const float4 *qrow = (const float4 *)(a.xqr + (uint64_t)q * a.ldr);
        const uint64_t *row = a.mask + tbase + (uint64_t)r * tl.words;
        const uint8_t *frow = a.gflag + ((tbase + (uint64_t)r * tl.words) >> 2);

        // Calls f(valid, hi, lo) once per lane and step until every set bit
        // of the row has been visited; each valid lane holds one neighbour's
        // key.  The row's unit flags (one per 4 mask words) are read 64 at a
        // time; the words of up to 16 flagged units are staged in LDS with
        // their bit prefix, and their set bits are dealt to the lanes in
        // turn, so only flagged words are read and dense words do not
        // serialise the distance work on one lane.
        auto for_each = [&](auto &&f) __attribute__((always_inline)) {
            const uint32_t nunits = (tl.used + 3) / 4;
            for (uint32_t u0 = 0; u0 < nunits; u0 += 64) {
                uint64_t nz = __ballot(u0 + lane < nunits && frow[u0 + lane] != 0);
                while (nz != 0) {
                    const uint32_t cnt = min(16u, (uint32_t)__popcll(nz));
                    const uint32_t slot = (uint32_t)lane >> 2;
                    uint64_t m = 0ull;
                    uint32_t wi = 0;
                    if (slot < cnt) {
                        wi = (u0 + (uint32_t)nth_set_bit(nz, slot)) * 4 + (lane & 3);
                        m = wi < tl.used ? row[wi] : 0ull;
                    }
                    for (uint32_t i = 0; i < cnt; ++i) nz &= nz - 1;
                    const uint32_t pc = __popcll(m);
                    uint32_t inc = pc;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const uint32_t v = __shfl_up(inc, o, 64);
                        if (lane >= o) inc += v;
                    }
                    const uint32_t total = __shfl(inc, 63, 64);
                    if (total == 0) continue;
                    cw[lane] = m;
                    ci[lane] = wi;
                    cb[lane] = inc - pc;
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    for (uint32_t j0 = 0; j0 < total; j0 += 64) {
                        const uint32_t j = j0 + lane;
                        const bool valid = j < total;
                        uint64_t kh = ~0ull;
                        uint32_t kl = ~0u;
                        if (valid) {
                            int lo = 0, hi = 63;  // the last staged word with cb[word] <= j
                            while (lo < hi) {
                                const int mid = (lo + hi + 1) >> 1;
                                if (cb[mid] <= j) lo = mid;
                                else hi = mid - 1;
                            }
                            const uint32_t p = ci[lo] * 64 + nth_set_bit(cw[lo], j - cb[lo]);
                            const int g = range_of(L.pref, nr, p);
                            const uint32_t sx = L.start[g] + (p - L.pref[g]);  // sorted point
                            const uint32_t pid = a.orig[sx];
                            const double s = canonical_d64(qrow, (const float4 *)(a.xr + (uint64_t)sx * a.ldr), d);
                            kh = (uint64_t)__double_as_longlong(s);
                            kl = pid;
                        }
                        f(valid, kh, kl);
                    }
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                }
            }
        };
        // append the valid lanes' keys at ehi/elo[*n ...]
        auto append = [&](bool valid, uint64_t kh, uint32_t kl, uint32_t &n) __attribute__((always_inline)) {
            const uint64_t b = __ballot(valid);
            const uint32_t below = __popcll(b & ((1ull << lane) - 1ull));
            if (valid && n + below < (uint32_t)kCap) {
                ehi[n + below] = kh;
                elo[n + below] = kl;
            }
            n += __popcll(b);
        };

        if (c < k) {
            // too few: report the query with what the next radius needs
            double ls = 0.0;
            uint32_t np = 0;
            for_each([&](bool v, uint64_t kh, uint32_t kl) {
                const double dd = __longlong_as_double((long long)kh);
                if (v && dd > 0.0) {
                    ls += 0.5 * log(a.e64 / dd);
                    ++np;
                }
            });
            for (int o = 32; o > 0; o >>= 1) {
                ls += __shfl_xor(ls, o, 64);
                np += __shfl_xor(np, o, 64);
            }
            if (lane == 0) {
                const uint32_t pos = atomicAdd(&L.nshort, 1u);
                L.soq[pos] = oq;
                L.snb[pos] = c | (np << 16);  // both below 2^16 (c < k <= 1024)
                L.sls[pos] = np > 0 ? ls : 0.0;
            }
            continue;
        }
        uint32_t nsel = 0;
        // The bucket of hist holding rank (0-based): its index, the count
        // in the buckets before it, and that count plus its own.
        auto pick = [&](uint32_t rank, uint32_t &dig, uint32_t &before, uint32_t &through)
                        __attribute__((always_inline)) {
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            uint32_t h4[4], s4 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h4[j] = hist[4 * lane + j];
                s4 += h4[j];
            }
            uint32_t inc = s4;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t v = __shfl_up(inc, o, 64);
                if (lane >= o) inc += v;
            }
            const uint32_t exc = inc - s4;
            const bool mine = exc <= rank && rank < inc;
            const int owner = __ffsll((unsigned long long)__ballot(mine)) - 1;
            uint32_t dg = 0, bf = exc, th = exc;
            if (mine) {
                uint32_t run = exc;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (rank >= run && rank < run + h4[j]) {
                        dg = 4 * lane + j;
                        bf = run;
                        th = run + h4[j];
                    }
                    run += h4[j];
                }
            }
            dig = __shfl(dg, owner, 64);
            before = __shfl(bf, owner, 64);
            through = __shfl(th, owner, 64);
        };
        auto clear_hist = [&]() __attribute__((always_inline)) {
            for (int i = lane; i < 256; i += 64) hist[i] = 0;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        };
        // value buckets: u = 256 D64 / E64 is monotone in D64 and, with
        // every neighbour at D64 <= E64, within [0, 256]; keys of equal D64
        // share a bucket
        const bool bucketed = a.e64 > 0.0 && a.e64 <= 1.0e300;
        const double sc = bucketed ? 256.0 / a.e64 : 0.0;
        auto ubin = [&](uint64_t kh, double &u) __attribute__((always_inline)) {
            u = __longlong_as_double((long long)kh) * sc;
            return u >= 255.0 ? 255u : (uint32_t)u;
        };
        if (c <= (uint32_t)kCap) {
            // all keys into LDS; with more than 2k of them, a histogram taken
            // on the way finds the bucket prefix that holds the k smallest,
            // and only that prefix is kept for the sort
            const bool cut = bucketed && c > 2 * k;
            if (cut) clear_hist();
            for_each([&](bool v, uint64_t kh, uint32_t kl) {
                append(v, kh, kl, nsel);
                double u;
                if (cut && v) atomicAdd(&hist[ubin(kh, u)], 1u);
            });
            if (cut) {
                uint32_t b0, before0, through0;
                pick(k - 1, b0, before0, through0);
                // in-place compaction in order: a chunk is read before it is
                // written, and writes land at or below the chunk's start
                const uint32_t ntot = min(nsel, (uint32_t)kCap);
                uint32_t m = 0;
                for (uint32_t j0 = 0; j0 < ntot; j0 += 64) {
                    const uint32_t j = j0 + lane;
                    uint64_t kh = 0;
                    uint32_t kl = 0;
                    bool keep = false;
                    if (j < ntot) {
                        kh = ehi[j];
                        kl = elo[j];
                        double u;
                        keep = ubin(kh, u) <= b0;
                    }
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    append(keep, kh, kl, m);
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                }
                nsel = m;
            }
        } else {
            bool done = false;
            // Usually one counting pass over the value buckets finds a
            // bucket prefix holding the k smallest keys and at most kCap
            // keys in all, and a second pass gathers it; a crowded bucket is
            // split once more into 256 sub-buckets.
            if (bucketed) {
                auto sub = [&](double u, uint32_t b0) __attribute__((always_inline)) {
                    const double v = (u - (double)b0) * 256.0;
                    return v >= 255.0 ? 255u : (uint32_t)v;
                };
                clear_hist();
                for_each([&](bool v, uint64_t kh, uint32_t kl) {
                    double u;
                    if (v) atomicAdd(&hist[ubin(kh, u)], 1u);
                });
                uint32_t b0, before0, through0;
                pick(k - 1, b0, before0, through0);
                if (through0 <= (uint32_t)kCap) {
                    for_each([&](bool v, uint64_t kh, uint32_t kl) {
                        double u;
                        append(v && ubin(kh, u) <= b0, kh, kl, nsel);
                    });
                    done = true;
                } else {
                    clear_hist();
                    for_each([&](bool v, uint64_t kh, uint32_t kl) {
                        double u;
                        if (v && ubin(kh, u) == b0) atomicAdd(&hist[sub(u, b0)], 1u);
                    });
                    uint32_t b1, before1, through1;
                    pick(k - 1 - before0, b1, before1, through1);
                    if (before0 + through1 <= (uint32_t)kCap) {
                        for_each([&](bool v, uint64_t kh, uint32_t kl) {
                            double u;
                            const uint32_t b = ubin(kh, u);
                            append(v && (b < b0 || (b == b0 && sub(u, b0) <= b1)), kh, kl, nsel);
                        });
                        done = true;
                    }
                }
            }
            if (!done) {
                // exact radix select of the k-th smallest 96-bit key, 8 bits
                // per pass (crowded ties, or an infinite radius)
                uint64_t ph = 0;
                uint32_t pl = 0, rank = k - 1;
                for (int p = 0; p < 12; ++p) {
                    clear_hist();
                    for_each([&](bool v, uint64_t kh, uint32_t kl) {
                        if (v && key_match(kh, kl, ph, pl, p)) atomicAdd(&hist[key_digit(kh, kl, p)], 1u);
                    });
                    uint32_t dig, before, through;
                    pick(rank, dig, before, through);
                    rank -= before;
                    if (p < 8) ph |= (uint64_t)dig << (56 - 8 * p);
                    else pl |= dig << (24 - 8 * (p - 8));
                }
                // the k keys at or below the k-th smallest
                nsel = 0;
                for_each([&](bool v, uint64_t kh, uint32_t kl) {
                    append(v && !key_less(ph, pl, kh, kl), kh, kl, nsel);
                });
            }
        }
        nsel = min(nsel, (uint32_t)kCap);
        const uint32_t S = pow2_at_least(nsel);
        for (uint32_t i = nsel + lane; i < S; i += 64) {
            ehi[i] = ~0ull;
            elo[i] = ~0u;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        wave_bitonic(ehi, elo, (int)S, lane);
        for (uint32_t i = lane; i < k; i += 64) {
            a.ids[(uint64_t)oq * k + i] = elo[i];
            if (a.dist) a.dist[(uint64_t)oq * k + i] = __longlong_as_double((long long)ehi[i]);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    __syncthreads();
    const uint32_t ns = L.nshort;
    if (ns != 0) {
        __shared__ uint32_t s_base;
        if (threadIdx.x == 0) s_base = atomicAdd(a.next_count, ns);
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < ns; i += blockDim.x) {
            a.next[s_base + i] = L.soq[i];
            a.next_nbrs[s_base + i] = L.snb[i];
            a.next_lsum[s_base + i] = L.sls[i];
        }
    }
}

// rows idx[i] of a row-major array, packed: out[i * d + j] = q[idx[i] * ldq + j]
__global__ __launch_bounds__(256) void k_gather_rows(const float *__restrict__ q, int64_t ldq,
                                                     const uint32_t *__restrict__ idx, uint64_t m,
                                                     int32_t d, int32_t ldo, float *__restrict__ out)
{
    const uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= m * (uint64_t)ldo) return;
    const uint64_t i = e / (uint64_t)ldo, j = e - i * (uint64_t)ldo;
    out[e] = j < (uint64_t)d ? q[(uint64_t)idx[i] * ldq + j] : 0.0f;
}

}  // namespace

int knn_max_k() { return kCap; }

hipError_t launch_knn_select(const KnnArgs &a, uint32_t ntiles, hipStream_t s)
{
    if (ntiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_knn_select, dim3(ntiles), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const float *q, int64_t ldq, const uint32_t *idx, uint64_t m, int32_t d,
                              int32_t ldo, float *out, hipStream_t s)
{
    if (ldo < d) return hipErrorInvalidValue;
    const uint64_t total = m * (uint64_t)ldo;
    if (total == 0) return hipSuccess;
    const uint64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)blocks), dim3(256), 0, s, q, ldq, idx, m, d, ldo, out);
    return hipGetLastError();
}

}  // namespace ersj
