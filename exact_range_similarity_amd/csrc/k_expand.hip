// Boundary re-check and result compaction for gfx950.
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. IV-F and IV-F1 (Fig. 5): the result mask holds
// one bit per query/candidate comparison; compaction keeps only the
// positions of its ones, and each position is turned back into the
// (query id, point id) pair of Sec. II-A1.
#include "ersj_internal.h"

namespace ersj {

namespace {

// One workgroup of kBandLists threads: keep min(count, lcap) entries of each
// band sub-list, prefix them, and report the total kept and the largest
// count (a count above lcap means the lists must grow).
__global__ __launch_bounds__(kBandLists) void k_band_prefix(const unsigned long long *__restrict__ bcount,
                                                            uint64_t lcap, uint64_t *__restrict__ lpref,
                                                            uint64_t *__restrict__ out)
{
    __shared__ uint64_t sc[kBandLists];
    __shared__ uint64_t sm[kBandLists];
    const uint32_t t = threadIdx.x;
    const uint64_t c = bcount[(uint64_t)t * kBandStride];
    sc[t] = c < lcap ? c : lcap;
    sm[t] = c;
    __syncthreads();
    if (t == 0) {
        uint64_t run = 0, mx = 0;
        for (uint32_t i = 0; i < kBandLists; ++i) {
            lpref[i] = run;
            run += sc[i];
            mx = sm[i] > mx ? sm[i] : mx;
        }
        lpref[kBandLists] = run;
        out[0] = run;
        out[1] = mx;
    }
}

// Binary64 squared distance in the input's own dimension order, every
// operation separately rounded (no contraction): the exact definition the
// result set is specified by.  Pairs at or below fl(eps*eps) get their bit.
// Both rows are read from row-major copies in sorted order (a row's d
// floats are contiguous: a few cache lines per pair).  Entry i of the kept
// band pairs lives in sub-list c (lpref[c] <= i < lpref[c+1]) at offset
// i - lpref[c].
__global__ __launch_bounds__(256) void k_recheck(const Boundary *__restrict__ bl, uint64_t lcap,
                                                 const uint64_t *__restrict__ lpref, uint64_t cnt,
                                                 const float *__restrict__ xr, const float *__restrict__ xqr,
                                                 int32_t d, double e64, uint64_t *__restrict__ mask,
                                                 uint8_t *__restrict__ gflag,
                                                 unsigned long long *__restrict__ nin,
                                                 uint32_t *__restrict__ rowcnt, uint64_t row_base)
{
#pragma clang fp contract(off)
    __shared__ uint64_t spref[kBandLists + 1];
    __shared__ uint32_t s_hits;
    for (uint32_t k = threadIdx.x; k <= kBandLists; k += blockDim.x) spref[k] = lpref[k];
    if (threadIdx.x == 0) s_hits = 0;
    __syncthreads();
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool hit = false;
    if (i < cnt) {
        uint32_t lo = 0, hi = kBandLists;  // largest c with spref[c] <= i
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (spref[mid] <= i) lo = mid;
            else hi = mid;
        }
        const Boundary e = bl[(uint64_t)lo * lcap + (i - spref[lo])];
        const float *qa = xqr + (uint64_t)e.q * (uint64_t)d;
        const float *xb = xr + (uint64_t)e.x * (uint64_t)d;
        double s = 0.0;
        for (int k = 0; k < d; ++k) {
            const double a = (double)qa[k];
            const double b = (double)xb[k];
            const double t = a - b;
            const double tt = t * t;
            s = s + tt;
        }
        if (s <= e64) {
            atomicOr((unsigned long long *)&mask[e.bit >> 6], 1ull << (e.bit & 63));
            gflag[e.bit >> 8] = 1;  // its 4-word unit now holds a bit
            atomicAdd(&rowcnt[e.q - row_base], 1u);
            hit = true;
        }
    }
    // one counter update per workgroup, into its slot
    const uint64_t hits = __ballot(hit);
    if (hits != 0 && (threadIdx.x & 63) == (uint32_t)(__ffsll((unsigned long long)hits) - 1))
        atomicAdd(&s_hits, (uint32_t)__popcll(hits));
    __syncthreads();
    if (threadIdx.x == 0 && s_hits != 0)
        atomicAdd(&nin[(uint64_t)(blockIdx.x % kHitSlots) * kBandStride], (unsigned long long)s_hits);
}

// position of the r-th (0-based) set bit of w; r < popcount(w)
__device__ __forceinline__ int nth_bit(uint64_t w, uint32_t r)
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

// Workgroup per row tile of the batch, wave per row.  A row's unit flags
// (one per 4 mask words) are read 256 at a time, four independent loads per
// lane, and the flagged units are listed in LDS in order; then the words of
// up to 16 listed units are staged with their bit prefix and their set bits
// are dealt to the lanes in turn (lane j takes the staged set bits j,
// j + 64, ...), so only flagged words are read, the pairs of a dense word
// are written by 64 lanes at once, and each wave's stores are consecutive.
// Pairs come out in candidate order.
__global__ __launch_bounds__(256) void k_expand(const Tile *__restrict__ tiles, uint32_t t0,
                                                const uint64_t *__restrict__ toff, uint64_t wbase,
                                                uint64_t row_base, const uint64_t *__restrict__ mask,
                                                const uint8_t *__restrict__ gflag,
                                                const uint64_t *__restrict__ roff,
                                                const uint32_t *__restrict__ rstart,
                                                const uint32_t *__restrict__ rpref,
                                                const uint32_t *__restrict__ nrng,
                                                const uint32_t *__restrict__ qorig,
                                                const uint32_t *__restrict__ orig,
                                                uint32_t *__restrict__ pairs)
{
    constexpr uint32_t kChunk = 256;  // unit flags scanned per pass
    __shared__ uint32_t s_pref[kMaxRanges + 1];
    __shared__ uint32_t s_start[kMaxRanges];
    __shared__ uint64_t s_words[4][64];
    __shared__ uint32_t s_widx[4][64];
    __shared__ uint32_t s_before[4][64];
    __shared__ uint32_t s_units[4][kChunk];
    const uint32_t t = t0 + blockIdx.x;
    const Tile tl = tiles[t];
    const uint32_t A = tl.cell;
    const uint32_t nr = nrng[A];
    if (threadIdx.x <= kMaxRanges)
        s_pref[threadIdx.x] = threadIdx.x <= nr ? rpref[(uint64_t)A * (kMaxRanges + 1) + threadIdx.x] : 0xffffffffu;
    if (threadIdx.x < kMaxRanges) s_start[threadIdx.x] = rstart[(uint64_t)A * kMaxRanges + threadIdx.x];
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint64_t *const cw = s_words[wave];
    uint32_t *const ci = s_widx[wave];
    uint32_t *const cb = s_before[wave];
    uint32_t *const lu = s_units[wave];
    const uint64_t tbase = toff[t] - wbase;
    const uint32_t nunits = (tl.used + 3) / 4;
    const bool al8 = ((uintptr_t)pairs & 7u) == 0;  // a pair in one 8-byte store
    for (uint32_t r = wave; r < tl.nrows; r += 4) {
        const uint32_t q = tl.row0 + r;
        const uint32_t qid = qorig[q];
        const uint64_t rw = tbase + (uint64_t)r * tl.words;  // first word of the row (a multiple of 8)
        const uint64_t *row = mask + rw;
        const uint8_t *frow = gflag + (rw >> 2);
        uint64_t out = roff[q - row_base];
        for (uint32_t c0 = 0; c0 < nunits; c0 += kChunk) {
            // the chunk's flags, four independent loads per lane, then the
            // flagged units listed in order
            uint8_t f[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t u = c0 + 64 * k + lane;
                f[k] = u < nunits ? frow[u] : 0;
            }
            uint32_t nf = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t nz = __ballot(f[k] != 0);
                if (f[k] != 0) lu[nf + __popcll(nz & ((1ull << lane) - 1ull))] = c0 + 64 * k + lane;
                nf += __popcll(nz);
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            for (uint32_t i0 = 0; i0 < nf; i0 += 16) {
                const uint32_t cnt = min(16u, nf - i0);
                const uint32_t slot = (uint32_t)lane >> 2;
                uint64_t m = 0ull;
                uint32_t wi = 0;
                if (slot < cnt) {
                    wi = lu[i0 + slot] * 4 + (lane & 3);
                    m = wi < tl.used ? row[wi] : 0ull;
                }
                const uint32_t pc = __popcll(m);
                uint32_t inc = pc;
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
                for (uint32_t j = lane; j < total; j += 64) {
                    int lo = 0, hi = 63;  // the last staged word with cb[word] <= j
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (cb[mid] <= j) lo = mid;
                        else hi = mid - 1;
                    }
                    const uint32_t p = ci[lo] * 64 + nth_bit(cw[lo], j - cb[lo]);
                    const int g = range_of(s_pref, nr, p);
                    const uint32_t x = s_start[g] + (p - s_pref[g]);
                    const uint64_t pos = out + j;
                    if (al8) {
                        ((uint2 *)pairs)[pos] = make_uint2(qid, orig[x]);
                    } else {
                        pairs[2 * pos] = qid;
                        pairs[2 * pos + 1] = orig[x];
                    }
                }
                out += total;
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            }
        }
    }
}

}  // namespace

hipError_t launch_band_prefix(const unsigned long long *bcount, uint64_t lcap, uint64_t *lpref,
                              uint64_t *out, hipStream_t s)
{
    hipLaunchKernelGGL(k_band_prefix, dim3(1), dim3(kBandLists), 0, s, bcount, lcap, lpref, out);
    return hipGetLastError();
}

hipError_t launch_recheck(const Boundary *bl, uint64_t lcap, const uint64_t *lpref, uint64_t cnt,
                          const float *xr, const float *xqr, int32_t d, double e64, uint64_t *mask,
                          uint8_t *gflag, unsigned long long *nin, uint32_t *rowcnt, uint64_t row_base,
                          hipStream_t s)
{
    if (cnt == 0) return hipSuccess;
    const uint64_t blocks = (cnt + 255) / 256;
    hipLaunchKernelGGL(k_recheck, dim3((unsigned)blocks), dim3(256), 0, s, bl, lcap, lpref, cnt, xr, xqr,
                       d, e64, mask, gflag, nin, rowcnt, row_base);
    return hipGetLastError();
}

hipError_t launch_expand(const Tile *tiles, uint32_t t0, uint32_t ntiles, const uint64_t *toff,
                         uint64_t wbase, uint64_t row_base, const uint64_t *mask, const uint8_t *gflag,
                         const uint64_t *roff, const uint32_t *rstart, const uint32_t *rpref,
                         const uint32_t *nrng, const uint32_t *qorig, const uint32_t *orig,
                         uint32_t *pairs, hipStream_t s)
{
    if (ntiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_expand, dim3(ntiles), dim3(256), 0, s, tiles, t0, toff, wbase, row_base, mask,
                       gflag, roff, rstart, rpref, nrng, qorig, orig, pairs);
    return hipGetLastError();
}

}  // namespace ersj
