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
// Both rows are read from row-major copies in sorted order, rows ldr
// floats apart (ldr: d rounded up to 4, the floats past d zero in both
// copies, so that their terms add an exact +0 to a sum that is never
// negative).  A lane takes its two rows 32 floats (one 128-byte line each)
// at a time: the 16 loads of a line pair are issued together, then its 32
// terms are summed in order.  The last chunk re-reads the row's last float4
// in place of those past its end and skips their terms.  Entry i of the kept
// band pairs lives in sub-list c (lpref[c] <= i < lpref[c+1]) at offset
// i - lpref[c].
constexpr int kRecheckChunk = 8;  // float4 per row per chunk
__global__ __launch_bounds__(256) void k_recheck(const Boundary *__restrict__ bl, uint64_t lcap,
                                                 const uint64_t *__restrict__ lpref, uint64_t cnt,
                                                 const float *__restrict__ xr, const float *__restrict__ xqr,
                                                 int32_t ldr, double e64, uint64_t *__restrict__ mask,
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
        const float4 *qa = (const float4 *)(xqr + (uint64_t)e.q * (uint64_t)ldr);
        const float4 *xb = (const float4 *)(xr + (uint64_t)e.x * (uint64_t)ldr);
        const int n4 = ldr >> 2;
        double s = 0.0;
        auto term = [&](float a, float b) __attribute__((always_inline)) {
            const double t = (double)a - (double)b;
            const double tt = t * t;
            s = s + tt;
        };
        int k4 = 0;
#pragma unroll 1
        for (; k4 + kRecheckChunk <= n4; k4 += kRecheckChunk) {
            float4 qv[kRecheckChunk], xv[kRecheckChunk];
#pragma unroll
            for (int c = 0; c < kRecheckChunk; ++c) {
                qv[c] = qa[k4 + c];
                xv[c] = xb[k4 + c];
            }
#pragma unroll
            for (int c = 0; c < kRecheckChunk; ++c) {
                term(qv[c].x, xv[c].x);
                term(qv[c].y, xv[c].y);
                term(qv[c].z, xv[c].z);
                term(qv[c].w, xv[c].w);
            }
        }
        if (k4 < n4) {
            float4 qv[kRecheckChunk], xv[kRecheckChunk];
#pragma unroll
            for (int c = 0; c < kRecheckChunk; ++c) {
                const int k = k4 + c < n4 ? k4 + c : n4 - 1;
                qv[c] = qa[k];
                xv[c] = xb[k];
            }
#pragma unroll
            for (int c = 0; c < kRecheckChunk; ++c) {
                if (k4 + c < n4) {
                    term(qv[c].x, xv[c].x);
                    term(qv[c].y, xv[c].y);
                    term(qv[c].z, xv[c].z);
                    term(qv[c].w, xv[c].w);
                }
            }
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

// position of the r-th (0-based) set bit of w; r < popcount(w).  Halving
// search in 32-bit pieces: at each width the low half's bit count decides
// which half holds the bit.
__device__ __forceinline__ int nth_bit(uint64_t w, uint32_t r)
{
    const uint32_t lo = (uint32_t)w;
    uint32_t c = (uint32_t)__popc(lo);
    const bool up = r >= c;
    uint32_t v = up ? (uint32_t)(w >> 32) : lo;
    int pos = up ? 32 : 0;
    r = up ? r - c : r;
#pragma unroll
    for (int sh = 16; sh > 0; sh >>= 1) {
        c = (uint32_t)__popc(v & ((1u << sh) - 1u));
        const bool u = r >= c;
        v = u ? v >> sh : v;
        pos += u ? sh : 0;
        r = u ? r - c : r;
    }
    return pos;
}

// Workgroup per row tile of the batch, all 256 threads on one pass at a
// time, so that a tile costs a few memory round trips rather than a few per
// row.  The tile's unit flags (one byte per 4 mask words; its rows' flag
// bytes are consecutive, words / 4 per row) are read 4 KiB per pass, four
// independent loads per thread, and the flagged units are listed in LDS in
// row-then-unit order.  The listed units are then taken 64 at a time: each
// thread loads one of their 256 words, a workgroup prefix sum of the words'
// bit counts places every set bit, and the bits are dealt to the threads in
// turn (thread i takes bits i, i + 256, ...).  A bit finds its word through
// a bit map of the words' first output bits and, per 64 output bits, the
// word that holds the first; a word's range of the cell's list is looked up
// once per word.  The tile's pairs fill its output range in row-then-
// candidate order, so bit j of a batch goes to the running offset + j.
constexpr uint32_t kFlagPass = 4096;   // flag bytes read per pass
constexpr uint32_t kUnitBatch = 64;    // listed units expanded per batch (256 words)
static_assert(kTileRows < 255, "rows of a tile are held in bytes (0xff: no row)");

// Exclusive prefix sum of v over the workgroup's 256 threads in thread
// order; *total gets the sum.  wtot: 4 words of LDS.  Ends with a barrier.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wtot, uint32_t *total)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
    }
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t t = wtot[w];
        before += w < wave ? t : 0u;
        all += t;
    }
    *total = all;
    return before + inc - v;
}

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
    __shared__ uint32_t s_pref[kMaxRanges + 1];
    __shared__ uint32_t s_start[kMaxRanges];
    __shared__ uint16_t s_list[kFlagPass];   // pass-relative byte offsets of flagged units
    __shared__ uint32_t s_ftot[16];          // flagged bytes per (load k, wave)
    __shared__ uint32_t s_wtot[4];
    // the batch's non-empty words in output order (index e), and the bit map
    // of their first output bits (256 x 64 bits: a batch holds at most 16384)
    __shared__ uint64_t s_word[256];
    __shared__ uint64_t s_starts[256];
    __shared__ uint32_t s_wi[256];       // word index in its row
    __shared__ uint32_t s_goff[256];     // point - candidate in the range of the word's first candidate
    __shared__ uint32_t s_gend[256];     // end of that range
    __shared__ uint16_t s_excl[256];     // first output bit
    __shared__ uint16_t s_first[256];    // non-empty word holding output bit 64 c
    __shared__ uint8_t s_erow[256];
    __shared__ uint32_t s_qid[kTileRows];
    const uint32_t t = t0 + blockIdx.x;
    const Tile tl = tiles[t];
    const uint32_t A = tl.cell;
    const uint32_t nr = nrng[A];
    const uint32_t tid = threadIdx.x;
    if (tid <= kMaxRanges) s_pref[tid] = tid <= nr ? rpref[(uint64_t)A * (kMaxRanges + 1) + tid] : 0xffffffffu;
    if (tid < kMaxRanges) s_start[tid] = rstart[(uint64_t)A * kMaxRanges + tid];
    if (tid < tl.nrows) s_qid[tid] = qorig[tl.row0 + tid];
    // the tile's rows own one contiguous output range, filled in row order
    // (a row's bits all lie in its flagged units, counted in its row count):
    // the batches' bits, taken in row-then-candidate order, land at
    // consecutive positions from the first row's offset
    uint64_t pos0 = roff[tl.row0 - row_base];
    const uint64_t tbase = toff[t] - wbase;         // first word of the tile (a multiple of 8)
    const uint64_t fb = tbase >> 2;                  // its first flag byte
    const uint32_t fstride = tl.words >> 2;          // flag bytes per row
    // o / fstride for a tile byte o (quotient < kTileRows): a float estimate,
    // off by at most one, then corrected
    const float frcp = 1.0f / (float)fstride;
    auto row_of = [&](uint32_t o) __attribute__((always_inline)) {
        uint32_t r = (uint32_t)((float)o * frcp);
        r = r * fstride > o ? r - 1 : r;
        r = (r + 1) * fstride <= o ? r + 1 : r;
        return r;
    };
    const uint32_t nunits = (tl.used + 3) >> 2;      // units that hold candidates
    const uint64_t nbytes = (uint64_t)tl.nrows * fstride;  // below 2^32 (rows <= kTileRows)
    if (nbytes == 0) return;                           // uniform: no barrier passed yet
    const uint32_t *gf32 = (const uint32_t *)gflag;  // 4-byte loads from the aligned dword below fb
    const uint64_t d0 = fb >> 2, d1 = (fb + nbytes + 3) >> 2;
    const bool al8 = ((uintptr_t)pairs & 7u) == 0;  // a pair in one 8-byte store
    const int wave = tid >> 6, lane = tid & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    __syncthreads();
    for (uint64_t c = d0; c < d1; c += kFlagPass / 4) {
        // flag dwords c + 256 k + tid; byte b of dword di is tile byte
        // 4 di + b - fb, listed if non-zero, inside the tile and on a unit
        // that holds candidates
        uint32_t f[4], fm[4], cnt[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t di = c + 256 * k + tid;
            f[k] = di < d1 ? gf32[di] : 0u;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t m = 0;
            if (f[k] != 0u) {
                const uint64_t di = c + 256 * k + tid;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int64_t o = (int64_t)(4 * di + b) - (int64_t)fb;
                    if (((f[k] >> (8 * b)) & 0xffu) != 0u && o >= 0 && (uint64_t)o < nbytes &&
                        (uint32_t)o - row_of((uint32_t)o) * fstride < nunits)
                        m |= 1u << b;
                }
            }
            fm[k] = m;
            cnt[k] = __popc(m);
        }
        // order: load k, then wave, lane, byte; counts 0..4 in three bit planes
        uint32_t pre[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t b0 = __ballot(cnt[k] & 1u), b1 = __ballot(cnt[k] & 2u), b2 = __ballot(cnt[k] & 4u);
            pre[k] = __popcll(b0 & below) + 2 * __popcll(b1 & below) + 4 * __popcll(b2 & below);
            if (lane == 0) s_ftot[4 * k + wave] = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
        }
        __syncthreads();
        uint32_t nl = 0, base[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (w == wave) base[k] = nl;
                nl += s_ftot[4 * k + w];
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t i = base[k] + pre[k];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (fm[k] & (1u << b)) s_list[i++] = (uint16_t)(4 * (256 * k + tid) + b);
        }
        __syncthreads();
        // thread tid: word tid & 3 of listed unit i0 + tid / 4; the next
        // batch's word is loaded while this batch's bits are expanded
        auto load_word = [&](uint32_t i0, uint64_t *m, uint32_t *wi, uint32_t *row) __attribute__((always_inline)) {
            const uint32_t e = i0 + (tid >> 2);
            *m = 0ull;
            *wi = 0;
            *row = 0xffu;
            if (e < nl) {
                const uint32_t o = (uint32_t)(4 * c + s_list[e] - fb);
                *row = row_of(o);
                *wi = (o - *row * fstride) * 4 + (tid & 3);
                if (*wi < tl.used) *m = mask[tbase + (uint64_t)*row * tl.words + *wi];
            }
        };
        uint64_t m_next = 0ull;
        uint32_t wi_next = 0, row_next = 0xffu;
        if (nl > 0) load_word(0, &m_next, &wi_next, &row_next);
        for (uint32_t i0 = 0; i0 < nl; i0 += kUnitBatch) {
            const uint64_t m = m_next;
            const uint32_t wi = wi_next, row = row_next;
            if (i0 + kUnitBatch < nl) load_word(i0 + kUnitBatch, &m_next, &wi_next, &row_next);
            const uint32_t pc = __popcll(m);
            s_starts[tid] = 0ull;
            // one scan for both the bit offsets (low 16 bits, at most 16384)
            // and the ranks of the non-empty words (high bits)
            uint32_t tot;
            const uint32_t ex = block_excl_scan(pc | (pc != 0u ? 1u << 16 : 0u), s_wtot, &tot);
            const uint32_t excl = ex & 0xffffu, e = ex >> 16, total = tot & 0xffffu;
            if (pc != 0u) {
                s_word[e] = m;
                s_wi[e] = wi;
                s_excl[e] = (uint16_t)excl;
                s_erow[e] = (uint8_t)row;
                const int g = range_of(s_pref, nr, wi * 64);
                s_goff[e] = s_start[g] - s_pref[g];
                s_gend[e] = s_pref[g + 1];
                atomicOr((unsigned long long *)&s_starts[excl >> 6], 1ull << (excl & 63u));
                const uint32_t c = (excl + 63u) >> 6;  // a 64-bit boundary inside the word's bits
                if (64u * c < excl + pc) s_first[c] = (uint16_t)e;
            }
            __syncthreads();
            // bit j of the batch -> (output position, query id, point): its
            // word is the last one starting at or before j, counted from the
            // word that holds bit 64 (j / 64); two bits per thread at a
            // time, so two gathers of orig are in flight
            auto locate = [&](uint32_t j, uint64_t *pos, uint32_t *qid, uint32_t *x) __attribute__((always_inline)) {
                const uint32_t c = j >> 6, b = j & 63u;
                const uint64_t after = ((2ull << b) - 1ull) & ~1ull;  // bits 1..b
                const uint32_t e = s_first[c] + (uint32_t)__popcll(s_starts[c] & after);
                const uint32_t p = s_wi[e] * 64 + (uint32_t)nth_bit(s_word[e], j - s_excl[e]);
                *x = p < s_gend[e] ? p + s_goff[e] : [&]() {
                    const int g = range_of(s_pref, nr, p);
                    return s_start[g] + (p - s_pref[g]);
                }();
                *qid = s_qid[s_erow[e]];
                *pos = pos0 + j;
            };
            auto put = [&](uint64_t pos, uint32_t qid, uint32_t id) __attribute__((always_inline)) {
                if (al8) {
                    ((uint2 *)pairs)[pos] = make_uint2(qid, id);
                } else {
                    pairs[2 * pos] = qid;
                    pairs[2 * pos + 1] = id;
                }
            };
            for (uint32_t j = tid; j < total; j += 512) {
                uint64_t pa, pb = 0;
                uint32_t qa, xa, qb = 0, xb = 0;
                const bool two = j + 256 < total;
                locate(j, &pa, &qa, &xa);
                if (two) locate(j + 256, &pb, &qb, &xb);
                const uint32_t ia = orig[xa];
                const uint32_t ib = two ? orig[xb] : 0u;
                put(pa, qa, ia);
                if (two) put(pb, qb, ib);
            }
            pos0 += total;
            __syncthreads();
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
                          const float *xr, const float *xqr, int32_t d, int32_t ldr, double e64, uint64_t *mask,
                          uint8_t *gflag, unsigned long long *nin, uint32_t *rowcnt, uint64_t row_base,
                          hipStream_t s)
{
    if (ldr < d || (ldr & 3) != 0 || ldr <= 0) return hipErrorInvalidValue;
    if (cnt == 0) return hipSuccess;
    const uint64_t blocks = (cnt + 255) / 256;
    hipLaunchKernelGGL(k_recheck, dim3((unsigned)blocks), dim3(256), 0, s, bl, lcap, lpref, cnt, xr, xqr,
                       ldr, e64, mask, gflag, nin, rowcnt, row_base);
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
