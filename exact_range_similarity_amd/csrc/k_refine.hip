// Candidate refinement for gfx950 (direct form on the vector ALUs).
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. IV-E (one thread block per group of queries
// sharing the same candidates; coordinates read dimension-major) and
// Sec. IV-F (one result bit per query/candidate comparison).
//
// Work item: (32 rows of a row tile of one cell, segment of the cell's
// candidate list).  A 256-thread workgroup holds 4 waves; wave w owns
// queries 8w..8w+7 of those 32 rows.  Lane l of a wave owns candidates
// c + l + 64j (j = 0..3) of each 256-candidate chunk, so one wave ballot of a
// comparison yields exactly one 64-bit mask word: bit l <-> candidate
// 64*word + l.  Query coordinates are wave-uniform (scalar loads); candidate
// coordinates come from the dimension-blocked layout, so a wave's load of a
// block is 1 KiB contiguous.  Every mask word of the tile's rows is written
// once, by exactly one wave, so the mask needs no clearing.
//
// Classification (fp32 squared distance s, binary64 reference D64):
//   s <= tlo           -> neighbour (bit set)
//   s >  thi           -> not a neighbour
//   otherwise          -> boundary: appended to a list and decided in
//                         binary64 by the re-check kernel.
// tlo and thi come from a forward error bound that holds for any summation
// order, so the dimension order used here (by variance) is free.
//
// Block pruning: before a chunk, the wave compares the bounding box of its
// 8 queries with that of the chunk's 256 candidates on the three grid axes
// (block 0 of the layout); when their squared gap exceeds tbox no pair in
// them is a neighbour, and the wave writes zero words without computing.
#include "ersj_internal.h"

namespace ersj {

namespace {

constexpr int kQW = 8;   // queries per wave
constexpr int kCW = 4;   // candidates per lane per chunk
constexpr int kChunk = 64 * kCW;

__global__ __launch_bounds__(256) void k_refine_direct(RefineArgs a)
{
    uint32_t rk, colx;
    work_item(blockIdx.x, a.ntiles, a.nseg * a.nsub, &rk, &colx);
    const uint32_t seg = colx / a.nsub, sub = colx - seg * a.nsub;
    const uint32_t t = a.order[a.ord0 + rk];
    const Tile tl = a.tiles[t];
    const uint32_t r_begin = sub * 32;  // rows of this work item: 32 from r_begin
    if (r_begin >= tl.nrows) return;
    const uint32_t srows = min(32u, tl.nrows - r_begin);
    const uint32_t A = tl.cell;
    const uint32_t nr = a.nrng[A];
    const uint32_t *pref_g = a.rpref + (uint64_t)A * (kMaxRanges + 1);
    const uint32_t U = pref_g[nr];
    const uint32_t c_begin = seg * a.seg_len;
    if (c_begin >= U) return;
    const uint32_t c_end = min(U, c_begin + a.seg_len);

    __shared__ uint32_t s_pref[kMaxRanges + 1];
    __shared__ uint32_t s_start[kMaxRanges];
    if (threadIdx.x <= kMaxRanges) s_pref[threadIdx.x] = threadIdx.x <= nr ? pref_g[threadIdx.x] : 0xffffffffu;
    if (threadIdx.x < kMaxRanges) s_start[threadIdx.x] = a.rstart[(uint64_t)A * kMaxRanges + threadIdx.x];
    __syncthreads();

    // wave index made provably uniform so query addresses use scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t kq0 = wave * kQW;
    if (kq0 >= srows) return;
    uint32_t qrow[kQW];
#pragma unroll
    for (int k = 0; k < kQW; ++k) qrow[k] = tl.row0 + r_begin + min(kq0 + k, srows - 1);
    const uint32_t nq = min((uint32_t)kQW, srows - kq0);
    const uint64_t mbase = a.toff[t] - a.wbase + (uint64_t)(r_begin + kq0) * tl.words;
    const uint64_t n = a.n;
    const float4 *__restrict__ xs = a.xs;
    const float4 *__restrict__ xq = a.xq;  // query rows (the points themselves in a self-join)
    uint64_t *__restrict__ mask = a.mask;
    Boundary *__restrict__ blist = band_list(a.blist, a.lcap);
    unsigned long long *__restrict__ bcount = band_counter(a.bcount);

    // the wave's query box over the first kBoxBlocks layout blocks (rows past
    // srows repeat the last; blocks past nb are zero padding)
    const uint64_t nqr = a.nqr;
    const int nb = a.nb;
    float4 qlo[kBoxBlocks], qhi[kBoxBlocks];
#pragma unroll
    for (int b = 0; b < kBoxBlocks; ++b) {
        qlo[b] = qhi[b] = b < nb ? xq[(uint64_t)b * nqr + qrow[0]] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 1; k < kQW; ++k) {
            const float4 q = b < nb ? xq[(uint64_t)b * nqr + qrow[k]] : make_float4(0.f, 0.f, 0.f, 0.f);
            qlo[b] = make_float4(fminf(qlo[b].x, q.x), fminf(qlo[b].y, q.y), fminf(qlo[b].z, q.z), fminf(qlo[b].w, q.w));
            qhi[b] = make_float4(fmaxf(qhi[b].x, q.x), fmaxf(qhi[b].y, q.y), fmaxf(qhi[b].z, q.z), fmaxf(qhi[b].w, q.w));
        }
    }
    const float tbox = a.tbox;
    uint64_t nskip = 0;
    uint32_t mycnt = 0;  // bits set in this lane's mask words (lane = query k * 4 + word j)

    for (uint32_t c = c_begin; c < c_end; c += kChunk) {
        uint32_t xi[kCW];
        bool xv[kCW];
#pragma unroll
        for (int j = 0; j < kCW; ++j) {
            const uint32_t p = c + lane + 64 * j;
            xv[j] = p < c_end;
            const uint32_t pp = xv[j] ? p : c_begin;
            const int g = range_of(s_pref, nr, pp);
            xi[j] = s_start[g] + (pp - s_pref[g]);
        }
        {
            float g2 = 0.f;
#pragma unroll
            for (int b = 0; b < kBoxBlocks; ++b) {
                float4 lo = make_float4(INFINITY, INFINITY, INFINITY, INFINITY);
                float4 hi = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
#pragma unroll
                for (int j = 0; j < kCW; ++j) {
                    if (xv[j]) {
                        const float4 v = b < nb ? xs[(uint64_t)b * n + xi[j]] : make_float4(0.f, 0.f, 0.f, 0.f);
                        lo = make_float4(fminf(lo.x, v.x), fminf(lo.y, v.y), fminf(lo.z, v.z), fminf(lo.w, v.w));
                        hi = make_float4(fmaxf(hi.x, v.x), fmaxf(hi.y, v.y), fmaxf(hi.z, v.z), fmaxf(hi.w, v.w));
                    }
                }
                wave_box4(lo, hi);
                g2 = gap4(qlo[b], qhi[b], lo, hi, g2);
            }
            if (__builtin_amdgcn_readfirstlane((int)(g2 > tbox)) != 0) {
                nskip += (uint64_t)nq * min((uint32_t)kChunk, c_end - c);
                if (lane < kQW * kCW) {
                    const int k = lane / kCW, j = lane % kCW;
                    const uint32_t w = (c >> 6) + j;
                    if ((uint32_t)k < nq && w < tl.words) mask[mbase + (uint64_t)k * tl.words + w] = 0ull;
                    // the chunk's 4 words are one flag unit
                    if (j == 0 && (uint32_t)k < nq && w < tl.words) a.gflag[(mbase + (uint64_t)k * tl.words + w) >> 2] = 0;
                }
                continue;
            }
        }
        float acc[kQW][kCW];
#pragma unroll
        for (int k = 0; k < kQW; ++k)
#pragma unroll
            for (int j = 0; j < kCW; ++j) acc[k][j] = 0.0f;

        for (int b = 0; b < a.nb; ++b) {
            const float4 *xb = xs + (uint64_t)b * n;
            float4 xv4[kCW];
#pragma unroll
            for (int j = 0; j < kCW; ++j) xv4[j] = xb[xi[j]];
#pragma unroll
            for (int k = 0; k < kQW; ++k) {
                const float4 q = xq[(uint64_t)b * a.nqr + qrow[k]];
#pragma unroll
                for (int j = 0; j < kCW; ++j) {
                    float t0 = q.x - xv4[j].x;
                    float t1 = q.y - xv4[j].y;
                    float t2 = q.z - xv4[j].z;
                    float t3 = q.w - xv4[j].w;
                    float s = acc[k][j];
                    s = fmaf(t0, t0, s);
                    s = fmaf(t1, t1, s);
                    s = fmaf(t2, t2, s);
                    s = fmaf(t3, t3, s);
                    acc[k][j] = s;
                }
            }
        }

        const uint32_t w0 = c >> 6;
        uint64_t myword = 0;
#pragma unroll
        for (int k = 0; k < kQW; ++k) {
#pragma unroll
            for (int j = 0; j < kCW; ++j) {
                const float s = acc[k][j];
                const bool in = xv[j] && s <= a.tlo;
                const bool bd = xv[j] && !(s <= a.tlo) && s <= a.thi;
                const uint64_t win = __ballot(in);
                const uint64_t wb = __ballot(bd);
                if (lane == k * kCW + j) myword = win;
                if (wb != 0 && (uint32_t)k < nq) {
                    const uint32_t cnt = __popcll(wb);
                    const int first = __ffsll((unsigned long long)wb) - 1;
                    unsigned long long base = 0;
                    if (lane == first) base = atomicAdd(bcount, (unsigned long long)cnt);
                    base = __shfl(base, first, 64);
                    if (bd) {
                        const uint64_t below = lane == 0 ? 0ull : (wb & (~0ull >> (64 - lane)));
                        const uint64_t idx = base + __popcll(below);
                        if (idx < a.lcap) {
                            Boundary e;
                            e.q = qrow[k];
                            e.x = xi[j];
                            e.bit = (mbase + (uint64_t)k * tl.words + w0 + j) * 64 + lane;
                            blist[idx] = e;
                        }
                    }
                }
            }
        }
        {
            const int k = lane / kCW, j = lane % kCW;
            const bool ok = lane < kQW * kCW && (uint32_t)k < nq && w0 + j < tl.words;
            if (ok) {
                mask[mbase + (uint64_t)k * tl.words + w0 + j] = myword;
                mycnt += __popcll(myword);
            }
            // the chunk's 4 words of a query are one flag unit (lanes 4k .. 4k+3)
            const uint64_t nzb = __ballot(ok && myword != 0);
            if (lane < kQW * kCW && j == 0 && (uint32_t)k < nq && w0 < tl.words)
                a.gflag[(mbase + (uint64_t)k * tl.words + w0) >> 2] = ((nzb >> lane) & 0xfull) ? 1 : 0;
        }
    }
    if (nskip != 0 && lane == 0)
        atomicAdd(&a.skipped[(uint64_t)(blockIdx.x % kHitSlots) * kBandStride], (unsigned long long)nskip);
    // the rows' neighbour counts (the binary64 re-check adds the band's):
    // the kCW lanes of a query sum their words' counts
    mycnt += __shfl_down(mycnt, 2, kCW);
    mycnt += __shfl_down(mycnt, 1, kCW);
    if (lane < kQW * kCW && lane % kCW == 0 && (uint32_t)(lane / kCW) < nq && mycnt != 0)
        atomicAdd(&a.rowcnt[tl.row0 + r_begin + kq0 + (uint32_t)(lane / kCW) - a.row_base], mycnt);
}

}  // namespace

hipError_t launch_refine_direct(const RefineArgs &a, hipStream_t s)
{
    const uint64_t blocks = (uint64_t)a.ntiles * a.nseg * a.nsub;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_refine_direct, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ersj
