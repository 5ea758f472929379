// Candidate refinement for gfx950, split-fp16 form on MFMA, for more than 64
// dimensions, with operands prepared once per point.
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. IV-E (a thread block per group of queries that
// share their candidates, staged through on-chip memory) and Sec. IV-F (one
// result bit per comparison).
//
// The split-fp16 arithmetic of k_refine_mfma.hip with one reference point
// for all pairs, the per-dimension mean r of the points (fp32): every point
// and query row is centred and scaled once, v = fl((x - r) s) (computed as
// fma(x, s, -(r s)), the same value while r s is exact), split into fp16
// halves and stored with its fp32 norm |v|^2 (k_prep16).  The band analysis
// of the split form holds for any fp32 reference shared by the two points of
// a pair; a single one pays off when the data lie around a common centre (for
// unit-norm rows the norms are about 1, less than the squared distance
// between two rows), and in high dimension it takes the centring and
// splitting out of the refinement loop, whose arithmetic is then the matrix
// products alone.
//
// Work item: (row tile of up to 128 query rows of one cell, segment of the
// cell's candidate list), in steps of 256 candidates.  Wave w computes rows
// 64 (w % 2) .. +63 against candidates 128 (w / 2) .. +127 of a step: two
// 32-row blocks times four 32-candidate groups, eight 32 x 32 accumulators.
// The step runs over the 16-dimension slabs; each slab's fp16 halves of the
// tile's rows (8 KiB) and of the step's candidates (16 KiB) are copied from
// HBM into one of two LDS buffers while the previous slab's 24 MFMAs per wave
// run: one barrier per slab.  After the last slab the accumulators are
// classified (classify_block, same band and thresholds as k_refine_mfma) and
// mask words leave every 512 candidates as aligned 64-byte row pieces.
//
// High parts only (HH): the dot product is the sum of the high-half
// products alone, one MFMA per slab instead of three.  Dropping h.l + l.h +
// l.l changes s^2 q'.x' by at most 2^-10 (1 + 2^-12) sum |v_q v_x| plus
// 2^-25 (|v_q| + |v_x|) (1 + 2^-11) + 2^-50 per dimension (|v - h| <=
// 2^-11 |v| + 2^-25), so the band grows by 2^-10 (1 + 2^-12) (Nq + Nx) and
// more pairs go to the binary64 re-check; the absolute part stays within
// the split form's absolute widening.  The prepared operands then hold the
// high halves only, two slabs in place of one slab's four parts, so a stage
// covers 32 dimensions with the same loads and LDS traffic as a 16-dimension
// stage of the three-product form, and runs 16 MFMAs per wave instead of 24.
//
// Partial test: the squared distance over the first kPartialDims dimensions
// of the layout bounds the full one from below.  After the stage that ends
// with dimension kPartialDims - 1, every 32 x 32 block is tested with the
// "out" rule of the classification, with the norms over those dimensions in
// place of the full ones (the same band coefficient: the partial value has
// fewer terms and fewer MFMA instructions behind it).  A block whose pairs
// are all out keeps zero bits and runs no further MFMA; a step whose blocks
// are all out loads and stages no further operand.
//
// The default path splits that work in two.  k_filter16 computes only the
// first kPartialDims dimensions, with each wave's query block held in
// registers for the whole work item and the candidates streamed through LDS,
// tests every block and hands the live ones on in a list (its partial dot
// product is the high-half one with either product count, so its "out" rule
// takes the high-half band coefficient); then
// k_refine_g16_blocks takes one wave per handed-on 32 x 32 block, operand
// fragments read straight from the prepared arrays (the slab layout is the
// MFMA operand layout: lane l takes row or candidate l % 32, half l / 32 of a
// slab), all slabs summed in one accumulator, classified like the tiles of
// k_refine_g16; its bits are ORed into the mask words (which k_refine_g16
// stored with that half-word zero), with the unit flags and row counts.
#include "refine_mfma_common.h"

#include <climits>
#include <type_traits>

namespace ersj {

namespace {

constexpr int kRowsG = 128;                         // query rows per work item
constexpr int kStepG = 256;                         // candidates per step
constexpr int kGroupStepsG = kGroupCands / kStepG;  // steps per 512-candidate word group
constexpr int kMaxStepsG = 8192 / kStepG;

struct G16 {
    static constexpr size_t A = 0;                                        // [2][4][kRowsG] x 16 B
    static constexpr size_t B = A + (size_t)2 * 4 * kRowsG * 16;           // [2][4][kStepG] x 16 B
    static constexpr size_t XI = B + (size_t)2 * 4 * kStepG * 16;          // [2][kStepG] u32
    static constexpr size_t NX = XI + (size_t)2 * kStepG * 4;              // [2][kStepG] f32
    static constexpr size_t QIN = NX + (size_t)2 * kStepG * 4;             // [kRowsG] f32
    static constexpr size_t QOUT = QIN + (size_t)kRowsG * 4;
    static constexpr size_t RCNT = QOUT + (size_t)kRowsG * 4;             // [kRowsG] u32
    static constexpr size_t PREF = RCNT + (size_t)kRowsG * 4;             // [kMaxRanges + 1] u32
    static constexpr size_t START = PREF + (size_t)(kMaxRanges + 1) * 4;  // [kMaxRanges] u32
    static constexpr size_t QOUTP = START + (size_t)kMaxRanges * 4;          // [kRowsG] f32
    static constexpr size_t NXP = QOUTP + (size_t)kRowsG * 4;               // [2][kStepG] f32
    static constexpr size_t ALIVE = NXP + (size_t)2 * kStepG * 4;           // [4] u32
    static constexpr size_t WORDS = (ALIVE + 16 + 63) & ~(size_t)63;        // [2][kRowsG][8] u64
    static constexpr size_t BYTES = WORDS + (size_t)2 * kRowsG * 8 * 8;
};

// Operands of one point set: centred, scaled, split, in slab-major parts
// (part 0: high halves of a slab's dimensions 0-7, 1: high 8-15, 2 and 3:
// the low halves), and the norms.  High parts only (hh): parts 0 and 1 of
// each slab, an odd slab count padded with one zero slab.
__global__ __launch_bounds__(256) void k_prep16(const float4 *__restrict__ xs, uint64_t n, int nb, int ns,
                                                const float4 *__restrict__ nrs, float s, bool hh,
                                                uint4 *__restrict__ P, uint64_t ps, float *__restrict__ N,
                                                float *__restrict__ NP)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float nrm = 0.f;
    for (int sl = 0; sl < ns; ++sl) {
        half8 h0, h1, l0, l1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = sl * 4 + j;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (b < nb) {
                const float4 x = xs[(uint64_t)b * n + i];
                const float4 r = nrs[b];
                v = make_float4(fmaf(x.x, s, r.x), fmaf(x.y, s, r.y), fmaf(x.z, s, r.z), fmaf(x.w, s, r.w));
            }
            nrm = fmaf(v.x, v.x, nrm);
            nrm = fmaf(v.y, v.y, nrm);
            nrm = fmaf(v.z, v.z, nrm);
            nrm = fmaf(v.w, v.w, nrm);
            half4 hh, ll;
            split16(v, hh, ll);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (j < 2) {
                    h0[(j & 1) * 4 + k] = hh[k];
                    l0[(j & 1) * 4 + k] = ll[k];
                } else {
                    h1[(j & 1) * 4 + k] = hh[k];
                    l1[(j & 1) * 4 + k] = ll[k];
                }
            }
        }
        if (sl * 16 + 16 == kPartialDims) NP[i] = nrm;
        if (hh) {
            P[((uint64_t)sl * 2 + 0) * ps + i] = *(const uint4 *)&h0;
            P[((uint64_t)sl * 2 + 1) * ps + i] = *(const uint4 *)&h1;
        } else {
            P[((uint64_t)sl * 4 + 0) * ps + i] = *(const uint4 *)&h0;
            P[((uint64_t)sl * 4 + 1) * ps + i] = *(const uint4 *)&h1;
            P[((uint64_t)sl * 4 + 2) * ps + i] = *(const uint4 *)&l0;
            P[((uint64_t)sl * 4 + 3) * ps + i] = *(const uint4 *)&l1;
        }
    }
    if (hh && (ns & 1)) {
        P[((uint64_t)ns * 2 + 0) * ps + i] = make_uint4(0u, 0u, 0u, 0u);
        P[((uint64_t)ns * 2 + 1) * ps + i] = make_uint4(0u, 0u, 0u, 0u);
    }
    N[i] = nrm;
}

// HH: a stage's four parts are the high halves of two slabs (parts 0, 1 of
// slab 2j and of slab 2j + 1); otherwise the four parts of one slab.
template <bool HH>
__global__ __launch_bounds__(256, 2) void k_refine_g16(RefineArgs a)
{
    using G = G16;
    uint32_t rk, colx;
    work_item(blockIdx.x, a.ntiles, a.nseg, &rk, &colx);
    const uint32_t seg = colx;
    const uint32_t t = a.order[a.ord0 + rk];
    const Tile tl = a.tiles[t];
    const uint32_t A = tl.cell;
    const uint32_t nr = a.nrng[A];
    const uint32_t *pref_g = a.rpref + (uint64_t)A * (kMaxRanges + 1);
    const uint32_t U = pref_g[nr];
    const uint32_t c_begin = seg * a.seg_len;
    if (c_begin >= U) return;
    const uint32_t c_end = min(U, c_begin + a.seg_len);
    const uint32_t nrows = min((uint32_t)kRowsG, tl.nrows);
    const uint32_t row0 = tl.row0;
    const int ns = HH ? ((a.nb + 3) / 4 + 1) / 2 : (a.nb + 3) / 4;  // stages per step
    // the stage that ends with dimension kPartialDims - 1 (nb > 16: a later
    // stage always follows)
    constexpr uint32_t chk = HH ? kPartialDims / 32 - 1 : kPartialDims / 16 - 1;

    extern __shared__ __align__(16) unsigned char smemg[];
    uint4 *const LA = (uint4 *)(smemg + G::A);
    uint4 *const LB = (uint4 *)(smemg + G::B);
    uint32_t *const LXI = (uint32_t *)(smemg + G::XI);
    float *const LNX = (float *)(smemg + G::NX);
    float *const LQIN = (float *)(smemg + G::QIN);
    float *const LQOUT = (float *)(smemg + G::QOUT);
    float *const LQOUTP = (float *)(smemg + G::QOUTP);
    float *const LNXP = (float *)(smemg + G::NXP);
    uint32_t *const LALIVE = (uint32_t *)(smemg + G::ALIVE);
    uint32_t *const LRCNT = (uint32_t *)(smemg + G::RCNT);
    uint32_t *const LPREF = (uint32_t *)(smemg + G::PREF);
    uint32_t *const LSTART = (uint32_t *)(smemg + G::START);
    uint64_t *const LWORDS = (uint64_t *)(smemg + G::WORDS);

    const int tid = threadIdx.x;
    const uint64_t n = a.ps, nqr = a.psq;  // part strides of the prepared arrays
    const uint4 *__restrict__ P = a.p16;
    const uint4 *__restrict__ PQ = a.p16q;
    const float *__restrict__ NP = a.n16;
    uint64_t *__restrict__ mask = a.mask;
    const uint32_t W = tl.words;
    const uint64_t mbase = a.toff[t] - a.wbase;

    if (tid <= kMaxRanges) LPREF[tid] = tid <= (int)nr ? pref_g[tid] : 0xffffffffu;
    if (tid < kMaxRanges) LSTART[tid] = a.rstart[(uint64_t)A * kMaxRanges + tid];
    if (tid < kRowsG) {
        const bool valid = (uint32_t)tid < nrows;
        const float nq = valid ? a.n16q[row0 + tid] : 0.f;
        LQIN[tid] = valid ? a.tlo - a.kp * nq - a.tabs : -INFINITY;
        LQOUT[tid] = valid ? a.thi - a.km * nq + a.tabs : -INFINITY;
        const float nqp = valid ? a.np16q[row0 + tid] : 0.f;
        LQOUTP[tid] = valid ? a.thi - a.km * nqp + a.tabs : -INFINITY;
        LRCNT[tid] = 0;
    }
    for (int e = tid; e < 2 * kRowsG * 8; e += 256) LWORDS[e] = 0ull;
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31, hi = lane >> 5;
    const int rh = wave & 1, cg = wave >> 1;
    const bool do0 = (uint32_t)(rh * 64) < nrows, do1 = (uint32_t)(rh * 64 + 32) < nrows;
    const uint32_t nsteps = (c_end - c_begin + kStepG - 1) / kStepG;  // <= kMaxStepsG
    const BandSink bsink{band_list(a.blist, a.lcap), band_counter(a.bcount), a.lcap, row0, mbase, W};

    // loader: lane l of wave w copies part w of query rows l and 64 + l, and
    // all four parts of candidate 64 w + l of the step
    const uint32_t qa = row0 + min((uint32_t)lane, nrows - 1), qb2 = row0 + min((uint32_t)(64 + lane), nrows - 1);
    uint32_t g_u = 0;
    const uint32_t idx0 = [&]() {
        const int g = range_of(LPREF, nr, c_begin);
        return LSTART[g] + (c_begin - LPREF[g]);
    }();
    auto cand_index = [&](uint32_t st) __attribute__((always_inline)) -> uint32_t {
        const uint32_t P0 = c_begin + st * kStepG;
        while (P0 >= (uint32_t)__builtin_amdgcn_readfirstlane(LPREF[g_u + 1])) ++g_u;
        const uint32_t p = P0 + (uint32_t)(wave * 64 + lane);
        if (p >= c_end) return idx0;
        uint32_t g = g_u;
        const uint32_t nxt = __builtin_amdgcn_readfirstlane(LPREF[g_u + 1]);
        if (P0 + kStepG > nxt) {
            while (p >= LPREF[g + 1]) ++g;
        }
        return LSTART[g] - LPREF[g] + p;
    };
    // the next stage's operands in flight (named registers: an array here
    // ends up in scratch memory)
    uint4 ra0, ra1, rb0, rb1, rb2, rb3;
    uint32_t ci = idx0;
    float cn = 0.f, cnp = 0.f;
    auto issue = [&](uint32_t st, uint32_t sl) __attribute__((always_inline)) {
        if (sl == 0) {
            ci = cand_index(st);
            cn = NP[ci];
            cnp = a.np16[ci];
        }
        ra0 = PQ[((uint64_t)sl * 4 + wave) * nqr + qa];
        ra1 = PQ[((uint64_t)sl * 4 + wave) * nqr + qb2];
        const uint4 *pc = P + (uint64_t)sl * 4 * n + ci;
        rb0 = pc[0];
        rb1 = pc[n];
        rb2 = pc[2 * n];
        rb3 = pc[3 * n];
    };
    auto deposit = [&](uint32_t u, uint32_t st, uint32_t sl) __attribute__((always_inline)) {
        const int buf = (int)(u & 1);
        uint4 *la = LA + (size_t)buf * 4 * kRowsG;
        uint4 *lb = LB + (size_t)buf * 4 * kStepG;
        la[wave * kRowsG + lane] = ra0;
        la[wave * kRowsG + 64 + lane] = ra1;
        lb[0 * kStepG + wave * 64 + lane] = rb0;
        lb[1 * kStepG + wave * 64 + lane] = rb1;
        lb[2 * kStepG + wave * 64 + lane] = rb2;
        lb[3 * kStepG + wave * 64 + lane] = rb3;
        if (sl == 0) {
            LXI[(st & 1) * kStepG + wave * 64 + lane] = ci;
            LNX[(st & 1) * kStepG + wave * 64 + lane] = cn;
            LNXP[(st & 1) * kStepG + wave * 64 + lane] = cnp;
        }
    };

    // accumulators start at zero and are cleared after each step's
    // classification (a select per stage would cost a vector instruction per
    // accumulator register)
    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[i][tt] = floatx16{};
    // blocks (bit 4 i + tt: rows rh 64 + 32 i, candidates cg 128 + 32 tt of
    // the step) not yet settled by the partial test (wave-uniform)
    uint32_t alive = 0xffu;
    bool step_dead = false;  // every block of the workgroup settled (uniform)
    unsigned long long npart = 0;  // comparisons settled by the partial test
    auto mma = [&](int buf) __attribute__((always_inline)) {
        const uint4 *la = LA + (size_t)buf * 4 * kRowsG;
        const uint4 *lb = LB + (size_t)buf * 4 * kStepG;
        half8 ah[2], al[2], bh[4], bl[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = rh * 64 + i * 32 + col;
            ah[i] = *(const half8 *)&la[hi * kRowsG + r];
            al[i] = *(const half8 *)&la[(2 + hi) * kRowsG + r];
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int c = cg * 128 + tt * 32 + col;
            bh[tt] = *(const half8 *)&lb[hi * kStepG + c];
            bl[tt] = *(const half8 *)&lb[(2 + hi) * kStepG + c];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (!(i == 0 ? do0 : do1)) continue;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                if ((alive >> (i * 4 + tt)) & 1u) acc[i][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bh[tt], acc[i][tt], 0, 0, 0);
        }
        if (HH) {
            // second slab of the stage: its high halves sit where the
            // three-product form keeps the low ones
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (!(i == 0 ? do0 : do1)) continue;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    if ((alive >> (i * 4 + tt)) & 1u) acc[i][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bl[tt], acc[i][tt], 0, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (!(i == 0 ? do0 : do1)) continue;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                if ((alive >> (i * 4 + tt)) & 1u) acc[i][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bl[tt], acc[i][tt], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (!(i == 0 ? do0 : do1)) continue;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                if ((alive >> (i * 4 + tt)) & 1u) acc[i][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bh[tt], acc[i][tt], 0, 0, 0);
        }
    };

    // partial test of the wave's live blocks; out-rule of classify_block
    // with the norms over the first kPartialDims dimensions
    auto partial_check = [&](uint32_t st) __attribute__((always_inline)) {
        uint32_t nal = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int cl = cg * 128 + tt * 32 + col;
            const uint32_t c0 = c_begin + st * kStepG + cg * 128 + tt * 32;
            const float xo = c0 + col < c_end ? a.km * LNXP[(st & 1) * kStepG + cl] : __builtin_nanf("");
            const uint32_t ncol = c0 < c_end ? min(32u, c_end - c0) : 0u;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (!((alive >> (i * 4 + tt)) & 1u)) continue;
                const int qb = rh * 2 + i;
                const float4 *qo4 = (const float4 *)LQOUTP + qb * 8 + hi;
                // one ballot per register, OR-ed as wave masks
                uint64_t nout = 0;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 qo = qo4[g * 2];
                    nout |= __ballot(fmaf(-2.0f, acc[i][tt][4 * g + 0], xo) <= qo.x);
                    nout |= __ballot(fmaf(-2.0f, acc[i][tt][4 * g + 1], xo) <= qo.y);
                    nout |= __ballot(fmaf(-2.0f, acc[i][tt][4 * g + 2], xo) <= qo.z);
                    nout |= __ballot(fmaf(-2.0f, acc[i][tt][4 * g + 3], xo) <= qo.w);
                }
                if (nout != 0) {
                    nal |= 1u << (i * 4 + tt);
                } else {
                    const uint32_t r0 = (uint32_t)(rh * 64 + i * 32);
                    const uint32_t nrow = r0 < nrows ? min(32u, nrows - r0) : 0u;
                    npart += (unsigned long long)nrow * ncol;
                }
            }
        }
        alive = nal;
    };

    int wsel = 0;  // group buffer of the current 512-candidate group (toggles at each flush)
    auto classify = [&](uint32_t st) __attribute__((always_inline)) {
        uint64_t *wg = LWORDS + (size_t)wsel * kRowsG * 8;
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
            const uint32_t cw = c_begin + st * kStepG + cg * 128 + w2 * 64;
            float xin[2], xout[2];
            uint32_t xid[2];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const int cl = cg * 128 + w2 * 64 + t2 * 32 + col;
                const float nx = LNX[(st & 1) * kStepG + cl];
                xid[t2] = LXI[(st & 1) * kStepG + cl];
                const bool valid = cw + 32 * t2 + col < c_end;
                xin[t2] = valid ? a.kp * nx : __builtin_nanf("");
                xout[t2] = valid ? a.km * nx : __builtin_nanf("");
            }
            const int wi = (int)(st % kGroupStepsG) * 4 + cg * 2 + w2;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (!(i == 0 ? do0 : do1)) continue;
                const int qb = rh * 2 + i;
                const uint32_t live = (alive >> (i * 4 + w2 * 2)) & 3u;
                if (live == 0) continue;
                classify_block(&acc[i][w2 * 2], xin, xout, LQIN, LQOUT, qb, lane, cw, live, bsink,
                               [&](int t2) { return xid[t2]; }, wg + (qb * 32 + col) * 8 + wi);
            }
        }
    };
    auto unit_flag = [&](int row, int j, uint32_t w, bool ok, bool nz) __attribute__((always_inline)) {
        const uint64_t b = __ballot(nz);
        if (ok && (j & 3) == 0) a.gflag[(mbase + (uint64_t)row * W + w) >> 2] = ((b >> (lane & ~3)) & 0xfull) ? 1 : 0;
    };
    auto flush = [&](uint32_t grp) __attribute__((always_inline)) {
        uint64_t *sw = LWORDS + (size_t)wsel * kRowsG * 8;
        for (int e = tid; e < kRowsG * 8; e += 256) {
            const int row = e >> 3, j = e & 7;
            const uint32_t c0 = c_begin + grp * kGroupCands + 64 * j;
            const uint32_t w = c0 >> 6;
            const bool ok = (uint32_t)row < nrows && w < W && c0 < c_end;
            const uint64_t v = sw[e];
            if (ok) {
                mask[mbase + (uint64_t)row * W + w] = v;
                const uint32_t pc = __popcll(v);
                if (pc != 0) atomicAdd(&LRCNT[row], pc);
            }
            unit_flag(row, j, w, ok, ok && v != 0);
            sw[e] = 0ull;
        }
    };

    if (nsteps > 0) {
        issue(0, 0);
        deposit(0, 0, 0);
    }
    __syncthreads();
    // stage (st, sl), it-th in order (LDS buffer it & 1)
    uint32_t st = 0, sl = 0, it = 0;
    while (st < nsteps) {
        const bool last_sl = sl + 1 == (uint32_t)ns;
        const uint32_t nst = last_sl ? st + 1 : st, nsl = last_sl ? 0 : sl + 1;
        // a settled step's later stages are neither loaded nor staged
        const bool more = nst < nsteps && !(step_dead && nst == st);
        if (more) issue(nst, nsl);
        if ((do0 || do1) && alive != 0) mma((int)(it & 1));
        if (sl == chk) {
            if (do0 || do1) partial_check(st);
            else alive = 0;
            if (lane == 0) LALIVE[wave] = alive;
        }
        if (last_sl) {
            if ((do0 || do1) && alive != 0) classify(st);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) acc[i][tt] = floatx16{};
        }
        if (more) deposit(it + 1, nst, nsl);
        __syncthreads();
        if (sl == chk) step_dead = (LALIVE[0] | LALIVE[1] | LALIVE[2] | LALIVE[3]) == 0u;
        if (last_sl) {
            alive = 0xffu;
            step_dead = false;
            if (st % kGroupStepsG == kGroupStepsG - 1 || st + 1 == nsteps) {
                flush(st / kGroupStepsG);
                wsel ^= 1;
            }
        }
        st = nst;
        sl = nsl;
        ++it;
    }
    if (lane == 0 && npart != 0)
        atomicAdd(&a.partial[(uint64_t)(blockIdx.x % kHitSlots) * kBandStride], npart);
    __syncthreads();
    for (int i = tid; i < (int)nrows; i += 256)
        if (LRCNT[i] != 0) atomicAdd(&a.rowcnt[row0 + i - a.row_base], LRCNT[i]);
}

// The filter's "out" rule, rearranged so that the MFMAs add each row's term.
// The classification's rule for a pair is out iff fl(xo - 2 s) > qo (s the
// accumulated dot product, xo = fl(km Nx), qo the row threshold); its proof
// starts from xo - 2 s* > qo - 2 E_s, s* the exact sum of the products and
// E_s the accumulation error the band charges.  Here the accumulator starts
// at c = filter_row_start(qo) >= qo / 2 + 2^-16 |qo / 2| (rounded up) and a
// pair is out iff acc < filter_col_bound(xo) <= xo / 2.  A start value adds
// at most 32.1u |c| to each instruction's error (the accumulation bound:
// 17 faithfully rounded terms, the accumulator one of them), 128.4u |c| over
// the four instructions of 64 dimensions, less than the slack: acc < xo / 2
// gives s* + qo / 2 < xo / 2 + E_s, the proof's premise.  An invalid row
// starts at -inf and an invalid column compares with NaN: out either way.
__device__ __forceinline__ float filter_row_start(float qo)
{
    if (!(qo > -INFINITY)) return -INFINITY;
    const double h = 0.5 * (double)qo;
    return __double2float_ru(h + fabs(h) * 0x1p-16 + 0x1p-140);
}

// xo / 2, exact for xo >= 2^-125; 0 (below it) under 2^-120
__device__ __forceinline__ float filter_col_bound(float xo) { return xo >= 0x1p-120f ? xo * 0.5f : 0.0f; }

// Filter over the first kPartialDims dimensions: work item as k_refine_g16;
// wave w holds query block w (rows 32 w .. 32 w + 31 of the tile) in
// registers, the high halves of its first kPartialDims dimensions, and the
// item's candidates pass through LDS kStepF at a time (one barrier a step).
// Each 32 x 32 block gets the partial test; a live block goes to the
// hand-on list, a settled one keeps zero bits.  The unit flags of the
// batch are cleared before the launch; a step with a live block zeroes the
// 4-word mask unit it covers in the block's rows, the only units whose
// words the block kernel, the re-check and the compaction touch.
//
// Operands go from global memory straight into LDS (16 bytes a lane, lane l
// at the wave's base + 16 l): while a step's MFMAs read one buffer, the next
// step's operands and column bounds arrive in the other.  Two buffers in
// separate LDS arrays, the steps in pairs, so that every access names its
// buffer and the only wait for the loads is the one before the barrier.
constexpr int kStepF = 128;
constexpr int kSlabsF = kPartialDims / 16;

// xb[i] = filter_col_bound(kmf NP[i]) for the n points, xb[n] = NaN (the
// bound of a position past a work item's end: never live)
__global__ __launch_bounds__(256) void k_col_bounds16(const float *__restrict__ NP, uint64_t n, float kmf,
                                                      float *__restrict__ xb)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) xb[i] = filter_col_bound(kmf * NP[i]);
    else if (i == n) xb[i] = __builtin_nanf("");
}

// Integer form of the partial test.  Over the first kPartialDims dimensions
// of the layout, d_i = x_i - r_i (r: the layout's means as fp32, the same
// for both point sets) rounds to q_i = rint(S d_i), S = 127 / M with M at
// least every |d_i| of both sets, so |q_i| <= 127 and d_i = q_i / S + e_i
// with |e_i| <= D = (1/2 + 2^-30) / S (the fp64 product S d_i is within
// 2^-46 of exact).  For two points, with N the exact squared norm of d and
// A = sum |q_i| of each,
//   |dq - dx|^2 = Nq + Nx - 2 dq.dx
//              >= Nq + Nx - 2 sum qq_i qx_i / S^2 - 2 D (Aq + Ax) / S - 128 D^2,
// since dq.dx = sum (qq_i / S + eq_i)(qx_i / S + ex_i).  The pair's squared
// distance exceeds E (and it is no neighbour) when, with T = S^2 / 2,
//   sum qq_i qx_i < T (Nq - 2 D Aq / S - 64 D^2 - E) + T (Nx - 2 D Ax / S - 64 D^2).
// The row term, evaluated in fp64, lowered by a relative 2^-40 of its
// magnitude and 2, and rounded down, is negated into the int32 accumulator's
// start (qs8); the column term, lowered the same way and rounded down, is
// the bound (xb8).  The int8 MFMA's sum is exact, so a block whose every
// accumulator stays below its column's bound is settled.  Ranges: the
// column term lies in [-4160, T 64 M^2 = 516128]; a row start above 2^30
// (a huge E) is clamped to 2^30, live against every bound; sums stay within
// 64 * 127^2 of the start, far from int32 overflow.

// bits of max |x_i - r_i| over the first kPartialDims dimensions of the
// rows (fp32 difference, within 2^-24 of exact), atomically maxed into *mx
__global__ __launch_bounds__(256) void k_maxabs8(const float4 *__restrict__ xs, uint64_t n,
                                                 const float4 *__restrict__ ref, unsigned int *__restrict__ mx)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float m = 0.f;
    if (i < n) {
#pragma unroll 4
        for (int b = 0; b < kPartialDims / 4; ++b) {
            const float4 x = xs[(uint64_t)b * n + i], r = ref[b];
            m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x - r.x), fabsf(x.y - r.y)), fmaxf(fabsf(x.z - r.z), fabsf(x.w - r.w))));
        }
    }
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0 && m > 0.f) atomicMax(mx, __float_as_uint(m));
}

// int8 operands of one point set: part p (dimensions 16 p .. 16 p + 15, slab
// p / 2 of 32, half p % 2) of row i at P[p * ps + i], one byte a dimension;
// the row start (rows) and the column bound (cols, with bound[n] = INT_MAX
// past the end) as derived above
__global__ __launch_bounds__(256) void k_prep8(const float4 *__restrict__ xs, uint64_t n,
                                               const float4 *__restrict__ ref, double S, double E,
                                               uint4 *__restrict__ P, uint64_t ps, int *__restrict__ start,
                                               int *__restrict__ bound)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) {
        if (i == n && bound) bound[n] = INT_MAX;
        return;
    }
    double N = 0.0, A = 0.0;
#pragma unroll 1
    for (int p = 0; p < kPartialDims / 16; ++p) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 x = xs[(uint64_t)(4 * p + j) * n + i], r = ref[4 * p + j];
            const double dv[4] = {(double)x.x - (double)r.x, (double)x.y - (double)r.y, (double)x.z - (double)r.z,
                                  (double)x.w - (double)r.w};
            uint32_t word = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                N = fma(dv[c], dv[c], N);
                const double qv = fmin(fmax(rint(dv[c] * S), -127.0), 127.0);
                A += fabs(qv);
                word |= ((uint32_t)(int)qv & 0xffu) << (8 * c);
            }
            w[j] = word;
        }
        P[(uint64_t)p * ps + i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const double D = (0.5 + 0x1p-30) / S, T = 0.5 * S * S;
    const double base = N - 2.0 * D * A / S - 64.0 * D * D;
    const double mag = N + 2.0 * D * A / S + 64.0 * D * D;  // bounds the terms' rounding
    if (bound) bound[i] = (int)fmin(floor(T * base - T * mag * 0x1p-40 - 2.0), 0x1p29);
    if (start) {
        const double v = T * (base - E) - T * (mag + E) * 0x1p-40 - 2.0;
        start[i] = v > -0x1p30 ? -(int)floor(v) : (1 << 30);  // (NaN from E = inf: 2^30)
    }
}

typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));

// PP: parts per slab of the prepared arrays (2: high halves only, 4: high
// and low); the fp16 form reads the high ones.  I8: the integer form of the
// same test (k_prep8's operands, row starts and column bounds; two int8
// MFMAs of 32 dimensions per block, exact int32 sums).
template <int PP, bool I8>
__global__ __launch_bounds__(256, 4) void k_filter16(RefineArgs a)
{
    using Acc = std::conditional_t<I8, intx16, floatx16>;
    // parts of a candidate in LDS: fp16 high halves of 4 slabs of 16
    // dimensions, or int8 values of 2 slabs of 32, two parts a slab
    constexpr int kParts = I8 ? 4 : 2 * kSlabsF;
    constexpr int kSl = kParts / 2;
    uint32_t rk, seg;
    work_item(blockIdx.x, a.ntiles, a.nseg, &rk, &seg);
    const uint32_t t = a.order[a.ord0 + rk];
    const Tile tl = a.tiles[t];
    const uint32_t A = tl.cell, nr = a.nrng[A];
    const uint32_t *pref_g = a.rpref + (uint64_t)A * (kMaxRanges + 1);
    const uint32_t U = pref_g[nr];
    const uint32_t c_begin = seg * a.seg_len;
    if (c_begin >= U) return;
    const uint32_t c_end = min(U, c_begin + a.seg_len);
    const uint32_t nrows = min((uint32_t)kRowsG, tl.nrows), row0 = tl.row0;

    // operand buffers: part p (= 2 slab + half) of candidate c at [p][c];
    // column bounds at [copy][c] (waves 0-1 and 2-3 each load a copy)
    __shared__ __align__(16) uint4 LB0[kParts * kStepF], LB1[kParts * kStepF];
    __shared__ __align__(16) float LX0[2 * kStepF], LX1[2 * kStepF];  // int bounds in the int8 form
    __shared__ __align__(16) float LQOUTP[kRowsG];                     // int starts in the int8 form
    __shared__ uint32_t LPREF[kMaxRanges + 1], LSTART[kMaxRanges];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, col = lane & 31, hi = lane >> 5;
    const uint64_t ps = a.ps, psq = a.psq;  // part strides of the prepared arrays
    if (tid <= kMaxRanges) LPREF[tid] = tid <= (int)nr ? pref_g[tid] : 0xffffffffu;
    if (tid < kMaxRanges) LSTART[tid] = a.rstart[(uint64_t)A * kMaxRanges + tid];
    if (tid < kRowsG) {
        const bool valid = (uint32_t)tid < nrows;
        if constexpr (I8) {
            // an invalid row starts far below every bound (-2^30 + 2^20 < -4160)
            LQOUTP[tid] = __builtin_bit_cast(float, valid ? a.qs8[row0 + tid] : -(1 << 30));
        } else {
            const float nqp = valid ? a.np16q[row0 + tid] : 0.f;
            LQOUTP[tid] = valid ? filter_row_start(a.thi - a.kmf * nqp + a.tabs) : -INFINITY;
        }
    }
    // the wave's query fragments: row 32 wave + l % 32, half l / 32 of each slab
    const uint32_t nrow_w = (uint32_t)(wave * 32) < nrows ? min(32u, nrows - (uint32_t)(wave * 32)) : 0u;
    const uint32_t q = row0 + min((uint32_t)(wave * 32 + col), nrows - 1);
    using Frag = std::conditional_t<I8, intx4, half8>;
    Frag af[kSl];
#pragma unroll
    for (int s = 0; s < kSl; ++s) {
        const uint4 v = I8 ? a.p8q[((uint64_t)s * 2 + hi) * a.ps8q + q] : a.p16q[((uint64_t)s * PP + hi) * psq + q];
        af[s] = __builtin_bit_cast(Frag, v);
    }
    const uint64_t mbase = a.toff[t] - a.wbase;
    const uint32_t W = tl.words;
    const uint32_t nsteps = (c_end - c_begin + kStepF - 1) / kStepF;
    __syncthreads();

    // loader: lane l of wave w stages candidate lc = 64 (w % 2) + l of the
    // step, parts kSl (w / 2) .. + kSl - 1
    const uint32_t lc = (uint32_t)tid & (kStepF - 1), lp0 = ((uint32_t)wave >> 1) * kSl;
    const uint32_t lbase = (uint32_t)(wave & 1) * 64;  // the wave's first candidate
    // the range of the candidate list holding the step's first position,
    // kept in scalar registers: [r_lo, r_hi) of the list are points r_st ..
    uint32_t g_u = (uint32_t)__builtin_amdgcn_readfirstlane(range_of(LPREF, nr, c_begin));
    uint32_t r_lo = __builtin_amdgcn_readfirstlane(LPREF[g_u]), r_hi = __builtin_amdgcn_readfirstlane(LPREF[g_u + 1]);
    uint32_t r_st = __builtin_amdgcn_readfirstlane(LSTART[g_u]);
    const uint32_t idx0 = r_st + (c_begin - r_lo);
    auto cand_index = [&](uint32_t st) __attribute__((always_inline)) -> uint32_t {
        const uint32_t P0 = c_begin + st * kStepF;
        while (P0 >= r_hi) {
            ++g_u;
            r_lo = r_hi;
            r_hi = __builtin_amdgcn_readfirstlane(LPREF[g_u + 1]);
            r_st = __builtin_amdgcn_readfirstlane(LSTART[g_u]);
        }
        const uint32_t p = P0 + lc;
        uint32_t ci = r_st - r_lo + p;
        if (P0 + kStepF > r_hi) {
            // a step across the end of a range (rare): each lane finds its own
            uint32_t g = g_u;
            while (p >= LPREF[g + 1]) ++g;
            ci = LSTART[g] - LPREF[g] + p;
        }
        return p < c_end ? ci : idx0;
    };
    // step st's operands and column bounds into buffer lb / lx: five loads
    // a lane on every call (a step past the end repeats the last step's
    // candidates, with NaN bounds, into a buffer nobody reads)
    auto issue = [&](uint32_t st, uint4 *lb, float *lx) __attribute__((always_inline)) {
        const uint32_t ci = cand_index(st < nsteps ? st : nsteps - 1);
        const uint32_t cx = c_begin + st * kStepF + lc < c_end ? ci : (uint32_t)a.n;
        const uint4 *pc = (I8 ? a.p8 : a.p16) + ci;
#pragma unroll
        for (int k = 0; k < kSl; ++k) {
            const uint32_t p = lp0 + (uint32_t)k;
            const uint64_t off = I8 ? (uint64_t)p * a.ps8 : ((uint64_t)(p >> 1) * PP + (p & 1)) * ps;
            __builtin_amdgcn_global_load_lds((const void *)(pc + off),
                                             (__attribute__((address_space(3))) void *)(lb + p * kStepF + lbase),
                                             16, 0, 0);
        }
        const void *xsrc = I8 ? (const void *)(a.xb8 + cx) : (const void *)(a.xb16 + cx);
        __builtin_amdgcn_global_load_lds(xsrc, (__attribute__((address_space(3))) void *)(lx + (wave >> 1) * kStepF + lbase),
                                         4, 0, 0);
    };
    unsigned long long npart = 0;
    uint4 *const dl = a.dlist + (uint64_t)(blockIdx.x % kBandLists) * a.dcap;
    unsigned long long *const dc = &a.dcount[(uint64_t)(blockIdx.x % kBandLists) * kBandStride];

    if (nsteps == 0) return;
    issue(0, LB0, LX0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the accumulators' start: register v of lane l holds row 8 (v / 4) +
    // v % 4 + 4 (l / 32) of the wave's block
    Acc crow;
    {
        const float4 *c4 = (const float4 *)LQOUTP + wave * 8 + hi;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 c = c4[g * 2];
            if constexpr (I8) {
                crow[4 * g + 0] = __builtin_bit_cast(int, c.x);
                crow[4 * g + 1] = __builtin_bit_cast(int, c.y);
                crow[4 * g + 2] = __builtin_bit_cast(int, c.z);
                crow[4 * g + 3] = __builtin_bit_cast(int, c.w);
            } else {
                crow[4 * g + 0] = c.x;
                crow[4 * g + 1] = c.y;
                crow[4 * g + 2] = c.z;
                crow[4 * g + 3] = c.w;
            }
        }
    }
    // step st reads (lb, lx) while step st + 1's operands load into (nb, nx)
    auto step = [&](uint32_t st, const uint4 *lb, const float *lx, uint4 *nb, float *nx)
                    __attribute__((always_inline)) {
        issue(st + 1, nb, nx);
        if (nrow_w != 0) {
            Acc acc[4];
#pragma unroll
            for (int s = 0; s < kSl; ++s) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const Frag bf = *(const Frag *)&lb[(s * 2 + hi) * kStepF + tt * 32 + col];
                    if constexpr (I8)
                        acc[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s], bf, s == 0 ? crow : acc[tt], 0, 0, 0);
                    else
                        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s], bf, s == 0 ? crow : acc[tt], 0, 0, 0);
                }
            }
            // partial test of the wave's four blocks: a lane's 16 registers
            // share its column, so the block is live iff some lane's largest
            // register reaches the lane's column bound
            bool hits[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const Acc v = acc[tt];
                bool &hit = hits[tt];
                if constexpr (I8) {
                    const int xb = __builtin_bit_cast(int, lx[tt * 32 + col]);
                    const int m0 = max(max(v[0], v[1]), v[2]), m1 = max(max(v[3], v[4]), v[5]);
                    const int m2 = max(max(v[6], v[7]), v[8]), m3 = max(max(v[9], v[10]), v[11]);
                    const int m4 = max(max(v[12], v[13]), v[14]);
                    hit = max(max(max(m0, m1), m2), max(max(m3, m4), v[15])) >= xb;
                } else {
                    const float xb = lx[tt * 32 + col];
                    const float m0 = fmaxf(fmaxf(v[0], v[1]), v[2]), m1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
                    const float m2 = fmaxf(fmaxf(v[6], v[7]), v[8]), m3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
                    const float m4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
                    hit = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), v[15])) >= xb;
                }
            }
            // one ballot settles the common step with no live block
            uint32_t live = 0;
            if (__ballot(hits[0] || hits[1] || hits[2] || hits[3]) != 0) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    if (__ballot(hits[tt]) != 0) live |= 1u << tt;
            }
            // comparisons settled here: the step's valid columns less those
            // of its live blocks
            {
                const uint32_t s0 = c_begin + st * kStepF;
                uint32_t cols = min((uint32_t)kStepF, c_end - s0);
                if (live != 0) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        if ((live >> tt) & 1u) cols -= min(32u, c_end - (s0 + tt * 32));
                }
                npart += (unsigned long long)nrow_w * cols;
            }
            if (live != 0) {
                // the step's two mask words lie in one 4-word unit of each
                // row (rows start on 8-word boundaries, steps on 2-word
                // ones, items on 512-candidate ones); a flagged unit is read
                // whole, so the unit is zeroed for the wave's rows (lane l:
                // row l % 32, bytes 16 (l / 32) .. + 15)
                {
                    const uint32_t r = (uint32_t)col;
                    if (r < nrow_w) {
                        const uint64_t wu = (mbase + (uint64_t)(wave * 32 + r) * W + ((c_begin + st * kStepF) >> 6)) & ~3ull;
                        ((uint4 *)(a.mask + wu))[hi] = make_uint4(0u, 0u, 0u, 0u);
                    }
                }
                // hand the live blocks on
                unsigned long long base = 0;
                if (lane == 0) base = atomicAdd(dc, (unsigned long long)__popc(live));
                base = __shfl(base, 0, 64);
                uint32_t j = 0;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    if (!((live >> tt) & 1u)) continue;
                    const uint32_t c0 = c_begin + st * kStepF + tt * 32;
                    if (lane == 0 && base + j < a.dcap) {
                        // the block's candidates are consecutive points when
                        // its valid positions lie in one range of the list
                        const int g = range_of(LPREF, nr, c0);
                        const bool one = min(c0 + 32u, U) <= LPREF[g + 1];
                        const uint32_t ci0 = one ? LSTART[g] - LPREF[g] + c0 : 0xffffffffu;
                        dl[base + j] = make_uint4(t, ((c0 >> 5) << 2) | (uint32_t)wave, ci0, min(32u, U - c0));
                    }
                    ++j;
                }
            }
        }
        // the next step's operands are in LDS, and every wave is done with
        // this step's buffer, before the next step starts
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    uint32_t st = 0;
    for (; st + 1 < nsteps; st += 2) {
        step(st, LB0, LX0, LB1, LX1);
        step(st + 1, LB1, LX1, LB0, LX0);
    }
    if (st < nsteps) step(st, LB0, LX0, LB1, LX1);
    if (lane == 0 && npart != 0)
        atomicAdd(&a.partial[(uint64_t)(blockIdx.x % kHitSlots) * kBandStride], npart);
}

// Sort keys of the handed-on blocks: entry e of the sub-lists taken in
// order (pref: exclusive prefix of their kept counts, kBandLists + 1
// entries) gets key = (the group of 2^kHandonGroupBits points holding its
// block's first candidate, gend when the candidates are not consecutive
// points) << qbits | (tile << 2 | query block), and value = its index in
// dlist.  In that order a group's candidate blocks (3 MB of operands at
// d = 384, within one XCD's L2) serve every query block live against them
// while that query block's entries are consecutive.
__global__ __launch_bounds__(256) void k_handon_keys(const uint4 *__restrict__ dl, uint64_t dcap,
                                                     const uint64_t *__restrict__ pref, uint64_t total, int qbits,
                                                     uint32_t gend, uint64_t *__restrict__ keys,
                                                     uint32_t *__restrict__ vals)
{
    const uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    uint32_t lo = 0, hi = kBandLists;  // largest sub-list k with pref[k] <= e
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (pref[mid] <= e) lo = mid;
        else hi = mid;
    }
    const uint64_t idx = (uint64_t)lo * dcap + (e - pref[lo]);
    const uint4 ent = dl[idx];
    const uint32_t grp = ent.z == 0xffffffffu ? gend : ent.z >> kHandonGroupBits;
    keys[e] = ((uint64_t)grp << qbits) | ((uint64_t)ent.x << 2 | (ent.y & 3u));
    vals[e] = (uint32_t)idx;
}

// The end of a handed-on block's refinement (k_refine_g16_blocks and
// k_refine_g16_runs): classification of its accumulated 32 x 32 block
// against the row thresholds this wave wrote to lqi / lqo (register v of
// lane l: row 8 (v / 4) + v % 4 + 4 (l / 32), column l % 32, the rules of
// classify_block), band pairs to the band list, bits ORed into the mask
// words with their unit flags and row counts.
__device__ __forceinline__ void g16_block_finish(const RefineArgs &a, const floatx16 &acc, uint32_t t,
                                                 const Tile &tl, uint32_t rb, uint32_t c0, uint32_t r, bool vr,
                                                 bool vc, uint32_t ci, float nx, const float *lqi,
                                                 const float *lqo)
{
    const int lane = threadIdx.x & 63, col = lane & 31, hi = lane >> 5;
    // the row thresholds written by this wave's lanes are read by all
    // of its lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // one 32 x 32 block: register v of lane l holds row 8 (v / 4) + v % 4
    // + 4 (l / 32), column l % 32 (the rules of classify_block)
    const float xin = vc ? a.kp * nx : __builtin_nanf(""), xout = vc ? a.km * nx : __builtin_nanf("");
    int wbits = 0;  // lane r < 32: the block's 32 bits of row r
    uint64_t band = 0;
    static_for(std::make_integer_sequence<int, 16>{}, [&](auto V) {
        constexpr int v = decltype(V)::value, i0 = 8 * (v / 4) + v % 4;
        const int row = i0 + 4 * hi;
        const float d2 = acc[v];
        const uint64_t bin = __ballot(fmaf(-2.0f, d2, xin) <= lqi[row]);
        const uint64_t bno = __ballot(fmaf(-2.0f, d2, xout) <= lqo[row]);
        band |= bno & ~bin;
        wbits = write_lane<i0>(wbits, (uint32_t)bin);
        wbits = write_lane<i0 + 4>(wbits, (uint32_t)(bin >> 32));
    });
    const uint64_t mbase = a.toff[t] - a.wbase;
    if (band != 0) {
        // rare: the band pairs, appended for the binary64 re-check
        Boundary *bl = band_list(a.blist, a.lcap);
        unsigned long long *bc = band_counter(a.bcount);
#pragma unroll 1
        for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v >> 2) + (v & 3) + 4 * hi;
            const float d2 = acc[v];
            const bool bd = !(fmaf(-2.0f, d2, xin) <= lqi[row]) && fmaf(-2.0f, d2, xout) <= lqo[row];
            const uint64_t bb = __ballot(bd);
            if (bb == 0) continue;
            const int first = __ffsll((unsigned long long)bb) - 1;
            unsigned long long base = 0;
            if (lane == first) base = atomicAdd(bc, (unsigned long long)__popcll(bb));
            base = __shfl(base, first, 64);
            if (bd) {
                const uint64_t below = lane == 0 ? 0ull : (bb & (~0ull >> (64 - lane)));
                const uint64_t idx = base + __popcll(below);
                if (idx < a.lcap) {
                    Boundary e;
                    e.q = tl.row0 + rb * 32 + (uint32_t)row;
                    e.x = ci;
                    e.bit = (mbase + (uint64_t)(rb * 32 + row) * tl.words) * 64 + c0 + (uint32_t)col;
                    bl[idx] = e;
                }
            }
        }
    }
    const uint64_t w = (uint64_t)(uint32_t)wbits << (c0 & 32u);
    if (lane < 32) {
        if (w != 0 && vr) {
            const uint64_t wi = mbase + (uint64_t)r * tl.words + (c0 >> 6);
            atomicOr((unsigned long long *)&a.mask[wi], (unsigned long long)w);
            a.gflag[wi >> 2] = 1;
            atomicAdd(&a.rowcnt[tl.row0 + r - a.row_base], (uint32_t)__popcll(w));
        }
    }
}

// One wave per handed-on block (see the file comment).  Grid: kBandLists x
// kDeferGroups workgroups; workgroup g reads sub-list g % kBandLists.
constexpr uint32_t kDeferGroups = 16;
template <bool HH>
__global__ __launch_bounds__(256, 3) void k_refine_g16_blocks(RefineArgs a)
{
    __shared__ __align__(16) float LQI[4][32];
    __shared__ __align__(16) float LQO[4][32];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
    // the entries of this wave: with a sorted order, XCD x (workgroups b
    // with b % kXcds = x) takes the x-th eighth of it, swept by all its
    // waves together (the grid is what the device holds at once, so the
    // waves of an XCD work on a window of consecutive entries and share
    // candidate operands in its L2); else sub-list b % kBandLists, strided
    // over the workgroups that share it
    uint64_t e_first, e_end, e_step;
    const uint4 *dl;
    if (a.dorder) {
        const uint32_t per = gridDim.x / kXcds, x = blockIdx.x % kXcds;
        const uint64_t len = (a.dtotal + kXcds - 1) / kXcds;
        const uint64_t x0 = (uint64_t)x * len;
        e_first = x0 + (uint64_t)(blockIdx.x / kXcds) * 4 + (uint64_t)wave;
        e_end = x0 + len < a.dtotal ? x0 + len : a.dtotal;
        e_step = (uint64_t)per * 4;
        dl = a.dlist;
    } else {
        const uint32_t sub = blockIdx.x % kBandLists, j0 = blockIdx.x / kBandLists, nj = gridDim.x / kBandLists;
        const unsigned long long cnt0 = a.dcount[(uint64_t)sub * kBandStride];
        e_first = (uint64_t)j0 * 4 + wave;
        e_end = cnt0 < a.dcap ? cnt0 : a.dcap;
        e_step = (uint64_t)nj * 4;
        dl = a.dlist + (uint64_t)sub * a.dcap;
    }
    const uint64_t n = a.ps, nqr = a.psq;  // part strides of the prepared arrays
    const int nsl = HH ? 2 * (((a.nb + 3) / 4 + 1) / 2) : (a.nb + 3) / 4;  // slabs (high parts: padded even)
    const int pp = HH ? 2 : 4;                                            // parts per slab
    // slabs whose operands are loaded together; the next chunk's loads are
    // in flight while a chunk's MFMAs run.  Every chunk loads all its slabs
    // (an index past the last slab repeats the last one and is not used), so
    // the loads in flight do not depend on the slab count.
    constexpr int kChunk = HH ? 4 : 2;
    struct Chunk {
        uint4 fa[kChunk], fb[kChunk], ga[kChunk], gb[kChunk];
    };
    for (uint64_t e = e_first; e < e_end; e += e_step) {
        const uint4 ent = a.dorder ? dl[a.dorder[e]] : dl[e];
        const uint32_t t = ent.x, rb = ent.y & 3u, c0 = (ent.y >> 2) << 5;
        const Tile tl = a.tiles[t];
        const uint32_t nrows = min((uint32_t)kTileRows, tl.nrows);
        const uint32_t r = rb * 32 + (uint32_t)col;
        const bool vr = r < nrows;
        const uint32_t q = tl.row0 + (vr ? r : nrows - 1);
        const uint32_t p = c0 + (uint32_t)col;
        const bool vc = (uint32_t)col < ent.w;
        uint32_t ci;
        if (ent.z != 0xffffffffu) {
            ci = ent.z + (vc ? (uint32_t)col : 0u);  // consecutive points
        } else {
            // the lane's candidate: range g with pref[g] <= p < pref[g + 1]
            const uint32_t A = tl.cell, nr = a.nrng[A];
            const uint32_t *pref = a.rpref + (uint64_t)A * (kMaxRanges + 1);
            uint32_t g = 0;
            if (vc) {
                uint32_t lo = 0, up = nr;  // pref[lo] <= p < pref[up]
                while (up - lo > 1) {
                    const uint32_t mid = (lo + up) >> 1;
                    if (pref[mid] <= p) lo = mid;
                    else up = mid;
                }
                g = lo;
            }
            ci = a.rstart[(uint64_t)A * kMaxRanges + g] + (vc ? p - pref[g] : 0u);
        }
        if (lane < 32) {
            const float nq = a.n16q[q];
            LQI[wave][col] = vr ? a.tlo - a.kp * nq - a.tabs : -INFINITY;
            LQO[wave][col] = vr ? a.thi - a.km * nq + a.tabs : -INFINITY;
        }
        const float nx = a.n16[ci];
        floatx16 acc = {};
        const uint4 *pq = a.p16q + (uint64_t)hi * nqr + q;
        const uint4 *pc = a.p16 + (uint64_t)hi * n + ci;
        auto load = [&](int s0) __attribute__((always_inline)) -> Chunk {
            Chunk c;
#pragma unroll
            for (int k = 0; k < kChunk; ++k) {
                const int sl = s0 + k < nsl ? s0 + k : nsl - 1;
                const uint64_t o = (uint64_t)sl * pp;
                c.fa[k] = pq[o * nqr];
                c.fb[k] = pc[o * n];
                if (!HH) {
                    c.ga[k] = pq[(o + 2) * nqr];
                    c.gb[k] = pc[(o + 2) * n];
                }
            }
            return c;
        };
        Chunk X = load(0);
#pragma unroll 1
        for (int s0 = 0; s0 < nsl; s0 += kChunk) {
            const Chunk Y = load(s0 + kChunk);
#pragma unroll
            for (int k = 0; k < kChunk; ++k) {
                if (s0 + k < nsl) {
                    const half8 ah = *(const half8 *)&X.fa[k], bh = *(const half8 *)&X.fb[k];
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc, 0, 0, 0);
                    if (!HH) {
                        const half8 al = *(const half8 *)&X.ga[k], bl = *(const half8 *)&X.gb[k];
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, acc, 0, 0, 0);
                    }
                }
            }
            X = Y;
        }
        g16_block_finish(a, acc, t, tl, rb, c0, r, vr, vc, ci, nx, LQI[wave], LQO[wave]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// The sorted hand-on list in the high-half form up to 24 slabs (384
// dimensions): each wave takes runs of kRunLen consecutive entries of its
// XCD's eighth of the order (the XCD's waves on consecutive runs, so that
// they share candidate operands in its L2).  The sort key puts the entries
// of one query block next to each other, so the wave keeps that block's
// fragments of every slab in registers and loads them again only when the
// query block changes; the candidate fragments stream through a ring of
// three registers, two slabs ahead.  NS: slabs held (8, 16 or 24, at
// least the operands' slab count; loads past the last slab repeat it and
// their MFMAs are skipped).
constexpr uint32_t kRunLen = 16;
template <int NS>
__global__ __launch_bounds__(256, NS > 16 ? 2 : 3) void k_refine_g16_runs(RefineArgs a)
{
    __shared__ __align__(16) float LQI[4][32];
    __shared__ __align__(16) float LQO[4][32];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 31, hi = lane >> 5;
    const uint32_t per = gridDim.x / kXcds, xcd = blockIdx.x % kXcds;
    const uint64_t len = (a.dtotal + kXcds - 1) / kXcds;
    const uint64_t x0 = (uint64_t)xcd * len, x1 = x0 + len < a.dtotal ? x0 + len : a.dtotal;
    const uint64_t gw = (uint64_t)(blockIdx.x / kXcds) * 4 + (uint64_t)wave, nw = (uint64_t)per * 4;
    const uint64_t n = a.ps, nqr = a.psq;  // part strides of the prepared arrays
    const int nsl = 2 * (((a.nb + 3) / 4 + 1) / 2);  // slabs of high halves (padded even), <= NS
    half8 qf[NS];
    uint32_t qkey = 0xffffffffu;
    for (uint64_t r0 = x0 + gw * kRunLen; r0 < x1; r0 += nw * kRunLen) {
        const uint64_t r1 = r0 + kRunLen < x1 ? r0 + kRunLen : x1;
        // the next entry is fetched while this one is refined
        uint4 nent = a.dlist[a.dorder[r0]];
        for (uint64_t e = r0; e < r1; ++e) {
            const uint4 ent = nent;
            if (e + 1 < r1) nent = a.dlist[a.dorder[e + 1]];
            const uint32_t t = ent.x, rb = ent.y & 3u, c0 = (ent.y >> 2) << 5;
            const Tile tl = a.tiles[t];
            const uint32_t nrows = min((uint32_t)kTileRows, tl.nrows);
            const uint32_t r = rb * 32 + (uint32_t)col;
            const bool vr = r < nrows;
            const uint32_t q = tl.row0 + (vr ? r : nrows - 1);
            const uint32_t p = c0 + (uint32_t)col;
            const bool vc = (uint32_t)col < ent.w;
            uint32_t ci;
            if (ent.z != 0xffffffffu) {
                ci = ent.z + (vc ? (uint32_t)col : 0u);  // consecutive points
            } else {
                // the lane's candidate: range g with pref[g] <= p < pref[g + 1]
                const uint32_t A = tl.cell, nr = a.nrng[A];
                const uint32_t *pref = a.rpref + (uint64_t)A * (kMaxRanges + 1);
                uint32_t g = 0;
                if (vc) {
                    uint32_t lo = 0, up = nr;
                    while (up - lo > 1) {
                        const uint32_t mid = (lo + up) >> 1;
                        if (pref[mid] <= p) lo = mid;
                        else up = mid;
                    }
                    g = lo;
                }
                ci = a.rstart[(uint64_t)A * kMaxRanges + g] + (vc ? p - pref[g] : 0u);
            }
            const uint32_t key = t << 2 | rb;
            if (key != qkey) {
                // a new query block: its fragments and row thresholds
                qkey = key;
                const uint4 *pq = a.p16q + (uint64_t)hi * nqr + q;
                static_for(std::make_integer_sequence<int, NS>{}, [&](auto S) {
                    constexpr int sl = decltype(S)::value;
                    const uint4 v = pq[(uint64_t)(sl < nsl ? sl : nsl - 1) * 2 * nqr];
                    qf[sl] = *(const half8 *)&v;
                });
                if (lane < 32) {
                    const float nq = a.n16q[q];
                    LQI[wave][col] = vr ? a.tlo - a.kp * nq - a.tabs : -INFINITY;
                    LQO[wave][col] = vr ? a.thi - a.km * nq + a.tabs : -INFINITY;
                }
            }
            const float nx = a.n16[ci];
            const uint4 *pc = a.p16 + (uint64_t)hi * n + ci;
            auto cload = [&](int sl) __attribute__((always_inline)) {
                return pc[(uint64_t)(sl < nsl ? sl : nsl - 1) * 2 * n];
            };
            // candidate fragments through a ring, kAhead slabs ahead (as deep
            // as the registers of the kernel's occupancy allow: a block's
            // loads come mostly from beyond L2, and only two or three waves
            // per SIMD hide their latency)
            constexpr int kAhead = NS == 24 ? 11 : NS == 16 ? 6 : 4;
            uint4 ring[kAhead + 1];
            static_for(std::make_integer_sequence<int, kAhead>{}, [&](auto S) {
                constexpr int sl = decltype(S)::value;
                ring[sl] = cload(sl);
            });
            floatx16 acc = {};
            static_for(std::make_integer_sequence<int, NS>{}, [&](auto S) {
                constexpr int sl = decltype(S)::value;
                if constexpr (sl + kAhead < NS) ring[(sl + kAhead) % (kAhead + 1)] = cload(sl + kAhead);
                if (sl < nsl)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qf[sl], *(const half8 *)&ring[sl % (kAhead + 1)], acc, 0, 0, 0);
            });
            g16_block_finish(a, acc, t, tl, rb, c0, r, vr, vc, ci, nx, LQI[wave], LQO[wave]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

}  // namespace

uint64_t prep16_stride(uint64_t n)
{
    // an odd number of 4 KiB pieces plus 128 bytes: the same row of
    // consecutive parts falls in different L2 channels and sets (a stride of
    // a power of two times 4 KiB put a block's 48 part lines in one set)
    const uint64_t units = (n + 511) / 512;  // 512 x 16 B = 8 KiB
    return (2 * units + 1) * 256 + 8;
}

hipError_t launch_prep16(const float4 *xs, uint64_t n, int nb, const float4 *nrs, float s, bool hh, uint4 *P,
                         uint64_t ps, float *N, float *NP, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    if (4 * nb <= kPartialDims || ps < n) return hipErrorInvalidValue;
    const int ns = (nb + 3) / 4;
    const uint64_t grid = (n + 255) / 256;
    if (grid > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_prep16, dim3((unsigned)grid), dim3(256), 0, st, xs, n, nb, ns, nrs, s, hh, P, ps, N, NP);
    return hipGetLastError();
}

hipError_t prepare_refine_g16(bool hh)
{
    return hipFuncSetAttribute(hh ? (const void *)k_refine_g16<true> : (const void *)k_refine_g16<false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)G16::BYTES);
}

hipError_t prepare_filter16() { return hipSuccess; }

hipError_t launch_maxabs8(const float4 *xs, uint64_t n, const float4 *ref, unsigned int *mx, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const uint64_t grid = (n + 255) / 256;
    if (grid > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_maxabs8, dim3((unsigned)grid), dim3(256), 0, st, xs, n, ref, mx);
    return hipGetLastError();
}

hipError_t launch_prep8(const float4 *xs, uint64_t n, const float4 *ref, double S, double E, uint4 *P, uint64_t ps,
                        int *start, int *bound, hipStream_t st)
{
    if (ps < n || !(S > 0.0)) return hipErrorInvalidValue;
    const uint64_t grid = (n + 1 + 255) / 256;
    if (grid > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_prep8, dim3((unsigned)grid), dim3(256), 0, st, xs, n, ref, S, E, P, ps, start, bound);
    return hipGetLastError();
}

hipError_t launch_col_bounds16(const float *np16, uint64_t n, float kmf, float *xb, hipStream_t st)
{
    const uint64_t grid = (n + 1 + 255) / 256;
    if (grid > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_col_bounds16, dim3((unsigned)grid), dim3(256), 0, st, np16, n, kmf, xb);
    return hipGetLastError();
}

hipError_t launch_filter16(const RefineArgs &a, bool hh, hipStream_t s)
{
    if (!a.dlist || !a.np16 || !a.np16q || !a.xb16) return hipErrorInvalidValue;
    if (a.seg_len % kGroupCands != 0) return hipErrorInvalidValue;
    const uint64_t blocks = (uint64_t)a.ntiles * a.nseg;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    RefineArgs args = a;
    void *params[] = {&args};
    const bool i8 = a.p8 && a.p8q && a.xb8 && a.qs8;
    const void *k = i8 ? (const void *)k_filter16<2, true>
                       : hh ? (const void *)k_filter16<2, false> : (const void *)k_filter16<4, false>;
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), params, 0, s);
}

hipError_t launch_handon_keys(const uint4 *dl, uint64_t dcap, const uint64_t *pref, uint64_t total, int qbits,
                              uint32_t gend, uint64_t *keys, uint32_t *vals, hipStream_t st)
{
    if (total == 0) return hipSuccess;
    if ((uint64_t)kBandLists * dcap > 0xffffffffull || qbits < 2 || qbits > 40) return hipErrorInvalidValue;
    const uint64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_handon_keys, dim3((unsigned)grid), dim3(256), 0, st, dl, dcap, pref, total, qbits, gend,
                       keys, vals);
    return hipGetLastError();
}

hipError_t launch_refine_g16_blocks(const RefineArgs &a, bool hh, hipStream_t s)
{
    if (!a.dlist || a.dcap == 0) return hipSuccess;
    const int nsl = 2 * (((a.nb + 3) / 4 + 1) / 2);
    // sorted order: as many workgroups as the device holds at once (three
    // per CU), a multiple of kXcds
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const uint32_t resident = ((uint32_t)cus * 3 + kXcds - 1) / kXcds * kXcds;
    if (a.dorder && hh && nsl <= 24) {
        // runs with the query block held in registers (24 slabs: two
        // workgroups per CU, the registers of three)
        if (a.dtotal == 0) return hipSuccess;
        const uint32_t two = ((uint32_t)cus * 2 + kXcds - 1) / kXcds * kXcds;
        if (nsl <= 8) hipLaunchKernelGGL(k_refine_g16_runs<8>, dim3(resident), dim3(256), 0, s, a);
        else if (nsl <= 16) hipLaunchKernelGGL(k_refine_g16_runs<16>, dim3(resident), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_refine_g16_runs<24>, dim3(two), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(a.dorder ? resident : kBandLists * kDeferGroups);
    if (hh) hipLaunchKernelGGL(k_refine_g16_blocks<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_refine_g16_blocks<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_refine_g16(const RefineArgs &a, bool hh, hipStream_t s)
{
    if (a.seg_len % kGroupCands != 0 || a.seg_len / kStepG > (uint32_t)kMaxStepsG) return hipErrorInvalidValue;
    if (!a.p16 || !a.p16q || !a.n16 || !a.n16q) return hipErrorInvalidValue;
    const uint64_t blocks = (uint64_t)a.ntiles * a.nseg;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    RefineArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(hh ? (const void *)k_refine_g16<true> : (const void *)k_refine_g16<false>,
                           dim3((unsigned)blocks), dim3(256), params, G16::BYTES, s);
}

}  // namespace ersj
