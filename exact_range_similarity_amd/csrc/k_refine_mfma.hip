// Candidate refinement for gfx950 with the dot products on MFMA.
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. IV-E (a thread block per group of queries that
// share their candidates; query and candidate tiles staged in on-chip
// memory, stored dimension-major) and Sec. IV-F (one result bit per
// comparison).
//
// Squared distances are formed as |q'|^2 + |x'|^2 - 2 q'.x' on coordinates
// centred on a reference point r of the row tile (q' = q - r, x' = x - r,
// fp32): the per-dimension median of the tile's rows (k_tile_ref), or the
// work item's first query row.
// F16 = false: q'.x' from v_mfma_f32_32x32x2f32.  F16 = true (split form):
// the centred coordinates are multiplied by a power of two s that keeps
// them below 2^14 and split into fp16 parts h + l (l = fl16(v - h)); the
// dot product h.h + h.l + l.h takes three v_mfma_f32_32x32x16_f16 per slab
// with fp32 accumulation, and norms and thresholds live in the same scaled
// domain (the host scales the thresholds by s^2).
//
// Work item: (row tile, candidate segment, row sub-block).  The 256-thread
// workgroup holds QB query blocks of 32 rows (QB = 4, 2 or 1 with growing
// d, to fit the query tile in LDS) and 4/QB candidate groups; wave w owns
// query block w % QB and candidate group w / QB and computes a 32 x 64
// block per step (two 32x32 accumulators) = one 64-bit mask word per row.
// A step covers 256/QB candidates; candidates are staged through LDS in
// slabs of 16 dimensions (double-buffered, loaded two slabs ahead, centred
// and squared once by the loading thread) and read by all QB query blocks.
//
// MFMA operands: lanes 0-31 carry dimension block 2s, lanes 32-63 block
// 2s+1 of the same query/candidate (column = lane % 32); the four components
// of a float4 feed four k = 2 steps.  Split form: lane l carries row (or
// column) l % 32 and the eight k = 8*(l/32) .. 8*(l/32)+7 of the slab's high
// (or low) halves.  The output element of register v in
// lane l is (row 8*(v/4) + 4*(l/32) + v%4, column l%32).
//
// Classification with a norm-proportional band.  With Nq = |q'|^2,
// Nx = |x'|^2, D = q'.x' (fp32, any summation order) and K = kp - 1:
//   in   iff  fma(-2, D, kp*Nx) <= tlo - kp*Nq
//   out  iff  fma(-2, D, km*Nx) >  thi - km*Nq          (km = 1 - K)
//   else boundary -> exact binary64 re-check.
// K >= 2.02*gamma(d_pad+2) + 6.1u covers the rounding of the centring, of
// the norms and dot products, and of these fp32 expressions, so "in" implies
// D64 <= fl(eps^2) and "out" implies D64 > fl(eps^2).  The split form's K
// adds the dropped l.l product, the split residues and the fp16 MFMA's
// accumulation error, and both sides move by an absolute term tabs for
// parts in fp16's subnormal range.  The host bounds the
// coordinates so that nothing here overflows; NaN never classifies.
//
// Block pruning: rows within a cell follow a fine Morton order, so a query
// block and a 64-candidate group are compact on the three grid axes (the
// first three dimensions of the layout).  When the gap between their
// bounding boxes there already exceeds eps (squared gaps summed in fp32 >
// tbox, a bound that covers the rounding), the pair of them holds no
// neighbour.  Each wave tests all its steps against the candidate groups'
// boxes (precomputed per 64-candidate chunk after the count pass) before
// the loop: steps that every wave passes are dropped (no loads, no staging,
// zero mask words), and in the others a wave skips its own far steps.
//
// A step's classification follows its last slab's MFMAs; the waves that
// share a SIMD overlap one's classification with another's matrix work.
// With QB = 4 the kernel stays within 128 VGPRs and, up to d = 32, 40 KiB of
// LDS, so four workgroups fit a CU.  Mask words collect in LDS and leave as
// aligned 64-byte row pieces every 512 candidates.
#include "refine_mfma_common.h"

namespace ersj {

namespace {

constexpr int kNB = 2;  // step buffers for norms / candidate ids

// Load registers of a slab: its own with a constant slab count (S is the
// slab's integral_constant), else the front of the shifted queue.
template <int NS, class S>
__device__ constexpr int slab_slot()
{
    if constexpr (NS > 0) return S::value;
    else return 0;
}

template <int QB>
struct Geometry {
    static constexpr int NCG = 4 / QB;            // candidate groups
    static constexpr int QR = 32 * QB;            // query rows per work item
    static constexpr int SC = 64 * NCG;           // candidates per step
    static constexpr int SPG = kGroupCands / SC;  // steps per mask-word group
    static constexpr int EPT = kSlab * SC / 256;   // slab elements staged per thread
};

template <int QB>
struct Lds {
    float4 *q;          // [nbs][QR] centred queries
    float4 *r;          // [nbs] reference point
    float4 *x;          // [2][kSlab][SC] centred candidate slab
    float *nxp;         // [kNB][kSlab][SC] partial candidate norms of a step
    uint32_t *xi;       // [kNB][SC] candidate point index of a step
    float *qin, *qout;  // [QR]
    uint32_t *rcnt;     // [QR] mask bits set per row by this work item
    float *nqmax;       // [QB] largest query norm of each query block
    uint64_t *words;    // [QR][8] mask words of the current 512-candidate group
    uint32_t *far;      // [4 waves][4] steps (bit s) each wave skips
    uint32_t *live;     // [kMaxSteps] steps some wave computes, ascending
    uint32_t *pref, *start;
};

template <int QB>
size_t lds_bytes(int nbs)
{
    using G = Geometry<QB>;
    return (size_t)nbs * (G::QR + 1) * 16 + (size_t)2 * kSlab * G::SC * 16 + (size_t)kNB * kSlab * G::SC * 4 +
           (size_t)kNB * G::SC * 4 + (size_t)3 * G::QR * 4 + (size_t)QB * 4 + (size_t)G::QR * 8 * 8 +
           (size_t)(16 + kMaxSteps) * 4 + (2 * kMaxRanges + 1) * 4;
}

template <int QB>
__device__ __forceinline__ Lds<QB> carve(float4 *smem, int nbs)
{
    using G = Geometry<QB>;
    Lds<QB> L;
    L.q = smem;
    L.r = L.q + nbs * G::QR;
    L.x = L.r + nbs;
    L.nxp = (float *)(L.x + 2 * kSlab * G::SC);
    L.xi = (uint32_t *)(L.nxp + kNB * kSlab * G::SC);
    L.qin = (float *)(L.xi + kNB * G::SC);
    L.qout = L.qin + G::QR;
    L.rcnt = (uint32_t *)(L.qout + G::QR);
    L.nqmax = (float *)(L.rcnt + G::QR);
    L.words = (uint64_t *)(L.nqmax + QB);
    L.far = (uint32_t *)(L.words + G::QR * 8);
    L.live = L.far + 16;
    L.pref = L.live + kMaxSteps;
    L.start = L.pref + (kMaxRanges + 1);
    return L;
}

template <int QB, int NS, bool F16>
__global__ __launch_bounds__(256, QB == 4 ? 4 : 1) void k_refine_mfma(RefineArgs a)
{
    using G = Geometry<QB>;
    uint32_t rk, colx;
    work_item(blockIdx.x, a.ntiles, a.nseg * a.nsub, &rk, &colx);
    const uint32_t seg = colx / a.nsub, sub = colx - seg * a.nsub;
    const uint32_t t = a.order[a.ord0 + rk];
    const Tile tl = a.tiles[t];
    const uint32_t r_begin = sub * G::QR;
    if (r_begin >= tl.nrows) return;
    const uint32_t A = tl.cell;
    const uint32_t nr = a.nrng[A];
    const uint32_t *pref_g = a.rpref + (uint64_t)A * (kMaxRanges + 1);
    const uint32_t U = pref_g[nr];
    const uint32_t c_begin = seg * a.seg_len;
    if (c_begin >= U) return;
    const uint32_t c_end = min(U, c_begin + a.seg_len);
    const uint32_t nrows = min((uint32_t)G::QR, tl.nrows - r_begin);
    const uint32_t row0 = tl.row0 + r_begin;
    const int nb = a.nb;
    // slabs per step: a compile-time constant when NS > 0 (d <= 16, d <= 32)
    const int nslab = NS > 0 ? NS : (nb + kSlab - 1) / kSlab;
    const int nbs = nslab * kSlab;

    extern __shared__ float4 smem[];
    const Lds<QB> L = carve<QB>(smem, nbs);

    const int tid = threadIdx.x;
    const uint64_t n = a.n;
    const float4 *__restrict__ xs = a.xs;
    const float4 *__restrict__ xq = a.xq;  // query rows (the points themselves in a self-join)
    const uint64_t nqr = a.nqr;
    uint64_t *__restrict__ mask = a.mask;
    const uint32_t W = tl.words;
    const uint64_t mbase = a.toff[t] - a.wbase + (uint64_t)r_begin * W;

    if (tid <= kMaxRanges) L.pref[tid] = tid <= (int)nr ? pref_g[tid] : 0xffffffffu;
    if (tid < kMaxRanges) L.start[tid] = a.rstart[(uint64_t)A * kMaxRanges + tid];
    for (int b = tid; b < nbs; b += 256)
        L.r[b] = b >= nb ? make_float4(0.f, 0.f, 0.f, 0.f) : a.tref ? a.tref[(uint64_t)t * nb + b]
                                                                     : xq[(uint64_t)b * nqr + row0];
    __syncthreads();
    for (int e = tid; e < nbs * G::QR; e += 256) {
        const int b = e / G::QR, i = e - b * G::QR;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (b < nb && (uint32_t)i < nrows) v = sub4(xq[(uint64_t)b * nqr + row0 + i], L.r[b]);
        if constexpr (F16) {
            // slab sl = b / kSlab holds [hi k 0-7, hi k 8-15, lo k 0-7, lo k 8-15][row]
            const int sl = b / kSlab, j = b % kSlab;
            half4 h, l;
            split16(scale4(v, a.s16), h, l);
            ((half4 *)&L.q[(sl * kSlab + j / 2) * G::QR + i])[j & 1] = h;
            ((half4 *)&L.q[(sl * kSlab + 2 + j / 2) * G::QR + i])[j & 1] = l;
        } else {
            L.q[e] = v;
        }
    }
    __syncthreads();
    for (int i = tid; i < G::QR; i += 256) {
        float nq = 0.f;
        for (int b = 0; b < nb; ++b) {
            float4 v;
            if constexpr (F16) {
                v = make_float4(0.f, 0.f, 0.f, 0.f);
                if ((uint32_t)i < nrows) v = scale4(sub4(xq[(uint64_t)b * nqr + row0 + i], L.r[b]), a.s16);
            } else {
                v = L.q[b * G::QR + i];
            }
            nq = fmaf(v.x, v.x, nq);
            nq = fmaf(v.y, v.y, nq);
            nq = fmaf(v.z, v.z, nq);
            nq = fmaf(v.w, v.w, nq);
        }
        const bool live = (uint32_t)i < nrows;
        const float tabs = F16 ? a.tabs : 0.f;
        L.qin[i] = live ? a.tlo - a.kp * nq - tabs : -INFINITY;
        L.qout[i] = live ? a.thi - a.km * nq + tabs : -INFINITY;
        L.rcnt[i] = 0;
        // the largest norm of each 32-row query block (rows past nrows: 0)
        float m = live ? nq : 0.f;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if ((i & 31) == 0) L.nqmax[i >> 5] = m;
    }
    for (int e = tid; e < G::QR * 8; e += 256) L.words[e] = 0ull;
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31, hi = lane >> 5;
    const int qb = wave % QB, cg = wave / QB;
    const bool active = (uint32_t)(qb * 32) < nrows;  // wave-uniform
    // the wave's query block box over the first kBoxBlocks layout blocks (raw
    // coordinates, valid rows only; blocks past nb are zero padding), the
    // same in every lane
    float4 qlo[kBoxBlocks], qhi[kBoxBlocks];
    {
        const uint32_t i = (uint32_t)(qb * 32 + (lane & 31));
#pragma unroll
        for (int b = 0; b < kBoxBlocks; ++b) {
            qlo[b] = make_float4(INFINITY, INFINITY, INFINITY, INFINITY);
            qhi[b] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (i < nrows) {
                qlo[b] = b < a.nb ? xq[(uint64_t)b * a.nqr + row0 + i] : make_float4(0.f, 0.f, 0.f, 0.f);
                qhi[b] = qlo[b];
            }
            wave_box4(qlo[b], qhi[b]);
        }
    }
    const float kp = a.kp, km = a.km;
    // the split-fp16 form classifies in the scaled domain (coordinates, norms
    // and thresholds multiplied by s, s^2 and s^2; host-side thresholds)
    //
    // Norm test of a candidate column against the wave's query block: with
    // v the centred (scaled) fp32 coordinates and N their computed norms,
    // |v_x - v_q| >= |v_x| - |v_q|, and the centring moves |v_x - v_q| by at
    // most u (|v_x| + |v_q|) from s |x - q|.  With g = gamma of the terms in
    // a norm (|N - |v|^2| <= g |v|^2), a candidate with
    //   N_x > tn = ((sqrt(max N_q) + sqrt(thi)) c1)^2 c2,
    //   c1 = 1 + g + 2^-18, c2 = 1 + 2 g + 2^-16,
    // has s |x - q| > sqrt(thi) for every row of the block, so it is out
    // there: c1^2 c2 exceeds the 1 + 3 g + 5 u the bounds need by more than
    // the rounding of the square roots, sums and products that form tn, and
    // thi already covers the binary64 definition.  A 32-candidate half whose
    // columns are all such skips its classification (its bits stay zero).
    // thi = inf gives tn = inf: no skip.
    const float tn = [&]() {
        const float nt = 4.0f * (float)nb + 4.0f;  // terms (and additions) in a norm
        const float g = nt * 0x1p-24f / (1.0f - nt * 0x1p-24f);
        const float c1 = 1.0f + g + 0x1p-18f, c2 = 1.0f + 2.0f * g + 0x1p-16f;
        const float sq = sqrtf(L.nqmax[qb]) * c1, st = sqrtf(a.thi) * c1;
        return ((sq + st) * (sq + st)) * c2;
    }();
    const BandSink bsink{band_list(a.blist, a.lcap), band_counter(a.bcount), a.lcap, row0, mbase, W};
    const uint32_t nsteps = (c_end - c_begin + G::SC - 1) / G::SC;
    const uint32_t qrows = active ? min(32u, nrows - (uint32_t)(qb * 32)) : 0u;
    const float tbox = a.tbox;

    // Block box test of every step up front: the wave's query box against
    // its candidate group's box (precomputed per 64-candidate chunk of the
    // cell's list).  Steps that every wave skips are dropped from the loop
    // (no loads, no staging); the wave skips its own far steps among the
    // rest.  Segments longer than kMaxSteps steps are not tested.
    const bool tested = tbox < INFINITY && nsteps <= (uint32_t)kMaxSteps;
    uint32_t far0 = 0, far1 = 0, far2 = 0, far3 = 0;
    uint64_t nskip = 0;  // comparisons this wave skipped
    if (tested) {
        const uint64_t cb0 = a.chunk_base[A] + (c_begin >> 6) + (uint32_t)cg;
        for (uint32_t st = 0; st < nsteps; ++st) {
            const uint32_t gs = c_begin + st * G::SC + cg * 64;
            uint32_t bit = 1;
            if (active && gs < c_end) {
                const float4 *cb = a.cbox + 2 * kBoxBlocks * (cb0 + st * (uint32_t)(G::SC / 64));
                float g2 = 0.f;
#pragma unroll
                for (int b = 0; b < kBoxBlocks; ++b) g2 = gap4(qlo[b], qhi[b], cb[2 * b], cb[2 * b + 1], g2);
                bit = __builtin_amdgcn_readfirstlane((int)(g2 > tbox));
            }
            if (bit) {
                const uint32_t m = 1u << (st & 31);
                if (st < 32) far0 |= m;
                else if (st < 64) far1 |= m;
                else if (st < 96) far2 |= m;
                else far3 |= m;
                if (gs < c_end) nskip += (uint64_t)qrows * min(64u, c_end - gs);
            }
        }
    }
    auto wave_far = [&](uint32_t st) __attribute__((always_inline)) {
        const uint32_t w = st < 32 ? far0 : st < 64 ? far1 : st < 96 ? far2 : far3;
        return ((w >> (st & 31)) & 1u) != 0;
    };
    uint32_t nlive = nsteps;
    if (tested) {
        if (lane == 0) {
            L.far[wave * 4 + 0] = far0;
            L.far[wave * 4 + 1] = far1;
            L.far[wave * 4 + 2] = far2;
            L.far[wave * 4 + 3] = far3;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t c = 0;
            for (uint32_t st = 0; st < nsteps; ++st) {
                const uint32_t i = st >> 5, m = 1u << (st & 31);
                if (!(L.far[i] & L.far[4 + i] & L.far[8 + i] & L.far[12 + i] & m)) L.live[c++] = st;
            }
            L.far[0] = c;  // read back below, after the barrier
        }
        __syncthreads();
        nlive = __builtin_amdgcn_readfirstlane(L.far[0]);
    }
    // step of live index i (i = nlive: past the segment, loads nothing new)
    auto live_step = [&](uint32_t i) __attribute__((always_inline)) {
        if (i >= nlive) return nsteps;
        return tested ? L.live[i] : i;
    };
    const uint32_t K = nlive * (uint32_t)nslab;

    // loader: element m of this thread is (block j = e / SC, candidate c =
    // e % SC), e = tid + 256 m.  Its candidate position advances by SC per
    // step, so the merged range it falls in is tracked incrementally (ranges
    // are visited in order); positions past the segment end reuse the first
    // candidate so that every load stays in bounds.
    uint32_t rg[G::EPT], rnext[G::EPT], roff[G::EPT], lxi[G::EPT];
    uint32_t idx0;
    {
        const int g = range_of(L.pref, nr, c_begin);
        idx0 = L.start[g] + (c_begin - L.pref[g]);
#pragma unroll
        for (int m = 0; m < G::EPT; ++m) {
            rg[m] = (uint32_t)g;
            rnext[m] = g + 1 < (int)nr ? L.pref[g + 1] : 0xffffffffu;
            roff[m] = L.start[g] - L.pref[g];
        }
    }
    auto set_cands = [&](uint32_t step) {
#pragma unroll
        for (int m = 0; m < G::EPT; ++m) {
            const uint32_t p = c_begin + step * G::SC + (uint32_t)((tid + 256 * m) % G::SC);
            if (p < c_end) {
                while (p >= rnext[m]) {
                    const uint32_t g = ++rg[m];
                    rnext[m] = g + 1 < nr ? L.pref[g + 1] : 0xffffffffu;
                    roff[m] = L.start[g] - L.pref[g];
                }
                lxi[m] = p + roff[m];
            } else {
                lxi[m] = idx0;
            }
        }
    };
    // Loads run kAhead slabs ahead of the staging.  With a constant slab
    // count the slab of a step has its own load registers (ld[sl]), loaded
    // one step ahead: a register is never copied while its load is in
    // flight, which would make the wave wait for that load at once.
    constexpr int kAhead = NS > 0 ? NS : 2;
    float4 ld[kAhead][G::EPT];
    uint32_t ldx[kAhead][G::EPT];
    // element offset of the next load: block b = lsl * kSlab + j of the
    // candidate, i.e. b * n + index, advanced by kSlab * n within a step
    uint64_t loff[G::EPT];
    const uint64_t slab_stride = (uint64_t)kSlab * n;
    auto load_slab = [&](int sl, float4 *dst, uint32_t *dx) {
#pragma unroll
        for (int m = 0; m < G::EPT; ++m) {
            const int b = sl * kSlab + (tid + 256 * m) / G::SC;
            dst[m] = b < nb ? xs[loff[m]] : make_float4(0.f, 0.f, 0.f, 0.f);
            dx[m] = lxi[m];
        }
    };
    auto restart_offsets = [&]() {
#pragma unroll
        for (int m = 0; m < G::EPT; ++m) loff[m] = (uint64_t)((tid + 256 * m) / G::SC) * n + lxi[m];
    };
    // load cursor: slab lsl of step lstep
    uint32_t lstep = 0;
    int lsl = 0;
    auto cursor_next = [&]() {
        if (++lsl == nslab) {
            lsl = 0;
            ++lstep;
            set_cands(live_step(lstep));
            restart_offsets();
        } else {
#pragma unroll
            for (int m = 0; m < G::EPT; ++m) loff[m] += slab_stride;
        }
    };
    set_cands(live_step(0));
    restart_offsets();
#pragma unroll
    for (int a2 = 0; a2 < kAhead; ++a2) {
        if ((uint32_t)a2 < K) load_slab(lsl, ld[a2], ldx[a2]);
        if ((uint32_t)a2 + 1 < K) cursor_next();
    }
    float nxp[G::EPT];
#pragma unroll
    for (int m = 0; m < G::EPT; ++m) nxp[m] = 0.f;
    floatx16 accC[2];
    int pend_group = -1;            // group whose words wait in L.words
    uint32_t pend_next = 0;         // next group with a live step (groups between are zero)
    const uint32_t ngroups = (nsteps + G::SPG - 1) / G::SPG;

    // classification of step s (accumulators in acc): mask words and band pairs
    auto epilogue = [&](uint32_t s, uint32_t bi, const floatx16 *acc) {
        const uint32_t cw = c_begin + s * G::SC + cg * 64;
        float xin[2], xout[2];
        uint32_t xid[2];
        uint32_t live = 0;  // halves to classify
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int cl = cg * 64 + 32 * tt + col;
            const float *np = L.nxp + (bi % kNB) * (kSlab * G::SC);
            float nxt = np[cl];
#pragma unroll
            for (int j = 1; j < kSlab; ++j) nxt += np[j * G::SC + cl];
            xid[tt] = L.xi[(bi % kNB) * G::SC + cl];
            // candidates past the segment end never classify: a NaN operand
            // makes both comparisons false (an infinity would not: with an
            // infinite eps, inf <= inf holds)
            const bool valid = cw + 32 * tt + col < c_end;
            xin[tt] = valid ? kp * nxt : __builtin_nanf("");
            xout[tt] = valid ? km * nxt : __builtin_nanf("");
            if (__ballot(!(nxt > tn)) != 0) live |= 1u << tt;  // a column not decided by its norm
        }
        if (live != 0)
            classify_block(acc, xin, xout, L.qin, L.qout, qb, lane, cw, live, bsink, [&](int tt) { return xid[tt]; },
                           L.words + (qb * 32 + (lane & 31)) * 8 + (s % G::SPG) * G::NCG + cg);
    };
    // unit flags: the 4 words of a unit sit in 4 consecutive lanes (e & 7
    // = j, units j 0-3 and 4-7 of a row); the first lane of the unit writes
    auto unit_flag = [&](int row, int j, uint32_t w, bool ok, bool nz) __attribute__((always_inline)) {
        const uint64_t b = __ballot(nz);
        if (ok && (j & 3) == 0) a.gflag[(mbase + (uint64_t)row * W + w) >> 2] = ((b >> (lane & ~3)) & 0xfull) ? 1 : 0;
    };
    auto flush = [&](uint32_t grp) {
        uint64_t *sw = L.words;
        for (int e = tid; e < G::QR * 8; e += 256) {
            const int row = e >> 3, j = e & 7;
            const uint32_t c0 = c_begin + grp * kGroupCands + 64 * j;
            const uint32_t w = c0 >> 6;
            const bool ok = (uint32_t)row < nrows && w < W && c0 < c_end;
            const uint64_t v = sw[e];
            if (ok) {
                mask[mbase + (uint64_t)row * W + w] = v;
                const uint32_t pc = __popcll(v);
                if (pc != 0) atomicAdd(&L.rcnt[row], pc);
            }
            unit_flag(row, j, w, ok, ok && v != 0);
            sw[e] = 0ull;  // words of steps the next group skips stay zero
        }
    };
    // groups without a live step: zero words
    auto zero_groups = [&](uint32_t g0, uint32_t g1) {
        for (uint32_t g = g0; g < g1; ++g) {
            for (int e = tid; e < G::QR * 8; e += 256) {
                const int row = e >> 3, j = e & 7;
                const uint32_t c0 = c_begin + g * kGroupCands + 64 * j;
                const uint32_t w = c0 >> 6;
                const bool ok = (uint32_t)row < nrows && w < W && c0 < c_end;
                if (ok) mask[mbase + (uint64_t)row * W + w] = 0ull;
                unit_flag(row, j, w, ok, false);
            }
        }
    };
    auto mfma_slab = [&](const float4 *xb, int sl, bool fresh) {
        if constexpr (F16) {
            // one k = 16 step: hi.hi + hi.lo + lo.hi (lo.lo is below the band)
            const half8 ah = *(const half8 *)&L.q[(sl * kSlab + hi) * G::QR + qb * 32 + col];
            const half8 al = *(const half8 *)&L.q[(sl * kSlab + 2 + hi) * G::QR + qb * 32 + col];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int cc = cg * 64 + 32 * tt + col;
                const half8 bh = *(const half8 *)&xb[hi * G::SC + cc];
                const half8 bl = *(const half8 *)&xb[(2 + hi) * G::SC + cc];
                if (fresh) {
                    const floatx16 z = {};
                    accC[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, z, 0, 0, 0);
                } else {
                    accC[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, accC[tt], 0, 0, 0);
                }
                accC[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, accC[tt], 0, 0, 0);
                accC[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, accC[tt], 0, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int s2 = 0; s2 < kSlab / 2; ++s2) {
            // block pairs past the last dimension block are zero padding
            if (s2 > 0 && sl * kSlab + 2 * s2 >= nb) break;
            const int jj = 2 * s2 + hi;
            const float4 av = L.q[(sl * kSlab + jj) * G::QR + qb * 32 + col];
            const float4 b0 = xb[jj * G::SC + cg * 64 + col];
            const float4 b1 = xb[jj * G::SC + cg * 64 + 32 + col];
            if (s2 == 0 && fresh) {
                const floatx16 z = {};
                accC[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b0.x, z, 0, 0, 0);
                accC[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b1.x, z, 0, 0, 0);
            } else {
                accC[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b0.x, accC[0], 0, 0, 0);
                accC[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b1.x, accC[1], 0, 0, 0);
            }
            accC[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, b0.y, accC[0], 0, 0, 0);
            accC[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, b1.y, accC[1], 0, 0, 0);
            accC[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, b0.z, accC[0], 0, 0, 0);
            accC[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, b1.z, accC[1], 0, 0, 0);
            accC[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, b0.w, accC[0], 0, 0, 0);
            accC[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, b1.w, accC[1], 0, 0, 0);
        }
    };

    // One slab: stage it, barrier, decide the step's block test (first
    // slab), flush a finished mask-word group and issue the loads kAhead
    // slabs ahead.  Returns the staged buffer.  With NS > 0 the slab index is
    // a constant and every per-slab condition folds.
    auto stage = [&](uint32_t k, uint32_t bi, auto SLC) __attribute__((always_inline)) {
        const int sl = SLC;
        float4 *xb = L.x + (k & 1) * (kSlab * G::SC);
        // stage the slab: centre on r, accumulate partial norms
#pragma unroll
        for (int m = 0; m < G::EPT; ++m) {
            const int e = tid + 256 * m;
            const int j = e / G::SC;
            constexpr int li = slab_slot<NS, decltype(SLC)>();
            const float4 c4 = F16 ? scale4(sub4(ld[li][m], L.r[sl * kSlab + j]), a.s16)
                                  : sub4(ld[li][m], L.r[sl * kSlab + j]);
            float s2 = nxp[m];
            s2 = fmaf(c4.x, c4.x, s2);
            s2 = fmaf(c4.y, c4.y, s2);
            s2 = fmaf(c4.z, c4.z, s2);
            s2 = fmaf(c4.w, c4.w, s2);
            nxp[m] = s2;
            if constexpr (F16) {
                // [hi k 0-7, hi k 8-15, lo k 0-7, lo k 8-15][candidate]
                const int c = e - j * G::SC;
                half4 h, l;
                split16(c4, h, l);
                ((half4 *)&xb[(j / 2) * G::SC + c])[j & 1] = h;
                ((half4 *)&xb[(2 + j / 2) * G::SC + c])[j & 1] = l;
            } else {
                xb[e] = c4;
            }
        }
        if (sl == nslab - 1) {
#pragma unroll
            for (int m = 0; m < G::EPT; ++m) {
                const int e = tid + 256 * m;
                L.nxp[(bi % kNB) * (kSlab * G::SC) + e] = nxp[m];
                if (e < G::SC) L.xi[(bi % kNB) * G::SC + e] = ldx[slab_slot<NS, decltype(SLC)>()][m];
                nxp[m] = 0.f;
            }
        }
        __syncthreads();
        if (pend_group >= 0) {
            // the group buffer is reused by the next group: with one slab
            // per step this step's classification follows in this same
            // iteration, so wait for the whole flush first
            flush((uint32_t)pend_group);
            zero_groups((uint32_t)pend_group + 1, pend_next);
            pend_group = -1;
            if (nslab == 1) __syncthreads();
        }
        if constexpr (NS == 0) {
#pragma unroll
            for (int a2 = 0; a2 + 1 < kAhead; ++a2) {
#pragma unroll
                for (int m = 0; m < G::EPT; ++m) {
                    ld[a2][m] = ld[a2 + 1][m];
                    ldx[a2][m] = ldx[a2 + 1][m];
                }
            }
        }
        if (k + kAhead < K) {
            if constexpr (NS > 0) {
                // this slab of the next step, into the registers just staged;
                // the slab after it is known here
                constexpr int li = slab_slot<NS, decltype(SLC)>();
                load_slab(li, ld[li], ldx[li]);
                if ((sl + kAhead + 1) % NS == 0) {
                    set_cands(live_step(bi + (uint32_t)((sl + kAhead + 1) / NS)));
                    restart_offsets();
                } else {
#pragma unroll
                    for (int m = 0; m < G::EPT; ++m) loff[m] += slab_stride;
                }
            } else {
                load_slab(lsl, ld[kAhead - 1], ldx[kAhead - 1]);
                cursor_next();
            }
        }
        return xb;
    };
    // groups before the first live step hold no neighbour
    zero_groups(0, nlive > 0 ? live_step(0) / G::SPG : ngroups);
    // Each live step branches once on the wave's own test, so the
    // accumulators are never live across steps; both branches stage the same
    // slabs and meet the same barriers.
    for (uint32_t bi = 0; bi < nlive; ++bi) {
        const uint32_t step = __builtin_amdgcn_readfirstlane(live_step(bi));
        const uint32_t k0 = bi * (uint32_t)nslab;
        float4 *xb0 = stage(k0, bi, std::integral_constant<int, 0>{});
        if (active && !wave_far(step)) {
            mfma_slab(xb0, 0, true);
            if constexpr (NS > 0) {
                static_for(std::make_integer_sequence<int, NS - 1>{}, [&](auto S) __attribute__((always_inline)) {
                    constexpr int sl = decltype(S)::value + 1;
                    mfma_slab(stage(k0 + sl, bi, std::integral_constant<int, sl>{}), sl, false);
                });
            } else {
                for (int sl = 1; sl < nslab; ++sl) mfma_slab(stage(k0 + sl, bi, sl), sl, false);
            }
            epilogue(step, bi, accC);
        } else {
            if constexpr (NS > 0) {
                static_for(std::make_integer_sequence<int, NS - 1>{}, [&](auto S) __attribute__((always_inline)) {
                    constexpr int sl = decltype(S)::value + 1;
                    stage(k0 + sl, bi, std::integral_constant<int, sl>{});
                });
            } else {
                for (int sl = 1; sl < nslab; ++sl) stage(k0 + sl, bi, sl);
            }
        }
        // flush the group after its last live step (at the next barrier)
        const uint32_t g = step / G::SPG;
        const uint32_t gn = bi + 1 < nlive ? live_step(bi + 1) / G::SPG : ngroups;
        if (gn != g) {
            pend_group = (int)g;
            pend_next = gn;
        }
    }
    __syncthreads();
    if (pend_group >= 0) {
        flush((uint32_t)pend_group);
        zero_groups((uint32_t)pend_group + 1, pend_next);
    }
    if (nskip != 0 && lane == 0)
        atomicAdd(&a.skipped[(uint64_t)(blockIdx.x % kHitSlots) * kBandStride], (unsigned long long)nskip);
    // the rows' neighbour counts (the binary64 re-check adds the band's)
    __syncthreads();
    for (int i = tid; i < (int)nrows; i += 256)
        if (L.rcnt[i] != 0) atomicAdd(&a.rowcnt[row0 + i - a.row_base], L.rcnt[i]);
}

}  // namespace

int refine_mfma_qblocks(int nb)
{
    const int nbs = (nb + kSlab - 1) / kSlab * kSlab;
    if (lds_bytes<4>(nbs) <= 64 * 1024) return 4;
    if (lds_bytes<2>(nbs) <= 80 * 1024) return 2;
    return 1;
}

size_t refine_mfma_lds_bytes(int nb)
{
    const int nbs = (nb + kSlab - 1) / kSlab * kSlab;
    switch (refine_mfma_qblocks(nb)) {
    case 4: return lds_bytes<4>(nbs);
    case 2: return lds_bytes<2>(nbs);
    default: return lds_bytes<1>(nbs);
    }
}

namespace {

// kernel instance for nb dimension blocks: query blocks per workgroup and
// slabs per step (1 and 2 are compiled as constants)
template <bool F16>
const void *mfma_kernel_t(int nb)
{
    const int nslab = (nb + kSlab - 1) / kSlab;
    switch (refine_mfma_qblocks(nb)) {
    case 4:
        if (nslab == 1) return (const void *)k_refine_mfma<4, 1, F16>;
        if (nslab == 2) return (const void *)k_refine_mfma<4, 2, F16>;
        return (const void *)k_refine_mfma<4, 0, F16>;
    case 2: return (const void *)k_refine_mfma<2, 0, F16>;
    default: return (const void *)k_refine_mfma<1, 0, F16>;
    }
}

const void *mfma_kernel(int nb, bool f16)
{
    return f16 ? mfma_kernel_t<true>(nb) : mfma_kernel_t<false>(nb);
}

}  // namespace

hipError_t prepare_refine_mfma(int nb, bool f16)
{
    return hipFuncSetAttribute(mfma_kernel(nb, f16), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)refine_mfma_lds_bytes(nb));
}

hipError_t launch_refine_mfma(const RefineArgs &a, bool f16, hipStream_t s)
{
    const uint64_t blocks = (uint64_t)a.ntiles * a.nseg * a.nsub;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    const size_t bytes = refine_mfma_lds_bytes(a.nb);
    RefineArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(mfma_kernel(a.nb, f16), dim3((unsigned)blocks), dim3(256), params, bytes, s);
}

}  // namespace ersj
