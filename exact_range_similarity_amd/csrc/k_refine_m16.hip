// Candidate refinement for gfx950, split-fp16 form on MFMA, for up to 64
// dimensions (one to four 16-dimension slabs).
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. IV-E (a thread block per group of queries that
// share their candidates, candidates staged through on-chip memory) and
// Sec. IV-F (one result bit per comparison).
//
// Block box test over dimensions 0-7 of the variance-ordered layout (the
// grid axes and the next ones), not only the grid axes: a cell's stencil
// often holds clusters that are close on the grid axes and far apart on the
// others.
//
// Arithmetic and classification are those of the split-fp16 form of
// k_refine_mfma.hip: coordinates centred on the tile's reference point r and
// scaled by the power of two s (computed as fma(x, s, -(r s)), which equals
// fl(x - r) s whenever r s is exact), split into fp16 halves h + l, dot
// products h.h + h.l + l.h on v_mfma_f32_32x32x16_f16 with fp32
// accumulation, fp32 norms of the scaled coordinates, and the same
// norm-proportional band, absolute slack and thresholds (classify_block).
//
// Work decomposition (what differs from k_refine_mfma):
//  - A workgroup (4 waves) takes one whole row tile (up to 128 query rows
//    of a cell) and a segment of the cell's candidate list.  Each wave
//    holds QBW 32-row query blocks (QBW = 2: rows 64 (w % 2) .. +63 against
//    candidates 64 (w / 2) .. +63 of a 128-candidate step, four 32 x 32
//    accumulators; QBW = 1: rows 32 w .. +31 against the 64 candidates of a
//    step, two accumulators and few enough registers for four waves per
//    SIMD).
//  - The query blocks' fp16 halves stay in registers for the whole work
//    item (the MFMA A operands), so LDS carries only candidates.
//  - A step's candidates are staged whole (all slabs) into one of two LDS
//    buffers: one barrier per step.  Each thread stages one candidate's
//    half of the dimension blocks; the loads for the next step are issued
//    before the current step's matrix work.
//  - Candidate positions map to points through the cell's merged ranges;
//    a step inside one range (the common case) takes a wave-uniform offset.
//  - Mask words of a 512-candidate group collect in LDS (two buffers,
//    alternating at each flush, up to three slabs; one buffer and a barrier
//    after each flush at four) and leave as aligned 64-byte row pieces, with
//    one flag byte per four words, as in k_refine_mfma.
#include "refine_mfma_common.h"

namespace ersj {

namespace {

constexpr int kRows = 128;  // query rows per work item (one tile)

template <int NS, int QBW>
struct M16 {
    static constexpr int RW = 4 / QBW;          // waves per candidate group (row groups)
    static constexpr int CG = QBW;              // candidate groups of 64 per step
    static constexpr int STEP = 64 * CG;        // candidates per step
    static constexpr int TPC = 256 / STEP;      // staging threads per candidate
    static constexpr int NBS = 4 * NS;          // float4 blocks per candidate (padded)
    static constexpr int PER = NBS / TPC;       // blocks staged per thread
    static constexpr int GS = kGroupCands / STEP;  // steps per 512-candidate mask-word group
    static constexpr int MAXST = 8192 / STEP;   // steps of the longest segment
    static constexpr int FW = MAXST / 64;       // 64-bit words of a step bit set (MAXST * CG = 128)
    static constexpr int WB = NS >= 4 ? 1 : 2;  // mask-word group buffers
    // LDS layout (bytes)
    static constexpr size_t X = 0;                                         // [2][NS][4][STEP] x 16 B
    static constexpr size_t NXP = X + (size_t)2 * NS * 4 * STEP * 16;       // [2][TPC][STEP] f32
    static constexpr size_t XI = NXP + (size_t)2 * TPC * STEP * 4;          // [2][STEP] u32
    static constexpr size_t NRS = XI + (size_t)2 * STEP * 4;                // [NBS] float4: -(r s)
    static constexpr size_t QIN = NRS + (size_t)NBS * 16;                   // [kRows] f32
    static constexpr size_t QOUT = QIN + (size_t)kRows * 4;
    static constexpr size_t RCNT = QOUT + (size_t)kRows * 4;               // [kRows] u32
    static constexpr size_t NQMAX = RCNT + (size_t)kRows * 4;               // [4] f32
    static constexpr size_t QBOX = NQMAX + 16;                              // [4 blocks][kBoxBlocks][2] float4
    static constexpr size_t FARU = QBOX + (size_t)4 * kBoxBlocks * 2 * 16;  // [128] u32: far bits per chunk
    static constexpr size_t LLB = FARU + (size_t)128 * 4;                   // [2] u64: live-step ballots
    static constexpr size_t LIVE = LLB + 16;                                // [MAXST] u32, count at MAXST + 1
    static constexpr size_t PREF = LIVE + (size_t)(MAXST + 4) * 4;          // [kMaxRanges + 1] u32
    static constexpr size_t START = PREF + (size_t)(kMaxRanges + 1) * 4;    // [kMaxRanges] u32
    static constexpr size_t WORDS = (START + (size_t)kMaxRanges * 4 + 63) & ~(size_t)63;  // [WB][kRows][8] u64
    static constexpr size_t BYTES = WORDS + (size_t)WB * kRows * 8 * 8;
};

template <int NS, int QBW, bool PK>
__global__ __launch_bounds__(256, QBW == 1 ? 4 : 2) void k_refine_m16(RefineArgs a)
{
    using G = M16<NS, QBW>;
    constexpr int kStep = G::STEP, kGroupSteps = G::GS, kMaxSteps16 = G::MAXST;
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
    const uint32_t nrows = min((uint32_t)kRows, tl.nrows);
    const uint32_t row0 = tl.row0;
    const int nb = a.nb;

    extern __shared__ __align__(16) unsigned char smem16[];
    uint4 *const LX = (uint4 *)(smem16 + G::X);
    float *const LNXP = (float *)(smem16 + G::NXP);
    uint32_t *const LXI = (uint32_t *)(smem16 + G::XI);
    float4 *const LNRS = (float4 *)(smem16 + G::NRS);
    float *const LQIN = (float *)(smem16 + G::QIN);
    float *const LQOUT = (float *)(smem16 + G::QOUT);
    uint32_t *const LRCNT = (uint32_t *)(smem16 + G::RCNT);
    float *const LNQMAX = (float *)(smem16 + G::NQMAX);
    float4 *const LQBOX = (float4 *)(smem16 + G::QBOX);
    uint32_t *const LFARU = (uint32_t *)(smem16 + G::FARU);
    uint64_t *const LLB = (uint64_t *)(smem16 + G::LLB);
    uint32_t *const LLIVE = (uint32_t *)(smem16 + G::LIVE);
    uint32_t *const LPREF = (uint32_t *)(smem16 + G::PREF);
    uint32_t *const LSTART = (uint32_t *)(smem16 + G::START);
    uint64_t *const LWORDS = (uint64_t *)(smem16 + G::WORDS);

    const int tid = threadIdx.x;
    const uint64_t n = a.n;
    const float4 *__restrict__ xs = a.xs;
    const float4 *__restrict__ xq = a.xq;
    const uint64_t nqr = a.nqr;
    uint64_t *__restrict__ mask = a.mask;
    const uint32_t W = tl.words;
    const uint64_t mbase = a.toff[t] - a.wbase;
    const float s16 = a.s16;

    if (tid <= kMaxRanges) LPREF[tid] = tid <= (int)nr ? pref_g[tid] : 0xffffffffu;
    if (tid < kMaxRanges) LSTART[tid] = a.rstart[(uint64_t)A * kMaxRanges + tid];
    if (tid < G::NBS) {
        // -(r s) per block; r s is exact unless it underflows (then off by
        // less than 2^-149, far inside the absolute slack)
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tid < nb) v = scale4(a.tref ? a.tref[(uint64_t)t * nb + tid] : xq[(uint64_t)tid * nqr + row0], -s16);
        LNRS[tid] = v;
    }
    if (tid < kRows) LRCNT[tid] = 0;
    for (int e = tid; e < G::WB * kRows * 8; e += 256) LWORDS[e] = 0ull;
    // dimension blocks past nb are zero padding: staged as zeros once here
    // and never written again
    for (int e = tid; e < 2 * NS * 4 * kStep; e += 256) LX[e] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31, hi = lane >> 5;
    const int rh = wave % G::RW, cg = wave / G::RW;  // row group, candidate group
    const int rbase = rh * 32 * QBW;                 // first row of the wave's query blocks

    // ---- query blocks: fp16 halves in registers, norms, thresholds ----
    half8 ah[QBW][NS], al[QBW][NS];
    float qnorm[QBW];
#pragma unroll
    for (int i = 0; i < QBW; ++i) {
        const uint32_t r = (uint32_t)(rbase + i * 32 + col);
        const bool valid = r < nrows;
        float nq = 0.f;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            if (PK && sl == NS - 1) {
                // the last slab holds one dimension block (4 dimensions): its
                // three products share one instruction, k 0-3 h.h, 4-7 h.l,
                // 8-11 l.h (row operand: h, h | l, 0)
                const int b = sl * 4;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (valid) {
                    const float4 x = xq[(uint64_t)b * nqr + row0 + r];
                    const float4 nr4 = LNRS[b];
                    v = make_float4(fmaf(x.x, s16, nr4.x), fmaf(x.y, s16, nr4.y), fmaf(x.z, s16, nr4.z),
                                    fmaf(x.w, s16, nr4.w));
                }
                if (hi == 0) {  // the row's norm takes the block once
                    nq = fmaf(v.x, v.x, nq);
                    nq = fmaf(v.y, v.y, nq);
                    nq = fmaf(v.z, v.z, nq);
                    nq = fmaf(v.w, v.w, nq);
                }
                half4 hh, ll;
                split16(v, hh, ll);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    ah[i][sl][k] = hi == 0 ? hh[k] : ll[k];
                    ah[i][sl][4 + k] = hi == 0 ? hh[k] : (_Float16)0.0f;
                    al[i][sl][k] = (_Float16)0.0f;
                    al[i][sl][4 + k] = (_Float16)0.0f;
                }
                continue;
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int b = sl * 4 + hi * 2 + h2;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (valid && b < nb) {
                    const float4 x = xq[(uint64_t)b * nqr + row0 + r];
                    const float4 nr4 = LNRS[b];
                    v = make_float4(fmaf(x.x, s16, nr4.x), fmaf(x.y, s16, nr4.y), fmaf(x.z, s16, nr4.z),
                                    fmaf(x.w, s16, nr4.w));
                }
                nq = fmaf(v.x, v.x, nq);
                nq = fmaf(v.y, v.y, nq);
                nq = fmaf(v.z, v.z, nq);
                nq = fmaf(v.w, v.w, nq);
                half4 hh, ll;
                split16(v, hh, ll);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    ah[i][sl][h2 * 4 + k] = hh[k];
                    al[i][sl][h2 * 4 + k] = ll[k];
                }
            }
        }
        // the row's other half of the dimensions sits in lane ^ 32
        nq += __shfl_xor(nq, 32, 64);
        qnorm[i] = valid ? nq : -1.0f;
    }
    // thresholds of the rows (lanes 0-31 of the waves of column group 0)
    if (cg == 0 && hi == 0) {
#pragma unroll
        for (int i = 0; i < QBW; ++i) {
            const int r = rbase + i * 32 + col;
            const bool valid = qnorm[i] >= 0.f;
            LQIN[r] = valid ? a.tlo - a.kp * qnorm[i] - a.tabs : -INFINITY;
            LQOUT[r] = valid ? a.thi - a.km * qnorm[i] + a.tabs : -INFINITY;
            float m = valid ? qnorm[i] : 0.f;
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
            if (col == 0) LNQMAX[r >> 5] = m;
        }
    }

    // ---- block box test of every step, up front ----
    // Each wave writes its query blocks' boxes over the first kBoxBlocks
    // layout blocks (dimensions 0-7: the grid axes and the next
    // highest-variance ones) to LDS; then thread u tests the segment's
    // 64-candidate chunk u against all four query blocks of the tile (bit q of
    // LFARU[u]: block q holds no neighbour there, or no row), and the waves
    // read their step bits and the live steps back with ballots.
    {
        const uint32_t r = (uint32_t)(rbase + (QBW == 2 ? hi : 0) * 32 + col);
#pragma unroll
        for (int b = 0; b < kBoxBlocks; ++b) {
            float4 lo = make_float4(INFINITY, INFINITY, INFINITY, INFINITY);
            float4 up = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (r < nrows) {
                lo = b < nb ? xq[(uint64_t)b * nqr + row0 + r] : make_float4(0.f, 0.f, 0.f, 0.f);
                up = lo;
            }
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) {
                lo.x = fminf(lo.x, __shfl_xor(lo.x, o, 64));
                lo.y = fminf(lo.y, __shfl_xor(lo.y, o, 64));
                lo.z = fminf(lo.z, __shfl_xor(lo.z, o, 64));
                lo.w = fminf(lo.w, __shfl_xor(lo.w, o, 64));
                up.x = fmaxf(up.x, __shfl_xor(up.x, o, 64));
                up.y = fmaxf(up.y, __shfl_xor(up.y, o, 64));
                up.z = fmaxf(up.z, __shfl_xor(up.z, o, 64));
                up.w = fmaxf(up.w, __shfl_xor(up.w, o, 64));
            }
            // lane 0 (and lane 32 for a second block) holds its block's box
            if (col == 0 && (QBW == 2 || hi == 0)) {
                const int q = (rbase >> 5) + (QBW == 2 ? hi : 0);
                LQBOX[(q * kBoxBlocks + b) * 2] = lo;
                LQBOX[(q * kBoxBlocks + b) * 2 + 1] = up;
            }
        }
    }
    const uint32_t nsteps = (c_end - c_begin + kStep - 1) / kStep;  // <= kMaxSteps16
    const uint32_t nunits = nsteps * G::CG;                         // <= 128 chunks
    const float tbox = a.tbox;
    const bool tested = tbox < INFINITY;
    __syncthreads();
    uint32_t nskip = 0;  // comparisons the box test settles (<= 8192 per chunk)
    if ((uint32_t)tid < 128u) {
        const uint32_t u = (uint32_t)tid;
        const uint32_t gs = c_begin + u * 64;
        uint32_t fm = 0xfu;
        if (u < nunits && gs < c_end) {
            const uint32_t ncol = min(64u, c_end - gs);
            float4 blo[kBoxBlocks], bhi[kBoxBlocks];
            if (tested) {
                const float4 *cb = a.cbox + 2 * kBoxBlocks * (a.chunk_base[A] + (gs >> 6));
#pragma unroll
                for (int b = 0; b < kBoxBlocks; ++b) {
                    blo[b] = cb[2 * b];
                    bhi[b] = cb[2 * b + 1];
                }
            }
            fm = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t rb = (uint32_t)q * 32;
                const uint32_t qr = rb < nrows ? min(32u, nrows - rb) : 0u;
                bool far_q = qr == 0;
                if (!far_q && tested) {
                    float g2 = 0.f;
#pragma unroll
                    for (int b = 0; b < kBoxBlocks; ++b)
                        g2 = gap4(LQBOX[(q * kBoxBlocks + b) * 2], LQBOX[(q * kBoxBlocks + b) * 2 + 1], blo[b], bhi[b], g2);
                    if (g2 > tbox) {
                        far_q = true;
                        nskip += qr * ncol;
                    }
                }
                fm |= (uint32_t)far_q << q;
            }
        }
        LFARU[u] = fm;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) nskip += __shfl_xor(nskip, o, 64);
    }
    __syncthreads();
    // the wave's step bits: block i far at step st (lanes take steps w2 64 + lane)
    uint64_t far[QBW][G::FW];
#pragma unroll
    for (int i = 0; i < QBW; ++i) {
        const int q = (rbase >> 5) + i;
#pragma unroll
        for (int w2 = 0; w2 < G::FW; ++w2) {
            const uint32_t st = (uint32_t)(w2 * 64 + lane);
            const bool f = st >= nsteps || ((LFARU[st * G::CG + cg] >> q) & 1u);
            far[i][w2] = __ballot(f);
        }
    }
    // live steps: some block of some candidate group is not far
    if ((uint32_t)tid < 128u) {
        const uint32_t st = (uint32_t)tid;
        bool live = false;
        if (st < nsteps) {
            uint32_t all = 0xfu;
#pragma unroll
            for (int c = 0; c < G::CG; ++c) all &= LFARU[st * G::CG + c];
            live = all != 0xfu;
        }
        const uint64_t bl = __ballot(live);
        if (lane == 0) LLB[wave] = bl;
    }
    __syncthreads();
    if ((uint32_t)tid < 128u) {
        const uint32_t st = (uint32_t)tid;
        const uint64_t b0 = LLB[0], b1 = LLB[1];
        const uint64_t below = (1ull << lane) - 1ull;
        const uint64_t mine = wave == 0 ? b0 : b1;
        if ((mine >> lane) & 1ull) LLIVE[(wave == 0 ? 0u : (uint32_t)__popcll(b0)) + __popcll(mine & below)] = st;
        if (tid == 0) LLIVE[kMaxSteps16 + 1] = (uint32_t)(__popcll(b0) + __popcll(b1));
    }
    __syncthreads();
    const uint32_t nlive = __builtin_amdgcn_readfirstlane(LLIVE[kMaxSteps16 + 1]);
    const uint32_t ngroups = (nsteps + kGroupSteps - 1) / kGroupSteps;

    // ---- the norm test's bound per query block (see k_refine_mfma) ----
    float tn[QBW];
    {
        const float nt = 4.0f * (float)nb + 4.0f;
        const float g = nt * 0x1p-24f / (1.0f - nt * 0x1p-24f);
        const float c1 = 1.0f + g + 0x1p-18f, c2 = 1.0f + 2.0f * g + 0x1p-16f;
        const float st = sqrtf(a.thi) * c1;
#pragma unroll
        for (int i = 0; i < QBW; ++i) {
            const float sq = sqrtf(LNQMAX[(rbase >> 5) + i]) * c1;
            tn[i] = ((sq + st) * (sq + st)) * c2;
        }
    }
    const BandSink bsink{band_list(a.blist, a.lcap), band_counter(a.bcount), a.lcap, row0, mbase, W};

    // ---- loader: thread t stages candidate c = t % STEP, blocks h + TPC m ----
    const int lc = tid % kStep, lh = tid / kStep;
    uint32_t g_u = 0;  // range of the step's first position (wave-uniform, advances)
    const uint32_t idx0 = [&]() {
        const int g = range_of(LPREF, nr, c_begin);
        return LSTART[g] + (c_begin - LPREF[g]);
    }();
    auto cand_index = [&](uint32_t st) __attribute__((always_inline)) -> uint32_t {
        const uint32_t P = c_begin + st * kStep;
        while (P >= (uint32_t)__builtin_amdgcn_readfirstlane(LPREF[g_u + 1])) ++g_u;
        const uint32_t p = P + (uint32_t)lc;
        if (p >= c_end) return idx0;
        uint32_t g = g_u;
        const uint32_t nxt = __builtin_amdgcn_readfirstlane(LPREF[g_u + 1]);
        if (P + kStep > nxt) {
            while (p >= LPREF[g + 1]) ++g;
        }
        return LSTART[g] - LPREF[g] + p;
    };
    float4 ld[G::PER];
    uint32_t ldi = idx0;
    auto issue = [&](uint32_t st) __attribute__((always_inline)) {
        ldi = cand_index(st);
#pragma unroll
        for (int m = 0; m < G::PER; ++m) {
            const int b = lh + G::TPC * m;
            ld[m] = b < nb ? xs[(uint64_t)b * n + ldi] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto stage = [&](int buf) __attribute__((always_inline)) {
        float s2 = 0.f;
        unsigned char *xb = (unsigned char *)(LX + (size_t)buf * NS * 4 * kStep);
#pragma unroll
        for (int m = 0; m < G::PER; ++m) {
            const int b = lh + G::TPC * m;  // wave-uniform
            if (b >= nb) continue;
            const float4 nr4 = LNRS[b];
            const float4 x = ld[m];
            const float4 v = make_float4(fmaf(x.x, s16, nr4.x), fmaf(x.y, s16, nr4.y), fmaf(x.z, s16, nr4.z),
                                         fmaf(x.w, s16, nr4.w));
            s2 = fmaf(v.x, v.x, s2);
            s2 = fmaf(v.y, v.y, s2);
            s2 = fmaf(v.z, v.z, s2);
            s2 = fmaf(v.w, v.w, s2);
            half4 hh, ll;
            split16(v, hh, ll);
            // slab b / 4, [hi k 0-7, hi k 8-15, lo k 0-7, lo k 8-15][candidate], 8 bytes per block;
            // a packed last slab: [h, l | h, 0] in parts 0 and 1 (k 12-15 stay zero)
            const int sl = b >> 2, p = (b & 3) >> 1, o = (b & 1) * 8;
            if (PK && sl == NS - 1) {
                *(half4 *)(xb + ((size_t)(sl * 4) * kStep + lc) * 16) = hh;
                *(half4 *)(xb + ((size_t)(sl * 4) * kStep + lc) * 16 + 8) = ll;
                *(half4 *)(xb + ((size_t)(sl * 4 + 1) * kStep + lc) * 16) = hh;
            } else {
                *(half4 *)(xb + ((size_t)(sl * 4 + p) * kStep + lc) * 16 + o) = hh;
                *(half4 *)(xb + ((size_t)(sl * 4 + 2 + p) * kStep + lc) * 16 + o) = ll;
            }
        }
        LNXP[(buf * G::TPC + lh) * kStep + lc] = s2;
        if (lh == 0) LXI[buf * kStep + lc] = ldi;
    };

    floatx16 acc[QBW][2];
    auto mma = [&](int buf, const bool (&dq)[QBW]) __attribute__((always_inline)) {
        const uint4 *xb = LX + (size_t)buf * NS * 4 * kStep;
        const int c0 = cg * 64 + col;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            const half8 bh[2] = {*(const half8 *)&xb[(sl * 4 + hi) * kStep + c0],
                                 *(const half8 *)&xb[(sl * 4 + hi) * kStep + c0 + 32]};
            const half8 bl[2] = {*(const half8 *)&xb[(sl * 4 + 2 + hi) * kStep + c0],
                                 *(const half8 *)&xb[(sl * 4 + 2 + hi) * kStep + c0 + 32]};
            const floatx16 z = {};
            // three products, each accumulator touched every 2 QBW instructions
            // (one for a packed last slab)
#pragma unroll
            for (int i = 0; i < QBW; ++i) {
                if (!dq[i]) continue;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    acc[i][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i][sl], bh[tt], sl == 0 ? z : acc[i][tt],
                                                                        0, 0, 0);
            }
            if (PK && sl == NS - 1) continue;
#pragma unroll
            for (int i = 0; i < QBW; ++i) {
                if (!dq[i]) continue;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    acc[i][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i][sl], bl[tt], acc[i][tt], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < QBW; ++i) {
                if (!dq[i]) continue;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    acc[i][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i][sl], bh[tt], acc[i][tt], 0, 0, 0);
            }
        }
    };

    // Mask words of the current group collect in group buffer wsel; with two
    // buffers it alternates at each flush, so the next group's words never
    // land in the buffer other threads are still flushing (groups between
    // two live steps are zero and take no buffer).
    int wsel = 0;
    // classification of live step st (buffer buf) into the group buffer
    auto epilogue = [&](uint32_t st, int buf, const bool (&dq)[QBW]) __attribute__((always_inline)) {
        const uint32_t cw = c_begin + st * kStep + cg * 64;
        float xin[2], xout[2], nxt[2];
        uint32_t xid[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int cl = cg * 64 + 32 * tt + col;
            float nsum = LNXP[(buf * G::TPC) * kStep + cl];
#pragma unroll
            for (int k = 1; k < G::TPC; ++k) nsum += LNXP[(buf * G::TPC + k) * kStep + cl];
            nxt[tt] = nsum;
            xid[tt] = LXI[buf * kStep + cl];
            const bool valid = cw + 32 * tt + col < c_end;
            xin[tt] = valid ? a.kp * nxt[tt] : __builtin_nanf("");
            xout[tt] = valid ? a.km * nxt[tt] : __builtin_nanf("");
        }
        uint64_t *wg = LWORDS + (size_t)wsel * kRows * 8;
        const int wi = (int)(st % kGroupSteps) * G::CG + cg;
#pragma unroll
        for (int i = 0; i < QBW; ++i) {
            if (!dq[i]) continue;
            uint32_t live = 0;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                if (__ballot(!(nxt[tt] > tn[i])) != 0) live |= 1u << tt;
            if (live == 0) continue;
            const int qb = (rbase >> 5) + i;
            classify_block(acc[i], xin, xout, LQIN, LQOUT, qb, lane, cw, live, bsink,
                           [&](int tt) { return xid[tt]; }, wg + (qb * 32 + col) * 8 + wi);
        }
    };

    auto unit_flag = [&](int row, int j, uint32_t w, bool ok, bool nz) __attribute__((always_inline)) {
        const uint64_t b = __ballot(nz);
        if (ok && (j & 3) == 0) a.gflag[(mbase + (uint64_t)row * W + w) >> 2] = ((b >> (lane & ~3)) & 0xfull) ? 1 : 0;
    };
    auto flush = [&](uint32_t grp) __attribute__((always_inline)) {
        uint64_t *sw = LWORDS + (size_t)wsel * kRows * 8;
        for (int e = tid; e < kRows * 8; e += 256) {
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
    auto zero_groups = [&](uint32_t g0, uint32_t g1) __attribute__((always_inline)) {
        for (uint32_t g = g0; g < g1; ++g) {
            for (int e = tid; e < kRows * 8; e += 256) {
                const int row = e >> 3, j = e & 7;
                const uint32_t c0 = c_begin + g * kGroupCands + 64 * j;
                const uint32_t w = c0 >> 6;
                const bool ok = (uint32_t)row < nrows && w < W && c0 < c_end;
                if (ok) mask[mbase + (uint64_t)row * W + w] = 0ull;
                unit_flag(row, j, w, ok, false);
            }
        }
    };

    // groups before the first live step hold no neighbour
    const uint32_t first_step = nlive > 0 ? LLIVE[0] : nsteps;
    zero_groups(0, nlive > 0 ? first_step / kGroupSteps : ngroups);
    if (nlive > 0) {
        issue(first_step);
        stage(0);
    }
    __syncthreads();
    for (uint32_t bi = 0; bi < nlive; ++bi) {
        const int buf = (int)(bi & 1);
        const uint32_t st = __builtin_amdgcn_readfirstlane(LLIVE[bi]);
        const bool more = bi + 1 < nlive;
        const uint32_t st_next = more ? __builtin_amdgcn_readfirstlane(LLIVE[bi + 1]) : nsteps;
        if (more) issue(st_next);
        bool dq[QBW];
        bool any = false;
#pragma unroll
        for (int i = 0; i < QBW; ++i) {
            uint64_t fw = 0;
#pragma unroll
            for (int w2 = 0; w2 < G::FW; ++w2)
                if ((int)(st >> 6) == w2) fw = far[i][w2];
            dq[i] = !((fw >> (st & 63)) & 1ull);
            any |= dq[i];
        }
        if (any) {
            mma(buf, dq);
            epilogue(st, buf, dq);
        }
        if (more) stage(buf ^ 1);
        __syncthreads();
        // flush the group after its last live step
        const uint32_t g = st / kGroupSteps;
        const uint32_t gn = more ? st_next / kGroupSteps : ngroups;
        if (gn != g) {
            flush(g);
            zero_groups(g + 1, gn);
            if (G::WB == 1) __syncthreads();
            else wsel ^= 1;
        }
    }
    if (nskip != 0 && lane == 0)
        atomicAdd(&a.skipped[(uint64_t)(blockIdx.x % kHitSlots) * kBandStride], (unsigned long long)nskip);
    __syncthreads();
    for (int i = tid; i < (int)nrows; i += 256)
        if (LRCNT[i] != 0) atomicAdd(&a.rowcnt[row0 + i - a.row_base], LRCNT[i]);
}

// one query block per wave up to two slabs (four waves per SIMD), two from
// three slabs on (the query halves fill the registers anyway)
constexpr int qbw_of(int ns) { return ns <= 2 ? 1 : 2; }

// one block in the last slab (nb % 4 == 1): that slab's products packed
// into one instruction
const void *m16_kernel(int nb)
{
    const int ns = (nb + 3) / 4;
    const bool pk = nb % 4 == 1;
    switch (ns) {
    case 1: return pk ? (const void *)k_refine_m16<1, 1, true> : (const void *)k_refine_m16<1, 1, false>;
    case 2: return pk ? (const void *)k_refine_m16<2, 1, true> : (const void *)k_refine_m16<2, 1, false>;
    case 3: return pk ? (const void *)k_refine_m16<3, 2, true> : (const void *)k_refine_m16<3, 2, false>;
    case 4: return pk ? (const void *)k_refine_m16<4, 2, true> : (const void *)k_refine_m16<4, 2, false>;
    default: return nullptr;
    }
}

size_t m16_lds(int ns)
{
    switch (ns) {
    case 1: return M16<1, 1>::BYTES;
    case 2: return M16<2, 1>::BYTES;
    case 3: return M16<3, 2>::BYTES;
    case 4: return M16<4, 2>::BYTES;
    default: return 0;
    }
}

uint32_t m16_step(int ns) { return (uint32_t)(64 * qbw_of(ns)); }

}  // namespace

// The split form for up to 64 dimensions.
bool refine_m16_supported(int nb) { return nb >= 1 && nb <= 16; }

hipError_t prepare_refine_m16(int nb)
{
    const int ns = (nb + 3) / 4;
    const void *k = m16_kernel(nb);
    if (!k) return hipErrorInvalidValue;
    return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)m16_lds(ns));
}

hipError_t launch_refine_m16(const RefineArgs &a, hipStream_t s)
{
    const int ns = (a.nb + 3) / 4;
    const void *k = m16_kernel(a.nb);
    if (!k) return hipErrorInvalidValue;
    if (a.seg_len % kGroupCands != 0 || a.seg_len > 8192u || a.seg_len % m16_step(ns) != 0)
        return hipErrorInvalidValue;
    const uint64_t blocks = (uint64_t)a.ntiles * a.nseg;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    RefineArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), params, m16_lds(ns), s);
}

}  // namespace ersj
