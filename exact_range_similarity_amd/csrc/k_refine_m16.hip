// Candidate refinement for gfx950, split-fp16 form on MFMA, for up to 64
// dimensions (one to four 16-dimension slabs).
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. IV-E (a thread block per group of queries that
// share their candidates, candidates staged through on-chip memory) and
// Sec. IV-F (one result bit per comparison).
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
//    of a cell) and a segment of the cell's candidate list, in steps of 128
//    candidates.  Wave w computes rows 64 (w % 2) .. +63 against candidates
//    64 (w / 2) .. +63 of each step: two 32-row query blocks times two
//    32-candidate halves, four 32 x 32 accumulators, 4096 pairs per step.
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

constexpr int kRows = 128;                      // query rows per work item (one tile)
constexpr int kStep = 128;                      // candidates per step
constexpr int kGroupSteps = kGroupCands / kStep;  // steps per 512-candidate mask-word group
constexpr int kMaxSteps16 = 8192 / kStep;       // steps of the longest segment

template <int NS>
struct M16 {
    static constexpr int NBS = 4 * NS;          // float4 blocks per candidate (padded)
    static constexpr int PER = NBS / 2;         // blocks staged per thread (two threads per candidate)
    static constexpr int WB = NS >= 4 ? 1 : 2;  // mask-word group buffers
    // LDS layout (bytes)
    static constexpr size_t X = 0;                                         // [2][NS][4][kStep] x 16 B
    static constexpr size_t NXP = X + (size_t)2 * NS * 4 * kStep * 16;      // [2][2][kStep] f32
    static constexpr size_t XI = NXP + (size_t)2 * 2 * kStep * 4;           // [2][kStep] u32
    static constexpr size_t NRS = XI + (size_t)2 * kStep * 4;               // [NBS] float4: -(r s)
    static constexpr size_t QIN = NRS + (size_t)NBS * 16;                   // [kRows] f32
    static constexpr size_t QOUT = QIN + (size_t)kRows * 4;
    static constexpr size_t RCNT = QOUT + (size_t)kRows * 4;               // [kRows] u32
    static constexpr size_t NQMAX = RCNT + (size_t)kRows * 4;               // [4] f32
    static constexpr size_t FAR = NQMAX + 16;                               // [4 waves] u64
    static constexpr size_t LIVE = FAR + 4 * 8;                             // [kMaxSteps16] u32 (+1)
    static constexpr size_t PREF = LIVE + (size_t)(kMaxSteps16 + 4) * 4;    // [kMaxRanges + 1] u32
    static constexpr size_t START = PREF + (size_t)(kMaxRanges + 1) * 4;    // [kMaxRanges] u32
    static constexpr size_t WORDS = (START + (size_t)kMaxRanges * 4 + 63) & ~(size_t)63;  // [WB][kRows][8] u64
    static constexpr size_t BYTES = WORDS + (size_t)WB * kRows * 8 * 8;
};

template <int NS>
__global__ __launch_bounds__(256, 2) void k_refine_m16(RefineArgs a)
{
    using G = M16<NS>;
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
    uint64_t *const LFAR = (uint64_t *)(smem16 + G::FAR);
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
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31, hi = lane >> 5;
    const int rh = wave & 1, cg = wave >> 1;  // row half, candidate group

    // ---- query blocks: fp16 halves in registers, norms, thresholds ----
    half8 ah[2][NS], al[2][NS];
    float qnorm[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t r = (uint32_t)(rh * 64 + i * 32 + col);
        const bool valid = r < nrows;
        float nq = 0.f;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
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
        for (int i = 0; i < 2; ++i) {
            const int r = rh * 64 + i * 32 + col;
            const bool valid = qnorm[i] >= 0.f;
            LQIN[r] = valid ? a.tlo - a.kp * qnorm[i] - a.tabs : -INFINITY;
            LQOUT[r] = valid ? a.thi - a.km * qnorm[i] + a.tabs : -INFINITY;
            float m = valid ? qnorm[i] : 0.f;
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
            if (col == 0) LNQMAX[rh * 2 + i] = m;
        }
    }

    // ---- block box test of every step, up front ----
    // the wave's two query blocks' boxes on the grid axes (lanes 0-31: block 0,
    // lanes 32-63: block 1), made wave-uniform
    float qlo[2][3], qhi[2][3];
    uint32_t qrows[2];
    {
        const uint32_t r = (uint32_t)(rh * 64 + hi * 32 + col);
        float4 lo = make_float4(INFINITY, INFINITY, INFINITY, 0.f), up = make_float4(-INFINITY, -INFINITY, -INFINITY, 0.f);
        if (r < nrows) {
            lo = xq[row0 + r];
            up = lo;
        }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            lo.x = fminf(lo.x, __shfl_xor(lo.x, o, 64));
            lo.y = fminf(lo.y, __shfl_xor(lo.y, o, 64));
            lo.z = fminf(lo.z, __shfl_xor(lo.z, o, 64));
            up.x = fmaxf(up.x, __shfl_xor(up.x, o, 64));
            up.y = fmaxf(up.y, __shfl_xor(up.y, o, 64));
            up.z = fmaxf(up.z, __shfl_xor(up.z, o, 64));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            qlo[i][0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lo.x), i * 32));
            qlo[i][1] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lo.y), i * 32));
            qlo[i][2] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lo.z), i * 32));
            qhi[i][0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(up.x), i * 32));
            qhi[i][1] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(up.y), i * 32));
            qhi[i][2] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(up.z), i * 32));
            const int rb = rh * 64 + i * 32;
            qrows[i] = (uint32_t)rb < nrows ? min(32u, nrows - (uint32_t)rb) : 0u;
        }
    }
    const uint32_t nsteps = (c_end - c_begin + kStep - 1) / kStep;  // <= kMaxSteps16
    const float tbox = a.tbox;
    const bool tested = tbox < INFINITY;
    // far0 / far1: steps in which query block 0 / 1 of this wave holds no
    // neighbour (box test) or no row; the wave skips a step when both are set
    uint64_t far0 = 0, far1 = 0;
    uint64_t nskip = 0;
    {
        const uint64_t cb0 = tested ? a.chunk_base[A] : 0;
        for (uint32_t st = 0; st < nsteps; ++st) {
            const uint32_t gs = c_begin + st * kStep + cg * 64;
            const uint64_t m = 1ull << st;
            if (gs >= c_end) {
                far0 |= m;
                far1 |= m;
                continue;
            }
            const uint32_t ncol = min(64u, c_end - gs);
            bool f0 = qrows[0] == 0, f1 = qrows[1] == 0;
            if (tested && !(f0 && f1)) {
                const float4 *cb = a.cbox + 2 * (cb0 + (gs >> 6));
                const float4 blo = cb[0], bhi = cb[1];
                if (!f0 && box_gap2(qlo[0], qhi[0], blo, bhi) > tbox) {
                    f0 = true;
                    nskip += (uint64_t)qrows[0] * ncol;
                }
                if (!f1 && box_gap2(qlo[1], qhi[1], blo, bhi) > tbox) {
                    f1 = true;
                    nskip += (uint64_t)qrows[1] * ncol;
                }
            }
            if (f0) far0 |= m;
            if (f1) far1 |= m;
        }
    }
    // far bits are wave-uniform (computed from uniform values); make it explicit
    far0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(far0 >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)far0);
    far1 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(far1 >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)far1);
    if (lane == 0) LFAR[wave] = far0 & far1;
    __syncthreads();
    if (tid == 0) {
        const uint64_t all = LFAR[0] & LFAR[1] & LFAR[2] & LFAR[3];
        uint32_t c = 0;
        for (uint32_t st = 0; st < nsteps; ++st)
            if (!((all >> st) & 1ull)) LLIVE[c++] = st;
        LLIVE[kMaxSteps16 + 1] = c;
    }
    __syncthreads();
    const uint32_t nlive = __builtin_amdgcn_readfirstlane(LLIVE[kMaxSteps16 + 1]);
    const uint32_t ngroups = (nsteps + kGroupSteps - 1) / kGroupSteps;

    // ---- the norm test's bound per query block (see k_refine_mfma) ----
    float tn[2];
    {
        const float nt = 4.0f * (float)nb + 4.0f;
        const float g = nt * 0x1p-24f / (1.0f - nt * 0x1p-24f);
        const float c1 = 1.0f + g + 0x1p-18f, c2 = 1.0f + 2.0f * g + 0x1p-16f;
        const float st = sqrtf(a.thi) * c1;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float sq = sqrtf(LNQMAX[rh * 2 + i]) * c1;
            tn[i] = ((sq + st) * (sq + st)) * c2;
        }
    }
    const BandSink bsink{band_list(a.blist, a.lcap), band_counter(a.bcount), a.lcap, row0, mbase, W};

    // ---- loader: thread t stages candidate c = t % 128, blocks h + 2 m ----
    const int lc = tid & (kStep - 1), lh = tid >> 7;
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
            const int b = lh + 2 * m;
            ld[m] = b < nb ? xs[(uint64_t)b * n + ldi] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto stage = [&](int buf) __attribute__((always_inline)) {
        float s2 = 0.f;
        unsigned char *xb = (unsigned char *)(LX + (size_t)buf * NS * 4 * kStep);
#pragma unroll
        for (int m = 0; m < G::PER; ++m) {
            const int b = lh + 2 * m;
            const float4 nr4 = LNRS[b];
            const float4 x = ld[m];
            float4 v = make_float4(fmaf(x.x, s16, nr4.x), fmaf(x.y, s16, nr4.y), fmaf(x.z, s16, nr4.z),
                                   fmaf(x.w, s16, nr4.w));
            if (b >= nb) v = make_float4(0.f, 0.f, 0.f, 0.f);
            s2 = fmaf(v.x, v.x, s2);
            s2 = fmaf(v.y, v.y, s2);
            s2 = fmaf(v.z, v.z, s2);
            s2 = fmaf(v.w, v.w, s2);
            half4 hh, ll;
            split16(v, hh, ll);
            // slab b / 4, [hi k 0-7, hi k 8-15, lo k 0-7, lo k 8-15][candidate], 8 bytes per block
            const int sl = b >> 2, p = (b & 3) >> 1, o = (b & 1) * 8;
            *(half4 *)(xb + ((size_t)(sl * 4 + p) * kStep + lc) * 16 + o) = hh;
            *(half4 *)(xb + ((size_t)(sl * 4 + 2 + p) * kStep + lc) * 16 + o) = ll;
        }
        LNXP[(buf * 2 + lh) * kStep + lc] = s2;
        if (lh == 0) LXI[buf * kStep + lc] = ldi;
    };

    floatx16 acc[2][2];
    auto mma = [&](int buf, bool do0, bool do1) __attribute__((always_inline)) {
        const uint4 *xb = LX + (size_t)buf * NS * 4 * kStep;
        const int c0 = cg * 64 + col;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            const half8 bh0 = *(const half8 *)&xb[(sl * 4 + hi) * kStep + c0];
            const half8 bh1 = *(const half8 *)&xb[(sl * 4 + hi) * kStep + c0 + 32];
            const half8 bl0 = *(const half8 *)&xb[(sl * 4 + 2 + hi) * kStep + c0];
            const half8 bl1 = *(const half8 *)&xb[(sl * 4 + 2 + hi) * kStep + c0 + 32];
            if (sl == 0) {
                const floatx16 z = {};
                if (do0) {
                    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][0], bh0, z, 0, 0, 0);
                    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][0], bh1, z, 0, 0, 0);
                }
                if (do1) {
                    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][0], bh0, z, 0, 0, 0);
                    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][0], bh1, z, 0, 0, 0);
                }
            } else {
                if (do0) {
                    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][sl], bh0, acc[0][0], 0, 0, 0);
                    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][sl], bh1, acc[0][1], 0, 0, 0);
                }
                if (do1) {
                    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][sl], bh0, acc[1][0], 0, 0, 0);
                    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][sl], bh1, acc[1][1], 0, 0, 0);
                }
            }
            if (do0) {
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][sl], bl0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0][sl], bl1, acc[0][1], 0, 0, 0);
            }
            if (do1) {
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][sl], bl0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1][sl], bl1, acc[1][1], 0, 0, 0);
            }
            if (do0) {
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[0][sl], bh0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[0][sl], bh1, acc[0][1], 0, 0, 0);
            }
            if (do1) {
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[1][sl], bh0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[1][sl], bh1, acc[1][1], 0, 0, 0);
            }
        }
    };

    // Mask words of the current group collect in group buffer wsel; with two
    // buffers it alternates at each flush, so the next group's words never
    // land in the buffer other threads are still flushing (groups between
    // two live steps are zero and take no buffer).
    int wsel = 0;
    // classification of live step st (buffer buf) into the group buffer
    auto epilogue = [&](uint32_t st, int buf, bool do0, bool do1) __attribute__((always_inline)) {
        const uint32_t cw = c_begin + st * kStep + cg * 64;
        float xin[2], xout[2], nxt[2];
        uint32_t xid[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int cl = cg * 64 + 32 * tt + col;
            nxt[tt] = LNXP[(buf * 2) * kStep + cl] + LNXP[(buf * 2 + 1) * kStep + cl];
            xid[tt] = LXI[buf * kStep + cl];
            const bool valid = cw + 32 * tt + col < c_end;
            xin[tt] = valid ? a.kp * nxt[tt] : __builtin_nanf("");
            xout[tt] = valid ? a.km * nxt[tt] : __builtin_nanf("");
        }
        uint64_t *wg = LWORDS + (size_t)wsel * kRows * 8;
        const int wi = (int)(st % kGroupSteps) * 2 + cg;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (!(i == 0 ? do0 : do1)) continue;
            uint32_t live = 0;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                if (__ballot(!(nxt[tt] > tn[i])) != 0) live |= 1u << tt;
            if (live == 0) continue;
            const int qb = rh * 2 + i;
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
        const bool do0 = !((far0 >> st) & 1ull), do1 = !((far1 >> st) & 1ull);
        if (do0 || do1) {
            mma(buf, do0, do1);
            epilogue(st, buf, do0, do1);
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

const void *m16_kernel(int ns)
{
    switch (ns) {
    case 1: return (const void *)k_refine_m16<1>;
    case 2: return (const void *)k_refine_m16<2>;
    case 3: return (const void *)k_refine_m16<3>;
    case 4: return (const void *)k_refine_m16<4>;
    default: return nullptr;
    }
}

size_t m16_lds(int ns)
{
    switch (ns) {
    case 1: return M16<1>::BYTES;
    case 2: return M16<2>::BYTES;
    case 3: return M16<3>::BYTES;
    case 4: return M16<4>::BYTES;
    default: return 0;
    }
}

}  // namespace

// Used for three and four slabs (33 to 64 dimensions).  With one or two
// slabs its two waves per SIMD (179 registers) hide load latency worse than
// k_refine_mfma's four, which is then faster (c2: 9.3 against 13.4 ms).
bool refine_m16_supported(int nb) { return nb > 8 && nb <= 16; }

hipError_t prepare_refine_m16(int nb)
{
    const int ns = (nb + 3) / 4;
    const void *k = m16_kernel(ns);
    if (!k) return hipErrorInvalidValue;
    return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)m16_lds(ns));
}

hipError_t launch_refine_m16(const RefineArgs &a, hipStream_t s)
{
    const int ns = (a.nb + 3) / 4;
    const void *k = m16_kernel(ns);
    if (!k) return hipErrorInvalidValue;
    if (a.seg_len % kStep != 0 || a.seg_len / kStep > (uint32_t)kMaxSteps16) return hipErrorInvalidValue;
    const uint64_t blocks = (uint64_t)a.ntiles * a.nseg;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    RefineArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), params, m16_lds(ns), s);
}

}  // namespace ersj
