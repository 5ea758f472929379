// Device helpers of the MFMA refinement kernel (k_refine_mfma.hip): operand
// types, the fp16 split, and the classification of a wave's 32 x 64 block of
// squared distances into result mask bits and band pairs.
//
// Method: "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
// Similarity Searches", Sec. IV-E (refinement of a group of queries against
// their shared candidates) and Sec. IV-F (one result bit per comparison).
#pragma once

#include "ersj_internal.h"

#include <utility>

namespace ersj {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kSlab = 4;          // dimension blocks (16 dims) per LDS slab
constexpr int kGroupCands = 512;  // candidates per mask-word flush
constexpr int kMaxSteps = 128;    // steps of a segment the block box test covers (8192 / 64)

__device__ __forceinline__ float4 sub4(float4 a, float4 b)
{
    return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}

__device__ __forceinline__ float4 scale4(float4 v, float s)
{
    return make_float4(v.x * s, v.y * s, v.z * s, v.w * s);
}

// Split of a (scaled) coordinate block into fp16 high and low parts:
// hi = fl16(v), lo = fl16(v - hi) (the difference is exact in fp32).
__device__ __forceinline__ void split16(float4 v, half4 &hi, half4 &lo)
{
    const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const _Float16 h = (_Float16)a[i];
        hi[i] = h;
        lo[i] = (_Float16)(a[i] - (float)h);
    }
}

// v_writelane_b32 through its LLVM intrinsic (clang has no builtin for it):
// writes a wave-uniform 32-bit value into one lane of a VGPR.  The compiler
// sees a real instruction and keeps the hazard wait states around it, which
// an asm statement would hide from it.
extern "C" __device__ int ersj_writelane(int val, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

template <int L>
__device__ __forceinline__ int write_lane(int old, uint32_t val)
{
    return ersj_writelane((int)val, L, old);
}

template <int... E, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, E...>, F &&f)
{
    (f(std::integral_constant<int, E>{}), ...);
}

// Where a work item's band pairs go, and how a mask bit is addressed.
struct BandSink {
    Boundary *blist;              // the workgroup's sub-list
    unsigned long long *bcount;   // its counter
    uint64_t bcap;                // entries per sub-list
    uint32_t row0;                // first query row of the work item (sorted order)
    uint64_t mbase;               // batch-relative first mask word of that row
    uint32_t W;                   // mask words per row of the tile
};

// Classification of a wave's 32 x 64 block: accumulator tt holds the dot
// products of the wave's 32 query rows with candidates 32 tt .. 32 tt + 31
// of the 64-candidate group starting at list position cw (register v of
// lane l: row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32).  With the row
// thresholds qin/qout (LDS, the work item's rows) and the lane's column
// terms xin = kp Nx, xout = km Nx (NaN: never classifies):
//   in   iff  fma(-2, D, xin)  <= qin[row]
//   out  iff  fma(-2, D, xout) >  qout[row]
// "In" pairs become mask bits: lane r < 32 of the wave gets row r's 64-bit
// word, stored to *wdst.  Pairs neither in nor out are appended to the band
// list for the binary64 re-check; xid(tt) gives the point index of the
// lane's column (called only for band pairs).  Only the 32-candidate halves
// tt with bit tt of live_tt set are classified (wave-uniform): the others
// are known to hold no neighbour and keep zero bits.
template <class XidFn>
__device__ __forceinline__ void classify_block(const floatx16 *acc, const float (&xin)[2], const float (&xout)[2],
                                               const float *qin, const float *qout, int qb, int lane,
                                               uint32_t cw, uint32_t live_tt, const BandSink &bs, XidFn &&xid,
                                               uint64_t *wdst)
{
    const int col = lane & 31, hi = lane >> 5;
    const float neg2 = -2.0f;
    int wlo = 0, whi = 0;
    uint64_t anyb = 0;
    // row thresholds come from LDS four rows at a time (rows
    // 8t + 4hi .. +3 of the query block for registers 4t .. 4t+3)
    const float4 *qin4 = (const float4 *)qin + qb * 8 + hi;
    const float4 *qout4 = (const float4 *)qout + qb * 8 + hi;
    float4 qi = make_float4(0.f, 0.f, 0.f, 0.f), qo = qi;
    // Groups of four registers (rows 8g .. 8g+3 and 8g+4 .. 8g+7 of a
    // tile).  "In" implies "not out" exactly (fl(kp*Nx) >= fl(km*Nx) and
    // qin <= qout under monotone rounding), so a group whose pairs are
    // all "out" - most of them - needs only the four "out" tests; its
    // mask half-words stay zero.
    static_for(std::make_integer_sequence<int, 8>{}, [&](auto E) {
        constexpr int g = decltype(E)::value / 2, tt = decltype(E)::value % 2;
        if (tt == 0) {
            qi = qin4[g * 2];
            qo = qout4[g * 2];
        }
        if (!(live_tt & (1u << tt))) return;
        uint64_t bno[4];
        uint64_t anyno = 0;
        static_for(std::make_integer_sequence<int, 4>{}, [&](auto J) {
            constexpr int j = decltype(J)::value;
            const float qov = j == 0 ? qo.x : j == 1 ? qo.y : j == 2 ? qo.z : qo.w;
            const float v2 = fmaf(neg2, acc[tt][4 * g + j], xout[tt]);
            bno[j] = __ballot(v2 <= qov);
            anyno |= bno[j];
        });
        if (anyno != 0) {
            static_for(std::make_integer_sequence<int, 4>{}, [&](auto J) {
                constexpr int j = decltype(J)::value;
                constexpr int i0 = 8 * g + j;
                const float qiv = j == 0 ? qi.x : j == 1 ? qi.y : j == 2 ? qi.z : qi.w;
                const float v1 = fmaf(neg2, acc[tt][4 * g + j], xin[tt]);
                const uint64_t bin = __ballot(v1 <= qiv);
                anyb |= bno[j] & ~bin;
                if (tt == 0) {
                    wlo = write_lane<i0>(wlo, (uint32_t)bin);
                    wlo = write_lane<i0 + 4>(wlo, (uint32_t)(bin >> 32));
                } else {
                    whi = write_lane<i0>(whi, (uint32_t)bin);
                    whi = write_lane<i0 + 4>(whi, (uint32_t)(bin >> 32));
                }
            });
        }
    });
    if (anyb != 0) {
        // rare: redo the classification for the band pairs and append
        // them for the binary64 re-check.  Rolled loops (indexed reads
        // of one accumulator vector, thresholds re-read from LDS) keep
        // this path from setting the kernel's register budget.
        const floatx16 a0 = acc[0], a1 = acc[1];
        auto band_tile = [&](const floatx16 &at, int tt) __attribute__((always_inline)) {
#pragma unroll 1
            for (int v = 0; v < 16; ++v) {
                const float dd = at[v];
                const int row = qb * 32 + (v >> 2) * 8 + (v & 3) + 4 * hi;
                const bool in = fmaf(neg2, dd, xin[tt]) <= qin[row];
                const bool nout = fmaf(neg2, dd, xout[tt]) <= qout[row];
                const bool bd = !in && nout;
                const uint64_t bbd = __ballot(bd);
                if (bbd == 0) continue;
                const uint32_t cnt = __popcll(bbd);
                const int first = __ffsll((unsigned long long)bbd) - 1;
                unsigned long long base = 0;
                if (lane == first) base = atomicAdd(bs.bcount, (unsigned long long)cnt);
                base = __shfl(base, first, 64);
                if (bd) {
                    const uint64_t below = lane == 0 ? 0ull : (bbd & (~0ull >> (64 - lane)));
                    const uint64_t idx = base + __popcll(below);
                    if (idx < bs.bcap) {
                        Boundary e;
                        e.q = bs.row0 + row;
                        e.x = xid(tt);
                        e.bit = (bs.mbase + (uint64_t)row * bs.W) * 64 + cw + 32 * tt + col;
                        bs.blist[idx] = e;
                    }
                }
            }
        };
        if (live_tt & 1u) band_tile(a0, 0);
        if (live_tt & 2u) band_tile(a1, 1);
    }
    if (lane < 32) *wdst = ((uint64_t)(uint32_t)whi << 32) | (uint64_t)(uint32_t)wlo;
}

}  // namespace ersj
