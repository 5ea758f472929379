// C ABI of libersj (see include/ersj.h): argument validation, the state
// machine build -> count -> plan -> fill, device memory ownership, and the
// host-side choices (grid dimensions and widths, fp32 classification band).
#include "ersj.h"
#include "ersj_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

using namespace ersj;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

enum State { kNone = 0, kBuilt = 1, kCounted = 2, kPlanned = 3 };

class DeviceGuard {
public:
    explicit DeviceGuard(int dev) : ok_(false)
    {
        if (hipGetDevice(&prev_) == hipSuccess) ok_ = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard()
    {
        if (ok_) (void)hipSetDevice(prev_);
    }
    bool ok() const { return ok_; }

private:
    int prev_ = 0;
    bool ok_;
};

}  // namespace

struct ersj_index {
    int device = 0;
    int state = kNone;
    ersj_options opt{};
    int64_t n = 0;
    int32_t d = 0, nb = 0;
    double eps = 0.0, e64 = 0.0;
    float tlo = 0.0f, thi = 0.0f;
    float tbox = INFINITY;  // block box test threshold (inf: off)
    float kp = 1.0f, km = 1.0f;
    float kmf = 1.0f;  // the d > 64 filter's partial test
    float s16 = 1.0f, tlo16 = 0.0f, thi16 = 0.0f, tabs = 0.0f;  // split-fp16 form (scaled domain)
    double maxabs = 0.0;
    GridParams gp{};
    std::vector<int32_t> perm, pinv;

    std::map<void *, size_t> live;
    uint64_t bytes = 0;

    // index
    float4 *xs = nullptr;
    float *xr = nullptr;  // the same rows in sorted order, input dimension order, row-major
                          // (stride recheck_stride(d), zero-padded)
    uint32_t *orig = nullptr;
    int64_t M = 0;
    uint32_t *cell_start = nullptr;
    uint64_t *cell_key = nullptr;
    uint32_t *lo_bits = nullptr, *hi_bits = nullptr;
    // query rows: the points themselves for the self-join (these alias the
    // arrays above), a separate set binned into the same grid after
    // ersj_set_queries (the semi-join)
    bool semi = false;
    int64_t nq = 0;
    float4 *xq = nullptr;
    float *xqr = nullptr;
    uint32_t *qorig = nullptr;
    int64_t Mq = 0;
    uint32_t *qcell_start = nullptr;
    uint64_t *qcell_key = nullptr;
    uint32_t *qlo_bits = nullptr, *qhi_bits = nullptr;
    double maxabs_q = 0.0;
    // count pass
    uint32_t *rstart = nullptr, *rpref = nullptr, *nrng = nullptr;
    uint32_t umax = 0;
    int64_t T = 0;
    Tile *tiles = nullptr;
    uint64_t *toff = nullptr, *coff = nullptr;
    uint64_t total_cand = 0, total_words = 0;
    float4 *cbox = nullptr;           // block box test: box of each 64-candidate chunk of each cell's list
    uint64_t *chunk_base = nullptr;   // first chunk of each cell
    // plan
    int32_t nbatch = 0;
    std::vector<uint32_t> hb;
    std::vector<uint64_t> hrows, hwords, hcands;
    uint64_t maxw = 0, maxrows = 0;
    uint32_t *order = nullptr;
    // fill
    uint64_t *mask = nullptr;
    uint8_t *gflag = nullptr;  // per 4 mask words (256 candidates): any bit set
    uint64_t mask_cap = 0;
    Boundary *blist = nullptr;
    uint64_t bcap = 0;
    uint4 *dlist = nullptr;  // blocks the d > 64 filter hands on (kBandLists sub-lists)
    uint64_t dcap = 0;       // entries per sub-list
    unsigned long long *counters = nullptr;  // band sub-list counters, then re-check hits
    uint64_t *lpref = nullptr;               // [kBandLists + 1] prefix, [2] kept / max count
    uint32_t *rowcnt = nullptr;
    uint64_t *roff = nullptr, *rscan = nullptr;
    uint64_t rows_cap = 0;
    int32_t ready_batch = -1;
    uint64_t ready_pairs = 0;
    // stats
    uint64_t last_cand = 0, last_pairs = 0, last_bnd = 0, last_in = 0, last_skip = 0, last_part = 0;
    bool last_filtered = false;  // the last batch went through the filter and the block kernel
    double ms_build = 0, ms_count = 0, ms_plan = 0, ms_refine = 0, ms_recheck = 0, ms_expand = 0;
    int64_t refine_launches = 0;
    uint64_t refined_cand = 0, skipped_cand = 0, partial_cand = 0;
    hipEvent_t ev[2] = {nullptr, nullptr};
    int32_t kernel_used = ERSJ_REFINE_DIRECT;
    bool box_order = false;  // rows of a cell in Morton order over its 8-dimension box
    bool tree_order = false;  // rows of a cell as the leaves of a balanced tree
    bool use_m16 = false;  // split-fp16 form on the whole-tile kernel (33 <= d <= 64)
    bool use_g16 = false;  // split-fp16 form on operands prepared per point (d > 64)
    bool g16_hh = false;   // ... with the high-half products alone
    bool g16_tiled = false;  // a batch overflowed the hand-on list: the tiled kernel alone from then on
    std::vector<double> mean;  // per input dimension (binary64 statistics of the points)
    float4 *tref = nullptr;  // per row tile: reference point of the MFMA kernels' centring
    uint4 *p16 = nullptr, *p16q = nullptr;  // prepared operands of points and query rows
    uint64_t ps16 = 0, ps16q = 0;           // their part strides
    float *n16 = nullptr, *n16q = nullptr;
    float *np16 = nullptr, *np16q = nullptr;  // their norms over the first kPartialDims dimensions
    float *xb16 = nullptr;  // the filter's column bound of each point (n + 1)
    // the filter's int8 form (null: the fp16 form): operands of points and
    // query rows, part strides, column bounds (n + 1) and row starts
    uint4 *p8 = nullptr, *p8q = nullptr;
    uint64_t ps8 = 0, ps8q = 0;
    int *xb8 = nullptr, *qs8 = nullptr;
    // host delivery: two device staging buffers, alternated by batch, drained
    // into the caller's host memory on a copy stream of its own
    hipStream_t copy_stream = nullptr;
    uint32_t *stage[2] = {nullptr, nullptr};
    uint64_t stage_cap[2] = {0, 0};
    hipEvent_t expanded[2] = {nullptr, nullptr}, copied[2] = {nullptr, nullptr};
    bool copy_pending[2] = {false, false};
    double ms_deliver = 0;  // host time waiting in ersj_host_sync
};

namespace {

int hip_fail(hipError_t e, const char *what)
{
    (void)hipGetLastError();
    if (e == hipErrorOutOfMemory) return fail(ERSJ_ERR_OOM, "%s: %s", what, hipGetErrorString(e));
    return fail(ERSJ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPC(expr, what)                                  \
    do {                                                  \
        hipError_t e__ = (expr);                          \
        if (e__ != hipSuccess) return hip_fail(e__, what); \
    } while (0)

#define TRY(expr)                  \
    do {                           \
        int r__ = (expr);          \
        if (r__ != ERSJ_OK) return r__; \
    } while (0)

// Device memory pool, per device, shared by all handles of the process.
// Released blocks are kept and handed out again for a request of the same
// rounded size, which spares a repeated join the hipMalloc and the
// device-synchronising hipFree of every buffer.  A released block may still
// be in use by work enqueued before its release, so it is reused only after a
// device-wide synchronisation (the guarantee hipFree gave).  When hipMalloc
// fails the pool frees what it holds and tries again; it keeps at most half
// of the device's memory.
struct PoolBlock {
    void *p;
    size_t bytes;
    bool ready;  // released before the last device synchronisation
};
struct DevicePool {
    std::vector<PoolBlock> blocks;
    size_t cached = 0, cap = 0;
};
std::mutex g_pool_mu;
std::map<int, DevicePool> g_pools;

size_t pool_round(size_t b)
{
    const size_t big = (size_t)2 << 20;
    return b <= ((size_t)1 << 20) ? (b + 255) & ~(size_t)255 : (b + big - 1) & ~(big - 1);
}

DevicePool &pool_of(int dev)
{
    DevicePool &pl = g_pools[dev];
    if (pl.cap == 0) {
        size_t fr = 0, tot = 0;
        pl.cap = hipMemGetInfo(&fr, &tot) == hipSuccess ? tot / 2 : ((size_t)1 << 30);
        (void)hipGetLastError();
    }
    return pl;
}

hipError_t pool_get(int dev, size_t bytes, void **out)
{
    {
        std::lock_guard<std::mutex> lk(g_pool_mu);
        DevicePool &pl = pool_of(dev);
        for (int pass = 0; pass < 2; ++pass) {
            for (size_t i = 0; i < pl.blocks.size(); ++i) {
                if (pl.blocks[i].bytes == bytes && pl.blocks[i].ready) {
                    *out = pl.blocks[i].p;
                    pl.cached -= bytes;
                    pl.blocks.erase(pl.blocks.begin() + (long)i);
                    return hipSuccess;
                }
            }
            bool pending = false;
            for (const PoolBlock &b : pl.blocks) pending |= b.bytes == bytes && !b.ready;
            if (!pending) break;
            // a block of this size awaits the work enqueued before its release
            if (hipDeviceSynchronize() != hipSuccess) break;
            for (PoolBlock &b : pl.blocks) b.ready = true;
        }
    }
    hipError_t e = hipMalloc(out, bytes);
    if (e == hipSuccess) return e;
    (void)hipGetLastError();
    {
        std::lock_guard<std::mutex> lk(g_pool_mu);
        DevicePool &pl = pool_of(dev);
        if (pl.blocks.empty()) return e;
        (void)hipDeviceSynchronize();
        for (const PoolBlock &b : pl.blocks) (void)hipFree(b.p);
        pl.blocks.clear();
        pl.cached = 0;
    }
    return hipMalloc(out, bytes);
}

void pool_put(int dev, void *p, size_t bytes)
{
    std::lock_guard<std::mutex> lk(g_pool_mu);
    DevicePool &pl = pool_of(dev);
    if (pl.cached + bytes > pl.cap) {
        (void)hipFree(p);
        return;
    }
    pl.blocks.push_back(PoolBlock{p, bytes, false});
    pl.cached += bytes;
}

// bytes the pool holds for the device (free for this library's reuse)
size_t pool_cached(int dev)
{
    std::lock_guard<std::mutex> lk(g_pool_mu);
    return pool_of(dev).cached;
}

template <typename T>
int dalloc(ersj_index *h, T **p, size_t count, const char *what)
{
    size_t bytes = count * sizeof(T);
    if (bytes == 0) bytes = 8;
    bytes = pool_round(bytes);
    if (h->opt.max_device_bytes && h->bytes + bytes > h->opt.max_device_bytes)
        return fail(ERSJ_ERR_OOM, "%s: %zu bytes would exceed max_device_bytes (%llu in use, cap %llu)",
                    what, bytes, (unsigned long long)h->bytes,
                    (unsigned long long)h->opt.max_device_bytes);
    void *q = nullptr;
    hipError_t e = pool_get(h->device, bytes, &q);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ERSJ_ERR_OOM, "%s: hipMalloc(%zu) failed: %s", what, bytes, hipGetErrorString(e));
    }
    h->live[q] = bytes;
    h->bytes += bytes;
    *p = (T *)q;
    return ERSJ_OK;
}

template <typename T>
void dfree(ersj_index *h, T *&p)
{
    if (!p) return;
    auto it = h->live.find((void *)p);
    if (it != h->live.end()) {
        h->bytes -= it->second;
        pool_put(h->device, (void *)p, it->second);
        h->live.erase(it);
    } else {
        (void)hipFree((void *)p);
    }
    p = nullptr;
}

// Temporaries of one call, released on every exit path.
struct Scratch {
    ersj_index *h;
    std::vector<void **> ptrs;
    explicit Scratch(ersj_index *hh) : h(hh) {}
    template <typename T>
    int get(T **p, size_t count, const char *what)
    {
        *p = nullptr;
        int r = dalloc(h, p, count, what);
        if (r == ERSJ_OK) ptrs.push_back((void **)p);
        return r;
    }
    ~Scratch()
    {
        for (void **p : ptrs) dfree(h, *p);
    }
};

double gamma_n(double n, double u) { return n * u / (1.0 - n * u); }

float round_down_f32(double v)
{
    if (v >= (double)FLT_MAX) return FLT_MAX;
    float f = (float)v;
    if ((double)f > v) f = std::nextafter(f, -INFINITY);
    return f;
}

float round_up_f32(double v)
{
    if (v > (double)FLT_MAX) return INFINITY;
    float f = (float)v;
    if ((double)f < v) f = std::nextafter(f, INFINITY);
    return f;
}

// fp32 thresholds.  For an fp32 squared distance s computed in any order
// (d_pad terms, each a rounded difference squared and accumulated with one
// rounding per step) |s - S| <= g32 * S, and the binary64 reference obeys
// |D64 - S| <= g64 * S, where S is the exact squared distance.  Hence
// s <= E(1 - 2(g32 + g64)) implies D64 <= E and s > E(1 + 2(g32 + g64))
// implies D64 > E (the factor 2 leaves room for the rounding of the
// thresholds themselves).  Below 2^-90 fp32 underflow breaks the relative
// bound on the "in" side, so nothing is accepted without the re-check there.
void thresholds(ersj_index *h)
{
    const double E = h->e64;
    if (std::isinf(E)) {
        h->tlo = INFINITY;
        h->thi = INFINITY;
        return;
    }
    const int dpad = h->nb * 4;
    const double g32 = gamma_n(dpad + 2, std::ldexp(1.0, -24));
    const double g64 = gamma_n(h->d + 2, std::ldexp(1.0, -53));
    const double delta = 2.0 * (g32 + g64);
    h->thi = std::max(round_up_f32(E * (1.0 + delta)), (float)std::ldexp(1.0, -80));
    if (E < std::ldexp(1.0, -90)) h->tlo = -1.0f;
    else h->tlo = round_down_f32(E * (1.0 - delta));
    // Block box test: the fp32 sum of three squared box gaps (gaps rounded
    // once, then up to three more roundings) is at most (1 + u)^5 times the
    // exact sum, which bounds the squared distance of every pair in the two
    // boxes from below; D64 is within gamma(d + 1) of the exact distance.
    // Above E (1 + 2^-20) the whole block is therefore out.
    h->tbox = h->opt.block_prune < 0 ? INFINITY : round_up_f32(E * (1.0 + std::ldexp(1.0, -20)) + std::ldexp(1.0, -140));
}

// MFMA refinement: dot products of tile-centred coordinates.  Usable when
// the centred values cannot overflow fp32 (|x'| <= 2 max|x| per coordinate,
// norms and dots <= 4 d_pad max|x|^2, kept below FLT_MAX / 16) and the
// query tile fits the LDS.  Band: K = 4 (d_pad + 8) u, twice the
// 2.02 gamma(d_pad + 2) + 6.1 u that the error analysis needs.
bool coords_feasible(const ersj_index *h, const char **why)
{
    const double dp = 4.0 * h->nb;
    const double m = std::max(h->maxabs, h->maxabs_q);  // points and query rows
    if (16.0 * dp * m * m >= 1e38) {
        *why = "coordinates too large for fp32 norms";
        return false;
    }
    return true;
}

bool mfma_feasible(const ersj_index *h, const char **why)
{
    if (refine_mfma_lds_bytes(h->nb) > 160 * 1024) {
        *why = "query tile exceeds the 160 KiB LDS (d too large)";
        return false;
    }
    return coords_feasible(h, why);
}

// Split-fp16 MFMA form, classified in a scaled domain.  Centred coordinates
// v (|v| <= M = 2 max|x|) are multiplied by s = 2^(14 - ceil(log2 M)), exact
// in fp32 (|v s| <= 2^15 < 65504), and split into hi = fl16(v s) and
// lo = fl16(v s - hi): v s = hi + lo + e, |e| <= 2^-22 |v s| + 2^-25 (the
// 2^-25 covers subnormal parts).  Then s^2 q'x' = hi.hi + hi.lo + lo.hi + r
// with |r| <= 3 * 2^-22 |s^2 q'x'| plus absolute terms below
// 2^-25 (|q's| + |x's|) * 1.01 per dimension.  The fp16 products are exact in
// fp32 (11-bit significands, exponents well inside fp32's range); each
// k = 16 MFMA sums 16 products and the accumulator, 17 terms, with at most
// 16 additions on any term's path whatever order the hardware takes.  Taking
// each addition only to be faithful (error below one ulp of its result, 2u
// relative), a term's relative error is below (1 + 2u)^16 - 1 < 32.1u, so an
// instruction errs by less than 32.1u (sum |ab| + |c|), and |c| is at most
// the sum of the earlier |ab| (to first order).  The band charges 36u for
// each of the 3 ceil(d_pad / 16) instructions of a tile, on top of the fp32
// kernel's K (a probe of v_mfma_f32_32x32x16_f16 measured at most 22.3u).  With
// sum |q'_k x'_k| <= (Nq + Nx) / 2 the relative part fits the
// norm-proportional band.  Norms come from the scaled coordinates and the
// thresholds are those of fl(eps^2) s^2 (s^2 a power of two, so the rounding
// analysis of the fp32 thresholds carries over); the absolute part, at most
// 2^-24 d_pad M s 1.02 in s^2 D, is charged twice over as tabs on both
// thresholds.  Admitted while s is a normal fp32 power of two.
bool mfma16_setup(ersj_index *h)
{
    const double M = 2.0 * std::max(h->maxabs, h->maxabs_q);
    int e = 14;
    if (M > 0.0) {
        int ex = 0;
        std::frexp(M, &ex);  // M < 2^ex
        e = 14 - ex;
    }
    if (e < -120 || e > 120) return false;
    const double s = std::ldexp(1.0, e);
    const double dpad = 4.0 * h->nb;
    const int nslab = (h->nb + 3) / 4;
    const double u = std::ldexp(1.0, -24);
    const double K = 4.0 * (dpad + 8.0) * u + 3.0 * std::ldexp(1.0, -22) + 36.0 * u * 3.0 * nslab * 1.01;
    h->kp = (float)(1.0 + K);
    h->km = (float)(1.0 - K);
    h->s16 = (float)s;
    h->tabs = round_up_f32(4.0 * u * dpad * (M * s) * 1.02);
    // thresholds of fl(eps^2) s^2, by the same rules as the fp32 ones
    const double E = h->e64 * s * s;
    if (std::isinf(E)) {
        h->tlo16 = h->tlo == INFINITY ? INFINITY : FLT_MAX;
        h->thi16 = INFINITY;
    } else {
        const double g32 = gamma_n(dpad + 2, u);
        const double g64 = gamma_n(h->d + 2, std::ldexp(1.0, -53));
        const double delta = 2.0 * (g32 + g64);
        h->thi16 = std::max(round_up_f32(E * (1.0 + delta)), (float)std::ldexp(1.0, -80));
        h->tlo16 = E < std::ldexp(1.0, -90) ? -1.0f : round_down_f32(E * (1.0 - delta));
    }
    return true;
}

int choose_kernel(ersj_index *h)
{
    const char *why = "";
    const bool ok = mfma_feasible(h, &why);
    // above 64 dimensions the split form runs on prepared operands, whose
    // LDS use does not grow with d: only the coordinate range limits it
    const char *why16 = "";
    const bool ok16 = h->nb > 16 ? coords_feasible(h, &why16) : ok;
    if (h->nb <= 16) why16 = why;
    int k = h->opt.refine_kernel;
    if (k == ERSJ_REFINE_MFMA && !ok)
        return fail(ERSJ_ERR_INVALID_ARG, "MFMA refinement not usable for this input: %s", why);
    if (k == ERSJ_REFINE_MFMA16 && !ok16)
        return fail(ERSJ_ERR_INVALID_ARG, "MFMA refinement not usable for this input: %s", why16);
    if (k == ERSJ_REFINE_AUTO) {
        // the split-fp16 form where its scale fits, else fp32 MFMA, else direct
        k = ok16 && mfma16_setup(h) ? ERSJ_REFINE_MFMA16 : ok ? ERSJ_REFINE_MFMA : ERSJ_REFINE_DIRECT;
    } else if (k == ERSJ_REFINE_MFMA16 && !mfma16_setup(h)) {
        return fail(ERSJ_ERR_INVALID_ARG, "split-fp16 refinement not usable: coordinate scale out of range");
    }
    h->kernel_used = k;
    if (k == ERSJ_REFINE_MFMA) {
        const double K = 4.0 * (4.0 * h->nb + 8.0) * std::ldexp(1.0, -24);
        h->kp = (float)(1.0 + K);
        h->km = (float)(1.0 - K);
        HIPC(prepare_refine_mfma(h->nb, false), "MFMA kernel LDS attribute");
    }
    h->use_m16 = k == ERSJ_REFINE_MFMA16 && refine_m16_supported(h->nb);
    h->use_g16 = k == ERSJ_REFINE_MFMA16 && h->nb > 16;
    h->g16_hh = h->use_g16 && h->opt.mfma_products != 3;
    if (h->use_g16) {
        // High-half products alone (k_refine_g16.hip): the dropped products
        // move s^2 q'.x' by at most 2^-10 (1 + 2^-12) sum |v_q v_x| (in the
        // squared distance at most twice that, <= 2^-10 (1 + 2^-12) (Nq + Nx))
        // plus absolute parts within tabs; one MFMA per slab (padded to an
        // even count) at 36u each, and the fp32 form's 4 (d_pad + 8) u.  The
        // filter's partial test forms high-half products alone with either
        // product count, so it always takes this coefficient (over its 64
        // dimensions it is larger than needed).
        const double u = std::ldexp(1.0, -24);
        const double K = 4.0 * (4.0 * h->nb + 8.0) * u + std::ldexp(1.0 + std::ldexp(1.0, -12), -10) +
                         36.0 * u * 2.0 * g16_stages(h->nb, true) * 1.01;
        h->kmf = (float)(1.0 - K);
        if (h->g16_hh) {
            h->kp = (float)(1.0 + K);
            h->km = (float)(1.0 - K);
        }
    }
    if (h->use_m16) HIPC(prepare_refine_m16(h->nb), "MFMA kernel LDS attribute");
    else if (h->use_g16) {
        HIPC(prepare_refine_g16(h->g16_hh), "MFMA kernel LDS attribute");
        HIPC(prepare_filter16(), "MFMA kernel LDS attribute");
    }
    else if (k == ERSJ_REFINE_MFMA16) HIPC(prepare_refine_mfma(h->nb, true), "MFMA kernel LDS attribute");
    return ERSJ_OK;
}

int sync(hipStream_t s, const char *what)
{
    HIPC(hipStreamSynchronize(s), what);
    return ERSJ_OK;
}

void timer_start(ersj_index *h, hipStream_t s)
{
    if (h->opt.timing) (void)hipEventRecord(h->ev[0], s);
}

double timer_stop(ersj_index *h, hipStream_t s)
{
    if (!h->opt.timing) return 0.0;
    float ms = 0.0f;
    (void)hipEventRecord(h->ev[1], s);
    (void)hipEventSynchronize(h->ev[1]);
    (void)hipEventElapsedTime(&ms, h->ev[0], h->ev[1]);
    return ms;
}

int ceil_log2(uint64_t v)
{
    int b = 0;
    while ((1ull << b) < v) ++b;
    return b;
}

void release_prepared(ersj_index *h)
{
    if (h->p16q != h->p16) dfree(h, h->p16q);
    if (h->n16q != h->n16) dfree(h, h->n16q);
    if (h->np16q != h->np16) dfree(h, h->np16q);
    h->np16q = nullptr;
    dfree(h, h->np16);
    dfree(h, h->xb16);
    h->p16q = nullptr;
    h->n16q = nullptr;
    dfree(h, h->p16);
    dfree(h, h->n16);
    if (h->p8q != h->p8) dfree(h, h->p8q);
    h->p8q = nullptr;
    dfree(h, h->p8);
    dfree(h, h->xb8);
    dfree(h, h->qs8);
}

void release_count(ersj_index *h)
{
    release_prepared(h);
    dfree(h, h->tref);
    dfree(h, h->rstart);
    dfree(h, h->rpref);
    dfree(h, h->nrng);
    dfree(h, h->tiles);
    dfree(h, h->toff);
    dfree(h, h->coff);
    dfree(h, h->cbox);
    dfree(h, h->chunk_base);
}

void release_plan(ersj_index *h)
{
    dfree(h, h->order);
    h->hb.clear();
    h->hrows.clear();
    h->hwords.clear();
    h->hcands.clear();
    h->nbatch = 0;
    h->ready_batch = -1;
}

// Rows binned into the grid (A4-A7): Morton keys of their cells (clamped as
// points or as queries), stable radix sort, runs of equal keys = cells, the
// rows of each cell put in their order (cell_order), gather into the
// dimension-blocked variance-ordered layout, and the cells' boxes on the grid
// axes.
struct Binned {
    float4 *xs = nullptr;
    float *xr = nullptr;
    uint32_t *orig = nullptr;
    int64_t M = 0;
    uint32_t *cell_start = nullptr;
    uint64_t *cell_key = nullptr;
    uint32_t *lo_bits = nullptr, *hi_bits = nullptr;
};

int bin_rows(ersj_index *h, const float *x, int64_t n, int64_t ld, bool queries, Binned *out, hipStream_t s)
{
    const int32_t d = h->d;
    Scratch tmp(h);
    uint64_t *k0 = nullptr, *k1 = nullptr, *hist = nullptr, *stmp = nullptr;
    uint32_t *v1 = nullptr;
    TRY(tmp.get(&k0, (size_t)n, "keys"));
    TRY(tmp.get(&k1, (size_t)n, "keys"));
    TRY(tmp.get(&v1, (size_t)n, "keys"));
    const size_t hent = radix_hist_entries(n);
    TRY(tmp.get(&hist, hent, "sort"));
    TRY(tmp.get(&stmp, std::max(scan_tmp_entries(hent), scan_tmp_entries(n + 1)), "scan"));
    TRY(dalloc(h, &out->orig, (size_t)n, "orig"));
    HIPC(launch_keys(x, n, ld, h->gp, queries, k0, out->orig, s), "keys kernel");
    HIPC(radix_sort(k0, out->orig, k1, v1, n, 3 * (h->gp.bits + h->gp.sub), hist, stmp, s), "radix sort");

    int32_t *dperm = nullptr;
    TRY(tmp.get(&dperm, (size_t)d, "perm"));
    HIPC(hipMemcpyAsync(dperm, h->perm.data(), sizeof(int32_t) * d, hipMemcpyHostToDevice, s), "perm copy");

    uint32_t *flags = nullptr;
    uint64_t *cid = nullptr;
    TRY(tmp.get(&flags, (size_t)n, "cells"));
    TRY(tmp.get(&cid, (size_t)n + 1, "cells"));
    HIPC(launch_cell_flags(k0, n, 3 * h->gp.sub, flags, s), "cell flags");
    HIPC(scan_u32(flags, cid, n, stmp, s), "cell scan");
    uint64_t M = 0;
    HIPC(hipMemcpyAsync(&M, cid + n, sizeof M, hipMemcpyDeviceToHost, s), "cell count copy");
    TRY(sync(s, "cells"));
    out->M = (int64_t)M;
    TRY(dalloc(h, &out->cell_start, (size_t)M + 1, "cells"));
    TRY(dalloc(h, &out->cell_key, (size_t)M, "cells"));
    TRY(dalloc(h, &out->lo_bits, (size_t)M * 3, "cells"));
    TRY(dalloc(h, &out->hi_bits, (size_t)M * 3, "cells"));
    HIPC(launch_cell_scatter(k0, 3 * h->gp.sub, flags, cid, n, out->cell_start, out->cell_key, s), "cell scatter");
    TRY(dalloc(h, &out->xs, (size_t)h->nb * n, "points"));
    if (h->box_order) {
        // rows gathered in cell order (up to 64 dimensions all of them,
        // above only the first kOrderDims), each cell's rows re-sorted by
        // their code in the cell's box (midpoint splits of the widest
        // extent), then moved (or, above 64 dimensions, gathered again) into
        // that order
        const bool wide = d > 64;
        const int nbw = wide ? std::min(h->nb, kOrderDims / 4) : h->nb;
        float4 *xs1 = nullptr;
        uint32_t *blo = nullptr, *bhi = nullptr, *bmask = nullptr, *orig1 = nullptr, *pos = nullptr;
        TRY(tmp.get(&xs1, (size_t)nbw * n, "cell order"));
        TRY(tmp.get(&blo, (size_t)M * kOrderDims, "cell order"));
        TRY(tmp.get(&bhi, (size_t)M * kOrderDims, "cell order"));
        TRY(tmp.get(&bmask, (size_t)M * kOrderDims, "cell order"));
        TRY(tmp.get(&orig1, (size_t)n, "cell order"));
        TRY(tmp.get(&pos, (size_t)n, "cell order"));
        HIPC(launch_gather(x, n, d, ld, out->orig, dperm, nbw, xs1, s), "gather kernel");
        HIPC(launch_cell_order_keys(xs1, n, std::min(nbw, kOrderDims / 4), cid, (int64_t)M, blo, bhi, bmask, k0, pos, s),
             "cell order kernels");
        HIPC(radix_sort(k0, pos, k1, v1, n, 24 + ceil_log2(M + 1), hist, stmp, s), "cell order sort");
        HIPC(hipMemcpyAsync(orig1, out->orig, sizeof(uint32_t) * n, hipMemcpyDeviceToDevice, s), "copy");
        if (wide) {
            HIPC(launch_permute_rows(nullptr, orig1, pos, n, 0, nullptr, out->orig, s), "row order");
            HIPC(launch_gather(x, n, d, ld, out->orig, dperm, h->nb, out->xs, s), "gather kernel");
        } else {
            HIPC(launch_permute_rows(xs1, orig1, pos, n, h->nb, out->xs, out->orig, s), "row permute kernel");
        }
    } else if (h->tree_order) {
        // rows gathered in cell order (up to 64 dimensions all of them,
        // above only the first kTreeDims), each cell's rows sorted level by
        // level into the leaf order of a balanced tree, then moved (or,
        // above 64 dimensions, gathered again) into that order
        const bool wide = d > 64;
        const int nbw = wide ? std::min(h->nb, kTreeDims / 4) : h->nb;
        float4 *xs1 = nullptr;
        uint32_t *orig1 = nullptr, *pos = nullptr, *ndim = nullptr, *cnt = nullptr, *maxsz = nullptr;
        uint32_t *nst[2] = {nullptr, nullptr}, *nsz[2] = {nullptr, nullptr};
        uint64_t *off = nullptr;
        TRY(tmp.get(&xs1, (size_t)nbw * n, "tree order"));
        TRY(tmp.get(&orig1, (size_t)n, "tree order"));
        TRY(tmp.get(&pos, (size_t)n, "tree order"));
        for (int k = 0; k < 2; ++k) {
            TRY(tmp.get(&nst[k], (size_t)n + 1, "tree order"));
            TRY(tmp.get(&nsz[k], (size_t)n + 1, "tree order"));
        }
        TRY(tmp.get(&ndim, (size_t)n + 1, "tree order"));
        TRY(tmp.get(&cnt, (size_t)n + 1, "tree order"));
        TRY(tmp.get(&off, (size_t)n + 2, "tree order"));
        TRY(tmp.get(&maxsz, 1, "tree order"));
        HIPC(launch_gather(x, n, d, ld, out->orig, dperm, nbw, xs1, s), "gather kernel");
        HIPC(launch_tree_roots(out->cell_start, (int64_t)M, nst[0], nsz[0], pos, n, maxsz, s), "tree roots");
        uint32_t big = 0;
        HIPC(hipMemcpyAsync(&big, maxsz, sizeof big, hipMemcpyDeviceToHost, s), "copy");
        TRY(sync(s, "tree order"));
        uint64_t K = M;
        int cur = 0;
        // every split leaves both children smaller than their parent
        for (int level = 0; big > (uint32_t)kTreeLeaf; ++level) {
            if (level >= 64 || K > (uint64_t)n) return fail(ERSJ_ERR_INTERNAL, "tree order did not converge");
            HIPC(launch_tree_level(xs1, n, std::min(nbw, kTreeDims / 4), pos, nst[cur], nsz[cur], (uint32_t)K, ndim, k0, k1, v1, hist, stmp,
                                   cnt, off, nst[cur ^ 1], nsz[cur ^ 1], maxsz, s),
                 "tree level");
            HIPC(hipMemcpyAsync(&K, off + K, sizeof K, hipMemcpyDeviceToHost, s), "copy");
            HIPC(hipMemcpyAsync(&big, maxsz, sizeof big, hipMemcpyDeviceToHost, s), "copy");
            TRY(sync(s, "tree order"));
            cur ^= 1;
        }
        HIPC(hipMemcpyAsync(orig1, out->orig, sizeof(uint32_t) * n, hipMemcpyDeviceToDevice, s), "copy");
        if (wide) {
            HIPC(launch_permute_rows(nullptr, orig1, pos, n, 0, nullptr, out->orig, s), "row order");
            HIPC(launch_gather(x, n, d, ld, out->orig, dperm, h->nb, out->xs, s), "gather kernel");
        } else {
            HIPC(launch_permute_rows(xs1, orig1, pos, n, h->nb, out->xs, out->orig, s), "row permute kernel");
        }
    } else {
        HIPC(launch_gather(x, n, d, ld, out->orig, dperm, h->nb, out->xs, s), "gather kernel");
    }
    // row-major copy in sorted order for the binary64 re-check, which sums
    // in the input's dimension order
    TRY(dalloc(h, &out->xr, (size_t)n * recheck_stride(d), "rows"));
    HIPC(launch_gather_rows(x, ld, out->orig, (uint64_t)n, d, recheck_stride(d), out->xr, s), "row gather kernel");
    HIPC(launch_cell_aabb(out->xs, cid, n, (int64_t)M, out->lo_bits, out->hi_bits, s), "cell boxes");
    TRY(sync(s, "bin"));
    return ERSJ_OK;
}

// A1 for any row set: per-dimension statistics (binary64) and the count of
// non-finite coordinates; returns the statistics on the host.
int row_stats(ersj_index *h, const float *x, int64_t n, int64_t ld, std::vector<double> *hst,
              hipStream_t s)
{
    const int32_t d = h->d;
    Scratch tmp(h);
    const int64_t T = stats_threads(n, d);
    double *part = nullptr, *st = nullptr;
    uint32_t *badp = nullptr;
    unsigned long long *bad = nullptr;
    TRY(tmp.get(&part, (size_t)T * 4, "stats"));
    TRY(tmp.get(&badp, (size_t)T, "stats"));
    TRY(tmp.get(&st, (size_t)d * 4, "stats"));
    TRY(tmp.get(&bad, 1, "stats"));
    HIPC(launch_stats(x, n, d, ld, part, badp, T, st, bad, s), "stats kernels");
    hst->assign((size_t)d * 4, 0.0);
    unsigned long long hbad = 0;
    HIPC(hipMemcpyAsync(hst->data(), st, sizeof(double) * d * 4, hipMemcpyDeviceToHost, s), "stats copy");
    HIPC(hipMemcpyAsync(&hbad, bad, sizeof hbad, hipMemcpyDeviceToHost, s), "stats copy");
    TRY(sync(s, "stats"));
    if (hbad) return fail(ERSJ_ERR_INVALID_ARG, "input holds %llu non-finite coordinates", hbad);
    return ERSJ_OK;
}

double max_abs(const std::vector<double> &hst, int32_t d)
{
    double m = 0.0;
    for (int k = 0; k < d; ++k) m = std::max(m, std::max(std::fabs(hst[k * 4 + 2]), std::fabs(hst[k * 4 + 3])));
    return m;
}

// The self-join's query rows are the points.
void alias_queries(ersj_index *h)
{
    h->semi = false;
    h->nq = h->n;
    h->xq = h->xs;
    h->xqr = h->xr;
    h->qorig = h->orig;
    h->Mq = h->M;
    h->qcell_start = h->cell_start;
    h->qcell_key = h->cell_key;
    h->qlo_bits = h->lo_bits;
    h->qhi_bits = h->hi_bits;
    h->maxabs_q = h->maxabs;
}

int do_build(ersj_index *h, const float *x, int64_t ld, hipStream_t s)
{
    const int64_t n = h->n;
    const int32_t d = h->d;
    // A1: per-dimension statistics and the non-finite check.
    std::vector<double> hst;
    TRY(row_stats(h, x, n, ld, &hst, s));
    h->maxabs = max_abs(hst, d);
    h->mean.resize(d);
    for (int k = 0; k < d; ++k) h->mean[k] = hst[k * 4 + 0];

    // A2: dimensions by descending variance (ties: lower id first); the first
    // three are the grid axes.  Cell width >= eps*(1 + 2^-20), widened so no
    // axis has more than 2^21 - 2 cells (stored coordinates run to G + 1).
    h->perm.resize(d);
    for (int k = 0; k < d; ++k) h->perm[k] = k;
    std::stable_sort(h->perm.begin(), h->perm.end(),
                     [&](int a, int b) { return hst[a * 4 + 1] > hst[b * 4 + 1]; });
    h->pinv.assign(d, 0);
    for (int j = 0; j < d; ++j) h->pinv[h->perm[j]] = j;
    GridParams gp{};
    gp.ndim = std::min(3, d);
    gp.reach = h->opt.grid_reach > 0 ? h->opt.grid_reach : 1;
    const double scale = h->opt.cell_width_scale > 1.0 ? h->opt.cell_width_scale : 1.0;
    const double gmax = std::ldexp(1.0, 21) - 2.0;
    int bits = 1;
    for (int a = 0; a < 3; ++a) {
        gp.dim[a] = a < gp.ndim ? h->perm[a] : 0;
        gp.lo[a] = 0.0;
        gp.w[a] = 1.0;
        gp.G[a] = 1;
        if (a >= gp.ndim) continue;
        const double mn = hst[gp.dim[a] * 4 + 2], mx = hst[gp.dim[a] * 4 + 3];
        const double range = mx - mn;
        gp.lo[a] = mn;
        double w = h->eps * scale * (1.0 + std::ldexp(1.0, -20)) / gp.reach;
        w = std::max(w, range / (gmax - 1.0));
        if (!(w > 0.0)) w = 1.0;
        gp.w[a] = w;
        double g = std::isinf(w) ? 1.0 : std::floor(range / w) + 1.0;
        g = std::min(g, gmax);
        gp.G[a] = (int32_t)g;
        bits = std::max(bits, ceil_log2((uint64_t)gp.G[a] + 2));
    }
    gp.bits = bits;
    // rows within a cell follow a Morton curve, so a block of consecutive rows
    // is compact and its bounding box prunes refinement work: over the cell's
    // own box in the first 8 dimensions (ordered after the cells are known,
    // so the cell key carries no sub-cell bits), or over 8 x 8 x 8 sub-cells
    // on the grid axes (fewer when the grid is near its 2^21 cap)
    // automatic: the box order wherever an MFMA kernel will refine: the
    // fp32 form and the split form up to 64 dimensions cover those 8
    // dimensions with 32-row and 64-candidate groups in their box test, and
    // above 64 dimensions the split form's partial test settles more 32 x 32
    // blocks when a block's rows lie close in the leading dimensions; the
    // direct kernel's 256-candidate groups stay compact on the grid axes only
    // under the sub-cell order
    // Above 64 dimensions a balanced tree over the first 64 layout
    // dimensions (split by the largest variance, 32-row leaves) groups rows
    // of clustered data far better than 8 dimensions can: fewer 32 x 32
    // blocks stay live after the split form's partial test.
    const char *why_not = "";
    const int rk = h->opt.refine_kernel;
    const bool mfma_order = coords_feasible(h, &why_not) && rk != ERSJ_REFINE_DIRECT;
    h->tree_order = h->opt.cell_order == 3 || (h->opt.cell_order == 0 && mfma_order && d > 64);
    h->box_order = !h->tree_order && (h->opt.cell_order == 2 || (h->opt.cell_order == 0 && mfma_order));
    gp.sub = h->box_order || h->tree_order ? 0 : std::min(3, 21 - bits);
    h->gp = gp;

    // A4-A7 for the points.
    Binned b;
    TRY(bin_rows(h, x, n, ld, false, &b, s));
    h->xs = b.xs;
    h->xr = b.xr;
    h->orig = b.orig;
    h->M = b.M;
    h->cell_start = b.cell_start;
    h->cell_key = b.cell_key;
    h->lo_bits = b.lo_bits;
    h->hi_bits = b.hi_bits;
    TRY(sync(s, "build"));
    alias_queries(h);
    thresholds(h);
    TRY(choose_kernel(h));
    return ERSJ_OK;
}

// Semi-join query rows (Sec. II-A): statistics for the non-finite check and
// the coordinate bound, then the same binning as the points, into the
// points' grid.
int do_queries(ersj_index *h, const float *q, int64_t nq, int64_t ldq, hipStream_t s)
{
    std::vector<double> hst;
    TRY(row_stats(h, q, nq, ldq, &hst, s));
    Binned b;
    TRY(bin_rows(h, q, nq, ldq, true, &b, s));
    h->semi = true;
    h->nq = nq;
    h->xq = b.xs;
    h->xqr = b.xr;
    h->qorig = b.orig;
    h->Mq = b.M;
    h->qcell_start = b.cell_start;
    h->qcell_key = b.cell_key;
    h->qlo_bits = b.lo_bits;
    h->qhi_bits = b.hi_bits;
    h->maxabs_q = max_abs(hst, h->d);
    TRY(choose_kernel(h));
    return ERSJ_OK;
}

void release_queries(ersj_index *h)
{
    if (h->semi) {
        dfree(h, h->xq);
        dfree(h, h->xqr);
        dfree(h, h->qorig);
        dfree(h, h->qcell_start);
        dfree(h, h->qcell_key);
        dfree(h, h->qlo_bits);
        dfree(h, h->qhi_bits);
    }
    alias_queries(h);
}

// Split-fp16 operands of the points and the query rows for k_refine_g16:
// centred on the points' per-dimension mean r (fp32, in the layout's
// variance order; padded dimensions 0), scaled by s16, split, with norms.
// The d > 64 filter's int8 operands (k_refine_g16.hip derives the test):
// centred on the layout's means as fp32, scaled by S = 127 / M, M the largest
// |x_i - r_i| over the first kPartialDims dimensions of both point sets,
// raised by 2^-20 over its fp32 evaluation; E the squared radius widened by
// the binary64 reference's rounding.  Left unset (the fp16 form runs) when
// M is not finite and positive.
int prepare_int8_filter(ersj_index *h, hipStream_t s)
{
    std::vector<float> ref(kPartialDims);
    for (int j = 0; j < kPartialDims; ++j) ref[j] = (float)h->mean[h->perm[j]];
    Scratch tmp(h);
    float4 *dref = nullptr;
    unsigned int *dmx = nullptr;
    TRY(tmp.get(&dref, (size_t)kPartialDims / 4, "int8 filter operands"));
    TRY(tmp.get(&dmx, 1, "int8 filter operands"));
    HIPC(hipMemcpyAsync(dref, ref.data(), sizeof(float) * ref.size(), hipMemcpyHostToDevice, s), "copy");
    HIPC(hipMemsetAsync(dmx, 0, sizeof(unsigned int), s), "clear");
    HIPC(launch_maxabs8(h->xs, (uint64_t)h->n, dref, dmx, s), "int8 filter operands");
    if (h->semi) HIPC(launch_maxabs8(h->xq, (uint64_t)h->nq, dref, dmx, s), "int8 filter operands");
    unsigned int bits = 0;
    HIPC(hipMemcpyAsync(&bits, dmx, sizeof bits, hipMemcpyDeviceToHost, s), "copy");
    TRY(sync(s, "int8 filter operands"));
    float mf = 0.0f;
    std::memcpy(&mf, &bits, sizeof mf);
    const double M = (double)mf * (1.0 + std::ldexp(1.0, -20));
    if (!(M > 0.0) || !std::isfinite(M)) return ERSJ_OK;
    const double S = 127.0 / M;
    const double g = std::max(std::ldexp(1.0, -30), 4.0 * gamma_n(h->d + 2, std::ldexp(1.0, -53)));
    const double E = std::isinf(h->e64) ? INFINITY : h->e64 * (1.0 + g);
    h->ps8 = prep16_stride((uint64_t)h->n);
    TRY(dalloc(h, &h->p8, (size_t)4 * (size_t)h->ps8, "int8 filter operands"));
    TRY(dalloc(h, &h->xb8, (size_t)h->n + 1, "int8 filter operands"));
    TRY(dalloc(h, &h->qs8, (size_t)h->nq, "int8 filter operands"));
    HIPC(launch_prep8(h->xs, (uint64_t)h->n, dref, S, E, h->p8, h->ps8, h->semi ? nullptr : h->qs8, h->xb8, s),
         "int8 filter operands");
    if (h->semi) {
        h->ps8q = prep16_stride((uint64_t)h->nq);
        TRY(dalloc(h, &h->p8q, (size_t)4 * (size_t)h->ps8q, "int8 filter operands"));
        HIPC(launch_prep8(h->xq, (uint64_t)h->nq, dref, S, E, h->p8q, h->ps8q, h->qs8, nullptr, s),
             "int8 filter operands");
    } else {
        h->p8q = h->p8;
        h->ps8q = h->ps8;
    }
    TRY(sync(s, "int8 filter operands"));  // ref and dref must outlive the kernels
    return ERSJ_OK;
}

int prepare_operands(ersj_index *h, hipStream_t s)
{
    const int nb = h->nb, ns = g16_stages(nb, h->g16_hh);
    std::vector<float> nrs((size_t)nb * 4, 0.0f);
    for (int j = 0; j < h->d; ++j) nrs[j] = -((float)h->mean[h->perm[j]] * h->s16);
    Scratch tmp(h);
    float4 *dnrs = nullptr;
    TRY(tmp.get(&dnrs, (size_t)nb, "operand preparation"));
    HIPC(hipMemcpyAsync(dnrs, nrs.data(), sizeof(float) * nrs.size(), hipMemcpyHostToDevice, s), "copy");
    h->ps16 = prep16_stride((uint64_t)h->n);
    TRY(dalloc(h, &h->p16, (size_t)ns * 4 * (size_t)h->ps16, "prepared operands"));
    TRY(dalloc(h, &h->n16, (size_t)h->n, "prepared operands"));
    TRY(dalloc(h, &h->np16, (size_t)h->n, "prepared operands"));
    HIPC(launch_prep16(h->xs, (uint64_t)h->n, nb, dnrs, h->s16, h->g16_hh, h->p16, h->ps16, h->n16, h->np16, s),
         "operand preparation");
    TRY(dalloc(h, &h->xb16, (size_t)h->n + 1, "prepared operands"));
    HIPC(launch_col_bounds16(h->np16, (uint64_t)h->n, h->kmf, h->xb16, s), "operand preparation");
    if (h->semi) {
        h->ps16q = prep16_stride((uint64_t)h->nq);
        TRY(dalloc(h, &h->p16q, (size_t)ns * 4 * (size_t)h->ps16q, "prepared operands"));
        TRY(dalloc(h, &h->n16q, (size_t)h->nq, "prepared operands"));
        TRY(dalloc(h, &h->np16q, (size_t)h->nq, "prepared operands"));
        HIPC(launch_prep16(h->xq, (uint64_t)h->nq, nb, dnrs, h->s16, h->g16_hh, h->p16q, h->ps16q, h->n16q,
                           h->np16q, s),
             "operand preparation");
    } else {
        h->p16q = h->p16;
        h->ps16q = h->ps16;
        h->n16q = h->n16;
        h->np16q = h->np16;
    }
    TRY(sync(s, "operand preparation"));  // the host copy of nrs and dnrs must outlive the kernels
    if (h->opt.filter_bits != 16) TRY(prepare_int8_filter(h, s));
    return ERSJ_OK;
}

int do_count(ersj_index *h, hipStream_t s)
{
    release_count(h);
    release_plan(h);
    const int64_t M = h->Mq;  // cells of the query rows
    Scratch tmp(h);
    uint32_t *tpc = nullptr;
    unsigned int *umax = nullptr;
    uint64_t *tbase = nullptr, *stmp = nullptr, *words = nullptr, *cands = nullptr;
    TRY(dalloc(h, &h->rstart, (size_t)M * kMaxRanges, "ranges"));
    TRY(dalloc(h, &h->rpref, (size_t)M * (kMaxRanges + 1), "ranges"));
    TRY(dalloc(h, &h->nrng, (size_t)M, "ranges"));
    TRY(tmp.get(&tpc, (size_t)M, "tiles"));
    TRY(tmp.get(&umax, 1, "tiles"));
    TRY(tmp.get(&tbase, (size_t)M + 1, "tiles"));
    TRY(tmp.get(&stmp, scan_tmp_entries(std::max<int64_t>(M, h->nq) + 1), "scan"));
    // Box pruning: drop neighbour cell B if its box lower distance to A's box
    // exceeds eps.  Computed in binary64 with relative error below 8u; the
    // margin keeps every pair with D64 <= E64 (|D64 - S| <= g64*S).
    const double pf = 1.0 + std::max(std::ldexp(1.0, -40), 16.0 * (h->d + 2) * std::ldexp(1.0, -53));
    const double prune_e2 = std::isinf(h->e64) ? INFINITY : h->e64 * pf;
    const CellSet home{h->qcell_key, h->qcell_start, h->qlo_bits, h->qhi_bits, h->Mq};
    const CellSet target{h->cell_key, h->cell_start, h->lo_bits, h->hi_bits, h->M};
    HIPC(launch_stencil(home, target, h->gp, prune_e2, h->rstart, h->rpref, h->nrng, tpc, umax, s),
         "stencil kernel");
    HIPC(scan_u32(tpc, tbase, M, stmp, s), "tile scan");
    uint64_t T = 0;
    HIPC(hipMemcpyAsync(&T, tbase + M, sizeof T, hipMemcpyDeviceToHost, s), "tile count copy");
    HIPC(hipMemcpyAsync(&h->umax, umax, sizeof(uint32_t), hipMemcpyDeviceToHost, s), "umax copy");
    TRY(sync(s, "stencil"));
    h->T = (int64_t)T;
    TRY(dalloc(h, &h->tiles, (size_t)T, "tiles"));
    TRY(dalloc(h, &h->toff, (size_t)T + 1, "tiles"));
    TRY(dalloc(h, &h->coff, (size_t)T + 1, "tiles"));
    TRY(tmp.get(&words, (size_t)T, "tiles"));
    TRY(tmp.get(&cands, (size_t)T, "tiles"));
    HIPC(launch_tiles(tbase, M, (int64_t)T, h->qcell_start, h->rpref, h->nrng, h->tiles, words, cands, s),
         "tiles kernel");
    HIPC(scan_u64(words, h->toff, (int64_t)T, stmp, s), "word scan");
    HIPC(scan_u64(cands, h->coff, (int64_t)T, stmp, s), "candidate scan");
    HIPC(hipMemcpyAsync(&h->total_words, h->toff + T, sizeof(uint64_t), hipMemcpyDeviceToHost, s), "copy");
    HIPC(hipMemcpyAsync(&h->total_cand, h->coff + T, sizeof(uint64_t), hipMemcpyDeviceToHost, s), "copy");
    if ((h->kernel_used == ERSJ_REFINE_MFMA || h->kernel_used == ERSJ_REFINE_MFMA16) && !h->use_g16 &&
        std::isfinite(h->tbox)) {
        // boxes of each cell list's 64-candidate chunks for the block box test
        uint32_t *ccnt = nullptr;
        TRY(tmp.get(&ccnt, (size_t)M, "chunk boxes"));
        TRY(dalloc(h, &h->chunk_base, (size_t)M + 1, "chunk boxes"));
        HIPC(launch_chunk_counts(h->rpref, h->nrng, M, ccnt, s), "chunk count kernel");
        HIPC(scan_u32(ccnt, h->chunk_base, M, stmp, s), "chunk scan");
        uint64_t nchunks = 0;
        HIPC(hipMemcpyAsync(&nchunks, h->chunk_base + M, sizeof nchunks, hipMemcpyDeviceToHost, s), "copy");
        TRY(sync(s, "chunk count"));
        float4 *pbox = nullptr;
        TRY(tmp.get(&pbox, (size_t)((h->n + 7) / 8 + 1) * 2 * kBoxBlocks, "point boxes"));
        HIPC(launch_point_boxes(h->xs, (uint64_t)h->n, h->nb, pbox, s), "point box kernel");
        TRY(dalloc(h, &h->cbox, (size_t)(nchunks + 1) * 2 * kBoxBlocks, "chunk boxes"));
        HIPC(launch_chunk_boxes(h->chunk_base, M, nchunks, h->rstart, h->rpref, h->nrng, h->xs, (uint64_t)h->n,
                                h->nb, pbox, h->cbox, s),
             "chunk box kernel");
    }
    if (h->use_g16) TRY(prepare_operands(h, s));
    if ((h->kernel_used == ERSJ_REFINE_MFMA || h->kernel_used == ERSJ_REFINE_MFMA16) && !h->use_g16) {
        // per-tile reference points of the MFMA kernels' centring
        TRY(dalloc(h, &h->tref, (size_t)h->T * h->nb, "tile references"));
        HIPC(launch_tile_ref(h->tiles, h->T, h->xq, (uint64_t)h->nq, h->nb, h->tref, s), "tile reference kernel");
    }
    TRY(sync(s, "count pass"));
    return ERSJ_OK;
}

// band-list entries a handle under max_device_bytes starts with: 1/64 of
// the cap, at least 4096 and at most 2^20 (the list still grows on
// overflow, within the cap)
uint64_t capped_band_entries(const ersj_index *h)
{
    const uint64_t e = h->opt.max_device_bytes / 64 / sizeof(Boundary);
    return std::min<uint64_t>(std::max<uint64_t>(e, 4096), 1ull << 20);
}

int do_plan(ersj_index *h, uint64_t budget_bytes, hipStream_t s)
{
    release_plan(h);
    if (budget_bytes == 0) {
        size_t fr = 0, tot = 0;
        HIPC(hipMemGetInfo(&fr, &tot), "hipMemGetInfo");
        fr += pool_cached(h->device);  // blocks this library keeps for reuse
        const uint64_t extra = (uint64_t)h->nq * 24 + (uint64_t)(1 << 22) * sizeof(Boundary);
        uint64_t b = (uint64_t)fr / 4 * 3;
        budget_bytes = b > extra ? b - extra : 8;
        if (h->opt.max_device_bytes) {
            // beside the mask and its flags a batch holds row counts, offsets
            // and their scan (24 bytes a row at most), the counters and the
            // band list
            const uint64_t room = h->opt.max_device_bytes > h->bytes ? h->opt.max_device_bytes - h->bytes : 0;
            // (each buffer above 1 MiB is rounded up to 2 MiB by the pool)
            const uint64_t bl = h->opt.boundary_capacity ? h->opt.boundary_capacity : capped_band_entries(h);
            const uint64_t reserve = (uint64_t)h->nq * 24 + bl * sizeof(Boundary) + (10ull << 20);
            budget_bytes = std::min<uint64_t>(budget_bytes, room > reserve ? room - reserve : 0);
        }
    }
    // a mask word costs 8 bytes plus a quarter byte of unit flags
    const uint64_t budget_words = budget_bytes / 33 * 4;
    if (budget_words == 0) return fail(ERSJ_ERR_BUDGET, "budget of %llu bytes holds no mask word",
                                       (unsigned long long)budget_bytes);
    Scratch tmp(h);
    const int64_t T = h->T;
    uint32_t *bounds = nullptr;
    uint64_t *rowb = nullptr, *wordb = nullptr, *candb = nullptr, *res = nullptr;
    TRY(tmp.get(&bounds, (size_t)T + 1, "plan"));
    TRY(tmp.get(&rowb, (size_t)T + 1, "plan"));
    TRY(tmp.get(&wordb, (size_t)T + 1, "plan"));
    TRY(tmp.get(&candb, (size_t)T + 1, "plan"));
    TRY(tmp.get(&res, 4, "plan"));
    HIPC(launch_plan(h->toff, h->coff, h->tiles, T, h->nq, budget_words, bounds, rowb, wordb, candb, res, s),
         "plan kernel");
    uint64_t hres[4];
    HIPC(hipMemcpyAsync(hres, res, sizeof hres, hipMemcpyDeviceToHost, s), "plan copy");
    TRY(sync(s, "plan"));
    if (hres[2]) {
        const uint64_t t = hres[2] - 1;
        uint64_t w2[2] = {0, 0};
        HIPC(hipMemcpy(w2, h->toff + t, sizeof w2, hipMemcpyDeviceToHost), "plan copy");
        return fail(ERSJ_ERR_BUDGET,
                    "row tile %llu needs %llu bytes of result mask, more than the budget of %llu bytes",
                    (unsigned long long)t, (unsigned long long)((w2[1] - w2[0]) * 8),
                    (unsigned long long)budget_bytes);
    }
    const int64_t nbat = (int64_t)hres[0];
    if (nbat > 0x7fffffff) return fail(ERSJ_ERR_BUDGET, "too many batches (%lld)", (long long)nbat);
    h->nbatch = (int32_t)nbat;
    h->maxw = hres[1];
    h->maxrows = hres[3];
    h->hb.resize(nbat + 1);
    h->hrows.resize(nbat + 1);
    h->hwords.resize(nbat + 1);
    h->hcands.resize(nbat + 1);
    HIPC(hipMemcpyAsync(h->hb.data(), bounds, sizeof(uint32_t) * (nbat + 1), hipMemcpyDeviceToHost, s), "copy");
    HIPC(hipMemcpyAsync(h->hrows.data(), rowb, sizeof(uint64_t) * (nbat + 1), hipMemcpyDeviceToHost, s), "copy");
    HIPC(hipMemcpyAsync(h->hwords.data(), wordb, sizeof(uint64_t) * (nbat + 1), hipMemcpyDeviceToHost, s), "copy");
    HIPC(hipMemcpyAsync(h->hcands.data(), candb, sizeof(uint64_t) * (nbat + 1), hipMemcpyDeviceToHost, s), "copy");

    // Launch order of the row tiles: by batch, heaviest cell first.
    const int ubits = std::max(1, ceil_log2((uint64_t)h->umax + 1));
    const int bbits = ceil_log2((uint64_t)nbat);
    uint64_t *k0 = nullptr, *k1 = nullptr, *hist = nullptr, *stmp = nullptr;
    uint32_t *v1 = nullptr;
    TRY(dalloc(h, &h->order, (size_t)T, "order"));
    TRY(tmp.get(&k0, (size_t)T, "order"));
    TRY(tmp.get(&k1, (size_t)T, "order"));
    TRY(tmp.get(&v1, (size_t)T, "order"));
    const size_t hent = radix_hist_entries(T);
    TRY(tmp.get(&hist, hent, "order"));
    TRY(tmp.get(&stmp, scan_tmp_entries(hent), "order"));
    HIPC(launch_order_keys(h->tiles, h->rpref, h->nrng, T, bounds, (int32_t)nbat, ubits, h->umax, k0,
                           h->order, s), "order keys");
    HIPC(radix_sort(k0, h->order, k1, v1, T, ubits + bbits, hist, stmp, s), "order sort");
    TRY(sync(s, "plan"));
    return ERSJ_OK;
}

// Boundary-list entries to start with: the caller's choice, else a share of
// the batch's candidates, raised to the largest list a previous overflow in
// this process needed (so repeated joins of similar data refine once).
std::atomic<uint64_t> g_bcap_hint{0};

uint64_t initial_bcap(const ersj_index *h)
{
    if (h->opt.boundary_capacity) return h->opt.boundary_capacity;
    if (h->opt.max_device_bytes) return capped_band_entries(h);
    uint64_t maxc = 0;
    for (int32_t b = 0; b < h->nbatch; ++b) maxc = std::max(maxc, h->hcands[b + 1] - h->hcands[b]);
    uint64_t cap = std::min<uint64_t>(std::max<uint64_t>(maxc / 4096, 1ull << 20), 1ull << 27);
    return std::max(cap, g_bcap_hint.load());
}

int ensure_fill_buffers(ersj_index *h)
{
    if (h->mask_cap < h->maxw) {
        dfree(h, h->mask);
        dfree(h, h->gflag);
        h->mask_cap = 0;
        TRY(dalloc(h, &h->mask, (size_t)h->maxw, "result mask"));
        TRY(dalloc(h, &h->gflag, (size_t)(h->maxw / 4 + 64), "mask unit flags"));
        h->mask_cap = h->maxw;
    }
    if (h->rows_cap < h->maxrows) {
        dfree(h, h->rowcnt);
        dfree(h, h->roff);
        dfree(h, h->rscan);
        h->rows_cap = 0;
        TRY(dalloc(h, &h->rowcnt, (size_t)h->maxrows, "row counts"));
        TRY(dalloc(h, &h->roff, (size_t)h->maxrows + 1, "row offsets"));
        TRY(dalloc(h, &h->rscan, scan_tmp_entries((int64_t)h->maxrows + 1), "row scan"));
        h->rows_cap = h->maxrows;
    }
    if (!h->counters) TRY(dalloc(h, &h->counters, (size_t)(2 * kBandLists + 3 * kHitSlots) * kBandStride, "counters"));

    if (!h->lpref) TRY(dalloc(h, &h->lpref, (size_t)kBandLists + 3, "band list prefix"));
    if (!h->blist) {
        const uint64_t cap = initial_bcap(h);
        TRY(dalloc(h, &h->blist, (size_t)cap, "boundary list"));
        h->bcap = cap;
    }
    return ERSJ_OK;
}

// Working memory of one batch's refinement, re-check and compaction: the
// handle's own buffers (ensure_fill_buffers), or carved from the fixed device
// scratch of the allocation-free entry point.
struct FillBufs {
    uint64_t *mask = nullptr;
    uint8_t *gflag = nullptr;
    Boundary *blist = nullptr;
    uint64_t bcap = 0;                         // band-list entries over all sub-lists
    uint4 *dlist = nullptr;                    // handed-on blocks (null: none)
    uint64_t dcap = 0;                         // entries per sub-list
    unsigned long long *counters = nullptr;    // band sub-list counters, then re-check hit slots
    uint64_t *lpref = nullptr;
    uint32_t *rowcnt = nullptr;
    uint64_t *roff = nullptr, *rscan = nullptr;
    bool grow = false;                         // band list may be reallocated on overflow
};

FillBufs handle_bufs(ersj_index *h)
{
    FillBufs fb;
    fb.mask = h->mask;
    fb.gflag = h->gflag;
    fb.blist = h->blist;
    fb.bcap = h->bcap;
    fb.dlist = h->dlist;
    fb.dcap = h->dcap;
    fb.counters = h->counters;
    fb.lpref = h->lpref;
    fb.rowcnt = h->rowcnt;
    fb.roff = h->roff;
    fb.rscan = h->rscan;
    fb.grow = true;
    return fb;
}

// Refine batch b into fb: mask words, band pairs re-checked in binary64, row
// counts and their offsets; *pairs = the batch's pair count.
int refine_into(ersj_index *h, int32_t b, hipStream_t s, FillBufs &fb, uint64_t *pairs)
{
    const uint32_t t0 = h->hb[b], t1 = h->hb[b + 1];
    const uint32_t ntiles = t1 - t0;
    const uint64_t rows = h->hrows[b + 1] - h->hrows[b];
    RefineArgs a{};
    a.xs = h->xs;
    a.n = (uint64_t)h->n;
    a.xq = h->xq;
    a.nqr = (uint64_t)h->nq;
    a.nb = h->nb;
    a.tiles = h->tiles;
    a.order = h->order;
    a.ord0 = t0;
    a.ntiles = ntiles;
    const bool f16 = h->kernel_used == ERSJ_REFINE_MFMA16;
    const bool mfma = h->kernel_used == ERSJ_REFINE_MFMA || f16;
    // row sub-blocks: the direct kernel covers 32 rows per work item, the
    // MFMA kernel 32 per query block it holds
    a.nsub = h->use_m16 || h->use_g16 ? 1u : (uint32_t)(kTileRows / (mfma ? 32 * refine_mfma_qblocks(h->nb) : 32));
    a.p16 = h->p16;
    a.p16q = h->p16q;
    a.ps = h->ps16;
    a.psq = h->ps16q;
    a.n16 = h->n16;
    a.n16q = h->n16q;
    a.np16 = h->np16;
    a.np16q = h->np16q;
    a.xb16 = h->xb16;
    if (h->p8) {
        a.p8 = h->p8;
        a.p8q = h->p8q;
        a.ps8 = h->ps8;
        a.ps8q = h->ps8q;
        a.xb8 = h->xb8;
        a.qs8 = h->qs8;
    }
    a.tref = h->tref;
    const uint64_t rows_items = (uint64_t)ntiles * a.nsub;
    uint32_t seg = 8192;
    auto nseg_of = [&](uint32_t sl) { return (h->umax + sl - 1) / sl; };
    while (seg > 512 && rows_items * nseg_of(seg) < 8192) seg /= 2;
    while (rows_items * nseg_of(seg) > 0x7fffffffull) seg *= 2;
    a.seg_len = seg;
    a.nseg = std::max<uint32_t>(1, nseg_of(seg));
    if (h->use_g16 && fb.grow && !h->opt.max_device_bytes && !h->g16_tiled) {
        // hand-on list of the d > 64 filter: room for a sixteenth of the
        // batch's 32 x 32 blocks (8 bytes an entry, 1/256 of its mask), at
        // least 2^20 entries; a batch with more live blocks is refined again
        // by the tiled kernel
        const uint64_t cand = h->hcands[b + 1] - h->hcands[b];
        const uint64_t want = std::max<uint64_t>(cand / 1024 / 16, 1ull << 20);
        const uint64_t need = (want + kBandLists - 1) / kBandLists;
        if (h->dcap < need) {
            dfree(h, h->dlist);
            h->dlist = nullptr;
            h->dcap = 0;
            if (dalloc(h, &h->dlist, (size_t)(need * kBandLists), "hand-on block list") == ERSJ_OK) h->dcap = need;
            else h->dlist = nullptr;  // refine without it
        }
        fb.dlist = h->dlist;
        fb.dcap = h->dcap;
    }
    a.rstart = h->rstart;
    a.rpref = h->rpref;
    a.nrng = h->nrng;
    a.toff = h->toff;
    a.wbase = h->hwords[b];
    a.mask = fb.mask;
    a.tlo = h->tlo;
    a.thi = h->thi;
    a.kp = h->kp;
    a.km = h->km;
    a.kmf = h->kmf;
    a.s16 = h->s16;
    a.tabs = h->tabs;
    if (f16) {
        a.tlo = h->tlo16;
        a.thi = h->thi16;
    }
    // band sub-list counters, re-check hit slots, skipped-comparison slots,
    // slots of comparisons decided from the first dimensions, handed-on block
    // sub-list counters
    const size_t ncount = (size_t)(2 * kBandLists + 3 * kHitSlots) * kBandStride;
    unsigned long long *const hits = fb.counters + (size_t)kBandLists * kBandStride;
    unsigned long long *const skipped = hits + (size_t)kHitSlots * kBandStride;
    a.tbox = h->tbox;
    a.skipped = skipped;
    a.partial = skipped + (size_t)kHitSlots * kBandStride;
    a.dcount = a.partial + (size_t)kHitSlots * kBandStride;
    a.dlist = fb.dlist;
    a.dcap = fb.dlist ? fb.dcap : 0;
    a.rowcnt = fb.rowcnt;
    a.row_base = h->hrows[b];
    a.cbox = h->cbox;
    a.chunk_base = h->chunk_base;
    a.gflag = fb.gflag;
    if (mfma && !h->cbox) a.tbox = INFINITY;  // no chunk boxes: no block test
    uint64_t bres[2] = {0, 0};  // kept band pairs, largest sub-list count
    uint64_t bcount = 0;
    for (int attempt = 0; attempt < 2; ++attempt) {
        const uint64_t lcap = fb.bcap / kBandLists;
        a.blist = fb.blist;
        a.bcount = fb.counters;
        a.lcap = lcap;
        // d > 64: the filter and the block kernel, or the tiled kernel alone
        const bool filter = h->use_g16 && a.dlist != nullptr;
        HIPC(launch_fill_u64((uint64_t *)fb.counters, 0, (int64_t)ncount, s), "clear counters");
        HIPC(launch_fill_u32(fb.rowcnt, 0, (int64_t)rows, s), "clear row counts");
        timer_start(h, s);
        if (filter) {
            // unit flags cleared here; the filter zeroes the mask units of
            // live blocks only
            const uint64_t words = h->hwords[b + 1] - h->hwords[b];
            HIPC(launch_fill_u64((uint64_t *)fb.gflag, 0, (int64_t)((words / 4 + 7) / 8), s), "clear unit flags");
            HIPC(launch_filter16(a, h->g16_hh, s), "filter kernel");
            // the live blocks, sorted by their candidates' first point, so
            // that the block kernel's waves on one XCD share candidate
            // operands in its L2 (a full sub-list sends the batch to the
            // tiled kernel below, without the block kernel)
            std::vector<unsigned long long> dh((size_t)kBandLists * kBandStride);
            HIPC(hipMemcpyAsync(dh.data(), a.dcount, dh.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost, s),
                 "copy");
            TRY(sync(s, "filter"));
            std::vector<uint64_t> pref(kBandLists + 1, 0);
            bool full = false;
            for (uint32_t k = 0; k < kBandLists; ++k) {
                const unsigned long long c = dh[(size_t)k * kBandStride];
                full |= c > a.dcap;
                pref[k + 1] = pref[k] + std::min<uint64_t>(c, a.dcap);
            }
            const uint64_t total = pref[kBandLists];
            Scratch stmp(h);
            a.dorder = nullptr;
            a.dtotal = 0;
            if (!full && total > 0 && (uint64_t)kBandLists * a.dcap <= 0xffffffffull) {
                uint64_t *dpref = nullptr, *k0 = nullptr, *k1 = nullptr, *hist = nullptr, *sc = nullptr;
                uint32_t *v0 = nullptr, *v1 = nullptr;
                const size_t hent = radix_hist_entries((int64_t)total);
                if (stmp.get(&dpref, kBandLists + 1, "block order") == ERSJ_OK &&
                    stmp.get(&k0, total, "block order") == ERSJ_OK && stmp.get(&k1, total, "block order") == ERSJ_OK &&
                    stmp.get(&v0, total, "block order") == ERSJ_OK && stmp.get(&v1, total, "block order") == ERSJ_OK &&
                    stmp.get(&hist, hent, "block order") == ERSJ_OK &&
                    stmp.get(&sc, scan_tmp_entries((int64_t)hent), "block order") == ERSJ_OK) {
                    HIPC(hipMemcpyAsync(dpref, pref.data(), sizeof(uint64_t) * pref.size(), hipMemcpyHostToDevice, s),
                         "copy");
                    // key bits: the query block (tile << 2 | block) below
                    // the 2^kHandonGroupBits-point group of the first candidate
                    const int qbits = std::max(2, ceil_log2((uint64_t)h->T * 4));
                    const uint32_t gend = (uint32_t)((uint64_t)h->n >> kHandonGroupBits) + 1;
                    const int kbits = qbits + ceil_log2((uint64_t)gend + 1);
                    HIPC(launch_handon_keys(a.dlist, a.dcap, dpref, total, qbits, gend, k0, v0, s), "block order keys");
                    HIPC(radix_sort(k0, v0, k1, v1, (int64_t)total, kbits, hist, sc, s), "block order sort");
                    a.dorder = v0;
                    a.dtotal = total;
                }
            }
            if (!full) HIPC(launch_refine_g16_blocks(a, h->g16_hh, s), "block refine kernel");
            TRY(sync(s, "block refine"));  // the pref copy and the sort buffers outlive the kernels
        } else {
            HIPC(h->use_g16   ? launch_refine_g16(a, h->g16_hh, s)
                 : h->use_m16 ? launch_refine_m16(a, s)
                 : mfma       ? launch_refine_mfma(a, f16, s)
                              : launch_refine_direct(a, s),
                 "refine kernel");
        }
        h->ms_refine += timer_stop(h, s);
        if (h->opt.timing) {
            h->refine_launches += 1;
            h->refined_cand += h->hcands[b + 1] - h->hcands[b];
        }
        HIPC(launch_band_prefix(fb.counters, lcap, fb.lpref, fb.lpref + kBandLists + 1, s), "band prefix");
        HIPC(hipMemcpyAsync(bres, fb.lpref + kBandLists + 1, sizeof bres, hipMemcpyDeviceToHost, s), "copy");
        std::vector<unsigned long long> dc;
        if (filter) {
            dc.resize((size_t)kBandLists * kBandStride);
            HIPC(hipMemcpyAsync(dc.data(), a.dcount, dc.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost, s),
                 "copy");
        }
        TRY(sync(s, "refine"));
        bool over = false;
        for (uint32_t k = 0; k < dc.size() / kBandStride; ++k) over |= dc[(size_t)k * kBandStride] > a.dcap;
        if (over) {
            // more live blocks than the hand-on list holds: this batch and the
            // later ones with the tiled kernel (every mask word is rewritten)
            h->g16_tiled = true;
            a.dlist = nullptr;
            a.dcap = 0;
            if (h->opt.timing) {
                h->refine_launches -= 1;
                h->refined_cand -= h->hcands[b + 1] - h->hcands[b];
            }
            --attempt;
            continue;
        }
        bcount = bres[0];
        h->last_filtered = filter;
        if (bres[1] <= lcap) break;
        // A band sub-list overflowed: grow them all and refine the batch
        // again (every mask word is rewritten, so the first result is
        // discarded).
        const uint64_t cap = (bres[1] + bres[1] / 4 + 64) * kBandLists;
        if (!fb.grow)
            return fail(ERSJ_ERR_SCRATCH,
                        "batch %d: %llu band pairs in one sub-list, the fixed scratch holds %llu per sub-list",
                        b, (unsigned long long)bres[1], (unsigned long long)lcap);
        dfree(h, h->blist);
        h->bcap = 0;
        TRY(dalloc(h, &h->blist, (size_t)cap, "boundary list"));
        h->bcap = cap;
        fb.blist = h->blist;
        fb.bcap = cap;
        if (!h->opt.boundary_capacity) {
            uint64_t cur = g_bcap_hint.load();
            while (cur < cap && !g_bcap_hint.compare_exchange_weak(cur, cap)) {
            }
        }
    }
    if (bres[1] > fb.bcap / kBandLists)
        return fail(ERSJ_ERR_INTERNAL, "band sub-list still overflows after growing it (%llu > %llu)",
                    (unsigned long long)bres[1], (unsigned long long)(fb.bcap / kBandLists));
    timer_start(h, s);
    HIPC(launch_recheck(fb.blist, fb.bcap / kBandLists, fb.lpref, bcount, h->xr, h->xqr, h->d, recheck_stride(h->d),
                        h->e64, fb.mask, fb.gflag, hits, fb.rowcnt, h->hrows[b], s),
         "re-check kernel");
    h->ms_recheck += timer_stop(h, s);
    timer_start(h, s);
    HIPC(scan_u32(fb.rowcnt, fb.roff, (int64_t)rows, fb.rscan, s), "row scan");
    uint64_t tot = 0;  // pairs
    uint64_t hs[3 * kHitSlots * kBandStride];  // re-check hits, skipped comparisons, partial decisions
    HIPC(hipMemcpyAsync(&tot, fb.roff + rows, sizeof tot, hipMemcpyDeviceToHost, s), "copy");
    HIPC(hipMemcpyAsync(hs, hits, sizeof hs, hipMemcpyDeviceToHost, s), "copy");
    TRY(sync(s, "row count"));
    for (uint32_t k = 1; k < kHitSlots; ++k) hs[0] += hs[k * kBandStride];
    uint64_t skip = 0;
    uint64_t part = 0;
    for (uint32_t k = 0; k < kHitSlots; ++k) skip += hs[(kHitSlots + k) * kBandStride];
    for (uint32_t k = 0; k < kHitSlots; ++k) part += hs[(2 * kHitSlots + k) * kBandStride];
    hs[1] = skip;
    h->ms_expand += timer_stop(h, s);
    h->last_cand = h->hcands[b + 1] - h->hcands[b];
    h->last_bnd = bcount;
    h->last_in = hs[0];
    h->last_skip = hs[1];
    h->last_part = part;
    if (h->opt.timing) h->skipped_cand += hs[1];
    if (h->opt.timing) h->partial_cand += part;
    h->last_pairs = tot;
    *pairs = tot;
    return ERSJ_OK;
}

// Refine batch b into the handle's own buffers (kept for a CAPACITY retry).
int do_refine(ersj_index *h, int32_t b, hipStream_t s)
{
    TRY(ensure_fill_buffers(h));
    FillBufs fb = handle_bufs(h);
    uint64_t tot = 0;
    TRY(refine_into(h, b, s, fb, &tot));
    h->ready_batch = b;
    h->ready_pairs = tot;
    return ERSJ_OK;
}


int expand_into(ersj_index *h, int32_t batch, uint32_t *d_pairs, const FillBufs &fb, hipStream_t s)
{
    const uint32_t t0 = h->hb[batch], t1 = h->hb[batch + 1];
    timer_start(h, s);
    HIPC(launch_expand(h->tiles, t0, t1 - t0, h->toff, h->hwords[batch], h->hrows[batch], fb.mask,
                       fb.gflag, fb.roff, h->rstart, h->rpref, h->nrng, h->qorig, h->orig, d_pairs, s),
         "expand kernel");
    h->ms_expand += timer_stop(h, s);
    return ERSJ_OK;
}

int expand_batch(ersj_index *h, int32_t batch, uint32_t *d_pairs, hipStream_t s)
{
    return expand_into(h, batch, d_pairs, handle_bufs(h), s);
}

// The allocation-free fill pass carves every buffer of a batch from the
// fixed device scratch (256-byte aligned pieces): mask words, unit flags,
// row counts, row offsets and their scan temporaries, counters, the band
// prefix, and the band list in what remains.
int noalloc_bufs(ersj_index *h, int32_t b, FillBufs *fb)
{
    void *base = nullptr;
    HIPC(noalloc_scratch(h->device, &base), "address of the fixed scratch");
    const uint64_t words = h->hwords[b + 1] - h->hwords[b];
    const uint64_t rows = h->hrows[b + 1] - h->hrows[b];
    uint64_t off = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = off;
        off += (bytes + 255) & ~(uint64_t)255;
        return at;
    };
    const uint64_t o_mask = take(words * 8);
    const uint64_t o_flag = take(words / 4 + 64);
    const uint64_t o_rcnt = take(rows * 4);
    const uint64_t o_roff = take((rows + 1) * 8);
    const uint64_t o_scan = take(scan_tmp_entries((int64_t)rows + 1) * 8);
    const uint64_t o_cnt = take((uint64_t)(2 * kBandLists + 3 * kHitSlots) * kBandStride * 8);
    const uint64_t o_lpref = take((uint64_t)(kBandLists + 3) * 8);
    const uint64_t min_band = (uint64_t)kBandLists * 64 * sizeof(Boundary);
    if (off + min_band > kNoallocScratchBytes)
        return fail(ERSJ_ERR_SCRATCH,
                    "batch %d needs %llu bytes of working memory (%llu mask words, %llu rows) plus a band list, "
                    "more than the %llu bytes of the fixed scratch; plan smaller batches",
                    b, (unsigned long long)off, (unsigned long long)words, (unsigned long long)rows,
                    (unsigned long long)kNoallocScratchBytes);
    char *p = (char *)base;
    fb->mask = (uint64_t *)(p + o_mask);
    fb->gflag = (uint8_t *)(p + o_flag);
    fb->rowcnt = (uint32_t *)(p + o_rcnt);
    fb->roff = (uint64_t *)(p + o_roff);
    fb->rscan = (uint64_t *)(p + o_scan);
    fb->counters = (unsigned long long *)(p + o_cnt);
    fb->lpref = (uint64_t *)(p + o_lpref);
    fb->blist = (Boundary *)(p + off);
    fb->bcap = (kNoallocScratchBytes - off) / sizeof(Boundary) / kBandLists * kBandLists;
    fb->grow = false;
    return ERSJ_OK;
}

// Copy stream (default priority) and its events, created on first use.
int ensure_delivery(ersj_index *h)
{
    if (h->copy_stream) return ERSJ_OK;
    HIPC(hipStreamCreateWithFlags(&h->copy_stream, hipStreamNonBlocking), "copy stream");
    for (int k = 0; k < 2; ++k) {
        HIPC(hipEventCreateWithFlags(&h->expanded[k], hipEventDisableTiming), "delivery event");
        HIPC(hipEventCreateWithFlags(&h->copied[k], hipEventDisableTiming), "delivery event");
    }
    return ERSJ_OK;
}

// ---- exact kNN driver -------------------------------------------------

// Device memory of one ersj_knn call (not tied to an index handle).
struct DevBuf {
    void *p = nullptr;
    DevBuf() = default;
    DevBuf(const DevBuf &) = delete;
    DevBuf &operator=(const DevBuf &) = delete;
    ~DevBuf()
    {
        if (p) (void)hipFree(p);
    }
    int get(size_t bytes, const char *what)
    {
        if (p) return ERSJ_OK;
        const hipError_t e = hipMalloc(&p, bytes ? bytes : 1);
        if (e != hipSuccess) {
            p = nullptr;
            (void)hipGetLastError();
            return fail(ERSJ_ERR_OOM, "cannot allocate %zu bytes for %s", bytes, what);
        }
        return ERSJ_OK;
    }
    template <typename T>
    T *as() const
    {
        return (T *)p;
    }
};

struct IndexGuard {
    ersj_index *h = nullptr;
    ~IndexGuard();
};

constexpr int kKnnFiniteRounds = ERSJ_KNN_MAX_ROUNDS - 1;

// Next radius factor from the queries that stayed short of k neighbours:
// query q had c_q neighbours within eps, np_q of them at a positive distance,
// and over those the sum L_q of log(eps / rho).  Pooled over the queries,
// m = sum np / sum L is the maximum-likelihood local dimension of Levina and
// Bickel (counts growing like radius^m), kept within [1, d]; with no
// neighbour at a positive distance anywhere, m = d (the local dimension
// cannot exceed the ambient one, so this grows the radius most cautiously).
// Neighbours at distance zero count toward k at any radius, so query q needs
// the radius times ((k - (c_q - np_q)) / max(np_q, 1/2))^(1/m), and passes
// the `cap` neighbours a row ranks in on-chip memory at (cap / c_q)^(1/m).
// The factor is the 95th percentile of the need, but no more than the 10th
// percentile of the cap factor (so few rows take the slower ranking path),
// within [lo, 4].
double knn_factor(int k, int cap, double lo, int d, const std::vector<uint32_t> &packed,
                  const std::vector<double> &lsum, double *dim)
{
    double sn = 0.0, sl = 0.0;
    for (size_t i = 0; i < packed.size(); ++i) {
        sn += (double)(packed[i] >> 16);
        sl += lsum[i];
    }
    double m = (sn > 0.0 && sl > 0.0) ? sn / sl : (double)d;
    m = std::min((double)d, std::max(1.0, m));
    *dim = m;
    const size_t q = packed.size();
    std::vector<double> need(q), room(q);
    for (size_t i = 0; i < q; ++i) {
        const double c = (double)(packed[i] & 0xffffu), np = (double)(packed[i] >> 16);
        need[i] = std::pow(((double)k - (c - np)) / std::max(0.5, np), 1.0 / m);
        room[i] = std::pow((double)cap / std::max(1.0, c), 1.0 / m);
    }
    const size_t a = std::min(q - 1, (size_t)std::ceil(0.95 * (double)q) - 1);
    std::nth_element(need.begin(), need.begin() + a, need.end());
    const size_t b = (size_t)std::floor(0.10 * (double)(q - 1));
    std::nth_element(room.begin(), room.begin() + b, room.end());
    const double f = std::min(need[a], room[b]);
    return std::isfinite(f) ? std::min(4.0, std::max(lo, f)) : 4.0;
}

}  // namespace

// =================================================================== ABI ==
extern "C" {

void ersj_default_options(ersj_options *opt)
{
    if (!opt) return;
    std::memset(opt, 0, sizeof *opt);
    opt->struct_size = sizeof *opt;
    opt->refine_kernel = ERSJ_REFINE_AUTO;
    opt->cell_width_scale = 1.0;
}

const char *ersj_last_error(void) { return g_err.c_str(); }

int ersj_release_cached(int32_t device, uint64_t *released)
{
    g_err.clear();
    if (released) *released = 0;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) {
        (void)hipGetLastError();
        ndev = 0;
    }
    int dev = device;
    if (dev == -1) {
        if (hipGetDevice(&dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(ERSJ_ERR_HIP, "no current HIP device");
        }
    }
    if (dev < 0 || dev >= ndev) return fail(ERSJ_ERR_INVALID_ARG, "device = %d is not a HIP device (%d present)", device, ndev);
    DeviceGuard g(dev);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select device %d", dev);
    std::lock_guard<std::mutex> lk(g_pool_mu);
    auto it = g_pools.find(dev);
    if (it == g_pools.end()) return ERSJ_OK;
    DevicePool &pl = it->second;
    if (!pl.blocks.empty()) (void)hipDeviceSynchronize();
    uint64_t bytes = 0;
    for (const PoolBlock &b : pl.blocks) {
        (void)hipFree(b.p);
        bytes += b.bytes;
    }
    (void)hipGetLastError();
    pl.blocks.clear();
    pl.cached = 0;
    if (released) *released = bytes;
    return ERSJ_OK;
}

void ersj_free(ersj_index *h)
{
    if (!h) return;
    DeviceGuard g(h->device);
    if (h->copy_stream) {
        // staging buffers may still be draining into host memory
        (void)hipStreamSynchronize(h->copy_stream);
        (void)hipStreamDestroy(h->copy_stream);
        for (int k = 0; k < 2; ++k) {
            if (h->expanded[k]) (void)hipEventDestroy(h->expanded[k]);
            if (h->copied[k]) (void)hipEventDestroy(h->copied[k]);
        }
    }
    for (auto &kv : h->live) pool_put(h->device, kv.first, kv.second);
    h->live.clear();
    for (hipEvent_t &e : h->ev)
        if (e) (void)hipEventDestroy(e);
    delete h;
}

int ersj_build_index(const float *d_x, int64_t n, int32_t d, int64_t ld, double eps,
                     const ersj_options *opt, void *stream, ersj_index **out)
{
    g_err.clear();
    if (!out) return fail(ERSJ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!d_x) return fail(ERSJ_ERR_INVALID_ARG, "d_x is NULL");
    if (n < 1 || n > 0xffffffffll) return fail(ERSJ_ERR_INVALID_ARG, "n = %lld outside [1, 2^32-1]", (long long)n);
    if (d < 1 || d > kMaxDim) return fail(ERSJ_ERR_INVALID_ARG, "d = %d outside [1, %d]", d, kMaxDim);
    if (ld < d) return fail(ERSJ_ERR_INVALID_ARG, "ld = %lld < d = %d", (long long)ld, d);
    if (ld > (int64_t)1 << 40) return fail(ERSJ_ERR_INVALID_ARG, "ld = %lld too large", (long long)ld);
    if (std::isnan(eps) || eps < 0.0) return fail(ERSJ_ERR_INVALID_ARG, "eps must be >= 0 (got %g)", eps);
    ersj_options o;
    ersj_default_options(&o);
    if (opt) {
        if (opt->struct_size < offsetof(ersj_options, timing) || opt->struct_size > sizeof o)
            return fail(ERSJ_ERR_INVALID_ARG, "options.struct_size = %u not supported", opt->struct_size);
        std::memcpy(&o, opt, opt->struct_size);
        o.struct_size = sizeof o;
        if (!(o.cell_width_scale >= 0.0) || std::isinf(o.cell_width_scale))
            return fail(ERSJ_ERR_INVALID_ARG, "cell_width_scale must be finite and >= 0");
        if (o.refine_kernel < ERSJ_REFINE_AUTO || o.refine_kernel > ERSJ_REFINE_MFMA16)
            return fail(ERSJ_ERR_INVALID_ARG, "unknown refine_kernel %d", o.refine_kernel);
        if (o.grid_reach < 0 || o.grid_reach > kMaxGridReach)
            return fail(ERSJ_ERR_INVALID_ARG, "grid_reach must be 0, 1 or 2 (got %d)", o.grid_reach);
        if (o.block_prune < -1 || o.block_prune > 1)
            return fail(ERSJ_ERR_INVALID_ARG, "block_prune must be -1, 0 or 1 (got %d)", o.block_prune);
        if (o.cell_order < 0 || o.cell_order > 3)
            return fail(ERSJ_ERR_INVALID_ARG, "cell_order must be 0, 1, 2 or 3 (got %d)", o.cell_order);
        if (o.mfma_products != 0 && o.mfma_products != 1 && o.mfma_products != 3)
            return fail(ERSJ_ERR_INVALID_ARG, "mfma_products must be 0, 1 or 3 (got %d)", o.mfma_products);
        if (o.filter_bits != 0 && o.filter_bits != 8 && o.filter_bits != 16)
            return fail(ERSJ_ERR_INVALID_ARG, "filter_bits must be 0, 8 or 16 (got %d)", o.filter_bits);
    }
    int dev = 0;
    HIPC(hipGetDevice(&dev), "hipGetDevice");
    ersj_index *h = new ersj_index();
    h->device = dev;
    h->opt = o;
    h->n = n;
    h->d = d;
    h->nb = (d + 3) / 4;
    h->eps = eps;
    h->e64 = eps * eps;
    h->kernel_used = ERSJ_REFINE_DIRECT;
    hipStream_t s = (hipStream_t)stream;
    int rc = ERSJ_OK;
    if (o.timing) {
        hipError_t e = hipEventCreate(&h->ev[0]);
        if (e == hipSuccess) e = hipEventCreate(&h->ev[1]);
        if (e != hipSuccess) rc = hip_fail(e, "hipEventCreate");
    }
    if (rc == ERSJ_OK) {
        timer_start(h, s);
        rc = do_build(h, d_x, ld, s);
        h->ms_build += timer_stop(h, s);
    }
    if (rc != ERSJ_OK) {
        std::string keep = g_err;
        (void)hipStreamSynchronize(s);
        ersj_free(h);
        g_err = keep;
        return rc;
    }
    h->state = kBuilt;
    *out = h;
    return ERSJ_OK;
}

int ersj_set_queries(ersj_index *h, const float *d_q, int64_t nq, int64_t ldq, void *stream)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (!d_q) return fail(ERSJ_ERR_INVALID_ARG, "d_q is NULL");
    if (nq < 1 || nq > 0xffffffffll)
        return fail(ERSJ_ERR_INVALID_ARG, "nq = %lld outside [1, 2^32-1]", (long long)nq);
    if (ldq < h->d) return fail(ERSJ_ERR_INVALID_ARG, "ldq = %lld < d = %d", (long long)ldq, h->d);
    if (ldq > (int64_t)1 << 40) return fail(ERSJ_ERR_INVALID_ARG, "ldq = %lld too large", (long long)ldq);
    if (h->state < kBuilt) return fail(ERSJ_ERR_STATE, "index not built");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select the handle's device");
    hipStream_t s = (hipStream_t)stream;
    // whatever was counted or planned belongs to the previous query rows
    release_plan(h);
    release_count(h);
    h->nbatch = 0;
    h->ready_batch = -1;
    h->total_cand = h->total_words = 0;
    h->T = 0;
    h->state = kBuilt;
    release_queries(h);
    timer_start(h, s);
    int rc = do_queries(h, d_q, nq, ldq, s);
    h->ms_build += timer_stop(h, s);
    if (rc != ERSJ_OK) {
        std::string keep = g_err;
        (void)hipStreamSynchronize(s);
        release_queries(h);
        (void)choose_kernel(h);
        g_err = keep;
        return rc;
    }
    return ERSJ_OK;
}

int ersj_count_pass(ersj_index *h, uint64_t *total_candidates, void *stream)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (h->state < kBuilt) return fail(ERSJ_ERR_STATE, "index not built");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select the handle's device");
    hipStream_t s = (hipStream_t)stream;
    timer_start(h, s);
    int rc = do_count(h, s);
    h->ms_count += timer_stop(h, s);
    if (rc != ERSJ_OK) {
        h->state = kBuilt;
        return rc;
    }
    h->state = kCounted;
    if (total_candidates) *total_candidates = h->total_cand;
    return ERSJ_OK;
}

int ersj_plan_batches(ersj_index *h, uint64_t budget_bytes, int32_t *n_batches, void *stream)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (!n_batches) return fail(ERSJ_ERR_INVALID_ARG, "n_batches is NULL");
    if (h->state < kCounted) return fail(ERSJ_ERR_STATE, "count_pass has not run");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select the handle's device");
    hipStream_t s = (hipStream_t)stream;
    timer_start(h, s);
    int rc = do_plan(h, budget_bytes, s);
    h->ms_plan += timer_stop(h, s);
    if (rc != ERSJ_OK) {
        release_plan(h);
        h->state = kCounted;
        return rc;
    }
    h->state = kPlanned;
    *n_batches = h->nbatch;
    return ERSJ_OK;
}

int ersj_fill_pass(ersj_index *h, int32_t batch, uint32_t *d_pairs, uint64_t capacity,
                   uint64_t *n_pairs, void *stream)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (!n_pairs) return fail(ERSJ_ERR_INVALID_ARG, "n_pairs is NULL");
    if (capacity > 0 && !d_pairs) return fail(ERSJ_ERR_INVALID_ARG, "d_pairs is NULL");
    if (h->state < kPlanned) return fail(ERSJ_ERR_STATE, "plan_batches has not run");
    if (batch < 0 || batch >= h->nbatch)
        return fail(ERSJ_ERR_INVALID_ARG, "batch %d outside [0, %d)", batch, h->nbatch);
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select the handle's device");
    hipStream_t s = (hipStream_t)stream;
    if (h->ready_batch != batch) {
        h->ready_batch = -1;
        int rc = do_refine(h, batch, s);
        if (rc != ERSJ_OK) return rc;
    }
    *n_pairs = h->ready_pairs;
    if (capacity < h->ready_pairs)
        return fail(ERSJ_ERR_CAPACITY, "batch %d has %llu pairs, capacity is %llu", batch,
                    (unsigned long long)h->ready_pairs, (unsigned long long)capacity);
    if (h->ready_pairs == 0) return ERSJ_OK;
    return expand_batch(h, batch, d_pairs, s);
}

int ersj_fill_pass_host(ersj_index *h, int32_t batch, uint32_t *host_pairs, uint64_t capacity,
                        uint64_t *n_pairs, void *stream)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (!n_pairs) return fail(ERSJ_ERR_INVALID_ARG, "n_pairs is NULL");
    if (capacity > 0 && !host_pairs) return fail(ERSJ_ERR_INVALID_ARG, "host_pairs is NULL");
    if (h->state < kPlanned) return fail(ERSJ_ERR_STATE, "plan_batches has not run");
    if (batch < 0 || batch >= h->nbatch)
        return fail(ERSJ_ERR_INVALID_ARG, "batch %d outside [0, %d)", batch, h->nbatch);
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select the handle's device");
    hipStream_t s = (hipStream_t)stream;
    if (h->ready_batch != batch) {
        h->ready_batch = -1;
        int rc = do_refine(h, batch, s);
        if (rc != ERSJ_OK) return rc;
    }
    *n_pairs = h->ready_pairs;
    if (capacity < h->ready_pairs)
        return fail(ERSJ_ERR_CAPACITY, "batch %d has %llu pairs, capacity is %llu", batch,
                    (unsigned long long)h->ready_pairs, (unsigned long long)capacity);
    if (h->ready_pairs == 0) return ERSJ_OK;
    TRY(ensure_delivery(h));
    const int k = batch & 1;
    if (h->stage_cap[k] < h->ready_pairs) {
        // the buffer may still be draining a batch two back
        if (h->copy_pending[k]) HIPC(hipEventSynchronize(h->copied[k]), "delivery wait");
        h->copy_pending[k] = false;
        dfree(h, h->stage[k]);
        h->stage_cap[k] = 0;
        const uint64_t cap = h->ready_pairs + h->ready_pairs / 8 + 1024;
        TRY(dalloc(h, &h->stage[k], (size_t)cap * 2, "delivery staging"));
        h->stage_cap[k] = cap;
    }
    // expand into staging buffer k after its previous copy has drained, then
    // copy it out on the copy stream while the caller's stream moves on
    if (h->copy_pending[k]) HIPC(hipStreamWaitEvent(s, h->copied[k], 0), "delivery order");
    TRY(expand_batch(h, batch, h->stage[k], s));
    HIPC(hipEventRecord(h->expanded[k], s), "delivery event");
    HIPC(hipStreamWaitEvent(h->copy_stream, h->expanded[k], 0), "delivery order");
    HIPC(hipMemcpyAsync(host_pairs, h->stage[k], sizeof(uint32_t) * 2 * h->ready_pairs, hipMemcpyDeviceToHost,
                        h->copy_stream), "delivery copy");
    HIPC(hipEventRecord(h->copied[k], h->copy_stream), "delivery event");
    h->copy_pending[k] = true;
    return ERSJ_OK;
}

int ersj_fill_pass_noalloc(ersj_index *h, int32_t batch, uint32_t *d_pairs, uint64_t capacity,
                           uint64_t *n_pairs, void *stream)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (!n_pairs) return fail(ERSJ_ERR_INVALID_ARG, "n_pairs is NULL");
    if (capacity > 0 && !d_pairs) return fail(ERSJ_ERR_INVALID_ARG, "d_pairs is NULL");
    if (h->state < kPlanned) return fail(ERSJ_ERR_STATE, "plan_batches has not run");
    if (batch < 0 || batch >= h->nbatch)
        return fail(ERSJ_ERR_INVALID_ARG, "batch %d outside [0, %d)", batch, h->nbatch);
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select the handle's device");
    hipStream_t s = (hipStream_t)stream;
    FillBufs fb;
    TRY(noalloc_bufs(h, batch, &fb));
    uint64_t tot = 0;
    TRY(refine_into(h, batch, s, fb, &tot));
    *n_pairs = tot;
    if (capacity < tot)
        return fail(ERSJ_ERR_CAPACITY, "batch %d has %llu pairs, capacity is %llu", batch,
                    (unsigned long long)tot, (unsigned long long)capacity);
    if (tot == 0) return ERSJ_OK;
    return expand_into(h, batch, d_pairs, fb, s);
}

int ersj_host_sync(ersj_index *h)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (!h->copy_stream) return ERSJ_OK;
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(ERSJ_ERR_HIP, "cannot select the handle's device");
    HIPC(hipStreamSynchronize(h->copy_stream), "delivery sync");
    h->copy_pending[0] = h->copy_pending[1] = false;
    return ERSJ_OK;
}

int ersj_batch_info(const ersj_index *h, int32_t batch, uint64_t *first_row, uint64_t *n_rows,
                    uint64_t *mask_words)
{
    g_err.clear();
    if (!h) return fail(ERSJ_ERR_INVALID_ARG, "handle is NULL");
    if (h->state < kPlanned) return fail(ERSJ_ERR_STATE, "plan_batches has not run");
    if (batch < 0 || batch >= h->nbatch)
        return fail(ERSJ_ERR_INVALID_ARG, "batch %d outside [0, %d)", batch, h->nbatch);
    if (first_row) *first_row = h->hrows[batch];
    if (n_rows) *n_rows = h->hrows[batch + 1] - h->hrows[batch];
    if (mask_words) *mask_words = h->hwords[batch + 1] - h->hwords[batch];
    return ERSJ_OK;
}

int ersj_get_stats(const ersj_index *h, ersj_stats *o)
{
    g_err.clear();
    if (!h || !o) return fail(ERSJ_ERR_INVALID_ARG, "NULL argument");
    std::memset(o, 0, sizeof *o);
    o->n = h->n;
    o->n_queries = h->nq;
    o->d = h->d;
    for (int a = 0; a < 3; ++a) {
        o->index_dims[a] = a < h->gp.ndim ? h->gp.dim[a] : -1;
        o->grid[a] = h->gp.G[a];
    }
    o->refine_kernel = h->kernel_used;
    o->cells = h->M;
    o->tiles = h->T;
    o->total_candidates = h->total_cand;
    o->total_mask_words = h->total_words;
    o->n_batches = h->nbatch;
    o->last_batch = h->ready_batch;
    o->max_batch_words = h->maxw;
    o->last_batch_candidates = h->last_cand;
    o->last_batch_pairs = h->last_pairs;
    o->last_boundary_pairs = h->last_bnd;
    o->last_recheck_in = h->last_in;
    o->device_bytes = h->bytes;
    o->build_ms = h->ms_build;
    o->count_ms = h->ms_count;
    o->plan_ms = h->ms_plan;
    o->refine_ms = h->ms_refine;
    o->recheck_ms = h->ms_recheck;
    o->expand_ms = h->ms_expand;
    o->refine_launches = h->refine_launches;
    o->refined_candidates = h->refined_cand;
    o->last_skipped = h->last_skip;
    o->skipped_candidates = h->skipped_cand;
    o->mfma_products = h->kernel_used != ERSJ_REFINE_MFMA16 ? 0 : h->g16_hh ? 1 : 3;
    o->last_partial = h->last_part;
    o->last_filtered = h->last_filtered ? 1 : 0;
    o->filter_bits = h->p8 ? 8 : h->use_g16 ? 16 : 0;
    o->partial_candidates = h->partial_cand;
    return ERSJ_OK;
}

int ersj_knn(const float *d_x, int64_t n, int32_t d, int64_t ld, const float *d_q, int64_t nq,
             int64_t ldq, int32_t k, double eps0, double growth, const ersj_options *opt,
             uint32_t *d_ids, double *d_dist2, ersj_knn_info *info, void *stream)
{
    g_err.clear();
    if (!d_x) return fail(ERSJ_ERR_INVALID_ARG, "d_x is NULL");
    if (!d_ids) return fail(ERSJ_ERR_INVALID_ARG, "d_ids is NULL");
    if (n < 1 || n > 0xffffffffll) return fail(ERSJ_ERR_INVALID_ARG, "n = %lld outside [1, 2^32-1]", (long long)n);
    if (d < 1 || d > kMaxDim) return fail(ERSJ_ERR_INVALID_ARG, "d = %d outside [1, %d]", d, kMaxDim);
    if (ld < d) return fail(ERSJ_ERR_INVALID_ARG, "ld = %lld < d = %d", (long long)ld, d);
    if (d_q) {
        if (nq < 1 || nq > 0xffffffffll)
            return fail(ERSJ_ERR_INVALID_ARG, "nq = %lld outside [1, 2^32-1]", (long long)nq);
        if (ldq < d) return fail(ERSJ_ERR_INVALID_ARG, "ldq = %lld < d = %d", (long long)ldq, d);
    } else {
        nq = n;
        ldq = ld;
    }
    const int64_t kmax = std::min<int64_t>(n, knn_max_k());
    if (k < 1 || k > kmax) return fail(ERSJ_ERR_INVALID_ARG, "k = %d outside [1, %lld]", k, (long long)kmax);
    if (!(eps0 > 0.0)) return fail(ERSJ_ERR_INVALID_ARG, "eps0 must be > 0 (got %g)", eps0);
    if (!(growth == 0.0 || (growth > 1.0 && std::isfinite(growth))))
        return fail(ERSJ_ERR_INVALID_ARG, "growth must be 0 or a finite factor > 1 (got %g)", growth);
    if (info) std::memset(info, 0, sizeof *info);
    hipStream_t s = (hipStream_t)stream;
    const float *qsrc = d_q ? d_q : d_x;

    DevBuf idx[2], nbrs, lsum, counter, qrows;
    TRY(idx[0].get(sizeof(uint32_t) * (size_t)nq, "kNN query lists"));
    TRY(idx[1].get(sizeof(uint32_t) * (size_t)nq, "kNN query lists"));
    TRY(nbrs.get(sizeof(uint32_t) * (size_t)nq, "kNN counts"));
    TRY(lsum.get(sizeof(double) * (size_t)nq, "kNN counts"));
    TRY(counter.get(sizeof(uint32_t), "kNN counter"));
    int cur = 0;  // idx[cur] lists the round's queries (round 0: all, in order)
    int64_t m = nq;
    double eps = eps0;
    uint64_t total = 0;
    int round = 0;
    while (m > 0) {
        if (round >= kKnnFiniteRounds) eps = INFINITY;
        const float *qb = qsrc;
        int64_t lq = ldq;
        if (round > 0) {
            TRY(qrows.get(sizeof(float) * (size_t)nq * (size_t)d, "kNN query rows"));
            HIPC(launch_gather_rows(qsrc, ldq, idx[cur].as<uint32_t>(), (uint64_t)m, d, d, qrows.as<float>(), s),
                 "kNN gather kernel");
            qb = qrows.as<float>();
            lq = d;
        }
        IndexGuard g;
        TRY(ersj_build_index(d_x, n, d, ld, eps, opt, stream, &g.h));
        TRY(ersj_set_queries(g.h, qb, m, lq, stream));
        uint64_t cand = 0;
        TRY(ersj_count_pass(g.h, &cand, stream));
        int32_t nbatch = 0;
        TRY(ersj_plan_batches(g.h, 0, &nbatch, stream));
        ersj_index *h = g.h;
        DeviceGuard dg(h->device);
        if (!dg.ok()) return fail(ERSJ_ERR_HIP, "cannot select the index's device");
        HIPC(hipMemsetAsync(counter.p, 0, sizeof(uint32_t), s), "clear kNN counter");
        KnnArgs a{};
        a.tiles = h->tiles;
        a.toff = h->toff;
        a.rpref = h->rpref;
        a.rstart = h->rstart;
        a.nrng = h->nrng;
        a.orig = h->orig;
        a.qorig = h->qorig;
        a.qmap = round > 0 ? idx[cur].as<uint32_t>() : nullptr;
        a.xr = h->xr;
        a.xqr = h->xqr;
        a.ldr = recheck_stride(d);
        a.d = d;
        a.k = (uint32_t)k;
        a.e64 = h->e64;
        a.next = idx[1 - cur].as<uint32_t>();
        a.next_count = counter.as<uint32_t>();
        a.next_nbrs = nbrs.as<uint32_t>();
        a.next_lsum = lsum.as<double>();
        a.ids = d_ids;
        a.dist = d_dist2;
        double select_ms = 0.0;
        for (int32_t b = 0; b < nbatch; ++b) {
            h->ready_batch = -1;
            TRY(do_refine(h, b, s));
            a.t0 = h->hb[b];
            a.wbase = h->hwords[b];
            a.row_base = h->hrows[b];
            a.mask = h->mask;
            a.gflag = h->gflag;
            a.rowcnt = h->rowcnt;
            timer_start(h, s);
            HIPC(launch_knn_select(a, h->hb[b + 1] - h->hb[b], s), "kNN select kernel");
            select_ms += timer_stop(h, s);
        }
        if (info) info->refine_kernel = h->kernel_used;
        if (info && h->opt.timing) {
            info->index_ms += h->ms_build + h->ms_count + h->ms_plan;
            info->refine_ms += h->ms_refine;
            info->recheck_ms += h->ms_recheck + h->ms_expand;
            info->select_ms += select_ms;
            info->refine_launches += h->refine_launches;
            info->computed_candidates += h->refined_cand - h->skipped_cand;
        }
        uint32_t left = 0;
        HIPC(hipMemcpyAsync(&left, counter.p, sizeof left, hipMemcpyDeviceToHost, s), "copy");
        HIPC(hipStreamSynchronize(s), "kNN round");
        total += cand;
        double dim = 0.0, next = eps;
        if (left > 0) {
            if (std::isinf(eps))
                return fail(ERSJ_ERR_HIP, "%u queries short of k neighbours at an infinite radius", left);
            double f = growth;
            if (growth == 0.0) {
                std::vector<uint32_t> hn(left);
                std::vector<double> hl(left);
                HIPC(hipMemcpy(hn.data(), nbrs.p, sizeof(uint32_t) * left, hipMemcpyDeviceToHost), "copy");
                HIPC(hipMemcpy(hl.data(), lsum.p, sizeof(double) * left, hipMemcpyDeviceToHost), "copy");
                // the floor rises after 20 rounds so that the radius keeps
                // growing geometrically toward the unbounded final round
                f = knn_factor(k, knn_max_k(), round < 20 ? 1.02 : 2.0, d, hn, hl, &dim);
            }
            next = eps * f;
            if (!(next > eps) || std::isinf(next)) next = INFINITY;
        }
        if (info && round < ERSJ_KNN_MAX_ROUNDS) {
            info->eps[round] = eps;
            info->queries[round] = m;
            info->candidates[round] = cand;
            info->dim_estimate[round] = dim;
        }
        ++round;
        m = left;
        cur = 1 - cur;
        eps = next;
    }
    if (info) {
        info->rounds = round;
        info->total_candidates = total;
    }
    return ERSJ_OK;
}

}  // extern "C"

namespace {
IndexGuard::~IndexGuard() { ersj_free(h); }
}  // namespace
