// C ABI of the library: argument checks, regime dispatch, the blocked
// driver (phase 2 loop) and the per-(device, stream) workspace cache.
//
// Dispatch follows the hierarchical framework of HSMA-TRSM ("Hierarchical
// Shared Memory-Aware Optimization for TRSM on GPU Platforms", section 4.1,
// Figure 2): m <= 64 takes the direct solve (kernel a); larger m takes the
// blocked algorithm of section 4.3 with the block size, and the order of
// phase 2, from the offline table of section 4.3.2.
//
// Blocked driver (section 4.3):
//   phase 1:  W_t = D_t^{-1} for every diagonal block (diag_inv_launch);
//   copy B_0 -> P (panel buffer, ld = ib);
//   for r = 0 .. nb-1:
//     solve:   B_r = g_r * W_r * P          (g_0 = alpha, else 1; triangular W)
//     then the next block row's right-hand side goes to P, in one of two
//     orders that form the same sums:
//     left-looking (the pages' order, "Phase 2"): one GEMM for block row
//              r+1 alone,  P = alpha B_{r+1} - L_{r+1, 0:r+1} X_{0:r+1},
//              K = (r+1) ib;
//     right-looking: every row below block r at once,
//              B_{r+1:} = beta_r B_{r+1:} - L_{r+1:, r} X_r  (beta_0 = alpha,
//              else 1), K = ib, with the rows of block r+1 routed to P.
// The table records which order measured faster for each (type, m, n);
// products with few output tiles are split along K (gemm_splitk_launch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "trsm.h"
#include "trsm_internal.h"
#include "trsm_kernels.h"

using namespace trsm;

namespace {

struct IbEntry {
    int dtype;
    int64_t m, n;  // the profiled problem: order of L, right-hand-side columns
    int ib;
    int left;  // phase-2 schedule that measured faster: 1 left-looking, 0 right-looking
};
#include "ib_table.inc"

bool log_enabled() {
    static const bool on = [] {
        const char *e = std::getenv("TRSM_LOG");
        return e && e[0] == '1';
    }();
    return on;
}

// ---- device checks and workspace cache ----------------------------------

std::mutex g_mu;
struct DevInfo {
    bool ok;   // gfx950
    int cus;   // compute units
};
std::map<int, DevInfo> g_dev;                                  // device -> properties
// Workspace per (device, stream, slot): slot 0 serves the solve (inverses,
// panel), slot 1 the staging copies of the general variants, which stay in
// use while the solve runs.  A call holds its slot's mutex from the moment
// it takes the buffer until it has enqueued its last kernel (WsLease), so a
// second host thread on the same stream can neither free nor replace the
// buffer while the first still has launches to enqueue that use it.  Slots
// are created under g_mu and never destroyed, so their addresses stay valid.
struct WsSlot {
    std::mutex mu;
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::map<std::tuple<int, hipStream_t, int>, std::unique_ptr<WsSlot>> g_ws;

class WsLease {
  public:
    WsLease() = default;
    WsLease(const WsLease &) = delete;
    WsLease &operator=(const WsLease &) = delete;
    void hold(std::mutex &mu) { lk_ = std::unique_lock<std::mutex>(mu); }

  private:
    std::unique_lock<std::mutex> lk_;
};

trsm_status_t check_device(int *dev_out, int *cus_out = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TRSM_STATUS_HIP_ERROR;
    *dev_out = dev;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_dev.find(dev);
    if (it == g_dev.end()) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TRSM_STATUS_HIP_ERROR;
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        it = g_dev.emplace(dev, DevInfo{ok, prop.multiProcessorCount}).first;
    }
    if (cus_out) *cus_out = it->second.cus;
    return it->second.ok ? TRSM_STATUS_SUCCESS : TRSM_STATUS_NOT_SUPPORTED;
}

// Takes the workspace of (dev, st, slot), at least `bytes` long, and holds
// it in `lease` until the lease is destroyed.  Growing it waits for the
// stream (every earlier call's kernels that use the old buffer have been
// enqueued before this one got the lease) and frees the old buffer.
trsm_status_t get_workspace(int dev, hipStream_t st, size_t bytes, void **out, WsLease &lease,
                            int slot = 0) {
    WsSlot *w = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto &e = g_ws[std::make_tuple(dev, st, slot)];
        if (!e) e.reset(new WsSlot);
        w = e.get();
    }
    lease.hold(w->mu);
    if (w->bytes < bytes) {
        if (w->ptr) {
            if (hipStreamSynchronize(st) != hipSuccess) return TRSM_STATUS_HIP_ERROR;
            (void)hipFree(w->ptr);
            w->ptr = nullptr;
            w->bytes = 0;
        }
        const char *fail = std::getenv("TRSM_FAIL_ALLOC");  // test hook
        if (fail && fail[0] == '1') return TRSM_STATUS_ALLOC_FAILED;
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return TRSM_STATUS_ALLOC_FAILED;
        }
        w->ptr = p;
        w->bytes = bytes;
    }
    *out = w->ptr;
    return TRSM_STATUS_SUCCESS;
}

// ---- launch profiling ----------------------------------------------------

struct ProfRec {
    trsm_profile_record_t r;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
uint32_t g_prof_kinds = 0xffffffffu;  // bit k: record launches of kind k
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    // Timing only: read after the host has synchronized on the stop event,
    // so no system-scope fence is needed.  A record after a kernel that
    // wrote tens of MB left a gap of about 6 us before the next launch with
    // the fence, 4.5 us without it (fp64 8192^2 solve, 15 such records).
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

// Records HIP events around one launch on `st` while profiling is on.
class LaunchTimer {
  public:
    LaunchTimer(int kind, int dt, int64_t m, int64_t n, int64_t k, int64_t batch, hipStream_t st)
        : st_(st) {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (!g_prof_on || kind < 0 || kind > 31 || !((g_prof_kinds >> kind) & 1u)) return;
        rec_.r = trsm_profile_record_t{kind, dt, m, n, k, batch, 0.0f};
        rec_.start = take_event();
        rec_.stop = take_event();
        if (rec_.start && rec_.stop && hipEventRecord(rec_.start, st_) == hipSuccess) active_ = true;
    }
    ~LaunchTimer() {
        if (!active_) return;
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (hipEventRecord(rec_.stop, st_) == hipSuccess) g_prof.push_back(rec_);
    }

  private:
    hipStream_t st_;
    ProfRec rec_{};
    bool active_ = false;
};

// ---- argument handling --------------------------------------------------

bool valid_dtype(int dt) {
    return dt == TRSM_R32F || dt == TRSM_R64F || dt == TRSM_C64F || dt == TRSM_C32F;
}

Scalar read_alpha(int dt, const void *alpha) {
    Scalar s{0.0, 0.0};
    if (dt == TRSM_R32F) s.re = *static_cast<const float *>(alpha);
    else if (dt == TRSM_R64F) s.re = *static_cast<const double *>(alpha);
    else if (dt == TRSM_C32F) {
        const float *a = static_cast<const float *>(alpha);
        s.re = a[0];
        s.im = a[1];
    } else {
        const double *a = static_cast<const double *>(alpha);
        s.re = a[0];
        s.im = a[1];
    }
    return s;
}

trsm_status_t check_args(int dt, int64_t m, int64_t n, const void *alpha, const void *A,
                         int64_t lda, const void *B, int64_t ldb) {
    if (!valid_dtype(dt)) return TRSM_STATUS_INVALID_VALUE;
    if (m < 0 || n < 0) return TRSM_STATUS_INVALID_VALUE;
    const int64_t mn1 = m > 1 ? m : 1;
    if (lda < mn1 || ldb < mn1) return TRSM_STATUS_INVALID_VALUE;
    if (m > 0 && n > 0 && (A == nullptr || B == nullptr || alpha == nullptr))
        return TRSM_STATUS_INVALID_VALUE;
    // element offsets must fit in int64 (the kernels index with int64)
    if (m > 0 && n > 0 && (ldb > INT64_MAX / n || lda > INT64_MAX / m)) return TRSM_STATUS_INVALID_VALUE;
    return TRSM_STATUS_SUCCESS;
}

trsm_status_t hip_status(hipError_t e) { return e == hipSuccess ? TRSM_STATUS_SUCCESS : TRSM_STATUS_HIP_ERROR; }

// Left-looking once an update has this many 64 x 64 tiles (four per CU).
bool valid_ib(int ib) { return ib == 64 || ib == 128 || ib == 256 || ib == 512 || ib == 1024; }

// Nearest tabulated problem for this data type (section 4.3.2: online
// lookup, nearest match).  The table is profiled at several (m, n); scale
// is compared in log space, |log2(m/m_e)| + |log2(n/n_e)|, so that a narrow
// B finds the narrow entries and a square one the square entries.
IbEntry select_entry(int dt, int64_t m, int64_t n) {
    IbEntry best{dt, 0, 0, 256, 0};
    double bestd = 1e300;
    const double lm = std::log2((double)(m > 1 ? m : 1)), ln = std::log2((double)(n > 1 ? n : 1));
    for (const IbEntry &e : kIbTable) {
        if (e.dtype != dt) continue;
        const double d = std::fabs(std::log2((double)e.m) - lm) + std::fabs(std::log2((double)e.n) - ln);
        if (d < bestd) {
            bestd = d;
            best = e;
        }
    }
    return best;
}

int select_ib(int dt, int64_t m, int64_t n) { return select_entry(dt, m, n).ib; }

// Phase 2 schedule.  Left-looking is the pages' order (section 4.3 "Phase 2"):
// block row r+1 is updated once, by all solved rows, with K = (r+1)*ib.
// Right-looking (each solved block row updates every row below it, M = rows
// left) does the same arithmetic in another order.  The offline sweep
// records which one measured faster for each (data type, m, n); a
// left-looking update of a narrow B has few output tiles and a long K, which
// split K (below) turns into enough workgroups.  TRSM_SCHEDULE=left|right
// overrides the table (tuning and tests).
bool use_left_looking(bool table_left) {
    const char *e = std::getenv("TRSM_SCHEDULE");
    if (e && std::strcmp(e, "left") == 0) return true;
    if (e && std::strcmp(e, "right") == 0) return false;
    return table_left;
}

// Split-K target for phase 2: a product with so few 64 x 32 tiles that
// fewer than this many workgroups would run is cut along K (a narrow B gives
// solve and update products a handful of tiles each with a K of ib or
// more).  TRSM_SPLITK=<workgroups> overrides it, 0 turns split-K off (tuning
// and tests).
constexpr int64_t kSplitKTarget = 1024;

int64_t splitk_target() {
    const char *e = std::getenv("TRSM_SPLITK");
    if (e && e[0] != '\0') {
        char *end = nullptr;
        const long long v = std::strtoll(e, &end, 10);
        if (end != e && *end == '\0' && v >= 0) return (int64_t)v;
    }
    return kSplitKTarget;
}

// Host-side plan of the blocked path for one problem: block size, phase-2
// order, the split-K factor of every product and the workspace it needs
// (inverses W, panel P, split-K partial sums).  Makes no HIP call.
struct BlockedPlan {
    int ib = 0;
    bool left = false;
    int64_t nb = 0;
    size_t wbytes = 0, pbytes = 0, partbytes = 0;
    std::vector<int> solve_parts, update_parts;
    size_t bytes() const { return wbytes + pbytes + partbytes; }
};

BlockedPlan plan_blocked(int dt, int64_t m, int64_t n, int ib, bool table_left) {
    BlockedPlan pl;
    pl.ib = ib;
    pl.left = use_left_looking(table_left);
    const size_t es = dtype_size(dt);
    pl.nb = (m + ib - 1) / ib;
    pl.wbytes = ((size_t)pl.nb * ib * ib * es + 255) & ~(size_t)255;
    // the panel buffer P doubles as the inversion's scratch (P is first
    // written after the inversion, in the same stream)
    size_t pbytes = (size_t)ib * n * es;
    const size_t tbytes = (size_t)diag_inv_tmp_elems(ib, m) * es;
    if (tbytes > pbytes) pbytes = tbytes;
    pl.pbytes = (pbytes + 255) & ~(size_t)255;
    // split-K factor of every phase-2 product, and the partial sums they need
    const int64_t target = splitk_target();
    pl.solve_parts.assign((size_t)pl.nb, 1);
    pl.update_parts.assign((size_t)pl.nb, 1);
    int64_t part_elems = 0;
    for (int64_t r = 0; r < pl.nb; ++r) {
        const int64_t r0 = r * ib;
        const int64_t bs = (m - r0) < ib ? (m - r0) : ib;
        int p = gemm_splitk_parts(dt, bs, n, bs, target);
        pl.solve_parts[(size_t)r] = p;
        if (p > 1) part_elems = std::max(part_elems, p * bs * n);
        if (r + 1 == pl.nb) break;
        const int64_t mrest = m - r0 - bs;
        const int64_t bsn = mrest < ib ? mrest : ib;
        p = pl.left ? gemm_splitk_parts(dt, bsn, n, r0 + bs, target)
                    : gemm_splitk_parts(dt, mrest, n, bs, target);
        pl.update_parts[(size_t)r] = p;
        if (p > 1) part_elems = std::max(part_elems, p * (pl.left ? bsn : mrest) * n);
    }
    pl.partbytes = (size_t)part_elems * es;
    return pl;
}

// Blocked path for one problem (m > 0, n > 0, alpha != 0), on the workspace
// `ws` of at least pl.bytes() bytes.
trsm_status_t exec_blocked(const BlockedPlan &pl, int dt, int64_t m, int64_t n, Scalar alpha,
                           const void *A, int64_t lda, void *B, int64_t ldb, void *ws,
                           hipStream_t st) {
    const bool left = pl.left;
    const int ib = pl.ib;
    const int64_t nb = pl.nb;
    const size_t es = dtype_size(dt);
    const std::vector<int> &solve_parts = pl.solve_parts, &update_parts = pl.update_parts;
    char *W = static_cast<char *>(ws);
    void *P = W + pl.wbytes;
    void *Part = pl.partbytes > 0 ? W + pl.wbytes + pl.pbytes : nullptr;
    const char *Ab = static_cast<const char *>(A);
    char *Bb = static_cast<char *>(B);
    if (log_enabled())
        std::fprintf(stderr, "[trsm] blocked dtype=%d m=%lld n=%lld ib=%d nb=%lld %s-looking\n", dt,
                     (long long)m, (long long)n, ib, (long long)nb, left ? "left" : "right");

    hipError_t e;
    {
        LaunchTimer t(TRSM_KERNEL_DIAG_INV, dt, m, ib, 0, nb, st);
        e = diag_inv_launch(dt, ib, m, A, lda, W, P, st);
    }
    if (e != hipSuccess) return TRSM_STATUS_HIP_ERROR;
    const int64_t bs0 = m < ib ? m : ib;
    {
        LaunchTimer t(TRSM_KERNEL_COPY, dt, bs0, n, 0, 1, st);
        e = copy_panel_launch(dt, bs0, n, B, ldb, P, ib, st);
    }
    if (e != hipSuccess) return TRSM_STATUS_HIP_ERROR;
    const Scalar one{1.0, 0.0};
    const Scalar minus_one{-1.0, 0.0};
    for (int64_t r = 0; r < nb; ++r) {
        const int64_t r0 = r * ib;
        const int64_t bs = (m - r0) < ib ? (m - r0) : ib;
        // solve: B_r = g_r * W_r * P
        GemmDesc sg{};
        sg.M = bs;
        sg.N = n;
        sg.K = bs;
        sg.A = W + (size_t)r * ib * ib * es;
        sg.lda = ib;
        sg.Bm = P;
        sg.ldb = ib;
        sg.C = nullptr;
        sg.ldc = ldb;
        sg.D = Bb + (size_t)r0 * es;
        sg.ldd = ldb;
        sg.D2 = nullptr;
        sg.ldd2 = ldb;
        sg.split = 0;
        sg.beta = Scalar{0.0, 0.0};
        sg.gamma = (r == 0) ? alpha : one;
        sg.a_lower = 1;
        {
            LaunchTimer t(TRSM_KERNEL_SOLVE_GEMM, dt, bs, n, bs, 1, st);
            e = gemm_splitk_launch(dt, sg, solve_parts[(size_t)r], Part, st);
        }
        if (e != hipSuccess) return TRSM_STATUS_HIP_ERROR;
        if (r + 1 == nb) break;
        const int64_t mrest = m - r0 - bs;
        const int64_t bsn = mrest < ib ? mrest : ib;
        if (left) {
            // next block row: P = alpha B_{r+1} - L[r+1, 0:r+1] X[0:r+1]
            GemmDesc ug{};
            ug.M = bsn;
            ug.N = n;
            ug.K = r0 + bs;
            ug.A = Ab + (size_t)(r0 + bs) * es;
            ug.lda = lda;
            ug.Bm = Bb;
            ug.ldb = ldb;
            ug.C = Bb + (size_t)(r0 + bs) * es;
            ug.ldc = ldb;
            ug.D = P;
            ug.ldd = ib;
            ug.ldd2 = ib;
            ug.beta = alpha;
            ug.gamma = minus_one;
            {
                LaunchTimer t(TRSM_KERNEL_UPDATE_GEMM, dt, bsn, n, r0 + bs, 1, st);
                e = gemm_splitk_launch(dt, ug, update_parts[(size_t)r], Part, st);
            }
            if (e != hipSuccess) return TRSM_STATUS_HIP_ERROR;
            continue;
        }
        // update: rows below block r
        GemmDesc ug{};
        ug.M = mrest;
        ug.N = n;
        ug.K = bs;
        ug.A = Ab + ((size_t)(r0 + bs) + (size_t)r0 * lda) * es;
        ug.lda = lda;
        ug.Bm = Bb + (size_t)r0 * es;
        ug.ldb = ldb;
        ug.C = Bb + (size_t)(r0 + bs) * es;
        ug.ldc = ldb;
        ug.D = Bb + (size_t)(r0 + bs) * es;
        ug.ldd = ldb;
        ug.D2 = P;
        ug.ldd2 = ib;
        ug.split = bsn;
        ug.beta = (r == 0) ? alpha : one;
        ug.gamma = minus_one;
        ug.a_lower = 0;
        {
            LaunchTimer t(TRSM_KERNEL_UPDATE_GEMM, dt, mrest, n, bs, 1, st);
            e = gemm_splitk_launch(dt, ug, update_parts[(size_t)r], Part, st);
        }
        if (e != hipSuccess) return TRSM_STATUS_HIP_ERROR;
    }
    return TRSM_STATUS_SUCCESS;
}

trsm_status_t run(int dt, int64_t m, int64_t n, const void *alpha_p, const void *A, int64_t lda,
                  int64_t sA, void *B, int64_t ldb, int64_t sB, int64_t batch, int ib_forced,
                  bool force_blocked, hipStream_t st) {
    if (m == 0 || n == 0 || batch == 0) return TRSM_STATUS_SUCCESS;
    int dev = 0;
    trsm_status_t s = check_device(&dev);
    if (s != TRSM_STATUS_SUCCESS) return s;
    const Scalar alpha = read_alpha(dt, alpha_p);
    if (alpha.re == 0.0 && alpha.im == 0.0) {
        if (log_enabled()) std::fprintf(stderr, "[trsm] alpha == 0: B <- 0\n");
        LaunchTimer t(TRSM_KERNEL_FILL, dt, m, n, 0, batch, st);
        return hip_status(fill_zero_launch(dt, m, n, B, ldb, sB, batch, st));
    }
    if (m <= 64 && !force_blocked) {
        if (log_enabled())
            std::fprintf(stderr, "[trsm] small dtype=%d m=%lld n=%lld batch=%lld\n", dt,
                         (long long)m, (long long)n, (long long)batch);
        LaunchTimer t(TRSM_KERNEL_SMALL, dt, m, n, 0, batch, st);
        return hip_status(small_lln_launch(dt, (int)m, n, alpha, A, lda, sA, B, ldb, sB, batch, st));
    }
    const IbEntry cfg = select_entry(dt, m, n);
    const BlockedPlan pl = plan_blocked(dt, m, n, ib_forced ? ib_forced : cfg.ib, cfg.left != 0);
    const size_t es = dtype_size(dt);
    void *ws = nullptr;
    WsLease lease;  // held until every launch below is enqueued
    s = get_workspace(dev, st, pl.bytes(), &ws, lease);
    if (s != TRSM_STATUS_SUCCESS) return s;
    for (int64_t p = 0; p < batch; ++p) {
        s = exec_blocked(pl, dt, m, n, alpha, static_cast<const char *>(A) + (size_t)(p * sA) * es,
                         lda, static_cast<char *>(B) + (size_t)(p * sB) * es, ldb, ws, st);
        if (s != TRSM_STATUS_SUCCESS) return s;
    }
    return TRSM_STATUS_SUCCESS;
}

}  // namespace

extern "C" {

trsm_status_t trsm_lln(trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                       const void *A, int64_t lda, void *B, int64_t ldb, hipStream_t stream) {
    try {
        trsm_status_t s = check_args(dtype, m, n, alpha, A, lda, B, ldb);
        if (s != TRSM_STATUS_SUCCESS) return s;
        return run(dtype, m, n, alpha, A, lda, 0, B, ldb, 0, 1, 0, false, stream);
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_lln_noalloc(trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                               const void *A, int64_t lda, void *B, int64_t ldb,
                               hipStream_t stream) {
    try {
        trsm_status_t s = check_args(dtype, m, n, alpha, A, lda, B, ldb);
        if (s != TRSM_STATUS_SUCCESS) return s;
        if (m == 0 || n == 0) return TRSM_STATUS_SUCCESS;
        const Scalar al = read_alpha(dtype, alpha);
        const bool direct = m <= 64 || (al.re == 0.0 && al.im == 0.0);
        // the blocked path's plan and its workspace size: host arithmetic only,
        // so an oversized problem is refused before any HIP call
        BlockedPlan pl;
        if (!direct) {
            const IbEntry cfg = select_entry(dtype, m, n);
            pl = plan_blocked(dtype, m, n, cfg.ib, cfg.left != 0);
            if (pl.bytes() > (size_t)TRSM_NOALLOC_MAX_WORKSPACE_BYTES) {
                if (log_enabled())
                    std::fprintf(stderr, "[trsm] noalloc: workspace %zu bytes > %llu\n", pl.bytes(),
                                 (unsigned long long)TRSM_NOALLOC_MAX_WORKSPACE_BYTES);
                return TRSM_STATUS_INVALID_VALUE;
            }
        }
        if (direct) return run(dtype, m, n, alpha, A, lda, 0, B, ldb, 0, 1, 0, false, stream);
        int dev = 0;
        s = check_device(&dev);
        if (s != TRSM_STATUS_SUCCESS) return s;
        void *ws = nullptr;
        size_t ws_bytes = 0;
        if (noalloc_scratch(dev, &ws, &ws_bytes) != hipSuccess) return TRSM_STATUS_HIP_ERROR;
        if (pl.bytes() > ws_bytes) return TRSM_STATUS_INVALID_VALUE;
        return exec_blocked(pl, dtype, m, n, al, A, lda, B, ldb, ws, stream);
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_lln_strided_batched(trsm_dtype_t dtype, int64_t m, int64_t n,
                                       const void *alpha, const void *A, int64_t lda,
                                       int64_t strideA, void *B, int64_t ldb, int64_t strideB,
                                       int64_t batch, hipStream_t stream) {
    try {
        if (batch < 0 || strideA < 0 || strideB < 0) return TRSM_STATUS_INVALID_VALUE;
        trsm_status_t s = check_args(dtype, m, n, alpha, A, lda, B, ldb);
        if (s != TRSM_STATUS_SUCCESS) return s;
        if (batch > 1 && m > 0 && n > 0 &&
            (strideA > INT64_MAX / batch || strideB > INT64_MAX / batch))
            return TRSM_STATUS_INVALID_VALUE;
        return run(dtype, m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, 0, false, stream);
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_solve(trsm_side_t side, trsm_fill_t uplo, trsm_op_t trans, trsm_diag_t diag,
                         trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                         const void *A, int64_t lda, void *B, int64_t ldb, hipStream_t stream) {
    try {
        if ((side != TRSM_LEFT && side != TRSM_RIGHT) || (uplo != TRSM_LOWER && uplo != TRSM_UPPER) ||
            (trans != TRSM_OP_N && trans != TRSM_OP_T && trans != TRSM_OP_C) ||
            (diag != TRSM_NON_UNIT && diag != TRSM_UNIT) || !valid_dtype(dtype) || m < 0 || n < 0)
            return TRSM_STATUS_INVALID_VALUE;
        const int64_t k = side == TRSM_LEFT ? m : n;  // order of A
        if (lda < (k > 1 ? k : 1) || ldb < (m > 1 ? m : 1)) return TRSM_STATUS_INVALID_VALUE;
        if (m > 0 && n > 0 && (A == nullptr || B == nullptr || alpha == nullptr))
            return TRSM_STATUS_INVALID_VALUE;
        if (m > 0 && n > 0 && (ldb > INT64_MAX / n || lda > INT64_MAX / k)) return TRSM_STATUS_INVALID_VALUE;
        if (m == 0 || n == 0) return TRSM_STATUS_SUCCESS;
        if (side == TRSM_LEFT && uplo == TRSM_LOWER && trans == TRSM_OP_N && diag == TRSM_NON_UNIT)
            return run(dtype, m, n, alpha, A, lda, 0, B, ldb, 0, 1, 0, false, stream);
        int dev = 0;
        trsm_status_t s = check_device(&dev);
        if (s != TRSM_STATUS_SUCCESS) return s;
        const Scalar al = read_alpha(dtype, alpha);
        if (al.re == 0.0 && al.im == 0.0) {
            LaunchTimer t(TRSM_KERNEL_FILL, dtype, m, n, 0, 1, stream);
            return hip_status(fill_zero_launch(dtype, m, n, B, ldb, 0, 1, stream));
        }
        // Every variant is a left-lower solve E' X' = alpha B' (section 2.1's
        // system).  E = op(A) on the left; on the right X op(A) = alpha B is
        // op(A)^T X^T = alpha B^T, so E = op(A)^T and the right-hand sides are
        // the rows of B.  An upper E becomes lower by reversing the order of
        // the unknowns: E' = J E J, B' = J B (J the reversal permutation).
        const bool e_trans = side == TRSM_LEFT ? trans != TRSM_OP_N : trans == TRSM_OP_N;
        const bool op_lower = (uplo == TRSM_LOWER) == (trans == TRSM_OP_N);
        const bool e_lower = side == TRSM_LEFT ? op_lower : !op_lower;
        const int rev = e_lower ? 0 : 1;
        const int64_t nrhs = side == TRSM_LEFT ? n : m;
        const bool b_in_place = side == TRSM_LEFT && !rev;  // B is already B'
        const size_t es = dtype_size(dtype);
        const size_t abytes = ((size_t)k * (size_t)k * es + 255) & ~(size_t)255;
        const size_t bbytes = b_in_place ? 0 : (size_t)k * (size_t)nrhs * es;
        void *ws = nullptr;
        WsLease lease;  // the staging slot, held until the copy back is enqueued
        s = get_workspace(dev, stream, abytes + bbytes, &ws, lease, 1);
        if (s != TRSM_STATUS_SUCCESS) return s;
        void *Ap = ws;
        void *Bp = static_cast<char *>(ws) + abytes;
        if (log_enabled())
            std::fprintf(stderr, "[trsm] variant side=%d uplo=%d trans=%d diag=%d: E %s%s\n", side,
                         uplo, trans, diag, e_trans ? "transposed" : "direct", rev ? ", reversed" : "");
        const Reflect fa{rev, rev, e_trans ? 1 : 0, trans == TRSM_OP_C ? 1 : 0, 1,
                         diag == TRSM_UNIT ? 1 : 0};
        {
            LaunchTimer t(TRSM_KERNEL_COPY, dtype, k, k, 0, 1, stream);
            if (transform_launch(dtype, k, k, A, lda, Ap, k, fa, stream) != hipSuccess)
                return TRSM_STATUS_HIP_ERROR;
        }
        if (b_in_place) return run(dtype, k, nrhs, alpha, Ap, k, 0, B, ldb, 0, 1, 0, false, stream);
        // B'(i, j) = B(rev ? k-1-i : i, j) on the left, B(j, rev ? k-1-i : i) on the right
        const Reflect fb{rev, 0, side == TRSM_RIGHT ? 1 : 0, 0, 0, 0};
        {
            LaunchTimer t(TRSM_KERNEL_COPY, dtype, k, nrhs, 0, 1, stream);
            if (transform_launch(dtype, k, nrhs, B, ldb, Bp, k, fb, stream) != hipSuccess)
                return TRSM_STATUS_HIP_ERROR;
        }
        s = run(dtype, k, nrhs, alpha, Ap, k, 0, Bp, k, 0, 1, 0, false, stream);
        if (s != TRSM_STATUS_SUCCESS) return s;
        // back: B(i, j) = B'(rev ? m-1-i : i, j) on the left, B'(rev ? n-1-j : j, i) on the right
        const Reflect fx = side == TRSM_LEFT ? Reflect{rev, 0, 0, 0, 0, 0} : Reflect{0, rev, 1, 0, 0, 0};
        LaunchTimer t(TRSM_KERNEL_COPY, dtype, m, n, 0, 1, stream);
        return hip_status(transform_launch(dtype, m, n, Bp, k, B, ldb, fx, stream));
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_lln_ex(trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                          const void *A, int64_t lda, void *B, int64_t ldb, int ib,
                          int force_blocked, hipStream_t stream) {
    try {
        if (ib != 0 && !valid_ib(ib))
            return TRSM_STATUS_INVALID_VALUE;
        trsm_status_t s = check_args(dtype, m, n, alpha, A, lda, B, ldb);
        if (s != TRSM_STATUS_SUCCESS) return s;
        return run(dtype, m, n, alpha, A, lda, 0, B, ldb, 0, 1, ib, force_blocked != 0, stream);
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_kernel_diag_inv(trsm_dtype_t dtype, int ib, int64_t m, const void *A,
                                   int64_t lda, void *W, hipStream_t stream) {
    try {
        if (!valid_dtype(dtype) || m < 0 || lda < (m > 1 ? m : 1)) return TRSM_STATUS_INVALID_VALUE;
        if (!valid_ib(ib)) return TRSM_STATUS_INVALID_VALUE;
        if (m == 0) return TRSM_STATUS_SUCCESS;
        if (A == nullptr || W == nullptr) return TRSM_STATUS_INVALID_VALUE;
        int dev = 0;
        trsm_status_t s = check_device(&dev);
        if (s != TRSM_STATUS_SUCCESS) return s;
        void *tmp = nullptr;
        WsLease lease;
        const size_t tbytes = (size_t)diag_inv_tmp_elems(ib, m) * dtype_size(dtype);
        if (tbytes > 0) {
            s = get_workspace(dev, stream, tbytes, &tmp, lease);
            if (s != TRSM_STATUS_SUCCESS) return s;
        }
        LaunchTimer t(TRSM_KERNEL_DIAG_INV, dtype, m, ib, 0, (m + ib - 1) / ib, stream);
        return hip_status(diag_inv_launch(dtype, ib, m, A, lda, W, tmp, stream));
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_kernel_gemm(trsm_dtype_t dtype, int64_t M, int64_t N, int64_t K,
                               const void *beta, const void *gamma, const void *A,
                               int64_t lda, const void *Bm, int64_t ldb, const void *C,
                               int64_t ldc, void *D, int64_t ldd, void *D2, int64_t ldd2,
                               int64_t split, int a_lower, hipStream_t stream) {
    try {
        if (!valid_dtype(dtype) || M < 0 || N < 0 || K < 0) return TRSM_STATUS_INVALID_VALUE;
        if (beta == nullptr || gamma == nullptr) return TRSM_STATUS_INVALID_VALUE;
        if (lda < (M > 1 ? M : 1) || ldb < (K > 1 ? K : 1) || ldd < (M > 1 ? M : 1))
            return TRSM_STATUS_INVALID_VALUE;
        if (a_lower && M != K) return TRSM_STATUS_INVALID_VALUE;
        if (split < 0 || split > M) return TRSM_STATUS_INVALID_VALUE;
        if (D2 != nullptr && ldd2 < (split > 1 ? split : 1)) return TRSM_STATUS_INVALID_VALUE;
        const Scalar b = read_alpha(dtype, beta);
        const Scalar g = read_alpha(dtype, gamma);
        const bool has_c = b.re != 0.0 || b.im != 0.0;
        if (has_c && (C == nullptr || ldc < (M > 1 ? M : 1))) return TRSM_STATUS_INVALID_VALUE;
        if (M == 0 || N == 0) return TRSM_STATUS_SUCCESS;
        if (D == nullptr || (K > 0 && (A == nullptr || Bm == nullptr))) return TRSM_STATUS_INVALID_VALUE;
        int dev = 0;
        trsm_status_t s = check_device(&dev);
        if (s != TRSM_STATUS_SUCCESS) return s;
        GemmDesc gd{};
        gd.M = M;
        gd.N = N;
        gd.K = K;
        gd.A = A;
        gd.lda = lda;
        gd.Bm = Bm;
        gd.ldb = ldb;
        gd.C = has_c ? C : nullptr;
        gd.ldc = has_c ? ldc : ldd;
        gd.D = D;
        gd.ldd = ldd;
        gd.D2 = D2;
        gd.ldd2 = ldd2;
        gd.split = D2 ? split : 0;
        gd.beta = b;
        gd.gamma = g;
        gd.a_lower = a_lower ? 1 : 0;
        LaunchTimer t(a_lower ? TRSM_KERNEL_SOLVE_GEMM : TRSM_KERNEL_UPDATE_GEMM, dtype, M, N, K, 1,
                      stream);
        return hip_status(gemm_launch(dtype, gd, stream));
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_profile_start(void) {
    try {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        for (ProfRec &r : g_prof) {
            (void)hipEventSynchronize(r.stop);
            g_event_pool.push_back(r.start);
            g_event_pool.push_back(r.stop);
        }
        g_prof.clear();
        g_prof_on = true;
        return TRSM_STATUS_SUCCESS;
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

trsm_status_t trsm_profile_select(uint32_t kind_mask) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_kinds = kind_mask;
    return TRSM_STATUS_SUCCESS;
}

trsm_status_t trsm_profile_stop(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = false;
    return TRSM_STATUS_SUCCESS;
}

int64_t trsm_profile_count(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    return (int64_t)g_prof.size();
}

trsm_status_t trsm_profile_read(int64_t i, trsm_profile_record_t *rec) {
    try {
        if (rec == nullptr) return TRSM_STATUS_INVALID_VALUE;
        ProfRec r;
        {
            std::lock_guard<std::mutex> lk(g_prof_mu);
            if (i < 0 || i >= (int64_t)g_prof.size()) return TRSM_STATUS_INVALID_VALUE;
            r = g_prof[(size_t)i];
        }
        if (hipEventSynchronize(r.stop) != hipSuccess) return TRSM_STATUS_HIP_ERROR;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return TRSM_STATUS_HIP_ERROR;
        *rec = r.r;
        rec->ms = ms;
        return TRSM_STATUS_SUCCESS;
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

int trsm_lln_select_ib(trsm_dtype_t dtype, int64_t m, int64_t n) {
    if (!valid_dtype(dtype) || m < 0 || n < 0) return 0;
    return select_ib(dtype, m, n);
}

const char *trsm_status_string(trsm_status_t status) {
    switch (status) {
        case TRSM_STATUS_SUCCESS: return "success";
        case TRSM_STATUS_INVALID_VALUE: return "invalid value";
        case TRSM_STATUS_ALLOC_FAILED: return "workspace allocation failed";
        case TRSM_STATUS_HIP_ERROR: return "HIP runtime error";
        case TRSM_STATUS_NOT_SUPPORTED: return "not supported";
        default: return "unknown status";
    }
}

trsm_status_t trsm_release_workspace(void) {
    try {
        // Slots are taken one at a time (never two locks together), and
        // g_mu is not held while waiting for a slot: a call holding a slot
        // may still need g_mu or a second slot.
        std::vector<std::pair<int, WsSlot *>> slots;
        {
            std::lock_guard<std::mutex> lk(g_mu);
            for (auto &kv : g_ws) slots.emplace_back(std::get<0>(kv.first), kv.second.get());
        }
        trsm_status_t s = TRSM_STATUS_SUCCESS;
        int cur = 0;
        const bool have_cur = hipGetDevice(&cur) == hipSuccess;
        for (auto &ds : slots) {
            std::lock_guard<std::mutex> lk(ds.second->mu);
            if (!ds.second->ptr) continue;
            if (hipSetDevice(ds.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
                s = TRSM_STATUS_HIP_ERROR;
            (void)hipFree(ds.second->ptr);
            ds.second->ptr = nullptr;
            ds.second->bytes = 0;
        }
        if (have_cur) (void)hipSetDevice(cur);
        return s;
    } catch (...) {
        return TRSM_STATUS_HIP_ERROR;
    }
}

}  // extern "C"
