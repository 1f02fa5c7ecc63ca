// api.hip -- host side of libsvgear.so: argument validation, workspace layout
// and the C entry points declared in include/svgear.h.  Every check runs before
// anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include "internal.h"

#define SVG_API extern "C" __attribute__((visibility("default")))

namespace svg {

SVG_HIDDEN size_t elem_bytes(int dtype) { return dtype == SVGEAR_BF16 ? 2 : 4; }

SVG_HIDDEN Layout make_layout(const svgear_shape& s)
{
    Layout L;
    memset(&L, 0, sizeof(L));
    const size_t H = s.H, Nq = s.Nq, Nk = s.Nk, d = s.d, Cq = s.Cq, Ck = s.Ck;
    const size_t eb = elem_bytes(s.dtype);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.labels_q = take(H * Nq * 4);
    L.qbar = take(H * Cq * d * 4);
    L.counts_q = take(H * Cq * 4);
    L.offsets_q = take(H * (Cq + 1) * 4);
    L.perm_q = take(H * Nq * 4);
    L.inv_perm_q = take(H * Nq * 4);
    L.Qp = take(H * Nq * d * eb);
    L.labels_k = take(H * Nk * 4);
    L.kbar = take(H * Ck * d * 4);
    L.vbar = take(H * Ck * d * 4);
    L.counts_k = take(H * Ck * 4);
    L.offsets_k = take(H * (Ck + 1) * 4);
    L.perm_k = take(H * Nk * 4);
    L.inv_perm_k = take(H * Nk * 4);
    L.Kp = take(H * Nk * d * eb);
    L.Vp = take(H * Nk * d * eb);
    L.log_ratio = take(H * Cq * Ck * 4);
    L.mask = take(H * Cq * Ck);
    L.sel_cost = take(H * 8);
    L.errs = take(256);   // device error words: [0] K side / stage calls, [16] Q side of svgear_forward
    L.scratch = off;

    // cluster scratch (sized for the larger side)
    const size_t N = Nq > Nk ? Nq : Nk, C = Cq > Ck ? Cq : Ck;
    const size_t ntiles = (N + kTile - 1) / kTile;
    off = 0;
    L.cl_cent64 = take(H * C * d * 8);
    L.cl_hi = take(H * C * d * 2);
    L.cl_lo = take(H * C * d * 2);
    L.cl_cnorm = take(H * C * 4);
    L.cl_cn64 = take(H * C * 8);
    L.cl_stats = take(H * 16);
    L.cl_flag = take(H * N * 4);
    L.cl_nflag = take(H * 4);
    L.cl_hist = take(H * ntiles * C * 4);
    L.cl_perm = take(H * N * 4);
    L.cl_sums = take(2 * H * C * d * 8);
    L.cl_range = take(H * kRangeStride * 4);
    L.cl_resid = take(H * C * 4);
    L.cl_labprev = take(H * N * 4);
    L.cl_bounds = take(3 * H * N * 4);
    L.cl_changed = take(H * C * 4);
    L.cl_moved = take(H * C * 4);
    L.cl_mlist = take(H * C * 4);
    L.cl_mpos = take(H * C * 4);
    L.cl_mcount = take(H * 4);
    L.cl_perm2 = take(H * N * 4);            // the previous update's bucket order
    L.cl_offs = take(2 * H * (C + 1) * 4);   // bucket offsets, current and previous
    L.cl_tokflag = take(H * N);              // per token: label changed in the last assignment
    L.cl_ipos = take(2 * H * N * 4);         // per token: its position in the current / previous bucket order
    L.cl_fpos = take(2 * H * N);             // the token flags by position in those orders
    L.cl_end = off;

    off = 0;
    L.pr_sbar = take(H * Cq * Ck * 4);
    L.pr_keys = take(H * Nk * 8);
    L.pr_pg = take(H * Ck * 4);
    L.pr_ctr = take(2 * H * 4);   // claim counters of the MFMA probe, per head and column slice
    L.pr_end = off;

    off = 0;
    // per-head states and histograms (one launch per pass, cleared together),
    // then the per-slice top-digit histograms and the digit words of the
    // two-launch route
    L.rt_state = take(H * 24);
    L.rt_hist = take(H * 4096 * 8);
    L.rt_top = take(route_top_bytes((int)H, (int)(s.Cq * s.Ck)));
    L.rt_part = take(H * 32 * 8);
    L.rt_end = off;

    off = 0;
    L.at_kvplanes = take(3 * H * Ck * d * 2);
    L.at_logm = take(H * Ck * 4);
    L.at_tiles = take(H * (Cq + 1) * 4 + 256);
    L.at_segs = take(H * Cq * Ck * 8);
    L.at_cinfo = take(H * Cq * 16);
    L.at_comp = take(H * Cq * Ck * 4);
    L.at_rows = take((size_t)kAttnSlots * Nk * 4);   // one routed-key row list per attention workgroup
    // work queues: meta (count, start, counter per XCD class), per-head class
    // counts and in-class prefixes, the queue itself (at most H (ceil(Nq / rows) + Cq) tiles)
    L.at_queue = take((3 * kXcd + H * kXcd + H * Cq + H * ((Nq + kAttnRows - 1) / kAttnRows + Cq)) * 4);
    L.at_end = off;

    size_t sc = L.cl_end;
    if (L.pr_end > sc) sc = L.pr_end;
    if (L.rt_end > sc) sc = L.rt_end;
    if (L.at_end > sc) sc = L.at_end;
    L.scratch2 = L.scratch + align256(sc);
    L.total = L.scratch2 + L.cl_end;
    return L;
}

// One side stream (default priority, non-blocking) and a fork/join event pair
// per device, created on first use and kept for the life of the process.  The
// mutex serialises the record/wait sequence of concurrent host callers.
struct SideStream {
    hipStream_t stream;
    hipEvent_t fork, join;
    std::mutex mu;
};

static SideStream* side_stream()
{
    constexpr int kMaxDev = 64;
    static SideStream g_side[kMaxDev];
    static bool g_ready[kMaxDev];
    static std::mutex g_init;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    std::lock_guard<std::mutex> lock(g_init);
    if (!g_ready[dev]) {
        SideStream& s = g_side[dev];
        if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess) {
            (void)hipStreamDestroy(s.stream);
            return nullptr;
        }
        g_ready[dev] = true;
    }
    return &g_side[dev];
}

SVG_HIDDEN int read_device_error(const int* err, hipStream_t st)
{
    int v = 0;
    if (hipMemcpyAsync(&v, err, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return -1;
    if (hipStreamSynchronize(st) != hipSuccess) return -1;
    return v;
}


}  // namespace svg

using namespace svg;

static int check_shape(const svgear_shape* s)
{
    if (!s) return SVGEAR_E_NULL;
    if (s->dtype != SVGEAR_F32 && s->dtype != SVGEAR_BF16) return SVGEAR_E_DTYPE;
    if (s->H < 1 || s->H > 65535) return SVGEAR_E_SHAPE;
    if (s->Nq < 1 || s->Nq > kMaxN || s->Nk < 1 || s->Nk > kMaxN) return SVGEAR_E_SHAPE;
    if (s->d != 64 && s->d != 128) return SVGEAR_E_SHAPE;
    if (s->Cq < 1 || s->Cq > s->Nq || s->Cq > kMaxC) return SVGEAR_E_SHAPE;
    if (s->Ck < 1 || s->Ck > s->Nk || s->Ck > kMaxC) return SVGEAR_E_SHAPE;
    if (s->iters < 1 || s->iters > 100) return SVGEAR_E_SHAPE;
    return SVGEAR_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validates a list of device pointers: all non-NULL and 16-byte aligned.
static int check_ptrs(std::initializer_list<const void*> ps)
{
    for (const void* p : ps)
        if (!p) return SVGEAR_E_NULL;
    for (const void* p : ps)
        if (!aligned(p, 16)) return SVGEAR_E_ALIGN;
    return SVGEAR_OK;
}

static int check_ws(const svgear_shape* s, void* ws, size_t ws_bytes, Layout* L)
{
    *L = make_layout(*s);
    if (!ws) return SVGEAR_E_NULL;
    if (!aligned(ws, 256)) return SVGEAR_E_ALIGN;
    if (ws_bytes < L->total) return SVGEAR_E_WORKSPACE;
    return SVGEAR_OK;
}

// Status of a device error word: out-of-range data first, then invalid indices.
static int device_status(int v)
{
    if (v < 0) return SVGEAR_E_HIP;
    if (v & ERR_RANGE) return SVGEAR_E_RANGE;
    if (v != 0) return SVGEAR_E_ARG;
    return SVGEAR_OK;
}

static int finish(hipError_t e, int flags, hipStream_t st, const int* err_word)
{
    if (e != hipSuccess) return SVGEAR_E_HIP;
    if (flags & SVGEAR_DEBUG_SYNC) {
        if (hipStreamSynchronize(st) != hipSuccess) return SVGEAR_E_HIP;
        if (err_word) return device_status(read_device_error(err_word, st));
    }
    return SVGEAR_OK;
}

SVG_API int svgear_version(void) { return 20000; }

SVG_API const char* svgear_status_string(int code)
{
    switch (code) {
    case SVGEAR_OK: return "ok";
    case SVGEAR_E_NULL: return "a required pointer is NULL";
    case SVGEAR_E_SHAPE: return "a size is out of range";
    case SVGEAR_E_DTYPE: return "unknown element type";
    case SVGEAR_E_ALIGN: return "a pointer is misaligned";
    case SVGEAR_E_WORKSPACE: return "workspace too small";
    case SVGEAR_E_RHO: return "rho must be in [0, 1]";
    case SVGEAR_E_HIP: return "HIP runtime error";
    case SVGEAR_E_ARG: return "invalid argument";
    case SVGEAR_E_RANGE: return "input values out of the supported range";
    default: return "unknown status";
    }
}

SVG_API int svgear_workspace_bytes(const svgear_shape* shape, size_t* bytes)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!bytes) return SVGEAR_E_NULL;
    *bytes = make_layout(*shape).total;
    return SVGEAR_OK;
}

// Byte offset, in the workspace's error region, of the Q-side word of svgear_forward.
constexpr size_t kErrQ = 64;

static int cluster_impl(const svgear_shape* shape, int side, const void* X, const void* V,
                        const int32_t* init_idx, int flags, int32_t* labels, float* cent,
                        float* vbar, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, void* Xp, void* Vp, void* ws, const Layout& L,
                        hipStream_t st, size_t scratch_off = 0, size_t err_off = 0)
{
    ClusterArgs a;
    a.H = shape->H;
    a.N = side == 0 ? shape->Nq : shape->Nk;
    a.C = side == 0 ? shape->Cq : shape->Ck;
    a.d = shape->d;
    a.iters = shape->iters;
    a.dtype = shape->dtype;
    a.side = side;
    a.flags = flags;
    a.X = X;
    a.V = V;
    a.init = init_idx;
    a.labels = labels;
    a.cent = cent;
    a.vbar = vbar;
    a.counts = counts;
    a.offsets = offsets;
    a.perm = perm;
    a.inv_perm = inv_perm;
    a.Xp = Xp;
    a.Vp = Vp;
    a.scratch = (char*)ws + (scratch_off ? scratch_off : L.scratch);
    a.err = (int*)((char*)ws + L.errs + err_off);
    a.L = &L;
    zero_words(a.err, 64, st);
    hipError_t e = launch_cluster(a, st);
    return finish(e, flags, st, a.err);
}

SVG_API int svgear_cluster(const svgear_shape* shape, int side, const void* X, const void* V,
                           const int32_t* init_idx, int flags, int32_t* labels, float* cent,
                           float* vbar, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv_perm, void* Xp, void* Vp, void* ws, size_t ws_bytes,
                           void* stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (side != 0 && side != 1) return SVGEAR_E_ARG;
    if (flags & ~(SVGEAR_LABELS_GIVEN | SVGEAR_DEBUG_SYNC)) return SVGEAR_E_ARG;
    rc = check_ptrs({X, labels, cent, counts, offsets, perm, inv_perm, Xp});
    if (rc) return rc;
    if (!(flags & SVGEAR_LABELS_GIVEN) && !init_idx) return SVGEAR_E_NULL;
    if (init_idx && !aligned(init_idx, 4)) return SVGEAR_E_ALIGN;
    if (side == 1) {
        rc = check_ptrs({V, vbar, Vp});
        if (rc) return rc;
    } else if (V || vbar || Vp) {
        return SVGEAR_E_ARG;
    }
    Layout L;
    rc = check_ws(shape, ws, ws_bytes, &L);
    if (rc) return rc;
    return cluster_impl(shape, side, X, V, init_idx, flags, labels, cent, vbar, counts, offsets,
                        perm, inv_perm, Xp, Vp, ws, L, (hipStream_t)stream);
}

static int probe_impl(const svgear_shape* shape, const float* qbar, const int32_t* counts_q,
                      const void* Kp, const void* Vp, const float* kbar, const float* vbar,
                      const int32_t* counts_k, const int32_t* offsets_k, int flags,
                      float* log_ratio, float* log_eps2, char* scratch, const Layout& L,
                      hipStream_t st)
{
    ProbeArgs a;
    a.H = shape->H;
    a.Nk = shape->Nk;
    a.d = shape->d;
    a.Cq = shape->Cq;
    a.Ck = shape->Ck;
    a.dtype = shape->dtype;
    a.flags = flags;
    a.qbar = qbar;
    a.counts_q = counts_q;
    a.Kp = Kp;
    a.Vp = Vp;
    a.kbar = kbar;
    a.vbar = vbar;
    a.counts_k = counts_k;
    a.offsets_k = offsets_k;
    a.log_ratio = log_ratio;
    a.log_eps2 = log_eps2;
    a.scratch = scratch;
    a.L = &L;
    hipError_t e = launch_probe(a, st);
    return finish(e, flags, st, nullptr);
}

static int check_probe_args(const svgear_shape* shape, const float* qbar, const int32_t* counts_q,
                            const void* Kp, const void* Vp, const float* kbar, const float* vbar,
                            const int32_t* counts_k, const int32_t* offsets_k, int flags,
                            const float* log_ratio, const float* log_eps2)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (flags & ~(SVGEAR_DEBUG_EPS | SVGEAR_DEBUG_SYNC | SVGEAR_PROBE_LOGIT | SVGEAR_PROBE_SCORE))
        return SVGEAR_E_ARG;
    if ((flags & SVGEAR_PROBE_SCORE) && (flags & (SVGEAR_PROBE_LOGIT | SVGEAR_DEBUG_EPS)))
        return SVGEAR_E_ARG;
    rc = check_ptrs({qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, log_ratio});
    if (rc) return rc;
    if (flags & SVGEAR_DEBUG_EPS) {
        rc = check_ptrs({log_eps2});
        if (rc) return rc;
    }
    return SVGEAR_OK;
}

SVG_API int svgear_probe(const svgear_shape* shape, const float* qbar, const int32_t* counts_q,
                         const void* Kp, const void* Vp, const float* kbar, const float* vbar,
                         const int32_t* counts_k, const int32_t* offsets_k, int flags,
                         float* log_ratio, float* log_eps2, void* ws, size_t ws_bytes,
                         void* stream)
{
    int rc = check_probe_args(shape, qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, flags,
                              log_ratio, log_eps2);
    if (rc) return rc;
    Layout L;
    rc = check_ws(shape, ws, ws_bytes, &L);
    if (rc) return rc;
    return probe_impl(shape, qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, flags,
                      log_ratio, log_eps2, (char*)ws + L.scratch, L, (hipStream_t)stream);
}

// ----------------------------------------------------------------------------- svgear_probe_noalloc
//
// The probe's scratch (its sbar table and, on the generic path, the per-key
// value terms) in a file-scope device array instead of a caller workspace.
// Each device that runs the library holds its own copy until the process ends.
// Its address on a device is fetched once, with that device current, and kept
// per device: host code never passes the array's own name to a kernel.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

static char* noalloc_scratch()
{
    constexpr int kMaxDev = 64;
    static char* g_ptr[kMaxDev];
    static std::mutex g_mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = (char*)p;
    }
    return g_ptr[dev];
}

SVG_API int svgear_probe_noalloc(const svgear_shape* shape, const float* qbar, const int32_t* counts_q,
                                 const void* Kp, const void* Vp, const float* kbar, const float* vbar,
                                 const int32_t* counts_k, const int32_t* offsets_k, int flags,
                                 float* log_ratio, float* log_eps2, void* stream)
{
    int rc = check_probe_args(shape, qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, flags,
                              log_ratio, log_eps2);
    if (rc) return rc;
    const Layout L = make_layout(*shape);
    if (L.pr_end > kNoAllocScratchBytes) return SVGEAR_E_WORKSPACE;
    char* base = noalloc_scratch();
    if (!base) return SVGEAR_E_HIP;
    return probe_impl(shape, qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, flags, log_ratio,
                      log_eps2, base, L, (hipStream_t)stream);
}

static int64_t budget_of(double rho, int Nq, int Nk)
{
    return (int64_t)floor((rho * (double)Nq) * (double)Nk);
}

SVG_API int svgear_route(const svgear_shape* shape, double rho, const float* log_ratio,
                         const int32_t* counts_q, const int32_t* counts_k, uint8_t* mask,
                         int64_t* sel_cost, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!(rho >= 0.0 && rho <= 1.0)) return SVGEAR_E_RHO;
    rc = check_ptrs({log_ratio, counts_q, counts_k, mask, sel_cost});
    if (rc) return rc;
    Layout L;
    rc = check_ws(shape, ws, ws_bytes, &L);
    if (rc) return rc;
    RouteArgs a;
    a.H = shape->H;
    a.Cq = shape->Cq;
    a.Ck = shape->Ck;
    a.budget = budget_of(rho, shape->Nq, shape->Nk);
    a.log_ratio = log_ratio;
    a.counts_q = counts_q;
    a.counts_k = counts_k;
    a.mask = mask;
    a.sel_cost = sel_cost;
    a.scratch = (char*)ws + L.scratch;
    a.L = &L;
    return finish(launch_route(a, (hipStream_t)stream), 0, (hipStream_t)stream, nullptr);
}

SVG_API int svgear_route_rows(const svgear_shape* shape, double rho, const float* log_ratio,
                              const int32_t* counts_q, const int32_t* counts_k, uint8_t* mask,
                              int64_t* sel_cost, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!(rho >= 0.0 && rho <= 1.0)) return SVGEAR_E_RHO;
    rc = check_ptrs({log_ratio, counts_q, counts_k, mask, sel_cost});
    if (rc) return rc;
    Layout L;
    rc = check_ws(shape, ws, ws_bytes, &L);
    if (rc) return rc;
    RouteArgs a;
    a.H = shape->H;
    a.Cq = shape->Cq;
    a.Ck = shape->Ck;
    a.budget = 0;
    a.log_ratio = log_ratio;
    a.counts_q = counts_q;
    a.counts_k = counts_k;
    a.mask = mask;
    a.sel_cost = sel_cost;
    return finish(launch_route_rows(a, rho, shape->Nk, (hipStream_t)stream), 0, (hipStream_t)stream,
                  nullptr);
}

static int attention_impl(const svgear_shape* shape, const void* Qp, const int32_t* offsets_q,
                          const int32_t* perm_q, const void* Kp, const void* Vp, const float* kbar,
                          const float* vbar, const int32_t* counts_k, const int32_t* offsets_k,
                          const uint8_t* mask, void* O, void* ws, const Layout& L, int flags,
                          hipStream_t st)
{
    AttnArgs a;
    a.H = shape->H;
    a.Nq = shape->Nq;
    a.Nk = shape->Nk;
    a.d = shape->d;
    a.Cq = shape->Cq;
    a.Ck = shape->Ck;
    a.dtype = shape->dtype;
    a.Qp = Qp;
    a.offsets_q = offsets_q;
    a.perm_q = perm_q;
    a.Kp = Kp;
    a.Vp = Vp;
    a.kbar = kbar;
    a.vbar = vbar;
    a.counts_k = counts_k;
    a.offsets_k = offsets_k;
    a.mask = mask;
    a.O = O;
    a.scratch = (char*)ws + L.scratch;
    a.L = &L;
    return finish(launch_attention(a, st), flags, st, nullptr);
}

SVG_API int svgear_attention(const svgear_shape* shape, const void* Qp, const int32_t* offsets_q,
                             const int32_t* perm_q, const void* Kp, const void* Vp,
                             const float* kbar, const float* vbar, const int32_t* counts_k,
                             const int32_t* offsets_k, const uint8_t* mask, void* O, void* ws,
                             size_t ws_bytes, void* stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    rc = check_ptrs({Qp, offsets_q, perm_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, mask, O});
    if (rc) return rc;
    Layout L;
    rc = check_ws(shape, ws, ws_bytes, &L);
    if (rc) return rc;
    return attention_impl(shape, Qp, offsets_q, perm_q, Kp, Vp, kbar, vbar, counts_k, offsets_k,
                          mask, O, ws, L, 0, (hipStream_t)stream);
}

SVG_API int svgear_forward(const svgear_shape* shape, double rho, const void* Q, const void* K,
                           const void* V, const int32_t* init_q, const int32_t* init_k, void* O,
                           const svgear_intermediates* im, int flags, void* ws, size_t ws_bytes,
                           void* stream)
{
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!(rho >= 0.0 && rho <= 1.0)) return SVGEAR_E_RHO;
    if (flags & ~SVGEAR_DEBUG_SYNC) return SVGEAR_E_ARG;
    rc = check_ptrs({Q, K, V, init_q, init_k, O});
    if (rc) return rc;
    Layout L;
    rc = check_ws(shape, ws, ws_bytes, &L);
    if (rc) return rc;
    svgear_intermediates I;
    memset(&I, 0, sizeof(I));
    if (im) I = *im;
    char* w = (char*)ws;
#define SVG_PICK(field, type)                                      \
    type field = I.field ? (type)I.field : (type)(w + L.field);    \
    if (!aligned((const void*)field, 16)) return SVGEAR_E_ALIGN;
    SVG_PICK(labels_q, int32_t*)
    SVG_PICK(qbar, float*)
    SVG_PICK(counts_q, int32_t*)
    SVG_PICK(offsets_q, int32_t*)
    SVG_PICK(perm_q, int32_t*)
    SVG_PICK(inv_perm_q, int32_t*)
    SVG_PICK(Qp, void*)
    SVG_PICK(labels_k, int32_t*)
    SVG_PICK(kbar, float*)
    SVG_PICK(vbar, float*)
    SVG_PICK(counts_k, int32_t*)
    SVG_PICK(offsets_k, int32_t*)
    SVG_PICK(perm_k, int32_t*)
    SVG_PICK(inv_perm_k, int32_t*)
    SVG_PICK(Kp, void*)
    SVG_PICK(Vp, void*)
    SVG_PICK(log_ratio, float*)
    SVG_PICK(mask, uint8_t*)
    SVG_PICK(sel_cost, int64_t*)
#undef SVG_PICK
    hipStream_t st = (hipStream_t)stream;
    // The two clusterings are independent: Q's runs on a side stream (its own
    // scratch) while K's runs on the caller's stream, then the caller's stream
    // waits for the side stream.
    SideStream* ss = side_stream();
    if (ss) {
        std::lock_guard<std::mutex> lock(ss->mu);
        if (hipEventRecord(ss->fork, st) != hipSuccess ||
            hipStreamWaitEvent(ss->stream, ss->fork, 0) != hipSuccess)
            return SVGEAR_E_HIP;
        const int rq = cluster_impl(shape, 0, Q, nullptr, init_q, 0, labels_q, qbar, nullptr,
                                    counts_q, offsets_q, perm_q, inv_perm_q, Qp, nullptr, ws, L,
                                    ss->stream, L.scratch2, kErrQ);
        const bool joined = hipEventRecord(ss->join, ss->stream) == hipSuccess;
        const int rk = cluster_impl(shape, 1, K, V, init_k, 0, labels_k, kbar, vbar, counts_k,
                                    offsets_k, perm_k, inv_perm_k, Kp, Vp, ws, L, st);
        if (!joined || hipStreamWaitEvent(st, ss->join, 0) != hipSuccess) return SVGEAR_E_HIP;
        if (rq) return rq;
        if (rk) return rk;
    } else {
        rc = cluster_impl(shape, 0, Q, nullptr, init_q, 0, labels_q, qbar, nullptr, counts_q,
                          offsets_q, perm_q, inv_perm_q, Qp, nullptr, ws, L, st, 0, kErrQ);
        if (rc) return rc;
        rc = cluster_impl(shape, 1, K, V, init_k, 0, labels_k, kbar, vbar, counts_k, offsets_k,
                          perm_k, inv_perm_k, Kp, Vp, ws, L, st);
        if (rc) return rc;
    }
    rc = probe_impl(shape, qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, 0, log_ratio,
                    nullptr, w + L.scratch, L, st);
    if (rc) return rc;
    RouteArgs ra;
    ra.H = shape->H;
    ra.Cq = shape->Cq;
    ra.Ck = shape->Ck;
    ra.budget = budget_of(rho, shape->Nq, shape->Nk);
    ra.log_ratio = log_ratio;
    ra.counts_q = counts_q;
    ra.counts_k = counts_k;
    ra.mask = mask;
    ra.sel_cost = sel_cost;
    ra.scratch = w + L.scratch;
    ra.L = &L;
    if (launch_route(ra, st) != hipSuccess) return SVGEAR_E_HIP;
    rc = attention_impl(shape, Qp, offsets_q, perm_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, mask,
                        O, ws, L, 0, st);
    if (rc || !(flags & SVGEAR_DEBUG_SYNC)) return rc;
    // Device-detected data errors of both clusterings (K side word first).
    if (hipStreamSynchronize(st) != hipSuccess) return SVGEAR_E_HIP;
    const int* err = (const int*)(w + L.errs);
    const int ek = read_device_error(err, st);
    const int eq = read_device_error((const int*)((const char*)err + kErrQ), st);
    if (ek < 0 || eq < 0) return SVGEAR_E_HIP;
    return device_status(ek | eq);
}
