// internal.h -- shared definitions of the svgear HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "svgear.h"

#define SVG_HIDDEN __attribute__((visibility("hidden")))

namespace svg {

using bf16 = uint16_t;

// ----------------------------------------------------------------------------- element types

__host__ __device__ __forceinline__ float bf16_to_f32(bf16 b)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)b << 16;
    return v.f;
}

// Round to nearest even; inputs are finite.
__host__ __device__ __forceinline__ bf16 f32_to_bf16(float f)
{
    union { uint32_t u; float f; } v;
    v.f = f;
    uint32_t u = v.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return bf16_to_f32(x); }

// Exact centroid sums.  For a head whose largest input magnitude is below 2^E,
// every value is scaled by 2^S (S = B - E, B = min(51, 62 - ceil(log2(N+1))))
// and split exactly into the nearest integer a and the remainder r = x 2^S - a
// (|r| <= 1/2); a and r 2^B are each turned into a 64-bit integer by the fp64
// magic-number add (exact: |a| < 2^51 and |r 2^B| < 2^51).  The second integer
// is exact whenever x is a multiple of 2^-(S+B), which holds for every value
// whose unit in the last place is at least that (checked once per head from the
// smallest non-zero magnitude; see fix_exact).  Both integers are summed
// modulo 2^64 in any order; the sums stay below 2^62 in magnitude, so they are
// the exact sums of the images, and the total is (hi + lo 2^-B) 2^-S.
constexpr double kFixMagic = 6755399441055744.0;               // 1.5 * 2^52
constexpr unsigned long long kFixMagicBits = 0x4338000000000000ull;
constexpr int kFixMaxExp = 56;   // supported inputs: finite with |x| < 2^56

// B for N tokens (host and device).
__host__ __device__ __forceinline__ int fix_base(int N)
{
    int lg = 0;
    while (lg < 31 && (1 << lg) <= N) ++lg;   // N < 2^lg
    return (62 - lg) < 51 ? (62 - lg) : 51;
}

// Smallest E with |x| < 2^E from the largest magnitude's fp32 bits (0 for an
// all-zero head; capped at kFixMaxExp, which fix_exact reports as out of range).
__device__ __forceinline__ int fix_exp(unsigned maxbits)
{
    if (maxbits == 0u) return 0;
    const int ef = (int)(maxbits >> 23);
    const int e = ef == 0 ? -126 : ef - 126;
    return e > kFixMaxExp ? kFixMaxExp : e;
}

// Per-head range words (fp32 bit patterns of magnitudes, updated with
// atomicMax on zero-initialised memory): w[0] = largest |x|, w[1] = ~(smallest
// non-zero |x| - 1) (0 while no non-zero value was seen).
// Whether the split above is exact for every value of the head, and the head
// is inside the supported range (finite, |x| < 2^kFixMaxExp).  prec: 8 (bf16)
// or 24 (fp32) significant bits.
__device__ __forceinline__ bool fix_exact(const unsigned* w, int base, int prec)
{
    const unsigned mx = w[0];
    if (mx >= 0x7F800000u) return false;                       // inf or NaN
    if (mx != 0u && (int)(mx >> 23) - 127 >= kFixMaxExp) return false;
    if (w[1] == 0u) return true;                               // all zeros
    const unsigned mn = ~w[1] + 1u;                            // smallest non-zero |x|
    const int ef = (int)(mn >> 23);
    const int ulp_e = (ef == 0 ? -126 : ef - 127) - (prec - 1);
    const int S = base - fix_exp(mx);
    return ulp_e >= -(S + base);
}

// The first integer image alone (magic-offset bits), for a head whose values
// all have a unit in the last place of at least 2^-S.
template <typename T>
__device__ __forceinline__ unsigned long long fix_hi(T x, double s)
{
    return (unsigned long long)__double_as_longlong(fma((double)to_f32<T>(x), s, kFixMagic));
}

// Adds the two integer images of x (scale s = 2^S, t = 2^B) to hi and lo.
template <typename T>
__device__ __forceinline__ void fix_add(T x, double s, double t, unsigned long long& hi,
                                        unsigned long long& lo)
{
    const double xv = (double)to_f32<T>(x);
    const double a = fma(xv, s, kFixMagic);          // magic + nearest integer of x 2^S
    const double r = fma(xv, s, kFixMagic - a);      // x 2^S - that integer, exactly
    hi += (unsigned long long)__double_as_longlong(a);
    lo += (unsigned long long)__double_as_longlong(fma(r, t, kFixMagic));
}

// Whether a head needs the remainder word at all: some non-zero value's unit in
// the last place lies below 2^-S (otherwise every image is exact in the first
// word and the second stays zero).  Needs the complete range words.
__device__ __forceinline__ bool fix_need_lo(const unsigned* w, int base, int prec)
{
    if (w[1] == 0u) return false;
    const unsigned mn = ~w[1] + 1u;
    const int ef = (int)(mn >> 23);
    const int ulp_e = (ef == 0 ? -126 : ef - 127) - (prec - 1);
    return ulp_e < fix_exp(w[0]) - base;
}

// Running range of bf16 data, two values per 32-bit word with packed 16-bit
// integer max/min: mx = largest magnitude, mn = smallest (magnitude - 1), so a
// zero (0xFFFF after the wrap) never wins the minimum.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
struct RangeBf16 {
    u16x2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
    __device__ __forceinline__ void add_max(unsigned w)
    {
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu));
    }
    __device__ __forceinline__ void add_min(unsigned w)
    {
        mn = __builtin_elementwise_min(mn, __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu) - u16x2_t{1, 1});
    }
    __device__ __forceinline__ void add(unsigned w)
    {
        const u16x2_t a = __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
        mx = __builtin_elementwise_max(mx, a);
        mn = __builtin_elementwise_min(mn, a - u16x2_t{1, 1});
    }
    // fp32-bit range words (see fix_exact)
    __device__ __forceinline__ unsigned max_word() const { return (unsigned)max(mx[0], mx[1]) << 16; }
    __device__ __forceinline__ unsigned min_word() const
    {
        const unsigned m = min(mn[0], mn[1]);
        return m == 0xFFFFu ? 0u : ~(((m + 1u) << 16) - 1u);
    }
};
// The same for fp32 data.
struct RangeF32 {
    unsigned mx = 0u, mn = 0u;
    __device__ __forceinline__ void add_max(unsigned w) { mx = max(mx, w & 0x7FFFFFFFu); }
    __device__ __forceinline__ void add_min(unsigned w) { mn = max(mn, ~((w & 0x7FFFFFFFu) - 1u)); }
    __device__ __forceinline__ void add(unsigned w)
    {
        const unsigned a = w & 0x7FFFFFFFu;
        mx = max(mx, a);
        mn = max(mn, ~(a - 1u));
    }
    __device__ __forceinline__ unsigned max_word() const { return mx; }
    __device__ __forceinline__ unsigned min_word() const { return mn; }
};
template <typename T> struct RangeOf;
template <> struct RangeOf<bf16> { using type = RangeBf16; };
template <> struct RangeOf<float> { using type = RangeF32; };

// Wave maxima of both words, then at most one atomic per wave and word (the
// minimum word only when the caller collected it).  The word is read first and
// the atomic issued only if it would raise it: once the first waves of a pass
// have recorded the head's extremes, the rest issue none (thousands of waves
// per head would otherwise serialise on the word in L2).
__device__ __forceinline__ void range_max_word(unsigned* w, unsigned v)
{
    if (v > __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(w, v);
}
__device__ __forceinline__ void range_commit(unsigned mx, unsigned mn, unsigned* w, bool with_min)
{
    for (int o = 32; o >= 1; o >>= 1) {
        mx = max(mx, (unsigned)__shfl_xor((int)mx, o));
        if (with_min) mn = max(mn, (unsigned)__shfl_xor((int)mn, o));
    }
    if ((threadIdx.x & 63) == 0) {
        range_max_word(w, mx);
        if (with_min) range_max_word(w + 1, mn);
    }
}

// Per-head range words: one 128-byte line per head ([0..1] of X, [2..3] of V).
constexpr int kRangeStride = 32;

// One probe term in log form: e = e^{2s} [em^2 P + 2 em Qd + R] with
// s = sbar - D, em = expm1(D), P = ||vbar||^2, Qd = vbar.(vbar - v),
// R = ||vbar - v||^2.  Returns x and f with e = e^x f.  For D > 0 the factor
// e^{-2D} is moved inside the bracket (x = 2 sbar, and with y = e^{-D},
// f = (1-y)^2 P + 2 y (1-y) Qd + y^2 R), so no intermediate overflows however
// far a key lies from its centroid.
__device__ __forceinline__ float probe_term(float sb, float dlt, float P, float Qd, float R, float& x)
{
    const bool pos = dlt > 0.f;
    const float em = expm1f(pos ? -dlt : dlt);  // in (-1, 0]
    const float y = 1.f + em;
    const float c1 = pos ? -2.f * em * y : 2.f * em;
    const float c2 = pos ? y * y : 1.f;
    x = 2.f * (pos ? sb : sb - dlt);
    return fmaxf(fmaf(em, em * P, fmaf(c1, Qd, c2 * R)), 0.f);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return f32_to_bf16(x); }

// ----------------------------------------------------------------------------- sizes

constexpr int kTile = 256;          // tokens per counting-sort / run-length tile
constexpr int kTileU = 2048;        // tokens per tile of the k-means' unstable bucket sorts
constexpr int kMaxC = 4096;         // largest cluster count
constexpr int kAttnRows = 256;      // query rows per attention tile (bf16, d = 128 kernel)
constexpr int kXcd = 8;             // XCDs per device: attention work queues
constexpr int kAttnSlots = 256;     // attention workgroups at most (one per CU), each with a row-list slot
constexpr int kMaxN = 1 << 20;      // largest token count

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device-detected invalid data (reported under SVGEAR_DEBUG_SYNC).
enum : int { ERR_INIT_INDEX = 1, ERR_LABEL = 2, ERR_RANGE = 4 };

// Workspace map.  [ intermediates of svgear_forward | stage scratch (union) |
// second cluster scratch ].  svgear_forward clusters Q in the second cluster
// scratch on a side stream while K is clustered in the first.
struct Layout {
    // forward intermediates
    size_t labels_q, qbar, counts_q, offsets_q, perm_q, inv_perm_q, Qp;
    size_t labels_k, kbar, vbar, counts_k, offsets_k, perm_k, inv_perm_k, Kp, Vp;
    size_t log_ratio, mask, sel_cost, errs;
    size_t scratch;  // start of the per-stage scratch
    // cluster scratch (relative to scratch)
    size_t cl_cent64, cl_hi, cl_lo, cl_cnorm, cl_cn64, cl_stats, cl_flag, cl_nflag,
        cl_hist, cl_perm, cl_sums, cl_range, cl_resid, cl_labprev, cl_bounds, cl_changed, cl_moved,
        cl_mlist, cl_mpos, cl_mcount, cl_perm2, cl_offs, cl_tokflag, cl_ipos, cl_fpos;
    size_t cl_end;
    // probe scratch (relative to scratch)
    size_t pr_sbar, pr_keys, pr_pg, pr_ctr;
    size_t pr_end;
    size_t rt_state, rt_hist, rt_top, rt_part, rt_end;   // route
    // attention scratch (relative to scratch)
    size_t at_kvplanes, at_logm, at_tiles, at_segs, at_cinfo, at_comp, at_rows, at_queue;
    size_t at_end;
    size_t scratch2;  // second cluster scratch (absolute offset)
    size_t total;
};

SVG_HIDDEN Layout make_layout(const svgear_shape& s);
SVG_HIDDEN size_t elem_bytes(int dtype);

// ----------------------------------------------------------------------------- launchers

struct ClusterArgs {
    int H, N, d, C, iters, dtype, side, flags;
    const void* X;
    const void* V;
    const int32_t* init;
    int32_t* labels;
    float* cent;
    float* vbar;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv_perm;
    void* Xp;
    void* Vp;
    char* scratch;      // cluster scratch base
    int* err;           // device error word (ERR_*), cleared by the caller
    const Layout* L;
};
SVG_HIDDEN hipError_t launch_cluster(const ClusterArgs& a, hipStream_t st);

// State of the MFMA k-means assignment (cluster scratch).
struct KmPlanes {
    bf16* hi;            // [H, C, d] bf16 hi plane of the fp64 centroids
    bf16* lo;            // [H, C, d] bf16 plane of the remainder
    float* cn32;         // [H, C] ||c||^2
    double* cn64;        // [H, C] ||c||^2
    unsigned* stats;     // [H, 4] split residual and ||c|| maxima (float bits)
    int32_t* flags;      // [H, N] tokens queued for the exact recheck
    int* nflag;          // [H]
    int* mlist;          // [H, C] centroids moved by the last update, ascending
    int* mpos;           // [H, C] position of a centroid in mlist, -1 if it did not move
    int* mcount;         // [H]
    float* ub_own;       // [H, N] upper bound of the distance to the own centroid
    float* lb_own;       // [H, N] lower bound of the same
    float* lb_rest;      // [H, N] lower bound of the distance to every other centroid
};
SVG_HIDDEN KmPlanes km_planes(const ClusterArgs& a);
SVG_HIDDEN hipError_t launch_km_prep(const ClusterArgs& a, const double* cent64, const KmPlanes& P,
                                     hipStream_t st);
// range: when non-NULL, the screen also records the per-head range words of X.
SVG_HIDDEN hipError_t launch_assign_mfma(const ClusterArgs& a, const double* cent64,
                                         const KmPlanes& P, bool partial, unsigned* range,
                                         hipStream_t st);
SVG_HIDDEN bool assign_mfma_supported(const ClusterArgs& a);

struct ProbeArgs {
    int H, Nk, d, Cq, Ck, dtype, flags;
    const float* qbar;
    const int32_t* counts_q;
    const void* Kp;
    const void* Vp;
    const float* kbar;
    const float* vbar;
    const int32_t* counts_k;
    const int32_t* offsets_k;
    float* log_ratio;
    float* log_eps2;
    char* scratch;
    const Layout* L;
};
SVG_HIDDEN hipError_t launch_probe(const ProbeArgs& a, hipStream_t st);

struct RouteArgs {
    int H, Cq, Ck;
    int64_t budget;
    const float* log_ratio;
    const int32_t* counts_q;
    const int32_t* counts_k;
    uint8_t* mask;
    int64_t* sel_cost;
    char* scratch;   // per-stage scratch (histograms and per-head states)
    const Layout* L;
};
SVG_HIDDEN hipError_t launch_route(const RouteArgs& a, hipStream_t st);
SVG_HIDDEN int route_slices(int H);
SVG_HIDDEN size_t route_top_bytes(int H, int nb);
SVG_HIDDEN hipError_t launch_route_rows(const RouteArgs& a, double rho, int Nk, hipStream_t st);
SVG_HIDDEN void zero_words(void* p, size_t bytes, hipStream_t st);

struct AttnArgs {
    int H, Nq, Nk, d, Cq, Ck, dtype;
    const void* Qp;
    const int32_t* offsets_q;
    const int32_t* perm_q;
    const void* Kp;
    const void* Vp;
    const float* kbar;
    const float* vbar;
    const int32_t* counts_k;
    const int32_t* offsets_k;
    const uint8_t* mask;
    void* O;
    char* scratch;
    const Layout* L;
};
SVG_HIDDEN hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

// Reads and clears the device error word of a stage scratch (synchronous).
SVG_HIDDEN int read_device_error(const int* err, hipStream_t st);

}  // namespace svg
