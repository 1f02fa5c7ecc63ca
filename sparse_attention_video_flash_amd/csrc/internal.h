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

// Exact fixed-point image of an input value.  x * 2^S is formed exactly in
// fp64 and added to 1.5 * 2^52, which rounds it to the nearest integer (an exact
// operation whenever x is a multiple of 2^-S, i.e. every input of magnitude at
// least 2^(-S+7) for bf16 or 2^(-S+23) for fp32, and |x| < 2^(51 - S)); the
// integer is read from the low bits.  Accumulating the raw bit patterns and
// subtracting count * bits(1.5 * 2^52) once at the end gives the sum of the
// integers modulo 2^64, which is the exact sum while it fits in 63 bits.
constexpr double kFixMagic = 6755399441055744.0;               // 1.5 * 2^52
constexpr unsigned long long kFixMagicBits = 0x4338000000000000ull;
template <typename T>
__device__ __forceinline__ unsigned long long fixed_bits(T x, double scale)
{
    return (unsigned long long)__double_as_longlong(fma((double)to_f32<T>(x), scale, kFixMagic));
}

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
constexpr int kMaxC = 4096;         // largest cluster count
constexpr int kAttnRows = 256;      // query rows per attention tile (bf16, d = 128 kernel)
constexpr int kXcd = 8;             // XCDs per device: attention work queues
constexpr int kMaxN = 1 << 20;      // largest token count

// Fixed-point scale 2^S of the exact centroid sums: |x| < 2^8 and N < 2^lgN give
// |sum| < 2^(8 + lgN + S) <= 2^62.
inline int fixed_point_shift(int N)
{
    int lg = 0;
    while ((1 << lg) <= N) ++lg;   // N < 2^lg
    return 62 - 8 - lg;
}

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
    size_t log_ratio, mask, sel_cost;
    size_t scratch;  // start of the per-stage scratch
    // cluster scratch (relative to scratch)
    size_t cl_err, cl_cent64, cl_hi, cl_lo, cl_cnorm, cl_cn64, cl_stats, cl_flag, cl_nflag,
        cl_hist, cl_perm, cl_sums, cl_resid, cl_labprev, cl_bounds, cl_changed, cl_moved,
        cl_mlist, cl_mpos, cl_mcount;
    size_t cl_end;
    // probe scratch (relative to scratch)
    size_t pr_err, pr_qplanes, pr_sbar, pr_keys, pr_pg;
    size_t pr_end;
    // attention scratch (relative to scratch)
    size_t at_err, at_kvplanes, at_logm, at_tiles, at_segs, at_nsegs, at_nkeys, at_comp, at_ncomp,
        at_rowmap, at_queue;
    size_t at_end;
    size_t scratch2;  // second cluster scratch (absolute offset)
    size_t total;
};

SVG_HIDDEN Layout make_layout(const svgear_shape& s);
SVG_HIDDEN size_t elem_bytes(int dtype);

// ----------------------------------------------------------------------------- launchers

struct ClusterArgs {
    int H, N, d, C, iters, dtype, side, flags, shift;
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
SVG_HIDDEN hipError_t launch_assign_mfma(const ClusterArgs& a, const double* cent64,
                                         const KmPlanes& P, bool partial, hipStream_t st);
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
};
SVG_HIDDEN hipError_t launch_route(const RouteArgs& a, hipStream_t st);
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
