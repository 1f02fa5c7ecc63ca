// assign_mfma.hip -- k-means assignment on bf16 MFMA for d = 128 (step 1 of the
// SVG-EAR pipeline: Flash k-means; review page inference-pipeline paragraph).
//
// The nearest centroid minimises d_m = ||c_m||^2 - 2 x.c_m (||x||^2 is common to
// all m).  Tokens x are bf16 (exact as MFMA operands); each fp64 centroid is
// split into bf16 hi + lo planes, so the screen evaluates
//     d~_m = fl(cn_m - 2 * acc_m),   acc_m = sum_t x_t hi_mt + x_t lo_mt  (fp32 MFMA)
// with |d~_m - d_m| <= E(x), a bound built from:
//   the split residual      2 ||x|| R,       R = max_m ||c_m - hi_m - lo_m||,
//   the MFMA accumulation   2 * 16 instructions, each rounding its result once
//                           (the products of an instruction are summed before
//                           one rounding), counted twice for margin: 64 u
//                           ||x|| ||c||max, u = 2^-24, plus a 1% margin,
//   cn_m and the final fma  u (||c||max^2 + 2 ||x|| ||c||max) each.
// The true nearest centroid is then within 2E of the screen's best, so a token
// whose second-best screen distance is more than 2E above its best keeps the
// screen's label; otherwise it is queued and k_recheck settles it in fp64 with
// the oracle's exact arithmetic (sum of (x_t - c_t)^2 in coordinate order,
// lowest index on ties).  The labels therefore equal those of a direct fp64
// evaluation.
//
// Later iterations.  Every settled token keeps rigorous bounds (in the same
// ||c||^2 - 2 x.c units) on its true distance to its own centroid (upper and
// lower) and on the distance to every other centroid (lower).  A centroid that
// the last update left bit-identical keeps all its distances, so iteration
// t > 0 screens every token against the moved centroids only
// (k_assign_partial): the own centroid's bounds are refreshed if it moved, the
// moved others give fresh bounds, and the label is decided when one candidate's
// upper bound lies below every other lower bound; any other token goes to the
// exact recheck, which also refreshes its bounds exactly.
#include "internal.h"

namespace svg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int KM_D = 128;
constexpr int KM_PITCH = KM_D * 2 + 16;         // bytes per centroid row of a plane
constexpr int KM_TOK = 256;                     // tokens per workgroup (4 waves x 64)

// A chunk of CB centroids staged in LDS: the hi plane, with LO the lo plane
// after it, then ||c||^2 (fp32) per centroid.  NV: 16-byte vectors per thread.
template <int CB, bool LO>
struct KmChunk {
    static constexpr int PLANE = CB * KM_PITCH;
    static constexpr int NPL = LO ? 2 : 1;
    static constexpr int BYTES = NPL * PLANE + CB * 4;
    static constexpr int NV = NPL * CB / 16;
};
// The full screens stage 32 centroids per chunk, double-buffered (35 KB of LDS
// with both planes): with at most 168 VGPRs, three workgroups (12 waves) share a
// CU and hide each other's token loads.
template <bool LO>
struct KmScreen {
    static constexpr int CB = 32;
    using Chunk = KmChunk<CB, LO>;
    static constexpr int LDS = 2 * Chunk::BYTES;
};
// The partial screen: 32 moved centroids, both planes, single-buffered (three
// workgroups per CU as well; the 168-VGPR limit spills a few prologue values).
using KmPartialChunk = KmChunk<32, true>;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Outward rounding of fp32 bounds (covers the rounding of the one or two fp32
// operations that formed them); infinities stay.
__device__ __forceinline__ float bound_up(float x)
{
    return __builtin_isinf(x) ? x : x + (fabsf(x) * 0x1p-22f + 0x1p-100f);
}
__device__ __forceinline__ float bound_dn(float x)
{
    return __builtin_isinf(x) ? x : x - (fabsf(x) * 0x1p-22f + 0x1p-100f);
}

// The partial screen is used for a head when at most a quarter of its
// centroids moved: with more, a full screen costs about the same and its fresh
// bounds save exact rechecks (bounds folded over many moved centroids are loose).
__device__ __forceinline__ bool km_partial_pays(int moved, int C) { return 4 * moved <= C; }

// Screen error bound E(x) for a token of norm nx (see the file comment).
__device__ __forceinline__ float screen_error(float nx, float R, float cmax)
{
    const float u = 5.9604645e-8f;  // 2^-24
    const float xn = nx * 1.0001f;
    return 1.01f * (2.f * xn * R + 64.f * u * xn * cmax + 2.f * u * (cmax * cmax + 2.f * xn * cmax));
}

// Per centroid: bf16 hi/lo planes, ||c||^2 (fp32 and fp64) and the split
// residual norm; the per-head R and ||c||max follow from k_plane_stats (one
// workgroup per head: atomics on two words per head from every centroid
// serialised in L2).
__global__ __launch_bounds__(256) void k_km_prep(const double* __restrict__ cent64, int C,
                                                 bf16* __restrict__ hi, bf16* __restrict__ lo,
                                                 float* __restrict__ cn32,
                                                 double* __restrict__ cn64,
                                                 float* __restrict__ resid)
{
    // one wave per centroid, two coordinates per lane (the layout of the
    // update's finalize, which prepares the later screens the same way)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + wave, h = blockIdx.y;
    if (m >= C) return;   // wave-uniform
    double a2 = 0.0, r2s = 0.0;
#pragma unroll
    for (int e = 0; e < KM_D / 64; ++e) {
        const size_t i = ((size_t)h * C + m) * KM_D + lane * (KM_D / 64) + e;
        const double c = cent64[i];
        const bf16 ch = f32_to_bf16((float)c);
        const double r1 = c - (double)bf16_to_f32(ch);
        const bf16 cl = f32_to_bf16((float)r1);
        const double r2 = r1 - (double)bf16_to_f32(cl);
        hi[i] = ch;
        lo[i] = cl;
        a2 = fma(c, c, a2);
        r2s = fma(r2, r2, r2s);
    }
    for (int o = 32; o >= 1; o >>= 1) {
        a2 += __shfl_xor(a2, o);
        r2s += __shfl_xor(r2s, o);
    }
    if (lane == 0) {
        cn64[(size_t)h * C + m] = a2;
        cn32[(size_t)h * C + m] = (float)a2;
        resid[(size_t)h * C + m] = (float)(sqrt(r2s) * (1.0 + 1e-6));
    }
}

// One thread's share of a chunk in registers: hi rows r, r + 16, ... (r = tid / 16,
// 16-byte column tid & 15), then the same lo rows; ||c||^2 of centroid tid.
template <int NV>
struct KmStage {
    u32x4_t v[NV];
    float cn;
};

template <int CB, bool LO>
__device__ __forceinline__ void km_load(KmStage<KmChunk<CB, LO>::NV>& s, const bf16* __restrict__ hi,
                                        const bf16* __restrict__ lo, const float* __restrict__ cn,
                                        int m0, int C, int tid)
{
    const int ch = tid & 15, r = tid >> 4;
#pragma unroll
    for (int i = 0; i < CB / 16; ++i) {
        const int m = m0 + r + 16 * i;
        const bool ok = m < C;
        s.v[i] = ok ? *(const u32x4_t*)(hi + (size_t)m * KM_D + ch * 8) : u32x4_t{0, 0, 0, 0};
        if (LO) s.v[CB / 16 + i] = ok ? *(const u32x4_t*)(lo + (size_t)m * KM_D + ch * 8) : u32x4_t{0, 0, 0, 0};
    }
    s.cn = (tid < CB && m0 + tid < C) ? cn[m0 + tid] : __builtin_inff();
}

template <int CB, bool LO>
__device__ __forceinline__ void km_store(const KmStage<KmChunk<CB, LO>::NV>& s, char* buf, int tid)
{
    using K = KmChunk<CB, LO>;
    const int ch = tid & 15, r = tid >> 4;
#pragma unroll
    for (int i = 0; i < CB / 16; ++i) {
        *(u32x4_t*)(buf + (r + 16 * i) * KM_PITCH + ch * 16) = s.v[i];
        if (LO) *(u32x4_t*)(buf + K::PLANE + (r + 16 * i) * KM_PITCH + ch * 16) = s.v[CB / 16 + i];
    }
    if (tid < CB) ((float*)(buf + K::NPL * K::PLANE))[tid] = s.cn;
}

// acc[tb] = (hi + lo rows of a 32-centroid block) x (token block tb)^T; the
// fragment reads are issued two k-steps ahead of their MFMAs, which bounds the
// registers they occupy.  Without LO the lo plane is known to be zero (the
// first assignment, whose centroids are input tokens and so exact in bf16):
// its MFMAs would add exact zeros, so skipping them leaves every accumulator
// bit-identical.
template <bool LO, int PLANE>
__device__ __forceinline__ void km_tile(f32x16_t acc[2], const char* rh, const bf16x8_t xf[2][8])
{
    const char* rl = rh + PLANE;
    acc[0] = acc[1] = f32x16_t{0};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const bf16x8_t ah = as_bf16x8(*(const u32x4_t*)(rh + s * 32));
        bf16x8_t al;
        if (LO) al = as_bf16x8(*(const u32x4_t*)(rl + s * 32));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xf[tb][s], acc[tb], 0, 0, 0);
            if (LO) acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xf[tb][s], acc[tb], 0, 0, 0);
        }
    }
    if (LO) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s = 0; s < 6; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    } else {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int s = 0; s < 6; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
}

// Screen: labels = screen argmin; near-ties appended to flags[h, *] (token ids).
// LO: whether the centroids' lo plane can be non-zero (km_tile).
template <bool LO>
__global__ __launch_bounds__(256, 3) void k_assign_mfma(
    const bf16* __restrict__ X, const bf16* __restrict__ hi, const bf16* __restrict__ lo,
    const float* __restrict__ cn32, const unsigned* __restrict__ stats, int N, int C,
    int32_t* __restrict__ labels, int32_t* __restrict__ flags, int* __restrict__ nflag,
    float* __restrict__ ub_own, float* __restrict__ lb_own, float* __restrict__ lb_rest,
    const int* __restrict__ mcount, unsigned* __restrict__ range)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int h = blockIdx.y;
    if (mcount && km_partial_pays(mcount[h], C)) return;   // k_assign_partial takes this head
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tcol = lane & 31, half = lane >> 5;
    const bf16* Xh = X + (size_t)h * N * KM_D;
    const bf16* hih = hi + (size_t)h * C * KM_D;
    const bf16* loh = lo + (size_t)h * C * KM_D;
    const float* cnh = cn32 + (size_t)h * C;

    constexpr int CB = KmScreen<LO>::CB;
    using K = typename KmScreen<LO>::Chunk;
    const int nchunk = (C + CB - 1) / CB;
    KmStage<K::NV> stg;
    // the first chunk is requested together with the token rows
    km_load<CB, LO>(stg, hih, loh, cnh, 0, C, tid);

    // Token fragments (B operand): token tok[tb], dims 16 s + 8 half + 0..7.
    bf16x8_t xf[2][8];
    float nx[2];
    int tok[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        tok[tb] = blockIdx.x * KM_TOK + wave * 64 + tb * 32 + tcol;
        const int row = tok[tb] < N ? tok[tb] : N - 1;
        const bf16* xp = Xh + (size_t)row * KM_D + half * 8;
#pragma unroll
        for (int s = 0; s < 8; ++s) xf[tb][s] = as_bf16x8(*(const u32x4_t*)(xp + 16 * s));
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4_t w = __builtin_bit_cast(u32x4_t, xf[tb][s]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __uint_as_float(w[e] << 16), b = __uint_as_float(w[e] & 0xFFFF0000u);
                ss = fmaf(a, a, ss);
                ss = fmaf(b, b, ss);
            }
        }
        ss += __shfl_xor(ss, 32);
        nx[tb] = sqrtf(ss);
    }
    if (range) {   // the first screen reads every row of X: its largest magnitude sets the sums' scale
        RangeBf16 rg;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const u32x4_t w = __builtin_bit_cast(u32x4_t, xf[tb][s]);
#pragma unroll
                for (int e = 0; e < 4; ++e) rg.add_max(w[e]);
            }
        range_commit(rg.max_word(), 0u, range + kRangeStride * h, false);
    }

    // per lane and token block: the two smallest screen distances, index of the first
    float b1[2], b2[2];
    int i1[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        b1[tb] = b2[tb] = __builtin_inff();
        i1[tb] = 0;
    }

    km_store<CB, LO>(stg, smem, tid);
    __syncthreads();
    for (int k = 0; k < nchunk; ++k) {
        char* buf = smem + (k & 1) * K::BYTES;
        const bool more = k + 1 < nchunk;
        if (more) km_load<CB, LO>(stg, hih, loh, cnh, (k + 1) * CB, C, tid);
        const float* s_cn = (const float*)(buf + K::NPL * K::PLANE);
#pragma unroll
        for (int cb = 0; cb < CB / 32; ++cb) {
            f32x16_t acc[2];
            km_tile<LO, K::PLANE>(acc, buf + (cb * 32 + tcol) * KM_PITCH + half * 16, xf);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = cb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                const float cnv = s_cn[r];  // +inf past the last centroid
                const int m = k * CB + r;
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    // the two smallest so far (b1 <= b2): the new second is the
                    // middle of (b1, b2, d), one v_med3 for max-then-min
                    const float d = fmaf(-2.f, acc[tb][i], cnv);
                    i1[tb] = d < b1[tb] ? m : i1[tb];
                    b2[tb] = __builtin_amdgcn_fmed3f(b1[tb], b2[tb], d);
                    b1[tb] = fminf(b1[tb], d);
                }
            }
        }
        if (more) {
            km_store<CB, LO>(stg, smem + ((k + 1) & 1) * K::BYTES, tid);
            __syncthreads();
        }
    }

    const float R = __uint_as_float(stats[4 * h + 0]);
    const float cmax = __uint_as_float(stats[4 * h + 1]);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        // merge with the partner half-wave (other centroid rows, same token)
        const float pb1 = __shfl_xor(b1[tb], 32), pb2 = __shfl_xor(b2[tb], 32);
        const int pi1 = __shfl_xor(i1[tb], 32);
        const bool take = pb1 < b1[tb] || (pb1 == b1[tb] && pi1 < i1[tb]);
        const float nb1 = take ? pb1 : b1[tb];
        const int ni1 = take ? pi1 : i1[tb];
        const float nb2 = fminf(fminf(b2[tb], pb2), fmaxf(b1[tb], pb1));
        if (half == 0 && tok[tb] < N) {
            const float E = screen_error(nx[tb], R, cmax);
            const size_t t = (size_t)h * N + tok[tb];
            labels[t] = ni1;
            if (!(nb2 - nb1 > 2.f * E)) {
                const int pos = atomicAdd(nflag + h, 1);
                flags[(size_t)h * N + pos] = tok[tb];
            } else {
                ub_own[t] = bound_up(nb1 + E);
                lb_own[t] = bound_dn(nb1 - E);
                lb_rest[t] = bound_dn(nb2 - E);
            }
        }
    }
}

// The moved centroids (list mlist[h, 0 .. mcount)) staged like km_load; rows
// past the list get ||c||^2 = +inf.  In two parts, so that the list entries
// can be requested before the token rows and the centroid rows after them.
template <int CB>
struct KmListIdx {
    int m[CB / 16];   // list entries of rows r, r + 16, ...
    int mc;           // list entry of centroid tid (the ||c||^2 lane)
};
template <int CB>
__device__ __forceinline__ void km_list_idx(KmListIdx<CB>& ix, const int* __restrict__ ml, int k0, int cnt,
                                            int tid)
{
    const int r = tid >> 4;
#pragma unroll
    for (int i = 0; i < CB / 16; ++i) {
        const int k = k0 + r + 16 * i;
        ix.m[i] = k < cnt ? ml[k] : -1;
    }
    ix.mc = (tid < CB && k0 + tid < cnt) ? ml[k0 + tid] : -1;
}
template <int CB>
__device__ __forceinline__ void km_list_rows(KmStage<KmChunk<CB, true>::NV>& s, const KmListIdx<CB>& ix,
                                             const bf16* __restrict__ hi, const bf16* __restrict__ lo,
                                             const float* __restrict__ cn, int tid)
{
    const int ch = tid & 15;
#pragma unroll
    for (int i = 0; i < CB / 16; ++i) {
        const int m = ix.m[i];
        const bool ok = m >= 0;
        s.v[i] = ok ? *(const u32x4_t*)(hi + (size_t)m * KM_D + ch * 8) : u32x4_t{0, 0, 0, 0};
        s.v[CB / 16 + i] = ok ? *(const u32x4_t*)(lo + (size_t)m * KM_D + ch * 8) : u32x4_t{0, 0, 0, 0};
    }
    s.cn = ix.mc >= 0 ? cn[ix.mc] : __builtin_inff();
}

// Iterations after the first: screen against the moved centroids only and
// decide from the stored bounds (file comment); undecided tokens are queued for
// the exact recheck.
__global__ __launch_bounds__(256, 3) void k_assign_partial(
    const bf16* __restrict__ X, const bf16* __restrict__ hi, const bf16* __restrict__ lo,
    const float* __restrict__ cn32, const unsigned* __restrict__ stats, const int* __restrict__ mlist,
    const int* __restrict__ mpos, const int* __restrict__ mcount, int N, int C,
    int32_t* __restrict__ labels,
    int32_t* __restrict__ flags, int* __restrict__ nflag, float* __restrict__ ub_own,
    float* __restrict__ lb_own, float* __restrict__ lb_rest)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int h = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tcol = lane & 31, half = lane >> 5;
    const bf16* Xh = X + (size_t)h * N * KM_D;
    const bf16* hih = hi + (size_t)h * C * KM_D;
    const bf16* loh = lo + (size_t)h * C * KM_D;
    const float* cnh = cn32 + (size_t)h * C;
    const int* ml = mlist + (size_t)h * C;
    const int cnt = mcount[h];
    if (!km_partial_pays(cnt, C)) return;   // k_assign_mfma takes this head

    // Requests in dependency order: the first chunk's list entries and the
    // labels, then the token rows, then what depends on the first two (the
    // chunk's centroid rows, the labels' list positions), so that the chains
    // of dependent loads overlap the token rows instead of following them.
    using K = KmPartialChunk;
    constexpr int CB = 32;
    const int nchunk = (cnt + CB - 1) / CB;
    KmListIdx<CB> ix;
    km_list_idx<CB>(ix, ml, 0, cnt, tid);
    int tok[2], lab[2], own[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        tok[tb] = blockIdx.x * KM_TOK + wave * 64 + tb * 32 + tcol;
        lab[tb] = labels[(size_t)h * N + (tok[tb] < N ? tok[tb] : N - 1)];
    }
    bf16x8_t xf[2][8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int row = tok[tb] < N ? tok[tb] : N - 1;
        const bf16* xp = Xh + (size_t)row * KM_D + half * 8;
#pragma unroll
        for (int s = 0; s < 8; ++s) xf[tb][s] = as_bf16x8(*(const u32x4_t*)(xp + 16 * s));
    }
    KmStage<K::NV> stg;
    km_list_rows<CB>(stg, ix, hih, loh, cnh, tid);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) own[tb] = mpos[(size_t)h * C + lab[tb]];   // list position or -1
    float nx[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4_t w = __builtin_bit_cast(u32x4_t, xf[tb][s]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __uint_as_float(w[e] << 16), b = __uint_as_float(w[e] & 0xFFFF0000u);
                ss = fmaf(a, a, ss);
                ss = fmaf(b, b, ss);
            }
        }
        ss += __shfl_xor(ss, 32);
        nx[tb] = sqrtf(ss);
    }

    // per lane and token block: the own centroid's screen value (if it moved),
    // and the two smallest over the other moved centroids, list position of the first
    float od[2], b1[2], b2[2];
    int i1[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        od[tb] = b1[tb] = b2[tb] = __builtin_inff();
        i1[tb] = 0;
    }

    // Single-buffered chunks (the moved list is short after the first few
    // iterations; it keeps the registers within the three-workgroup limit);
    // the first chunk's rows were requested with the token rows.
    for (int k = 0; k < nchunk; ++k) {
        char* const buf = smem;
        {
            if (k > 0) {
                km_list_idx<CB>(ix, ml, k * CB, cnt, tid);
                km_list_rows<CB>(stg, ix, hih, loh, cnh, tid);
            }
            __syncthreads();   // the previous chunk's readers are done
            km_store<CB, true>(stg, buf, tid);
            __syncthreads();
        }
        {
            const float* s_cn = (const float*)(buf + K::NPL * K::PLANE);
#pragma unroll
            for (int cb = 0; cb < CB / 32; ++cb) {
                f32x16_t acc[2];
                km_tile<true, K::PLANE>(acc, buf + (cb * 32 + tcol) * KM_PITCH + half * 16, xf);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = cb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                    const float cnv = s_cn[r];  // +inf past the list
                    const int m = k * CB + r;   // list position
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        const float d = fmaf(-2.f, acc[tb][i], cnv);
                        const bool is_own = m == own[tb];
                        od[tb] = is_own ? d : od[tb];
                        const float dd = is_own ? __builtin_inff() : d;
                        i1[tb] = dd < b1[tb] ? m : i1[tb];
                        b2[tb] = __builtin_amdgcn_fmed3f(b1[tb], b2[tb], dd);   // as in the full screen
                        b1[tb] = fminf(b1[tb], dd);
                    }
                }
            }
        }
    }

    const float R = __uint_as_float(stats[4 * h + 0]);
    const float cmax = __uint_as_float(stats[4 * h + 1]);
    // the stored bounds, fetched only now (held through the screen they would
    // be spilled, and each spill would wait for its load)
    float pub[2], plb[2], plr[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const size_t t = (size_t)h * N + (tok[tb] < N ? tok[tb] : N - 1);
        pub[tb] = ub_own[t];
        plb[tb] = lb_own[t];
        plr[tb] = lb_rest[t];
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const float pb1 = __shfl_xor(b1[tb], 32), pb2 = __shfl_xor(b2[tb], 32);
        const int pi1 = __shfl_xor(i1[tb], 32);
        const float pod = __shfl_xor(od[tb], 32);
        const bool take = pb1 < b1[tb] || (pb1 == b1[tb] && pi1 < i1[tb]);
        const float nb1 = take ? pb1 : b1[tb];
        const int ni1 = take ? pi1 : i1[tb];
        const float nb2 = fminf(fminf(b2[tb], pb2), fmaxf(b1[tb], pb1));
        const float nod = fminf(od[tb], pod);   // at most one half saw the own centroid
        if (half == 0 && tok[tb] < N) {
            const float E = screen_error(nx[tb], R, cmax);
            const size_t t = (size_t)h * N + tok[tb];
            const bool own_moved = nod < __builtin_inff();
            const float UBa = own_moved ? bound_up(nod + E) : pub[tb];
            const float LBa = own_moved ? bound_dn(nod - E) : plb[tb];
            const float LBr = plr[tb];
            const float LBo1 = bound_dn(nb1 - E), UBo1 = bound_up(nb1 + E), LBo2 = bound_dn(nb2 - E);
            if (UBa < fminf(LBr, LBo1)) {
                ub_own[t] = UBa;
                lb_own[t] = LBa;
                lb_rest[t] = fminf(LBr, LBo1);
            } else if (UBo1 < fminf(fminf(LBr, LBa), LBo2)) {
                labels[t] = ml[ni1];
                ub_own[t] = UBo1;
                lb_own[t] = LBo1;
                lb_rest[t] = fminf(fminf(LBr, LBa), LBo2);
            } else {
                const int pos = atomicAdd(nflag + h, 1);
                flags[(size_t)h * N + pos] = tok[tb];
            }
        }
    }
}

// Exact settlement of queued tokens (few per head), one workgroup per token at a
// time (the queues of all heads dealt to the whole grid).
// Pass 1: every centroid's ||c||^2 - 2 x.c in fp64, each thread owning whole
// centroid rows (16-byte loads, x broadcast from LDS).  Pass 2: for every
// centroid within a tolerance of the minimum, the distance exactly as the
// oracle evaluates it (sum of (x_t - c_t)^2 in coordinate order, no fusion),
// rows staged in LDS; the smallest wins, lowest index first.
constexpr int RC_ROWS = 8, RC_MAXCAND = 64, RC_HEADS = 1024;
__global__ __launch_bounds__(256) void k_recheck(const bf16* __restrict__ X,
                                                 const double* __restrict__ cent64,
                                                 const double* __restrict__ cn64,
                                                 const unsigned* __restrict__ stats, int N, int C,
                                                 const int32_t* __restrict__ flags,
                                                 const int* __restrict__ nflag,
                                                 int32_t* __restrict__ labels,
                                                 float* __restrict__ ub_own,
                                                 float* __restrict__ lb_own,
                                                 float* __restrict__ lb_rest)
{
#pragma clang fp contract(off)
    __shared__ double s_x[KM_D];
    extern __shared__ double s_d[];   // [C], sized at launch
    __shared__ double s_rb[4];
    __shared__ int s_ri[4];
    __shared__ double s_c[RC_ROWS][KM_D];
    __shared__ int s_cand[RC_MAXCAND];
    __shared__ int s_nc, s_win;
    __shared__ int s_hp[RC_HEADS + 1], s_ws[4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // The queued tokens of all heads form one list (heads in order), dealt to
    // every workgroup of the grid, so a head with many queued tokens does not
    // wait on its own share of workgroups.  Heads in segments of RC_HEADS: the
    // exclusive prefix of their queue lengths in s_hp.
    const int H = (int)gridDim.y;
    const int wg = (int)(blockIdx.y * gridDim.x + blockIdx.x), nwg = (int)(gridDim.x * gridDim.y);
    for (int h0 = 0; h0 < H; h0 += RC_HEADS) {
    const int hn = min(RC_HEADS, H - h0);
    {
        constexpr int PER = RC_HEADS / 256;
        int v[PER], loc = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int j = tid * PER + i;
            v[i] = j < hn ? nflag[h0 + j] : 0;
            loc += v[i];
        }
        int incl = loc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        __syncthreads();   // the previous segment's readers of s_hp and s_ws are done
        if (lane == 63) s_ws[wave] = incl;
        __syncthreads();
        int ex = incl - loc;
#pragma unroll
        for (int w = 0; w < 3; ++w) ex += w < wave ? s_ws[w] : 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int j = tid * PER + i;
            if (j < hn) s_hp[j] = ex;
            ex += v[i];
        }
        if (tid == 255) s_hp[hn] = ex;   // the segment's total
        __syncthreads();
    }
    const int total = s_hp[hn];
    for (int e = wg; e < total; e += nwg) {
        int lo = 0, hi = hn - 1;   // the head: last j with s_hp[j] <= e
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_hp[mid] <= e) lo = mid; else hi = mid - 1;
        }
        const int h = h0 + lo;
        const double* ch = cent64 + (size_t)h * C * KM_D;
        const double* cnh = cn64 + (size_t)h * C;
        const double cmax = (double)__uint_as_float(stats[4 * h + 1]);
        const int token = flags[(size_t)h * N + (e - s_hp[lo])];
        __syncthreads();
        if (tid < KM_D) s_x[tid] = (double)bf16_to_f32(X[((size_t)h * N + token) * KM_D + tid]);
        __syncthreads();
        for (int m = tid; m < C; m += 256) {
            const double2* cr = (const double2*)(ch + (size_t)m * KM_D);
            double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
#pragma unroll 4
            for (int t = 0; t < KM_D / 2; t += 2) {
                const double2 a = cr[t], b = cr[t + 1];
                d0 = fma(s_x[2 * t], a.x, d0);
                d1 = fma(s_x[2 * t + 1], a.y, d1);
                d2 = fma(s_x[2 * t + 2], b.x, d2);
                d3 = fma(s_x[2 * t + 3], b.y, d3);
            }
            s_d[m] = fma(-2.0, (d0 + d1) + (d2 + d3), cnh[m]);
        }
        __syncthreads();
        double dmin = __builtin_inf();
        for (int m = tid; m < C; m += 256) dmin = fmin(dmin, s_d[m]);
        for (int o = 32; o >= 1; o >>= 1) dmin = fmin(dmin, __shfl_xor(dmin, o));
        if (lane == 0) s_rb[wave] = dmin;
        __syncthreads();
        dmin = fmin(fmin(s_rb[0], s_rb[1]), fmin(s_rb[2], s_rb[3]));
        double xx = 0.0;
        for (int t = 0; t < KM_D; ++t) xx = fma(s_x[t], s_x[t], xx);
        // |dot form - exact form| <= 260 * 2^-53 * (||x|| + ||c||)^2 for every centroid,
        // so the exact minimiser lies within twice that of the dot-form minimum.
        const double nxc = sqrt(xx) + cmax;
        const double tol = 0x1p-42 * nxc * nxc;
        // candidates (usually one or two): collected in one pass (their order
        // does not matter: the smallest distance wins, the lowest index on
        // ties), their rows staged in LDS RC_ROWS at a time for the sequential
        // exact sums; more than RC_MAXCAND of them are taken block by block
        double best = __builtin_inf();
        int bi = 0x7fffffff;
        auto settle = [&](int nc) {
            for (int k0 = 0; k0 < nc; k0 += RC_ROWS) {
                const int kn = min(RC_ROWS, nc - k0);
                for (int k = tid; k < kn * KM_D; k += 256)
                    s_c[k / KM_D][k % KM_D] = ch[(size_t)s_cand[k0 + k / KM_D] * KM_D + k % KM_D];
                __syncthreads();
                if (tid < kn) {
                    const int m = s_cand[k0 + tid];
                    double sd = 0.0;
                    for (int t = 0; t < KM_D; ++t) {
                        const double w = __dsub_rn(s_x[t], s_c[tid][t]);
                        sd = __dadd_rn(sd, __dmul_rn(w, w));
                    }
                    if (sd < best || (sd == best && m < bi)) {
                        best = sd;
                        bi = m;
                    }
                }
                __syncthreads();
            }
        };
        if (tid == 0) s_nc = 0;
        __syncthreads();
        for (int m = tid; m < C; m += 256)
            if (s_d[m] <= dmin + tol) {
                const int k = atomicAdd(&s_nc, 1);
                if (k < RC_MAXCAND) s_cand[k] = m;
            }
        __syncthreads();
        const int ntot = s_nc;
        if (ntot <= RC_MAXCAND) {
            settle(ntot);
        } else {
            for (int m0 = 0; m0 < C; m0 += RC_MAXCAND) {
                __syncthreads();   // every thread has read s_nc
                if (tid == 0) s_nc = 0;
                __syncthreads();
                if (tid < RC_MAXCAND && m0 + tid < C && s_d[m0 + tid] <= dmin + tol)
                    s_cand[atomicAdd(&s_nc, 1)] = m0 + tid;
                __syncthreads();
                settle(s_nc);
            }
        }
        for (int o = 32; o >= 1; o >>= 1) {
            const double ob = __shfl_xor(best, o);
            const int oi = __shfl_xor(bi, o);
            if (ob < best || (ob == best && oi < bi)) {
                best = ob;
                bi = oi;
            }
        }
        __syncthreads();
        if (lane == 0) {
            s_rb[wave] = best;
            s_ri[wave] = bi;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < 4; ++w)
                if (s_rb[w] < best || (s_rb[w] == best && s_ri[w] < bi)) {
                    best = s_rb[w];
                    bi = s_ri[w];
                }
            // No candidate only with non-finite distances (an out-of-range input,
            // reported as ERR_RANGE): keep the screen's label, which is in range.
            if (bi >= C) bi = labels[(size_t)h * N + token];
            labels[(size_t)h * N + token] = bi;
            s_win = bi;
        }
        __syncthreads();
        // Bounds for the later partial screens: the winner's exact distance
        // (shifted by ||x||^2 into the screen's units), and the smallest dot-form
        // value of the others; both widened by tol, which exceeds their errors.
        const int win = s_win;
        double second = __builtin_inf();
        for (int m = tid; m < C; m += 256)
            if (m != win) second = fmin(second, s_d[m]);
        for (int o = 32; o >= 1; o >>= 1) second = fmin(second, __shfl_xor(second, o));
        __syncthreads();
        if (lane == 0) s_rb[wave] = second;
        __syncthreads();
        if (tid == 0) {
            second = fmin(fmin(s_rb[0], s_rb[1]), fmin(s_rb[2], s_rb[3]));
            const double own = best - xx;
            const size_t t = (size_t)h * N + token;
            ub_own[t] = __double2float_ru(own + tol);
            lb_own[t] = __double2float_rd(own - tol);
            lb_rest[t] = __double2float_rd(second - tol);
        }
    }
    }
}

SVG_HIDDEN KmPlanes km_planes(const ClusterArgs& a)
{
    const Layout& L = *a.L;
    char* s = a.scratch;
    KmPlanes P;
    P.hi = (bf16*)(s + L.cl_hi);
    P.lo = (bf16*)(s + L.cl_lo);
    P.cn32 = (float*)(s + L.cl_cnorm);
    P.cn64 = (double*)(s + L.cl_cn64);
    P.stats = (unsigned*)(s + L.cl_stats);
    P.flags = (int32_t*)(s + L.cl_flag);
    P.nflag = (int*)(s + L.cl_nflag);
    P.mlist = (int*)(s + L.cl_mlist);
    P.mpos = (int*)(s + L.cl_mpos);
    P.mcount = (int*)(s + L.cl_mcount);
    const size_t HN = (size_t)a.H * a.N;
    P.ub_own = (float*)(s + L.cl_bounds);
    P.lb_own = P.ub_own + HN;
    P.lb_rest = P.lb_own + HN;
    return P;
}

SVG_HIDDEN bool assign_mfma_supported(const ClusterArgs& a)
{
    return a.dtype == SVGEAR_BF16 && a.d == KM_D;
}

SVG_HIDDEN hipError_t launch_km_prep(const ClusterArgs& a, const double* cent64, const KmPlanes& P,
                                     hipStream_t st)
{
    hipLaunchKernelGGL(k_km_prep, dim3((a.C + 3) / 4, a.H), dim3(256), 0, st, cent64, a.C, P.hi, P.lo, P.cn32,
                       P.cn64, (float*)(a.scratch + a.L->cl_resid));
    return hipGetLastError();
}

SVG_HIDDEN hipError_t launch_assign_mfma(const ClusterArgs& a, const double* cent64,
                                         const KmPlanes& P, bool partial, unsigned* range,
                                         hipStream_t st)
{
    // With `partial`, both screens are launched and each head runs in the one
    // its moved-centroid count selects (decided on the device).
    // The first screen (not partial) runs on the initial centroids, input
    // tokens exact in bf16, whose lo plane is zero.
    const dim3 grid((a.N + KM_TOK - 1) / KM_TOK, a.H);
    if (partial)
        hipLaunchKernelGGL(k_assign_mfma<true>, grid, dim3(256), KmScreen<true>::LDS, st, (const bf16*)a.X, P.hi, P.lo,
                           P.cn32, P.stats, a.N, a.C, a.labels, P.flags, P.nflag, P.ub_own, P.lb_own,
                           P.lb_rest, (const int*)P.mcount, (unsigned*)nullptr);
    else
        hipLaunchKernelGGL(k_assign_mfma<false>, grid, dim3(256), KmScreen<false>::LDS, st, (const bf16*)a.X, P.hi, P.lo,
                           P.cn32, P.stats, a.N, a.C, a.labels, P.flags, P.nflag, P.ub_own, P.lb_own,
                           P.lb_rest, (const int*)nullptr, range);
    if (partial)
        hipLaunchKernelGGL(k_assign_partial, grid, dim3(256), KmPartialChunk::BYTES, st, (const bf16*)a.X, P.hi,
                           P.lo, P.cn32, P.stats, P.mlist, P.mpos, P.mcount, a.N, a.C, a.labels,
                           P.flags, P.nflag, P.ub_own, P.lb_own, P.lb_rest);
    hipLaunchKernelGGL(k_recheck, dim3(256, a.H), dim3(256), (size_t)a.C * 8, st, (const bf16*)a.X, cent64, P.cn64,
                       P.stats, a.N, a.C, P.flags, P.nflag, a.labels, P.ub_own, P.lb_own, P.lb_rest);
    return hipGetLastError();
}

}  // namespace svg
