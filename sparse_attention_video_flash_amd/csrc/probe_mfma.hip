// probe_mfma.hip -- value-aware centroid probe on bf16 MFMA for d = 128 and
// Cq <= 256 (steps 2-3 of the SVG-EAR pipeline, review page inference-pipeline
// paragraph; German summary 2B, including its single-pass streaming kernel that
// never writes logits to device memory).
//
// For key cluster g and its keys j (contiguous after reordering) and every
// query cluster c:  D = tau qbar_c.(kbar_g - k_j) is evaluated with
// v_mfma_f32_16x16x32_bf16 from bf16 hi/lo planes of both factors (products
// hi.hi + hi.lo + lo.hi; the differences are formed in fp32 per key), so D is
// exactly 0 for a key equal to its centroid and small D keep their accuracy.
// Then, as in the generic kernel,
//     e = e^{2s} [expm1(D)^2 ||vbar_g||^2 + 2 expm1(D) vbar_g.delta_j + ||delta_j||^2],
// s = sbar - D (in the overflow-free form of probe_term), is folded into a
// per-(c, g) running log-sum-exp.  Keys are the
// MFMA rows and query clusters the columns, so each lane owns one c and the
// sums over keys stay in-lane until one exchange across the four row groups.
// One wave handles one key cluster; the query-centroid planes of the head sit
// in LDS for the whole workgroup.
#include "internal.h"

namespace svg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int PR_D = 128;
constexpr int PR_MAXCQ = 256;
constexpr int PR_PITCH = PR_D * 2 + 16;  // bytes per query-centroid row of a plane

__device__ __forceinline__ bf16x8_t pr_as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int NCB>
__global__ __launch_bounds__(256) void k_probe_mfma(
    const float* __restrict__ qbar, const int32_t* __restrict__ counts_q, const bf16* __restrict__ Kp,
    const float* __restrict__ kbar, const float* __restrict__ sbar, const float2* __restrict__ keys,
    const float* __restrict__ pg, const int32_t* __restrict__ offsets_k, int Nk, int Cq, int Ck,
    float tau, float* __restrict__ log_ratio, float* __restrict__ log_eps2)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int h = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    constexpr int ncb = NCB;            // 16-column blocks of query clusters
    const int cqp = ncb * 16;
    char* qhi = smem;
    char* qlo = smem + (size_t)cqp * PR_PITCH;

    // Query-centroid planes of this head (rows past Cq are zero).
    for (int k = tid; k < cqp * PR_D; k += 256) {
        const int c = k / PR_D, t = k - c * PR_D;
        const float v = c < Cq ? qbar[((size_t)h * Cq + c) * PR_D + t] : 0.f;
        const bf16 vh = f32_to_bf16(v);
        *(bf16*)(qhi + c * PR_PITCH + t * 2) = vh;
        *(bf16*)(qlo + c * PR_PITCH + t * 2) = f32_to_bf16(v - bf16_to_f32(vh));
    }
    __syncthreads();

    const int col = lane & 15, grp = lane >> 4;   // MFMA column (query cluster) / row group
    const int32_t* ok = offsets_k + (size_t)h * (Ck + 1);
    for (int g = blockIdx.x * 4 + wave; g < Ck; g += gridDim.x * 4) {
        const int j0 = ok[g], j1 = ok[g + 1];
        const int mg = j1 - j0;
        float* lr_out = log_ratio + (size_t)h * Cq * Ck + g;
        if (mg == 0) {
            for (int c = lane; c < Cq; c += 64) lr_out[(size_t)c * Ck] = -__builtin_inff();
            continue;
        }
        // k-bar_g for this lane's dims: 32 ks + 8 grp + 0..7, ks = 0..3
        float kb[4][8];
        const float* kbp = kbar + ((size_t)h * Ck + g) * PR_D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) kb[ks][e] = kbp[32 * ks + e];
        const float P = pg[(size_t)h * Ck + g];

        float M[NCB], S[NCB], sb[NCB];
#pragma unroll
        for (int cb = 0; cb < ncb; ++cb) {
            M[cb] = -__builtin_inff();
            S[cb] = 0.f;
            const int c = cb * 16 + col;
            sb[cb] = c < Cq ? sbar[((size_t)h * Cq + c) * Ck + g] : 0.f;
        }
        for (int jb = j0; jb < j1; jb += 16) {
            // A operand: differences kbar_g - k_j (row j = jb + col) as hi/lo planes
            const int jr = jb + col;
            const bool rv = jr < j1;
            bf16x8_t ah[4], al[4];
            const bf16* kp = Kp + ((size_t)h * Nk + (rv ? jr : j0)) * PR_D + 8 * grp;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4_t w = *(const u32x4_t*)(kp + 32 * ks);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned bits = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
                    const float df = rv ? kb[ks][e] - __uint_as_float(bits) : 0.f;
                    const bf16 dh = f32_to_bf16(df);
                    ah[ks][e] = __builtin_bit_cast(__bf16, dh);
                    al[ks][e] = __builtin_bit_cast(__bf16, f32_to_bf16(df - bf16_to_f32(dh)));
                }
            }
            // per-key scalars for this lane's rows jb + 4 grp + r
            float2 kq[4];
            bool kv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = jb + 4 * grp + r;
                kv[r] = j < j1;
                kq[r] = kv[r] ? keys[(size_t)h * Nk + j] : make_float2(0.f, 0.f);
            }
#pragma unroll
            for (int cb = 0; cb < ncb; ++cb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                const char* bh = qhi + (cb * 16 + col) * PR_PITCH + 16 * grp;
                const char* bl = qlo + (cb * 16 + col) * PR_PITCH + 16 * grp;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8_t qh = pr_as_bf16x8(*(const u32x4_t*)(bh + 64 * ks));
                    const bf16x8_t ql = pr_as_bf16x8(*(const u32x4_t*)(bl + 64 * ks));
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], qh, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], ql, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], qh, acc, 0, 0, 0);
                }
                const int c = cb * 16 + col;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (!kv[r]) continue;
                    float x;
                    const float f = probe_term(sb[cb], tau * acc[r], P, kq[r].x, kq[r].y, x);
                    if (log_eps2 && c < Cq)
                        log_eps2[((size_t)h * Cq + c) * Nk + jb + 4 * grp + r] =
                            f > 0.f ? x + logf(f) : -__builtin_inff();
                    if (f > 0.f) {
                        if (x > M[cb]) {
                            S[cb] = fmaf(S[cb], __expf(M[cb] - x), f);
                            M[cb] = x;
                        } else {
                            S[cb] = fmaf(f, __expf(x - M[cb]), S[cb]);
                        }
                    }
                }
            }
        }
        // combine the four row groups (lanes col, col + 16, col + 32, col + 48)
#pragma unroll
        for (int cb = 0; cb < ncb; ++cb) {
            float m = M[cb], sacc = S[cb];
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float om = __shfl_xor(m, o), os = __shfl_xor(sacc, o);
                const float mn = fmaxf(m, om);
                if (mn == -__builtin_inff()) continue;
                sacc = sacc * __expf(m - mn) + os * __expf(om - mn);
                m = mn;
            }
            const int c = cb * 16 + col;
            if (grp == 0 && c < Cq) {
                float lr = -__builtin_inff();
                if (counts_q[(size_t)h * Cq + c] > 0 && sacc > 0.f) lr = m + logf(sacc) - logf((float)mg);
                lr_out[(size_t)c * Ck] = lr;
            }
        }
    }
}

SVG_HIDDEN bool probe_mfma_supported(const ProbeArgs& a)
{
    return a.dtype == SVGEAR_BF16 && a.d == PR_D && a.Cq <= PR_MAXCQ;
}

SVG_HIDDEN hipError_t launch_probe_mfma(const ProbeArgs& a, const float* sbar, const float2* keys,
                                        const float* pg, hipStream_t st)
{
    const int cqp = ((a.Cq + 15) / 16) * 16;
    const size_t lds = 2 * (size_t)cqp * PR_PITCH;
    int blocks = (a.Ck + 3) / 4;
    if (blocks > 64) blocks = 64;
    float* eps = (a.flags & SVGEAR_DEBUG_EPS) ? a.log_eps2 : nullptr;
    const float tau = 1.0f / sqrtf((float)PR_D);
#define SVG_PROBE_CASE(n)                                                                          \
    case n:                                                                                        \
        hipLaunchKernelGGL(k_probe_mfma<n>, dim3(blocks, a.H), dim3(256), lds, st, a.qbar,         \
                           a.counts_q, (const bf16*)a.Kp, a.kbar, sbar, keys, pg, a.offsets_k,     \
                           a.Nk, a.Cq, a.Ck, tau, a.log_ratio, eps);                               \
        break;
    switch (cqp / 16) {
        SVG_PROBE_CASE(1) SVG_PROBE_CASE(2) SVG_PROBE_CASE(3) SVG_PROBE_CASE(4)
        SVG_PROBE_CASE(5) SVG_PROBE_CASE(6) SVG_PROBE_CASE(7) SVG_PROBE_CASE(8)
        SVG_PROBE_CASE(9) SVG_PROBE_CASE(10) SVG_PROBE_CASE(11) SVG_PROBE_CASE(12)
        SVG_PROBE_CASE(13) SVG_PROBE_CASE(14) SVG_PROBE_CASE(15) SVG_PROBE_CASE(16)
    default: return hipErrorInvalidValue;
    }
#undef SVG_PROBE_CASE
    return hipGetLastError();
}

}  // namespace svg
