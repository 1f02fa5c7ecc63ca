// attention.hip -- step 4 of the SVG-EAR pipeline (review page, inference-
// pipeline paragraph, step 4; German summary 2A): hybrid attention.  Exact
// blocks use the keys and values of the routed key clusters; every skipped key
// cluster g enters the same softmax once, as its centroid with logit
// tau q.kbar_g + ln m_g and value vbar_g (each of its m_g keys replaced by the
// centroid).  Output rows go back to token order.
//
// This file holds the generic kernel (any dtype, d in {64, 128}; fp32 used for
// the fp32 workload) and the dispatch; the bf16 MFMA kernel is attn_mfma.hip.
#include "internal.h"

namespace svg {

__device__ __forceinline__ float wave_sum(float v)
{
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// One block of 4 waves per reordered query row; the waves split the key
// clusters, each runs an online softmax, and the partial states are merged.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_attention_generic(
    const T* __restrict__ Qp, const int32_t* __restrict__ offsets_q,
    const int32_t* __restrict__ perm_q, const T* __restrict__ Kp, const T* __restrict__ Vp,
    const float* __restrict__ kbar, const float* __restrict__ vbar,
    const int32_t* __restrict__ offsets_k, const uint8_t* __restrict__ mask, int Nq, int Nk,
    int Cq, int Ck, float tau, T* __restrict__ O)
{
    constexpr int EPL = D / 64;
    __shared__ float s_m[4], s_l[4];
    __shared__ float s_acc[4][D];
    const int r = blockIdx.x, h = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // query cluster of reordered row r
    const int32_t* oq = offsets_q + (size_t)h * (Cq + 1);
    int lo = 0, hi = Cq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (oq[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const int c = lo;
    float q[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[e] = to_f32<T>(Qp[((size_t)h * Nq + r) * D + lane * EPL + e]);
    const uint8_t* mrow = mask + ((size_t)h * Cq + c) * Ck;
    const int32_t* ok = offsets_k + (size_t)h * (Ck + 1);
    float m = -__builtin_inff(), l = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    auto add_term = [&](float s, const float* v) {
        if (s > m) {
            const float a = expf(m - s);
            l *= a;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] *= a;
            m = s;
        }
        const float p = expf(s - m);
        l += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, v[e], acc[e]);
    };
    for (int g = wave; g < Ck; g += 4) {
        const int j0 = ok[g], j1 = ok[g + 1];
        if (j1 == j0) continue;
        if (mrow[g]) {
            for (int j = j0; j < j1; ++j) {
                float part = 0.f, v[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    part = fmaf(q[e], to_f32<T>(Kp[((size_t)h * Nk + j) * D + lane * EPL + e]), part);
                    v[e] = to_f32<T>(Vp[((size_t)h * Nk + j) * D + lane * EPL + e]);
                }
                add_term(tau * wave_sum(part), v);
            }
        } else {
            float part = 0.f, v[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                part = fmaf(q[e], kbar[((size_t)h * Ck + g) * D + lane * EPL + e], part);
                v[e] = vbar[((size_t)h * Ck + g) * D + lane * EPL + e];
            }
            add_term(tau * wave_sum(part) + logf((float)(j1 - j0)), v);
        }
    }
    if (lane == 0) {
        s_m[wave] = m;
        s_l[wave] = l;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[wave][lane * EPL + e] = acc[e];
    __syncthreads();
    if (wave == 0) {
        float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
        float Ls = 0.f, out[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) out[e] = 0.f;
        for (int w = 0; w < 4; ++w) {
            if (s_m[w] == -__builtin_inff()) continue;
            const float a = expf(s_m[w] - M);
            Ls += a * s_l[w];
#pragma unroll
            for (int e = 0; e < EPL; ++e) out[e] = fmaf(a, s_acc[w][lane * EPL + e], out[e]);
        }
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        const int tok = perm_q[(size_t)h * Nq + r];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            O[((size_t)h * Nq + tok) * D + lane * EPL + e] = from_f32<T>(out[e] * inv);
    }
}

SVG_HIDDEN hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t st);
SVG_HIDDEN bool attention_mfma_supported(const AttnArgs& a);

template <typename T, int D>
static hipError_t run_attention(const AttnArgs& a, hipStream_t st)
{
    if (attention_mfma_supported(a)) return launch_attention_mfma(a, st);
    const float tau = 1.0f / sqrtf((float)D);
    hipLaunchKernelGGL((k_attention_generic<T, D>), dim3(a.Nq, a.H), dim3(256), 0, st,
                       (const T*)a.Qp, a.offsets_q, a.perm_q, (const T*)a.Kp, (const T*)a.Vp,
                       a.kbar, a.vbar, a.offsets_k, a.mask, a.Nq, a.Nk, a.Cq, a.Ck, tau, (T*)a.O);
    return hipGetLastError();
}

SVG_HIDDEN hipError_t launch_attention(const AttnArgs& a, hipStream_t st)
{
    if (a.dtype == SVGEAR_BF16)
        return a.d == 128 ? run_attention<bf16, 128>(a, st) : run_attention<bf16, 64>(a, st);
    return a.d == 128 ? run_attention<float, 128>(a, st) : run_attention<float, 64>(a, st);
}

}  // namespace svg
