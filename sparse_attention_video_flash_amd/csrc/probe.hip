// probe.hip -- steps 2 and 3 of the SVG-EAR pipeline (review page, inference-
// pipeline paragraph; German summary 2B): the value-aware centroid probe and the
// block error-to-cost ratio, streamed without writing logits to device memory.
//
// For query cluster c and key j of key cluster g, with s = tau qbar_c.k_j,
// sbar = tau qbar_c.kbar_g, D = sbar - s and delta_j = vbar_g - v_j,
//     e[c,j] = || e^sbar vbar_g - e^s v_j ||^2
//            = e^{2s} [ expm1(D)^2 ||vbar_g||^2 + 2 expm1(D) vbar_g.delta_j + ||delta_j||^2 ].
// The bracket is a norm, hence >= 0, and does not cancel when the compensation
// is accurate (small D, small delta).  The block sum over j is accumulated as a
// running log-sum-exp in the exponent 2s, so the ratio is produced as ln r
// without overflow: ln r = ln sum_j e[c,j] - ln m_g.
#include "internal.h"

namespace svg {

// Per key (reordered order): (vbar_g.delta_j, ||delta_j||^2), and per key
// cluster ||vbar_g||^2, for the generic probe (the MFMA probe forms them while
// it stages its keys).  One block per key cluster; 16 lanes per key row.
// With logit_only the values drop out: (0, 0) per key and 1 per cluster, which
// turns the bracket into expm1(D)^2, i.e. e = (e^sbar - e^s)^2.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_key_scalars(const T* __restrict__ Vp,
                                                     const float* __restrict__ vbar,
                                                     const int32_t* __restrict__ offsets_k, int Nk,
                                                     int Ck, float2* __restrict__ keys,
                                                     float* __restrict__ pg, int logit_only)
{
    if (logit_only) {
        const int g = blockIdx.x, h = blockIdx.y;
        if (threadIdx.x == 0) pg[(size_t)h * Ck + g] = 1.f;
        const int j0 = offsets_k[(size_t)h * (Ck + 1) + g], j1 = offsets_k[(size_t)h * (Ck + 1) + g + 1];
        for (int j = j0 + (int)threadIdx.x; j < j1; j += 256) keys[(size_t)h * Nk + j] = make_float2(0.f, 0.f);
        return;
    }
    constexpr int EPT = D / 16;  // elements per thread
    const int g = blockIdx.x, h = blockIdx.y;
    const int sub = threadIdx.x & 15, row = threadIdx.x >> 4;
    const float* vb = vbar + ((size_t)h * Ck + g) * D + sub * EPT;
    float vbr[EPT];
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        vbr[e] = vb[e];
        p = fmaf(vbr[e], vbr[e], p);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) p += __shfl_xor(p, o, 16);
    if (threadIdx.x == 0) pg[(size_t)h * Ck + g] = p;
    const int j0 = offsets_k[(size_t)h * (Ck + 1) + g], j1 = offsets_k[(size_t)h * (Ck + 1) + g + 1];
    // eight rows per pass, their loads issued together
    constexpr int RU = 8;
    for (int jb = j0; jb < j1; jb += 16 * RU) {
        T vv[RU][EPT];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int j = min(jb + row + 16 * u, j1 - 1);
            const T* v = Vp + ((size_t)h * Nk + j) * D + sub * EPT;
#pragma unroll
            for (int e = 0; e < EPT; ++e) vv[u][e] = v[e];
        }
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            float qd = 0.f, r = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                float dl = vbr[e] - to_f32<T>(vv[u][e]);
                qd = fmaf(vbr[e], dl, qd);
                r = fmaf(dl, dl, r);
            }
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                qd += __shfl_xor(qd, o, 16);
                r += __shfl_xor(r, o, 16);
            }
            const int j = jb + row + 16 * u;
            if (sub == 0 && j < j1) keys[(size_t)h * Nk + j] = make_float2(qd, r);
        }
    }
}

// sbar[c, g] = tau qbar_c . kbar_g, accumulated in fp64 in dimension order and
// rounded once to fp32.  A workgroup takes SB_C query clusters x 64 key
// clusters: the 64 kbar rows are staged in LDS (row pitch D + 1 floats, so the
// 64 lanes of a wave, one row each, read one dimension from distinct banks) and
// the SB_C qbar rows as fp64 (broadcast reads); wave w owns query clusters
// w, w + 4, ..., so each kbar value read from LDS feeds SB_C / 4 products.
constexpr int SB_C = 32;

template <int D>
__global__ __launch_bounds__(256) void k_sbar(const float* __restrict__ qbar,
                                              const float* __restrict__ kbar, int Cq, int Ck,
                                              double tau, float* __restrict__ sbar)
{
    constexpr int NR = SB_C / 4;   // query clusters per wave
    __shared__ float s_k[64][D + 1];
    __shared__ double s_q[SB_C][D];
    const int c0 = blockIdx.x * SB_C, g0 = blockIdx.y * 64, h = blockIdx.z, tid = threadIdx.x;
    // 64 rows x D floats as float4, all loads of a thread issued together
    constexpr int V4 = 64 * D / 4 / 256;
    float4 kv[V4];
#pragma unroll
    for (int u = 0; u < V4; ++u) {
        const int i = tid + 256 * u, r = i / (D / 4), t4 = i - r * (D / 4), g = g0 + r;
        kv[u] = g < Ck ? *(const float4*)(kbar + ((size_t)h * Ck + g) * D + 4 * t4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    constexpr int Q4 = SB_C * D / 4 / 256;   // the qbar rows likewise
    float4 qv[Q4];
#pragma unroll
    for (int u = 0; u < Q4; ++u) {
        const int i = tid + 256 * u, r = i / (D / 4), t4 = i - r * (D / 4), c = c0 + r;
        qv[u] = c < Cq ? *(const float4*)(qbar + ((size_t)h * Cq + c) * D + 4 * t4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < Q4; ++u) {
        const int i = tid + 256 * u, r = i / (D / 4), t4 = i - r * (D / 4);
        s_q[r][4 * t4] = (double)qv[u].x;
        s_q[r][4 * t4 + 1] = (double)qv[u].y;
        s_q[r][4 * t4 + 2] = (double)qv[u].z;
        s_q[r][4 * t4 + 3] = (double)qv[u].w;
    }
#pragma unroll
    for (int u = 0; u < V4; ++u) {
        const int i = tid + 256 * u, r = i / (D / 4), t4 = i - r * (D / 4);
        s_k[r][4 * t4] = kv[u].x;
        s_k[r][4 * t4 + 1] = kv[u].y;
        s_k[r][4 * t4 + 2] = kv[u].z;
        s_k[r][4 * t4 + 3] = kv[u].w;
    }
    __syncthreads();
    const int w = tid >> 6, gl = tid & 63, g = g0 + gl;
    if (g >= Ck) return;
    double s[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) s[k] = 0.0;
#pragma unroll 4
    for (int t = 0; t < D; ++t) {
        const double kt = (double)s_k[gl][t];
#pragma unroll
        for (int k = 0; k < NR; ++k) s[k] = fma(s_q[w + 4 * k][t], kt, s[k]);
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int c = c0 + w + 4 * k;
        if (c < Cq) sbar[((size_t)h * Cq + c) * Ck + g] = (float)(tau * s[k]);
    }
}

// Attention-score comparator: row c of ln r is sbar[c, g] minus the row's
// log-sum-exp of sbar[c, g'] + ln m_g' over non-empty key clusters, so
// m_g e^{ln r} is the centroid estimate of the attention mass on block (c, g).
// One workgroup per (c, h); max and sum are block reductions in fp32.
__global__ __launch_bounds__(256) void k_score_ratio(const float* __restrict__ sbar,
                                                     const int32_t* __restrict__ counts_q,
                                                     const int32_t* __restrict__ counts_k, int Cq,
                                                     int Ck, float* __restrict__ log_ratio)
{
    __shared__ float s_red[256];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const float* sb = sbar + ((size_t)h * Cq + c) * Ck;
    const int32_t* ck = counts_k + (size_t)h * Ck;
    float mx = -INFINITY;
    for (int g = tid; g < Ck; g += 256)
        if (ck[g] > 0) mx = fmaxf(mx, sb[g] + logf((float)ck[g]));
    s_red[tid] = mx;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) s_red[tid] = fmaxf(s_red[tid], s_red[tid + off]);
        __syncthreads();
    }
    mx = s_red[0];
    __syncthreads();
    float sum = 0.0f;
    for (int g = tid; g < Ck; g += 256)
        if (ck[g] > 0) sum += expf(sb[g] + logf((float)ck[g]) - mx);
    s_red[tid] = sum;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) s_red[tid] += s_red[tid + off];
        __syncthreads();
    }
    const float lse = mx + logf(s_red[0]);
    const bool row_ok = counts_q[(size_t)h * Cq + c] > 0;
    float* out = log_ratio + ((size_t)h * Cq + c) * Ck;
    for (int g = tid; g < Ck; g += 256) out[g] = (row_ok && ck[g] > 0) ? sb[g] - lse : -INFINITY;
}

// Generic probe: one block per key cluster g, one thread per query cluster c.
// The differences kbar_g - k_j of the cluster's keys are staged in LDS 32 at a
// time, so D = tau qbar.(kbar_g - k_j) is formed directly: it is exactly zero
// when a key equals its centroid, and small differences keep their accuracy.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_probe_generic(
    const float* __restrict__ qbar, const int32_t* __restrict__ counts_q, const T* __restrict__ Kp,
    const float* __restrict__ kbar, const float* __restrict__ sbar, const float2* __restrict__ keys,
    const float* __restrict__ pg,
    const int32_t* __restrict__ offsets_k, int Nk, int Cq, int Ck, float tau,
    float* __restrict__ log_ratio, float* __restrict__ log_eps2)
{
    constexpr int KB = 32;
    __shared__ float s_k[KB][D + 1];
    __shared__ float2 s_ks[KB];
    const int g = blockIdx.x, h = blockIdx.y;
    const int j0 = offsets_k[(size_t)h * (Ck + 1) + g], j1 = offsets_k[(size_t)h * (Ck + 1) + g + 1];
    const float P = pg[(size_t)h * Ck + g];
    const float* kb = kbar + ((size_t)h * Ck + g) * D;
    for (int c0 = 0; c0 < Cq; c0 += 256) {
        const int c = c0 + threadIdx.x;
        const bool act = c < Cq;
        float q[D];
        float sb = 0.f;
        if (act) {
#pragma unroll
            for (int t = 0; t < D; ++t) q[t] = qbar[((size_t)h * Cq + c) * D + t];
            sb = sbar[((size_t)h * Cq + c) * Ck + g];
        }
        float M = -__builtin_inff(), S = 0.f;
        for (int jb = j0; jb < j1; jb += KB) {
            const int kn = min(KB, j1 - jb);
            __syncthreads();
            for (int k = threadIdx.x; k < kn * D; k += 256)
                s_k[k / D][k % D] = kb[k % D] - to_f32<T>(Kp[((size_t)h * Nk + jb) * D + k]);
            if ((int)threadIdx.x < kn) s_ks[threadIdx.x] = keys[(size_t)h * Nk + jb + threadIdx.x];
            __syncthreads();
            if (!act) continue;
            for (int jj = 0; jj < kn; ++jj) {
                float dot = 0.f;
#pragma unroll 16
                for (int t = 0; t < D; ++t) dot = fmaf(q[t], s_k[jj][t], dot);
                const float dlt = tau * dot;   // sbar - s
                const float2 kq = s_ks[jj];
                float x;
                const float f = probe_term(sb, dlt, P, kq.x, kq.y, x);
                if (log_eps2)
                    log_eps2[((size_t)h * Cq + c) * Nk + jb + jj] =
                        f > 0.f ? x + logf(f) : -__builtin_inff();
                if (f > 0.f) {
                    if (x > M) {
                        S = S * expf(M - x) + f;
                        M = x;
                    } else {
                        S += f * expf(x - M);
                    }
                }
            }
        }
        if (act) {
            const int nq = counts_q[(size_t)h * Cq + c];
            const int mg = j1 - j0;
            float lr = -__builtin_inff();
            if (nq > 0 && mg > 0 && S > 0.f) lr = M + logf(S) - logf((float)mg);
            log_ratio[((size_t)h * Cq + c) * Ck + g] = lr;
        }
    }
}

SVG_HIDDEN hipError_t launch_probe_mfma(const ProbeArgs& a, const float* sbar, hipStream_t st);
SVG_HIDDEN bool probe_mfma_supported(const ProbeArgs& a);

template <typename T, int D>
static hipError_t run_probe(const ProbeArgs& a, hipStream_t st)
{
    const Layout& L = *a.L;
    float* sbar = (float*)(a.scratch + L.pr_sbar);
    float2* keys = (float2*)(a.scratch + L.pr_keys);
    float* pg = (float*)(a.scratch + L.pr_pg);
    const float tau = 1.0f / sqrtf((float)D);
    if (a.flags & SVGEAR_PROBE_SCORE) {
        hipLaunchKernelGGL((k_sbar<D>), dim3((a.Cq + SB_C - 1) / SB_C, (a.Ck + 63) / 64, a.H), dim3(256), 0, st, a.qbar,
                           a.kbar, a.Cq, a.Ck, 1.0 / sqrt((double)D), sbar);
        hipLaunchKernelGGL(k_score_ratio, dim3(a.Cq, a.H), dim3(256), 0, st, sbar, a.counts_q,
                           a.counts_k, a.Cq, a.Ck, a.log_ratio);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_sbar<D>), dim3((a.Cq + SB_C - 1) / SB_C, (a.Ck + 63) / 64, a.H), dim3(256), 0, st, a.qbar,
                       a.kbar, a.Cq, a.Ck, 1.0 / sqrt((double)D), sbar);
    // the MFMA probe forms its per-key value terms itself (one read of K_p and V_p)
    if (probe_mfma_supported(a)) return launch_probe_mfma(a, sbar, st);
    hipLaunchKernelGGL((k_key_scalars<T, D>), dim3(a.Ck, a.H), dim3(256), 0, st, (const T*)a.Vp,
                       a.vbar, a.offsets_k, a.Nk, a.Ck, keys, pg, (a.flags & SVGEAR_PROBE_LOGIT) ? 1 : 0);
    hipLaunchKernelGGL((k_probe_generic<T, D>), dim3(a.Ck, a.H), dim3(256), 0, st, a.qbar,
                       a.counts_q, (const T*)a.Kp, a.kbar, sbar, keys, pg, a.offsets_k, a.Nk, a.Cq, a.Ck,
                       tau, a.log_ratio, (a.flags & SVGEAR_DEBUG_EPS) ? a.log_eps2 : nullptr);
    return hipGetLastError();
}

SVG_HIDDEN hipError_t launch_probe(const ProbeArgs& a, hipStream_t st)
{
    if (a.dtype == SVGEAR_BF16) return a.d == 128 ? run_probe<bf16, 128>(a, st) : run_probe<bf16, 64>(a, st);
    return a.d == 128 ? run_probe<float, 128>(a, st) : run_probe<float, 64>(a, st);
}

}  // namespace svg
