// probe_mfma.hip -- value-aware centroid probe on bf16 MFMA for d = 128 and
// Cq <= 256 (steps 2-3 of the SVG-EAR pipeline, review page inference-pipeline
// paragraph; German summary 2B, including its single-pass streaming kernel that
// never writes logits to device memory).
//
// For key cluster g and its keys j (contiguous after reordering) and every
// query cluster c:  s = tau qbar_c.k_j is evaluated with
// v_mfma_f32_16x16x32_bf16: k_j is exact in bf16 and the fp32 centroid qbar_c
// is split exactly into three bf16 planes, so the three products are exact and
// only the fp32 accumulation rounds (absolute error about 2^-24 tau
// sum_t |qbar_t k_t|, independent of how far the key lies from its centroid).
// D = sbar - s with sbar = tau qbar_c.kbar_g (fp64, rounded once); a key equal
// to its centroid in every coordinate gets D = 0 exactly.  The estimate
//     e = e^{2s} [expm1(D)^2 ||vbar_g||^2 + 2 expm1(D) vbar_g.delta_j + ||delta_j||^2],
// s = sbar - D, delta_j = vbar_g - v_j, is rewritten as e = e^{2 sbar} e^{u} f
// with u = 2 max(-D, 0) and f the bracket with e^{-2D} moved inside when D > 0
// (so f never overflows); sum_j e^{u} f is accumulated per (c, g) against a
// shift on u that moves only when some u outgrows it by 2^64.
//
// Work split: a workgroup (4 waves) takes one key cluster at a time.  Per chunk
// of 64 keys its threads load the K and V rows once: the K rows go to LDS (the
// MFMA A operand), and from the V rows they form the per-key scalars
// vbar.delta_j and ||delta_j||^2 (16 lanes per row), so K_p and V_p are each
// read once by the whole probe.  Wave w owns the query-centroid column blocks
// cb = w, w + 4, ... whose bf16 planes stay in its registers for the whole
// launch.  Keys are the MFMA rows, so each lane's partial sums stay in-lane
// until one exchange across the four row groups.
#include "internal.h"

namespace svg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int PR_D = 128;
constexpr int PR_MAXCQ = 256;
constexpr int PR_KC = 64;                   // keys per staged chunk
constexpr int PR_PITCH = PR_D * 2 + 16;     // bytes per key row in LDS (272)
constexpr int PR_LDS = PR_KC * PR_PITCH + PR_KC * 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kShiftStep = 64.f;          // log2 headroom before the shift moves

__device__ __forceinline__ bf16x8_t pr_as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// expm1(a) for a <= 0, given w = e^a: a degree-5 Taylor polynomial near 0
// (truncation below 1.3e-9 relative for |a| <= 1/16), w - 1 elsewhere.
__device__ __forceinline__ float expm1_nonpos(float a, float w)
{
    const float p =
        a * fmaf(a, fmaf(a, fmaf(a, fmaf(a, 1.f / 120.f, 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
    return a > -0.0625f ? p : w - 1.f;
}

// Splits 8 fp32 values exactly into three packed bf16 planes, x = h + m + l
// (round to nearest even at each step; each remainder is exact in fp32).
__device__ __forceinline__ void split8x3(const float x[8], u32x4_t& h, u32x4_t& m, u32x4_t& l)
{
    bf16x8_t a, b, c;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)x[k];
        const float r1 = x[k] - (float)a[k];
        b[k] = (__bf16)r1;
        c[k] = (__bf16)(r1 - (float)b[k]);
    }
    h = __builtin_bit_cast(u32x4_t, a);
    m = __builtin_bit_cast(u32x4_t, b);
    l = __builtin_bit_cast(u32x4_t, c);
}

// Sum over the 16 lanes of a row group (lanes 16 k .. 16 k + 15).
__device__ __forceinline__ float sum16(float v)
{
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 16);
    return v;
}

// With one column block per wave the kernel fits three waves per SIMD (at most
// 168 VGPRs), with two (the three bf16 planes of two blocks stay in registers)
// two waves per SIMD.  A workgroup covers a slice of 4 NCBW column blocks
// (blockIdx.z); with more query clusters than one slice holds, the slices are
// separate workgroups over the same keys (the key-side staging is repeated per
// slice).
template <int NCBW, bool EPS>
__global__ __launch_bounds__(256, NCBW == 1 ? 3 : 2) void k_probe_mfma(
    const float* __restrict__ qbar, const int32_t* __restrict__ counts_q, const bf16* __restrict__ Kp,
    const bf16* __restrict__ Vp, const float* __restrict__ kbar, const float* __restrict__ vbar,
    const float* __restrict__ sbar, const int32_t* __restrict__ offsets_k, int Nk, int Cq, int Ck,
    float tau, int logit_only, float* __restrict__ log_ratio, float* __restrict__ log_eps2)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* const a_k = smem;
    float4* const s_ks = (float4*)(smem + PR_KC * PR_PITCH);   // (vbar.delta, ||delta||^2, equal, -)
    const int h = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;   // A row / D column, and row group
    const int ncb = (Cq + 15) / 16;
    const int cbw = blockIdx.z * 4 * NCBW + wave;   // this wave's first column block
    const int c_lo = blockIdx.z * 4 * NCBW * 16, c_hi = min(Cq, c_lo + 4 * NCBW * 16);

    // B fragments of this wave's column blocks: centroid cb*16 + col, dims
    // 32 ks + 8 grp + 0..7, split exactly into three bf16 planes.
    bf16x8_t bh[NCBW][4], bm[NCBW][4], bl[NCBW][4];
#pragma unroll
    for (int i = 0; i < NCBW; ++i) {
        const int c = (cbw + 4 * i) * 16 + col;
        const bool cv = c < Cq;
        const float* qp = qbar + ((size_t)h * Cq + (cv ? c : 0)) * PR_D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = cv ? qp[32 * ks + e] : 0.f;
            u32x4_t p0, p1, p2;
            split8x3(x, p0, p1, p2);
            bh[i][ks] = pr_as_bf16x8(p0);
            bm[i][ks] = pr_as_bf16x8(p1);
            bl[i][ks] = pr_as_bf16x8(p2);
        }
    }

    const int sch = tid & 15, srow = tid >> 4;   // staging: dims 8 sch.., rows srow + 16 i
    const int32_t* ok = offsets_k + (size_t)h * (Ck + 1);
    for (int g = blockIdx.x; g < Ck; g += gridDim.x) {
        const int j0 = ok[g], j1 = ok[g + 1];
        const int mg = j1 - j0;
        if (mg == 0) {
            for (int c = c_lo + tid; c < c_hi; c += 256) log_ratio[((size_t)h * Cq + c) * Ck + g] = -__builtin_inff();
            continue;
        }
        // this thread's 8 dims of kbar_g and vbar_g; P = ||vbar_g||^2 (1 for the
        // logit-only estimate, whose value terms vanish)
        float kb8[8], vb8[8];
        {
            const float* kbp = kbar + ((size_t)h * Ck + g) * PR_D + 8 * sch;
            const float* vbp = vbar + ((size_t)h * Ck + g) * PR_D + 8 * sch;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kb8[e] = kbp[e];
                vb8[e] = logit_only ? 0.f : vbp[e];
            }
        }
        float P = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) P = fmaf(vb8[e], vb8[e], P);
        P = logit_only ? 1.f : sum16(P);
        float sb[NCBW], sh[NCBW], S[NCBW];
#pragma unroll
        for (int i = 0; i < NCBW; ++i) {
            const int c = (cbw + 4 * i) * 16 + col;
            sb[i] = c < Cq ? sbar[((size_t)h * Cq + c) * Ck + g] : 0.f;
            sh[i] = 0.f;
            S[i] = 0.f;
        }
        for (int jc = j0; jc < j1; jc += PR_KC) {
            const int nv = min(PR_KC, j1 - jc);
            // rows of this chunk: K to LDS as is; per-key scalars from V
            u32x4_t kw[4], vw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jc + min(srow + 16 * i, nv - 1);
                kw[i] = *(const u32x4_t*)(Kp + ((size_t)h * Nk + j) * PR_D + 8 * sch);
                vw[i] = logit_only ? u32x4_t{0, 0, 0, 0} : *(const u32x4_t*)(Vp + ((size_t)h * Nk + j) * PR_D + 8 * sch);
            }
            __syncthreads();   // the previous chunk's readers are done
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = srow + 16 * i;
                *(u32x4_t*)(a_k + r * PR_PITCH + sch * 16) = kw[i];
                float qd = 0.f, rr = 0.f, ne = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned kb = (e & 1) ? (kw[i][e >> 1] & 0xFFFF0000u) : (kw[i][e >> 1] << 16);
                    const unsigned vb = (e & 1) ? (vw[i][e >> 1] & 0xFFFF0000u) : (vw[i][e >> 1] << 16);
                    ne += __uint_as_float(kb) != kb8[e] ? 1.f : 0.f;
                    const float dl = vb8[e] - __uint_as_float(vb);
                    qd = fmaf(vb8[e], dl, qd);
                    rr = fmaf(dl, dl, rr);
                }
                qd = sum16(qd);
                rr = sum16(rr);
                ne = sum16(ne);
                if (sch == 0) s_ks[r] = make_float4(qd, rr, ne == 0.f ? 1.f : 0.f, 0.f);
            }
            __syncthreads();

            const int ntile = (nv + 15) / 16;
            for (int kt = 0; kt < ntile; ++kt) {
                bf16x8_t ak[4];
                const int arow = kt * 16 + col;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    ak[ks] = pr_as_bf16x8(*(const u32x4_t*)(a_k + arow * PR_PITCH + (32 * ks + 8 * grp) * 2));
                const int kr0 = kt * 16 + 4 * grp;   // this lane's rows kr0 .. kr0 + 3
                float4 kq[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) kq[r] = s_ks[kr0 + r];
#pragma unroll
                for (int i = 0; i < NCBW; ++i) {
                    if (cbw + 4 * i >= ncb) continue;   // wave-uniform
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[ks], bh[i][ks], acc, 0, 0, 0);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[ks], bm[i][ks], acc, 0, 0, 0);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[ks], bl[i][ks], acc, 0, 0, 0);
                    float f[4], u[4];
                    float umax = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // D = sbar - s; exactly 0 for a key equal to its centroid
                        const float D = kq[r].z != 0.f ? 0.f : sb[i] - tau * acc[r];
                        const float ad = fabsf(D);
                        const float w = __builtin_amdgcn_exp2f(-ad * kLog2e);   // e^{-|D|}
                        const float em = expm1_nonpos(-ad, w);
                        const bool pos = D > 0.f;
                        const float c1 = pos ? -2.f * em * w : 2.f * em;
                        const float c2 = pos ? w * w : 1.f;
                        const float fr = fmaxf(fmaf(em, em * P, fmaf(c1, kq[r].x, c2 * kq[r].y)), 0.f);
                        f[r] = kr0 + r < nv ? fr : 0.f;
                        // log2 e^{2|D|} for D <= 0; 0 where the term vanishes, so no
                        // exponent of a zero term can overflow
                        u[r] = (pos || !(f[r] > 0.f)) ? 0.f : (2.f * kLog2e) * ad;
                        umax = fmaxf(umax, u[r]);
                    }
                    if (__any(umax > sh[i] + kShiftStep)) {
                        const float ns = fmaxf(sh[i], umax);
                        S[i] *= __builtin_amdgcn_exp2f(sh[i] - ns);
                        sh[i] = ns;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[i] = fmaf(f[r], __builtin_amdgcn_exp2f(u[r] - sh[i]), S[i]);
                    if (EPS) {
                        const int c = (cbw + 4 * i) * 16 + col;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (c < Cq && kr0 + r < nv)
                                log_eps2[((size_t)h * Cq + c) * Nk + jc + kr0 + r] =
                                    f[r] > 0.f ? 2.f * sb[i] + kLn2 * u[r] + logf(f[r]) : -__builtin_inff();
                    }
                }
            }
        }
        // combine the four row groups (lanes col, col + 16, col + 32, col + 48)
#pragma unroll
        for (int i = 0; i < NCBW; ++i) {
            if (cbw + 4 * i >= ncb) continue;
            float m = sh[i], s = S[i];
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float om = __shfl_xor(m, o), os = __shfl_xor(s, o);
                const float mn = fmaxf(m, om);
                s = s * __builtin_amdgcn_exp2f(m - mn) + os * __builtin_amdgcn_exp2f(om - mn);
                m = mn;
            }
            const int c = (cbw + 4 * i) * 16 + col;
            if (grp == 0 && c < Cq) {
                float lr = -__builtin_inff();
                if (counts_q[(size_t)h * Cq + c] > 0 && s > 0.f)
                    lr = 2.f * sb[i] + kLn2 * (m + __log2f(s)) - logf((float)mg);
                log_ratio[((size_t)h * Cq + c) * Ck + g] = lr;
            }
        }
    }
}

SVG_HIDDEN bool probe_mfma_supported(const ProbeArgs& a)
{
    return a.dtype == SVGEAR_BF16 && a.d == PR_D && a.Cq <= PR_MAXCQ;
}

SVG_HIDDEN hipError_t launch_probe_mfma(const ProbeArgs& a, const float* sbar, hipStream_t st)
{
    const int ncb = (a.Cq + 15) / 16;
    const int ncbw = ncb > 4 ? 2 : 1;                  // column blocks per wave
    const int slices = (ncb + 4 * ncbw - 1) / (4 * ncbw);
    // about 1536 workgroups in all: two rounds of three per CU (measured best of
    // 768 to 2304 at the Wan and HunyuanVideo shapes)
    int gx = (1536 + a.H * slices - 1) / (a.H * slices);
    if (gx > a.Ck) gx = a.Ck;
    float* eps = (a.flags & SVGEAR_DEBUG_EPS) ? a.log_eps2 : nullptr;
    const int logit_only = (a.flags & SVGEAR_PROBE_LOGIT) ? 1 : 0;
    const float tau = 1.0f / sqrtf((float)PR_D);
#define SVG_PROBE_CASE(n)                                                                          \
    case n:                                                                                        \
        if (eps)                                                                                   \
            hipLaunchKernelGGL((k_probe_mfma<n, true>), dim3(gx, a.H, slices), dim3(256), PR_LDS, st, \
                               a.qbar, a.counts_q, (const bf16*)a.Kp, (const bf16*)a.Vp, a.kbar,   \
                               a.vbar, sbar, a.offsets_k, a.Nk, a.Cq, a.Ck, tau, logit_only,       \
                               a.log_ratio, eps);                                                  \
        else                                                                                       \
            hipLaunchKernelGGL((k_probe_mfma<n, false>), dim3(gx, a.H, slices), dim3(256), PR_LDS, st, \
                               a.qbar, a.counts_q, (const bf16*)a.Kp, (const bf16*)a.Vp, a.kbar,   \
                               a.vbar, sbar, a.offsets_k, a.Nk, a.Cq, a.Ck, tau, logit_only,       \
                               a.log_ratio, eps);                                                  \
        break;
    switch (ncbw) {
        SVG_PROBE_CASE(1) SVG_PROBE_CASE(2)
    default: return hipErrorInvalidValue;
    }
#undef SVG_PROBE_CASE
    return hipGetLastError();
}

}  // namespace svg
