// attn_mfma.hip -- hybrid attention on bf16 MFMA for d = 128 (step 4 of the
// SVG-EAR pipeline: exact blocks plus parameter-free centroid compensation,
// review page inference-pipeline paragraph; German summary 2A).
//
// One workgroup (4 waves) owns a tile of BM = 128 reordered query rows of one
// query cluster c; each wave owns 32 queries.  Scores are computed transposed,
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every lane holds one query
// column and the softmax row statistics stay inside a lane (one exchange with
// the partner half-wave per tile for the running max).  The probabilities are
// already laid out as the B operand of O^T = V^T P^T, provided the value tile
// is stored transposed in LDS with key slots permuted (bits 2 and 3 of the key
// index swapped), so each lane reads its 8 keys with one 16-byte load.
//
// Key tiles of BN = 64:
//   1. compensation tiles: the centroids of all key clusters, split into bf16
//      hi + lo planes (k-bar and v-bar are fp32), logits tau q.kbar_g + ln m_g,
//      masked to the clusters that are skipped for c and non-empty;
//   2. exact tiles: the keys of every routed (mask = 1) key cluster, segment by
//      segment (a segment's last tile is masked), K/V double-buffered in LDS
//      with the next tile's global loads in flight during the current tile.
// One online softmax (base-2 exponent) covers both kinds of terms.
#include "internal.h"

namespace svg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int AT_BM = 128;
constexpr int AT_BN = 64;
constexpr int AT_D = 128;
constexpr int AT_THREADS = 256;
constexpr int K_PITCH = AT_D * 2 + 16;   // bytes per key row of a K tile in LDS
constexpr int V_PITCH = AT_BN * 2 + 16;  // bytes per d row of a transposed V tile
constexpr int K_BUF = AT_BN * K_PITCH;   // 17408
constexpr int V_BUF = AT_D * V_PITCH;    // 18432
constexpr int AT_LDS = 2 * K_BUF + 2 * V_BUF + AT_BN * 4;

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// ----------------------------------------------------------------------------- prep kernels

// Split centroids into bf16 hi/lo planes; ln m_g in base-2 units (-inf if empty).
__global__ void k_comp_planes(const float* __restrict__ kbar, const float* __restrict__ vbar,
                              const int32_t* __restrict__ counts_k, int Ck, bf16* __restrict__ kbh,
                              bf16* __restrict__ kbl, bf16* __restrict__ vbh, bf16* __restrict__ vbl,
                              float* __restrict__ logm2)
{
    const int g = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const size_t i = ((size_t)h * Ck + g) * AT_D + t;
    const float k = kbar[i], v = vbar[i];
    const bf16 kh = f32_to_bf16(k), vh = f32_to_bf16(v);
    kbh[i] = kh;
    kbl[i] = f32_to_bf16(k - bf16_to_f32(kh));
    vbh[i] = vh;
    vbl[i] = f32_to_bf16(v - bf16_to_f32(vh));
    if (t == 0) {
        const int m = counts_k[(size_t)h * Ck + g];
        logm2[(size_t)h * Ck + g] = m > 0 ? log2f((float)m) : -__builtin_inff();
    }
}

// Routed key segments of each (head, query cluster), in key-cluster order:
// (first reordered key, length) of every g with mask[c, g] = 1 and m_g > 0.
__global__ __launch_bounds__(256) void k_seg_list(const uint8_t* __restrict__ mask,
                                                  const int32_t* __restrict__ offsets_k, int Cq,
                                                  int Ck, int2* __restrict__ segs,
                                                  int* __restrict__ nsegs)
{
    __shared__ int s_cnt[256];
    const int c = blockIdx.x, h = blockIdx.y;
    const uint8_t* mrow = mask + ((size_t)h * Cq + c) * Ck;
    const int32_t* ok = offsets_k + (size_t)h * (Ck + 1);
    int2* out = segs + ((size_t)h * Cq + c) * Ck;
    int base = 0;
    for (int g0 = 0; g0 < Ck; g0 += 256) {
        const int g = g0 + threadIdx.x;
        int sel = 0, start = 0, len = 0;
        if (g < Ck) {
            start = ok[g];
            len = ok[g + 1] - start;
            sel = mrow[g] && len > 0;
        }
        s_cnt[threadIdx.x] = sel;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            int v = threadIdx.x >= off ? s_cnt[threadIdx.x - off] : 0;
            __syncthreads();
            s_cnt[threadIdx.x] += v;
            __syncthreads();
        }
        if (sel) out[base + s_cnt[threadIdx.x] - 1] = make_int2(start, len);
        base += s_cnt[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) nsegs[(size_t)h * Cq + c] = base;
}

// Per head: first query tile of each cluster (exclusive prefix of ceil(n_c/BM)).
__global__ __launch_bounds__(1024) void k_tile_prefix(const int32_t* __restrict__ offsets_q, int Cq,
                                                      int* __restrict__ tstart)
{
    __shared__ int s_part[1024];
    const int h = blockIdx.x;
    const int32_t* oq = offsets_q + (size_t)h * (Cq + 1);
    const int per = (Cq + 1023) / 1024;
    const int c0 = threadIdx.x * per;
    int local = 0;
    for (int k = 0; k < per; ++k)
        if (c0 + k < Cq) local += (oq[c0 + k + 1] - oq[c0 + k] + AT_BM - 1) / AT_BM;
    s_part[threadIdx.x] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
        __syncthreads();
        s_part[threadIdx.x] += v;
        __syncthreads();
    }
    int run = s_part[threadIdx.x] - local;
    int* ts = tstart + (size_t)h * (Cq + 1);
    for (int k = 0; k < per; ++k) {
        if (c0 + k < Cq) {
            ts[c0 + k] = run;
            run += (oq[c0 + k + 1] - oq[c0 + k] + AT_BM - 1) / AT_BM;
        }
    }
    if (threadIdx.x == 1023) ts[Cq] = s_part[1023];
}

// ----------------------------------------------------------------------------- tile staging

struct Stage {
    u32x4_t k[4];  // rows kr + 16 i, chunk kc
    u32x4_t v[4];  // keys 4 vg + i, chunk vc
};

// Global -> registers.  Rows at or beyond nvalid are zero.
__device__ __forceinline__ void stage_load(Stage& s, const bf16* __restrict__ Kbase,
                                           const bf16* __restrict__ Vbase, int nvalid, int tid)
{
    const int kc = tid & 15, kr = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = kr + 16 * i;
        s.k[i] = r < nvalid ? *(const u32x4_t*)(Kbase + (size_t)r * AT_D + kc * 8) : u32x4_t{0, 0, 0, 0};
    }
    const int vc = tid & 15, vg = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * vg + i;
        s.v[i] = r < nvalid ? *(const u32x4_t*)(Vbase + (size_t)r * AT_D + vc * 8) : u32x4_t{0, 0, 0, 0};
    }
}

// Registers -> LDS: K row-major, V transposed with permuted key slots.
__device__ __forceinline__ void stage_store(const Stage& s, char* kbuf, char* vbuf, int tid)
{
    const int kc = tid & 15, kr = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4_t*)(kbuf + (kr + 16 * i) * K_PITCH + kc * 16) = s.k[i];
    const int vc = tid & 15, vg = tid >> 4;
    const int key0 = 4 * vg;
    const int slot0 = (key0 & 32) + swap23(key0 & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // d = 8 vc + 2j (low halves) and 8 vc + 2j + 1 (high halves)
        const unsigned a0 = s.v[0][j], a1 = s.v[1][j], a2 = s.v[2][j], a3 = s.v[3][j];
        u32x2_t lo, hi;
        lo[0] = (a0 & 0xFFFFu) | (a1 << 16);
        lo[1] = (a2 & 0xFFFFu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
        const int d = 8 * vc + 2 * j;
        *(u32x2_t*)(vbuf + d * V_PITCH + slot0 * 2) = lo;
        *(u32x2_t*)(vbuf + (d + 1) * V_PITCH + slot0 * 2) = hi;
    }
}

// ----------------------------------------------------------------------------- per-tile math

struct Softmax {
    float m;      // running max (base-2 logits), shared by both half-waves
    float l;      // this half-wave's partial sum of probabilities
    f32x16_t o[4];  // O^T blocks: d rows 32 db + ..., query column lane & 31
};

// S^T for a 64-key tile: two 32x32 blocks.
__device__ __forceinline__ void tile_scores(f32x16_t acc[2], const char* kbuf, const bf16x8_t qf[8],
                                            int lane)
{
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        f32x16_t a = {0};
        const char* kr = kbuf + (kb * 32 + row) * K_PITCH + half * 16;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8_t kf = as_bf16x8(*(const u32x4_t*)(kr + s * 32));
            a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], a, 0, 0, 0);
        }
        acc[kb] = a;
    }
}

__device__ __forceinline__ void tile_scores_acc(f32x16_t acc[2], const char* kbuf,
                                                const bf16x8_t qf[8], int lane)
{
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        f32x16_t a = acc[kb];
        const char* kr = kbuf + (kb * 32 + row) * K_PITCH + half * 16;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8_t kf = as_bf16x8(*(const u32x4_t*)(kr + s * 32));
            a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], a, 0, 0, 0);
        }
        acc[kb] = a;
    }
}

// Online softmax update with the tile's base-2 logits x[kb][i]; returns the
// probabilities as PV B-operand fragments pf[kb*2 + ks].
__device__ __forceinline__ void softmax_update(Softmax& st, f32x16_t x[2], bf16x8_t pf[4])
{
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[kb][i]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(st.m, mloc);
    const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(st.m - muse);
    st.m = mnew;
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8_t f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = __builtin_amdgcn_exp2f(x[kb][8 * ks + i] - muse);
                sum += p;
                f[i] = (__bf16)p;
            }
            pf[kb * 2 + ks] = f;
        }
    }
    st.l = fmaf(st.l, alpha, sum);
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db] *= alpha;
}

// O^T += V^T P^T for one 64-key tile held transposed in vbuf.
__device__ __forceinline__ void tile_pv(Softmax& st, const char* vbuf, const bf16x8_t pf[4], int lane)
{
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const char* vr = vbuf + (db * 32 + row) * V_PITCH + half * 16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {  // kk = kb * 2 + ks: slots 16 kk + 8 half
            const bf16x8_t vf = as_bf16x8(*(const u32x4_t*)(vr + kk * 32));
            st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], st.o[db], 0, 0, 0);
        }
    }
}

// ----------------------------------------------------------------------------- main kernel

__global__ __launch_bounds__(AT_THREADS, 2) void k_attn_mfma(
    const bf16* __restrict__ Qp, const int32_t* __restrict__ offsets_q,
    const int32_t* __restrict__ perm_q, const bf16* __restrict__ Kp, const bf16* __restrict__ Vp,
    const bf16* __restrict__ kbh, const bf16* __restrict__ kbl, const bf16* __restrict__ vbh,
    const bf16* __restrict__ vbl, const float* __restrict__ logm2, const uint8_t* __restrict__ mask,
    const int2* __restrict__ segs, const int* __restrict__ nsegs, const int* __restrict__ tstart,
    int Nq, int Nk, int Cq, int Ck, float scale2, bf16* __restrict__ O)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* const kbuf0 = smem;
    char* const vbuf0 = smem + 2 * K_BUF;
    float* s_bias = (float*)(smem + 2 * K_BUF + 2 * V_BUF);
#define KBUF(b) (kbuf0 + (b) * K_BUF)
#define VBUF(b) (vbuf0 + (b) * V_BUF)

    const int h = blockIdx.y, t = blockIdx.x;
    const int* ts = tstart + (size_t)h * (Cq + 1);
    if (t >= ts[Cq]) return;
    int lo = 0, hi = Cq - 1;  // query cluster: last c with ts[c] <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ts[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int c = lo;
    const int32_t* oq = offsets_q + (size_t)h * (Cq + 1);
    const int q0 = oq[c] + (t - ts[c]) * AT_BM;
    const int nrows = min(AT_BM, oq[c + 1] - q0);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int qcol = lane & 31, half = lane >> 5;

    // Q^T fragments (B operand): query q0 + 32 wave + qcol, dims 16 s + 8 half + 0..7.
    bf16x8_t qf[8];
    {
        const int r = wave * 32 + qcol;
        const int qrow = q0 + (r < nrows ? r : 0);
        const bf16* qp = Qp + ((size_t)h * Nq + qrow) * AT_D + half * 8;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*(const u32x4_t*)(qp + 16 * s));
    }

    Softmax st;
    st.m = -__builtin_inff();
    st.l = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db] = f32x16_t{0};

    const uint8_t* mrow = mask + ((size_t)h * Cq + c) * Ck;
    const float* lm = logm2 + (size_t)h * Ck;

    // 1. compensation tiles
    for (int g0 = 0; g0 < Ck; g0 += AT_BN) {
        const int nv = min(AT_BN, Ck - g0);
        float b = -__builtin_inff();
        if (tid < AT_BN && tid < nv && !mrow[g0 + tid]) b = lm[g0 + tid];
        if (!__syncthreads_or(b != -__builtin_inff())) continue;
        if (tid < AT_BN) s_bias[tid] = b;
        Stage sh, sl;
        const size_t cb = ((size_t)h * Ck + g0) * AT_D;
        stage_load(sh, kbh + cb, vbh + cb, nv, tid);
        stage_load(sl, kbl + cb, vbl + cb, nv, tid);
        stage_store(sh, KBUF(0), VBUF(0), tid);
        stage_store(sl, KBUF(1), VBUF(1), tid);
        __syncthreads();
        f32x16_t acc[2];
        tile_scores(acc, KBUF(0), qf, lane);
        tile_scores_acc(acc, KBUF(1), qf, lane);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kt = kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                acc[kb][i] = fmaf(acc[kb][i], scale2, s_bias[kt]);
            }
        bf16x8_t pf[4];
        softmax_update(st, acc, pf);
        tile_pv(st, VBUF(0), pf, lane);
        tile_pv(st, VBUF(1), pf, lane);
        __syncthreads();
    }

    // 2. exact tiles, double-buffered
    const int ns = nsegs[(size_t)h * Cq + c];
    const int2* sl = segs + ((size_t)h * Cq + c) * Ck;
    const bf16* Kh = Kp + (size_t)h * Nk * AT_D;
    const bf16* Vh = Vp + (size_t)h * Nk * AT_D;
    if (ns > 0) {
        int si = 0, off = 0;
        int2 sg = sl[0];
        int cur_start = sg.x, cur_n = min(AT_BN, sg.y);
        Stage sbuf;
        stage_load(sbuf, Kh + (size_t)cur_start * AT_D, Vh + (size_t)cur_start * AT_D, cur_n, tid);
        stage_store(sbuf, KBUF(0), VBUF(0), tid);
        __syncthreads();
        int buf = 0;
        while (true) {
            // advance to the next tile
            off += AT_BN;
            if (off >= sg.y) {
                ++si;
                off = 0;
                if (si < ns) sg = sl[si];
            }
            const bool has_next = si < ns;
            const int nxt_start = sg.x + off;
            const int nxt_n = has_next ? min(AT_BN, sg.y - off) : 0;
            if (has_next)
                stage_load(sbuf, Kh + (size_t)nxt_start * AT_D, Vh + (size_t)nxt_start * AT_D, nxt_n,
                           tid);
            f32x16_t acc[2];
            tile_scores(acc, KBUF(buf), qf, lane);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kt = kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                    acc[kb][i] = kt < cur_n ? acc[kb][i] * scale2 : -__builtin_inff();
                }
            bf16x8_t pf[4];
            softmax_update(st, acc, pf);
            tile_pv(st, VBUF(buf), pf, lane);
            if (!has_next) break;
            stage_store(sbuf, KBUF(buf ^ 1), VBUF(buf ^ 1), tid);
            __syncthreads();
            buf ^= 1;
            cur_n = nxt_n;
        }
    }

    // 3. normalise, stage the tile in LDS as [query][d], store rows in token order
    const float ltot = st.l + __shfl_xor(st.l, 32);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    __syncthreads();
#undef KBUF
#undef VBUF
    char* ost = smem;  // 128 rows x K_PITCH bytes = 2 K buffers
    {
        const int r = wave * 32 + qcol;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + g4 * 8 + half * 4;
                u32x2_t w;
                w[0] = (unsigned)f32_to_bf16(st.o[db][4 * g4 + 0] * inv) |
                       ((unsigned)f32_to_bf16(st.o[db][4 * g4 + 1] * inv) << 16);
                w[1] = (unsigned)f32_to_bf16(st.o[db][4 * g4 + 2] * inv) |
                       ((unsigned)f32_to_bf16(st.o[db][4 * g4 + 3] * inv) << 16);
                *(u32x2_t*)(ost + r * K_PITCH + d * 2) = w;
            }
    }
    __syncthreads();
    const int32_t* pq = perm_q + (size_t)h * Nq + q0;
    for (int k = tid; k < AT_BM * 16; k += AT_THREADS) {
        const int r = k >> 4, ch = k & 15;
        if (r < nrows) {
            const int tok = pq[r];
            *(u32x4_t*)(O + ((size_t)h * Nq + tok) * AT_D + ch * 8) =
                *(const u32x4_t*)(ost + r * K_PITCH + ch * 16);
        }
    }
}

// ----------------------------------------------------------------------------- dispatch

SVG_HIDDEN bool attention_mfma_supported(const AttnArgs& a)
{
    return a.dtype == SVGEAR_BF16 && a.d == AT_D;
}

SVG_HIDDEN hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t st)
{
    const Layout& L = *a.L;
    char* s = a.scratch;
    const size_t plane = (size_t)a.H * a.Ck * AT_D;
    bf16* kbh = (bf16*)(s + L.at_kvplanes);
    bf16* kbl = kbh + plane;
    bf16* vbh = kbl + plane;
    bf16* vbl = vbh + plane;
    float* logm2 = (float*)(s + L.at_logm);
    int* tstart = (int*)(s + L.at_tiles);
    int2* segs = (int2*)(s + L.at_segs);
    int* nsegs = (int*)(s + L.at_nsegs);
    hipLaunchKernelGGL(k_comp_planes, dim3(a.Ck, a.H), dim3(AT_D), 0, st, a.kbar, a.vbar, a.counts_k,
                       a.Ck, kbh, kbl, vbh, vbl, logm2);
    hipLaunchKernelGGL(k_seg_list, dim3(a.Cq, a.H), dim3(256), 0, st, a.mask, a.offsets_k, a.Cq,
                       a.Ck, segs, nsegs);
    hipLaunchKernelGGL(k_tile_prefix, dim3(a.H), dim3(1024), 0, st, a.offsets_q, a.Cq, tstart);
    const int max_tiles = (a.Nq + AT_BM - 1) / AT_BM + a.Cq;
    const float scale2 = (float)(1.4426950408889634 / sqrt((double)AT_D));
    hipLaunchKernelGGL(k_attn_mfma, dim3(max_tiles, a.H), dim3(AT_THREADS), AT_LDS, st,
                       (const bf16*)a.Qp, a.offsets_q, a.perm_q, (const bf16*)a.Kp,
                       (const bf16*)a.Vp, kbh, kbl, vbh, vbl, logm2, a.mask, segs, nsegs, tstart,
                       a.Nq, a.Nk, a.Cq, a.Ck, scale2, (bf16*)a.O);
    return hipGetLastError();
}

}  // namespace svg
