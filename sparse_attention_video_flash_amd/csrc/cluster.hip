// cluster.hip -- step 1 of the SVG-EAR pipeline (review page, inference-pipeline
// paragraph, step 1; German summary 2A): Flash k-means of Q and K, stable
// counting-sort reordering so that same-cluster tokens are contiguous, and the
// centroid means (V-bar over K's clusters).
//
// Exactness strategy.  The assignment picks the nearest centroid in squared
// Euclidean distance with ties to the lowest index.  Centroids are kept in fp64
// and are the exact member means: member rows are summed as 64-bit fixed-point
// integers (every bf16/fp32 input with |x| < 256 and magnitude above 2^-S is an
// exact multiple of 2^-S), so the sum is order-independent and integer atomics
// keep it deterministic; one rounding to fp64 and one fp64 division follow.
// Distances are either evaluated directly in fp64 (generic kernel) or screened
// with bf16 MFMA and re-evaluated in fp64 whenever the screen cannot separate
// the best two candidates (assign_mfma.hip).
#include "internal.h"

namespace svg {

__global__ void k_zero_words(uint32_t* __restrict__ p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

SVG_HIDDEN void zero_words(void* p, size_t bytes, hipStream_t st)
{
    size_t n = bytes / 4;
    if (n == 0) return;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero_words, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)p, n);
}

// Initial centroids: the rows X[h, init[h, m]].
template <typename T>
__global__ void k_init_centroids(const T* __restrict__ X, const int32_t* __restrict__ init, int N,
                                 int d, int C, double* __restrict__ cent64, int* __restrict__ err)
{
    const int m = blockIdx.x, h = blockIdx.y;
    int idx = init[(size_t)h * C + m];
    if (idx < 0 || idx >= N) {
        if (threadIdx.x == 0) atomicOr(err, ERR_INIT_INDEX);
        idx = idx < 0 ? 0 : N - 1;
    }
    for (int t = threadIdx.x; t < d; t += blockDim.x)
        cent64[((size_t)h * C + m) * d + t] = (double)to_f32<T>(X[((size_t)h * N + idx) * d + t]);
}

// Exact assignment: distance sum_t (x_t - c_t)^2 in fp64, coordinate order,
// no contraction; strict '<' keeps the lowest index on ties.  One token per
// thread, centroids staged through LDS in chunks.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_assign_exact(const T* __restrict__ X,
                                                      const double* __restrict__ cent64, int N,
                                                      int C, int32_t* __restrict__ labels)
{
#pragma clang fp contract(off)
    constexpr int CH = 32768 / (D * 8);  // centroids per 32 KB chunk
    __shared__ double s_c[CH * D];
    const int h = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    float xr[D];  // exact copies of the inputs
    if (i < N) {
        const T* x = X + ((size_t)h * N + i) * D;
#pragma unroll
        for (int t = 0; t < D; ++t) xr[t] = to_f32<T>(x[t]);
    }
    double best = __builtin_inf();
    int bi = 0;
    const double* cb = cent64 + (size_t)h * C * D;
    for (int m0 = 0; m0 < C; m0 += CH) {
        const int cn = min(CH, C - m0);
        __syncthreads();
        for (int k = threadIdx.x; k < cn * D; k += 256) s_c[k] = cb[(size_t)m0 * D + k];
        __syncthreads();
        if (i < N) {
            for (int m = 0; m < cn; ++m) {
                double s = 0.0;
#pragma unroll 16
                for (int t = 0; t < D; ++t) {
                    double u = __dsub_rn((double)xr[t], s_c[m * D + t]);
                    s = __dadd_rn(s, __dmul_rn(u, u));
                }
                if (s < best) {
                    best = s;
                    bi = m0 + m;
                }
            }
        }
    }
    if (i < N) labels[(size_t)h * N + i] = bi;
}

// Exact member sums.  Each wave walks 64 consecutive tokens; a run of equal
// labels is accumulated in 64-bit fixed point (scale 2^shift) and flushed with
// one integer atomic per coordinate, plus the run length into the count.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_fixed_sums(const T* __restrict__ X,
                                                    const int32_t* __restrict__ labels, int N,
                                                    int C, int shift,
                                                    unsigned long long* __restrict__ sums,
                                                    int* __restrict__ cnt, int* __restrict__ err)
{
    constexpr int EPL = D / 64;
    const int h = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i0 = (blockIdx.x * 4 + wave) * 64;
    if (i0 >= N) return;
    const int i1 = min(i0 + 64, N);
    const double scale = ldexp(1.0, shift);
    const int32_t* lab = labels + (size_t)h * N;
    long long acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0;
    int cur = lab[i0], run = 0;
    auto flush = [&]() {
        if (cur >= 0 && cur < C) {
            unsigned long long* s = sums + ((size_t)h * C + cur) * D + lane * EPL;
#pragma unroll
            for (int e = 0; e < EPL; ++e) atomicAdd(s + e, (unsigned long long)acc[e]);
            if (lane == 0) atomicAdd(cnt + (size_t)h * C + cur, run);
        } else if (lane == 0) {
            atomicOr(err, ERR_LABEL);
        }
    };
    for (int i = i0; i < i1; ++i) {
        const int l = lab[i];
        if (l != cur) {
            flush();
            cur = l;
            run = 0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = 0;
        }
        const T* x = X + ((size_t)h * N + i) * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += (long long)((double)to_f32<T>(x[e]) * scale);
        ++run;
    }
    flush();
}

// Centroid = exact sum / count in fp64; an empty cluster keeps its centroid
// (k-means) or becomes zero (plain means).  Optionally writes fp32 copies and
// the counts; then clears the sums and counts for the next pass.
__global__ void k_finalize_means(unsigned long long* __restrict__ sums, int* __restrict__ cnt,
                                 int d, int C, int shift, int zero_empty, double* __restrict__ cent64,
                                 float* __restrict__ cent_out)
{
    const int m = blockIdx.x, h = blockIdx.y;
    const size_t row = (size_t)h * C + m;
    const int n = cnt[row];
    const double inv_scale = ldexp(1.0, -shift);
    for (int t = threadIdx.x; t < d; t += blockDim.x) {
        double c;
        if (n > 0) {
            c = ((double)(long long)sums[row * d + t] * inv_scale) / (double)n;
            cent64[row * d + t] = c;
        } else if (zero_empty) {
            c = 0.0;
            cent64[row * d + t] = c;
        } else {
            c = cent64[row * d + t];
        }
        if (cent_out) cent_out[row * d + t] = (float)c;
        sums[row * d + t] = 0ull;
    }
    __syncthreads();
    if (threadIdx.x == 0) cnt[row] = 0;
}

// ----------------------------------------------------------------------------- counting sort

// Per-tile label histogram (tiles of kTile consecutive tokens).
__global__ __launch_bounds__(256) void k_tile_hist(const int32_t* __restrict__ labels, int N, int C,
                                                   int ntiles, int* __restrict__ hist,
                                                   int* __restrict__ err)
{
    extern __shared__ int s_h[];
    const int tile = blockIdx.x, h = blockIdx.y;
    for (int c = threadIdx.x; c < C; c += 256) s_h[c] = 0;
    __syncthreads();
    const int i = tile * kTile + threadIdx.x;
    if (i < N) {
        int l = labels[(size_t)h * N + i];
        if (l < 0 || l >= C) {
            atomicOr(err, ERR_LABEL);
        } else {
            atomicAdd(&s_h[l], 1);
        }
    }
    __syncthreads();
    int* out = hist + ((size_t)h * ntiles + tile) * C;
    for (int c = threadIdx.x; c < C; c += 256) out[c] = s_h[c];
}

// Per head: exclusive prefix of every label's tile counts (in place), the
// label counts, and their exclusive prefix (cluster offsets).
__global__ __launch_bounds__(1024) void k_hist_scan(int* __restrict__ hist, int C, int ntiles,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets)
{
    __shared__ int s_part[1024];
    const int h = blockIdx.x;
    int* hb = hist + (size_t)h * ntiles * C;
    for (int c = threadIdx.x; c < C; c += 1024) {
        int run = 0;
        for (int t = 0; t < ntiles; ++t) {
            int v = hb[(size_t)t * C + c];
            hb[(size_t)t * C + c] = run;
            run += v;
        }
        counts[(size_t)h * C + c] = run;
    }
    __syncthreads();
    // exclusive scan of counts[h, 0..C): each thread owns a contiguous chunk
    const int per = (C + 1023) / 1024;
    const int c0 = threadIdx.x * per;
    int local = 0;
    for (int k = 0; k < per; ++k)
        if (c0 + k < C) local += counts[(size_t)h * C + c0 + k];
    s_part[threadIdx.x] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
        __syncthreads();
        s_part[threadIdx.x] += v;
        __syncthreads();
    }
    int run = s_part[threadIdx.x] - local;
    for (int k = 0; k < per; ++k) {
        if (c0 + k < C) {
            offsets[(size_t)h * (C + 1) + c0 + k] = run;
            run += counts[(size_t)h * C + c0 + k];
        }
    }
    if (threadIdx.x == 1023) offsets[(size_t)h * (C + 1) + C] = s_part[1023];
}

// Stable scatter: position = offset of the label + tokens of that label in
// earlier tiles + earlier tokens of that label in this tile.  Copies the rows
// of X (and V) to their reordered positions.
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ labels, int N, int C,
                                                 int ntiles, const int* __restrict__ hist,
                                                 const int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm,
                                                 int32_t* __restrict__ inv_perm,
                                                 const uint4* __restrict__ X, uint4* __restrict__ Xp,
                                                 const uint4* __restrict__ V, uint4* __restrict__ Vp,
                                                 int row_chunks)
{
    __shared__ int s_lab[kTile];
    __shared__ int s_pos[kTile];
    const int tile = blockIdx.x, h = blockIdx.y;
    const int i = tile * kTile + threadIdx.x;
    int l = -1;
    if (i < N) {
        l = labels[(size_t)h * N + i];
        if (l < 0 || l >= C) l = -1;  // reported by k_tile_hist
    }
    s_lab[threadIdx.x] = l;
    __syncthreads();
    int pos = -1;
    if (l >= 0) {
        int rank = 0;
        for (int j = 0; j < (int)threadIdx.x; ++j) rank += (s_lab[j] == l);
        pos = offsets[(size_t)h * (C + 1) + l] + hist[((size_t)h * ntiles + tile) * C + l] + rank;
        perm[(size_t)h * N + pos] = i;
        inv_perm[(size_t)h * N + i] = pos;
    }
    s_pos[threadIdx.x] = pos;
    __syncthreads();
    if (!X) return;
    const int rows = min(kTile, N - tile * kTile);
    for (int k = threadIdx.x; k < rows * row_chunks; k += 256) {
        const int r = k / row_chunks, ch = k - r * row_chunks;
        const int p = s_pos[r];
        if (p < 0) continue;
        const size_t src = ((size_t)h * N + tile * kTile + r) * row_chunks + ch;
        const size_t dst = ((size_t)h * N + p) * row_chunks + ch;
        Xp[dst] = X[src];
        if (V) Vp[dst] = V[src];
    }
}

// ----------------------------------------------------------------------------- driver

SVG_HIDDEN hipError_t launch_assign_mfma(const ClusterArgs& a, const double* cent64, int* err,
                                         hipStream_t st);
SVG_HIDDEN bool assign_mfma_supported(const ClusterArgs& a);

template <typename T, int D>
static hipError_t run_cluster(const ClusterArgs& a, hipStream_t st)
{
    const Layout& L = *a.L;
    char* s = a.scratch;
    int* err = (int*)(s + L.cl_err);
    double* cent64 = (double*)(s + L.cl_cent64);
    unsigned long long* sums = (unsigned long long*)(s + L.cl_sums);
    int* cnt = (int*)(s + L.cl_cnt);
    int* hist = (int*)(s + L.cl_hist);
    const int H = a.H, N = a.N, C = a.C;
    const T* X = (const T*)a.X;
    const dim3 grid_sums((N + 255) / 256, H), grid_cent(C, H);
    const int cthreads = D;

    zero_words(sums, (size_t)H * C * D * 8, st);
    zero_words(cnt, (size_t)H * C * 4, st);

    if (!(a.flags & SVGEAR_LABELS_GIVEN)) {
        hipLaunchKernelGGL((k_init_centroids<T>), grid_cent, dim3(cthreads), 0, st, X, a.init, N,
                           D, C, cent64, err);
        const bool mfma = assign_mfma_supported(a);
        for (int it = 0; it < a.iters; ++it) {
            if (mfma) {
                hipError_t e = launch_assign_mfma(a, cent64, err, st);
                if (e != hipSuccess) return e;
            } else {
                hipLaunchKernelGGL((k_assign_exact<T, D>), dim3((N + 255) / 256, H), dim3(256), 0,
                                   st, X, cent64, N, C, a.labels);
            }
            hipLaunchKernelGGL((k_fixed_sums<T, D>), grid_sums, dim3(256), 0, st, X, a.labels, N, C,
                               a.shift, sums, cnt, err);
            const bool last = it == a.iters - 1;
            hipLaunchKernelGGL(k_finalize_means, grid_cent, dim3(cthreads), 0, st, sums, cnt, D, C,
                               a.shift, 0, cent64, last ? a.cent : (float*)nullptr);
        }
    } else {
        hipLaunchKernelGGL((k_fixed_sums<T, D>), grid_sums, dim3(256), 0, st, X, a.labels, N, C,
                           a.shift, sums, cnt, err);
        hipLaunchKernelGGL(k_finalize_means, grid_cent, dim3(cthreads), 0, st, sums, cnt, D, C,
                           a.shift, 1, cent64, a.cent);
    }

    // Reorder (stable counting sort) and gather rows.
    const int ntiles = (N + kTile - 1) / kTile;
    hipLaunchKernelGGL(k_tile_hist, dim3(ntiles, H), dim3(256), (size_t)C * 4, st, a.labels, N, C,
                       ntiles, hist, err);
    hipLaunchKernelGGL(k_hist_scan, dim3(H), dim3(1024), 0, st, hist, C, ntiles, a.counts,
                       a.offsets);
    const int row_chunks = (int)(D * sizeof(T) / 16);
    hipLaunchKernelGGL(k_scatter, dim3(ntiles, H), dim3(256), 0, st, a.labels, N, C, ntiles, hist,
                       a.offsets, a.perm, a.inv_perm, (const uint4*)a.X, (uint4*)a.Xp,
                       (const uint4*)a.V, (uint4*)a.Vp, row_chunks);

    // V-bar: mean of V over the key clusters (zero for an empty cluster).
    if (a.side == 1) {
        hipLaunchKernelGGL((k_fixed_sums<T, D>), grid_sums, dim3(256), 0, st, (const T*)a.V,
                           a.labels, N, C, a.shift, sums, cnt, err);
        hipLaunchKernelGGL(k_finalize_means, grid_cent, dim3(cthreads), 0, st, sums, cnt, D, C,
                           a.shift, 1, cent64, a.vbar);
    }
    return hipGetLastError();
}

SVG_HIDDEN hipError_t launch_cluster(const ClusterArgs& a, hipStream_t st)
{
    if (a.dtype == SVGEAR_BF16) {
        return a.d == 128 ? run_cluster<bf16, 128>(a, st) : run_cluster<bf16, 64>(a, st);
    }
    return a.d == 128 ? run_cluster<float, 128>(a, st) : run_cluster<float, 64>(a, st);
}

}  // namespace svg
