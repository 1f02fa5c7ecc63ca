// cluster.hip -- step 1 of the SVG-EAR pipeline (review page, inference-pipeline
// paragraph, step 1; German summary 2A): Flash k-means of Q and K, stable
// counting-sort reordering so that same-cluster tokens are contiguous, and the
// centroid means (V-bar over K's clusters).
//
// Exactness strategy.  The assignment picks the nearest centroid in squared
// Euclidean distance with ties to the lowest index.  Centroids are kept in fp64
// and are the exact member means: member rows are summed as 64-bit fixed-point
// integers (every bf16/fp32 input with |x| < 256 and magnitude above 2^-S is an
// exact multiple of 2^-S), so the sum does not depend on the order of the rows;
// one rounding to fp64 and one fp64 division follow.  Each update buckets the
// token ids by label and one block per cluster sums its rows (no atomics).
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

// Per-label exclusive prefix of the tile counts, in place, and the label
// counts.  One block per 32 labels of a head, 64 tiles per pass: thread
// (group g, label) holds tiles 8 g .. 8 g + 7 of its label in registers, the
// eight group sums are scanned through LDS, and each thread writes its tiles'
// prefixes (a two-level scan, eight dependent steps instead of 64).
constexpr int HC_L = 32, HC_G = 256 / HC_L, HC_R = 8, HC_T = HC_G * HC_R;
__global__ __launch_bounds__(256) void k_hist_cols(int* __restrict__ hist, int C, int ntiles,
                                                   int32_t* __restrict__ counts)
{
    __shared__ int s_g[HC_G][HC_L];
    const int h = blockIdx.y, l0 = blockIdx.x * HC_L;
    const int lab = threadIdx.x & (HC_L - 1), g = threadIdx.x / HC_L;
    const bool lv = l0 + lab < C;
    int* hb = hist + (size_t)h * ntiles * C + (lv ? l0 + lab : 0);
    int run = 0;
    for (int t0 = 0; t0 < ntiles; t0 += HC_T) {
        int v[HC_R];
        int local = 0;
#pragma unroll
        for (int k = 0; k < HC_R; ++k) {
            const int t = t0 + g * HC_R + k;
            v[k] = (lv && t < ntiles) ? hb[(size_t)t * C] : 0;
            local += v[k];
        }
        s_g[g][lab] = local;
        __syncthreads();
        int pre = run, tot = 0;
#pragma unroll
        for (int q = 0; q < HC_G; ++q) {
            const int x = s_g[q][lab];
            pre += q < g ? x : 0;
            tot += x;
        }
#pragma unroll
        for (int k = 0; k < HC_R; ++k) {
            const int t = t0 + g * HC_R + k;
            if (lv && t < ntiles) hb[(size_t)t * C] = pre;
            pre += v[k];
        }
        run += tot;
        __syncthreads();   // s_g is rewritten by the next pass
    }
    if (g == 0 && lv) counts[(size_t)h * C + l0 + lab] = run;
}

// Per head: cluster offsets = exclusive prefix of the counts.  Also clears the
// per-head words the next k-means iteration accumulates into (stats, nflag).
__global__ __launch_bounds__(1024) void k_count_scan(const int32_t* __restrict__ counts, int C,
                                                     int32_t* __restrict__ offsets,
                                                     unsigned* __restrict__ stats,
                                                     int* __restrict__ nflag)
{
    __shared__ int s_part[1024];
    const int h = blockIdx.x;
    const int per = (C + 1023) / 1024;
    const int c0 = threadIdx.x * per;
    int local = 0;
    for (int k = 0; k < per; ++k)
        if (c0 + k < C) local += counts[(size_t)h * C + c0 + k];
    s_part[threadIdx.x] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int v = (int)threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
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
    if (stats && threadIdx.x < 4) stats[4 * h + threadIdx.x] = 0u;
    if (nflag && threadIdx.x == 0) nflag[h] = 0;
}

// Unstable bucket fill: every token goes to its cluster's range (order within a
// cluster does not matter to the exact sums).  Ranks inside a tile come from
// LDS atomics.
__global__ __launch_bounds__(256) void k_bucket(const int32_t* __restrict__ labels, int N, int C,
                                                int ntiles, const int* __restrict__ hist,
                                                const int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ perm)
{
    extern __shared__ int s_r[];
    const int tile = blockIdx.x, h = blockIdx.y;
    for (int c = threadIdx.x; c < C; c += 256) s_r[c] = 0;
    __syncthreads();
    const int i = tile * kTile + threadIdx.x;
    if (i < N) {
        const int l = labels[(size_t)h * N + i];
        if (l >= 0 && l < C) {
            const int rank = atomicAdd(&s_r[l], 1);
            const int pos =
                offsets[(size_t)h * (C + 1) + l] + hist[((size_t)h * ntiles + tile) * C + l] + rank;
            perm[(size_t)h * N + pos] = i;
        }
    }
}

// Cluster means from exact fixed-point sums.  The bucketed token order is cut
// into chunks of MC_ROWS positions, one block each; a block sums the rows of
// every cluster segment in its chunk as 64-bit integers (scale 2^shift) and adds
// them to the cluster's running sums with integer atomics (exact, so the order
// does not matter).  k_cluster_finalize then turns the sums into means.  The
// fixed-point image of each element is its value times 2^shift rounded to the
// nearest integer (fixed_bits), exact for every input that is a multiple of
// 2^-shift.
constexpr int MC_ROWS = 512;

template <typename T, int D>
__global__ __launch_bounds__(256) void k_cluster_chunks(const T* __restrict__ X,
                                                        const int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ offsets, int N,
                                                        int C, int shift,
                                                        unsigned long long* __restrict__ sums,
                                                        const int* __restrict__ changed)
{
    constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;               // chunks per row
    constexpr int RPP = 256 / CPR;             // rows per pass
    __shared__ long long s_sum[RPP][D];
    __shared__ int s_idx[MC_ROWS];
    const int h = blockIdx.y;
    const int p0 = blockIdx.x * MC_ROWS;
    if (p0 >= N) return;
    const int p1 = min(N, p0 + MC_ROWS);
    const int32_t* oh = offsets + (size_t)h * (C + 1);
    const int ch = threadIdx.x % CPR, rg = threadIdx.x / CPR;
    const T* Xh = X + (size_t)h * N * D + ch * EPC;
    const double scale = ldexp(1.0, shift);
    for (int k = threadIdx.x; k < p1 - p0; k += 256) s_idx[k] = perm[(size_t)h * N + p0 + k];
    // first cluster whose range ends after p0
    int lo_c = 0, hi_c = C - 1;
    while (lo_c < hi_c) {
        const int mid = (lo_c + hi_c) >> 1;
        if (oh[mid + 1] > p0) hi_c = mid; else lo_c = mid + 1;
    }
    __syncthreads();
    const int* chh = changed ? changed + (size_t)h * C : nullptr;
    for (int m = lo_c; m < C && oh[m] < p1; ++m) {
        const int a0 = max(oh[m], p0) - p0, a1 = min(oh[m + 1], p1) - p0;
        if (a1 <= a0) continue;
        if (chh && !chh[m]) continue;   // membership unchanged: its mean is unchanged
        unsigned long long acc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] = 0;
        int j = a0 + rg;
        for (; j + 3 * RPP < a1; j += 4 * RPP) {
            uint4 w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = *(const uint4*)(Xh + (size_t)s_idx[j + u * RPP] * D);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const T* v = (const T*)&w[u];
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[e] += fixed_bits<T>(v[e], scale);
            }
        }
        for (; j < a1; j += RPP) {
            const uint4 w0 = *(const uint4*)(Xh + (size_t)s_idx[j] * D);
            const T* v0 = (const T*)&w0;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[e] += fixed_bits<T>(v0[e], scale);
        }
        // remove the offset carried by every accumulated row
        const unsigned long long rows = (unsigned long long)((a1 - a0 - rg + RPP - 1) / RPP);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] -= rows * kFixMagicBits;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s_sum[rg][ch * EPC + e] = (long long)acc[e];
        __syncthreads();
        if ((int)threadIdx.x < D) {
            long long tot = 0;
#pragma unroll
            for (int g = 0; g < RPP; ++g) tot += s_sum[g][threadIdx.x];
            atomicAdd(sums + ((size_t)h * C + m) * D + threadIdx.x, (unsigned long long)tot);
        }
        __syncthreads();
    }
}

// centroid = (double)sum * 2^-shift / count for every non-empty cluster (one
// wave per cluster); an empty cluster keeps its centroid (k-means) or becomes
// zero (plain means).  Optionally writes an fp32 copy; with PLANES also the
// bf16 hi/lo planes, ||c||^2 (fp32, fp64) and the split residual norm that the
// MFMA screen of the next assignment needs.  Clears the sums for the next pass.
// With `changed`, only clusters whose membership changed are recomputed (the
// others' sums are zero and their centroids stand); `moved` records whether
// a recomputed centroid differs from its previous value in any bit.
template <int D, bool PLANES>
__global__ __launch_bounds__(256) void k_cluster_finalize(
    const int32_t* __restrict__ counts, int C, int shift, int zero_empty,
    unsigned long long* __restrict__ sums, double* __restrict__ cent64, float* __restrict__ cent_out,
    bf16* __restrict__ hi, bf16* __restrict__ lo, float* __restrict__ cn32,
    double* __restrict__ cn64, float* __restrict__ resid, const int* __restrict__ changed,
    int* __restrict__ moved)
{
    constexpr int EPL = D / 64;
    const int h = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const double inv_scale = ldexp(1.0, -shift);
    for (int m = blockIdx.x * 4 + wave; m < C; m += gridDim.x * 4) {
        const size_t row = (size_t)h * C + m;
        if (changed && !changed[row]) continue;   // wave-uniform
        const int n = counts[row];
        double a2 = 0.0, r2s = 0.0;
        bool mv = false;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const size_t i = row * D + lane * EPL + e;
            double c;
            if (n > 0) {
                c = ((double)(long long)sums[i] * inv_scale) / (double)n;
                mv |= c != cent64[i];
                cent64[i] = c;
                sums[i] = 0ull;
            } else if (zero_empty) {
                c = 0.0;
                cent64[i] = c;
            } else {
                c = cent64[i];
            }
            if (cent_out) cent_out[i] = (float)c;
            if constexpr (PLANES) {
                const bf16 chh = f32_to_bf16((float)c);
                const double r1 = c - (double)bf16_to_f32(chh);
                const bf16 cl = f32_to_bf16((float)r1);
                const double r2 = r1 - (double)bf16_to_f32(cl);
                hi[i] = chh;
                lo[i] = cl;
                a2 = fma(c, c, a2);
                r2s = fma(r2, r2, r2s);
            }
        }
        if (moved) {
            const bool any = __any(mv);
            if (lane == 0) moved[row] = any ? 1 : 0;
        }
        if constexpr (PLANES) {
            for (int o = 32; o >= 1; o >>= 1) {
                a2 += __shfl_xor(a2, o);
                r2s += __shfl_xor(r2s, o);
            }
            if (lane == 0) {
                cn64[row] = a2;
                cn32[row] = (float)a2;
                resid[row] = (float)(sqrt(r2s) * (1.0 + 1e-6));
            }
        }
    }
}

// Label changes of one assignment: both clusters of every token whose label
// changed are marked (their members, hence their means, changed); the labels are
// then kept for the next comparison.  With mark == 0 only the copy is made.
__global__ __launch_bounds__(256) void k_label_diff(const int32_t* __restrict__ labels,
                                                    int32_t* __restrict__ prev, int N, int C,
                                                    int mark, int* __restrict__ changed)
{
    const int h = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= N) return;
    const size_t t = (size_t)h * N + i;
    const int now = labels[t];
    if (mark) {
        const int was = prev[t];
        if (now != was) {
            if (was >= 0 && was < C) changed[(size_t)h * C + was] = 1;
            if (now >= 0 && now < C) changed[(size_t)h * C + now] = 1;
        }
    }
    prev[t] = now;
}

// Per head: the ascending list of moved centroids (the only ones the next
// assignment has to evaluate) and each centroid's position in it (-1 if it did
// not move); both flag arrays are then cleared for the next round.
__global__ __launch_bounds__(1024) void k_moved_list(int C, int* __restrict__ changed,
                                                     int* __restrict__ moved, int* __restrict__ mlist,
                                                     int* __restrict__ mpos, int* __restrict__ mcount)
{
    __shared__ int s_part[1024];
    const int h = blockIdx.x;
    int* mv = moved + (size_t)h * C;
    int* ch = changed + (size_t)h * C;
    int base = 0;
    for (int m0 = 0; m0 < C; m0 += 1024) {
        const int m = m0 + threadIdx.x;
        const int f = (m < C) ? mv[m] : 0;
        s_part[threadIdx.x] = f;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int v = (int)threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
            __syncthreads();
            s_part[threadIdx.x] += v;
            __syncthreads();
        }
        if (f) mlist[(size_t)h * C + base + s_part[threadIdx.x] - 1] = m;
        if (m < C) {
            mpos[(size_t)h * C + m] = f ? base + s_part[threadIdx.x] - 1 : -1;
            mv[m] = 0;
            ch[m] = 0;
        }
        base += s_part[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) mcount[h] = base;
}

// Per-head maxima, over all clusters, of the split residual and of ||c|| (the
// bounds of the next MFMA screen).
__global__ __launch_bounds__(256) void k_plane_stats(int C, const double* __restrict__ cn64,
                                                     const float* __restrict__ resid,
                                                     unsigned* __restrict__ stats)
{
    __shared__ float s_r[256], s_c[256];
    const int h = blockIdx.x;
    float rmax = 0.f, cmax = 0.f;
    for (int m = threadIdx.x; m < C; m += 256) {
        const size_t row = (size_t)h * C + m;
        rmax = fmaxf(rmax, resid[row]);
        cmax = fmaxf(cmax, (float)(sqrt(cn64[row]) * (1.0 + 1e-6)));
    }
    s_r[threadIdx.x] = rmax;
    s_c[threadIdx.x] = cmax;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o) {
            s_r[threadIdx.x] = fmaxf(s_r[threadIdx.x], s_r[threadIdx.x + o]);
            s_c[threadIdx.x] = fmaxf(s_c[threadIdx.x], s_c[threadIdx.x + o]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        stats[4 * h + 0] = __float_as_uint(s_r[0]);
        stats[4 * h + 1] = __float_as_uint(s_c[0]);
    }
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


template <typename T, int D>
static hipError_t run_cluster(const ClusterArgs& a, hipStream_t st)
{
    const Layout& L = *a.L;
    char* s = a.scratch;
    int* err = (int*)(s + L.cl_err);
    double* cent64 = (double*)(s + L.cl_cent64);
    int* hist = (int*)(s + L.cl_hist);
    int32_t* pwork = (int32_t*)(s + L.cl_perm);
    const int H = a.H, N = a.N, C = a.C;
    const T* X = (const T*)a.X;
    const int ntiles = (N + kTile - 1) / kTile;
    const dim3 gtiles(ntiles, H), gcent(C, H), gcols((C + HC_L - 1) / HC_L, H);
    const bool mfma = assign_mfma_supported(a);
    const KmPlanes P = km_planes(a);
    unsigned long long* sums = (unsigned long long*)(s + L.cl_sums);
    float* resid = (float*)(s + L.cl_resid);
    const dim3 gchunks((N + MC_ROWS - 1) / MC_ROWS, H), gfin((C + 3) / 4 < 64 ? (C + 3) / 4 : 64, H);
    zero_words(sums, (size_t)H * C * D * 8, st);
    // plain mean pass (no planes)
    auto mean_pass = [&](const T* src, const int32_t* order, int zero_empty, float* out) {
        hipLaunchKernelGGL((k_cluster_chunks<T, D>), gchunks, dim3(256), 0, st, src, order, a.offsets,
                           N, C, a.shift, sums, (const int*)nullptr);
        hipLaunchKernelGGL((k_cluster_finalize<D, false>), gfin, dim3(256), 0, st, a.counts, C,
                           a.shift, zero_empty, sums, cent64, out, (bf16*)nullptr, (bf16*)nullptr,
                           (float*)nullptr, (double*)nullptr, (float*)nullptr, (const int*)nullptr,
                           (int*)nullptr);
    };

    // counting-sort front half: tile histograms, per-label tile prefixes, counts, offsets
    auto sort_front = [&](unsigned* stats, int* nflag) {
        hipLaunchKernelGGL(k_tile_hist, gtiles, dim3(256), (size_t)C * 4, st, a.labels, N, C,
                           ntiles, hist, err);
        hipLaunchKernelGGL(k_hist_cols, gcols, dim3(256), 0, st, hist, C, ntiles, a.counts);
        hipLaunchKernelGGL(k_count_scan, dim3(H), dim3(1024), 0, st, a.counts, C, a.offsets, stats,
                           nflag);
    };

    if (!(a.flags & SVGEAR_LABELS_GIVEN)) {
        hipLaunchKernelGGL((k_init_centroids<T>), gcent, dim3(D), 0, st, X, a.init, N, D, C, cent64,
                           err);
        if (mfma) {
            zero_words(P.stats, (size_t)H * 16, st);
            zero_words(P.nflag, (size_t)H * 4, st);
            hipError_t e = launch_km_prep(a, cent64, P, st);
            if (e != hipSuccess) return e;
        }
        // With the MFMA screen, iteration 0 evaluates every centroid; later
        // iterations only the centroids that moved in the last update, against
        // per-token bounds on the distances to all others (see assign_mfma.hip).
        // Updates recompute only the clusters whose membership changed.
        int* changed = (int*)(s + L.cl_changed);
        int* moved = (int*)(s + L.cl_moved);
        int32_t* labprev = (int32_t*)(s + L.cl_labprev);
        if (mfma) {
            zero_words(changed, (size_t)H * C * 4, st);
            zero_words(moved, (size_t)H * C * 4, st);
        }
        for (int it = 0; it < a.iters; ++it) {
            if (mfma) {
                hipError_t e = launch_assign_mfma(a, cent64, P, it > 0, st);
                if (e != hipSuccess) return e;
            } else {
                hipLaunchKernelGGL((k_assign_exact<T, D>), dim3((N + 255) / 256, H), dim3(256), 0,
                                   st, X, cent64, N, C, a.labels);
            }
            if (it == a.iters - 1) break;
            // update: unstable bucket order + exact per-cluster means (and next planes)
            if (mfma)
                hipLaunchKernelGGL(k_label_diff, dim3((N + 255) / 256, H), dim3(256), 0, st, a.labels,
                                   labprev, N, C, it > 0 ? 1 : 0, changed);
            sort_front(nullptr, mfma ? P.nflag : nullptr);
            hipLaunchKernelGGL(k_bucket, gtiles, dim3(256), (size_t)C * 4, st, a.labels, N, C,
                               ntiles, hist, a.offsets, pwork);
            if (mfma && D == 128) {
                const int* chg = it > 0 ? changed : nullptr;
                hipLaunchKernelGGL((k_cluster_chunks<T, D>), gchunks, dim3(256), 0, st, X, pwork,
                                   a.offsets, N, C, a.shift, sums, chg);
                hipLaunchKernelGGL((k_cluster_finalize<D, D == 128>), gfin, dim3(256), 0, st, a.counts,
                                   C, a.shift, 0, sums, cent64, (float*)nullptr, P.hi, P.lo, P.cn32,
                                   P.cn64, resid, chg, moved);
                hipLaunchKernelGGL(k_plane_stats, dim3(H), dim3(256), 0, st, C, P.cn64, resid,
                                   P.stats);
                hipLaunchKernelGGL(k_moved_list, dim3(H), dim3(1024), 0, st, C, changed, moved,
                                   P.mlist, P.mpos, P.mcount);
            } else {
                mean_pass(X, pwork, 0, (float*)nullptr);
            }
        }
    }

    // Final reorder (stable counting sort), rows gathered, means of the final labels.
    sort_front(nullptr, nullptr);
    const int row_chunks = (int)(D * sizeof(T) / 16);
    hipLaunchKernelGGL(k_scatter, gtiles, dim3(256), 0, st, a.labels, N, C, ntiles, hist, a.offsets,
                       a.perm, a.inv_perm, (const uint4*)a.X, (uint4*)a.Xp, (const uint4*)a.V,
                       (uint4*)a.Vp, row_chunks);
    mean_pass(X, a.perm, (a.flags & SVGEAR_LABELS_GIVEN) ? 1 : 0, a.cent);
    // V-bar: mean of V over the key clusters (zero for an empty cluster).  cent64
    // is no longer needed and serves as scratch.
    if (a.side == 1) mean_pass((const T*)a.V, a.perm, 1, a.vbar);
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
