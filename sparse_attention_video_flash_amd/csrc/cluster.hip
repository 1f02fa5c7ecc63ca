// cluster.hip -- step 1 of the SVG-EAR pipeline (review page, inference-pipeline
// paragraph, step 1; German summary 2A): Flash k-means of Q and K, stable
// counting-sort reordering so that same-cluster tokens are contiguous, and the
// centroid means (V-bar over K's clusters).
//
// Exactness strategy.  The assignment picks the nearest centroid in squared
// Euclidean distance with ties to the lowest index.  Centroids are kept in fp64
// and are the exact member means: member rows are summed as pairs of 64-bit
// fixed-point integers at a power-of-two scale chosen per head from the
// largest input magnitude (internal.h, fix_add), so the sum does not depend on
// the order of the rows; one rounding to fp64 and one fp64 division follow.
// The kernels that first read a tensor (the first assignment, the scatter)
// record its per-head range; a head whose values cannot all be captured
// exactly (or that holds a non-finite value) raises ERR_RANGE.  Each update buckets the
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
                                                      int C, int32_t* __restrict__ labels,
                                                      unsigned* __restrict__ range)
{
#pragma clang fp contract(off)
    constexpr int CH = 32768 / (D * 8);  // centroids per 32 KB chunk
    __shared__ double s_c[CH * D];
    const int h = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    float xr[D];  // exact copies of the inputs
    unsigned rmx = 0u;
    if (i < N) {
        const T* x = X + ((size_t)h * N + i) * D;
#pragma unroll
        for (int t = 0; t < D; ++t) {
            xr[t] = to_f32<T>(x[t]);
            rmx = max(rmx, __float_as_uint(xr[t]) & 0x7FFFFFFFu);
        }
    }
    if (range) range_commit(rmx, 0u, range + kRangeStride * h, false);   // largest magnitude (sets the scale)
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

// The label comparison of one k-means assignment, fused into the histogram
// pass that reads the labels anyway: both clusters of every token whose label
// changed are marked (their members, hence their means, changed); the labels
// are kept for the next comparison (with mark == 0 only the copy is made);
// tokflag records per token whether its label changed (all set with mark ==
// 0), and fpos_prev the same flag at the token's position in the previous
// bucket order (ipos_prev; the delta updates).  prev == nullptr: no comparison.
struct LabelDiff {
    int32_t* prev;
    int mark;
    int* changed;
    uint8_t* tokflag;
    const int32_t* ipos_prev;
    uint8_t* fpos_prev;
};

// Per-tile label histogram (tiles of tt consecutive tokens, tt a multiple of
// 256), with the optional label comparison.
__global__ __launch_bounds__(256) void k_tile_hist(const int32_t* __restrict__ labels, int N, int C,
                                                   int ntiles, int tt, int* __restrict__ hist,
                                                   int* __restrict__ err, LabelDiff ld)
{
    extern __shared__ int s_h[];
    const int tile = blockIdx.x, h = blockIdx.y;
    for (int c = threadIdx.x; c < C; c += 256) s_h[c] = 0;
    __syncthreads();
    const int i1 = min(N, (tile + 1) * tt);
    for (int i = tile * tt + (int)threadIdx.x; i < i1; i += 256) {
        const size_t t = (size_t)h * N + i;
        const int l = labels[t];
        if (l < 0 || l >= C) {
            atomicOr(err, ERR_LABEL);
        } else {
            atomicAdd(&s_h[l], 1);
        }
        if (ld.prev) {
            bool moved = true;
            if (ld.mark) {
                const int was = ld.prev[t];
                moved = l != was;
                if (moved) {
                    if (was >= 0 && was < C) ld.changed[(size_t)h * C + was] = 1;
                    if (l >= 0 && l < C) ld.changed[(size_t)h * C + l] = 1;
                }
                if (ld.fpos_prev) {   // every token with a valid label had a position
                    const int ip = ld.ipos_prev[t];
                    if (ip >= 0 && ip < N) ld.fpos_prev[(size_t)h * N + ip] = moved ? 1 : 0;
                }
            }
            ld.prev[t] = l;
            if (ld.tokflag) ld.tokflag[t] = moved ? 1 : 0;
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
// cluster does not matter to the exact sums).  Ranks inside a tile (tt tokens)
// come from LDS atomics.  With tokflag (the delta updates of the k-means): also
// each token's position (ipos) and its flag by position (fpos).
__global__ __launch_bounds__(256) void k_bucket(const int32_t* __restrict__ labels, int N, int C,
                                                int ntiles, int tt, const int* __restrict__ hist,
                                                const int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ perm,
                                                const uint8_t* __restrict__ tokflag,
                                                int32_t* __restrict__ ipos, uint8_t* __restrict__ fpos)
{
    extern __shared__ int s_r[];
    const int tile = blockIdx.x, h = blockIdx.y;
    for (int c = threadIdx.x; c < C; c += 256) s_r[c] = 0;
    __syncthreads();
    const int i1 = min(N, (tile + 1) * tt);
    for (int i = tile * tt + (int)threadIdx.x; i < i1; i += 256) {
        const int l = labels[(size_t)h * N + i];
        if (l >= 0 && l < C) {
            const int rank = atomicAdd(&s_r[l], 1);
            const int pos =
                offsets[(size_t)h * (C + 1) + l] + hist[((size_t)h * ntiles + tile) * C + l] + rank;
            perm[(size_t)h * N + pos] = i;
            if (tokflag) {
                ipos[(size_t)h * N + i] = pos;
                fpos[(size_t)h * N + pos] = tokflag[(size_t)h * N + i];
            }
        }
    }
}

// Cluster means from exact fixed-point sums.  The bucketed token order is cut
// into chunks of MC_ROWS positions, one block each; a block sums the rows of
// every cluster segment in its chunk as 64-bit integers (fix_hi, or both words
// of fix_add, at the head's scale) and adds them to the cluster's running sums
// with integer atomics (exact, so the order does not matter).
// k_cluster_finalize then turns the sums into means.
//
// MODE selects the instantiation: the one-word kernel serves the heads whose
// values are all captured by the first word (fix_need_lo false; the usual
// case), the two-word kernel the others, each returning at once for a head the
// other serves; both are launched.  With collect (a pass that reads every row
// while the smallest magnitude is not yet known: the first update of the
// k-means, or the only pass of a tensor) the one-word kernel runs for every
// head and records the smallest non-zero magnitude; a head that then turns out
// to need the second word has its sums cleared (k_clear_two_word_heads) and
// redone by the two-word kernel.
//
// DELTA: an update after the first, which adds to the running sums (kept from
// the previous update) only the rows of the tokens whose label changed:
// blockIdx.z = 0 walks the current bucket order (perm1, offsets1, flags1: each
// such token joins its new cluster), blockIdx.z = 1 the previous iteration's
// bucket order (perm2, offsets2, flags2: it leaves its old one, its image
// negated, which is exact).  The flags are stored by bucket position.  The
// sums are integers, so the result equals a full re-summation bit for bit.  A
// chunk packs its flagged rows' token indices to the front of s_idx and cuts
// the cluster segments at the prefix sums of the flags.
constexpr int MC_ROWS = 512;

enum : int { CH_ONE = 0, CH_ONE_COLLECT = 1, CH_TWO = 2 };
template <typename T, int D, int MODE, bool GATHER, bool DELTA>
__global__ __launch_bounds__(256) void k_cluster_chunks(const T* __restrict__ X,
                                                        const int32_t* __restrict__ perm1,
                                                        const int32_t* __restrict__ offsets1, int N,
                                                        int C, unsigned* __restrict__ range,
                                                        unsigned long long* __restrict__ sums,
                                                        const int* __restrict__ changed, int rev,
                                                        uint4* __restrict__ Xp,
                                                        const uint8_t* __restrict__ flags1,
                                                        const int32_t* __restrict__ perm2,
                                                        const int32_t* __restrict__ offsets2,
                                                        const uint8_t* __restrict__ flags2, int drows)
{
    static_assert(!DELTA || (MODE != CH_ONE_COLLECT && !GATHER), "delta passes neither collect nor gather");
    constexpr bool TWO = MODE == CH_TWO, COLLECT = MODE == CH_ONE_COLLECT;
    constexpr unsigned kSign = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;   // negates every element of a word
    constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;               // chunks per row
    constexpr int RPP = 256 / CPR;             // rows per pass
    constexpr int PREC = sizeof(T) == 2 ? 8 : 24;
    __shared__ long long s_sum[RPP][D];
    // delta passes touch few rows per position: longer chunks (drows positions,
    // at most ROWS, a multiple of 256), fewer workgroups
    constexpr int ROWS = DELTA ? 4 * MC_ROWS : MC_ROWS;
    constexpr int PPT = ROWS / 256;   // most positions per thread in the flag scan
    const int rows_c = DELTA ? drows : MC_ROWS;
    const int ppt = rows_c / 256;
    __shared__ int s_idx[ROWS];
    __shared__ int s_pre[DELTA ? ROWS + 1 : 1];   // exclusive prefix sums of the chunk's flags
    __shared__ int s_first, s_wsum[4];
    const bool neg = DELTA && blockIdx.z == 1;
    const int32_t* const perm = neg ? perm2 : perm1;
    const int32_t* const offsets = neg ? offsets2 : offsets1;
    const int h = rev ? (int)gridDim.y - 1 - (int)blockIdx.y : (int)blockIdx.y;
    const int base = fix_base(N);
    unsigned* rg4 = range + kRangeStride * h;
    if (TWO ? !fix_need_lo(rg4, base, PREC) : (!COLLECT && fix_need_lo(rg4, base, PREC)))
        return;   // a head the other instantiation serves
    const int32_t* oh = offsets + (size_t)h * (C + 1);
    const int ch = threadIdx.x % CPR, rg = threadIdx.x / CPR;
    const T* Xh = X + (size_t)h * N * D + ch * EPC;
    const double sc = ldexp(1.0, base - fix_exp(rg4[0])), tc = ldexp(1.0, base);
    unsigned long long* sums_lo = sums + (size_t)gridDim.y * C * D;
    const int* chh = changed ? changed + (size_t)h * C : nullptr;
    using R = typename RangeOf<T>::type;
    R rgx;
    // chunks of ROWS positions, gridDim.x apart (the two-word kernel, which
    // serves few heads if any, runs on a smaller grid)
    for (int p0 = blockIdx.x * rows_c; p0 < N; p0 += (int)gridDim.x * rows_c) {
        const int p1 = min(N, p0 + rows_c);
        // first cluster whose range ends after p0: the number of clusters that
        // end at or before it (the offsets do not decrease), counted in parallel
        __syncthreads();   // the previous chunk is done with s_idx, s_first and s_wsum
        if (threadIdx.x == 0) s_first = 0;
        __syncthreads();
        {
            int n_before = 0;
            for (int m = threadIdx.x; m < C; m += 256) n_before += oh[m + 1] <= p0;
            if (n_before) atomicAdd(&s_first, n_before);
        }
        __syncthreads();
        const int lo_c = s_first;
        if (chh) {   // no changed cluster in the chunk: nothing to sum
            bool any = false;
            for (int m = lo_c + (int)threadIdx.x; m < C && oh[m] < p1; m += 256)
                any |= chh[m] != 0 && oh[m + 1] > oh[m];
            if (__syncthreads_or(any) == 0) continue;
        }
        if (!DELTA) {
            for (int k = threadIdx.x; k < p1 - p0; k += 256) s_idx[k] = perm[(size_t)h * N + p0 + k];
            __syncthreads();
        } else {
            // PPT consecutive positions per thread: flags (stored in bucket
            // order), block-wide exclusive scan, then the flagged rows' token
            // indices packed to the front in order
            const uint8_t* const fl = (neg ? flags2 : flags1) + (size_t)h * N + p0;
            const int n = p1 - p0, k0 = ppt * (int)threadIdx.x;
            int fk[PPT];
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                fk[i] = i < ppt && k0 + i < n ? fl[k0 + i] : 0;
                cnt += fk[i];
            }
            // inclusive scan within each wave, then across the four waves
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o);
                if (lane >= o) incl += v;
            }
            if (lane == 63) s_wsum[wave] = incl;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < 3; ++w) incl += w < wave ? s_wsum[w] : 0;
            int ex = incl - cnt;
            if (k0 < n && k0 + ppt >= n) s_pre[n] = incl;   // the thread holding the last position
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                if (i < ppt && k0 + i < n) s_pre[k0 + i] = ex;
                if (fk[i]) s_idx[ex] = perm[(size_t)h * N + p0 + k0 + i];
                ex += fk[i];
            }
            __syncthreads();
            if (s_pre[n] == 0) continue;   // no flagged row in the chunk (uniform)
        }
        for (int m = lo_c; m < C && oh[m] < p1; ++m) {
            int a0 = max(oh[m], p0) - p0, a1 = min(oh[m + 1], p1) - p0;
            if (DELTA && a1 > a0) {   // the segment's flagged rows, packed
                a0 = s_pre[a0];
                a1 = s_pre[a1];
            }
            if (a1 <= a0) continue;
            if (chh && !chh[m]) continue;   // membership unchanged: its mean is unchanged
            unsigned long long ah[EPC], al[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) ah[e] = al[e] = 0;
            auto add_row = [&](uint4 w) {
                if (neg) { w.x ^= kSign; w.y ^= kSign; w.z ^= kSign; w.w ^= kSign; }
                const T* v = (const T*)&w;
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    if (TWO) fix_add<T>(v[e], sc, tc, ah[e], al[e]);
                    else ah[e] += fix_hi<T>(v[e], sc);
                }
                if (COLLECT) { rgx.add_min(w.x); rgx.add_min(w.y); rgx.add_min(w.z); rgx.add_min(w.w); }
            };
            // GATHER (the final pass): the rows are also written out in bucket order
            auto put = [&](int jj, const uint4 w) {
                if (GATHER) Xp[((size_t)h * N + p0 + jj) * CPR + ch] = w;
            };
            int j = a0 + rg;
            for (; j + 3 * RPP < a1; j += 4 * RPP) {
                uint4 w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) w[u] = *(const uint4*)(Xh + (size_t)s_idx[j + u * RPP] * D);
#pragma unroll
                for (int u = 0; u < 4; ++u) { put(j + u * RPP, w[u]); add_row(w[u]); }
            }
            for (; j < a1; j += RPP) {
                const uint4 w = *(const uint4*)(Xh + (size_t)s_idx[j] * D);
                put(j, w);
                add_row(w);
            }
            // remove the offset carried by every accumulated image; reduce the
            // first word's row groups, then (if summed) the second word's
            const unsigned long long rows = (unsigned long long)((a1 - a0 - rg + RPP - 1) / RPP);
#pragma unroll
            for (int e = 0; e < EPC; ++e) s_sum[rg][ch * EPC + e] = (long long)(ah[e] - rows * kFixMagicBits);
            __syncthreads();
            if ((int)threadIdx.x < D) {
                long long tot = 0;
#pragma unroll
                for (int g = 0; g < RPP; ++g) tot += s_sum[g][threadIdx.x];
                atomicAdd(sums + ((size_t)h * C + m) * D + threadIdx.x, (unsigned long long)tot);
            }
            __syncthreads();
            if (TWO) {
#pragma unroll
                for (int e = 0; e < EPC; ++e) s_sum[rg][ch * EPC + e] = (long long)(al[e] - rows * kFixMagicBits);
                __syncthreads();
                if ((int)threadIdx.x < D) {
                    long long tot = 0;
#pragma unroll
                    for (int g = 0; g < RPP; ++g) tot += s_sum[g][threadIdx.x];
                    atomicAdd(sums_lo + ((size_t)h * C + m) * D + threadIdx.x, (unsigned long long)tot);
                }
                __syncthreads();
            }
        }
    }
    if (COLLECT) range_commit(0u, rgx.min_word(), rg4, true);
}

// After a collecting one-word pass: clears the sums of every head that needs
// the second word (they are then summed again by the two-word kernel).
__global__ __launch_bounds__(256) void k_clear_two_word_heads(const unsigned* __restrict__ range, int N,
                                                              int prec, size_t per_head,
                                                              unsigned long long* __restrict__ sums)
{
    const int h = blockIdx.y;
    if (!fix_need_lo(range + kRangeStride * h, fix_base(N), prec)) return;
    unsigned long long* p = sums + (size_t)h * per_head;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < per_head; i += (size_t)gridDim.x * 256) p[i] = 0ull;
}

// Value of the two fixed-point sums of one element: (hi + lo 2^-B) 2^-S,
// rounded once in all but pathological cases (hi's fp64 rounding error is
// carried into the small part).
__device__ __forceinline__ double fix_value(unsigned long long hi, unsigned long long lo, double inv_s,
                                            double inv_t)
{
    const long long hs = (long long)hi;
    const double hd = (double)hs;
    const long long hr = hs - (long long)hd;   // exact: |hr| <= 2^9
    return (hd + fma((double)(long long)lo, inv_t, (double)hr)) * inv_s;
}

// centroid = (value of the fixed-point sums) / count for every non-empty
// cluster (one wave per cluster); with err, also checks the head's range
// (ERR_RANGE: values the exact sums cannot capture, or out of range); an empty cluster keeps its centroid (k-means) or becomes
// zero (plain means).  Optionally writes an fp32 copy; with PLANES also the
// bf16 hi/lo planes, ||c||^2 (fp32, fp64) and the split residual norm that the
// MFMA screen of the next assignment needs.  Clears the sums for the next pass,
// unless keep (the k-means delta updates add to them).  With `changed`, only
// clusters whose membership changed are recomputed (the others' centroids
// stand); `moved` records whether a recomputed centroid differs from its
// previous value in any bit.
template <int D, bool PLANES>
__global__ __launch_bounds__(256) void k_cluster_finalize(
    const int32_t* __restrict__ counts, int C, int N, const unsigned* __restrict__ range, int prec,
    int collect, int* __restrict__ err, int zero_empty, unsigned long long* __restrict__ sums,
    double* __restrict__ cent64,
    float* __restrict__ cent_out,
    bf16* __restrict__ hi, bf16* __restrict__ lo, float* __restrict__ cn32,
    double* __restrict__ cn64, float* __restrict__ resid, const int* __restrict__ changed,
    int* __restrict__ moved, int keep)
{
    constexpr int EPL = D / 64;
    const int h = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int base = fix_base(N);
    const double inv_s = ldexp(1.0, fix_exp(range[kRangeStride * h]) - base), inv_t = ldexp(1.0, -base);
    unsigned long long* sums_lo = sums + (size_t)gridDim.y * C * D;
    const bool need_lo = fix_need_lo(range + kRangeStride * h, base, prec);
    // the head's range is complete here: report values the sums cannot capture
    if (err && blockIdx.x == 0 && threadIdx.x == 0 && !fix_exact(range + kRangeStride * h, base, prec))
        atomicOr(err, ERR_RANGE);
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
                c = fix_value(sums[i], need_lo ? sums_lo[i] : 0ull, inv_s, inv_t) / (double)n;
                mv |= c != cent64[i];
                cent64[i] = c;
                if (!keep) {   // the next pass sums from zero (keep: the next update adds to them)
                    sums[i] = 0ull;
                    if (need_lo) sums_lo[i] = 0ull;
                }
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
// of X (and V) to their reordered positions and records the largest magnitude
// of V and, when range_x is given, of X.
template <typename T>
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ labels, int N, int C,
                                                 int ntiles, const int* __restrict__ hist,
                                                 const int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm,
                                                 int32_t* __restrict__ inv_perm,
                                                 const uint4* __restrict__ X, uint4* __restrict__ Xp,
                                                 const uint4* __restrict__ V, uint4* __restrict__ Vp,
                                                 int row_chunks,
                                                 unsigned* __restrict__ range_x,
                                                 unsigned* __restrict__ range_v, int rev)
{
    __shared__ int s_lab[kTile];
    __shared__ int s_pos[kTile];
    const int tile = blockIdx.x;
    const int h = rev ? (int)gridDim.y - 1 - (int)blockIdx.y : (int)blockIdx.y;
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
    if (!X && !V) return;
    const int rows = min(kTile, N - tile * kTile);
    using R = typename RangeOf<T>::type;
    R rx, rv;
    for (int k = threadIdx.x; k < rows * row_chunks; k += 256) {
        const int r = k / row_chunks, ch = k - r * row_chunks;
        const int p = s_pos[r];
        if (p < 0) continue;
        const size_t src = ((size_t)h * N + tile * kTile + r) * row_chunks + ch;
        const size_t dst = ((size_t)h * N + p) * row_chunks + ch;
        if (X) {
            const uint4 xw = X[src];
            Xp[dst] = xw;
            if (range_x) { rx.add_max(xw.x); rx.add_max(xw.y); rx.add_max(xw.z); rx.add_max(xw.w); }
        }
        if (V) {
            const uint4 vw = V[src];
            Vp[dst] = vw;
            rv.add_max(vw.x); rv.add_max(vw.y); rv.add_max(vw.z); rv.add_max(vw.w);
        }
    }
    if (X && range_x) range_commit(rx.max_word(), 0u, range_x + kRangeStride * h, false);
    if (V) range_commit(rv.max_word(), 0u, range_v + kRangeStride * h, false);
}

// ----------------------------------------------------------------------------- driver


template <typename T, int D>
static hipError_t run_cluster(const ClusterArgs& a, hipStream_t st)
{
    const Layout& L = *a.L;
    char* s = a.scratch;
    int* err = a.err;
    double* cent64 = (double*)(s + L.cl_cent64);
    int* hist = (int*)(s + L.cl_hist);
    int32_t* pwork = (int32_t*)(s + L.cl_perm);
    const int H = a.H, N = a.N, C = a.C;
    const T* X = (const T*)a.X;
    const int ntiles = (N + kTile - 1) / kTile;
    const dim3 gtiles(ntiles, H), gcent(C, H), gcols((C + HC_L - 1) / HC_L, H);
    const bool mfma = assign_mfma_supported(a);
    const KmPlanes P = km_planes(a);
    unsigned long long* sums = (unsigned long long*)(s + L.cl_sums);   // [2][H, C, d]
    float* resid = (float*)(s + L.cl_resid);
    // per-head range words: [h][0..1] of X, [h][2..3] of V, one line per head (see fix_exact)
    unsigned* range = (unsigned*)(s + L.cl_range);
    unsigned* range_x = range;
    unsigned* range_v = range + 2;
    const int nchunks = (N + MC_ROWS - 1) / MC_ROWS;
    const dim3 gchunks(nchunks, H), gtwo(nchunks < 16 ? nchunks : 16, H), gfin((C + 3) / 4 < 64 ? (C + 3) / 4 : 64, H);
    zero_words(sums, (size_t)2 * H * C * D * 8, st);
    zero_words(range, (size_t)H * kRangeStride * 4, st);
    // plain mean pass (no planes)
    constexpr int kPrec = sizeof(T) == 2 ? 8 : 24;
    // Exact sums of the rows of src in `order` (bucketed by label): the
    // one-word instantiation, then (collect) the clearing of heads that need
    // two words, then the two-word instantiation for those heads.
    // rev: heads in reverse order.  Consecutive passes over X alternate the
    // direction (screens forward, updates and the scatter backward, the final
    // means forward), so each starts on the heads the previous one just read,
    // which the last-level cache still holds.
    auto chunk_pass = [&](const T* src, unsigned* rg, const int32_t* order, const int* chg, int collect,
                          int rev, uint4* xp, const int32_t* offs) {
        const uint8_t* nf = nullptr;
        // (a collecting pass runs only while the range is unknown, before any gather)
        if (collect) {
            hipLaunchKernelGGL((k_cluster_chunks<T, D, CH_ONE_COLLECT, false, false>), gchunks, dim3(256), 0, st,
                               src, order, offs, N, C, rg, sums, chg, rev, (uint4*)nullptr, nf, order, offs, nf, MC_ROWS);
            hipLaunchKernelGGL(k_clear_two_word_heads, dim3(16, H), dim3(256), 0, st, rg, N, kPrec,
                               (size_t)C * D, sums);
        } else if (xp) {
            hipLaunchKernelGGL((k_cluster_chunks<T, D, CH_ONE, true, false>), gchunks, dim3(256), 0, st, src, order,
                               offs, N, C, rg, sums, chg, rev, xp, nf, order, offs, nf, MC_ROWS);
        } else {
            hipLaunchKernelGGL((k_cluster_chunks<T, D, CH_ONE, false, false>), gchunks, dim3(256), 0, st, src, order,
                               offs, N, C, rg, sums, chg, rev, xp, nf, order, offs, nf, MC_ROWS);
        }
        if (xp)
            hipLaunchKernelGGL((k_cluster_chunks<T, D, CH_TWO, true, false>), gtwo, dim3(256), 0, st, src, order,
                               offs, N, C, rg, sums, chg, rev, xp, nf, order, offs, nf, MC_ROWS);
        else
            hipLaunchKernelGGL((k_cluster_chunks<T, D, CH_TWO, false, false>), gtwo, dim3(256), 0, st, src, order,
                               offs, N, C, rg, sums, chg, rev, xp, nf, order, offs, nf, MC_ROWS);
    };
    // an update after the first: the flagged tokens join their clusters (current
    // bucket order) and leave their previous ones (previous bucket order)
    auto delta_pass = [&](const int32_t* order, const int32_t* offs, const uint8_t* flags,
                          const int32_t* order_prev, const int32_t* offs_prev, const uint8_t* flags_prev,
                          const int* chg) {
        // the delta passes' chunk: the longest (up to 2,048 positions) that still
        // gives about four workgroups per CU
        int dr = 4 * MC_ROWS;
        while (dr > MC_ROWS && (size_t)((N + dr - 1) / dr) * H < 1024) dr /= 2;
        const int nd = (N + dr - 1) / dr;
        hipLaunchKernelGGL((k_cluster_chunks<T, D, CH_ONE, false, true>), dim3(nd, H, 2), dim3(256), 0, st, X,
                           order, offs, N, C, range_x, sums, chg, 1, (uint4*)nullptr, flags, order_prev, offs_prev, flags_prev, dr);
        hipLaunchKernelGGL((k_cluster_chunks<T, D, CH_TWO, false, true>), dim3(nd < 16 ? nd : 16, H, 2), dim3(256), 0, st, X,
                           order, offs, N, C, range_x, sums, chg, 1, (uint4*)nullptr, flags, order_prev, offs_prev, flags_prev, dr);
    };
    // plain mean pass (no planes); checks the range
    auto mean_pass = [&](const T* src, unsigned* rg, const int32_t* order, int collect, int zero_empty,
                         float* out, int rev, uint4* xp) {
        chunk_pass(src, rg, order, (const int*)nullptr, collect, rev, xp, a.offsets);
        hipLaunchKernelGGL((k_cluster_finalize<D, false>), gfin, dim3(256), 0, st, a.counts, C, N,
                           rg, kPrec, collect, err, zero_empty, sums, cent64, out, (bf16*)nullptr,
                           (bf16*)nullptr, (float*)nullptr, (double*)nullptr, (float*)nullptr,
                           (const int*)nullptr, (int*)nullptr, 0);
    };

    // counting-sort front half: tile histograms (tiles of tt tokens; with ld, the
    // label comparison of the k-means as well), per-label tile prefixes, counts,
    // offsets.  The stable final sort uses kTile-token tiles (the scatter ranks
    // within a tile by scanning it); the unstable sorts of the k-means updates
    // use tiles of kTileU tokens, which keeps the tile histograms small.
    auto sort_front = [&](unsigned* stats, int* nflag, int32_t* offs, int tt, const LabelDiff& ld) {
        const int nt = (N + tt - 1) / tt;
        hipLaunchKernelGGL(k_tile_hist, dim3(nt, H), dim3(256), (size_t)C * 4, st, a.labels, N, C,
                           nt, tt, hist, err, ld);
        hipLaunchKernelGGL(k_hist_cols, gcols, dim3(256), 0, st, hist, C, nt, a.counts);
        hipLaunchKernelGGL(k_count_scan, dim3(H), dim3(1024), 0, st, a.counts, C, offs, stats,
                           nflag);
    };
    const LabelDiff no_diff = {nullptr, 0, nullptr, nullptr, nullptr, nullptr};

    if (!(a.flags & SVGEAR_LABELS_GIVEN)) {
        hipLaunchKernelGGL((k_init_centroids<T>), gcent, dim3(D), 0, st, X, a.init, N, D, C, cent64,
                           err);
        if (mfma) {
            zero_words(P.stats, (size_t)H * 16, st);
            zero_words(P.nflag, (size_t)H * 4, st);
            hipError_t e = launch_km_prep(a, cent64, P, st);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(k_plane_stats, dim3(H), dim3(256), 0, st, C, P.cn64, resid, P.stats);
        }
        // With the MFMA screen, iteration 0 evaluates every centroid; later
        // iterations only the centroids that moved in the last update, against
        // per-token bounds on the distances to all others (see assign_mfma.hip).
        // The first update sums every token; later ones (MFMA path) add only the
        // tokens whose label changed to the kept sums, and the means of only the
        // clusters whose membership changed are recomputed.
        int* changed = (int*)(s + L.cl_changed);
        int* moved = (int*)(s + L.cl_moved);
        int32_t* labprev = (int32_t*)(s + L.cl_labprev);
        // With the MFMA path the running sums persist from update to update
        // (delta passes); the bucket orders and offsets alternate between two
        // buffers so that the previous ones are at hand.
        const bool delta = mfma && D == 128;
        uint8_t* tokflag = (uint8_t*)(s + L.cl_tokflag);
        int32_t* const order2[2] = {pwork, (int32_t*)(s + L.cl_perm2)};
        int32_t* const offs2[2] = {(int32_t*)(s + L.cl_offs), (int32_t*)(s + L.cl_offs) + (size_t)H * (C + 1)};
        int32_t* const ipos2[2] = {(int32_t*)(s + L.cl_ipos), (int32_t*)(s + L.cl_ipos) + (size_t)H * N};
        uint8_t* const fpos2[2] = {(uint8_t*)(s + L.cl_fpos), (uint8_t*)(s + L.cl_fpos) + (size_t)H * N};
        if (mfma) {
            zero_words(changed, (size_t)H * C * 4, st);
            zero_words(moved, (size_t)H * C * 4, st);
        }
        for (int it = 0; it < a.iters; ++it) {
            if (mfma) {
                hipError_t e = launch_assign_mfma(a, cent64, P, it > 0, it == 0 ? range_x : nullptr, st);
                if (e != hipSuccess) return e;
            } else {
                hipLaunchKernelGGL((k_assign_exact<T, D>), dim3((N + 255) / 256, H), dim3(256), 0,
                                   st, X, cent64, N, C, a.labels, it == 0 ? range_x : nullptr);
            }
            if (it == a.iters - 1) break;
            // update: unstable bucket order + exact per-cluster means (and next planes)
            LabelDiff ld = no_diff;
            if (mfma) {
                ld.prev = labprev;
                ld.mark = it > 0 ? 1 : 0;
                ld.changed = changed;
                ld.tokflag = delta ? tokflag : nullptr;
                ld.ipos_prev = delta ? ipos2[(it + 1) & 1] : nullptr;
                ld.fpos_prev = delta ? fpos2[(it + 1) & 1] : nullptr;
            }
            int32_t* const order = delta ? order2[it & 1] : pwork;
            int32_t* const offs = delta ? offs2[it & 1] : a.offsets;
            sort_front(nullptr, mfma ? P.nflag : nullptr, offs, kTileU, ld);
            hipLaunchKernelGGL(k_bucket, dim3((N + kTileU - 1) / kTileU, H), dim3(256), (size_t)C * 4, st,
                               a.labels, N, C, (N + kTileU - 1) / kTileU, kTileU, hist, offs, order,
                               delta ? tokflag : nullptr, ipos2[it & 1], fpos2[it & 1]);
            if (delta) {
                const int* chg = it > 0 ? changed : nullptr;
                if (it == 0)   // the first update reads every row: it also records the smallest magnitude
                    chunk_pass(X, range_x, order, nullptr, 1, 1, nullptr, offs);
                else
                    delta_pass(order, offs, fpos2[it & 1], order2[(it - 1) & 1], offs2[(it - 1) & 1],
                               fpos2[(it - 1) & 1], chg);
                hipLaunchKernelGGL((k_cluster_finalize<D, D == 128>), gfin, dim3(256), 0, st, a.counts,
                                   C, N, range_x, kPrec, it == 0 ? 1 : 0, it == 0 ? err : nullptr, 0, sums,
                                   cent64, (float*)nullptr, P.hi, P.lo, P.cn32, P.cn64, resid, chg, moved, 1);
                hipLaunchKernelGGL(k_plane_stats, dim3(H), dim3(256), 0, st, C, P.cn64, resid,
                                   P.stats);
                hipLaunchKernelGGL(k_moved_list, dim3(H), dim3(1024), 0, st, C, changed, moved,
                                   P.mlist, P.mpos, P.mcount);
            } else {
                // the first update reads every row: it also records the smallest magnitude
                mean_pass(X, range_x, pwork, it == 0 ? 1 : 0, 0, (float*)nullptr, 1, nullptr);
            }
        }
        if (delta && a.iters >= 2) zero_words(sums, (size_t)2 * H * C * D * 8, st);   // the final pass sums from zero
    }

    // Final reorder (stable counting sort), rows gathered, means of the final labels.
    sort_front(nullptr, nullptr, a.offsets, kTile, no_diff);
    // The scatter records the largest magnitude of V, and of X unless the k-means
    // has its range (its first assignment the largest, its first update the
    // smallest magnitude); a mean pass that collects records the smallest.
    const int row_chunks = (int)(D * sizeof(T) / 16);
    const bool given = (a.flags & SVGEAR_LABELS_GIVEN) != 0;
    const bool x_known = !given && a.iters >= 2;
    // With the range of X known, the final mean pass gathers the rows of X
    // itself (they are read there anyway); otherwise the scatter does, since
    // the mean pass needs the largest magnitude first.
    hipLaunchKernelGGL((k_scatter<T>), gtiles, dim3(256), 0, st, a.labels, N, C, ntiles, hist, a.offsets,
                       a.perm, a.inv_perm, x_known ? nullptr : (const uint4*)a.X, (uint4*)a.Xp,
                       (const uint4*)a.V, (uint4*)a.Vp, row_chunks, x_known ? nullptr : range_x, range_v, 1);
    mean_pass(X, range_x, a.perm, x_known ? 0 : 1, given ? 1 : 0, a.cent, 0,
              x_known ? (uint4*)a.Xp : nullptr);
    // V-bar: mean of V over the key clusters (zero for an empty cluster).  cent64
    // is no longer needed and serves as scratch.
    if (a.side == 1) mean_pass((const T*)a.V, range_v, a.perm, 1, 1, a.vbar, 0, nullptr);
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
