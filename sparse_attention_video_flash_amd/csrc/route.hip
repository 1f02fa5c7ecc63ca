// route.hip -- step 3 of the SVG-EAR pipeline (review page, inference-pipeline
// paragraph, step 3, and the weaknesses paragraph that names greedy selection as
// an approximate 0-1 knapsack): per head, take blocks in descending ratio order
// (equal ratios: lower block index first) while their summed cost
// counts_q[c] * counts_k[g] stays within the budget; stop at the first block that
// does not fit.
//
// No sort is materialised.  The selected set is "every block before the first
// block whose inclusive prefix cost exceeds the budget", so it is enough to find
// that block: a radix select over the 32-bit order key, one byte per pass, with
// cost-weighted (int64) LDS histograms, then an in-order prefix scan over the
// blocks that share the final key (the tie group, ordered by block index).  One
// workgroup per head; the ratio array stays in L2 between passes.
#include "internal.h"

namespace svg {

// Order-preserving map of a float to uint32 (NaN goes below -inf).
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kRouteThreads = 1024;

__device__ long long block_sum_i64(long long v, long long* s_red)
{
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s_red[w] = v;
    __syncthreads();
    long long t = 0;
    for (int k = 0; k < kRouteThreads / 64; ++k) t += s_red[k];
    return t;
}

// Block b = c Ck + g of this thread in a sweep b = b0 + threadIdx.x, b0 += kRouteThreads:
// (c, g) advanced without a division per step.
struct BlockWalk {
    int c, g, dc, dg;
    __device__ BlockWalk(int Ck)
    {
        c = (int)threadIdx.x / Ck;
        g = (int)threadIdx.x - c * Ck;
        dc = kRouteThreads / Ck;
        dg = kRouteThreads - dc * Ck;
    }
    __device__ void next(int Ck)
    {
        c += dc;
        g += dg;
        if (g >= Ck) {
            g -= Ck;
            ++c;
        }
    }
};

__global__ __launch_bounds__(kRouteThreads) void k_route(const float* __restrict__ log_ratio,
                                                         const int32_t* __restrict__ counts_q,
                                                         const int32_t* __restrict__ counts_k,
                                                         int Cq, int Ck, long long budget,
                                                         uint8_t* __restrict__ mask,
                                                         long long* __restrict__ sel_cost)
{
    __shared__ long long s_hist[256];
    __shared__ long long s_red[kRouteThreads / 64];
    __shared__ long long s_scan[kRouteThreads];
    __shared__ int s_cq[kMaxC], s_ck[kMaxC];
    __shared__ int s_stop;
    __shared__ uint32_t s_prefix;
    __shared__ long long s_base;
    __shared__ int s_found;

    const int h = blockIdx.x;
    const int nb = Cq * Ck;
    const float* lr = log_ratio + (size_t)h * nb;
    for (int i = threadIdx.x; i < Cq; i += kRouteThreads) s_cq[i] = counts_q[(size_t)h * Cq + i];
    for (int i = threadIdx.x; i < Ck; i += kRouteThreads) s_ck[i] = counts_k[(size_t)h * Ck + i];
    __syncthreads();

    // Radix select of the key of the first block that does not fit.
    uint32_t prefix = 0;     // determined high bits of the crossing key
    long long base = 0;      // cost of all blocks with a larger key
    bool crosses = true;
    for (int pass = 0; pass < 4 && crosses; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int b = threadIdx.x; b < 256; b += kRouteThreads) s_hist[b] = 0;
        __syncthreads();
        BlockWalk bw(Ck);
        for (int b0 = 0; b0 < nb; b0 += kRouteThreads, bw.next(Ck)) {
            const int b = b0 + threadIdx.x;
            uint32_t key = 0;
            long long w = 0;
            if (b < nb) {
                key = order_key(lr[b]);
                const bool match = pass == 0 || (key >> (shift + 8)) == prefix;
                if (match) w = (long long)s_cq[bw.c] * (long long)s_ck[bw.g];
            }
            if (w) atomicAdd((unsigned long long*)&s_hist[(key >> shift) & 255u], (unsigned long long)w);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            long long acc = base;
            int found = 0;
            for (int bk = 255; bk >= 0; --bk) {
                if (acc + s_hist[bk] > budget) {
                    s_prefix = (prefix << 8) | (uint32_t)bk;
                    found = 1;
                    break;
                }
                acc += s_hist[bk];
            }
            s_found = found;
            s_base = acc;
        }
        __syncthreads();
        crosses = s_found != 0;
        if (crosses) {
            prefix = s_prefix;
            base = s_base;
        }
        __syncthreads();
    }

    // Tie group (key == prefix) in block-index order: the first block whose
    // inclusive prefix cost exceeds the budget stops the walk.  Sweeps with no
    // member of the group skip the scan.
    int stop = nb;
    if (crosses) {
        if (threadIdx.x == 0) s_stop = nb;
        __syncthreads();
        long long run = base;
        BlockWalk bw(Ck);
        for (int b0 = 0; b0 < nb; b0 += kRouteThreads, bw.next(Ck)) {
            const int b = b0 + threadIdx.x;
            long long w = 0;
            if (b < nb && order_key(lr[b]) == prefix) w = (long long)s_cq[bw.c] * (long long)s_ck[bw.g];
            if (!__syncthreads_or(w > 0)) continue;
            s_scan[threadIdx.x] = w;
            __syncthreads();
            for (int off = 1; off < kRouteThreads; off <<= 1) {
                long long v = (int)threadIdx.x >= off ? s_scan[threadIdx.x - off] : 0;
                __syncthreads();
                s_scan[threadIdx.x] += v;
                __syncthreads();
            }
            if (w > 0 && run + s_scan[threadIdx.x] > budget) atomicMin(&s_stop, b);
            run += s_scan[kRouteThreads - 1];
            __syncthreads();
            if (s_stop < nb) break;
        }
        stop = s_stop;
    }

    long long used = 0;
    uint8_t* mk = mask + (size_t)h * nb;
    BlockWalk bw(Ck);
    for (int b0 = 0; b0 < nb; b0 += kRouteThreads, bw.next(Ck)) {
        const int b = b0 + threadIdx.x;
        if (b >= nb) continue;
        bool sel = true;
        if (crosses) {
            const uint32_t key = order_key(lr[b]);
            sel = key > prefix || (key == prefix && b < stop);
        }
        mk[b] = sel ? 1 : 0;
        if (sel) used += (long long)s_cq[bw.c] * (long long)s_ck[bw.g];
    }
    used = block_sum_i64(used, s_red);
    if (threadIdx.x == 0) sel_cost[h] = used;
}

SVG_HIDDEN hipError_t launch_route(const RouteArgs& a, hipStream_t st)
{
    hipLaunchKernelGGL(k_route, dim3(a.H), dim3(kRouteThreads), 0, st, a.log_ratio, a.counts_q,
                       a.counts_k, a.Cq, a.Ck, (long long)a.budget, a.mask,
                       (long long*)a.sel_cost);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- per-cluster budgets
//
// The other reading of the budget ([R] future-work paragraph: one density
// budget for every query cluster): query cluster c may spend
// B_c = floor((rho * n_c) * Nk) pairs on its own row of blocks, chosen greedily
// in descending ratio order (equal ratios: lower key-cluster index first), the
// longest prefix that fits.  One workgroup per (head, row): the row's order
// keys are sorted in LDS (bitonic, 64-bit keys = descending order key, then
// index), then an inclusive cost scan marks the prefix.  The row's selected
// cost is added to sel_cost[h] (integer atomics, exact).
constexpr int kRowThreads = 256;
constexpr int kRowMax = 4096;

__global__ __launch_bounds__(kRowThreads) void k_route_rows(const float* __restrict__ log_ratio,
                                                            const int32_t* __restrict__ counts_q,
                                                            const int32_t* __restrict__ counts_k,
                                                            int Cq, int Ck, int Nk, double rho,
                                                            uint8_t* __restrict__ mask,
                                                            unsigned long long* __restrict__ sel_cost)
{
    __shared__ unsigned long long s_key[kRowMax];
    __shared__ long long s_part[kRowThreads];
    const int c = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x;
    int n = 1;
    while (n < Ck) n <<= 1;
    const float* lr = log_ratio + ((size_t)h * Cq + c) * Ck;
    for (int i = tid; i < n; i += kRowThreads)
        s_key[i] = i < Ck ? ((unsigned long long)(~order_key(lr[i])) << 32) | (unsigned)i : ~0ull;
    __syncthreads();
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < n; i += kRowThreads) {
                const int l = i ^ j;
                if (l > i) {
                    const unsigned long long a = s_key[i], b = s_key[l];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        s_key[i] = b;
                        s_key[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    // costs in sorted order, thread-contiguous runs, then a block scan of the runs
    const long long nc = counts_q[(size_t)h * Cq + c];
    const int32_t* ck = counts_k + (size_t)h * Ck;
    const long long budget = (long long)floor((rho * (double)nc) * (double)Nk);
    const int per = (Ck + kRowThreads - 1) / kRowThreads;
    const int p0 = tid * per;
    long long run = 0;
    for (int k = 0; k < per && p0 + k < Ck; ++k) run += nc * ck[(int)(s_key[p0 + k] & 0xffffffffu)];
    s_part[tid] = run;
    __syncthreads();
    for (int off = 1; off < kRowThreads; off <<= 1) {
        const long long v = tid >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += v;
        __syncthreads();
    }
    long long cum = s_part[tid] - run;
    long long mine = 0;
    uint8_t* mrow = mask + ((size_t)h * Cq + c) * Ck;
    for (int k = 0; k < per && p0 + k < Ck; ++k) {
        const int g = (int)(s_key[p0 + k] & 0xffffffffu);
        const long long w = nc * ck[g];
        cum += w;
        const bool take = cum <= budget;
        mrow[g] = take ? 1 : 0;
        if (take) mine += w;
    }
    s_part[tid] = mine;
    __syncthreads();
    if (tid == 0) {
        long long tot = 0;
        for (int k = 0; k < kRowThreads; ++k) tot += s_part[k];
        atomicAdd(sel_cost + h, (unsigned long long)tot);
    }
}

SVG_HIDDEN hipError_t launch_route_rows(const RouteArgs& a, double rho, int Nk, hipStream_t st)
{
    zero_words(a.sel_cost, (size_t)a.H * 8, st);
    hipLaunchKernelGGL(k_route_rows, dim3(a.Cq, a.H), dim3(kRowThreads), 0, st, a.log_ratio,
                       a.counts_q, a.counts_k, a.Cq, a.Ck, Nk, rho, a.mask,
                       (unsigned long long*)a.sel_cost);
    return hipGetLastError();
}

}  // namespace svg
