// route.hip -- step 3 of the SVG-EAR pipeline (review page, inference-pipeline
// paragraph, step 3, and the weaknesses paragraph that names greedy selection as
// an approximate 0-1 knapsack): per head, take blocks in descending ratio order
// (equal ratios: lower block index first) while their summed cost
// counts_q[c] * counts_k[g] stays within the budget; stop at the first block that
// does not fit.
//
// No sort is materialised.  Every block gets a distinct composite key
//     K(b) = order_key(ln r_b) * 2^IB + (2^IB - 1 - b),   IB = bits of the block count,
// so that the selection order is exactly descending K, and the selected set is
// "every block whose K exceeds that of the first block whose inclusive prefix
// cost exceeds the budget" (all blocks if none does).  That crossing key is
// found by a radix select, 12 bits per pass, most significant digit first, with
// cost-weighted (int64) histograms: the blocks still in play are those whose
// higher digits equal the digits chosen so far.  Each pass is one launch of
// several workgroups per head (a slice of the head's blocks each, LDS
// histogram, then integer atomics into the head's histogram in device memory);
// the last workgroup of a head to finish scans that histogram and records the
// chosen digit and the cost before it for the next pass.  A last launch writes
// the mask and the selected cost.
#include "internal.h"

namespace svg {

// Order-preserving map of a float to uint32 (NaN goes below -inf).
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int RT_DIGIT = 12;
constexpr int RT_BINS = 1 << RT_DIGIT;
constexpr int RT_THREADS = 256;
constexpr int RT_PER = RT_BINS / RT_THREADS;   // bins per thread in the scan

// Per head, in device memory: the digits chosen so far (prefix), the cost of
// every block ahead of the blocks still in play (base), whether some block
// crosses the budget, the per-slice selected costs and the arrival counter.
struct RouteState {
    unsigned long long prefix;
    long long base;
    int crosses;
    unsigned arrived;
};

struct RouteGeom {
    int nb, IB, npass, Ck;
    __device__ unsigned long long key(float lr, int b) const
    {
        return ((unsigned long long)order_key(lr) << IB) | (unsigned long long)(((1u << IB) - 1u) - (unsigned)b);
    }
    __device__ int shift(int pass) const { return RT_DIGIT * (npass - 1 - pass); }
};

// This workgroup's slice of the head's blocks.
__device__ __forceinline__ void route_slice(int nb, int& b0, int& b1)
{
    b0 = (int)(((long long)nb * blockIdx.x) / gridDim.x);
    b1 = (int)(((long long)nb * (blockIdx.x + 1)) / gridDim.x);
}

// True for the last workgroup of head h to get here; the arrival counter is
// reset for the next launch.  The workgroup's device-memory atomics (and
// device-scope stores) have completed before it counts itself (every wave waits
// for its memory counters, then the barrier), and the last one reads them with
// device-scope loads: no cache write-back fence is needed, which over many
// workgroups would cost far more than the work itself.
__device__ bool route_last_arrival(RouteState* st, int* s_flag)
{
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) expcnt(0) lgkmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned n = __hip_atomic_fetch_add(&st->arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = n == gridDim.x - 1;
        if (*s_flag) st->arrived = 0;
    }
    __syncthreads();
    return *s_flag != 0;
}

__global__ __launch_bounds__(RT_THREADS) void k_route_pass(
    const float* __restrict__ log_ratio, const int32_t* __restrict__ counts_q,
    const int32_t* __restrict__ counts_k, RouteGeom gm, int pass, long long budget,
    unsigned long long* __restrict__ ghist, RouteState* __restrict__ state)
{
    __shared__ unsigned long long s_hist[RT_BINS];
    __shared__ long long s_part[RT_THREADS];
    __shared__ int s_flag;
    const int h = blockIdx.y, tid = threadIdx.x;
    RouteState* st = state + h;
    const unsigned long long prefix = pass > 0 ? st->prefix : 0ull;
    if (pass > 0 && !st->crosses) return;   // every block fits: nothing left to choose
    const int sh = gm.shift(pass);
    for (int i = tid; i < RT_BINS; i += RT_THREADS) s_hist[i] = 0ull;
    __syncthreads();
    const float* lr = log_ratio + (size_t)h * gm.nb;
    const int32_t* cq = counts_q + (size_t)h * (gm.nb / gm.Ck);
    const int32_t* ck = counts_k + (size_t)h * gm.Ck;
    int b0, b1;
    route_slice(gm.nb, b0, b1);
    for (int b = b0 + tid; b < b1; b += RT_THREADS) {
        const unsigned long long K = gm.key(lr[b], b);
        if (pass > 0 && (K >> (sh + RT_DIGIT)) != prefix) continue;
        const int c = b / gm.Ck, g = b - c * gm.Ck;
        const long long w = (long long)cq[c] * (long long)ck[g];
        if (w) atomicAdd(&s_hist[(K >> sh) & (RT_BINS - 1)], (unsigned long long)w);
    }
    __syncthreads();
    unsigned long long* gh = ghist + (size_t)h * RT_BINS;
    for (int i = tid; i < RT_BINS; i += RT_THREADS)
        if (s_hist[i]) __hip_atomic_fetch_add(&gh[i], s_hist[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!route_last_arrival(st, &s_flag)) return;

    // The last workgroup: scan the head's histogram from the top digit down.
    // Thread t owns digits RT_BINS - 1 - RT_PER t - j, j = 0 .. RT_PER - 1.
    long long v[RT_PER], sum = 0;
#pragma unroll
    for (int j = 0; j < RT_PER; ++j) {
        const int dg = RT_BINS - 1 - RT_PER * tid - j;
        v[j] = (long long)__hip_atomic_load(&gh[dg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sum += v[j];
    }
    s_part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < RT_THREADS; off <<= 1) {   // inclusive scan over threads
        const long long t = tid >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += t;
        __syncthreads();
    }
    const long long base = pass > 0 ? st->base : 0;
    long long acc = base + s_part[tid] - sum;   // cost ahead of this thread's digits
    if (tid == 0) s_flag = -1;
    __syncthreads();
    if (acc <= budget && acc + sum > budget) {   // the crossing digit is one of this thread's
#pragma unroll
        for (int j = 0; j < RT_PER; ++j) {
            if (acc + v[j] > budget) {
                st->prefix = (prefix << RT_DIGIT) | (unsigned long long)(RT_BINS - 1 - RT_PER * tid - j);
                st->base = acc;
                st->crosses = 1;
                s_flag = tid;
                break;
            }
            acc += v[j];
        }
    }
    __syncthreads();
    if (s_flag < 0 && tid == 0) st->crosses = 0;   // the whole head fits (first pass only)
    for (int i = tid; i < RT_BINS; i += RT_THREADS) gh[i] = 0ull;   // clean for the next pass
}

// Mask and selected cost: block b is selected when no block crosses the budget
// or K(b) exceeds the crossing key.  Per-slice costs are summed by the last
// workgroup of the head (exact integers).
__global__ __launch_bounds__(RT_THREADS) void k_route_mask(
    const float* __restrict__ log_ratio, const int32_t* __restrict__ counts_q,
    const int32_t* __restrict__ counts_k, RouteGeom gm, RouteState* __restrict__ state,
    long long* __restrict__ part, uint8_t* __restrict__ mask, long long* __restrict__ sel_cost)
{
    __shared__ long long s_red[RT_THREADS / 64];
    __shared__ int s_flag;
    const int h = blockIdx.y, tid = threadIdx.x;
    RouteState* st = state + h;
    const bool crosses = st->crosses != 0;
    const unsigned long long Kx = st->prefix;
    const float* lr = log_ratio + (size_t)h * gm.nb;
    const int32_t* cq = counts_q + (size_t)h * (gm.nb / gm.Ck);
    const int32_t* ck = counts_k + (size_t)h * gm.Ck;
    uint8_t* mk = mask + (size_t)h * gm.nb;
    int b0, b1;
    route_slice(gm.nb, b0, b1);
    long long used = 0;
    for (int b = b0 + tid; b < b1; b += RT_THREADS) {
        const bool sel = !crosses || gm.key(lr[b], b) > Kx;
        mk[b] = sel ? 1 : 0;
        if (sel) {
            const int c = b / gm.Ck, g = b - c * gm.Ck;
            used += (long long)cq[c] * (long long)ck[g];
        }
    }
    for (int o = 32; o >= 1; o >>= 1) used += __shfl_xor(used, o);
    if ((tid & 63) == 0) s_red[tid >> 6] = used;
    __syncthreads();
    if (tid == 0) {
        long long t = 0;
        for (int k = 0; k < RT_THREADS / 64; ++k) t += s_red[k];
        __hip_atomic_store(&part[(size_t)h * gridDim.x + blockIdx.x], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!route_last_arrival(st, &s_flag)) return;
    if (tid == 0) {
        long long t = 0;
        for (int k = 0; k < (int)gridDim.x; ++k)
            t += __hip_atomic_load(&part[(size_t)h * gridDim.x + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sel_cost[h] = t;
    }
}

SVG_HIDDEN int route_slices(int H)
{
    int s = 480 / (H > 0 ? H : 1);
    return s < 1 ? 1 : (s > 32 ? 32 : s);
}

SVG_HIDDEN hipError_t launch_route(const RouteArgs& a, hipStream_t st)
{
    const int nb = a.Cq * a.Ck;
    int IB = 1;
    while ((1 << IB) < nb) ++IB;
    RouteGeom gm{nb, IB, (32 + IB + RT_DIGIT - 1) / RT_DIGIT, a.Ck};
    const int S = route_slices(a.H);
    const Layout& L = *a.L;
    unsigned long long* ghist = (unsigned long long*)(a.scratch + L.rt_hist);
    RouteState* state = (RouteState*)(a.scratch + L.rt_state);
    long long* part = (long long*)(a.scratch + L.rt_part);
    // the histograms and states are contiguous: one fill clears both
    zero_words(ghist, L.rt_end - L.rt_hist, st);
    const dim3 grid(S, a.H);
    for (int p = 0; p < gm.npass; ++p)
        hipLaunchKernelGGL(k_route_pass, grid, dim3(RT_THREADS), 0, st, a.log_ratio, a.counts_q,
                           a.counts_k, gm, p, (long long)a.budget, ghist, state);
    hipLaunchKernelGGL(k_route_mask, grid, dim3(RT_THREADS), 0, st, a.log_ratio, a.counts_q, a.counts_k,
                       gm, state, part, a.mask, (long long*)a.sel_cost);
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
