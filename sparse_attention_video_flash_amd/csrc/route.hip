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
// higher digits equal the digits chosen so far.  Heads of up to 2^18 blocks
// take two launches: per-slice top-digit histograms and the top 24 key bits of
// every block, then one workgroup per head for every later pass and the mask
// (k_route_top, k_route_head).  Larger heads take one launch per pass, several
// workgroups per head (a slice of the head's blocks each, LDS histogram, then
// integer atomics into the head's histogram in device memory); the last
// workgroup of a head to finish scans that histogram and records the chosen
// digit and the cost before it for the next pass, and a last launch writes the
// mask and the selected cost.
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
    // digits aligned at the bottom of the key (the first may be narrower)
    __device__ int shift(int pass) const { return RT_DIGIT * (npass - 1 - pass); }
    // digits aligned at the top of the key, so that the first two are bits of
    // the ratio's order key whatever IB is (the last may be narrower)
    __device__ int tshift(int pass) const
    {
        const int s = 32 + IB - RT_DIGIT * (pass + 1);
        return s > 0 ? s : 0;
    }
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

// ----------------------------------------------------------------------------- heads of up to 2^18 blocks
//
// Two launches.  The digits are aligned at the top of the key (the last pass
// takes what is left), so the first two are the top 24 bits of the order key of
// a block's ratio (its "word"), whatever the block count: a first digit of
// the full 12 bits keeps few blocks in play however many index bits follow.
// k_route_top: S workgroups per head, each over a slice of the head's blocks:
// the LDS histogram of the top digit, written whole to its own slot (no
// device-memory atomics, nothing to clear), and every block's word (a row of P
// words per head, P = the block count rounded up to 4).  k_route_head: one
// workgroup of 1024 threads per head sums the S histograms and scans them; the
// second pass sweeps the words (four per 16-byte load); the third sweeps them
// again and only the blocks whose word equals the chosen 24-bit prefix load
// their ratio: they are kept as composite keys in an LDS list, so that the
// later passes read no device memory unless more than RH_CAND blocks share the
// prefix (then they sweep the words again).  A last sweep of the words writes
// the mask, the blocks of the listed prefix taking theirs from the list.  The
// selected cost needs no sweep: it is the cost ahead of the crossing key, which
// the last pass's scan yields (the whole head's cost when nothing crosses).
constexpr int RH_THREADS = 1024;
constexpr int RH_CAND = 8192;
constexpr int RH_MAX_BLOCKS = 1 << 18;
constexpr int RH_BATCH = 16;        // ratios loaded together per thread of k_route_top
constexpr int RH_SLICES = 16;       // at most this many slices per head
constexpr int RH_SLICE_BLOCKS = 8192;   // blocks per slice aimed at
constexpr int RH_SLICE_LOAD = 8;    // slice histograms loaded together per thread
constexpr int RH_VEC = 4;           // words per 16-byte load

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int route_word_pitch(int nb) { return (nb + RH_VEC - 1) / RH_VEC * RH_VEC; }

SVG_HIDDEN int route_top_slices(int nb)
{
    const int s = (nb + RH_SLICE_BLOCKS - 1) / RH_SLICE_BLOCKS;
    return s < 1 ? 1 : (s > RH_SLICES ? RH_SLICES : s);
}

SVG_HIDDEN size_t route_top_bytes(int H, int nb)
{
    if (nb > RH_MAX_BLOCKS) return 0;
    return align256((size_t)H * route_top_slices(nb) * RT_BINS * 8) + (size_t)H * route_word_pitch(nb) * 4;
}

struct RhStep {
    int c, g, dc, dg, Ck;
    __device__ void start(int b, int stride, int Ck_)
    {
        Ck = Ck_;
        c = b / Ck;
        g = b - c * Ck;
        dc = stride / Ck;
        dg = stride - dc * Ck;
    }
    __device__ void next()
    {
        c += dc;
        g += dg;
        if (g >= Ck) {
            g -= Ck;
            ++c;
        }
    }
};

__global__ __launch_bounds__(RT_THREADS) void k_route_top(
    const float* __restrict__ log_ratio, const int32_t* __restrict__ counts_q,
    const int32_t* __restrict__ counts_k, RouteGeom gm, unsigned long long* __restrict__ part,
    uint32_t* __restrict__ words)
{
    extern __shared__ int s_cnt[];   // counts_q of the head, then counts_k
    __shared__ unsigned long long s_hist[RT_BINS];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int Cq = gm.nb / gm.Ck;
    for (int i = tid; i < RT_BINS; i += RT_THREADS) s_hist[i] = 0ull;
    for (int i = tid; i < Cq; i += RT_THREADS) s_cnt[i] = counts_q[(size_t)h * Cq + i];
    for (int i = tid; i < gm.Ck; i += RT_THREADS) s_cnt[Cq + i] = counts_k[(size_t)h * gm.Ck + i];
    __syncthreads();
    const float* lr = log_ratio + (size_t)h * gm.nb;
    uint32_t* wh = words + (size_t)h * route_word_pitch(gm.nb);
    constexpr int wsh = 32 - 2 * RT_DIGIT;   // the word: the top 24 bits of the order key
    int b0, b1;
    route_slice(gm.nb, b0, b1);
    RhStep cg;
    cg.start(b0 + tid, RT_THREADS, gm.Ck);
    for (int bb = b0 + tid; bb < b1; bb += RT_THREADS * RH_BATCH) {
        float v[RH_BATCH];
#pragma unroll
        for (int u = 0; u < RH_BATCH; ++u) {
            const int b = bb + u * RT_THREADS;
            v[u] = b < b1 ? lr[b] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < RH_BATCH; ++u, cg.next()) {
            const int b = bb + u * RT_THREADS;
            if (b >= b1) continue;
            const unsigned w24 = order_key(v[u]) >> wsh;
            wh[b] = w24;
            const long long w = (long long)s_cnt[cg.c] * (long long)s_cnt[Cq + cg.g];
            atomicAdd(&s_hist[w24 >> RT_DIGIT], (unsigned long long)w);
        }
    }
    __syncthreads();
    unsigned long long* out = part + ((size_t)h * gridDim.x + blockIdx.x) * RT_BINS;
    for (int i = tid; i < RT_BINS; i += RT_THREADS) out[i] = s_hist[i];
}

// Scan of a histogram from the top digit down, thread t holding digits
// RT_BINS - 1 - 4t - j in v[j].  When the running cost (from base) first exceeds
// the budget inside digit dg, the owner records dg and the cost ahead of it in
// s_dig / s_base; s_dig must be -1 on entry and stays so when everything fits.
// s_total receives base plus the whole histogram.
__device__ void rh_scan(const long long (&v)[RT_BINS / RH_THREADS], long long* s_wsum, long long base,
                        long long budget, int* s_dig, long long* s_base, long long* s_total)
{
    constexpr int PER = RT_BINS / RH_THREADS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    long long sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) sum += v[j];
    long long inc = sum;   // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const long long t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    long long acc = base + inc - sum;
    for (int k = 0; k < wave; ++k) acc += s_wsum[k];
    if (tid == RH_THREADS - 1) *s_total = acc + sum;
    if (acc <= budget && acc + sum > budget) {   // exactly one thread
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (acc + v[j] > budget) {
                *s_dig = RT_BINS - 1 - PER * tid - j;
                *s_base = acc;
                break;
            }
            acc += v[j];
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(RH_THREADS) void k_route_head(
    const float* __restrict__ log_ratio, const int32_t* __restrict__ counts_q,
    const int32_t* __restrict__ counts_k, RouteGeom gm, int S, long long budget,
    const unsigned long long* __restrict__ part, const uint32_t* __restrict__ words,
    uint8_t* __restrict__ mask, long long* __restrict__ sel_cost)
{
    constexpr int PER = RT_BINS / RH_THREADS;
    extern __shared__ int s_cnt[];   // counts_q of the head, then counts_k
    __shared__ unsigned long long s_hist[RT_BINS];
    __shared__ unsigned long long s_cand[RH_CAND];
    __shared__ long long s_wsum[RH_THREADS / 64];
    __shared__ long long s_base, s_total;
    __shared__ int s_dig, s_ncand;
    const int h = blockIdx.x, tid = threadIdx.x;
    const int Cq = gm.nb / gm.Ck;
    int* s_cq = s_cnt;
    int* s_ck = s_cnt + Cq;
    for (int i = tid; i < Cq; i += RH_THREADS) s_cq[i] = counts_q[(size_t)h * Cq + i];
    for (int i = tid; i < gm.Ck; i += RH_THREADS) s_ck[i] = counts_k[(size_t)h * gm.Ck + i];
    if (tid == 0) {
        s_ncand = 0;
        s_dig = -1;
    }
    const float* lr = log_ratio + (size_t)h * gm.nb;
    const int nvec = route_word_pitch(gm.nb) / RH_VEC;
    const u32x4* wv = (const u32x4*)(words + (size_t)h * route_word_pitch(gm.nb));
    const unsigned ibm = (1u << gm.IB) - 1u;
    auto cost = [&](int b) {
        const int c = b / gm.Ck, g = b - c * gm.Ck;
        return (unsigned long long)((long long)s_cq[c] * (long long)s_ck[g]);
    };
    // the blocks of vector iv: bit e set where the word tests true
    auto select = [&](const u32x4& w4, int iv, auto pred) {
        unsigned in = 0;
#pragma unroll
        for (int e = 0; e < RH_VEC; ++e) in |= (pred(w4[e]) ? 1u : 0u) << e;
        const int bb = iv * RH_VEC;
        if (bb + RH_VEC > gm.nb) in &= (1u << (gm.nb - bb)) - 1u;   // words past the blocks
        return in;
    };

    // First pass: the sum of the slices' histograms of the top digit.  This
    // thread's four digits are adjacent (32 bytes per slice); the slices were
    // written by other workgroups, so their loads go past this L2 and are all
    // issued before the first is used.
    long long v[PER] = {0, 0, 0, 0};
    {
        static_assert(PER == 4, "four digits per thread");
        const u64x2* ph = (const u64x2*)(part + (size_t)h * S * RT_BINS + (RT_BINS - PER * (tid + 1)));
        for (int k0 = 0; k0 < S; k0 += RH_SLICE_LOAD) {
            u64x2 x[RH_SLICE_LOAD][2];
#pragma unroll
            for (int q = 0; q < RH_SLICE_LOAD; ++q) {
                if (k0 + q < S) {
                    x[q][0] = ph[(size_t)(k0 + q) * (RT_BINS / 2)];
                    x[q][1] = ph[(size_t)(k0 + q) * (RT_BINS / 2) + 1];
                } else {
                    x[q][0] = x[q][1] = u64x2{0, 0};
                }
            }
#pragma unroll
            for (int q = 0; q < RH_SLICE_LOAD; ++q) {   // ascending addresses: digits top - 3 .. top
                v[3] += (long long)x[q][0][0];
                v[2] += (long long)x[q][0][1];
                v[1] += (long long)x[q][1][0];
                v[0] += (long long)x[q][1][1];
            }
        }
    }
    __syncthreads();
    rh_scan(v, s_wsum, 0, budget, &s_dig, &s_base, &s_total);
    const bool crosses = s_dig >= 0;
    unsigned long long prefix = crosses ? (unsigned)s_dig : 0u;
    long long base = s_base;
    long long used = s_total;
    unsigned w2 = 0;   // the 24-bit prefix once the second pass has chosen it
    for (int pass = 1; crosses && pass < gm.npass; ++pass) {
        const int sh = gm.tshift(pass), hs = gm.tshift(pass - 1);   // this digit: key bits sh .. hs - 1
        const unsigned long long dm = (1ull << (hs - sh)) - 1ull;
        __syncthreads();   // everyone has read s_dig, s_base and s_total
        for (int i = tid; i < RT_BINS; i += RH_THREADS) s_hist[i] = 0ull;
        if (tid == 0) s_dig = -1;
        __syncthreads();
        const int nc = s_ncand;
        if (pass == 1) {
            // second digit straight from the words; block 4 iv + e is query
            // cluster c, key cluster g + e (wrapped), (c, g) stepped per vector
            const unsigned d0 = (unsigned)prefix;
            RhStep cg;
            cg.start(tid * RH_VEC, RH_THREADS * RH_VEC, gm.Ck);
            for (int iv = tid; iv < nvec; iv += RH_THREADS, cg.next()) {
                const u32x4 w4 = wv[iv];
                const unsigned in = select(w4, iv, [&](unsigned w) { return (w >> RT_DIGIT) == d0; });
                if (!in) continue;
#pragma unroll
                for (int e = 0; e < RH_VEC; ++e) {
                    int c = cg.c, g = cg.g + e;
                    while (g >= gm.Ck) {   // once at most unless C_k < 4
                        g -= gm.Ck;
                        ++c;
                    }
                    if ((in >> e) & 1u)
                        atomicAdd(&s_hist[w4[e] & (RT_BINS - 1)],
                                  (unsigned long long)((long long)s_cq[c] * (long long)s_ck[g]));
                }
            }
        } else if (pass == 2 || nc > RH_CAND) {
            // the blocks of the 24-bit prefix: their keys (listed by the third
            // pass; a later pass tests the rest of the prefix on the key)
            for (int iv = tid; iv < nvec; iv += RH_THREADS) {
                const u32x4 w4 = wv[iv];
                unsigned in = select(w4, iv, [&](unsigned w) { return w == w2; });
                if (!in) continue;
                float r[RH_VEC];
#pragma unroll
                for (int e = 0; e < RH_VEC; ++e) r[e] = ((in >> e) & 1u) ? lr[iv * RH_VEC + e] : 0.f;
                int pos = 0;
                if (pass == 2) pos = atomicAdd(&s_ncand, __popc(in));
#pragma unroll
                for (int e = 0; e < RH_VEC; ++e) {
                    if (!((in >> e) & 1u)) continue;
                    const int b = iv * RH_VEC + e;
                    const unsigned long long K = gm.key(r[e], b);
                    if (pass == 2) {
                        if (pos < RH_CAND) s_cand[pos] = K;
                        ++pos;
                    } else if ((K >> hs) != prefix) {
                        continue;
                    }
                    atomicAdd(&s_hist[(K >> sh) & dm], cost(b));
                }
            }
        } else {
            for (int i = tid; i < nc; i += RH_THREADS) {
                const unsigned long long K = s_cand[i];
                if ((K >> hs) != prefix) continue;
                atomicAdd(&s_hist[(K >> sh) & dm], cost((int)(ibm - (unsigned)(K & ibm))));
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j) v[j] = (long long)s_hist[RT_BINS - 1 - PER * tid - j];
        rh_scan(v, s_wsum, base, budget, &s_dig, &s_base, &s_total);
        prefix = (prefix << (hs - sh)) | (unsigned long long)s_dig;   // a later digit always crosses
        base = s_base;
        if (pass == 1) w2 = (unsigned)prefix;
    }
    if (crosses) used = base;   // the cost of every block whose key exceeds the crossing key
    // Mask: every block whose key exceeds the crossing key (all when none
    // crosses).  The words above the crossing key's 24-bit prefix are taken, those
    // below are not; the blocks of the prefix itself take their key from the list.
    const int nc = s_ncand;
    const bool listed = nc <= RH_CAND;
    uint8_t* mk = mask + (size_t)h * gm.nb;
    // whole vectors whose four words all differ from the prefix write four mask
    // bytes at once where the row is 4-byte aligned
    const bool aligned = (((uintptr_t)mk) & 3u) == 0;
    for (int iv = tid; iv < nvec; iv += RH_THREADS) {
        const u32x4 w4 = wv[iv];
        const int bb = iv * RH_VEC;
        if (aligned && bb + RH_VEC <= gm.nb &&
            (!crosses || (w4[0] != w2 && w4[1] != w2 && w4[2] != w2 && w4[3] != w2))) {
            unsigned m4 = 0;
#pragma unroll
            for (int e = 0; e < RH_VEC; ++e) m4 |= ((!crosses || w4[e] > w2) ? 1u : 0u) << (8 * e);
            *(uint32_t*)(mk + bb) = m4;
            continue;
        }
#pragma unroll
        for (int e = 0; e < RH_VEC; ++e) {
            const int b = bb + e;
            if (b >= gm.nb) break;
            const unsigned w = w4[e];
            if (!crosses || w != w2) {
                mk[b] = (!crosses || w > w2) ? 1 : 0;
            } else if (!listed) {
                mk[b] = gm.key(lr[b], b) > prefix ? 1 : 0;
            }
        }
    }
    if (crosses && listed) {
        for (int i = tid; i < nc; i += RH_THREADS) {
            const unsigned long long K = s_cand[i];
            mk[ibm - (unsigned)(K & ibm)] = K > prefix ? 1 : 0;
        }
    }
    if (tid == 0) sel_cost[h] = used;
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
    const Layout& L = *a.L;
    if (nb <= RH_MAX_BLOCKS) {
        const int S = route_top_slices(nb);
        unsigned long long* top = (unsigned long long*)(a.scratch + L.rt_top);
        uint32_t* words = (uint32_t*)(a.scratch + L.rt_top + align256((size_t)a.H * S * RT_BINS * 8));
        const size_t lds = (size_t)(a.Cq + a.Ck) * 4;
        hipLaunchKernelGGL(k_route_top, dim3(S, a.H), dim3(RT_THREADS), lds, st, a.log_ratio, a.counts_q,
                           a.counts_k, gm, top, words);
        hipLaunchKernelGGL(k_route_head, dim3(a.H), dim3(RH_THREADS), lds, st, a.log_ratio, a.counts_q,
                           a.counts_k, gm, S, (long long)a.budget, top, words, a.mask, (long long*)a.sel_cost);
        return hipGetLastError();
    }
    const int S = route_slices(a.H);
    unsigned long long* ghist = (unsigned long long*)(a.scratch + L.rt_hist);
    RouteState* state = (RouteState*)(a.scratch + L.rt_state);
    long long* part = (long long*)(a.scratch + L.rt_part);
    // the states and histograms are contiguous: one fill clears both
    zero_words(a.scratch + L.rt_state, L.rt_top - L.rt_state, st);
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
