// attn_mfma.hip -- hybrid attention on bf16 MFMA for d = 128 (step 4 of the
// SVG-EAR pipeline: exact blocks plus parameter-free centroid compensation,
// review page inference-pipeline paragraph; German summary 2A).
//
// One workgroup (8 waves) owns a tile of BM = 256 reordered query rows of one
// query cluster c; each wave owns 32 queries.  Scores are computed transposed,
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every lane holds one query
// column and the softmax row statistics stay inside a lane (one exchange with
// the partner half-wave per tile for the running max).  The probabilities are
// then already the B operand of O^T = V^T P^T; the V^T operand is read from the
// row-major value tile with ds_read_b64_tr_b16 (within each 16-lane group,
// result lane i, element k comes from source lane 4k + i/4, element i % 4), two
// loads per fragment.
//
// Key tiles of BN = 64 rows, packed: a tile takes the next 64 entries of the
// cluster's key list, so no tile is padded at a key-cluster boundary.
//   1. compensation tiles: the centroids of the key clusters that are skipped
//      for c and non-empty, with logit tau q.kbar_g + ln m_g: k-bar (fp32) split
//      into bf16 hi + lo planes, since the logit enters an exponential; v-bar
//      rounded once to bf16, as every value and weight of the PV product is;
//   2. exact tiles: the keys of every routed key cluster.
// Both kinds are gathered by row index straight from global memory into LDS
// (buffer loads with the lds flag), two buffers deep, the next tile's loads in
// flight during the current tile's math.  One online softmax (base-2
// exponent, lazily raised reference max) covers both kinds of terms.
//
// The kernel is persistent (one workgroup per CU) and takes query tiles from
// eight work queues, one per XCD: tiles are dealt to queue c mod 8 by query
// cluster, so the tiles of one cluster, which read the same keys, run
// together on one XCD and share its L2 (see the queue kernels below).
#include "internal.h"

namespace svg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int AT_WAVES = 8;                  // 32 query rows per wave; one workgroup per CU
constexpr int AT_BM = 32 * AT_WAVES;
constexpr int AT_BN = 64;
constexpr int AT_D = 128;
constexpr int AT_THREADS = 64 * AT_WAVES;
// Key and value tiles: 64 rows of 256 B, unpadded, the 16-B chunks of each row
// XOR-swizzled so that the score reads (16 rows, one chunk) and the transpose
// reads (4 rows, 4 chunks) hit distinct banks.  The exact tiles are written
// straight from global memory into LDS (one buffer load with the lds flag
// fills 4 rows of one operand), two buffers deep.
constexpr int ROW_B = AT_D * 2;          // 256
constexpr int T_BUF = AT_BN * ROW_B;     // 16384
constexpr int AT_NBUF = 2;
constexpr int K_PITCH = AT_D * 2 + 16;   // output staging rows (272 B)
// Compensation tiles: k-bar hi, k-bar lo and v-bar (bf16) planes of 64
// centroids per buffer, two buffers, then the two buffers' biases.
constexpr int C_BUF = 3 * T_BUF;
constexpr int C_AREA = 2 * C_BUF + 2 * AT_BN * 4;
constexpr int at_max(int a, int b) { return a > b ? a : b; }
constexpr int AT_AREA = at_max(C_AREA, at_max(AT_NBUF * 2 * T_BUF, AT_BM * K_PITCH));
// The exact phase's segment table (at most kMaxC (end, delta) pairs) sits
// after its two tile buffers.
constexpr int AT_TAB_OFF = AT_NBUF * 2 * T_BUF;
constexpr int AT_JOB_OFF = at_max(AT_AREA, AT_TAB_OFF + kMaxC * 8);
constexpr int AT_LDS = AT_JOB_OFF + 16;   // + job slot
static_assert(AT_LDS <= 160 * 1024, "LDS of one workgroup");
static_assert(kAttnSlots >= 1, "row-list slots");
static_assert(AT_BM == kAttnRows, "tile rows as sized in the workspace layout");
constexpr int AT_XCD = 8;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS chunk position of 16-B chunk c of tile row r (an involution in c).
__device__ __forceinline__ int k_pos(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int v_pos(int r, int c) { return c ^ ((r & 3) << 2); }

// ----------------------------------------------------------------------------- prep kernels

// k-bar split into bf16 hi/lo planes, v-bar rounded to bf16; ln m_g in base-2
// units (-inf if empty).
__global__ void k_comp_planes(const float* __restrict__ kbar, const float* __restrict__ vbar,
                              const int32_t* __restrict__ counts_k, int Ck, bf16* __restrict__ kbh,
                              bf16* __restrict__ kbl, bf16* __restrict__ vbh, float* __restrict__ logm2)
{
    const int g = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const size_t i = ((size_t)h * Ck + g) * AT_D + t;
    const float k = kbar[i], v = vbar[i];
    const bf16 kh = f32_to_bf16(k);
    kbh[i] = kh;
    kbl[i] = f32_to_bf16(k - bf16_to_f32(kh));
    vbh[i] = f32_to_bf16(v);
    if (t == 0) {
        const int m = counts_k[(size_t)h * Ck + g];
        logm2[(size_t)h * Ck + g] = m > 0 ? log2f((float)m) : -__builtin_inff();
    }
}

// Per (head, query cluster), in key-cluster order: the routed segments of every
// g with mask[c, g] = 1 and m_g > 0, as a table of (end, delta) pairs over the
// packed key list (list positions pref_s .. end_s - 1 hold the reordered key
// rows pref_s + delta_s .. end_s - 1 + delta_s of cluster s's segment), and the
// list of compensated clusters (mask = 0, m_g > 0); cinfo holds (routed keys,
// segments, compensated clusters).
__global__ __launch_bounds__(256) void k_seg_list(const uint8_t* __restrict__ mask,
                                                  const int32_t* __restrict__ offsets_k, int Cq,
                                                  int Ck, int2* __restrict__ segs,
                                                  int4* __restrict__ cinfo, int* __restrict__ comp)
{
    __shared__ int s_a[256], s_b[256];
    extern __shared__ int s_seg[];       // [Ck] first rows, [Ck + 1] key prefixes of routed segments
    int* const s_start = s_seg;
    int* const s_pref = s_seg + Ck;
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const uint8_t* mrow = mask + ((size_t)h * Cq + c) * Ck;
    const int32_t* ok = offsets_k + (size_t)h * (Ck + 1);
    int2* out = segs + ((size_t)h * Cq + c) * Ck;
    int* cout = comp + ((size_t)h * Cq + c) * Ck;
    int base = 0, cbase = 0;
    for (int g0 = 0; g0 < Ck; g0 += 256) {
        const int g = g0 + tid;
        int sel = 0, cmp = 0, start = 0, len = 0;
        if (g < Ck) {
            start = ok[g];
            len = ok[g + 1] - start;
            sel = mrow[g] && len > 0;
            cmp = !mrow[g] && len > 0;
        }
        s_a[tid] = sel;
        s_b[tid] = cmp;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int va = tid >= off ? s_a[tid - off] : 0;
            const int vb = tid >= off ? s_b[tid - off] : 0;
            __syncthreads();
            s_a[tid] += va;
            s_b[tid] += vb;
            __syncthreads();
        }
        if (sel) {
            const int si = base + s_a[tid] - 1;
            s_start[si] = start;
            s_pref[si] = len;
        }
        if (cmp) cout[cbase + s_b[tid] - 1] = g;
        base += s_a[255];
        cbase += s_b[255];
        __syncthreads();
    }
    // exclusive prefix of the segment lengths (contiguous runs per thread)
    const int per = (base + 255) / 256, s0 = tid * per;
    int run = 0;
    for (int k = 0; k < per && s0 + k < base; ++k) run += s_pref[s0 + k];
    s_a[tid] = run;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int v = tid >= off ? s_a[tid - off] : 0;
        __syncthreads();
        s_a[tid] += v;
        __syncthreads();
    }
    int acc = s_a[tid] - run;
    for (int k = 0; k < per && s0 + k < base; ++k) {
        const int len = s_pref[s0 + k];
        out[s0 + k] = make_int2(acc + len, s_start[s0 + k] - acc);
        acc += len;
    }
    if (tid == 0) cinfo[(size_t)h * Cq + c] = make_int4(s_a[255], base, cbase, 0);   // keys, segments, comp
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
        int v = (int)threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
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

// Work queues.  Query tiles are dealt to eight queues by query cluster
// (c mod 8), one per XCD: workgroup w starts on queue w mod 8, the XCD it is
// dispatched to, so the tiles of one cluster, which read the same keys, run
// together on one XCD and share its L2; within a queue tiles go head by head,
// so all XCDs work on the same few heads at a time.  A workgroup that finds
// its queue empty moves on to the next queue.
// Per head: tiles per class and the exclusive prefix of tiles within the class.
__global__ __launch_bounds__(256) void k_queue_count(const int* __restrict__ tstart, int Cq,
                                                     int* __restrict__ cnt, int* __restrict__ pre)
{
    __shared__ int s_part[256];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int x = tid >> 5, l = tid & 31;           // class x, 32 threads per class
    const int* ts = tstart + (size_t)h * (Cq + 1);
    const int nx = Cq > x ? (Cq - x + kXcd - 1) / kXcd : 0;  // members c = x + 8 q, q < nx
    const int per = (nx + 31) / 32;
    const int q0 = l * per;
    int local = 0;
    for (int k = 0; k < per; ++k) {
        const int q = q0 + k;
        if (q < nx) {
            const int c = x + kXcd * q;
            local += ts[c + 1] - ts[c];
        }
    }
    s_part[tid] = local;
    __syncthreads();
    for (int off = 1; off < 32; off <<= 1) {
        const int v = l >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += v;
        __syncthreads();
    }
    int run = s_part[tid] - local;
    for (int k = 0; k < per; ++k) {
        const int q = q0 + k;
        if (q < nx) {
            const int c = x + kXcd * q;
            pre[(size_t)h * Cq + c] = run;
            run += ts[c + 1] - ts[c];
        }
    }
    if (l == 31) cnt[h * kXcd + x] = s_part[tid];
}

// Queue entries (logical tile h * tiles_per_head + tile-in-head), class-major,
// then head, cluster and tile; meta[x] = length of queue x, meta[8 + x] = its
// first entry.
__global__ __launch_bounds__(256) void k_queue_fill(const int* __restrict__ tstart,
                                                    const int* __restrict__ cnt,
                                                    const int* __restrict__ pre, int H, int Cq,
                                                    int tiles_per_head, int* __restrict__ meta,
                                                    int* __restrict__ list)
{
    __shared__ int s_base[kXcd];
    const int h = blockIdx.x, tid = threadIdx.x;
    if (tid < kXcd) {
        const int x = tid;
        int start = 0, off = 0, tot = 0;
        for (int y = 0; y < x; ++y)
            for (int g = 0; g < H; ++g) start += cnt[g * kXcd + y];
        for (int g = 0; g < H; ++g) {
            if (g < h) off += cnt[g * kXcd + x];
            tot += cnt[g * kXcd + x];
        }
        s_base[x] = start + off;
        if (h == 0) {
            meta[x] = tot;
            meta[kXcd + x] = start;
        }
    }
    __syncthreads();
    const int* ts = tstart + (size_t)h * (Cq + 1);
    for (int c = tid; c < Cq; c += 256) {
        const int base = s_base[c % kXcd] + pre[(size_t)h * Cq + c];
        for (int t = ts[c]; t < ts[c + 1]; ++t) list[base + (t - ts[c])] = h * tiles_per_head + t;
    }
}

// ----------------------------------------------------------------------------- per-tile math

struct Softmax {
    float m;        // running max of the base-2 logits, shared by both half-waves
    float l;        // this half-wave's partial sum of probabilities
    f32x16_t o[4];  // O^T blocks: d rows 32 db + ..., query column lane & 31
};

// acc (+)= K Q^T for a 64-key tile: two 32x32 blocks, the two accumulation
// chains interleaved and the fragment reads scheduled two steps ahead.
__device__ __forceinline__ void tile_scores(f32x16_t acc[2], const char* kbuf, const bf16x8_t qf[8],
                                            int lane)
{
    __builtin_amdgcn_s_setprio(1);
    const int row = lane & 31, half = lane >> 5;
    const char* kr0 = kbuf + row * ROW_B;
    const char* kr1 = kr0 + 32 * ROW_B;   // row + 32: same swizzle
    f32x16_t a0 = acc[0], a1 = acc[1];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int off = k_pos(row, 2 * s + half) * 16;
        const bf16x8_t k0 = as_bf16x8(*(const u32x4_t*)(kr0 + off));
        const bf16x8_t k1 = as_bf16x8(*(const u32x4_t*)(kr1 + off));
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], a1, 0, 0, 0);
    }
    // pipeline: 6 reads up front, then (2 MFMA, 2 reads) x 5, then 6 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    acc[0] = a0;
    acc[1] = a1;
    __builtin_amdgcn_s_setprio(0);
}

// Lane l and lane l ^ 32 hold the two halves of one query column: after
// v_permlane32_swap the pair of results is {own value, partner's value} in
// every lane, so symmetric combinations need no LDS round trip.
__device__ __forceinline__ float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online softmax with raw scores x (logit = x * scale2 + bias, base 2) against
// a lazily raised reference max st.m: O and l are rescaled only when some
// lane's tile max exceeds the reference by more than kLazy, so the weights
// stay at most 2^kLazy.  O and l always share one reference, so the final
// O / l is unchanged, and bf16 and fp32 keep their relative precision at any
// such magnitude.  The normaliser sums the bf16-rounded weights that the PV
// product uses (v_dot2 against ones).  Returns the weights as PV B-operand
// fragments pf[kb * 2 + ks].
constexpr float kLazy = 8.f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void softmax_update(Softmax& st, const f32x16_t x[2], float scale2,
                                               bf16x8_t pf[4])
{
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[kb][i]);
    mloc = pair_max(mloc) * scale2;
    if (__any(mloc > st.m + kLazy)) {
        const float mnew = fmaxf(st.m, mloc);
        const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);   // 0 while st.m = -inf
        st.l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) st.o[db] *= alpha;
        st.m = mnew;
    }
    const float muse = st.m == -__builtin_inff() ? 0.f : st.m;
    const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    float sum = st.l;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8_t f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                f[i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(x[kb][8 * ks + i], scale2, -muse));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{f[2 * j], f[2 * j + 1]}, one, sum, false);
            pf[kb * 2 + ks] = f;
        }
    }
    st.l = sum;
}

// O^T += V^T P^T for one 64-key tile held row-major in vbuf (transpose loads),
// the transpose reads scheduled ahead of the MFMAs.
__device__ __forceinline__ void tile_pv(Softmax& st, const char* vbuf, const bf16x8_t pf[4], int lane)
{
    __builtin_amdgcn_s_setprio(1);
    const int j = lane & 15, grp = lane >> 4;
    const int half = grp >> 1;
    // row 4 half + j / 4 (+16 kk, +8 for the second load), column 16 (grp & 1) + 4 (j & 3)
    // + 32 db elements: chunk 2 (grp & 1) + (j & 3) / 2 + 4 db, whose swizzled
    // position is the same chunk with db replaced by db ^ ((j >> 2) & 3).
    const int jr = (j >> 2) & 3;
    const char* base = vbuf + (4 * half + (j >> 2)) * ROW_B + (2 * (grp & 1) + ((j >> 1) & 1)) * 16 + (j & 1) * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const char* a = base + (16 * kk) * ROW_B + (db ^ jr) * 64;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a);
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a + 8 * ROW_B));
            const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
            const bf16x8_t vf = as_bf16x8(u32x4_t{l2[0], l2[1], h2[0], h2[1]});
            st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], st.o[db], 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int s = 0; s < 13; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_s_setprio(0);
}

// softmax_update and tile_pv fused, with the same arithmetic in the same
// order: the weights of keys 16 kk .. 16 kk + 15 are formed while the MFMAs
// of the previous 16 keys run, and the transpose reads of each k-step are
// issued one step ahead, so the exponentials overlap the matrix work of the
// same wave instead of preceding it.
__device__ __forceinline__ void softmax_pv(Softmax& st, const f32x16_t x[2], float scale2, const char* vbuf,
                                           int lane)
{
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[kb][i]);
    mloc = pair_max(mloc) * scale2;
    if (__any(mloc > st.m + kLazy)) {
        const float mnew = fmaxf(st.m, mloc);
        const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);   // 0 while st.m = -inf
        st.l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) st.o[db] *= alpha;
        st.m = mnew;
    }
    const float muse = st.m == -__builtin_inff() ? 0.f : st.m;
    const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    float sum = st.l;
    // the V^T fragments as in tile_pv
    const int j = lane & 15, grp = lane >> 4;
    const int half = grp >> 1;
    const int jr = (j >> 2) & 3;
    const char* base = vbuf + (4 * half + (j >> 2)) * ROW_B + (2 * (grp & 1) + ((j >> 1) & 1)) * 16 + (j & 1) * 8;
    auto vfrag = [&](int kk, int db) {
        const char* a = base + (16 * kk) * ROW_B + (db ^ jr) * 64;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a + 8 * ROW_B));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        return as_bf16x8(u32x4_t{l2[0], l2[1], h2[0], h2[1]});
    };
    // weights of keys 16 kk + 2 pr, + 1 (pr = 0..3), packed into f
    auto weights2 = [&](int kk, int pr, bf16x8_t& f) {
        const int kb = kk >> 1, ks = kk & 1;
#pragma unroll
        for (int i = 2 * pr; i < 2 * pr + 2; ++i)
            f[i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(x[kb][8 * ks + i], scale2, -muse));
        sum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{f[2 * pr], f[2 * pr + 1]}, one, sum, false);
        asm volatile("" : "+v"(sum));   // keeps the sum's step in its slot of the schedule
    };
    __builtin_amdgcn_s_setprio(1);
    bf16x8_t vf[2][4];
    bf16x8_t pf[2];
#pragma unroll
    for (int db = 0; db < 4; ++db) vf[0][db] = vfrag(0, db);
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) weights2(0, pr, pf[0]);
    __builtin_amdgcn_sched_barrier(0);
    // step kk: each MFMA is followed by the reads of one fragment of step
    // kk + 1 and a quarter of its weights; the order is pinned so that the
    // exponentials issue while the MFMA before them runs
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk & 1][db], pf[kk & 1], st.o[db], 0, 0, 0);
            if (kk + 1 < 4) {
                vf[(kk + 1) & 1][db] = vfrag(kk + 1, db);
                weights2(kk + 1, db, pf[(kk + 1) & 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    st.l = sum;
    __builtin_amdgcn_s_setprio(0);
}

// Tile rows past nvalid get -inf.  Row kb 32 + 8 (i / 4) + 4 half + i % 4 is
// compared as the constant kb 32 + 8 (i / 4) + i % 4 against nvalid - 4 half
// (no per-row index registers).
__device__ __forceinline__ void mask_rows(f32x16_t x[2], int nvalid, int half)
{
    const int lim = nvalid - 4 * half;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kt = kb * 32 + (i >> 2) * 8 + (i & 3);
            x[kb][i] = kt < lim ? x[kb][i] : -__builtin_inff();
        }
}

// ----------------------------------------------------------------------------- exact tiles

typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup barrier without the LDS release fence of __syncthreads (which
// would also wait for every load-to-LDS still in flight, including the tiles
// requested for later steps).  Every wave has already waited for its own loads
// of the tile the barrier publishes, and all reads of the tile being retired
// fed MFMAs before the barrier; the empty asm statements and the scheduling
// barriers keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void tile_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

constexpr int FILL_ROWS = AT_BN / AT_WAVES;   // tile rows each wave fills
constexpr int FILL_N = FILL_ROWS / 4;          // 4-row instructions per operand and wave

// Fill tile buffer b (K rows at b, V rows at b + T_BUF): wave w writes rows
// FILL_ROWS w .. FILL_ROWS (w + 1) - 1, one 4-row instruction per operand and
// step; lane l writes LDS chunk l & 15 of its row and so reads the global
// chunk that the swizzle places there.
__device__ __forceinline__ void tile_fill(char* b, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int wv, const int r[FILL_N], const int kx[FILL_N], int vx)
{
    char* kb = b + FILL_ROWS * wv * ROW_B;
    char* vb = b + T_BUF + FILL_ROWS * wv * ROW_B;
#pragma unroll
    for (int i = 0; i < FILL_N; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(kb + 4 * i * ROW_B), 16, r[i] * ROW_B + kx[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < FILL_N; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(vb + 4 * i * ROW_B), 16, r[i] * ROW_B + vx, 0, 0, 0);
}

// Row list: the packed routed-key list of one (head, query cluster), list
// position -> reordered key row, written by the whole workgroup into its own
// slot of device memory from the segment table tab (in LDS, ns entries
// (end_s, delta_s): positions end_{s-1} .. end_s - 1 hold rows position +
// delta_s).  Wave w writes segments w, w + 8, ..., its lanes consecutive
// positions of the segment, so every store is coalesced.
__device__ __forceinline__ void row_list(int* __restrict__ w, const int2* __restrict__ tab, int ns)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int s = wave; s < ns; s += AT_WAVES) {
        const int2 e = tab[s];
        const int begin = s > 0 ? tab[s - 1].x : 0;
        for (int q = begin + lane; q < e.x; q += 64) w[q] = q + e.y;
    }
}

// The exact tiles of one query tile: the routed keys, rows rm[0 .. nk), in
// 64-key tiles through two LDS buffers.  Each step requests the row indices of
// tile t + 2, then the rows of tile t + 1 straight into the other buffer, then
// computes tile t; the loads land during the math.  The two buffers and
// the row list are distinct restrict-qualified pointers and the loop is
// unrolled by two, so the compiler sees that the loads in flight never alias
// the buffer being read and adds no wait of its own before the reads; the
// explicit wait before each barrier covers this wave's loads and the barrier
// publishes every wave's rows.  Loads past the last tile use clamped rows into
// a buffer no one reads; all loads drain before returning.
__device__ __forceinline__ void exact_tiles(char* __restrict__ b0, char* __restrict__ b1, Softmax& st,
                                            const bf16x8_t qf[8], __amdgpu_buffer_rsrc_t rk,
                                            __amdgpu_buffer_rsrc_t rv, const int* __restrict__ rm, int nk,
                                            int wave, int lane, bool wact, float scale2)
{
    const int ntiles = (nk + AT_BN - 1) / AT_BN;
    const int half = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lr = FILL_ROWS * wv + (lane >> 4), p = lane & 15;
    int kx[FILL_N];
#pragma unroll
    for (int i = 0; i < FILL_N; ++i) kx[i] = k_pos(lr + 4 * i, p) * 16;
    const int vx = v_pos(lr, p) * 16;   // rows lr + 4 i share it
    int ra[FILL_N], rb[FILL_N];
#define ROWS(SET, T)                                                                          \
    _Pragma("unroll") for (int i = 0; i < FILL_N; ++i)                                        \
        SET[i] = rm[min((T) * AT_BN + lr + 4 * i, nk - 1)];
    ROWS(ra, 0)
    ROWS(rb, 1)
    tile_fill(b0, rk, rv, wv, ra, kx, vx);
    __builtin_amdgcn_s_waitcnt(0x0F70 | 0);
    tile_barrier();
#define EXACT_STEP(T, CUR, NXT, RT, RN)                                                       \
    {                                                                                         \
        ROWS(RT, (T) + 2)                /* rows of tile T + 2 (set of tile T, now free) */   \
        tile_fill(NXT, rk, rv, wv, RN, kx, vx);   /* tile T + 1 */                            \
        if (wact && (T) < ntiles) {                                                           \
            f32x16_t acc[2] = {f32x16_t{0}, f32x16_t{0}};                                     \
            tile_scores(acc, CUR, qf, lane);                                                  \
            const int nvalid = nk - (T) * AT_BN;                                              \
            if (nvalid < AT_BN) mask_rows(acc, nvalid, half);                                 \
            softmax_pv(st, acc, scale2, CUR + T_BUF, lane);                                   \
        }                                                                                     \
        __builtin_amdgcn_s_waitcnt(0x0F70 | 0);   /* tile T + 1 landed */                     \
        tile_barrier();                                                                       \
    }
    for (int t = 0; t < ntiles; t += 2) {
        EXACT_STEP(t, b0, b1, ra, rb)
        EXACT_STEP(t + 1, b1, b0, rb, ra)
    }
#undef EXACT_STEP
#undef ROWS
}

// ----------------------------------------------------------------------------- compensation tiles

// The compensation tiles of one query tile: the key clusters skipped for this
// query cluster and non-empty (packed list cl, nc entries), 64 per tile.  A
// tile holds the bf16 hi and lo planes of k-bar, v-bar in bf16, and the
// biases log2 m_g of its centroids; like the exact tiles, its rows are gathered by index
// straight into LDS (the bias with one dword load per lane, by wave 0), two
// buffers deep, the next tile's loads in flight during the current tile's math.
__device__ __forceinline__ void comp_fill(char* b, float* bias, __amdgpu_buffer_rsrc_t rkh,
                                          __amdgpu_buffer_rsrc_t rkl, __amdgpu_buffer_rsrc_t rvh,
                                          __amdgpu_buffer_rsrc_t rlm, int wv,
                                          const int r[FILL_N], int br, const int kx[FILL_N], int vx)
{
    char* kh = b + FILL_ROWS * wv * ROW_B;
#pragma unroll
    for (int i = 0; i < FILL_N; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rkh, (lds_ptr)(kh + 4 * i * ROW_B), 16, r[i] * ROW_B + kx[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rkl, (lds_ptr)(kh + T_BUF + 4 * i * ROW_B), 16, r[i] * ROW_B + kx[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < FILL_N; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvh, (lds_ptr)(kh + 2 * T_BUF + 4 * i * ROW_B), 16, r[i] * ROW_B + vx, 0, 0, 0);
    }
    if (wv == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rlm, (lds_ptr)bias, 4, br * 4, 0, 0, 0);
}

__device__ __forceinline__ void comp_tiles(char* __restrict__ c0, char* __restrict__ c1, float* __restrict__ bias0,
                                           float* __restrict__ bias1, Softmax& st, const bf16x8_t qf[8],
                                           __amdgpu_buffer_rsrc_t rkh, __amdgpu_buffer_rsrc_t rkl,
                                           __amdgpu_buffer_rsrc_t rvh,
                                           __amdgpu_buffer_rsrc_t rlm, const int* __restrict__ cl, int nc,
                                           int wave, int lane, bool wact, float scale2)
{
    const int ntiles = (nc + AT_BN - 1) / AT_BN;
    const int half = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lr = FILL_ROWS * wv + (lane >> 4), p = lane & 15;
    int kx[FILL_N];
#pragma unroll
    for (int i = 0; i < FILL_N; ++i) kx[i] = k_pos(lr + 4 * i, p) * 16;
    const int vx = v_pos(lr, p) * 16;   // rows lr + 4 i share it
    int ra[FILL_N], rb[FILL_N], ba, bb;
#define CROWS(SET, B, T)                                                                      \
    _Pragma("unroll") for (int i = 0; i < FILL_N; ++i)                                        \
        SET[i] = cl[min((T) * AT_BN + lr + 4 * i, nc - 1)];                                   \
    B = cl[min((T) * AT_BN + lane, nc - 1)];
    CROWS(ra, ba, 0)
    CROWS(rb, bb, 1)
    comp_fill(c0, bias0, rkh, rkl, rvh, rlm, wv, ra, ba, kx, vx);
    __builtin_amdgcn_s_waitcnt(0x0F70 | 0);
    tile_barrier();
#define COMP_STEP(T, CUR, NXT, BCUR, BNXT, RT, BT, RN, BN)                                    \
    {                                                                                         \
        CROWS(RT, BT, (T) + 2)           /* rows of tile T + 2 (set of tile T, now free) */   \
        comp_fill(NXT, BNXT, rkh, rkl, rvh, rlm, wv, RN, BN, kx, vx);   /* tile T + 1 */      \
        if (wact && (T) < ntiles) {                                                           \
            f32x16_t acc[2] = {f32x16_t{0}, f32x16_t{0}};                                     \
            tile_scores(acc, CUR, qf, lane);                                                  \
            tile_scores(acc, CUR + T_BUF, qf, lane);                                          \
            /* logit = acc * scale2 + bias: fold the bias in as acc + bias / scale2 */        \
            _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                  \
                _Pragma("unroll") for (int i = 0; i < 16; ++i) {                              \
                    const int kt = kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);               \
                    acc[kb][i] = fmaf(BCUR[kt], 1.0f / scale2, acc[kb][i]);                   \
                }                                                                             \
            const int nvalid = nc - (T) * AT_BN;                                              \
            if (nvalid < AT_BN) mask_rows(acc, nvalid, half);                                 \
            softmax_pv(st, acc, scale2, CUR + 2 * T_BUF, lane);                               \
        }                                                                                     \
        __builtin_amdgcn_s_waitcnt(0x0F70 | 0);   /* tile T + 1 and rows of T + 2 landed */   \
        tile_barrier();                                                                       \
    }
    for (int t = 0; t < ntiles; t += 2) {
        COMP_STEP(t, c0, c1, bias0, bias1, ra, ba, rb, bb)
        COMP_STEP(t + 1, c1, c0, bias1, bias0, rb, bb, ra, ba)
    }
#undef COMP_STEP
#undef CROWS
}

// ----------------------------------------------------------------------------- main kernel

#define KBUF(b) (smem + (b) * 2 * T_BUF)
#define VBUF(b) (smem + (b) * 2 * T_BUF + T_BUF)

// One query tile: logical index h * tiles_per_head + tile-in-head.
__device__ __forceinline__ void attn_tile(
    int logical, char* smem, const bf16* __restrict__ Qp,
    const int32_t* __restrict__ offsets_q, const int32_t* __restrict__ perm_q,
    const bf16* __restrict__ Kp, const bf16* __restrict__ Vp, const bf16* __restrict__ kbh,
    const bf16* __restrict__ kbl, const bf16* __restrict__ vbh,
    const float* __restrict__ logm2, const int2* __restrict__ segs, const int4* __restrict__ cinfo,
    const int* __restrict__ comp, const int* __restrict__ tstart, int* __restrict__ rows, int Nq,
    int Nk, int Cq, int Ck, int tiles_per_head, float scale2, bf16* __restrict__ O)
{
    const int h = logical / tiles_per_head, t = logical - h * tiles_per_head;
    const int* ts = tstart + (size_t)h * (Cq + 1);
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
    const bool wact = wave * 32 < nrows;  // waves whose 32 query rows are all padding skip the math

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

    const size_t hc = (size_t)h * Cq + c;
    const float* lm = logm2 + (size_t)h * Ck;
    const int4 ci = cinfo[hc];   // (routed keys, segments, compensated clusters)

    // 1. compensation tiles: packed list of skipped non-empty key clusters
    const int nc = ci.z;
    if (nc > 0) {
        const size_t pb = (size_t)h * Ck * AT_D;
        const int plane_bytes = Ck * AT_D * 2;
        const __amdgpu_buffer_rsrc_t rkh = __builtin_amdgcn_make_buffer_rsrc((void*)(kbh + pb), (short)0, plane_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rkl = __builtin_amdgcn_make_buffer_rsrc((void*)(kbl + pb), (short)0, plane_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rvh = __builtin_amdgcn_make_buffer_rsrc((void*)(vbh + pb), (short)0, plane_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rlm = __builtin_amdgcn_make_buffer_rsrc((void*)lm, (short)0, Ck * 4, 0x00020000);
        float* const cb = (float*)(smem + 2 * C_BUF);
        comp_tiles(smem, smem + C_BUF, cb, cb + AT_BN, st, qf, rkh, rkl, rvh, rlm, comp + hc * Ck, nc, wave,
                   lane, wact, scale2);
    }

    // 2. exact tiles (packed routed keys); their row window uses the LDS half
    // that the exact tiles leave free (the compensation tiles, which use it, are
    // done: their last step ended in a barrier)
    const int nk = ci.x;
    if (nk > 0) {
        const size_t head_bytes = (size_t)Nk * AT_D * 2;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Kp + (size_t)h * Nk * AT_D), (short)0, (int)head_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Vp + (size_t)h * Nk * AT_D), (short)0, (int)head_bytes, 0x00020000);
        const int ns = ci.y;
        int2* const tab = (int2*)(smem + AT_TAB_OFF);
        const int2* sgh = segs + hc * Ck;
        for (int k = tid; k < ns; k += AT_THREADS) tab[k] = sgh[k];
        __syncthreads();
        row_list(rows, tab, ns);
        __syncthreads();   // the slot's rows are visible to every wave of the workgroup
        exact_tiles(KBUF(0), KBUF(1), st, qf, rk, rv, rows, nk, wave, lane, wact, scale2);
    }

    // 3. normalise, stage the tile in LDS as [query][d], store rows in token order
    const float ltot = pair_sum(st.l);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    __syncthreads();
    char* ost = smem;  // AT_BM rows x K_PITCH bytes
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

// planes: the k-bar hi, k-bar lo and v-bar planes, [H, Ck, d] bf16 each,
// one after another; qmeta: the work-queue region (lengths, starts, counters,
// per-head counts and prefixes, then the queue itself).
__global__ __launch_bounds__(AT_THREADS, 2) void k_attn_mfma(
    const bf16* __restrict__ Qp, const int32_t* __restrict__ offsets_q,
    const int32_t* __restrict__ perm_q, const bf16* __restrict__ Kp, const bf16* __restrict__ Vp,
    const bf16* __restrict__ planes, const float* __restrict__ logm2, const int2* __restrict__ segs,
    const int4* __restrict__ cinfo, const int* __restrict__ comp, const int* __restrict__ tstart,
    int* __restrict__ qmeta, int* __restrict__ rowbuf, int H, int Nq, int Nk, int Cq, int Ck,
    int tiles_per_head, float scale2, bf16* __restrict__ O)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    int* const s_job = (int*)(smem + AT_JOB_OFF);
    const size_t plane = (size_t)H * Ck * AT_D;
    const bf16* const kbh = planes;
    const bf16* const kbl = planes + plane;
    const bf16* const vbh = planes + 2 * plane;
    int* const qctr = qmeta + 2 * AT_XCD;
    const int* const qlist = qmeta + 3 * AT_XCD + (size_t)H * AT_XCD + (size_t)H * Cq;

    const int x0 = blockIdx.x % AT_XCD;
    for (int k = 0; k < AT_XCD; ++k) {
        const int x = (x0 + k) % AT_XCD;
        const int qlen = qmeta[x], qstart = qmeta[AT_XCD + x];
        for (;;) {
            __syncthreads();  // the previous tile is done with LDS (s_job included)
            if (threadIdx.x == 0) *s_job = atomicAdd(qctr + x, 1);
            __syncthreads();
            const int j = *s_job;
            if (j >= qlen) break;
            attn_tile(qlist[qstart + j], smem, Qp, offsets_q, perm_q, Kp, Vp, kbh, kbl,
                      vbh, logm2, segs, cinfo, comp, tstart, rowbuf + (size_t)blockIdx.x * Nk, Nq,
                      Nk, Cq, Ck, tiles_per_head, scale2, O);
        }
    }
}
#undef KBUF
#undef VBUF

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
    float* logm2 = (float*)(s + L.at_logm);
    int* tstart = (int*)(s + L.at_tiles);
    int2* segs = (int2*)(s + L.at_segs);
    int4* cinfo = (int4*)(s + L.at_cinfo);
    int* comp = (int*)(s + L.at_comp);
    hipLaunchKernelGGL(k_comp_planes, dim3(a.Ck, a.H), dim3(AT_D), 0, st, a.kbar, a.vbar, a.counts_k,
                       a.Ck, kbh, kbl, vbh, logm2);
    hipLaunchKernelGGL(k_seg_list, dim3(a.Cq, a.H), dim3(256), (2 * a.Ck + 1) * 4, st, a.mask, a.offsets_k, a.Cq,
                       a.Ck, segs, cinfo, comp);
    hipLaunchKernelGGL(k_tile_prefix, dim3(a.H), dim3(1024), 0, st, a.offsets_q, a.Cq, tstart);
    const int tiles_per_head = (a.Nq + AT_BM - 1) / AT_BM + a.Cq;
    int* qmeta = (int*)(s + L.at_queue);       // [8] lengths, [8] starts, [8] counters
    int* qcnt = qmeta + 3 * AT_XCD;            // [H][8]
    int* qpre = qcnt + (size_t)a.H * AT_XCD;   // [H][Cq]
    int* qlist = qpre + (size_t)a.H * a.Cq;    // [total tiles]
    hipLaunchKernelGGL(k_queue_count, dim3(a.H), dim3(256), 0, st, tstart, a.Cq, qcnt, qpre);
    hipLaunchKernelGGL(k_queue_fill, dim3(a.H), dim3(256), 0, st, tstart, qcnt, qpre, a.H, a.Cq,
                       tiles_per_head, qmeta, qlist);
    zero_words(qmeta + 2 * AT_XCD, AT_XCD * 4, st);
    // persistent: one workgroup per CU (two waves per SIMD, the occupancy the register use allows)
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        ncu = 0;
    // one 8-wave workgroup per CU (two waves per SIMD), each with its own row-list slot
    const int nwg = ncu > 0 && ncu < kAttnSlots ? ncu : kAttnSlots;
    const float scale2 = (float)(1.4426950408889634 / sqrt((double)AT_D));
    hipLaunchKernelGGL(k_attn_mfma, dim3(nwg), dim3(AT_THREADS), AT_LDS, st,
                       (const bf16*)a.Qp, a.offsets_q, a.perm_q, (const bf16*)a.Kp,
                       (const bf16*)a.Vp, (const bf16*)kbh, logm2, segs, (const int4*)cinfo, comp, tstart,
                       qmeta, (int*)(s + L.at_rows), a.H, a.Nq, a.Nk, a.Cq, a.Ck, tiles_per_head, scale2,
                       (bf16*)a.O);
    return hipGetLastError();
}

}  // namespace svg
