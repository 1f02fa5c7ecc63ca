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
// to its centroid in every coordinate is treated as D = 0 exactly.  The estimate
//     e = e^{2s} [expm1(D)^2 ||vbar_g||^2 + 2 expm1(D) vbar_g.delta_j + ||delta_j||^2]
//       = || e^{sbar} vbar_g - e^{s} v_j ||^2,
// s = sbar - D, delta_j = vbar_g - v_j, is evaluated with the larger of the two
// exponentials factored out, e = e^{2 sbar} e^{2 max(-D, 0)} f, f a quadratic in
// expm1(-|D|) with per-key coefficients (so f never overflows); sum_j
// e^{2 max(-D, 0)} f is accumulated per (c, g) against a shift that moves only
// when some exponent outgrows it by 2^64.
//
// Work split: a workgroup (4 waves) walks its key clusters in chunks of 64
// keys.  The K and V rows of a chunk go straight from device memory into one of
// two LDS buffers (the next chunk's loads land during the current chunk's math);
// the K rows are the MFMA A operand, and from the V rows the threads form the
// per-key scalars vbar.delta_j and ||delta_j||^2 (16 lanes per row, DPP sums),
// so K_p and V_p are each read once by the whole probe.  Wave w owns the query-centroid column blocks
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kShiftStep = 64.f;          // log2 headroom before the shift moves

__device__ __forceinline__ bf16x8_t pr_as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// expm1(-x) for x >= 0, given w = e^{-x}: x^2 / 2 - x for x < 2^-8 (the
// truncation, below x^3 / 6, is under 2^-17 relative), w - 1 elsewhere (the
// rounding of w, 2^-24, is then at most 2^-16 of |w - 1|).
__device__ __forceinline__ float expm1_nonpos(float x, float w)
{
    return x < 0x1p-8f ? fmaf(0.5f * x, x, -x) : w - 1.f;
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

// Sum (bitwise or) over the 16 lanes of a row group (lanes 16 k .. 16 k + 15), left in every
// lane of the group: rotations by 8 and 4 within the row, then the two quad
// swaps, all as DPP moves (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ unsigned dppu(unsigned v)
{
    return (unsigned)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ unsigned or16(unsigned v)
{
    v |= dppu<0x128>(v);
    v |= dppu<0x124>(v);
    v |= dppu<0x4E>(v);
    v |= dppu<0xB1>(v);
    return v;
}
__device__ __forceinline__ float sum16(float v)
{
    v += dpp<0x128>(v);   // row_ror:8
    v += dpp<0x124>(v);   // row_ror:4
    v += dpp<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    return v;
}

// Chunk buffers (two): the K and V rows of 64 keys (256 B each, the 16-B chunk
// c of row r at position c ^ (r mod 16), so that the fragment reads of 16 rows
// at one chunk and the per-key reads of one row's 16 chunks are both free of
// bank conflicts), then, for the first chunk of a key cluster, k-bar and v-bar
// of the cluster (fp32) and the sbar column of the workgroup's query clusters.
constexpr int PR_T = PR_KC * 256;
constexpr int PR_KB = 2 * PR_T, PR_VB = PR_KB + PR_D * 4, PR_SB = PR_VB + PR_D * 4;
constexpr int PR_BUF = PR_SB + PR_MAXCQ * 4;
constexpr int PR_LDS2 = 2 * PR_BUF;   // plus the per-key rows, 1.3 KB

typedef __attribute__((address_space(3))) void* pr_lds_ptr;

// A workgroup barrier for LDS only: this wave's LDS accesses complete, then
// s_barrier (the memory clobber keeps the compiler from moving any access
// across it).  Unlike __syncthreads it does not wait for outstanding
// device-memory loads, so the next chunk's loads into LDS stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int pr_pos(int r, int c) { return c ^ (r & 15); }

// The chunk a workgroup works on: key cluster g of head h (g >= Ck: no work
// left), keys jc .. min(jc + 64, j1) - 1, j0 the cluster's first key.
struct PrChunk {
    int h, g, j0, jc, j1;
};

// Thread 0 only: the first non-empty key cluster from the claim g of head h on.
// A claim past the head's last cluster moves the workgroup to the next head
// (left counts the heads still to try); empty clusters get ln r = -inf.
__device__ __forceinline__ int4 pr_resolve(int g, int& h, int& left, int* __restrict__ ctr,
                                        const int32_t* __restrict__ offsets_k, int H, int Cq, int Ck,
                                        int c_lo, int c_hi, float* __restrict__ log_ratio)
{
    for (;;) {
        if (g < Ck) {
            const int32_t* ok = offsets_k + (size_t)h * (Ck + 1);
            const int j0 = ok[g], j1 = ok[g + 1];
            if (j1 > j0) return make_int4(h, g, j0, j1);
            for (int c = c_lo; c < c_hi; ++c) log_ratio[((size_t)h * Cq + c) * Ck + g] = -__builtin_inff();
        } else {
            if (--left <= 0) return make_int4(0, Ck, 0, 0);
            h = h + 1 == H ? 0 : h + 1;
        }
        g = atomicAdd(ctr + h, 1);
    }
}

// With one column block per wave the kernel fits three waves per SIMD by its
// registers, with two (the three bf16 planes of two blocks stay in registers)
// two; its LDS (two chunk buffers, 69 KB) allows two workgroups per CU.  A
// workgroup covers a slice of 4 NCBW column blocks (blockIdx.y); with more
// query clusters than one slice holds, the slices are separate workgroups over
// the same keys (the key-side loads are repeated per slice).
//
// Work distribution: one resident round of workgroups; the (head, key cluster)
// items are claimed at run time from one counter per head and slice.
// Workgroup w starts on head w H / G and, once that head's clusters are all
// claimed, moves on to the following heads, so every workgroup stays busy until
// the last cluster is claimed, whatever the cluster sizes.  Thread 0 claims the
// cluster after next while the current chunk is computed (the atomic is in
// flight during the math).
template <int NCBW, bool EPS>
__global__ __launch_bounds__(256, 2) void k_probe_mfma(
    const float* __restrict__ qbar, const int32_t* __restrict__ counts_q, const bf16* __restrict__ Kp,
    const bf16* __restrict__ Vp, const float* __restrict__ kbar, const float* __restrict__ vbar,
    const float* __restrict__ sbar, const int32_t* __restrict__ offsets_k, int H, int Nk, int Cq, int Ck,
    float tau, int logit_only, int* __restrict__ ctr, float* __restrict__ log_ratio,
    float* __restrict__ log_eps2)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // Per-key coefficients of the chunk's rows (see the pair loop) and the
    // claimed clusters, in arrays of their own: the compiler then knows that
    // writing them cannot touch the chunk buffers that loads are filling.
    __shared__ float4 s_ks[PR_KC];   // (alpha1, beta0, beta1, R)
    __shared__ float s_ka[PR_KC];    // alpha0
    __shared__ int4 s_item[2];       // [0] first cluster, [1] the next
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int col = lane & 15, grp = lane >> 4;   // A row / D column, and row group
    const int ncb = (Cq + 15) / 16;
    const int cbw = blockIdx.y * 4 * NCBW + wave;   // this wave's first column block
    const int c_lo = blockIdx.y * 4 * NCBW * 16, c_hi = min(Cq, c_lo + 4 * NCBW * 16);
    int* const ctr_s = ctr + (size_t)blockIdx.y * H;

    // B fragments of this wave's column blocks for head h: centroid cb*16 + col,
    // dims 32 ks + 8 grp + 0..7, split exactly into three bf16 planes.
    bf16x8_t bh[NCBW][4], bm[NCBW][4], bl[NCBW][4];
    bool qlive[NCBW];   // query cluster cb*16 + col is non-empty
    auto load_b = [&](int h) {
#pragma unroll
        for (int i = 0; i < NCBW; ++i) {
            const int c = (cbw + 4 * i) * 16 + col;
            const bool cv = c < Cq;
            qlive[i] = cv && counts_q[(size_t)h * Cq + c] > 0;
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
    };
    auto item = [&](int k) -> PrChunk {
        const int4 v = s_item[k];
        const int j0 = __builtin_amdgcn_readfirstlane(v.z);
        return PrChunk{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y), j0, j0,
                       __builtin_amdgcn_readfirstlane(v.w)};
    };

    // Loads of a chunk straight into LDS buffer b: wave w fills rows
    // 16 w .. 16 w + 15 of K and V (4 rows per instruction; rows past the
    // cluster repeat its last key); with the cluster's first chunk, waves 0-3
    // also fetch k-bar, v-bar and the sbar column.
    auto issue = [&](char* b, const PrChunk& it) {
        const int h = it.h;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Kp + (size_t)h * Nk * PR_D), (short)0, Nk * PR_D * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Vp + (size_t)h * Nk * PR_D), (short)0, Nk * PR_D * 2, 0x00020000);
        const int nv = min(PR_KC, it.j1 - it.jc);
        const int p = lane & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * wv + 4 * i + (lane >> 4);
            const int off = (it.jc + min(r, nv - 1)) * 256 + pr_pos(r, p) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (pr_lds_ptr)(b + (16 * wv + 4 * i) * 256), 16, off, 0, 0, 0);
            if (!logit_only)   // the logit-only estimate reads no values
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (pr_lds_ptr)(b + PR_T + (16 * wv + 4 * i) * 256), 16, off,
                                                         0, 0, 0);
        }
        if (it.jc == it.j0) {
            if (wv == 0 && lane < 32) {
                const __amdgpu_buffer_rsrc_t rkb = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(kbar + (size_t)h * Ck * PR_D), (short)0, Ck * PR_D * 4, 0x00020000);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rkb, (pr_lds_ptr)(b + PR_KB), 16, it.g * PR_D * 4 + lane * 16, 0, 0, 0);
            }
            if (wv == 1 && lane < 32) {
                const __amdgpu_buffer_rsrc_t rvb = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(vbar + (size_t)h * Ck * PR_D), (short)0, Ck * PR_D * 4, 0x00020000);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rvb, (pr_lds_ptr)(b + PR_VB), 16, it.g * PR_D * 4 + lane * 16, 0, 0, 0);
            }
            if (wv >= 2) {
                const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(sbar + (size_t)h * Cq * Ck), (short)0, Cq * Ck * 4, 0x00020000);
                const int c = c_lo + (wv - 2) * 64 + lane;
                const int cc = min(c, Cq - 1);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (pr_lds_ptr)(b + PR_SB + (wv - 2) * 256), 4,
                                                         (cc * Ck + it.g) * 4, 0, 0, 0);
            }
        }
    };

    // the first two clusters, claimed by thread 0 starting at the home head
    int hh = (int)(((long long)blockIdx.x * H) / gridDim.x), left = H, pend = 0;
    if (tid == 0) {
        const int4 a = pr_resolve(atomicAdd(ctr_s + hh, 1), hh, left, ctr_s, offsets_k, H, Cq, Ck, c_lo, c_hi,
                                  log_ratio);
        s_item[0] = a;
        s_item[1] = a.y < Ck ? pr_resolve(atomicAdd(ctr_s + hh, 1), hh, left, ctr_s, offsets_k, H, Cq, Ck, c_lo,
                                          c_hi, log_ratio)
                             : a;
    }
    __syncthreads();
    PrChunk cur = item(0);
    int bhead = -1;   // the head whose planes bh, bm, bl hold
    const int sch = tid & 15, srow = tid >> 4;   // per-key terms: dims 8 sch.., rows srow + 16 i
    float vb8[8], P = 0.f;
    unsigned kbw[4], kmw[4];   // k-bar as packed bf16 and the bits that decide equality
    float sb[NCBW], sh[NCBW], S[NCBW];
    if (cur.g < Ck) issue(smem, cur);
    int bsel = 0;
    while (cur.g < Ck) {
        char* const b = smem + bsel * PR_BUF;
        // This wave's loads of the current chunk have landed and its LDS
        // accesses (thread 0's claim above included) are complete -- the
        // barrier's own fence does not wait for the LDS write -- then every
        // wave's; the other buffer's readers are done.
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        __syncthreads();
        PrChunk nxt = cur;
        nxt.jc += PR_KC;
        bool took = false;   // the next cluster taken from s_item[1], which thread 0 refills
        if (nxt.jc >= nxt.j1) {
            nxt = item(1);
            took = nxt.g < Ck;
        }
        if (took && tid == 0) pend = atomicAdd(ctr_s + hh, 1);
        if (nxt.g < Ck) issue(smem + (bsel ^ 1) * PR_BUF, nxt);   // lands during this chunk's math

        const int nv = min(PR_KC, cur.j1 - cur.jc);
        const int h = cur.h;
        if (cur.jc == cur.j0) {   // a new cluster: its centroids, P = ||vbar||^2, sbar; sums restart
            if (h != bhead) {     // (and a new head: its query-centroid planes)
                load_b(h);
                bhead = h;
            }
            const float* kbl = (const float*)(b + PR_KB) + 8 * sch;
            const float* vbl = (const float*)(b + PR_VB) + 8 * sch;
#pragma unroll
            for (int e = 0; e < 8; ++e) vb8[e] = logit_only ? 0.f : vbl[e];
            // A key (bf16) equals k-bar only where every coordinate of k-bar is a
            // bf16 value; then the packed words are compared, the sign of a
            // zero ignored.  Otherwise the pattern is a NaN no finite key holds.
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const unsigned lo = __float_as_uint(kbl[2 * w]), hi = __float_as_uint(kbl[2 * w + 1]);
                const bool rep = ((lo | hi) & 0xFFFFu) == 0;
                kbw[w] = rep ? (lo >> 16) | hi : 0x7FC07FC0u;
                kmw[w] = ((lo & 0x7FFFFFFFu) == 0 ? 0x7FFFu : 0xFFFFu) |
                         ((hi & 0x7FFFFFFFu) == 0 ? 0x7FFF0000u : 0xFFFF0000u);
            }
            P = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) P = fmaf(vb8[e], vb8[e], P);
            P = logit_only ? 1.f : sum16(P);
            const float* sbl = (const float*)(b + PR_SB);
#pragma unroll
            for (int i = 0; i < NCBW; ++i) {
                const int c = (cbw + 4 * i) * 16 + col;
                sb[i] = c < Cq ? sbl[c - c_lo] : 0.f;
                sh[i] = 0.f;
                S[i] = 0.f;
            }
        }
        // Per-key coefficients from the LDS rows, delta = vbar - v_j:
        //   R = ||delta||^2, beta0 = 2 vbar.delta, alpha0 = ||vbar||^2,
        //   beta1 = 2 (R - vbar.delta) = -2 delta.v_j, alpha1 = ||v_j||^2 = alpha0 - beta0 + R;
        // a key equal to its centroid keeps only R (its D is exactly zero), and
        // rows past the chunk's keys are all zero.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = srow + 16 * i;
            const u32x4_t kw = *(const u32x4_t*)(b + r * 256 + pr_pos(r, sch) * 16);
            const u32x4_t vw = *(const u32x4_t*)(b + PR_T + r * 256 + pr_pos(r, sch) * 16);
            float qd = 0.f, rr = 0.f;
            unsigned ne = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) ne |= (kw[w] ^ kbw[w]) & kmw[w];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned vb = (e & 1) ? (vw[e >> 1] & 0xFFFF0000u) : (vw[e >> 1] << 16);
                const float dl = vb8[e] - __uint_as_float(vb);
                qd = fmaf(vb8[e], dl, qd);
                rr = fmaf(dl, dl, rr);
            }
            // (the logit-only estimate loads no values: vbar = e_1 and delta = 0)
            qd = sum16(qd);
            rr = sum16(rr);
            ne = or16(ne);
            if (logit_only) qd = rr = 0.f;
            if (sch == 0) {
                const bool live = r < nv, moved = ne != 0;
                const float b0 = 2.f * qd;
                s_ks[r] = live ? make_float4(moved ? fmaxf(P - b0 + rr, 0.f) : 0.f, moved ? b0 : 0.f,
                                             moved ? 2.f * rr - b0 : 0.f, rr)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
                s_ka[r] = live && moved ? P : 0.f;
            }
        }
        lds_barrier();

        const int ntile = (nv + 15) / 16;
        for (int kt = 0; kt < ntile; ++kt) {
            bf16x8_t ak[4];
            const int arow = kt * 16 + col;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                ak[ks] = pr_as_bf16x8(*(const u32x4_t*)(b + arow * 256 + pr_pos(arow, 4 * ks + grp) * 16));
            const int kr0 = kt * 16 + 4 * grp;   // this lane's rows kr0 .. kr0 + 3
            float4 kq[4];
            float ka[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                kq[r] = s_ks[kr0 + r];
                ka[r] = s_ka[kr0 + r];
            }
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
                // Per pair, D = sbar - s and em = expm1(-|D|):
                //   D <= 0:  e = e^{2 s}    ||delta + em vbar||^2  = e^{2 sbar} e^{-2D} f,
                //   D > 0:   e = e^{2 sbar} ||delta - em v_j||^2   = e^{2 sbar} f,
                // f = (alpha em + beta) em + R with (alpha, beta) = (alpha0, beta0)
                // or (alpha1, beta1): the larger exponential is factored out, so
                // nothing overflows however far the key lies from its centroid.
                // S sums f e^{u} with u = log2 e^{2 max(-D, 0)} - sh.
                float f[4], u[4];
                float umax = -__builtin_inff();
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float D = fmaf(-tau, acc[r], sb[i]);
                    const float ad = fabsf(D);
                    const float w = __builtin_amdgcn_exp2f(-ad * kLog2e);   // e^{-|D|}
                    const float em = expm1_nonpos(ad, w);
                    const bool pos = D > 0.f;
                    const float al = pos ? kq[r].x : ka[r];
                    const float be = pos ? kq[r].z : kq[r].y;
                    f[r] = fmaxf(fmaf(fmaf(al, em, be), em, kq[r].w), 0.f);
                    u[r] = fmaf(2.f * kLog2e, fmaxf(-D, 0.f), -sh[i]);
                    umax = fmaxf(umax, u[r]);
                }
                if (__any(umax > kShiftStep)) {   // rare: raise the shift
                    const float up = fmaxf(umax, 0.f);
                    S[i] *= __builtin_amdgcn_exp2f(-up);
                    sh[i] += up;
#pragma unroll
                    for (int r = 0; r < 4; ++r) u[r] -= up;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i] = fmaf(f[r], __builtin_amdgcn_exp2f(u[r]), S[i]);
                if (EPS) {
                    const int c = (cbw + 4 * i) * 16 + col;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (c < Cq && kr0 + r < nv)
                            log_eps2[((size_t)h * Cq + c) * Nk + cur.jc + kr0 + r] =
                                f[r] > 0.f ? 2.f * sb[i] + kLn2 * (u[r] + sh[i]) + logf(f[r]) : -__builtin_inff();
                }
            }
        }
        if (cur.jc + PR_KC >= cur.j1) {   // the cluster's last chunk: combine the four row groups
            const int mg = cur.j1 - cur.j0;
#pragma unroll
            for (int i = 0; i < NCBW; ++i) {
                if (cbw + 4 * i >= ncb) continue;
                float m = sh[i], s2 = S[i];
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    const float om = __shfl_xor(m, o), os = __shfl_xor(s2, o);
                    const float mn = fmaxf(m, om);
                    s2 = s2 * __builtin_amdgcn_exp2f(m - mn) + os * __builtin_amdgcn_exp2f(om - mn);
                    m = mn;
                }
                const int c = (cbw + 4 * i) * 16 + col;
                if (grp == 0 && c < Cq) {
                    float lr = -__builtin_inff();
                    if (qlive[i] && s2 > 0.f)
                        lr = 2.f * sb[i] + kLn2 * (m + __log2f(s2)) - logf((float)mg);
                    log_ratio[((size_t)h * Cq + c) * Ck + cur.g] = lr;
                }
            }
        }
        if (took && tid == 0)   // read by every thread before the barrier above
            s_item[1] = pr_resolve(pend, hh, left, ctr_s, offsets_k, H, Cq, Ck, c_lo, c_hi, log_ratio);
        cur = nxt;
        bsel ^= 1;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | 0);   // no load is left in flight
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
    // one resident round: two workgroups per CU over the slices
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        ncu = 256;
    long long gx = (2LL * ncu + slices - 1) / slices;
    if (gx > (long long)a.H * a.Ck) gx = (long long)a.H * a.Ck;
    int* ctr = (int*)(a.scratch + a.L->pr_ctr);
    zero_words(ctr, (size_t)slices * a.H * 4, st);
    float* eps = (a.flags & SVGEAR_DEBUG_EPS) ? a.log_eps2 : nullptr;
    const int logit_only = (a.flags & SVGEAR_PROBE_LOGIT) ? 1 : 0;
    const float tau = 1.0f / sqrtf((float)PR_D);
#define SVG_PROBE_CASE(n)                                                                          \
    case n:                                                                                        \
        if (eps)                                                                                   \
            hipLaunchKernelGGL((k_probe_mfma<n, true>), dim3((int)gx, slices), dim3(256), PR_LDS2, st,  \
                               a.qbar, a.counts_q, (const bf16*)a.Kp, (const bf16*)a.Vp, a.kbar,   \
                               a.vbar, sbar, a.offsets_k, a.H, a.Nk, a.Cq, a.Ck, tau, logit_only,  \
                               ctr, a.log_ratio, eps);                                                  \
        else                                                                                       \
            hipLaunchKernelGGL((k_probe_mfma<n, false>), dim3((int)gx, slices), dim3(256), PR_LDS2, st,  \
                               a.qbar, a.counts_q, (const bf16*)a.Kp, (const bf16*)a.Vp, a.kbar,   \
                               a.vbar, sbar, a.offsets_k, a.H, a.Nk, a.Cq, a.Ck, tau, logit_only,  \
                               ctr, a.log_ratio, eps);                                                  \
        break;
    switch (ncbw) {
        SVG_PROBE_CASE(1) SVG_PROBE_CASE(2)
    default: return hipErrorInvalidValue;
    }
#undef SVG_PROBE_CASE
    return hipGetLastError();
}

}  // namespace svg
