/*
 * svgear.h -- C ABI of libsvgear.so: one SVG-EAR routed attention call
 * (cluster -> probe -> route -> hybrid attention) on an MI355X (gfx950).
 *
 * The method is the one described in "SVG-EAR: Parameter-Free Linear
 * Compensation for Sparse Video Generation via Error-aware Routing"; each entry
 * point below cites the passage that defines its operation:
 *   [R]  the Chinese review page (paper.rainbus.top), inference-pipeline
 *        paragraph, steps (1)-(5), and its weaknesses paragraph;
 *   [DE] the German gist.science page, technical summary, sections 2A-2C;
 *   [IT] the Italian gist.science page, technical summary, sections 2A-2C.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a DEVICE pointer to contiguous, row-major memory
 *   owned by the caller.  The library allocates no device memory and keeps no
 *   state between calls apart from loaded code objects and, per device, one
 *   side stream and two events that svgear_forward creates on first use and
 *   keeps until the process ends.
 * - Heads are independent.  Q is [H, Nq, d]; K and V are [H, Nk, d], in the
 *   element type given by svgear_shape.dtype (fp32 or bf16).  Cluster-indexed
 *   arrays are [H, C, ...], block arrays [H, Cq, Ck] with block (c, g) at
 *   c*Ck + g.  tau = 1/sqrt(d).
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *   default stream).  Only SVGEAR_DEBUG_SYNC makes a call wait for its work.
 * - `ws` is a caller-owned device workspace of at least
 *   svgear_workspace_bytes() bytes, 256-byte aligned.  Its contents need not be
 *   initialised and are clobbered.  Two calls that overlap in time must not
 *   share a workspace.
 * - All argument checks run on the host before anything is enqueued: a call
 *   that returns an error has enqueued nothing.  Errors are negative
 *   svgear_status codes; nothing is thrown across the ABI.  Asynchronous kernel
 *   faults surface as SVGEAR_E_HIP from a later synchronising call.
 * - Results are deterministic: identical inputs give bitwise identical outputs
 *   (integer atomics only; no floating-point atomics).
 * - Input values.  Any finite values with |x| < 2^56 are supported.  The
 *   clustering sums the members of a cluster exactly (two 64-bit fixed-point
 *   words per element at a power-of-two scale chosen per head from its largest
 *   magnitude M < 2^E), which captures every value whose unit in the last place
 *   is at least 2^(E - 2B), B = min(51, 62 - ceil(log2(N + 1))): for bf16 that
 *   is every non-zero |x| >= 2^(E + 7 - 2B) (2^(E - 83) at N = 75,600), for
 *   fp32 every |x| >= 2^(E + 23 - 2B).  A head with a non-finite value, a value
 *   of magnitude 2^56 or more, or a non-zero value below that floor is
 *   detected on the device; under SVGEAR_DEBUG_SYNC the call then returns
 *   SVGEAR_E_RANGE (without it, results of such a head are unspecified).
 */
#ifndef SVGEAR_H
#define SVGEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SVGEAR_OK = 0,
    SVGEAR_E_NULL = -1,      /* a required pointer is NULL                               */
    SVGEAR_E_SHAPE = -2,     /* a size is out of range (see svgear_shape)                */
    SVGEAR_E_DTYPE = -3,     /* unknown element type                                     */
    SVGEAR_E_ALIGN = -4,     /* a pointer is not 16-byte aligned (workspace: 256-byte)   */
    SVGEAR_E_WORKSPACE = -5, /* ws_bytes is smaller than svgear_workspace_bytes()        */
    SVGEAR_E_RHO = -6,       /* rho is NaN or outside [0, 1]                             */
    SVGEAR_E_HIP = -7,       /* the HIP runtime reported an error                        */
    SVGEAR_E_ARG = -8,       /* another invalid argument (side, flags); under
                                SVGEAR_DEBUG_SYNC also an init or label index out of range */
    SVGEAR_E_RANGE = -9      /* under SVGEAR_DEBUG_SYNC: an input value is out of the
                                supported range (see "Input values" above)                  */
} svgear_status;

typedef enum { SVGEAR_F32 = 0, SVGEAR_BF16 = 1 } svgear_dtype;

/* Problem shape.  Valid ranges: H >= 1; 1 <= Nq, Nk <= 2^20; d in {64, 128};
 * 1 <= Cq <= min(Nq, 4096); 1 <= Ck <= min(Nk, 4096); 1 <= iters <= 100. */
typedef struct {
    int32_t H, Nq, Nk, d, Cq, Ck, iters;
    int32_t dtype; /* svgear_dtype */
} svgear_shape;

enum {
    SVGEAR_LABELS_GIVEN = 1, /* svgear_cluster: skip k-means, reorder by the labels passed in */
    SVGEAR_DEBUG_EPS = 2,    /* svgear_probe: also write ln(e[c, j]) per key              */
    SVGEAR_DEBUG_SYNC = 4,   /* synchronise the stream before returning, report faults    */
    SVGEAR_PROBE_LOGIT = 8,  /* svgear_probe: logit-only estimate (no values), see below  */
    SVGEAR_PROBE_SCORE = 16  /* svgear_probe: attention-score comparator, see below       */
};

/* Per-call pointers of svgear_forward's intermediate results.  Any member may be
 * NULL, in which case the result lives in the workspace.  Shapes as in the
 * per-stage entry points below. */
typedef struct {
    int32_t* labels_q;   /* [H, Nq]      */
    float* qbar;         /* [H, Cq, d]   */
    int32_t* counts_q;   /* [H, Cq]      */
    int32_t* offsets_q;  /* [H, Cq + 1]  */
    int32_t* perm_q;     /* [H, Nq]      */
    int32_t* inv_perm_q; /* [H, Nq]      */
    void* Qp;            /* [H, Nq, d]   */
    int32_t* labels_k;   /* [H, Nk]      */
    float* kbar;         /* [H, Ck, d]   */
    float* vbar;         /* [H, Ck, d]   */
    int32_t* counts_k;   /* [H, Ck]      */
    int32_t* offsets_k;  /* [H, Ck + 1]  */
    int32_t* perm_k;     /* [H, Nk]      */
    int32_t* inv_perm_k; /* [H, Nk]      */
    void* Kp;            /* [H, Nk, d]   */
    void* Vp;            /* [H, Nk, d]   */
    float* log_ratio;    /* [H, Cq, Ck]  */
    uint8_t* mask;       /* [H, Cq, Ck]  */
    int64_t* sel_cost;   /* [H]          */
} svgear_intermediates;

/* Host only.  Writes the workspace size (bytes) that suffices for every entry
 * point called with this shape.  Returns SVGEAR_E_NULL / _SHAPE / _DTYPE on bad
 * arguments. */
int svgear_workspace_bytes(const svgear_shape* shape, size_t* bytes);

/* Step 1 of [R] (also [DE] 2A, [IT] 2A): semantic clustering and reordering.
 * side 0 clusters Q (N = Nq, C = Cq); side 1 clusters K (N = Nk, C = Ck) and
 * also reorders V and averages it over K's clusters.
 *
 * k-means: initial centroids are the rows X[h, init_idx[h, m]] (init_idx
 * [H, C], distinct values in [0, N)); then `iters` Lloyd iterations, each an
 * assignment to the nearest centroid in squared Euclidean distance (ties to
 * the lowest cluster index) followed by a mean update (an empty cluster keeps
 * its centroid).  Outputs: labels [H, N] from the last assignment; cent
 * [H, C, d] fp32 = the member means (rounded from exact sums); counts [H, C];
 * offsets [H, C+1] (exclusive prefix of counts); perm [H, N] (token at each
 * reordered position, a stable sort by label) and inv_perm [H, N]; Xp [H, N, d]
 * = X rows in reordered order (same dtype as X).  Side 1 additionally writes
 * vbar [H, C, d] fp32 (mean of V over each key cluster; zero if empty) and
 * Vp [H, N, d].  With SVGEAR_LABELS_GIVEN, `labels` is an input (values in
 * [0, C)) and init_idx may be NULL; k-means is skipped, cent holds the member
 * means (zero for an empty cluster).  V/vbar/Vp must be NULL on side 0 and
 * non-NULL on side 1.  Errors: _NULL, _SHAPE, _DTYPE, _ALIGN, _WORKSPACE, _ARG
 * (side or flags), _HIP; under SVGEAR_DEBUG_SYNC also _RANGE (see "Input
 * values") and _ARG for an init or label index outside its range. */
int svgear_cluster(const svgear_shape* shape, int side, const void* X, const void* V,
                   const int32_t* init_idx, int flags, int32_t* labels, float* cent, float* vbar,
                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* Xp,
                   void* Vp, void* ws, size_t ws_bytes, void* stream);

/* Steps 2 and 3 of [R] (also [DE] 2B, [IT] 2B): value-aware centroid probe and
 * error-to-cost ratio.  For query cluster c and reordered key j of key cluster
 * g:  e[c, j] = || exp(tau qbar_c . kbar_g) vbar_g - exp(tau qbar_c . k_j) v_j ||^2,
 * and the block ratio is r[c, g] = (sum over the block's n_c * m_g pairs of e)
 * / (n_c * m_g) = mean over j in g of e[c, j].  Writes log_ratio [H, Cq, Ck] =
 * ln r (fp32; -inf when n_c * m_g == 0 or r == 0): the natural log keeps the
 * full range of exp(2 tau q.k) without overflow and preserves the order.
 * Kp, Vp are the reordered keys/values [H, Nk, d] and offsets_k their cluster
 * ranges, as written by svgear_cluster.  With SVGEAR_DEBUG_EPS, log_eps2
 * [H, Cq, Nk] (reordered key order) receives ln e[c, j]; otherwise it may be
 * NULL.  Logits never go to device memory.
 * With SVGEAR_PROBE_LOGIT the estimate ignores the values ([R] step 2 labels
 * the printed formula the value-aware version; the German summary 2B describes
 * the probe as a logit difference):
 *     e[c, j] = ( exp(tau qbar_c . kbar_g) - exp(tau qbar_c . k_j) )^2,
 * block ratio and output as above; Vp and vbar are then not read (they must
 * still be valid pointers).
 * With SVGEAR_PROBE_SCORE the ratio is the attention-score rule that the pages
 * argue against ([R] novelty paragraph; [DE] 1 and 2B), read as the centroid
 * estimate of the attention mass of block (c, g) per pair of the block:
 *     ln r[c, g] = tau qbar_c . kbar_g
 *                  - ln sum_{g': m_g' > 0} m_g' exp(tau qbar_c . kbar_g'),
 * -inf where n_c m_g = 0.  Only qbar, kbar and the counts are read (the other
 * pointers must still be valid); it cannot be combined with
 * SVGEAR_PROBE_LOGIT or SVGEAR_DEBUG_EPS (SVGEAR_E_ARG).
 * Errors as svgear_cluster. */
int svgear_probe(const svgear_shape* shape, const float* qbar, const int32_t* counts_q,
                 const void* Kp, const void* Vp, const float* kbar, const float* vbar,
                 const int32_t* counts_k, const int32_t* offsets_k, int flags, float* log_ratio,
                 float* log_eps2, void* ws, size_t ws_bytes, void* stream);

/* svgear_probe without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, operation and errors as svgear_probe, minus
 * ws / ws_bytes: the probe's scratch is a device array inside the library of
 * 64 MiB, one per device, held until the process ends.  A shape whose probe scratch exceeds it (about
 * 4 H Cq Ck + 8 H Nk + 4 H Ck bytes) returns SVGEAR_E_WORKSPACE before anything
 * is enqueued.  The call allocates nothing.  All calls on one device share that
 * array: two calls that overlap in time on one device (on different streams
 * or from different threads) race and must be serialised by the caller. */
int svgear_probe_noalloc(const svgear_shape* shape, const float* qbar, const int32_t* counts_q,
                         const void* Kp, const void* Vp, const float* kbar, const float* vbar,
                         const int32_t* counts_k, const int32_t* offsets_k, int flags,
                         float* log_ratio, float* log_eps2, void* stream);

/* Step 3 of [R] with its weaknesses paragraph (greedy 0-1 knapsack heuristic):
 * per head, blocks are ordered by ratio, largest first (equal log_ratio: lower
 * block index first); with cost w = counts_q[c] * counts_k[g] and budget
 * B = floor((rho * Nq) * Nk) (fp64), the longest prefix of that order whose
 * total cost is <= B is selected.  Writes mask [H, Cq, Ck] (1 = exact block)
 * and sel_cost [H] (int64 total cost of the selection).  rho in [0, 1].
 * ws holds the selection's scratch (per-slice digit histograms, the top key
 * bits of every block, per-head states); calls that overlap on one workspace
 * race.
 * Errors: _NULL, _SHAPE, _RHO, _ALIGN, _WORKSPACE, _HIP. */
int svgear_route(const svgear_shape* shape, double rho, const float* log_ratio,
                 const int32_t* counts_q, const int32_t* counts_k, uint8_t* mask,
                 int64_t* sel_cost, void* ws, size_t ws_bytes, void* stream);

/* The other reading of the density budget ([R] future-work paragraph: the
 * same budget for every query cluster): each query cluster c selects within its
 * own row, B_c = floor((rho * counts_q[c]) * Nk) pairs (fp64), greedily in
 * descending ratio order (equal log_ratio: lower key-cluster index first), the
 * longest prefix whose total cost counts_q[c] * counts_k[g] is <= B_c.  Same
 * arguments, outputs and errors as svgear_route; sel_cost[h] is the total over
 * the head's rows.  Not used by svgear_forward (which routes per head). */
int svgear_route_rows(const svgear_shape* shape, double rho, const float* log_ratio,
                      const int32_t* counts_q, const int32_t* counts_k, uint8_t* mask,
                      int64_t* sel_cost, void* ws, size_t ws_bytes, void* stream);

/* Step 4 of [R] (also [DE] 2A, [IT] 2A): hybrid attention.  For each reordered
 * query row of cluster c (rows offsets_q[c] .. offsets_q[c+1] of Qp), one
 * softmax over (a) exact logits tau q.k_j with value v_j for the keys of every
 * key cluster g with mask[c, g] = 1, and (b) one compensation logit
 * tau q.kbar_g + ln m_g with value vbar_g for every g with mask[c, g] = 0 and
 * m_g = counts_k[g] > 0 (each skipped key replaced by its centroid).  The row
 * is written to O [H, Nq, d] at token position perm_q[row] (token order; same
 * dtype as Q).  Errors as svgear_cluster. */
int svgear_attention(const svgear_shape* shape, const void* Qp, const int32_t* offsets_q,
                     const int32_t* perm_q, const void* Kp, const void* Vp, const float* kbar,
                     const float* vbar, const int32_t* counts_k, const int32_t* offsets_k,
                     const uint8_t* mask, void* O, void* ws, size_t ws_bytes, void* stream);

/* Steps 1-4 of [R] in one call: cluster Q and K, probe, route, hybrid
 * attention, all enqueued without host synchronisation.  O [H, Nq, d]
 * receives the output in token order.  init_q [H, Cq] and init_k [H, Ck] are
 * the k-means initial token indices.  im may be NULL.  The Q clustering runs
 * on a per-device side stream (default priority) forked from `stream` by an
 * event and joined back by another before the probe, so it overlaps the K
 * clustering; everything else runs on `stream`, and when the call returns all
 * of its work is ordered on `stream` (safe under stream capture).  `stream`
 * must belong to the current device.  flags: 0 or SVGEAR_DEBUG_SYNC, which
 * waits for the call and reports the data errors the clusterings detect on the
 * device (SVGEAR_E_RANGE, or SVGEAR_E_ARG for an init index outside [0, N)).
 * Errors as the stages, and _ARG for other flags. */
int svgear_forward(const svgear_shape* shape, double rho, const void* Q, const void* K,
                   const void* V, const int32_t* init_q, const int32_t* init_k, void* O,
                   const svgear_intermediates* im, int flags, void* ws, size_t ws_bytes,
                   void* stream);

/* Static description of a status code. */
const char* svgear_status_string(int code);

/* ABI version (major * 10000 + minor * 100 + patch). */
int svgear_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SVGEAR_H */
