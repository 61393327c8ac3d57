/*
 * zeta.h -- C ABI of the MI355X (gfx950) ZETA causal top-k attention library (libzeta.so).
 *
 * Method: "ZETA: Leveraging Z-order Curves for Efficient Top-k Attention".
 *   [R] rebuttal page (paperhub.cn/paper/j9VVzueEbG)     [S] summary page (atlas.scime.ai)
 *   [A] arXiv abstract page (fugumt.com, 2501.14577v2)
 *
 * Problem statement ([S] "Problem" and "Approach", [A]): for every query of a causal
 * sequence, retrieve in parallel the k past tokens nearest on a 1-D Z-order curve of the
 * low-dimensional (d_K = 3) queries and keys, and combine their values with a trainable
 * Cauchy kernel.  The calls below take q, k [B,H,N,3] fp32, v [B,H,N,dv], gamma [H] and k,
 * and return the selected index tensor next to the output.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers to dense row-major memory owned by the
 *     caller.  The library allocates nothing; scratch memory is the caller's workspace (size
 *     from zeta_workspace_bytes), except for zeta_fwd_noalloc, whose scratch the library
 *     holds per GPU.  State kept between calls: a thread-local error string, the
 *     thread-local event list of the measurement hook zeta_set_stage_events (off unless a
 *     caller sets it), and zeta_fwd_noalloc's per-device scratch address.  Calls are
 *     re-entrant; calls that share a workspace must not overlap.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued on it
 *     asynchronously; no call synchronises the host.
 *   - Arguments are validated on the host before anything is launched; on any error the
 *     outputs are untouched and a status other than ZETA_OK is returned.  A launch or
 *     runtime failure returns ZETA_ERR_HIP (outputs then undefined).  zeta_last_error()
 *     gives a thread-local description of the last failure.  Nothing is thrown.
 *   - Validity: B, H, N >= 1; 1 <= topk <= ZETA_MAX_TOPK; dv >= 8, dv % 8 == 0,
 *     dv <= ZETA_MAX_DV; v_dtype is ZETA_F32 or ZETA_BF16; B*H*N*topk < 2^31;
 *     N < 2^30; pointers non-null.
 *   - gamma must be > 0 (not checked on the device; gamma <= 0 gives undefined values).
 */
#ifndef ZETA_H
#define ZETA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZETA_MAX_TOPK 256
#define ZETA_MAX_DV 512

typedef enum zeta_status {
    ZETA_OK = 0,
    ZETA_ERR_INVALID_ARGUMENT = 1,
    ZETA_ERR_UNSUPPORTED = 2,
    ZETA_ERR_WORKSPACE_TOO_SMALL = 3,
    ZETA_ERR_HIP = 4
} zeta_status;

typedef enum zeta_dtype { ZETA_F32 = 0, ZETA_BF16 = 1 } zeta_dtype;

/* Problem shape.  d_K = d_Q = 3 is fixed ([R] answer W2/A2 "Details about experiments").
 * v_dtype is a zeta_dtype; v, out, dout and dv share it.                                 */
typedef struct zeta_shape {
    int64_t B, H, N; /* batch, heads, sequence length                                    */
    int64_t dv;      /* value width                                                      */
    int64_t topk;    /* k: keys kept per query                                           */
    int32_t v_dtype; /* zeta_dtype                                                       */
    int32_t reserved;/* must be 0                                                        */
} zeta_shape;

typedef enum zeta_ws_kind { ZETA_WS_SELECT = 0, ZETA_WS_FWD = 1, ZETA_WS_BWD = 2 } zeta_ws_kind;

/* Workspace bytes needed by zeta_select / zeta_fwd / zeta_bwd for `shape` (0 if the shape
 * is invalid).  The workspace must be 256-byte aligned device memory.                    */
size_t zeta_workspace_bytes(const zeta_shape *shape, int32_t kind);

/* Z-order code of `rows` points x [rows][3] fp32 -> codes [rows] uint32.
 * [R] answer W2/A2 "Clarification of Binary Expansion and Precision": each coordinate is
 * discretised on a fixed grid and the bits of the three cells are interleaved.  Here:
 * cell = clamp(floor(128 x) + 512, 0, 1023) (fixed range [-4,4), 10 bits, NaN -> 0), and
 * bit b of axis a becomes bit 3b+a of a 30-bit code.  rows >= 0 (0 is a no-op).           */
zeta_status zeta_encode(const float *x, int64_t rows, uint32_t *codes, void *stream);

/* Number of levels of the merge-sort tree for sequence length N: floor(log2 N) + 1.     */
int32_t zeta_tree_levels(int64_t N);

/* Per-(b,h) merge-sort tree of key codes (diagnostic export; zeta_select builds it in its
 * workspace).  [R] answers W3/A3 and W2/A2 ("Clarification"): keys are sorted on the
 * Z-order line (radix sort) so a query's neighbours are found by binary search.  For the
 * causal mask the keys are kept sorted per aligned power-of-two block of positions:
 * level l holds every block [m 2^l, (m+1) 2^l) (the last one possibly shorter) sorted.
 * Entries are (code << 32) | j.  Layout [BH][levels][N] uint64.
 *   tree_asc : each block ordered by (code ascending, j ascending)
 *   tree_desc: each block ordered by (code ascending, j descending)
 * zk: codes [BH][N].                                                                     */
zeta_status zeta_build_tree(int64_t BH, int64_t N, const uint32_t *zk, uint64_t *tree_asc,
                            uint64_t *tree_desc, void *stream);

/* Exact causal top-k selection ([R] W3/A3, W2/A2; [S] "Approach").  For every query
 * (b,h,i): order the keys j <= i by (|zq_i - zk_j|, j), where |.| is the absolute
 * difference of the unsigned Z-order codes, and write the first min(topk, i+1) positions
 * to idx[b,h,i,0..), ascending in that order; the remaining slots are -1.
 * q, k: [B,H,N,3] fp32.  idx: [B,H,N,topk] int32 (output).                               */
zeta_status zeta_select(const zeta_shape *shape, const float *q, const float *k, int32_t *idx,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Forward: selection as zeta_select, then the Adaptive Cauchy-softmax over the selected
 * set ([R] answer W2/A2 "Discussion on its robustness"; answer W3/A3 on Euclidean
 * distance):
 *     s_ij = 1 / (1 + ||q_i - k_j||^2 / gamma_h^2),  o_i = sum_j s_ij v_j / sum_j s_ij,
 * with the raw fp32 q, k, fp32 arithmetic and fp32 accumulation; o is rounded once to
 * v_dtype (nearest even).  v, out: [B,H,N,dv] v_dtype.  gamma: [H] fp32, shared over B.
 * idx: [B,H,N,topk] int32 output, kept by the caller for zeta_bwd.                        */
zeta_status zeta_fwd(const zeta_shape *shape, const float *q, const float *k, const void *v,
                     const float *gamma, void *out, int32_t *idx, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Backward of zeta_fwd with the selection idx held fixed ([R] answers W3/A3 and Q2: the
 * forward+backward pass is the training cost; gamma is trained).  With a_ij = s_ij/S_i,
 * g_ij = dO_i . v_j, D_i = sum_j a_ij g_ij, c_ij = a_ij s_ij (g_ij - D_i):
 *     dq_i = -(2/gamma^2) sum_j c_ij (q_i - k_j)          dq: [B,H,N,3] fp32
 *     dk_j =  (2/gamma^2) sum_i c_ij (q_i - k_j)          dk: [B,H,N,3] fp32
 *     dv_j =  sum_i a_ij dO_i                             dv: [B,H,N,dv] v_dtype
 *     dgamma_h = (2/gamma_h^3) sum_{b,i,j} c_ij d_ij      dgamma: [H] fp32
 * Every sum runs in a fixed order (a key's pairs are sorted by query, then reduced by a
 * fixed butterfly), so results are bitwise reproducible: no floating-point atomics.
 * dout: [B,H,N,dv] v_dtype.
 * idx is expected to be the selection zeta_fwd returned: slot r of query i is used when
 * r < min(topk, i+1) and its entry is >= 0, and the entry is clamped to at most i; other
 * slots are ignored.  An index tensor that is not a valid selection therefore gives
 * meaningless but bounded results (no access outside the buffers).                      */
zeta_status zeta_bwd(const zeta_shape *shape, const float *q, const float *k, const void *v,
                     const float *gamma, const int32_t *idx, const void *dout, float *dq,
                     float *dk, void *dv, float *dgamma, void *workspace,
                     size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): zeta_fwd without a workspace argument.  Its
 * scratch is a device array of ZETA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends; the first zeta_fwd_noalloc call on a GPU looks up its
 * address (hipGetSymbolAddress) and keeps it.  The call allocates nothing.  Shapes whose
 * forward workspace (zeta_workspace_bytes(shape, ZETA_WS_FWD)) exceeds the scratch return
 * ZETA_ERR_WORKSPACE_TOO_SMALL, outputs untouched (B1 H8 N65536 dv128 k32 needs about
 * 101 MB and fits).  The scratch is that of the calling thread's current device, and
 * `stream` must belong to that device.  Every call on one GPU shares its scratch: no part
 * of it needs to start at zero (a call reads only what it wrote itself), and calls that
 * overlap on one GPU (other streams or threads) race, so serialise them.  Otherwise exactly
 * zeta_fwd: exact causal selection, same kernels, same results.                          */
#define ZETA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
zeta_status zeta_fwd_noalloc(const zeta_shape *shape, const float *q, const float *k,
                             const void *v, const float *gamma, void *out, int32_t *idx,
                             void *stream);

/* ---------------------------------------------------------------------------------------
 * Selection variants (the _ex calls).  NULL options = the exact causal selection with
 * 10-bit cells, i.e. the calls above.
 *
 *   ZETA_SELECT_EXACT    exact top-k by (|dz|, j), as zeta_select; with causal = 0 every
 *                        key j < N competes for every query (the unmasked form of the same
 *                        problem, [S] "Problem": the causal mask is what prevents one
 *                        search over the whole sorted sequence).
 *   ZETA_SELECT_CHUNKED  the pages' chunked causal search ([S] "Approach": sort and chunk
 *                        the keys; [R] answer W2/A2 "Details about experiments": 4-32
 *                        chunks; "Clarification": the window centred at the query's
 *                        insertion position).  Reading taken: chunks are the aligned blocks
 *                        of L positions, L the smallest power of two with L * chunks >= N;
 *                        each chunk's keys sorted by (code, j); for every chunk up to the
 *                        query's own, the min(k, chunk size) sorted entries starting
 *                        floor(k/2) before the insertion position (shifted to lie inside
 *                        the chunk); keys j > i dropped; the first k candidates by
 *                        (|dz|, j).  An approximation of the exact selection: a query may
 *                        get fewer than min(k, i+1) keys (-1 slots anywhere after the
 *                        picks) or none.  causal must be 1.
 *   ZETA_SELECT_CURVES   several Z-order curves ([R], on the asymmetry of interleaving):
 *                        curves = 3 takes the coordinate orders (K1,K2,K3), (K2,K3,K1),
 *                        (K3,K1,K2); curves = 6 all six orders (K1,K2,K3), (K1,K3,K2),
 *                        (K2,K3,K1), (K2,K1,K3), (K3,K1,K2), (K3,K2,K1).  Each curve takes
 *                        its exact top-(k / curves); idx lists curve 0's picks, then each
 *                        later curve's picks not listed yet; -1 in the remaining slots.
 *
 * bits = 12: the pages' own precision ([R] answer W2/A2 "Clarification of Binary Expansion
 * and Precision": a 4096-cell grid, three 12-bit components interleaved into 36 bits held in
 * a 64-bit integer).  Reading taken: the same fixed range [-4, 4), cell = clamp(floor(512 x)
 * + 2048, 0, 4095), NaN -> 0; bit b of axis a -> bit 3b + a.  Any mode; needs N < 2^28.
 * A query with no selected key outputs zero and passes no gradient.  zeta_bwd_ex uses only
 * `causal` from the options: slot r of query i is used when r < min(k, i+1) (causal) or
 * r < min(k, N) and idx >= 0; entries are clamped to the last usable key.
 * The stage events of zeta_set_stage_events keep their meaning; with several curves stages
 * 1 and 2 cover the first curve and stage 3 the remaining curves and the merge.            */
#define ZETA_MAX_CHUNKS 1024

typedef enum zeta_select_mode {
    ZETA_SELECT_EXACT = 0,
    ZETA_SELECT_CHUNKED = 1,
    ZETA_SELECT_CURVES = 2
} zeta_select_mode;

typedef struct zeta_select_opts {
    int32_t mode;     /* zeta_select_mode                                                   */
    int32_t causal;   /* 1: keys j <= i;  0: every key j < N (EXACT and CURVES only)        */
    int32_t bits;     /* bits per axis of the codes: 10, or 12 (N < 2^28)                   */
    int32_t chunks;   /* CHUNKED: number of chunks C, 1 <= C <= ZETA_MAX_CHUNKS              */
    int32_t curves;   /* CURVES: 3 or 6 (and topk >= curves)                                */
    int32_t reserved; /* must be 0                                                          */
} zeta_select_opts;

/* As the calls without _ex, for the selection variant in `opts` (NULL = exact, causal,
 * 10 bits).  Invalid options: ZETA_ERR_INVALID_ARGUMENT or ZETA_ERR_UNSUPPORTED (and 0
 * from zeta_workspace_bytes_ex).                                                          */
size_t zeta_workspace_bytes_ex(const zeta_shape *shape, const zeta_select_opts *opts,
                               int32_t kind);
zeta_status zeta_select_ex(const zeta_shape *shape, const zeta_select_opts *opts,
                           const float *q, const float *k, int32_t *idx, void *workspace,
                           size_t workspace_bytes, void *stream);
zeta_status zeta_fwd_ex(const zeta_shape *shape, const zeta_select_opts *opts, const float *q,
                        const float *k, const void *v, const float *gamma, void *out,
                        int32_t *idx, void *workspace, size_t workspace_bytes, void *stream);
zeta_status zeta_bwd_ex(const zeta_shape *shape, const zeta_select_opts *opts, const float *q,
                        const float *k, const void *v, const float *gamma, const int32_t *idx,
                        const void *dout, float *dq, float *dk, void *dv, float *dgamma,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Measurement hook (for timing individual kernels from the caller).  Hands this thread a
 * list of `count` hipEvent_t handles (created by the caller, with timing enabled).  Every
 * following zeta_select / zeta_fwd / zeta_bwd call on this thread records events[0] on its
 * stream before its first launch and events[s] after stage s, for as many stages as the
 * call has and `count` allows:
 *   zeta_select, zeta_fwd: 1 encode (q and k) and the query processing order (which the
 *                          select and the gather use), 2 tree build, 3 select kernel,
 *                          4 the processing order when stage 1 did not build it (chunked
 *                          search, 12-bit cells), 5 gather kernel (4, 5: zeta_fwd only);
 *   zeta_bwd:              1 encode and processing orders, 2 per-query kernel,
 *                          3 selection transpose (radix passes and segment starts),
 *                          4 per-key kernel, 5 dgamma reduction.
 * events = NULL or count = 0 turns recording off.  The events stay owned by the caller and
 * must outlive the calls that record them.                                               */
zeta_status zeta_set_stage_events(void *const *events, int32_t count);

/* Measurement hook: the rate of the scattered row gathers that the gather and backward
 * kernels make (whose rows are mostly L2 hits, so that rate, not HBM bandwidth, bounds them).
 * `groups` groups of 16 lanes each read `rows_per_group` rows of `row_bytes` bytes from
 * table [table_rows][row_bytes], 16 bytes per lane, the loads of eight rows in flight
 * together, rows drawn uniformly by a counter-based hash of (seed, group, row number); each
 * group writes one word folded from what it loaded to sink[group].  Bytes read per call:
 * groups * rows_per_group * row_bytes.  table: device, 16-byte aligned; table_rows a power of
 * two <= 2^32; row_bytes a multiple of 16 in [16, 256]; rows_per_group a multiple of 8 in
 * [8, 2^20]; 1 <= groups <= 2^34; sink: device uint32 [groups].  Validated on the host.  */
zeta_status zeta_probe_row_gather(const void *table, int64_t table_rows, int32_t row_bytes,
                                  int64_t groups, int32_t rows_per_group, uint32_t seed,
                                  uint32_t *sink, void *stream);

/* Static description of a status code.                                                   */
const char *zeta_status_string(zeta_status status);

/* Thread-local description of the last failure of a call on this thread ("" if none).  */
const char *zeta_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZETA_H */
