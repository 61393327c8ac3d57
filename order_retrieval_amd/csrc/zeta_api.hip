// zeta_api.hip -- the C ABI of include/zeta.h: validation, workspace plan, launch order.
//
// Everything is validated on the host before the first launch; the library allocates
// nothing (scratch lives in the caller's workspace) and never synchronises the stream.
#include <stdio.h>

#include <mutex>
#include <string>

#include "zeta.h"
#include "zeta_internal.hpp"

// Device scratch of zeta_fwd_noalloc: one array per GPU, held from the library's first use on
// that GPU until the process ends.  In host code its name is only a handle for
// hipGetSymbolAddress; the device address is looked up once per device and used everywhere.
static __device__ __align__(256) unsigned char scratch[ZETA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
thread_local zeta::StageEvents g_marks;

zeta_status fail(zeta_status st, const char* msg) {
    g_last_error = msg;
    return st;
}

zeta_status fail_hip(const char* what, hipError_t e) {
    char buf[256];
    snprintf(buf, sizeof buf, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
    g_last_error = buf;
    return ZETA_ERR_HIP;
}

int levels_of(int64_t N) {
    int l = 0;
    while ((int64_t(2) << l) <= N) ++l;
    return l + 1;
}

size_t align_up(size_t x) { return (x + zeta::kAlign - 1) & ~(zeta::kAlign - 1); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

zeta_status check_shape(const zeta_shape* sh) {
    if (!sh) return fail(ZETA_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (sh->B < 1 || sh->H < 1 || sh->N < 1)
        return fail(ZETA_ERR_INVALID_ARGUMENT, "B, H and N must be >= 1");
    if (sh->topk < 1) return fail(ZETA_ERR_INVALID_ARGUMENT, "topk must be >= 1");
    if (sh->topk > zeta::kMaxTopK) return fail(ZETA_ERR_UNSUPPORTED, "topk above ZETA_MAX_TOPK");
    if (sh->dv < 8 || sh->dv % 8 != 0)
        return fail(ZETA_ERR_UNSUPPORTED, "dv must be a positive multiple of 8");
    if (sh->dv > zeta::kMaxDv) return fail(ZETA_ERR_UNSUPPORTED, "dv above ZETA_MAX_DV");
    if (sh->v_dtype != ZETA_F32 && sh->v_dtype != ZETA_BF16)
        return fail(ZETA_ERR_UNSUPPORTED, "v_dtype must be ZETA_F32 or ZETA_BF16");
    if (sh->reserved != 0) return fail(ZETA_ERR_INVALID_ARGUMENT, "reserved must be 0");
    if (sh->N >= (int64_t(1) << 30)) return fail(ZETA_ERR_UNSUPPORTED, "N must be < 2^30");
    const int64_t lim = int64_t(1) << 31;
    if (sh->B > lim || sh->H > lim || sh->B * sh->H > lim / sh->N ||
        sh->B * sh->H * sh->N > (lim - 1) / sh->topk)
        return fail(ZETA_ERR_UNSUPPORTED, "B*H*N*topk must be < 2^31");
    return ZETA_OK;
}

zeta_status preflight() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip("no usable HIP device", e);
    return ZETA_OK;
}

// Resolved selection options (NULL options = exact, causal, 10 bits per axis).
struct Opts {
    int mode = ZETA_SELECT_EXACT;
    bool causal = true;
    int bits = 10;
    int chunks = 0;
    int curves = 0;
};

zeta_status resolve_opts(const zeta_select_opts* o, const zeta_shape* sh, Opts& r) {
    r = Opts{};
    if (!o) return ZETA_OK;
    if (o->reserved != 0) return fail(ZETA_ERR_INVALID_ARGUMENT, "opts.reserved must be 0");
    if (o->causal != 0 && o->causal != 1)
        return fail(ZETA_ERR_INVALID_ARGUMENT, "opts.causal must be 0 or 1");
    r.causal = o->causal == 1;
    r.mode = o->mode;
    r.bits = o->bits;
    r.chunks = o->chunks;
    r.curves = o->curves;
    if (r.bits != 10 && r.bits != 12)
        return fail(ZETA_ERR_INVALID_ARGUMENT, "opts.bits must be 10 or 12");
    if (r.bits == 12 && sh->N >= (int64_t(1) << 28))
        return fail(ZETA_ERR_UNSUPPORTED, "12-bit codes need N < 2^28");
    switch (r.mode) {
        case ZETA_SELECT_EXACT:
            break;
        case ZETA_SELECT_CHUNKED:
            if (!r.causal)
                return fail(ZETA_ERR_UNSUPPORTED, "the chunked search is a causal search");
            if (r.chunks < 1 || r.chunks > ZETA_MAX_CHUNKS)
                return fail(ZETA_ERR_INVALID_ARGUMENT, "opts.chunks must be in [1, ZETA_MAX_CHUNKS]");
            break;
        case ZETA_SELECT_CURVES:
            if (r.curves != 3 && r.curves != 6)
                return fail(ZETA_ERR_INVALID_ARGUMENT, "opts.curves must be 3 or 6");
            if (sh->topk < r.curves)
                return fail(ZETA_ERR_INVALID_ARGUMENT, "topk must be >= opts.curves");
            break;
        default:
            return fail(ZETA_ERR_INVALID_ARGUMENT, "unknown opts.mode");
    }
    return ZETA_OK;
}

// log2 of the chunk length: the smallest power of two L with L * chunks >= N.
int chunk_level(int64_t N, int chunks) {
    const int64_t want = (N + chunks - 1) / chunks;
    int l = 0;
    while ((int64_t(1) << l) < want) ++l;
    return l;
}

// Tree levels a selection needs: every level of the exact search; for the chunked search
// only up to the chunk level (which is above the top level when 2^lvl > N).  Under the
// causal mask a query sees i + 1 <= N keys, so a run of 2^l keys needs 2^l <= N - 1 except
// for the last query when N is a power of two; that query takes its one run of N keys as
// two runs of the level below, and the top level (a whole merge pass) is not built.
int tree_levels(const zeta_shape* sh, const Opts& o, int first) {
    if (o.mode == ZETA_SELECT_CHUNKED) return chunk_level(sh->N, o.chunks) + 1;
    if (o.causal && sh->N >= 2) {
        // N = 2K: the level below the top is shorter than the short runs, keep the top
        const int lv = levels_of(sh->N - 1);
        return lv - 1 >= first ? lv : levels_of(sh->N);
    }
    return levels_of(sh->N);
}

// Lowest tree level the selection reads (the levels below it are not written).
int tree_first(const zeta_shape* sh, const Opts& o) {
    if (o.mode == ZETA_SELECT_CHUNKED) return chunk_level(sh->N, o.chunks);
    const int k = o.mode == ZETA_SELECT_CURVES ? static_cast<int>(sh->topk) / o.curves
                                               : static_cast<int>(sh->topk);
    return zeta::select_first_level(k);
}

// Curve coordinate orders of the several-curve variant (rebuttal page, on the asymmetry of
// interleaving): 3 curves (K1,K2,K3), (K2,K3,K1), (K3,K1,K2); 6 curves in the order
// (K1,K2,K3), (K1,K3,K2), (K2,K3,K1), (K2,K1,K3), (K3,K1,K2), (K3,K2,K1).
int curve_perm(int curves, int c) {
    static constexpr int k3[3] = {zeta::perm_code(0, 1, 2), zeta::perm_code(1, 2, 0),
                                  zeta::perm_code(2, 0, 1)};
    static constexpr int k6[6] = {zeta::perm_code(0, 1, 2), zeta::perm_code(0, 2, 1),
                                  zeta::perm_code(1, 2, 0), zeta::perm_code(1, 0, 2),
                                  zeta::perm_code(2, 0, 1), zeta::perm_code(2, 1, 0)};
    return curves == 3 ? k3[c] : k6[c];
}

struct FwdPlan {
    size_t zq, zk, tasc, tdesc, perm, ohist, sel, total;
    int levels;  // tree levels of the selection
    int first;   // lowest level it reads
    int base;    // lowest level stored (levels below are never stored)
    int stored;  // levels stored per (b,h) and tree
};

FwdPlan plan_fwd(const zeta_shape* sh, const Opts& o) {
    const int64_t BHN = sh->B * sh->H * sh->N;
    FwdPlan p{};
    p.first = tree_first(sh, o);
    p.levels = tree_levels(sh, o, p.first);
    p.base = zeta::tree_store_base(p.levels, p.first);
    p.stored = p.levels > p.base ? p.levels - p.base : 0;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += align_up(bytes);
        return at;
    };
    const size_t code_bytes = o.bits == 12 ? sizeof(uint64_t) : sizeof(uint32_t);
    p.zq = take(code_bytes * BHN);
    p.zk = take(code_bytes * BHN);
    p.tasc = take(sizeof(uint64_t) * BHN * p.stored);
    p.tdesc = take(sizeof(uint64_t) * BHN * p.stored);
    p.perm = take(sizeof(uint32_t) * BHN);
    p.ohist = take(sizeof(uint32_t) * zeta::order_scratch_words(sh->B * sh->H, sh->N));
    // several curves: each curve's picks, [curves][BHN][topk / curves]
    p.sel = take(o.mode == ZETA_SELECT_CURVES
                     ? sizeof(int32_t) * BHN * static_cast<size_t>(sh->topk / o.curves) * o.curves
                     : 0);
    p.total = off;
    return p;
}

struct BwdPlan {
    size_t qs, qr, rq, dg, dgp, r0, r1, hist, totals, counts, offs, ends, zq, pq, zk, pk, ohist,
        total;
    int64_t P, tiles;
};

BwdPlan plan_bwd(const zeta_shape* sh, const Opts& o) {
    const int64_t BH = sh->B * sh->H, N = sh->N, K = sh->topk;
    BwdPlan p{};
    p.P = static_cast<int64_t>(zeta::bwd_pairs_per_head(N, static_cast<int>(K), o.causal));
    p.tiles = zeta::bwd_tiles_per_head(N * K);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += align_up(bytes);
        return at;
    };
    p.qs = take(2 * sizeof(float) * BH * N * K);
    p.qr = take(4 * sizeof(float) * BH * N);
    p.rq = take(sizeof(uint32_t) * BH * N);
    p.dg = take(sizeof(float) * BH * N);
    p.dgp = take(sizeof(float) * sh->H * zeta::dgamma_chunks(sh->B, N));
    // rec1: the second radix ping-pong buffer of 8-byte records when keys need more than 16
    // bits; otherwise it takes only the final 4-byte slot list
    int key_bits = 0;
    while ((int64_t(1) << key_bits) < N) ++key_bits;
    // 4-byte records from the first radix pass when keys fit 16 bits, else 8-byte ones
    p.r0 = take((zeta::bwd_records_packed(N, static_cast<int>(K)) ? 4 : 8) * BH * p.P);
    p.r1 = take((key_bits <= 16 ? 4 : 8) * BH * p.P);
    p.hist = take(sizeof(uint32_t) * BH * 256 * p.tiles);
    p.totals = take(sizeof(uint32_t) * BH * 256);
    p.counts = take(sizeof(uint32_t) * BH);
    p.offs = take(sizeof(uint32_t) * BH * (N + 1));
    p.ends = take(sizeof(uint32_t) * BH * (N + 1));
    // query and key codes (and their processing orders) adjacent, so one order build covers
    // both as 2 BH slices
    p.zq = take(sizeof(uint32_t) * 2 * BH * N);
    p.zk = p.zq + sizeof(uint32_t) * BH * N;
    p.pq = take(sizeof(uint32_t) * 2 * BH * N);
    p.pk = p.pq + sizeof(uint32_t) * BH * N;
    p.ohist = take(sizeof(uint32_t) * zeta::order_scratch_words(2 * BH, N));
    p.total = off;
    return p;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

zeta_status check_ws(void* ws, size_t have, size_t need) {
    if (!ws) return fail(ZETA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned(ws, zeta::kAlign))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (have < need) return fail(ZETA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
    return ZETA_OK;
}

zeta_status check_qk(const float* q, const float* k) {
    if (!q || !k) return fail(ZETA_ERR_INVALID_ARGUMENT, "q or k is NULL");
    if (!aligned(q, 4) || !aligned(k, 4))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "q and k must be 4-byte aligned");
    return ZETA_OK;
}

// Stage marks: 0 start, 1 after encoding, 2 after the tree, 3 after the selection (several
// curves: 1 and 2 are recorded after the first curve's encode and tree, 3 after the merge).
zeta_status run_select(const zeta_shape* sh, const Opts& o, const float* q, const float* k,
                       int32_t* idx, void* ws, hipStream_t s) {
    const FwdPlan p = plan_fwd(sh, o);
    const int64_t BH = sh->B * sh->H, N = sh->N, BHN = BH * N;
    const int L = p.levels;
    const int topk = static_cast<int>(sh->topk);
    uint32_t* zq = at<uint32_t>(ws, p.zq);
    uint32_t* zk = at<uint32_t>(ws, p.zk);
    uint64_t* ta = at<uint64_t>(ws, p.tasc);
    uint64_t* td = at<uint64_t>(ws, p.tdesc);
    g_marks.record(0, s);
    const int ncurves = o.mode == ZETA_SELECT_CURVES ? o.curves : 1;
    const int per = o.mode == ZETA_SELECT_CURVES ? topk / o.curves : topk;
    const bool wide = o.bits == 12;  // 36-bit codes
    uint64_t* zq64 = at<uint64_t>(ws, p.zq);
    uint64_t* zk64 = at<uint64_t>(ws, p.zk);
    for (int c = 0; c < ncurves; ++c) {
        const int perm = o.mode == ZETA_SELECT_CURVES ? curve_perm(o.curves, c) : zeta::kPermIdentity;
        hipError_t e;
        if (wide) {
            e = zeta::launch_encode36_perm(q, BHN, perm, zq64, s);
            if (e == hipSuccess) e = zeta::launch_encode36_perm(k, BHN, perm, zk64, s);
        } else if (o.mode != ZETA_SELECT_CHUNKED) {
            // the codes and the query processing order of the select (and later of the
            // gather)
            e = zeta::launch_encode_order(q, zq, k, zk, BH, N, perm, false,
                                          at<uint32_t>(ws, p.perm), at<uint32_t>(ws, p.ohist), s);
        } else {
            e = zeta::launch_encode2_perm(q, zq, k, zk, BHN, perm, s);
        }
        if (e != hipSuccess) return fail_hip("encode launch", e);
        if (c == 0) g_marks.record(1, s);
        e = wide ? zeta::launch_build_tree36(BH, N, L, p.first, zk64, ta, td, s)
                 : zeta::launch_build_tree(BH, N, L, p.first, zk, ta, td, s);
        if (e != hipSuccess) return fail_hip("tree launch", e);
        if (c == 0) g_marks.record(2, s);
        int32_t* dst = idx;
        int kk = topk;
        if (o.mode == ZETA_SELECT_CURVES) {
            dst = at<int32_t>(ws, p.sel) + static_cast<int64_t>(c) * BHN * per;
            kk = per;
        }
        if (o.mode == ZETA_SELECT_CHUNKED) {
            const int lvl = chunk_level(N, o.chunks);
            e = wide ? zeta::launch_select_chunked36(BH, N, p.stored, p.base, lvl, topk, zq64, ta,
                                                     idx, s)
                     : zeta::launch_select_chunked(BH, N, p.stored, p.base, lvl, topk, zq, ta, idx,
                                                   s);
        } else {
            e = wide ? zeta::launch_select36(BH, N, p.stored, p.base, kk, o.causal, zq64, zk64, ta,
                                             td, nullptr, dst, s)
                     : zeta::launch_select(BH, N, p.stored, p.base, kk, o.causal, zq, zk, ta, td,
                                           at<uint32_t>(ws, p.perm), dst, s);
        }
        if (e != hipSuccess) return fail_hip("select launch", e);
    }
    if (o.mode == ZETA_SELECT_CURVES) {
        hipError_t e = zeta::launch_curves_merge(BHN, o.curves, per, topk, at<int32_t>(ws, p.sel),
                                                 idx, s);
        if (e != hipSuccess) return fail_hip("merge launch", e);
    }
    g_marks.record(3, s);
    return ZETA_OK;
}

zeta_status check_fwd_args(const float* q, const float* k, const void* v, const float* gamma,
                           const void* out, const int32_t* idx) {
    zeta_status st = check_qk(q, k);
    if (st != ZETA_OK) return st;
    if (!v || !gamma || !out || !idx) return fail(ZETA_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned(v, 16) || !aligned(out, 16))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "v and out must be 16-byte aligned");
    if (!aligned(gamma, 4) || !aligned(idx, 4))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "gamma and idx must be 4-byte aligned");
    return ZETA_OK;
}

// The forward's launches on a validated call: selection, processing order, gather.
zeta_status run_fwd(const zeta_shape* shape, const Opts& o, const float* q, const float* k,
                    const void* v, const float* gamma, void* out, int32_t* idx, void* workspace,
                    hipStream_t s) {
    const FwdPlan p = plan_fwd(shape, o);
    zeta_status st = run_select(shape, o, q, k, idx, workspace, s);
    if (st != ZETA_OK) return st;
    uint32_t* perm = at<uint32_t>(workspace, p.perm);
    // The exact and several-curve selections with 10-bit cells built the query processing
    // order already (from the last curve's codes: the order only schedules work).  Otherwise
    // it is built here from 10-bit query codes, written over the 36-bit ones with 12-bit
    // cells (the order buckets by the top code bits, which both share).
    hipError_t e = hipSuccess;
    if (o.bits == 12 || o.mode == ZETA_SELECT_CHUNKED) {
        uint32_t* zo = at<uint32_t>(workspace, p.zq);
        if (o.bits == 12) e = zeta::launch_encode(q, shape->B * shape->H * shape->N, zo, s);
        if (e == hipSuccess)
            e = zeta::launch_order(shape->B * shape->H, shape->N, zo, perm,
                                   at<uint32_t>(workspace, p.ohist), s);
        if (e != hipSuccess) return fail_hip("order launch", e);
    }
    g_marks.record(4, s);
    e = zeta::launch_gather(shape->B * shape->H, shape->H, shape->N, shape->dv,
                            static_cast<int>(shape->topk), o.causal, shape->v_dtype == ZETA_BF16, q,
                            k, v, gamma, idx, perm, out, s);
    if (e != hipSuccess) return fail_hip("gather launch", e);
    g_marks.record(5, s);
    return ZETA_OK;
}

// Device address of the no-allocation scratch on the calling thread's current device, looked
// up on the first call on that device (with it current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

zeta_status scratch_of_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip("no usable HIP device", e);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ZETA_ERR_UNSUPPORTED, "zeta_fwd_noalloc supports device ordinals below 64");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip("hipGetSymbolAddress(scratch)", e);
        if (!p) return fail(ZETA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ZETA_OK;
}

}  // namespace

extern "C" {

size_t zeta_workspace_bytes_ex(const zeta_shape* shape, const zeta_select_opts* opts,
                               int32_t kind) {
    if (check_shape(shape) != ZETA_OK) return 0;
    Opts o;
    if (resolve_opts(opts, shape, o) != ZETA_OK) return 0;
    switch (kind) {
        case ZETA_WS_SELECT:
        case ZETA_WS_FWD:
            return plan_fwd(shape, o).total;
        case ZETA_WS_BWD:
            return plan_bwd(shape, o).total;
        default:
            g_last_error = "unknown workspace kind";
            return 0;
    }
}

size_t zeta_workspace_bytes(const zeta_shape* shape, int32_t kind) {
    return zeta_workspace_bytes_ex(shape, nullptr, kind);
}

int32_t zeta_tree_levels(int64_t N) { return N < 1 ? 0 : levels_of(N); }

zeta_status zeta_encode(const float* x, int64_t rows, uint32_t* codes, void* stream) {
    g_last_error.clear();
    if (rows < 0) return fail(ZETA_ERR_INVALID_ARGUMENT, "rows must be >= 0");
    if (rows == 0) return ZETA_OK;
    if (!x || !codes) return fail(ZETA_ERR_INVALID_ARGUMENT, "x or codes is NULL");
    if (!aligned(x, 4) || !aligned(codes, 4))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "x and codes must be 4-byte aligned");
    zeta_status st = preflight();
    if (st != ZETA_OK) return st;
    hipError_t e = zeta::launch_encode(x, rows, codes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZETA_OK : fail_hip("encode launch", e);
}

zeta_status zeta_build_tree(int64_t BH, int64_t N, const uint32_t* zk, uint64_t* tree_asc,
                            uint64_t* tree_desc, void* stream) {
    g_last_error.clear();
    if (BH < 1 || N < 1) return fail(ZETA_ERR_INVALID_ARGUMENT, "BH and N must be >= 1");
    if (N >= (int64_t(1) << 30) || BH > (int64_t(1) << 31) / N)
        return fail(ZETA_ERR_UNSUPPORTED, "BH*N must be < 2^31 and N < 2^30");
    if (!zk || !tree_asc || !tree_desc) return fail(ZETA_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned(zk, 4) || !aligned(tree_asc, 8) || !aligned(tree_desc, 8))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "misaligned pointer");
    zeta_status st = preflight();
    if (st != ZETA_OK) return st;
    hipError_t e = zeta::launch_build_tree(BH, N, levels_of(N), 0, zk, tree_asc, tree_desc,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZETA_OK : fail_hip("tree launch", e);
}

zeta_status zeta_select_ex(const zeta_shape* shape, const zeta_select_opts* opts, const float* q,
                           const float* k, int32_t* idx, void* workspace, size_t workspace_bytes,
                           void* stream) {
    g_last_error.clear();
    zeta_status st = check_shape(shape);
    if (st != ZETA_OK) return st;
    Opts o;
    if ((st = resolve_opts(opts, shape, o)) != ZETA_OK) return st;
    if ((st = check_qk(q, k)) != ZETA_OK) return st;
    if (!idx || !aligned(idx, 4)) return fail(ZETA_ERR_INVALID_ARGUMENT, "idx NULL or misaligned");
    if ((st = check_ws(workspace, workspace_bytes, plan_fwd(shape, o).total)) != ZETA_OK) return st;
    if ((st = preflight()) != ZETA_OK) return st;
    return run_select(shape, o, q, k, idx, workspace, static_cast<hipStream_t>(stream));
}

zeta_status zeta_select(const zeta_shape* shape, const float* q, const float* k, int32_t* idx,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return zeta_select_ex(shape, nullptr, q, k, idx, workspace, workspace_bytes, stream);
}

zeta_status zeta_fwd_ex(const zeta_shape* shape, const zeta_select_opts* opts, const float* q,
                        const float* k, const void* v, const float* gamma, void* out,
                        int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    zeta_status st = check_shape(shape);
    if (st != ZETA_OK) return st;
    Opts o;
    if ((st = resolve_opts(opts, shape, o)) != ZETA_OK) return st;
    if ((st = check_fwd_args(q, k, v, gamma, out, idx)) != ZETA_OK) return st;
    if ((st = check_ws(workspace, workspace_bytes, plan_fwd(shape, o).total)) != ZETA_OK) return st;
    if ((st = preflight()) != ZETA_OK) return st;
    return run_fwd(shape, o, q, k, v, gamma, out, idx, workspace,
                   static_cast<hipStream_t>(stream));
}

zeta_status zeta_fwd_noalloc(const zeta_shape* shape, const float* q, const float* k,
                             const void* v, const float* gamma, void* out, int32_t* idx,
                             void* stream) {
    g_last_error.clear();
    zeta_status st = check_shape(shape);
    if (st != ZETA_OK) return st;
    const Opts o;  // the exact causal selection with 10-bit cells
    if ((st = check_fwd_args(q, k, v, gamma, out, idx)) != ZETA_OK) return st;
    const size_t need = plan_fwd(shape, o).total;
    if (need > ZETA_NOALLOC_SCRATCH_BYTES) {
        char buf[192];
        snprintf(buf, sizeof buf,
                 "this shape's forward needs %zu bytes of scratch; zeta_fwd_noalloc holds %zu "
                 "(ZETA_NOALLOC_SCRATCH_BYTES)",
                 need, static_cast<size_t>(ZETA_NOALLOC_SCRATCH_BYTES));
        return fail(ZETA_ERR_WORKSPACE_TOO_SMALL, buf);
    }
    if ((st = preflight()) != ZETA_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != ZETA_OK) return st;
    return run_fwd(shape, o, q, k, v, gamma, out, idx, ws, static_cast<hipStream_t>(stream));
}

zeta_status zeta_fwd(const zeta_shape* shape, const float* q, const float* k, const void* v,
                     const float* gamma, void* out, int32_t* idx, void* workspace,
                     size_t workspace_bytes, void* stream) {
    return zeta_fwd_ex(shape, nullptr, q, k, v, gamma, out, idx, workspace, workspace_bytes,
                       stream);
}

zeta_status zeta_bwd_ex(const zeta_shape* shape, const zeta_select_opts* opts, const float* q,
                        const float* k, const void* v, const float* gamma, const int32_t* idx,
                        const void* dout, float* dq, float* dk, void* dv, float* dgamma,
                        void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    zeta_status st = check_shape(shape);
    if (st != ZETA_OK) return st;
    Opts o;
    if ((st = resolve_opts(opts, shape, o)) != ZETA_OK) return st;
    if ((st = check_qk(q, k)) != ZETA_OK) return st;
    if (!v || !gamma || !idx || !dout || !dq || !dk || !dv || !dgamma)
        return fail(ZETA_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned(v, 16) || !aligned(dout, 16) || !aligned(dv, 16))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "v, dout and dv must be 16-byte aligned");
    if (!aligned(gamma, 4) || !aligned(idx, 4) || !aligned(dq, 4) || !aligned(dk, 4) ||
        !aligned(dgamma, 4))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "misaligned pointer");
    const BwdPlan p = plan_bwd(shape, o);
    if ((st = check_ws(workspace, workspace_bytes, p.total)) != ZETA_OK) return st;
    if ((st = preflight()) != ZETA_OK) return st;
    zeta::BwdBuffers b{};
    b.coef = at<float2>(workspace, p.qs);
    b.qrec = at<float4>(workspace, p.qr);
    b.rank_q = at<uint32_t>(workspace, p.rq);
    b.dg_row = at<float>(workspace, p.dg);
    b.dg_part = at<float>(workspace, p.dgp);
    b.rec0 = at<uint2>(workspace, p.r0);
    b.rec1 = at<uint2>(workspace, p.r1);
    b.hist = at<uint32_t>(workspace, p.hist);
    b.totals = at<uint32_t>(workspace, p.totals);
    b.counts = at<uint32_t>(workspace, p.counts);
    b.offs = at<uint32_t>(workspace, p.offs);
    b.ends = at<uint32_t>(workspace, p.ends);
    b.zq = at<uint32_t>(workspace, p.zq);
    b.perm_q = at<uint32_t>(workspace, p.pq);
    b.zk = at<uint32_t>(workspace, p.zk);
    b.perm_k = at<uint32_t>(workspace, p.pk);
    b.ohist = at<uint32_t>(workspace, p.ohist);
    b.P = p.P;
    b.tiles = p.tiles;
    hipError_t e = zeta::launch_bwd(shape->B * shape->H, shape->H, shape->N, shape->dv,
                                    static_cast<int>(shape->topk), o.causal,
                                    shape->v_dtype == ZETA_BF16, q, k, v, gamma, idx, dout, dq, dk,
                                    dv, dgamma, b, g_marks, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZETA_OK : fail_hip("backward launch", e);
}

zeta_status zeta_bwd(const zeta_shape* shape, const float* q, const float* k, const void* v,
                     const float* gamma, const int32_t* idx, const void* dout, float* dq,
                     float* dk, void* dv, float* dgamma, void* workspace,
                     size_t workspace_bytes, void* stream) {
    return zeta_bwd_ex(shape, nullptr, q, k, v, gamma, idx, dout, dq, dk, dv, dgamma, workspace,
                       workspace_bytes, stream);
}

zeta_status zeta_probe_row_gather(const void* table, int64_t table_rows, int32_t row_bytes,
                                  int64_t groups, int32_t rows_per_group, uint32_t seed,
                                  uint32_t* sink, void* stream) {
    g_last_error.clear();
    if (!table || !sink) return fail(ZETA_ERR_INVALID_ARGUMENT, "table or sink is NULL");
    if (!aligned(table, 16) || !aligned(sink, 4))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "table must be 16-byte and sink 4-byte aligned");
    if (table_rows < 1 || table_rows > (int64_t(1) << 32) || (table_rows & (table_rows - 1)) != 0)
        return fail(ZETA_ERR_INVALID_ARGUMENT, "table_rows must be a power of two <= 2^32");
    if (row_bytes < 16 || row_bytes > 256 || row_bytes % 16 != 0)
        return fail(ZETA_ERR_INVALID_ARGUMENT, "row_bytes must be a multiple of 16 in [16, 256]");
    if (rows_per_group < 8 || rows_per_group % 8 != 0 || rows_per_group > (1 << 20))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "rows_per_group must be a multiple of 8 in [8, 2^20]");
    if (groups < 1 || groups > (int64_t(1) << 34))
        return fail(ZETA_ERR_INVALID_ARGUMENT, "groups must be in [1, 2^34]");
    zeta_status st = preflight();
    if (st != ZETA_OK) return st;
    hipError_t e = zeta::launch_probe_row_gather(table, table_rows, row_bytes, groups,
                                                 rows_per_group, seed, sink,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZETA_OK : fail_hip("probe launch", e);
}

zeta_status zeta_set_stage_events(void* const* events, int32_t count) {
    g_last_error.clear();
    if (count < 0) return fail(ZETA_ERR_INVALID_ARGUMENT, "count must be >= 0");
    g_marks.ev = count > 0 ? events : nullptr;
    g_marks.n = events ? count : 0;
    return ZETA_OK;
}

const char* zeta_status_string(zeta_status status) {
    switch (status) {
        case ZETA_OK: return "ZETA_OK";
        case ZETA_ERR_INVALID_ARGUMENT: return "ZETA_ERR_INVALID_ARGUMENT";
        case ZETA_ERR_UNSUPPORTED: return "ZETA_ERR_UNSUPPORTED";
        case ZETA_ERR_WORKSPACE_TOO_SMALL: return "ZETA_ERR_WORKSPACE_TOO_SMALL";
        case ZETA_ERR_HIP: return "ZETA_ERR_HIP";
        default: return "unknown zeta_status";
    }
}

const char* zeta_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
