// backward.hip -- gradients of the Cauchy-weighted top-k attention with the selection fixed.
//
// "ZETA: Leveraging Z-order Curves for Efficient Top-k Attention", rebuttal page: answers
// W3/A3 and Q2 time the forward+backward pass used for training; answer W2/A2 ("Discussion
// on its robustness") makes gamma trainable.  With s = 1/(1 + d/gamma^2), a = s/S,
// g_ij = dO_i . v_j, D_i = sum_j a_ij g_ij and c_ij = a_ij s_ij (g_ij - D_i):
//     dq_i = -(2/gamma^2) sum_j c_ij (q_i - k_j)        dv_j = sum_i a_ij dO_i
//     dk_j =  (2/gamma^2) sum_i c_ij (q_i - k_j)        dgamma = (2/gamma^3) sum c_ij d_ij
//
// Pipeline (no floating-point atomics anywhere, so results are bitwise reproducible):
//   1. per-query pass (queries in the Z-order processing order): recompute s, gather v rows
//      for g, write a_ij and c_ij of every selection slot and the query record {q_i, i}, both
//      at the query's rank in that order, and dq_i and the query's dgamma term;
//   2. selection transpose, a stable radix sort of the pairs of every (b,h) by key: a global
//      pass on the low byte of j builds 8-byte records {j, slot} grouped by that byte (the
//      slot named by the query's rank);
//   3. keys below 2^16: one workgroup per low-byte group sorts it on the high byte and writes
//      every key's segment bounds, leaving the slots in contiguous per-key segments (queries
//      ascending inside a segment); larger keys: global passes on the further bytes, then
//      the segment starts from the sorted keys;
//   4. per-key pass (keys in Z-order): each key gathers its pairs' {a_ij, c_ij}, query records
//      and dO_i rows and reduces its segment in a fixed order (dv, dk).  The pairs of keys
//      close on the curve come from queries close on the curve, whose ranks are close, so the
//      rank layout keeps those gathers inside a few cache lines;
//   5. dgamma: fixed-order reduction per head over the batch and the queries (one workgroup
//      per head, or two levels for long heads).
// g_ij = dO_i . v_j is formed once, on the query side, which owns dO_i; the key side only
// scales and adds rows.
#include "zeta_internal.hpp"
#include "vec_io.hpp"
#include "xlane.hpp"

namespace zeta {

constexpr int kRadixThreads = 256;
constexpr int kRadixItems = 16;
constexpr int kRadixTile = kRadixThreads * kRadixItems;

// A selection slot r of query i is a pair when r < min(topk, keys the query may use) (i+1
// under the causal mask, else N) and it holds an index >= 0; the index is clamped to the
// last usable key, so an index tensor that is not a valid selection still never leads
// outside the buffers (the result is then meaningless but defined).
__device__ __forceinline__ int64_t clamp_index(int32_t j, int64_t jmax) {
    return j < 0 ? 0 : (j > jmax ? jmax : j);
}

// Unsigned division by a divisor fixed for the launch (the selection width): a multiply-high,
// a subtract and two shifts, exact for every 32-bit numerator (Granlund and Montgomery,
// "Division by Invariant Integers using Multiplication", unsigned division by a run-time
// invariant divisor).
struct DivU32 {
    uint32_t m;  // low 32 bits of the 33-bit multiplier
    int sh1, sh2;
};

static DivU32 make_div(uint32_t d) {
    int l = 0;
    while ((uint64_t(1) << l) < d) ++l;  // ceil(log2 d)
    DivU32 r;
    r.m = static_cast<uint32_t>((((uint64_t(1) << l) - d) << 32) / d + 1);
    r.sh1 = l < 1 ? l : 1;
    r.sh2 = l > 1 ? l - 1 : 0;
    return r;
}

__device__ __forceinline__ uint32_t div_u32(uint32_t n, const DivU32& d) {
    const uint32_t t = __umulhi(d.m, n);
    return (t + ((n - t) >> d.sh1)) >> d.sh2;
}

struct PairSpec {
    int topk;
    int causal;
    int64_t N;
    DivU32 by_topk;  // division by topk
};

// j: the index stored in slot e.
__device__ __forceinline__ bool pair_item(int32_t j, int64_t e, const PairSpec& ps,
                                          uint32_t& key) {
    const uint32_t i = div_u32(static_cast<uint32_t>(e), ps.by_topk);
    const uint32_t r = static_cast<uint32_t>(e) - i * static_cast<uint32_t>(ps.topk);
    const int64_t nk = ps.causal ? static_cast<int64_t>(i) + 1 : ps.N;
    if (r >= nk) return false;  // slot beyond min(topk, nk)
    if (j < 0) return false;    // no selection in this slot
    key = static_cast<uint32_t>(clamp_index(j, nk - 1));
    return true;
}


// ---------------------------------------------------------------------------- 1. queries
// One 16-lane row (a DPP row) per query i, four queries per wavefront, taken in the Z-order
// processing order.  Each lane owns one slot of every group of 16 (query_slot_of_lane): it
// loads their indices and key rows and forms s, the distance terms and later a, c and the
// dq / dgamma terms.  The row keeps its chunks of dO_i in registers and walks the slots in
// batches of eight: the index comes from the owning lane by a DPP row broadcast, every lane
// loads its chunks of the v_j row (the batch's loads are issued together) and forms its
// parts of g_ij = dO_i . v_j, and one row reduce-scatter completes the batch's eight dot
// products in their owners.
constexpr int kRowLanes = 16;  // lanes per query or key
constexpr int kRowLoads = 8;   // rows whose loads are issued together
static_assert(kRowLoads == 8 && kRowLanes == 16, "two 8-slot reduce-scatters per 16-slot group");

// Slot ownership in the per-query pass: inside each group of 16 slots, lane l of the row owns
// slot (l & 1) * 8 + l / 2 (even lanes the first eight, odd lanes the last eight), which is
// where an 8-slot row reduce-scatter leaves each slot's total.
__device__ __forceinline__ int query_slot_of_lane(int l) { return (l & 1) * 8 + (l >> 1); }
constexpr int query_lane_of_slot(int s) { return (s & 7) * 2 + (s >> 3); }
// Workgroup sizes (measured): more curve neighbours per workgroup share a CU's L1 in the
// per-query pass (64 queries: 0.290 ms, 32: 0.297, 16: 0.315); the per-key pass keeps 256
// (8 keys: the same; 20 or 40 keys: 0.45 and 0.49 ms against 0.384).
constexpr int kQueryThreads = 1024;  // workgroup of the per-query pass
constexpr int kKeyThreads = 256;    // workgroup of the per-key pass
constexpr int kQueryRows = kQueryThreads / kRowLanes;  // queries per workgroup (one (b,h))
constexpr int kKeyRows = kKeyThreads / kRowLanes;      // keys per workgroup (one (b,h))

// g for slots L0 .. L0 + 7 of a 16-slot group: every lane forms its part of each dot product
// (its dO_i chunks with its chunks of the slot's value row; the row name comes from the
// slot's owner, and the batch's loads are issued together), then one row reduce-scatter
// leaves each slot's total in its owner.
template <bool BF16, bool O32, int CPL, int L0>
__device__ __forceinline__ void query_slots(const typename VecIO<BF16>::elem_t* __restrict__ vh,
                                            int dv, const int (&coff)[CPL], uint32_t jo,
                                            const float (&go)[CPL][VecIO<BF16>::kElems],
                                            int lrow, float& gmine) {
    using IO = VecIO<BF16>;
    using R = typename IO::raw_t;
    constexpr int E = IO::kElems;
    R raw[kRowLoads][CPL];
    static_for<0, kRowLoads>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        // an empty slot names key 0's row, g unused
        const uint32_t nm = row_bcast<query_lane_of_slot(L0 + w)>(jo);
#pragma unroll
        for (int c = 0; c < CPL; ++c) raw[w][c] = RowRef<BF16, O32>::load(vh, nm, dv, coff[c]);
    });
    float parts[kRowLoads];
    static_for<0, kRowLoads>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float x[E];
            IO::unpack(raw[w][c], x);
#pragma unroll
            for (int e = 0; e < E; ++e) part += go[c][e] * x[e];
        }
        parts[w] = part;
    });
    const float g = row_reduce_scatter8(parts, lrow);  // slot L0 + lrow / 2
    if ((lrow & 1) == L0 / kRowLoads) gmine = g;
}

template <bool BF16, bool O32, int CPL, int U>
__global__ void __launch_bounds__(kQueryThreads) zeta_bwd_query_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ gamma, const int32_t* __restrict__ idx,
    const void* __restrict__ dout, const uint32_t* __restrict__ order, int64_t N, int64_t H,
    int dv, int topk, int causal, int64_t tph, int64_t tiles, int64_t per_xcd,
    float2* __restrict__ coef, float4* __restrict__ qrec, float* __restrict__ dq,
    float* __restrict__ dg_row) {
    using IO = VecIO<BF16>;
    using T = typename IO::elem_t;
    constexpr int E = IO::kElems;
    const int64_t tile = xcd_tile(blockIdx.x, per_xcd);
    if (tile >= tiles) return;  // uniform over the workgroup
    const int64_t bh = tile / tph;  // uniform: tiles never straddle two (b,h)
    const int lrow = threadIdx.x & (kRowLanes - 1);
    const int64_t pos = (tile - bh * tph) * kQueryRows + threadIdx.x / kRowLanes;
    const bool live = pos < N;
    const int64_t pp = live ? pos : N - 1;  // a row past the end reads a real query, stores nothing
    const int chunks = dv / E;
    const int64_t i = order ? static_cast<int64_t>(order[bh * N + pp]) : pp;
    const int64_t row = bh * N + i;
    const float g = gamma[bh % H];
    const float inv_g2 = 1.0f / (g * g);
    const float q0 = q[3 * row], q1 = q[3 * row + 1], q2 = q[3 * row + 2];
    const int64_t nk = causal ? i + 1 : N;  // keys the query may use
    const int m = live ? static_cast<int>(nk < topk ? nk : topk) : 0;
    const int32_t* ir = idx + row * topk;
    const float* kh = k + bh * N * 3;
    const T* vh = static_cast<const T*>(v) + bh * N * dv;

    // every setup load reads a clamped position and is held live before any test, so the
    // loads of a kind are in flight together
    float go[CPL][E];
    int coff[CPL];  // element offset of the lane's chunks (clamped; chunks past the row meet go = 0)
    typename IO::raw_t graw[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lrow + c * kRowLanes;
        coff[c] = (ch < chunks ? ch : chunks - 1) * E;
        graw[c] = IO::load_raw(static_cast<const T*>(dout) + row * dv + coff[c]);
    }
    int32_t jr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = query_slot_of_lane(lrow) + u * kRowLanes;
        jr[u] = ir[r < topk ? r : topk - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) keep(jr[u]);
    bool sel[U];
    Point3 kp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        sel[u] = query_slot_of_lane(lrow) + u * kRowLanes < m && jr[u] >= 0;
        jr[u] = sel[u] ? static_cast<int32_t>(clamp_index(jr[u], nk - 1)) : 0;
        kp[u] = load_point(kh, jr[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) keep(kp[u]);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        IO::unpack(graw[c], go[c]);
        if (lrow + c * kRowLanes >= chunks)
#pragma unroll
            for (int e = 0; e < E; ++e) go[c][e] = 0.0f;
    }

    uint32_t jo[U];
    float so[U], dx[U], dy[U], dz[U], gg[U];
    float ssum = 0.0f, nsel = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        jo[u] = 0;  // not selected: names key 0's row, never summed
        so[u] = dx[u] = dy[u] = dz[u] = gg[u] = 0.0f;
        if (sel[u]) {
            jo[u] = RowRef<BF16, O32>::name(jr[u], dv);
            nsel += 1.0f;
            dx[u] = q0 - kp[u].x;
            dy[u] = q1 - kp[u].y;
            dz[u] = q2 - kp[u].z;
            so[u] = 1.0f / (1.0f + (dx[u] * dx[u] + dy[u] * dy[u] + dz[u] * dz[u]) * inv_g2);
            ssum += so[u];
        }
    }
    const float S = group_sum(ssum, kRowLanes);
    nsel = group_sum(nsel, kRowLanes);
    // the longest selection among the wavefront's four queries sets the trip count
    int most = m;
    most = max(most, __shfl_xor(most, 16, 64));
    most = max(most, __shfl_xor(most, 32, 64));

    static_for<0, U>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (u * kRowLanes < most) {
            static_for<0, kRowLanes / kRowLoads>([&](auto bc) {
                constexpr int b = decltype(bc)::value;
                if (u * kRowLanes + b * kRowLoads < most)
                    query_slots<BF16, O32, CPL, b * kRowLoads>(vh, dv, coff, jo[u], go, lrow, gg[u]);
            });
        }
    });

    float tsum = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (sel[u]) tsum += so[u] * gg[u];
    const float inv_S = nsel > 0.0f ? 1.0f / S : 0.0f;  // an empty selection passes no gradient
    const float D = group_sum(tsum, kRowLanes) * inv_S;

    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, ag = 0.0f;
    float2* cr = coef + (bh * N + pp) * topk;  // slots of the query's rank
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (sel[u]) {
            const float a = so[u] * inv_S;
            const float c = a * so[u] * (gg[u] - D);
            if (live) cr[query_slot_of_lane(lrow) + u * kRowLanes] = make_float2(a, c);
            a0 += c * dx[u];
            a1 += c * dy[u];
            a2 += c * dz[u];
            ag += c * (dx[u] * dx[u] + dy[u] * dy[u] + dz[u] * dz[u]);
        }
    }
    a0 = group_sum(a0, kRowLanes);
    a1 = group_sum(a1, kRowLanes);
    a2 = group_sum(a2, kRowLanes);
    ag = group_sum(ag, kRowLanes);
    if (live && lrow == 0) {
        const float f = -2.0f * inv_g2;
        dq[3 * row] = f * a0;
        dq[3 * row + 1] = f * a1;
        dq[3 * row + 2] = f * a2;
        dg_row[row] = 2.0f * inv_g2 / g * ag;
        qrec[bh * N + pp] = make_float4(q0, q1, q2, __uint_as_float(static_cast<uint32_t>(i)));
    }
}

// The per-query pass for selections wider than 64 slots: the slots are taken in batches of
// 64 (four per lane) in two passes over the row's selection.  The first pass forms s_ij and
// g_ij batch by batch (as above), keeps their running sums S_i and sum_j s_ij g_ij, and parks
// {s_ij, g_ij} in the slot's coefficient entry; the second pass, with D_i known, reads them
// back (the lane that wrote an entry reads it), forms a_ij and c_ij, overwrites the entry with
// {a_ij, c_ij} and adds the dq and dgamma terms.
constexpr int kWideU = 4;
constexpr int kWideBatch = kWideU * kRowLanes;

template <bool BF16, bool O32, int CPL>
__global__ void __launch_bounds__(kQueryThreads) zeta_bwd_query_wide_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ gamma, const int32_t* __restrict__ idx,
    const void* __restrict__ dout, const uint32_t* __restrict__ order, int64_t N, int64_t H,
    int dv, int topk, int causal, int64_t tph, int64_t tiles, int64_t per_xcd,
    float2* __restrict__ coef, float4* __restrict__ qrec, float* __restrict__ dq,
    float* __restrict__ dg_row) {
    using IO = VecIO<BF16>;
    using T = typename IO::elem_t;
    constexpr int E = IO::kElems;
    constexpr int U = kWideU;
    const int64_t tile = xcd_tile(blockIdx.x, per_xcd);
    if (tile >= tiles) return;  // uniform over the workgroup
    const int64_t bh = tile / tph;  // uniform: tiles never straddle two (b,h)
    const int lrow = threadIdx.x & (kRowLanes - 1);
    const int64_t pos = (tile - bh * tph) * kQueryRows + threadIdx.x / kRowLanes;
    const bool live = pos < N;
    const int64_t pp = live ? pos : N - 1;  // a row past the end reads a real query, stores nothing
    const int chunks = dv / E;
    const int64_t i = order ? static_cast<int64_t>(order[bh * N + pp]) : pp;
    const int64_t row = bh * N + i;
    const float g = gamma[bh % H];
    const float inv_g2 = 1.0f / (g * g);
    const float q0 = q[3 * row], q1 = q[3 * row + 1], q2 = q[3 * row + 2];
    const int64_t nk = causal ? i + 1 : N;  // keys the query may use
    const int m = live ? static_cast<int>(nk < topk ? nk : topk) : 0;
    const int32_t* ir = idx + row * topk;
    const float* kh = k + bh * N * 3;
    const T* vh = static_cast<const T*>(v) + bh * N * dv;
    float2* cr = coef + (bh * N + pp) * topk;  // slots of the query's rank

    float go[CPL][E];
    int coff[CPL];  // element offset of the lane's chunks (clamped; chunks past the row meet go = 0)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lrow + c * kRowLanes;
        coff[c] = (ch < chunks ? ch : chunks - 1) * E;
        IO::unpack(IO::load_raw(static_cast<const T*>(dout) + row * dv + coff[c]), go[c]);
        if (ch >= chunks)
#pragma unroll
            for (int e = 0; e < E; ++e) go[c][e] = 0.0f;
    }
    int most = m;
    most = max(most, __shfl_xor(most, 16, 64));
    most = max(most, __shfl_xor(most, 32, 64));
    const int batches = (most + kWideBatch - 1) / kWideBatch;

    // slot u of the lane in batch sb: selected?, its key (clamped) and point
    auto slot_setup = [&](int sb, int32_t (&jr)[U], bool (&sel)[U], Point3 (&kp)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = sb + query_slot_of_lane(lrow) + u * kRowLanes;
            jr[u] = ir[r < topk ? r : topk - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) keep(jr[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            sel[u] = sb + query_slot_of_lane(lrow) + u * kRowLanes < m && jr[u] >= 0;
            jr[u] = sel[u] ? static_cast<int32_t>(clamp_index(jr[u], nk - 1)) : 0;
            kp[u] = load_point(kh, jr[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) keep(kp[u]);
    };

    // pass 1: s, g, their sums; {s, g} parked in the slot's entry
    float ssum = 0.0f, nsel = 0.0f, tsum = 0.0f;
    for (int bt = 0; bt < batches; ++bt) {
        const int sb = bt * kWideBatch;
        int32_t jr[U];
        bool sel[U];
        Point3 kp[U];
        slot_setup(sb, jr, sel, kp);
        uint32_t jo[U];
        float so[U], gg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            jo[u] = 0;  // not selected: names key 0's row, never summed
            so[u] = gg[u] = 0.0f;
            if (sel[u]) {
                jo[u] = RowRef<BF16, O32>::name(jr[u], dv);
                const float dx = q0 - kp[u].x, dy = q1 - kp[u].y, dz = q2 - kp[u].z;
                so[u] = 1.0f / (1.0f + (dx * dx + dy * dy + dz * dz) * inv_g2);
            }
        }
        const int left = most - sb;
        static_for<0, U>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            if (u * kRowLanes < left) {
                static_for<0, kRowLanes / kRowLoads>([&](auto bc) {
                    constexpr int b = decltype(bc)::value;
                    if (u * kRowLanes + b * kRowLoads < left)
                        query_slots<BF16, O32, CPL, b * kRowLoads>(vh, dv, coff, jo[u], go, lrow,
                                                                   gg[u]);
                });
            }
        });
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sel[u]) {
                ssum += so[u];
                nsel += 1.0f;
                tsum += so[u] * gg[u];
                if (live) cr[sb + query_slot_of_lane(lrow) + u * kRowLanes] = make_float2(so[u], gg[u]);
            }
        }
    }
    const float S = group_sum(ssum, kRowLanes);
    nsel = group_sum(nsel, kRowLanes);
    const float inv_S = nsel > 0.0f ? 1.0f / S : 0.0f;  // an empty selection passes no gradient
    const float D = group_sum(tsum, kRowLanes) * inv_S;

    // pass 2: a, c from the parked {s, g}; the dq and dgamma terms
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, ag = 0.0f;
    for (int bt = 0; bt < batches; ++bt) {
        const int sb = bt * kWideBatch;
        int32_t jr[U];
        bool sel[U];
        Point3 kp[U];
        slot_setup(sb, jr, sel, kp);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sel[u] && live) {
                const int r = sb + query_slot_of_lane(lrow) + u * kRowLanes;
                const float2 sg = cr[r];
                const float dx = q0 - kp[u].x, dy = q1 - kp[u].y, dz = q2 - kp[u].z;
                const float a = sg.x * inv_S;
                const float c = a * sg.x * (sg.y - D);
                cr[r] = make_float2(a, c);
                a0 += c * dx;
                a1 += c * dy;
                a2 += c * dz;
                ag += c * (dx * dx + dy * dy + dz * dz);
            }
        }
    }
    a0 = group_sum(a0, kRowLanes);
    a1 = group_sum(a1, kRowLanes);
    a2 = group_sum(a2, kRowLanes);
    ag = group_sum(ag, kRowLanes);
    if (live && lrow == 0) {
        const float f = -2.0f * inv_g2;
        dq[3 * row] = f * a0;
        dq[3 * row + 1] = f * a1;
        dq[3 * row + 2] = f * a2;
        dg_row[row] = 2.0f * inv_g2 / g * ag;
        qrec[bh * N + pp] = make_float4(q0, q1, q2, __uint_as_float(static_cast<uint32_t>(i)));
    }
}

template <bool BF16, bool O32, int CPL>
static hipError_t launch_query_c(int64_t BH, int64_t N, int64_t H, int dv, int topk,
                                 int causal, const float* q, const float* k, const void* v,
                                 const float* gamma, const int32_t* idx, const void* dout,
                                 const uint32_t* order, float2* coef, float4* qrec, float* dq,
                                 float* dg_row, hipStream_t s) {
    const int64_t tph = (N + kQueryRows - 1) / kQueryRows;
    const int64_t tiles = BH * tph;
    const int64_t per = xcd_per(tiles);
    const int u = (topk + kRowLanes - 1) / kRowLanes;  // slots per lane
    auto kern = u <= 1 ? zeta_bwd_query_kernel<BF16, O32, CPL, 1>
              : u <= 2 ? zeta_bwd_query_kernel<BF16, O32, CPL, 2>
              : u <= 4 ? zeta_bwd_query_kernel<BF16, O32, CPL, 4>
                       : zeta_bwd_query_wide_kernel<BF16, O32, CPL>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(per * kXcds)), dim3(kQueryThreads), 0, s,
                       q, k, v,
                       gamma, idx, dout, order, N, H, dv, topk, causal, tph, tiles, per, coef,
                       qrec, dq, dg_row);
    return hipGetLastError();
}

template <bool BF16, int CPL>
static hipError_t launch_query_o(int64_t BH, int64_t N, int64_t H, int dv, int topk,
                                 int causal, const float* q, const float* k, const void* v,
                                 const float* gamma, const int32_t* idx, const void* dout,
                                 const uint32_t* order, float2* coef, float4* qrec, float* dq,
                                 float* dg_row, hipStream_t s) {
    if (rows_fit_32(N, dv, sizeof(typename VecIO<BF16>::elem_t)))
        return launch_query_c<BF16, true, CPL>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, coef, qrec, dq, dg_row, s);
    return launch_query_c<BF16, false, CPL>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, coef, qrec, dq, dg_row, s);
}

template <bool BF16>
static hipError_t launch_query(int64_t BH, int64_t N, int64_t H, int dv, int topk, int causal,
                               const float* q, const float* k, const void* v, const float* gamma,
                               const int32_t* idx, const void* dout, const uint32_t* order,
                               float2* coef, float4* qrec, float* dq, float* dg_row,
                               hipStream_t s) {
    const int cpl = (dv / VecIO<BF16>::kElems + kRowLanes - 1) / kRowLanes;
    if (cpl <= 1)
        return launch_query_o<BF16, 1>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, coef, qrec, dq, dg_row, s);
    if (cpl <= 2)
        return launch_query_o<BF16, 2>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, coef, qrec, dq, dg_row, s);
    if (BF16 || cpl <= 4)  // bf16 rows have <= 64 chunks
        return launch_query_o<BF16, 4>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, coef, qrec, dq, dg_row, s);
    return launch_query_o<BF16, BF16 ? 4 : 8>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, coef, qrec, dq, dg_row, s);
}

// ---------------------------------------------------------------------------- 2. transpose
// Every pair travels through the sort as one 8-byte record {j, p}, p = rank(i) * topk + r
// the pair's slot in the per-query pass's rank-ordered coefficients.  Pass 0 reads the
// selection in pair order (coalesced) and builds the records; later passes move records.
// The key kernel then reads each key's pairs as one contiguous run of records.
// A tile's items are loaded from clamped positions (item min(e, items - 1); with no items at
// all, position 0, inside the buffers) and all held live before any is tested, so the loads
// are in flight together.  Pass 0 loads the slot's index into rec.x and turns it into the
// record {j, e} (or an invalid item) afterwards.
template <bool FIRST>
__device__ __forceinline__ uint2 load_item(const int32_t* __restrict__ idx,
                                           const uint2* __restrict__ rin, int64_t e,
                                           int64_t items) {
    const int64_t ec = e < items ? e : (items > 0 ? items - 1 : 0);
    if (FIRST) return make_uint2(static_cast<uint32_t>(idx[ec]), 0u);
    return rin[ec];
}

template <bool FIRST>
__device__ __forceinline__ bool make_item(uint2& rec, int64_t e, int64_t items,
                                          const PairSpec& ps) {
    if (e >= items) return false;
    if (FIRST) {
        uint32_t key;
        if (!pair_item(static_cast<int32_t>(rec.x), e, ps, key)) return false;
        rec = make_uint2(key, static_cast<uint32_t>(e));
    }
    return true;
}

// Digit counts of one tile of items.  Pass 0 takes every selection slot (items = N * topk)
// and keeps the pairs; later passes take the first counts[bh] records.
template <bool FIRST>
__global__ void __launch_bounds__(kRadixThreads) zeta_radix_hist_kernel(
    const int32_t* __restrict__ idx, const uint2* __restrict__ rin, int64_t slots,
    const uint32_t* __restrict__ counts, int64_t in_stride, int shift, int64_t tiles,
    PairSpec ps, uint32_t* __restrict__ hist) {
    __shared__ uint32_t cnt[256];
    const int64_t bh = blockIdx.y;
    const int64_t items = FIRST ? slots : static_cast<int64_t>(counts[bh]);
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRadixTile;
    uint2 rec[kRadixItems];
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it)
        rec[it] = load_item<FIRST>(idx + bh * in_stride, rin + bh * in_stride,
                                   t0 + it * kRadixThreads + threadIdx.x, items);
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it) keep(rec[it].x);
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it)
        if (make_item<FIRST>(rec[it], t0 + it * kRadixThreads + threadIdx.x, items, ps))
            atomicAdd(&cnt[(rec[it].x >> shift) & 255u], 1u);
    __syncthreads();
    hist[(bh * 256 + threadIdx.x) * tiles + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of one (b,h, digit) row of per-tile counts (in place) and its total.
__global__ void __launch_bounds__(64) zeta_radix_scan_kernel(uint32_t* __restrict__ hist,
                                                             int64_t tiles,
                                                             uint32_t* __restrict__ totals) {
    const int64_t rowid = static_cast<int64_t>(blockIdx.y) * 256 + blockIdx.x;
    uint32_t* h = hist + rowid * tiles;
    const int lane = threadIdx.x;
    const int64_t per = (tiles + 63) / 64;
    const int64_t b0 = lane * per;
    const int64_t b1 = b0 + per < tiles ? b0 + per : tiles;
    uint32_t local = 0;
    for (int64_t t = b0; t < b1; ++t) local += h[t];
    uint32_t incl = local;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    uint32_t run = incl - local;
    for (int64_t t = b0; t < b1; ++t) {
        const uint32_t c = h[t];
        h[t] = run;
        run += c;
    }
    if (lane == 63) totals[rowid] = incl;
}

// Stable scatter of one tile.  Wavefront w owns the tile's items [w*1024, (w+1)*1024) in
// input order (iteration-major, then lane), ranks each item among the equal digits of its
// iteration with 8 ballots, and keeps a running count per digit in its own LDS row, so the
// item's rank inside its wavefront needs no barrier.  The four wavefronts' counts then give
// every item its slot in the tile sorted by digit (equal digits in input order); the tile is
// staged in LDS in that order and written out with consecutive lanes on consecutive slots
// of a digit's run, so the global writes are coalesced.  Pass 0 also records the number of
// pairs of each (b,h) in counts[bh] (the sum of the digit totals).
template <bool FIRST, bool PACK>
__global__ void __launch_bounds__(kRadixThreads) zeta_radix_scatter_kernel(
    const int32_t* __restrict__ idx, const uint2* __restrict__ rin, int64_t slots,
    uint32_t* __restrict__ counts, int64_t in_stride, int shift, int64_t tiles, PairSpec ps,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ totals, int64_t P,
    const uint32_t* __restrict__ rank_of, uint2* __restrict__ rout) {
    constexpr int kWaves = kRadixThreads / 64;
    constexpr int kWaveItems = kRadixTile / kWaves;
    __shared__ uint2 stage[kRadixTile];
    __shared__ uint32_t scan[256];
    __shared__ uint32_t local[256];
    __shared__ int32_t delta[256];
    __shared__ uint32_t wcnt[kWaves][256];
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRadixTile + wave * kWaveItems;
    const int64_t items = FIRST ? slots : static_cast<int64_t>(counts[bh]);

    uint2 rec[kRadixItems];
    uint32_t okmask = 0;
    {
        const int64_t off = bh * in_stride;
        // pass 0: the rank of the slot's query in the processing order (slot e belongs to
        // query e / topk; clamped positions, in flight with the indices)
        uint32_t rk[kRadixItems];
#pragma unroll
        for (int it = 0; it < kRadixItems; ++it) {
            rec[it] = load_item<FIRST>(idx + off, rin + off, t0 + it * 64 + lane, items);
            if constexpr (FIRST) {
                const int64_t e = t0 + it * 64 + lane;
                const int64_t ec = e < items ? e : (items > 0 ? items - 1 : 0);
                rk[it] = rank_of[bh * ps.N + div_u32(static_cast<uint32_t>(ec), ps.by_topk)];
            }
        }
#pragma unroll
        for (int it = 0; it < kRadixItems; ++it) {
            keep(rec[it]);
            if constexpr (FIRST) keep(rk[it]);
        }
#pragma unroll
        for (int it = 0; it < kRadixItems; ++it) {
            if (make_item<FIRST>(rec[it], t0 + it * 64 + lane, items, ps)) {
                okmask |= 1u << it;
                if constexpr (FIRST) {
                    // the record names the slot r of the query's rank: rank * topk + r
                    const uint32_t e = rec[it].y;
                    const uint32_t r = e - div_u32(e, ps.by_topk) * static_cast<uint32_t>(ps.topk);
                    rec[it].y = rk[it] * static_cast<uint32_t>(ps.topk) + r;
                }
            }
        }
    }

#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcnt[w][tid] = 0;
    scan[tid] = totals[bh * 256 + tid];
    __syncthreads();

    // rank of every item among the equal digits before it in this wavefront
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t lrank[kRadixItems];
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it) {
        const bool valid = (okmask >> it) & 1u;
        const uint32_t digit = valid ? (rec[it].x >> shift) & 255u : 0u;
        const uint64_t peers = digit_peers<8>(digit, valid);
        // every lane reads the running count before the group's first lane advances it (LDS
        // operations of one wavefront take effect in program order)
        const uint32_t before = valid ? wcnt[wave][digit] : 0u;
        if (valid && (peers & lt) == 0) wcnt[wave][digit] = before + __popcll(peers);
        lrank[it] = before + __popcll(peers & lt);
    }
    __syncthreads();

    // digit tid: its count in the tile, and the exclusive scans of the digit totals (global
    // start of the digit) and of the tile's counts (start of the digit in the staged tile)
    uint32_t tile_cnt = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tile_cnt += wcnt[w][tid];
    local[tid] = tile_cnt;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive Hillis-Steele scans
        const uint32_t y = tid >= o ? scan[tid - o] : 0u;
        const uint32_t z = tid >= o ? local[tid - o] : 0u;
        __syncthreads();
        scan[tid] += y;
        local[tid] += z;
        __syncthreads();
    }
    const uint32_t lstart = local[tid] - tile_cnt;
    const uint32_t gstart =
        scan[tid] - totals[bh * 256 + tid] + hist[(bh * 256 + tid) * tiles + blockIdx.x];
    const uint32_t tile_items = local[255];
    if (FIRST && blockIdx.x == 0 && tid == 255) counts[bh] = scan[255];
    delta[tid] = static_cast<int32_t>(gstart) - static_cast<int32_t>(lstart);
    uint32_t run = lstart;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {  // the wavefronts' shares of the digit, in order
        const uint32_t c = wcnt[w][tid];
        wcnt[w][tid] = run;
        run += c;
    }
    __syncthreads();

#pragma unroll
    for (int it = 0; it < kRadixItems; ++it) {
        if ((okmask >> it) & 1u) {
            const uint32_t digit = (rec[it].x >> shift) & 255u;
            stage[wcnt[wave][digit] + lrank[it]] = rec[it];
        }
    }
    __syncthreads();

    uint2* out = rout + bh * P;
    uint32_t* out32 = reinterpret_cast<uint32_t*>(rout) + bh * P;
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it) {
        const int t = it * kRadixThreads + tid;  // slot in the staged tile
        if (t < static_cast<int>(tile_items)) {
            const uint2 r = stage[t];
            // packed: the low byte of j is the bucket the record lands in, so a 4-byte record
            // holds the high byte of j (bits 24..31) and the slot (below 2^24)
            if constexpr (PACK)
                out32[delta[(r.x >> shift) & 255u] + t] = ((r.x >> 8) << 24) | r.y;
            else
                out[delta[(r.x >> shift) & 255u] + t] = r;
        }
    }
}

// ---------------------------------------------------------------------------- 3. segments
// Keys below 2^16: the one global pass sorts the records stably by the low byte of j, so
// bucket b holds the pairs of the keys j with j mod 256 = b (every bucket about 1/256 of the
// pairs, whatever the key popularity) in ascending slot order.  The bucket implies the low
// byte, so that pass writes 4-byte records: the high byte of j above a 24-bit slot.  One
// workgroup per bucket
// finishes the sort on the high byte of j: it counts the bucket's digits (one per key),
// writes every key's segment [begin, end) from their exclusive scan, and scatters the records
// stably a tile at a time (ranked by ballots and staged in LDS like a radix tile), so the
// slots p land in contiguous runs inside the bucket's range, ascending p inside a key.
// A key's segment is contiguous; the segments are not in key order (the per-key pass only
// needs each one's bounds).

// Inclusive sum over the workgroup's 256 threads of one value each (wavefront shuffles, then
// the four wavefront totals).  `part` holds 4 words; the caller syncs before reusing it.
__device__ __forceinline__ uint32_t scan256_incl(uint32_t v, uint32_t* part) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) part[wave] = x;
    __syncthreads();
    for (int w = 0; w < wave; ++w) x += part[w];
    return x;
}

// The per-group sort's tile: twelve records per thread (measured: 127 VGPRs and four waves
// per SIMD; 0.177 ms for the transpose against 0.186 with sixteen, and no gain with 8, 10 or
// 14).
constexpr int kBucketItems = 12;
constexpr int kBucketTile = kRadixThreads * kBucketItems;

__global__ void __launch_bounds__(kRadixThreads) zeta_bucket_sort_kernel(
    const uint32_t* __restrict__ rin, const uint32_t* __restrict__ totals, int64_t N, int64_t P,
    uint32_t* __restrict__ slots, uint32_t* __restrict__ begin, uint32_t* __restrict__ end) {
    static_assert(kRadixThreads == 256, "one thread per digit");
    constexpr int kWaves = kRadixThreads / 64;
    constexpr int kWaveItems = kBucketTile / kWaves;
    __shared__ uint2 stage[kBucketTile];
    __shared__ uint32_t wcnt[kWaves][256];
    __shared__ uint32_t run[256];   // bucket-relative output position of each digit's next record
    __shared__ int32_t delta[256];
    __shared__ uint32_t part[kWaves];
    const int64_t bh = blockIdx.y;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    // the bucket's records [s0, s1): the pass's digit totals are the bucket sizes
    uint32_t s0, s1;
    {
        const uint32_t incl = scan256_incl(totals[bh * 256 + tid], part);
        if (tid == b) run[0] = incl;
        __syncthreads();
        s1 = run[0];
        s0 = s1 - totals[bh * 256 + b];
        __syncthreads();
    }
    const uint32_t n = s1 - s0;
    const uint32_t* rb = rin + bh * P + s0;
    // record e of the bucket as {high byte of j << 8, slot}, from its 4-byte form
    auto rec_at = [&](uint32_t e) -> uint2 {
        const uint32_t w = rb[e];
        return make_uint2((w >> 24) << 8, w & 0xFFFFFFu);
    };

    // digit counts over the bucket; the first tile stays in registers for the scatter
    run[tid] = 0;
    __syncthreads();
    // (loads from clamped positions, all in flight before any is used; an empty bucket
    // loads nothing)
    uint2 rec[kBucketItems];
    auto load_tile = [&](uint32_t c0) {
#pragma unroll
        for (int it = 0; it < kBucketItems; ++it) {
            const uint32_t e = c0 + wave * kWaveItems + it * 64 + lane;
            rec[it] = rec_at(e < n ? e : n - 1);
        }
#pragma unroll
        for (int it = 0; it < kBucketItems; ++it) keep(rec[it]);
    };
    for (uint32_t c0 = 0; c0 < n; c0 += kBucketTile) {
        if (c0 == 0) {
            load_tile(0);  // stays in registers for the scatter
#pragma unroll
            for (int it = 0; it < kBucketItems; ++it)
                if (wave * kWaveItems + it * 64 + lane < n) atomicAdd(&run[rec[it].x >> 8], 1u);
        } else {
            uint32_t dg[kBucketItems];
#pragma unroll
            for (int it = 0; it < kBucketItems; ++it) {
                const uint32_t e = c0 + wave * kWaveItems + it * 64 + lane;
                dg[it] = rec_at(e < n ? e : n - 1).x;
            }
#pragma unroll
            for (int it = 0; it < kBucketItems; ++it) keep(dg[it]);
#pragma unroll
            for (int it = 0; it < kBucketItems; ++it)
                if (c0 + wave * kWaveItems + it * 64 + lane < n) atomicAdd(&run[dg[it] >> 8], 1u);
        }
    }
    __syncthreads();
    {
        const uint32_t c = run[tid];
        const uint32_t ex = scan256_incl(c, part) - c;
        const int64_t j = static_cast<int64_t>(tid) * 256 + b;  // the key of digit tid
        if (j < N) {
            begin[bh * (N + 1) + j] = s0 + ex;
            end[bh * (N + 1) + j] = s0 + ex + c;
        }
        __syncthreads();
        run[tid] = ex;
    }

    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t* out = slots + bh * P + s0;
    for (uint32_t c0 = 0; c0 < n; c0 += kBucketTile) {
        if (c0 > 0) load_tile(c0);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) wcnt[w][tid] = 0;
        __syncthreads();
        // rank of every record among the equal digits before it in this wavefront's share
        uint32_t lrank[kBucketItems];
#pragma unroll
        for (int it = 0; it < kBucketItems; ++it) {
            const bool valid = c0 + wave * kWaveItems + it * 64 + lane < n;
            const uint32_t digit = rec[it].x >> 8;
            const uint64_t peers = digit_peers<8>(digit, valid);
            const uint32_t before = valid ? wcnt[wave][digit] : 0u;
            if (valid && (peers & lt) == 0) wcnt[wave][digit] = before + __popcll(peers);
            lrank[it] = before + __popcll(peers & lt);
        }
        __syncthreads();
        uint32_t tile_cnt = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tile_cnt += wcnt[w][tid];
        const uint32_t lstart = scan256_incl(tile_cnt, part) - tile_cnt;
        delta[tid] = static_cast<int32_t>(run[tid]) - static_cast<int32_t>(lstart);
        uint32_t r = lstart;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = wcnt[w][tid];
            wcnt[w][tid] = r;
            r += c;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kBucketItems; ++it) {
            if (c0 + wave * kWaveItems + it * 64 + lane < n)
                stage[wcnt[wave][rec[it].x >> 8] + lrank[it]] = rec[it];
        }
        __syncthreads();
        const uint32_t items = n - c0 < kBucketTile ? n - c0 : kBucketTile;
#pragma unroll
        for (int it = 0; it < kBucketItems; ++it) {
            const uint32_t t = it * kRadixThreads + tid;
            if (t < items) {
                const uint2 rr = stage[t];
                out[delta[rr.x >> 8] + static_cast<int32_t>(t)] = rr.y;
            }
        }
        run[tid] += tile_cnt;
        __syncthreads();
    }
}

// Keys of more than 16 bits: the global passes sort the records fully by j, and
// offs[j] = first record of key j, offs[N] = number of pairs (key j's segment is
// [offs[j], offs[j+1])).
__global__ void __launch_bounds__(256) zeta_segment_offsets_kernel(const uint2* __restrict__ recs,
                                                                    const uint32_t* __restrict__ counts,
                                                                    int64_t P, int64_t N,
                                                                    uint32_t* __restrict__ offs) {
    const int64_t bh = blockIdx.y;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t cnt = counts[bh];
    uint32_t* oh = offs + bh * (N + 1);
    if (cnt == 0) {  // no pairs: every segment empty
        if (t == 0)
            for (int64_t jj = 0; jj <= N; ++jj) oh[jj] = 0;
        return;
    }
    if (t >= cnt) return;
    const uint2* rh = recs + bh * P;
    const int64_t kk = rh[t].x;
    const int64_t lo = t == 0 ? 0 : static_cast<int64_t>(rh[t - 1].x) + 1;
    for (int64_t jj = lo; jj <= kk; ++jj) oh[jj] = static_cast<uint32_t>(t);
    if (t == cnt - 1)
        for (int64_t jj = kk + 1; jj <= N; ++jj) oh[jj] = static_cast<uint32_t>(cnt);
}

// ---------------------------------------------------------------------------- 4. keys
// One 16-lane row (a DPP row) per key j, four keys per wavefront, keys taken in their Z-order
// processing order: the queries that selected a key are near it on the curve, so keys that
// run together read overlapping dO rows and L2 serves the repeats.  A key's pairs are a
// contiguous run of records, taken 16 at a time: lane l of the row owns record l of the batch
// (its slot is loaded two batches ahead) and loads the slot's {a_ij, c_ij} and its query's
// record {q_i, i} one batch ahead (both written by the per-query pass at the query's rank).
// The row then walks the batch's records in order: i and a_ij come from the owning lane
// by a DPP row broadcast, every lane loads its chunks of the dO_i row (the loads of kKeyLoads
// records are issued together) and adds a_ij dO_i to its chunks of dv_j; the owning lane adds
// c_ij (q_i - k_j) to the dk sum.  No LDS traffic; the trip counts are uniform over the
// wavefront (the longest of its four keys) and a key's sums run in a fixed order.
constexpr int kKeyRow = kRowLanes;        // lanes per key
constexpr int kKeyLoads = kRowLoads;      // records whose dO loads are issued together
static_assert(kKeyRow % kKeyLoads == 0 && kRowLanes % kRowLoads == 0, "whole load groups");

template <bool BF16, bool O32, int CPL, int U0>
__device__ __forceinline__ void key_records(const typename VecIO<BF16>::elem_t* __restrict__ doh,
                                            int dv, const int (&coff)[CPL], uint32_t io,
                                            float ao, float (&acc)[CPL][VecIO<BF16>::kElems]) {
    using IO = VecIO<BF16>;
    using R = typename IO::raw_t;
    constexpr int E = IO::kElems;
    R raw[kKeyLoads][CPL];
    static_for<0, kKeyLoads>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const uint32_t nm = row_bcast<U0 + u>(io);
#pragma unroll
        for (int c = 0; c < CPL; ++c) raw[u][c] = RowRef<BF16, O32>::load(doh, nm, dv, coff[c]);
    });
    static_for<0, kKeyLoads>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const float a = row_bcast<U0 + u>(ao);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float x[E];
            IO::unpack(raw[u][c], x);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[c][e] += a * x[e];
        }
    });
}

template <bool BF16, bool O32, int CPL>
__global__ void __launch_bounds__(kKeyThreads) zeta_bwd_key_kernel(
    const float* __restrict__ k, const float* __restrict__ gamma,
    const void* __restrict__ dout, const float2* __restrict__ coef,
    const float4* __restrict__ qrec,
    const uint32_t* __restrict__ slots, int slot_stride, const uint32_t* __restrict__ seg_lo,
    const uint32_t* __restrict__ seg_hi, const uint32_t* __restrict__ order, int64_t N,
    int64_t H, int dv, int topk, DivU32 slot_div,
    int64_t P, int64_t tph, int64_t tiles, int64_t per_xcd, float* __restrict__ dk,
    void* __restrict__ dvout) {
    using IO = VecIO<BF16>;
    using T = typename IO::elem_t;
    constexpr int E = IO::kElems;
    const int64_t tile = xcd_tile(blockIdx.x, per_xcd);
    if (tile >= tiles) return;  // uniform over the workgroup
    const int64_t bh = tile / tph;  // uniform: tiles never straddle two (b,h)
    const int lrow = threadIdx.x & (kKeyRow - 1);
    const int64_t pos0 = (tile - bh * tph) * kKeyRows;  // the workgroup's keys
    // The workgroup's keys go to its rows by decreasing pair count, so each wavefront's four
    // keys have similar counts and few of its row slots idle (a wavefront runs as long as its
    // longest key).  Which row sums a key does not change the key's sums.
    __shared__ uint32_t wcount[kKeyRows];
    __shared__ int wkey[kKeyRows];
    if (threadIdx.x < kKeyRows) {
        const int64_t p = pos0 + threadIdx.x;
        const int64_t pc = p < N ? p : N - 1;
        const int64_t jj = order ? static_cast<int64_t>(order[bh * N + pc]) : pc;
        wcount[threadIdx.x] =
            p < N ? seg_hi[bh * (N + 1) + jj] - seg_lo[bh * (N + 1) + jj] : 0u;
    }
    __syncthreads();
    if (threadIdx.x < kKeyRows) {
        const uint32_t c = wcount[threadIdx.x];
        int rank = 0;
#pragma unroll
        for (int u = 0; u < kKeyRows; ++u) {
            const uint32_t cu = wcount[u];
            rank += (cu > c || (cu == c && u < static_cast<int>(threadIdx.x))) ? 1 : 0;
        }
        wkey[rank] = static_cast<int>(threadIdx.x);
    }
    __syncthreads();
    const int64_t pos = pos0 + wkey[threadIdx.x / kKeyRow];
    const bool live = pos < N;
    const int64_t pp = live ? pos : N - 1;  // a row past the end reads a real key, stores nothing
    const int64_t j = order ? static_cast<int64_t>(order[bh * N + pp]) : pp;
    const int64_t row = bh * N + j;
    const int chunks = dv / E;
    const float gm = gamma[bh % H];
    const float k0 = k[3 * row], k1 = k[3 * row + 1], k2 = k[3 * row + 2];
    const uint32_t seg0 = seg_lo[bh * (N + 1) + j];
    const int cnt = live ? static_cast<int>(seg_hi[bh * (N + 1) + j] - seg0) : 0;
    const uint32_t* rh = slots + (bh * P + seg0) * slot_stride;
    const float4* qrh = qrec + bh * N;
    const float2* cf = coef + bh * N * topk;
    const T* doh = static_cast<const T*>(dout) + bh * N * dv;

    float acc[CPL][E];
    int coff[CPL];  // element offset of the lane's chunks (clamped; never stored past the row)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lrow + c * kKeyRow;
        coff[c] = (ch < chunks ? ch : chunks - 1) * E;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[c][e] = 0.0f;
    }
    // the longest of the wavefront's four keys sets the trip counts
    int most = cnt;
    most = max(most, __shfl_xor(most, 16, 64));
    most = max(most, __shfl_xor(most, 32, 64));

    // Records past the key's run repeat its last record with a = 0, so they add 0 * dO_i for
    // a row the key sums anyway (exactly nothing unless that row is not finite, and then the
    // key's sum already is not).  A key with no pairs stores zeros.
    const int last = cnt > 0 ? cnt - 1 : 0;
    auto slot_at = [&](int p) -> uint32_t {
        return cnt > 0 ? rh[(p < last ? p : last) * slot_stride] : 0u;
    };
    // two-deep: while a batch's dO rows load, the next batch's {a, c} and query record and
    // the slot after it are in flight
    uint32_t slot_next = slot_at(lrow);
    float2 ac_next = cf[slot_next];
    float4 q_next = qrh[div_u32(slot_next, slot_div)];  // the slot's query: q_i and i
    if (kKeyRow < most) slot_next = slot_at(lrow + kKeyRow);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
    for (int first = 0; first < most; first += kKeyRow) {  // batches of 16 records
        const int p = first + lrow;
        const bool own = p < cnt;
        const float2 ac = ac_next;
        const float4 qi = q_next;
        if (first + kKeyRow < most) {  // uniform
            ac_next = cf[slot_next];
            q_next = qrh[div_u32(slot_next, slot_div)];
            if (first + 2 * kKeyRow < most) slot_next = slot_at(p + 2 * kKeyRow);
        }
        const float dx = qi.x - k0, dy = qi.y - k1, dz = qi.z - k2;
        const float ao = own ? ac.x : 0.0f;
        const uint32_t nm = RowRef<BF16, O32>::name(__float_as_uint(qi.w), dv);
        static_for<0, kKeyRow / kKeyLoads>([&](auto bc) {
            constexpr int b = decltype(bc)::value * kKeyLoads;
            if (first + b < most)  // uniform
                key_records<BF16, O32, CPL, b>(doh, dv, coff, nm, ao, acc);
        });
        if (own) {
            s0 += ac.y * dx;
            s1 += ac.y * dy;
            s2 += ac.y * dz;
        }
    }
    s0 = group_sum(s0, kKeyRow);
    s1 = group_sum(s1, kKeyRow);
    s2 = group_sum(s2, kKeyRow);
    if (live) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = lrow + c * kKeyRow;
            if (ch < chunks) {
                if (cnt == 0)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[c][e] = 0.0f;
                IO::store(static_cast<T*>(dvout) + row * dv + ch * E, acc[c]);
            }
        }
        if (lrow == 0) {
            // dk_j = (2/gamma^2) sum_i c_ij (q_i - k_j)
            const float f = 2.0f / (gm * gm);
            dk[3 * row] = f * s0;
            dk[3 * row + 1] = f * s1;
            dk[3 * row + 2] = f * s2;
        }
    }
}

// A key's pairs: slots[(segment start + r) * slot_stride], r < seg_hi[j] - seg_lo[j].
struct KeySegments {
    const uint32_t* slots;
    int stride;
    const uint32_t* lo;
    const uint32_t* hi;
};

template <bool BF16, bool O32>
static hipError_t launch_key_o(int64_t BH, int64_t H, int64_t N, int dv, int topk,
                               const float* k, const float* gamma,
                               const void* dout, const BwdBuffers& ws, const KeySegments& sg,
                               const uint32_t* order, float* dk, void* dvout, hipStream_t s) {
    const int chunks = dv / VecIO<BF16>::kElems;
    const int cpl = (chunks + kKeyRow - 1) / kKeyRow;
    const int64_t tph = (N + kKeyRows - 1) / kKeyRows;
    const int64_t tiles = BH * tph;
    const int64_t per = xcd_per(tiles);
    auto kern = cpl <= 1 ? zeta_bwd_key_kernel<BF16, O32, 1>
              : cpl <= 2 ? zeta_bwd_key_kernel<BF16, O32, 2>
              : cpl <= 4 ? zeta_bwd_key_kernel<BF16, O32, 4>
                         : zeta_bwd_key_kernel<BF16, O32, BF16 ? 4 : 8>;  // bf16: <= 64 chunks
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(per * kXcds)), dim3(kKeyThreads), 0, s, k,
                       gamma, dout, ws.coef, ws.qrec, sg.slots, sg.stride, sg.lo, sg.hi, order, N, H, dv,
                       topk,
                       make_div(static_cast<uint32_t>(topk)), ws.P, tph, tiles, per, dk, dvout);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_key(int64_t BH, int64_t H, int64_t N, int dv, int topk,
                             const float* k, const float* gamma,
                             const void* dout, const BwdBuffers& ws, const KeySegments& sg,
                             const uint32_t* order, float* dk, void* dvout, hipStream_t s) {
    if (rows_fit_32(N, dv, sizeof(typename VecIO<BF16>::elem_t)))
        return launch_key_o<BF16, true>(BH, H, N, dv, topk, k, gamma, dout, ws, sg, order, dk, dvout, s);
    return launch_key_o<BF16, false>(BH, H, N, dv, topk, k, gamma, dout, ws, sg, order, dk, dvout, s);
}

// ---------------------------------------------------------------------------- 5. dgamma
// Two fixed-order levels: workgroups sum chunks of kDgChunk per-query terms of a head (8
// loads in flight per thread, then an LDS tree), and one wavefront per head sums the chunk
// partials in chunk order.
constexpr int kDgChunk = 2048;
__global__ void __launch_bounds__(256) zeta_dgamma_partial_kernel(const float* __restrict__ dg_row,
                                                                   int64_t B, int64_t H, int64_t N,
                                                                   int64_t chunks,
                                                                   float* __restrict__ part) {
    __shared__ float red[256];
    const int64_t h = blockIdx.y;
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kDgChunk;
    const int64_t total = B * N;
    float x[kDgChunk / 256];
#pragma unroll
    for (int u = 0; u < kDgChunk / 256; ++u) {  // clamped positions: the loads issue together
        int64_t f = f0 + u * 256 + threadIdx.x;
        f = f < total ? f : total - 1;
        const int64_t b = f / N, i = f - b * N;
        x[u] = dg_row[(b * H + h) * N + i];
    }
#pragma unroll
    for (int u = 0; u < kDgChunk / 256; ++u) keep(x[u]);
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < kDgChunk / 256; ++u)
        if (f0 + u * 256 + threadIdx.x < total) acc += x[u];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[h * chunks + blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(64) zeta_dgamma_final_kernel(const float* __restrict__ part,
                                                                int64_t chunks,
                                                                float* __restrict__ dgamma) {
    const int64_t h = blockIdx.x;
    float acc = 0.0f;
    for (int64_t c = threadIdx.x; c < chunks; c += 64) acc += part[h * chunks + c];
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (threadIdx.x == 0) dgamma[h] = acc;
}

// Up to kDgHeadMax terms per head: one workgroup per head sums them all (each thread its
// strided share, eight loads in flight, then an LDS tree), one launch instead of two.
constexpr int kDgHeadThreads = 1024;
constexpr int64_t kDgHeadMax = int64_t(1) << 18;
__global__ void __launch_bounds__(kDgHeadThreads) zeta_dgamma_head_kernel(
    const float* __restrict__ dg_row, int64_t B, int64_t H, int64_t N, float* __restrict__ dgamma) {
    __shared__ float red[kDgHeadThreads];
    const int64_t h = blockIdx.x;
    const int tid = threadIdx.x;
    float acc = 0.0f;
    for (int64_t b = 0; b < B; ++b) {
        const float* row = dg_row + (b * H + h) * N;
        for (int64_t i0 = 0; i0 < N; i0 += 8 * kDgHeadThreads) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {  // clamped positions: the loads issue together
                const int64_t i = i0 + u * kDgHeadThreads + tid;
                x[u] = row[i < N ? i : N - 1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) keep(x[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u * kDgHeadThreads + tid < N) acc += x[u];
        }
    }
    red[tid] = acc;
    __syncthreads();
    for (int w = kDgHeadThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) dgamma[h] = red[0];
}

int64_t dgamma_chunks(int64_t B, int64_t N) { return (B * N + kDgChunk - 1) / kDgChunk; }

// ---------------------------------------------------------------------------- host
size_t bwd_pairs_per_head(int64_t N, int topk, bool causal) {
    if (!causal) return static_cast<size_t>(N * (N < topk ? N : topk));
    if (N <= topk) return static_cast<size_t>(N * (N + 1) / 2);
    return static_cast<size_t>(int64_t(topk) * (topk + 1) / 2 + (N - topk) * topk);
}

int64_t bwd_tiles_per_head(int64_t items) { return (items + kRadixTile - 1) / kRadixTile; }

bool bwd_records_packed(int64_t N, int topk) {
    // keys below 2^16 (the bucket holds their low byte) and slots below 2^24
    return N <= (int64_t(1) << 16) && N * topk <= (int64_t(1) << 24);
}
static_assert(int64_t(1) << 16 << 8 == int64_t(1) << 24 && kMaxTopK <= 256,
              "keys below 2^16 with at most 256 slots each have slots below 2^24");


// items: slots of pass 0 (N * topk), else the upper bound P of the pairs per (b,h) (the
// grid size; the kernels stop at the device-side count).
template <bool FIRST, bool PACK = false>
static void radix_pass(int64_t BH, const int32_t* idx, const uint2* rin, int64_t items,
                       int64_t stride, int shift, const PairSpec& ps, const BwdBuffers& ws,
                       uint2* rout, hipStream_t s) {
    const int64_t tiles = bwd_tiles_per_head(items);
    dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(BH));
    hipLaunchKernelGGL(zeta_radix_hist_kernel<FIRST>, grid, dim3(kRadixThreads), 0, s, idx, rin,
                       items, ws.counts, stride, shift, tiles, ps, ws.hist);
    hipLaunchKernelGGL(zeta_radix_scan_kernel, dim3(256, static_cast<unsigned>(BH)), dim3(64), 0, s,
                       ws.hist, tiles, ws.totals);
    hipLaunchKernelGGL((zeta_radix_scatter_kernel<FIRST, PACK>), grid, dim3(kRadixThreads), 0, s, idx, rin,
                       items, ws.counts, stride, shift, tiles, ps, ws.hist, ws.totals, ws.P, ws.rank_q, rout);
}

template <bool BF16>
static hipError_t launch_bwd_t(int64_t BH, int64_t H, int64_t N, int dv, int topk, bool causal,
                               const float* q, const float* k, const void* v, const float* gamma,
                               const int32_t* idx, const void* dout, float* dq, float* dk,
                               void* dvout, float* dgamma, const BwdBuffers& ws,
                               const StageEvents& marks, hipStream_t s) {
    const int64_t rows = BH * N;
    marks.record(0, s);
    // the key codes and order follow the query ones in memory (zk = zq + BH N, perm_k =
    // perm_q + BH N): one order build takes both as 2 BH slices
    hipError_t e = launch_encode_order(q, ws.zq, k, ws.zk, BH, N, kPermIdentity, true,
                                       ws.perm_q, ws.ohist, s, ws.rank_q);
    if (e != hipSuccess) return e;
    marks.record(1, s);
    e = launch_query<BF16>(BH, N, H, dv, topk, causal ? 1 : 0, q, k, v, gamma, idx, dout,
                           ws.perm_q, ws.coef, ws.qrec, dq, ws.dg_row, s);
    if (e != hipSuccess) return e;
    marks.record(2, s);

    int bits = 0;
    while ((int64_t(1) << bits) < N) ++bits;
    const PairSpec ps{topk, causal ? 1 : 0, N, make_div(static_cast<uint32_t>(topk))};
    KeySegments sg{};
    if (bits <= 16) {
        // one global pass on the low byte of j writing 4-byte records (N k <= 2^24 here,
        // since topk <= 256), then one workgroup per low-byte bucket
        radix_pass<true, true>(BH, idx, nullptr, N * topk, N * topk, 0, ps, ws, ws.rec0, s);
        uint32_t* sl = reinterpret_cast<uint32_t*>(ws.rec1);
        hipLaunchKernelGGL(zeta_bucket_sort_kernel,
                           dim3(static_cast<unsigned>(N < 256 ? N : 256), static_cast<unsigned>(BH)),
                           dim3(kRadixThreads), 0, s, reinterpret_cast<const uint32_t*>(ws.rec0),
                           ws.totals, N, ws.P, sl, ws.offs, ws.ends);
        sg = KeySegments{sl, 1, ws.offs, ws.ends};
    } else {
        // LSD passes over every byte of j, then the segment starts from the sorted keys
        radix_pass<true>(BH, idx, nullptr, N * topk, N * topk, 0, ps, ws, ws.rec0, s);
        uint2* cur = ws.rec0;
        for (int shift = 8; shift < bits; shift += 8) {
            uint2* nxt = cur == ws.rec0 ? ws.rec1 : ws.rec0;
            radix_pass<false>(BH, nullptr, cur, ws.P, ws.P, shift, ps, ws, nxt, s);
            cur = nxt;
        }
        hipLaunchKernelGGL(zeta_segment_offsets_kernel,
                           dim3(static_cast<unsigned>((ws.P + 255) / 256), static_cast<unsigned>(BH)),
                           dim3(256), 0, s, cur, ws.counts, ws.P, N, ws.offs);
        sg = KeySegments{reinterpret_cast<const uint32_t*>(cur) + 1, 2, ws.offs, ws.offs + 1};
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    marks.record(3, s);
    e = launch_key<BF16>(BH, H, N, dv, topk, k, gamma, dout, ws, sg, ws.perm_k, dk, dvout, s);
    if (e != hipSuccess) return e;
    marks.record(4, s);
    const int64_t dch = dgamma_chunks(BH / H, N);
    if ((BH / H) * N <= kDgHeadMax) {
        hipLaunchKernelGGL(zeta_dgamma_head_kernel, dim3(static_cast<unsigned>(H)),
                           dim3(kDgHeadThreads), 0, s, ws.dg_row, BH / H, H, N, dgamma);
    } else {
        hipLaunchKernelGGL(zeta_dgamma_partial_kernel,
                           dim3(static_cast<unsigned>(dch), static_cast<unsigned>(H)), dim3(256), 0,
                           s, ws.dg_row, BH / H, H, N, dch, ws.dg_part);
        hipLaunchKernelGGL(zeta_dgamma_final_kernel, dim3(static_cast<unsigned>(H)), dim3(64), 0, s,
                           ws.dg_part, dch, dgamma);
    }
    marks.record(5, s);
    return hipGetLastError();
}

hipError_t launch_bwd(int64_t BH, int64_t H, int64_t N, int64_t dv, int topk, bool causal, bool bf16,
                      const float* q, const float* k, const void* v, const float* gamma,
                      const int32_t* idx, const void* dout, float* dq, float* dk, void* dvout,
                      float* dgamma, const BwdBuffers& ws, const StageEvents& marks,
                      hipStream_t s) {
    if (BH * N <= 0) return hipSuccess;
    if (bf16)
        return launch_bwd_t<true>(BH, H, N, (int)dv, topk, causal, q, k, v, gamma, idx, dout, dq, dk, dvout, dgamma, ws, marks, s);
    return launch_bwd_t<false>(BH, H, N, (int)dv, topk, causal, q, k, v, gamma, idx, dout, dq, dk, dvout, dgamma, ws, marks, s);
}

}  // namespace zeta
