// gather.hip -- Adaptive Cauchy-softmax weighted gather of the selected value rows.
//
// "ZETA: Leveraging Z-order Curves for Efficient Top-k Attention", rebuttal page, answer
// W3/A3 ("Justification for Euclidean Distance Claim": similarity is the Euclidean
// distance) and answer W2/A2 ("Discussion on its robustness": Cauchy softmax with a
// trainable scale gamma acting as a temperature; gamma = 1 gives the Student-t kernel):
//     s_ij = 1 / (1 + ||q_i - k_j||^2 / gamma_h^2),   o_i = sum_j s_ij v_j / sum_j s_ij
// over the k selected keys only ("the use of the top-k tokens for attention" in W3/A3).
//
// HBM-bound gather: per query k value rows of dv elements (k * dv * |v| bytes) dominate.
// Queries are taken in Z-order buckets (order.hip) with an XCD-aware tile mapping, so the
// rows that concurrent queries select overlap and are served from L2.
// Each lane keeps fp32 accumulators for its 16-byte chunk(s) of the row, so every selected
// row is read with coalesced 16 B-per-lane loads.  The output is rounded once to the value
// dtype.
#include "zeta_internal.hpp"
#include "vec_io.hpp"
#include "xlane.hpp"

namespace zeta {

// One 16-lane row (a DPP row) per query, four queries per wavefront; a workgroup's 16 queries
// belong to one (b,h), so the slice bases are uniform.  Lane l owns slots l, 16 + l, ...: it
// loads their indices and key rows and computes the weights, so all of the row's index and key
// loads are in flight at once.  A slot is selected when it lies within min(k, keys the query
// may use) and holds an index >= 0 (the exact selection fills all of them; the chunked and
// several-curve selections can leave -1 there); an unselected slot carries weight -1 and names
// row 0, and a query with no selected slot outputs zero.  The row then walks the slots in
// order: the value row's name and the weight come from the owning lane by a DPP row broadcast,
// every lane loads its 16-byte chunk(s) of the value row (the loads of kGatherLoads slots are
// issued together, none waits on another load) and accumulates in fp32.
constexpr int kGatherLanes = 16;
constexpr int kGatherLoads = 8;
// Large workgroups: the 64 queries of one workgroup are neighbours on the curve and share
// one CU's L1, which then serves more of their selected rows.
constexpr int kGatherThreads = 1024;
constexpr int kGatherRows = kGatherThreads / kGatherLanes;  // queries per workgroup

template <bool BF16, bool O32, int CPL, int L0>
__device__ __forceinline__ void gather_slots(const typename VecIO<BF16>::elem_t* __restrict__ vh,
                                             int dv, const int (&coff)[CPL], uint32_t jo, float so,
                                             float (&acc)[CPL][VecIO<BF16>::kElems]) {
    using IO = VecIO<BF16>;
    using Ref = RowRef<BF16, O32>;
    using R = typename IO::raw_t;
    constexpr int E = IO::kElems;
    R raw[kGatherLoads][CPL];
    static_for<0, kGatherLoads>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        const uint32_t nm = row_bcast<L0 + w>(jo);
#pragma unroll
        for (int c = 0; c < CPL; ++c) raw[w][c] = Ref::load(vh, nm, dv, coff[c]);
    });
    static_for<0, kGatherLoads>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        const float s = row_bcast<L0 + w>(so);
#pragma unroll
        for (int c = 0; c < CPL; ++c) keep(raw[w][c]);  // the load stays ahead of the test
        if (!(s < 0.0f)) {  // slot selected (a NaN weight is summed and propagates)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float x[E];
                IO::unpack(raw[w][c], x);
#pragma unroll
                for (int e = 0; e < E; ++e) acc[c][e] += s * x[e];
            }
        }
    });
}

template <bool BF16, bool O32, int CPL, int U, bool MULTI>
__global__ void __launch_bounds__(kGatherThreads) zeta_cauchy_gather_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ gamma, const int32_t* __restrict__ idx,
    const uint32_t* __restrict__ order, void* __restrict__ out, int64_t N, int64_t H, int dv,
    int topk, int causal, int64_t tph, int64_t tiles, int64_t per_xcd) {
    using IO = VecIO<BF16>;
    using Ref = RowRef<BF16, O32>;
    using T = typename IO::elem_t;
    constexpr int E = IO::kElems;
    constexpr int kBatch = U * kGatherLanes;  // slots per batch
    const int64_t tile = xcd_tile(blockIdx.x, per_xcd);
    if (tile >= tiles) return;  // uniform over the workgroup
    const int64_t bh = tile / tph;  // uniform: tiles never straddle two (b,h)
    const int lrow = threadIdx.x & (kGatherLanes - 1);
    const int64_t pos = (tile - bh * tph) * kGatherRows + threadIdx.x / kGatherLanes;
    const bool live = pos < N;
    const int64_t pp = live ? pos : N - 1;  // a row past the end reads a real query, stores nothing
    const int chunks = dv / E;
    const int64_t i = order ? static_cast<int64_t>(order[bh * N + pp]) : pp;
    const int64_t row = bh * N + i;
    const float g = gamma[bh % H];
    const float inv_g2 = 1.0f / (g * g);
    const float q0 = q[3 * row], q1 = q[3 * row + 1], q2 = q[3 * row + 2];
    // slots that may hold a selection: min(k, keys the query may use); empty ones hold -1
    const int64_t nk = causal ? i + 1 : N;
    const int m = live ? static_cast<int>(nk < topk ? nk : topk) : 0;
    const int64_t jmax = nk - 1;
    const int32_t* ir = idx + row * topk;
    const float* kh = k + bh * N * 3;
    const T* vh = static_cast<const T*>(v) + bh * N * dv;
    // the longest selection among the wavefront's four queries sets the trip count
    int most = m;
    most = max(most, __shfl_xor(most, 16, 64));
    most = max(most, __shfl_xor(most, 32, 64));

    float acc[CPL][E];
    int coff[CPL];  // element offset of the lane's chunks (clamped; never stored past the row)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lrow + c * kGatherLanes;
        coff[c] = (ch < chunks ? ch : chunks - 1) * E;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[c][e] = 0.0f;
    }
    float ssum = 0.0f, nsel = 0.0f;
    // Slots are taken kBatch at a time (one batch unless k > 64): the weights are summed
    // unnormalised and the output is scaled by 1 / S once at the end.
    const int batches = MULTI ? (most + kBatch - 1) / kBatch : 1;
    for (int bt = 0; bt < batches; ++bt) {
        const int sb = bt * kBatch;  // first slot of the batch
        // the index and key-row loads read clamped positions and are held live before any
        // test, so the loads of a kind are in flight together
        int32_t jr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = sb + lrow + u * kGatherLanes;
            jr[u] = ir[r < topk ? r : topk - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) keep(jr[u]);
        bool sel[U];
        Point3 kp[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            sel[u] = sb + lrow + u * kGatherLanes < m && jr[u] >= 0;
            // a selection has j <= jmax; clamping keeps every access in bounds
            jr[u] = sel[u] ? (jr[u] > jmax ? static_cast<int32_t>(jmax) : jr[u]) : 0;
            kp[u] = load_point(kh, jr[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) keep(kp[u]);
        uint32_t jo[U];
        float so[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            jo[u] = 0;
            so[u] = -1.0f;
            if (sel[u]) {
                const float d0 = q0 - kp[u].x, d1 = q1 - kp[u].y, d2 = q2 - kp[u].z;
                jo[u] = Ref::name(jr[u], dv);
                so[u] = 1.0f / (1.0f + (d0 * d0 + d1 * d1 + d2 * d2) * inv_g2);
                ssum += so[u];
                nsel += 1.0f;
            }
        }
        const int left = most - sb;  // slots of this batch any query of the wavefront uses
        static_for<0, U>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            if (u * kGatherLanes < left) {
                static_for<0, kGatherLanes / kGatherLoads>([&](auto bc) {
                    constexpr int b = decltype(bc)::value;
                    if (u * kGatherLanes + b * kGatherLoads < left)
                        gather_slots<BF16, O32, CPL, b * kGatherLoads>(vh, dv, coff, jo[u], so[u],
                                                                       acc);
                });
            }
        });
    }
    ssum = group_sum(ssum, kGatherLanes);
    nsel = group_sum(nsel, kGatherLanes);

    if (live) {
        const float inv_S = nsel > 0.0f ? 1.0f / ssum : 0.0f;  // an empty selection outputs 0
        T* orow = static_cast<T*>(out) + row * dv;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = lrow + c * kGatherLanes;
            if (ch < chunks) {
                float x[E];
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = acc[c][e] * inv_S;
                IO::store(orow + ch * E, x);
            }
        }
    }
}

template <bool BF16, bool O32, int CPL>
static hipError_t launch_gather_c(int64_t BH, int64_t N, int64_t H, int dv, int topk,
                                  int causal, const float* q, const float* k, const void* v,
                                  const float* gamma, const int32_t* idx, const uint32_t* order,
                                  void* out, hipStream_t s) {
    const int64_t tph = (N + kGatherRows - 1) / kGatherRows;
    const int64_t tiles = BH * tph;
    const int64_t per = xcd_per(tiles);
    // slots per lane: 1, 2 or 4 in one batch; above 64 slots, batches of 4 per lane
    const int u = (topk + kGatherLanes - 1) / kGatherLanes;
    auto kern = u <= 1 ? zeta_cauchy_gather_kernel<BF16, O32, CPL, 1, false>
              : u <= 2 ? zeta_cauchy_gather_kernel<BF16, O32, CPL, 2, false>
              : u <= 4 ? zeta_cauchy_gather_kernel<BF16, O32, CPL, 4, false>
                       : zeta_cauchy_gather_kernel<BF16, O32, CPL, 4, true>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(per * kXcds)), dim3(kGatherThreads), 0, s, q, k, v,
                       gamma, idx, order, out, N, H, dv, topk, causal, tph, tiles, per);
    return hipGetLastError();
}

template <bool BF16, int CPL>
static hipError_t launch_gather_o(int64_t BH, int64_t N, int64_t H, int dv, int topk,
                                  int causal, const float* q, const float* k, const void* v,
                                  const float* gamma, const int32_t* idx, const uint32_t* order,
                                  void* out, hipStream_t s) {
    if (rows_fit_32(N, dv, sizeof(typename VecIO<BF16>::elem_t)))
        return launch_gather_c<BF16, true, CPL>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, order, out, s);
    return launch_gather_c<BF16, false, CPL>(BH, N, H, dv, topk, causal, q, k, v, gamma, idx, order, out, s);
}

hipError_t launch_gather(int64_t BH, int64_t H, int64_t N, int64_t dv, int topk, bool causal,
                         bool bf16, const float* q, const float* k, const void* v,
                         const float* gamma, const int32_t* idx, const uint32_t* order, void* out,
                         hipStream_t s) {
    const int cz = causal ? 1 : 0;
    if (BH * N <= 0) return hipSuccess;
    const int cpl = static_cast<int>((dv / (bf16 ? 8 : 4) + kGatherLanes - 1) / kGatherLanes);
    const int d = static_cast<int>(dv);
    if (bf16) {  // bf16 rows have <= 64 chunks
        if (cpl <= 1) return launch_gather_o<true, 1>(BH, N, H, d, topk, cz, q, k, v, gamma, idx, order, out, s);
        if (cpl <= 2) return launch_gather_o<true, 2>(BH, N, H, d, topk, cz, q, k, v, gamma, idx, order, out, s);
        return launch_gather_o<true, 4>(BH, N, H, d, topk, cz, q, k, v, gamma, idx, order, out, s);
    }
    if (cpl <= 1) return launch_gather_o<false, 1>(BH, N, H, d, topk, cz, q, k, v, gamma, idx, order, out, s);
    if (cpl <= 2) return launch_gather_o<false, 2>(BH, N, H, d, topk, cz, q, k, v, gamma, idx, order, out, s);
    if (cpl <= 4) return launch_gather_o<false, 4>(BH, N, H, d, topk, cz, q, k, v, gamma, idx, order, out, s);
    return launch_gather_o<false, 8>(BH, N, H, d, topk, cz, q, k, v, gamma, idx, order, out, s);
}

}  // namespace zeta
