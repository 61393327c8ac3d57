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
//   1. per-query pass: recompute s, gather v rows for g, write the query's 1/S_i and D_i,
//      dq_i and the query's dgamma term;
//   2. selection transpose: stable LSD radix sort (8-bit digits) of the pairs of every (b,h)
//      by j, carrying 8-byte records {j, i}; queries stay ascending inside a key's segment;
//   3. segment starts offs[j] from the sorted keys;
//   4. per-key pass (keys in Z-order): each key recomputes s_ij, g_ij = dO_i . v_j (it reads the dO_i rows for
//      dv_j anyway), a_ij and c_ij from the query's 1/S_i and D_i, and reduces its segment
//      in a fixed order (dv, dk);
//   5. dgamma: two-level fixed-order reduction per head over the batch and the queries.
// Recomputing a and c on the key side keeps the sorted records at 8 bytes (half of what
// carrying a and c would take) and saves writing and re-reading two per-pair arrays.
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

struct PairSpec {
    int topk;
    int causal;
    int64_t N;
};

__device__ __forceinline__ bool pair_item(const int32_t* __restrict__ idx, int64_t e,
                                          const PairSpec& ps, uint32_t& key) {
    const uint32_t i = static_cast<uint32_t>(e) / static_cast<uint32_t>(ps.topk);
    const uint32_t r = static_cast<uint32_t>(e) - i * static_cast<uint32_t>(ps.topk);
    const int64_t nk = ps.causal ? static_cast<int64_t>(i) + 1 : ps.N;
    if (r >= nk) return false;  // slot beyond min(topk, nk)
    const int32_t j = idx[e];
    if (j < 0) return false;    // no selection in this slot
    key = static_cast<uint32_t>(clamp_index(j, nk - 1));
    return true;
}


// ---------------------------------------------------------------------------- 1. queries
// One 16-lane row (a DPP row) per query i, four queries per wavefront, taken in the Z-order
// processing order.  Lane l owns slots l, 16 + l, ...: it loads their indices and key rows
// and forms s, the distance terms and later a, c and the dq / dgamma terms.  The row keeps
// its chunks of dO_i in registers and walks the slots in order: the index comes from the
// owning lane by a DPP row broadcast, every lane loads its chunks of the v_j row (the loads
// of kRowLoads slots are issued together) and a DPP butterfly over the row completes
// g_ij = dO_i . v_j, which the owning lane keeps.
constexpr int kRowLanes = 16;  // lanes per query or key
constexpr int kRowLoads = 8;   // rows whose loads are issued together

template <bool BF16, int CPL, int L0>
__device__ __forceinline__ void query_slots(const typename VecIO<BF16>::elem_t* __restrict__ vh,
                                            int dv, const int (&coff)[CPL], int32_t jo,
                                            const float (&go)[CPL][VecIO<BF16>::kElems],
                                            int lrow, float& gmine) {
    using IO = VecIO<BF16>;
    using R = typename IO::raw_t;
    constexpr int E = IO::kElems;
    R raw[kRowLoads][CPL];
    static_for<0, kRowLoads>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        const int32_t j = static_cast<int32_t>(row_bcast<L0 + w>(static_cast<uint32_t>(jo)));
        const int64_t jr = j < 0 ? 0 : j;  // an empty slot reads key 0's row; its g is unused
#pragma unroll
        for (int c = 0; c < CPL; ++c) raw[w][c] = IO::load_raw(vh + jr * dv + coff[c]);
    });
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
        const float g = group_sum(part, kRowLanes);
        if (lrow == L0 + w) gmine = g;
    });
}

template <bool BF16, int CPL, int U>
__global__ void __launch_bounds__(256) zeta_bwd_query_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ gamma, const int32_t* __restrict__ idx,
    const void* __restrict__ dout, const uint32_t* __restrict__ order, int64_t rows, int64_t N,
    int64_t H, int dv, int topk, int causal, int64_t tiles, int64_t per_xcd,
    float2* __restrict__ qstat, float* __restrict__ dq, float* __restrict__ dg_row) {
    using IO = VecIO<BF16>;
    using T = typename IO::elem_t;
    constexpr int E = IO::kElems;
    const int64_t tile = xcd_tile(blockIdx.x, per_xcd);
    if (tile >= tiles) return;  // uniform over the workgroup
    const int lrow = threadIdx.x & (kRowLanes - 1);
    const int64_t t = tile * (blockDim.x / kRowLanes) + threadIdx.x / kRowLanes;
    const bool live = t < rows;
    const int64_t tt = live ? t : rows - 1;  // a row past the end reads a real query, stores nothing
    const int chunks = dv / E;
    const int64_t bh = tt / N;
    const int64_t i = order ? static_cast<int64_t>(order[tt]) : tt - bh * N;
    const int64_t row = bh * N + i;
    const float g = gamma[bh % H];
    const float inv_g2 = 1.0f / (g * g);
    const float q0 = q[3 * row], q1 = q[3 * row + 1], q2 = q[3 * row + 2];
    const int64_t nk = causal ? i + 1 : N;  // keys the query may use
    const int m = live ? static_cast<int>(nk < topk ? nk : topk) : 0;
    const int32_t* ir = idx + row * topk;
    const float* kh = k + bh * N * 3;
    const T* vh = static_cast<const T*>(v) + bh * N * dv;

    float go[CPL][E];
    int coff[CPL];  // element offset of the lane's chunks (clamped; chunks past the row meet go = 0)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lrow + c * kRowLanes;
        coff[c] = (ch < chunks ? ch : chunks - 1) * E;
#pragma unroll
        for (int e = 0; e < E; ++e) go[c][e] = 0.0f;
        if (ch < chunks) IO::load(static_cast<const T*>(dout) + row * dv + ch * E, go[c]);
    }

    int32_t jo[U];
    float so[U], dx[U], dy[U], dz[U], gg[U];
    float ssum = 0.0f, nsel = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = lrow + u * kRowLanes;
        jo[u] = -1;  // not selected: never summed
        so[u] = dx[u] = dy[u] = dz[u] = gg[u] = 0.0f;
        const int32_t jr = r < m ? ir[r] : -1;
        if (jr >= 0) {
            const int32_t j = static_cast<int32_t>(clamp_index(jr, nk - 1));
            jo[u] = j;
            nsel += 1.0f;
            dx[u] = q0 - kh[3 * j];
            dy[u] = q1 - kh[3 * j + 1];
            dz[u] = q2 - kh[3 * j + 2];
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
                    query_slots<BF16, CPL, b * kRowLoads>(vh, dv, coff, jo[u], go, lrow, gg[u]);
            });
        }
    });

    float tsum = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (jo[u] >= 0) tsum += so[u] * gg[u];
    const float inv_S = nsel > 0.0f ? 1.0f / S : 0.0f;  // an empty selection passes no gradient
    const float D = group_sum(tsum, kRowLanes) * inv_S;

    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, ag = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (jo[u] >= 0) {
            const float a = so[u] * inv_S;
            const float c = a * so[u] * (gg[u] - D);
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
        qstat[row] = make_float2(inv_S, D);
    }
}

template <bool BF16, int CPL>
static hipError_t launch_query_c(int64_t rows, int64_t N, int64_t H, int dv, int topk,
                                 int causal, const float* q, const float* k, const void* v,
                                 const float* gamma, const int32_t* idx, const void* dout,
                                 const uint32_t* order, float2* qstat, float* dq, float* dg_row,
                                 hipStream_t s) {
    const int64_t tiles = (rows + (256 / kRowLanes) - 1) / (256 / kRowLanes);
    const int64_t per = xcd_per(tiles);
    const int u = (topk + kRowLanes - 1) / kRowLanes;  // slots per lane (<= 4)
    auto kern = u <= 1 ? zeta_bwd_query_kernel<BF16, CPL, 1>
              : u <= 2 ? zeta_bwd_query_kernel<BF16, CPL, 2>
                       : zeta_bwd_query_kernel<BF16, CPL, 4>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(per * kXcds)), dim3(256), 0, s, q, k, v,
                       gamma, idx, dout, order, rows, N, H, dv, topk, causal, tiles, per, qstat, dq,
                       dg_row);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_query(int64_t rows, int64_t N, int64_t H, int dv, int topk, int causal,
                               const float* q, const float* k, const void* v, const float* gamma,
                               const int32_t* idx, const void* dout, const uint32_t* order,
                               float2* qstat, float* dq, float* dg_row, hipStream_t s) {
    const int cpl = (dv / VecIO<BF16>::kElems + kRowLanes - 1) / kRowLanes;
    if (cpl <= 1)
        return launch_query_c<BF16, 1>(rows, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, qstat, dq, dg_row, s);
    if (cpl <= 2)
        return launch_query_c<BF16, 2>(rows, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, qstat, dq, dg_row, s);
    if (BF16 || cpl <= 4)  // bf16 rows have <= 64 chunks
        return launch_query_c<BF16, 4>(rows, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, qstat, dq, dg_row, s);
    return launch_query_c<BF16, BF16 ? 4 : 8>(rows, N, H, dv, topk, causal, q, k, v, gamma, idx, dout, order, qstat, dq, dg_row, s);
}

// ---------------------------------------------------------------------------- 2. transpose
// Every pair travels through the sort as one 8-byte record {j, i}.  Pass 0 reads the
// selection in pair order (coalesced) and builds the records; later passes move records.
// The key kernel then reads each key's pairs as one contiguous run of records.
template <bool FIRST>
__device__ __forceinline__ bool load_pair(const int32_t* __restrict__ idx,
                                          const uint2* __restrict__ rin, int64_t e,
                                          const PairSpec& ps, uint2& rec) {
    if (FIRST) {
        uint32_t key;
        if (!pair_item(idx, e, ps, key)) return false;
        rec = make_uint2(key, static_cast<uint32_t>(e) / static_cast<uint32_t>(ps.topk));
        return true;
    }
    rec = rin[e];
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
    uint32_t keys[kRadixItems];
    bool valid[kRadixItems];
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it) {
        const int64_t e = t0 + it * kRadixThreads + threadIdx.x;
        valid[it] = false;
        keys[it] = 0;
        if (e < items) {
            if (FIRST)
                valid[it] = pair_item(idx + bh * in_stride, e, ps, keys[it]);
            else {
                valid[it] = true;
                keys[it] = rin[bh * in_stride + e].x;
            }
        }
    }
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it)
        if (valid[it]) atomicAdd(&cnt[(keys[it] >> shift) & 255u], 1u);
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
template <bool FIRST>
__global__ void __launch_bounds__(kRadixThreads) zeta_radix_scatter_kernel(
    const int32_t* __restrict__ idx, const uint2* __restrict__ rin, int64_t slots,
    uint32_t* __restrict__ counts, int64_t in_stride, int shift, int64_t tiles, PairSpec ps,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ totals, int64_t P,
    uint2* __restrict__ rout) {
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
#pragma unroll
        for (int it = 0; it < kRadixItems; ++it) {
            const int64_t e = t0 + it * 64 + lane;
            rec[it] = make_uint2(0, 0);
            if (e < items && load_pair<FIRST>(idx + off, rin + off, e, ps, rec[it]))
                okmask |= 1u << it;
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
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (digit >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
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
#pragma unroll
    for (int it = 0; it < kRadixItems; ++it) {
        const int t = it * kRadixThreads + tid;  // slot in the staged tile
        if (t < static_cast<int>(tile_items)) {
            const uint2 r = stage[t];
            out[delta[(r.x >> shift) & 255u] + t] = r;
        }
    }
}

// ---------------------------------------------------------------------------- 3. offsets
// offs[j] = first record of key j (records sorted by key), offs[N] = number of pairs.
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
// contiguous run of records, taken kKeyBatch at a time: lane l of the row owns records l and
// 16 + l of the batch, loads their q_i and the query's {1/S_i, D_i} and forms s_ij, a_ij and
// a_ij s_ij.  The row then walks the batch's records in order: i and a_ij come from the owning
// lane by a DPP row broadcast, every lane loads its chunks of the dO_i row (the loads of
// kKeyLoads records are issued together), adds a_ij dO_i to its chunks of dv_j and its part
// of g_ij = dO_i . v_j, and a DPP butterfly over the row completes g_ij, which the owning lane
// keeps for c_ij and the dk term.  No LDS traffic; the trip counts are uniform over the
// wavefront (the longest of its four keys) and a key's sums run in a fixed order.
constexpr int kKeyRow = kRowLanes;        // lanes per key
constexpr int kKeyRecs = 2;               // records per lane per batch
constexpr int kKeyBatch = kKeyRow * kKeyRecs;
constexpr int kKeyLoads = kRowLoads;      // records whose dO loads are issued together
static_assert(kKeyRow % kKeyLoads == 0 && kRowLanes % kRowLoads == 0, "whole load groups");

template <bool BF16, int CPL, int U0>
__device__ __forceinline__ void key_records(const typename VecIO<BF16>::elem_t* __restrict__ doh,
                                            int dv, const int (&coff)[CPL], uint32_t io,
                                            float ao, int lrow, int left, float (&vj)[CPL][VecIO<BF16>::kElems],
                                            float (&acc)[CPL][VecIO<BF16>::kElems], float& gmine) {
    using IO = VecIO<BF16>;
    using R = typename IO::raw_t;
    constexpr int E = IO::kElems;
    R raw[kKeyLoads][CPL];
    static_for<0, kKeyLoads>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const int64_t i = row_bcast<U0 + u>(io);
#pragma unroll
        for (int c = 0; c < CPL; ++c) raw[u][c] = IO::load_raw(doh + i * dv + coff[c]);
    });
    static_for<0, kKeyLoads>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const float a = row_bcast<U0 + u>(ao);
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float x[E];
            IO::unpack(raw[u][c], x);
#pragma unroll
            for (int e = 0; e < E; ++e) part += x[e] * vj[c][e];
            if (U0 + u < left) {
#pragma unroll
                for (int e = 0; e < E; ++e) acc[c][e] += a * x[e];
            }
        }
        const float g = group_sum(part, kKeyRow);
        if (lrow == U0 + u) gmine = g;
    });
}

template <bool BF16, int CPL>
__global__ void __launch_bounds__(256) zeta_bwd_key_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ gamma, const void* __restrict__ dout,
    const float2* __restrict__ qstat, const uint2* __restrict__ recs,
    const uint32_t* __restrict__ offs, const uint32_t* __restrict__ order, int64_t rows,
    int64_t N, int64_t H, int dv, int64_t P, int64_t tiles, int64_t per_xcd,
    float* __restrict__ dk, void* __restrict__ dvout) {
    using IO = VecIO<BF16>;
    using T = typename IO::elem_t;
    constexpr int E = IO::kElems;
    const int64_t tile = xcd_tile(blockIdx.x, per_xcd);
    if (tile >= tiles) return;  // uniform over the workgroup
    const int lane64 = threadIdx.x & 63;
    const int lrow = lane64 & (kKeyRow - 1);
    const int64_t t = tile * (blockDim.x / kKeyRow) + threadIdx.x / kKeyRow;  // processing order
    const bool live = t < rows;
    const int64_t tt = live ? t : rows - 1;  // a row past the end reads a real key, stores nothing
    const int64_t row = order ? (tt / N) * N + order[tt] : tt;
    const int chunks = dv / E;
    const int64_t bh = row / N;
    const int64_t j = row - bh * N;
    const float gm = gamma[bh % H];
    const float inv_g2 = 1.0f / (gm * gm);
    const float k0 = k[3 * row], k1 = k[3 * row + 1], k2 = k[3 * row + 2];
    const uint32_t seg0 = offs[bh * (N + 1) + j];
    const int cnt = live ? static_cast<int>(offs[bh * (N + 1) + j + 1] - seg0) : 0;
    const uint2* rh = recs + bh * P + seg0;
    const float* qh = q + bh * N * 3;
    const float2* sh = qstat + bh * N;
    const T* doh = static_cast<const T*>(dout) + bh * N * dv;

    float vj[CPL][E], acc[CPL][E];
    int coff[CPL];  // element offset of the lane's chunks (clamped; chunks past the row meet vj = 0)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lrow + c * kKeyRow;
        coff[c] = (ch < chunks ? ch : chunks - 1) * E;
#pragma unroll
        for (int e = 0; e < E; ++e) vj[c][e] = acc[c][e] = 0.0f;
        if (ch < chunks) IO::load(static_cast<const T*>(v) + row * dv + ch * E, vj[c]);
    }
    // the longest of the wavefront's four keys sets the trip counts
    int most = cnt;
    most = max(most, __shfl_xor(most, 16, 64));
    most = max(most, __shfl_xor(most, 32, 64));

    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
    for (int base = 0; base < most; base += kKeyBatch) {
#pragma unroll
        for (int r = 0; r < kKeyRecs; ++r) {
            const int first = base + r * kKeyRow;  // the batch's records r*16 .. r*16+15
            if (first >= most) break;               // uniform
            const int p = first + lrow;
            const bool own = p < cnt;
            // records past the key's run name query 0 (inside the buffers) and carry a = 0
            const uint32_t io = own ? rh[p].y : 0u;
            const float dx = qh[3 * io] - k0, dy = qh[3 * io + 1] - k1, dz = qh[3 * io + 2] - k2;
            const float2 st = sh[io];
            const float sv = 1.0f / (1.0f + (dx * dx + dy * dy + dz * dz) * inv_g2);
            const float ao = own ? sv * st.x : 0.0f;
            const int left = cnt - first;  // records of this key from position `first` on
            float gmine = 0.0f;
            static_for<0, kKeyRow / kKeyLoads>([&](auto bc) {
                constexpr int b = decltype(bc)::value * kKeyLoads;
                if (first + b < most)  // uniform
                    key_records<BF16, CPL, b>(doh, dv, coff, io, ao, lrow, left, vj, acc, gmine);
            });
            if (own) {
                const float c = ao * sv * (gmine - st.y);
                s0 += c * dx;
                s1 += c * dy;
                s2 += c * dz;
            }
        }
    }
    s0 = group_sum(s0, kKeyRow);
    s1 = group_sum(s1, kKeyRow);
    s2 = group_sum(s2, kKeyRow);
    if (live) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = lrow + c * kKeyRow;
            if (ch < chunks) IO::store(static_cast<T*>(dvout) + row * dv + ch * E, acc[c]);
        }
        if (lrow == 0) {
            // dk_j = (2/gamma^2) sum_i c_ij (q_i - k_j)
            const float f = 2.0f * inv_g2;
            dk[3 * row] = f * s0;
            dk[3 * row + 1] = f * s1;
            dk[3 * row + 2] = f * s2;
        }
    }
}

template <bool BF16>
static hipError_t launch_key(int64_t BH, int64_t H, int64_t N, int dv, const float* q,
                             const float* k, const void* v, const float* gamma, const void* dout,
                             const BwdBuffers& ws, const uint2* recs, const uint32_t* order,
                             float* dk, void* dvout, hipStream_t s) {
    const int64_t rows = BH * N;
    const int chunks = dv / VecIO<BF16>::kElems;
    const int cpl = (chunks + kKeyRow - 1) / kKeyRow;
    const int64_t tiles = (rows + (256 / kKeyRow) - 1) / (256 / kKeyRow);
    const int64_t per = xcd_per(tiles);
    auto kern = cpl <= 1 ? zeta_bwd_key_kernel<BF16, 1>
              : cpl <= 2 ? zeta_bwd_key_kernel<BF16, 2>
              : cpl <= 4 ? zeta_bwd_key_kernel<BF16, 4>
                         : zeta_bwd_key_kernel<BF16, BF16 ? 4 : 8>;  // bf16 rows have <= 64 chunks
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(per * kXcds)), dim3(256), 0, s, q, k, v,
                       gamma, dout, ws.qstat, recs, ws.offs, order, rows, N, H, dv, ws.P, tiles,
                       per, dk, dvout);
    return hipGetLastError();
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
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < kDgChunk / 256; ++u) {
        const int64_t f = f0 + u * 256 + threadIdx.x;
        if (f < total) {
            const int64_t b = f / N, i = f - b * N;
            acc += dg_row[(b * H + h) * N + i];
        }
    }
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

int64_t dgamma_chunks(int64_t B, int64_t N) { return (B * N + kDgChunk - 1) / kDgChunk; }

// ---------------------------------------------------------------------------- host
size_t bwd_pairs_per_head(int64_t N, int topk, bool causal) {
    if (!causal) return static_cast<size_t>(N * (N < topk ? N : topk));
    if (N <= topk) return static_cast<size_t>(N * (N + 1) / 2);
    return static_cast<size_t>(int64_t(topk) * (topk + 1) / 2 + (N - topk) * topk);
}

int64_t bwd_tiles_per_head(int64_t items) { return (items + kRadixTile - 1) / kRadixTile; }

// items: slots of pass 0 (N * topk), else the upper bound P of the pairs per (b,h) (the
// grid size; the kernels stop at the device-side count).
template <bool FIRST>
static void radix_pass(int64_t BH, const int32_t* idx, const uint2* rin, int64_t items,
                       int64_t stride, int shift, const PairSpec& ps, const BwdBuffers& ws,
                       uint2* rout, hipStream_t s) {
    const int64_t tiles = bwd_tiles_per_head(items);
    dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(BH));
    hipLaunchKernelGGL(zeta_radix_hist_kernel<FIRST>, grid, dim3(kRadixThreads), 0, s, idx, rin,
                       items, ws.counts, stride, shift, tiles, ps, ws.hist);
    hipLaunchKernelGGL(zeta_radix_scan_kernel, dim3(256, static_cast<unsigned>(BH)), dim3(64), 0, s,
                       ws.hist, tiles, ws.totals);
    hipLaunchKernelGGL(zeta_radix_scatter_kernel<FIRST>, grid, dim3(kRadixThreads), 0, s, idx, rin,
                       items, ws.counts, stride, shift, tiles, ps, ws.hist, ws.totals, ws.P, rout);
}

template <bool BF16>
static hipError_t launch_bwd_t(int64_t BH, int64_t H, int64_t N, int dv, int topk, bool causal,
                               const float* q, const float* k, const void* v, const float* gamma,
                               const int32_t* idx, const void* dout, float* dq, float* dk,
                               void* dvout, float* dgamma, const BwdBuffers& ws,
                               const StageEvents& marks, hipStream_t s) {
    const int64_t rows = BH * N;
    marks.record(0, s);
    hipError_t e = launch_encode(q, rows, ws.zq, s);
    if (e == hipSuccess) e = launch_order(BH, N, ws.zq, ws.perm_q, ws.ohist, s);
    if (e == hipSuccess) e = launch_encode(k, rows, ws.zk, s);
    if (e == hipSuccess) e = launch_order(BH, N, ws.zk, ws.perm_k, ws.ohist, s);
    if (e != hipSuccess) return e;
    marks.record(1, s);
    e = launch_query<BF16>(rows, N, H, dv, topk, causal ? 1 : 0, q, k, v, gamma, idx, dout,
                           ws.perm_q, ws.qstat,
                           dq, ws.dg_row, s);
    if (e != hipSuccess) return e;
    marks.record(2, s);

    int bits = 0;
    while ((int64_t(1) << bits) < N) ++bits;
    const int passes = bits <= 8 ? 1 : (bits + 7) / 8;
    const PairSpec ps{topk, causal ? 1 : 0, N};
    radix_pass<true>(BH, idx, nullptr, N * topk, N * topk, 0, ps, ws, ws.rec0, s);
    uint2* cur = ws.rec0;
    for (int p = 1; p < passes; ++p) {
        uint2* nxt = (p & 1) ? ws.rec1 : ws.rec0;
        radix_pass<false>(BH, nullptr, cur, ws.P, ws.P, 8 * p, ps, ws, nxt, s);
        cur = nxt;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zeta_segment_offsets_kernel,
                       dim3(static_cast<unsigned>((ws.P + 255) / 256), static_cast<unsigned>(BH)),
                       dim3(256), 0, s, cur, ws.counts, ws.P, N, ws.offs);
    marks.record(3, s);
    e = launch_key<BF16>(BH, H, N, dv, q, k, v, gamma, dout, ws, cur, ws.perm_k, dk, dvout, s);
    if (e != hipSuccess) return e;
    marks.record(4, s);
    const int64_t dch = dgamma_chunks(BH / H, N);
    hipLaunchKernelGGL(zeta_dgamma_partial_kernel,
                       dim3(static_cast<unsigned>(dch), static_cast<unsigned>(H)), dim3(256), 0, s,
                       ws.dg_row, BH / H, H, N, dch, ws.dg_part);
    hipLaunchKernelGGL(zeta_dgamma_final_kernel, dim3(static_cast<unsigned>(H)), dim3(64), 0, s,
                       ws.dg_part, dch, dgamma);
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
