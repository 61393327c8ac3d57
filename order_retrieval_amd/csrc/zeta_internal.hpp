// zeta_internal.hpp -- shared declarations of the HIP kernels' launchers and device helpers.
// Internal to libzeta.so; the public surface is include/zeta.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zeta {

constexpr int kMaxTopK = 256;
constexpr int kMaxDv = 512;
constexpr size_t kAlign = 256;

// ----------------------------------------------------------------------------- device
// bf16 is carried as raw 16-bit patterns; widening is exact, narrowing rounds to nearest
// even (finite inputs; NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Workgroups of a launch are dispatched round-robin over the 8 XCDs of an MI355X.  Kernels
// that gather rows map the hardware block index to a logical tile so that each XCD walks
// one contiguous eighth of the tiles in order: its L2 then serves one slice of the
// processing order.  Launch kXcds * per_xcd blocks (per_xcd = ceil(tiles / kXcds)); blocks
// whose tile is >= tiles exit.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_tile(int64_t block, int64_t per_xcd) {
    return (block % kXcds) * per_xcd + block / kXcds;
}
inline int64_t xcd_per(int64_t tiles) { return (tiles + kXcds - 1) / kXcds; }

// One 12-byte point (x, y, z) of a q or k row, read with a single 12-byte load (the rows
// are 4-byte aligned).
struct __attribute__((packed, aligned(4))) Point3 {
    float x, y, z;
};
__device__ __forceinline__ Point3 load_point(const float* rows, int64_t r) {
    return *reinterpret_cast<const Point3*>(rows + 3 * r);
}
__device__ __forceinline__ void keep(Point3& p) {
    asm volatile("" : "+v"(p.x), "+v"(p.y), "+v"(p.z));
}

// Marks a loaded value as used here.  Placed after a batch of loads from clamped (always
// valid) positions, it keeps each load unconditional: without it the compiler may move a load
// behind the later test that decides whether its value matters, and then wait on that load
// alone, so the batch no longer has its loads in flight together.
__device__ __forceinline__ void keep(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep(int32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep(uint64_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep(uint2& x) { asm volatile("" : "+v"(x.x), "+v"(x.y)); }
__device__ __forceinline__ void keep(uint4& x) {
    asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}
__device__ __forceinline__ void keep(float4& x) {
    asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}

// Optional events recorded between the stages of one call (measurement hook).
struct StageEvents {
    void* const* ev = nullptr;
    int n = 0;
    void record(int stage, hipStream_t s) const {
        if (stage < n && ev[stage]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[stage]), s);
    }
};

// ----------------------------------------------------------------------------- launchers
// Each returns the hipError_t of its launches (hipSuccess when nothing was launched).
hipError_t launch_encode(const float* x, int64_t rows, uint32_t* z, hipStream_t s);
// Curve coordinate order: axis a of the code reads coordinate (perm >> 2a) & 3.
constexpr int perm_code(int c0, int c1, int c2) { return c0 | (c1 << 2) | (c2 << 4); }
constexpr int kPermIdentity = perm_code(0, 1, 2);
hipError_t launch_encode_perm(const float* x, int64_t rows, int perm, uint32_t* z, hipStream_t s);
// Both point sets (queries and keys, rows points each) in one launch.
hipError_t launch_encode2_perm(const float* q, uint32_t* zq, const float* k, uint32_t* zk,
                               int64_t rows, int perm, hipStream_t s);
// Levels 0 .. first-1 are not written.
// The trees store levels tree_store_base(levels, first) .. levels - 1 of every (b,h), as
// [BH][levels - base][N].
int tree_store_base(int levels, int first);
hipError_t launch_build_tree(int64_t BH, int64_t N, int levels, int first, const uint32_t* zk,
                             uint64_t* tree_asc, uint64_t* tree_desc, hipStream_t s);
// 12-bit cells: 36-bit codes (uint64), tree entries (code << 28) | j, N < 2^28.
hipError_t launch_encode36_perm(const float* x, int64_t rows, int perm, uint64_t* z,
                                hipStream_t s);
hipError_t launch_build_tree36(int64_t BH, int64_t N, int levels, int first, const uint64_t* zk,
                               uint64_t* tree_asc, uint64_t* tree_desc, hipStream_t s);
hipError_t launch_select36(int64_t BH, int64_t N, int stored, int base, int topk, bool causal,
                           const uint64_t* zq, const uint64_t* zk, const uint64_t* tree_asc,
                           const uint64_t* tree_desc, const uint32_t* order, int32_t* idx,
                           hipStream_t s);
hipError_t launch_select_chunked36(int64_t BH, int64_t N, int stored, int base, int lvl,
                                   int topk,
                                   const uint64_t* zq, const uint64_t* ta, int32_t* idx,
                                   hipStream_t s);
// order: processing order of the queries (per (b,h) positions), or null for position order.
// zk: the key codes (runs shorter than 2K are read from them, not from the tree).
hipError_t launch_select(int64_t BH, int64_t N, int stored, int base, int topk, bool causal,
                         const uint32_t* zq, const uint32_t* zk, const uint64_t* tree_asc,
                         const uint64_t* tree_desc, const uint32_t* order, int32_t* idx,
                         hipStream_t s);
// Lowest tree level the exact selection reads for this topk.
int select_first_level(int topk);
// Chunked search over the aligned chunks of 2^lvl positions (tree level lvl).
hipError_t launch_select_chunked(int64_t BH, int64_t N, int stored, int base, int lvl, int topk,
                                 const uint32_t* zq, const uint64_t* ta, int32_t* idx,
                                 hipStream_t s);
// Merge of several curves' selections sel [curves][rows][per] into idx [rows][topk].
hipError_t launch_curves_merge(int64_t rows, int curves, int per, int topk, const int32_t* sel,
                               int32_t* idx, hipStream_t s);
hipError_t launch_gather(int64_t BH, int64_t H, int64_t N, int64_t dv, int topk, bool causal,
                         bool bf16, const float* q, const float* k, const void* v,
                         const float* gamma, const int32_t* idx, const uint32_t* order, void* out,
                         hipStream_t s);
// Processing order: per (b,h), positions bucketed by the top code bits (order.hip).
// scratch: order_scratch_words(BH, N) words.
size_t order_scratch_words(int64_t BH, int64_t N);
// Codes of q and k (curve order `perm`) and the processing order of the queries, and of the
// keys too when order_keys (then zk must be zq + BH N, and `order` and `scratch` hold 2 BH
// slices), in three launches.  rank_of, when not null, takes the inverse of the queries'
// order: rank_of[bh N + i] = the rank of query i ([BHN] words).
hipError_t launch_encode_order(const float* q, uint32_t* zq, const float* k, uint32_t* zk,
                               int64_t BH, int64_t N, int perm, bool order_keys,
                               uint32_t* order, uint32_t* scratch, hipStream_t s,
                               uint32_t* rank_of = nullptr);
hipError_t launch_order(int64_t BH, int64_t N, const uint32_t* codes, uint32_t* perm,
                        uint32_t* scratch, hipStream_t s);

// Measurement: `groups` groups of 16 lanes each read rows_per_group rows (row_bytes bytes,
// 16 per lane) drawn from table [table_rows] (a power of two); one word per group to sink.
hipError_t launch_probe_row_gather(const void* table, int64_t table_rows, int row_bytes,
                                   int64_t groups, int rows_per_group, uint32_t seed,
                                   uint32_t* sink, hipStream_t s);

struct BwdBuffers {
    float2* coef;     // [BH][N][topk] per selection slot {a_ij, c_ij}, queries in processing order
    float4* qrec;     // [BH][N] per query in processing order: {q_i, i}
    uint32_t* rank_q; // [BH][N] rank of each query in its processing order
    float* dg_row;    // [BHN] per-query dgamma contributions
    float* dg_part;   // [H][dgamma_chunks] partial sums
    uint2* rec0;      // [BH][P] radix-sort ping-pong records {j, p}; with keys below 2^16
    uint2* rec1;      // rec1 takes the final slot list (u32 p per pair, in key segments)
    uint32_t* hist;   // [BH][256][tiles] per-tile digit counts, scanned in place
    uint32_t* totals; // [BH][256] digit totals
    uint32_t* counts; // [BH] pairs of each (b,h)
    uint32_t* offs;   // [BH][N+1] segment starts of the key-sorted pair list
    uint32_t* ends;   // [BH][N+1] segment ends (keys below 2^16: segments not in key order)
    uint32_t* zq;     // [BHN] query codes
    uint32_t* perm_q; // [BHN] query processing order
    uint32_t* zk;     // [BHN] key codes
    uint32_t* perm_k; // [BHN] key processing order
    uint32_t* ohist;  // order_scratch_words(2 BH, N) words for the processing orders
    int64_t P;        // upper bound of the pairs per (b,h)
    int64_t tiles;    // radix tiles per (b,h)
};
size_t bwd_pairs_per_head(int64_t N, int topk, bool causal);
int64_t bwd_tiles_per_head(int64_t P);
// Keys below 2^16 and slots below 2^24: the first radix pass writes 4-byte records.
bool bwd_records_packed(int64_t N, int topk);
int64_t dgamma_chunks(int64_t B, int64_t N);
hipError_t launch_bwd(int64_t BH, int64_t H, int64_t N, int64_t dv, int topk, bool causal, bool bf16,
                      const float* q, const float* k, const void* v, const float* gamma,
                      const int32_t* idx, const void* dout, float* dq, float* dk, void* dvout,
                      float* dgamma, const BwdBuffers& ws, const StageEvents& marks,
                      hipStream_t s);

}  // namespace zeta
