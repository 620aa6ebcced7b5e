// rse_device.h -- device-side building blocks shared by the library's
// kernels: object layouts in HBM, key hashing, row initialisation, rounding,
// row addressing and 64-lane wavefront helpers.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rse.h"

namespace rse {

constexpr int WAVE = 64;

// ------------------------------------------------------------ layouts ----
// IDMap device memory: [header 256 B][dir: TableDir x n][slots]
constexpr uint64_t EMPTY_KEY = 0x8000000000000000ull;   // INT64_MIN
constexpr uint64_t EMPTY_VAL = ~0ull;
constexpr uint64_t PENDING_BASE = 1ull << 62;            // value = base + first lookup index
constexpr int BUCKET = 8;                                // slots per 128-byte bucket

struct Slot {
    uint64_t key;
    uint64_t val;
};

struct TableDir {
    int64_t slot_base;   // first slot of this table's region
    int64_t n_buckets;   // region size in buckets
    int64_t max_keys;    // floor(max_load * slots)
    uint64_t salt;       // per-table hash salt
    int64_t n_keys;      // live keys (device counter)
    uint64_t side_val;   // value of key EMPTY_KEY, or EMPTY_VAL / pending
    int64_t new_keys;    // scratch: keys added by the current call
    int64_t pad;
};
static_assert(sizeof(TableDir) == 64, "TableDir size");

struct MapHeader {
    int32_t status;
    int32_t n_tables;
    int32_t merged;
    int32_t pad0;
    int64_t pad[30];
};
static_assert(sizeof(MapHeader) == 256, "MapHeader size");

// EmbeddingBlocks metadata: [header 256 B][chunk pointers x max_chunks]
struct BlocksHeader {
    int64_t rows_used;
    int32_t status;
    int32_t pad0;
    int64_t free_head;    // free-list entries already handed out
    int64_t free_count;   // free-list entries left, from free_head on
    int64_t pad[28];
};
static_assert(sizeof(BlocksHeader) == 256, "BlocksHeader size");

// ------------------------------------------------- global row access ----
// Row addresses are computed from integers (chunk base + offset), so the
// compiler cannot tell which memory they point to and would use FLAT
// instructions.  FLAT accesses are tracked by both the vector-memory and the
// LDS counters, so every wait for an LDS read (or for the chunk-table read of
// the next row) would also wait for all row loads in flight.  Rows are
// therefore read and written through explicit global-address-space pointers
// with clang vector types (HIP's uint4/float4 are structs, whose copies lose
// the address space).
#define RSE_GLOBAL __attribute__((address_space(1)))
#define RSE_LDS __attribute__((address_space(3)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 gload_u4(const void* p) { return *(const RSE_GLOBAL u32x4*)p; }
__device__ __forceinline__ f32x4 gload_f4(const void* p) { return *(const RSE_GLOBAL f32x4*)p; }
__device__ __forceinline__ void gstore_u4(void* p, u32x4 v) { *(RSE_GLOBAL u32x4*)p = v; }
__device__ __forceinline__ void gstore_f4(void* p, f32x4 v) { *(RSE_GLOBAL f32x4*)p = v; }
// The same with the nontemporal hint when NT: the access streams through the
// caches (for data read or written once, so that it does not displace lines
// that are read again).
template <bool NT> __device__ __forceinline__ u32x4 gload_u4x(const void* p) {
    if (NT) return __builtin_nontemporal_load((const RSE_GLOBAL u32x4*)p);
    return *(const RSE_GLOBAL u32x4*)p;
}
template <bool NT> __device__ __forceinline__ f32x4 gload_f4x(const void* p) {
    if (NT) return __builtin_nontemporal_load((const RSE_GLOBAL f32x4*)p);
    return *(const RSE_GLOBAL f32x4*)p;
}
template <bool NT> __device__ __forceinline__ void gstore_u4x(void* p, u32x4 v) {
    if (NT) __builtin_nontemporal_store(v, (RSE_GLOBAL u32x4*)p);
    else *(RSE_GLOBAL u32x4*)p = v;
}
template <bool NT> __device__ __forceinline__ void gstore_f4x(void* p, f32x4 v) {
    if (NT) __builtin_nontemporal_store(v, (RSE_GLOBAL f32x4*)p);
    else *(RSE_GLOBAL f32x4*)p = v;
}

// Everything a kernel needs to address rows (passed by value).  Kernels on
// the hot path stage the chunk-pointer table in LDS (stage_chunks) so that a
// row address costs an LDS read instead of a dependent global load.
constexpr int LDS_CHUNKS = 512;

struct RowsView {
    const uint64_t* chunks;   // device chunk-pointer table
    int64_t row_bytes;
    int32_t shift;            // log2(rows per chunk)
    int32_t n_chunks;
    uint64_t mask;            // rows per chunk - 1
    __device__ __forceinline__ char* row(int64_t r) const {
        const uint64_t base = ((const RSE_GLOBAL uint64_t*)chunks)[(uint64_t)r >> shift];
        return reinterpret_cast<char*>(base + ((uint64_t)r & mask) * (uint64_t)row_bytes);
    }
    __device__ __forceinline__ bool lds_ok() const { return n_chunks <= LDS_CHUNKS; }
    // s: the LDS copy made by stage_chunks.  The two table reads are typed
    // by address space so that they stay an LDS read and a global read (one
    // FLAT read through a selected pointer would tie the counters together).
    __device__ __forceinline__ char* row(const uint64_t* s, int64_t r) const {
        const uint64_t c = (uint64_t)r >> shift;
        const uint64_t base = lds_ok() ? ((const RSE_LDS uint64_t*)s)[c] : ((const RSE_GLOBAL uint64_t*)chunks)[c];
        return reinterpret_cast<char*>(base + ((uint64_t)r & mask) * (uint64_t)row_bytes);
    }
};

// All threads of the block must call this (it synchronises the block).
__device__ __forceinline__ void stage_chunks(uint64_t* s, const RowsView& rv) {
    const int n = rv.n_chunks < LDS_CHUNKS ? rv.n_chunks : LDS_CHUNKS;
    for (int i = threadIdx.x; i < n; i += blockDim.x) s[i] = rv.chunks[i];
    __syncthreads();
}

// ------------------------------------------------------------ hashing ----
// Bucket hash: MurmurHash3's 64-bit finaliser (Appleby), salted per table.
__device__ __forceinline__ uint64_t fmix64(uint64_t k) {
    k ^= k >> 33;
    k *= 0xFF51AFD7ED558CCDull;
    k ^= k >> 33;
    k *= 0xC4CEB9FE1A85EC53ull;
    k ^= k >> 33;
    return k;
}

// Map a 64-bit hash onto [0, n) without division (multiply-high range
// reduction, Lemire 2019).
__device__ __forceinline__ int64_t reduce_range(uint64_t h, int64_t n) {
    return (int64_t)__umul64hi(h, (uint64_t)n);
}

// ------------------------------------------------------- row init -------
// SplitMix64 output function (Steele, Lea & Flood 2014; Vigna's reference).
__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr uint64_t SM64_GAMMA = 0x9E3779B97F4A7C15ull;

// Initial value of column c: an exact multiple of 2^-27 in [-1/16, 1/16)
// for fp32 storage; an exact multiple of 2^-11 (8 significant bits) for
// bf16 storage.
__device__ __forceinline__ float init_value(uint64_t key, uint32_t table, int c, uint64_t seed,
                                            bool bf16) {
    const uint64_t x = (key ^ ((seed + (uint64_t)table) * SM64_GAMMA)) + (uint64_t)(c + 1) * SM64_GAMMA;
    const uint64_t h = splitmix64_mix(x);
    if (!bf16) {
        const int32_t q = (int32_t)(h >> 40) - (1 << 23);
        return (float)q * 0x1p-27f;
    }
    const int32_t q = (int32_t)(h >> 56) - 128;
    return (float)q * 0x1p-11f;
}

// ---------------------------------------------------------- rounding ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Exact bf16 -> bf16 bits of a float with at most 8 significant bits.
__device__ __forceinline__ uint16_t f32_to_bf16_exact(float f) {
    return (uint16_t)(__float_as_uint(f) >> 16);
}

// double -> bf16, round to nearest even, with a single rounding: convert to
// fp32 rounding to odd (truncate, then force the last bit if inexact), then
// round that to bf16 to nearest even.  Rounding to odd into a format with at
// least two more bits makes the second rounding correct (Boldo & Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd", IEEE TC 2008).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
    if (x != x) return 0x7FC0;
    const float t = __double2float_rz(x);
    uint32_t u = __float_as_uint(t);
    if ((double)t != x) u |= 1u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ------------------------------------------------------ wave helpers ----
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
    return __shfl_xor(v, mask, WAVE);
}

template <typename T>
__device__ __forceinline__ T shfl_idx(T v, int src) {
    return __shfl(v, src, WAVE);
}

// Kernels made of short dependent memory round trips (probe, pair building,
// radix passes, segment index) often share CUs with another stream's
// bandwidth-bound kernel: their waves ask for instruction issue first, so
// they finish sooner and leave the GPU to the large kernel (measured on the
// two-stream click-log step: about 1% faster).
__device__ __forceinline__ void latency_bound_priority() { __builtin_amdgcn_s_setprio(3); }

// Status helpers: first error wins.
__device__ __forceinline__ void set_status(int32_t* st, int32_t code) {
    atomicCAS(st, 0, code);
}

}  // namespace rse
