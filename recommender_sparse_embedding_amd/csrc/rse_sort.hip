// rse_sort.hip -- stable LSD radix sort of (32-bit key, 32-bit value) pairs
// for the sparse backward ("RecIS：阿里开源推荐系统统一训练框架", "代码架构":
// duplicate gradients are merged without floating-point atomics; here by
// sorting lookups by row and reducing each run).
//
// Per 8-bit digit pass, three kernels:
//   count:   per tile (4096 keys) digit histogram -> hist[digit][tile], and the
//            pass's global digit totals (integer atomics);
//   offsets: one block per digit scans its row of hist and adds the digit's
//            base (sum of the smaller digits' totals);
//   scatter: each tile ranks its keys stably (row by row of 256 keys: a
//            digit-match mask per wave from 8 ballots, per-wave counts in LDS,
//            running per-digit counts), then writes every pair to
//            offset[digit][tile] + rank.
// Keys only use the low `bits` bits, so the number of passes is
// ceil(bits / 8), set by the table's row capacity.
#include "rse_sort.h"

using namespace rse;
using namespace rse_host;

namespace {

constexpr int SB = 256;            // threads per sort block
constexpr int ITEMS = SORT_TILE / SB;

__global__ __launch_bounds__(SB) void k_count(const uint32_t* keys, int64_t n, int shift, int nbits,
                                             uint32_t* hist, int64_t n_tiles, uint32_t* totals) {
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
    const uint32_t dmask = (1u << nbits) - 1;
#pragma unroll 4
    for (int k = 0; k < ITEMS; ++k) {
        const int64_t i = base + k * SB + threadIdx.x;
        if (i < n) atomicAdd(&h[(keys[i] >> shift) & dmask], 1u);
    }
    __syncthreads();
    const uint32_t c = h[threadIdx.x];
    hist[(int64_t)threadIdx.x * n_tiles + blockIdx.x] = c;
    if (c) atomicAdd(&totals[threadIdx.x], c);
}

// One block per digit: exclusive scan of hist[digit][0..n_tiles) plus base.
__global__ __launch_bounds__(SB) void k_offsets(uint32_t* hist, int64_t n_tiles,
                                               const uint32_t* totals) {
    const int dg = blockIdx.x;
    __shared__ uint32_t s_base;
    __shared__ uint32_t wsum[SB / WAVE];
    __shared__ uint32_t s_carry;
    if (threadIdx.x == 0) {
        uint32_t b = 0;
        for (int k = 0; k < dg; ++k) b += totals[k];
        s_base = b;
        s_carry = 0;
    }
    __syncthreads();
    uint32_t* row = hist + (int64_t)dg * n_tiles;
    const int lane = lane_id();
    const int w = threadIdx.x / WAVE;
    for (int64_t c0 = 0; c0 < n_tiles; c0 += SB) {
        const int64_t k = c0 + threadIdx.x;
        const uint32_t v = k < n_tiles ? row[k] : 0;
        uint32_t x = v;
        for (int o = 1; o < WAVE; o <<= 1) {
            const uint32_t y = __shfl_up(x, o, WAVE);
            if (lane >= o) x += y;
        }
        if (lane == WAVE - 1) wsum[w] = x;
        __syncthreads();
        uint32_t pre = 0, tot = 0;
        for (int q = 0; q < SB / WAVE; ++q) {
            if (q < w) pre += wsum[q];
            tot += wsum[q];
        }
        const uint32_t carry = s_carry;
        if (k < n_tiles) row[k] = s_base + carry + pre + x - v;
        __syncthreads();
        if (threadIdx.x == 0) s_carry = carry + tot;
        __syncthreads();
    }
}

__global__ __launch_bounds__(SB) void k_scatter(const uint32_t* keys_in, const uint32_t* vals_in,
                                               uint32_t* keys_out, uint32_t* vals_out, int64_t n,
                                               int shift, int nbits, const uint32_t* offsets,
                                               int64_t n_tiles) {
    __shared__ uint32_t s_run[256];
    __shared__ uint32_t s_cnt[SB / WAVE][256];
    __shared__ uint32_t s_off[256];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = tid / WAVE;
    s_run[tid] = 0;
    s_off[tid] = offsets[(int64_t)tid * n_tiles + blockIdx.x];
#pragma unroll
    for (int q = 0; q < SB / WAVE; ++q) s_cnt[q][tid] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
    const uint32_t dmask = (1u << nbits) - 1;
    const unsigned long long lt_mask = (1ull << lane) - 1;
    for (int k = 0; k < ITEMS; ++k) {
        const int64_t i = base + (int64_t)k * SB + tid;
        const bool valid = i < n;
        uint32_t key = 0, val = 0, dg = 0;
        if (valid) {
            key = keys_in[i];
            val = vals_in[i];
            dg = (key >> shift) & dmask;
        }
        unsigned long long peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (dg >> b) & 1u;
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint32_t wrank = (uint32_t)__popcll(peers & lt_mask);
        if (valid && wrank == 0) s_cnt[w][dg] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t r = s_run[dg] + wrank;
            for (int q = 0; q < w; ++q) r += s_cnt[q][dg];
            const uint32_t pos = s_off[dg] + r;
            keys_out[pos] = key;
            vals_out[pos] = val;
        }
        __syncthreads();
        uint32_t add = 0;
#pragma unroll
        for (int q = 0; q < SB / WAVE; ++q) {
            add += s_cnt[q][tid];
            s_cnt[q][tid] = 0;
        }
        s_run[tid] += add;
        __syncthreads();
    }
}

}  // namespace

namespace rse_host {

size_t sort_workspace(int64_t n, int64_t* n_tiles_out) {
    const int64_t n_tiles = (n + SORT_TILE - 1) / SORT_TILE;
    if (n_tiles_out) *n_tiles_out = n_tiles;
    // hist [256][n_tiles] + totals [MAX_PASSES][256]
    return align_up((size_t)256 * (size_t)(n_tiles > 0 ? n_tiles : 1) * 4, 256) +
           align_up((size_t)SORT_MAX_PASSES * 256 * 4, 256);
}

// Sorts (k0, v0) by the low `bits` bits; ping-pongs through (k1, v1).  The
// result ends in (k0, v0) if the number of passes is even, else in (k1, v1);
// *result_in_alt reports which.  `totals` must be zeroed for all passes
// beforehand (see sort_totals).
int radix_sort_pairs(uint32_t* k0, uint32_t* v0, uint32_t* k1, uint32_t* v1, int64_t n, int bits,
                     void* ws, bool* result_in_alt, hipStream_t s) {
    int64_t n_tiles = 0;
    sort_workspace(n, &n_tiles);
    Carver c(ws);
    uint32_t* hist = c.take<uint32_t>((size_t)256 * (size_t)(n_tiles > 0 ? n_tiles : 1));
    uint32_t* totals = c.take<uint32_t>((size_t)SORT_MAX_PASSES * 256);
    const int passes = (bits + 7) / 8;
    if (passes > SORT_MAX_PASSES) return RSE_ERR_UNSUPPORTED;
    bool alt = false;
    if (n > 0) {
        for (int p = 0; p < passes; ++p) {
            const int shift = 8 * p;
            const int nbits = bits - shift < 8 ? bits - shift : 8;
            uint32_t* ki = alt ? k1 : k0;
            uint32_t* vi = alt ? v1 : v0;
            uint32_t* ko = alt ? k0 : k1;
            uint32_t* vo = alt ? v0 : v1;
            uint32_t* tot = totals + 256 * p;
            hipLaunchKernelGGL(k_count, dim3((unsigned)n_tiles), dim3(SB), 0, s, ki, n, shift, nbits,
                               hist, n_tiles, tot);
            hipLaunchKernelGGL(k_offsets, dim3(256), dim3(SB), 0, s, hist, n_tiles, tot);
            {
                TraceScope ts(RSE_K_SORT_SCATTER, s);
                hipLaunchKernelGGL(k_scatter, dim3((unsigned)n_tiles), dim3(SB), 0, s, ki, vi, ko, vo, n,
                                   shift, nbits, hist, n_tiles);
            }
            alt = !alt;
        }
    }
    *result_in_alt = alt;
    return launch_status();
}

uint32_t* sort_totals(void* ws, int64_t n) {
    int64_t n_tiles = 0;
    sort_workspace(n, &n_tiles);
    Carver c(ws);
    c.take<uint32_t>((size_t)256 * (size_t)(n_tiles > 0 ? n_tiles : 1));
    return c.take<uint32_t>((size_t)SORT_MAX_PASSES * 256);
}

}  // namespace rse_host
