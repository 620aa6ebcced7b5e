// rse_sort.hip -- stable LSD radix sort of (32-bit key, 32-bit value) pairs
// for the sparse backward ("RecIS：阿里开源推荐系统统一训练框架", "代码架构":
// duplicate gradients are merged without floating-point atomics; here by
// sorting lookups by row and reducing each run).
//
// Pairs are stored interleaved, one 8-byte (key, value) word each, so the
// scattered runs a pass writes are twice as long in bytes as with separate
// key and value arrays.  One kernel per digit pass (digits of up to 9 bits,
// so 26-bit row keys take three passes); the digit histograms of every pass
// are computed beforehand by the pair-building kernel.  A pass runs a bounded number of blocks; each
// repeatedly:
//   1. takes the next tile (8192 pairs) from an atomic counter, so every tile
//      it may wait on belongs to a block that is already running;
//   2. ranks the tile's keys stably: each wave owns 1024 consecutive pairs
//      and walks them 64 at a time, building a digit-match mask per lane from
//      one ballot per digit bit and keeping wave-private running counts in
//      LDS, so no block barrier is needed per row;
//   3. publishes its per-digit counts, then looks back over the preceding
//      tiles' published counts (decoupled look-back, Merrill & Garland 2016)
//      to get its global offset per digit, and publishes the inclusive sums;
//   4. reorders the tile in LDS by digit and writes it out, so consecutive
//      lanes write consecutive addresses of each digit's run.
// Look-back waits are bounded: on a timeout the pass raises an error flag
// and writes nothing (the caller reports RSE_ERR_HIP) instead of hanging.  A
// pass whose error flag is already raised when a block starts does nothing.
#include "rse_sort.h"

using namespace rse;
using namespace rse_host;

namespace {

constexpr int SB = 512;                         // threads per sort block
constexpr int ITEMS = SORT_TILE / SB;           // 16 pairs per thread
constexpr int SWAVES = SB / WAVE;
constexpr int PER_WAVE = SORT_TILE / SWAVES;    // 1024 consecutive pairs per wave
constexpr uint32_t ST_AGG = 1u << 30;           // tile count published
constexpr uint32_t ST_INC = 2u << 30;           // inclusive prefix published
constexpr uint32_t ST_VAL = (1u << 30) - 1u;
constexpr uint32_t SPIN_LIMIT = 1u << 22;
constexpr int LOOK = 8;                         // predecessors read per look-back step
// Blocks per pass, each looping over tiles.  Measured beside the step's
// large kernels: capping a pass at 64-128 blocks made the step slower (the
// pass takes longer and the apply waits for it); at 256 and above the step
// time no longer changes, so the cap only saves launching one block per
// tile for very large batches.
constexpr int64_t SORT_BLOCKS = 1024;

__device__ __forceinline__ uint32_t load_state(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_state(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive scan over `bins` (<= 512) values, up to two per thread; returns through
// `out`; `tmp` holds SWAVES words.
__device__ void block_scan_bins(const uint32_t* in, uint32_t* out, int bins, uint32_t* tmp) {
    const int tid = threadIdx.x, lane = lane_id(), w = tid / WAVE;
    const int d0 = 2 * tid;
    const uint32_t a = d0 < bins ? in[d0] : 0u;
    const uint32_t b = d0 + 1 < bins ? in[d0 + 1] : 0u;
    const uint32_t s = a + b;
    uint32_t x = s;
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) tmp[w] = x;
    __syncthreads();
    uint32_t pre = 0;
    for (int q = 0; q < w; ++q) pre += tmp[q];
    const uint32_t ex = pre + x - s;
    if (d0 < bins) out[d0] = ex;
    if (d0 + 1 < bins) out[d0 + 1] = ex + a;
    __syncthreads();
}

__global__ __launch_bounds__(SB) void k_onesweep(const uint2* pairs_in, uint2* pairs_out, int64_t n, int shift,
                                                int width, const uint32_t* totals, uint32_t* state,
                                                uint32_t* tile_ctr, uint32_t* error, uint32_t n_tiles) {
    latency_bound_priority();
    __shared__ uint32_t s_wcnt[SWAVES][SORT_MAX_BINS];   // wave running counts -> wave prefixes
    __shared__ uint32_t s_cnt[SORT_MAX_BINS];            // tile count per digit
    __shared__ uint32_t s_pre[SORT_MAX_BINS];            // tile-local exclusive prefix per digit
    __shared__ uint32_t s_base[SORT_MAX_BINS];           // global exclusive prefix of the digit
    __shared__ uint32_t s_glob[SORT_MAX_BINS];           // output position of the digit's first pair here
    __shared__ uint32_t s_k[SORT_TILE];
    __shared__ uint32_t s_v[SORT_TILE];
    __shared__ uint32_t s_tmp[SWAVES];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_fail;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / WAVE;
    const int bins = 1 << width;
    const uint32_t dmask = (uint32_t)bins - 1u;
    // global exclusive prefix per digit, once per block: the digit totals
    // are the sum of their copies
    for (int d = tid; d < bins; d += SB) {
        uint32_t t = 0;
#pragma unroll
        for (int c = 0; c < SORT_TOTAL_COPIES; ++c) t += totals[c * SORT_COPY_STRIDE + d];
        s_cnt[d] = t;
    }
    __syncthreads();
    block_scan_bins(s_cnt, s_base, bins, s_tmp);
    // persistent: take tiles until none is left (or the pass has failed)
    for (;;) {
    if (tid == 0) {
        s_tile = atomicAdd(tile_ctr, 1u);
        s_fail = load_state(error) != 0u;     // raised before or during the pass: stop
    }
    for (int d = tid; d < SWAVES * SORT_MAX_BINS; d += SB) (&s_wcnt[0][0])[d] = 0;
    __syncthreads();
    const uint32_t tile = s_tile;
    if (s_fail || tile >= n_tiles) break;
    const int64_t base = (int64_t)tile * SORT_TILE;
    const int64_t tile_n = n - base < SORT_TILE ? n - base : SORT_TILE;

    // 1-2. stable rank within the wave's 1024 pairs
    uint32_t key[ITEMS], val[ITEMS], wr[ITEMS];
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int64_t i = base + (int64_t)w * PER_WAVE + k * WAVE + lane;
        const bool v = i < n;
        const uint2 pr = v ? pairs_in[i] : make_uint2(0u, 0u);
        key[k] = pr.x;
        val[k] = pr.y;
    }
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int64_t i = base + (int64_t)w * PER_WAVE + k * WAVE + lane;
        const bool v = i < n;
        const uint32_t d = (key[k] >> shift) & dmask;
        unsigned long long peers = __ballot(v);
        for (int b = 0; b < width; ++b) {
            const bool bit = (d >> b) & 1u;
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint32_t r = (uint32_t)__popcll(peers & lt);
        const uint32_t old = v ? s_wcnt[w][d] : 0u;      // every lane reads before the leader writes
        wr[k] = old + r;
        if (v && r == 0) s_wcnt[w][d] = old + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    // per digit: tile count, wave prefixes; publish the tile count
    for (int d = tid; d < bins; d += SB) {
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < SWAVES; ++q) {
            const uint32_t x = s_wcnt[q][d];
            s_wcnt[q][d] = c;
            c += x;
        }
        s_cnt[d] = c;
        store_state(&state[(int64_t)tile * SORT_MAX_BINS + d], (tile == 0 ? ST_INC : ST_AGG) | c);
    }
    __syncthreads();
    block_scan_bins(s_cnt, s_pre, bins, s_tmp);
    // 3. decoupled look-back per digit, LOOK predecessors read at once: their
    // counts are added newest first until an inclusive prefix is found
    // (tile 0 always publishes one, so the walk ends); a predecessor that
    // has published nothing yet is polled again.
    for (int d = tid; d < bins; d += SB) {
        uint32_t ex = 0;
        if (tile > 0) {
            int64_t t = (int64_t)tile - 1;      // newest predecessor not yet added
            uint32_t spins = 0;
            bool timed_out = false;
            while (true) {
                uint32_t st[LOOK];
#pragma unroll
                for (int u = 0; u < LOOK; ++u) {
                    const int64_t tt = t - u >= 0 ? t - u : 0;
                    st[u] = load_state(&state[tt * SORT_MAX_BINS + d]);
                }
                bool done = false, stall = false;
                int used = 0;
#pragma unroll
                for (int u = 0; u < LOOK; ++u) {
                    if (done || stall) continue;
                    if (st[u] & ST_INC) {
                        ex += st[u] & ST_VAL;
                        done = true;
                    } else if (st[u] & ST_AGG) {
                        ex += st[u] & ST_VAL;
                        ++used;
                    } else {
                        stall = true;
                    }
                }
                if (done) break;
                t -= used;
                if (stall) {
                    ++spins;
                    if (spins > SPIN_LIMIT || ((spins & 1023u) == 0 && load_state(error))) {
                        s_fail = 1;
                        atomicExch(error, 1u);
                        timed_out = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (!timed_out) store_state(&state[(int64_t)tile * SORT_MAX_BINS + d], ST_INC | (ex + s_cnt[d]));
        }
        s_glob[d] = s_base[d] + ex;
    }
    __syncthreads();
    if (s_fail) break;
    // 4. reorder in LDS by digit, then write runs out
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int64_t i = base + (int64_t)w * PER_WAVE + k * WAVE + lane;
        if (i < n) {
            const uint32_t d = (key[k] >> shift) & dmask;
            const uint32_t pos = s_pre[d] + s_wcnt[w][d] + wr[k];
            s_k[pos] = key[k];
            s_v[pos] = val[k];
        }
    }
    __syncthreads();
    for (int x = tid; x < tile_n; x += SB) {
        const uint32_t kk = s_k[x];
        const uint32_t d = (kk >> shift) & dmask;
        const uint32_t o = s_glob[d] + ((uint32_t)x - s_pre[d]);
        if ((int64_t)o < n) {                 // always, when the totals match the keys
            pairs_out[o] = make_uint2(kk, s_v[x]);     // one 8-byte store per pair
        } else {
            atomicExch(error, 1u);
        }
    }
    __syncthreads();                          // LDS is reused by the next tile
    }
}

}  // namespace

namespace rse_host {

SortPlan sort_plan(int bits) {
    SortPlan p;
    if (bits < 1) bits = 1;
    p.passes = (bits + 8) / 9;
    p.width = (bits + p.passes - 1) / p.passes;
    return p;
}

static int64_t tiles_of(int64_t n) { return (n + SORT_TILE - 1) / SORT_TILE; }

size_t sort_workspace(int64_t n, int64_t* n_tiles_out) {
    const int64_t n_tiles = tiles_of(n > 0 ? n : 1);
    if (n_tiles_out) *n_tiles_out = n_tiles;
    return align_up((size_t)SORT_TOTAL_COPIES * SORT_COPY_STRIDE * 4, 256) +
           align_up((size_t)SORT_MAX_PASSES * n_tiles * SORT_MAX_BINS * 4, 256) + 256 + 256;
}

SortPrep sort_prep(void* ws, int64_t n) {
    const int64_t n_tiles = tiles_of(n > 0 ? n : 1);
    Carver c(ws);
    SortPrep p;
    p.totals = c.take<uint32_t>((size_t)SORT_TOTAL_COPIES * SORT_COPY_STRIDE);
    p.state = c.take<uint32_t>((size_t)SORT_MAX_PASSES * n_tiles * SORT_MAX_BINS);
    p.tile_ctr = c.take<uint32_t>(SORT_MAX_PASSES);
    p.error = c.take<uint32_t>(1);
    p.state_words = (int64_t)SORT_MAX_PASSES * n_tiles * SORT_MAX_BINS;
    return p;
}

bool sort_supported(int64_t n, int bits) {
    // a digit count or an inclusive prefix is at most n and must fit the
    // 30-bit value field of the look-back state
    return bits >= 1 && bits <= 32 && sort_plan(bits).passes <= SORT_MAX_PASSES && n >= 0 &&
           n <= (int64_t)ST_VAL;
}

int radix_sort_pairs(uint2* p0, uint2* p1, int64_t n, int bits, void* ws, bool* result_in_alt, hipStream_t s) {
    if (!sort_supported(n, bits)) return RSE_ERR_UNSUPPORTED;
    const SortPlan plan = sort_plan(bits);
    const int64_t n_tiles = tiles_of(n);
    SortPrep p = sort_prep(ws, n);
    bool alt = false;
    if (n > 0) {
        for (int ps = 0; ps < plan.passes; ++ps) {
            const int shift = plan.width * ps;
            const int width = bits - shift < plan.width ? bits - shift : plan.width;
            uint2* pi = alt ? p1 : p0;
            uint2* po = alt ? p0 : p1;
            TraceScope ts(RSE_K_SORT_SCATTER, s);
            const int64_t grid = n_tiles < SORT_BLOCKS ? n_tiles : SORT_BLOCKS;
            hipLaunchKernelGGL(k_onesweep, dim3((unsigned)grid), dim3(SB), 0, s, pi, po, n, shift, width,
                               p.totals + ps * SORT_MAX_BINS, p.state + (int64_t)ps * n_tiles * SORT_MAX_BINS,
                               p.tile_ctr + ps, p.error, (uint32_t)n_tiles);
            alt = !alt;
        }
    }
    *result_in_alt = alt;
    return launch_status();
}

}  // namespace rse_host
