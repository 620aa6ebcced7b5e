// rse_bwd.hip -- sparse backward and fused row-wise optimizer update.
//
// Semantics: "阿里 RecIS：搜广推训练的背景与难点" (backward touches only the
// looked-up rows); "DLRM — Meta 把工业推荐模型拆成 4 个标准积木", "踩过的坑" 4
// (sparse optimizer: only rows seen in the batch are updated);
// "RecIS：阿里开源推荐系统统一训练框架", "代码架构" (fused sparse-gradient
// update with fewer atomics).
//
// Pipeline, in two calls that may run on different streams:
//   prepare (needs only the row offsets and bag offsets, so it can overlap
//   the forward):  reset -> pairs: (row, bag) per lookup, row as a 32-bit
//   key (-1 -> a key above every row, sorted last) -> stable radix sort by
//   row -> index of the segments (runs of equal rows);
//   apply (needs the upstream gradient):  segmented reduction with the
//   optimizer fused in -> combine of long segments.
//
// Segmented reduction.  A segment is all lookups of one row (a run of the
// sorted keys).  An index kernel classifies every segment: one lookup,
// 2..LONG_T lookups ("short"), or longer ("long", whose head is listed as
// owner); the first two kinds go to lists.  The work kernel then runs three
// kinds of blocks side by side:
//   - long: the sorted lookups are cut into pieces of P = 32 or 64 lookups
//     (32 for fp32 rows of dim 16 and less, 64 otherwise); each piece
//     sums the part of a long segment it holds (at its start, continuing an
//     earlier piece, and/or at its end, continuing past it) into a carry
//     slot, 4-8 gradient rows in flight, in lookup order, in fp64;
//   - singles: each group of lanes takes a few one-lookup segments and loads
//     all their rows (weights + state) and gradient rows at once;
//   - short: each group takes one short segment, loads its row, sums its
//     gradient rows 4-8 at a time in lookup order, and updates the row.
// After each window of pieces, the work kernel adds every run of one long
// segment's piece partials into the run's first piece (in piece order); the
// combine kernel adds those run sums of each long segment in a fixed order
// (round-robin over a block's groups, then group order) and updates its row.
// The lists' order depends on timing, but every segment is reduced and
// updated independently, so results do not.  Only integer atomics are used.
#include <algorithm>
#include <cmath>

#include "rse_sort.h"

using namespace rse;
using namespace rse_host;

namespace {

// Lookups per piece: Geo<D, BF16>::P (below), never less than P_MIN (the
// workspace's carry slots are sized for P_MIN).
constexpr int P_MIN = 32;
// Longest segment reduced by one group.  At least P - 1, so that a longer
// segment cannot lie strictly inside one piece (the long role handles the
// segments at a piece's start and at its last head only).
constexpr int LONG_T = 64;
constexpr int HALO = LONG_T + 1;
#ifndef RSE_N_XCD
#define RSE_N_XCD 8
#endif
constexpr int N_XCD = RSE_N_XCD;

// Optimizer constants.  The bias corrections are applied as products with
// 1 / (1 - b1^t) and sqrt(1 / (1 - b2^t)), computed once on the host.
struct OptParams {
    double lr, eps, b1, b2, omb1, omb2, inv_bc1, sq_inv_bc2;
};

// Device counters of one call.  The three list lengths sit on separate
// 128-byte lines: each index block adds to them once, and atomics on one
// line serialise.
struct Ctr {
    unsigned long long bad;
    unsigned long long pad0[15];
    unsigned long long n_single;  // one-lookup segments
    unsigned long long pad1[15];
    unsigned long long n_multi;   // segments of 2..LONG_T lookups
    unsigned long long pad2[15];
    unsigned long long n_owners;  // longer segments (their heads are listed in owners)
    unsigned long long pad3[15];
};

constexpr int IX_BLOCK = 512;                      // index kernel: positions per block and thread
constexpr int IX_TILE = 4096;
constexpr int IX_PER = IX_TILE / IX_BLOCK;
constexpr int IX_WIN = IX_TILE + HALO + 1;
constexpr int IX_MASKS = (IX_WIN + 63) / 64;

struct Multi {                   // a segment of 2..LONG_T lookups
    uint32_t start;              // position of its first lookup in the sorted order
    uint32_t len;
    uint32_t key;                // its row
    uint32_t pad;
};

struct Owner {                   // a long segment (more than LONG_T lookups)
    uint32_t head;               // position of its first lookup in the sorted order
    uint32_t len;                // its length if the index kernel saw its end, else 0
    uint32_t key;                // its row
    uint32_t pad;
};

struct BwdArgs {
    RowsView rv;
    const uint2* pairs;          // sorted lookups: x = row, y = gradient row of its bag
    const int64_t* bag_off;
    const double* inv_len;       // mean pooling: 1 / bag length, per gradient row
    const float* grad;           // [batch, n_tables, dim]; sorted values index its rows
    int64_t batch;
    int32_t n_tables;
    int32_t mean;
    int64_t n;                   // lookups (sorted pairs)
    uint32_t invalid;            // key of lookups without a row (sorted last)
    int32_t l_blocks;            // work kernel: blocks [0, l_blocks) take long pieces,
    int32_t s_blocks;            // the next s_blocks one-lookup segments, the rest short ones
    Ctr* ctr;
    double* carry;               // [n_pieces][2][dim]
    Owner* owners;               // long segments
    uint2* singles;              // (row, gradient row) of one-lookup segments
    Multi* multis;
    int64_t* n_unique;
    const uint32_t* sort_err;    // set if a radix pass timed out: nothing is updated
    int32_t* status;             // the blocks' sticky status
    OptParams op;
};

template <int D, bool BF16>
struct Geo {
    static constexpr int VEC = BF16 ? 8 : 4;     // weight elements per lane (16 bytes)
    static constexpr int LPR = D / VEC;
    static constexpr int BLOCK = (64 * LPR < 256) ? 64 * LPR : 256;
    static constexpr int GPB = BLOCK / LPR;      // pieces (groups) per block, <= 64
    // Lookups per piece.  fp32 rows of at most 4 lanes (dim 16 and less)
    // take 32: more, shorter pieces spread a small batch's hot-row gathers
    // over more groups (multi-hot dim-16 update 0.032 -> 0.024 ms).  Other
    // rows take 64 (measured with 32: bf16 dim-32 update +3.5%, click-log
    // step +2%).
    static constexpr int P = (!BF16 && LPR <= 4) ? 32 : 64;
    static_assert(P >= P_MIN && LONG_T >= P - 1, "piece length");
    static constexpr int WIN = GPB * P + 2 * HALO;
    // gradient rows a group keeps in flight: 128 bytes per lane either way
    // (a bf16 row holds 8 elements per lane, so its fp32 gradient row takes
    // 32 bytes per lane); fewer registers, more resident waves
    static constexpr int GRAD_U = VEC >= 8 ? 4 : 8;
};

// ------------------------------------------------------------- pairs -----
__global__ void k_bwd_reset(Ctr* ctr, SortPrep sp) {
    if (threadIdx.x == 0) {
        ctr->bad = 0;
        ctr->n_single = 0;
        ctr->n_multi = 0;
        ctr->n_owners = 0;
        *sp.error = 0;
    }
    if (threadIdx.x < SORT_MAX_PASSES) sp.tile_ctr[threadIdx.x] = 0;
    for (int k = threadIdx.x; k < SORT_TOTAL_COPIES * SORT_COPY_STRIDE; k += blockDim.x) sp.totals[k] = 0;
}

// An apply with no lookups still reports its distinct-row count (0).
__global__ void k_zero_count(int64_t* n_unique) {
    if (threadIdx.x == 0) *n_unique = 0;
}

// Key = row (or `invalid`), value = the lookup's gradient row b * n_tables + t
// (the layout of grad), so the reduction reads gradients without any
// division.  Each block takes a contiguous run of bags, PAIRS_BAGS bags at a
// time: their offsets are staged in LDS (and checked), then the threads take
// the lookups of those bags in coalesced strides, PAIRS_U per thread in
// flight, each finding its bag by binary search in LDS.  Malformed bag
// offsets or rows beyond the capacity mark the call bad (nothing is updated).
// The kernel also builds the radix sort's digit histograms of every pass
// (block-local in LDS, then added to one of the totals' copies) and clears the sort's
// look-back state; on bad input it raises the sort's error flag so that no
// pass runs (unwritten keys would not match the totals).
constexpr int PAIRS_BLOCK = 256;
constexpr int PAIRS_BAGS = 1024;     // bags staged at a time (one-hot: 4 lookups per thread)
constexpr int PAIRS_U = 4;
constexpr int PAIRS_GRID = 2048;     // bounds the histogram flush: a few thousand atomics per bin

__global__ __launch_bounds__(PAIRS_BLOCK) void k_pairs(const int64_t* row_off, const int64_t* bag_off,
                                                       int64_t n_bags, int64_t n_ids, int64_t batch,
                                                       int32_t n_tables, int64_t capacity, uint32_t invalid,
                                                       uint2* pairs, Ctr* ctr, int32_t* status,
                                                       SortPrep sp, int passes, int width) {
    latency_bound_priority();
    __shared__ uint32_t s_hist[SORT_MAX_PASSES * SORT_MAX_BINS];
    __shared__ int64_t s_off[PAIRS_BAGS + 1];
    __shared__ int s_bad;
    for (int q = threadIdx.x; q < SORT_MAX_PASSES * SORT_MAX_BINS; q += blockDim.x) s_hist[q] = 0;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < sp.state_words;
         q += (int64_t)gridDim.x * blockDim.x)
        sp.state[q] = 0;
    if (threadIdx.x == 0) s_bad = 0;
    bool bad = false;                  // a row beyond the capacity (this thread)
    const int64_t per = (n_bags + gridDim.x - 1) / gridDim.x;
    const int64_t jb0 = (int64_t)blockIdx.x * per;
    const int64_t jb1 = jb0 + per < n_bags ? jb0 + per : n_bags;
    for (int64_t j0 = jb0; j0 < jb1; j0 += PAIRS_BAGS) {
        const int nbk = (int)(jb1 - j0 < PAIRS_BAGS ? jb1 - j0 : PAIRS_BAGS);
        __syncthreads();               // s_off of the previous run has been read
        for (int q = threadIdx.x; q <= nbk; q += PAIRS_BLOCK) s_off[q] = bag_off[j0 + q];
        __syncthreads();
        for (int q = threadIdx.x; q < nbk; q += PAIRS_BLOCK) {
            const int64_t j = j0 + q;
            const int64_t s = s_off[q], e = s_off[q + 1];
            if (s < 0 || e < s || e > n_ids || (j == 0 && s != 0) || (j == n_bags - 1 && e != n_ids)) s_bad = 1;
        }
        __syncthreads();
        if (s_bad) break;
        const int64_t L0 = s_off[0], L1 = s_off[nbk];
        for (int64_t i0 = L0 + threadIdx.x; i0 < L1; i0 += (int64_t)PAIRS_BLOCK * PAIRS_U) {
            int64_t r[PAIRS_U];
#pragma unroll
            for (int u = 0; u < PAIRS_U; ++u) {
                const int64_t i = i0 + (int64_t)u * PAIRS_BLOCK;
                r[u] = row_off[i < L1 ? i : L1 - 1];
            }
#pragma unroll
            for (int u = 0; u < PAIRS_U; ++u) {
                const int64_t i = i0 + (int64_t)u * PAIRS_BLOCK;
                if (i >= L1) break;
                // the bag of lookup i: the last k < nbk with s_off[k] <= i
                int lo = 0, hi = nbk;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_off[mid] <= i) lo = mid;
                    else hi = mid;
                }
                const int64_t j = j0 + lo;
                const uint32_t t = (uint32_t)((uint64_t)j / (uint64_t)batch);
                const uint32_t gr = (uint32_t)(j - (int64_t)t * batch) * (uint32_t)n_tables + t;
                uint32_t k = invalid;
                if (r[u] >= 0) {
                    if (r[u] >= capacity) bad = true;
                    else k = (uint32_t)r[u];
                }
                pairs[i] = make_uint2(k, gr);
                sort_hist_add(s_hist, k, passes, width);
            }
        }
    }
    if (bad || (threadIdx.x == 0 && s_bad)) {
        ctr->bad = 1;
        atomicExch(sp.error, 2u);
        atomicCAS(status, 0, (int32_t)RSE_ERR_BAD_INPUT);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < passes * SORT_MAX_BINS; q += blockDim.x)
        if (s_hist[q]) atomicAdd(&sp.totals[(blockIdx.x % SORT_TOTAL_COPIES) * SORT_COPY_STRIDE + q], s_hist[q]);
}

// ------------------------------------------------------ grad gather ------
template <int D, bool BF16>
__device__ __forceinline__ const float* grad_row(const BwdArgs& a, uint32_t gr, int li) {
    return a.grad + (int64_t)gr * D + li * Geo<D, BF16>::VEC;
}

// 1 / length of the bag whose gradient row is gr = b * n_tables + t (mean
// pooling only; a bag that holds a lookup is not empty).  One division per
// lookup; each element's share is then a product (within one fp64 rounding
// of the quotient).
__device__ __forceinline__ double inv_bag_len(const BwdArgs& a, uint32_t gr) { return a.inv_len[gr]; }

// Mean pooling: 1 / length of every bag, indexed by the bag's gradient row
// b * n_tables + t, computed once per bag before the update (each lookup
// then reads one 8-byte value that stays in L2, instead of two bag offsets
// and an fp64 division; the values are the same).
__global__ void k_inv_len(const int64_t* bag_off, int64_t batch, int32_t n_tables, double* inv) {
    const int64_t n_bags = batch * n_tables;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_bags;
         j += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = j / batch, b = j - t * batch;
        const int64_t len = bag_off[j + 1] - bag_off[j];
        inv[b * n_tables + t] = len > 0 ? 1.0 / (double)len : 0.0;
    }
}

template <int VEC, bool NT = false>
__device__ __forceinline__ void load_grad(float* out, const float* src) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
        const f32x4 v = gload_f4x<NT>(src + k);
        out[k] = v.x;
        out[k + 1] = v.y;
        out[k + 2] = v.z;
        out[k + 3] = v.w;
    }
}

template <int VEC, bool MEAN>
__device__ __forceinline__ void add_grad(double* acc, const float* gv, double inv_len) {
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        double g = (double)gv[k];
        if (MEAN) g = g * inv_len;
        acc[k] += g;
    }
}

// acc += sum over window positions [x, y) of the LDS-staged bag ids, in
// order.  U gradient rows are loaded together (all loads issued before any
// is used); a last step shorter than U repeats the range's last row (masked
// out of the sum), so a ragged end costs one round trip, not one per row.
template <int D, bool BF16, bool MEAN, bool ONCE>
__device__ __forceinline__ void sum_range(const BwdArgs& a, const uint32_t* s_vals, int x, int y, int li,
                                          double* acc) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int U = Geo<D, BF16>::GRAD_U;
    for (int q = x; q < y; q += U) {
        float gv[U][VEC];
        uint32_t j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = s_vals[q + u < y ? q + u : y - 1];
#pragma unroll
        for (int u = 0; u < U; ++u) load_grad<VEC, ONCE>(gv[u], grad_row<D, BF16>(a, j[u], li));
        double inv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) inv[u] = MEAN ? inv_bag_len(a, j[u]) : 1.0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (q + u < y) add_grad<VEC, MEAN>(acc, gv[u], inv[u]);
    }
}

// ---------------------------------------------------------- epilogue -----
// sqrt(x) for fp32 x >= 0 (zero, normal, subnormal or infinite) to about
// 1e-14 relative: the fp32 reciprocal square root refined by one Newton step
// in fp64 (relative error e -> 1.5 e^2), then multiplied by x.  Small inputs
// are scaled by an exact power of two first.  Far cheaper than a correctly
// rounded fp64 square root, and the result rounds to the same fp32 / bf16
// storage value except within ~1e-14 of a rounding boundary.
__device__ __forceinline__ double sqrt_refined(float x) {
    const bool small = x < 0x1p-100f;
    const float xs = small ? x * 0x1p100f : x;
    const double xd = (double)xs;
    const double y0 = (double)__builtin_amdgcn_rsqf(xs);
    const double y1 = y0 * (1.5 - 0.5 * xd * y0 * y0);
    double r = xd * y1;
    r = small ? r * 0x1p-50 : r;
    r = xs == 0.0f ? 0.0 : r;
    return xs == __builtin_inff() ? (double)xs : r;
}

// 1 / d for fp64 d >= 0 to about 1e-14 relative: d = m * 2^e with m in
// [0.5, 1), the fp32 reciprocal of m refined by one Newton step in fp64
// (error e -> e^2), then scaled by 2^-e.  d = 0 gives infinity, d = infinity
// gives 0.
__device__ __forceinline__ double rcp_refined(double d) {
    const double m = __builtin_amdgcn_frexp_mant(d);
    const int e = __builtin_amdgcn_frexp_exp(d);
    const double r0 = (double)__builtin_amdgcn_rcpf((float)m);
    const double r = __builtin_amdgcn_ldexp(r0 * (2.0 - m * r0), -e);
    return d == 0.0 ? __builtin_inf() : (d == __builtin_inf() ? 0.0 : r);
}

template <int D, bool BF16>
struct RowRegs {
    static constexpr int VEC = Geo<D, BF16>::VEC;
    u32x4 w;
    float st0[VEC];
    float st1[VEC];
};

template <int D, bool BF16, int OPT, bool NT = false>
__device__ __forceinline__ void load_row(const char* row, int li, RowRegs<D, BF16>& r) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int64_t W_BYTES = (int64_t)D * (BF16 ? 2 : 4);
    r.w = gload_u4x<NT>(row + li * 16);
    const float* st0 = reinterpret_cast<const float*>(row + W_BYTES) + li * VEC;
    if (OPT != RSE_SGD) load_grad<VEC, NT>(r.st0, st0);
    if (OPT == RSE_ADAM) load_grad<VEC, NT>(r.st1, st0 + D);
}

template <int D, bool BF16, int OPT, bool NT = false>
__device__ __forceinline__ void finish_row(const BwdArgs& a, char* row, int li, const RowRegs<D, BF16>& r,
                                           const double* g) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int64_t W_BYTES = (int64_t)D * (BF16 ? 2 : 4);
    double w[VEC];
    if (!BF16) {
        w[0] = __uint_as_float(r.w.x);
        w[1] = __uint_as_float(r.w.y);
        w[2] = __uint_as_float(r.w.z);
        w[3] = __uint_as_float(r.w.w);
    } else {
        const uint32_t q4[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w[2 * k] = __uint_as_float(q4[k] << 16);
            w[2 * k + 1] = __uint_as_float(q4[k] & 0xFFFF0000u);
        }
    }
    float* st0 = reinterpret_cast<float*>(row + W_BYTES) + li * VEC;
    float* st1 = st0 + D;
    double wn[VEC];
    if (OPT == RSE_SGD) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) wn[k] = w[k] - a.op.lr * g[k];
    } else if (OPT == RSE_ADAGRAD) {
        float acc[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float an = (float)((double)r.st0[k] + g[k] * g[k]);
            acc[k] = an;
            wn[k] = w[k] - a.op.lr * (g[k] * rcp_refined(sqrt_refined(an) + a.op.eps));
        }
#pragma unroll
        for (int k = 0; k < VEC; k += 4)
            gstore_f4x<NT>(st0 + k, f32x4{acc[k], acc[k + 1], acc[k + 2], acc[k + 3]});
    } else {
        float m[VEC], v[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float mn = (float)(a.op.b1 * (double)r.st0[k] + a.op.omb1 * g[k]);
            const float vn = (float)(a.op.b2 * (double)r.st1[k] + a.op.omb2 * g[k] * g[k]);
            m[k] = mn;
            v[k] = vn;
            // m / (1 - b1^t) and sqrt(v / (1 - b2^t)) = sqrt(v) * sqrt(1 / (1 - b2^t))
            const double mh = (double)mn * a.op.inv_bc1;
            const double sv = sqrt_refined(vn) * a.op.sq_inv_bc2;
            wn[k] = w[k] - a.op.lr * (mh * rcp_refined(sv + a.op.eps));
        }
#pragma unroll
        for (int k = 0; k < VEC; k += 4) {
            gstore_f4x<NT>(st0 + k, f32x4{m[k], m[k + 1], m[k + 2], m[k + 3]});
            gstore_f4x<NT>(st1 + k, f32x4{v[k], v[k + 1], v[k + 2], v[k + 3]});
        }
    }
    u32x4 out;
    if (!BF16) {
        out = u32x4{__float_as_uint((float)wn[0]), __float_as_uint((float)wn[1]), __float_as_uint((float)wn[2]),
                    __float_as_uint((float)wn[3])};
    } else {
        uint32_t q4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            q4[k] = (uint32_t)f64_to_bf16_rne(wn[2 * k]) | ((uint32_t)f64_to_bf16_rne(wn[2 * k + 1]) << 16);
        out = u32x4{q4[0], q4[1], q4[2], q4[3]};
    }
    gstore_u4x<NT>(row + li * 16, out);
}

// ------------------------------------------------- segmented update ------
// Head flags of the LDS window as one 64-bit mask per 64 positions (one
// ballot per wave-sized chunk), so the bounds of a segment are found with a
// few bit scans instead of walking the keys.
template <int NMASK>
struct HeadMasks {
    unsigned long long m[NMASK];
};

// First head strictly after window position x (x in [0, wn)); wn if none.
template <int NMASK>
__device__ __forceinline__ int next_head(const unsigned long long* m, int x, int wn) {
    if (x + 1 >= wn) return wn;
    int c = (x + 1) >> 6;
    unsigned long long bits = (x + 1) & 63 ? (m[c] & (~0ull << ((x + 1) & 63))) : m[c];
    while (true) {
        if (bits) return (c << 6) + __ffsll((long long)bits) - 1;
        if (++c >= NMASK || (c << 6) >= wn) return wn;
        bits = m[c];
    }
}

// Last head at or before window position x (position 0 is always a head).
__device__ __forceinline__ int prev_head(const unsigned long long* m, int x) {
    int c = x >> 6;
    unsigned long long bits = m[c] & (((x & 63) == 63) ? ~0ull : ((2ull << (x & 63)) - 1));
    while (!bits) bits = m[--c];
    return (c << 6) + 63 - __clzll((long long)bits);
}

// ----------------------------------------------------------- index -------
// Each block classifies the segments whose first lookup lies in its tile of
// IX_TILE sorted positions.  It stages the tile's keys plus one position
// before and HALO after (a segment of <= LONG_T lookups ends inside that
// window; one reaching past it is long) and marks heads with one ballot per
// 64 positions.  Each thread classifies IX_PER consecutive positions; a
// block-wide exclusive scan of the per-thread counts (three 16-bit fields of
// one 64-bit word) places the block's entries, and one atomic add per
// non-empty list reserves them (the order of blocks in a list is not
// fixed; nothing depends on it).
__device__ __forceinline__ uint64_t block_scan_u64(uint64_t v, uint64_t* s_wsum, uint64_t* total) {
    const int lane = lane_id(), w = threadIdx.x / WAVE;
    uint64_t x = v;
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint64_t y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) s_wsum[w] = x;
    __syncthreads();
    uint64_t pre = 0, all = 0;
    for (int q = 0; q < IX_BLOCK / WAVE; ++q) {
        if (q < w) pre += s_wsum[q];
        all += s_wsum[q];
    }
    *total = all;
    return pre + x - v;
}

__global__ __launch_bounds__(IX_BLOCK) void k_seg_index(BwdArgs a) {
    latency_bound_priority();
    __shared__ uint32_t s_keys[IX_WIN];
    __shared__ unsigned long long s_head[IX_MASKS];
    __shared__ uint64_t s_wsum[IX_BLOCK / WAVE];
    __shared__ unsigned long long s_base[3];
    if (a.ctr->bad || *a.sort_err) return;
    const int64_t n = a.n;
    const int64_t tile = blockIdx.x;
    const int64_t t0 = tile * IX_TILE;
    const int64_t t1 = t0 + IX_TILE < n ? t0 + IX_TILE : n;
    const int64_t w0 = t0 > 0 ? t0 - 1 : 0;
    const int64_t w1 = t1 + HALO < n ? t1 + HALO : n;
    const int wn = (int)(w1 - w0);
    const int lane = lane_id();
    for (int q = threadIdx.x; q < wn; q += IX_BLOCK) s_keys[q] = a.pairs[w0 + q].x;
    __syncthreads();
    for (int c = threadIdx.x / WAVE; c < IX_MASKS; c += IX_BLOCK / WAVE) {
        const int q = c * 64 + lane;
        const bool h = q < wn && (q == 0 ? w0 == 0 : s_keys[q] != s_keys[q - 1]);
        const unsigned long long m = __ballot(h);
        if (lane == 0) s_head[c] = m;
    }
    __syncthreads();
    const int x_first = (int)(t0 - w0) + (int)threadIdx.x * IX_PER;
    const int x_end = (int)(t1 - w0);
    int cls[IX_PER];          // 0 one lookup, 1 short, 2 long, 3 none
    int len[IX_PER];
    uint64_t cnt = 0;         // per-class counts in 16-bit fields
#pragma unroll
    for (int u = 0; u < IX_PER; ++u) {
        const int x = x_first + u;
        cls[u] = 3;
        len[u] = 0;
        if (x < x_end && ((s_head[x >> 6] >> (x & 63)) & 1ull) && s_keys[x] != a.invalid) {
            const int e = next_head<IX_MASKS>(s_head, x, wn);
            const bool ends_here = e < wn || w1 == n;
            const int l = e - x;
            cls[u] = (!ends_here || l > LONG_T) ? 2 : (l == 1 ? 0 : 1);
            len[u] = ends_here ? l : 0;      // a long segment's length only if it ends in the window
            cnt += 1ull << (16 * cls[u]);
        }
    }
    uint64_t total = 0;
    const uint64_t at = block_scan_u64(cnt, s_wsum, &total);
    if (threadIdx.x == 0) {
        const unsigned long long c0 = total & 0xFFFF, c1 = (total >> 16) & 0xFFFF, c2 = (total >> 32) & 0xFFFF;
        s_base[0] = c0 ? atomicAdd(&a.ctr->n_single, c0) : 0;
        s_base[1] = c1 ? atomicAdd(&a.ctr->n_multi, c1) : 0;
        s_base[2] = c2 ? atomicAdd(&a.ctr->n_owners, c2) : 0;
    }
    __syncthreads();
    uint64_t pos[3] = {s_base[0] + (at & 0xFFFF), s_base[1] + ((at >> 16) & 0xFFFF), s_base[2] + ((at >> 32) & 0xFFFF)};
#pragma unroll
    for (int u = 0; u < IX_PER; ++u) {
        const int x = x_first + u;
        const uint32_t p = (uint32_t)(w0 + x);
        if (cls[u] == 0) {
            a.singles[pos[0]++] = make_uint2(s_keys[x], a.pairs[p].y);
        } else if (cls[u] == 1) {
            Multi m;
            m.start = p;
            m.len = (uint32_t)len[u];
            m.key = s_keys[x];
            m.pad = 0;
            a.multis[pos[1]++] = m;
        } else if (cls[u] == 2) {
            Owner ow;
            ow.head = p;
            ow.len = (uint32_t)len[u];
            ow.key = s_keys[x];
            ow.pad = 0;
            a.owners[pos[2]++] = ow;
        }
    }
}

// ------------------------------------------------------------ work -------
// Long role, one piece per group: the part of a long segment at the
// piece's start (continuing an earlier piece) goes to carry slot 0, the part
// of a long segment starting in the piece (continuing past it) to slot 1.
// Returns whether slot 0 was written.
template <int D, bool BF16, bool MEAN, bool ONCE, int NMASK>
__device__ __forceinline__ bool walk_long(const BwdArgs& a, const uint32_t* s_keys, const uint32_t* s_vals,
                                          const unsigned long long* s_head, int wn, int64_t k, int x0, int xb,
                                          int li) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    auto is_head = [&](int q) -> bool { return (s_head[q >> 6] >> (q & 63)) & 1ull; };
    auto carry = [&](int slot, const double* acc) {
        double* dst = a.carry + ((int64_t)k * 2 + slot) * D + li * VEC;
#pragma unroll
        for (int c = 0; c < VEC; ++c) dst[c] = acc[c];
    };
    // lookups without a row sort last: stop at the head of that run
    int lim = xb;
    if (s_keys[xb - 1] == a.invalid) lim = prev_head(s_head, xb - 1);
    if (lim <= x0) return false;
    bool wrote0 = false;
    if (!is_head(x0)) {
        const int h = prev_head(s_head, x0);
        const int e = next_head<NMASK>(s_head, x0, wn);
        if (e - h > LONG_T) {
            double acc[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
            sum_range<D, BF16, MEAN, ONCE>(a, s_vals, x0, e < lim ? e : lim, li, acc);
            carry(0, acc);
            wrote0 = true;
        }
    }
    const int hl = prev_head(s_head, lim - 1);
    if (hl >= x0 && next_head<NMASK>(s_head, hl, wn) - hl > LONG_T) {
        double acc[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
        sum_range<D, BF16, MEAN, ONCE>(a, s_vals, hl, xb, li, acc);
        carry(1, acc);
    }
    return wrote0;
}

// Singles role: SPG one-lookup segments per group, their rows and gradient
// rows all requested before any is used; the group's next entries are
// requested before this round's rows, so a round waits for one memory round
// trip.
template <int D, bool BF16, int OPT, bool MEAN, bool ONCE, int SPG>
__device__ __forceinline__ void role_singles(const BwdArgs& a, const uint64_t* s_chunks, int64_t gid,
                                             int64_t n_groups, int li, int64_t lo, int64_t ns) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    if (lo + gid * SPG >= ns) return;
    uint2 e[SPG];
#pragma unroll
    for (int u = 0; u < SPG; ++u) e[u] = a.singles[lo + gid * SPG + u < ns ? lo + gid * SPG + u : ns - 1];
    for (int64_t i0 = lo + gid * SPG; i0 < ns; i0 += n_groups * SPG) {
        const int64_t inx = i0 + n_groups * SPG;
        uint2 en[SPG];
#pragma unroll
        for (int u = 0; u < SPG; ++u) en[u] = a.singles[inx + u < ns ? inx + u : ns - 1];
        char* rp[SPG];
        RowRegs<D, BF16> rr[SPG];
        float gv[SPG][VEC];
#pragma unroll
        for (int u = 0; u < SPG; ++u) {
            rp[u] = a.rv.row(s_chunks, e[u].x);
            load_row<D, BF16, OPT, ONCE>(rp[u], li, rr[u]);
        }
#pragma unroll
        for (int u = 0; u < SPG; ++u) load_grad<VEC, ONCE>(gv[u], grad_row<D, BF16>(a, e[u].y, li));
        double inv[SPG];
#pragma unroll
        for (int u = 0; u < SPG; ++u) inv[u] = MEAN ? inv_bag_len(a, e[u].y) : 1.0;
#pragma unroll
        for (int u = 0; u < SPG; ++u) {
            if (i0 + u < ns) {
                double acc[VEC];
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
                add_grad<VEC, MEAN>(acc, gv[u], inv[u]);
                finish_row<D, BF16, OPT, ONCE>(a, rp[u], li, rr[u], acc);
            }
        }
#pragma unroll
        for (int u = 0; u < SPG; ++u) e[u] = en[u];
    }
}

// Short role: one segment of 2..LONG_T lookups per group; its row is
// requested with its first gradient rows, which are summed U at a time.  The
// group's next segment descriptor is requested with this segment's row, and
// that segment's first U bag ids before this one's update, so a segment
// waits for one memory round trip per U lookups.
template <int D, bool BF16, int OPT, bool MEAN, bool ONCE>
__device__ __forceinline__ void role_multis(const BwdArgs& a, const uint64_t* s_chunks, int64_t gid,
                                            int64_t n_groups, int li, int64_t lo, int64_t nm) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int U = Geo<D, BF16>::GRAD_U;
    if (lo + gid >= nm) return;
    Multi m = a.multis[lo + gid];
    uint32_t j[U];
#pragma unroll
    for (int u = 0; u < U; ++u) j[u] = a.pairs[m.start + (u < (int)m.len ? u : m.len - 1)].y;
    for (int64_t i = lo + gid; i < nm; i += n_groups) {
        const int64_t inx = i + n_groups;
        const Multi mn = a.multis[inx < nm ? inx : nm - 1];
        char* rp = a.rv.row(s_chunks, m.key);
        RowRegs<D, BF16> rr;
        load_row<D, BF16, OPT, ONCE>(rp, li, rr);
        double acc[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
        uint32_t c0 = 0;
        while (true) {
            float gv[U][VEC];
#pragma unroll
            for (int u = 0; u < U; ++u) load_grad<VEC, ONCE>(gv[u], grad_row<D, BF16>(a, j[u], li));
            double inv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) inv[u] = MEAN ? inv_bag_len(a, j[u]) : 1.0;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u < m.len) add_grad<VEC, MEAN>(acc, gv[u], inv[u]);
            c0 += U;
            if (c0 >= m.len) break;
#pragma unroll
            for (int u = 0; u < U; ++u) j[u] = a.pairs[m.start + (c0 + u < m.len ? c0 + u : m.len - 1)].y;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = a.pairs[mn.start + (u < (int)mn.len ? u : mn.len - 1)].y;
        finish_row<D, BF16, OPT, ONCE>(a, rp, li, rr, acc);
        m = mn;
    }
}

template <int D, bool BF16>
constexpr int singles_per_group() {
    return 2;
}

template <int D, bool BF16, int OPT, bool MEAN, bool ONCE>
__global__ __launch_bounds__((Geo<D, BF16>::BLOCK)) void k_seg_work(BwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int LPR = G::LPR, GPB = G::GPB, WIN = G::WIN, P = G::P;
    constexpr int NMASK = (WIN + 63) / 64;
    __shared__ uint32_t s_keys[WIN];
    __shared__ uint32_t s_vals[WIN];
    __shared__ unsigned long long s_head[NMASK];
    __shared__ uint64_t s_chunks[LDS_CHUNKS];
    __shared__ int s_run[GPB];     // per piece: 1 slot 0 written, 2 segment goes on into the next piece
    stage_chunks(s_chunks, a.rv);
    if (a.ctr->bad) return;
    if (*a.sort_err) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicCAS(a.status, 0, (int32_t)RSE_ERR_HIP);
        return;
    }
    const int g = threadIdx.x / LPR;
    const int li = threadIdx.x % LPR;
    // Roles are spread evenly over the block index (blocks start roughly in
    // index order), so gathers of long pieces and row updates of short
    // segments run side by side, in groups of N_XCD consecutive blocks (one
    // per XCD: workgroups are dispatched to the XCDs round-robin): group q is
    // the floor(q*L/Q)-th long group if that count steps at q, else a
    // one-lookup or short group, spread the same way among the rest.  Within
    // a role, XCD x takes the x-th contiguous band of the role's work (its
    // windows, or its stretch of the segment lists, which the index kernel
    // fills roughly in sorted order), so the rows and gradient rows one XCD
    // touches at a time come from a narrow stretch of the sorted order.
    const int64_t xcd = blockIdx.x % N_XCD;
    const int64_t q = blockIdx.x / N_XCD;
    const int64_t Q = gridDim.x / N_XCD;
    const int64_t L8 = a.l_blocks / N_XCD, S8 = a.s_blocks / N_XCD;
    const int64_t lq = q * L8 / Q, lq1 = (q + 1) * L8 / Q;
    if (lq1 == lq) {
        const int64_t rest = Q - L8;
        const int64_t r = q - lq1;
        const int64_t sq = r * S8 / rest, sq1 = (r + 1) * S8 / rest;
        if (sq1 > sq) {
            const int64_t ns = (int64_t)a.ctr->n_single;
            role_singles<D, BF16, OPT, MEAN, ONCE, singles_per_group<D, BF16>()>(
                a, s_chunks, sq * GPB + g, S8 * GPB, li, xcd * ns / N_XCD, (xcd + 1) * ns / N_XCD);
        } else {
            const int64_t nm = (int64_t)a.ctr->n_multi;
            role_multis<D, BF16, OPT, MEAN, ONCE>(a, s_chunks, (r - sq1) * GPB + g, (rest - S8) * GPB, li, xcd * nm / N_XCD,
                                      (xcd + 1) * nm / N_XCD);
        }
        return;
    }
    const int64_t n = a.n;
    const int64_t n_pieces = (n + P - 1) / P;
    const int lane = lane_id();
    const int wave = threadIdx.x / WAVE;
    // one window of GPB pieces per long block, XCD x taking windows
    // [x * L8, (x + 1) * L8)
    for (int64_t pb = (xcd * L8 + lq) * GPB; pb < n_pieces && pb < (xcd + 1) * L8 * GPB; pb += L8 * GPB) {
        const int64_t blk_a = pb * P;
        const int64_t blk_b = (pb + GPB) * P < n ? (pb + GPB) * P : n;
        const int64_t w0 = blk_a - HALO > 0 ? blk_a - HALO : 0;
        const int64_t w1 = blk_b + HALO < n ? blk_b + HALO : n;
        const int wn = (int)(w1 - w0);
        __syncthreads();
        for (int q = threadIdx.x; q < wn; q += G::BLOCK) {
            const uint2 pr = a.pairs[w0 + q];
            s_keys[q] = pr.x;
            s_vals[q] = pr.y;
        }
        __syncthreads();
        // window position 0 counts as a head: a segment reaching back to it
        // is at least HALO long, i.e. long either way
        for (int c = wave; c < NMASK; c += G::BLOCK / WAVE) {
            const int q = c * 64 + lane;
            const bool h = q < wn && (q == 0 || s_keys[q] != s_keys[q - 1]);
            const unsigned long long m = __ballot(h);
            if (lane == 0) s_head[c] = m;
        }
        __syncthreads();
        const int64_t k = pb + g;
        bool wrote0 = false, spans = false;
        if (k < n_pieces) {
            const int x0 = (int)(k * P - w0);
            const int xb = (int)((k * P + P < n ? k * P + P : n) - w0);
            wrote0 = walk_long<D, BF16, MEAN, ONCE, NMASK>(a, s_keys, s_vals, s_head, wn, k, x0, xb, li);
            // no head in [x0, xb]: the segment at the piece's start fills the
            // piece and goes on into the next one
            spans = k + 1 < n_pieces && next_head<NMASK>(s_head, x0 - 1, wn) > xb;
        }
        if (li == 0) s_run[g] = (wrote0 ? 1 : 0) | (spans ? 2 : 0);
        __syncthreads();       // the window's carries are written and visible to the block
        // Runs of slot-0 partials of one long segment over consecutive pieces
        // of this window are added (in piece order) into the run's first
        // piece: the combine then reads one partial per run, the run's first
        // piece being the segment's second piece or a multiple of GPB.
        const bool lead = (s_run[g] & 1) && (g == 0 || (s_run[g - 1] & 3) != 3);
        if (lead && g + 1 < GPB && (s_run[g] & 2) && (s_run[g + 1] & 1)) {
            double* dst = a.carry + (k * 2) * D + li * G::VEC;
            double acc[G::VEC];
#pragma unroll
            for (int c = 0; c < G::VEC; ++c) acc[c] = dst[c];
            for (int q = g + 1; q < GPB && (s_run[q] & 1) && (s_run[q - 1] & 2); ++q) {
                const double* src = a.carry + ((pb + q) * 2) * D + li * G::VEC;
#pragma unroll
                for (int c = 0; c < G::VEC; ++c) acc[c] += src[c];
            }
#pragma unroll
            for (int c = 0; c < G::VEC; ++c) dst[c] = acc[c];
        }
    }
}

// ------------------------------------------------- long segment combine --
// The pieces a long segment covers are its head's piece k0 (partial in
// carry slot 1) and the following pieces k0+1..k1 whose first position lies
// in the segment.  The work kernel has added the slot-0 partials of each of
// its windows' runs into the run's first piece: k0+1 and every multiple of
// its GPB in (k0+1, k1].  Blocks take chunks of owners, one per group:
//  - a segment whose length the index kernel saw (it ended inside the index
//    window: nearly every segment of up to a few thousand lookups) is
//    finished by its group alone: k1 follows from head and length, its row
//    is requested with its first partials, the partials are added in list
//    order (U loads in flight) and the row is updated;
//  - the others (the hottest rows) are then taken one at a time by the
//    whole block: k1 from block-wide counts over combine_search x block size
//    piece heads at a time (the pieces of a segment form a prefix), the
//    partials added round-robin per group (U loads in flight, in list
//    order) then in group order, and the row updated by group 0.
// Either way a segment's sum has one fixed order, the same on every run.
// Block 0 also writes the number of distinct rows (one-lookup + short + long
// segments).  Row addresses are read from the global chunk table.  A chunk
// is one owner per group for rows of up to 8 lanes (a block of 16 groups
// used to take one owner at a time, though most long segments have only 2-3
// partials: merged-table combine 150 -> 58 us alone) and one owner per
// block for wider rows (click-log and behaviour-sequence: their hottest
// rows, of unknown length, would otherwise wait in line behind the other
// owners of their block; sequence combine 15 -> 22 us with 4 per block).
constexpr int CB_GROUPS = 4;
template <int D, bool BF16>
constexpr int combine_block() {
    return CB_GROUPS * Geo<D, BF16>::LPR < 64 ? 64 : CB_GROUPS * Geo<D, BF16>::LPR;
}
template <int D, bool BF16>
constexpr int combine_search() {
    constexpr int wide = 16 * Geo<D, BF16>::LPR < 64 ? 64 : (16 * Geo<D, BF16>::LPR > 512 ? 512 : 16 * Geo<D, BF16>::LPR);
    return wide / combine_block<D, BF16>() > 1 ? wide / combine_block<D, BF16>() : 1;
}

template <int D, bool BF16>
constexpr int combine_owners_per_block() {
    return Geo<D, BF16>::LPR <= 8 ? combine_block<D, BF16>() / Geo<D, BF16>::LPR : 1;
}

template <int D, bool BF16, int OPT>
__global__ __launch_bounds__((combine_block<D, BF16>())) void k_combine(BwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int VEC = G::VEC, LPR = G::LPR, BLOCK = combine_block<D, BF16>(), GPB = BLOCK / LPR;
    constexpr int U = 4;
    constexpr int CB_SEARCH = combine_search<D, BF16>();
    constexpr int P = G::P;
    constexpr int64_t WG = G::GPB;          // the work kernel's pieces per window
    constexpr int OPB = combine_owners_per_block<D, BF16>();
    __shared__ double s_part[GPB][D];
    __shared__ int64_t s_coop[GPB];         // owners of the chunk left to the whole block
    if (a.ctr->bad || *a.sort_err) {
        if (blockIdx.x == 0 && threadIdx.x == 0) *a.n_unique = 0;    // nothing was updated
        return;
    }
    const int64_t n_pieces = (a.n + P - 1) / P;
    const int64_t n_owners = (int64_t)a.ctr->n_owners;
    const int g = threadIdx.x / LPR;
    const int li = threadIdx.x % LPR;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *a.n_unique = (int64_t)(a.ctr->n_single + a.ctr->n_multi + (unsigned long long)n_owners);
    // partial t of a segment's list: t = 0 slot 1 of k0, t = 1 slot 0 of
    // k0+1, t >= 2 slot 0 of the (t-1)-th multiple of WG after k0+1
    auto item = [&](int64_t k0, int64_t t) -> const double* {
        const int64_t k = t == 0 ? k0 : (t == 1 ? k0 + 1 : ((k0 + 1) / WG + t - 1) * WG);
        return a.carry + (k * 2 + (t == 0 ? 1 : 0)) * D + li * VEC;
    };
    auto n_items_of = [&](int64_t k0, int64_t k1) -> int64_t {
        return k1 > k0 ? 2 + (k1 / WG - (k0 + 1) / WG) : 1;
    };
    for (int64_t ob = (int64_t)blockIdx.x * OPB; ob < n_owners; ob += (int64_t)gridDim.x * OPB) {
        __syncthreads();       // s_coop and s_part of the previous chunk have been read
        const int64_t o = ob + g;
        bool coop = false;
        if (g < OPB && o < n_owners) {
            const Owner ow = a.owners[o];
            if (ow.len == 0) {
                coop = true;
            } else {
                const int64_t h = ow.head;
                const int64_t k0 = h / P;
                const int64_t n_items = n_items_of(k0, (h + (int64_t)ow.len - 1) / P);
                char* row = a.rv.row(ow.key);
                RowRegs<D, BF16> rr;
                load_row<D, BF16, OPT>(row, li, rr);
                double acc[VEC];
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
                for (int64_t t0 = 0; t0 < n_items; t0 += U) {
                    double src[U][VEC];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const double* p = item(k0, t0 + u < n_items ? t0 + u : n_items - 1);
#pragma unroll
                        for (int c = 0; c < VEC; ++c) src[u][c] = p[c];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (t0 + u < n_items)
#pragma unroll
                            for (int c = 0; c < VEC; ++c) acc[c] += src[u][c];
                }
                finish_row<D, BF16, OPT>(a, row, li, rr, acc);
            }
        }
        if (li == 0) s_coop[g] = coop ? o : -1;
        __syncthreads();
        for (int q = 0; q < OPB; ++q) {
            const int64_t oc = s_coop[q];      // the same for every thread of the block
            if (oc < 0) continue;
            __syncthreads();                   // s_part of the previous owner has been read
            const Owner ow = a.owners[oc];
            const int64_t h = ow.head;
            const uint32_t key = ow.key;
            const int64_t k0 = h / P;
            int64_t k1 = k0;
            for (int64_t kb = k0 + 1;; kb += BLOCK * CB_SEARCH) {
                uint32_t kk[CB_SEARCH];
#pragma unroll
                for (int u = 0; u < CB_SEARCH; ++u) {
                    const int64_t k = kb + u * BLOCK + threadIdx.x;
                    kk[u] = a.pairs[(k < n_pieces ? k : n_pieces - 1) * P].x;
                }
                int cnt = 0;
#pragma unroll
                for (int u = 0; u < CB_SEARCH; ++u)
                    cnt += __syncthreads_count(kb + u * BLOCK + threadIdx.x < n_pieces && kk[u] == key);
                k1 += cnt;
                if (cnt < BLOCK * CB_SEARCH) break;
            }
            const int64_t n_items = n_items_of(k0, k1);
            double acc[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
            for (int64_t tq = g; tq < n_items; tq += U * GPB) {
                double src[U][VEC];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const double* p = item(k0, tq + u * GPB < n_items ? tq + u * GPB : n_items - 1);
#pragma unroll
                    for (int c = 0; c < VEC; ++c) src[u][c] = p[c];
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (tq + u * GPB < n_items)
#pragma unroll
                        for (int c = 0; c < VEC; ++c) acc[c] += src[u][c];
            }
#pragma unroll
            for (int c = 0; c < VEC; ++c) s_part[g][li * VEC + c] = acc[c];
            __syncthreads();
            if (g == 0) {
                double tot[VEC];
#pragma unroll
                for (int c = 0; c < VEC; ++c) tot[c] = s_part[0][li * VEC + c];
#pragma unroll 1
                for (int q2 = 1; q2 < GPB; ++q2)
#pragma unroll
                    for (int c = 0; c < VEC; ++c) tot[c] += s_part[q2][li * VEC + c];
                char* row = a.rv.row(key);
                RowRegs<D, BF16> rr;
                load_row<D, BF16, OPT>(row, li, rr);
                finish_row<D, BF16, OPT>(a, row, li, rr, tot);
            }
        }
    }
}

// Workspace of one call.
struct BwdWs {
    Ctr* ctr;
    uint2* p0;
    uint2* p1;
    double* carry;
    Owner* owners;
    uint2* singles;
    Multi* multis;
    void* sort_ws;
    double* inv_len;
};

BwdWs carve(void* base, int64_t n_ids, int64_t n_bags, int32_t dim, size_t* total) {
    Carver c(base);
    BwdWs w;
    const size_t n = (size_t)(n_ids > 0 ? n_ids : 1);
    const size_t n_pieces = (n + P_MIN - 1) / P_MIN;    // carry slots for any piece length
    w.ctr = c.take<Ctr>(1);
    w.p0 = c.take<uint2>(n);
    w.p1 = c.take<uint2>(n);
    w.carry = c.take<double>(n_pieces * 2 * (size_t)dim);
    w.owners = c.take<Owner>(n / (LONG_T + 1) + 1);
    w.singles = c.take<uint2>(n);
    w.multis = c.take<Multi>(n / 2 + 1);
    w.sort_ws = c.take<char>(sort_workspace((int64_t)n, nullptr));
    w.inv_len = c.take<double>((size_t)(n_bags > 0 ? n_bags : 1));
    if (total) *total = c.size();
    return w;
}

template <int D, bool BF16, int OPT>
int launch_update(BwdArgs a, int64_t n_ids, hipStream_t s) {
    using G = Geo<D, BF16>;
    const int64_t n_pieces = (n_ids + G::P - 1) / G::P;
    // long pieces: one block per GPB pieces; one-lookup and short segments:
    // grid-stride pools (their counts are only known on the device), sized
    // for a few passes when one lookup in ~16 starts a segment
    // every count a multiple of N_XCD (one block of each group of N_XCD per
    // XCD); the long role has one block per window of GPB pieces
    a.l_blocks = (int32_t)(N_XCD * ((n_pieces + (int64_t)G::GPB * N_XCD - 1) / ((int64_t)G::GPB * N_XCD)));
    // with 32 or more lanes per row (rows of 512 bytes and up) half as many
    // pool blocks keep as many bytes in flight, and more of them crowd out
    // the long-piece blocks (measured: click-log update 0.338 -> 0.328 ms;
    // the dim-64 and dim-32 workloads are slower with the smaller pools)
    constexpr int POOL_CAP = G::LPR >= 32 ? 1024 : 2048;
    a.s_blocks = N_XCD * ((fill_blocks(n_ids, G::GPB * singles_per_group<D, BF16>() * 8, POOL_CAP) + N_XCD - 1) / N_XCD);
    const int m_blocks = N_XCD * ((fill_blocks(n_ids, G::GPB * 16, POOL_CAP) + N_XCD - 1) / N_XCD);
    const int64_t work_blocks = (int64_t)a.l_blocks + a.s_blocks + m_blocks;
    constexpr int CB = combine_block<D, BF16>();
    // one chunk of owners per block; at most n / (LONG_T + 1) + 1 owners
    const int cblocks = fill_blocks(n_ids / (LONG_T + 1) + 1, combine_owners_per_block<D, BF16>(), 2048 * 512 / CB);
    {
        TraceScope ts(RSE_K_SEG_UPDATE, s);
        // With no more lookups than bags (one-hot batches), a gradient row is
        // read about once, like every touched row: the update then reads
        // and writes both with the nontemporal hint, so that they stream
        // through the caches and leave in place the lines that are read
        // again, such as the sorted pairs (click-log update 0.29 -> 0.27 ms,
        // step 0.60 -> 0.56 ms).  With longer bags a gradient row is read
        // once per lookup and should stay cached between its reads.
        const dim3 grid((unsigned)work_blocks), block(G::BLOCK);
        if (a.n <= (int64_t)a.n_tables * a.batch) {
            if (a.mean) hipLaunchKernelGGL((k_seg_work<D, BF16, OPT, true, true>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_seg_work<D, BF16, OPT, false, true>), grid, block, 0, s, a);
        } else {
            if (a.mean) hipLaunchKernelGGL((k_seg_work<D, BF16, OPT, true, false>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_seg_work<D, BF16, OPT, false, false>), grid, block, 0, s, a);
        }
    }
    {
        TraceScope ts(RSE_K_COMBINE, s);
        hipLaunchKernelGGL((k_combine<D, BF16, OPT>), dim3(cblocks), dim3(CB), 0, s, a);
    }
    return launch_status();
}

template <int D, bool BF16>
int dispatch_opt(const BwdArgs& a, int optim, int64_t n_ids, hipStream_t s) {
    switch (optim) {
        case RSE_SGD: return launch_update<D, BF16, RSE_SGD>(a, n_ids, s);
        case RSE_ADAGRAD: return launch_update<D, BF16, RSE_ADAGRAD>(a, n_ids, s);
        case RSE_ADAM: return launch_update<D, BF16, RSE_ADAM>(a, n_ids, s);
        default: return RSE_ERR_INVALID_ARG;
    }
}

int dispatch(const BwdArgs& a, int dim, bool bf, int optim, int64_t n_ids, hipStream_t s) {
    switch (dim) {
        case 4: return bf ? RSE_ERR_UNSUPPORTED : dispatch_opt<4, false>(a, optim, n_ids, s);
        case 8: return bf ? dispatch_opt<8, true>(a, optim, n_ids, s) : dispatch_opt<8, false>(a, optim, n_ids, s);
        case 16: return bf ? dispatch_opt<16, true>(a, optim, n_ids, s) : dispatch_opt<16, false>(a, optim, n_ids, s);
        case 32: return bf ? dispatch_opt<32, true>(a, optim, n_ids, s) : dispatch_opt<32, false>(a, optim, n_ids, s);
        case 64: return bf ? dispatch_opt<64, true>(a, optim, n_ids, s) : dispatch_opt<64, false>(a, optim, n_ids, s);
        case 128: return bf ? dispatch_opt<128, true>(a, optim, n_ids, s) : dispatch_opt<128, false>(a, optim, n_ids, s);
        case 256: return bf ? dispatch_opt<256, true>(a, optim, n_ids, s) : dispatch_opt<256, false>(a, optim, n_ids, s);
        default: return RSE_ERR_UNSUPPORTED;
    }
}

int bit_length(uint64_t x) {
    int b = 0;
    while (x) {
        ++b;
        x >>= 1;
    }
    return b;
}

}  // namespace

extern "C" {

int rse_bwd_workspace_size(int64_t n_ids, int32_t n_tables, int64_t batch, int32_t dim, size_t* bytes_out) {
    if (!bytes_out || n_ids < 0 || n_tables <= 0 || batch < 0 || dim <= 0) return RSE_ERR_INVALID_ARG;
    carve(nullptr, n_ids, (int64_t)n_tables * batch, dim, bytes_out);
    return RSE_OK;
}

int embedding_bag_bwd_prepare(rse_blocks* blocks, const int64_t* d_row_off, int64_t n_ids,
                              const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch, void* d_ws,
                              size_t ws_bytes, rse_bwd_plan* plan_out, void* stream) {
    if (!blocks || !d_bag_offsets || !d_ws || !plan_out) return RSE_ERR_INVALID_ARG;
    if (n_ids < 0 || n_tables <= 0 || batch < 0) return RSE_ERR_INVALID_ARG;
    if (n_ids > 0 && !d_row_off) return RSE_ERR_INVALID_ARG;
    const int64_t n_bags = (int64_t)n_tables * batch;
    if (n_ids > RSE_MAX_BWD_IDS || n_bags > (int64_t)0xFFFFFFFFll) return RSE_ERR_INVALID_ARG;
    size_t need = 0;
    BwdWs w = carve(d_ws, n_ids, n_bags, blocks->dim, &need);
    if (ws_bytes < need) return RSE_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    SortPrep sp = sort_prep(w.sort_ws, n_ids);
    const int64_t capacity = blocks->capacity();
    int bits = bit_length((uint64_t)capacity);
    if (bits < 1) bits = 1;
    const uint32_t invalid = bits >= 32 ? 0xFFFFFFFFu : ((1u << bits) - 1u);
    // every host-side check comes before the first launch
    if (!sort_supported(n_ids, bits)) return RSE_ERR_UNSUPPORTED;
    rse_bwd_plan plan;
    plan.n_ids = n_ids;
    plan.n_bags = n_bags;
    plan.invalid = invalid;
    plan.key_bits = bits;
    plan.sorted_in_alt = 0;
    plan.dim = blocks->dim;
    hipLaunchKernelGGL(k_bwd_reset, dim3(1), dim3(256), 0, s, w.ctr, sp);
    if (n_ids > 0 && n_bags > 0) {
        const SortPlan sp_plan = sort_plan(bits);
        sp.state_words = sp.state_words / SORT_MAX_PASSES * sp_plan.passes;   // only the passes that run
        // enough blocks for the bags (one staging run each) and for the lookups
        // (a few strides per thread when bags are long)
        const int64_t pairs_units = std::max((n_bags + PAIRS_BAGS - 1) / PAIRS_BAGS,
                                             (n_ids + PAIRS_BLOCK * PAIRS_U * 4 - 1) / (PAIRS_BLOCK * PAIRS_U * 4));
        hipLaunchKernelGGL(k_pairs, dim3(fill_blocks(pairs_units, 1, PAIRS_GRID)), dim3(PAIRS_BLOCK), 0, s,
                           d_row_off,
                           d_bag_offsets, n_bags, n_ids, batch, n_tables, capacity, invalid, w.p0, w.ctr,
                           &blocks->header()->status, sp, sp_plan.passes, sp_plan.width);
        bool alt = false;
        const int rc = radix_sort_pairs(w.p0, w.p1, n_ids, bits, w.sort_ws, &alt, s);
        if (rc) return rc;
        plan.sorted_in_alt = alt ? 1 : 0;
        // the segment index needs only the sorted pairs
        BwdArgs ia = {};
        ia.pairs = alt ? w.p1 : w.p0;
        ia.n = n_ids;
        ia.invalid = invalid;
        ia.ctr = w.ctr;
        ia.sort_err = sp.error;
        ia.owners = w.owners;
        ia.singles = w.singles;
        ia.multis = w.multis;
        const int64_t ix_blocks = (n_ids + IX_TILE - 1) / IX_TILE;
        hipLaunchKernelGGL(k_seg_index, dim3((unsigned)ix_blocks), dim3(IX_BLOCK), 0, s, ia);
    }
    const int rc = launch_status();
    if (rc == RSE_OK) *plan_out = plan;
    return rc;
}

int embedding_bag_bwd_apply(rse_blocks* blocks, const rse_bwd_plan* plan, const int64_t* d_bag_offsets,
                            int32_t n_tables, int64_t batch, int32_t pooling, const float* d_grad,
                            const rse_optim* opt, int64_t* d_n_unique_out, void* d_ws, size_t ws_bytes,
                            void* stream) {
    if (!blocks || !plan || !d_bag_offsets || !opt || !d_n_unique_out || !d_ws) return RSE_ERR_INVALID_ARG;
    if (n_tables <= 0 || batch < 0 || plan->n_ids < 0 || plan->n_ids > RSE_MAX_BWD_IDS)
        return RSE_ERR_INVALID_ARG;
    const int64_t n_ids = plan->n_ids;
    const int64_t n_bags = (int64_t)n_tables * batch;
    if (plan->n_bags != n_bags || plan->dim != blocks->dim) return RSE_ERR_INVALID_ARG;
    if (plan->key_bits < 1 || plan->key_bits > 32) return RSE_ERR_INVALID_ARG;
    if (n_ids > 0 && !d_grad) return RSE_ERR_INVALID_ARG;
    if (pooling != RSE_SUM && pooling != RSE_MEAN) return RSE_ERR_INVALID_ARG;
    if (opt->kind != blocks->optim) return RSE_ERR_INVALID_ARG;
    if (opt->kind == RSE_ADAM && opt->step < 1) return RSE_ERR_INVALID_ARG;
    size_t need = 0;
    BwdWs w = carve(d_ws, n_ids, n_bags, blocks->dim, &need);
    if (ws_bytes < need) return RSE_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    SortPrep sp = sort_prep(w.sort_ws, n_ids);
    if (n_ids == 0 || n_bags == 0) {
        hipLaunchKernelGGL(k_zero_count, dim3(1), dim3(64), 0, s, d_n_unique_out);
        return launch_status();
    }

    BwdArgs a;
    a.rv = blocks->view();
    a.pairs = plan->sorted_in_alt ? w.p1 : w.p0;
    a.bag_off = d_bag_offsets;
    a.inv_len = w.inv_len;
    a.grad = d_grad;
    a.batch = batch;
    a.n_tables = n_tables;
    a.mean = pooling == RSE_MEAN;
    a.n = n_ids;
    a.invalid = plan->invalid;
    a.l_blocks = 0;
    a.s_blocks = 0;
    a.ctr = w.ctr;
    a.carry = w.carry;
    a.owners = w.owners;
    a.singles = w.singles;
    a.multis = w.multis;
    a.n_unique = d_n_unique_out;
    a.sort_err = sp.error;
    a.status = &blocks->header()->status;
    a.op.lr = opt->lr;
    a.op.eps = opt->eps;
    a.op.b1 = opt->beta1;
    a.op.b2 = opt->beta2;
    a.op.omb1 = 1.0 - opt->beta1;
    a.op.omb2 = 1.0 - opt->beta2;
    a.op.inv_bc1 = opt->kind == RSE_ADAM ? 1.0 / (1.0 - std::pow(opt->beta1, (double)opt->step)) : 1.0;
    a.op.sq_inv_bc2 = opt->kind == RSE_ADAM ? std::sqrt(1.0 / (1.0 - std::pow(opt->beta2, (double)opt->step))) : 1.0;
    if (a.mean)
        hipLaunchKernelGGL(k_inv_len, dim3(fill_blocks(n_bags, 256, 4096)), dim3(256), 0, s, d_bag_offsets, batch,
                           n_tables, w.inv_len);
    return dispatch(a, blocks->dim, blocks->w_dtype == RSE_BF16, opt->kind, n_ids, s);
}

int embedding_bag_bwd_update(rse_blocks* blocks, const int64_t* d_row_off, int64_t n_ids,
                             const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch,
                             int32_t pooling, const float* d_grad, const rse_optim* opt,
                             int64_t* d_n_unique_out, void* d_ws, size_t ws_bytes, void* stream) {
    if (!blocks || !d_bag_offsets || !opt || !d_n_unique_out || !d_ws) return RSE_ERR_INVALID_ARG;
    if (n_ids > 0 && (!d_row_off || !d_grad)) return RSE_ERR_INVALID_ARG;
    if (pooling != RSE_SUM && pooling != RSE_MEAN) return RSE_ERR_INVALID_ARG;
    if (opt->kind != blocks->optim) return RSE_ERR_INVALID_ARG;
    if (opt->kind == RSE_ADAM && opt->step < 1) return RSE_ERR_INVALID_ARG;
    rse_bwd_plan plan;
    int rc = embedding_bag_bwd_prepare(blocks, d_row_off, n_ids, d_bag_offsets, n_tables, batch, d_ws, ws_bytes,
                                       &plan, stream);
    if (rc) return rc;
    return embedding_bag_bwd_apply(blocks, &plan, d_bag_offsets, n_tables, batch, pooling, d_grad, opt,
                                   d_n_unique_out, d_ws, ws_bytes, stream);
}

}  // extern "C"
