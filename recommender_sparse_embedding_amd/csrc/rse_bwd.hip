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
//   row;
//   apply (needs the upstream gradient):  reset of its counters ->
//   segmented reduction with the optimizer fused in -> combine of long
//   segments.
//
// Segmented reduction.  The sorted lookups are cut into pieces of P = 64.
// A segment (all lookups of one row) of length <= LONG_T = 128 is reduced
// entirely by the group of lanes whose piece holds its first lookup, in
// lookup order, in fp64, and the row is updated right there: the gradient
// row never goes to memory.  A longer segment is reduced piecewise: every
// piece it covers writes its fp64 partial to a carry slot, and the piece
// holding its first lookup is listed as owner; the combine kernel adds the
// partials in a fixed order (round-robin over a block's groups, then group
// order) and updates the row.  Each block stages the keys and bag ids of its
// pieces (plus LONG_T + 1 on either side) in LDS, so segment bounds are found
// without global binary searches.  Only integer atomics (counters) are used;
// results do not depend on timing.
#include <cmath>

#include "rse_sort.h"

using namespace rse;
using namespace rse_host;

namespace {

constexpr int P = 64;            // lookups per piece
constexpr int LONG_T = 128;      // longest segment reduced by one group
constexpr int HALO = LONG_T + 1;
constexpr int MAX_SEG_BLOCKS = 65535;

struct OptParams {
    double lr, eps, b1, b2, omb1, omb2, bc1, bc2;
};

struct Ctr {                     // device counters of one call
    unsigned long long n_owners;
    unsigned long long bad;
    unsigned long long pad[6];
};

struct BwdArgs {
    RowsView rv;
    const uint32_t* keys;        // sorted rows
    const uint32_t* vals;        // bag of each sorted lookup
    const int64_t* bag_off;
    const float* grad;           // [batch, n_tables, dim]; sorted values index its rows
    int64_t batch;
    int32_t n_tables;
    int32_t mean;
    int64_t n;                   // lookups (sorted pairs)
    uint32_t invalid;            // key of lookups without a row (sorted last)
    int32_t n_seg_blocks;        // grid of the segmented-update kernel
    Ctr* ctr;
    double* carry;               // [n_pieces][2][dim]
    uint32_t* owners;            // head positions of long segments
    uint32_t* blk_unique;        // rows finished per segmented-update block
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
    static constexpr int WIN = GPB * P + 2 * HALO;
};

// ------------------------------------------------------------- pairs -----
__global__ void k_bwd_reset(Ctr* ctr, SortPrep sp) {
    if (threadIdx.x == 0) {
        ctr->n_owners = 0;
        ctr->bad = 0;
        *sp.error = 0;
    }
    if (threadIdx.x < SORT_MAX_PASSES) sp.tile_ctr[threadIdx.x] = 0;
    for (int k = threadIdx.x; k < SORT_MAX_PASSES * SORT_MAX_BINS; k += blockDim.x) sp.totals[k] = 0;
}

// Counters of one apply (so a prepared sort may be applied more than once).
__global__ void k_apply_reset(Ctr* ctr, int64_t* n_unique) {
    if (threadIdx.x == 0) {
        ctr->n_owners = 0;
        *n_unique = 0;
    }
}

// One thread per bag: key = row (or `invalid`), value = bag.  Malformed bag
// offsets or rows beyond the capacity mark the call bad (nothing is updated).
// The value is the lookup's gradient row b * n_tables + t (the layout of
// grad), so the reduction reads gradients without any division.  The kernel
// also builds the radix sort's digit histograms of every pass (block-local in
// LDS, then added to the totals) and clears the sort's look-back state; on bad
// input it raises the sort's error flag so that no pass runs (unwritten keys
// would not match the totals).
__global__ __launch_bounds__(256) void k_pairs(const int64_t* row_off, const int64_t* bag_off, int64_t n_bags,
                                               int64_t n_ids, int64_t batch, int32_t n_tables, int64_t capacity,
                                               uint32_t invalid, uint32_t* keys, uint32_t* vals, Ctr* ctr,
                                               int32_t* status, SortPrep sp, int passes, int width) {
    __shared__ uint32_t s_hist[SORT_MAX_PASSES * SORT_MAX_BINS];
    for (int q = threadIdx.x; q < SORT_MAX_PASSES * SORT_MAX_BINS; q += blockDim.x) s_hist[q] = 0;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < sp.state_words;
         q += (int64_t)gridDim.x * blockDim.x)
        sp.state[q] = 0;
    __syncthreads();
    bool bad = false;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_bags;
         j += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = bag_off[j], e = bag_off[j + 1];
        if (s < 0 || e < s || e > n_ids || (j == 0 && s != 0) || (j == n_bags - 1 && e != n_ids)) {
            bad = true;
            continue;
        }
        const uint32_t t = (uint32_t)((uint64_t)j / (uint64_t)batch);
        const uint32_t gr = (uint32_t)(j - (int64_t)t * batch) * (uint32_t)n_tables + t;
        for (int64_t i = s; i < e; ++i) {
            const int64_t r = row_off[i];
            uint32_t k = invalid;
            if (r >= 0) {
                if (r >= capacity) bad = true;
                else k = (uint32_t)r;
            }
            keys[i] = k;
            vals[i] = gr;
            sort_hist_add(s_hist, k, passes, width);
        }
    }
    if (bad) {
        ctr->bad = 1;
        atomicExch(sp.error, 2u);
        atomicCAS(status, 0, (int32_t)RSE_ERR_BAD_INPUT);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < passes * SORT_MAX_BINS; q += blockDim.x)
        if (s_hist[q]) atomicAdd(&sp.totals[q], s_hist[q]);
}

// ------------------------------------------------------ grad gather ------
template <int D, bool BF16>
__device__ __forceinline__ const float* grad_row(const BwdArgs& a, uint32_t gr, int li) {
    return a.grad + (int64_t)gr * D + li * Geo<D, BF16>::VEC;
}

// Length of the bag whose gradient row is gr = b * n_tables + t (mean only).
__device__ __forceinline__ double bag_len(const BwdArgs& a, uint32_t gr) {
    const uint32_t b = gr / (uint32_t)a.n_tables;
    const uint32_t t = gr - b * (uint32_t)a.n_tables;
    const int64_t j = (int64_t)t * a.batch + b;
    return (double)(a.bag_off[j + 1] - a.bag_off[j]);
}

template <int VEC>
__device__ __forceinline__ void load_grad(float* out, const float* src) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
        const f32x4 v = gload_f4(src + k);
        out[k] = v.x;
        out[k + 1] = v.y;
        out[k + 2] = v.z;
        out[k + 3] = v.w;
    }
}

template <int VEC>
__device__ __forceinline__ void add_grad(double* acc, const float* gv, bool mean, double len) {
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        double g = (double)gv[k];
        if (mean) g = g / len;
        acc[k] += g;
    }
}

// acc += sum over window positions [x, y) of the LDS-staged bag ids, in
// order.  U gradient rows are loaded together (all loads issued before any
// is used); a tail shorter than U is loaded one row at a time.
template <int D, bool BF16>
__device__ __forceinline__ void sum_range(const BwdArgs& a, const uint32_t* s_vals, int x, int y, int li,
                                          double* acc) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int U = 8;
    int q = x;
    for (; q + U <= y; q += U) {
        float gv[U][VEC];
        uint32_t j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = s_vals[q + u];
#pragma unroll
        for (int u = 0; u < U; ++u) load_grad<VEC>(gv[u], grad_row<D, BF16>(a, j[u], li));
        double len[U];
#pragma unroll
        for (int u = 0; u < U; ++u) len[u] = a.mean ? bag_len(a, j[u]) : 1.0;
#pragma unroll
        for (int u = 0; u < U; ++u) add_grad<VEC>(acc, gv[u], a.mean, len[u]);
    }
    for (; q < y; ++q) {
        float gv[VEC];
        const uint32_t j = s_vals[q];
        load_grad<VEC>(gv, grad_row<D, BF16>(a, j, li));
        const double len = a.mean ? bag_len(a, j) : 1.0;
        add_grad<VEC>(acc, gv, a.mean, len);
    }
}

// ---------------------------------------------------------- epilogue -----
// Row update in fp64, rounded once to the storage types.  Lane li owns
// elements [li*VEC, li*VEC + VEC).  The row and its state are loaded before
// the gradient gather so both are in flight together.
template <int D, bool BF16>
struct RowRegs {
    static constexpr int VEC = Geo<D, BF16>::VEC;
    u32x4 w;
    float st0[VEC];
    float st1[VEC];
};

template <int D, bool BF16, int OPT>
__device__ __forceinline__ void load_row(const char* row, int li, RowRegs<D, BF16>& r) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int64_t W_BYTES = (int64_t)D * (BF16 ? 2 : 4);
    r.w = gload_u4(row + li * 16);
    const float* st0 = reinterpret_cast<const float*>(row + W_BYTES) + li * VEC;
    if (OPT != RSE_SGD) load_grad<VEC>(r.st0, st0);
    if (OPT == RSE_ADAM) load_grad<VEC>(r.st1, st0 + D);
}

template <int D, bool BF16, int OPT>
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
            wn[k] = w[k] - a.op.lr * (g[k] / (sqrt((double)an) + a.op.eps));
        }
#pragma unroll
        for (int k = 0; k < VEC; k += 4)
            gstore_f4(st0 + k, f32x4{acc[k], acc[k + 1], acc[k + 2], acc[k + 3]});
    } else {
        float m[VEC], v[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float mn = (float)(a.op.b1 * (double)r.st0[k] + a.op.omb1 * g[k]);
            const float vn = (float)(a.op.b2 * (double)r.st1[k] + a.op.omb2 * g[k] * g[k]);
            m[k] = mn;
            v[k] = vn;
            const double mh = (double)mn / a.op.bc1;
            const double vh = (double)vn / a.op.bc2;
            wn[k] = w[k] - a.op.lr * (mh / (sqrt(vh) + a.op.eps));
        }
#pragma unroll
        for (int k = 0; k < VEC; k += 4) {
            gstore_f4(st0 + k, f32x4{m[k], m[k + 1], m[k + 2], m[k + 3]});
            gstore_f4(st1 + k, f32x4{v[k], v[k + 1], v[k + 2], v[k + 3]});
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
    gstore_u4(row + li * 16, out);
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

// One piece's lookups.  A long segment's part in the piece (at the start,
// continuing an earlier piece, or at the end, continuing past it) is summed
// as a plain run, 8 gradient rows in flight, into a carry slot.  The short
// segments in between are walked CH lookups at a time: the CH gradient rows
// and the rows (weights + state) of every segment starting among them are
// loaded together, then consumed in order, and a segment is finished
// (optimizer applied) at its last lookup, which may lie past the piece end.
template <int D, bool BF16, int OPT, int NMASK>
__device__ __forceinline__ void walk_piece(const BwdArgs& a, const uint32_t* s_keys, const uint32_t* s_vals,
                                           const unsigned long long* s_head, const uint64_t* s_chunks, int wn,
                                           int64_t w0, int64_t k, int x0, int xb, int li, uint32_t& finished) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int CH = 4;
    auto is_head = [&](int q) -> bool { return (s_head[q >> 6] >> (q & 63)) & 1ull; };
    auto carry = [&](int slot, const double* acc) {
        double* dst = a.carry + ((int64_t)k * 2 + slot) * D + li * VEC;
#pragma unroll
        for (int c = 0; c < VEC; ++c) dst[c] = acc[c];
    };
    // lookups without a row sort last: stop at the head of that run
    int lim = xb;
    if (s_keys[xb - 1] == a.invalid) lim = prev_head(s_head, xb - 1);
    if (lim <= x0) return;
    int p = x0;
    if (!is_head(p)) {
        const int h = prev_head(s_head, p);
        const int e = next_head<NMASK>(s_head, p, wn);
        if (e - h > LONG_T) {
            const int e2 = e < lim ? e : lim;
            double acc[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
            sum_range<D, BF16>(a, s_vals, p, e2, li, acc);
            carry(0, acc);
            p = e2;
        } else {
            p = e;                   // short: finished by the piece holding its head
        }
    }
    if (p >= lim) return;
    // the last segment starting in the piece: long (summed into slot 1) or
    // short (the walk runs to its end)
    const int hl = prev_head(s_head, lim - 1);
    const int el = next_head<NMASK>(s_head, hl, wn);
    const bool tail_long = el - hl > LONG_T;
    const int qend = tail_long ? hl : el;
    double acc[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
    RowRegs<D, BF16> cur;
    char* cur_row = nullptr;
    int cur_end = p;
    for (int q = p; q < qend; q += CH) {
        float gv[CH][VEC];
        uint32_t j[CH];
        bool hd[CH];
        RowRegs<D, BF16> rr[CH];
        char* rp[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int qq = q + u < qend ? q + u : qend - 1;
            j[u] = s_vals[qq];
            hd[u] = q + u < qend && is_head(q + u);
        }
#pragma unroll
        for (int u = 0; u < CH; ++u) load_grad<VEC>(gv[u], grad_row<D, BF16>(a, j[u], li));
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            rp[u] = nullptr;
            if (hd[u]) {
                rp[u] = a.rv.row(s_chunks, s_keys[q + u]);
                load_row<D, BF16, OPT>(rp[u], li, rr[u]);
            }
        }
        double len[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) len[u] = a.mean ? bag_len(a, j[u]) : 1.0;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int x = q + u;
            if (x < qend) {
                if (hd[u]) {
                    cur_end = next_head<NMASK>(s_head, x, wn);
                    cur = rr[u];
                    cur_row = rp[u];
#pragma unroll
                    for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
                }
                add_grad<VEC>(acc, gv[u], a.mean, len[u]);
                if (x + 1 == cur_end) {
                    finish_row<D, BF16, OPT>(a, cur_row, li, cur, acc);
                    ++finished;
                }
            }
        }
    }
    if (tail_long) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
        sum_range<D, BF16>(a, s_vals, hl, xb, li, acc);
        carry(1, acc);
        if (li == 0) {
            const unsigned long long pos = atomicAdd(&a.ctr->n_owners, 1ull);
            a.owners[pos] = (uint32_t)(w0 + hl);
        }
    }
}

template <int D, bool BF16, int OPT>
__global__ __launch_bounds__((Geo<D, BF16>::BLOCK)) void k_seg_update(BwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int LPR = G::LPR, GPB = G::GPB, WIN = G::WIN;
    constexpr int NMASK = (WIN + 63) / 64;
    __shared__ uint32_t s_keys[WIN];
    __shared__ uint32_t s_vals[WIN];
    __shared__ unsigned long long s_head[NMASK];
    __shared__ uint64_t s_chunks[LDS_CHUNKS];
    __shared__ uint32_t s_done;
    stage_chunks(s_chunks, a.rv);
    if (threadIdx.x == 0) s_done = 0;
    if (a.ctr->bad) return;
    if (*a.sort_err) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicCAS(a.status, 0, (int32_t)RSE_ERR_HIP);
        return;
    }
    const int64_t n = a.n;
    const int64_t n_pieces = (n + P - 1) / P;
    const int g = threadIdx.x / LPR;
    const int li = threadIdx.x % LPR;
    const int lane = lane_id();
    const int wave = threadIdx.x / WAVE;
    uint32_t finished = 0;

    for (int64_t pb = (int64_t)blockIdx.x * GPB; pb < n_pieces; pb += (int64_t)gridDim.x * GPB) {
        const int64_t blk_a = pb * P;
        const int64_t blk_b = (pb + GPB) * P < n ? (pb + GPB) * P : n;
        const int64_t w0 = blk_a - HALO > 0 ? blk_a - HALO : 0;
        const int64_t w1 = blk_b + HALO < n ? blk_b + HALO : n;
        const int wn = (int)(w1 - w0);
        __syncthreads();
        for (int q = threadIdx.x; q < wn; q += G::BLOCK) {
            s_keys[q] = a.keys[w0 + q];
            s_vals[q] = a.vals[w0 + q];
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
        if (k >= n_pieces) continue;
        const int x0 = (int)(k * P - w0);
        const int xb = (int)((k * P + P < n ? k * P + P : n) - w0);
        walk_piece<D, BF16, OPT, NMASK>(a, s_keys, s_vals, s_head, s_chunks, wn, w0, k, x0, xb, li, finished);
    }
    // rows finished by this block (one LDS add per group), no global atomics
    if (li == 0 && finished) atomicAdd(&s_done, finished);
    __syncthreads();
    if (threadIdx.x == 0) a.blk_unique[blockIdx.x] = s_done;
}

// ------------------------------------------------- long segment combine --
// One block per owner (grid-stride).  The pieces a long segment covers are
// its head's piece k0 (partial in carry slot 1) and the following pieces
// whose first key is still the segment's (slot 0); they form a prefix, so
// one block-wide count per 2^8 pieces finds the last one.  Partials are added
// round-robin per group (U loads in flight, added in piece order) then in
// group order, so the sum is the same on every run.  Block 0 also totals the
// distinct rows.  512 threads: the longest segment's partials are read in a
// few rounds.
constexpr int COMBINE_BLOCK = 512;

template <int D, bool BF16, int OPT>
__global__ __launch_bounds__(COMBINE_BLOCK) void k_combine(BwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int VEC = G::VEC, LPR = G::LPR, BLOCK = COMBINE_BLOCK, GPB = BLOCK / LPR;
    constexpr int U = 4;
    __shared__ double s_part[GPB][D];
    __shared__ uint64_t s_chunks[LDS_CHUNKS];
    __shared__ unsigned long long s_sum[BLOCK / WAVE];
    stage_chunks(s_chunks, a.rv);
    if (a.ctr->bad || *a.sort_err) return;
    const int64_t n_owners = (int64_t)a.ctr->n_owners;
    const int64_t n_pieces = (a.n + P - 1) / P;
    const int g = threadIdx.x / LPR;
    const int li = threadIdx.x % LPR;
    if (blockIdx.x == 0) {
        unsigned long long c = 0;
        const int nb = a.n_seg_blocks;
        for (int b0 = 0; b0 < nb; b0 += 8 * BLOCK) {
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int b = b0 + u * BLOCK + (int)threadIdx.x;
                v[u] = a.blk_unique[b < nb ? b : nb - 1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (b0 + u * BLOCK + (int)threadIdx.x < nb) c += v[u];
        }
        for (int o = WAVE / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, WAVE);
        if (lane_id() == 0) s_sum[threadIdx.x / WAVE] = c;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long t = (unsigned long long)n_owners;
            for (int w = 0; w < BLOCK / WAVE; ++w) t += s_sum[w];
            *a.n_unique = (int64_t)t;
        }
    }
    for (int64_t o = blockIdx.x; o < n_owners; o += gridDim.x) {
        const int64_t h = a.owners[o];
        const uint32_t key = a.keys[h];
        const int64_t k0 = h / P;
        int64_t k1 = k0;
        for (int64_t kb = k0 + 1;; kb += BLOCK) {
            const int64_t k = kb + threadIdx.x;
            const bool in = k < n_pieces && a.keys[k * P] == key;
            const int cnt = __syncthreads_count(in);
            k1 += cnt;
            if (cnt < BLOCK) break;
        }
        double acc[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
        for (int64_t kq = k0 + g; kq <= k1; kq += U * GPB) {
            double src[U][VEC];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t k = kq + u * GPB <= k1 ? kq + u * GPB : k1;
                const double* p = a.carry + (k * 2 + (k == k0 ? 1 : 0)) * D + li * VEC;
#pragma unroll
                for (int c = 0; c < VEC; ++c) src[u][c] = p[c];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (kq + u * GPB <= k1)
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
            for (int q = 1; q < GPB; ++q)
#pragma unroll
                for (int c = 0; c < VEC; ++c) tot[c] += s_part[q][li * VEC + c];
            char* row = a.rv.row(s_chunks, key);
            RowRegs<D, BF16> rr;
            load_row<D, BF16, OPT>(row, li, rr);
            finish_row<D, BF16, OPT>(a, row, li, rr, tot);
        }
        __syncthreads();       // s_part is reused by the next owner
    }
}

// Workspace of one call.
struct BwdWs {
    Ctr* ctr;
    uint32_t* k0;
    uint32_t* v0;
    uint32_t* k1;
    uint32_t* v1;
    double* carry;
    uint32_t* owners;
    uint32_t* blk_unique;
    void* sort_ws;
};

BwdWs carve(void* base, int64_t n_ids, int32_t dim, size_t* total) {
    Carver c(base);
    BwdWs w;
    const size_t n = (size_t)(n_ids > 0 ? n_ids : 1);
    const size_t n_pieces = (n + P - 1) / P;
    w.ctr = c.take<Ctr>(1);
    w.k0 = c.take<uint32_t>(n);
    w.v0 = c.take<uint32_t>(n);
    w.k1 = c.take<uint32_t>(n);
    w.v1 = c.take<uint32_t>(n);
    w.carry = c.take<double>(n_pieces * 2 * (size_t)dim);
    w.owners = c.take<uint32_t>(n_pieces);
    w.blk_unique = c.take<uint32_t>(MAX_SEG_BLOCKS);
    w.sort_ws = c.take<char>(sort_workspace((int64_t)n, nullptr));
    if (total) *total = c.size();
    return w;
}

template <int D, bool BF16, int OPT>
int launch_update(BwdArgs a, int64_t n_ids, hipStream_t s) {
    using G = Geo<D, BF16>;
    const int64_t n_pieces = (n_ids + P - 1) / P;
    const int blocks = fill_blocks(n_pieces, G::GPB, MAX_SEG_BLOCKS);
    a.n_seg_blocks = blocks;
    {
        TraceScope ts(RSE_K_SEG_UPDATE, s);
        hipLaunchKernelGGL((k_seg_update<D, BF16, OPT>), dim3(blocks), dim3(G::BLOCK), 0, s, a);
    }
    const int cblocks = fill_blocks(n_pieces, 1, 2048);
    {
        TraceScope ts(RSE_K_COMBINE, s);
        hipLaunchKernelGGL((k_combine<D, BF16, OPT>), dim3(cblocks), dim3(COMBINE_BLOCK), 0, s, a);
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
    carve(nullptr, n_ids, dim, bytes_out);
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
    BwdWs w = carve(d_ws, n_ids, blocks->dim, &need);
    if (ws_bytes < need) return RSE_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    SortPrep sp = sort_prep(w.sort_ws, n_ids);
    const int64_t capacity = blocks->capacity();
    int bits = bit_length((uint64_t)capacity);
    if (bits < 1) bits = 1;
    const uint32_t invalid = bits >= 32 ? 0xFFFFFFFFu : ((1u << bits) - 1u);
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
        // grid bounded so the per-block histogram flush stays a few hundred atomics per bin
        hipLaunchKernelGGL(k_pairs, dim3(fill_blocks(n_bags, 256, 512)), dim3(256), 0, s, d_row_off,
                           d_bag_offsets, n_bags, n_ids, batch, n_tables, capacity, invalid, w.k0, w.v0, w.ctr,
                           &blocks->header()->status, sp, sp_plan.passes, sp_plan.width);
        bool alt = false;
        const int rc = radix_sort_pairs(w.k0, w.v0, w.k1, w.v1, n_ids, bits, w.sort_ws, &alt, s);
        if (rc) return rc;
        plan.sorted_in_alt = alt ? 1 : 0;
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
    BwdWs w = carve(d_ws, n_ids, blocks->dim, &need);
    if (ws_bytes < need) return RSE_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    SortPrep sp = sort_prep(w.sort_ws, n_ids);
    hipLaunchKernelGGL(k_apply_reset, dim3(1), dim3(64), 0, s, w.ctr, d_n_unique_out);
    if (n_ids == 0 || n_bags == 0) return launch_status();

    BwdArgs a;
    a.rv = blocks->view();
    a.keys = plan->sorted_in_alt ? w.k1 : w.k0;
    a.vals = plan->sorted_in_alt ? w.v1 : w.v0;
    a.bag_off = d_bag_offsets;
    a.grad = d_grad;
    a.batch = batch;
    a.n_tables = n_tables;
    a.mean = pooling == RSE_MEAN;
    a.n = n_ids;
    a.invalid = plan->invalid;
    a.n_seg_blocks = 0;
    a.ctr = w.ctr;
    a.carry = w.carry;
    a.owners = w.owners;
    a.blk_unique = w.blk_unique;
    a.n_unique = d_n_unique_out;
    a.sort_err = sp.error;
    a.status = &blocks->header()->status;
    a.op.lr = opt->lr;
    a.op.eps = opt->eps;
    a.op.b1 = opt->beta1;
    a.op.b2 = opt->beta2;
    a.op.omb1 = 1.0 - opt->beta1;
    a.op.omb2 = 1.0 - opt->beta2;
    a.op.bc1 = opt->kind == RSE_ADAM ? 1.0 - std::pow(opt->beta1, (double)opt->step) : 1.0;
    a.op.bc2 = opt->kind == RSE_ADAM ? 1.0 - std::pow(opt->beta2, (double)opt->step) : 1.0;
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
