// rse_bwd.hip -- sparse backward and fused row-wise optimizer update.
//
// Semantics: "阿里 RecIS：搜广推训练的背景与难点" (backward touches only the
// looked-up rows); "DLRM — Meta 把工业推荐模型拆成 4 个标准积木", "踩过的坑" 4
// (sparse optimizer: only rows seen in the batch are updated);
// "RecIS：阿里开源推荐系统统一训练框架", "代码架构" (fused sparse-gradient
// update with fewer atomics).
//
// Pipeline (one stream):
//   reset -> pairs: (row, bag) per lookup, row as a 32-bit key (-1 -> a key
//   above every row, sorted last) -> stable radix sort by row -> segmented
//   reduction with the optimizer fused in -> combine of long segments.
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

struct OptParams {
    double lr, eps, b1, b2, omb1, omb2, bc1, bc2;
};

struct Ctr {                     // device counters of one call
    unsigned long long n_valid;
    unsigned long long n_owners;
    unsigned long long bad;
    unsigned long long pad[5];
};

struct BwdArgs {
    RowsView rv;
    const uint32_t* keys;        // sorted rows
    const uint32_t* vals;        // bag of each sorted lookup
    const int64_t* bag_off;
    const float* grad;           // [batch, n_tables, dim]
    int64_t batch;
    int32_t n_tables;
    int32_t mean;
    Ctr* ctr;
    double* carry;               // [n_pieces][2][dim]
    uint32_t* owners;            // head positions of long segments
    unsigned long long* n_unique;
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
__global__ void k_bwd_reset(Ctr* ctr, uint32_t* totals, int n_totals, unsigned long long* n_unique) {
    if (threadIdx.x == 0) {
        ctr->n_valid = 0;
        ctr->n_owners = 0;
        ctr->bad = 0;
        *n_unique = 0;
    }
    for (int k = threadIdx.x; k < n_totals; k += blockDim.x) totals[k] = 0;
}

// One thread per bag: key = row (or `invalid`), value = bag.  Malformed bag
// offsets or rows beyond the capacity mark the call bad (nothing is updated).
__global__ void k_pairs(const int64_t* row_off, const int64_t* bag_off, int64_t n_bags, int64_t n_ids,
                        int64_t capacity, uint32_t invalid, uint32_t* keys, uint32_t* vals, Ctr* ctr,
                        int32_t* status) {
    unsigned long long valid = 0;
    bool bad = false;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_bags;
         j += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = bag_off[j], e = bag_off[j + 1];
        if (s < 0 || e < s || e > n_ids || (j == 0 && s != 0) || (j == n_bags - 1 && e != n_ids)) {
            bad = true;
            continue;
        }
        for (int64_t i = s; i < e; ++i) {
            const int64_t r = row_off[i];
            uint32_t k = invalid;
            if (r >= 0) {
                if (r >= capacity) bad = true;
                else {
                    k = (uint32_t)r;
                    ++valid;
                }
            }
            keys[i] = k;
            vals[i] = (uint32_t)j;
        }
    }
    // wave-aggregated counter update
    const unsigned long long any = __ballot(valid != 0);
    if (any) {
        unsigned long long v = valid;
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
        if (lane_id() == 0) atomicAdd(&ctr->n_valid, v);
    }
    if (bad) {
        ctr->bad = 1;
        atomicCAS(status, 0, (int32_t)RSE_ERR_BAD_INPUT);
    }
}

// ------------------------------------------------------ grad gather ------
template <int D, bool BF16>
__device__ __forceinline__ const float* grad_row(const BwdArgs& a, uint32_t j, int li) {
    using G = Geo<D, BF16>;
    const int64_t t = (int64_t)j / a.batch;
    const int64_t b = (int64_t)j - t * a.batch;
    return a.grad + (b * a.n_tables + t) * D + li * G::VEC;
}

template <int VEC>
__device__ __forceinline__ void load_grad(float* out, const float* src) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + k);
        out[k] = v.x;
        out[k + 1] = v.y;
        out[k + 2] = v.z;
        out[k + 3] = v.w;
    }
}

// acc += sum over sorted positions [x, y) (LDS window based at w0) in order.
template <int D, bool BF16>
__device__ __forceinline__ void sum_range(const BwdArgs& a, const uint32_t* s_vals, int64_t w0, int64_t x,
                                          int64_t y, int li, double* acc) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int U = 4;
    for (int64_t q = x; q < y; q += U) {
        float gv[U][VEC];
        double sc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (q + u < y) {
                const uint32_t j = s_vals[q + u - w0];
                load_grad<VEC>(gv[u], grad_row<D, BF16>(a, j, li));
                sc[u] = a.mean ? (double)(a.bag_off[j + 1] - a.bag_off[j]) : 1.0;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (q + u < y) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    double g = (double)gv[u][k];
                    if (a.mean) g = g / sc[u];
                    acc[k] += g;
                }
            }
        }
    }
}

// ---------------------------------------------------------- epilogue -----
// Row update in fp64, rounded once to the storage types.  Lane li owns
// elements [li*VEC, li*VEC + VEC).
template <int D, bool BF16, int OPT>
__device__ __forceinline__ void update_row(const BwdArgs& a, uint32_t row_idx, int li, const double* g) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    constexpr int64_t W_BYTES = (int64_t)D * (BF16 ? 2 : 4);
    char* row = a.rv.row(row_idx);
    uint4 wq = *reinterpret_cast<const uint4*>(row + li * 16);
    double w[VEC];
    if (!BF16) {
        w[0] = __uint_as_float(wq.x);
        w[1] = __uint_as_float(wq.y);
        w[2] = __uint_as_float(wq.z);
        w[3] = __uint_as_float(wq.w);
    } else {
        const uint32_t q4[4] = {wq.x, wq.y, wq.z, wq.w};
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
        load_grad<VEC>(acc, st0);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float an = (float)((double)acc[k] + g[k] * g[k]);
            acc[k] = an;
            wn[k] = w[k] - a.op.lr * (g[k] / (sqrt((double)an) + a.op.eps));
        }
#pragma unroll
        for (int k = 0; k < VEC; k += 4)
            *reinterpret_cast<float4*>(st0 + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
    } else {
        float m[VEC], v[VEC];
        load_grad<VEC>(m, st0);
        load_grad<VEC>(v, st1);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float mn = (float)(a.op.b1 * (double)m[k] + a.op.omb1 * g[k]);
            const float vn = (float)(a.op.b2 * (double)v[k] + a.op.omb2 * g[k] * g[k]);
            m[k] = mn;
            v[k] = vn;
            const double mh = (double)mn / a.op.bc1;
            const double vh = (double)vn / a.op.bc2;
            wn[k] = w[k] - a.op.lr * (mh / (sqrt(vh) + a.op.eps));
        }
#pragma unroll
        for (int k = 0; k < VEC; k += 4) {
            *reinterpret_cast<float4*>(st0 + k) = make_float4(m[k], m[k + 1], m[k + 2], m[k + 3]);
            *reinterpret_cast<float4*>(st1 + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
        }
    }
    uint4 out;
    if (!BF16) {
        out = make_uint4(__float_as_uint((float)wn[0]), __float_as_uint((float)wn[1]),
                         __float_as_uint((float)wn[2]), __float_as_uint((float)wn[3]));
    } else {
        uint32_t q4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            q4[k] = (uint32_t)f64_to_bf16_rne(wn[2 * k]) | ((uint32_t)f64_to_bf16_rne(wn[2 * k + 1]) << 16);
        out = make_uint4(q4[0], q4[1], q4[2], q4[3]);
    }
    reinterpret_cast<uint4*>(row)[li] = out;
}

// ------------------------------------------------- segmented update ------
template <int D, bool BF16, int OPT>
__global__ __launch_bounds__((Geo<D, BF16>::BLOCK)) void k_seg_update(BwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int VEC = G::VEC, LPR = G::LPR, GPB = G::GPB, WIN = G::WIN;
    __shared__ uint32_t s_keys[WIN];
    __shared__ uint32_t s_vals[WIN];
    if (a.ctr->bad) return;
    const int64_t n_valid = (int64_t)a.ctr->n_valid;
    const int64_t n_pieces = (n_valid + P - 1) / P;
    const int g = threadIdx.x / LPR;
    const int li = threadIdx.x % LPR;
    unsigned long long finished = 0;

    for (int64_t pb = (int64_t)blockIdx.x * GPB; pb < n_pieces; pb += (int64_t)gridDim.x * GPB) {
        const int64_t blk_a = pb * P;
        const int64_t blk_b = (pb + GPB) * P < n_valid ? (pb + GPB) * P : n_valid;
        const int64_t w0 = blk_a - HALO > 0 ? blk_a - HALO : 0;
        const int64_t w1 = blk_b + HALO < n_valid ? blk_b + HALO : n_valid;
        __syncthreads();
        for (int64_t q = w0 + threadIdx.x; q < w1; q += G::BLOCK) {
            s_keys[q - w0] = a.keys[q];
            s_vals[q - w0] = a.vals[q];
        }
        __syncthreads();
        const int64_t k = pb + g;
        if (k >= n_pieces) continue;
        const int64_t a0 = k * P;
        const int64_t b0 = a0 + P < n_valid ? a0 + P : n_valid;
        auto K = [&](int64_t q) -> uint32_t { return s_keys[q - w0]; };
        // same-key run around q, counted up to HALO each way (within the window)
        auto fwd_run = [&](int64_t q, uint32_t key) -> int64_t {
            int64_t e = q;
            const int64_t lim = (q + HALO < w1) ? q + HALO : w1;
            while (e < lim && K(e) == key) ++e;
            return e - q;              // >= HALO means "long" (or window end)
        };
        auto bwd_run = [&](int64_t q, uint32_t key) -> int64_t {
            int64_t h = q;
            const int64_t lim = (q - HALO > w0) ? q - HALO : w0;
            while (h > lim && K(h - 1) == key) --h;
            return q - h;
        };
        int64_t p = a0;
        if (p > 0 && K(p) == K(p - 1)) {
            // segment started in an earlier piece
            const uint32_t key = K(p);
            const int64_t nb = bwd_run(p, key);
            const int64_t nf = fwd_run(p, key);
            const bool at_end = p + nf == n_valid;   // window end is the data end
            const bool is_long = nb + nf > LONG_T || (!at_end && p + nf == w1);
            if (is_long) {
                int64_t e = p;
                while (e < b0 && K(e) == key) ++e;
                double acc[VEC];
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
                sum_range<D, BF16>(a, s_vals, w0, p, e, li, acc);
                double* dst = a.carry + ((int64_t)k * 2 + 0) * D + li * VEC;
#pragma unroll
                for (int c = 0; c < VEC; ++c) dst[c] = acc[c];
                p = e;
            } else {
                p += nf;
            }
        }
        while (p < b0) {
            const uint32_t key = K(p);
            const int64_t nf = fwd_run(p, key);
            const bool at_end = p + nf == n_valid;
            const bool is_long = nf > LONG_T || (!at_end && p + nf == w1);
            double acc[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
            if (!is_long) {
                sum_range<D, BF16>(a, s_vals, w0, p, p + nf, li, acc);
                update_row<D, BF16, OPT>(a, key, li, acc);
                ++finished;
                p += nf;
            } else {
                sum_range<D, BF16>(a, s_vals, w0, p, b0, li, acc);
                double* dst = a.carry + ((int64_t)k * 2 + 1) * D + li * VEC;
#pragma unroll
                for (int c = 0; c < VEC; ++c) dst[c] = acc[c];
                if (li == 0) {
                    const unsigned long long pos = atomicAdd(&a.ctr->n_owners, 1ull);
                    a.owners[pos] = (uint32_t)p;
                }
                p = b0;
            }
        }
    }
    if (li == 0 && finished) atomicAdd(a.n_unique, finished);
}

// ------------------------------------------------- long segment combine --
// One block per owner (grid-stride): partials of the pieces the segment
// covers, added round-robin per group then in group order.
template <int D, bool BF16, int OPT>
__global__ __launch_bounds__((Geo<D, BF16>::BLOCK)) void k_combine(BwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int VEC = G::VEC, LPR = G::LPR, GPB = G::GPB;
    __shared__ double s_part[GPB][D];
    __shared__ int64_t s_end;
    if (a.ctr->bad) return;
    const int64_t n_valid = (int64_t)a.ctr->n_valid;
    const int64_t n_owners = (int64_t)a.ctr->n_owners;
    const int g = threadIdx.x / LPR;
    const int li = threadIdx.x % LPR;
    for (int64_t o = blockIdx.x; o < n_owners; o += gridDim.x) {
        const int64_t h = a.owners[o];
        const uint32_t key = a.keys[h];
        __syncthreads();
        if (threadIdx.x == 0) {
            // end of the run: first position after h with a different key
            int64_t lo = h, hi = n_valid;   // keys[lo] == key; keys[hi] != key (or end)
            while (hi - lo > 1) {
                const int64_t mid = lo + (hi - lo) / 2;
                if (a.keys[mid] == key) lo = mid;
                else hi = mid;
            }
            s_end = hi;
        }
        __syncthreads();
        const int64_t e = s_end;
        const int64_t k0 = h / P;
        const int64_t k1 = (e - 1) / P;
        double acc[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
        for (int64_t k = k0 + g; k <= k1; k += GPB) {
            const double* src = a.carry + (k * 2 + (k == k0 ? 1 : 0)) * D + li * VEC;
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] += src[c];
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) s_part[g][li * VEC + c] = acc[c];
        __syncthreads();
        if (g == 0) {
            double tot[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) tot[c] = s_part[0][li * VEC + c];
            for (int q = 1; q < GPB; ++q)
#pragma unroll
                for (int c = 0; c < VEC; ++c) tot[c] += s_part[q][li * VEC + c];
            update_row<D, BF16, OPT>(a, key, li, tot);
            if (li == 0) atomicAdd(a.n_unique, 1ull);
        }
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
    w.sort_ws = c.take<char>(sort_workspace((int64_t)n, nullptr));
    if (total) *total = c.size();
    return w;
}

template <int D, bool BF16, int OPT>
int launch_update(const BwdArgs& a, int64_t n_ids, hipStream_t s) {
    using G = Geo<D, BF16>;
    const int64_t n_pieces = (n_ids + P - 1) / P;
    const int blocks = fill_blocks(n_pieces, G::GPB, 65535);
    hipLaunchKernelGGL((k_seg_update<D, BF16, OPT>), dim3(blocks), dim3(G::BLOCK), 0, s, a);
    const int cblocks = fill_blocks(n_pieces, 1, 2048);
    hipLaunchKernelGGL((k_combine<D, BF16, OPT>), dim3(cblocks), dim3(G::BLOCK), 0, s, a);
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

int embedding_bag_bwd_update(rse_blocks* blocks, const int64_t* d_row_off, int64_t n_ids,
                             const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch,
                             int32_t pooling, const float* d_grad, const rse_optim* opt,
                             int64_t* d_n_unique_out, void* d_ws, size_t ws_bytes, void* stream) {
    if (!blocks || !d_bag_offsets || !opt || !d_n_unique_out || !d_ws) return RSE_ERR_INVALID_ARG;
    if (n_ids < 0 || n_tables <= 0 || batch < 0) return RSE_ERR_INVALID_ARG;
    if (n_ids > 0 && (!d_row_off || !d_grad)) return RSE_ERR_INVALID_ARG;
    if (pooling != RSE_SUM && pooling != RSE_MEAN) return RSE_ERR_INVALID_ARG;
    if (opt->kind != blocks->optim) return RSE_ERR_INVALID_ARG;
    if (opt->kind == RSE_ADAM && opt->step < 1) return RSE_ERR_INVALID_ARG;
    const int64_t n_bags = (int64_t)n_tables * batch;
    if (n_ids > (int64_t)0xFFFFFFFFll || n_bags > (int64_t)0xFFFFFFFFll) return RSE_ERR_INVALID_ARG;
    size_t need = 0;
    BwdWs w = carve(d_ws, n_ids, blocks->dim, &need);
    if (ws_bytes < need) return RSE_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    unsigned long long* n_unique = reinterpret_cast<unsigned long long*>(d_n_unique_out);
    uint32_t* totals = sort_totals(w.sort_ws, n_ids > 0 ? n_ids : 1);
    hipLaunchKernelGGL(k_bwd_reset, dim3(1), dim3(256), 0, s, w.ctr, totals, SORT_MAX_PASSES * 256, n_unique);
    if (n_ids == 0 || n_bags == 0) return launch_status();

    const int64_t capacity = blocks->capacity();
    int bits = bit_length((uint64_t)capacity);
    if (bits < 1) bits = 1;
    const uint32_t invalid = bits >= 32 ? 0xFFFFFFFFu : ((1u << bits) - 1u);
    hipLaunchKernelGGL(k_pairs, dim3(fill_blocks(n_bags, 256, 8192)), dim3(256), 0, s, d_row_off,
                       d_bag_offsets, n_bags, n_ids, capacity, invalid, w.k0, w.v0, w.ctr,
                       &blocks->header()->status);
    bool alt = false;
    int rc = radix_sort_pairs(w.k0, w.v0, w.k1, w.v1, n_ids, bits, w.sort_ws, &alt, s);
    if (rc) return rc;

    BwdArgs a;
    a.rv = blocks->view();
    a.keys = alt ? w.k1 : w.k0;
    a.vals = alt ? w.v1 : w.v0;
    a.bag_off = d_bag_offsets;
    a.grad = d_grad;
    a.batch = batch;
    a.n_tables = n_tables;
    a.mean = pooling == RSE_MEAN;
    a.ctr = w.ctr;
    a.carry = w.carry;
    a.owners = w.owners;
    a.n_unique = n_unique;
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

}  // extern "C"
