// rse_fwd.hip -- pooled embedding gather (EmbeddingBag forward, "DLRM模型的核心
// 价值与工业落地挑战" section 2.1: sum pooling over variable-length bags;
// "RecIS：阿里开源推荐系统统一训练框架", "代码架构": vectorised lookup loads).
//
// HBM-bound: each lookup reads one row (dim * 4 or dim * 2 bytes) and each
// bag writes one fp32 row.  A row is read by a group of LPR lanes with one
// 16-byte load per lane (dwordx4), so a 64-lane wave reads 64/LPR rows per
// instruction with every byte of each 64-byte segment used.  Rows are
// accumulated in fp64 (cheap: the kernel moves ~4 bytes per flop) in bag
// order, so the pooled value is the exactly rounded fp32 of the sum in all
// but pathological cases.
//
// Three schedules, chosen by the mean bag length:
//  - one-hot (mean <= 1.5): a group takes a chunk of up to 8 bags with no
//    loop, all its rows in flight at once; chunks that are not one-hot fall
//    back to a bag-by-bag walk;
//  - group-per-bags: each group owns 4 consecutive bags and walks their
//    lookups as one flat range, UNROLL rows in flight, closing a bag whenever
//    the range crosses its end offset (short bags);
//  - wave-per-bag: the wave's groups split one bag's lookups round-robin and
//    combine with xor-shuffles in a fixed tree (long bags).
#include "rse_host.h"

using namespace rse;
using namespace rse_host;

namespace {

constexpr int FWD_BLOCK = 256;

template <int D, bool BF16>
struct Geo {
    static constexpr int VEC = BF16 ? 8 : 4;    // elements per lane (16 bytes)
    static constexpr int LPR = D / VEC;         // lanes per row
    static constexpr int GROUPS = WAVE / LPR;   // rows per wave-wide load
    static_assert(LPR >= 1 && LPR <= WAVE && (WAVE % LPR) == 0, "dim");
};

template <bool BF16>
__device__ __forceinline__ void widen_add(double* acc, const u32x4& q) {
    if (!BF16) {
        acc[0] += (double)__uint_as_float(q.x);
        acc[1] += (double)__uint_as_float(q.y);
        acc[2] += (double)__uint_as_float(q.z);
        acc[3] += (double)__uint_as_float(q.w);
    } else {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[2 * k] += (double)__uint_as_float(w[k] << 16);
            acc[2 * k + 1] += (double)__uint_as_float(w[k] & 0xFFFF0000u);
        }
    }
}


// Pooled rows are written once and not read again by this kernel: stream
// them past the caches so hot embedding rows stay resident.  Mean pooling
// multiplies by 1 / len (one division per bag, within one fp64 rounding of
// the quotient); an empty bag (len 0) stores its zero sum.
template <int VEC, bool MEAN>
__device__ __forceinline__ void store_out(float* dst, const double* acc, int64_t len) {
    const double inv = MEAN && len > 0 ? 1.0 / (double)len : 1.0;
    float f[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) f[k] = (float)(MEAN ? acc[k] * inv : acc[k]);
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
        const f32x4 v = {f[k], f[k + 1], f[k + 2], f[k + 3]};
        __builtin_nontemporal_store(v, (RSE_GLOBAL f32x4*)(dst + k));
    }
}

struct FwdArgs {
    RowsView rv;
    const int64_t* row_off;
    const int64_t* bag_off;
    int64_t n_bags;
    int64_t batch;
    int64_t n_ids;
    int64_t capacity;          // rows addressable through the chunk table
    int32_t* status;           // blocks' sticky status
    int32_t n_tables;
    int32_t mean;
    float* out;
};

// Offsets outside [0, n_ids] or decreasing, and rows beyond the capacity, are
// malformed input: the bag is skipped (or the row ignored) and the sticky
// status set, so nothing is read out of bounds.
__device__ __forceinline__ void flag_bad(const FwdArgs& a) {
    atomicCAS(a.status, 0, (int32_t)RSE_ERR_BAD_INPUT);
}

// The bag offsets must start at 0 and end at n_ids; checked once per call
// (block 0).  Offsets that break this are reported, and every bag is still
// bounded by [0, n_ids], so nothing is read out of bounds.
__device__ __forceinline__ void check_endpoints(const FwdArgs& a) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && (a.bag_off[0] != 0 || a.bag_off[a.n_bags] != a.n_ids))
        flag_bad(a);
}

// Row loads are issued unconditionally (a missing or rejected row reads a
// dummy row and is masked out of the sum), so all UNROLL loads of a group
// are in flight together instead of being serialised behind branches.
__device__ __forceinline__ const char* dummy_row(const uint64_t* s_chunks, const RowsView& rv) {
    return reinterpret_cast<const char*>(rv.lds_ok() ? ((const RSE_LDS uint64_t*)s_chunks)[0]
                                                     : ((const RSE_GLOBAL uint64_t*)rv.chunks)[0]);
}

// ---------------------------------------------------- one-hot bags ------
// One chunk of BPG consecutive bags per group of LPR lanes, straight-line
// (no loop: every wait covers exactly the loads it needs, and the stores are
// the group's last instructions).  In the one-hot layout bag j holds exactly
// lookup j.  Lane k < BPG loads bag k's two offsets and its row offset and
// builds its row address (chunk table in LDS, reads clamped so none is
// conditional); a group ballot decides whether the whole chunk is one-hot
// and in range; the addresses are shuffled to all lanes and the BPG rows
// loaded together.  Any other chunk (longer or empty bags, malformed
// offsets, rows past the capacity) is done bag by bag by chunk_general.
template <int D, bool BF16, bool MEAN>
__device__ __forceinline__ void chunk_general(const FwdArgs& a, const uint64_t* s_chunks, int64_t jb,
                                                        int nb, int li) {
    constexpr int VEC = Geo<D, BF16>::VEC;
    for (int k = 0; k < nb; ++k) {
        const int64_t j = jb + k;
        const int64_t s0 = a.bag_off[j], e0 = a.bag_off[j + 1];
        if (s0 < 0 || e0 < s0 || e0 > a.n_ids) {     // malformed: the bag's output is not written
            if (li == 0) flag_bad(a);
            continue;
        }
        double acc[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] = 0.0;
        for (int64_t i = s0; i < e0; ++i) {
            const int64_t r = a.row_off[i];
            if (r >= a.capacity) {
                if (li == 0) flag_bad(a);
            } else if (r >= 0) {
                widen_add<BF16>(acc, gload_u4(a.rv.row(s_chunks, r) + li * 16));
            }
        }
        const int64_t t = (int64_t)((uint64_t)j / (uint64_t)a.batch);
        const int64_t b = j - t * a.batch;
        store_out<VEC, MEAN>(a.out + (b * a.n_tables + t) * D + li * VEC, acc, e0 - s0);
    }
}

template <int D, bool BF16, bool MEAN, int BPG, bool LDS_TAB>
__global__ __launch_bounds__(FWD_BLOCK) void k_fwd_onehot(FwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int VEC = G::VEC, LPR = G::LPR, GROUPS = G::GROUPS;
    static_assert(BPG <= LPR && BPG <= 32, "one lane per bag of a chunk");
    __shared__ uint64_t s_chunks[LDS_CHUNKS];
    check_endpoints(a);
    const int lane = lane_id();
    const int g = lane / LPR;
    const int li = lane % LPR;
    const int gbase = g * LPR;
    const int64_t c = ((int64_t)blockIdx.x * FWD_BLOCK + threadIdx.x) / WAVE * GROUPS + g;
    const int64_t n_chunk = (a.n_bags + BPG - 1) / BPG;
    const bool live = c < n_chunk;
    const int64_t jb = (live ? c : n_chunk - 1) * BPG;
    const int nb = (int)(a.n_bags - jb < BPG ? a.n_bags - jb : BPG);
    // lane k's bag (lanes past the chunk repeat its last bag); the host
    // launches this kernel only with n_ids >= 1 and capacity >= 1
    const int64_t j = jb + (li < nb ? li : nb - 1);
    const int64_t lo = a.bag_off[j];
    const int64_t hi = a.bag_off[j + 1];
    const int64_t r = a.row_off[j < a.n_ids ? j : a.n_ids - 1];
    if (LDS_TAB) stage_chunks(s_chunks, a.rv);
    if (!live) return;

    const bool one = lo == j && hi == j + 1;
    const bool in_range = r < a.capacity;
    const bool valid = one && r >= 0 && in_range;
    const uint64_t ci = valid ? ((uint64_t)r >> a.rv.shift) : 0;
    const uint64_t base = LDS_TAB ? ((const RSE_LDS uint64_t*)s_chunks)[ci]
                                  : ((const RSE_GLOBAL uint64_t*)a.rv.chunks)[ci];
    const uint64_t p = base + (valid ? ((uint64_t)r & a.rv.mask) * (uint64_t)a.rv.row_bytes : 0);
    const uint64_t gmask = LPR == 64 ? ~0ull : ((1ull << LPR) - 1);
    const uint64_t not_simple = (__ballot(li < BPG && !(one && in_range)) >> gbase) & gmask;
    const uint32_t vbits = (uint32_t)((__ballot(li < BPG && valid) >> gbase) & ((1ull << BPG) - 1));
    if (not_simple != 0 || nb != BPG) {
        chunk_general<D, BF16, MEAN>(a, s_chunks, jb, nb, li);
        return;
    }
    u32x4 q[BPG];
#pragma unroll
    for (int k = 0; k < BPG; ++k) {
        const uint64_t pk = __shfl(p, gbase + k, WAVE);
        q[k] = gload_u4(reinterpret_cast<const char*>(pk) + li * 16);
    }
    uint64_t t = (uint64_t)jb / (uint64_t)a.batch;
    uint64_t b = (uint64_t)jb - t * (uint64_t)a.batch;
#pragma unroll
    for (int k = 0; k < BPG; ++k) {
        float* dst = a.out + ((int64_t)b * a.n_tables + (int64_t)t) * D + li * VEC;
        const bool v = (vbits >> k) & 1u;
        if (!BF16) {
            const u32x4 w = v ? q[k] : u32x4{0u, 0u, 0u, 0u};
            __builtin_nontemporal_store(f32x4{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                                              __uint_as_float(w.w)},
                                        (RSE_GLOBAL f32x4*)dst);
        } else {
            const u32x4 w = v ? q[k] : u32x4{0u, 0u, 0u, 0u};
            __builtin_nontemporal_store(f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                                              __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)},
                                        (RSE_GLOBAL f32x4*)dst);
            __builtin_nontemporal_store(f32x4{__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xFFFF0000u),
                                              __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xFFFF0000u)},
                                        (RSE_GLOBAL f32x4*)(dst + 4));
        }
        if (++b == (uint64_t)a.batch) {
            b = 0;
            ++t;
        }
    }
}

// ----------------------------------------------------- group per bags ----
// Each group owns BPG = 4 consecutive bags: their 5 offsets are loaded
// together and kept in registers, and the group walks the bags' lookups as
// one flat range, UNROLL rows in flight, closing a bag (one store, no load)
// whenever the range crosses its end.  The row offsets of the next UNROLL
// lookups are requested while the current rows are in flight, so each step
// waits for one memory round trip instead of two.
// Offsets of a chunk's 4 bags, as five scalars so that they stay in
// registers (an array indexed in a loop would be moved to LDS).
struct BagOffs4 {
    int64_t o0, o1, o2, o3, o4;
    __device__ __forceinline__ int64_t at(int k) const {
        return k <= 0 ? o0 : k == 1 ? o1 : k == 2 ? o2 : k == 3 ? o3 : o4;
    }
};

template <int D, bool BF16, bool MEAN, int BPG, int UNROLL>
__global__ __launch_bounds__(FWD_BLOCK) void k_fwd_groups(FwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int VEC = G::VEC, LPR = G::LPR, GROUPS = G::GROUPS;
    __shared__ uint64_t s_chunks[LDS_CHUNKS];
    stage_chunks(s_chunks, a.rv);
    check_endpoints(a);
    const int lane = lane_id();
    const int g = lane / LPR;
    const int li = lane % LPR;
    const int64_t gid = ((int64_t)blockIdx.x * FWD_BLOCK + threadIdx.x) / WAVE * GROUPS + g;
    const int64_t n_groups = (int64_t)gridDim.x * (FWD_BLOCK / WAVE) * GROUPS;
    const bool can_load = a.capacity > 0;
    const char* dummy = can_load ? dummy_row(s_chunks, a.rv) : nullptr;

    for (int64_t jb = gid * BPG; jb < a.n_bags; jb += n_groups * BPG) {
        const int nb = (int)(a.n_bags - jb < BPG ? a.n_bags - jb : BPG);
        // start of bag jb + k for k < nb; the end of the last bag after that
        static_assert(BPG == 4, "BagOffs4");
        BagOffs4 bo;
        bo.o0 = a.bag_off[jb];
        bo.o1 = a.bag_off[jb + (1 < nb ? 1 : nb)];
        bo.o2 = a.bag_off[jb + (2 < nb ? 2 : nb)];
        bo.o3 = a.bag_off[jb + (3 < nb ? 3 : nb)];
        bo.o4 = a.bag_off[jb + nb];
        const bool ok = bo.o0 >= 0 && bo.o1 >= bo.o0 && bo.o2 >= bo.o1 && bo.o3 >= bo.o2 && bo.o4 >= bo.o3 &&
                        bo.o4 <= a.n_ids;
        if (!ok) {
            if (li == 0) flag_bad(a);
            continue;
        }
        const int64_t first = bo.o0, last = bo.o4;
        uint32_t t = (uint32_t)((uint64_t)jb / (uint64_t)a.batch);
        uint32_t b = (uint32_t)(jb - (int64_t)t * a.batch);
        double acc[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[k] = 0.0;
        int k = 0;                     // open bag of the chunk
        int64_t bag_start = first;
        int64_t bag_end = bo.at(1);
// closes the open bag: one store, then the next bag opens
#define RSE_CLOSE_BAG()                                                              \
    do {                                                                             \
        const int64_t len = bag_end - bag_start;                                     \
        float* dst = a.out + ((int64_t)b * a.n_tables + t) * D + li * VEC;          \
        store_out<VEC, MEAN>(dst, acc, len);                                         \
        for (int c = 0; c < VEC; ++c) acc[c] = 0.0;                                  \
        if (++b == (uint32_t)a.batch) {                                              \
            b = 0;                                                                   \
            ++t;                                                                     \
        }                                                                            \
        ++k;                                                                         \
        bag_start = bag_end;                                                         \
        bag_end = bo.at(k + 1);                                                      \
    } while (0)

        if (last > first) {
            int64_t rn[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) rn[u] = a.row_off[first + u < last ? first + u : last - 1];
            for (int64_t i = first; i < last; i += UNROLL) {
                int64_t r[UNROLL];
                bool v[UNROLL];
                u32x4 q[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    r[u] = rn[u];
                    v[u] = i + u < last && r[u] >= 0 && r[u] < a.capacity;
                    if (i + u < last && r[u] >= a.capacity && li == 0) flag_bad(a);
                }
                if (can_load) {
#pragma unroll
                    for (int u = 0; u < UNROLL; ++u)
                        q[u] = gload_u4((v[u] ? a.rv.row(s_chunks, r[u]) : dummy) + li * 16);
                }
                const int64_t inx = i + UNROLL;
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) rn[u] = a.row_off[inx + u < last ? inx + u : last - 1];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const int64_t ii = i + u;
                    if (ii >= last) break;
                    while (ii >= bag_end) RSE_CLOSE_BAG();   // finished (possibly empty) bags
                    if (v[u]) widen_add<BF16>(acc, q[u]);
                }
            }
        }
        // close the open bag and any trailing empty ones
        while (k < nb) RSE_CLOSE_BAG();
#undef RSE_CLOSE_BAG
    }
}

// ------------------------------------------------------- wave per bag ----
// The wave's groups split one bag's lookups round-robin (the next step's row
// offsets requested while the current rows are in flight) and combine with
// xor-shuffles in a fixed tree.
template <int D, bool BF16, bool MEAN, int UNROLL>
__global__ __launch_bounds__(FWD_BLOCK) void k_fwd_wave(FwdArgs a) {
    using G = Geo<D, BF16>;
    constexpr int VEC = G::VEC, LPR = G::LPR, GROUPS = G::GROUPS;
    constexpr int64_t STEP = (int64_t)GROUPS * UNROLL;
    __shared__ uint64_t s_chunks[LDS_CHUNKS];
    stage_chunks(s_chunks, a.rv);
    check_endpoints(a);
    const int lane = lane_id();
    const int g = lane / LPR;
    const int li = lane % LPR;
    const int64_t wid = ((int64_t)blockIdx.x * FWD_BLOCK + threadIdx.x) / WAVE;
    const int64_t n_waves = (int64_t)gridDim.x * (FWD_BLOCK / WAVE);
    const bool can_load = a.capacity > 0;
    const char* dummy = can_load ? dummy_row(s_chunks, a.rv) : nullptr;
    for (int64_t j = wid; j < a.n_bags; j += n_waves) {
        const int64_t s = a.bag_off[j];
        const int64_t e = a.bag_off[j + 1];
        if (s < 0 || e < s || e > a.n_ids) {
            if (lane == 0) flag_bad(a);
            continue;
        }
        double acc[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[k] = 0.0;
        if (e > s) {
            int64_t rn[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t ii = s + g + (int64_t)u * GROUPS;
                rn[u] = a.row_off[ii < e ? ii : e - 1];
            }
            for (int64_t i = s + g; i < e + g; i += STEP) {
                int64_t r[UNROLL];
                bool v[UNROLL];
                u32x4 q[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const int64_t ii = i + (int64_t)u * GROUPS;
                    r[u] = rn[u];
                    v[u] = ii < e && r[u] >= 0 && r[u] < a.capacity;
                    if (ii < e && r[u] >= a.capacity && li == 0) flag_bad(a);
                }
                if (can_load) {
#pragma unroll
                    for (int u = 0; u < UNROLL; ++u)
                        q[u] = gload_u4((v[u] ? a.rv.row(s_chunks, r[u]) : dummy) + li * 16);
                }
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const int64_t ii = i + STEP + (int64_t)u * GROUPS;
                    rn[u] = a.row_off[ii < e ? ii : e - 1];
                }
                if (can_load) {
#pragma unroll
                    for (int u = 0; u < UNROLL; ++u)
                        if (v[u]) widen_add<BF16>(acc, q[u]);
                }
            }
        }
        // fixed xor tree across the groups
#pragma unroll
        for (int m = LPR; m < WAVE; m <<= 1) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[k] += shfl_xor_f64(acc[k], m);
        }
        if (g == 0) {
            const int64_t t = (int64_t)((uint64_t)j / (uint64_t)a.batch);
            const int64_t b = j - t * a.batch;
            const int64_t len = e - s;
            store_out<VEC, MEAN>(a.out + (b * a.n_tables + t) * D + li * VEC, acc, len);
        }
    }
}

#ifndef RSE_FWD_ONEHOT_BPG
#define RSE_FWD_ONEHOT_BPG 8
#endif

template <int D, bool BF16, bool MEAN>
int launch_fwd_p(const FwdArgs& a, int64_t n_ids, hipStream_t s) {
    using G = Geo<D, BF16>;
    TraceScope ts(RSE_K_FWD, s);
    const double avg = a.n_bags > 0 ? (double)n_ids / (double)a.n_bags : 0.0;
    constexpr int WAVES = FWD_BLOCK / WAVE;
    if (avg >= 2.0 * G::GROUPS && G::GROUPS > 1) {
        const int blocks = fill_blocks(a.n_bags, WAVES, 256 * 32);
        hipLaunchKernelGGL((k_fwd_wave<D, BF16, MEAN, 4>), dim3(blocks), dim3(FWD_BLOCK), 0, s, a);
    } else if (avg <= 1.5 && n_ids > 0 && a.capacity > 0) {
        // one-hot: one chunk of BPG bags per group, all its rows in flight
        constexpr int BPG = G::LPR < RSE_FWD_ONEHOT_BPG ? G::LPR : RSE_FWD_ONEHOT_BPG;
        const int64_t chunks = (a.n_bags + BPG - 1) / BPG;
        const int64_t per_block = WAVES * G::GROUPS;
        const int64_t blocks = (chunks + per_block - 1) / per_block;
        if (blocks > 0x7FFFFFFFll) return RSE_ERR_INVALID_ARG;
        if (a.rv.n_chunks <= LDS_CHUNKS)
            hipLaunchKernelGGL((k_fwd_onehot<D, BF16, MEAN, BPG, true>), dim3((unsigned)blocks), dim3(FWD_BLOCK), 0, s, a);
        else
            hipLaunchKernelGGL((k_fwd_onehot<D, BF16, MEAN, BPG, false>), dim3((unsigned)blocks), dim3(FWD_BLOCK), 0, s,
                               a);
    } else {
        constexpr int BPG = 4;
        const int64_t groups = (a.n_bags + BPG - 1) / BPG;
        const int blocks = fill_blocks(groups, WAVES * G::GROUPS, 256 * 32);
        hipLaunchKernelGGL((k_fwd_groups<D, BF16, MEAN, BPG, 4>), dim3(blocks), dim3(FWD_BLOCK), 0, s, a);
    }
    return launch_status();
}

template <int D, bool BF16>
int launch_fwd(const FwdArgs& a, int64_t n_ids, hipStream_t s) {
    return a.mean ? launch_fwd_p<D, BF16, true>(a, n_ids, s) : launch_fwd_p<D, BF16, false>(a, n_ids, s);
}

}  // namespace

extern "C" int embedding_bag_fwd(const rse_blocks* blocks, const int64_t* d_row_off, int64_t n_ids,
                                 const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch,
                                 int32_t pooling, float* d_out, void* stream) {
    if (!blocks || !d_bag_offsets || n_ids < 0 || n_tables <= 0 || batch < 0)
        return RSE_ERR_INVALID_ARG;
    if (pooling != RSE_SUM && pooling != RSE_MEAN) return RSE_ERR_INVALID_ARG;
    if (n_ids > 0 && !d_row_off) return RSE_ERR_INVALID_ARG;
    const int64_t n_bags = (int64_t)n_tables * batch;
    if (n_bags == 0) return RSE_OK;
    if (n_bags > (int64_t)0xFFFFFFFFll) return RSE_ERR_INVALID_ARG;
    if (!d_out) return RSE_ERR_INVALID_ARG;
    FwdArgs a;
    a.rv = blocks->view();
    a.row_off = d_row_off;
    a.bag_off = d_bag_offsets;
    a.n_bags = n_bags;
    a.batch = batch;
    a.n_ids = n_ids;
    a.capacity = blocks->capacity();
    a.status = &blocks->header()->status;
    a.n_tables = n_tables;
    a.mean = pooling == RSE_MEAN;
    a.out = d_out;
    hipStream_t s = as_stream(stream);
    const bool bf = blocks->w_dtype == RSE_BF16;
    switch (blocks->dim) {
        case 4: return bf ? RSE_ERR_UNSUPPORTED : launch_fwd<4, false>(a, n_ids, s);
        case 8: return bf ? launch_fwd<8, true>(a, n_ids, s) : launch_fwd<8, false>(a, n_ids, s);
        case 16: return bf ? launch_fwd<16, true>(a, n_ids, s) : launch_fwd<16, false>(a, n_ids, s);
        case 32: return bf ? launch_fwd<32, true>(a, n_ids, s) : launch_fwd<32, false>(a, n_ids, s);
        case 64: return bf ? launch_fwd<64, true>(a, n_ids, s) : launch_fwd<64, false>(a, n_ids, s);
        case 128: return bf ? launch_fwd<128, true>(a, n_ids, s) : launch_fwd<128, false>(a, n_ids, s);
        case 256: return bf ? launch_fwd<256, true>(a, n_ids, s) : launch_fwd<256, false>(a, n_ids, s);
        default: return RSE_ERR_UNSUPPORTED;
    }
}
