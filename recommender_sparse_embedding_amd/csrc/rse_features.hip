// rse_features.hip -- fused feature transforms: raw feature values -> int64
// ids in one launch for every table ("RecIS：阿里开源推荐系统统一训练框架",
// "Feature Engine": Hash, Mod and Bucketize, with small operations merged
// into one GPU kernel launch).
//
// The pages name the operations only; the definitions (each table's program
// of up to four operations on its 64-bit raw values) are stated in rse.h.
// The kernel is a single streaming pass: one lookup per thread, its table
// found by a binary search over the table bounds held in LDS, its program
// read through the cache (a wave's 64 consecutive lookups nearly always
// belong to one table, so the reads coincide), 8 bytes read and 8 written
// per lookup.  Bucketize searches the table's boundaries, which stay in L2.
#include <new>

#include "rse_host.h"

using namespace rse;
using namespace rse_host;

struct rse_features {
    int32_t n_tables;
    int64_t n_boundaries;
    char* d_mem;      // FtHeader, programs [n_tables], boundaries [n_boundaries]
    size_t prog_off;
    size_t bnd_off;
};

namespace {

struct FtHeader {
    int32_t status;
    int32_t n_tables;
    int64_t pad[31];
};
static_assert(sizeof(FtHeader) == 256, "FtHeader size");

constexpr int FT_BLOCK = 256;

struct FtArgs {
    const uint64_t* raw;
    int64_t n;
    const int64_t* bounds;
    int64_t stride;
    int32_t n_tables;
    int32_t pad;
    const rse_feature_program* progs;
    const double* bnd;
    int64_t* ids;
    FtHeader* h;
};

__device__ __forceinline__ uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

// xxHash64 (Collet's published algorithm) of one 8-byte little-endian word:
// an input shorter than 32 bytes starts from seed + prime 5, adds its length,
// folds in its one 8-byte lane and ends with the avalanche.
__device__ __forceinline__ uint64_t xxh64_word(uint64_t w, uint64_t seed) {
    constexpr uint64_t P1 = 0x9E3779B185EBCA87ull, P2 = 0xC2B2AE3D27D4EB4Full, P3 = 0x165667B19E3779F9ull,
                       P4 = 0x85EBCA77C2B2AE63ull, P5 = 0x27D4EB2F165667C5ull;
    uint64_t h = seed + P5 + 8;
    h ^= rotl64(w * P2, 31) * P1;
    h = rotl64(h, 27) * P1 + P4;
    h ^= h >> 33;
    h *= P2;
    h ^= h >> 29;
    h *= P3;
    h ^= h >> 32;
    return h;
}

// Floor modulo by m > 0 (result in [0, m)).
__device__ __forceinline__ int64_t floor_mod(int64_t v, int64_t m) {
    const int64_t r = v % m;
    return r < 0 ? r + m : r;
}

// Number of boundaries <= x (upper bound); NaN counts all of them.
__device__ __forceinline__ int64_t bucket_of(double x, const double* b, int32_t n) {
    if (x != x) return n;
    int32_t lo = 0, hi = n;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (b[mid] <= x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ int table_of_lookup(const int64_t* sb, int n_tables, int64_t i) {
    int lo = 0, hi = n_tables;            // sb[lo] <= i < sb[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sb[mid] <= i) lo = mid;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(FT_BLOCK) void k_features(FtArgs a) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    __syncthreads();
    for (int t = threadIdx.x; t < a.n_tables; t += blockDim.x)
        if (sb[t + 1] < sb[t]) s_bad = 1;
    if (threadIdx.x == 0 && (sb[0] != 0 || sb[a.n_tables] != a.n)) s_bad = 1;
    __syncthreads();
    if (s_bad) {                          // malformed bounds: report, write nothing
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicCAS(&a.h->status, 0, (int32_t)RSE_ERR_BAD_INPUT);
        return;
    }
    for (int64_t i = (int64_t)blockIdx.x * FT_BLOCK + threadIdx.x; i < a.n; i += (int64_t)gridDim.x * FT_BLOCK) {
        const int t = table_of_lookup(sb, a.n_tables, i);
        const rse_feature_program* p = a.progs + t;
        uint64_t v = a.raw[i];
        const int n_ops = p->n_ops;
        for (int k = 0; k < n_ops; ++k) {
            const rse_feature_op op = p->ops[k];
            if (op.kind == RSE_FT_HASH) {
                v = xxh64_word(v, (uint64_t)op.arg);
            } else if (op.kind == RSE_FT_MOD) {
                v = (uint64_t)floor_mod((int64_t)v, op.arg);
            } else if (op.kind == RSE_FT_BUCKETIZE) {
                v = (uint64_t)bucket_of(__longlong_as_double((long long)v), a.bnd + op.arg, op.n_boundaries);
            }
        }
        a.ids[i] = (int64_t)v;
    }
}

__global__ void k_ft_clear(FtHeader* h, int32_t n_tables) {
    h->status = 0;
    h->n_tables = n_tables;
}

// Host check of one program against the definitions: kinds, arguments, the
// value's type along the chain, boundaries in range, ascending, no NaN.
bool program_ok(const rse_feature_program& p, const double* bnd, int64_t n_bnd) {
    if (p.input != RSE_FT_INT64 && p.input != RSE_FT_FLOAT64) return false;
    if (p.n_ops < 0 || p.n_ops > RSE_FT_MAX_OPS) return false;
    bool is_float = p.input == RSE_FT_FLOAT64;
    for (int k = 0; k < p.n_ops; ++k) {
        const rse_feature_op& op = p.ops[k];
        switch (op.kind) {
            case RSE_FT_IDENTITY:
                break;
            case RSE_FT_HASH:
                is_float = false;
                break;
            case RSE_FT_MOD:
                if (is_float || op.arg <= 0) return false;
                break;
            case RSE_FT_BUCKETIZE: {
                if (!is_float || op.arg < 0 || op.n_boundaries < 0 || op.arg + op.n_boundaries > n_bnd) return false;
                for (int64_t j = 0; j < op.n_boundaries; ++j) {
                    const double b = bnd[op.arg + j];
                    if (b != b || (j > 0 && b < bnd[op.arg + j - 1])) return false;
                }
                is_float = false;
                break;
            }
            default:
                return false;
        }
    }
    return !is_float;
}

void layout(int32_t n_tables, int64_t n_boundaries, size_t* prog_off, size_t* bnd_off, size_t* total) {
    *prog_off = sizeof(FtHeader);
    *bnd_off = align_up(*prog_off + (size_t)n_tables * sizeof(rse_feature_program), 256);
    *total = *bnd_off + (size_t)n_boundaries * sizeof(double);
}

}  // namespace

extern "C" {

int rse_features_mem_size(int32_t n_tables, int64_t n_boundaries, size_t* bytes_out) {
    if (!bytes_out || n_tables <= 0 || n_tables > RSE_MAX_TABLES || n_boundaries < 0) return RSE_ERR_INVALID_ARG;
    size_t a, b;
    layout(n_tables, n_boundaries, &a, &b, bytes_out);
    return RSE_OK;
}

int rse_features_create(rse_features** out, void* d_mem, size_t mem_bytes, const rse_feature_program* programs,
                        int32_t n_tables, const double* boundaries, int64_t n_boundaries, void* stream) {
    if (!out || !d_mem || !programs || (n_boundaries > 0 && !boundaries)) return RSE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(d_mem) % 256) return RSE_ERR_INVALID_ARG;
    size_t need = 0;
    int rc = rse_features_mem_size(n_tables, n_boundaries, &need);
    if (rc) return rc;
    if (mem_bytes < need) return RSE_ERR_WORKSPACE;
    for (int t = 0; t < n_tables; ++t)
        if (!program_ok(programs[t], boundaries, n_boundaries)) return RSE_ERR_INVALID_ARG;
    rse_features* f = new (std::nothrow) rse_features();
    if (!f) return RSE_ERR_INVALID_ARG;
    f->n_tables = n_tables;
    f->n_boundaries = n_boundaries;
    f->d_mem = static_cast<char*>(d_mem);
    layout(n_tables, n_boundaries, &f->prog_off, &f->bnd_off, &need);
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(k_ft_clear, dim3(1), dim3(1), 0, s, reinterpret_cast<FtHeader*>(f->d_mem), n_tables);
    bool ok = hipMemcpyAsync(f->d_mem + f->prog_off, programs, (size_t)n_tables * sizeof(rse_feature_program),
                             hipMemcpyHostToDevice, s) == hipSuccess;
    if (ok && n_boundaries > 0)
        ok = hipMemcpyAsync(f->d_mem + f->bnd_off, boundaries, (size_t)n_boundaries * sizeof(double),
                            hipMemcpyHostToDevice, s) == hipSuccess;
    // the host arrays are the sources of asynchronous copies: wait for them
    if (!ok || hipStreamSynchronize(s) != hipSuccess) {
        delete f;
        return RSE_ERR_HIP;
    }
    rc = launch_status();
    if (rc) {
        delete f;
        return rc;
    }
    *out = f;
    return RSE_OK;
}

int rse_features_destroy(rse_features* f) {
    delete f;
    return RSE_OK;
}

int feature_transform(const rse_features* f, const int64_t* d_raw, int64_t n, const int64_t* d_bounds,
                      int64_t stride, int64_t* d_ids_out, void* stream) {
    if (!f || !d_bounds || n < 0 || stride <= 0) return RSE_ERR_INVALID_ARG;
    if (n > 0 && (!d_raw || !d_ids_out)) return RSE_ERR_INVALID_ARG;
    FtArgs a;
    a.raw = reinterpret_cast<const uint64_t*>(d_raw);
    a.n = n;
    a.bounds = d_bounds;
    a.stride = stride;
    a.n_tables = f->n_tables;
    a.pad = 0;
    a.progs = reinterpret_cast<const rse_feature_program*>(f->d_mem + f->prog_off);
    a.bnd = reinterpret_cast<const double*>(f->d_mem + f->bnd_off);
    a.ids = d_ids_out;
    a.h = reinterpret_cast<FtHeader*>(f->d_mem);
    hipLaunchKernelGGL(k_features, dim3(fill_blocks(n, FT_BLOCK, 2048)), dim3(FT_BLOCK), 0, as_stream(stream), a);
    return launch_status();
}

int rse_features_status(rse_features* f, int32_t* status_out, void* stream) {
    if (!f || !status_out) return RSE_ERR_INVALID_ARG;
    FtHeader h;
    if (hipMemcpyAsync(&h, f->d_mem, sizeof(h), hipMemcpyDeviceToHost, as_stream(stream)) != hipSuccess)
        return RSE_ERR_HIP;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return RSE_ERR_HIP;
    *status_out = h.status;
    return RSE_OK;
}

}  // extern "C"
