// rse_host.h -- host-side handle definitions and helpers shared by the
// library's translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/rse.h"
#include "rse_device.h"

struct rse_blocks {
    int32_t dim;
    int32_t w_dtype;
    int32_t optim;
    int32_t shift;          // log2(rows per chunk)
    int32_t max_chunks;
    int32_t n_chunks;
    int64_t row_bytes;
    uint64_t seed;
    char* d_meta;           // BlocksHeader followed by the chunk table
    std::vector<uint64_t> chunks;   // host copy of the chunk table
    uint32_t* d_free = nullptr;     // free list of rows (caller memory), or null
    int64_t free_cap = 0;

    rse::BlocksHeader* header() const { return reinterpret_cast<rse::BlocksHeader*>(d_meta); }
    uint64_t* chunk_table() const {
        return reinterpret_cast<uint64_t*>(d_meta + sizeof(rse::BlocksHeader));
    }
    int64_t capacity() const { return (int64_t)n_chunks << shift; }
    rse::RowsView view() const {
        rse::RowsView v;
        v.chunks = chunk_table();
        v.row_bytes = row_bytes;
        v.shift = shift;
        v.n_chunks = n_chunks;
        v.mask = (1ull << shift) - 1;
        return v;
    }
    int state_per_elem() const { return optim == RSE_SGD ? 0 : (optim == RSE_ADAGRAD ? 1 : 2); }
};

struct rse_idmap {
    int32_t n_tables;       // regions
    int32_t merged;
    int64_t total_slots;
    double max_load;
    char* d_mem;            // MapHeader, TableDir[n_tables], slots
    std::vector<rse::TableDir> dir;   // host copy of the static directory
    // age tracking: one stamp per row (caller memory), written with `clock`
    uint32_t* d_stamps = nullptr;
    int64_t n_stamps = 0;
    uint32_t clock = 0;
    // admission: count-min sketch [depth][width] (caller memory)
    uint32_t* d_sketch = nullptr;
    int32_t sk_depth = 0;
    int64_t sk_width = 0;
    uint32_t admit_min = 0;
    uint64_t sk_salt[8] = {};

    size_t mem_bytes() const;
    bool admission_on() const { return d_sketch && admit_min > 1 && sk_width > 0; }

    rse::MapHeader* header() const { return reinterpret_cast<rse::MapHeader*>(d_mem); }
    rse::TableDir* d_dir() const {
        return reinterpret_cast<rse::TableDir*>(d_mem + sizeof(rse::MapHeader));
    }
    rse::Slot* d_slots() const;
};

namespace rse_host {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Returns RSE_ERR_HIP if the last launch failed.
inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? RSE_OK : RSE_ERR_HIP;
}

inline bool dim_supported(int32_t dim, int32_t w_dtype) {
    if (w_dtype == RSE_F32) return dim == 4 || dim == 8 || dim == 16 || dim == 32 || dim == 64 ||
                                   dim == 128 || dim == 256;
    if (w_dtype == RSE_BF16) return dim == 8 || dim == 16 || dim == 32 || dim == 64 || dim == 128 ||
                                    dim == 256;
    return false;
}

// Kernel trace (rse_trace.hip): launch sites call trace_mark before and
// after launching a traceable kernel; it is a no-op unless that kernel is
// being traced.
extern int g_trace_kernel;
void trace_mark(int kernel, hipStream_t s, bool after);

struct TraceScope {
    int kernel;
    hipStream_t s;
    TraceScope(int k, hipStream_t st) : kernel(k), s(st) {
        if (g_trace_kernel == kernel) trace_mark(kernel, s, false);
    }
    ~TraceScope() {
        if (g_trace_kernel == kernel) trace_mark(kernel, s, true);
    }
};

// Number of blocks that keeps every CU busy for a grid-stride kernel.
inline int fill_blocks(int64_t work_items, int items_per_block, int max_blocks) {
    int64_t b = (work_items + items_per_block - 1) / items_per_block;
    if (b < 1) b = 1;
    if (b > max_blocks) b = max_blocks;
    return (int)b;
}

// Sequence of fixed-size workspace carve-outs, each 256-byte aligned.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* p) : base(static_cast<char*>(p)) {}
    template <typename T>
    T* take(size_t count) {
        off = align_up(off, 256);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
    size_t size() const { return align_up(off, 256); }
};

}  // namespace rse_host
