// rse_blocks.hip -- EmbeddingBlocks: chunked rows of weights plus optimizer
// state that grow by whole chunks without moving existing rows ("RecIS：
// 阿里开源推荐系统统一训练框架", section "Embedding Engine").
//
// The chunk-pointer table and the row counter live in caller device memory
// (the blocks' metadata); chunks are caller allocations registered with
// blocks_grow.  A row is addressed as chunk[row >> shift] + (row & mask) *
// row_bytes, so a lookup costs one extra (cached) 8-byte load.
#include <new>

#include "rse_host.h"

using namespace rse;
using namespace rse_host;

namespace {

__global__ void k_blocks_clear(BlocksHeader* h, uint64_t* chunks, int32_t max_chunks) {
    const int tid = blockIdx.x * blockDim.x + threadIdx.x;
    if (tid == 0) {
        h->rows_used = 0;
        h->status = 0;
        h->free_head = 0;
        h->free_count = 0;
    }
    for (int i = tid; i < max_chunks; i += gridDim.x * blockDim.x) chunks[i] = 0;
}

__global__ void k_set_chunk(uint64_t* chunks, int32_t idx, uint64_t ptr) { chunks[idx] = ptr; }

__global__ void k_clear_status32(int32_t* st) { *st = 0; }

// One group of `lanes` threads per row: widen weights to fp32, copy state.
template <bool BF16>
__global__ void k_read_rows(RowsView rv, const int64_t* offs, int64_t n, int dim, int k_state,
                            float* w_out, float* st_out) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t per_row = (int64_t)dim * (1 + k_state);
    for (int64_t e = tid; e < n * per_row; e += stride) {
        const int64_t q = e / per_row;
        const int64_t c = e - q * per_row;
        const char* row = rv.row(offs[q]);
        if (c < dim) {
            float v;
            if (BF16) v = bf16_to_f32(((const RSE_GLOBAL uint16_t*)row)[c]);
            else v = ((const RSE_GLOBAL float*)row)[c];
            w_out[q * dim + c] = v;
        } else if (st_out) {
            const int64_t w_bytes = (int64_t)dim * (BF16 ? 2 : 4);
            st_out[q * (per_row - dim) + (c - dim)] =
                ((const RSE_GLOBAL float*)(row + w_bytes))[c - dim];
        }
    }
}

// Inverse of k_read_rows: weights from fp32 (bf16 storage rounds to nearest
// even, exact for values read from bf16 rows), state copied.  Offsets outside
// the capacity are reported and skipped.
template <bool BF16>
__global__ void k_write_rows(RowsView rv, int64_t capacity, const int64_t* offs, int64_t n, int dim, int k_state,
                             const float* w_in, const float* st_in, int32_t* status) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t per_row = (int64_t)dim * (1 + k_state);
    for (int64_t e = tid; e < n * per_row; e += stride) {
        const int64_t q = e / per_row;
        const int64_t c = e - q * per_row;
        const int64_t r = offs[q];
        if (r < 0 || r >= capacity) {
            if (c == 0) atomicCAS(status, 0, (int32_t)RSE_ERR_BAD_INPUT);
            continue;
        }
        char* row = rv.row(r);
        if (c < dim) {
            const float v = w_in[q * dim + c];
            if (BF16) ((RSE_GLOBAL uint16_t*)row)[c] = f64_to_bf16_rne((double)v);
            else ((RSE_GLOBAL float*)row)[c] = v;
        } else if (st_in) {
            const int64_t w_bytes = (int64_t)dim * (BF16 ? 2 : 4);
            ((RSE_GLOBAL float*)(row + w_bytes))[c - dim] = st_in[q * (per_row - dim) + (c - dim)];
        }
    }
}

__global__ void k_set_rows_used(BlocksHeader* h, int64_t rows) { h->rows_used = rows; }

__global__ void k_reset_free_list(BlocksHeader* h) {
    h->free_head = 0;
    h->free_count = 0;
}

}  // namespace

extern "C" {

int rse_blocks_row_bytes(int32_t dim, int32_t w_dtype, int32_t optim, int64_t* row_bytes_out) {
    if (!row_bytes_out || optim < RSE_SGD || optim > RSE_ADAM) return RSE_ERR_INVALID_ARG;
    if (!dim_supported(dim, w_dtype)) return RSE_ERR_UNSUPPORTED;
    const int k = optim == RSE_SGD ? 0 : (optim == RSE_ADAGRAD ? 1 : 2);
    const int64_t w = (int64_t)dim * (w_dtype == RSE_BF16 ? 2 : 4);
    *row_bytes_out = (int64_t)align_up((size_t)(w + (int64_t)k * dim * 4), 16);
    return RSE_OK;
}

int rse_blocks_meta_size(int32_t max_chunks, size_t* bytes_out) {
    if (!bytes_out || max_chunks <= 0) return RSE_ERR_INVALID_ARG;
    *bytes_out = align_up(sizeof(BlocksHeader) + (size_t)max_chunks * 8, 256);
    return RSE_OK;
}

int rse_blocks_create(rse_blocks** out, void* d_meta, size_t meta_bytes, int32_t dim,
                      int32_t w_dtype, int32_t optim, int32_t rows_per_chunk_log2,
                      int32_t max_chunks, uint64_t init_seed, void* stream) {
    if (!out || !d_meta || max_chunks <= 0) return RSE_ERR_INVALID_ARG;
    if (rows_per_chunk_log2 < 4 || rows_per_chunk_log2 > 32) return RSE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(d_meta) % 256) return RSE_ERR_INVALID_ARG;
    int64_t rb = 0;
    int rc = rse_blocks_row_bytes(dim, w_dtype, optim, &rb);
    if (rc) return rc;
    size_t need = 0;
    rse_blocks_meta_size(max_chunks, &need);
    if (meta_bytes < need) return RSE_ERR_WORKSPACE;
    rse_blocks* b = new (std::nothrow) rse_blocks();
    if (!b) return RSE_ERR_INVALID_ARG;
    b->dim = dim;
    b->w_dtype = w_dtype;
    b->optim = optim;
    b->shift = rows_per_chunk_log2;
    b->max_chunks = max_chunks;
    b->n_chunks = 0;
    b->row_bytes = rb;
    b->seed = init_seed;
    b->d_meta = static_cast<char*>(d_meta);
    hipLaunchKernelGGL(k_blocks_clear, dim3(fill_blocks(max_chunks, 256, 64)), dim3(256), 0,
                       as_stream(stream), b->header(), b->chunk_table(), max_chunks);
    rc = launch_status();
    if (rc) {
        delete b;
        return rc;
    }
    *out = b;
    return RSE_OK;
}

int rse_blocks_destroy(rse_blocks* blocks) {
    delete blocks;
    return RSE_OK;
}

int blocks_grow(rse_blocks* b, void* d_chunk, size_t chunk_bytes, void* stream) {
    if (!b || !d_chunk) return RSE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(d_chunk) % 256) return RSE_ERR_INVALID_ARG;
    if (b->n_chunks >= b->max_chunks) return RSE_ERR_MAX_CHUNKS;
    const uint64_t need = (uint64_t)b->row_bytes << b->shift;
    if ((uint64_t)chunk_bytes < need) return RSE_ERR_CHUNK_TOO_SMALL;
    if (((int64_t)(b->n_chunks + 1) << b->shift) > RSE_MAX_ROWS + 1) return RSE_ERR_TOO_MANY_ROWS;
    hipLaunchKernelGGL(k_set_chunk, dim3(1), dim3(1), 0, as_stream(stream), b->chunk_table(),
                       b->n_chunks, (uint64_t)reinterpret_cast<uintptr_t>(d_chunk));
    int rc = launch_status();
    if (rc) return rc;
    b->chunks.push_back((uint64_t)reinterpret_cast<uintptr_t>(d_chunk));
    b->n_chunks += 1;
    return RSE_OK;
}

int rse_blocks_capacity(const rse_blocks* b, int64_t* rows_capacity_out, int64_t* rows_per_chunk_out,
                        int32_t* n_chunks_out) {
    if (!b) return RSE_ERR_INVALID_ARG;
    if (rows_capacity_out) *rows_capacity_out = b->capacity();
    if (rows_per_chunk_out) *rows_per_chunk_out = (int64_t)1 << b->shift;
    if (n_chunks_out) *n_chunks_out = b->n_chunks;
    return RSE_OK;
}

int rse_blocks_status(rse_blocks* b, int64_t* rows_used_out, int32_t* status_out, void* stream) {
    if (!b) return RSE_ERR_INVALID_ARG;
    BlocksHeader h;
    if (hipMemcpyAsync(&h, b->header(), sizeof(h), hipMemcpyDeviceToHost, as_stream(stream)) !=
        hipSuccess)
        return RSE_ERR_HIP;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return RSE_ERR_HIP;
    if (rows_used_out) *rows_used_out = h.rows_used;
    if (status_out) *status_out = h.status;
    return RSE_OK;
}

int rse_blocks_clear_status(rse_blocks* b, void* stream) {
    if (!b) return RSE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_clear_status32, dim3(1), dim3(1), 0, as_stream(stream), &b->header()->status);
    return launch_status();
}

int rse_blocks_read_rows(const rse_blocks* b, const int64_t* d_offs, int64_t n, float* d_w_out,
                         float* d_state_out, void* stream) {
    if (!b || n < 0 || (n > 0 && (!d_offs || !d_w_out))) return RSE_ERR_INVALID_ARG;
    if (n == 0) return RSE_OK;
    const int k = b->state_per_elem();
    const int64_t work = n * b->dim * (1 + k);
    const dim3 grid(fill_blocks(work, 256, 4096));
    if (b->w_dtype == RSE_BF16)
        hipLaunchKernelGGL(k_read_rows<true>, grid, dim3(256), 0, as_stream(stream), b->view(), d_offs,
                           n, b->dim, k, d_w_out, k ? d_state_out : nullptr);
    else
        hipLaunchKernelGGL(k_read_rows<false>, grid, dim3(256), 0, as_stream(stream), b->view(), d_offs,
                           n, b->dim, k, d_w_out, k ? d_state_out : nullptr);
    return launch_status();
}

int rse_blocks_write_rows(rse_blocks* b, const int64_t* d_offs, int64_t n, const float* d_w,
                          const float* d_state, void* stream) {
    if (!b || n < 0 || (n > 0 && (!d_offs || !d_w))) return RSE_ERR_INVALID_ARG;
    const int k = b->state_per_elem();
    if (n > 0 && k > 0 && !d_state) return RSE_ERR_INVALID_ARG;
    if (n == 0) return RSE_OK;
    const int64_t work = n * b->dim * (1 + k);
    const dim3 grid(fill_blocks(work, 256, 4096));
    if (b->w_dtype == RSE_BF16)
        hipLaunchKernelGGL(k_write_rows<true>, grid, dim3(256), 0, as_stream(stream), b->view(), b->capacity(),
                           d_offs, n, b->dim, k, d_w, k ? d_state : nullptr, &b->header()->status);
    else
        hipLaunchKernelGGL(k_write_rows<false>, grid, dim3(256), 0, as_stream(stream), b->view(), b->capacity(),
                           d_offs, n, b->dim, k, d_w, k ? d_state : nullptr, &b->header()->status);
    return launch_status();
}

int rse_blocks_set_rows_used(rse_blocks* b, int64_t rows_used, void* stream) {
    if (!b || rows_used < 0 || rows_used > b->capacity()) return RSE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_set_rows_used, dim3(1), dim3(1), 0, as_stream(stream), b->header(), rows_used);
    return launch_status();
}

const char* rse_status_str(int status) {
    switch (status) {
        case RSE_OK: return "RSE_OK";
        case RSE_ERR_INVALID_ARG: return "RSE_ERR_INVALID_ARG";
        case RSE_ERR_UNSUPPORTED: return "RSE_ERR_UNSUPPORTED";
        case RSE_ERR_WORKSPACE: return "RSE_ERR_WORKSPACE";
        case RSE_ERR_IDMAP_FULL: return "RSE_ERR_IDMAP_FULL";
        case RSE_ERR_NEED_GROW: return "RSE_ERR_NEED_GROW";
        case RSE_ERR_CHUNK_TOO_SMALL: return "RSE_ERR_CHUNK_TOO_SMALL";
        case RSE_ERR_MAX_CHUNKS: return "RSE_ERR_MAX_CHUNKS";
        case RSE_ERR_HIP: return "RSE_ERR_HIP";
        case RSE_ERR_BAD_INPUT: return "RSE_ERR_BAD_INPUT";
        case RSE_ERR_TOO_MANY_ROWS: return "RSE_ERR_TOO_MANY_ROWS";
        default: return "RSE_ERR_UNKNOWN";
    }
}

int rse_version(void) { return 100; }

int rse_blocks_set_free_list(rse_blocks* blocks, uint32_t* d_free, int64_t capacity, void* stream) {
    if (!blocks || capacity < 0 || (capacity > 0 && !d_free)) return RSE_ERR_INVALID_ARG;
    blocks->d_free = capacity > 0 ? d_free : nullptr;
    blocks->free_cap = capacity > 0 ? capacity : 0;
    hipLaunchKernelGGL(k_reset_free_list, dim3(1), dim3(1), 0, as_stream(stream), blocks->header());
    return launch_status();
}

int rse_blocks_free_status(rse_blocks* blocks, int64_t* head_out, int64_t* count_out, void* stream) {
    if (!blocks) return RSE_ERR_INVALID_ARG;
    BlocksHeader h;
    if (hipMemcpyAsync(&h, blocks->header(), sizeof(h), hipMemcpyDeviceToHost, as_stream(stream)) != hipSuccess)
        return RSE_ERR_HIP;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return RSE_ERR_HIP;
    if (head_out) *head_out = h.free_head;
    if (count_out) *count_out = h.free_count;
    return RSE_OK;
}

}  // extern "C"
