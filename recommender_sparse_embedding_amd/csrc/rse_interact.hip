// rse_interact.hip -- DLRM pairwise dot interaction on the pooled embeddings
// ("DLRM — Meta 把工业推荐模型拆成 4 个标准积木", "核心思想" item 3 and
// "案例 3": the dense vector and the N pooled embeddings of a sample are
// stacked, all pairwise dot products are taken, the strict upper triangle is
// kept and concatenated after the dense vector: [4,3,4] -> [4,6] -> [4,10]).
//
// Per sample b, with F = n_tables + 1 vectors x_0 = dense[b, :] and
// x_{t+1} = pooled[b, t, :] (dim d each), and the P = F(F-1)/2 pairs (i < j)
// in row-major order (0,1), (0,2), ..., (0,F-1), (1,2), ...:
//   forward:  out[b, 0:d] = x_0;  out[b, d + p(i,j)] = x_i . x_j
//   backward: with g_ij = dout[b, d + p(i,j)] (and g_ji = g_ij),
//             dx_i = sum_{j != i} g_ij x_j;  ddense = dout[b, 0:d] + dx_0;
//             dpooled[b, t, :] = dx_{t+1}
// Shapes with F <= 32 and d in {32, 64, 128} run on the matrix cores
// (below); the others on the vector kernels here, whose products of fp32
// values are exact in fp64 and are accumulated in fp64, rounded once.
//
// Both kernels stage a sample's vectors in LDS (fp32, row stride d + 1 so
// that a column of rows falls in different banks) and work on 4 x 4 register
// tiles: the forward on tiles of pairs (4 x 4 dot products per thread, 8 LDS
// reads per 16 fused multiply-adds), split over KS adjacent lanes along d
// (interleaved: lane s takes elements s, s + KS, ...) when a sample has few
// tiles, the KS partial sums added by shuffles; the backward on tiles of
// (4 vectors x 4 elements K, K + d/4, ...), the symmetric pair matrix G
// staged in LDS beside X.
#include "rse_host.h"

using namespace rse;
using namespace rse_host;

namespace {

constexpr int IB = 256;                 // threads per block
constexpr size_t IX_LDS_MAX = 64 * 1024;  // LDS bytes per block for one sample

__device__ __forceinline__ int64_t pair_index(int i, int j, int F) {
    // row-major index of (i, j), i < j, in the strict upper triangle of F x F
    return (int64_t)i * F - (int64_t)i * (i + 1) / 2 + (j - i - 1);
}

// Upper-triangle tile (I, J), I <= J, of an nb x nb grid of 4 x 4 tiles.
__device__ __forceinline__ void tile_of(int tile, int nb, int& I, int& J) {
    int r = 0, left = tile;
    while (left >= nb - r) {
        left -= nb - r;
        ++r;
    }
    I = r;
    J = r + left;
}

// Loads sample b's F vectors into s_x (row stride d + 1): each wave copies
// whole rows, 64 consecutive floats per load (the sample's pooled rows are
// contiguous in [batch, n_tables, dim]).
__device__ __forceinline__ void stage_vectors(float* s_x, const float* dense, const float* pooled, int64_t b,
                                              int T, int d) {
    const int F = T + 1, st = d + 1;
    const int lane = lane_id(), wave = threadIdx.x / WAVE, n_waves = blockDim.x / WAVE;
    const float* prow = pooled + b * (int64_t)T * d;
    for (int i = wave; i < F; i += n_waves) {
        const float* src = i == 0 ? dense + b * d : prow + (int64_t)(i - 1) * d;
        for (int k = lane; k < d; k += WAVE) s_x[i * st + k] = src[k];
    }
}

__global__ __launch_bounds__(IB) void k_dot_fwd(const float* dense, const float* pooled, int64_t B, int T, int d,
                                                int ks, float* out) {
    extern __shared__ float s_x[];
    const int F = T + 1, st = d + 1, nb = (F + 3) / 4;
    const int n_tiles = nb * (nb + 1) / 2;
    const int64_t P = (int64_t)F * (F - 1) / 2;
    const int64_t row = d + P;
    for (int64_t b = blockIdx.x; b < B; b += gridDim.x) {
        __syncthreads();                         // s_x of the previous sample is no longer read
        stage_vectors(s_x, dense, pooled, b, T, d);
        for (int k = threadIdx.x; k < d; k += blockDim.x) out[b * row + k] = dense[b * d + k];
        __syncthreads();
        // tiles x ks lanes; the ks lanes of a tile are adjacent (ks divides 64)
        for (int w = threadIdx.x; w < ((n_tiles * ks + 63) / 64) * 64; w += blockDim.x) {
            const int tile = w / ks, sub = w - tile * ks;
            const bool live = tile < n_tiles;
            int I = 0, J = 0;
            if (live) tile_of(tile, nb, I, J);
            double acc[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
            // lane `sub` of the tile takes elements sub, sub + ks, ... (adjacent
            // lanes read adjacent words: no bank conflicts among them)
            const int k1 = live ? d : 0;
            int ri[4], rj[4];
            bool vi[4], vj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vi[r] = 4 * I + r < F;
                vj[r] = 4 * J + r < F;
                ri[r] = (vi[r] ? 4 * I + r : 0) * st;
                rj[r] = (vj[r] ? 4 * J + r : 0) * st;
            }
            for (int k = sub; k < k1; k += ks) {
                double xi[4], xj[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xi[r] = vi[r] ? (double)s_x[ri[r] + k] : 0.0;
                    xj[r] = vj[r] ? (double)s_x[rj[r] + k] : 0.0;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[r][c] = __fma_rn(xi[r], xj[c], acc[r][c]);
            }
            // add the ks partial sums (lanes sub = 0..ks-1 of the tile)
            for (int m = 1; m < ks; m <<= 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[r][c] += shfl_xor_f64(acc[r][c], m);
            }
            if (live && sub == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int i = 4 * I + r, j = 4 * J + c;
                        if (i < j && j < F) out[b * row + d + pair_index(i, j, F)] = (float)acc[r][c];
                    }
            }
        }
    }
}

__global__ __launch_bounds__(IB) void k_dot_bwd(const float* dense, const float* pooled, const float* dout,
                                                int64_t B, int T, int d, float* ddense, float* dpooled) {
    extern __shared__ float s_mem[];
    const int F = T + 1, st = d + 1, nb = (F + 3) / 4, kb = (d + 3) / 4;
    const int64_t P = (int64_t)F * (F - 1) / 2;
    const int64_t row = d + P;
    float* s_x = s_mem;                          // F x (d + 1)
    float* s_g = s_mem + F * st;                 // F x F, symmetric, zero diagonal
    for (int64_t b = blockIdx.x; b < B; b += gridDim.x) {
        __syncthreads();
        stage_vectors(s_x, dense, pooled, b, T, d);
        // the pair gradients (a contiguous run per row i of the triangle)
        // into both halves of the symmetric matrix; zero diagonal
        {
            const int lane = lane_id(), wave = threadIdx.x / WAVE, n_waves = blockDim.x / WAVE;
            for (int i = wave; i < F; i += n_waves) {
                const float* src = dout + b * row + d + pair_index(i, i + 1, F) - (i + 1);   // src[j] for j > i
                // row i writes its diagonal and (i, j), (j, i) for j > i, so
                // every entry has exactly one writer
                for (int j = i + lane; j < F; j += WAVE) {
                    const float g = j > i ? src[j] : 0.0f;
                    s_g[i * F + j] = g;
                    if (j > i) s_g[j * F + i] = g;
                }
            }
        }
        __syncthreads();
        // tile = (4 vectors I, 4 elements K)
        for (int tile = threadIdx.x; tile < nb * kb; tile += blockDim.x) {
            const int I = tile / kb, K = tile - I * kb;
            double acc[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
            // elements K, K + kb, K + 2 kb, K + 3 kb: adjacent lanes (adjacent K)
            // read adjacent words
            bool vi[4], vk[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vi[r] = 4 * I + r < F;
                vk[r] = K + r * kb < d;
            }
            for (int j = 0; j < F; ++j) {
                double g[4], x[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    g[r] = vi[r] ? (double)s_g[(4 * I + r) * F + j] : 0.0;
                    x[r] = vk[r] ? (double)s_x[j * st + K + r * kb] : 0.0;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[r][c] = __fma_rn(g[r], x[c], acc[r][c]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * I + r;
                if (!vi[r]) continue;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int k = K + c * kb;
                    if (!vk[c]) continue;
                    if (i == 0) ddense[b * d + k] = (float)((double)dout[b * row + k] + acc[r][c]);
                    else dpooled[(b * T + (i - 1)) * (int64_t)d + k] = (float)acc[r][c];
                }
            }
        }
    }
}

// ------------------------------------------------ matrix-core path ------
// For F <= 32 vectors per sample and d in {32, 64, 128} the interaction is
// a batch of small dense contractions: the forward's Gram matrix X X^T
// (F x d by d x F) and the backward's G X (F x F by F x d).  One wave takes
// one sample at a time: its F vectors are staged in LDS (row stride d + 4,
// 16-byte aligned), then v_mfma_f32_32x32x2_f32 accumulates 32 x 32 tiles
// in fp32 (rows and columns past F read as zero).
//
// v_mfma_f32_32x32x2_f32: lane l supplies A[l % 32][l / 32] and
// B[l / 32][l % 32]; accumulator register r of lane l holds
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  In the forward both operands
// are X (B = X^T holds the same values lane for lane); the two k positions of
// an instruction are taken from the two halves of the block's k range, so
// each lane reads 4 consecutive floats of its row per 4 instructions.
// Precision: fp32 products and sums over blocks of at most 64 elements,
// the blocks added in fp64: |error| <= 65 * 2^-24 * sum_k |x_ik x_jk| for a
// dot product (backward: <= 33 * 2^-24 * sum_j |g_ij| |x_jk|, plus one
// rounding of the dense gradient's sum).
typedef float f32x16 __attribute__((ext_vector_type(16)));


constexpr int MF_MAX_F = 32;

__device__ __forceinline__ int mf_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Wave-level ordering of a wave's own LDS writes before its other lanes
// read them (each wave works in its own part of LDS).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sample b's F vectors as NPF 16-byte pieces per lane (piece q = u * 64 +
// lane: row q / (D/4), four floats at column 4 (q % (D/4))); rows past F
// are not loaded.  The loads are issued for the next sample while the
// current one is computed, then written to LDS (row stride D + 4).
template <int D>
struct MfVectors {
    static constexpr int Q = D / 4, ST = D + 4, NPF = (MF_MAX_F * Q + WAVE - 1) / WAVE;
    f32x4 v[NPF];
    __device__ __forceinline__ void load(const float* dense, const float* pooled, int64_t b, int T, int lane) {
        const int F = T + 1;
        const f32x4* drow = reinterpret_cast<const f32x4*>(dense + b * D);
        const f32x4* prow = reinterpret_cast<const f32x4*>(pooled + b * (int64_t)T * D);
#pragma unroll
        for (int u = 0; u < NPF; ++u) {
            const int q = u * WAVE + lane;
            const int r = q / Q, c = q % Q;
            if (q < F * Q) v[u] = r == 0 ? drow[c] : prow[(int64_t)(r - 1) * Q + c];
        }
    }
    __device__ __forceinline__ void store(float* x, int T, int lane) const {
        const int F = T + 1;
#pragma unroll
        for (int u = 0; u < NPF; ++u) {
            const int q = u * WAVE + lane;
            if (q < F * Q) *reinterpret_cast<f32x4*>(x + (q / Q) * ST + (q % Q) * 4) = v[u];
        }
    }
};

template <int D>
__global__ __launch_bounds__(256) void k_dot_fwd_mfma(const float* dense, const float* pooled, int64_t B, int T,
                                                      float* out) {
    extern __shared__ float smem[];
    constexpr int ST = D + 4, KB = D < 64 ? D : 64, KH = KB / 2, NB = D / KB;
    constexpr bool PREFETCH = D <= 128;         // the next sample's vectors in registers
    const int F = T + 1;
    const int64_t P = (int64_t)F * T / 2, ROW = D + P;
    const int lane = lane_id(), w = threadIdx.x / WAVE, W = blockDim.x / WAVE;
    float* x = smem + w * F * ST;
    const int row = lane & 31, half = lane >> 5;
    const int64_t nw = (int64_t)gridDim.x * W;
    MfVectors<D> pf;
    int64_t b = (int64_t)blockIdx.x * W + w;
    if (PREFETCH && b < B) pf.load(dense, pooled, b, T, lane);
    for (; b < B; b += nw) {
        if (!PREFETCH) pf.load(dense, pooled, b, T, lane);
        pf.store(x, T, lane);
        wave_sync();
        if (PREFETCH && b + nw < B) pf.load(dense, pooled, b + nw, T, lane);
        // one fp32 accumulator tile per block of KB elements
        f32x16 c[NB];
        const float* xr = x + (row < F ? row : 0) * ST + half * KH;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            c[nb] = f32x16{};
#pragma unroll
            for (int s = 0; s < KH; s += 4) {
                f32x4 v = *reinterpret_cast<const f32x4*>(xr + nb * KB + s);
                if (row >= F) v = f32x4{0.f, 0.f, 0.f, 0.f};
                c[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v.x, v.x, c[nb], 0, 0, 0);
                c[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v.y, v.y, c[nb], 0, 0, 0);
                c[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v.z, v.z, c[nb], 0, 0, 0);
                c[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v.w, v.w, c[nb], 0, 0, 0);
            }
        }
        float* o = out + b * ROW;
        for (int cc = lane; cc < D; cc += WAVE) o[cc] = x[cc];
        const int j = row;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = mf_row(r, lane);
            double v = 0.0;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) v += (double)c[nb][r];
            if (i < j && j < F) o[D + pair_index(i, j, F)] = (float)v;
        }
        wave_sync();                            // x is rewritten for the next sample
    }
}

// LDS per wave of the backward: X (F rows, stride D + 4), the pair row of
// the output gradient (P floats) and the symmetric pair matrix G (32 x 33,
// zero outside F x F and on the diagonal).  The backward is held to two
// waves per SIMD (256 registers; click-log shape 0.95 -> 0.61 ms: the
// second wave hides the first one's loads and scattered G reads); the
// forward gains nothing from that and keeps its registers.
constexpr int MF_GS = MF_MAX_F + 1;
constexpr int MF_MAX_P = MF_MAX_F * (MF_MAX_F - 1) / 2;

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_dot_bwd_mfma(const float* dense, const float* pooled, const float* dout,
                                                      int64_t B, int T, float* ddense, float* dpooled) {
    extern __shared__ float smem[];
    constexpr int ST = D + 4, NPP = (MF_MAX_P + WAVE - 1) / WAVE;
    const int F = T + 1;
    const int P = F * T / 2;
    const int64_t ROW = D + P;
    const int lane = lane_id(), w = threadIdx.x / WAVE, W = blockDim.x / WAVE;
    float* x = smem + w * (F * ST + MF_MAX_P + MF_MAX_F * MF_GS);
    float* gp = x + F * ST;                     // the sample's pair gradients, row-major pairs
    float* g = gp + MF_MAX_P;
    const int row = lane & 31, half = lane >> 5;
    const int64_t nw = (int64_t)gridDim.x * W;
    MfVectors<D> pf;
    float pv[NPP];
    constexpr bool PREFETCH = D <= 128;
    int64_t b = (int64_t)blockIdx.x * W + w;
    auto load_pairs = [&](int64_t bb) {
        const float* go = dout + bb * ROW + D;
#pragma unroll
        for (int u = 0; u < NPP; ++u) {
            const int p = u * WAVE + lane;
            if (p < P) pv[u] = go[p];
        }
    };
    if (PREFETCH && b < B) {
        pf.load(dense, pooled, b, T, lane);
        load_pairs(b);
    }
    for (; b < B; b += nw) {
        if (!PREFETCH) {
            pf.load(dense, pooled, b, T, lane);
            load_pairs(b);
        }
        pf.store(x, T, lane);
#pragma unroll
        for (int u = 0; u < NPP; ++u) {
            const int p = u * WAVE + lane;
            if (p < P) gp[p] = pv[u];
        }
        wave_sync();
        for (int e = lane; e < MF_MAX_F * MF_MAX_F; e += WAVE) {
            const int i = e >> 5, j = e & 31;
            const int lo = i < j ? i : j, hi = i < j ? j : i;
            g[i * MF_GS + j] = (hi < F && lo != hi) ? gp[pair_index(lo, hi, F)] : 0.f;
        }
        wave_sync();
        if (PREFETCH && b + nw < B) {
            pf.load(dense, pooled, b + nw, T, lane);
            load_pairs(b + nw);
        }
        const int ksteps = (F + 1) / 2;
        for (int cb = 0; cb < D; cb += 32) {
            f32x16 c = {};
            for (int s = 0; s < ksteps; ++s) {
                const int k = 2 * s + half;
                const float a = g[row * MF_GS + k];
                const float bv = k < F ? x[k * ST + cb + row] : 0.f;
                c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv, c, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = mf_row(r, lane);
                const int col = cb + row;
                if (i >= F) continue;
                if (i == 0)
                    ddense[b * D + col] = (float)((double)c[r] + (double)dout[b * ROW + col]);
                else
                    dpooled[(b * T + (i - 1)) * (int64_t)D + col] = c[r];
            }
        }
        wave_sync();
    }
}

// Waves per block of the matrix-core kernels: as many samples as fit 64 KiB
// of LDS, at most 4.
int mf_waves(size_t per_wave) {
    const size_t w = (64 * 1024) / per_wave;
    return (int)(w < 1 ? 1 : (w > 4 ? 4 : w));
}

bool mf_ok(int32_t n_tables, int32_t dim) {
    return n_tables + 1 <= MF_MAX_F && (dim == 32 || dim == 64 || dim == 128);
}

int check_shape(int64_t batch, int32_t n_tables, int32_t dim, size_t* lds_fwd, size_t* lds_bwd) {
    if (batch < 0 || n_tables < 1 || dim < 1 || dim > 4096) return RSE_ERR_INVALID_ARG;
    const int64_t F = (int64_t)n_tables + 1;
    *lds_fwd = (size_t)F * (dim + 1) * sizeof(float);
    *lds_bwd = *lds_fwd + (size_t)F * F * sizeof(float);
    if (*lds_bwd > IX_LDS_MAX) return RSE_ERR_UNSUPPORTED;
    return RSE_OK;
}

int grid_for(int64_t batch) { return fill_blocks(batch, 1, 256 * 8); }

}  // namespace

extern "C" {

int dlrm_interaction_fwd(const float* d_dense, const float* d_pooled, int64_t batch, int32_t n_tables,
                         int32_t dim, float* d_out, void* stream) {
    size_t lf = 0, lb = 0;
    int rc = check_shape(batch, n_tables, dim, &lf, &lb);
    if (rc) return rc;
    if (batch == 0) return RSE_OK;
    if (!d_dense || !d_pooled || !d_out) return RSE_ERR_INVALID_ARG;
    const int F = n_tables + 1, nb = (F + 3) / 4, n_tiles = nb * (nb + 1) / 2;
    if (mf_ok(n_tables, dim)) {
        const size_t per_wave = (size_t)F * (dim + 4) * sizeof(float);
        const int W = mf_waves(per_wave);
        const dim3 grid(fill_blocks(batch, W, 256 * 8)), block(W * WAVE);
        const size_t lds = per_wave * W;
        hipStream_t st = as_stream(stream);
        TraceScope ts(RSE_K_INTERACT, st);
        switch (dim) {
            case 32: hipLaunchKernelGGL(k_dot_fwd_mfma<32>, grid, block, lds, st, d_dense, d_pooled, batch, (int)n_tables, d_out); break;
            case 64: hipLaunchKernelGGL(k_dot_fwd_mfma<64>, grid, block, lds, st, d_dense, d_pooled, batch, (int)n_tables, d_out); break;
            default: hipLaunchKernelGGL(k_dot_fwd_mfma<128>, grid, block, lds, st, d_dense, d_pooled, batch, (int)n_tables, d_out); break;
        }
        return launch_status();
    }
    // split d over ks adjacent lanes while the block has idle threads
    int ks = 1;
    while (ks < 64 && n_tiles * ks * 2 <= IB && dim / (ks * 2) >= 4) ks *= 2;
    TraceScope ts(RSE_K_INTERACT, as_stream(stream));
    hipLaunchKernelGGL(k_dot_fwd, dim3(grid_for(batch)), dim3(IB), lf, as_stream(stream), d_dense, d_pooled, batch,
                       (int)n_tables, (int)dim, ks, d_out);
    return launch_status();
}

int dlrm_interaction_bwd(const float* d_dense, const float* d_pooled, const float* d_dout, int64_t batch,
                         int32_t n_tables, int32_t dim, float* d_ddense, float* d_dpooled, void* stream) {
    size_t lf = 0, lb = 0;
    int rc = check_shape(batch, n_tables, dim, &lf, &lb);
    if (rc) return rc;
    if (batch == 0) return RSE_OK;
    if (!d_dense || !d_pooled || !d_dout || !d_ddense || !d_dpooled) return RSE_ERR_INVALID_ARG;
    if (mf_ok(n_tables, dim)) {
        const int F = n_tables + 1;
        const size_t per_wave = ((size_t)F * (dim + 4) + MF_MAX_P + (size_t)MF_MAX_F * MF_GS) * sizeof(float);
        const int W = mf_waves(per_wave);
        const dim3 grid(fill_blocks(batch, W, 256 * 8)), block(W * WAVE);
        const size_t lds = per_wave * W;
        hipStream_t st = as_stream(stream);
        switch (dim) {
            case 32: hipLaunchKernelGGL(k_dot_bwd_mfma<32>, grid, block, lds, st, d_dense, d_pooled, d_dout, batch, (int)n_tables, d_ddense, d_dpooled); break;
            case 64: hipLaunchKernelGGL(k_dot_bwd_mfma<64>, grid, block, lds, st, d_dense, d_pooled, d_dout, batch, (int)n_tables, d_ddense, d_dpooled); break;
            default: hipLaunchKernelGGL(k_dot_bwd_mfma<128>, grid, block, lds, st, d_dense, d_pooled, d_dout, batch, (int)n_tables, d_ddense, d_dpooled); break;
        }
        return launch_status();
    }
    hipLaunchKernelGGL(k_dot_bwd, dim3(grid_for(batch)), dim3(IB), lb, as_stream(stream), d_dense, d_pooled, d_dout,
                       batch, (int)n_tables, (int)dim, d_ddense, d_dpooled);
    return launch_status();
}

}  // extern "C"
