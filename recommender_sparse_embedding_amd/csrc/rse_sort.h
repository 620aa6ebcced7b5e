// rse_sort.h -- internal interface of the device radix sort.
#pragma once

#include "rse_host.h"

namespace rse_host {

// keys per sort tile (512 threads x 16; 90 KB of LDS per block).  Against
// 4096-key tiles a pass takes as long alone, but beside the other stream's
// kernels the merged-table step ran 3% faster (7.50 -> 7.26 ms) and the
// click-log step the same.
constexpr int SORT_TILE = 8192;
constexpr int SORT_MAX_PASSES = 4;   // 32-bit keys
constexpr int SORT_MAX_BINS = 512;   // digits of up to 9 bits
// The digit totals are kept in several copies that blocks of the pair
// kernel add to in turn (the totals are the sum over copies): a few hundred
// blocks adding to one word each would queue behind each other.
constexpr int SORT_TOTAL_COPIES = 8;
constexpr int64_t SORT_COPY_STRIDE = (int64_t)SORT_MAX_PASSES * SORT_MAX_BINS;

// Digit plan for keys of `bits` bits: passes of at most 9 bits each.
struct SortPlan {
    int passes;
    int width;                       // bits per digit (last pass may use fewer)
};
SortPlan sort_plan(int bits);

// Workspace bytes for sorting n pairs.
size_t sort_workspace(int64_t n, int64_t* n_tiles_out);

// Device pointers inside the sort workspace that the pair-building kernel
// fills before the passes: per-pass digit totals (SORT_TOTAL_COPIES copies
// of SORT_MAX_PASSES x SORT_MAX_BINS, must start at zero) and the look-back
// state (zeroed by the pair kernel).  `error` is nonzero if a pass failed or
// was skipped.
struct SortPrep {
    uint32_t* totals;        // [SORT_TOTAL_COPIES][SORT_MAX_PASSES][SORT_MAX_BINS]
    uint32_t* state;         // [SORT_MAX_PASSES][n_tiles][SORT_MAX_BINS]
    uint32_t* tile_ctr;      // [SORT_MAX_PASSES] dynamic tile counters
    uint32_t* error;         // look-back timeout flag
    int64_t state_words;     // words of `state` to zero
};
SortPrep sort_prep(void* ws, int64_t n);

// Whether radix_sort_pairs accepts n pairs of `bits`-bit keys (host only;
// callers check this before enqueueing anything).
bool sort_supported(int64_t n, int bits);

// Sorts the (key, value) pairs p0 (x = key, y = value) by the low `bits`
// bits of the key, stably, ping-ponging through p1; the result ends in p1 if
// *result_in_alt.  Requires the digit totals of every pass to be in
// prep.totals (summed over its copies) and the rest of prep to be zero (the
// caller's pair kernel does both).
int radix_sort_pairs(uint2* p0, uint2* p1, int64_t n, int bits, void* ws, bool* result_in_alt, hipStream_t s);

// Device helper for the pair kernel: adds key's digits of every pass to
// block-local histograms (LDS, [SORT_MAX_PASSES][SORT_MAX_BINS]).
__device__ __forceinline__ void sort_hist_add(uint32_t* lds_hist, uint32_t key, int passes, int width) {
    const uint32_t mask = (1u << width) - 1u;
    for (int p = 0; p < passes; ++p)
        atomicAdd(&lds_hist[p * SORT_MAX_BINS + ((key >> (p * width)) & mask)], 1u);
}

}  // namespace rse_host
