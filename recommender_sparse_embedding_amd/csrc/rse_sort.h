// rse_sort.h -- internal interface of the device radix sort.
#pragma once

#include "rse_host.h"

namespace rse_host {

constexpr int SORT_TILE = 4096;      // keys per sort block
constexpr int SORT_MAX_PASSES = 4;   // 32-bit keys

// Workspace bytes for sorting n pairs (hist + per-pass digit totals).
size_t sort_workspace(int64_t n, int64_t* n_tiles_out);

// Pointer to the per-pass digit totals inside the workspace (256 * 4 per
// pass); they must be zero before radix_sort_pairs runs.
uint32_t* sort_totals(void* ws, int64_t n);

int radix_sort_pairs(uint32_t* k0, uint32_t* v0, uint32_t* k1, uint32_t* v1, int64_t n, int bits,
                     void* ws, bool* result_in_alt, hipStream_t s);

}  // namespace rse_host
