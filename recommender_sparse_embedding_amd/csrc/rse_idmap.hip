// rse_idmap.hip -- IDMap: feature ID -> row offset ("RecIS：阿里开源推荐系统统一
// 训练框架", "Embedding Engine": the first level of the two-level table;
// "阿里 RecIS：搜广推训练的背景与难点": raw IDs over a huge sparse range need
// a map, not a dense or modulo-indexed table).
//
// Layout: per table a region of 16-byte slots {key, value} in buckets of 8
// slots (128 bytes, one cache line).  A bucket is read by 8 lanes of a
// wavefront with one 16-byte load each and compared by ballot; a 64-lane
// wave takes 64 lookups at a time and has the first buckets of all of them
// in flight together.  Buckets are probed linearly from the bucket chosen by
// a salted 64-bit mix.
//
// find_or_insert runs as a fixed chain of kernels on one stream:
//   reset -> probe (hits resolved; misses CAS-claim a slot and record their
//   lookup index as a pending value with atomicMin, so the slot ends up
//   holding the FIRST lookup of that key) -> mark first-sight lookups and
//   count them per tile of lookups -> decide (capacity / load checks and the
//   scan of the tile counts, single block) -> rank each tile's first sights
//   in lookup order and commit them (or roll back every pending slot) ->
//   resolve pending lookups and initialise new rows.
// New offsets are therefore rows_used + rank, identical to inserting the
// keys one by one in lookup order, and independent of thread timing.  Only
// integer atomics are used.  Kernels after the probe exit at once when the
// batch has no miss.
#include <mutex>
#include <new>

#include "rse_host.h"

using namespace rse;
using namespace rse_host;

rse::Slot* rse_idmap::d_slots() const {
    return reinterpret_cast<rse::Slot*>(
        d_mem + align_up(sizeof(MapHeader) + (size_t)n_tables * sizeof(TableDir), 256));
}

namespace {

constexpr int PROBE_BLOCK = 256;
constexpr int SCAN_TILE = 4096;          // lookups per scan block (256 x 16)
constexpr uint32_t SIDE_MARK = 0xFFFFFFFFu;   // slot index meaning "side slot"

// Workspace of one call.
struct Ws {
    unsigned long long* ctr;   // [0] misses [1] overflow [2] bad input [3] ok
                               // [4] rows_used before [5] new keys [6] status code
    uint32_t* miss_list;       // lookup indices that missed (any order)
    uint32_t* slot_of;         // per lookup: claimed slot (SIDE_MARK for the side slot)
    uint32_t* flag;            // per lookup: 0 hit, 1 pending, 2 first sight
    uint32_t* tile_sum;        // per scan tile
    uint64_t* new_key;         // per new row (by rank): key
    uint32_t* new_tab;         // per new row: table index used by the init
};

Ws carve(void* base, int64_t n_ids, size_t* total) {
    Carver c(base);
    Ws w;
    const size_t n = (size_t)(n_ids > 0 ? n_ids : 1);
    const size_t tiles = (n + SCAN_TILE - 1) / SCAN_TILE;
    w.ctr = c.take<unsigned long long>(32);
    w.miss_list = c.take<uint32_t>(n);
    w.slot_of = c.take<uint32_t>(n);
    w.flag = c.take<uint32_t>(n);
    w.tile_sum = c.take<uint32_t>(tiles + 1);
    w.new_key = c.take<uint64_t>(n);
    w.new_tab = c.take<uint32_t>(n);
    if (total) *total = c.size();
    return w;
}

struct ProbeArgs {
    Slot* slots;
    TableDir* dir;
    const int64_t* ids;
    int64_t n_ids;
    const int64_t* bounds;
    int64_t stride;
    int32_t n_tables;       // logical tables of the call
    int32_t merged;
    int32_t insert;
    int32_t pad;
    int64_t* row_off;
    Ws ws;
};

// -------------------------------------------------------------- reset ----
__global__ void k_reset(Ws ws, TableDir* dir, int32_t n_regions, int64_t n_tiles) {
    const int tid = threadIdx.x;
    if (tid < 32) ws.ctr[tid] = 0;
    for (int r = tid; r < n_regions; r += blockDim.x) dir[r].new_keys = 0;
    for (int64_t k = tid; k <= n_tiles; k += blockDim.x) ws.tile_sum[k] = 0;
}

// Table of lookup i: the t with bounds[t] <= i < bounds[t+1] (bounds in LDS,
// possibly with empty tables).
__device__ __forceinline__ int table_of(const int64_t* sb, int n_tables, int64_t i) {
    int lo = 0, hi = n_tables;            // invariant: sb[lo] <= i < sb[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sb[mid] <= i) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Loads the table bounds into LDS and checks them (same verdict in every
// block).  Returns false if malformed.
__device__ bool load_bounds(int64_t* sb, const int64_t* bounds, int64_t stride, int n_tables,
                            int64_t n_ids) {
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    for (int t = threadIdx.x; t <= n_tables; t += blockDim.x) {
        sb[t] = bounds[(int64_t)t * stride];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < n_tables; t += blockDim.x)
        if (sb[t + 1] < sb[t]) s_bad = 1;
    if (threadIdx.x == 0 && (sb[0] != 0 || sb[n_tables] != n_ids)) s_bad = 1;
    __syncthreads();
    return s_bad == 0;
}

// -------------------------------------------------------------- probe ----
// Results of the first-bucket pass, one per lookup: a value below
// PENDING_BASE is the row offset found, the codes below are the rest.
constexpr uint64_t RES_SLOW = ~0ull;          // needs the full probe
constexpr uint64_t RES_ABSENT = ~0ull - 1;    // not in the map, nothing inserted
constexpr uint64_t RES_BAD = ~0ull - 2;       // id out of range (merged mode)
constexpr uint64_t RES_NONE = ~0ull - 3;      // lane past the end of the batch

// Full probe of one lookup by the 8 lanes of a group: kind 0 hit, 1 pending
// (a miss, inserted), 2 absent, 3 overflow.  `side`: the key is the empty
// marker itself, kept in a per-table side slot.
__device__ __forceinline__ void probe_full(const ProbeArgs& a, int64_t i, uint64_t key, int region, bool side,
                                           int sub, int gshift, int& kind, uint64_t& val, uint32_t& slot_idx) {
    kind = 2;
    val = 0;
    slot_idx = 0;
    if (side) {
        const uint64_t v = a.dir[region].side_val;
        if (v < PENDING_BASE) {
            kind = 0;
            val = v;
        } else if (a.insert) {
            if (sub == 0) atomicMin((unsigned long long*)&a.dir[region].side_val,
                                    (unsigned long long)(PENDING_BASE + (uint64_t)i));
            kind = 1;
            slot_idx = SIDE_MARK;
        }
        return;
    }
    const TableDir d = a.dir[region];
    int64_t b = reduce_range(fmix64(key ^ d.salt), d.n_buckets);
    int64_t probes = 0;
    while (true) {
        const int64_t sidx = d.slot_base + b * BUCKET;
        const Slot s = a.slots[sidx + sub];
        const uint32_t m = (uint32_t)(__ballot(s.key == key) >> gshift) & 0xFFu;
        if (m) {
            const int src = __ffs(m) - 1;
            const uint64_t v = shfl_idx(s.val, gshift + src);
            if (v < PENDING_BASE) {
                kind = 0;
                val = v;
            } else {
                // inserted by another lookup of this batch: join it
                if (sub == 0)
                    atomicMin((unsigned long long*)&a.slots[sidx + src].val,
                              (unsigned long long)(PENDING_BASE + (uint64_t)i));
                kind = 1;
                slot_idx = (uint32_t)(sidx + src);
            }
            return;
        }
        const uint32_t e = (uint32_t)(__ballot(s.key == EMPTY_KEY) >> gshift) & 0xFFu;
        if (e) {
            if (!a.insert) return;
            // Claim the first truly empty slot of the bucket, in slot order.
            // A slot never returns to empty within the call, so slots seen as
            // non-empty are skipped safely; a CAS that returns our key means
            // another lookup got there first.
            int claimed = -1;
            if (sub == 0) {
                uint32_t rem = e;
                while (rem) {
                    const int q = __ffs(rem) - 1;
                    rem &= rem - 1;
                    const unsigned long long old = atomicCAS((unsigned long long*)&a.slots[sidx + q].key,
                                                             (unsigned long long)EMPTY_KEY, (unsigned long long)key);
                    if (old == EMPTY_KEY || old == key) {
                        atomicMin((unsigned long long*)&a.slots[sidx + q].val,
                                  (unsigned long long)(PENDING_BASE + (uint64_t)i));
                        claimed = q;
                        break;
                    }
                }
            }
            claimed = shfl_idx(claimed, gshift);
            if (claimed >= 0) {
                kind = 1;
                slot_idx = (uint32_t)(sidx + claimed);
                return;
            }
            // bucket filled up meanwhile: continue with the next one
        }
        if (++probes >= d.n_buckets) {
            kind = 3;
            return;
        }
        b = (b + 1 == d.n_buckets) ? 0 : b + 1;
    }
}

// 64 lookups per wave per iteration.  (1) One lane per lookup: id, table,
// key and first bucket.  (2) Eight lanes per lookup: the first buckets of all
// 64 lookups are loaded together (eight rounds, one 16-byte slot per lane per
// round, all in flight at once) and matched; a committed key found there, or
// a key found absent when nothing is inserted, is settled and written one
// lane per lookup.  (3) The rest (keys being inserted or joined, keys further
// along their chain, the empty-marker key) take the full probe, eight at a
// time.  Most lookups of a steady-state batch are settled by (2), which costs
// three dependent memory round trips per 64 lookups.
__global__ __launch_bounds__(PROBE_BLOCK) void k_probe(ProbeArgs a) {
    latency_bound_priority();
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    const bool ok_bounds = load_bounds(sb, a.bounds, a.stride, a.n_tables, a.n_ids);
    if (!ok_bounds) {
        if (blockIdx.x == 0 && threadIdx.x == 0) a.ws.ctr[2] = 1;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n_ids;
             i += (int64_t)gridDim.x * blockDim.x) {
            a.row_off[i] = -1;
            a.ws.flag[i] = 0;
        }
        return;
    }
    const int lane = lane_id();
    const int g = lane >> 3;           // group within the wave
    const int sub = lane & 7;          // slot within the bucket
    const int gshift = g * 8;
    const int64_t wave_global = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;

    for (int64_t base = wave_global * WAVE; base < a.n_ids; base += n_waves * WAVE) {
        // (1) lanes past the end repeat the last lookup's reads, so that every
        // load is issued unconditionally
        const int64_t i = base + lane;
        const bool active = i < a.n_ids;
        const int64_t ic = active ? i : a.n_ids - 1;
        const int t = table_of(sb, a.n_tables, ic);
        uint64_t key = (uint64_t)a.ids[ic];
        int region = t;
        uint64_t res = RES_SLOW;
        if (a.merged) {
            if (key >= (1ull << 56)) res = RES_BAD;   // also rejects negative ids
            key = ((uint64_t)t << 56) | key;
            region = 0;
        }
        const RSE_GLOBAL TableDir* dp = (const RSE_GLOBAL TableDir*)(a.dir + region);
        const int64_t slot_base = dp->slot_base;
        const int64_t n_buckets = dp->n_buckets;
        const uint64_t salt = dp->salt;
        const bool first = active && res == RES_SLOW && key != EMPTY_KEY;
        const int64_t sidx0 = first ? slot_base + reduce_range(fmix64(key ^ salt), n_buckets) * BUCKET : 0;
        if (!active) res = RES_NONE;

        // (2) round r: group g reads the first bucket of lookup 8r + g
        u32x4 pre[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t sidx = shfl_idx(sidx0, r * 8 + g);
            pre[r] = gload_u4(a.slots + sidx + sub);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int src = r * 8 + g;
            const uint64_t key_r = shfl_idx(key, src);
            const uint64_t sk = ((uint64_t)pre[r].y << 32) | pre[r].x;
            const uint64_t sv = ((uint64_t)pre[r].w << 32) | pre[r].z;
            const uint32_t m = (uint32_t)(__ballot(sk == key_r) >> gshift) & 0xFFu;
            const uint32_t e = (uint32_t)(__ballot(sk == EMPTY_KEY) >> gshift) & 0xFFu;
            const uint64_t v = shfl_idx(sv, gshift + (m ? __ffs(m) - 1 : 0));
            uint64_t rg = RES_SLOW;
            if (m) {
                if (v < PENDING_BASE) rg = v;
            } else if (e && !a.insert) {
                rg = RES_ABSENT;
            }
            // back to one lane per lookup: lane 8r + g' takes group g''s result
            const uint64_t mine = shfl_idx(rg, (lane & 7) * 8);
            if ((lane >> 3) == r && first) res = mine;
        }
        if (res != RES_SLOW && res != RES_NONE) {
            a.row_off[i] = res < PENDING_BASE ? (int64_t)res : -1;
            a.ws.flag[i] = 0;
            if (res == RES_BAD) a.ws.ctr[2] = 1;
        }

        // (3) the full probe for the rest: group g takes the g-th lowest
        uint64_t slow = __ballot(res == RES_SLOW);
        while (slow) {
            uint64_t mg = slow;
            for (int k = 0; k < g; ++k) mg &= mg - 1;
            const bool has = mg != 0;
            const int src = has ? __ffsll((long long)mg) - 1 : 0;
            for (int k = 0; k < 8; ++k) slow &= slow - 1;
            const uint64_t key_r = shfl_idx(key, src);
            const int region_r = shfl_idx(region, src);
            const int64_t ir = base + src;
            int kind = 2;
            uint64_t val = 0;
            uint32_t slot_idx = 0;
            if (has) probe_full(a, ir, key_r, region_r, key_r == EMPTY_KEY, sub, gshift, kind, val, slot_idx);
            // write results (one lane per group) and append misses to the list
            const bool leader = has && sub == 0;
            const bool is_miss = leader && kind == 1;
            const unsigned long long mm = __ballot(is_miss);
            unsigned long long pos0 = 0;
            if (mm) {
                if (lane == __ffsll((long long)mm) - 1)
                    pos0 = atomicAdd(&a.ws.ctr[0], (unsigned long long)__popcll(mm));
                pos0 = __shfl(pos0, __ffsll((long long)mm) - 1, WAVE);
            }
            if (leader) {
                if (kind == 0) {
                    a.row_off[ir] = (int64_t)val;
                    a.ws.flag[ir] = 0;
                } else if (kind == 1) {
                    const unsigned long long below = mm & ((1ull << lane) - 1);
                    a.ws.miss_list[pos0 + __popcll(below)] = (uint32_t)ir;
                    a.ws.slot_of[ir] = slot_idx;
                    a.ws.flag[ir] = 1;
                    a.row_off[ir] = -1;
                } else {
                    a.row_off[ir] = -1;
                    a.ws.flag[ir] = 0;
                    if (kind == 3) a.ws.ctr[1] = 1;
                }
            }
        }
    }
}

// ----------------------------------------------------------- mark heads --
__device__ __forceinline__ int region_of_slot(const TableDir* dir, int n_regions, uint32_t s) {
    int lo = 0, hi = n_regions;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((uint64_t)dir[mid].slot_base <= s) lo = mid;
        else hi = mid;
    }
    return lo;
}

struct MarkArgs {
    Slot* slots;
    TableDir* dir;
    int32_t n_regions;
    int32_t merged;
    const int64_t* ids;
    const int64_t* bounds;
    int64_t stride;
    int32_t n_tables;
    int32_t pad;
    Ws ws;
};

// A pending lookup is the first sight of its key iff the slot's pending value
// names it.  First sights are counted per region for the load check, and per
// tile of SCAN_TILE lookups for the ranks (one atomic add per tile per wave:
// a wave's entries of the miss list come from few tiles).
__global__ void k_mark(MarkArgs a) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    __shared__ uint32_t s_new[RSE_MAX_TABLES];   // per-region first sights of this block
    const unsigned long long n_miss = a.ws.ctr[0];
    if (n_miss == 0) return;
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x) s_new[r] = 0;
    __syncthreads();
    for (unsigned long long q = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; q < n_miss;
         q += (unsigned long long)gridDim.x * blockDim.x) {
        const uint32_t i = a.ws.miss_list[q];
        const uint32_t s = a.ws.slot_of[i];
        int region;
        uint64_t v;
        if (s == SIDE_MARK) {
            region = a.merged ? 0 : table_of(sb, a.n_tables, i);
            v = a.dir[region].side_val;
        } else {
            region = region_of_slot(a.dir, a.n_regions, s);
            v = a.slots[s].val;
        }
        const bool first = v == PENDING_BASE + (uint64_t)i;
        if (first) {
            a.ws.flag[i] = 2;
            atomicAdd(&s_new[region], 1u);
        }
        const uint32_t tile = i / SCAN_TILE;
        unsigned long long pend = __ballot(first);
        while (pend) {
            const int src = __ffsll((long long)pend) - 1;
            const uint32_t tl = __shfl(tile, src, WAVE);
            const unsigned long long same = __ballot(first && tile == tl) & pend;
            if (lane_id() == src) atomicAdd(&a.ws.tile_sum[tl], (uint32_t)__popcll(same));
            pend &= ~same;
        }
    }
    __syncthreads();
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x)
        if (s_new[r]) atomicAdd((unsigned long long*)&a.dir[r].new_keys, (unsigned long long)s_new[r]);
}

constexpr int DECIDE_BLOCK = 256;   // small, so that it finds room beside other streams' kernels

// Block-wide exclusive scan of DECIDE_BLOCK values (one per thread); returns
// the total.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* out_excl) {
    constexpr int NW = DECIDE_BLOCK / WAVE;
    __shared__ uint32_t wsum[NW];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    uint32_t x = v;
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) wsum[w] = x;
    __syncthreads();
    uint32_t wprefix = 0, total = 0;
    for (int k = 0; k < NW; ++k) {
        if (k < w) wprefix += wsum[k];
        total += wsum[k];
    }
    __syncthreads();
    *out_excl = wprefix + x - v;
    return total;
}

struct DecideArgs {
    TableDir* dir;
    int32_t n_regions;
    int32_t pad;
    BlocksHeader* bh;
    MapHeader* mh;
    int64_t capacity;
    int64_t* n_new_out;
    int64_t n_tiles;
    Ws ws;
};

// Single block: scans the tile sums, then decides whether the call commits
// and advances the counters.
__global__ __launch_bounds__(DECIDE_BLOCK) void k_decide(DecideArgs a) {
    __shared__ int s_fail;
    __shared__ uint32_t s_carry;
    const bool any_miss = a.ws.ctr[0] != 0;
    uint32_t total = 0;
    if (any_miss) {
        if (threadIdx.x == 0) s_carry = 0;
        __syncthreads();
        for (int64_t base = 0; base < a.n_tiles; base += DECIDE_BLOCK) {
            const int64_t k = base + threadIdx.x;
            const uint32_t v = k < a.n_tiles ? a.ws.tile_sum[k] : 0;
            uint32_t ex;
            const uint32_t t = block_exclusive_scan(v, &ex);
            const uint32_t carry = s_carry;
            if (k < a.n_tiles) a.ws.tile_sum[k] = carry + ex;
            __syncthreads();
            if (threadIdx.x == 0) s_carry = carry + t;
            __syncthreads();
        }
        total = s_carry;
    }
    if (threadIdx.x == 0) s_fail = 0;
    __syncthreads();
    // per-region load check
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x) {
        const TableDir d = a.dir[r];
        if (d.n_keys + d.new_keys > d.max_keys) atomicCAS(&s_fail, 0, (int)RSE_ERR_IDMAP_FULL);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int fail = 0;
        if (a.ws.ctr[2]) fail = RSE_ERR_BAD_INPUT;
        else if (a.ws.ctr[1] || s_fail) fail = RSE_ERR_IDMAP_FULL;
        const int64_t used = a.bh->rows_used;
        if (!fail && used + (int64_t)total > a.capacity) fail = RSE_ERR_NEED_GROW;
        a.ws.ctr[4] = (unsigned long long)used;
        a.ws.ctr[5] = total;
        if (!fail) {
            a.ws.ctr[3] = 1;
            a.bh->rows_used = used + (int64_t)total;
            *a.n_new_out = (int64_t)total;
        } else {
            a.ws.ctr[3] = 0;
            *a.n_new_out = 0;
            atomicCAS(&a.mh->status, 0, fail);
        }
    }
    __syncthreads();
    if (a.ws.ctr[3]) {
        for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x) {
            a.dir[r].n_keys += a.dir[r].new_keys;
        }
    }
}

// --------------------------------------------------- rank and commit ----
struct CommitArgs {
    Slot* slots;
    TableDir* dir;
    int32_t n_regions;
    int32_t merged;
    const int64_t* ids;
    const int64_t* bounds;
    int64_t stride;
    int32_t n_tables;
    int32_t pad;
    int64_t n;
    Ws ws;
};

// One block per tile of SCAN_TILE lookups (16 per thread).  If the call
// commits, the tile's first sights get their ranks (the tile's prefix from
// k_decide plus a block scan, i.e. the exclusive scan over all lookups) and
// publish offset rows_used + rank into their slot; otherwise they release
// their slot.
__global__ __launch_bounds__(256) void k_rank_commit(CommitArgs a) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    __shared__ uint32_t wsum[4];
    if (a.ws.ctr[0] == 0) return;
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    const bool ok = a.ws.ctr[3] != 0;
    const uint64_t used = a.ws.ctr[4];
    const int64_t i0 = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * 16;
    uint32_t f[16];
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t i = i0 + k;
        f[k] = (i < a.n && a.ws.flag[i] == 2) ? 1u : 0u;
        c += f[k];
    }
    // block exclusive scan of c (256 threads); the barrier also covers sb
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    uint32_t x = c;
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) wsum[w] = x;
    __syncthreads();
    uint32_t pre = a.ws.tile_sum[blockIdx.x];
    for (int k = 0; k < w; ++k) pre += wsum[k];
    uint32_t rk = pre + x - c;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (!f[k]) continue;
        const int64_t i = i0 + k;
        const uint32_t s = a.ws.slot_of[i];
        const int t = table_of(sb, a.n_tables, i);
        const int region = a.merged ? 0 : t;
        if (ok) {
            const uint64_t off = used + rk;
            uint64_t key = (uint64_t)a.ids[i];
            if (a.merged) key = ((uint64_t)t << 56) | key;
            if (s == SIDE_MARK) a.dir[region].side_val = off;
            else a.slots[s].val = off;
            a.ws.new_key[rk] = key;
            a.ws.new_tab[rk] = (uint32_t)region;
        } else if (s == SIDE_MARK) {
            a.dir[region].side_val = EMPTY_VAL;
        } else {
            a.slots[s].key = EMPTY_KEY;
            a.slots[s].val = EMPTY_VAL;
        }
        ++rk;
    }
}

// ------------------------------------------------- resolve and init -----
struct FinishArgs {
    Slot* slots;
    TableDir* dir;
    int32_t merged;
    int32_t n_tables;
    const int64_t* bounds;
    int64_t stride;
    int64_t* row_off;
    RowsView rv;
    int64_t row_bytes;
    uint64_t seed;
    int32_t dim;
    int32_t pad;
    Ws ws;
};

// One grid-stride range over two kinds of items: first every pending lookup
// (it reads its key's final offset, or -1 if the call did not commit), then
// every 16 bytes of the new rows (weights from the key hash, state zero;
// rows are consecutive so the writes are contiguous).
template <bool BF16>
__global__ void k_finish(FinishArgs a) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    const uint64_t n_miss = a.ws.ctr[0];
    if (n_miss == 0) return;
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    __syncthreads();
    const bool ok = a.ws.ctr[3] != 0;
    const uint64_t n_new = ok ? a.ws.ctr[5] : 0;
    const uint64_t used = a.ws.ctr[4];
    const int64_t q_per_row = a.row_bytes / 16;
    const int64_t w_q = (int64_t)a.dim * (BF16 ? 2 : 4) / 16;   // 16-byte units of weights
    const int per_q = BF16 ? 8 : 4;
    const uint64_t total = n_miss + n_new * (uint64_t)q_per_row;
    for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (uint64_t)gridDim.x * blockDim.x) {
        if (e < n_miss) {
            const uint32_t i = a.ws.miss_list[e];
            int64_t v = -1;
            if (ok) {
                const uint32_t s = a.ws.slot_of[i];
                if (s == SIDE_MARK) {
                    const int region = a.merged ? 0 : table_of(sb, a.n_tables, i);
                    v = (int64_t)a.dir[region].side_val;
                } else {
                    v = (int64_t)a.slots[s].val;
                }
            }
            a.row_off[i] = v;
            continue;
        }
        const uint64_t ee = e - n_miss;
        const uint64_t r = ee / (uint64_t)q_per_row;
        const int64_t qi = (int64_t)(ee - r * (uint64_t)q_per_row);
        char* row = a.rv.row((int64_t)(used + r));
        u32x4 out = u32x4{0u, 0u, 0u, 0u};
        if (qi < w_q) {
            const uint64_t key = a.ws.new_key[r];
            const uint32_t tab = a.ws.new_tab[r];
            uint32_t wv[4];
            if (!BF16) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    wv[k] = __float_as_uint(init_value(key, tab, (int)(qi * per_q + k), a.seed, false));
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = f32_to_bf16_exact(init_value(key, tab, (int)(qi * per_q + 2 * k), a.seed, true));
                    const uint32_t hi = f32_to_bf16_exact(init_value(key, tab, (int)(qi * per_q + 2 * k + 1), a.seed, true));
                    wv[k] = lo | (hi << 16);
                }
            }
            out = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
        gstore_u4(row + (int64_t)qi * 16, out);
    }
}

// ------------------------------------------------------------ create -----
__global__ void k_clear_slots(Slot* slots, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        slots[i].key = EMPTY_KEY;
        slots[i].val = EMPTY_VAL;
    }
}

__global__ void k_clear_header(MapHeader* h, int32_t n_tables, int32_t merged) {
    if (threadIdx.x == 0) {
        h->status = 0;
        h->n_tables = n_tables;
        h->merged = merged;
    }
}

__global__ void k_clear_status(MapHeader* h) { h->status = 0; }

// ------------------------------------------------------------ export -----
__global__ void k_export(const Slot* slots, const TableDir* dir, int32_t n_regions, int64_t total_slots,
                         int64_t* keys, int32_t* tabs, int64_t* offs, int64_t capacity,
                         unsigned long long* count) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t s = tid; s < total_slots; s += stride) {
        const Slot sl = slots[s];
        if (sl.key == EMPTY_KEY) continue;
        const unsigned long long p = atomicAdd(count, 1ull);
        if ((int64_t)p < capacity) {
            keys[p] = (int64_t)sl.key;
            tabs[p] = region_of_slot(dir, n_regions, (uint32_t)s);
            offs[p] = (int64_t)sl.val;
        }
    }
    for (int64_t r = tid; r < n_regions; r += stride) {
        const uint64_t v = dir[r].side_val;
        if (v >= PENDING_BASE) continue;
        const unsigned long long p = atomicAdd(count, 1ull);
        if ((int64_t)p < capacity) {
            keys[p] = (int64_t)EMPTY_KEY;
            tabs[p] = (int32_t)r;
            offs[p] = (int64_t)v;
        }
    }
}

__global__ void k_zero_u64(unsigned long long* p) { *p = 0; }

// ------------------------------------------------------------ import -----
// Entries (key, region, offset) of a saved map, in three kernels: count the
// entries per region (and reject a bad region or offset), decide whether
// every region stays within its load limit, then insert (one thread per
// entry, probing from its bucket and claiming an empty slot by CAS).  The
// set of entries decides the map's contents; the slot each key lands in may
// depend on timing, which nothing observes.
__global__ void k_import_reset(TableDir* dir, int32_t n_regions, MapHeader* h) {
    for (int r = threadIdx.x; r < n_regions; r += blockDim.x) dir[r].new_keys = 0;
    if (threadIdx.x == 0) h->pad[0] = 0;
}

__global__ void k_import_count(TableDir* dir, int32_t n_regions, const int32_t* tabs, const int64_t* offs,
                               int64_t n, MapHeader* h) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t r = tabs[i];
        if (r < 0 || r >= n_regions || offs[i] < 0 || (uint64_t)offs[i] >= PENDING_BASE) {
            atomicCAS(&h->status, 0, (int32_t)RSE_ERR_BAD_INPUT);
            continue;
        }
        atomicAdd((unsigned long long*)&dir[r].new_keys, 1ull);
    }
}

__global__ void k_import_decide(TableDir* dir, int32_t n_regions, MapHeader* h) {
    __shared__ int s_fail;
    if (threadIdx.x == 0) s_fail = h->status;
    __syncthreads();
    for (int r = threadIdx.x; r < n_regions; r += blockDim.x)
        if (dir[r].n_keys + dir[r].new_keys > dir[r].max_keys) atomicCAS(&s_fail, 0, (int)RSE_ERR_IDMAP_FULL);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (s_fail) atomicCAS(&h->status, 0, s_fail);
        h->pad[0] = s_fail ? 0 : 1;        // go flag for k_import_insert
    }
    __syncthreads();
    if (!s_fail)
        for (int r = threadIdx.x; r < n_regions; r += blockDim.x) dir[r].n_keys += dir[r].new_keys;
}

__global__ void k_import_insert(Slot* slots, TableDir* dir, const int64_t* keys, const int32_t* tabs,
                                const int64_t* offs, int64_t n, MapHeader* h) {
    if (h->pad[0] != 1) return;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t key = (uint64_t)keys[i];
        const TableDir d = dir[tabs[i]];
        const uint64_t off = (uint64_t)offs[i];
        if (key == EMPTY_KEY) {
            const unsigned long long old = atomicCAS((unsigned long long*)&dir[tabs[i]].side_val,
                                                     (unsigned long long)EMPTY_VAL, (unsigned long long)off);
            if (old != EMPTY_VAL) atomicCAS(&h->status, 0, (int32_t)RSE_ERR_BAD_INPUT);   // duplicate key
            continue;
        }
        int64_t b = reduce_range(fmix64(key ^ d.salt), d.n_buckets);
        bool done = false;
        for (int64_t probes = 0; probes < d.n_buckets && !done; ++probes) {
            const int64_t base = d.slot_base + b * BUCKET;
            for (int q = 0; q < BUCKET && !done; ++q) {
                const uint64_t k = slots[base + q].key;
                if (k == key) {                       // duplicate key
                    atomicCAS(&h->status, 0, (int32_t)RSE_ERR_BAD_INPUT);
                    done = true;
                } else if (k == EMPTY_KEY) {
                    const unsigned long long old = atomicCAS((unsigned long long*)&slots[base + q].key,
                                                             (unsigned long long)EMPTY_KEY, (unsigned long long)key);
                    if (old == EMPTY_KEY) {
                        slots[base + q].val = off;
                        done = true;
                    } else if (old == key) {
                        atomicCAS(&h->status, 0, (int32_t)RSE_ERR_BAD_INPUT);
                        done = true;
                    }
                }
            }
            b = (b + 1 == d.n_buckets) ? 0 : b + 1;
        }
        if (!done) atomicCAS(&h->status, 0, (int32_t)RSE_ERR_IDMAP_FULL);
    }
}

}  // namespace

extern "C" {

int rse_idmap_mem_size(int32_t n_tables, const int64_t* slots_per_table, size_t* bytes_out) {
    if (!bytes_out || !slots_per_table || n_tables <= 0 || n_tables > RSE_MAX_TABLES)
        return RSE_ERR_INVALID_ARG;
    int64_t total = 0;
    for (int t = 0; t < n_tables; ++t) {
        if (slots_per_table[t] <= 0) return RSE_ERR_INVALID_ARG;
        total += (int64_t)align_up((size_t)slots_per_table[t], BUCKET);
    }
    if (total > (int64_t)0xFFFFF000ll) return RSE_ERR_INVALID_ARG;   // slot index fits 32 bits
    *bytes_out = align_up(sizeof(MapHeader) + (size_t)n_tables * sizeof(TableDir), 256) +
                 (size_t)total * sizeof(Slot);
    return RSE_OK;
}

int rse_idmap_create(rse_idmap** out, void* d_mem, size_t mem_bytes, int32_t n_tables,
                     const int64_t* slots_per_table, double max_load, int32_t merged,
                     uint64_t hash_seed, void* stream) {
    if (!out || !d_mem) return RSE_ERR_INVALID_ARG;
    if (!(max_load > 0.0 && max_load <= 0.95)) return RSE_ERR_INVALID_ARG;
    if (merged && n_tables != 1) return RSE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(d_mem) % 256) return RSE_ERR_INVALID_ARG;
    size_t need = 0;
    int rc = rse_idmap_mem_size(n_tables, slots_per_table, &need);
    if (rc) return rc;
    if (mem_bytes < need) return RSE_ERR_WORKSPACE;
    rse_idmap* m = new (std::nothrow) rse_idmap();
    if (!m) return RSE_ERR_INVALID_ARG;
    m->n_tables = n_tables;
    m->merged = merged ? 1 : 0;
    m->max_load = max_load;
    m->d_mem = static_cast<char*>(d_mem);
    m->dir.resize(n_tables);
    int64_t base = 0;
    uint64_t sm = hash_seed;
    for (int t = 0; t < n_tables; ++t) {
        const int64_t slots = (int64_t)align_up((size_t)slots_per_table[t], BUCKET);
        TableDir& d = m->dir[t];
        d.slot_base = base;
        d.n_buckets = slots / BUCKET;
        d.max_keys = (int64_t)(max_load * (double)slots);
        // per-table salt: successive SplitMix64 outputs of the seed
        sm += SM64_GAMMA;
        uint64_t z = sm;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        d.salt = z ^ (z >> 31);
        d.n_keys = 0;
        d.side_val = EMPTY_VAL;
        d.new_keys = 0;
        d.pad = 0;
        base += slots;
    }
    m->total_slots = base;
    hipStream_t s = as_stream(stream);
    if (hipMemcpyAsync(m->d_dir(), m->dir.data(), sizeof(TableDir) * n_tables, hipMemcpyHostToDevice,
                       s) != hipSuccess) {
        delete m;
        return RSE_ERR_HIP;
    }
    hipLaunchKernelGGL(k_clear_header, dim3(1), dim3(64), 0, s, m->header(), n_tables, m->merged);
    hipLaunchKernelGGL(k_clear_slots, dim3(fill_blocks(base, 256, 8192)), dim3(256), 0, s, m->d_slots(),
                       base);
    rc = launch_status();
    if (rc) {
        delete m;
        return rc;
    }
    // the host copy of the directory is the source of an async copy: keep it
    // alive by keeping the handle; make sure it has landed before returning
    if (hipStreamSynchronize(s) != hipSuccess) {
        delete m;
        return RSE_ERR_HIP;
    }
    *out = m;
    return RSE_OK;
}

int rse_idmap_destroy(rse_idmap* map) {
    delete map;
    return RSE_OK;
}

int rse_idmap_workspace_size(int64_t n_ids, size_t* bytes_out) {
    if (!bytes_out || n_ids < 0) return RSE_ERR_INVALID_ARG;
    carve(nullptr, n_ids, bytes_out);
    return RSE_OK;
}

}  // extern "C"

namespace {

// The find-or-insert chain over a given workspace (caller memory or the
// library's static scratch).
int find_or_insert_impl(rse_idmap* map, rse_blocks* blocks, const int64_t* d_ids, int64_t n_ids,
                        const int64_t* d_bounds, int64_t stride, int32_t n_tables,
                        int32_t insert_missing, int64_t* d_row_off_out, int64_t* d_n_new_out,
                        void* d_ws, size_t ws_bytes, void* stream) {
    if (!map || !blocks || !d_bounds || !d_n_new_out || !d_ws) return RSE_ERR_INVALID_ARG;
    if (n_ids < 0 || stride <= 0 || n_tables <= 0) return RSE_ERR_INVALID_ARG;
    if (n_ids > 0 && (!d_ids || !d_row_off_out)) return RSE_ERR_INVALID_ARG;
    if (n_ids > (int64_t)0xFFFFFFFFll) return RSE_ERR_INVALID_ARG;
    if (map->merged) {
        if (n_tables > RSE_MAX_MERGED_TABLES) return RSE_ERR_INVALID_ARG;
    } else if (n_tables != map->n_tables) {
        return RSE_ERR_INVALID_ARG;
    }
    size_t need = 0;
    Ws ws = carve(d_ws, n_ids, &need);
    if (ws_bytes < need) return RSE_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);

    const int64_t n_tiles = (n_ids + SCAN_TILE - 1) / SCAN_TILE;
    hipLaunchKernelGGL(k_reset, dim3(1), dim3(256), 0, s, ws, map->d_dir(), map->n_tables, n_tiles);

    ProbeArgs pa;
    pa.slots = map->d_slots();
    pa.dir = map->d_dir();
    pa.ids = d_ids;
    pa.n_ids = n_ids;
    pa.bounds = d_bounds;
    pa.stride = stride;
    pa.n_tables = n_tables;
    pa.merged = map->merged;
    pa.insert = insert_missing ? 1 : 0;
    pa.pad = 0;
    pa.row_off = d_row_off_out;
    pa.ws = ws;
    // 64 lookups per wave per iteration; enough waves to fill 256 CUs
    const int probe_blocks = fill_blocks((n_ids + WAVE - 1) / WAVE, PROBE_BLOCK / 64, 256 * 16);
    {
        TraceScope ts(RSE_K_PROBE, s);
        hipLaunchKernelGGL(k_probe, dim3(probe_blocks), dim3(PROBE_BLOCK), 0, s, pa);
    }

    const int miss_blocks = fill_blocks(n_ids, 256, 2048);
    MarkArgs ma;
    ma.slots = pa.slots;
    ma.dir = pa.dir;
    ma.n_regions = map->n_tables;
    ma.merged = map->merged;
    ma.ids = d_ids;
    ma.bounds = d_bounds;
    ma.stride = stride;
    ma.n_tables = n_tables;
    ma.pad = 0;
    ma.ws = ws;
    hipLaunchKernelGGL(k_mark, dim3(miss_blocks), dim3(256), 0, s, ma);

    const dim3 tiles_grid((unsigned)(n_tiles > 0 ? n_tiles : 1));
    DecideArgs da;
    da.dir = pa.dir;
    da.n_regions = map->n_tables;
    da.pad = 0;
    da.bh = blocks->header();
    da.mh = map->header();
    da.capacity = blocks->capacity();
    da.n_new_out = d_n_new_out;
    da.n_tiles = n_tiles;
    da.ws = ws;
    hipLaunchKernelGGL(k_decide, dim3(1), dim3(DECIDE_BLOCK), 0, s, da);

    CommitArgs ca;
    ca.slots = pa.slots;
    ca.dir = pa.dir;
    ca.n_regions = map->n_tables;
    ca.merged = map->merged;
    ca.ids = d_ids;
    ca.bounds = d_bounds;
    ca.stride = stride;
    ca.n_tables = n_tables;
    ca.pad = 0;
    ca.n = n_ids;
    ca.ws = ws;
    hipLaunchKernelGGL(k_rank_commit, tiles_grid, dim3(256), 0, s, ca);

    FinishArgs fa;
    fa.slots = pa.slots;
    fa.dir = pa.dir;
    fa.merged = map->merged;
    fa.n_tables = n_tables;
    fa.bounds = d_bounds;
    fa.stride = stride;
    fa.row_off = d_row_off_out;
    fa.rv = blocks->view();
    fa.row_bytes = blocks->row_bytes;
    fa.seed = blocks->seed;
    fa.dim = blocks->dim;
    fa.pad = 0;
    fa.ws = ws;
    const int64_t finish_work = n_ids * (1 + blocks->row_bytes / 16);
    const dim3 finish_grid(fill_blocks(finish_work, 256, 8192));
    if (blocks->w_dtype == RSE_BF16)
        hipLaunchKernelGGL(k_finish<true>, finish_grid, dim3(256), 0, s, fa);
    else
        hipLaunchKernelGGL(k_finish<false>, finish_grid, dim3(256), 0, s, fa);
    return launch_status();
}

// ------------------------------------------------- allocation-free find --
// Scratch of idmap_find_or_insert_noalloc: one copy per GPU, allocated by
// the runtime when the library's code object is loaded on that GPU and held
// until the process ends.  Its size is the workspace of
// RSE_NOALLOC_MAX_IDS lookups (checked when a device is first used).
constexpr size_t NOALLOC_SCRATCH_BYTES = 52ull << 20;
__device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` per GPU

// Device address of the current GPU's scratch.  In host code `scratch` is a
// host-side stand-in, never a device address: kernels get this pointer.
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return RSE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        size_t need = 0;
        carve(nullptr, RSE_NOALLOC_MAX_IDS, &need);
        if (need > NOALLOC_SCRATCH_BYTES) return RSE_ERR_UNSUPPORTED;
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RSE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RSE_OK;
}

}  // namespace

extern "C" {

int idmap_find_or_insert(rse_idmap* map, rse_blocks* blocks, const int64_t* d_ids, int64_t n_ids,
                         const int64_t* d_bounds, int64_t stride, int32_t n_tables,
                         int32_t insert_missing, int64_t* d_row_off_out, int64_t* d_n_new_out,
                         void* d_ws, size_t ws_bytes, void* stream) {
    return find_or_insert_impl(map, blocks, d_ids, n_ids, d_bounds, stride, n_tables, insert_missing,
                               d_row_off_out, d_n_new_out, d_ws, ws_bytes, stream);
}

int idmap_find_or_insert_noalloc(rse_idmap* map, rse_blocks* blocks, const int64_t* d_ids, int64_t n_ids,
                                 const int64_t* d_bounds, int64_t stride, int32_t n_tables,
                                 int32_t insert_missing, int64_t* d_row_off_out, int64_t* d_n_new_out,
                                 void* stream) {
    if (!map || !blocks) return RSE_ERR_INVALID_ARG;
    if (n_ids > RSE_NOALLOC_MAX_IDS) return RSE_ERR_WORKSPACE;
    void* ws = nullptr;
    const int rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    // k_reset clears the scratch's counters and tile sums at the start of
    // every call; everything else is written before it is read
    return find_or_insert_impl(map, blocks, d_ids, n_ids, d_bounds, stride, n_tables, insert_missing,
                               d_row_off_out, d_n_new_out, ws, NOALLOC_SCRATCH_BYTES, stream);
}

int rse_idmap_import(rse_idmap* map, const int64_t* d_keys, const int32_t* d_tables, const int64_t* d_offs,
                     int64_t n, void* stream) {
    if (!map || n < 0) return RSE_ERR_INVALID_ARG;
    if (n > 0 && (!d_keys || !d_tables || !d_offs)) return RSE_ERR_INVALID_ARG;
    if (n == 0) return RSE_OK;
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(k_import_reset, dim3(1), dim3(256), 0, s, map->d_dir(), map->n_tables, map->header());
    const dim3 grid(fill_blocks(n, 256, 8192));
    hipLaunchKernelGGL(k_import_count, grid, dim3(256), 0, s, map->d_dir(), map->n_tables, d_tables, d_offs, n,
                       map->header());
    hipLaunchKernelGGL(k_import_decide, dim3(1), dim3(256), 0, s, map->d_dir(), map->n_tables, map->header());
    hipLaunchKernelGGL(k_import_insert, grid, dim3(256), 0, s, map->d_slots(), map->d_dir(), d_keys, d_tables,
                       d_offs, n, map->header());
    return launch_status();
}

int rse_idmap_status(rse_idmap* map, int32_t* status_out, int64_t* n_keys_out, void* stream) {
    if (!map) return RSE_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    MapHeader h;
    if (hipMemcpyAsync(&h, map->header(), sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess)
        return RSE_ERR_HIP;
    std::vector<TableDir> dir(map->n_tables);
    if (n_keys_out && hipMemcpyAsync(dir.data(), map->d_dir(), sizeof(TableDir) * map->n_tables,
                                     hipMemcpyDeviceToHost, s) != hipSuccess)
        return RSE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return RSE_ERR_HIP;
    if (status_out) *status_out = h.status;
    if (n_keys_out)
        for (int t = 0; t < map->n_tables; ++t) n_keys_out[t] = dir[t].n_keys;
    return RSE_OK;
}

int rse_idmap_clear_status(rse_idmap* map, void* stream) {
    if (!map) return RSE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(1), 0, as_stream(stream), map->header());
    return launch_status();
}

int rse_idmap_export(rse_idmap* map, int64_t* d_keys_out, int32_t* d_table_out, int64_t* d_off_out,
                     int64_t capacity, int64_t* d_count_out, void* stream) {
    if (!map || !d_count_out || capacity < 0) return RSE_ERR_INVALID_ARG;
    if (capacity > 0 && (!d_keys_out || !d_table_out || !d_off_out)) return RSE_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    unsigned long long* cnt = reinterpret_cast<unsigned long long*>(d_count_out);
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(1), 0, s, cnt);
    hipLaunchKernelGGL(k_export, dim3(fill_blocks(map->total_slots, 256, 8192)), dim3(256), 0, s,
                       map->d_slots(), map->d_dir(), map->n_tables, map->total_slots, d_keys_out,
                       d_table_out, d_off_out, capacity, cnt);
    return launch_status();
}

}  // extern "C"
