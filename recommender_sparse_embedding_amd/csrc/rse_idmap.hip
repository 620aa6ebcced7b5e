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
#include <algorithm>
#include <mutex>
#include <new>

#include "rse_host.h"

using namespace rse;
using namespace rse_host;

rse::Slot* rse_idmap::d_slots() const {
    return reinterpret_cast<rse::Slot*>(
        d_mem + align_up(sizeof(MapHeader) + (size_t)n_tables * sizeof(TableDir), 256));
}

size_t rse_idmap::mem_bytes() const {
    return align_up(sizeof(MapHeader) + (size_t)n_tables * sizeof(TableDir), 256) +
           (size_t)total_slots * sizeof(Slot);
}

namespace {

constexpr int PROBE_BLOCK = 256;
constexpr int SCAN_TILE = 4096;          // lookups per scan block (256 x 16)
constexpr uint32_t SIDE_MARK = 0xFFFFFFFFu;   // slot index meaning "side slot"

// Workspace of one call.
struct Ws {
    unsigned long long* ctr;   // [0] any miss [1] overflow [2] bad input [3] ok
                               // [4] rows_used before [5] new keys [6] status code
                               // [7] free-list head before [8] rows taken from it
                               // [9] admission candidates [10] admitted lookups
    uint32_t* slot_of;         // per lookup: claimed slot (SIDE_MARK for the side slot)
    uint32_t* flag;            // per lookup: 0 hit, 1 pending, 2 first sight
    uint32_t* tile_sum;        // per scan tile
    uint64_t* new_key;         // per new row (by rank): key
    uint32_t* new_tab;         // per new row: table index used by the init
    // Admission lists, in memory that k_rank_commit fills only later: the
    // candidates (lookups of absent keys) over new_key, the admitted ones
    // over new_tab.
    uint32_t* cand;
    uint32_t* admitted;
};

Ws carve(void* base, int64_t n_ids, size_t* total) {
    Carver c(base);
    Ws w;
    const size_t n = (size_t)(n_ids > 0 ? n_ids : 1);
    const size_t tiles = (n + SCAN_TILE - 1) / SCAN_TILE;
    w.ctr = c.take<unsigned long long>(32);
    w.slot_of = c.take<uint32_t>(n);
    w.flag = c.take<uint32_t>(n);
    w.tile_sum = c.take<uint32_t>(tiles + 1);
    w.new_key = c.take<uint64_t>(n);
    w.new_tab = c.take<uint32_t>(n);
    w.cand = reinterpret_cast<uint32_t*>(w.new_key);
    w.admitted = w.new_tab;
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
    int32_t collect;        // list absent lookups as admission candidates
    int64_t* row_off;
    const uint32_t* list;   // probe only these lookups (with *list_n), or null: all
    const unsigned long long* list_n;
    uint32_t* stamps;       // per-row last-seen clock, or null
    int64_t n_stamps;
    uint32_t clock;
    int32_t pad2;
    Ws ws;
};

// Appends `value` for every lane with `me` set, one atomic per wave.
__device__ __forceinline__ void wave_append(bool me, uint32_t value, unsigned long long* counter, uint32_t* list) {
    const unsigned long long mm = __ballot(me);
    if (!mm) return;
    const int leader = __ffsll((long long)mm) - 1;
    unsigned long long pos0 = 0;
    if (lane_id() == leader) pos0 = atomicAdd(counter, (unsigned long long)__popcll(mm));
    pos0 = __shfl(pos0, leader, WAVE);
    if (me) list[pos0 + __popcll(mm & ((1ull << lane_id()) - 1))] = value;
}

// Block-buffered append: a wave reserves room in the block's LDS buffer with
// an LDS atomic and writes its entries there; entries past the buffer go to
// the list directly (wave_append).  The block flushes its buffer with one
// global atomic at its end (block_append_flush), so a kernel whose waves
// nearly all append pays one same-address atomic per block, not per wave.
constexpr int APPEND_BUF = 2048;

__device__ __forceinline__ void block_append(bool me, uint32_t value, uint32_t* s_buf, uint32_t* s_n,
                                             unsigned long long* counter, uint32_t* list) {
    const unsigned long long mm = __ballot(me);
    if (!mm) return;
    const int leader = __ffsll((long long)mm) - 1;
    uint32_t p0 = 0;
    if (lane_id() == leader) p0 = atomicAdd(s_n, (uint32_t)__popcll(mm));
    p0 = __shfl(p0, leader, WAVE);
    const uint32_t p = p0 + (uint32_t)__popcll(mm & ((1ull << lane_id()) - 1));
    if (me && p < (uint32_t)APPEND_BUF) s_buf[p] = value;
    wave_append(me && p >= (uint32_t)APPEND_BUF, value, counter, list);
}

// All threads of the block, after every block_append of the block and a
// barrier.
__device__ __forceinline__ void block_append_flush(const uint32_t* s_buf, uint32_t s_n, unsigned long long* s_base,
                                                   unsigned long long* counter, uint32_t* list) {
    const uint32_t n = s_n < (uint32_t)APPEND_BUF ? s_n : (uint32_t)APPEND_BUF;
    if (threadIdx.x == 0) *s_base = n ? atomicAdd(counter, (unsigned long long)n) : 0;
    __syncthreads();
    for (uint32_t k = threadIdx.x; k < n; k += blockDim.x) list[*s_base + k] = s_buf[k];
}

__device__ __forceinline__ void stamp_row(uint32_t* stamps, int64_t n_stamps, uint32_t clock, uint64_t off) {
    if (stamps && off < (uint64_t)n_stamps) stamps[off] = clock;
}

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
    __shared__ int s_any_miss;
    __shared__ uint32_t s_cand[APPEND_BUF];        // admission candidates of this block
    __shared__ uint32_t s_ncand;
    __shared__ unsigned long long s_cbase;
    if (threadIdx.x == 0) {                        // ordered by the barriers in load_bounds
        s_any_miss = 0;
        s_ncand = 0;
    }
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
    const int64_t n_items = a.list ? (int64_t)*a.list_n : a.n_ids;

    for (int64_t base = wave_global * WAVE; base < n_items; base += n_waves * WAVE) {
        // (1) lanes past the end repeat the last item's reads, so that every
        // load is issued unconditionally
        const int64_t q = base + lane;
        const bool active = q < n_items;
        const int64_t qc = active ? q : n_items - 1;
        const int64_t i = a.list ? (int64_t)a.list[qc] : qc;    // lookup index
        const int t = table_of(sb, a.n_tables, i);
        uint64_t key = (uint64_t)a.ids[i];
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
            if (res < PENDING_BASE) stamp_row(a.stamps, a.n_stamps, a.clock, res);
        }
        if (a.collect) block_append(res == RES_ABSENT, (uint32_t)i, s_cand, &s_ncand, &a.ws.ctr[9], a.ws.cand);

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
            const int64_t ir = shfl_idx(i, src);
            int kind = 2;
            uint64_t val = 0;
            uint32_t slot_idx = 0;
            if (has) probe_full(a, ir, key_r, region_r, key_r == EMPTY_KEY, sub, gshift, kind, val, slot_idx);
            // write results (one lane per group); a miss is left pending,
            // flagged for the later kernels, which find it by its flag
            const bool leader = has && sub == 0;
            if (leader && kind == 1) s_any_miss = 1;
            if (a.collect)
                block_append(leader && kind == 2, (uint32_t)ir, s_cand, &s_ncand, &a.ws.ctr[9], a.ws.cand);
            if (leader) {
                if (kind == 0) {
                    a.row_off[ir] = (int64_t)val;
                    a.ws.flag[ir] = 0;
                    stamp_row(a.stamps, a.n_stamps, a.clock, val);
                } else if (kind == 1) {
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
    // One store per block that saw a miss, instead of a global atomic per
    // wave: same-address atomics from every CU serialize, and with a few
    // misses in most waves they dominated the kernel.
    __syncthreads();
    if (threadIdx.x == 0 && s_any_miss) a.ws.ctr[0] = 1;
    if (a.collect) block_append_flush(s_cand, s_ncand, &s_cbase, &a.ws.ctr[9], a.ws.cand);
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
    int64_t n_ids;
    Ws ws;
};

// One block per tile of SCAN_TILE lookups (16 per thread, as in
// k_rank_commit).  A pending lookup (flag 1) is the first sight of its key
// iff the slot's pending value names it.  The block writes its tile's count
// of first sights (no atomics: the tile is the block's) and adds its
// per-region counts to the regions' totals for the load check, one atomic per
// region present in the tile (usually one: lookups are table-major).
__global__ __launch_bounds__(256) void k_mark(MarkArgs a) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    __shared__ uint32_t s_new[RSE_MAX_TABLES];   // per-region first sights of this tile
    __shared__ uint32_t wsum[4];
    if (a.ws.ctr[0] == 0) return;
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x) s_new[r] = 0;
    __syncthreads();
    // The flags and claimed slots of the thread's 16 lookups are read
    // together, then the slot values of the pending ones (the others read
    // slot 0, masked out), so a wave waits for two round trips however many
    // of its lookups are pending.
    const int64_t i0 = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * 16;
    uint32_t f[16], sl[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const bool in = i0 + k < a.n_ids;
        f[k] = in ? a.ws.flag[i0 + k] : 0u;
        sl[k] = in ? a.ws.slot_of[i0 + k] : 0u;
    }
    uint64_t sv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) sv[k] = a.slots[f[k] == 1 && sl[k] != SIDE_MARK ? sl[k] : 0].val;
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (f[k] != 1) continue;
        const int64_t i = i0 + k;
        // the lookup's region, as the probe formed it: its table, or 0 when merged
        const int region = a.merged ? 0 : table_of(sb, a.n_tables, i);
        const uint64_t v = sl[k] == SIDE_MARK ? a.dir[region].side_val : sv[k];
        if (v == PENDING_BASE + (uint64_t)i) {
            a.ws.flag[i] = 2;
            atomicAdd(&s_new[region], 1u);
            ++c;
        }
    }
    for (int o = WAVE / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, WAVE);
    if (lane_id() == 0) wsum[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) a.ws.tile_sum[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x)
        if (s_new[r]) atomicAdd((unsigned long long*)&a.dir[r].new_keys, (unsigned long long)s_new[r]);
}

// ---------------------------------------------------------- admission --
// Count-min sketch of the lookups of absent keys.  Counter j of a key in
// region r is fmix64(key ^ r * gamma ^ salt_j) reduced to [0, width); the
// estimate is the minimum over the rows.  Increments are integer atomics, so
// the counters after a call do not depend on thread timing.
struct AdmitArgs {
    const int64_t* ids;
    const int64_t* bounds;
    int64_t stride;
    int32_t n_tables;
    int32_t merged;
    uint32_t* sketch;
    int64_t width;
    int32_t depth;
    uint32_t threshold;
    uint64_t salt[8];
    Ws ws;
};

__device__ __forceinline__ int64_t sketch_cell(uint64_t key, uint32_t region, uint64_t salt, int64_t width) {
    return reduce_range(fmix64(key ^ ((uint64_t)region * SM64_GAMMA) ^ salt), width);
}

// Key and region of candidate lookup i.
__device__ __forceinline__ void cand_key(const AdmitArgs& a, const int64_t* sb, uint32_t i, uint64_t& key,
                                         uint32_t& region) {
    const int t = table_of(sb, a.n_tables, i);
    key = (uint64_t)a.ids[i];
    region = (uint32_t)t;
    if (a.merged) {
        key |= (uint64_t)t << 56;
        region = 0;
    }
}

// Counts the candidates (undo 0), or takes the counts back (undo 1, after
// k_decide, for a call that does not commit).  Nothing is counted for a call
// with a bad id.
__global__ void k_admit_count(AdmitArgs a, int32_t undo) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    const unsigned long long n = a.ws.ctr[9];
    if (n == 0 || a.ws.ctr[2] != 0) return;
    if (undo && a.ws.ctr[3] != 0) return;
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    __syncthreads();
    for (unsigned long long q = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; q < n;
         q += (unsigned long long)gridDim.x * blockDim.x) {
        uint64_t key;
        uint32_t region;
        cand_key(a, sb, a.ws.cand[q], key, region);
        for (int j = 0; j < a.depth; ++j) {
            uint32_t* c = a.sketch + (int64_t)j * a.width + sketch_cell(key, region, a.salt[j], a.width);
            if (undo) atomicSub(c, 1u);
            else atomicAdd(c, 1u);
        }
    }
}

// Lists the candidates whose estimate reaches the threshold.
__global__ void k_admit_pick(AdmitArgs a) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    __shared__ uint32_t s_buf[APPEND_BUF];
    __shared__ uint32_t s_n;
    __shared__ unsigned long long s_base;
    const unsigned long long n = a.ws.ctr[9];
    if (n == 0 || a.ws.ctr[2] != 0) return;
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    for (unsigned long long q0 = (unsigned long long)blockIdx.x * blockDim.x; q0 < n;
         q0 += (unsigned long long)gridDim.x * blockDim.x) {
        const unsigned long long q = q0 + threadIdx.x;
        bool pick = false;
        uint32_t i = 0;
        if (q < n) {
            i = a.ws.cand[q];
            uint64_t key;
            uint32_t region;
            cand_key(a, sb, i, key, region);
            uint32_t est = 0xFFFFFFFFu;
            for (int j = 0; j < a.depth; ++j)
                est = min(est, a.sketch[(int64_t)j * a.width + sketch_cell(key, region, a.salt[j], a.width)]);
            pick = est >= a.threshold;
        }
        block_append(pick, i, s_buf, &s_n, &a.ws.ctr[10], a.ws.admitted);
    }
    __syncthreads();
    block_append_flush(s_buf, s_n, &s_base, &a.ws.ctr[10], a.ws.admitted);
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
        // new keys take listed free rows first, then rows past rows_used
        const int64_t used = a.bh->rows_used;
        const int64_t head = a.bh->free_head;
        const int64_t take = min((int64_t)total, a.bh->free_count);
        const int64_t tail = (int64_t)total - take;
        if (!fail && used + tail > a.capacity) fail = RSE_ERR_NEED_GROW;
        a.ws.ctr[4] = (unsigned long long)used;
        a.ws.ctr[5] = total;
        a.ws.ctr[7] = (unsigned long long)head;
        a.ws.ctr[8] = (unsigned long long)take;
        if (!fail) {
            a.ws.ctr[3] = 1;
            a.bh->rows_used = used + tail;
            a.bh->free_head = head + take;
            a.bh->free_count -= take;
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
    const uint32_t* free_list;
    Ws ws;
};

// Row of the new key ranked rk: listed free rows first, then rows_used on.
__device__ __forceinline__ uint64_t new_row_of(const Ws& ws, const uint32_t* free_list, uint64_t rk) {
    const uint64_t take = ws.ctr[8];
    return rk < take ? (uint64_t)free_list[ws.ctr[7] + rk] : ws.ctr[4] + (rk - take);
}

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
            const uint64_t off = new_row_of(a.ws, a.free_list, rk);
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
    const uint32_t* free_list;
    uint32_t* stamps;
    int64_t n_stamps;
    uint32_t clock;
    int32_t pad2;
    int64_t n_ids;
    Ws ws;
};

// One grid-stride range over two kinds of items: first every lookup, of
// which the pending ones (flag 1 or 2) read their key's final offset, or -1
// if the call did not commit, and stamp the row; then every 16 bytes of the
// new rows (weights from the key
// hash, state zero; recycled rows come from the ascending free list and the
// rest are consecutive, so the writes are mostly contiguous).
template <bool BF16>
__global__ void k_finish(FinishArgs a) {
    __shared__ int64_t sb[RSE_MAX_TABLES + 1];
    if (a.ws.ctr[0] == 0) return;
    for (int t = threadIdx.x; t <= a.n_tables; t += blockDim.x) sb[t] = a.bounds[(int64_t)t * a.stride];
    __syncthreads();
    const bool ok = a.ws.ctr[3] != 0;
    const uint64_t n_new = ok ? a.ws.ctr[5] : 0;
    const uint64_t n_look = (uint64_t)a.n_ids;      // lookups scanned for pending ones
    const int64_t q_per_row = a.row_bytes / 16;
    const int64_t w_q = (int64_t)a.dim * (BF16 ? 2 : 4) / 16;   // 16-byte units of weights
    const int per_q = BF16 ? 8 : 4;
    const uint64_t total = n_look + n_new * (uint64_t)q_per_row;
    for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (uint64_t)gridDim.x * blockDim.x) {
        if (e < n_look) {
            const uint32_t i = (uint32_t)e;
            if (a.ws.flag[i] == 0) continue;
            int64_t v = -1;
            if (ok) {
                const uint32_t s = a.ws.slot_of[i];
                if (s == SIDE_MARK) {
                    const int region = a.merged ? 0 : table_of(sb, a.n_tables, i);
                    v = (int64_t)a.dir[region].side_val;
                } else {
                    v = (int64_t)a.slots[s].val;
                }
                stamp_row(a.stamps, a.n_stamps, a.clock, (uint64_t)v);
            }
            a.row_off[i] = v;
            continue;
        }
        const uint64_t ee = e - n_look;
        const uint64_t r = ee / (uint64_t)q_per_row;
        const int64_t qi = (int64_t)(ee - r * (uint64_t)q_per_row);
        char* row = a.rv.row((int64_t)new_row_of(a.ws, a.free_list, r));
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

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

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

// ------------------------------------------------------------ rehash -----
// Copies the keys of one map into another (cleared) map with the same
// regions, keeping their offsets, and drops the keys whose row was last seen
// before a minimum clock.  With a free list attached to the blocks, the
// free list is then rebuilt as every row below rows_used that no kept key
// references, ascending.  Kernels: clear the destination and a row bitmap;
// count kept keys per region and mark their rows; decide (every region
// within its load limit); insert; then count, scan and write the free rows.
// A failed decision leaves the source, the blocks and the free list as they
// were.
constexpr int FL_BLOCK = 256;            // one 32-row bitmap word per thread
constexpr int64_t FL_TILE_ROWS = FL_BLOCK * 32;

struct RehashWs {
    unsigned long long* ctr;   // [0] go flag
    uint32_t* bitmap;          // one bit per row: referenced by a kept key
    uint32_t* tile_sum;        // free rows per tile of FL_TILE_ROWS rows, then their scan
    uint32_t* keep;            // one bit per source slot (then side slot): kept
};

RehashWs carve_rehash(void* base, int64_t rows, int64_t src_slots, size_t* total) {
    Carver c(base);
    RehashWs w;
    const int64_t words = (rows + 31) / 32;
    const int64_t tiles = (rows + FL_TILE_ROWS - 1) / FL_TILE_ROWS;
    w.ctr = c.take<unsigned long long>(16);
    w.bitmap = c.take<uint32_t>((size_t)(words > 0 ? words : 1));
    w.tile_sum = c.take<uint32_t>((size_t)tiles + 1);
    w.keep = c.take<uint32_t>((size_t)(src_slots + 31) / 32 + 1);
    if (total) *total = c.size();
    return w;
}

struct RehashArgs {
    const Slot* src_slots;
    const TableDir* src_dir;
    int64_t src_total;
    int32_t n_regions;
    int32_t use_stamps;
    Slot* dst_slots;
    TableDir* dst_dir;
    MapHeader* dh;
    const uint32_t* stamps;
    int64_t n_stamps;
    uint32_t min_clock;
    int32_t pad;
    int64_t bitmap_rows;
    RehashWs ws;
};

__device__ __forceinline__ bool rh_keep(const RehashArgs& a, uint64_t off) {
    return !a.use_stamps || off >= (uint64_t)a.n_stamps || a.stamps[off] >= a.min_clock;
}

// Region bases in LDS, for region_of_slot without global loads.
__device__ __forceinline__ void stage_region_bases(uint64_t* s_base, const TableDir* dir, int n_regions) {
    for (int r = threadIdx.x; r < n_regions; r += blockDim.x) s_base[r] = (uint64_t)dir[r].slot_base;
    __syncthreads();
}

__device__ __forceinline__ int region_of_slot_lds(const uint64_t* s_base, int n_regions, uint64_t s) {
    int lo = 0, hi = n_regions;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_base[mid] <= s) lo = mid;
        else hi = mid;
    }
    return lo;
}

__global__ void k_rh_reset(RehashArgs a, int64_t n_words, int64_t n_keep_words) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t w = tid; w < n_words; w += (int64_t)gridDim.x * blockDim.x) a.ws.bitmap[w] = 0;
    for (int64_t w = tid; w < n_keep_words; w += (int64_t)gridDim.x * blockDim.x) a.ws.keep[w] = 0;
    for (int64_t r = tid; r < a.n_regions; r += (int64_t)gridDim.x * blockDim.x) {
        a.dst_dir[r].n_keys = 0;
        a.dst_dir[r].side_val = EMPTY_VAL;
        a.dst_dir[r].new_keys = 0;
    }
    if (tid == 0) {
        a.dh->status = 0;
        a.ws.ctr[0] = 0;
    }
}

// One thread per source slot (the side slots after them): a committed
// key, its offset and region, or false for an empty slot.
__device__ __forceinline__ bool rh_slot(const RehashArgs& a, const uint64_t* s_base, int64_t s, uint64_t& key,
                                        uint64_t& off, int& region) {
    if (s < a.src_total) {
        const Slot sl = a.src_slots[s];
        if (sl.key == EMPTY_KEY || sl.val >= PENDING_BASE) return false;
        key = sl.key;
        off = sl.val;
        region = region_of_slot_lds(s_base, a.n_regions, (uint64_t)s);
    } else {
        region = (int)(s - a.src_total);
        off = a.src_dir[region].side_val;
        if (off >= PENDING_BASE) return false;
        key = EMPTY_KEY;
    }
    return true;
}

// Decides which keys stay (their stamps are read here only: the decision is
// kept as one bit per source slot), counts them per region and marks their
// rows.
__global__ void k_rh_count(RehashArgs a) {
    __shared__ uint32_t s_cnt[RSE_MAX_TABLES];
    __shared__ uint64_t s_base[RSE_MAX_TABLES];
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x) s_cnt[r] = 0;
    stage_region_bases(s_base, a.src_dir, a.n_regions);
    const int64_t n = a.src_total + a.n_regions;
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < n; s += (int64_t)gridDim.x * blockDim.x) {
        uint64_t key, off;
        int region;
        if (!rh_slot(a, s_base, s, key, off, region) || !rh_keep(a, off)) continue;
        if (off >= (uint64_t)a.bitmap_rows) {           // an offset past the blocks' capacity
            atomicCAS(&a.dh->status, 0, (int32_t)RSE_ERR_BAD_INPUT);
            continue;
        }
        atomicAdd(&s_cnt[region], 1u);
        atomicOr(&a.ws.bitmap[off >> 5], 1u << (off & 31));
        if (a.use_stamps) atomicOr(&a.ws.keep[s >> 5], 1u << (s & 31));
    }
    __syncthreads();
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x)
        if (s_cnt[r]) atomicAdd((unsigned long long*)&a.dst_dir[r].new_keys, (unsigned long long)s_cnt[r]);
}

__global__ void k_rh_decide(RehashArgs a) {
    __shared__ int s_fail;
    if (threadIdx.x == 0) s_fail = a.dh->status;
    __syncthreads();
    for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x)
        if (a.dst_dir[r].new_keys > a.dst_dir[r].max_keys) atomicCAS(&s_fail, 0, (int)RSE_ERR_IDMAP_FULL);
    __syncthreads();
    if (!s_fail)
        for (int r = threadIdx.x; r < a.n_regions; r += blockDim.x) a.dst_dir[r].n_keys = a.dst_dir[r].new_keys;
    if (threadIdx.x == 0) {
        if (s_fail) atomicCAS(&a.dh->status, 0, s_fail);
        a.ws.ctr[0] = s_fail ? 0 : 1;
    }
}

// Keys are distinct per region in the source, so an insert only has to find
// an empty slot along its chain.
__global__ void k_rh_insert(RehashArgs a) {
    __shared__ uint64_t s_base[RSE_MAX_TABLES];
    if (a.ws.ctr[0] != 1) return;
    stage_region_bases(s_base, a.src_dir, a.n_regions);
    const int64_t n = a.src_total + a.n_regions;
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < n; s += (int64_t)gridDim.x * blockDim.x) {
        if (a.use_stamps && !((a.ws.keep[s >> 5] >> (s & 31)) & 1u)) continue;
        uint64_t key, off;
        int region;
        if (!rh_slot(a, s_base, s, key, off, region)) continue;
        if (key == EMPTY_KEY) {
            a.dst_dir[region].side_val = off;
            continue;
        }
        const TableDir d = a.dst_dir[region];
        int64_t b = reduce_range(fmix64(key ^ d.salt), d.n_buckets);
        bool done = false;
        for (int64_t probes = 0; probes < d.n_buckets && !done; ++probes) {
            const int64_t base = d.slot_base + b * BUCKET;
            for (int q = 0; q < BUCKET && !done; ++q) {
                if (a.dst_slots[base + q].key != EMPTY_KEY) continue;
                const unsigned long long old = atomicCAS((unsigned long long*)&a.dst_slots[base + q].key,
                                                         (unsigned long long)EMPTY_KEY, (unsigned long long)key);
                if (old == EMPTY_KEY) {
                    a.dst_slots[base + q].val = off;
                    done = true;
                }
            }
            b = (b + 1 == d.n_buckets) ? 0 : b + 1;
        }
        if (!done) atomicCAS(&a.dh->status, 0, (int32_t)RSE_ERR_IDMAP_FULL);
    }
}

struct FreeArgs {
    const uint32_t* bitmap;
    BlocksHeader* bh;
    uint32_t* free_list;
    uint32_t* tile_sum;
    int64_t n_tiles;
    const unsigned long long* go;
};

// Free rows among the 32 of bitmap word w (rows below rows_used only).
__device__ __forceinline__ uint32_t free_bits(const FreeArgs& a, int64_t w, int64_t rows) {
    const int64_t r0 = w * 32;
    if (r0 >= rows) return 0u;
    const uint32_t valid = rows - r0 >= 32 ? 0xFFFFFFFFu : ((1u << (rows - r0)) - 1u);
    return ~a.bitmap[w] & valid;
}

// Block-wide exclusive scan of FL_BLOCK values; returns the total.
__device__ uint32_t fl_block_scan(uint32_t v, uint32_t* excl) {
    __shared__ uint32_t wsum[FL_BLOCK / WAVE];
    const int lane = lane_id();
    const int w = threadIdx.x / WAVE;
    uint32_t x = v;
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) wsum[w] = x;
    __syncthreads();
    uint32_t pre = 0, total = 0;
    for (int k = 0; k < FL_BLOCK / WAVE; ++k) {
        if (k < w) pre += wsum[k];
        total += wsum[k];
    }
    __syncthreads();
    *excl = pre + x - v;
    return total;
}

__global__ __launch_bounds__(FL_BLOCK) void k_fl_count(FreeArgs a) {
    if (*a.go != 1) return;
    const int64_t rows = a.bh->rows_used;
    const int64_t w = (int64_t)blockIdx.x * FL_BLOCK + threadIdx.x;
    uint32_t ex;
    const uint32_t t = fl_block_scan((uint32_t)__popc(free_bits(a, w, rows)), &ex);
    if (threadIdx.x == 0) a.tile_sum[blockIdx.x] = t;
}

__global__ __launch_bounds__(FL_BLOCK) void k_fl_scan(FreeArgs a) {
    __shared__ uint32_t s_carry;
    if (*a.go != 1) return;
    if (threadIdx.x == 0) s_carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < a.n_tiles; base += FL_BLOCK) {
        const int64_t k = base + threadIdx.x;
        const uint32_t v = k < a.n_tiles ? a.tile_sum[k] : 0;
        uint32_t ex;
        const uint32_t t = fl_block_scan(v, &ex);
        const uint32_t carry = s_carry;
        if (k < a.n_tiles) a.tile_sum[k] = carry + ex;
        __syncthreads();
        if (threadIdx.x == 0) s_carry = carry + t;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.bh->free_head = 0;
        a.bh->free_count = s_carry;
    }
}

__global__ __launch_bounds__(FL_BLOCK) void k_fl_write(FreeArgs a) {
    if (*a.go != 1) return;
    const int64_t rows = a.bh->rows_used;
    const int64_t w = (int64_t)blockIdx.x * FL_BLOCK + threadIdx.x;
    uint32_t bits = free_bits(a, w, rows);
    uint32_t ex;
    fl_block_scan((uint32_t)__popc(bits), &ex);
    uint64_t pos = (uint64_t)a.tile_sum[blockIdx.x] + ex;
    while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        a.free_list[pos++] = (uint32_t)(w * 32 + b);
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
    // every row a lookup can resolve to must have a stamp
    if (map->d_stamps && map->n_stamps < blocks->capacity()) return RSE_ERR_INVALID_ARG;
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
    // With admission the probe runs twice: first without inserting, listing
    // the lookups of absent keys; then, after the sketch has counted them,
    // with inserting, over the admitted ones only.
    const bool admit = insert_missing && map->admission_on();
    pa.insert = insert_missing && !admit ? 1 : 0;
    pa.collect = admit ? 1 : 0;
    pa.row_off = d_row_off_out;
    pa.list = nullptr;
    pa.list_n = nullptr;
    pa.stamps = map->d_stamps;
    pa.n_stamps = map->n_stamps;
    pa.clock = map->clock;
    pa.pad2 = 0;
    pa.ws = ws;
    // 64 lookups per wave per iteration; enough waves to fill 256 CUs
    const int probe_blocks = fill_blocks((n_ids + WAVE - 1) / WAVE, PROBE_BLOCK / 64, 256 * 16);
    {
        TraceScope ts(RSE_K_PROBE, s);
        hipLaunchKernelGGL(k_probe, dim3(probe_blocks), dim3(PROBE_BLOCK), 0, s, pa);
    }

    const int miss_blocks = fill_blocks(n_ids, 256, 2048);
    AdmitArgs aa;
    if (admit) {
        aa.ids = d_ids;
        aa.bounds = d_bounds;
        aa.stride = stride;
        aa.n_tables = n_tables;
        aa.merged = map->merged;
        aa.sketch = map->d_sketch;
        aa.width = map->sk_width;
        aa.depth = map->sk_depth;
        aa.threshold = map->admit_min;
        for (int j = 0; j < 8; ++j) aa.salt[j] = map->sk_salt[j];
        aa.ws = ws;
        hipLaunchKernelGGL(k_admit_count, dim3(miss_blocks), dim3(256), 0, s, aa, 0);
        hipLaunchKernelGGL(k_admit_pick, dim3(miss_blocks), dim3(256), 0, s, aa);
        ProbeArgs pb = pa;
        pb.insert = 1;
        pb.collect = 0;
        pb.list = ws.admitted;
        pb.list_n = &ws.ctr[10];
        hipLaunchKernelGGL(k_probe, dim3(probe_blocks), dim3(PROBE_BLOCK), 0, s, pb);
    }
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
    ma.n_ids = n_ids;
    ma.ws = ws;
    const dim3 tiles_grid((unsigned)(n_tiles > 0 ? n_tiles : 1));
    hipLaunchKernelGGL(k_mark, tiles_grid, dim3(256), 0, s, ma);

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
    if (admit) hipLaunchKernelGGL(k_admit_count, dim3(miss_blocks), dim3(256), 0, s, aa, 1);

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
    ca.free_list = blocks->d_free;
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
    fa.free_list = blocks->d_free;
    fa.stamps = map->d_stamps;
    fa.n_stamps = map->n_stamps;
    fa.clock = map->clock;
    fa.pad2 = 0;
    fa.n_ids = n_ids;
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

// ------------------------------------------- admission, age, eviction --
int rse_idmap_set_stamps(rse_idmap* map, uint32_t* d_stamps, int64_t n_stamps) {
    if (!map || n_stamps < 0 || (n_stamps > 0 && !d_stamps)) return RSE_ERR_INVALID_ARG;
    map->d_stamps = n_stamps > 0 ? d_stamps : nullptr;
    map->n_stamps = n_stamps > 0 ? n_stamps : 0;
    return RSE_OK;
}

int rse_idmap_set_clock(rse_idmap* map, uint32_t clock) {
    if (!map) return RSE_ERR_INVALID_ARG;
    map->clock = clock;
    return RSE_OK;
}

int rse_idmap_set_admission(rse_idmap* map, uint32_t* d_sketch, int32_t depth, int64_t width, uint32_t threshold,
                            uint64_t seed, void* stream) {
    if (!map) return RSE_ERR_INVALID_ARG;
    if (threshold <= 1) {
        map->d_sketch = nullptr;
        map->sk_depth = 0;
        map->sk_width = 0;
        map->admit_min = threshold;
        return RSE_OK;
    }
    if (!d_sketch || depth < 1 || depth > 8 || width < 1) return RSE_ERR_INVALID_ARG;
    map->d_sketch = d_sketch;
    map->sk_depth = depth;
    map->sk_width = width;
    map->admit_min = threshold;
    // row salts: successive SplitMix64 outputs of the seed
    uint64_t sm = seed;
    for (int j = 0; j < 8; ++j) {
        sm += SM64_GAMMA;
        uint64_t z = sm;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        map->sk_salt[j] = j < depth ? z ^ (z >> 31) : 0;
    }
    const int64_t n = (int64_t)depth * width;
    hipLaunchKernelGGL(k_fill_u32, dim3(fill_blocks(n, 256, 4096)), dim3(256), 0, as_stream(stream), d_sketch, n,
                       0u);
    return launch_status();
}

int rse_idmap_rehash_workspace_size(const rse_idmap* src, const rse_blocks* blocks, size_t* bytes_out) {
    if (!src || !blocks || !bytes_out) return RSE_ERR_INVALID_ARG;
    carve_rehash(nullptr, blocks->capacity(), src->total_slots + src->n_tables, bytes_out);
    return RSE_OK;
}

int rse_idmap_rehash(rse_idmap* dst, rse_idmap* src, rse_blocks* blocks, uint32_t min_clock, void* d_ws,
                     size_t ws_bytes, void* stream) {
    if (!dst || !src || !blocks || !d_ws || dst == src) return RSE_ERR_INVALID_ARG;
    if (dst->n_tables != src->n_tables || dst->merged != src->merged) return RSE_ERR_INVALID_ARG;
    const char* d0 = dst->d_mem;
    const char* s0 = src->d_mem;
    if (d0 < s0 + src->mem_bytes() && s0 < d0 + dst->mem_bytes()) return RSE_ERR_INVALID_ARG;
    const int64_t cap = blocks->capacity();
    if (src->d_stamps && src->n_stamps < cap) return RSE_ERR_INVALID_ARG;
    if (blocks->d_free && blocks->free_cap < cap) return RSE_ERR_INVALID_ARG;
    size_t need = 0;
    const int64_t n_src = src->total_slots + src->n_tables;
    RehashWs ws = carve_rehash(d_ws, cap, n_src, &need);
    if (ws_bytes < need) return RSE_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);

    RehashArgs a;
    a.src_slots = src->d_slots();
    a.src_dir = src->d_dir();
    a.src_total = src->total_slots;
    a.n_regions = src->n_tables;
    a.use_stamps = src->d_stamps ? 1 : 0;
    a.dst_slots = dst->d_slots();
    a.dst_dir = dst->d_dir();
    a.dh = dst->header();
    a.stamps = src->d_stamps;
    a.n_stamps = src->n_stamps;
    a.min_clock = min_clock;
    a.pad = 0;
    a.bitmap_rows = cap;
    a.ws = ws;
    const int64_t n_words = (cap + 31) / 32;
    hipLaunchKernelGGL(k_clear_slots, dim3(fill_blocks(dst->total_slots, 256, 8192)), dim3(256), 0, s,
                       dst->d_slots(), dst->total_slots);
    const int64_t n_keep_words = src->d_stamps ? (n_src + 31) / 32 : 0;
    const int64_t reset_items = std::max<int64_t>(std::max<int64_t>(n_words, n_keep_words), src->n_tables);
    hipLaunchKernelGGL(k_rh_reset, dim3(fill_blocks(reset_items, 256, 4096)), dim3(256), 0, s, a, n_words,
                       n_keep_words);
    const dim3 grid(fill_blocks(src->total_slots + src->n_tables, 256, 8192));
    hipLaunchKernelGGL(k_rh_count, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_rh_decide, dim3(1), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_rh_insert, grid, dim3(256), 0, s, a);
    if (blocks->d_free && cap > 0) {
        FreeArgs f;
        f.bitmap = ws.bitmap;
        f.bh = blocks->header();
        f.free_list = blocks->d_free;
        f.tile_sum = ws.tile_sum;
        f.n_tiles = (cap + FL_TILE_ROWS - 1) / FL_TILE_ROWS;
        f.go = ws.ctr;
        hipLaunchKernelGGL(k_fl_count, dim3((unsigned)f.n_tiles), dim3(FL_BLOCK), 0, s, f);
        hipLaunchKernelGGL(k_fl_scan, dim3(1), dim3(FL_BLOCK), 0, s, f);
        hipLaunchKernelGGL(k_fl_write, dim3((unsigned)f.n_tiles), dim3(FL_BLOCK), 0, s, f);
    }
    // the destination takes over the source's policies
    dst->d_stamps = src->d_stamps;
    dst->n_stamps = src->n_stamps;
    dst->clock = src->clock;
    dst->d_sketch = src->d_sketch;
    dst->sk_depth = src->sk_depth;
    dst->sk_width = src->sk_width;
    dst->admit_min = src->admit_min;
    for (int j = 0; j < 8; ++j) dst->sk_salt[j] = src->sk_salt[j];
    return launch_status();
}

}  // extern "C"
