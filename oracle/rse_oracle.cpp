// rse_oracle.cpp -- plain, slow, single-threaded CPU oracle for the sparse
// embedding training step (ID map find-or-insert, pooled bag gather, sparse
// backward with duplicate merge, row-wise SGD / Adagrad / Adam update).
//
// TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
// the test suite, the smoke check and the benchmark's CPU-baseline leg load
// it.  It shares no source, header, table or helper with the HIP library, and
// neither side includes or links the other.
//
// Everything is written the obvious way: std::unordered_map per table for the
// ID map, a loop per bag for pooling, a std::map from row offset to a double
// accumulator for the gradient merge, and one double-precision update per
// touched element, rounded once to the storage type.
//
// Sources (web pages held as text; cited by page title and section):
//  * "阿里 RecIS：搜广推训练的背景与难点" (muyuuuu.github.io), the passage after
//    the two-tower model: a lookup reads only the indexed row and backward
//    updates only that row; the toy nn.Embedding(10,4) / ids {2,5,7} /
//    loss = sum(e^2) / SGD lr 0.1 example; the modulo-sharding collision
//    example that motivates a hash map keyed by the raw ID.
//  * "RecIS：阿里开源推荐系统统一训练框架" (pomoai.com), section "Embedding
//    Engine": a two-level table, IDMap (feature ID -> offset) over
//    EmbeddingBlocks (parameters plus optimizer state) that grows without
//    moving rows; tables with the same attributes can be merged into one.
//  * "DLRM模型的核心价值与工业落地挑战" (mokono.cn), section 2.1: EmbeddingBag
//    with sum pooling over variable-length inputs and sparse gradients.
//  * "DLRM — Meta 把工业推荐模型拆成 4 个标准积木" (estelledc.github.io),
//    "踩过的坑" item 4: only rows seen in the batch are updated, with a sparse
//    optimizer of the SparseAdam kind.
//
// Readings where the pages are silent (each one is a definition here):
//  * new keys receive offsets 0,1,2,... in order of first sight, scanning the
//    lookups in array order (table-major, then sample, then position in bag);
//  * a new row is initialised from its key by a counter-based hash
//    (SplitMix64 finaliser, Vigna's published algorithm) and its optimizer
//    state starts at zero;
//  * Adagrad keeps one fp32 accumulator per weight element, eps outside the
//    square root;  Adam is the lazy form of Kingma & Ba (2015) Algorithm 1
//    with one global step counter per table group;
//  * mean pooling divides by the bag length; an empty bag pools to zero and
//    has no gradient; a missing key (offset -1) contributes nothing;
//  * bf16 storage rounds the final double value to nearest, ties to even.
//
// Feature admission and eviction ("RecIS：阿里开源推荐系统统一训练框架",
// "代码架构": a hook on the hash table for feature admission and eviction;
// the policies themselves are not given, so these are definitions here):
//  * admission (off unless a threshold above 1 is set): a count-min sketch of
//    `depth` rows of `width` uint32 counters counts every lookup of a key that
//    is absent from the map when the call starts (all lookups of the call are
//    counted before any is inserted); an absent key is inserted only if its
//    estimate -- the minimum of its counters after the call's counts -- is at
//    least the threshold; otherwise its lookups get offset -1.  Counter j of a
//    key is fmix64(key ^ map_index * golden ^ salt_j) reduced to [0, width)
//    by a 64x64 multiply-high (murmur3 fmix64; salt_j = the (j+1)-th
//    SplitMix64 output of the sketch seed);
//  * age: with tracking on, every lookup that resolves to a row stamps the
//    row with the current clock (a caller-set integer, typically the step);
//  * eviction (rehash with a minimum clock): keys whose row's stamp is below
//    the minimum leave the map; every other key keeps its offset;
//  * recycling (when on): the rehash lists every row below the row counter
//    that no remaining key references, ascending; new keys take rows from
//    that list in order before new rows are appended.  A reused row starts
//    over from its new key's initial value and zero optimizer state.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <unordered_map>
#include <vector>

namespace {

enum { W_F32 = 0, W_BF16 = 1 };
enum { OPT_SGD = 0, OPT_ADAGRAD = 1, OPT_ADAM = 2 };
enum { POOL_SUM = 0, POOL_MEAN = 1 };

// ---------------------------------------------------------------- init ----
// SplitMix64 output function (Steele, Lea & Flood 2014; Vigna's public
// domain reference): two xor-shift-multiply rounds and a final xor-shift.
uint64_t splitmix64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

const uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;  // SplitMix64 increment

// MurmurHash3's 64-bit finaliser (Appleby, public domain).
uint64_t fmix64(uint64_t k) {
    k ^= k >> 33;
    k *= 0xFF51AFD7ED558CCDull;
    k ^= k >> 33;
    k *= 0xC4CEB9FE1A85EC53ull;
    k ^= k >> 33;
    return k;
}
const double INIT_SCALE = 1.0 / 16.0;           // sigma = 2^-4

// Value of column c of a freshly inserted row (exact in the storage type).
double init_value(uint64_t key, int32_t table, int32_t c, uint64_t seed, int32_t wdtype) {
    uint64_t x = (key ^ ((seed + (uint64_t)(uint32_t)table) * GOLDEN)) + (uint64_t)(c + 1) * GOLDEN;
    uint64_t h = splitmix64_mix(x);
    if (wdtype == W_F32) {
        int64_t q = (int64_t)(h >> 40) - (int64_t)(1 << 23);  // in [-2^23, 2^23)
        return std::ldexp((double)q, -23) * INIT_SCALE;
    } else {
        int64_t q = (int64_t)(h >> 56) - 128;                 // in [-128, 128)
        return std::ldexp((double)q, -7) * INIT_SCALE;
    }
}

// ----------------------------------------------------------- rounding ----
float round_to_f32(double x) { return (float)x; }  // C conversion: nearest-even

// Nearest bf16 value to x, ties to even, computed directly from the double
// (no intermediate fp32 rounding).  bf16 has fp32's exponent range and 8
// significant bits.
uint16_t round_to_bf16(double x) {
    if (std::isnan(x)) return 0x7FC0;
    double ax = std::fabs(x);
    bool neg = std::signbit(x);
    double r;
    if (ax == 0.0) {
        r = 0.0;
    } else {
        int e;
        std::frexp(ax, &e);                      // ax = f * 2^e, f in [0.5, 1)
        int ulp_exp = e - 8;                     // 8 significant bits
        if (ulp_exp < -133) ulp_exp = -133;      // subnormal spacing 2^-133
        double scaled = std::ldexp(ax, -ulp_exp);
        double q = std::nearbyint(scaled);       // default mode: ties to even
        r = std::ldexp(q, ulp_exp);
    }
    if (r >= 0x1p128) {                          // overflow -> infinity
        return neg ? 0xFF80 : 0x7F80;
    }
    float f = (float)r;                          // exact: r has <= 8 bits
    uint32_t u;
    std::memcpy(&u, &f, 4);
    uint16_t b = (uint16_t)(u >> 16);
    if (neg) b |= 0x8000;
    return b;
}

double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
}

// --------------------------------------------------------------- model ----
struct Row {
    std::vector<double> w;       // exact widening of the stored value
    std::vector<float> state;    // Adagrad: acc[d];  Adam: m[d] then v[d]
};

struct Table {
    int32_t dim, wdtype, optim, n_tables, merged;
    uint64_t seed;
    double lr, eps, beta1, beta2;
    int64_t step = 0;
    // One map per logical table; in merged mode a single map keyed by
    // (table << 56) | id.
    std::vector<std::unordered_map<int64_t, int64_t>> maps;
    int64_t n_rows = 0;
    std::vector<int64_t> row_key;      // offset -> key
    std::vector<int32_t> row_table;    // offset -> map index
    std::unordered_map<int64_t, Row> rows;  // materialised (touched) rows
    // Last backward step, for inspection by tests.
    std::map<int64_t, std::vector<double>> last_grad;
    std::map<int64_t, int64_t> last_count;

    // Admission, age and recycling (definitions in the file header).
    bool track = false;
    uint32_t clock = 0;
    std::vector<uint32_t> last_seen;   // per row
    uint32_t admit_min = 0;
    int32_t sk_depth = 0;
    int64_t sk_width = 0;
    std::vector<uint64_t> sk_salt;
    std::vector<uint32_t> sketch;      // [depth][width]
    bool recycle = false;
    std::vector<int64_t> free_rows;    // ascending, from the last rehash
    size_t free_next = 0;

    bool admission_on() const { return admit_min > 1 && sk_width > 0; }

    int64_t sketch_cell(uint64_t key, int32_t m, int j) const {
        const uint64_t h = fmix64(key ^ ((uint64_t)(uint32_t)m * GOLDEN) ^ sk_salt[j]);
        return (int64_t)(((unsigned __int128)h * (uint64_t)sk_width) >> 64);
    }

    uint32_t estimate(uint64_t key, int32_t m) const {
        uint32_t e = UINT32_MAX;
        for (int j = 0; j < sk_depth; ++j) e = std::min(e, sketch[(size_t)j * sk_width + sketch_cell(key, m, j)]);
        return e;
    }

    // Row for a new key: the next listed free row, else a new one.
    int64_t new_row(int64_t key, int32_t m) {
        int64_t off;
        if (recycle && free_next < free_rows.size()) {
            off = free_rows[free_next++];
            row_key[off] = key;
            row_table[off] = m;
            rows.erase(off);
        } else {
            off = n_rows++;
            row_key.push_back(key);
            row_table.push_back(m);
            last_seen.push_back(0);
        }
        return off;
    }

    int state_per_elem() const {
        return optim == OPT_SGD ? 0 : (optim == OPT_ADAGRAD ? 1 : 2);
    }

    // Current row contents; an untouched row is its initial value.
    void fetch(int64_t off, Row& r) const {
        auto it = rows.find(off);
        if (it != rows.end()) {
            r = it->second;
            return;
        }
        r.w.resize(dim);
        for (int c = 0; c < dim; ++c)
            r.w[c] = init_value((uint64_t)row_key[off], row_table[off], c, seed, wdtype);
        r.state.assign((size_t)dim * state_per_elem(), 0.0f);
    }
};

}  // namespace

extern "C" {

void* orc_create(int32_t dim, int32_t wdtype, int32_t optim, int32_t n_tables, int32_t merged,
                 uint64_t seed, double lr, double eps, double beta1, double beta2) {
    if (dim <= 0 || n_tables <= 0 || (wdtype != W_F32 && wdtype != W_BF16) || optim < 0 || optim > 2)
        return nullptr;
    if (merged && n_tables > 127) return nullptr;
    Table* t = new Table();
    t->dim = dim; t->wdtype = wdtype; t->optim = optim; t->n_tables = n_tables; t->merged = merged;
    t->seed = seed; t->lr = lr; t->eps = eps; t->beta1 = beta1; t->beta2 = beta2;
    t->maps.resize(merged ? 1 : n_tables);
    return t;
}

void orc_destroy(void* h) { delete (Table*)h; }

// Key formation and find-or-insert in canonical (array) order.  Table t's
// lookups are ids[bounds[t*stride] .. bounds[(t+1)*stride]) (with the bag
// offsets and stride = batch this is the table-major bag layout).
// Returns 0, or -1 on a bad argument.
int orc_find_or_insert(void* h, const int64_t* ids, int64_t n_ids, const int64_t* bounds,
                       int64_t stride, int32_t n_tables, int32_t insert_missing,
                       int64_t* row_off_out, int64_t* n_new_out) {
    Table* T = (Table*)h;
    if (n_tables != T->n_tables || stride <= 0) return -1;
    if (bounds[0] != 0 || bounds[(int64_t)n_tables * stride] != n_ids) return -1;
    for (int32_t t = 0; t < n_tables; ++t)
        if (bounds[(int64_t)(t + 1) * stride] < bounds[(int64_t)t * stride]) return -1;
    // keys and map indices of every lookup (and the merged-mode id check)
    std::vector<int64_t> keys(n_ids);
    std::vector<int32_t> mi(n_ids);
    for (int32_t t = 0; t < n_tables; ++t) {
        for (int64_t i = bounds[(int64_t)t * stride]; i < bounds[(int64_t)(t + 1) * stride]; ++i) {
            int64_t key = ids[i];
            int32_t m = t;
            if (T->merged) {
                if (key < 0 || key >= (int64_t(1) << 56)) return -1;
                key = (int64_t)(((uint64_t)t << 56) | (uint64_t)key);
                m = 0;
            }
            keys[i] = key;
            mi[i] = m;
        }
    }
    // admission: count every lookup of a key absent at the start of the call
    const bool admit = insert_missing && T->admission_on();
    if (admit) {
        for (int64_t i = 0; i < n_ids; ++i) {
            if (T->maps[mi[i]].count(keys[i])) continue;
            for (int j = 0; j < T->sk_depth; ++j)
                T->sketch[(size_t)j * T->sk_width + T->sketch_cell((uint64_t)keys[i], mi[i], j)] += 1u;
        }
    }
    int64_t n_new = 0;
    for (int64_t i = 0; i < n_ids; ++i) {
        auto& map = T->maps[mi[i]];
        auto it = map.find(keys[i]);
        int64_t off = -1;
        if (it != map.end()) {
            off = it->second;
        } else if (insert_missing && (!admit || T->estimate((uint64_t)keys[i], mi[i]) >= T->admit_min)) {
            off = T->new_row(keys[i], mi[i]);
            map.emplace(keys[i], off);
            ++n_new;
        }
        row_off_out[i] = off;
        if (off >= 0 && T->track) T->last_seen[off] = T->clock;
    }
    *n_new_out = n_new;
    return 0;
}

// Pooled forward: out[b, t, :] = sum (or mean) of the bag's rows, in double,
// rounded once to fp32.  Layout of out: [batch, n_tables, dim].
int orc_fwd(void* h, const int64_t* row_off, const int64_t* bag_offsets, int32_t n_tables,
            int64_t batch, int32_t pooling, float* out) {
    Table* T = (Table*)h;
    const int64_t n_bags = (int64_t)n_tables * batch;
    const int d = T->dim;
    std::vector<double> s(d);
    Row r;
    for (int64_t j = 0; j < n_bags; ++j) {
        const int64_t t = j / batch, b = j % batch;
        std::fill(s.begin(), s.end(), 0.0);
        const int64_t len = bag_offsets[j + 1] - bag_offsets[j];
        for (int64_t i = bag_offsets[j]; i < bag_offsets[j + 1]; ++i) {
            if (row_off[i] < 0) continue;
            T->fetch(row_off[i], r);
            for (int c = 0; c < d; ++c) s[c] += r.w[c];
        }
        if (pooling == POOL_MEAN && len > 0)
            for (int c = 0; c < d; ++c) s[c] /= (double)len;
        float* o = out + (b * n_tables + t) * d;
        for (int c = 0; c < d; ++c) o[c] = round_to_f32(s[c]);
    }
    return 0;
}

// Sparse backward and update.  grad has the layout of out.  Each lookup i in
// bag j contributes G[b, t, :] (divided by the bag length for mean pooling)
// to its row; contributions to the same row are summed in double in lookup
// order; then the optimizer runs once per touched row.  Untouched rows are
// not visited.
int orc_bwd_update(void* h, const int64_t* row_off, const int64_t* bag_offsets, int32_t n_tables,
                   int64_t batch, int32_t pooling, const float* grad, int64_t* n_unique_out) {
    Table* T = (Table*)h;
    const int64_t n_bags = (int64_t)n_tables * batch;
    const int d = T->dim;
    T->last_grad.clear();
    T->last_count.clear();
    for (int64_t j = 0; j < n_bags; ++j) {
        const int64_t t = j / batch, b = j % batch;
        const int64_t len = bag_offsets[j + 1] - bag_offsets[j];
        const float* g = grad + (b * n_tables + t) * d;
        for (int64_t i = bag_offsets[j]; i < bag_offsets[j + 1]; ++i) {
            const int64_t o = row_off[i];
            if (o < 0) continue;
            auto& acc = T->last_grad[o];
            if (acc.empty()) acc.assign(d, 0.0);
            for (int c = 0; c < d; ++c) {
                double gi = (double)g[c];
                if (pooling == POOL_MEAN) gi = gi / (double)len;
                acc[c] += gi;
            }
            T->last_count[o] += 1;
        }
    }
    T->step += 1;
    const double t_step = (double)T->step;
    const double bc1 = 1.0 - std::pow(T->beta1, t_step);
    const double bc2 = 1.0 - std::pow(T->beta2, t_step);
    Row r;
    for (auto& kv : T->last_grad) {
        const int64_t o = kv.first;
        const std::vector<double>& g = kv.second;
        T->fetch(o, r);
        for (int c = 0; c < d; ++c) {
            double w = r.w[c];
            double w_new;
            if (T->optim == OPT_SGD) {
                w_new = w - T->lr * g[c];
            } else if (T->optim == OPT_ADAGRAD) {
                float a = round_to_f32((double)r.state[c] + g[c] * g[c]);
                r.state[c] = a;
                w_new = w - T->lr * (g[c] / (std::sqrt((double)a) + T->eps));
            } else {
                float m = round_to_f32(T->beta1 * (double)r.state[c] + (1.0 - T->beta1) * g[c]);
                float v = round_to_f32(T->beta2 * (double)r.state[d + c] + (1.0 - T->beta2) * g[c] * g[c]);
                r.state[c] = m;
                r.state[d + c] = v;
                double m_hat = (double)m / bc1;
                double v_hat = (double)v / bc2;
                w_new = w - T->lr * (m_hat / (std::sqrt(v_hat) + T->eps));
            }
            r.w[c] = (T->wdtype == W_F32) ? (double)round_to_f32(w_new)
                                          : bf16_to_double(round_to_bf16(w_new));
        }
        T->rows[o] = r;
    }
    *n_unique_out = (int64_t)T->last_grad.size();
    return 0;
}

int64_t orc_n_rows(void* h) { return ((Table*)h)->n_rows; }
int64_t orc_step(void* h) { return ((Table*)h)->step; }

// Copies rows (weights widened to fp32, exact for both storage types) and
// their optimizer state ([n, state_per_elem * dim]).  Either output may be null.
int orc_get_rows(void* h, const int64_t* offs, int64_t n, float* w_out, float* state_out) {
    Table* T = (Table*)h;
    const int d = T->dim, k = T->state_per_elem();
    Row r;
    for (int64_t q = 0; q < n; ++q) {
        if (offs[q] < 0 || offs[q] >= T->n_rows) return -1;
        T->fetch(offs[q], r);
        if (w_out)
            for (int c = 0; c < d; ++c) w_out[q * d + c] = (float)r.w[c];
        if (state_out)
            for (int c = 0; c < k * d; ++c) state_out[q * k * d + c] = r.state[c];
    }
    return 0;
}

// Map contents in offset order: key (merged key in merged mode) and map index.
int orc_map_dump(void* h, int64_t* keys_out, int32_t* table_out) {
    Table* T = (Table*)h;
    for (int64_t o = 0; o < T->n_rows; ++o) {
        keys_out[o] = T->row_key[o];
        table_out[o] = T->row_table[o];
    }
    return 0;
}

// Offsets touched by the last backward step, ascending, with their counts.
int64_t orc_touched(void* h, int64_t* offs_out, int64_t* counts_out) {
    Table* T = (Table*)h;
    int64_t q = 0;
    for (auto& kv : T->last_count) {
        if (offs_out) offs_out[q] = kv.first;
        if (counts_out) counts_out[q] = kv.second;
        ++q;
    }
    return q;
}

// Merged gradient of one row from the last backward step (double, [dim]).
int orc_last_grad(void* h, int64_t off, double* g_out) {
    Table* T = (Table*)h;
    auto it = T->last_grad.find(off);
    if (it == T->last_grad.end()) return -1;
    for (int c = 0; c < T->dim; ++c) g_out[c] = it->second[c];
    return 0;
}

// Restore a saved state ("RecIS：阿里开源推荐系统统一训练框架", "Saver"): the
// table's maps, rows and step counter are replaced by n entries (key, map
// index, offset) with their weights [n, dim] (exact in the storage type) and
// state [n, k * dim], and the row counter set to n_rows.  Offsets must be
// distinct and below n_rows; every row below n_rows must be listed.
// Returns 0, or -1 on a bad argument.
int orc_import(void* h, const int64_t* keys, const int32_t* tables, const int64_t* offs, const float* w,
               const float* state, int64_t n, int64_t n_rows, int64_t step) {
    Table* T = (Table*)h;
    const int d = T->dim, k = T->state_per_elem();
    if (n != n_rows || n < 0) return -1;
    for (auto& m : T->maps) m.clear();
    T->rows.clear();
    T->last_grad.clear();
    T->last_count.clear();
    T->row_key.assign(n_rows, 0);
    T->row_table.assign(n_rows, -1);
    for (int64_t i = 0; i < n; ++i) {
        if (offs[i] < 0 || offs[i] >= n_rows || tables[i] < 0 || tables[i] >= (int32_t)T->maps.size()) return -1;
        if (T->row_table[offs[i]] != -1) return -1;
        if (!T->maps[tables[i]].emplace(keys[i], offs[i]).second) return -1;
        T->row_key[offs[i]] = keys[i];
        T->row_table[offs[i]] = tables[i];
        Row r;
        r.w.resize(d);
        for (int c = 0; c < d; ++c) r.w[c] = (double)w[i * d + c];
        r.state.assign(state ? state + i * k * d : nullptr, state ? state + (i + 1) * k * d : nullptr);
        T->rows[offs[i]] = r;
    }
    T->n_rows = n_rows;
    T->step = step;
    T->last_seen.assign(n_rows, 0);
    T->free_rows.clear();
    T->free_next = 0;
    return 0;
}

// ------------------------------------------- admission, age, eviction ----
// Tracking on: lookups stamp their rows with the clock (stamps start at 0).
int orc_set_tracking(void* h, int32_t on) {
    Table* T = (Table*)h;
    T->track = on != 0;
    std::fill(T->last_seen.begin(), T->last_seen.end(), 0u);
    return 0;
}

int orc_set_clock(void* h, uint32_t clock) {
    ((Table*)h)->clock = clock;
    return 0;
}

// Admission with a fresh (zero) sketch; threshold <= 1 turns it off.
int orc_set_admission(void* h, int32_t depth, int64_t width, uint32_t threshold, uint64_t seed) {
    Table* T = (Table*)h;
    if (threshold > 1 && (depth < 1 || depth > 8 || width < 1)) return -1;
    T->admit_min = threshold;
    T->sk_depth = threshold > 1 ? depth : 0;
    T->sk_width = threshold > 1 ? width : 0;
    T->sk_salt.clear();
    for (int j = 0; j < T->sk_depth; ++j) T->sk_salt.push_back(splitmix64_mix(seed + (uint64_t)(j + 1) * GOLDEN));
    T->sketch.assign((size_t)T->sk_depth * (size_t)T->sk_width, 0u);
    return 0;
}

// Recycling on or off; either way the free list starts empty.
int orc_set_recycling(void* h, int32_t on) {
    Table* T = (Table*)h;
    T->recycle = on != 0;
    T->free_rows.clear();
    T->free_next = 0;
    return 0;
}

// Rehash: keys whose row was last seen before min_clock leave the map (only
// with tracking on); with recycling on, the free list becomes every row
// below the row counter that no remaining key references, ascending.
// Returns the number of keys kept.
int64_t orc_rehash(void* h, uint32_t min_clock) {
    Table* T = (Table*)h;
    std::vector<char> referenced((size_t)T->n_rows, 0);
    int64_t kept = 0;
    for (auto& map : T->maps) {
        for (auto it = map.begin(); it != map.end();) {
            const int64_t off = it->second;
            if (!T->track || T->last_seen[off] >= min_clock) {
                referenced[off] = 1;
                ++kept;
                ++it;
            } else {
                it = map.erase(it);
            }
        }
    }
    if (T->recycle) {
        T->free_rows.clear();
        T->free_next = 0;
        for (int64_t o = 0; o < T->n_rows; ++o)
            if (!referenced[o]) T->free_rows.push_back(o);
    }
    return kept;
}

// Live entries (key, map index, offset) in no particular order; returns n.
int64_t orc_entries(void* h, int64_t* keys_out, int32_t* tabs_out, int64_t* offs_out) {
    Table* T = (Table*)h;
    int64_t q = 0;
    for (size_t m = 0; m < T->maps.size(); ++m) {
        for (auto& kv : T->maps[m]) {
            if (keys_out) {
                keys_out[q] = kv.first;
                tabs_out[q] = (int32_t)m;
                offs_out[q] = kv.second;
            }
            ++q;
        }
    }
    return q;
}

// Sketch counters [depth * width]; returns depth * width.
int64_t orc_sketch(void* h, uint32_t* out) {
    Table* T = (Table*)h;
    if (out) std::copy(T->sketch.begin(), T->sketch.end(), out);
    return (int64_t)T->sketch.size();
}

uint32_t orc_estimate(void* h, int64_t key, int32_t m) {
    Table* T = (Table*)h;
    return T->admission_on() ? T->estimate((uint64_t)key, m) : 0u;
}

// Row stamps [n_rows].
int orc_last_seen(void* h, uint32_t* out) {
    Table* T = (Table*)h;
    std::copy(T->last_seen.begin(), T->last_seen.end(), out);
    return 0;
}

// Free list: the rows not yet handed out, in order; returns their number
// (out may be null) and the number already handed out.
int64_t orc_free_list(void* h, int64_t* out, int64_t* handed_out) {
    Table* T = (Table*)h;
    const int64_t n = (int64_t)(T->free_rows.size() - T->free_next);
    if (out)
        for (int64_t q = 0; q < n; ++q) out[q] = T->free_rows[T->free_next + q];
    if (handed_out) *handed_out = (int64_t)T->free_next;
    return n;
}

double orc_init_value(uint64_t key, int32_t table, int32_t c, uint64_t seed, int32_t wdtype) {
    return init_value(key, table, c, seed, wdtype);
}

uint64_t orc_splitmix64_mix(uint64_t z) { return splitmix64_mix(z); }

uint16_t orc_round_bf16(double x) { return round_to_bf16(x); }

}  // extern "C"
