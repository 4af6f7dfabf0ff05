// The C ABI of libqlinear.so: argument validation (host only, before any HIP
// call), the per-shape config table, kernel-instance lookup and launch.
//
// Dispatch follows the approach of "Building a High-Performance and Portable
// vLLM Linear Backend with Helion" ("Kernel Implementation" section): the
// algorithm variant (Standard / Split-K / Swap-AB) and the low-level launch
// configuration are data chosen per input shape by an offline sweep, not a
// hand-written rule such as "Swap-AB below 32 tokens".  On the call path the
// choice is a table lookup keyed by (format, N, K) and the token count M.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cctype>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <memory>
#include <mutex>
#include <sstream>
#include <string>
#include <unordered_map>
#include <vector>

#include "qlin_internal.h"

#include "qlin_config_table.inc"   // kDefaultTable: the tuned table as text

using namespace qlin;

namespace {

const int64_t kMaxMN = int64_t(1) << 24;
const int64_t kMaxK = int64_t(1) << 20;
const int64_t kMaxKInt8 = (int64_t(1) << 17) - 16;   // |acc| <= K*128*128 < 2^31
const int64_t kMaxLd = (int64_t(1) << 31) - 1;

// Workspace layout: [counters: kCounterBytes][split partials].  The counter
// region sits at a fixed place for every config, so partials written by one
// config never land on the counters another config relies on being zero.
const size_t kCounterBytes = 128 * 1024;
// STREAM_TOK: LDS bytes for a workgroup's token rows, weight tiles per
// workgroup at most (kTokLds / kTokTiles in qlin_stream_tok.h).
const int64_t kTokLdsBytes = 80 * 1024;
const int64_t kTokTiles = 4;
const int64_t kMaxCounters = (int64_t)(kCounterBytes / 4);

int fmt_bit(int fmt, int scal)
{
    if (scal == SC_BLOCK)
        return FB_BLOCK;
    return fmt == FMT_INT8 ? FB_INT8 : FB_FP8;
}

const std::vector<Instance> &registry()
{
    static const std::vector<Instance> all = [] {
        std::vector<Instance> r;
        const Instance *(*fns[])(int *) = {
            stream_instances_fp8, stream_instances_int8, stream_instances_block,
            tile_instances_fp8, tile_instances_int8, tile_instances_block,
            stream_lds_instances_fp8, stream_lds_instances_int8, stream_lds_instances_block,
            tile_h_instances_fp8, tile_h_instances_int8, gemv_instances,
            stream_tok_instances_fp8, stream_tok_instances_int8, stream_own_instances,
        };
        for (auto f : fns) {
            int n = 0;
            const Instance *p = f(&n);
            r.insert(r.end(), p, p + n);
        }
        // Every LDS-ring instance also runs with spread row placement
        // (waves_n = 2): the same kernel, rows shared evenly over a grid
        // sized to the CU count instead of one tile of tile_n rows each.
        const size_t n = r.size();
        for (size_t i = 0; i < n; ++i)
            if (r[i].cfg.kernel == QLIN_KERNEL_STREAM_LDS) {
                Instance twin = r[i];
                twin.cfg.waves_n = 2;
                r.push_back(twin);
            }
        return r;
    }();
    return all;
}

// Compute units of the current device (256 on MI355X; also the answer when
// no device is visible, so host-only queries stay deterministic).
int cu_count()
{
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0)
        return v;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    cached.store(cus, std::memory_order_relaxed);
    return cus;
}

bool same_shape(const qlin_config &a, const qlin_config &b)
{
    return a.kernel == b.kernel && a.variant == b.variant && a.tile_m == b.tile_m &&
           a.tile_n == b.tile_n && a.tile_k == b.tile_k && a.waves_n == b.waves_n &&
           a.waves_k == b.waves_k && a.stages == b.stages;
}

const Instance *find_instance(int fmt, int scal, const qlin_config &c)
{
    const int bit = fmt_bit(fmt, scal);
    for (const Instance &in : registry())
        if ((in.fmt_mask & bit) && same_shape(in.cfg, c))
            return &in;
    return nullptr;
}

// ---------------------------------------------------------------------------
// Config table
// ---------------------------------------------------------------------------
struct Entry {
    int bit;
    bool grouped;        // a grouped (mixture-of-experts) call; M = rows-per-expert bound
    int64_t N, K, M;
    qlin_config cfg;
};

// The table in use.  A lookup reads it through an acquire load and never
// takes a lock; a replacement installs a new table and keeps every earlier
// one alive until the process ends, so a lookup that raced a replacement
// still reads valid memory (tables are a few KB and replaced rarely).
// Entries with an index from (grouped, format, N, K) to that shape's entries,
// so a lookup visits only the handful of tuned token counts of its shape.
struct Table {
    std::vector<Entry> entries;
    std::unordered_map<uint64_t, std::vector<const Entry *>> by_shape;
    size_t size() const { return entries.size(); }
};

uint64_t shape_key(bool grouped, int bit, int64_t N, int64_t K)
{
    return ((((uint64_t)grouped << 3 | (uint64_t)bit) << 25 | (uint64_t)N) << 21) | (uint64_t)K;
}

const std::vector<const Entry *> &entries_of(const Table &t, bool grouped, int bit, int64_t N,
                                             int64_t K)
{
    static const std::vector<const Entry *> none;
    if (N <= 0 || N > kMaxMN || K <= 0 || K > kMaxK)
        return none;
    const auto it = t.by_shape.find(shape_key(grouped, bit, N, K));
    return it == t.by_shape.end() ? none : it->second;
}

std::atomic<const Table *> g_table{nullptr};
std::once_flag g_table_once;
std::mutex g_table_mutex;                       // serialises replacements
std::vector<std::unique_ptr<Table>> g_tables;   // every table installed so far
std::atomic<int> g_log{0};

bool parse_table(const std::string &text, std::vector<Entry> &out)
{
    std::istringstream in(text);
    std::string line;
    std::vector<Entry> t;
    while (std::getline(in, line)) {
        const size_t h = line.find('#');
        if (h != std::string::npos)
            line.resize(h);
        std::istringstream ls(line);
        std::string fmt;
        if (!(ls >> fmt))
            continue;  // blank or comment
        Entry e;
        e.grouped = fmt == "grouped";
        if (e.grouped && !(ls >> fmt))
            return false;
        if (fmt == "fp8")
            e.bit = FB_FP8;
        else if (fmt == "int8")
            e.bit = FB_INT8;
        else if (fmt == "block_fp8")
            e.bit = FB_BLOCK;
        else
            return false;
        qlin_config &c = e.cfg;
        if (!(ls >> e.N >> e.K >> e.M >> c.kernel >> c.variant >> c.tile_m >> c.tile_n >> c.tile_k >>
              c.waves_n >> c.waves_k >> c.stages >> c.split_k >> c.reduce))
            return false;
        std::string extra;
        if (ls >> extra)
            return false;
        if (e.N <= 0 || e.K <= 0 || e.M <= 0)
            return false;
        if (e.grouped && e.cfg.split_k != 1)
            return false;   // grid.z of a grouped launch carries the expert
        t.push_back(e);
    }
    out.swap(t);
    return true;
}

void install_table(std::vector<Entry> entries)
{
    std::unique_ptr<Table> t(new Table);
    t->entries = std::move(entries);
    for (const Entry &e : t->entries)
        if (e.N <= kMaxMN && e.K <= kMaxK)
            t->by_shape[shape_key(e.grouped, e.bit, e.N, e.K)].push_back(&e);
    std::lock_guard<std::mutex> lk(g_table_mutex);
    g_tables.push_back(std::move(t));
    g_table.store(g_tables.back().get(), std::memory_order_release);
}

// First use: QLIN_LOG, then the table from QLIN_CONFIG when it names a
// readable, well-formed file, else the compiled-in one.
const Table &table()
{
    std::call_once(g_table_once, [] {
        const char *e = std::getenv("QLIN_LOG");
        g_log.store((e && *e && *e != '0') ? 1 : 0, std::memory_order_relaxed);
        std::vector<Entry> t;
        bool ok = false;
        const char *path = std::getenv("QLIN_CONFIG");
        if (path && *path) {
            std::ifstream f(path);
            if (f) {
                std::stringstream ss;
                ss << f.rdbuf();
                ok = parse_table(ss.str(), t);
            }
        }
        if (!ok)
            parse_table(kDefaultTable, t);
        install_table(std::move(t));
    });
    return *g_table.load(std::memory_order_acquire);
}

int ilog2_exact(int v)
{
    if (v <= 0 || (v & (v - 1)))
        return -1;
    int l = 0;
    while ((1 << l) < v)
        ++l;
    return l;
}

bool spread_rows(const qlin_config &c)
{
    return c.kernel == QLIN_KERNEL_STREAM_LDS && c.waves_n == 2;
}

// Stream kernels: grid (weight tiles, token tiles); tile kernel: one flat
// dimension over all output tiles (remapped in-kernel for XCD locality).
// Spread placement (LDS-ring kernel): 8-row units over a grid.x that is a
// multiple of the CUs left per (token tile, grid.z) slice, each workgroup
// taking at most tile_n rows.  `z` is grid.z (split_k, or 1 for grouped
// calls, whose grid.z holds the groups).
void grid_of(const qlin_config &c, int64_t M, int64_t N, int64_t z, int64_t *gx, int64_t *gy)
{
    const int64_t tn = (N + c.tile_n - 1) / c.tile_n;
    const int64_t tm = (M + c.tile_m - 1) / c.tile_m;
    if (c.kernel == QLIN_KERNEL_TILE) {
        *gx = tn * tm;
        *gy = 1;
    } else if (c.kernel == QLIN_KERNEL_STREAM_TOK) {
        // one workgroup per CU over (token tile, split), enough of them that
        // none holds more than kTokTiles tiles of 16 * waves_k rows
        const int64_t blocks = (N + 15) / 16;
        const int64_t per = std::max<int64_t>(1, cu_count() / (tm * std::max<int64_t>(1, z)));
        const int64_t need = (blocks + kTokTiles * c.waves_k - 1) / (kTokTiles * c.waves_k);
        *gx = std::max<int64_t>(1, std::min(blocks, std::max(per, need)));
        *gy = tm;
    } else if (spread_rows(c)) {
        const int64_t units = (N + 7) / 8;
        const int64_t need = (units + c.tile_n / 8 - 1) / (c.tile_n / 8);
        const int64_t slots = std::max<int64_t>(1, cu_count() / (tm * std::max<int64_t>(1, z)));
        *gx = std::min(units, (need + slots - 1) / slots * slots);
        *gy = tm;
    } else {
        *gx = tn;
        *gy = tm;
    }
}

// Built-in choice for shapes the table does not cover.
qlin_config default_config(int fmt, int scal, int64_t M, int64_t N, int64_t K)
{
    qlin_config c;
    std::memset(&c, 0, sizeof c);
    const int64_t KS = (K + 127) / 128;
    bool have_tile = false;
    for (const Instance &in : registry())
        if (in.cfg.kernel == QLIN_KERNEL_TILE && (in.fmt_mask & fmt_bit(fmt, scal)))
            have_tile = true;
    const bool tc = scal == SC_TC;
    if (M > 64 && have_tile && K % 128 == 0) {
        // Largest tile that still gives most CUs a tile of their own; the
        // sweep's picks at the tuned prefill points follow the same pattern
        // (256x256 for big M*N, 128x128 at 4 stages, else 64x128 at 4 stages).
        const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
        c.kernel = QLIN_KERNEL_TILE;
        c.variant = QLIN_SWAP_AB;          // built for all three formats
        c.tile_k = 128;
        if (tc && M >= 1024 && t128 >= 512) {
            c.tile_m = 256, c.tile_n = 256, c.waves_n = 2, c.waves_k = 4, c.stages = 2;
        } else if (t128 >= 192 || !tc) {
            c.tile_m = 128, c.tile_n = 128, c.waves_n = 2, c.waves_k = 2, c.stages = tc ? 4 : 2;
            if (!tc && t128 < 192)
                c.tile_m = 64, c.waves_n = 1, c.waves_k = 4;
        } else {
            c.tile_m = 64, c.tile_n = 128, c.waves_n = 1, c.waves_k = 4, c.stages = 4;
        }
    } else {
        // 16 weight rows per workgroup, 4 waves splitting K, 4 steps of loads
        // in flight per wave: the shape the sweep picks for most decode points.
        c.kernel = QLIN_KERNEL_STREAM;
        c.variant = QLIN_SWAP_AB;
        c.tile_m = M <= 16 ? 16 : 32;
        c.tile_n = 16;
        c.tile_k = 512;
        c.waves_n = 1;
        c.waves_k = 4;
        c.stages = 2;
    }
    int64_t gx, gy;
    grid_of(c, M, N, c.split_k, &gx, &gy);
    const int64_t kw = c.kernel == QLIN_KERNEL_STREAM ? c.waves_k : 1;
    // Split K until the grid covers the CUs (tiles: half of them; a tile's
    // workgroup holds a whole CU's LDS), keeping >= 8 K steps per split for
    // tiles.
    const int64_t want = c.kernel == QLIN_KERNEL_TILE ? 128 : 256;
    const int64_t min_steps = c.kernel == QLIN_KERNEL_TILE ? 8 : 1;
    int split = 1;
    while (gx * gy * split < want && split * 2 <= 256 && split * 2 * kw * min_steps <= KS)
        split *= 2;
    c.split_k = split;
    if (c.kernel == QLIN_KERNEL_TILE && split > 1)
        c.reduce = QLIN_REDUCE_TWO_PASS;   // what the sweep picks for split tiles
    else
        c.reduce = gx * gy <= kMaxCounters ? QLIN_REDUCE_LAST_ARRIVER : QLIN_REDUCE_TWO_PASS;
    return c;
}

qlin_status check_config(int fmt, int scal, int64_t M, int64_t N, int64_t K,
                         const qlin_config &c, const Instance **inst);

// Grouped (mixture-of-experts) calls: split_k = 1 (grid.z is the expert).
// The config comes from the table's grouped entries, tuned per (format, N,
// K, rows-per-expert bound) on 128-expert layers.  Shapes without entries
// use a rule read off an earlier sweep of every instance over (K, N) =
// (2048, 1536) and (768, 2048) at 1-52 rows per expert: up to 3 rows the
// GEMV kernel when K >= 2048 and otherwise the LDS-ring stream kernel with
// 8-token tiles, the register stream kernel with 16x64 tiles up to 16, a
// 64x128 tile up to 64 and a 128x128 tile beyond; a choice the library
// lacks for the format falls back to the table's config with split_k = 1.
qlin_config grouped_config(int fmt, int scal, int64_t M, int64_t N, int64_t K);

qlin_config select_config(int fmt, int scal, int64_t M, int64_t N, int64_t K)
{
    const int bit = fmt_bit(fmt, scal);
    const Entry *best = nullptr, *largest = nullptr;
    for (const Entry *e : entries_of(table(), false, bit, N, K)) {
        if (e->M >= M && (!best || e->M < best->M))
            best = e;
        if (!largest || e->M > largest->M)
            largest = e;
    }
    // Beyond the tuned M range the largest entry is used, unless the call is
    // a prefill far past tables tuned only for decode (M <= 64), where a
    // decode config would re-stream the weights once per 16-32 tokens.
    if (!best && largest && !(M > 64 && M > 2 * largest->M))
        best = largest;
    // An entry that does not fit this M (or names an instance the library
    // lacks) falls back to the built-in default rather than failing.
    if (best && check_config(fmt, scal, M, N, K, best->cfg, nullptr) == QLIN_OK)
        return best->cfg;
    return default_config(fmt, scal, M, N, K);
}

qlin_config grouped_config(int fmt, int scal, int64_t M, int64_t N, int64_t K)
{
    // Tuned entries first: the one for (fmt, N, K) with the smallest
    // rows-per-expert bound >= M, else the largest bound.
    const int bit = fmt_bit(fmt, scal);
    const Entry *best = nullptr, *largest = nullptr;
    for (const Entry *e : entries_of(table(), true, bit, N, K)) {
        if (e->M >= M && (!best || e->M < best->M))
            best = e;
        if (!largest || e->M > largest->M)
            largest = e;
    }
    if (!best)
        best = largest;
    if (best && check_config(fmt, scal, M, N, K, best->cfg, nullptr) == QLIN_OK)
        return best->cfg;
    auto make = [](int kernel, int tm, int tn, int tk, int wn, int wk, int st) {
        qlin_config c;
        std::memset(&c, 0, sizeof c);
        c.kernel = kernel;
        c.variant = QLIN_SWAP_AB;
        c.tile_m = tm, c.tile_n = tn, c.tile_k = tk;
        c.waves_n = wn, c.waves_k = wk, c.stages = st;
        c.split_k = 1;
        c.reduce = QLIN_REDUCE_LAST_ARRIVER;
        return c;
    };
    qlin_config pick =
        M <= 3 && K >= 2048 && scal == SC_TC ? make(QLIN_KERNEL_GEMV, M == 1 ? 1 : 2, 8, 2048, 1, 4, 2)
        : M <= 3  ? make(QLIN_KERNEL_STREAM_LDS, 8, 16, 512, 1, 4, 4)
        : M <= 16 ? make(QLIN_KERNEL_STREAM, 16, 64, 128, 1, 4, 2)
        : M <= 64 ? (scal == SC_TC ? make(QLIN_KERNEL_TILE, 64, 128, 128, 1, 4, 4)
                                   : make(QLIN_KERNEL_TILE, 64, 128, 128, 1, 4, 2))
                  : make(QLIN_KERNEL_TILE, 128, 128, 128, 2, 2, 2);
    if (pick.kernel == QLIN_KERNEL_GEMV)
        pick.variant = QLIN_STANDARD;     // the GEMV kernel has no Swap-AB form
    if (check_config(fmt, scal, M, N, K, pick, nullptr) == QLIN_OK)
        return pick;
    qlin_config c = select_config(fmt, scal, M, N, K);
    c.split_k = 1;
    c.reduce = QLIN_REDUCE_LAST_ARRIVER;
    return c;
}

qlin_status check_config(int fmt, int scal, int64_t M, int64_t N, int64_t K,
                         const qlin_config &c, const Instance **inst)
{
    const Instance *in = find_instance(fmt, scal, c);
    if (!in)
        return QLIN_ERR_BAD_CONFIG;
    const int64_t KS = (K + 127) / 128;
    if (ilog2_exact(c.split_k) < 0 || c.split_k > 256 || c.split_k > KS)
        return QLIN_ERR_BAD_CONFIG;
    if (c.reduce != QLIN_REDUCE_TWO_PASS && c.reduce != QLIN_REDUCE_LAST_ARRIVER)
        return QLIN_ERR_BAD_CONFIG;
    if (c.kernel == QLIN_KERNEL_TILE && K % 128 != 0)
        return QLIN_ERR_BAD_CONFIG;   // the LDS ring copies whole 128-byte K steps
    if (c.kernel == QLIN_KERNEL_STREAM_LDS && (K % 256 != 0 || c.split_k > K / 256))
        return QLIN_ERR_BAD_CONFIG;   // 256-byte K units keep the LDS swizzle in range
    if (c.kernel == QLIN_KERNEL_GEMV && c.split_k != 1)
        return QLIN_ERR_BAD_CONFIG;   // a wave covers a weight row's whole K
    if (c.kernel == QLIN_KERNEL_STREAM_TOK) {
        if (K % 256 != 0 || c.split_k > K / 256)
            return QLIN_ERR_BAD_CONFIG;
        const int64_t units = (K / 256 + c.split_k - 1) / c.split_k;
        if (units * 256 * c.tile_m > kTokLdsBytes)
            return QLIN_ERR_BAD_CONFIG;   // the split's token rows must fit the LDS area
        if (c.split_k > 1 && c.reduce != QLIN_REDUCE_TWO_PASS)
            return QLIN_ERR_BAD_CONFIG;   // partials are combined by the second pass
    }
    int64_t gx, gy;
    grid_of(c, M, N, c.split_k, &gx, &gy);
    if (gx > 0x7fffffff || gy > 65535)
        return QLIN_ERR_BAD_CONFIG;
    if (c.split_k > 1 && c.reduce == QLIN_REDUCE_LAST_ARRIVER && gx * gy > kMaxCounters)
        return QLIN_ERR_BAD_CONFIG;   // one counter per output tile must fit its region
    if (inst)
        *inst = in;
    return QLIN_OK;
}

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

size_t ws_bytes(const qlin_config &c, int64_t M, int64_t N)
{
    if (c.split_k <= 1 || M == 0 || N == 0)
        return 0;
    return kCounterBytes + round256((size_t)c.split_k * (size_t)M * (size_t)N * 4);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

qlin_status validate(const Problem &pb)
{
    if (pb.fmt != FMT_E4M3 && pb.fmt != FMT_INT8)
        return QLIN_ERR_BAD_ARGUMENT;
    if (pb.scal == SC_BLOCK && pb.fmt != FMT_E4M3)
        return QLIN_ERR_BAD_ARGUMENT;
    if (pb.M < 0 || pb.N < 0 || pb.M > kMaxMN || pb.N > kMaxMN)
        return QLIN_ERR_BAD_SHAPE;
    if (pb.K <= 0 || pb.K % 16 != 0 || pb.K > kMaxK)
        return QLIN_ERR_BAD_SHAPE;
    if (pb.fmt == FMT_INT8 && pb.K > kMaxKInt8)
        return QLIN_ERR_BAD_SHAPE;
    if (pb.scal == SC_BLOCK && (pb.K % 128 != 0 || pb.N % 128 != 0))
        return QLIN_ERR_BAD_SHAPE;
    if (pb.M == 0 || pb.N == 0)
        return QLIN_OK;
    const bool raw = pb.acc_out != nullptr;
    if (!pb.A || !pb.B || (!raw && (!pb.sA || !pb.sB || !pb.Y)))
        return QLIN_ERR_NULL_POINTER;
    if (pb.lda < pb.K || pb.ldb < pb.K || pb.lda % 16 || pb.ldb % 16 || pb.lda > kMaxLd ||
        pb.ldb > kMaxLd)
        return QLIN_ERR_BAD_STRIDE;
    if (raw ? (pb.ldacc < pb.N || pb.ldacc > kMaxLd) : (pb.ldy < pb.N || pb.ldy > kMaxLd))
        return QLIN_ERR_BAD_STRIDE;
    if (!aligned(pb.A, 16) || !aligned(pb.B, 16))
        return QLIN_ERR_MISALIGNED;
    if (raw ? !aligned(pb.acc_out, 16)
            : (!aligned(pb.Y, 16) || !aligned(pb.sA, 4) || !aligned(pb.sB, 4)))
        return QLIN_ERR_MISALIGNED;
    return QLIN_OK;
}

qlin_status run(const Problem &pb, const qlin_config *cfg_in)
{
    qlin_status st = validate(pb);
    if (st != QLIN_OK)
        return st;
    if (pb.M == 0 || pb.N == 0)
        return cfg_in ? (find_instance(pb.fmt, pb.scal, *cfg_in) ? QLIN_OK : QLIN_ERR_BAD_CONFIG)
                      : QLIN_OK;
    const bool grouped = pb.groups > 0;
    if (grouped) {
        if (pb.groups > 65535)
            return QLIN_ERR_BAD_SHAPE;
        if (!pb.group_off)
            return QLIN_ERR_NULL_POINTER;
        if (!aligned(pb.group_off, 4))
            return QLIN_ERR_MISALIGNED;
        if (pb.b_gstride < 0 || pb.b_gstride % 16 || pb.sb_gstride < 0)
            return QLIN_ERR_BAD_STRIDE;
        if (cfg_in && cfg_in->split_k != 1)
            return QLIN_ERR_BAD_CONFIG;   // grid.z carries the group
        if (cfg_in && cfg_in->kernel == QLIN_KERNEL_STREAM_TOK)
            return QLIN_ERR_BAD_CONFIG;   // its grid.z is the split and it has no group entry
    }
    const qlin_config cfg = cfg_in    ? *cfg_in
                            : grouped ? grouped_config(pb.fmt, pb.scal, pb.M, pb.N, pb.K)
                                      : select_config(pb.fmt, pb.scal, pb.M, pb.N, pb.K);
    const Instance *inst = nullptr;
    st = check_config(pb.fmt, pb.scal, pb.M, pb.N, pb.K, cfg, &inst);
    if (st != QLIN_OK)
        return st;
    const size_t need = ws_bytes(cfg, pb.M, pb.N);
    if (need) {
        if (!pb.ws || pb.ws_bytes < need)
            return QLIN_ERR_WORKSPACE;
        if (!aligned(pb.ws, 16))
            return QLIN_ERR_MISALIGNED;
    }
    if (g_log.load(std::memory_order_relaxed) > 0)
        std::fprintf(stderr,
                     "[qlinear] fmt=%d scal=%d M=%lld N=%lld K=%lld -> kernel=%d variant=%d "
                     "tile=%dx%dx%d waves=%dx%d stages=%d split_k=%d reduce=%d\n",
                     pb.fmt, pb.scal, (long long)pb.M, (long long)pb.N, (long long)pb.K, cfg.kernel,
                     cfg.variant, cfg.tile_m, cfg.tile_n, cfg.tile_k, cfg.waves_n, cfg.waves_k,
                     cfg.stages, cfg.split_k, cfg.reduce);

    KArgs a;
    std::memset(&a, 0, sizeof a);
    a.A = static_cast<const uint8_t *>(pb.A);
    a.B = static_cast<const uint8_t *>(pb.B);
    a.sA = pb.sA;
    a.sB = pb.sB;
    a.Y = static_cast<uint16_t *>(pb.Y);
    a.acc_out = pb.acc_out;
    a.M = (int)pb.M;
    a.N = (int)pb.N;
    a.K = (int)pb.K;
    a.lda = (int)pb.lda;
    a.ldb = (int)pb.ldb;
    a.ldy = (int)pb.ldy;
    a.ldacc = (int)pb.ldacc;
    a.G = (int)(pb.K / 128);
    a.split_k = cfg.split_k;
    const int64_t KS = (pb.K + 127) / 128;
    a.steps_per_split = (int)((KS + cfg.split_k - 1) / cfg.split_k);
    a.reduce = cfg.reduce;
    if (cfg.split_k > 1) {
        a.counters = static_cast<int32_t *>(pb.ws);
        a.part = static_cast<char *>(pb.ws) + kCounterBytes;
    }
    if (grouped) {
        a.group_off = pb.group_off;
        a.b_gstride = pb.b_gstride;
        a.sb_gstride = pb.sb_gstride;
    }
    int64_t gx, gy;
    grid_of(cfg, pb.M, pb.N, grouped ? 1 : cfg.split_k, &gx, &gy);
    if (spread_rows(cfg))
        a.nspread = (int)((pb.N + 7) / 8);
    const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)(grouped ? pb.groups : cfg.split_k));
    hipError_t e = inst->fn(a, grid, pb.stream);
    if (e == hipSuccess && cfg.split_k > 1 && cfg.reduce == QLIN_REDUCE_TWO_PASS)
        e = launch_reduce(pb.fmt, pb.scal, a, pb.stream);
    return e == hipSuccess ? QLIN_OK : QLIN_ERR_HIP;
}

Problem make_problem(int fmt, int scal, int64_t M, int64_t N, int64_t K, const void *A,
                     int64_t lda, const float *sA, const void *B, int64_t ldb, const float *sB,
                     void *Y, int64_t ldy, void *ws, size_t wsb, void *stream)
{
    Problem pb;
    std::memset(&pb, 0, sizeof pb);
    pb.fmt = fmt;
    pb.scal = scal;
    pb.M = M;
    pb.N = N;
    pb.K = K;
    pb.A = A;
    pb.lda = lda;
    pb.sA = sA;
    pb.B = B;
    pb.ldb = ldb;
    pb.sB = sB;
    pb.Y = Y;
    pb.ldy = ldy;
    pb.ws = ws;
    pb.ws_bytes = wsb;
    pb.stream = static_cast<hipStream_t>(stream);
    return pb;
}

int fmt_of(qlin_dtype dt) { return dt == QLIN_INT8 ? FMT_INT8 : (dt == QLIN_E4M3 ? FMT_E4M3 : -1); }

}  // namespace

namespace qlin {

qlin_status run_problem(const Problem &pb, const qlin_config *cfg) { return run(pb, cfg); }

qlin_status check_problem(const Problem &pb) { return validate(pb); }

Problem problem(int fmt, int scal, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                const float *sA, const void *B, int64_t ldb, const float *sB, void *Y,
                int64_t ldy, void *ws, size_t ws_bytes, void *stream)
{
    return make_problem(fmt, scal, M, N, K, A, lda, sA, B, ldb, sB, Y, ldy, ws, ws_bytes, stream);
}

size_t selected_workspace_bytes(int fmt, int scal, int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0)
        return 0;
    return ws_bytes(select_config(fmt, scal, M, N, K), M, N);
}

size_t counter_bytes() { return kCounterBytes; }

}  // namespace qlin

extern "C" {

qlin_status qlin_scaled_mm_cfg(qlin_dtype dt, int64_t M, int64_t N, int64_t K, const void *A,
                               int64_t lda, const float *a_scale, const void *B, int64_t ldb,
                               const float *b_scale, void *Y, int64_t ldy, void *workspace,
                               size_t workspace_bytes, void *stream, const qlin_config *cfg)
{
    const int fmt = fmt_of(dt);
    if (fmt < 0)
        return QLIN_ERR_BAD_ARGUMENT;
    return run(make_problem(fmt, SC_TC, M, N, K, A, lda, a_scale, B, ldb, b_scale, Y, ldy,
                            workspace, workspace_bytes, stream),
               cfg);
}

qlin_status qlin_scaled_mm(qlin_dtype dt, int64_t M, int64_t N, int64_t K, const void *A,
                           int64_t lda, const float *a_scale, const void *B, int64_t ldb,
                           const float *b_scale, void *Y, int64_t ldy, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    return qlin_scaled_mm_cfg(dt, M, N, K, A, lda, a_scale, B, ldb, b_scale, Y, ldy, workspace,
                              workspace_bytes, stream, nullptr);
}

qlin_status qlin_block_scaled_mm_cfg(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                                     const float *a_scale, const void *B, int64_t ldb,
                                     const float *b_scale, void *Y, int64_t ldy, void *workspace,
                                     size_t workspace_bytes, void *stream, const qlin_config *cfg)
{
    return run(make_problem(FMT_E4M3, SC_BLOCK, M, N, K, A, lda, a_scale, B, ldb, b_scale, Y, ldy,
                            workspace, workspace_bytes, stream),
               cfg);
}

qlin_status qlin_block_scaled_mm(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                                 const float *a_scale, const void *B, int64_t ldb,
                                 const float *b_scale, void *Y, int64_t ldy, void *workspace,
                                 size_t workspace_bytes, void *stream)
{
    return qlin_block_scaled_mm_cfg(M, N, K, A, lda, a_scale, B, ldb, b_scale, Y, ldy, workspace,
                                    workspace_bytes, stream, nullptr);
}

qlin_status qlin_grouped_scaled_mm(qlin_dtype dt, int64_t groups, const int32_t *group_offsets,
                                   int64_t max_rows, int64_t N, int64_t K, const void *A,
                                   int64_t lda, const float *a_scale, const void *B, int64_t ldb,
                                   int64_t b_group_stride, const float *b_scale,
                                   int64_t b_scale_group_stride, void *Y, int64_t ldy, void *stream,
                                   const qlin_config *cfg)
{
    const int fmt = fmt_of(dt);
    if (fmt < 0)
        return QLIN_ERR_BAD_ARGUMENT;
    if (groups < 0)
        return QLIN_ERR_BAD_SHAPE;
    if (groups == 0)
        return QLIN_OK;
    Problem pb = make_problem(fmt, SC_TC, max_rows, N, K, A, lda, a_scale, B, ldb, b_scale, Y, ldy,
                              nullptr, 0, stream);
    pb.groups = groups;
    pb.group_off = group_offsets;
    pb.b_gstride = b_group_stride;
    pb.sb_gstride = b_scale_group_stride;
    return run(pb, cfg);
}

qlin_status qlin_grouped_block_scaled_mm(int64_t groups, const int32_t *group_offsets,
                                         int64_t max_rows, int64_t N, int64_t K, const void *A,
                                         int64_t lda, const float *a_scale, const void *B,
                                         int64_t ldb, int64_t b_group_stride, const float *b_scale,
                                         int64_t b_scale_group_stride, void *Y, int64_t ldy,
                                         void *stream, const qlin_config *cfg)
{
    if (groups < 0)
        return QLIN_ERR_BAD_SHAPE;
    if (groups == 0)
        return QLIN_OK;
    Problem pb = make_problem(FMT_E4M3, SC_BLOCK, max_rows, N, K, A, lda, a_scale, B, ldb, b_scale,
                              Y, ldy, nullptr, 0, stream);
    pb.groups = groups;
    pb.group_off = group_offsets;
    pb.b_gstride = b_group_stride;
    pb.sb_gstride = b_scale_group_stride;
    return run(pb, cfg);
}

qlin_status qlin_int8_accumulate(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                                 const void *B, int64_t ldb, int32_t *acc, int64_t ldacc,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const qlin_config *cfg)
{
    Problem pb = make_problem(FMT_INT8, SC_TC, M, N, K, A, lda, nullptr, B, ldb, nullptr, nullptr,
                              0, workspace, workspace_bytes, stream);
    pb.acc_out = acc;
    pb.ldacc = ldacc;
    if (!acc && M > 0 && N > 0)
        return QLIN_ERR_NULL_POINTER;
    return run(pb, cfg);
}

qlin_status qlin_select_config(qlin_scaling sc, qlin_dtype dt, int64_t M, int64_t N, int64_t K,
                               qlin_config *out)
{
    const int fmt = fmt_of(dt);
    if (fmt < 0 || (sc != QLIN_TOKEN_CHANNEL && sc != QLIN_BLOCK128) ||
        (sc == QLIN_BLOCK128 && fmt != FMT_E4M3))
        return QLIN_ERR_BAD_ARGUMENT;
    if (!out)
        return QLIN_ERR_NULL_POINTER;
    if (M < 0 || N < 0 || K <= 0)
        return QLIN_ERR_BAD_SHAPE;
    *out = select_config(fmt, sc == QLIN_BLOCK128 ? SC_BLOCK : SC_TC, M, N, K);
    return QLIN_OK;
}

qlin_status qlin_select_grouped_config(qlin_scaling sc, qlin_dtype dt, int64_t max_rows, int64_t N,
                                       int64_t K, qlin_config *out)
{
    const int fmt = fmt_of(dt);
    if (fmt < 0 || (sc != QLIN_TOKEN_CHANNEL && sc != QLIN_BLOCK128) ||
        (sc == QLIN_BLOCK128 && fmt != FMT_E4M3))
        return QLIN_ERR_BAD_ARGUMENT;
    if (!out)
        return QLIN_ERR_NULL_POINTER;
    *out = grouped_config(fmt, sc == QLIN_BLOCK128 ? SC_BLOCK : SC_TC, max_rows, N, K);
    return QLIN_OK;
}

qlin_status qlin_check_config(qlin_scaling sc, qlin_dtype dt, int64_t M, int64_t N, int64_t K,
                              const qlin_config *cfg)
{
    const int fmt = fmt_of(dt);
    if (fmt < 0 || (sc != QLIN_TOKEN_CHANNEL && sc != QLIN_BLOCK128) ||
        (sc == QLIN_BLOCK128 && fmt != FMT_E4M3))
        return QLIN_ERR_BAD_ARGUMENT;
    if (!cfg)
        return QLIN_ERR_NULL_POINTER;
    if (M < 0 || N < 0 || K <= 0 || K % 16)
        return QLIN_ERR_BAD_SHAPE;
    return check_config(fmt, sc == QLIN_BLOCK128 ? SC_BLOCK : SC_TC, M, N, K, *cfg, nullptr);
}

size_t qlin_workspace_size(qlin_scaling sc, qlin_dtype dt, int64_t M, int64_t N, int64_t K,
                           const qlin_config *cfg)
{
    const int fmt = fmt_of(dt);
    if (fmt < 0 || M <= 0 || N <= 0 || K <= 0)
        return 0;
    const int scal = sc == QLIN_BLOCK128 ? SC_BLOCK : SC_TC;
    const qlin_config c = cfg ? *cfg : select_config(fmt, scal, M, N, K);
    return ws_bytes(c, M, N);
}

qlin_status qlin_kernel_instance(int32_t i, qlin_config *out, int32_t *fmt_mask)
{
    const std::vector<Instance> &r = registry();
    if (i < 0 || (size_t)i >= r.size())
        return QLIN_ERR_BAD_ARGUMENT;
    if (!out || !fmt_mask)
        return QLIN_ERR_NULL_POINTER;
    *out = r[i].cfg;
    *fmt_mask = r[i].fmt_mask;
    return QLIN_OK;
}

qlin_status qlin_load_config_table(const char *path)
{
    std::vector<Entry> t;
    if (!path || !*path) {
        parse_table(kDefaultTable, t);
    } else {
        std::ifstream f(path);
        if (!f)
            return QLIN_ERR_CONFIG_FILE;
        std::stringstream ss;
        ss << f.rdbuf();
        if (!parse_table(ss.str(), t))
            return QLIN_ERR_CONFIG_FILE;
    }
    table();            // the first-use load must not replace this table later
    install_table(std::move(t));
    return QLIN_OK;
}

int32_t qlin_config_table_size(void)
{
    return (int32_t)table().size();
}

const char *qlin_status_string(qlin_status s)
{
    switch (s) {
    case QLIN_OK: return "ok";
    case QLIN_ERR_NULL_POINTER: return "null pointer";
    case QLIN_ERR_BAD_SHAPE: return "bad shape";
    case QLIN_ERR_BAD_STRIDE: return "bad leading dimension";
    case QLIN_ERR_MISALIGNED: return "misaligned pointer";
    case QLIN_ERR_WORKSPACE: return "workspace missing or too small";
    case QLIN_ERR_BAD_CONFIG: return "invalid or unbuilt config";
    case QLIN_ERR_CONFIG_FILE: return "config table file unreadable or malformed";
    case QLIN_ERR_HIP: return "HIP launch failed";
    case QLIN_ERR_BAD_ARGUMENT: return "bad argument";
    }
    return "unknown status";
}

int32_t qlin_abi_version(void) { return QLINEAR_ABI_VERSION; }

int32_t qlin_stream_capture_id(void *stream, unsigned long long *capture_id)
{
    if (!capture_id)
        return -1;
    *capture_id = 0;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    if (hipStreamGetCaptureInfo(static_cast<hipStream_t>(stream), &st, &id) != hipSuccess)
        return -1;
    if (st != hipStreamCaptureStatusActive)
        return 0;
    *capture_id = id;
    return 1;
}

}  // extern "C"
