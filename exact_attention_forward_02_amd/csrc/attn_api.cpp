// attn_api.cpp -- C ABI of the gfx950 fused attention forward and of its
// split-key variant and merge (declared in include/attn_fwd.h): argument
// validation, device checks, the tile schedule parameters, and the launches
// on the caller's stream.

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "attn_fwd.h"
#include "attn_params.h"

namespace {

static_assert(attn::kBwdScratchRows == ATTN_BWD_NOALLOC_MAX_ROWS,
              "the header states the scratch size of attn_bwd_noalloc");
constexpr int kAbiVersion = 8;
constexpr int kMaxSplits = 4096;
constexpr int kMaxDevices = 64;
constexpr int kXcds = 8;                 // MI355X: 8 accelerator complex dies
constexpr int kTilesPerXcdWave = 32;     // concurrent workgroups per XCD (32 CUs x 1)
constexpr float kDefaultThreshold = 8.0f;  // log2 units: a factor of 256
constexpr int kTileOverhead = 2;         // per-tile cost beyond its key blocks (Q in, O out),
                                         // in key-block units, for the varlen schedule

// -1 unknown, 0 not gfx950, 1 gfx950
std::atomic<int> g_arch_ok[kMaxDevices];
// compute units of each device (0 unknown)
std::atomic<int> g_cu_count[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Launch log: with ATTN_LOG set to a non-empty value other than "0", every
// launch prints its kernel, instantiation and grid to stderr.  Off by default.
bool log_enabled() {
    static const bool on = [] {
        const char* e = getenv("ATTN_LOG");
        return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
    }();
    return on;
}
void log_launch(const char* fmt, ...) {
    if (!log_enabled()) return;
    va_list ap;
    va_start(ap, fmt);
    fputs("[attn] ", stderr);
    vfprintf(stderr, fmt, ap);
    fputc('\n', stderr);
    va_end(ap);
}

// Element strides of the four 16-bit tensors: (batch, head, row), head dim contiguous.
struct Strides {
    attn_strides q, k, v, o;
};

Strides contiguous_strides(int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v) {
    Strides st;
    st.q = {(long long)Hq * Lq * d_qk, (long long)Lq * d_qk, d_qk};
    st.k = {(long long)Hkv * Lk * d_qk, (long long)Lk * d_qk, d_qk};
    st.v = {(long long)Hkv * Lk * d_v, (long long)Lk * d_v, d_v};
    st.o = {(long long)Hq * Lq * d_v, (long long)Lq * d_v, d_v};
    return st;
}

// Strides are non-negative multiples of 8 elements (16 bytes, so every row
// starts 16-byte aligned), rows at least a head-dim apart, and every element
// offset and the byte extent of the rows the kernel addresses with 32-bit
// offsets (one K or V head, 32 rows of Q) fits.
int check_strides(const Strides& st, int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v) {
    const attn_strides* all[4] = {&st.q, &st.k, &st.v, &st.o};
    const int dims[4] = {d_qk, d_qk, d_v, d_v};
    const long long heads[4] = {Hq, Hkv, Hkv, Hq};
    const long long rows[4] = {Lq, Lk, Lk, Lq};
    for (int t = 0; t < 4; ++t) {
        const attn_strides& a = *all[t];
        if (a.batch < 0 || a.head < 0 || a.row < dims[t]) return ATTN_ERR_BAD_STRIDE;
        if (a.batch % 8 || a.head % 8 || a.row % 8) return ATTN_ERR_BAD_STRIDE;
        if (a.row > INT32_MAX) return ATTN_ERR_TOO_LARGE;
        // largest element offset, in 64-bit arithmetic without overflow
        const double last = (double)(B - 1) * a.batch + (double)(heads[t] - 1) * a.head +
                            (double)(rows[t] - 1) * a.row + dims[t];
        if (last > 9.0e18) return ATTN_ERR_TOO_LARGE;
    }
    const long long k_extent = (long long)(Lk - 1) * st.k.row * 2 + d_qk * 2;
    const long long v_extent = (long long)(Lk - 1) * st.v.row * 2 + d_v * 2;
    const long long q_extent = 31LL * st.q.row * 2 + d_qk * 2;
    if (k_extent > INT32_MAX || v_extent > INT32_MAX || q_extent > INT32_MAX)
        return ATTN_ERR_TOO_LARGE;
    return ATTN_OK;
}

int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v, float scale) {
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_PTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1) return ATTN_ERR_BAD_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
    const bool dims_ok = (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) ||
                         (d_qk == 192 && d_v == 128);
    if (!dims_ok) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    if (!(scale > 0.0f) || !isfinite(scale)) return ATTN_ERR_BAD_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return ATTN_ERR_MISALIGNED;
    // row counts must fit 32-bit row indices in the kernel
    const long long q_rows = (long long)B * Hq * Lq;
    const long long kv_rows = (long long)B * Hkv * Lk;
    if (q_rows > INT32_MAX || kv_rows > INT32_MAX) return ATTN_ERR_TOO_LARGE;
    return ATTN_OK;
}

// Checks that the current device is a gfx950 and reports its compute units.
int check_device(int* n_cu = nullptr) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return ATTN_ERR_NO_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED_ARCH;
    int ok = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (ok < 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_HIP;
        ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
        g_cu_count[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 0,
                              std::memory_order_relaxed);
        g_arch_ok[dev].store(ok, std::memory_order_relaxed);
    }
    if (n_cu) *n_cu = g_cu_count[dev].load(std::memory_order_relaxed);
    return ok ? ATTN_OK : ATTN_ERR_UNSUPPORTED_ARCH;
}

// Largest divisor of n that is <= cap (at least 1).
int largest_divisor_at_most(int n, int cap) {
    for (int d = cap < n ? cap : n; d > 1; --d)
        if (n % d == 0) return d;
    return 1;
}

// 64 * ceil(ceil(Lk / 64) / n_split): keys per split
int split_keys(int Lk, int n_split) {
    const int nb = (Lk + attn::kBlockN - 1) / attn::kBlockN;
    return attn::kBlockN * ((nb + n_split - 1) / n_split);
}

// Heads of one K/V head packed into a workgroup: Gp divides G and the 8 waves.
int packed_heads(int G) { return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1; }

// The kernel divides by these launch constants with a multiply and a shift.
void set_divisors(attn::FwdParams& p) {
    p.div_sec = attn::make_fast_div((uint32_t)(p.sec_units * p.n_m));
    p.div_sec_units = attn::make_fast_div((uint32_t)p.sec_units);
    p.div_units_kv = attn::make_fast_div((uint32_t)p.units_kv);
    p.div_hg = attn::make_fast_div((uint32_t)p.n_hg);
    p.div_hkv = attn::make_fast_div((uint32_t)p.Hkv);
    p.div_gp = attn::make_fast_div((uint32_t)p.Gp);
}

int fill_schedule(attn::FwdParams& p, bool causal) {
    p.G = p.Hq / p.Hkv;
    // query heads that share a K/V head are packed into one workgroup, one
    // head per wave group, so the K/V block is loaded once for all of them
    p.Gp = packed_heads(p.G);
    p.n_hg = p.G / p.Gp;
    p.bm_pos = attn::kRowsPerWave * attn::kWaves / p.Gp;
    p.n_m = (p.Lq + p.bm_pos - 1) / p.bm_pos;
    const long long units_kv = (long long)p.B * p.Hkv * p.n_hg;
    const long long units = units_kv * p.n_split;
    const long long tiles = units * p.n_m;
    if (tiles > INT32_MAX) return ATTN_ERR_TOO_LARGE;
    p.units_kv = (int)units_kv;
    p.units = (int)units;
    // XCD-aware order: workgroup i is dispatched to XCD i % 8; give each XCD
    // a contiguous range of units so the K/V blocks it streams stay in its L2.
    // Under the causal mask the key splits of a head differ in work (a late
    // split holds keys only the last position tiles see), so contiguous
    // ranges of split units would leave some XCDs far busier than others:
    // causal split launches keep the plain order.
    p.xcd_mode = (p.units % kXcds == 0 && !(causal && p.n_split > 1)) ? 1 : 0;
    p.upx = p.xcd_mode ? p.units / kXcds : p.units;
    // units per cache section: enough tiles to occupy one XCD at a time
    int cap = kTilesPerXcdWave / p.n_m;
    if (cap < 1) cap = 1;
    p.sec_units = largest_divisor_at_most(p.upx, cap);
    set_divisors(p);
    return ATTN_OK;
}

// o is the 16-bit output when n_split == 0 (whole key range), else the fp32
// per-split output [n_split, B, Hq, Lq, d_v]; strides default to contiguous
// [B, H, L, d] tensors
int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
        int Hkv, int Lq, int Lk, int d_qk, int d_v, int causal, float scale, void* stream,
        float threshold, unsigned long long* counter, bool debug, int n_split,
        const Strides* strides = nullptr, bool fp16 = false) {
    int rc = check_args(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d_qk, d_v, scale);
    if (rc != ATTN_OK) return rc;
    const Strides st =
        strides ? *strides : contiguous_strides(Hq, Hkv, Lq, Lk, d_qk, d_v);
    rc = check_strides(st, B, Hq, Hkv, Lq, Lk, d_qk, d_v);
    if (rc != ATTN_OK) return rc;
    if (n_split < 0 || n_split > kMaxSplits) return ATTN_ERR_BAD_ARGUMENT;
    // per-split rows are addressed with 64-bit offsets; the split count times
    // the rows must still fit the 32-bit row range of one launch's tiles
    if ((long long)(n_split > 0 ? n_split : 1) * B * Hq * Lq > INT32_MAX)
        return ATTN_ERR_TOO_LARGE;
    attn::FwdParams p;
    memset(&p, 0, sizeof p);
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    if (n_split == 0) {
        p.o = static_cast<uint16_t*>(o);
        p.n_split = 1;
        p.split_blocks = (Lk + attn::kBlockN - 1) / attn::kBlockN;
    } else {
        p.o_part = static_cast<float*>(o);
        p.n_split = n_split;
        p.split_blocks = split_keys(Lk, n_split) / attn::kBlockN;
    }
    p.lse = lse;
    p.rescale_count = counter;
    p.q_sb = st.q.batch;
    p.q_sh = st.q.head;
    p.q_sr = (int)st.q.row;
    p.k_sb = st.k.batch;
    p.k_sh = st.k.head;
    p.k_sr = (int)st.k.row;
    p.v_sb = st.v.batch;
    p.v_sh = st.v.head;
    p.v_sr = (int)st.v.row;
    p.o_sb = st.o.batch;
    p.o_sh = st.o.head;
    p.o_sr = (int)st.o.row;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Lq = Lq;
    p.Lk = Lk;
    p.scale = scale;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    p.threshold = threshold;
    rc = fill_schedule(p, causal != 0);
    if (rc != ATTN_OK) return rc;
    int n_cu = 0;
    rc = check_device(&n_cu);
    if (rc != ATTN_OK) return rc;
    // Persistent grid: one workgroup per CU (its registers allow no second
    // one), each looping over its tiles, as many as a multiple of 8 keeps
    // every workgroup on the XCD of its tiles.
    const long long tiles = (long long)p.units * p.n_m;
    long long grid = tiles;
    const long long slots = (long long)(n_cu / kXcds) * kXcds;
    if (slots > 0 && tiles > slots) grid = slots;
    p.grid = (int)grid;
    p.chain = attn::fwd_chained(p, d_qk, d_v, causal != 0) ? 1 : 0;
    log_launch("attn_fwd_kernel<%d,%d,%s%s%s> grid %d, %d tiles (units %d x position tiles %d), "
               "splits %d, query heads per workgroup %d, xcd_mode %d, chained %d",
               d_qk, d_v, causal ? "causal" : "full", debug ? ",debug" : "", fp16 ? ",fp16" : "",
               p.grid, p.units * p.n_m, p.units, p.n_m, p.n_split, p.Gp, p.xcd_mode, p.chain);
    hipError_t err = attn::launch_fwd(p, d_qk, d_v, causal != 0, debug, fp16,
                                      static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

// Schedule of a packed variable-length batch ("Flash Attention 4 ..." review,
// method part on scheduling: variable-length batches are ordered by the
// execution time of their work tiles, longest first).  A tile is (sequence,
// unit = (K/V head, head group), position block m); its cost is the number of
// 64-key blocks it visits plus a fixed per-tile overhead.
//  1. Units are dealt to the 8 XCDs longest first, each to the least loaded
//     XCD, so each XCD streams whole K/V heads through its own L2.
//  2. On each XCD, the units (longest first) are grouped into sections of at
//     most kTilesPerXcdWave tiles (or one larger unit), so the tiles running
//     at one time share few K/V heads.
//  3. Section by section, tiles are assigned longest first to the least
//     loaded of the XCD's kTilesPerXcdWave workgroups (LPT).
//  4. The kernel gives workgroup slot s of an XCD, in round r, the local tile
//     r * 32 + s (r even) or r * 32 + 31 - s (r odd); each slot's r-th
//     assigned tile is written there, and slots with fewer tiles are padded
//     with empty (all-zero) records.  Record 8 * local + x belongs to XCD x.
// The balance assumes 32 workgroups per XCD (256 CUs); with fewer, the kernel
// still runs every record exactly once, only less evenly.
int build_varlen_plan(const int* cu_q, const int* cu_k, int n_seq, int Hq, int Hkv, int causal,
                      std::vector<int>* out) {
    if (!cu_q || !cu_k) return ATTN_ERR_NULL_PTR;
    if (n_seq < 1 || Hq < 1 || Hkv < 1) return ATTN_ERR_BAD_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
    if (cu_q[0] != 0 || cu_k[0] != 0) return ATTN_ERR_BAD_SHAPE;
    for (int s = 0; s < n_seq; ++s)
        if (cu_q[s + 1] < cu_q[s] || cu_k[s + 1] < cu_k[s]) return ATTN_ERR_BAD_SHAPE;
    const int G = Hq / Hkv, Gp = packed_heads(G), n_hg = G / Gp;
    const int bm_pos = attn::kRowsPerWave * attn::kWaves / Gp;
    const int units_per_seq = Hkv * n_hg;
    // key blocks the tile at position block m of a (lq, lk) sequence visits
    auto tile_blocks = [&](long long lq, long long lk, long long m) {
        long long kend = lk;
        if (causal) kend = std::min(lk, std::min(lq, (m + 1) * bm_pos) - 1 + lk - lq + 1);
        return kend > 0 ? (kend + attn::kBlockN - 1) / attn::kBlockN : 0;
    };
    struct Unit {
        long long cost;
        int seq, ukv, n_m;
    };
    std::vector<Unit> units;
    for (int s = 0; s < n_seq; ++s) {
        const long long lq = cu_q[s + 1] - cu_q[s], lk = cu_k[s + 1] - cu_k[s];
        if (lq == 0) continue;  // no query rows: nothing to compute or write
        const int n_m = (int)((lq + bm_pos - 1) / bm_pos);
        long long cost = 0;
        for (int m = 0; m < n_m; ++m) cost += tile_blocks(lq, lk, m) + kTileOverhead;
        for (int u = 0; u < units_per_seq; ++u) units.push_back({cost, s, u, n_m});
    }
    // 1. units longest first (ties: sequence, then unit), each to the least loaded XCD
    std::stable_sort(units.begin(), units.end(),
                     [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
    std::vector<std::vector<Unit>> xcd_units(kXcds);
    long long xcd_load[kXcds] = {0};
    for (const Unit& u : units) {
        int best = 0;
        for (int x = 1; x < kXcds; ++x)
            if (xcd_load[x] < xcd_load[best]) best = x;
        xcd_units[best].push_back(u);
        xcd_load[best] += u.cost;
    }
    struct Tile {
        long long cost;
        int rec[attn::kPlanInts];
    };
    constexpr int kSlots = kTilesPerXcdWave;
    // slot_tiles[x][s]: the tiles workgroup slot s of XCD x runs, in order
    std::vector<std::vector<std::vector<Tile>>> slot_tiles(kXcds,
                                                           std::vector<std::vector<Tile>>(kSlots));
    size_t rounds = 0;
    for (int x = 0; x < kXcds; ++x) {
        long long load[kSlots] = {0};
        std::vector<Tile> sec;
        auto flush = [&]() {
            // 3. the section's tiles longest first, each to the least loaded slot
            std::stable_sort(sec.begin(), sec.end(),
                             [](const Tile& a, const Tile& b) { return a.cost > b.cost; });
            for (const Tile& t : sec) {
                int best = 0;
                for (int s = 1; s < kSlots; ++s)
                    if (load[s] < load[best]) best = s;
                slot_tiles[x][best].push_back(t);
                load[best] += t.cost;
            }
            sec.clear();
        };
        for (const Unit& u : xcd_units[x]) {
            // 2. a section holds at most kSlots tiles, or one unit
            if (!sec.empty() && sec.size() + (size_t)u.n_m > (size_t)kSlots) flush();
            const int lq = cu_q[u.seq + 1] - cu_q[u.seq], lk = cu_k[u.seq + 1] - cu_k[u.seq];
            for (int m = 0; m < u.n_m; ++m) {
                Tile t;
                t.cost = tile_blocks(lq, lk, m) + kTileOverhead;
                const int rec[attn::kPlanInts] = {cu_q[u.seq], lq, cu_k[u.seq], lk, u.ukv, m, 0, 0};
                memcpy(t.rec, rec, sizeof rec);
                sec.push_back(t);
            }
        }
        if (!sec.empty()) flush();
        for (int s = 0; s < kSlots; ++s) rounds = std::max(rounds, slot_tiles[x][s].size());
    }
    const size_t n_records = rounds * kSlots * kXcds;
    if (n_records * attn::kPlanInts > (size_t)INT32_MAX) return ATTN_ERR_TOO_LARGE;
    // 4. lay the records out where the kernel's round order looks for them
    out->assign(n_records * attn::kPlanInts, 0);
    for (int x = 0; x < kXcds; ++x)
        for (int s = 0; s < kSlots; ++s)
            for (size_t r = 0; r < slot_tiles[x][s].size(); ++r) {
                const size_t local = r * kSlots + ((r & 1) ? kSlots - 1 - s : s);
                memcpy(out->data() + (local * kXcds + x) * attn::kPlanInts,
                       slot_tiles[x][s][r].rec, sizeof(int) * attn::kPlanInts);
            }
    return ATTN_OK;
}

struct ArchCacheInit {
    ArchCacheInit() {
        for (auto& a : g_arch_ok) a.store(-1, std::memory_order_relaxed);
        for (auto& a : g_cu_count) a.store(0, std::memory_order_relaxed);
    }
} g_arch_cache_init;

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Lq, int Lk, int d_qk, int d_v, int causal, float scale,
             void* stream) {
    return run(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d_qk, d_v, causal, scale, stream,
               kDefaultThreshold, nullptr, false, 0);
}

int attn_fwd_dbg(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v, int causal, float scale,
                 void* stream, float rescale_threshold, int exp_mode,
                 unsigned long long* rescale_count) {
    if (!(rescale_threshold >= 0.0f) || !isfinite(rescale_threshold))
        return ATTN_ERR_BAD_ARGUMENT;
    if (exp_mode != 0) return ATTN_ERR_BAD_ARGUMENT;  // only v_exp_f32 is built
    return run(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d_qk, d_v, causal, scale, stream,
               rescale_threshold, rescale_count, true, 0);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                int Hkv, int Lq, int Lk, int d_qk, int d_v, attn_strides q_strides,
                attn_strides k_strides, attn_strides v_strides, attn_strides o_strides,
                int dtype, int causal, float scale, void* stream) {
    if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP16) return ATTN_ERR_BAD_ARGUMENT;
    const Strides st = {q_strides, k_strides, v_strides, o_strides};
    return run(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d_qk, d_v, causal, scale, stream,
               kDefaultThreshold, nullptr, false, 0, &st, dtype == ATTN_DTYPE_FP16);
}

}  // extern "C"

namespace {

// Validation and launch of the backward pass; delta == nullptr takes D's rows
// from the library's static device scratch instead of a caller buffer.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv,
            int Lq, int Lk, int d_qk, int d_v, int causal, float scale, void* stream,
            bool fp16 = false) {
    const bool own_delta = delta == nullptr;
    if (!dout || !dq || !dk || !dv) return ATTN_ERR_NULL_PTR;
    // the forward's argument rules, with o and lse as inputs here
    int rc = check_args(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d_qk, d_v, scale);
    if (rc != ATTN_OK) return rc;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        (!own_delta && !aligned(delta, 4)))
        return ATTN_ERR_MISALIGNED;
    const Strides st = contiguous_strides(Hq, Hkv, Lq, Lk, d_qk, d_v);
    rc = check_strides(st, B, Hq, Hkv, Lq, Lk, d_qk, d_v);
    if (rc != ATTN_OK) return rc;
    if ((long long)B * Hkv * ((Lk + 127) / 128) > INT32_MAX ||
        (long long)B * Hq * ((Lq + 127) / 128) > INT32_MAX)
        return ATTN_ERR_TOO_LARGE;
    // the dK/dV kernel addresses one query head of Q and of dO with 32-bit
    // buffer offsets
    if ((long long)Lq * d_qk * 2 > INT32_MAX || (long long)Lq * d_v * 2 > INT32_MAX)
        return ATTN_ERR_TOO_LARGE;
    if (own_delta && (long long)B * Hq * Lq > attn::kBwdScratchRows) return ATTN_ERR_SCRATCH;
    rc = check_device();
    if (rc != ATTN_OK) return rc;
    if (own_delta && attn::bwd_scratch_rows(&delta) != hipSuccess) return ATTN_ERR_HIP;
    attn::BwdParams p;
    memset(&p, 0, sizeof p);
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<const uint16_t*>(o);
    p.dout = static_cast<const uint16_t*>(dout);
    p.lse = lse;
    p.delta = delta;
    p.dq = static_cast<uint16_t*>(dq);
    p.dk = static_cast<uint16_t*>(dk);
    p.dv = static_cast<uint16_t*>(dv);
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Lq = Lq;
    p.Lk = Lk;
    p.G = Hq / Hkv;
    p.scale = scale;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    log_launch("attn_bwd<%d,%d,%s%s>: delta, dK/dV and dQ kernels%s", d_qk, d_v,
               causal ? "causal" : "full", fp16 ? ",fp16" : "",
               own_delta ? " (D in the static scratch)" : "");
    hipError_t err = attn::launch_bwd(p, d_qk, d_v, causal != 0, fp16,
                                      static_cast<hipStream_t>(stream));
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv,
             int Lq, int Lk, int d_qk, int d_v, int causal, float scale, void* stream) {
    if (!delta) return ATTN_ERR_NULL_PTR;
    return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, d_qk, d_v,
                   causal, scale, stream);
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq,
                int Hkv, int Lq, int Lk, int d_qk, int d_v, int dtype, int causal, float scale,
                void* stream) {
    if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP16) return ATTN_ERR_BAD_ARGUMENT;
    if (!delta) return ATTN_ERR_NULL_PTR;
    return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, d_qk, d_v,
                   causal, scale, stream, dtype == ATTN_DTYPE_FP16);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                     int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v, int causal, float scale,
                     void* stream) {
    return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, B, Hq, Hkv, Lq, Lk, d_qk, d_v,
                   causal, scale, stream);
}

int attn_split_keys(int Lk, int n_split) {
    if (Lk < 1) return -ATTN_ERR_BAD_SHAPE;
    if (n_split < 1 || n_split > kMaxSplits) return -ATTN_ERR_BAD_ARGUMENT;
    return split_keys(Lk, n_split);
}

int attn_fwd_decode(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                    int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v, int causal,
                    float scale, int n_split, void* stream) {
    int rc = check_args(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, d_qk, d_v, scale);
    if (rc != ATTN_OK) return rc;
    if (n_split < 1 || n_split > kMaxSplits) return ATTN_ERR_BAD_ARGUMENT;
    if ((long long)Lq * (Hq / Hkv) > attn::kDecRows) return ATTN_ERR_BAD_ARGUMENT;
    rc = check_strides(contiguous_strides(Hq, Hkv, Lq, Lk, d_qk, d_v), B, Hq, Hkv, Lq, Lk, d_qk,
                       d_v);
    if (rc != ATTN_OK) return rc;
    const long long grid = (long long)n_split * B * Hkv;
    if ((long long)n_split * B * Hq * Lq > INT32_MAX || grid > INT32_MAX) return ATTN_ERR_TOO_LARGE;
    attn::DecParams p;
    memset(&p, 0, sizeof p);
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Lq = Lq;
    p.Lk = Lk;
    p.G = Hq / Hkv;
    p.R = Lq * p.G;
    p.n_split = n_split;
    p.split_w = split_keys(Lk, n_split);
    p.grid = (int)grid;
    p.scale = scale;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    p.threshold = kDefaultThreshold;
    rc = check_device();
    if (rc != ATTN_OK) return rc;
    log_launch("attn_decode_kernel<%d,%d,%s> grid %d (splits %d of %d keys), rows per K/V head %d",
               d_qk, d_v, causal ? "causal" : "full", p.grid, p.n_split, p.split_w, p.R);
    if (attn::launch_decode(p, d_qk, d_v, causal != 0, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return ATTN_ERR_HIP;
    return ATTN_OK;
}

int attn_fwd_split(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v, int causal,
                   float scale, int n_split, void* stream) {
    if (n_split < 1 || n_split > kMaxSplits) return ATTN_ERR_BAD_ARGUMENT;
    // few query rows per K/V head: the key-streaming decode kernel
    if (Hkv >= 1 && Hq % Hkv == 0 && Lq >= 1 && (long long)Lq * (Hq / Hkv) <= attn::kDecRows)
        return attn_fwd_decode(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, d_qk, d_v, causal,
                               scale, n_split, stream);
    return run(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, d_qk, d_v, causal, scale, stream,
               kDefaultThreshold, nullptr, false, n_split);
}

int attn_merge(const float* o_part, const float* lse_part, void* o, float* lse, int n_split,
               long long rows, int d_v, void* stream) {
    if (!o_part || !lse_part || !o || !lse) return ATTN_ERR_NULL_PTR;
    if (n_split < 1 || n_split > kMaxSplits || rows < 0) return ATTN_ERR_BAD_ARGUMENT;
    if (d_v != 64 && d_v != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    if (!aligned(o_part, 16) || !aligned(o, 16) || !aligned(lse_part, 4) || !aligned(lse, 4))
        return ATTN_ERR_MISALIGNED;
    int rc = check_device();
    if (rc != ATTN_OK) return rc;
    log_launch("attn_merge_kernel<%d>: %lld rows, %d splits", d_v, rows, n_split);
    hipError_t err = attn::launch_merge(o_part, lse_part, static_cast<uint16_t*>(o), lse,
                                        n_split, rows, d_v, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

int attn_varlen_plan(const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seq, int Hq,
                     int Hkv, int causal, int* plan, int capacity, int* n_records) {
    if (!n_records) return ATTN_ERR_NULL_PTR;
    std::vector<int> recs;
    const int rc = build_varlen_plan(cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, causal, &recs);
    if (rc != ATTN_OK) return rc;
    const int n = (int)(recs.size() / attn::kPlanInts);
    *n_records = n;
    if (plan == nullptr) return ATTN_OK;
    if (capacity < n) return ATTN_ERR_BAD_ARGUMENT;
    if (!recs.empty()) memcpy(plan, recs.data(), sizeof(int) * recs.size());
    return ATTN_OK;
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* plan, int n_records, int total_q, int total_k, int Hq, int Hkv,
                    int d_qk, int d_v, int causal, float scale, void* stream) {
    if (!plan) return ATTN_ERR_NULL_PTR;
    if (total_q < 1 || total_k < 0 || n_records < 0) return ATTN_ERR_BAD_SHAPE;
    if (n_records % kXcds != 0) return ATTN_ERR_BAD_ARGUMENT;
    // the forward's argument rules on a batch of one token-major "sequence"
    int rc = check_args(q, k, v, o, lse, 1, Hq, Hkv, total_q, total_k > 0 ? total_k : 1, d_qk,
                        d_v, scale);
    if (rc != ATTN_OK) return rc;
    if (!aligned(plan, 16)) return ATTN_ERR_MISALIGNED;
    // every sequence's K and V rows lie in one tensor of less than 2^31 bytes,
    // so the kernel's 32-bit buffer offsets reach all of them
    if ((long long)total_k * Hkv * d_qk * 2 > INT32_MAX ||
        (long long)total_k * Hkv * d_v * 2 > INT32_MAX ||
        (long long)total_q * Hq > INT32_MAX)
        return ATTN_ERR_TOO_LARGE;
    if (n_records == 0) return ATTN_OK;  // no query rows in the batch
    attn::FwdParams p;
    memset(&p, 0, sizeof p);
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.plan = plan;
    p.total_q = total_q;
    p.total_k = total_k;
    // token-major [T, H, d]: a row is one token, heads are d apart
    p.q_sh = d_qk;
    p.q_sr = Hq * d_qk;
    p.k_sh = d_qk;
    p.k_sr = Hkv * d_qk;
    p.v_sh = d_v;
    p.v_sr = Hkv * d_v;
    p.o_sh = d_v;
    p.o_sr = Hq * d_v;
    p.B = 1;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Lq = 1;
    p.Lk = 1;
    p.G = Hq / Hkv;
    p.Gp = packed_heads(p.G);
    p.n_hg = p.G / p.Gp;
    p.bm_pos = attn::kRowsPerWave * attn::kWaves / p.Gp;
    p.n_split = 1;
    p.split_blocks = (total_k + attn::kBlockN - 1) / attn::kBlockN;
    p.units_kv = Hkv * p.n_hg;
    // the records are the tiles, interleaved by XCD
    p.units = n_records;
    p.n_m = 1;
    p.xcd_mode = 1;
    p.upx = n_records / kXcds;
    p.sec_units = 1;
    set_divisors(p);
    p.scale = scale;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    p.threshold = kDefaultThreshold;
    int n_cu = 0;
    rc = check_device(&n_cu);
    if (rc != ATTN_OK) return rc;
    long long grid = n_records;
    const long long slots = (long long)(n_cu / kXcds) * kXcds;
    if (slots > 0 && grid > slots) grid = slots;
    p.grid = (int)grid;
    log_launch("attn_fwd_kernel<%d,%d,%s,varlen> grid %d, %d tile records", d_qk, d_v,
               causal ? "causal" : "full", p.grid, n_records);
    hipError_t err = attn::launch_fwd(p, d_qk, d_v, causal != 0, false, false,
                                      static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
        case ATTN_ERR_BAD_SHAPE: return "B, Hq, Hkv, Lq and Lk must all be >= 1";
        case ATTN_ERR_GQA_RATIO: return "Hq must be a multiple of Hkv";
        case ATTN_ERR_UNSUPPORTED_HEAD_DIM:
            return "unsupported (d_qk, d_v): use (64,64), (128,128) or (192,128)";
        case ATTN_ERR_BAD_SCALE: return "scale must be finite and > 0";
        case ATTN_ERR_MISALIGNED:
            return "q, k, v and o must be 16-byte aligned and lse 4-byte aligned";
        case ATTN_ERR_TOO_LARGE: return "problem too large for the kernel's index types";
        case ATTN_ERR_NO_DEVICE: return "no HIP device is visible";
        case ATTN_ERR_UNSUPPORTED_ARCH: return "the current device is not gfx950 (MI355X)";
        case ATTN_ERR_HIP: return "the HIP runtime reported an error";
        case ATTN_ERR_BAD_ARGUMENT:
            return "argument out of range (rescale threshold finite and >= 0, exp mode 0, split "
                   "count in [1, 4096], merge rows >= 0, dtype bf16 or fp16)";
        case ATTN_ERR_BAD_STRIDE:
            return "strides must be >= 0 and multiples of 8 elements, with row strides of at "
                   "least the head dim";
        case ATTN_ERR_SCRATCH:
            return "B * Hq * Lq exceeds the rows of the allocation-free entry point's static "
                   "scratch (ATTN_BWD_NOALLOC_MAX_ROWS)";
        default: return "unknown attn status";
    }
}

int attn_abi_version(void) { return kAbiVersion; }

}  // extern "C"
