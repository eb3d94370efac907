// attn_api.cpp -- C ABI of the gfx950 fused attention forward and of its
// split-key variant and merge (declared in include/attn_fwd.h): argument
// validation, device checks, the tile schedule parameters, and the launches
// on the caller's stream.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include <hip/hip_runtime_api.h>

#include "attn_fwd.h"
#include "attn_params.h"

namespace {

constexpr int kAbiVersion = 4;
constexpr int kMaxSplits = 4096;
constexpr int kMaxDevices = 64;
constexpr int kXcds = 8;                 // MI355X: 8 accelerator complex dies
constexpr int kTilesPerXcdWave = 32;     // concurrent workgroups per XCD (32 CUs x 1)
constexpr float kDefaultThreshold = 8.0f;  // log2 units: a factor of 256

// -1 unknown, 0 not gfx950, 1 gfx950
std::atomic<int> g_arch_ok[kMaxDevices];
// compute units of each device (0 unknown)
std::atomic<int> g_cu_count[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

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

int fill_schedule(attn::FwdParams& p) {
    p.G = p.Hq / p.Hkv;
    // query heads that share a K/V head are packed into one workgroup, one
    // head per wave group, so the K/V block is loaded once for all of them
    p.Gp = (p.G % 8 == 0) ? 8 : (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
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
    p.xcd_mode = (p.units % kXcds == 0) ? 1 : 0;
    p.upx = p.xcd_mode ? p.units / kXcds : p.units;
    // units per cache section: enough tiles to occupy one XCD at a time
    int cap = kTilesPerXcdWave / p.n_m;
    if (cap < 1) cap = 1;
    p.sec_units = largest_divisor_at_most(p.upx, cap);
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
    rc = fill_schedule(p);
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
    hipError_t err = attn::launch_fwd(p, d_qk, d_v, causal != 0, debug, fp16,
                                      static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return ATTN_ERR_HIP;
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
                 void* stream, float rescale_threshold, unsigned long long* rescale_count) {
    if (!(rescale_threshold >= 0.0f) || !isfinite(rescale_threshold))
        return ATTN_ERR_BAD_ARGUMENT;
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

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv,
             int Lq, int Lk, int d_qk, int d_v, int causal, float scale, void* stream) {
    if (!dout || !dq || !dk || !dv || !delta) return ATTN_ERR_NULL_PTR;
    // the forward's argument rules, with o and lse as inputs here
    int rc = check_args(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d_qk, d_v, scale);
    if (rc != ATTN_OK) return rc;
    if (!(d_qk == d_v && (d_qk == 64 || d_qk == 128))) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(delta, 4))
        return ATTN_ERR_MISALIGNED;
    const Strides st = contiguous_strides(Hq, Hkv, Lq, Lk, d_qk, d_v);
    rc = check_strides(st, B, Hq, Hkv, Lq, Lk, d_qk, d_v);
    if (rc != ATTN_OK) return rc;
    if ((long long)B * Hkv * ((Lk + 127) / 128) > INT32_MAX ||
        (long long)B * Hq * ((Lq + 127) / 128) > INT32_MAX)
        return ATTN_ERR_TOO_LARGE;
    rc = check_device();
    if (rc != ATTN_OK) return rc;
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
    hipError_t err = attn::launch_bwd(p, d_qk, causal != 0, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_split_keys(int Lk, int n_split) {
    if (Lk < 1) return -ATTN_ERR_BAD_SHAPE;
    if (n_split < 1 || n_split > kMaxSplits) return -ATTN_ERR_BAD_ARGUMENT;
    return split_keys(Lk, n_split);
}

int attn_fwd_split(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v, int causal,
                   float scale, int n_split, void* stream) {
    if (n_split < 1 || n_split > kMaxSplits) return ATTN_ERR_BAD_ARGUMENT;
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
    hipError_t err = attn::launch_merge(o_part, lse_part, static_cast<uint16_t*>(o), lse,
                                        n_split, rows, d_v, static_cast<hipStream_t>(stream));
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
            return "argument out of range (rescale threshold finite and >= 0, split count in "
                   "[1, 4096], merge rows >= 0, dtype bf16 or fp16)";
        case ATTN_ERR_BAD_STRIDE:
            return "strides must be >= 0 and multiples of 8 elements, with row strides of at "
                   "least the head dim";
        default: return "unknown attn status";
    }
}

int attn_abi_version(void) { return kAbiVersion; }

}  // extern "C"
