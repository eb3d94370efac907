// attn_params.h -- launch parameters shared by the C ABI layer and the
// gfx950 kernels.  Internal to the library; not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace attn {

// Work decomposition constants of the forward kernel.
constexpr int kWaves = 8;            // waves per workgroup: two groups of 4, one wave
                                     // of each group per SIMD
constexpr int kGroupWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;     // query rows owned by one wave (MFMA N)
constexpr int kBlockN = 64;          // keys per K/V block
constexpr int kPlanInts = 8;         // ints per tile record of a packed variable-length
                                     // batch: q0, Lq, k0, Lk, unit, position block, 0, 0

// Division by a launch constant d >= 1 as a multiply and a shift, exact for
// numerators n < 2^31: n / d = (mulhi(n, mul) + n) >> shift, with shift =
// ceil(log2 d) and mul = floor(2^32 (2^shift - d) / d) + 1 (T. Granlund and
// P. Montgomery, "Division by invariant integers using multiplication",
// PLDI 1994, section 4).  (mul + 2^32) / 2^(32 + shift) exceeds 1 / d by at
// most 2^-(32 + shift), so for n < 2^31 the product exceeds n / d by less than
// 2^-(shift + 1) <= 1 / (2 d): too little to reach the next multiple of 1 / d.
// mulhi(n, mul) < n keeps the sum below 2^32.
struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};

inline FastDiv make_fast_div(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const unsigned long long m = (((1ull << 32) * ((1ull << l) - d)) / d) + 1;
    return FastDiv{(uint32_t)m, l};
}

struct FwdParams {
    // q, k, v, o: 16-bit elements (bf16 or fp16), element (b, h, i, c) at
    // b * s_b + h * s_h + i * s_r + c with the strides below
    const uint16_t* q;   // [B, Hq, Lq, dqk]
    const uint16_t* k;   // [B, Hkv, Lk, dqk]
    const uint16_t* v;   // [B, Hkv, Lk, dv]
    uint16_t* o;         // [B, Hq, Lq, dv] (whole-key output), or
    float* o_part;       // [n_split, B, Hq, Lq, dv] fp32 (per-split output) when set
    float* lse;          // [B, Hq, Lq] fp32, or [n_split, B, Hq, Lq] with o_part
    unsigned long long* rescale_count;  // optional event counter
    // Packed variable-length batch (nullptr otherwise): tile records in
    // schedule order, kPlanInts ints each; q, k, v, o are token-major
    // [T, H, d] and lse is [Hq, total_q].  The launch's Lq and Lk are unused.
    const int* plan;
    int total_q, total_k;  // query and key tokens of the packed batch

    int B, Hq, Hkv, Lq, Lk;
    int G;          // Hq / Hkv: query heads per K/V head
    int Gp;         // query heads packed into one workgroup (divides G and kWaves)
    int n_hg;       // G / Gp: head groups per K/V head
    int bm_pos;     // query positions per tile = kRowsPerWave * kWaves / Gp
    int n_m;        // position tiles per head group = ceil(Lq / bm_pos)
    int n_split;      // key splits (1: the whole key range)
    int split_blocks; // key blocks per split
    int units_kv;   // B * Hkv * n_hg: groups of query heads sharing one K/V head
    int units;      // units_kv * n_split
    int xcd_mode;   // 1: workgroup i runs on XCD i % 8, which owns a contiguous
                    //    range of units (upx of them)
    int upx;        // units per XCD when xcd_mode
    int sec_units;  // units per cache section (divides upx, or units)
    int grid;       // workgroups launched; each processes tiles i, i + grid, ...
                    // (a multiple of 8 when smaller than the tile count)
    // the divisors of a tile's coordinates: sec_units * n_m, sec_units,
    // units_kv, n_hg, Hkv and Gp
    FastDiv div_sec, div_sec_units, div_units_kv, div_hg, div_hkv, div_gp;
    int chain;      // 1: each workgroup's tiles run as one chained sweep (fwd_chained)

    long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;  // batch and head strides
    int q_sr, k_sr, v_sr, o_sr;  // row strides (elements); one K or V head spans
                                 // less than 2^31 bytes (checked on the host)

    float scale;        // softmax scale (natural units), used for lse
    float scale_log2;   // scale * log2(e): base-2 exponent multiplier
    float threshold;    // conditional rescale threshold, log2 units
};

// Launches the forward kernel instantiation matching (dqk, dv, causal, debug,
// element type); debug is bf16 only.
hipError_t launch_fwd(const FwdParams& p, int dqk, int dv, bool causal, bool debug, bool fp16,
                      hipStream_t stream);

// Whether a launch can run each workgroup's tiles as one chained sweep: non-causal,
// one key split, equal head dims, and every tile's key range long enough for
// its hand-offs (2 C + 2 blocks, C = d / 16 one-KiB chunks per wave slice) and
// an even number of blocks (every tile then starts on the same stage buffers).
// The sweep counts a workgroup's blocks, and twice that in phases, in ints.
// Needs the schedule and grid filled in; the host stores the answer in p.chain.
inline bool fwd_chained(const FwdParams& p, int dqk, int dv, bool causal) {
    if (causal || dqk != dv || p.plan != nullptr || p.n_split != 1 || p.o_part != nullptr)
        return false;
    const long long nblk = (p.Lk + kBlockN - 1) / kBlockN;
    const long long tiles = (long long)p.units * p.n_m;
    const long long per_wg = (tiles + p.grid - 1) / p.grid + 1;
    if (per_wg * nblk >= (1ll << 29)) return false;
    return nblk >= 2 * (dqk / 16) + 2 && nblk % 2 == 0;
}

// Backward pass (contiguous [B, H, L, d] tensors, bf16 or fp16; q, k, dq, dk
// rows of d_qk elements, v, o, dout, dv rows of d_v).
struct BwdParams {
    const uint16_t* q;     // [B, Hq, Lq, d_qk]
    const uint16_t* k;     // [B, Hkv, Lk, d_qk]
    const uint16_t* v;     // [B, Hkv, Lk, d_v]
    const uint16_t* o;     // [B, Hq, Lq, d_v]  forward output
    const uint16_t* dout;  // [B, Hq, Lq, d_v]  gradient of the loss w.r.t. o
    const float* lse;      // [B, Hq, Lq]       forward lse
    float* delta;          // [B, Hq, Lq]       D_i = dO_i . O_i (written)
    uint16_t* dq;          // [B, Hq, Lq, d_qk]
    uint16_t* dk;          // [B, Hkv, Lk, d_qk]
    uint16_t* dv;          // [B, Hkv, Lk, d_v]
    int B, Hq, Hkv, Lq, Lk, G;
    float scale, scale_log2;
};

hipError_t launch_bwd(const BwdParams& p, int dqk, int dv, bool causal, bool fp16,
                      hipStream_t stream);

// Rows of D (one float each) that the file-scope device array `scratch` of the
// allocation-free backward entry point holds: 4 Mi rows, 16 MiB per device.
constexpr long long kBwdScratchRows = 4LL << 20;

// Device address of the current device's copy of that array, looked up with
// hipGetSymbolAddress on the first call per device and kept; allocates nothing.
hipError_t bwd_scratch_rows(float** rows);

// Split-key forward for few query rows per K/V head (decoding): at most
// kDecRows = Lq * Hq / Hkv rows, contiguous bf16 [B, H, L, d] tensors,
// (d_qk, d_v) in {(64, 64), (128, 128), (192, 128)}.  Writes the same
// per-split states as the fused kernel's split path.
constexpr int kDecWaves = 4;   // waves per workgroup, each streaming a quarter of the split
constexpr int kDecKeys = 16;   // keys per wave step
constexpr int kDecRows = 16;   // query rows served per K/V head

struct DecParams {
    const uint16_t* q;  // [B, Hq, Lq, d_qk]
    const uint16_t* k;  // [B, Hkv, Lk, d_qk]
    const uint16_t* v;  // [B, Hkv, Lk, d_v]
    float* o_part;      // [n_split, B, Hq, Lq, d_v] fp32
    float* lse_part;    // [n_split, B, Hq, Lq]
    int B, Hq, Hkv, Lq, Lk;
    int G;        // Hq / Hkv
    int R;        // Lq * G <= kDecRows: rows per K/V head
    int n_split;  // key splits
    int split_w;  // keys per split (a multiple of 64)
    int grid;     // n_split * B * Hkv workgroups
    float scale, scale_log2, threshold;
};

hipError_t launch_decode(const DecParams& p, int dqk, int dv, bool causal, hipStream_t stream);

// Merges n_split partial states per row: o_part [n_split, rows, dv] fp32,
// lse_part [n_split, rows] -> o [rows, dv] bf16, lse [rows].
hipError_t launch_merge(const float* o_part, const float* lse_part, uint16_t* o, float* lse,
                        int n_split, long long rows, int dv, hipStream_t stream);

}  // namespace attn
