// attn_fwd_kernel.hip -- fused exact-attention forward for gfx950 (MI355X).
//
// One workgroup = 8 waves, two per SIMD; each wave owns 32 query rows for
// the whole key sweep (rows are split across waves, never keys, so no
// cross-wave output reduction: "Infra: Flash Attention", FA2 split-Q
// figure).  Keys are visited in blocks of 64; each block of K and V is staged
// through LDS, double buffered, and consumed by bf16 MFMA with fp32
// accumulation.  The two waves of a SIMD alternate between an MFMA phase and
// a softmax phase (the ping-pong described at the sweep below).  The grid is
// persistent, one workgroup per CU looping over tiles of 256 query rows.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// keys on the MFMA M axis, the wave's 32 queries on N.  In the 32x32
// accumulator lane l holds query (l & 31) and 16 of its 32 keys, the other 16
// sitting in lane l ^ 32, so a row maximum or row sum is an in-lane reduction
// plus one v_permlane32_swap.  The output is accumulated transposed as well,
// O^T = V^T P^T: the S^T accumulator registers, converted to bf16, are
// exactly the B operand of the PV MFMA once V^T is read with the matching key
// permutation, so P never leaves registers.  O^T puts all of one query's
// outputs in one lane pair, which makes the per-row rescale a per-lane scalar.
//
// Online softmax ("Flash Attention 4 ..." ch. 13, section on online softmax
// and conditional rescaling): the reference `ref` is kept in raw q.k units,
// exponents are base 2 with scale_log2 = scale * log2(e); the first block a
// row sees adopts its own max; later blocks move the reference only when
// delta = (ref - cand) * scale_log2 < -threshold, and then scale O and l by
// 2^delta.  The O multiply runs under a wave-uniform branch taken when any
// row of the wave moved its reference; the LDS barrier is never skipped
// (same chapter, section on why conditional rescaling pays off).
//
// Causal mask aligned bottom-right (query i sees keys j <= i + Lk - Lq):
// blocks past a tile's last visible key are not loaded, a wave skips the
// blocks past its own rows' last key, and blocks crossing the diagonal or
// the end of the keys are masked element by element ("Flash Attention 4
// ..." ch. 13, section on causal attention and GQA).  With grouped-query
// attention, the waves of one workgroup serve up to 4 query heads that share
// one K/V head, so each K/V block is loaded once for all of them (same
// section: K/V are not replicated per query head).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_params.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

// The 16-bit element type of Q, K, V, O and of P in the PV product: bf16 or
// fp16, with the MFMA forms of that type and fp32 accumulation.  Conversions
// from fp32 round to nearest even.
template <bool FP16>
struct Elem;
template <>
struct Elem<false> {
    using x8 = bf16x8;
    using x4 = bf16x4;
    using scalar = __bf16;
    static __device__ __forceinline__ f32x16 mfma32(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Elem<true> {
    using x8 = f16x8;
    using x4 = f16x4;
    using scalar = _Float16;
    static __device__ __forceinline__ f32x16 mfma32(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <int DQK, int DV>
struct Shape {
    static constexpr int kChunksK = DQK / 8;               // 16-byte chunks per K row
    static constexpr int kChunksV = DV / 8;                // 16-byte chunks per V row
    static constexpr int kKBytes = kBlockN * DQK * 2;      // one K block in LDS
    static constexpr int kVBytes = kBlockN * DV * 2;       // one V block in LDS
    // K blocks are copied by the 4 waves of group 1, V blocks by those of
    // group 0: 1 KiB direct copies per copying wave
    static constexpr int kKCopies = kChunksK / kGroupWaves;
    static constexpr int kVCopies = kChunksV / kGroupWaves;
    static constexpr int kKSteps = DQK / 16;               // MFMA k-steps for S
    static constexpr int kDvBlocks = DV / 32;              // 32-wide output blocks
    static_assert(kChunksK % kGroupWaves == 0 && kChunksV % kGroupWaves == 0,
                  "blocks split evenly");
    static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims must fit the MFMA tiles");
};

// K block in LDS: 64 key rows of DQK bf16, 16-byte chunk c of row r stored at
// slot c ^ kswz(r).  The 16 lanes that read one chunk column of 16
// consecutive rows (S^T operand, ds_read_b128) then hit 16 distinct bank
// groups.  The XOR only touches the low bits, so the slot stays in the row.
template <int DQK>
__device__ __forceinline__ int kswz(int r) {
    return (DQK == 128) ? (r & 15) : ((r >> 1) & 7);
}

// V block in LDS: 64 key rows of DV bf16 (row-major, as in HBM), chunk c of
// row r stored at slot c ^ vswz(r).  The PV operand is read with
// ds_read_b64_tr_b16: a 16-lane group reads 8 bytes from each of 4
// consecutive rows (r = 0..3) at 2 adjacent chunks; the two groups of a
// half-wave read the next 2 chunks.  The swizzle gives the 4 rows distinct
// chunk bits so that neither a 16-lane (128-byte) nor a 32-lane (256-byte)
// access window repeats a bank.
template <int DV>
__device__ __forceinline__ int vswz(int r) {
    const int q = r & 3;
    return (DV == 128) ? (4 * q + 2 * (q >> 1)) : (4 * (q & 1) + 2 * (q >> 1));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ float pair_max(float x) {
    // lanes l and l ^ 32 hold the two halves of one query's keys
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Copy 16 bytes per lane from global memory straight into LDS through a
// buffer descriptor: lane l reads at byte soff + voff (soff wave-uniform) and
// its data lands at lds_dst + 16 * l (one contiguous KiB per wave).  The
// buffer form (rather than the global-address form) lets LDS reads issued
// after it wait for just the reads they need.  Offsets at or
// past the descriptor's record count read as zero instead of faulting.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                            uint32_t soff, void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_dst, 16, voff, soff, 0, 0);
}

// A wave-uniform pointer held in VGPRs, moved to SGPRs (a buffer descriptor
// built from it then needs no per-lane loop).
template <typename T>
__device__ __forceinline__ const T* uniform(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Raw buffer descriptor over [base, base + bytes): 32-bit data format, no stride.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// n / d for 0 <= n < 2^31 with f = make_fast_div(d)
__device__ __forceinline__ int fdiv(int n, FastDiv f) {
    return (int)((__umulhi((uint32_t)n, f.mul) + (uint32_t)n) >> f.shift);
}

// Tile t of the launch -> its key split, K/V head, and this wave's query head
// and first query row.  With xcd_mode, tile t runs on XCD t % 8 (the
// hardware deals workgroups round-robin over the 8 XCDs, and a persistent
// grid is a multiple of 8) and each XCD owns a contiguous range of upx
// units; within it, sections of sec_units units are swept position tile by
// position tile, so the workgroups an XCD runs at one time share their K/V
// blocks in its L2.
struct TileCoord {
    int split, bk, hq, pos0, qw;
    int Lq, Lk;    // query rows and keys of the tile's sequence
    size_t qrow0;  // row of (b, hq, position 0) in lse
    size_t qbase, obase, kbase, vbase;  // element offsets of (b, head, row 0)
};

template <bool CAUSAL, bool VARLEN>
__device__ __forceinline__ TileCoord tile_coord(const FwdParams& p, int t, int wave) {
    TileCoord c;
    if constexpr (VARLEN) {
        // A packed variable-length batch: the host's record of tile t gives
        // its sequence's token offsets and lengths, its unit (K/V head, head
        // group) and its position block, already in schedule order.  A record
        // that does not fit the tensors becomes an empty tile.
        const int* rec = p.plan + kPlanInts * t;
        int q0 = rec[0], lq = rec[1], k0 = rec[2], lk = rec[3], unit = rec[4], m = rec[5];
        const bool ok = q0 >= 0 && lq > 0 && lk >= 0 && k0 >= 0 && q0 <= p.total_q - lq &&
                        k0 <= p.total_k - lk && unit >= 0 && unit < p.units_kv && m >= 0 &&
                        m * p.bm_pos < lq;
        if (!ok) q0 = lq = k0 = lk = unit = m = 0;
        const int kvh = fdiv(unit, p.div_hg);
        const int hg = unit - kvh * p.n_hg;
        c.Lq = lq;
        c.Lk = lk;
        c.split = 0;
        c.bk = kvh;
        const int wg = fdiv(wave, p.div_gp);
        c.hq = kvh * p.G + hg * p.Gp + (wave - wg * p.Gp);
        c.pos0 = m * p.bm_pos;
        c.qw = c.pos0 + wg * kRowsPerWave;
        c.qrow0 = (size_t)c.hq * p.total_q + q0;  // lse is [Hq, total_q]
        c.qbase = (size_t)q0 * p.q_sr + (size_t)c.hq * p.q_sh;
        c.obase = (size_t)q0 * p.o_sr + (size_t)c.hq * p.o_sh;
        c.kbase = (size_t)k0 * p.k_sr + (size_t)kvh * p.k_sh;
        c.vbase = (size_t)k0 * p.v_sr + (size_t)kvh * p.v_sh;
        return c;
    }
    const int per_sec = p.sec_units * p.n_m;
    int local = t, base = 0;
    if (p.xcd_mode) {
        local = t >> 3;
        base = (t & 7) * p.upx;
    }
    const int sec = fdiv(local, p.div_sec);
    const int r = local - sec * per_sec;
    const int mo = fdiv(r, p.div_sec_units);
    const int unit = base + sec * p.sec_units + (r - mo * p.sec_units);
    // causal tiles are ordered heaviest first (longest processing time first)
    const int m = CAUSAL ? (p.n_m - 1 - mo) : mo;
    c.Lq = p.Lq;
    c.Lk = p.Lk;
    c.split = fdiv(unit, p.div_units_kv);  // key split of this tile (0 without splits)
    const int ukv = unit - c.split * p.units_kv;
    c.bk = fdiv(ukv, p.div_hg);  // b * Hkv + kv head
    const int hg = ukv - c.bk * p.n_hg;
    const int b = fdiv(c.bk, p.div_hkv);
    const int kvh = c.bk - b * p.Hkv;
    const int wg = fdiv(wave, p.div_gp);
    c.hq = kvh * p.G + hg * p.Gp + (wave - wg * p.Gp);
    c.pos0 = m * p.bm_pos;
    c.qw = c.pos0 + wg * kRowsPerWave;  // first row of this wave
    c.qrow0 = (size_t)(b * p.Hq + c.hq) * p.Lq;
    c.qbase = (size_t)(b * p.q_sb + c.hq * p.q_sh);
    c.obase = (size_t)(b * p.o_sb + c.hq * p.o_sh);
    c.kbase = (size_t)(b * p.k_sb + kvh * p.k_sh);
    c.vbase = (size_t)(b * p.v_sb + kvh * p.v_sh);
    return c;
}

// Key range of a tile and of one wave: the split's blocks [jb0, jb0 +
// split_blocks), cut at the end of the keys and, with the causal mask, after
// the last key the tile's (the wave's) rows can see.  The tile visits nblk
// blocks from jb0; the wave's own blocks are the prefix [0, nact).
struct KeyRange {
    int jb0, nblk, nact;
};

template <bool CAUSAL>
__device__ __forceinline__ KeyRange key_range(const FwdParams& p, const TileCoord& c) {
    KeyRange r;
    r.jb0 = c.split * p.split_blocks;
    const int kbeg = r.jb0 * kBlockN;
    const int ksplit = min(c.Lk, kbeg + p.split_blocks * kBlockN);
    int kend = ksplit;
    int wend = ksplit;
    if (CAUSAL) {
        const int off = c.Lk - c.Lq;
        const int tile_last = min(c.Lq, c.pos0 + p.bm_pos) - 1;
        kend = min(ksplit, tile_last + off + 1);
        const int wave_last = min(c.Lq, c.qw + kRowsPerWave) - 1;
        wend = min(ksplit, wave_last + off + 1);
    }
    r.nblk = kend > kbeg ? (kend - kbeg + kBlockN - 1) / kBlockN : 0;
    r.nact = (c.qw < c.Lq && wend > kbeg) ? min(r.nblk, (wend - kbeg + kBlockN - 1) / kBlockN)
                                          : 0;
    return r;
}

template <int DQK, int DV, bool CAUSAL, bool DEBUG, bool FP16, bool VARLEN, bool CHAIN>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(const FwdParams p) {
    using S = Shape<DQK, DV>;
    using E = Elem<FP16>;
    using ex8 = typename E::x8;
    using ex4 = typename E::x4;
    constexpr int kRowK = DQK * 2;  // bytes per K row in LDS
    constexpr int kRowV = DV * 2;   // bytes per V row in LDS
    // row strides in HBM, bytes (equal to the LDS rows when contiguous)
    const int k_rb = p.k_sr * 2;
    const int v_rb = p.v_sr * 2;
    const int q_rb = p.q_sr * 2;
    // two stage buffers each for K and V, distinct objects so that reads of
    // one buffer are never ordered behind copies into the other
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[S::kKBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[S::kKBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[S::kVBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[S::kVBytes];
    // Per-wave slices that carry the next tile's Q in and the last tile's O
    // out (equal head dims only: a slice row then fits both).  Slice rows use
    // the K block's row layout and swizzle.
    constexpr bool kStage = DQK == DV;
    constexpr int kRowQ = DQK * 2;                          // bytes per Q (and O) row
    constexpr int kSlice = kRowsPerWave * kRowQ;            // bytes per wave
    constexpr int kSliceChunks = kSlice / 1024;             // 1 KiB wave copies per slice
    // (16-byte alignment places it after the K/V buffers, which then keep LDS
    // addresses below 64 KiB that fit the read instructions' offset field)
    __shared__ __attribute__((aligned(16))) unsigned char lds_s[kStage ? kWaves * kSlice : 16];

    // Bring every kernel argument the sweep uses into SGPRs now: a scalar
    // load still in flight inside the loop would force each LDS wait there to
    // drain all outstanding LDS reads instead of only the oldest ones.
    const float c2 = p.scale_log2;
    const float threshold = p.threshold;
    // Weight bound of the softmax fast path: a row whose weights against its
    // reference all stay below 2^(threshold - 1/64) cannot move, whatever the
    // rounding of the exact rule's own test, which the rows closer to the
    // boundary take.
    const float thr_weight = __builtin_amdgcn_exp2f(threshold - 0.015625f);
    const float scale = p.scale;
    float* const lse_out = p.lse;
    uint16_t* const o_out = p.o;
    float* const o_part = p.o_part;
    unsigned long long* const rescale_count = p.rescale_count;
    asm volatile("" ::"s"(c2), "s"(threshold), "s"(scale), "s"(lse_out), "s"(o_out),
                 "s"(o_part), "s"(rescale_count));
    asm volatile("" ::"s"(thr_weight));

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    // waves are spread round-robin over the 4 SIMDs: waves w and w + 4 share
    // one; the two wave groups alternate between MFMA and VALU phases
    const int grp = wave / kGroupWaves;
    // The wave index for the tile coordinates.  The chained sweep computes
    // them inside its sweep, where the pointers derived from it would
    // otherwise take vector registers: there it is made wave-uniform.
    const int wave_t = CHAIN ? __builtin_amdgcn_readfirstlane(wave) : wave;

    // ---- tiles of this workgroup ---------------------------------------------
    // With one workgroup per CU the grid is persistent: each workgroup runs
    // one tile per round.  While a tile's key sweep runs, each wave prefetches
    // its rows of the next tile's Q into its own LDS slice and drains the
    // previous tile's output from that slice, a chunk per key-block pair, and
    // the last pair copies the next tile's first K block, so tiles follow each
    // other without a load burst between them.  Round r takes the workgroups'
    // next cnt tiles in the order of the tile index (per XCD with xcd_mode,
    // which keeps every tile on its XCD), reversed in odd rounds: causal tiles
    // come heaviest first, so a workgroup that gets a heavy tile in one round
    // gets a light one in the next.
    const int n_tiles = p.units * p.n_m;
    const int xcd = p.xcd_mode ? (int)(blockIdx.x & 7) : 0;
    const int slot = p.xcd_mode ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    const int per_round = p.xcd_mode ? (int)(gridDim.x >> 3) : (int)gridDim.x;
    const int n_local = p.xcd_mode ? (n_tiles >> 3) : n_tiles;
    // tile of round r, or -1 when the workgroup has none
    auto tile_of_round = [&](int r) __attribute__((always_inline)) {
        const int first = r * per_round;
        const int cnt = min(per_round, n_local - first);
        if (slot >= cnt) return -1;
        const int local = first + ((r & 1) ? cnt - 1 - slot : slot);
        return p.xcd_mode ? (local << 3) | xcd : local;
    };
    // Causal tiles of odd rounds sweep their keys from the last block down.
    // Round r and r + 1 pair heavy with light tiles (the snake above), so the
    // tiles of an odd round, which start as the previous round's tiles finish,
    // all finish together; swept downward they all reach block 0 at that
    // moment and so visit the same key block at the same time, which keeps a
    // head's K/V blocks shared in the XCD's L2 instead of fetched once per
    // tile.  The online softmax takes the keys in any order: rows whose
    // first blocks are masked keep an empty state until their first visible
    // key adopts its maximum.
    auto sweep_down = [&](int r) __attribute__((always_inline)) {
        return CAUSAL && !VARLEN && (r & 1) != 0;
    };
    int round = 0;
    int tile = tile_of_round(0);
    if (tile < 0) return;  // only if the grid exceeds the tiles (workgroup-uniform)

    // per-tile values of this wave (set_tile).  The sweep visits the tile's
    // blocks in local order j = 0 .. nblk - 1, key block jb0 + blk(j); the
    // wave computes on local blocks [jact0, jact1).
    int split, qw, jb0, nblk, jact1;
    int jact0 = 0;
    bool desc = false;  // the sweep runs from the last key block down
    size_t qrow0;  // row index of (b, hq, position 0) in lse
    size_t qrow_w, orow_w;  // element offsets of this wave's first Q and O rows
    __amdgpu_buffer_rsrc_t krsrc, vrsrc;
    // query rows and keys of the tile's sequence (the launch's Lq and Lk
    // unless the batch is packed with variable lengths)
    int Lq_t = p.Lq, Lk_t = p.Lk;
    int off = p.Lk - p.Lq;  // causal diagonal offset
    // byte extent of a K (V) head's rows for its buffer descriptor; empty
    // when a packed sequence has no keys
    auto kv_bytes = [&](int lk, int rb, int row) __attribute__((always_inline)) {
        return (VARLEN && lk <= 0) ? 0u : (uint32_t)(lk - 1) * rb + row;
    };
    auto set_tile = [&](int t) __attribute__((always_inline)) {
        const TileCoord c = tile_coord<CAUSAL, VARLEN>(p, t, wave_t);
        if constexpr (VARLEN) {
            Lq_t = c.Lq;
            Lk_t = c.Lk;
            off = c.Lk - c.Lq;
        }
        split = c.split;
        qw = c.qw;
        qrow0 = c.qrow0;
        qrow_w = c.qbase + (size_t)c.qw * p.q_sr;
        orow_w = c.obase + (size_t)c.qw * p.o_sr;
        const KeyRange r = key_range<CAUSAL>(p, c);
        jb0 = r.jb0;
        nblk = r.nblk;
        // the wave's own blocks are the first nact in key order: a prefix of an
        // upward sweep, a suffix of a downward one
        jact1 = r.nact;
        if constexpr (CAUSAL && !VARLEN) {
            desc = sweep_down(round);
            jact0 = desc ? r.nblk - r.nact : 0;
            jact1 = desc ? r.nblk : r.nact;
        }
        // one descriptor per K/V head; a head spans less than 2^31 bytes
        // (checked on the host), so 32-bit byte offsets address all of it
        krsrc = make_rsrc(p.k + c.kbase, kv_bytes(c.Lk, k_rb, kRowK));
        vrsrc = make_rsrc(p.v + c.vbase, kv_bytes(c.Lk, v_rb, kRowV));
    };
    set_tile(tile);

    // ---- Q fragment, resident in registers for the whole sweep -----------
    // lane holds Q[qw + l32][16 ks + 8 hi .. +7] for every k-step ks
    ex8 qf[S::kKSteps];
    // rows qw_ .. of the tile whose first Q row of this wave is at element
    // qrow_w_ (lq_ query rows in its sequence)
    auto load_q_rows = [&](int qw_, size_t qrow_w_, int lq_) __attribute__((always_inline)) {
        const int qi = qw_ + l32;
        const bool ok = qi < lq_;
        // lanes past Lq point at row 0 of the head (never read past the tensor)
        const uint16_t* src =
            p.q + (ok ? qrow_w_ + (size_t)l32 * p.q_sr : qrow_w_ - (size_t)qw_ * p.q_sr) + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks) {
            u32x4 w = ok ? load16(src + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
            qf[ks] = __builtin_bit_cast(ex8, w);
        }
    };
    load_q_rows(qw, qrow_w, Lq_t);

    // ---- direct global -> LDS copies of one K or V block -------------------
    // The copies are issued by the waves whose phase at that moment is the
    // softmax one (group 1 copies K, group 0 copies V), so the wave running
    // MFMAs issues nothing else.  Copy n of the block fills LDS slots
    // [64 n, 64 n + 64); lane l takes
    // slot 64 n + l = (row r, stored chunk c') and fetches source chunk
    // c' ^ swizzle(r) of key row key0 + r (rows are row-stride bytes apart in
    // HBM and DQK * 2 apart in LDS).  The per-lane byte offsets within a
    // block are fixed, so they are computed once.  In a block that runs
    // past the last key, the rows past it lie beyond the descriptor's range
    // and arrive as zeros: their scores are masked to -inf and their weights
    // are exactly 0.
    const int wq = wave % kGroupWaves;  // index of the wave within its group
    uint32_t koff[S::kKCopies], voff_copy[S::kVCopies];
#pragma unroll
    for (int i = 0; i < S::kKCopies; ++i) {
        const int slot = 64 * (wq * S::kKCopies + i) + lane;
        const int r = slot / S::kChunksK;
        const int c = (slot - r * S::kChunksK) ^ kswz<DQK>(r);
        koff[i] = r * k_rb + 16 * c;
    }
#pragma unroll
    for (int i = 0; i < S::kVCopies; ++i) {
        const int slot = 64 * (wq * S::kVCopies + i) + lane;
        const int r = slot / S::kChunksV;
        const int c = (slot - r * S::kChunksV) ^ vswz<DV>(r);
        voff_copy[i] = r * v_rb + 16 * c;
    }

    // The block offset goes in the scalar offset operand and this wave's LDS
    // destination is a scalar too, so a copy needs no vector arithmetic.
    const int kdst = __builtin_amdgcn_readfirstlane(1024 * S::kKCopies * wq);
    const int vdst = __builtin_amdgcn_readfirstlane(1024 * S::kVCopies * wq);
    // key block (relative to jb0) of local block j of the sweep
    auto blk = [&](int j) __attribute__((always_inline)) {
        return (CAUSAL && !VARLEN && desc) ? nblk - 1 - j : j;
    };
    auto copy_kblock = [&](__amdgpu_buffer_rsrc_t rs, int key0, unsigned char* dst)
                           __attribute__((always_inline)) {
        const uint32_t boff = (uint32_t)key0 * k_rb;
        // an opaque copy of the wave's offset: the destinations are formed
        // here with one scalar add each, not precomputed for every buffer
        // and copy and held (or spilled) across the sweep
        int kd = kdst;
        asm volatile("" : "+s"(kd));
#pragma unroll
        for (int i = 0; i < S::kKCopies; ++i)
            copy_to_lds(rs, koff[i], boff, dst + kd + 1024 * i);
    };
    auto copy_k = [&](int jl, unsigned char* dst) __attribute__((always_inline)) {
        copy_kblock(krsrc, (jb0 + blk(jl)) * kBlockN, dst);
    };
    auto copy_vblock = [&](__amdgpu_buffer_rsrc_t rs, int key0, unsigned char* dst)
                           __attribute__((always_inline)) {
        const uint32_t boff = (uint32_t)key0 * v_rb;
        int vd = vdst;
        asm volatile("" : "+s"(vd));
#pragma unroll
        for (int i = 0; i < S::kVCopies; ++i)
            copy_to_lds(rs, voff_copy[i], boff, dst + vd + 1024 * i);
    };
    auto copy_v = [&](int jl, unsigned char* dst) __attribute__((always_inline)) {
        copy_vblock(vrsrc, (jb0 + blk(jl)) * kBlockN, dst);
    };

    // ---- LDS read offsets (bytes within a block buffer) -----------------------
    // S^T operand: row 32 mb + l32, chunk 2 ks + hi (mb adds 32 rows).  The
    // swizzle XORs the low 4 (d = 128) or 3 (other widths) bits of the chunk
    // index, so the lane-dependent part of the offset repeats every
    // kReadTable k-steps and the rest is a constant.
    constexpr int kReadTable = (DQK == 128) ? 8 : 4;
    int kread[kReadTable];
#pragma unroll
    for (int ks = 0; ks < kReadTable; ++ks)
        kread[ks] = (l32 * S::kChunksK + ((2 * ks + hi) ^ kswz<DQK>(l32))) * 16;
    // PV operand (transposed V reads): 16-lane group g = lane / 16 with index
    // 4 r + j reads row 16 G + 8 t + 4 (g / 2) + r, dims 32 i + 16 (g & 1) +
    // 4 j .. +3, so lane l receives V[keys][32 i + (l & 31)] for the keys
    // whose P values its accumulator registers hold.  G and t add whole rows.
    int vread[S::kDvBlocks];
    {
        const int tg = lane >> 4, ti = lane & 15, tr = ti >> 2, tj = ti & 3;
        const int row = 4 * (tg >> 1) + tr;
        const int cl = 2 * (tg & 1) + (tj >> 1);
#pragma unroll
        for (int i = 0; i < S::kDvBlocks; ++i)
            vread[i] = row * kRowV + 16 * ((4 * i + cl) ^ vswz<DV>(row)) + 8 * (tj & 1);
    }

    // ---- running state (reset at each tile) -----------------------------------
    f32x16 oacc[S::kDvBlocks];
    float ref;  // exponent reference, raw q.k units
    float ell;  // this lane's share of sum P (fp32 P), for lse
    // Compensation of ell (Kahan-Neumaier): minus the low-order part that the
    // running fp32 sum has rounded away.  After the reference settles, later
    // blocks can each add far less than half an ulp of ell (millions of keys
    // with scores far below the maximum); uncompensated, that mass would be
    // lost and lse biased low by up to its share of the sum.
    float ell_c;
    // Row sums of the bf16 P that feed the PV product (they normalise O with
    // exactly the weights it was built from), accumulated by a 16x16x32 MFMA
    // with a 0/1 selector as A: in that shape lane l supplies B column l % 16
    // from k-group l / 16, so with A[m][k] = 1 iff m and k's group have equal
    // parity, even rows of D sum the P of query l % 16 (groups 0, 2) and odd
    // rows those of query l % 16 + 16 (groups 1, 3).  Lane l then finds its
    // own query's sum in register (l / 16) & 1 of the accumulator.
    f32x4 ell_o;
    // the per-row state; O itself is cleared separately (reset_state), or not
    // at all where the tile's first PV product starts from a zero accumulator
    auto reset_rows = [&]() __attribute__((always_inline)) {
        ref = kNegInf;
        ell = 0.0f;
        ell_c = 0.0f;
        ell_o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };
    auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < S::kDvBlocks; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
        reset_rows();
    };
    ex8 sel;
    {
        using es = typename E::scalar;
        const es v = (((lane & 15) ^ (lane >> 4)) & 1) ? (es)0.0f : (es)1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sel[i] = v;
    }
    f32x16 s[kBlockN / 32];  // scores of the block between its M and V phases
    ex8 pb[kBlockN / 16];  // its 16-bit weights between its V and M phases

    // ---- MFMA phase M(j): O^T += V^T P^T for block j, then S^T = K Q^T for
    // block j + 1 (j = -1: scores of block 0 only) --------------------------
    // The phase is a sequence of MFMA units, each with one LDS operand: 16 PV
    // units (g, i) and 16 score units (ks, mb).  Operands are loaded kAhead
    // units before their MFMA into a small register ring, and scheduling
    // barriers keep that order, so LDS latency overlaps earlier MFMAs instead
    // of stalling each one.
    constexpr int kPvUnits = (kBlockN / 16) * S::kDvBlocks;
    constexpr int kSUnits = S::kKSteps * (kBlockN / 32);
    constexpr int kAhead = 4;
    auto load_pv = [&](int u, const unsigned char* vl) __attribute__((always_inline)) {
        const int g = u / S::kDvBlocks, i = u % S::kDvBlocks;
        i16x4 part[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
            part[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vl + vread[i] + (16 * g + 8 * t) * kRowV));
        return __builtin_bit_cast(
            ex8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto load_s = [&](int u, const unsigned char* kl) __attribute__((always_inline)) {
        const int ks = u / (kBlockN / 32), mb = u % (kBlockN / 32);
        return *reinterpret_cast<const ex8*>(kl + kread[ks % kReadTable] +
                                                (ks / kReadTable) * kReadTable * 32 +
                                                mb * 32 * kRowK);
    };
    // pvz: the PV product is the tile's first, its first k-step starts O from
    // an inline zero accumulator.  epic: the PV product is the tile's last; all
    // PV units run first, then epi(-1) and, after score unit k, epi(k) (the
    // tile's epilogue in pieces beside the score MFMAs)
    auto m_units = [&](bool do_pv, bool do_s, const unsigned char* kl, const unsigned char* vl,
                       auto pvz, auto epic, auto&& epi) __attribute__((always_inline)) {
        constexpr bool kPvZero = decltype(pvz)::value;
        constexpr bool kEpi = decltype(epic)::value;
        const f32x16 zero = {};
        // one MFMA unit: PV unit u < kPvUnits, else score unit u - kPvUnits; the
        // first k-step of a score block starts from an inline zero accumulator
        auto mfma_unit = [&](int u, ex8 a) __attribute__((always_inline)) {
            if (u < kPvUnits) {
                const int g = u / S::kDvBlocks, i = u % S::kDvBlocks;
                oacc[i] = E::mfma32(a, pb[g], (kPvZero && g == 0) ? zero : oacc[i]);
            } else {
                const int v = u - kPvUnits;
                const int ks = v / (kBlockN / 32), mb = v % (kBlockN / 32);
                s[mb] = E::mfma32(a, qf[ks], ks == 0 ? zero : s[mb]);
            }
        };
        // the bf16 row sums need no LDS operand: they run while the first
        // operands of the ring are still in flight
        auto row_sums = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < kBlockN / 16; ++g)
                ell_o = E::mfma16(sel, pb[g], ell_o);
            __builtin_amdgcn_sched_barrier(0);
        };
        if (do_pv || do_s) {
            auto load = [&](int u) __attribute__((always_inline)) {
                return u < kPvUnits ? load_pv(u, vl) : load_s(u - kPvUnits, kl);
            };
            if (do_pv && do_s) {
                // PV units (two transposed 8-byte LDS reads each) and score units
                // (one 16-byte read) alternate, which spreads the LDS demand
                // evenly over the phase instead of saturating it in one half
                constexpr int kUnits = kPvUnits + kSUnits;
                static_assert(kSUnits >= kPvUnits, "every PV unit has a score partner");
                auto order = [](int n) {
                    if (kEpi) return n;
                    return n < 2 * kPvUnits ? ((n & 1) ? kPvUnits + (n >> 1) : (n >> 1))
                                            : kPvUnits + n - kPvUnits;
                };
                ex8 ring[kAhead];
#pragma unroll
                for (int n = 0; n < kAhead; ++n) ring[n] = load(order(n));
                row_sums();
#pragma unroll
                for (int n = 0; n < kUnits; ++n) {
                    const ex8 a = ring[n % kAhead];
                    if (n + kAhead < kUnits) ring[n % kAhead] = load(order(n + kAhead));
                    mfma_unit(order(n), a);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (kEpi) {
                        if (n >= kPvUnits - 1) {
                            epi(n - kPvUnits);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            } else if (do_pv) {
                ex8 ring[kAhead];
#pragma unroll
                for (int u = 0; u < kAhead; ++u) ring[u] = load(u);
                row_sums();
#pragma unroll
                for (int u = 0; u < kPvUnits; ++u) {
                    const ex8 a = ring[u % kAhead];
                    if (u + kAhead < kPvUnits) ring[u % kAhead] = load(u + kAhead);
                    mfma_unit(u, a);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                ex8 ring[kAhead];
#pragma unroll
                for (int u = 0; u < kAhead; ++u) ring[u] = load(kPvUnits + u);
#pragma unroll
                for (int u = 0; u < kSUnits; ++u) {
                    const ex8 a = ring[u % kAhead];
                    if (u + kAhead < kSUnits) ring[u % kAhead] = load(kPvUnits + u + kAhead);
                    mfma_unit(kPvUnits + u, a);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    auto m_phase = [&](int j, const unsigned char* kl, const unsigned char* vl)
                       __attribute__((always_inline)) {
        constexpr bool kDown = CAUSAL && !VARLEN;  // launches that may sweep downward
        const bool do_pv = j >= (kDown ? jact0 : 0) && j < jact1;
        const bool do_s = (!kDown || j + 1 >= jact0) && j + 1 < jact1;
        m_units(do_pv, do_s, kl, vl, std::false_type{}, std::false_type{}, [](int) {});
    };

    // ---- VALU phase V(j): online softmax of block j's scores -----------------
    // fresh: the tile's first block, whose O is not read (its PV product
    // starts from zero), so a reference move need not rescale it
    auto softmax = [&](int j, bool fresh) __attribute__((always_inline)) {
        const int key0 = (jb0 + blk(j)) * kBlockN;
        // mask keys past the end or past the causal diagonal
        const bool need_mask =
            (key0 + kBlockN > Lk_t) || (CAUSAL && key0 + kBlockN - 1 > qw + off);
        if (need_mask) {
            const int qi = qw + l32;
            const int klim = CAUSAL ? min(Lk_t, qi + off + 1) : Lk_t;
#pragma unroll
            for (int mb = 0; mb < kBlockN / 32; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + mb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key >= klim) s[mb][r] = kNegInf;
                }
        }

        // P = 2^(x * c2 - refc), rounded to bf16 in registers, with this lane's
        // share of their fp32 sum (returned).  The scores stay in s, so the
        // weights can be formed again against another reference.  Groups of 8
        // independent instructions back to back, since this wave is the only
        // VALU issuer on its SIMD while the other wave runs MFMAs.
        auto weights = [&](float refc) __attribute__((always_inline)) {
            float rs[8];
            static_assert(sizeof(pb) / sizeof(pb[0]) == 2 * (kBlockN / 32),
                          "one group of 8 weights per half score block");
#pragma unroll
            for (int g = 0; g < kBlockN / 16; ++g) {
                const int mb = g >> 1, t = g & 1;
                f32x8 e;
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = fmaf(s[mb][8 * t + i], c2, -refc);
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(e[i]);
                if (g == 0) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) rs[i] = e[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) rs[i] += e[i];
                }
                pb[g] = __builtin_convertvector(e, ex8);
            }
            return ((rs[0] + rs[1]) + (rs[2] + rs[3])) + ((rs[4] + rs[5]) + (rs[6] + rs[7]));
        };
        // The reference moves only when the block maximum exceeds it by more
        // than the threshold, i.e. when some weight against the current
        // reference exceeds 2^threshold.  So once every row of the wave has a
        // reference, the weights are formed against it first: if no lane's
        // sum of them reaches thr_weight, no weight does and no row moves,
        // and the block maximum is never needed.  Otherwise (or while some
        // row has no reference yet) the rule runs in full below and decides
        // exactly as it would alone.
        float bsum = 0.0f;
        bool done = false;
        const bool attempted = !__ballot(ref == kNegInf);
        if (attempted) {
            bsum = weights(ref * c2);
            done = !__ballot(!(bsum <= thr_weight));
        }
        if (!done) {
            // block max of this row (raw units), two independent chains
            float bm0 = fmaxf(s[0][0], s[0][1]);
            float bm1 = fmaxf(s[kBlockN / 32 - 1][0], s[kBlockN / 32 - 1][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) {
                bm0 = fmaxf(fmaxf(bm0, s[0][r]), s[0][r + 1]);
                bm1 = fmaxf(fmaxf(bm1, s[kBlockN / 32 - 1][r]), s[kBlockN / 32 - 1][r + 1]);
            }
            static_assert(kBlockN / 32 == 2, "two 32-key score blocks per key block");
            const float bmax = pair_max(fmaxf(bm0, bm1));

            // Conditional rescale decision, branch-free.  delta is -inf when
            // the row had no reference yet (the first block with a visible key
            // adopts its own max: scale 0 applied to an empty state) and NaN
            // while the row has seen no visible key at all (nothing moves).
            const float cand = fmaxf(ref, bmax);
            const float delta = (ref - cand) * c2;
            const bool moved = delta < -threshold;
            const float acc_scale = moved ? __builtin_amdgcn_exp2f(delta) : 1.0f;
            if (DEBUG && rescale_count != nullptr) {
                // events count reference moves after the first one of a row
                const unsigned long long ev = __ballot(moved && ref != kNegInf && qw + l32 < Lq_t);
                if (lane == 0 && ev)
                    atomicAdd(rescale_count,
                              (unsigned long long)__builtin_popcountll(ev & 0xffffffffull));
            }
            ref = moved ? cand : ref;
            const bool any_moved = __ballot(moved) != 0;
            if (any_moved) {  // wave-uniform: some row of this wave moved its reference
                if (!fresh) {
#pragma unroll
                    for (int i = 0; i < S::kDvBlocks; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[i][r] *= acc_scale;
                }
                ell *= acc_scale;
                ell_c *= acc_scale;
                // only the register holding this lane's own query matters
                ell_o *= acc_scale;
            }
            // the weights against the final references (unless the attempt
            // above formed them and no row moved)
            if (!attempted || any_moved) bsum = weights((ref == kNegInf) ? 0.0f : ref * c2);
        }
        const float y = bsum - ell_c;
        const float t = ell + y;
        ell_c = (t - ell) - y;
        ell = t;
    };
    auto v_phase = [&](int j) __attribute__((always_inline)) {
        if (j >= jact1) return;
        if constexpr (CAUSAL && !VARLEN) {
            if (j < jact0) return;
        }
        softmax(j, false);
    };

    // ---- ping-pong sweep over key blocks ---------------------------------------
    // A wave's work is the sequence M(-1), V(0), M(0), V(1), M(1), ... with
    // local phase lambda: lambda = 0 is M(-1), odd lambda = 2 j + 1 is V(j),
    // even lambda = 2 j + 2 is M(j).  Group 0 runs local phase lambda in global
    // phase phi = lambda and group 1 one phase later, so on each SIMD one wave
    // issues MFMA work while the other issues softmax VALU work.  M(j) reads
    // stage j + 1 = {K(j + 1), V(j)} in global phases 2 j + 2 and 2 j + 3.
    // Stage t + 1 is copied during phases 2 t (K) and 2 t + 1 (V) into the
    // buffers stage t - 1 used, and a workgroup barrier after phase 2 t + 1
    // both publishes it and retires every read of stage t - 1.  Nothing else
    // synchronises the waves: the two groups start each two-phase window on
    // opposite phase kinds and keep that pairing by themselves.  Stages
    // alternate between buffers 0 and 1, so the phase loop is unrolled by four
    // to make every buffer a compile-time choice.
    // The wave in its MFMA phase runs at a raised issue priority: its MFMAs
    // (one every 32 cycles) then issue as soon as their operands are in,
    // instead of waiting behind the partner wave's stream of softmax VALU
    // instructions, which otherwise wins arbitration whenever its wave is the
    // older one.
    // Phase phi = base + C (base a multiple of 4) of a wave of group G.  The
    // sweep is compiled once per group, so whether a phase is an MFMA or a
    // softmax phase is known at compile time and the only branches left in
    // the loop test wave-uniform scalars.
    auto work = [&](auto gc, auto cc, int base, const unsigned char* kl, const unsigned char* vl)
                    __attribute__((always_inline)) {
        constexpr int G = decltype(gc)::value;
        constexpr int C = decltype(cc)::value;
        const int lam = base + C - G;
        if (lam < 0) return;
        if constexpr (((C - G) & 1) != 0) {
            __builtin_amdgcn_s_setprio(0);
            v_phase(lam >> 1);
        } else {
            __builtin_amdgcn_s_setprio(2);
            m_phase((lam >> 1) - 1, kl, vl);
        }
    };

    // ---- this wave's LDS slice: next tile's Q in, previous tile's O out -------
    // Chunk k of a slice is its k-th KiB, rows [k R, (k + 1) R) with R = 1024 /
    // row bytes; a chunk moves with one 16-byte-per-lane instruction.  Each
    // wave owns its slice, so the hand-offs below need no workgroup barrier:
    // LDS accesses of one wave execute in order, and the copies of the next
    // tile's Q are complete at the barrier that closes the pair issuing them.
    unsigned char* const slice = lds_s + __builtin_amdgcn_readfirstlane(kSlice * wave);
    int pend = 0;                // 1: the slice holds an output tile not yet stored
    uint16_t* pend_dst = o_out;  // its first row in O
    int pend_rows = 0;           // its rows inside Lq
    auto store_o_chunk = [&](int k) __attribute__((always_inline)) {
        const int sl = 64 * k + lane;
        const int r = sl / S::kChunksV;
        const int c = sl % S::kChunksV;
        const u32x4 x = *reinterpret_cast<const u32x4*>(slice + r * kRowQ + 16 * (c ^ kswz<DV>(r)));
        if (r < pend_rows) *reinterpret_cast<u32x4*>(pend_dst + (size_t)r * p.o_sr + 8 * c) = x;
    };
    // next tile: this wave's Q rows and the tile's first K block
    const uint16_t* nq_src = p.q;
    int nq_rows = 0;
    bool nk_copy = false;
    int nk_key0 = 0;
    __amdgpu_buffer_rsrc_t nk_rsrc = krsrc;
    auto prefetch_q_chunk = [&](int k) __attribute__((always_inline)) {
        const int sl = 64 * k + lane;
        const int r = sl / S::kChunksK;
        const int c = (sl % S::kChunksK) ^ kswz<DQK>(r);
        const int rr = min(r, nq_rows - 1);  // rows past Lq repeat the last row
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(uniform(nq_src), (uint32_t)((kRowsPerWave - 1) * q_rb + kRowQ));
        copy_to_lds(rs, (uint32_t)(rr * q_rb + 16 * c), 0, slice + 1024 * k);
    };
    auto load_q_slice = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks)
            qf[ks] = *reinterpret_cast<const ex8*>(slice + kread[ks % kReadTable] +
                                                      (ks / kReadTable) * kReadTable * 32);
    };
    // Pair u of the sweep (phases 2u, 2u + 1), 1 <= u <= nblk.  Output chunk
    // k goes out in pair min(1 + k, nblk).  The next tile's Q chunk k comes in
    // during pair nblk - C + k (C chunks per slice) when the sweep has more
    // than C pairs after the first, else together with output chunk k.
    // Spread over the sweep, neither competes for HBM with the other
    // workgroups' tile boundaries.  The chunk ranges are computed rather than
    // tested chunk by chunk, so no per-chunk address stays live across the
    // sweep.
    auto pair_io = [&](int u) __attribute__((always_inline)) {
        if constexpr (kStage) {
            int klo = u - 1;
            int khi = (u == nblk) ? kSliceChunks : min(u, kSliceChunks);
            if (pend) {
#pragma unroll 1
                for (int k = max(klo, 0); k < khi; ++k) store_o_chunk(k);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (nblk > kSliceChunks) {
                klo = u - nblk + kSliceChunks;
                khi = klo + 1;
            }
            if (nq_rows > 0) {
#pragma unroll 1
                for (int k = max(klo, 0); k < min(khi, kSliceChunks); ++k) prefetch_q_chunk(k);
            }
        }
    };

    // next tile's Q rows of this wave, for head shapes without slices: loaded
    // straight into the Q registers once the sweep is over, so that the loads
    // run under the epilogue (packed variable-length batches load them after
    // the epilogue: their registers have no room to carry the coordinates
    // through the sweep)
    constexpr bool kQEarly = !kStage && !VARLEN;
    int nq_qw = 0, nq_lq = 0;
    size_t nq_qrow = 0;

    // ---- epilogue of a tile: O = U / l (bf16), lse = scale * ref + ln l -------
    // Piece k of the output into the slice: row l32 of the slice; this lane's
    // 4 columns 32 i + 8 r4 + 4 hi (i = k / 4, r4 = k % 4) are the half hi of
    // 16-byte chunk 4 i + r4.  The caller's row index orow comes through an
    // empty asm, so that these per-lane addresses are computed where they are
    // used, not hoisted out of the tile loop and kept in registers.
    auto out_piece = [&](int k, float inv, int orow) __attribute__((always_inline)) {
        const int i = k >> 2, r4 = k & 3;
        f32x4 x = {oacc[i][4 * r4 + 0] * inv, oacc[i][4 * r4 + 1] * inv,
                   oacc[i][4 * r4 + 2] * inv, oacc[i][4 * r4 + 3] * inv};
        const ex4 y = __builtin_convertvector(x, ex4);
        *reinterpret_cast<ex4*>(slice + orow * kRowQ + 16 * ((4 * i + r4) ^ kswz<DV>(orow)) +
                                8 * hi) = y;
    };
    // 1 / l for O's normalisation; lse stored (the output rows' head)
    auto out_head = [&]() __attribute__((always_inline)) {
        const int qi = qw + l32;
        const float ell_row = pair_sum(ell - ell_c);
        const float ell_o_row = ((lane >> 4) & 1) ? ell_o[1] : ell_o[0];
        const float inv = ell_o_row > 0.0f ? 1.0f / ell_o_row : 0.0f;
        const float lse_row = ell_row > 0.0f ? ref * scale + logf(ell_row) : kNegInf;
        if (hi == 0 && qi < Lq_t) lse_out[qrow0 + qi] = lse_row;
        return inv;
    };
    auto epilogue = [&]() __attribute__((always_inline)) {
        const int qi = qw + l32;
        const float ell_row = pair_sum(ell - ell_c);
        const float ell_o_row = ((lane >> 4) & 1) ? ell_o[1] : ell_o[0];
        const float inv = ell_o_row > 0.0f ? 1.0f / ell_o_row : 0.0f;
        const float lse_row = ell_row > 0.0f ? ref * scale + logf(ell_row) : kNegInf;
        if (o_part == nullptr) {
            if constexpr (kStage) {
                int orow = l32;
                asm volatile("" : "+v"(orow));
#pragma unroll
                for (int k = 0; k < 4 * S::kDvBlocks; ++k) out_piece(k, inv, orow);
                pend = 1;
                pend_rows = max(0, min(kRowsPerWave, Lq_t - qw));
                pend_dst = o_out + orow_w;
            } else if (qi < Lq_t) {
                uint16_t* orow = o_out + orow_w + (size_t)l32 * p.o_sr;
#pragma unroll
                for (int i = 0; i < S::kDvBlocks; ++i) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        f32x4 x = {oacc[i][4 * r4 + 0] * inv, oacc[i][4 * r4 + 1] * inv,
                                   oacc[i][4 * r4 + 2] * inv, oacc[i][4 * r4 + 3] * inv};
                        const ex4 y = __builtin_convertvector(x, ex4);
                        *reinterpret_cast<ex4*>(orow + 32 * i + 8 * r4 + 4 * hi) = y;
                    }
                }
            }
            if (hi == 0 && qi < Lq_t) lse_out[qrow0 + qi] = lse_row;
        } else if (qi < Lq_t) {
            // one split's state in fp32: its normalised output and lse
            const size_t prow = (size_t)split * p.B * p.Hq * p.Lq + qrow0 + qi;
            float* orow = o_part + prow * DV;
#pragma unroll
            for (int i = 0; i < S::kDvBlocks; ++i) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 x = {oacc[i][4 * r4 + 0] * inv, oacc[i][4 * r4 + 1] * inv,
                               oacc[i][4 * r4 + 2] * inv, oacc[i][4 * r4 + 3] * inv};
                    *reinterpret_cast<f32x4*>(orow + 32 * i + 8 * r4 + 4 * hi) = x;
                }
            }
            if (hi == 0) lse_out[prow] = lse_row;
        }
    };

    // ---- ping-pong sweep over key blocks, tile after tile -----------------------
    if (nblk > 0 && grp == 1) copy_k(0, lds_k0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- chained sweep: all tiles of the workgroup as one sequence of blocks ---
    // Without the causal mask and without key splits every tile visits the
    // same nblk blocks, so the workgroup's tiles form one sweep over
    // n_mine * nblk blocks, block J being local block J - tstart of the tile
    // that starts at tstart.  The ping-pong above then runs unchanged across
    // tile boundaries: the MFMA phase with the PV product of a tile's last
    // block also computes the scores of the next tile's first block, with the
    // next tile's Q, which the wave loaded from its slice at the end of the
    // softmax phase before.  That MFMA phase runs its PV units first and then,
    // beside its score MFMAs, finishes the tile: lse stored, O normalised
    // into the slice piece by piece.  The softmax phase of the next tile's
    // first block switches the wave's tile and resets the row state; the next
    // tile's first PV product starts O from zero.  The pipeline neither
    // drains nor refills between tiles.  A wave's hand-offs are keyed to the local block l of its
    // softmax phase: output chunk k leaves in l = k + 1 and the next tile's Q
    // chunk k arrives in l = nblk - 1 - C + k (C chunks per slice), so the
    // two never overlap when nblk >= 2 C + 2; the copies of a block that
    // belongs to the next tile (K is copied up to two blocks ahead) use that
    // tile's descriptors.  Every wave computes every block, also a wave whose
    // rows lie past Lq (it stores nothing).
    if constexpr (CHAIN) {
        static_assert(!CAUSAL && !VARLEN && kStage,
                      "chained sweeps are for non-causal launches with slices");
        const int nb = nblk;
        const int n_mine = (n_local - slot + per_round - 1) / per_round;
        const int total = n_mine * nb;
        int tstart = 0;   // sweep index of this wave's current tile's block 0
        int tile_n = -1;  // the tile after it, or -1
        __amdgpu_buffer_rsrc_t nv_rsrc = vrsrc;
        // the next tile's rows as set_tile would set them: the switch to
        // it then only copies
        int nx_qw = 0;
        size_t nx_qrow0 = 0, nx_orow_w = 0;
        auto prepare_next = [&]() __attribute__((always_inline)) {
            tile_n = tile_of_round(round + 1);
            nq_rows = 0;
            if (tile_n >= 0) {
                const TileCoord c = tile_coord<CAUSAL, VARLEN>(p, tile_n, wave_t);
                nk_rsrc = make_rsrc(p.k + c.kbase, kv_bytes(c.Lk, k_rb, kRowK));
                nv_rsrc = make_rsrc(p.v + c.vbase, kv_bytes(c.Lk, v_rb, kRowV));
                nq_rows = max(0, min(kRowsPerWave, c.Lq - c.qw));
                nq_src = p.q + c.qbase + (size_t)(nq_rows > 0 ? c.qw : 0) * p.q_sr;
                nx_qw = c.qw;
                nx_qrow0 = c.qrow0;
                nx_orow_w = c.obase + (size_t)c.qw * p.o_sr;
            }
        };
        prepare_next();
        reset_state();
        auto copy_k_at = [&](int J, unsigned char* dst) __attribute__((always_inline)) {
            const int l = J - tstart;
            if (l < nb)
                copy_kblock(krsrc, l * kBlockN, dst);
            else if (tile_n >= 0)
                copy_kblock(nk_rsrc, (l - nb) * kBlockN, dst);
        };
        auto copy_v_at = [&](int J, unsigned char* dst) __attribute__((always_inline)) {
            const int l = J - tstart;
            if (l < nb)
                copy_vblock(vrsrc, l * kBlockN, dst);
            else if (tile_n >= 0)
                copy_vblock(nv_rsrc, (l - nb) * kBlockN, dst);
        };
        auto hand_off = [&](int l) __attribute__((always_inline)) {
            if (pend && l >= 1 && l <= kSliceChunks) store_o_chunk(l - 1);
            __builtin_amdgcn_sched_barrier(0);
            const int k = l - (nb - 1 - kSliceChunks);
            if (nq_rows > 0 && k >= 0 && k < kSliceChunks) prefetch_q_chunk(k);
        };
        // V(J).  Only edge pairs (see below) hold a tile's first or last
        // block for some wave, so only they test for the tile switch and
        // for the load of the next tile's Q.
        auto v_chain = [&](int J, auto edgec) __attribute__((always_inline)) {
            constexpr bool kEdge = decltype(edgec)::value;
            if constexpr (kEdge) {
                if (J >= total) return;
                if (J - tstart == nb) {  // the next tile's first block
                    // (the previous tile's output is in the slice already:
                    // the MFMA phase before wrote it, see tile_pairs)
                    ++round;
                    tile = tile_n;
                    qw = nx_qw;
                    qrow0 = nx_qrow0;
                    orow_w = nx_orow_w;
                    krsrc = nk_rsrc;
                    vrsrc = nv_rsrc;
                    tstart += nb;
                    prepare_next();
                    reset_rows();
                }
            }
            softmax(J - tstart, kEdge && J == tstart);
            if constexpr (kEdge) {
                // the scores of the next tile's first block, in the coming
                // MFMA phase, take the next tile's Q
                if (J - tstart == nb - 1 && nq_rows > 0) load_q_slice();
            }
        };
        // Pair t of the sweep (phases 2 t, 2 t + 1) reads stage t from the
        // buffers kl, vl and fills stage t + 1 into kn, vn.  Group 0 runs
        // M(t - 1) then V(t), group 1 V(t - 1) then M(t - 1).  MK selects
        // the MFMA units of M(t - 1): 0 both products, 1 scores only (the
        // first pair), 2 PV only (the last pair), 3 both with the PV
        // product starting O from zero (M(t - 1) holds a tile's first PV),
        // 4 both with the PV units first and the finished tile's output
        // written into the slice in pieces beside the score units (M(t - 1)
        // holds a tile's last PV and the next tile's first scores).
        auto pair = [&](auto gc, auto mk, auto edgec, int t, const unsigned char* kl,
                        const unsigned char* vl, unsigned char* kn, unsigned char* vn)
                        __attribute__((always_inline)) {
            constexpr int G = decltype(gc)::value;
            constexpr int MK = decltype(mk)::value;
            auto m = [&]() __attribute__((always_inline)) {
                __builtin_amdgcn_s_setprio(2);
                float inv = 0.0f;
                int orow = 0;
                m_units(MK != 1, MK != 2, kl, vl, std::integral_constant<bool, MK == 3>{},
                        std::integral_constant<bool, MK == 4>{},
                        [&](int k) __attribute__((always_inline)) {
                            if (k < 0) {
                                inv = out_head();
                                orow = l32;
                                asm volatile("" : "+v"(orow));
                                pend = 1;
                                pend_rows = max(0, min(kRowsPerWave, Lq_t - qw));
                                pend_dst = o_out + orow_w;
                            } else {
                                out_piece(k, inv, orow);
                            }
                        });
            };
            if constexpr (G == 0) {
                m();
                hand_off(t - tstart);
                if (MK != 2) {
                    copy_v_at(t, vn);
                    __builtin_amdgcn_s_setprio(0);
                    v_chain(t, edgec);
                }
            } else {
                hand_off(t - 1 - tstart);
                copy_k_at(t + 1, kn);
                if (MK != 1) {
                    __builtin_amdgcn_s_setprio(0);
                    v_chain(t - 1, edgec);
                }
                m();
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        // The pairs of the tile whose first block is tb (nblk is even, so
        // every tile starts on stage buffers 0).  In pair tb both groups' MFMA
        // phase holds the previous tile's last PV product, and writes that
        // tile's output (MK 4); a wave's tile switch falls
        // in pair tb (group 0) or tb + 1 (group 1), its load of the next Q
        // in pair tb + nb - 1 (group 0) or the next tile's pair tb + nb
        // (group 1): these are the edge pairs, and the loop between them
        // holds only the steady form of a pair.
        auto tile_pairs = [&](auto gc, auto firstc, int tb) __attribute__((always_inline)) {
            using Both = std::integral_constant<int, 0>;
            using SOnly = std::integral_constant<int, 1>;
            using Finish = std::integral_constant<int, 4>;
            using First = std::conditional_t<decltype(firstc)::value, SOnly, Finish>;
            using Edge = std::true_type;
            using Plain = std::false_type;
            using PvFirst = std::integral_constant<int, 3>;
            pair(gc, First{}, Edge{}, tb, lds_k0, lds_v0, lds_k1, lds_v1);
            pair(gc, PvFirst{}, Edge{}, tb + 1, lds_k1, lds_v1, lds_k0, lds_v0);
            for (int t = tb + 2; t < tb + nb - 2; t += 2) {
                pair(gc, Both{}, Plain{}, t, lds_k0, lds_v0, lds_k1, lds_v1);
                pair(gc, Both{}, Plain{}, t + 1, lds_k1, lds_v1, lds_k0, lds_v0);
            }
            pair(gc, Both{}, Plain{}, tb + nb - 2, lds_k0, lds_v0, lds_k1, lds_v1);
            pair(gc, Both{}, Edge{}, tb + nb - 1, lds_k1, lds_v1, lds_k0, lds_v0);
        };
        auto chain_sweep = [&](auto gc) __attribute__((always_inline)) {
            tile_pairs(gc, std::true_type{}, 0);
            for (int tb = nb; tb < total; tb += nb) tile_pairs(gc, std::false_type{}, tb);
            pair(gc, std::integral_constant<int, 2>{}, std::true_type{}, total, lds_k0,
                 lds_v0, lds_k1, lds_v1);
        };
        if (grp == 0)
            chain_sweep(std::integral_constant<int, 0>{});
        else
            chain_sweep(std::integral_constant<int, 1>{});
        epilogue();
#pragma unroll 1
        for (int k = 0; k < kSliceChunks; ++k) store_o_chunk(k);
        return;
    }

    for (;;) {
        const int tile_n = tile_of_round(round + 1);
        const bool has_next = tile_n >= 0;
        nq_rows = 0;
        nk_copy = false;
        if (has_next) {
            const TileCoord c = tile_coord<CAUSAL, VARLEN>(p, tile_n, wave);
            const KeyRange r = key_range<CAUSAL>(p, c);
            nk_copy = r.nblk > 0;
            // its first block: the first or the last of its key range
            nk_key0 = (r.jb0 + (sweep_down(round + 1) ? r.nblk - 1 : 0)) * kBlockN;
            nk_rsrc = make_rsrc(p.k + c.kbase, kv_bytes(c.Lk, k_rb, kRowK));
            if (kStage) {
                nq_rows = max(0, min(kRowsPerWave, c.Lq - c.qw));
                nq_src = p.q + c.qbase + (size_t)(nq_rows > 0 ? c.qw : 0) * p.q_sr;
            } else if (kQEarly) {
                nq_qw = c.qw;
                nq_qrow = c.qbase + (size_t)c.qw * p.q_sr;
                nq_lq = c.Lq;
            }
        }
        reset_state();
        // Both groups run the same pairs and barriers; only the order of their
        // phase kinds differs.  In each phase the group in its softmax phase
        // also issues that phase's copy (group 1: K at even phases, group 0:
        // V at odd phases) and its own slice hand-offs.
        auto sweep = [&](auto gc) __attribute__((always_inline)) {
            constexpr int G = decltype(gc)::value;
            using C0 = std::integral_constant<int, 0>;
            using C1 = std::integral_constant<int, 1>;
            using C2 = std::integral_constant<int, 2>;
            using C3 = std::integral_constant<int, 3>;
            const int nphase = 2 * nblk + 2;
            for (int phi = 0; phi < nphase; phi += 4) {
                const int t = phi >> 1;  // pair t reads stage t (buffers 0)
                if constexpr (G == 1) {
                    pair_io(t);
                    if (t + 1 < nblk)
                        copy_k(t + 1, lds_k1);
                    else if (t == nblk && nk_copy)
                        copy_kblock(nk_rsrc, nk_key0, lds_k0);  // next tile's stage 0
                }
                work(gc, C0{}, phi, lds_k0, lds_v0);
                if constexpr (G == 0) {
                    pair_io(t);
                    if (t < nblk) copy_v(t, lds_v1);
                }
                work(gc, C1{}, phi, lds_k0, lds_v0);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (phi + 2 >= nphase) break;
                if constexpr (G == 1) {
                    pair_io(t + 1);
                    if (t + 2 < nblk)
                        copy_k(t + 2, lds_k0);
                    else if (t + 1 == nblk && nk_copy)
                        copy_kblock(nk_rsrc, nk_key0, lds_k0);
                }
                work(gc, C2{}, phi, lds_k1, lds_v1);
                if constexpr (G == 0) {
                    pair_io(t + 1);
                    if (t + 1 < nblk) copy_v(t + 1, lds_v0);
                }
                work(gc, C3{}, phi, lds_k1, lds_v1);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
        };
        if (nblk > 0) {
            if (grp == 0)
                sweep(std::integral_constant<int, 0>{});
            else
                sweep(std::integral_constant<int, 1>{});
        } else {
            // a tile without visible keys: only the hand-offs
            if constexpr (kStage) {
                if (pend) {
#pragma unroll 1
                    for (int k = 0; k < kSliceChunks; ++k) store_o_chunk(k);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (nq_rows > 0) {
#pragma unroll 1
                    for (int k = 0; k < kSliceChunks; ++k) prefetch_q_chunk(k);
                }
            }
            if (nk_copy && grp == 1) copy_kblock(nk_rsrc, nk_key0, lds_k0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        pend = 0;
        // the sweep no longer reads Q: the next tile's rows load now
        if (kQEarly && has_next) load_q_rows(nq_qw, nq_qrow, nq_lq);

        // The next tile's Q leaves the slice before this tile's O enters it.
        if (kStage && nq_rows > 0) load_q_slice();
        epilogue();
        if (!has_next) break;
        ++round;
        tile = tile_n;
        set_tile(tile);
        if (!kStage && !kQEarly) load_q_rows(qw, qrow_w, Lq_t);
    }
    // the last tile's output
    if constexpr (kStage) {
        if (pend) {
#pragma unroll 1
            for (int k = 0; k < kSliceChunks; ++k) store_o_chunk(k);
        }
    }
}

template <int DQK, int DV, bool CAUSAL, bool DEBUG, bool FP16, bool VARLEN = false,
          bool CHAIN = false>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
    dim3 grid((unsigned)p.grid), block(kThreads);
    FwdParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(
            &attn_fwd_kernel<DQK, DV, CAUSAL, DEBUG, FP16, VARLEN, CHAIN>),
        grid, block, args, 0, stream);
}

// Non-causal launches run the chained sweep when the host set p.chain
// (fwd_chained in attn_params.h states when).
template <int DQK, int DV, bool DEBUG, bool FP16>
hipError_t launch_noncausal(const FwdParams& p, hipStream_t stream) {
    if constexpr (DQK == DV) {
        if (p.chain) return launch_one<DQK, DV, false, DEBUG, FP16, false, true>(p, stream);
    }
    return launch_one<DQK, DV, false, DEBUG, FP16>(p, stream);
}

template <int DQK, int DV>
hipError_t launch_dims(const FwdParams& p, bool causal, bool debug, bool fp16,
                       hipStream_t stream) {
    if (p.plan != nullptr) {  // packed variable-length batch (bf16)
        if (debug || fp16) return hipErrorInvalidValue;
        return causal ? launch_one<DQK, DV, true, false, false, true>(p, stream)
                      : launch_one<DQK, DV, false, false, false, true>(p, stream);
    }
    if (fp16) {
        if (debug) return hipErrorInvalidValue;  // the debug variant is bf16 only
        return causal ? launch_one<DQK, DV, true, false, true>(p, stream)
                      : launch_noncausal<DQK, DV, false, true>(p, stream);
    }
    if (causal)
        return debug ? launch_one<DQK, DV, true, true, false>(p, stream)
                     : launch_one<DQK, DV, true, false, false>(p, stream);
    return debug ? launch_noncausal<DQK, DV, true, false>(p, stream)
                 : launch_noncausal<DQK, DV, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int dqk, int dv, bool causal, bool debug, bool fp16,
                      hipStream_t stream) {
    if (dqk == 64 && dv == 64) return launch_dims<64, 64>(p, causal, debug, fp16, stream);
    if (dqk == 128 && dv == 128) return launch_dims<128, 128>(p, causal, debug, fp16, stream);
    if (dqk == 192 && dv == 128) return launch_dims<192, 128>(p, causal, debug, fp16, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
