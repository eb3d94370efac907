// attn_fwd_kernel.hip -- fused exact-attention forward for gfx950 (MI355X).
//
// One workgroup = 4 waves; each wave owns 32 query rows for the whole key
// sweep (rows are split across waves, never keys, so no cross-wave output
// reduction: "Infra: Flash Attention", FA2 split-Q figure).  Keys are visited
// in blocks of 64; each block of K and V is staged through LDS, double
// buffered, and consumed by bf16 MFMA with fp32 accumulation.
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
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

template <int DQK, int DV>
struct Shape {
    static constexpr int kChunksK = DQK / 8;               // 16-byte chunks per K row
    static constexpr int kChunksV = DV / 8;                // 16-byte chunks per V row
    static constexpr int kKBytes = kBlockN * DQK * 2;      // one K block in LDS
    static constexpr int kVBytes = kBlockN * DV * 2;       // one V block in LDS
    static constexpr int kKCopies = kChunksK / kWaves;     // 1 KiB direct copies / wave
    static constexpr int kVCopies = kChunksV / kWaves;
    static constexpr int kKSteps = DQK / 16;               // MFMA k-steps for S
    static constexpr int kDvBlocks = DV / 32;              // 32-wide output blocks
    static_assert(kChunksK % kWaves == 0 && kChunksV % kWaves == 0, "blocks split evenly");
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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// Copy 16 bytes per lane from global memory straight into LDS: lane l's data
// lands at lds_dst + 16 * l (the destination is one contiguous KiB per wave).
__device__ __forceinline__ void copy_to_lds(const unsigned char* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}

// Heads up to 128 wide keep two score tiles in registers and overlap the next
// block's QK^T with the current block's softmax; wider heads would spill.
template <int DQK>
constexpr bool kPipelined = DQK <= 128;

template <int DQK, int DV, bool CAUSAL, bool DEBUG>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const FwdParams p) {
    using S = Shape<DQK, DV>;
    constexpr int kRowK = DQK * 2;  // bytes per K row
    constexpr int kRowV = DV * 2;   // bytes per V row
    // two buffers each for K and V, distinct objects so that reads of one
    // buffer are never ordered behind copies into the other
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[S::kKBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[S::kKBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[S::kVBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[S::kVBytes];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // ---- tile of this workgroup: (unit, position tile m) ------------------
    int unit, mo;
    {
        const int per_sec = p.sec_units * p.n_m;
        int local = blockIdx.x, base = 0;
        if (p.xcd_mode) {
            local = blockIdx.x >> 3;
            base = (blockIdx.x & 7) * p.upx;
        }
        const int sec = local / per_sec;
        const int r = local - sec * per_sec;
        mo = r / p.sec_units;
        unit = base + sec * p.sec_units + (r - mo * p.sec_units);
    }
    // causal tiles are ordered heaviest first (longest processing time first)
    const int m = CAUSAL ? (p.n_m - 1 - mo) : mo;
    const int hg = unit % p.n_hg;
    const int bk = unit / p.n_hg;  // b * Hkv + kv head
    const int kvh = bk % p.Hkv;
    const int b = bk / p.Hkv;
    const int hq = kvh * p.G + hg * p.Gp + (wave % p.Gp);
    const int pos0 = m * p.bm_pos;
    const int qw = pos0 + (wave / p.Gp) * kRowsPerWave;  // first row of this wave
    const int off = p.Lk - p.Lq;                          // causal diagonal offset

    const unsigned char* kbase =
        reinterpret_cast<const unsigned char*>(p.k + (size_t)bk * p.Lk * DQK);
    const unsigned char* vbase =
        reinterpret_cast<const unsigned char*>(p.v + (size_t)bk * p.Lk * DV);
    const size_t qrow0 = (size_t)(b * p.Hq + hq) * p.Lq;

    // key range of the tile and of this wave
    int kend = p.Lk;
    int wend = p.Lk;
    if (CAUSAL) {
        const int tile_last = min(p.Lq, pos0 + p.bm_pos) - 1;
        kend = min(p.Lk, tile_last + off + 1);
        const int wave_last = min(p.Lq, qw + kRowsPerWave) - 1;
        wend = min(p.Lk, wave_last + off + 1);
    }
    const int nblk = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;
    const bool wave_rows = qw < p.Lq;

    // ---- Q fragment, resident in registers for the whole sweep -----------
    // lane holds Q[qw + l32][16 ks + 8 hi .. +7] for every k-step ks
    bf16x8 qf[S::kKSteps];
    {
        const int qi = qw + l32;
        const bool ok = qi < p.Lq;
        const uint16_t* src = p.q + (qrow0 + (ok ? qi : 0)) * DQK + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks) {
            u32x4 w = ok ? load16(src + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
            qf[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // ---- direct global -> LDS copies of one K or V block -------------------
    // Copy n of the workgroup fills LDS slots [64 n, 64 n + 64); lane l takes
    // slot 64 n + l = (row r, stored chunk c') and fetches source chunk
    // c' ^ swizzle(r) of key row key0 + r.  The per-lane byte offsets within
    // a block are fixed, so they are computed once.  In a block that runs
    // past the last key, rows are clamped to the last key: those rows are
    // masked to -inf (K) or weighted by exactly 0 (V).
    uint32_t koff[S::kKCopies], voff_copy[S::kVCopies];
#pragma unroll
    for (int i = 0; i < S::kKCopies; ++i) {
        const int slot = 64 * (wave * S::kKCopies + i) + lane;
        const int r = slot / S::kChunksK;
        const int c = (slot - r * S::kChunksK) ^ kswz<DQK>(r);
        koff[i] = r * kRowK + 16 * c;
    }
#pragma unroll
    for (int i = 0; i < S::kVCopies; ++i) {
        const int slot = 64 * (wave * S::kVCopies + i) + lane;
        const int r = slot / S::kChunksV;
        const int c = (slot - r * S::kChunksV) ^ vswz<DV>(r);
        voff_copy[i] = r * kRowV + 16 * c;
    }

    auto copy_k = [&](int jb, unsigned char* dst) {
        const int key0 = jb * kBlockN;
        const unsigned char* src = kbase + (size_t)key0 * kRowK;
        if (key0 + kBlockN <= p.Lk) {
#pragma unroll
            for (int i = 0; i < S::kKCopies; ++i)
                copy_to_lds(src + koff[i], dst + 1024 * (wave * S::kKCopies + i));
        } else {
            const int last = p.Lk - 1 - key0;
#pragma unroll
            for (int i = 0; i < S::kKCopies; ++i) {
                const int r = (int)koff[i] / kRowK;
                const int rr = min(r, last);
                copy_to_lds(src + (koff[i] - (uint32_t)((r - rr) * kRowK)),
                            dst + 1024 * (wave * S::kKCopies + i));
            }
        }
    };
    auto copy_v = [&](int jb, unsigned char* dst) {
        const int key0 = jb * kBlockN;
        const unsigned char* src = vbase + (size_t)key0 * kRowV;
        if (key0 + kBlockN <= p.Lk) {
#pragma unroll
            for (int i = 0; i < S::kVCopies; ++i)
                copy_to_lds(src + voff_copy[i], dst + 1024 * (wave * S::kVCopies + i));
        } else {
            const int last = p.Lk - 1 - key0;
#pragma unroll
            for (int i = 0; i < S::kVCopies; ++i) {
                const int r = (int)voff_copy[i] / kRowV;
                const int rr = min(r, last);
                copy_to_lds(src + (voff_copy[i] - (uint32_t)((r - rr) * kRowV)),
                            dst + 1024 * (wave * S::kVCopies + i));
            }
        }
    };

    // ---- LDS read offsets (bytes within a block buffer) -----------------------
    // S^T operand: row 32 mb + l32, chunk 2 ks + hi (mb adds 32 rows)
    int kread[S::kKSteps];
#pragma unroll
    for (int ks = 0; ks < S::kKSteps; ++ks)
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

    // ---- running state -------------------------------------------------------
    f32x16 oacc[S::kDvBlocks];
#pragma unroll
    for (int i = 0; i < S::kDvBlocks; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
    float ref = kNegInf;  // exponent reference, raw q.k units
    float ell = 0.0f;     // this lane's share of sum P (fp32 P), for lse
    float ell_o = 0.0f;   // this lane's share of sum P (bf16 P), normalises O
    const float c2 = p.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    auto active = [&](int jb) { return wave_rows && jb * kBlockN < wend; };

    // S^T = K Q^T for 64 keys x 32 queries: two 32x32 tiles
    auto compute_s = [&](const unsigned char* kl, f32x16 (&s)[kBlockN / 32]) {
#pragma unroll
        for (int mb = 0; mb < kBlockN / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[mb][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks) {
#pragma unroll
            for (int mb = 0; mb < kBlockN / 32; ++mb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    kl + kread[ks] + mb * 32 * kRowK);
                s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
            }
        }
    };

    // Online softmax of one block's scores, then O^T += V^T P^T.  With
    // next_tag = true, the scores of the next block (K from next_kl, into
    // s_next) are computed in the same straight-line stretch as the
    // exponentials and the PV product, so that the MFMA work of both can
    // interleave with the VALU work.
    auto softmax_pv = [&](auto next_tag, int jb, f32x16 (&s)[kBlockN / 32],
                          const unsigned char* vl, const unsigned char* next_kl,
                          f32x16 (&s_next)[kBlockN / 32]) {
        const int key0 = jb * kBlockN;
        // mask keys past the end or past the causal diagonal
        const bool need_mask =
            (key0 + kBlockN > p.Lk) || (CAUSAL && key0 + kBlockN - 1 > qw + off);
        if (need_mask) {
            const int qi = qw + l32;
            const int klim = CAUSAL ? min(p.Lk, qi + off + 1) : p.Lk;
#pragma unroll
            for (int mb = 0; mb < kBlockN / 32; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + mb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key >= klim) s[mb][r] = kNegInf;
                }
        }

        // block max of this row (raw units)
        float bmax = kNegInf;
#pragma unroll
        for (int mb = 0; mb < kBlockN / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[mb][r]);
        bmax = pair_max(bmax);

        // conditional rescale decision
        const float cand = fmaxf(ref, bmax);
        bool moved = false;
        float acc_scale = 1.0f;
        if (ref == kNegInf) {
            ref = cand;  // first visible block: adopt its max, state is empty
        } else {
            const float delta = (ref - cand) * c2;
            if (delta < -p.threshold) {
                moved = true;
                acc_scale = __builtin_amdgcn_exp2f(delta);
                ref = cand;
            }
        }
        const unsigned long long vote = __ballot(moved);
        if (vote) {  // wave-uniform: some row of this wave moved its reference
#pragma unroll
            for (int i = 0; i < S::kDvBlocks; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= acc_scale;
            ell *= acc_scale;
            ell_o *= acc_scale;
            if (DEBUG && p.rescale_count != nullptr && lane == 0)
                atomicAdd(p.rescale_count,
                          (unsigned long long)__builtin_popcountll(vote & 0xffffffffull));
        }

        // P = 2^(x * c2 - ref * c2), rounded to bf16 in registers.  Two row
        // sums: the fp32 P for lse, and the bf16 P that feed the PV product,
        // which normalises O with exactly the weights it was built from.
        const float refc = (ref == kNegInf) ? 0.0f : ref * c2;
        float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float rb[2] = {0.0f, 0.0f};
        bf16x8 pb[kBlockN / 16];
#pragma unroll
        for (int mb = 0; mb < kBlockN / 32; ++mb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x8 e;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    e[i] = __builtin_amdgcn_exp2f(fmaf(s[mb][8 * t + i], c2, -refc));
                    rs[i & 3] += e[i];
                }
                const bf16x8 pk = __builtin_convertvector(e, bf16x8);
                pb[2 * mb + t] = pk;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bf16x2 pr = {pk[2 * i], pk[2 * i + 1]};
                    rb[i & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rb[i & 1], false);
                }
            }
        }
        ell += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        ell_o += rb[0] + rb[1];

        if constexpr (decltype(next_tag)::value) compute_s(next_kl, s_next);

        // O^T += V^T P^T, 16 keys per MFMA; the V^T operand comes from two
        // transposed LDS reads of row-major V
#pragma unroll
        for (int g = 0; g < kBlockN / 16; ++g) {
#pragma unroll
            for (int i = 0; i < S::kDvBlocks; ++i) {
                i16x4 part[2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    part[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(vl + vread[i] + (16 * g + 8 * t) * kRowV));
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g], oacc[i], 0, 0, 0);
            }
        }
    };

    // ---- sweep over key blocks --------------------------------------------
    f32x16 sa[kBlockN / 32], sb[kBlockN / 32];
    if constexpr (kPipelined<DQK>) {
        // Software pipelined.  Step j: copy K(j+2) and V(j+1) into the free
        // buffers, compute the scores of block j+1 (MFMA work independent of
        // the rest of the step), then the softmax and PV product of block j,
        // whose scores were computed in step j-1.  K runs one block ahead of
        // V, so K(j+1) and V(j) are resident during step j.  Even steps read K
        // from lds_k1 and V from lds_v0; odd steps the other buffers.
        if (nblk > 0) {
            copy_k(0, lds_k0);
            copy_v(0, lds_v0);
            if (nblk > 1) copy_k(1, lds_k1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (active(0)) compute_s(lds_k0, sa);
        }
        // a wave's active blocks are a prefix [0, nact) of the tile's blocks
        const int nact =
            wave_rows ? min(nblk, (wend + kBlockN - 1) / kBlockN) : 0;
        const std::true_type with_next{};
        const std::false_type last{};
        for (int jb = 0; jb < nblk; jb += 2) {
            // even step j = jb
            if (jb + 2 < nblk) copy_k(jb + 2, lds_k0);
            if (jb + 1 < nblk) copy_v(jb + 1, lds_v1);
            if (jb + 1 < nact)
                softmax_pv(with_next, jb, sa, lds_v0, lds_k1, sb);
            else if (jb < nact)
                softmax_pv(last, jb, sa, lds_v0, lds_k1, sb);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (jb + 1 >= nblk) break;
            // odd step j = jb + 1
            if (jb + 3 < nblk) copy_k(jb + 3, lds_k1);
            if (jb + 2 < nblk) copy_v(jb + 2, lds_v0);
            if (jb + 2 < nact)
                softmax_pv(with_next, jb + 1, sb, lds_v1, lds_k0, sa);
            else if (jb + 1 < nact)
                softmax_pv(last, jb + 1, sb, lds_v1, lds_k0, sa);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else {
        // One score tile live (wide heads): step j copies block j+1 into the
        // free buffers, then computes scores, softmax and PV of block j.
        if (nblk > 0) {
            copy_k(0, lds_k0);
            copy_v(0, lds_v0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        for (int jb = 0; jb < nblk; jb += 2) {
            if (jb + 1 < nblk) {
                copy_k(jb + 1, lds_k1);
                copy_v(jb + 1, lds_v1);
            }
            if (active(jb)) {
                compute_s(lds_k0, sa);
                softmax_pv(std::false_type{}, jb, sa, lds_v0, lds_k1, sb);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (jb + 1 >= nblk) break;
            if (jb + 2 < nblk) {
                copy_k(jb + 2, lds_k0);
                copy_v(jb + 2, lds_v0);
            }
            if (active(jb + 1)) {
                compute_s(lds_k1, sa);
                softmax_pv(std::false_type{}, jb + 1, sa, lds_v1, lds_k0, sb);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        (void)sb;
    }

    // ---- epilogue: O = U / l (bf16), lse = scale * ref + ln l ----------------
    const int qi = qw + l32;
    const float ell_row = pair_sum(ell);
    const float ell_o_row = pair_sum(ell_o);
    if (qi < p.Lq) {
        const float inv = ell_o_row > 0.0f ? 1.0f / ell_o_row : 0.0f;
        uint16_t* orow = p.o + (qrow0 + qi) * DV;
#pragma unroll
        for (int i = 0; i < S::kDvBlocks; ++i) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                typedef float f32x4 __attribute__((ext_vector_type(4)));
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                f32x4 x = {oacc[i][4 * r4 + 0] * inv, oacc[i][4 * r4 + 1] * inv,
                           oacc[i][4 * r4 + 2] * inv, oacc[i][4 * r4 + 3] * inv};
                const bf16x4 y = __builtin_convertvector(x, bf16x4);
                *reinterpret_cast<bf16x4*>(orow + 32 * i + 8 * r4 + 4 * hi) = y;
            }
        }
        if (hi == 0)
            p.lse[qrow0 + qi] = ell_row > 0.0f ? ref * p.scale + logf(ell_row) : kNegInf;
    }
}

template <int DQK, int DV, bool CAUSAL, bool DEBUG>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
    const long long tiles = (long long)p.units * p.n_m;
    dim3 grid((unsigned)tiles), block(kThreads);
    FwdParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<DQK, DV, CAUSAL, DEBUG>),
                           grid, block, args, 0, stream);
}

template <int DQK, int DV>
hipError_t launch_dims(const FwdParams& p, bool causal, bool debug, hipStream_t stream) {
    if (causal)
        return debug ? launch_one<DQK, DV, true, true>(p, stream)
                     : launch_one<DQK, DV, true, false>(p, stream);
    return debug ? launch_one<DQK, DV, false, true>(p, stream)
                 : launch_one<DQK, DV, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int dqk, int dv, bool causal, bool debug,
                      hipStream_t stream) {
    if (dqk == 64 && dv == 64) return launch_dims<64, 64>(p, causal, debug, stream);
    if (dqk == 128 && dv == 128) return launch_dims<128, 128>(p, causal, debug, stream);
    if (dqk == 192 && dv == 128) return launch_dims<192, 128>(p, causal, debug, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
