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
    static constexpr int kKBytes = kBlockN * DQK * 2;      // one K block in LDS
    static constexpr int kVBytes = kBlockN * DV * 2;       // one V^T block in LDS
    static constexpr int kBufBytes = kKBytes + kVBytes;
    static constexpr int kLdsBytes = 2 * kBufBytes;        // double buffered
    static constexpr int kKLoads = kBlockN * kChunksK / kThreads;  // 16 B loads / thread
    static constexpr int kVItems = (kBlockN / 4) * (DV / 8);      // (4 keys x 8 dv) items
    static constexpr int kVIters = (kVItems + kThreads - 1) / kThreads;
    static constexpr int kKSteps = DQK / 16;               // MFMA k-steps for S
    static constexpr int kDvBlocks = DV / 32;              // 32-wide output blocks
    static_assert(kBlockN * kChunksK % kThreads == 0, "K block must split evenly");
    static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims must fit the MFMA tiles");
};

// Byte offset of 16-byte chunk c of key row r in a K block.  The chunk index
// is XOR-swizzled with the row so that the 16 lanes reading one chunk column
// of 16 consecutive rows hit 16 distinct bank groups.
template <int DQK>
__device__ __forceinline__ int k_offset(int r, int c) {
    const int swz = (DQK == 128) ? (r & 15) : ((r >> 1) & 7);
    return r * (DQK * 2) + ((c ^ swz) << 4);
}

// V^T block: row = output dim (DV rows), 64 keys per row (128 bytes).  Within
// each group of 16 keys the keys are permuted so that one 16-byte chunk holds
// the 8 keys a lane feeds to one PV MFMA: lane half h takes keys
// {4h..4h+3, 8+4h..8+4h+3}.  Key kk sits in chunk 2*(kk/16) + ((kk>>2)&1) at
// element ((kk>>3)&1)*4 + (kk&3).  Chunks are XOR-swizzled by row pair.
__device__ __forceinline__ int vt_offset(int row, int chunk) {
    return row * (kBlockN * 2) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

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

template <int DQK, int DV, bool CAUSAL, bool DEBUG>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const FwdParams p) {
    using S = Shape<DQK, DV>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[S::kLdsBytes];

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

    const uint16_t* kbase = p.k + (size_t)bk * p.Lk * DQK;
    const uint16_t* vbase = p.v + (size_t)bk * p.Lk * DV;
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

    // ---- K/V block staging: global -> registers -> LDS --------------------
    u32x4 kst[S::kKLoads];
    u32x4 vst[S::kVIters][4];

    auto load_block = [&](int jb) {
        const int key0 = jb * kBlockN;
#pragma unroll
        for (int it = 0; it < S::kKLoads; ++it) {
            const int item = tid + it * kThreads;
            const int r = item / S::kChunksK;
            const int c = item - r * S::kChunksK;
            const int key = key0 + r;
            kst[it] = key < p.Lk ? load16(kbase + (size_t)key * DQK + 8 * c)
                                 : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < S::kVIters; ++it) {
            const int item = tid + it * kThreads;
            if (item < S::kVItems) {
                const int kg = item & 15;  // group of 4 keys
                const int c8 = item >> 4;  // 8-wide chunk of the value dim
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = key0 + 4 * kg + e;
                    vst[it][e] = key < p.Lk ? load16(vbase + (size_t)key * DV + 8 * c8)
                                            : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };

    auto store_block = [&](int buf) {
        unsigned char* kl = lds + buf * S::kBufBytes;
        unsigned char* vl = kl + S::kKBytes;
#pragma unroll
        for (int it = 0; it < S::kKLoads; ++it) {
            const int item = tid + it * kThreads;
            const int r = item / S::kChunksK;
            const int c = item - r * S::kChunksK;
            *reinterpret_cast<u32x4*>(kl + k_offset<DQK>(r, c)) = kst[it];
        }
#pragma unroll
        for (int it = 0; it < S::kVIters; ++it) {
            const int item = tid + it * kThreads;
            if (item < S::kVItems) {
                const int kg = item & 15;
                const int c8 = item >> 4;
                // 4 keys x 8 dims -> 8 rows of V^T, 4 consecutive slots each
                const int chunk = 2 * (kg >> 2) + (kg & 1);
                const int elem_byte = ((kg >> 1) & 1) * 8;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t a0 = vst[it][0][e], a1 = vst[it][1][e];
                    const uint32_t a2 = vst[it][2][e], a3 = vst[it][3][e];
                    const u32x2 even = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
                    const u32x2 odd = {(a0 >> 16) | (a1 & 0xffff0000u),
                                       (a2 >> 16) | (a3 & 0xffff0000u)};
                    const int row = 8 * c8 + 2 * e;
                    *reinterpret_cast<u32x2*>(vl + vt_offset(row, chunk) + elem_byte) = even;
                    *reinterpret_cast<u32x2*>(vl + vt_offset(row + 1, chunk) + elem_byte) = odd;
                }
            }
        }
    };

    // ---- running state -------------------------------------------------------
    f32x16 oacc[S::kDvBlocks];
#pragma unroll
    for (int i = 0; i < S::kDvBlocks; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
    float ref = kNegInf;  // exponent reference, raw q.k units
    float ell = 0.0f;     // this lane's share of the denominator
    const float c2 = p.scale_log2;

    if (nblk > 0) {
        load_block(0);
        store_block(0);
        __syncthreads();
    }

    for (int jb = 0; jb < nblk; ++jb) {
        const int buf = jb & 1;
        if (jb + 1 < nblk) load_block(jb + 1);
        const int key0 = jb * kBlockN;

        if (wave_rows && key0 < wend) {
            const unsigned char* kl = lds + buf * S::kBufBytes;
            const unsigned char* vl = kl + S::kKBytes;

            // S^T = K Q^T for 64 keys x 32 queries: two 32x32 tiles
            f32x16 s[kBlockN / 32];
#pragma unroll
            for (int mb = 0; mb < kBlockN / 32; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[mb][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < S::kKSteps; ++ks) {
#pragma unroll
                for (int mb = 0; mb < kBlockN / 32; ++mb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        kl + k_offset<DQK>(mb * 32 + l32, 2 * ks + hi));
                    s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
                }
            }

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
                if (DEBUG && p.rescale_count != nullptr && lane == 0)
                    atomicAdd(p.rescale_count,
                              (unsigned long long)__builtin_popcountll(vote & 0xffffffffull));
            }

            // P = 2^(x * c2 - ref * c2), kept in registers as bf16
            const float refc = (ref == kNegInf) ? 0.0f : ref * c2;
            float rs = 0.0f;
            bf16x8 pb[kBlockN / 16];
#pragma unroll
            for (int mb = 0; mb < kBlockN / 32; ++mb) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x8 e;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        e[i] = __builtin_amdgcn_exp2f(fmaf(s[mb][8 * t + i], c2, -refc));
                        rs += e[i];
                    }
                    pb[2 * mb + t] = __builtin_convertvector(e, bf16x8);
                }
            }
            ell += rs;

            // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
            for (int g = 0; g < kBlockN / 16; ++g) {
#pragma unroll
                for (int i = 0; i < S::kDvBlocks; ++i) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        vl + vt_offset(32 * i + l32, 2 * g + hi));
                    oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g], oacc[i], 0, 0, 0);
                }
            }
        }

        if (jb + 1 < nblk) store_block(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = U / l (bf16), lse = scale * ref + ln l ----------------
    const int qi = qw + l32;
    const float ell_row = pair_sum(ell);
    if (qi < p.Lq) {
        const float inv = ell_row > 0.0f ? 1.0f / ell_row : 0.0f;
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
