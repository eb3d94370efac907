// attn_decode_kernel.hip -- split-key attention forward for few query rows
// per K/V head (decoding), gfx950.
//
// When a K/V head serves at most 16 query rows (Lq positions times the
// G = Hq / Hkv query heads that share it), the fused kernel's 32-row MFMA
// tiles run mostly on padding and the key stream is paced by them rather
// than by HBM.  This kernel streams keys instead: the rows sit on the N side
// of 16x16 MFMAs, every wave walks its own contiguous run of keys, and the
// run's state is merged with the other waves' at the end.  Its output is the
// split-key path's: for each key split, the normalised output of the split
// and its log-sum-exp, merged afterwards by attn_merge ("Infra: Flash
// Attention", sections on computing softmax in segments and on prefill
// versus decode).
//
// Per 16-key step of a wave:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, K rows as A (from LDS), the
//                    query rows as B (registers); lane l holds keys
//                    4 (l / 16) + i of row l % 16
//   online softmax   base 2, reference moved only when the block maximum
//                    passes it by more than the threshold ("Flash Attention 4
//                    ..." ch. 13, online softmax with conditional rescaling);
//                    the causal mask is aligned bottom-right
//   O^T += V^T P^T   v_mfma_f32_16x16x16_bf16: the score accumulator, rounded
//                    to bf16, is the B operand as it stands; V^T comes from
//                    ds_read_b64_tr_b16 on the row-major V rows
// K and V rows are copied from HBM straight into the wave's own LDS slots
// (buffer loads to LDS), two steps ahead of their use, so the waves need no
// barrier until the final merge.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kNegInf = -__builtin_inff();
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecStages = 3;  // LDS slots per wave: two steps in flight while one is computed
constexpr int kDecLook = kDecStages - 1;

template <int DQK, int DV>
struct Dec {
    static constexpr int kChunksK = DQK / 8;               // 16-byte chunks per K row
    static constexpr int kChunksV = DV / 8;                // and per V row
    static constexpr int kRowK = DQK * 2;                  // bytes per K row
    static constexpr int kRowV = DV * 2;                   // bytes per V row
    static constexpr int kKBytes = kDecKeys * kRowK;       // 16 rows of K
    static constexpr int kVBytes = kDecKeys * kRowV;       // 16 rows of V
    static constexpr int kCopiesK = kKBytes / 1024;        // 1 KiB wave copies per block
    static constexpr int kCopiesV = kVBytes / 1024;
    static constexpr int kCopies = kCopiesK + kCopiesV;    // copy instructions per step
    static constexpr int kStageBytes = kKBytes + kVBytes;  // K rows, then V rows
    static constexpr int kWaveBytes = kDecStages * kStageBytes;
    static constexpr int kKSteps = DQK / 32;               // k-steps of the score product
    static constexpr int kDvBlocks = DV / 16;              // 16-wide blocks of the output
    static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "whole wave copies");
    // the final merge keeps each wave's O^T [DV][16] and its row statistics in
    // the wave's own slots
    static_assert(DV * kDecRows * 4 + 3 * kDecRows * 4 <= kWaveBytes, "merge area fits");
};

// K rows in LDS: chunk c of row r stored at slot c ^ kswz(r), so the 16 rows
// one score operand read touches (same chunk) hit distinct bank groups (8
// distinct groups when the row has 8 or 24 chunks: the XOR must keep the slot
// inside its aligned group of 8 and so inside the row).
template <int DQK>
__device__ __forceinline__ int kswz(int r) {
    return (DQK == 128) ? (r & 15) : (r & 7);
}
// V rows in LDS: chunk c of row r at slot c ^ vswz(r).  A transposed read
// takes 8 bytes from each of 4 consecutive rows at two adjacent chunks; the
// XOR moves consecutive rows to different 32-byte windows.
template <int DV>
__device__ __forceinline__ int vswz(int r) {
    return (DV == 128) ? 2 * (r & 7) : 2 * (r & 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from HBM into LDS: lane l reads at byte soff + voff and
// its data lands at lds_dst + 16 l.  Every K and V byte is read exactly once
// here, so the loads carry the non-temporal cache policy (aux bit 1): they do
// not displace reusable lines (measured 5.87 -> 6.41 TB/s on one decode step
// of B8 Hq32 Hkv8 over 32k keys).
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                            uint32_t soff, void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_dst, 16, voff, soff, 0,
                                             kStreamPolicy);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their
// maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ float xor_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xor_sum(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(kDecThreads) void attn_decode_kernel(const DecParams p) {
    using S = Dec<DQK, DV>;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kDecWaves * S::kWaveBytes];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;  // the row this lane's accumulators belong to
    const int lg = lane >> 4;   // its group of 4 keys (score product) or dims (output)

    // workgroup -> (key split, batch, K/V head)
    const int unit = blockIdx.x / p.n_split;
    const int split = blockIdx.x - unit * p.n_split;
    const int kvh = unit % p.Hkv;
    const int b = unit / p.Hkv;
    const size_t head = (size_t)(b * p.Hkv + kvh) * p.Lk;  // row of key 0 of the head
    // one head's rows span less than 2^31 bytes (checked on the host)
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + head * DQK, (uint32_t)p.Lk * S::kRowK);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + head * DV, (uint32_t)p.Lk * S::kRowV);

    // Row n of the 16 is query position n % Lq of query head kvh * G + n / Lq;
    // rows n >= R are padding (zero queries, never stored).
    const int n = l16;
    const bool row_ok = n < p.R;
    const int hq = kvh * p.G + (row_ok ? n / p.Lq : 0);
    const int qi = row_ok ? n % p.Lq : 0;
    // keys this row may see: all, or with the bottom-right causal mask those
    // up to qi + Lk - Lq
    const int klim = CAUSAL ? min(p.Lk, qi + p.Lk - p.Lq + 1) : p.Lk;

    // query rows as the B operand: lane l holds row l % 16, dims 32 ks + 8 lg .. + 7
    bf16x8 qf[S::kKSteps];
    {
        const uint16_t* qrow = p.q + ((size_t)(b * p.Hq + hq) * p.Lq + qi) * DQK;
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks) {
            const u32x4 w = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg)
                                   : u32x4{0u, 0u, 0u, 0u};
            qf[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // this wave's keys: a quarter of the split, in 16-key steps
    const int W = p.split_w;  // keys per split, a multiple of 64
    const int k0 = split * W;
    const int k1 = min(p.Lk, k0 + W);
    const int wk0 = k0 + wave * (W / kDecWaves);
    const int wk1 = min(k1, wk0 + W / kDecWaves);
    const int nsteps = wk1 > wk0 ? (wk1 - wk0 + kDecKeys - 1) / kDecKeys : 0;

    unsigned char* const wlds = lds + __builtin_amdgcn_readfirstlane(wave * S::kWaveBytes);

    // per-lane copy offsets within a 16-row block: copy c, lane l fills LDS
    // slot 64 c + l = (row r, stored chunk c') from source chunk c' ^ swizzle(r)
    uint32_t koff[S::kCopiesK], voff[S::kCopiesV];
    int krow[S::kCopiesK], vrow[S::kCopiesV];
#pragma unroll
    for (int c = 0; c < S::kCopiesK; ++c) {
        const int sl = 64 * c + lane;
        const int r = sl / S::kChunksK;
        const int cs = sl - r * S::kChunksK;
        krow[c] = r;
        koff[c] = r * S::kRowK + 16 * (cs ^ kswz<DQK>(r));
    }
#pragma unroll
    for (int c = 0; c < S::kCopiesV; ++c) {
        const int sl = 64 * c + lane;
        const int r = sl / S::kChunksV;
        const int cs = sl - r * S::kChunksV;
        vrow[c] = r;
        voff[c] = r * S::kRowV + 16 * (cs ^ vswz<DV>(r));
    }
    // copies of step t into slot t % kDecStages; rows past the last key repeat the
    // last key (masked to -inf, weighted by exactly 0)
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int key0 = wk0 + kDecKeys * t;
        unsigned char* slot = wlds + (t % kDecStages) * S::kStageBytes;
        int sd = __builtin_amdgcn_readfirstlane((int)(slot - lds));
        const int last = p.Lk - 1 - key0;
#pragma unroll
        for (int c = 0; c < S::kCopiesK; ++c) {
            const uint32_t back = (uint32_t)(max(krow[c] - last, 0) * S::kRowK);
            copy_to_lds(krs, koff[c] - back, (uint32_t)key0 * S::kRowK, lds + sd + 1024 * c);
        }
#pragma unroll
        for (int c = 0; c < S::kCopiesV; ++c) {
            const uint32_t back = (uint32_t)(max(vrow[c] - last, 0) * S::kRowV);
            copy_to_lds(vrs, voff[c] - back, (uint32_t)key0 * S::kRowV,
                        lds + sd + S::kKBytes + 1024 * c);
        }
    };

    // LDS read offsets: score operand (row l % 16, chunk 4 ks + lg) and the
    // transposed V read (16-lane group lg, index 4 r + j: row 4 lg + r, dims
    // 16 blk + 4 j .. + 3; lane l then receives dim 16 blk + l % 16 of rows
    // 4 lg .. 4 lg + 3)
    int kread[S::kKSteps];
#pragma unroll
    for (int ks = 0; ks < S::kKSteps; ++ks)
        kread[ks] = l16 * S::kRowK + 16 * ((4 * ks + lg) ^ kswz<DQK>(l16));
    int vread[S::kDvBlocks];
    {
        const int r = 4 * lg + (l16 >> 2);
        const int j = l16 & 3;
#pragma unroll
        for (int blk = 0; blk < S::kDvBlocks; ++blk)
            vread[blk] = r * S::kRowV + 16 * ((2 * blk + (j >> 1)) ^ vswz<DV>(r)) + 8 * (j & 1);
    }

    const float c2 = p.scale_log2;
    f32x4 oacc[S::kDvBlocks];
#pragma unroll
    for (int blk = 0; blk < S::kDvBlocks; ++blk) oacc[blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float ref = kNegInf;  // reference of row l % 16, raw q.k units
    float ell = 0.0f, ell_c = 0.0f;  // fp32 sum of P over this lane's keys, compensated
    float ell_o = 0.0f;              // sum of the bf16 P that enter the PV product

    for (int t = 0; t < min(kDecLook, nsteps); ++t) issue(t);
    for (int t = 0; t < nsteps; ++t) {
        // step t's copies have landed once only those of the steps issued
        // after it remain in flight (kCopies instructions per step)
        static_assert(kDecLook == 2, "one wait per possible number of later steps");
        if (min(nsteps, t + kDecLook) - (t + 1) == 1)
            wait_vmcnt<S::kCopies>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
        // step t + kDecLook reuses the slot of step t - 1, whose reads have returned
        if (t + kDecLook < nsteps) issue(t + kDecLook);
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char* kl = wlds + (t % kDecStages) * S::kStageBytes;
        const unsigned char* vl = kl + S::kKBytes;
        const int key0 = wk0 + kDecKeys * t;

        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + kread[ks]);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], s, 0, 0, 0);
        }
        // keys past the end, past the wave's run or past the row's causal limit
        const int lim = min(klim, wk1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (key0 + 4 * lg + i >= lim) s[i] = kNegInf;

        const float bmax = xor_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        const float cand = fmaxf(ref, bmax);
        const float delta = (ref - cand) * c2;  // -inf on the first visible block, NaN before
        const bool moved = delta < -p.threshold;
        const float acc_scale = moved ? __builtin_amdgcn_exp2f(delta) : 1.0f;
        ref = moved ? cand : ref;
        if (__ballot(moved)) {
#pragma unroll
            for (int blk = 0; blk < S::kDvBlocks; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[blk][i] *= acc_scale;
            ell *= acc_scale;
            ell_c *= acc_scale;
            ell_o *= acc_scale;
        }
        const float refc = (ref == kNegInf) ? 0.0f : ref * c2;
        f32x4 pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -refc));
        const bf16x4 pb = __builtin_convertvector(pv, bf16x4);
        const float bsum = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        const float y = bsum - ell_c;
        const float tt = ell + y;
        ell_c = (tt - ell) - y;
        ell = tt;
        ell_o += ((float)pb[0] + (float)pb[1]) + ((float)pb[2] + (float)pb[3]);

        const i16x4 pbi = __builtin_bit_cast(i16x4, pb);
#pragma unroll
        for (int blk = 0; blk < S::kDvBlocks; ++blk) {
            const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vl + vread[blk]));
            oacc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbi, oacc[blk], 0, 0, 0);
        }
    }

    // ---- merge of the waves' states and the split's output -------------------
    // row statistics over the 4 lane groups that hold a row's keys
    const float ell_row = xor_sum(ell - ell_c);
    const float ell_o_row = xor_sum(ell_o);
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with its slots
    // wave w's area: O^T [DV][16] fp32, then ref, ell and ell_o of the 16 rows
    float* area = reinterpret_cast<float*>(wlds);
#pragma unroll
    for (int blk = 0; blk < S::kDvBlocks; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) area[(16 * blk + 4 * lg + i) * kDecRows + l16] = oacc[blk][i];
    if (lane < kDecRows) {
        area[DV * kDecRows + lane] = ref;
        area[DV * kDecRows + kDecRows + lane] = ell_row;
        area[DV * kDecRows + 2 * kDecRows + lane] = ell_o_row;
    }
    __syncthreads();

    // thread t covers output dim t % DV of rows t / DV, t / DV + kDecThreads / DV, ...
    const int dim = tid % DV;
    for (int r = tid / DV; r < p.R; r += kDecThreads / DV) {
        float m = kNegInf;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            const float* a = reinterpret_cast<const float*>(lds + w * S::kWaveBytes);
            m = fmaxf(m, a[DV * kDecRows + r]);
        }
        float L = 0.0f, Lo = 0.0f, u = 0.0f;
        if (m != kNegInf) {
#pragma unroll
            for (int w = 0; w < kDecWaves; ++w) {
                const float* a = reinterpret_cast<const float*>(lds + w * S::kWaveBytes);
                const float rw = a[DV * kDecRows + r];
                const float e = (rw == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((rw - m) * c2);
                L += e * a[DV * kDecRows + kDecRows + r];
                Lo += e * a[DV * kDecRows + 2 * kDecRows + r];
                u += e * a[dim * kDecRows + r];
            }
        }
        const int hq_r = kvh * p.G + r / p.Lq;
        const int qi_r = r % p.Lq;
        const size_t prow = (((size_t)split * p.B + b) * p.Hq + hq_r) * p.Lq + qi_r;
        p.o_part[prow * DV + dim] = Lo > 0.0f ? u / Lo : 0.0f;
        if (dim == 0) p.lse_part[prow] = L > 0.0f ? m * p.scale + logf(L) : kNegInf;
    }
}

template <int DQK, int DV, bool CAUSAL>
hipError_t launch_d(const DecParams& p, hipStream_t stream) {
    DecParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_decode_kernel<DQK, DV, CAUSAL>),
                           dim3((unsigned)p.grid), dim3(kDecThreads), args, 0, stream);
}

template <int DQK, int DV>
hipError_t launch_dims(const DecParams& p, bool causal, hipStream_t stream) {
    return causal ? launch_d<DQK, DV, true>(p, stream) : launch_d<DQK, DV, false>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecParams& p, int dqk, int dv, bool causal, hipStream_t stream) {
    if (dqk == 64 && dv == 64) return launch_dims<64, 64>(p, causal, stream);
    if (dqk == 128 && dv == 128) return launch_dims<128, 128>(p, causal, stream);
    if (dqk == 192 && dv == 128) return launch_dims<192, 128>(p, causal, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
