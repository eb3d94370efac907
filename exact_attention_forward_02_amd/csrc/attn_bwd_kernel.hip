// attn_bwd_kernel.hip -- backward pass of exact attention for gfx950 (MI355X).
//
// Gradients of <dO, O> by recomputation ("Infra: Flash Attention", section on
// why the backward pass recomputes, and the section deriving the gradients
// block by block): with P = exp(scale * Q K^T - lse) rebuilt from the
// forward's lse,
//     dV = P^T dO,   dP = dO V^T,   D_i = dO_i . O_i,
//     dS = P (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
// Three kernels, none of which writes any intermediate to HBM:
//   attn_bwd_delta_kernel  D_i = dO_i . O_i, one row per 16 (or 8) lanes;
//   attn_bwd_dkdv_kernel   one workgroup per (K/V head, 128 keys): each wave
//                          owns 32 keys, holds their K and V rows as MFMA
//                          operands, and accumulates dK^T and dV^T over every
//                          query block of every query head the K/V head
//                          serves (grouped-query attention needs no atomics);
//   attn_bwd_dq_kernel     one workgroup per (query head, 128 queries): each
//                          wave owns 32 query rows, holds its Q and dO rows as
//                          MFMA operands, and streams K/V blocks through LDS,
//                          like the forward pass.
// MFMA v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Operand A is read
// from LDS (rows with ds_read_b128, transposed with ds_read_b64_tr_b16);
// operand B is a register fragment: the wave's own K/V or Q/dO rows, or the
// bf16 P / dS fragments, whose row order the transposed reads follow.  The
// causal mask is bottom-right aligned (query i sees keys j <= i + Lk - Lq).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdThreads = 256;  // 4 waves, one per SIMD
constexpr int kBlk = 64;          // rows of a staged Q/dO (or K/V) block
constexpr float kLog2e = 1.4426950408889634f;

// LDS block layout: row r of D bf16, 16-byte chunk c stored at c ^ swz(r).
// The swizzle depends on r mod 4 only, so the transposed reads (4 rows at a
// time) and the row reads both address any 4-aligned row group the same way.
template <int D>
__device__ __forceinline__ int swz(int r) {
    const int q = r & 3;
    return (D == 128) ? (4 * q + 2 * (q >> 1)) : (4 * (q & 1) + 2 * (q >> 1));
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Stage rows [row0, row0 + 64) of a [L, D] head (rows past L repeat row
// L - 1; callers mask them) into an LDS block.
template <int D>
__device__ __forceinline__ void stage_rows(const uint16_t* head, int row0, int L,
                                           unsigned char* dst, int tid) {
    constexpr int kChunks = D / 8;
#pragma unroll
    for (int n = 0; n < kBlk * kChunks / kBwdThreads; ++n) {
        const int c = tid + n * kBwdThreads;
        const int r = c / kChunks;
        const int ch = c % kChunks;
        const int row = min(row0 + r, L - 1);
        const u32x4 x = load16(head + (size_t)row * D + 8 * ch);
        *reinterpret_cast<u32x4*>(dst + r * (D * 2) + 16 * (ch ^ swz<D>(r))) = x;
    }
}

// A operand from rows of an LDS block: lane l reads row m0 + (l & 31),
// elements 16 ks + 8 (l >> 5) .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const unsigned char* blk, int m0, int ks, int lane) {
    const int m = m0 + (lane & 31);
    const int ch = 2 * ks + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(blk + m * (D * 2) + 16 * (ch ^ swz<D>(m)));
}

// Per-lane byte offset of the transposed reads: with 16-lane group g = l / 16
// and index 4 r + j inside it, the lane reads 8 bytes of row 4 (g / 2) + r at
// columns 32 i + 16 (g & 1) + 4 j .. + 3 (i added by the caller).
template <int D>
__device__ __forceinline__ int tr_offset(int lane, int i) {
    const int tg = lane >> 4, ti = lane & 15, tr = ti >> 2, tj = ti & 3;
    const int row = 4 * (tg >> 1) + tr;
    const int cl = 2 * (tg & 1) + (tj >> 1);
    return row * (D * 2) + 16 * ((4 * i + cl) ^ swz<D>(row)) + 8 * (tj & 1);
}

// A operand = (block rows 16 g .. 16 g + 15)^T, columns 32 i .. 32 i + 31:
// lane l receives column 32 i + (l & 31) at the 8 rows whose values the
// B fragment g (rows 8 (r >> 2) + 4 (l >> 5) + (r & 3) of an accumulator)
// carries in the same order.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* blk, int off, int g) {
    i16x4 part[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        part[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(blk + off + (16 * g + 8 * t) * (D * 2)));
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator register r for lane half hi: 8 (r >> 2) + 4 hi + (r & 3).
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// ---- D_i = dO_i . O_i --------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const BwdParams p, long long rows) {
    constexpr int kLanes = D / 8;  // lanes per row, 16 bytes each
    constexpr int kRows = 256 / kLanes;
    const long long row = (long long)blockIdx.x * kRows + threadIdx.x / kLanes;
    const int c = threadIdx.x % kLanes;
    float acc = 0.0f;
    if (row < rows) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, load16(p.dout + row * D + 8 * c));
        const bf16x8 b = __builtin_bit_cast(bf16x8, load16(p.o + row * D + 8 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
#pragma unroll
    for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kLanes);
    if (row < rows && c == 0) p.delta[row] = acc;
}

// ---- dK, dV ------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void attn_bwd_dkdv_kernel(const BwdParams p) {
    constexpr int kKs = D / 16;   // k-steps over the head dim
    constexpr int kDb = D / 32;   // 32-wide output blocks
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf[kBlk * D * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char dobuf[kBlk * D * 2];
    __shared__ __attribute__((aligned(16))) float lsebuf[kBlk];
    __shared__ __attribute__((aligned(16))) float dbuf[kBlk];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int nkb = (p.Lk + 127) / 128;
    const int bk = blockIdx.x / nkb;  // b * Hkv + kv head
    const int kb = blockIdx.x % nkb;
    const int b = bk / p.Hkv, hk = bk % p.Hkv;
    const int key0 = kb * 128 + wave * 32;  // this wave's first key
    const int key = key0 + l32;             // the key of this lane's accumulator column
    const int off = p.Lk - p.Lq;
    const float c2 = p.scale_log2;

    // the wave's K and V rows as B operands (rows past Lk repeat the last key)
    const int krow = min(key, p.Lk - 1);
    const uint16_t* kh = p.k + (size_t)bk * p.Lk * D;
    const uint16_t* vh = p.v + (size_t)bk * p.Lk * D;
    bf16x8 kf[kKs], vf[kKs];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
        kf[ks] = __builtin_bit_cast(bf16x8, load16(kh + (size_t)krow * D + 16 * ks + 8 * hi));
        vf[ks] = __builtin_bit_cast(bf16x8, load16(vh + (size_t)krow * D + 16 * ks + 8 * hi));
    }
    f32x16 dkt[kDb], dvt[kDb];
#pragma unroll
    for (int i = 0; i < kDb; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkt[i][r] = dvt[i][r] = 0.0f;
    int tro[kDb];
#pragma unroll
    for (int i = 0; i < kDb; ++i) tro[i] = tr_offset<D>(lane, i);

    // causal: queries before qstart see none of this workgroup's keys
    int qb0 = 0;
    if (CAUSAL) qb0 = max(0, kb * 128 - off) / kBlk;
    const int nqb = (p.Lq + kBlk - 1) / kBlk;
    const f32x16 zero = {};
    for (int g = 0; g < p.G; ++g) {
        const size_t qrow0 = (size_t)(b * p.Hq + hk * p.G + g) * p.Lq;
        for (int qb = qb0; qb < nqb; ++qb) {
            const int i0 = qb * kBlk;
            __syncthreads();  // the previous block's reads are done
            stage_rows<D>(p.q + qrow0 * D, i0, p.Lq, qbuf, tid);
            stage_rows<D>(p.dout + qrow0 * D, i0, p.Lq, dobuf, tid);
            if (tid < kBlk) {
                const int i = min(i0 + tid, p.Lq - 1);
                lsebuf[tid] = p.lse[qrow0 + i];
                dbuf[tid] = p.delta[qrow0 + i];
            }
            __syncthreads();
#pragma unroll
            for (int sub = 0; sub < kBlk / 32; ++sub) {
                const int m0 = 32 * sub;
                // every key of this wave is past the last query of the sub-block
                if (CAUSAL && key0 > i0 + m0 + 31 + off) continue;
                f32x16 s = zero, dp = zero;
#pragma unroll
                for (int ks = 0; ks < kKs; ++ks) {
                    s = mfma(row_frag<D>(qbuf, m0, ks, lane), kf[ks], s);
                    dp = mfma(row_frag<D>(dobuf, m0, ks, lane), vf[ks], dp);
                }
                // P and dS at rows i0 + m0 + acc_row(r), column key
                f32x16 pv, ds;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(lsebuf + m0 + 8 * g4 + 4 * hi);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dbuf + m0 + 8 * g4 + 4 * hi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g4 + e;
                        const int i = i0 + m0 + acc_row(r, hi);
                        bool ok = i < p.Lq && key < p.Lk;
                        if (CAUSAL) ok = ok && key <= i + off;
                        const float pr =
                            ok ? __builtin_amdgcn_exp2f(s[r] * c2 - l4[e] * kLog2e) : 0.0f;
                        pv[r] = pr;
                        ds[r] = pr * (dp[r] - d4[e]);
                    }
                }
                bf16x8 pb[2], db[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x8 e1, e2;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        e1[e] = pv[8 * t + e];
                        e2[e] = ds[8 * t + e];
                    }
                    pb[t] = __builtin_convertvector(e1, bf16x8);
                    db[t] = __builtin_convertvector(e2, bf16x8);
                }
                // dV^T += dO^T P,  dK^T += Q^T dS  (fragment 2 sub + t = rows 16 (2 sub + t) ..)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < kDb; ++i) {
                        dvt[i] = mfma(tr_frag<D>(dobuf, tro[i], 2 * sub + t), pb[t], dvt[i]);
                        dkt[i] = mfma(tr_frag<D>(qbuf, tro[i], 2 * sub + t), db[t], dkt[i]);
                    }
            }
        }
    }
    // lane holds key `key`, columns 32 i + 8 (r >> 2) + 4 hi + (r & 3)
    if (key < p.Lk) {
        uint16_t* dkrow = p.dk + ((size_t)bk * p.Lk + key) * D;
        uint16_t* dvrow = p.dv + ((size_t)bk * p.Lk + key) * D;
#pragma unroll
        for (int i = 0; i < kDb; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 xk = {dkt[i][4 * r4] * p.scale, dkt[i][4 * r4 + 1] * p.scale,
                                  dkt[i][4 * r4 + 2] * p.scale, dkt[i][4 * r4 + 3] * p.scale};
                const f32x4 xv = {dvt[i][4 * r4], dvt[i][4 * r4 + 1], dvt[i][4 * r4 + 2],
                                  dvt[i][4 * r4 + 3]};
                *reinterpret_cast<bf16x4*>(dkrow + 32 * i + 8 * r4 + 4 * hi) =
                    __builtin_convertvector(xk, bf16x4);
                *reinterpret_cast<bf16x4*>(dvrow + 32 * i + 8 * r4 + 4 * hi) =
                    __builtin_convertvector(xv, bf16x4);
            }
    }
}

// ---- dQ ----------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void attn_bwd_dq_kernel(const BwdParams p) {
    constexpr int kKs = D / 16;
    constexpr int kDb = D / 32;
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf[kBlk * D * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf[kBlk * D * 2];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int nqb = (p.Lq + 127) / 128;
    const int bh = blockIdx.x / nqb;  // b * Hq + query head
    const int qb = blockIdx.x % nqb;
    const int b = bh / p.Hq, hq = bh % p.Hq;
    const int bk = b * p.Hkv + hq / p.G;
    const int q0 = qb * 128 + wave * 32;  // this wave's first query
    const int qi = q0 + l32;              // the query of this lane's column
    const int off = p.Lk - p.Lq;
    const float c2 = p.scale_log2;
    const size_t qrow0 = (size_t)bh * p.Lq;

    // Q and dO rows as B operands (rows past Lq read row 0 and are not stored)
    const int qr = qi < p.Lq ? qi : 0;
    bf16x8 qf[kKs], gf[kKs];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
        qf[ks] = __builtin_bit_cast(bf16x8, load16(p.q + (qrow0 + qr) * D + 16 * ks + 8 * hi));
        gf[ks] = __builtin_bit_cast(bf16x8, load16(p.dout + (qrow0 + qr) * D + 16 * ks + 8 * hi));
    }
    const float lse_q = p.lse[qrow0 + qr];
    const float d_q = p.delta[qrow0 + qr];
    f32x16 dqt[kDb];
#pragma unroll
    for (int i = 0; i < kDb; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[i][r] = 0.0f;
    int tro[kDb];
#pragma unroll
    for (int i = 0; i < kDb; ++i) tro[i] = tr_offset<D>(lane, i);

    // keys of the workgroup and of this wave
    int kend = p.Lk, wend = p.Lk;
    if (CAUSAL) {
        kend = min(p.Lk, min(p.Lq, qb * 128 + 128) - 1 + off + 1);
        wend = min(p.Lk, min(p.Lq, q0 + 32) - 1 + off + 1);
    }
    const int nkb = kend > 0 ? (kend + kBlk - 1) / kBlk : 0;
    const uint16_t* kh = p.k + (size_t)bk * p.Lk * D;
    const uint16_t* vh = p.v + (size_t)bk * p.Lk * D;
    const f32x16 zero = {};
    for (int jb = 0; jb < nkb; ++jb) {
        const int j0 = jb * kBlk;
        __syncthreads();
        stage_rows<D>(kh, j0, p.Lk, kbuf, tid);
        stage_rows<D>(vh, j0, p.Lk, vbuf, tid);
        __syncthreads();
        if (q0 >= p.Lq || j0 >= wend) continue;  // no visible key of this block for the wave
        bf16x8 db[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            f32x16 st = zero, dpt = zero;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                st = mfma(row_frag<D>(kbuf, 32 * mb, ks, lane), qf[ks], st);
                dpt = mfma(row_frag<D>(vbuf, 32 * mb, ks, lane), gf[ks], dpt);
            }
            f32x16 ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = j0 + 32 * mb + acc_row(r, hi);
                bool ok = j < p.Lk && qi < p.Lq;
                if (CAUSAL) ok = ok && j <= qi + off;
                const float pr = ok ? __builtin_amdgcn_exp2f(st[r] * c2 - lse_q * kLog2e) : 0.0f;
                ds[r] = pr * (dpt[r] - d_q);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x8 e;
#pragma unroll
                for (int x = 0; x < 8; ++x) e[x] = ds[8 * t + x];
                db[2 * mb + t] = __builtin_convertvector(e, bf16x8);
            }
        }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < kDb; ++i) dqt[i] = mfma(tr_frag<D>(kbuf, tro[i], g), db[g], dqt[i]);
    }
    if (qi < p.Lq) {
        uint16_t* row = p.dq + (qrow0 + qi) * D;
#pragma unroll
        for (int i = 0; i < kDb; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 x = {dqt[i][4 * r4] * p.scale, dqt[i][4 * r4 + 1] * p.scale,
                                 dqt[i][4 * r4 + 2] * p.scale, dqt[i][4 * r4 + 3] * p.scale};
                *reinterpret_cast<bf16x4*>(row + 32 * i + 8 * r4 + 4 * hi) =
                    __builtin_convertvector(x, bf16x4);
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
    BwdParams arg = p;
    const long long rows = (long long)p.B * p.Hq * p.Lq;
    {
        constexpr int kRows = 256 / (D / 8);
        const long long blocks = (rows + kRows - 1) / kRows;
        void* args[] = {&arg, const_cast<long long*>(&rows)};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_delta_kernel<D>),
                                       dim3((unsigned)blocks), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&arg};
    {
        const long long blocks = (long long)p.B * p.Hkv * ((p.Lk + 127) / 128);
        hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, CAUSAL>),
                            dim3((unsigned)blocks), dim3(kBwdThreads), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    const long long blocks = (long long)p.B * p.Hq * ((p.Lq + 127) / 128);
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, CAUSAL>),
                           dim3((unsigned)blocks), dim3(kBwdThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d == 64) return causal ? launch_bwd_t<64, true>(p, stream) : launch_bwd_t<64, false>(p, stream);
    if (d == 128)
        return causal ? launch_bwd_t<128, true>(p, stream) : launch_bwd_t<128, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
