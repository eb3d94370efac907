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
// Both main kernels stream their blocks of 64 rows through two LDS stages,
// filled by direct-to-LDS buffer copies while the other stage is computed on,
// with one barrier per block.
// MFMA v_mfma_f32_32x32x16 (bf16 or fp16 inputs) with fp32 accumulation.
// Operand A is read from LDS (rows with ds_read_b128, transposed with
// ds_read_b64_tr_b16); operand B is a register fragment: the wave's own K/V
// or Q/dO rows, or the 16-bit P / dS fragments, whose row order the
// transposed reads follow.  The causal mask is bottom-right aligned (query i
// sees keys j <= i + Lk - Lq).  Q and K rows have d_qk elements, V, O and dO
// rows d_v (64/64, 128/128 or 192/128); P and dS enter the products in the
// inputs' 16-bit type.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "attn_params.h"

namespace attn {

// D_i of the allocation-free entry point (attn_bwd_noalloc): one float per
// query row, a fixed 16 MiB that each device running the library holds until
// the process ends.  Host code never passes this name to a kernel (in host
// code it is only a stand-in for the symbol): it looks up the device address
// once per device (bwd_scratch_rows) and passes that.
static __device__ __align__(256) float scratch[kBwdScratchRows];

hipError_t bwd_scratch_rows(float** rows) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static float* addr[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float*>(ptr);
    }
    *rows = addr[dev];
    return hipSuccess;
}
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// The 16-bit element type of the tensors and of P and dS in the products,
// with its MFMA form; conversions from fp32 round to nearest even.
template <bool FP16>
struct Elem;
template <>
struct Elem<false> {
    using x8 = bf16x8;
    using x4 = bf16x4;
    static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Elem<true> {
    using x8 = f16x8;
    using x4 = f16x4;
    static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kBwdThreads = 256;  // 4 waves, one per SIMD
constexpr int kBlk = 64;          // rows of a staged Q/dO (or K/V) block
constexpr float kLog2e = 1.4426950408889634f;

// LDS block layout: row r of D bf16, 16-byte chunk c stored at c ^ swz(r).
// Each block is read two ways: by rows (ds_read_b128, 16 lanes reading one
// chunk column of 16 consecutive rows) and transposed (ds_read_b64_tr_b16,
// 32 lanes reading 8 bytes of 4 consecutive rows at 4 adjacent chunks).
// With 64 banks of 4 bytes, the row read is conflict-free when the 16 rows
// land on 16 distinct bank groups, and the transposed read when the 4 rows
// have distinct chunk bits 2-3 (d = 128).  For 128-byte (d = 64) and
// 384-byte (d = 192) rows, rows r and r + 1 start half a bank space apart, so
// the even rows of 16 need distinct swizzles in the low 3 bits (row reads),
// and rows r and r + 2 of a transposed read's 4 must differ in bit 2 (the
// two 16-byte chunks of a row stay together): 4 ((r >> 1) & 1) | ((r >> 2) & 3)
// does both.  The XOR only touches the low 3 bits, so a chunk stays in its
// row (d / 8 is a multiple of 8).
template <int D>
__device__ __forceinline__ int swz(int r) {
    return (D == 128) ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Copy 16 (or 4) bytes per lane from global memory straight into LDS through
// a buffer descriptor: lane l reads at byte voff of the buffer and its data
// lands at lds_dst + 16 l (4 l), one contiguous KiB (256 bytes) per wave.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                              void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                             void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_dst, 4, voff, 0, 0, 0);
}

// Barrier after which every wave's copies issued so far have landed: each
// wave first waits for all of its own outstanding memory operations (the
// compiler's own waits before a barrier do not cover LDS written by a copy).
__device__ __forceinline__ void wait_copies_and_sync() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// A wave-uniform pointer held in VGPRs, moved to SGPRs.
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

// The copies that fill one LDS block of 64 rows of a [L, D] head: 16-byte
// slot s of the block (row s / (D / 8), position s % (D / 8)) holds chunk
// position ^ swz(row) of that row, so the copy that writes slot s reads that
// chunk.  Each of the 4 waves issues kCopies copies of 64 slots; rows past L
// read row L - 1 (their products are masked by the caller).
template <int D>
struct BlockCopies {
    static constexpr int kChunks = D / 8;
    static constexpr int kCopies = kBlk * kChunks / 64 / (kBwdThreads / 64);
    int slot0;  // this lane's slot in the wave's first copy
    int dst;    // this wave's first copy, bytes into the block

    __device__ __forceinline__ void init(int wave, int lane) {
        slot0 = 64 * kCopies * wave + lane;
        dst = __builtin_amdgcn_readfirstlane(1024 * kCopies * wave);
    }
    // rows [row0, row0 + 64) of the head that rs covers into blk; rows past
    // the head's last row lie beyond the descriptor's range and arrive as zeros
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int row0,
                                          unsigned char* blk) const {
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int slot = slot0 + 64 * i;
            const int r = slot / kChunks;
            const uint32_t col = 16u * (uint32_t)((slot % kChunks) ^ swz<D>(r));
            const uint32_t off = (uint32_t)(row0 + r) * (D * 2) + col;
            copy16_to_lds(rs, off, blk + dst + 1024 * i);
        }
    }
};

// A operand from rows of an LDS block: lane l reads row m0 + (l & 31),
// elements 16 ks + 8 (l >> 5) .. +7.
template <int D, typename X8>
__device__ __forceinline__ X8 row_frag(const unsigned char* blk, int m0, int ks, int lane) {
    const int m = m0 + (lane & 31);
    const int ch = 2 * ks + (lane >> 5);
    return *reinterpret_cast<const X8*>(blk + m * (D * 2) + 16 * (ch ^ swz<D>(m)));
}

// Per-lane byte offsets of the transposed reads: with 16-lane group g = l / 16
// and index 4 r + j inside it, the lane reads 8 bytes of row 4 (g / 2) + r
// (+ 8 for the second read) at columns 32 i + 16 (g & 1) + 4 j .. + 3.  The
// swizzle of a row depends on it mod 16, so both reads get their own offset;
// the block offset 16 g' added later keeps the row mod 16.
template <int D>
struct TrOffsets {
    int off[D / 32][2];
    __device__ __forceinline__ void init(int lane) {
        const int tg = lane >> 4, ti = lane & 15, tr = ti >> 2, tj = ti & 3;
        const int cl = 2 * (tg & 1) + (tj >> 1);
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = 4 * (tg >> 1) + tr + 8 * t;
                off[i][t] = row * (D * 2) + 16 * ((4 * i + cl) ^ swz<D>(row)) + 8 * (tj & 1);
            }
    }
};

// A operand = (block rows 16 g .. 16 g + 15)^T, columns 32 i .. 32 i + 31:
// lane l receives column 32 i + (l & 31) at the 8 rows whose values the
// B fragment g (rows 8 (r >> 2) + 4 (l >> 5) + (r & 3) of an accumulator)
// carries in the same order.
template <int D, typename X8>
__device__ __forceinline__ X8 tr_frag(const unsigned char* blk, const TrOffsets<D>& tro, int i,
                                      int g) {
    i16x4 part[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        part[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(blk + tro.off[i][t] + 16 * g * (D * 2)));
    return __builtin_bit_cast(X8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup order.  The hardware deals workgroups round-robin over the 8
// XCDs (workgroup x to XCD x % 8), each with its own L2.  Without a causal
// mask every workgroup does the same work, and the index is remapped so that
// each XCD runs a contiguous range of logical indices: the workgroups of one
// head run on one XCD at about the same time and share that head's blocks in
// its L2.  With the mask, the index is kept, and the caller orders logical
// indices from the most work to the least (longest first).
__device__ __forceinline__ int xcd_contiguous(int x, int n) {
    const int q = n / 8, r = n % 8, k = x % 8;
    return k * q + min(k, r) + x / 8;
}

// Row of accumulator register r for lane half hi: 8 (r >> 2) + 4 hi + (r & 3).
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// ---- D_i = dO_i . O_i --------------------------------------------------------
template <int D, bool FP16>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const BwdParams p, long long rows) {
    using X8 = typename Elem<FP16>::x8;
    constexpr int kLanes = D / 8;  // lanes per row, 16 bytes each
    constexpr int kRows = 256 / kLanes;
    const long long row = (long long)blockIdx.x * kRows + threadIdx.x / kLanes;
    const int c = threadIdx.x % kLanes;
    float acc = 0.0f;
    if (row < rows) {
        const X8 a = __builtin_bit_cast(X8, load16(p.dout + row * D + 8 * c));
        const X8 b = __builtin_bit_cast(X8, load16(p.o + row * D + 8 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
#pragma unroll
    for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kLanes);
    if (row < rows && c == 0) p.delta[row] = acc;
}

// ---- dK, dV ------------------------------------------------------------------
// PART selects the outputs: kBwdBoth computes dK and dV together; kBwdOnlyDV
// and kBwdOnlyDK split them over two launches that each recompute S (the
// second also dP), for head shapes whose dK and dV accumulators, K and V rows
// and pipeline state do not fit one wave's registers together (d_qk = 192).
constexpr int kBwdBoth = 0, kBwdOnlyDV = 1, kBwdOnlyDK = 2;

template <int DQK, int DV, bool FP16, bool CAUSAL, int PART>
__global__ __launch_bounds__(kBwdThreads, 1) void attn_bwd_dkdv_kernel(const BwdParams p) {
    using E = Elem<FP16>;
    using X8 = typename E::x8;
    using X4 = typename E::x4;
    constexpr bool kDoDV = PART != kBwdOnlyDK;
    constexpr bool kDoDK = PART != kBwdOnlyDV;
    constexpr int kKsQ = DQK / 16;                // k-steps of S = Q K^T
    constexpr int kKsV = kDoDK ? DV / 16 : 0;     // k-steps of dP = dO V^T
    constexpr int kDbQ = kDoDK ? DQK / 32 : 0;    // 32-wide blocks of dK
    constexpr int kDbV = kDoDV ? DV / 32 : 0;     // 32-wide blocks of dV
    // two stages of (Q block, dO block, lse, D), filled by direct-to-LDS copies
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf0[kBlk * DQK * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char dobuf0[kBlk * DV * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf1[kBlk * DQK * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char dobuf1[kBlk * DV * 2];
    __shared__ __attribute__((aligned(256))) float lse0[kBlk], dl0[kBlk], lse1[kBlk], dl1[kBlk];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int nkb = (p.Lk + 127) / 128;
    const int nbk = p.B * p.Hkv;
    int bk, kb;  // b * Hkv + kv head, and the key block
    if (CAUSAL) {
        // the first key blocks see the most query rows
        kb = blockIdx.x / nbk;
        bk = blockIdx.x % nbk;
    } else {
        const int x = xcd_contiguous(blockIdx.x, nbk * nkb);
        bk = x / nkb;
        kb = x % nkb;
    }
    const int b = bk / p.Hkv, hk = bk % p.Hkv;
    const int key0 = kb * 128 + wave * 32;  // this wave's first key
    const int key = key0 + l32;             // the key of this lane's accumulator column
    const int off = p.Lk - p.Lq;
    const float c2 = p.scale_log2;

    // the wave's K and V rows as B operands (rows past Lk repeat the last key)
    const int krow = min(key, p.Lk - 1);
    const uint16_t* kh = p.k + (size_t)bk * p.Lk * DQK;
    const uint16_t* vh = p.v + (size_t)bk * p.Lk * DV;
    // (arrays a pass does not use keep one unused element)
    X8 kf[kKsQ], vf[kKsV > 0 ? kKsV : 1];
#pragma unroll
    for (int ks = 0; ks < kKsQ; ++ks)
        kf[ks] = __builtin_bit_cast(X8, load16(kh + (size_t)krow * DQK + 16 * ks + 8 * hi));
#pragma unroll
    for (int ks = 0; ks < kKsV; ++ks)
        vf[ks] = __builtin_bit_cast(X8, load16(vh + (size_t)krow * DV + 16 * ks + 8 * hi));
    f32x16 dkt[kDbQ > 0 ? kDbQ : 1], dvt[kDbV > 0 ? kDbV : 1];
#pragma unroll
    for (int i = 0; i < kDbQ; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkt[i][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < kDbV; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dvt[i][r] = 0.0f;
    TrOffsets<DQK> troq;
    troq.init(lane);
    TrOffsets<DV> trov;
    trov.init(lane);
    BlockCopies<DQK> cpq;
    cpq.init(wave, lane);
    BlockCopies<DV> cpv;
    cpv.init(wave, lane);

    // causal: query blocks before qb0 see none of this workgroup's keys
    int qb0 = 0;
    if (CAUSAL) qb0 = max(0, kb * 128 - off) / kBlk;
    const int nqb = (p.Lq + kBlk - 1) / kBlk;
    const int nq = nqb - qb0;   // query blocks per head, >= 1
    const int nt = p.G * nq;    // steps: (query head of the group, query block)
    const size_t head0 = (size_t)(b * p.Hq + hk * p.G) * p.Lq;

    // stage t: Q and dO rows of its block by every wave, and D by wave 1
    // (one 4-byte copy of 64 rows).  Wave 0 loads the block's lse into a
    // register instead; just before the barrier that publishes the stage it
    // stores the exponent's row term lse * log2(e), or +inf for a row past
    // Lq, whose weights then come out exactly 0 (publish_lse).  Each score
    // then needs one fma before its exponential, and no test for the query
    // tail.
    float lse_pend = 0.0f;
    auto issue = [&](int t, unsigned char* qb, unsigned char* dob, float* db)
                     __attribute__((always_inline)) {
        const int g = t / nq;
        const int i0 = (qb0 + t % nq) * kBlk;
        const size_t r0 = head0 + (size_t)g * p.Lq;
        if (wave == 0) lse_pend = p.lse[r0 + min(i0 + lane, p.Lq - 1)];
        cpq.issue(make_rsrc(uniform(p.q + r0 * DQK), (uint32_t)p.Lq * (DQK * 2)), i0, qb);
        cpv.issue(make_rsrc(uniform(p.dout + r0 * DV), (uint32_t)p.Lq * (DV * 2)), i0, dob);
        if (wave == 1)
            copy4_to_lds(make_rsrc(uniform(p.delta + r0), (uint32_t)p.Lq * 4),
                         (uint32_t)min(i0 + lane, p.Lq - 1) * 4, db);
    };
    auto publish_lse = [&](int t, float* lb) __attribute__((always_inline)) {
        if (wave == 0) {
            const int i0 = (qb0 + t % nq) * kBlk;
            lb[lane] = i0 + lane < p.Lq ? lse_pend * kLog2e : __builtin_inff();
        }
    };
    // One step (64 query rows = sub-blocks 0 and 1 of 32 rows) is a sequence
    // of MFMA units in four quarters, each unit with one LDS operand:
    //   quarter 0  S(0), dP(0)     A = Q / dO rows of sub-block 0 (the k-steps
    //                              of S and dP alternate while both last)
    //   quarter 1  S(1), dP(1)     (sub-block 1), with P(0), dS(0) formed on
    //                              the VALU, spread over its units
    //   quarter 2  dV(0), dK(0)    A = dO^T / Q^T of sub-block 0, B = P(0) /
    //                              dS(0), with P(1), dS(1) formed likewise
    //   quarter 3  dV(1), dK(1)
    // Operands are loaded kAhead units before their MFMA into a register ring
    // and scheduling barriers keep that order, so LDS latency and the
    // softmax arithmetic overlap earlier MFMAs instead of stalling each one.
    constexpr int kAhead = 4;
    constexpr int kSD = kKsQ + kKsV;           // units of an S / dP quarter
    constexpr int kVK = 2 * (kDbV + kDbQ);     // units of a dV / dK quarter
    constexpr int kUnits = 2 * kSD + 2 * kVK;
    // causal: query rows i that see this lane's key: i >= imin
    const int imin = key - off;
    const f32x16 zero = {};
    f32x16 sacc[2], dpacc[2], pv, dsv;
    X8 pb[2][2], db[2][2];
    f32x4 l4[4], d4[4];
    // unit n -> (quarter, position in it)
    auto quarter = [](int n) { return n < kSD ? 0 : n < 2 * kSD ? 1 : n < 2 * kSD + kVK ? 2 : 3; };
    auto qpos = [](int n) {
        return n < kSD ? n : n < 2 * kSD ? n - kSD : n < 2 * kSD + kVK ? n - 2 * kSD
                                                                        : n - 2 * kSD - kVK;
    };
    // S / dP quarter position u: S(k-step) or dP(k-step), alternating while
    // both have k-steps left
    auto sd_unit = [](int u, bool* is_dp, int* ks) {
        constexpr int kBoth = 2 * (kKsQ < kKsV ? kKsQ : kKsV);
        if (u < kBoth) {
            *is_dp = (u & 1) != 0;
            *ks = u >> 1;
        } else {
            *is_dp = kKsV > kKsQ;
            *ks = kBoth / 2 + (u - kBoth);
        }
    };
    // dV / dK quarter position u: row group t2 (16 query rows), then dV(i) and
    // dK(i) alternating while both have blocks left
    auto vk_unit = [](int u, bool* is_dk, int* t2, int* i) {
        constexpr int kPer = kDbV + kDbQ;
        constexpr int kBoth = 2 * (kDbV < kDbQ ? kDbV : kDbQ);
        *t2 = u / kPer;
        const int w = u % kPer;
        if (w < kBoth) {
            *is_dk = (w & 1) != 0;
            *i = w >> 1;
        } else {
            *is_dk = kDbQ > kDbV;
            *i = kBoth / 2 + (w - kBoth);
        }
    };
    auto load = [&](int n, const unsigned char* qbuf, const unsigned char* dobuf)
                    __attribute__((always_inline)) {
        const int qt = quarter(n), u = qpos(n);
        const int sub = qt & 1;
        if (qt < 2) {  // S / dP unit of sub-block sub
            bool is_dp;
            int ks;
            sd_unit(u, &is_dp, &ks);
            return is_dp ? row_frag<DV, X8>(dobuf, 32 * sub, ks, lane)
                         : row_frag<DQK, X8>(qbuf, 32 * sub, ks, lane);
        }
        bool is_dk;
        int t2, i;
        vk_unit(u, &is_dk, &t2, &i);
        return is_dk ? tr_frag<DQK, X8>(qbuf, troq, i, 2 * sub + t2)
                     : tr_frag<DV, X8>(dobuf, trov, i, 2 * sub + t2);
    };
    auto mfma_unit = [&](int n, X8 a) __attribute__((always_inline)) {
        const int qt = quarter(n), u = qpos(n);
        const int sub = qt & 1;
        if (qt < 2) {
            bool is_dp;
            int ks;
            sd_unit(u, &is_dp, &ks);
            if (is_dp)
                dpacc[sub] = E::mfma(a, vf[ks], ks == 0 ? zero : dpacc[sub]);
            else
                sacc[sub] = E::mfma(a, kf[ks], ks == 0 ? zero : sacc[sub]);
        } else {
            bool is_dk;
            int t2, i;
            vk_unit(u, &is_dk, &t2, &i);
            if (is_dk)
                dkt[i] = E::mfma(a, db[sub][t2], dkt[i]);
            else
                dvt[i] = E::mfma(a, pb[sub][t2], dvt[i]);
        }
    };
    // P and dS of sub-block sub at accumulator element r (row i0 + 32 sub +
    // acc_row(r), column key); after elements 7 and 15, their 16-bit fragments
    // (P for the dV products, dS for the dK products).  Rows past Lq carry an
    // infinite row term (weight 0).  A key past Lk only ever meets its own
    // accumulator column, which is never stored, so it needs no mask.  Under
    // the causal mask, the steps whose rows do not all see the wave's last
    // key (diag, wave-uniform) zero the weights of the rows before each
    // lane's key, 8 at a time, with selects: a row that sees no key at all
    // has lse = -inf and an infinite weight there.
    auto softmax_elem = [&](int sub, int r, int i0, bool diag) __attribute__((always_inline)) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[sub][r], c2, -l4[r >> 2][r & 3]));
        pv[r] = pr;
        if constexpr (kDoDK) dsv[r] = pr * (dpacc[sub][r] - d4[r >> 2][r & 3]);
        if ((r & 7) == 7) {
            const int t2 = r >> 3;
            if (CAUSAL && diag) {
                // element r is row i0 + 32 sub + acc_row(r, hi)
                const int lo = imin - i0 - 32 * sub - 4 * hi;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r2 = 8 * t2 + e;
                    const bool ok = acc_row(r2, 0) >= lo;
                    pv[r2] = ok ? pv[r2] : 0.0f;
                    if constexpr (kDoDK) dsv[r2] = ok ? dsv[r2] : 0.0f;
                }
            }
            f32x8 e1, e2;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                e1[e] = pv[8 * t2 + e];
                if constexpr (kDoDK) e2[e] = dsv[8 * t2 + e];
            }
            if constexpr (kDoDV) pb[sub][t2] = __builtin_convertvector(e1, X8);
            if constexpr (kDoDK) db[sub][t2] = __builtin_convertvector(e2, X8);
        }
    };
    auto load_rowstats = [&](int sub, const float* lsebuf, const float* dbuf)
                             __attribute__((always_inline)) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            l4[g4] = *reinterpret_cast<const f32x4*>(lsebuf + 32 * sub + 8 * g4 + 4 * hi);
            if constexpr (kDoDK)
                d4[g4] = *reinterpret_cast<const f32x4*>(dbuf + 32 * sub + 8 * g4 + 4 * hi);
        }
    };
    auto compute = [&](int t, const unsigned char* qbuf, const unsigned char* dobuf,
                       const float* lsebuf, const float* dbuf) __attribute__((always_inline)) {
        const int i0 = (qb0 + t % nq) * kBlk;
        const bool diag = CAUSAL && i0 < key0 + 31 - off;
        X8 ring[kAhead];
#pragma unroll
        for (int n = 0; n < kAhead; ++n) ring[n] = load(n, qbuf, dobuf);
        auto unit = [&](int n) __attribute__((always_inline)) {
            const X8 a = ring[n % kAhead];
            if (n + kAhead < kUnits) ring[n % kAhead] = load(n + kAhead, qbuf, dobuf);
            mfma_unit(n, a);
            // the 16 softmax elements of the previous sub-block, spread over
            // the units of quarters 1 and 2 in order
            const int qt = quarter(n), u = qpos(n);
            if (qt == 1 || qt == 2) {
                const int len = qt == 1 ? kSD : kVK;
#pragma unroll
                for (int r = (16 * u + len - 1) / len; r < (16 * (u + 1) + len - 1) / len; ++r)
                    softmax_elem(qt - 1, r, i0, diag);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // four loops, one per quarter, each short enough to be unrolled in full
#pragma unroll
        for (int n = 0; n < kSD; ++n) unit(n);
        load_rowstats(0, lsebuf, dbuf);
#pragma unroll
        for (int n = kSD; n < 2 * kSD; ++n) unit(n);
        load_rowstats(1, lsebuf, dbuf);
#pragma unroll
        for (int n = 2 * kSD; n < 2 * kSD + kVK; ++n) unit(n);
#pragma unroll
        for (int n = 2 * kSD + kVK; n < kUnits; ++n) unit(n);
    };
    // One barrier per step: every wave's copies of stage t have landed (each
    // wave waits for its own before the barrier), its row terms are stored,
    // and every wave is done with stage t - 1, whose buffers the copies of
    // stage t + 1 then refill.
    issue(0, qbuf0, dobuf0, dl0);
    for (int t = 0; t < nt; t += 2) {
        publish_lse(t, lse0);
        wait_copies_and_sync();
        if (t + 1 < nt) issue(t + 1, qbuf1, dobuf1, dl1);
        compute(t, qbuf0, dobuf0, lse0, dl0);
        if (t + 1 < nt) {
            publish_lse(t + 1, lse1);
            wait_copies_and_sync();
            if (t + 2 < nt) issue(t + 2, qbuf0, dobuf0, dl0);
            compute(t + 1, qbuf1, dobuf1, lse1, dl1);
        }
    }
    // lane holds key `key`, columns 32 i + 8 (r >> 2) + 4 hi + (r & 3)
    if (key < p.Lk) {
        uint16_t* dkrow = p.dk + ((size_t)bk * p.Lk + key) * DQK;
        uint16_t* dvrow = p.dv + ((size_t)bk * p.Lk + key) * DV;
#pragma unroll
        for (int i = 0; i < kDbQ; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 xk = {dkt[i][4 * r4] * p.scale, dkt[i][4 * r4 + 1] * p.scale,
                                  dkt[i][4 * r4 + 2] * p.scale, dkt[i][4 * r4 + 3] * p.scale};
                *reinterpret_cast<X4*>(dkrow + 32 * i + 8 * r4 + 4 * hi) =
                    __builtin_convertvector(xk, X4);
            }
#pragma unroll
        for (int i = 0; i < kDbV; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 xv = {dvt[i][4 * r4], dvt[i][4 * r4 + 1], dvt[i][4 * r4 + 2],
                                  dvt[i][4 * r4 + 3]};
                *reinterpret_cast<X4*>(dvrow + 32 * i + 8 * r4 + 4 * hi) =
                    __builtin_convertvector(xv, X4);
            }
    }
}

// ---- dQ ----------------------------------------------------------------------
// Two waves per SIMD where the registers allow (d_qk <= 128), one otherwise.
template <int DQK, int DV, bool FP16, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, (DQK <= 128 ? 2 : 1)) void attn_bwd_dq_kernel(
    const BwdParams p) {
    using E = Elem<FP16>;
    using X8 = typename E::x8;
    using X4 = typename E::x4;
    constexpr int kKsQ = DQK / 16;
    constexpr int kKsV = DV / 16;
    constexpr int kDbQ = DQK / 32;
    // two stages of (K block, V block), filled by direct-to-LDS copies
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[kBlk * DQK * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf0[kBlk * DV * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf1[kBlk * DQK * 2];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf1[kBlk * DV * 2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int nqb = (p.Lq + 127) / 128;
    const int nbh = p.B * p.Hq;
    int bh, qb;  // b * Hq + query head, and the query block
    if (CAUSAL) {
        // the last query blocks see the most keys
        qb = nqb - 1 - (int)blockIdx.x / nbh;
        bh = blockIdx.x % nbh;
    } else {
        const int x = xcd_contiguous(blockIdx.x, nbh * nqb);
        bh = x / nqb;
        qb = x % nqb;
    }
    const int b = bh / p.Hq, hq = bh % p.Hq;
    const int bk = b * p.Hkv + hq / p.G;
    const int q0 = qb * 128 + wave * 32;  // this wave's first query
    const int qi = q0 + l32;              // the query of this lane's column
    const int off = p.Lk - p.Lq;
    const float c2 = p.scale_log2;
    const size_t qrow0 = (size_t)bh * p.Lq;

    // Q and dO rows as B operands (rows past Lq read row 0 and are not stored)
    const int qr = qi < p.Lq ? qi : 0;
    X8 qf[kKsQ], gf[kKsV];
#pragma unroll
    for (int ks = 0; ks < kKsQ; ++ks)
        qf[ks] = __builtin_bit_cast(X8, load16(p.q + (qrow0 + qr) * DQK + 16 * ks + 8 * hi));
#pragma unroll
    for (int ks = 0; ks < kKsV; ++ks)
        gf[ks] = __builtin_bit_cast(X8, load16(p.dout + (qrow0 + qr) * DV + 16 * ks + 8 * hi));
    const float lse2_q = p.lse[qrow0 + qr] * kLog2e;  // the exponent's row term
    const float d_q = p.delta[qrow0 + qr];
    // the last key this lane's query sees (a lane past Lq reads row 0 and is
    // never stored)
    const int jlast = CAUSAL ? min(p.Lk - 1, qi + off) : p.Lk - 1;
    f32x16 dqt[kDbQ];
#pragma unroll
    for (int i = 0; i < kDbQ; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[i][r] = 0.0f;
    TrOffsets<DQK> tro;
    tro.init(lane);
    BlockCopies<DQK> cpk;
    cpk.init(wave, lane);
    BlockCopies<DV> cpv;
    cpv.init(wave, lane);

    // keys of the workgroup and of this wave
    int kend = p.Lk, wend = p.Lk;
    if (CAUSAL) {
        kend = min(p.Lk, min(p.Lq, qb * 128 + 128) - 1 + off + 1);
        wend = min(p.Lk, min(p.Lq, q0 + 32) - 1 + off + 1);
    }
    const int nkb = kend > 0 ? (kend + kBlk - 1) / kBlk : 0;
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(uniform(p.k + (size_t)bk * p.Lk * DQK), (uint32_t)p.Lk * (DQK * 2));
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(uniform(p.v + (size_t)bk * p.Lk * DV), (uint32_t)p.Lk * (DV * 2));
    auto issue = [&](int jb, unsigned char* kbuf, unsigned char* vbuf)
                     __attribute__((always_inline)) {
        cpk.issue(krs, jb * kBlk, kbuf);
        cpv.issue(vrs, jb * kBlk, vbuf);
    };
    const f32x16 zero = {};
    // A block is a list of MFMA units, each with one LDS operand: the S / dP
    // units of key rows 0..31 (the k-steps of S and dP alternate while both
    // last), those of rows 32..63, then the dQ units (row group g, output
    // block i).  Operands are loaded kAhead units before their MFMA into a
    // register ring, and scheduling barriers keep that order, so the loads of
    // the next units are in flight while the softmax of a row group runs and
    // while earlier MFMAs execute, instead of each MFMA waiting for its own.
    constexpr int kAheadQ = 2;
    constexpr int kSDq = kKsQ + kKsV;
    constexpr int kUnitsQ = 2 * kSDq + 4 * kDbQ;
    auto sd_unit = [](int u, bool* is_dp, int* ks) {
        constexpr int kBoth = 2 * (kKsQ < kKsV ? kKsQ : kKsV);
        if (u < kBoth) {
            *is_dp = (u & 1) != 0;
            *ks = u >> 1;
        } else {
            *is_dp = kKsV > kKsQ;
            *ks = kBoth / 2 + (u - kBoth);
        }
    };
    auto compute = [&](int jb, const unsigned char* kbuf, const unsigned char* vbuf)
                       __attribute__((always_inline)) {
        const int j0 = jb * kBlk;
        if (q0 >= p.Lq || j0 >= wend) return;  // no visible key of this block for the wave
        X8 db[4];
        f32x16 st, dpt;
        auto load = [&](int n) __attribute__((always_inline)) {
            if (n < 2 * kSDq) {
                const int mb = n / kSDq;
                bool is_dp;
                int ks;
                sd_unit(n % kSDq, &is_dp, &ks);
                return is_dp ? row_frag<DV, X8>(vbuf, 32 * mb, ks, lane)
                             : row_frag<DQK, X8>(kbuf, 32 * mb, ks, lane);
            }
            const int g = (n - 2 * kSDq) / kDbQ, i = (n - 2 * kSDq) % kDbQ;
            return tr_frag<DQK, X8>(kbuf, tro, i, g);
        };
        auto mfma_unit = [&](int n, X8 a) __attribute__((always_inline)) {
            if (n < 2 * kSDq) {
                bool is_dp;
                int ks;
                sd_unit(n % kSDq, &is_dp, &ks);
                if (is_dp)
                    dpt = E::mfma(a, gf[ks], ks == 0 ? zero : dpt);
                else
                    st = E::mfma(a, qf[ks], ks == 0 ? zero : st);
            } else {
                const int g = (n - 2 * kSDq) / kDbQ, i = (n - 2 * kSDq) % kDbQ;
                dqt[i] = E::mfma(a, db[g], dqt[i]);
            }
        };
        // dS of key rows 32 mb .. 32 mb + 31 from the finished S and dP
        auto softmax_m = [&](int mb, auto maskc) __attribute__((always_inline)) {
            constexpr bool kMask = decltype(maskc)::value;
            // element r holds key j0 + 32 mb + acc_row(r, hi), visible iff
            // acc_row(r, 0) <= lim: one compare with a constant
            const int lim = jlast - j0 - 32 * mb - 4 * hi;
            f32x16 ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -lse2_q));
                ds[r] = (!kMask || acc_row(r, 0) <= lim ? pr : 0.0f) * (dpt[r] - d_q);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x8 e;
#pragma unroll
                for (int x = 0; x < 8; ++x) e[x] = ds[8 * t + x];
                db[2 * mb + t] = __builtin_convertvector(e, X8);
            }
        };
        // blocks whose keys all exist and, under the causal mask, all lie at
        // or before every row's last visible key need no test (wave-uniform)
        const bool full = j0 + kBlk <= p.Lk && (!CAUSAL || j0 + kBlk - 1 <= q0 + off) &&
                          q0 + 32 <= p.Lq;
        auto softmax = [&](int mb) __attribute__((always_inline)) {
            if (full)
                softmax_m(mb, std::false_type{});
            else
                softmax_m(mb, std::true_type{});
        };
        X8 ring[kAheadQ];
#pragma unroll
        for (int n = 0; n < kAheadQ; ++n) ring[n] = load(n);
        auto unit = [&](int n) __attribute__((always_inline)) {
            const X8 a = ring[n % kAheadQ];
            if (n + kAheadQ < kUnitsQ) ring[n % kAheadQ] = load(n + kAheadQ);
            mfma_unit(n, a);
            __builtin_amdgcn_sched_barrier(0);
        };
        // three loops, each short enough to be unrolled in full
#pragma unroll
        for (int n = 0; n < kSDq; ++n) unit(n);
        softmax(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = kSDq; n < 2 * kSDq; ++n) unit(n);
        softmax(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 2 * kSDq; n < kUnitsQ; ++n) unit(n);
    };
    // one barrier per block, as in the dK/dV kernel
    if (nkb > 0) issue(0, kbuf0, vbuf0);
    for (int jb = 0; jb < nkb; jb += 2) {
        wait_copies_and_sync();
        if (jb + 1 < nkb) issue(jb + 1, kbuf1, vbuf1);
        compute(jb, kbuf0, vbuf0);
        if (jb + 1 < nkb) {
            wait_copies_and_sync();
            if (jb + 2 < nkb) issue(jb + 2, kbuf0, vbuf0);
            compute(jb + 1, kbuf1, vbuf1);
        }
    }
    if (qi < p.Lq) {
        uint16_t* row = p.dq + (qrow0 + qi) * DQK;
#pragma unroll
        for (int i = 0; i < kDbQ; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 x = {dqt[i][4 * r4] * p.scale, dqt[i][4 * r4 + 1] * p.scale,
                                 dqt[i][4 * r4 + 2] * p.scale, dqt[i][4 * r4 + 3] * p.scale};
                *reinterpret_cast<X4*>(row + 32 * i + 8 * r4 + 4 * hi) =
                    __builtin_convertvector(x, X4);
            }
    }
}

template <int DQK, int DV, bool FP16, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
    BwdParams arg = p;
    const long long rows = (long long)p.B * p.Hq * p.Lq;
    {
        constexpr int kRows = 256 / (DV / 8);
        const long long blocks = (rows + kRows - 1) / kRows;
        void* args[] = {&arg, const_cast<long long*>(&rows)};
        hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_delta_kernel<DV, FP16>),
                            dim3((unsigned)blocks), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&arg};
    {
        const long long blocks = (long long)p.B * p.Hkv * ((p.Lk + 127) / 128);
        auto launch = [&](const void* kernel) {
            return hipLaunchKernel(kernel, dim3((unsigned)blocks), dim3(kBwdThreads), args, 0,
                                   stream);
        };
        hipError_t e;
        if constexpr (DQK > 128) {
            // dV, then dK, in launches of their own (see PART)
            e = launch(reinterpret_cast<const void*>(
                &attn_bwd_dkdv_kernel<DQK, DV, FP16, CAUSAL, kBwdOnlyDV>));
            if (e != hipSuccess) return e;
            e = launch(reinterpret_cast<const void*>(
                &attn_bwd_dkdv_kernel<DQK, DV, FP16, CAUSAL, kBwdOnlyDK>));
        } else {
            e = launch(reinterpret_cast<const void*>(
                &attn_bwd_dkdv_kernel<DQK, DV, FP16, CAUSAL, kBwdBoth>));
        }
        if (e != hipSuccess) return e;
    }
    const long long blocks = (long long)p.B * p.Hq * ((p.Lq + 127) / 128);
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<DQK, DV, FP16, CAUSAL>),
                           dim3((unsigned)blocks), dim3(kBwdThreads), args, 0, stream);
}

template <int DQK, int DV>
hipError_t launch_bwd_dims(const BwdParams& p, bool causal, bool fp16, hipStream_t stream) {
    if (fp16)
        return causal ? launch_bwd_t<DQK, DV, true, true>(p, stream)
                      : launch_bwd_t<DQK, DV, true, false>(p, stream);
    return causal ? launch_bwd_t<DQK, DV, false, true>(p, stream)
                  : launch_bwd_t<DQK, DV, false, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int dqk, int dv, bool causal, bool fp16,
                      hipStream_t stream) {
    if (dqk == 64 && dv == 64) return launch_bwd_dims<64, 64>(p, causal, fp16, stream);
    if (dqk == 128 && dv == 128) return launch_bwd_dims<128, 128>(p, causal, fp16, stream);
    if (dqk == 192 && dv == 128) return launch_bwd_dims<192, 128>(p, causal, fp16, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
