// attn_merge_kernel.hip -- merge of per-split attention states (gfx950).
//
// A split of the keys leaves, per query row, the split's normalised output
// O_g and its log-sum-exp lse_g.  With the reference at lse_g that split's
// softmax denominator is exactly 1, so its state is (m, l, u) = (lse_g, 1,
// O_g), and the two-block merge rule of "Infra: Flash Attention" (section on
// computing softmax in segments: common reference m = max, each state scaled
// by e^{m_g - m}, denominators and numerators added) applied to all splits at
// once gives
//     m = max_g lse_g,   w_g = e^{lse_g - m},   l = sum_g w_g,
//     O = (sum_g w_g O_g) / l,   lse = m + ln l.
// A split that holds no visible key has lse_g = -inf and weight 0; a row no
// split reaches gets O = 0 and lse = -inf.  Splitting the keys and merging
// the states is the decode path of the same page (section on prefill versus
// decode).
//
// The merge reads every split's output once and writes the result once, so
// it is bound by HBM bandwidth: each lane moves 16 contiguous bytes per split
// and the lanes of a wave cover whole rows, which keeps every access
// coalesced.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// DV / 4 lanes per row, each holding 4 consecutive output columns.
template <int DV>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, uint16_t* __restrict__ o,
    float* __restrict__ lse, int n_split, long long rows) {
    constexpr int kLanesPerRow = DV / 4;
    constexpr int kRowsPerBlock = kMergeThreads / kLanesPerRow;
    const int t = threadIdx.x;
    const long long row = (long long)blockIdx.x * kRowsPerBlock + t / kLanesPerRow;
    const int c = 4 * (t % kLanesPerRow);
    if (row >= rows) return;

    float m = -__builtin_inff();
    for (int g = 0; g < n_split; ++g) m = fmaxf(m, lse_part[(size_t)g * rows + row]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float l = 0.0f;
    if (m != -__builtin_inff()) {
        for (int g = 0; g < n_split; ++g) {
            const float lg = lse_part[(size_t)g * rows + row];
            // e^{lg - m}, exactly 0 for a split without keys
            const float w = __builtin_amdgcn_exp2f((lg - m) * kLog2e);
            const f32x4 x = *reinterpret_cast<const f32x4*>(o_part + ((size_t)g * rows + row) * DV + c);
            acc += w * x;
            l += w;
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const f32x4 y = acc * inv;
    *reinterpret_cast<bf16x4*>(o + (size_t)row * DV + c) = __builtin_convertvector(y, bf16x4);
    if (c == 0) lse[row] = l > 0.0f ? m + logf(l) : -__builtin_inff();
}

template <int DV>
hipError_t launch_merge_dv(const float* o_part, const float* lse_part, uint16_t* o, float* lse,
                           int n_split, long long rows, hipStream_t stream) {
    constexpr int kRowsPerBlock = kMergeThreads / (DV / 4);
    const long long blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    void* args[] = {&o_part, &lse_part, &o, &lse, &n_split, &rows};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_merge_kernel<DV>),
                           dim3((unsigned)blocks), dim3(kMergeThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_merge(const float* o_part, const float* lse_part, uint16_t* o, float* lse,
                        int n_split, long long rows, int dv, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (dv == 64) return launch_merge_dv<64>(o_part, lse_part, o, lse, n_split, rows, stream);
    if (dv == 128) return launch_merge_dv<128>(o_part, lse_part, o, lse, n_split, rows, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
