/*
 * attn_fwd.h -- C ABI of the fused exact-attention forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * What it computes (per batch b and query head h):
 *     O   = softmax(scale * Q K^T) V                 softmax along the keys
 *     lse = log sum_j exp(scale * q_i . k_j)         natural log, per query row
 * with the key/value head h / (Hq / Hkv) serving query head h (grouped-query
 * attention), and, when causal != 0, the mask aligned to the bottom-right
 * corner: query i attends keys j <= i + Lk - Lq.
 * Definitions: "Infra: Flash Attention" (pufanyi.com), opening section and
 * Algorithm 1 (O and L = m + log l); "Flash Attention 4: 在 Blackwell 上把
 * Softmax 接进 Tensor Core 流水线" (fangpin gpu-hpc-book ch. 13), sections on
 * online softmax with conditional rescaling and on causal attention and GQA.
 * The score matrix is never written to memory: keys are visited block by
 * block with an online softmax whose base-2 reference moves only when the
 * block maximum exceeds it by more than 8 (log2 units).
 *
 * Tensor layouts (all contiguous, row-major, device memory):
 *     q    [B, Hq,  Lq, d_qk]   bfloat16
 *     k    [B, Hkv, Lk, d_qk]   bfloat16
 *     v    [B, Hkv, Lk, d_v ]   bfloat16
 *     o    [B, Hq,  Lq, d_v ]   bfloat16 (output, rounded to nearest even)
 *     lse  [B, Hq,  Lq]         float32  (output)
 * A query row with no visible key (causal with Lq > Lk) gets O = 0 and
 * lse = -inf.
 *
 * Ownership: every pointer is a device pointer owned by the caller; the
 * library allocates no memory.  o and lse must not overlap the inputs or each
 * other.  q, k, v and o must be 16-byte aligned, lse 4-byte aligned.
 *
 * Asynchrony: the call enqueues one kernel on `stream` (a hipStream_t; NULL
 * means the null stream) and returns.  The return value reports argument
 * errors (checked before any HIP call) and launch errors; faults during
 * execution surface at the caller's next synchronisation.  The library keeps
 * no mutable state between calls except a per-device cache of the
 * architecture check, and may be called from several host threads.
 *
 * Logging: with the environment variable ATTN_LOG set (to anything but "0"),
 * every launch prints its kernel, instantiation and grid to stderr.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_PTR = 1,              /* a required pointer is NULL */
    ATTN_ERR_BAD_SHAPE = 2,             /* B, Hq, Hkv, Lq or Lk < 1 */
    ATTN_ERR_GQA_RATIO = 3,             /* Hq is not a multiple of Hkv */
    ATTN_ERR_UNSUPPORTED_HEAD_DIM = 4,  /* (d_qk, d_v) not one of (64,64), (128,128), (192,128) */
    ATTN_ERR_BAD_SCALE = 5,             /* scale not finite or not > 0 */
    ATTN_ERR_MISALIGNED = 6,            /* q/k/v/o not 16-byte or lse not 4-byte aligned */
    ATTN_ERR_TOO_LARGE = 7,             /* a row or tile count does not fit the index types */
    ATTN_ERR_NO_DEVICE = 8,             /* no HIP device is visible */
    ATTN_ERR_UNSUPPORTED_ARCH = 9,      /* the current device is not gfx950 */
    ATTN_ERR_HIP = 10,                  /* the HIP runtime reported an error at launch */
    ATTN_ERR_BAD_ARGUMENT = 11,         /* a debug-only argument, a split count, a
                                           merge row count or a dtype is out of range */
    ATTN_ERR_BAD_STRIDE = 12,           /* a stride is negative, not a multiple of 8
                                           elements, or a row stride is below the
                                           head dim */
    ATTN_ERR_SCRATCH = 13               /* attn_bwd_noalloc: B * Hq * Lq exceeds
                                           ATTN_BWD_NOALLOC_MAX_ROWS */
};

/* Element types of attn_fwd_ex. */
enum attn_dtype {
    ATTN_DTYPE_BF16 = 0,
    ATTN_DTYPE_FP16 = 1
};

/* Element strides of a [B, H, L, d] tensor whose head dim is contiguous:
 * element (b, h, i, c) sits at b * batch + h * head + i * row + c. */
typedef struct attn_strides {
    long long batch;
    long long head;
    long long row;
} attn_strides;

/*
 * attn_fwd -- fused attention forward.
 *   q, k, v     inputs as laid out above
 *   o, lse      outputs as laid out above
 *   B, Hq, Hkv  batch, query heads, key/value heads (Hq % Hkv == 0)
 *   Lq, Lk      query and key sequence lengths (any values >= 1)
 *   d_qk, d_v   head dims: (64,64), (128,128) or (192,128)
 *   causal      0: full attention; nonzero: bottom-right causal mask
 *   scale       softmax scale applied to q.k (callers usually pass
 *               1/sqrt(d_qk)); must be finite and > 0
 *   stream      hipStream_t to enqueue on (NULL: the null stream)
 * Returns ATTN_OK or one of the codes above.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
             int causal, float scale, void* stream);

/*
 * attn_fwd_dbg -- attn_fwd with the conditional-rescale threshold exposed and
 * an event counter, for checking the rescale rule of "Flash Attention 4 ..."
 * ch. 13 (section on online softmax and conditional rescaling).
 *   rescale_threshold  log2-units threshold tau >= 0 (finite): the reference
 *                      moves when (ref - cand) * scale * log2(e) < -tau.
 *                      0 rescales at every increase of the running max; the
 *                      production entry point uses 8.
 *   exp_mode           how the exponentials 2^x are evaluated: 0 = the
 *                      hardware v_exp_f32 for every element (the only mode
 *                      built; the FA4 review's exp-emulation section describes
 *                      a partial polynomial, which on gfx950 would cost more
 *                      VALU time than it saves).  Any other value returns
 *                      ATTN_ERR_BAD_ARGUMENT.
 *   rescale_count      device pointer to one unsigned 64-bit counter, or NULL.
 *                      When given, the kernel atomically adds the number of
 *                      (query row, key block) pairs, after the row's first
 *                      visible block, at which the row's reference moved.  The
 *                      caller zeroes it beforehand.
 * Other arguments and returns as attn_fwd; ATTN_ERR_BAD_ARGUMENT for a bad
 * threshold or exp_mode.
 */
int attn_fwd_dbg(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
                 int causal, float scale, void* stream,
                 float rescale_threshold, int exp_mode, unsigned long long* rescale_count);

/*
 * attn_fwd_ex -- attn_fwd for any element strides and for fp16 as well as
 * bf16 elements.  "Flash Attention 4: 在 Blackwell 上把 Softmax 接进 Tensor
 * Core 流水线" (fangpin gpu-hpc-book ch. 13), in the section with its usage
 * example, calls the kernel on fp16 Q, K, V and O laid out [B, S, H, D]; with
 * strides that layout is (batch, head, row) = (S*H*d, d, H*d), and the
 * contiguous [B, H, L, d] layout of attn_fwd is (H*L*d, L*d, d).  Views into
 * a packed QKV tensor work the same way.
 *   q_strides, k_strides, v_strides, o_strides
 *               element strides of the four tensors (the head dim is
 *               contiguous).  Each stride is >= 0 and a multiple of 8
 *               elements (so rows start 16-byte aligned); row strides are at
 *               least the head dim.  One K or V head ((Lk - 1) * row + d
 *               elements) and 32 rows of Q must span less than 2^31 bytes.
 *               o must not overlap q, k, v or lse.
 *   dtype       ATTN_DTYPE_BF16 or ATTN_DTYPE_FP16: the element type of q, k,
 *               v and o.  The weights P enter the PV product in the same type
 *               (fp16 has 3 more mantissa bits than bf16; P <= 2^8 fits its
 *               range); accumulation is fp32 either way.
 *   lse         float32 [B, Hq, Lq], contiguous, as in attn_fwd.
 * Other arguments, ownership, asynchrony and errors as attn_fwd;
 * ATTN_ERR_BAD_STRIDE for a stride outside the rules above,
 * ATTN_ERR_BAD_ARGUMENT for another dtype.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
                attn_strides q_strides, attn_strides k_strides, attn_strides v_strides,
                attn_strides o_strides, int dtype, int causal, float scale, void* stream);

/*
 * Split-key path.  "Infra: Flash Attention" (section on prefill versus
 * decode) notes that the merge rule of its section on computing softmax in
 * segments does not fix the order of the keys: the key sequence may be cut
 * into segments that are computed separately and whose states are merged
 * afterwards.  That gives work to many CUs when there are few query rows
 * (decode), and it is the combine step when different devices hold
 * different key ranges.
 *
 * attn_split_keys -- keys per split for Lk keys in n_split splits: the key
 * blocks of 64 are dealt out in contiguous runs, so split s covers keys
 * [s * W, min(Lk, (s + 1) * W)) with W = 64 * ceil(ceil(Lk / 64) / n_split).
 * Trailing splits may be empty.  Returns W, or -ATTN_ERR_BAD_SHAPE /
 * -ATTN_ERR_BAD_ARGUMENT for Lk < 1 or n_split outside [1, 4096].
 */
int attn_split_keys(int Lk, int n_split);

/*
 * attn_fwd_split -- the forward pass restricted to each key split.
 *   o_part    float32 [n_split, B, Hq, Lq, d_v]: split s's softmax-normalised
 *             output over the visible keys of split s (16-byte aligned)
 *   lse_part  float32 [n_split, B, Hq, Lq]: split s's log-sum-exp (4-byte
 *             aligned); a row with no visible key in split s gets O = 0 and
 *             lse = -inf
 *   n_split   1 .. 4096
 * Other arguments, layouts, ownership, asynchrony and errors as attn_fwd (the
 * causal mask and GQA mapping are the same; the rescale threshold is 8).
 * attn_merge turns the per-split states into attn_fwd's o and lse.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
                   int causal, float scale, int n_split, void* stream);

/*
 * attn_merge -- merge n_split per-split states row by row:
 *     m = max_g lse_g,  w_g = exp(lse_g - m),  l = sum_g w_g,
 *     O = sum_g w_g O_g / l  (rounded to bfloat16),  lse = m + ln l,
 * the two-block merge rule of "Infra: Flash Attention" applied to states
 * (m, l, u) = (lse_g, 1, O_g).  Rows that no split reaches get O = 0 and
 * lse = -inf.
 *   o_part    float32 [n_split, rows, d_v] (16-byte aligned)
 *   lse_part  float32 [n_split, rows]
 *   o         bfloat16 [rows, d_v] output (16-byte aligned); lse float32 [rows]
 *   rows      number of query rows, >= 0 (B * Hq * Lq for attn_fwd_split's
 *             output); d_v 64 or 128
 * One kernel on `stream`; errors as attn_fwd (ATTN_ERR_BAD_ARGUMENT for
 * rows < 0 or n_split outside [1, 4096], ATTN_ERR_UNSUPPORTED_HEAD_DIM for
 * another d_v).
 */
int attn_merge(const float* o_part, const float* lse_part, void* o, float* lse,
               int n_split, long long rows, int d_v, void* stream);

/*
 * attn_bwd -- gradients of the attention forward pass ("Infra: Flash
 * Attention", sections on why the backward pass recomputes and on computing
 * the gradients block by block): for a loss L with dL/dO = dout,
 *     P = exp(scale * Q K^T - lse)   (recomputed from the forward's lse),
 *     dV = P^T dout,  dP = dout V^T,  D_i = dout_i . o_i,
 *     dS = P (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,
 * with the same causal mask and grouped-query head mapping as attn_fwd (a
 * K/V head's dK and dV sum over the query heads it serves).
 *   q, k, v, o, lse  as attn_fwd's inputs and outputs (contiguous [B, H, L, d]
 *                    bf16; lse float32 [B, Hq, Lq]) from the forward call
 *   dout             bfloat16 [B, Hq, Lq, d_v]
 *   dq               bfloat16 [B, Hq, Lq, d_qk] (output)
 *   dk, dv           bfloat16 [B, Hkv, Lk, d_qk] and [B, Hkv, Lk, d_v] (output)
 *   delta            float32 [B, Hq, Lq] (output, and the kernels' scratch:
 *                    D_i = dout_i . o_i)
 *   (d_qk, d_v)      (64,64), (128,128) or (192,128)
 *                    (ATTN_ERR_UNSUPPORTED_HEAD_DIM otherwise)
 * All pointers are caller-owned device pointers; outputs must not overlap
 * the inputs or each other; every 16-bit tensor is 16-byte aligned, lse and
 * delta 4-byte aligned.  One query head of Q and of dout must span less than
 * 2^31 bytes (ATTN_ERR_TOO_LARGE).  Three kernels are enqueued on `stream`;
 * errors as attn_fwd.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
             int causal, float scale, void* stream);

/*
 * attn_bwd_ex -- attn_bwd for bf16 or fp16 tensors: dtype ATTN_DTYPE_BF16 or
 * ATTN_DTYPE_FP16 is the element type of q, k, v, o, dout, dq, dk and dv, and
 * of P and dS in the products (the FA4 chapter's usage example runs fp16).
 * Other arguments, layouts and errors as attn_bwd; ATTN_ERR_BAD_ARGUMENT for
 * another dtype.
 */
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, float* delta,
                int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
                int dtype, int causal, float scale, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight loops, harnesses that forbid
 * hipMalloc): the same kernels and the same dq, dk and dv, bit for bit, with
 * D = rowsum(dout * o) kept in a fixed device array inside the library instead
 * of a caller's delta buffer.  Nothing is allocated by this call or by the
 * library: the array is a file-scope device variable of
 * ATTN_BWD_NOALLOC_MAX_ROWS floats (16 MiB), which each device the library
 * runs on holds until the process ends; its device address is looked up once
 * per device on the first call there.
 *   Arguments as attn_bwd without delta.
 *   Returns ATTN_ERR_SCRATCH when B * Hq * Lq > ATTN_BWD_NOALLOC_MAX_ROWS
 *   (checked before any HIP call); other errors as attn_bwd.
 * Every call on one device shares that device's array, and D is written in
 * full by each call before its kernels read it, so no clearing is needed; but
 * calls that overlap on one device (on different streams, or from different
 * host threads without ordering) race on the array and must not be issued.
 */
#define ATTN_BWD_NOALLOC_MAX_ROWS (4LL << 20)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
                     int causal, float scale, void* stream);

/*
 * attn_fwd_decode -- attn_fwd_split's per-split states, computed by a kernel
 * that streams the keys for few query rows per K/V head: at most 16 rows,
 * Lq * (Hq / Hkv) <= 16, as in decoding one or a few new tokens per sequence
 * ("Infra: Flash Attention", section on prefill versus decode).  Arguments,
 * layouts, splits, head shapes and outputs as attn_fwd_split (contiguous
 * bf16 tensors; (d_qk, d_v) one of (64,64), (128,128), (192,128)).
 * Returns ATTN_ERR_BAD_ARGUMENT when Lq * (Hq / Hkv) > 16 or n_split is
 * outside [1, 4096]; other errors as attn_fwd.  attn_fwd_split calls it by
 * itself for every shape it accepts, so this entry point only pins the
 * choice.  One kernel on `stream`.
 */
int attn_fwd_decode(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                    int B, int Hq, int Hkv, int Lq, int Lk, int d_qk, int d_v,
                    int causal, float scale, int n_split, void* stream);

/*
 * Packed variable-length batches ("Flash Attention 4 ..." review, method part
 * on scheduling: variable-length batches are scheduled by the execution time
 * of their work tiles, longest first).  n_seq sequences are packed along the
 * token axis; sequence s owns query tokens [cu_seqlens_q[s], cu_seqlens_q[s+1])
 * and key tokens [cu_seqlens_k[s], cu_seqlens_k[s+1]), and its queries attend
 * only its own keys, with the causal mask aligned bottom-right inside the
 * sequence (query i of Lq_s sees keys j <= i + Lk_s - Lq_s).  A sequence may
 * be empty; rows of a sequence without visible keys get O = 0, lse = -inf.
 *
 * attn_varlen_plan -- host-side schedule of such a batch, computed on the
 * CPU from HOST arrays cu_seqlens_q and cu_seqlens_k (n_seq + 1 ints each,
 * starting at 0, non-decreasing).  Writes *n_records, the number of tile
 * records (a multiple of 8), and, when plan is not NULL, the records
 * themselves: ATTN_VARLEN_RECORD_INTS ints each into the host buffer plan of
 * `capacity` records.  The order is the schedule: K/V heads dealt to the
 * chip's 8 dies longest first, tiles longest first within each die's
 * sections.  The plan depends on the sequence lengths, Hq, Hkv and causal.
 * Returns ATTN_ERR_NULL_PTR (cu arrays or n_records NULL),
 * ATTN_ERR_BAD_SHAPE (n_seq < 1, Hq or Hkv < 1, offsets not starting at 0 or
 * decreasing), ATTN_ERR_GQA_RATIO, ATTN_ERR_BAD_ARGUMENT (capacity too small)
 * or ATTN_ERR_TOO_LARGE.  No HIP call is made.
 */
#define ATTN_VARLEN_RECORD_INTS 8
int attn_varlen_plan(const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seq, int Hq,
                     int Hkv, int causal, int* plan, int capacity, int* n_records);

/*
 * attn_fwd_varlen -- attention forward over a packed variable-length batch.
 *   q    [total_q, Hq,  d_qk]  bfloat16, token-major and contiguous
 *   k    [total_k, Hkv, d_qk]  bfloat16
 *   v    [total_k, Hkv, d_v ]  bfloat16
 *   o    [total_q, Hq,  d_v ]  bfloat16 (output)
 *   lse  [Hq, total_q]         float32 (output)
 *   plan the records of attn_varlen_plan for this batch, Hq, Hkv and causal,
 *        copied to DEVICE memory (16-byte aligned); n_records of them
 * A record that does not fit total_q / total_k / the head counts is treated as
 * an empty tile, so a stale plan cannot make the kernel read or write out of
 * bounds; a plan built for other lengths gives wrong rows.  Other arguments,
 * ownership, asynchrony and errors as attn_fwd (one kernel on `stream`), with
 * ATTN_ERR_BAD_SHAPE for total_q < 1 or total_k < 0, ATTN_ERR_BAD_ARGUMENT for
 * n_records not a multiple of 8, and ATTN_ERR_TOO_LARGE when K or V spans
 * 2^31 bytes or more.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* plan, int n_records, int total_q, int total_k, int Hq, int Hkv,
                    int d_qk, int d_v, int causal, float scale, void* stream);

/* attn_status_string -- static, NUL-terminated description of a status code
 * (never NULL; unknown codes give "unknown attn status"). */
const char* attn_status_string(int status);

/* attn_abi_version -- version of this ABI (incremented on any change to the
 * signatures or semantics above). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
