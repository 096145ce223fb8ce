/*
 * fa355.h — C ABI of libfa355: the fused, tiled attention forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * Pages cited (title, then the section on that page):
 *   [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
 *   [AI] "AIInfra笔记01"                                   (kwkr.cn/news/547341)
 *   [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)
 *
 * The operation.  For every batch index b, head h and query row i:
 *
 *     s_ij    = scale * sum_d q[b,h,i,d] * k[b,h,j,d]            j visible to i
 *     o[b,h,i,:] = sum_j exp(s_ij) * v[b,h,j,:] / sum_j exp(s_ij)
 *     lse[b,h,i] = ln sum_j exp(s_ij)
 *
 * that is, scaled dot-product attention with a row softmax ([OP §2.1], the
 * scores-times-scale, softmax, times-v form; [DF §2.1], the three stages QKᵀ,
 * softmax, PV), computed without the score matrix ever reaching memory: the
 * query rows are cut into tiles, key/value tiles stream past them, and each row
 * keeps a running max and exp-sum that are folded into the output once all of
 * its key tiles are seen ([DF §2.2], first and second layers; [OP §1], fusion
 * and tiling).  The per-row log-sum-exp is the softmax statistic kept for a
 * backward pass ([DF §2.2], third layer; [AI §3.2] sizes it as one float per
 * row).  With causal != 0, key j is visible to row i iff j <= i + (Lk - Lq)
 * ([DF §4.1], causal flag; diagonal included; for Lq < Lk the queries are taken
 * as the last Lq positions of the keys, "bottom-right" alignment).
 *
 * Precision: q, k, v and o are fp16 or bf16; products are accumulated in fp32;
 * the softmax runs in fp32 ([OP §4.1]: half-precision inputs, fp32 softmax
 * accumulation).  The attention weights are rounded to the input type before
 * they multiply v, and o is divided by the sum of those rounded weights; lse is
 * taken from the fp32 sum.  o is rounded to nearest even.
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (same type as hipStream_t; NULL = the null stream of the current device). */
struct ihipStream_t;
typedef struct ihipStream_t* fa_stream_t;

typedef enum {
  FA_DTYPE_F16 = 0,  /* IEEE binary16 */
  FA_DTYPE_BF16 = 1  /* bfloat16 */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,         /* q, k, v, o or lse is NULL                                         */
  FA_ERR_SHAPE = -2,        /* B, H, Lq or Lk < 1, or a size beyond the limits below              */
  FA_ERR_HEAD_DIM = -3,     /* D is not 64 or 128                                                */
  FA_ERR_DTYPE = -4,        /* dtype is not FA_DTYPE_F16 or FA_DTYPE_BF16                        */
  FA_ERR_ALIGN = -5,        /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned        */
  FA_ERR_SCALE = -6,        /* scale is NaN or infinite                                          */
  FA_ERR_CAUSAL_SHAPE = -7, /* causal with Lq > Lk (rows would have no visible key)              */
  FA_ERR_DEVICE = -8,       /* the current device has no gfx950 code object for the kernel       */
  FA_ERR_LAUNCH = -9,       /* the kernel launch failed (HIP code in fa_last_hip_error())        */
  FA_ERR_STRIDE = -10,      /* fa_fwd_strided: a stride < 0, or a row stride < D                 */
  FA_ERR_SPLITS = -11,      /* fa_fwd_splitkv: num_splits outside 1..256                         */
  FA_ERR_WORKSPACE = -12,   /* fa_fwd_splitkv / fa_bwd: workspace smaller than its size query    */
  FA_ERR_DROPOUT = -13      /* dropout probability outside [0, 1), or round((1-p)*256) == 0      */
} fa_status;

/*
 * fa_fwd — enqueue one fused attention forward pass on `stream`.
 *
 * Arguments (all device pointers, allocated and owned by the caller):
 *   q    [B, H, Lq, D]  dense row-major, element type `dtype`; read only.
 *   k    [B, H, Lk, D]  dense row-major, `dtype`; read only.
 *   v    [B, H, Lk, D]  dense row-major, `dtype`; read only.
 *   o    [B, H, Lq, D]  dense row-major, `dtype`; written (every element).
 *   lse  [B, H, Lq]     fp32; written (every element), natural log.
 *   B, H, Lq, Lk        batch, heads, query rows, key rows (all >= 1).
 *   D                   head dimension: 64 or 128.
 *   scale               logit multiplier, any finite value (typically 1/sqrt(D));
 *                       applied in fp32 to the fp32 dot products.
 *   causal              0: every key is visible; non-zero: key j visible to row i iff
 *                       j <= i + (Lk - Lq), which requires Lq <= Lk.
 *   dtype               FA_DTYPE_F16 or FA_DTYPE_BF16 (q, k, v and o share it).
 *   stream              HIP stream to enqueue on.
 *
 * Limits: ((L + 256)*D + D)*2 must stay below 2^32 bytes for L = Lq and L = Lk
 * (one head's slab is addressed with 32-bit offsets: L < 16,776,959 at
 * D = 128), and B*H*ceil(Lq/256) < 2^22 workgroups.
 *
 * Semantics: validation happens on the host before any HIP call; an invalid
 * argument returns its FA_ERR_* code and enqueues nothing.  On success one
 * kernel is enqueued and the call returns at once (asynchronous: o and lse are
 * valid when the stream reaches that point).  The library allocates no memory,
 * keeps no pointer after returning, never synchronises, never prints and never
 * aborts.  o and lse must not overlap q, k or v (not checked).  The result is
 * bitwise reproducible: the same inputs give the same bits on every call.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Lq, int Lk, int D, float scale, int causal, int dtype,
           fa_stream_t stream);

/*
 * fa_fwd_strided — fa_fwd on strided views: the same operation, result and
 * semantics, with q, k, v and o given by element strides instead of the dense
 * [B, H, L, D] layout, so that [B, L, H, D] tensors and a packed qkv buffer of
 * shape [B, L, 3, H, D] are used in place, with no copies.  These are the call
 * forms the pages' interfaces take ([DF §4.1], attention on (batch, sequence,
 * heads, head-dim) tensors; [AI §4.2], the packed-qkv call).
 *
 * Element (b, h, i, d) of q is at q + (b*q_stride[0] + h*q_stride[1] +
 * i*q_stride[2] + d) elements; likewise k, v (rows 0..Lk-1) and o.  Each
 * *_stride points to three int64 values in host memory, read during the call
 * only.  The head dim is contiguous.  lse stays dense [B, H, Lq] fp32.
 *
 * Extra checks, before any HIP call: the stride pointers are non-NULL
 * (FA_ERR_NULL); every stride is >= 0 and every row stride >= D (FA_ERR_STRIDE;
 * batch or head strides of 0 broadcast one slab, e.g. K/V shared by all heads);
 * every stride is a multiple of 8 elements, so that each row starts on a 16-byte
 * boundary (FA_ERR_ALIGN); ((L + 256)*row_stride + D)*2 < 2^32 for each tensor
 * (FA_ERR_SHAPE).  Rows of o must not overlap each other or q, k, v (not
 * checked).  fa_fwd is this call with the dense strides.
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                   int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                   const int64_t* o_stride, float scale, int causal, int dtype, fa_stream_t stream);

/*
 * fa_fwd_splitkv — fa_fwd_strided with the keys of every (batch, head, query
 * tile) divided into num_splits equal ranges computed by separate workgroups,
 * then merged: each range yields its unnormalised output and the running max
 * and exp-sums of its rows, and a second kernel combines them exactly (the
 * streaming update of [DF §2.2] applied across ranges), so the result equals
 * one pass up to fp32 rounding.  This fills the GPU when B*H*ceil(Lq/256) is
 * small; it is also the merge a multi-GPU split of the keys would use.
 *
 *   num_splits        1..256 (FA_ERR_SPLITS otherwise); 1 is fa_fwd_strided and
 *                     ignores the workspace.
 *   workspace         device memory of at least
 *                     fa_fwd_splitkv_workspace_size(B, H, Lq, D, num_splits)
 *                     bytes (FA_ERR_WORKSPACE), 256-byte aligned (FA_ERR_ALIGN),
 *                     owned by the caller, overwritten by the call, free again
 *                     once the stream has passed it; NULL is FA_ERR_NULL when
 *                     num_splits > 1.  (Lq + 256)*D*4 must stay below 2^32.
 *
 * Two kernels are enqueued on stream (partials, then merge).  Calls that share
 * one workspace must be ordered on one stream.
 */
size_t fa_fwd_splitkv_workspace_size(int B, int H, int Lq, int D, int num_splits);

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                   int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                   const int64_t* o_stride, float scale, int causal, int dtype, int num_splits, void* workspace,
                   size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_fwd_splitkv_noalloc — fa_fwd_splitkv without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory at the
 * time of the call: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.
 *
 * The partials live in a device array of FA_NOALLOC_SCRATCH_BYTES compiled into
 * the library; each GPU the library runs on holds its own copy from the first
 * call on that GPU until the process ends.  The arguments and results are those
 * of fa_fwd_splitkv with the same num_splits (the same kernels; bitwise equal
 * outputs).  The call allocates nothing (no hipMalloc, no library allocation);
 * its first call on a device looks up that device's copy of the array once.
 *
 *   fa_fwd_splitkv_workspace_size(B, H, Lq, D, num_splits) must not exceed
 *   FA_NOALLOC_SCRATCH_BYTES (FA_ERR_WORKSPACE otherwise; nothing enqueued).
 *   num_splits = 1 is fa_fwd_strided and touches no scratch memory.
 *
 * Every call on one GPU uses that GPU's one array: calls that may overlap on a
 * GPU (different streams, or different host threads without ordering) race on
 * it and give wrong results; order them on one stream.  No part of the array
 * needs clearing between calls (each call writes every partial it reads).
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                           int Lk, int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                           const int64_t* o_stride, float scale, int causal, int dtype, int num_splits,
                           fa_stream_t stream);

/*
 * fa_bwd — enqueue the attention backward pass on `stream`: the gradients of
 * o (the forward operation above) with respect to q, k and v for an upstream
 * gradient dout of o.
 *
 * [DF §2.2] (third layer, recomputation): no score matrix is stored; the score
 * tiles are recomputed from q and k, and the probabilities from the forward
 * pass's lse: P_ij = exp(s_ij - lse_i) on visible pairs (the same visibility
 * rule as fa_fwd, including causal with Lq <= Lk).  The gradients are those of
 * the forward definition:
 *
 *     dv_j  = sum_i P_ij dout_i
 *     dS_ij = P_ij * (dout_i . v_j - D_i),   D_i = dout_i . o_i
 *     dq_i  = scale * sum_j dS_ij k_j,       dk_j = scale * sum_i dS_ij q_i
 *
 * (D_i = sum_j P_ij (dout_i . v_j) because the row of P sums to one.)
 *
 *   q, o, dout [B, H, Lq, D]   dense row-major, `dtype`, read only; o and lse
 *                              must be the outputs of fa_fwd on the same q, k,
 *                              v, scale and causal flag.
 *   k, v       [B, H, Lk, D]   dense row-major, `dtype`, read only.
 *   lse        [B, H, Lq]      fp32, natural log (fa_fwd's output), read only.
 *   dq         [B, H, Lq, D]   written, `dtype` (rounded to nearest even).
 *   dk, dv     [B, H, Lk, D]   written, `dtype`.
 *   workspace                  at least fa_bwd_workspace_size(B, H, Lq) bytes,
 *                              256-byte aligned, device memory owned by the
 *                              caller (2 fp32 values per query row, rows
 *                              padded to a multiple of 4), written
 *                              by the call; calls sharing one workspace must be
 *                              ordered on one stream.
 *   B, H, Lq, Lk, D, scale, causal, dtype, stream: as for fa_fwd.
 *
 * dq, dk, dv must not overlap each other or the inputs.  q, k, v, o, dout, dq,
 * dk, dv must be 16-byte aligned (FA_ERR_ALIGN), lse 4-byte aligned.  Every
 * pointer is required (FA_ERR_NULL).  Limits: (L + 256)*D*2 < 2^32 bytes for
 * L = Lq and L = Lk (FA_ERR_SHAPE).  Two kernels are enqueued (dq, which
 * also writes every row's D_i and lse_i*log2(e) to the workspace, then dk and
 * dv, which read them); the call returns without synchronising.
 * Precision: fp32 accumulation; P and dS are rounded to `dtype` as matrix-core
 * operands (at D = 128 dk's dS is formed from P as rounded).  Each output element is written by exactly one thread, in a fixed
 * order, so results are bitwise reproducible.
 */
size_t fa_bwd_workspace_size(int B, int H, int Lq);

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int Lq, int Lk, int D, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_fwd_dropout / fa_bwd_dropout — fa_fwd and fa_bwd with dropout on the
 * attention weights ([DF §4.1] passes a dropout probability with the call; the
 * pages give no random number generator, so the generator below is a reading).
 *
 *     o[b,h,i,:] = sum_j P_ij * M_ij * v[b,h,j,:],   P_ij = exp(s_ij - lse_i)
 *
 * with M_ij = 256/T if the weight is kept and 0 otherwise, T = round((1 -
 * dropout_p) * 256) in [1, 256] (the keep probability is T/256, so the expected
 * output is the output without dropout).  lse is that of the scores, as
 * without dropout.  Keep bits: Philox4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011) with key (seed & 0xffffffff, seed >> 32)
 * and counter (j / 4, i / 4, b*H + h, 0); output word w, byte n is the byte of
 * row 4*(i/4) + w and key 4*(j/4) + n; the weight is kept iff that byte < T.  The
 * same seed and dropout_p must be passed to fa_bwd_dropout, whose gradients are
 * those of this output (the mask is recomputed, never stored).
 * dropout_p = 0 is exactly fa_fwd / fa_bwd.  Other arguments, layouts and errors
 * as for fa_fwd and fa_bwd; FA_ERR_DROPOUT for dropout_p outside [0, 1) or T == 0.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                   int D, float scale, int causal, int dtype, float dropout_p, uint64_t seed, fa_stream_t stream);

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk, int D, float scale, int causal,
                   int dtype, float dropout_p, uint64_t seed, void* workspace, size_t workspace_bytes,
                   fa_stream_t stream);

/*
 * fa_fwd_dropout_strided — fa_fwd_dropout on strided views (the strides of
 * fa_fwd_strided, with its checks).
 */
int fa_fwd_dropout_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                           int Lk, int D, const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
                           const int64_t* o_stride, float scale, int causal, int dtype, float dropout_p,
                           uint64_t seed, fa_stream_t stream);

/*
 * fa_bwd_strided — fa_bwd (and, with dropout_p > 0, fa_bwd_dropout) on strided
 * views: `strides` points to 24 int64 values, the (batch, head, row) element
 * strides of q, k, v, o, dout, dq, dk, dv in that order (each head dim
 * contiguous), so [B, L, H, D] tensors and packed qkv / dqkv buffers are used in
 * place.  Strides must be >= 0 with a row stride >= D (FA_ERR_STRIDE) and
 * multiples of 8 elements (FA_ERR_ALIGN); ((L + 256) * row_stride + D) * 2 must
 * stay below 2^32 per tensor (FA_ERR_SHAPE).  lse and the workspace stay dense.
 * Output views (dq, dk, dv) must not overlap each other or the inputs.  NULL
 * strides: FA_ERR_NULL.  fa_bwd and fa_bwd_dropout are this call with the dense
 * strides.
 */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk, int D, const int64_t* strides,
                   float scale, int causal, int dtype, float dropout_p, uint64_t seed, void* workspace,
                   size_t workspace_bytes, fa_stream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_status_string(int status);

/* The hipError_t behind the calling thread's last FA_ERR_LAUNCH or FA_ERR_DEVICE (0 if none). */
int fa_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

/*
 * fa_fwd_launch_shape — the grid of the attention kernel that fa_fwd
 * (fa_fwd_strided, fa_fwd_dropout with num_splits = 1, fa_fwd_splitkv with
 * num_splits) launches for these sizes on the calling thread's current device:
 * for callers that plan around it, and for tests of the launch forms.  No device
 * memory is touched and nothing is enqueued; the device's CU count is read once.
 *
 *   workgroups           workgroups of the attention kernel (written)
 *   rows_per_workgroup   query rows of one work item (written): 256, or 128 in
 *                        the two-key-group form, taken by a single pass whose
 *                        grid of 256-row items would not exceed the CU count
 *   items_per_workgroup  1, or 2 in the paired form (written): two-key-group
 *                        grids without dropout whose items outnumber the CUs
 *                        (causal ones only when each XCD's block of items holds
 *                        whole pairs of heads); a workgroup then runs a heavy
 *                        and a light causal query block
 *
 * Returns FA_OK, or the status fa_fwd would return for these sizes:
 * FA_ERR_NULL (an output pointer is NULL), FA_ERR_SHAPE, FA_ERR_HEAD_DIM,
 * FA_ERR_CAUSAL_SHAPE, FA_ERR_DROPOUT, FA_ERR_SPLITS (num_splits outside
 * 1..256, or above 1 with dropout).  When the CU count cannot be read the
 * 256-row form is reported, as the forward call would then launch it.
 */
int fa_fwd_launch_shape(int B, int H, int Lq, int Lk, int D, int causal, float dropout_p, int num_splits,
                        int* workgroups, int* rows_per_workgroup, int* items_per_workgroup);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
