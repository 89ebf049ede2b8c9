/*
 * fa.h — C ABI of the MI355X (gfx950) exact attention forward library (libfa.so).
 *
 * One call computes, for every (batch b, head h) slice of contiguous tensors,
 *     S = Q K^T,  P = softmax_row(s S),  O = P V,  LSE_i = ln sum_j exp(s S_ij)
 * with the FlashAttention-2 loop order: a workgroup keeps one block of query rows
 * on chip, streams blocks of K and V, updates the per-row online-softmax state
 * (running raw maximum m, sum l, unnormalised numerator U rescaled by
 * alpha = exp(s (m - m'))) and normalises once at the end. S and P never reach
 * device memory.
 *
 * Sources for the operation: "用 CuTe 读懂 FlashAttention：一次 forward 的完整流程"
 * (blog.qingsen.net) — the notation block (S, P, O, s = 1/sqrt(D)), step 4 (the
 * online-softmax state and recurrence), the causal section (top-left alignment,
 * Fig. 11) and the final section (O = U / l, LSE = s m + log l); "CUDA 算子工程"
 * ch. 14 §14.5 (FA2 forward: inputs Q, K, V in [N, d], outputs O in [N, d] and
 * LSE in [N]).
 *
 * Every entry point is a plain C function; no C++ or framework type crosses it.
 * Functions return a status code and never throw, print or abort.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle, declared exactly as the HIP runtime headers declare it, so that
 * this header needs none of them (a repeated identical typedef is valid C and C++). */
typedef struct ihipStream_t* hipStream_t;

/* Element type of Q, K, V and O. */
typedef enum {
  FA_F16 = 0,  /* IEEE binary16 */
  FA_BF16 = 1  /* bfloat16 */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,           /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,          /* a size is negative, or Hq is not a positive multiple of Hk */
  FA_ERR_UNSUPPORTED_HEADDIM = 3,/* d is not 64 or 128 */
  FA_ERR_BAD_SCALE = 4,          /* scale is not finite or not > 0 */
  FA_ERR_BAD_DTYPE = 5,          /* dtype is not FA_F16 / FA_BF16 */
  FA_ERR_MISALIGNED = 6,         /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
  FA_ERR_TOO_LARGE = 7,          /* (N + 512) * row stride >= 2^30 elements, B * H * N >= 2^31, or the grid exceeds 2^31-1 workgroups */
  FA_ERR_UNSUPPORTED_TILE = 8,   /* (block_m, block_n) not among the compiled tile shapes */
  FA_ERR_HIP = 9,                /* the HIP runtime refused a launch of this call (that launch's own status;
                                    an error pending from an earlier HIP call of the thread is left as it was) */
  FA_ERR_BAD_STRIDE = 10,        /* a stride is negative or not a multiple of 8 elements, or a row stride < d */
  FA_ERR_BAD_SPLITS = 11,        /* num_splits outside [1, 256] */
  FA_ERR_WORKSPACE = 12,         /* workspace (split-KV or backward) NULL, not 16-byte aligned or too small */
  FA_ERR_SCRATCH_LIMIT = 13      /* fa_fwd_split_noalloc: the partials exceed FA_SPLIT_SCRATCH_BYTES */
} fa_status;

/* Size of the per-GPU scratch array fa_fwd_split_noalloc uses (64 MiB). */
#define FA_SPLIT_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fa_fwd — exact attention forward, asynchronous on `stream`.
 *
 *   q, k, v : device pointers to [B, H, N, d] contiguous tensors of `dtype`
 *             (row-major; element (b,h,i,c) at ((b*H + h)*N + i)*d + c). Read only.
 *   o       : device pointer to a [B, H, N, d] contiguous tensor of `dtype`; fully
 *             overwritten. Must not overlap q, k or v.
 *   lse     : device pointer to a [B, H, N] contiguous float32 tensor; fully
 *             overwritten with ln sum_{valid j} exp(scale * q_i . k_j).
 *   B, H, N : batch, heads, sequence length (queries and keys alike). N need not
 *             be a multiple of any tile size.
 *   d       : head dimension, 64 or 128.
 *   scale   : the softmax scale s (the caller passes 1/sqrt(d) for standard
 *             attention; there is no default at this level). Finite and > 0.
 *   causal  : nonzero masks key j > query i (top-left alignment, j <= i valid).
 *   dtype   : FA_F16 or FA_BF16. Scores, softmax state and accumulators are fp32;
 *             the softmax weights are rounded to `dtype` (round-to-nearest-even)
 *             for the P·V product and O is rounded to `dtype` at the end.
 *   stream  : the HIP stream to enqueue on (NULL = the default stream).
 *
 * Ownership: the caller allocates and frees every buffer. The library allocates
 * nothing, keeps no state between calls and does not synchronise; the call
 * returns once the kernel is enqueued. A device fault surfaces at the caller's
 * next synchronisation. B*H*N == 0 is a no-op that returns FA_OK.
 * Errors: arguments are validated before anything is launched; on any status
 * other than FA_OK nothing was enqueued (FA_ERR_HIP: the launch itself failed).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                 fa_dtype dtype, hipStream_t stream);

/*
 * fa_fwd_tiled — fa_fwd with an explicit tile shape: block_m query rows per
 * workgroup and block_n keys per K/V tile (fa_fwd picks these itself). The tile is
 * the blocking of "用 CuTe 读懂 FlashAttention" (its opening example fixes
 * BlockM = BlockN = 64: one thread block per 64 query rows walking K/V in blocks of
 * 64 keys); the 128-row single-head workload names that tile. Used for testing and
 * tuning. Supported shapes are reported by fa_tile_supported; any other pair returns
 * FA_ERR_UNSUPPORTED_TILE without launching.
 */
fa_status fa_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                       fa_dtype dtype, hipStream_t stream, int block_m, int block_n);

/*
 * fa_fwd_ex — the general form of fa_fwd, asynchronous on `stream`: unequal query and
 * key lengths, grouped K/V heads and strided tensors.
 *
 *   q, o    : [B, Hq, Nq, d] of `dtype`; o fully overwritten.
 *   k, v    : [B, Hk, Nk, d] of `dtype`. Query head h reads K/V head h / (Hq / Hk)
 *             (Hq must be a positive multiple of Hk: Hk = Hq is plain multi-head
 *             attention, Hk = 1 shares one K/V head among all query heads). This is
 *             the grouping of "CUDA 算子工程：手写 FlashAttention v2 之路" ch. 14,
 *             §14.7.1 (one K/V head serving the query heads of its group), with
 *             consecutive query heads forming a group.
 *   lse     : [B, Hq, Nq] contiguous float32, fully overwritten.
 *   *_strides: {batch, head, row} element strides of that tensor, d contiguous; NULL
 *             means contiguous (the arbitrary strides that "用 CuTe 读懂 FlashAttention"
 *             lists among its tutorial's limitations). Each stride is a non-negative multiple of 8 elements
 *             (rows stay 16-byte aligned) and the row stride is at least d. K and V
 *             may share storage or broadcast (stride 0); the rows of o must not
 *             overlap each other or q, k, v.
 *   causal  : nonzero masks key j > i + Nk - Nq for query i, the bottom-right
 *             alignment ("用 CuTe 读懂 FlashAttention", causal section, names it as
 *             the one that differs from top-left only when the lengths differ): the
 *             last query sees every key. With Nq = Nk this is fa_fwd's mask. A query
 *             with no visible key (Nq > Nk, i < Nq - Nk) gets O = 0 and LSE = -inf.
 *   block_m, block_n: a compiled tile, or 0, 0 for the tile fa_fwd would choose for
 *             B, Hq and Nq (for the packed row count when grouped heads are packed, see
 *             below).
 *   Other arguments, ownership and errors as for fa_fwd; additionally
 *   FA_ERR_BAD_STRIDE. Nk = 0 is allowed (every row gets O = 0, LSE = -inf; k and v
 *   may then be NULL). B*Hq*Nq == 0 is a no-op.
 */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d,
                    const int64_t* q_strides, const int64_t* k_strides,
                    const int64_t* v_strides, const int64_t* o_strides,
                    float scale, int causal, fa_dtype dtype, hipStream_t stream,
                    int block_m, int block_n);

/*
 * fa_fwd_split — fa_fwd_ex with the keys of every query block divided into up to
 * num_splits ranges, each handled by its own workgroup (split-KV: "CUDA 算子工程：手写
 * FlashAttention v2 之路" ch. 14, §14.7.1, for long key sequences with few query
 * blocks, as in decoding, where one workgroup per query block would leave most of the
 * GPU idle). Range k of a row leaves its partial output O_k = U_k / l_k (fp32) and
 * LSE_k in `workspace`; a second kernel on the same stream merges them with the
 * online-softmax algebra of "用 CuTe 读懂 FlashAttention" step 4 applied to whole
 * ranges: LSE = ln sum_k exp(LSE_k), O = sum_k exp(LSE_k - LSE) O_k.
 *
 *   num_splits: 1..256. The ranges are whole key tiles, so fewer ranges than asked
 *             are used when Nk has fewer tiles; 1 is exactly fa_fwd_ex (no workspace
 *             needed). fa_split_default suggests a count.
 *   workspace: device memory owned by the caller, 16-byte aligned, of at least
 *             fa_split_workspace_bytes(B, Hq, Nq, d, num_splits) bytes. Its contents
 *             on entry do not matter; it is in use until the merge kernel has run (stream
 *             order), so calls that overlap on different streams need separate
 *             workspaces. May be NULL when no split is made.
 *   Other arguments, results and errors as fa_fwd_ex; additionally FA_ERR_BAD_SPLITS
 *   and FA_ERR_WORKSPACE. The result equals fa_fwd_ex's up to rounding.
 *
 * With Hq > Hk and fewer than 64 query rows per head (decoding, a few draft tokens)
 * fa_fwd_ex and fa_fwd_split process the query heads that share a K/V head as the
 * rows of one slice, so that each K/V tile is read once for the whole group. With one
 * row per head this holds for any layout; with more, q and o must be head-contiguous
 * (head stride = Nq row strides, as in a contiguous [B, Hq, Nq, d]), and other
 * layouts run unpacked. The results do not depend on it beyond rounding.
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d,
                       const int64_t* q_strides, const int64_t* k_strides,
                       const int64_t* v_strides, const int64_t* o_strides,
                       float scale, int causal, fa_dtype dtype, hipStream_t stream,
                       int block_m, int block_n, int num_splits, void* workspace,
                       size_t workspace_bytes);

/*
 * fa_fwd_split_noalloc — fa_fwd_split without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc. The partials go to a scratch array that the library
 * holds in each GPU's memory (FA_SPLIT_SCRATCH_BYTES, 64 MiB, allocated when the
 * library's code is loaded on that GPU and kept until the process ends); the call itself
 * allocates and frees nothing. Its device address is looked up on the first call on a
 * device (the device current at the call, which must be the device of `stream`).
 *
 *   Arguments, results and other errors as fa_fwd_split with num_splits ranges.
 *   FA_ERR_SCRATCH_LIMIT (nothing launched) when fa_split_workspace_bytes(B, Hq, Nq,
 *   d, num_splits) exceeds FA_SPLIT_SCRATCH_BYTES; FA_ERR_HIP if the scratch address
 *   cannot be obtained. num_splits = 1 does not touch the scratch.
 *
 * The scratch array is shared by every call on a GPU and holds the last call's
 * partials; no contents need clearing between calls (every range writes its partials
 * before the merge reads them). Calls that overlap on one GPU (different streams, or
 * different host threads without ordering) race on it and give wrong results:
 * serialise them, or use fa_fwd_split with separate workspaces.
 */
fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t B, int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d,
                               const int64_t* q_strides, const int64_t* k_strides,
                               const int64_t* v_strides, const int64_t* o_strides,
                               float scale, int causal, fa_dtype dtype, hipStream_t stream,
                               int block_m, int block_n, int num_splits);

/* Workspace bytes fa_fwd_split needs for these sizes and num_splits: 4 (d + 1) bytes
 * per range and query row; 0 if num_splits = 1 or an argument is out of range. */
size_t fa_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t d, int num_splits);

/* A split count for fa_fwd_split (>= 1): enough key ranges that query blocks times
 * ranges fill the GPU's workgroup slots (two per compute unit for blocks at most half
 * full, else as many as fit), at most one range per 8 key tiles and at most 256; 1 when
 * the query blocks alone fill the GPU. Grouped heads with fewer than 64 rows count as
 * packed (assuming head-contiguous q and o). block_m, block_n as in fa_fwd_ex (0, 0:
 * the default tile). */
int fa_split_default(int64_t B, int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d, int causal,
                     int block_m, int block_n);

/*
 * fa_bwd — gradients of the attention forward, asynchronous on `stream`: for
 * O = softmax(scale q k^T) v (fa_fwd's result, causal as there) and dout = dL/dO,
 * writes dq = dL/dq, dk = dL/dk, dv = dL/dv. The pages define the forward; the
 * forward's LSE output is kept for this pass ("CUDA 算子工程：手写 FlashAttention v2
 * 之路" ch. 14 §14.5). The gradients are the forward differentiated:
 * P = exp(scale q k^T - LSE) (recomputed from `lse`), dv = P^T dout,
 * dP = dout v^T, D = rowsum(dout * o), dS = P * (dP - D), dq = scale dS k,
 * dk = scale dS^T q.
 *
 *   q, k, v, o, dout: device pointers to [B, H, N, d] contiguous tensors of `dtype`
 *             (o as returned by fa_fwd for these q, k, v, scale, causal). Read only.
 *   lse     : [B, H, N] contiguous float32, as returned by fa_fwd.
 *   dq, dk, dv: [B, H, N, d] contiguous `dtype`, fully overwritten; must not overlap
 *             the inputs or each other.
 *   workspace: device memory owned by the caller, 16-byte aligned, of at least
 *             fa_bwd_workspace_bytes(B, H, N) bytes (per query row: -D and the LSE
 *             in base-2 units); contents on entry do not matter; in use until the
 *             last kernel of the call has run.
 *   B, H, N, d, scale, causal, dtype, stream: as for fa_fwd.
 * Arithmetic: products in `dtype` on the matrix cores with fp32 accumulation; P and
 * dS are rounded to `dtype` (round-to-nearest-even) before the products that use
 * them. dq is computed by its own kernel (no atomics): results are deterministic.
 * Errors as for fa_fwd, plus FA_ERR_WORKSPACE; B*H*N == 0 is a no-op.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                 int64_t d, float scale, int causal, fa_dtype dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd_ex — fa_bwd for grouped K/V heads and unequal lengths, as fa_fwd_ex computes
 * them: q, o, dout, dq are [B, Hq, Nq, d], k, v, dk, dv are [B, Hk, Nk, d] (contiguous),
 * lse [B, Hq, Nq]; query head h reads K/V head h / (Hq / Hk), so dk and dv of a K/V
 * head sum the contributions of its Hq / Hk query heads; causal masks key
 * j > i + Nk - Nq (bottom-right). o and lse come from fa_fwd_ex on the same inputs.
 * Rows that see no key get dq = 0. The workspace holds 8 bytes per query row:
 * fa_bwd_workspace_bytes(B, Hq, Nq). Other arguments and errors as for fa_bwd; Nq = 0
 * writes dk = dv = 0, Nk = 0 writes dq = 0.
 */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hk,
                    int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, fa_dtype dtype,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes fa_bwd needs: 8 per query row (B * H * N * 8); 0 for an empty or
 * negative size. For fa_bwd_ex pass H = Hq and N = Nq. */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N);

/* 1 if (block_m, block_n) is compiled for head dimension d, else 0. */
int fa_tile_supported(int64_t d, int block_m, int block_n);

/* The tile shape fa_fwd would choose for these arguments (written to *block_m,
 * *block_n); returns FA_OK, or FA_ERR_UNSUPPORTED_HEADDIM / FA_ERR_NULL_PTR. */
fa_status fa_default_tile(int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                          int* block_m, int* block_n);

/* Static description of a status code. Never NULL. */
const char* fa_status_str(fa_status status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
