/*
 * fa.h -- C ABI of the MI355X (gfx950) fused attention forward library (libfa.so).
 *
 * The operation, per batch b and query head hq (hk = hq / (Hq / Hkv)):
 *
 *     S   = Q[b,hq] . K[b,hk]^T * scale  (+ bias[b,hq])          [Nq x Nk]
 *     S_ij = -inf  if causal and j > i   (top-left aligned)
 *     O[b,hq]   = softmax_rows(S) . V[b,hk]                        [Nq x D]
 *     LSE[b,hq] = log(sum_j exp(S_ij))  (natural log, per row)     [Nq]
 *
 * This is the attention of "FlashAttention principles and Triton practice"
 * (xnwp.cn/news/15505, §2.1) computed the tiled way of §2.2 there and of the
 * kwkr.cn/news/592482 tutorial (§2.2-§2.3): K/V column blocks are streamed past
 * a resident Q row block with the online softmax update, so S and P are never
 * written to memory.  The per-row statistic kept for a recompute-based backward
 * (kwkr.cn §2.4) is emitted as one LSE value per row.  The optional additive
 * logit term is the fused "logit residual" of the Block Attention Residual post
 * (iqiancheng.github.io): it is added to the already-scaled logits, tile by
 * tile, before the softmax.  Grouped-query attention maps query head hq to KV
 * head hq / (Hq / Hkv), i.e. contiguous groups.
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense, contiguous, row-major device memory owned by the
 *    caller:  q, o [B, Hq, Nq, D];  k, v [B, Hkv, Nk, D];
 *    bias [B, Hq, Nq, Nk] (may be NULL);  lse [B, Hq, Nq] float32.
 *  - q, k, v, bias and o share one element type (fa_dtype); lse is float32.
 *  - q, k, v, o and bias must be 16-byte aligned; lse 4-byte aligned.
 *  - o and lse must not overlap each other or any input.
 *  - scale is used as given (pass 1/sqrt(D) for the usual attention); any
 *    finite value, including 0 and negative values, is accepted.
 *  - A row that sees no key (Nk == 0) gets O = 0 and LSE = -inf.
 *  - B == 0, Hq == 0 or Nq == 0 is an empty problem: nothing is launched.
 *  - The library allocates no memory, never synchronises and never copies
 *    between host and device.  It keeps no state between calls, except for
 *    the one scratch array per GPU that fa_forward_split_noalloc uses (a
 *    static device array, not an allocation).  Every other entry point is
 *    reentrant.
 *  - Errors in the arguments are reported synchronously, as a nonzero status,
 *    before anything is launched.  A launch failure reported by the runtime is
 *    FA_ERR_HIP.  Faults during execution surface at the caller's next
 *    synchronisation on the stream.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, bias and o.
 * FA_DTYPE_FP8_E4M3: q, k and v in the OCP 8-bit E4M3 format (bias 7, largest
 * finite 448, the gfx950 native FP8); o is bf16; no bias.  The FP8 direction
 * of "FlashAttention principles and Triton practice" (xnwp.cn/news/15505), §7,
 * which asks for its precision loss to be evaluated: the probabilities are
 * rounded to E4M3 for the P.V product (the other arithmetic as for 16-bit
 * inputs).  fa_forward (fused), fa_forward_window and the key-split entry
 * points (fa_forward_split, fa_forward_split_noalloc: the decode step over an
 * FP8 KV cache), with or without the causal mask, D = 64 or 128; the other
 * entry points return FA_ERR_DTYPE for it. */
typedef enum fa_dtype {
  FA_DTYPE_BF16 = 0,
  FA_DTYPE_FP16 = 1,
  FA_DTYPE_FP32 = 2,
  FA_DTYPE_FP8_E4M3 = 3
} fa_dtype;

/* Status codes returned by every entry point. */
typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1, /* q, o or lse is NULL while the problem is not empty, or    */
                           /* k or v is NULL while Nk > 0                             */
  FA_ERR_BAD_SIZE = 2,     /* a size is negative, or Hkv < 1 while Hq > 0                */
  FA_ERR_HEAD_GROUPS = 3,  /* Hq is not a multiple of Hkv                                */
  FA_ERR_HEAD_DIM = 4,     /* D is not 64 or 128, nor 80, 96 or 256 with bf16/fp16 (80   */
                           /* and 96 run in 128-wide tiles, per the xnwp.cn post, §5.1   */
                           /* and §6.4: a block narrower than the head drops or misreads */
                           /* columns); the backward takes 256 without a logit term, its */
                           /* fp32 form 64 and 128, and the residual chain 64 to 128.    */
                           /* Other sizes are rejected, never silently truncated         */
  FA_ERR_DTYPE = 5,        /* dtype is not one of fa_dtype                               */
  FA_ERR_SCALE = 6,        /* scale is NaN or infinite                                   */
  FA_ERR_ALIGNMENT = 7,    /* a tensor pointer is not aligned as required above          */
  FA_ERR_OVERLAP = 8,      /* o or lse overlaps another buffer                           */
  FA_ERR_TOO_LARGE = 9,    /* a size exceeds the kernel's index range: B, Hq, Nq, Nk     */
                           /* < 2^30; B*Hq*ceil(Nq/128) < 2^31; one head's Q and one     */
                           /* head's K (Nq*D or Nk*D elements) < 2^31 bytes; with a bias, */
                           /* 128*Nk elements < 2^31 bytes                               */
  FA_ERR_HIP = 10,         /* the HIP runtime rejected the launch                        */
  FA_ERR_WORKSPACE = 11,   /* key-split workspace is NULL, too small or misaligned       */
  FA_ERR_SCRATCH_LIMIT = 12 /* fa_forward_split_noalloc: the partials need more than      */
                            /* FA_SPLIT_SCRATCH_BYTES                                    */
} fa_status;

/*
 * Validate the arguments of fa_forward without touching the GPU (pure host
 * code: no HIP call, no pointer dereference).  Returns FA_OK or the first
 * fa_status that applies.
 */
int fa_check_args(const void* q, const void* k, const void* v, const void* bias,
                  const void* o, const float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                  float scale, int causal, int dtype);

/*
 * Fused attention forward.  Writes o (dtype, rounded to nearest even) and lse
 * (float32) for every (b, hq, row).  bias may be NULL.  causal != 0 applies the
 * top-left causal mask.  stream is a hipStream_t (NULL = the null stream); the
 * work is enqueued on it and the call returns without waiting.
 *
 * Arithmetic: products in the input type on the matrix cores with float32
 * accumulation; softmax statistics in float32; the probabilities are rounded to
 * the input type before the P.V product (float32 inputs keep them in float32).
 */
int fa_forward(const void* q, const void* k, const void* v, const void* bias,
               void* o, float* lse,
               int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
               float scale, int causal, int dtype, void* stream);

/*
 * Causal sliding-window attention: fa_forward with causal = 1 and each query
 * row i limited to its window most recent keys, i - window < j <= i (the
 * window mask that "FlashAttention principles and Triton practice",
 * xnwp.cn/news/15505, §3.1, and the kwkr.cn/news/592482 tutorial's closing
 * remarks name as a variant of the same kernel).  Key tiles wholly outside a
 * row block's windows are skipped, so the work grows with Nq * window rather
 * than Nq * Nk.  window >= 1 (FA_ERR_BAD_SIZE otherwise; window >= Nk is the
 * plain causal result); everything else as fa_forward.
 */
int fa_forward_window(const void* q, const void* k, const void* v, const void* bias,
                      void* o, float* lse,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                      float scale, int64_t window, int dtype, void* stream);

/*
 * Block Attention Residual chain, forward of one layer ("Block Attention
 * Residual" Triton kernel post, iqiancheng.github.io: the A_i formula and the
 * 4-layer block diagram).  Inside a block, each layer adds the previous
 * layer's pre-softmax logits to its own, and those carry the layer before, so
 * layer p of a block (p = 0..3) sees
 *     S = sum over l = 0..p of Q_l K_l^T * scale     (+ causal mask)
 * and O = softmax(S) V_p, LSE as fa_forward.  The logits are recomputed tile
 * by tile from the layers' Q and K; no Nq x Nk tensor is read or written.
 *
 *   q_layers, k_layers: HOST arrays of num_layers DEVICE pointers, oldest
 *     layer first (the block's first layer) and the current layer last; every
 *     Q_l is [B, Hq, Nq, D] and every K_l [B, Hkv, Nk, D], all of dtype, with
 *     the GQA head mapping of fa_forward for every layer;
 *   num_layers: 1 .. 4 (FA_ERR_BAD_SIZE otherwise); 1 is fa_forward without
 *     a bias (a block's first layer);
 *   v: the current layer's V, [B, Hkv, Nk, D];
 *   o, lse, sizes, scale, causal, stream: as fa_forward; scale multiplies every
 *     layer's product.
 * bf16 and fp16 only (FA_ERR_DTYPE for fp32); D = 64, 80, 96 or 128
 * (FA_ERR_HEAD_DIM otherwise).  Errors as fa_forward for each layer's
 * (Q_l, K_l) with v, o and lse, plus FA_ERR_NULL_POINTER for a NULL array.
 * The arrays are read during the call only.
 */
int fa_forward_chain(const void* const* q_layers, const void* const* k_layers,
                     int64_t num_layers, const void* v, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                     float scale, int causal, int dtype, void* stream);

/*
 * Key-split ("flash-decode") forward.
 *
 * The same operation as fa_forward, for problems whose query-row blocks alone
 * cannot fill the GPU (few heads, short Nq, decode steps with Nq = 1 against a
 * long Nk).  Two launches on `stream`:
 *  1. the keys of each KV head are cut into num_splits contiguous ranges of
 *     64-key tiles; one workgroup per (b, hk, 128-row block, range) runs the
 *     fused forward over its range and writes the range's normalised partial
 *     output O_s (float32) and LSE_s into the workspace.  The Hq/Hkv query
 *     heads that share a KV head are packed into one row space of
 *     (Hq/Hkv)*Nq rows, so a decode step with Nq = 1 still fills row blocks;
 *  2. fa_merge's kernel combines the num_splits partials of every row into o
 *     (dtype; bf16 for FP8 inputs) and lse with the merge of the
 *     kwkr.cn/news/592482 tutorial,
 *     §2.2 (closing remarks there name flash decode as an extension of the
 *     fused kernel).
 * Results equal fa_forward's up to float32 rounding order.  All conventions of
 * fa_forward apply; in addition:
 *  - 1 <= num_splits <= 1024, else FA_ERR_BAD_SIZE.  Splits beyond the number
 *    of visible 64-key tiles of a row block compute nothing and are merged
 *    away;
 *  - workspace: device memory owned by the caller, 16-byte aligned, at least
 *    fa_split_workspace_bytes(B, Hq, Nq, D, num_splits) bytes
 *    (workspace_bytes states its size), not overlapping any other argument;
 *    else FA_ERR_WORKSPACE (FA_ERR_OVERLAP for an overlap).  Its contents on
 *    entry are ignored and on return are unspecified.  Two calls that run at
 *    the same time need two workspaces;
 *  - (Hq/Hkv)*Nq*D elements must stay below 2^31 bytes, and
 *    B*Hkv*ceil((Hq/Hkv)*Nq/128)*num_splits below 2^31, else FA_ERR_TOO_LARGE.
 * Empty problems (B, Hq or Nq == 0) launch nothing and may pass a NULL
 * workspace.
 */
int fa_forward_split(const void* q, const void* k, const void* v, const void* bias,
                     void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                     float scale, int causal, int dtype,
                     int64_t num_splits, void* workspace, int64_t workspace_bytes,
                     void* stream);

/*
 * fa_forward_split for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The caller passes inputs and outputs only; the float32 partials that
 * fa_forward_split keeps in the caller's workspace go instead to a scratch
 * array of FA_SPLIT_SCRATCH_BYTES that the library holds on each GPU it runs
 * on, from the first call on that GPU until the process ends.  Nothing is
 * allocated, freed or cleared per call (every partial row is written before
 * the merge reads it).
 *
 * Arguments, results and errors are those of fa_forward_split without
 * workspace / workspace_bytes, plus FA_ERR_SCRATCH_LIMIT when
 * fa_split_workspace_bytes(B, Hq, Nq, D, num_splits) exceeds
 * FA_SPLIT_SCRATCH_BYTES (32 MiB: with 16 splits at D = 128, up to 4064
 * query rows B*Hq*Nq); nothing is launched then.  The work runs on
 * the current device, so stream must belong to it; FA_ERR_HIP if the
 * runtime cannot give the scratch array's address there.
 *
 * All calls on one GPU share its scratch array: two calls whose work can
 * overlap on that GPU (different streams without ordering between them, or
 * different host threads) race on it and may return wrong results.  Calls
 * ordered on one stream are safe.
 */
#define FA_SPLIT_SCRATCH_BYTES ((int64_t)32 << 20)
int fa_forward_split_noalloc(const void* q, const void* k, const void* v, const void* bias,
                             void* o, float* lse,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                             int64_t D, float scale, int causal, int dtype, int64_t num_splits,
                             void* stream);

/*
 * Workspace size of fa_forward_split, in bytes, through *bytes:
 * partial O, float32 [num_splits][B*Hq*Nq][D], then partial LSE, float32
 * [num_splits][B*Hq*Nq], from the next 256-byte boundary.  Pure host code.
 * Returns FA_ERR_BAD_SIZE for negative sizes or num_splits outside
 * [1, 1024], FA_ERR_HEAD_DIM for D not 64, 80, 96 or 128, FA_ERR_NULL_POINTER for a
 * NULL bytes.
 */
int fa_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t D,
                             int64_t num_splits, int64_t* bytes);

/*
 * The split count the library suggests for a problem, through *num_splits
 * (pure host code).  It aims for about 512 workgroups (two per compute unit
 * of the 256, the number resident at once) while keeping at least four
 * 64-key tiles per split; 1 when the row blocks alone reach that.  Same size errors as
 * fa_split_workspace_bytes, plus FA_ERR_HEAD_GROUPS.
 */
int fa_split_count(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                   int64_t* num_splits);

/*
 * Merge of normalised partial attention results over disjoint key sets
 * (kwkr.cn/news/592482 tutorial, §2.2, for several states at once): the
 * combine step of a key-split or key-sharded forward.
 *
 *   part_o   float32 [num_parts][rows][D]   partial outputs, each normalised
 *   part_lse float32 [num_parts][rows]      their natural-log LSEs (-inf: the
 *                                           part saw no key of that row)
 *   o        dtype   [rows][D]              out: sum_s w_s O_s / sum_s w_s,
 *                                           w_s = exp(LSE_s - max_s LSE_s)
 *   lse      float32 [rows]                 out: log(sum_s exp(LSE_s))
 * A row with no finite LSE_s (or num_parts == 0) gets O = 0 and LSE = -inf;
 * the O_s of a part with LSE_s = -inf is not read.  D: a multiple of 4 in
 * [4, 65536] (FA_ERR_HEAD_DIM).  part_o and o 16-byte aligned, part_lse and
 * lse 4-byte aligned; o and lse must not overlap each other or the partials.
 * rows == 0 launches nothing.  Enqueued on stream; returns without waiting.
 */
int fa_merge(const float* part_o, const float* part_lse, int64_t num_parts, int64_t rows,
             int64_t D, void* o, float* lse, int dtype, void* stream);

/*
 * Backward of fa_forward: gradients of a loss with respect to q, k and v,
 * given its gradient dout with respect to o.
 *
 * The forward keeps neither S nor P; they are recomputed from q, k (and bias)
 * and the saved per-row lse ("FlashAttention principles and Triton practice",
 * xnwp.cn/news/15505, §2.3 and §4.3; kwkr.cn/news/592482 tutorial, §2.4).  With
 * P = exp(S - LSE) per row:
 *     dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id,  dS = P o (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q,
 * with dK and dV summed over the query heads that share a KV head.  The bias
 * is taken as a constant (its gradient, dS itself, is not produced) and lse as
 * an auxiliary output with no incoming gradient.
 *
 *   q, k, v, bias, scale, causal: exactly as passed to fa_forward;
 *   o, lse:  that call's outputs (o in dtype, lse float32);
 *   dout:    gradient of the loss w.r.t. o, [B, Hq, Nq, D], dtype;
 *   dq:      out, [B, Hq, Nq, D], dtype;
 *   dk, dv:  out, [B, Hkv, Nk, D], dtype;
 *   workspace: device scratch owned by the caller, 16-byte aligned, at least
 *     fa_backward_workspace_bytes(B, Hq, Nq) bytes; holds D_i and LSE_i*log2(e)
 *     (float32) on return.  NULL is allowed when B*Hq*Nq == 0.
 * bf16 and fp16: head sizes 64, 80, 96, 128, and 256 without a logit term
 * (FA_ERR_HEAD_DIM for 256 with one).  Products run on the matrix cores with
 * float32 accumulation; P and dS are rounded to the input type before their
 * products, as P is in the forward.  Two kernels are enqueued on stream (dQ,
 * which also forms the row sums D_i, then dK/dV).  fp32: head sizes 64 and
 * 128 (FA_ERR_HEAD_DIM otherwise), every step in fp32 vector arithmetic with
 * no rounding of P or dS; three kernels (dQ with D_i, then dV, then dK).
 * FP8 has no backward (FA_ERR_DTYPE).  Results are deterministic (no atomics:
 * dQ has its own kernel).  Errors as for fa_forward, plus
 * FA_ERR_NULL_POINTER for a missing dout/dq (rows present) or dk/dv/k/v (keys
 * present), FA_ERR_WORKSPACE, and FA_ERR_OVERLAP if dq, dk, dv or the
 * workspace overlap an input or each other.  With no query rows (B, Hq or
 * Nq == 0) but keys present, dk and dv are set to zero.  The call returns
 * without waiting.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* bias,
                const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                float scale, int causal, int dtype,
                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Backward of fa_forward_window: as fa_backward, with causal = 1 and the same
 * window (window >= 1, FA_ERR_BAD_SIZE otherwise).
 */
int fa_backward_window(const void* q, const void* k, const void* v, const void* bias,
                       const void* o, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                       float scale, int64_t window, int dtype,
                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Backward of fa_forward_chain.  The Block Attention Residual post
 * (iqiancheng.github.io, "v1") trains through its fused chain, with the
 * softmax statistic kept for the backward.  With S = sum over the block's
 * layers l of Q_l K_l^T * scale (the current layer's logits), P = softmax(S)
 * and dS = P o (dP - D_i) as in fa_backward:
 *   dq_layers[l] = scale * dS K_l,
 *   dk_layers[l] = scale * dS^T Q_l  (summed over the query heads of a KV head),
 *   dv           = P^T dO.
 * These are the gradients through this layer's attention only: what the
 * earlier layers receive through their own attention is the caller's to add.
 *   q_layers, k_layers, num_layers, v, scale, causal: as passed to
 *     fa_forward_chain (oldest layer first); o, lse: its outputs;
 *   dout: gradient of the loss w.r.t. o, [B, Hq, Nq, D], dtype;
 *   dq_layers[l]: out, [B, Hq, Nq, D]; dk_layers[l]: out, [B, Hkv, Nk, D];
 *   dv: out, [B, Hkv, Nk, D]; all dtype;
 *   workspace, workspace_bytes: as for fa_backward.
 * bf16 and fp16, D = 64, 80, 96 or 128 (FA_ERR_HEAD_DIM), 1 to 4 layers
 * (FA_ERR_BAD_SIZE); NULL layer arrays give FA_ERR_NULL_POINTER.  Every
 * layer's arguments are checked as fa_backward checks its own, and
 * FA_ERR_OVERLAP is returned if an output overlaps any layer's input or
 * another output.  One layer is fa_backward.  Otherwise two kernels per layer
 * l are enqueued on stream in layer order (dQ of layer l, then dK of layer l,
 * with dV formed alongside layer 0's), each recomputing the summed logits; the
 * call returns without waiting.  Deterministic (no atomics).
 */
int fa_backward_chain(const void* const* q_layers, const void* const* k_layers,
                      int64_t num_layers, const void* v, const void* o, const float* lse,
                      const void* dout, void* const* dq_layers, void* const* dk_layers, void* dv,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                      float scale, int causal, int dtype,
                      void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes of fa_backward through *bytes: float32 [B*Hq*Nq] twice,
 * the second part from the next 256-byte boundary.  Pure host code. */
int fa_backward_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t* bytes);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_status_string(int status);

/* Static version string of the library, e.g. "fa 0.1.0 gfx950". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
