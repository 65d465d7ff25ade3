/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * The operations are the FlashAttention-2 forward pass (fa_fwd; fa_fwd_kv
 * for separate query and key lengths; fa_fwd_decode, the same split over the
 * keys for a few queries) and its gradients (fa_bwd).  What the forward pass computes is
 * exact attention (FlashAttention-2 abstract, searcharxiv abstract page,
 * "Abstract": attention computed exactly, in memory linear in the sequence
 * length): for every batch b, head h and query row i
 *
 *     s_ij  = scale * <q_i, k_j>                 for keys j in A(i)
 *     LSE_i = ln sum_{j in A(i)} exp(s_ij)         (natural log)
 *     o_i   = sum_{j in A(i)} exp(s_ij - LSE_i) v_j
 *
 * with A(i) = {0..S-1}, or {0..i} when causal (query and key lengths are
 * equal, so key j is kept iff j <= i).  It is computed tile by tile with an
 * online softmax (IPLEX blog "FlashAttention-2: making long-context attention
 * run efficiently on GPUs", section "Tiling preserves the attention
 * calculation"), so the S x S score matrix never reaches device memory, and the
 * result equals the definition up to floating-point rounding.  The per-row
 * logsumexp is an output of this library; the pages do not mention it.
 *
 * All entry points are plain C: no HIP or torch types appear here.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h> /* size_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o.  Accumulation is always fp32. */
typedef enum { FA_DTYPE_FP16 = 0, FA_DTYPE_BF16 = 1 } fa_dtype;

/* Status codes returned by the entry points (0 = success, negative = error). */
enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a pointer argument is NULL (non-empty problem)       */
  FA_ERR_SHAPE = -2,     /* B, H, S or Sk negative, or causal not 0/1            */
  FA_ERR_HEAD_DIM = -3,  /* d not 64, 128, 192 or 256 (every entry point)       */
  FA_ERR_DTYPE = -4,     /* dtype is not an fa_dtype value                       */
  FA_ERR_SCALE = -5,     /* scale is NaN, infinite or negative                   */
  FA_ERR_ALIGN = -6,     /* a tensor (or a stride) not 16-byte aligned, or lse/delta not 4-byte */
  FA_ERR_ALIAS = -7,     /* an output overlaps an input or another output        */
  FA_ERR_TOO_LARGE = -8, /* S*d or Sk*d >= 2^30, or the grid exceeds 2^31-1      */
  FA_ERR_HIP = -9,       /* the HIP runtime rejected the launch (see below)      */
  FA_ERR_WORKSPACE = -10, /* fa_fwd_decode: workspace missing, short or unaligned */
  FA_ERR_STRIDE = -11,   /* strided entry points: a stride negative, a row stride
                            below d, or the output's strides not one-to-one   */
  FA_ERR_SCRATCH = -12   /* fa_fwd_decode_noalloc: the shapes need more than
                            FA_DECODE_NOALLOC_MAX_BYTES of scratch            */
};

/*
 * fa_fwd -- enqueue the exact-attention forward pass on `stream`.
 *
 * Arguments (all device pointers, caller-owned):
 *   q, k, v  [B][H][S][d] dense row-major tensors of `dtype` (fp16 or bf16).
 *   o        [B][H][S][d] dense row-major output of `dtype` (same as inputs).
 *   lse      [B][H][S]    dense fp32 output: LSE_i, natural log, of the scaled
 *                         and masked scores.
 *   B, H, S  batch, heads, sequence length (query length = key length).
 *            B*H*S == 0 is an empty problem: nothing is read or written and
 *            FA_OK is returned (pointers may then be NULL).
 *   d        head dimension: 64 or 128 (the pages' benchmark head sizes), or
 *            192 or 256 (wide heads: four wavefronts of 32 query rows per
 *            work-group, one per SIMD, instead of eight).
 *   causal   0 = no mask; 1 = keep key j for query i iff j <= i.
 *   scale    multiplies every score before the softmax; must be finite and
 *            >= 0 (0 gives uniform weights).  Callers normally pass
 *            1/sqrt(d) rounded to fp32.
 *   dtype    an fa_dtype value.
 *   stream   a hipStream_t passed as void*; NULL is the default stream.
 *
 * Behaviour: arguments are validated on the host before any HIP call; on a
 * validation error nothing is enqueued.  The kernels are enqueued
 * asynchronously and the call returns without synchronising.  The library
 * allocates no device or host memory and keeps no state between calls, so it
 * is reentrant and thread-safe.  Results are deterministic: each output element
 * is written by exactly one thread, with no atomics.  On any error o and lse
 * are left unspecified.  No exception or abort crosses this boundary.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int S, int d, int causal, float scale, int dtype,
           void* stream);

/*
 * fa_fwd_kv -- fa_fwd with separate query and key lengths.
 *
 * The pages set the processing of a whole prompt apart from generating one
 * token at a time, and say the two are bound differently (IPLEX blog
 * "FlashAttention-2: making long-context attention run efficiently on GPUs",
 * section "Document the implementation difference").  In generation the Sq
 * new queries are the last Sq positions of a sequence whose first Sk
 * positions carry the keys; the pages give no mask for this shape, and this
 * library takes the end-aligned reading:
 *
 *     A(i) = {0..Sk-1}                       when causal = 0
 *     A(i) = {j : j <= i + Sk - Sq}          when causal = 1
 *
 * so Sq = Sk is fa_fwd's square mask and a single query sees every key.  A
 * row whose A(i) is empty (causal, Sq > Sk, rows i < Sq - Sk; or Sk = 0)
 * gets o_i = 0 and LSE_i = -inf.
 *
 * Arguments: as for fa_fwd, except
 *   q, o     [B][H][Sq][d];   lse [B][H][Sq];
 *   k, v     [B][H][Sk][d]    (may be NULL when Sk == 0: never read);
 *   Sq, Sk   query and key lengths, each >= 0 with Sq*d, Sk*d < 2^30.
 * Behaviour, ownership and errors: as for fa_fwd.  fa_fwd_kv(..., S, S, ...)
 * gives bitwise the same results as fa_fwd(..., S, ...).
 */
int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Sq, int Sk, int d, int causal, float scale,
              int dtype, void* stream);

/*
 * fa_fwd_strided -- fa_fwd_kv on tensors with arbitrary batch, head and row
 * strides (e.g. [B][S][H][d] "BSHD" tensors, or a slice of a larger key/value
 * cache), so callers need not copy into the dense layout.
 *
 * strides: host array of 12 element strides, read during the call:
 *     { q_batch, q_head, q_row,  k_batch, k_head, k_row,
 *       v_batch, v_head, v_row,  o_batch, o_head, o_row }
 * element (b, h, i, c) of q is at q + q_batch*b + q_head*h + q_row*i + c (in
 * elements of `dtype`); d is always contiguous.  lse stays dense [B][H][Sq].
 * Requirements (checked before any HIP call):
 *   - strides >= 0 and multiples of 8 elements (16-byte rows), else
 *     FA_ERR_STRIDE / FA_ERR_ALIGN;
 *   - every row stride >= d, also for a single row (FA_ERR_STRIDE);
 *   - o's strides map distinct positions to distinct elements
 *     (FA_ERR_STRIDE);
 *   - (rows + 512) * row_stride * 2 + 2d < 2^32 for every tensor
 *     (32-bit offsets within a head, FA_ERR_TOO_LARGE);
 *   - o and lse must not overlap the byte range any input spans
 *     (FA_ERR_ALIAS; the inputs may overlap each other).
 * Results are bitwise those of fa_fwd_kv on the same values in the dense
 * layout.  Everything else as fa_fwd_kv.
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int H, int Sq, int Sk, int d,
                   const long long* strides, int causal, float scale,
                   int dtype, void* stream);

/*
 * fa_fwd_decode -- fa_fwd_kv for a few queries over many keys (token-by-token
 * decoding), split over the keys.
 *
 * Same operation, arguments and results as fa_fwd_kv (end-aligned causal
 * mask; rows without keys give o = 0, LSE = -inf), computed another way.
 * The pages set decoding apart from prompt processing because its
 * bottleneck differs (IPLEX blog "FlashAttention-2: making long-context
 * attention run efficiently on GPUs", section "Document the implementation
 * difference"): with Sq small there are about Sq flops per byte of K and V,
 * so the pass is bound by HBM bandwidth and needs many more work-groups than
 * B*H query blocks give.  fa_fwd_decode therefore splits each head's keys
 * into disjoint ranges, computes a partial output and partial LSE per range,
 * and merges them exactly:
 *     LSE_i = ln sum_r exp(LSE_ir),   o_i = sum_r exp(LSE_ir - LSE_i) o_ir.
 * Any Sq is accepted; it pays for Sq up to a few dozen rows, fa_fwd_kv for
 * longer query blocks.  Results match fa_fwd_kv to rounding, not bitwise.
 *
 * Extra arguments:
 *   workspace        device memory for the partial results, caller-owned,
 *                    16-byte aligned, not overlapping any tensor, at least
 *                    fa_fwd_decode_workspace_size(B, H, Sq, Sk, d) bytes.
 *                    Its contents on entry do not matter and on return are
 *                    unspecified; calls that share a workspace must be
 *                    ordered on one stream.
 *   workspace_bytes  its size in bytes.
 * Errors: as fa_fwd_kv, plus FA_ERR_WORKSPACE (checked after the shape
 * checks) and FA_ERR_ALIAS when the workspace overlaps a tensor.  The two
 * kernels (split pass, then merge) are enqueued on `stream`; no memory is
 * allocated and the results are deterministic.
 */
int fa_fwd_decode(const void* q, const void* k, const void* v, void* o,
                  float* lse, int B, int H, int Sq, int Sk, int d, int causal,
                  float scale, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Workspace bytes fa_fwd_decode needs for these shapes (a pure function of
 * its arguments: the key split is chosen from the shapes alone).  Returns 0
 * when B*H*Sq == 0 or the arguments are invalid (d not 64, 128, 192 or 256,
 * a negative size); then fa_fwd_decode needs no workspace or fails validation.
 */
size_t fa_fwd_decode_workspace_size(int B, int H, int Sq, int Sk, int d);

/*
 * fa_fwd_decode_noalloc -- fa_fwd_decode for callers that cannot allocate
 * (code under stream or graph capture, tight serving loops, harnesses that
 * forbid allocation): the same operation, validation and kernels, but the
 * partial results live in a library-owned device array of
 * FA_DECODE_NOALLOC_MAX_BYTES, so the caller passes only q, k, v, o and lse
 * (dense layout, as for fa_fwd_decode) and no workspace.
 *
 * Limit: shapes whose fa_fwd_decode_workspace_size(B, H, Sq, Sk, d) exceeds
 * FA_DECODE_NOALLOC_MAX_BYTES return FA_ERR_SCRATCH before anything is
 * enqueued (16 MiB covers, e.g., every single-token step with B*H*d up to
 * about 4M).
 *
 * Memory: each device the library runs this on holds its own copy of the
 * array until the process ends.  The first call on a device looks up that
 * copy's address (hipGetSymbolAddress, with the stream's device current);
 * no call allocates or frees anything.  Nothing in the array needs clearing:
 * every partial the merge reads is written first by the same call.
 *
 * Concurrency: all calls on one device share that device's array.  Calls
 * ordered on one stream are fine; calls that may overlap on one device
 * (different streams, different threads without ordering) race on it and
 * give wrong results.
 *
 * Arguments and other errors: as fa_fwd_decode without the workspace
 * arguments.  Results are bitwise those of fa_fwd_decode on the same inputs.
 */
#define FA_DECODE_NOALLOC_MAX_BYTES (16u << 20)
int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                          float* lse, int B, int H, int Sq, int Sk, int d,
                          int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_decode_strided -- fa_fwd_decode on strided tensors (strides and
 * their requirements as for fa_fwd_strided), e.g. the first Sk rows of a
 * [B][S_max][H][d] key/value cache.  Results are bitwise those of
 * fa_fwd_decode on the same values in the dense layout; the workspace size
 * does not depend on the strides.
 */
int fa_fwd_decode_strided(const void* q, const void* k, const void* v, void* o,
                          float* lse, int B, int H, int Sq, int Sk, int d,
                          const long long* strides, int causal, float scale,
                          int dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * fa_bwd -- enqueue the gradients of the exact-attention forward pass.
 *
 * The pages state that the method trains GPT-style models (searcharxiv
 * abstract page, "Abstract") and that its gradients match the plain
 * calculation up to rounding (IPLEX blog, section "Tiling preserves the
 * attention calculation"); they give no algorithm for them.  With dO the
 * gradient of a scalar loss with respect to o, this computes the gradients of
 * that loss with respect to q, k and v, per (b, h):
 *
 *     P_ij  = exp(s_ij - LSE_i) for j in A(i), 0 otherwise
 *     dv    = P^T dO
 *     D_i   = sum_c dO_ic o_ic
 *     dS_ij = P_ij (dO_i . v_j - D_i)
 *     dq    = scale * dS k,      dk = scale * dS^T q
 *
 * recomputing P tile by tile from q, k and the forward pass's LSE, so no
 * S x S matrix reaches device memory.
 *
 * Arguments (all device pointers, caller-owned):
 *   q, k, v     the forward pass's inputs, [B][H][S][d] of `dtype`.
 *   o, lse      the forward pass's outputs for exactly these inputs, causal
 *               flag and scale (o [B][H][S][d] of `dtype`, lse [B][H][S] fp32).
 *   dout        dO, [B][H][S][d] of `dtype`.
 *   dq, dk, dv  [B][H][S][d] outputs of `dtype`.
 *   delta       [B][H][S] fp32 buffer the call writes D_i into (scratch that
 *               the caller provides, so the library allocates nothing; its
 *               contents on return are D_i).
 *   B, H, S, d, causal, scale, dtype, stream: as for fa_fwd (d = 64, 128,
 *               192 or 256).
 *
 * Behaviour: as fa_fwd (host validation before any HIP call, asynchronous,
 * no allocation, no state, deterministic: no atomics).  Two kernels are
 * enqueued in order on `stream`: the first writes delta and dq, the second
 * reads delta and writes dk and dv.  dq, dk, dv and delta must not overlap
 * any input or each other (FA_ERR_ALIAS).  On any error the outputs are left
 * unspecified.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int S, int d, int causal, float scale, int dtype,
           void* stream);

/*
 * fa_bwd_kv -- fa_bwd with separate query and key lengths: the gradients of
 * fa_fwd_kv (same end-aligned causal mask: key j is kept for query row i iff
 * j <= i + Sk - Sq).
 *
 *   q, o, dout, dq  [B][H][Sq][d];  lse, delta  [B][H][Sq] fp32;
 *   k, v, dk, dv    [B][H][Sk][d].
 *
 * A query row that keeps no key (causal with Sq > Sk, rows i < Sq - Sk; its
 * forward output is the constant 0 and its LSE -inf) gets dq = 0 and adds
 * nothing to dk and dv.  With Sq = 0 the call writes dk = dv = 0 and the
 * query-side pointers may be NULL; with Sk = 0 it writes dq = 0 and delta
 * and the key-side pointers may be NULL; B*H == 0 or Sq = Sk = 0 is a no-op.
 * With Sq = Sk the results are bitwise those of fa_bwd.  Errors and
 * behaviour otherwise as fa_bwd.
 */
int fa_bwd_kv(const void* q, const void* k, const void* v, const void* o,
              const float* lse, const void* dout, void* dq, void* dk, void* dv,
              float* delta, int B, int H, int Sq, int Sk, int d, int causal,
              float scale, int dtype, void* stream);

/*
 * fa_bwd_strided -- fa_bwd_kv on strided tensors, e.g. q, k, v, o, dout and
 * the gradients in the [B][S][H][d] layout, or slices of a packed QKV buffer.
 *
 *   strides  host array of 24 element strides: batch, head and row stride of
 *            q, k, v, o, dout, dq, dk, dv in that order (each tensor's
 *            element (b, h, i, c) is at ptr[b*sb + h*sh + i*rs + c]).  Each
 *            tensor must satisfy fa_fwd_strided's requirements (strides >= 0
 *            and multiples of 8, rs >= d, row offsets within 32 bits); dq, dk
 *            and dv must also be one-to-one (FA_ERR_STRIDE), and the byte
 *            ranges they span must not overlap an input, lse, delta or each
 *            other (FA_ERR_ALIAS).  lse and delta stay dense [B][H][Sq].
 * Results are bitwise those of fa_bwd_kv on the same values in the dense
 * layout.  Errors and behaviour otherwise as fa_bwd_kv.
 */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk,
                   void* dv, float* delta, int B, int H, int Sq, int Sk, int d,
                   const long long* strides, int causal, float scale,
                   int dtype, void* stream);

/* Static English text for a status code; never NULL. */
const char* fa_status_string(int status);

/* Text of the HIP error behind the calling thread's last FA_ERR_HIP; "" if none. */
const char* fa_last_hip_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
