/*
 * fa.h -- C ABI of libfa: fused, tiled exact attention for AMD Instinct MI355X (gfx950).
 *
 * The operation is exact attention, O = softmax(scale * Q K^T [+ causal mask]) V
 * ("How Flash Attention Works: Tiling, Softmax, GPU I/O", section "How Flash
 * Attention Works: The Exact-Attention Idea"; the same formula with scale =
 * 1/sqrt(d_k) in "attn-flash-equivalence", section "Standard attention I/O is
 * the bottleneck").  The forward pass never writes the N x N score matrix to
 * device memory: it keeps a running row max and normaliser per query row and
 * rescales the partial output as key/value tiles stream past ("How Flash
 * Attention Works", sections "Tiling Q, K, and V for Fast On-Chip Memory" and
 * "Online Softmax Without the Full Score Matrix").  Its only side output is one
 * log-sum-exp per row, from which the backward pass recomputes the score tiles
 * (same page, section "The Backward Pass: Recomputation Instead of Stored
 * Activations").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors q, k, v, o, dout, dq, dk, dv are device pointers to contiguous
 *    [B, H, N, d] arrays, row-major with d fastest, all of one element type
 *    (fa_dtype).  Offsets are computed in 64-bit.
 *  - lse is a device pointer to a contiguous fp32 [B, H, N] array holding
 *    LSE_i = ln sum_j exp(scale * q_i . k_j) over the keys row i may see.
 *  - Causal mask: query i sees key j iff j <= i (causal = 1); causal = 0 sees all.
 *  - Supported: d in {64, 128}; N >= 1; B, H >= 1; B*H*N < 2^31; scale finite.
 *    Anything else returns an error; there is no slower fallback path.
 *  - Every pointer must be 16-byte aligned.  Outputs must not alias inputs.
 *  - The caller owns every buffer and keeps it alive until the work queued on
 *    `stream` has finished.  The library allocates, frees and caches no device
 *    memory and holds no mutable global state; calls are reentrant.  (The one
 *    exception is fa_bwd_static, which keeps its row sums in a fixed device
 *    array instead of a caller's workspace.)
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is queued asynchronously; the library never synchronises.
 *  - Return value: FA_OK or a negative fa_status.  Arguments are validated
 *    before any HIP call, so an invalid call queues nothing.  A launch failure
 *    is reported as FA_ERR_HIP; faults during execution surface at the caller's
 *    next synchronisation.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* NULL/misaligned pointer, bad size, non-finite scale, causal not 0/1 */
  FA_ERR_UNSUPPORTED = -2, /* a head dimension or dtype this library has no kernel for */
  FA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_HIP = -4,         /* the HIP runtime refused a launch (no device, bad stream, ...) */
  FA_ERR_TOO_LARGE = -5    /* fa_bwd_static only: B * H * N above FA_STATIC_SCRATCH_ROWS */
} fa_status;

/*
 * Forward pass.  Writes o = softmax(scale * q k^T [+ mask]) v and, if lse is
 * not NULL, the per-row log-sum-exp.  Query blocks stream all (or, causal,
 * all earlier) key/value tiles through on-chip memory; only o and lse reach
 * device memory ("How Flash Attention Works", section "Kernel Fusion and
 * Incremental Output Accumulation").
 *   q, k, v : [B,H,N,d] inputs, dtype `dtype`
 *   o       : [B,H,N,d] output, dtype `dtype` (rounded to nearest even)
 *   lse     : [B,H,N] fp32 output, or NULL to skip it (inference)
 * 16-bit dtypes multiply in the matrix cores with fp32 accumulation; the
 * softmax weights are rounded to `dtype` before they multiply v.  FA_F32
 * computes in fp32 throughout.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal,
           fa_dtype dtype, void *stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (fp32 per-row
 * D_i = sum_c dout_ic * o_ic).  Returns 0 for sizes fa_bwd would reject.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype);

/*
 * Backward pass: gradients of L = sum(dout * o) with respect to q, k and v.
 * o and lse must come from fa_fwd with the same q, k, v, scale and causal
 * (a contract, not checked).  Score tiles are recomputed from q, k and lse,
 * tile by tile; no probability matrix is read or written ("How Flash Attention
 * Works", section "The Backward Pass: Recomputation Instead of Stored
 * Activations").  The gradient formulas are the chain rule on the forward
 * definition:  dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
 * dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *   dq, dk, dv : [B,H,N,d] outputs, dtype `dtype`
 *   workspace  : device buffer of at least fa_bwd_workspace_bytes() bytes,
 *                contents on entry ignored, clobbered on exit
 * The result is deterministic: no atomics, fixed summation order.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const void *dout, const float *lse,
           void *dq, void *dk, void *dv,
           void *workspace, size_t workspace_bytes,
           int B, int H, int N, int d, float scale, int causal,
           fa_dtype dtype, void *stream);

/*
 * The stages of the backward pass, for callers that schedule them themselves
 * (for instance dK/dV and dQ on two streams once the row sums are done, or
 * timing each stage).  fa_bwd(...) is exactly
 *     fa_bwd_dq_rowsum(...); fa_bwd_dkdv(...);
 * on one stream: the dQ stage forms the row sums D on the way (it holds each
 * query's dout row already, so D costs one read of o and no launch of its
 * own) and leaves them in the workspace for the dK/dV stage.  The same
 * result, up to the summation order of D, comes from
 *     fa_bwd_rowsum(...); then fa_bwd_dkdv(...) and fa_bwd_dq(...) in any order.
 * Arguments mean what they mean for fa_bwd; each stage validates the
 * arguments it uses.  The workspace carries D between stages, so it must not
 * be reused in between.
 *   fa_bwd_rowsum    : workspace <- D_i = sum_c dout_ic * o_ic (fp32)
 *   fa_bwd_dq_rowsum : dq, and workspace <- D (reads q, k, v, o, dout, lse)
 *   fa_bwd_dkdv      : dk, dv   (reads q, k, v, dout, lse, workspace)
 *   fa_bwd_dq        : dq       (reads q, k, v, dout, lse, workspace)
 */
int fa_bwd_rowsum(const void *o, const void *dout, void *workspace, size_t workspace_bytes,
                  int B, int H, int N, int d, fa_dtype dtype, void *stream);
int fa_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout, const float *lse,
                const void *workspace, size_t workspace_bytes, void *dk, void *dv,
                int B, int H, int N, int d, float scale, int causal, fa_dtype dtype, void *stream);
int fa_bwd_dq(const void *q, const void *k, const void *v, const void *dout, const float *lse,
              const void *workspace, size_t workspace_bytes, void *dq,
              int B, int H, int N, int d, float scale, int causal, fa_dtype dtype, void *stream);
int fa_bwd_dq_rowsum(const void *q, const void *k, const void *v, const void *o, const void *dout,
                     const float *lse, void *workspace, size_t workspace_bytes, void *dq,
                     int B, int H, int N, int d, float scale, int causal, fa_dtype dtype, void *stream);

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments, results and validation without the workspace, whose row sums D
 * live in a fixed device array of FA_STATIC_SCRATCH_ROWS fp32 values (16 MiB)
 * instead.  Every GPU the library runs on holds its own copy of that array
 * from its first fa_bwd_static call until the process ends; the call itself
 * allocates nothing.  Its address on a device is looked up once, on the
 * first call whose `stream` runs on that device.
 *   B * H * N above FA_STATIC_SCRATCH_ROWS returns FA_ERR_TOO_LARGE.
 * All fa_bwd_static calls on one device share the array: calls that overlap
 * in time on one GPU (concurrent streams) race and give wrong gradients;
 * order them on one stream, or use fa_bwd with a workspace each.  Nothing
 * needs clearing between calls: each call writes every row sum it reads.
 */
#define FA_STATIC_SCRATCH_ROWS (1 << 22)
int fa_bwd_static(const void *q, const void *k, const void *v, const void *o,
                  const void *dout, const float *lse,
                  void *dq, void *dk, void *dv,
                  int B, int H, int N, int d, float scale, int causal,
                  fa_dtype dtype, void *stream);

/*
 * Unequal query and key counts, and padded batches.  The pages tie the causal
 * mask to autoregressive decoding and apply causal masking and padding tile by
 * tile ("How Flash Attention Works", sections "How Flash Attention Works:
 * The Exact-Attention Idea" and "Tiling Q, K, and V for Fast On-Chip
 * Memory"); they fix neither the causal alignment for unequal counts nor the
 * output of padding rows, and these entry points take the readings below.
 *   q, o, dout, dq : [B,H,Nq,d];  k, v, dk, dv : [B,H,Nk,d];  lse : fp32 [B,H,Nq]
 *   seqlens_q, seqlens_k : NULL, or device pointers to int32[B] (4-byte
 *       aligned): sequence b has lq_b = seqlens_q[b] real queries and
 *       lk_b = seqlens_k[b] real keys; NULL means Nq (Nk) for every b.
 *       Values are read on the device and clamped into [0, Nq] / [0, Nk],
 *       so an out-of-range length cannot make a kernel read or write outside
 *       the arrays.  They must stay unchanged until the queued work is done.
 *   Causal mask, bottom-right aligned: the lq_b queries are the last lq_b
 *       positions of the lk_b-key sequence, so query i sees key j iff
 *       j <= i + (lk_b - lq_b).  With Nq = Nk and no lengths this is fa_fwd /
 *       fa_bwd exactly; with one query (decoding against a key cache) the
 *       query sees every key.
 *   Rows past a length (padding), and rows that see no key (causal with
 *       lq_b > lk_b, or lk_b = 0), get o = 0 and lse = -inf; they contribute
 *       nothing to any gradient, and dq rows past lq_b and dk / dv rows past
 *       lk_b are written as 0.
 * Other conventions, validation and errors are those of fa_fwd / fa_bwd, with
 * Nq >= 1, Nk >= 1, B*H*Nq < 2^31 and B*H*Nk < 2^31.  fa_bwd_kv's workspace is
 * fa_bwd_workspace_bytes(B, H, Nq, d, dtype); its o and lse must come from
 * fa_fwd_kv with the same arguments.
 */
int fa_fwd_kv(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int Nq, int Nk, int d,
              const int *seqlens_q, const int *seqlens_k,
              float scale, int causal, fa_dtype dtype, void *stream);
int fa_bwd_kv(const void *q, const void *k, const void *v, const void *o,
              const void *dout, const float *lse,
              void *dq, void *dk, void *dv,
              void *workspace, size_t workspace_bytes,
              int B, int H, int Nq, int Nk, int d,
              const int *seqlens_q, const int *seqlens_k,
              float scale, int causal, fa_dtype dtype, void *stream);

/*
 * Split-key forward, for few query rows against many keys (decoding against a
 * key cache): with B * H * ceil(Nq / 128) workgroups only, most compute units
 * would idle.  The key range is cut into num_splits pieces of whole 64-key
 * tiles; each (batch, head, 128-query block, piece) runs the fa_fwd_kv
 * algorithm on its keys and writes an fp32 partial output and log-sum-exp into
 * `workspace`, and a merge pass combines them with the same rescale the online
 * softmax applies tile by tile ("How Flash Attention Works", section "Online
 * Softmax Without the Full Score Matrix"):
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * With Nq = 1 (one query row per head, plain decoding) the pieces run a
 * streaming kernel instead of the tiled one: no LDS staging, every wave reads
 * whole consecutive key rows straight into registers.
 * Arguments, layout, lengths and causal alignment are those of fa_fwd_kv; the
 * result equals fa_fwd_kv's up to rounding order, and fa_bwd_kv accepts it.
 *   num_splits : 1 .. 256; 1 is fa_fwd_kv itself (workspace unused, may be
 *                NULL).  fa_fwd_kv_split_hint suggests a value.
 *   workspace  : device buffer of at least fa_fwd_kv_split_workspace_bytes()
 *                bytes, 16-byte aligned, not overlapping any other argument;
 *                contents on entry ignored, clobbered on exit.
 * 16-bit dtypes only: FA_F32 with num_splits > 1 returns FA_ERR_UNSUPPORTED.
 * B * H * ceil(Nq / 128) * num_splits must stay below 2^31 (the launch grid).
 */
size_t fa_fwd_kv_split_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);
int fa_fwd_kv_split_hint(int B, int H, int Nq, int Nk, int d);
int fa_fwd_kv_split(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int Nq, int Nk, int d,
                    const int *seqlens_q, const int *seqlens_k,
                    float scale, int causal, int num_splits,
                    void *workspace, size_t workspace_bytes,
                    fa_dtype dtype, void *stream);

/*
 * Block-sparse attention.  The pages name a block-sparse extension studied
 * beside the dense algorithm as a separate configuration ("FlashAttention"
 * glossary entry, its definition) and fix no mask format; this one is:
 *   block_mask : device pointer (not NULL; no alignment needed) to uint8
 *                [B, H, nb, nb], nb = ceil(N / FA_SPARSE_BLOCK).  Entry
 *                (b, h, i, j) = 0 removes the scores of query rows
 *                [128 i, 128 i + 128) against keys [128 j, 128 j + 128);
 *                any other value keeps them.  The causal mask, if set,
 *                applies on top.  Removed tiles are skipped: not loaded, no
 *                matrix or softmax work.  The mask must not change until the
 *                queued work is done.
 * Rows that see no key get o = 0 and lse = -inf and contribute nothing to any
 * gradient.  N may be at most 524288 (4096 blocks); larger N returns
 * FA_ERR_UNSUPPORTED.  Other arguments, validation and errors are those of
 * fa_fwd / fa_bwd; fa_bwd_sparse needs o and lse from fa_fwd_sparse with the
 * same mask.
 */
#define FA_SPARSE_BLOCK 128
int fa_fwd_sparse(const void *q, const void *k, const void *v, void *o, float *lse,
                  int B, int H, int N, int d, const unsigned char *block_mask,
                  float scale, int causal, fa_dtype dtype, void *stream);
int fa_bwd_sparse(const void *q, const void *k, const void *v, const void *o,
                  const void *dout, const float *lse,
                  void *dq, void *dk, void *dv,
                  void *workspace, size_t workspace_bytes,
                  int B, int H, int N, int d, const unsigned char *block_mask,
                  float scale, int causal, fa_dtype dtype, void *stream);

/*
 * Attention dropout inside the fused kernel.  The pages count dropout among
 * the steps an unfused pipeline runs as separate kernels and put it inside the
 * one fused kernel ("How Flash Attention Works", sections "Why Standard
 * Attention Becomes a GPU Memory I/O Bottleneck" and "Kernel Fusion and
 * Incremental Output Accumulation"); they fix no random number generator and
 * no mask layout.  These entry points take:
 *   O = (P o Z) V with P = softmax(scale * q k^T [+ causal]) and
 *   Z_ij = keep_ij / (1 - dropout_p).  lse is that of P (before dropout), so
 *   fa_bwd_dropout recomputes P exactly as fa_bwd does.
 *   keep_ij: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 *   Numbers: As Easy as 1, 2, 3", SC 2011) with key (seed mod 2^32,
 *   seed >> 32) and counter (j >> 2, i, b * H + h, offset) yields four 32-bit
 *   words; word (j & 3) decides key j of query row i, kept iff
 *   word >= floor(dropout_p * 2^32).  Nothing is stored: the backward pass
 *   regenerates the same words.  Calls with the same (seed, offset) draw the
 *   same mask; advance offset (or change seed) for a fresh one.
 *   dropout_p : in [0, 1), else FA_ERR_INVALID_ARG (NaN included).  0 runs
 *               the fa_fwd / fa_bwd kernels and gives their results.
 * Other arguments, validation and errors are those of fa_fwd / fa_bwd;
 * fa_bwd_dropout needs o and lse from fa_fwd_dropout with the same arguments,
 * and computes the gradients of sum(dout * O) for that fixed mask:
 *   dV = (P o Z)^T dO,  dS = P o (Z o (dO V^T) - D),  D_i = sum_c dO_ic O_ic,
 *   dQ = scale dS K,  dK = scale dS^T Q.
 */
int fa_fwd_dropout(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed, unsigned int offset,
                   fa_dtype dtype, void *stream);
int fa_bwd_dropout(const void *q, const void *k, const void *v, const void *o,
                   const void *dout, const float *lse,
                   void *dq, void *dk, void *dv,
                   void *workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed, unsigned int offset,
                   fa_dtype dtype, void *stream);

/*
 * Forward pass on 8-bit floating-point inputs.  The pages say FlashAttention 3
 * adds lower-precision paths where the hardware has them ("How Flash Attention
 * Works", section "FlashAttention 1 vs 2 vs 3") and fix no format, scaling or
 * output type; this entry point takes:
 *   q, k, v : device pointers to uint8 [B,H,N,d] OCP E4M3 codes ("OCP 8-bit
 *             Floating Point Specification (OFP8)", revision 1.0: sign, 4
 *             exponent bits with bias 7, 3 mantissa bits, no infinities,
 *             S.1111.111 = NaN), 16-byte aligned
 *   descale_q, descale_k, descale_v : one real factor per tensor; the
 *             attention inputs are descale_x * E4M3(x)
 *   o       : bf16 [B,H,N,d] output, o = softmax(scale * Q K^T [+ causal]) V
 *             on the dequantised Q, K, V (rounded to nearest even)
 *   lse     : fp32 [B,H,N] log-sum-exp of the dequantised scaled scores, or NULL
 * Q K^T and P V run on the 8-bit matrix cores with fp32 accumulation; the
 * softmax weights are rounded to E4M3 (round to nearest even, relative error
 * at most 2^-4 above 2^-6) before they multiply v, which bounds the error of
 * each output by about 2^-4 * sum_j P_ij |v_jc| beyond the bf16 rounding.
 * NaN codes propagate.  d in {64, 128}; N >= 1; B*H*N < 2^31; scale and the
 * factors finite, scale * descale_q * descale_k finite in fp32; causal in
 * {0, 1}.  Outputs must not overlap inputs.  Errors and stream semantics are
 * those of fa_fwd.  There is no 8-bit backward pass.
 */
int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int H, int N, int d, float scale, int causal,
               float descale_q, float descale_k, float descale_v, void *stream);

/*
 * The 8-bit forward with the input format chosen by the caller; fa_fwd_fp8 is
 * this call with fmt = FA_FP8_E4M3.  With FA_FP8_E5M2, q, k and v hold OCP
 * E5M2 codes (same specification: sign, 5 exponent bits with bias 15, 2
 * mantissa bits, S.11111.00 = infinity, S.11111.mm with mm != 0 = NaN;
 * largest finite magnitude 57344), the attention inputs are descale_x *
 * E5M2(x), and everything else -- arguments, layout, output type, the E4M3
 * rounding of the softmax weights and its error bound, errors -- is as for
 * fa_fwd_fp8.  The codes must be finite: the outputs of a row whose scores or
 * values meet an infinity or NaN are unspecified.  fmt outside the enum:
 * FA_ERR_INVALID_ARG.
 */
typedef enum { FA_FP8_E4M3 = 0, FA_FP8_E5M2 = 1 } fa_fp8_format;

int fa_fwd_fp8_fmt(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int N, int d, float scale, int causal,
                   float descale_q, float descale_k, float descale_v,
                   fa_fp8_format fmt, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *fa_status_string(int status);

/* Library version as an integer: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
