/*
 * osattn — fused online-softmax scaled-dot-product attention for AMD MI355X (gfx950).
 *
 * C ABI.  Plain device pointers and integer sizes; no C++ or framework types.
 * Every entry point only enqueues work on the given HIP stream and returns; it
 * never synchronises and never allocates device memory.  All but one keep no
 * global state, so calls are re-entrant; the exception, attn_bwd_noalloc, keeps its
 * workspace in a fixed device array per GPU (see its comment).  Faults inside a
 * kernel surface at the caller's next synchronisation on that stream.
 *
 * Operation (FlashAttention-2 page, "Standard Attention" and the FA2 inner loop;
 * ml-notes page, why scores are divided by sqrt(d)):
 *
 *     S   = scale * Q K^T,        S_ij = -inf for j > i when causal
 *     O   = softmax_rows(S) V
 *     LSE = ln sum_j exp(S_ij)    per query row
 *
 * computed tile by tile with a running row max and running denominator so that
 * no N x N matrix is ever written to memory.  The backward pass (softmax-backward
 * page, "Backpropagating Through Softmax": the row JVP P*(dP - <P, dP>)) rebuilds
 * P from LSE and forms
 *
 *     D  = rowsum(dO * O),  dS = P * (dO V^T - D),
 *     dV = P^T dO,  dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 * Layouts (all row-major and contiguous, element type given by `dtype`):
 *     q, o, dO, dq : [B][H][N][d]
 *     k, v, dk, dv : [B][Hkv][N][d]
 *     lse          : [B][H][N]  float32, natural-log units
 * Query head h reads key/value head h / (H / Hkv) (grouped-query attention,
 * contiguous groups); dk and dv of a key/value head sum over its query heads.
 * The causal mask is square and top-left aligned: query i sees keys 0..i.
 *
 * Supported: dtype in {ATTN_F32, ATTN_F16, ATTN_BF16}; d in {64, 128}; any
 * N >= 1; H a multiple of Hkv.  Inputs and outputs use `dtype`; arithmetic
 * accumulates in float32; softmax statistics are float32.  Outputs are rounded
 * to nearest even.
 */
#ifndef OSATTN_H
#define OSATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 } attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,      /* a required pointer is NULL                                */
  ATTN_ERR_SHAPE = -2,     /* B, H, Hkv or N < 1, or a tensor exceeds 2^31 rows         */
  ATTN_ERR_HEAD_DIM = -3,  /* d not in {64, 128}                                         */
  ATTN_ERR_GQA = -4,       /* H not a multiple of Hkv                                    */
  ATTN_ERR_DTYPE = -5,     /* dtype not an attn_dtype_t value                            */
  ATTN_ERR_SCALE = -6,     /* scale not finite or not > 0                                */
  ATTN_ERR_ALIGN = -7,     /* a tensor base address is not 16-byte aligned               */
  ATTN_ERR_WORKSPACE = -8, /* workspace NULL or smaller than attn_bwd_workspace_bytes()  */
  ATTN_ERR_LAUNCH = -9,    /* the HIP runtime rejected a kernel launch                   */
  ATTN_ERR_SCRATCH = -10   /* attn_bwd_noalloc: problem needs more than its fixed scratch */
} attn_status_t;

/*
 * Forward pass.  Reads q, k, v; writes o (fully overwritten) and lse.
 *   scale  : multiplies Q K^T before masking and softmax (usually 1/sqrt(d)).
 *   causal : 0 or 1.
 *   stream : a hipStream_t (NULL = the default stream).
 * Returns ATTN_OK or a negative attn_status_t; on a validation error nothing
 * is launched and no output is touched.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Hkv, int N, int d, float scale, int causal,
             int dtype, void* stream);

/*
 * Forward pass under a general mask (FlashAttention-2 page, causal masking "Option A":
 * mask the score tile, then the online softmax, with the mask predicate replaced):
 * query row i of batch b sees exactly the keys j with
 *     kv_lo[b*Nq + i] <= j <= kv_hi[b*Nq + i]
 * (device int32 arrays [B][Nq], the same for every head; values are clamped to
 * 0 .. Nk-1).  Causal (kv_lo = 0, kv_hi = i), causal with the queries at the end of
 * a longer key sequence (kv_hi = i + Nk - Nq), sliding windows, prefix-LM masks and
 * document masks of packed variable-length sequences are all such intervals.  A row
 * whose interval holds no key gets O = 0 and LSE = -inf.
 *     q, o : [B][H][Nq][d]      k, v : [B][Hkv][Nk][d]      lse : [B][H][Nq]
 * Tiles wholly outside a wave's rows' intervals are skipped, so cost follows the
 * number of visible pairs.  Same dtypes, d and return codes as attn_fwd (kv_lo and
 * kv_hi must be 4-byte aligned).
 */
int attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                    const int* kv_lo, const int* kv_hi, int dtype, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for these sizes: two float32 values
 * per query row (D = rowsum(dO * O) and LSE * log2(e)), each array rounded up to
 * 256 bytes.  Returns 0 for invalid sizes.  Callers should always ask this
 * function rather than assume the formula.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int dtype);

/*
 * Backward pass.  Reads q, k, v, o, lse (as written by attn_fwd with the same
 * arguments) and dO; writes dq, dk, dv (fully overwritten).  `workspace` is
 * caller-owned device memory of at least attn_bwd_workspace_bytes() bytes; its
 * contents on entry do not matter and on return are unspecified.  Two calls that
 * may overlap in time need distinct workspaces.
 * Same validation and return codes as attn_fwd, plus ATTN_ERR_WORKSPACE.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dO, void* dq, void* dk, void* dv,
             int B, int H, int Hkv, int N, int d, float scale, int causal,
             int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three kernels of attn_bwd, callable one at a time (for example to time
 * each, or to put them on different streams).  Running attn_bwd_preprocess,
 * then attn_bwd_dkdv and attn_bwd_dq (in either order, or concurrently once
 * the preprocess is complete) with the same arguments and workspace gives the
 * same dq, dk, dv as attn_bwd.
 *
 * attn_bwd_preprocess (softmax-backward page, the row dot product of the
 * softmax JVP; FlashAttention-2 page, backward pass): reads o, lse, dO and
 * writes D = rowsum(dO * O) and LSE * log2(e) into the workspace.  It reads no
 * q, k, v; Hkv only enters the size validation.
 *
 * attn_bwd_dkdv (FlashAttention-2 page, backward pass: the key/value block owns
 * its gradients and loops over query tiles): reads q, k, v, dO and the
 * workspace filled by attn_bwd_preprocess (lse itself is read by the float32
 * kernels only); writes dk and dv (fully overwritten).
 *
 * attn_bwd_dq (the separate-pass dQ of the FlashAttention-2 backward): reads
 * the same inputs and writes dq (fully overwritten).
 *
 * Each entry point validates like attn_bwd and returns the same codes; the
 * workspace is only read by attn_bwd_dkdv and attn_bwd_dq.
 */
int attn_bwd_preprocess(const void* o, const float* lse, const void* dO,
                        int B, int H, int Hkv, int N, int d, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                  const void* dO, void* dk, void* dv,
                  int B, int H, int Hkv, int N, int d, float scale, int causal,
                  int dtype, const void* workspace, size_t workspace_bytes,
                  void* stream);
int attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                const void* dO, void* dq,
                int B, int H, int Hkv, int N, int d, float scale, int causal,
                int dtype, const void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * Split-KV forward for few queries against many keys (decoding).
 *
 * Same operation as attn_fwd with Nq queries and Nk keys/values per head:
 *     q, o : [B][H][Nq][d]      k, v : [B][Hkv][Nk][d]      lse : [B][H][Nq]
 * The causal mask, when asked for, is aligned bottom-right: query i is position
 * i + Nk - Nq of the sequence and sees keys 0 .. i + Nk - Nq (for Nq == Nk this
 * is attn_fwd's mask); causal calls need Nk >= Nq.
 *
 * The key axis is cut into n_splits chunks computed in parallel; each chunk
 * keeps the online-softmax state (running max, denominator, unnormalised
 * output) over its keys and the chunks are then merged exactly by rescaling
 * them to a common max (ml-notes page, the split-K notes of the sparse
 * attention kernel; attnres-kernel-lab page, the exact two-partition merge;
 * FlashAttention-2 page, inner loop).  n_splits = 0 lets the library choose;
 * a request above one chunk per 32 keys is capped there.
 *
 * dtype must be ATTN_F16 or ATTN_BF16 (ATTN_ERR_DTYPE otherwise); d in {64, 128}.
 * `workspace` is caller-owned device memory of at least
 * attn_fwd_splitkv_workspace_bytes() for the same arguments (fp32 chunk
 * outputs and logsumexps); its contents on entry do not matter.  Calls that may
 * overlap in time need distinct workspaces.  Returns ATTN_OK or a negative
 * attn_status_t (ATTN_ERR_SHAPE also for n_splits < 0, causal with Nk < Nq, and
 * B * H * Nq of 2^26 rows or more, or chunkings whose launch would count 2^32
 * work-items or more; the workspace query returns 0 for those); on a validation
 * error nothing is launched.
 */
size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d,
                                        int causal, int dtype, int n_splits);
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                     int causal, int dtype, int n_splits, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Backward pass under the interval mask of attn_fwd_masked (same kv_lo, kv_hi,
 * Nq, Nk; lse as written by attn_fwd_masked).  Writes dq [B][H][Nq][d] and dk, dv
 * [B][Hkv][Nk][d] (fully overwritten; keys no query sees get zero gradients, rows
 * that see no key get dq = 0).  The workspace holds D and LSE * log2(e) per query
 * row and a 4-int summary of the intervals per 64-row query tile, which the dK/dV
 * kernel uses to skip query tiles that cannot see its keys.  Same validation and
 * return codes as attn_bwd.
 */
size_t attn_bwd_masked_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d,
                                       int dtype);
int attn_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                    const int* kv_lo, const int* kv_hi, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Row softmax, log-softmax and cross-entropy with logits (softmax-backward page on
 * shreyansh26.github.io): rows of `cols` elements, row-major and contiguous, in
 * `dtype` (fp32 statistics inside).  x, y, dy, dx, logits, dlogits: [rows][cols];
 * targets: int32 [rows]; loss, lse, dloss: float32 [rows].
 *
 * rowsoftmax_fwd: y = softmax(x) per row, or log-softmax x - logsumexp(x) when
 *   log_softmax = 1.
 * rowsoftmax_bwd: from the forward's output y and the upstream gradient dy,
 *   softmax:     dx = y * (dy - rowsum(dy * y))   (the row Jacobian-vector product)
 *   log-softmax: dx = dy - exp(y) * rowsum(dy)
 * rowxent_fwd: per-row loss logsumexp(x) - x[target] and the row logsumexp (kept
 *   for the backward); a row whose target is outside 0 .. cols-1 is ignored (loss 0).
 * rowxent_bwd: dlogits = dloss[row] * (softmax(x) - onehot(target)), softmax rebuilt
 *   from the saved logsumexp; zero for ignored rows.  A mean over the batch is
 *   dloss = 1/rows.
 *
 * Arrays of elements must be 16-byte aligned, int32/float32 row arrays 4-byte
 * aligned.  Returns ATTN_OK or ATTN_ERR_NULL / _SHAPE (rows or cols < 1, rows >=
 * 2^31, cols > 2^30, log_softmax not 0/1) / _DTYPE / _ALIGN / _LAUNCH; nothing is launched on a
 * validation error.  Only enqueues on `stream`.
 */
int rowsoftmax_fwd(const void* x, void* y, long long rows, int cols, int log_softmax,
                   int dtype, void* stream);
int rowsoftmax_bwd(const void* y, const void* dy, void* dx, long long rows, int cols,
                   int log_softmax, int dtype, void* stream);
int rowxent_fwd(const void* logits, const int* targets, float* loss, float* lse,
                long long rows, int cols, int dtype, void* stream);
int rowxent_bwd(const void* logits, const int* targets, const float* lse,
                const float* dloss, void* dlogits, long long rows, int cols, int dtype,
                void* stream);

/*
 * fp8 forward (the FlashAttention-2 page's forward with 8-bit operands; ml-notes page,
 * reduced-precision notes: low-precision products, fp32 accumulation and softmax
 * statistics).  q, k, v are e4m3 codes (OCP 8-bit float: bias 7, subnormals, no
 * infinity), one byte per element, q [B][H][N][d], k and v [B][Hkv][N][d]; the
 * values they stand for are code * descale_q (resp. _k, _v).  Computes
 *   O = softmax(scale * Q K^T) V   (causal: key j <= query i),  LSE as attn_fwd,
 * O in bf16 [B][H][N][d], LSE fp32 [B][H][N].  The probabilities are rounded to
 * e4m3 (times 256) for the P V product and the row sums are taken from those same
 * rounded values, so O is a convex combination of V rows with 8-bit weights: its
 * distance to the exact result is bounded by 2^-4 (relative) of the weighted spread
 * of V around it, not by bf16 rounding.  d must be 64 or 128 (ATTN_ERR_HEAD_DIM).
 * workspace: device memory of attn_fwd_fp8_workspace_bytes(B, Hkv, N, d) bytes
 * (V transposed per head: B * Hkv * d * N rounded up to 128, then to 256 bytes; 0
 * for invalid sizes), 16-byte aligned; its contents need no initialisation.
 * Scales and descales must be finite and > 0 (ATTN_ERR_SCALE).  Other errors as
 * attn_fwd; only enqueues on `stream`.
 */
size_t attn_fwd_fp8_workspace_bytes(int B, int Hkv, int N, int d);
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Hkv, int N, int d, float scale, float descale_q, float descale_k,
                 float descale_v, int causal, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory or hand
 * in a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, results and return codes as attn_bwd without
 * the workspace: it launches the same three kernels, their workspace (D and
 * LSE * log2(e)) placed in a fixed device array of ATTN_NOALLOC_SCRATCH_BYTES inside
 * the library.  Each GPU the library runs on holds its own copy of that array from
 * the library's load until the process ends; the first call on a GPU looks up its
 * address there (with that GPU current).  The call allocates nothing (no hipMalloc,
 * no allocating library routine).
 * Limit: attn_bwd_workspace_bytes() <= ATTN_NOALLOC_SCRATCH_BYTES, i.e. B * H * N
 * <= 4194304 query rows; a larger problem returns ATTN_ERR_SCRATCH and launches
 * nothing.  The array needs no clearing (every call writes all it reads), but all
 * calls on one GPU share it: calls that may overlap in time on the same GPU (other
 * streams, other host threads) race, and the caller must serialise them.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dO, void* dq, void* dk, void* dv,
                     int B, int H, int Hkv, int N, int d, float scale, int causal,
                     int dtype, void* stream);

/* A static, human-readable name for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* OSATTN_H */
