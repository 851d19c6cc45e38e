/*
 * nmspmv.h -- C ABI of libnmspmv, N:M semi-structured sparse matrix-vector
 * products for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one that SparseDecoding names as the decode-time hot
 * path: "SparseDecoding: Decoding-Aware Pruning for Accurate and Efficient
 * LLM Inference" (humanity-list story page, section "Abstract") -- decoding
 * is memory-bound and dominated by sparse matrix-vector products, and the
 * paper's system contribution is an N:M sparse matrix-vector kernel that
 * indexes kept weights with a bitmask and walks them with a fixed step.  The
 * bedrocknews arXiv 2610.12327v1 article adds that N:M means a fixed count
 * kept in every small block, and that the product is a sparse matrix times a
 * single vector rather than a batch.
 *
 * ---- Storage format (the readings this library fixes) --------------------
 * W is R x K, row-major, [out][in] (a PyTorch Linear weight); K is the
 * reduction axis.  Every M-wide group of columns [g*M, g*M + M) of a row keeps
 * exactly N entries (stored values may be zero).
 *   values [R][K*N/M]  16-bit words; group g of a row starts at value g*N
 *                      (fixed step) and holds its kept entries in ascending
 *                      column order.  No column-index or row-pointer arrays.
 *   masks  [R][K/8]    uint8 keep bitmap, one bit per dense column, least
 *                      significant bit first: bit (c % 8) of byte c/8 of a row
 *                      is set iff column c is kept.  (For M = 4 a byte holds
 *                      two groups, the even group in the low nibble.)
 *
 * ---- Conventions shared by every call -------------------------------------
 * - All pointers are device pointers (hipMalloc or a torch CUDA tensor).  The
 *   caller allocates and frees every buffer; the library keeps no
 *   allocations and no per-call state except one device word per GPU that
 *   nm_pack uses to report errors.  Calls are thread-safe.
 * - dtype is NM_FP16 (IEEE binary16) or NM_BF16 (bfloat16); W, values, x and y
 *   all use it.
 * - Shapes: R >= 0, K >= 0, K % 8 == 0, M in {4, 8}, 1 <= N < M, K % M == 0,
 *   1 <= B <= 32, R below 2^31 - 1024 (2 R for the gated calls) and K
 *   below 2^31.  Anything else returns NM_ERR_BAD_SHAPE
 *   (or NM_ERR_UNSUPPORTED for a dtype that is not one of the two) before
 *   any work is queued; outputs are then untouched.
 * - Alignment: W, values, masks and x must be 16-byte aligned; y 2-byte
 *   aligned; keep needs none.  Rows are contiguous, no strides.  y must not
 *   overlap any input.  Violations return NM_ERR_INVALID_ARG.
 * - stream is a hipStream_t (NULL = the null stream).  nm_spmv and
 *   nm_gemv_dense only enqueue work and return; nm_pack waits for its own
 *   work to finish.
 * - x must be finite.  With Inf or NaN in x the outputs are unspecified
 *   (a pruned column may or may not contribute 0 * Inf).
 */
#ifndef NMSPMV_H
#define NMSPMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NM_OK = 0,
    NM_ERR_INVALID_ARG = 1, /* null pointer, misalignment, overlapping output */
    NM_ERR_BAD_SHAPE = 2,   /* R, K, N, M or B outside the accepted set */
    NM_ERR_UNSUPPORTED = 3, /* dtype not NM_FP16 / NM_BF16 */
    NM_ERR_BAD_MASK = 4,    /* nm_pack: a keep-mask group without exactly N kept */
    NM_ERR_NONFINITE = 5,   /* nm_pack top-N: a NaN weight */
    NM_ERR_HIP = 6          /* the HIP runtime reported an error */
} nm_status;

typedef enum { NM_FP16 = 0, NM_BF16 = 1 } nm_dtype;

/*
 * nm_pack -- prune a dense W to N:M and pack it (the offline step that turns
 * a pruned weight into the bitmask-indexed form of the SparseDecoding
 * abstract; the pruning choice itself is the caller's, or top-N here).
 *   W      [R][K] 16-bit weights (dtype).
 *   keep   [R][K] bytes, nonzero = keep, or NULL.  With a keep-mask every
 *          group must have exactly N nonzero bytes, else NM_ERR_BAD_MASK;
 *          kept words (NaN included) are copied bit for bit.  With NULL the N
 *          entries of largest |w| are kept per group, the lower column
 *          winning a tie (-0 and +0 tie); a NaN anywhere gives
 *          NM_ERR_NONFINITE.
 *   values [R][K*N/M] 16-bit, masks [R][K/8] bytes: outputs, fully written.
 * Every group is checked before anything is written: on NM_ERR_BAD_MASK or
 * NM_ERR_NONFINITE the outputs are untouched.  The call returns when the
 * packed outputs are complete on the device.
 */
int nm_pack(const void* W, const uint8_t* keep, int64_t R, int64_t K, int N, int M, int dtype,
            void* values, uint8_t* masks, void* stream);

/*
 * nm_spmv -- y = W_sparse * x for 1..32 activation vectors: the decode-time
 * N:M sparse matrix-vector product of the SparseDecoding abstract and of the
 * "Key points" of "SparseDecoding Makes LLM Pruning Aware of Generation".
 *   values, masks  packed as nm_pack writes them (R rows, K dense columns).
 *                  The mask contents are not validated; a bitmap whose groups
 *                  do not hold exactly N bits gives unspecified y but never
 *                  an out-of-bounds access.
 *   x [B][K] 16-bit, y [B][R] 16-bit (output).
 *   y[b][r] = sum over kept columns c of W[r][c] * x[b][c]; every product and
 *   sum is formed in fp32 (in an unspecified order) and the sum is rounded
 *   once to the output dtype, to nearest even.  (Batches of a few vectors
 *   and up -- about 5 for nm_spmv, 3 where K is long, 4 for nm_gemv_dense --
 *   run on the matrix cores with fp32 accumulation; the arithmetic contract
 *   is the same.)
 * Enqueues on stream and returns; y is complete when the stream reaches it.
 */
int nm_spmv(const void* values, const uint8_t* masks, int64_t R, int64_t K, int N, int M, int dtype,
            const void* x, int B, void* y, void* stream);

/*
 * nm_gemv_dense -- the dense baseline y = W * x: the same decode projection
 * with the weight left unpruned, i.e. the comparison path that a sparse
 * speedup has to be read against.  The eucax.ai insights page on
 * SparseDecoding names that baseline as the missing piece of the published
 * speedup (section 3, "Reading the 1.48x result correctly") and asks for it to
 * be fixed and measured at the same operating point (section 6, "A
 * validation plan before adoption"); this call is that baseline, built on the
 * same kernel skeleton and fused the same way as nm_spmv.
 *   W [R][K], x [B][K], y [B][R], all dtype; fp32 accumulation, one rounding.
 * Same shape rules as nm_spmv without N and M (K % 8 == 0).
 */
int nm_gemv_dense(const void* W, int64_t R, int64_t K, int dtype, const void* x, int B, void* y, void* stream);

/*
 * nm_spmv_multi -- count (1..4) packed matrices with the same K, N:M and dtype
 * multiplied by the same x in one launch: y_i = W_i x for every i.  This is
 * the decode-layer fusion of projections that read one activation (q, k and
 * v; gate and up), so the per-launch start-up and drain are paid once.
 *   values[i], masks[i]  part i packed as nm_pack writes it, R[i] rows.
 *   y[i]                 [B][R[i]] output of part i.
 * Each y[i] equals what nm_spmv would give for part i alone up to fp32
 * summation order (the row split across lanes may differ); rules as for
 * nm_spmv, applied per part, plus: no y[i] may overlap another y[j], and the
 * total row count must stay below 2^31 - 1024.  count outside 1..4 is
 * NM_ERR_BAD_SHAPE; NULL array arguments are NM_ERR_INVALID_ARG.
 */
int nm_spmv_multi(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t K,
                  int N, int M, int dtype, const void* x, int B, void* const* y, void* stream);

/* nm_gemv_dense_multi -- the dense baseline of nm_spmv_multi: y_i = W_i x for
 * count (1..4) dense [R[i]][K] matrices sharing x, in one launch. */
int nm_gemv_dense_multi(int count, const void* const* W, const int64_t* R, int64_t K, int dtype, const void* x, int B,
                        void* const* y, void* stream);

/*
 * ---- K-split workspace (batched products on few rows) ------------------------
 * At a few vectors and up the products run on the matrix cores in 16-row
 * tiles.  A short matrix (the down projections: few rows, long K) then has
 * too few tiles to fill the GPU unless each tile's K is cut into slices, and
 * a slice's wave stages its own copy of x: at 8 vectors about as many x bytes
 * as weight bytes.  With a workspace the library can instead give each block
 * several tiles sharing one staged x over one range of K, and add the ranges'
 * fp32 partial sums at the end (the last block of each tile group adds them in
 * range order, so results are deterministic; they may differ from the
 * workspace-free call's in the last bit, as another fp32 summation order).
 *
 * nm_workspace_bytes -- the workspace size these calls need (a constant of
 * this library version, about 16 MB).
 *
 * nm_spmv_multi_ws, nm_gemv_dense_multi_ws -- nm_spmv_multi and
 * nm_gemv_dense_multi with a workspace: device memory of at least
 * nm_workspace_bytes() bytes, 256-byte aligned, zero-filled before its first
 * use (the library leaves it in a reusable state after every completed call),
 * not overlapping any input or output; workspace_bytes smaller, misalignment
 * or overlap give NM_ERR_INVALID_ARG.  workspace NULL = the plain call.  Calls
 * that may run at the same time (other streams, other threads) need
 * workspaces of their own; the caller owns and frees it.
 */
int64_t nm_workspace_bytes(void);
int nm_spmv_multi_ws(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t K,
                     int N, int M, int dtype, const void* x, int B, void* const* y, void* workspace,
                     int64_t workspace_bytes, void* stream);
int nm_gemv_dense_multi_ws(int count, const void* const* W, const int64_t* R, int64_t K, int dtype, const void* x,
                           int B, void* const* y, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * nm_spmv_multi_noalloc -- nm_spmv_multi with the K-split workspace taken
 * from the library itself, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops).  Arguments and rules as
 * for nm_spmv_multi; it calls no hipMalloc or other allocating routine.  The
 * workspace is a file-scope device array of nm_workspace_bytes() bytes in the
 * library's code object, one per GPU, held until the process ends; its
 * address is taken once per device, on the first call there, which also
 * clears its counters (a small kernel on the call's stream).  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and give wrong results -- serialize them.  The array
 * holds 16 MB of partial sums and 16384 tile-group counters: the K-split plan
 * is chosen only for calls whose partial sums fit it (the same limit as with
 * a caller's workspace), so no shape that nm_spmv_multi accepts needs more;
 * the others run without splitting.
 */
int nm_spmv_multi_noalloc(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R,
                          int64_t K, int N, int M, int dtype, const void* x, int B, void* const* y, void* stream);

/*
 * nm_spmv_swiglu -- the gated-MLP input of a decode layer in one launch:
 *   h[b][r] = SiLU(g) * u,  g = (W_gate x_b)[r],  u = (W_up x_b)[r],
 *   SiLU(t) = t / (1 + e^-t).
 * The models the SparseDecoding pages evaluate (Llama-3.1-8B, Llama-3.3-70B,
 * Qwen3-14B/32B; "SparseDecoding: Decoding-Aware Pruning ...", Abstract) use
 * this SiLU-gated MLP; the pages themselves do not describe the layer, so
 * this fusion of the two N:M products that share x is this library's own.
 *   values_gate, masks_gate, values_up, masks_up  two packed [R][K] matrices
 *                  (nm_pack layout) with the same K, N:M and dtype.
 *   x [B][K], h [B][R] (output), dtype as in nm_spmv.
 * g and u are the fp32 sums nm_spmv would form (never rounded to 16 bits);
 * SiLU and the product are evaluated in double precision (fp32 would flush
 * SiLU(g) to 0 below g = -88.7, where bf16 still represents h) and the result
 * is rounded to fp32, then to dtype, to nearest even.  Rules as for nm_spmv,
 * plus: h must not overlap any input.
 */
int nm_spmv_swiglu(const void* values_gate, const uint8_t* masks_gate, const void* values_up, const uint8_t* masks_up,
                   int64_t R, int64_t K, int N, int M, int dtype, const void* x, int B, void* h, void* stream);

/* nm_gemv_dense_swiglu -- the dense baseline of nm_spmv_swiglu: h = SiLU(W_gate x) * (W_up x)
 * for dense [R][K] W_gate and W_up, in one launch; rules as for nm_gemv_dense. */
int nm_gemv_dense_swiglu(const void* W_gate, const void* W_up, int64_t R, int64_t K, int dtype, const void* x, int B,
                         void* h, void* stream);

/*
 * ---- Decoding-aware calibration -----------------------------------------------
 * SparseDecoding builds its pruning objective from the inputs each layer sees
 * while the dense model generates, prefill excluded, and guides pruning with
 * the objective's Hessian ("SparseDecoding: Decoding-Aware Pruning ...",
 * Abstract; "SparseDecoding Makes LLM Pruning Aware of Generation", Key points
 * and the section on why fixed-text calibration misses).  The pages give no
 * formula; these two calls implement the plainest reading, and their output
 * enters the sparse path through nm_pack's keep-mask.
 *
 * nm_calib_accumulate -- H += sum over decode rows t of x_t x_t^T: the Hessian
 * (up to a constant) of a linear layer's squared output error over its inputs
 * at decode steps.
 *   X [T][K] 16-bit (dtype): the layer's input rows, in any order.
 *   decode [T] bytes: nonzero marks a decode-step row; zero rows (prefill)
 *          do not enter H.  NULL = every row is a decode step.
 *   H [K][K] fp32, row-major, accumulated in place (zero it before the first
 *          call); calls add up, so rows can be streamed in batches.
 * Products of two 16-bit values are exact in fp32; the sums are fp32 (matrix
 * cores) in an unspecified order.  K % 8 == 0, K <= 65536; X 16-byte and H
 * 4-byte aligned; H must not overlap X or decode.  Enqueues and returns.
 */
int nm_calib_accumulate(const void* X, const uint8_t* decode, int64_t T, int64_t K, int dtype, float* H, void* stream);

/*
 * nm_calib_keep_mask -- the N:M keep-mask from a calibration Hessian: per
 * M-group of each row keep the N columns of largest saliency w^2 * H_jj (the
 * optimal-brain-surgeon saliency with H taken diagonal), the lower column on
 * equal saliency; a NaN saliency ranks below every number (-inf included),
 * NaNs among themselves the lower column first.  The saliency is
 * formed exactly (double), so the mask is fully determined by W and H's
 * diagonal.
 *   W [R][K] 16-bit (dtype); h: H_jj = h[j * h_stride] (h_stride = K + 1 on a
 *   full row-major H, 1 on a diagonal vector); keep [R][K] bytes, written 1
 *   (keep) or 0, exactly N ones per group: pass it to nm_pack.
 * Shape rules as for nm_pack, h_stride >= 1; W 16-byte, keep 8-byte and h
 * 4-byte aligned; keep must not overlap W or h.  Enqueues and returns.
 */
int nm_calib_keep_mask(const void* W, const float* h, int64_t h_stride, int64_t R, int64_t K, int N, int M, int dtype,
                       uint8_t* keep, void* stream);

/*
 * ---- Hybrid sparse + dense rows -------------------------------------------------
 * The Spense abstract ("Semi-structured 2:4 sparsity ...", on the
 * thelatestinai.com page for arXiv 2610.02598) splits a weight matrix into a
 * 2:4-sparse region and a dense region and stresses choosing the dense region
 * well; it fixes neither the region's shape nor the rule.  This library's
 * reading: the dense region is a set of whole rows (output channels), the rows
 * whose pruning loses most,  L_r = sum over the row's pruned columns c of
 * w[r][c]^2 * h[c]  (h the calibration Hessian's diagonal, or 1).  The sparse
 * rows are packed as nm_pack packs them, the dense rows kept as they are, and
 * two row lists say where each part's rows go in y.
 *
 * nm_hybrid_row_loss -- L_r for every row, in double: W [R][K] 16-bit (2-byte
 * aligned); keep as in nm_pack (NULL: the top-N magnitude rule decides what is
 * pruned); h[c * h_stride] fp32 (4-byte aligned) or NULL for 1; loss [R] double
 * (8-byte aligned, output).  Terms are summed per row in column order, one
 * rounding per term.  Waits for completion.  A keep-mask group without N kept
 * -> NM_ERR_BAD_MASK; a NaN weight under the magnitude rule ->
 * NM_ERR_NONFINITE (loss then unspecified).
 */
int nm_hybrid_row_loss(const void* W, const uint8_t* keep, const float* h, int64_t h_stride, int64_t R, int64_t K, int N,
                       int M, int dtype, double* loss, void* stream);

/* nm_hybrid_select_rows -- flags[r] = 1 for the n_dense (0..R) rows of largest
 * loss, 0 elsewhere; a NaN loss ranks below every number (-inf included) and
 * equal to another NaN, the lower row first among equals.  loss [R] double (8-byte aligned), flags [R] bytes.  Enqueues. */
int nm_hybrid_select_rows(const double* loss, int64_t R, int64_t n_dense, uint8_t* flags, void* stream);

/*
 * nm_hybrid_pack -- build the hybrid matrix from W and the row flags (exactly
 * n_dense nonzero, else NM_ERR_BAD_MASK): rows_dense [n_dense] and
 * rows_sparse [R - n_dense] (int32, 4-byte aligned) list the flagged and the
 * other rows in increasing order; W_dense [n_dense][K] holds the flagged rows
 * of W; values / masks hold the other rows packed as nm_pack packs them (keep
 * as in nm_pack, indexed by the rows of W).  Alignment and error rules as for
 * nm_pack; no output may overlap an input or another output.  Waits for
 * completion.
 */
int nm_hybrid_pack(const void* W, const uint8_t* keep, const uint8_t* flags, int64_t n_dense, int64_t R, int64_t K,
                   int N, int M, int dtype, void* values, uint8_t* masks, void* W_dense, int32_t* rows_sparse,
                   int32_t* rows_dense, void* stream);

/*
 * nm_spmv_hybrid -- y = W_hybrid x: y[b][rows_sparse[i]] from sparse row i as
 * nm_spmv computes it, y[b][rows_dense[j]] from dense row j as nm_gemv_dense
 * does.  The lists must partition 0..R-1 (as nm_hybrid_pack writes them);
 * otherwise y is unspecified, but entries are clamped into 0..R-1, never
 * written out of bounds.  Rules as for nm_spmv (x [B][K], y [B][R], B <= 32).
 * With one to three vectors and 2:4 or 4:8 rows (K % 16 == 0) both parts
 * usually run in a single launch.  Enqueues.
 */
int nm_spmv_hybrid(const void* values, const uint8_t* masks, const int32_t* rows_sparse, const void* W_dense,
                   const int32_t* rows_dense, int64_t n_dense, int64_t R, int64_t K, int N, int M, int dtype,
                   const void* x, int B, void* y, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* nm_status_string(int status);

/* Library ABI version: 100 * major + minor. */
int nm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NMSPMV_H */
