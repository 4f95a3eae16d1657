/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library, libgdn.so.
 *
 * The operation (per head, per token t):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * i.e. decay the carried state, predict v_t from the DECAYED state, write
 * beta_t times the prediction error along k_t, then read the NEW state with
 * q_t.  Sources: "On State Reduction in Linear Attention" (reading notes),
 * paper Sec. 2.1, Eqs. (1)-(2) (DeltaNet write, readout o_t = S_t q_t, state
 * S in R^{dv x dk}) with the input-dependent decay of Gated DeltaNet; and
 * "Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
 * Routing" (reading notes), paper Sec. 3.3, Eqs. 15-17 (decay first, then compare
 * with the target, then write) and the per-token data flow of Eq. 8 (the
 * output reads the updated state).  No query scale is applied.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc'd or equivalent),
 *    owned by the caller, except in the host-side channel selection
 *    (gdn_drrqr_select).  The library never allocates device memory, frees
 *    or synchronises inside these calls; work is enqueued on `stream` (a
 *    hipStream_t passed as void*, NULL = the null stream) and completes
 *    asynchronously.
 *  - Layouts are dense, contiguous, row-major:
 *        q, k   [B, T, H, dk]      v, o  [B, T, H, dv]
 *        alpha, beta  [B, T, H]    S     [B, H, dv, dk]   (a state row is
 *                                                          one value channel)
 *    The decode step drops the T axis.
 *  - q/k/v use `in_dtype` (GDN_F32 or GDN_BF16); o uses `out_dtype`;
 *    alpha, beta and the state are always float32.
 *  - Supported head sizes: dk in {64, 128} (dk = 64 is the channel-pruned,
 *    "state halved" width of "On State Reduction in Linear Attention",
 *    paper Sec. 3.2-3.3), dv in {64, 128}.
 *  - Preconditions not checked (checking would cost a pass over the data):
 *    q and k are already unit-L2-normalised (and already gathered to the
 *    kept channels when pruned; the *_qk entry points below do both inside
 *    the kernels); alpha in (0, 1]; beta in [0, 1].  Outside
 *    these ranges the same formula is applied but results are untested.
 *  - Errors: argument errors are returned synchronously BEFORE any HIP call
 *    (GDN_EINVAL: null pointer, negative size, zero B/H; GDN_ESHAPE:
 *    unsupported dk/dv or dtype; GDN_EWORKSPACE: workspace too small).  A
 *    failed launch returns GDN_EHIP.  Faults during execution surface at the
 *    caller's next synchronisation.  No exception or abort crosses the ABI.
 *  - Results are bitwise deterministic for a given shape, dtype and device
 *    (no atomics).  The library keeps no mutable global state, except the
 *    device scratch of gdn_prefill_noalloc and its per-device address.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gdn_status {
  GDN_OK = 0,
  GDN_EINVAL = 1,
  GDN_ESHAPE = 2,
  GDN_EWORKSPACE = 3,
  GDN_EHIP = 4
};

enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 };

/* Human-readable name of a status code (static string, never NULL). */
const char* gdn_status_str(int status);

/* Library version string, "MAJOR.MINOR.PATCH". */
const char* gdn_version(void);

/* ------------------------------------------------------------------------
 * Prefill over whole sequences (chunked form).
 *
 * Bytes of device workspace gdn_prefill needs for these sizes (0 for T = 0 or
 * an unsupported dk/dv).  It holds, per 64-token chunk and head, the
 * chunk's triangular delta correction, its decay-masked query-key products
 * and its gate prefix sums (33,792 bytes), and, when B*H heads alone are too
 * few to fill the GPU and T spans at least 16 chunks, buffers for splitting
 * each sequence into segments that run in parallel (per head: T*dk*2 bytes,
 * and per segment dv*dk*4 + dk*dk*4 + dv*dk*2 bytes).  The size covers
 * every dtype combination.
 */
size_t gdn_prefill_workspace_bytes(int B, int T, int H, int dk, int dv);

/*
 * How gdn_prefill will split the work for these sizes and dtypes: returns
 * the number of sequence segments per head (1 = no segmentation, every head
 * scanned start to end by one set of workgroups) and, if seg_chunks is not
 * NULL, the number of 64-token chunks per segment.  Returns 0 for invalid
 * arguments.  Pure host computation; no HIP call.
 */
int gdn_prefill_segments(int B, int T, int H, int dk, int dv, int in_dtype,
                         int out_dtype, int* seg_chunks);

/*
 * Runs the recurrence over T tokens for B*H independent heads.
 *   q, k, v      inputs, in_dtype, layouts above.
 *   alpha, beta  [B, T, H] float32.
 *   S0           [B, H, dv, dk] float32 initial state, or NULL for zero.
 *   o            [B, T, H, dv] out_dtype (may be NULL only if T == 0).
 *   ST           [B, H, dv, dk] float32 final state, or NULL to skip it.
 *                ST may be the same pointer as S0 (updated in place); no
 *                other overlap between outputs and inputs is allowed.
 *   workspace    device scratch of at least gdn_prefill_workspace_bytes().
 * The result equals the token-by-token recurrence up to rounding; the
 * chunked evaluation order is an exact re-association of it.
 * T == 0 copies S0 (or zeros) into ST.
 */
int gdn_prefill(const void* q, const void* k, const void* v,
                const float* alpha, const float* beta, const float* S0,
                void* o, float* ST,
                int B, int T, int H, int dk, int dv,
                int in_dtype, int out_dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two phases of gdn_prefill, exposed so a caller can time or schedule
 * them separately.  gdn_prefill == gdn_prefill_prepare then gdn_prefill_scan
 * on the same stream with the same workspace and the same dtypes (prepare
 * takes the output dtype because only fp32 outputs read the low half of the
 * split query-key tile, which it then also writes; a scan with another
 * out_dtype than its prepare's is not supported and its outputs are
 * undefined).
 *   prepare: per 64-token chunk, independent of the state: the gate prefix
 *            sums and per-token decay factors, the unit-lower-triangular
 *            delta correction (I + A)^{-1} with A_ji = beta_j e^{g_j - g_i}
 *            k_j.k_i (i < j), stored times diag(beta), and the
 *            decay-masked query-key products; written to workspace.  When
 *            the scan will segment the sequence (below), it writes per-token
 *            exponent rows instead of the query-key products, which that
 *            scan forms itself from the q and k it stages.
 *   scan:    sequential over chunks, parallel over heads and 64-row groups
 *            of the state: reads q, k, v and the chunk tiles, writes o and
 *            ST.  With bf16 inputs and outputs and few heads it also splits
 *            each sequence into segments (extra "transition" rows give each
 *            segment's affine map of its incoming state), chains the
 *            segment states, and corrects the outputs of later segments;
 *            it then also writes the segment buffers of the workspace.
 */
int gdn_prefill_prepare(const void* q, const void* k,
                        const float* alpha, const float* beta,
                        int B, int T, int H, int dk, int dv, int in_dtype,
                        int out_dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

int gdn_prefill_scan(const void* q, const void* k, const void* v,
                     const float* S0, void* o, float* ST,
                     int B, int T, int H, int dk, int dv,
                     int in_dtype, int out_dtype,
                     void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * gdn_prefill without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * The workspace lives in a static device array of GDN_NOALLOC_SCRATCH_BYTES
 * (256 MiB) that each device the library runs this call on holds until the
 * process ends.  Sizes with gdn_prefill_workspace_bytes(B, T, H, dk, dv)
 * above that return GDN_EWORKSPACE, checked before any HIP call (the
 * 16-head, 16,384-token layer with dk = dv = 128 needs 236 MiB; B = 8,
 * T = 4096, H = 16 needs 264 MiB and is rejected).  The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress);
 * no call allocates or frees memory.  Every call on one device shares the
 * array: calls that overlap on one device (different streams, or host
 * threads without ordering between them) race and their results are
 * undefined.  All other arguments, results, layouts and errors are those of
 * gdn_prefill; the results equal gdn_prefill's bitwise.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

int gdn_prefill_noalloc(const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const float* S0,
                        void* o, float* ST, int B, int T, int H, int dk, int dv,
                        int in_dtype, int out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * One decode token for a batch of carried states.
 *   q, k [B, H, dk]; v [B, H, dv] (in_dtype); alpha, beta [B, H] float32;
 *   S_in [B, H, dv, dk] float32; S_out same shape (S_out == S_in allowed:
 *   in-place update; no partial overlap); o [B, H, dv] out_dtype.
 * Each state element is read once and written once.  Uses no workspace.
 */
int gdn_decode_step(const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta,
                    const float* S_in, float* S_out, void* o,
                    int B, int H, int dk, int dv,
                    int in_dtype, int out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * The input path of a channel-pruned layer, fused into the kernels.
 *
 * "On State Reduction in Linear Attention", paper Sec. 3.2-3.3, prunes a layer by
 * keeping a per-head subset I_h of the query/key channels and recomputing
 * the L2 normalisation over the kept channels.  These variants take q and
 * k as the raw projection output, rows of dk_in elements, and apply
 *     q_t <- q_scale * P_I q_t / |P_I q_t|,   k_t <- P_I k_t / |P_I k_t|
 * (P_I keeps channels[h][0..dk-1] of head h's row, in that order; without
 * l2norm the division is skipped; a kept vector that is all zero stays
 * zero) before the recurrence, with no pass over q/k outside the kernels.
 *   channels   [H, dk] int32 device array, 16-byte aligned, each entry in
 *              [0, dk_in), or NULL: the rows are dk wide and all kept (dk_in
 *              must equal dk, else GDN_ESHAPE).  The kernels clamp an entry
 *              outside [0, dk_in) to the nearest end of the row (0 or
 *              dk_in - 1): no read leaves the row, and the results are those
 *              of the clamped subset (no error is reported; checking on the
 *              host would need a copy of the device array).
 *   dk_in      row width of q and k in memory (1 .. 2^20 with channels).
 *   l2norm     1: normalise q and k over the kept channels; 0: do not.
 *   q_scale    multiplies the (normalised) query; 1 for none.
 * With channels, q and k need only their element alignment (2 or 4 bytes);
 * without, 16 bytes as elsewhere.  All other arguments, layouts (with dk
 * the kept width of S0/ST/S) and errors are those of gdn_prefill and
 * gdn_decode_step.  With channels == NULL, l2norm == 0 and q_scale == 1
 * the results equal gdn_prefill's / gdn_decode_step's bitwise.
 *
 * Workspace of gdn_prefill_qk: gdn_prefill's, plus (gather != 0, i.e.
 * channels given) a gathered copy of the kept q/k channels,
 * 2 * B*T*H*dk elements of in_dtype, that the scan reads.  0 for an
 * unsupported dk/dv/dtype or T == 0.
 */
size_t gdn_prefill_qk_workspace_bytes(int B, int T, int H, int dk, int dv,
                                      int in_dtype, int gather);

int gdn_prefill_qk(const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* S0,
                   void* o, float* ST, int B, int T, int H, int dk, int dv,
                   int dk_in, const int* channels, int l2norm, float q_scale,
                   int in_dtype, int out_dtype, void* workspace,
                   size_t workspace_bytes, void* stream);

int gdn_decode_step_qk(const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta,
                       const float* S_in, float* S_out, void* o, int B, int H,
                       int dk, int dv, int dk_in, const int* channels,
                       int l2norm, float q_scale, int in_dtype, int out_dtype,
                       void* stream);

/* ------------------------------------------------------------------------
 * Generalised gates, recurrent form.
 *
 * "Linear Attention Architectures" (reading notes), paper Sec. 3.4 (Kimi
 * Delta Attention, Eqs. 18-20) and paper Sec. 3.5 (Gated DeltaNet-2, Eqs. 21-24) refine the scalar gates of the
 * gated delta rule: a retention alpha per KEY channel, applied on the key
 * side of the state, and separate erase (b, key side) and write (w, value
 * side) gates.  Per head and token:
 *     S~  = S_{t-1} diag(alpha_t)
 *     S_t = S~ (I - (b_t * k_t) k_t^T) + (w_t * v_t) k_t^T
 *     o_t = S_t q_t
 * (* element-wise).  b = w = beta_t * 1 is Kimi Delta Attention; with
 * alpha_t = a_t * 1 as well it is gdn_prefill's recurrence.
 *   q, k         [B, T, H, dk] in_dtype, 16-byte aligned.
 *   v            [B, T, H, dv] in_dtype.
 *   alpha, b     [B, T, H, dk] float32, 16-byte aligned; alpha in (0, 1].
 *   w            [B, T, H, dv] float32.
 *   S0           [B, H, dv, dk] float32 or NULL (zero); ST the final state
 *                or NULL; ST may alias S0.
 *   o            [B, T, H, dv] out_dtype.
 * T == 1 is the decode step (one streaming pass over the state).  The
 * kernel runs the tokens in order (no chunked form), so long sequences are
 * bound by the per-token dependency chain.  Uses no workspace.  Errors as
 * for gdn_prefill; T == 0 copies S0 (or zeros) into ST.
 */
int gdn_gated_recurrent(const void* q, const void* k, const void* v,
                        const float* alpha, const float* b, const float* w,
                        const float* S0, void* o, float* ST, int B, int T,
                        int H, int dk, int dv, int in_dtype, int out_dtype,
                        void* stream);

/*
 * The same generalised gates over whole sequences in chunked form (64-token
 * chunks; bf16 inputs).  Inside a chunk the per-key-channel retention enters
 * through its per-channel cumulative log G_j: the erase and query keys of
 * token j are weighted by e^{G_j}, the key of token i in the state update by
 * e^{G_C - G_i}, and the chunk's key-key and query-key products by
 * e^{G_j - G_i} per channel, formed as products of factors weighted against
 * a reference token in the middle of each 16-token block; T = (I + A)^{-1}
 * with A_ji = sum_d b_jd k_jd k_id e^{G_jd - G_id} (i < j).  The products run
 * on bf16 MFMA with split-bf16 operands and fp32 accumulation.  Retentions
 * below about 3e-5 per token (log2 < -15) may underflow a weighted factor;
 * results are untested there.
 * Arguments and layouts as gdn_gated_recurrent, plus
 *   workspace   device memory of at least gdn_gated_prefill_workspace_bytes()
 *               bytes, 16-byte aligned: per head and chunk the T and P tiles
 *               (32,768 bytes), the weighted keys and queries (6 * 64 * dk * 2
 *               bytes) and e^{G_C} (dk * 4 bytes).
 * fp32 inputs (in_dtype GDN_F32) and T == 0 run gdn_gated_recurrent (no
 * workspace used; the workspace size is then 0).  Errors as gdn_prefill.
 */
size_t gdn_gated_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int in_dtype);
int gdn_gated_prefill(const void* q, const void* k, const void* v,
                      const float* alpha, const float* b, const float* w,
                      const float* S0, void* o, float* ST, int B, int T, int H,
                      int dk, int dv, int in_dtype, int out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward pass of gdn_prefill's recurrence.
 *
 * The pages train these layers ("Linear Attention Architectures" reading
 * notes, the training set-ups of its experiments; "On State Reduction in
 * Linear Attention", the recovery fine-tuning of pruned layers) but print
 * no backward pass: these are the exact gradients of the forward step of
 * gdn_prefill (S~ = alpha S_{t-1}, S_t = S~ + beta (v - S~ k) k^T,
 * o_t = S_t q_t) for the loss L = sum_t <do_t, o_t> + <dST, S_T>.
 *   q, k          [B, T, H, dk] in_dtype, 16-byte aligned.
 *   v             [B, T, H, dv] in_dtype, element-aligned.
 *   d_o           [B, T, H, dv] in_dtype (the gradient of o), 16-byte
 *                 aligned for bf16, element-aligned for fp32.
 *   alpha, beta   [B, T, H] float32.
 *   S0            [B, H, dv, dk] float32 or NULL (zero initial state).
 *   dST           [B, H, dv, dk] float32 or NULL (no gradient on S_T).
 *   dq, dk        [B, T, H, dk] float32, 4-byte aligned (written).
 *   dv            [B, T, H, dv] float32 (written).
 *   dalpha, dbeta [B, T, H] float32 (written).
 *   dS0           [B, H, dv, dk] float32 or NULL (not wanted); it may alias
 *                 dST or S0 exactly, not partly (every read of dST and S0
 *                 precedes the write of dS0 on the stream).
 *   workspace     device memory of at least gdn_backward_workspace_bytes()
 *                 bytes for these sizes and in_dtype, 16-byte aligned,
 *                 owned by the caller; NULL allowed when that size is 0
 *                 (T == 0).
 * All pointers are device pointers; the call is asynchronous on `stream`.
 *
 * bf16 inputs run the chunked form (64-token chunks, the products on bf16
 * MFMA with split-bf16 operands wherever a state, a state gradient or an
 * intermediate enters): the prepare phase of gdn_prefill (also storing T
 * itself), a forward sweep that stores the state at the start of every
 * chunk, a backward sweep over the chunks in reverse that stores the state
 * gradient at the end of every chunk (and writes dS0), and one fully
 * parallel pass over (batch, head, chunk) that forms every gradient of the
 * chunk's tokens.  The workspace then holds, per head and chunk, the
 * prepare tiles (33,792 bytes), T (16,384 bytes) and two dv x dk fp32
 * states: 181,248 bytes per head and chunk at dk = dv = 128, so 1.48 GB at
 * B = 8, T = 4096, H = 16.
 * fp32 inputs run the recurrent form: each wave reruns its state rows
 * forward, storing a checkpoint every 8 tokens, then steps back through
 * each 8-token block with the block's states in registers; its workspace
 * grows as B H (T / 8) dv dk 4 bytes (checkpoints) plus per-workgroup
 * partial sums (4.3 GB + 2.2 GB at B = 8, T = 4096, H = 16, dk = dv = 128).
 * Sums over the dv rows of a head (dq, dk, dalpha, dbeta) are taken in a
 * fixed order in both forms, so results are reproducible bit for bit.
 * Errors: GDN_ESHAPE for dk or dv outside {64, 128} or an unknown dtype;
 * GDN_EINVAL for a NULL or misaligned required pointer, bad sizes or a
 * partial overlap of dS0; GDN_EWORKSPACE for a missing or short workspace;
 * GDN_EHIP if a launch fails.  T == 0 writes dS0 = dST (or zeros).
 */
size_t gdn_backward_workspace_bytes(int B, int T, int H, int dk, int dv, int in_dtype);
int gdn_backward(const void* q, const void* k, const void* v,
                 const float* alpha, const float* beta, const float* S0,
                 const void* d_o, const float* dST, float* dq, float* dk,
                 float* dv_, float* dalpha, float* dbeta, float* dS0, int B,
                 int T, int H, int dk_, int dv, int in_dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * DRRQR channel selection (calibration time, HOST memory and host code).
 *
 * "On State Reduction in Linear Attention" (reading notes), paper Sec. 3.4 with
 * Algorithm 2 and App. B.2: choose which k of a head's n key/query channels
 * a pruned layer keeps, from calibration samples M = [K_cal; Q_cal] (rows =
 * samples, one column per channel).  A QR with column pivoting gives the
 * first choice; then, while some rho_ij = sqrt((A^{-1}B)_ij^2 +
 * (gamma_j / omega_i)^2) exceeds f (A, B, C the blocks of the triangular
 * factor, omega_i = 1 / ||row i of A^{-1}||, gamma_j = ||column j of C||),
 * the kept column i and the dropped column j of the largest rho_ij trade
 * places (strong rank-revealing QR).  At the end every such trade would
 * grow the volume spanned by the kept columns by at most a factor f, and
 * with c_f = sqrt(1 + f^2 k (n - k)): sigma_i(A) >= sigma_i(M) / c_f,
 * ||C||_2 <= c_f sigma_{k+1}(M).
 *   M          [rows, n] float64, row-major, HOST pointer; rows >= n.
 *   k          channels kept, 1 <= k < n (n <= 4096).
 *   f          tolerance >= 1 (the swap threshold).
 *   max_swaps  bound on the number of trades (>= 0).
 *   selected   [k] int32 HOST output: the kept channel indices, in the
 *              order of the final factor's first k columns.
 *   swaps      trades made, or NULL;  rho_max  final largest rho_ij, or NULL.
 * fp64 throughout; no GPU work, no stream.  Unlike the other entry points it
 * allocates HOST memory (a column-major copy of M, rows * n doubles, and
 * O(n^2) more), freed before it returns.  GDN_EINVAL for bad sizes, a null
 * pointer, f < 1, or rank(M) < k.
 */
int gdn_drrqr_select(const double* M, int rows, int n, int k, double f,
                     int max_swaps, int* selected, int* swaps, double* rho_max);

/* ------------------------------------------------------------------------
 * Rank-r truncation of carried states.
 *
 * Replaces each state S (dv x dk) by U_r U_r^T S, where U_r holds the r
 * leading left singular vectors of S, i.e. projects the state onto its top-r
 * left singular directions.  "How much of its state does Gated DeltaNet
 * use?", §3, applies this to every head's carried state at each
 * 256-token segment boundary (r equal to the state width is the unchanged
 * model).  The stable rank er(S) = ||S||_F^2 / sigma_1(S)^2 is "On State
 * Reduction in Linear Attention", paper Sec. 2.2, Eq. (5).
 *
 * Bytes of workspace gdn_truncate_rank needs when r < min(dv, dk):
 * BH * min(dv, dk) * dv * 8 (the unit singular vectors, fp64).  0 for
 * invalid sizes.
 */
size_t gdn_truncate_workspace_bytes(int BH, int dv, int dk);

/*
 *   S          [BH, dv, dk] float32 states, updated in place.
 *   BH         number of states (1 .. 65535).
 *   r          rank kept, >= 1.  r >= min(dv, dk) leaves S unchanged.
 *   er_out     [BH] float32: the stable rank of each RESULT (NaN for a zero
 *              state), or NULL to skip it.
 *   workspace  device scratch of at least gdn_truncate_workspace_bytes();
 *              may be NULL when r >= min(dv, dk).
 * The left singular vectors are the leading eigenvectors of the symmetric
 * S S^T, found in fp64 by Householder tridiagonalisation, Sturm-sequence
 * bisection for the r largest eigenvalues and inverse iteration; the
 * projection is fp32.  When sigma_r == sigma_{r+1} the leading
 * r-dimensional subspace is not unique and the result is one valid choice.  Errors as for the other entry points
 * (GDN_EINVAL for r < 1, a null S, BH out of range or misalignment).
 */
int gdn_truncate_rank(float* S, int BH, int dv, int dk, int r, float* er_out,
                      void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
