// Internal launchers of libgdn (C++ linkage; the exported C ABI is in
// include/gdn.h).  Each assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

constexpr int kChunk = 64;     // tokens per prefill chunk
constexpr int kSlice = 16;     // state rows per prefill scan workgroup
// Per (head, chunk) workspace: delta correction T [64x64], masked query-key
// products P [64x64], gate block (g, beta, gamma, decay-to-end) [4x64].
constexpr size_t kChunkWsFloats = 2 * kChunk * kChunk + 4 * kChunk;

// Sequence segmentation of a prefill (used when B*H alone cannot fill the
// chip).  The map from a segment's incoming state S_in to its outputs and
// final state is affine: S_end = S_in X + S_loc and o_t = o_loc_t + S_in x^_t
// with X = the product of the segment's transitions alpha (I - beta k k^T),
// x^_t = X_t q_t.  Phase 1 runs every segment from a zero state (segment 0
// from S0) together with dk "transition rows" that start at the identity and
// see v = 0 (they evolve exactly like state rows, giving X and x^); phase 2
// chains S_in(s) = S_end(s-1) over the segments; phase 3 adds S_in(s) x^_t
// to the outputs of segments >= 1.
struct SegArgs {
  int nseg;          // segments per head (1: unsegmented, the fields below unused)
  int seg_chunks;    // chunks per segment (the last may be shorter)
  float* S_fin;      // [BH][nseg][dv][dk] final real-row state of each segment
  void* X_fin;       // [BH][nseg][2][dk][dk] bf16: X^T of segments >= 1, hi then lo part
  void* S_in;        // [BH][nseg][dv][dk] bf16: incoming state of each segment, rounded
  void* xhat;        // [BH][T][dk] bf16, x^_t for tokens of segments >= 1
};

// The input path of a channel-pruned layer, applied inside the kernels
// ("On State Reduction in Linear Attention", paper Sec. 3.2-3.3: keep a per-head
// subset of the query/key channels and recompute the normalisation over the
// kept channels), plus an optional query scale.
struct QkArgs {
  const int* chan;   // [H][dk] kept channels of each head's dk_in-wide q/k
                     // rows, or nullptr: the rows are dk wide, all kept
  int dk_in;         // width of the q/k rows in memory (dk without chan)
  int l2norm;        // 1: divide q and k by their norms over the kept channels
  float qscale;      // multiplies the (normalised) query
  void* qk_out;      // prefill with chan: the gathered copy, k then q,
                     // [2][B][T][H][dk] in the input type (the scan reads it)
  void* t_out = nullptr;   // if set, the prepare kernel also writes T itself
                     // (without diag(beta)) as bf16 hi/lo 64x64 tiles,
                     // kTuBytes per (batch, head, chunk) (the backward pass)
};
constexpr size_t kTuBytes = 2 * 64 * 64 * 2;
inline QkArgs qk_identity(int dk) { return QkArgs{nullptr, dk, 0, 1.f, nullptr}; }

// Bytes of the gathered q/k copy of a prefill with a channel subset.
inline size_t qk_copy_bytes(int B, int T, int H, int dk, int in_dtype) {
  return 2 * (size_t)B * T * H * dk * (in_dtype == 1 ? 2 : 4);
}

struct PrefillPlan {
  int nchunks, nseg, seg_chunks;
  size_t chunk_bytes;       // per-chunk tiles (prepare -> scan)
  size_t xhat_off, sfin_off, xfin_off, sin_off;
  size_t total_bytes;
};

// Segmentation aims for one scan workgroup (one head-segment) per CU of
// the 256 on MI355X, and is used only when B*H heads leave at least
// kMinSegsPerHead segments per head to fill it.
#ifndef GDN_SCAN_TARGET_BLOCKS
#define GDN_SCAN_TARGET_BLOCKS 256
#endif
constexpr int kScanTargetBlocks = GDN_SCAN_TARGET_BLOCKS;
constexpr int kMinSegsPerHead = 4;
constexpr int kMinSegChunks = 8;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Every argument check of gdn_prefill except the workspace's (no HIP call);
// returns a gdn_status.
int prefill_args(const void* q, const void* k, const void* v, const float* alpha,
                 const float* beta, const float* S0, const void* o, const float* ST,
                 int B, int T, int H, int dk, int dv, int in_dtype, int out_dtype);

// Plan for bf16 inputs and outputs (the only case that is segmented); the
// workspace it sizes also covers every other dtype combination.
inline PrefillPlan plan_prefill(int B, int T, int H, int dk, int dv) {
  PrefillPlan p{};
  p.nchunks = (T + kChunk - 1) / kChunk;
  p.chunk_bytes = (size_t)B * H * p.nchunks * kChunkWsFloats * sizeof(float);
  p.nseg = 1;
  p.seg_chunks = p.nchunks;
  const int per_head_target = kScanTargetBlocks / (B * H > 0 ? B * H : 1);
  if (per_head_target >= kMinSegsPerHead && p.nchunks >= 2 * kMinSegChunks) {
    int nseg = per_head_target;
    nseg = nseg < p.nchunks / kMinSegChunks ? nseg : p.nchunks / kMinSegChunks;
    if (nseg > 1) {
      p.seg_chunks = (p.nchunks + nseg - 1) / nseg;
      p.nseg = (p.nchunks + p.seg_chunks - 1) / p.seg_chunks;
    }
  }
  size_t off = align256(p.chunk_bytes);
  if (p.nseg > 1) {
    const size_t BH = (size_t)B * H;
    p.xhat_off = off;
    off = align256(off + BH * T * dk * 2);
    p.sfin_off = off;
    off = align256(off + BH * p.nseg * dv * dk * 4);
    p.xfin_off = off;
    off = align256(off + BH * p.nseg * dk * dk * 4);
    p.sin_off = off;
    off = align256(off + BH * p.nseg * dv * dk * 2);
  }
  p.total_bytes = off;
  return p;
}

hipError_t launch_decode(const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta,
                         const float* S_in, float* S_out, void* o, int BH,
                         int H, int dk, int dv, int in_dtype, int out_dtype,
                         const QkArgs& qa, hipStream_t stream);

// write_pl: also store the lo part of P (read only when outputs are fp32).
// scan_forms_p (bf16 inputs, segmented scan only): store no P; the scan forms
// it from its K and Q tiles and two per-token exponent rows written instead.
hipError_t launch_prefill_prepare(const void* q, const void* k,
                                  const float* alpha, const float* beta,
                                  float* ws, int B, int T, int H, int dk,
                                  int in_dtype, bool write_pl, bool scan_forms_p,
                                  const QkArgs& qa, hipStream_t stream);

// Phase 1 (+ phases 2 and 3 when the plan segments the sequence).  `ws` is
// the whole workspace (per-chunk tiles first, then the segment buffers).
hipError_t launch_prefill_scan(const void* q, const void* k, const void* v,
                               const float* S0, void* o, float* ST, void* ws,
                               int B, int T, int H, int dk, int dv,
                               int in_dtype, int out_dtype, hipStream_t stream);

// Rank-r truncation S <- U_r U_r^T S of BH states [dv, dk] in place, and
// er[BH] (may be NULL) = stable rank of the result; U is a workspace of
// BH * min(dv, dk) * dv doubles (unused when r >= min(dv, dk)).
hipError_t launch_truncate(float* S, int BH, int dv, int dk, int r, float* er,
                           double* U, hipStream_t stream);

hipError_t launch_state_fill(const float* S0, float* ST, size_t n,
                             hipStream_t stream);

// DRRQR channel selection on host memory (fp64): 0, or 1 if rank(M) < k.
int drrqr_select(const double* M, int rows, int n, int k, double f, int max_swaps,
                 int* selected, int* swaps_out, double* rho_out);

// The generalised gates (per-key-channel retention alpha [B,T,H,dk], erase
// gate b [B,T,H,dk], write gate w [B,T,H,dv]) in recurrent form, T >= 1.
hipError_t launch_gated_recurrent(const void* q, const void* k, const void* v,
                                  const float* alpha, const float* bgate,
                                  const float* wgate, const float* S0, float* ST,
                                  void* o, int B, int T, int H, int dk, int dv,
                                  int in_dtype, int out_dtype, hipStream_t stream);

// Backward pass of the gated delta rule in recurrent form: workspace sizing
// (floats; ckpt_floats gets the checkpoint part) and the launch (two kernels).
size_t backward_ws_floats(int B, int T, int H, int dk, int dv, size_t* ckpt_floats);
hipError_t launch_backward(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, const void* dO,
                           const float* dST, float* dq, float* dk, float* dv_out,
                           float* dalpha, float* dbeta, float* dS0, int B, int T, int H,
                           int dkk, int dv, int in_dtype, float* ws, hipStream_t stream);

// The backward pass in chunked form (bf16 inputs): workspace bytes (the
// prepare phase's tiles, T itself, the state at the start and the state
// gradient at the end of every chunk) and the launch (prepare, forward
// sweep, backward chain, chunk gradients).
size_t backward_chunked_ws_bytes(int B, int T, int H, int dk, int dv);
hipError_t launch_backward_chunked(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta, const float* S0,
                                   const void* d_o, const float* dST, float* dq, float* dkey,
                                   float* dval, float* dalpha, float* dbeta, float* dS0,
                                   int B, int T, int H, int dk, int dv, void* workspace,
                                   hipStream_t stream);
// The generalised gates in chunked form (bf16 inputs): workspace bytes and
// the launch (prepare, then the scan).
size_t gated_chunked_ws_bytes(int B, int T, int H, int dk);
hipError_t launch_gated_chunked(const void* q, const void* k, const void* v,
                                const float* alpha, const float* bgate, const float* wgate,
                                const float* S0, float* ST, void* o, int B, int T, int H,
                                int dk, int dv, int out_dtype, void* workspace,
                                hipStream_t stream);
// The backward pass's forward sweep: the prefill scan storing the state at
// the start of every chunk (bf16 inputs; ws holds the prepare tiles).
hipError_t launch_scan_states(const void* k, const void* v, const float* S0,
                              const float* ws, float* Sc, int B, int T, int H,
                              int dk, int dv, hipStream_t stream);

}  // namespace gdn
