// Exported C ABI of libgdn (declared in include/gdn.h): argument validation,
// workspace sizing and dispatch to the gfx950 kernels.  Validation happens
// before any HIP call, so argument errors can be tested without a GPU.
#include <stdint.h>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

bool dtype_ok(int d) { return d == GDN_F32 || d == GDN_BF16; }
bool dims_ok(int dk, int dv) {
  return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}
bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}
int to_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_EHIP; }

size_t prefill_ws_bytes(int B, int T, int H, int dk, int dv) {
  if (B <= 0 || H <= 0 || T <= 0) return 0;
  return gdn::plan_prefill(B, T, H, dk, dv).total_bytes;
}

// Common shape/dtype checks of the prefill entry points.
int check_prefill_shape(int B, int T, int H, int dk, int dv, int in_dtype,
                        int out_dtype) {
  if (B <= 0 || H <= 0 || T < 0) return GDN_EINVAL;
  if (B > 65535 || H > 65535) return GDN_EINVAL;     // grid y/z limits
  if ((long long)B * H * (dv / 16) > 0x7FFFFFFFLL) return GDN_EINVAL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GDN_ESHAPE;
  if (!dims_ok(dk, dv)) return GDN_ESHAPE;
  return GDN_OK;
}

// Checks of the input-path arguments: without channels the rows are dk
// wide; with them any width up to 2^20, the index table 16-byte aligned.
int check_qk(int dk, int dk_in, const int* channels, int l2norm) {
  if (l2norm != 0 && l2norm != 1) return GDN_EINVAL;
  if (channels == nullptr) return dk_in == dk ? GDN_OK : GDN_ESHAPE;
  if (dk_in < 1 || dk_in > (1 << 20)) return GDN_ESHAPE;
  if (!aligned(channels, 16)) return GDN_EINVAL;
  return GDN_OK;
}

// Bytes of workspace of a prefill with the input path: the plain prefill's,
// then (with a channel subset) the gathered q/k copy.
size_t prefill_qk_ws_bytes(int B, int T, int H, int dk, int dv, int in_dtype,
                           bool gather) {
  const size_t base = prefill_ws_bytes(B, T, H, dk, dv);
  if (base == 0 || !gather) return base;
  return gdn::align256(base) + gdn::qk_copy_bytes(B, T, H, dk, in_dtype);
}

// Validation and launch of the prepare phase.  fp32 outputs: also store the
// lo part of P, which only the fp32-output scan reads.  q/k rows read whole
// need 16-byte alignment; gathered ones only their element's.
int prepare_checked(const void* q, const void* k, const float* alpha,
                    const float* beta, int B, int T, int H, int dk, int dv,
                    int in_dtype, int out_dtype, const gdn::QkArgs& qa,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  if (T == 0) return GDN_OK;
  if (!q || !k || !alpha || !beta) return GDN_EINVAL;
  const uintptr_t qa_align = qa.chan ? (in_dtype == GDN_BF16 ? 2 : 4) : 16;
  if (!aligned(q, qa_align) || !aligned(k, qa_align) || !aligned(alpha, 4) ||
      !aligned(beta, 4))
    return GDN_EINVAL;
  if (!workspace || !aligned(workspace, 16)) return GDN_EWORKSPACE;
  if (workspace_bytes < prefill_qk_ws_bytes(B, T, H, dk, dv, in_dtype, qa.chan != nullptr))
    return GDN_EWORKSPACE;
  // the segmented scan (bf16 in and out) forms P itself
  const bool scan_forms_p = gdn::plan_prefill(B, T, H, dk, dv).nseg > 1 &&
                            in_dtype == GDN_BF16 && out_dtype == GDN_BF16;
  return to_status(gdn::launch_prefill_prepare(
      q, k, alpha, beta, static_cast<float*>(workspace), B, T, H, dk, in_dtype,
      out_dtype == GDN_F32, scan_forms_p, qa, static_cast<hipStream_t>(stream)));
}

// The scan's checks that do not depend on q/k (shared by the prefills).
int check_scan_rest(const void* v, void* o, const float* S0, const float* ST,
                    int B, int H, int dk, int dv) {
  if (!v || !o) return GDN_EINVAL;
  if (!aligned(v, 16) || !aligned(o, 16)) return GDN_EINVAL;
  if ((S0 && !aligned(S0, 16)) || (ST && !aligned(ST, 16))) return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  if (ST && S0 && ST != S0 && (ST < S0 + nstate && S0 < ST + nstate))
    return GDN_EINVAL;                               // partial overlap
  return GDN_OK;
}

}  // namespace

namespace gdn {

// Every argument check of gdn_prefill except the workspace's; no HIP call.
int prefill_args(const void* q, const void* k, const void* v, const float* alpha,
                 const float* beta, const float* S0, const void* o, const float* ST,
                 int B, int T, int H, int dk, int dv, int in_dtype, int out_dtype) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  if ((S0 && !aligned(S0, 16)) || (ST && !aligned(ST, 16))) return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  if (ST && S0 && ST != S0 && (ST < S0 + nstate && S0 < ST + nstate))
    return GDN_EINVAL;                               // partial overlap
  if (T == 0) return GDN_OK;
  if (!q || !k || !v || !o || !alpha || !beta) return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(alpha, 4) || !aligned(beta, 4))
    return GDN_EINVAL;
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_EINVAL: return "GDN_EINVAL: invalid argument (null pointer, bad size or misaligned buffer)";
    case GDN_ESHAPE: return "GDN_ESHAPE: unsupported head size or dtype (dk, dv in {64, 128}; f32 or bf16)";
    case GDN_EWORKSPACE: return "GDN_EWORKSPACE: workspace missing or too small (gdn_*_workspace_bytes()); for gdn_prefill_noalloc, the sizes need more than GDN_NOALLOC_SCRATCH_BYTES";
    case GDN_EHIP: return "GDN_EHIP: HIP launch failed";
    default: return "GDN_UNKNOWN_STATUS";
  }
}

const char* gdn_version(void) { return "0.1.0"; }

size_t gdn_prefill_workspace_bytes(int B, int T, int H, int dk, int dv) {
  if (!dims_ok(dk, dv)) return 0;
  return prefill_ws_bytes(B, T, H, dk, dv);
}

int gdn_prefill_segments(int B, int T, int H, int dk, int dv, int in_dtype,
                         int out_dtype, int* seg_chunks) {
  if (check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype) != GDN_OK) return 0;
  if (T == 0) {
    if (seg_chunks) *seg_chunks = 0;
    return 1;
  }
  const gdn::PrefillPlan p = gdn::plan_prefill(B, T, H, dk, dv);
  const bool seg = p.nseg > 1 && in_dtype == GDN_BF16 && out_dtype == GDN_BF16;
  if (seg_chunks) *seg_chunks = seg ? p.seg_chunks : p.nchunks;
  return seg ? p.nseg : 1;
}

int gdn_prefill_prepare(const void* q, const void* k, const float* alpha,
                        const float* beta, int B, int T, int H, int dk, int dv,
                        int in_dtype, int out_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return prepare_checked(q, k, alpha, beta, B, T, H, dk, dv, in_dtype, out_dtype,
                         gdn::qk_identity(dk), workspace, workspace_bytes, stream);
}

int gdn_prefill_scan(const void* q, const void* k, const void* v,
                     const float* S0, void* o, float* ST, int B, int T, int H,
                     int dk, int dv, int in_dtype, int out_dtype,
                     void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  if ((S0 && !aligned(S0, 16)) || (ST && !aligned(ST, 16))) return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  if (ST && S0 && ST != S0 &&
      (ST < S0 + nstate && S0 < ST + nstate))
    return GDN_EINVAL;                               // partial overlap
  if (T == 0)
    return to_status(gdn::launch_state_fill(S0, ST, nstate,
                                            static_cast<hipStream_t>(stream)));
  if (!q || !k || !v || !o) return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16))
    return GDN_EINVAL;
  if (!workspace || !aligned(workspace, 16)) return GDN_EWORKSPACE;
  if (workspace_bytes < prefill_ws_bytes(B, T, H, dk, dv)) return GDN_EWORKSPACE;
  return to_status(gdn::launch_prefill_scan(
      q, k, v, S0, o, ST, workspace, B, T, H, dk, dv,
      in_dtype, out_dtype, static_cast<hipStream_t>(stream)));
}

int gdn_prefill(const void* q, const void* k, const void* v,
                const float* alpha, const float* beta, const float* S0,
                void* o, float* ST, int B, int T, int H, int dk, int dv,
                int in_dtype, int out_dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  if (T > 0) {
    // validate everything the scan needs before launching the prepare
    if (!q || !k || !v || !o || !alpha || !beta) return GDN_EINVAL;
    if (!aligned(v, 16) || !aligned(o, 16)) return GDN_EINVAL;
    if ((S0 && !aligned(S0, 16)) || (ST && !aligned(ST, 16)))
      return GDN_EINVAL;
    const size_t nstate = (size_t)B * H * dv * dk;
    if (ST && S0 && ST != S0 && (ST < S0 + nstate && S0 < ST + nstate))
      return GDN_EINVAL;
    st = prepare_checked(q, k, alpha, beta, B, T, H, dk, dv, in_dtype,
                         out_dtype, gdn::qk_identity(dk), workspace,
                         workspace_bytes, stream);
    if (st != GDN_OK) return st;
  }
  return gdn_prefill_scan(q, k, v, S0, o, ST, B, T, H, dk, dv, in_dtype,
                          out_dtype, workspace, workspace_bytes, stream);
}

int gdn_decode_step(const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, const float* S_in,
                    float* S_out, void* o, int B, int H, int dk, int dv,
                    int in_dtype, int out_dtype, void* stream) {
  if (B <= 0 || H <= 0) return GDN_EINVAL;
  if ((long long)B * H * dv > 0x7FFFFFFFLL) return GDN_EINVAL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GDN_ESHAPE;
  if (!dims_ok(dk, dv)) return GDN_ESHAPE;
  if (!q || !k || !v || !alpha || !beta || !S_in || !S_out || !o)
    return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(S_in, 16) || !aligned(S_out, 16) ||
      !aligned(alpha, 4) || !aligned(beta, 4))
    return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  if (S_out != S_in && S_out < S_in + nstate && S_in < S_out + nstate)
    return GDN_EINVAL;                               // partial overlap
  return to_status(gdn::launch_decode(q, k, v, alpha, beta, S_in, S_out, o,
                                      B * H, H, dk, dv, in_dtype, out_dtype,
                                      gdn::qk_identity(dk),
                                      static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_qk_workspace_bytes(int B, int T, int H, int dk, int dv,
                                      int in_dtype, int gather) {
  if (!dims_ok(dk, dv) || !dtype_ok(in_dtype)) return 0;
  return prefill_qk_ws_bytes(B, T, H, dk, dv, in_dtype, gather != 0);
}

int gdn_prefill_qk(const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* S0,
                   void* o, float* ST, int B, int T, int H, int dk, int dv,
                   int dk_in, const int* channels, int l2norm, float q_scale,
                   int in_dtype, int out_dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  st = check_qk(dk, dk_in, channels, l2norm);
  if (st != GDN_OK) return st;
  if (T == 0) {
    // no token: the final state is the initial one (q, k never read)
    return gdn_prefill_scan(q, k, v, S0, o, ST, B, T, H, dk, dv, in_dtype,
                            out_dtype, workspace, workspace_bytes, stream);
  }
  st = check_scan_rest(v, o, S0, ST, B, H, dk, dv);
  if (st != GDN_OK) return st;
  gdn::QkArgs qa{channels, dk_in, l2norm, q_scale, nullptr};
  if (channels) {
    if (!workspace) return GDN_EWORKSPACE;
    qa.qk_out = static_cast<char*>(workspace) +
                gdn::align256(prefill_ws_bytes(B, T, H, dk, dv));
  }
  st = prepare_checked(q, k, alpha, beta, B, T, H, dk, dv, in_dtype,
                       out_dtype, qa, workspace, workspace_bytes, stream);
  if (st != GDN_OK) return st;
  // the scan reads the kept channels: the gathered copy, or q/k themselves
  const void* qs = q;
  const void* ks = k;
  if (channels) {
    ks = qa.qk_out;
    qs = static_cast<const char*>(qa.qk_out) +
         gdn::qk_copy_bytes(B, T, H, dk, in_dtype) / 2;
  }
  return to_status(gdn::launch_prefill_scan(
      qs, ks, v, S0, o, ST, workspace, B, T, H, dk, dv, in_dtype, out_dtype,
      static_cast<hipStream_t>(stream)));
}

int gdn_decode_step_qk(const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta,
                       const float* S_in, float* S_out, void* o, int B, int H,
                       int dk, int dv, int dk_in, const int* channels,
                       int l2norm, float q_scale, int in_dtype, int out_dtype,
                       void* stream) {
  if (B <= 0 || H <= 0) return GDN_EINVAL;
  if ((long long)B * H * dv > 0x7FFFFFFFLL) return GDN_EINVAL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GDN_ESHAPE;
  if (!dims_ok(dk, dv)) return GDN_ESHAPE;
  int st = check_qk(dk, dk_in, channels, l2norm);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !alpha || !beta || !S_in || !S_out || !o)
    return GDN_EINVAL;
  const uintptr_t qk_align = channels ? (in_dtype == GDN_BF16 ? 2 : 4) : 16;
  if (!aligned(q, qk_align) || !aligned(k, qk_align) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(S_in, 16) || !aligned(S_out, 16) ||
      !aligned(alpha, 4) || !aligned(beta, 4))
    return GDN_EINVAL;
  if ((long long)B * H * dk_in > 0x7FFFFFFFLL) return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  if (S_out != S_in && S_out < S_in + nstate && S_in < S_out + nstate)
    return GDN_EINVAL;                               // partial overlap
  const gdn::QkArgs qa{channels, dk_in, l2norm, q_scale, nullptr};
  return to_status(gdn::launch_decode(q, k, v, alpha, beta, S_in, S_out, o,
                                      B * H, H, dk, dv, in_dtype, out_dtype,
                                      qa, static_cast<hipStream_t>(stream)));
}

int gdn_gated_recurrent(const void* q, const void* k, const void* v,
                        const float* alpha, const float* b, const float* w,
                        const float* S0, void* o, float* ST, int B, int T,
                        int H, int dk, int dv, int in_dtype, int out_dtype,
                        void* stream) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  if ((S0 && !aligned(S0, 16)) || (ST && !aligned(ST, 16))) return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  if (ST && S0 && ST != S0 && (ST < S0 + nstate && S0 < ST + nstate))
    return GDN_EINVAL;                               // partial overlap
  if (T == 0)
    return to_status(gdn::launch_state_fill(S0, ST, nstate,
                                            static_cast<hipStream_t>(stream)));
  if (!q || !k || !v || !alpha || !b || !w || !o) return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(alpha, 16) ||
      !aligned(b, 16) || !aligned(v, in_dtype == GDN_BF16 ? 2 : 4) ||
      !aligned(w, 4) || !aligned(o, out_dtype == GDN_BF16 ? 2 : 4))
    return GDN_EINVAL;
  return to_status(gdn::launch_gated_recurrent(
      q, k, v, alpha, b, w, S0, ST, o, B, T, H, dk, dv, in_dtype, out_dtype,
      static_cast<hipStream_t>(stream)));
}

size_t gdn_gated_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int in_dtype) {
  if (check_prefill_shape(B, T, H, dk, dv, in_dtype, GDN_F32) != GDN_OK || T == 0) return 0;
  return in_dtype == GDN_BF16 ? gdn::gated_chunked_ws_bytes(B, T, H, dk) : 0;
}

int gdn_gated_prefill(const void* q, const void* k, const void* v, const float* alpha,
                      const float* b, const float* w, const float* S0, void* o, float* ST,
                      int B, int T, int H, int dk, int dv, int in_dtype, int out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  if (in_dtype != GDN_BF16 || T == 0)      // fp32 inputs (and T == 0): the recurrent form
    return gdn_gated_recurrent(q, k, v, alpha, b, w, S0, o, ST, B, T, H, dk, dv, in_dtype,
                               out_dtype, stream);
  if ((S0 && !aligned(S0, 16)) || (ST && !aligned(ST, 16))) return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  if (ST && S0 && ST != S0 && (ST < S0 + nstate && S0 < ST + nstate))
    return GDN_EINVAL;                               // partial overlap
  if (!q || !k || !v || !alpha || !b || !w || !o) return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 2) || !aligned(alpha, 16) ||
      !aligned(b, 16) || !aligned(w, 4) || !aligned(o, out_dtype == GDN_BF16 ? 2 : 4))
    return GDN_EINVAL;
  if (!workspace || !aligned(workspace, 16)) return GDN_EWORKSPACE;
  if (workspace_bytes < gdn::gated_chunked_ws_bytes(B, T, H, dk)) return GDN_EWORKSPACE;
  return to_status(gdn::launch_gated_chunked(q, k, v, alpha, b, w, S0, ST, o, B, T, H, dk, dv,
                                             out_dtype, workspace,
                                             static_cast<hipStream_t>(stream)));
}

size_t gdn_backward_workspace_bytes(int B, int T, int H, int dk, int dv, int in_dtype) {
  if (check_prefill_shape(B, T, H, dk, dv, in_dtype, GDN_F32) != GDN_OK || T == 0) return 0;
  return in_dtype == GDN_BF16 ? gdn::backward_chunked_ws_bytes(B, T, H, dk, dv)
                              : gdn::backward_ws_floats(B, T, H, dk, dv, nullptr) * sizeof(float);
}

int gdn_backward(const void* q, const void* k, const void* v, const float* alpha,
                 const float* beta, const float* S0, const void* d_o, const float* dST,
                 float* dq, float* dkey, float* dval, float* dalpha, float* dbeta,
                 float* dS0, int B, int T, int H, int dk, int dv, int in_dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_prefill_shape(B, T, H, dk, dv, in_dtype, GDN_F32);
  if (st != GDN_OK) return st;
  if ((long long)B * H * T * (2 * dk + 2) / 256 >= 0x7FFFFFFFLL) return GDN_EINVAL;
  if ((S0 && !aligned(S0, 16)) || (dST && !aligned(dST, 16)) || (dS0 && !aligned(dS0, 16)))
    return GDN_EINVAL;
  const size_t nstate = (size_t)B * H * dv * dk;
  auto partial = [&](const float* x) {
    return x && dS0 && x != dS0 && (x < dS0 + nstate && dS0 < x + nstate);
  };
  if (partial(dST) || partial(S0)) return GDN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return dS0 ? to_status(gdn::launch_state_fill(dST, dS0, nstate, s)) : GDN_OK;
  if (!q || !k || !v || !alpha || !beta || !d_o || !dq || !dkey || !dval || !dalpha || !dbeta)
    return GDN_EINVAL;
  const uintptr_t ev = in_dtype == GDN_BF16 ? 2 : 4;
  const uintptr_t eo = in_dtype == GDN_BF16 ? 16 : 4;     // bf16 d_o rows are read in 16-byte units
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, ev) || !aligned(d_o, eo) ||
      !aligned(alpha, 4) || !aligned(beta, 4) || !aligned(dq, 4) || !aligned(dkey, 4) ||
      !aligned(dval, 4) || !aligned(dalpha, 4) || !aligned(dbeta, 4))
    return GDN_EINVAL;
  if (!workspace || !aligned(workspace, 16)) return GDN_EWORKSPACE;
  if (workspace_bytes < gdn_backward_workspace_bytes(B, T, H, dk, dv, in_dtype))
    return GDN_EWORKSPACE;
  if (in_dtype == GDN_BF16)
    return to_status(gdn::launch_backward_chunked(q, k, v, alpha, beta, S0, d_o, dST, dq, dkey,
                                                  dval, dalpha, dbeta, dS0, B, T, H, dk, dv,
                                                  workspace, s));
  return to_status(gdn::launch_backward(q, k, v, alpha, beta, S0, d_o, dST, dq, dkey, dval,
                                        dalpha, dbeta, dS0, B, T, H, dk, dv, in_dtype,
                                        static_cast<float*>(workspace), s));
}

int gdn_drrqr_select(const double* M, int rows, int n, int k, double f,
                     int max_swaps, int* selected, int* swaps, double* rho_max) {
  if (!M || !selected) return GDN_EINVAL;
  if (n < 2 || n > 4096 || k < 1 || k >= n || rows < n || max_swaps < 0)
    return GDN_EINVAL;
  if (!(f >= 1.0)) return GDN_EINVAL;
  return gdn::drrqr_select(M, rows, n, k, f, max_swaps, selected, swaps, rho_max) == 0
             ? GDN_OK
             : GDN_EINVAL;
}

size_t gdn_truncate_workspace_bytes(int BH, int dv, int dk) {
  if (BH <= 0 || !dims_ok(dk, dv)) return 0;
  return (size_t)BH * (dv < dk ? dv : dk) * dv * sizeof(double);
}

int gdn_truncate_rank(float* S, int BH, int dv, int dk, int r, float* er_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (BH <= 0 || BH > 65535 || r < 1) return GDN_EINVAL;
  if (!dims_ok(dk, dv)) return GDN_ESHAPE;
  if (!S || !aligned(S, 16)) return GDN_EINVAL;
  if (er_out && !aligned(er_out, 4)) return GDN_EINVAL;
  const bool project = r < (dv < dk ? dv : dk);
  if (project) {
    if (!workspace || !aligned(workspace, 16)) return GDN_EWORKSPACE;
    if (workspace_bytes < gdn_truncate_workspace_bytes(BH, dv, dk))
      return GDN_EWORKSPACE;
  }
  return to_status(gdn::launch_truncate(
      S, BH, dv, dk, r, er_out, static_cast<double*>(workspace),
      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
