// The gated delta rule with generalised gates, in recurrent form, on gfx950.
//
// Per head and token ("Linear Attention Architectures" reading notes,
// paper Sec. 3.4 Kimi Delta Attention and paper Sec. 3.5 Gated DeltaNet-2):
//     S~  = S_{t-1} diag(alpha_t)        per-key-channel retention, applied on
//                                        the key-feature side of the state
//     e   = b_t * k_t                    direction the erase reads (key side)
//     z   = w_t * v_t                    content written (value side)
//     S_t = S~ (I - e k_t^T) + z k_t^T   erase and write both along k_t
//     o_t = S_t q_t
// b = w = beta * 1 is Kimi Delta Attention, and with alpha = a * 1 as well
// the gated delta rule of the chunked kernels.
//
// Per state row s_i (value channel i, dk floats):
//     s~ = s_i * alpha                p = s~ . e       r = s~ . q
//     u  = w_i v_i - p
//     s_i' = s~ + u k                 o_i = r + u (k . q)
// Rows evolve independently, so one wave carries 4 NG rows of one head
// through all T tokens with the rows in registers (16 lanes per row, 4 dk/64
// floats each; the dot products are 16-lane DPP sums).  The inputs of the
// next P tokens are loaded ahead into a register ring, and the outputs of
// a group of P tokens are stored together after it, so the loads of later
// tokens are not drained by the compiler's wait for a store.  T == 1 is the
// decode step: a single streaming pass over the state, HBM-bound like the
// plain decode kernel; it runs the P = 1 instance, whose small register
// footprint keeps many waves (and bytes) in flight, and at dk=64 with
// enough waves it paces its state stores as the plain decode kernel does
// (every row formed first, then one store at a time, each waited for).
// Sequences of bf16 inputs have a chunked form (gdn_gated_chunk.hip); this
// recurrent form serves fp32 inputs and is bound by the per-token latency
// of the dependent chain.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

template <int F, int NG>
struct TokIn {
  float4 k[F], q[F], a[F], b[F];
  float v[NG], w[NG];
};

}  // namespace

// P: tokens whose inputs are in flight (a register ring); NG: groups of 4
// rows per wave (the token's key-side inputs are loaded once for all of
// them); HAS_S0: an initial state is given (a compile-time choice keeps the
// state loads out of a branch, after which the compiler's waits would drain
// every load in flight); WPB: waves per workgroup; PACED: the final state is
// stored one 1 KB group at a time, each store waited for.
template <int DK, int P, int NG, bool HAS_S0, typename TIn, typename TOut, int WPB = 4,
          bool PACED = false>
__global__ __launch_bounds__(64 * WPB) void gated_recurrent_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ bgate, const float* __restrict__ wgate,
    const float* S0, float* ST, TOut* __restrict__ o, int BH, int H, int T,
    int dv) {
  // The one-token instance (P = 1) is launched only for T == 1; fixing T
  // there leaves its step without a branch.  With the run-time T (a token
  // loop, a guarded prefetch) the decode took 24.2 instead of 23.4 us at
  // B=64, H=16, dk=dv=128.
  if constexpr (P == 1) T = 1;
  constexpr int F = DK / 64;            // float4 per lane per row
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * WPB + (threadIdx.x >> 6);
  const int slices = dv / (4 * NG);
  const int head = wave / slices;
  if (head >= BH) return;
  const int row0 = (wave - head * slices) * 4 * NG + (lane >> 4);   // row of group 0
  const int sub = lane & 15;
  const int b = head / H, h = head - b * H;

  // inputs of token t (0 <= t < T)
  auto load_tok = [&](TokIn<F, NG>& x, int t) {
    const size_t tok = ((size_t)b * T + t) * H + h;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int c = 64 * f + 4 * sub;
      x.k[f] = load4(k + tok * DK + c);
      x.q[f] = load4(q + tok * DK + c);
      x.a[f] = *reinterpret_cast<const float4*>(alpha + tok * DK + c);
      x.b[f] = *reinterpret_cast<const float4*>(bgate + tok * DK + c);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      x.v[g] = load1(v + tok * dv + row0 + 4 * g);
      x.w[g] = wgate[tok * dv + row0 + 4 * g];
    }
  };

  TokIn<F, NG> ring[P];
#pragma unroll
  for (int i = 0; i < P; ++i) load_tok(ring[i], min(i, T - 1));

  // rows row0 + 4 g of the state, lane's columns 64 f + 4 sub .. + 3; loaded
  // after the first tokens' inputs, which the first step needs first
  // (vector-memory loads return in order)
  floatx4 s[NG][F];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const size_t srow = ((size_t)head * dv + row0 + 4 * g) * DK;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      if constexpr (HAS_S0) {
        s[g][f] = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(S0 + srow + 64 * f + 4 * sub));
      } else {
        s[g][f] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }


  // Tokens run in groups of SP = P * R (R ring turns); the outputs of a
  // group are stored after it, so the compiler's drain of every load in
  // flight (which it inserts at the first load wait after a store) happens
  // once per group instead of once per ring turn.
  constexpr int R = P > 1 ? 4 : 1;
  constexpr int SP = P * R;
  for (int t0 = 0; t0 < T; t0 += SP) {
    float ob[SP][NG];
#pragma unroll
    for (int j = 0; j < SP; ++j) {
      const int i = j % P;                // ring slot of token t0 + j
      const TokIn<F, NG> x = ring[i];
      // unconditional (clamped) prefetch: a load under a branch would make
      // the compiler's waits after it drain every load in flight.  The
      // one-token instance has no next token.
      if constexpr (P > 1) load_tok(ring[i], min(t0 + j + P, T - 1));
#pragma unroll
      for (int g = 0; g < NG; ++g) ob[j][g] = 0.f;
      if (t0 + j >= T) continue;          // past the last token (uniform per wave)
      float kq = 0.f;
#pragma unroll
      for (int f = 0; f < F; ++f)
        kq += x.k[f].x * x.q[f].x + x.k[f].y * x.q[f].y + x.k[f].z * x.q[f].z +
              x.k[f].w * x.q[f].w;
      kq = sum16(kq);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float p = 0.f, r = 0.f;
        floatx4 sa[F];
#pragma unroll
        for (int f = 0; f < F; ++f) {
          sa[f] = floatx4{s[g][f][0] * x.a[f].x, s[g][f][1] * x.a[f].y,
                          s[g][f][2] * x.a[f].z, s[g][f][3] * x.a[f].w};
          p += sa[f][0] * (x.b[f].x * x.k[f].x) + sa[f][1] * (x.b[f].y * x.k[f].y) +
               sa[f][2] * (x.b[f].z * x.k[f].z) + sa[f][3] * (x.b[f].w * x.k[f].w);
          r += sa[f][0] * x.q[f].x + sa[f][1] * x.q[f].y + sa[f][2] * x.q[f].z +
               sa[f][3] * x.q[f].w;
        }
        p = sum16(p);
        r = sum16(r);
        const float u = x.w[g] * x.v[g] - p;
#pragma unroll
        for (int f = 0; f < F; ++f)
          s[g][f] = floatx4{sa[f][0] + u * x.k[f].x, sa[f][1] + u * x.k[f].y,
                            sa[f][2] + u * x.k[f].z, sa[f][3] + u * x.k[f].w};
        ob[j][g] = r + u * kq;
      }
    }
    if (sub == 0) {
#pragma unroll
      for (int j = 0; j < SP; ++j)
#pragma unroll
        for (int g = 0; g < NG; ++g)
          if (t0 + j < T)
            store1(o + (((size_t)b * T + t0 + j) * H + h) * dv + row0 + 4 * g, ob[j][g]);
    }
  }

  if (ST != nullptr) {
    // paced: nothing of the arithmetic is scheduled between the waits
    if constexpr (PACED) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const size_t srow = ((size_t)head * dv + row0 + 4 * g) * DK;
#pragma unroll
      for (int f = 0; f < F; ++f) {
        __builtin_nontemporal_store(s[g][f],
                                    reinterpret_cast<floatx4*>(ST + srow + 64 * f + 4 * sub));
        if constexpr (PACED) {
          if (g + 1 < NG || f + 1 < F) wait_vmem();
        }
      }
    }
  }
}

constexpr long kSimds = 1024;   // 256 CUs x 4 SIMDs
constexpr long kPaced = 4096;   // 16 resident waves on each of 256 CUs

hipError_t launch_gated_recurrent(const void* q, const void* k, const void* v,
                                  const float* alpha, const float* bgate,
                                  const float* wgate, const float* S0, float* ST,
                                  void* o, int B, int T, int H, int dk, int dv,
                                  int in_dtype, int out_dtype, hipStream_t stream) {
  const int BH = B * H;
  // T == 1 (decode), measured at B=64, H=16, dv=128 over 18 rotating random
  // state sets with fresh inputs per step: at dk=64, 32 rows per wave with
  // paced stores and one wave per workgroup once the grid has kPaced such
  // waves (11.74 us per step, against 11.87 with 4 waves per workgroup,
  // 12.73 for the same layout unpaced and 13.42 for 16 unpaced rows per
  // wave); else 16 rows per wave.  At dk=128, 8 rows per wave (24.15 us,
  // against 25.0 with 16, 27.6 with 4, and 25.2-25.3 paced with 8 or 16).
  // A token's key-side inputs (k, q and the two per-channel gates) are read
  // once per wave, i.e. once per 8-32 rows.  Longer
  // sequences: a ring of 4 tokens in flight (at B=8, T=4096, dk=64, 4 rows
  // per wave: 2.8 ms against 3.7 ms with 2), and as many rows per wave as
  // still leave one wave per SIMD: the sequence form is bound by VALU issue,
  // and the per-token work shared by a wave's rows (k.q, b * k, the
  // addresses and conversions) is then spread over more rows (same shape:
  // 2.68 ms with 4 rows, 1.67 ms with 8, 1.64 ms with 16 per wave).
#define GDN_GATED_K(DK, P, NG, S0_, TI, TO, W, PC)                                            \
  hipLaunchKernelGGL((gated_recurrent_kernel<DK, P, NG, S0_, TI, TO, W, PC>),                 \
                     dim3((unsigned)(((long)BH * (dv / (4 * NG)) + W - 1) / W)), dim3(64 * W), \
                     0, stream, static_cast<const TI*>(q), static_cast<const TI*>(k),          \
                     static_cast<const TI*>(v), alpha, bgate, wgate, S0, ST,                   \
                     static_cast<TO*>(o), BH, H, T, dv)
#define GDN_GATED_P(DK, P, NG, TI, TO, W, PC)                          \
  do {                                                                 \
    if (S0 != nullptr) GDN_GATED_K(DK, P, NG, true, TI, TO, W, PC);    \
    else GDN_GATED_K(DK, P, NG, false, TI, TO, W, PC);                 \
  } while (0)
#define GDN_GATED(DK, TI, TO)                                                                 \
  do {                                                                                        \
    if (T == 1) {                                                                             \
      if constexpr (DK == 64) {                                                               \
        if ((long)BH * dv / 32 >= kPaced) GDN_GATED_P(DK, 1, 8, TI, TO, 1, true);            \
        else GDN_GATED_P(DK, 1, 4, TI, TO, 4, false);                                        \
      } else {                                                                                \
        GDN_GATED_P(DK, 1, 2, TI, TO, 4, false);                                              \
      }                                                                                       \
    } else if ((long)BH * dv / 16 >= kSimds) GDN_GATED_P(DK, 4, 4, TI, TO, 4, false);        \
    else if ((long)BH * dv / 8 >= kSimds) GDN_GATED_P(DK, 4, 2, TI, TO, 4, false);           \
    else GDN_GATED_P(DK, 4, 1, TI, TO, 4, false);                                            \
  } while (0)
  const bool ib = in_dtype == 1, ob = out_dtype == 1;
  if (dk == 128) {
    if (ib && ob) GDN_GATED(128, bf16, bf16);
    else if (ib) GDN_GATED(128, bf16, float);
    else if (ob) GDN_GATED(128, float, bf16);
    else GDN_GATED(128, float, float);
  } else {
    if (ib && ob) GDN_GATED(64, bf16, bf16);
    else if (ib) GDN_GATED(64, bf16, float);
    else if (ob) GDN_GATED(64, float, bf16);
    else GDN_GATED(64, float, float);
  }
#undef GDN_GATED
#undef GDN_GATED_P
#undef GDN_GATED_K
  return hipGetLastError();
}

}  // namespace gdn
