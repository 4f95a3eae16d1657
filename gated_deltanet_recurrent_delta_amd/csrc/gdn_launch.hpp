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

hipError_t launch_decode(const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta,
                         const float* S_in, float* S_out, void* o, int BH,
                         int dk, int dv, int in_dtype, int out_dtype,
                         hipStream_t stream);

hipError_t launch_prefill_prepare(const void* q, const void* k,
                                  const float* alpha, const float* beta,
                                  float* ws, int B, int T, int H, int dk,
                                  int in_dtype, hipStream_t stream);

hipError_t launch_prefill_scan(const void* q, const void* k, const void* v,
                               const float* S0, void* o, float* ST,
                               const float* ws, int B, int T, int H, int dk,
                               int dv, int in_dtype, int out_dtype,
                               hipStream_t stream);

hipError_t launch_state_fill(const float* S0, float* ST, size_t n,
                             hipStream_t stream);

}  // namespace gdn
