// GSA gated aggregation (Speed3R technical summary section 2.1, gated
// aggregation; Italian summary section 2, "Aggregazione Guidata"): a learnable
// sigmoid gate conditioned on the query mixes the two branches per token:
//   g = sigmoid(q . W[h]^T + b[h]) in (0,1)^2,  o = g0 * o_cmp + g1 * o_slc.
//
// Work split: 8 threads per (token, head) row, each owning 8 consecutive d;
// the two 64-term dot products are finished with 3 butterfly steps inside the
// 8-lane group. Streams Q, O_cmp, O_slc once and writes O once.
#include "common.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void gsa_gate_kernel(Geom g, const T* __restrict__ q,
                                                       const T* o_cmp, const T* o_slc,
                                                       const float* __restrict__ w,
                                                       const float* __restrict__ b, T* o) {
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = tid >> 3;  // t * H + h
  const int chunk = (int)(tid & 7);
  const bool valid = row < g.T * g.n_heads;
  const long long r = valid ? row : 0;
  const int h = (int)(r % g.n_heads);
  const long long off = r * kHeadDim + chunk * 8;
  float x[8];
  Chunk8<T>::load(q + off, x);
  const float* w0 = w + (long long)h * 2 * kHeadDim + chunk * 8;
  const float* w1 = w0 + kHeadDim;
  float z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    z0 = fmaf(x[e], w0[e], z0);
    z1 = fmaf(x[e], w1[e], z1);
  }
#pragma unroll
  for (int sh = 1; sh < 8; sh <<= 1) {
    z0 += __shfl_xor(z0, sh, 8);
    z1 += __shfl_xor(z1, sh, 8);
  }
  if (!valid) return;
  const float g0 = 1.f / (1.f + expf(-(z0 + b[2 * h])));
  const float g1 = 1.f / (1.f + expf(-(z1 + b[2 * h + 1])));
  float a[8], s[8];
  Chunk8<T>::load(o_cmp + off, a);
  Chunk8<T>::load(o_slc + off, s);
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = g0 * a[e] + g1 * s[e];
  Chunk8<T>::store(o + off, a);
}

}  // namespace

hipError_t launch_gsa_gate(const Geom& g, bool is_bf16, const void* q, const void* o_cmp,
                           const void* o_slc, const float* w, const float* b, void* o,
                           hipStream_t stream) {
  const long long threads = g.T * g.n_heads * 8;
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (is_bf16) {
    hipLaunchKernelGGL(gsa_gate_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(o_cmp),
                       static_cast<const bf16*>(o_slc), w, b, static_cast<bf16*>(o));
  } else {
    hipLaunchKernelGGL(gsa_gate_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const float*>(q), static_cast<const float*>(o_cmp),
                       static_cast<const float*>(o_slc), w, b, static_cast<float*>(o));
  }
  return hipGetLastError();
}

}  // namespace sga
