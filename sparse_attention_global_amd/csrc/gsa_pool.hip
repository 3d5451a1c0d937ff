// GSA compression (Speed3R technical summary section 2.1, compression branch):
// 4x4 average pooling of K and V over each frame's patch grid into the coarse
// context, plus the mean query of every query block (the pooled query whose
// logit against a pooled key is the block score used for selection).
//
// Windows that overhang the grid average only their in-grid tokens. Special
// tokens are never pooled into K/V; they form one extra query block per frame.
//
// Work split: one thread per (query block, head, 8-element chunk of d); eight
// consecutive threads cover one 128-byte head row and the heads of a token are
// adjacent, so every token read is a contiguous 2 KB run across the workgroup.
// Pure HBM streaming: Q, K, V are each read once.
#include "common.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void gsa_pool_kernel(Geom g, const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       const T* __restrict__ v, T* k_cmp,
                                                       T* v_cmp, float* k_cmp_f32,
                                                       float* q_blk_f32) {
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int chunk = (int)(tid & 7);
  const int h = (int)((tid >> 3) % g.n_heads);
  const long long b = (tid >> 3) / g.n_heads;  // query block f*nqb + j
  if (b >= (long long)g.n_frames * g.nqb) return;
  const int f = (int)(b / g.nqb);
  const int j = (int)(b % g.nqb);
  const long long rs = (long long)g.n_heads * kHeadDim;
  const long long col = (long long)h * kHeadDim + chunk * 8;
  const long long frame0 = (long long)f * g.L;
  const bool want_q = q_blk_f32 != nullptr;

  float sq[8], sk[8], sv[8], x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sq[e] = sk[e] = sv[e] = 0.f;

  if (j == g.nb) {  // the frame's special tokens: pooled query only
    if (!want_q) return;
    for (int s = 0; s < g.n_special; ++s) {
      Chunk8<T>::load(q + (frame0 + s) * rs + col, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sq[e] += x[e];
    }
    const float inv = 1.f / (float)g.n_special;
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[e] *= inv;
    store_f32x8(q_blk_f32 + b * rs + col, sq);
    return;
  }

  const int by = j / g.nbw, bx = j % g.nbw;
  const int r0 = 4 * by, r1 = min(r0 + 4, g.grid_h);
  const int c0 = 4 * bx, c1 = min(c0 + 4, g.grid_w);
  for (int r = r0; r < r1; ++r) {
    for (int c = c0; c < c1; ++c) {
      const long long row = frame0 + g.n_special + (long long)r * g.grid_w + c;
      Chunk8<T>::load(k + row * rs + col, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sk[e] += x[e];
      Chunk8<T>::load(v + row * rs + col, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] += x[e];
      if (want_q) {
        Chunk8<T>::load(q + row * rs + col, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) sq[e] += x[e];
      }
    }
  }
  const float inv = 1.f / (float)((r1 - r0) * (c1 - c0));
#pragma unroll
  for (int e = 0; e < 8; ++e) { sk[e] *= inv; sv[e] *= inv; sq[e] *= inv; }
  const long long kj = (long long)f * g.nb + j;
  Chunk8<T>::store(k_cmp + kj * rs + col, sk);
  Chunk8<T>::store(v_cmp + kj * rs + col, sv);
  if (k_cmp_f32 != nullptr) store_f32x8(k_cmp_f32 + kj * rs + col, sk);
  if (want_q) store_f32x8(q_blk_f32 + b * rs + col, sq);
}

}  // namespace

hipError_t launch_gsa_pool(const Geom& g, bool is_bf16, const void* q, const void* k,
                           const void* v, void* k_cmp, void* v_cmp, float* k_cmp_f32,
                           float* q_blk_f32, hipStream_t stream) {
  const long long threads = (long long)g.n_frames * g.nqb * g.n_heads * 8;
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (is_bf16) {
    hipLaunchKernelGGL(gsa_pool_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), static_cast<bf16*>(k_cmp),
                       static_cast<bf16*>(v_cmp), k_cmp_f32, q_blk_f32);
  } else {
    hipLaunchKernelGGL(gsa_pool_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), static_cast<float*>(k_cmp),
                       static_cast<float*>(v_cmp), k_cmp_f32, q_blk_f32);
  }
  return hipGetLastError();
}

}  // namespace sga
