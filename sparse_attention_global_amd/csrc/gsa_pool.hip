// GSA compression (Speed3R technical summary section 2.1, compression branch):
// 4x4 average pooling of K and V over each frame's patch grid into the coarse
// context, plus the mean query of every query block (the pooled query whose
// logit against a pooled key is the block score used for selection).
//
// Windows that overhang the grid average only their in-grid tokens, or, with
// include_pad, the grid counts as zero-padded to whole windows (the in-grid
// sum over 16). Special tokens are never pooled into K/V; they form one extra
// query block per frame. The mean queries are always over the block's tokens.
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
                                                       float* q_blk_f32, int include_pad) {
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
  const float inv_kv = include_pad ? 1.f / 16.f : inv;
#pragma unroll
  for (int e = 0; e < 8; ++e) { sk[e] *= inv_kv; sv[e] *= inv_kv; sq[e] *= inv; }
  const long long kj = (long long)f * g.nb + j;
  Chunk8<T>::store(k_cmp + kj * rs + col, sk);
  Chunk8<T>::store(v_cmp + kj * rs + col, sv);
  if (k_cmp_f32 != nullptr) store_f32x8(k_cmp_f32 + kj * rs + col, sk);
  if (want_q) store_f32x8(q_blk_f32 + b * rs + col, sq);
}

// bf16 copy of the fp32 pooled queries (the block-level compressed branch's
// query operand): 8 values per thread.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const f32x4* __restrict__ x, u32x4* __restrict__ y,
                                                       long long n8) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = x[2 * i], b = x[2 * i + 1];
  y[i] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
               pack_bf16x2(b[2], b[3])};
}

// Nearest upsampling of per-block outputs to the tokens (Speed3R technical
// summary section 2.1: the compressed results brought back to full
// resolution): o[t, h] = o_blk[block(t), h], block(t) the query block of token
// t (its 4x4 window, or its frame's special-token block). A thread per 16-byte
// chunk; CH chunks per (token, head) row.
template <int CH>
__global__ __launch_bounds__(256) void upsample_kernel(Geom g, const u32x4* __restrict__ o_blk,
                                                      u32x4* __restrict__ o) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per_token = (long long)g.n_heads * CH;
  if (i >= g.T * per_token) return;
  const long long t = i / per_token, within = i % per_token;
  const int f = (int)(t / g.L), p = (int)(t % g.L) - g.n_special;
  long long b = (long long)f * g.nqb;
  if (p < 0) {
    b += g.nb;
  } else {
    b += (long long)((p / g.grid_w) >> 2) * g.nbw + ((p % g.grid_w) >> 2);
  }
  o[i] = o_blk[b * per_token + within];
}

}  // namespace

hipError_t launch_cast_bf16(const float* x, void* y, long long n, hipStream_t stream) {
  const long long n8 = n / 8;
  const long long blocks = (n8 + 255) / 256;
  if (n % 8 != 0 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4*>(x), static_cast<u32x4*>(y), n8);
  return hipGetLastError();
}

hipError_t launch_gsa_upsample(const Geom& g, bool is_bf16, const void* o_blk, void* o,
                               hipStream_t stream) {
  const int ch = is_bf16 ? 8 : 16;
  const long long n = g.T * g.n_heads * ch;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (is_bf16) {
    hipLaunchKernelGGL(upsample_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const u32x4*>(o_blk), static_cast<u32x4*>(o));
  } else {
    hipLaunchKernelGGL(upsample_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const u32x4*>(o_blk), static_cast<u32x4*>(o));
  }
  return hipGetLastError();
}

hipError_t launch_gsa_pool(const Geom& g, bool is_bf16, int include_pad, const void* q,
                           const void* k, const void* v, void* k_cmp, void* v_cmp,
                           float* k_cmp_f32, float* q_blk_f32, hipStream_t stream) {
  const long long threads = (long long)g.n_frames * g.nqb * g.n_heads * 8;
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (is_bf16) {
    hipLaunchKernelGGL(gsa_pool_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), static_cast<bf16*>(k_cmp),
                       static_cast<bf16*>(v_cmp), k_cmp_f32, q_blk_f32, include_pad);
  } else {
    hipLaunchKernelGGL(gsa_pool_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), static_cast<float*>(k_cmp),
                       static_cast<float*>(v_cmp), k_cmp_f32, q_blk_f32, include_pad);
  }
  return hipGetLastError();
}

}  // namespace sga
