// AVGGT compaction (AVGGT technical summary section 2.2): the key/value rows a
// query of another frame sees -- the frame's special tokens and its patches on
// the s_h x s_w grid (exact copies), and one mean key/value standing in for
// the dropped patches.
//
// Output layout: the kept part [N * mk, H, d] (frame-major; specials, then the
// kept patches in row-major grid order) followed by the mean part [N, H, d]
// when any patch is dropped. mk = S + ceil(gh/sh) * ceil(gw/sw).
//
// Work split: a workgroup per (frame, group of 8 heads): 64 threads cover the
// group's 8 x 8 sixteen-byte chunks of a token (1 KB contiguous) and 4 slices
// of threads walk interleaved tokens; the slices' partial sums of the dropped
// patches meet in LDS. K and V are read once.
#include "common.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void sga_compact_kernel(Geom g, int s_h, int s_w,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v, T* c_k,
                                                          T* c_v) {
  __shared__ float part[2][4][64][9];
  const int f = blockIdx.x;
  const int slice = threadIdx.x >> 6;
  const int pair = blockIdx.y * 64 + (threadIdx.x & 63);
  const bool pvalid = pair < g.n_heads * 8;
  const int h = pvalid ? pair >> 3 : 0;
  const int chunk = pair & 7;
  const long long rs = (long long)g.n_heads * kHeadDim;
  const long long col = (long long)h * kHeadDim + chunk * 8;
  const long long frame0 = (long long)f * g.L;
  const int nkh = (g.grid_h + s_h - 1) / s_h, nkw = (g.grid_w + s_w - 1) / s_w;
  const int mk = g.n_special + nkh * nkw;
  const int n_patch = g.grid_h * g.grid_w;
  const int n_drop = n_patch - nkh * nkw;
  float x[8];

  if (pvalid) {
    for (int i = slice; i < mk; i += 4) {
      long long src;
      if (i < g.n_special) {
        src = frame0 + i;
      } else {
        const int p = i - g.n_special;
        src = frame0 + g.n_special + (long long)(p / nkw) * s_h * g.grid_w + (p % nkw) * s_w;
      }
      const long long dst = (long long)f * mk + i;
      Chunk8<T>::load(k + src * rs + col, x);
      Chunk8<T>::store(c_k + dst * rs + col, x);
      Chunk8<T>::load(v + src * rs + col, x);
      Chunk8<T>::store(c_v + dst * rs + col, x);
    }
  }
  if (n_drop == 0) return;

  float sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
  if (pvalid) {
    for (int p = slice; p < n_patch; p += 4) {
      const int r = p / g.grid_w, c = p % g.grid_w;
      if (r % s_h == 0 && c % s_w == 0) continue;
      const long long row = frame0 + g.n_special + p;
      Chunk8<T>::load(k + row * rs + col, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sk[e] += x[e];
      Chunk8<T>::load(v + row * rs + col, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] += x[e];
    }
  }
  const int tl = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    part[0][slice][tl][e] = sk[e];
    part[1][slice][tl][e] = sv[e];
  }
  __syncthreads();
  if (slice != 0 || !pvalid) return;
  const float inv = 1.f / (float)n_drop;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sk[e] = (((part[0][0][tl][e] + part[0][1][tl][e]) + part[0][2][tl][e]) + part[0][3][tl][e]) * inv;
    sv[e] = (((part[1][0][tl][e] + part[1][1][tl][e]) + part[1][2][tl][e]) + part[1][3][tl][e]) * inv;
  }
  const long long dst = (long long)g.n_frames * mk + f;
  Chunk8<T>::store(c_k + dst * rs + col, sk);
  Chunk8<T>::store(c_v + dst * rs + col, sv);
}

// Token-level diagonal (AVGGT technical summary section 2.2, the diagonal
// kept): a query whose patch was dropped adds its own key/value to the
// softmax it already has over the compacted sets, given as the normalised
// output o and the log-sum-exp lse: o' = (e^lse o + e^s v_t) / (e^lse + e^s),
// s = q_t . k_t / sqrt(d). Eight lanes per (token, head), 16 bytes each.
__global__ __launch_bounds__(256) void sga_diag_merge_kernel(Geom g, int s_h, int s_w,
                                                             const u32x4* __restrict__ q,
                                                             const u32x4* __restrict__ k,
                                                             const u32x4* __restrict__ v,
                                                             u32x4* __restrict__ o,
                                                             const float* __restrict__ lse) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)g.T * g.n_heads * 8) return;
  const long long th = i >> 3;
  const long long t = th / g.n_heads;
  const int h = (int)(th % g.n_heads);
  const int p = (int)(t % g.L) - g.n_special;
  // the 8 lanes of a (token, head) take the same branch
  if (p < 0) return;                                             // a special token: kept
  if ((p / g.grid_w) % s_h == 0 && (p % g.grid_w) % s_w == 0) return;  // a kept patch
  const u32x4 qa = q[i], ka = k[i];
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dot = fmaf(lo_bf16(qa[e]), lo_bf16(ka[e]), dot);
    dot = fmaf(hi_bf16(qa[e]), hi_bf16(ka[e]), dot);
  }
  dot += __shfl_xor(dot, 1, 8);
  dot += __shfl_xor(dot, 2, 8);
  dot += __shfl_xor(dot, 4, 8);
  const float s = dot * 0.125f;  // 1/sqrt(64)
  const float l0 = lse[t * g.n_heads + h];
  const float mx = fmaxf(l0, s);
  const float a = expf(l0 - mx), b = expf(s - mx);
  const float inv = 1.f / (a + b);
  const u32x4 oa = o[i], va = v[i];
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    out[e] = pack_bf16x2((lo_bf16(oa[e]) * a + lo_bf16(va[e]) * b) * inv,
                         (hi_bf16(oa[e]) * a + hi_bf16(va[e]) * b) * inv);
  o[i] = out;
}

}  // namespace

hipError_t launch_sga_diag_merge(const Geom& g, int s_h, int s_w, const void* q, const void* k,
                                 const void* v, void* o, const float* lse, hipStream_t stream) {
  const long long n = (long long)g.T * g.n_heads * 8;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sga_diag_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g, s_h, s_w,
                     static_cast<const u32x4*>(q), static_cast<const u32x4*>(k),
                     static_cast<const u32x4*>(v), static_cast<u32x4*>(o), lse);
  return hipGetLastError();
}

hipError_t launch_sga_compact(const Geom& g, bool is_bf16, int s_h, int s_w, const void* k,
                              const void* v, void* c_k, void* c_v, hipStream_t stream) {
  dim3 grid((unsigned)g.n_frames, (unsigned)((g.n_heads * 8 + 63) / 64));
  if (is_bf16) {
    hipLaunchKernelGGL(sga_compact_kernel<bf16>, grid, dim3(256), 0, stream, g, s_h, s_w,
                       static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                       static_cast<bf16*>(c_k), static_cast<bf16*>(c_v));
  } else {
    hipLaunchKernelGGL(sga_compact_kernel<float>, grid, dim3(256), 0, stream, g, s_h, s_w,
                       static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<float*>(c_k), static_cast<float*>(c_v));
  }
  return hipGetLastError();
}

}  // namespace sga
