// fp32 attention of the forms the bf16 flash kernel serves (dense/compressed,
// frame, AVGGT subsampled), for fp32 layers: a workgroup of kSplit waves per
// 64 queries and one head; lane l of every wave owns query l, and wave w visits
// the w-th of every kSplit consecutive keys of the query's key set with an
// exact online softmax (expf, every product and sum in fp32). The waves' partial
// results (running maximum, sum and unnormalised output) then merge through
// LDS. The key set follows the same definitions as the bf16 kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* ck;
  const float* cv;
  float* o;
  float* lse;
  Geom g;
  long long n_keys;
  int mode;
  int mk;
  int has_mean;
  float mean_bias;  // natural-log units
  int token_diag;   // SUBSAMPLED: own frame subsampled too, plus the query's own key if dropped
  int s_h, s_w;
};

constexpr int kSplit = 8;  // waves per workgroup, each visiting every kSplit-th key

__global__ __launch_bounds__(64 * kSplit) void flash_f32_kernel(F32Args A) {
  __shared__ float part[kSplit][kHeadDim + 2][64];  // per wave: acc[d], m, l of each lane's query
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long t = (long long)blockIdx.x * 64 + lane;
  const int h = blockIdx.y;
  const bool valid = t < A.g.T;
  const long long rs = (long long)A.g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;
  const long long tq = valid ? t : 0;
  const int f = (int)(tq / A.g.L);
  float qv[kHeadDim], acc[kHeadDim];
  const float* qp = A.q + tq * rs + hoff;
  for (int e = 0; e < kHeadDim; ++e) { qv[e] = qp[e] * 0.125f; acc[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  unsigned int seq = 0;  // position of the next key in the query's key set
  auto visit = [&](const float* kp, const float* vp, float bias) {
    if ((seq++ % kSplit) != (unsigned int)wave) return;
    float s = bias;
    for (int e = 0; e < kHeadDim; ++e) s = fmaf(qv[e], kp[e], s);
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float pe = expf(s - m_new);
    for (int e = 0; e < kHeadDim; ++e) acc[e] = fmaf(acc[e], alpha, pe * vp[e]);
    l = l * alpha + pe;
    m = m_new;
  };
  if (A.mode == FLASH_GLOBAL) {
    for (long long u = 0; u < A.n_keys; ++u) visit(A.k + u * rs + hoff, A.v + u * rs + hoff, 0.f);
  } else {
    const bool diag = A.mode == FLASH_SUBSAMPLED && A.token_diag;
    const long long f0 = (long long)f * A.g.L;
    if (!diag)
      for (long long u = f0; u < f0 + A.g.L; ++u) visit(A.k + u * rs + hoff, A.v + u * rs + hoff, 0.f);
    if (A.mode == FLASH_SUBSAMPLED) {
      for (long long r = 0; r < (long long)A.g.n_frames * A.mk; ++r) {
        if (!diag && r / A.mk == f) continue;
        visit(A.ck + r * rs + hoff, A.cv + r * rs + hoff, 0.f);
      }
      if (A.has_mean)
        for (int g2 = 0; g2 < A.g.n_frames; ++g2) {
          if (!diag && g2 == f) continue;
          const long long r = (long long)A.g.n_frames * A.mk + g2;
          visit(A.ck + r * rs + hoff, A.cv + r * rs + hoff, A.mean_bias);
        }
      if (diag) {  // the query's own key when its patch was dropped
        const int p = (int)(tq - f0) - A.g.n_special;
        if (p >= 0 && ((p / A.g.grid_w) % A.s_h != 0 || (p % A.g.grid_w) % A.s_w != 0))
          visit(A.k + tq * rs + hoff, A.v + tq * rs + hoff, 0.f);
      }
    }
  }
  // merge the waves' partial results: M = max m_w, L = sum l_w e^(m_w - M),
  // O = sum acc_w e^(m_w - M) / L (a wave that met no key has m_w = -inf, l_w = 0)
  for (int e = 0; e < kHeadDim; ++e) part[wave][e][lane] = acc[e];
  part[wave][kHeadDim][lane] = m;
  part[wave][kHeadDim + 1][lane] = l;
  __syncthreads();
  if (wave != 0 || !valid) return;
  float mm = -INFINITY;
  for (int w = 0; w < kSplit; ++w) mm = fmaxf(mm, part[w][kHeadDim][lane]);
  float sc[kSplit], ll = 0.f;
  for (int w = 0; w < kSplit; ++w) {
    const float mw = part[w][kHeadDim][lane];
    sc[w] = mw == -INFINITY ? 0.f : expf(mw - mm);
    ll = fmaf(part[w][kHeadDim + 1][lane], sc[w], ll);
  }
  float* op = A.o + t * rs + hoff;
  for (int e = 0; e < kHeadDim; ++e) {
    float o = 0.f;
    for (int w = 0; w < kSplit; ++w) o = fmaf(part[w][e][lane], sc[w], o);
    op[e] = o / ll;
  }
  if (A.lse) A.lse[t * A.g.n_heads + h] = mm + logf(ll);
}

}  // namespace

hipError_t launch_flash_f32(const FlashLaunch& p, hipStream_t stream) {
  F32Args A{};
  A.q = static_cast<const float*>(p.q);
  A.k = static_cast<const float*>(p.k);
  A.v = static_cast<const float*>(p.v);
  A.ck = static_cast<const float*>(p.ck);
  A.cv = static_cast<const float*>(p.cv);
  A.o = static_cast<float*>(p.o);
  A.lse = p.lse;
  A.g = p.g;
  A.n_keys = p.n_keys;
  A.mode = p.mode;
  A.mk = p.mk;
  A.has_mean = p.has_mean;
  A.mean_bias = p.mean_bias2 * 0.6931471805599453f;
  A.token_diag = p.token_diag;
  A.s_h = p.s_h > 0 ? p.s_h : 1;
  A.s_w = p.s_w > 0 ? p.s_w : 1;
  dim3 grid((unsigned)((p.g.T + 63) / 64), (unsigned)p.g.n_heads);
  hipLaunchKernelGGL(flash_f32_kernel, grid, dim3(64 * kSplit), 0, stream, A);
  return hipGetLastError();
}

}  // namespace sga
