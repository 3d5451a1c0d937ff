// GSA block selection (Speed3R technical summary section 2.1, selection branch;
// the Italian summary's S_guide matrix, and its section on the fused kernel:
// selection streams through on-chip memory and never materialises the score
// matrix).
//
// Per head h and query block b, score(j) = q_blk[b,h] . k_cmp[j,h] / sqrt(d)
// for every competing pooled key j; the top_k best (larger score first, ties
// to the lower j) are returned as an ascending index set. The competing keys
// are all pooled keys, or those after the reference frame's blocks when that
// frame is kept whole (Speed3R technical summary section 2.2, VGGT adaptation).
//
// Scores: fp32-accurate products on the bf16 matrix cores via the three-term
// split x = hi + lo (hi = bf16(x), lo = bf16(x - hi)):
//   q.k ~= qhi.khi + qhi.klo + qlo.khi,
// whose dropped term and residuals are ~2^-16 relative -- far inside the 1e-3
// score gap the selection is checked at. The 1/sqrt(64) scale is exact.
//
// Work split: a workgroup of W waves owns 32*W query blocks of one head; every
// wave owns 32 of them and streams all pooled keys in tiles of 64 through LDS
// (double buffered). Each lane keeps, for its query block, a threshold (the
// current K-th best); a tile whose lane-wise maximum stays below it costs one
// max tree and one compare. Candidates that beat it are inserted into a sorted
// per-block list in LDS, one half-wave at a time so the two lanes sharing a
// block never race.
#include "common.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

constexpr int kTileN = 64;
constexpr int kTileBytes = kTileN * 128;      // one bf16 plane of a 64-key tile
constexpr int kStageBytes = 2 * kTileBytes;   // hi + lo planes

__device__ __forceinline__ int t_off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ bool beats(float s, int j, float ts, int tj) {
  return s > ts || (s == ts && j < tj);
}

// Split 8 fp32 values into bf16 hi and lo parts (packed pairs).
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t ph = pack_bf16x2(x[2 * j], x[2 * j + 1]);
    hi[j] = ph;
    lo[j] = pack_bf16x2(x[2 * j] - lo_bf16(ph), x[2 * j + 1] - hi_bf16(ph));
  }
}

__global__ __launch_bounds__(256) void gsa_topk_kernel(Geom g, const float* __restrict__ q_blk,
                                                       const float* __restrict__ k_cmp,
                                                       long long n_cand, int j0,
                                                       int top_k, int n_rowtiles,
                                                       int32_t* __restrict__ idx,
                                                       float* __restrict__ score) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int waves = blockDim.x >> 6;
  const int h = blockIdx.x / n_rowtiles;
  const long long row0 = (long long)(blockIdx.x % n_rowtiles) * 32 * waves;
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const long long rs = (long long)g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long row = row0 + wave * 32 + li;
  const bool rvalid = row < n_rows;

  // per-row sorted lists: [wave][32 rows][top_k + 1] (padded stride)
  const int stride = top_k + 1;
  float* lv = reinterpret_cast<float*>(smem + 2 * kStageBytes);
  int* lj = reinterpret_cast<int*>(lv + waves * 32 * stride);
  float* my_v = lv + (wave * 32 + li) * stride;
  int* my_j = lj + (wave * 32 + li) * stride;
  for (int p = hh; p < top_k; p += 2) { my_v[p] = -INFINITY; my_j[p] = 0x7fffffff; }

  // pooled-query operand (B of S^T = K Q^T), hi and lo planes
  u32x4 qh[4], ql[4];
  {
    const float* qp = q_blk + (rvalid ? row : 0) * rs + hoff + hh * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
      const f32x4 a = *reinterpret_cast<const f32x4*>(qp + ks * 16);
      const f32x4 b = *reinterpret_cast<const f32x4*>(qp + ks * 16 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = rvalid ? a[e] : 0.f; x[4 + e] = rvalid ? b[e] : 0.f; }
      split8(x, qh[ks], ql[ks]);
    }
  }

  // loader: thread -> (key tid>>2 of the tile, d range 16*(tid&3) .. +16)
  const int nthreads = blockDim.x;
  f32x4 kreg[2][4];
  auto load_tile = [&](long long u0) {
    for (int slot = 0; slot < 2; ++slot) {
      const int item = tid + slot * nthreads;  // 256 items = 64 keys x 4 quarters
      if (item >= 256) break;
      const long long u = u0 + (item >> 2);
      const int quarter = item & 3;
      if (u < n_cand) {
        const float* kp = k_cmp + u * rs + hoff + quarter * 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) kreg[slot][e] = *reinterpret_cast<const f32x4*>(kp + 4 * e);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) kreg[slot][e] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* hi_p = smem + stage * kStageBytes;
    unsigned char* lo_p = hi_p + kTileBytes;
    for (int slot = 0; slot < 2; ++slot) {
      const int item = tid + slot * nthreads;
      if (item >= 256) break;
      const int key = item >> 2, quarter = item & 3;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = kreg[slot][2 * half][e];
          x[4 + e] = kreg[slot][2 * half + 1][e];
        }
        u32x4 hi, lo;
        split8(x, hi, lo);
        const int chunk = 2 * quarter + half;
        st16(hi_p + t_off(key, chunk), hi);
        st16(lo_p + t_off(key, chunk), lo);
      }
    }
  };

  const float scale = 0.125f;  // 1/sqrt(64), exact
  float tau_s = -INFINITY;
  int tau_j = 0x7fffffff;
  const long long n_tiles = (n_cand + kTileN - 1) / kTileN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (long long it = 0; it < n_tiles; ++it) {
    const int stage = (int)(it & 1);
    const long long u0 = it * kTileN;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(u0 + kTileN);
    const unsigned char* hi_p = smem + stage * kStageBytes;
    const unsigned char* lo_p = hi_p + kTileBytes;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 ah = ld16(hi_p + t_off(kb * 32 + li, 2 * ks + hh));
        const u32x4 al = ld16(lo_p + t_off(kb * 32 + li, 2 * ks + hh));
        acc = mfma32(al, qh[ks], acc);
        acc = mfma32(ah, ql[ks], acc);
        acc = mfma32(ah, qh[ks], acc);
      }
      s[kb] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const long long j = u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        s[kb][i] = (j < n_cand) ? s[kb][i] * scale : -INFINITY;
        mx = fmaxf(mx, s[kb][i]);
      }
    // candidates can only beat the threshold if their score reaches it
    if (__any(rvalid && mx >= tau_s)) {
      for (int half = 0; half < 2; ++half) {
        if (hh == half && rvalid && mx >= tau_s) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float sv = s[kb][i];
              const int j = (int)(u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3));
              if (beats(sv, j, tau_s, tau_j)) {
                int p = top_k - 1;
                while (p > 0 && beats(sv, j, my_v[p - 1], my_j[p - 1])) {
                  my_v[p] = my_v[p - 1];
                  my_j[p] = my_j[p - 1];
                  --p;
                }
                my_v[p] = sv;
                my_j[p] = j;
                tau_s = my_v[top_k - 1];
                tau_j = my_j[top_k - 1];
              }
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        tau_s = my_v[top_k - 1];
        tau_j = my_j[top_k - 1];
      }
    }
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- write the set in ascending index order ---------------------------------
  if (rvalid && hh == 0) {
    int32_t* ip = idx + ((long long)h * n_rows + row) * top_k;
    float* sp = score ? score + ((long long)h * n_rows + row) * top_k : nullptr;
    int prev = -1;
    for (int o = 0; o < top_k; ++o) {
      int best = 0x7fffffff, bp = 0;
      for (int p = 0; p < top_k; ++p) {
        const int jj = my_j[p];
        if (jj > prev && jj < best) { best = jj; bp = p; }
      }
      ip[o] = best + j0;
      if (sp) sp[o] = my_v[bp];
      prev = best;
    }
  }
}

// ---------------------------------------------------------------------------
// Register-list variant for top_k <= kRegK (the common case, top-16).
//
// Each lane keeps the best kRegK scores of its own key half in registers,
// sorted best first. A lane meets its keys in increasing index order, so a new
// score ties an entry only with a higher index and beats it only when strictly
// larger: the insertion is a fixed compare/select network over the list, with
// no divergent loop and no LDS. A tile costs one max tree and one compare when
// no lane's maximum beats its threshold; otherwise each of the lane's 32 scores
// that some lane needs is pushed through the network (masked to the lanes
// whose score beats their threshold). At the end the two lanes of a block swap
// lists (v_permlane32_swap) and keep the best top_k of the two sorted lists
// with a bitonic merge: the first list against the second reversed, then
// log2(kRegK) half-cleaner stages.
// ---------------------------------------------------------------------------
constexpr int kRegK = 16;

// Entry order: larger score first; equal scores, lower index first.
__device__ __forceinline__ bool better(float s, int j, float ts, int tj) {
  return s > ts || (s == ts && j < tj);
}

// Occupancy: 4 workgroups (4 waves per SIMD, 128 VGPRs); measured at 128 frames
// 2.46 ms against 2.76 ms at 3 waves per SIMD and 3.40 ms at 2.
template <bool FULL>  // FULL: top_k == kRegK, the threshold is the list's last slot
__global__ __launch_bounds__(256, 4) void gsa_topk_reg_kernel(Geom g, const float* __restrict__ q_blk,
                                                           const float* __restrict__ k_cmp,
                                                           long long n_cand, int j0,
                                                           int top_k, int n_rowtiles,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ score) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int h = blockIdx.x / n_rowtiles;
  const long long row0 = (long long)(blockIdx.x % n_rowtiles) * 128;
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const long long rs = (long long)g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long row = row0 + wave * 32 + li;
  const bool rvalid = row < n_rows;

  // pooled-query operand scaled by 1/sqrt(64) = 1/8 (exact), hi and lo planes
  u32x4 qh[4], ql[4];
  {
    const float* qp = q_blk + (rvalid ? row : 0) * rs + hoff + hh * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
      const f32x4 a = *reinterpret_cast<const f32x4*>(qp + ks * 16);
      const f32x4 b = *reinterpret_cast<const f32x4*>(qp + ks * 16 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = rvalid ? a[e] * 0.125f : 0.f;
        x[4 + e] = rvalid ? b[e] * 0.125f : 0.f;
      }
      split8(x, qh[ks], ql[ks]);
    }
  }

  // loader: thread -> (key tid>>2 of the tile, d range 16*(tid&3) .. +16)
  f32x4 kreg[4];
  auto load_tile = [&](long long u0) {
    const long long u = u0 + (tid >> 2);
    const int quarter = tid & 3;
    if (u < n_cand) {
      const float* kp = k_cmp + u * rs + hoff + quarter * 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) kreg[e] = *reinterpret_cast<const f32x4*>(kp + 4 * e);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kreg[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* hi_p = smem + stage * kStageBytes;
    unsigned char* lo_p = hi_p + kTileBytes;
    const int key = tid >> 2, quarter = tid & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = kreg[2 * half][e];
        x[4 + e] = kreg[2 * half + 1][e];
      }
      u32x4 hi, lo;
      split8(x, hi, lo);
      const int chunk = 2 * quarter + half;
      st16(hi_p + t_off(key, chunk), hi);
      st16(lo_p + t_off(key, chunk), lo);
    }
  };

  float lv[kRegK];
  int lj[kRegK];
#pragma unroll
  for (int p = 0; p < kRegK; ++p) { lv[p] = -INFINITY; lj[p] = 0x7fffffff; }
  float tau = -INFINITY;  // lv[top_k - 1]
  const int kth = top_k - 1;

  const long long n_tiles = (n_cand + kTileN - 1) / kTileN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (long long it = 0; it < n_tiles; ++it) {
    const int stage = (int)(it & 1);
    const long long u0 = it * kTileN;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(u0 + kTileN);
    const unsigned char* hi_p = smem + stage * kStageBytes;
    const unsigned char* lo_p = hi_p + kTileBytes;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 ah = ld16(hi_p + t_off(kb * 32 + li, 2 * ks + hh));
        const u32x4 al = ld16(lo_p + t_off(kb * 32 + li, 2 * ks + hh));
        acc = mfma32(al, qh[ks], acc);
        acc = mfma32(ah, ql[ks], acc);
        acc = mfma32(ah, qh[ks], acc);
      }
      s[kb] = acc;
    }
    if (!more) {  // the last tile: keys past the end score -inf
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const long long j = u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (j >= n_cand) s[kb][i] = -INFINITY;
        }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    if (__any(rvalid && mx > tau)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float sv = s[kb][i];
          const bool c = rvalid && sv > tau;
          if (__any(c)) {
            const int j = (int)u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            // b(p) = the candidate lands at or before slot p (monotone in p);
            // walk from the tail so slot p - 1 is read before it is written
#pragma unroll
            for (int p = kRegK - 1; p >= 1; --p) {
              const bool b = c && sv > lv[p];
              const bool bp = sv > lv[p - 1];
              const float tv = bp ? lv[p - 1] : sv;
              const int tj = bp ? lj[p - 1] : j;
              lv[p] = b ? tv : lv[p];
              lj[p] = b ? tj : lj[p];
            }
            {
              const bool b = c && sv > lv[0];
              lv[0] = b ? sv : lv[0];
              lj[0] = b ? j : lj[0];
            }
            if (FULL) {
              tau = lv[kRegK - 1];
            } else {
              float t = lv[0];
#pragma unroll
              for (int p = 1; p < kRegK; ++p) t = (p == kth) ? lv[p] : t;
              tau = t;
            }
          }
        }
    }
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- merge the block's two lists (lanes l and l + 32) ------------------------
  // partner's list: v_permlane32_swap leaves lane l < 32 the upper half's value
  float pv[kRegK];
  int pj[kRegK];
#pragma unroll
  for (int p = 0; p < kRegK; ++p) {
    const auto rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(lv[p]), __float_as_uint(lv[p]),
                                                     false, false);
    const auto rj = __builtin_amdgcn_permlane32_swap((uint32_t)lj[p], (uint32_t)lj[p], false, false);
    pv[p] = __uint_as_float(rv[1]);
    pj[p] = (int)rj[1];
  }
  // bitonic merge of two sorted (best-first) lists: the best kRegK of the union
  // are max(a[p], b[kRegK-1-p]), a bitonic sequence; half-cleaners sort it
#pragma unroll
  for (int p = 0; p < kRegK; ++p) {
    const float bv = pv[kRegK - 1 - p];
    const int bj = pj[kRegK - 1 - p];
    if (!better(lv[p], lj[p], bv, bj)) { lv[p] = bv; lj[p] = bj; }
  }
#pragma unroll
  for (int half = kRegK / 2; half >= 1; half >>= 1)
#pragma unroll
    for (int p = 0; p < kRegK; ++p)
      if ((p & half) == 0) {
        const int q = p + half;
        if (!better(lv[p], lj[p], lv[q], lj[q])) {
          const float tv = lv[p]; lv[p] = lv[q]; lv[q] = tv;
          const int tj = lj[p]; lj[p] = lj[q]; lj[q] = tj;
        }
      }
  // the best top_k, written in ascending index order
  if (rvalid && hh == 0) {
    int32_t* ip = idx + ((long long)h * n_rows + row) * top_k;
    float* sp = score ? score + ((long long)h * n_rows + row) * top_k : nullptr;
    int prev = -1;
    for (int o = 0; o < top_k; ++o) {
      int best = 0x7fffffff;
      float bv = 0.f;
#pragma unroll
      for (int p = 0; p < kRegK; ++p) {
        const bool in = p < top_k && lj[p] > prev && lj[p] < best;
        best = in ? lj[p] : best;
        bv = in ? lv[p] : bv;
      }
      ip[o] = best + j0;
      if (sp) sp[o] = bv;
      prev = best;
    }
  }
}

}  // namespace

hipError_t launch_gsa_topk(const Geom& g, const float* q_blk, const float* k_cmp, int top_k,
                           int first, int32_t* idx, float* score, hipStream_t stream) {
  const long long n_rows = (long long)g.n_frames * g.nqb;
  // the kernels see the competing keys only, indexed from 0, and add `first`
  // to the indices they write
  const long long n_cand = (long long)g.n_frames * g.nb - first;
  const float* kc = k_cmp + (long long)first * g.n_heads * kHeadDim;
  if (top_k <= kRegK) {
    const int n_rowtiles = (int)((n_rows + 127) / 128);
    const long long grid = (long long)n_rowtiles * g.n_heads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (top_k == kRegK) {
      hipLaunchKernelGGL(gsa_topk_reg_kernel<true>, dim3((unsigned)grid), dim3(256), 2 * kStageBytes,
                         stream, g, q_blk, kc, n_cand, first, top_k, n_rowtiles, idx, score);
    } else {
      hipLaunchKernelGGL(gsa_topk_reg_kernel<false>, dim3((unsigned)grid), dim3(256), 2 * kStageBytes,
                         stream, g, q_blk, kc, n_cand, first, top_k, n_rowtiles, idx, score);
    }
    return hipGetLastError();
  }
  int waves = 4;
  auto lds_for = [&](int w) { return (size_t)2 * kStageBytes + (size_t)w * 32 * (top_k + 1) * 8; };
  if (lds_for(waves) > 160 * 1024) waves = 2;
  const int n_rowtiles = (int)((n_rows + 32 * waves - 1) / (32 * waves));
  const long long grid = (long long)n_rowtiles * g.n_heads;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gsa_topk_kernel, dim3((unsigned)grid), dim3(64 * waves), lds_for(waves), stream,
                     g, q_blk, kc, n_cand, first, top_k, n_rowtiles, idx, score);
  return hipGetLastError();
}

}  // namespace sga
