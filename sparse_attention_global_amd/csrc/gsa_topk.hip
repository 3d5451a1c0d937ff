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
// Work split, common to the kernels below: a workgroup owns 32 query blocks
// of one head per wave and streams the competing pooled keys in tiles of 64
// through LDS (double buffered); in the MFMA layout the lanes l and l + 32
// hold the same query block's scores for different keys. Three selections:
//   top_k <= 16:     per-lane sorted register lists, merged at the end
//                    (gsa_topk_reg_kernel);
//   16 < top_k:      a score bound, then a filter and a wave-wide sort
//                    (gsa_topk_bound_kernel, gsa_topk_wide_kernel);
//   its fallback:    sorted per-block lists in LDS, inserted one half-wave at
//                    a time (gsa_topk_kernel), for the blocks the filter
//                    could not hold.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

constexpr int kTileN = 64;
constexpr int kTileBytes = kTileN * 128;      // one bf16 plane of a 64-key tile
constexpr int kStageBytes = 2 * kTileBytes;   // hi + lo planes

__device__ __forceinline__ int t_off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// Whether any lane of the wave holds p (a lane mask from one compare; HIP's
// __any materialises the predicate and compares it again).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

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

// only (nullable): per (head, query block) flags; a workgroup none of whose
// blocks is flagged returns at once (the wide kernel's overflow fallback).
// ---------------------------------------------------------------------------
// Key planes: the competing pooled keys split once into bf16 hi and lo parts,
// per head and key 64 hi values then 64 lo values (256 bytes), so that a
// 64-key tile is one contiguous 16 KiB run of a head that loads straight into
// LDS (16-byte buffer loads into LDS: no VGPR staging, no conversion in the
// selection loops).
// ---------------------------------------------------------------------------
constexpr int kPlaneRowBytes = 256;
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
// Lane l's 16 bytes at rsrc + voff land at lds_dst + 16 l (lds_dst wave-uniform);
// a lane reading past the extent gets zeros. The data is in LDS once vmcnt
// counts the load done.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_dst, 16,
                                           (int)voff, 0, 0, 0);
}

// Waits until this wave's direct-to-LDS loads have landed, then meets the other
// waves: every wave's share of the tile is in LDS. __syncthreads() alone does
// not suffice: its workgroup-scope fence waits for LDS accesses but not for
// vector memory loads, so another wave could read a stage before it is filled.
__device__ __forceinline__ void loads_landed_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); lgkmcnt and expcnt unconstrained
  __syncthreads();
}

// planes[h][key] = (hi[64], lo[64]) of scale * k_cmp[key, h, :] (fp32 product,
// then split): a thread per 8 values. scale 1 leaves the keys exact.
__global__ __launch_bounds__(256) void split_keys_kernel(const float* __restrict__ k_cmp, long long n_keys,
                                                        int n_heads, float scale, u32x4* __restrict__ planes) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_keys * n_heads * 8) return;
  const int chunk = (int)(i & 7);
  const long long kh = i >> 3;
  const long long key = kh / n_heads;
  const int h = (int)(kh % n_heads);
  const float* src = k_cmp + kh * kHeadDim + chunk * 8;
  float x[8];
  const f32x4 a = *reinterpret_cast<const f32x4*>(src);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e] * scale; x[4 + e] = b[e] * scale; }
  u32x4 hi, lo;
  split8(x, hi, lo);
  u32x4* dst = planes + ((long long)h * n_keys + key) * (kPlaneRowBytes / 16);
  dst[chunk] = hi;
  dst[8 + chunk] = lo;
}

// Loads 64-key tiles of one head's planes into an LDS stage laid out as the
// MFMA reads want it: the hi plane (8 KiB) then the lo plane, key row r at
// r * 128 bytes, logical 16-byte chunk c at physical chunk c ^ (r & 7). Each
// of the 256 threads issues 4 loads per tile; its source chunks are fixed.
struct PlaneTiles {
  const unsigned char* head;  // this head's planes at the first competing key
  long long n_keys;           // competing keys
  uint32_t voff[4];

  __device__ __forceinline__ void init(const void* planes, long long n_total, int h, long long first,
                                       long long n_cand, int tid) {
    head = static_cast<const unsigned char*>(planes) + ((long long)h * n_total + first) * kPlaneRowBytes;
    n_keys = n_cand;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = q * 4096 + tid * 16;      // LDS byte offset this thread fills
      const int plane = o >> 13, r = (o & 8191) >> 7, pc = (o >> 4) & 7;
      voff[q] = (uint32_t)(r * kPlaneRowBytes + plane * 128 + ((pc ^ (r & 7)) << 4));
    }
  }
  // keys u0 .. u0 + 63 into `stage` (rows past the end load as zeros)
  __device__ __forceinline__ void issue(long long u0, unsigned char* stage, int wave) const {
    const long long rows = min((long long)kTileN, n_keys - u0);
    const auto rsrc = buffer_rsrc(head + u0 * kPlaneRowBytes, rows * kPlaneRowBytes);
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_dma16(rsrc, voff[q], stage + q * 4096 + wave * 1024);
  }
};

__global__ __launch_bounds__(256) void gsa_topk_kernel(Geom g, const float* __restrict__ q_blk,
                                                       const float* __restrict__ k_cmp,
                                                       long long n_cand, int j0,
                                                       int top_k, int n_rowtiles,
                                                       const uint8_t* __restrict__ only,
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
  if (only != nullptr && !__syncthreads_or(rvalid && only[(long long)h * n_rows + row] != 0)) return;

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

    // both key halves against one query chunk back to back (a shared B
    // operand); each score keeps its product order lo.hi, hi.lo, hi.hi
    f32x16 s[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) { s[0][i] = 0.f; s[1][i] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 ah0 = ld16(hi_p + t_off(li, 2 * ks + hh));
      const u32x4 al0 = ld16(lo_p + t_off(li, 2 * ks + hh));
      const u32x4 ah1 = ld16(hi_p + t_off(32 + li, 2 * ks + hh));
      const u32x4 al1 = ld16(lo_p + t_off(32 + li, 2 * ks + hh));
      s[0] = mfma32(al0, qh[ks], s[0]);
      s[1] = mfma32(al1, qh[ks], s[1]);
      s[0] = mfma32(ah0, ql[ks], s[0]);
      s[1] = mfma32(ah1, ql[ks], s[1]);
      s[0] = mfma32(ah0, qh[ks], s[0]);
      s[1] = mfma32(ah1, qh[ks], s[1]);
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
    if (wave_any(rvalid && mx >= tau_s)) {
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
// Tiles between refreshes of the block-wide 16th best (top_k == 16).
#ifndef SGA_TOPK_UNION_EVERY
#define SGA_TOPK_UNION_EVERY 8
#endif
constexpr int kUnionEvery = SGA_TOPK_UNION_EVERY;

// Entry order: larger score first; equal scores, lower index first.
__device__ __forceinline__ bool better(float s, int j, float ts, int tj) {
  return s > ts || (s == ts && j < tj);
}

// Occupancy: 4 workgroups (4 waves per SIMD, 128 VGPRs); measured at 128 frames
// 2.46 ms against 2.76 ms at 3 waves per SIMD and 3.40 ms at 2.
// Listed rows (the blocks the two-stage selection could not certify): per
// head the first count[h] entries of rows[h][.] ([H][n_rows] int32). The list
// positions below `cap` (a multiple of 128) are split over n_seg key segments:
// workgroup (h, tile, seg) streams segment seg of the keys for list entries
// 128 tile .. 128 tile + 127 and stores each lane's list (exact scores, key
// indices) to seg_val / seg_idx [H][cap][n_seg][32], for the merge kernel.
// Positions from `cap` on stream all keys in segment 0's workgroup and write
// their result directly.
struct RegList {
  const int32_t* rows;
  const int32_t* count;
  int n_seg;
  int cap;
  float* seg_val;
  int32_t* seg_idx;
};

// list.rows == nullptr: workgroup w of head h selects rows 128 w .. 128 w + 127.
template <bool FULL>  // FULL: top_k == kRegK, the threshold is the list's last slot
__global__ __launch_bounds__(256, 4) void gsa_topk_reg_kernel(Geom g, const float* __restrict__ q_blk,
                                                           const void* __restrict__ planes,
                                                           long long n_total, long long n_cand, int j0,
                                                           int top_k, int n_rowtiles,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ score, RegList list) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int segs = list.rows != nullptr ? list.n_seg : 1;
  const int seg = blockIdx.x % segs;
  const int wg = blockIdx.x / segs;
  const int h = wg / n_rowtiles;
  const long long row0 = (long long)(wg % n_rowtiles) * 128;
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const long long rs = (long long)g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long pos = row0 + wave * 32 + li;  // the row, or the list position
  long long row = pos;
  bool rvalid = row < n_rows;
  bool split = false;
  const long long n_tiles_all = (n_cand + kTileN - 1) / kTileN;
  long long it0 = 0, it1 = n_tiles_all;
  if (list.rows != nullptr) {  // (uniform over the workgroup: it returns before any barrier)
    const long long cnt = list.count[h];
    if (row0 >= cnt) return;
    split = row0 < list.cap;
    if (!split && seg != 0) return;
    rvalid = pos < cnt;
    row = rvalid ? (long long)list.rows[(long long)h * n_rows + pos] : 0;
    if (split) {
      const long long per = (n_tiles_all + segs - 1) / segs;
      it0 = min(n_tiles_all, seg * per);
      it1 = min(n_tiles_all, it0 + per);
    }
  }

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

  PlaneTiles tiles;
  tiles.init(planes, n_total, h, j0, n_cand, tid);

  float lv[kRegK];
  int lj[kRegK];
#pragma unroll
  for (int p = 0; p < kRegK; ++p) { lv[p] = -INFINITY; lj[p] = 0x7fffffff; }
  float tau = -INFINITY;   // lv[top_k - 1]
  float tblk = -INFINITY;  // the 16th best of the block's two lists (top_k == 16)
  const int kth = top_k - 1;

  if (it0 < it1) tiles.issue(it0 * kTileN, smem, wave);

  for (long long it = it0; it < it1; ++it) {
    const int stage = (int)((it - it0) & 1);
    const long long u0 = it * kTileN;
    const bool more = it + 1 < it1;
    // tile it has landed in every wave's loads, and every wave is done with
    // the other stage
    loads_landed_barrier();
    if (more) tiles.issue(u0 + kTileN, smem + (stage ^ 1) * kStageBytes, wave);
    const unsigned char* hi_p = smem + stage * kStageBytes;
    const unsigned char* lo_p = hi_p + kTileBytes;

    // both key halves against one query chunk back to back (a shared B
    // operand); each score keeps its product order lo.hi, hi.lo, hi.hi
    f32x16 s[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) { s[0][i] = 0.f; s[1][i] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 ah0 = ld16(hi_p + t_off(li, 2 * ks + hh));
      const u32x4 al0 = ld16(lo_p + t_off(li, 2 * ks + hh));
      const u32x4 ah1 = ld16(hi_p + t_off(32 + li, 2 * ks + hh));
      const u32x4 al1 = ld16(lo_p + t_off(32 + li, 2 * ks + hh));
      s[0] = mfma32(al0, qh[ks], s[0]);
      s[1] = mfma32(al1, qh[ks], s[1]);
      s[0] = mfma32(ah0, ql[ks], s[0]);
      s[1] = mfma32(ah1, ql[ks], s[1]);
      s[0] = mfma32(ah0, qh[ks], s[0]);
      s[1] = mfma32(ah1, qh[ks], s[1]);
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
    // A block-wide bound on this lane's candidates: the partner lane holds
    // top_k keys of the block scoring at least its threshold, and (with 16
    // slots, refreshed every kUnionEvery tiles) the union of the two lists
    // holds 16 keys scoring at least its 16th best. A key scoring below either
    // cannot reach the block's final set; a key tying it still may (a lower
    // index wins), so it is kept.
    float tp;
    {
      const auto tsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tau), __float_as_uint(tau), false, false);
      tp = fmaxf(tblk, __uint_as_float(hh ? tsw[0] : tsw[1]));
    }
    if (wave_any(rvalid && mx > tau && mx >= tp)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float sv = s[kb][i];
          const bool c = rvalid && sv > tau && sv >= tp;
          if (wave_any(c)) {
            const int j = (int)u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            // Slot p of the new list is the median of (old p - 1, sv, old p):
            // the list is sorted, so that is old p - 1 when sv goes before it,
            // sv when it lands at p, old p otherwise. A lane that does not
            // insert (sv <= tau <= every slot up to top_k - 1) keeps those
            // slots; an invalid row's lane may change its list, never written.
            // Walk from the tail so slot p - 1 is read before it is written;
            // strict compares keep an equal score behind the earlier key.
#pragma unroll
            for (int p = kRegK - 1; p >= 1; --p) {
              const int tj = sv > lv[p] ? j : lj[p];
              lj[p] = sv > lv[p - 1] ? lj[p - 1] : tj;
              lv[p] = __builtin_amdgcn_fmed3f(lv[p - 1], sv, lv[p]);
            }
            lj[0] = sv > lv[0] ? j : lj[0];
            lv[0] = fmaxf(sv, lv[0]);
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
    if (FULL && (it % kUnionEvery) == kUnionEvery - 1) {
      // the union's 16th best: the best 16 of two lists sorted best first are
      // max(a[p], b[15 - p]) (as in the final merge), so their minimum
      float u = INFINITY;
#pragma unroll
      for (int p = 0; p < kRegK; ++p) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lv[kRegK - 1 - p]),
                                                        __float_as_uint(lv[kRegK - 1 - p]), false, false);
        u = fminf(u, fmaxf(lv[p], __uint_as_float(hh ? r[0] : r[1])));
      }
      tblk = u;
    }
  }

  if (split) {  // this segment's lists, for the merge kernel
    if (rvalid) {
      const long long base = (((long long)h * list.cap + pos) * segs + seg) * 32 + hh * 16;
#pragma unroll
      for (int p = 0; p < kRegK; ++p) {
        list.seg_val[base + p] = lv[p];
        list.seg_idx[base + p] = lj[p] == 0x7fffffff ? 0x7fffffff : lj[p] + j0;
      }
    }
    return;
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


// ---------------------------------------------------------------------------
// Two-stage selection for top_k <= 16 (the default path while a lane's key
// positions fit 16 bits, i.e. at most 2048 key tiles).
//
// Stage 1 (gsa_topk_approx_kernel) ranks by a single bf16 product per score,
// s1 = bf16(q/8) . bf16(k), one third of the exact path's matrix-core work. A
// list entry is one 32-bit word: the score's 16-bit order-preserving bucket
// (sign, exponent, 7 mantissa bits) above a 16-bit inverted lane position, so
// a larger word is a higher bucket or, within a bucket, an earlier key, and the
// insertion network is one v_med3_u32 per slot. Each lane keeps its 16 best
// words; a key enters iff its bucket is above the 16th word's bucket, i.e.
// iff s1 reaches that bucket's upper edge U. Every key a lane drops therefore
// has s1 < U of the lane's final 16th word.
//
// Stage 2 (gsa_topk_rescore_kernel) scores the block's 32 candidates exactly
// (fp32, the same arithmetic for every candidate), sorts them (larger score
// first, ties to the lower index) and certifies the result: with
//   |s1 - s| <= (2^-7 + 2^-16 + 2^-17) sum_i |q_i k_i| <= 2^-6.9 |q| max|k|
// (bf16 rounding of both operands, 64 fp32 additions) as the bound E, a
// dropped key scores below max(U_A, U_B) + E, so when the K-th best candidate
// scores strictly above that, the candidates' top-K is the block's top-K.
// Blocks that miss the certificate (about 1% at 1000 frames, top-16) are
// listed per head and selected again by the exact register kernel.
// ---------------------------------------------------------------------------
constexpr int kApproxMaxTiles = 2048;  // lane positions (32 per tile) fit 16 bits
constexpr int kKnormChunks = 256;      // partial maxima of |k|^2 per head

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_order_key(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
// The smallest score whose bucket lies above the bucket of list word w (w != 0).
__device__ __forceinline__ float bucket_upper(uint32_t w) {
  const uint32_t b = w >> 16;
  return b >= 0xff7fu ? INFINITY : from_order_key((b + 1u) << 16);
}
__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

// Per (head, chunk) maximum of |k|^2 over the fp32 pooled keys; workgroup 0
// also clears the per-head counts of the blocks stage 2 cannot certify.
__global__ __launch_bounds__(256) void kmax_partial_kernel(const float* __restrict__ k_cmp, long long n_keys,
                                                           int n_heads, float* __restrict__ out,
                                                           int32_t* __restrict__ fail_count) {
  if (blockIdx.x == 0 && (int)threadIdx.x < n_heads) fail_count[threadIdx.x] = 0;
  const int h = blockIdx.x / kKnormChunks, chunk = blockIdx.x % kKnormChunks;
  const long long per = (n_keys + kKnormChunks - 1) / kKnormChunks;
  const long long r0 = chunk * per, r1 = min(r0 + per, n_keys);
  const int t = threadIdx.x, part = t & 7;
  float best = 0.f;
  for (long long r = r0 + (t >> 3); r < r1; r += 32) {
    const float* kp = k_cmp + (r * n_heads + h) * kHeadDim + part * 8;
    const f32x4 a = *reinterpret_cast<const f32x4*>(kp);
    const f32x4 b = *reinterpret_cast<const f32x4*>(kp + 4);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(a[e], a[e], fmaf(b[e], b[e], acc));
#pragma unroll
    for (int sh = 1; sh < 8; sh <<= 1) acc += __shfl_xor(acc, sh);
    best = fmaxf(best, acc);
  }
#pragma unroll
  for (int sh = 8; sh < 64; sh <<= 1) best = fmaxf(best, __shfl_xor(best, sh));
  __shared__ float wmax[4];
  if ((t & 63) == 0) wmax[t >> 6] = best;
  __syncthreads();
  if (t == 0) out[blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// Stage 1: a workgroup owns 128 query blocks of one head (32 per wave) and
// streams the hi plane of the competing keys through LDS, double buffered;
// cand[h][row][32] receives lane hh = 0's 16 words then lane hh = 1's, each
// lane's list best first.
__global__ __launch_bounds__(256, 4) void gsa_topk_approx_kernel(Geom g, const float* __restrict__ q_blk,
                                                              const void* __restrict__ planes,
                                                              long long n_total, long long n_cand, int j0,
                                                              int n_rowtiles, uint32_t* __restrict__ cand) {
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

  // pooled-query operand: bf16(q / 8) (the scale is exact)
  u32x4 qh[4];
  {
    const float* qp = q_blk + (rvalid ? row : 0) * rs + hoff + hh * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(qp + ks * 16);
      const f32x4 b = *reinterpret_cast<const f32x4*>(qp + ks * 16 + 4);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        qh[ks][e] = rvalid ? pack_bf16x2(a[2 * e] * 0.125f, a[2 * e + 1] * 0.125f) : 0u;
        qh[ks][2 + e] = rvalid ? pack_bf16x2(b[2 * e] * 0.125f, b[2 * e + 1] * 0.125f) : 0u;
      }
    }
  }

  // hi plane of a 64-key tile: key row r (128 B) at r * 128 in the stage,
  // logical chunk c at physical chunk c ^ (r & 7); two 16-byte loads per thread
  const unsigned char* head = static_cast<const unsigned char*>(planes) +
                              ((long long)h * n_total + j0) * kPlaneRowBytes;
  uint32_t voff[2];
#pragma unroll
  for (int qd = 0; qd < 2; ++qd) {
    const int o = qd * 4096 + tid * 16;
    const int r = o >> 7, pc = (o >> 4) & 7;
    voff[qd] = (uint32_t)(r * kPlaneRowBytes + ((pc ^ (r & 7)) << 4));
  }
  auto issue = [&](long long u0, unsigned char* stage) {
    const long long rows = min((long long)kTileN, n_cand - u0);
    const auto rsrc = buffer_rsrc(head + u0 * kPlaneRowBytes, rows * kPlaneRowBytes);
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) lds_dma16(rsrc, voff[qd], stage + qd * 4096 + wave * 1024);
  };

  uint32_t lv[kRegK];
#pragma unroll
  for (int p = 0; p < kRegK; ++p) lv[p] = 0u;  // 0: empty (no real score maps to word 0)
  // a key enters iff s1 >= ut: any finite key while the list is not full; no
  // key of a row past the end
  constexpr float kAnyFinite = -3.4028234663852886e38f;
  float ut = rvalid ? kAnyFinite : INFINITY;

  const int n_tiles = (int)((n_cand + kTileN - 1) / kTileN);
  issue(0, smem);
  for (int it = 0; it < n_tiles; ++it) {
    const int stage = it & 1;
    const long long u0 = (long long)it * kTileN;
    const bool more = it + 1 < n_tiles;
    loads_landed_barrier();
    if (more) issue(u0 + kTileN, smem + (stage ^ 1) * kTileBytes);
    const unsigned char* hi_p = smem + stage * kTileBytes;

    f32x16 s[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) { s[0][i] = 0.f; s[1][i] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 a0 = ld16(hi_p + t_off(li, 2 * ks + hh));
      const u32x4 a1 = ld16(hi_p + t_off(32 + li, 2 * ks + hh));
      s[0] = mfma32(a0, qh[ks], s[0]);
      s[1] = mfma32(a1, qh[ks], s[1]);
    }
    if (!more) {  // the last tile: keys past the end score -inf (never enter)
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
    if (wave_any(mx >= ut)) {
      // ut is refreshed once per tile: a stale (lower) threshold only lets more
      // keys through the network, which keeps the best 16 words either way
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float sv = s[kb][i];
          const bool c = sv >= ut;
          if (wave_any(c)) {
            // the new word, or 0 (below every slot: the list stays) where the
            // lane does not take this key; slot p becomes the median of
            // (old p - 1, new, old p), walking from the tail
            const uint32_t pos = (uint32_t)(it * 32 + kb * 16 + i);
            const uint32_t x = c ? ((order_key(sv) & 0xffff0000u) | (0xffffu - pos)) : 0u;
#pragma unroll
            for (int p = kRegK - 1; p >= 1; --p) lv[p] = med3u(lv[p - 1], x, lv[p]);
            lv[0] = max(lv[0], x);
          }
        }
      if (rvalid) ut = lv[kRegK - 1] ? bucket_upper(lv[kRegK - 1]) : kAnyFinite;
    }
  }
  if (rvalid) {
    u32x4* dst = reinterpret_cast<u32x4*>(cand + ((long long)h * n_rows + row) * 32 + hh * 16);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) dst[c4] = u32x4{lv[4 * c4], lv[4 * c4 + 1], lv[4 * c4 + 2], lv[4 * c4 + 3]};
  }
}

// Stage 2: 32 lanes per (head, query block), lane c holding candidate c of
// the block's two lists. Exact fp32 scores, a bitonic sort across the 32
// lanes, the certificate, then the block's top_k (ascending indices) or its
// entry in the head's list of blocks for the exact kernel.
__global__ __launch_bounds__(256) void gsa_topk_rescore_kernel(Geom g, const float* __restrict__ q_blk,
                                                               const float* __restrict__ k_cmp, int j0,
                                                               int top_k, const uint32_t* __restrict__ cand,
                                                               const float* __restrict__ kmax_part,
                                                               int32_t* __restrict__ idx, float* __restrict__ score,
                                                               int32_t* __restrict__ fail_count,
                                                               int32_t* __restrict__ fail_rows) {
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const long long pair = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
  const int c = threadIdx.x & 31;
  const int lane = threadIdx.x & 63;
  const bool pvalid = pair < n_rows * g.n_heads;
  const long long pr = pvalid ? pair : 0;
  const int h = (int)(pr / n_rows);
  const long long row = pr % n_rows;
  const long long rs = (long long)g.n_heads * kHeadDim;

  // max |k| of the head (partials of |k|^2, rounded up for their own fp32 error)
  float k2 = 0.f;
  for (int i = c; i < kKnormChunks; i += 32) k2 = fmaxf(k2, kmax_part[h * kKnormChunks + i]);
#pragma unroll
  for (int sh = 1; sh < 32; sh <<= 1) k2 = fmaxf(k2, __shfl_xor(k2, sh));
  const float kmax = sqrtf(k2 * 1.0001f);

  const uint32_t w = cand[pr * 32 + c];
  const uint32_t wa = __shfl(w, (lane & 32) + 15);   // lane hh = 0's 16th word
  const uint32_t wb = __shfl(w, (lane & 32) + 31);   // lane hh = 1's
  // candidate c's key: list c / 16, lane position p = 0xffff - (low 16 bits)
  long long j = 0x7fffffffffffLL;
  float sc = -INFINITY;
  const float* qp = q_blk + row * rs + (long long)h * kHeadDim;
  float q2 = 0.f;
  if (w != 0u) {
    const int p = 0xffff - (int)(w & 0xffffu);
    const int hh = c >> 4;
    const long long jl = (long long)(p >> 5) * kTileN + ((p >> 4) & 1) * 32 + 8 * ((p >> 2) & 3) + 4 * hh + (p & 3);
    j = jl + j0;
    const float* kp = k_cmp + (j * g.n_heads + h) * kHeadDim;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < kHeadDim; e += 4) {
      const f32x4 qa = *reinterpret_cast<const f32x4*>(qp + e);
      const f32x4 ka = *reinterpret_cast<const f32x4*>(kp + e);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = fmaf(qa[r] * 0.125f, ka[r], acc);
    }
    sc = acc;
  }
#pragma unroll
  for (int e = 0; e < kHeadDim; e += 4) {
    const f32x4 qa = *reinterpret_cast<const f32x4*>(qp + e);
#pragma unroll
    for (int r = 0; r < 4; ++r) q2 = fmaf(qa[r] * 0.125f, qa[r] * 0.125f, q2);
  }
  // bitonic sort across the 32 lanes: larger score first, ties to the lower key
  int jj = (int)min(j, 0x7fffffffLL);
#pragma unroll
  for (int size = 2; size <= 32; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride >= 1; stride >>= 1) {
      const float os = __shfl_xor(sc, stride);
      const int oj = __shfl_xor(jj, stride);
      const bool other_better = os > sc || (os == sc && oj < jj);
      const bool lower = (c & stride) == 0;          // this lane keeps the better of the pair ...
      const bool desc = (c & size) == 0 || size == 32;  // ... in a descending run
      const bool take = (lower == desc) ? other_better : !other_better;
      if (take) { sc = os; jj = oj; }
    }
  // certificate
  const float sk = __shfl(sc, (lane & 32) + top_k - 1);
  const float ua = wa ? bucket_upper(wa) : -INFINITY;
  const float ub = wb ? bucket_upper(wb) : -INFINITY;
  const float e_bound = 0.0083733f * sqrtf(q2) * kmax + 1e-30f;   // 2^-6.9 |q/8| max|k|
  const bool certified = sk > fmaxf(ua, ub) + e_bound;
  // each of the first top_k lanes: its key's rank by index among them
  int rank = 0;
  for (int o = 0; o < top_k; ++o) {
    const int oj = __shfl(jj, (lane & 32) + o);
    rank += (oj < jj) ? 1 : 0;
  }
  if (!pvalid) return;
  if (certified) {
    if (c < top_k) {
      idx[pr * top_k + rank] = jj;
      if (score) score[pr * top_k + rank] = sc;
    }
  } else if (c == 0) {
    const int at = atomicAdd(&fail_count[h], 1);
    fail_rows[(long long)h * n_rows + at] = (int32_t)row;
  }
}

// The split fallback's merge: one wave per listed block gathers the n_seg x 2
// segment lists (n_seg / 2 entries per lane), takes the top_k by top_k rounds
// of a wave-wide best (larger score, then lower index), and writes them in
// ascending index order.
constexpr int kFallbackSegs = 8;
constexpr int kFallbackCap = 4096;  // listed rows per head taken in split mode

__device__ __forceinline__ bool seg_better(float s, int j, float ts, int tj) {
  return s > ts || (s == ts && j < tj);
}

__global__ __launch_bounds__(256) void gsa_topk_seg_merge_kernel(Geom g, int top_k, int cap,
                                                                 const int32_t* __restrict__ rows,
                                                                 const int32_t* __restrict__ count,
                                                                 const float* __restrict__ seg_val,
                                                                 const int32_t* __restrict__ seg_idx,
                                                                 int32_t* __restrict__ idx,
                                                                 float* __restrict__ score) {
  constexpr int kPer = kFallbackSegs * 32 / 64;  // entries per lane
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const int lane = threadIdx.x & 63;
  const long long wv = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int h = (int)(wv / cap);
  const long long pos = wv % cap;
  if (h >= g.n_heads) return;
  const long long cnt = min((long long)count[h], (long long)cap);
  if (pos >= cnt) return;  // (uniform over the wave)
  const long long base = ((long long)h * cap + pos) * kFallbackSegs * 32;
  float v[kPer];
  int j[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    v[e] = seg_val[base + e * 64 + lane];
    j[e] = seg_idx[base + e * 64 + lane];
    if (j[e] == 0x7fffffff) v[e] = -INFINITY;
  }
  float win_v = -INFINITY;
  int win_j = 0x7fffffff;
  for (int k = 0; k < top_k; ++k) {
    float bv = v[0];
    int bj = j[0];
#pragma unroll
    for (int e = 1; e < kPer; ++e)
      if (seg_better(v[e], j[e], bv, bj)) { bv = v[e]; bj = j[e]; }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const float ov = __shfl_xor(bv, sh);
      const int oj = __shfl_xor(bj, sh);
      if (seg_better(ov, oj, bv, bj)) { bv = ov; bj = oj; }
    }
    if (lane == k) { win_v = bv; win_j = bj; }
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (j[e] == bj) { v[e] = -INFINITY; j[e] = 0x7fffffff; }
  }
  int rank = 0;
  for (int o = 0; o < top_k; ++o) rank += (__shfl(win_j, o) < win_j) ? 1 : 0;
  if (lane < top_k) {
    const long long row = rows[(long long)h * n_rows + pos];
    idx[((long long)h * n_rows + row) * top_k + rank] = win_j;
    if (score) score[((long long)h * n_rows + row) * top_k + rank] = win_v;
  }
}

// ---------------------------------------------------------------------------
// Wide selection, kRegK < top_k <= 128: bound, filter, sort.
//
// 1. Bound (gsa_topk_bound_kernel). Every other 64-key tile is scored; for
//    each of its 32 score positions in a tile (a fixed residue of the key
//    index mod 64) a lane keeps the DEPTH largest scores seen: 32*DEPTH values
//    per lane from disjoint key buckets, all distinct candidates. K distinct
//    candidates scoring at least x make x a lower bound of the block's K-th
//    best score, so min(the ceil(K/2)-th value of one lane, the floor(K/2)-th
//    of the other) is one. DEPTH is 2 up to top-64 and 4 beyond.
// 2. Filter (gsa_topk_wide_kernel). All keys are scored again; every score at
//    or above the bound is appended, as a 64-bit key (order-preserving score
//    bits, then the inverted index, so a larger key is the better candidate
//    under the tie rule), to the lane's own region of its workgroup's buffer;
//    the count keeps going past the region.
// 3. Select (same kernel). One wave per query block loads the block's keys,
//    sorts them with a bitonic network across the wave (2 to 16 keys per
//    lane), keeps the first top_k and writes their indices in ascending order.
// A block with a lane past its region (heavy ties, adversarial scores) is
// flagged and recomputed afterwards by the LDS-list kernel, which is exact
// with the same tie rule. The filter kernel is persistent, one workgroup per
// buffer slot, so the buffer scales with the machine, not with the problem.
// ---------------------------------------------------------------------------
constexpr int kWideCap = 512;                      // appended keys per lane
constexpr int kWideRows = 128;                     // query blocks per workgroup
constexpr long long kWideMaxSlots = 1024;          // buffer slots (persistent workgroups)
constexpr long long kWideSlotKeys = (long long)kWideRows * 2 * kWideCap;

// One head's competing pooled keys streamed through LDS in 64-key tiles
// (double buffered) and scored against each lane's pooled query with the
// three-term split; visit(s, u0) gets the lane's 32 scores of a tile (keys
// past the end scored -inf).
struct ScoreStream {
  unsigned char* smem;
  PlaneTiles tiles;
  long long n_cand, rs, hoff;
  int tid, wave, li, hh;
  u32x4 qh[4], ql[4];

  __device__ __forceinline__ void load_q(const float* q_blk, long long row, bool rvalid) {
    // scaled by 1/sqrt(64) = 1/8 (exact), hi and lo planes
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
  // tiles it = 0, stride, 2*stride, ... of the key range
  template <class Visit>
  __device__ __forceinline__ void run(int stride, Visit&& visit) {
    const long long n_ktiles = (n_cand + kTileN - 1) / kTileN;
    __syncthreads();  // every wave is done with the stages of a previous stream
    tiles.issue(0, smem, wave);
    int stage = 0;
    for (long long it = 0; it < n_ktiles; it += stride) {
      const long long u0 = it * kTileN;
      const bool more = it + stride < n_ktiles;
      // tile it has landed in every wave's loads, and every wave is done with
      // the other stage
      loads_landed_barrier();
      if (more) tiles.issue(u0 + (long long)stride * kTileN, smem + (stage ^ 1) * kStageBytes, wave);
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
      if (u0 + kTileN > n_cand) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const long long j = u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (j >= n_cand) s[kb][i] = -INFINITY;
          }
      }
      visit(s, u0);
      stage ^= 1;
    }
  }
};

template <int DEPTH>
__global__ __launch_bounds__(256, 2) void gsa_topk_bound_kernel(Geom g, const float* __restrict__ q_blk,
                                                               const void* __restrict__ planes,
                                                               long long n_total, long long first,
                                                               long long n_cand, int top_k,
                                                               int n_rowtiles,
                                                               float* __restrict__ bound) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int V = 32 * DEPTH;  // values per lane
  const int h = blockIdx.x / n_rowtiles;
  const long long row0 = (long long)(blockIdx.x % n_rowtiles) * kWideRows;
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long row = row0 + wave * 32 + li;
  const bool rvalid = row < n_rows;

  ScoreStream st;
  st.smem = smem;
  st.tiles.init(planes, n_total, h, first, n_cand, tid);
  st.n_cand = n_cand;
  st.rs = (long long)g.n_heads * kHeadDim;
  st.hoff = (long long)h * kHeadDim;
  st.tid = tid;
  st.wave = wave;
  st.li = li;
  st.hh = hh;
  st.load_q(q_blk, row, rvalid);

  // m[d * 32 + p]: the (d+1)-th largest score seen at position p
  float m[V];
#pragma unroll
  for (int p = 0; p < V; ++p) m[p] = -INFINITY;
  st.run(2, [&](const f32x16 (&s)[2], long long) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = kb * 16 + i;
        float x = s[kb][i];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {  // x sinks to its place; the smallest falls off
          const float hi = fmaxf(m[d * 32 + p], x);
          x = fminf(m[d * 32 + p], x);
          m[d * 32 + p] = hi;
        }
      }
  });
  // the c-th largest of the lane's V values, by a bitwise search over their
  // order-preserving integer images: the largest t with c values >= t
  uint32_t o[V];
#pragma unroll
  for (int p = 0; p < V; ++p) {
    const uint32_t u = __float_as_uint(m[p]);
    o[p] = u ^ ((u & 0x80000000u) ? 0xffffffffu : 0x80000000u);
  }
  auto kth = [&](int c) {
    uint32_t t = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      int n = 0;
#pragma unroll
      for (int p = 0; p < V; ++p) n += o[p] >= cand ? 1 : 0;
      t = n >= c ? cand : t;
    }
    return __uint_as_float(t ^ ((t & 0x80000000u) ? 0x80000000u : 0xffffffffu));
  };
  const float x_hi = kth((top_k + 1) / 2);
  const float x_lo = kth(top_k / 2);
  // lane l < 32 contributes its ceil(K/2)-th value, lane l + 32 its floor(K/2)-th
  const float mine = hh == 0 ? x_hi : x_lo;
  const float tau = fminf(mine, __shfl_xor(mine, 32, 64));
  if (rvalid && hh == 0) bound[(long long)h * n_rows + row] = tau;
}

__device__ __forceinline__ uint64_t order_key(float s, int j) {
  uint32_t u = __float_as_uint(s);
  u ^= (u & 0x80000000u) ? 0xffffffffu : 0x80000000u;
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xffffffffu - (uint32_t)key); }
__device__ __forceinline__ float key_score(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u ^= (u & 0x80000000u) ? 0x80000000u : 0xffffffffu;
  return __uint_as_float(u);
}

// Bitonic sort, descending, of the 64*E keys of a wave held lane-major
// (key e = lane*E + r in a[r] of lane e/E).
template <int E>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&a)[E], int lane) {
#pragma unroll
  for (int k = 2; k <= 64 * E; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= E) {  // partners in lane ^ (j / E), same register
        const int lm = j / E;
        const bool lower = (lane & lm) == 0;
        const bool desc = ((lane * E) & k) == 0;
        const bool take_max = lower == desc;
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const uint64_t o = __shfl_xor(a[r], lm, 64);
          const bool keep = take_max ? (a[r] > o) : (a[r] < o);
          a[r] = keep ? a[r] : o;
        }
      } else {       // partners in the same lane
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const int p = r ^ j;
          if (p > r) {
            const bool desc = (k >= E) ? (((lane * E) & k) == 0) : ((r & k) == 0);
            const uint64_t x = a[r], y = a[p];
            const bool sw = desc ? (x < y) : (x > y);
            a[r] = sw ? y : x;
            a[p] = sw ? x : y;
          }
        }
      }
    }
  }
}

// Sorts a query block's n0 + n1 appended keys (E per lane), keeps the first
// top_k and writes their indices (+ j0) ascending, with their scores.
template <int E>
__device__ __forceinline__ void select_block(const uint64_t* __restrict__ rb, int n0, int n1,
                                             int top_k, int lane, uint64_t* lds, int j0,
                                             int32_t* __restrict__ ip, float* __restrict__ sp) {
  uint64_t a[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int e = lane * E + r;
    a[r] = e < n0 ? rb[e] : (e < n0 + n1 ? rb[kWideCap + e - n0] : 0ull);
  }
  wave_sort_desc<E>(a, lane);
#pragma unroll
  for (int r = 0; r < E; ++r)
    if (lane * E + r < top_k) lds[lane * E + r] = a[r];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int e = lane; e < top_k; e += 64) {
    const uint64_t key = lds[e];
    const int j = key_index(key);
    int pos = 0;
    for (int f = 0; f < top_k; ++f) pos += key_index(lds[f]) < j ? 1 : 0;
    ip[pos] = j + j0;
    if (sp) sp[pos] = key_score(key);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

__global__ __launch_bounds__(256, 3) void gsa_topk_wide_kernel(Geom g, const float* __restrict__ q_blk,
                                                              const void* __restrict__ planes,
                                                              long long n_total,
                                                              long long n_cand, int j0, int top_k,
                                                              int n_rowtiles, long long n_tiles,
                                                              const float* __restrict__ bound,
                                                              uint64_t* __restrict__ buf,
                                                              uint8_t* __restrict__ flags,
                                                              int32_t* __restrict__ idx,
                                                              float* __restrict__ score) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* sel_lds = reinterpret_cast<uint64_t*>(smem + 2 * kStageBytes);
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  uint64_t* slot = buf + (long long)blockIdx.x * kWideSlotKeys;
  uint64_t* my_keys = slot + ((long long)(wave * 32 + li) * 2 + hh) * kWideCap;
  uint64_t* wave_lds = sel_lds + wave * 128;

  ScoreStream st;
  st.smem = smem;
  st.n_cand = n_cand;
  st.rs = (long long)g.n_heads * kHeadDim;
  st.tid = tid;
  st.wave = wave;
  st.li = li;
  st.hh = hh;

  for (long long t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int h = (int)(t / n_rowtiles);
    const long long row0 = (t % n_rowtiles) * kWideRows;
    const long long row = row0 + wave * 32 + li;
    const bool rvalid = row < n_rows;
    st.hoff = (long long)h * kHeadDim;
    st.tiles.init(planes, n_total, h, j0, n_cand, tid);
    st.load_q(q_blk, row, rvalid);
    const float tau = rvalid ? bound[(long long)h * n_rows + row] : INFINITY;

    // ---- filter: append every score >= tau ------------------------------------
    int cnt = 0;
    st.run(1, [&](const f32x16 (&s)[2], long long u0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float sv = s[kb][i];
          const bool c = sv >= tau && sv > -INFINITY;
          if (wave_any(c)) {
            if (c) {
              const int j = (int)u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
              if (cnt < kWideCap) my_keys[cnt] = order_key(sv, j);
              ++cnt;
            }
          }
        }
    });
    const int other = __shfl_xor(cnt, 32, 64);
    const bool over = cnt > kWideCap || other > kWideCap || cnt + other < top_k;
    if (rvalid && hh == 0) flags[(long long)h * n_rows + row] = over ? 1 : 0;
    // the keys were written by other lanes of this wave, through the vector
    // caches: make them visible to the loads below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // ---- select: one query block at a time per wave ---------------------------
    for (int r = 0; r < 32; ++r) {
      const long long brow = row0 + wave * 32 + r;
      if (brow >= n_rows) break;
      const int n0 = __builtin_amdgcn_readlane(cnt, r);
      const int n1 = __builtin_amdgcn_readlane(cnt, r + 32);
      if (n0 > kWideCap || n1 > kWideCap || n0 + n1 < top_k) continue;
      const uint64_t* rb = slot + (long long)(wave * 32 + r) * 2 * kWideCap;
      int32_t* ip = idx + ((long long)h * n_rows + brow) * top_k;
      float* sp = score ? score + ((long long)h * n_rows + brow) * top_k : nullptr;
      const int n = n0 + n1;
      if (n <= 128) select_block<2>(rb, n0, n1, top_k, lane, wave_lds, j0, ip, sp);
      else if (n <= 256) select_block<4>(rb, n0, n1, top_k, lane, wave_lds, j0, ip, sp);
      else if (n <= 512) select_block<8>(rb, n0, n1, top_k, lane, wave_lds, j0, ip, sp);
      else select_block<16>(rb, n0, n1, top_k, lane, wave_lds, j0, ip, sp);
    }
  }
}

// Workgroups of a kernel that fit on the device at once.

// ---------------------------------------------------------------------------
// Probability-mean block scores (the block score read as probabilities: the
// mean over a query block's tokens of their compressed-branch softmax
// probabilities, Speed3R technical summary section 2.1), top_k <= 16.
//
// The key planes hold log2(e) k~ (fp32 product, then split), so the products
// below are logits in log2 units.
// 1. gsa_token_lse_kernel: every token's log-sum-exp over all pooled keys. The
//    token's bf16 query times 1/8 is exact in bf16, so two bf16 products per
//    operand chunk (q k_hi + q k_lo) give fp32-accurate logits; the layout is
//    the selection's (S^T = K Q^T, a lane per token, its 32 of every 64 keys),
//    with an online log-sum-exp per lane, merged with the partner lane.
// 2. gsa_topk_prob_kernel: a wave takes two query blocks, their member tokens
//    as the 32 MFMA rows (S = Q K^T: a lane per key, 8 rows of each block in
//    each half-wave). A block's probability sum for a key is the lane's 8
//    terms plus its partner's; the lane of the first half keeps the first
//    block's register list (the keys = its lane mod 32), the second half the
//    second block's, and at the end the 32 lists of a block are sorted
//    together.
// ---------------------------------------------------------------------------

// Token row of member m (0..15) of query block b, or -1 for an empty slot (a
// window's out-of-grid position, a specials block's slot >= S, b past the end).
__device__ __forceinline__ long long member_row(const Geom& g, long long b, int m) {
  if (b >= (long long)g.n_frames * g.nqb) return -1;
  const int f = (int)(b / g.nqb), j = (int)(b % g.nqb);
  const long long base = (long long)f * g.L;
  if (j == g.nb) return m < g.n_special ? base + m : -1;
  const int r = 4 * (j / g.nbw) + (m >> 2), c = 4 * (j % g.nbw) + (m & 3);
  if (r >= g.grid_h || c >= g.grid_w) return -1;
  return base + g.n_special + (long long)r * g.grid_w + c;
}

// The 8 values d = 16 ks + 8 hh .. + 7 of a bf16 row times 1/8 (exact), or 0.
__device__ __forceinline__ void load_row_eighth(const bf16* row, bool valid, int hh, u32x4 (&x)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 w = valid ? ld16(row + hh * 8 + ks * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) x[ks][j] = pack_bf16x2(lo_bf16(w[j]) * 0.125f, hi_bf16(w[j]) * 0.125f);
  }
}

// lse2[t, h] = log2 sum_j exp2(s_tj log2 e), s_tj = q_t . k~_j / 8, over all
// n_total pooled keys (planes of log2(e) k~); 128 tokens of one head per
// workgroup.
__global__ __launch_bounds__(256, 4) void gsa_token_lse_kernel(Geom g, const bf16* __restrict__ q,
                                                              const void* __restrict__ planes,
                                                              long long n_total, int n_rowtiles,
                                                              float* __restrict__ lse2) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int h = blockIdx.x / n_rowtiles;
  const long long row0 = (long long)(blockIdx.x % n_rowtiles) * 128;
  const long long rs = (long long)g.n_heads * kHeadDim;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long t = row0 + wave * 32 + li;
  const bool tvalid = t < g.T;
  u32x4 qb[4];
  load_row_eighth(q + (tvalid ? t : 0) * rs + (long long)h * kHeadDim, tvalid, hh, qb);

  PlaneTiles tiles;
  tiles.init(planes, n_total, h, 0, n_total, tid);
  // m2: the lane's reference (log2 units), l: the sum of exp2(s - m2) over the
  // lane's keys so far. The accumulators start at -m2, so the MFMA returns
  // s - m2 and a term costs one exp2. The reference moves only on the first
  // tile (to its maximum) and when a tile's terms sum past 2^32, where that
  // tile is taken again against its own maximum.
  float m2 = 0.f, l = 0.f;
  const long long n_tiles = (n_total + kTileN - 1) / kTileN;
  tiles.issue(0, smem, wave);
  for (long long it = 0; it < n_tiles; ++it) {
    const int stage = (int)(it & 1);
    const long long u0 = it * kTileN;
    const bool more = it + 1 < n_tiles;
    loads_landed_barrier();
    if (more) tiles.issue(u0 + kTileN, smem + (stage ^ 1) * kStageBytes, wave);
    const unsigned char* hi_p = smem + stage * kStageBytes;
    const unsigned char* lo_p = hi_p + kTileBytes;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = -m2;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 ah = ld16(hi_p + t_off(kb * 32 + li, 2 * ks + hh));
        const u32x4 al = ld16(lo_p + t_off(kb * 32 + li, 2 * ks + hh));
        acc = mfma32(al, qb[ks], acc);
        acc = mfma32(ah, qb[ks], acc);
      }
      s[kb] = acc;
    }
    if (!more) {  // the last tile: keys past the end take no part
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const long long j = u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (j >= n_total) s[kb][i] = -INFINITY;
        }
    }
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ts += __builtin_amdgcn_exp2f(s[kb][i]);
    if (it == 0 || !(ts <= 0x1p32f)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      // (a lane whose keys in this tile all lie past the end keeps its
      // reference: -inf - -inf would be NaN)
      const float sh = mx > -INFINITY ? mx : 0.f;
      ts = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) ts += __builtin_amdgcn_exp2f(s[kb][i] - sh);
      // (on the first tile l is 0 and sh may lie far below the start value)
      l = it == 0 ? 0.f : l * __builtin_amdgcn_exp2f(-sh);
      m2 += sh;
    }
    l += ts;
  }
  // a lane with no key at all (only when every key fits one tile) holds l = 0
  const float me = l > 0.f ? m2 : -INFINITY;
  const float mo = __shfl_xor(me, 32), lo = __shfl_xor(l, 32);
  const float mm = fmaxf(me, mo);
  const float lt = l * __builtin_amdgcn_exp2f(me - mm) + lo * __builtin_amdgcn_exp2f(mo - mm);
  if (tvalid && hh == 0) lse2[t * g.n_heads + h] = mm + __log2f(lt);
}

constexpr int kProbBlocksPerWG = 8;  // two query blocks per wave

template <bool FULL>  // FULL: top_k == kRegK
__global__ __launch_bounds__(256, 3) void gsa_topk_prob_kernel(Geom g, const bf16* __restrict__ q,
                                                              const void* __restrict__ planes,
                                                              long long n_total, long long n_cand, int j0,
                                                              int top_k, const float* __restrict__ lse2,
                                                              int n_wg_per_head, int32_t* __restrict__ idx,
                                                              float* __restrict__ score) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int h = blockIdx.x / n_wg_per_head;
  const long long wg = blockIdx.x % n_wg_per_head;
  const long long n_qb = (long long)g.n_frames * g.nqb;
  const long long rs = (long long)g.n_heads * kHeadDim;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long b_wave = wg * kProbBlocksPerWG + 2 * wave;

  // A operand: MFMA row li = member li % 16 of block b_wave + li / 16
  u32x4 qa[4];
  {
    const long long r = member_row(g, b_wave + (li >> 4), li & 15);
    load_row_eighth(q + (r >= 0 ? r : 0) * rs + (long long)h * kHeadDim, r >= 0, hh, qa);
  }
  // this lane's 16 result rows m = 8 (i / 4) + 4 hh + i % 4 (i < 8: block
  // b_wave, else b_wave + 1) take -lse2 of their token, -inf for an empty slot
  float nl[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = 8 * (i >> 2) + 4 * hh + (i & 3);
    const long long r = member_row(g, b_wave + (m >> 4), m & 15);
    nl[i] = r >= 0 ? -lse2[r * g.n_heads + h] : -INFINITY;
  }
  // the block whose list this lane keeps (first half: b_wave), its token count
  int cnt = 0;
#pragma unroll
  for (int m = 0; m < 16; ++m) cnt += member_row(g, b_wave + hh, m) >= 0 ? 1 : 0;
  const float inv = cnt > 0 ? 1.f / (float)cnt : 0.f;

  PlaneTiles tiles;
  tiles.init(planes, n_total, h, j0, n_cand, tid);
  float lv[kRegK];
  int lj[kRegK];
#pragma unroll
  for (int p = 0; p < kRegK; ++p) { lv[p] = -INFINITY; lj[p] = 0x7fffffff; }
  float tau = -INFINITY;
  const int kth = top_k - 1;

  const long long n_tiles = (n_cand + kTileN - 1) / kTileN;
  tiles.issue(0, smem, wave);
  for (long long it = 0; it < n_tiles; ++it) {
    const int stage = (int)(it & 1);
    const long long u0 = it * kTileN;
    const bool more = it + 1 < n_tiles;
    loads_landed_barrier();
    if (more) tiles.issue(u0 + kTileN, smem + (stage ^ 1) * kStageBytes, wave);
    const unsigned char* hi_p = smem + stage * kStageBytes;
    const unsigned char* lo_p = hi_p + kTileBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // the accumulator starts at -lse2 of its row, so the MFMA returns the
      // log2 probability (-inf for an empty slot)
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = nl[i];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 bh = ld16(hi_p + t_off(kb * 32 + li, 2 * ks + hh));
        const u32x4 bl = ld16(lo_p + t_off(kb * 32 + li, 2 * ks + hh));
        acc = mfma32(qa[ks], bl, acc);
        acc = mfma32(qa[ks], bh, acc);
      }
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) p0 += __builtin_amdgcn_exp2f(acc[i]);
#pragma unroll
      for (int i = 8; i < 16; ++i) p1 += __builtin_amdgcn_exp2f(acc[i]);
      p0 += __shfl_xor(p0, 32);
      p1 += __shfl_xor(p1, 32);
      const int j = (int)u0 + kb * 32 + li;
      const float sv = (j < n_cand) ? (hh == 0 ? p0 : p1) * inv : -INFINITY;
      if (wave_any(sv > tau)) {
        // the median insertion network of gsa_topk_reg_kernel
#pragma unroll
        for (int p = kRegK - 1; p >= 1; --p) {
          const int tj = sv > lv[p] ? j : lj[p];
          lj[p] = sv > lv[p - 1] ? lj[p - 1] : tj;
          lv[p] = __builtin_amdgcn_fmed3f(lv[p - 1], sv, lv[p]);
        }
        lj[0] = sv > lv[0] ? j : lj[0];
        lv[0] = fmaxf(sv, lv[0]);
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

  // ---- each block's 32 lists (512 keys) sorted together -----------------------
  __syncthreads();  // every wave is done with the stages: they hold the lists now
  uint64_t* lists = reinterpret_cast<uint64_t*>(smem) + wave * 2 * 32 * kRegK;
  uint64_t* sel_lds = reinterpret_cast<uint64_t*>(smem + 2 * kStageBytes) + wave * kRegK;
#pragma unroll
  for (int p = 0; p < kRegK; ++p) lists[hh * 32 * kRegK + li * kRegK + p] = order_key(lv[p], lj[p]);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const long long b = b_wave + side;
    if (b >= n_qb) break;  // wave-uniform
    int32_t* ip = idx + ((long long)h * n_qb + b) * top_k;
    float* sp = score ? score + ((long long)h * n_qb + b) * top_k : nullptr;
    select_block<8>(lists + side * 32 * kRegK, 32 * kRegK, 0, top_k, lane, sel_lds, j0, ip, sp);
  }
}

}  // namespace

// Workgroups of `kernel` the device holds at once (occupancy x compute units).
int resident_workgroups(const void* kernel, int threads, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static int cus[64] = {0};
  int n_cu = 256;
  if (dev >= 0 && dev < 64) {
    if (cus[dev] == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus[dev] = prop.multiProcessorCount;
    }
    if (cus[dev] > 0) n_cu = cus[dev];
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return per_cu * n_cu;
}

static size_t round_up256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace: the key planes (every pooled key, N*nb*H*256 bytes); for wide
// selection then the per-workgroup key buffers, the bounds and the flags.
static size_t planes_bytes(const Geom& g) {
  return round_up256((size_t)g.n_frames * g.nb * g.n_heads * kPlaneRowBytes);
}

size_t gsa_topk_prob_workspace(const Geom& g) {
  return planes_bytes(g) + round_up256((size_t)g.T * g.n_heads * sizeof(float));
}

hipError_t launch_gsa_topk_prob(const Geom& g, const void* q, const float* k_cmp, int top_k, int first,
                                int32_t* idx, float* score, void* ws, hipStream_t stream) {
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const long long n_total = (long long)g.n_frames * g.nb;
  const long long n_cand = n_total - first;
  if (top_k < 1 || top_k > kRegK || top_k > n_cand) return hipErrorInvalidValue;
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* planes = w;
  float* lse2 = reinterpret_cast<float*>(w + planes_bytes(g));
  {
    const long long n = n_total * g.n_heads * 8;
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(split_keys_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k_cmp, n_total,
                       g.n_heads, kLog2e, static_cast<u32x4*>(planes));
    if (hipError_t e = hipGetLastError()) return e;
  }
  const bf16* qb = static_cast<const bf16*>(q);
  {
    const int n_rowtiles = (int)((g.T + 127) / 128);
    const long long grid = (long long)n_rowtiles * g.n_heads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gsa_token_lse_kernel, dim3((unsigned)grid), dim3(256), 2 * kStageBytes, stream, g, qb,
                       planes, n_total, n_rowtiles, lse2);
    if (hipError_t e = hipGetLastError()) return e;
  }
  const int n_wg = (int)((n_rows + kProbBlocksPerWG - 1) / kProbBlocksPerWG);
  const long long grid = (long long)n_wg * g.n_heads;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t lds = 2 * kStageBytes + 4 * kRegK * sizeof(uint64_t);
  if (top_k == kRegK) {
    hipLaunchKernelGGL(gsa_topk_prob_kernel<true>, dim3((unsigned)grid), dim3(256), lds, stream, g, qb, planes,
                       n_total, n_cand, first, top_k, lse2, n_wg, idx, score);
  } else {
    hipLaunchKernelGGL(gsa_topk_prob_kernel<false>, dim3((unsigned)grid), dim3(256), lds, stream, g, qb, planes,
                       n_total, n_cand, first, top_k, lse2, n_wg, idx, score);
  }
  return hipGetLastError();
}

// The two-stage selection serves top_k <= 16 while a lane's key positions fit
// 16 bits; its workspace: stage 1's candidate words, the key-norm partials,
// the per-head counts and lists of blocks it could not certify.
static bool two_stage(const Geom& g, int top_k) {
  return top_k <= kRegK && ((long long)g.n_frames * g.nb + kTileN - 1) / kTileN <= kApproxMaxTiles;
}
struct TwoStageLayout {
  int cap = 0;  // listed rows per head whose fallback is split over key segments
  size_t cand = 0, kpart = 0, count = 0, rows = 0, seg = 0, total = 0;
};
// cap: listed rows per head whose fallback is split (a multiple of 128; the
// rest stream every key in one workgroup)
static TwoStageLayout two_stage_layout(const Geom& g, int cap = kFallbackCap) {
  TwoStageLayout l;
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const size_t n = (size_t)n_rows * g.n_heads;
  l.cap = (int)min((long long)cap, (n_rows + 127) / 128 * 128);
  l.cand = round_up256(n * 32 * sizeof(uint32_t));
  l.kpart = round_up256((size_t)g.n_heads * kKnormChunks * sizeof(float));
  l.count = round_up256((size_t)g.n_heads * sizeof(int32_t));
  l.rows = round_up256(n * sizeof(int32_t));
  l.seg = round_up256((size_t)g.n_heads * l.cap * kFallbackSegs * 32 * sizeof(float));
  l.total = l.cand + l.kpart + l.count + l.rows + 2 * l.seg;
  return l;
}

size_t gsa_topk_workspace(const Geom& g, int top_k) { return gsa_topk_workspace(g, top_k, kFallbackCap); }

size_t gsa_topk_workspace(const Geom& g, int top_k, int cap) {
  if (two_stage(g, top_k)) return planes_bytes(g) + two_stage_layout(g, cap).total;
  if (top_k <= kRegK) return planes_bytes(g);
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const long long tiles = (n_rows + kWideRows - 1) / kWideRows * g.n_heads;
  const long long slots = tiles < kWideMaxSlots ? tiles : kWideMaxSlots;
  return planes_bytes(g) + round_up256((size_t)slots * kWideSlotKeys * sizeof(uint64_t)) +
         round_up256((size_t)(n_rows * g.n_heads) * sizeof(float)) +
         round_up256((size_t)(n_rows * g.n_heads));
}

int gsa_topk_split_cap(const Geom& g, int top_k, size_t bytes) {
  if (!two_stage(g, top_k)) return gsa_topk_workspace(g, top_k) <= bytes ? kFallbackCap : -1;
  for (int cap = kFallbackCap; cap >= 0; cap -= 128)
    if (gsa_topk_workspace(g, top_k, cap) <= bytes) return cap;
  return -1;
}

hipError_t launch_gsa_topk(const Geom& g, const float* q_blk, const float* k_cmp, int top_k,
                           int first, int32_t* idx, float* score, void* ws, hipStream_t stream) {
  return launch_gsa_topk(g, q_blk, k_cmp, top_k, first, idx, score, ws, stream, kFallbackCap);
}

hipError_t launch_gsa_topk(const Geom& g, const float* q_blk, const float* k_cmp, int top_k,
                           int first, int32_t* idx, float* score, void* ws, hipStream_t stream, int cap) {
  const long long n_rows = (long long)g.n_frames * g.nqb;
  const long long n_total = (long long)g.n_frames * g.nb;
  // the kernels see the competing keys only, indexed from 0, and add `first`
  // to the indices they write
  const long long n_cand = n_total - first;
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* planes = w;
  w += planes_bytes(g);
  {
    const long long n = n_total * g.n_heads * 8;
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(split_keys_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k_cmp, n_total,
                       g.n_heads, 1.f, static_cast<u32x4*>(planes));
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (two_stage(g, top_k)) {
    const TwoStageLayout lay = two_stage_layout(g, cap);
    uint32_t* cand = reinterpret_cast<uint32_t*>(w);
    float* kpart = reinterpret_cast<float*>(w + lay.cand);
    int32_t* fail_count = reinterpret_cast<int32_t*>(w + lay.cand + lay.kpart);
    int32_t* fail_rows = reinterpret_cast<int32_t*>(w + lay.cand + lay.kpart + lay.count);
    const int n_rowtiles = (int)((n_rows + 127) / 128);
    const long long grid = (long long)n_rowtiles * g.n_heads;
    const long long pairs_threads = n_rows * g.n_heads * 32;
    if (grid > 0x7fffffffLL || (pairs_threads + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kmax_partial_kernel, dim3(g.n_heads * kKnormChunks), dim3(256), 0, stream, k_cmp,
                       n_total, g.n_heads, kpart, fail_count);
    if (hipError_t e = hipGetLastError()) return e;
    hipLaunchKernelGGL(gsa_topk_approx_kernel, dim3((unsigned)grid), dim3(256), 2 * kTileBytes, stream, g, q_blk,
                       planes, n_total, n_cand, first, n_rowtiles, cand);
    if (hipError_t e = hipGetLastError()) return e;
    hipLaunchKernelGGL(gsa_topk_rescore_kernel, dim3((unsigned)((pairs_threads + 255) / 256)), dim3(256), 0,
                       stream, g, q_blk, k_cmp, first, top_k, cand, kpart, idx, score, fail_count, fail_rows);
    if (hipError_t e = hipGetLastError()) return e;
    // the blocks the certificate missed, selected again exactly: the first
    // lay.cap per head with their keys split over kFallbackSegs workgroups
    // (a few hundred blocks would otherwise each stream every key in one
    // workgroup), then merged
    const RegList fl{fail_rows, fail_count, kFallbackSegs, lay.cap,
                     reinterpret_cast<float*>(w + lay.cand + lay.kpart + lay.count + lay.rows),
                     reinterpret_cast<int32_t*>(w + lay.cand + lay.kpart + lay.count + lay.rows + lay.seg)};
    const long long fgrid = grid * kFallbackSegs;
    if (fgrid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (top_k == kRegK) {
      hipLaunchKernelGGL(gsa_topk_reg_kernel<true>, dim3((unsigned)fgrid), dim3(256), 2 * kStageBytes,
                         stream, g, q_blk, planes, n_total, n_cand, first, top_k, n_rowtiles, idx, score, fl);
    } else {
      hipLaunchKernelGGL(gsa_topk_reg_kernel<false>, dim3((unsigned)fgrid), dim3(256), 2 * kStageBytes,
                         stream, g, q_blk, planes, n_total, n_cand, first, top_k, n_rowtiles, idx, score, fl);
    }
    if (hipError_t e = hipGetLastError()) return e;
    // (no split capacity -- the allocation-free entry point on its largest
    // problems -- leaves nothing to merge)
    const long long mwaves = (long long)g.n_heads * lay.cap;
    if (mwaves == 0) return hipSuccess;
    hipLaunchKernelGGL(gsa_topk_seg_merge_kernel, dim3((unsigned)((mwaves + 3) / 4)), dim3(256), 0, stream, g,
                       top_k, lay.cap, fail_rows, fail_count, fl.seg_val, fl.seg_idx, idx, score);
    return hipGetLastError();
  }
  if (top_k <= kRegK) {
    const int n_rowtiles = (int)((n_rows + 127) / 128);
    const long long grid = (long long)n_rowtiles * g.n_heads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (top_k == kRegK) {
      hipLaunchKernelGGL(gsa_topk_reg_kernel<true>, dim3((unsigned)grid), dim3(256), 2 * kStageBytes,
                         stream, g, q_blk, planes, n_total, n_cand, first, top_k, n_rowtiles, idx, score,
                         RegList{});
    } else {
      hipLaunchKernelGGL(gsa_topk_reg_kernel<false>, dim3((unsigned)grid), dim3(256), 2 * kStageBytes,
                         stream, g, q_blk, planes, n_total, n_cand, first, top_k, n_rowtiles, idx, score,
                         RegList{});
    }
    return hipGetLastError();
  }
  // wide: the bound, then filter and sort in a persistent kernel, then the
  // LDS-list kernel for the blocks it flagged
  const int n_rowtiles = (int)((n_rows + kWideRows - 1) / kWideRows);
  const long long tiles = (long long)n_rowtiles * g.n_heads;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long slots = tiles < kWideMaxSlots ? tiles : kWideMaxSlots;
  uint64_t* buf = reinterpret_cast<uint64_t*>(w);
  w += round_up256((size_t)slots * kWideSlotKeys * sizeof(uint64_t));
  float* bound = reinterpret_cast<float*>(w);
  w += round_up256((size_t)(n_rows * g.n_heads) * sizeof(float));
  uint8_t* flags = reinterpret_cast<uint8_t*>(w);
  if (top_k <= 64) {
    hipLaunchKernelGGL(gsa_topk_bound_kernel<2>, dim3((unsigned)tiles), dim3(256), 2 * kStageBytes, stream,
                       g, q_blk, planes, n_total, (long long)first, n_cand, top_k, n_rowtiles, bound);
  } else {
    hipLaunchKernelGGL(gsa_topk_bound_kernel<4>, dim3((unsigned)tiles), dim3(256), 2 * kStageBytes, stream,
                       g, q_blk, planes, n_total, (long long)first, n_cand, top_k, n_rowtiles, bound);
  }
  if (hipError_t e = hipGetLastError()) return e;
  const size_t lds_wide = 2 * kStageBytes + 4 * 128 * sizeof(uint64_t);
  long long grid = resident_workgroups(reinterpret_cast<const void*>(gsa_topk_wide_kernel), 256, lds_wide);
  if (grid > slots) grid = slots;
  hipLaunchKernelGGL(gsa_topk_wide_kernel, dim3((unsigned)grid), dim3(256), lds_wide, stream, g, q_blk, planes,
                     n_total, n_cand, first, top_k, n_rowtiles, tiles, bound, buf, flags, idx, score);
  if (hipError_t e = hipGetLastError()) return e;
  const float* kc = k_cmp + (long long)first * g.n_heads * kHeadDim;
  int waves = 4;
  auto lds_for = [&](int w) { return (size_t)2 * kStageBytes + (size_t)w * 32 * (top_k + 1) * 8; };
  if (lds_for(waves) > 160 * 1024) waves = 2;
  const int n_lds_tiles = (int)((n_rows + 32 * waves - 1) / (32 * waves));
  const long long lds_grid = (long long)n_lds_tiles * g.n_heads;
  if (lds_grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gsa_topk_kernel, dim3((unsigned)lds_grid), dim3(64 * waves), lds_for(waves), stream,
                     g, q_blk, kc, n_cand, first, top_k, n_lds_tiles, flags, idx, score);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free selection entry point: one file-scope device
// array per GPU the library runs on, held until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a stand-in
// for the symbol): its device address is looked up once per device, with that
// device current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace sga
