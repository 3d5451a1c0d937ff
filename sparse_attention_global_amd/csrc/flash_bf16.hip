// Tiled softmax attention for gfx950, bf16 in / fp32 accumulate, head_dim 64.
//
// One kernel serves every attention form of the layer whose keys are the same
// for a whole tile of queries:
//   GLOBAL      dense global attention (all T tokens) and the GSA compressed
//               branch (all pooled keys): keys [0, n_keys) of K/V;
//   FRAME       frame attention: the keys of the query's own frame;
//   SUBSAMPLED  AVGGT subsampled attention: the own frame whole, then the
//               compacted set of all frames with the own frame's rows masked.
//
// Work split: a workgroup of 4 waves owns 128 consecutive query rows of one
// head (never straddling a frame in FRAME/SUBSAMPLED mode); each wave owns 32.
// The per-tile math (attn_tile.hpp) keeps every per-query quantity inside the
// lane that owns the query.
//
// Data movement: keys stream in tiles of 64 through a ring of LDS stages.
// Every K row and every V^T row of a tile moves from HBM/L2 straight into LDS
// with 16-byte direct loads (global_load_lds_dwordx4) issued one or two tiles
// ahead -- no registers, no VALU address work per tile, no LDS write
// instructions. The swizzled LDS layouts are produced by choosing which
// 16-byte chunk each lane fetches. V^T comes from a staging pass (vt_prepare)
// that already holds V transposed in the MFMA operand's key order. A tile is
// consumed after an explicit vmcnt wait and a bare s_barrier (a full
// __syncthreads fence would drain the prefetches).
//
// Launch order: GLOBAL walks heads outermost, so the workgroups that the
// hardware spreads round-robin over the 8 XCDs at any moment share one head's
// K/V stream in every XCD's L2. FRAME/SUBSAMPLED give each XCD a contiguous
// range of (head, frame, tile) so the tiles of one frame meet in one L2.
#include <type_traits>

#include "attn_tile.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;         // 128 queries per workgroup
constexpr int kRowsPerWave = 64 / kWaves;    // K rows and V^T rows each wave fetches per tile
constexpr int kLoadsPerTile = 2 * kRowsPerWave / 8;  // 16-byte direct loads per lane per tile
constexpr int kStageBytes = kTileKBytes + kTileVBytes;
// Occupancy: the kernel is issue- and latency-bound, so it runs with more
// resident waves and a shorter LDS ring rather than fewer waves with a deep
// prefetch (measured on MI355X at 128 frames: 4 stages / 2 waves per SIMD
// 35.3%, 3 / 3 38.1%, 2 / 4 39.0% of bf16 peak for dense attention; the
// subsampled form, with more scalar bookkeeping, does best at 3 / 3).
template <int MODE>
struct Ring {
  static constexpr int stages = (MODE == 2) ? 3 : 2;
  static constexpr int wg_per_cu = (MODE == 2) ? 3 : 4;
};

enum { MODE_GLOBAL = 0, MODE_FRAME = 1, MODE_SUBSAMPLED = 2 };

struct FlashArgs {
  const bf16* q;
  bf16* o;
  float* lse;
  Geom g;
  const bf16* k;     // keys [rows, H, d]
  const bf16* vt;    // V^T staging of the values (vt_prepare)
  long long vt_ld;   // V^T row length (columns)
  long long n_keys;  // GLOBAL: keys
  int vt_pitch;      // FRAME/SUBSAMPLED: V^T columns per frame (L rounded up to 64)
  const bf16* ck;    // SUBSAMPLED: compacted keys, kept part [N*mk] then means [N]
  const bf16* cvt;   // SUBSAMPLED: V^T staging of the compacted values
  long long cvt_ld;
  int mk;            // SUBSAMPLED: kept rows per frame
  int has_mean;      // SUBSAMPLED: one mean row per frame follows the kept part
  float mean_bias2;  // SUBSAMPLED: log2(#dropped) added to mean rows' logits, or 0
  float scale_log2;  // log2(e) / sqrt(d)
  int n_qtiles;      // GLOBAL: tiles over T; else tiles per frame
  int n_logical;     // logical workgroups
  int remap;         // 1: give each XCD a contiguous range of logical workgroups
};

// A contiguous run of keys: K rows k_row0.. of `k`, V^T columns vt_col0.. of `vt`.
struct Segment {
  const bf16* k;
  long long k_row0;
  const bf16* vt;
  long long vt_col0;
  long long vt_ld;
  long long n;
};

__device__ __forceinline__ void lds_dma16(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// Wait until at most N direct loads of this lane are in flight, then meet the
// other waves: every wave's loads of the tile about to be read have landed and
// every wave is done reading the stage about to be refilled.
template <int N>
__device__ __forceinline__ void wait_and_meet() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt <= N; lgkmcnt, expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int MODE>
__global__ __launch_bounds__(kThreads, Ring<MODE>::wg_per_cu) void flash_bf16_kernel(FlashArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int kStages = Ring<MODE>::stages;  // LDS ring
  constexpr int kAhead = kStages - 1;          // tiles in flight ahead of the one consumed

  int lid = blockIdx.x;
  if (A.remap) {
    const int per = (A.n_logical + 7) >> 3;
    lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  if (lid >= A.n_logical) return;
  int h, f = 0;
  long long q0, q_end;
  if (MODE == MODE_GLOBAL) {
    h = lid / A.n_qtiles;
    q0 = (long long)(lid % A.n_qtiles) * kBlockM;
    q_end = min(q0 + kBlockM, A.g.T);
  } else {
    const int per_head = A.g.n_frames * A.n_qtiles;
    h = lid / per_head;
    const int rem = lid % per_head;
    f = rem / A.n_qtiles;
    q0 = (long long)f * A.g.L + (long long)(rem % A.n_qtiles) * kBlockM;
    q_end = min(q0 + kBlockM, (long long)(f + 1) * A.g.L);
  }

  // ---- key segments ----------------------------------------------------------
  Segment seg0, seg1;
  if (MODE == MODE_GLOBAL) {
    seg0 = Segment{A.k, 0, A.vt, 0, A.vt_ld, A.n_keys};
  } else {
    seg0 = Segment{A.k, (long long)f * A.g.L, A.vt, (long long)f * A.vt_pitch, A.vt_ld, A.g.L};
  }
  seg1 = Segment{A.ck, 0, A.cvt, 0, A.cvt_ld,
                 MODE == MODE_SUBSAMPLED ? (long long)A.g.n_frames * (A.mk + A.has_mean) : 0};
  const long long nt0 = (seg0.n + kTileKeys - 1) / kTileKeys;
  const long long n_tiles = nt0 + (seg1.n + kTileKeys - 1) / kTileKeys;
  // compacted rows of the own frame (masked), the mean rows (log-count bias)
  const long long own0 = (long long)f * A.mk, own1 = own0 + A.mk;
  const long long mean0 = (long long)A.g.n_frames * A.mk;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long rs = (long long)A.g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;
  const float c = A.scale_log2;

  // ---- direct tile loads -------------------------------------------------------
  // lane -> row r = wave * kRowsPerWave + 8 i + lane / 8 of the tile (a key row of
  // K, a d row of V^T) and physical 16-byte chunk lane % 8. Every address is a
  // per-tile scalar base plus a per-lane 32-bit offset fixed for the kernel, and
  // the LDS destination is wave-uniform, so issuing a tile costs no VALU work.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int ld_r = lane >> 3, ld_p = lane & 7;
  uint32_t k_off[kRowsPerWave / 8], v_off0[kRowsPerWave / 8], v_off1[kRowsPerWave / 8];
#pragma unroll
  for (int i = 0; i < kRowsPerWave / 8; ++i) {
    const int r = wave_u * kRowsPerWave + 8 * i + ld_r;
    const int kc = ld_p ^ ld_r;                               // K swizzle: chunk ^ (r & 7)
    const int vc = ld_p ^ ld_r ^ ((2 * wave_u + i) & 7);      // V^T swizzle: chunk ^ swz(r)
    k_off[i] = (uint32_t)((r * rs + kc * 8) * 2);
    v_off0[i] = (uint32_t)((r * seg0.vt_ld + vc * 8) * 2);
    v_off1[i] = (uint32_t)((r * seg1.vt_ld + vc * 8) * 2);
  }
  auto issue_tile = [&](long long j, unsigned char* stage) {
    const bool second = j >= nt0;
    const Segment& sg = second ? seg1 : seg0;
    const long long u0 = (second ? j - nt0 : j) * kTileKeys;
    const char* kb = reinterpret_cast<const char*>(sg.k + (sg.k_row0 + u0) * rs + hoff);
    const char* vb = reinterpret_cast<const char*>(sg.vt + hoff * sg.vt_ld + sg.vt_col0 + u0);
    unsigned char* kdst = stage + wave_u * kRowsPerWave * 128;
    unsigned char* vdst = kdst + kTileKBytes;
    if (u0 + kTileKeys <= sg.n) {
#pragma unroll
      for (int i = 0; i < kRowsPerWave / 8; ++i) {
        lds_dma16(kb + k_off[i], kdst + 8 * i * 128);
        lds_dma16(vb + (second ? v_off1[i] : v_off0[i]), vdst + 8 * i * 128);
      }
    } else {  // last tile of a segment: rows past its end re-read its last row (masked)
#pragma unroll
      for (int i = 0; i < kRowsPerWave / 8; ++i) {
        const long long r = wave_u * kRowsPerWave + 8 * i + ld_r;
        const long long clamp = (u0 + r < sg.n) ? 0 : (sg.n - 1 - u0 - r) * rs * 2;
        lds_dma16(kb + k_off[i] + clamp, kdst + 8 * i * 128);
        lds_dma16(vb + (second ? v_off1[i] : v_off0[i]), vdst + 8 * i * 128);
      }
    }
  };

  // logit mask/bias of tile j (boundary tiles only), applied in registers
  auto needs_mask = [&](long long j) -> bool {
    if (j < nt0) return (j + 1) * kTileKeys > seg0.n;
    if (MODE != MODE_SUBSAMPLED) return false;
    const long long a = (j - nt0) * kTileKeys, b = a + kTileKeys;
    return b > seg1.n || (a < own1 && b > own0) || (A.has_mean && b > mean0);
  };
  auto apply_mask = [&](long long j, f32x16 s[2]) {
    const bool second = j >= nt0;
    const long long u0 = (second ? j - nt0 : j) * kTileKeys;
    const long long n = second ? seg1.n : seg0.n;
    const float bias = A.mean_bias2 / c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const long long u = u0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        bool ok = u < n;
        float add = 0.f;
        if (MODE == MODE_SUBSAMPLED && second) {
          ok = ok && !(u >= own0 && u < own1) && !(A.has_mean && u == mean0 + f);
          if (A.has_mean && u >= mean0) add = bias;
        }
        s[kb][i] = ok ? s[kb][i] + add : -INFINITY;
      }
  };

  const long long qrow = q0 + wave * 32 + li;
  const bool qvalid = qrow < q_end;
  u32x4 qB[4];
  load_q_operand(A.q + (qvalid ? qrow : q0) * rs + hoff, qvalid, qB);

  WaveAttnState st;
  st.init();
  TileLaneOffsets off;
  off.init();

#pragma unroll
  for (int j = 0; j < kAhead; ++j)
    if (j < n_tiles) issue_tile(j, smem + j * kStageBytes);
  static_assert(kStages >= 2 && kStages <= 4, "ring of 2 to 4 stages");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  auto body = [&](long long j, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int refill = (cur + kAhead) % kStages;
    const long long left = n_tiles - 1 - j;  // tiles after j already in flight: min(kAhead-1, left)
    if (left >= kAhead - 1) {
      wait_and_meet<(kAhead - 1) * kLoadsPerTile>();
    } else if (kAhead > 2 && left == 1) {
      wait_and_meet<kLoadsPerTile>();
    } else {
      wait_and_meet<0>();
    }
    if (j + kAhead < n_tiles) issue_tile(j + kAhead, smem + refill * kStageBytes);
    const unsigned char* stage = smem + cur * kStageBytes;
    f32x16 s[2];
    st.scores(stage, off, qB, s);
    if (needs_mask(j)) apply_mask(j, s);
    st.consume(s, stage, off, c, false, true);
  };
  for (long long j = 0; j < n_tiles; j += kStages) {
    body(j, I0{});
    if (j + 1 < n_tiles) body(j + 1, I1{});
    if constexpr (kStages > 2) {
      if (j + 2 < n_tiles) body(j + 2, std::integral_constant<int, 2>{});
    }
    if constexpr (kStages > 3) {
      if (j + 3 < n_tiles) body(j + 3, std::integral_constant<int, 3>{});
    }
  }
  st.finish(A.o + qrow * rs + hoff, A.lse ? A.lse + qrow * A.g.n_heads + h : nullptr, qvalid, c);
}

}  // namespace

size_t flash_bf16_workspace(const FlashLaunch& p) {
  if (p.mode == FLASH_GLOBAL) {
    const long long ld = (p.n_keys + 63) / 64 * 64;
    return (size_t)p.g.n_heads * kHeadDim * ld * 2;
  }
  const long long pitch = (p.g.L + 63) / 64 * 64;
  size_t bytes = (size_t)p.g.n_heads * kHeadDim * pitch * p.g.n_frames * 2;
  if (p.mode == FLASH_SUBSAMPLED) {
    const long long rows = (long long)p.g.n_frames * (p.mk + p.has_mean);
    bytes += (size_t)p.g.n_heads * kHeadDim * ((rows + 63) / 64 * 64) * 2;
  }
  return bytes;
}

hipError_t launch_flash_bf16(const FlashLaunch& p, void* ws, hipStream_t stream) {
  FlashArgs A{};
  A.q = static_cast<const bf16*>(p.q);
  A.o = static_cast<bf16*>(p.o);
  A.lse = p.lse;
  A.g = p.g;
  A.k = static_cast<const bf16*>(p.k);
  A.n_keys = p.n_keys;
  A.ck = static_cast<const bf16*>(p.ck);
  A.mk = p.mk;
  A.has_mean = p.has_mean;
  A.mean_bias2 = p.mean_bias2;
  A.scale_log2 = kLog2e / sqrtf((float)kHeadDim);
  bf16* vt = static_cast<bf16*>(ws);
  hipError_t e;
  long long n_logical;
  if (p.mode == FLASH_GLOBAL) {
    A.vt_ld = (p.n_keys + 63) / 64 * 64;
    e = launch_vt_prepare(p.v, p.g.n_heads, p.n_keys, p.n_keys, A.vt_ld, A.vt_ld, vt, stream);
    if (e != hipSuccess) return e;
    A.n_qtiles = (int)((p.g.T + kBlockM - 1) / kBlockM);
    n_logical = (long long)A.n_qtiles * p.g.n_heads;
    A.remap = 0;
  } else {
    A.vt_pitch = (p.g.L + 63) / 64 * 64;
    A.vt_ld = (long long)A.vt_pitch * p.g.n_frames;
    e = launch_vt_prepare(p.v, p.g.n_heads, p.g.T, p.g.L, A.vt_pitch, A.vt_ld, vt, stream);
    if (e != hipSuccess) return e;
    if (p.mode == FLASH_SUBSAMPLED) {
      const long long rows = (long long)p.g.n_frames * (p.mk + p.has_mean);
      A.cvt_ld = (rows + 63) / 64 * 64;
      bf16* cvt = vt + (size_t)p.g.n_heads * kHeadDim * A.vt_ld;
      e = launch_vt_prepare(p.cv, p.g.n_heads, rows, rows, A.cvt_ld, A.cvt_ld, cvt, stream);
      if (e != hipSuccess) return e;
      A.cvt = cvt;
    }
    A.n_qtiles = (p.g.L + kBlockM - 1) / kBlockM;
    n_logical = (long long)A.n_qtiles * p.g.n_frames * p.g.n_heads;
    A.remap = 1;
  }
  A.vt = vt;
  if (n_logical > 0x7ffffff0LL) return hipErrorInvalidValue;
  A.n_logical = (int)n_logical;
  const int grid = A.remap ? ((A.n_logical + 7) / 8) * 8 : A.n_logical;
  switch (p.mode) {
    case FLASH_GLOBAL:
      hipLaunchKernelGGL(flash_bf16_kernel<MODE_GLOBAL>, dim3(grid), dim3(kThreads),
                         Ring<MODE_GLOBAL>::stages * kStageBytes, stream, A);
      break;
    case FLASH_FRAME:
      hipLaunchKernelGGL(flash_bf16_kernel<MODE_FRAME>, dim3(grid), dim3(kThreads),
                         Ring<MODE_FRAME>::stages * kStageBytes, stream, A);
      break;
    default:
      hipLaunchKernelGGL(flash_bf16_kernel<MODE_SUBSAMPLED>, dim3(grid), dim3(kThreads),
                         Ring<MODE_SUBSAMPLED>::stages * kStageBytes, stream, A);
      break;
  }
  return hipGetLastError();
}

}  // namespace sga
