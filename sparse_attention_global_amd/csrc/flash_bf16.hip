// Tiled softmax attention for gfx950, bf16 in / fp32 accumulate, head_dim 64.
//
// One kernel serves every attention form of the layer whose keys are the same
// for a whole tile of queries:
//   GLOBAL      dense global attention (all T tokens) and the GSA compressed
//               branch (all pooled keys): keys [0, n_keys) of K/V;
//   FRAME       frame attention: the keys of the query's own frame;
//   SUBSAMPLED  AVGGT subsampled attention: the own frame whole, then the kept
//               rows of every other frame, then their mean rows.
//
// Work split: a workgroup of 4 waves owns 128 consecutive query rows of one
// head (never straddling a frame in FRAME/SUBSAMPLED mode); each wave owns 32.
// Keys stream through LDS in tiles of 64, double buffered, one barrier per
// tile: the next tile's global loads are issued before the current tile's
// MFMA/softmax work and written to the other LDS stage after it. The per-tile
// math (attn_tile.hpp) keeps every per-query quantity in the owning lane.
//
// Launch order: GLOBAL walks heads outermost, so the workgroups that the
// hardware spreads round-robin over the 8 XCDs at any moment share one head's
// K/V stream in every XCD's L2. FRAME/SUBSAMPLED give each XCD a contiguous
// range of (head, frame, tile) so the tiles of one frame meet in one L2.
#include "attn_tile.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;  // 128 queries per workgroup

enum { MODE_GLOBAL = 0, MODE_FRAME = 1, MODE_SUBSAMPLED = 2 };

struct FlashArgs {
  const bf16* q;
  const bf16* k;   // GLOBAL: [n_keys,H,d]; FRAME/SUBSAMPLED: [T,H,d]
  const bf16* v;
  const bf16* ck;  // SUBSAMPLED: compacted keys, kept part [N*mk,H,d] then means [N,H,d]
  const bf16* cv;
  bf16* o;
  float* lse;
  Geom g;
  long long n_keys;  // GLOBAL only
  int mk;            // SUBSAMPLED: kept rows per frame (specials + grid-kept)
  int has_mean;      // SUBSAMPLED: frames carry a mean row
  float mean_bias2;  // SUBSAMPLED: log2(#dropped) added to mean rows' logits, or 0
  float scale_log2;  // log2(e) / sqrt(d)
  int n_qtiles;      // GLOBAL: tiles over T; else tiles per frame
  int n_logical;     // logical workgroups
  int remap;         // 1: give each XCD a contiguous range of logical workgroups
};

struct KeyRow {
  const bf16* k;
  const bf16* v;
  float bias;  // log2 units
};

// Row pointers (head offset applied) and logit bias of key u of this tile's key set.
template <int MODE>
__device__ __forceinline__ KeyRow key_row(const FlashArgs& A, long long hoff, int f, long long nk,
                                          long long u) {
  const long long rs = (long long)A.g.n_heads * kHeadDim;
  KeyRow kr{A.k, A.v, 0.f};
  long long row = 0;
  if (u >= nk) {
    kr.bias = -INFINITY;
  } else if (MODE == MODE_GLOBAL) {
    row = u;
  } else if (MODE == MODE_FRAME) {
    row = (long long)f * A.g.L + u;
  } else {
    const int L = A.g.L;
    const long long kept_n = (long long)(A.g.n_frames - 1) * A.mk;
    if (u < L) {
      row = (long long)f * L + u;
    } else if (u < L + kept_n) {
      const long long w = u - L;  // skip frame f's own kept rows
      row = w + (w >= (long long)f * A.mk ? A.mk : 0);
      kr.k = A.ck;
      kr.v = A.cv;
    } else {
      const long long w = u - L - kept_n;  // skip frame f's own mean row
      row = (long long)A.g.n_frames * A.mk + w + (w >= f ? 1 : 0);
      kr.k = A.ck;
      kr.v = A.cv;
      kr.bias = A.mean_bias2;
    }
  }
  kr.k += row * rs + hoff;
  kr.v += row * rs + hoff;
  return kr;
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void flash_bf16_kernel(FlashArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  int lid = blockIdx.x;
  if (A.remap) {
    const int per = (A.n_logical + 7) >> 3;
    lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  if (lid >= A.n_logical) return;
  int h, f = 0;
  long long q0, q_end, nk;
  if (MODE == MODE_GLOBAL) {
    h = lid / A.n_qtiles;
    q0 = (long long)(lid % A.n_qtiles) * kBlockM;
    q_end = min(q0 + kBlockM, A.g.T);
    nk = A.n_keys;
  } else {
    const int per_head = A.g.n_frames * A.n_qtiles;
    h = lid / per_head;
    const int rem = lid % per_head;
    f = rem / A.n_qtiles;
    q0 = (long long)f * A.g.L + (long long)(rem % A.n_qtiles) * kBlockM;
    q_end = min(q0 + kBlockM, (long long)(f + 1) * A.g.L);
    nk = (MODE == MODE_FRAME) ? A.g.L
                              : A.g.L + (long long)(A.g.n_frames - 1) * (A.mk + A.has_mean);
  }
  // keys from this index on carry a logit bias: the masked tail, and in
  // SUBSAMPLED mode with a log-count the mean rows
  long long bias_from = nk;
  if (MODE == MODE_SUBSAMPLED && A.mean_bias2 != 0.f)
    bias_from = A.g.L + (long long)(A.g.n_frames - 1) * A.mk;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31;
  const long long rs = (long long)A.g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;
  const float c = A.scale_log2;

  const long long qrow = q0 + wave * 32 + li;
  const bool qvalid = qrow < q_end;
  u32x4 qB[4];
  load_q_operand(A.q + (qvalid ? qrow : q0) * rs + hoff, qvalid, qB);

  WaveAttnState st;
  st.init();
  TileLaneOffsets off;
  off.init();

  // loader: keys (tid >> 3) and (tid >> 3) + 32 of a tile, 16-byte chunk tid & 7
  const int ld_key = tid >> 3, ld_chunk = tid & 7;
  u32x4 kreg[2], vreg[2];
  float breg[2];
  // GLOBAL and FRAME keys are contiguous rows: walk a pointer; SUBSAMPLED maps
  // every key through its segment
  const long long key_base = (MODE == MODE_FRAME) ? (long long)f * A.g.L : 0;
  auto load_tile = [&](long long u0) {
    const bool full = u0 + kTileKeys <= nk;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const long long u = u0 + ld_key + 32 * i;
      if (MODE != MODE_SUBSAMPLED && full) {
        const long long o = (key_base + u) * rs + hoff + ld_chunk * 8;
        kreg[i] = ld16(A.k + o);
        vreg[i] = ld16(A.v + o);
        breg[i] = 0.f;
      } else {
        const KeyRow kr = key_row<MODE>(A, hoff, f, nk, u);
        const bool ok = u < nk;
        kreg[i] = ok ? ld16(kr.k + ld_chunk * 8) : u32x4{0, 0, 0, 0};
        vreg[i] = ok ? ld16(kr.v + ld_chunk * 8) : u32x4{0, 0, 0, 0};
        breg[i] = kr.bias;
      }
    }
  };
  auto store_tile = [&](unsigned char* sp) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      tile_store_kv(sp, ld_key + 32 * i, ld_chunk, kreg[i], vreg[i]);
      if (ld_chunk == 0) tile_bias(sp)[ld_key + 32 * i] = breg[i];
    }
  };

  unsigned char* const stage0 = smem;
  unsigned char* const stage1 = smem + kTileStageBytes;
  const long long n_tiles = (nk + kTileKeys - 1) / kTileKeys;
  load_tile(0);
  store_tile(stage0);
  __syncthreads();
  // two tiles per iteration so each stage's LDS offsets are immediates
  for (long long it = 0; it < n_tiles; it += 2) {
    {
      const long long u0 = it * kTileKeys;
      const bool more = it + 1 < n_tiles;
      if (more) load_tile(u0 + kTileKeys);
      st.step(stage0, off, qB, c, u0 + kTileKeys > bias_from, true);
      if (more) store_tile(stage1);
      __syncthreads();
    }
    if (it + 1 < n_tiles) {
      const long long u0 = (it + 1) * kTileKeys;
      const bool more = it + 2 < n_tiles;
      if (more) load_tile(u0 + kTileKeys);
      st.step(stage1, off, qB, c, u0 + kTileKeys > bias_from, true);
      if (more) store_tile(stage0);
      __syncthreads();
    }
  }
  st.finish(A.o + qrow * rs + hoff, A.lse ? A.lse + qrow * A.g.n_heads + h : nullptr, qvalid, c);
}

}  // namespace

hipError_t launch_flash_bf16(const FlashLaunch& p, hipStream_t stream) {
  FlashArgs A{};
  A.q = static_cast<const bf16*>(p.q);
  A.k = static_cast<const bf16*>(p.k);
  A.v = static_cast<const bf16*>(p.v);
  A.ck = static_cast<const bf16*>(p.ck);
  A.cv = static_cast<const bf16*>(p.cv);
  A.o = static_cast<bf16*>(p.o);
  A.lse = p.lse;
  A.g = p.g;
  A.n_keys = p.n_keys;
  A.mk = p.mk;
  A.has_mean = p.has_mean;
  A.mean_bias2 = p.mean_bias2;
  A.scale_log2 = kLog2e / sqrtf((float)kHeadDim);
  long long n_logical;
  if (p.mode == FLASH_GLOBAL) {
    A.n_qtiles = (int)((p.g.T + kBlockM - 1) / kBlockM);
    n_logical = (long long)A.n_qtiles * p.g.n_heads;
    A.remap = 0;
  } else {
    A.n_qtiles = (p.g.L + kBlockM - 1) / kBlockM;
    n_logical = (long long)A.n_qtiles * p.g.n_frames * p.g.n_heads;
    A.remap = 1;
  }
  if (n_logical > 0x7ffffff0LL) return hipErrorInvalidValue;
  A.n_logical = (int)n_logical;
  const int grid = A.remap ? ((A.n_logical + 7) / 8) * 8 : A.n_logical;
  const size_t lds = 2 * kTileStageBytes;
  switch (p.mode) {
    case FLASH_GLOBAL:
      hipLaunchKernelGGL(flash_bf16_kernel<MODE_GLOBAL>, dim3(grid), dim3(kThreads), lds, stream, A);
      break;
    case FLASH_FRAME:
      hipLaunchKernelGGL(flash_bf16_kernel<MODE_FRAME>, dim3(grid), dim3(kThreads), lds, stream, A);
      break;
    default:
      hipLaunchKernelGGL(flash_bf16_kernel<MODE_SUBSAMPLED>, dim3(grid), dim3(kThreads), lds, stream, A);
      break;
  }
  return hipGetLastError();
}

}  // namespace sga
