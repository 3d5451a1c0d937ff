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
// Work split: a workgroup of 4 waves owns consecutive query rows of one head
// (never straddling a frame in FRAME/SUBSAMPLED mode): 256 in GLOBAL mode and
// for a frame's whole 256-row tiles in SUBSAMPLED mode (each wave 64, as two
// 32-query halves sharing every K/V^T operand read), 128 in FRAME mode and for
// the rest of a SUBSAMPLED frame (each wave 32). The per-tile math
// (attn_tile.hpp) keeps every per-query quantity inside the lane that owns the
// query.
//
// Softmax: the scale log2(e)/sqrt(d) is folded into Q (rounded once to bf16),
// and every query starts its accumulator at minus an upper bound of its logits,
// |q'| max|k| (a small key-norm pass supplies max|k| per head), so the MFMA
// returns logit - bound and a probability costs a single v_exp: no per-score
// scaling, subtraction or running maximum, and no rescaling (attn_tile.hpp,
// FlashWaveState). A workgroup whose rows' probabilities underflowed because
// the bound was far above their true maximum flags itself, and a second launch
// of the kernel redoes exactly those workgroups with the online softmax.
//
// Data movement: keys stream in tiles of 64 through a ring of LDS stages.
// Every K row and every V^T row of a tile moves from HBM/L2 straight into LDS
// with 16-byte direct buffer loads (buffer_load_dwordx4 ... lds) issued two
// tiles ahead (in the two-half configuration two tiles at a time, one barrier
// per two tiles) -- no registers, no VALU address work per tile, no LDS write
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

enum { MODE_GLOBAL = 0, MODE_FRAME = 1, MODE_SUBSAMPLED = 2 };

// Tiling per mode: waves per workgroup (32 queries each), workgroups per CU,
// LDS ring stages (16 KiB each), and how many waves issue the tile loads
// (64 K rows + 64 V^T rows of 128 B per tile, spread evenly over them).
// Measured for dense attention at 128 frames (% of bf16 peak): 4 waves x 3
// workgroups x 3 stages 46.6; 12 x 1 x 3 (8 loading) 45.6; 8 x 1 x 5 43.2;
// 6 x 2 x 3 38.8 (the register budget then allows only 2 waves per SIMD).
template <int W, int G, int S, int D, int Q, int P = 1>
struct TileCfg {
  static constexpr int waves = W;
  static constexpr int wg_per_cu = G;
  static constexpr int stages = S;
  static constexpr int dma_waves = D;
  static constexpr int halves = Q;  // 32-query halves per wave
  static constexpr int group = P;   // > 1: 2P stages refilled P at a time, one barrier per P tiles
  static constexpr int threads = W * 64;
  static constexpr int block_m = W * 32 * Q;
  static constexpr int rows_per_wave = 64 / D;           // K rows and V^T rows per loading wave
  static constexpr int loads_per_tile = 2 * rows_per_wave / 8;  // 16-byte loads per lane
  static_assert(D <= W && 64 % D == 0 && rows_per_wave % 8 == 0, "load split");
  static_assert(S >= 2 && S <= 9, "ring");
  static_assert(P == 1 || S == 2 * P, "groups of P tiles use a 2P-stage ring");
};
// GLOBAL: two 32-query halves per wave sharing every LDS operand read (64
// queries a wave, 256 a workgroup, 2 workgroups = 2 waves per SIMD): measured
// on a register/LDS-only probe of the tile arithmetic, 63% of the bf16 peak
// against 51% for one half per wave at 3 waves per SIMD. FRAME/SUBSAMPLED keep
// one half per wave (a frame's 1374 queries fill 128-query tiles better).
// GLOBAL stages its tiles in groups of 2 (4 stages, a barrier per 2 tiles).
// 8 waves x 512 queries x 1 workgroup per CU (groups of 2, 3 or 4 tiles) moves
// half the bytes from L2 into LDS and runs at a 6-8% higher clock, but the two
// waves of a SIMD then wait on each other at the barriers: no faster.
// SUBSAMPLED runs a frame's queries in two launches (PART 0 and 1): the whole
// 256-query tiles with two halves per wave, the rest of the frame (1374 = 5 x
// 256 + 94) with one half per wave, so that no frame pays for a mostly empty
// 256-query tile.
template <int MODE, int PART = 0>
struct Cfg : TileCfg<4, 3, 3, 4, 1> {};
template <>
struct Cfg<0, 0> : TileCfg<4, 2, 4, 4, 2, 2> {};
template <>
struct Cfg<2, 0> : TileCfg<4, 2, 4, 4, 2, 2> {};
// the rest of a SUBSAMPLED frame when it fits 96 rows: 3 waves (2 of them
// loading the tiles), 3 workgroups per CU
template <>
struct Cfg<2, 2> : TileCfg<3, 3, 3, 2, 1> {};
constexpr int kStageBytes = kTileKBytes + kTileVBytes;
// Key-norm partial maxima per head (the logit bound's max|k|).
constexpr int kNormChunks = 256;
// Margin on |q'| max|k| for the rounding of the norms, of the fp32 scores and
// of the bf16 mean keys (the normalised result does not depend on it).
constexpr float kBoundMargin = 1.0078125f;  // 1 + 2^-7
// A row whose probabilities against the bound sum below this is redone exactly:
// every key then within 2^-25 of the row's total weight is a normal float.
constexpr float kLooseBoundSum = 8.271806125530277e-25f;  // 2^-80
// Occupancy of the one-half configuration (FRAME, the rest of a SUBSAMPLED
// frame): 3 workgroups (12 waves) per CU with a 3-stage LDS ring (144 KiB).
// Measured on MI355X at 128 frames (dense attention, % of bf16 peak): 3 stages
// and 3 workgroups 44-46%; 2 / 3 43%; 2 / 4, where the 128-VGPR budget makes the
// compiler spill inside the tile loop, 37%. A ping-pong schedule of two
// barrier-locked wave groups per SIMD (one group on MFMA while the other
// computes probabilities) reached only 30-39%: the per-phase barriers, LDS
// waits and scalar work cost more than the forced overlap gains, where three
// free-running waves per SIMD overlap MFMA and VALU work by themselves.

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
  int token_diag;    // SUBSAMPLED: 1 = no whole own frame; own compacted rows and mean kept
  float bound_extra; // added to every query's logit bound: mean_bias2 if mean rows exist
  const float* knorm2;  // [H, kNormChunks] maxima of |k|^2
  unsigned char* redo;  // [n_logical] 1: the workgroup's rows need the exact pass
  float scale_log2;  // log2(e) / sqrt(d)
  int n_qtiles;      // GLOBAL: tiles over T; else tiles per frame
  int q_off, q_span; // FRAME/SUBSAMPLED: the query rows [q_off, q_off + q_span) of each frame
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

// 16-byte direct load into LDS through a buffer resource: the base and the
// extent are wave-uniform (SGPRs) and the lane's 32-bit offset is fixed for the
// kernel; a lane whose 16 bytes reach past the extent gets zeros, no access.
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                          unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds_dst, 16, (int)voff, 0, 0, 0);
}

// Wait until at most N direct loads of this lane are in flight and its LDS
// reads have returned, then meet the other waves: every wave's loads of the
// tile about to be read have landed and every wave is done reading the stage
// about to be refilled. (The compiler may leave a tile's last LDS reads in
// flight across the barrier, their MFMAs after it; lgkmcnt(0) keeps the refill
// of that stage behind them.)
template <int N>
__device__ __forceinline__ void wait_and_meet() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  // vmcnt <= N (bits 3:0 and 15:14), lgkmcnt = 0 (bits 11:8), expcnt unconstrained
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// EXACT = false: the main pass against the logit bound; every workgroup records
// in A.redo whether some row's probabilities underflowed. EXACT = true: only the
// recorded workgroups run, redoing their rows with the exact online softmax.
template <int MODE, bool EXACT, int PART>
__device__ __forceinline__ void flash_tile(const FlashArgs& A, int lid, unsigned char* smem) {
  using C = Cfg<MODE, PART>;
  constexpr int kStages = C::stages;
  constexpr int kAhead = kStages - 1;  // tiles in flight ahead of the one consumed
  constexpr int kBlockM = C::block_m;
  constexpr int kRowsPerWave = C::rows_per_wave;
  constexpr int kLoadsPerTile = C::loads_per_tile;

  if (lid >= A.n_logical) return;
  if (EXACT && A.redo[lid] == 0) return;
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
    q0 = (long long)f * A.g.L + A.q_off + (long long)(rem % A.n_qtiles) * kBlockM;
    q_end = min(q0 + kBlockM, (long long)f * A.g.L + A.q_off + A.q_span);
  }

  // ---- key segments ----------------------------------------------------------
  Segment seg0, seg1;
  const bool token_diag = MODE == MODE_SUBSAMPLED && A.token_diag != 0;
  if (MODE == MODE_GLOBAL) {
    seg0 = Segment{A.k, 0, A.vt, 0, A.vt_ld, A.n_keys};
  } else {
    seg0 = Segment{A.k, (long long)f * A.g.L, A.vt, (long long)f * A.vt_pitch, A.vt_ld,
                   token_diag ? 0 : A.g.L};
  }
  seg1 = Segment{A.ck, 0, A.cvt, 0, A.cvt_ld,
                 MODE == MODE_SUBSAMPLED ? (long long)A.g.n_frames * (A.mk + A.has_mean) : 0};
  // tile counts fit 32 bits (at most 2^31 keys per segment, 64 per tile): the
  // per-tile bookkeeping below stays in 32-bit scalar arithmetic
  const int nt0 = (int)((seg0.n + kTileKeys - 1) / kTileKeys);
  const int n_tiles = nt0 + (int)((seg1.n + kTileKeys - 1) / kTileKeys);
  // compacted rows of the own frame (masked unless token_diag), the mean rows
  // (log-count bias)
  const long long own0 = token_diag ? 0 : (long long)f * A.mk;
  const long long own1 = token_diag ? 0 : own0 + A.mk;
  const long long mean0 = (long long)A.g.n_frames * A.mk;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const long long rs = (long long)A.g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;
  const float c = A.scale_log2;

  // ---- direct tile loads -------------------------------------------------------
  // lane -> row r = wave * kRowsPerWave + 8 i + lane / 8 of the tile (a key row of
  // K, a d row of V^T) and physical 16-byte chunk lane % 8. Every load is a
  // per-tile buffer resource (scalar) plus a per-lane 32-bit offset fixed for the
  // kernel, and the LDS destination is wave-uniform, so issuing a tile costs no
  // VALU work. A segment's last tile limits the K resource to its valid rows:
  // the rows past the end load as zeros (and are masked).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int ld_r = lane >> 3, ld_p = lane & 7;
  uint32_t k_off[kRowsPerWave / 8], v_off0[kRowsPerWave / 8], v_off1[kRowsPerWave / 8];
#pragma unroll
  for (int i = 0; i < kRowsPerWave / 8; ++i) {
    const int r = wave_u * kRowsPerWave + 8 * i + ld_r;
    const int kc = ld_p ^ ld_r;                               // K swizzle: chunk ^ (r & 7)
    const int vc = ld_p ^ ld_r ^ ((wave_u * (kRowsPerWave / 8) + i) & 7);  // V^T: chunk ^ swz(r)
    k_off[i] = (uint32_t)((r * rs + kc * 8) * 2);
    v_off0[i] = (uint32_t)(r * 128 + vc * 16);  // V^T tiles are 64 x 64 contiguous blocks
    v_off1[i] = v_off0[i];
  }
  // Per segment, fixed for the kernel: the byte address of this head's first K
  // row and first V^T column, the V^T extent and the key count. A tile then
  // costs one 32x32-bit product and a few adds on the scalar unit; the key and
  // byte counts fit 31 bits (checked at launch).
  const int row_bytes = (int)(rs * 2);
  // (a head's V^T is ld / 64 tiles of 64 d-rows x 128 B: 128 B per column)
  const char* const kb0 = reinterpret_cast<const char*>(seg0.k + seg0.k_row0 * rs + hoff);
  const char* const vb0 = reinterpret_cast<const char*>(seg0.vt) + (h * seg0.vt_ld + seg0.vt_col0) * 128;
  const int n0 = (int)seg0.n;
  const char* kb1 = kb0;
  const char* vb1 = vb0;
  int n1 = n0;
  if (MODE == MODE_SUBSAMPLED) {
    kb1 = reinterpret_cast<const char*>(seg1.k + seg1.k_row0 * rs + hoff);
    vb1 = reinterpret_cast<const char*>(seg1.vt) + (h * seg1.vt_ld + seg1.vt_col0) * 128;
    n1 = (int)seg1.n;
  }
  auto issue_tile = [&](int j, unsigned char* stage) {
    const bool second = MODE == MODE_SUBSAMPLED && j >= nt0;
    const int u0 = (second ? j - nt0 : j) * kTileKeys;
    const int rows = min(kTileKeys, (second ? n1 : n0) - u0);
    const auto kr = buffer_rsrc((second ? kb1 : kb0) + (long long)u0 * row_bytes, rows * row_bytes);
    const auto vr = buffer_rsrc((second ? vb1 : vb0) + (long long)u0 * 128, kTileVBytes);
    unsigned char* kdst = stage + wave_u * kRowsPerWave * 128;
    unsigned char* vdst = kdst + kTileKBytes;
    if (C::dma_waves < C::waves && wave_u >= C::dma_waves) return;
#pragma unroll
    for (int i = 0; i < kRowsPerWave / 8; ++i) {
      lds_dma16(kr, k_off[i], kdst + 8 * i * 128);
      lds_dma16(vr, second ? v_off1[i] : v_off0[i], vdst + 8 * i * 128);
    }
  };

  // ---- tile order: every clean tile first, the masked ones after -------------
  // Tile t (t < nt0: segment 0, else segment 1 tile t - nt0) needs a logit mask
  // or bias when it holds a segment's end, the query frame's own compacted rows,
  // the own frame's mean row, or mean rows that carry the log-count bias. Those
  // few tiles run after the clean ones, in a loop of their own, so that the
  // masking code never occupies registers of the main loop. The order does not
  // matter to the softmax sum. Unbiased mean rows are ordinary keys, so only the
  // tile tm holding the own frame's mean row leaves the clean range (when it
  // lies in [b1, m1); elsewhere it is masked already).
  //   clean:  segment 0 [0, c0), segment 1 [0, a1) and [b1, m1) without tm
  //   masked: segment 0 [c0, nt0), segment 1 [a1, min(b1, m1)), tm, [m1, nt1)
  const int nt1 = n_tiles - nt0;
  const int c0 = (int)(seg0.n / kTileKeys);
  int a1 = 0, b1 = 0, m1 = 0, tm = 0x7fffffff;
  if (MODE == MODE_SUBSAMPLED) {
    const bool mean_biased = A.has_mean && A.mean_bias2 != 0.f;
    const long long clean_end = mean_biased ? min(mean0, seg1.n) : seg1.n;
    m1 = (int)(clean_end / kTileKeys);
    a1 = min((int)(own0 / kTileKeys), m1);
    b1 = (int)((own1 + kTileKeys - 1) / kTileKeys);
    if (A.has_mean && !mean_biased && !token_diag) {
      const int t = (int)((mean0 + f) / kTileKeys);
      if (t >= b1 && t < m1) tm = t;
    }
  }
  const int ex = tm != 0x7fffffff ? 1 : 0;
  const int n_r2 = max(0, m1 - b1) - ex;
  const int n_clean = c0 + a1 + n_r2;
  auto tile_of = [&](int j) -> int {
    if (j < c0) return j;
    j -= c0;
    if (j < a1) return nt0 + j;
    j -= a1;
    if (j < n_r2) {
      const int t = b1 + j;
      return nt0 + t + (t >= tm ? 1 : 0);
    }
    j -= n_r2;
    if (j < nt0 - c0) return c0 + j;
    j -= nt0 - c0;
    const int own_masked = min(b1, m1) - a1;
    if (j < own_masked) return nt0 + a1 + j;
    j -= own_masked;
    if (ex) {
      if (j == 0) return nt0 + tm;
      --j;
    }
    return nt0 + m1 + j;
  };
  // (logits in log2 units: the mean rows' bias adds as it is). Every bound is
  // taken relative to the half-tile's first key and clamped to [-1, 64], so the
  // per-score tests are 32-bit compares against wave-uniform values.
  auto apply_mask = [&](int j, int kb, f32x16& s) {
    const bool second = j >= nt0;
    const long long u0 = (long long)(second ? j - nt0 : j) * kTileKeys + kb * 32;
    auto rel = [&](long long x) { return (int)max(-1LL, min(x - u0, 64LL)); };
    const int lim = rel(second ? seg1.n : seg0.n);
    int own_a = 64, own_b = 64, own_mean = -1, mean_a = 64;
    if (MODE == MODE_SUBSAMPLED && second) {
      own_a = rel(own0);
      own_b = rel(own1);
      if (A.has_mean) {
        own_mean = token_diag ? -1 : rel(mean0 + f);
        mean_a = rel(mean0);
      }
    }
    // the lane's key base is made opaque here so that the 16 key offsets are
    // formed inside the (rare) masked tile instead of being hoisted out of the
    // tile loop into 16 live registers
    int ubase = 4 * hh;
    asm volatile("" : "+v"(ubase));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = 8 * (i >> 2) + ubase + (i & 3);
      const bool ok = u < lim && !(u >= own_a && u < own_b) && u != own_mean;
      s[i] = ok ? s[i] + (u >= mean_a ? A.mean_bias2 : 0.f) : -INFINITY;
    }
  };

  constexpr int kHalves = C::halves;
  long long qrow[kHalves];
  bool qvalid[kHalves];
  u32x4 qB[kHalves][4];
#pragma unroll
  for (int hq = 0; hq < kHalves; ++hq) {
    qrow[hq] = q0 + (wave * kHalves + hq) * 32 + li;
    qvalid[hq] = qrow[hq] < q_end;
    load_q_operand_scaled(A.q + (qvalid[hq] ? qrow[hq] : q0) * rs + hoff, qvalid[hq], c, qB[hq]);
  }

  TileLaneOffsets off;
  off.init();

  // The tile loop: a ring of kStages LDS stages, kAhead tiles in flight, in
  // the order tile_of(0), tile_of(1), ... (the ring's first loads are issued by
  // drive below)
  // wait for tile j (the tiles after it in flight: min(kAhead - 1, left)), meet
  // the other waves (all done with tile j - 1's stage), refill that stage
  // (waves that issue no loads have nothing outstanding: every wait passes)
  auto enter = [&](int j, unsigned char* refill_stage) {
    const int left = n_tiles - 1 - j;
    if (left >= kAhead - 1) {
      wait_and_meet<(kAhead - 1) * kLoadsPerTile>();
    } else if (kAhead > 2 && left == kAhead - 2) {
      wait_and_meet<(kAhead > 2 ? kAhead - 2 : 0) * kLoadsPerTile>();
    } else if (kAhead > 3 && left == kAhead - 3) {
      wait_and_meet<(kAhead > 3 ? kAhead - 3 : 0) * kLoadsPerTile>();
    } else if (left > 0) {
      // (deeper rings: wait for everything rather than track each count)
      wait_and_meet<0>();
    } else {
      wait_and_meet<0>();
    }
    if (j + kAhead < n_tiles) issue_tile(tile_of(j + kAhead), refill_stage);
  };
  // The clean tiles in whole rounds of the ring while the tile issued ahead is
  // clean as well: its index then comes from the three clean ranges alone and
  // every wait keeps kAhead - 1 tiles in flight. The rest (a partial round, the
  // last kAhead clean tiles and the masked ones) run one by one with runtime
  // stage addresses.
  auto clean_tile = [&](int j) -> int {
    if (j < c0) return j;
    j -= c0;
    if (j < a1) return nt0 + j;
    const int t = b1 + (j - a1);
    return nt0 + t + (t >= tm ? 1 : 0);
  };
  auto enter_clean = [&](int j, unsigned char* refill_stage) {
    wait_and_meet<(kAhead - 1) * kLoadsPerTile>();
    issue_tile(clean_tile(j + kAhead), refill_stage);
  };
  const int n_main = max(0, n_clean - kAhead) / kStages * kStages;
  auto run_rest = [&](auto&& step) {
    for (int j = n_main; j < n_tiles; ++j) {
      const int cur = (int)(j % kStages);
      enter(j, smem + ((cur + kAhead) % kStages) * kStageBytes);
      step(tile_of(j), smem + cur * kStageBytes);
    }
  };
  // The whole key stream: clean(stage) for each tile of the main rounds (all
  // clean), rest(t, stage) for tile t of the others.
  //   ring:  kAhead tiles in flight; one wait and barrier per tile.
  //   groups of P tiles (P = C::group > 1): stages [0, P) and [P, 2P)
  //          alternate; at each barrier (every P tiles) the group just freed
  //          is refilled with the tiles P ahead, whose loads then have P
  //          tiles' time to land -- a barrier per P tiles, for 2P stages.
  auto drive = [&](auto&& clean, auto&& rest) {
    if constexpr (C::group == 1) {
#pragma unroll
      for (int j = 0; j < kAhead; ++j)
        if (j < n_tiles) issue_tile(tile_of(j), smem + j * kStageBytes);
      for (int j = 0; j < n_main; j += kStages) {
#pragma unroll
        for (int cur = 0; cur < kStages; ++cur) {
          enter_clean(j + cur, smem + ((cur + kAhead) % kStages) * kStageBytes);
          clean(smem + cur * kStageBytes);
        }
      }
      run_rest(rest);
    } else {
      constexpr int P = C::group;
#pragma unroll
      for (int i = 0; i < P; ++i)
        if (i < n_tiles) issue_tile(tile_of(i), smem + i * kStageBytes);
      // main rounds of 2P clean tiles; every tile issued ahead is clean too
      const int n_main_g = max(0, n_clean - P) / (2 * P) * (2 * P);
      for (int j = 0; j < n_main_g; j += 2 * P) {
        wait_and_meet<0>();
#pragma unroll
        for (int i = 0; i < P; ++i) issue_tile(clean_tile(j + P + i), smem + (P + i) * kStageBytes);
#pragma unroll
        for (int i = 0; i < P; ++i) clean(smem + i * kStageBytes);
        wait_and_meet<0>();
#pragma unroll
        for (int i = 0; i < P; ++i) issue_tile(clean_tile(j + 2 * P + i), smem + i * kStageBytes);
#pragma unroll
        for (int i = 0; i < P; ++i) clean(smem + (P + i) * kStageBytes);
      }
      for (int j = n_main_g; j < n_tiles; j += P) {
        wait_and_meet<0>();
        const int sj = j % (2 * P);  // 0 or P: the group's first stage
        const int so = P - sj;       // the other group's first stage
        for (int i = 0; i < P; ++i)
          if (j + P + i < n_tiles) issue_tile(tile_of(j + P + i), smem + (so + i) * kStageBytes);
        for (int i = 0; i < P; ++i)
          if (j + i < n_tiles) rest(tile_of(j + i), smem + (sj + i) * kStageBytes);
      }
    }
  };
  bf16* orow[kHalves];
  float* lse_ptr[kHalves];
#pragma unroll
  for (int hq = 0; hq < kHalves; ++hq) {
    orow[hq] = A.o + qrow[hq] * rs + hoff;
    lse_ptr[hq] = A.lse ? A.lse + qrow[hq] * A.g.n_heads + h : nullptr;
  }
  if constexpr (EXACT) {
    // scores already in log2 units, so c = 1
    WaveAttnState ex[kHalves];
#pragma unroll
    for (int hq = 0; hq < kHalves; ++hq) ex[hq].init();
    auto step = [&](int t, const unsigned char* stage, bool masked) {
#pragma unroll
      for (int hq = 0; hq < kHalves; ++hq) {
        f32x16 sc[2];
        ex[hq].scores(stage, off, qB[hq], sc);
        if (masked) {
          apply_mask(t, 0, sc[0]);
          apply_mask(t, 1, sc[1]);
        }
        ex[hq].consume(sc, stage, off, 1.f, false, true);
      }
    };
    drive([&](const unsigned char* stage) { step(0, stage, false); },
          [&](int t, const unsigned char* stage) { step(t, stage, true); });
#pragma unroll
    for (int hq = 0; hq < kHalves; ++hq) ex[hq].finish(orow[hq], lse_ptr[hq], qvalid[hq], 1.f);
  } else {
    // Upper bound of the query's logits (log2 units): |q'| max|k| with a margin
    // for the rounding of |q'|, of max|k| and of the bf16 mean keys, plus the
    // mean rows' bias. The key-norm partials are per (head, chunk) maxima of |k|^2.
    float bound[kHalves];
    {
      float k2 = 0.f;
      for (int i = lane; i < kNormChunks; i += 64) k2 = fmaxf(k2, A.knorm2[h * kNormChunks + i]);
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) k2 = fmaxf(k2, __shfl_xor(k2, sh));
#pragma unroll
      for (int hq = 0; hq < kHalves; ++hq) {
        float q2 = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float a0 = lo_bf16(qB[hq][ks][jj]), a1 = hi_bf16(qB[hq][ks][jj]);
            q2 = fmaf(a0, a0, fmaf(a1, a1, q2));
          }
        q2 = sum_halves(q2);
        bound[hq] = sqrtf(q2) * sqrtf(k2) * kBoundMargin + A.bound_extra;
      }
    }
    // A bound far above a row's true maximum leaves its probabilities below
    // the fp32 range: the workgroup is then redone by the exact pass.
    bool loose = false;
    if constexpr (kHalves == 1) {
      FlashWaveState st;
      st.init(bound[0]);
      drive([&](const unsigned char* stage) { st.tile<false>(stage, off, qB[0], [](int, f32x16&) {}); },
            [&](int t, const unsigned char* stage) {
              st.tile<true>(stage, off, qB[0], [&](int kb, f32x16& s) { apply_mask(t, kb, s); });
            });
      loose = !(sum_halves(st.l) >= kLooseBoundSum);
      st.finish(orow[0], lse_ptr[0], qvalid[0]);
    } else {
      FlashWaveState2 st;
      st.init(bound[0], bound[1]);
      drive([&](const unsigned char* stage) { st.tile<false>(stage, off, qB[0], qB[1], [](int, f32x16&) {}); },
            [&](int t, const unsigned char* stage) {
              st.tile<true>(stage, off, qB[0], qB[1], [&](int kb, f32x16& s) { apply_mask(t, kb, s); });
            });
      loose = !(sum_halves(st.a.l) >= kLooseBoundSum) || !(sum_halves(st.b.l) >= kLooseBoundSum);
      st.a.finish(orow[0], lse_ptr[0], qvalid[0]);
      st.b.finish(orow[1], lse_ptr[1], qvalid[1]);
    }
    const int any_loose = __syncthreads_or(loose);
    if (tid == 0) A.redo[lid] = any_loose ? 1 : 0;
  }
}

// The kernel: one workgroup per logical workgroup (remapped per XCD in
// FRAME/SUBSAMPLED mode). A persistent grid that keeps the resident
// workgroups streaming the same keys in step was measured slower at every
// size (1000 frames: 43.8-45.8% of the bf16 peak against 48-49%).
template <int MODE, bool EXACT, int PART>
__global__ __launch_bounds__((Cfg<MODE, PART>::threads), (Cfg<MODE, PART>::wg_per_cu)) void flash_bf16_kernel(
    FlashArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int lid = blockIdx.x;
  if (A.remap) {
    const int per = (A.n_logical + 7) >> 3;
    lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  flash_tile<MODE, EXACT, PART>(A, lid, smem);
}

// Per (head, chunk) maximum of |k|^2 over the rows of K: a workgroup per
// (head, chunk), 8 lanes per 128-byte key row.
__global__ __launch_bounds__(256) void knorm_partial_kernel(const bf16* __restrict__ k,
                                                            long long n_rows, int n_heads,
                                                            float* __restrict__ out) {
  const int h = blockIdx.x / kNormChunks, chunk = blockIdx.x % kNormChunks;
  const long long per = (n_rows + kNormChunks - 1) / kNormChunks;
  const long long r0 = chunk * per, r1 = min(r0 + per, n_rows);
  const long long rs = (long long)n_heads * kHeadDim;
  const int t = threadIdx.x, part = t & 7;
  float best = 0.f;
  for (long long r = r0 + (t >> 3); r < r1; r += 32) {
    const u32x4 w = ld16(k + r * rs + (long long)h * kHeadDim + part * 8);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = lo_bf16(w[j]), a1 = hi_bf16(w[j]);
      acc = fmaf(a0, a0, fmaf(a1, a1, acc));
    }
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

}  // namespace

// Workspace: the V^T staging (a multiple of 8 KiB), then the key-norm partials.
// V^T row length (columns) of the staging of K/V (and of the compacted set).
static long long vt_ld_main(const FlashLaunch& p) {
  if (p.mode == FLASH_GLOBAL) return (p.n_keys + 63) / 64 * 64;
  return (long long)((p.g.L + 63) / 64 * 64) * p.g.n_frames;
}
static long long vt_ld_compact(const FlashLaunch& p) {
  if (p.mode != FLASH_SUBSAMPLED) return 0;
  return ((long long)p.g.n_frames * (p.mk + p.has_mean) + 63) / 64 * 64;
}
// The launches of one call: the query rows [q_off, q_off + q_span) of every
// frame (FRAME/SUBSAMPLED; GLOBAL: all of T) in tiles of block_m, with the
// tile configuration `part` (Cfg<mode, part>).
struct LaunchPart {
  int part, block_m, q_off, q_span, n_qtiles;
  long long n_logical;
};
static int launch_parts(const FlashLaunch& p, LaunchPart out[2]) {
  if (p.mode == FLASH_GLOBAL) {
    const int bm = Cfg<MODE_GLOBAL>::block_m;
    const long long nq = (p.g.T + bm - 1) / bm;
    out[0] = LaunchPart{0, bm, 0, 0, (int)min(nq, 0x7fffffffLL), nq * p.g.n_heads};
    return 1;
  }
  const long long per_frame = (long long)p.g.n_frames * p.g.n_heads;
  if (p.mode == FLASH_FRAME) {
    const int bm = Cfg<MODE_FRAME>::block_m;
    const int nq = (p.g.L + bm - 1) / bm;
    out[0] = LaunchPart{0, bm, 0, p.g.L, nq, nq * per_frame};
    return 1;
  }
  // SUBSAMPLED: whole two-half tiles, then the rest in one one-half tile of 96
  // or 128 rows when it fits one (else the two-half tiles cover the frame)
  const int bm = Cfg<MODE_SUBSAMPLED, 0>::block_m, bt = Cfg<MODE_SUBSAMPLED, 1>::block_m,
            bs = Cfg<MODE_SUBSAMPLED, 2>::block_m;
  const int rest = p.g.L % bm;
  const int main_rows = (rest == 0 || rest > bt) ? p.g.L : p.g.L - rest;
  int n = 0;
  if (main_rows > 0) {
    const int nq = (main_rows + bm - 1) / bm;
    out[n++] = LaunchPart{0, bm, 0, main_rows, nq, nq * per_frame};
  }
  if (main_rows < p.g.L) {
    const int r = p.g.L - main_rows;  // 1 .. bt rows: one tile
    const int part = r <= bs ? 2 : 1;
    out[n++] = LaunchPart{part, part == 2 ? bs : bt, main_rows, r, 1, per_frame};
  }
  return n;
}
static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace: the V^T staging (a multiple of 8 KiB), the key-norm partials,
// the per-workgroup redo flags.
static size_t vt_bytes(const FlashLaunch& p) {
  return (size_t)p.g.n_heads * kHeadDim * (vt_ld_main(p) + vt_ld_compact(p)) * 2;
}
static size_t norm_bytes(const FlashLaunch& p) {
  return round256((size_t)p.g.n_heads * kNormChunks * sizeof(float));
}

// one redo flag byte per logical workgroup of each launch
static size_t flag_bytes(const FlashLaunch& p) {
  LaunchPart parts[2];
  const int n = launch_parts(p, parts);
  size_t b = 0;
  for (int i = 0; i < n; ++i) b += round256((size_t)parts[i].n_logical);
  return b;
}

size_t flash_bf16_workspace(const FlashLaunch& p) {
  return vt_bytes(p) + norm_bytes(p) + flag_bytes(p);
}

static bool parts_fit(const FlashLaunch& p) {
  LaunchPart parts[2];
  const int n = launch_parts(p, parts);
  for (int i = 0; i < n; ++i)
    if (parts[i].n_logical > 0x7ffffff0LL || (long long)parts[i].n_qtiles * parts[i].block_m > 0x7fffffffLL)
      return false;
  return true;
}

bool flash_bf16_fits(const FlashLaunch& p) {
  // buffer extents of one tile: 64 K rows, 64 V^T rows, in 31 bits
  const long long lim = 0x7fffffffLL;
  return (long long)kTileKeys * p.g.n_heads * kHeadDim * 2 <= lim &&
         (long long)kHeadDim * vt_ld_main(p) * 2 <= lim &&
         (long long)kHeadDim * vt_ld_compact(p) * 2 <= lim && parts_fit(p);
}

hipError_t launch_flash_bf16(const FlashLaunch& p, void* ws, hipStream_t stream) {
  if (!flash_bf16_fits(p)) return hipErrorInvalidValue;
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
  A.token_diag = p.token_diag;
  A.scale_log2 = kLog2e / sqrtf((float)kHeadDim);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  bf16* vt = reinterpret_cast<bf16*>(wsb);
  float* knorm2 = reinterpret_cast<float*>(wsb + vt_bytes(p));
  unsigned char* const redo = wsb + vt_bytes(p) + norm_bytes(p);
  A.vt = vt;
  A.vt_ld = vt_ld_main(p);
  hipError_t e;
  if (p.mode == FLASH_GLOBAL) {
    e = launch_vt_prepare(p.v, p.g.n_heads, p.n_keys, p.n_keys, A.vt_ld, A.vt_ld, vt, stream);
    if (e != hipSuccess) return e;
    A.remap = 0;
  } else {
    A.vt_pitch = (p.g.L + 63) / 64 * 64;
    if (!(p.mode == FLASH_SUBSAMPLED && p.token_diag)) {  // token_diag reads no whole frame
      e = launch_vt_prepare(p.v, p.g.n_heads, p.g.T, p.g.L, A.vt_pitch, A.vt_ld, vt, stream);
      if (e != hipSuccess) return e;
    }
    if (p.mode == FLASH_SUBSAMPLED) {
      const long long rows = (long long)p.g.n_frames * (p.mk + p.has_mean);
      A.cvt_ld = vt_ld_compact(p);
      bf16* cvt = vt + (size_t)p.g.n_heads * kHeadDim * A.vt_ld;
      e = launch_vt_prepare(p.cv, p.g.n_heads, rows, rows, A.cvt_ld, A.cvt_ld, cvt, stream);
      if (e != hipSuccess) return e;
      A.cvt = cvt;
    }
    A.remap = 1;
  }
  // key-norm partials over every key the queries can meet (the compacted
  // rows are copies and means of these, covered by the bound's margin)
  const long long norm_rows = p.mode == FLASH_GLOBAL ? p.n_keys : p.g.T;
  hipLaunchKernelGGL(knorm_partial_kernel, dim3(p.g.n_heads * kNormChunks), dim3(256), 0, stream,
                     static_cast<const bf16*>(p.k), norm_rows, p.g.n_heads, knorm2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  A.knorm2 = knorm2;
  A.bound_extra = (p.mode == FLASH_SUBSAMPLED && p.has_mean) ? p.mean_bias2 : 0.f;
  // per launch part: the main pass, then the exact pass over the workgroups
  // it flagged (each part with its own redo flags)
  LaunchPart parts[2];
  const int n_parts = launch_parts(p, parts);
  size_t flag_off = 0;
  for (int i = 0; i < n_parts; ++i) {
    const LaunchPart& lp = parts[i];
    A.n_qtiles = lp.n_qtiles;
    A.q_off = lp.q_off;
    A.q_span = lp.q_span;
    A.n_logical = (int)lp.n_logical;
    A.redo = redo + flag_off;
    flag_off += round256((size_t)lp.n_logical);
    const int grid = A.remap ? ((A.n_logical + 7) / 8) * 8 : A.n_logical;
    auto launch = [&](auto kernel, auto cfg) {
      using C = decltype(cfg);
      hipLaunchKernelGGL(kernel, dim3(grid), dim3(C::threads), C::stages * kStageBytes, stream, A);
    };
    switch (p.mode) {
      case FLASH_GLOBAL:
        launch(flash_bf16_kernel<MODE_GLOBAL, false, 0>, Cfg<MODE_GLOBAL>{});
        launch(flash_bf16_kernel<MODE_GLOBAL, true, 0>, Cfg<MODE_GLOBAL>{});
        break;
      case FLASH_FRAME:
        launch(flash_bf16_kernel<MODE_FRAME, false, 0>, Cfg<MODE_FRAME>{});
        launch(flash_bf16_kernel<MODE_FRAME, true, 0>, Cfg<MODE_FRAME>{});
        break;
      default:
        if (lp.part == 0) {
          launch(flash_bf16_kernel<MODE_SUBSAMPLED, false, 0>, Cfg<MODE_SUBSAMPLED, 0>{});
          launch(flash_bf16_kernel<MODE_SUBSAMPLED, true, 0>, Cfg<MODE_SUBSAMPLED, 0>{});
        } else if (lp.part == 1) {
          launch(flash_bf16_kernel<MODE_SUBSAMPLED, false, 1>, Cfg<MODE_SUBSAMPLED, 1>{});
          launch(flash_bf16_kernel<MODE_SUBSAMPLED, true, 1>, Cfg<MODE_SUBSAMPLED, 1>{});
        } else {
          launch(flash_bf16_kernel<MODE_SUBSAMPLED, false, 2>, Cfg<MODE_SUBSAMPLED, 2>{});
          launch(flash_bf16_kernel<MODE_SUBSAMPLED, true, 2>, Cfg<MODE_SUBSAMPLED, 2>{});
        }
        break;
    }
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess) return le;
  }
  return hipGetLastError();
}

}  // namespace sga
