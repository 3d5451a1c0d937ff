// One 64-key step of online-softmax attention for a wave owning 32 queries
// (gfx950, v_mfma_f32_32x32x16_bf16, head_dim 64), shared by every bf16
// attention kernel of the library.
//
// Formulation: scores are computed transposed, S^T = K Q^T, so lane l owns
// query (l % 32) and 16 keys of each 32-key block (keys 8g + 4(l/32) + r at
// element 4g + r). The output is accumulated transposed, O^T += V^T P^T, so the
// same lane owns every per-query quantity (running max, running sum, rescale
// factor) and P^T feeds the MFMA B operand straight from its score registers.
//
// LDS stage layout (kTileStageBytes):
//   K tile    64 keys x 128 B; 16-byte chunk c of key row r lives at chunk
//             c ^ (r & 7), so the 16-byte operand reads of 8 consecutive lanes
//             (8 rows, one logical chunk) cover all 32 banks.
//   V^T tile  64 d-rows x 128 B of keys. Within every 16-key group the key
//             offset 8a + 4hh + r sits at column 8hh + 4a + r, so one 16-byte
//             read returns exactly the 8 keys of a lane's MFMA B slots; chunk x
//             of row d lives at x ^ ((d & 7) ^ ((d >> 3) & 7)). The loader
//             transposes in registers: a thread holding two consecutive keys'
//             8-value chunks packs (key, key+1) pairs per d with v_perm and
//             writes them as dwords (the pair is adjacent in the column order).
//             16-byte LDS reads run about 3x the bandwidth of the gfx950 LDS
//             transpose read, which is why V is transposed on the way in.
//   bias      64 floats added (log2 units) to the tile's logits when asked
#pragma once

#include "common.hpp"

namespace sga {

constexpr int kTileKeys = 64;
constexpr int kTileKBytes = kTileKeys * 128;
constexpr int kTileVBytes = kHeadDim * 128;
constexpr int kTileStageBytes = kTileKBytes + kTileVBytes + kTileKeys * 4;
constexpr float kLazyRescaleLog2 = 8.0f;

__device__ __forceinline__ int tile_k_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}
__device__ __forceinline__ int tile_vt_off(int d, int pos) {
  const int swz = (d & 7) ^ ((d >> 3) & 7);
  return kTileKBytes + d * 128 + (((pos >> 3) ^ swz) << 4) + ((pos & 7) << 1);
}
// Column of key offset u (0..63) inside a V^T row: within each 16-key group the
// offset 8a + 4hh + r moves to 8hh + 4a + r.
__device__ __forceinline__ int tile_vt_pos(int u) {
  const int o = u & 15;
  const int a = o >> 3, hh = (o >> 2) & 1, r = o & 3;
  return (u & ~15) | (hh << 3) | (a << 2) | r;
}

// Write the 16-byte chunk `chunk` (8 d-values) of keys u and u + 1 (u even)
// into a stage: K rows as they are, V transposed as (u, u + 1) dword pairs.
__device__ __forceinline__ void tile_store_kv_pair(unsigned char* stage, int u, int chunk,
                                                  const u32x4& ka, const u32x4& kb,
                                                  const u32x4& va, const u32x4& vb) {
  st16(stage + tile_k_off(u, chunk), ka);
  st16(stage + tile_k_off(u + 1, chunk), kb);
  const int pos = tile_vt_pos(u);  // pos(u + 1) = pos(u) + 1
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = chunk * 8 + 2 * j;
    // perm(x, y, sel) picks bytes of {x: 4..7, y: 0..3}
    const uint32_t lo = __builtin_amdgcn_perm(vb[j], va[j], 0x05040100u);  // (va.lo, vb.lo)
    const uint32_t hi = __builtin_amdgcn_perm(vb[j], va[j], 0x07060302u);  // (va.hi, vb.hi)
    *reinterpret_cast<uint32_t*>(stage + tile_vt_off(d, pos)) = lo;
    *reinterpret_cast<uint32_t*>(stage + tile_vt_off(d + 1, pos)) = hi;
  }
}
__device__ __forceinline__ float* tile_bias(unsigned char* stage) {
  return reinterpret_cast<float*>(stage + kTileKBytes + kTileVBytes);
}

// Q^T operand of a wave: lane l loads d = 16 ks + 8 (l/32) .. +8 of its query row.
__device__ __forceinline__ void load_q_operand(const bf16* qrow_ptr, bool valid, u32x4 qB[4]) {
  const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qB[ks] = valid ? ld16(qrow_ptr + hh * 8 + ks * 16) : u32x4{0, 0, 0, 0};
  }
}

// Per-lane byte offsets (within a stage) of the lane's MFMA operand reads,
// computed once per kernel so the tile loop does no address arithmetic.
struct TileLaneOffsets {
  uint32_t k[4];  // K rows li (+32 kb as an immediate), chunk 2 ks + hh
  // V^T row 32 db + li (+4096 db as an immediate), keys 32 kb + 16 mm + 8 hh:
  // the swizzled chunk (4 kb + 2 mm + hh) ^ swz(d) depends on kb and db only
  // through kb ^ db, so four offsets (a = kb ^ db, mm) cover all eight reads
  uint32_t v[4];
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5, li = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) k[ks] = (uint32_t)tile_k_off(li, 2 * ks + hh);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)  // db = 0, kb = a
        v[2 * a + mm] = (uint32_t)tile_vt_off(li, a * 32 + 16 * mm + 8 * hh);
  }
  __device__ __forceinline__ uint32_t v_off(int db, int kb, int mm) const {
    return v[2 * (kb ^ db) + mm] + db * 32 * 128;
  }
};

struct WaveAttnState {
  f32x16 oacc[2];  // O^T for d 0..31 and 32..63 of query (l % 32)
  float m;         // running max, raw logit units
  float l;         // this half-wave's share of the running sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < 16; ++i) { oacc[0][i] = 0.f; oacc[1][i] = 0.f; }
    m = -INFINITY;
    l = 0.f;
  }

  // Start from a normalised partial result: orow is the query's output over
  // some keys (bf16 [d]) and lse their log-sum-exp in natural-log units of the
  // scaled logits; it then counts as one key of logit lse and value orow.
  __device__ __forceinline__ void init_from(const bf16* orow, float lse) {
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(orow + db * 32 + 8 * g4 + 4 * hh);
        oacc[db][4 * g4 + 0] = lo_bf16(w[0]);
        oacc[db][4 * g4 + 1] = hi_bf16(w[0]);
        oacc[db][4 * g4 + 2] = lo_bf16(w[1]);
        oacc[db][4 * g4 + 3] = hi_bf16(w[1]);
      }
    m = lse * 8.f;  // raw logit units: the logits here are q.k, scaled by 1/sqrt(64) = 1/8
    l = 0.5f;       // each half-wave holds half of the sum, 1
  }

  // Scores of one 64-key tile: S^T = K Q^T for two 32-key blocks.
  __device__ __forceinline__ void scores(const unsigned char* stage, const TileLaneOffsets& off,
                                         const u32x4 qB[4], f32x16 s[2]) const {
    u32x4 ka[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = ld16(stage + off.k[ks] + kb * 32 * 128);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma32(ka[kb][ks], qB[ks], acc);
      s[kb] = acc;
    }
  }

  // Softmax of a tile's scores and O^T += V^T P^T with the tile's values.
  // c = log2(e)/sqrt(d); use_bias adds the stage's bias row; inactive lanes
  // (a query not attending these keys) skip the tile. The V^T operands are
  // requested before the softmax so their LDS latency hides behind it.
  __device__ __forceinline__ void consume(f32x16 s[2], const unsigned char* stage,
                                          const TileLaneOffsets& off, float c, bool use_bias,
                                          bool active) {
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const float* bs = reinterpret_cast<const float*>(stage + kTileKBytes + kTileVBytes);

    if (use_bias) {
      const float inv_c = 1.f / c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + kb * 32 + 8 * g4 + 4 * hh);
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][4 * g4 + r] = fmaf(b4[r], inv_c, s[kb][4 * g4 + r]);
        }
    }

    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    mx = max_halves(mx);
    if (!active) mx = -INFINITY;
    const float m_new = fmaxf(m, mx);
    if (__any(active && (m_new - m) * c > kLazyRescaleLog2)) {
      if (active) {
        const float alpha = fast_exp2((m - m_new) * c);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) { oacc[0][i] *= alpha; oacc[1][i] *= alpha; }
      }
    }
    // a lane that has seen no key yet (m = -inf) must not form inf - inf
    const float mc = (m == -INFINITY) ? 0.f : m * c;
    u32x4 pB[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = active ? fast_exp2(fmaf(s[kb][i], c, -mc)) : 0.f;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pB[kb][mm][j] = pack_bf16x2(p[8 * mm + 2 * j], p[8 * mm + 2 * j + 1]);
    }
    // running sum of the bf16-rounded probabilities the PV product uses
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) l = sum_bf16x8(pB[kb][mm], l);

#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          oacc[db] = mfma32(ld16(stage + off.v_off(db, kb, mm)), pB[kb][mm], oacc[db]);
  }

  // One whole 64-key tile: scores then softmax + PV.
  __device__ __forceinline__ void step(const unsigned char* stage, const TileLaneOffsets& off,
                                       const u32x4 qB[4], float c, bool use_bias, bool active) {
    f32x16 s[2];
    scores(stage, off, qB, s);
    consume(s, stage, off, c, use_bias, active);
  }

  // Normalise and store query (l % 32)'s row (if valid); lse in natural-log units.
  __device__ __forceinline__ void finish(bf16* orow, float* lse_ptr, bool valid, float c) {
    const int hh = (threadIdx.x & 63) >> 5;
    const float l_tot = sum_halves(l);
    const float inv = 1.f / l_tot;
    if (!valid) return;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hh;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (lse_ptr != nullptr && hh == 0) *lse_ptr = (m * c + __log2f(l_tot)) * 0.6931471805599453f;
  }

  // As finish, but store g_mix * mix_row + g_self * (this row), the normalised
  // row taken before rounding (a gated aggregation of two branch outputs).
  __device__ __forceinline__ void finish_mixed(bf16* orow, const bf16* mix_row, float g_mix, float g_self,
                                               bool valid) {
    const int hh = (threadIdx.x & 63) >> 5;
    const float l_tot = sum_halves(l);
    const float inv = 1.f / l_tot;
    if (!valid) return;
    const float gs = g_self * inv;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hh;
        const u32x2 mx = *reinterpret_cast<const u32x2*>(mix_row + d0);
        u32x2 w;
        w[0] = pack_bf16x2(fmaf(g_mix, lo_bf16(mx[0]), oacc[db][4 * g4 + 0] * gs),
                           fmaf(g_mix, hi_bf16(mx[0]), oacc[db][4 * g4 + 1] * gs));
        w[1] = pack_bf16x2(fmaf(g_mix, lo_bf16(mx[1]), oacc[db][4 * g4 + 2] * gs),
                           fmaf(g_mix, hi_bf16(mx[1]), oacc[db][4 * g4 + 3] * gs));
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
  }
};

// Q' operand with the softmax scale folded in: bf16(q * c), nearest-even, so
// that K Q'^T is the logit in log2 units.
__device__ __forceinline__ void load_q_operand_scaled(const bf16* qrow_ptr, bool valid, float c,
                                                      u32x4 qB[4]) {
  load_q_operand(qrow_ptr, valid, qB);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j) qB[ks][j] = pack_bf16x2(lo_bf16(qB[ks][j]) * c, hi_bf16(qB[ks][j]) * c);
}

// ---------------------------------------------------------------------------
// Streaming softmax against a fixed upper bound (the flash kernel's main pass).
//
// With Q' = bf16(q c) the MFMA returns logits S' in log2 units. Every logit of
// a query is at most b = |q'| max_k |k| (Cauchy-Schwarz), so with the
// accumulator started at -b (broadcast in `negm`) the MFMA returns S' - b <= 0
// and each probability is one v_exp: no scaling, subtraction, running maximum
// or rescaling per score. The normalised result does not depend on the
// reference; a fixed one only risks underflow when b exceeds the row's true
// maximum by more than the fp32 exponent range can absorb, which the caller
// detects from the final sum and then redoes the rows with the exact online
// softmax (WaveAttnState with c = 1).
// ---------------------------------------------------------------------------
struct FlashWaveState {
  f32x16 oacc[2];  // O^T for d 0..31 and 32..63 of query (l % 32)
  f32x16 negm;     // -b in every element
  float m;         // the reference b, log2 units
  float l;         // this half-wave's share of sum exp2(S' - b)

  __device__ __forceinline__ void init(float bound) {
#pragma unroll
    for (int i = 0; i < 16; ++i) { oacc[0][i] = 0.f; oacc[1][i] = 0.f; negm[i] = -bound; }
    m = bound;
    l = 0.f;
  }

  // One staged 64-key tile, straight-line: both halves' scores, then for each
  // half its probabilities and O^T += V^T P^T. With MASKED, mask(kb, s) applies
  // the tile's key mask and logit bias (log2 units) to half kb's scores.
  // Consecutive MFMAs share their B operand (the two key halves against one Q
  // chunk; the two d halves against one P chunk): fewer operand bits toggle
  // on a power-limited clock, and each accumulator chain keeps its order.
  template <bool MASKED, class MaskFn>
  __device__ __forceinline__ void tile(const unsigned char* stage, const TileLaneOffsets& off,
                                       const u32x4 qB[4], MaskFn&& mask) {
    f32x16 s[2];
    {
      u32x4 ka[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = ld16(stage + off.k[ks] + kb * 32 * 128);
      s[0] = mfma32(ka[0][0], qB[0], negm);
      s[1] = mfma32(ka[1][0], qB[0], negm);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
        s[0] = mfma32(ka[0][ks], qB[ks], s[0]);
        s[1] = mfma32(ka[1][ks], qB[ks], s[1]);
      }
    }
    if constexpr (MASKED) {
      mask(0, s[0]);
      mask(1, s[1]);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 va[4];
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) va[2 * db + mm] = ld16(stage + off.v_off(db, kb, mm));
      u32x4 pB[2];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = fast_exp2(s[kb][8 * mm + i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) pB[mm][j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
        l = sum_bf16x8(pB[mm], l);
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int db = 0; db < 2; ++db) oacc[db] = mfma32(va[2 * db + mm], pB[mm], oacc[db]);
    }
  }

  // Normalise and store query (l % 32)'s row (if valid); lse in natural-log units.
  __device__ __forceinline__ void finish(bf16* orow, float* lse_ptr, bool valid) {
    const int hh = (threadIdx.x & 63) >> 5;
    const float l_tot = sum_halves(l);
    const float inv = 1.f / l_tot;
    if (!valid) return;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hh;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (lse_ptr != nullptr && hh == 0) *lse_ptr = (m + __log2f(l_tot)) * 0.6931471805599453f;
  }
};

// Two 32-query halves per wave (64 queries) against the same staged tile:
// every K and V^T operand read from LDS feeds both halves' MFMAs, and the two
// halves' independent chains (one half's probabilities while the other's
// products run on the matrix core) give the scheduler work to overlap within
// the wave. Per half the arithmetic is FlashWaveState's, in the same order.
// The MFMAs go in a snake order (each shares its A or its B operand with the
// one before: fewer operand bits toggle on a power-limited clock).
struct FlashWaveState2 {
  FlashWaveState a, b;

  // Both halves start from the larger of the lane's two bounds (one register
  // vector for both: -max(b_a, b_b) is still at least each query's logits).
  __device__ __forceinline__ void init(float bound_a, float bound_b) {
    const float bound = fmaxf(bound_a, bound_b);
    a.init(bound);
    b.init(bound);
  }

  template <bool MASKED, class MaskFn>
  __device__ __forceinline__ void tile(const unsigned char* stage, const TileLaneOffsets& off,
                                       const u32x4 qa[4], const u32x4 qb[4], MaskFn&& mask) {
    f32x16 sa[2], sb[2];
    {
      u32x4 ka[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = ld16(stage + off.k[ks] + kb * 32 * 128);
      sa[0] = mfma32(ka[0][0], qa[0], a.negm);
      sa[1] = mfma32(ka[1][0], qa[0], a.negm);
      sb[1] = mfma32(ka[1][0], qb[0], a.negm);
      sb[0] = mfma32(ka[0][0], qb[0], a.negm);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
        sa[0] = mfma32(ka[0][ks], qa[ks], sa[0]);
        sa[1] = mfma32(ka[1][ks], qa[ks], sa[1]);
        sb[1] = mfma32(ka[1][ks], qb[ks], sb[1]);
        sb[0] = mfma32(ka[0][ks], qb[ks], sb[0]);
      }
    }
    if constexpr (MASKED) {
      mask(0, sa[0]);
      mask(1, sa[1]);
      mask(0, sb[0]);
      mask(1, sb[1]);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 va[4];
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) va[2 * db + mm] = ld16(stage + off.v_off(db, kb, mm));
      u32x4 pa[2], pb[2];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        float p[8], r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = fast_exp2(sa[kb][8 * mm + i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) pa[mm][j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
        a.l = sum_bf16x8(pa[mm], a.l);
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = fast_exp2(sb[kb][8 * mm + i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[mm][j] = pack_bf16x2(r[2 * j], r[2 * j + 1]);
        b.l = sum_bf16x8(pb[mm], b.l);
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        a.oacc[0] = mfma32(va[mm], pa[mm], a.oacc[0]);
        b.oacc[0] = mfma32(va[mm], pb[mm], b.oacc[0]);
        b.oacc[1] = mfma32(va[2 + mm], pb[mm], b.oacc[1]);
        a.oacc[1] = mfma32(va[2 + mm], pa[mm], a.oacc[1]);
      }
    }
  }
};

}  // namespace sga
