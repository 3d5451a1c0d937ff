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
//   K tile  64 keys x 128 B; 16-byte chunk c of key row r lives at chunk c ^ (r & 7),
//           so the 16-byte operand reads of 8 consecutive lanes (8 rows, one
//           logical chunk) cover all 32 banks.
//   V tile  64 keys x 128 B, row-major like K; chunk c of row r lives at
//           c ^ ((r & 3) << 1). The PV operand is read with the gfx950 LDS
//           transpose load (ds_read_b64_tr_b16): inside a group of 16 lanes,
//           lane j names an 8-byte piece M[j][0..3] and lane i receives
//           M[4e + i/4][i % 4] for e = 0..3. Pointing lane j at
//           V[key0 + j/4][d0 + 4 (j % 4)] hands lane i the column d0 + i for the
//           four keys key0 .. key0 + 3 -- the A-operand layout of V^T. The
//           swizzle keeps those 4 rows x 32 bytes on 32 distinct banks.
//   bias    64 floats added (log2 units) to the tile's logits when asked
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
__device__ __forceinline__ int tile_v_off(int row, int chunk) {
  return kTileKBytes + row * 128 + ((chunk ^ ((row & 3) << 1)) << 4);
}

// Write one 16-byte chunk (8 d-values) of key u's K and V rows into a stage.
__device__ __forceinline__ void tile_store_kv(unsigned char* stage, int u, int chunk,
                                             const u32x4& kw, const u32x4& vw) {
  st16(stage + tile_k_off(u, chunk), kw);
  st16(stage + tile_v_off(u, chunk), vw);
}
__device__ __forceinline__ float* tile_bias(unsigned char* stage) {
  return reinterpret_cast<float*>(stage + kTileKBytes + kTileVBytes);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// Transposing 8-byte LDS read (see the layout note above).
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
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
  uint32_t v[2];  // V rows 4 hh + (l % 16) / 4, columns 32 db + 16 ((l / 16) % 2) + 4 (l % 4);
                  // the key block 32 kb + 16 mm + 8 r adds as an immediate
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5, li = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) k[ks] = (uint32_t)tile_k_off(li, 2 * ks + hh);
    const int j = lane & 15, gd = (lane >> 4) & 1;
    const int row = 4 * hh + (j >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int byte = 2 * (db * 32 + 16 * gd + 4 * (j & 3));
      v[db] = (uint32_t)(tile_v_off(row, byte >> 4) + (byte & 15));
    }
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

  // One 64-key tile. c = log2(e)/sqrt(d). use_bias adds the stage's bias row;
  // inactive lanes (a query not attending these keys) skip the tile.
  // Operand reads are issued in batches ahead of the MFMAs that consume them;
  // the V^T operands are requested before the softmax so their LDS latency
  // hides behind it.
  __device__ __forceinline__ void step(const unsigned char* stage, const TileLaneOffsets& off,
                                       const u32x4 qB[4], float c, bool use_bias, bool active) {
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const float* bs = reinterpret_cast<const float*>(stage + kTileKBytes + kTileVBytes);

    u32x4 ka[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = ld16(stage + off.k[ks] + kb * 32 * 128);
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma32(ka[kb][ks], qB[ks], acc);
      s[kb] = acc;
    }
    // V^T operands: slots 0..3 and 4..7 of MFMA (db, kb, mm) are the keys
    // 32 kb + 16 mm + {0, 8} + 4 hh + 0..3 of column 32 db + (l % 32)
    u32x4 va[8];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const unsigned char* p = stage + off.v[db] + (kb * 32 + 16 * mm) * 128;
          const u32x2 lo = lds_read_tr16(p);
          const u32x2 hi = lds_read_tr16(p + 8 * 128);
          va[4 * db + 2 * kb + mm] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }

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
          oacc[db] = mfma32(va[4 * db + 2 * kb + mm], pB[kb][mm], oacc[db]);
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
};

}  // namespace sga
