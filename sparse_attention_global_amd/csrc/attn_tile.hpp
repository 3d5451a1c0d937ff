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
// LDS stage layout (kStageBytes):
//   K tile   64 keys x 128 B; 16-byte chunk c of key row r lives at chunk c ^ (r & 7)
//   V^T tile 64 d-rows x 128 B of keys; the keys of every 16-key group are
//            permuted (vt_pos) so that one 16-byte read returns the 8 keys a
//            lane's B slots hold; chunk x of row d lives at x ^ swz(d)
//   bias     64 floats added (log2 units) to the tile's logits when asked
// Both swizzles make the 16-byte reads of 8 consecutive lanes hit 8 distinct
// chunks (all 32 banks) and spread the transposed 2-byte V writes.
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
  return d * 128 + (((pos >> 3) ^ swz) << 4) + ((pos & 7) << 1);
}
// Column of key offset u (0..63) inside a V^T row: within each 16-key group the
// offset 8a + 4hh + r moves to 8hh + 4a + r.
__device__ __forceinline__ int tile_vt_pos(int u) {
  const int o = u & 15;
  const int a = o >> 3, hh = (o >> 2) & 1, r = o & 3;
  return (u & ~15) | (hh << 3) | (a << 2) | r;
}

// Write one 16-byte chunk (8 d-values) of key u's K and V rows into a stage.
__device__ __forceinline__ void tile_store_kv(unsigned char* stage, int u, int chunk,
                                             const u32x4& kw, const u32x4& vw) {
  st16(stage + tile_k_off(u, chunk), kw);
  unsigned char* vs = stage + kTileKBytes;
  const int pos = tile_vt_pos(u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = chunk * 8 + 2 * j;
    *reinterpret_cast<uint16_t*>(vs + tile_vt_off(d, pos)) = (uint16_t)(vw[j] & 0xffffu);
    *reinterpret_cast<uint16_t*>(vs + tile_vt_off(d + 1, pos)) = (uint16_t)(vw[j] >> 16);
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
  __device__ __forceinline__ void step(const unsigned char* stage, const u32x4 qB[4], float c,
                                       bool use_bias, bool active) {
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5, li = lane & 31;
    const unsigned char* ks = stage;
    const unsigned char* vs = stage + kTileKBytes;
    const float* bs = reinterpret_cast<const float*>(stage + kTileKBytes + kTileVBytes);

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int kstep = 0; kstep < 4; ++kstep) {
        const u32x4 a = ld16(ks + tile_k_off(kb * 32 + li, 2 * kstep + hh));
        acc = mfma32(a, qB[kstep], acc);
      }
      s[kb] = acc;
    }
    if (use_bias) {
      const float inv_c = 1.f / c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + kb * 32 + 8 * g4 + 4 * hh);
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][4 * g4 + r] += b4[r] * inv_c;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
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
      for (int i = 0; i < 16; ++i) {
        p[i] = active ? fast_exp2(fmaf(s[kb][i], c, -mc)) : 0.f;
        l += p[i];
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pB[kb][mm][j] = pack_bf16x2(p[8 * mm + 2 * j], p[8 * mm + 2 * j + 1]);
    }

#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = db * 32 + li;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const u32x4 a = ld16(vs + tile_vt_off(d, kb * 32 + 16 * mm + 8 * hh));
          oacc[db] = mfma32(a, pB[kb][mm], oacc[db]);
        }
    }
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
