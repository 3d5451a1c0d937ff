// Device-side building blocks shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sga {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// geometry (plain values copied into every kernel's arguments)
// ---------------------------------------------------------------------------
struct Geom {
  int n_frames, n_special, grid_h, grid_w, n_heads;
  int L;        // tokens per frame
  long long T;  // tokens in all frames
  int nbh, nbw, nb, nqb;  // pooled windows (4x4) per frame, query blocks per frame
};

// Row stride of a [rows, H, 64] tensor, in elements.
__device__ __forceinline__ long long row_stride(const Geom& g) { return (long long)g.n_heads * kHeadDim; }

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest-even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 x = {a, b};
  bf16x2 y = __builtin_convertvector(x, bf16x2);
  return __builtin_bit_cast(uint32_t, y);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (gfx950)
// ---------------------------------------------------------------------------
// 32x32x16 bf16 -> fp32. Operand A: lane l holds row (l % 32) and 8 k-values of
// half (l / 32); operand B: lane l holds column (l % 32) and the same 8 k slots.
// Result: lane l holds column (l % 32), rows 8*g + 4*(l/32) + r at element 4*g + r.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------
// v_permlane32_swap with both operands = x leaves every lane holding the pair
// {x[l], x[l ^ 32]}; symmetric reductions over the pair need not know which
// element is which.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// l + the sum of the 8 bf16 values packed in w (v_dot2 with (1, 1)). The lanes
// are named explicitly: indexing the vector inside an unrolled loop and
// bit-casting the element to bf16x2 miscompiles (every term read lane 0).
__device__ __forceinline__ float sum_bf16x8(const u32x4& w, float l) {
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)w.x), ones, l, false);
  l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)w.y), ones, l, false);
  l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)w.z), ones, l, false);
  l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)w.w), ones, l, false);
  return l;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 16-byte vector memory access
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------------------
// 8 consecutive elements of one head row, widened to / narrowed from fp32
// ---------------------------------------------------------------------------
template <typename T>
struct Chunk8;  // 8 consecutive elements of one head row, widened to fp32

template <>
struct Chunk8<bf16> {
  __device__ static void load(const bf16* p, float* x) {
    const u32x4 w = ld16(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = lo_bf16(w[j]);
      x[2 * j + 1] = hi_bf16(w[j]);
    }
  }
  __device__ static void store(bf16* p, const float* x) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
    st16(p, w);
  }
};

template <>
struct Chunk8<float> {
  __device__ static void load(const float* p, float* x) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b[j]; }
  }
  __device__ static void store(float* p, const float* x) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};

__device__ __forceinline__ void store_f32x8(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

}  // namespace sga
