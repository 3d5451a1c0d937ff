// V^T staging for the bf16 attention kernels: one pass that rewrites a value
// tensor [rows, H, 64] as, per head and 64-column tile, 64 rows of d holding the
// tile's keys as columns (each tile one contiguous 8 KiB block, so a tile load
// touches one or two memory pages, whatever the key count),
//   vt[((h * (ld / 64) + col / 64) * 64 + d) * 64 + col % 64] = V[key(col), h, d]
// (0 where col holds no key), in the column order the MFMA B operand wants:
// inside every 16-column group,
// column 8hh + 4a + r holds key offset 8a + 4hh + r (bits 2 and 3 swapped; the
// map is its own inverse). Keys may be grouped in segments of seg_len padded to
// seg_pad columns (seg_pad a multiple of 64), so every segment (a frame) starts
// on a 64-column boundary; unpadded staging is one segment of all rows.
//
// With V^T in this form the attention kernels move every K and V^T tile from
// HBM straight into LDS with 16-byte direct loads, no register staging and no
// in-kernel transpose.
//
// Work split: a workgroup per (head, 64-column tile): 64 keys x 128 B read
// coalesced, transposed through LDS, written as 64 rows of 128 B.
#include "common.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

__global__ __launch_bounds__(256) void vt_prepare_kernel(const bf16* __restrict__ v, int n_heads,
                                                         long long n_rows, long long seg_len,
                                                         long long seg_pad, long long ld,
                                                         bf16* __restrict__ vt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][64 + 8];  // [col][d], padded rows
  const long long n_ctiles = ld / 64;
  const int h = (int)(blockIdx.x / n_ctiles);
  const long long col0 = (blockIdx.x % n_ctiles) * 64;
  const long long rs = (long long)n_heads * kHeadDim;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int item = t + 256 * i;  // 64 columns x 8 chunks
    const int cl = item >> 3, chunk = item & 7;
    const long long col = col0 + cl;
    const long long seg = col / seg_pad;
    const int q = (int)(col % seg_pad);
    const long long p = (q & ~15) | (q & 3) | ((q & 4) << 1) | ((q & 8) >> 1);  // swap bits 2, 3
    const long long key = seg * seg_len + p;
    u32x4 w = u32x4{0, 0, 0, 0};
    if (p < seg_len && key < n_rows) w = ld16(v + key * rs + (long long)h * kHeadDim + chunk * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[cl][chunk * 8 + 2 * j] = (uint16_t)(w[j] & 0xffffu);
      tile[cl][chunk * 8 + 2 * j + 1] = (uint16_t)(w[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int item = t + 256 * i;  // 64 d-rows x 8 column chunks
    const int d = item >> 3, cc = item & 7;
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[cc * 8 + 2 * j][d] | ((uint32_t)tile[cc * 8 + 2 * j + 1][d] << 16);
    st16(vt + (((long long)h * n_ctiles + col0 / 64) * kHeadDim + d) * 64 + cc * 8, w);
  }
}

}  // namespace

hipError_t launch_vt_prepare(const void* v, int n_heads, long long n_rows, long long seg_len,
                             long long seg_pad, long long ld, void* vt, hipStream_t stream) {
  const long long blocks = (long long)n_heads * (ld / 64);
  if (blocks > 0x7fffffffLL || ld % 64 != 0 || seg_pad % 64 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vt_prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const bf16*>(v), n_heads, n_rows, seg_len, seg_pad, ld,
                     static_cast<bf16*>(vt));
  return hipGetLastError();
}

}  // namespace sga
