// Host-side launch interface between the C ABI (capi.cpp) and the kernels.
// Every launcher enqueues on `stream` and returns the launch status; argument
// validation has already happened in the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace sga {

enum FlashMode { FLASH_GLOBAL = 0, FLASH_FRAME = 1, FLASH_SUBSAMPLED = 2 };

struct FlashLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* ck;  // SUBSAMPLED: compacted keys (kept part, then mean rows)
  const void* cv;  // SUBSAMPLED: compacted values, same rows
  void* o;
  float* lse;
  Geom g;
  long long n_keys;  // GLOBAL: keys in K/V
  int mode;          // FlashMode
  int mk;            // SUBSAMPLED: kept rows per frame
  int has_mean;      // SUBSAMPLED: one mean row per frame follows the kept part
  float mean_bias2;  // SUBSAMPLED: log2(#dropped) or 0
  int token_diag;    // SUBSAMPLED: 1 = the own frame is subsampled like the others (its
                     // compacted rows and mean kept); the query's own key is not added here
  int s_h, s_w;      // SUBSAMPLED, token_diag (fp32): the strides, to find dropped queries
};

// Workgroups of `kernel` (threads per workgroup, dynamic LDS bytes) that the
// current device holds resident at once: occupancy per CU times the CU count.
int resident_workgroups(const void* kernel, int threads, size_t lds);

// bf16 MFMA flash attention (flash_bf16.hip). ws holds the V^T staging of the
// values (and of the compacted values in SUBSAMPLED mode), the key-norm
// partials and the redo flags; its size is flash_bf16_workspace(p).
// flash_bf16_fits(p) is false for sizes past the kernel's 31-bit tile extents.
size_t flash_bf16_workspace(const FlashLaunch& p);
bool flash_bf16_fits(const FlashLaunch& p);
hipError_t launch_flash_bf16(const FlashLaunch& p, void* ws, hipStream_t stream);
// V^T staging (vt_prepare.hip), tile-major: head h's 64-column tile t is the
// 64 x 64 block vt[((h*(ld/64) + t)*64 + d)*64 + c] = v[key(64t + c), h, d], keys
// in segments of seg_len padded to seg_pad columns, MFMA key order in 16-column groups.
hipError_t launch_vt_prepare(const void* v, int n_heads, long long n_rows, long long seg_len,
                             long long seg_pad, long long ld, void* vt, hipStream_t stream);
// fp32 attention of the same forms (attn_f32.hip).
hipError_t launch_flash_f32(const FlashLaunch& p, hipStream_t stream);

// GSA pooling (gsa_pool.hip). is_bf16 selects the I/O dtype.
hipError_t launch_gsa_pool(const Geom& g, bool is_bf16, int include_pad, const void* q,
                           const void* k, const void* v, void* k_cmp, void* v_cmp,
                           float* k_cmp_f32, float* q_blk_f32, hipStream_t stream);

// Block-level compressed branch (gsa_pool.hip): x (n fp32, n % 8 == 0) to
// bf16; per-block outputs [N*nqb, H, d] copied to every token of the block.
hipError_t launch_cast_bf16(const float* x, void* y, long long n, hipStream_t stream);
hipError_t launch_gsa_upsample(const Geom& g, bool is_bf16, const void* o_blk, void* o,
                               hipStream_t stream);

// What the GSA selection branch always keeps (the values of the C ABI's
// SGA_KEEP_* flags): every special token; every token of reference frame 0.
constexpr int kKeepSpecial = 1;
constexpr int kKeepRefFrame = 2;

// Number of always-kept tokens: frame 0 whole (with kKeepRefFrame), then the
// special tokens of the remaining frames (with kKeepSpecial).
inline long long kept_rows(const Geom& g, int keep) {
  const bool ref = (keep & kKeepRefFrame) != 0;
  const long long specials = (keep & kKeepSpecial) ? (long long)(g.n_frames - (ref ? 1 : 0)) * g.n_special : 0;
  return (ref ? (long long)g.L : 0) + specials;
}

// GSA top-K block selection (gsa_topk.hip). Pooled keys first .. N*nb-1
// compete; idx holds global indices. ws: gsa_topk_workspace(g, top_k) bytes
// (the wide selection's per-workgroup key buffers and overflow flags; none
// for top_k <= 16).
size_t gsa_topk_workspace(const Geom& g, int top_k);
// The same with the split-fallback capacity `cap` (listed rows per head, a
// multiple of 128; launch_gsa_topk must get the same value), and the largest
// such capacity whose workspace fits `bytes` (-1: none fits).
size_t gsa_topk_workspace(const Geom& g, int top_k, int cap);
int gsa_topk_split_cap(const Geom& g, int top_k, size_t bytes);
// Probability-mean block scores (gsa_topk.hip): top-K (<= 16) per (head, query
// block) of the mean over the block's tokens of their compressed softmax
// probabilities (q bf16 [T, H, d]); keys j >= first compete, every pooled key
// normalises. ws: gsa_topk_prob_workspace(g) bytes (key planes, then the
// tokens' log-sum-exp).
size_t gsa_topk_prob_workspace(const Geom& g);
hipError_t launch_gsa_topk_prob(const Geom& g, const void* q, const float* k_cmp, int top_k, int first,
                                int32_t* idx, float* score, void* ws, hipStream_t stream);
hipError_t launch_gsa_topk(const Geom& g, const float* q_blk, const float* k_cmp, int top_k,
                           int first, int32_t* idx, float* score, void* ws, hipStream_t stream);
hipError_t launch_gsa_topk(const Geom& g, const float* q_blk, const float* k_cmp, int top_k,
                           int first, int32_t* idx, float* score, void* ws, hipStream_t stream, int cap);
// The allocation-free selection's scratch: a file-scope device array of
// kNoAllocScratchBytes per GPU (gsa_topk.hip); noalloc_scratch gives its
// device address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void** ptr);

// GSA fine attention (gsa_fine.hip); bf16 MFMA or fp32. keep: kKeep* flags.
// fp32 visits the kept tokens itself. bf16 takes them through o_init/lse_init
// (required when kept_rows(g, keep) > 0): every query's softmax starts from
// that partial result (the attention over the kept tokens, normalised, and its
// log-sum-exp) and the selected windows continue it. With kKeepRefFrame a
// window of frame 0 in idx contributes nothing (frame 0 is already counted).
// gate (nullable): write g0 * o_cmp + g1 * (the fine result) instead, with
// g = sigmoid(q . w[h]^T + b[h]) (the gated aggregation of launch_gsa_gate);
// o must not alias o_cmp.
struct FineGate {
  const void* o_cmp;
  const float* w;
  const float* b;
};
hipError_t launch_gsa_fine(const Geom& g, bool is_bf16, const void* q, const void* k,
                           const void* v, const int32_t* idx, int top_k, int keep,
                           void* o, float* lse, const bf16* o_init, const float* lse_init,
                           const FineGate* gate, hipStream_t stream);
// The kept tokens' keys and values, gathered contiguously ([kept_rows, H, d],
// in kept_rows order) for the dense kernel (gsa_fine.hip).
hipError_t launch_gather_kept(const Geom& g, int keep, const void* k, const void* v, void* k_s,
                              void* v_s, hipStream_t stream);

// GSA gate (gsa_gate.hip).
hipError_t launch_gsa_gate(const Geom& g, bool is_bf16, const void* q, const void* o_cmp,
                           const void* o_slc, const float* w, const float* b, void* o,
                           hipStream_t stream);

// AVGGT compaction (sga_compact.hip): kept part [N*mk,H,d], then mean rows [N,H,d].
hipError_t launch_sga_compact(const Geom& g, bool is_bf16, int s_h, int s_w, const void* k,
                              const void* v, void* c_k, void* c_v, hipStream_t stream);
// AVGGT token-level diagonal, bf16 (sga_compact.hip): every query whose patch
// was dropped (r % s_h or c % s_w nonzero) merges its own key/value into its
// normalised output o and log-sum-exp lse (natural log) over the rest.
hipError_t launch_sga_diag_merge(const Geom& g, int s_h, int s_w, const void* q, const void* k,
                                 const void* v, void* o, const float* lse, hipStream_t stream);

}  // namespace sga
