// C ABI of the library (include/sga.h): host-side validation, then dispatch to
// the kernel launchers. Nothing is enqueued unless every check passes; no C++
// exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/sga.h"
#include "kernels.hpp"

static_assert(SGA_KEEP_SPECIAL == sga::kKeepSpecial && SGA_KEEP_REF_FRAME == sga::kKeepRefFrame,
              "keep flags of the C ABI and the kernels agree");

namespace {

thread_local std::string g_last_error;

sga_status fail(sga_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sga_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return SGA_OK;
  return fail(SGA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr long long kMaxRows = 0x7fffffffLL;  // token and pooled-row counts fit int32

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                              \
  do {                                                                              \
    if ((p) == nullptr) return fail(SGA_ERR_INVALID_ARG, "%s must not be null", #p); \
    if (!aligned16(p)) return fail(SGA_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p); \
  } while (0)

#define REQUIRE_OPT_PTR(p)                                                          \
  do {                                                                              \
    if ((p) != nullptr && !aligned16(p))                                            \
      return fail(SGA_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p);            \
  } while (0)

// Validate a geometry and derive the kernels' view of it.
sga_status make_geom(const sga_geom* in, sga::Geom* g) {
  if (in == nullptr) return fail(SGA_ERR_INVALID_ARG, "geom must not be null");
  if (in->n_frames < 1 || in->grid_h < 1 || in->grid_w < 1 || in->n_heads < 1)
    return fail(SGA_ERR_INVALID_ARG, "n_frames, grid_h, grid_w and n_heads must be >= 1");
  if (in->n_special < 0 || in->n_special > 16)
    return fail(SGA_ERR_INVALID_ARG, "n_special must lie in [0, 16]");
  if (in->head_dim != 64) return fail(SGA_ERR_UNSUPPORTED, "head_dim %d: only 64 is supported", in->head_dim);
  if (in->dtype != SGA_BF16 && in->dtype != SGA_F32)
    return fail(SGA_ERR_INVALID_ARG, "dtype %d is neither SGA_BF16 nor SGA_F32", in->dtype);
  const long long L = (long long)in->n_special + (long long)in->grid_h * in->grid_w;
  const long long T = L * in->n_frames;
  if (L > kMaxRows || T > kMaxRows) return fail(SGA_ERR_INVALID_ARG, "token count exceeds 2^31 - 1");
  if (T * in->n_heads > (1LL << 40)) return fail(SGA_ERR_INVALID_ARG, "T * n_heads too large");
  g->n_frames = in->n_frames;
  g->n_special = in->n_special;
  g->grid_h = in->grid_h;
  g->grid_w = in->grid_w;
  g->n_heads = in->n_heads;
  g->L = (int)L;
  g->T = T;
  g->nbh = (in->grid_h + 3) / 4;
  g->nbw = (in->grid_w + 3) / 4;
  g->nb = g->nbh * g->nbw;
  g->nqb = g->nb + (in->n_special > 0 ? 1 : 0);
  if ((long long)g->nqb * in->n_frames > kMaxRows)
    return fail(SGA_ERR_INVALID_ARG, "pooled block count exceeds 2^31 - 1");
  return SGA_OK;
}

sga_status check_block(int32_t block) {
  if (block != 4) return fail(SGA_ERR_UNSUPPORTED, "block %d: only 4x4 pooling is supported", block);
  return SGA_OK;
}

sga_status check_keep(const sga::Geom& g, int32_t keep) {
  if (keep < 0 || keep > (SGA_KEEP_SPECIAL | SGA_KEEP_REF_FRAME))
    return fail(SGA_ERR_INVALID_ARG, "keep %d must be a combination of SGA_KEEP_SPECIAL and SGA_KEEP_REF_FRAME", keep);
  if ((keep & SGA_KEEP_REF_FRAME) && g.n_frames < 2)
    return fail(SGA_ERR_INVALID_ARG, "SGA_KEEP_REF_FRAME needs at least 2 frames");
  return SGA_OK;
}

// First pooled key that competes in the top-K: the reference frame's blocks
// are kept whole, so they do not compete.
int first_candidate(const sga::Geom& g, int32_t keep) { return (keep & SGA_KEEP_REF_FRAME) ? g.nb : 0; }

sga_status check_topk(const sga::Geom& g, int32_t top_k, int32_t keep) {
  if (sga_status st = check_keep(g, keep)) return st;
  const long long n_cand = (long long)g.n_frames * g.nb - first_candidate(g, keep);
  if (top_k < 1 || top_k > n_cand || top_k > 128)
    return fail(SGA_ERR_INVALID_ARG, "top_k %d must lie in [1, min(competing blocks = %lld, 128)]", top_k,
                n_cand);
  return SGA_OK;
}

// The probability-mean selection: bf16 only, top_k <= 16 (register lists).
sga_status check_topk_prob(const sga_geom* geom, const sga::Geom& g, int32_t top_k, int32_t keep) {
  if (sga_status st = check_topk(g, top_k, keep)) return st;
  if (geom->dtype != SGA_BF16)
    return fail(SGA_ERR_UNSUPPORTED, "probability-mean block scores take bf16 queries only");
  if (top_k > 16) return fail(SGA_ERR_UNSUPPORTED, "probability-mean block scores: top_k %d > 16", top_k);
  return SGA_OK;
}

// Rows per frame of the compacted set (kept part) and whether a mean row exists.
void compact_shape(const sga::Geom& g, int s_h, int s_w, int* mk, int* has_mean, int* n_drop) {
  const int kh = (g.grid_h + s_h - 1) / s_h, kw = (g.grid_w + s_w - 1) / s_w;
  *mk = g.n_special + kh * kw;
  *n_drop = g.grid_h * g.grid_w - kh * kw;
  *has_mean = *n_drop > 0 ? 1 : 0;
}

size_t elt_size(const sga_geom* g) { return g->dtype == SGA_BF16 ? 2 : 4; }

sga_status check_fits(const sga::FlashLaunch& p) {
  if (!sga::flash_bf16_fits(p))
    return fail(SGA_ERR_UNSUPPORTED, "too many keys or heads for the bf16 kernel's 31-bit tile extents");
  return SGA_OK;
}

// gsa_sparse_attn workspace (bf16 with a non-empty kept set): gathered K and V
// of the kept tokens (frame 0 whole when the reference frame is kept, then the
// special tokens of the remaining frames), the queries' log-sum-exp over them,
// the dense staging.
struct FineLayout {
  long long rows = 0;
  size_t kv = 0, lse = 0, flash = 0, total = 0;
};
// FlashLaunch of a dense_global_attn call (validated geometry and keys).
sga::FlashLaunch dense_launch(const sga::Geom& g, int64_t n_keys, int32_t frame_local) {
  sga::FlashLaunch p{};
  p.g = g;
  p.n_keys = n_keys == 0 ? g.T : n_keys;
  p.mode = frame_local ? sga::FLASH_FRAME : sga::FLASH_GLOBAL;
  return p;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

FineLayout fine_layout(const sga::Geom& g, bool bf, int keep) {
  FineLayout lay;
  lay.rows = sga::kept_rows(g, keep);
  if (!bf || lay.rows == 0) return lay;
  lay.kv = round256((size_t)lay.rows * g.n_heads * sga::kHeadDim * 2);
  lay.lse = round256((size_t)g.T * g.n_heads * sizeof(float));
  lay.flash = round256(sga::flash_bf16_workspace(dense_launch(g, lay.rows, 0)));
  lay.total = 2 * lay.kv + lay.lse + lay.flash;
  return lay;
}


// gsa_compressed_pooled workspace: (bf16) the pooled queries in bf16, the
// per-block outputs, the dense kernel's staging for the pooled keys.
struct PooledLayout {
  sga::Geom gq;  // the geometry seen by the dense kernel: one query per block
  size_t q = 0, o = 0, flash = 0, total = 0;
};
PooledLayout pooled_layout(const sga::Geom& g, bool bf) {
  PooledLayout lay;
  lay.gq = g;
  lay.gq.T = (long long)g.n_frames * g.nqb;
  const size_t elems = (size_t)lay.gq.T * g.n_heads * sga::kHeadDim;
  lay.q = bf ? round256(elems * 2) : 0;
  lay.o = round256(elems * (bf ? 2 : 4));
  lay.flash = bf ? round256(sga::flash_bf16_workspace(dense_launch(lay.gq, (long long)g.n_frames * g.nb, 0))) : 0;
  lay.total = lay.q + lay.o + lay.flash;
  return lay;
}

// Workspace layout of subsampled_global_attn (bf16 and fp32): compacted keys,
// compacted values, then (bf16) the attention kernel's V^T staging.
void subsampled_layout(const sga_geom* geom, const sga::Geom& g, int s_h, int s_w,
                              size_t* half, size_t* flash) {
  int mk, has_mean, n_drop;
  compact_shape(g, s_h, s_w, &mk, &has_mean, &n_drop);
  const size_t rows = (size_t)g.n_frames * (size_t)(mk + has_mean);
  *half = round256(rows * (size_t)g.n_heads * 64 * elt_size(geom));
  *flash = 0;
  if (geom->dtype == SGA_BF16) {
    sga::FlashLaunch p{};
    p.g = g;
    p.mode = sga::FLASH_SUBSAMPLED;
    p.mk = mk;
    p.has_mean = has_mean;
    *flash = round256(sga::flash_bf16_workspace(p));
  }
}

}  // namespace

extern "C" {

sga_status dense_global_attn(const sga_geom* geom, const void* q, const void* k, const void* v,
                             int64_t n_keys, int32_t frame_local, void* o, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  REQUIRE_OPT_PTR(lse);
  if (frame_local != 0 && frame_local != 1) return fail(SGA_ERR_INVALID_ARG, "frame_local must be 0 or 1");
  if (n_keys < 0 || n_keys > kMaxRows) return fail(SGA_ERR_INVALID_ARG, "n_keys %lld out of range", (long long)n_keys);
  if (frame_local && n_keys != 0)
    return fail(SGA_ERR_INVALID_ARG, "frame_local attention takes its keys from the frame: n_keys must be 0");
  sga::FlashLaunch p = dense_launch(g, n_keys, frame_local);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (geom->dtype != SGA_BF16) return from_hip(sga::launch_flash_f32(p, s), "dense_global_attn launch");
  if (sga_status st = check_fits(p)) return st;
  const size_t need = sga::flash_bf16_workspace(p);
  if (ws == nullptr || ws_bytes < need)
    return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? 0 : ws_bytes);
  if (!aligned16(ws)) return fail(SGA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  return from_hip(sga::launch_flash_bf16(p, ws, s), "dense_global_attn launch");
}

sga_status gsa_compress(const sga_geom* geom, int32_t block, int32_t include_pad, const void* q,
                        const void* k, const void* v, void* k_cmp, void* v_cmp, float* k_cmp_f32,
                        float* q_blk_f32, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (sga_status st = check_block(block)) return st;
  if (include_pad != 0 && include_pad != 1) return fail(SGA_ERR_INVALID_ARG, "include_pad must be 0 or 1");
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(k_cmp);
  REQUIRE_PTR(v_cmp);
  REQUIRE_OPT_PTR(k_cmp_f32);
  REQUIRE_OPT_PTR(q_blk_f32);
  if (q_blk_f32 != nullptr) REQUIRE_PTR(q);
  return from_hip(sga::launch_gsa_pool(g, geom->dtype == SGA_BF16, include_pad, q, k, v, k_cmp, v_cmp, k_cmp_f32,
                                       q_blk_f32, static_cast<hipStream_t>(stream)),
                  "gsa_compress launch");
}

sga_status gsa_compressed_pooled(const sga_geom* geom, int32_t block, const float* q_blk_f32,
                                 const void* k_cmp, const void* v_cmp, void* o_cmp, void* ws,
                                 size_t ws_bytes, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (sga_status st = check_block(block)) return st;
  REQUIRE_PTR(q_blk_f32);
  REQUIRE_PTR(k_cmp);
  REQUIRE_PTR(v_cmp);
  REQUIRE_PTR(o_cmp);
  const bool bf = geom->dtype == SGA_BF16;
  const PooledLayout lay = pooled_layout(g, bf);
  if (ws == nullptr || ws_bytes < lay.total)
    return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                ws == nullptr ? 0 : ws_bytes);
  if (!aligned16(ws)) return fail(SGA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  sga::FlashLaunch p = dense_launch(lay.gq, (long long)g.n_frames * g.nb, 0);
  unsigned char* w = static_cast<unsigned char*>(ws);
  p.q = bf ? static_cast<const void*>(w) : static_cast<const void*>(q_blk_f32);
  p.k = k_cmp;
  p.v = v_cmp;
  p.o = w + lay.q;
  if (bf) {
    if (sga_status st = check_fits(p)) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf) {
    if (hipError_t e = sga::launch_cast_bf16(q_blk_f32, w, lay.gq.T * g.n_heads * sga::kHeadDim, s))
      return from_hip(e, "gsa_compressed_pooled (cast) launch");
    if (hipError_t e = sga::launch_flash_bf16(p, w + lay.q + lay.o, s))
      return from_hip(e, "gsa_compressed_pooled (attention) launch");
  } else {
    if (hipError_t e = sga::launch_flash_f32(p, s)) return from_hip(e, "gsa_compressed_pooled (attention) launch");
  }
  return from_hip(sga::launch_gsa_upsample(g, bf, w + lay.q, o_cmp, s), "gsa_compressed_pooled (upsample) launch");
}

sga_status gsa_select_topk(const sga_geom* geom, int32_t block, const float* q_blk_f32,
                           const float* k_cmp_f32, int32_t top_k, int32_t keep, int32_t* idx,
                           float* score, void* ws, size_t ws_bytes, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (sga_status st = check_block(block)) return st;
  if (sga_status st = check_topk(g, top_k, keep)) return st;
  REQUIRE_PTR(q_blk_f32);
  REQUIRE_PTR(k_cmp_f32);
  REQUIRE_PTR(idx);
  REQUIRE_OPT_PTR(score);
  const size_t need = sga::gsa_topk_workspace(g, top_k);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? 0 : ws_bytes);
  if (need > 0 && !aligned16(ws)) return fail(SGA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  return from_hip(sga::launch_gsa_topk(g, q_blk_f32, k_cmp_f32, top_k, first_candidate(g, keep), idx,
                                       score, ws, static_cast<hipStream_t>(stream)),
                  "gsa_select_topk launch");
}

sga_status gsa_select_topk_noalloc(const sga_geom* geom, int32_t block, const float* q_blk_f32,
                                   const float* k_cmp_f32, int32_t top_k, int32_t keep, int32_t* idx,
                                   float* score, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (sga_status st = check_block(block)) return st;
  if (sga_status st = check_topk(g, top_k, keep)) return st;
  REQUIRE_PTR(q_blk_f32);
  REQUIRE_PTR(k_cmp_f32);
  REQUIRE_PTR(idx);
  REQUIRE_OPT_PTR(score);
  const int cap = sga::gsa_topk_split_cap(g, top_k, sga::kNoAllocScratchBytes);
  if (cap < 0)
    return fail(SGA_ERR_UNSUPPORTED,
                "gsa_select_topk_noalloc: the selection needs %zu bytes of scratch, more than the %zu bytes it holds",
                sga::gsa_topk_workspace(g, top_k, 0), sga::kNoAllocScratchBytes);
  void* ws = nullptr;
  if (hipError_t e = sga::noalloc_scratch(&ws)) return from_hip(e, "gsa_select_topk_noalloc scratch lookup");
  return from_hip(sga::launch_gsa_topk(g, q_blk_f32, k_cmp_f32, top_k, first_candidate(g, keep), idx, score, ws,
                                       static_cast<hipStream_t>(stream), cap),
                  "gsa_select_topk_noalloc launch");
}

// The fine branch into `out`; with gate, its gated aggregation with o_cmp.
static sga_status sparse_attn(const sga_geom* geom, int32_t block, const void* q, const void* k,
                              const void* v, const int32_t* idx, int32_t top_k, int32_t keep,
                              void* out, float* lse, const sga::FineGate* gate, void* ws,
                              size_t ws_bytes, void* stream, const char* what) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (sga_status st = check_block(block)) return st;
  if (sga_status st = check_topk(g, top_k, keep)) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(idx);
  const char* out_name = gate ? "o" : "o_slc";
  if (out == nullptr) return fail(SGA_ERR_INVALID_ARG, "%s must not be null", out_name);
  if (!aligned16(out)) return fail(SGA_ERR_INVALID_ARG, "%s must be 16-byte aligned", out_name);
  REQUIRE_OPT_PTR(lse);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = geom->dtype == SGA_BF16;
  const FineLayout lay = fine_layout(g, bf, keep);
  if (lay.total == 0)
    return from_hip(sga::launch_gsa_fine(g, bf, q, k, v, idx, top_k, keep, out, lse, nullptr, nullptr,
                                         gate, s),
                    what);
  if (ws == nullptr || ws_bytes < lay.total)
    return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                ws == nullptr ? 0 : ws_bytes);
  if (!aligned16(ws)) return fail(SGA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  // the kept tokens through the dense kernel: `out` and the log-sum-exp hold
  // that partial result, which the window kernel continues (in place)
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* k_s = w;
  void* v_s = w + lay.kv;
  float* lse_s = reinterpret_cast<float*>(w + 2 * lay.kv);
  void* flash_ws = w + 2 * lay.kv + lay.lse;
  sga::FlashLaunch p = dense_launch(g, lay.rows, 0);
  p.q = q;
  p.k = k_s;
  p.v = v_s;
  p.o = out;
  p.lse = lse_s;
  if (sga_status st = check_fits(p)) return st;
  if (hipError_t e = sga::launch_gather_kept(g, keep, k, v, k_s, v_s, s))
    return from_hip(e, "gsa_sparse_attn (kept tokens) launch");
  if (hipError_t e = sga::launch_flash_bf16(p, flash_ws, s))
    return from_hip(e, "gsa_sparse_attn (kept tokens attention) launch");
  return from_hip(sga::launch_gsa_fine(g, bf, q, k, v, idx, top_k, keep, out, lse,
                                       static_cast<const sga::bf16*>(out), lse_s, gate, s),
                  what);
}

sga_status gsa_select_topk_probability(const sga_geom* geom, int32_t block, const void* q,
                                       const float* k_cmp_f32, int32_t top_k, int32_t keep, int32_t* idx,
                                       float* score, void* ws, size_t ws_bytes, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (sga_status st = check_block(block)) return st;
  if (sga_status st = check_topk_prob(geom, g, top_k, keep)) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cmp_f32);
  REQUIRE_PTR(idx);
  REQUIRE_OPT_PTR(score);
  const size_t need = sga::gsa_topk_prob_workspace(g);
  if (ws == nullptr || ws_bytes < need)
    return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? 0 : ws_bytes);
  if (!aligned16(ws)) return fail(SGA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  return from_hip(sga::launch_gsa_topk_prob(g, q, k_cmp_f32, top_k, first_candidate(g, keep), idx, score, ws,
                                            static_cast<hipStream_t>(stream)),
                  "gsa_select_topk_probability launch");
}

sga_status gsa_sparse_attn(const sga_geom* geom, int32_t block, const void* q, const void* k,
                           const void* v, const int32_t* idx, int32_t top_k, int32_t keep,
                           void* o_slc, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return sparse_attn(geom, block, q, k, v, idx, top_k, keep, o_slc, lse, nullptr, ws, ws_bytes, stream,
                     "gsa_sparse_attn launch");
}

sga_status gsa_sparse_attn_gated(const sga_geom* geom, int32_t block, const void* q, const void* k,
                                 const void* v, const int32_t* idx, int32_t top_k, int32_t keep,
                                 const void* o_cmp, const float* w_gate, const float* b_gate, void* o,
                                 void* ws, size_t ws_bytes, void* stream) {
  REQUIRE_PTR(o_cmp);
  REQUIRE_PTR(w_gate);
  if (b_gate == nullptr) return fail(SGA_ERR_INVALID_ARG, "b_gate must not be null");
  if (o != nullptr && o == o_cmp) return fail(SGA_ERR_INVALID_ARG, "o must not alias o_cmp");
  const sga::FineGate gate{o_cmp, w_gate, b_gate};
  return sparse_attn(geom, block, q, k, v, idx, top_k, keep, o, nullptr, &gate, ws, ws_bytes, stream,
                     "gsa_sparse_attn_gated launch");
}

sga_status gsa_gate(const sga_geom* geom, const void* q, const void* o_cmp, const void* o_slc,
                    const float* w_gate, const float* b_gate, void* o, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(o_cmp);
  REQUIRE_PTR(o_slc);
  REQUIRE_PTR(w_gate);
  if (b_gate == nullptr) return fail(SGA_ERR_INVALID_ARG, "b_gate must not be null");
  REQUIRE_PTR(o);
  return from_hip(sga::launch_gsa_gate(g, geom->dtype == SGA_BF16, q, o_cmp, o_slc, w_gate, b_gate, o,
                                       static_cast<hipStream_t>(stream)),
                  "gsa_gate launch");
}

sga_status sga_compact(const sga_geom* geom, int32_t stride_h, int32_t stride_w, const void* k,
                       const void* v, void* c_k, void* c_v, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (stride_h < 1 || stride_w < 1) return fail(SGA_ERR_INVALID_ARG, "strides must be >= 1");
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(c_k);
  REQUIRE_PTR(c_v);
  return from_hip(sga::launch_sga_compact(g, geom->dtype == SGA_BF16, stride_h, stride_w, k, v, c_k, c_v,
                                          static_cast<hipStream_t>(stream)),
                  "sga_compact launch");
}

sga_status sga_workspace_size(const sga_geom* geom, int32_t op, int32_t param0, int32_t param1,
                              size_t* bytes) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  if (bytes == nullptr) return fail(SGA_ERR_INVALID_ARG, "bytes must not be null");
  if (op == SGA_OP_DENSE) {
    if (param0 < 0 || (param1 != 0 && param1 != 1) || (param1 && param0 != 0))
      return fail(SGA_ERR_INVALID_ARG, "dense workspace: n_keys >= 0, frame_local 0/1 (n_keys 0 if 1)");
    *bytes = geom->dtype == SGA_BF16 ? sga::flash_bf16_workspace(dense_launch(g, param0, param1)) : 0;
    return SGA_OK;
  }
  if (op == SGA_OP_POOLED) {
    if (param0 != 0 || param1 != 0) return fail(SGA_ERR_INVALID_ARG, "pooled workspace: param0 = param1 = 0");
    *bytes = pooled_layout(g, geom->dtype == SGA_BF16).total;
    return SGA_OK;
  }
  if (op == SGA_OP_TOPK) {
    if (sga_status st = check_topk(g, param0, param1)) return st;
    *bytes = sga::gsa_topk_workspace(g, param0);
    return SGA_OK;
  }
  if (op == SGA_OP_TOPK_PROB) {
    if (sga_status st = check_topk_prob(geom, g, param0, param1)) return st;
    *bytes = sga::gsa_topk_prob_workspace(g);
    return SGA_OK;
  }
  if (op == SGA_OP_FINE) {
    if (param1 != 0) return fail(SGA_ERR_INVALID_ARG, "fine workspace: param1 must be 0");
    if (sga_status st = check_keep(g, param0)) return st;
    *bytes = fine_layout(g, geom->dtype == SGA_BF16, param0).total;
    return SGA_OK;
  }
  if (op != SGA_OP_SUBSAMPLED) return fail(SGA_ERR_INVALID_ARG, "unknown op %d", op);
  if (param0 < 1 || param1 < 1) return fail(SGA_ERR_INVALID_ARG, "strides must be >= 1");
  size_t half, flash;
  subsampled_layout(geom, g, param0, param1, &half, &flash);
  *bytes = 2 * half + flash;
  return SGA_OK;
}

sga_status subsampled_global_attn(const sga_geom* geom, int32_t stride_h, int32_t stride_w,
                                  int32_t mode, int32_t mean_log_count, const void* q,
                                  const void* k, const void* v, void* o, void* ws,
                                  size_t ws_bytes, void* stream) {
  sga::Geom g;
  if (sga_status st = make_geom(geom, &g)) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  if (mode < 0 || mode > 2)
    return fail(SGA_ERR_INVALID_ARG, "mode must be 0 (subsampled), 1 (frame) or 2 (token diagonal)");
  if (mean_log_count != 0 && mean_log_count != 1)
    return fail(SGA_ERR_INVALID_ARG, "mean_log_count must be 0 or 1");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = geom->dtype == SGA_BF16;
  sga::FlashLaunch p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.g = g;
  if (mode == 1) {  // frame attention: the V^T staging is a prefix of the workspace
    p.mode = sga::FLASH_FRAME;
    if (!bf) return from_hip(sga::launch_flash_f32(p, s), "subsampled_global_attn (frame) launch");
    if (sga_status st = check_fits(p)) return st;
    const size_t need = sga::flash_bf16_workspace(p);
    if (ws == nullptr || ws_bytes < need)
      return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? 0 : ws_bytes);
    if (!aligned16(ws)) return fail(SGA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
    return from_hip(sga::launch_flash_bf16(p, ws, s), "subsampled_global_attn (frame) launch");
  }
  if (stride_h < 1 || stride_w < 1) return fail(SGA_ERR_INVALID_ARG, "strides must be >= 1");
  size_t need = 0;
  if (sga_status st = sga_workspace_size(geom, SGA_OP_SUBSAMPLED, stride_h, stride_w, &need)) return st;
  if (ws == nullptr || ws_bytes < need)
    return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? 0 : ws_bytes);
  if (!aligned16(ws)) return fail(SGA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  int mk, has_mean, n_drop;
  compact_shape(g, stride_h, stride_w, &mk, &has_mean, &n_drop);
  p.mode = sga::FLASH_SUBSAMPLED;
  p.mk = mk;
  p.has_mean = has_mean;
  if (bf) {
    if (sga_status st = check_fits(p)) return st;
  }
  size_t half, flash;
  subsampled_layout(geom, g, stride_h, stride_w, &half, &flash);
  unsigned char* c_k = static_cast<unsigned char*>(ws);
  unsigned char* c_v = c_k + half;
  if (hipError_t e = sga::launch_sga_compact(g, bf, stride_h, stride_w, k, v, c_k, c_v, s))
    return from_hip(e, "subsampled_global_attn (compact) launch");
  p.ck = c_k;
  p.cv = c_v;
  p.mean_bias2 = (mean_log_count && n_drop > 0) ? (float)std::log2((double)n_drop) : 0.f;
  p.token_diag = mode == 2 ? 1 : 0;
  p.s_h = stride_h;
  p.s_w = stride_w;
  if (mode == 2 && bf && n_drop > 0) {
    // the compacted sets through the attention kernel, which then leaves the
    // log-sum-exp in the part of its workspace that holds the whole frames'
    // V^T in mode 0 (unused here, and larger than T * H floats); the dropped
    // queries then merge their own key
    unsigned char* flash_ws = c_k + 2 * half;
    p.lse = reinterpret_cast<float*>(flash_ws);
    if (hipError_t e = sga::launch_flash_bf16(p, flash_ws, s))
      return from_hip(e, "subsampled_global_attn launch");
    return from_hip(sga::launch_sga_diag_merge(g, stride_h, stride_w, q, k, v, o, p.lse, s),
                    "subsampled_global_attn (diagonal) launch");
  }
  return from_hip(bf ? sga::launch_flash_bf16(p, c_k + 2 * half, s) : sga::launch_flash_f32(p, s),
                  "subsampled_global_attn launch");
}

const char* sga_last_error(void) { return g_last_error.c_str(); }

int32_t sga_version(void) { return 60200; }

}  // extern "C"
