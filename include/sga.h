/*
 * sga.h -- C ABI of the global cross-frame attention layer on MI355X (gfx950).
 *
 * One layer of a VGGT-style multi-view reconstruction transformer in which the
 * tokens of all N frames attend to each other, in three forms:
 *   - dense softmax attention (and its per-frame variant),
 *   - Speed3R global sparse attention (GSA): pooled K/V, compressed attention,
 *     top-K block selection, fine attention on the selected blocks, a gate,
 *   - AVGGT subsampled global attention.
 *
 * Tensor layout (every Q/K/V/O argument): [rows, n_heads, head_dim], contiguous,
 * element (t, h, c) at offset (t * n_heads + h) * head_dim + c. Token order:
 * frame-major; inside a frame the n_special special tokens (camera first, then
 * registers) precede the grid_h x grid_w patches in row-major order.
 * Notation: L = n_special + grid_h * grid_w, T = n_frames * L.
 *
 * Ownership: every buffer is device memory allocated by the caller; the
 * library never allocates, frees or retains a caller pointer. Scratch space
 * comes only through an explicit workspace argument.
 * Streams: every call enqueues its kernels on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without synchronising.
 * Errors: all arguments are validated on the host before anything is
 * enqueued; on a non-OK status nothing was enqueued and sga_last_error()
 * describes the problem. A failed launch returns SGA_ERR_HIP. Pointers must
 * be 16-byte aligned. Only head_dim == 64 is supported.
 */
#ifndef SGA_H
#define SGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SGA_OK = 0,
  SGA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer     */
  SGA_ERR_UNSUPPORTED = 2, /* valid request this build does not implement    */
  SGA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  SGA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed      */
} sga_status;

typedef enum { SGA_BF16 = 0, SGA_F32 = 1 } sga_dtype;

typedef struct {
  int32_t n_frames;  /* N >= 1                                             */
  int32_t n_special; /* S special tokens per frame, 0..16                  */
  int32_t grid_h;    /* patch grid rows >= 1                               */
  int32_t grid_w;    /* patch grid columns >= 1                            */
  int32_t n_heads;   /* H >= 1                                             */
  int32_t head_dim;  /* d, must be 64                                      */
  int32_t dtype;     /* sga_dtype of Q/K/V/O and pooled K/V                */
} sga_geom;

/*
 * Dense global attention (VGG-T3 technical summary section 1; Speed3R
 * technical summary section 1; AVGGT technical summary section 1):
 *   O[t,h] = sum_u softmax_u(Q[t,h] . K[u,h] / sqrt(d)) V[u,h].
 * q, o:   [T, H, d].   k, v: [n_keys, H, d]; n_keys == 0 means T.
 * frame_local == 1 restricts the keys of a query to its own frame (the
 *   global-to-frame conversion of AVGGT section 2.2); requires n_keys == 0.
 * A nonzero n_keys with other K/V tensors serves the GSA compressed branch
 *   (Speed3R section 2.1): k, v = the pooled K/V of gsa_compress and
 *   n_keys = N * nb.
 * lse (nullable): [T, H] fp32, natural-log log-sum-exp of the scaled logits.
 * ws: scratch of sga_workspace_size(geom, SGA_OP_DENSE, n_keys, frame_local)
 *   bytes (bf16: the values staged transposed for the matrix cores; fp32: none,
 *   ws may be NULL).
 */
sga_status dense_global_attn(const sga_geom* geom, const void* q, const void* k,
                             const void* v, int64_t n_keys, int32_t frame_local,
                             void* o, float* lse, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * GSA compression (Speed3R section 2.1, compression branch): block x block
 * average pooling of K and V over the patch grid, averaging only the tokens
 * that fall inside the grid (include_pad == 0), or with the grid zero-padded
 * to whole windows (include_pad == 1: the in-grid sum over block^2; the
 * configuration's "37x37 padded to 40x40" read literally). Only block == 4 is
 * supported. The mean queries are over each block's tokens either way.
 *   nbh = ceil(grid_h/4), nbw = ceil(grid_w/4), nb = nbh*nbw,
 *   nqb = nb + (n_special > 0 ? 1 : 0).
 * Pooled key j = f*nb + by*nbw + bx covers patch rows 4by..4by+3 and columns
 * 4bx..4bx+3 of frame f. Special tokens are not pooled.
 * k_cmp, v_cmp: [N*nb, H, d] in geom->dtype (rounded once).
 * k_cmp_f32 (nullable): [N*nb, H, d] fp32 pooled keys (input of selection).
 * q_blk_f32 (nullable; needs q): [N*nqb, H, d] fp32 mean query of every query
 *   block: the windows of a frame in pooled-key order, then one block holding
 *   the frame's special tokens.
 */
sga_status gsa_compress(const sga_geom* geom, int32_t block, int32_t include_pad,
                        const void* q, const void* k, const void* v, void* k_cmp,
                        void* v_cmp, float* k_cmp_f32, float* q_blk_f32, void* stream);

/*
 * GSA compressed branch at block level (Speed3R section 2.1, compression
 * branch: the coarse results are upsampled to full resolution): the mean query
 * of every query block (q_blk_f32 of gsa_compress) attends over the N*nb
 * pooled keys/values, and every token of the block takes that output (nearest
 * upsampling). The alternative to the token-level branch, where every token's
 * own query attends (dense_global_attn with n_keys = N*nb).
 * q_blk_f32: [N*nqb, H, d] fp32. k_cmp, v_cmp: [N*nb, H, d], o_cmp: [T, H, d],
 * in geom->dtype.
 * ws: sga_workspace_size(geom, SGA_OP_POOLED, 0, 0, &bytes) bytes: the
 *   per-block outputs, and for bf16 the pooled queries in bf16 and the dense
 *   kernel's staging.
 */
sga_status gsa_compressed_pooled(const sga_geom* geom, int32_t block, const float* q_blk_f32,
                                 const void* k_cmp, const void* v_cmp, void* o_cmp, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * What the GSA selection branch always keeps (gsa_select_topk, gsa_sparse_attn):
 * SGA_KEEP_SPECIAL: every special token of every frame (the camera tokens the
 *   Speed3R VGGT adaptation keeps, Italian summary section 2; the special
 *   tokens kept in AVGGT section 2.2).
 * SGA_KEEP_REF_FRAME: every token of frame 0, VGGT's reference frame (Speed3R
 *   technical summary section 2.2, architecture adaptation: the selection
 *   branch always keeps the reference frame's information). Its pooled blocks
 *   then take no part in the top-K, which competes among the blocks of frames
 *   1..N-1 only, so no token is counted twice. Needs N >= 2.
 */
enum { SGA_KEEP_SPECIAL = 1, SGA_KEEP_REF_FRAME = 2 };

/*
 * GSA block selection (Speed3R section 2.1, selection branch; the Italian
 * summary's S_guide score matrix): per head h and query block b the score of
 * pooled key j is q_blk[b,h] . k_cmp[j,h] / sqrt(d) (the mean over the block's
 * tokens of their compressed logits); the top_k best j are kept, ties going to
 * the lower j. The score matrix is never materialised.
 * keep: SGA_KEEP_* flags; with SGA_KEEP_REF_FRAME only j >= nb compete.
 * idx:   [H, N*nqb, top_k] int32 global pooled-key indices, each row ascending.
 * score (nullable): [H, N*nqb, top_k] fp32, the score of each idx entry.
 * 1 <= top_k <= min(competing keys, 128); competing keys = N*nb, or (N-1)*nb
 * with SGA_KEEP_REF_FRAME.
 * ws: sga_workspace_size(geom, SGA_OP_TOPK, top_k, keep, &bytes) bytes: the
 *   pooled keys split into bf16 hi/lo planes (N*nb*H*256 bytes); for
 *   top_k > 16 then the candidate buffers of the threshold-and-sort selection
 *   (at most 1 GiB), a score bound and a flag byte per (head, query block).
 */
sga_status gsa_select_topk(const sga_geom* geom, int32_t block, const float* q_blk_f32,
                           const float* k_cmp_f32, int32_t top_k, int32_t keep,
                           int32_t* idx, float* score, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * gsa_select_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and errors as
 * gsa_select_topk; its scratch is a file-scope device array of
 * SGA_NOALLOC_SCRATCH_BYTES per GPU, held by the library until the process
 * ends. A problem whose selection scratch does not fit returns
 * SGA_ERR_UNSUPPORTED (for top_k <= 16 and 16 heads, up to about 20,000 pooled
 * blocks). Every call on one GPU uses that GPU's single array: calls that
 * overlap in time on the same GPU (other streams, other threads) race and
 * must be serialised by the caller. Nothing is allocated or freed.
 */
#define SGA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
sga_status gsa_select_topk_noalloc(const sga_geom* geom, int32_t block, const float* q_blk_f32,
                                   const float* k_cmp_f32, int32_t top_k, int32_t keep,
                                   int32_t* idx, float* score, void* stream);

/*
 * GSA block selection with probability-mean block scores (the alternative
 * reading of the selection branch's block score, Speed3R section 2.1: the
 * attention of the compressed branch guides the selection): the score of
 * pooled key j for query block b is the mean over b's tokens t of
 * exp(s_tj - lse_t), s_tj = q[t,h] . k_cmp[j,h] / sqrt(d), lse_t the log of
 * sum_j' exp(s_tj') over all N*nb pooled keys (also with SGA_KEEP_REF_FRAME,
 * where only j >= nb compete). The top_k best j are kept, ties going to the
 * lower j.
 * q: [T, H, d] bf16 (the token queries; bf16 only, else SGA_ERR_UNSUPPORTED).
 * k_cmp_f32, keep, idx, score: as gsa_select_topk; score holds the mean
 *   probabilities. 1 <= top_k <= min(competing keys, 16); above 16:
 *   SGA_ERR_UNSUPPORTED.
 * ws: sga_workspace_size(geom, SGA_OP_TOPK_PROB, top_k, keep, &bytes) bytes:
 *   the key planes of gsa_select_topk, then every token's log-sum-exp (fp32
 *   [T, H]).
 * Accuracy: the keys enter as bf16 hi + lo planes, so each logit is within
 *   2^-18 * sum_i |q_i k_i| / sqrt(d) of its exact value and a reported score
 *   within a relative 2^-17 * max_(t,j) sum_i |q_i k_i| / sqrt(d) (plus fp32
 *   rounding) of the exact mean probability.
 */
sga_status gsa_select_topk_probability(const sga_geom* geom, int32_t block, const void* q,
                                       const float* k_cmp_f32, int32_t top_k, int32_t keep,
                                       int32_t* idx, float* score, void* ws, size_t ws_bytes,
                                       void* stream);

/*
 * GSA fine attention (Speed3R section 2.1, selection branch): each query of
 * query block b attends to the in-grid tokens of the pooled blocks listed in
 * idx[h, b, :] plus what `keep` (SGA_KEEP_* flags) always keeps: every special
 * token of every frame and/or every token of the reference frame 0. One
 * softmax over the union.
 * idx: [H, N*nqb, top_k] int32 entries in [0, N*nb) (in [nb, N*nb) with
 *   SGA_KEEP_REF_FRAME), distinct within a row; an entry outside that range
 *   contributes nothing.
 * o_slc: [T, H, d]. lse (nullable): [T, H] fp32.
 * ws: sga_workspace_size(geom, SGA_OP_FINE, keep, 0, &bytes) bytes. bf16 with
 *   a non-empty kept set: the kept tokens' keys and values gathered
 *   contiguously, the log-sum-exp of every query over them, and the dense
 *   kernel's staging for them (the kept part runs through the dense attention
 *   kernel, the selected windows then continue its softmax). Otherwise 0
 *   bytes and ws may be NULL.
 */
sga_status gsa_sparse_attn(const sga_geom* geom, int32_t block, const void* q,
                           const void* k, const void* v, const int32_t* idx,
                           int32_t top_k, int32_t keep, void* o_slc,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * GSA gated aggregation (Speed3R section 2.1; Italian summary section 2):
 *   g = sigmoid(Q[t,h] . w_gate[h]^T + b_gate[h]) in (0,1)^2,
 *   O[t,h] = g0 * o_cmp[t,h] + g1 * o_slc[t,h].
 * w_gate: [H, 2, d] fp32, b_gate: [H, 2] fp32 (device). o may alias o_cmp or o_slc.
 */
sga_status gsa_gate(const sga_geom* geom, const void* q, const void* o_cmp,
                    const void* o_slc, const float* w_gate, const float* b_gate,
                    void* o, void* stream);

/*
 * GSA fine attention with the gated aggregation folded in (Speed3R section
 * 2.1, selection branch then gated aggregation; the single fused pass of
 * Speed3R section 2.2 takes the gate into the selection branch's epilogue):
 * O = g0 * o_cmp + g1 * (gsa_sparse_attn's result), g as in gsa_gate. The
 * fine result enters the gate unrounded, except that with a non-empty kept set
 * in bf16 the kept tokens' partial result (normalised, from the dense kernel)
 * is rounded to bf16 once before the selected windows continue its softmax,
 * exactly as in gsa_sparse_attn. Same arguments and
 * workspace as gsa_sparse_attn, plus o_cmp [T, H, d] (the compressed branch
 * output), w_gate [H, 2, d] fp32 and b_gate [H, 2] fp32; the fine branch's
 * output and log-sum-exp are not stored. o must not alias o_cmp (an error).
 */
sga_status gsa_sparse_attn_gated(const sga_geom* geom, int32_t block, const void* q,
                                 const void* k, const void* v, const int32_t* idx,
                                 int32_t top_k, int32_t keep, const void* o_cmp,
                                 const float* w_gate, const float* b_gate, void* o,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * AVGGT compaction (AVGGT section 2.2): for every frame, its special tokens and
 * its patches with r % stride_h == 0 and c % stride_w == 0 (copied exactly),
 * and -- when any patch is dropped -- one mean K / mean V over the dropped
 * patches.
 * Layout of c_k (and c_v): the kept part [N*mk, H, d] (frame-major; per frame
 * the specials, then the kept patches in row-major grid order), followed when
 * any patch is dropped by the mean part [N, H, d] (frame f's mean at row N*mk+f).
 * mk = S + ceil(gh/sh) * ceil(gw/sw). Rows: N*(mk + has_mean), in geom->dtype.
 */
sga_status sga_compact(const sga_geom* geom, int32_t stride_h, int32_t stride_w,
                       const void* k, const void* v, void* c_k, void* c_v, void* stream);

/*
 * AVGGT subsampled global attention (AVGGT section 2.2): every query is kept;
 * a query of frame f attends to every token of frame f and to the compacted
 * set of every other frame (sga_compact). mode 1 is the frame-attention
 * conversion of the early layers. mode 2 reads the kept diagonal at token
 * level: a query attends to the compacted set of every frame, its own frame
 * included, plus its own key/value when its patch was dropped. With
 * mean_log_count == 1 the mean token's logit gets log(#dropped) added.
 * ws: sga_workspace_size(geom, SGA_OP_SUBSAMPLED, stride_h, stride_w, &bytes)
 * bytes: the compacted keys and values (sga_compact layout, each region
 * rounded up to 256 bytes), then for bf16 the values staged transposed.
 */
sga_status subsampled_global_attn(const sga_geom* geom, int32_t stride_h, int32_t stride_w,
                                  int32_t mode, int32_t mean_log_count, const void* q,
                                  const void* k, const void* v, void* o, void* ws,
                                  size_t ws_bytes, void* stream);

enum { SGA_OP_SUBSAMPLED = 1, SGA_OP_DENSE = 2, SGA_OP_FINE = 3, SGA_OP_TOPK = 4, SGA_OP_POOLED = 5,
       SGA_OP_TOPK_PROB = 6 };

/* Workspace bytes an operation needs (0 if none). SGA_OP_DENSE: param0 =
 * n_keys (0 = T), param1 = frame_local. SGA_OP_SUBSAMPLED: param0, param1 =
 * stride_h, stride_w (covers every mode). SGA_OP_FINE: param0 = keep (the
 * SGA_KEEP_* flags of gsa_sparse_attn), param1 unused (0). SGA_OP_TOPK:
 * param0 = top_k, param1 = keep (as gsa_select_topk); SGA_OP_TOPK_PROB the
 * same for gsa_select_topk_probability. SGA_OP_POOLED (gsa_compressed_pooled):
 * param0 = param1 = 0. */
sga_status sga_workspace_size(const sga_geom* geom, int32_t op, int32_t param0,
                              int32_t param1, size_t* bytes);

/* Thread-local description of the last non-OK status of this thread. */
const char* sga_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t sga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGA_H */
