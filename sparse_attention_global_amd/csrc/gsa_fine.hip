// GSA fine attention (Speed3R technical summary section 2.1, selection branch):
// every query of query block b attends to the in-grid tokens of the pooled
// blocks selected for b and, when asked, to the always-kept tokens: every
// special token of every frame (the camera tokens of the VGGT adaptation in
// the Italian summary; the special tokens of AVGGT section 2.2) and every token
// of the reference frame 0 (the VGGT adaptation, Speed3R technical summary
// section 2.2).
//
// bf16: the kept tokens are the same keys for every query, so that part is
// dense attention over them: the C ABI gathers them and runs the dense
// kernel, which leaves every query's normalised partial output and its
// log-sum-exp. This kernel then starts each query's online softmax from that
// partial result (as one pre-merged key: logit = its log-sum-exp, value = its
// output) and adds the selected windows, so the result is one softmax over
// the union of the key sets.
// Work split: a workgroup of 4 waves owns 8 consecutive query blocks of one
// head; each wave owns two of them as the 32 MFMA columns (block b0 in columns
// 0..15, block b0 + 1 in columns 16..31, member m of a 4x4 window at grid
// offset (m / 4, m % 4); a specials block holds its S tokens). Each wave
// gathers its own blocks' selected tokens into a private LDS stage, packed
// without gaps: a tile takes the next selected windows whose in-grid tokens
// fit 64 keys (4 whole windows, up to 64 one-token corner windows). While one
// block's keys are processed the other block's 16 columns sit out.
#include "attn_tile.hpp"
#include "kernels.hpp"

namespace sga {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 256;
constexpr int kBlocksPerWG = 2 * kWaves;
// per wave: its LDS stage plus the token rows of the tile being gathered
constexpr int kWaveLdsBytes = kTileStageBytes + kTileKeys * 4;

struct FineArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const int32_t* idx;  // [H, N*nqb, top_k]
  bf16* o;
  float* lse;
  const bf16* o_init;     // nullable: partial result each query starts from
  const float* lse_init;  // its log-sum-exp (natural log of the scaled logits)
  const bf16* o_cmp;      // nullable: gate the result with the compressed branch
  const float* w_gate;    // [H, 2, d] with o_cmp
  const float* b_gate;    // [H, 2]
  Geom g;
  int top_k;
  int w_lo;          // first pooled window that may contribute (nb when frame 0 is kept whole)
  int n_wg_per_head;
  float c;
};

// Token row of member m (0..15) of query block b, or -1 if the slot is empty.
__device__ __forceinline__ long long block_member_row(const Geom& g, long long b, int m) {
  if (b >= (long long)g.n_frames * g.nqb) return -1;
  const int f = (int)(b / g.nqb), j = (int)(b % g.nqb);
  const long long base = (long long)f * g.L;
  if (j == g.nb) return m < g.n_special ? base + m : -1;
  const int r = 4 * (j / g.nbw) + (m >> 2), c = 4 * (j % g.nbw) + (m & 3);
  if (r >= g.grid_h || c >= g.grid_w) return -1;
  return base + g.n_special + (long long)r * g.grid_w + c;
}

// In-grid token count of pooled window w; 0 for a window index outside
// [w_lo, N*nb), which therefore selects nothing.
__device__ __forceinline__ int window_count(const Geom& g, int w_lo, int w) {
  if (w < w_lo || w >= g.n_frames * g.nb) return 0;
  const int j = w % g.nb;
  return min(4, g.grid_h - 4 * (j / g.nbw)) * min(4, g.grid_w - 4 * (j % g.nbw));
}

// Token row of the i-th in-grid token (0 <= i < window_count) of window w,
// row-major over the window's in-grid part; token rows fit 31 bits.
__device__ __forceinline__ int window_token_row(const Geom& g, int w, int i) {
  const int f = w / g.nb, j = w % g.nb;
  const int r0 = 4 * (j / g.nbw), c0 = 4 * (j % g.nbw);
  const int cc = min(4, g.grid_w - c0);
  return f * g.L + g.n_special + (r0 + i / cc) * g.grid_w + c0 + i % cc;
}

__global__ __launch_bounds__(kThreads, 2) void gsa_fine_bf16_kernel(FineArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const Geom& g = A.g;
  const int h = blockIdx.x / A.n_wg_per_head;
  const long long wg = blockIdx.x % A.n_wg_per_head;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31;
  const int side = li >> 4;  // which of the wave's two blocks owns this column
  const long long rs = (long long)g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;
  const long long n_qb = (long long)g.n_frames * g.nqb;
  const long long b_wave = wg * kBlocksPerWG + 2 * wave;

  const long long qrow = block_member_row(g, b_wave + side, li & 15);
  const bool qvalid = qrow >= 0;
  u32x4 qB[4];
  load_q_operand(A.q + (qvalid ? qrow : 0) * rs + hoff, qvalid, qB);

  WaveAttnState st;
  st.init();
  if (A.o_init != nullptr && qvalid) {
    st.init_from(A.o_init + qrow * rs + hoff, A.lse_init[qrow * g.n_heads + h]);
  }
  TileLaneOffsets off;
  off.init();
  const float c = A.c;

  // ---- each wave's selected windows, private LDS stage -----------------------
  unsigned char* my_stage = smem + wave * kWaveLdsBytes;
  int* my_rows = reinterpret_cast<int*>(my_stage + kTileStageBytes);  // a tile's token rows
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // The next tile to gather: block side gsd (0, 1) from its selected window gwn
  // on. A tile's keys and values are loaded into registers while the previous
  // tile runs; tile_n keys of side tile_sd.
  int gsd = 0, gwn = 0, tile_n = 0, tile_sd = 0;
  u32x4 kreg[4][2], vreg[4][2];
  auto gather_next = [&]() -> bool {
    while (gsd < 2) {
      const long long b = b_wave + gsd;
      if (b >= n_qb || gwn >= A.top_k) {
        ++gsd;
        gwn = 0;
        continue;
      }
      // lane l looks at selected window gwn + l; the windows whose running
      // token count stays within 64 (a prefix of the lanes) form the tile
      const int32_t* sel = A.idx + ((long long)h * n_qb + b) * A.top_k;
      const int wi = gwn + lane;
      const int w = wi < A.top_k ? sel[wi] : -1;
      const int cnt = window_count(g, A.w_lo, w);
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const int n_w = __popcll(__ballot(wi < A.top_k && incl <= kTileKeys));  // >= 1
      const int total = __shfl(incl, n_w - 1);
      gwn += n_w;
      if (total == 0) continue;
      if (lane < n_w) {
        for (int i = 0; i < cnt; ++i) my_rows[incl - cnt + i] = window_token_row(g, w, i);
      }
      wave_sync();
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        const int u = 2 * ((lane >> 3) + 8 * part);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (u + i < total) {
            const long long row = my_rows[u + i];
            kreg[part][i] = ld16(A.k + row * rs + hoff + (lane & 7) * 8);
            vreg[part][i] = ld16(A.v + row * rs + hoff + (lane & 7) * 8);
          } else {
            kreg[part][i] = u32x4{0, 0, 0, 0};
            vreg[part][i] = u32x4{0, 0, 0, 0};
          }
        }
      }
      tile_n = total;
      tile_sd = gsd;
      return true;
    }
    return false;
  };
  // gather tile t, run tile t - 1 from the stage while tile t's loads are in
  // flight, then stage tile t
  int cur_sd = 0, cur_n = 0;
  bool staged = false;
  for (;;) {
    const bool more = gather_next();
    if (staged) {
      // the stage is this wave's own: a wave-level wait and barrier suffice
      wave_sync();
      st.step(my_stage, off, qB, c, true, side == cur_sd);
      wave_sync();
    }
    if (!more) break;
    cur_sd = tile_sd;
    cur_n = tile_n;
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      const int u = 2 * ((lane >> 3) + 8 * part);
      tile_store_kv_pair(my_stage, u, lane & 7, kreg[part][0], kreg[part][1], vreg[part][0], vreg[part][1]);
      if ((lane & 7) == 0) {
        tile_bias(my_stage)[u] = u < cur_n ? 0.f : -INFINITY;
        tile_bias(my_stage)[u + 1] = u + 1 < cur_n ? 0.f : -INFINITY;
      }
    }
    staged = true;
  }

  if (A.o_cmp == nullptr) {
    st.finish(A.o + (qvalid ? qrow : 0) * rs + hoff,
              A.lse ? A.lse + (qvalid ? qrow : 0) * g.n_heads + h : nullptr, qvalid, c);
    return;
  }
  // gated aggregation (the gate of gsa_gate.hip) on the unrounded fine row:
  // the gate logits q . W[h]^T from the lane's 32 query values (d = 16 ks +
  // 8 hh + e, the Q operand), the other 32 in lane l ^ 32
  const int hh = lane >> 5;
  const float* w0 = A.w_gate + (long long)h * 2 * kHeadDim;
  const float* w1 = w0 + kHeadDim;
  float z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = 16 * ks + 8 * hh + 2 * jj;
      const float a0 = lo_bf16(qB[ks][jj]), a1 = hi_bf16(qB[ks][jj]);
      z0 = fmaf(a1, w0[d + 1], fmaf(a0, w0[d], z0));
      z1 = fmaf(a1, w1[d + 1], fmaf(a0, w1[d], z1));
    }
  z0 += __shfl_xor(z0, 32);
  z1 += __shfl_xor(z1, 32);
  const float g0 = 1.f / (1.f + expf(-(z0 + A.b_gate[2 * h])));
  const float g1 = 1.f / (1.f + expf(-(z1 + A.b_gate[2 * h + 1])));
  const long long r = qvalid ? qrow : 0;
  st.finish_mixed(A.o + r * rs + hoff, A.o_cmp + r * rs + hoff, g0, g1, qvalid);
}

// fp32 path: one thread per (query, head), exact online softmax over the same
// key set (the kept tokens, then the selected windows' in-grid tokens).
__global__ __launch_bounds__(64) void gsa_fine_f32_kernel(Geom g, const float* __restrict__ q,
                                                          const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          const int32_t* __restrict__ idx,
                                                          int top_k, int keep,
                                                          float* __restrict__ o,
                                                          float* __restrict__ lse,
                                                          const float* __restrict__ o_cmp,
                                                          const float* __restrict__ w_gate,
                                                          const float* __restrict__ b_gate) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  if (t >= g.T) return;
  const long long rs = (long long)g.n_heads * kHeadDim;
  const long long hoff = (long long)h * kHeadDim;
  const int f = (int)(t / g.L), p = (int)(t % g.L);
  long long b;
  if (p < g.n_special) {
    b = (long long)f * g.nqb + g.nb;
  } else {
    const int r = (p - g.n_special) / g.grid_w, cc = (p - g.n_special) % g.grid_w;
    b = (long long)f * g.nqb + (r >> 2) * g.nbw + (cc >> 2);
  }
  float qv[kHeadDim], acc[kHeadDim];
  const float* qp = q + t * rs + hoff;
  for (int e = 0; e < kHeadDim; ++e) { qv[e] = qp[e] * 0.125f; acc[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](long long row) {
    const float* kp = k + row * rs + hoff;
    float s = 0.f;
    for (int e = 0; e < kHeadDim; ++e) s = fmaf(qv[e], kp[e], s);
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float pe = expf(s - m_new);
    const float* vp = v + row * rs + hoff;
    for (int e = 0; e < kHeadDim; ++e) acc[e] = fmaf(acc[e], alpha, pe * vp[e]);
    l = l * alpha + pe;
    m = m_new;
  };
  const bool ref = (keep & kKeepRefFrame) != 0;
  if (ref)
    for (long long row = 0; row < g.L; ++row) visit(row);
  if (keep & kKeepSpecial)
    for (int ff = ref ? 1 : 0; ff < g.n_frames; ++ff)
      for (int s = 0; s < g.n_special; ++s) visit((long long)ff * g.L + s);
  const long long n_qb = (long long)g.n_frames * g.nqb;
  const int32_t* sel = idx + ((long long)h * n_qb + b) * top_k;
  for (int i = 0; i < top_k; ++i) {
    const int n = window_count(g, ref ? g.nb : 0, sel[i]);
    for (int j = 0; j < n; ++j) visit(window_token_row(g, sel[i], j));
  }
  float* op = o + t * rs + hoff;
  if (o_cmp != nullptr) {  // gated aggregation (the gate of gsa_gate.hip)
    const float* w0 = w_gate + (long long)h * 2 * kHeadDim;
    float z0 = 0.f, z1 = 0.f;
    for (int e = 0; e < kHeadDim; ++e) {
      z0 = fmaf(qp[e], w0[e], z0);
      z1 = fmaf(qp[e], w0[kHeadDim + e], z1);
    }
    const float g0 = 1.f / (1.f + expf(-(z0 + b_gate[2 * h])));
    const float g1 = 1.f / (1.f + expf(-(z1 + b_gate[2 * h + 1])));
    const float* cp = o_cmp + t * rs + hoff;
    for (int e = 0; e < kHeadDim; ++e) op[e] = g0 * cp[e] + g1 * (acc[e] / l);
    return;
  }
  for (int e = 0; e < kHeadDim; ++e) op[e] = acc[e] / l;
  if (lse) lse[t * g.n_heads + h] = m + logf(l);
}

// k_s[u] = k[row of kept token u], likewise v, in kept_rows order: frame 0's
// L tokens when it is kept whole, then the special tokens (u' = f' * S + s) of
// the frames after it. A thread per 16-byte chunk.
__global__ __launch_bounds__(256) void gather_kept_kernel(Geom g, long long n_ref, int f0, long long n,
                                                          const u32x4* __restrict__ k,
                                                          const u32x4* __restrict__ v,
                                                          u32x4* __restrict__ k_s,
                                                          u32x4* __restrict__ v_s) {
  const long long chunks_per_row = (long long)g.n_heads * kHeadDim / 8;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const long long u = i / chunks_per_row, ch = i % chunks_per_row;
  long long row = u;
  if (u >= n_ref) {
    const long long us = u - n_ref;
    row = (f0 + us / g.n_special) * g.L + us % g.n_special;
  }
  k_s[i] = k[row * chunks_per_row + ch];
  v_s[i] = v[row * chunks_per_row + ch];
}

}  // namespace

hipError_t launch_gather_kept(const Geom& g, int keep, const void* k, const void* v, void* k_s,
                              void* v_s, hipStream_t stream) {
  const bool ref = (keep & kKeepRefFrame) != 0;
  const long long n = kept_rows(g, keep) * g.n_heads * kHeadDim / 8;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kept_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                     ref ? (long long)g.L : 0LL, ref ? 1 : 0, n, static_cast<const u32x4*>(k),
                     static_cast<const u32x4*>(v), static_cast<u32x4*>(k_s), static_cast<u32x4*>(v_s));
  return hipGetLastError();
}

hipError_t launch_gsa_fine(const Geom& g, bool is_bf16, const void* q, const void* k,
                           const void* v, const int32_t* idx, int top_k, int keep,
                           void* o, float* lse, const bf16* o_init, const float* lse_init,
                           const FineGate* gate, hipStream_t stream) {
  if (gate != nullptr && (gate->o_cmp == nullptr || gate->w == nullptr || gate->b == nullptr))
    return hipErrorInvalidValue;
  if (!is_bf16) {
    dim3 grid((unsigned)((g.T + 63) / 64), (unsigned)g.n_heads);
    hipLaunchKernelGGL(gsa_fine_f32_kernel, grid, dim3(64), 0, stream, g,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), idx, top_k, keep,
                       static_cast<float*>(o), lse,
                       gate ? static_cast<const float*>(gate->o_cmp) : nullptr,
                       gate ? gate->w : nullptr, gate ? gate->b : nullptr);
    return hipGetLastError();
  }
  // bf16: the kept tokens come in through o_init / lse_init only
  if (kept_rows(g, keep) > 0 && (o_init == nullptr || lse_init == nullptr)) return hipErrorInvalidValue;
  FineArgs A{};
  A.q = static_cast<const bf16*>(q);
  A.k = static_cast<const bf16*>(k);
  A.v = static_cast<const bf16*>(v);
  A.idx = idx;
  A.o = static_cast<bf16*>(o);
  A.lse = lse;
  A.g = g;
  A.top_k = top_k;
  A.w_lo = (keep & kKeepRefFrame) ? g.nb : 0;
  A.o_init = o_init;
  A.lse_init = lse_init;
  if (gate != nullptr) {
    A.o_cmp = static_cast<const bf16*>(gate->o_cmp);
    A.w_gate = gate->w;
    A.b_gate = gate->b;
  }
  A.c = kLog2e / sqrtf((float)kHeadDim);
  const long long n_qb = (long long)g.n_frames * g.nqb;
  A.n_wg_per_head = (int)((n_qb + kBlocksPerWG - 1) / kBlocksPerWG);
  const long long grid = (long long)A.n_wg_per_head * g.n_heads;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gsa_fine_bf16_kernel, dim3((unsigned)grid), dim3(kThreads),
                     kWaves * kWaveLdsBytes, stream, A);
  return hipGetLastError();
}

}  // namespace sga
