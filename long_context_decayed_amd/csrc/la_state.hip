// Chunk-parallel state passes of the gfx950 lightning-attention prefill:
// the decay-power table, pass A (per-chunk aggregates, MFMA) and pass B (the
// scan over chunks).  The blockwise scheme is described in la_output.hip.
//
// The MiniMax-M1 fact sheet (archdb), "linear / SSM layer configuration"
// field: linear attention with a fixed per-head exponential decay and a d x d
// (128 x 128) state per head.  Per (batch, head), with lam = decay[h]:
//     S_t = lam S_{t-1} + k_t^T v_t,   o_t = q_t S_t.
// A chunk c of L_c tokens hands on S_end = lam^(L_c) S_start + U_c with
// U_c = sum_s lam^(L_c-1-s) k_s^T v_s, so the chunk start states follow from
// the aggregates by a short serial scan.

#include <hip/hip_runtime.h>

#include "la_device.h"
#include "la_kernels.h"

namespace la {

// ---------------------------------------------------------------------------
// Decay-power table: tbl[h][e] = lam_h^e, e in [0, stride), computed in double
// and rounded once to float.
__global__ void la_decay_table(const float* __restrict__ decay, float* __restrict__ tbl, int stride) {
  const int h = blockIdx.x;
  const double lam = (double)decay[h];
  for (int e = threadIdx.x; e < stride; e += blockDim.x) tbl[(int64_t)h * stride + e] = (float)pow_int(lam, e);
}

// ---------------------------------------------------------------------------
// Pass A.  One workgroup per (bh, chunk); D/32 waves, wave w owns columns
// [32w, 32w + 32) of the chunk aggregate U (fp32 accumulators).  For each
// sub-tile of n valid tokens: U = lam^n U + sum_{s<n} lam^(n-1-s) k_s^T v_s.
// Operands with the token index along the contraction are read from the
// row-major LDS tiles with transpose reads.  For full sub-tiles the decay
// lam^(63-s) of token s = 16kk + 8h + i is the wave-uniform power
// lam^(55-16kk-i) times the per-half-wave power lam^(8(1-h)).
template <typename TIn, int D, bool REV>
__global__ __launch_bounds__(D * 2, sizeof(TIn) == 2 ? 3 : 1) void la_chunk_state(const TIn* __restrict__ k, const TIn* __restrict__ v,
                                                           const float* __restrict__ tbl_all,
                                                           float* __restrict__ ws, int H, int N, int L, int nc,
                                                           int tbl_stride) {
  typedef Mfma<TIn> M;
  typedef typename M::op_t op_t;
  constexpr int NW = D / 32;
  constexpr int NT = NW * 64;
  // Row stride: 32 bytes past a multiple of 128 (bf16), so the 16 lanes of a
  // transpose read (4 rows x 32 contiguous bytes) and the 8 lanes of a 16-byte
  // row store each touch 32 distinct banks.
  constexpr int PAD = sizeof(TIn) == 2 ? 16 : 4;
  constexpr int LD = D + PAD;
  constexpr int NRT = D / 32;
  __shared__ __attribute__((aligned(16))) TIn Ks[kSub * LD];
  __shared__ __attribute__((aligned(16))) TIn Vs[kSub * LD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5;
  const int bh = blockIdx.x / nc, c = blockIdx.x - (blockIdx.x / nc) * nc;
  const int hh = bh % H;
  constexpr int RS = REV ? -D : D;  // elements from one token's row to the next (REV: rows last first)
  const int64_t base = (int64_t)bh * N * D + (REV ? (int64_t)(N - 1) * D : 0);
  const TIn* kb = k + base;
  const TIn* vb = v + base;
  const int t_begin = c * L;
  const int t_end = min(N, t_begin + L);
  const float* tb = tbl_all + (int64_t)hh * tbl_stride;  // lam^e, e <= 64
  const float lane_f = tb[8 * (1 - hf)];

  f32x16 U[NRT];
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt) U[kt] = zero16();

  RowTile<TIn, D, NT> pk, pv;
  pk.template load<RS>(kb, t_begin, t_end, tid);
  pv.template load<RS>(vb, t_begin, t_end, tid);
  for (int t0 = t_begin; t0 < t_end; t0 += kSub) {
    const int n = min(kSub, t_end - t0);
    pk.template store<LD>(Ks, tid);
    pv.template store<LD>(Vs, tid);
    __syncthreads();
    if (t0 + kSub < t_end) {  // next sub-tile's loads overlap this one's MFMAs
      pk.template load<RS>(kb, t0 + kSub, t_end, tid);
      pv.template load<RS>(vb, t0 + kSub, t_end, tid);
    }
    const float dn = tb[n];
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt) U[kt] *= dn;
    const bool full = n == kSub;
#pragma unroll
    for (int kk = 0; kk < kSub / M::KW; ++kk) {
      const op_t vraw = M::ld_tr_nat(Vs, LD, M::KW * kk, 32 * w, lane);
      float x[M::EPL];
#pragma unroll
      for (int i = 0; i < M::EPL; ++i) {
        float dec;
        if (M::EPL == 8 && full) {
          dec = tb[55 - 16 * kk - i] * lane_f;
        } else {
          const int s = M::KW * kk + M::EPL * hf + i;
          dec = (s < n) ? tb[max(n - 1 - s, 0)] : 0.0f;
        }
        x[i] = M::to_f32(M::elem(vraw, i)) * dec;
      }
      op_t bhi, blo;
      M::split(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        const op_t a = M::ld_tr_nat(Ks, LD, M::KW * kk, 32 * kt, lane);
        U[kt] = M::mma(a, bhi, U[kt]);
        if (M::kSplit) U[kt] = M::mma(a, blo, U[kt]);
      }
    }
    __syncthreads();
  }

  float* dst = ws + ((int64_t)bh * nc + c) * D * D + 32 * w + (lane & 31);
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
    for (int j = 0; j < 16; ++j) dst[(32 * kt + crow(j, hf)) * D] = U[kt][j];
}

// ---------------------------------------------------------------------------
// Pass A, bf16 inputs: the fast path.  Same aggregate, organised like the
// block-64 output kernel: wave w owns columns [32w, 32w + 32) of U, the K and
// V sub-tiles arrive by 16-byte LDS DMA into swizzled tiles, double-buffered
// so that the next sub-tile's transfer overlaps this one's MFMAs (one
// barrier per sub-tile), and the sub-tiles are taken from the last to the
// first.  In that order the decay of token s of a full sub-tile b,
// lam^(L_c - 1 - (64b + s)) = lam^(L_c - 64(b+1)) lam^(63 - s), is a
// sub-tile scalar u_b (kept in double, u_(b-1) = u_b lam^64) times the
// per-token power, so U is never rescaled.  Only the last sub-tile of the
// sequence can be partial (n < 64 tokens, factors lam^(n-1-s)); it comes
// first and then sets u to lam^n.
//   Token s = trbase(kk) + trow(i, h) of a full sub-tile (the row order of
// the transpose-read operands): lam^(63-s) u = ul[i] * (lam^(56-trbase(kk)-
// 16(i>>2)) u) with the per-lane ul[i] = lam^(7 - 4h - (i & 3)).
//   With skip_decaying set, heads that decay within their chunk return at
// once: the warm-start output pass needs no aggregates.  With `only`, just
// the heads whose flag is set run (their warm start failed its check).  REV reads the
// tokens last first (token t of the pass is row N-1-t), for the reverse-time
// passes of the backward; the aggregates start from zero either way.  SILU:
// k and v are pre-activations, given SiLU in LDS as each tile arrives (as in
// the output pass).
//   UNIT: lam = 1 (plain causal linear attention): every factor is 1, so V
// enters the MFMA as the bf16 input itself (one MFMA per step instead of the
// hi + lo pair), the same values as the general path gives there.
template <int D, bool REV, bool SILU, bool UNIT>
__device__ __forceinline__ void chunk_state64_body(bf16 (*Ks)[kSub * D], bf16 (*Vs)[kSub * D],
                                                   const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                   const float* __restrict__ decay, const float* __restrict__ tbl_all,
                                                   float* __restrict__ ws, int H, int N, int L, int nc,
                                                   int tbl_stride) {
  typedef Mfma<bf16> M;
  typedef M::op_t op_t;
  constexpr int NW = D / 32;
  constexpr int NRT = D / 32;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int bh = blockIdx.x / nc, c = blockIdx.x - (blockIdx.x / nc) * nc;
  const int hh = bh % H;
  constexpr int RS = REV ? -D : D;  // elements from one token's row to the next
  const int64_t base = (int64_t)bh * N * D + (REV ? (int64_t)(N - 1) * D : 0);
  const bf16* kb = k + base;
  const bf16* vb = v + base;
  const int t_begin = c * L;
  const int lc = min(N, t_begin + L) - t_begin;  // tokens in this chunk, >= 1
  const float* tb = tbl_all + (int64_t)hh * tbl_stride;  // lam^e, e <= 64

  float ul[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ul[i] = tb[7 - 4 * hf - (i & 3)];
  const double lam = (double)decay[hh];
  const double lam64 = pow_int(lam, kSub);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the factors are in registers before any transfer

  f32x16 U[NRT];
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt) U[kt] = zero16();

  const int nsub = (lc + kSub - 1) / kSub;
  const int n_last = lc - (nsub - 1) * kSub;  // 1..64
  {
    const int64_t off = (int64_t)(t_begin + (nsub - 1) * kSub) * RS;
    dma_tile<D, NW, RS>(kb + off, Ks[0], n_last, w, lane);
    dma_tile<D, NW, RS>(vb + off, Vs[0], n_last, w, lane);
  }
  double ud = 1.0;  // u_b of the next full sub-tile
  int b = nsub - 1, cur = 0;
  if (n_last < kSub) {
    // The partial last sub-tile (peeled, so the main loop has one path):
    // tokens s < n_last get lam^(n_last-1-s), the rest 0.
    if constexpr (SILU) {
      wait_vmem<0>();
      silu_own<D, NW>(Ks[0], n_last, w, lane);
      silu_own<D, NW>(Vs[0], n_last, w, lane);
    }
    sync_lds_after_vmem<0>();
    if (b > 0) {
      const int64_t off = (int64_t)(t_begin + (b - 1) * kSub) * RS;
      dma_tile<D, NW, RS>(kb + off, Ks[1], kSub, w, lane);
      dma_tile<D, NW, RS>(vb + off, Vs[1], kSub, w, lane);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const op_t vraw = ld_tr8<D, false>(Vs[0], trbase(kk), 32 * w, lane);
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int s = trbase(kk) + trow(i, hf);
        x[i] = s < n_last ? (float)vraw[i] * tb[max(n_last - 1 - s, 0)] : 0.0f;
      }
      op_t bhi, blo;
      M::split(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        const op_t a = ld_tr8<D, false>(Ks[0], trbase(kk), 32 * kt, lane);
        U[kt] = M::mma(a, bhi, U[kt]);
        U[kt] = M::mma(a, blo, U[kt]);
      }
    }
    ud = pow_int(lam, n_last);
    --b;
    cur = 1;
  }
  for (; b >= 0; --b, cur ^= 1) {
    // Sub-tile b (full) is in buffer cur and visible; every wave is done
    // with the other buffer, which now receives sub-tile b - 1.
    if constexpr (SILU) {
      wait_vmem<0>();
      silu_own<D, NW>(Ks[cur], kSub, w, lane);
      silu_own<D, NW>(Vs[cur], kSub, w, lane);
    }
    sync_lds_after_vmem<0>();
    if (b > 0) {
      const int64_t off = (int64_t)(t_begin + (b - 1) * kSub) * RS;
      dma_tile<D, NW, RS>(kb + off, Ks[cur ^ 1], kSub, w, lane);
      dma_tile<D, NW, RS>(vb + off, Vs[cur ^ 1], kSub, w, lane);
    }
    const bf16* Kc = Ks[cur];
    const bf16* Vc = Vs[cur];
    if constexpr (UNIT) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const op_t vraw = ld_tr8<D, false>(Vc, trbase(kk), 32 * w, lane);
#pragma unroll
        for (int kt = 0; kt < NRT; ++kt) U[kt] = M::mma(ld_tr8<D, false>(Kc, trbase(kk), 32 * kt, lane), vraw, U[kt]);
      }
      continue;
    }
    const float u = (float)ud;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const op_t vraw = ld_tr8<D, false>(Vc, trbase(kk), 32 * w, lane);
      const float wk0 = tb[56 - trbase(kk)] * u, wk1 = tb[40 - trbase(kk)] * u;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)vraw[i] * ul[i] * (i < 4 ? wk0 : wk1);
      op_t bhi, blo;
      M::split(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        const op_t a = ld_tr8<D, false>(Kc, trbase(kk), 32 * kt, lane);
        U[kt] = M::mma(a, bhi, U[kt]);
        U[kt] = M::mma(a, blo, U[kt]);
      }
    }
    ud *= lam64;
  }

  // U tile kt, register j of lane (h, l): row 32kt + crow(j, h), column 32w + l.
  float* dst = ws + ((int64_t)bh * nc + c) * D * D + 32 * w + l32;
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
    for (int j = 0; j < 16; ++j) dst[(32 * kt + crow(j, hf)) * D] = U[kt][j];
}

template <int D, bool REV, bool SILU>
__global__ __launch_bounds__(D * 2, 2) void la_chunk_state64(const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                             const float* __restrict__ decay,
                                                             const float* __restrict__ tbl_all, float* __restrict__ ws,
                                                             int H, int N, int L, int nc, int tbl_stride,
                                                             int skip_decaying, int Lw, const int* __restrict__ only) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][kSub * D];
  const int bh = blockIdx.x / nc;
  const float lam = decay[bh % H];
  if (only) {
    if (!only[bh]) return;  // the exact path for the heads whose warm start failed its check
  } else if (skip_decaying && decays_within_chunk(carry_span(lam), Lw)) {
    return;  // judged by the warm chunk
  }
  if (lam == 1.0f)
    chunk_state64_body<D, REV, SILU, true>(Ks, Vs, k, v, decay, tbl_all, ws, H, N, L, nc, tbl_stride);
  else
    chunk_state64_body<D, REV, SILU, false>(Ks, Vs, k, v, decay, tbl_all, ws, H, N, L, nc, tbl_stride);
}

// ---------------------------------------------------------------------------
// Pass B.  One thread per 4 consecutive state elements of one (bh); serial
// over chunks.  ws holds U_c on entry and Sstart_c on exit.  With warm set,
// a head that decays within its chunk has its final state in its last
// chunk's slot already (warm-start pass), which is only copied to kv_out.
// With undecayed set, kv_in enters the first token without decay (chunk 0
// hands on lam^(L_0 - 1) kv_in + U_0); with scale_out, kv_out receives lam
// times the final state (the backward's gradient of the initial state).
// part: 0 every head; 1 only the heads that do not decay within their chunk
// (the scan proper); 2 only the decaying heads' copy (after their pass),
// except those whose flag is set; 3 the scan proper of the flagged heads
// only (their warm start failed its check: the exact path).
__global__ __launch_bounds__(256) void la_chunk_scan(const float* __restrict__ decay, float* __restrict__ ws,
                                                     const float* __restrict__ kv_in, float* __restrict__ kv_out,
                                                     int BH, int H, int N, int L, int nc, int D, int warm,
                                                     int undecayed, int scale_out, const int* __restrict__ slots,
                                                     int64_t num_slots, int Lw, int part,
                                                     const int* __restrict__ flags) {
  const int per = D * D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)BH * per) return;
  const int bh = (int)(gid / per), e4 = (int)(gid - (int64_t)bh * per);
  const int64_t srow = state_row(bh, H, slots, num_slots);  // kv_in / kv_out row; -1: none
  if (srow < 0) {
    kv_in = nullptr;
    kv_out = nullptr;
  }
  const float out_f = scale_out ? decay[bh % H] : 1.0f;
  const bool flagged = flags && flags[bh];
  if (part == 3 && !flagged) return;
  if (part != 3 && warm && decays_within_chunk(carry_span(decay[bh % H]), Lw)) {  // judged by the warm chunk
    if (kv_out && part != 1 && !flagged)
      reinterpret_cast<f32x4*>(kv_out)[srow * per + e4] =
          out_f * reinterpret_cast<const f32x4*>(ws)[((int64_t)bh * nc + nc - 1) * per + e4];
    return;
  }
  if (part == 2) return;
  const double lam = (double)decay[bh % H];
  const float dl = (float)pow_int(lam, L);
  const float dlast = (float)pow_int(lam, N - (nc - 1) * L);
  // chunk 0's factor on the state it receives (one power less when undecayed)
  const float d0 = (float)pow_int(lam, (nc == 1 ? N : L) - (undecayed ? 1 : 0));
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
  if (kv_in) S = reinterpret_cast<const f32x4*>(kv_in)[srow * per + e4];
  f32x4* U = reinterpret_cast<f32x4*>(ws) + (int64_t)bh * nc * per + e4;
  int c = 0;
  for (; c + 4 <= nc; c += 4) {
    f32x4 u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = U[(int64_t)(c + i) * per];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      U[(int64_t)(c + i) * per] = S;
      const float f = (c + i == 0) ? d0 : (c + i == nc - 1) ? dlast : dl;
      S = f * S + u[i];
    }
  }
  for (; c < nc; ++c) {
    const f32x4 u = U[(int64_t)c * per];
    U[(int64_t)c * per] = S;
    const float f = (c == 0) ? d0 : (c == nc - 1) ? dlast : dl;
    S = f * S + u;
  }
  if (kv_out) reinterpret_cast<f32x4*>(kv_out)[srow * per + e4] = out_f * S;
}

// ---------------------------------------------------------------------------
// The warm-start check.  Chunk c > 0 of a decaying head starts from W_c, the
// state its warm-up window of span tokens builds from zero, and leaves out
// lam^span X_c, X_c the state just before that window (computed by chunk
// c - 1, which passes that token).  Both enter every row t of the chunk
// with the same factor lam^(t - c0 + 1), so the omission is below the
// rounding of the carried term when lam^span max|X_c| <= 2^-24 max|W_c| (the
// largest entries; each row's error then stays under 2^-24 sum_j |q_j| max|W|,
// the fp32 rounding bound of q W itself).  On the workloads' inputs the ratio
// is about lam^span <= 2^-30; a state 2^6 times larger than the window's own
// (a burst of large keys and values just before a window, or a window of
// zeros) fails it, and the head is then run on the exact path.  lam = 0 has
// span 0 and omits nothing.  NaN or inf in either fails the check.  One wave
// per bh; every flag is written.
//   The same workgroup then hands on the head's final state, which the
// warm-start pass left in the head's last chunk slot of ws: copied to kv_out
// (times lam with scale_out, the backward's initial-state gradient) for a
// decaying head that passed the check.  A flagged head's final state comes
// from its exact re-run; the other heads' from the scan.
__global__ __launch_bounds__(256) void la_warm_guard(const float* __restrict__ decay, const float* __restrict__ guard,
                                                     int* __restrict__ flags, int H, int ncw, int Lw, int nw,
                                                     const float* __restrict__ ws, float* __restrict__ kv_out, int nc,
                                                     int D, int scale_out, const int* __restrict__ slots,
                                                     int64_t num_slots) {
  __shared__ int bad_s;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const float lam = decay[bh % H];
  const int span = carry_span(lam);
  const bool warm = decays_within_chunk(span, Lw);
  if (tid < 64) {
    bool bad = false;
    if (span > 0 && warm) {
      const double f = pow_int((double)lam, span);
      for (int c = 1 + lane; c < ncw; c += 64) {
        const float* xs = guard + ((int64_t)bh * ncw + c - 1) * kGuardSlots;
        const float* wsl = guard + ((int64_t)bh * ncw + c) * kGuardSlots + 4;
        float x = 0.0f, wv = 0.0f;
        for (int w = 0; w < nw; ++w) {  // as bit patterns: a NaN stays the largest
          x = __uint_as_float(max(__float_as_uint(x), __float_as_uint(xs[w])));
          wv = __uint_as_float(max(__float_as_uint(wv), __float_as_uint(wsl[w])));
        }
        if (!((double)x * f <= 0x1p-24 * (double)wv)) bad = true;
      }
    }
    bad = __any(bad);
    if (lane == 0) {
      flags[bh] = bad ? 1 : 0;
      bad_s = bad ? 1 : 0;
    }
  }
  __syncthreads();
  if (!warm || bad_s || !kv_out) return;
  const int64_t srow = state_row(bh, H, slots, num_slots);
  if (srow < 0) return;  // a slot out of range keeps no final state
  const float out_f = scale_out ? lam : 1.0f;
  const int per = D * D / 4;
  const f32x4* src = reinterpret_cast<const f32x4*>(ws) + ((int64_t)bh * nc + nc - 1) * per;
  f32x4* dst = reinterpret_cast<f32x4*>(kv_out) + srow * per;
  for (int e = tid; e < per; e += 256) dst[e] = out_f * src[e];
}

hipError_t launch_warm_guard(const PrefillArgs& a, hipStream_t st) {
  if (!a.guard || !a.flags || !a.warm_start) return hipErrorInvalidValue;
  hipLaunchKernelGGL(la_warm_guard, dim3((unsigned)(a.B * a.H)), dim3(256), 0, st, a.decay, (const float*)a.guard,
                     a.flags, (int)a.H, a.nc_warm, (int)a.L_warm, (int)(a.d / 32), (const float*)a.states, a.kv_out,
                     a.nc, (int)a.d, a.scale_kv_out ? 1 : 0, a.slots, a.num_slots);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dst[bh] = src[bh]^T for BH fp32 d x d states (the backward passes take the
// transposed initial state and final-state gradient).  One thread per
// element; writes are contiguous.
__global__ __launch_bounds__(256) void la_transpose_states(const float* __restrict__ src, float* __restrict__ dst,
                                                           int64_t BH, int D) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)D * D;
  if (gid >= BH * per) return;
  const int64_t bh = gid / per;
  const int e = (int)(gid - bh * per), i = e / D, j = e - (e / D) * D;
  dst[gid] = src[bh * per + (int64_t)j * D + i];
}

hipError_t launch_transpose_states(const float* src, float* dst, int64_t BH, int64_t d, hipStream_t st) {
  const int64_t n = BH * d * d;
  hipLaunchKernelGGL(la_transpose_states, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst, BH, (int)d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side launchers on `st`: the table and pass A; pass B.

template <typename TIn, int D>
static hipError_t launch_aggregate_t(const PrefillArgs& a, hipStream_t st) {
  const int BH = (int)(a.B * a.H);
  const int nc = a.nc;
  // the exact path of heads whose warm start failed its check reuses the table
  if (!a.rerun)
    hipLaunchKernelGGL(la_decay_table, dim3((unsigned)a.H), dim3(256), 0, st, a.decay, a.tbl, a.tbl_stride);
  const int* only = a.rerun ? a.flags : nullptr;
  if constexpr (sizeof(TIn) == 2) {
    if (a.rev)  // the backward: no SiLU
      hipLaunchKernelGGL((la_chunk_state64<D, true, false>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                         (const bf16*)a.k, (const bf16*)a.v, a.decay, (const float*)a.tbl, a.states, (int)a.H,
                         (int)a.N, (int)a.L, nc, a.tbl_stride, a.warm_start ? 1 : 0, (int)a.L_warm, only);
    else if (a.silu)
      hipLaunchKernelGGL((la_chunk_state64<D, false, true>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                         (const bf16*)a.k, (const bf16*)a.v, a.decay, (const float*)a.tbl, a.states, (int)a.H,
                         (int)a.N, (int)a.L, nc, a.tbl_stride, a.warm_start ? 1 : 0, (int)a.L_warm, only);
    else
      hipLaunchKernelGGL((la_chunk_state64<D, false, false>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                         (const bf16*)a.k, (const bf16*)a.v, a.decay, (const float*)a.tbl, a.states, (int)a.H,
                         (int)a.N, (int)a.L, nc, a.tbl_stride, a.warm_start ? 1 : 0, (int)a.L_warm, only);
  } else if (a.silu || a.rerun) {
    return hipErrorInvalidValue;  // SiLU and the warm-start check: bf16 inputs only
  } else if (a.rev)
    hipLaunchKernelGGL((la_chunk_state<TIn, D, true>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st, (const TIn*)a.k,
                       (const TIn*)a.v, (const float*)a.tbl, a.states, (int)a.H, (int)a.N, (int)a.L, nc,
                       a.tbl_stride);
  else
    hipLaunchKernelGGL((la_chunk_state<TIn, D, false>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                       (const TIn*)a.k, (const TIn*)a.v, (const float*)a.tbl, a.states, (int)a.H, (int)a.N,
                       (int)a.L, nc, a.tbl_stride);
  return hipGetLastError();
}

hipError_t launch_aggregate_pass(const PrefillArgs& a, hipStream_t st) {
  if (a.in_dtype == kBF16)
    return a.d == 128 ? launch_aggregate_t<bf16, 128>(a, st) : launch_aggregate_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_aggregate_t<float, 128>(a, st) : launch_aggregate_t<float, 64>(a, st);
}

hipError_t launch_scan_pass(const PrefillArgs& a, hipStream_t st, int part) {
  const int BH = (int)(a.B * a.H);
  const int D = (int)a.d;
  const int64_t threads = (int64_t)BH * D * D / 4;
  hipLaunchKernelGGL(la_chunk_scan, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a.decay, a.states,
                     a.kv_in, a.kv_out, BH, (int)a.H, (int)a.N, (int)a.L, a.nc, D, a.warm_start ? 1 : 0,
                     a.rev ? 1 : 0, a.scale_kv_out ? 1 : 0, a.slots, a.num_slots, (int)a.L_warm, part,
                     (const int*)a.flags);
  return hipGetLastError();
}

}  // namespace la
