// Prefill kernels of causal decayed linear attention for gfx950.
//
// The MiniMax-M1 fact sheet (archdb), "linear / SSM layer configuration"
// field: linear attention with a fixed per-head exponential decay and a d x d
// (128 x 128) state per head.  Per (batch, head), with lam = decay[h]:
//     S_t = lam S_{t-1} + k_t^T v_t,   o_t = q_t S_t.
//
// Blockwise form computed here.  Tokens are split into chunks of L tokens,
// chunks into blocks of BLK tokens (L % BLK == 0, blocks aligned to chunk
// starts).  For a block starting at token t_b with start state S_b, the rows
// r of the block get
//     o_r = lam^(r+1) q_r S_b  +  sum_{s <= r in block} lam^(r-s) (q_r . k_s) v_s
// and the block hands on S_{b+1} = lam^BLK S_b + sum_s lam^(BLK-1-s) k_s^T v_s.
// Only non-negative powers of lam appear (all from the table T[e] = lam^e,
// 0 <= e <= BLK), so nothing overflows; powers that underflow are correctly 0.
//
// Three passes make long sequences fill the chip:
//   A  la_chunk_state : per chunk, its aggregate U_c = sum_s lam^(L_c-1-s) k_s^T v_s,
//                       all chunks in parallel (MFMA);
//   B  la_chunk_scan  : per (batch, head), S <- kv_in; for c: Sstart_c = S,
//                       S = lam^(L_c) S + U_c; kv_out = S (elementwise, fp32);
//   C  la_chunk_output: per chunk, the block loop above from Sstart_c (MFMA).
//
// Precision recipe (bf16 inputs): products of two bf16 inputs are exact in the
// fp32 MFMA accumulator.  Quantities formed in fp32 that feed an MFMA are
// rounded: the masked, decayed scores P (one bf16), the state S used in q S
// and the decayed values lam^(..) v used in the state update (both as a bf16
// hi + lo pair, ~16 significant bits).  Accumulation is fp32 throughout and
// the state stays fp32.

#include <hip/hip_runtime.h>

#include "la_device.h"
#include "la_kernels.h"

namespace la {

constexpr int kSub = 64;  // rows per sub-tile (one LDS stage)

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
// The next sub-tile's K and V are loaded into registers while the current
// one is contracted; operands with the token index along the contraction are
// read from the row-major LDS tiles with transpose reads.
template <typename TIn, int D>
__global__ __launch_bounds__(D * 2) void la_chunk_state(const TIn* __restrict__ k, const TIn* __restrict__ v,
                                                        const float* __restrict__ tbl_all, float* __restrict__ ws,
                                                        int H, int N, int L, int nc, int tbl_stride) {
  typedef Mfma<TIn> M;
  typedef typename M::op_t op_t;
  constexpr int NW = D / 32;
  constexpr int NT = NW * 64;
  constexpr int PAD = 16 / sizeof(TIn);
  constexpr int LD = D + PAD;
  constexpr int NRT = D / 32;
  __shared__ __attribute__((aligned(16))) TIn Ks[kSub * LD];
  __shared__ __attribute__((aligned(16))) TIn Vs[kSub * LD];
  __shared__ float tbl[kSub + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5;
  const int bh = blockIdx.x / nc, c = blockIdx.x - (blockIdx.x / nc) * nc;
  const int hh = bh % H;
  const int64_t base = (int64_t)bh * N * D;
  const TIn* kb = k + base;
  const TIn* vb = v + base;
  const int t_begin = c * L;
  const int t_end = min(N, t_begin + L);

  for (int e = tid; e <= kSub; e += NT) tbl[e] = tbl_all[(int64_t)hh * tbl_stride + e];

  f32x16 U[NRT];
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt) U[kt] = zero16();

  RowTile<TIn, D, NT> pk, pv;
  pk.load(kb, t_begin, t_end, tid);
  pv.load(vb, t_begin, t_end, tid);
  for (int t0 = t_begin; t0 < t_end; t0 += kSub) {
    const int n = min(kSub, t_end - t0);
    pk.template store<LD>(Ks, tid);
    pv.template store<LD>(Vs, tid);
    __syncthreads();
    if (t0 + kSub < t_end) {
      pk.load(kb, t0 + kSub, t_end, tid);
      pv.load(vb, t0 + kSub, t_end, tid);
    }
    const float dn = tbl[n];
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt) U[kt] *= dn;
#pragma unroll
    for (int kk = 0; kk < kSub / M::KW; ++kk) {
      // B operand: lam^(n-1-s) v[s][32w + n'] for s = KW*kk + EPL*hf + i.
      const op_t vraw = M::ld_tr_nat(Vs, LD, M::KW * kk, 32 * w, lane);
      float x[M::EPL];
#pragma unroll
      for (int i = 0; i < M::EPL; ++i) {
        const int s = M::KW * kk + M::EPL * hf + i;
        const float dec = (s < n) ? tbl[max(n - 1 - s, 0)] : 0.0f;
        x[i] = M::to_f32(M::elem(vraw, i)) * dec;
      }
      op_t bhi, blo;
      M::split(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        // A operand: K^T[dk = 32kt + n'][s]
        const op_t a = M::ld_tr_nat(Ks, LD, M::KW * kk, 32 * kt, lane);
        U[kt] = M::mma(a, bhi, U[kt]);
        if (M::kSplit) U[kt] = M::mma(a, blo, U[kt]);
      }
    }
    __syncthreads();
  }

  float* dst = ws + ((int64_t)bh * nc + c) * D * D;
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
    for (int j = 0; j < 16; ++j) dst[(32 * kt + crow(j, hf)) * D + 32 * w + (lane & 31)] = U[kt][j];
}

// ---------------------------------------------------------------------------
// Pass B.  One thread per 4 consecutive state elements of one (bh); serial
// over chunks.  ws holds U_c on entry and Sstart_c on exit.
__global__ __launch_bounds__(256) void la_chunk_scan(const float* __restrict__ decay, float* __restrict__ ws,
                                                     const float* __restrict__ kv_in, float* __restrict__ kv_out,
                                                     int BH, int H, int N, int L, int nc, int D) {
  const int per = D * D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)BH * per) return;
  const int bh = (int)(gid / per), e4 = (int)(gid - (int64_t)bh * per);
  const double lam = (double)decay[bh % H];
  const float dl = (float)pow_int(lam, L);
  const float dlast = (float)pow_int(lam, N - (nc - 1) * L);
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
  if (kv_in) S = reinterpret_cast<const f32x4*>(kv_in)[(int64_t)bh * per + e4];
  f32x4* U = reinterpret_cast<f32x4*>(ws) + (int64_t)bh * nc * per + e4;
  int c = 0;
  for (; c + 4 <= nc; c += 4) {
    f32x4 u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = U[(int64_t)(c + i) * per];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      U[(int64_t)(c + i) * per] = S;
      const float f = (c + i == nc - 1) ? dlast : dl;
      S = f * S + u[i];
    }
  }
  for (; c < nc; ++c) {
    const f32x4 u = U[(int64_t)c * per];
    U[(int64_t)c * per] = S;
    const float f = (c == nc - 1) ? dlast : dl;
    S = f * S + u;
  }
  if (kv_out) reinterpret_cast<f32x4*>(kv_out)[(int64_t)bh * per + e4] = S;
}

// ---------------------------------------------------------------------------
// Pass C.  One workgroup per (bh, chunk); D/32 waves.  Wave w owns columns
// [32w, 32w + 32) of the fp32 state S (NRT accumulator tiles) and of the
// output.  LDS: Q of the current sub-tile, K and V of every sub-tile of the
// current block (BLK/64 slots), the decay table.  The next sub-tile's Q, K, V
// are loaded into registers while the current one is computed.
//
// Per 64-row sub-tile (row r, position p = 64*jb + r in its block):
//   inter  acc = diag(lam^(p+1)) Q S_b                    (S_b as bf16 hi + lo)
//   intra  acc += (P^T)^T V, P^T = K Q^T masked by lam^(p-s) for s <= p
//   update S += sum_s lam^(BLK-1-s) k_s^T v_s               (decayed v as hi + lo)
// with S pre-decayed by lam^BLK once per block.  With BLK = 64 the state is
// split into hi/lo on the fly; with longer blocks the block-start split is
// kept in registers for the block's later sub-tiles.
template <typename TIn, typename TOut, int D, int BLK>
__global__ __launch_bounds__(D * 2, (BLK == 64 && sizeof(TIn) == 2) ? 2 : 1) void la_chunk_output(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                         const TIn* __restrict__ v, TOut* __restrict__ o,
                                                         const float* __restrict__ tbl_all,
                                                         const float* __restrict__ sstart, int H, int N, int L,
                                                         int nc, int tbl_stride) {
  typedef Mfma<TIn> M;
  typedef typename M::op_t op_t;
  constexpr int NW = D / 32;
  constexpr int NT = NW * 64;
  constexpr int PAD = 16 / sizeof(TIn);
  constexpr int LD = D + PAD;
  constexpr int NRT = D / 32;
  constexpr int NS = BLK / kSub;
  constexpr int G = 32 / M::KW;  // operand groups per 32-row accumulator tile
  constexpr int SNAP = (NS > 1) ? NRT : 1;
  __shared__ __attribute__((aligned(16))) TIn Qs[kSub * LD];
  __shared__ __attribute__((aligned(16))) TIn Ks[NS * kSub * LD];
  __shared__ __attribute__((aligned(16))) TIn Vs[NS * kSub * LD];
  __shared__ float tbl[BLK + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int bh = blockIdx.x / nc, c = blockIdx.x - (blockIdx.x / nc) * nc;
  const int hh = bh % H;
  const int64_t base = (int64_t)bh * N * D;
  const TIn* qb = q + base;
  const TIn* kb = k + base;
  const TIn* vb = v + base;
  TOut* ob = o + base;
  const int t_begin = c * L;
  const int t_end = min(N, t_begin + L);
  const int col = 32 * w + l32;  // this lane's value column

  for (int e = tid; e <= BLK; e += NT) tbl[e] = tbl_all[(int64_t)hh * tbl_stride + e];

  f32x16 S[NRT];
  {
    const float* src = sstart + ((int64_t)bh * nc + c) * D * D;
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) S[kt][j] = src[(32 * kt + crow(j, hf)) * D + col];
  }
  op_t Shi[SNAP][G], Slo[SNAP][G];

  constexpr bool kPrefetch = !(BLK == 64 && sizeof(TIn) == 2);
  RowTile<TIn, D, NT> pq, pk, pv;
  if (kPrefetch) {
    pq.load(qb, t_begin, t_end, tid);
    pk.load(kb, t_begin, t_end, tid);
    pv.load(vb, t_begin, t_end, tid);
  }

  int jb = 0;  // sub-tile index within the current block
  for (int t0 = t_begin; t0 < t_end; t0 += kSub, jb = (jb + 1 == NS) ? 0 : jb + 1) {
    TIn* Kj = Ks + jb * kSub * LD;
    TIn* Vj = Vs + jb * kSub * LD;
    if (!kPrefetch) {
      pq.load(qb, t0, t_end, tid);
      pk.load(kb, t0, t_end, tid);
      pv.load(vb, t0, t_end, tid);
    }
    pq.template store<LD>(Qs, tid);
    pk.template store<LD>(Kj, tid);
    pv.template store<LD>(Vj, tid);
    __syncthreads();
    if (kPrefetch && t0 + kSub < t_end) {
      pq.load(qb, t0 + kSub, t_end, tid);
      pk.load(kb, t0 + kSub, t_end, tid);
      pv.load(vb, t0 + kSub, t_end, tid);
    }

    // Inter-block: acc[rt] = diag(lam^(p+1)) Q S_b.
    f32x16 acc[2];
    acc[0] = zero16();
    acc[1] = zero16();
    if constexpr (NS == 1) {
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float x[M::EPL];
#pragma unroll
          for (int i = 0; i < M::EPL; ++i) x[i] = S[kt][g * M::EPL + i];
          op_t hi, lo;
          M::split(x, hi, lo);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const op_t a = M::ld_cperm(Qs + (32 * rt + l32) * LD + 32 * kt, g, hf);
            acc[rt] = M::mma(a, hi, acc[rt]);
            if (M::kSplit) acc[rt] = M::mma(a, lo, acc[rt]);
          }
        }
        S[kt] *= tbl[BLK];
      }
    } else {
      if (jb == 0) {
        // Block start: keep S_b as MFMA B operands, then pre-decay S by lam^BLK.
        const float dblk = tbl[BLK];
#pragma unroll
        for (int kt = 0; kt < SNAP; ++kt) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float x[M::EPL];
#pragma unroll
            for (int i = 0; i < M::EPL; ++i) x[i] = S[kt][g * M::EPL + i];
            M::split(x, Shi[kt][g], Slo[kt][g]);
          }
          S[kt] *= dblk;
        }
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const TIn* qrow = Qs + (32 * rt + l32) * LD;
#pragma unroll
        for (int kt = 0; kt < SNAP; ++kt) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const op_t a = M::ld_cperm(qrow + 32 * kt, g, hf);
            acc[rt] = M::mma(a, Shi[kt][g], acc[rt]);
            if (M::kSplit) acc[rt] = M::mma(a, Slo[kt][g], acc[rt]);
          }
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[rt][j] *= tbl[kSub * jb + 32 * rt + crow(j, hf) + 1];

    // Intra-block: for every earlier-or-current sub-tile jk of the block,
    // P^T = K_jk Q^T (32x32 tiles), masked and decayed by lam^(p-s), then acc += P V_jk.
    for (int jk = 0; jk <= jb; ++jk) {
      const TIn* Kk = Ks + jk * kSub * LD;
      const TIn* Vk = Vs + jk * kSub * LD;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          if (jk == jb && st > rt) continue;
          f32x16 p = zero16();
          const TIn* krow = Kk + (32 * st + l32) * LD;
          const TIn* qrow = Qs + (32 * rt + l32) * LD;
#pragma unroll
          for (int kk = 0; kk < D / M::KW; ++kk) {
            const op_t a = M::ld_nat(krow + M::KW * kk + M::EPL * hf);
            const op_t b = M::ld_nat(qrow + M::KW * kk + M::EPL * hf);
            p = M::mma(a, b, p);
          }
          // p[j] = P^T[s][r] with s = 32st + crow(j, hf), r = 32rt + l32 (tile-local).
          const int rdiff = kSub * (jb - jk) + 32 * (rt - st) + l32;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int dif = rdiff - crow(j, hf);
            p[j] = (dif >= 0) ? p[j] * tbl[dif < 0 ? 0 : dif] : 0.0f;
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float x[M::EPL];
#pragma unroll
            for (int i = 0; i < M::EPL; ++i) x[i] = p[g * M::EPL + i];
            const op_t pa = M::cvt(x);
            const op_t vop = M::ld_tr_cperm(Vk, LD, 32 * st, g, 32 * w, lane);
            acc[rt] = M::mma(pa, vop, acc[rt]);
          }
        }
      }
    }

    // State update: S += sum_s lam^(BLK-1-s) k_s^T v_s over this sub-tile
    // (S was pre-decayed by lam^BLK at the block start).
#pragma unroll
    for (int kk = 0; kk < kSub / M::KW; ++kk) {
      const op_t vraw = M::ld_tr_nat(Vj, LD, M::KW * kk, 32 * w, lane);
      float x[M::EPL];
#pragma unroll
      for (int i = 0; i < M::EPL; ++i) {
        const int s = M::KW * kk + M::EPL * hf + i;
        x[i] = M::to_f32(M::elem(vraw, i)) * tbl[BLK - 1 - (kSub * jb + s)];
      }
      op_t bhi, blo;
      M::split(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        const op_t a = M::ld_tr_nat(Kj, LD, M::KW * kk, 32 * kt, lane);
        S[kt] = M::mma(a, bhi, S[kt]);
        if (M::kSplit) S[kt] = M::mma(a, blo, S[kt]);
      }
    }

    // Store this sub-tile's rows.
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + 32 * rt + crow(j, hf);
        if (t < t_end) ob[(int64_t)t * D + col] = from_f32<TOut>(acc[rt][j]);
      }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Pass C, block = 64, bf16 inputs: the fast path.  Same arithmetic as
// la_chunk_output with BLK = 64, organised to cut per-element VALU work:
//   * the 3 masked, decayed score tiles P^T (32x32) of a sub-tile are each
//     computed by one wave and shared through LDS as ready-made bf16 MFMA A
//     operands (instead of every wave recomputing all three);
//   * the mask/decay factors of the score tiles and the row factors
//     lam^(r+1) of the inter term are per-lane tables built once in LDS;
//   * the decays lam^(63-s) of the state update are a wave-uniform power
//     times a per-half-wave power (no per-element lookups);
//   * full sub-tiles store without per-element bounds checks.
template <typename TOut, int D>
__global__ __launch_bounds__(D * 2, 2) void la_chunk_output64(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                              const bf16* __restrict__ v, TOut* __restrict__ o,
                                                              const float* __restrict__ tbl_all,
                                                              const float* __restrict__ sstart, int H, int N, int L,
                                                              int nc, int tbl_stride) {
  typedef Mfma<bf16> M;
  typedef M::op_t op_t;
  constexpr int NW = D / 32;
  constexpr int NT = NW * 64;
  constexpr int LD = D + 8;
  constexpr int NRT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Qs[kSub * LD];
  __shared__ __attribute__((aligned(16))) bf16 Ks[kSub * LD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kSub * LD];
  __shared__ __attribute__((aligned(16))) op_t Pbuf[3][2][64];     // score tiles as A operands
  __shared__ __attribute__((aligned(16))) f32x4 dP[2][4][64];      // [diag/off][j/4][lane]
  __shared__ __attribute__((aligned(16))) f32x4 dRow[2][4][64];    // [rt][j/4][lane]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int bh = blockIdx.x / nc, c = blockIdx.x - (blockIdx.x / nc) * nc;
  const int hh = bh % H;
  const int64_t base = (int64_t)bh * N * D;
  const bf16* qb = q + base;
  const bf16* kb = k + base;
  const bf16* vb = v + base;
  TOut* ob = o + base;
  const int t_begin = c * L;
  const int t_end = min(N, t_begin + L);
  const int col = 32 * w + l32;
  const float* tb = tbl_all + (int64_t)hh * tbl_stride;  // lam^e, e <= 64

  // Per-lane decay tables.
  for (int e = tid; e < 2 * 16 * 64; e += NT) {
    const int t = e >> 10, j = (e >> 6) & 15, ln = e & 63;
    const int dif = 32 * t + (ln & 31) - crow(j, ln >> 5);
    dP[t][j >> 2][ln][j & 3] = dif >= 0 ? tb[dif] : 0.0f;
    const int rt = t;
    dRow[rt][j >> 2][ln][j & 3] = tb[32 * rt + crow(j, ln >> 5) + 1];
  }
  const float lane_f = tb[8 * (1 - hf)];  // lam^(8(1-hf)): the half-wave part of lam^(63-s)
  const float d64 = tb[64];

  f32x16 S[NRT];
  {
    const float* src = sstart + ((int64_t)bh * nc + c) * D * D;
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) S[kt][j] = src[(32 * kt + crow(j, hf)) * D + col];
  }

  RowTile<bf16, D, NT> pq, pk, pv;
  for (int t0 = t_begin; t0 < t_end; t0 += kSub) {
    pq.load(qb, t0, t_end, tid);
    pk.load(kb, t0, t_end, tid);
    pv.load(vb, t0, t_end, tid);
    pq.template store<LD>(Qs, tid);
    pk.template store<LD>(Ks, tid);
    pv.template store<LD>(Vs, tid);
    __syncthreads();

    // Score tiles: tile i = (st, rt) in {(0,0), (0,1), (1,1)}, computed by wave i % NW.
    for (int ti = w; ti < 3; ti += NW) {
      const int st = ti == 2 ? 1 : 0, rt = ti == 0 ? 0 : 1;
      f32x16 p = zero16();
      const bf16* krow = Ks + (32 * st + l32) * LD + 8 * hf;
      const bf16* qrow = Qs + (32 * rt + l32) * LD + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) p = M::mma(M::ld_nat(krow + 16 * kk), M::ld_nat(qrow + 16 * kk), p);
      const int t = rt - st;
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const f32x4 f = dP[t][jq][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * jq + e] *= f[e];
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = p[8 * g + i];
        Pbuf[ti][g][lane] = M::cvt(x);
      }
    }

    // Inter-block term with S split into bf16 hi + lo on the fly; then S *= lam^64.
    f32x16 acc[2];
    acc[0] = zero16();
    acc[1] = zero16();
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = S[kt][8 * g + i];
        op_t hi, lo;
        M::split(x, hi, lo);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const op_t a = M::ld_cperm(Qs + (32 * rt + l32) * LD + 32 * kt, g, hf);
          acc[rt] = M::mma(a, hi, acc[rt]);
          acc[rt] = M::mma(a, lo, acc[rt]);
        }
      }
      S[kt] *= d64;
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const f32x4 f = dRow[rt][jq][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[rt][4 * jq + e] *= f[e];
      }
    __syncthreads();  // score tiles visible

    // Intra-block term: acc[rt] += P V over the shared score tiles.
#pragma unroll
    for (int ti = 0; ti < 3; ++ti) {
      const int st = ti == 2 ? 1 : 0, rt = ti == 0 ? 0 : 1;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const op_t vop = M::ld_tr_cperm(Vs, LD, 32 * st, g, 32 * w, lane);
        acc[rt] = M::mma(Pbuf[ti][g][lane], vop, acc[rt]);
      }
    }

    // State update: S += sum_s lam^(63-s) k_s^T v_s.
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const op_t vraw = M::ld_tr_nat(Vs, LD, 16 * kk, 32 * w, lane);
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)vraw[i] * (tb[55 - 16 * kk - i] * lane_f);
      op_t bhi, blo;
      M::split(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        const op_t a = M::ld_tr_nat(Ks, LD, 16 * kk, 32 * kt, lane);
        S[kt] = M::mma(a, bhi, S[kt]);
        S[kt] = M::mma(a, blo, S[kt]);
      }
    }

    // Store this sub-tile's rows.
    TOut* orow = ob + (int64_t)t0 * D + col;
    if (t0 + kSub <= t_end) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 16; ++j) orow[(32 * rt + crow(j, hf)) * D] = from_f32<TOut>(acc[rt][j]);
    } else {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = 32 * rt + crow(j, hf);
          if (t0 + r < t_end) orow[r * D] = from_f32<TOut>(acc[rt][j]);
        }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers.

template <typename TIn, typename TOut, int D, int BLK>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const int BH = (int)(a.B * a.H);
  const int nc = a.nc;
  hipLaunchKernelGGL(la_decay_table, dim3((unsigned)a.H), dim3(256), 0, st, a.decay, a.tbl, a.tbl_stride);
  hipLaunchKernelGGL((la_chunk_state<TIn, D>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                     (const TIn*)a.k, (const TIn*)a.v, (const float*)a.tbl, a.states, (int)a.H, (int)a.N,
                     (int)a.L, nc, a.tbl_stride);
  {
    const int64_t threads = (int64_t)BH * D * D / 4;
    hipLaunchKernelGGL(la_chunk_scan, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a.decay,
                       a.states, a.kv_in, a.kv_out, BH, (int)a.H, (int)a.N, (int)a.L, nc, D);
  }
  if (a.evt_begin) {
    hipError_t e = hipEventRecord((hipEvent_t)a.evt_begin, st);
    if (e != hipSuccess) return e;
  }
  if constexpr (BLK == 64 && sizeof(TIn) == 2)
    hipLaunchKernelGGL((la_chunk_output64<TOut, D>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (TOut*)a.out, (const float*)a.tbl,
                       (const float*)a.states, (int)a.H, (int)a.N, (int)a.L, nc, a.tbl_stride);
  else
    hipLaunchKernelGGL((la_chunk_output<TIn, TOut, D, BLK>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                       (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, (TOut*)a.out, (const float*)a.tbl,
                       (const float*)a.states, (int)a.H, (int)a.N, (int)a.L, nc, a.tbl_stride);
  if (a.evt_end) {
    hipError_t e = hipEventRecord((hipEvent_t)a.evt_end, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

template <typename TIn, typename TOut, int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t st) {
  switch (a.block) {
    case 64: return launch_prefill_t<TIn, TOut, D, 64>(a, st);
    case 128: return launch_prefill_t<TIn, TOut, D, 128>(a, st);
    case 256: return launch_prefill_t<TIn, TOut, D, 256>(a, st);
  }
  return hipErrorInvalidValue;
}

bool prefill_supported(int in_dtype, int out_dtype, int64_t d, int64_t block) {
  if (d != 64 && d != 128) return false;
  if (block != 64 && block != 128 && block != 256) return false;
  if (in_dtype == kBF16) return out_dtype == kBF16 || out_dtype == kF32;
  if (in_dtype == kF32 && out_dtype == kF32) return d == 64 || block == 64;  // LDS limit for fp32 tiles
  return false;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.in_dtype == kBF16 && a.out_dtype == kBF16) {
    if (a.d == 128) return launch_prefill_d<bf16, bf16, 128>(a, st);
    return launch_prefill_d<bf16, bf16, 64>(a, st);
  }
  if (a.in_dtype == kBF16 && a.out_dtype == kF32) {
    if (a.d == 128) return launch_prefill_d<bf16, float, 128>(a, st);
    return launch_prefill_d<bf16, float, 64>(a, st);
  }
  if (a.d == 128) return launch_prefill_t<float, float, 128, 64>(a, st);
  return launch_prefill_d<float, float, 64>(a, st);
}

}  // namespace la
