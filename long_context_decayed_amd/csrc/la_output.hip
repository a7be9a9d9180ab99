// Output pass (pass C) of the gfx950 lightning-attention prefill.
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
//                       all chunks in parallel (MFMA)                   [la_state.hip]
//   B  la_chunk_scan  : per (batch, head), S <- kv_in; for c: Sstart_c = S,
//                       S = lam^(L_c) S + U_c; kv_out = S (fp32)         [la_state.hip]
//   C  la_chunk_output: per chunk, the block loop above from Sstart_c (MFMA) [here]
// With bf16 inputs and block 64, a head that decays within its chunk takes
// none of the three: la_chunk_output64 in warm-start mode computes each of
// its chunks (of the longer warm-start chunk length) from the state built by
// the carry_span tokens before the chunk (from zero; older tokens weigh at
// most 2^-30 there), so Q, K and V of such a head are read about once and
// nothing waits on a scan.  In the forward, that pass and pass C of the
// other heads are one launch (la_chunk_output64_mixed).
//
// Precision recipe (bf16 inputs): products of two bf16 inputs are exact in the
// fp32 MFMA accumulator.  Quantities formed in fp32 that feed an MFMA are
// rounded: the state S used in q S, the decayed values lam^(..) v used in
// the state update and the masked, decayed scores P go in as a bf16 hi + lo
// pair (~16 significant bits; a single bf16 P was the dominant error).
// Accumulation is fp32 throughout and the state stays fp32.

#include <hip/hip_runtime.h>

#include "la_device.h"
#include "la_kernels.h"

namespace la {

// log2 of the distance between the two workgroups of a pair.  Workgroups
// are dealt to the 8 XCDs in turn, so i and i + 8 land on one XCD and share
// its L2.  (Measured on the 1,048,576-token, 64-head backward: 43.2 ms at
// distance 8, 44.2 ms at distance 1, 44.3 ms unpaired.)
constexpr int kPairShift = 3;

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
// kept in registers for the block's later sub-tiles.  REV: the reverse-time
// passes of the backward (rows last first; the initial state enters the
// first token undecayed, so the first block of chunk 0 takes one decay power
// less in its rows and in the state it hands on), as in la_chunk_output64.
template <typename TIn, typename TOut, int D, int BLK, bool REV>
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
  constexpr int RS = REV ? -D : D;  // elements from one token's row to the next
  const int64_t base = (int64_t)bh * N * D + (REV ? (int64_t)(N - 1) * D : 0);
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
    pq.template load<RS>(qb, t_begin, t_end, tid);
    pk.template load<RS>(kb, t_begin, t_end, tid);
    pv.template load<RS>(vb, t_begin, t_end, tid);
  }

  int jb = 0;  // sub-tile index within the current block
  for (int t0 = t_begin; t0 < t_end; t0 += kSub, jb = (jb + 1 == NS) ? 0 : jb + 1) {
    TIn* Kj = Ks + jb * kSub * LD;
    TIn* Vj = Vs + jb * kSub * LD;
    if (!kPrefetch) {
      pq.template load<RS>(qb, t0, t_end, tid);
      pk.template load<RS>(kb, t0, t_end, tid);
      pv.template load<RS>(vb, t0, t_end, tid);
    }
    pq.template store<LD>(Qs, tid);
    pk.template store<LD>(Kj, tid);
    pv.template store<LD>(Vj, tid);
    __syncthreads();
    if (kPrefetch && t0 + kSub < t_end) {
      pq.template load<RS>(qb, t0 + kSub, t_end, tid);
      pk.template load<RS>(kb, t0 + kSub, t_end, tid);
      pv.template load<RS>(vb, t0 + kSub, t_end, tid);
    }

    // REV: the first block of chunk 0 takes one decay power less.
    const int sh = (REV && c == 0 && t0 - t_begin < BLK) ? 1 : 0;
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
        S[kt] *= tbl[BLK - sh];
      }
    } else {
      if (jb == 0) {
        // Block start: keep S_b as MFMA B operands, then pre-decay S by lam^BLK.
        const float dblk = tbl[BLK - sh];
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
      for (int j = 0; j < 16; ++j) acc[rt][j] *= tbl[kSub * jb + 32 * rt + crow(j, hf) + 1 - sh];

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
          // Scores are fed as bf16 hi + lo: over windows longer than 64
          // tokens a single bf16 rounding of P is the dominant error.
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float x[M::EPL];
#pragma unroll
            for (int i = 0; i < M::EPL; ++i) x[i] = p[g * M::EPL + i];
            op_t pa, pl;
            M::split(x, pa, pl);
            const op_t vop = M::ld_tr_cperm(Vk, LD, 32 * st, g, 32 * w, lane);
            acc[rt] = M::mma(pa, vop, acc[rt]);
            if (M::kSplit) acc[rt] = M::mma(pl, vop, acc[rt]);
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
        if (t < t_end) ob[(int64_t)t * RS + col] = from_f32<TOut>(acc[rt][j]);
      }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Pass C, block = 64, bf16 inputs: the fast path.  Same arithmetic as
// la_chunk_output with BLK = 64, organised around what binds it on MI355X:
// streaming the tiles from HBM (the kernel with its arithmetic taken out runs
// within 10% of it), then VALU + MFMA issue per SIMD, vector-memory
// instruction issue, LDS.
//   * the output is computed transposed, O^T = S^T diag Q^T + V^T P^T: with
//     the accumulator holding O^T, each lane owns one token row and 4
//     consecutive columns per register quad, so after a lane-half swap a
//     64 x 32 block of bf16 O leaves in 4 stores of 16 bytes per lane, and
//     the inter-term decay lam^(p+1) is one per-lane factor;
//   * the state's accumulator rows hold the features in an order with bits 2
//     and 3 of the row index swapped, so the 8 features a lane contributes to
//     one MFMA step are contiguous in Q and K: one 16-byte LDS read;
//   * Q, K and V tiles arrive by 16-byte LDS DMA; K is kept twice in LDS, as
//     the row-read operand of the score tiles and as the transpose-read
//     operand of the state update, so that each copy is needed in one phase
//     only; the second copy is made from the first inside LDS;
//   * the 3 causal 32x32 score tiles P^T = K Q^T of a sub-tile are computed
//     by one wave each, masked, decayed and shared through LDS as bf16 hi + lo
//     MFMA operands (~16 bits of P);
//   * decay factors are per-lane powers times wave-uniform powers; the masked
//     factors of the two diagonal score tiles come from a per-lane LDS table
//     built once per workgroup;
//   * software pipeline over the two compute phases of a sub-tile: Q and the
//     score copy of K are only read in phase 1 (inter term and scores), so
//     the next ones are requested at the barrier that ends phase 1 and waited
//     for at the one that ends phase 2; V and the update copy of K are only
//     read in phase 2 (P V and the state update), so after that barrier the
//     next V is requested, ahead of this sub-tile's output stores, and waited
//     for at the end of the next phase 1, during which the K copy is made
//     (with 4 waves by the one that computes no score tile).
// Two workgroups per CU (77 KiB of LDS each, 78.5 KiB with the fused
// epilogue's buffers).
//
// Two modes, by where the chunk's start state comes from:
//   kWarmStart  heads that decay within their chunk (decays_within_chunk),
//               whose state at any token is, to 2^-30 of the older state's
//               own weight, made by the last carry_span tokens alone: chunk 0
//               starts from kv_in (or zero); chunk c > 0 starts from zero
//               carry_span tokens early and runs those tokens through the
//               state update only (no outputs), then the chunk with outputs.
//               The last chunk stores its end state (the final state) to its
//               `states` slot.  One pass over Q, K, V, plus K and V of the
//               warm-up tokens.  Other heads return at once.
//   kFromStart  the chunk from its true start state Sstart_c (read from
//               `states` after the scan), for the other heads; decaying heads
//               return at once.
// Which heads decay is judged against Lw, the warm-start chunk, in every
// kernel alike.  The warm-start pass chunks by Lw (L = Lw, nc = its chunk
// count), the other passes by the scan's chunk; `states` holds nc_ws slots
// per head (the scan's chunks) and the warm-start pass leaves each final
// state in the last of them.
// REV: the reverse-time passes of the backward.  Token t of the pass is row
// N-1-t of the tensors (rows are read and written last first), and the
// initial state enters the first token undecayed: S_0 = kv_in + k_0^T v_0,
// as the gradient of the final state does in the adjoint recurrence.  Only
// the first sub-tile of chunk 0 differs: its rows take lam^p instead of
// lam^(p+1) and it hands the state on decayed by lam^(n-1) instead of lam^n.
// SILU: q, k, v are pre-activations; every tile gets SiLU in LDS (silu_own)
// by the waves that brought it, between their own wait and the barrier
// that publishes it (the fact sheet's "linear / SSM layer configuration"
// field puts SiLU on Q, K and V), so the activations never make an HBM pass.
//
// Paired launch (pair_shift >= 0): two problems of one shape, with their own
// tensors and chunk states, share a grid; workgroup i serves problem
// (i >> pair_shift) & 1, so the two workgroups of one (bh, chunk) start
// 2^pair_shift apart and read the tensors the problems share at about the
// same time, the second often from L2.  The backward's dK and dV passes run
// this way: both read Q and dO.
enum { kWarmStart = 0, kFromStart = 1 };
constexpr int kEtab = 64;  // entries of the diagonal-tile factor table (60 used)

struct Operands {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  void* o;
  float* states;       // chunk states of this problem
  const float* kv_in;  // initial states, or null
  // Warm-start check (forward, or null): per (bh, warm-start chunk) slot of
  // kGuardSlots floats, [0, NW) the largest |S| per wave of the state just
  // before the next chunk's warm-up window, [4, 4 + NW) that of the state
  // the chunk's own warm-up builds (see la_warm_guard in la_state.hip).
  float* guard;
  // Heads to run (pass C of the heads whose warm start failed the check), or
  // null: every head of the launch's kind.
  const int* only;
  // Epilogue (EPI kernels): per-head RMSNorm weights [H][D] (null: no norm),
  // its eps, and the gate's pre-activation [B][H][N][D] (null: no gate).
  const float* gamma;
  float eps;
  const bf16* gate;
};

// Largest |x| over this wave's share of the state (each lane's 16 NRT
// accumulators), taken on the bit patterns of |x| so that a NaN (above +inf)
// is not lost; lane 0 stores it to dst.
template <int NRT>
__device__ __forceinline__ void store_wave_absmax(const f32x16 (&S)[NRT], float* dst, int lane) {
  uint32_t m = 0u;
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
    for (int j = 0; j < 16; ++j) m = max(m, __float_as_uint(S[kt][j]) & 0x7fffffffu);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if (lane == 0) *dst = __uint_as_float(m);
}

// The workgroup body: chunk blk of the (bh, chunk) grid of problem pi, on the
// LDS sm of the calling kernel.
template <typename TOut, int D, int MODE, bool REV, bool SILU, bool EPI, bool UNIT = false>
__device__ __forceinline__ void chunk_output64_body(bf16* Qs, bf16* Ks, bf16* Kt, bf16* Vs,
                                                    Mfma<bf16>::op_t (*Pbuf)[2][2][64], f32x4* Etab,
                                                    f32x4 (*Nbuf)[32], float* Gam, int blk,
                                                    int pi, Operands p0, Operands p1, const float* __restrict__ decay,
                                                    const float* __restrict__ tbl_all, int H, int N, int L, int nc,
                                                    int tbl_stride, const int* __restrict__ slots, int64_t num_slots,
                                                    int warm, int Lw, int nc_ws) {
  typedef Mfma<bf16> M;
  typedef M::op_t op_t;
  constexpr int NW = D / 32;
  constexpr int NRT = D / 32;
  constexpr int MAXT = (3 + NW - 1) / NW;  // score tiles per wave
  constexpr int kStores = sizeof(TOut) == 2 ? 2 * 2 : 2 * 4;  // output store instructions per sub-tile
  // EPI: out = RMSNorm_head(o) * gamma[h] * sigmoid(gate) instead of o (the
  // MiniMax-M1 fact sheet's "linear / SSM layer configuration" field puts an
  // RMSNorm on the output, its "output gate" field a sigmoid gate after it).
  constexpr bool kDefer = sizeof(TOut) == 2;  // bf16 rows are stored during the next sub-tile's phase 1
  constexpr int RS = REV ? -D : D;             // elements from one token's row to the next

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const bf16* __restrict__ q = pi ? p1.q : p0.q;
  const bf16* __restrict__ k = pi ? p1.k : p0.k;
  const bf16* __restrict__ v = pi ? p1.v : p0.v;
  TOut* __restrict__ o = static_cast<TOut*>(pi ? p1.o : p0.o);
  float* __restrict__ states = pi ? p1.states : p0.states;
  const float* __restrict__ kv_in = pi ? p1.kv_in : p0.kv_in;
  const int bh = blk / nc, c = blk - (blk / nc) * nc;
  const int hh = bh % H;
  const int span = carry_span(decay[hh]);
  const bool decaying = warm && decays_within_chunk(span, Lw);  // warm = 0: every head from its start state
  if (decaying != (MODE == kWarmStart)) return;
  const int* __restrict__ only = pi ? p1.only : p0.only;
  if (only && !only[bh]) return;
  float* __restrict__ guard = pi ? p1.guard : p0.guard;
  static_assert(!(EPI && REV), "the epilogue is a forward step");
  // UNIT: lam = 1 (no decay; the head is plain causal linear attention).
  // Every factor is then 1, so V enters the state update as the bf16 input
  // itself (one MFMA per step instead of the hi + lo pair) and the decays of
  // S, of the inter term and of the off-diagonal score tile are skipped: the
  // same values as the general path, whose factors and lo parts are exactly
  // 1 and 0 there.  Only heads that do not decay within a chunk (kFromStart).
  static_assert(!(UNIT && MODE == kWarmStart), "lam = 1 never takes the warm start");
  const float* __restrict__ gamma = p0.gamma;  // forward launches carry one problem
  const bf16* __restrict__ gate = p0.gate;
  const int t_begin = c * L;
  const int t_end = min(N, t_begin + L);
  const int64_t base = (int64_t)bh * N * D + (REV ? (int64_t)(N - 1) * D : 0);
  const bf16* qb = q + base;
  const bf16* kb = k + base;
  const bf16* vb = v + base;
  TOut* ob = o + base;
  const int col = 32 * w + l32;
  const float* tb = tbl_all + (int64_t)hh * tbl_stride;  // lam^e, e <= 64

  // Decay factors (all exponents non-negative), j = 4jq + jj:
  //   update, s = trbase(kk) + trow(i, h):
  //           lam^(63-s) = wl[kk][i] = lam^(56-trbase(kk)-16(i>>2)) * ul[i],  ul[i] = lam^(7-4h-(i&3))
  //   inter,  token p = 32rt + l:      lam^(p+1)  = rf[rt]
  //   off-diagonal score tile (r = 32 + l, s = crow(j, h)):
  //           lam^(r-s) = lam^(24-8jq) * ol[jj],  ol[jj] = lam^(l+4-4h+4-jj)
  //   diagonal tile (r = l, s = crow(j, h)), d = r - s = l - 4h - 8jq - jj:
  //           lam^d for d >= 0, 0 (masked) for d < 0.  The four factors of
  //           one jq depend on l - 4h - 8jq alone (in [-28, 31]), so they are
  //           kept once per value in an LDS table, Etab[l - 4h - 8jq + 28][jj]
  //           (64 entries of 16 bytes; consecutive lanes read consecutive
  //           entries).
  // They are loaded here, before the tile loop, so that the loop issues no
  // vector-memory loads of its own.
  float ol[4], ul[8], rf[2], wl[4][8];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) ol[jj] = tb[l32 + 8 - 4 * hf - jj];
#pragma unroll
  for (int i = 0; i < 8; ++i) ul[i] = tb[7 - 4 * hf - (i & 3)];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int i = 0; i < 8; ++i) wl[kk][i] = ul[i] * tb[56 - trbase(kk) - 16 * (i >> 2)];
  rf[0] = tb[l32 + 1];
  rf[1] = tb[l32 + 33];
  const float d64 = tb[64];
  // Warm-start mode hands on the exact final state, so its last sub-tile,
  // when partial (n < 64 tokens, only at the end of the sequence), decays the
  // state by lam^n and weights token s by lam^(n-1-s): lam^e for e < 64 is
  // kept one per lane and fetched by lane shuffle.
  float tlane = 0.0f, d_last = 0.0f;
  const int n_last = (t_end - t_begin) - kSub * ((t_end - t_begin - 1) / kSub);  // tokens of the last sub-tile
  if constexpr (MODE == kWarmStart) {
    tlane = tb[lane];
    d_last = tb[n_last];
  }
  // REV, first sub-tile of chunk 0: lam^p for row p (taken from the
  // neighbouring lane's rf when needed, so that nothing more stays live
  // across the loop), state decayed by lam^63 (lam^(n-1) if it is also the
  // last, partial one).
  float d_first = 0.0f;
  if constexpr (REV) d_first = (t_end - t_begin <= kSub) ? tb[n_last - 1] : tb[63];
  for (int e = tid; e < kEtab; e += NW * 64) {
    const int dd = e - 28;
    Etab[e] = f32x4{dd >= 0 ? tb[dd] : 0.0f, dd >= 1 ? tb[dd - 1] : 0.0f, dd >= 2 ? tb[dd - 2] : 0.0f,
                    dd >= 3 ? tb[dd - 3] : 0.0f};
  }
  const f32x4* etab_lane = Etab + (l32 - 4 * hf + 28);  // this lane's entry for jq = 0
  if constexpr (EPI) {
    // the head's norm weights, made visible by the barrier after the first tiles
    for (int e = tid; e < D; e += NW * 64) Gam[e] = gamma ? gamma[(int64_t)hh * D + e] : 1.0f;
  }

  // State tile kt, register j of lane (h, n): feature 32kt + pf(crow(j, h)),
  // value column col, where pf swaps bits 2 and 3:
  //   pf(crow(j, h)) = 16(j >> 3) + 8h + 4((j >> 2) & 1) + (j & 3).
  f32x16 S[NRT];
  const int64_t srow = (MODE == kWarmStart && c == 0 && kv_in != nullptr) ? state_row(bh, H, slots, num_slots) : -1;
  const float* s_src = MODE == kFromStart ? states + ((int64_t)bh * nc_ws + c) * D * D
                                          : (srow >= 0 ? kv_in + srow * D * D : nullptr);
  if (s_src) {
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        S[kt][j] = s_src[(32 * kt + 16 * (j >> 3) + 8 * hf + 4 * ((j >> 2) & 1) + (j & 3)) * D + col];
  } else {
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt) S[kt] = zero16();
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the state and the factors are in registers

  // State update over one full sub-tile in (Kx, Vx): S += sum_s lam^(63-s)
  // k_s^T v_s, tokens s = trbase(kk) + trow(i, h).
  auto update_full = [&](const bf16* Kx, const bf16* Vx) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const op_t vraw = ld_tr8<D, false>(Vx, trbase(kk), 32 * w, lane);
      if constexpr (UNIT) {
#pragma unroll
        for (int kt = 0; kt < NRT; ++kt) S[kt] = M::mma(ld_tr8<D, true>(Kx, trbase(kk), 32 * kt, lane), vraw, S[kt]);
        continue;
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)vraw[i] * wl[kk][i];
      op_t bhi, blo;
      M::split(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        const op_t a = ld_tr8<D, true>(Kx, trbase(kk), 32 * kt, lane);
        S[kt] = M::mma(a, bhi, S[kt]);
        S[kt] = M::mma(a, blo, S[kt]);
      }
    }
  };

  if constexpr (MODE == kWarmStart) {
    if (c > 0 && span > 0) {
      // Warm-up: the span tokens before the chunk (whole sub-tiles, as the
      // chunk start and span are multiples of 64) through the state update
      // alone, from S = 0, double-buffered in (Kt, Vs) and (Ks, Qs).
      const int nwu = span / kSub;
      const int64_t off0 = (int64_t)(t_begin - span) * RS;
      dma_tile<D, NW, RS>(kb + off0, Kt, kSub, w, lane);
      dma_tile<D, NW, RS>(vb + off0, Vs, kSub, w, lane);
      for (int j = 0; j < nwu; ++j) {
        const bool odd = (j & 1) != 0;
        // Sub-tile j is visible; every wave is done with the other buffer.
        if constexpr (SILU) {
          wait_vmem<0>();
          silu_own<D, NW>(odd ? Ks : Kt, kSub, w, lane);
          silu_own<D, NW>(odd ? Qs : Vs, kSub, w, lane);
        }
        sync_lds_after_vmem<0>();
        if (j + 1 < nwu) {
          const int64_t offn = off0 + (int64_t)(j + 1) * kSub * RS;
          dma_tile<D, NW, RS>(kb + offn, odd ? Kt : Ks, kSub, w, lane);
          dma_tile<D, NW, RS>(vb + offn, odd ? Vs : Qs, kSub, w, lane);
        }
#pragma unroll
        for (int kt = 0; kt < NRT; ++kt) S[kt] *= d64;
        update_full(odd ? Ks : Kt, odd ? Qs : Vs);
      }
      __syncthreads();  // every wave is done with the warm-up tiles
      if (guard) store_wave_absmax<NRT>(S, guard + ((int64_t)bh * nc + c) * kGuardSlots + 4 + w, lane);
    }
  }
  // Warm start: the token before the next chunk's warm-up window, where the
  // state that window leaves out is this chunk's (none for the last chunk).
  const int t_mark = (MODE == kWarmStart && guard && c + 1 < nc && span > 0) ? t_end - span : -1;

  {
    const int nv = min(kSub, t_end - t_begin);
    const int64_t off = (int64_t)t_begin * RS;
    dma_tile<D, NW, RS>(qb + off, Qs, nv, w, lane);
    dma_tile<D, NW, RS>(kb + off, Ks, nv, w, lane);
    dma_tile<D, NW, RS>(kb + off, Kt, nv, w, lane);
    dma_tile<D, NW, RS>(vb + off, Vs, nv, w, lane);
    if constexpr (SILU) {
      wait_vmem<0>();
      silu_own<D, NW>(Qs, nv, w, lane);
      silu_own<D, NW>(Ks, nv, w, lane);
      silu_own<D, NW>(Kt, nv, w, lane);
      silu_own<D, NW>(Vs, nv, w, lane);
    }
    sync_lds_after_vmem<0>();
  }
  // bf16 output of the previous sub-tile, packed and lane-swapped, stored
  // one instruction per step of the next inter loop so that the stores
  // trickle out instead of queueing all at once behind the CU's store path.
  uint4 pend[2][2];
  bool have_pend = false;
  int t_pend = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += kSub) {
    const bool more = t0 + kSub < t_end;
    const bool first = REV && c == 0 && t0 == t_begin;
    const int nv_next = min(kSub, t_end - t0 - kSub);
    const int64_t off_next = (int64_t)(t0 + kSub) * RS;
    if (MODE == kWarmStart && t0 == t_mark)  // S is the state after token t0 - 1
      store_wave_absmax<NRT>(S, guard + ((int64_t)bh * nc + c) * kGuardSlots + w, lane);

    // Phase 1.  Inter term acc[rt] = S_b^T Q^T for tokens 32rt + l (S split
    // into bf16 hi + lo on the fly) and this wave's score tiles P^T = K Q^T,
    // sharing the Q operands; then S *= lam^64.
    f32x16 acc[2], pt[MAXT];
    acc[0] = zero16();
    acc[1] = zero16();
#pragma unroll
    for (int m = 0; m < MAXT; ++m) pt[m] = zero16();
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int f0 = 32 * kt + 16 * g + 8 * hf;
        const op_t qa0 = ld_row8<D>(Qs, l32, f0);
        const op_t qa1 = ld_row8<D>(Qs, 32 + l32, f0);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = S[kt][8 * g + i];
        op_t hi, lo;
        M::split(x, hi, lo);
        acc[0] = M::mma(hi, qa0, acc[0]);
        acc[1] = M::mma(hi, qa1, acc[1]);
        acc[0] = M::mma(lo, qa0, acc[0]);
        acc[1] = M::mma(lo, qa1, acc[1]);
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
          const int ti = w + m * NW;
          if (ti < 3) {
            const int st = ti == 2 ? 1 : 0, rt = ti == 0 ? 0 : 1;
            const op_t ka = ld_row8<D>(Ks, 32 * st + l32, f0);
            pt[m] = M::mma(ka, rt ? qa1 : qa0, pt[m]);
          }
        }
      }
      if constexpr (UNIT) {
      } else if (REV && first)
        S[kt] *= d_first;
      else if constexpr (MODE == kWarmStart)
        S[kt] *= more ? d64 : d_last;
      else
        S[kt] *= d64;
      if constexpr (kDefer) {
        // The pending sub-tile is a full one (only the last can be partial).
        static_assert(4 % NRT == 0, "whole stores per step");
        if (have_pend) {
#pragma unroll
          for (int q = 0; q < 4 / NRT; ++q) {
            const int e = kt * (4 / NRT) + q, rt = e >> 1, pp = e & 1;
            bf16* orow = reinterpret_cast<bf16*>(ob) + (int64_t)(t_pend + 32 * rt + l32) * RS + 32 * w + 16 * pp + 8 * hf;
            *reinterpret_cast<uint4*>(orow) = pend[rt][pp];
          }
        }
      }
    }
    // This sub-tile's K^T copy from its score copy (in LDS since the last
    // barrier; the previous K^T is no longer read): with 4 waves by the one
    // that has no score tile, in its share of phase 1, else by all waves.
    if (t0 != t_begin) {
      constexpr int CW = (NW == 4) ? 1 : NW;            // copying waves
      constexpr int NCH = kSub * D * 2 / 16 / (CW * 64);  // 16-byte chunks per lane
      if (NW != 4 || w == NW - 1) {
        const int ct = (NW == 4) ? lane : tid;
        const uint4* ksrc = reinterpret_cast<const uint4*>(Ks);
        uint4* kdst = reinterpret_cast<uint4*>(Kt);
#pragma unroll
        for (int b = 0; b < NCH; b += 4) {
          uint4 tmp[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) tmp[i] = ksrc[ct + CW * 64 * (b + i)];
#pragma unroll
          for (int i = 0; i < 4; ++i) kdst[ct + CW * 64 * (b + i)] = tmp[i];
        }
      }
    }
    // Mask, decay and publish the score tiles as hi + lo operands.
#pragma unroll
    for (int m = 0; m < MAXT; ++m) {
      const int ti = w + m * NW;
      if (ti < 3) {
        if (ti == 1) {
          if constexpr (!UNIT) {
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
              const float u = tb[24 - 8 * jq];
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) pt[m][4 * jq + jj] *= ol[jj] * u;
            }
          }
        } else {
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const f32x4 f = etab_lane[-8 * jq];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) pt[m][4 * jq + jj] *= f[jj];
          }
        }
        // operand g, element i: register 4g + 8(i >> 2) + (i & 3), the score of
        // token 8g + trow(i, h) of the tile, to match the V rows of phase 2
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = pt[m][4 * g + 8 * (i >> 2) + (i & 3)];
          op_t hi, lo;
          M::split(x, hi, lo);
          Pbuf[ti][g][0][lane] = hi;
          Pbuf[ti][g][1][lane] = lo;
        }
      }
    }
    // Inter-term decay lam^(p+1), one factor per lane and token tile.  Written
    // element by element: as a vector-by-scalar product the compiler hoists a
    // 16-wide copy of each factor out of the loop (30 registers).
    float r_tile[2] = {rf[0], rf[1]};
    if (!UNIT && REV && first) {
      // lam^p = rf of row p - 1: lane l - 1 of the same tile, or for l = 0,
      // lam^0 = 1 (tile 0) and lam^32 = rf[0] of lane 31 (tile 1).
      const float up0 = __shfl(rf[0], lane - 1), up1 = __shfl(rf[1], lane - 1), top = __shfl(rf[0], lane + 31);
      r_tile[0] = l32 == 0 ? 1.0f : up0;
      r_tile[1] = l32 == 0 ? top : up1;
    }
    if constexpr (!UNIT) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float r = r_tile[rt];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[rt][j] *= r;
      }
    }

    // This sub-tile's V and K^T copy (requested before the previous
    // sub-tile's kStores output stores, which may still be in flight) and
    // the score tiles become visible; Q and the score copy of K are free.
    if constexpr (SILU) {
      if (t0 != t_begin) {  // the first sub-tile's V came with the initial tiles
        wait_vmem<kStores>();
        silu_own<D, NW>(Vs, min(kSub, t_end - t0), w, lane);
      }
    }
    sync_lds_after_vmem<kStores>();
    if (more) {
      dma_tile<D, NW, RS>(qb + off_next, Qs, nv_next, w, lane);
      dma_tile<D, NW, RS>(kb + off_next, Ks, nv_next, w, lane);
    }
    // EPI: this sub-tile's gate values, 8 bf16 per (token tile, column pair)
    // at the columns this lane owns after the lane-half swap below; they
    // arrive during phase 2 and are waited for at its closing barrier.
    uint4 gq[2][2];
    if constexpr (EPI) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int t = t0 + 32 * rt + l32;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
          gq[rt][pp] = (gate && t < t_end) ? *reinterpret_cast<const uint4*>(
                                                 gate + base + (int64_t)t * D + 32 * w + 16 * pp + 8 * hf)
                                           : make_uint4(0u, 0u, 0u, 0u);
      }
    }

    // Phase 2.  Intra-block term acc[rt] += V^T P^T over the shared score tiles.
#pragma unroll
    for (int ti = 0; ti < 3; ++ti) {
      const int st = ti == 2 ? 1 : 0, rt = ti == 0 ? 0 : 1;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const op_t vop = ld_tr8<D, false>(Vs, 32 * st + 8 * g, 32 * w, lane);
        acc[rt] = M::mma(vop, Pbuf[ti][g][0][lane], acc[rt]);
        acc[rt] = M::mma(vop, Pbuf[ti][g][1][lane], acc[rt]);
      }
    }

    // State update.  A partial last sub-tile of warm-start mode is added
    // after the loop.
    if (!(MODE == kWarmStart && !more && t_end - t0 < kSub)) update_full(Kt, Vs);

    // EPI: each token's sum of squares over this wave's 32 columns (the lane
    // and its partner in the other half hold 16 each), published in Nbuf for
    // the other waves by the barrier below (Nbuf is read after it and not
    // written again before the next sub-tile's first barrier).
    if constexpr (EPI) {
      if (gamma) {
        float ss[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          float a = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) a = __builtin_fmaf(acc[rt][j], acc[rt][j], a);
          ss[rt] = a + __shfl_xor(a, 32);
        }
        if (hf == 0) {
          reinterpret_cast<float*>(&Nbuf[0][l32])[w] = ss[0];
          reinterpret_cast<float*>(&Nbuf[1][l32])[w] = ss[1];
        }
      }
    }

    // The next sub-tile's Q and K (and this wave's older stores) are done
    // and visible; V, K^T and the score tiles are free from here on.
    if constexpr (SILU) {
      if (more) {
        wait_vmem<0>();
        silu_own<D, NW>(Qs, nv_next, w, lane);
        silu_own<D, NW>(Ks, nv_next, w, lane);
      }
    }
    if constexpr (EPI) {
      // The gate values count as used here, where every load of this wave
      // is waited for anyway: the compiler, which cannot see the transfers
      // issued from inline assembly, would otherwise wait for the gate
      // loads in the epilogue below with a count that also covers the next
      // V tile requested right after this barrier.
      asm volatile("" : : "v"(gq[0][0].x), "v"(gq[0][1].x), "v"(gq[1][0].x), "v"(gq[1][1].x));
    }
    sync_lds_after_vmem<0>();
    if (more) {
      dma_tile<D, NW, RS>(vb + off_next, Vs, nv_next, w, lane);
    }

    // Output rows.  Lane (h, l) holds token t0 + 32rt + l, columns 32w + 8jq
    // + 4h + jj.  bf16: the two lane halves trade quads (v_permlane32_swap)
    // so that each lane owns 8 consecutive columns 32w + 16p + 8h .. + 7 of
    // column pair p, stored as 16 bytes (the two halves then write 32
    // contiguous bytes of each row) during the next sub-tile, or below after
    // the last one.  fp32: four 16-byte stores per token tile, here.
    if constexpr (EPI) {
      // Lane halves trade fp32 quads first, so that each lane holds the 8
      // consecutive columns 32w + 16pp + 8h .. + 7 of its token, then
      // y = ((o * inv) * gamma) * sigmoid(gate) per element (inv = 1 /
      // sqrt(mean(o^2) + eps) over the token's d columns, the four waves'
      // partial sums added in wave order), rounded once.
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float inv = 1.0f;
        if (gamma) {
          const f32x4 p = Nbuf[rt][l32];
          float sum = p[0];
#pragma unroll
          for (int i = 1; i < NW; ++i) sum += p[i];
          inv = 1.0f / sqrtf(sum * (1.0f / D) + p0.eps);
        }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int ja = 8 * pp, jb = 8 * pp + 4;  // quads jq = 2pp (kept by h = 0), 2pp + 1 (kept by h = 1)
          float y[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[rt][ja + i]),
                                                             __float_as_uint(acc[rt][jb + i]), false, false);
            y[i] = __uint_as_float(sw[0]);      // column 8h + i of the pair
            y[4 + i] = __uint_as_float(sw[1]);  // column 8h + 4 + i
          }
          const int c0 = 32 * w + 16 * pp + 8 * hf;
          const f32x4 ga = *reinterpret_cast<const f32x4*>(Gam + c0);
          const f32x4 gb = *reinterpret_cast<const f32x4*>(Gam + c0 + 4);
          const bf16x8 gv = __builtin_bit_cast(bf16x8, gq[rt][pp]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float sg = gate ? sigmoid_hw((float)gv[i]) : 1.0f;
            y[i] = ((y[i] * inv) * (i < 4 ? ga[i] : gb[i - 4])) * sg;
          }
          if constexpr (kDefer) {
            pend[rt][pp] = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                      pack_bf16x2(y[6], y[7]));
          } else {
            const int t = t0 + 32 * rt + l32;
            if (t < t_end) {
              float* orow = reinterpret_cast<float*>(ob) + (int64_t)t * RS + c0;
              *reinterpret_cast<f32x4*>(orow) = f32x4{y[0], y[1], y[2], y[3]};
              *reinterpret_cast<f32x4*>(orow + 4) = f32x4{y[4], y[5], y[6], y[7]};
            }
          }
        }
      }
      if constexpr (kDefer) {
        have_pend = true;
        t_pend = t0;
      }
    } else if constexpr (kDefer) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int ja = 8 * pp, jb = 8 * pp + 4;  // quads jq = 2pp (kept by h = 0), 2pp + 1 (kept by h = 1)
          const uint32_t a0 = pack_bf16x2(acc[rt][ja], acc[rt][ja + 1]), a1 = pack_bf16x2(acc[rt][ja + 2], acc[rt][ja + 3]);
          const uint32_t b0 = pack_bf16x2(acc[rt][jb], acc[rt][jb + 1]), b1 = pack_bf16x2(acc[rt][jb + 2], acc[rt][jb + 3]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
          pend[rt][pp] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
      have_pend = true;
      t_pend = t0;
    } else {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int t = t0 + 32 * rt + l32;
        if (t < t_end) {
          TOut* orow = ob + (int64_t)t * RS + 32 * w + 4 * hf;
#pragma unroll
          for (int jq = 0; jq < 4; ++jq)
            *reinterpret_cast<f32x4*>(orow + 8 * jq) =
                f32x4{acc[rt][4 * jq], acc[rt][4 * jq + 1], acc[rt][4 * jq + 2], acc[rt][4 * jq + 3]};
        }
      }
    }
  }
  if constexpr (kDefer) {
    // The last sub-tile (possibly partial).
    if (have_pend) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int t = t_pend + 32 * rt + l32;
        if (t < t_end) {
          bf16* orow = reinterpret_cast<bf16*>(ob) + (int64_t)t * RS + 32 * w + 8 * hf;
          *reinterpret_cast<uint4*>(orow) = pend[rt][0];
          *reinterpret_cast<uint4*>(orow + 16) = pend[rt][1];
        }
      }
    }
  }
  if (MODE == kWarmStart && c == nc - 1) {
    // Partial last sub-tile (n < 64 tokens, still in Vs and Kt): S += sum_{s<n}
    // lam^(n-1-s) k_s^T v_s; S was decayed by lam^n in its phase 1.
    const int n = (t_end - t_begin) - kSub * ((t_end - t_begin - 1) / kSub);
    if (n < kSub) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const op_t vraw = ld_tr8<D, false>(Vs, trbase(kk), 32 * w, lane);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = n - 1 - (trbase(kk) + trow(i, hf));
          const float f = __shfl(tlane, e < 0 ? 0 : e);
          x[i] = e >= 0 ? (float)vraw[i] * f : 0.0f;
        }
        op_t bhi, blo;
        M::split(x, bhi, blo);
#pragma unroll
        for (int kt = 0; kt < NRT; ++kt) {
          const op_t a = ld_tr8<D, true>(Kt, trbase(kk), 32 * kt, lane);
          S[kt] = M::mma(a, bhi, S[kt]);
          S[kt] = M::mma(a, blo, S[kt]);
        }
      }
    }
    // The final state, natural (feature, column) order, to the last chunk's
    // slot.  The lane's column and half are taken from the hardware lane id
    // here, so that they need not stay live (or spilled) across the loop.
    const int ln = __lane_id(), lh = ln >> 5;
    float* dst = states + ((int64_t)bh * nc_ws + nc_ws - 1) * D * D + 32 * w + (ln & 31);
#pragma unroll
    for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        dst[(32 * kt + 16 * (j >> 3) + 8 * lh + 4 * ((j >> 2) & 1) + (j & 3)) * D] = S[kt][j];
  }
}

// kFromStart body with the head's decay looked at once: lam = 1 takes the
// UNIT instantiation (not with SiLU and the epilogue together, where the
// two bodies in one kernel would spill registers; the general body is
// exact at lam = 1 too).
template <typename TOut, int D, bool REV, bool SILU, bool EPI>
__device__ __forceinline__ void chunk_output64_from_start(bf16* Qs, bf16* Ks, bf16* Kt, bf16* Vs,
                                                          Mfma<bf16>::op_t (*Pbuf)[2][2][64], f32x4* Etab,
                                                          f32x4 (*Nbuf)[32], float* Gam, int blk, int pi, Operands p0,
                                                          Operands p1, const float* __restrict__ decay,
                                                          const float* __restrict__ tbl_all, int H, int N, int L,
                                                          int nc, int tbl_stride, const int* __restrict__ slots,
                                                          int64_t num_slots, int warm, int Lw, int nc_ws) {
  if (!(SILU && EPI) && decay[(blk / nc) % H] == 1.0f)
    chunk_output64_body<TOut, D, kFromStart, REV, SILU, EPI, !(SILU && EPI)>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, blk, pi, p0,
                                                                   p1, decay, tbl_all, H, N, L, nc, tbl_stride, slots,
                                                                   num_slots, warm, Lw, nc_ws);
  else
    chunk_output64_body<TOut, D, kFromStart, REV, SILU, EPI, false>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, blk, pi, p0,
                                                                    p1, decay, tbl_all, H, N, L, nc, tbl_stride, slots,
                                                                    num_slots, warm, Lw, nc_ws);
}

// One problem, or two in one grid (pair_shift >= 0, see above).
template <typename TOut, int D, int MODE, bool REV, bool SILU, bool EPI>
__global__ __launch_bounds__(D * 2, 2) void la_chunk_output64(Operands p0, Operands p1,
                                                              const float* __restrict__ decay,
                                                              const float* __restrict__ tbl_all, int H, int N, int L,
                                                              int nc, int tbl_stride, const int* __restrict__ slots,
                                                              int64_t num_slots, int warm, int nblk, int pair_shift,
                                                              int Lw, int nc_ws) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Ks[kSub * D];  // score operands (phase 1)
  __shared__ __attribute__((aligned(16))) bf16 Kt[kSub * D];  // update operands (phase 2)
  __shared__ __attribute__((aligned(16))) bf16 Vs[kSub * D];
  __shared__ __attribute__((aligned(16))) Mfma<bf16>::op_t Pbuf[3][2][2][64];  // [tile][g][hi/lo][lane]
  __shared__ __attribute__((aligned(16))) f32x4 Etab[kEtab];                    // diagonal-tile factors
  __shared__ __attribute__((aligned(16))) f32x4 Nbuf[2][32];  // epilogue: per-wave sums of squares [tile][token]
  __shared__ __attribute__((aligned(16))) float Gam[D];        // epilogue: the head's norm weights
  int blk = blockIdx.x, pi = 0;
  if (pair_shift >= 0) {
    pi = (blk >> pair_shift) & 1;
    blk = ((blk >> (pair_shift + 1)) << pair_shift) | (blk & ((1 << pair_shift) - 1));
    if (blk >= nblk) return;  // padding of the last group
  }
  if constexpr (MODE == kFromStart)
    chunk_output64_from_start<TOut, D, REV, SILU, EPI>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, blk, pi, p0, p1, decay,
                                                       tbl_all, H, N, L, nc, tbl_stride, slots, num_slots, warm, Lw,
                                                       nc_ws);
  else
    chunk_output64_body<TOut, D, MODE, REV, SILU, EPI>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, blk, pi, p0, p1, decay,
                                                       tbl_all, H, N, L, nc, tbl_stride, slots, num_slots, warm, Lw,
                                                       nc_ws);
}

// The warm-start pass and the other heads' output pass (pass C) in one grid:
// workgroups [0, n_warm) take the warm-start pass's chunks (Lw tokens), the
// rest pass C's (L tokens, from the scanned start states); each returns at
// once for a head of the other kind.  One launch lets the few workgroups of a
// layer's non-decaying heads fill the rounds the warm-start pass leaves
// partly empty, and the other way round.
template <typename TOut, int D, bool SILU, bool EPI>
__global__ __launch_bounds__(D * 2, 2) void la_chunk_output64_mixed(Operands p0, const float* __restrict__ decay,
                                                                    const float* __restrict__ tbl_all, int H, int N,
                                                                    int L, int nc, int Lw, int ncw, int tbl_stride,
                                                                    const int* __restrict__ slots, int64_t num_slots,
                                                                    int n_warm) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Ks[kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Kt[kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kSub * D];
  __shared__ __attribute__((aligned(16))) Mfma<bf16>::op_t Pbuf[3][2][2][64];
  __shared__ __attribute__((aligned(16))) f32x4 Etab[kEtab];
  __shared__ __attribute__((aligned(16))) f32x4 Nbuf[2][32];
  __shared__ __attribute__((aligned(16))) float Gam[D];
  const int b = blockIdx.x;
  // Warm-start chunks in reverse order, last head first: with ALiBi-style
  // slopes, which shrink with the head index, the longest warm-ups come first
  // and the short chunks fill the last round (measured 0.2-1% faster than in
  // head order at 1024 warm-start workgroups).
  if (b < n_warm)
    chunk_output64_body<TOut, D, kWarmStart, false, SILU, EPI>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, n_warm - 1 - b, 0, p0, p0, decay,
                                                          tbl_all, H, N, Lw, ncw, tbl_stride, slots, num_slots, 1, Lw,
                                                          nc);
  else
    chunk_output64_from_start<TOut, D, false, SILU, EPI>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, b - n_warm, 0, p0, p0, decay,
                                                          tbl_all, H, N, L, nc, tbl_stride, slots, num_slots, 1, Lw,
                                                          nc);
}

// The same for the backward's reverse-time dK and dV passes, paired as above:
// the grid's first n_warm_grid workgroups are the two problems' warm-start
// chunks (paired, pair_shift = kPairShift, nblk_w per problem), the rest their
// pass-C chunks (paired likewise, nblk_c per problem).
template <typename TOut, int D>
__global__ __launch_bounds__(D * 2, 2) void la_chunk_output64_mixed_pair(
    Operands p0, Operands p1, const float* __restrict__ decay, const float* __restrict__ tbl_all, int H, int N, int L,
    int nc, int Lw, int ncw, int tbl_stride, int nblk_w, int nblk_c, int n_warm_grid) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Ks[kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Kt[kSub * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kSub * D];
  __shared__ __attribute__((aligned(16))) Mfma<bf16>::op_t Pbuf[3][2][2][64];
  __shared__ __attribute__((aligned(16))) f32x4 Etab[kEtab];
  __shared__ __attribute__((aligned(16))) f32x4 Nbuf[2][32];
  __shared__ __attribute__((aligned(16))) float Gam[D];
  const bool warm_part = (int)blockIdx.x < n_warm_grid;
  const int b = warm_part ? (int)blockIdx.x : (int)blockIdx.x - n_warm_grid;
  const int pi = (b >> kPairShift) & 1;
  const int blk = ((b >> (kPairShift + 1)) << kPairShift) | (b & ((1 << kPairShift) - 1));
  if (blk >= (warm_part ? nblk_w : nblk_c)) return;  // padding of a last group
  if (warm_part)
    chunk_output64_body<TOut, D, kWarmStart, true, false, false>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, blk, pi, p0, p1, decay, tbl_all,
                                                          H, N, Lw, ncw, tbl_stride, nullptr, 0, 1, Lw, nc);
  else
    chunk_output64_from_start<TOut, D, true, false, false>(Qs, Ks, Kt, Vs, Pbuf, Etab, Nbuf, Gam, blk, pi, p0, p1, decay, tbl_all,
                                                          H, N, L, nc, tbl_stride, nullptr, 0, 1, Lw, nc);
}

// ---------------------------------------------------------------------------
// Host-side launcher: the output pass on `st`, bracketed by the optional
// timing events.

// The events bracket the kernel that writes every output row: the
// warm-start pass when there is one (bf16 inputs, block 64), else this one.
static Operands operands_of(const PrefillArgs& a) {
  return Operands{(const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.out, a.states, a.kv_in,
                  a.warm_start ? a.guard : nullptr, a.rerun ? a.flags : nullptr, a.gamma, a.eps,
                  (const bf16*)a.gate};
}

// One problem (b == nullptr), or two of one shape in one grid (the pair's
// flags, decays and table are a's).
template <typename TOut, int D, int MODE>
static void launch_fast(const PrefillArgs& a, hipStream_t st, const PrefillArgs* b = nullptr) {
  // the warm-start pass chunks by the warm chunk, the others by the scan's
  const int ncm = MODE == kWarmStart ? a.nc_warm : a.nc;
  const int Lm = (int)(MODE == kWarmStart ? a.L_warm : a.L);
  const int nblk = (int)(a.B * a.H * ncm);
  const int shift = b ? kPairShift : -1;
  const int64_t half = int64_t(1) << kPairShift;  // workgroups of one problem per group of the pair
  const unsigned grid = b ? (unsigned)((nblk + half - 1) / half * 2 * half) : (unsigned)nblk;
  const Operands p0 = operands_of(a), p1 = b ? operands_of(*b) : p0;
#define LA_FAST(REV, SILU, EPI)                                                                               \
  hipLaunchKernelGGL((la_chunk_output64<TOut, D, MODE, REV, SILU, EPI>), dim3(grid), dim3(D * 2), 0, st, p0, p1, \
                     a.decay, (const float*)a.tbl, (int)a.H, (int)a.N, Lm, ncm, a.tbl_stride, a.slots,            \
                     a.num_slots, a.warm_start ? 1 : 0, nblk, shift, (int)a.L_warm, a.nc)
  if (a.rev)  // the backward: no SiLU, no epilogue
    LA_FAST(true, false, false);
  else if (a.epi && a.silu)
    LA_FAST(false, true, true);
  else if (a.epi)
    LA_FAST(false, false, true);
  else if (a.silu)
    LA_FAST(false, true, false);
  else
    LA_FAST(false, false, false);
#undef LA_FAST
}

template <typename TIn, typename TOut, int D, int BLK>
static hipError_t launch_output_t(const PrefillArgs& a, hipStream_t st) {
  // SiLU and the epilogue: block-64 bf16 kernels only, the epilogue forward only
  if ((a.silu || a.epi) && !(BLK == 64 && sizeof(TIn) == 2)) return hipErrorInvalidValue;
  if (a.epi && a.rev) return hipErrorInvalidValue;
  const int BH = (int)(a.B * a.H);
  const int nc = a.nc;
  const bool timed = !a.warm_start && !a.rerun;
  if (timed && a.evt_begin) {
    hipError_t e = hipEventRecord((hipEvent_t)a.evt_begin, st);
    if (e != hipSuccess) return e;
  }
  if constexpr (BLK == 64 && sizeof(TIn) == 2)
    launch_fast<TOut, D, kFromStart>(a, st);
  else if (a.rev) {
    // the backward's reverse passes reach the general kernel with fp32 inputs at block 64 only
    if constexpr (BLK == 64 && sizeof(TIn) == 4)
      hipLaunchKernelGGL((la_chunk_output<TIn, TOut, D, BLK, true>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                         (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, (TOut*)a.out, (const float*)a.tbl,
                         (const float*)a.states, (int)a.H, (int)a.N, (int)a.L, nc, a.tbl_stride);
    else
      return hipErrorInvalidValue;
  } else
    hipLaunchKernelGGL((la_chunk_output<TIn, TOut, D, BLK, false>), dim3((unsigned)(BH * nc)), dim3(D * 2), 0, st,
                       (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, (TOut*)a.out, (const float*)a.tbl,
                       (const float*)a.states, (int)a.H, (int)a.N, (int)a.L, nc, a.tbl_stride);
  if (timed && a.evt_end) {
    hipError_t e = hipEventRecord((hipEvent_t)a.evt_end, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

template <typename TOut, int D>
static hipError_t launch_mixed_t(const PrefillArgs& a, hipStream_t st) {
  if (a.evt_begin) {
    hipError_t e = hipEventRecord((hipEvent_t)a.evt_begin, st);
    if (e != hipSuccess) return e;
  }
  const int n_warm = (int)(a.B * a.H * a.nc_warm);
  const unsigned grid = (unsigned)(n_warm + a.B * a.H * a.nc);
  const Operands p0 = operands_of(a);
#define LA_MIXED(SILU, EPI)                                                                                   \
  hipLaunchKernelGGL((la_chunk_output64_mixed<TOut, D, SILU, EPI>), dim3(grid), dim3(D * 2), 0, st, p0, a.decay, \
                     (const float*)a.tbl, (int)a.H, (int)a.N, (int)a.L, a.nc, (int)a.L_warm, a.nc_warm,        \
                     a.tbl_stride, a.slots, a.num_slots, n_warm)
  if (a.epi && a.silu)
    LA_MIXED(true, true);
  else if (a.epi)
    LA_MIXED(false, true);
  else if (a.silu)
    LA_MIXED(true, false);
  else
    LA_MIXED(false, false);
#undef LA_MIXED
  if (a.evt_end) {
    hipError_t e = hipEventRecord((hipEvent_t)a.evt_end, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

template <typename TOut, int D>
static void launch_mixed_pair_t(const PrefillArgs& a, const PrefillArgs& b, hipStream_t st) {
  const int half = 1 << kPairShift;
  const int nblk_w = (int)(a.B * a.H * a.nc_warm), nblk_c = (int)(a.B * a.H * a.nc);
  const int n_warm_grid = (nblk_w + half - 1) / half * 2 * half;
  const unsigned grid = (unsigned)(n_warm_grid + (nblk_c + half - 1) / half * 2 * half);
  hipLaunchKernelGGL((la_chunk_output64_mixed_pair<TOut, D>), dim3(grid), dim3(D * 2), 0, st, operands_of(a),
                     operands_of(b), a.decay, (const float*)a.tbl, (int)a.H, (int)a.N, (int)a.L, a.nc,
                     (int)a.L_warm, a.nc_warm, a.tbl_stride, nblk_w, nblk_c, n_warm_grid);
}

hipError_t launch_mixed_pair(const PrefillArgs& a, const PrefillArgs& b, hipStream_t st) {
  if (!a.warm_start || !a.rev || a.silu || a.epi || b.epi || a.in_dtype != kBF16 || a.block != 64 || b.in_dtype != kBF16 ||
      b.block != 64 || a.B != b.B || a.H != b.H || a.N != b.N || a.nc != b.nc || a.d != b.d ||
      a.out_dtype != b.out_dtype || a.rev != b.rev || a.warm_start != b.warm_start || a.silu != b.silu ||
      a.L != b.L || a.L_warm != b.L_warm)
    return hipErrorInvalidValue;
  if (a.out_dtype == kBF16) {
    if (a.d == 128) launch_mixed_pair_t<bf16, 128>(a, b, st);
    else launch_mixed_pair_t<bf16, 64>(a, b, st);
  } else {
    if (a.d == 128) launch_mixed_pair_t<float, 128>(a, b, st);
    else launch_mixed_pair_t<float, 64>(a, b, st);
  }
  return hipGetLastError();
}

hipError_t launch_mixed_pass(const PrefillArgs& a, hipStream_t st) {
  if (!a.warm_start || a.rev || a.in_dtype != kBF16 || a.block != 64) return hipErrorInvalidValue;
  if (a.out_dtype == kBF16) return a.d == 128 ? launch_mixed_t<bf16, 128>(a, st) : launch_mixed_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_mixed_t<float, 128>(a, st) : launch_mixed_t<float, 64>(a, st);
}


template <typename TIn, typename TOut, int D>
static hipError_t launch_output_d(const PrefillArgs& a, hipStream_t st) {
  switch (a.block) {
    case 64: return launch_output_t<TIn, TOut, D, 64>(a, st);
    case 128: return launch_output_t<TIn, TOut, D, 128>(a, st);
    case 256: return launch_output_t<TIn, TOut, D, 256>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t launch_pair_mode(const PrefillArgs& a, const PrefillArgs& b, hipStream_t st) {
  if (a.epi || b.epi) return hipErrorInvalidValue;
  if (a.in_dtype != kBF16 || b.in_dtype != kBF16 || a.block != 64 || b.block != 64 || a.B != b.B || a.H != b.H ||
      a.N != b.N || a.nc != b.nc || a.d != b.d || a.out_dtype != b.out_dtype || a.rev != b.rev ||
      a.warm_start != b.warm_start || a.silu != b.silu || a.L != b.L || a.L_warm != b.L_warm)
    return hipErrorInvalidValue;
  if (MODE == kWarmStart && !a.warm_start) return hipErrorInvalidValue;
  if (a.out_dtype == kBF16) {
    if (a.d == 128) launch_fast<bf16, 128, MODE>(a, st, &b);
    else launch_fast<bf16, 64, MODE>(a, st, &b);
  } else {
    if (a.d == 128) launch_fast<float, 128, MODE>(a, st, &b);
    else launch_fast<float, 64, MODE>(a, st, &b);
  }
  return hipGetLastError();
}

hipError_t launch_output_pair(const PrefillArgs& a, const PrefillArgs& b, hipStream_t st) {
  return launch_pair_mode<kFromStart>(a, b, st);
}

hipError_t launch_output_pass(const PrefillArgs& a, hipStream_t st) {
  if (a.in_dtype == kBF16 && a.out_dtype == kBF16)
    return a.d == 128 ? launch_output_d<bf16, bf16, 128>(a, st) : launch_output_d<bf16, bf16, 64>(a, st);
  if (a.in_dtype == kBF16 && a.out_dtype == kF32)
    return a.d == 128 ? launch_output_d<bf16, float, 128>(a, st) : launch_output_d<bf16, float, 64>(a, st);
  if (a.d == 128) return launch_output_t<float, float, 128, 64>(a, st);
  return launch_output_d<float, float, 64>(a, st);
}

}  // namespace la
