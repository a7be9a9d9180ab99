// Decode step of causal decayed linear attention for gfx950: for every
// (sequence, head) pair, S <- lam S + k^T v and o = q S (the one-token case
// of the recurrence; the MiniMax-M1 fact sheet (archdb), "linear / SSM layer
// configuration" field, gives the fixed per-head decay and the d x d state).
//
// The step is bound by HBM: each pair streams its fp32 d x d state in and
// back out (2 * 4 * d^2 bytes) against 4 d^2 flops.  A workgroup serves two
// pairs with 128 threads each; thread (rg, cg) of a pair owns 4 consecutive
// value columns [4cg, 4cg + 4) of rows rg, rg + RG, ... (32 rows at d = 128),
// so every thread keeps 32 16-byte non-temporal loads in flight and a wave
// covers whole contiguous rows.  (Measured on MI355X: 128 threads x 2 pairs
// per workgroup moves the state at ~6.1 TB/s against ~5.5 TB/s for 256
// threads x 1 pair.)  The products k[i] v[j] of two bf16 values are exact in
// fp32; o is reduced over the RG row groups in LDS in a fixed order and
// rounded once to bf16.
//
// Serving form: with a slot table, batch row b reads and writes the state of
// pool slot slots[b] (states [num_slots][H][d][d], in place); a row whose
// slot lies outside [0, num_slots) is idle: its output is zero and no state
// is touched.
//
// Several layers in one launch: rows are grouped by layer (rows_per_layer
// rows each, layer-major), and each layer has its own decays ([layer][H]),
// state pool ([layer][num_slots][H][d][d]), slot table rows and norm weights,
// so a serving loop can step every lightning layer's ready tokens at once
// (for example requests pipelined across layers).  A single-layer call is
// the case rows_per_layer = B.
//
// Fused form (the layer's elementwise steps either side of the core; the
// MiniMax-M1 fact sheet, "linear / SSM layer configuration" and "output gate"
// fields): SiLU on q, k, v as they are read; per-head RMSNorm of o over its d
// features, o / sqrt(mean(o^2) + eps) * gamma[h]; then o * sigmoid(gate).
// Each is optional; the row of o is whole in the threads that store it, so
// they add no memory pass.

#include <hip/hip_runtime.h>

#include "la_device.h"
#include "la_kernels.h"

namespace la {

constexpr int kDecThreads = 128;  // threads per (sequence, head) pair
constexpr int kDecPairs = 2;      // pairs per workgroup

template <int D>
__global__ __launch_bounds__(kDecThreads * kDecPairs) void la_decode_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ decay, bf16* __restrict__ o, const float* kv_in, float* kv_out, int H, int64_t pairs,
    const int* __restrict__ slots, int64_t num_slots, int silu, const float* __restrict__ gamma, float eps,
    const bf16* __restrict__ gate, int64_t rows_per_layer) {
  constexpr int TPR = D / 4;              // threads per row
  constexpr int RG = kDecThreads / TPR;   // row groups
  constexpr int RPT = D / RG;             // rows per thread
  __shared__ float qs[kDecPairs][D], ks[kDecPairs][D];
  __shared__ f32x4 part[kDecPairs][RG][TPR];

  const int sub = threadIdx.x / kDecThreads, tid = threadIdx.x % kDecThreads;
  const int64_t pair = (int64_t)blockIdx.x * kDecPairs + sub;
  bool valid = pair < pairs;  // no early return: every thread reaches the barriers
  const int cg = tid % TPR, rg = tid / TPR;
  const int64_t b = pair / H, hh = pair - (pair / H) * H;
  const int64_t layer = b / rows_per_layer;  // 0 for a single-layer call
  const int64_t lh = layer * H + hh;         // this pair's (layer, head): decay and norm weights
  // state row of this pair within the layer's pool: the row itself, or its slot
  int64_t srow = b - layer * rows_per_layer;
  bool idle = false;
  if (slots && valid) {
    srow = slots[b];
    idle = srow < 0 || srow >= num_slots;
    valid = !idle;
  }
  srow += layer * num_slots;  // the layer's pool (num_slots rows each)
  const float lam = valid ? decay[lh] : 0.0f;
  if (valid && tid < D) {
    const float qf = (float)q[pair * D + tid], kf = (float)k[pair * D + tid];
    qs[sub][tid] = silu ? silu_hw(qf) : qf;
    ks[sub][tid] = silu ? silu_hw(kf) : kf;
  }
  f32x4 vv = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const bf16x4 vb = *reinterpret_cast<const bf16x4*>(v + pair * D + 4 * cg);
    vv = f32x4{(float)vb[0], (float)vb[1], (float)vb[2], (float)vb[3]};
    if (silu)
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = silu_hw(vv[i]);
  }
  const int64_t sbase = (srow * H + hh) * D * D;
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    if (valid && kv_in)
      s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kv_in + sbase + (int64_t)(rg + RG * i) * D) + cg);
    else
      s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    s[i] = lam * s[i] + ks[sub][row] * vv;
    acc += qs[sub][row] * s[i];
  }
  if (valid && kv_out) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(kv_out + sbase + (int64_t)(rg + RG * i) * D) + cg);
  }
  part[sub][rg][cg] = acc;
  __syncthreads();
  if ((valid || idle) && tid < TPR) {
    f32x4 r = part[sub][0][tid];
#pragma unroll
    for (int g = 1; g < RG; ++g) r += part[sub][g][tid];
    if (gamma) {
      // the TPR lanes of this group hold the whole row: reduce across them
      float ss = r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
#pragma unroll
      for (int m = TPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, TPR);
      const float inv = 1.0f / sqrtf(ss / (float)D + eps);
      const f32x4 gm = *reinterpret_cast<const f32x4*>(gamma + lh * D + 4 * tid);
      r = r * inv * gm;
    }
    if (gate) {
      const bf16x4 gb = *reinterpret_cast<const bf16x4*>(gate + pair * D + 4 * tid);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] *= sigmoid_hw((float)gb[i]);
    }
    bf16x4 ob;
#pragma unroll
    for (int i = 0; i < 4; ++i) ob[i] = idle ? (bf16)0.0f : (bf16)r[i];
    *reinterpret_cast<bf16x4*>(o + pair * D + 4 * tid) = ob;
  }
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* decay, void* out,
                         const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t d, hipStream_t st,
                         const int* slots, int64_t num_slots, const DecodeFusion* fz, int64_t num_layers) {
  const int silu = fz ? fz->silu : 0;
  const float* gamma = fz ? fz->gamma : nullptr;
  const float eps = fz ? fz->eps : 0.0f;
  const bf16* gate = fz ? (const bf16*)fz->gate : nullptr;
  const int64_t pairs = num_layers * B * H;
  // without a slot table a layer's rows use its first B pool rows
  const int64_t pool = (slots || num_layers > 1) ? num_slots : 0;
  const unsigned grid = (unsigned)((pairs + kDecPairs - 1) / kDecPairs);
  if (d == 128)
    hipLaunchKernelGGL(la_decode_kernel<128>, dim3(grid), dim3(kDecThreads * kDecPairs), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, decay, (bf16*)out, kv_in, kv_out, (int)H, pairs, slots,
                       pool, silu, gamma, eps, gate, B);
  else
    hipLaunchKernelGGL(la_decode_kernel<64>, dim3(grid), dim3(kDecThreads * kDecPairs), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, decay, (bf16*)out, kv_in, kv_out, (int)H, pairs, slots,
                       pool, silu, gamma, eps, gate, B);
  return hipGetLastError();
}

}  // namespace la
