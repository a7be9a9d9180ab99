// Decode step of causal decayed linear attention for gfx950: for every
// (sequence, head) pair, S <- lam S + k^T v and o = q S (the one-token case
// of the recurrence; the MiniMax-M1 fact sheet (archdb), "linear / SSM layer
// configuration" field, gives the fixed per-head decay and the d x d state).
//
// The step is bound by HBM: each pair streams its fp32 d x d state in and
// back out (2 * 4 * d^2 bytes) against 4 d^2 flops.  One workgroup of 256
// threads per pair; thread (rg, cg) owns 4 consecutive value columns
// [4cg, 4cg + 4) of rows rg, rg + RG, ...; a wave reads whole 512-byte rows,
// so every access is a coalesced 16-byte load or store that bypasses the
// caches (the state is touched once per step).  The products k[i] v[j] of
// two bf16 values are exact in fp32; o is reduced over the RG row groups in
// LDS in a fixed order and rounded once to bf16.

#include <hip/hip_runtime.h>

#include "la_device.h"
#include "la_kernels.h"

namespace la {

template <int D>
__global__ __launch_bounds__(256) void la_decode_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                        const bf16* __restrict__ v,
                                                        const float* __restrict__ decay, bf16* __restrict__ o,
                                                        const float* kv_in, float* kv_out, int H) {
  constexpr int TPR = D / 4;       // threads per row
  constexpr int RG = 256 / TPR;    // row groups
  constexpr int RPT = D / RG;      // rows per thread
  __shared__ float qs[D], ks[D];
  __shared__ f32x4 part[RG][TPR];

  const int tid = threadIdx.x;
  const int64_t pair = blockIdx.x;
  const int cg = tid % TPR, rg = tid / TPR;
  const float lam = decay[pair % H];
  if (tid < D) {
    qs[tid] = (float)q[pair * D + tid];
    ks[tid] = (float)k[pair * D + tid];
  }
  f32x4 vv;
  {
    const bf16x4 vb = *reinterpret_cast<const bf16x4*>(v + pair * D + 4 * cg);
    vv = f32x4{(float)vb[0], (float)vb[1], (float)vb[2], (float)vb[3]};
  }
  const int64_t sbase = pair * D * D;
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    if (kv_in)
      s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kv_in + sbase + (int64_t)(rg + RG * i) * D) + cg);
    else
      s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    s[i] = lam * s[i] + ks[row] * vv;
    acc += qs[row] * s[i];
  }
  if (kv_out) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(kv_out + sbase + (int64_t)(rg + RG * i) * D) + cg);
  }
  part[rg][cg] = acc;
  __syncthreads();
  if (tid < TPR) {
    f32x4 r = part[0][tid];
#pragma unroll
    for (int g = 1; g < RG; ++g) r += part[g][tid];
    bf16x4 ob;
#pragma unroll
    for (int i = 0; i < 4; ++i) ob[i] = (bf16)r[i];
    *reinterpret_cast<bf16x4*>(o + pair * D + 4 * tid) = ob;
  }
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* decay, void* out,
                         const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t d, hipStream_t st) {
  const unsigned pairs = (unsigned)(B * H);
  if (d == 128)
    hipLaunchKernelGGL(la_decode_kernel<128>, dim3(pairs), dim3(256), 0, st, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, decay, (bf16*)out, kv_in, kv_out, (int)H);
  else
    hipLaunchKernelGGL(la_decode_kernel<64>, dim3(pairs), dim3(256), 0, st, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, decay, (bf16*)out, kv_in, kv_out, (int)H);
  return hipGetLastError();
}

}  // namespace la
