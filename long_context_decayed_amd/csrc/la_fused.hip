// Elementwise steps either side of the lightning-attention core, as
// standalone passes for the prefill: SiLU on Q, K, V (prologue) and the
// per-head RMSNorm and sigmoid gate of the output (epilogue).  The MiniMax-M1
// fact sheet (archdb) places them in its "linear / SSM layer configuration"
// field (SiLU on Q, K, V; RMSNorm on the output) and its "output gate" field
// (a sigmoid gate after that norm, before the output projection).
//
// The block-64 prefill kernels can also apply SiLU to the tiles as they load
// them and the norm and gate in the path that stores the output rows
// (la_output.hip, la_state.hip; the same silu_hw and sigmoid_hw, so the
// results agree bit for bit with these passes); these passes serve the other
// prefill forms (blocks 128 and 256, fp32 inputs) and callers that want the
// steps on their own.  The decode step fuses all of them (la_decode.hip).  Both passes here are bound by HBM: 16-byte
// non-temporal loads and stores (the data is touched once), one row of d
// features per d/8 lanes, the row's sum of squares reduced across those lanes.

#include <hip/hip_runtime.h>

#include "la_device.h"
#include "la_kernels.h"

namespace la {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// y = o / sqrt(mean(o^2) + eps) * gamma[h] * sigmoid(g) per row of d features.
// Each lane group of TPR lanes handles RU rows, 256/TPR*RU rows per block; all
// loads of a thread are issued before any arithmetic.
template <typename TO, int D>
__global__ __launch_bounds__(256) void la_norm_gate(const TO* __restrict__ o, const bf16* __restrict__ gate,
                                                    const float* __restrict__ gamma, float eps, bf16* out,
                                                    int64_t rows, int H, int64_t N) {
  constexpr int TPR = D / 8, RPB = 256 / TPR, RU = 4;
  const int part = threadIdx.x % TPR;
  const int64_t row0 = (int64_t)blockIdx.x * RPB * RU + threadIdx.x / TPR;
  float x[RU][8];
  bf16x8 gv[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int64_t row = row0 + (int64_t)u * RPB;
    if (row < rows) {
      const TO* src = o + row * D + 8 * part;
      if constexpr (sizeof(TO) == 2) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src)));
#pragma unroll
        for (int i = 0; i < 8; ++i) x[u][i] = (float)b[i];
      } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[u][i] = a[i];
          x[u][4 + i] = b[i];
        }
      }
      if (gate)
        gv[u] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gate + row * D + 8 * part)));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int64_t row = row0 + (int64_t)u * RPB;
    if (gamma) {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[u][i] * x[u][i];
#pragma unroll
      for (int m = TPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, TPR);
      const float inv = 1.0f / sqrtf(ss / (float)D + eps);
      if (row < rows) {
        const int hh = (int)((row / N) % H);
        const float* gm = gamma + (int64_t)hh * D + 8 * part;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[u][i] *= inv * gm[i];
      }
    }
    if (row < rows) {
      if (gate)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[u][i] *= sigmoid_hw((float)gv[u][i]);
      bf16x8 y;
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = (bf16)x[u][i];
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, y), reinterpret_cast<u32x4*>(out + row * D + 8 * part));
    }
  }
}

// x <- x * sigmoid(x): 4 chunks of 8 bf16 elements per thread, all loads
// issued before any arithmetic.
__global__ __launch_bounds__(256) void la_silu(bf16* __restrict__ x, int64_t n8, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * blockDim.x * 4 + threadIdx.x;
  bf16x8 b[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = base + u * 256;
    if (i < n8) b[u] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + 8 * i)));
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = base + u * 256;
    if (i < n8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = (float)b[u][j];
        b[u][j] = (bf16)silu_hw(f);
      }
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, b[u]), reinterpret_cast<u32x4*>(x + 8 * i));
    }
  }
  // a tail of n % 8 elements, one thread
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t j = 8 * n8; j < n; ++j) {
      const float f = (float)x[j];
      x[j] = (bf16)silu_hw(f);
    }
}

hipError_t launch_norm_gate(const void* o, int o_dtype, const void* gate, const float* gamma, float eps, void* out,
                            int64_t rows, int64_t H, int64_t N, int64_t d, hipStream_t st) {
  const int64_t rows_per_block = (256 / (d / 8)) * 4;
  const unsigned grid = (unsigned)((rows + rows_per_block - 1) / rows_per_block);
  if (o_dtype == kBF16) {
    if (d == 128)
      hipLaunchKernelGGL((la_norm_gate<bf16, 128>), dim3(grid), dim3(256), 0, st, (const bf16*)o, (const bf16*)gate,
                         gamma, eps, (bf16*)out, rows, (int)H, N);
    else
      hipLaunchKernelGGL((la_norm_gate<bf16, 64>), dim3(grid), dim3(256), 0, st, (const bf16*)o, (const bf16*)gate,
                         gamma, eps, (bf16*)out, rows, (int)H, N);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((la_norm_gate<float, 128>), dim3(grid), dim3(256), 0, st, (const float*)o,
                         (const bf16*)gate, gamma, eps, (bf16*)out, rows, (int)H, N);
    else
      hipLaunchKernelGGL((la_norm_gate<float, 64>), dim3(grid), dim3(256), 0, st, (const float*)o,
                         (const bf16*)gate, gamma, eps, (bf16*)out, rows, (int)H, N);
  }
  return hipGetLastError();
}

hipError_t launch_silu(void* x, int64_t n, hipStream_t st) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 1023) / 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(la_silu, dim3((unsigned)blocks), dim3(256), 0, st, (bf16*)x, n8, n);
  return hipGetLastError();
}

}  // namespace la
