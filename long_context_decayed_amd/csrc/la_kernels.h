// Host-side interface between the C ABI (la_abi.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

enum { kBF16 = 0, kF32 = 1 };

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* decay;
  void* out;
  const float* kv_in;
  float* kv_out;
  int64_t B, H, N, d, block, L;
  int nc;          // number of chunks, ceil(N / L)
  int in_dtype, out_dtype;
  float* tbl;      // workspace: [H][tbl_stride] decay powers
  int tbl_stride;  // >= block + 1
  float* states;   // workspace: [B*H][nc][d][d]
  void* evt_begin; // optional hipEvent_t around the output kernel
  void* evt_end;
};

// Passes A and B (decay table, chunk aggregates, chunk scan): la_state.hip.
hipError_t launch_state_passes(const PrefillArgs& a, hipStream_t st);
// Pass C (outputs), with the optional timing events around it: la_output.hip.
hipError_t launch_output_pass(const PrefillArgs& a, hipStream_t st);

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* decay, void* out,
                         const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t d, hipStream_t st);

}  // namespace la
