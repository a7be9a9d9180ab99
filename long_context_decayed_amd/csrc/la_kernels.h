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
  bool warm_start; // bf16 inputs, block 64: decaying heads take the warm-start pass
  bool rev;        // tokens last first, kv_in entering undecayed (backward; bf16, block 64 only)
  bool scale_kv_out; // kv_out = lam * final state (backward: gradient of kv_in)
  const int* slots;  // optional slot table: kv_in / kv_out rows of pool slots (device int32[B])
  int64_t num_slots;
  void* evt_begin; // optional hipEvent_t pair around the kernel that writes every output row
  void* evt_end;
};

// Decay table and pass A (chunk aggregates; with warm_start, of the heads
// that do not decay within their chunk only): la_state.hip.
hipError_t launch_aggregate_pass(const PrefillArgs& a, hipStream_t st);
// Warm-start output pass of the decaying heads (every output row and their
// final state); only with warm_start: la_output.hip.
hipError_t launch_warm_start_pass(const PrefillArgs& a, hipStream_t st);
// Pass B (chunk scan: start states, final state; with warm_start, the
// decaying heads' final states are only copied out): la_state.hip.
hipError_t launch_scan_pass(const PrefillArgs& a, hipStream_t st);
// Pass C (outputs from the chunk start states; with warm_start, of the
// heads that do not decay within their chunk only): la_output.hip.
hipError_t launch_output_pass(const PrefillArgs& a, hipStream_t st);

// Decode step; with `slots` (device int32[B]) batch row b uses state row
// slots[b] of kv_in / kv_out ([num_slots][H][d][d]); rows out of range idle.
// dst[bh] = src[bh]^T for BH fp32 d x d states: la_state.hip.
hipError_t launch_transpose_states(const float* src, float* dst, int64_t BH, int64_t d, hipStream_t st);

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* decay, void* out,
                         const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t d, hipStream_t st,
                         const int* slots = nullptr, int64_t num_slots = 0);

}  // namespace la
