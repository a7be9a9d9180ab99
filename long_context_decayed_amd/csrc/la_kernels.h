// Host-side interface between the C ABI (la_abi.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

enum { kBF16 = 0, kF32 = 1 };

// Floats per (bh, warm-start chunk) slot of the warm-start check: the
// per-wave largest |S| of the state just before the next chunk's warm-up
// window ([0, 4)) and of the state the chunk's own warm-up builds ([4, 8)).
constexpr int kGuardSlots = 8;

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
  int64_t L_warm;  // chunk of the warm-start pass (>= L); which heads decay within a chunk is judged by it
  int nc_warm;     // ceil(N / L_warm)
  int in_dtype, out_dtype;
  float* tbl;      // workspace: [H][tbl_stride] decay powers
  int tbl_stride;  // >= block + 1
  float* states;   // workspace: [B*H][nc][d][d]
  bool warm_start; // bf16 inputs, block 64: decaying heads take the warm-start pass
  bool rev;        // tokens last first, kv_in entering undecayed (backward; bf16, block 64 only)
  bool scale_kv_out; // kv_out = lam * final state (backward: gradient of kv_in)
  bool silu;         // q, k, v are pre-activations: SiLU applied as tiles load (bf16, block 64, forward only)
  const int* slots;  // optional slot table: kv_in / kv_out rows of pool slots (device int32[B])
  int64_t num_slots;
  void* evt_begin; // optional hipEvent_t pair around the kernel that writes every output row
  void* evt_end;
  // Warm-start check (forward passes with warm_start): guard, kGuardSlots
  // floats per (bh, warm-start chunk), written by the warm-start chunks;
  // flags, one int per bh, set by the check for the heads whose warm start
  // left out a state that is not negligible.  Null: no check.
  float* guard;
  int* flags;
  bool rerun;      // run only the heads whose flag is set, on the exact path
  // Epilogue (forward, bf16 inputs, block 64): out = RMSNorm_head(o) *
  // gamma[h] * sigmoid(gate) in the kernels that write the output rows;
  // gamma [H][d] or null (no norm), gate [B][H][N][d] bf16 or null (no gate).
  bool epi;
  const float* gamma;
  float eps;
  const void* gate;
};

// Decay table and pass A (chunk aggregates; with warm_start, of the heads
// that do not decay within their chunk only): la_state.hip.
hipError_t launch_aggregate_pass(const PrefillArgs& a, hipStream_t st);
// Pass B (chunk scan: start states, final state; with warm_start, the
// decaying heads' final states are only copied out); part 0 every head, 1 the
// scan of the other heads only, 2 the decaying heads' copy only (those whose
// flag is set excepted), 3 the scan of the flagged heads only: la_state.hip.
hipError_t launch_scan_pass(const PrefillArgs& a, hipStream_t st, int part = 0);
// The warm-start check: flags[bh] = 1 for a decaying head when some chunk's
// warm-up window left out a state above 2^-24 of the state it starts from;
// the decaying heads that pass it have their final states copied to kv_out
// (the work of scan part 2 for them) (la_state.hip).
hipError_t launch_warm_guard(const PrefillArgs& a, hipStream_t st);
// Pass C (outputs from the chunk start states; with warm_start, of the
// heads that do not decay within their chunk only): la_output.hip.
hipError_t launch_output_pass(const PrefillArgs& a, hipStream_t st);
// The warm-start pass and pass C in one launch (warm_start, forward only):
// every output row, and the decaying heads' final states; after pass B of the
// other heads.  Timing events bracket it: la_output.hip.
hipError_t launch_mixed_pass(const PrefillArgs& a, hipStream_t st);
// The same for two reverse-time problems of one shape paired as in
// launch_output_pair (the backward's dK and dV passes): la_output.hip.
hipError_t launch_mixed_pair(const PrefillArgs& a, const PrefillArgs& b, hipStream_t st);

// Two problems of one shape (bf16 inputs, block 64) in one grid, the two
// workgroups of each (bh, chunk) side by side, so that tensors both read
// are fetched from HBM about once: pass C of a and b (without the warm
// start; with it, launch_mixed_pair).  Each problem has its own tensors and
// chunk states; flags, decays and the decay table are a's: la_output.hip.
hipError_t launch_output_pair(const PrefillArgs& a, const PrefillArgs& b, hipStream_t st);

// dst[bh] = src[bh]^T for BH fp32 d x d states: la_state.hip.
hipError_t launch_transpose_states(const float* src, float* dst, int64_t BH, int64_t d, hipStream_t st);

// Optional elementwise steps fused into the decode step: SiLU on q, k, v;
// per-head RMSNorm of o (gamma [H][d], eps); o * sigmoid(gate), gate bf16 [B][H][d].
struct DecodeFusion {
  int silu;
  const float* gamma;
  float eps;
  const void* gate;
};

// Decode step (la_decode.hip); with `slots` (device int32[B]) batch row b uses
// state row slots[b] of kv_in / kv_out ([num_slots][H][d][d]); rows whose slot
// is out of range are idle.  num_layers > 1: q, k, v, out are
// [num_layers][B][H][d], decay [num_layers][H], gamma [num_layers][H][d],
// slots [num_layers][B] and the states [num_layers][num_slots][H][d][d] (row b
// of a layer without a slot table uses its pool row b).
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* decay, void* out,
                         const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t d, hipStream_t st,
                         const int* slots = nullptr, int64_t num_slots = 0, const DecodeFusion* fz = nullptr,
                         int64_t num_layers = 1);

// Per-head RMSNorm of o (bf16 or fp32 [rows][d], rows = B*H*N, head of a row =
// (row / N) % H) times gamma [H][d] when given, times sigmoid(gate) when given
// (bf16 [rows][d]), into bf16 out (may be o itself when o is bf16): la_fused.hip.
hipError_t launch_norm_gate(const void* o, int o_dtype, const void* gate, const float* gamma, float eps, void* out,
                            int64_t rows, int64_t H, int64_t N, int64_t d, hipStream_t st);
// x <- x * sigmoid(x) over n bf16 elements in place: la_fused.hip.
hipError_t launch_silu(void* x, int64_t n, hipStream_t st);

}  // namespace la
