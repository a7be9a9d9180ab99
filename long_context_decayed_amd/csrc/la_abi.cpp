// C ABI of the lightning-attention library: argument validation, chunk choice,
// workspace layout and the calls into the kernel launchers.  Every check runs
// before the first HIP call, so validation errors never touch the device.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/lightning_attn.h"
#include "la_kernels.h"

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 24;  // keeps N * d < 2^31 for per-head offsets
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxHeadTokens = int64_t(1) << 48;  // B * H * N: byte counts stay far inside int64

// Sizes the byte arithmetic below can hold: B, H and the row count (B * H,
// or num_slots * H for a state pool) below 2^31 each, B * H * N <= 2^48.
bool dims_fit(int64_t B, int64_t H, int64_t N, int64_t pool_rows = 0) {
  if (B > kMaxGrid || H > kMaxGrid || N > kMaxTokens || pool_rows > kMaxGrid) return false;
  if (B * H > kMaxGrid || pool_rows * H > kMaxGrid) return false;
  return B * H * N <= kMaxHeadTokens;
}

// dtype / head-dim / block combinations the kernels are built for.  fp32
// tiles are twice as large, so fp32 with d = 128 is limited to block 64 by
// the 160 KiB of LDS per CU.
bool prefill_supported(int in_dtype, int out_dtype, int64_t d, int64_t block) {
  if (d != 64 && d != 128) return false;
  if (block != 64 && block != 128 && block != 256) return false;
  if (in_dtype == LA_DTYPE_BF16) return out_dtype == LA_DTYPE_BF16 || out_dtype == LA_DTYPE_F32;
  if (in_dtype == LA_DTYPE_F32 && out_dtype == LA_DTYPE_F32) return d == 64 || block == 64;
  return false;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// An input and an output state tensor are either the same tensor (in place:
// every (b, h) state is read before it is written) or apart.
bool states_apart_or_same(const void* in, const void* out, int64_t bytes) {
  return in == out || !overlap(in, bytes, out, bytes);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_block(int64_t block) { return block == 64 || block == 128 || block == 256; }

// Default chunk: 16384 tokens, halved while the chunk-parallel passes would
// launch fewer than 2048 workgroups, never below a floor of N/8 (a power of
// two, clamped to [256, 1024], and at least the block), and never longer
// than the sequence rounded up to a whole block.
int64_t pick_chunk(int64_t B, int64_t H, int64_t N, int64_t block) {
  // Long chunks keep the chunk-state traffic small: each chunk moves four
  // d x d fp32 states through HBM across the three passes (at d = 128 and
  // 256 tokens as many bytes as q, k, v and o); enough of them keep four
  // rounds of resident workgroups (2 per CU) busy.  On short sequences the
  // state traffic weighs more than the extra rounds, hence the floor.
  int64_t L = 16384;
  int64_t floor_l = 256;
  while (floor_l < 1024 && 16 * floor_l <= N) floor_l *= 2;
  if (floor_l < block) floor_l = block;
  while (L > floor_l && B * H * ceil_div(N, L) < 2048) L /= 2;
  const int64_t cap = ceil_div(N, block) * block;
  if (L > cap) L = cap;
  return L;
}

// Default warm-start chunk: the scan's chunk L doubled up to twice (4L) while
// the warm-start pass keeps at least kResidentGroups workgroups (one full
// round at two per CU) and the chunk stays within the sequence.  Longer
// chunks let more heads take the warm start (a carry span up to half the
// chunk) and shorten its warm-up windows relative to the chunk, while the
// heads on the exact path keep the shorter chunks and the workgroups they
// need; fewer workgroups than one round would leave CUs idle.
constexpr int64_t kResidentGroups = 512;  // 256 CUs x 2 workgroups of the block-64 kernels

int64_t pick_warm_chunk(int64_t B, int64_t H, int64_t N, int64_t L) {
  int64_t Lw = L;
  const int64_t cap = ceil_div(N, L) * L;
  while (Lw < 4 * L && 2 * Lw <= kMaxTokens && 2 * Lw <= cap && B * H * ceil_div(N, 2 * Lw) >= kResidentGroups)
    Lw *= 2;
  return Lw;
}

int resolve_chunk(int64_t B, int64_t H, int64_t N, int64_t block, int64_t chunk, int64_t* L) {
  if (B < 1 || H < 1 || N < 1 || !valid_block(block)) return LA_ERR_INVALID;
  if (chunk == 0) {
    *L = pick_chunk(B, H, N, block);
  } else {
    if (chunk < 0 || chunk % block != 0 || chunk > kMaxTokens) return LA_ERR_INVALID;
    *L = chunk;
  }
  return LA_OK;
}

// The warm-start chunk for (chunk, warm_chunk): 0 takes the default (with
// chunk 0, pick_warm_chunk; with an explicit chunk, that chunk); otherwise a
// positive multiple of 64 (the warm-start kernels' block), at least L.
int resolve_warm_chunk(int64_t B, int64_t H, int64_t N, int64_t chunk, int64_t warm_chunk, int64_t L,
                       int64_t* Lw) {
  if (warm_chunk == 0) {
    *Lw = chunk == 0 ? pick_warm_chunk(B, H, N, L) : L;
    return LA_OK;
  }
  if (warm_chunk < L || warm_chunk % 64 != 0 || warm_chunk > kMaxTokens) return LA_ERR_INVALID;
  *Lw = warm_chunk;
  return LA_OK;
}

int64_t tbl_stride_for(int64_t block) { return ((block + 1 + 63) / 64) * 64; }

// Workspace: the decay-power table, the chunk states [B*H][nc][d][d], the
// warm-start check's slots (kGuardSlots floats per (bh, chunk); the
// warm-start chunks are never more than the scan's) and its flags (one int
// per bh), each part 256-byte aligned.
size_t workspace_layout(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block, int64_t L, size_t* tbl_bytes,
                        size_t* guard_off = nullptr, size_t* flags_off = nullptr) {
  const size_t tb = (size_t)H * (size_t)tbl_stride_for(block) * sizeof(float);
  const size_t tb_al = (tb + 255) / 256 * 256;
  const size_t nc = (size_t)ceil_div(N, L);
  const size_t bh = (size_t)B * (size_t)H;
  if (tbl_bytes) *tbl_bytes = tb_al;
  const size_t g = (tb_al + bh * nc * (size_t)d * (size_t)d * sizeof(float) + 255) / 256 * 256;
  const size_t f = (g + bh * nc * la::kGuardSlots * sizeof(float) + 255) / 256 * 256;
  if (guard_off) *guard_off = g;
  if (flags_off) *flags_off = f;
  return f + bh * sizeof(int);
}

int from_hip(hipError_t e) {
  if (e == hipSuccess) return LA_OK;
  if (e == hipErrorOutOfMemory) return LA_ERR_NOMEM;
  return LA_ERR_HIP;
}

int validate_prefill(const void* q, const void* k, const void* v, const float* decay, const void* out,
                     const float* kv_in, const float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                     int64_t block, int in_dtype, int out_dtype, int64_t chunk, int64_t* L) {
  if (!q || !k || !v || !decay || !out) return LA_ERR_INVALID;
  if (B < 1 || H < 1 || N < 1 || d < 1) return LA_ERR_INVALID;
  if (!valid_block(block)) return LA_ERR_INVALID;
  if ((in_dtype != LA_DTYPE_BF16 && in_dtype != LA_DTYPE_F32) ||
      (out_dtype != LA_DTYPE_BF16 && out_dtype != LA_DTYPE_F32))
    return LA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(decay, 4) ||
      !aligned(kv_in, 16) || !aligned(kv_out, 16))
    return LA_ERR_INVALID;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  if (!prefill_supported(in_dtype, out_dtype, d, block)) return LA_ERR_UNSUPPORTED;
  if (!dims_fit(B, H, N)) return LA_ERR_UNSUPPORTED;
  int rc = resolve_chunk(B, H, N, block, chunk, L);
  if (rc != LA_OK) return rc;
  if (B * H > kMaxGrid || B * H * ceil_div(N, *L) > kMaxGrid) return LA_ERR_UNSUPPORTED;
  const int64_t in_es = in_dtype == LA_DTYPE_BF16 ? 2 : 4, out_es = out_dtype == LA_DTYPE_BF16 ? 2 : 4;
  const int64_t in_bytes = B * H * N * d * in_es, out_bytes = B * H * N * d * out_es;
  const int64_t st_bytes = B * H * d * d * 4;
  const int64_t dec_bytes = H * 4;
  if (overlap(out, out_bytes, q, in_bytes) || overlap(out, out_bytes, k, in_bytes) ||
      overlap(out, out_bytes, v, in_bytes) || overlap(out, out_bytes, kv_in, st_bytes) ||
      overlap(out, out_bytes, kv_out, st_bytes) || overlap(out, out_bytes, decay, dec_bytes) ||
      !states_apart_or_same(kv_in, kv_out, st_bytes))
    return LA_ERR_INVALID;
  if (overlap(kv_out, st_bytes, q, in_bytes) || overlap(kv_out, st_bytes, k, in_bytes) ||
      overlap(kv_out, st_bytes, v, in_bytes) || overlap(kv_out, st_bytes, decay, dec_bytes))
    return LA_ERR_INVALID;
  return LA_OK;
}

// The kernels of one prefill-shaped pass, in order, on `st`.  Without the
// warm start: pass A, the scan, pass C.  With it (forward passes only; the
// backward's reverse passes use the paired launches): pass A and the scan of
// the heads that do not decay within a chunk, then one launch for every
// output row (the decaying heads' warm-start pass and the others' pass C side
// by side), then the decaying heads' final states copied out (after every
// chunk has read kv_in, which may be kv_out).
// With the warm-start check (a.guard and a.flags set), after the output
// launch the check flags the decaying heads whose warm start left out a
// state that is not negligible and copies out the others' final states (in
// place of that copy); the flagged heads are run again on the exact path
// (pass A, scan, pass C of the flagged heads only: three launches whose
// workgroups return at once when no head is flagged).
hipError_t run_passes(const la::PrefillArgs& a, hipStream_t st) {
  if (a.warm_start && a.rev) return hipErrorInvalidValue;
  hipError_t e = la::launch_aggregate_pass(a, st);
  if (a.warm_start) {
    if (e == hipSuccess) e = la::launch_scan_pass(a, st, 1);
    if (e == hipSuccess) e = la::launch_mixed_pass(a, st);
    const bool check = a.guard && a.flags;
    // the check also hands on the final states of the decaying heads that pass it
    if (e == hipSuccess) e = check ? la::launch_warm_guard(a, st) : la::launch_scan_pass(a, st, 2);
    if (check) {
      la::PrefillArgs r = a;
      r.warm_start = false;
      r.rerun = true;
      r.evt_begin = nullptr;
      r.evt_end = nullptr;
      if (e == hipSuccess) e = la::launch_aggregate_pass(r, st);
      if (e == hipSuccess) e = la::launch_scan_pass(r, st, 3);
      if (e == hipSuccess) e = la::launch_output_pass(r, st);
    }
    return e;
  }
  if (e == hipSuccess) e = la::launch_scan_pass(a, st);
  if (e == hipSuccess) e = la::launch_output_pass(a, st);
  return e;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// The epilogue of lightning_attn_fwd_fused (null: none).
struct Epilogue {
  const float* gamma;
  float eps;
  const void* gate;
};

int prefill_run(const void* q, const void* k, const void* v, const float* decay, void* out, const float* kv_in,
                float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t block, int in_dtype,
                int out_dtype, int64_t L, int64_t Lw, void* workspace, size_t workspace_bytes, void* evt_begin,
                void* evt_end, void* stream, const int* slots, int64_t num_slots, unsigned int flags,
                const Epilogue* epi = nullptr);

constexpr unsigned int kFwdFlags = LA_FLAG_EXACT | LA_FLAG_SILU_QKV;

// SiLU on the tiles is built into the block-64 bf16 kernels only.
bool flags_supported(unsigned int flags, int in_dtype, int64_t block) {
  return !(flags & LA_FLAG_SILU_QKV) || (in_dtype == LA_DTYPE_BF16 && block == 64);
}

}  // namespace

extern "C" {

int lightning_attn_fwd_ex(const void* q, const void* k, const void* v, const float* decay, void* out,
                          const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                          int64_t block, int in_dtype, int out_dtype, int64_t chunk, int64_t warm_chunk,
                          unsigned int flags, void* workspace, size_t workspace_bytes, void* evt_begin, void* evt_end,
                          void* stream) {
  if (flags & ~kFwdFlags) return LA_ERR_INVALID;
  int64_t L = 0, Lw = 0;
  int rc = validate_prefill(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, in_dtype, out_dtype, chunk, &L);
  if (rc != LA_OK) return rc;
  rc = resolve_warm_chunk(B, H, N, chunk, warm_chunk, L, &Lw);
  if (rc != LA_OK) return rc;
  if (!flags_supported(flags, in_dtype, block)) return LA_ERR_UNSUPPORTED;
  return prefill_run(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, in_dtype, out_dtype, L, Lw, workspace,
                     workspace_bytes, evt_begin, evt_end, stream, nullptr, 0, flags);
}

int lightning_attn_fwd_slots(const void* q, const void* k, const void* v, const float* decay, void* out,
                             float* states, const int32_t* slots, int64_t B, int64_t H, int64_t N, int64_t d,
                             int64_t num_slots, int64_t block, int in_dtype, int out_dtype, unsigned int flags,
                             void* stream) {
  if (flags & ~kFwdFlags) return LA_ERR_INVALID;
  if (!states || !slots || num_slots < 1) return LA_ERR_INVALID;
  if (!aligned(states, 16) || !aligned(slots, 4)) return LA_ERR_INVALID;
  if (!dims_fit(B, H, N, num_slots)) return LA_ERR_UNSUPPORTED;
  // validate the token tensors alone, then the pool against them
  int64_t L = 0;
  int rc = validate_prefill(q, k, v, decay, out, nullptr, nullptr, B, H, N, d, block, in_dtype, out_dtype, 0, &L);
  if (rc != LA_OK) return rc;
  if (!flags_supported(flags, in_dtype, block)) return LA_ERR_UNSUPPORTED;
  const int64_t in_es = in_dtype == LA_DTYPE_BF16 ? 2 : 4, out_es = out_dtype == LA_DTYPE_BF16 ? 2 : 4;
  const int64_t in_bytes = B * H * N * d * in_es, out_bytes = B * H * N * d * out_es;
  const int64_t pool_bytes = num_slots * H * d * d * 4;
  if (overlap(states, pool_bytes, q, in_bytes) || overlap(states, pool_bytes, k, in_bytes) ||
      overlap(states, pool_bytes, v, in_bytes) || overlap(states, pool_bytes, out, out_bytes) ||
      overlap(states, pool_bytes, slots, B * 4) || overlap(out, out_bytes, slots, B * 4) ||
      overlap(states, pool_bytes, decay, H * 4))
    return LA_ERR_INVALID;
  return prefill_run(q, k, v, decay, out, states, states, B, H, N, d, block, in_dtype, out_dtype, L,
                     pick_warm_chunk(B, H, N, L), nullptr, 0, nullptr, nullptr, stream, (const int*)slots, num_slots,
                     flags);
}

int lightning_attn_fwd_fused(const void* q, const void* k, const void* v, const float* decay, const float* gamma,
                             float eps, const void* gate, void* out, const float* kv_in, float* kv_out, int64_t B,
                             int64_t H, int64_t N, int64_t d, int out_dtype, int64_t chunk, int64_t warm_chunk,
                             unsigned int flags, void* workspace, size_t workspace_bytes, void* evt_begin,
                             void* evt_end, void* stream) {
  if (flags & ~kFwdFlags) return LA_ERR_INVALID;
  if (!(eps >= 0.0f) || eps > 1.0f) return LA_ERR_INVALID;
  if (!aligned(gamma, 16) || !aligned(gate, 16)) return LA_ERR_INVALID;
  int64_t L = 0, Lw = 0;
  int rc = validate_prefill(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, 64, LA_DTYPE_BF16, out_dtype, chunk, &L);
  if (rc != LA_OK) return rc;
  rc = resolve_warm_chunk(B, H, N, chunk, warm_chunk, L, &Lw);
  if (rc != LA_OK) return rc;
  const int64_t out_bytes = B * H * N * d * (out_dtype == LA_DTYPE_BF16 ? 2 : 4), gate_bytes = B * H * N * d * 2;
  const int64_t st_bytes = B * H * d * d * 4;
  if (overlap(out, out_bytes, gate, gate_bytes) || overlap(out, out_bytes, gamma, H * d * 4) ||
      overlap(kv_out, st_bytes, gate, gate_bytes) || overlap(kv_out, st_bytes, gamma, H * d * 4))
    return LA_ERR_INVALID;
  const Epilogue epi{gamma, eps, gate};
  return prefill_run(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, 64, LA_DTYPE_BF16, out_dtype, L, Lw, workspace,
                     workspace_bytes, evt_begin, evt_end, stream, nullptr, 0, flags, &epi);
}

}  // extern "C"

namespace {

int prefill_run(const void* q, const void* k, const void* v, const float* decay, void* out, const float* kv_in,
                float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t block, int in_dtype,
                int out_dtype, int64_t L, int64_t Lw, void* workspace, size_t workspace_bytes, void* evt_begin,
                void* evt_end, void* stream, const int* slots, int64_t num_slots, unsigned int flags,
                const Epilogue* epi) {
  const bool exact = (flags & LA_FLAG_EXACT) != 0;
  size_t tbl_bytes = 0, guard_off = 0, flags_off = 0;
  const size_t need = workspace_layout(B, H, N, d, block, L, &tbl_bytes, &guard_off, &flags_off);
  if (workspace) {
    if (workspace_bytes < need) return LA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return LA_ERR_INVALID;
    // the passes write the workspace: it may overlap none of the arguments
    const int64_t in_bytes = B * H * N * d * (in_dtype == LA_DTYPE_BF16 ? 2 : 4);
    const int64_t out_bytes = B * H * N * d * (out_dtype == LA_DTYPE_BF16 ? 2 : 4);
    const int64_t st_bytes = B * H * d * d * 4, wsb = (int64_t)need;
    if (overlap(workspace, wsb, q, in_bytes) || overlap(workspace, wsb, k, in_bytes) ||
        overlap(workspace, wsb, v, in_bytes) || overlap(workspace, wsb, out, out_bytes) ||
        overlap(workspace, wsb, kv_in, st_bytes) || overlap(workspace, wsb, kv_out, st_bytes) ||
        overlap(workspace, wsb, decay, H * 4))
      return LA_ERR_INVALID;
    if (epi && (overlap(workspace, wsb, epi->gamma, H * d * 4) || overlap(workspace, wsb, epi->gate, B * H * N * d * 2)))
      return LA_ERR_INVALID;
  }

  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (!ws) {
    hipError_t e = hipMallocAsync(&ws, need, st);
    if (e != hipSuccess) return e == hipErrorOutOfMemory ? LA_ERR_NOMEM : LA_ERR_HIP;
  }
  la::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.out = out;
  a.kv_in = kv_in;
  a.kv_out = kv_out;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.block = block;
  a.L = L;
  a.nc = (int)ceil_div(N, L);
  a.L_warm = Lw;
  a.nc_warm = (int)ceil_div(N, Lw);
  a.in_dtype = in_dtype == LA_DTYPE_BF16 ? la::kBF16 : la::kF32;
  a.out_dtype = out_dtype == LA_DTYPE_BF16 ? la::kBF16 : la::kF32;
  a.tbl = (float*)ws;
  a.tbl_stride = (int)tbl_stride_for(block);
  a.states = (float*)((char*)ws + tbl_bytes);
  a.warm_start = a.in_dtype == la::kBF16 && block == 64 && !exact;
  a.rev = false;
  a.scale_kv_out = false;
  a.silu = (flags & LA_FLAG_SILU_QKV) != 0;
  a.slots = slots;
  a.num_slots = num_slots;
  a.evt_begin = evt_begin;
  a.evt_end = evt_end;
  a.guard = a.warm_start ? (float*)((char*)ws + guard_off) : nullptr;
  a.flags = a.warm_start ? (int*)((char*)ws + flags_off) : nullptr;
  a.rerun = false;
  a.epi = epi != nullptr;
  a.gamma = epi ? epi->gamma : nullptr;
  a.eps = epi ? epi->eps : 0.0f;
  a.gate = epi ? epi->gate : nullptr;
  hipError_t e = run_passes(a, st);
  if (!workspace) {
    hipError_t f = hipFreeAsync(ws, st);
    if (e == hipSuccess) e = f;
  }
  return from_hip(e);
}

}  // namespace

extern "C" {

int lightning_attn_fwd(const void* q, const void* k, const void* v, const float* decay, void* out,
                       const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                       int64_t block, void* stream) {
  return lightning_attn_fwd_ex(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, LA_DTYPE_BF16,
                               LA_DTYPE_BF16, 0, 0, 0u, nullptr, 0, nullptr, nullptr, stream);
}

int lightning_attn_fwd_f32(const void* q, const void* k, const void* v, const float* decay, void* out,
                           const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N, int64_t d,
                           int64_t block, void* stream) {
  return lightning_attn_fwd_ex(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, LA_DTYPE_F32,
                               LA_DTYPE_F32, 0, 0, 0u, nullptr, 0, nullptr, nullptr, stream);
}

int lightning_attn_fwd_bf16_f32out(const void* q, const void* k, const void* v, const float* decay,
                                   void* out, const float* kv_in, float* kv_out, int64_t B, int64_t H,
                                   int64_t N, int64_t d, int64_t block, void* stream) {
  return lightning_attn_fwd_ex(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, LA_DTYPE_BF16,
                               LA_DTYPE_F32, 0, 0, 0u, nullptr, 0, nullptr, nullptr, stream);
}

// Backward workspace: the forward layout (decay table, chunk states of the
// first problem), chunk states of the second (the dK and dV passes run side by
// side), then the transposed S0 and dS_N.
size_t bwd_workspace_layout(int64_t B, int64_t H, int64_t N, int64_t d, int64_t L, size_t* states2_off,
                            size_t* s0t_off, size_t* dsnt_off) {
  size_t tbl_bytes = 0;
  const size_t fwd = align256(workspace_layout(B, H, N, d, 64, L, &tbl_bytes));
  const size_t states = align256(fwd - tbl_bytes);
  const size_t st = align256((size_t)(B * H * d * d) * sizeof(float));
  if (states2_off) *states2_off = fwd;
  if (s0t_off) *s0t_off = fwd + states;
  if (dsnt_off) *dsnt_off = fwd + states + st;
  return fwd + states + 2 * st;
}

size_t lightning_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || !dims_fit(B, H, N)) return 0;
  return bwd_workspace_layout(B, H, N, d, pick_chunk(B, H, N, 64), nullptr, nullptr, nullptr);
}

int lightning_attn_bwd(const void* q, const void* k, const void* v, const float* decay, const void* dout,
                       const float* kv_in, const float* dkv_out, void* dq, void* dk, void* dv, float* dkv_in,
                       int64_t B, int64_t H, int64_t N, int64_t d, int in_dtype, int out_dtype, unsigned int flags,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (flags & ~LA_FLAG_EXACT) return LA_ERR_INVALID;
  if (!q || !k || !v || !decay || !dout || !dq || !dk || !dv) return LA_ERR_INVALID;
  if (B < 1 || H < 1 || N < 1 || d < 1) return LA_ERR_INVALID;
  if ((in_dtype != LA_DTYPE_BF16 && in_dtype != LA_DTYPE_F32) ||
      (out_dtype != LA_DTYPE_BF16 && out_dtype != LA_DTYPE_F32))
    return LA_ERR_INVALID;
  const void* ptrs16[] = {q, k, v, dout, dq, dk, dv, kv_in, dkv_out, dkv_in};
  for (const void* p : ptrs16)
    if (!aligned(p, 16)) return LA_ERR_INVALID;
  if (!aligned(decay, 4)) return LA_ERR_INVALID;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  if (!prefill_supported(in_dtype, out_dtype, d, 64)) return LA_ERR_UNSUPPORTED;
  if (!dims_fit(B, H, N)) return LA_ERR_UNSUPPORTED;
  const int64_t L = pick_chunk(B, H, N, 64);
  if (B * H > kMaxGrid || B * H * ceil_div(N, L) > kMaxGrid) return LA_ERR_UNSUPPORTED;
  const int64_t in_bytes = B * H * N * d * (in_dtype == LA_DTYPE_BF16 ? 2 : 4);
  const int64_t out_bytes = B * H * N * d * (out_dtype == LA_DTYPE_BF16 ? 2 : 4);
  const int64_t st_bytes = B * H * d * d * 4;
  // outputs: apart from every input and from each other; dkv_in may be dkv_out itself
  const void* outs[] = {dq, dk, dv};
  const void* ins[] = {q, k, v, dout};
  for (const void* o : outs) {
    for (const void* i : ins)
      if (overlap(o, out_bytes, i, in_bytes)) return LA_ERR_INVALID;
    if (overlap(o, out_bytes, kv_in, st_bytes) || overlap(o, out_bytes, dkv_out, st_bytes) ||
        overlap(o, out_bytes, dkv_in, st_bytes))
      return LA_ERR_INVALID;
  }
  if (overlap(dq, out_bytes, dk, out_bytes) || overlap(dq, out_bytes, dv, out_bytes) ||
      overlap(dk, out_bytes, dv, out_bytes))
    return LA_ERR_INVALID;
  for (const void* o : outs)
    if (overlap(o, out_bytes, decay, H * 4)) return LA_ERR_INVALID;
  if (overlap(dkv_in, st_bytes, decay, H * 4)) return LA_ERR_INVALID;
  if (dkv_in && dkv_in != dkv_out) {
    for (const void* i : ins)
      if (overlap(dkv_in, st_bytes, i, in_bytes)) return LA_ERR_INVALID;
    if (overlap(dkv_in, st_bytes, kv_in, st_bytes) || overlap(dkv_in, st_bytes, dkv_out, st_bytes))
      return LA_ERR_INVALID;
  }
  size_t states2_off = 0, s0t_off = 0, dsnt_off = 0;
  const size_t need = bwd_workspace_layout(B, H, N, d, L, &states2_off, &s0t_off, &dsnt_off);
  if (workspace) {
    if (workspace_bytes < need) return LA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return LA_ERR_INVALID;
    const int64_t wsb = (int64_t)need;
    for (const void* i : ins)
      if (overlap(workspace, wsb, i, in_bytes)) return LA_ERR_INVALID;
    for (const void* o : outs)
      if (overlap(workspace, wsb, o, out_bytes)) return LA_ERR_INVALID;
    if (overlap(workspace, wsb, kv_in, st_bytes) || overlap(workspace, wsb, dkv_out, st_bytes) ||
        overlap(workspace, wsb, dkv_in, st_bytes) || overlap(workspace, wsb, decay, H * 4))
      return LA_ERR_INVALID;
  }

  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (!ws) {
    hipError_t e = hipMallocAsync(&ws, need, st);
    if (e != hipSuccess) return e == hipErrorOutOfMemory ? LA_ERR_NOMEM : LA_ERR_HIP;
  }
  size_t tbl_bytes = 0, guard_off = 0, flags_off = 0;
  workspace_layout(B, H, N, d, 64, L, &tbl_bytes, &guard_off, &flags_off);
  float* s0t = (float*)((char*)ws + s0t_off);
  float* dsnt = (float*)((char*)ws + dsnt_off);

  la::PrefillArgs a{};  // silu stays false: the backward takes activated inputs
  a.decay = decay;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.block = 64;
  a.L = L;
  a.nc = (int)ceil_div(N, L);
  a.L_warm = pick_warm_chunk(B, H, N, L);
  a.nc_warm = (int)ceil_div(N, a.L_warm);
  a.in_dtype = in_dtype == LA_DTYPE_BF16 ? la::kBF16 : la::kF32;
  a.out_dtype = out_dtype == LA_DTYPE_BF16 ? la::kBF16 : la::kF32;
  a.tbl = (float*)ws;
  a.tbl_stride = (int)tbl_stride_for(64);
  a.states = (float*)((char*)ws + tbl_bytes);
  a.warm_start = a.in_dtype == la::kBF16 && !(flags & LA_FLAG_EXACT);
  a.slots = nullptr;
  a.num_slots = 0;
  a.evt_begin = nullptr;
  a.evt_end = nullptr;
  // every pass takes the warm-start check (the dQ pass through run_passes,
  // the paired dK and dV passes below)
  a.guard = a.warm_start ? (float*)((char*)ws + guard_off) : nullptr;
  a.flags = a.warm_start ? (int*)((char*)ws + flags_off) : nullptr;
  a.rerun = false;
  a.epi = false;
  a.gamma = nullptr;
  a.eps = 0.0f;
  a.gate = nullptr;

  hipError_t e = hipSuccess;
  if (kv_in) e = la::launch_transpose_states(kv_in, s0t, B * H, d, st);
  if (e == hipSuccess && dkv_out) e = la::launch_transpose_states(dkv_out, dsnt, B * H, d, st);
  // dQ: dq_t = dO_t S_t^T, a forward pass over (dO, V, K) from S0^T.
  if (e == hipSuccess) {
    a.q = dout;
    a.k = v;
    a.v = k;
    a.out = dq;
    a.kv_in = kv_in ? s0t : nullptr;
    a.kv_out = nullptr;
    a.rev = false;
    a.scale_kv_out = false;
    e = run_passes(a, st);
  }
  // dK: dk_t = v_t G_t^T, G^T run last token first over (V, dO, Q) from dSN^T.
  la::PrefillArgs ak = a;  // reuses a's check slots and flags once the dQ pass is done with them
  ak.q = v;
  ak.k = dout;
  ak.v = q;
  ak.out = dk;
  ak.kv_in = dkv_out ? dsnt : nullptr;
  ak.kv_out = nullptr;
  ak.rev = true;
  ak.scale_kv_out = false;
  // dV: dv_t = k_t G_t, G run last token first over (K, Q, dO) from dSN; its
  // final state is G_0, and dS0 = lam G_0.
  la::PrefillArgs av = ak;
  av.q = k;
  av.k = q;
  av.v = dout;
  av.out = dv;
  av.kv_in = dkv_out;
  av.kv_out = dkv_in;
  av.scale_kv_out = true;
  av.states = (float*)((char*)ws + states2_off);
  // the second region has the forward layout's room after its chunk states
  if (a.warm_start) {
    av.guard = (float*)((char*)ws + states2_off + (guard_off - tbl_bytes));
    av.flags = (int*)((char*)ws + states2_off + (flags_off - tbl_bytes));
  }
  if (a.in_dtype == la::kBF16) {
    // Both read Q and dO: their workgroups for one chunk run side by side, so
    // those tiles come from HBM about once.
    if (e == hipSuccess) e = la::launch_aggregate_pass(ak, st);
    if (e == hipSuccess) e = la::launch_aggregate_pass(av, st);
    if (a.warm_start) {
      // as in the forward: the other heads' scans, one launch for every
      // output row of both passes, the warm-start check of each pass, the
      // decaying heads' final states, and the exact path for the flagged
      // heads of either pass (paired as well)
      if (e == hipSuccess) e = la::launch_scan_pass(ak, st, 1);
      if (e == hipSuccess) e = la::launch_scan_pass(av, st, 1);
      if (e == hipSuccess) e = la::launch_mixed_pair(ak, av, st);
      if (e == hipSuccess) e = la::launch_warm_guard(ak, st);
      if (e == hipSuccess) e = la::launch_warm_guard(av, st);
      la::PrefillArgs rk = ak, rv = av;
      rk.warm_start = rv.warm_start = false;
      rk.rerun = rv.rerun = true;
      if (e == hipSuccess) e = la::launch_aggregate_pass(rk, st);
      if (e == hipSuccess) e = la::launch_aggregate_pass(rv, st);
      if (e == hipSuccess) e = la::launch_scan_pass(rk, st, 3);
      if (e == hipSuccess) e = la::launch_scan_pass(rv, st, 3);
      if (e == hipSuccess) e = la::launch_output_pair(rk, rv, st);
    } else {
      if (e == hipSuccess) e = la::launch_scan_pass(ak, st);
      if (e == hipSuccess) e = la::launch_scan_pass(av, st);
      if (e == hipSuccess) e = la::launch_output_pair(ak, av, st);
    }
  } else {
    if (e == hipSuccess) e = run_passes(ak, st);
    if (e == hipSuccess) e = run_passes(av, st);
  }
  if (!workspace) {
    hipError_t f = hipFreeAsync(ws, st);
    if (e == hipSuccess) e = f;
  }
  return from_hip(e);
}

int64_t lightning_attn_fwd_chunk(int64_t B, int64_t H, int64_t N, int64_t block, int64_t chunk) {
  int64_t L = 0;
  if (resolve_chunk(B, H, N, block, chunk, &L) != LA_OK) return -1;
  return L;
}

int64_t lightning_attn_fwd_warm_chunk(int64_t B, int64_t H, int64_t N, int64_t block, int64_t chunk,
                                      int64_t warm_chunk) {
  int64_t L = 0, Lw = 0;
  if (resolve_chunk(B, H, N, block, chunk, &L) != LA_OK) return -1;
  if (resolve_warm_chunk(B, H, N, chunk, warm_chunk, L, &Lw) != LA_OK) return -1;
  return Lw;
}

size_t lightning_attn_fwd_workspace_bytes_ex(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                                             int64_t chunk) {
  int64_t L = 0;
  if (d < 1 || resolve_chunk(B, H, N, block, chunk, &L) != LA_OK) return 0;
  return workspace_layout(B, H, N, d, block, L, nullptr);
}

size_t lightning_attn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block) {
  return lightning_attn_fwd_workspace_bytes_ex(B, H, N, d, block, 0);
}

int lightning_attn_decode_step(const void* q, const void* k, const void* v, const float* decay, void* out,
                               const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t d,
                               void* stream) {
  if (!q || !k || !v || !decay || !out) return LA_ERR_INVALID;
  if (B < 1 || H < 1 || d < 1) return LA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(decay, 4) ||
      !aligned(kv_in, 16) || !aligned(kv_out, 16))
    return LA_ERR_INVALID;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  if (!dims_fit(B, H, 1)) return LA_ERR_UNSUPPORTED;
  const int64_t vec_bytes = B * H * d * 2, st_bytes = B * H * d * d * 4;
  if (overlap(out, vec_bytes, q, vec_bytes) || overlap(out, vec_bytes, k, vec_bytes) ||
      overlap(out, vec_bytes, v, vec_bytes) || overlap(out, vec_bytes, kv_in, st_bytes) ||
      overlap(out, vec_bytes, kv_out, st_bytes) || overlap(out, vec_bytes, decay, H * 4) ||
      !states_apart_or_same(kv_in, kv_out, st_bytes))
    return LA_ERR_INVALID;
  if (overlap(kv_out, st_bytes, q, vec_bytes) || overlap(kv_out, st_bytes, k, vec_bytes) ||
      overlap(kv_out, st_bytes, v, vec_bytes) || overlap(kv_out, st_bytes, decay, H * 4))
    return LA_ERR_INVALID;
  return from_hip(la::launch_decode(q, k, v, decay, out, kv_in, kv_out, B, H, d, (hipStream_t)stream));
}

int lightning_attn_decode_slots(const void* q, const void* k, const void* v, const float* decay, void* out,
                                float* states, const int32_t* slots, int64_t B, int64_t H, int64_t d,
                                int64_t num_slots, void* stream) {
  if (!q || !k || !v || !decay || !out || !states || !slots) return LA_ERR_INVALID;
  if (B < 1 || H < 1 || d < 1 || num_slots < 1) return LA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(decay, 4) ||
      !aligned(states, 16) || !aligned(slots, 4))
    return LA_ERR_INVALID;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  if (!dims_fit(B, H, 1, num_slots)) return LA_ERR_UNSUPPORTED;
  const int64_t vec_bytes = B * H * d * 2, pool_bytes = num_slots * H * d * d * 4;
  if (overlap(out, vec_bytes, q, vec_bytes) || overlap(out, vec_bytes, k, vec_bytes) ||
      overlap(out, vec_bytes, v, vec_bytes) || overlap(out, vec_bytes, states, pool_bytes) ||
      overlap(out, vec_bytes, slots, B * 4) || overlap(states, pool_bytes, slots, B * 4) ||
      overlap(out, vec_bytes, decay, H * 4) || overlap(states, pool_bytes, q, vec_bytes) ||
      overlap(states, pool_bytes, k, vec_bytes) || overlap(states, pool_bytes, v, vec_bytes) ||
      overlap(states, pool_bytes, decay, H * 4))
    return LA_ERR_INVALID;
  return from_hip(la::launch_decode(q, k, v, decay, out, states, states, B, H, d, (hipStream_t)stream,
                                    (const int*)slots, num_slots));
}

int lightning_attn_decode_fused(const void* q, const void* k, const void* v, const float* decay, void* out,
                                float* states, const int32_t* slots, int64_t num_slots, int silu,
                                const float* gamma, float eps, const void* gate, int64_t B, int64_t H, int64_t d,
                                void* stream) {
  if (!q || !k || !v || !decay || !out || !states) return LA_ERR_INVALID;
  if (B < 1 || H < 1 || d < 1 || num_slots < 1) return LA_ERR_INVALID;
  if (!slots && num_slots < B) return LA_ERR_INVALID;
  if (!(eps >= 0.0f) || eps > 1.0f) return LA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(decay, 4) ||
      !aligned(states, 16) || !aligned(slots, 4) || !aligned(gamma, 16) || !aligned(gate, 16))
    return LA_ERR_INVALID;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  if (!dims_fit(B, H, 1, num_slots)) return LA_ERR_UNSUPPORTED;
  const int64_t vec_bytes = B * H * d * 2, pool_bytes = num_slots * H * d * d * 4;
  if (overlap(out, vec_bytes, q, vec_bytes) || overlap(out, vec_bytes, k, vec_bytes) ||
      overlap(out, vec_bytes, v, vec_bytes) || overlap(out, vec_bytes, states, pool_bytes) ||
      overlap(out, vec_bytes, slots, B * 4) || overlap(states, pool_bytes, slots, B * 4) ||
      overlap(out, vec_bytes, gate, vec_bytes) || overlap(out, vec_bytes, gamma, H * d * 4) ||
      overlap(states, pool_bytes, gate, vec_bytes) || overlap(states, pool_bytes, gamma, H * d * 4) ||
      overlap(out, vec_bytes, decay, H * 4) || overlap(states, pool_bytes, q, vec_bytes) ||
      overlap(states, pool_bytes, k, vec_bytes) || overlap(states, pool_bytes, v, vec_bytes) ||
      overlap(states, pool_bytes, decay, H * 4))
    return LA_ERR_INVALID;
  la::DecodeFusion fz{silu ? 1 : 0, gamma, eps, gate};
  return from_hip(la::launch_decode(q, k, v, decay, out, states, states, B, H, d, (hipStream_t)stream,
                                    (const int*)slots, num_slots, &fz));
}

int lightning_attn_decode_layers(const void* q, const void* k, const void* v, const float* decay, void* out,
                                 float* states, const int32_t* slots, int64_t num_layers, int64_t B, int64_t H,
                                 int64_t d, int64_t num_slots, int silu, const float* gamma, float eps,
                                 const void* gate, void* stream) {
  if (!q || !k || !v || !decay || !out || !states) return LA_ERR_INVALID;
  if (num_layers < 1 || B < 1 || H < 1 || d < 1 || num_slots < 1) return LA_ERR_INVALID;
  if (!slots && num_slots < B) return LA_ERR_INVALID;
  if (!(eps >= 0.0f) || eps > 1.0f) return LA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(decay, 4) ||
      !aligned(states, 16) || !aligned(slots, 4) || !aligned(gamma, 16) || !aligned(gate, 16))
    return LA_ERR_INVALID;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  // every layer's rows and pool as one of num_layers times the size
  if (num_layers > kMaxGrid || !dims_fit(num_layers * B, H, 1, num_layers * num_slots)) return LA_ERR_UNSUPPORTED;
  if (num_layers * B > kMaxGrid || num_layers * num_slots > kMaxGrid) return LA_ERR_UNSUPPORTED;
  const int64_t vec_bytes = num_layers * B * H * d * 2, pool_bytes = num_layers * num_slots * H * d * d * 4;
  const int64_t slot_bytes = num_layers * B * 4, gamma_bytes = num_layers * H * d * 4;
  if (overlap(out, vec_bytes, q, vec_bytes) || overlap(out, vec_bytes, k, vec_bytes) ||
      overlap(out, vec_bytes, v, vec_bytes) || overlap(out, vec_bytes, states, pool_bytes) ||
      overlap(out, vec_bytes, slots, slot_bytes) || overlap(states, pool_bytes, slots, slot_bytes) ||
      overlap(out, vec_bytes, gate, vec_bytes) || overlap(out, vec_bytes, gamma, gamma_bytes) ||
      overlap(states, pool_bytes, gate, vec_bytes) || overlap(states, pool_bytes, gamma, gamma_bytes) ||
      overlap(states, pool_bytes, q, vec_bytes) || overlap(states, pool_bytes, k, vec_bytes) ||
      overlap(states, pool_bytes, v, vec_bytes) || overlap(states, pool_bytes, decay, num_layers * H * 4) ||
      overlap(out, vec_bytes, decay, num_layers * H * 4))
    return LA_ERR_INVALID;
  la::DecodeFusion fz{silu ? 1 : 0, gamma, eps, gate};
  return from_hip(la::launch_decode(q, k, v, decay, out, states, states, B, H, d, (hipStream_t)stream,
                                    (const int*)slots, num_slots, &fz, num_layers));
}

int lightning_attn_norm_gate(const void* o, int o_dtype, const void* gate, const float* gamma, float eps, void* out,
                             int64_t B, int64_t H, int64_t N, int64_t d, void* stream) {
  if (!o || !out) return LA_ERR_INVALID;
  if (B < 1 || H < 1 || N < 1 || d < 1) return LA_ERR_INVALID;
  if (o_dtype != LA_DTYPE_BF16 && o_dtype != LA_DTYPE_F32) return LA_ERR_INVALID;
  if (!(eps >= 0.0f) || eps > 1.0f) return LA_ERR_INVALID;
  if (!aligned(o, 16) || !aligned(out, 16) || !aligned(gate, 16) || !aligned(gamma, 16)) return LA_ERR_INVALID;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  if (!dims_fit(B, H, N)) return LA_ERR_UNSUPPORTED;
  const int64_t rows = B * H * N;
  if (rows * (d / 8) / 256 + 1 > kMaxGrid) return LA_ERR_UNSUPPORTED;
  const int64_t o_bytes = rows * d * (o_dtype == LA_DTYPE_BF16 ? 2 : 4), y_bytes = rows * d * 2;
  const bool in_place = out == o && o_dtype == LA_DTYPE_BF16;
  if (!in_place && overlap(out, y_bytes, o, o_bytes)) return LA_ERR_INVALID;
  if (overlap(out, y_bytes, gate, y_bytes) || overlap(out, y_bytes, gamma, H * d * 4)) return LA_ERR_INVALID;
  return from_hip(la::launch_norm_gate(o, o_dtype == LA_DTYPE_BF16 ? la::kBF16 : la::kF32, gate, gamma, eps, out,
                                       rows, H, N, d, (hipStream_t)stream));
}

int lightning_attn_silu(void* x, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && !x)) return LA_ERR_INVALID;
  if (!aligned(x, 16)) return LA_ERR_INVALID;
  if (n > (int64_t(1) << 44)) return LA_ERR_UNSUPPORTED;  // the grid of 8192-element workgroups fits 31 bits
  if (n == 0) return LA_OK;
  return from_hip(la::launch_silu(x, n, (hipStream_t)stream));
}

const char* lightning_attn_strerror(int status) {
  switch (status) {
    case LA_OK: return "ok";
    case LA_ERR_INVALID: return "invalid argument";
    case LA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LA_ERR_HIP: return "HIP runtime error";
    case LA_ERR_NOMEM: return "out of device memory";
    case LA_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

int lightning_attn_runtime_version(int* version) {
  if (!version) return LA_ERR_INVALID;
  return hipRuntimeGetVersion(version) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Prefill without allocation: the workspace of lightning_attn_fwd_ex lives in
// a file-scope device array, one copy per GPU the library runs on, held until
// the process ends.  Host code never passes the array's name to a kernel (in
// host code it is a stand-in, not a device address): the device address is
// fetched once per device with hipGetSymbolAddress and kept per device.

static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (its device address).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LA_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // racing first calls store the same address
  }
  *out = p;
  return LA_OK;
}

}  // namespace

extern "C" int lightning_attn_fwd_noalloc(const void* q, const void* k, const void* v, const float* decay, void* out,
                                          const float* kv_in, float* kv_out, int64_t B, int64_t H, int64_t N,
                                          int64_t d, int in_dtype, int out_dtype, int64_t chunk, int64_t warm_chunk,
                                          unsigned int flags, void* stream) {
  if (flags & ~kFwdFlags) return LA_ERR_INVALID;
  const int64_t block = 64;
  int64_t L = 0, Lw = 0;
  int rc = validate_prefill(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, in_dtype, out_dtype, chunk, &L);
  if (rc != LA_OK) return rc;
  if (!flags_supported(flags, in_dtype, block)) return LA_ERR_UNSUPPORTED;
  if (chunk == 0) {
    // the default chunk, doubled until its chunk states fit the scratch array
    while (workspace_layout(B, H, N, d, block, L, nullptr) > LA_NOALLOC_SCRATCH_BYTES && 2 * L <= kMaxTokens &&
           L < ceil_div(N, block) * block)
      L *= 2;
    if (B * H * ceil_div(N, L) > kMaxGrid) return LA_ERR_UNSUPPORTED;
  }
  if (workspace_layout(B, H, N, d, block, L, nullptr) > LA_NOALLOC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
  if (warm_chunk == 0) {
    // the default warm-start chunk of lightning_attn_fwd_ex, at least L
    const int64_t L0 = pick_chunk(B, H, N, block);
    Lw = pick_warm_chunk(B, H, N, L0);
    if (Lw < L) Lw = L;
  } else {
    rc = resolve_warm_chunk(B, H, N, L, warm_chunk, L, &Lw);
    if (rc != LA_OK) return rc;
  }
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != LA_OK) return rc;
  if (stream) {
    // the array's address is the current device's copy: a stream of another
    // device would run the kernels against it
    int cur = -1;
    hipDevice_t sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
      return LA_ERR_HIP;
    if (sdev != cur) return LA_ERR_INVALID;
  }
  return prefill_run(q, k, v, decay, out, kv_in, kv_out, B, H, N, d, block, in_dtype, out_dtype, L, Lw, ws,
                     LA_NOALLOC_SCRATCH_BYTES, nullptr, nullptr, stream, nullptr, 0, flags);
}
