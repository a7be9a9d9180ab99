// Device-side building blocks shared by the gfx950 lightning-attention kernels:
// MFMA operand traits, the 32x32 accumulator layout, LDS operand loaders and
// the bf16 hi/lo split.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kSub = 64;  // token rows per LDS stage of the prefill kernels

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Accumulator layout of every 32x32 MFMA on CDNA: lane l, register j holds
// row crow(j, l/32), column l%32.
__device__ __forceinline__ int crow(int j, int hf) { return 8 * (j >> 2) + 4 * hf + (j & 3); }

// lam^e in double by binary powering (lam^0 = 1, including lam = 0).
__device__ __forceinline__ double pow_int(double x, int e) {
  double r = 1.0, b = x;
  while (e > 0) {
    if (e & 1) r *= b;
    b *= b;
    e >>= 1;
  }
  return r;
}

// Rows after a chunk start whose outputs still feel the chunk's start state
// by more than 2^-30 of its own weight: the state enters row r scaled by
// lam^(r+1), and lam^(r+1) <= 2^-30 once r + 1 >= 30 ln 2 / -ln lam.  Rounded
// up to whole 64-token sub-tiles; 0 for lam = 0; INT32_MAX for lam >= 1 (no
// decay).  Computed in double so that every kernel classifies a head alike.
__device__ __forceinline__ int carry_span(float lam) {
  if (lam == 0.0f) return 0;
  if (!(lam > 0.0f && lam < 1.0f)) return 0x7fffffff;  // negative, >= 1 or NaN: never dropped
  const double t = 20.79441541679836 / -log((double)lam);  // 30 ln 2 / -ln lam
  if (!(t < 1.0e9)) return 0x7fffffff;
  const int64_t r = (int64_t)ceil(t);
  return (int)(((r + 63) / 64) * 64);
}

// A head decays within its chunk of L tokens when 2 carry_span <= L.  Each
// chunk of such a head is then computed from the state that the carry_span
// tokens before it build from zero, with no scan over chunks (a warm-up of at
// most half a chunk; the omission bound does not depend on the ratio).
__device__ __forceinline__ bool decays_within_chunk(int span, int L) { return 2ll * (long long)span <= (long long)L; }

// Row of the initial / final state array that (batch, head) pair bh uses:
// bh itself, or, with a slot table, slot slots[b] of a pool of num_slots
// (each of H heads); -1 when the slot is out of range (no state: start from
// zero and keep no final state).
__device__ __forceinline__ int64_t state_row(int64_t bh, int H, const int* slots, int64_t num_slots) {
  if (!slots) return bh;
  const int64_t b = bh / H, s = slots[b];
  return (s >= 0 && s < num_slots) ? s * H + (bh - b * H) : -1;
}

// MFMA traits.  One instruction contracts KW elements; every lane contributes
// EPL of them (lanes 0-31 and 32-63 split the contraction).  A and B use the
// same (lane half, element) -> k correspondence, so any fixed permutation of
// the contraction index is allowed as long as both operands follow it.
template <typename T>
struct Mfma;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// RNE of two floats into one dword of two bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, output lane l receives, as element j (j < 4), the 16-bit value at
// (address given by lane 4j + l/4 of the group) + 2 * (l % 4) bytes.  If lane
// 4j + q of a group points at row (r + j), column (c + 4q) of a row-major
// tile, output lane l of the group holds rows r..r+3 of column c + l.
__device__ __forceinline__ bf16x4 ds_tr4(const bf16* p) {
  const shortx4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

template <>
struct Mfma<bf16> {
  static constexpr int KW = 16;
  static constexpr int EPL = 8;
  static constexpr bool kSplit = true;  // fp32 operands are fed as bf16 hi + lo
  typedef bf16x8 op_t;
  static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // EPL contiguous elements.
  static __device__ __forceinline__ op_t ld_nat(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  // Elements at columns crow(g*EPL + i, hf), i < EPL, of a row: two runs of 4.
  static __device__ __forceinline__ op_t ld_cperm(const bf16* row, int g, int hf) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 16 * g + 4 * hf);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 * g + 8 + 4 * hf);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Operand with lane L = 32h + n holding X[row0 + 8h + i][col0 + n], i < 8,
  // from a row-major LDS tile X with row stride ld (two transpose reads).
  static __device__ __forceinline__ op_t ld_tr_nat(const bf16* X, int ld, int row0, int col0, int lane) {
    const int h = lane >> 5, j = (lane & 15) >> 2;
    const bf16* p = X + (row0 + 8 * h + j) * ld + col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const bf16x4 lo = ds_tr4(p), hi = ds_tr4(p + 4 * ld);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Same, with element i taken from row row0 + crow(8g + i, h) (the row order
  // of an accumulator tile used as an operand).
  static __device__ __forceinline__ op_t ld_tr_cperm(const bf16* X, int ld, int row0, int g, int col0, int lane) {
    const int h = lane >> 5, j = (lane & 15) >> 2;
    const bf16* p = X + (row0 + 16 * g + 4 * h + j) * ld + col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const bf16x4 lo = ds_tr4(p), hi = ds_tr4(p + 8 * ld);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ op_t cvt(const float* x) {
    return __builtin_bit_cast(op_t, uint4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                          pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])});
  }
  // x ~= hi + lo: hi = x truncated to bf16 (its top 16 bits), lo = RNE(x - hi).
  // x - hi is exact in fp32 and |x - hi| < 2^-7 |x|, so |x - hi - lo| < 2^-16 |x|.
  // No contraction: were the product that forms x fused into x - hi, lo would
  // depend on the compiler's choice per instantiation, and the fp32- and
  // bf16-output kernels would no longer agree bit for bit.
  static __device__ __forceinline__ void split(const float* x, op_t& hi, op_t& lo) {
#pragma clang fp contract(off)
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b0 = __float_as_uint(x[2 * i]), b1 = __float_as_uint(x[2 * i + 1]);
      const float r0 = x[2 * i] - __uint_as_float(b0 & 0xffff0000u);
      const float r1 = x[2 * i + 1] - __uint_as_float(b1 & 0xffff0000u);
      h[i] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // {hi16(b0), hi16(b1)}
      l[i] = pack_bf16x2(r0, r1);
    }
    hi = __builtin_bit_cast(op_t, uint4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(op_t, uint4{l[0], l[1], l[2], l[3]});
  }
  static __device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
  static __device__ __forceinline__ bf16 elem(op_t x, int i) { return x[i]; }
};

template <>
struct Mfma<float> {
  static constexpr int KW = 2;
  static constexpr int EPL = 1;
  static constexpr bool kSplit = false;
  typedef float op_t;
  static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ op_t ld_nat(const float* p) { return *p; }
  static __device__ __forceinline__ op_t ld_cperm(const float* row, int g, int hf) { return row[crow(g, hf)]; }
  static __device__ __forceinline__ op_t ld_tr_nat(const float* X, int ld, int row0, int col0, int lane) {
    return X[(row0 + (lane >> 5)) * ld + col0 + (lane & 31)];
  }
  static __device__ __forceinline__ op_t ld_tr_cperm(const float* X, int ld, int row0, int g, int col0, int lane) {
    return X[(row0 + crow(g, lane >> 5)) * ld + col0 + (lane & 31)];
  }
  static __device__ __forceinline__ op_t cvt(const float* x) { return x[0]; }
  static __device__ __forceinline__ void split(const float* x, op_t& hi, op_t& lo) {
    hi = x[0];
    lo = 0.0f;
  }
  static __device__ __forceinline__ float to_f32(float x) { return x; }
  static __device__ __forceinline__ float elem(op_t x, int) { return x; }
};

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// 64 rows of a [N][D] head held in registers between a global load and an
// LDS store (so the next tile's loads overlap the current tile's compute).
// Rows at or beyond t_end read as zero.  16-byte accesses; a wave covers
// whole contiguous rows.
template <typename T, int D, int NT>
struct RowTile {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = D / VEC;
  static constexpr int TOTAL = 64 * CPR;
  static_assert(TOTAL % NT == 0, "tile must split evenly over the workgroup");
  static constexpr int PER = TOTAL / NT;
  uint4 r[PER];

  // Rows t0 .. t0 + 63 (those below t_end; zeros beyond) of a row-major
  // [N][D] array; row t at src + t * RS elements (RS = -D: rows last first).
  template <int RS = D>
  __device__ __forceinline__ void load(const T* __restrict__ src, int t0, int t_end, int tid) {
    const T* base = src + (int64_t)t0 * RS;
    if (t0 + 64 <= t_end) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int idx = tid + i * NT;
        r[i] = *reinterpret_cast<const uint4*>(base + (idx / CPR) * RS + (idx % CPR) * VEC);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int idx = tid + i * NT;
        const int row = idx / CPR;
        if (t0 + row < t_end)
          r[i] = *reinterpret_cast<const uint4*>(base + row * RS + (idx % CPR) * VEC);
        else
          r[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  // Store with 8-byte writes into a tile whose row stride is an odd number
  // of 8-byte units: lane c of a row writes the even or the odd half of its
  // 16 bytes first depending on bit 3 of c, so the 16 lanes of each write
  // instruction cover 16 distinct half-rows of banks.
  template <int LD>
  __device__ __forceinline__ void store_halves(T* __restrict__ dst, int tid) const {
    static_assert((LD * sizeof(T)) % 8 == 0, "8-byte aligned rows");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CPR, cc = idx % CPR;
      const bool odd_first = (cc >> 3) & 1;
      const uint2 lo = make_uint2(r[i].x, r[i].y), hi = make_uint2(r[i].z, r[i].w);
      T* p = dst + row * LD + cc * VEC;
      *reinterpret_cast<uint2*>(p + (odd_first ? VEC / 2 : 0)) = odd_first ? hi : lo;
      *reinterpret_cast<uint2*>(p + (odd_first ? 0 : VEC / 2)) = odd_first ? lo : hi;
    }
  }
  // Store into an unpadded tile (row stride D) whose 16-byte chunks are
  // XOR-swizzled by 2 * (row % 4): chunk c of row r lands at chunk
  // c ^ (2 * (r & 3)).  8 lanes writing 8 aligned chunks of a row still cover
  // 8 distinct bank groups.
  __device__ __forceinline__ void store_swz(T* __restrict__ dst, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CPR, cc = idx % CPR;
      *reinterpret_cast<uint4*>(dst + row * D + ((cc ^ (2 * (row & 3))) * VEC)) = r[i];
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(T* __restrict__ dst, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CPR, cc = idx % CPR;
      *reinterpret_cast<uint4*>(dst + row * LD + cc * VEC) = r[i];
    }
  }
};

// ---------------------------------------------------------------------------
// Swizzled LDS tiles of the bf16 fast paths: 64 rows x D bf16, unpadded,
// 16-byte chunk c of row r stored at chunk c ^ swz<D>(r).  At D = 128 a row is
// 256 bytes, one pass over all 64 banks, and
//   swz(r) = ((r & 3) << 2) | ((r >> 2) & 3):
//   * 16-byte row reads (16 lanes = 16 consecutive rows at one chunk) see swz
//     take all 16 values on r % 16, so the 16 lanes cover all 64 banks;
//   * transpose reads (32 lanes = rows r0..r0+3, r0 % 4 == 0, x four
//     adjacent chunks c0..c0+3, c0 % 4 == 0) see (r & 3) << 2 send each row's
//     four chunks to a different aligned group of four, while (r >> 2) & 3,
//     equal for the 4 rows, only permutes within a group: 16 distinct chunks.
// At D = 64 (8 chunks per row) swz(r) = 2(r & 3) | ((r >> 2) & 1) does the
// same over half as many banks per row.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (2 * (r & 3)) | ((r >> 2) & 1);
}
// Element offset of (row, col) within the tile (row stride D).
template <int D>
__device__ __forceinline__ int swz_at(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row)) << 3) | (col & 7));
}

// LDS DMA.  The tiles reach LDS without passing through registers: with
// global_load_lds_dwordx4 lane i of a wave moves 16 bytes from its own global
// address to LDS byte address m0 + 16 i (m0 is wave-uniform), so one
// instruction fills 1 KiB of a tile, and each lane fetches the global chunk
// that belongs at its swizzled slot.  A tile with rows past the end of the
// sequence is moved row by row with 4-byte transfers, the missing rows being
// zero-filled with ordinary LDS stores.
// Completion is tracked by the wave's vector-memory counter, which counts
// loads, LDS DMA and stores in issue order: each wave waits for its own
// transfers (vmcnt(n), n = vector-memory instructions it issued after them)
// and then the barrier publishes them to the other waves.  The transfers are
// issued from inline assembly so that the compiler, which cannot tell which
// tile a transpose read touches, does not make every LDS read wait for them;
// the waits are explicit, in sync_lds_after_vmem.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}
// m0 (the LDS base of the transfer) is saved and restored around it.
__device__ __forceinline__ void dma_dword(const void* g, uint32_t m0) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(g), "s"(m0)
      : "memory");
}
// Full-tile form: wave-uniform base in SGPRs plus a per-lane 32-bit byte
// offset (the scalar-base addressing of global instructions), so the
// instruction needs no 64-bit address arithmetic of its own; m0 is written
// and not restored.  The compiler emits no m0 use of its own in these
// kernels (no LDS-DMA builtins, no indexed register access, no messages),
// which a host test checks on the built code objects, so nothing it holds in
// m0 can be lost.  One wait state separates the m0 write from the transfer.
__device__ __forceinline__ void dma_dwordx4_sbase(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(m0)
               : "memory");
}

// Wait until at most N of this wave's vector-memory instructions are in
// flight and its LDS operations are done, then barrier.  Also a compiler
// barrier for memory accesses.
template <int N>
__device__ __forceinline__ void sync_lds_after_vmem() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}
// Wait until at most N of this wave's vector-memory instructions are in
// flight (no barrier).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// sigmoid(x) = 1 / (1 + e^-x) and SiLU(x) = x sigmoid(x) with the hardware
// base-2 exponential and reciprocal (about 1 ulp each, far below the bf16
// rounding every caller applies next): every kernel that applies SiLU or the
// gate uses these, so SiLU fused into a tile load equals the SiLU pass
// bit for bit.  x -> -inf gives e^-x = inf and a product of -0; x -> +inf
// gives x.
__device__ __forceinline__ float sigmoid_hw(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}
__device__ __forceinline__ float silu_hw(float x) { return x * sigmoid_hw(x); }

// Rows [0, nvalid) of a 64-row tile (src: its row 0, wave-uniform; row r at
// src + r * RS elements, RS = -D for a tile read last row first) into the
// swizzled LDS tile dst; rows >= nvalid become zero.  The NW waves split the
// instructions.  Full tile: NI / NW 16-byte instructions per wave.
template <int D, int NW, int RS = D>
__device__ __forceinline__ void dma_tile(const bf16* __restrict__ src, bf16* dst, int nvalid, int w, int lane) {
  const uint32_t t0 = lds_addr(dst);
  if (nvalid >= kSub) {
    constexpr int CPR = D / 8, RPI = 64 / CPR, NI = kSub / RPI;
    // Row r sits at src + r * RS; the lowest address of the tile is row 0
    // (RS > 0) or row 63 (RS < 0), and every lane's offset from it is >= 0.
    constexpr int kLow = RS < 0 ? (kSub - 1) * RS : 0;
    const bf16* low = src + kLow;
    const int rr = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int m = 0; m < NI / NW; ++m) {
      const int qi = w + NW * m;
      const int row = RPI * qi + rr;
      const uint32_t off = (uint32_t)(row * RS - kLow + ((pc ^ swz<D>(row)) << 3)) * (uint32_t)sizeof(bf16);
      dma_dwordx4_sbase(low, off, t0 + 1024 * qi);
    }
  } else if (lane < D / 2) {
    for (int r = w; r < kSub; r += NW) {
      if (r < nvalid)
        dma_dword(src + r * RS + (((lane >> 2) ^ swz<D>(r)) << 3) + 2 * (lane & 3), t0 + 2 * r * D);
      else
        *reinterpret_cast<uint32_t*>(dst + r * D + 2 * lane) = 0u;
    }
  }
}

// SiLU in place over the part of an LDS tile that this wave's dma_tile call
// (same nvalid) wrote: the wave calls it after waiting for its own transfers
// and before the barrier that publishes the tile, so no other wave reads the
// tile in between.  Each lane rewrites exactly the bytes its transfers
// brought (16 per full-tile instruction, 4 per row of a partial tile); the
// zero rows of a partial tile stay zero (SiLU(0) = 0).  Values are rounded
// to bf16 once, as a SiLU pass over the tensor would store them.
template <int D, int NW>
__device__ __forceinline__ void silu_own(bf16* dst, int nvalid, int w, int lane) {
  if (nvalid >= kSub) {
    constexpr int CPR = D / 8, RPI = 64 / CPR, NI = kSub / RPI;
#pragma unroll
    for (int m = 0; m < NI / NW; ++m) {
      bf16x8* p = reinterpret_cast<bf16x8*>(reinterpret_cast<char*>(dst) + 1024 * (w + NW * m) + 16 * lane);
      bf16x8 x = *p;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (bf16)silu_hw((float)x[j]);
      *p = x;
    }
  } else if (lane < D / 2) {
    for (int r = w; r < nvalid; r += NW) {
      bf16x2* p = reinterpret_cast<bf16x2*>(dst + r * D + 2 * lane);
      bf16x2 x = *p;
      x[0] = (bf16)silu_hw((float)x[0]);
      x[1] = (bf16)silu_hw((float)x[1]);
      *p = x;
    }
  }
}

// 16-byte row operand: elements col .. col + 7 (col % 8 == 0) of a row.
template <int D>
__device__ __forceinline__ bf16x8 ld_row8(const bf16* X, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(X + swz_at<D>(row, col));
}

// Row order of the transpose-read operands: element i of lane L = 32h + n
// holds row row0 + trow(i, h), trow(i, h) = 16(i >> 2) + 4h + (i & 3), so one
// MFMA step contracts rows row0 + {0..7, 16..23}, and the steps at row0 =
// trbase(kk) = 8(kk & 1) + 32(kk >> 1), kk < 4, cover a 64-row sub-tile.  (Any
// fixed order of the contraction index works when both operands and the
// decay factors follow it; this one keeps the two halves of a read 16 rows
// apart, where the swizzle repeats.)
__device__ __forceinline__ int trow(int i, int h) { return 16 * (i >> 2) + 4 * h + (i & 3); }
__device__ __forceinline__ int trbase(int kk) { return 8 * (kk & 1) + 32 * (kk >> 1); }

// Transpose-read operand: lane L = 32h + n gets, as element i < 8, X[row0 +
// trow(i, h)][col0 + cn(n)] with cn(n) = n, or, with PI, n with bits 2 and 3
// swapped (the feature order of the state's accumulator rows); row0 % 4 == 0.
// Within a group of 16 lanes, lane 4j + q points at row row0 + 4h + j and the
// 4 columns of piece q (piece ((q & 1) << 1 | q >> 1) with PI); the second
// read is 16 rows further down, at the same swizzle (swz depends on r % 16),
// so its address is the first one's plus an immediate offset.
template <int D, bool PI>
__device__ __forceinline__ bf16x8 ld_tr8(const bf16* X, int row0, int col0, int lane) {
  const int h = lane >> 5, j = (lane & 15) >> 2, q = lane & 3;
  const int qq = PI ? (((q & 1) << 1) | (q >> 1)) : q;
  const int row = row0 + 4 * h + j;
  const bf16* p = X + swz_at<D>(row, col0 + 16 * ((lane >> 4) & 1) + 4 * qq);
  const bf16x4 lo = ds_tr4(p), hi = ds_tr4(p + 16 * D);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace la
