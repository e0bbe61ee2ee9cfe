// Device-side building blocks shared by the forward and backward kernels:
// operand vector types, the gfx950 MFMA wrappers, half-precision packing and
// small LDS / global access helpers.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_xcd.hpp"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element-type tags.  Storage is always 16-bit; the tag selects the MFMA
// flavour and the fp32 -> half rounding (round-to-nearest-even for both).
struct BF16 {
  static constexpr bool is_bf16 = true;
};
struct F16 {
  static constexpr bool is_bf16 = false;
};

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate that waits for vmcnt == 0 only (expcnt and lgkmcnt at
// their maxima): vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14.
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);
constexpr float kLn2 = 0.6931471805599453f;

// v_mfma_f32_32x32x16_{bf16,f16}: C[32x32] += A[32x16] * B[16x32].
// Lane L holds A row (L % 32), B column (L % 32), each with the 8 k-values
// 8*(L/32) .. 8*(L/32)+7 of the 16-wide k slice (the same k mapping for A
// and B), and C column (L % 32), rows 8*(i/4) + 4*(L/32) + (i%4), i = 0..15.
template <typename T>
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b,
                                               const f32x16& c) {
  if constexpr (T::is_bf16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Two fp32 -> one packed pair of halves, round-to-nearest-even.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (T::is_bf16) {
    bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = __builtin_convertvector((f32x2){lo, hi}, f16x2);
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <typename T>
__device__ __forceinline__ uint16_t to_half_bits(float x) {
  return static_cast<uint16_t>(pack2<T>(x, 0.0f) & 0xffffu);
}

// Eight consecutive fp32 values -> one 16-byte MFMA operand.
template <typename T>
__device__ __forceinline__ u32x4 pack8(const float* v) {
  return (u32x4){pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]),
                 pack2<T>(v[4], v[5]), pack2<T>(v[6], v[7])};
}

// acc + lo(w) + hi(w) for a packed pair of halves w (v_dot2c_f32_{bf16,f16}).
template <typename T>
__device__ __forceinline__ float sum2_acc(uint32_t w, float acc) {
  if constexpr (T::is_bf16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                  (f16x2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
  }
}

template <typename T>
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  if constexpr (T::is_bf16) {
    return __uint_as_float(bits16 << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
  }
}

// Dot product of two packed 8-half vectors in fp32 (used by the backward
// preprocess; products are exact in fp32, sums round).
template <typename T>
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b) {
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    s += half_bits_to_float<T>(a[w] & 0xffffu) * half_bits_to_float<T>(b[w] & 0xffffu);
    s += half_bits_to_float<T>(a[w] >> 16) * half_bits_to_float<T>(b[w] >> 16);
  }
  return s;
}

// Raw buffer resource (stride 0) over `bytes` bytes at p, for buffer
// instructions: a uniform 64-bit base in scalar registers plus 32-bit vector
// and scalar offsets, so per-access address arithmetic stays 32-bit.  The
// last dword is the gfx9 raw-buffer format word (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0), bytes, 0x00020000);
}

// fp32 -> int32 rounding half up in one instruction: floor(x + 0.5).
__device__ __forceinline__ int32_t cvt_rpi(float x) {
  int32_t r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Largest magnitude among eight packed halves.
template <typename T>
__device__ __forceinline__ float absmax8(const u32x4& a) {
  float m = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    m = fmaxf(m, fabsf(half_bits_to_float<T>(a[w] & 0xffffu)));
    m = fmaxf(m, fabsf(half_bits_to_float<T>(a[w] >> 16)));
  }
  return m;
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ u32x4 lds_read16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void lds_write16(uint16_t* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Permutation of the 32 rows of an MFMA A operand that makes the C layout of
// the product give each lane 8 consecutive row indices per 16-row slice:
// swaps bits 2 and 3 of the row index (an involution).  With A row m holding
// item sigma(m), C value i of lane L is item 16*(i/8) + 8*(L/32) + (i%8).
__device__ __forceinline__ int sigma32(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
__host__ __device__ constexpr int c_item(int i, int hh) {
  return 16 * (i / 8) + 8 * hh + (i % 8);
}
// Row of C value i of lane half hh when A rows are in natural order.
__host__ __device__ constexpr int c_row(int i, int hh) {
  return 8 * (i / 4) + 4 * hh + (i % 4);
}

// sigma32 applied to the low 5 bits of a tile row index.
__device__ __forceinline__ int sigma_row(int r) { return (r & ~31) | sigma32(r & 31); }

// ---------------------------------------------------------------- LDS tiles
//
// Tiles are stored row-major with W halves per row (W = 32, 64 or 128, no
// padding) and the 16-byte chunks of each row XOR-swizzled by a function of
// the row.  The swizzle keeps two access patterns free of bank conflicts on
// the 64-bank LDS:
//   * row reads (ds_read_b128): 16 consecutive rows, same logical chunk;
//   * transposed reads (ds_read_b64_tr_b16): 4 consecutive rows starting at
//     a multiple of 4, an aligned block of 4 logical chunks.
// W = 32 (4 chunks, four rows per 256-byte bank line): g(r) = r/4 % 4.
// W = 64 (8 chunks, two rows per 256-byte bank line): g(r) = bitrev3(r/2 % 8).
// W = 128 (16 chunks, one row per bank line): g(r) = bitrev4(r % 16).
template <int W>
__device__ __forceinline__ int swz(int r) {
  static_assert(W == 32 || W == 64 || W == 128, "tile width");
  if constexpr (W == 32) {
    return (r >> 2) & 3;
  } else if constexpr (W == 64) {
    const int u = (r >> 1) & 7;
    return ((u & 1) << 2) | (u & 2) | ((u >> 2) & 1);
  } else {
    const int u = r & 15;
    return ((u & 1) << 3) | ((u & 2) << 1) | ((u & 4) >> 1) | ((u & 8) >> 3);
  }
}
// Chunk swizzle of a width-64 tile that is written with ds_write_b128 (the
// backward's dS^T tile).  gfx950 serves 128-bit LDS stores eight lanes at a
// time across 128 bytes of banks, so the rows written by eight consecutive
// lanes must use eight different chunks; swz<64> gives rows 2k and 2k+1 the
// same chunk and was measured to spend 16% of the store cycles in bank
// conflicts.  g(r) = (r % 8) ^ 4*((r / 2) % 2) permutes the chunks of every
// eight rows, and rows r and r+2 differ in chunk bit 2, which keeps the
// transposed reads (four consecutive rows, an aligned block of four logical
// chunks) conflict-free as well (both measured: no conflict cycles).
__device__ __forceinline__ int swz_st(int r) {
  const int u = r & 7;
  return u ^ ((u & 2) << 1);
}

// Element offset of (row r, column col) in a swizzled tile of width W.
template <int W>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * W + ((((col >> 3) ^ swz<W>(r)) << 3) | (col & 7));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) * lds_s16x4_ptr;

__device__ __forceinline__ u32x2 lds_read_tr8(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
  return __builtin_bit_cast(u32x2, v);
}

// MFMA 32x32x16 operand gathered "transposed" from a k-major swizzled tile
// X[k][n] (row = k, n contiguous): lane L receives X[k0 + 8*(L/32) + e]
// [n0 + L%32], e = 0..7 -- the B operand for X = B[k][n], or the A operand
// A[m][k] = X[k][m].
//
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane i of a group receives
// as its element j the (i%4)-th half of the 8 bytes addressed by lane
// 4j + i/4 of the same group.  So lane s of group G addresses row
// k0 + 8*(G/2) + s/4 (+4 for the second read) at column n0 + 16*(G%2) + 4*(s%4).
// With SIGMA_ROWS the tile stores logical row r at row sigma_row(r).
template <int W, bool SIGMA_ROWS>
__device__ __forceinline__ u32x4 tr_operand(const uint16_t* tile, int k0, int n0, int lane) {
  const int G = lane >> 4, s = lane & 15;
  int r0 = k0 + 8 * (G >> 1) + (s >> 2);
  int r1 = r0 + 4;
  if constexpr (SIGMA_ROWS) {
    r0 = sigma_row(r0);
    r1 = sigma_row(r1);
  }
  const int col = n0 + 16 * (G & 1) + 4 * (s & 3);
  const u32x2 lo = lds_read_tr8(tile + tile_off<W>(r0, col));
  const u32x2 hi = lds_read_tr8(tile + tile_off<W>(r1, col));
  return (u32x4){lo[0], lo[1], hi[0], hi[1]};
}

// max(x, value of lane L^32): v_permlane32_swap exchanges the two 32-lane
// halves, so the max of its two results is the pairwise max in every lane.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------- hoisted LDS offsets
//
// Byte offsets (relative to a tile's base) that a lane uses for its MFMA
// operand reads.  They depend on the lane only, so they are computed once
// per kernel; inside the loops the tile base and the compile-time block
// offsets become immediate offsets of the ds_read instructions.  The
// swizzle has a period of 16 rows, so every block offset used below is a
// multiple of 16 rows.

// Row read of chunk (2*kc + hh) at row (rbase + l32), rbase a multiple of 32:
// offset = rbase*2W + row_off<W>(lane, kc).
template <int W>
__device__ __forceinline__ uint32_t row_off(int lane, int kc) {
  const int l32 = lane & 31, hh = lane >> 5;
  return static_cast<uint32_t>(l32 * 2 * W + ((32 * kc) ^ (16 * (hh ^ swz<W>(l32)))));
}

// tr_operand read t (0, 1) for k0 = 0, n0 = 32*j: add k0*2W for other k0
// (a multiple of 16).  SIGMA: rows stored under sigma_row.  ST: the tile
// uses swz_st (width 64) instead of swz<W>.
template <int W, bool SIGMA, bool ST = false>
__device__ __forceinline__ uint32_t tr_off(int lane, int t, int j) {
  static_assert(!ST || W == 64, "swz_st is defined for width 64");
  const int G = lane >> 4, s = lane & 15;
  int r = 8 * (G >> 1) + (s >> 2) + 4 * t;
  if constexpr (SIGMA) r = sigma32(r);
  const int col = 16 * (G & 1) + 4 * (s & 3);
  const int sw = ST ? swz_st(r) : swz<W>(r);
  const int off = r * 2 * W + ((((col >> 3) ^ sw) << 4) | ((col & 7) << 1));
  return static_cast<uint32_t>(off ^ (64 * j));
}

__device__ __forceinline__ u32x4 lds_ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + off);
}
__device__ __forceinline__ void lds_st16(void* base, uint32_t off, const u32x4& v) {
  *reinterpret_cast<u32x4*>(static_cast<char*>(base) + off) = v;
}
__device__ __forceinline__ u32x4 lds_tr16(const void* base, uint32_t off0, uint32_t off1) {
  const u32x2 lo = lds_read_tr8(reinterpret_cast<const uint16_t*>(
      static_cast<const char*>(base) + off0));
  const u32x2 hi = lds_read_tr8(reinterpret_cast<const uint16_t*>(
      static_cast<const char*>(base) + off1));
  return (u32x4){lo[0], lo[1], hi[0], hi[1]};
}

// Asynchronous 16-byte copy global -> LDS (global_load_lds_dwordx4): lane i
// writes LDS bytes [ldst + 16*i, ldst + 16*i + 16); ldst must be the same in
// every lane.  Completion is tracked by vmcnt.  Kept as a plain (non-template)
// function: referenced from inside kernel templates directly, the builtin
// makes the host compilation pass drop those kernels' launch stubs.
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 16, 0, 0);
}

// LDS poisoning for debug builds (compiled with -DFA_POISON_LDS=1, as
// libfa_poison.so): every LDS array of a kernel is filled with all-ones bits
// -- a NaN as bf16, f16, fp32 and E4M3 -- when the workgroup starts, so a
// read of LDS the kernel has not written reaches the outputs as NaN instead
// of as whatever an earlier workgroup left there.  Every thread of the
// workgroup must reach the call (it ends in a barrier).  A no-op otherwise.
#ifndef FA_POISON_LDS
#define FA_POISON_LDS 0
#endif
template <typename A>
__device__ __forceinline__ void poison_one(A& a) {
  static_assert(sizeof(A) % 4 == 0, "LDS arrays are whole words");
  uint32_t* w = reinterpret_cast<uint32_t*>(&a);
  for (int i = static_cast<int>(threadIdx.x); i < static_cast<int>(sizeof(A) / 4);
       i += static_cast<int>(blockDim.x))
    w[i] = 0xFFFFFFFFu;
}
template <typename... A>
__device__ __forceinline__ void poison_lds(A&... arrays) {
  if constexpr (FA_POISON_LDS != 0) {
    (poison_one(arrays), ...);
    __syncthreads();
  }
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

}  // namespace fa
