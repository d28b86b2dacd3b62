// Device helpers shared by the selection kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsai {

constexpr int kWave = 64;

// Pointers into LDS carry the LDS address space so helpers that are not
// inlined still compile to ds_* instructions.
#define DSAI_LDS __attribute__((address_space(3)))
typedef DSAI_LDS uint32_t lds_u32;
typedef DSAI_LDS char lds_char;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// (the compiler builtin takes the predicate as a lane mask, so a compare
// feeds it directly)
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Make LDS writes of this wave visible to its other lanes and keep the
// compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Order-preserving map of an fp32 score to uint32: a > b as floats iff
// key(a) > key(b); -0 is mapped like +0 so the two compare equal.  Inputs
// are finite or -inf (never NaN).
__device__ __forceinline__ uint32_t ord_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ord_key of a score known not to be -0.
__device__ __forceinline__ uint32_t ord_key_nz(float s) {
  const uint32_t b = __float_as_uint(s);
  return (int32_t)b < 0 ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float ord_to_float(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

// Cross-lane steps use DPP moves (no LDS round trip).  A row is 16 lanes.
// Lanes whose DPP source lies outside their row read 0; rows outside
// ROW_MASK read 0.  Every helper below must be called by all 64 lanes.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}

constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kDppRowShr1 = 0x111;      // row_shr:n = 0x110 + n
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row -> the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 -> rows 2 and 3

__device__ __forceinline__ uint32_t lane_value(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// Inclusive sum over lanes [0, lane].
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_mov<kDppRowShr1>(x);
  x += dpp_mov<kDppRowShr1 + 1>(x);
  x += dpp_mov<kDppRowShr1 + 3>(x);
  x += dpp_mov<kDppRowShr1 + 7>(x);
  x += dpp_mov<kDppRowBcast15, 0xA>(x);
  x += dpp_mov<kDppRowBcast31, 0xC>(x);
  return x;
}

// Inclusive sum over lanes [lane, 63].
__device__ __forceinline__ uint32_t wave_incl_suffix(uint32_t x) {
  const uint32_t incl = wave_incl_scan(x);
  return lane_value(incl, kWave - 1) - incl + x;
}

// Reduction over all lanes (the same value in every lane).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
  x = op(x, dpp_mov<kDppQuadXor1>(x));
  x = op(x, dpp_mov<kDppQuadXor2>(x));
  x = op(x, dpp_mov<kDppRowHalfMirror>(x));
  x = op(x, dpp_mov<kDppRowMirror>(x));
  return op(op(lane_value(x, 0), lane_value(x, 16)), op(lane_value(x, 32), lane_value(x, 48)));
}

__device__ __forceinline__ uint32_t wave_and(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return a & b; });
}

__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return a | b; });
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ float wave_fmin(float x) {
  return __uint_as_float(wave_reduce(__float_as_uint(x), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

__device__ __forceinline__ float wave_fmax(float x) {
  return __uint_as_float(wave_reduce(__float_as_uint(x), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

}  // namespace dsai
