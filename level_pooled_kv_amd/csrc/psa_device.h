// Device-side helpers shared by the gfx950 kernels of the PSA forward path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16_t { uint16_t bits; };   // storage type of bf16 tensors

// 16 bytes moved as one unit.
struct alignas(16) U128 { uint32_t w[4]; };

__device__ __forceinline__ U128 ld128(const void* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  U128 r; r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w; return r;
}
// 16-byte load marked nontemporal (streaming): for data read once, so that the caches do
// not give its lines priority over the lines later steps read.
__device__ __forceinline__ U128 ld128_stream(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  U128 r; r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3]; return r;
}
__device__ __forceinline__ void st128(void* p, const U128& r) {
  *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v; v[0] = (__bf16)lo; v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Element traits of an I/O dtype: how many elements one 16-byte load holds.
template <typename T> struct io_traits;
template <> struct io_traits<bf16_t> { static constexpr int per16 = 8; };
template <> struct io_traits<float>  { static constexpr int per16 = 4; };

// Unpack one 16-byte chunk into floats.
template <typename T> __device__ __forceinline__ void unpack16(const U128& r, float* out);
template <> __device__ __forceinline__ void unpack16<bf16_t>(const U128& r, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { out[2 * i] = bf16_lo(r.w[i]); out[2 * i + 1] = bf16_hi(r.w[i]); }
}
template <> __device__ __forceinline__ void unpack16<float>(const U128& r, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(r.w[i]);
}

// Pack floats of one 16-byte chunk into the I/O dtype (round to nearest even).
template <typename T> __device__ __forceinline__ U128 pack16(const float* in);
template <> __device__ __forceinline__ U128 pack16<bf16_t>(const float* in) {
  U128 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.w[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
  return r;
}
template <> __device__ __forceinline__ U128 pack16<float>(const float* in) {
  U128 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.w[i] = __float_as_uint(in[i]);
  return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Value of lane (lane ^ M), from VALU cross-lane ops only (no LDS round trip): DPP
// quad permutes for 1 and 2, a half-row mirror (lane ^ 7) then a quad reverse (^ 3)
// for 4, a row rotate by 8 for 8, and the gfx950 row swaps for 16 and 32 (with
// a = b = x, permlane16_swap returns {x[l & ~16], x[l | 16]} per lane and
// permlane32_swap {x[l & ~32], x[l | 32]}).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lane) {
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
  else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);
  else if constexpr (M == 4) {
    const int m7 = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, true);
    return (uint32_t)__builtin_amdgcn_mov_dpp(m7, 0x1B, 0xF, 0xF, true);
  } else if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, true);
  else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    static_assert(M == 32, "lane distance");
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64); every lane
// of a group receives its group's total.
template <int G>
__device__ __forceinline__ float group_sum(float x, int lane) {
  if constexpr (G >= 2) x += __uint_as_float(xor_lane<1>(__float_as_uint(x), lane));
  if constexpr (G >= 4) x += __uint_as_float(xor_lane<2>(__float_as_uint(x), lane));
  if constexpr (G >= 8) x += __uint_as_float(xor_lane<4>(__float_as_uint(x), lane));
  if constexpr (G >= 16) x += __uint_as_float(xor_lane<8>(__float_as_uint(x), lane));
  if constexpr (G >= 32) x += __uint_as_float(xor_lane<16>(__float_as_uint(x), lane));
  if constexpr (G >= 64) x += __uint_as_float(xor_lane<32>(__float_as_uint(x), lane));
  return x;
}

}  // namespace psa
