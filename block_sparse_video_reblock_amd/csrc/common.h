// Device-side helpers shared by the gfx950 kernels: bf16 conversion, MFMA operand types,
// wave64 reductions, orderable float keys.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define BSA_DEV __device__ __forceinline__

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kWave = 64;
constexpr int kBlock = 64;

// bf16 <-> fp32 (round to nearest even; inputs are finite)
BSA_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
BSA_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
BSA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// hardware round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32)
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
BSA_DEV uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> BSA_DEV float load_as_f32(const T* p);
template <> BSA_DEV float load_as_f32<float>(const float* p) { return *p; }
template <> BSA_DEV float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// wave64 reductions (xor butterfly over all 64 lanes)
BSA_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
BSA_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// DPP lane move within rows of 16 lanes (all lanes active).  CTRL: 0xB1 = lane ^ 1,
// 0x4E = lane ^ 2 (quad permutations), 0x141 = mirror within 8 lanes, 0x140 = mirror within 16.
template <int CTRL>
BSA_DEV float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over each row of 16 lanes, on every lane of the row
BSA_DEV float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}
// Combine each lane with lane ^ 32 (v_permlane32_swap: with both operands x, the two results
// hold x of the other half-wave in one and x itself in the other, on every lane)
BSA_DEV float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
BSA_DEV float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// wave64 sum, wave-uniform result (DPP within rows, then the four row totals)
BSA_DEV float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
BSA_DEV float wave_total(float x) {
  x = row16_sum(x);
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Monotone map float -> uint32 (a < b  <=>  key(a) < key(b)); -0.0 maps like +0.0.
BSA_DEV uint32_t orderable_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// number of set bits of a 64-bit lane mask below this lane
BSA_DEV int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  return __popcll(mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}
