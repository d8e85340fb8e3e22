// Device-side helpers shared by the gfx950 kernels: storage traits, 16-byte vector loads,
// widening to fp32, dot products over 16-byte chunks, DPP and shuffle reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum DType : int { F32 = 0, F16 = 1, BF16 = 2 };

// One 16-byte vector: the unit every lane loads and stores.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT> struct Elem;
template <> struct Elem<F32> {
  static constexpr int bytes = 4;
  static constexpr int per16 = 4;  // elements in 16 bytes
};
template <> struct Elem<F16> {
  static constexpr int bytes = 2;
  static constexpr int per16 = 8;
};
template <> struct Elem<BF16> {
  static constexpr int bytes = 2;
  static constexpr int per16 = 8;
};

// Reinterpretations take their operand by value: __builtin_bit_cast applied directly to an
// element of an ext_vector lvalue (v[i]) reads element 0 whatever i is, so every vector
// element is first copied into a scalar.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// The same load with the non-temporal cache policy (global_load ... nt): for data read once
// per launch, the KV cache rows. On gfx950 this policy reads HBM about 12% faster than the
// default one, in streams and in random 4 KiB tiles alike (read probe, both policies).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// 16 stored bytes -> Elem<DT>::per16 fp32 values, exactly.
template <int DT> __device__ __forceinline__ void widen(const u32x4& v, float* f);
template <> __device__ __forceinline__ void widen<F32>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = as_f32(v[i]);
}
template <> __device__ __forceinline__ void widen<BF16>(const u32x4& v, float* f) {
  // a bfloat16 is the upper half of a binary32: shifting it into place is exact
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = as_f32(v[i] << 16);
    f[2 * i + 1] = as_f32(v[i] & 0xFFFF0000u);
  }
}
template <> __device__ __forceinline__ void widen<F16>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = as_f16x2(v[i]);
    f[2 * i] = (float)h[0];
    f[2 * i + 1] = (float)h[1];
  }
}

// acc + sum over the 16-byte chunk of q[e]*k[e], in fp32. For 16-bit storage the products of
// two 16-bit values are exact in fp32 and v_dot2 adds two of them per instruction.
template <int DT> __device__ __forceinline__ float dot16(const u32x4& q, const u32x4& k, float acc);
template <> __device__ __forceinline__ float dot16<F32>(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(as_f32(q[i]), as_f32(k[i]), acc);
  return acc;
}
template <> __device__ __forceinline__ float dot16<BF16>(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[i]), as_bf16x2(k[i]), acc, false);
  return acc;
}
template <> __device__ __forceinline__ float dot16<F16>(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2(as_f16x2(q[i]), as_f16x2(k[i]), acc, false);
  return acc;
}

// fp32 -> storage, round to nearest, ties to even; NaN stays NaN.
template <int DT> __device__ __forceinline__ uint32_t narrow_bits(float x);
template <> __device__ __forceinline__ uint32_t narrow_bits<F32>(float x) { return as_u32(x); }
template <> __device__ __forceinline__ uint32_t narrow_bits<F16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <> __device__ __forceinline__ uint32_t narrow_bits<BF16>(float x) {
  uint32_t u = as_u32(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Stores one output element of dtype out_dtype (fp32, or rounded to nearest-even 16 bits).
__device__ __forceinline__ void store_out(void* out, size_t idx, float y, int out_dtype) {
  if (out_dtype == F32) {
    reinterpret_cast<float*>(out)[idx] = y;
  } else if (out_dtype == BF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)narrow_bits<BF16>(y);
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)narrow_bits<F16>(y);
  }
}

// DPP lane permutations inside a row of 16 lanes (gfx9 encodings).
enum : int {
  DPP_XOR1 = 0xB1,         // quad_perm [1,0,3,2]
  DPP_XOR2 = 0x4E,         // quad_perm [2,3,0,1]
  DPP_HALF_MIRROR = 0x141, // lane i <-> 7-i inside each half row
  DPP_MIRROR = 0x140,      // lane i <-> 15-i inside each row
};

template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of a group ends with the
// same bits (each step adds a value and its partner's, and fp addition commutes).
template <int N> __device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<DPP_XOR1>(x);
  if constexpr (N >= 4) x += dpp<DPP_XOR2>(x);
  if constexpr (N >= 8) x += dpp<DPP_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_MIRROR>(x);
  return x;
}

// Max over each aligned row of 16 lanes (DPP); every lane of a row ends with the same value.
__device__ __forceinline__ float xor_max_row16(float x) {
  x = fmaxf(x, dpp<DPP_XOR1>(x));
  x = fmaxf(x, dpp<DPP_XOR2>(x));
  x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_MIRROR>(x));
  return x;
}

// Reductions across lanes whose ids differ in bits >= log2(STRIDE): combine lane l with
// l ^ STRIDE, l ^ 2*STRIDE, ..., l ^ 32 (ds_bpermute through the LDS crossbar).
template <int STRIDE> __device__ __forceinline__ float xor_max_from(float x) {
#pragma unroll
  for (int s = STRIDE; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s, 64));
  return x;
}
template <int STRIDE> __device__ __forceinline__ float xor_sum_from(float x) {
#pragma unroll
  for (int s = STRIDE; s < 64; s <<= 1) x += __shfl_xor(x, s, 64);
  return x;
}

}  // namespace pkv
