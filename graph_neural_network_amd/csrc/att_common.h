// Lane-level helpers shared by the fused attention kernels (forward and
// backward): a lane's 16-byte slices of a node row, their decoding, row
// stores, per-head lane sums and the exponential.
#pragma once
#include "gnn_internal.h"

namespace gnn {
namespace att {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on v_exp_f32 alone.  Softmax arguments are <= 0 (differences from the
// running maximum), and results below 2^-126 of the maximum, which the
// hardware may flush to zero, do not change any sum at fp32 precision.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
template <typename T, int N>
__device__ __forceinline__ void load_row(const T* p, float (&o)[N]);

template <>
__device__ __forceinline__ void load_row<uint16_t, 8>(const uint16_t* p, float (&o)[8]) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  o[0] = dev::bf16_lo(v.x); o[1] = dev::bf16_hi(v.x); o[2] = dev::bf16_lo(v.y); o[3] = dev::bf16_hi(v.y);
  o[4] = dev::bf16_lo(v.z); o[5] = dev::bf16_hi(v.z); o[6] = dev::bf16_lo(v.w); o[7] = dev::bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void load_row<uint16_t, 16>(const uint16_t* p, float (&o)[16]) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint4 w = *reinterpret_cast<const uint4*>(p + 8);
  o[0] = dev::bf16_lo(v.x); o[1] = dev::bf16_hi(v.x); o[2] = dev::bf16_lo(v.y); o[3] = dev::bf16_hi(v.y);
  o[4] = dev::bf16_lo(v.z); o[5] = dev::bf16_hi(v.z); o[6] = dev::bf16_lo(v.w); o[7] = dev::bf16_hi(v.w);
  o[8] = dev::bf16_lo(w.x); o[9] = dev::bf16_hi(w.x); o[10] = dev::bf16_lo(w.y); o[11] = dev::bf16_hi(w.y);
  o[12] = dev::bf16_lo(w.z); o[13] = dev::bf16_hi(w.z); o[14] = dev::bf16_lo(w.w); o[15] = dev::bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void load_row<float, 4>(const float* p, float (&o)[4]) {
  float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
template <>
__device__ __forceinline__ void load_row<float, 8>(const float* p, float (&o)[8]) {
  float4 v = *reinterpret_cast<const float4*>(p);
  float4 w = *reinterpret_cast<const float4*>(p + 4);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; o[4] = w.x; o[5] = w.y; o[6] = w.z; o[7] = w.w;
}

template <int N>
__device__ __forceinline__ void store_row(float* p, const float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; k += 4)
    *reinterpret_cast<float4*>(p + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
}

// The same to global memory as streaming (non-temporal) stores: output rows
// are not read again by the kernel, and kept out of L2 they leave it to the
// gathered rows.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void store_row_nt(float* p, const float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; k += 4)
    __builtin_nontemporal_store(nt_f32x4{v[k], v[k + 1], v[k + 2], v[k + 3]}, reinterpret_cast<nt_f32x4*>(p + k));
}

// The same for any VEL = 1, 2, 4, 8, ... elements: 16-byte pieces where the
// slice allows them, else one 8-, 4-byte or single-element store.
template <int VEL>
__device__ __forceinline__ void store_elems(float* p, const float (&v)[VEL]) {
  if constexpr (VEL % 4 == 0) {
    store_row<VEL>(p, v);
  } else if constexpr (VEL == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int k = 0; k < VEL; ++k) p[k] = v[k];
  }
}
template <int VEL>
__device__ __forceinline__ void store_elems_nt(float* p, const float (&v)[VEL]) {
  if constexpr (VEL % 4 == 0) {
    store_row_nt<VEL>(p, v);
  } else {
#pragma unroll
    for (int k = 0; k < VEL; ++k) __builtin_nontemporal_store(v[k], p + k);
  }
}

// A lane's slice of one node row, VB bytes (2, 4, 8, 16 or 32), kept as raw
// 32-bit words until used (a 2-byte slice sits in the low half of its word,
// the high half zero).
template <int VB>
struct RawB {
  uint32_t u[VB >= 4 ? VB / 4 : 1];
};
// 16 NV bytes: the slices of the 16- and 32-byte lane mappings
template <int NV>
using Raw = RawB<16 * NV>;

template <typename T, int VB>
__device__ __forceinline__ void load_rawb(const T* p, RawB<VB>& r) {
  if constexpr (VB == 2) {
    r.u[0] = (uint32_t)*reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (VB == 4) {
    r.u[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (VB == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.u[0] = v.x; r.u[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < VB / 16; ++k) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[k];
      r.u[4 * k] = v.x; r.u[4 * k + 1] = v.y; r.u[4 * k + 2] = v.z; r.u[4 * k + 3] = v.w;
    }
  }
}
template <typename T, int NV>
__device__ __forceinline__ void load_raw(const T* p, Raw<NV>& r) {
  load_rawb<T, 16 * NV>(p, r);
}

// The same slice through a buffer resource whose base is a node row held in
// scalar registers (a row shared by the whole wave): the lane's byte offset
// is the only per-lane address operand, so a gather costs no vector ALU
// work.  num_records bounds the row; the descriptor's last word is the one
// the gfx9 family (gfx950 included) takes for raw untyped buffer access.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, bytes, kBufferWord3);
}
template <int VB>
__device__ __forceinline__ void load_rawb_buf(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, RawB<VB>& r) {
  if constexpr (VB == 2) {
    r.u[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, byte_off, 0, 0);
  } else if constexpr (VB == 4) {
    r.u[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, 0);
  } else if constexpr (VB == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off, 0, 0);
    r.u[0] = v[0]; r.u[1] = v[1];
  } else {
#pragma unroll
    for (int k = 0; k < VB / 16; ++k) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off + 16 * k, 0, 0);
      r.u[4 * k] = v[0]; r.u[4 * k + 1] = v[1]; r.u[4 * k + 2] = v[2]; r.u[4 * k + 3] = v[3];
    }
  }
}

// The same through one descriptor over a whole array (below 2 GB): the
// row's byte offset is a scalar operand (soffset), so a row costs one scalar
// multiply instead of a descriptor of its own.
template <int VB>
__device__ __forceinline__ void load_rawb_buf_so(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, uint32_t row_off,
                                                 RawB<VB>& r) {
  if constexpr (VB == 2) {
    r.u[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, byte_off, row_off, 0);
  } else if constexpr (VB == 4) {
    r.u[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, row_off, 0);
  } else if constexpr (VB == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off, row_off, 0);
    r.u[0] = v[0]; r.u[1] = v[1];
  } else {
#pragma unroll
    for (int k = 0; k < VB / 16; ++k) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off + 16 * k, row_off, 0);
      r.u[4 * k] = v[0]; r.u[4 * k + 1] = v[1]; r.u[4 * k + 2] = v[2]; r.u[4 * k + 3] = v[3];
    }
  }
}

// Row c (>= 0) of an array at byte stride ld_bytes (below 4 GB) from base:
// one unsigned 32 x 32 -> 64 multiply-add (v_mad_u64_u32) per address
// instead of a signed 64-bit product.
template <typename T>
__device__ __forceinline__ const T* row_at(const T* base, int c, uint32_t ld_bytes) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + (uint64_t)(uint32_t)c * ld_bytes);
}

// element k of a raw slice as float
template <typename T, int VB>
__device__ __forceinline__ float elemb(const RawB<VB>& r, int k) {
  if constexpr (sizeof(T) == 2) return (k & 1) ? dev::bf16_hi(r.u[k >> 1]) : dev::bf16_lo(r.u[k >> 1]);
  else return __uint_as_float(r.u[k]);
}
template <typename T, int NV>
__device__ __forceinline__ float elem(const Raw<NV>& r, int k) {
  return elemb<T, 16 * NV>(r, k);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Sum over aligned groups of LPH lanes (a head's lanes).  Groups up to 16
// lanes use DPP lane swaps (no LDS round trip): xor 1 and xor 2 inside a quad,
// then the half-row mirror (lane i <-> 7 - i) and the row mirror
// (i <-> 15 - i), each of which pairs the lane with the other half of its
// group once the halves are summed.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int LPH>
__device__ __forceinline__ float head_sum(float t) {
  if constexpr (LPH > 1) t += dpp<0xB1>(t);   // quad_perm [1, 0, 3, 2]
  if constexpr (LPH > 2) t += dpp<0x4E>(t);   // quad_perm [2, 3, 0, 1]
  if constexpr (LPH > 4) t += dpp<0x141>(t);  // row_half_mirror
  if constexpr (LPH > 8) t += dpp<0x140>(t);  // row_mirror
  if constexpr (LPH > 16) t += __shfl_xor(t, 16, 64);
  if constexpr (LPH > 32) t += __shfl_xor(t, 32, 64);
  return t;
}

// head_sum with the lanes per head known only at run time (a power of two
// up to 64): xor shuffles through the LDS crossbar, for the generic mapping.
__device__ __forceinline__ float head_sum_rt(float t, int lph) {
  for (int o = 1; o < lph; o <<= 1) t += __shfl_xor(t, o, 64);
  return t;
}

}  // namespace att
}  // namespace gnn
