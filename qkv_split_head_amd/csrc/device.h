// Device helpers for the qkvnr kernels (gfx950, wave64).
//
// Lane geometry.  Every tensor is moved in 16-byte chunks, one per lane:
// 8 bf16 or 4 fp32 values (EPC, elements per chunk).  A head of D values is
// LPH = D / EPC consecutive lanes (8 or 16 for bf16, 16 or 32 for fp32), so a
// wave iteration covers HPI = 64 / LPH whole heads and a head never straddles
// a row of DPP lanes it cannot reach.
//
// Chunk order inside a head.  Rotate-half RoPE pairs value i with value
// i + R/2 (R = D here), i.e. chunk c with chunk c + LPH/2.  Lanes load their
// head's chunks in "mirror" order: lane li of the head holds chunk li for
// li < LPH/2 and chunk 3*LPH/2 - 1 - li above that, so the partner of lane li
// is lane LPH - 1 - li, which DPP reaches in one VALU op (row_half_mirror for
// 8 lanes, row_mirror for 16) without touching LDS.  The 8 (or 16) lanes of a
// head still cover one contiguous 128 (or 256) byte span, so loads and stores
// stay fully coalesced.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkvnr {

constexpr int kWave = 64;

template <typename IO>
struct Chunk;
template <>
struct Chunk<uint16_t> {  // bf16 bit patterns
  static constexpr int EPC = 8;
};
template <>
struct Chunk<float> {
  static constexpr int EPC = 4;
};

// ---------------------------------------------------------------- cross-lane

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int PATTERN>
__device__ __forceinline__ float swizzle(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), PATTERN));
}

// DPP controls (GCN/CDNA encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within 16
// ds_swizzle bitmask mode: and 0x1F, xor mask in bits 14:10.
constexpr int kSwzXor16 = (16 << 10) | 0x1F;
constexpr int kSwzXor31 = (31 << 10) | 0x1F;

// Sum over the LPH lanes of a head; every lane of the head gets the same bits
// (each step adds a pair of values in both orders, and fp add commutes).
template <int LPH>
__device__ __forceinline__ float head_sum(float v) {
  static_assert(LPH == 8 || LPH == 16 || LPH == 32 || LPH == 64, "head lane count");
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  if constexpr (LPH >= 16) v += dpp<kRowMirror>(v);
  if constexpr (LPH >= 32) v += swizzle<kSwzXor16>(v);
  if constexpr (LPH >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// A lane permutation in which every lane has a source lane (the mirrors):
// bound_ctrl set and full masks, so the old value is never read and the
// compiler folds the move into the instruction that uses it (v_mul_f32_dpp)
// instead of zeroing a register and moving into it.
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Value held by the rotate-half partner lane (lane LPH-1-li of the same head).
template <int LPH>
__device__ __forceinline__ float partner(float v) {
  static_assert(LPH == 8 || LPH == 16 || LPH == 32, "head lane count");
  if constexpr (LPH == 8) return dpp_perm<kRowHalfMirror>(v);
  else if constexpr (LPH == 16) return dpp_perm<kRowMirror>(v);
  else return swizzle<kSwzXor31>(v);
}

// Chunk of the head that lane li (0 <= li < LPH) holds: mirror order above LPH/2.
template <int LPH>
__device__ __forceinline__ int chunk_of_lane(int li) {
  return li < LPH / 2 ? li : (3 * LPH / 2 - 1 - li);
}

// ---------------------------------------------------------------- storage

__device__ __forceinline__ void unpack(const uint4& c, float (&f)[8]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void unpack(const uint4& c, float (&f)[4]) {
  f[0] = __uint_as_float(c.x);
  f[1] = __uint_as_float(c.y);
  f[2] = __uint_as_float(c.z);
  f[3] = __uint_as_float(c.w);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Round two fp32 values to bf16 (nearest-even) and pack them: one two-source
// v_cvt_pk_bf16_f32 (two one-value conversions cost a shift and an or more).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint4 pack(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__device__ __forceinline__ uint4 pack(const float (&f)[4]) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Streaming variants: the same 16-byte access with the non-temporal hint.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16_nt(void* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------- RoPE angles

// cos and sin of the angle 2 pi * p * turns_per_pos, where turns_per_pos is
// theta^(-2f/R) / (2 pi) for pair f (tabled on the host).  The product is
// formed in fp64 (p < 2^31, so the angle keeps ~1e-10 rad at any position),
// reduced to (-1/2, 1/2] turns exactly in fp64, and only then evaluated in fp32.
__device__ __forceinline__ void rope_cos_sin(int32_t p, double turns_per_pos, float& c, float& s) {
  const double t = static_cast<double>(p) * turns_per_pos;
  const double fr = t - rint(t);
  sincospif(static_cast<float>(2.0 * fr), &s, &c);
}

}  // namespace qkvnr
