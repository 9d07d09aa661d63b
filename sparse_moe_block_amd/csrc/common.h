// Shared device helpers for the ZAYA1 block kernels (gfx950 / CDNA4).
//
// Element types: activations are either bf16 (stored as uint16_t, bf16_t below) or
// fp32; the residual stream is always fp32. Every rounding to bf16 is IEEE
// round-to-nearest-even, done explicitly so results do not depend on compiler
// conversion defaults.
//
// MFMA fragments: both supported element types use a 16x16 output tile over a
// 32-long slice of K. Lane l supplies row (l % 16) of each operand and the eight
// consecutive K elements [8*(l/16), 8*(l/16)+8); lane l receives output rows
// 4*(l/16)+i, i < 4, of column (l % 16). For bf16 this is one
// v_mfma_f32_16x16x32_bf16; for fp32 it is eight v_mfma_f32_16x16x4_f32, the s-th
// taking element s of every lane's eight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zaya {

typedef uint16_t bf16_t;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // native 16-byte register quad
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): one v_cvt_pk_bf16_f32. Checked
// against the bit-level rounding rule on all 2^32 inputs, denormals and NaNs included.
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// acc + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (v_dot2_f32_bf16: the products
// are exact in fp32, the sum accumulates in fp32).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), acc, false);
}

// Cached tokens of sequence b: a null table means every sequence is fresh.
__device__ __forceinline__ int cached_len(const int32_t* cache_len, int b) { return cache_len ? cache_len[b] : 0; }

// Round an fp32 value to the act type and back.
template <typename T> struct Act;
template <> struct Act<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static float rnd(float f) { return bf2f(f2bf(f)); }
  __device__ __forceinline__ static bf16_t cvt(float f) { return f2bf(f); }
  __device__ __forceinline__ static float tof(bf16_t h) { return bf2f(h); }
};
template <> struct Act<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float rnd(float f) { return f; }
  __device__ __forceinline__ static float cvt(float f) { return f; }
  __device__ __forceinline__ static float tof(float h) { return h; }
};

// Four consecutive act values <-> four floats (8 bytes of bf16 or 16 bytes of fp32).
__device__ __forceinline__ void load4(const bf16_t* p, float* v) {
  uint2 r = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(r.x << 16);
  v[1] = __uint_as_float(r.x & 0xFFFF0000u);
  v[2] = __uint_as_float(r.y << 16);
  v[3] = __uint_as_float(r.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  float4 r = *reinterpret_cast<const float4*>(p);
  v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi);
__device__ __forceinline__ void store4(bf16_t* p, const float* v) {  // v already rounded or not: rounds here
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Two floats -> packed bf16 pair (low half = lo), hardware round-to-nearest-even.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// MFMA fragment traits.
template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  struct frag { uint4 v; };  // 8 bf16
  static constexpr int kFragBytes = 16;
  __device__ __forceinline__ static frag load(const bf16_t* p) { return frag{*reinterpret_cast<const uint4*>(p)}; }
  __device__ __forceinline__ static frag zero() { return frag{make_uint4(0, 0, 0, 0)}; }
  __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
                                                   c, 0, 0, 0);
  }
  // Build a fragment from 8 floats (each rounded to the nearest bf16).
  __device__ __forceinline__ static frag pack(const float* f) {
    frag r;
    r.v.x = pack_bf16x2(f[0], f[1]);
    r.v.y = pack_bf16x2(f[2], f[3]);
    r.v.z = pack_bf16x2(f[4], f[5]);
    r.v.w = pack_bf16x2(f[6], f[7]);
    return r;
  }
};
template <> struct Mfma<float> {
  struct frag { float4 a, b; };  // 8 fp32
  static constexpr int kFragBytes = 32;
  __device__ __forceinline__ static frag load(const float* p) {
    return frag{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  __device__ __forceinline__ static frag zero() { return frag{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)}; }
  __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, b.a.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, b.a.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, b.a.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, b.a.w, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, b.b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, b.b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, b.b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, b.b.w, c, 0, 0, 0);
    return c;
  }
  __device__ __forceinline__ static frag pack(const float* f) {
    return frag{make_float4(f[0], f[1], f[2], f[3]), make_float4(f[4], f[5], f[6], f[7])};
  }
};

// Reductions over aligned groups of N lanes (N a power of two, 2 .. 64); every lane of a
// group ends with the same result. Inside a 16-lane row the partners come from DPP moves
// (lane ^ 1 and ^ 2 by quad permutes, then the mirror of each 8-lane half and of the
// row, each pairing one half's lanes with the other's), which stay in the vector ALU;
// the steps across rows are cross-lane reads.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int N, class Op>
__device__ __forceinline__ float lane_group_reduce(float v, Op op) {
  static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "group of 2 .. 64 lanes");
  v = op(v, dpp_mov<0xB1>(v));                          // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) v = op(v, dpp_mov<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) v = op(v, dpp_mov<0x141>(v));   // row_half_mirror
  if constexpr (N >= 16) v = op(v, dpp_mov<0x140>(v));  // row_mirror
  if constexpr (N >= 32) v = op(v, __shfl_xor(v, 16, 64));
  if constexpr (N >= 64) v = op(v, __shfl_xor(v, 32, 64));
  return v;
}
struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) { return lane_group_reduce<N>(v, OpAdd{}); }
__device__ __forceinline__ float wave_sum(float v) { return lane_group_reduce<64>(v, OpAdd{}); }
__device__ __forceinline__ float wave_max(float v) { return lane_group_reduce<64>(v, OpMax{}); }

// Non-contracted fp32 ops: the residual stream is float32 op by op.
__device__ __forceinline__ float fadd(float a, float b) { return __fadd_rn(a, b); }
__device__ __forceinline__ float fmul(float a, float b) { return __fmul_rn(a, b); }

// XCD-aware remap of a linear workgroup id: the hardware deals consecutive ids to the
// 8 XCDs in turn; this returns a logical id such that consecutive logical ids run on
// the same XCD (sharing its L2). Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  if (nwg % 8) return wg;
  return (wg % 8) * (nwg / 8) + wg / 8;
}

}  // namespace zaya
