// Device-side helpers shared by the gfx950 kernels of libgdr: element types,
// bf16 packing, LDS fragment loads and the 16x16x32 bf16 MFMA step.
//
// MFMA lane layout used throughout (v_mfma_f32_16x16x32_bf16, wave64):
//   A operand (16 rows x 32 k): lane l supplies row (l % 16), k = 8*(l/16) .. +7
//   B operand (32 k x 16 cols): lane l supplies col (l % 16), k = 8*(l/16) .. +7
//   accumulator (16 x 16):      lane l holds rows 4*(l/16) + i (i = 0..3), col (l % 16)
// Both operands are kept in LDS "k-contiguous": A as [row][k], B as [col][k].
// A and B use the same (lane group, element) -> k assignment, so the
// contraction covers every k exactly once whatever order the hardware uses
// inside an instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kWave = 64;

__device__ __forceinline__ f32x4 f4zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

// float -> bf16 (round to nearest even, the gfx950 v_cvt_pk_bf16_f32 rounding)
__device__ __forceinline__ __bf16 f2bf(float x) { return (__bf16)x; }

// hi/lo split: hi = bf16(x), lo = bf16(x - hi); hi + lo carries ~16 mantissa bits.
__device__ __forceinline__ void split_bf(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// Input element loads (2 or 4 consecutive elements) as float.
template <typename T> struct In;
template <> struct In<float> {
  static __device__ __forceinline__ float2 load2(const float* p) { return *(const float2*)p; }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};
template <> struct In<__bf16> {
  static __device__ __forceinline__ float2 load2(const __bf16* p) {
    bf16x2 v = *(const bf16x2*)p;
    return make_float2((float)v.x, (float)v.y);
  }
  static __device__ __forceinline__ float load1(const __bf16* p) { return (float)*p; }
  static __device__ __forceinline__ void store4(__bf16* p, f32x4 v) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
    bf16x4 o;
    o.x = (__bf16)v.x; o.y = (__bf16)v.y; o.z = (__bf16)v.z; o.w = (__bf16)v.w;
    *(bf16x4*)p = o;
  }
  static __device__ __forceinline__ void store1(__bf16* p, float v) { *p = (__bf16)v; }
};

// One MFMA operand fragment: 8 bf16 (hi) and, for split precision, 8 more (lo).
template <bool SPLIT> struct Frag {
  bf16x8 hi;
  bf16x8 lo;
};

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += A * B with 1 MFMA (hi*hi) or 3 MFMAs (hi*hi + hi*lo + lo*hi).
template <bool SPLIT>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<SPLIT>& a, const Frag<SPLIT>& b) {
  acc = mfma_bf16(a.hi, b.hi, acc);
  if constexpr (SPLIT) {
    acc = mfma_bf16(a.hi, b.lo, acc);
    acc = mfma_bf16(a.lo, b.hi, acc);
  }
}

// Load this lane's 8-element slice of a 16-row fragment from a k-contiguous
// LDS matrix: rows row0 + (lane % 16), k = k0 + 8*(lane/16) .. +7.
// Slices at or beyond kend are returned as zeros (tiles are 16-aligned, so a
// slice is either wholly valid or wholly past the end). The lo plane, when
// present, sits `plane` bytes after the hi plane.
template <bool SPLIT>
__device__ __forceinline__ Frag<SPLIT> ldfrag(const char* base, int plane, int ld, int row0, int k0,
                                              int kend, int lane) {
  Frag<SPLIT> f;
  const int k = k0 + 8 * (lane >> 4);
  if (k < kend) {
    const __bf16* p = (const __bf16*)base + (row0 + (lane & 15)) * ld + k;
    f.hi = *(const bf16x8*)p;
    if constexpr (SPLIT) f.lo = *(const bf16x8*)((const char*)p + plane);
  } else {
    f.hi = bf16x8{};
    if constexpr (SPLIT) f.lo = bf16x8{};
  }
  return f;
}

// Store 4 consecutive values (k-contiguous) as bf16 hi [+ lo] planes.
template <bool SPLIT>
__device__ __forceinline__ void st4(char* base, int plane, int off_elems, f32x4 v) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  bf16x4 h, l;
  __bf16 t0, t1, t2, t3, u0, u1, u2, u3;
  split_bf(v.x, t0, u0); split_bf(v.y, t1, u1); split_bf(v.z, t2, u2); split_bf(v.w, t3, u3);
  h.x = t0; h.y = t1; h.z = t2; h.w = t3;
  *(bf16x4*)((__bf16*)base + off_elems) = h;
  if constexpr (SPLIT) {
    l.x = u0; l.y = u1; l.z = u2; l.w = u3;
    *(bf16x4*)((char*)((__bf16*)base + off_elems) + plane) = l;
  }
}

// Store 2 consecutive values as bf16 hi [+ lo].
template <bool SPLIT>
__device__ __forceinline__ void st2(char* base, int plane, int off_elems, float a, float b) {
  bf16x2 h, l;
  __bf16 t0, t1, u0, u1;
  split_bf(a, t0, u0); split_bf(b, t1, u1);
  h.x = t0; h.y = t1;
  *(bf16x2*)((__bf16*)base + off_elems) = h;
  if constexpr (SPLIT) {
    l.x = u0; l.y = u1;
    *(bf16x2*)((char*)((__bf16*)base + off_elems) + plane) = l;
  }
}

// Store 1 value as bf16 hi [+ lo].
template <bool SPLIT>
__device__ __forceinline__ void st1(char* base, int plane, int off_elems, float a) {
  __bf16 h, l;
  split_bf(a, h, l);
  ((__bf16*)base)[off_elems] = h;
  if constexpr (SPLIT) *(__bf16*)((char*)((__bf16*)base + off_elems) + plane) = l;
}

// Scale an 8-element fragment (hi [+ lo]) by per-k factors s[0..7], re-rounding.
template <bool SPLIT>
__device__ __forceinline__ void scale_frag(Frag<SPLIT>& f, const float* s) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = (float)f.hi[e];
    if constexpr (SPLIT) x += (float)f.lo[e];
    x *= s[e];
    __bf16 h, l;
    split_bf(x, h, l);
    f.hi[e] = h;
    if constexpr (SPLIT) f.lo[e] = l;
  }
}

// Workgroup index -> linear work index that places consecutive work items of
// one group (e.g. the value tiles of one head) on the same XCD. Workgroups are
// dispatched round-robin over the 8 XCDs of an MI355X; each XCD has its own L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks, int group) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  const int per = nblocks / kXcd;
  if (per % group != 0) return bid;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace gdr
