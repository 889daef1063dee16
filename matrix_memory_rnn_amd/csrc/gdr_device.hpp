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

// Raw (undecoded) input words, so loads can be issued early and decoded late.
// R2 holds two consecutive elements, R8 eight. Loads are unconditional: callers
// clamp the row index into range and replace out-of-range rows afterwards with
// `sel`, which keeps the loads branch-free so they issue back to back.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
template <typename T> struct Raw;
template <> struct Raw<__bf16> {
  typedef uint32_t R2;
  typedef u32x4 R8;
  typedef __attribute__((ext_vector_type(2))) uint32_t R4;
  static __device__ __forceinline__ R2 ld2(const __bf16* p) { return *(const uint32_t*)p; }
  static __device__ __forceinline__ R4 ld4(const __bf16* p) { return *(const R4*)p; }
  static __device__ __forceinline__ R8 ld8(const __bf16* p) { return *(const u32x4*)p; }
  static __device__ __forceinline__ f32x4 un4(R4 r) { return f32x4{lo(r[0]), hi(r[0]), lo(r[1]), hi(r[1])}; }
  static __device__ __forceinline__ R4 pad4(float x) { const uint32_t w = pad2(x); return R4{w, w}; }
  static __device__ __forceinline__ R4 sel(bool ok, R4 r, R4 p) { return R4{ok ? r[0] : p[0], ok ? r[1] : p[1]}; }
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  static __device__ __forceinline__ float2 un2(R2 r) { return make_float2(lo(r), hi(r)); }
  static __device__ __forceinline__ void un8(const R8& r, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = lo(r[i]); o[2 * i + 1] = hi(r[i]); }
  }
  static __device__ __forceinline__ R2 pad2(float x) {  // both halves = bf16(x), x exact in bf16
    const uint32_t h = __float_as_uint(x) >> 16;
    return h | (h << 16);
  }
  static __device__ __forceinline__ R2 sel(bool ok, R2 r, R2 p) { return ok ? r : p; }
  static __device__ __forceinline__ R8 zero8() { return u32x4{0u, 0u, 0u, 0u}; }
  static __device__ __forceinline__ R8 sel(bool ok, const R8& r, const R8& p) {
    return u32x4{ok ? r[0] : p[0], ok ? r[1] : p[1], ok ? r[2] : p[2], ok ? r[3] : p[3]};
  }
};
template <> struct Raw<float> {
  typedef float2 R2;
  typedef f32x4 R4;
  struct R8 { f32x4 a, b; };
  static __device__ __forceinline__ R2 ld2(const float* p) { return *(const float2*)p; }
  static __device__ __forceinline__ R4 ld4(const float* p) { return *(const f32x4*)p; }
  static __device__ __forceinline__ f32x4 un4(R4 r) { return r; }
  static __device__ __forceinline__ R4 pad4(float x) { return f32x4{x, x, x, x}; }
  static __device__ __forceinline__ R4 sel(bool ok, R4 r, R4 p) {
    return f32x4{ok ? r[0] : p[0], ok ? r[1] : p[1], ok ? r[2] : p[2], ok ? r[3] : p[3]};
  }
  static __device__ __forceinline__ R8 ld8(const float* p) {
    R8 r;
    r.a = *(const f32x4*)p;
    r.b = *(const f32x4*)(p + 4);
    return r;
  }
  static __device__ __forceinline__ float2 un2(R2 r) { return r; }
  static __device__ __forceinline__ void un8(const R8& r, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[i] = r.a[i]; o[4 + i] = r.b[i]; }
  }
  static __device__ __forceinline__ R2 pad2(float x) { return make_float2(x, x); }
  static __device__ __forceinline__ R2 sel(bool ok, R2 r, R2 p) {
    return make_float2(ok ? r.x : p.x, ok ? r.y : p.y);
  }
  static __device__ __forceinline__ R8 zero8() { return R8{f4zero(), f4zero()}; }
  static __device__ __forceinline__ R8 sel(bool ok, const R8& r, const R8& p) {
    R8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) { o.a[i] = ok ? r.a[i] : p.a[i]; o.b[i] = ok ? r.b[i] : p.b[i]; }
    return o;
  }
};

// Operand precision modes of the contractions. Every LDS operand matrix is
// k-contiguous ([row][k]) and occupies two bf16 "planes" worth of bytes when
// its mode needs them:
//   kBF  — one bf16 plane; 1 MFMA 16x16x32 bf16 per 32-k step.
//   kSP  — bf16 hi plane + bf16 lo plane (x ~ hi + lo, ~16 mantissa bits);
//          3 MFMAs (hi*hi + hi*lo + lo*hi) per step.
//   kF32 — one fp32 plane (the same bytes as hi + lo); 8 MFMAs 16x16x4 fp32
//          per 32-k step, i.e. fp32 products with fp32 accumulation.
// In kF32 the element offset and row pitch are counted in fp32 elements.
constexpr int kBF = 0, kSP = 1, kF32 = 2;

template <int MODE> struct Frag;
template <> struct Frag<kBF> { bf16x8 hi; };
template <> struct Frag<kSP> { bf16x8 hi, lo; };
template <> struct Frag<kF32> { f32x4 a, b; };

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A * B over one 32-wide k step.
template <int MODE>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<MODE>& a, const Frag<MODE>& b) {
  if constexpr (MODE == kBF) {
    acc = mfma_bf16(a.hi, b.hi, acc);
  } else if constexpr (MODE == kSP) {
    acc = mfma_bf16(a.hi, b.hi, acc);
    acc = mfma_bf16(a.hi, b.lo, acc);
    acc = mfma_bf16(a.lo, b.hi, acc);
  } else {
    // instruction e takes k = k0 + 8*(lane/16) + e: lane group g supplies the
    // instruction's k index g, so the 8 instructions cover the 32 k once.
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32(a.a[e], b.a[e], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32(a.b[e], b.b[e], acc);
  }
}

// Load this lane's 8-element slice of a 16-row fragment from a k-contiguous
// LDS matrix: rows row0 + (lane % 16), k = k0 + 8*(lane/16) .. +7.
// Slices at or beyond kend are returned as zeros (tiles are 16-aligned, so a
// slice is either wholly valid or wholly past the end). The lo plane (kSP)
// sits `plane` bytes after the hi plane.
template <int MODE>
__device__ __forceinline__ Frag<MODE> ldfrag(const char* base, int plane, int ld, int row0, int k0,
                                             int kend, int lane) {
  Frag<MODE> f;
  const int k = k0 + 8 * (lane >> 4);
  const int off = (row0 + (lane & 15)) * ld + k;
  if constexpr (MODE == kF32) {
    if (k < kend) {
      const float* p = (const float*)base + off;
      f.a = *(const f32x4*)p;
      f.b = *(const f32x4*)(p + 4);
    } else {
      f.a = f4zero();
      f.b = f4zero();
    }
  } else {
    if (k < kend) {
      const __bf16* p = (const __bf16*)base + off;
      f.hi = *(const bf16x8*)p;
      if constexpr (MODE == kSP) f.lo = *(const bf16x8*)((const char*)p + plane);
    } else {
      f.hi = bf16x8{};
      if constexpr (MODE == kSP) f.lo = bf16x8{};
    }
  }
  return f;
}

// Stores of 4 / 2 / 1 consecutive values in the array's mode.
template <int MODE>
__device__ __forceinline__ void st4(char* base, int plane, int off, f32x4 v) {
  if constexpr (MODE == kF32) {
    *(f32x4*)((float*)base + off) = v;
  } else {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
    bf16x4 h, l;
    __bf16 t0, t1, t2, t3, u0, u1, u2, u3;
    split_bf(v.x, t0, u0); split_bf(v.y, t1, u1); split_bf(v.z, t2, u2); split_bf(v.w, t3, u3);
    h.x = t0; h.y = t1; h.z = t2; h.w = t3;
    *(bf16x4*)((__bf16*)base + off) = h;
    if constexpr (MODE == kSP) {
      l.x = u0; l.y = u1; l.z = u2; l.w = u3;
      *(bf16x4*)((char*)((__bf16*)base + off) + plane) = l;
    }
  }
}

template <int MODE>
__device__ __forceinline__ void st2(char* base, int plane, int off, float a, float b) {
  if constexpr (MODE == kF32) {
    *(float2*)((float*)base + off) = make_float2(a, b);
  } else {
    bf16x2 h, l;
    __bf16 t0, t1, u0, u1;
    split_bf(a, t0, u0); split_bf(b, t1, u1);
    h.x = t0; h.y = t1;
    *(bf16x2*)((__bf16*)base + off) = h;
    if constexpr (MODE == kSP) {
      l.x = u0; l.y = u1;
      *(bf16x2*)((char*)((__bf16*)base + off) + plane) = l;
    }
  }
}

template <int MODE>
__device__ __forceinline__ void st1(char* base, int plane, int off, float a) {
  if constexpr (MODE == kF32) {
    ((float*)base)[off] = a;
  } else {
    __bf16 h, l;
    split_bf(a, h, l);
    ((__bf16*)base)[off] = h;
    if constexpr (MODE == kSP) *(__bf16*)((char*)((__bf16*)base + off) + plane) = l;
  }
}

// acc += A * B with A a split bf16 fragment (hi + lo planes, about 16
// mantissa bits) and B a plain bf16 one: two MFMAs.
__device__ __forceinline__ void mma_split(f32x4& acc, const Frag<kSP>& a, const Frag<kBF>& b) {
  acc = mfma_bf16(a.hi, b.hi, acc);
  acc = mfma_bf16(a.lo, b.hi, acc);
}

// Read one element back as float.
template <int MODE>
__device__ __forceinline__ float ld1(const char* base, int plane, int off) {
  if constexpr (MODE == kF32) return ((const float*)base)[off];
  float x = (float)((const __bf16*)base)[off];
  if constexpr (MODE == kSP) x += (float)*(const __bf16*)((const char*)((const __bf16*)base + off) + plane);
  return x;
}

// Scale an 8-element fragment by per-k factors s[0..7].
template <int MODE>
__device__ __forceinline__ void scale_frag(Frag<MODE>& f, const float* s) {
  if constexpr (MODE == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.a[e] *= s[e]; f.b[e] *= s[4 + e]; }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = (float)f.hi[e];
      if constexpr (MODE == kSP) x += (float)f.lo[e];
      x *= s[e];
      __bf16 h, l;
      split_bf(x, h, l);
      f.hi[e] = h;
      if constexpr (MODE == kSP) f.lo[e] = l;
    }
  }
}

// One 16 x 16 output tile of A B^T on the fp32 matrix cores: A [m][k] and
// B [n][k] fp32 in LDS, k contiguous (pitches lda, ldb in floats, multiples
// of 4), k in [0, K). Accumulator entry e of a lane is row m0 + 4 (lane / 16)
// + e, column n0 + lane % 16.
__device__ __forceinline__ void tile_nt(f32x4& acc, const float* A, int lda, int m0, const float* B, int ldb,
                                        int n0, int K, int lane) {
  for (int k0 = 0; k0 < K; k0 += 32) {
    const Frag<kF32> a = ldfrag<kF32>((const char*)A, 0, lda, m0, k0, K, lane);
    const Frag<kF32> b = ldfrag<kF32>((const char*)B, 0, ldb, n0, k0, K, lane);
    mma<kF32>(acc, a, b);
  }
}

// The same tile for K = 16: lane group g supplies k = 4g .. 4g+3 of its row,
// instruction e takes k = 4g + e from group g, so four instructions cover the
// 16 k once (tile_nt would run eight, half of them on zeros).
__device__ __forceinline__ void tile_nt16(f32x4& acc, const float* A, int lda, int m0, const float* B, int ldb,
                                          int n0, int lane) {
  const int k = 4 * (lane >> 4);
  const f32x4 a = *(const f32x4*)(A + (m0 + (lane & 15)) * lda + k);
  const f32x4 b = *(const f32x4*)(B + (n0 + (lane & 15)) * ldb + k);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], b[e], acc);
}

// A staging loop x = tid, tid + NT, .. < N over compile-time N and NT, fully
// unrolled, so that the loads of all its iterations are issued before the
// first of them is used: a plain strided loop (whose trip count the compiler
// cannot see) waits for each iteration's loads before issuing the next. Loads
// inside must be unconditional to be issued together: clamp the row with
// row_in and select the value afterwards.
#define GDR_STAGE_FOR(x, N, NT)                                                       \
  _Pragma("unroll") for (int x##_it = 0; x##_it < ((N) + (NT) - 1) / (NT); ++x##_it) \
    if (const int x = tid + x##_it * (NT); (N) % (NT) == 0 || x < (N))

// Row t of a sequence of T rows, or its last row when t is past the end (the
// caller replaces what it read there).
__device__ __forceinline__ int row_in(int t, int T) { return t < T ? t : T - 1; }

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

// ---- gate activations of "Muir: ..." (§2.1 "Gated DeltaNet-2", §4.1 eq.(9)
// and the gate list after it), evaluated in fp32 from the logits:
//   log alpha = -exp(a_log) * softplus(z_f),  b = 2 sigmoid(z_b),
//   w = sigmoid(z_w),  gamma = gamma_stat * 2 sigmoid(z_q).
// softplus(z) = max(z, 0) + log(1 + e^{-|z|}) has no overflow for large |z|
// and gives 0 at z = -inf (alpha = 1, the identity padding of a ragged tail).
// The hardware exp2/log2/reciprocal forms (__expf, __logf, v_rcp_f32, about
// 1 ulp each) keep the prologue cheap; log(1 + x) for x below float epsilon
// returns 0 instead of x, an absolute error under 6e-8 in softplus.
__device__ __forceinline__ float gate_softplus(float z) { return fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z))); }
__device__ __forceinline__ float gate_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }
// alpha from its logit; rate = exp(a_log) of the head
__device__ __forceinline__ float gate_alpha(float z, float rate) { return __expf(-rate * gate_softplus(z)); }

}  // namespace gdr
