// Helpers shared by the chunkwise kernels of the channel-wise gated delta
// rule (the fused single-kernel form and the two-kernel intra/scan form):
// block-pair indexing, the exact in-block decay fallback, wave-local LDS
// ordering and fp32 operand slices.
#pragma once

#include "gdr_device.hpp"

namespace gdr {

constexpr float kGuardMin = 8.673617379884035e-19f;  // 2^-60

constexpr int align16(int x) { return (x + 15) / 16 * 16; }
constexpr int imax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ int pidx(int I, int J) { return I * (I + 1) / 2 + J; }

__device__ __forceinline__ void pair_of(int p, int& I, int& J) {
  I = 0;
  while ((I + 1) * (I + 2) / 2 <= p) ++I;
  J = p - I * (I + 1) / 2;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 8 consecutive fp32 values from LDS as an operand slice of the given mode.
template <int MODE>
__device__ __forceinline__ Frag<MODE> frag_f32(const float* p, bool valid) {
  Frag<MODE> f;
  f32x4 a = valid ? *(const f32x4*)p : f4zero();
  f32x4 b = valid ? *(const f32x4*)(p + 4) : f4zero();
  if constexpr (MODE == kF32) {
    f.a = a;
    f.b = b;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h, l;
      split_bf(a[e], h, l);
      f.hi[e] = h;
      if constexpr (MODE == kSP) f.lo[e] = l;
      split_bf(b[e], h, l);
      f.hi[4 + e] = h;
      if constexpr (MODE == kSP) f.lo[4 + e] = l;
    }
  }
  return f;
}

// Gate values as the exact path reads them: the stored gates, or (GATED, the
// Muir gate prologue) the gates formed from their logits: alpha from z_f,
// b = 2 sigmoid(z_b), and the query scaled by gamma = gstat * 2 sigmoid(z_q)
// (gz = this head's gstat row or NULL, zq NULL for z_q = 0).
template <typename Tin, bool GATED>
struct GateRead {
  const Tin* zq;
  const float* gz;
  float rate;
  __device__ __forceinline__ float alpha(const Tin* p) const {
    const float x = In<Tin>::load1(p);
    if constexpr (GATED) return gate_alpha(x, rate);
    else return x;
  }
  __device__ __forceinline__ float erase(const Tin* p) const {
    const float x = In<Tin>::load1(p);
    if constexpr (GATED) return 2.f * gate_sigmoid(x);
    else return x;
  }
  __device__ __forceinline__ float query(const Tin* q, size_t off, int j) const {
    const float x = In<Tin>::load1(q + off);
    if constexpr (GATED) {
      const float z = zq ? In<Tin>::load1(zq + off) : 0.f;
      return x * (gz ? gz[j] : 1.f) * 2.f * gate_sigmoid(z);
    } else {
      return x;
    }
  }
};

// Exact in-block Gram entries for the tile (I, I) from alpha products (slow path).
template <typename Tin, int DK, bool GATED = false>
__device__ void exact_diag(const Tin* __restrict__ k, const Tin* __restrict__ bg,
                           const Tin* __restrict__ q, const Tin* __restrict__ al,
                           size_t seqK, int t0, int T, int t, int s0, f32x4& lv, f32x4& mv,
                           GateRead<Tin, GATED> gr = GateRead<Tin, GATED>{nullptr, nullptr, 1.f}) {
  float aL[4] = {0.f, 0.f, 0.f, 0.f}, aM[4] = {0.f, 0.f, 0.f, 0.f};
  const int tg = t0 + t;
  if (tg < T && t >= s0) {
    for (int j = 0; j < DK; ++j) {
      const size_t rt = seqK + (size_t)tg * DK + j;
      const float kt = In<Tin>::load1(k + rt);
      const float kh = kt * gr.erase(bg + rt);
      const float qt = gr.query(q, rt, j);
      float p = 1.f;  // prod_{r=s+1..t} alpha_r
      for (int s = t; s >= s0; --s) {
        if (s < t) p *= gr.alpha(al + seqK + (size_t)(t0 + s + 1) * DK + j);
        const int e = s - s0;
        if (e < 4) {
          const float ks = In<Tin>::load1(k + seqK + (size_t)(t0 + s) * DK + j) * p;
          if (s < t) aL[e] += kh * ks;
          aM[e] += qt * ks;
        }
      }
    }
  }
  lv = f32x4{aL[0], aL[1], aL[2], aL[3]};
  mv = f32x4{aM[0], aM[1], aM[2], aM[3]};
}

// Off-diagonal pair index q -> (I, J), J < I.
__device__ __forceinline__ void offpair_of(int q, int& I, int& J) {
  I = 1;
  while ((I + 1) * I / 2 <= q) ++I;
  J = q - I * (I - 1) / 2;
}

}  // namespace gdr
