// One-token decode step of the channel-wise gated delta rule on gfx950.
//
// Per (sequence n, head h), "Muir: Linear Attention with Sensitivity-Allocated
// Gating and Matched-Filter Readout", §2.1 eq.(1):
//     S <- (I - k^T (b*k)) Diag(alpha) S + k^T (w*v),   o = q S.
// Expanded so the d_k x d_v state is read once and written once:
//     r = (alpha*b*k) S,  p = (alpha*q) S          (one pass over S)
//     u = w*v - r
//     S <- Diag(alpha) S + k^T u,  o = p + (q . k) u.
// The step is a streaming read-modify-write of S (HBM-bound): one workgroup
// per state, 256 threads, each thread holding DK*DV/256 state elements as
// float4 rows segments (d_v contiguous, so every wave reads whole rows).
//
// GATED (the Muir gate prologue, "Muir: ...", §2.1 and §4.1): alpha, bgate and
// wgate hold the logits z_f, z_b, z_w; alpha = exp(-exp(a_log) softplus(z_f)),
// b = 2 sigmoid(z_b), w = sigmoid(z_w) and the query is gamma * q with
// gamma = gamma_stat * 2 sigmoid(z_q), all formed here in fp32.
#include "gdr_device.hpp"
#include "gdr_internal.h"

namespace gdr {

template <typename Tin, int DK, int DV, bool GATED>
__global__ __launch_bounds__(256) void gdn2_decode_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ alpha, const Tin* __restrict__ bgate, const Tin* __restrict__ wgate,
    float* __restrict__ S, Tin* __restrict__ o, const Tin* __restrict__ zq,
    const float* __restrict__ alog, const float* __restrict__ gstat, int H) {
  constexpr int TPR = DV / 4;                 // threads per state row (float4 each)
  constexpr int RPP = 256 / TPR;              // rows per pass
  constexpr int NPASS = (DK + RPP - 1) / RPP;
  __shared__ float s_qa[DK], s_kb[DK], s_al[DK], s_k[DK], s_vh[DV], s_qh[DK];
  __shared__ float s_red[2][RPP][DV];
  __shared__ float s_qk;

  const int tid = threadIdx.x;
  const size_t head = blockIdx.x;
  const size_t offK = head * DK, offV = head * DV;
  float* Sh = S + head * DK * DV;

  const int c4 = (tid % TPR) * 4;
  const int rg = tid / TPR;
  // issue the state loads first: they are the bulk of the traffic
  f32x4 st[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int j = rg + RPP * p;
    st[p] = (rg < RPP && j < DK) ? *(const f32x4*)(Sh + (size_t)j * DV + c4) : f4zero();
  }
  float rate = 1.f;
  if constexpr (GATED) rate = expf(alog[head % H]);
  for (int j = tid; j < DK; j += 256) {
    float a = In<Tin>::load1(alpha + offK + j);
    const float kk = In<Tin>::load1(k + offK + j);
    float bb = In<Tin>::load1(bgate + offK + j);
    float qq = In<Tin>::load1(q + offK + j);
    if constexpr (GATED) {
      a = gate_alpha(a, rate);
      bb = 2.f * gate_sigmoid(bb);
      const float zz = zq ? In<Tin>::load1(zq + offK + j) : 0.f;
      qq *= (gstat ? gstat[(head % H) * DK + j] : 1.f) * 2.f * gate_sigmoid(zz);
    }
    s_al[j] = a;
    s_k[j] = kk;
    s_kb[j] = a * bb * kk;
    s_qa[j] = a * qq;
    s_qh[j] = qq;
  }
  for (int c = tid; c < DV; c += 256) {
    float ww = In<Tin>::load1(wgate + offV + c);
    if constexpr (GATED) ww = gate_sigmoid(ww);
    s_vh[c] = ww * In<Tin>::load1(v + offV + c);
  }
  __syncthreads();
  if (tid < 64) {  // q . k by one wave
    float acc = 0.f;
    for (int j = tid; j < DK; j += 64) acc += s_qh[j] * s_k[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (tid == 0) s_qk = acc;
  }

  f32x4 r = f4zero(), pq = f4zero();
  if (rg < RPP) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int j = rg + RPP * p;
      if (j < DK) {
        const float kb = s_kb[j], qa = s_qa[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] += kb * st[p][e];
          pq[e] += qa * st[p][e];
        }
      }
    }
    *(f32x4*)&s_red[0][rg][c4] = r;
    *(f32x4*)&s_red[1][rg][c4] = pq;
  }
  __syncthreads();
  // every thread needs u for its 4 columns: sum the RPP partials
  f32x4 u = f4zero(), pr = f4zero();
  for (int x = 0; x < RPP; ++x) {
    const f32x4 a = *(const f32x4*)&s_red[0][x][c4];
    const f32x4 b = *(const f32x4*)&s_red[1][x][c4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { u[e] += a[e]; pr[e] += b[e]; }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = s_vh[c4 + e] - u[e];
  if (rg < RPP) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int j = rg + RPP * p;
      if (j < DK) {
        const float a = s_al[j], kk = s_k[j];
        f32x4 nv;
#pragma unroll
        for (int e = 0; e < 4; ++e) nv[e] = a * st[p][e] + kk * u[e];
        // non-temporal: the new state is not read again in this step (at
        // 512 x 16 heads, a state larger than the last-level cache, 63% of
        // HBM peak with plain stores, 82% with these)
        __builtin_nontemporal_store(nv, (f32x4*)(Sh + (size_t)j * DV + c4));
      }
    }
  }
  if (rg == 0) {
    const float qk = s_qk;
    f32x4 ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = pr[e] + qk * u[e];
    In<Tin>::store4(o + offV + c4, ov);
  }
}

template <typename Tin, int DK, int DV>
static int launch_decode(const DecodeArgs& a) {
  const Tin *q = (const Tin*)a.q, *k = (const Tin*)a.k, *v = (const Tin*)a.v;
  const Tin *al = (const Tin*)a.alpha, *bg = (const Tin*)a.b, *wg = (const Tin*)a.w;
  float* S = a.S;
  Tin* o = (Tin*)a.o;
  const Tin* zq = (const Tin*)a.zq;
  const float *alog = a.a_log, *gst = a.gamma_stat;
  int H = a.H;
  void* args[] = {&q, &k, &v, &al, &bg, &wg, &S, &o, &zq, &alog, &gst, &H};
  const void* kern = a.gated ? (const void*)gdn2_decode_kernel<Tin, DK, DV, true>
                             : (const void*)gdn2_decode_kernel<Tin, DK, DV, false>;
  hipError_t e = hipLaunchKernel(kern, dim3(a.N * a.H), dim3(256), args, 0, (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

template <typename Tin, int DK>
static int decode_dv(const DecodeArgs& a) {
  switch (a.dv) {
    case 16: return launch_decode<Tin, DK, 16>(a);
    case 32: return launch_decode<Tin, DK, 32>(a);
    case 64: return launch_decode<Tin, DK, 64>(a);
    case 128: return launch_decode<Tin, DK, 128>(a);
  }
  return GDR_ERR_UNSUPPORTED;
}

template <typename Tin>
static int decode_dk(const DecodeArgs& a) {
  switch (a.dk) {
    case 16: return decode_dv<Tin, 16>(a);
    case 32: return decode_dv<Tin, 32>(a);
    case 64: return decode_dv<Tin, 64>(a);
    case 128: return decode_dv<Tin, 128>(a);
  }
  return GDR_ERR_UNSUPPORTED;
}

int decode_launch(const DecodeArgs& a) {
  return a.dtype == GDR_BF16 ? decode_dk<__bf16>(a) : decode_dk<float>(a);
}

}  // namespace gdr
