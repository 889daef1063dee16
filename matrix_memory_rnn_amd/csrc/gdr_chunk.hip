// Chunkwise forward of the channel-wise gated delta rule on gfx950.
//
// Method: "Muir: Linear Attention with Sensitivity-Allocated Gating and
// Matched-Filter Readout", §2.1 eq.(1) evaluated with the chunkwise UT form of
// §2.2. For one chunk of C tokens starting from state S0 (rows t = 0..C-1):
//   L[t][s] = <k^_t, pi_{t,s} * k_s>  (t > s),   M[t][s] = <q_t, pi_{t,s} * k_s>  (t >= s),
//   T = I + L,   R = V^ - K^_pi S0,   V~ = T^{-1} R,
//   O = Q_pi S0 + M V~,   S_C = Diag(pi_C) S0 + K~^T V~,
// with k^ = b*k, v^ = w*v, pi_{t,s} = prod_{r=s+1..t} alpha_r, rows of K^_pi,
// Q_pi are pi_t * k^_t, pi_t * q_t (pi_t = prod_{r<=t} alpha_r) and rows of K~
// are pi_{C,s} * k_s. (§2.2 states T V~ = V^ - K^_pi S0; solving it with the
// explicit T^{-1} applied to the VT value columns of this workgroup avoids the
// d_k-wide Y = T^{-1} K^_pi of the page's fused solve.)
//
// Decays. The chunk is cut into 16-row blocks. Per block and channel the kernel
// keeps the inclusive prefix product P_t (from the block start through t), the
// exclusive suffix product Qs_s (after s to the block end) and the block total
// G. Every pi needed is then a product of factors <= 1:
//   cross-block (t in block I, s in block J < I):
//       pi_{t,s} = P_t * prod_{J<K<I} G_K * Qs_s
//   (the boundary-pivot split of §4.2, with pivots at the 16-row boundaries);
//   in-block (t >= s in block I): pi_{t,s} = P_t * (Qs_s / G_I), used only
//   when G_I >= 2^-60 on every channel of the block, so Qs_s/G_I <= 2^60 stays
//   in range; otherwise that diagonal tile is recomputed exactly from products
//   of alphas (slow path, never taken unless some channel decays below 2^-60
//   within 16 tokens).
// No logarithm, exponential or division by a cumulative decay is taken.
//
// Work split: one workgroup (256 threads, 4 waves) per (sequence b, head h,
// value tile of VT columns). Value columns of S evolve independently (eq.(1)
// acts on S from the left), so the tiles need no communication; each walks
// all chunks of its head, holding its S tile (d_k x VT, fp32) in registers.
//
// Precision: operands of every contraction are bf16 in LDS with fp32
// accumulation. For float32 inputs (SPLIT) every operand carries a second bf16
// plane with the rounding residual and each product takes three MFMAs
// (hi*hi + hi*lo + lo*hi). T^{-1} is always built from split operands.
#include "gdr_device.hpp"
#include "gdr_internal.h"

namespace gdr {

constexpr float kGuardMin = 8.673617379884035e-19f;  // 2^-60

template <int DK, int VT, int CM, bool SPLIT>
struct ChunkSmem {
  static constexpr int NS = SPLIT ? 2 : 1;
  static constexpr int NBM = CM / 16;
  static constexpr int LDK = DK + 8;   // bf16 pitch, rows of length DK
  static constexpr int LDC = CM + 8;   // bf16 pitch, rows of length C
  static constexpr int LDF = CM + 4;   // fp32 pitch, rows of length C
  static constexpr int LDZ = 24;       // bf16 pitch of the 16x16 merge scratch
  static constexpr int P_CK = CM * LDK * 2;
  static constexpr int P_CC = CM * LDC * 2;
  static constexpr int P_KC = DK * LDC * 2;
  static constexpr int P_VC = VT * LDC * 2;
  static constexpr int P_VK = VT * LDK * 2;
  static constexpr int P_Z = 16 * LDZ * 2;
  // region X, first use (prep -> Gram): row-block-relative operands
  static constexpr int KR = 0;                       // k^ * P          [C][DK]
  static constexpr int QR = KR + NS * P_CK;          // q * P           [C][DK]
  static constexpr int KC = QR + NS * P_CK;          // k * Qs          [C][DK]
  static constexpr int KHP = KC + NS * P_CK;         // -(k^ * pi_t)    [C][DK]
  static constexpr int QHP = KHP + NS * P_CK;        // q * pi_t        [C][DK]
  static constexpr int VH = QHP + NS * P_CK;         // v^ (fp32)       [VT][C]
  static constexpr int X1_END = VH + VT * LDF * 4;
  // region X, second use (after the Gram products)
  static constexpr int LF = 0;                       // L (fp32)        [C][C]
  static constexpr int LB = LF + CM * LDF * 4;       // L hi/lo         [C][C]
  static constexpr int TN = LB + 2 * P_CC;           // T^-1 hi/lo      [t][s]
  static constexpr int TT = TN + 2 * P_CC;           // T^-T hi/lo      [s][t]
  static constexpr int ZT = TT + 2 * P_CC;           // 4 waves x 16x16 hi/lo
  static constexpr int RT = ZT + 4 * 2 * P_Z;        // R^T             [VT][C]
  static constexpr int X2_END = RT + NS * P_VC;
  static constexpr int X_END = X1_END > X2_END ? X1_END : X2_END;
  // persistent across the chunk
  static constexpr int MB = (X_END + 15) / 16 * 16;  // M               [t][s]
  static constexpr int KTT = MB + NS * P_CC;         // K~^T            [DK][C]
  static constexpr int VTT = KTT + NS * P_KC;        // V~^T            [VT][C]
  static constexpr int S0T = VTT + NS * P_VC;        // S0^T            [VT][DK]
  static constexpr int GS = S0T + NS * P_VK;         // G (fp32)        [NB][DK]
  static constexpr int PIC = GS + NBM * DK * 4;      // pi_C (fp32)     [DK]
  static constexpr int FLAG = PIC + DK * 4;          // guard flags     [4]
  static constexpr int TOTAL = FLAG + 16;
  static_assert(TOTAL <= 160 * 1024, "chunk kernel LDS exceeds 160 KiB");
};

__device__ __forceinline__ void pair_of(int p, int& I, int& J) {
  I = 0;
  while ((I + 1) * (I + 2) / 2 <= p) ++I;
  J = p - I * (I + 1) / 2;
}

// Exact in-block Gram entries for the tile (I, I) from alpha products (slow path).
template <typename Tin, int DK>
__device__ void exact_diag(const Tin* __restrict__ k, const Tin* __restrict__ bg,
                           const Tin* __restrict__ q, const Tin* __restrict__ al,
                           size_t seqK, int t0, int T, int t, int s0, f32x4& lv, f32x4& mv) {
  float aL[4] = {0.f, 0.f, 0.f, 0.f}, aM[4] = {0.f, 0.f, 0.f, 0.f};
  const int tg = t0 + t;
  if (tg < T && t >= s0) {
    for (int j = 0; j < DK; ++j) {
      const float kt = In<Tin>::load1(k + seqK + (size_t)tg * DK + j);
      const float kh = kt * In<Tin>::load1(bg + seqK + (size_t)tg * DK + j);
      const float qt = In<Tin>::load1(q + seqK + (size_t)tg * DK + j);
      float p = 1.f;  // prod_{r=s+1..t} alpha_r
      for (int s = t; s >= s0; --s) {
        if (s < t) p *= In<Tin>::load1(al + seqK + (size_t)(t0 + s + 1) * DK + j);
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

template <typename Tin, int DK, int VT, int CM, bool SPLIT>
__global__ __launch_bounds__(256, 1) void gdn2_chunk_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ alpha, const Tin* __restrict__ bgate, const Tin* __restrict__ wgate,
    const float* __restrict__ S0, Tin* __restrict__ o, float* S_out, int T, int DV, int C) {
  using L = ChunkSmem<DK, VT, CM, SPLIT>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NVL = VT / 16;                       // 16-col value tiles per workgroup
  constexpr int NST = (DK / 16) * NVL;               // S accumulator tiles
  constexpr int MAXS = (NST + 3) / 4;
  constexpr int NBM = CM / 16;
  constexpr int MAXP = (NBM * (NBM + 1) / 2 + 3) / 4;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nvt = DV / VT;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int bh = lin / nvt, vt0 = (lin % nvt) * VT;
  const int NB = C / 16, NP = NB * (NB + 1) / 2;
  const int nchunks = (T + C - 1) / C;
  const size_t seqK = (size_t)bh * T * DK;
  const size_t seqV = (size_t)bh * T * DV;
  const size_t stOff = (size_t)bh * DK * DV;

  float* GS = (float*)(smem + L::GS);
  float* PIC = (float*)(smem + L::PIC);
  int* FLAGS = (int*)(smem + L::FLAG);
  float* VH = (float*)(smem + L::VH);
  float* LF = (float*)(smem + L::LF);

  // ---- state tile -> registers and S0^T (bf16) in LDS
  f32x4 Sacc[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    Sacc[i] = f4zero();
    const int tile = wid + 4 * i;
    if (tile < NST) {
      const int jt = tile / NVL, vl = tile % NVL;
      if (S0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Sacc[i][e] = S0[stOff + (size_t)(16 * jt + 4 * g + e) * DV + vt0 + 16 * vl + c16];
      }
      st4<SPLIT>(smem + L::S0T, L::P_VK, (16 * vl + c16) * L::LDK + 16 * jt + 4 * g, Sacc[i]);
    }
  }
  if (tid < 4) FLAGS[tid] = 0;
  __syncthreads();

  f32x4 Oacc[NVL];

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * C;

    // ================= prep, pass 1: block prefix products and block totals
    const int items = NB * (DK / 2);
    const bool act = tid < items;
    const int I0 = tid / (DK / 2), j = 2 * (tid % (DK / 2));
    float2 ra[16], rk[16], rb[16], rq[16], P[16];
    if (act) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 16 * I0 + r;
        if (t < T) {
          const size_t off = seqK + (size_t)t * DK + j;
          ra[r] = In<Tin>::load2(alpha + off);
          rk[r] = In<Tin>::load2(k + off);
          rb[r] = In<Tin>::load2(bgate + off);
          rq[r] = In<Tin>::load2(q + off);
        } else {  // identity padding past the end of the sequence
          ra[r] = make_float2(1.f, 1.f);
          rk[r] = rb[r] = rq[r] = make_float2(0.f, 0.f);
        }
      }
      float2 p = make_float2(1.f, 1.f);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p.x *= ra[r].x;
        p.y *= ra[r].y;
        P[r] = p;
      }
      GS[I0 * DK + j] = p.x;
      GS[I0 * DK + j + 1] = p.y;
      if (!(p.x >= kGuardMin && p.y >= kGuardMin)) FLAGS[I0] = 1;
    }
    // v^ = w * v into VH[v][t] (fp32)
    {
      const int nvi = C * (VT / 8);
      for (int it = tid; it < nvi; it += 256) {
        const int t = it / (VT / 8), vv = (it % (VT / 8)) * 8;
        const int tg = t0 + t;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float2 vv2 = make_float2(0.f, 0.f), ww2 = make_float2(0.f, 0.f);
          if (tg < T) {
            const size_t off = seqV + (size_t)tg * DV + vt0 + vv + e;
            vv2 = In<Tin>::load2(v + off);
            ww2 = In<Tin>::load2(wgate + off);
          }
          VH[(vv + e) * L::LDF + t] = vv2.x * ww2.x;
          VH[(vv + e + 1) * L::LDF + t] = vv2.y * ww2.y;
        }
      }
    }
    __syncthreads();

    // ================= prep, pass 2: scaled operands
    if (act) {
      float2 Bst = make_float2(1.f, 1.f), E = make_float2(1.f, 1.f), pic = make_float2(1.f, 1.f);
      for (int J = 0; J < NB; ++J) {
        const float gx = GS[J * DK + j], gy = GS[J * DK + j + 1];
        if (J < I0) { Bst.x *= gx; Bst.y *= gy; }
        if (J > I0) { E.x *= gx; E.y *= gy; }
        pic.x *= gx; pic.y *= gy;
      }
      if (I0 == 0) { PIC[j] = pic.x; PIC[j + 1] = pic.y; }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tl = 16 * I0 + r;
        const float khx = rb[r].x * rk[r].x, khy = rb[r].y * rk[r].y;
        const float krx = khx * P[r].x, kry = khy * P[r].y;
        const float qrx = rq[r].x * P[r].x, qry = rq[r].y * P[r].y;
        const int off = tl * L::LDK + j;
        st2<SPLIT>(smem + L::KR, L::P_CK, off, krx, kry);
        st2<SPLIT>(smem + L::QR, L::P_CK, off, qrx, qry);
        st2<SPLIT>(smem + L::KHP, L::P_CK, off, -krx * Bst.x, -kry * Bst.y);
        st2<SPLIT>(smem + L::QHP, L::P_CK, off, qrx * Bst.x, qry * Bst.y);
      }
      float ktx[16], kty[16];
      float2 qs = make_float2(1.f, 1.f);
#pragma unroll
      for (int r = 15; r >= 0; --r) {
        const float kcx = rk[r].x * qs.x, kcy = rk[r].y * qs.y;
        st2<SPLIT>(smem + L::KC, L::P_CK, (16 * I0 + r) * L::LDK + j, kcx, kcy);
        ktx[r] = kcx * E.x;
        kty[r] = kcy * E.y;
        qs.x *= ra[r].x;
        qs.y *= ra[r].y;
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        st4<SPLIT>(smem + L::KTT, L::P_KC, j * L::LDC + 16 * I0 + 4 * r4,
                   f32x4{ktx[4 * r4], ktx[4 * r4 + 1], ktx[4 * r4 + 2], ktx[4 * r4 + 3]});
        st4<SPLIT>(smem + L::KTT, L::P_KC, (j + 1) * L::LDC + 16 * I0 + 4 * r4,
                   f32x4{kty[4 * r4], kty[4 * r4 + 1], kty[4 * r4 + 2], kty[4 * r4 + 3]});
      }
    }
    __syncthreads();

    // ================= Gram tiles, R = V^ - K^_pi S0, O^T = S0^T Q_pi^T
    f32x4 gL[MAXP], gM[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      gL[i] = f4zero();
      gM[i] = f4zero();
      const int p = wid + 4 * i;
      if (p < NP) {
        int I, J;
        pair_of(p, I, J);
        const bool scaled = (I == J) || (I > J + 1);
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          Frag<SPLIT> A = ldfrag<SPLIT>(smem + L::KC, L::P_CK, L::LDK, 16 * J, k0, DK, lane);
          const int kk = k0 + 8 * g;
          if (scaled && kk < DK) {
            float s[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (I == J) {
                s[e] = 1.f / GS[I * DK + kk + e];
              } else {
                float d = 1.f;
                for (int K = J + 1; K < I; ++K) d *= GS[K * DK + kk + e];
                s[e] = d;
              }
            }
            scale_frag<SPLIT>(A, s);
          }
          Frag<SPLIT> BL = ldfrag<SPLIT>(smem + L::KR, L::P_CK, L::LDK, 16 * I, k0, DK, lane);
          Frag<SPLIT> BM = ldfrag<SPLIT>(smem + L::QR, L::P_CK, L::LDK, 16 * I, k0, DK, lane);
          mma<SPLIT>(gL[i], A, BL);
          mma<SPLIT>(gM[i], A, BM);
        }
      }
    }
    f32x4 Racc[NVL];
    if (wid < NB) {
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl) {
        Racc[vl] = *(const f32x4*)(VH + (16 * vl + c16) * L::LDF + 16 * wid + 4 * g);
        Oacc[vl] = f4zero();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          Frag<SPLIT> Kp = ldfrag<SPLIT>(smem + L::KHP, L::P_CK, L::LDK, 16 * wid, k0, DK, lane);
          Frag<SPLIT> St = ldfrag<SPLIT>(smem + L::S0T, L::P_VK, L::LDK, 16 * vl, k0, DK, lane);
          Frag<SPLIT> Qp = ldfrag<SPLIT>(smem + L::QHP, L::P_CK, L::LDK, 16 * wid, k0, DK, lane);
          mma<SPLIT>(Racc[vl], Kp, St);
          mma<SPLIT>(Oacc[vl], St, Qp);
        }
      }
    }
    __syncthreads();

    // ================= write L (fp32 + hi/lo), M, R^T into the reused region
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int p = wid + 4 * i;
      if (p < NP) {
        int I, J;
        pair_of(p, I, J);
        const int t = 16 * I + c16, s0 = 16 * J + 4 * g;
        f32x4 lv = gL[i], mv = gM[i];
        if (I == J) {
          if (FLAGS[I]) exact_diag<Tin, DK>(k, bgate, q, alpha, seqK, t0, T, t, s0, lv, mv);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (s0 + e >= t) lv[e] = 0.f;
            if (s0 + e > t) mv[e] = 0.f;
          }
        }
        *(f32x4*)(LF + t * L::LDF + s0) = lv;
        st4<true>(smem + L::LB, L::P_CC, t * L::LDC + s0, lv);
        st4<SPLIT>(smem + L::MB, L::P_CC, t * L::LDC + s0, mv);
      }
    }
    if (wid < NB) {
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl)
        st4<SPLIT>(smem + L::RT, L::P_VC, (16 * vl + c16) * L::LDC + 16 * wid + 4 * g, Racc[vl]);
    }
    __syncthreads();

    // ================= T^{-1}: diagonal 16x16 blocks by forward substitution (fp32)
    if (wid == 0 && g < NB) {
      const int I = g, cc = c16;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* Lrow = LF + (16 * I + r) * L::LDF + 16 * I;
        float acc = (r == cc) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) acc -= Lrow[m] * x[m];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) st1<true>(smem + L::TN, L::P_CC, (16 * I + r) * L::LDC + 16 * I + cc, x[r]);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        st4<true>(smem + L::TT, L::P_CC, (16 * I + cc) * L::LDC + 16 * I + 4 * r4,
                  f32x4{x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]});
    }
    if (tid < 4) FLAGS[tid] = 0;  // last read above; set again in the next chunk's pass 1
    __syncthreads();

    // ================= T^{-1}: off-diagonal blocks, X_IJ = -D_I sum_{J<=K<I} L_IK X_KJ
    for (int d = 1; d < NB; ++d) {
      const int J = wid, I = J + d;
      const bool mact = I < NB;
      char* zt = smem + L::ZT + wid * 2 * L::P_Z;
      if (mact) {
        f32x4 z = f4zero();
        for (int k0 = 16 * J; k0 < 16 * I; k0 += 32) {
          Frag<true> A = ldfrag<true>(smem + L::LB, L::P_CC, L::LDC, 16 * I, k0, 16 * I, lane);
          Frag<true> B = ldfrag<true>(smem + L::TT, L::P_CC, L::LDC, 16 * J, k0, 16 * I, lane);
          mma<true>(z, A, B);
        }
        st4<true>(zt, L::P_Z, c16 * L::LDZ + 4 * g, z);
      }
      __syncthreads();
      if (mact) {
        f32x4 x = f4zero();
        Frag<true> A = ldfrag<true>(smem + L::TN, L::P_CC, L::LDC, 16 * I, 16 * I, 16 * I + 16, lane);
        Frag<true> B = ldfrag<true>(zt, L::P_Z, L::LDZ, 0, 0, 16, lane);
        mma<true>(x, A, B);
        x = -x;
        st4<true>(smem + L::TT, L::P_CC, (16 * J + c16) * L::LDC + 16 * I + 4 * g, x);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st1<true>(smem + L::TN, L::P_CC, (16 * I + 4 * g + e) * L::LDC + 16 * J + c16, x[e]);
      }
      __syncthreads();
    }

    // ================= V~ = T^{-1} R
    if (wid < NB) {
      const int I = wid, kend = 16 * (I + 1);
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl) {
        f32x4 acc = f4zero();
        for (int k0 = 0; k0 < kend; k0 += 32) {
          Frag<SPLIT> A = ldfrag<SPLIT>(smem + L::TN, L::P_CC, L::LDC, 16 * I, k0, kend, lane);
          Frag<SPLIT> B = ldfrag<SPLIT>(smem + L::RT, L::P_VC, L::LDC, 16 * vl, k0, kend, lane);
          mma<SPLIT>(acc, A, B);
        }
        st4<SPLIT>(smem + L::VTT, L::P_VC, (16 * vl + c16) * L::LDC + 16 * I + 4 * g, acc);
      }
    }
    __syncthreads();

    // ================= O^T += V~^T M^T, store O; S <- Diag(pi_C) S + K~^T V~
    if (wid < NB) {
      const int I = wid, kend = 16 * (I + 1);
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl) {
        for (int k0 = 0; k0 < kend; k0 += 32) {
          Frag<SPLIT> A = ldfrag<SPLIT>(smem + L::VTT, L::P_VC, L::LDC, 16 * vl, k0, kend, lane);
          Frag<SPLIT> B = ldfrag<SPLIT>(smem + L::MB, L::P_CC, L::LDC, 16 * I, k0, kend, lane);
          mma<SPLIT>(Oacc[vl], A, B);
        }
        const int t = t0 + 16 * I + c16;
        if (t < T) In<Tin>::store4(o + seqV + (size_t)t * DV + vt0 + 16 * vl + 4 * g, Oacc[vl]);
      }
    }
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + 4 * i;
      if (tile < NST) {
        const int jt = tile / NVL, vl = tile % NVL;
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[i][e] *= PIC[16 * jt + 4 * g + e];
        for (int k0 = 0; k0 < C; k0 += 32) {
          Frag<SPLIT> A = ldfrag<SPLIT>(smem + L::KTT, L::P_KC, L::LDC, 16 * jt, k0, C, lane);
          Frag<SPLIT> B = ldfrag<SPLIT>(smem + L::VTT, L::P_VC, L::LDC, 16 * vl, k0, C, lane);
          mma<SPLIT>(Sacc[i], A, B);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + 4 * i;
      if (tile < NST) {
        const int jt = tile / NVL, vl = tile % NVL;
        st4<SPLIT>(smem + L::S0T, L::P_VK, (16 * vl + c16) * L::LDK + 16 * jt + 4 * g, Sacc[i]);
      }
    }
  }

  if (S_out) {
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + 4 * i;
      if (tile < NST) {
        const int jt = tile / NVL, vl = tile % NVL;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S_out[stOff + (size_t)(16 * jt + 4 * g + e) * DV + vt0 + 16 * vl + c16] = Sacc[i][e];
      }
    }
  }
}

// ------------------------------------------------------------------ host launch
template <typename Tin, int DK, int VT, int CM>
static int launch_chunk(const ChunkArgs& a) {
  constexpr bool SPLIT = std::is_same<Tin, float>::value;
  using L = ChunkSmem<DK, VT, CM, SPLIT>;
  auto kern = gdn2_chunk_kernel<Tin, DK, VT, CM, SPLIT>;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL) !=
        hipSuccess)
      return GDR_ERR_LAUNCH;
    attr_set = true;
  }
  const int nblocks = a.B * a.H * (a.dv / VT);
  const Tin *q = (const Tin*)a.q, *k = (const Tin*)a.k, *v = (const Tin*)a.v;
  const Tin *al = (const Tin*)a.alpha, *bg = (const Tin*)a.b, *wg = (const Tin*)a.w;
  const float* S0 = a.S0;
  Tin* o = (Tin*)a.o;
  float* So = a.S_out;
  int T = a.T, DV = a.dv, C = a.chunk;
  void* args[] = {&q, &k, &v, &al, &bg, &wg, &S0, &o, &So, &T, &DV, &C};
  hipError_t e = hipLaunchKernel((const void*)kern, dim3(nblocks), dim3(256), args, L::TOTAL,
                                 (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

template <typename Tin, int CM_SPLIT128>
static int dispatch_dk(const ChunkArgs& a, int VT) {
  constexpr bool SPLIT = std::is_same<Tin, float>::value;
  if constexpr (SPLIT) {
    switch (a.dk) {
      case 16: return launch_chunk<Tin, 16, 16, 64>(a);
      case 32: return launch_chunk<Tin, 32, 16, 64>(a);
      case 64: return launch_chunk<Tin, 64, 16, 64>(a);
      case 128: return launch_chunk<Tin, 128, 16, CM_SPLIT128>(a);
    }
  } else {
    if (VT == 16) {
      switch (a.dk) {
        case 16: return launch_chunk<Tin, 16, 16, 64>(a);
        case 32: return launch_chunk<Tin, 32, 16, 64>(a);
        case 64: return launch_chunk<Tin, 64, 16, 64>(a);
        case 128: return launch_chunk<Tin, 128, 16, 64>(a);
      }
    } else {
      switch (a.dk) {
        case 16: return launch_chunk<Tin, 16, 32, 64>(a);
        case 32: return launch_chunk<Tin, 32, 32, 64>(a);
        case 64: return launch_chunk<Tin, 64, 32, 64>(a);
        case 128: return launch_chunk<Tin, 128, 32, 64>(a);
      }
    }
  }
  return GDR_ERR_UNSUPPORTED;
}

int chunk_fwd_launch(const ChunkArgs& a) {
  if (a.dtype == GDR_BF16) return dispatch_dk<__bf16, 32>(a, a.dv == 16 ? 16 : 32);
  return dispatch_dk<float, 32>(a, 16);
}

}  // namespace gdr
