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
// are pi_{C,s} * k_s. (§2.2 states T V~ = V^ - K^_pi S0; solving it on the VT
// value columns of this workgroup avoids the d_k-wide Y = T^{-1} K^_pi of the
// page's fused solve and never forms the off-diagonal blocks of T^{-1}.)
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
// Work split: one workgroup (512 threads, 8 waves) per (sequence b, head h,
// value tile of VT columns). Value columns of S evolve independently (eq.(1)
// acts on S from the left), so the tiles need no communication; each walks
// all chunks of its head, holding its S tile (d_k x VT, fp32) in registers.
//
// Phases per chunk (8 waves, 8 workgroup barriers):
//   prep 1  block totals G, v^ = w*v                          (all waves, VALU)
//   prep 2  Kr = k^*P, Qr = q*P, Kc = k*Qs, K~^T, per-pair scale vectors
//   Gram    L^T, M^T tiles = (Kc*D) [Kr; Qr]^T                (MFMA)
//   write   L as fp32 16x16 blocks, M
//   solve   wave 0: D_I = (I + L_II)^{-1} by forward substitution; waves 1-7
//           meanwhile: R = V^ - Kr (B_I * S0) and O^T = (B_I * S0)^T Qr^T;
//           then L'_IJ = D_I L_IJ (MFMA, one off-diagonal block per wave)
//   V~      block forward substitution, in place over R, one wave per value
//           tile: V~_I = D_I R_I - sum_{J<I} L'_IJ V~_J (T V~ = R, block rows)
//   end     O^T += V~^T M^T, store O; S <- Diag(pi_C) S + K~^T V~
// The next chunk's inputs are fetched into registers during the current chunk.
//
// Precision: bf16 inputs use bf16 operands with fp32 accumulation, except
// T^{-1}, which is built from hi/lo split operands (~16 bits). fp32 inputs use
// fp32 operands and fp32 MFMA (16x16x4) throughout.
#include "gdr_chunk_common.hpp"
#include "gdr_internal.h"
#include "gdr_host.hpp"

namespace gdr {

template <int DK, int VT, int CM, bool SPLIT>
struct ChunkSmem {
  static constexpr int NS = SPLIT ? 2 : 1;           // bf16 planes' worth of bytes per operand element
  static constexpr int NBM = CM / 16;
  static constexpr int NPM = NBM * (NBM + 1) / 2;    // lower-triangular 16x16 block pairs
  static constexpr int LDK = DK + 8;                 // pitch (elements), rows of length DK
  static constexpr int LDC = CM + 8;                 // pitch (elements), rows of length C
  static constexpr int LDF = CM + 4;                 // fp32 pitch of v^
  static constexpr int LDB = 20;                     // fp32 pitch of a 16x16 block
  static constexpr int P_CK = CM * LDK * 2;
  static constexpr int P_CC = CM * LDC * 2;
  static constexpr int P_KC = DK * LDC * 2;
  static constexpr int P_VC = VT * LDC * 2;
  static constexpr int P_VK = VT * LDK * 2;
  static constexpr int BLK = 16 * LDB * 4;
  static constexpr int KR = 0;                       // k^ * P   [C][DK]
  static constexpr int QR = KR + NS * P_CK;          // q * P    [C][DK]
  static constexpr int KC = QR + NS * P_CK;          // k * Qs   [C][DK]   (Gram only, then reused:)
  static constexpr int LBK = KC;                     //   L blocks, fp32 [pair][t][s]
  static constexpr int TBN = LBK + NPM * BLK;        //   D_I = (I + L_II)^-1, fp32 [I][t][s]
  static constexpr int X_END = imax(KC + NS * P_CK, TBN + NBM * BLK);
  static constexpr int VH = align16(X_END);          // v^ fp32   [VT][C]
  static constexpr int TL = VH + VT * LDF * 4;       // [.. -L'_IJ .. | D_I] rows, T mode, [t][s]
  static constexpr int VR = TL + 2 * P_CC;           // R, then V~ in place, T mode, [VT][C]
  static constexpr int MB = VR + 2 * P_VC;           // M         [t][s]
  static constexpr int KTT = MB + NS * P_CC;         // K~^T      [DK][C]
  static constexpr int VTT = KTT + NS * P_KC;        // V~^T      [VT][C]
  static constexpr int S0T = VTT + NS * P_VC;        // S0^T      [VT][DK]
  static constexpr int SCL = S0T + NS * P_VK;        // Gram scale vectors fp32 [pair][DK]
  static constexpr int GS = SCL + NPM * DK * 4;      // block totals G fp32 [NB][DK]
  static constexpr int BS = GS + NBM * DK * 4;       // decay to block start fp32 [NB][DK]
  static constexpr int PIC = BS + NBM * DK * 4;      // pi_C fp32 [DK]
  static constexpr int FLAG = PIC + DK * 4;          // guard flags [4]
  static constexpr int TOTAL = FLAG + 16;
  static_assert(TOTAL <= 160 * 1024, "chunk kernel LDS exceeds 160 KiB");
};

constexpr int kThreads = 512;  // 8 waves: two per SIMD

template <typename Tin, int DK, int VT, int CM, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void gdn2_chunk_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ alpha, const Tin* __restrict__ bgate, const Tin* __restrict__ wgate,
    const float* __restrict__ S0, Tin* __restrict__ o, float* S_out, int T, int DV, int C) {
  using L = ChunkSmem<DK, VT, CM, SPLIT>;
  constexpr int MM = SPLIT ? kF32 : kBF;   // main operands
  constexpr int MT = SPLIT ? kF32 : kSP;   // triangular solve
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NW = kThreads / 64;
  constexpr int NVL = VT / 16;                       // 16-col value tiles per workgroup
  constexpr int NST = (DK / 16) * NVL;               // S accumulator tiles
  constexpr int MAXS = (NST + NW - 1) / NW;
  constexpr int NBM = CM / 16;
  constexpr int MAXP = (L::NPM + NW - 1) / NW;       // Gram pairs per wave
  constexpr int MAXQ = (L::NPM - NBM + NW - 1) / NW; // off-diagonal pairs per wave
  constexpr int MAXJ = (NBM * NVL + NW - 2) / (NW - 1);  // R/O jobs per wave (waves 1..)

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nvt = DV / VT;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int bh = lin / nvt, vt0 = (lin % nvt) * VT;
  const int NB = C / 16, NP = NB * (NB + 1) / 2, NQ = NB * (NB - 1) / 2, NJ = NB * NVL;
  const int nchunks = (T + C - 1) / C;
  const size_t seqK = (size_t)bh * T * DK;
  const size_t seqV = (size_t)bh * T * DV;
  const size_t stOff = (size_t)bh * DK * DV;

  float* GS = (float*)(smem + L::GS);
  float* BS = (float*)(smem + L::BS);
  float* SCL = (float*)(smem + L::SCL);
  float* PIC = (float*)(smem + L::PIC);
  int* FLAGS = (int*)(smem + L::FLAG);
  float* VH = (float*)(smem + L::VH);
  float* LBK = (float*)(smem + L::LBK);
  float* TBN = (float*)(smem + L::TBN);
  constexpr int BLKF = 16 * L::LDB;                  // floats per block

  // ---- state tile -> registers and S0^T in LDS
  f32x4 Sacc[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    Sacc[i] = f4zero();
    const int tile = wid + NW * i;
    if (tile < NST) {
      const int jt = tile / NVL, vl = tile % NVL;
      if (S0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Sacc[i][e] = S0[stOff + (size_t)(16 * jt + 4 * g + e) * DV + vt0 + 16 * vl + c16];
      }
      st4<MM>(smem + L::S0T, L::P_VK, (16 * vl + c16) * L::LDK + 16 * jt + 4 * g, Sacc[i]);
    }
  }
  if (tid < 4) FLAGS[tid] = 0;
  __syncthreads();

  f32x4 Oacc[MAXJ];

  // ---- input staging. Lanes l and l^32 of a wave share channels (j, j+1) of
  // one 16-row block I0 and take its rows 0-7 (h = 0) and 8-15 (h = 1); the
  // half-block products are exchanged across the pair. A v^ item is 8
  // consecutive value columns of one row. Loads are branch-free (rows clamped,
  // padding selected afterwards) and the next chunk's are issued while this
  // chunk's Gram products run.
  using RW = Raw<Tin>;
  const int h = lane >> 5;
  const int fp = wid * 32 + (lane & 31);
  const bool act = fp < NB * (DK / 2);
  const int I0 = act ? fp / (DK / 2) : 0, j = act ? 2 * (fp % (DK / 2)) : 0;
  const int r0 = 16 * I0 + 8 * h;                    // first chunk row of this thread
  const int nvi = C * (VT / 8);
  const bool vact = tid < nvi;
  const int vrow = vact ? tid / (VT / 8) : 0, vcol = vact ? (tid % (VT / 8)) * 8 : 0;
  typename RW::R2 xa[8], xk[8], xb[8], xq[8];
  typename RW::R8 xv, xw;
  // per-head base pointers; offsets within a head are 32-bit (T * d < 2^31)
  const Tin* __restrict__ qh = q + seqK + j;
  const Tin* __restrict__ kh = k + seqK + j;
  const Tin* __restrict__ ah = alpha + seqK + j;
  const Tin* __restrict__ bh_ = bgate + seqK + j;
  const Tin* __restrict__ vh_ = v + seqV + vt0 + vcol;
  const Tin* __restrict__ wh_ = wgate + seqV + vt0 + vcol;
  auto issue = [&](int chk) {
    const int tb = chk * C;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int t = tb + r0 + r;
      const int off = (t < T ? t : T - 1) * DK;
      xa[r] = RW::ld2(ah + off);
      xk[r] = RW::ld2(kh + off);
      xb[r] = RW::ld2(bh_ + off);
      xq[r] = RW::ld2(qh + off);
    }
    const int tv = tb + vrow;
    const int offv = (tv < T ? tv : T - 1) * DV;
    xv = RW::ld8(vh_ + offv);
    xw = RW::ld8(wh_ + offv);
  };
  issue(0);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * C;
    // identity padding past the end of the sequence: alpha = 1, k = b = q = 0, v = w = 0
    {
      const typename RW::R2 one = RW::pad2(1.f), zero = RW::pad2(0.f);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool ok = t0 + r0 + r < T;
        xa[r] = RW::sel(ok, xa[r], one);
        xk[r] = RW::sel(ok, xk[r], zero);
        xb[r] = RW::sel(ok, xb[r], zero);
        xq[r] = RW::sel(ok, xq[r], zero);
      }
      const bool okv = t0 + vrow < T;
      xv = RW::sel(okv, xv, RW::zero8());
      xw = RW::sel(okv, xw, RW::zero8());
    }

    // ================= prep 1: half-block products -> block totals G; v^
    float2 ph = make_float2(1.f, 1.f);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float2 a = RW::un2(xa[r]);
      ph.x *= a.x;
      ph.y *= a.y;
    }
    const float2 po = make_float2(__shfl_xor(ph.x, 32, 64), __shfl_xor(ph.y, 32, 64));
    const float2 p0 = h ? po : ph, p1 = h ? ph : po;   // products of rows 0-7 and 8-15
    if (act && h == 0) {
      const float gx = p0.x * p1.x, gy = p0.y * p1.y;
      GS[I0 * DK + j] = gx;
      GS[I0 * DK + j + 1] = gy;
      if (!(gx >= kGuardMin && gy >= kGuardMin)) FLAGS[I0] = 1;
    }
    if (vact) {
      float fv[8], fw[8];
      RW::un8(xv, fv);
      RW::un8(xw, fw);
#pragma unroll
      for (int e = 0; e < 8; ++e) VH[(vcol + e) * L::LDF + vrow] = fv[e] * fw[e];
    }
    __syncthreads();

    // ================= prep 2: scaled operands and per-pair scale vectors
    if (act) {
      float2 Bst = make_float2(1.f, 1.f), E = make_float2(1.f, 1.f), pic = make_float2(1.f, 1.f);
      for (int J = 0; J < NB; ++J) {
        const float gx = GS[J * DK + j], gy = GS[J * DK + j + 1];
        if (J < I0) { Bst.x *= gx; Bst.y *= gy; }
        if (J > I0) { E.x *= gx; E.y *= gy; }
        pic.x *= gx; pic.y *= gy;
      }
      if (h == 0) {
        if (I0 == 0) { PIC[j] = pic.x; PIC[j + 1] = pic.y; }
        BS[I0 * DK + j] = Bst.x;
        BS[I0 * DK + j + 1] = Bst.y;
        // scale of pair (I0, J): 1/G_I0 on the diagonal (in-block ratio), the
        // product of the block totals strictly between J and I0 below it
        const float gx = GS[I0 * DK + j], gy = GS[I0 * DK + j + 1];
        SCL[pidx(I0, I0) * DK + j] = __builtin_amdgcn_rcpf(gx);
        SCL[pidx(I0, I0) * DK + j + 1] = __builtin_amdgcn_rcpf(gy);
        float2 d = make_float2(1.f, 1.f);
        for (int J = I0 - 1; J >= 0; --J) {
          SCL[pidx(I0, J) * DK + j] = d.x;
          SCL[pidx(I0, J) * DK + j + 1] = d.y;
          d.x *= GS[J * DK + j];
          d.y *= GS[J * DK + j + 1];
        }
      }
      float2 P = h ? p0 : make_float2(1.f, 1.f);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float2 a = RW::un2(xa[r]), kk = RW::un2(xk[r]), bb = RW::un2(xb[r]), qq = RW::un2(xq[r]);
        P.x *= a.x;
        P.y *= a.y;
        const int off = (r0 + r) * L::LDK + j;
        st2<MM>(smem + L::KR, L::P_CK, off, bb.x * kk.x * P.x, bb.y * kk.y * P.y);
        st2<MM>(smem + L::QR, L::P_CK, off, qq.x * P.x, qq.y * P.y);
      }
      float ktx[8], kty[8];
      float2 qs = h ? make_float2(1.f, 1.f) : p1;
#pragma unroll
      for (int r = 7; r >= 0; --r) {
        const float2 kk = RW::un2(xk[r]), a = RW::un2(xa[r]);
        const float kcx = kk.x * qs.x, kcy = kk.y * qs.y;
        st2<MM>(smem + L::KC, L::P_CK, (r0 + r) * L::LDK + j, kcx, kcy);
        ktx[r] = kcx * E.x;
        kty[r] = kcy * E.y;
        qs.x *= a.x;
        qs.y *= a.y;
      }
#pragma unroll
      for (int r4 = 0; r4 < 2; ++r4) {
        st4<MM>(smem + L::KTT, L::P_KC, j * L::LDC + r0 + 4 * r4,
                f32x4{ktx[4 * r4], ktx[4 * r4 + 1], ktx[4 * r4 + 2], ktx[4 * r4 + 3]});
        st4<MM>(smem + L::KTT, L::P_KC, (j + 1) * L::LDC + r0 + 4 * r4,
                f32x4{kty[4 * r4], kty[4 * r4 + 1], kty[4 * r4 + 2], kty[4 * r4 + 3]});
      }
    }
    __syncthreads();
    // the next chunk's loads overlap the Gram MFMAs and stay in flight through the chunk
    if (ch + 1 < nchunks) issue(ch + 1);

    // ================= Gram tiles: L^T, M^T of pair (I, J) = (Kc_J * scale) [Kr_I; Qr_I]^T
    f32x4 gL[MAXP], gM[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      gL[i] = f4zero();
      gM[i] = f4zero();
      const int p = wid + NW * i;
      if (p < NP) {
        int I, J;
        pair_of(p, I, J);
        const bool scaled = (I == J) || (I > J + 1);
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          Frag<MM> A = ldfrag<MM>(smem + L::KC, L::P_CK, L::LDK, 16 * J, k0, DK, lane);
          const int kk = k0 + 8 * g;
          if (scaled && kk < DK) {
            const float* sp = SCL + p * DK + kk;
            const f32x4 s0 = *(const f32x4*)sp, s1 = *(const f32x4*)(sp + 4);
            const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
            scale_frag<MM>(A, sv);
          }
          Frag<MM> BL = ldfrag<MM>(smem + L::KR, L::P_CK, L::LDK, 16 * I, k0, DK, lane);
          Frag<MM> BM = ldfrag<MM>(smem + L::QR, L::P_CK, L::LDK, 16 * I, k0, DK, lane);
          mma<MM>(gL[i], A, BL);
          mma<MM>(gM[i], A, BM);
        }
      }
    }
    __syncthreads();

    // ================= write L (fp32 blocks) and M
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int p = wid + NW * i;
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
        *(f32x4*)(LBK + p * BLKF + c16 * L::LDB + 4 * g) = lv;
        st4<MM>(smem + L::MB, L::P_CC, t * L::LDC + s0, mv);
      }
    }
    __syncthreads();

    if (wid == 0) {
      // ============= D_I = (I + L_II)^{-1}: forward substitution, lane = (block g, column c16)
      if (tid < 4) FLAGS[tid] = 0;  // last read above; set again by the next chunk's prep 1
      const int I = g, cc = c16;
      const bool live = I < NB;
      const float* Lb = LBK + (live ? pidx(I, I) : 0) * BLKF;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc0 = (r == cc) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
        for (int m4 = 0; 4 * m4 < r; ++m4) {
          const f32x4 lv = *(const f32x4*)(Lb + r * L::LDB + 4 * m4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * m4 + e;
            if (m < r) {
              if (m & 1) acc1 -= lv[e] * x[m];
              else acc0 -= lv[e] * x[m];
            }
          }
        }
        x[r] = acc0 + acc1;
      }
      if (live) {
        float* Tn = TBN + I * BLKF;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Tn[r * L::LDB + cc] = x[r];
          st1<MT>(smem + L::TL, L::P_CC, (16 * I + r) * L::LDC + 16 * I + cc, x[r]);
        }
      }
    } else {
      // ============= waves 1..: R = V^ - Kr (B_I * S0) and O^T = (B_I * S0)^T Qr^T
#pragma unroll
      for (int i = 0; i < MAXJ; ++i) {
        const int job = (wid - 1) + (NW - 1) * i;
        if (job < NJ) {
          const int I = job / NVL, vl = job % NVL;
          f32x4 r = f4zero();
          Oacc[i] = f4zero();
#pragma unroll
          for (int k0 = 0; k0 < DK; k0 += 32) {
            Frag<MM> Sf = ldfrag<MM>(smem + L::S0T, L::P_VK, L::LDK, 16 * vl, k0, DK, lane);
            const int kk = k0 + 8 * g;
            if (I > 0 && kk < DK) {
              const float* bp = BS + I * DK + kk;
              const f32x4 b0 = *(const f32x4*)bp, b1 = *(const f32x4*)(bp + 4);
              const float sv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
              scale_frag<MM>(Sf, sv);
            }
            Frag<MM> Kf = ldfrag<MM>(smem + L::KR, L::P_CK, L::LDK, 16 * I, k0, DK, lane);
            Frag<MM> Qf = ldfrag<MM>(smem + L::QR, L::P_CK, L::LDK, 16 * I, k0, DK, lane);
            mma<MM>(r, Kf, Sf);
            mma<MM>(Oacc[i], Sf, Qf);
          }
          const f32x4 vh = *(const f32x4*)(VH + (16 * vl + c16) * L::LDF + 16 * I + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = vh[e] - r[e];
          st4<MT>(smem + L::VR, L::P_VC, (16 * vl + c16) * L::LDC + 16 * I + 4 * g, r);
        }
      }
    }
    __syncthreads();

    // ================= L'_IJ = D_I L_IJ (I > J), stored negated in the rows of TL
#pragma unroll
    for (int i = 0; i < MAXQ; ++i) {
      const int qq = wid + NW * i;
      if (qq < NQ) {
        int I, J;
        offpair_of(qq, I, J);
        const int p = pidx(I, J);
        const bool ok = g < 2;  // k = m spans one 16-row block
        Frag<MT> A = frag_f32<MT>(TBN + I * BLKF + c16 * L::LDB + 8 * (g & 1), ok);
        // B[k = m][n = s] = L_IJ[m][s]: gather column s of the fp32 block
        float lc[8];
        const float* lb = LBK + p * BLKF + c16;
#pragma unroll
        for (int e = 0; e < 8; ++e) lc[e] = ok ? lb[(8 * (g & 1) + e) * L::LDB] : 0.f;
        Frag<MT> B = frag_f32<MT>(lc, true);
        f32x4 acc = f4zero();
        mma<MT>(acc, A, B);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st1<MT>(smem + L::TL, L::P_CC, (16 * I + 4 * g + e) * L::LDC + 16 * J + c16, -acc[e]);
      }
    }
    __syncthreads();

    // ================= V~: block forward substitution in place over R (one wave per value tile)
    if (wid < NVL) {
      const int vl = wid;
      for (int I = 0; I < NB; ++I) {
        const int kend = 16 * (I + 1);
        f32x4 acc = f4zero();
        for (int k0 = 0; k0 < kend; k0 += 32) {
          Frag<MT> A = ldfrag<MT>(smem + L::TL, L::P_CC, L::LDC, 16 * I, k0, kend, lane);
          Frag<MT> B = ldfrag<MT>(smem + L::VR, L::P_VC, L::LDC, 16 * vl, k0, kend, lane);
          mma<MT>(acc, A, B);
        }
        const int off = (16 * vl + c16) * L::LDC + 16 * I + 4 * g;
        st4<MT>(smem + L::VR, L::P_VC, off, acc);
        st4<MM>(smem + L::VTT, L::P_VC, off, acc);
        wave_lds_sync();
      }
    }
    __syncthreads();

    // ================= O^T += V~^T M^T and store O; S <- Diag(pi_C) S + K~^T V~
    if (wid > 0) {
#pragma unroll
      for (int i = 0; i < MAXJ; ++i) {
        const int job = (wid - 1) + (NW - 1) * i;
        if (job < NJ) {
          const int I = job / NVL, vl = job % NVL, kend = 16 * (I + 1);
          for (int k0 = 0; k0 < kend; k0 += 32) {
            Frag<MM> A = ldfrag<MM>(smem + L::VTT, L::P_VC, L::LDC, 16 * vl, k0, kend, lane);
            Frag<MM> B = ldfrag<MM>(smem + L::MB, L::P_CC, L::LDC, 16 * I, k0, kend, lane);
            mma<MM>(Oacc[i], A, B);
          }
          const int t = t0 + 16 * I + c16;
          if (t < T) In<Tin>::store4(o + seqV + (size_t)t * DV + vt0 + 16 * vl + 4 * g, Oacc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + NW * i;
      if (tile < NST) {
        const int jt = tile / NVL, vl = tile % NVL;
        const f32x4 pc = *(const f32x4*)(PIC + 16 * jt + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[i][e] *= pc[e];
        for (int k0 = 0; k0 < C; k0 += 32) {
          Frag<MM> A = ldfrag<MM>(smem + L::KTT, L::P_KC, L::LDC, 16 * jt, k0, C, lane);
          Frag<MM> B = ldfrag<MM>(smem + L::VTT, L::P_VC, L::LDC, 16 * vl, k0, C, lane);
          mma<MM>(Sacc[i], A, B);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + NW * i;
      if (tile < NST) {
        const int jt = tile / NVL, vl = tile % NVL;
        st4<MM>(smem + L::S0T, L::P_VK, (16 * vl + c16) * L::LDK + 16 * jt + 4 * g, Sacc[i]);
      }
    }
  }

  if (S_out) {
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + NW * i;
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
  if (!allow_lds((const void*)kern, L::TOTAL)) return GDR_ERR_LAUNCH;
  const int nblocks = a.B * a.H * (a.dv / VT);
  const Tin *q = (const Tin*)a.q, *k = (const Tin*)a.k, *v = (const Tin*)a.v;
  const Tin *al = (const Tin*)a.alpha, *bg = (const Tin*)a.b, *wg = (const Tin*)a.w;
  const float* S0 = a.S0;
  Tin* o = (Tin*)a.o;
  float* So = a.S_out;
  int T = a.T, DV = a.dv, C = a.chunk;
  void* args[] = {&q, &k, &v, &al, &bg, &wg, &S0, &o, &So, &T, &DV, &C};
  hipError_t e = hipLaunchKernel((const void*)kern, dim3(nblocks), dim3(kThreads), args, L::TOTAL,
                                 (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

int chunk_fwd_launch(const ChunkArgs& a) {
  if (a.dtype == GDR_BF16) {
    if (a.dv == 16) {
      switch (a.dk) {
        case 16: return launch_chunk<__bf16, 16, 16, 64>(a);
        case 32: return launch_chunk<__bf16, 32, 16, 64>(a);
        case 64: return launch_chunk<__bf16, 64, 16, 64>(a);
        case 128: return launch_chunk<__bf16, 128, 16, 64>(a);
      }
    } else {
      switch (a.dk) {
        case 16: return launch_chunk<__bf16, 16, 32, 64>(a);
        case 32: return launch_chunk<__bf16, 32, 32, 64>(a);
        case 64: return launch_chunk<__bf16, 64, 32, 64>(a);
        case 128: return launch_chunk<__bf16, 128, 32, 64>(a);
      }
    }
  } else {
    // fp32 operands take twice the LDS: chunks of at most 32 rows for d_k >= 64
    switch (a.dk) {
      case 16: return launch_chunk<float, 16, 16, 64>(a);
      case 32: return launch_chunk<float, 32, 16, 64>(a);
      case 64: return launch_chunk<float, 64, 16, 32>(a);
      case 128: return launch_chunk<float, 128, 16, 32>(a);
    }
  }
  return GDR_ERR_UNSUPPORTED;
}

}  // namespace gdr
