// RWKV-7's generalized delta rule on gfx950: chunkwise forward (two kernels
// through a workspace) and the one-token decode step.
//
// "Exponential gates and matrix memory: xLSTM and RWKV-7", §13.3 and the
// solution to Exercise 13.5, in this library's orientation (state
// S[d_k, d_v], row vectors, o = q S):
//     S_t = (Diag(w_t) - c_t a_t^T a_t) S_{t-1} + kw_t^T u_t,   o_t = q_t S_t.
// The removal reads the previous, undecayed state: e_t = c_t a_t S_{t-1}.
//
// Chunkwise form (chunk of C tokens from S0; Lambda_t = sum_{r<=t} log w_r,
// pi_t = e^{Lambda_t}, every decay below a product of w over an interval,
// evaluated as exp of a non-positive difference of Lambda):
//   y_t = c_t a_t
//   L_a[t,s] = <y_t, e^{Lambda_{t-1} - Lambda_s} a_s>,  L_z likewise with kw_s (s < t)
//   M_a[t,s] = <q_t, e^{Lambda_t - Lambda_s} a_s>,      M_z likewise with kw_s (s <= t)
//   (I + L_a) [E0 | G] = [L_z U | Y_pi'],  (Y_pi')_t = y_t e^{Lambda_{t-1}}
//   the removal amounts E = E0 + G S0, and
//   O   = Q_pi S0 - M_a E + M_z U,
//   S_C = Diag(pi_C) S0 - A~^T E + Z~^T U   (A~_s, Z~_s = e^{Lambda_C - Lambda_s} a_s, kw_s).
// The intra kernel does every chunk independently and writes G, E0, M_a,
// Q_pi, A~^T, pi_C, O_z = M_z U and Z~^T (fp32); the scan walks the chunks of
// each head: E = E0 + G S0, O = Q_pi S0 - M_a E + O_z,
// S = Diag(pi_C) S0 - A~^T E + Z~^T U (U read from the input), on the fp32
// matrix cores. Keeping Z~^T (d_k x C) in the record instead of the product
// Z~^T U (d_k x d_v) makes the record a third smaller and moves that product
// from the intra kernel to the scan, where it costs no extra load time.
#include "gdr_device.hpp"
#include "gdr_internal.h"
#include "gdr_host.hpp"

namespace gdr {

namespace {

constexpr int kR7ScanThreads = 512;    // scan: eight waves, two per SIMD
constexpr int kR7ScanWaves = kR7ScanThreads / 64;
constexpr int kR7IntraThreads = 512;   // intra: eight waves, two per SIMD
constexpr int kR7IntraWaves = kR7IntraThreads / 64;

// Record of one (b, h, chunk), fp32 element offsets.
struct R7Layout {
  int g, e0, ma, qp, at, pic, oz, zt, floats;
};
__host__ __device__ inline R7Layout r7_layout(int dk, int dv, int C) {
  R7Layout r;
  r.g = 0;                    // G     [t][j]  C x dk
  r.e0 = r.g + C * dk;        // E0    [t][v]  C x dv
  r.ma = r.e0 + C * dv;       // M_a   [t][s]  C x C (lower, diagonal included)
  r.qp = r.ma + C * C;        // Q_pi  [t][j]  C x dk
  r.at = r.qp + C * dk;       // A~^T  [j][s]  dk x C
  r.pic = r.at + dk * C;      // pi_C  [j]     dk
  r.oz = r.pic + dk;          // O_z   [t][v]  C x dv
  r.zt = r.oz + C * dv;       // Z~^T  [j][s]  dk x C
  r.floats = (r.zt + dk * C + 3) / 4 * 4;
  return r;
}

}  // namespace

size_t rwkv7_ws_bytes(int B, int H, int T, int dk, int dv, int chunk) {
  const size_t nch = ((size_t)T + chunk - 1) / chunk;
  return (size_t)B * H * nch * r7_layout(dk, dv, chunk).floats * 4;
}

// ------------------------------------------------------------------ intra-chunk kernel
// One workgroup (four waves) per (b, h, chunk), fp32 throughout. The four
// decay-scaled Gram matrices are fp32 MFMA products over the key channels,
// split at the 16-row blocks of the chunk as the GDN-2 forward splits its
// Gram: for row block I with pivot p = 16 I - 1 (Lambda_{-1} = 0),
//   M[t][s] = sum_j (q_t e^{Lambda_t - Lambda_p})_j (a_s e^{Lambda_p - Lambda_s})_j,
//   L[t][s] = sum_j (c_t a_t e^{Lambda_{t-1} - Lambda_p})_j (a_s e^{Lambda_p - Lambda_s})_j,
// and likewise with kw_s. The left factors are <= 1; the right ones are <= 1
// for s <= p and at most 1 / (the block's decay) inside the block, so a block
// in which some channel decays below 2^-60 takes exact pairwise factors for
// its diagonal tile instead. The products with U (L_z U, M_z U) are MFMA
// tiles too; the unit lower-triangular solve runs one column per thread.
template <typename E, int DK, int CM>
__global__ __launch_bounds__(kR7IntraThreads) void rwkv7_intra_kernel(
    const E* __restrict__ q, const E* __restrict__ w, const E* __restrict__ a, const float* __restrict__ c,
    const E* __restrict__ kw, const E* __restrict__ u, float* __restrict__ ws, int T, int DV) {
  constexpr int P = DK + 4, PC = CM + 4, NB = CM / 16;
  extern __shared__ __attribute__((aligned(16))) float r7s[];
  float* Lam = r7s;                     // Lambda [t][j]
  float* Al = Lam + CM * P;             // a      [t][j]
  float* Zl = Al + CM * P;              // kw     [t][j]
  float* Ql = Zl + CM * P;              // q      [t][j]
  float* cv = Ql + CM * P;              // c      [t]
  float* La = cv + CM;                  // L_a    [t][s]
  float* Lz = La + CM * PC;             // L_z
  float* Ma = Lz + CM * PC;             // M_a
  float* Mz = Ma + CM * PC;             // M_z
  float* TMP = Mz + CM * PC;
  // phase G
  float* Aq = TMP;                      // q_t e^{Lambda_t - Lambda_p}         [16][j]
  float* Ay = Aq + 16 * P;              // c_t a_t e^{Lambda_{t-1} - Lambda_p} [16][j]
  float* Ba = Ay + 16 * P;              // a_s e^{Lambda_p - Lambda_s}          [s][j]
  float* Bz = Ba + CM * P;              // kw_s e^{Lambda_p - Lambda_s}         [s][j]
  // phase R
  const int NX = DV + DK + 4;
  float* UT = TMP;                      // u^T  [v][s]
  float* Xl = UT + DV * PC;             // [L_z U | Y_pi'] -> [E0 | G]  [t][col]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nch = (T + CM - 1) / CM;
  const int bh = blockIdx.x / nch, ch = blockIdx.x % nch, t0 = ch * CM;
  const size_t sK = (size_t)bh * T * DK, sV = (size_t)bh * T * DV;
  const R7Layout RL = r7_layout(DK, DV, CM);
  // record stores carry the non-temporal cache policy (4K shape: 1.058 ->
  // 1.041 ms for the forward, as for the GDN-2 record's small stores)
  float* rec = ws + ((size_t)bh * nch + ch) * RL.floats;
  __shared__ int gflag[4];
  static_assert(CM * DK / 8 <= kR7IntraThreads && CM * 128 / 8 <= kR7IntraThreads,
                "one 8-element piece of each input per thread (d_v <= 128)");
  // Every input of the chunk is loaded up front, 16 bytes per lane and at
  // most one piece per thread and input (u too, though it is staged only
  // after the Gram phase), so all their latencies overlap. The loads are
  // unconditional (rows clamped into the sequence); rows past T become
  // identity steps below: w = 1, a = kw = q = 0, c = 0, u = 0.
  using RW = Raw<E>;
  const int kt = tid / (DK / 8), kj = 8 * (tid % (DK / 8));          // [t][j] piece of this thread
  const size_t koff = sK + (size_t)row_in(t0 + (kt < CM ? kt : 0), T) * DK + kj;
  const typename RW::R8 rq = RW::ld8(q + koff), rw = RW::ld8(w + koff), ra = RW::ld8(a + koff),
                        rz = RW::ld8(kw + koff);
  // u pieces: consecutive threads take consecutive rows t (so the transposed
  // LDS writes below hit distinct banks), then the next 8 value columns
  const int ut = tid % CM, uv = 8 * (tid / CM);
  const bool u_on = uv < DV;
  const typename RW::R8 ru = RW::ld8(u + sV + (size_t)row_in(t0 + ut, T) * DV + (u_on ? uv : 0));
  const float c0 = c[(size_t)bh * T + row_in(t0 + (tid < CM ? tid : 0), T)];
  if (kt < CM) {
    const bool ok = t0 + kt < T;
    float fq[8], fw[8], fa[8], fz[8];
    RW::un8(rq, fq);
    RW::un8(rw, fw);
    RW::un8(ra, fa);
    RW::un8(rz, fz);
#pragma unroll
    for (int h4 = 0; h4 < 2; ++h4) {
      f32x4 vl, va, vz, vq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vl[e] = ok ? logf(fw[4 * h4 + e]) : 0.f;
        va[e] = ok ? fa[4 * h4 + e] : 0.f;
        vz[e] = ok ? fz[4 * h4 + e] : 0.f;
        vq[e] = ok ? fq[4 * h4 + e] : 0.f;
      }
      const int o4 = kt * P + kj + 4 * h4;
      *(f32x4*)&Lam[o4] = vl;
      *(f32x4*)&Al[o4] = va;
      *(f32x4*)&Zl[o4] = vz;
      *(f32x4*)&Ql[o4] = vq;
    }
  }
  if (tid < CM) cv[tid] = t0 + tid < T ? c0 : 0.f;
  if (tid < 4) gflag[tid] = 0;
  // the Gram tiles above the diagonal blocks are never formed: zero
  GDR_STAGE_FOR(x, 4 * CM * PC, kR7IntraThreads) La[x] = 0.f;
  __syncthreads();
  GDR_STAGE_FOR(j, DK, kR7IntraThreads) {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < CM; ++t) {
      acc += Lam[t * P + j];
      Lam[t * P + j] = acc;
    }
    // blocks in which channel j decays below 2^-60 (log 2^-60 = -41.59)
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      const float lp = I > 0 ? Lam[(16 * I - 1) * P + j] : 0.f;
      if (Lam[(16 * I + 15) * P + j] - lp < -41.5f) gflag[I] = 1;
    }
  }
  __syncthreads();
  // ---- phase G: the Gram matrices, one row block at a time
  for (int I = 0; I < NB; ++I) {
    const int p = 16 * I - 1, ns = 16 * (I + 1);
    GDR_STAGE_FOR(x, 16 * DK, kR7IntraThreads) {
      const int tl = x / DK, j = x % DK, t = 16 * I + tl;
      const float lp = I > 0 ? Lam[p * P + j] : 0.f;
      const float lt1 = t > 0 ? Lam[(t - 1) * P + j] : 0.f;
      Aq[tl * P + j] = Ql[t * P + j] * __expf(Lam[t * P + j] - lp);
      Ay[tl * P + j] = cv[t] * Al[t * P + j] * __expf(lt1 - lp);
    }
    GDR_STAGE_FOR(x, CM * DK, kR7IntraThreads) {
      const int s2 = x / DK, j = x % DK;
      if (s2 < ns) {
        const float lp = I > 0 ? Lam[p * P + j] : 0.f;
        const float e = __expf(lp - Lam[s2 * P + j]);
        Ba[s2 * P + j] = Al[s2 * P + j] * e;
        Bz[s2 * P + j] = Zl[s2 * P + j] * e;
      }
    }
    __syncthreads();
    const bool exact = gflag[I] != 0;
    // tiles (which, J): which = 0 M_a, 1 M_z, 2 L_a, 3 L_z; J = 0 .. I
    for (int tile = wid; tile < 4 * (I + 1); tile += kR7IntraWaves) {
      const int which = tile % 4, J = tile / 4;
      const float* A = which < 2 ? Aq : Ay;
      const float* Bm = (which & 1) ? Bz : Ba;
      f32x4 acc = f4zero();
      tile_nt(acc, A, P, 0, Bm, P, 16 * J, DK, lane);
      float* G = which == 0 ? Ma : which == 1 ? Mz : which == 2 ? La : Lz;
      const bool strict = which >= 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * (lane >> 4) + e, s2 = 16 * J + (lane & 15);
        float val = acc[e];
        if (exact && J == I) {
          // the pairwise decays of the diagonal tile, exact
          val = 0.f;
          if (strict ? s2 < t : s2 <= t) {
            const float* Xs = (which & 1) ? Zl : Al;
            for (int j = 0; j < DK; ++j) {
              const float ls = Lam[s2 * P + j];
              const float lt = strict ? (t > 0 ? Lam[(t - 1) * P + j] : 0.f) : Lam[t * P + j];
              const float lhs = strict ? cv[t] * Al[t * P + j] : Ql[t * P + j];
              val += lhs * __expf(lt - ls) * Xs[s2 * P + j];
            }
          }
        }
        G[t * PC + s2] = (strict ? s2 < t : s2 <= t) ? val : 0.f;
      }
    }
    __syncthreads();
  }
  // ---- phase R
  if (u_on) {
    float fu[8];
    RW::un8(ru, fu);
    const bool ok = t0 + ut < T;
#pragma unroll
    for (int e = 0; e < 8; ++e) UT[(uv + e) * PC + ut] = ok ? fu[e] : 0.f;
  }
  GDR_STAGE_FOR(x, CM * DK, kR7IntraThreads) {
    const int t = x / DK, j = x % DK;
    const float lt1 = t > 0 ? Lam[(t - 1) * P + j] : 0.f;
    Xl[t * NX + DV + j] = cv[t] * Al[t * P + j] * __expf(lt1);                 // Y_pi'
    __builtin_nontemporal_store(__expf(Lam[t * P + j]) * Ql[t * P + j], &rec[RL.qp + t * DK + j]);
  }
  GDR_STAGE_FOR(x, DK * CM, kR7IntraThreads) {   // A~^T, Z~^T, rows j: consecutive threads store consecutive s
    const int j = x / CM, s2 = x % CM;
    const float e = __expf(Lam[(CM - 1) * P + j] - Lam[s2 * P + j]);
    __builtin_nontemporal_store(e * Al[s2 * P + j], &rec[RL.at + j * CM + s2]);
    __builtin_nontemporal_store(e * Zl[s2 * P + j], &rec[RL.zt + j * CM + s2]);
  }
  GDR_STAGE_FOR(j, DK, kR7IntraThreads) __builtin_nontemporal_store(__expf(Lam[(CM - 1) * P + j]), &rec[RL.pic + j]);
  GDR_STAGE_FOR(x, CM * CM, kR7IntraThreads) __builtin_nontemporal_store(Ma[(x / CM) * PC + x % CM], &rec[RL.ma + x]);
  __syncthreads();
  // L_z U into the right-hand side; O_z = M_z U to the record
  {
    constexpr int NT = CM / 16;
    const int NV = DV / 16;
    for (int tile = wid; tile < 2 * NT * NV; tile += kR7IntraWaves) {
      f32x4 acc = f4zero();
      const int which = tile / (NT * NV), r = tile % (NT * NV), it = r / NV, vt = r % NV;
      tile_nt(acc, which == 0 ? Lz : Mz, PC, 16 * it, UT, PC, 16 * vt, CM, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * it + 4 * (lane >> 4) + e, v = 16 * vt + (lane & 15);
        if (which == 0) Xl[t * NX + v] = acc[e];
        else __builtin_nontemporal_store(acc[e], &rec[RL.oz + t * DV + v]);
      }
    }
  }
  __syncthreads();
  // (I + L_a) X = RHS by forward substitution, one column per thread
  // Row t of L_a is read as 16-byte pieces when step t comes up; the
  // scheduling barrier keeps the compiler from hoisting every row's loads to
  // the top (which needs several hundred registers and spills at two waves
  // per SIMD). Two partial sums halve the dependent chain of a step.
  for (int col = tid; col < DV + DK; col += kR7IntraThreads) {
    float x[CM];
#pragma unroll
    for (int t = 0; t < CM; ++t) x[t] = Xl[t * NX + col];
#pragma unroll
    for (int t = 1; t < CM; ++t) {
      float acc0 = x[t], acc1 = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < t; s4 += 4) {
        const f32x4 l4 = *(const f32x4*)&La[t * PC + s4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (s4 + e < t) {
            if (e & 1) acc1 -= l4[e] * x[s4 + e];
            else acc0 -= l4[e] * x[s4 + e];
          }
      }
      x[t] = acc0 + acc1;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < CM; ++t) {
      if (col < DV) __builtin_nontemporal_store(x[t], &rec[RL.e0 + t * DV + col]);
      else __builtin_nontemporal_store(x[t], &rec[RL.g + t * DK + col - DV]);
    }
  }
}

// ------------------------------------------------------------------ chunk scan
// Per (b, h, VT value columns) (VT = 32, or 16 for d_v = 16), walking the
// chunks: E = E0 + G S0, O = Q_pi S0 - M_a E + O_z,
// S = Diag(pi_C) S0 - A~^T E + Z~^T U on the fp32 matrix cores, with the
// chunk's U slice read from the input u. The next chunk's record slices and
// U load into registers while the current chunk is worked on.
template <typename E, int DK, int CM, int VT>
__global__ __launch_bounds__(kR7ScanThreads) void rwkv7_scan_kernel(const float* __restrict__ ws,
                                                                 const E* __restrict__ u,
                                                                 const float* __restrict__ S0, E* __restrict__ o,
                                                                 float* __restrict__ S_out, int T, int DV) {
  constexpr int NW8 = kR7ScanWaves;
  constexpr int LY = DK + 4, LC = CM + 4, NST = DK / 16, PER = (NST + NW8 - 1) / NW8, NT = CM / 16, NHV = VT / 16;
  constexpr int NTH = kR7ScanThreads;
  // f32x4 pieces of each slice (4-element pieces of U) and the loads per thread
  constexpr int QA = CM * DK / 4, QM = CM * CM / 4, QT = DK * CM / 4, QE = CM * VT / 4, QU = CM * VT / 4;
  constexpr int NA = (QA + NTH - 1) / NTH, NM = (QM + NTH - 1) / NTH, NAT = (QT + NTH - 1) / NTH,
                NE = (QE + NTH - 1) / NTH, NU = (QU + NTH - 1) / NTH;
  using RW = Raw<E>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* Gl = (float*)smem;             // G     [t][j]
  float* Qpl = Gl + CM * LY;            // Q_pi  [t][j]
  float* Mal = Qpl + CM * LY;           // M_a   [t][s]
  float* ATl = Mal + CM * LC;           // A~^T  [j][s]
  float* STl = ATl + DK * LC;           // S^T   [v][j]
  float* ETl = STl + VT * LY;           // E^T   [v][s]
  float* E0l = ETl + VT * LC;           // E0    [t][v]
  float* OZl = E0l + CM * VT;           // O_z   [t][v]
  float* ZTl = OZl + CM * VT;           // Z~^T  [j][s]
  float* UTl = ZTl + DK * LC;           // U^T   [v][s]
  float* PIl = UTl + VT * LC;           // pi_C  [j]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, vl = lane & 15;
  // the value tiles of one head on one XCD, so its record slices are read
  // from HBM once and then hit that XCD's L2
  const int nvt = DV / VT, lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int bh = lin / nvt, v0 = (lin % nvt) * VT;
  const int nch = (T + CM - 1) / CM;
  const R7Layout RL = r7_layout(DK, DV, CM);
  f32x4 S[PER][NHV];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int J = wid + NW8 * i;
#pragma unroll
    for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * J + 4 * (lane >> 4) + e;
        S[i][hv][e] = (J < NST && S0) ? S0[((size_t)bh * DK + row) * DV + v0 + 16 * hv + vl] : 0.f;
      }
  }
  f32x4 pg[NA], pq[NA], pm[NM], pa[NAT], pz[NAT], pe[NE], po[NE];
  typename RW::R4 pu[NU];
  float pp = 0.f;
  auto fetch = [&](int c) {
    const float* rec = ws + ((size_t)bh * nch + c) * RL.floats;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int x = tid + NTH * i;
      if (QA % NTH == 0 || x < QA) {
        const int t = x / (DK / 4), j0 = 4 * (x % (DK / 4));
        pg[i] = *(const f32x4*)&rec[RL.g + t * DK + j0];
        pq[i] = *(const f32x4*)&rec[RL.qp + t * DK + j0];
      }
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int x = tid + NTH * i;
      if (QM % NTH == 0 || x < QM) pm[i] = *(const f32x4*)&rec[RL.ma + 4 * x];
    }
#pragma unroll
    for (int i = 0; i < NAT; ++i) {
      const int x = tid + NTH * i;
      if (QT % NTH == 0 || x < QT) {
        pa[i] = *(const f32x4*)&rec[RL.at + 4 * x];
        pz[i] = *(const f32x4*)&rec[RL.zt + 4 * x];
      }
    }
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int x = tid + NTH * i;
      if (QE % NTH == 0 || x < QE) {
        const int t = x / (VT / 4), q0 = 4 * (x % (VT / 4));
        pe[i] = *(const f32x4*)&rec[RL.e0 + t * DV + v0 + q0];
        po[i] = *(const f32x4*)&rec[RL.oz + t * DV + v0 + q0];
      }
    }
    // U: consecutive threads take consecutive rows t (the transposed LDS
    // writes in stage then hit distinct banks); rows past T are clamped
    // here and zeroed in stage
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int x = tid + NTH * i;
      if (QU % NTH == 0 || x < QU) {
        const int t = x % CM, q0 = 4 * (x / CM);
        pu[i] = RW::ld4(u + ((size_t)bh * T + row_in(c * CM + t, T)) * DV + v0 + q0);
      }
    }
    if (tid < DK) pp = rec[RL.pic + tid];
  };
  auto stage = [&](int c) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int x = tid + NTH * i;
      if (QA % NTH == 0 || x < QA) {
        const int t = x / (DK / 4), j0 = 4 * (x % (DK / 4));
        *(f32x4*)&Gl[t * LY + j0] = pg[i];
        *(f32x4*)&Qpl[t * LY + j0] = pq[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int x = tid + NTH * i;
      if (QM % NTH == 0 || x < QM) *(f32x4*)&Mal[(x / (CM / 4)) * LC + 4 * (x % (CM / 4))] = pm[i];
    }
#pragma unroll
    for (int i = 0; i < NAT; ++i) {
      const int x = tid + NTH * i;
      if (QT % NTH == 0 || x < QT) {
        *(f32x4*)&ATl[(x / (CM / 4)) * LC + 4 * (x % (CM / 4))] = pa[i];
        *(f32x4*)&ZTl[(x / (CM / 4)) * LC + 4 * (x % (CM / 4))] = pz[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int x = tid + NTH * i;
      if (QE % NTH == 0 || x < QE) {
        *(f32x4*)&E0l[4 * x] = pe[i];
        *(f32x4*)&OZl[4 * x] = po[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int x = tid + NTH * i;
      if (QU % NTH == 0 || x < QU) {
        const int t = x % CM, q0 = 4 * (x / CM);
        const bool ok = c * CM + t < T;
        const f32x4 uu = RW::un4(pu[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) UTl[(q0 + e) * LC + t] = ok ? uu[e] : 0.f;
      }
    }
    if (tid < DK) PIl[tid] = pp;
  };
  fetch(0);
  for (int c = 0; c < nch; ++c) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int J = wid + NW8 * i;
      if (J < NST) {
#pragma unroll
        for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
          for (int e = 0; e < 4; ++e) STl[(16 * hv + vl) * LY + 16 * J + 4 * (lane >> 4) + e] = S[i][hv][e];
      }
    }
    stage(c);
    if (c + 1 < nch) fetch(c + 1);
    __syncthreads();
    // Jobs 0 .. NP-1: E = E0 + G S0 for output tile p (to LDS, transposed);
    // jobs NP .. 2NP-1: the readout's Q_pi S0 for tile p, kept in the
    // registers of the wave that then finishes that tile of O
    constexpr int NP = NT * NHV, NJOB = 2 * NP, PJ = (NJOB + NW8 - 1) / NW8;
    f32x4 oacc[PJ];
#pragma unroll
    for (int i = 0; i < PJ; ++i) {
      const int job = wid + NW8 * i;
      oacc[i] = f4zero();
      if (job < NJOB) {
        const int p = job % NP, it = p / NHV, hv = p % NHV;
        if (job < NP) {
          f32x4 acc = f4zero();
          tile_nt(acc, Gl, LY, 16 * it, STl, LY, 16 * hv, DK, lane);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * it + 4 * (lane >> 4) + e;
            ETl[(16 * hv + vl) * LC + t] = E0l[t * VT + 16 * hv + vl] + acc[e];
          }
        } else {
          tile_nt(oacc[i], Qpl, LY, 16 * it, STl, LY, 16 * hv, DK, lane);
        }
      }
    }
    __syncthreads();
    // O = Q_pi S0 - M_a E + O_z
#pragma unroll
    for (int i = 0; i < PJ; ++i) {
      const int job = wid + NW8 * i;
      if (job >= NP && job < NJOB) {
        const int p = job - NP, it = p / NHV, hv = p % NHV;
        f32x4 me = f4zero();
        tile_nt(me, Mal, LC, 16 * it, ETl, LC, 16 * hv, CM, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * it + 4 * (lane >> 4) + e;
          if (c * CM + t < T)
            In<E>::store1(o + ((size_t)bh * T + c * CM + t) * DV + v0 + 16 * hv + vl,
                          oacc[i][e] - me[e] + OZl[t * VT + 16 * hv + vl]);
        }
      }
    }
    // S <- Diag(pi_C) S - A~^T E + Z~^T U
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int J = wid + NW8 * i;
      if (J < NST) {
#pragma unroll
        for (int hv = 0; hv < NHV; ++hv) {
          f32x4 ae = f4zero(), zu = f4zero();
          tile_nt(ae, ATl, LC, 16 * J, ETl, LC, 16 * hv, CM, lane);
          tile_nt(zu, ZTl, LC, 16 * J, UTl, LC, 16 * hv, CM, lane);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * J + 4 * (lane >> 4) + e;
            S[i][hv][e] = PIl[row] * S[i][hv][e] - ae[e] + zu[e];
          }
        }
      }
    }
    __syncthreads();
  }
  if (S_out) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int J = wid + NW8 * i;
      if (J < NST) {
#pragma unroll
        for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S_out[((size_t)bh * DK + 16 * J + 4 * (lane >> 4) + e) * DV + v0 + 16 * hv + vl] = S[i][hv][e];
      }
    }
  }
}

// ------------------------------------------------------------------ decode step
// Per (n, h): r = a S and p = (q * w) S from one read of S, e = c r,
// S <- Diag(w) S - a^T e + kw^T u,  o = p - (q . a) e + (q . kw) u.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void rwkv7_decode_kernel(const E* __restrict__ q, const E* __restrict__ w,
                                                           const E* __restrict__ a, const float* __restrict__ c,
                                                           const E* __restrict__ kw, const E* __restrict__ u,
                                                           float* __restrict__ S, E* __restrict__ o) {
  constexpr int TPR = DV / 4, RPP = 256 / TPR, NPASS = (DK + RPP - 1) / RPP;
  __shared__ float s_a[DK], s_qw[DK], s_w[DK], s_kw[DK], s_q[DK], s_u[DV];
  __shared__ float s_red[2][RPP][DV];
  __shared__ float s_dot[2];
  const int tid = threadIdx.x;
  const size_t head = blockIdx.x;
  const size_t offK = head * DK, offV = head * DV;
  float* Sh = S + head * DK * DV;
  const int c4 = (tid % TPR) * 4, rg = tid / TPR;
  f32x4 st[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int j = rg + RPP * p;
    st[p] = (rg < RPP && j < DK) ? *(const f32x4*)(Sh + (size_t)j * DV + c4) : f4zero();
  }
  for (int j = tid; j < DK; j += 256) {
    const float ww = (float)w[offK + j], qq = (float)q[offK + j];
    s_a[j] = (float)a[offK + j];
    s_w[j] = ww;
    s_kw[j] = (float)kw[offK + j];
    s_q[j] = qq;
    s_qw[j] = qq * ww;
  }
  for (int v = tid; v < DV; v += 256) s_u[v] = (float)u[offV + v];
  __syncthreads();
  if (tid < 64) {   // q . a and q . kw by one wave
    float da = 0.f, dz = 0.f;
    for (int j = tid; j < DK; j += 64) {
      da += s_q[j] * s_a[j];
      dz += s_q[j] * s_kw[j];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      da += __shfl_xor(da, off, 64);
      dz += __shfl_xor(dz, off, 64);
    }
    if (tid == 0) {
      s_dot[0] = da;
      s_dot[1] = dz;
    }
  }
  f32x4 r = f4zero(), pq = f4zero();
  if (rg < RPP) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int j = rg + RPP * p;
      if (j < DK) {
        const float aj = s_a[j], qw = s_qw[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] += aj * st[p][e];
          pq[e] += qw * st[p][e];
        }
      }
    }
    *(f32x4*)&s_red[0][rg][c4] = r;
    *(f32x4*)&s_red[1][rg][c4] = pq;
  }
  __syncthreads();
  const float cc = c[head];
  f32x4 ev = f4zero(), pr = f4zero();
  for (int x = 0; x < RPP; ++x) {
    const f32x4 a4 = *(const f32x4*)&s_red[0][x][c4];
    const f32x4 b4 = *(const f32x4*)&s_red[1][x][c4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { ev[e] += a4[e]; pr[e] += b4[e]; }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) ev[e] *= cc;
  if (rg < RPP) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int j = rg + RPP * p;
      if (j < DK) {
        const float ww = s_w[j], aj = s_a[j], zj = s_kw[j];
        f32x4 nv;
#pragma unroll
        for (int e = 0; e < 4; ++e) nv[e] = ww * st[p][e] - aj * ev[e] + zj * s_u[c4 + e];
        *(f32x4*)(Sh + (size_t)j * DV + c4) = nv;
      }
    }
  }
  if (rg == 0) {
    const float da = s_dot[0], dz = s_dot[1];
    f32x4 ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = pr[e] - da * ev[e] + dz * s_u[c4 + e];
    In<E>::store4(o + offV + c4, ov);
  }
}

// ------------------------------------------------------------------ host launch
template <typename E, int DK, int CM>
static int r7_launch(const Rwkv7Args& a, void* ws) {
  const int BH = a.B * a.H, nch = (a.T + CM - 1) / CM;
  int T = a.T, DV = a.dv;
  const hipStream_t st = (hipStream_t)a.stream;
  float* wsf = (float*)ws;
  {
    const int P = DK + 4, PC = CM + 4, NX = DV + DK + 4;
    const int tg = (2 * 16 + 2 * CM) * P, tr = DV * PC + CM * NX;
    const int lds = 4 * (4 * CM * P + CM + 4 * CM * PC + (tg > tr ? tg : tr));
    auto kern = rwkv7_intra_kernel<E, DK, CM>;
    if (!allow_lds((const void*)kern, lds)) return GDR_ERR_LAUNCH;
    const E *q = (const E*)a.q, *w = (const E*)a.w, *aa = (const E*)a.a, *kw = (const E*)a.kw, *u = (const E*)a.u;
    const float* c = a.c;
    void* args[] = {&q, &w, &aa, &c, &kw, &u, &wsf, &T, &DV};
    if (hipLaunchKernel((const void*)kern, dim3(BH * nch), dim3(kR7IntraThreads), args, lds, st) != hipSuccess)
      return GDR_ERR_LAUNCH;
  }
  {
    // 32-column value tiles where d_v allows, else 16
    constexpr int LY = DK + 4, LC = CM + 4;
    const int vt = a.dv % 32 == 0 ? 32 : 16;
    const int lds = 4 * (2 * CM * LY + CM * LC + DK * LC + vt * LY + vt * LC + 2 * CM * vt + DK * LC + vt * LC + DK);
    const void* kern = vt == 32 ? (const void*)rwkv7_scan_kernel<E, DK, CM, 32>
                                : (const void*)rwkv7_scan_kernel<E, DK, CM, 16>;
    if (!allow_lds(kern, lds)) return GDR_ERR_LAUNCH;
    const float* wsc = wsf;
    const E* u = (const E*)a.u;
    const float* S0 = a.S0;
    E* o = (E*)a.o;
    float* So = a.S_out;
    void* args[] = {&wsc, &u, &S0, &o, &So, &T, &DV};
    if (hipLaunchKernel(kern, dim3(BH * (DV / vt)), dim3(kR7ScanThreads), args, lds, st) != hipSuccess)
      return GDR_ERR_LAUNCH;
  }
  return GDR_OK;
}

template <typename E, int CM>
static int r7_dk(const Rwkv7Args& a, void* ws) {
  switch (a.dk) {
    case 16: return r7_launch<E, 16, CM>(a, ws);
    case 32: return r7_launch<E, 32, CM>(a, ws);
    case 64: return r7_launch<E, 64, CM>(a, ws);
    case 128: return r7_launch<E, 128, CM>(a, ws);
  }
  return GDR_ERR_UNSUPPORTED;
}

int rwkv7_fwd_launch(const Rwkv7Args& a, void* ws) {
  if (a.dtype == GDR_BF16) return a.chunk == 16 ? r7_dk<__bf16, 16>(a, ws) : r7_dk<__bf16, 32>(a, ws);
  return a.chunk == 16 ? r7_dk<float, 16>(a, ws) : r7_dk<float, 32>(a, ws);
}

template <typename E, int DK>
static int r7_decode_dv(const Rwkv7Args& a) {
  const E *q = (const E*)a.q, *w = (const E*)a.w, *aa = (const E*)a.a, *kw = (const E*)a.kw, *u = (const E*)a.u;
  const float* c = a.c;
  float* S = a.S_out;
  E* o = (E*)a.o;
  void* args[] = {&q, &w, &aa, &c, &kw, &u, &S, &o};
  const void* kern = nullptr;
  switch (a.dv) {
    case 16: kern = (const void*)rwkv7_decode_kernel<E, DK, 16>; break;
    case 32: kern = (const void*)rwkv7_decode_kernel<E, DK, 32>; break;
    case 64: kern = (const void*)rwkv7_decode_kernel<E, DK, 64>; break;
    case 128: kern = (const void*)rwkv7_decode_kernel<E, DK, 128>; break;
    default: return GDR_ERR_UNSUPPORTED;
  }
  return hipLaunchKernel(kern, dim3(a.B * a.H), dim3(256), args, 0, (hipStream_t)a.stream) == hipSuccess
             ? GDR_OK
             : GDR_ERR_LAUNCH;
}

template <typename E>
static int r7_decode_dk(const Rwkv7Args& a) {
  switch (a.dk) {
    case 16: return r7_decode_dv<E, 16>(a);
    case 32: return r7_decode_dv<E, 32>(a);
    case 64: return r7_decode_dv<E, 64>(a);
    case 128: return r7_decode_dv<E, 128>(a);
  }
  return GDR_ERR_UNSUPPORTED;
}

int rwkv7_decode_launch(const Rwkv7Args& a) {
  return a.dtype == GDR_BF16 ? r7_decode_dk<__bf16>(a) : r7_decode_dk<float>(a);
}

}  // namespace gdr
