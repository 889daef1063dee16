// Two-kernel chunkwise forward of the xLSTM mLSTM cell on gfx950
// ("Exponential gates and matrix memory: xLSTM and RWKV-7", §13.4 and the
// solution to Exercise 13.6), [d_k, d_v] state orientation, through a
// caller-provided workspace.
//
// With F_t = sum_{r<=t} log sigmoid(f~_r), a_s = i~_s - F_s and the chunk-local
// running max A_t = max_{s<=t} a_s, the stabiliser of the page's recurrence is
// m_t = F_t + mu_t with mu_t = max(m0, A_t). Every term splits into a part
// that depends only on the chunk and a factor <= 1 that depends on m0:
//   h^_t = e^{m0 - mu_t} q_t C0 + e^{A_t - mu_t} H_t,
//          H_t = sum_{s<=t} e^{a_s - A_t} (q_t . k_s) v_s        (same for n^ with v = 1)
//   C_C  = e^{m0 - mu_C} C0 + e^{A_C - mu_C} sum_s e^{a_s - A_C} k_s^T v_s,
//   h_t  = h^_t / max(|n^_t|, e^{-m_t}),  m_C = F_C + mu_C.
// The intra kernel computes the chunk-only parts (H, its normaliser row N,
// K~ = e^{a_s - A_C} k_s, V^T, F, A) for every chunk in parallel into a
// workspace record; the scan walks the chunks of each head doing q C0, the
// combination and the state update. All exponents are <= 0.
#include "gdr_device.hpp"
#include "gdr_internal.h"
#include "gdr_host.hpp"

namespace gdr {

namespace {

constexpr int align16m(int x) { return (x + 15) / 16 * 16; }

// Workspace record of one (b, h, chunk); es = element size of the input dtype.
// Row-major form: H [t][v], V^T [v][s], K~^T [j][s]. Fragment form (fm; bf16,
// d_k and C multiples of 32): the same matrices cut into the 16-row operand
// tiles of the 16x16x32 MFMA, each tile 1 KiB of consecutive bytes in lane
// order (lane 16g + c of tile (R, S) holds row 16R + c, k = 32S + 8g .. +7),
// H in 16x16 accumulator tiles (512 B, lane 16g + c holds t = 16I + c,
// v = 16V + 4g .. +3), plus q in the operand tiles.
struct MRec {
  int hi, vt, kt, qf, ni, f, a, bytes;
};
__host__ __device__ __forceinline__ MRec mrec_layout(int dk, int dv, int C, int es, bool fm = false) {
  MRec r;
  r.hi = 0;                     // H     C x dv (input precision)
  r.vt = r.hi + C * dv * es;    // V^T   dv x C
  r.kt = r.vt + dv * C * es;    // K~^T  dk x C
  r.qf = r.kt + dk * C * es;    // q     C x dk (fragment form only)
  r.ni = r.qf + (fm ? C * dk * es : 0);   // N [t] fp32
  r.f = r.ni + C * 4;           // F     [t] fp32
  r.a = r.f + C * 4;            // A     [t] fp32
  r.bytes = align16m(r.a + C * 4);
  return r;
}

// Whether the two-kernel mLSTM path of these shapes uses the fragment-form
// record and the register scan (which addresses a head's records with 32-bit
// offsets).
__host__ __forceinline__ bool mlstm_fm(int dtype, int dk, int dv, int C, long long T) {
  if (dtype != GDR_BF16 || dk % 32 != 0 || C % 32 != 0 || dv % 16 != 0) return false;
  const long long nchunks = (T + C - 1) / C;
  return nchunks * mrec_layout(dk, dv, C, 2, true).bytes < (1LL << 31);
}

__device__ __forceinline__ float log_sigmoid2(float x) {
  // log sigmoid(x) = min(x, 0) - log1p(exp(-|x|))
  return fminf(x, 0.f) - log1pf(__expf(-fabsf(x)));
}

// 16-byte slot swizzle of a row with n slots: rows 16 apart in a fragment
// read fall on distinct bank groups.
__device__ __forceinline__ int mswz(int r, int n) { return n >= 16 ? (r & 15) : (r / (16 / n)) % n; }

template <typename E> struct MOut;
template <> struct MOut<float> {
  static __device__ __forceinline__ void quad(float* p, f32x4 v) { *(f32x4*)p = v; }
  static __device__ __forceinline__ void oct(float* p, const float* x) {
    *(f32x4*)p = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};
template <> struct MOut<__bf16> {
  static __device__ __forceinline__ void quad(__bf16* p, f32x4 v) { In<__bf16>::store4(p, v); }
  static __device__ __forceinline__ void oct(__bf16* p, const float* x) {
    bf16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (__bf16)x[e];
    *(bf16x8*)p = h;
  }
};

// An operand slice holding `val` in row 0 of a 16-row tile and 0 elsewhere
// (the normaliser's "value" column); c16 = -1 gives a zero slice.
template <int MODE>
__device__ __forceinline__ Frag<MODE> ones_row0(int c16, float val = 1.f) {
  Frag<MODE> f;
  const float x = c16 == 0 ? val : 0.f;
  if constexpr (MODE == kF32) {
    f.a = f32x4{x, x, x, x};
    f.b = f.a;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.hi[e] = (__bf16)x;
  }
  return f;
}

}  // namespace

// ============================================================================ intra kernel
constexpr int kMThreads = 512;

template <typename Tin, int DK, int CM>
struct MIntraSmem {
  static constexpr bool F32 = std::is_same<Tin, float>::value;
  static constexpr int NS = F32 ? 2 : 1;            // bf16 planes' worth of bytes per element
  static constexpr int DVM = F32 ? 128 : 256;       // largest d_v
  static constexpr int LDK = DK + 8, LDC = CM + 8;
  static constexpr int QS = 0;                       // q   [t][j]
  static constexpr int KS = QS + NS * CM * LDK * 2;  // k   [s][j]
  static constexpr int VS = KS + NS * CM * LDK * 2;  // V^T [v][s], 8-row slots swizzled per 16 columns
  static constexpr int WS = VS + NS * DVM * LDC * 2; // W   [t][s]
  static constexpr int SC = align16m(WS + NS * CM * LDC * 2);  // fp32 F, a, A
  static constexpr int WP = SC + 3 * CM * 4;         // fp32 row sums of W per s-block [J][t]
  static constexpr int TOTAL = WP + (CM / 16) * CM * 4;
  static_assert(TOTAL <= 160 * 1024, "mLSTM intra kernel LDS exceeds 160 KiB");
};

// QC: the fragment-form record also gets the tile-order copy of q (the
// register scan reads it; the wide scan reads q from the input instead and
// leaves that part of the record unwritten).
template <typename Tin, int DK, int CM, bool FM, bool QC = true>
__global__ __launch_bounds__(kMThreads, 2) void mlstm_intra_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ i_tilde, const float* __restrict__ f_tilde, char* __restrict__ ws,
    int T, int DV, int nchunks, int nitems) {
  using L = MIntraSmem<Tin, DK, CM>;
  constexpr bool F32 = L::F32;
  constexpr int MM = F32 ? kF32 : kBF;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NW = kMThreads / 64;
  constexpr int NB = CM / 16;
  constexpr int NP = NB * (NB + 1) / 2;
  constexpr int MAXP = (NP + NW - 1) / NW;
  constexpr int ES = sizeof(Tin);
  constexpr int KP = DK * ES / 16;                  // 16-byte pieces per q / k row
  constexpr int NPQ = (CM * KP + kMThreads - 1) / kMThreads;
  constexpr int NPV = (CM * L::DVM * ES / 16 + kMThreads - 1) / kMThreads;
  constexpr int EP = 16 / ES;                       // elements per piece
  constexpr int XM = CM / 8 - 1;
  typedef u32x4 P16;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const MRec RL = mrec_layout(DK, DV, CM, ES, FM);
  static_assert(!FM || (!F32 && DK % 32 == 0 && CM % 32 == 0), "fragment-form record shape");
  const int VP = DV * ES / 16;                       // pieces per v row
  const int NVT = DV / 16 + 1;                       // value tiles + the normaliser tile
  float* sF = (float*)(smem + L::SC);
  float* sa = sF + CM;
  float* sAm = sa + CM;
  float* sWP = (float*)(smem + L::WP);
  auto voff = [](int col, int t) { return col * L::LDC + 8 * ((t >> 3) ^ ((col >> 4) & XM)) + (t & 7); };

  int item = blockIdx.x;
  if (item >= nitems) return;

  P16 xq[NPQ], xk[NPQ], xv[NPV];
  float xf = 0.f, xi = 0.f;
  auto issue = [&](int it) {
    const int bh = it / nchunks, tb = (it % nchunks) * CM;
    const char* qh = (const char*)(q + (size_t)bh * T * DK);
    const char* kh = (const char*)(k + (size_t)bh * T * DK);
    const char* vh = (const char*)(v + (size_t)bh * T * DV);
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      int p = tid + kMThreads * i;
      p = p < CM * KP ? p : 0;
      const int r = p / KP, c = p % KP, t = tb + r;
      const size_t off = (size_t)(t < T ? t : T - 1) * DK * ES + 16 * c;
      // non-temporal: each input row is read once (the 8K path 1.8% faster)
      xq[i] = __builtin_nontemporal_load((const P16*)(qh + off));
      xk[i] = __builtin_nontemporal_load((const P16*)(kh + off));
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      int p = tid + kMThreads * i;
      p = p < CM * VP ? p : 0;
      const int r = p / VP, c = p % VP, t = tb + r;
      xv[i] = __builtin_nontemporal_load((const P16*)(vh + (size_t)(t < T ? t : T - 1) * DV * ES + 16 * c));
    }
    const int tg = tb + (lane < CM ? lane : 0);
    const size_t og = (size_t)bh * T + (tg < T ? tg : T - 1);
    xf = f_tilde[og];
    xi = i_tilde[og];
  };
  // bf16: the next item's inputs are fetched during this item's products;
  // fp32 fetches at the start of each item
  if constexpr (!F32) issue(item);

  for (; item < nitems; item += gridDim.x) {
    if constexpr (F32) issue(item);
    const int t0 = (item % nchunks) * CM;
    char* rec = ws + (size_t)item * RL.bytes;

    // ---- q, k -> LDS as they are; v -> V^T; rows past T are zero
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int p = tid + kMThreads * i;
      if (p < CM * KP) {
        const int r = p / KP, c = p % KP;
        const bool ok = t0 + r < T;
        const P16 z = {0u, 0u, 0u, 0u};
        *(P16*)(smem + L::QS + (r * L::LDK) * 2 * L::NS + 16 * c) = ok ? xq[i] : z;
        *(P16*)(smem + L::KS + (r * L::LDK) * 2 * L::NS + 16 * c) = ok ? xk[i] : z;
      }
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int p = tid + kMThreads * i;
      if (p < CM * VP) {
        const int r = p / VP, c0 = (p % VP) * EP;
        const bool ok = t0 + r < T;
        if constexpr (F32) {
          const f32x4 x = __builtin_bit_cast(f32x4, xv[i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) ((float*)(smem + L::VS))[voff(c0 + e, r)] = ok ? x[e] : 0.f;
        } else {
          const u32x4 x = xv[i];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t hv = (uint16_t)(x[e >> 1] >> (16 * (e & 1)));
            ((uint16_t*)(smem + L::VS))[voff(c0 + e, r)] = ok ? hv : (uint16_t)0;
          }
        }
      }
    }
    // ---- gates: F (prefix sum of log sigmoid f~), a = i~ - F, A (prefix max of a)
    if (wid == 0) {
      const int t = lane;
      const bool valid = t < CM && t0 + t < T;
      float F = valid ? log_sigmoid2(xf) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(F, off, 64);
        if (lane >= off) F += y;
      }
      const float a = valid ? xi - F : -INFINITY;
      float A = a;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(A, off, 64);
        if (lane >= off) A = fmaxf(A, y);
      }
      if (t < CM) {
        sF[t] = F;
        sa[t] = a;
        sAm[t] = A;
        ((float*)(rec + RL.f))[t] = F;
        ((float*)(rec + RL.a))[t] = A;
      }
    }
    __syncthreads();
    if constexpr (!F32) {
      // always issued (item 0 after the last, an L2-resident re-read), so
      // the loads in flight do not depend on a branch and the compiler's
      // wait counts stay exact
      issue(item + (int)gridDim.x < nitems ? item + (int)gridDim.x : 0);
    }

    // ---- W[t][s] = (q_t . k_s) e^{a_s - A_t}, s <= t (transposed score tiles)
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int p = wid + NW * i;
      if (p < NP) {
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= p) ++I;
        const int J = p - I * (I + 1) / 2;
        f32x4 acc = f4zero();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          Frag<MM> A = ldfrag<MM>(smem + L::KS, 0, L::LDK, 16 * J, k0, DK, lane);
          Frag<MM> B = ldfrag<MM>(smem + L::QS, 0, L::LDK, 16 * I, k0, DK, lane);
          mma<MM>(acc, A, B);
        }
        const int t = 16 * I + c16, s0 = 16 * J + 4 * g;
        const float At = sAm[t];
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = s0 + e;
          w[e] = s <= t ? acc[e] * __expf(sa[s] - At) : 0.f;
        }
        st4<MM>(smem + L::WS, 0, t * L::LDC + s0, w);
        // the normaliser's sums are taken in fp32 before W is rounded to the
        // operand precision: they can cancel, and a rounded W would leave an
        // error of the order of the terms in a small sum
        float rs = (w[0] + w[1]) + (w[2] + w[3]);
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        if (g == 0) sWP[J * CM + t] = rs;
      }
    }
    __syncthreads();

    // ---- H^T = V^T W^T: tile (value tile vt, t-block I); the last "tile"
    // is the normaliser N[t] = sum_s W[t][s] from the fp32 block sums
    const int nht = NVT * NB;
    for (int qi = wid; qi < nht; qi += NW) {
      const int vt = qi / NB, I = qi % NB, kend = 16 * (I + 1);
      const bool nt = vt == NVT - 1;
      if (nt) {
        if (g == 0) {
          const int t = 16 * I + c16;
          float N = 0.f;
          for (int J = 0; J <= I; ++J) N += sWP[J * CM + t];
          ((float*)(rec + RL.ni))[t] = N;
        }
        continue;
      }
      f32x4 acc = f4zero();
#pragma unroll
      for (int k0 = 0; k0 < CM; k0 += 32) {
        if (k0 < kend) {
          const int kk = k0 + 8 * g;
          Frag<MM> A = ldfrag<MM>(smem + L::VS, 0, L::LDC, 16 * vt, 8 * ((kk >> 3) ^ (vt & XM)) - 8 * g,
                                  CM, lane);
          Frag<MM> B = ldfrag<MM>(smem + L::WS, 0, L::LDC, 16 * I, k0, kend, lane);
          if (kk >= kend) A = ones_row0<MM>(-1);   // zero slice (B is zero there too)
          mma<MM>(acc, A, B);
        }
      }
      const int t = 16 * I + c16;
      if constexpr (FM) MOut<Tin>::quad((Tin*)(rec + RL.hi) + ((I * (DV / 16) + vt) * 64 + lane) * 4, acc);
      else MOut<Tin>::quad((Tin*)(rec + RL.hi) + t * DV + 16 * vt + 4 * g, acc);
    }

    // ---- K~^T = (e^{a_s - A_C} k_s)^T and V^T to the record (16-byte pieces;
    // in the fragment form piece p is lane p % 64 of tile p / 64, so the
    // stores are consecutive)
    const float AC = sAm[CM - 1];
    constexpr int SP = CM / 8;
    constexpr int KSC = CM / 32;
    for (int p = tid; p < DK * SP; p += kMThreads) {
      int j, s0;
      if constexpr (FM) {
        const int f = p >> 6, l = p & 63;
        j = 16 * (f / KSC) + (l & 15);
        s0 = 32 * (f % KSC) + 8 * (l >> 4);
      } else {
        j = p / SP;
        s0 = (p % SP) * 8;
      }
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ld1<MM>(smem + L::KS, 0, (s0 + e) * L::LDK + j) * __expf(sa[s0 + e] - AC);
      MOut<Tin>::oct((Tin*)(rec + RL.kt) + (FM ? 8 * p : j * CM + s0), x);
    }
    for (int p = tid; p < DV * SP; p += kMThreads) {
      int col, s0;
      if constexpr (FM) {
        const int f = p >> 6, l = p & 63;
        col = 16 * (f / KSC) + (l & 15);
        s0 = 32 * (f % KSC) + 8 * (l >> 4);
      } else {
        col = p / SP;
        s0 = (p % SP) * 8;
      }
      const char* src = smem + L::VS + (size_t)voff(col, s0) * ES;
      char* dst = rec + RL.vt + (FM ? 16 * p : (col * CM + s0) * ES);
      *(P16*)dst = *(const P16*)src;
      if constexpr (F32) *(P16*)(dst + 16) = *(const P16*)(src + 16);
    }
    if constexpr (FM && QC) {
      // q (rows past T are zero in LDS) in the operand tiles of the readout
      constexpr int KSQ = DK / 32;
      for (int p = tid; p < CM * DK / 8; p += kMThreads) {
        const int f = p >> 6, l = p & 63;
        const int r = 16 * (f / KSQ) + (l & 15), c = 4 * (f % KSQ) + (l >> 4);
        *(P16*)(rec + RL.qf + 16 * p) = *(const P16*)(smem + L::QS + r * L::LDK * 2 + 16 * c);
      }
    }
    __syncthreads();
  }
}

// ============================================================================ scan kernel
constexpr int kMScanThreads = 512;

template <typename Tin, int DK, int VT, int CM>
struct MScanSmem {
  static constexpr bool F32 = std::is_same<Tin, float>::value;
  static constexpr int ES = sizeof(Tin);
  static constexpr int WQ = DK * ES, WC = CM * ES, WH = VT * ES;   // row bytes
  static constexpr int Q = 0;                        // q     [t][j]
  static constexpr int KT = Q + CM * WQ;             // K~^T  [j][s]
  static constexpr int VTS = KT + DK * WC;           // V^T   [v][s], this tile's rows
  static constexpr int HI = VTS + VT * WC;           // H     [t][v], this tile's columns
  static constexpr int SF = HI + CM * WH;            // F, A, N fp32 (record order N, F, A)
  static constexpr int STAGE = align16m(SF + 3 * CM * 4);
  static constexpr int NS = F32 ? 2 : 1;
  static constexpr int NVA = VT / 16 + 1;            // value tiles + the normaliser tile
  static constexpr int LDK = DK + 8;
  static constexpr int S0T = STAGE;                  // [C | n]^T [v][j]
  static constexpr int TOTAL = S0T + 2 * 16 * NVA * LDK * 2;   // fp32, or bf16 hi + lo planes
  static_assert(TOTAL <= 160 * 1024, "mLSTM scan LDS exceeds 160 KiB");
  // 16-byte pieces of one chunk: q rows (from the input), then the record parts
  static constexpr int NQP = CM * WQ / 16;
  static constexpr int NKP = DK * WC / 16, NVP = VT * WC / 16, NHP = CM * WH / 16, NSP = 3 * CM * 4 / 16;
  static constexpr int NRP = NKP + NVP + NHP + NSP;
};

template <typename Tin, int DK, int VT, int CM>
__global__ __launch_bounds__(kMScanThreads, 2) void mlstm_scan_kernel(
    const Tin* __restrict__ q, const char* __restrict__ ws, const float* __restrict__ C0,
    const float* __restrict__ n0, const float* __restrict__ m0, Tin* __restrict__ h, float* C_out,
    float* n_out, float* m_out, int T, int DV) {
  using L = MScanSmem<Tin, DK, VT, CM>;
  constexpr bool F32 = L::F32;
  constexpr int MM = F32 ? kF32 : kBF;
  // the state copy that q reads: fp32, or bf16 hi + lo planes (the readout's
  // sums can cancel, so a single bf16 rounding of the state is not enough)
  constexpr int SM = F32 ? kF32 : kSP;
  constexpr int NW = kMScanThreads / 64;
  constexpr int NVL = VT / 16, NVA = L::NVA;
  constexpr int NB = CM / 16;
  constexpr int KS = DK >= 32 ? DK / 32 : 1;
  constexpr int KSC = CM >= 32 ? CM / 32 : 1;
  // Roles: waves w < NB read out t-block w (every value tile and the
  // normaliser, so each normalises its own rows); the other NU waves update
  // the state, wave NB + u owning j-blocks u, u + NU, ... with every value
  // tile. The two run side by side on the same S0 and chunk data.
  static_assert(NB < NW, "needs a wave for the state update");
  constexpr int NU = NW - NB;
  constexpr int NJB = DK / 16;
  constexpr int JPW = (NJB + NU - 1) / NU;
  constexpr int MAXU = JPW * NVA;
  constexpr int NPQ = (L::NQP + kMScanThreads - 1) / kMScanThreads;
  constexpr int NPR = (L::NRP + kMScanThreads - 1) / kMScanThreads;
  constexpr int LDK = L::LDK;
  constexpr int P_S = 16 * NVA * LDK * 2;
  typedef u32x4 P16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* S0T = smem + L::S0T;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nvt = DV / VT;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int bh = lin / nvt, vt0 = (lin % nvt) * VT;
  const int nchunks = (T + CM - 1) / CM;
  const MRec RL = mrec_layout(DK, DV, CM, L::ES);
  const char* wsh = ws + (size_t)bh * nchunks * RL.bytes;
  const char* qh = (const char*)(q + (size_t)bh * T * DK);

  // ---- piece plan (fixed for the pass): q pieces by row; record pieces by offset
  int qr[NPQ], qlo[NPQ];
#pragma unroll
  for (int i = 0; i < NPQ; ++i) {
    int p = tid + kMScanThreads * i;
    if (p >= L::NQP) p = L::NQP - 1;
    constexpr int n = L::WQ / 16;
    const int r = p / n, c = p % n;
    qr[i] = r * L::WQ + 16 * c;
    qlo[i] = L::Q + r * L::WQ + 16 * (c ^ mswz(r, n));
  }
  int rgo[NPR], rlo[NPR];
#pragma unroll
  for (int i = 0; i < NPR; ++i) {
    int p = tid + kMScanThreads * i;
    if (p >= L::NRP) p = L::NRP - 1;
    int go, lo;
    if (p < L::NKP) {
      constexpr int n = L::WC / 16;
      const int r = p / n, c = p % n;
      go = RL.kt + r * L::WC + 16 * c;
      lo = L::KT + r * L::WC + 16 * (c ^ mswz(r, n));
    } else if (p < L::NKP + L::NVP) {
      constexpr int n = L::WC / 16;
      const int qq = p - L::NKP, r = qq / n, c = qq % n;
      go = RL.vt + (vt0 + r) * L::WC + 16 * c;
      lo = L::VTS + r * L::WC + 16 * (c ^ mswz(r, n));
    } else if (p < L::NKP + L::NVP + L::NHP) {
      constexpr int n = L::WH >= 16 ? L::WH / 16 : 1;
      const int qq = p - L::NKP - L::NVP, r = qq / n, c = qq % n;
      go = RL.hi + (r * DV + vt0) * L::ES + 16 * c;
      lo = L::HI + r * L::WH + 16 * (c ^ mswz(r, n));
    } else {
      const int qq = p - L::NKP - L::NVP - L::NHP;
      go = RL.ni + 16 * qq;
      lo = L::SF + 16 * qq;
    }
    rgo[i] = go;
    rlo[i] = lo;
  }
  struct Set {
    P16 q[NPQ], r[NPR];
  };
  auto load = [&](int ch, Set& x) {
    const int c = ch < nchunks ? ch : nchunks - 1;
    const char* rec = wsh + (size_t)c * RL.bytes;
    const int t0 = c * CM;
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int row = qr[i] / L::WQ, t = t0 + row;
      const size_t off = (size_t)(t < T ? t : T - 1) * L::WQ + (qr[i] - row * L::WQ);
      x.q[i] = *(const P16*)(qh + off);
    }
#pragma unroll
    for (int i = 0; i < NPR; ++i) x.r[i] = *(const P16*)(rec + rgo[i]);
  };
  auto stage = [&](const Set& x) {
#pragma unroll
    for (int i = 0; i < NPQ; ++i) *(P16*)(smem + qlo[i]) = x.q[i];
#pragma unroll
    for (int i = 0; i < NPR; ++i) *(P16*)(smem + rlo[i]) = x.r[i];
  };
  // fragment of a staged swizzled row-major matrix (row bytes w)
  auto sfrag = [&](int moff, int w, int row0, int k0) {
    const int n = w / 16;
    const int r = row0 + c16;
    Frag<MM> f;
    if constexpr (F32) {
      const int c = ((k0 >> 2) + 2 * g) & (n - 1);   // 8 fp32 = two slots
      f.a = *(const f32x4*)(smem + moff + r * w + 16 * (c ^ mswz(r, n)));
      f.b = *(const f32x4*)(smem + moff + r * w + 16 * ((c + 1) ^ mswz(r, n)));
    } else {
      const int c = ((k0 >> 3) + g) & (n - 1);
      f.hi = *(const bf16x8*)(smem + moff + r * w + 16 * (c ^ mswz(r, n)));
    }
    return f;
  };

  // ---- state [C | n] (j-block, value tile incl. normaliser) in registers, S0^T in LDS
  const bool have_state = C0 != nullptr;
  float mprev = have_state ? m0[bh] : -INFINITY;
  const bool uw = wid >= NB;                        // state-update wave
  const int uid = wid - NB;
  f32x4 Sacc[MAXU];
#pragma unroll
  for (int i = 0; i < MAXU; ++i) {
    Sacc[i] = f4zero();
    const int jt = uid + NU * (i / NVA), vl = i % NVA;
    if (uw && jt < NJB) {
      if (have_state) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * jt + 4 * g + e;
          if (vl < NVL) Sacc[i][e] = C0[(size_t)bh * DK * DV + (size_t)j * DV + vt0 + 16 * vl + c16];
          else Sacc[i][e] = c16 == 0 ? n0[(size_t)bh * DK + j] : 0.f;
        }
      }
      st4<SM>(S0T, P_S, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[i]);
    }
  }

  // one chunk. Phase 1 (no barrier inside): readout waves form q C0 for
  // their t-block, combine it with H and N, normalise and store h; update
  // waves form the new [C | n] in registers. Phase 2, after a barrier (all
  // reads of S0^T and of the stage done): update waves write S0^T.
  auto compute = [&](int ch) {
    const int t0 = ch * CM;
    const float* stF = (const float*)(smem + L::SF + CM * 4);
    const float* stA = (const float*)(smem + L::SF + 2 * CM * 4);
    const float* stN = (const float*)(smem + L::SF);
    if (!uw) {
      const int I = wid;
      f32x4 acc[NVA];
#pragma unroll
      for (int vl = 0; vl < NVA; ++vl) acc[vl] = f4zero();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bool kv = 32 * s + 8 * g < DK;
        Frag<MM> B = sfrag(L::Q, L::WQ, 16 * I, 32 * s);
        if (!kv) B = ones_row0<MM>(-1);
#pragma unroll
        for (int vl = 0; vl < NVA; ++vl) {
          if constexpr (F32) {
            Frag<MM> A = ldfrag<MM>(S0T, P_S, LDK, 16 * vl, 32 * s, DK, lane);
            mma<MM>(acc[vl], A, B);
          } else {
            mma_split(acc[vl], ldfrag<kSP>(S0T, P_S, LDK, 16 * vl, 32 * s, DK, lane), B);
          }
        }
      }
      // acc[vl][e] = (q_t C0)[v = 16vl + 4g + e] for t = 16I + c16; the
      // normaliser tile's row 0 (lanes g = 0, e = 0) is q_t . n0
      const int t = 16 * I + c16, tg = t0 + t;
      const float At = stA[t];
      const float mu = fmaxf(mprev, At);
      const float si = __expf(At - mu);
      const float se = mprev == -INFINITY ? 0.f : __expf(mprev - mu);
      const float nq = __shfl(acc[NVL][0], c16, 64);   // lane (g = 0, c16) holds q_t . n0
      const float nbar = se * nq + si * stN[t];
      const float den = fmaxf(fabsf(nbar), __expf(-(stF[t] + mu)));
      const float inv = 1.f / den;
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl) {
        // H[t][16vl + 4g .. +3]
        constexpr int n = L::WH >= 16 ? L::WH / 16 : 1;
        const int byte = (16 * vl + 4 * g) * L::ES;
        const int c = byte / 16;
        const char* hp = smem + L::HI + t * L::WH + 16 * (c ^ mswz(t, n)) + (byte & 15);
        f32x4 hv;
        if constexpr (F32) {
          hv = *(const f32x4*)hp;
        } else {
          typedef __attribute__((ext_vector_type(2))) uint32_t u2;
          hv = Raw<__bf16>::un4(*(const u2*)hp);
        }
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (se * acc[vl][e] + si * hv[e]) * inv;
        if (tg < T) In<Tin>::store4(h + ((size_t)bh * T + tg) * DV + vt0 + 16 * vl + 4 * g, o);
      }
    } else {
      // [C | n] <- e^{m0 - mu_C} [C | n] + e^{A_C - mu_C} K~^T [V | 1]
      const float AC = stA[CM - 1];
      const float muC = fmaxf(mprev, AC);
      const float dI = __expf(AC - muC);
      const float dC = mprev == -INFINITY ? 0.f : __expf(mprev - muC);
#pragma unroll
      for (int i = 0; i < MAXU; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[i][e] *= dC;
      // e^{A_C - mu_C} is folded into the shared [V | 1] operand slices
      const float dv8[8] = {dI, dI, dI, dI, dI, dI, dI, dI};
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        const bool kv = 32 * s + 8 * g < CM;
        Frag<MM> Bv[NVA];
#pragma unroll
        for (int vl = 0; vl < NVA; ++vl) {
          if (vl < NVL) {
            Bv[vl] = sfrag(L::VTS, L::WC, 16 * vl, 32 * s);
            scale_frag<MM>(Bv[vl], dv8);
          } else {
            Bv[vl] = ones_row0<MM>(c16, dI);
          }
          if (!kv) Bv[vl] = ones_row0<MM>(-1);
        }
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          const int jt = uid + NU * jj;
          if (jt < NJB) {
            Frag<MM> A = sfrag(L::KT, L::WC, 16 * jt, 32 * s);
#pragma unroll
            for (int vl = 0; vl < NVA; ++vl) mma<MM>(Sacc[jj * NVA + vl], A, Bv[vl]);
          }
        }
      }
    }
    mprev = stF[CM - 1] + fmaxf(mprev, stA[CM - 1]);
    __syncthreads();
    if (uw) {
#pragma unroll
      for (int i = 0; i < MAXU; ++i) {
        const int jt = uid + NU * (i / NVA), vl = i % NVA;
        if (jt < NJB) st4<SM>(S0T, P_S, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[i]);
      }
    }
  };

  // ---- pipeline: two register sets in turn, loads two chunks ahead of use,
  // one LDS stage written between chunks
  Set X0, X1;
  load(0, X0);
  load(1, X1);
  stage(X0);
  __syncthreads();
  load(2, X0);
  for (int ch = 0; ch < nchunks; ch += 2) {
    compute(ch);
    stage(X1);
    __syncthreads();
    load(ch + 3, X1);
    if (ch + 1 >= nchunks) break;
    compute(ch + 1);
    stage(X0);
    __syncthreads();
    load(ch + 4, X0);
  }

  if (C_out && uw) {
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
      const int jt = uid + NU * (i / NVA), vl = i % NVA;
      if (jt < NJB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * jt + 4 * g + e;
          if (vl < NVL) C_out[(size_t)bh * DK * DV + (size_t)j * DV + vt0 + 16 * vl + c16] = Sacc[i][e];
          else if (c16 == 0 && vt0 == 0) n_out[(size_t)bh * DK + j] = Sacc[i][e];
        }
      }
    }
  }
  if (C_out && tid == 0 && vt0 == 0) m_out[bh] = mprev;
}

// ============================================================================ register scan
// Fragment-form records (bf16, d_k and C multiples of 32). The roles and the
// arithmetic are those of the scan above, but no record byte passes through
// LDS: every operand tile is 1 KiB (H: 512 B) of consecutive bytes in lane
// order, loaded straight into registers with full cache lines. Each wave
// keeps three register sets and refills one as soon as its chunk is done
// with it, so loads run two chunks ahead. Only
// the copy [C | n]^T of the state that q reads goes through LDS, as bf16 hi +
// lo planes (about 16 mantissa bits: the readout's sums can cancel) and
// double buffered: the update waves write the next chunk's copy while the
// readout waves read this chunk's, and one barrier per chunk separates the
// two.
constexpr int kMScanRgSets = 3;

__device__ __forceinline__ void rg_phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}
template <int N> struct RgI { static constexpr int value = N; };

template <int DK, int VT, int CM>
__global__ __launch_bounds__(kMScanThreads, 1) void mlstm_scan_rg_kernel(
    const char* __restrict__ ws, const float* __restrict__ C0,
    const float* __restrict__ n0, const float* __restrict__ m0, __bf16* __restrict__ h, float* C_out,
    float* n_out, float* m_out, int T, int DV) {
  constexpr int NS = kMScanRgSets;
  constexpr int NW = kMScanThreads / 64;
  constexpr int NB = CM / 16, NU = NW - NB;            // readout waves, update waves
  constexpr int NVL = VT / 16, NVA = NVL + 1;           // value tiles + the normaliser tile
  constexpr int KS = DK / 32, KSC = CM / 32;
  constexpr int NJB = DK / 16, JPW = (NJB + NU - 1) / NU;
  constexpr int LDK = DK + 8;                           // row pitch: 16-byte fragment reads conflict free
  constexpr int PL = 16 * NVA * LDK;                    // elements of one plane of the state copy
  static_assert(DK % 32 == 0 && CM % 32 == 0 && NB < NW && NS == 3, "register mLSTM scan shape");
  typedef __attribute__((ext_vector_type(2))) uint32_t u2;
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  // [C | n]^T [v][j]: copy b (chunk parity) plane p (hi, lo) at (2b + p) PL
  extern __shared__ __attribute__((aligned(16))) __bf16 S0T[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int nvt = DV / VT;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int bh = lin / nvt, vt0 = (lin % nvt) * VT;
  const int nchunks = (T + CM - 1) / CM;
  const MRec RL = mrec_layout(DK, DV, CM, 2, true);
  // the records of this head through one buffer resource: the wave-uniform
  // part of every offset is the scalar offset; past the last chunk the loads
  // repeat it
  const char* wsh = ws + (size_t)bh * nchunks * RL.bytes;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wsh), 0, nchunks * RL.bytes, 0x00020000);
  auto cbase = [&](int ch) { return (ch < nchunks ? ch : nchunks - 1) * RL.bytes; };
  auto ld16 = [&](int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, soff, 0));
  };
  auto ld4 = [&](int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wr, voff, soff, 0));
  };
  const int l16 = 16 * lane;
  float mprev = C0 != nullptr ? m0[bh] : -INFINITY;

  // hand-unrolled walk over the register sets with a single exit, so the
  // compiler's wait counts stay exact; leftover chunks after it
  auto walk = [&](auto&& step) {
    int ch = 0;
    for (; ch + 3 <= nchunks; ch += 3) {
      step(ch, RgI<0>{});
      step(ch + 1, RgI<1>{});
      step(ch + 2, RgI<2>{});
    }
    if (ch < nchunks) step(ch, RgI<0>{});
    if (ch + 1 < nchunks) step(ch + 1, RgI<1>{});
  };

  if (wid < NB) {
    // ================= readout: t-block I, every value tile and the normaliser
    const int I = wid;
    struct Set {
      u32x4 q[KS];
      u2 hv[NVL];
      float sA, sN, sF, aC, fC;
    };
    Set R[NS];
    // h rows t0 + 16 I + c16 from chunk ch: rows past T are not written (the
    // row offset is in the lane offset, which the bounds check covers)
    const int lh = (c16 * DV + 4 * g) * 2;
    auto load = [&](int ch, Set& X) {
      const int cb = cbase(ch);
#pragma unroll
      for (int s = 0; s < KS; ++s) X.q[s] = ld16(l16, cb + RL.qf + (I * KS + s) * 1024);
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl)
        X.hv[vl] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(
                                              wr, 8 * lane, cb + RL.hi + (I * (DV / 16) + vt0 / 16 + vl) * 512, 0));
      X.sA = ld4(4 * c16, cb + RL.a + 64 * I);
      X.sN = ld4(4 * c16, cb + RL.ni + 64 * I);
      X.sF = ld4(4 * c16, cb + RL.f + 64 * I);
      X.aC = ld4(0, cb + RL.a + 4 * (CM - 1));
      X.fC = ld4(0, cb + RL.f + 4 * (CM - 1));
    };
    __syncthreads();                                    // first state copy written
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      load(u, R[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      const __bf16* SB = S0T + 2 * (ch & 1) * PL;
      f32x4 acc[NVA];
#pragma unroll
      for (int vl = 0; vl < NVA; ++vl) acc[vl] = f4zero();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 B = __builtin_bit_cast(bf16x8, R[u].q[s]);
#pragma unroll
        for (int vl = 0; vl < NVA; ++vl) {
          const int o = (16 * vl + c16) * LDK + 32 * s + 8 * g;
          acc[vl] = mfma_bf16(*(const bf16x8*)(SB + o), B, acc[vl]);
          acc[vl] = mfma_bf16(*(const bf16x8*)(SB + PL + o), B, acc[vl]);
        }
      }
      // acc[vl][e] = (q_t C0)[v = 16vl + 4g + e] for t = 16I + c16; the
      // normaliser tile's row 0 (lanes g = 0, e = 0) is q_t . n0
      const float At = R[u].sA;
      const float mu = fmaxf(mprev, At);
      const float si = __expf(At - mu);
      const float se = mprev == -INFINITY ? 0.f : __expf(mprev - mu);
      const float nq = __shfl(acc[NVL][0], c16, 64);
      const float nbar = se * nq + si * R[u].sN;
      const float inv = 1.f / fmaxf(fabsf(nbar), __expf(-(R[u].sF + mu)));
      const int t0 = ch * CM;
      const __amdgpu_buffer_rsrc_t hr =
          __builtin_amdgcn_make_buffer_rsrc(h + ((size_t)bh * T + t0) * DV, 0, (T - t0) * DV * 2, 0x00020000);
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl) {
        const f32x4 hv = Raw<__bf16>::un4(R[u].hv[vl]);
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)((se * acc[vl][e] + si * hv[e]) * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, o), hr, lh + (16 * I * DV + vt0 + 16 * vl) * 2,
                                              0, 0);
      }
      mprev = R[u].fC + fmaxf(mprev, R[u].aC);
      load(ch + NS, R[u]);
      rg_phase_barrier();
    });
  } else {
    // ================= state update: j-blocks uid, uid + NU, .. of every value tile
    const int uid = wid - NB;
    struct Set {
      u32x4 k[JPW][KSC], v[NVL][KSC];
      float aC, fC;
    };
    Set U[NS];
    auto load = [&](int ch, Set& X) {
      const int cb = cbase(ch);
      // every wave issues the same loads on every path (a wave with fewer
      // j-blocks repeats its last one and never uses it): with a branch here
      // the compiler could not count the loads in flight and would wait for
      // all of them at the next use
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int jt = uid + NU * jj < NJB ? uid + NU * jj : NJB - 1;
#pragma unroll
        for (int s = 0; s < KSC; ++s) X.k[jj][s] = ld16(l16, cb + RL.kt + (jt * KSC + s) * 1024);
      }
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl)
#pragma unroll
        for (int s = 0; s < KSC; ++s) X.v[vl][s] = ld16(l16, cb + RL.vt + ((vt0 / 16 + vl) * KSC + s) * 1024);
      X.aC = ld4(0, cb + RL.a + 4 * (CM - 1));
      X.fC = ld4(0, cb + RL.f + 4 * (CM - 1));
    };
    f32x4 Sacc[JPW][NVA];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jt = uid + NU * jj;
#pragma unroll
      for (int vl = 0; vl < NVA; ++vl) {
        Sacc[jj][vl] = f4zero();
        if (jt < NJB) {
          if (C0 != nullptr) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = 16 * jt + 4 * g + e;
              if (vl < NVL) Sacc[jj][vl][e] = C0[(size_t)bh * DK * DV + (size_t)j * DV + vt0 + 16 * vl + c16];
              else Sacc[jj][vl][e] = c16 == 0 ? n0[(size_t)bh * DK + j] : 0.f;
            }
          }
          st4<kSP>((char*)S0T, PL * 2, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[jj][vl]);
        }
      }
    }
    __syncthreads();                                    // first state copy written
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      load(u, U[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The set the previous chunk used is refilled (for chunk ch + NS - 1) at
    // the start of each chunk, its loads interleaved with the products below:
    // issued in one burst, they wait for the load queue at the end of the
    // chunk, on the way to the barrier.
    constexpr int NLU = JPW * KSC + NVL * KSC + 2;
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      load(ch + NS - 1, U[(u + NS - 1) % NS]);
      // [C | n] <- e^{m0 - mu_C} [C | n] + e^{A_C - mu_C} K~^T [V | 1]
      const float AC = U[u].aC;
      const float muC = fmaxf(mprev, AC);
      const float dI = __expf(AC - muC);
      const float dC = mprev == -INFINITY ? 0.f : __expf(mprev - muC);
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int vl = 0; vl < NVA; ++vl)
#pragma unroll
          for (int e = 0; e < 4; ++e) Sacc[jj][vl][e] *= dC;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        bf16x8 Bv[NVA];
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl) {
          const bf16x8 x = __builtin_bit_cast(bf16x8, U[u].v[vl][s]);
#pragma unroll
          for (int e = 0; e < 8; ++e) Bv[vl][e] = (__bf16)((float)x[e] * dI);
        }
        const __bf16 one = (__bf16)(c16 == 0 ? dI : 0.f);
#pragma unroll
        for (int e = 0; e < 8; ++e) Bv[NVL][e] = one;
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          if (uid + NU * jj < NJB) {
            const bf16x8 A = __builtin_bit_cast(bf16x8, U[u].k[jj][s]);
#pragma unroll
            for (int vl = 0; vl < NVA; ++vl) Sacc[jj][vl] = mfma_bf16(A, Bv[vl], Sacc[jj][vl]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NLU; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one buffer load
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      }
      __bf16* SN = S0T + 2 * ((ch + 1) & 1) * PL;
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int jt = uid + NU * jj;
        if (jt < NJB) {
#pragma unroll
          for (int vl = 0; vl < NVA; ++vl)
            st4<kSP>((char*)SN, PL * 2, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[jj][vl]);
        }
      }
      mprev = U[u].fC + fmaxf(mprev, AC);
      rg_phase_barrier();
    });
    if (C_out) {
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int jt = uid + NU * jj;
        if (jt < NJB) {
#pragma unroll
          for (int vl = 0; vl < NVA; ++vl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = 16 * jt + 4 * g + e;
              if (vl < NVL) C_out[(size_t)bh * DK * DV + (size_t)j * DV + vt0 + 16 * vl + c16] = Sacc[jj][vl][e];
              else if (c16 == 0 && vt0 == 0) n_out[(size_t)bh * DK + j] = Sacc[jj][vl][e];
            }
        }
      }
      if (uid == 0 && lane == 0 && vt0 == 0) m_out[bh] = mprev;
    }
  }
}

// ============================================================================ segmented wide scan
// The register scan with 64 value columns per workgroup (a quarter of the
// record bytes per column: q and K~^T are shared by every column of a
// workgroup) and the chunks of a head cut into segments, so that few heads
// still give a workgroup per CU.
//
// The chunk map of the mLSTM is scalar-decay affine: over a segment g whose
// log-forget gates sum to F_g, a start (C, n, m) goes to
//   m' = max(m + F_g, mQ),   [C | n]' = e^{m + F_g - m'} [C | n] + e^{mQ - m'} [Q | nQ],
// where (Q, nQ, mQ) is the segment's own end state from a zero start
// (m = -inf): the page's stabiliser recurrence m_t = max(log f_t + m_{t-1}, i~_t)
// unrolls to the same maximum either way. The chunks of a head are cut into a
// short first segment and P segments of L chunks, and two launches of P
// workgroups per (head, 64-column tile) run them:
//   phase 0: segment 0 scanned from (C0, n0, m0) (h stored, its end state kept
//            for the others) beside the maps of segments 1 .. P-1 (state
//            only, from a zero start); segment 0 needs no map, and its length
//            is chosen so it takes about as long as a map pass over L chunks;
//   phase 1: segments 1 .. P scanned, each from segment 0's end state with the
//            maps of the segments between applied in its prologue; the last
//            one writes (C, n, m)_T.
// C0 is read only in phase 0 and C_out written only in phase 1, so C_out may
// be C0.
// The normaliser n is fp32 throughout (no extra MFMA tile): the update waves
// accumulate K~^T against a bf16(e^{A_C - mu_C}) operand and the readout waves
// form q_t . n0 from their q fragments. The V tile of a chunk is loaded once
// per workgroup and passed to all update waves through LDS.
constexpr int kMSegTargetUnits = 256;   // workgroups the segmented scan aims for (one per CU)
constexpr int kMWideVT = 64;

template <int DK, int CM>
struct MWideSmem {
  static constexpr int NVL = kMWideVT / 16, KSC = CM / 32;
  static constexpr int LDK = DK + 8;
  static constexpr int PL = 16 * NVL * LDK;              // bf16 elements of one plane of the state copy
  static constexpr int S0T = 0;                          // [buffer][plane] state copy [v][j]
  static constexpr int NL = S0T + 4 * PL * 2;            // [buffer] n fp32 [j]
  static constexpr int VS = NL + 2 * DK * 4;             // [buffer] V tile operand slices, 1 KiB each
  static constexpr int VSTAGE = NVL * KSC * 1024;
  static constexpr int TOTAL = VS + 2 * VSTAGE;
  static_assert(TOTAL <= 160 * 1024, "wide mLSTM scan LDS exceeds 160 KiB");
};

// One (head, segment, 64-column tile): chunks c0 .. c0 + nchunks - 1 of head
// bh. Start (Cs, ns, ms) indexed by head (NULL: zero state, m = -inf), then
// the first nmaps maps (slots m * BH + bh of Qmap, nQ, mF) applied in order.
// MAP: state only, the end state, its stabiliser and the summed log-forget
// to (Qo, nQo, mFo); otherwise h stored and the end state to (Cend, nend,
// mend) (indexed by head) unless Cend is NULL.
template <int DK, int CM, bool MAP>
__device__ __forceinline__ void mlstm_wide_body(
    char* smem, const char* __restrict__ ws, int bh, int BH, int ntot, int c0, int nchunks, int vt0,
    const float* __restrict__ Cs, const float* __restrict__ ns, const float* __restrict__ ms, int nmaps,
    const float* __restrict__ Qmap, const float* __restrict__ nQ, const float* __restrict__ mF,
    __bf16* __restrict__ h, float* Cend, float* nend, float* mend, float* Qo, float* nQo, float* mFo, int T, int DV,
    const __bf16* __restrict__ qin) {
  using L = MWideSmem<DK, CM>;
  constexpr int NS = kMScanRgSets;
  constexpr int NW = kMScanThreads / 64;
  constexpr int NB = CM / 16, NU = NW - NB;             // readout waves, update waves
  constexpr int NVL = L::NVL;
  constexpr int KS = DK / 32, KSC = L::KSC;
  constexpr int NJB = DK / 16, JPW = (NJB + NU - 1) / NU;
  constexpr int LDK = L::LDK, PL = L::PL;
  constexpr int NVT = NVL * KSC, VPW = NVT / NB;        // V slices per chunk, per readout wave
  // every update wave holds JPW whole j-blocks: no branch in its chunk loop
  // (a branch there leaves the compiler waiting for every load in flight at
  // the loop's back edge)
  static_assert(DK % 64 == 0 && CM == 64 && NB < NW && NS == 3 && NVT % NB == 0 && NJB % NU == 0,
                "wide mLSTM scan shape");
  typedef __attribute__((ext_vector_type(2))) uint32_t u2;
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  __bf16* S0T = (__bf16*)(smem + L::S0T);
  float* NLs = (float*)(smem + L::NL);
  char* VS = smem + L::VS;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const MRec RL = mrec_layout(DK, DV, CM, 2, true);
  const char* wsh = ws + ((size_t)bh * ntot + c0) * RL.bytes;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wsh), 0, nchunks * RL.bytes, 0x00020000);
  auto cbase = [&](int ch) { return (ch < nchunks ? ch : nchunks - 1) * RL.bytes; };
  auto ld16 = [&](int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, soff, 0));
  };
  auto ld4 = [&](int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wr, voff, soff, 0));
  };
  const int l16 = 16 * lane;
  // the stabiliser this segment starts from: ms (or -inf), then each map
  float mprev = -INFINITY;
  if constexpr (!MAP) {
    if (Cs != nullptr) mprev = ms[bh];
    for (int gq = 0; gq < nmaps; ++gq) {
      const size_t sl = (size_t)gq * BH + bh;
      mprev = fmaxf(mprev + mF[2 * sl + 1], mF[2 * sl]);
    }
  }

  auto walk = [&](auto&& step) {
    int ch = 0;
    for (; ch + 3 <= nchunks; ch += 3) {
      step(ch, RgI<0>{});
      step(ch + 1, RgI<1>{});
      step(ch + 2, RgI<2>{});
    }
    if (ch < nchunks) step(ch, RgI<0>{});
    if (ch + 1 < nchunks) step(ch + 1, RgI<1>{});
  };

  // V tile of a chunk: slices p = VPW I .. VPW I + VPW - 1 (vl = p / KSC,
  // s = p % KSC) are loaded by readout wave I and staged in LDS a chunk
  // ahead, already scaled by the chunk's e^{A_C - mu_C} (once per workgroup,
  // not once per update wave), and read by every update wave
  auto stage_v = [&](const u32x4* X, int I, int buf, float dI) {
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, X[i]);
      bf16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (__bf16)((float)x[e] * dI);
      *(bf16x8*)(VS + buf * L::VSTAGE + (VPW * I + i) * 1024 + l16) = y;
    }
  };
  // e^{A_C - mu_C} of a chunk whose A_C is aC, entered with stabiliser m
  auto write_scale = [](float m, float aC) { return __expf(aC - fmaxf(m, aC)); };

  if (wid < NB) {
    // ================= readout: t-block I, 64 value columns (MAP: V tile only)
    const int I = wid;
    struct Set {
      u32x4 q[MAP ? 1 : KS];
      u2 hv[NVL];
      u32x4 v[VPW];
      float sA, sN, sF, aC, fC;
    };
    Set R[NS];
    const int lh = (c16 * DV + 4 * g) * 2;
    // q of this head from the segment's first row to row T, straight from the
    // input (rows past T read as zero): lane l of t-block I reads row
    // 16 I + l % 16, columns 32 s + 8 (l / 16) .. +7, the B operand of the
    // readout's 16x16x32 MFMA
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(qin) + ((size_t)bh * T + (size_t)c0 * CM) * DK, 0, (T - c0 * CM) * DK * 2, 0x00020000);
    const int lq = ((16 * I + c16) * DK + 8 * g) * 2;
    auto load = [&](int ch, Set& X) {
      const int cb = cbase(ch);
#pragma unroll
      for (int i = 0; i < VPW; ++i) {
        const int p = VPW * I + i;
        X.v[i] = ld16(l16, cb + RL.vt + ((vt0 / 16 + p / KSC) * KSC + p % KSC) * 1024);
      }
      X.aC = ld4(0, cb + RL.a + 4 * (CM - 1));
      X.fC = ld4(0, cb + RL.f + 4 * (CM - 1));
      if constexpr (!MAP) {
        const int qb = (ch < nchunks ? ch : nchunks - 1) * CM * DK * 2;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          X.q[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, lq, qb + 64 * s, 0));
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl)
          X.hv[vl] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(
                                                wr, 8 * lane, cb + RL.hi + (I * (DV / 16) + vt0 / 16 + vl) * 512, 0));
        X.sA = ld4(4 * c16, cb + RL.a + 64 * I);
        X.sN = ld4(4 * c16, cb + RL.ni + 64 * I);
        X.sF = ld4(4 * c16, cb + RL.f + 64 * I);
      }
    };
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      load(u, R[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage_v(R[0].v, I, 0, write_scale(mprev, R[0].aC));
    __syncthreads();                                    // first state copy and V tile written
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      if constexpr (!MAP) {
        const __bf16* SB = S0T + 2 * (ch & 1) * PL;
        const float* Nb = NLs + (ch & 1) * DK;
        f32x4 acc[NVL];
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl) acc[vl] = f4zero();
        float qn = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 B = __builtin_bit_cast(bf16x8, R[u].q[s]);
          // hi planes of the four tiles, then the lo planes: no MFMA waits on
          // the one just issued
          bf16x8 Fh[NVL], Fl[NVL];
#pragma unroll
          for (int vl = 0; vl < NVL; ++vl) {
            const int o = (16 * vl + c16) * LDK + 32 * s + 8 * g;
            Fh[vl] = *(const bf16x8*)(SB + o);
            Fl[vl] = *(const bf16x8*)(SB + PL + o);
          }
#pragma unroll
          for (int vl = 0; vl < NVL; ++vl) acc[vl] = mfma_bf16(Fh[vl], B, acc[vl]);
#pragma unroll
          for (int vl = 0; vl < NVL; ++vl) acc[vl] = mfma_bf16(Fl[vl], B, acc[vl]);
          // q_t . n0 over this lane's 8 k of the slice
          const f32x4 na = *(const f32x4*)(Nb + 32 * s + 8 * g);
          const f32x4 nb = *(const f32x4*)(Nb + 32 * s + 8 * g + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) qn += (float)B[e] * na[e] + (float)B[4 + e] * nb[e];
        }
        qn += __shfl_xor(qn, 16, 64);
        qn += __shfl_xor(qn, 32, 64);
        // acc[vl][e] = (q_t C0)[v = vt0 + 16vl + 4g + e], t = 16I + c16; qn = q_t . n0
        const float At = R[u].sA;
        const float mu = fmaxf(mprev, At);
        const float si = __expf(At - mu);
        const float se = mprev == -INFINITY ? 0.f : __expf(mprev - mu);
        const float nbar = se * qn + si * R[u].sN;
        const float inv = 1.f / fmaxf(fabsf(nbar), __expf(-(R[u].sF + mu)));
        const int t0 = (c0 + ch) * CM;
        const __amdgpu_buffer_rsrc_t hr =
            __builtin_amdgcn_make_buffer_rsrc(h + ((size_t)bh * T + t0) * DV, 0, (T - t0) * DV * 2, 0x00020000);
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl) {
          const f32x4 hv = Raw<__bf16>::un4(R[u].hv[vl]);
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)((se * acc[vl][e] + si * hv[e]) * inv);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, o), hr, lh + (16 * I * DV + vt0 + 16 * vl) * 2,
                                                0, 0);
        }
      }
      mprev = R[u].fC + fmaxf(mprev, R[u].aC);
      // the next chunk's V tile (loaded two chunks ago), then this set refilled
      stage_v(R[(u + 1) % NS].v, I, (ch + 1) & 1, write_scale(mprev, R[(u + 1) % NS].aC));
      load(ch + NS, R[u]);
      rg_phase_barrier();
    });
  } else {
    // ================= state update: j-blocks uid, uid + NU, .. of the 64 columns
    const int uid = wid - NB;
    struct Set {
      u32x4 k[JPW][KSC];
      float aC, fC;
    };
    Set U[NS];
    auto load = [&](int ch, Set& X) {
      const int cb = cbase(ch);
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int jt = uid + NU * jj;
#pragma unroll
        for (int s = 0; s < KSC; ++s) X.k[jj][s] = ld16(l16, cb + RL.kt + (jt * KSC + s) * 1024);
      }
      X.aC = ld4(0, cb + RL.a + 4 * (CM - 1));
      X.fC = ld4(0, cb + RL.f + 4 * (CM - 1));
    };
    // state: Sacc[jj][vl][e] = C[j = 16 jt + 4g + e][v = vt0 + 16 vl + c16];
    // nr[jj][e] = n[j = 16 jt + 4g + e] (the same in all 16 columns)
    f32x4 Sacc[JPW][NVL], nr[JPW];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      nr[jj] = f4zero();
#pragma unroll
      for (int vl = 0; vl < NVL; ++vl) Sacc[jj][vl] = f4zero();
    }
    // element (jj, vl, e) of a [dk][dv] array / element (jj, e) of a [dk] one
    auto cidx = [&](int jj, int vl, int e) { return (size_t)(16 * (uid + NU * jj) + 4 * g + e) * DV + vt0 + 16 * vl + c16; };
    auto nidx = [&](int jj) { return 16 * (uid + NU * jj) + 4 * g; };
    if constexpr (!MAP) {
      if (Cs != nullptr) {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          nr[jj] = *(const f32x4*)(ns + (size_t)bh * DK + nidx(jj));
#pragma unroll
          for (int vl = 0; vl < NVL; ++vl)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[jj][vl][e] = Cs[(size_t)bh * DK * DV + cidx(jj, vl, e)];
        }
      }
      // the maps of the segments before this one, in order
      float mcur = Cs != nullptr ? ms[bh] : -INFINITY;
      for (int gq = 0; gq < nmaps; ++gq) {
        const size_t sl = (size_t)gq * BH + bh;
        const float mQ = mF[2 * sl], me = fmaxf(mcur + mF[2 * sl + 1], mQ);
        const float a = __expf(mcur + mF[2 * sl + 1] - me), b = __expf(mQ - me);
        const float* Qs = Qmap + sl * DK * DV;
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          const f32x4 nq = *(const f32x4*)(nQ + sl * DK + nidx(jj));
#pragma unroll
          for (int e = 0; e < 4; ++e) nr[jj][e] = a * nr[jj][e] + b * nq[e];
#pragma unroll
          for (int vl = 0; vl < NVL; ++vl)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[jj][vl][e] = a * Sacc[jj][vl][e] + b * Qs[cidx(jj, vl, e)];
        }
        mcur = me;
      }
    }
    auto put_state = [&](int buf) {
      if constexpr (!MAP) {
        __bf16* SN = S0T + 2 * buf * PL;
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          const int jt = uid + NU * jj;
#pragma unroll
          for (int vl = 0; vl < NVL; ++vl)
            st4<kSP>((char*)SN, PL * 2, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[jj][vl]);
          if (c16 == 0) *(f32x4*)(NLs + buf * DK + 16 * jt + 4 * g) = nr[jj];
        }
      }
    };
    put_state(0);
    __syncthreads();                                    // first state copy and V tile written
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      load(u, U[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // L2 warm-up: the workgroups of a segment touch the record's 128-byte
    // lines that this launch reads (H, V^T, K~^T; MAP: V^T and K~^T), one dword per
    // lane of every update wave, kPF chunks ahead, so that their loads hit L2
    // (each line is read by every workgroup of the segment). The values are
    // folded into `sink` three chunks later, which keeps the loads alive
    // without waiting for them early.
    constexpr int kPF = 5;
    constexpr bool kTouch = !MAP;   // the map pass reads less and ran slower with them
    const int tb = MAP ? RL.vt : 0;
    const int nlines = ((MAP ? RL.qf - RL.vt : RL.qf) + 127) / 128;
    const int pl = ((vt0 / kMWideVT) * NU + uid) * 64 + lane;
    const int v_pf = tb + (pl < nlines ? pl : nlines - 1) * 128;
    auto touch = [&](int ch) { return __builtin_amdgcn_raw_buffer_load_b32(wr, v_pf, cbase(ch), 0); };
    uint32_t sink = 0, PFV[3] = {0u, 0u, 0u};
    if constexpr (kTouch) {
#pragma unroll
      for (int u = 0; u < 3; ++u) PFV[u] = touch(kPF - 3 + u);
    }
    float Fsum = 0.f;
    constexpr int NLU = JPW * KSC + 2;
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      // the touch first: issued after this set's loads, the compiler would
      // wait for every load in flight at the loop's back edge
      if constexpr (kTouch) {
        sink ^= PFV[u];
        PFV[u] = touch(ch + kPF);
      }
      load(ch + NS - 1, U[(u + NS - 1) % NS]);
      // [C | n] <- e^{m0 - mu_C} [C | n] + e^{A_C - mu_C} K~^T [V | 1]
      const float AC = U[u].aC;
      const float muC = fmaxf(mprev, AC);
      const float dI = __expf(AC - muC);
      const float dC = mprev == -INFINITY ? 0.f : __expf(mprev - muC);
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl)
#pragma unroll
          for (int e = 0; e < 4; ++e) Sacc[jj][vl][e] *= dC;
      // V arrives scaled by dI; n takes the row sums of K~^T on the matrix
      // cores against an operand holding bf16(dI) in every entry (as the
      // scaled V it is rounded to bf16)
      const char* Vb = VS + (ch & 1) * L::VSTAGE;
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) nr[jj][e] *= dC;
      bf16x8 ones;
#pragma unroll
      for (int e = 0; e < 8; ++e) ones[e] = (__bf16)dI;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl) {
          const bf16x8 Bv = *(const bf16x8*)(Vb + (vl * KSC + s) * 1024 + l16);
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            Sacc[jj][vl] = mfma_bf16(__builtin_bit_cast(bf16x8, U[u].k[jj][s]), Bv, Sacc[jj][vl]);
        }
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) nr[jj] = mfma_bf16(__builtin_bit_cast(bf16x8, U[u].k[jj][s]), ones, nr[jj]);
      }
#pragma unroll
      for (int i = 0; i < NLU; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one buffer load
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      }
      put_state((ch + 1) & 1);
      mprev = U[u].fC + fmaxf(mprev, AC);
      Fsum += U[u].fC;
      rg_phase_barrier();
    });
    if constexpr (kTouch) {
#pragma unroll
      for (int u = 0; u < 3; ++u) sink ^= PFV[u];
    }
    if (sink == 0x7fc00001u && T < 0) h[0] = (__bf16)0.f;   // never true (T > 0): keeps the touches alive
    if constexpr (MAP) {
      // this segment's end state from a zero start, its stabiliser and F_g
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int jt = uid + NU * jj;
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Qo[(size_t)(16 * jt + 4 * g + e) * DV + vt0 + 16 * vl + c16] = Sacc[jj][vl][e];
        if (c16 == 0 && vt0 == 0) *(f32x4*)(nQo + 16 * jt + 4 * g) = nr[jj];
      }
      if (uid == 0 && lane == 0 && vt0 == 0) {
        mFo[0] = mprev;
        mFo[1] = Fsum;
      }
    } else if (Cend != nullptr) {
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int jt = uid + NU * jj;
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Cend[(size_t)bh * DK * DV + (size_t)(16 * jt + 4 * g + e) * DV + vt0 + 16 * vl + c16] = Sacc[jj][vl][e];
        if (c16 == 0 && vt0 == 0) *(f32x4*)(nend + (size_t)bh * DK + 16 * jt + 4 * g) = nr[jj];
      }
      if (uid == 0 && lane == 0 && vt0 == 0) mend[bh] = mprev;
    }
  }
}

// The two launches of the segmented wide scan (PHASE 0 and 1, see above):
// grid B*H * P * (d_v / 64) workgroups; segment 0 has L0 chunks, segments
// 1 .. P have L (the last one possibly fewer). E0 holds segment 0's end state:
// [B*H][dk][dv], then [B*H][dk], then [B*H].
template <int DK, int CM, int PHASE>
__global__ __launch_bounds__(kMScanThreads, 1) void mlstm_scan_wide_kernel(
    const char* __restrict__ ws, const float* __restrict__ C0, const float* __restrict__ n0,
    const float* __restrict__ m0, __bf16* __restrict__ h, float* C_out, float* n_out, float* m_out, int T, int DV,
    int L0, int L, float* __restrict__ Qmap, float* __restrict__ nQ, float* __restrict__ mF, float* __restrict__ E0,
    const __bf16* __restrict__ qin) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nvt = DV / kMWideVT;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int ntot = (T + CM - 1) / CM;
  const int P = (ntot - L0 + L - 1) / L;               // segments after the first
  const int unit = lin / nvt, vt0 = (lin % nvt) * kMWideVT;
  const int bh = unit / P, sl = unit % P;
  const int BH = gridDim.x / (nvt * P);
  float* E0C = E0;
  float* E0n = E0 + (size_t)BH * DK * DV;
  float* E0m = E0n + (size_t)BH * DK;
  if constexpr (PHASE == 0) {
    if (sl == 0) {
      mlstm_wide_body<DK, CM, false>(smem, ws, bh, BH, ntot, 0, L0, vt0, C0, n0, m0, 0, Qmap, nQ, mF, h, E0C, E0n,
                                     E0m, nullptr, nullptr, nullptr, T, DV, qin);
    } else {
      const int c0 = L0 + (sl - 1) * L;
      const size_t slot = (size_t)(sl - 1) * BH + bh;
      mlstm_wide_body<DK, CM, true>(smem, ws, bh, BH, ntot, c0, ntot - c0 < L ? ntot - c0 : L, vt0, nullptr,
                                    nullptr, nullptr, 0, Qmap, nQ, mF, h, nullptr, nullptr, nullptr,
                                    Qmap + slot * DK * DV, nQ + slot * DK, mF + 2 * slot, T, DV, qin);
    }
  } else {
    // segment sl + 1 from segment 0's end state and the maps of segments 1 .. sl
    const int c0 = L0 + sl * L;
    const bool last = sl == P - 1;
    mlstm_wide_body<DK, CM, false>(smem, ws, bh, BH, ntot, c0, ntot - c0 < L ? ntot - c0 : L, vt0, E0C, E0n, E0m,
                                   sl, Qmap, nQ, mF, h, last ? C_out : nullptr, last ? n_out : nullptr,
                                   last ? m_out : nullptr, nullptr, nullptr, nullptr, T, DV, qin);
  }
}

// ------------------------------------------------------------------ host launch
// The segmented wide scan's plan from the shapes alone: P segments of L
// chunks after a first segment of L0, or false where the register scan is
// used (enough workgroups without segments, short sequences, or shapes the
// wide scan does not take). P workgroups per (head, tile) in each launch; the
// first segment, scanned beside the maps, is about a third of the others
// (a map pass over a chunk costs about a third of a scan step).
static bool mseg_plan(int B, int H, int T, int dk, int dv, int chunk, int dtype, int* L0, int* L) {
  if (!mlstm_fm(dtype, dk, dv, chunk, T) || chunk != 64 || dk % 64 != 0 || dv % kMWideVT != 0) return false;
  const long long units = (long long)B * H * (dv / kMWideVT);
  const int ntot = (T + chunk - 1) / chunk;
  if (units * 2 > kMSegTargetUnits || ntot < 32) return false;
  int P = (int)(kMSegTargetUnits / units);
  if (P > ntot / 12) P = ntot / 12;                  // segments of about 12 chunks or more
  int l = (3 * ntot + 3 * P) / (3 * P + 1);          // ceil(3 ntot / (3P + 1))
  int l0 = ntot - P * l;
  if (l0 < 1) {
    l = (ntot - 1) / P;
    l0 = ntot - P * l;
  }
  *L0 = l0;
  *L = l;
  return true;
}

static size_t mrecords_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  const int es = dtype == GDR_BF16 ? 2 : 4;
  const size_t nchunks = ((size_t)T + chunk - 1) / chunk;
  return (size_t)B * H * nchunks * (size_t)mrec_layout(dk, dv, chunk, es, mlstm_fm(dtype, dk, dv, chunk, T)).bytes;
}

// Buffers of the segmented scan after the records (fp32): maps [P-1][BH] of
// [dk][dv], [dk] and (mQ, F); segment 0's end state: [BH][dk][dv], [BH][dk],
// [BH].
struct MSegBufs {
  float *Q, *nQ, *mF, *E0;
  size_t bytes;
};
static MSegBufs mseg_bufs(char* base, int BH, int dk, int dv, int P) {
  MSegBufs b;
  const size_t nm = (size_t)(P - 1) * BH;
  float* p = (float*)base;
  b.Q = p;   p += nm * dk * dv;
  b.nQ = p;  p += nm * dk;
  b.mF = p;  p += (2 * nm + 3) / 4 * 4;                 // padded: E0's n part takes 16-byte accesses
  b.E0 = p;  p += (size_t)BH * (dk * dv + dk + 1);
  b.bytes = (size_t)((char*)p - base);
  return b;
}

size_t mlstm_ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  size_t n = mrecords_bytes(B, H, T, dk, dv, chunk, dtype);
  int L0, L;
  if (mseg_plan(B, H, T, dk, dv, chunk, dtype, &L0, &L)) {
    const int ntot = (T + chunk - 1) / chunk, P = (ntot - L0 + L - 1) / L;
    n = (n + 255) / 256 * 256 + mseg_bufs(nullptr, B * H, dk, dv, P).bytes;
  }
  return n;
}

template <typename Tin, int DK, int CM, bool FM, bool QC = true>
static int launch_mintra(const MlstmArgs& a, char* ws) {
  using L = MIntraSmem<Tin, DK, CM>;
  auto kern = mlstm_intra_kernel<Tin, DK, CM, FM, QC>;
  if (!allow_lds((const void*)kern, L::TOTAL)) return GDR_ERR_LAUNCH;
  int nchunks = (a.T + CM - 1) / CM;
  int nitems = a.B * a.H * nchunks;
  const int cus = stream_cus(a.stream);
  const int grid = nitems < cus ? nitems : cus;
  const Tin *q = (const Tin*)a.q, *k = (const Tin*)a.k, *v = (const Tin*)a.v;
  const float *it = a.i_tilde, *ft = a.f_tilde;
  int T = a.T, DV = a.dv;
  void* args[] = {&q, &k, &v, &it, &ft, &ws, &T, &DV, &nchunks, &nitems};
  hipError_t e = hipLaunchKernel((const void*)kern, dim3(grid), dim3(kMThreads), args, L::TOTAL,
                                 (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

template <typename Tin, int DK, int VT, int CM>
static int launch_mscan(const MlstmArgs& a, const char* ws) {
  using L = MScanSmem<Tin, DK, VT, CM>;
  auto kern = mlstm_scan_kernel<Tin, DK, VT, CM>;
  if (!allow_lds((const void*)kern, L::TOTAL)) return GDR_ERR_LAUNCH;
  const int nblocks = a.B * a.H * (a.dv / VT);
  const Tin* q = (const Tin*)a.q;
  const float *C0 = a.C0, *n0 = a.n0, *m0 = a.m0;
  Tin* h = (Tin*)a.h;
  float *Co = a.C_out, *no = a.n_out, *mo = a.m_out;
  int T = a.T, DV = a.dv;
  void* args[] = {&q, &ws, &C0, &n0, &m0, &h, &Co, &no, &mo, &T, &DV};
  hipError_t e = hipLaunchKernel((const void*)kern, dim3(nblocks), dim3(kMScanThreads), args, L::TOTAL,
                                 (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

template <int DK, int VT, int CM>
static int launch_mscan_rg(const MlstmArgs& a, const char* ws) {
  auto kern = mlstm_scan_rg_kernel<DK, VT, CM>;
  constexpr int lds = 4 * 16 * (VT / 16 + 1) * (DK + 8) * 2;   // two copies x two planes
  static_assert(lds <= 160 * 1024, "register mLSTM scan LDS exceeds 160 KiB");
  if (!allow_lds((const void*)kern, lds)) return GDR_ERR_LAUNCH;
  const int nblocks = a.B * a.H * (a.dv / VT);
  const float *C0 = a.C0, *n0 = a.n0, *m0 = a.m0;
  __bf16* h = (__bf16*)a.h;
  float *Co = a.C_out, *no = a.n_out, *mo = a.m_out;
  int T = a.T, DV = a.dv;
  void* args[] = {&ws, &C0, &n0, &m0, &h, &Co, &no, &mo, &T, &DV};
  hipError_t e = hipLaunchKernel((const void*)kern, dim3(nblocks), dim3(kMScanThreads), args, lds,
                                 (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

// Segmented wide scan: phase 0 (segment 0 and the maps), then phase 1.
template <int DK, int CM>
static int launch_mscan_wide(const MlstmArgs& a, char* ws, int L0, int L) {
  using L_ = MWideSmem<DK, CM>;
  auto k0 = mlstm_scan_wide_kernel<DK, CM, 0>;
  auto k1 = mlstm_scan_wide_kernel<DK, CM, 1>;
  if (!allow_lds((const void*)k0, L_::TOTAL) || !allow_lds((const void*)k1, L_::TOTAL)) return GDR_ERR_LAUNCH;
  const int BH = a.B * a.H, nvt = a.dv / kMWideVT;
  const int ntot = (a.T + CM - 1) / CM, P = (ntot - L0 + L - 1) / L;
  const size_t rec = (mrecords_bytes(a.B, a.H, a.T, DK, a.dv, CM, GDR_BF16) + 255) / 256 * 256;
  const MSegBufs sb = mseg_bufs(ws + rec, BH, DK, a.dv, P);
  hipStream_t st = (hipStream_t)a.stream;
  const char* wsc = ws;
  const float *C0 = a.C0, *n0 = a.n0, *m0 = a.m0;
  __bf16* h = (__bf16*)a.h;
  float *Co = a.C_out, *no = a.n_out, *mo = a.m_out;
  float *Q = sb.Q, *nQ = sb.nQ, *mF = sb.mF, *E0 = sb.E0;
  int T = a.T, DV = a.dv;
  const __bf16* qin = (const __bf16*)a.q;
  void* args[] = {&wsc, &C0, &n0, &m0, &h, &Co, &no, &mo, &T, &DV, &L0, &L, &Q, &nQ, &mF, &E0, &qin};
  const dim3 grid(BH * P * nvt);
  if (hipLaunchKernel((const void*)k0, grid, dim3(kMScanThreads), args, L_::TOTAL, st) != hipSuccess)
    return GDR_ERR_LAUNCH;
  if (hipLaunchKernel((const void*)k1, grid, dim3(kMScanThreads), args, L_::TOTAL, st) != hipSuccess)
    return GDR_ERR_LAUNCH;
  return GDR_OK;
}

template <typename Tin, int DK, int CM>
static int mlstm_pair(const MlstmArgs& a, char* ws) {
  // value tiles of 32 columns when that still gives a workgroup per CU, else 16
  const bool wide = a.dv >= 32 && (long long)a.B * a.H * (a.dv / 32) >= stream_cus(a.stream);
  if constexpr (std::is_same<Tin, __bf16>::value && DK % 32 == 0 && CM % 32 == 0) {
    if (mlstm_fm(a.dtype, DK, a.dv, CM, a.T)) {
      if constexpr (CM == 64 && DK % 64 == 0) {
        int L0, L;
        if (mseg_plan(a.B, a.H, a.T, DK, a.dv, CM, a.dtype, &L0, &L)) {
          const int st = launch_mintra<Tin, DK, CM, true, false>(a, ws);
          if (st != GDR_OK) return st;
          return launch_mscan_wide<DK, CM>(a, ws, L0, L);
        }
      }
      const int st = launch_mintra<Tin, DK, CM, true>(a, ws);
      if (st != GDR_OK) return st;
      if (!wide) return launch_mscan_rg<DK, 16, CM>(a, ws);
      return launch_mscan_rg<DK, 32, CM>(a, ws);
    }
  }
  const int st = launch_mintra<Tin, DK, CM, false>(a, ws);
  if (st != GDR_OK) return st;
  if (!wide) return launch_mscan<Tin, DK, 16, CM>(a, ws);
  return launch_mscan<Tin, DK, 32, CM>(a, ws);
}

template <typename Tin, int CM>
static int mlstm_ws_dk(const MlstmArgs& a, char* ws) {
  switch (a.dk) {
    case 16: return mlstm_pair<Tin, 16, CM>(a, ws);
    case 32: return mlstm_pair<Tin, 32, CM>(a, ws);
    case 64: return mlstm_pair<Tin, 64, CM>(a, ws);
    case 128: return mlstm_pair<Tin, 128, CM>(a, ws);
    case 256:
      if constexpr (std::is_same<Tin, __bf16>::value) return mlstm_pair<Tin, 256, CM>(a, ws);
      break;
  }
  return GDR_ERR_UNSUPPORTED;
}

template <typename Tin>
static int mlstm_ws_chunk(const MlstmArgs& a, char* ws) {
  switch (a.chunk) {
    case 16: return mlstm_ws_dk<Tin, 16>(a, ws);
    case 32: return mlstm_ws_dk<Tin, 32>(a, ws);
    case 64: return mlstm_ws_dk<Tin, 64>(a, ws);
  }
  return GDR_ERR_UNSUPPORTED;
}

int mlstm_ws_launch(const MlstmArgs& a, void* ws) {
  if (a.dtype == GDR_BF16) return mlstm_ws_chunk<__bf16>(a, (char*)ws);
  return mlstm_ws_chunk<float>(a, (char*)ws);
}

}  // namespace gdr
