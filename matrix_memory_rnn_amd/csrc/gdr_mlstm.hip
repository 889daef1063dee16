// Chunkwise forward of the xLSTM mLSTM cell with its log-domain stabiliser on
// gfx950 ("Exponential gates and matrix memory: xLSTM and RWKV-7", §13.4 and
// the solution to Exercise 13.6), in the [d_k, d_v] state orientation.
//
// Per chunk of C tokens with incoming state (C0, n0, m0):
//   F_t   = sum_{r<=t} log sigmoid(f_tilde_r)           (within the chunk)
//   a_s   = i_tilde_s - F_s
//   mu_t  = max(m0, max_{s<=t} a_s),   m_t = F_t + mu_t  (the running max of
//           m_t = max(log f_t + m_{t-1}, i_tilde_t), unrolled)
//   h^_t  = e^{m0 - mu_t} q_t C0 + sum_{s<=t} (q_t . k_s) e^{a_s - mu_t} v_s
//   n^_t  = e^{m0 - mu_t} q_t . n0 + sum_{s<=t} (q_t . k_s) e^{a_s - mu_t}
//   h_t   = h^_t / max(|n^_t|, e^{-m_t})
//   C_C   = e^{m0 - mu_C} C0 + sum_s e^{a_s - mu_C} k_s^T v_s   (n likewise)
// Every exponent above is <= 0 by construction of mu. The normaliser n rides
// along as an extra value column (a 16-wide tile whose first column is n and
// whose value row is all ones), so h^ and n^ come out of the same MFMAs.
//
// One workgroup (256 threads) per (b, h, value tile of VT columns); the tile
// walks the chunks sequentially, holding its [C | n] state slice in registers.
//
// Precision: bf16 inputs use bf16 MFMA operands with fp32 accumulation; fp32
// inputs keep fp32 operands in LDS and use fp32 MFMA (16x16x4).
#include "gdr_device.hpp"
#include "gdr_internal.h"
#include "gdr_host.hpp"

namespace gdr {

template <int DK, int VT, int CM, bool SPLIT>
struct MlstmSmem {
  static constexpr int NS = SPLIT ? 2 : 1;
  static constexpr int NVA = VT / 16 + 1;  // value tiles incl. the normaliser tile
  static constexpr int VA = 16 * NVA;
  static constexpr int LDK = DK + 8;
  static constexpr int LDC = CM + 8;
  static constexpr int P_Q = CM * LDK * 2;
  static constexpr int P_KT = DK * LDC * 2;
  static constexpr int P_V = VA * LDC * 2;
  static constexpr int P_W = CM * LDC * 2;
  static constexpr int P_C0 = VA * LDK * 2;
  static constexpr int Q = 0;
  static constexpr int K = Q + NS * P_Q;
  static constexpr int KT = K + NS * P_Q;
  static constexpr int VTR = KT + NS * P_KT;   // [v][s] raw values, ones row for n
  static constexpr int VTW = VTR + NS * P_V;   // [v][s] scaled by e^{a_s - mu_C}
  static constexpr int W = VTW + NS * P_V;     // [t][s] (q.k) e^{a_s - mu_t}
  static constexpr int C0T = W + NS * P_W;     // [v][j] state^T (+ n row): fp32, or bf16 hi + lo planes
  static constexpr int SC = C0T + 2 * P_C0;    // fp32 scalars: a, mu, m, wstate, nbar
  static constexpr int WP = SC + 5 * CM * 4 + 16;   // fp32 row sums of W per s-block [J][t]
  static constexpr int TOTAL = WP + (CM / 16) * CM * 4;
  static_assert(TOTAL <= 160 * 1024, "mLSTM kernel LDS exceeds 160 KiB");
};

__device__ __forceinline__ float log_sigmoid(float x) {
  // log sigmoid(x) = -softplus(-x) = min(x, 0) - log1p(exp(-|x|))
  return fminf(x, 0.f) - log1pf(__expf(-fabsf(x)));
}

template <typename Tin, int DK, int VT, int CM, bool SPLIT>
__global__ __launch_bounds__(256, 1) void mlstm_chunk_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ i_tilde, const float* __restrict__ f_tilde,
    const float* __restrict__ C0, const float* __restrict__ n0, const float* __restrict__ m0,
    Tin* __restrict__ h, float* C_out, float* n_out, float* m_out, int T, int DV, int C) {
  using L = MlstmSmem<DK, VT, CM, SPLIT>;
  constexpr int MM = SPLIT ? kF32 : kBF;  // fp32 inputs: fp32 MFMA; bf16 inputs: bf16 MFMA
  // the state copy that q reads: fp32, or bf16 hi + lo planes (the readout's
  // sums can cancel, so a single bf16 rounding of the state is not enough)
  constexpr int SM = SPLIT ? kF32 : kSP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NVL = VT / 16, NVA = L::NVA;
  constexpr int NST = (DK / 16) * NVA;
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
  const size_t seqK = (size_t)bh * T * DK, seqV = (size_t)bh * T * DV, seqG = (size_t)bh * T;

  float* sA = (float*)(smem + L::SC);
  float* sMu = sA + CM;
  float* sM = sMu + CM;
  float* sWs = sM + CM;
  float* sN = sWs + CM;
  float* sWP = (float*)(smem + L::WP);

  // ---- state slice [C | n] -> registers and C0^T (bf16)
  const bool have_state = (C0 != nullptr);
  float mprev = have_state ? m0[bh] : -INFINITY;
  f32x4 Sacc[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    Sacc[i] = f4zero();
    const int tile = wid + 4 * i;
    if (tile < NST) {
      const int jt = tile / NVA, vl = tile % NVA;
      if (have_state) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * jt + 4 * g + e;
          if (vl < NVL) Sacc[i][e] = C0[(size_t)bh * DK * DV + (size_t)j * DV + vt0 + 16 * vl + c16];
          else Sacc[i][e] = (c16 == 0) ? n0[(size_t)bh * DK + j] : 0.f;
        }
      }
      st4<SM>(smem + L::C0T, L::P_C0, (16 * vl + c16) * L::LDK + 16 * jt + 4 * g, Sacc[i]);
    }
  }
  __syncthreads();

  // ---- input staging: item (s, j0) = 8 consecutive channels of row s, with
  // lanes running along s so that one load feeds q, k ([s][j], 16-byte LDS
  // writes) and k^T ([j][s], 2-byte writes to consecutive addresses) without
  // bank conflicts. Loads are branch-free (row clamped, padding selected) and,
  // for bf16 inputs, issued one chunk ahead.
  using RW = Raw<Tin>;
  constexpr bool PF = !SPLIT;
  constexpr int KG = DK / 8;
  constexpr int NIT = (CM * KG + 255) / 256;
  constexpr int NIV = (CM * (VT / 8) + 255) / 256;
  typename RW::R8 cq[NIT], ck[NIT], nq[NIT], nk[NIT], cvv[NIV], nvv[NIV];
  float cf = 0.f, ci = 0.f, nf = 0.f, ni = 0.f;
  auto issue = [&](int chk, typename RW::R8* xq, typename RW::R8* xk, typename RW::R8* xv, float& xf,
                   float& xi) {
    const int tb = chk * C;
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int it = tid + 256 * i;
      const int s = it % C, j0 = (it / C) * 8;
      const int tg = tb + s;
      const size_t off = seqK + (size_t)(tg < T ? tg : T - 1) * DK + (j0 < DK ? j0 : 0);
      xq[i] = RW::ld8(q + off);
      xk[i] = RW::ld8(k + off);
    }
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      const int it = tid + 256 * i;
      const int s = it % C, v0 = (it / C) * 8;
      const int tg = tb + s;
      xv[i] = RW::ld8(v + seqV + (size_t)(tg < T ? tg : T - 1) * DV + vt0 + (v0 < VT ? v0 : 0));
    }
    if (wid == 0) {
      const int tg = tb + (lane < C ? lane : 0);
      const size_t og = seqG + (tg < T ? tg : T - 1);
      xf = f_tilde[og];
      xi = i_tilde[og];
    }
  };
  if (PF) issue(0, nq, nk, nvv, nf, ni);
  // rows of the normaliser tile below its first row are constant zero
  for (int it = tid; it < (L::VA - VT - 1) * CM; it += 256) {
    st1<MM>(smem + L::VTR, L::P_V, (VT + 1 + it / CM) * L::LDC + it % CM, 0.f);
    st1<MM>(smem + L::VTW, L::P_V, (VT + 1 + it / CM) * L::LDC + it % CM, 0.f);
  }

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * C;
    if constexpr (PF) {
#pragma unroll
      for (int i = 0; i < NIT; ++i) { cq[i] = nq[i]; ck[i] = nk[i]; }
#pragma unroll
      for (int i = 0; i < NIV; ++i) cvv[i] = nvv[i];
      cf = nf;
      ci = ni;
      if (ch + 1 < nchunks) issue(ch + 1, nq, nk, nvv, nf, ni);
    } else {
      issue(ch, cq, ck, cvv, cf, ci);
    }
    // ---------------- gates: F, a, mu, m (wave 0, one lane per token)
    if (wid == 0) {
      const int t = lane;
      const bool valid = (t < C) && (t0 + t < T);
      const float lf = valid ? log_sigmoid(cf) : 0.f;
      const float it = valid ? ci : -INFINITY;
      float F = lf;  // inclusive prefix sum over the chunk
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(F, off, 64);
        if (lane >= off) F += y;
      }
      const float a = it - F;
      float cm = a;  // inclusive prefix max
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(cm, off, 64);
        if (lane >= off) cm = fmaxf(cm, y);
      }
      const float mu = fmaxf(mprev, cm);
      const float muC = __shfl(mu, C - 1, 64);
      if (t < C) {
        sA[t] = a;
        sMu[t] = mu;
        sM[t] = F + mu;
        sWs[t] = valid ? __expf(a - muC) : 0.f;
      }
    }
    // ---------------- q, k, k^T, v^T (+ the ones row of the normaliser)
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int it = tid + 256 * i;
      if (it < C * KG) {
        const int s = it % C, j0 = (it / C) * 8;
        const bool ok = t0 + s < T;
        float fq[8], fk[8];
        RW::un8(RW::sel(ok, cq[i], RW::zero8()), fq);
        RW::un8(RW::sel(ok, ck[i], RW::zero8()), fk);
        st4<MM>(smem + L::Q, L::P_Q, s * L::LDK + j0, f32x4{fq[0], fq[1], fq[2], fq[3]});
        st4<MM>(smem + L::Q, L::P_Q, s * L::LDK + j0 + 4, f32x4{fq[4], fq[5], fq[6], fq[7]});
        st4<MM>(smem + L::K, L::P_Q, s * L::LDK + j0, f32x4{fk[0], fk[1], fk[2], fk[3]});
        st4<MM>(smem + L::K, L::P_Q, s * L::LDK + j0 + 4, f32x4{fk[4], fk[5], fk[6], fk[7]});
#pragma unroll
        for (int e = 0; e < 8; ++e) st1<MM>(smem + L::KT, L::P_KT, (j0 + e) * L::LDC + s, fk[e]);
      }
    }
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      const int it = tid + 256 * i;
      if (it < C * (VT / 8)) {
        const int s = it % C, v0 = (it / C) * 8;
        const bool ok = t0 + s < T;
        float fv[8];
        RW::un8(RW::sel(ok, cvv[i], RW::zero8()), fv);
#pragma unroll
        for (int e = 0; e < 8; ++e) st1<MM>(smem + L::VTR, L::P_V, (v0 + e) * L::LDC + s, fv[e]);
      }
    }
    if (tid < C) st1<MM>(smem + L::VTR, L::P_V, VT * L::LDC + tid, (t0 + tid < T) ? 1.f : 0.f);
    __syncthreads();
    // scaled values for the state update
    for (int it = tid; it < (VT + 1) * C; it += 256) {
      const int s = it % C, vr = it / C;
      const float val = ld1<MM>(smem + L::VTR, L::P_V, vr * L::LDC + s);
      st1<MM>(smem + L::VTW, L::P_V, vr * L::LDC + s, val * sWs[s]);
    }

    // ---------------- scores (transposed tiles) and the inter-chunk readout
    f32x4 gP[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      gP[i] = f4zero();
      const int p = wid + 4 * i;
      if (p < NP) {
        int tb = 0;
        while ((tb + 1) * (tb + 2) / 2 <= p) ++tb;
        const int sb = p - tb * (tb + 1) / 2;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          Frag<MM> A = ldfrag<MM>(smem + L::K, L::P_Q, L::LDK, 16 * sb, k0, DK, lane);
          Frag<MM> B = ldfrag<MM>(smem + L::Q, L::P_Q, L::LDK, 16 * tb, k0, DK, lane);
          mma<MM>(gP[i], A, B);
        }
      }
    }
    f32x4 Hin[NVA];
    if (wid < NB) {
#pragma unroll
      for (int vl = 0; vl < NVA; ++vl) {
        Hin[vl] = f4zero();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          Frag<MM> B = ldfrag<MM>(smem + L::Q, L::P_Q, L::LDK, 16 * wid, k0, DK, lane);
          if constexpr (MM == kBF) {
            mma_split(Hin[vl], ldfrag<kSP>(smem + L::C0T, L::P_C0, L::LDK, 16 * vl, k0, DK, lane), B);
          } else {
            Frag<MM> A = ldfrag<MM>(smem + L::C0T, L::P_C0, L::LDK, 16 * vl, k0, DK, lane);
            mma<MM>(Hin[vl], A, B);
          }
        }
      }
    }
    __syncthreads();
    // W[t][s] = (q_t . k_s) e^{a_s - mu_t}, s <= t
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int p = wid + 4 * i;
      if (p < NP) {
        int tb = 0;
        while ((tb + 1) * (tb + 2) / 2 <= p) ++tb;
        const int sb = p - tb * (tb + 1) / 2;
        const int t = 16 * tb + c16, s0 = 16 * sb + 4 * g;
        const float mut = sMu[t];
        f32x4 wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = s0 + e;
          wv[e] = (s <= t) ? gP[i][e] * __expf(sA[s] - mut) : 0.f;
        }
        st4<MM>(smem + L::W, L::P_W, t * L::LDC + s0, wv);
        // the normaliser's sums in fp32, before W is rounded to the operand
        // precision (they can cancel)
        float rs = (wv[0] + wv[1]) + (wv[2] + wv[3]);
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        if (g == 0) sWP[sb * CM + t] = rs;
      }
    }
    __syncthreads();

    // ---------------- intra-chunk readout and normaliser
    f32x4 Hx[NVA];
    if (wid < NB) {
      const int tb = wid, kend = 16 * (tb + 1);
      const int t = 16 * tb + c16;
      const float winter = (mprev == -INFINITY) ? 0.f : __expf(mprev - sMu[t]);
#pragma unroll
      for (int vl = 0; vl < NVA; ++vl) {
        f32x4 acc = f4zero();
        for (int k0 = 0; k0 < kend; k0 += 32) {
          Frag<MM> A = ldfrag<MM>(smem + L::VTR, L::P_V, L::LDC, 16 * vl, k0, kend, lane);
          Frag<MM> B = ldfrag<MM>(smem + L::W, L::P_W, L::LDC, 16 * tb, k0, kend, lane);
          mma<MM>(acc, A, B);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) Hx[vl][e] = winter * Hin[vl][e] + acc[e];
      }
      if (g == 0) {
        // q_t . n0 (row 0 of the normaliser tile) plus the fp32 sums of W
        float ws = 0.f;
        for (int J = 0; J <= tb; ++J) ws += sWP[J * CM + t];
        sN[t] = winter * Hin[NVL][0] + ws;
      }
    }
    __syncthreads();
    if (wid < NB) {
      const int t = 16 * wid + c16, tg = t0 + t;
      const float den = fmaxf(fabsf(sN[t]), __expf(-sM[t]));
      const float inv = 1.f / den;
      if (tg < T) {
#pragma unroll
        for (int vl = 0; vl < NVL; ++vl) {
          f32x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = Hx[vl][e] * inv;
          In<Tin>::store4(h + seqV + (size_t)tg * DV + vt0 + 16 * vl + 4 * g, hv);
        }
      }
    }

    // ---------------- state update: C <- e^{m0 - mu_C} C + K^T (w .* [V | 1])
    const float muC = sMu[C - 1];
    const float dstate = (mprev == -INFINITY) ? 0.f : __expf(mprev - muC);
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + 4 * i;
      if (tile < NST) {
        const int jt = tile / NVA, vl = tile % NVA;
        f32x4 acc = f4zero();
        for (int k0 = 0; k0 < C; k0 += 32) {
          Frag<MM> A = ldfrag<MM>(smem + L::KT, L::P_KT, L::LDC, 16 * jt, k0, C, lane);
          Frag<MM> B = ldfrag<MM>(smem + L::VTW, L::P_V, L::LDC, 16 * vl, k0, C, lane);
          mma<MM>(acc, A, B);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[i][e] = dstate * Sacc[i][e] + acc[e];
      }
    }
    mprev = sM[C - 1];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + 4 * i;
      if (tile < NST) {
        const int jt = tile / NVA, vl = tile % NVA;
        st4<SM>(smem + L::C0T, L::P_C0, (16 * vl + c16) * L::LDK + 16 * jt + 4 * g, Sacc[i]);
      }
    }
  }

  if (C_out) {
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + 4 * i;
      if (tile < NST) {
        const int jt = tile / NVA, vl = tile % NVA;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * jt + 4 * g + e;
          if (vl < NVL) C_out[(size_t)bh * DK * DV + (size_t)j * DV + vt0 + 16 * vl + c16] = Sacc[i][e];
          else if (c16 == 0 && vt0 == 0) n_out[(size_t)bh * DK + j] = Sacc[i][e];
        }
      }
    }
    if (tid == 0 && vt0 == 0) m_out[bh] = mprev;
  }
}

template <typename Tin, int DK, int VT, int CM>
static int launch_mlstm(const MlstmArgs& a) {
  constexpr bool SPLIT = std::is_same<Tin, float>::value;
  using L = MlstmSmem<DK, VT, CM, SPLIT>;
  auto kern = mlstm_chunk_kernel<Tin, DK, VT, CM, SPLIT>;
  if (!allow_lds((const void*)kern, L::TOTAL)) return GDR_ERR_LAUNCH;
  const int nblocks = a.B * a.H * (a.dv / VT);
  const Tin *q = (const Tin*)a.q, *k = (const Tin*)a.k, *v = (const Tin*)a.v;
  const float *it = a.i_tilde, *ft = a.f_tilde, *C0 = a.C0, *n0 = a.n0, *m0 = a.m0;
  Tin* h = (Tin*)a.h;
  float *Co = a.C_out, *no = a.n_out, *mo = a.m_out;
  int T = a.T, DV = a.dv, C = a.chunk;
  void* args[] = {&q, &k, &v, &it, &ft, &C0, &n0, &m0, &h, &Co, &no, &mo, &T, &DV, &C};
  hipError_t e = hipLaunchKernel((const void*)kern, dim3(nblocks), dim3(256), args, L::TOTAL,
                                 (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

template <typename Tin, int VT>
static int mlstm_dk(const MlstmArgs& a) {
  constexpr bool SPLIT = std::is_same<Tin, float>::value;
  switch (a.dk) {
    case 16: return launch_mlstm<Tin, 16, VT, 64>(a);
    case 32: return launch_mlstm<Tin, 32, VT, 64>(a);
    case 64: return launch_mlstm<Tin, 64, VT, 64>(a);
    case 128: return launch_mlstm<Tin, 128, VT, 64>(a);
    case 256:
      // 16-column tiles: the state copy's two bf16 planes of 32 columns and
      // the staged chunk do not fit the LDS together at d_k = 256
      if constexpr (!SPLIT) return launch_mlstm<Tin, 256, 16, 64>(a);
      break;
  }
  return GDR_ERR_UNSUPPORTED;
}

int mlstm_launch(const MlstmArgs& a) {
  if (a.dtype == GDR_BF16) return a.dv == 16 ? mlstm_dk<__bf16, 16>(a) : mlstm_dk<__bf16, 32>(a);
  return mlstm_dk<float, 16>(a);
}

}  // namespace gdr
