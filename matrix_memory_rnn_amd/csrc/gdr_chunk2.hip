// Two-kernel chunkwise forward of the channel-wise gated delta rule on gfx950.
//
// Method: "Muir: Linear Attention with Sensitivity-Allocated Gating and
// Matched-Filter Readout", §2.1 eq.(1) in the chunkwise form of §2.2, with
// the fused right-hand side [V^ | K^_pi] of §4.2. Per chunk of C tokens
// starting from state S0:
//   [U | Y] = T^{-1} [V^ | K^_pi],   V~ = U - Y S0,
//   O = Q_pi S0 + M V~,   S_C = Diag(pi_C) S0 + K~^T V~
// (T = I + L; L, M, Q_pi, K^_pi, K~ and pi_C as in gdr_chunk.hip). Only the
// three products with S0 depend on the state, so the work is split:
//
//   gdn2_chunk_intra_kernel — every (b, h, chunk) independently, all chunks
//     of all heads in parallel: block decay products, Gram tiles, T^{-1}
//     applied to the d_v + d_k right-hand-side columns by block forward
//     substitution. Writes one record per (b, h, chunk) to a caller-provided
//     workspace: Y, U^T, M, Q_pi, K~^T (input precision) and pi_C (fp32).
//   gdn2_chunk_scan_kernel — one workgroup per (b, h, value tile) walks the
//     chunks of its head in order: V~ = U - Y S0, O, S. Its MFMA operands come
//     from the record straight into registers, one chunk ahead.
//
// Compared with the single fused kernel this moves the S0-independent work
// (about three quarters of it) off the sequential path and does it once per
// chunk instead of once per value tile, at the price of writing and reading
// the record once.
#include "gdr_chunk_common.hpp"
#include "gdr_internal.h"
#include "gdr_host.hpp"
#include "gdr_record.hpp"

namespace gdr {

template <typename E> struct Out;
template <> struct Out<float> {
  static __device__ __forceinline__ void pair(float* p, float a, float b) { *(float2*)p = make_float2(a, b); }
  static __device__ __forceinline__ void quad(float* p, f32x4 v) { *(f32x4*)p = v; }
  static __device__ __forceinline__ void oct(float* p, const float* x) {
    *(f32x4*)p = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};
template <> struct Out<__bf16> {
  static __device__ __forceinline__ void pair(__bf16* p, float a, float b) {
    bf16x2 h;
    h.x = (__bf16)a;
    h.y = (__bf16)b;
    *(bf16x2*)p = h;
  }
  static __device__ __forceinline__ void quad(__bf16* p, f32x4 v) { In<__bf16>::store4(p, v); }
  static __device__ __forceinline__ void oct(__bf16* p, const float* x) {
    bf16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (__bf16)x[e];
    *(bf16x8*)p = h;
  }
};

typedef __attribute__((ext_vector_type(2))) uint32_t u2_t;

// Stores into one workspace record through a buffer resource: byte offsets
// are 32-bit (constant parts become immediates), values converted to the
// record's element type. The 4- and 8-byte stores carry the non-temporal
// cache policy (nt): measured on the 4K workload, the scan that reads the
// record back runs 124 -> 121 us with the intra kernel unchanged (nt on the
// 16-byte stores as well slowed the intra kernel by a fifth).
constexpr int kRecNt = 2;   // cache-policy operand of the buffer stores: nt
// The intra kernel's input loads are non-temporal too (each input row is read
// once): with the record stores above, intra 129 -> 116 us and the scan after
// it 120 -> 129 us, 0.2497 -> 0.2451 ms per 4K step (interleaved runs; with
// plain record stores the scan lost more than the intra kernel gained).
constexpr int kInNt = 2;
template <typename E> struct RecSt;
template <> struct RecSt<float> {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ void pair(int off, float a, float b) const {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, make_float2(a, b)), r, off, 0, kRecNt);
  }
  __device__ __forceinline__ void quad(int off, f32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
  }
  __device__ __forceinline__ void oct(int off, const float* x) const {
    quad(off, f32x4{x[0], x[1], x[2], x[3]});
    quad(off + 16, f32x4{x[4], x[5], x[6], x[7]});
  }
  __device__ __forceinline__ void raw16(int off, u32x4 v) const { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
};
template <> struct RecSt<__bf16> {
  __amdgpu_buffer_rsrc_t r;
  static __device__ __forceinline__ uint32_t pk(float a, float b) {
    bf16x2 h;
    h.x = (__bf16)a;
    h.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ __forceinline__ void pair(int off, float a, float b) const {
    __builtin_amdgcn_raw_buffer_store_b32(pk(a, b), r, off, 0, kRecNt);
  }
  __device__ __forceinline__ void quad(int off, f32x4 v) const {
    const float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
    __builtin_amdgcn_raw_buffer_store_b64(u2_t{pk(v0, v1), pk(v2, v3)}, r, off, 0, kRecNt);
  }
  __device__ __forceinline__ void oct(int off, const float* x) const {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{pk(x[0], x[1]), pk(x[2], x[3]), pk(x[4], x[5]), pk(x[6], x[7])},
                                           r, off, 0, 0);
  }
  __device__ __forceinline__ void raw16(int off, u32x4 v) const { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
};

// Right-looking forward substitution step for columns 4*M4 .. 4*M4+3 of a
// unit lower-triangular 16x16 system (rows of L in LDS with pitch LDB): once
// x[m] is final it is subtracted from every later row, so the dependent chain
// is one FMA per row and the other updates run alongside.
template <int M4, int LDB>
__device__ __forceinline__ void fs_load(const float* Lb, f32x4* lc) {
#pragma unroll
  for (int r = 4 * M4 + 1; r < 16; ++r) lc[r] = *(const f32x4*)(Lb + r * LDB + 4 * M4);
}
template <int M4>
__device__ __forceinline__ void fs_apply(const f32x4* lc, float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * M4 + e;
#pragma unroll
    for (int r = m + 1; r < 16; ++r) x[r] -= lc[r][e] * x[m];
  }
}
template <int M4, int LDB>
__device__ __forceinline__ void fs_group(const float* Lb, float* x) {
  f32x4 lc[16];
  fs_load<M4, LDB>(Lb, lc);
  fs_apply<M4>(lc, x);
}

// ============================================================================ intra kernel
constexpr int kIntraThreads = 512;

constexpr int kMaxDv = 128;

template <typename Tin, int DK, int CM>
struct IntraSmem {
  static constexpr bool F32 = std::is_same<Tin, float>::value;
  static constexpr int NS = F32 ? 2 : 1;           // bf16 planes' worth of bytes per MM operand element
  static constexpr int ES = sizeof(Tin);
  static constexpr int NBM = CM / 16;
  static constexpr int NPM = NBM * (NBM + 1) / 2;
  static constexpr int LDK = DK + 8, LDC = CM + 8, LDB = 20, LDY = DK + 8;
  static constexpr int P_CK = CM * LDK * 2;
  static constexpr int P_CC = CM * LDC * 2;
  static constexpr int P_XC = (kMaxDv + DK) * LDC * 2;
  // precision of the triangular solve: bf16 operands with fp32 accumulation
  // for bf16 inputs (one plane per solve buffer), fp32 for fp32 inputs
  static constexpr int MT = F32 ? kF32 : kBF;
  static constexpr int NPL = MT == kBF ? 1 : 2;     // planes (bytes / 2 per element) of XR and TL
  static constexpr int BLK = 16 * LDB * 4;
  // [V^ | K^_pi]^T, solved in place, T mode [col][t]. With bf16 inputs it has
  // a region of its own and is filled during prep, so no input register is
  // live across the next item's prefetch; with fp32 (no prefetch) it lies
  // over the prep / Gram operands to fit in 160 KiB.
  static constexpr bool XR_EARLY = !F32;
  static constexpr int XR_BYTES = NPL * P_XC;
  static constexpr int AB = XR_EARLY ? XR_BYTES : 0;   // base of the phase A / phase B area
  // phase A: prep and Gram operands
  static constexpr int KR = AB;                     // k^ * P   [t][j]
  static constexpr int QR = KR + NS * P_CK;         // q * P    [t][j]
  static constexpr int KC = QR + NS * P_CK;         // k * Qs   [t][j]
  static constexpr int A_END = KC + NS * P_CK;
  // fp32, phase B (over phase A, after the Gram products): L blocks, D_I,
  // the [-L' | D] rows and the right-hand sides
  static constexpr int LBK = AB;                    // L blocks fp32 [pair][t][s]
  static constexpr int TBN_B = LBK + NPM * BLK;     // D_I fp32 [I][t][s]
  static constexpr int TL_B = TBN_B + NBM * BLK;    // [.. -L'_IJ .. | D_I] rows, T mode [t][s]
  static constexpr int XR = XR_EARLY ? 0 : TL_B + 2 * P_CC;
  static constexpr int B_END = XR_EARLY ? AB : XR + XR_BYTES;
  // Y staging [t][j] (input precision): bf16 over phase A (dead once the
  // solve starts), fp32 in a region of its own
  static constexpr int YS_BYTES = CM * LDY * ES;
  static_assert(F32 || YS_BYTES <= A_END - AB, "Y staging fits over the Gram operands");
  static constexpr int YS = F32 ? align16(imax(A_END, B_END)) : AB;
  static constexpr int X_END = F32 ? YS + YS_BYTES : imax(A_END, B_END);
  static constexpr int SCL = align16(X_END);        // Gram scale vectors fp32 [pair][j]
  static constexpr int GS = SCL + NPM * DK * 4;     // block totals fp32 [I][j]
  static constexpr int FLAG = GS + NBM * DK * 4;    // guard flags [4]
  // bf16: staging for records in F order, so the record stores are 16-byte
  // and coalesced: Q_pi [t][j] after prep, then U^T [v][t] during the solve
  static constexpr int LDU = kMaxDv + 8, LDUT = CM + 8;
  static constexpr int US = align16(FLAG + 16);
  // bf16: the diagonal L blocks, D_I and the [-L' | D] rows have regions of
  // their own, written while other waves still read the Gram operands
  static constexpr int LBD = US + imax(CM * LDU, kMaxDv * LDUT) * 2;   // diagonal L fp32 [I][t][s]
  static constexpr int TBN = F32 ? TBN_B : LBD + NBM * BLK;
  static constexpr int TL = F32 ? TL_B : TBN + NBM * BLK;
  // bf16: -L_IJ of the off-diagonal pairs in accumulator lane order (8 bytes
  // per lane), read by every wave to form the L' blocks it needs
  static constexpr int LT = TL + P_CC;
  static constexpr int TOTAL = F32 ? FLAG + 16 : LT + (NBM * (NBM - 1) / 2) * 512;
  static_assert(TOTAL <= 160 * 1024, "intra kernel LDS exceeds 160 KiB");
};

// GATED: alpha, bgate and wgate hold the gate logits z_f, z_b, z_w of the Muir
// page (§2.1, §4.1) and the gates are formed here in fp32 (gate_alpha,
// 2 gate_sigmoid, gate_sigmoid); q is read as the gain-modulated query
// gamma * q with gamma = gstat[h] * 2 sigmoid(z_q) (zq NULL: z_q = 0; gstat
// NULL: ones), and alog[h] is the head's log-rate.
// INNT: the bf16 input loads take the non-temporal cache policy (kInNt). The
// launcher turns it off for the gate prologue (4K shape: 0.2808 ms per step
// with plain loads against 0.2840).
template <typename Tin, int DK, int CM, bool FM, bool GATED, bool INNT = true>
__global__ __launch_bounds__(kIntraThreads, 2) void gdn2_chunk_intra_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ alpha, const Tin* __restrict__ bgate, const Tin* __restrict__ wgate,
    char* __restrict__ ws, int T, int DV, int nchunks, int nitems, const Tin* __restrict__ zq,
    const float* __restrict__ alog, const float* __restrict__ gstat, int H) {
  using L = IntraSmem<Tin, DK, CM>;
  constexpr bool F32 = L::F32;
  static_assert(!FM || (!F32 && DK % 32 == 0 && CM % 32 == 0), "F order needs bf16, d_k and C multiples of 32");
  constexpr int MM = F32 ? kF32 : kBF;   // Gram operands
  constexpr int MT = L::MT;              // triangular solve
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NW = kIntraThreads / 64;
  constexpr int NB = CM / 16;
  constexpr int NP = L::NPM;
  constexpr int NQ = NB * (NB - 1) / 2;
  constexpr int MAXP = (NP + NW - 1) / NW;
  constexpr int MAXQ = (NQ + NW - 1) / NW;
  constexpr int MAXX = ((kMaxDv + DK) / 16 + NW - 1) / NW;
  constexpr int MAXVI = (CM * kMaxDv / 8 + kIntraThreads - 1) / kIntraThreads;
  constexpr int BLKF = 16 * L::LDB;

  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const RecLayout RL = rec_layout(DK, DV, CM, sizeof(Tin));
  const int NX = (DV + DK) / 16;
  // XR element offset of (column col, row t): the 8-row slots of a column are
  // XOR-swizzled by the column's 16-column group, so the transposed 2-byte
  // writes of a v^ row (16 lanes, columns 8 apart) spread over distinct banks
  // while a 16-column fragment read still sees one uniform slot order
  constexpr int XM = CM / 8 - 1;
  auto xoff = [](int col, int t) { return col * L::LDC + 8 * ((t >> 3) ^ ((col >> 4) & XM)) + (t & 7); };
  // record element offsets: row-major, or F order for the 32x32x16 scan
  auto o_tk = [](int t, int jj) { return FM ? fm_off(t, jj, DK) : t * DK + jj; };   // Y, Q_pi
  auto o_kt = [](int jj, int t) { return FM ? fm_off(jj, t, CM) : jj * CM + t; };   // K~^T
  auto o_m = [](int t, int s) { return FM ? fm_off(t, s, CM) : t * CM + s; };       // M
  auto o_ut = [](int vv, int t) { return FM ? fu_off(vv, t, CM) : vv * CM + t; };    // U^T

  float* GS = (float*)(smem + L::GS);
  float* SCL = (float*)(smem + L::SCL);
  int* FLAGS = (int*)(smem + L::FLAG);
  float* LBK = (float*)(smem + L::LBK);
  float* TBN = (float*)(smem + L::TBN);
  Tin* YS = (Tin*)(smem + L::YS);

  int item = blockIdx.x;
  if (item >= nitems) return;
  if (tid < 4) FLAGS[tid] = 0;

  // ---- input staging (as in the fused kernel): lanes l and l^32 share
  // channels (j, j+1) of block I0, rows 0-7 (h = 0) and 8-15 (h = 1).
  using RW = Raw<Tin>;
  const int h = lane >> 5;
  const int fp = wid * 32 + (lane & 31);
  const bool act = fp < NB * (DK / 2);
  const int I0 = act ? fp / (DK / 2) : 0, j = act ? 2 * (fp % (DK / 2)) : 0;
  const int r0 = 16 * I0 + 8 * h;
  // v^ items: 8 consecutive value columns of one row (coalesced loads)
  const int nvi = CM * (DV / 8);
  typename RW::R2 xa[8], xk[8], xb[8], xq[8];
  typename RW::R8 xv[MAXVI], xw[MAXVI];
  // GATED: query-gain logits z_q (zero when not given)
  typename RW::R2 xz[GATED ? 8 : 1];
  // parts: 1 = alpha and k, 2 = b and q, 4 = v and w
  auto issue = [&](int it, int parts) {
    const int bh = it / nchunks, tb = (it % nchunks) * CM;
    if constexpr (!F32) {
      // bf16: buffer loads over one sequence of each input; rows past T lie
      // past the buffer's end and read as zero (alpha is set to 1 there by
      // the caller), the row step is the instruction's immediate offset
      constexpr int ES = (int)sizeof(Tin);
      const unsigned nbK = (unsigned)T * DK * ES, nbV = (unsigned)T * DV * ES;
      const size_t sK = (size_t)bh * T * DK, sV = (size_t)bh * T * DV;
      const int vo = ((tb + r0) * DK + j) * ES;
      auto rs = [&](const Tin* base, size_t off, unsigned nb) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<Tin*>(base + off), 0, nb, 0x00020000);
      };
      if (parts & 1) {
        const __amdgpu_buffer_rsrc_t ra = rs(alpha, sK, nbK), rk = rs(k, sK, nbK);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          xa[r] = __builtin_amdgcn_raw_buffer_load_b32(ra, vo + r * DK * ES, 0, INNT ? kInNt : 0);
          xk[r] = __builtin_amdgcn_raw_buffer_load_b32(rk, vo + r * DK * ES, 0, INNT ? kInNt : 0);
        }
      }
      if (parts & 2) {
        const __amdgpu_buffer_rsrc_t rb = rs(bgate, sK, nbK), rq = rs(q, sK, nbK);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          xb[r] = __builtin_amdgcn_raw_buffer_load_b32(rb, vo + r * DK * ES, 0, INNT ? kInNt : 0);
          xq[r] = __builtin_amdgcn_raw_buffer_load_b32(rq, vo + r * DK * ES, 0, INNT ? kInNt : 0);
        }
        if constexpr (GATED) {
          // no z_q: a buffer of zero records, every load reads zero
          const __amdgpu_buffer_rsrc_t rz = zq ? rs(zq, sK, nbK) : rs(q, 0, 0u);
#pragma unroll
          for (int r = 0; r < 8; ++r) xz[r] = __builtin_amdgcn_raw_buffer_load_b32(rz, vo + r * DK * ES, 0, INNT ? kInNt : 0);
        }
      }
      if (parts & 4) {
        const __amdgpu_buffer_rsrc_t rv = rs(v, sV, nbV), rw = rs(wgate, sV, nbV);
#pragma unroll
        for (int i = 0; i < MAXVI; ++i) {
          const int idx = tid + kIntraThreads * i;
          const int vrow = idx / (DV / 8), vcol = (idx % (DV / 8)) * 8;
          // items past the tile read past the buffer's end (zero)
          const int vv = idx < nvi ? ((tb + vrow) * DV + vcol) * ES : 0x7ffffff0;
          xv[i] = __builtin_bit_cast(typename RW::R8, __builtin_amdgcn_raw_buffer_load_b128(rv, vv, 0, INNT ? kInNt : 0));
          xw[i] = __builtin_bit_cast(typename RW::R8, __builtin_amdgcn_raw_buffer_load_b128(rw, vv, 0, INNT ? kInNt : 0));
        }
      }
    } else {
      const size_t sK = (size_t)bh * T * DK + j, sV = (size_t)bh * T * DV;
      if (parts & 1) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = tb + r0 + r;
          const size_t off = sK + (size_t)(t < T ? t : T - 1) * DK;
          xa[r] = RW::ld2(alpha + off);
          xk[r] = RW::ld2(k + off);
        }
      }
      if (parts & 2) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = tb + r0 + r;
          const size_t off = sK + (size_t)(t < T ? t : T - 1) * DK;
          xb[r] = RW::ld2(bgate + off);
          xq[r] = RW::ld2(q + off);
          if constexpr (GATED) xz[r] = zq ? RW::ld2(zq + off) : RW::pad2(0.f);
        }
      }
      if (parts & 4) {
#pragma unroll
        for (int i = 0; i < MAXVI; ++i) {
          const int idx = tid + kIntraThreads * i;
          const int vi = idx < nvi ? idx : 0;
          const int vrow = vi / (DV / 8), vcol = (vi % (DV / 8)) * 8;
          const int tv = tb + vrow;
          const size_t off = sV + (size_t)(tv < T ? tv : T - 1) * DV + vcol;
          xv[i] = RW::ld8(v + off);
          xw[i] = RW::ld8(wgate + off);
        }
      }
    }
  };
  // bf16: the next item's inputs are fetched while this item is worked on;
  // fp32 (twice the registers) fetches at the start of each item.
  // in the order the loop issues them (v and w first), so that the wait
  // counts at the top of the loop can be exact
  if constexpr (!F32) {
    issue(item, 4);
    __builtin_amdgcn_sched_barrier(0);
    issue(item, 1);
    __builtin_amdgcn_sched_barrier(0);
    issue(item, 2);
  }
  __syncthreads();

  for (; item < nitems; item += gridDim.x) {
    if constexpr (F32) issue(item, 7);
    // the item whose inputs are fetched during this one: the next of this
    // workgroup, or item 0 after the last (the loads are always issued, so the
    // wait counts do not depend on a branch; every workgroup's last fetch
    // reads the same item, which the L2 serves)
    const int nxt = item + (int)gridDim.x < nitems ? item + (int)gridDim.x : 0;
    // lane-derived values through an empty asm once per item: lane
    // predicates formed from them are computed where they are used instead of
    // being kept (and spilled) as scalar lane masks across the loop
    int hq = h, gq = g, cq = c16;
    asm volatile("" : "+v"(hq), "+v"(gq), "+v"(cq));
    const bool actq = (NB * (DK / 2) >= kIntraThreads / 2) || act;
    const int bh = item / nchunks, t0 = (item % nchunks) * CM;
    const size_t seqK = (size_t)bh * T * DK;
    char* rec = ws + (size_t)item * RL.bytes;
    const RecSt<Tin> RS{__builtin_amdgcn_make_buffer_rsrc(rec, 0, RL.bytes, 0x00020000)};
    constexpr int ES = (int)sizeof(Tin);

    // identity padding past the end of the sequence: alpha = 1, k = b = q = 0,
    // v = w = 0 (bf16: the buffer loads already read zeros there). GATED: the
    // decay logit -inf gives alpha = 1.
    float vh[MAXVI][8];
    float rate = 1.f, gsx = 1.f, gsy = 1.f;
    const float* gzh = nullptr;
    if constexpr (GATED) {
      const int hh = bh % H;
      rate = expf(alog[hh]);
      if (gstat) {
        gzh = gstat + (size_t)hh * DK;
        gsx = gzh[j];
        gsy = gzh[j + 1];
      }
    }
    // the exact in-block path reads the gates itself (from their logits when GATED)
    const GateRead<Tin, GATED> gread{zq, gzh, rate};
    {
      const typename RW::R2 one = RW::pad2(GATED ? -__builtin_inff() : 1.f), zero = RW::pad2(0.f);
      if (t0 + CM > T) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const bool ok = t0 + r0 + r < T;
          xa[r] = RW::sel(ok, xa[r], one);
          if constexpr (F32) {
            xk[r] = RW::sel(ok, xk[r], zero);
            xb[r] = RW::sel(ok, xb[r], zero);
            xq[r] = RW::sel(ok, xq[r], zero);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < MAXVI; ++i) {
        const int idx = tid + kIntraThreads * i;
        float fv[8], fw[8];
        RW::un8(xv[i], fv);
        RW::un8(xw[i], fw);
        if constexpr (GATED) {
#pragma unroll
          for (int e = 0; e < 8; ++e) fw[e] = gate_sigmoid(fw[e]);
        }
        if constexpr (F32) {
          const bool okv = idx < nvi && t0 + idx / (DV / 8) < T;
#pragma unroll
          for (int e = 0; e < 8; ++e) vh[i][e] = okv ? fv[e] * fw[e] : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) vh[i][e] = fv[e] * fw[e];
        }
      }
    }

    if constexpr (L::XR_EARLY) {
#pragma unroll
      for (int i = 0; i < MAXVI; ++i) {
        const int idx = tid + kIntraThreads * i;
        if (idx < nvi) {
          const int vrow = idx / (DV / 8), vcol = (idx % (DV / 8)) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) st1<MT>(smem + L::XR, L::P_XC, xoff(vcol + e, vrow), vh[i][e]);
        }
      }
    }
    // bf16: the next item's inputs are fetched in three parts spread over
    // this item (v and w here, alpha and k with the Gram products, b and q
    // with D_I), so that the loads of all CUs reach HBM as a steady stream
    // rather than in one burst per item
    if constexpr (!F32) {
      issue(nxt, 4);
    }

    // ================= prep 1: half-block products -> block totals G
    // GATED: the decays are formed from their logits once, here, in fp32
    float2 af[GATED ? 8 : 1];
    if constexpr (GATED) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float2 z = RW::un2(xa[r]);
        af[r] = make_float2(gate_alpha(z.x, rate), gate_alpha(z.y, rate));
      }
    }
    auto alpha_at = [&](int r) {
      if constexpr (GATED) return af[r];
      else return RW::un2(xa[r]);
    };
    float2 ph = make_float2(1.f, 1.f);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float2 a = alpha_at(r);
      ph.x *= a.x;
      ph.y *= a.y;
    }
    const float2 po = make_float2(__shfl_xor(ph.x, 32, 64), __shfl_xor(ph.y, 32, 64));
    const float2 p0 = hq ? po : ph, p1 = hq ? ph : po;
    if (actq && hq == 0) {
      const float gx = p0.x * p1.x, gy = p0.y * p1.y;
      GS[I0 * DK + j] = gx;
      GS[I0 * DK + j + 1] = gy;
      if (!(gx >= kGuardMin && gy >= kGuardMin)) FLAGS[I0] = 1;
    }
    __syncthreads();

    // ================= prep 2: Gram operands, Q_pi, K~^T, pi_C, scale vectors
    float2 khp[8];
    if (actq) {
      float2 Bst = make_float2(1.f, 1.f), E = make_float2(1.f, 1.f), pic = make_float2(1.f, 1.f);
      for (int J = 0; J < NB; ++J) {
        const float gx = GS[J * DK + j], gy = GS[J * DK + j + 1];
        if (J < I0) { Bst.x *= gx; Bst.y *= gy; }
        if (J > I0) { E.x *= gx; E.y *= gy; }
        pic.x *= gx;
        pic.y *= gy;
      }
      if (hq == 0) {
        if (I0 == 0) RecSt<float>{RS.r}.pair(RL.pic + 4 * j, pic.x, pic.y);
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
      float2 P = hq ? p0 : make_float2(1.f, 1.f);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float2 a = alpha_at(r), kk = RW::un2(xk[r]);
        float2 bb = RW::un2(xb[r]), qq = RW::un2(xq[r]);
        if constexpr (GATED) {
          const float2 zz = RW::un2(xz[r]);
          bb = make_float2(2.f * gate_sigmoid(bb.x), 2.f * gate_sigmoid(bb.y));
          qq = make_float2(qq.x * gsx * 2.f * gate_sigmoid(zz.x), qq.y * gsy * 2.f * gate_sigmoid(zz.y));
        }
        P.x *= a.x;
        P.y *= a.y;
        const float krx = bb.x * kk.x * P.x, kry = bb.y * kk.y * P.y;
        const float qrx = qq.x * P.x, qry = qq.y * P.y;
        const int off = (r0 + r) * L::LDK + j;
        st2<MM>(smem + L::KR, L::P_CK, off, krx, kry);
        st2<MM>(smem + L::QR, L::P_CK, off, qrx, qry);
        khp[r] = make_float2(Bst.x * krx, Bst.y * kry);
        if constexpr (FM)   // staged [t][j] in US, stored in F order after the Gram tiles
          Out<Tin>::pair((Tin*)(smem + L::US) + (r0 + r) * L::LDU + j, Bst.x * qrx, Bst.y * qry);
        else
          RS.pair(RL.qp + o_tk(r0 + r, j) * ES, Bst.x * qrx, Bst.y * qry);
      }
      float ktx[8], kty[8];
      float2 qs = hq ? make_float2(1.f, 1.f) : p1;
#pragma unroll
      for (int r = 7; r >= 0; --r) {
        const float2 kk = RW::un2(xk[r]), a = alpha_at(r);
        const float kcx = kk.x * qs.x, kcy = kk.y * qs.y;
        st2<MM>(smem + L::KC, L::P_CK, (r0 + r) * L::LDK + j, kcx, kcy);
        ktx[r] = kcx * E.x;
        kty[r] = kcy * E.y;
        qs.x *= a.x;
        qs.y *= a.y;
      }
      RS.oct(RL.kt + o_kt(j, r0) * ES, ktx);
      RS.oct(RL.kt + o_kt(j + 1, r0) * ES, kty);
      if constexpr (L::XR_EARLY) {
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
          const float2* kp = khp + 4 * r4;
          st4<MT>(smem + L::XR, L::P_XC, xoff(DV + j, r0 + 4 * r4),
                  f32x4{kp[0].x, kp[1].x, kp[2].x, kp[3].x});
          st4<MT>(smem + L::XR, L::P_XC, xoff(DV + j + 1, r0 + 4 * r4),
                  f32x4{kp[0].y, kp[1].y, kp[2].y, kp[3].y});
        }
      }
    }
    __syncthreads();

    // ================= Gram tiles: L^T, M^T of pair (I, J) = (Kc_J * scale) [Kr_I; Qr_I]^T
    if constexpr (!F32) {
      issue(nxt, 1);
    }
    if constexpr (F32) {
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

      if constexpr (FM) {
        // Q_pi from its staging rows to the record: consecutive threads write
        // consecutive F-order pieces (US is free again before the solve)
        for (int idx = tid; idx < CM * DK / 8; idx += kIntraThreads) {
          const int q2 = idx >> 6, t = 32 * (q2 / (DK / 16)) + (idx & 31), pc = 2 * (q2 % (DK / 16)) + ((idx >> 5) & 1);
          RS.raw16(RL.qp + 16 * idx, *(const u32x4*)(smem + L::US + 2 * (t * L::LDU + 8 * pc)));
        }
      }

      // ================= L blocks (fp32, LDS), M (record), right-hand sides [V^ | K^_pi]^T
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int p = wid + NW * i;
        if (p < NP) {
          int I, J;
          pair_of(p, I, J);
          const int t = 16 * I + c16, s0 = 16 * J + 4 * g;
          f32x4 lv = gL[i], mv = gM[i];
          if (I == J) {
            if (FLAGS[I]) exact_diag<Tin, DK, GATED>(k, bgate, q, alpha, seqK, t0, T, t, s0, lv, mv, gread);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (s0 + e >= t) lv[e] = 0.f;
              if (s0 + e > t) mv[e] = 0.f;
            }
          }
          *(f32x4*)(LBK + p * BLKF + c16 * L::LDB + 4 * g) = lv;
          RS.quad(RL.m + o_m(t, s0) * ES, mv);
          // F order: the scan multiplies M in 32-column slices up to the
          // diagonal, so the block right of an even diagonal block is zero
          if constexpr (FM) {
            if (I == J && (I & 1) == 0) RS.quad(RL.m + o_m(t, s0 + 16) * ES, f4zero());
          }
        }
      }
      if constexpr (!L::XR_EARLY) {
#pragma unroll
        for (int i = 0; i < MAXVI; ++i) {
          const int idx = tid + kIntraThreads * i;
          if (idx < nvi) {
            const int vrow = idx / (DV / 8), vcol = (idx % (DV / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) st1<MT>(smem + L::XR, L::P_XC, xoff(vcol + e, vrow), vh[i][e]);
          }
        }
      }
      if (!L::XR_EARLY && act) {
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
          const float2* kp = khp + 4 * r4;
          st4<MT>(smem + L::XR, L::P_XC, xoff(DV + j, r0 + 4 * r4),
                  f32x4{kp[0].x, kp[1].x, kp[2].x, kp[3].x});
          st4<MT>(smem + L::XR, L::P_XC, xoff(DV + j + 1, r0 + 4 * r4),
                  f32x4{kp[0].y, kp[1].y, kp[2].y, kp[3].y});
        }
      }
      __syncthreads();

      // ================= D_I = (I + L_II)^{-1} by forward substitution (wave 0)
      if (wid == 0) {
        if (tid < 4) FLAGS[tid] = 0;  // read above; set again by the next item's prep 1
        const int I = g, cc = c16;
        const bool live = I < NB;
        const float* Lb = LBK + (live ? pidx(I, I) : 0) * BLKF;
        // right-looking: once x[m] is final it is subtracted from every later
        // row at once, so the dependent chain is one FMA per row
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.f : 0.f;
        fs_group<0, L::LDB>(Lb, x);
        fs_group<1, L::LDB>(Lb, x);
        fs_group<2, L::LDB>(Lb, x);
        fs_group<3, L::LDB>(Lb, x);
        if (live) {
          float* Tn = TBN + I * BLKF;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            Tn[r * L::LDB + cc] = x[r];
            st1<MT>(smem + L::TL, L::P_CC, (16 * I + r) * L::LDC + 16 * I + cc, x[r]);
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
          const bool ok = g < 2;
          Frag<MT> A = frag_f32<MT>(TBN + I * BLKF + c16 * L::LDB + 8 * (g & 1), ok);
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
    } else {
      // bf16: waves 0 .. NB-1 take the diagonal pairs (I, I) and form
      // D_I = (I + L_II)^{-1} right away; the other waves take the
      // off-diagonal pairs and keep their L_IJ in registers for
      // L'_IJ = D_I L_IJ after the barrier. L is formed as L[t][s]
      // (A = Kr_I, B = scaled Kc_J: the A and B lane layouts coincide), M as
      // M^T[s][t].
      constexpr int NOW = NW - NB;                           // waves of the off-diagonal pairs
      constexpr int MAXO = NQ > 0 ? (NQ + NOW - 1) / NOW : 1;
      static_assert(NB < NW, "one wave per diagonal block and at least one more");
      const bool dwave = wid < NB;
      float* LBD = (float*)(smem + L::LBD);
      // the fragments of a pair are read before the first product, so the
      // reads overlap; pairs with J = I - 1 have unit scale vectors
      auto gram = [&](int I, int J, f32x4& l, f32x4& m) {
        constexpr int KS = (DK + 31) / 32;
        const int p = pidx(I, J);
        const bool scaled = (I == J) || (I > J + 1);
        Frag<MM> A[KS], BL[KS], BM[KS];
        f32x4 sa[KS], sb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          A[ks] = ldfrag<MM>(smem + L::KC, L::P_CK, L::LDK, 16 * J, 32 * ks, DK, lane);
          BL[ks] = ldfrag<MM>(smem + L::KR, L::P_CK, L::LDK, 16 * I, 32 * ks, DK, lane);
          BM[ks] = ldfrag<MM>(smem + L::QR, L::P_CK, L::LDK, 16 * I, 32 * ks, DK, lane);
        }
        if (scaled) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            // slices past d_k (d_k = 16) are zero fragments: any finite scale
            const int kk = 32 * ks + 8 * g < DK ? 32 * ks + 8 * g : 0;
            sa[ks] = *(const f32x4*)(SCL + p * DK + kk);
            sb[ks] = *(const f32x4*)(SCL + p * DK + kk + 4);
          }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const float sv[8] = {sa[ks][0], sa[ks][1], sa[ks][2], sa[ks][3],
                                 sb[ks][0], sb[ks][1], sb[ks][2], sb[ks][3]};
            scale_frag<MM>(A[ks], sv);
          }
        }
        l = f4zero();
        m = f4zero();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          mma<MM>(l, BL[ks], A[ks]);
          mma<MM>(m, A[ks], BM[ks]);
        }
      };
      // M rows t = 16 I + c16, columns 16 J + 4g .. to the record
      auto store_m = [&](int I, int J, const f32x4& mv) {
        const int t = 16 * I + c16, s0 = 16 * J + 4 * g;
        RS.quad(RL.m + o_m(t, s0) * ES, mv);
        // F order: the scan multiplies M in 32-column slices up to the
        // diagonal, so the block right of an even diagonal block is zero
        if constexpr (FM) {
          if (I == J && (I & 1) == 0) RS.quad(RL.m + o_m(t, s0 + 16) * ES, f4zero());
        }
      };
      // waves past the off-diagonal pairs' full rounds have spare time in
      // the Gram phase
      constexpr int NLIGHT = NQ % NOW == 0 ? 0 : NOW - NQ % NOW;
      // Q_pi from its staging rows to the record: consecutive threads write
      // consecutive F-order pieces (US is free again before the solve)
      auto qpi_store = [&](int t0i, int nthr) {
        for (int idx = t0i; idx < CM * DK / 8; idx += nthr) {
          const int q2 = idx >> 6, t = 32 * (q2 / (DK / 16)) + (idx & 31),
                    pc = 2 * (q2 % (DK / 16)) + ((idx >> 5) & 1);
          RS.raw16(RL.qp + 16 * idx, *(const u32x4*)(smem + L::US + 2 * (t * L::LDU + 8 * pc)));
        }
      };
      if (dwave) {
        const int I = wid;
        f32x4 lv, mv;
        gram(I, I, lv, mv);
        const int t = 16 * I + cq, s0 = 16 * I + 4 * gq;
        // entry e is L[4g + e][c16]: strictly lower part only
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (cq >= 4 * gq + e) lv[e] = 0.f;
        if (FLAGS[I]) {
          // exact products, formed for row t = c16 and columns 4g .. 4g+3 (the
          // M layout), brought to the L layout through LDS
          float* Lb = LBD + I * BLKF;   // L_II [t][s], fp32
          f32x4 lx;
          exact_diag<Tin, DK, GATED>(k, bgate, q, alpha, seqK, t0, T, t, s0, lx, mv, gread);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (s0 + e >= t) lx[e] = 0.f;
          *(f32x4*)(Lb + c16 * L::LDB + 4 * g) = lx;
          wave_lds_sync();
#pragma unroll
          for (int e = 0; e < 4; ++e) lv[e] = Lb[(4 * g + e) * L::LDB + c16];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (s0 + e > t) mv[e] = 0.f;
        store_m(I, I, mv);
        // column cc of D_I by right-looking substitution; L[r][m] is entry
        // r % 4 of lane 16 (r / 4) + m, read as a wave-uniform scalar (every
        // lane group computes the column; group 0 writes it)
        // column cc of D_I by right-looking substitution over the rows of
        // L_II, staged in LDS and read as broadcast rows (every lane group
        // computes the column; group 0 writes it). Lane reads of the
        // accumulator instead would hold up to 15 scalars per step, and the
        // scalar registers they take cost more spills than the LDS round trip.
        const int cc = c16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.f : 0.f;
        {
          float* Lq = LBD + I * BLKF;
#pragma unroll
          for (int e = 0; e < 4; ++e) Lq[(4 * g + e) * L::LDB + c16] = lv[e];
          wave_lds_sync();
          fs_group<0, L::LDB>(Lq, x);
          fs_group<1, L::LDB>(Lq, x);
          fs_group<2, L::LDB>(Lq, x);
          fs_group<3, L::LDB>(Lq, x);
        }
        if (gq == 0) {
          float* Tn = TBN + I * BLKF;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            Tn[r * L::LDB + cc] = x[r];
            st1<MT>(smem + L::TL, L::P_CC, (16 * I + r) * L::LDC + 16 * I + cc, x[r]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < MAXO; ++i) {
          const int qq = (wid - NB) + NOW * i;
          if (qq < NQ) {
            int I, J;
            offpair_of(qq, I, J);
            f32x4 mv, lv;
            gram(I, J, lv, mv);
            store_m(I, J, mv);
            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
            *(bf16x4*)(smem + L::LT + 512 * qq + 8 * lane) =
                bf16x4{(__bf16)(-lv[0]), (__bf16)(-lv[1]), (__bf16)(-lv[2]), (__bf16)(-lv[3])};
          }
        }
        if constexpr (FM && NLIGHT > 0) {
          // the waves with one pair fewer store Q_pi here
          if (wid >= NW - NLIGHT) qpi_store(tid - 64 * (NW - NLIGHT), 64 * NLIGHT);
        }
      }
      __syncthreads();

      __syncthreads();
      // the last part of the next item's loads
      issue(nxt, 2);
      if (tid < 4) FLAGS[tid] = 0;   // read above; set again by the next item's prep 1
      if constexpr (FM && NLIGHT == 0) qpi_store(tid, kIntraThreads);
    }

    // ================= block forward substitution over all d_v + d_k columns:
    // X_I = D_I R_I - sum_{J<I} L'_IJ X_J. U^T and Y go to staging rows in LDS.
    auto stage_x = [&](int I, int ct, const f32x4& x) {
      if (16 * ct < DV) {
        if constexpr (FM) {
          // staged as U^T rows in LDS, stored in F order after the solve
          Out<Tin>::quad((Tin*)(smem + L::US) + (16 * ct + c16) * L::LDUT + 16 * I + 4 * g, x);
        } else {
          RS.quad(RL.ut + o_ut(16 * ct + c16, 16 * I + 4 * g) * ES, x);
        }
      } else {
        const int jj = 16 * ct - DV + c16;
#pragma unroll
        for (int e = 0; e < 4; ++e) YS[(16 * I + 4 * g + e) * L::LDY + jj] = (Tin)x[e];
      }
    };
    if constexpr (MT == kBF) {
      // bf16 operands: the solved blocks stay in registers. A 32-wide k step
      // over blocks (J0, J1) = (2p, 2p + 1) takes, in lane group g, the rows
      // 4g .. 4g+3 of J0 and then of J1: exactly the accumulator entries a
      // lane holds for X_J0 and X_J1 of its column, so a solved block feeds
      // the next products without a trip through LDS. The rows of [-L' | D]
      // in TL are read with their columns in the same order.
      typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
      const bf16x4 z4 = bf16x4{};
      const __bf16* TLb = (const __bf16*)(smem + L::TL);
      const __bf16* XRb = (const __bf16*)(smem + L::XR);
      // lane indices through an empty asm: the operand addresses below are
      // formed here rather than hoisted out of the item loop, where they
      // would hold registers across every phase
      int sr = c16, sg = g;
      asm volatile("" : "+v"(sr), "+v"(sg));
      bf16x4 X[NB][MAXX];
      // every operand read up front (none of them depends on the solve): the
      // right-hand sides, D_I (rows of the diagonal blocks of TL), and
      // -L'_IJ for J < I, formed here by every wave as (L'_IJ)^T = L_IJ^T D_I^T
      // from -L_IJ in accumulator lane order (the A operand as it stands) and
      // rows of D_I: the product lands in lane (g, m) as row m, columns
      // 4g .. 4g+3 of -L'_IJ, which is this step's A operand layout
      bf16x4 DI[NB], Lp[NB][NB], RHs[NB][MAXX];
      const int sl = 16 * sg + sr;
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        DI[I] = *(const bf16x4*)(TLb + (16 * I + sr) * L::LDC + 16 * I + 4 * sg);
#pragma unroll
        for (int i = 0; i < MAXX; ++i) {
          const int ct = wid + NW * i;
          RHs[I][i] = ct < NX ? *(const bf16x4*)(XRb + xoff(16 * ct + sr, 16 * I + 4 * sg)) : z4;
        }
      }
#pragma unroll
      for (int I = 1; I < NB; ++I) {
        const f32x4 d4 = *(const f32x4*)(TBN + I * BLKF + sr * L::LDB + 4 * sg);
        const bf16x8 Bd = bf16x8{(__bf16)d4[0], (__bf16)d4[1], (__bf16)d4[2], (__bf16)d4[3],
                                 (__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
#pragma unroll
        for (int J = 0; J < I; ++J) {
          const bf16x4 lt = *(const bf16x4*)(smem + L::LT + 512 * (I * (I - 1) / 2 + J) + 8 * sl);
          const f32x4 pr = mfma_bf16(__builtin_shufflevector(lt, z4, 0, 1, 2, 3, 4, 5, 6, 7), Bd, f4zero());
          Lp[I][J] = bf16x4{(__bf16)pr[0], (__bf16)pr[1], (__bf16)pr[2], (__bf16)pr[3]};
        }
      }
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        const bf16x4* RH = RHs[I];
        f32x4 acc[MAXX];
#pragma unroll
        for (int i = 0; i < MAXX; ++i) acc[i] = f4zero();
#pragma unroll
        for (int pp = 0; 2 * pp <= I; ++pp) {
          const int J0 = 2 * pp, J1 = 2 * pp + 1;
          const bf16x4 a0 = J0 < I ? Lp[I][J0] : DI[I];
          const bf16x4 a1 = J1 < I ? Lp[I][J1] : (J1 == I ? DI[I] : z4);
          const bf16x8 A = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int i = 0; i < MAXX; ++i) {
            if (wid + NW * i < NX) {
              const bf16x4 b0 = J0 < I ? X[J0][i] : RH[i];
              const bf16x4 b1 = J1 < I ? X[J1][i] : (J1 == I ? RH[i] : z4);
              acc[i] = mfma_bf16(A, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), acc[i]);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < MAXX; ++i) {
          const int ct = wid + NW * i;
          if (ct < NX) {
            X[I][i] = bf16x4{(__bf16)acc[i][0], (__bf16)acc[i][1], (__bf16)acc[i][2], (__bf16)acc[i][3]};
            stage_x(I, ct, acc[i]);
          }
        }
      }
    } else {
      // fp32 operands: in place in XR, one block row after the other
      for (int I = 0; I < NB; ++I) {
        const int kend = 16 * (I + 1);
        f32x4 acc[MAXX];
#pragma unroll
        for (int i = 0; i < MAXX; ++i) acc[i] = f4zero();
#pragma unroll
        for (int k0 = 0; k0 < CM; k0 += 32) {
          if (k0 < kend) {
            Frag<MT> A = ldfrag<MT>(smem + L::TL, L::P_CC, L::LDC, 16 * I, k0, kend, lane);
#pragma unroll
            for (int i = 0; i < MAXX; ++i) {
              const int ct = wid + NW * i;
              if (ct < NX) {
                // rows 16ct + c16 share the slot swizzle ct & XM
                const int kk = k0 + 8 * g;
                Frag<MT> B = ldfrag<MT>(smem + L::XR, L::P_XC, L::LDC, 16 * ct,
                                        8 * ((kk >> 3) ^ (ct & XM)) - 8 * g, kk < kend ? CM : 0, lane);
                mma<MT>(acc[i], A, B);
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < MAXX; ++i) {
          const int ct = wid + NW * i;
          if (ct < NX) {
            st4<MT>(smem + L::XR, L::P_XC, xoff(16 * ct + c16, 16 * I + 4 * g), acc[i]);
            stage_x(I, ct, acc[i]);
          }
        }
        wave_lds_sync();
      }
    }
    __syncthreads();

    // ================= Y rows to the record (16-byte pieces)
    constexpr int YPR = DK * (int)sizeof(Tin) / 16;  // 16-byte pieces per row
    for (int idx = tid; idx < CM * YPR; idx += kIntraThreads) {
      if constexpr (FM) {
        // consecutive threads write consecutive F-order pieces
        static_assert(!FM || sizeof(Tin) == 2, "F order is bf16");
        const int q2 = idx >> 6, t = 32 * (q2 / (DK / 16)) + (idx & 31), pc = 2 * (q2 % (DK / 16)) + ((idx >> 5) & 1);
        RS.raw16(RL.y + 16 * idx, *(const u32x4*)((const char*)(YS + t * L::LDY) + 16 * pc));
      } else {
        const int t = idx / YPR, pc = idx % YPR;
        RS.raw16(RL.y + o_tk(t, 16 * pc / ES) * ES, *(const u32x4*)((const char*)(YS + t * L::LDY) + 16 * pc));
      }
    }
    if constexpr (FM) {
      // U^T in F order: each 32-byte lane slot holds t = 32*i2 + 8q + 4*hh + e
      // of column v = 32*vt + l%32 (entry 4q + e): four 8-byte runs of a US row
      typedef __attribute__((ext_vector_type(2))) uint32_t u2;
      const char* USb = smem + L::US;
      const int nslots = (DV / 32) * (CM / 32) * 64;
      for (int sidx = tid; sidx < nslots; sidx += kIntraThreads) {
        const int ln = sidx & 63, blk = sidx >> 6;
        const int vv = 32 * (blk / (CM / 32)) + (ln & 31), tb = 32 * (blk % (CM / 32)) + 4 * (ln >> 5);
        const char* row = USb + 2 * (vv * L::LDUT + tb);
        const u2 a0 = *(const u2*)(row), a1 = *(const u2*)(row + 16), a2 = *(const u2*)(row + 32),
                 a3 = *(const u2*)(row + 48);
        RS.raw16(RL.ut + 32 * sidx, u32x4{a0.x, a0.y, a1.x, a1.y});
        RS.raw16(RL.ut + 32 * sidx + 16, u32x4{a2.x, a2.y, a3.x, a3.y});
      }
    }
  }
}

// ============================================================================ scan kernel
constexpr int kScanThreads = 512;

// One 8-element operand slice of a k-contiguous record matrix (global memory),
// loaded unconditionally (from `safe` when the slice lies outside the matrix).
// Padding slices are zeroed where the operand is used (zsel): branch-free
// loads with no use until then let the compiler count outstanding loads
// exactly, so a prefetch is not waited for early.
template <int MODE, typename E>
__device__ __forceinline__ Frag<MODE> gfrag(const E* p, const E* safe, bool valid) {
  const E* a = valid ? p : safe;
  Frag<MODE> f;
  if constexpr (MODE == kF32) {
    f.a = *(const f32x4*)a;
    f.b = *(const f32x4*)(a + 4);
  } else {
    f.hi = *(const bf16x8*)a;
  }
  return f;
}

template <int MODE>
__device__ __forceinline__ Frag<MODE> zsel(bool valid, const Frag<MODE>& x) {
  if (valid) return x;
  Frag<MODE> z;
  if constexpr (MODE == kF32) {
    z.a = f4zero();
    z.b = f4zero();
  } else {
    z.hi = bf16x8{};
  }
  return z;
}

template <typename Tin, int DK, int VT, int CM>
__global__ __launch_bounds__(kScanThreads, 1) void gdn2_chunk_scan_kernel(
    const char* __restrict__ ws, const float* __restrict__ S0, Tin* __restrict__ o, float* S_out,
    int T, int DV) {
  constexpr bool F32 = std::is_same<Tin, float>::value;
  constexpr int MM = F32 ? kF32 : kBF;
  constexpr int NW = kScanThreads / 64;
  constexpr int NVL = VT / 16;
  constexpr int NST = (DK / 16) * NVL;              // S tiles (j-block, value block)
  constexpr int MAXS = (NST + NW - 1) / NW;
  constexpr int NT = (CM / 16) * NVL;               // V~ / O tiles (t-block, value block)
  constexpr int MAXV = (NT + NW - 1) / NW;
  constexpr int KS = DK >= 32 ? DK / 32 : 1;        // 32-wide k steps over d_k
  constexpr int KSC = CM >= 32 ? CM / 32 : 1;       // 32-wide k steps over the chunk
  constexpr int LDK = DK + 8, LDC = CM + 8;
  constexpr int NSP = F32 ? 2 : 1;
  constexpr int P_VK = VT * LDK * 2, P_VC = VT * LDC * 2;
  __shared__ __attribute__((aligned(16))) char smem[NSP * (P_VK + P_VC)];
  char* S0T = smem;                                 // S0^T  [v][j]
  char* VTT = smem + NSP * P_VK;                    // V~^T  [v][t]

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nvt = DV / VT;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int bh = lin / nvt, vt0 = (lin % nvt) * VT;
  const int nchunks = (T + CM - 1) / CM;
  const size_t stOff = (size_t)bh * DK * DV;
  const RecLayout RL = rec_layout(DK, DV, CM, sizeof(Tin));
  const char* wsh = ws + (size_t)bh * nchunks * RL.bytes;

  // ---- state tile in registers (fp32), S0^T in LDS
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
      st4<MM>(S0T, P_VK, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[i]);
    }
  }

  // ---- per-chunk operand fragments. V~/O tile i of this wave is (t-block I,
  // value block vl); S tile i is (j-block jt, value block vl).
  struct Ops {
    Frag<MM> y[MAXV][KS];    // Y rows t (A of Y S0)
    Frag<MM> qp[MAXV][KS];   // Q_pi rows t (B of S0^T Q_pi^T)
    Frag<MM> m[MAXV][KSC];   // M rows t (B of V~^T M^T)
    typename Raw<Tin>::R4 u[MAXV];  // U[t..t+3][v] from U^T, undecoded until use
    Frag<MM> kt[MAXS][KSC];  // K~^T rows j (A of K~^T V~)
    f32x4 pc[MAXS];          // pi_C[j..j+3]
  };
  auto fetch = [&](int ch, Ops& x) {
    const char* rec = wsh + (size_t)ch * RL.bytes;
    const Tin* Yp = (const Tin*)(rec + RL.y);
    const Tin* UTp = (const Tin*)(rec + RL.ut);
    const Tin* Mp = (const Tin*)(rec + RL.m);
    const Tin* QPp = (const Tin*)(rec + RL.qp);
    const Tin* KTp = (const Tin*)(rec + RL.kt);
    const float* PCp = (const float*)(rec + RL.pic);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int tile = wid + NW * i;
      const bool ok = tile < NT;
      const int I = ok ? tile / NVL : 0, vl = ok ? tile % NVL : 0;
      const int t = 16 * I + c16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int kk = 32 * s + 8 * g;
        x.y[i][s] = gfrag<MM>(Yp + t * DK + kk, Yp, ok && kk < DK);
        x.qp[i][s] = gfrag<MM>(QPp + t * DK + kk, QPp, ok && kk < DK);
      }
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        const int kk = 32 * s + 8 * g;
        x.m[i][s] = gfrag<MM>(Mp + t * CM + kk, Mp, ok && kk < 16 * (I + 1));
      }
      const Tin* up = UTp + (vt0 + 16 * vl + c16) * CM + 16 * I + 4 * g;
      x.u[i] = Raw<Tin>::ld4(up);                          // unused when !ok (then I = vl = 0)
    }
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + NW * i;
      const bool ok = tile < NST;
      const int jt = ok ? tile / NVL : 0;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        const int kk = 32 * s + 8 * g;
        x.kt[i][s] = gfrag<MM>(KTp + (16 * jt + c16) * CM + kk, KTp, ok && kk < CM);
      }
      x.pc[i] = *(const f32x4*)(PCp + 16 * jt + 4 * g);   // jt = 0 when unused
    }
  };

  // one chunk: V~ = U - Y S0 -> V~^T (LDS) and O^T = S0^T Q_pi^T; then
  // O^T += V~^T M^T, store O; S <- Diag(pi_C) S + K~^T V~, S^T -> LDS
  auto step = [&](int ch, const Ops& cur) {
    const int t0 = ch * CM;
    f32x4 oacc[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      oacc[i] = f4zero();
      const int tile = wid + NW * i;
      if (tile < NT) {
        const int I = tile / NVL, vl = tile % NVL;
        f32x4 acc = f4zero();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          Frag<MM> Sf = ldfrag<MM>(S0T, P_VK, LDK, 16 * vl, 32 * s, DK, lane);
          const bool kv = 32 * s + 8 * g < DK;
          mma<MM>(acc, zsel<MM>(kv, cur.y[i][s]), Sf);      // rows t, cols v
          mma<MM>(oacc[i], Sf, zsel<MM>(kv, cur.qp[i][s])); // rows v, cols t
        }
        // acc[e] = (Y S0)[16I + 4g + e][16vl + c16]; u[e] = U[16I + 4g + e][16vl + c16]
        const f32x4 u = Raw<Tin>::un4(cur.u[i]);
        f32x4 vt;
#pragma unroll
        for (int e = 0; e < 4; ++e) vt[e] = u[e] - acc[e];
        st4<MM>(VTT, P_VC, (16 * vl + c16) * LDC + 16 * I + 4 * g, vt);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int tile = wid + NW * i;
      if (tile < NT) {
        const int I = tile / NVL, vl = tile % NVL, kend = 16 * (I + 1);
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
          if (32 * s < kend) {
            Frag<MM> A = ldfrag<MM>(VTT, P_VC, LDC, 16 * vl, 32 * s, kend, lane);
            mma<MM>(oacc[i], A, zsel<MM>(32 * s + 8 * g < kend, cur.m[i][s]));
          }
        }
        // oacc[e] = O[t = 16I + c16][v = 16vl + 4g + e]
        const int t = t0 + 16 * I + c16;
        if (t < T) In<Tin>::store4(o + ((size_t)bh * T + t) * DV + vt0 + 16 * vl + 4 * g, oacc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + NW * i;
      if (tile < NST) {
        const int jt = tile / NVL, vl = tile % NVL;
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[i][e] *= cur.pc[i][e];
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
          Frag<MM> B = ldfrag<MM>(VTT, P_VC, LDC, 16 * vl, 32 * s, CM, lane);
          mma<MM>(Sacc[i], zsel<MM>(32 * s + 8 * g < CM, cur.kt[i][s]), B);
        }
        st4<MM>(S0T, P_VK, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[i]);
      }
    }
    __syncthreads();
  };

  if constexpr (F32) {
    // fp32 operands take twice the registers: no prefetch
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
      Ops cur;
      fetch(ch, cur);
      step(ch, cur);
    }
  } else {
    // two operand sets used in turn (no register copies), each filled one
    // chunk ahead of its use
    Ops opA, opB;
    fetch(0, opA);
    __syncthreads();
    for (int ch = 0; ch < nchunks; ch += 2) {
      if (ch + 1 < nchunks) fetch(ch + 1, opB);
      step(ch, opA);
      if (ch + 1 >= nchunks) break;
      if (ch + 2 < nchunks) fetch(ch + 2, opA);
      step(ch + 1, opB);
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

// ============================================================================ staged scan kernel (bf16)
// The same chunk pass as gdn2_chunk_scan_kernel with the record slice of each
// chunk (Y, Q_pi, M, K~^T, pi_C and this workgroup's U^T rows) loaded once per
// workgroup with 16-byte coalesced loads, two chunks ahead, into two register
// sets used in turn; at the end of a chunk the set holding the next chunk is
// written to one of two LDS stages, from which every MFMA operand is read.
// Rows of a staged matrix keep their global byte layout up to an XOR swizzle
// of their 16-byte slots (slot ^ swz(row)), which makes both the row-wise
// stores and the 16-row fragment reads free of bank conflicts.
template <int DK, int VT, int CM>
struct StagedScan {
  static constexpr int WY = DK * 2, WC = CM * 2;   // row bytes of [.][DK] and [.][C] bf16 matrices
  static constexpr int Y = 0;                       // Y      [t][j]
  static constexpr int QP = Y + CM * WY;            // Q_pi   [t][j]
  static constexpr int M = QP + CM * WY;            // M      [t][s]
  static constexpr int KT = M + CM * WC;            // K~^T   [j][s]
  static constexpr int UT = KT + DK * WC;           // U^T    [v][t], this workgroup's VT rows
  static constexpr int PC = UT + VT * WC;           // pi_C   fp32 [j]
  static constexpr int STAGE = (PC + DK * 4 + 15) / 16 * 16;
  static constexpr int LDK = DK + 8, LDC = CM + 8;
  static constexpr int S0T = 2 * STAGE;             // S0^T  [v][j] bf16
  static constexpr int VTT = S0T + VT * LDK * 2;    // V~^T  [v][t] bf16
  static constexpr int TOTAL = VTT + VT * LDC * 2;
  static_assert(TOTAL <= 160 * 1024, "staged scan LDS exceeds 160 KiB");
  // 16-byte pieces of one stage, in load order
  static constexpr int NY = CM * WY / 16, NU = VT * WC / 16, NM = CM * WC / 16, NK = DK * WC / 16;
  static constexpr int NPC = DK * 4 / 16;
  static constexpr int B_Y = 0, B_U = B_Y + NY, B_M = B_U + NU, B_Q = B_M + NM, B_K = B_Q + NY;
  static constexpr int B_P = B_K + NK, NPIECE = B_P + NPC;
};

// Slot swizzle of a row with n 16-byte slots (n = 2, 4, 8 or 16): rows that
// are 16 apart in a fragment read land on distinct bank groups.
__device__ __forceinline__ int swz(int r, int n) { return (r / (16 / n)) % n; }

template <int DK, int VT, int CM>
__global__ __launch_bounds__(kScanThreads, 1) void gdn2_chunk_scan_staged_kernel(
    const char* __restrict__ ws, const float* __restrict__ S0, __bf16* __restrict__ o, float* S_out,
    int T, int DV) {
  using L = StagedScan<DK, VT, CM>;
  constexpr int MM = kBF;
  constexpr int NW = kScanThreads / 64;
  constexpr int NVL = VT / 16;
  constexpr int NST = (DK / 16) * NVL;
  constexpr int MAXS = (NST + NW - 1) / NW;
  constexpr int NT = (CM / 16) * NVL;
  constexpr int MAXV = (NT + NW - 1) / NW;
  constexpr int KS = DK >= 32 ? DK / 32 : 1;
  constexpr int KSC = CM >= 32 ? CM / 32 : 1;
  constexpr int NPT = (L::NPIECE + kScanThreads - 1) / kScanThreads;  // pieces per thread
  constexpr int LDK = L::LDK, LDC = L::LDC;
  constexpr int P_VK = VT * LDK * 2, P_VC = VT * LDC * 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* S0T = smem + L::S0T;
  char* VTT = smem + L::VTT;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nvt = DV / VT;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int bh = lin / nvt, vt0 = (lin % nvt) * VT;
  const int nchunks = (T + CM - 1) / CM;
  const size_t stOff = (size_t)bh * DK * DV;
  const RecLayout RL = rec_layout(DK, DV, CM, 2);
  const char* wsh = ws + (size_t)bh * nchunks * RL.bytes;

  // ---- the pieces this thread moves: global byte offset in a record, LDS byte offset in a stage
  int gof[NPT], lof[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    int p = tid + kScanThreads * i;
    if (p >= L::NPIECE) p = L::NPIECE - 1;           // duplicate of the last piece (same value)
    int g0, l0, q, w, base_l;
    bool rowsw = true;
    if (p < L::B_U) { q = p - L::B_Y; w = L::WY; g0 = RL.y; base_l = L::Y; }
    else if (p < L::B_M) { q = p - L::B_U; w = L::WC; g0 = RL.ut + vt0 * L::WC; base_l = L::UT; }
    else if (p < L::B_Q) { q = p - L::B_M; w = L::WC; g0 = RL.m; base_l = L::M; }
    else if (p < L::B_K) { q = p - L::B_Q; w = L::WY; g0 = RL.qp; base_l = L::QP; }
    else if (p < L::B_P) { q = p - L::B_K; w = L::WC; g0 = RL.kt; base_l = L::KT; }
    else { q = p - L::B_P; w = DK * 4; g0 = RL.pic; base_l = L::PC; rowsw = false; }
    const int n = w / 16, r = q / n, c = q % n;
    gof[i] = g0 + r * w + 16 * c;
    l0 = base_l + r * w + 16 * (rowsw ? (c ^ swz(r, n)) : c);
    lof[i] = l0;
  }
  auto load = [&](int ch, u32x4* R) {
    const char* rec = wsh + (size_t)(ch < nchunks ? ch : nchunks - 1) * RL.bytes;
#pragma unroll
    for (int i = 0; i < NPT; ++i) R[i] = *(const u32x4*)(rec + gof[i]);
  };
  auto stage = [&](const u32x4* R, int st) {
    char* base = smem + st * L::STAGE;
#pragma unroll
    for (int i = 0; i < NPT; ++i) *(u32x4*)(base + lof[i]) = R[i];
  };
  // fragment of a staged row-major matrix: rows row0 + c16, 8 elements from k0 + 8g
  auto sfrag = [&](const char* stg, int moff, int w, int row0, int k0) {
    const int n = w / 16, r = row0 + c16, c = ((k0 >> 3) + g) & (n - 1);
    Frag<MM> f;
    f.hi = *(const bf16x8*)(stg + moff + r * w + 16 * (c ^ swz(r, n)));
    return f;
  };

  // ---- state tile in registers (fp32), S0^T in LDS
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
      st4<MM>(S0T, P_VK, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[i]);
    }
  }

  auto compute = [&](int ch, const char* stg) {
    const int t0 = ch * CM;
    f32x4 oacc[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      oacc[i] = f4zero();
      const int tile = wid + NW * i;
      if (tile < NT) {
        const int I = tile / NVL, vl = tile % NVL;
        f32x4 acc = f4zero();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bool kv = 32 * s + 8 * g < DK;
          Frag<MM> Sf = ldfrag<MM>(S0T, P_VK, LDK, 16 * vl, 32 * s, DK, lane);
          mma<MM>(acc, zsel<MM>(kv, sfrag(stg, L::Y, L::WY, 16 * I, 32 * s)), Sf);
          mma<MM>(oacc[i], Sf, zsel<MM>(kv, sfrag(stg, L::QP, L::WY, 16 * I, 32 * s)));
        }
        // U[t = 16I + 4g + e][v = 16vl + c16] from U^T row v: 8 bytes in slot 2I + g/2
        const int vr = 16 * vl + c16, uc = 2 * I + (g >> 1);
        typedef __attribute__((ext_vector_type(2))) uint32_t u2;
        const u2 uw = *(const u2*)(stg + L::UT + vr * L::WC + 16 * (uc ^ swz(vr, L::WC / 16)) + 8 * (g & 1));
        const f32x4 u = Raw<__bf16>::un4(uw);
        f32x4 vt;
#pragma unroll
        for (int e = 0; e < 4; ++e) vt[e] = u[e] - acc[e];
        st4<MM>(VTT, P_VC, (16 * vl + c16) * LDC + 16 * I + 4 * g, vt);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int tile = wid + NW * i;
      if (tile < NT) {
        const int I = tile / NVL, vl = tile % NVL, kend = 16 * (I + 1);
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
          if (32 * s < kend) {
            Frag<MM> A = ldfrag<MM>(VTT, P_VC, LDC, 16 * vl, 32 * s, kend, lane);
            mma<MM>(oacc[i], A, zsel<MM>(32 * s + 8 * g < kend, sfrag(stg, L::M, L::WC, 16 * I, 32 * s)));
          }
        }
        const int t = t0 + 16 * I + c16;
        if (t < T) In<__bf16>::store4(o + ((size_t)bh * T + t) * DV + vt0 + 16 * vl + 4 * g, oacc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int tile = wid + NW * i;
      if (tile < NST) {
        const int jt = tile / NVL, vl = tile % NVL;
        const f32x4 pc = *(const f32x4*)(stg + L::PC + 4 * (16 * jt + 4 * g));
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[i][e] *= pc[e];
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
          Frag<MM> B = ldfrag<MM>(VTT, P_VC, LDC, 16 * vl, 32 * s, CM, lane);
          mma<MM>(Sacc[i], zsel<MM>(32 * s + 8 * g < CM, sfrag(stg, L::KT, L::WC, 16 * jt, 32 * s)), B);
        }
        st4<MM>(S0T, P_VK, (16 * vl + c16) * LDK + 16 * jt + 4 * g, Sacc[i]);
      }
    }
  };

  // ---- pipeline: register set R0 holds even chunks, R1 odd ones; loads are
  // unconditional (past the end they repeat the last chunk) so the compiler
  // can count outstanding loads exactly
  u32x4 R0[NPT], R1[NPT];
  load(0, R0);
  load(1, R1);
  stage(R0, 0);
  __syncthreads();
  load(2, R0);
  for (int ch = 0; ch < nchunks; ch += 2) {
    compute(ch, smem);
    stage(R1, 1);
    __syncthreads();
    load(ch + 3, R1);
    if (ch + 1 >= nchunks) break;
    compute(ch + 1, smem + L::STAGE);
    stage(R0, 0);
    __syncthreads();
    load(ch + 4, R0);
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

// ============================================================================ F-order scan
// The chunk pass of the scan kernels above for a bf16 record in F order, with
// 32x32x16 MFMAs: one workgroup of ten waves per (b, h, 32 value columns).
// Each record operand has a single consumer wave, so every wave loads its own
// fragments straight from the record into registers (1 KiB coalesced per
// slice); only S0, V~ and a partial O pass through LDS. Two barriers split a
// chunk into phase 1 and phase 2, and every wave computes in one phase and
// reloads its registers (for a later chunk) in the other: a load can stall
// its wave at issue while the memory pipeline is busy, and that way the stall
// holds up no other wave.
//   V,  waves 0-1 (I2 = w):    phase 1  V~ rows t = 32*I2.. = U - Y S0 -> LDS (as V~^T)
//   O1, waves 2-3 (I2 = w-2):  phase 1  P = S0^T Q_pi^T -> LDS (fp32)
//   O2, waves 4-5 (I2 = w-4):  phase 2  O^T = P + V~^T M^T, stored
//   S,  waves 6-9 (J2 = w-6):  phase 2  state rows 32*J2..: S = Diag(pi_C) S + K~^T V~ -> LDS
// The S waves also touch the record PF chunks ahead so that the other loads
// hit L2. 32x32x16 lane layout (l = 32h + r): A[m = r][k = 8h + i],
// B[k = 8h + i][n = r], accumulator entry 4q + e = D[m = 8q + 4h + e][n = r].
typedef __attribute__((ext_vector_type(16))) float f32x16;
constexpr int kScanFmWaves = 10;
constexpr int kScanFmThreads = 64 * kScanFmWaves;
constexpr int kSegTargetUnits = 256;  // scan workgroups the segmented scan aims for (one per CU)
constexpr int kScanFmPrefetch = 3;   // chunks ahead that the record is pulled into L2
constexpr int kScanFmSets = 3;       // register sets per wave: loads run NS - 1 chunks ahead

__device__ __forceinline__ f32x16 mma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <int N> struct Ic { static constexpr int value = N; };
__device__ __forceinline__ f32x16 f16zero() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
// Workgroup barrier that the compiler may not schedule anything across, so
// each phase keeps its own instructions.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// Sequence segments: with seg < the chunk count, the chunks of a head are
// split into segments of seg chunks, one workgroup per (b, h, segment, value
// tile), and segment g starts from the state Sseg[g][b*H + h] that the
// segment pass left there (g = 0: S0); only the last segment writes S_out.
// With seg >= the chunk count there is one segment, starting from S0.
// OUT_H: every chunk-start state goes to Hst, fp32 [b*H + h][chunk][d_k][d_v]
// (the backward's saved states); without OUT_O no outputs are stored. Both
// are compile-time choices: a run-time branch around the stores would leave
// the compiler unable to count the loads in flight, and it would then wait
// for all of them.
template <int DK, int CM, int PF, int NS, bool OUT_O = true, bool OUT_H = false>
__global__ __launch_bounds__(kScanFmThreads, 1) void gdn2_chunk_scan_fm_kernel(
    const char* __restrict__ ws, const float* __restrict__ S0, __bf16* __restrict__ o, float* S_out,
    int T, int DV, int seg, const float* __restrict__ Sseg, float* __restrict__ Hst) {
  constexpr int NI2 = CM / 32, NJ2 = DK / 32, KSD = DK / 16, KSC = CM / 16;
  constexpr int LDK = DK + 8, LDC = CM + 8;      // LDS row pitches (elements): 16-byte reads conflict free
  static_assert(DK % 32 == 0 && CM % 32 == 0 && NJ2 <= 4 && NI2 <= 2, "F-order scan shape");
  __shared__ __attribute__((aligned(16))) __bf16 S0T[32 * LDK];   // S0^T [v][j] (bf16 copy of the state)
  __shared__ __attribute__((aligned(16))) __bf16 VTT[32 * LDC];   // V~^T [v][t]
  __shared__ __attribute__((aligned(16))) f32x4 OP[2][4][64];     // partial O^T per row block, per lane

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r = lane & 31;
  const int nvt = DV / 32;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, nvt);
  const int ntot = (T + CM - 1) / CM;                  // chunks of the sequence
  const int nseg = (ntot + seg - 1) / seg;
  const int unit = lin / nvt, vt = lin % nvt, vt0 = 32 * vt;
  const int bh = unit / nseg, sg = unit % nseg;
  const int c0 = sg * seg;                             // first chunk of this segment
  const int nchunks = ntot - c0 < seg ? ntot - c0 : seg;
  const size_t stOff = (size_t)bh * DK * DV;
  // start state: S0 (or zero) for one segment, else this segment's slot
  const float* S0w = nseg == 1 ? S0 : Sseg + ((size_t)sg * (gridDim.x / (nvt * nseg)) + bh) * DK * DV;
  float* S_outw = sg == nseg - 1 ? S_out : nullptr;
  const RecLayout RL = rec_layout(DK, DV, CM, 2);
  const char* wsh = ws + ((size_t)bh * ntot + c0) * RL.bytes;
  // the records of this head through a buffer resource; the wave-uniform
  // part of each offset goes in the scalar offset, past the last chunk the
  // loads repeat it
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wsh), 0, nchunks * RL.bytes, 0x00020000);
  auto ld16 = [&](int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff, soff, 0));
  };
  auto cbase = [&](int ch) { return (ch < nchunks ? ch : nchunks - 1) * RL.bytes; };
  const int l16 = lane * 16;
  auto s0frag = [&](int s) { return *(const u32x4*)(S0T + r * LDK + 16 * s + 8 * h); };
  auto vfrag = [&](int s) { return *(const u32x4*)(VTT + r * LDC + 16 * s + 8 * h); };
  // Each role walks all chunks with two barriers per chunk. Its loop is
  // unrolled by hand over the register sets (every set keeps its registers)
  // and has a single exit (so the compiler's wait counts stay exact), with the
  // leftover chunks after it.
  static_assert(NS == 3 && PF == 3, "the role loops below are unrolled for three register sets");
  auto walk = [&](auto&& step) {
    int ch = 0;
    for (; ch + 3 <= nchunks; ch += 3) {
      step(ch, Ic<0>{});
      step(ch + 1, Ic<1>{});
      step(ch + 2, Ic<2>{});
    }
    if (ch < nchunks) step(ch, Ic<0>{});
    if (ch + 1 < nchunks) step(ch + 1, Ic<1>{});
  };

  if (wid < 2) {
    // ================= V: V~ = U - Y S0, rows t = 32*I2 .., to V~^T in LDS
    const int I2 = wid;
    const bool live = NI2 >= 2 || I2 < NI2;
    const int b_y = RL.y + I2 * KSD * 1024, b_u = RL.ut + (vt * NI2 + I2) * 2048;
    constexpr int NPV = KSD + 2;
    u32x4 R[NS][NPV];
    auto load = [&](int ch, u32x4* X) {
      const int cb = cbase(ch);
#pragma unroll
      for (int s = 0; s < KSD; ++s) X[s] = ld16(l16, cb + b_y + 1024 * s);
#pragma unroll
      for (int s = 0; s < 2; ++s) X[KSD + s] = ld16(lane * 32, cb + b_u + 16 * s);
    };
    __syncthreads();                                    // S0^T written
    __builtin_amdgcn_s_waitcnt(0);   // nothing outstanding: keeps merged code from loosening the counts below
    if (live) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        load(u, R[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      if (live) {
        f32x16 acc = f16zero();
#pragma unroll
        for (int s = 0; s < KSD; ++s) acc = mma32(R[u][s], s0frag(s), acc);
        // entry 4q + e is (t = 32 I2 + 8q + 4h + e, v = r): four consecutive t
        typedef __attribute__((ext_vector_type(2))) uint32_t u2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4& up = R[u][KSD + (q >> 1)];
          const f32x4 uu = Raw<__bf16>::un4(u2{up[2 * (q & 1)], up[2 * (q & 1) + 1]});
          In<__bf16>::store4(VTT + r * LDC + 32 * I2 + 8 * q + 4 * h,
                             f32x4{uu[0] - acc[4 * q], uu[1] - acc[4 * q + 1], uu[2] - acc[4 * q + 2],
                                   uu[3] - acc[4 * q + 3]});
        }
      }
      phase_barrier();                                  // A: V~ ready
      // the set just used, for chunk ch + NS
      if (live) load(ch + NS, R[u]);
      phase_barrier();                                  // B: S0 ready
    });
  } else if (wid < 4) {
    // ================= O1: P = S0^T Q_pi^T, rows t = 32*I2 ..
    const int I2 = wid - 2;
    const bool live = NI2 >= 2 || I2 < NI2;
    const int b_q = RL.qp + I2 * KSD * 1024;
    u32x4 RQ[NS][KSD];
    auto load = [&](int ch, u32x4* X) {
      const int cb = cbase(ch);
#pragma unroll
      for (int s = 0; s < KSD; ++s) X[s] = ld16(l16, cb + b_q + 1024 * s);
    };
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);
    if (live) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        load(u, RQ[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      if (live) {
        f32x16 acc = f16zero();
#pragma unroll
        for (int s = 0; s < KSD; ++s) acc = mma32(s0frag(s), RQ[u][s], acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) OP[I2][q][lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      }
      phase_barrier();                                  // A
      if (live) load(ch + NS, RQ[u]);
      phase_barrier();                                  // B
    });
  } else if (wid < 6) {
    // ================= O2: O^T = P + V~^T M^T, rows t = 32*I2 .., stored
    auto run = [&](auto Ic2) {
      constexpr int I2 = decltype(Ic2)::value;
      constexpr int NM = 2 * (I2 + 1) < KSC ? 2 * (I2 + 1) : KSC;   // M slices up to the diagonal
      const int b_m = RL.m + I2 * KSC * 1024;
      // O of this head from the chunk's first row to row T through a buffer
      // resource: rows past T are dropped by the hardware. Lane l stores row
      // t0 + 32 I2 + l % 32, columns vt0 + 8q + 4h ..
      const int oct = ((32 * I2 + r) * DV + vt0 + 4 * h) * 2;
      u32x4 RM[NS][NM];
      auto load = [&](int ch, u32x4* X) {
        const int cb = cbase(ch);
#pragma unroll
        for (int s = 0; s < NM; ++s) X[s] = ld16(l16, cb + b_m + 1024 * s);
      };
      __syncthreads();
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int u = 0; u < NS - 1; ++u) {
        load(u, RM[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
      walk([&](int ch, auto Uc) {
        constexpr int u = decltype(Uc)::value;
        // phase 1 is idle here: reload the set the previous chunk used, for
        // chunk ch + NS - 1
        load(ch + NS - 1, RM[(u + NS - 1) % NS]);
        phase_barrier();                                // A
        f32x16 acc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 pq = OP[I2][q][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * q + e] = pq[e];
        }
#pragma unroll
        for (int s = 0; s < NM; ++s) acc = mma32(vfrag(s), RM[u][s], acc);
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
        typedef __attribute__((ext_vector_type(2))) uint32_t u2;
        const int t0 = (c0 + ch) * CM;
        if constexpr (OUT_O) {
          const __amdgpu_buffer_rsrc_t orsrc =
              __builtin_amdgcn_make_buffer_rsrc(o + ((size_t)bh * T + t0) * DV, 0, (T - t0) * DV * 2, 0x00020000);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bf16x4 x = bf16x4{(__bf16)acc[4 * q], (__bf16)acc[4 * q + 1], (__bf16)acc[4 * q + 2],
                                    (__bf16)acc[4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, x), orsrc, oct + 16 * q, 0, 0);
          }
        }
        phase_barrier();                                // B
      });
    };
    const int I2 = wid - 4;
    if (NI2 < 2 && I2 >= NI2) {
      __syncthreads();
      walk([&](int, auto) { phase_barrier(); phase_barrier(); });
    } else if (I2 == 0) {
      run(Ic<0>{});
    } else {
      run(Ic<(NI2 >= 2 ? 1 : 0)>{});
    }
  } else {
    // ================= S: state rows 32*J2 .. of columns vt0 .. vt0+31
    const int J2 = wid - 6;
    const bool live = NJ2 >= 4 || J2 < NJ2;
    const int b_k = RL.kt + J2 * KSC * 1024, b_p = RL.pic + 128 * J2;
    u32x4 RK[NS][KSC];
    float RP[NS];
    auto load = [&](int ch, u32x4* X, float& pv) {
      const int cb = cbase(ch);
#pragma unroll
      for (int s = 0; s < KSC; ++s) X[s] = ld16(l16, cb + b_k + 1024 * s);
      pv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wrsrc, 4 * r, cb + b_p, 0));  // pi_C[32 J2 + r]
    };
    // L2 warm-up: three S waves of each value-tile workgroup of a head touch
    // the record's 128-byte lines, one dword per lane, PF chunks ahead; the
    // values are folded into `sink` when that chunk comes up, so the loads
    // are kept and never waited for early
    constexpr int kLine = 128;
    const int nlines = (RL.bytes + kLine - 1) / kLine;
    const int pl = (vt % 4) * 192 + (J2 % 3) * 64 + lane;
    const int v_pf = (pl < nlines ? pl : nlines - 1) * kLine;
    const bool toucher = live && J2 < 3;
    auto touch = [&](int ch) { return __builtin_amdgcn_raw_buffer_load_b32(wrsrc, v_pf, cbase(ch), 0); };
    uint32_t sink = 0, PFV[PF];
    const int pbase = 16 * h;                           // lane byte address of pi_C row 4h

    f32x16 Sacc;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Sacc[4 * q + e] = (live && S0w) ? S0w[(nseg == 1 ? stOff : 0) + (size_t)(32 * J2 + 8 * q + 4 * h + e) * DV + vt0 + r]
                                        : 0.f;
    auto st_s0t = [&]() {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        In<__bf16>::store4(S0T + r * LDK + 32 * J2 + 8 * q + 4 * h,
                           f32x4{Sacc[4 * q], Sacc[4 * q + 1], Sacc[4 * q + 2], Sacc[4 * q + 3]});
    };
    if (live) st_s0t();
    __syncthreads();                                    // S0^T written
    __builtin_amdgcn_s_waitcnt(0);
    if (live) {
      if (toucher) {
#pragma unroll
        for (int u = 0; u < PF; ++u) PFV[u] = touch(u);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NS - 1; ++u) {
        load(u, RK[u], RP[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    auto step = [&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      if (live) {
        // phase 1 is idle here: reload the set the previous chunk used (for
        // chunk ch + NS - 1), touch the record PF chunks ahead, scale the state
        load(ch + NS - 1, RK[(u + NS - 1) % NS], RP[(u + NS - 1) % NS]);
        __builtin_amdgcn_sched_barrier(0);
        if (toucher) {
          sink ^= PFV[u % PF];
          PFV[u % PF] = touch(ch + PF);
        }
        if constexpr (OUT_H) {                          // the chunk-start state, fp32
          float* hc = Hst + (((size_t)bh * ntot + c0 + ch) * DK + 32 * J2 + 4 * h) * DV + vt0 + r;
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)   // non-temporal (4K backward 2.49 -> 2.46 ms)
              __builtin_nontemporal_store(Sacc[4 * q + e], &hc[(size_t)(8 * q + e) * DV]);
        }
        // entry 4q + e is row 32 J2 + 8q + 4h + e, whose pi_C lane 8q + 4h + e
        // holds: one lane permute per entry (the constant part of the lane
        // address is the instruction's offset)
        const int pb = __float_as_int(RP[u % NS]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Sacc[4 * q + e] *= __int_as_float(__builtin_amdgcn_ds_bpermute(pbase + 4 * (8 * q + e), pb));
      }
      phase_barrier();                                  // A
      if (live) {
#pragma unroll
        for (int s = 0; s < KSC; ++s) Sacc = mma32(RK[u % NS][s], vfrag(s), Sacc);
        st_s0t();
      }
      phase_barrier();                                  // B
    };
    walk(step);
    if (live) {
      if (toucher) {
#pragma unroll
        for (int u = 0; u < PF; ++u) sink ^= PFV[u];
        if (sink == 0x7fc00001u && T < 0) o[0] = (__bf16)0.f;   // never true (T > 0): keeps the touches alive
      }
      if (S_outw) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S_outw[stOff + (size_t)(32 * J2 + 8 * q + 4 * h + e) * DV + vt0 + r] = Sacc[4 * q + e];
      }
    }
  }
}

// ------------------------------------------------------------------ sequence segments
//
// The chunk maps of "Muir: ...", §4.2 eq.(10) are affine in the state:
// S_C = A_c S_0 + K~^T U with A_c = Diag(pi_C) - K~^T Y. So a run of chunks
// (a segment g) maps its start state affinely, S_end = P_g S_start + Q_g, and
// a head with few value tiles but many chunks can walk its segments side by
// side:
//   seg_state:   every (b, h, segment but the last, one or two 32-column tiles of
//                [Q | P]) walks the segment from [0 | I]: the Q tiles with the
//                record's U, the P tiles with U = 0 (d_k identity columns
//                carried through the homogeneous map), giving [Q_g | P_g]
//                (fp32); two tiles per workgroup read the chunk's Y and K~^T
//                once for both;
//   seg_combine: per (b, h, value tile), S_start(g + 1) = P_g S_start(g) + Q_g
//                in order over the segments, from S_start(0) = S0;
//   the F-order scan then walks every segment from its start state and
//   writes O (and S_T from the last segment).
// The state tile walk of seg_state is the V~ / state-update half of the
// F-order scan (the same MFMA layouts), without the readout.

// Augmented state [Q_g | P_g] of (segment g, head bh): rows j, DV + DK columns.
__host__ __device__ __forceinline__ size_t seg_aug_off(int g, int bh, int BH, int DK, int DV) {
  return ((size_t)g * BH + bh) * DK * (DV + DK);
}

constexpr int kSegThreads = 64 * 6;   // seg_state: V~ waves (C/32) and state waves (d_k/32), at most 6

template <int DK, int CM, int NTW>
__global__ __launch_bounds__(kSegThreads) void gdn2_chunk_seg_state_kernel(const char* __restrict__ ws,
                                                                            float* __restrict__ Saug, int T,
                                                                            int DV, int seg) {
  constexpr int NI2 = CM / 32, NJ2 = DK / 32, KSD = DK / 16, KSC = CM / 16;
  constexpr int LDK = DK + 8, LDC = CM + 8;
  static_assert(DK % 32 == 0 && CM % 32 == 0 && NJ2 <= 4 && NI2 <= 2, "F-order segment shape");
  static_assert(NTW == 1 || NTW == 2, "one or two 32-column tiles per workgroup");
  // bf16 copy of the state tiles, [col][j], and V~^T [col][t]; NTW tiles side by side
  __shared__ __attribute__((aligned(16))) __bf16 S0T[NTW * 32 * LDK];
  __shared__ __attribute__((aligned(16))) __bf16 VTT[NTW * 32 * LDC];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r = lane & 31;
  const int nvt = DV / 32, ntile = nvt + DK / 32, ngrp = ntile / NTW;
  // the maps of segments 0 .. nseg - 2 (the last segment's map is never used)
  const int ntot = (T + CM - 1) / CM, nseg = (ntot + seg - 1) / seg, nmap = nseg - 1;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x, ngrp);
  const int unit = lin / ngrp, tile0 = NTW * (lin % ngrp);
  const int bh = unit / nmap, sg = unit % nmap;
  const int BH = gridDim.x / (ngrp * nmap);
  // column tiles of P (U = 0, identity start); with NTW = 2 the host keeps
  // nvt even, so both tiles of a workgroup are of one kind
  const bool ptile = tile0 >= nvt;
  const int c0 = sg * seg, nch = ntot - c0 < seg ? ntot - c0 : seg;
  const RecLayout RL = rec_layout(DK, DV, CM, 2);
  const char* wsh = ws + ((size_t)bh * ntot + c0) * RL.bytes;
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wsh), 0, nch * RL.bytes, 0x00020000);
  auto ld16 = [&](int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff, soff, 0));
  };
  // past the segment's last chunk the loads repeat it (never used)
  auto cbase = [&](int ch) { return (ch < nch ? ch : nch - 1) * RL.bytes; };
  const int l16 = lane * 16;
  auto s0frag = [&](int t, int s) { return *(const u32x4*)(S0T + (32 * t + r) * LDK + 16 * s + 8 * h); };
  auto vfrag = [&](int t, int s) { return *(const u32x4*)(VTT + (32 * t + r) * LDC + 16 * s + 8 * h); };
  // each role walks the chunks with three register sets (the operands of the
  // next two chunks load while this one's are used), unrolled by hand over
  // the sets with a single exit so the wait counts stay exact
  auto walk = [&](auto&& step) {
    int ch = 0;
    for (; ch + 3 <= nch; ch += 3) {
      step(ch, Ic<0>{});
      step(ch + 1, Ic<1>{});
      step(ch + 2, Ic<2>{});
    }
    if (ch < nch) step(ch, Ic<0>{});
    if (ch + 1 < nch) step(ch + 1, Ic<1>{});
  };

  if (wid < NI2) {
    // ================= V: V~ rows 32 wid .. = U - Y S (U = 0 for P tiles) -> V~^T in LDS
    const int I2 = wid;
    u32x4 RY[3][KSD], RU[3][NTW][2];
    // P tiles read U at an offset past the buffer's end: the loads return zero
    // (and every path issues the same loads)
    const int ub = ptile ? 0x7ffffff0 : lane * 32;
    auto load = [&](int ch, u32x4* Y, u32x4 (*U)[2]) {
      const int cb = cbase(ch);
#pragma unroll
      for (int s = 0; s < KSD; ++s) Y[s] = ld16(l16, cb + RL.y + I2 * KSD * 1024 + 1024 * s);
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) U[t][s] = ld16(ub, cb + RL.ut + ((ptile ? 0 : tile0 + t) * NI2 + I2) * 2048 + 16 * s);
    };
    __syncthreads();                                    // initial state copy written
    __builtin_amdgcn_s_waitcnt(0);
    load(0, RY[0], RU[0]);
    load(1, RY[1], RU[1]);
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      load(ch + 2, RY[(u + 2) % 3], RU[(u + 2) % 3]);
      f32x16 acc[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[t] = f16zero();
#pragma unroll
      for (int s = 0; s < KSD; ++s)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[t] = mma32(RY[u][s], s0frag(t, s), acc[t]);
      typedef __attribute__((ext_vector_type(2))) uint32_t u2;
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4& up = RU[u][t][q >> 1];
          const f32x4 uu = Raw<__bf16>::un4(u2{up[2 * (q & 1)], up[2 * (q & 1) + 1]});
          In<__bf16>::store4(VTT + (32 * t + r) * LDC + 32 * I2 + 8 * q + 4 * h,
                             f32x4{uu[0] - acc[t][4 * q], uu[1] - acc[t][4 * q + 1], uu[2] - acc[t][4 * q + 2],
                                   uu[3] - acc[t][4 * q + 3]});
        }
      phase_barrier();                                  // A: V~ ready
      phase_barrier();                                  // B: state copy ready
    });
  } else if (wid < NI2 + NJ2) {
    // ================= S: state rows 32 J2 .. of this workgroup's NTW x 32
    // columns (entry 4q + e of tile t is row 32 J2 + 8q + 4h + e, column
    // 32 (tile0 + t) + r), from [0 | I]
    const int J2 = wid - NI2;
    u32x4 RK[3][KSC];
    float RP[3];
    auto load = [&](int ch, u32x4* X, float& pv) {
      const int cb = cbase(ch);
#pragma unroll
      for (int s = 0; s < KSC; ++s) X[s] = ld16(l16, cb + RL.kt + J2 * KSC * 1024 + 1024 * s);
      pv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wrsrc, 4 * r, cb + RL.pic + 128 * J2, 0));
    };
    f32x16 Sacc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int pcol = 32 * (tile0 + t - nvt) + r;     // P tile: the identity column of this lane
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Sacc[t][4 * q + e] = (ptile && 32 * J2 + 8 * q + 4 * h + e == pcol) ? 1.f : 0.f;
    }
    auto st_s0t = [&]() {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          In<__bf16>::store4(S0T + (32 * t + r) * LDK + 32 * J2 + 8 * q + 4 * h,
                             f32x4{Sacc[t][4 * q], Sacc[t][4 * q + 1], Sacc[t][4 * q + 2], Sacc[t][4 * q + 3]});
    };
    st_s0t();
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);
    const int pbase = 16 * h;
    load(0, RK[0], RP[0]);
    load(1, RK[1], RP[1]);
    walk([&](int ch, auto Uc) {
      constexpr int u = decltype(Uc)::value;
      load(ch + 2, RK[(u + 2) % 3], RP[(u + 2) % 3]);
      const int pb = __float_as_int(RP[u]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = __int_as_float(__builtin_amdgcn_ds_bpermute(pbase + 4 * (8 * q + e), pb));
#pragma unroll
          for (int t = 0; t < NTW; ++t) Sacc[t][4 * q + e] *= f;
        }
      phase_barrier();                                  // A
#pragma unroll
      for (int s = 0; s < KSC; ++s)
#pragma unroll
        for (int t = 0; t < NTW; ++t) Sacc[t] = mma32(RK[u][s], vfrag(t, s), Sacc[t]);
      st_s0t();
      phase_barrier();                                  // B
    });
    float* out = Saug + seg_aug_off(sg, bh, BH, DK, DV);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int col = ptile ? DV + 32 * (tile0 + t - nvt) + r : 32 * (tile0 + t) + r;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          out[(size_t)(32 * J2 + 8 * q + 4 * h + e) * (DV + DK) + col] = Sacc[t][4 * q + e];
    }
  } else {
    __syncthreads();
    walk([&](int, auto) { phase_barrier(); phase_barrier(); });
  }
}

// Segment start states: per (b, h, 32-column value tile), in segment order,
// Sseg[g] = S_start(g) and S_start(g + 1) = P_g S_start(g) + Q_g (fp32).
// The products run on the fp32 matrix cores (16x16x4, fp32 products and
// accumulation): P_g in LDS as [j][k], the state tile transposed as [v][k];
// each of the four waves holds whole 16 x 16 output tiles in accumulator
// layout (entry e of a lane: row 16 jt + 4 (lane / 16) + e, column
// 16 vl + lane % 16).
template <int DK>
__global__ __launch_bounds__(256) void gdn2_chunk_seg_combine_kernel(const float* __restrict__ Saug,
                                                                      const float* __restrict__ S0,
                                                                      float* __restrict__ Sseg, int DV,
                                                                      int nseg) {
  constexpr int LP = DK + 4;                           // LDS row pitch (floats)
  constexpr int NT = DK / 8, TPW = NT / 4;             // 16 x 16 tiles of the DK x 32 tile, per wave
  static_assert(NT % 4 == 0, "whole tiles per wave");
  __shared__ __attribute__((aligned(16))) float Pl[DK][LP];
  __shared__ __attribute__((aligned(16))) float St[32][LP];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int nvt = DV / 32;
  const int bh = blockIdx.x / nvt, vt = blockIdx.x % nvt;
  const int BH = gridDim.x / nvt;
  // element e of this lane's entry of tile i: row, column of the DK x DV state
  auto row = [&](int i, int e) { return 16 * ((wid + 4 * i) >> 1) + 4 * g4 + e; };
  auto col = [&](int i) { return 32 * vt + 16 * ((wid + 4 * i) & 1) + c16; };
  f32x4 sv[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[i][e] = S0 ? S0[((size_t)bh * DK + row(i, e)) * DV + col(i)] : 0.f;
  for (int g = 0; g < nseg; ++g) {
    float* dst = Sseg + ((size_t)g * BH + bh) * DK * DV;
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(size_t)row(i, e) * DV + col(i)] = sv[i][e];
    if (g == nseg - 1) break;
    const float* aug = Saug + seg_aug_off(g, bh, BH, DK, DV);
    __syncthreads();                                   // the previous step's reads of Pl / St are done
#pragma unroll
    for (int i = 0; i < TPW; ++i) *(f32x4*)&St[col(i) - 32 * vt][row(i, 0)] = sv[i];
    // P_g: columns DV .. DV + DK of the augmented rows; unrolled, so all of
    // its loads are in flight together
    GDR_STAGE_FOR(x, DK * DK / 4, 256) {
      const int rr = x / (DK / 4), cc = 4 * (x % (DK / 4));
      *(f32x4*)&Pl[rr][cc] = *(const f32x4*)(aug + (size_t)rr * (DV + DK) + DV + cc);
    }
    f32x4 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)                       // Q_g
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] = aug[(size_t)row(i, e) * (DV + DK) + col(i)];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      tile_nt(acc[i], &Pl[0][0], LP, 16 * ((wid + 4 * i) >> 1), &St[0][0], LP, 16 * ((wid + 4 * i) & 1), DK, lane);
#pragma unroll
    for (int i = 0; i < TPW; ++i) sv[i] = acc[i];
  }
}

// ------------------------------------------------------------------ host launch

// Segment length (chunks) of the sequence-segmented scan, or 0 for the plain
// scan. Segments pay only when the (b, h, value tile) workgroups of the plain
// scan leave most of the GPU's 256 compute units idle and the chunk chain is
// long: then the chain is cut into nseg segments so that about 256 scan
// workgroups run side by side, each segment at least 16 chunks long. The
// plan depends on the shapes alone (the workspace size has to).
static int seg_plan(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  if (!fm_path(dk, dv, chunk, dtype, T)) return 0;
  const long long units = (long long)B * H * (dv / 32);
  const int ntot = (T + chunk - 1) / chunk;
  if (units * 2 > kSegTargetUnits || ntot < 32) return 0;
  int nseg = (int)(kSegTargetUnits / units);
  if (nseg > ntot / 16) nseg = ntot / 16;
  if (nseg < 2) return 0;
  return (ntot + nseg - 1) / nseg;
}

static size_t seg_extra_bytes(int B, int H, int T, int dk, int dv, int chunk, int seg) {
  const int ntot = (T + chunk - 1) / chunk, nseg = (ntot + seg - 1) / seg;
  return (size_t)nseg * B * H * dk * ((size_t)(dv + dk) + dv) * 4;
}

static size_t records_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  const int es = dtype == GDR_BF16 ? 2 : 4;
  const size_t nchunks = ((size_t)T + chunk - 1) / chunk;
  return (size_t)B * H * nchunks * (size_t)rec_layout(dk, dv, chunk, es).bytes;
}

size_t chunk_ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype, bool allow_seg) {
  size_t n = records_bytes(B, H, T, dk, dv, chunk, dtype);
  const int seg = allow_seg ? seg_plan(B, H, T, dk, dv, chunk, dtype) : 0;
  if (seg) n = (n + 255) / 256 * 256 + seg_extra_bytes(B, H, T, dk, dv, chunk, seg);
  return n;
}

template <typename Tin, int DK, int CM, bool FM, bool GATED>
static int launch_intra_g(const ChunkArgs& a, char* ws) {
  using L = IntraSmem<Tin, DK, CM>;
  // non-temporal input loads only for the plain gates: with the gate
  // prologue (4K shape) plain loads measured 0.2808 ms against 0.2840
  const void* kern = (const void*)gdn2_chunk_intra_kernel<Tin, DK, CM, FM, GATED, !GATED>;
  if (!allow_lds(kern, L::TOTAL)) return GDR_ERR_LAUNCH;
  int nchunks = (a.T + CM - 1) / CM;
  int nitems = a.B * a.H * nchunks;
  // one resident workgroup per CU, each walking items with a stride of the grid
  const int cus = stream_cus(a.stream);
  const int grid = nitems < cus ? nitems : cus;
  const Tin *q = (const Tin*)a.q, *k = (const Tin*)a.k, *v = (const Tin*)a.v;
  const Tin *al = (const Tin*)a.alpha, *bg = (const Tin*)a.b, *wg = (const Tin*)a.w;
  const Tin* zq = (const Tin*)a.zq;
  const float *alog = a.a_log, *gst = a.gamma_stat;
  int T = a.T, DV = a.dv, H = a.H;
  void* args[] = {&q, &k, &v, &al, &bg, &wg, &ws, &T, &DV, &nchunks, &nitems, &zq, &alog, &gst, &H};
  hipError_t e = hipLaunchKernel(kern, dim3(grid), dim3(kIntraThreads), args, L::TOTAL, (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

template <typename Tin, int DK, int CM, bool FM>
static int launch_intra(const ChunkArgs& a, char* ws) {
  return a.gated ? launch_intra_g<Tin, DK, CM, FM, true>(a, ws) : launch_intra_g<Tin, DK, CM, FM, false>(a, ws);
}

template <typename Tin, int DK, int VT, int CM>
static int launch_scan(const ChunkArgs& a, const char* ws) {
  const void* kern;
  int lds = 0;
  if constexpr (std::is_same<Tin, __bf16>::value) {
    using L = StagedScan<DK, VT, CM>;
    kern = (const void*)gdn2_chunk_scan_staged_kernel<DK, VT, CM>;
    lds = L::TOTAL;
    if (!allow_lds(kern, lds)) return GDR_ERR_LAUNCH;
  } else {
    kern = (const void*)gdn2_chunk_scan_kernel<Tin, DK, VT, CM>;
  }
  const int nblocks = a.B * a.H * (a.dv / VT);
  const float* S0 = a.S0;
  Tin* o = (Tin*)a.o;
  float* So = a.S_out;
  int T = a.T, DV = a.dv;
  void* args[] = {&ws, &S0, &o, &So, &T, &DV};
  hipError_t e = hipLaunchKernel(kern, dim3(nblocks), dim3(kScanThreads), args, lds, (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

template <int DK, int CM>
static int launch_scan_fm(const ChunkArgs& a, const char* ws) {
  const void* kern = (const void*)gdn2_chunk_scan_fm_kernel<DK, CM, kScanFmPrefetch, kScanFmSets>;
  const float* S0 = a.S0;
  __bf16* o = (__bf16*)a.o;
  float* So = a.S_out;
  int T = a.T, DV = a.dv;
  const int ntot = (T + CM - 1) / CM;
  const int BH = a.B * a.H;
  int seg = a.no_seg ? 0 : seg_plan(a.B, a.H, a.T, DK, a.dv, CM, a.dtype);
  const float* Sseg = nullptr;
  if (seg) {
    // segment pass and start states, then every segment's scan from its start
    const size_t rec = (records_bytes(a.B, a.H, T, DK, a.dv, CM, GDR_BF16) + 255) / 256 * 256;
    const int nseg = (ntot + seg - 1) / seg;
    float* Saug = (float*)(const_cast<char*>(ws) + rec);
    float* Ss = Saug + (size_t)nseg * BH * DK * (a.dv + DK);
    const int ntile = a.dv / 32 + DK / 32;
    void* a1[] = {&ws, &Saug, &T, &DV, &seg};
    // two 32-column tiles per workgroup where both the value and the P
    // columns split into pairs (the shared operands are read once for both)
    const bool pair = (a.dv / 32) % 2 == 0 && (DK / 32) % 2 == 0;
    hipError_t e = pair ? hipLaunchKernel((const void*)gdn2_chunk_seg_state_kernel<DK, CM, 2>,
                                          dim3((nseg - 1) * BH * (ntile / 2)), dim3(kSegThreads), a1, 0,
                                          (hipStream_t)a.stream)
                        : hipLaunchKernel((const void*)gdn2_chunk_seg_state_kernel<DK, CM, 1>,
                                          dim3((nseg - 1) * BH * ntile), dim3(kSegThreads), a1, 0,
                                          (hipStream_t)a.stream);
    if (e != hipSuccess) return GDR_ERR_LAUNCH;
    int nsg = nseg;
    void* a2[] = {&Saug, &S0, &Ss, &DV, &nsg};
    e = hipLaunchKernel((const void*)gdn2_chunk_seg_combine_kernel<DK>, dim3(BH * (a.dv / 32)), dim3(256), a2, 0,
                        (hipStream_t)a.stream);
    if (e != hipSuccess) return GDR_ERR_LAUNCH;
    Sseg = Ss;
  } else {
    seg = ntot;
  }
  const int nblocks = BH * (a.dv / 32) * ((ntot + seg - 1) / seg);
  float* Hst = nullptr;
  void* args[] = {&ws, &S0, &o, &So, &T, &DV, &seg, &Sseg, &Hst};
  hipError_t e = hipLaunchKernel(kern, dim3(nblocks), dim3(kScanFmThreads), args, 0, (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

// Chunk-start states of the F-order records in `ws` (written by the intra
// kernel for these shapes) for the backward: the F-order scan without outputs,
// one segment per head.
template <int DK, int CM>
static int launch_states_fm(const ChunkArgs& a, const char* ws, float* Hst) {
  const void* kern = (const void*)gdn2_chunk_scan_fm_kernel<DK, CM, kScanFmPrefetch, kScanFmSets, false, true>;
  const float* S0 = a.S0;
  __bf16* o = nullptr;
  float* So = nullptr;
  const float* Sseg = nullptr;
  int T = a.T, DV = a.dv;
  int seg = (T + CM - 1) / CM;
  const int nblocks = a.B * a.H * (a.dv / 32);
  void* args[] = {&ws, &S0, &o, &So, &T, &DV, &seg, &Sseg, &Hst};
  hipError_t e = hipLaunchKernel(kern, dim3(nblocks), dim3(kScanFmThreads), args, 0, (hipStream_t)a.stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

int chunk_states_fm_launch(const ChunkArgs& a, const void* ws, float* Hst) {
  if (!fm_path(a.dk, a.dv, a.chunk, a.dtype, a.T)) return GDR_ERR_UNSUPPORTED;
  switch (a.dk * 1000 + a.chunk) {
    case 32032: return launch_states_fm<32, 32>(a, (const char*)ws, Hst);
    case 32064: return launch_states_fm<32, 64>(a, (const char*)ws, Hst);
    case 64032: return launch_states_fm<64, 32>(a, (const char*)ws, Hst);
    case 64064: return launch_states_fm<64, 64>(a, (const char*)ws, Hst);
    case 128032: return launch_states_fm<128, 32>(a, (const char*)ws, Hst);
    case 128064: return launch_states_fm<128, 64>(a, (const char*)ws, Hst);
  }
  return GDR_ERR_UNSUPPORTED;
}

template <typename Tin, int DK, int CM>
static int launch_pair(const ChunkArgs& a, char* ws, int phases) {
  // bf16 records with d_k, d_v and C multiples of 32 are written in F order
  // for the 32x32x16 scan. Every workgroup walks all chunks of its head, so
  // the time is the per-chunk time times the chunk count whether or not the
  // workgroups fill the GPU, and the F-order scan's chunk is the shorter one
  // also with few heads (the staged scan's 16-column tiles only add
  // workgroups). The decision depends only on the shapes, so the intra and
  // scan phases (also as separate calls) take the same one. The F-order scan
  // addresses a head's records with 32-bit offsets.
  if constexpr (std::is_same<Tin, __bf16>::value && DK % 32 == 0 && CM % 32 == 0) {
    if (fm_path(DK, a.dv, CM, a.dtype, a.T)) {
      if (phases & 1) {
        const int st = launch_intra<Tin, DK, CM, true>(a, ws);
        if (st != GDR_OK) return st;
      }
      if (!(phases & 2)) return GDR_OK;
      return launch_scan_fm<DK, CM>(a, ws);
    }
  }
  if (phases & 1) {
    const int st = launch_intra<Tin, DK, CM, false>(a, ws);
    if (st != GDR_OK) return st;
  }
  if (!(phases & 2)) return GDR_OK;
  // value tiles of 32 columns when that still gives a workgroup per CU, else 16
  const bool wide = a.dv >= 32 && (long long)a.B * a.H * (a.dv / 32) >= stream_cus(a.stream);
  if constexpr (std::is_same<Tin, float>::value) {
    return launch_scan<Tin, DK, 16, CM>(a, ws);
  } else {
    if (!wide) return launch_scan<Tin, DK, 16, CM>(a, ws);
    return launch_scan<Tin, DK, 32, CM>(a, ws);
  }
}

template <typename Tin, int CM>
static int dispatch_dk(const ChunkArgs& a, char* ws, int phases) {
  switch (a.dk) {
    case 16: return launch_pair<Tin, 16, CM>(a, ws, phases);
    case 32: return launch_pair<Tin, 32, CM>(a, ws, phases);
    case 64: return launch_pair<Tin, 64, CM>(a, ws, phases);
    case 128: return launch_pair<Tin, 128, CM>(a, ws, phases);
  }
  return GDR_ERR_UNSUPPORTED;
}

template <typename Tin>
static int dispatch_chunk(const ChunkArgs& a, char* ws, int phases) {
  switch (a.chunk) {
    case 16: return dispatch_dk<Tin, 16>(a, ws, phases);
    case 32: return dispatch_dk<Tin, 32>(a, ws, phases);
    case 64: return dispatch_dk<Tin, 64>(a, ws, phases);
  }
  return GDR_ERR_UNSUPPORTED;
}

int chunk_fwd_ws_launch(const ChunkArgs& a, void* ws, int phases) {
  if (a.dtype == GDR_BF16) return dispatch_chunk<__bf16>(a, (char*)ws, phases);
  return dispatch_chunk<float>(a, (char*)ws, phases);
}

}  // namespace gdr
