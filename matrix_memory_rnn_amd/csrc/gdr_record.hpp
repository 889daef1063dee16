// Workspace record of the two-kernel chunk forward: one record per
// (b, h, chunk), written by the intra-chunk kernel and read by the scans and
// the backward kernels. Layouts only; no arithmetic of the method.
#pragma once

#include "gdr_device.hpp"
#include "../../include/gdr.h"

namespace gdr {

// Byte layout of the workspace record of one (b, h, chunk); es = element size.
struct RecLayout {
  int y, ut, m, qp, kt, pic, bytes;
};
__host__ __device__ __forceinline__ RecLayout rec_layout(int dk, int dv, int C, int es) {
  RecLayout r;
  r.y = 0;                          // Y      [t][j]  C x dk
  r.ut = r.y + C * dk * es;         // U^T    [v][t]  dv x C
  r.m = r.ut + dv * C * es;         // M      [t][s]  C x C (entries above the diagonal blocks unused)
  r.qp = r.m + C * C * es;          // Q_pi   [t][j]  C x dk
  r.kt = r.qp + C * dk * es;        // K~^T   [j][s]  dk x C
  r.pic = r.kt + dk * C * es;       // pi_C   fp32    dk
  r.bytes = r.pic + dk * 4;
  return r;
}

// "F order" of the bf16 record, read by the 32x32x16 MFMA scan: every matrix
// is stored so that one 32x32x16 operand slice is 1 KiB of consecutive bytes,
// lane l's 16 bytes at 16*l. For a row-major R x K matrix (Y, Q_pi, M: rows t;
// K~^T: rows j) the 8 elements k = 8c .. 8c+7 of row r form 16-byte piece
// ((r/32)*(K/16) + c/2)*64 + (c%2)*32 + r%32 (element offset returned).
__host__ __device__ __forceinline__ int fm_off(int r, int k, int K) {
  return ((((r >> 5) * (K >> 4) + (k >> 4)) * 64 + ((k >> 3) & 1) * 32 + (r & 31)) << 3) + (k & 7);
}
// U^T in F order: for value tile v/32 and row block t/32, lane l holds the 16
// entries t = 32*(t/32) + 8q + 4*(l/32) + e (q, e = 0..3; entry 4q + e) of
// column v = 32*(v/32) + l%32, contiguous: the accumulator layout of V~.
__host__ __device__ __forceinline__ int fu_off(int v, int t, int C) {
  return ((((v >> 5) * (C >> 5) + (t >> 5)) * 64 + ((t >> 2) & 1) * 32 + (v & 31)) << 4) +
         (((t >> 3) & 3) << 2) + (t & 3);
}

// Stores of record entries from fp32 values.
// Whether the F-order (fragment-major) record serves these shapes: bf16,
// d_k, d_v and C multiples of 32, one head's records under 2 GiB (the scans
// address a head's records with 32-bit offsets).
inline bool fm_path(int dk, int dv, int chunk, int dtype, long long T) {
  if (dtype != GDR_BF16 || dk % 32 || dv % 32 || chunk % 32) return false;
  return ((T + chunk - 1) / chunk) * (long long)rec_layout(dk, dv, chunk, 2).bytes < (1LL << 31);
}

}  // namespace gdr
