// C-ABI entry points of libgdr: host-side argument validation, then dispatch
// to the gfx950 kernel launchers. Validation touches no GPU state, so every
// error code is returned before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_internal.h"

namespace {

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool is_pow2_dim(int d, int maxd) {
  return d == 16 || d == 32 || d == 64 || d == 128 || (maxd >= 256 && d == 256);
}

size_t esize(int dtype) { return dtype == GDR_BF16 ? 2 : 4; }

// Common checks on the sizes; returns GDR_OK or an error.
int check_sizes(long long B, long long H, long long T, int dk, int dv, int dtype, int maxd) {
  if (dtype != GDR_F32 && dtype != GDR_BF16) return GDR_ERR_DTYPE;
  if (B < 1 || H < 1 || T < 1 || dk < 1 || dv < 1) return GDR_ERR_SHAPE;
  // element offsets are formed in 64-bit; grid sizes must fit in 31 bits
  if (B * H > (1LL << 24) || B * H * T > (1LL << 40)) return GDR_ERR_SHAPE;
  // byte offsets within one head are 32-bit signed in the kernels
  if (T * (long long)(dk > dv ? dk : dv) * (long long)esize(dtype) >= (1LL << 31)) return GDR_ERR_SHAPE;
  if (!is_pow2_dim(dk, maxd) || !is_pow2_dim(dv, maxd)) return GDR_ERR_UNSUPPORTED;
  return GDR_OK;
}

// Input checks of the chunkwise entry points: pointers, sizes, chunk, alignment.
int check_chunk_inputs(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                       const void* w, int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  if (!q || !k || !v || !alpha || !b || !w) return GDR_ERR_NULL;
  int st = check_sizes(B, H, T, dk, dv, dtype, 128);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDR_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, alpha, b, w};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDR_ERR_ALIGN;
  return GDR_OK;
}

// Checks shared by the chunkwise entry points that write o (and S_out).
int check_chunk(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                const void* w, const float* S0, const void* o, const float* S_out, int B, int H,
                int T, int dk, int dv, int chunk, int dtype) {
  if (!o) return GDR_ERR_NULL;
  int st = check_chunk_inputs(q, k, v, alpha, b, w, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  const void* outs[] = {S0, o, S_out};
  for (const void* p : outs)
    if (!aligned16(p)) return GDR_ERR_ALIGN;
  const size_t es = esize(dtype);
  const size_t nK = (size_t)B * H * T * dk * es, nV = (size_t)B * H * T * dv * es;
  const size_t nS = (size_t)B * H * dk * dv * sizeof(float);
  const void* ins[] = {q, k, alpha, b};
  for (const void* p : ins) {
    if (overlap(o, nV, p, nK)) return GDR_ERR_ALIAS;
    if (overlap(S_out, nS, p, nK)) return GDR_ERR_ALIAS;
  }
  if (overlap(o, nV, v, nV) || overlap(o, nV, w, nV) || overlap(o, nV, S0, nS) || overlap(o, nV, S_out, nS))
    return GDR_ERR_ALIAS;
  if (overlap(S_out, nS, v, nV) || overlap(S_out, nS, w, nV)) return GDR_ERR_ALIAS;
  if (S_out && S0 && S_out != S0 && overlap(S_out, nS, S0, nS)) return GDR_ERR_ALIAS;
  return GDR_OK;
}

// Workspace checks of the two-kernel chunk forward: present, aligned, large
// enough, and clear of every other buffer.
int check_workspace(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                    const void* w, const float* S0, const void* o, const float* S_out, int B, int H,
                    int T, int dk, int dv, int chunk, int dtype, const void* workspace,
                    size_t workspace_bytes) {
  if (!workspace) return GDR_ERR_NULL;
  if (!aligned16(workspace)) return GDR_ERR_ALIGN;
  const size_t need = gdr::chunk_ws_bytes(B, H, T, dk, dv, chunk, dtype);
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE;
  const size_t es = esize(dtype);
  const size_t nK = (size_t)B * H * T * dk * es, nV = (size_t)B * H * T * dv * es;
  const size_t nS = (size_t)B * H * dk * dv * sizeof(float);
  struct R { const void* p; size_t n; };
  const R bufs[] = {{q, nK}, {k, nK}, {alpha, nK}, {b, nK}, {v, nV}, {w, nV},
                    {S0, nS}, {o, nV}, {S_out, nS}};
  for (const R& x : bufs)
    if (overlap(workspace, need, x.p, x.n)) return GDR_ERR_ALIAS;
  return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_version(void) { return 200; }  // 0.2.0

const char* gdr_status_string(int status) {
  switch (status) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL: return "a required pointer is NULL";
    case GDR_ERR_SHAPE: return "a size is out of range";
    case GDR_ERR_DTYPE: return "unknown dtype code";
    case GDR_ERR_UNSUPPORTED: return "sizes valid but not supported by this build (head dim or chunk)";
    case GDR_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case GDR_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case GDR_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case GDR_ERR_WORKSPACE: return "the workspace is smaller than gdr_chunk_workspace_size reports";
  }
  return "unknown status";
}

int gdr_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                  const void* w, const float* S0, void* o, float* S_out, int B, int H, int T, int dk,
                  int dv, int chunk, int dtype, void* stream) {
  int st = check_chunk(q, k, v, alpha, b, w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  if (dtype == GDR_F32 && dk >= 64 && chunk > 32) return GDR_ERR_UNSUPPORTED;
  gdr::ChunkArgs a{q, k, v, alpha, b, w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::chunk_fwd_launch(a);
}

int gdr_chunk_workspace_size(int B, int H, int T, int dk, int dv, int chunk, int dtype, size_t* bytes) {
  if (!bytes) return GDR_ERR_NULL;
  *bytes = 0;
  int st = check_sizes(B, H, T, dk, dv, dtype, 128);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDR_ERR_UNSUPPORTED;
  *bytes = gdr::chunk_ws_bytes(B, H, T, dk, dv, chunk, dtype);
  return GDR_OK;
}

int gdr_chunk_fwd_ws(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                     const void* w, const float* S0, void* o, float* S_out, int B, int H, int T,
                     int dk, int dv, int chunk, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_chunk(q, k, v, alpha, b, w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  st = check_workspace(q, k, v, alpha, b, w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype, workspace,
                       workspace_bytes);
  if (st != GDR_OK) return st;
  gdr::ChunkArgs a{q, k, v, alpha, b, w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::chunk_fwd_ws_launch(a, workspace, 3);
}

int gdr_chunk_intra(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                    const void* w, int B, int H, int T, int dk, int dv, int chunk, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_chunk_inputs(q, k, v, alpha, b, w, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  st = check_workspace(q, k, v, alpha, b, w, nullptr, nullptr, nullptr, B, H, T, dk, dv, chunk, dtype,
                       workspace, workspace_bytes);
  if (st != GDR_OK) return st;
  gdr::ChunkArgs a{q, k, v, alpha, b, w, nullptr, nullptr, nullptr, B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::chunk_fwd_ws_launch(a, workspace, 1);
}

int gdr_chunk_scan(const void* workspace, size_t workspace_bytes, const float* S0, void* o, float* S_out,
                   int B, int H, int T, int dk, int dv, int chunk, int dtype, void* stream) {
  if (!workspace || !o) return GDR_ERR_NULL;
  int st = check_sizes(B, H, T, dk, dv, dtype, 128);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDR_ERR_UNSUPPORTED;
  const void* ptrs[] = {workspace, S0, o, S_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDR_ERR_ALIGN;
  const size_t need = gdr::chunk_ws_bytes(B, H, T, dk, dv, chunk, dtype);
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE;
  const size_t nV = (size_t)B * H * T * dv * esize(dtype);
  const size_t nS = (size_t)B * H * dk * dv * sizeof(float);
  if (overlap(o, nV, workspace, need) || overlap(S_out, nS, workspace, need) ||
      overlap(S0, nS, workspace, need) || overlap(o, nV, S0, nS) || overlap(o, nV, S_out, nS))
    return GDR_ERR_ALIAS;
  if (S_out && S0 && S_out != S0 && overlap(S_out, nS, S0, nS)) return GDR_ERR_ALIAS;
  gdr::ChunkArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, S0, o, S_out, B, H, T, dk, dv,
                   chunk, dtype, stream};
  return gdr::chunk_fwd_ws_launch(a, const_cast<void*>(workspace), 2);
}

int gdr_decode_step(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                    const void* w, float* S, void* o, int N, int H, int dk, int dv, int dtype,
                    void* stream) {
  if (!q || !k || !v || !alpha || !b || !w || !S || !o) return GDR_ERR_NULL;
  int st = check_sizes(N, H, 1, dk, dv, dtype, 128);
  if (st != GDR_OK) return st;
  const void* ptrs[] = {q, k, v, alpha, b, w, S, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDR_ERR_ALIGN;
  const size_t es = esize(dtype);
  const size_t nK = (size_t)N * H * dk * es, nV = (size_t)N * H * dv * es;
  const size_t nS = (size_t)N * H * dk * dv * sizeof(float);
  const void* insK[] = {q, k, alpha, b};
  for (const void* p : insK)
    if (overlap(o, nV, p, nK) || overlap(S, nS, p, nK)) return GDR_ERR_ALIAS;
  if (overlap(o, nV, v, nV) || overlap(o, nV, w, nV) || overlap(o, nV, S, nS)) return GDR_ERR_ALIAS;
  if (overlap(S, nS, v, nV) || overlap(S, nS, w, nV)) return GDR_ERR_ALIAS;
  gdr::DecodeArgs a{q, k, v, alpha, b, w, S, o, N, H, dk, dv, dtype, stream};
  return gdr::decode_launch(a);
}

}  // extern "C"

namespace {

// Checks of the mLSTM entry points (everything but the workspace).
int check_mlstm(const void* q, const void* k, const void* v, const float* i_tilde,
                const float* f_tilde, const float* C0, const float* n0, const float* m0, void* h,
                float* C_out, float* n_out, float* m_out, int B, int H, int T, int dk, int dv,
                int chunk, int dtype) {
  if (!q || !k || !v || !i_tilde || !f_tilde || !h) return GDR_ERR_NULL;
  const bool s_in = C0 || n0 || m0, s_out = C_out || n_out || m_out;
  if (s_in && !(C0 && n0 && m0)) return GDR_ERR_NULL;
  if (s_out && !(C_out && n_out && m_out)) return GDR_ERR_NULL;
  int st = check_sizes(B, H, T, dk, dv, dtype, 256);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDR_ERR_UNSUPPORTED;
  if (dtype == GDR_F32 && dk > 128) return GDR_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, i_tilde, f_tilde, C0, n0, m0, h, C_out, n_out, m_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDR_ERR_ALIGN;
  const size_t es = esize(dtype);
  const size_t nK = (size_t)B * H * T * dk * es, nV = (size_t)B * H * T * dv * es;
  const size_t nG = (size_t)B * H * T * sizeof(float);
  const size_t nC = (size_t)B * H * dk * dv * sizeof(float), nN = (size_t)B * H * dk * sizeof(float);
  const size_t nM = (size_t)B * H * sizeof(float);
  struct R { const void* p; size_t n; };
  const R ins[] = {{q, nK}, {k, nK}, {v, nV}, {i_tilde, nG}, {f_tilde, nG}};
  const R outs[] = {{h, nV}, {C_out, nC}, {n_out, nN}, {m_out, nM}};
  for (const R& x : outs) {
    for (const R& y : ins)
      if (overlap(x.p, x.n, y.p, y.n)) return GDR_ERR_ALIAS;
    for (const R& y : outs)
      if (x.p != y.p && overlap(x.p, x.n, y.p, y.n)) return GDR_ERR_ALIAS;
  }
  const R st_in[] = {{C0, nC}, {n0, nN}, {m0, nM}};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 4; ++j) {
      if (j == 0) {
        if (overlap(outs[0].p, outs[0].n, st_in[i].p, st_in[i].n)) return GDR_ERR_ALIAS;
        continue;
      }
      // C_out may be C0 (each workgroup reads and writes only its own value
      // columns); n and m are shared by all value tiles of a head, so their
      // outputs must not overlap any initial-state buffer
      if (i == 0 && j == 1 && outs[j].p == st_in[i].p) continue;
      if (overlap(outs[j].p, outs[j].n, st_in[i].p, st_in[i].n)) return GDR_ERR_ALIAS;
    }
  return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_mlstm_fwd(const void* q, const void* k, const void* v, const float* i_tilde,
                  const float* f_tilde, const float* C0, const float* n0, const float* m0, void* h,
                  float* C_out, float* n_out, float* m_out, int B, int H, int T, int dk, int dv,
                  int chunk, int dtype, void* stream) {
  int st = check_mlstm(q, k, v, i_tilde, f_tilde, C0, n0, m0, h, C_out, n_out, m_out, B, H, T, dk, dv,
                       chunk, dtype);
  if (st != GDR_OK) return st;
  gdr::MlstmArgs a{q, k, v, i_tilde, f_tilde, C0, n0, m0, h, C_out, n_out, m_out,
                   B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::mlstm_launch(a);
}

int gdr_mlstm_workspace_size(int B, int H, int T, int dk, int dv, int chunk, int dtype, size_t* bytes) {
  if (!bytes) return GDR_ERR_NULL;
  *bytes = 0;
  int st = check_sizes(B, H, T, dk, dv, dtype, 256);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDR_ERR_UNSUPPORTED;
  *bytes = gdr::mlstm_ws_bytes(B, H, T, dk, dv, chunk, dtype);
  return GDR_OK;
}

int gdr_mlstm_fwd_ws(const void* q, const void* k, const void* v, const float* i_tilde,
                     const float* f_tilde, const float* C0, const float* n0, const float* m0, void* h,
                     float* C_out, float* n_out, float* m_out, int B, int H, int T, int dk, int dv,
                     int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mlstm(q, k, v, i_tilde, f_tilde, C0, n0, m0, h, C_out, n_out, m_out, B, H, T, dk, dv,
                       chunk, dtype);
  if (st != GDR_OK) return st;
  if (dtype == GDR_F32 && dv > 128) return GDR_ERR_UNSUPPORTED;
  if (!workspace) return GDR_ERR_NULL;
  if (!aligned16(workspace)) return GDR_ERR_ALIGN;
  const size_t need = gdr::mlstm_ws_bytes(B, H, T, dk, dv, chunk, dtype);
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE;
  const size_t es = esize(dtype);
  const size_t nK = (size_t)B * H * T * dk * es, nV = (size_t)B * H * T * dv * es;
  const size_t nG = (size_t)B * H * T * sizeof(float);
  const size_t nC = (size_t)B * H * dk * dv * sizeof(float), nN = (size_t)B * H * dk * sizeof(float);
  const size_t nM = (size_t)B * H * sizeof(float);
  struct R { const void* p; size_t n; };
  const R bufs[] = {{q, nK}, {k, nK}, {v, nV}, {i_tilde, nG}, {f_tilde, nG}, {C0, nC}, {n0, nN},
                    {m0, nM}, {h, nV}, {C_out, nC}, {n_out, nN}, {m_out, nM}};
  for (const R& x : bufs)
    if (overlap(workspace, need, x.p, x.n)) return GDR_ERR_ALIAS;
  gdr::MlstmArgs a{q, k, v, i_tilde, f_tilde, C0, n0, m0, h, C_out, n_out, m_out,
                   B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::mlstm_ws_launch(a, workspace);
}

}  // extern "C"
