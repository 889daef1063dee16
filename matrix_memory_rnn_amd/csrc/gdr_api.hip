// C-ABI entry points of libgdr: host-side argument validation, then dispatch
// to the gfx950 kernel launchers. Validation touches no GPU state, so every
// error code is returned before anything is enqueued. Built with GDR_DEBUG
// defined, each entry point also checks its inputs' values on the GPU (see
// gdr_debug.hpp) after the host checks and before its first compute kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gdr_internal.h"
#include "gdr_host.hpp"

#ifdef GDR_DEBUG
#include "gdr_debug.hpp"
// Runs a value check and returns its status from the entry point on failure.
#define GDR_DEBUG_CHECK(call)            \
  do {                                   \
    const int gdr_dbg_st_ = (call);      \
    if (gdr_dbg_st_ != GDR_OK) return gdr_dbg_st_; \
  } while (0)
#else
// Release build: the value checks are not compiled.
#define GDR_DEBUG_CHECK(call) \
  do {                        \
  } while (0)
#endif

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

// Checks of the decode entry points.
int check_decode(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                 const void* w, const float* S, const void* o, int N, int H, int dk, int dv, int dtype) {
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
  return GDR_OK;
}

#ifdef GDR_DEBUG
// Value checks of the debug build, one per family of entry points. Sequence
// tensors have B*H*T rows, states B*H; `sname` names the state argument.
using gdr::dbg::Arg;
constexpr int kFin = gdr::dbg::kFinite, kUnit = gdr::dbg::kUnitDecay;

int precheck_gdn(void* stream, const void* q, const void* k, const void* v, const void* alpha,
                 const void* b, const void* w, const float* S, const char* sname, long long B, long long H,
                 long long T, int dk, int dv, int dtype) {
  const size_t nK = (size_t)(B * H * T) * dk, nV = (size_t)(B * H * T) * dv, nS = (size_t)(B * H) * dk * dv;
  const Arg a[] = {{"q", q, nK, dtype, kFin},         {"k", k, nK, dtype, kFin}, {"v", v, nV, dtype, kFin},
                   {"alpha", alpha, nK, dtype, kUnit}, {"b", b, nK, dtype, kFin}, {"w", w, nV, dtype, kFin},
                   {sname, S, nS, GDR_F32, kFin}};
  return gdr::dbg::check(stream, a, 7);
}

int precheck_muir(void* stream, const void* q, const void* k, const void* v, const void* zf, const void* zb,
                  const void* zw, const void* zq, const float* a_log, const float* gamma, const float* S,
                  const char* sname, long long B, long long H, long long T, int dk, int dv, int dtype) {
  const size_t nK = (size_t)(B * H * T) * dk, nV = (size_t)(B * H * T) * dv, nS = (size_t)(B * H) * dk * dv;
  const Arg a[] = {{"q", q, nK, dtype, kFin},      {"k", k, nK, dtype, kFin},
                   {"v", v, nV, dtype, kFin},      {"z_f", zf, nK, dtype, kFin},
                   {"z_b", zb, nK, dtype, kFin},   {"z_w", zw, nV, dtype, kFin},
                   {"z_q", zq, nK, dtype, kFin},   {"a_log", a_log, (size_t)H, GDR_F32, kFin},
                   {"gamma_stat", gamma, (size_t)H * dk, GDR_F32, kFin}, {sname, S, nS, GDR_F32, kFin}};
  return gdr::dbg::check(stream, a, 10);
}

int precheck_mlstm(void* stream, const void* q, const void* k, const void* v, const float* it, const float* ft,
                   const float* C0, const float* n0, const float* m0, int B, int H, int T, int dk, int dv,
                   int dtype) {
  const size_t n = (size_t)B * H * T, nh = (size_t)B * H;
  const Arg a[] = {{"q", q, n * dk, dtype, kFin},   {"k", k, n * dk, dtype, kFin},
                   {"v", v, n * dv, dtype, kFin},   {"i_tilde", it, n, GDR_F32, kFin},
                   {"f_tilde", ft, n, GDR_F32, kFin}, {"C0", C0, nh * dk * dv, GDR_F32, kFin},
                   {"n0", n0, nh * dk, GDR_F32, kFin}, {"m0", m0, nh, GDR_F32, gdr::dbg::kFiniteOrNegInf}};
  return gdr::dbg::check(stream, a, 8);
}

int precheck_rwkv7(void* stream, const void* q, const void* w, const void* a_, const float* c, const void* kw,
                   const void* u, const float* S, const char* sname, int B, int H, int T, int dk, int dv,
                   int dtype) {
  const size_t n = (size_t)B * H * T, nS = (size_t)B * H * dk * dv;
  const Arg a[] = {{"q", q, n * dk, dtype, kFin},  {"w", w, n * dk, dtype, kUnit}, {"a", a_, n * dk, dtype, kFin},
                   {"c", c, n, GDR_F32, kFin},     {"kw", kw, n * dk, dtype, kFin}, {"u", u, n * dv, dtype, kFin},
                   {sname, S, nS, GDR_F32, kFin}};
  return gdr::dbg::check(stream, a, 7);
}

int precheck_bwd_extra(void* stream, const void* dO, const float* dS_T, int B, int H, int T, int dk, int dv,
                       int dtype) {
  const Arg a[] = {{"dO", dO, (size_t)B * H * T * dv, dtype, kFin},
                   {"dS_T", dS_T, (size_t)B * H * dk * dv, GDR_F32, kFin}};
  return gdr::dbg::check(stream, a, 2);
}

int precheck_state(void* stream, const float* S, const char* sname, int B, int H, int dk, int dv) {
  const Arg a[] = {{sname, S, (size_t)B * H * dk * dv, GDR_F32, kFin}};
  return gdr::dbg::check(stream, a, 1);
}
#endif  // GDR_DEBUG

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
    case GDR_ERR_TOO_LARGE:
      return "one head needs more scratch than the library's static array holds (GDR_NOALLOC_SCRATCH_BYTES)";
    case GDR_ERR_PRECONDITION:
      return "an input is not finite, or a decay lies outside (0, 1] (debug library; gdr_debug_violation names it)";
  }
  return "unknown status";
}

int gdr_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                  const void* w, const float* S0, void* o, float* S_out, int B, int H, int T, int dk,
                  int dv, int chunk, int dtype, void* stream) {
  int st = check_chunk(q, k, v, alpha, b, w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  if (dtype == GDR_F32 && dk >= 64 && chunk > 32) return GDR_ERR_UNSUPPORTED;
  GDR_DEBUG_CHECK(precheck_gdn(stream, q, k, v, alpha, b, w, S0, "S0", B, H, T, dk, dv, dtype));
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
  GDR_DEBUG_CHECK(precheck_gdn(stream, q, k, v, alpha, b, w, S0, "S0", B, H, T, dk, dv, dtype));
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
  GDR_DEBUG_CHECK(precheck_gdn(stream, q, k, v, alpha, b, w, nullptr, "S0", B, H, T, dk, dv, dtype));
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
  GDR_DEBUG_CHECK(precheck_state(stream, S0, "S0", B, H, dk, dv));
  gdr::ChunkArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, S0, o, S_out, B, H, T, dk, dv,
                   chunk, dtype, stream};
  return gdr::chunk_fwd_ws_launch(a, const_cast<void*>(workspace), 2);
}

int gdr_decode_step(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                    const void* w, float* S, void* o, int N, int H, int dk, int dv, int dtype,
                    void* stream) {
  int st = check_decode(q, k, v, alpha, b, w, S, o, N, H, dk, dv, dtype);
  if (st != GDR_OK) return st;
  GDR_DEBUG_CHECK(precheck_gdn(stream, q, k, v, alpha, b, w, S, "S", N, H, 1, dk, dv, dtype));
  gdr::DecodeArgs a{q, k, v, alpha, b, w, S, o, N, H, dk, dv, dtype, stream};
  return gdr::decode_launch(a);
}


}  // extern "C"

namespace {

// Extra checks of the Muir gate-prologue entry points: z_q (optional) is a
// [.., dk] input like q; a_log [H] and gamma_stat [H, dk] (optional) are
// float32, 4-byte aligned, and no output may overlap them.
int check_muir_extra(const void* zq, const float* a_log, const float* gamma_stat, const void* o,
                     size_t no, const float* S_out, size_t nS, size_t nK, int H, int dk) {
  if (!a_log) return GDR_ERR_NULL;
  if (!aligned16(zq)) return GDR_ERR_ALIGN;
  if (((uintptr_t)a_log & 3u) || ((uintptr_t)gamma_stat & 3u)) return GDR_ERR_ALIGN;
  struct R { const void* p; size_t n; };
  const R ins[] = {{zq, nK}, {a_log, (size_t)H * 4}, {gamma_stat, (size_t)H * dk * 4}};
  for (const R& x : ins)
    if (overlap(o, no, x.p, x.n) || overlap(S_out, nS, x.p, x.n)) return GDR_ERR_ALIAS;
  return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_muir_chunk_fwd_ws(const void* q, const void* k, const void* v, const void* z_f, const void* z_b,
                          const void* z_w, const void* z_q, const float* a_log, const float* gamma_stat,
                          const float* S0, void* o, float* S_out, int B, int H, int T, int dk, int dv,
                          int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_chunk(q, k, v, z_f, z_b, z_w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  const size_t es = esize(dtype);
  st = check_muir_extra(z_q, a_log, gamma_stat, o, (size_t)B * H * T * dv * es, S_out,
                        (size_t)B * H * dk * dv * 4, (size_t)B * H * T * dk * es, H, dk);
  if (st != GDR_OK) return st;
  st = check_workspace(q, k, v, z_f, z_b, z_w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype, workspace,
                       workspace_bytes);
  if (st != GDR_OK) return st;
  if (overlap(workspace, gdr::chunk_ws_bytes(B, H, T, dk, dv, chunk, dtype), z_q, (size_t)B * H * T * dk * es))
    return GDR_ERR_ALIAS;
  GDR_DEBUG_CHECK(precheck_muir(stream, q, k, v, z_f, z_b, z_w, z_q, a_log, gamma_stat, S0, "S0", B, H, T, dk,
                                dv, dtype));
  gdr::ChunkArgs a{q, k, v, z_f, z_b, z_w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype, stream};
  a.gated = true;
  a.zq = z_q;
  a.a_log = a_log;
  a.gamma_stat = gamma_stat;
  return gdr::chunk_fwd_ws_launch(a, workspace, 3);
}

int gdr_muir_decode_step(const void* q, const void* k, const void* v, const void* z_f, const void* z_b,
                         const void* z_w, const void* z_q, const float* a_log, const float* gamma_stat,
                         float* S, void* o, int N, int H, int dk, int dv, int dtype, void* stream) {
  int st = check_decode(q, k, v, z_f, z_b, z_w, S, o, N, H, dk, dv, dtype);
  if (st != GDR_OK) return st;
  const size_t es = esize(dtype);
  st = check_muir_extra(z_q, a_log, gamma_stat, o, (size_t)N * H * dv * es, S,
                        (size_t)N * H * dk * dv * 4, (size_t)N * H * dk * es, H, dk);
  if (st != GDR_OK) return st;
  GDR_DEBUG_CHECK(precheck_muir(stream, q, k, v, z_f, z_b, z_w, z_q, a_log, gamma_stat, S, "S", N, H, 1, dk, dv,
                                dtype));
  gdr::DecodeArgs a{q, k, v, z_f, z_b, z_w, S, o, N, H, dk, dv, dtype, stream};
  a.gated = true;
  a.zq = z_q;
  a.a_log = a_log;
  a.gamma_stat = gamma_stat;
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
  GDR_DEBUG_CHECK(precheck_mlstm(stream, q, k, v, i_tilde, f_tilde, C0, n0, m0, B, H, T, dk, dv, dtype));
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
  GDR_DEBUG_CHECK(precheck_mlstm(stream, q, k, v, i_tilde, f_tilde, C0, n0, m0, B, H, T, dk, dv, dtype));
  gdr::MlstmArgs a{q, k, v, i_tilde, f_tilde, C0, n0, m0, h, C_out, n_out, m_out,
                   B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::mlstm_ws_launch(a, workspace);
}

}  // extern "C"

// ------------------------------------------------------------------ backward
extern "C" int gdr_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk, int dtype,
                                            size_t* bytes) {
  if (!bytes) return GDR_ERR_NULL;
  *bytes = 0;
  int st = check_sizes(B, H, T, dk, dv, dtype, 128);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDR_ERR_UNSUPPORTED;
  *bytes = gdr::chunk_bwd_ws_bytes(B, H, T, dk, dv, chunk, dtype);
  return GDR_OK;
}

extern "C" int gdr_chunk_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                             const void* w, const float* S0, const void* dO, const float* dS_T, float* dq,
                             float* dk_, float* dv_, float* dalpha, float* db, float* dw, float* dS0, int B,
                             int H, int T, int dk, int dv, int chunk, int dtype, void* workspace,
                             size_t workspace_bytes, int records_ready, void* stream) {
  int st = check_chunk_inputs(q, k, v, alpha, b, w, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  if (!dO || !dq || !dk_ || !dv_ || !dalpha || !db || !dw || !workspace) return GDR_ERR_NULL;
  const void* al[] = {S0, dO, dS_T, dq, dk_, dv_, dalpha, db, dw, dS0, workspace};
  for (const void* p : al)
    if (!aligned16(p)) return GDR_ERR_ALIGN;
  const size_t need = gdr::chunk_bwd_ws_bytes(B, H, T, dk, dv, chunk, dtype);
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE;
  const size_t es = esize(dtype), n = (size_t)B * H * T;
  const size_t nK = n * dk * es, nV = n * dv * es, nS = (size_t)B * H * dk * dv * 4;
  struct R { const void* p; size_t n; };
  const R ins[] = {{q, nK}, {k, nK}, {alpha, nK}, {b, nK}, {v, nV}, {w, nV}, {S0, nS}, {dO, nV}, {dS_T, nS}};
  const R outs[] = {{dq, n * dk * 4}, {dk_, n * dk * 4}, {dalpha, n * dk * 4}, {db, n * dk * 4},
                    {dv_, n * dv * 4}, {dw, n * dv * 4}, {dS0, nS}, {workspace, need}};
  for (const R& x : outs) {
    for (const R& y : ins)
      if (overlap(x.p, x.n, y.p, y.n)) return GDR_ERR_ALIAS;
    for (const R& y : outs)
      if (x.p != y.p && overlap(x.p, x.n, y.p, y.n)) return GDR_ERR_ALIAS;
  }
  GDR_DEBUG_CHECK(precheck_gdn(stream, q, k, v, alpha, b, w, S0, "S0", B, H, T, dk, dv, dtype));
  GDR_DEBUG_CHECK(precheck_bwd_extra(stream, dO, dS_T, B, H, T, dk, dv, dtype));
  gdr::ChunkBwdArgs a{q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk_, dv_, dalpha, db, dw, dS0,
                      B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::chunk_bwd_launch(a, workspace, records_ready != 0);
}

// ------------------------------------------------------------------ RWKV-7
namespace {

int check_rwkv7(const void* q, const void* w, const void* a, const float* c, const void* kw, const void* u,
                const float* S0, const void* o, const float* S_out, int B, int H, int T, int dk, int dv,
                int dtype) {
  if (!q || !w || !a || !c || !kw || !u || !o) return GDR_ERR_NULL;
  int st = check_sizes(B, H, T, dk, dv, dtype, 128);
  if (st != GDR_OK) return st;
  const void* ptrs[] = {q, w, a, c, kw, u, S0, o, S_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDR_ERR_ALIGN;
  const size_t es = esize(dtype), n = (size_t)B * H * T;
  const size_t nK = n * dk * es, nV = n * dv * es, nS = (size_t)B * H * dk * dv * 4;
  struct R { const void* p; size_t n; };
  const R ins[] = {{q, nK}, {w, nK}, {a, nK}, {c, n * 4}, {kw, nK}, {u, nV}};
  for (const R& x : ins) {
    if (overlap(o, nV, x.p, x.n) || overlap(S_out, nS, x.p, x.n)) return GDR_ERR_ALIAS;
  }
  if (overlap(o, nV, S0, nS) || overlap(o, nV, S_out, nS)) return GDR_ERR_ALIAS;
  if (S_out && S0 && S_out != S0 && overlap(S_out, nS, S0, nS)) return GDR_ERR_ALIAS;
  return GDR_OK;
}

}  // namespace

extern "C" int gdr_rwkv7_workspace_size(int B, int H, int T, int dk, int dv, int chunk, size_t* bytes) {
  if (!bytes) return GDR_ERR_NULL;
  *bytes = 0;
  int st = check_sizes(B, H, T, dk, dv, GDR_F32, 128);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32) return GDR_ERR_UNSUPPORTED;
  *bytes = gdr::rwkv7_ws_bytes(B, H, T, dk, dv, chunk);
  return GDR_OK;
}

extern "C" int gdr_rwkv7_fwd(const void* q, const void* w, const void* a, const float* c, const void* kw,
                             const void* u, const float* S0, void* o, float* S_out, int B, int H, int T, int dk,
                             int dv, int chunk, int dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int st = check_rwkv7(q, w, a, c, kw, u, S0, o, S_out, B, H, T, dk, dv, dtype);
  if (st != GDR_OK) return st;
  if (chunk != 16 && chunk != 32) return GDR_ERR_UNSUPPORTED;
  if (!workspace) return GDR_ERR_NULL;
  if (!aligned16(workspace)) return GDR_ERR_ALIGN;
  const size_t need = gdr::rwkv7_ws_bytes(B, H, T, dk, dv, chunk);
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE;
  const size_t es = esize(dtype), n = (size_t)B * H * T, nS = (size_t)B * H * dk * dv * 4;
  const void* bufs[] = {q, w, a, kw};
  for (const void* p : bufs)
    if (overlap(workspace, need, p, n * dk * es)) return GDR_ERR_ALIAS;
  if (overlap(workspace, need, u, n * dv * es) || overlap(workspace, need, o, n * dv * es) ||
      overlap(workspace, need, c, n * 4) || overlap(workspace, need, S0, nS) ||
      overlap(workspace, need, S_out, nS))
    return GDR_ERR_ALIAS;
  GDR_DEBUG_CHECK(precheck_rwkv7(stream, q, w, a, c, kw, u, S0, "S0", B, H, T, dk, dv, dtype));
  gdr::Rwkv7Args r{q, w, a, c, kw, u, S0, o, S_out, B, H, T, dk, dv, chunk, dtype, stream};
  return gdr::rwkv7_fwd_launch(r, workspace);
}

extern "C" int gdr_rwkv7_decode_step(const void* q, const void* w, const void* a, const float* c, const void* kw,
                                     const void* u, float* S, void* o, int N, int H, int dk, int dv, int dtype,
                                     void* stream) {
  if (!S) return GDR_ERR_NULL;
  int st = check_rwkv7(q, w, a, c, kw, u, nullptr, o, S, N, H, 1, dk, dv, dtype);
  if (st != GDR_OK) return st;
  GDR_DEBUG_CHECK(precheck_rwkv7(stream, q, w, a, c, kw, u, S, "S", N, H, 1, dk, dv, dtype));
  gdr::Rwkv7Args r{q, w, a, c, kw, u, nullptr, o, S, N, H, 1, dk, dv, 16, dtype, stream};
  return gdr::rwkv7_decode_launch(r);
}

// ------------------------------------------------------------------ no-allocation entry point
//
// gdr_chunk_fwd_noalloc runs the two-kernel chunk forward through a scratch
// array that lives in the library's code object instead of a caller
// workspace. Each GPU the library runs on holds its own copy of the array
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory, so its device address is looked up once per device with
// hipGetSymbolAddress and only that address is passed to kernels.

namespace {

constexpr size_t kScratchBytes = GDR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

// per-device device address of `scratch` (null until first looked up)
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's `scratch`; called with that device current.
// Concurrent first calls look up the same address, so the race is benign.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" int gdr_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                                     const void* b, const void* w, const float* S0, void* o, float* S_out,
                                     int B, int H, int T, int dk, int dv, int chunk, int dtype,
                                     void* stream) {
  int st = check_chunk(q, k, v, alpha, b, w, S0, o, S_out, B, H, T, dk, dv, chunk, dtype);
  if (st != GDR_OK) return st;
  // heads are independent: they go through the scratch array in groups of
  // consecutive (b, h) pairs, as many per group as the array holds
  const size_t per_head = gdr::chunk_ws_bytes(1, 1, T, dk, dv, chunk, dtype, false);
  if (per_head > kScratchBytes) return GDR_ERR_TOO_LARGE;
  GDR_DEBUG_CHECK(precheck_gdn(stream, q, k, v, alpha, b, w, S0, "S0", B, H, T, dk, dv, dtype));
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GDR_ERR_LAUNCH;
  if (gdr::stream_device(stream) != dev) return GDR_ERR_LAUNCH;
  char* ws = (char*)scratch_ptr(dev);
  if (!ws) return GDR_ERR_LAUNCH;
  const long long heads = (long long)B * H;
  const long long group = (long long)(kScratchBytes / per_head);
  const size_t es = esize(dtype);
  for (long long h0 = 0; h0 < heads; h0 += group) {
    const int g = (int)(heads - h0 < group ? heads - h0 : group);
    const size_t oK = (size_t)h0 * T * dk * es, oV = (size_t)h0 * T * dv * es;
    const size_t oS = (size_t)h0 * dk * dv;
    gdr::ChunkArgs a{(const char*)q + oK, (const char*)k + oK, (const char*)v + oV,
                     (const char*)alpha + oK, (const char*)b + oK, (const char*)w + oV,
                     S0 ? S0 + oS : nullptr, (char*)o + oV, S_out ? S_out + oS : nullptr,
                     1, g, T, dk, dv, chunk, dtype, stream};
    a.no_seg = true;   // records only: the scratch is sized per head
    st = gdr::chunk_fwd_ws_launch(a, ws, 3);
    if (st != GDR_OK) return st;
  }
  return GDR_OK;
}
