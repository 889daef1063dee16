// Internal host-side interface between the C-ABI entry points (gdr_api.hip)
// and the kernel launchers. Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>
#include <type_traits>

#include "../../include/gdr.h"

namespace gdr {

struct ChunkArgs {
  const void *q, *k, *v, *alpha, *b, *w;
  const float* S0;
  void* o;
  float* S_out;
  int B, H, T, dk, dv, chunk, dtype;
  void* stream;
  // gate logits in place of the gates (alpha, b, w hold z_f, z_b, z_w): the
  // Muir gate prologue; zq (may be NULL), a_log [H], gamma_stat [H, dk] (may be NULL)
  bool gated = false;
  const void* zq = nullptr;
  const float* a_log = nullptr;
  const float* gamma_stat = nullptr;
  // plain chunk scan even where the sequence-segmented one would be used
  bool no_seg = false;
};

struct DecodeArgs {
  const void *q, *k, *v, *alpha, *b, *w;
  float* S;
  void* o;
  int N, H, dk, dv, dtype;
  void* stream;
  // Muir gate prologue, as in ChunkArgs
  bool gated = false;
  const void* zq = nullptr;
  const float* a_log = nullptr;
  const float* gamma_stat = nullptr;
};

struct ChunkBwdArgs {
  const void *q, *k, *v, *alpha, *b, *w;
  const float* S0;
  const void* dO;
  const float* dS_T;
  float *dq_out, *dk_out, *dv_out, *dalpha_out, *db_out, *dw_out, *dS0;
  int B, H, T, dk, dv, chunk, dtype;
  void* stream;
};

// RWKV-7 generalized delta rule: decay w, removal direction a, removal
// coefficient c (fp32 [B,H,T] or [N,H]), write key kw, value u; for the decode
// step S_out is the resident state and B the sequence count.
struct Rwkv7Args {
  const void *q, *w, *a;
  const float* c;
  const void *kw, *u;
  const float* S0;
  void* o;
  float* S_out;
  int B, H, T, dk, dv, chunk, dtype;
  void* stream;
};

struct MlstmArgs {
  const void *q, *k, *v;
  const float *i_tilde, *f_tilde, *C0, *n0, *m0;
  void* h;
  float *C_out, *n_out, *m_out;
  int B, H, T, dk, dv, chunk, dtype;
  void* stream;
};

int chunk_fwd_launch(const ChunkArgs& a);
// two-kernel form (intra-chunk kernel over all chunks, then the chunk scan)
// allow_seg: include the buffers of the sequence-segmented scan where the
// shapes take it (false for callers that launch with no_seg)
size_t chunk_ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype, bool allow_seg = true);
// phases: bit 0 = intra-chunk kernel (writes the workspace), bit 1 = chunk scan
int chunk_fwd_ws_launch(const ChunkArgs& a, void* ws, int phases);
// chunkwise backward: workspace = the forward records, then the backward's
// own buffers; records_ready skips recomputing the records
size_t chunk_bwd_ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype);
// Every chunk-start state (fp32, [b*H + h][chunk][dk][dv]) from F-order
// records; GDR_ERR_UNSUPPORTED for shapes without them.
int chunk_states_fm_launch(const ChunkArgs& a, const void* ws, float* Hst);
int chunk_bwd_launch(const ChunkBwdArgs& a, void* ws, bool records_ready);
int decode_launch(const DecodeArgs& a);
size_t rwkv7_ws_bytes(int B, int H, int T, int dk, int dv, int chunk);
int rwkv7_fwd_launch(const Rwkv7Args& a, void* ws);
int rwkv7_decode_launch(const Rwkv7Args& a);
int mlstm_launch(const MlstmArgs& a);
// two-kernel form (intra-chunk kernel over all chunks, then the chunk scan)
size_t mlstm_ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype);
int mlstm_ws_launch(const MlstmArgs& a, void* ws);

}  // namespace gdr
