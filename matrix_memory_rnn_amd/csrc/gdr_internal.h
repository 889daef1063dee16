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
};

struct DecodeArgs {
  const void *q, *k, *v, *alpha, *b, *w;
  float* S;
  void* o;
  int N, H, dk, dv, dtype;
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
size_t chunk_ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype);
// phases: bit 0 = intra-chunk kernel (writes the workspace), bit 1 = chunk scan
int chunk_fwd_ws_launch(const ChunkArgs& a, void* ws, int phases);
int decode_launch(const DecodeArgs& a);
int mlstm_launch(const MlstmArgs& a);
// two-kernel form (intra-chunk kernel over all chunks, then the chunk scan)
size_t mlstm_ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype);
int mlstm_ws_launch(const MlstmArgs& a, void* ws);

}  // namespace gdr
