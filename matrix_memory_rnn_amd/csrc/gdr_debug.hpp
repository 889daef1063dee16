// Input checks of the GDR_DEBUG build of libgdr.
//
// The kernels take two things on trust that the host cannot see without
// reading device memory: every input element is finite, and every decay
// (alpha of the gated delta rule, w of RWKV-7) lies in (0, 1], the domain of
// the per-channel decay in "Muir: Linear Attention with Sensitivity-Allocated
// Gating and Matched-Filter Readout" §2.1 eq.(1). A build with GDR_DEBUG
// defined checks both before it enqueues any compute kernel: one small
// grid-stride kernel reads every input once and sets a per-argument bit in a
// device word, the word is copied back, and the stream is synchronised. A
// violation returns GDR_ERR_PRECONDITION with nothing else enqueued, and
// gdr_debug_violation() names the arguments that failed.
//
// The check synchronises the stream, so debug builds cannot be captured into a
// HIP graph, and it reads every input once more (about one extra pass over the
// inputs per call). Release builds compile none of this.
#pragma once

#include <stddef.h>

namespace gdr::dbg {

enum Kind : int {
  kFinite = 0,         // every element finite
  kUnitDecay = 1,      // every element in (0, 1]
  kFiniteOrNegInf = 2  // finite or -inf (the mLSTM stabiliser m0)
};

struct Arg {
  const char* name;  // argument name as in gdr.h
  const void* p;     // device pointer; null means "not passed" and is skipped
  size_t n;          // element count
  int dtype;         // GDR_F32 or GDR_BF16
  int kind;          // Kind
};

constexpr int kMaxArgs = 16;

// Runs the checks of `args` on `stream` and waits for them. Returns GDR_OK,
// GDR_ERR_PRECONDITION (and records the failing names for
// gdr_debug_violation on the calling thread), or GDR_ERR_LAUNCH.
int check(void* stream, const Arg* args, int nargs);

}  // namespace gdr::dbg
