// The GDR_DEBUG input checks (declared in gdr_debug.hpp) and the two exported
// queries gdr_debug_build / gdr_debug_violation, which every build has.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr.h"

#ifdef GDR_DEBUG

#include <atomic>
#include <mutex>
#include <string>

#include "gdr_debug.hpp"
#include "gdr_host.hpp"

namespace gdr::dbg {
namespace {

struct ArgTable {
  const void* p[kMaxArgs];
  unsigned long long n[kMaxArgs];
  int dtype[kMaxArgs];
  int kind[kMaxArgs];
};

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 2048;

__device__ inline bool element_ok(float x, int kind) {
  if (kind == kUnitDecay) return x > 0.f && x <= 1.f;  // false for NaN
  if (kind == kFiniteOrNegInf) return isfinite(x) || x == -INFINITY;
  return isfinite(x);
}

// Grid (blocks, arguments): block row y reads argument y with a grid-stride
// loop and sets bit y of *flag if any element breaks its rule.
__global__ void __launch_bounds__(kThreads) check_kernel(ArgTable t, unsigned* flag) {
  const int y = blockIdx.y;
  const unsigned long long n = t.n[y];
  const int kind = t.kind[y];
  const unsigned long long stride = (unsigned long long)gridDim.x * kThreads;
  bool bad = false;
  if (t.dtype[y] == GDR_BF16) {
    const uint16_t* p = (const uint16_t*)t.p[y];
    for (unsigned long long i = (unsigned long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
      bad |= !element_ok(__uint_as_float((unsigned)p[i] << 16), kind);
  } else {
    const float* p = (const float*)t.p[y];
    for (unsigned long long i = (unsigned long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
      bad |= !element_ok(p[i], kind);
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1u << y);
}

__global__ void clear_kernel(unsigned* flag) {
  if (threadIdx.x == 0) *flag = 0u;
}

// One violation word per device, looked up per device like any device symbol.
static __device__ unsigned violation_word;

constexpr int kMaxDevices = 64;
std::atomic<void*> g_word[kMaxDevices];
std::mutex g_mu;  // the word is shared by every call on a device

thread_local std::string t_violation;

void* word_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_word[dev].load(std::memory_order_acquire);
  if (p) return p;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(violation_word));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !p) return nullptr;
  g_word[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

int check(void* stream, const Arg* args, int nargs) {
  t_violation.clear();
  if (nargs > kMaxArgs) return GDR_ERR_LAUNCH;
  ArgTable t{};
  int m = 0;
  unsigned long long most = 0;
  const Arg* used[kMaxArgs];
  for (int i = 0; i < nargs; ++i) {
    if (!args[i].p || args[i].n == 0) continue;
    t.p[m] = args[i].p;
    t.n[m] = args[i].n;
    t.dtype[m] = args[i].dtype;
    t.kind[m] = args[i].kind;
    used[m] = &args[i];
    if (args[i].n > most) most = args[i].n;
    ++m;
  }
  if (m == 0) return GDR_OK;
  unsigned* word = (unsigned*)word_ptr(stream_device(stream));
  if (!word) return GDR_ERR_LAUNCH;
  unsigned long long blocks = (most + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  unsigned h = 0;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    hipStream_t s = (hipStream_t)stream;
    clear_kernel<<<1, 64, 0, s>>>(word);
    check_kernel<<<dim3((unsigned)blocks, m), kThreads, 0, s>>>(t, word);
    if (hipGetLastError() != hipSuccess) return GDR_ERR_LAUNCH;
    if (hipMemcpyAsync(&h, word, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess) return GDR_ERR_LAUNCH;
    if (hipStreamSynchronize(s) != hipSuccess) return GDR_ERR_LAUNCH;
  }
  if (h == 0) return GDR_OK;
  for (int i = 0; i < m; ++i)
    if (h & (1u << i)) {
      if (!t_violation.empty()) t_violation += ", ";
      t_violation += used[i]->name;
    }
  return GDR_ERR_PRECONDITION;
}

}  // namespace gdr::dbg

extern "C" int gdr_debug_build(void) { return 1; }

extern "C" const char* gdr_debug_violation(void) { return gdr::dbg::t_violation.c_str(); }

#else  // release build: no checks

extern "C" int gdr_debug_build(void) { return 0; }

extern "C" const char* gdr_debug_violation(void) { return ""; }

#endif
