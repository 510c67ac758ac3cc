// The split-K GEMM entry point for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): its split-K partial sums live in one file-scope device
// array of a fixed size instead of a per-call workspace.
//
// Host code never passes the array's name to a kernel: in host code that
// name is a host-side stand-in, not the device address.  The device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept per device; every use goes through it.
#include <mutex>

#include "../../include/s1.h"
#include "../../include/s1_kernels.h"
#include "internal.h"

namespace s1 {
namespace {

constexpr size_t SCRATCH_BYTES = (size_t)S1K_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on the current device (looked up on the
// first call per device).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(S1_EDEVICE, hip_msg(e, "s1k_gemm_noalloc: no device"));
  if (dev < 0 || dev >= MAX_DEVICES) return set_error(S1_EDEVICE, "s1k_gemm_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(S1_EDEVICE, hip_msg(e, "s1k_gemm_noalloc: scratch address lookup"));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return S1_OK;
}

}  // namespace
}  // namespace s1

using namespace s1;

extern "C" int s1k_gemm_noalloc(int32_t dtype, const void* A, const void* W, float* C, int32_t M, int32_t N,
                                int32_t K, int32_t split_k, void* hip_stream) {
  const bool bf16 = dtype == S1_BF16;
  if ((dtype != S1_BF16 && dtype != S1_F32) || M < 0 || N < 0 || K < 1 || split_k < 1 || K % (bf16 ? 8 : 4) ||
      (split_k > 1 && N % 4) || !A || !W || !C)
    return set_error(S1_EINVAL, "s1k_gemm_noalloc: unsupported arguments");
  if ((long long)split_k * M * N * (long long)sizeof(float) > (long long)SCRATCH_BYTES)
    return set_error(S1_EINVAL, "s1k_gemm_noalloc: split_k * M * N * 4 bytes exceed the " +
                                    std::to_string(SCRATCH_BYTES) + "-byte scratch");
  GemmArgs g{};
  g.A = A;
  g.W = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = K;
  g.ldw = K;
  g.out0 = C;
  g.ld0 = N;
  float* ws = nullptr;
  if (split_k > 1) {
    void* p = nullptr;
    const int rc = scratch_ptr(&p);
    if (rc) return rc;
    ws = static_cast<float*>(p);
  }
  // every split writes its whole partial slab before the ordered reduction
  // reads it, so nothing in the scratch needs clearing
  const hipError_t e = launch_gemm(bf16, EPI_F32, g, split_k, ws, static_cast<hipStream_t>(hip_stream), GEMM_AUTO);
  return e == hipSuccess ? S1_OK : set_error(S1_EDEVICE, hip_msg(e, "s1k_gemm_noalloc"));
}
