// chain_noalloc.hip -- the chain selected inverse without a caller-provided
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The chain kernels' scratch (the collect -> distribute state and, for few
// long b = 32 chains, the segment and separator buffers) lives in one
// file-scope device array of fixed size.  Its device address is looked up
// once per device with hipGetSymbolAddress (the array's name is not a device
// address in host code) and passed to the same kernels the workspace entry
// points launch.  Every location the kernels read is written earlier in the
// same call, so nothing has to be cleared between calls.  All calls on one
// device share the array: calls that overlap in time on one device race.
#include <mutex>

#include "internal.h"

namespace selinv {
namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;  // 256 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// The array's device address on the current device (looked up once per
// device), or nullptr with the HIP error in *err.
void *device_scratch(hipError_t *err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

template <typename T>
int chain_noalloc(int64_t B, int64_t L, int32_t b, const T *diag, const T *lower, T *G_diag,
                  T *G_lower, double *logdet, int32_t *info, void *stream) {
  if (B < 0 || L < 1 || b < 1 || b > SELINV_MAX_B || B > 0x7fffffff)
    return SELINV_ERR_INVALID_ARG;
  if (B == 0) return SELINV_OK;
  if (!diag || !G_diag || !logdet) return SELINV_ERR_INVALID_ARG;
  if (L > 1 && (!lower || !G_lower)) return SELINV_ERR_INVALID_ARG;
  auto misaligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(diag) || misaligned(G_diag) ||
      (L > 1 && (misaligned(lower) || misaligned(G_lower))))
    return SELINV_ERR_INVALID_ARG;
  const size_t need = chain_workspace_bytes(sizeof(T), B, L, b);
  if (need > kScratchBytes) return SELINV_ERR_SCRATCH_LIMIT;
  hipError_t e = hipSuccess;
  void *ws = device_scratch(&e);
  if (!ws) return SELINV_ERR_HIP;
  e = chain_launch<T>(B, L, b, diag, lower, G_diag, G_lower, logdet, info, ws,
                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELINV_OK : SELINV_ERR_HIP;
}

}  // namespace
}  // namespace selinv

extern "C" size_t selinv_chain_static_scratch_bytes(void) { return selinv::kScratchBytes; }

extern "C" int selinv_chain_noalloc_f64(int64_t B, int64_t L, int32_t b, const double *diag,
                                        const double *lower, double *G_diag, double *G_lower,
                                        double *logdet, int32_t *info, void *stream) {
  return selinv::chain_noalloc<double>(B, L, b, diag, lower, G_diag, G_lower, logdet, info,
                                       stream);
}

extern "C" int selinv_chain_noalloc_f32(int64_t B, int64_t L, int32_t b, const float *diag,
                                        const float *lower, float *G_diag, float *G_lower,
                                        double *logdet, int32_t *info, void *stream) {
  return selinv::chain_noalloc<float>(B, L, b, diag, lower, G_diag, G_lower, logdet, info,
                                      stream);
}
