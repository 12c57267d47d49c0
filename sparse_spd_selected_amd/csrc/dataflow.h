// dataflow.h -- ordering between the workgroups of one kernel, for level-set
// schedules (tree collect / distribute) run as a single launch per pass
// instead of one launch per level.
//
// A flag word per producer position records how far it has got; a consumer
// waits for the flags of the positions it reads.  Workgroup indices put every
// producer before its consumers (collect: deepest level first; distribute:
// root level first).  Workgroups are started in index order, so a producer
// has always started before a consumer waits for it, and the lowest
// unfinished workgroup never waits: the pass cannot deadlock.
//
// Coherence: the per-XCD L2 caches are not coherent with one another, and
// an agent-scope fence writes back (release) or invalidates (acquire) a whole
// L2 -- at one publish per wavefront that costs several times the work
// itself.  Instead every value that one workgroup of a kernel writes and
// another workgroup of the same kernel reads is written and read with
// device-coherent accesses (agent-scope atomic loads and stores), which are
// performed at the point of coherence.  A producer sets its flag only after
// its vector memory counter has drained, i.e. after all its stores have
// completed there; a consumer issues its coherent loads only after it has
// seen the flag.  The workgroup-scope fences keep the compiler from moving
// those accesses across the handshake.  Values read only by a later kernel
// need none of this (a kernel boundary orders them).
//
// Every wait is bounded: after `wait_ticks` of the 100 MHz constant clock it
// sets *timeout and gives up, and every later wait of the call gives up at
// once, so a schedule that cannot make progress ends with an error report
// (info = -1, NaN results) instead of hanging.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "rows8.h"

namespace selinv {
namespace df {

template <typename T>
__device__ __forceinline__ T load_coherent(const T *p) {
  using U = typename std::conditional<sizeof(T) == 8, uint64_t, uint32_t>::type;
  const U u = __hip_atomic_load(reinterpret_cast<const U *>(p), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(T, u);
}

template <typename T>
__device__ __forceinline__ void store_coherent(T *p, T v) {
  using U = typename std::conditional<sizeof(T) == 8, uint64_t, uint32_t>::type;
  __hip_atomic_store(reinterpret_cast<U *>(p), __builtin_bit_cast(U, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Reads of values that other workgroups of the same launch stored with
// store_coherent, performed at the point of coherence as load_coherent's
// are (the same cache policy, sc1) but as plain buffer loads: the compiler
// waits for every atomic load before the next one is issued, while these can
// be in flight together.  Reads must follow the handshake (acquire()), and
// the region [base, base + n) must be smaller than 2^31 bytes.
template <typename T>
struct CoherentReader {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte values");
  static constexpr int kWord3 = 0x00020000;  // untyped buffer access (gfx9 family)
  static constexpr int kSc1 = 16;            // cache policy: device scope
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ CoherentReader(const T *base, int64_t n)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(base), static_cast<short>(0),
                                            static_cast<int>(n * int64_t(sizeof(T))), kWord3)) {}
  __device__ __forceinline__ T operator[](int64_t i) const {
    const int off = static_cast<int>(i * int64_t(sizeof(T)));
    if constexpr (sizeof(T) == 8)
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSc1));
    else
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1));
  }
};

// Row i of an 8 x 8 state block stored interleaved, element (i, c) at
// c * 8 + i, so that each coherent access instruction covers 64 contiguous
// bytes of a slot.
template <typename T>
__device__ __forceinline__ r8::Row<T> load_interleaved(const T *P, int i) {
  r8::Row<T> r;
#pragma unroll
  for (int c = 0; c < 8; ++c) r.v[c] = load_coherent(P + c * 8 + i);
  return r;
}

template <typename T>
__device__ __forceinline__ void store_interleaved(T *P, int i, const r8::Row<T> &r) {
#pragma unroll
  for (int c = 0; c < 8; ++c) store_coherent(P + c * 8 + i, r.v[c]);
}

// Row i of a b x b block that a consumer reads back as rows, kept in a
// row-major array as the transpose of those rows: element (i, c) at
// c * b + i (contiguous across the rows of a slot).  For a block that is
// symmetric in exact arithmetic (a diagonal block of A^-1) the array holds
// that block either way.
template <typename T>
__device__ __forceinline__ r8::Row<T> load_transposed(const T *P, int b, int i) {
  r8::Row<T> r;
#pragma unroll
  for (int c = 0; c < 8; ++c) r.v[c] = (i < b && c < b) ? load_coherent(P + c * b + i) : T(0);
  return r;
}

template <typename T>
__device__ __forceinline__ void store_transposed(T *P, int b, int i, const r8::Row<T> &r) {
  if (i >= b) return;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    if (c < b) store_coherent(P + c * b + i, r.v[c]);
}

// The end of a wait that starts now and lasts `ticks` (clamped, so that a
// huge limit cannot wrap around).
__device__ __forceinline__ uint64_t deadline_after(uint64_t ticks) {
  const uint64_t cap = uint64_t(1) << 62;
  return static_cast<uint64_t>(wall_clock64()) + (ticks < cap ? ticks : cap);
}

// Lanes sub, sub + stride, ... of [beg, end) wait until flags[c] >= want.
__device__ __forceinline__ void wait_flags(const int32_t *flags, int64_t beg, int64_t end,
                                           int32_t want, int sub, int stride, int32_t *timeout,
                                           uint64_t deadline) {
  for (int64_t c = beg + sub; c < end; c += stride) {
    while (__hip_atomic_load(flags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
      if (__hip_atomic_load(timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
      if (static_cast<uint64_t>(wall_clock64()) >= deadline) {
        __hip_atomic_store(timeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

__device__ __forceinline__ bool timed_out(int32_t *timeout) {
  return __hip_atomic_load(timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// After the waits of a workgroup: no coherent load moves above this point.
__device__ __forceinline__ void acquire() {
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Sets flags[p] = value (for the lanes with `mine`) once every store of the
// workgroup has completed.
__device__ __forceinline__ void publish(int32_t *flags, int64_t p, bool mine, int32_t value) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores have completed
  __syncthreads();
  if (mine) __hip_atomic_store(flags + p, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// flags[0 .. n) = 0, *first_fail = INT32_MAX (if given), *timeout = 0
static __global__ __launch_bounds__(256) void init_kernel(int64_t n, int32_t *__restrict__ flags,
                                                          int32_t *__restrict__ first_fail,
                                                          int32_t *__restrict__ timeout) {
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t k = k0; k < n; k += static_cast<int64_t>(gridDim.x) * blockDim.x) flags[k] = 0;
  if (k0 == 0) {
    if (first_fail) *first_fail = INT32_MAX;
    *timeout = 0;
  }
}

inline hipError_t launch_init(int64_t n, int32_t *flags, int32_t *first_fail, int32_t *timeout,
                              hipStream_t s) {
  const int64_t g = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(g < 1 ? 1 : (g > 1024 ? 1024 : g));
  hipLaunchKernelGGL(init_kernel, dim3(grid), dim3(256), 0, s, n, flags, first_fail, timeout);
  return hipGetLastError();
}

}  // namespace df

// Bound of every dataflow wait, in ticks of the 100 MHz constant clock
// (default 2^24, about 0.17 s); set by selinv_set_wait_limit.
uint64_t wait_limit_ticks();

}  // namespace selinv
