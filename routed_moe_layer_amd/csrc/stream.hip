// Chunk-streamed front end: the device side of a fixed ring of token slots with
// independent readiness generations ("[RFC] Chunk-ready symmetric-buffer protocol for
// streaming MegaMoE inputs", sections "Fixed-capacity ring", "Independent readiness
// generations" and "Memory ordering"), for one rank.
//
// Per slot s the ring holds one 64-byte counter record (RingSlot).  A producer of a
// payload part (the routing part: expert ids and route weights; the layout part: x) owns
// one sequence counter per slot; its k-th use of the slot publishes generation k.  The
// consumer owns its own per-slot sequence and reads the slot once both ready generations
// reach its next generation; it then publishes that generation as consumed, after which
// the producers may overwrite the slot.  Every sequence lives in device memory, so a
// captured launch sequence stays consistent over any number of replays (no epoch comes
// from the host), and 32-bit generations are compared by signed difference.
//
// Waits are one-thread kernels polling with system-scope acquire loads, bounded by a
// wall-clock deadline: a wait that expires records a status code (the first one wins) and
// ends, so a missing publish never leaves a wave spinning.  Publishes are system-scope
// release stores issued after the payload writes that precede them on the same stream.
#include "common.h"
#include <algorithm>

#include "kernels.h"

namespace rmoe {

__device__ __forceinline__ uint32_t load_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ bool reached(uint32_t gen, uint32_t want) {
  return static_cast<int32_t>(gen - want) >= 0;
}

__global__ __launch_bounds__(64) void ring_init_kernel(uint32_t* __restrict__ words, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    words[i] = 0u;
}

// Wait until *a (and *b when given) reach *seq + add, or until `ticks` of the constant
// wall clock have passed; then status gets `code` unless an earlier failure is recorded.
__global__ __launch_bounds__(64) void ring_wait_kernel(const uint32_t* a, const uint32_t* b,
                                                       const uint32_t* seq, uint32_t add,
                                                       int64_t ticks, uint32_t* status,
                                                       uint32_t code) {
  if (threadIdx.x != 0) return;
  const uint32_t want = *seq + add;
  const int64_t deadline = wall_clock64() + ticks;
  while (true) {
    const bool ok = reached(load_acquire(a), want) && (b == nullptr || reached(load_acquire(b), want));
    if (ok) return;
    if (wall_clock64() > deadline) {
      atomicCAS(status, 0u, code);
      return;
    }
    __builtin_amdgcn_s_sleep(4);
  }
}

// Advance the owner's sequence of one slot and publish it.
__global__ __launch_bounds__(64) void ring_publish_kernel(uint32_t* gen, uint32_t* seq) {
  if (threadIdx.x != 0) return;
  const uint32_t v = *seq + 1u;
  *seq = v;
  __hip_atomic_store(gen, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Copy of a slot's expert ids or route weights into the stream's rows (sealed scheduling),
// in 2-byte units, so that the slot can be released before the stream ends.
__global__ __launch_bounds__(256) void slot_copy_kernel(uint16_t* __restrict__ dst,
                                                        const uint16_t* __restrict__ src,
                                                        int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    dst[i] = src[i];
}

// Copy of a slot's expert ids into the consumer's own buffer -- or, when the ring's status
// word records a failure (an expired wait: the slot may hold stale or half-written data),
// -1 for every id, so that the layer drops the chunk's rows and its output rows are zero.
__global__ __launch_bounds__(256) void slot_ids_kernel(int32_t* __restrict__ dst,
                                                       const int32_t* __restrict__ src,
                                                       int64_t n, const uint32_t* status) {
  const bool failed = load_acquire(status) != 0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    dst[i] = failed ? -1 : src[i];
}

hipError_t launch_slot_ids(int32_t* dst, const int32_t* src, int64_t n, const uint32_t* status,
                           hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((n + 255) / 256, 1024);
  slot_ids_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream>>>(dst, src, n,
                                                                               status);
  return hipGetLastError();
}

hipError_t launch_slot_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 2;
  if (n <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((n + 255) / 256, 1024);
  slot_copy_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream>>>(
      static_cast<uint16_t*>(dst), static_cast<const uint16_t*>(src), n);
  return hipGetLastError();
}

hipError_t launch_ring_init(uint32_t* words, int n, hipStream_t stream) {
  const int blocks = (n + 63) / 64 < 64 ? (n + 63) / 64 : 64;
  ring_init_kernel<<<dim3(blocks > 0 ? blocks : 1), dim3(64), 0, stream>>>(words, n);
  return hipGetLastError();
}

hipError_t launch_ring_wait(const uint32_t* a, const uint32_t* b, const uint32_t* seq,
                            uint32_t add, int64_t ticks, uint32_t* status, uint32_t code,
                            hipStream_t stream) {
  ring_wait_kernel<<<dim3(1), dim3(64), 0, stream>>>(a, b, seq, add, ticks, status, code);
  return hipGetLastError();
}

hipError_t launch_ring_publish(uint32_t* gen, uint32_t* seq, hipStream_t stream) {
  ring_publish_kernel<<<dim3(1), dim3(64), 0, stream>>>(gen, seq);
  return hipGetLastError();
}

}  // namespace rmoe
