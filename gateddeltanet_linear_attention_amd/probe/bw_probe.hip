// bw_probe.hip -- streaming-bandwidth ceilings for the benchmark's context lines.
//
// Not part of the gated-delta-rule path: a plain kernel with the verify launch's memory
// traffic and none of its work.  Each block reads one tile of src once (F4 float4 per
// thread, 256-byte runs per 16 lanes) and writes it to n_out destination copies with
// non-temporal 16-byte stores, so n_out = 4 is the verify's 1 read : 4 writes of state
// and n_out = 1 a plain copy.  Three schedules: 512 threads x 2 float4 (16 KiB tiles),
// and 256 threads x 2 or x 4 float4 (8 or 16 KiB tiles) issuing their loads at raised
// wave priority, which is what the verify kernel does; the benchmark reports the best
// as the ceiling.  Built as its own library (libgdn_probe.so); nothing in libgdn.so
// calls it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int THREADS, int F4, bool PRIO>
__global__ __launch_bounds__(THREADS) void stream_kernel(const f32x4 *src, f32x4 *dst, int64_t n4, int n_out) {
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(3);
  const int64_t base = int64_t(blockIdx.x) * (THREADS * F4) + threadIdx.x;
  f32x4 x[F4];
#pragma unroll
  for (int m = 0; m < F4; ++m) {
    const int64_t i = base + int64_t(m) * THREADS;
    x[m] = i < n4 ? src[i] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  for (int c = 0; c < n_out; ++c)
#pragma unroll
    for (int m = 0; m < F4; ++m) {
      const int64_t i = base + int64_t(m) * THREADS;
      if (i < n4) __builtin_nontemporal_store(x[m], dst + int64_t(c) * n4 + i);
    }
}

template <int THREADS, int F4, bool PRIO>
int launch(const void *src, void *dst, int64_t n4, int n_out, hipStream_t stream) {
  constexpr int64_t tile = THREADS * F4;
  const int64_t blocks = (n4 + tile - 1) / tile;
  if (blocks > INT32_MAX) return -1;
  hipLaunchKernelGGL((stream_kernel<THREADS, F4, PRIO>), dim3(unsigned(blocks)), dim3(THREADS), 0, stream,
                     static_cast<const f32x4 *>(src), static_cast<f32x4 *>(dst), n4, n_out);
  return int(hipGetLastError());
}

}  // namespace

extern "C" {

// Reads n_bytes of src once and writes them to n_out consecutive copies at dst
// (dst holds n_out * n_bytes), with schedule `shape`: 0 = 512 x 2 float4, 1 = 256 x 2
// with the priority prologue, 2 = 256 x 4 with it.  n_bytes a positive multiple of 16,
// 1 <= n_out <= 8, both pointers 16-byte aligned device memory.  Returns 0, -1 for bad
// arguments (nothing launched), or the HIP error of the launch.  Asynchronous on
// `stream` (a hipStream_t).
int gdn_probe_stream(const void *src, void *dst, int64_t n_bytes, int32_t n_out, int32_t shape, void *stream) {
  if (!src || !dst || n_bytes <= 0 || n_bytes % 16 != 0 || n_out < 1 || n_out > 8) return -1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return -1;
  const int64_t n4 = n_bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (shape) {
    case 0: return launch<512, 2, false>(src, dst, n4, n_out, s);
    case 1: return launch<256, 2, true>(src, dst, n4, n_out, s);
    case 2: return launch<256, 4, true>(src, dst, n4, n_out, s);
    default: return -1;
  }
}

}  // extern "C"
