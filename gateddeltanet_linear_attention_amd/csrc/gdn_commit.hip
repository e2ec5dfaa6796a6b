// gdn_commit.hip -- rollback to the accepted draft length.
//
// After verification, row r's committed state becomes its checkpoint slot a_r
// (the state after the previous bonus token and a_r accepted drafts); rejected
// drafts leave no trace (onnxruntime-genai pull request "Run chained MTP drafting
// in the batch Engine", sections "Correctness fix" and "Rollback fix and
// corrected quality disposition").  a_r is read on the device, never on the
// host.  The copy is a plain bit copy with 16-byte coalesced accesses; an a_r
// outside [0, T_r) leaves the row untouched and raises the row's status bit.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kF4PerThread = 4;
constexpr int kF4PerBlock = kThreads * kF4PerThread;  // 16 KiB per block

__global__ __launch_bounds__(kThreads) void commit_kernel(CommitArgs args, int blocks_per_row) {
  const int r = blockIdx.x / blocks_per_row;
  const int part = blockIdx.x % blocks_per_row;
  const int acc = args.accepted[r];
  if (acc < 0 || acc >= args.ntok[r]) {
    if (part == 0 && threadIdx.x == 0) {
      const int row = args.row_base + r;
      atomicOr(args.status + (row >> 5), 1u << (row & 31));
    }
    return;
  }
  const int64_t n4 = args.row_floats / 4;
  const float4 *src = reinterpret_cast<const float4 *>(
      args.ckpt + (int64_t(r) * args.ck_slots + acc) * args.row_floats);
  float4 *dst = reinterpret_cast<float4 *>(args.pool + int64_t(args.dst[r]) * args.row_floats);
  const int64_t base = int64_t(part) * kF4PerBlock + threadIdx.x;
  float4 x[kF4PerThread];
#pragma unroll
  for (int m = 0; m < kF4PerThread; ++m) {
    const int64_t idx = base + int64_t(m) * kThreads;
    if (idx < n4) {  // each checkpoint is read once: keep it out of the caches
      const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + idx));
      x[m] = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
#pragma unroll
  for (int m = 0; m < kF4PerThread; ++m) {
    const int64_t idx = base + int64_t(m) * kThreads;
    // the committed state is read again only by the row's next call, a whole model
    // step later: write it through, leaving no dirty lines to be evicted later
    if (idx < n4)
      __builtin_nontemporal_store(f32x4{x[m].x, x[m].y, x[m].z, x[m].w},
                                  reinterpret_cast<f32x4 *>(dst + idx));
  }
}

}  // namespace

hipError_t launch_commit(const CommitArgs &args, hipStream_t stream) {
  if (args.n_rows <= 0) return hipSuccess;
  const int64_t n4 = args.row_floats / 4;
  const int blocks_per_row = int((n4 + kF4PerBlock - 1) / kF4PerBlock);
  dim3 grid(unsigned(args.n_rows) * unsigned(blocks_per_row));
  hipLaunchKernelGGL(commit_kernel, grid, dim3(kThreads), 0, stream, args, blocks_per_row);
  return hipGetLastError();
}

}  // namespace gdn
