// gdn_commit.hip -- rollback to the accepted draft length.
//
// After verification, row r's committed state becomes its checkpoint slot a_r
// (the state after the previous bonus token and a_r accepted drafts); rejected
// drafts leave no trace (onnxruntime-genai pull request "Run chained MTP drafting
// in the batch Engine", sections "Correctness fix" and "Rollback fix and
// corrected quality disposition").  a_r is read on the device, never on the
// host.  The copy is a plain bit copy with 16-byte coalesced accesses; an a_r
// outside [0, T_r) leaves the row untouched and raises the row's status bit.  The
// fold kernel below commits delta checkpoints the same way by re-applying the
// accepted steps' rank-1 factors.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Copy blocks move THREADS * F4 float4, every load of a thread issued before its
// first store.  Large commits take 64 KiB blocks (with 16 KiB blocks the 32 MiB
// commit of 16 rows took 10 % longer); small ones take 8 KiB blocks, so that one
// row's 2 MiB spreads over 256 compute units (against 16 KiB blocks, a batch-1
// verify + commit step replayed from a graph took 8.37 instead of 7.97 us per layer;
// 4 and 16 KiB blocks, and 64-thread blocks, were slower).
constexpr int kCopyBigThreads = 512, kCopyBigF4 = 8;
constexpr int kCopySmallThreads = 128, kCopySmallF4 = 4;
constexpr int64_t kCopyBigMinBlocks = 512;  // big blocks once a launch has at least this many
// fold blocks: 16 KiB of state each
constexpr int kFoldThreads = 256;
constexpr int kFoldF4 = 4;
constexpr int kFoldF4PerBlock = kFoldThreads * kFoldF4;

template <int THREADS, int F4>
__global__ __launch_bounds__(THREADS) void commit_kernel(CommitArgs args, int blocks_per_row) {
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
  const int64_t base = int64_t(part) * (THREADS * F4) + threadIdx.x;
  float4 x[F4];
#pragma unroll
  for (int m = 0; m < F4; ++m) {
    const int64_t idx = base + int64_t(m) * THREADS;
    if (idx < n4) {  // each checkpoint is read once: keep it out of the caches
      const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + idx));
      x[m] = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
#pragma unroll
  for (int m = 0; m < F4; ++m) {
    const int64_t idx = base + int64_t(m) * THREADS;
    // the committed state is read again only by the row's next call, a whole model
    // step later: write it through, leaving no dirty lines to be evicted later
    if (idx < n4)
      __builtin_nontemporal_store(f32x4{x[m].x, x[m].y, x[m].z, x[m].w},
                                  reinterpret_cast<f32x4 *>(dst + idx));
  }
}

// Fold commit of delta checkpoints: the committed state becomes the accepted prefix
// of the window applied to the source state, S <- fmaf(c_i, k_t[d] ks_t, alpha_t S) per
// element and token -- the verify kernel's own update, operation for operation, so the
// result is bit-identical to the state the window reached after that prefix.  A block
// streams 16 KiB of one (row, head) state: four float4 per thread, each inside one
// state row i.
template <int D>
__global__ __launch_bounds__(kFoldThreads) void fold_kernel(FoldArgs args, int blocks_per_unit) {
  constexpr int N4 = D * D / 4;  // float4 per (row, head) state
  const int part = blockIdx.x % blocks_per_unit;
  const int unit = blockIdx.x / blocks_per_unit;
  const int h = unit % args.n_v, r = unit / args.n_v;
  const int row = args.row_base + r;
  // a_r is read first, as a vector load (a scalar load would share one out-of-order
  // counter with the arguments the addresses below need), and checked once every
  // load is in flight
  int acc_idx = row;
  asm volatile("" : "+v"(acc_idx));
  const int acc_raw = args.accepted[acc_idx];
  const int hq = h / args.group, src = args.src[r], ntok = args.ntok[r];
  // every token's factors and keys are loaded before the first update (tokens past the
  // window are clamped to its last one and never applied): one memory round trip
  float cf[kMaxWindow][kFoldF4], al[kMaxWindow], ks[kMaxWindow];
  uint2 kw[kMaxWindow][kFoldF4];
#pragma unroll
  for (int t = 0; t < kMaxWindow; ++t) {
    const int tt = min(t, ntok - 1);
    const float *dl = args.delta + ((size_t(row) * args.ck_slots + tt) * args.n_v + h) * (D + 4);
    const uint16_t *kr = args.k + ((size_t(args.tok0[r]) + tt) * args.n_qk + hq) * D;
    al[t] = dl[D];
    ks[t] = dl[D + 1];  // the key's scale factor (1 unless normalised in the kernel)
#pragma unroll
    for (int m = 0; m < kFoldF4; ++m) {
      const int idx = min(part * kFoldF4PerBlock + m * kFoldThreads + int(threadIdx.x), N4 - 1);
      cf[t][m] = dl[(4 * idx) / D];
      kw[t][m] = *reinterpret_cast<const uint2 *>(kr + (4 * idx) % D);
    }
  }
  float4 x[kFoldF4];
#pragma unroll
  for (int m = 0; m < kFoldF4; ++m) {
    const int idx = part * kFoldF4PerBlock + m * kFoldThreads + int(threadIdx.x);
    x[m] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (idx < N4 && src >= 0) {
      const f32x4 y = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4 *>(args.pool_in + (size_t(src) * args.n_v + h) * D * D) + idx);
      x[m] = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
  asm volatile("" ::: "memory");  // keeps the loads above from sinking below the exit
  const int acc = __builtin_amdgcn_readfirstlane(acc_raw);
  if (acc < 0 || acc >= ntok) {
    if (part == 0 && h == 0 && threadIdx.x == 0) atomicOr(args.status + (row >> 5), 1u << (row & 31));
    return;
  }
#pragma unroll
  for (int t = 0; t < kMaxWindow; ++t) {
    if (t > acc) break;
#pragma unroll
    for (int m = 0; m < kFoldF4; ++m) {
      const float c = cf[t][m], alpha = al[t], f = ks[t];
      x[m].x = fmaf(c, __uint_as_float(kw[t][m].x << 16) * f, alpha * x[m].x);
      x[m].y = fmaf(c, __uint_as_float(kw[t][m].x & 0xFFFF0000u) * f, alpha * x[m].y);
      x[m].z = fmaf(c, __uint_as_float(kw[t][m].y << 16) * f, alpha * x[m].z);
      x[m].w = fmaf(c, __uint_as_float(kw[t][m].y & 0xFFFF0000u) * f, alpha * x[m].w);
    }
  }
#pragma unroll
  for (int m = 0; m < kFoldF4; ++m) {
    const int idx = part * kFoldF4PerBlock + m * kFoldThreads + int(threadIdx.x);
    if (idx < N4)
      __builtin_nontemporal_store(f32x4{x[m].x, x[m].y, x[m].z, x[m].w},
                                  reinterpret_cast<f32x4 *>(args.pool_out + (size_t(args.dst[r]) * args.n_v + h) * D * D) + idx);
  }
}

// Checkpoint select: the accepted checkpoint becomes the committed state where it is.
// One thread per row; the table entry is written with an ordinary vector store.
__global__ __launch_bounds__(kRowsPerLaunch) void select_kernel(SelectArgs args) {
  const int r = threadIdx.x;
  if (r >= args.n_rows) return;
  const int acc = args.accepted[r];
  if (acc < 0 || acc >= args.ntok[r]) {
    atomicOr(args.status + (r >> 5), 1u << (r & 31));
    return;
  }
  args.slot_table[r] = args.bank[r] * args.ck_slots + acc;
}

}  // namespace

hipError_t launch_select(const SelectArgs &args, hipStream_t stream) {
  if (args.n_rows <= 0) return hipSuccess;
  if (args.n_rows > kRowsPerLaunch) return hipErrorInvalidValue;
  hipLaunchKernelGGL(select_kernel, dim3(1), dim3(kRowsPerLaunch), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_fold(const FoldArgs &args, int d, hipStream_t stream) {
  if (args.n_rows <= 0) return hipSuccess;
  if (args.n_rows > kRowsPerLaunch) return hipErrorInvalidValue;
  for (int r = 0; r < args.n_rows; ++r)  // the kernel holds a whole window's factors in registers
    if (args.ntok[r] < 1 || args.ntok[r] > kMaxWindow) return hipErrorInvalidValue;
  const int n4 = d * d / 4;
  const int bpu = (n4 + kFoldF4PerBlock - 1) / kFoldF4PerBlock;
  const dim3 grid(unsigned(args.n_rows) * unsigned(args.n_v) * unsigned(bpu));
  if (d == 128)
    hipLaunchKernelGGL(fold_kernel<128>, grid, dim3(kFoldThreads), 0, stream, args, bpu);
  else if (d == 16)
    hipLaunchKernelGGL(fold_kernel<16>, grid, dim3(kFoldThreads), 0, stream, args, bpu);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs &args, hipStream_t stream) {
  if (args.n_rows <= 0) return hipSuccess;
  const int64_t n4 = args.row_floats / 4;
  constexpr int64_t big = kCopyBigThreads * kCopyBigF4, small = kCopySmallThreads * kCopySmallF4;
  const int64_t big_blocks = (n4 + big - 1) / big;
  if (big_blocks * args.n_rows >= kCopyBigMinBlocks) {
    hipLaunchKernelGGL((commit_kernel<kCopyBigThreads, kCopyBigF4>), dim3(unsigned(args.n_rows * big_blocks)),
                       dim3(kCopyBigThreads), 0, stream, args, int(big_blocks));
  } else {
    const int64_t blocks = (n4 + small - 1) / small;
    hipLaunchKernelGGL((commit_kernel<kCopySmallThreads, kCopySmallF4>), dim3(unsigned(args.n_rows * blocks)),
                       dim3(kCopySmallThreads), 0, stream, args, int(blocks));
  }
  return hipGetLastError();
}

}  // namespace gdn
