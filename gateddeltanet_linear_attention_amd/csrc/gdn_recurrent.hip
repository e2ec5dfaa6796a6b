// gdn_recurrent.hip -- token-by-token gated delta rule on gfx950: decode, draft
// verification with per-token state checkpoints, and short transaction rows.
//
// Per (row, value head) the state S is d_v x d_k fp32 (64 KiB at d = 128).  The
// rows of S (value channels) evolve independently:
//     u_i   = S[i,:] . k_t
//     S[i,:] <- alpha_t S[i,:] + beta_t (v_t[i] - alpha_t u_i) k_t
//     o_t[i] = S[i,:] . q_t
// which is S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t
// (the gated delta rule, Yang, Kautz & Hatamizadeh, ICLR 2025).
//
// Mapping.  LPR lanes own one state row; lane `sub` of the group holds the
// float4 columns {sub + LPR*j}, so one wave-wide float4 access covers 64/LPR
// rows in LPR*16-byte contiguous runs (128 B runs at d = 128): coalesced HBM
// reads of the state and writes of every checkpoint.  The two dot products per
// token are a fixed-order in-lane FMA chain followed by an xor butterfly over the
// LPR lanes, which leaves every lane of the group with bit-identical sums.
//
// Bit-exactness.  Decode, verify and transaction rows all run this one kernel
// instantiation per d; the per-row arithmetic (element ownership, FMA order,
// butterfly, gate code) does not depend on the row's token count, the launch's
// row count or the grid.  So the checkpoint after j+1 verify tokens is
// bit-identical to j+1 decode launches: both compute the same sequence of fp32
// operations on the same values, and fp32 state round-trips through memory
// exactly ("Native three-step MTP", section "What changed": state-update
// rounding consistent between decode and verification).  Built with
// -ffp-contract=off; every fused multiply-add is an explicit fmaf.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// fp32 gates: alpha = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b),
// softplus(x) = max(x, 0) + log1p(exp(-|x|)) (no overflow for any x).
__device__ __forceinline__ void eval_gates(float a, float b, float A_log, float dt_bias,
                                           float &alpha, float &beta) {
  const float x = a + dt_bias;
  const float sp = fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
  alpha = expf(-(expf(A_log) * sp));
  beta = 1.0f / (1.0f + expf(-b));
}

template <int LPR>
__device__ __forceinline__ float group_sum(float p) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) p += __shfl_xor(p, m, 64);
  return p;
}

template <int D, int LPR, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void recurrent_kernel(RecurrentArgs args) {
  constexpr int NV = D / LPR / 4;                  // float4 per lane per state row
  constexpr int ROWS = WAVES * 64 / LPR;           // state rows per block
  constexpr int TILES = D / ROWS;                  // blocks per (row, head)
  static_assert(NV >= 1 && D % (LPR * 4) == 0 && D % ROWS == 0, "bad tiling");
  constexpr size_t UNIT = size_t(D) * D;

  const int sub = threadIdx.x % LPR;
  int bid = blockIdx.x;
  const int tile = bid % TILES;
  bid /= TILES;
  const int h = bid % args.n_v;
  const int r = bid / args.n_v;
  const int hq = h / args.group;
  const int i = tile * ROWS + int(threadIdx.x) / LPR;  // state row (value channel)

  const int ntok = args.ntok[r], tok0 = args.tok0[r];
  const int src = args.src[r], dst = args.dst[r], ck_first = args.ck_first[r];
  const int ck_row = args.ck_row[r];
  const int n_v = args.n_v, n_qk = args.n_qk;

  float s[NV][4];
  if (src >= 0) {
    const float4 *p = reinterpret_cast<const float4 *>(
        args.state_in + (size_t(src) * n_v + h) * UNIT + size_t(i) * D);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const float4 x = p[sub + LPR * j];
      s[j][0] = x.x; s[j][1] = x.y; s[j][2] = x.z; s[j][3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) s[j][0] = s[j][1] = s[j][2] = s[j][3] = 0.0f;
  }
  const float A_log = args.A_log[h], dt_bias = args.dt_bias[h];

  for (int t = 0; t < ntok; ++t) {
    const size_t tok = size_t(tok0) + t;
    float alpha, beta;
    eval_gates(args.a[tok * n_v + h], args.b[tok * n_v + h], A_log, dt_bias, alpha, beta);
    const uint2 *kp = reinterpret_cast<const uint2 *>(args.k + (tok * n_qk + hq) * D);
    const uint2 *qp = reinterpret_cast<const uint2 *>(args.q + (tok * n_qk + hq) * D);
    float kk[NV][4], qq[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint2 kw = kp[sub + LPR * j], qw = qp[sub + LPR * j];
      kk[j][0] = bf16_lo(kw.x); kk[j][1] = bf16_hi(kw.x);
      kk[j][2] = bf16_lo(kw.y); kk[j][3] = bf16_hi(kw.y);
      qq[j][0] = bf16_lo(qw.x); qq[j][1] = bf16_hi(qw.x);
      qq[j][2] = bf16_lo(qw.y); qq[j][3] = bf16_hi(qw.y);
    }
    const float vi = __uint_as_float(uint32_t(args.v[(tok * n_v + h) * D + i]) << 16);

    // u = S[i,:] . k
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) p = fmaf(s[j][e], kk[j][e], p);
    const float u = group_sum<LPR>(p);
    // S[i,:] <- alpha S[i,:] + beta (v_i - alpha u) k
    const float c = beta * (vi - alpha * u);
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[j][e] = fmaf(c, kk[j][e], alpha * s[j][e]);
    // o_i = S[i,:] . q
    float po = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) po = fmaf(s[j][e], qq[j][e], po);
    const float oi = group_sum<LPR>(po);
    if (sub == 0) args.o[(tok * n_v + h) * D + i] = to_bf16(oi);

    if (t >= ck_first) {
      float4 *cp = reinterpret_cast<float4 *>(
          args.ckpt + ((size_t(ck_row) * args.ck_slots + (t - ck_first)) * n_v + h) * UNIT +
          size_t(i) * D);
#pragma unroll
      for (int j = 0; j < NV; ++j)
        cp[sub + LPR * j] = make_float4(s[j][0], s[j][1], s[j][2], s[j][3]);
    }
  }

  if (dst >= 0) {
    float4 *p = reinterpret_cast<float4 *>(args.state_out + (size_t(dst) * n_v + h) * UNIT +
                                           size_t(i) * D);
#pragma unroll
    for (int j = 0; j < NV; ++j) p[sub + LPR * j] = make_float4(s[j][0], s[j][1], s[j][2], s[j][3]);
  }
}

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs &args, int d, hipStream_t stream) {
  if (args.n_rows <= 0) return hipSuccess;
  if (d == 128) {
    constexpr int D = 128, LPR = 8, WAVES = 4;
    constexpr int TILES = D / (WAVES * 64 / LPR);
    dim3 grid(unsigned(args.n_rows) * unsigned(args.n_v) * TILES);
    hipLaunchKernelGGL((recurrent_kernel<D, LPR, WAVES>), grid, dim3(64 * WAVES), 0, stream, args);
  } else if (d == 16) {
    constexpr int D = 16, LPR = 4, WAVES = 1;
    constexpr int TILES = D / (WAVES * 64 / LPR);
    dim3 grid(unsigned(args.n_rows) * unsigned(args.n_v) * TILES);
    hipLaunchKernelGGL((recurrent_kernel<D, LPR, WAVES>), grid, dim3(64 * WAVES), 0, stream, args);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
