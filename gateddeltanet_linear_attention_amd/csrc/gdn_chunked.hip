// gdn_chunked.hip -- chunkwise (UT / WY) gated delta rule for long prefill rows,
// publishing the state checkpoints a row asks for at its last positions.
//
// Within a chunk of C = 64 tokens starting from state S_c, with the log-space
// cumulative decay G_t = g_1 + ... + g_t (g = log alpha) and the value each token
// writes, u_t = beta_t (v_t - alpha_t S_{t-1} k_t):
//     S_t = e^{G_t} S_c + sum_{s<=t} e^{G_t - G_s} u_s k_s^T                    (1)
// Stacking the u_t as rows of U gives (I + A) U = diag(beta) V - diag(beta e^G) K S_c^T,
// A_ts = beta_t e^{G_t - G_s} k_t.k_s (s < t).  With T = (I + A)^{-1}:
//     W = T diag(beta e^G) K,   U' = T diag(beta) V,   U = U' - W S_c^T
//     O = diag(e^G) Q S_c^T + (Gamma o Q K^T) U,  Gamma_ts = e^{G_t - G_s} (s <= t)
//     S_{c+1} = e^{G_n} S_c + U^T diag(e^{G_n - G}) K
// (Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
// Sequence Length", NeurIPS 2024, sec. 3, with the decay of the gated delta rule of
// Yang, Kautz & Hatamizadeh, ICLR 2025).  When q and k arrive unnormalised, K and Q
// stand for diag(rk) K and diag(rq) Q (rk_t = 1/|k_t|, rq_t = 1/(|q_t| sqrt(d_k))):
// the factors are applied to the exact bf16 products and folded into the diagonal
// scalings above, so the matrix cores still see the bf16 inputs.  A checkpoint at in-chunk position j is
// (1) truncated at s <= j: one more rank-64 product per requested position, so a
// long prefill in a ragged batch still publishes the intermediate states a draft
// rollback needs (the gap named in the onnxruntime-genai pull request "Run chained
// MTP drafting in the batch Engine", section "Correctness fix").
//
// Four kernels, same stream:
//   chunk_prep_kernel  one block per (chunk, value head), all chunks in parallel:
//       gates, fp64 prefix sum of g, K K^T and Q K^T, forward substitution for T,
//       W, U', K^T and the decay factors -> workspace.
//   chunk_scan_kernel  one block per (row, value head, 16 state rows), chunks in
//       order, only the sequential part: U = U' - W S_c^T and the state carry (the
//       state tile stays in LDS; the next chunk's operands are fetched during the
//       current one); each chunk's start state and U^T -> workspace.
//   chunk_out_kernel   one block per (chunk, value head, half of the value
//       channels), all in parallel: the outputs O.
//   chunk_ckpt_kernel  one block per (row, tail checkpoint, value head, 16 value
//       rows): the requested checkpoints, from the recorded chunk state.
// The contractions run on the fp32 matrix cores (v_mfma_f32_16x16x4_f32, 157 TF dense
// on MI355X): the state tolerance (relative 1e-4) rules out rounding the fp32 operands
// T, W, U, S to bf16.  Two products run on the bf16 cores at fp32 accuracy: K K^T and
// Q K^T (bf16 inputs, exact products), and the carry's U^T diag(.) K, whose K is bf16
// and whose fp32 factor is split into three bf16 parts that sum to it to within a unit
// in its last place.  A wave loads all operand fragments of a product
// before its first matrix instruction and interleaves independent accumulation
// chains, so global-memory latency is paid once per phase, not once per k step.
// Decays are formed only as differences G_t - G_s with s <= t, from an fp64 prefix
// sum (|G| reaches hundreds within a chunk under strong decay, where differences of
// fp32 sums would lose ~1e-5 relative).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = 64;       // chunk length
constexpr int VT = 16;      // state rows per scan block
constexpr int LDC = C + 4;  // padded LDS row length (floats) for C-wide rows
constexpr int LDB = C + 4;  // padded LDS row length (bf16) for C-wide rows

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ float4 zf4() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }
__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

// One 16-wide k block of acc(16x16) += A(16 x K) * B(K x 16) on the matrix cores.
// Lane l (r = l % 16, g = l / 16) holds a = A[r][kb+4g .. kb+4g+3] and
// b = B[kb+4g .. kb+4g+3][r]: a permutation of k inside the block, the same on
// both sides.  After all k blocks, lane l holds C[4g + v][r] in acc[v].
__device__ __forceinline__ floatx4 mma4(floatx4 acc, float4 a, float4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
  return acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// x = hi + mid + lo to fp32 precision in three bf16 parts, each the round to nearest of
// what the parts before it leave (every subtraction is exact), written as the bits of
// the lane's four values per part.  A bf16 matrix product of these parts against an
// exactly-bf16 operand then reproduces the fp32 product to fp32 accuracy (the bf16x3
// split: Henry, Tang & Heinecke, "Leveraging the bfloat16 Artificial Intelligence
// Datatype for Higher-Precision Computations", ARITH 2019).
struct Parts4 {  // one 4-token piece in three parts, bf16 bits
  uint2 h, m, l;
};
// the three parts of one value, packed at bit 16 * `hi` of the three words
__device__ __forceinline__ void split3_into(float v, int hi, uint32_t &h, uint32_t &m, uint32_t &l) {
  const uint32_t bh = to_bf16(v);
  const float r1 = v - __uint_as_float(bh << 16);
  const uint32_t bm = to_bf16(r1);
  const uint32_t bl = to_bf16(r1 - __uint_as_float(bm << 16));
  h |= bh << (16 * hi);
  m |= bm << (16 * hi);
  l |= bl << (16 * hi);
}
__device__ __forceinline__ Parts4 split3x4(float4 x) {
  uint32_t h0 = 0, m0 = 0, l0 = 0, h1 = 0, m1 = 0, l1 = 0;
  split3_into(x.x, 0, h0, m0, l0);
  split3_into(x.y, 1, h0, m0, l0);
  split3_into(x.z, 0, h1, m1, l1);
  split3_into(x.w, 1, h1, m1, l1);
  return Parts4{make_uint2(h0, h1), make_uint2(m0, m1), make_uint2(l0, l1)};
}

// Two 4-token pieces (bf16 bits) as one 8-wide operand of v_mfma_f32_16x16x32_bf16.
__device__ __forceinline__ bf16x8 pieces8(uint2 a, uint2 b) {
  return __builtin_bit_cast(bf16x8, u32x4v{a.x, a.y, b.x, b.y});
}

// acc(16x16) += A(16 x 64 tokens) * B(64 tokens x 16) with A given as the bf16x3 parts of
// its four 4-token pieces (lane (r, g): A[r][16 kb + 4 g + e]) and B exactly bf16 in
// the same pieces (B[16 kb + 4 g + e][r]): each 32-wide matrix instruction takes pieces
// kb = 2 m, 2 m + 1 (a permutation of the token index, the same on both sides), parts
// hi, mid, lo in that order.  Output layout as mma4's.
__device__ __forceinline__ floatx4 mma_bf16x3_32(floatx4 acc, Parts4 a0, Parts4 a1, uint2 b0, uint2 b1) {
  const bf16x8 b = pieces8(b0, b1);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pieces8(a0.h, a1.h), b, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pieces8(a0.m, a1.m), b, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(pieces8(a0.l, a1.l), b, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma_bf16x3_64(floatx4 acc, Parts4 a0, Parts4 a1, Parts4 a2, Parts4 a3,
                                                 uint2 b0, uint2 b1, uint2 b2, uint2 b3) {
  return mma_bf16x3_32(mma_bf16x3_32(acc, a0, a1, b0, b1), a2, a3, b2, b3);
}

// bf16 operand of v_mfma_f32_16x16x32_bf16 for 32-wide k block kb of row t of a
// row-major bf16 matrix (row pitch ld elements, rows t >= n read as zero): lane
// (r, g) feeds row element 32 kb + 8 g + e, e = 0..7, one 16-byte load.  Blocks
// past the row width d (d = 16) are zero.
template <int D>
__device__ __forceinline__ bf16x8 frag32_row(const uint16_t *base, int64_t ld, int t, int kb, int n, int g4) {
  const int c = 32 * kb + 8 * g4;
  u32x4v w = {0u, 0u, 0u, 0u};
  if (t < n && c < D) w = *reinterpret_cast<const u32x4v *>(base + int64_t(t) * ld + c);
  return __builtin_bit_cast(bf16x8, w);
}

// Which row of the launch owns launch-local chunk `c` (rows are few: scalar scan).
__device__ __forceinline__ int row_of_chunk(const ChunkArgs &args, int c) {
  int row = 0;
  for (int i = 1; i < args.n_rows; ++i)
    if (args.chunk_start[i] <= c) row = i;
  return row;
}

// Workspace of one (chunk, value head): W [C][D], U'^T [D][C], P [C][C], G [C] fp64,
// eG[t] = e^{G_t}, eL[s] = e^{G_{n-1} - G_s} rk_s (s < n, else 0), K^T [D][C] bf16 with
// each row's tokens in kt_pos order (below), the chunk's start state Sc [D][D], U^T
// [D][C], and the factors rk, rq [C] that scale each token's k and q (1 unless q/k
// are normalised in the kernels).
// Token m = 16 kb + 4 g + e of a chunk sits at 16 g + 4 kb + e of a stored K^T row, so
// the MFMA lane group g finds its four 4-token pieces (kb = 0..3) in 32 contiguous bytes.
__device__ __forceinline__ int kt_pos(int m) { return 16 * ((m >> 2) & 3) + 4 * (m >> 4) + (m & 3); }

template <int D>
struct Ws {
  float *W, *U, *P, *eG, *eL, *Sc, *Ut, *rk, *rq;
  double *G;
  uint16_t *Kt;
  __device__ Ws(float *base) {
    W = base;
    U = base + C * D;
    P = base + 2 * C * D;
    G = reinterpret_cast<double *>(base + 2 * C * D + C * C);
    eG = base + 2 * C * D + C * C + 2 * C;
    eL = eG + C;
    Kt = reinterpret_cast<uint16_t *>(eL + C);
    Sc = eL + C + D * C / 2;
    Ut = Sc + D * D;
    rk = Ut + D * C;
    rq = rk + C;
  }
};

// q/k normalisation of the fused input mode: x / sqrt(sum x^2 + eps), q also by
// 1/sqrt(d_k).
constexpr float kNormEps = 1e-6f;
template <int D>
constexpr float inv_sqrt_d() {
  static_assert(D == 16 || D == 128, "head width");
  return D == 16 ? 0.25f : 0.0883883476483184405501f;
}

template <int D>
__global__ __launch_bounds__(256) void chunk_prep_kernel(ChunkArgs args) {
  __shared__ double sG[C];
  __shared__ __attribute__((aligned(16))) float sBeta[C];  // beta_m
  __shared__ __attribute__((aligned(16))) float sSK[C];    // beta_m e^{G_m}
  __shared__ __attribute__((aligned(16))) float sA[C * LDC];  // strictly lower A, then T = (I + A)^{-1}
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * LDB];  // K^T (bf16): row d, column token m
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * LDB];  // V^T (bf16)
  __shared__ float sRk[C], sRq[C];  // per-token k and q scale factors (1: inputs taken as given)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int cl = blockIdx.x, h = blockIdx.y;
  const int row = row_of_chunk(args, cl);
  const int cin = cl - args.chunk_start[row];
  const int c0 = cin * C;
  const int n = min(C, args.len[row] - c0);
  const int64_t tok_base = int64_t(args.tok0[row]) + c0;
  const int n_v = args.n_v, n_qk = args.n_qk, hq = h / args.group;
  const int64_t ldqk = int64_t(n_qk) * D, ldv = int64_t(n_v) * D;
  const uint16_t *Kc = args.k + tok_base * ldqk + int64_t(hq) * D;
  const uint16_t *Qc = args.q + tok_base * ldqk + int64_t(hq) * D;
  const uint16_t *Vc = args.v + tok_base * ldv + int64_t(h) * D;
  Ws<D> ws(args.ws + (int64_t(args.chunk0[row] + cin) * n_v + h) * ChunkArgs::ws_unit_floats(D));

  auto frag32 = [&](const uint16_t *base, int64_t ld, int t, int kb) {
    return frag32_row<D>(base, ld, t, kb, n, g4);
  };

  // 1. gates and the fp64 inclusive prefix sum of g (tokens t >= n: g = beta = 0);
  //    K^T and V^T staged in LDS, with the k and q norms when normalising.
  double G = 0.0, Gl = 0.0;  // wave 0: lane t's prefix sum G_t and the chunk's last one
  if (w == 0) {
    float gf = 0.0f, bt = 0.0f;
    if (lane < n) {
      const int64_t tk = tok_base + lane;
      const float x = args.a[tk * n_v + h] + args.dt_bias[h];
      const float sp = fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
      gf = -(expf(args.A_log[h]) * sp);
      bt = 1.0f / (1.0f + expf(-args.b[tk * n_v + h]));
    }
    G = gf;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(G, off, 64);
      if (lane >= off) G += y;
    }
    sG[lane] = G;
    sBeta[lane] = bt;
    sSK[lane] = bt * float(exp(G));
    Gl = __shfl(G, n - 1, 64);
    ws.G[lane] = G;
    ws.eG[lane] = float(exp(G));
  }
  // Transposing stage: lane (m_lo, dg) of wave mh loads 4 dims of token
  // m = 16 mh + m_lo, so the 16 lanes of a group write 16 consecutive columns of a
  // K^T row and the 4 groups land on disjoint banks (row pitch 136 B).
  {
    const int m = 16 * w + (lane & 15), dg = lane >> 4;
    const bool norm = args.qk_norm != 0;
    float ssk = 0.0f, ssq = 0.0f;  // this lane's D/4 dims of token m
    for (int it = 0; it < D / 16; ++it) {
      const int d4 = (4 * it + dg) * 4;
      uint2 kw = make_uint2(0u, 0u), vw = kw, qw = kw;
      if (m < n) {
        kw = *reinterpret_cast<const uint2 *>(Kc + int64_t(m) * ldqk + d4);
        vw = *reinterpret_cast<const uint2 *>(Vc + int64_t(m) * ldv + d4);
        if (norm) qw = *reinterpret_cast<const uint2 *>(Qc + int64_t(m) * ldqk + d4);
      }
      if (norm) {
        const float4 kf = unpack_bf16x4(kw), qf = unpack_bf16x4(qw);
        ssk = fmaf(kf.x, kf.x, ssk); ssk = fmaf(kf.y, kf.y, ssk);
        ssk = fmaf(kf.z, kf.z, ssk); ssk = fmaf(kf.w, kf.w, ssk);
        ssq = fmaf(qf.x, qf.x, ssq); ssq = fmaf(qf.y, qf.y, ssq);
        ssq = fmaf(qf.z, qf.z, ssq); ssq = fmaf(qf.w, qf.w, ssq);
      }
      sKt[(d4 + 0) * LDB + m] = uint16_t(kw.x);
      sKt[(d4 + 1) * LDB + m] = uint16_t(kw.x >> 16);
      sKt[(d4 + 2) * LDB + m] = uint16_t(kw.y);
      sKt[(d4 + 3) * LDB + m] = uint16_t(kw.y >> 16);
      sVt[(d4 + 0) * LDB + m] = uint16_t(vw.x);
      sVt[(d4 + 1) * LDB + m] = uint16_t(vw.x >> 16);
      sVt[(d4 + 2) * LDB + m] = uint16_t(vw.y);
      sVt[(d4 + 3) * LDB + m] = uint16_t(vw.y >> 16);
    }
    if (norm) {  // the 4 lanes of token m (lane bits 4 and 5) hold its partial sums
      ssk += __shfl_xor(ssk, 16, 64);
      ssk += __shfl_xor(ssk, 32, 64);
      ssq += __shfl_xor(ssq, 16, 64);
      ssq += __shfl_xor(ssq, 32, 64);
    }
    if (dg == 0) {
      sRk[m] = !norm ? 1.0f : m < n ? 1.0f / sqrtf(ssk + kNormEps) : 0.0f;
      sRq[m] = !norm ? 1.0f : m < n ? 1.0f / sqrtf(ssq + kNormEps) * inv_sqrt_d<D>() : 0.0f;
    }
  }
  lds_barrier();
  if (w == 0) {
    // with the k factors known: the carry's decays e^{G_n - G_s} rk_s and the
    // diagonal beta e^G rk of W (read in step 4, after further barriers)
    const float rk = sRk[lane];
    ws.eL[lane] = lane < n ? float(exp(Gl - G)) * rk : 0.0f;
    sSK[lane] *= rk;
    ws.rk[lane] = rk;
    ws.rq[lane] = sRq[lane];
  }
  // K^T to the workspace for the scan and checkpoint kernels: row d is 64 contiguous
  // bf16, 4-token pieces placed by kt_pos
  for (int idx = tid; idx < D * (C / 4); idx += 256) {
    const int d = idx / (C / 4), m4 = (idx % (C / 4)) * 4;
    *reinterpret_cast<uint2 *>(ws.Kt + d * C + kt_pos(m4)) = *reinterpret_cast<const uint2 *>(sKt + d * LDB + m4);
  }

  // 2. K K^T -> A (strictly lower, scaled) and Q K^T -> P (lower with diagonal) on
  //    the bf16 matrix cores: K and Q are bf16, so every product is exact in fp32 and
  //    only the fp32 accumulation rounds.  Wave w owns row block w: it loads the
  //    fragments once (its Q rows, the K rows of all four blocks), computes tiles
  //    (w, tj <= w) and writes zeros to the tiles right of the diagonal.
  {
    constexpr int NK32 = (D + 31) / 32;  // 32-wide k blocks over d (D = 16: half of one)
    bf16x8 fk[4][NK32], fa[NK32], fq[NK32];  // fa: this wave's K rows (register arrays
#pragma unroll                                 // are indexed by constants only)
    for (int kb = 0; kb < NK32; ++kb) {
      fq[kb] = frag32(Qc, ldqk, 16 * w + r16, kb);
      fa[kb] = frag32(Kc, ldqk, 16 * w + r16, kb);
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) fk[tj][kb] = frag32(Kc, ldqk, 16 * tj + r16, kb);
    }
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      floatx4 kk = zero4(), qk = zero4();
      if (tj <= w) {
#pragma unroll
        for (int kb = 0; kb < NK32; ++kb) {
          kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[kb], fk[tj][kb], kk, 0, 0, 0);
          qk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq[kb], fk[tj][kb], qk, 0, 0, 0);
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * w + 4 * g4 + v, s = 16 * tj + r16;
        float av = 0.0f, pv = 0.0f;
        if (s <= t) {
          const float dec = expf(float(sG[t] - sG[s]));
          pv = dec * (qk[v] * sRq[t] * sRk[s]);
          if (s < t) av = sBeta[t] * dec * (kk[v] * sRk[t] * sRk[s]);
        }
        if (tj <= w) sA[t * LDC + s] = av;  // the upper blocks of sA hold T below
        ws.P[t * C + s] = pv;
      }
    }
  }
  lds_barrier();

  // 3. T = (I + A)^{-1}, A strictly lower triangular, by 16x16 blocks:
  //    T_ii = (I + A_ii)^{-1}, then T_ij = -T_ii (sum_{j<=k<i} A_ik T_kj) for i > j,
  //    one sub-diagonal at a time.  T_ii overwrites A_ii (no longer needed); T_ij
  //    (i > j) is stored at block (j, i) of sA, right of the diagonal, so A's lower
  //    blocks stay intact until the last product.
  {
    // diagonal blocks, one per wave: lane j < 16 holds column j of T_ww and runs the
    // forward substitution T[t][j] = [t == j] - sum_{m<t} A[t][m] T[m][j]
    float* Aw = sA + (16 * w) * LDC + 16 * w;
    if (lane < 16) {
      float Tc[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) Tc[t] = (t == lane) ? 1.0f : 0.0f;
#pragma unroll
      for (int t = 1; t < 16; ++t) {
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int m = 0; m < t; m += 4) {
          const float4 ar = *reinterpret_cast<const float4 *>(Aw + t * LDC + m);
          p0 = fmaf(ar.x, Tc[m + 0], p0);
          p1 = fmaf(ar.y, Tc[m + 1], p1);
          p0 = fmaf(ar.z, Tc[m + 2], p0);
          p1 = fmaf(ar.w, Tc[m + 3], p1);
        }
        Tc[t] -= p0 + p1;  // A[t][m] = 0 for m >= t within the block
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) Aw[t * LDC + lane] = Tc[t];
    }
    lds_barrier();
    // T_ij block (i > j) lives at rows 16 j.., columns 16 i.. of sA
    auto tblk = [&](int i, int j) -> float * {
      return i == j ? sA + (16 * i) * LDC + 16 * i : sA + (16 * j) * LDC + 16 * i;
    };
    // B fragment of a 16x16 block X (lane (r, g) feeds X[4g + e][r], e = 0..3)
    auto bfrag = [&](const float *X) {
      return make_float4(X[(4 * g4 + 0) * LDC + r16], X[(4 * g4 + 1) * LDC + r16],
                         X[(4 * g4 + 2) * LDC + r16], X[(4 * g4 + 3) * LDC + r16]);
    };
    auto afrag = [&](const float *X) {  // A fragment: X[r][4g + e]
      return *reinterpret_cast<const float4 *>(X + r16 * LDC + 4 * g4);
    };
    for (int lvl = 1; lvl < 4; ++lvl) {
      const int i = w, j = w - lvl;
      if (j >= 0) {
        // X = sum_{k=j}^{i-1} A_ik T_kj, then T_ij = -T_ii X (X's result layout is the
        // B-operand layout of the second product)
        floatx4 x = zero4();
        for (int k = j; k < i; ++k)
          x = mma4(x, afrag(sA + (16 * i) * LDC + 16 * k), bfrag(tblk(k, j)));
        floatx4 y = mma4(zero4(), afrag(tblk(i, i)), make_float4(x[0], x[1], x[2], x[3]));
        float *dstb = tblk(i, j);
#pragma unroll
        for (int v = 0; v < 4; ++v) dstb[(4 * g4 + v) * LDC + r16] = -y[v];
      }
      lds_barrier();
    }
  }

  // 4. W = T diag(beta e^G) K and U' = T diag(beta) V.  Wave w owns column tiles
  //    {2w, 2w+1} of every row tile (T is lower triangular: k < 16(ti+1)).
  for (int nt = 2 * w; nt < 2 * w + 2 && nt < D / 16; ++nt) {
    for (int ti = 0; ti < 4; ++ti) {
      floatx4 wa = zero4(), ua = zero4();
      for (int kb = 0; kb <= ti; ++kb) {
        const int k0 = 16 * kb + 4 * g4;
        // block (ti, kb) of T: the diagonal block in place, the others right of it
        const float *tb = kb == ti ? sA + (16 * ti) * LDC + 16 * ti : sA + (16 * kb) * LDC + 16 * ti;
        const float4 tr = *reinterpret_cast<const float4 *>(tb + r16 * LDC + 4 * g4);
        const float4 sk = *reinterpret_cast<const float4 *>(sSK + k0);
        const float4 sb = *reinterpret_cast<const float4 *>(sBeta + k0);
        const int d = 16 * nt + r16;
        const float4 kt = unpack_bf16x4(*reinterpret_cast<const uint2 *>(sKt + d * LDB + k0));
        const float4 vt = unpack_bf16x4(*reinterpret_cast<const uint2 *>(sVt + d * LDB + k0));
        wa = mma4(wa, mul4(tr, sk), kt);
        ua = mma4(ua, mul4(tr, sb), vt);
      }
      const int d = 16 * nt + r16;
#pragma unroll
      for (int v = 0; v < 4; ++v) ws.W[(16 * ti + 4 * g4 + v) * D + d] = wa[v];
      // U'^T: the lane's 4 tokens are contiguous
      *reinterpret_cast<float4 *>(ws.U + d * C + 16 * ti + 4 * g4) = make_float4(ua[0], ua[1], ua[2], ua[3]);
    }
  }
}

// Operands of one chunk that a scan wave needs: its W rows, its U' values, the
// carry's decay factors and the K^T fragments of its state column tiles.
template <int D>
struct ScanFrag {
  static constexpr int NKB = D / 16;
  static constexpr int NT_W = (D / 16 + 3) / 4;
  float4 wf[NKB], el;
  uint2 kp[NT_W][4];  // K^T pieces kb = 0..3 of each column tile, bf16 bits
  float4 up;
  float e_last;
  __device__ void load(const Ws<D> &ws, int n, int w, int r16, int g4, int i0) {
    const int t_me = 16 * w + r16;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      wf[kb] = *reinterpret_cast<const float4 *>(ws.W + t_me * D + 16 * kb + 4 * g4);
    // the carry's decay factors of the 4 tokens whose U this lane writes
    el = *reinterpret_cast<const float4 *>(ws.eL + 16 * w + 4 * g4);
#pragma unroll
    for (int q = 0; q < NT_W; ++q) {
      // a wave without a q-th column tile loads the last tile and never uses it:
      // unconditional loads keep the prefetch free of branches, whose waits would
      // expose its latency
      const int nt = min(w + 4 * q, D / 16 - 1);
      const uint4 *kr = reinterpret_cast<const uint4 *>(ws.Kt + (16 * nt + r16) * C + 16 * g4);
      const uint4 k01 = kr[0], k23 = kr[1];  // pieces kb = 0, 1 and 2, 3 (kt_pos order)
      kp[q][0] = make_uint2(k01.x, k01.y);
      kp[q][1] = make_uint2(k01.z, k01.w);
      kp[q][2] = make_uint2(k23.x, k23.y);
      kp[q][3] = make_uint2(k23.z, k23.w);
    }
    up = *reinterpret_cast<const float4 *>(ws.U + (i0 + r16) * C + 16 * w + 4 * g4);
    e_last = ws.eG[n - 1];
  }
};

// A wave keeps two chunks' operands live (170 VGPRs), capped so that two blocks share
// a CU: one 2048-token row has 256 (unit, tile) chains, one per CU, but a transaction
// with several long prefill rows has more chains than CUs, and two of them then run
// on each CU at once (the 16-row mixed transaction with 4 prefills of 883-3702 tokens
// took 1012-1025 instead of 1075-1090 us; the single row is unchanged).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void chunk_scan_kernel(ChunkArgs args, int n_units) {
  constexpr int LDS_ = D + 4;
  constexpr int TILES = D / VT;
  constexpr int NKB = D / 16;
  constexpr int NT_W = (D / 16 + 3) / 4;  // state column tiles per wave
  constexpr size_t UNIT = size_t(D) * D;
  // state tile (row i, column d), double-buffered: chunk c reads sSb[c & 1] and writes
  // the next state to sSb[(c + 1) & 1], so no barrier is needed between the last read
  // of a state and the write of the next one
  __shared__ __attribute__((aligned(16))) float sSb[2][VT * LDS_];
  // U^T diag(e^{G_n - G}) of this tile (row i, token s) as its three bf16x3 parts
  __shared__ __attribute__((aligned(16))) uint16_t sUp[3][VT * LDB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  // Blocks of one (row, head) unit are spaced 8 apart in launch order, which places
  // all its tiles on one of the 8 chiplets and lets them share that L2's copy of the
  // chunk operands (W, K^T).
  const int b = blockIdx.x;
  const int k8 = b >> 3;
  const int tile = k8 % TILES;
  const int unit = (k8 / TILES) * 8 + (b & 7);
  if (unit >= n_units) return;
  const int h = unit % args.n_v;
  const int row = unit / args.n_v;
  const int i0 = tile * VT;
  const int L = args.len[row];
  const int nch = (L + C - 1) / C;
  const int n_v = args.n_v;
  const int src = args.src[row], dst = args.dst[row];
  auto ws_of = [&](int c) {
    return Ws<D>(args.ws + (int64_t(args.chunk0[row] + c) * n_v + h) * ChunkArgs::ws_unit_floats(D));
  };

  for (int idx = tid; idx < VT * (D / 4); idx += 256) {
    const int i = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
    float4 x = zf4();
    if (src >= 0)
      x = *reinterpret_cast<const float4 *>(args.state_in + (int64_t(src) * n_v + h) * UNIT +
                                            int64_t(i0 + i) * D + d4);
    *reinterpret_cast<float4 *>(sSb[0] + i * LDS_ + d4) = x;
  }

  // One chunk of the recurrence with its operand fragments f.
  auto body = [&](int c, const ScanFrag<D> &f) {
    const Ws<D> ws = ws_of(c);
    const float *sS = sSb[c & 1];
    float *sS_next = sSb[(c + 1) & 1];
    lds_barrier();  // the state tile of this chunk is in place; the last chunk's reads of sUp are done

    // U = U' - W S_c^T for tokens 16w..16w+15 of this tile's 16 value channels,
    // in two interleaved partial chains
    floatx4 ua = zero4(), ub = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; kb += 2) {
      ua = mma4(ua, f.wf[kb], *reinterpret_cast<const float4 *>(sS + r16 * LDS_ + 16 * kb + 4 * g4));
      if (kb + 1 < NKB)
        ub = mma4(ub, f.wf[kb + 1], *reinterpret_cast<const float4 *>(sS + r16 * LDS_ + 16 * (kb + 1) + 4 * g4));
    }
    // record S_c for the output and checkpoint kernels (issued behind the products)
#pragma unroll
    for (int idx = tid; idx < VT * (D / 4); idx += 256) {
      const int i = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
      *reinterpret_cast<float4 *>(ws.Sc + int64_t(i0 + i) * D + d4) =
          *reinterpret_cast<const float4 *>(sS + i * LDS_ + d4);
    }
    {
      // this lane's tokens 16w + 4g4 + (0..3) of value channel i0 + r16: contiguous in
      // both U^T buffers; LDS gets U^T diag(e^{G_n - G}), as the carry uses it, split
      // into bf16x3 parts once here (K is bf16, so the carry runs on the bf16 matrix
      // cores at fp32 accuracy)
      const float4 u = make_float4(f.up.x - (ua[0] + ub[0]), f.up.y - (ua[1] + ub[1]),
                                   f.up.z - (ua[2] + ub[2]), f.up.w - (ua[3] + ub[3]));
      const Parts4 part = split3x4(mul4(u, f.el));
      const int o = r16 * LDB + 16 * w + 4 * g4;
      *reinterpret_cast<uint2 *>(sUp[0] + o) = part.h;
      *reinterpret_cast<uint2 *>(sUp[1] + o) = part.m;
      *reinterpret_cast<uint2 *>(sUp[2] + o) = part.l;
      *reinterpret_cast<float4 *>(ws.Ut + (i0 + r16) * C + 16 * w + 4 * g4) = u;
    }
    lds_barrier();  // U^T of the tile complete

    // S_{c+1} = e^{G_n} S_c + U^T diag(e^{G_n - G}) K on this wave's column tiles
    auto lds_parts = [&](int kb) {
      const int o = r16 * LDB + 16 * kb + 4 * g4;
      Parts4 r;
      r.h = *reinterpret_cast<const uint2 *>(sUp[0] + o);
      r.m = *reinterpret_cast<const uint2 *>(sUp[1] + o);
      r.l = *reinterpret_cast<const uint2 *>(sUp[2] + o);
      return r;
    };
    const Parts4 a0 = lds_parts(0), a1 = lds_parts(1), a2 = lds_parts(2), a3 = lds_parts(3);
    floatx4 snew[NT_W];
#pragma unroll
    for (int q = 0; q < NT_W; ++q) {
      const int nt = w + 4 * q;
      floatx4 acc = zero4();
      if (nt < D / 16) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = f.e_last * sS[(4 * g4 + v) * LDS_ + 16 * nt + r16];
        acc = mma_bf16x3_64(acc, a0, a1, a2, a3, f.kp[q][0], f.kp[q][1], f.kp[q][2], f.kp[q][3]);
      }
      snew[q] = acc;
    }
#pragma unroll
    for (int q = 0; q < NT_W; ++q) {
      const int nt = w + 4 * q;
      if (nt < D / 16)
#pragma unroll
        for (int v = 0; v < 4; ++v) sS_next[(4 * g4 + v) * LDS_ + 16 * nt + r16] = snew[q][v];
    }
  };
  auto frag_load = [&](ScanFrag<D> &f, int c) {
    c = min(c, nch - 1);  // past the end: reload the last chunk, never read
    f.load(ws_of(c), min(C, L - c * C), w, r16, g4, i0);
  };

  // Chunks in pairs with two fragment sets: the next chunk's operands are in flight
  // while this chunk's products run (fetching two chunks ahead was measured slower).
  ScanFrag<D> fa, fb;
  frag_load(fa, 0);
  for (int c = 0; c < nch; c += 2) {
    frag_load(fb, c + 1);
    body(c, fa);
    if (c + 1 >= nch) break;
    frag_load(fa, c + 2);
    body(c + 1, fb);
  }
  lds_barrier();
  if (dst >= 0) {
    const float *sS = sSb[nch & 1];
    for (int idx = tid; idx < VT * (D / 4); idx += 256) {
      const int i = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
      *reinterpret_cast<float4 *>(args.state_out + (int64_t(dst) * n_v + h) * UNIT +
                                  int64_t(i0 + i) * D + d4) =
          *reinterpret_cast<const float4 *>(sS + i * LDS_ + d4);
    }
  }
}

// Outputs of one (chunk, value head, half of the value channels) from the chunk's
// start state S_c and U recorded by the scan: O = diag(e^G) Q S_c^T + P U.  The
// block stages its half of S_c and of U^T in LDS once; wave w computes tokens
// 16w..16w+15 (Q and P rows in registers) against every 16-channel tile of the half.
template <int D>
__global__ __launch_bounds__(256) void chunk_out_kernel(ChunkArgs args) {
  constexpr int NKB = D / 16;
  constexpr int NH = D / 16 >= 2 ? 2 : 1;  // value-channel parts per chunk
  constexpr int DH = D / NH;              // value channels per part
  constexpr int NTP = DH / 16;            // 16-wide column tiles per part
  constexpr int LDS_ = D + 4;
  __shared__ __attribute__((aligned(16))) float sSc[DH * LDS_];  // S_c rows of this part
  __shared__ __attribute__((aligned(16))) float sU[DH * LDC];    // U^T rows of this part
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int cl = blockIdx.x, h = blockIdx.y, part = blockIdx.z;
  const int row = row_of_chunk(args, cl);
  const int cin = cl - args.chunk_start[row];
  const int c0 = cin * C;
  const int n = min(C, args.len[row] - c0);
  const int64_t tok_base = int64_t(args.tok0[row]) + c0;
  const int n_v = args.n_v, n_qk = args.n_qk, hq = h / args.group;
  const int64_t ldqk = int64_t(n_qk) * D;
  const Ws<D> ws(args.ws + (int64_t(args.chunk0[row] + cin) * n_v + h) * ChunkArgs::ws_unit_floats(D));
  const int i_base = part * DH;

  for (int idx = tid; idx < DH * (D / 4); idx += 256) {
    const int i = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
    *reinterpret_cast<float4 *>(sSc + i * LDS_ + d4) =
        *reinterpret_cast<const float4 *>(ws.Sc + int64_t(i_base + i) * D + d4);
  }
  for (int idx = tid; idx < DH * (C / 4); idx += 256) {
    const int i = idx / (C / 4), s4 = (idx % (C / 4)) * 4;
    *reinterpret_cast<float4 *>(sU + i * LDC + s4) =
        *reinterpret_cast<const float4 *>(ws.Ut + (i_base + i) * C + s4);
  }
  const int t_me = 16 * w + r16;
  const uint16_t *Qc = args.q + tok_base * ldqk + int64_t(hq) * D;
  const uint16_t *qrow = Qc + int64_t(min(t_me, n - 1)) * ldqk;  // rows past the end: never stored
  float4 qf[NKB], pf[4];
  float eg[4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    qf[kb] = unpack_bf16x4(*reinterpret_cast<const uint2 *>(qrow + 16 * kb + 4 * g4));
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) pf[kb] = *reinterpret_cast<const float4 *>(ws.P + t_me * C + 16 * kb + 4 * g4);
#pragma unroll
  for (int v = 0; v < 4; ++v) eg[v] = ws.eG[16 * w + 4 * g4 + v] * ws.rq[16 * w + 4 * g4 + v];
  lds_barrier();

#pragma unroll
  for (int q = 0; q < NTP; ++q) {
    const float *srow = sSc + (16 * q + r16) * LDS_;
    const float *urow = sU + (16 * q + r16) * LDC;
    floatx4 oa = zero4(), ob = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; kb += 2) {
      oa = mma4(oa, qf[kb], *reinterpret_cast<const float4 *>(srow + 16 * kb + 4 * g4));
      if (kb + 1 < NKB) ob = mma4(ob, qf[kb + 1], *reinterpret_cast<const float4 *>(srow + 16 * (kb + 1) + 4 * g4));
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) oa[v] = eg[v] * (oa[v] + ob[v]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)  // P is zero right of the diagonal block
      if (kb <= w) oa = mma4(oa, pf[kb], *reinterpret_cast<const float4 *>(urow + 16 * kb + 4 * g4));
    const int i = i_base + 16 * q + r16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = 16 * w + 4 * g4 + v;
      if (t < n) args.o[((tok_base + t) * n_v + h) * D + i] = to_bf16(oa[v]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void chunk_ckpt_kernel(ChunkArgs args) {
  constexpr size_t UNIT = size_t(D) * D;
  constexpr int MT = D / 16;
  __shared__ __attribute__((aligned(16))) float sScale[C];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  int b = blockIdx.x;
  const int mi = b % MT;
  b /= MT;
  const int h = b % args.n_v;
  b /= args.n_v;
  const int j = b % args.ck_slots;
  const int row = b / args.ck_slots;
  const int n_tail = args.n_tail[row];
  if (j >= n_tail) return;
  const int L = args.len[row];
  const int p = L - n_tail + j;  // checkpoint slot j: state after p + 1 tokens
  const int cin = p / C;
  const int jj = p - cin * C;
  const int n_v = args.n_v;
  const Ws<D> ws(args.ws + (int64_t(args.chunk0[row] + cin) * n_v + h) * ChunkArgs::ws_unit_floats(D));
  // scale_s = e^{G_j' - G_s} rk_s for s <= j' (else 0, a select so an overflowed
  // exponential on the masked side cannot become a NaN), rounded exactly as the
  // carry's factors, so the checkpoint at a row's last position is bit-identical
  // to the final state the scan publishes
  if (w == 0) sScale[lane] = lane <= jj ? float(exp(ws.G[jj] - ws.G[lane])) * ws.rk[lane] : 0.0f;
  lds_barrier();
  // the scan's carry operation, part for part: at a row's last position the scaled U
  // values, their bf16x3 split and the matrix-instruction sequence are the scan's own
  auto scaled_parts = [&](int kb) {
    return split3x4(mul4(*reinterpret_cast<const float4 *>(ws.Ut + (16 * mi + r16) * C + 16 * kb + 4 * g4),
                         *reinterpret_cast<const float4 *>(sScale + 16 * kb + 4 * g4)));
  };
  const Parts4 a0 = scaled_parts(0), a1 = scaled_parts(1), a2 = scaled_parts(2), a3 = scaled_parts(3);
  const float ej = ws.eG[jj];
  float *cdst = args.ckpt + ((int64_t(args.ck_row[row]) * args.ck_slots + j) * n_v + h) * UNIT;
  for (int nt = 2 * w; nt < 2 * w + 2 && nt < D / 16; ++nt) {
    const uint2 *kr = reinterpret_cast<const uint2 *>(ws.Kt + (16 * nt + r16) * C + 16 * g4);  // pieces 0..3
    float sc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = ws.Sc[int64_t(16 * mi + 4 * g4 + v) * D + 16 * nt + r16];
    floatx4 acc;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = ej * sc[v];
    acc = mma_bf16x3_64(acc, a0, a1, a2, a3, kr[0], kr[1], kr[2], kr[3]);
#pragma unroll
    for (int v = 0; v < 4; ++v) cdst[int64_t(16 * mi + 4 * g4 + v) * D + 16 * nt + r16] = acc[v];
  }
}

template <int D>
hipError_t launch_d(const ChunkArgs &args, int n_chunks, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_prep_kernel<D>, dim3(unsigned(n_chunks), unsigned(args.n_v)), dim3(256), 0,
                     stream, args);
  const int n_units = args.n_rows * args.n_v;
  const int groups = (n_units + 7) / 8;  // units are dealt to the 8 chiplets in groups of 8
  hipLaunchKernelGGL(chunk_scan_kernel<D>, dim3(unsigned(groups * 8 * (D / VT))), dim3(256), 0, stream,
                     args, n_units);
  hipLaunchKernelGGL(chunk_out_kernel<D>, dim3(unsigned(n_chunks), unsigned(args.n_v), unsigned(D / 16 >= 2 ? 2 : 1)),
                     dim3(256), 0, stream, args);
  int any_tail = 0;
  for (int r = 0; r < args.n_rows; ++r) any_tail |= args.n_tail[r];
  if (any_tail)
    hipLaunchKernelGGL(chunk_ckpt_kernel<D>, dim3(unsigned(args.n_rows * args.ck_slots * args.n_v * (D / 16))),
                       dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

// Workspace of gdn_chunked_prefill_with_checkpoints_static: a file-scope device array,
// one copy per GPU, resident from the library's load until the process ends.  In host
// code its name is only a stand-in for the symbol: kernels get the address that
// hipGetSymbolAddress returns for the current GPU, never the name.
__device__ __align__(256) float scratch[GDN_STATIC_WS_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];  // per GPU, filled on first use
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_workspace(void **ptr, size_t *bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  *bytes = GDN_STATIC_WS_BYTES;
  return hipSuccess;
}

hipError_t launch_chunked(const ChunkArgs &args, int d, int n_chunks, hipStream_t stream) {
  if (args.n_rows <= 0 || n_chunks <= 0) return hipSuccess;
  if (d == 128) return launch_d<128>(args, n_chunks, stream);
  if (d == 16) return launch_d<16>(args, n_chunks, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
