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
// scalings above, so the matrix cores still see the bf16 inputs.  A checkpoint at
// in-chunk position j is (1) truncated at s <= j: one more rank-64 product per
// requested position, so a long prefill in a ragged batch still publishes the
// intermediate states a draft rollback needs (the gap named in the onnxruntime-genai
// pull request "Run chained MTP drafting in the batch Engine", section "Correctness fix").
//
// Two kernels, same stream:
//   chunk_prep_kernel   one block per (chunk, value head), all chunks in parallel:
//       gates, fp64 prefix sum of g, K K^T and Q K^T, forward substitution for T,
//       W, U', P = Gamma o Q K^T, K^T and the decay factors -> workspace.
//   chunk_chain_kernel  one block per (row, value head, 16 value channels), chunks in
//       order: U = U' - W S_c^T, the state carry, the requested checkpoints and the
//       final state in four waves, the outputs O of the block's channels in four more.
//       The state tile never leaves the block: each carrying lane keeps its part in
//       registers, and LDS holds the bf16 parts that the products read.
// Every product runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, 2.5 PF dense
// on MI355X) at fp32 accuracy: an fp32 operand enters as three bf16 parts that sum to it
// to within 2^-24 of its magnitude (hi, the round of what hi leaves, the round of what
// both leave; every subtraction exact), and the products of the parts that matter are
// accumulated in fp32 -- three when the other operand is exactly bf16 (K, Q, V), six when
// both are fp32 (the bf16x3 split: Henry, Tang & Heinecke, "Leveraging the bfloat16
// Artificial Intelligence Datatype for Higher-Precision Computations", ARITH 2019).  The
// prep kernel's T products run on the fp32 matrix cores.  Decays are formed only as
// differences G_t - G_s with s <= t, from an fp64 prefix sum (|G| reaches hundreds within a
// chunk under strong decay, where differences of fp32 sums would lose ~1e-5 relative).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = 64;       // chunk length
constexpr int VT = 16;      // state rows (value channels) per chain block
constexpr int LDC = C + 4;  // padded LDS row length (floats) for C-wide rows
constexpr int LDB = C + 4;  // padded LDS row length (bf16) for C-wide rows (prep)
constexpr int LDP = C + 8;  // row length (bf16) of C-wide part buffers: 16-B aligned rows

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ float4 zf4() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }
__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

// One 16-wide k block of acc(16x16) += A(16 x K) * B(K x 16) on the fp32 matrix cores.
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

// acc(16x16) += A(16 x 32) * B(32 x 16) on the bf16 matrix cores: lane (r, g) gives
// A[r][8g .. 8g+7] and B[8g .. 8g+7][r]; lane (r, g) then holds C[4g + v][r] in acc[v].
__device__ __forceinline__ floatx4 mfma_bf16(bf16x8 a, bf16x8 b, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// Two fp32 values to bf16 bits, round to nearest even (v_cvt_pk_bf16_f32), packed
// low-first.
__device__ __forceinline__ uint32_t bf16x2_rn(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
}

// The three bf16 parts of two values, each part the round of what the parts before it
// leave; every subtraction is exact, and hi + mid + lo equals the value to within
// 2^-24 of its magnitude.
__device__ __forceinline__ void split_pair(float x, float y, uint32_t &h, uint32_t &m, uint32_t &l) {
  h = bf16x2_rn(x, y);
  const float rx = x - __uint_as_float(h << 16), ry = y - __uint_as_float(h & 0xFFFF0000u);
  m = bf16x2_rn(rx, ry);
  l = bf16x2_rn(rx - __uint_as_float(m << 16), ry - __uint_as_float(m & 0xFFFF0000u));
}

struct Parts8 {  // eight values as three bf16x8 matrix operands
  bf16x8 h, m, l;
};
struct Parts4 {  // four values as three 8-byte pieces (bf16 bits)
  uint2 h, m, l;
};
__device__ __forceinline__ Parts4 split4(float4 a) {
  uint32_t h0, m0, l0, h1, m1, l1;
  split_pair(a.x, a.y, h0, m0, l0);
  split_pair(a.z, a.w, h1, m1, l1);
  return Parts4{make_uint2(h0, h1), make_uint2(m0, m1), make_uint2(l0, l1)};
}

// acc += A B with A in parts and B exactly bf16 (three products, smallest first)
__device__ __forceinline__ floatx4 mma3a(floatx4 acc, const Parts8 &a, bf16x8 b) {
  acc = mfma_bf16(a.l, b, acc);
  acc = mfma_bf16(a.m, b, acc);
  return mfma_bf16(a.h, b, acc);
}
// acc += A B with A exactly bf16 and B in parts
__device__ __forceinline__ floatx4 mma3b(floatx4 acc, bf16x8 a, const Parts8 &b) {
  acc = mfma_bf16(a, b.l, acc);
  acc = mfma_bf16(a, b.m, acc);
  return mfma_bf16(a, b.h, acc);
}
// acc += A B with both in parts: the six products whose parts reach 2^-16 of the
// leading one (the three below that are dropped: 2^-24 relative)
__device__ __forceinline__ floatx4 mma6(floatx4 acc, const Parts8 &a, const Parts8 &b) {
  acc = mfma_bf16(a.l, b.h, acc);
  acc = mfma_bf16(a.m, b.m, acc);
  acc = mfma_bf16(a.h, b.l, acc);
  acc = mfma_bf16(a.m, b.h, acc);
  acc = mfma_bf16(a.h, b.m, acc);
  return mfma_bf16(a.h, b.h, acc);
}

// Part buffers in LDS: three planes of rows of bf16.  A lane writes four consecutive
// values of one row (8 B per plane) and reads eight (16 B per plane).
template <int PITCH>
__device__ __forceinline__ void lds_put4(uint16_t *buf, int plane_elems, int row, int col, const Parts4 &p) {
  uint16_t *q = buf + row * PITCH + col;
  *reinterpret_cast<uint2 *>(q) = p.h;
  *reinterpret_cast<uint2 *>(q + plane_elems) = p.m;
  *reinterpret_cast<uint2 *>(q + 2 * plane_elems) = p.l;
}
template <int PITCH>
__device__ __forceinline__ Parts8 lds_get8(const uint16_t *buf, int plane_elems, int row, int col) {
  const uint16_t *q = buf + row * PITCH + col;
  return Parts8{*reinterpret_cast<const bf16x8 *>(q), *reinterpret_cast<const bf16x8 *>(q + plane_elems),
                *reinterpret_cast<const bf16x8 *>(q + 2 * plane_elems)};
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

// Workspace of one (chunk, value head).  The chain kernel's operands are stored in
// fragment order: every 16-byte piece a lane of a wave takes for one matrix instruction
// sits at piece index lane of a 1 KiB block, so each of the chain kernel's loads reads
// 1 KiB contiguous (a wave reading 16 rows of 64 bytes instead measured ~3x slower per
// load, which bounded the chain).  With token tile tt (16 tokens), 32-wide block kb,
// bf16 part plane p (hi, mid, lo: their sum is the fp32 value to within 2^-24 of it),
// 16-wide state column tile nt and lane l = r + 16 g:
//   WF [tt][kb][p][l]  W[16 tt + r][32 kb + 8 g + e]      (e = 0..7, bf16 parts; in a
//                      streamed workspace fp32 [tt][kb][l][e], 32 bytes per lane)
//   QF [tt][kb][l]     Q[16 tt + r][32 kb + 8 g + e]      (bf16, the input q)
//   KF [nt][kb][l]     K[32 kb + 8 g + e][16 nt + r]      (bf16, kb < 2: tokens)
//   PF [b][p][l]       P[16 tt + r][32 kb + 8 g + e]      (bf16 parts, block b = pblk(tt, kb))
//   UF [nt][tt][l]     U'[16 tt + 4 g + v][16 nt + r]     (fp32, v = 0..3)
// with P[t][s] = e^{G_t - G_s} rq_t rk_s q_t.k_s for s <= t, else 0; then G [C] fp64,
// eG[t] = e^{G_t}, eL[s] = e^{G_{n-1} - G_s} rk_s (s < n, else 0), rk[s] (the factor
// token s's key is scaled by) and eGq[t] = e^{G_t} rq_t (the factor of the output's state
// term); rk = rq = 1 unless q/k are normalised in the kernels.  P is zero right of the
// diagonal, so the blocks (tt < 2, kb = 1) are not stored.  For d = 16 the pieces of
// lanes g >= 2 of WF lie past the head width and are not written (the chain kernel reads
// zeros in their place); QF holds zeros there.
// A workspace store: cached (NT = false), or streamed past the caches (NT = true).  The
// chain kernel reads the workspace right after this one; when it fits well within the
// 256 MB last-level cache it is read from there (the 2048-token prefill's 138 MB: 103 us
// cached against 120 us streamed), and when it does not, streaming the writes spares the
// caches (the 4-prefill transaction's 750 MB: 690 -> 662 us) and W goes out in fp32, an
// eighth less to write and read (the same transaction 650 -> 625 us; in the cached form the
// chain kernel's split of W measured 2 us slower per 2048-token prefill).
template <bool NT, typename T>
__device__ __forceinline__ void ws_st(T *p, T v) {
  if constexpr (NT) {
    if constexpr (sizeof(T) == 8) {
      typedef unsigned int u32x2s __attribute__((ext_vector_type(2)));
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2s, v), reinterpret_cast<u32x2s *>(p));
    } else {
      typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4s, v), reinterpret_cast<u32x4s *>(p));
    }
  } else {
    *p = v;
  }
}

template <int D, bool W32>
struct Ws {
  static constexpr int NK = D >= 32 ? D / 32 : 1;  // 32-wide blocks over d
  static constexpr int NT = D / 16;                // 16-wide state column tiles
  static constexpr int64_t UNIT = chunk_ws_unit_floats(D, W32);  // floats per (chunk, value head)
  static constexpr int64_t QK = chunk_ws_qk_floats(D);           // floats per (chunk, qk-head)
  uint16_t *WF, *QF, *KF, *PF;
  float *WF32, *UF, *eG, *eL, *rk, *eGq;
  double *G;
  // the value-head unit at `base`, its qk-head's Q and K^T at `qk`
  __device__ Ws(float *base, float *qk) {
    WF = reinterpret_cast<uint16_t *>(base);
    WF32 = base;
    PF = W32 ? reinterpret_cast<uint16_t *>(base + 4 * NK * 512) : WF + 4 * NK * 3 * 512;
    UF = reinterpret_cast<float *>(PF + 6 * 3 * 512);
    G = reinterpret_cast<double *>(UF + NT * 4 * 256);
    eG = reinterpret_cast<float *>(G + C);
    eL = eG + C;
    rk = eL + C;
    eGq = rk + C;
    QF = reinterpret_cast<uint16_t *>(qk);
    KF = QF + 4 * NK * 512;
  }
  // the units of workspace chunk `chunk`, value head h of qk-head hq
  __device__ Ws(const ChunkArgs &a, int64_t chunk, int h, int hq)
      : Ws(a.ws + (chunk * a.n_v + h) * UNIT, a.ws_qk + (chunk * a.n_qk + hq) * QK) {}
  // element offset of lane l's 16-byte piece in 1-KiB fragment block `blk` of a bf16 array
  static __device__ __forceinline__ int piece(int blk, int l) { return (blk * 64 + l) * 8; }
  // P block of token tile tt and 32-wide key block kb (kb = 1 only for tt >= 2)
  static __device__ __forceinline__ int pblk(int tt, int kb) { return tt < 2 ? tt : 2 * tt - 2 + kb; }
};

// q/k normalisation of the fused input mode: x / sqrt(sum x^2 + eps), q also by
// 1/sqrt(d_k).
constexpr float kNormEps = 1e-6f;
template <int D>
constexpr float inv_sqrt_d() {
  static_assert(D == 16 || D == 128, "head width");
  return D == 16 ? 0.25f : 0.0883883476483184405501f;
}

// V has no LDS buffer of its own: its rows are loaded into registers (whole 16-byte row
// pieces) while T is solved, and written transposed into the K buffer once step 4 holds
// its K^T columns.  36 KiB of LDS and at most 128 registers give four blocks per CU
// instead of three (with V^T staged beside K from the start: 53.5 KiB), one round of blocks
// for a 2048-token row (prefill 102 -> 97 us, transaction 616 -> 604 us).
template <int D, bool NT>
__global__ __launch_bounds__(256, 3) void chunk_prep_kernel(ChunkArgs args) {
  __shared__ double sG[C];
  __shared__ __attribute__((aligned(16))) float sBeta[C];  // beta_m
  __shared__ __attribute__((aligned(16))) float sSK[C];    // beta_m e^{G_m}
  __shared__ __attribute__((aligned(16))) float sA[C * LDC];  // strictly lower A, then T = (I + A)^{-1}
  constexpr int LDK = D + 8;  // row length (bf16) of sK: 16-B aligned rows
  __shared__ __attribute__((aligned(16))) uint16_t sK[C * LDK];   // K (bf16): row token m, column d
  __shared__ float sRk[C];  // per-token k scale factors (1: inputs taken as given)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  // Block id -> (chunk, value head).  Blocks are dealt to the 8 chiplets by id % 8; with
  // qk-heads in multiples of 8, the value heads of one qk-head go to one chiplet, chunk
  // by chunk, so they share its L2 copy of the chunk's q and k rows and gate lines
  // (4-prefill transaction: 345 -> 203 MB fetched by this kernel, about the inputs once).
  int cl, h;
  {
    const int id = blockIdx.x, nc = gridDim.x / args.n_v;
    if (args.n_qk % 8 == 0) {
      const int x = id % 8, j = id / 8, per = args.n_v / 8;  // per: value heads per chiplet and chunk
      cl = j / per;
      const int l = j % per;
      h = (x + 8 * (l / args.group)) * args.group + l % args.group;
    } else {
      cl = id % nc;
      h = id / nc;
    }
  }
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
  Ws<D, NT> ws(args, args.chunk0[row] + cin, h, hq);
  // Q and K^T depend on the qk-head only: the first of its value heads stores them
  const bool qk_owner = h == hq * args.group;

  auto frag32 = [&](const uint16_t *base, int64_t ld, int t, int kb) {
    return frag32_row<D>(base, ld, t, kb, n, g4);
  };

  // 1. gates and the fp64 inclusive prefix sum of g (tokens t >= n: g = beta = 0);
  //    K in LDS, with the k and q norms when normalising.
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
  // K rows to sK, with the k norms when normalising.
  // Thread tid takes 8 dims (16 bytes) of one token, so each load instruction reads whole
  // 256-byte rows of 4 tokens (a wave reading 16 rows of 32 bytes instead measured ~3x
  // slower per byte).  Rows past the chunk's end are zero.
  {
    constexpr int TPT = D / 8;       // threads per token
    constexpr int TPR = 256 / TPT;   // tokens per round
    const bool norm = args.qk_norm != 0;
    const int d8 = 8 * (tid % TPT);
#pragma unroll
    for (int it = 0; it < (C + TPR - 1) / TPR; ++it) {
      const int m = tid / TPT + TPR * it;
      if (m >= C) break;
      uint4 kw = make_uint4(0u, 0u, 0u, 0u);
      if (m < n) kw = *reinterpret_cast<const uint4 *>(Kc + int64_t(m) * ldqk + d8);
      *reinterpret_cast<uint4 *>(sK + m * LDK + d8) = kw;
      if (norm) {  // the TPT consecutive lanes of token m hold its partial sums
        const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ss = fmaf(bf16_lo(kk[e]), bf16_lo(kk[e]), ss);
          ss = fmaf(bf16_hi(kk[e]), bf16_hi(kk[e]), ss);
        }
#pragma unroll
        for (int off = 1; off < TPT; off <<= 1) ss += __shfl_xor(ss, off, 64);
        if (d8 == 0) sRk[m] = m < n ? 1.0f / sqrtf(ss + kNormEps) : 0.0f;
      } else if (d8 == 0) {
        sRk[m] = 1.0f;
      }
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
  }
  // K^T in fragment order for the chain kernel's carry: piece (nt, kb, l = r + 16 g) is
  // K^T[16 nt + r][32 kb + 8 g .. +7], a column of sK
  for (int idx = tid; qk_owner && idx < (D / 16) * 2 * 64; idx += 256) {
    const int nt = idx >> 7, kb = (idx >> 6) & 1, l = idx & 63;
    const uint16_t *src = sK + (32 * kb + 8 * (l >> 4)) * LDK + 16 * nt + (l & 15);
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = uint32_t(src[(2 * e) * LDK]) | (uint32_t(src[(2 * e + 1) * LDK]) << 16);
    ws_st<NT>(reinterpret_cast<uint4 *>(ws.KF + idx * 8), make_uint4(wv[0], wv[1], wv[2], wv[3]));
  }

  // 2. K K^T -> A (strictly lower, scaled) and Q K^T -> P (lower with diagonal) on
  //    the bf16 matrix cores: K and Q are bf16, so every product is exact in fp32 and
  //    only the fp32 accumulation rounds.  Wave w owns row block w: it loads the
  //    fragments once (its Q rows, the K rows of all four blocks), computes tiles
  //    (w, tj <= w) and writes zeros to the tiles right of the diagonal.  Q K^T is
  //    formed transposed (lane: token 16 w + r16, keys 16 tj + 4 g4 + v), so each lane
  //    holds 4 consecutive columns of a P row and P goes out in parts, in fragment order
  //    (the two blocks that are zero everywhere, rows < 32 and keys >= 32, are not stored).
  //    The wave's Q fragments are the chain kernel's: stored as they are.
  {
    constexpr int NK32 = (D + 31) / 32;  // 32-wide k blocks over d (D = 16: half of one)
    bf16x8 fk[4][NK32], fa[NK32], fq[NK32];  // fa: this wave's K rows (register arrays
    const bf16x8 z8 = __builtin_bit_cast(bf16x8, u32x4v{0u, 0u, 0u, 0u});  // are indexed by constants only)
    float ssq = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NK32; ++kb) {
      const int col = 32 * kb + 8 * g4;
      fq[kb] = frag32(Qc, ldqk, 16 * w + r16, kb);
#pragma unroll
      for (int tj = 0; tj < 4; ++tj)
        fk[tj][kb] = col < D ? *reinterpret_cast<const bf16x8 *>(sK + (16 * tj + r16) * LDK + col) : z8;
      fa[kb] = col < D ? *reinterpret_cast<const bf16x8 *>(sK + (16 * w + r16) * LDK + col) : z8;
      if (qk_owner)
        ws_st<NT>(reinterpret_cast<uint4 *>(ws.QF + Ws<D, NT>::piece(w * NK32 + kb, lane)), __builtin_bit_cast(uint4, fq[kb]));
#pragma unroll
      for (int e = 0; e < 8; ++e) ssq = fmaf(float(fq[kb][e]), float(fq[kb][e]), ssq);
    }
    // q's factor for the lane's row t = 16 w + r16: its 4 lanes (g4) hold the partial sums
    const int t_q = 16 * w + r16;
    float rq = 1.0f;
    if (args.qk_norm) {
      ssq += __shfl_xor(ssq, 16, 64);
      ssq += __shfl_xor(ssq, 32, 64);
      rq = t_q < n ? 1.0f / sqrtf(ssq + kNormEps) * inv_sqrt_d<D>() : 0.0f;
    }
    if (g4 == 0) ws.eGq[t_q] = float(exp(sG[t_q])) * rq;
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      floatx4 kk = zero4(), qk = zero4();
      if (tj <= w) {
#pragma unroll
        for (int kb = 0; kb < NK32; ++kb) {
          kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[kb], fk[tj][kb], kk, 0, 0, 0);
          qk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[tj][kb], fq[kb], qk, 0, 0, 0);
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * w + 4 * g4 + v, s = 16 * tj + r16;
        float av = 0.0f;
        if (s < t) av = sBeta[t] * expf(float(sG[t] - sG[s])) * (kk[v] * sRk[t] * sRk[s]);
        if (tj <= w) sA[t * LDC + s] = av;  // the upper blocks of sA hold T below
      }
      float pv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * w + r16, s = 16 * tj + 4 * g4 + v;
        pv[v] = s <= t ? expf(float(sG[t] - sG[s])) * (qk[v] * rq * sRk[s]) : 0.0f;
      }
      // lane (r16, g4) holds P[16 w + r16][16 tj + 4 g4 + 0..3]: half of the 16-byte piece
      // of lane r16 + 16 (2 (tj & 1) + g4 / 2) in block (pblk(w, tj / 2), part)
      if (w >= 2 || tj < 2) {  // wave-uniform
        const Parts4 pp = split4(make_float4(pv[0], pv[1], pv[2], pv[3]));
        const int l2 = r16 + 16 * (2 * (tj & 1) + (g4 >> 1)), half = 4 * (g4 & 1);
        const int pb = Ws<D, NT>::pblk(w, tj >> 1) * 3;
        ws_st<NT>(reinterpret_cast<uint2 *>(ws.PF + Ws<D, NT>::piece(pb + 0, l2) + half), pp.h);
        ws_st<NT>(reinterpret_cast<uint2 *>(ws.PF + Ws<D, NT>::piece(pb + 1, l2) + half), pp.m);
        ws_st<NT>(reinterpret_cast<uint2 *>(ws.PF + Ws<D, NT>::piece(pb + 2, l2) + half), pp.l);
      }
    }
  }
  lds_barrier();

  // V rows for step 4, loaded now so their latency overlaps the T solve: thread tid takes
  // 8 dims of token tid / (D / 8) + 256 / (D / 8) * it, as the K staging did (zero past
  // the chunk's end)
  constexpr int VTPT = D / 8, VTPR = 256 / VTPT, VNIT = (C + VTPR - 1) / VTPR;
  uint4 vrow[VNIT];
#pragma unroll
  for (int it = 0; it < VNIT; ++it) {
    const int m = tid / VTPT + VTPR * it;
    vrow[it] = make_uint4(0u, 0u, 0u, 0u);
    if (m < n) vrow[it] = *reinterpret_cast<const uint4 *>(Vc + int64_t(m) * ldv + 8 * (tid % VTPT));
  }

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

  // 4. W = T diag(beta e^G rk) K (stored as three bf16 parts) and U' = T diag(beta) V on
  //    the bf16 matrix cores: K and V are exact bf16 operands, and each scaled row of T
  //    enters in three parts.  Wave w owns state column tiles nt = 2w, 2w+1; T is lower
  //    triangular, so row tile ti needs only the 32-token blocks kb <= ti / 2.  W comes out
  //    transposed (lane: token 16 ti + r16, columns 16 nt + 4 g4 + 0..3), U' as
  //    U'[16 ti + 4 g4 + v][16 nt + r16]: both in the chain kernel's fragment order.
  {
    bf16x8 kt8[2][2], vt8[2][2];  // K and V columns d = 16 nt + r16, tokens 32 kb + 8 g4 + 0..7
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = 16 * min(2 * w + j, D / 16 - 1) + r16;  // waves without a tile read tile 0, unused
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int s0 = 32 * kb + 8 * g4;
        uint32_t kw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kw[e] = uint32_t(sK[(s0 + 2 * e) * LDK + d]) | (uint32_t(sK[(s0 + 2 * e + 1) * LDK + d]) << 16);
        kt8[j][kb] = __builtin_bit_cast(bf16x8, u32x4v{kw[0], kw[1], kw[2], kw[3]});
      }
    }
    lds_barrier();  // every wave holds its K^T columns: the K buffer takes V^T
    {
      uint16_t *sVt = sK;  // V^T (bf16): row d, column token m, pitch LDB
      static_assert(D * LDB <= C * LDK, "V^T fits the K buffer");
      const int d8 = 8 * (tid % VTPT);
#pragma unroll
      for (int it = 0; it < VNIT; ++it) {
        const int m = tid / VTPT + VTPR * it;
        if (m >= C) break;
        const uint32_t vv[4] = {vrow[it].x, vrow[it].y, vrow[it].z, vrow[it].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sVt[(d8 + 2 * e) * LDB + m] = uint16_t(vv[e]);
          sVt[(d8 + 2 * e + 1) * LDB + m] = uint16_t(vv[e] >> 16);
        }
      }
      lds_barrier();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int d = 16 * min(2 * w + j, D / 16 - 1) + r16;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int s0 = 32 * kb + 8 * g4;
          const uint2 v0 = *reinterpret_cast<const uint2 *>(sVt + d * LDB + s0);  // 8-B aligned rows
          const uint2 v1 = *reinterpret_cast<const uint2 *>(sVt + d * LDB + s0 + 4);
          vt8[j][kb] = __builtin_bit_cast(bf16x8, u32x4v{v0.x, v0.y, v1.x, v1.y});
        }
      }
    }
    const bool has0 = 2 * w < D / 16, has1 = 2 * w + 1 < D / 16;
    for (int ti = 0; ti < 4; ++ti) {
      floatx4 wa[2] = {zero4(), zero4()}, ua[2] = {zero4(), zero4()};
      for (int kb = 0; kb <= ti / 2; ++kb) {
        // T[16 ti + r16][32 kb + 8 g4 + 0..7]: token block j = 2 kb + g4 / 2 of row tile ti,
        // stored right of the diagonal at rows 16 j when j < ti, in place when j == ti, zero above
        const int j = 2 * kb + (g4 >> 1), c = 8 * (g4 & 1);
        float4 x0 = zf4(), x1 = zf4();
        if (j <= ti) {
          const float *src = j < ti ? sA + (16 * j + r16) * LDC + 16 * ti + c : sA + (16 * ti + r16) * LDC + 16 * ti + c;
          x0 = *reinterpret_cast<const float4 *>(src);
          x1 = *reinterpret_cast<const float4 *>(src + 4);
        }
        const int s0 = 32 * kb + 8 * g4;
        const float4 sk0 = *reinterpret_cast<const float4 *>(sSK + s0), sk1 = *reinterpret_cast<const float4 *>(sSK + s0 + 4);
        const float4 sb0 = *reinterpret_cast<const float4 *>(sBeta + s0), sb1 = *reinterpret_cast<const float4 *>(sBeta + s0 + 4);
        const Parts4 k0 = split4(mul4(x0, sk0)), k1 = split4(mul4(x1, sk1));
        const Parts4 b0 = split4(mul4(x0, sb0)), b1 = split4(mul4(x1, sb1));
        const Parts8 tk{__builtin_bit_cast(bf16x8, u32x4v{k0.h.x, k0.h.y, k1.h.x, k1.h.y}),
                        __builtin_bit_cast(bf16x8, u32x4v{k0.m.x, k0.m.y, k1.m.x, k1.m.y}),
                        __builtin_bit_cast(bf16x8, u32x4v{k0.l.x, k0.l.y, k1.l.x, k1.l.y})};
        const Parts8 tv{__builtin_bit_cast(bf16x8, u32x4v{b0.h.x, b0.h.y, b1.h.x, b1.h.y}),
                        __builtin_bit_cast(bf16x8, u32x4v{b0.m.x, b0.m.y, b1.m.x, b1.m.y}),
                        __builtin_bit_cast(bf16x8, u32x4v{b0.l.x, b0.l.y, b1.l.x, b1.l.y})};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          wa[jj] = mma3b(wa[jj], kb == 0 ? kt8[jj][0] : kt8[jj][1], tk);
          ua[jj] = mma3a(ua[jj], tv, kb == 0 ? vt8[jj][0] : vt8[jj][1]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        if (!(jj == 0 ? has0 : has1)) continue;
        const int nt = 2 * w + jj;
        // W in parts, in fragment order: lane (r16, g4) holds W[16 ti + r16][16 nt + 4 g4 + 0..3],
        // half of the piece of lane r16 + 16 (2 (nt & 1) + g4 / 2) in block (ti, nt / 2, part)
        const int l2 = r16 + 16 * (2 * (nt & 1) + (g4 >> 1)), half = 4 * (g4 & 1);
        if constexpr (NT) {  // streamed: W in fp32, lane l2's 32-byte piece of block (ti, nt / 2)
          const int wb = ti * Ws<D, NT>::NK + (nt >> 1);
          ws_st<NT>(reinterpret_cast<float4 *>(ws.WF32 + (wb * 64 + l2) * 8 + half),
                    make_float4(wa[jj][0], wa[jj][1], wa[jj][2], wa[jj][3]));
        } else {
          const Parts4 wp = split4(make_float4(wa[jj][0], wa[jj][1], wa[jj][2], wa[jj][3]));
          const int wb = (ti * Ws<D, NT>::NK + (nt >> 1)) * 3;
          ws_st<NT>(reinterpret_cast<uint2 *>(ws.WF + Ws<D, NT>::piece(wb + 0, l2) + half), wp.h);
          ws_st<NT>(reinterpret_cast<uint2 *>(ws.WF + Ws<D, NT>::piece(wb + 1, l2) + half), wp.m);
          ws_st<NT>(reinterpret_cast<uint2 *>(ws.WF + Ws<D, NT>::piece(wb + 2, l2) + half), wp.l);
        }
        // U': lane (r16, g4) holds U'[16 ti + 4 g4 + v][16 nt + r16], the piece of block (nt, ti)
        ws_st<NT>(reinterpret_cast<float4 *>(ws.UF + ((nt * 4 + ti) * 64 + lane) * 4),
                  make_float4(ua[jj][0], ua[jj][1], ua[jj][2], ua[jj][3]));
      }
    }
  }
}

// One chunk's operands of a chain wave (w < 4, lane = r16 + 16 g4), fetched a chunk
// ahead; every load reads one 1-KiB fragment block of the workspace (2 KiB for fp32 W).
template <int D, bool W32, int TPB>
struct CarryOps {
  static constexpr int NK = Ws<D, W32>::NK;
  static constexpr int NT = (D / 16 + 3) / 4;  // 16-wide state column tiles per wave
  // W[16 w + r16][32 kb + 8 g4 + 0..7] (zero past d): in parts as stored, or in fp32 from
  // a streamed workspace, split where it is used (the same parts the prep kernel forms)
  Parts8 w[W32 ? 1 : NK];
  float4 wf[W32 ? NK : 1][2];
  bf16x8 kt[NT][2];   // K^T[16 nt + r16][32 kb + 8 g4 + 0..7], nt = w + 4 q
  float4 up[TPB];     // U'[16 w + 4 g4 + v][i0_j + r16], v = 0..3, for each of the block's tiles j
  float4 el;          // eL[16 w + 4 g4 + v]
  float e_last;       // e^{G_{n-1}}
  // Two groups, each loaded where the chunk before has matrix work to hide it behind:
  // (a) W of block kb, used by the U stage; (b) K^T, U', eL, e_last, used by the U
  // exchange and the carry.
  __device__ void load_a(const Ws<D, W32> &ws, int kb, int wv, int lane) {
    const int g4 = lane >> 4;
    if constexpr (W32) {
      const float4 *src = reinterpret_cast<const float4 *>(ws.WF32 + ((wv * NK + kb) * 64 + lane) * 8);
      if (32 * kb + 8 * g4 < D) {
        wf[kb][0] = src[0];
        wf[kb][1] = src[1];
      } else {
        wf[kb][0] = wf[kb][1] = zf4();
      }
    } else {
      const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4v{0u, 0u, 0u, 0u});
      const int b3 = (wv * NK + kb) * 3;
      w[kb] = 32 * kb + 8 * g4 < D ? Parts8{frag(ws.WF, b3, lane), frag(ws.WF, b3 + 1, lane), frag(ws.WF, b3 + 2, lane)}
                                   : Parts8{z, z, z};
    }
  }
  __device__ Parts8 w_parts(int kb) const {
    if constexpr (W32) {
      const Parts4 a = split4(wf[kb][0]), b = split4(wf[kb][1]);
      return Parts8{__builtin_bit_cast(bf16x8, u32x4v{a.h.x, a.h.y, b.h.x, b.h.y}),
                    __builtin_bit_cast(bf16x8, u32x4v{a.m.x, a.m.y, b.m.x, b.m.y}),
                    __builtin_bit_cast(bf16x8, u32x4v{a.l.x, a.l.y, b.l.x, b.l.y})};
    } else {
      return w[kb];
    }
  }
  __device__ void load_b(const Ws<D, W32> &ws, int n, int wv, int lane, int tile) {
    const int g4 = lane >> 4;
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) {
      // a wave without a qt-th tile loads the last one and never uses it: unconditional
      // loads keep the prefetch free of branches
      const int nt = min(wv + 4 * qt, D / 16 - 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kt[qt][kb] = frag(ws.KF, nt * 2 + kb, lane);
    }
#pragma unroll
    for (int j = 0; j < TPB; ++j) up[j] = *reinterpret_cast<const float4 *>(ws.UF + (((tile * TPB + j) * 4 + wv) * 64 + lane) * 4);
    el = *reinterpret_cast<const float4 *>(ws.eL + 16 * wv + 4 * g4);
    e_last = ws.eG[n - 1];
  }
  __device__ void load(const Ws<D, W32> &ws, int n, int wv, int lane, int tile) {
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) load_a(ws, kb, wv, lane);
    load_b(ws, n, wv, lane, tile);
  }
  static __device__ __forceinline__ bf16x8 frag(const uint16_t *a, int blk, int lane) {
    return *reinterpret_cast<const bf16x8 *>(a + Ws<D, false>::piece(blk, lane));
  }
};

// One chunk's operands of an output wave (token tile t = w - 4), fetched a chunk ahead.
template <int D, bool W32>
struct OutOps {
  static constexpr int NK = Ws<D, W32>::NK;
  bf16x8 q[NK];       // Q[16 t + r16][32 kb + 8 g4 + 0..7] (zero past d)
  Parts8 p[2];        // P[16 t + r16][32 kb + 8 g4 + 0..7] in parts (kb = 1: t >= 2 only)
  float egq;          // eGq[16 t + r16]
  __device__ void load_q(const Ws<D, W32> &ws, int kb, int t, int lane) {
    q[kb] = CarryOps<D, W32, 1>::frag(ws.QF, t * NK + kb, lane);
  }
  __device__ void load_p(const Ws<D, W32> &ws, int t, int lane) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb == 1 && t < 2) break;  // that block of P is zero (wave-uniform)
      const int b3 = Ws<D, false>::pblk(t, kb) * 3;
      p[kb] = Parts8{CarryOps<D, W32, 1>::frag(ws.PF, b3, lane), CarryOps<D, W32, 1>::frag(ws.PF, b3 + 1, lane),
                     CarryOps<D, W32, 1>::frag(ws.PF, b3 + 2, lane)};
    }
    egq = ws.eGq[16 * t + (lane & 15)];
  }
  __device__ void load(const Ws<D, W32> &ws, int t, int lane) {
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) load_q(ws, kb, t, lane);
    load_p(ws, t, lane);
  }
};

// A 16-byte store that bypasses the caches on its way to memory (dense states are
// written once and not read back by this call).
__device__ __forceinline__ void store_nt(float *dst, float4 x) {
  __builtin_nontemporal_store(floatx4{x.x, x.y, x.z, x.w}, reinterpret_cast<floatx4 *>(dst));
}
__device__ __forceinline__ void store_nt(float *dst, floatx4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<floatx4 *>(dst));
}

// The chains of one (row, value head) and TPB tiles of 16 value channels (tile j:
// i0 + 16 j .. i0 + 16 j + 15): chunks in order, in blocks of 8 waves, two per SIMD.
// Waves 0..3 carry the state: wave w owns tokens 16w..16w+15 of each chunk for U and
// state column tiles w and w + 4 for the carry.
// Waves 4..7 compute the outputs: wave 4 + t those of tokens 16t..16t+15.  Per chunk:
//   A  chain waves: U = U' - W S_c^T for their tokens (S_c's parts from LDS, W split in
//      registers); U^T diag(e^{G_n - G}) and U^T in parts -> LDS.
//      output waves: (Q S_c^T)^T for their tokens from the same S_c parts.   barrier
//   B  chain waves: the carry S_{c+1} = e^{G_n} S_c + U^T diag(.) K on their column
//      tiles, the checkpoints this chunk holds, S_{c+1}'s parts -> LDS.
//      output waves: O = diag(e^G rq) Q S_c^T + P U for their tokens (U's parts from
//      LDS), stored.                                                          barrier
// The output products are off the carry's path: on a SIMD the output wave's matrix and
// vector work fills the chain wave's waits (one 4-wave block doing both kinds of work:
// 2048-token prefill 108 us; this layout 101; the carry alone, outputs skipped, 90).
// Every wave passes the same sequence of barriers (the checkpoint positions are uniform
// over the block).
// The state stays in the chain waves' registers in the carry's output layout (lane
// (r16, g4) of wave w holds S[i0 + r16][16 nt + 4 g4 + v]), which is also where the
// next carry's accumulator starts from; LDS holds the parts of S_c that the U and output
// products read, in two buffers used alternately (chunk c reads one while S_{c+1} is
// written to the other).  Blocks of one (row, head) unit are spaced 8 apart in launch
// order, which places all its tiles on one of the 8 chiplets and lets them share that
// L2's copy of the chunk operands (W, K^T, P).
// Two tiles per block (TPB = 2) share each wave's W, K^T, Q and P registers and their
// splitting, and run their products interleaved; a block step takes about 1.3 times as
// long as with one tile, so the form pays where the chains outnumber the CUs (rows of
// 2048 tokens, 32 value heads: two rows 206 -> 174 us, four 431 -> 366 us; the 4-prefill
// transaction 572 -> 527 us), and a single such row (256 chains) keeps one tile per block
// on every CU (96 against 113 us).
template <int D, bool W32, int TPB>
__global__ __launch_bounds__(512) void chunk_chain_kernel(ChunkArgs args, int n_units) {
  constexpr int TILES = D / VT / TPB;  // blocks per unit; each holds TPB 16-channel tiles
  static_assert(TILES >= 1, "tiles per block");
  constexpr int NK = CarryOps<D, W32, TPB>::NK;
  constexpr int NT = CarryOps<D, W32, TPB>::NT;
  constexpr int LDS_ = D + 8;     // S part row (bf16): 16-B aligned rows
  constexpr int SPL = VT * LDS_;  // elements per plane of S parts
  constexpr int UPL = VT * LDP;   // elements per plane of U parts
  constexpr size_t UNIT = size_t(D) * D;
  __shared__ __attribute__((aligned(16))) uint16_t sS[2][TPB][3 * SPL];  // S_c in parts: row i, column d
  __shared__ __attribute__((aligned(16))) uint16_t sUc[TPB][3 * UPL];    // (U^T diag(e^{G_n - G})): row i, token s
  __shared__ __attribute__((aligned(16))) uint16_t sUr[TPB][3 * UPL];    // U^T
  __shared__ __attribute__((aligned(16))) uint16_t sUt[TPB][3 * UPL];    // U^T diag(e^{G_j - G}) of a checkpoint

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int r16 = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.x;
  const int k8 = b >> 3;
  const int tile = k8 % TILES;
  const int unit = (k8 / TILES) * 8 + (b & 7);
  if (unit >= n_units) return;  // the whole block
  // unit -> (row, value head): with qk-heads in multiples of 8, the value heads of one
  // qk-head go to one chiplet (unit % 8), as in the prep kernel, and share its L2 copy
  // of their Q and K^T
  int h, row;
  if (args.n_qk % 8 == 0) {
    const int x = unit % 8, j = unit / 8, per = args.n_v / 8;
    row = j / per;
    const int l = j % per;
    h = (x + 8 * (l / args.group)) * args.group + l % args.group;
  } else {
    h = unit % args.n_v;
    row = unit / args.n_v;
  }
  const int i0 = tile * TPB * VT;  // tile j of the block: channels i0 + 16 j .. + 15
  const int L = args.len[row];
  const int nch = (L + C - 1) / C;
  const int n_v = args.n_v;
  const int src = args.src[row], dst = args.dst[row];
  const int tail0 = L - args.n_tail[row];  // first position with a checkpoint
  const int hq = h / args.group;
  auto ws_of = [&](int c) { return Ws<D, W32>(args, args.chunk0[row] + c, h, hq); };
  // parts of S_c for 32-wide d block kb (lane (r16, g4): S_c[i0 + 16 j + r16][32 kb + 8 g4 + e]
  // from tile j's buffer)
  auto s_parts = [&](const uint16_t *buf, int kb) {
    const int col = 32 * kb + 8 * g4;
    if (col < D) return lds_get8<LDS_>(buf, SPL, r16, col);
    const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4v{0u, 0u, 0u, 0u});
    return Parts8{z, z, z};
  };
  // the checkpoint positions of chunk c: p in [max(tail0, c0), c0 + n); each but the
  // row's last takes two barriers (the output waves pass them too)
  auto tail_barriers = [&](int c0, int n) {
    for (int p = max(tail0, c0); p < c0 + n; ++p)
      if (p != L - 1) {
        lds_barrier();
        lds_barrier();
      }
  };

  if (w >= 4) {  // ------------------------------------------------ output waves
    const int t = w - 4;
    lds_barrier();  // the start state's parts
    auto body = [&](int c, const OutOps<D, W32> &f, OutOps<D, W32> &nx) {
      const int cn = min(c + 1, nch - 1);
      const Ws<D, W32> wsn = ws_of(cn);
      const int c0 = c * C;
      const int n = min(C, L - c0);
      const int64_t tok_base = int64_t(args.tok0[row]) + c0;
      floatx4 oq[TPB];
#pragma unroll
      for (int j = 0; j < TPB; ++j) oq[j] = zero4();
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        Parts8 sp[TPB];
#pragma unroll
        for (int j = 0; j < TPB; ++j) sp[j] = s_parts(sS[c & 1][j], kb);
        nx.load_q(wsn, kb, t, lane);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch stays where it is issued
#pragma unroll
        for (int j = 0; j < TPB; ++j) oq[j] = mma3a(oq[j], sp[j], f.q[kb]);  // O^T: rows are channels, columns tokens
      }
      lds_barrier();  // U of all 64 tokens in LDS
      // O^T = S_c Q^T diag(e^G rq) + U^T P^T, lane (r16, g4) holding
      // O[16 t + r16][i0 + 16 j + 4 g4 + 0..3] (one 8-byte store per tile)
      floatx4 op[TPB];
#pragma unroll
      for (int j = 0; j < TPB; ++j) {
        op[j] = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)  // P is zero right of the diagonal: tokens >= 32 only for t >= 2
          if (kb == 0 || t >= 2) op[j] = mma6(op[j], lds_get8<LDP>(sUr[j], UPL, r16, 32 * kb + 8 * g4), f.p[kb]);
      }
      const float egq = f.egq;
      nx.load_p(wsn, t, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (16 * t + r16 < n) {
#pragma unroll
        for (int j = 0; j < TPB; ++j) {
          const uint2 ob = make_uint2(bf16x2_rn(egq * oq[j][0] + op[j][0], egq * oq[j][1] + op[j][1]),
                                      bf16x2_rn(egq * oq[j][2] + op[j][2], egq * oq[j][3] + op[j][3]));
          *reinterpret_cast<uint2 *>(args.o + ((tok_base + 16 * t + r16) * n_v + h) * D + i0 + 16 * j + 4 * g4) = ob;
        }
      }
      tail_barriers(c0, n);
      lds_barrier();  // S_{c+1}'s parts complete; every read of this chunk's U parts done
    };
    OutOps<D, W32> fa, fb;
    fa.load(ws_of(0), t, lane);
    for (int c = 0; c < nch; c += 2) {
      body(c, fa, fb);
      if (c + 1 >= nch) break;
      body(c + 1, fb, fa);
    }
    return;
  }

  // --------------------------------------------------------------- chain waves
  // every wave has all NT column tiles when D / 16 is a multiple of 4 (d = 128)
  auto has_tile = [&](int q) { return (D / 16) % 4 == 0 || w + 4 * q < D / 16; };
  // the start state: registers, and its parts in LDS
  float4 S[TPB][NT];
#pragma unroll
  for (int j = 0; j < TPB; ++j)
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      S[j][q] = zf4();
      if (src >= 0 && has_tile(q))
        S[j][q] = *reinterpret_cast<const float4 *>(args.state_in + (int64_t(src) * n_v + h) * UNIT +
                                                    int64_t(i0 + 16 * j + r16) * D + 16 * (w + 4 * q) + 4 * g4);
    }
  auto put_state = [&](int buf) {
#pragma unroll
    for (int j = 0; j < TPB; ++j)
#pragma unroll
      for (int q = 0; q < NT; ++q)
        if (has_tile(q)) lds_put4<LDS_>(sS[buf][j], SPL, r16, 16 * (w + 4 * q) + 4 * g4, split4(S[j][q]));
  };
  put_state(0);
  lds_barrier();

  auto body = [&](int c, const CarryOps<D, W32, TPB> &f, CarryOps<D, W32, TPB> &nx) {
    const Ws<D, W32> ws = ws_of(c);
    // the next chunk's operands (past the end: the last chunk again, never read)
    const int cn = min(c + 1, nch - 1);
    const Ws<D, W32> wsn = ws_of(cn);
    const int nn = min(C, L - cn * C);
    const int c0 = c * C;
    const int n = min(C, L - c0);

    // A. U = U' - W S_c^T for tokens 16w..16w+15, each tile's channels (two accumulators
    //    interleave the chains; W is split once for all tiles)
    floatx4 ua[TPB], ub[TPB];
#pragma unroll
    for (int j = 0; j < TPB; ++j) ua[j] = ub[j] = zero4();
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      Parts8 sp[TPB];
#pragma unroll
      for (int j = 0; j < TPB; ++j) sp[j] = s_parts(sS[c & 1][j], kb);
      nx.load_a(wsn, kb, w, lane);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch stays where it is issued
      const Parts8 wp = f.w_parts(kb);
#pragma unroll
      for (int j = 0; j < TPB; ++j) {
        if (kb & 1)
          ub[j] = mma6(ub[j], wp, sp[j]);
        else
          ua[j] = mma6(ua[j], wp, sp[j]);
      }
    }
    float4 u[TPB];
#pragma unroll
    for (int j = 0; j < TPB; ++j) {
      ua[j] += ub[j];
      u[j] = make_float4(f.up[j].x - ua[j][0], f.up[j].y - ua[j][1], f.up[j].z - ua[j][2], f.up[j].w - ua[j][3]);
      lds_put4<LDP>(sUc[j], UPL, r16, 16 * w + 4 * g4, split4(mul4(u[j], f.el)));
      lds_put4<LDP>(sUr[j], UPL, r16, 16 * w + 4 * g4, split4(u[j]));
    }
    nx.load_b(wsn, nn, w, lane, tile);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // U of all 64 tokens in LDS

    // B. the carry on the wave's column tiles
    float4 Sn[TPB][NT];
#pragma unroll
    for (int j = 0; j < TPB; ++j) {
      const Parts8 uc0 = lds_get8<LDP>(sUc[j], UPL, r16, 8 * g4), uc1 = lds_get8<LDP>(sUc[j], UPL, r16, 32 + 8 * g4);
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        floatx4 a = {f.e_last * S[j][q].x, f.e_last * S[j][q].y, f.e_last * S[j][q].z, f.e_last * S[j][q].w};
        if (has_tile(q)) {
          a = mma3b(a, f.kt[q][0], uc0);
          a = mma3b(a, f.kt[q][1], uc1);
        }
        Sn[j][q] = make_float4(a[0], a[1], a[2], a[3]);
      }
    }
    // checkpoints at the positions p of this chunk with p >= tail0: slot p - tail0
    const int p_hi = c0 + n;
    for (int p = max(tail0, c0); p < p_hi; ++p) {  // uniform over the block
      float *cdst = args.ckpt + ((int64_t(args.ck_row[row]) * args.ck_slots + (p - tail0)) * n_v + h) * UNIT +
                    int64_t(i0 + r16) * D + 4 * g4;
      if (p == L - 1) {  // the row's last state is the carry's result
#pragma unroll
        for (int j = 0; j < TPB; ++j)
#pragma unroll
          for (int q = 0; q < NT; ++q)
            if (has_tile(q)) store_nt(cdst + 16 * j * D + 16 * (w + 4 * q), Sn[j][q]);
        continue;
      }
      const int jj = p - c0;
      const double Gj = ws.G[jj];
      float sc[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int s = 16 * w + 4 * g4 + v;
        sc[v] = s <= jj ? float(exp(Gj - ws.G[s])) * ws.rk[s] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < TPB; ++j)
        lds_put4<LDP>(sUt[j], UPL, r16, 16 * w + 4 * g4, split4(mul4(u[j], make_float4(sc[0], sc[1], sc[2], sc[3]))));
      lds_barrier();
      const float ej = ws.eG[jj];
#pragma unroll
      for (int j = 0; j < TPB; ++j)
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          if (!has_tile(q)) continue;
          floatx4 a = {ej * S[j][q].x, ej * S[j][q].y, ej * S[j][q].z, ej * S[j][q].w};
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) a = mma3b(a, f.kt[q][kb], lds_get8<LDP>(sUt[j], UPL, r16, 32 * kb + 8 * g4));
          store_nt(cdst + 16 * j * D + 16 * (w + 4 * q), a);
        }
      lds_barrier();  // sUt is rewritten by the next position
    }
#pragma unroll
    for (int j = 0; j < TPB; ++j)
#pragma unroll
      for (int q = 0; q < NT; ++q) S[j][q] = Sn[j][q];
    put_state((c + 1) & 1);
    lds_barrier();  // S_{c+1}'s parts complete; every read of this chunk's U parts done
  };
  // Chunks in pairs with two operand sets: while chunk c runs on one set, chunk c + 1's
  // operands are loaded into the other, spread over the chunk's matrix work.  Every
  // load of chunk c precedes every load of chunk c + 1, so waiting for chunk c's
  // operands (loads complete in issue order) never waits for the next chunk's.  The
  // scheduling barriers after each prefetch group keep the compiler from sinking those
  // loads toward their use a chunk later: a load issued last is one whose wait drains
  // every load before it.
  CarryOps<D, W32, TPB> fa, fb;
  fa.load(ws_of(0), min(C, L), w, lane, tile);
  for (int c = 0; c < nch; c += 2) {
    body(c, fa, fb);
    if (c + 1 >= nch) break;
    body(c + 1, fb, fa);
  }
  if (dst >= 0) {
#pragma unroll
    for (int j = 0; j < TPB; ++j)
#pragma unroll
      for (int q = 0; q < NT; ++q)
        if (has_tile(q))
          store_nt(args.state_out + (int64_t(dst) * n_v + h) * UNIT + int64_t(i0 + 16 * j + r16) * D + 16 * (w + 4 * q) +
                       4 * g4,
                   S[j][q]);
  }
}

template <int D, bool NT>
hipError_t launch_form(const ChunkArgs &args, int n_chunks, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_prep_kernel<D, NT>), dim3(unsigned(n_chunks) * unsigned(args.n_v)), dim3(256), 0, stream,
                     args);
  const int n_units = args.n_rows * args.n_v;
  const int groups = (n_units + 7) / 8;  // units are dealt to the 8 chiplets in groups of 8
  // two 16-channel tiles per block when the chains outnumber the chip's 256 CUs (one
  // chain block per CU)
  constexpr int TPB2 = D % (2 * VT) == 0 ? 2 : 1;
  if (TPB2 == 2 && int64_t(n_units) * (D / VT) > 256)
    hipLaunchKernelGGL((chunk_chain_kernel<D, NT, TPB2>), dim3(unsigned(groups * 8 * (D / VT / TPB2))),
                       dim3(512), 0, stream, args, n_units);
  else
    hipLaunchKernelGGL((chunk_chain_kernel<D, NT, 1>), dim3(unsigned(groups * 8 * (D / VT))), dim3(512), 0, stream,
                       args, n_units);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ChunkArgs &args, int n_chunks, hipStream_t stream) {
  // a streamed workspace (see chunk_ws_streamed and ws_st) holds W in fp32
  return args.ws_streamed ? launch_form<D, true>(args, n_chunks, stream) : launch_form<D, false>(args, n_chunks, stream);
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
