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
// rows in LPR*16-byte contiguous runs (256 B runs at d = 128): coalesced HBM
// reads of the state and writes of every checkpoint.  The two dot products per
// token are a fixed-order in-lane FMA chain followed by a DPP butterfly over the
// LPR lanes, which leaves every lane of the group with bit-identical sums.
// A block stages the window's q, k, v slice and gates in LDS once (one memory
// latency per block instead of one per token), and checkpoints are written with
// non-temporal stores: the traffic is one state read to T checkpoint writes, and
// streaming the writes past the caches is what lets it approach the HBM peak.
//
// Modes (one instantiation each, same per-token code): chain (decode, verify windows
// with or without checkpoints, short transaction rows), replay (each row's accepted
// prefix re-run from the committed state, the result written back: rollback without
// stored states), tree (each window token runs from its parent's state) and delta
// (each step's rank-1 factors stored instead of the state, optionally after folding
// the previous window's accepted prefix into the state).  Raw q/k are normalised in
// the staging lanes when the caller asks for it.
//
// Bit-exactness.  The per-row arithmetic (element ownership within the row's LPR
// lanes, FMA order, butterfly, gate and normalisation code) is the same in every
// mode and both lane layouts (one or two state rows per lane), and does not depend
// on the row's token count, the launch's row count or the grid.  So the checkpoint
// after j+1 verify tokens is bit-identical to j+1 decode launches, a replayed or
// folded commit to the checkpoint it replaces: each computes the same sequence of
// fp32 operations on the same values, and fp32 state round-trips through memory
// exactly ("Native three-step MTP", section "What changed": state-update rounding
// consistent between decode and verification).  Built with -ffp-contract=off;
// every fused multiply-add is an explicit fmaf.
#include <hip/hip_runtime.h>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// fp32 gates: alpha = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b),
// softplus(x) = max(x, 0) + log1p(exp(-|x|)) (no overflow for any x).
__device__ __forceinline__ void eval_gates(float a, float b, float A_log, float dt_bias,
                                           float &alpha, float &beta) {
  const float x = a + dt_bias;
  const float sp = fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
  alpha = expf(-(expf(A_log) * sp));
  beta = 1.0f / (1.0f + expf(-b));
}

// Sum over the LPR (4, 8 or 16) consecutive lanes of a row group with DPP lane
// moves: swap neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), add
// the mirrored half-row (lane i <- 7-i, the other quad's sum), then the mirrored
// row (lane i <- 15-i, the other half-row's sum).  Each step adds two partial sums
// of the same shape, so every lane of the group ends with the same bits.
__device__ __forceinline__ float dpp_add(float p, int ctrl_id) {
  int moved;
  // Every source lane of these patterns lies in the same row, so bound_ctrl never
  // applies; setting it lets the compiler fold the move into the add (v_add_f32_dpp).
  switch (ctrl_id) {
    case 0: moved = __builtin_amdgcn_update_dpp(0, __float_as_int(p), 0xB1, 0xF, 0xF, true); break;
    case 1: moved = __builtin_amdgcn_update_dpp(0, __float_as_int(p), 0x4E, 0xF, 0xF, true); break;
    case 2: moved = __builtin_amdgcn_update_dpp(0, __float_as_int(p), 0x141, 0xF, 0xF, true); break;
    default: moved = __builtin_amdgcn_update_dpp(0, __float_as_int(p), 0x140, 0xF, 0xF, true); break;
  }
  return p + __int_as_float(moved);
}

template <int LPR>
__device__ __forceinline__ float group_sum(float p) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "row groups of 4, 8 or 16 lanes");
  p = dpp_add(p, 0);
  p = dpp_add(p, 1);
  if (LPR >= 8) p = dpp_add(p, 2);
  if (LPR == 16) p = dpp_add(p, 3);
  return p;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// q/k normalisation of the fused input mode: x / sqrt(sum x^2 + eps), q also by
// 1/sqrt(d_k).
constexpr float kNormEps = 1e-6f;
template <int D>
constexpr float inv_sqrt_d() {
  static_assert(D == 16 || D == 128, "head width");
  return D == 16 ? 0.25f : 0.0883883476483184405501f;
}

// Squared norm of a D-vector held as one float4 by each of D/4 consecutive lanes
// (a quad at D = 16, half a wave at D = 128): in-lane chain, DPP butterfly over the
// lane group, then at D = 128 the two 16-lane halves swapped and added.  Every lane
// of the group ends with the same bits, and the result does not depend on where in
// the wave the group sits.
template <int D>
__device__ __forceinline__ float sq_norm(const float4 &x) {
  float p = x.x * x.x;
  p = fmaf(x.y, x.y, p);
  p = fmaf(x.z, x.z, p);
  p = fmaf(x.w, x.w, p);
  if constexpr (D == 16) {
    return group_sum<4>(p);
  } else {
    static_assert(D == 128, "head width");
    p = group_sum<16>(p);
    return p + __shfl_xor(p, 16, 64);
  }
}

// Checkpoints are written once and read at most once (by commit), after the whole
// window: stream them past the caches.
__device__ __forceinline__ void store_nt(float *p, const float (&x)[4]) {
  f32x4 v = {x[0], x[1], x[2], x[3]};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}

// Instantiations: kChain (decode, verify windows, short transaction rows), kReplay
// (gdn_commit_replay: accepted counts on the device, no outputs, no checkpoints), kTree
// (gdn_verify_tree: every window token runs from its parent's state), kDelta
// (gdn_verify_window_delta: each step's rank-1 factors instead of the states) and kSelect
// (gdn_verify_window_select: checkpoints into pool banks, the source slot from a device
// table).  All compile the same per-token arithmetic, so they round identically.
enum Mode { kChain = 0, kReplay = 1, kTree = 2, kDelta = 3, kSelect = 4 };

// STREAM: the launch streams dense states out (checkpoints, a decode's new state, a
// replayed commit).  A block issues its token and state loads at raised wave priority,
// ahead of the arithmetic and stores of older blocks on the same SIMDs, so with several
// rounds of blocks per CU the memory system always holds the next round's reads; and
// each output goes straight to memory from the lane that reduced it, so a block retires
// as soon as its last store is issued.  (Launches that write no dense state measured
// slower in this form.)
// NTLOAD: the state is read with non-temporal loads (each byte is read once per launch).
// Measured on the 16-row launches: in-place decode 15.3 -> 12.4 us, select verify 30.1 ->
// 29.9 us, and the commit that follows a verify runs ~0.4 us faster; the verify with dense
// checkpoints alone measured 29.25 -> 29.45 us, so it keeps plain loads.
template <int D, int LPR, int RPL, int WAVES, int MODE, bool STREAM, bool NTLOAD>
__global__ __launch_bounds__(64 * WAVES) void recurrent_kernel(RecurrentArgs args) {
  if constexpr (STREAM) __builtin_amdgcn_s_setprio(3);
  constexpr bool REPLAY = MODE == kReplay, TREE = MODE == kTree;
  constexpr int NV = D / LPR / 4;                  // float4 per lane per state row
  constexpr int ROWS = WAVES * 64 / LPR * RPL;     // state rows per block
  constexpr int TILES = D / ROWS;                  // blocks per (row, head)
  constexpr int TB = kMaxWindow;                   // every row's tokens are staged at once
  static_assert(NV >= 1 && D % (LPR * 4) == 0 && D % ROWS == 0, "bad tiling");
  constexpr size_t UNIT = size_t(D) * D;
  // The row's tokens' inputs, shared by the block: k and q widened to fp32 once,
  // the block's slice of v, and the two gates.
  __shared__ float4 sK[TB][D / 4], sQ[TB][D / 4];
  __shared__ float sV[TB][ROWS];
  __shared__ float sAlpha[TB], sBeta[TB];
  __shared__ float sKs[TB];          // the factor each key was scaled by (1: none)
  __shared__ uint16_t sO[TB][ROWS];  // outputs, written back coalesced at the end (launches without STREAM)

  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  // a 3-D grid (tile, value head, row): no divisions ahead of the first loads (the 16-row
  // K=3 select verify: 29.69 against 29.83 us with the same blocks numbered in one
  // dimension); blocks are dispatched in the same order either way
  const int tile = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int i_local = (tid / LPR) * RPL;  // first of this lane's RPL state rows in the block
  const int i0 = tile * ROWS + i_local;

  // Every argument the loads ahead of the state need, read up front and pinned in scalar
  // registers: the compiler then issues all of them as one round of scalar loads with a
  // single wait, where it otherwise spread them over three dependent rounds (the 16-row
  // K=3 select verify: 29.26 against 29.63 us; the copy form's verify 28.9 against 29.6,
  // the in-place decode 12.07 against 12.46).
  int ntok = args.ntok[r];
  const int tok0 = args.tok0[r];
  int src = args.src[r];
  const int dst = args.dst[r], ck_first = args.ck_first[r];
  const int ck_row = args.ck_row[r];
  const int n_v = args.n_v, n_qk = args.n_qk, group = args.group;
  const int prev_ntok = MODE == kSelect ? args.prev_ntok[r] : 0;
  const int prev_bank = MODE == kSelect ? args.prev_bank[r] : 0;
  {
    const uint16_t *const qp = args.q, *const kp = args.k, *const vp = args.v;
    const float *const ap = args.a, *const bp = args.b, *const alp = args.A_log, *const dtp = args.dt_bias;
    const void *const tabp = args.src_table, *const paccp = args.prev_accepted, *const sip = args.state_in;
    const int cks = args.ck_slots, nsl = args.n_slots;
    asm volatile("" ::"s"(ntok), "s"(tok0), "s"(src), "s"(dst), "s"(ck_first), "s"(ck_row), "s"(prev_ntok),
                 "s"(prev_bank), "s"(group), "s"(qp), "s"(kp), "s"(vp), "s"(ap), "s"(bp), "s"(alp), "s"(dtp),
                 "s"(tabp), "s"(paccp), "s"(sip), "s"(cks), "s"(nsl), "s"(n_v), "s"(n_qk));
  }
  constexpr bool write_o = !REPLAY;
  // replay: a_r is read first, as a vector load like the select table below, and
  // checked once the state loads are in flight
  int acc_raw = 0;
  if constexpr (REPLAY) {
    int idx = ck_row;
    asm volatile("" : "+v"(idx));
    acc_raw = args.accepted[idx];
  }

  // checkpoint select: the row's source slot is read first, as a vector load (the
  // index is hidden from the compiler's uniformity analysis), so waiting for it later
  // leaves the token loads issued after it in flight
  int sel_raw = 0, pacc_raw = 0;
  if constexpr (MODE == kSelect) {
    int idx = r;
    asm volatile("" : "+v"(idx));
    sel_raw = args.src_table[idx];
    // a pending commit's count; issued unconditionally (from the table itself when there
    // is none) so the number of loads in flight stays fixed for the waits below
    pacc_raw = (args.prev_accepted ? args.prev_accepted : args.src_table)[idx];
  }
  __builtin_amdgcn_sched_barrier(0);  // those loads go out before the division below
  const int hq = h / group;

  // The row's token inputs are loaded before the state: one counter tracks loads in
  // issue order, so the waits that staging needs then leave the state loads in
  // flight, and staging (gates, q/k normalisation, LDS writes) overlaps their latency.
  // Thread x holds float4 column group x % (D/4) of token x / (D/4) of k (and q), the
  // v value at x / ROWS, x % ROWS of the block's slice, and the gate logits of token
  // x.  Every load is issued unconditionally (indexes past the window clamped to its
  // last token, results unused): with a fixed number of loads after each one, the
  // compiler can wait for exactly the ones it needs.
  static_assert(kMaxWindow * (D / 4) <= 64 * WAVES && kMaxWindow * ROWS <= 64 * WAVES,
                "one pass stages a window");
  const int kt = tid / (D / 4), kc = tid % (D / 4);
  const int vt = tid / ROWS, vr = tid % ROWS;
  uint2 kw, qw = make_uint2(0u, 0u);
  {
    const size_t tk = size_t(tok0) + min(kt, ntok - 1);
    kw = reinterpret_cast<const uint2 *>(args.k + (tk * n_qk + hq) * D)[kc];
    if (write_o) qw = reinterpret_cast<const uint2 *>(args.q + (tk * n_qk + hq) * D)[kc];
  }
  const uint32_t vw = args.v[((size_t(tok0) + min(vt, ntok - 1)) * n_v + h) * D + tile * ROWS + vr];
  const size_t tg = size_t(tok0) + min(tid, ntok - 1);
  const float ga = args.a[tg * n_v + h], gb = args.b[tg * n_v + h];
  const float A_log_h = args.A_log[h], dt_bias_h = args.dt_bias[h];
  // every scalar the state address needs is in registers before the wait for the slot:
  // the compiler would otherwise load some of them only once the slot has arrived
  const float *const state_in = args.state_in;
  const int ck_slots = args.ck_slots, n_slots = args.n_slots;
  if constexpr (MODE == kSelect) asm volatile("" ::"s"(state_in), "s"(ck_slots), "s"(n_slots), "s"(prev_ntok),
                                              "s"(prev_bank));
  __builtin_amdgcn_sched_barrier(0);  // keep every token load ahead of the state loads
  // the state is loaded from the selected slot clamped into the pool; the check that it
  // lies outside every bank this launch writes runs after staging, while those loads are
  // in flight -- a refused row leaves before any store
  constexpr bool select = MODE == kSelect;
  int sel_src = select ? __builtin_amdgcn_readfirstlane(sel_raw) : 0;
  // the previous window's commit first: its accepted checkpoint becomes the committed
  // state (and the table entry), exactly as a gdn_commit_select launch before this one;
  // the table store (or the status bit of a count out of range, the entry then kept)
  // waits until the state loads are issued, so no store sits ahead of them
  int pending = 0;  // 1: store the new table entry, 2: flag the row
  if (select) {
    // branch-free, so the row's previous bank and token count (read with the other
    // per-row arguments, above) are not loaded only once the count has arrived
    const int pacc = __builtin_amdgcn_readfirstlane(pacc_raw);
    const bool ok = pacc >= 0 && pacc < prev_ntok;
    const bool fold = args.prev_accepted != nullptr;
    sel_src = fold && ok ? prev_bank * ck_slots + pacc : sel_src;
    pending = fold ? (ok ? 1 : 2) : 0;
  }
  if (select) src = min(max(sel_src, -1), n_slots - 1);

  // the committed state (slot -1: zero; slot 0, which every pool has, is read and
  // discarded, keeping the load unconditional)
  float s[RPL][NV][4];
#pragma unroll
  for (int q = 0; q < RPL; ++q) {
    const float4 *p = reinterpret_cast<const float4 *>(
        state_in + (size_t(max(src, 0)) * n_v + h) * UNIT + size_t(i0 + q) * D);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if constexpr (NTLOAD) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + sub + LPR * j));
        s[q][j][0] = x[0]; s[q][j][1] = x[1]; s[q][j][2] = x[2]; s[q][j][3] = x[3];
      } else {
        const float4 x = p[sub + LPR * j];
        s[q][j][0] = x.x; s[q][j][1] = x.y; s[q][j][2] = x.z; s[q][j][3] = x.w;
      }
    }
  }
  if constexpr (STREAM) __builtin_amdgcn_s_setprio(0);  // every load of the block is issued
  if (select && pending != 0 && tile == 0 && h == 0 && tid == 0) {
    if (pending == 1) args.src_table[r] = sel_src;
    else atomicOr(args.status + (r >> 5), 1u << (r & 31));
  }
  if constexpr (REPLAY) {
    // Replay of the accepted prefix: the bonus token and a_r drafts, the same
    // sequence of operations as the first a_r + 1 tokens of the window, so the
    // state it leaves is bit-identical to that window's checkpoint slot a_r.  The
    // token loads above are clamped to the whole window; the empty asm keeps the
    // compiler from sinking the state loads below this exit (4 % on the commit).
    asm volatile("" ::: "memory");
    const int acc = __builtin_amdgcn_readfirstlane(acc_raw);
    if (acc < 0 || acc >= ntok) {
      if (tile == 0 && h == 0 && tid == 0) atomicOr(args.status + (ck_row >> 5), 1u << (ck_row & 31));
      return;  // the whole block leaves before any store or barrier
    }
    ntok = acc + 1;
  }
  if constexpr (MODE == kDelta) {
    if (args.fold_k) {
      // commit the previous window first: fold its accepted prefix into the state
      // (the fold kernel's operation sequence) and publish it in place
      const int acc = args.fold_accepted[ck_row];
      if (acc < 0 || acc >= args.fold_ntok[r]) {
        if (tile == 0 && h == 0 && tid == 0) atomicOr(args.status + (ck_row >> 5), 1u << (ck_row & 31));
        return;  // the whole block leaves before any barrier
      }
      // the whole window's factors and keys in one round of loads (tokens past the
      // window clamped to its last one, never applied)
      float fa[TB], fs[TB], fc[TB][RPL];
      uint2 fk[TB][NV];
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const int tt = min(t, args.fold_ntok[r] - 1);
        const float *dl = args.fold_delta + ((size_t(ck_row) * args.ck_slots + tt) * n_v + h) * (D + 4);
        const uint2 *kr = reinterpret_cast<const uint2 *>(
            args.fold_k + ((size_t(args.fold_tok0[r]) + tt) * n_qk + hq) * D);
        fa[t] = dl[D];
        fs[t] = dl[D + 1];
#pragma unroll
        for (int q = 0; q < RPL; ++q) fc[t][q] = dl[i0 + q];
#pragma unroll
        for (int j = 0; j < NV; ++j) fk[t][j] = kr[sub + LPR * j];
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t > acc) break;
#pragma unroll
        for (int q = 0; q < RPL; ++q)
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            s[q][j][0] = fmaf(fc[t][q], bf16_lo(fk[t][j].x) * fs[t], fa[t] * s[q][j][0]);
            s[q][j][1] = fmaf(fc[t][q], bf16_hi(fk[t][j].x) * fs[t], fa[t] * s[q][j][1]);
            s[q][j][2] = fmaf(fc[t][q], bf16_lo(fk[t][j].y) * fs[t], fa[t] * s[q][j][2]);
            s[q][j][3] = fmaf(fc[t][q], bf16_hi(fk[t][j].y) * fs[t], fa[t] * s[q][j][3]);
          }
      }
#pragma unroll
      for (int q = 0; q < RPL; ++q) {
        float4 *p = reinterpret_cast<float4 *>(args.state_out + (size_t(src) * n_v + h) * UNIT +
                                               size_t(i0 + q) * D);
#pragma unroll
        for (int j = 0; j < NV; ++j) p[sub + LPR * j] = make_float4(s[q][j][0], s[q][j][1], s[q][j][2], s[q][j][3]);
      }
    }
  }

  // stage the window in LDS; with raw q/k the D/4 threads of a token first reduce its
  // squared norm among themselves and scale (every lane takes part, those past the
  // window with zeros)
  {
    float4 kf = make_float4(bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y));
    float4 qf = make_float4(bf16_lo(qw.x), bf16_hi(qw.x), bf16_lo(qw.y), bf16_hi(qw.y));
    float fk = 1.0f;
    if (args.qk_norm) {
      fk = 1.0f / sqrtf(sq_norm<D>(kf) + kNormEps);
      kf = make_float4(kf.x * fk, kf.y * fk, kf.z * fk, kf.w * fk);
      if (write_o) {
        const float fq = (1.0f / sqrtf(sq_norm<D>(qf) + kNormEps)) * inv_sqrt_d<D>();
        qf = make_float4(qf.x * fq, qf.y * fq, qf.z * fq, qf.w * fq);
      }
    }
    if (kt < ntok) {
      sK[kt][kc] = kf;
      if (write_o) sQ[kt][kc] = qf;
      if (kc == 0) sKs[kt] = fk;
    }
  }
  if (vt < ntok) sV[vt][vr] = __uint_as_float(vw << 16);
  if (tid < ntok) eval_gates(ga, gb, A_log_h, dt_bias_h, sAlpha[tid], sBeta[tid]);
  lds_barrier();
  if (select) {
    // The selected slot must lie in the pool and outside every bank this launch writes.
    // Checked here, after staging and before any store: its one load (lane j reads row
    // j's bank from the argument block) completes with the state loads issued before it,
    // which the first step waits for anyway (checked before staging, as 64 scalar
    // compares, it delayed every block: 31.3 against 30.1 us on the 16-row K=3 verify).
    const int ln = tid & 63;
    const int bank_j = ln < args.n_rows ? args.ck_row[ln] : -1;
    const int sel_bank = sel_src >= 0 ? sel_src / args.ck_slots : -2;
    const bool bad = sel_src < -1 || sel_src >= args.n_slots || __ballot(bank_j == sel_bank) != 0ull;
    if (bad) {
      if (tile == 0 && h == 0 && tid == 0) atomicOr(args.status + (r >> 5), 1u << (r & 31));
      return;  // the whole block leaves before any store (its one barrier is behind it)
    }
  }
  if (src < 0) {  // after staging: replacing a register whose load is in flight would wait for it
#pragma unroll
    for (int q = 0; q < RPL; ++q)
#pragma unroll
      for (int j = 0; j < NV; ++j) s[q][j][0] = s[q][j][1] = s[q][j][2] = s[q][j][3] = 0.0f;
  }

  // Token t of the window applied to state rows st, with its output and checkpoint.
  auto step = [&](int t, float (&st)[RPL][NV][4]) {
    const float alpha = sAlpha[t], beta = sBeta[t];
    if (MODE == kDelta && tile == 0 && tid == 0)
      *reinterpret_cast<float2 *>(args.delta + ((size_t(ck_row) * args.ck_slots + t) * n_v + h) * (D + 4) + D) =
          make_float2(alpha, sKs[t]);
    float kk[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const float4 kw = sK[t][sub + LPR * j];
      kk[j][0] = kw.x; kk[j][1] = kw.y; kk[j][2] = kw.z; kk[j][3] = kw.w;
    }
#pragma unroll
    for (int q = 0; q < RPL; ++q) {
      const float vi = sV[t][i_local + q];
      // u = S[i,:] . k
      float p = 0.0f;
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) p = fmaf(st[q][j][e], kk[j][e], p);
      const float u = group_sum<LPR>(p);
      // S[i,:] <- alpha S[i,:] + beta (v_i - alpha u) k
      const float c = beta * (vi - alpha * u);
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[q][j][e] = fmaf(c, kk[j][e], alpha * st[q][j][e]);
      if (MODE == kDelta && sub == 0)  // the step's factors: c_i, and alpha once per head
        args.delta[((size_t(ck_row) * args.ck_slots + t) * n_v + h) * (D + 4) + i0 + q] = c;
      if (write_o) {
        // o_i = S[i,:] . q
        float po = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const float4 qw = sQ[t][sub + LPR * j];
          po = fmaf(st[q][j][0], qw.x, po);
          po = fmaf(st[q][j][1], qw.y, po);
          po = fmaf(st[q][j][2], qw.z, po);
          po = fmaf(st[q][j][3], qw.w, po);
        }
        const float oi = group_sum<LPR>(po);
        if (sub == 0) {
          if constexpr (STREAM)
            args.o[((size_t(tok0) + t) * n_v + h) * D + i0 + q] = to_bf16(oi);
          else
            sO[t][i_local + q] = to_bf16(oi);
        }
      }
      if (!REPLAY && t >= ck_first) {
        float *cp = args.ckpt + ((size_t(ck_row) * args.ck_slots + (t - ck_first)) * n_v + h) * UNIT +
                    size_t(i0 + q) * D;
#pragma unroll
        for (int j = 0; j < NV; ++j) store_nt(cp + 4 * (sub + LPR * j), st[q][j]);
      }
    }
  };
  auto copy_state = [&](float (&to)[RPL][NV][4], const float (&from)[RPL][NV][4]) {
#pragma unroll
    for (int q = 0; q < RPL; ++q)
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) to[q][j][e] = from[q][j][e];
  };

  if constexpr (TREE) {
    // node states stay in registers (indexed by constants only); token t starts
    // from its parent's state, or from the committed state s
    float node[TB][RPL][NV][4];
    const uint32_t tree = args.tree[r];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t >= ntok) break;
      const int par = int((tree >> (8 * t)) & 0xFFu) - 1;
      float cur[RPL][NV][4];
      copy_state(cur, s);
#pragma unroll
      for (int k = 0; k < t; ++k)
        if (par == k) copy_state(cur, node[k]);
      step(t, cur);
      copy_state(node[t], cur);
    }
  } else {
#pragma unroll 1
    for (int t = 0; t < ntok; ++t) step(t, s);
  }
  if (write_o && !STREAM) {
    lds_barrier();  // every output of the block is in sO
    for (int x = tid; x < ntok * ROWS; x += 64 * WAVES) {
      const int t = x / ROWS, rr = x % ROWS;
      args.o[((size_t(tok0) + t) * n_v + h) * D + tile * ROWS + rr] = sO[t][rr];
    }
  }

  if (dst >= 0) {
    // A new state bound for another slot is streamed past the caches like a checkpoint;
    // one written over the state just read is stored plainly (measured on the 16-row
    // decode with cached state loads: out of place 12.95 -> 11.95 us with non-temporal
    // stores, in place 15.25 plain against 15.9 non-temporal).
    const bool stream_out = dst != src;
#pragma unroll
    for (int q = 0; q < RPL; ++q) {
      float *p = args.state_out + (size_t(dst) * n_v + h) * UNIT + size_t(i0 + q) * D;
      if (stream_out) {
#pragma unroll
        for (int j = 0; j < NV; ++j) store_nt(p + 4 * (sub + LPR * j), s[q][j]);
      } else {
#pragma unroll
        for (int j = 0; j < NV; ++j)
          reinterpret_cast<float4 *>(p)[sub + LPR * j] = make_float4(s[q][j][0], s[q][j][1], s[q][j][2], s[q][j][3]);
      }
    }
  }
}

}  // namespace

template <int D, int LPR, int RPL, int WAVES, int MODE, bool STREAM, bool NTLOAD = false>
static void launch_one(const RecurrentArgs &args, hipStream_t stream) {
  constexpr int TILES = D / (WAVES * 64 / LPR * RPL);
  const dim3 grid(TILES, unsigned(args.n_v), unsigned(args.n_rows));
  hipLaunchKernelGGL((recurrent_kernel<D, LPR, RPL, WAVES, MODE, STREAM, NTLOAD>), grid, dim3(64 * WAVES), 0, stream,
                     args);
}

template <int D, int LPR, int RPL, int WAVES>
static void launch_d(const RecurrentArgs &args, hipStream_t stream) {
  // dense states streamed out: checkpoints, or a row's new state written to its slot
  bool writes_state = args.ckpt != nullptr;
  for (int r = 0; r < args.n_rows; ++r) writes_state |= args.dst[r] >= 0;
  if (args.accepted)
    launch_one<D, LPR, RPL, WAVES, kReplay, true, true>(args, stream);
  else if (args.delta)
    launch_one<D, LPR, RPL, WAVES, kDelta, false>(args, stream);
  else if constexpr (RPL == 1) {  // trees always store checkpoints: one lane layout
    if (args.tree_mode)
      launch_one<D, LPR, RPL, WAVES, kTree, true>(args, stream);
    else if (args.src_table)
      launch_one<D, LPR, RPL, WAVES, kSelect, true, true>(args, stream);
    else if (args.ckpt)
      launch_one<D, LPR, RPL, WAVES, kChain, true>(args, stream);
    else if (writes_state)  // decode: the new state goes to a slot
      launch_one<D, LPR, RPL, WAVES, kChain, true, true>(args, stream);
    else
      launch_one<D, LPR, RPL, WAVES, kChain, false>(args, stream);
  } else if (args.src_table)
    launch_one<D, LPR, RPL, WAVES, kSelect, true, true>(args, stream);
  else if (args.ckpt)
    launch_one<D, LPR, RPL, WAVES, kChain, true>(args, stream);
  else if (writes_state)
    launch_one<D, LPR, RPL, WAVES, kChain, true, true>(args, stream);
  else
    launch_one<D, LPR, RPL, WAVES, kChain, false>(args, stream);
}

hipError_t launch_recurrent(const RecurrentArgs &args, int d, hipStream_t stream) {
  if (args.n_rows <= 0) return hipSuccess;
  if (args.n_rows > kRowsPerLaunch) return hipErrorInvalidValue;
  for (int r = 0; r < args.n_rows; ++r)  // the kernel stages a row's tokens in fixed LDS arrays
    if (args.ntok[r] < 1 || args.ntok[r] > kMaxWindow) return hipErrorInvalidValue;
  // replay writes neither outputs nor checkpoints; every other call writes outputs
  if (args.accepted ? (args.o || args.ckpt || !args.status || args.tree_mode || args.delta) : !args.o)
    return hipErrorInvalidValue;
  if (args.delta && (args.ckpt || args.tree_mode)) return hipErrorInvalidValue;
  // checkpoint select: chain windows into the pool, all rows of the call in this launch
  if (args.src_table && (args.accepted || args.delta || args.tree_mode || !args.status || !args.ckpt ||
                         args.n_slots < 1))
    return hipErrorInvalidValue;
  if (args.fold_k) {
    if (!args.delta || !args.fold_delta || !args.fold_accepted || !args.status || !args.state_out)
      return hipErrorInvalidValue;
    for (int r = 0; r < args.n_rows; ++r)
      if (args.src[r] < 0 || args.fold_ntok[r] < 1 || args.fold_ntok[r] > kMaxWindow) return hipErrorInvalidValue;
  }
  if (args.tree_mode)  // parents precede their children; byte 0 is the committed state
    for (int r = 0; r < args.n_rows; ++r)
      for (int t = 0; t < args.ntok[r]; ++t)
        if (int((args.tree[r] >> (8 * t)) & 0xFFu) > t) return hipErrorInvalidValue;
  if (d == 128) {
    // A launch that stores no dense checkpoints moves little data per block and waits
    // mostly on its state loads; with two rounds of blocks or more, two state rows per
    // lane halve the block count (that wait is paid once) and double the loads each lane
    // has in flight.  Each state row keeps its 16 lanes, columns and butterfly, so every
    // result is bit-identical in both layouts.
    // Otherwise (checkpoints, dense or into pool banks) one row per lane in 4-wave
    // blocks: smaller blocks turn over more often, which keeps each CU's loads and
    // stores interleaved (the 16-row K=3 select verify: 31.2 us with two rows per lane
    // in 8-wave blocks, 29.8 with one).
    if (!args.ckpt && !args.tree_mode && int64_t(args.n_rows) * args.n_v >= 512)
      launch_d<128, 16, 2, 8>(args, stream);
    else
      launch_d<128, 16, 1, 4>(args, stream);
  } else if (d == 16)
    launch_d<16, 4, 1, 1>(args, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdn
