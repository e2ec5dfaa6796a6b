// gdn_internal.h -- launch interface between the C-ABI layer (gdn_api.cpp) and
// the HIP kernels.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Rows per kernel launch: per-row metadata travels in the kernel argument
// block (validated on the host, read by the kernel from scalar registers), so a
// call with more rows is split into several launches on the same stream.
constexpr int kRowsPerLaunch = 64;

// Longest row the recurrent kernel runs: a verify window of k_max + 1 <= 4 tokens
// (decode rows have 1; longer transaction rows take the chunked path).
constexpr int kMaxWindow = 4;

// Recurrent (token-by-token) kernel shared by decode, verify and the short rows
// of a transaction.  Row r of the launch runs 1 <= ntok[r] <= kMaxWindow tokens starting at packed
// token tok0[r] from pool slot src[r] (-1: zero state); the state after token t
// is stored to slot t - ck_first[r] of checkpoint row ck_row[r] when
// t >= ck_first[r]; the final
// state goes to pool slot dst[r] when dst[r] >= 0.
struct RecurrentArgs {
  const uint16_t *q, *k, *v;        // bf16 bits
  const float *a, *b, *A_log, *dt_bias;
  const float *state_in;            // pool (read)
  float *state_out;                 // pool (final-state write); may alias state_in
  float *ckpt;                      // checkpoint buffer of the whole call (may be null: none stored)
  uint16_t *o;                      // bf16 bits (may be null: outputs not written)
  // Replay (may be null): row r runs only its first accepted[ck_row[r]] + 1 tokens,
  // read on the device; a count outside [0, ntok[r]) leaves the row untouched and
  // sets bit ck_row[r] of status.
  const int32_t *accepted;
  uint32_t *status;
  // Tree windows (tree_mode != 0): byte t of tree[r] is the parent of window token t
  // plus one (0: the committed state); token t then runs from its parent's state.
  int32_t tree_mode;
  uint32_t tree[kRowsPerLaunch];
  // Delta checkpoints (may be null): the rank-1 factors of every window step instead
  // of the states, laid out as delta_row_floats below.
  float *delta;
  // Pending fold (delta mode, may be null): before its window, row r folds tokens
  // 0..fold_accepted[ck_row[r]] of the previous window (fold_ntok[r] tokens at packed
  // token fold_tok0[r] of fold_k, factors in fold_delta) into its source state and
  // writes the result back to slot src[r]; a count outside [0, fold_ntok[r]) leaves
  // the row untouched (no fold, no window) and sets bit ck_row[r] of status.
  const uint16_t *fold_k;
  const float *fold_delta;
  const int32_t *fold_accepted;
  int32_t fold_tok0[kRowsPerLaunch];
  int32_t fold_ntok[kRowsPerLaunch];
  int32_t n_qk, n_v, group;         // heads; group = n_v / n_qk
  int32_t ck_slots;                 // k_max + 1
  int32_t n_rows;                   // rows in this launch
  int32_t tok0[kRowsPerLaunch];
  int32_t ntok[kRowsPerLaunch];
  int32_t src[kRowsPerLaunch];
  int32_t dst[kRowsPerLaunch];
  int32_t ck_first[kRowsPerLaunch];
  int32_t ck_row[kRowsPerLaunch];   // checkpoint row (index of the row in the call)
  int32_t qk_norm;                  // GDN_QK_L2NORM: normalise q and k in the kernel
  // Checkpoint select (may be null): the launch holds every row of the call (row r of
  // the launch is row r of the call), checkpoints go to pool slots ck_row[r] * ck_slots
  // + j (ckpt == state_out == the pool, ck_row = the bank), and row r's source slot is
  // src_table[r] on the device.  A source outside [-1, n_slots) or inside any row's bank
  // leaves the row untouched and sets bit r of status.
  int32_t *src_table;
  int32_t n_slots;
  // Pending select commit (checkpoint select only, may be null): row r first commits the
  // previous window -- slot prev_bank[r] * ck_slots + prev_accepted[r] (device) when that
  // count lies in [0, prev_ntok[r]), written to src_table[r] and used as the source; a
  // count outside that range leaves src_table[r] as it was (the window then runs from it)
  // and sets bit r of status.
  const int32_t *prev_accepted;
  int32_t prev_bank[kRowsPerLaunch];
  int32_t prev_ntok[kRowsPerLaunch];
};

// Commit: row r copies checkpoint slot accepted[r] of its ckpt row to pool slot
// dst[r] if 0 <= accepted[r] < ntok[r], else sets bit row_base+r of status.
struct CommitArgs {
  const float *ckpt;                // checkpoint rows of this launch
  float *pool;
  const int32_t *accepted;          // device, this launch's rows
  uint32_t *status;                 // device, whole call
  int64_t row_floats;               // H_v * d_v * d_k
  int32_t ck_slots;
  int32_t n_rows;
  int32_t row_base;                 // index of this launch's first row in the call
  int32_t ntok[kRowsPerLaunch];
  int32_t dst[kRowsPerLaunch];
};

// Delta checkpoint of one (call row r, window token t, value head h): d + 4 floats at
// ((r * ck_slots + t) * n_v + h) * (d + 4): c[0..d), c_i = beta_t (v_t[i] - alpha_t
// u_i), alpha_t at [d] and the key's scale factor ks_t at [d + 1] (1 unless q/k are
// normalised in the kernel; the last 2 floats pad rows to 16 bytes).  The step is
// S_t[i][d'] = fmaf(c_i, k_t[d'] * ks_t, alpha_t S_{t-1}[i][d']) for every element.
constexpr int delta_row_floats(int d) { return d + 4; }

// Fold commit: row r of the launch applies window tokens 0..accepted[row_base + r]
// of its delta checkpoints to the state of slot src[r] (-1: zero) and writes slot
// dst[r]; an accepted count outside [0, ntok[r]) leaves the row untouched and sets
// its status bit.
struct FoldArgs {
  const uint16_t *k;                // bf16 bits, packed window tokens
  const float *delta;               // delta checkpoints of the whole call
  const float *pool_in;
  float *pool_out;
  const int32_t *accepted;          // device, whole call
  uint32_t *status;                 // device, whole call
  int32_t n_qk, n_v, group, ck_slots;
  int32_t n_rows;
  int32_t row_base;
  int32_t tok0[kRowsPerLaunch];
  int32_t ntok[kRowsPerLaunch];
  int32_t src[kRowsPerLaunch];
  int32_t dst[kRowsPerLaunch];
};

// Chunked prefill (chunk = 64 tokens).  Launch-local row r owns chunks
// [chunk_start[r], chunk_start[r] + ceil(len[r] / 64)) of the prep grid and
// workspace chunks starting at chunk0[r] (numbered over the whole call); its
// tail checkpoint j (j < n_tail[r]) is the state after len[r] - n_tail[r] + j + 1
// tokens, stored to checkpoint row ck_row[r].
constexpr int kChunk = 64;

// Workspace floats per (chunk, value head), the chain kernel's operands in 1-KiB
// fragment blocks: W in three bf16 parts [4][d/32][3] blocks (w32: fp32 [4][d/32] blocks
// of 2 KiB), the six nonzero blocks of P in three bf16 parts [6][3], U' [d/16][4] blocks
// of 256 fp32 each, then the 64 fp64 prefix sums of the log-decay and four 64-float
// factor vectors.
constexpr int64_t chunk_ws_unit_floats(int d, bool w32) {
  const int64_t nk = d >= 32 ? d / 32 : 1, nt = d / 16;
  return (w32 ? 2048 : 3072) * nk + 4608 + 1024 * nt + 2 * kChunk + 4 * kChunk;
}
// Workspace floats per (chunk, qk-head), after all the value-head units: Q [4][d/32] and
// K^T [d/16][2] fragment blocks, which the value heads sharing the qk-head read alike.
constexpr int64_t chunk_ws_qk_floats(int d) {
  const int64_t nk = d >= 32 ? d / 32 : 1, nt = d / 16;
  return 1024 * nk + 512 * nt;
}
constexpr int64_t chunk_ws_floats(int64_t chunks, int n_v, int n_qk, int d, bool w32) {
  return chunks * (n_v * chunk_ws_unit_floats(d, w32) + n_qk * chunk_ws_qk_floats(d));
}

// A call's workspace is streamed: written past the caches, with W in fp32 (the chain
// kernel forms its parts), when with W in parts it would exceed 160 MiB.  Such a call is
// bound by the workspace traffic, which fp32 W cuts by 14 % (d = 128, two value heads
// per qk-head); a smaller one is read back from the last-level cache, and there the
// parts, formed once by the prep kernel, keep that work off the chain's serial path.
constexpr int64_t kStreamedWsBytes = int64_t(160) << 20;
constexpr bool chunk_ws_streamed(int64_t chunks, int n_v, int n_qk, int d) {
  return chunk_ws_floats(chunks, n_v, n_qk, d, false) * 4 > kStreamedWsBytes;
}

struct ChunkArgs {
  const uint16_t *q, *k, *v;
  const float *a, *b, *A_log, *dt_bias;
  const float *state_in;
  float *state_out;
  float *ckpt;
  uint16_t *o;
  float *ws;                        // the (chunk, value head) units
  float *ws_qk;                     // the (chunk, qk-head) units, after all the others
  int32_t n_qk, n_v, group;
  int32_t ck_slots;
  int32_t n_rows;
  int32_t tok0[kRowsPerLaunch];
  int32_t len[kRowsPerLaunch];
  int32_t chunk_start[kRowsPerLaunch];
  int32_t chunk0[kRowsPerLaunch];
  int32_t src[kRowsPerLaunch];
  int32_t dst[kRowsPerLaunch];
  int32_t n_tail[kRowsPerLaunch];
  int32_t ck_row[kRowsPerLaunch];
  int32_t qk_norm;                  // GDN_QK_L2NORM: normalise q and k in the kernels
  int32_t ws_streamed;              // the call's workspace form (chunk_ws_streamed over all its chunks)
};

// Checkpoint select commit: slot_table[r] = bank[r] * ck_slots + accepted[r] when
// 0 <= accepted[r] < ntok[r], else the entry is left and bit r of status is set.
struct SelectArgs {
  const int32_t *accepted;          // device
  int32_t *slot_table;              // device
  uint32_t *status;                 // device
  int32_t ck_slots;
  int32_t n_rows;                   // <= kRowsPerLaunch
  int32_t ntok[kRowsPerLaunch];
  int32_t bank[kRowsPerLaunch];
};

hipError_t launch_recurrent(const RecurrentArgs &args, int d, hipStream_t stream);
hipError_t launch_select(const SelectArgs &args, hipStream_t stream);
hipError_t launch_chunked(const ChunkArgs &args, int d, int n_chunks, hipStream_t stream);
// The current GPU's copy of the static chunked workspace (GDN_STATIC_WS_BYTES): its
// device address, looked up once per GPU and kept.
hipError_t static_workspace(void **ptr, size_t *bytes);
hipError_t launch_commit(const CommitArgs &args, hipStream_t stream);
hipError_t launch_fold(const FoldArgs &args, int d, hipStream_t stream);

}  // namespace gdn
