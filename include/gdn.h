/*
 * gdn.h -- C ABI of libgdn: the gated-delta-rule (GatedDeltaNet) recurrent-state
 * hot path of K-draft multi-token-prediction speculative decoding, on one AMD
 * Instinct MI355X (gfx950).
 *
 * The operation.  Per (row r, value head h), with the q/k head hq = h / (H_v/H_qk)
 * (contiguous groups of value heads share one q/k head), and S a d_v x d_k fp32
 * matrix (row-major, k contiguous):
 *     alpha_t = exp(-exp(A_log[h]) * softplus(a_t + dt_bias[h])),  beta_t = sigmoid(b_t)
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 * This is the gated delta rule (Yang, Kautz & Hatamizadeh, "Gated Delta Networks:
 * Improving Mamba2 with Delta Rule", ICLR 2025).  Gates are evaluated in fp32 and
 * the state update is rounded identically in decode and in verification ("Native
 * three-step MTP", section "What changed").  Verification publishes the state
 * after every window token so that a rejected draft is undone by restoring the
 * checkpoint at the accepted length; a long prefill in the same ragged batch goes
 * through a chunked form that still publishes the checkpoints its row asks for
 * (onnxruntime-genai pull request "Run chained MTP drafting in the batch Engine",
 * sections "Correctness fix" and "Rollback fix and corrected quality disposition").
 *
 * Conventions shared by every call.
 *  - Supported shapes: d_k == d_v in {16, 128}; H_v a multiple of H_qk and at most
 *    GDN_MAX_V_HEADS; 0 <= k_max <= 3.  Anything else returns GDN_E_UNSUPPORTED.
 *  - Rows are packed in order; row r owns tokens [cu_r, cu_r + L_r) of the packed
 *    token dimension N, cu_r = L_0 + ... + L_{r-1}; a row's tokens are in time order.
 *  - Device arrays (caller-allocated, caller-owned; the library allocates nothing):
 *      q, k   bf16 bits [N][H_qk][d_k]        v    bf16 bits [N][H_v][d_v]
 *      a, b   fp32 [N][H_v] (gate logits)     A_log, dt_bias fp32 [H_v]
 *      o      bf16 bits [N][H_v][d_v]         (round to nearest even)
 *      state_pool fp32 [n_slots][H_v][d_v][d_k]   committed states, one slot per row
 *      ckpt   fp32 [n_rows][k_max+1][H_v][d_v][d_k]  checkpoint slot j of row r
 *  - Host arrays (validated before anything is launched): per-row token counts,
 *    slot indices and checkpoint counts.  A source slot of -1 means the zero state.
 *    A call with rows needs n_slots >= 1 (GDN_E_RANGE otherwise): the kernels read
 *    slot 0 in place of a zero source and discard it.
 *  - Alignment: q, k, v, o, state_pool, ckpt and the workspace 16 B; a, b, A_log,
 *    dt_bias 4 B.  Otherwise GDN_E_ALIGN.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronises the host.  Ordering across streams (publish a
 *    prefill before a dependent verify, "Native three-step MTP", section "What
 *    changed") is the caller's, through events.
 *  - Fail closed: every argument is checked before the first launch, so on any error
 *    code but GDN_E_HIP nothing is launched and nothing is written.  GDN_E_HIP is the
 *    runtime refusing a launch; a call that launches several kernels (more than 64
 *    rows, or a chunked prefill) may have run the launches before it.
 *  - The library holds no mutable global state but one table: the per-GPU address of
 *    the static workspace of gdn_chunked_prefill_with_checkpoints_static, filled once
 *    per GPU under a lock.  Calls are thread-safe, except that calls of that entry point
 *    overlapping on one GPU share its workspace (see there).
 *
 * Interface notes (choices in the signatures below, with their reasons).
 *  - Token offsets are not passed: rows are packed in order, so row r's first token is
 *    the sum of the host token counts before it, which the library computes while it
 *    validates them (a separate device offset array could disagree with the counts).
 *  - gdn_commit_accepted takes the window lengths as a host array, like every other
 *    per-row count: they were fixed when the window was launched, so only the accepted
 *    counts need to stay on the device.
 *  - gdn_chunked_workspace_bytes takes the per-row token counts, not a token total: the
 *    workspace holds one unit per (chunk, value head) and a smaller one per (chunk,
 *    qk-head), and chunks never span rows.
 *  - gdn_plan_transaction returns one route per row: the plan depends on row lengths
 *    only (every row gets its checkpoints on either route), so no checkpoint counts and
 *    no plan structure are needed.
 *  - Streams are passed as void * (a hipStream_t), so the header needs no HIP header.
 *  - gdn_dims carries a flags word (GDN_QK_L2NORM).
 *  - Beyond decode, verification, the copy commit, the chunked prefill and the
 *    transaction planner, the library offers other rollback forms (replay, rank-1
 *    factors, checkpoint select), token-tree verification and a chunked prefill that
 *    allocates nothing; each is described at its declaration.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_VERSION 7
#define GDN_MAX_K 3 /* largest k_max: at most 4 checkpoint slots per row */
#define GDN_MAX_V_HEADS 1024 /* largest H_v */

typedef struct gdn_dims {
  int32_t n_qk_heads; /* H_qk */
  int32_t n_v_heads;  /* H_v, a multiple of H_qk */
  int32_t d_k;        /* key / query width */
  int32_t d_v;        /* value width (== d_k) */
  int32_t k_max;      /* largest draft count per row; checkpoint slots per row = k_max + 1 */
  uint32_t flags;     /* 0, or GDN_QK_L2NORM; other bits: GDN_E_UNSUPPORTED */
} gdn_dims;

/*
 * GDN_QK_L2NORM -- fused input side.  q and k arrive as raw projections; every
 * call that reads them (decode, verification in every mode, replay, chunked
 * prefill, transactions) first normalises each (token, q/k head) vector:
 *     k_hat = k / sqrt(sum_j k_j^2 + 1e-6),  q_hat = q / sqrt(sum_j q_j^2 + 1e-6) / sqrt(d_k)
 * in fp32 from the bf16 inputs (the normalised values are not rounded back to
 * bf16), and runs the rule on k_hat, q_hat (the gated delta rule normalises its
 * queries and keys, Yang, Kautz & Hatamizadeh, ICLR 2025; the pages are silent).
 * The recurrent calls normalise a token identically whatever its window position,
 * so the decode/verify bit-consistency holds in this mode too.  Without the flag q
 * and k are taken as already normalised and scaled.
 */
#define GDN_QK_L2NORM 1u

enum {
  GDN_OK = 0,
  GDN_E_NULL = -1,        /* a required pointer is NULL */
  GDN_E_UNSUPPORTED = -2, /* shape outside the supported set */
  GDN_E_RANGE = -3,       /* a token count, slot index or checkpoint count is out of range */
  GDN_E_ALIAS = -4,       /* two rows write one slot, a row writes a slot another reads, or buffers overlap */
  GDN_E_ALIGN = -5,       /* a device pointer is misaligned */
  GDN_E_WORKSPACE = -6,   /* workspace missing or too small */
  GDN_E_HIP = -7          /* the HIP runtime refused a launch */
};

/* Routes chosen by gdn_plan_transaction. */
enum { GDN_ROUTE_RECURRENT = 0, GDN_ROUTE_CHUNKED = 1 };

/*
 * gdn_decode_step -- one token per row (token r belongs to row r, N = n_rows).
 * Reads the state of slot src_slot[r] (-1: zero state), applies the rule once,
 * writes o[r] and the new state to slot dst_slot[r] (== src_slot[r] updates in
 * place).  Decode is the single-token case of the verify window below: both run
 * one device routine, so verify checkpoint j is bit-identical to j+1 decode calls
 * (decode fixes the rounding that verification must reproduce: "Native three-step
 * MTP", section "What changed").  In place or into another slot, the bits are the
 * same; a new state bound for another slot is streamed past the caches, which
 * measured slightly faster than updating in place (a caller with two slot sets per
 * request can alternate between them).
 * Errors: GDN_E_RANGE for a slot outside [0, n_slots) (src may be -1);
 * GDN_E_ALIAS if two rows share a dst slot or a dst slot is another row's src.
 */
int gdn_decode_step(const gdn_dims *dims, int32_t n_rows, const uint16_t *q,
                    const uint16_t *k, const uint16_t *v, const float *a,
                    const float *b, const float *A_log, const float *dt_bias,
                    float *state_pool, int32_t n_slots, const int32_t *src_slot,
                    const int32_t *dst_slot, uint16_t *o, void *stream);

/*
 * gdn_verify_window -- draft verification.  Row r runs T_r = row_tokens[r] tokens
 * (1 <= T_r <= k_max + 1: the previous bonus token and K_r = T_r - 1 drafts) from
 * the committed state in slot src_slot[r] (-1: zero state).  Writes o for all N
 * tokens and checkpoint slot j of row r = the state after j + 1 window tokens,
 * for j < T_r; slots j >= T_r are not touched.  The state pool is only read:
 * nothing is published until gdn_commit_accepted (transactional publication, the
 * pull request's "Summary").  ckpt must not overlap state_pool or o (GDN_E_ALIAS).
 * ckpt may be NULL: then only o is written, and the row is committed with
 * gdn_commit_replay instead of gdn_commit_accepted.
 */
int gdn_verify_window(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *a, const float *b, const float *A_log,
                      const float *dt_bias, const float *state_pool, int32_t n_slots,
                      const int32_t *src_slot, float *ckpt, uint16_t *o, void *stream);

/*
 * gdn_commit_accepted -- rollback to the accepted length.  accepted (device
 * int32 [n_rows]) holds a_r, the number of accepted drafts of row r; the committed
 * state becomes checkpoint slot a_r (the state after the bonus token and a_r
 * drafts), copied bit for bit to slot dst_slot[r].  row_tokens[r] is the row's
 * window length T_r.  A row whose a_r is outside [0, T_r - 1] is left untouched
 * and bit (r % 32) of status[r / 32] is set (status: device uint32
 * [(n_rows + 31) / 32]; bits are OR-ed in, the caller clears them).  Accepted
 * lengths stay on the device: no host readback.  Restoring the checkpoint at the
 * accepted length is how a rejected draft is undone (pull request "Run chained MTP
 * drafting in the batch Engine", sections "Correctness fix" and "Rollback fix and
 * corrected quality disposition"); device-resident draft data follows its "Summary".
 */
int gdn_commit_accepted(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                        const float *ckpt, const int32_t *accepted, float *state_pool,
                        int32_t n_slots, const int32_t *dst_slot, uint32_t *status,
                        void *stream);

/*
 * gdn_verify_tree -- draft verification of a token tree (topk > 1 drafting; the
 * pages verify chains only and refuse tree shapes, "Occamy 1.0 MTP", section "MTP1
 * runtime").  As gdn_verify_window, except that window token t of row r runs from
 * the state of its parent p = parents[cu_r + t] (host int32, one per packed token;
 * p = -1: the committed state in slot src_slot[r]) instead of from token t - 1:
 * checkpoint slot t of row r = the state of node t (its root path applied to the
 * committed state) and o_t = S_t q_t.  Nodes are in topological order: parents[cu_r]
 * = -1 and -1 <= p < t, else GDN_E_RANGE.  A chain (p = t - 1) gives bit for bit
 * the result of gdn_verify_window.  Commit the accepted path's last node n_r with
 * gdn_commit_accepted(accepted[r] = n_r).  ckpt is required.
 */
int gdn_verify_tree(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                    const int32_t *parents, const uint16_t *q, const uint16_t *k,
                    const uint16_t *v, const float *a, const float *b, const float *A_log,
                    const float *dt_bias, const float *state_pool, int32_t n_slots,
                    const int32_t *src_slot, float *ckpt, uint16_t *o, void *stream);

/*
 * gdn_commit_replay -- rollback without checkpoints: the pull request thread's
 * closing note replaces dense recurrent checkpoints with a replay of the
 * recurrent state.  Row r re-runs the first a_r + 1 tokens of its window (row_tokens[r] =
 * T_r tokens packed as for gdn_verify_window; the bonus token and the a_r accepted
 * drafts) from the committed state in slot src_slot[r] (-1: zero state) and
 * writes the resulting state to slot dst_slot[r] (== src_slot[r] commits in
 * place).  accepted (device int32 [n_rows]) is read on the device.  Decode,
 * verify and replay run one device routine, so the state written is bit-identical
 * to checkpoint slot a_r of gdn_verify_window on the same window, i.e. to what
 * gdn_commit_accepted would publish.  No outputs are written.  A row whose a_r is
 * outside [0, T_r - 1] is left untouched and bit (r % 32) of status[r / 32] is set
 * (status: device uint32 [(n_rows + 31) / 32], bits OR-ed in).
 * Errors: GDN_E_RANGE for a dst slot < 0 or any slot >= n_slots; GDN_E_ALIAS if two
 * rows share a dst slot or a dst slot is another row's src.
 */
int gdn_commit_replay(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *a, const float *b, const float *A_log,
                      const float *dt_bias, const int32_t *accepted, float *state_pool,
                      int32_t n_slots, const int32_t *src_slot, const int32_t *dst_slot,
                      uint32_t *status, void *stream);

/*
 * gdn_verify_window_delta / gdn_commit_delta -- rollback from compact exact
 * checkpoints.  Each step of the rule is a rank-1 update applied elementwise,
 * S_t[i][d] = fmaf(c_i, k_t[d], alpha_t S_{t-1}[i][d]) with c_i = beta_t (v_t[i] -
 * alpha_t (S_{t-1} k_t)_i), so the state after window token j is determined bit for
 * bit by the committed state, the keys and the factors (c, alpha_t) of tokens 0..j.
 * gdn_verify_window_delta is gdn_verify_window storing those factors instead of the
 * states: delta (device fp32 [n_rows][k_max+1][H_v][d_v + 4], 16-byte aligned)
 * receives, for window token t < T_r of row r and value head h, c at
 * [r][t][h][0..d_v), alpha_t at [r][t][h][d_v] and the factor the step's key was
 * scaled by at [r][t][h][d_v + 1] (1 unless GDN_QK_L2NORM; 2 floats of padding):
 * (d_v + 4) * 4 bytes per (token, head) instead of d_v * d_k * 4.
 * gdn_commit_delta folds tokens 0..a_r of row r (accepted: device int32 [n_rows];
 * k: the same packed window keys) into the state of slot src_slot[r] (-1: zero) and
 * writes slot dst_slot[r] (== src_slot[r] commits in place): bit-identical to
 * checkpoint slot a_r of gdn_verify_window on the same window.  A row whose a_r is
 * outside [0, T_r - 1] is left untouched and sets bit (r % 32) of status[r / 32].
 * Errors as gdn_verify_window and gdn_commit_replay.
 */
int gdn_verify_window_delta(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                            const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const float *a, const float *b, const float *A_log,
                            const float *dt_bias, const float *state_pool, int32_t n_slots,
                            const int32_t *src_slot, float *delta, uint16_t *o, void *stream);
int gdn_commit_delta(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                     const uint16_t *k, const float *delta, const int32_t *accepted,
                     float *state_pool, int32_t n_slots, const int32_t *src_slot,
                     const int32_t *dst_slot, uint32_t *status, void *stream);

/*
 * gdn_verify_window_delta_fold -- a verification step that first commits the
 * row's previous window: exactly gdn_commit_delta(prev_row_tokens, prev_k,
 * prev_delta, prev_accepted, src = dst = slot) followed by gdn_verify_window_delta
 * from slot[r] into delta, in one launch (the committed state is folded while it is
 * in registers and written back to slot[r] before the window runs; bit for bit the
 * same results).  slot[r] >= 0, distinct across rows; delta and prev_delta are two
 * different buffers (alternate them between steps).  A row whose prev_accepted is
 * outside [0, prev_row_tokens[r] - 1] is left untouched -- no fold, no outputs, no
 * factors -- and sets bit (r % 32) of status[r / 32].
 */
int gdn_verify_window_delta_fold(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                                 const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const float *a, const float *b, const float *A_log,
                                 const float *dt_bias, float *state_pool, int32_t n_slots,
                                 const int32_t *slot, float *delta, uint16_t *o,
                                 const int32_t *prev_row_tokens, const uint16_t *prev_k,
                                 const float *prev_delta, const int32_t *prev_accepted,
                                 uint32_t *status, void *stream);

/*
 * gdn_verify_window_select / gdn_commit_select -- rollback by selecting the accepted
 * checkpoint instead of copying it (the checkpoint-select form of the commit).  The
 * checkpoints live in the state pool: row r writes pool slots bank[r] * (k_max + 1) + j
 * for j < T_r (bank: host int32 [n_rows], >= 0, distinct across rows, (bank[r] + 1) *
 * (k_max + 1) <= n_slots).  Its source slot is read on the device from slot_table[r]
 * (device int32 [n_rows]; -1: zero state), so accepted counts never visit the host
 * (the pull request keeps draft data on the device, "Summary").  gdn_commit_select sets
 * slot_table[r] = bank[r] * (k_max + 1) + accepted[r]: the state after the accepted
 * prefix becomes the committed state where it already is, bit-identical to what
 * gdn_commit_accepted would copy.  A caller alternates each row between two banks, so a
 * window never writes over the state it starts from.  Checked on the device: a source
 * slot outside [-1, n_slots) or inside any bank of the call leaves the row untouched (no
 * outputs, no checkpoints); an accepted count outside [0, T_r) leaves slot_table[r]
 * unchanged; either sets bit (r % 32) of status[r / 32].  n_rows <= 64 per call
 * (GDN_E_RANGE otherwise): the banks of a call are checked in one launch.
 */
int gdn_verify_window_select(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                             const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *a, const float *b, const float *A_log,
                             const float *dt_bias, float *state_pool, int32_t n_slots,
                             const int32_t *slot_table, const int32_t *bank, uint16_t *o,
                             uint32_t *status, void *stream);
int gdn_commit_select(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                      const int32_t *accepted, const int32_t *bank, int32_t n_slots,
                      int32_t *slot_table, uint32_t *status, void *stream);

/*
 * gdn_verify_window_select_commit -- gdn_commit_select of the previous window followed
 * by gdn_verify_window_select of this one, in one launch: row r first makes slot
 * prev_bank[r] * (k_max + 1) + accepted[r] its committed state (and slot_table[r]) when
 * 0 <= accepted[r] < prev_row_tokens[r], then verifies this window from it into bank[r].
 * The results are those of the two calls bit for bit, including an accepted count out of
 * range: slot_table[r] is left as it was, bit (r % 32) of status[r / 32] is set, and the
 * window runs from the entry it was left at.  Saves a launch per layer per step, which a
 * latency-bound batch of one request feels most.  prev_row_tokens, prev_bank: host int32
 * [n_rows], the previous call's row_tokens and bank; accepted: device int32 [n_rows].
 * Errors as gdn_verify_window_select, plus GDN_E_RANGE for prev_row_tokens outside
 * [1, k_max + 1] or a previous bank outside the pool, GDN_E_ALIAS when a previous bank is
 * one this window writes.
 */
int gdn_verify_window_select_commit(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                                    const int32_t *prev_row_tokens, const int32_t *prev_bank,
                                    const int32_t *accepted, const uint16_t *q, const uint16_t *k,
                                    const uint16_t *v, const float *a, const float *b,
                                    const float *A_log, const float *dt_bias, float *state_pool,
                                    int32_t n_slots, int32_t *slot_table, const int32_t *bank,
                                    uint16_t *o, uint32_t *status, void *stream);

/*
 * gdn_chunked_workspace_bytes -- device workspace that gdn_chunked_prefill_with_
 * checkpoints and gdn_run_transaction need for these rows (0 on a bad argument, or
 * for rows of more than GDN_MAX_CHUNK_UNITS (chunk, value head) units in all).
 * A workspace that would pass 160 MiB holds W in fp32 instead of three bf16 parts,
 * so the size is not linear in the token count across that point.
 */
#define GDN_MAX_CHUNK_UNITS ((int64_t)1 << 24) /* chunks x value heads in one call */
size_t gdn_chunked_workspace_bytes(const gdn_dims *dims, int32_t n_rows,
                                   const int32_t *row_tokens, int32_t chunk);

/*
 * gdn_chunked_prefill_with_checkpoints -- long rows in the chunkwise (UT / WY)
 * form of the rule, chunk = 64 tokens, chunks starting at each row's first token
 * (the last chunk of a row may be partial; chunks never span rows).  Row r runs
 * L_r = row_tokens[r] >= 1 tokens from slot src_slot[r] (-1: zero state), writes
 * o for all its tokens, the final state to slot dst_slot[r] (-1: not written),
 * and checkpoint slot j = the state after L_r - n_tail[r] + j + 1 tokens for
 * j < n_tail[r] <= min(L_r, k_max + 1), the same slot meaning as a verify window,
 * so gdn_commit_accepted works on either path: a long prefill that takes the
 * chunked form still publishes the checkpoints that draft rejection needs (the pull
 * request's "Correctness fix").  The chunkwise form is the gated delta rule's
 * blocked (UT transform / WY representation) evaluation (Yang, Kautz & Hatamizadeh,
 * ICLR 2025).  Matches the sequential rule to fp32 rounding, not bit for bit.
 * Errors: GDN_E_WORKSPACE if ws_bytes < gdn_chunked_workspace_bytes(...);
 * GDN_E_UNSUPPORTED for chunk != 64; GDN_E_RANGE for more than GDN_MAX_CHUNK_UNITS
 * (chunk, value head) units; slot checks as gdn_decode_step.
 */
int gdn_chunked_prefill_with_checkpoints(
    const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens, int32_t chunk,
    const int32_t *n_tail, const uint16_t *q, const uint16_t *k, const uint16_t *v,
    const float *a, const float *b, const float *A_log, const float *dt_bias,
    float *state_pool, int32_t n_slots, const int32_t *src_slot,
    const int32_t *dst_slot, float *ckpt, uint16_t *o, void *workspace,
    size_t ws_bytes, void *stream);

/*
 * gdn_chunked_prefill_with_checkpoints_static -- gdn_chunked_prefill_with_checkpoints
 * for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The caller still passes every input
 * and output; the workspace is a device array that the library itself holds, one per
 * GPU, GDN_STATIC_WS_BYTES long, resident from the library's load until the process
 * ends.  The call allocates and frees nothing: on its first use on a GPU it looks up
 * that GPU's copy of the array (hipGetSymbolAddress) and keeps the address.
 * Same arguments, results and errors as gdn_chunked_prefill_with_checkpoints without
 * workspace/ws_bytes, plus: GDN_E_WORKSPACE when gdn_chunked_workspace_bytes(...)
 * exceeds GDN_STATIC_WS_BYTES (the call is refused, nothing runs), GDN_E_HIP if the
 * lookup fails.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (two streams, two host threads) race and must be ordered by the
 * caller.  Nothing in the array has to start at zero: each call writes every
 * workspace value before it reads it.
 */
#define GDN_STATIC_WS_BYTES ((size_t)128 << 20) /* 128 MiB per GPU */
int gdn_chunked_prefill_with_checkpoints_static(
    const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens, int32_t chunk,
    const int32_t *n_tail, const uint16_t *q, const uint16_t *k, const uint16_t *v,
    const float *a, const float *b, const float *A_log, const float *dt_bias,
    float *state_pool, int32_t n_slots, const int32_t *src_slot,
    const int32_t *dst_slot, float *ckpt, uint16_t *o, void *stream);

/*
 * gdn_plan_transaction -- the per-row execution plan of a packed ragged batch
 * (pure host function, deterministic).  A row of at most k_max + 1 tokens goes to
 * the recurrent kernel shared with decode (route GDN_ROUTE_RECURRENT), so its
 * checkpoints are bit-consistent with decode; a longer row goes to the chunked
 * kernels (GDN_ROUTE_CHUNKED).  Every row gets the checkpoints it asks for on
 * either route: one plan is never forced on the whole batch, the fault described
 * in the pull request's "Correctness fix".  route: host int32 [n_rows].
 */
int gdn_plan_transaction(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                         int32_t *route);

/*
 * gdn_run_transaction -- one mixed ragged transaction: plans the rows
 * (gdn_plan_transaction) and launches both routes on `stream`.  Row r runs
 * row_tokens[r] tokens from src_slot[r] (-1: zero state), writes o for its tokens,
 * checkpoint slots j < n_ckpt[r] <= min(L_r, k_max + 1) (state after
 * L_r - n_ckpt[r] + j + 1 tokens) and, if dst_slot[r] >= 0, its final state.
 * A verify row passes n_ckpt = T_r and dst = -1 (commit later); a prefill row
 * passes n_ckpt = 0 and its dst slot.  workspace as gdn_chunked_workspace_bytes
 * (may be NULL/0 when no row is longer than k_max + 1).  GDN_E_RANGE when the rows
 * routed to the chunked kernels hold more than GDN_MAX_CHUNK_UNITS (chunk, value head)
 * units; otherwise errors as gdn_chunked_prefill_with_checkpoints.
 */
int gdn_run_transaction(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                        const int32_t *n_ckpt, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, const float *a, const float *b,
                        const float *A_log, const float *dt_bias, float *state_pool,
                        int32_t n_slots, const int32_t *src_slot, const int32_t *dst_slot,
                        float *ckpt, uint16_t *o, void *workspace, size_t ws_bytes,
                        void *stream);

/* Human-readable name of a return code. */
const char *gdn_status_str(int code);

/* GDN_VERSION of the built library. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H_ */
