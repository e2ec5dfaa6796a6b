// gdn_api.cpp -- the libgdn C ABI (include/gdn.h): host-side validation, the
// per-row planner and kernel launches.  Everything is checked before the first
// launch, so a call that returns an error has written nothing (fail closed).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

using gdn::kRowsPerLaunch;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void *p, size_t pb, const void *q, size_t qb) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return pb && qb && a < b + qb && b < a + pb;
}

int check_dims(const gdn_dims *d) {
  if (!d) return GDN_E_NULL;
  if (d->d_k != d->d_v || (d->d_k != 16 && d->d_k != 128)) return GDN_E_UNSUPPORTED;
  if (d->n_qk_heads <= 0 || d->n_v_heads <= 0 || d->n_v_heads % d->n_qk_heads)
    return GDN_E_UNSUPPORTED;
  // keeps every launch's grid (rows x heads x blocks per head x threads) far below 2^32
  if (d->n_v_heads > GDN_MAX_V_HEADS) return GDN_E_UNSUPPORTED;
  if (d->k_max < 0 || d->k_max > GDN_MAX_K) return GDN_E_UNSUPPORTED;
  if (d->flags & ~GDN_QK_L2NORM) return GDN_E_UNSUPPORTED;
  return GDN_OK;
}

struct Sizes {
  size_t unit_floats;  // d_v * d_k
  size_t row_floats;   // H_v * unit
  size_t ck_row_floats;  // (k_max + 1) * row
};

Sizes sizes_of(const gdn_dims *d) {
  Sizes s;
  s.unit_floats = size_t(d->d_v) * size_t(d->d_k);
  s.row_floats = size_t(d->n_v_heads) * s.unit_floats;
  s.ck_row_floats = size_t(d->k_max + 1) * s.row_floats;
  return s;
}

// Token inputs shared by every compute call (o may be absent only where the call
// writes no outputs).
int check_tokens(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                 const float *b, const float *A_log, const float *dt_bias, const uint16_t *o,
                 bool need_o = true) {
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || (need_o && !o)) return GDN_E_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || (o && !aligned(o, 16))) return GDN_E_ALIGN;
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(A_log, 4) || !aligned(dt_bias, 4))
    return GDN_E_ALIGN;
  return GDN_OK;
}

// Source slots may be -1 (zero state); destination slots must be distinct and
// must not be read by another row of the same launch set.
int check_slots(int32_t n_rows, int32_t n_slots, const int32_t *src, const int32_t *dst) {
  if (n_rows > 0 && n_slots < 1) return GDN_E_RANGE;  // kernels read slot 0 for source -1
  for (int32_t r = 0; r < n_rows; ++r) {
    if (src && (src[r] < -1 || src[r] >= n_slots)) return GDN_E_RANGE;
    if (dst && (dst[r] < -1 || dst[r] >= n_slots)) return GDN_E_RANGE;
  }
  if (!dst) return GDN_OK;
  std::vector<int32_t> d;
  for (int32_t r = 0; r < n_rows; ++r)
    if (dst[r] >= 0) d.push_back(dst[r]);
  std::vector<int32_t> sorted = d;
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return GDN_E_ALIAS;
  if (src)
    for (int32_t r = 0; r < n_rows; ++r) {
      if (dst[r] < 0) continue;
      for (int32_t r2 = 0; r2 < n_rows; ++r2)
        if (r2 != r && src[r2] == dst[r]) return GDN_E_ALIAS;
    }
  return GDN_OK;
}

void fill_common(gdn::RecurrentArgs &ra, const gdn_dims *d, const uint16_t *q,
                 const uint16_t *k, const uint16_t *v, const float *a, const float *b,
                 const float *A_log, const float *dt_bias, const float *state_in,
                 float *state_out, float *ckpt, uint16_t *o) {
  memset(&ra, 0, sizeof(ra));
  ra.q = q; ra.k = k; ra.v = v; ra.a = a; ra.b = b; ra.A_log = A_log; ra.dt_bias = dt_bias;
  ra.state_in = state_in; ra.state_out = state_out; ra.ckpt = ckpt; ra.o = o;
  ra.n_qk = d->n_qk_heads; ra.n_v = d->n_v_heads;
  ra.group = d->n_v_heads / d->n_qk_heads;
  ra.ck_slots = d->k_max + 1;
  ra.qk_norm = (d->flags & GDN_QK_L2NORM) ? 1 : 0;
}

// Runs rows `rows` (indices into the call's rows) through the recurrent kernel,
// kRowsPerLaunch at a time; row r keeps its own token offset and checkpoint row.
int launch_recurrent_rows(const gdn_dims *d, const gdn::RecurrentArgs &proto,
                          const std::vector<int32_t> &rows, const std::vector<int64_t> &cu,
                          const int32_t *ntok, const int32_t *src, const int32_t *dst,
                          const int32_t *n_ck, hipStream_t stream,
                          const int32_t *parents = nullptr,
                          const int32_t *fold_ntok = nullptr, const int64_t *fold_cu = nullptr,
                          const int32_t *ck_rows = nullptr) {
  for (size_t base = 0; base < rows.size(); base += kRowsPerLaunch) {
    gdn::RecurrentArgs ra = proto;
    const size_t n = std::min<size_t>(kRowsPerLaunch, rows.size() - base);
    ra.n_rows = int32_t(n);
    for (size_t j = 0; j < n; ++j) {
      const int32_t r = rows[base + j];
      ra.tok0[j] = int32_t(cu[r]);
      ra.ntok[j] = ntok[r];
      ra.src[j] = src ? src[r] : -1;
      ra.dst[j] = dst ? dst[r] : -1;
      ra.ck_first[j] = n_ck ? ntok[r] - n_ck[r] : ntok[r];
      ra.ck_row[j] = ck_rows ? ck_rows[r] : r;
      if (parents) {  // byte t: parent of window token t, plus one
        uint32_t packed = 0;
        for (int32_t t = 0; t < ntok[r]; ++t) packed |= uint32_t(parents[cu[r] + t] + 1) << (8 * t);
        ra.tree[j] = packed;
      }
    }
    ra.tree_mode = parents ? 1 : 0;
    if (fold_ntok)
      for (size_t j = 0; j < n; ++j) {
        ra.fold_tok0[j] = int32_t(fold_cu[rows[base + j]]);
        ra.fold_ntok[j] = fold_ntok[rows[base + j]];
      }
    if (gdn::launch_recurrent(ra, d->d_k, stream) != hipSuccess) return GDN_E_HIP;
  }
  return GDN_OK;
}

int64_t chunks_of(int32_t len) { return (int64_t(len) + gdn::kChunk - 1) / gdn::kChunk; }

// Runs rows `rows` through the chunked kernels, kRowsPerLaunch at a time;
// workspace chunks are numbered over all of `rows`.
int launch_chunked_rows(const gdn_dims *d, const gdn::ChunkArgs &proto,
                        const std::vector<int32_t> &rows, const std::vector<int64_t> &cu,
                        const int32_t *len, const int32_t *n_tail, const int32_t *src,
                        const int32_t *dst, hipStream_t stream) {
  int64_t chunk_base = 0, chunks = 0;
  for (int32_t r : rows) chunks += chunks_of(len[r]);
  // one layout for the call: the qk-head units follow all the value-head units
  const bool streamed = gdn::chunk_ws_streamed(chunks, d->n_v_heads, d->n_qk_heads, d->d_k);
  float *const ws_qk = proto.ws + chunks * d->n_v_heads * gdn::chunk_ws_unit_floats(d->d_k, streamed);
  for (size_t base = 0; base < rows.size(); base += kRowsPerLaunch) {
    gdn::ChunkArgs ca = proto;
    ca.ws_streamed = streamed ? 1 : 0;
    ca.ws_qk = ws_qk;
    const size_t n = std::min<size_t>(kRowsPerLaunch, rows.size() - base);
    ca.n_rows = int32_t(n);
    int32_t local = 0;
    for (size_t j = 0; j < n; ++j) {
      const int32_t r = rows[base + j];
      ca.tok0[j] = int32_t(cu[r]);
      ca.len[j] = len[r];
      ca.chunk_start[j] = local;
      ca.chunk0[j] = int32_t(chunk_base + local);
      ca.src[j] = src ? src[r] : -1;
      ca.dst[j] = dst ? dst[r] : -1;
      ca.n_tail[j] = n_tail ? n_tail[r] : 0;
      ca.ck_row[j] = r;
      local += int32_t(chunks_of(len[r]));
    }
    if (gdn::launch_chunked(ca, d->d_k, local, stream) != hipSuccess) return GDN_E_HIP;
    chunk_base += local;
  }
  return GDN_OK;
}

// The prep kernel runs one 256-thread block per (chunk, value head) in a 1-D grid, whose
// work-item count must stay below 2^32.
bool chunk_units_fit(const gdn_dims *d, const std::vector<int32_t> &rows, const int32_t *len) {
  int64_t chunks = 0;
  for (int32_t r : rows) chunks += chunks_of(len[r]);
  return chunks * d->n_v_heads <= GDN_MAX_CHUNK_UNITS;
}

size_t chunked_ws_bytes(const gdn_dims *d, const std::vector<int32_t> &rows, const int32_t *len) {
  int64_t chunks = 0;
  for (int32_t r : rows) chunks += chunks_of(len[r]);
  const bool streamed = gdn::chunk_ws_streamed(chunks, d->n_v_heads, d->n_qk_heads, d->d_k);
  return size_t(gdn::chunk_ws_floats(chunks, d->n_v_heads, d->n_qk_heads, d->d_k, streamed)) * 4;
}

void fill_chunk_common(gdn::ChunkArgs &ca, const gdn_dims *d, const uint16_t *q, const uint16_t *k,
                       const uint16_t *v, const float *a, const float *b, const float *A_log,
                       const float *dt_bias, float *pool, float *ckpt, uint16_t *o, void *ws) {
  memset(&ca, 0, sizeof(ca));
  ca.q = q; ca.k = k; ca.v = v; ca.a = a; ca.b = b; ca.A_log = A_log; ca.dt_bias = dt_bias;
  ca.state_in = pool; ca.state_out = pool; ca.ckpt = ckpt; ca.o = o;
  ca.ws = static_cast<float *>(ws);
  ca.n_qk = d->n_qk_heads; ca.n_v = d->n_v_heads;
  ca.group = d->n_v_heads / d->n_qk_heads;
  ca.ck_slots = d->k_max + 1;
  ca.qk_norm = (d->flags & GDN_QK_L2NORM) ? 1 : 0;
}

// Shared checks of a packed batch whose rows run from src to dst slots with some
// checkpoints each (chunked prefill and transactions).  Fills cu on success.
int check_packed(const gdn_dims *dims, int32_t n_rows, const int32_t *len, const int32_t *n_ck,
                 const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                 const float *b, const float *A_log, const float *dt_bias, float *state_pool,
                 int32_t n_slots, const int32_t *src_slot, const int32_t *dst_slot, float *ckpt,
                 uint16_t *o, std::vector<int64_t> &cu) {
  int rc;
  if (!len || !n_ck || !src_slot || !dst_slot) return GDN_E_NULL;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, o))) return rc;
  if (!state_pool) return GDN_E_NULL;
  if (!aligned(state_pool, 16)) return GDN_E_ALIGN;
  bool any_ck = false;
  for (int32_t r = 0; r < n_rows; ++r) {
    if (len[r] < 1) return GDN_E_RANGE;
    if (n_ck[r] < 0 || n_ck[r] > len[r] || n_ck[r] > dims->k_max + 1) return GDN_E_RANGE;
    any_ck |= n_ck[r] > 0;
  }
  if (any_ck && !ckpt) return GDN_E_NULL;
  if (ckpt && !aligned(ckpt, 16)) return GDN_E_ALIGN;
  if ((rc = check_slots(n_rows, n_slots, src_slot, dst_slot))) return rc;
  cu.assign(size_t(n_rows) + 1, 0);
  for (int32_t r = 0; r < n_rows; ++r) cu[r + 1] = cu[r] + len[r];
  if (cu[n_rows] > INT32_MAX) return GDN_E_RANGE;
  const Sizes s = sizes_of(dims);
  const size_t pool_b = size_t(n_slots) * s.row_floats * 4;
  const size_t ck_b = ckpt ? size_t(n_rows) * s.ck_row_floats * 4 : 0;
  const size_t o_b = size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2;
  if (overlap(ckpt, ck_b, state_pool, pool_b) || overlap(o, o_b, ckpt, ck_b) ||
      overlap(o, o_b, state_pool, pool_b))
    return GDN_E_ALIAS;
  return GDN_OK;
}

int check_workspace(void *ws, size_t ws_bytes, size_t need, const void *pool, size_t pool_b,
                    const void *ckpt, size_t ck_b, const void *o, size_t o_b) {
  if (need == 0) return GDN_OK;
  if (!ws || ws_bytes < need) return GDN_E_WORKSPACE;
  if (!aligned(ws, 16)) return GDN_E_ALIGN;
  if (overlap(ws, need, pool, pool_b) || overlap(ws, need, ckpt, ck_b) || overlap(ws, need, o, o_b))
    return GDN_E_ALIAS;
  return GDN_OK;
}

std::vector<int64_t> prefix(int32_t n_rows, const int32_t *ntok) {
  std::vector<int64_t> cu(size_t(n_rows) + 1, 0);
  for (int32_t r = 0; r < n_rows; ++r) cu[r + 1] = cu[r] + ntok[r];
  return cu;
}

// Chunked prefill with a caller workspace, or (use_static) with the library's static
// per-GPU array; every argument is checked before the array is looked up.
int chunked_prefill(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens, int32_t chunk,
                    const int32_t *n_tail, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *a, const float *b, const float *A_log, const float *dt_bias,
                    float *state_pool, int32_t n_slots, const int32_t *src_slot, const int32_t *dst_slot,
                    float *ckpt, uint16_t *o, void *workspace, size_t ws_bytes, bool use_static,
                    hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (chunk != gdn::kChunk) return GDN_E_UNSUPPORTED;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  std::vector<int64_t> cu;
  if ((rc = check_packed(dims, n_rows, row_tokens, n_tail, q, k, v, a, b, A_log, dt_bias,
                         state_pool, n_slots, src_slot, dst_slot, ckpt, o, cu)))
    return rc;
  std::vector<int32_t> rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  if (!chunk_units_fit(dims, rows, row_tokens)) return GDN_E_RANGE;
  const Sizes s = sizes_of(dims);
  const size_t need = chunked_ws_bytes(dims, rows, row_tokens);
  if (use_static) {
    if (need > GDN_STATIC_WS_BYTES) return GDN_E_WORKSPACE;
    if (gdn::static_workspace(&workspace, &ws_bytes) != hipSuccess) return GDN_E_HIP;
  }
  if ((rc = check_workspace(workspace, ws_bytes, need, state_pool, size_t(n_slots) * s.row_floats * 4,
                            ckpt, ckpt ? size_t(n_rows) * s.ck_row_floats * 4 : 0, o,
                            size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2)))
    return rc;
  gdn::ChunkArgs proto;
  fill_chunk_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, ckpt, o, workspace);
  return launch_chunked_rows(dims, proto, rows, cu, row_tokens, n_tail, src_slot, dst_slot, stream);
}

}  // namespace

extern "C" {

int gdn_version(void) { return GDN_VERSION; }

const char *gdn_status_str(int code) {
  switch (code) {
    case GDN_OK: return "ok";
    case GDN_E_NULL: return "null pointer";
    case GDN_E_UNSUPPORTED: return "unsupported shape";
    case GDN_E_RANGE: return "token count, slot or checkpoint count out of range";
    case GDN_E_ALIAS: return "aliasing slots or overlapping buffers";
    case GDN_E_ALIGN: return "misaligned device pointer";
    case GDN_E_WORKSPACE: return "workspace missing or too small";
    case GDN_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int gdn_decode_step(const gdn_dims *dims, int32_t n_rows, const uint16_t *q, const uint16_t *k,
                    const uint16_t *v, const float *a, const float *b, const float *A_log,
                    const float *dt_bias, float *state_pool, int32_t n_slots,
                    const int32_t *src_slot, const int32_t *dst_slot, uint16_t *o,
                    void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, o))) return rc;
  if (!state_pool || !src_slot || !dst_slot) return GDN_E_NULL;
  if (!aligned(state_pool, 16)) return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r)
    if (dst_slot[r] < 0) return GDN_E_RANGE;
  if ((rc = check_slots(n_rows, n_slots, src_slot, dst_slot))) return rc;
  const Sizes s = sizes_of(dims);
  if (overlap(o, size_t(n_rows) * s.row_floats / dims->d_k * 2, state_pool,
              size_t(n_slots) * s.row_floats * 4))
    return GDN_E_ALIAS;

  std::vector<int32_t> ones(static_cast<size_t>(n_rows), 1), rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  const std::vector<int64_t> cu = prefix(n_rows, ones.data());
  gdn::RecurrentArgs proto;
  fill_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, state_pool, nullptr, o);
  return launch_recurrent_rows(dims, proto, rows, cu, ones.data(), src_slot, dst_slot, nullptr,
                               static_cast<hipStream_t>(stream));
}

int gdn_verify_window(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                      const float *b, const float *A_log, const float *dt_bias,
                      const float *state_pool, int32_t n_slots, const int32_t *src_slot,
                      float *ckpt, uint16_t *o, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens) return GDN_E_NULL;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, o))) return rc;
  if (!state_pool || !src_slot) return GDN_E_NULL;
  if (!aligned(state_pool, 16) || (ckpt && !aligned(ckpt, 16))) return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r)
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
  if ((rc = check_slots(n_rows, n_slots, src_slot, nullptr))) return rc;
  const Sizes s = sizes_of(dims);
  const std::vector<int64_t> cu = prefix(n_rows, row_tokens);
  if (cu.back() > INT32_MAX) return GDN_E_RANGE;  // token offsets are int32
  const size_t pool_b = size_t(n_slots) * s.row_floats * 4;
  const size_t ck_b = ckpt ? size_t(n_rows) * s.ck_row_floats * 4 : 0;
  const size_t o_b = size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2;
  if (overlap(ckpt, ck_b, state_pool, pool_b) || overlap(o, o_b, ckpt, ck_b) ||
      overlap(o, o_b, state_pool, pool_b))
    return GDN_E_ALIAS;

  std::vector<int32_t> rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  gdn::RecurrentArgs proto;
  fill_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, nullptr, ckpt, o);
  return launch_recurrent_rows(dims, proto, rows, cu, row_tokens, src_slot, nullptr,
                               ckpt ? row_tokens : nullptr, static_cast<hipStream_t>(stream));
}

int gdn_verify_tree(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                    const int32_t *parents, const uint16_t *q, const uint16_t *k,
                    const uint16_t *v, const float *a, const float *b, const float *A_log,
                    const float *dt_bias, const float *state_pool, int32_t n_slots,
                    const int32_t *src_slot, float *ckpt, uint16_t *o, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens || !parents) return GDN_E_NULL;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, o))) return rc;
  if (!state_pool || !src_slot || !ckpt) return GDN_E_NULL;
  if (!aligned(state_pool, 16) || !aligned(ckpt, 16)) return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r)
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
  const std::vector<int64_t> cu = prefix(n_rows, row_tokens);
  if (cu.back() > INT32_MAX) return GDN_E_RANGE;  // token offsets are int32
  for (int32_t r = 0; r < n_rows; ++r) {
    if (parents[cu[r]] != -1) return GDN_E_RANGE;  // the window's first token follows the committed state
    for (int32_t t = 1; t < row_tokens[r]; ++t)
      if (parents[cu[r] + t] < -1 || parents[cu[r] + t] >= t) return GDN_E_RANGE;
  }
  if ((rc = check_slots(n_rows, n_slots, src_slot, nullptr))) return rc;
  const Sizes s = sizes_of(dims);
  const size_t pool_b = size_t(n_slots) * s.row_floats * 4;
  const size_t ck_b = size_t(n_rows) * s.ck_row_floats * 4;
  const size_t o_b = size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2;
  if (overlap(ckpt, ck_b, state_pool, pool_b) || overlap(o, o_b, ckpt, ck_b) ||
      overlap(o, o_b, state_pool, pool_b))
    return GDN_E_ALIAS;

  std::vector<int32_t> rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  gdn::RecurrentArgs proto;
  fill_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, nullptr, ckpt, o);
  return launch_recurrent_rows(dims, proto, rows, cu, row_tokens, src_slot, nullptr, row_tokens,
                               static_cast<hipStream_t>(stream), parents);
}

int gdn_verify_window_delta(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                            const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                            const float *b, const float *A_log, const float *dt_bias,
                            const float *state_pool, int32_t n_slots, const int32_t *src_slot,
                            float *delta, uint16_t *o, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens) return GDN_E_NULL;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, o))) return rc;
  if (!state_pool || !src_slot || !delta) return GDN_E_NULL;
  if (!aligned(state_pool, 16) || !aligned(delta, 16)) return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r)
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
  if ((rc = check_slots(n_rows, n_slots, src_slot, nullptr))) return rc;
  const Sizes s = sizes_of(dims);
  const std::vector<int64_t> cu = prefix(n_rows, row_tokens);
  if (cu.back() > INT32_MAX) return GDN_E_RANGE;  // token offsets are int32
  const size_t pool_b = size_t(n_slots) * s.row_floats * 4;
  const size_t dl_b = size_t(n_rows) * size_t(dims->k_max + 1) * size_t(dims->n_v_heads) *
                      size_t(gdn::delta_row_floats(dims->d_v)) * 4;
  const size_t o_b = size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2;
  if (overlap(delta, dl_b, state_pool, pool_b) || overlap(o, o_b, delta, dl_b) ||
      overlap(o, o_b, state_pool, pool_b))
    return GDN_E_ALIAS;
  std::vector<int32_t> rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  gdn::RecurrentArgs proto;
  fill_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, nullptr, nullptr, o);
  proto.delta = delta;
  return launch_recurrent_rows(dims, proto, rows, cu, row_tokens, src_slot, nullptr, nullptr,
                               static_cast<hipStream_t>(stream));
}

int gdn_verify_window_delta_fold(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                                 const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const float *a, const float *b, const float *A_log,
                                 const float *dt_bias, float *state_pool, int32_t n_slots,
                                 const int32_t *slot, float *delta, uint16_t *o,
                                 const int32_t *prev_row_tokens, const uint16_t *prev_k,
                                 const float *prev_delta, const int32_t *prev_accepted,
                                 uint32_t *status, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens || !prev_row_tokens) return GDN_E_NULL;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, o))) return rc;
  if (!state_pool || !slot || !delta || !prev_k || !prev_delta || !prev_accepted || !status)
    return GDN_E_NULL;
  if (!aligned(state_pool, 16) || !aligned(delta, 16) || !aligned(prev_delta, 16) || !aligned(prev_k, 16) ||
      !aligned(prev_accepted, 4) || !aligned(status, 4))
    return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r) {
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
    if (prev_row_tokens[r] < 1 || prev_row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
    if (slot[r] < 0) return GDN_E_RANGE;  // the folded state is published to it
  }
  if ((rc = check_slots(n_rows, n_slots, slot, slot))) return rc;
  const Sizes s = sizes_of(dims);
  const std::vector<int64_t> cu = prefix(n_rows, row_tokens), pcu = prefix(n_rows, prev_row_tokens);
  if (cu.back() > INT32_MAX || pcu.back() > INT32_MAX) return GDN_E_RANGE;  // token offsets are int32
  const size_t pool_b = size_t(n_slots) * s.row_floats * 4;
  const size_t dl_b = size_t(n_rows) * size_t(dims->k_max + 1) * size_t(dims->n_v_heads) *
                      size_t(gdn::delta_row_floats(dims->d_v)) * 4;
  const size_t o_b = size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2;
  if (overlap(delta, dl_b, state_pool, pool_b) || overlap(o, o_b, delta, dl_b) ||
      overlap(o, o_b, state_pool, pool_b) || overlap(delta, dl_b, prev_delta, dl_b) ||
      overlap(prev_delta, dl_b, state_pool, pool_b))
    return GDN_E_ALIAS;
  std::vector<int32_t> rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  gdn::RecurrentArgs proto;
  fill_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, state_pool, nullptr, o);
  proto.delta = delta;
  proto.fold_k = prev_k;
  proto.fold_delta = prev_delta;
  proto.fold_accepted = prev_accepted;
  proto.status = status;
  return launch_recurrent_rows(dims, proto, rows, cu, row_tokens, slot, nullptr, nullptr,
                               static_cast<hipStream_t>(stream), nullptr, prev_row_tokens, pcu.data());
}

int gdn_commit_delta(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                     const uint16_t *k, const float *delta, const int32_t *accepted,
                     float *state_pool, int32_t n_slots, const int32_t *src_slot,
                     const int32_t *dst_slot, uint32_t *status, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens || !k || !delta || !accepted || !state_pool || !src_slot || !dst_slot || !status)
    return GDN_E_NULL;
  if (!aligned(k, 16) || !aligned(delta, 16) || !aligned(state_pool, 16) || !aligned(accepted, 4) ||
      !aligned(status, 4))
    return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r) {
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
    if (dst_slot[r] < 0) return GDN_E_RANGE;
  }
  if ((rc = check_slots(n_rows, n_slots, src_slot, dst_slot))) return rc;
  const Sizes s = sizes_of(dims);
  const size_t dl_b = size_t(n_rows) * size_t(dims->k_max + 1) * size_t(dims->n_v_heads) *
                      size_t(gdn::delta_row_floats(dims->d_v)) * 4;
  if (overlap(delta, dl_b, state_pool, size_t(n_slots) * s.row_floats * 4)) return GDN_E_ALIAS;
  const std::vector<int64_t> cu = prefix(n_rows, row_tokens);
  if (cu.back() > INT32_MAX) return GDN_E_RANGE;  // token offsets are int32
  for (int32_t r0 = 0; r0 < n_rows; r0 += kRowsPerLaunch) {
    gdn::FoldArgs fa;
    memset(&fa, 0, sizeof(fa));
    const int32_t n = std::min<int32_t>(kRowsPerLaunch, n_rows - r0);
    fa.k = k;
    fa.delta = delta;
    fa.pool_in = state_pool;
    fa.pool_out = state_pool;
    fa.accepted = accepted;
    fa.status = status;
    fa.n_qk = dims->n_qk_heads;
    fa.n_v = dims->n_v_heads;
    fa.group = dims->n_v_heads / dims->n_qk_heads;
    fa.ck_slots = dims->k_max + 1;
    fa.n_rows = n;
    fa.row_base = r0;
    for (int32_t j = 0; j < n; ++j) {
      fa.tok0[j] = int32_t(cu[r0 + j]);
      fa.ntok[j] = row_tokens[r0 + j];
      fa.src[j] = src_slot[r0 + j];
      fa.dst[j] = dst_slot[r0 + j];
    }
    if (gdn::launch_fold(fa, dims->d_k, static_cast<hipStream_t>(stream)) != hipSuccess) return GDN_E_HIP;
  }
  return GDN_OK;
}

int gdn_commit_replay(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                      const float *b, const float *A_log, const float *dt_bias,
                      const int32_t *accepted, float *state_pool, int32_t n_slots,
                      const int32_t *src_slot, const int32_t *dst_slot, uint32_t *status,
                      void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens) return GDN_E_NULL;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, nullptr, false))) return rc;
  if (!accepted || !state_pool || !src_slot || !dst_slot || !status) return GDN_E_NULL;
  if (!aligned(state_pool, 16) || !aligned(accepted, 4) || !aligned(status, 4)) return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r) {
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
    if (dst_slot[r] < 0) return GDN_E_RANGE;
  }
  if ((rc = check_slots(n_rows, n_slots, src_slot, dst_slot))) return rc;

  std::vector<int32_t> rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  const std::vector<int64_t> cu = prefix(n_rows, row_tokens);
  if (cu.back() > INT32_MAX) return GDN_E_RANGE;  // token offsets are int32
  gdn::RecurrentArgs proto;
  fill_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, state_pool, nullptr, nullptr);
  proto.accepted = accepted;
  proto.status = status;
  return launch_recurrent_rows(dims, proto, rows, cu, row_tokens, src_slot, dst_slot, nullptr,
                               static_cast<hipStream_t>(stream));
}

// Banks of a checkpoint-select call: inside the pool, distinct, one launch of rows.
static int check_banks(const gdn_dims *dims, int32_t n_rows, int32_t n_slots, const int32_t *bank) {
  if (n_rows > kRowsPerLaunch) return GDN_E_RANGE;
  const int64_t per_bank = dims->k_max + 1;
  for (int32_t r = 0; r < n_rows; ++r)
    if (bank[r] < 0 || (int64_t(bank[r]) + 1) * per_bank > n_slots) return GDN_E_RANGE;
  std::vector<int32_t> sorted(bank, bank + n_rows);
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return GDN_E_ALIAS;
  return GDN_OK;
}

// Checkpoint-select verification, optionally committing the previous window first
// (prev_* non-null): both forms are checked in full before the one launch.
static int verify_select(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                  const int32_t *prev_row_tokens, const int32_t *prev_bank, const int32_t *accepted,
                  const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a, const float *b,
                  const float *A_log, const float *dt_bias, float *state_pool, int32_t n_slots,
                  int32_t *slot_table, const int32_t *bank, uint16_t *o, uint32_t *status, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens || !slot_table || !bank || !status) return GDN_E_NULL;
  if ((rc = check_tokens(q, k, v, a, b, A_log, dt_bias, o))) return rc;
  if (!state_pool) return GDN_E_NULL;
  if (!aligned(state_pool, 16) || !aligned(slot_table, 4) || !aligned(status, 4)) return GDN_E_ALIGN;
  if (accepted && !aligned(accepted, 4)) return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r)
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
  if ((rc = check_banks(dims, n_rows, n_slots, bank))) return rc;
  if (prev_bank) {
    for (int32_t r = 0; r < n_rows; ++r)
      if (prev_row_tokens[r] < 1 || prev_row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
    if ((rc = check_banks(dims, n_rows, n_slots, prev_bank))) return rc;
    // the committed checkpoint must not be a slot this window writes
    for (int32_t r = 0; r < n_rows; ++r)
      for (int32_t j = 0; j < n_rows; ++j)
        if (prev_bank[r] == bank[j]) return GDN_E_ALIAS;
  }
  const std::vector<int64_t> cu = prefix(n_rows, row_tokens);
  if (cu.back() > INT32_MAX) return GDN_E_RANGE;  // token offsets are int32
  const Sizes s = sizes_of(dims);
  const size_t pool_b = size_t(n_slots) * s.row_floats * 4;
  const size_t o_b = size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2;
  if (overlap(o, o_b, state_pool, pool_b) || overlap(slot_table, size_t(n_rows) * 4, state_pool, pool_b) ||
      overlap(status, size_t((n_rows + 31) / 32) * 4, state_pool, pool_b) ||
      (accepted && overlap(accepted, size_t(n_rows) * 4, state_pool, pool_b)))
    return GDN_E_ALIAS;

  std::vector<int32_t> rows(static_cast<size_t>(n_rows));
  for (int32_t r = 0; r < n_rows; ++r) rows[r] = r;
  gdn::RecurrentArgs proto;
  fill_common(proto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, state_pool, state_pool, o);
  proto.src_table = slot_table;
  proto.status = status;
  proto.n_slots = n_slots;
  if (prev_bank) {  // one launch holds every row of a select call (n_rows <= 64, checked above)
    proto.prev_accepted = accepted;
    for (int32_t r = 0; r < n_rows; ++r) {
      proto.prev_bank[r] = prev_bank[r];
      proto.prev_ntok[r] = prev_row_tokens[r];
    }
  }
  return launch_recurrent_rows(dims, proto, rows, cu, row_tokens, nullptr, nullptr, row_tokens, stream, nullptr,
                               nullptr, nullptr, bank);
}


int gdn_verify_window_select(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                             const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                             const float *b, const float *A_log, const float *dt_bias, float *state_pool,
                             int32_t n_slots, const int32_t *slot_table, const int32_t *bank, uint16_t *o,
                             uint32_t *status, void *stream) {
  // without a pending commit the kernel only reads the table
  return verify_select(dims, n_rows, row_tokens, nullptr, nullptr, nullptr, q, k, v, a, b, A_log, dt_bias,
                       state_pool, n_slots, const_cast<int32_t *>(slot_table), bank, o, status,
                       static_cast<hipStream_t>(stream));
}

int gdn_verify_window_select_commit(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                                    const int32_t *prev_row_tokens, const int32_t *prev_bank,
                                    const int32_t *accepted, const uint16_t *q, const uint16_t *k,
                                    const uint16_t *v, const float *a, const float *b, const float *A_log,
                                    const float *dt_bias, float *state_pool, int32_t n_slots,
                                    int32_t *slot_table, const int32_t *bank, uint16_t *o, uint32_t *status,
                                    void *stream) {
  if (n_rows > 0 && (!prev_row_tokens || !prev_bank || !accepted)) return GDN_E_NULL;
  return verify_select(dims, n_rows, row_tokens, prev_row_tokens, prev_bank, accepted, q, k, v, a, b, A_log,
                       dt_bias, state_pool, n_slots, slot_table, bank, o, status,
                       static_cast<hipStream_t>(stream));
}

int gdn_commit_select(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                      const int32_t *accepted, const int32_t *bank, int32_t n_slots, int32_t *slot_table,
                      uint32_t *status, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens || !accepted || !bank || !slot_table || !status) return GDN_E_NULL;
  if (!aligned(accepted, 4) || !aligned(slot_table, 4) || !aligned(status, 4)) return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r)
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
  if ((rc = check_banks(dims, n_rows, n_slots, bank))) return rc;
  gdn::SelectArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.accepted = accepted;
  sa.slot_table = slot_table;
  sa.status = status;
  sa.ck_slots = dims->k_max + 1;
  sa.n_rows = n_rows;
  for (int32_t r = 0; r < n_rows; ++r) {
    sa.ntok[r] = row_tokens[r];
    sa.bank[r] = bank[r];
  }
  return gdn::launch_select(sa, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK : GDN_E_HIP;
}

int gdn_commit_accepted(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                        const float *ckpt, const int32_t *accepted, float *state_pool,
                        int32_t n_slots, const int32_t *dst_slot, uint32_t *status,
                        void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens || !ckpt || !accepted || !state_pool || !dst_slot || !status) return GDN_E_NULL;
  if (!aligned(ckpt, 16) || !aligned(state_pool, 16) || !aligned(accepted, 4) ||
      !aligned(status, 4))
    return GDN_E_ALIGN;
  for (int32_t r = 0; r < n_rows; ++r) {
    if (row_tokens[r] < 1 || row_tokens[r] > dims->k_max + 1) return GDN_E_RANGE;
    if (dst_slot[r] < 0) return GDN_E_RANGE;
  }
  if ((rc = check_slots(n_rows, n_slots, nullptr, dst_slot))) return rc;
  const Sizes s = sizes_of(dims);
  if (overlap(ckpt, size_t(n_rows) * s.ck_row_floats * 4, state_pool,
              size_t(n_slots) * s.row_floats * 4))
    return GDN_E_ALIAS;

  for (int32_t r0 = 0; r0 < n_rows; r0 += kRowsPerLaunch) {
    gdn::CommitArgs ca;
    memset(&ca, 0, sizeof(ca));
    const int32_t n = std::min<int32_t>(kRowsPerLaunch, n_rows - r0);
    ca.ckpt = ckpt + size_t(r0) * s.ck_row_floats;
    ca.pool = state_pool;
    ca.accepted = accepted + r0;
    ca.status = status;
    ca.row_floats = int64_t(s.row_floats);
    ca.ck_slots = dims->k_max + 1;
    ca.n_rows = n;
    ca.row_base = r0;
    for (int32_t j = 0; j < n; ++j) {
      ca.ntok[j] = row_tokens[r0 + j];
      ca.dst[j] = dst_slot[r0 + j];
    }
    if (gdn::launch_commit(ca, static_cast<hipStream_t>(stream)) != hipSuccess) return GDN_E_HIP;
  }
  return GDN_OK;
}

int gdn_plan_transaction(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                         int32_t *route) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  if (!row_tokens || !route) return GDN_E_NULL;
  for (int32_t r = 0; r < n_rows; ++r)
    if (row_tokens[r] < 1) return GDN_E_RANGE;
  for (int32_t r = 0; r < n_rows; ++r)
    route[r] = row_tokens[r] <= dims->k_max + 1 ? GDN_ROUTE_RECURRENT : GDN_ROUTE_CHUNKED;
  return GDN_OK;
}

size_t gdn_chunked_workspace_bytes(const gdn_dims *dims, int32_t n_rows,
                                   const int32_t *row_tokens, int32_t chunk) {
  if (check_dims(dims) || n_rows < 0 || chunk != gdn::kChunk) return 0;
  if (n_rows == 0) return 0;
  if (!row_tokens) return 0;
  std::vector<int32_t> rows;
  for (int32_t r = 0; r < n_rows; ++r) {
    if (row_tokens[r] < 1) return 0;
    rows.push_back(r);
  }
  if (!chunk_units_fit(dims, rows, row_tokens)) return 0;
  return chunked_ws_bytes(dims, rows, row_tokens);
}

int gdn_chunked_prefill_with_checkpoints(
    const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens, int32_t chunk,
    const int32_t *n_tail, const uint16_t *q, const uint16_t *k, const uint16_t *v,
    const float *a, const float *b, const float *A_log, const float *dt_bias,
    float *state_pool, int32_t n_slots, const int32_t *src_slot, const int32_t *dst_slot,
    float *ckpt, uint16_t *o, void *workspace, size_t ws_bytes, void *stream) {
  return chunked_prefill(dims, n_rows, row_tokens, chunk, n_tail, q, k, v, a, b, A_log, dt_bias,
                         state_pool, n_slots, src_slot, dst_slot, ckpt, o, workspace, ws_bytes, false,
                         static_cast<hipStream_t>(stream));
}

int gdn_chunked_prefill_with_checkpoints_static(
    const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens, int32_t chunk,
    const int32_t *n_tail, const uint16_t *q, const uint16_t *k, const uint16_t *v,
    const float *a, const float *b, const float *A_log, const float *dt_bias,
    float *state_pool, int32_t n_slots, const int32_t *src_slot, const int32_t *dst_slot,
    float *ckpt, uint16_t *o, void *stream) {
  return chunked_prefill(dims, n_rows, row_tokens, chunk, n_tail, q, k, v, a, b, A_log, dt_bias,
                         state_pool, n_slots, src_slot, dst_slot, ckpt, o, nullptr, 0, true,
                         static_cast<hipStream_t>(stream));
}

int gdn_run_transaction(const gdn_dims *dims, int32_t n_rows, const int32_t *row_tokens,
                        const int32_t *n_ckpt, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, const float *a, const float *b, const float *A_log,
                        const float *dt_bias, float *state_pool, int32_t n_slots,
                        const int32_t *src_slot, const int32_t *dst_slot, float *ckpt,
                        uint16_t *o, void *workspace, size_t ws_bytes, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_rows < 0 || n_slots < 0) return GDN_E_RANGE;
  if (n_rows == 0) return GDN_OK;
  std::vector<int64_t> cu;
  if ((rc = check_packed(dims, n_rows, row_tokens, n_ckpt, q, k, v, a, b, A_log, dt_bias,
                         state_pool, n_slots, src_slot, dst_slot, ckpt, o, cu)))
    return rc;
  std::vector<int32_t> route(static_cast<size_t>(n_rows));
  if ((rc = gdn_plan_transaction(dims, n_rows, row_tokens, route.data()))) return rc;
  std::vector<int32_t> rec, chk;
  for (int32_t r = 0; r < n_rows; ++r) (route[r] == GDN_ROUTE_RECURRENT ? rec : chk).push_back(r);
  if (!chunk_units_fit(dims, chk, row_tokens)) return GDN_E_RANGE;
  const Sizes s = sizes_of(dims);
  const size_t need = chunked_ws_bytes(dims, chk, row_tokens);
  if ((rc = check_workspace(workspace, ws_bytes, need, state_pool, size_t(n_slots) * s.row_floats * 4,
                            ckpt, ckpt ? size_t(n_rows) * s.ck_row_floats * 4 : 0, o,
                            size_t(cu[n_rows]) * size_t(dims->n_v_heads) * size_t(dims->d_v) * 2)))
    return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  gdn::RecurrentArgs rproto;
  fill_common(rproto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, state_pool, ckpt, o);
  if ((rc = launch_recurrent_rows(dims, rproto, rec, cu, row_tokens, src_slot, dst_slot, n_ckpt, st)))
    return rc;
  gdn::ChunkArgs cproto;
  fill_chunk_common(cproto, dims, q, k, v, a, b, A_log, dt_bias, state_pool, ckpt, o, workspace);
  return launch_chunked_rows(dims, cproto, chk, cu, row_tokens, n_ckpt, src_slot, dst_slot, st);
}

}  // extern "C"
