// C ABI of the FP8 ring KV cache: argument checks, host-side tables, workspace sizing, and
// dispatch to the kernels.  No entry point allocates device memory or synchronises.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/kvring.h"
#include "kvring_common.hpp"
#include "kvring_internal.hpp"

namespace kvring {
// kv_window.hip
hipError_t launch_window_advance(const void* src, void* dst, const void* fresh, int32_t window,
                                 int32_t n, int64_t row_bytes, hipStream_t stream);
}  // namespace kvring

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_ring(const kv_ring_desc* r) {
  if (!r) return KV_RING_ERR_NULL;
  if (!r->k || !r->v || !r->k_scale || !r->v_scale) return KV_RING_ERR_NULL;
  if (r->heads < 1 || r->heads > kvring::kMaxHeads || r->slots < 1 || r->slots > (1 << 20)) return KV_RING_ERR_SHAPE;
  if (r->head_dim != 64 && r->head_dim != 128) return KV_RING_ERR_SHAPE;
  if (!aligned(r->k, 16) || !aligned(r->v, 16) || !aligned(r->k_scale, 4) || !aligned(r->v_scale, 4))
    return KV_RING_ERR_ALIGN;
  return KV_RING_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return KV_RING_OK;
  if (!ws) return KV_RING_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return KV_RING_ERR_ALIGN;
  if (have < need) return KV_RING_ERR_WORKSPACE;
  return KV_RING_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? KV_RING_OK : KV_RING_ERR_LAUNCH; }

double rope_theta(int32_t i, int32_t head_dim, double base) {
  return std::pow(base, -(2.0 * i) / (double)head_dim);
}

// Three-axis positions: the head_dim/2 pairs are cut into contiguous bands (frame, row,
// column), each a 1-D rotary embedding of dimension 2 * pairs on its own coordinate.  Fills,
// for every pair, its axis and its frequency; `bands` NULL gives row and column floor(P/3)
// pairs each and the frame the rest.
int band_frequencies(const int32_t* bands, int32_t head_dim, double base, int32_t axis[64],
                     double theta[64]) {
  const int32_t p = head_dim / 2;
  int32_t cut[3] = {p - 2 * (p / 3), p / 3, p / 3};
  if (bands) {
    for (int b = 0; b < 3; ++b) {
      if (bands[b] < 0 || bands[b] > p) return KV_RING_ERR_SHAPE;
      cut[b] = bands[b];
    }
    if (cut[0] + cut[1] + cut[2] != p) return KV_RING_ERR_SHAPE;
  }
  int32_t k = 0;
  for (int32_t b = 0; b < 3; ++b)
    for (int32_t j = 0; j < cut[b]; ++j, ++k) {
      axis[k] = b;
      theta[k] = rope_theta(j, 2 * cut[b], base);
    }
  return KV_RING_OK;
}

int check_delta_rotate(const kv_ring_desc* ring, int32_t ring_head, int32_t filled, double rope_base,
                       void* workspace, size_t workspace_bytes) {
  int st = check_ring(ring);
  if (st) return st;
  if (ring_head < 0 || ring_head >= ring->slots || filled < 0 || filled > ring->slots) return KV_RING_ERR_RANGE;
  if (!(rope_base > 0.0)) return KV_RING_ERR_SHAPE;
  return check_workspace(workspace, workspace_bytes,
                         kv_ring_workspace_bytes(KV_RING_OP_DELTA_ROTATE, ring->heads, ring->slots,
                                                 ring->head_dim, 0));
}

bool delta_in_range(int64_t d) { return d > -(int64_t(1) << 31) && d < (int64_t(1) << 31); }

}  // namespace

extern "C" {

int64_t kv_ring_codes_bytes(int32_t heads, int32_t slots, int32_t head_dim) {
  if (heads < 1 || slots < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  return (int64_t)heads * kvring::tile_count(slots) * kvring::kTile * head_dim;
}

int64_t kv_ring_k_offset(int64_t slot, int32_t channel, int32_t head_dim) {
  if (slot < 0 || (head_dim != 64 && head_dim != 128) || channel < 0 || channel >= head_dim) return -1;
  return kvring::k_code_offset(slot, channel & ~15, head_dim) + (channel & 15);
}

int64_t kv_ring_v_offset(int64_t slot, int32_t channel, int32_t head_dim) {
  if (slot < 0 || (head_dim != 64 && head_dim != 128) || channel < 0 || channel >= head_dim) return -1;
  return kvring::v_code_offset(slot & ~int64_t(15), channel, head_dim) + (slot & 15);
}


int kv_ring_rope_table(float* host_out, int64_t n_pos, int32_t head_dim, double base) {
  if (!host_out) return KV_RING_ERR_NULL;
  if (n_pos < 1 || (head_dim != 64 && head_dim != 128) || !(base > 0.0)) return KV_RING_ERR_SHAPE;
  const int32_t half = head_dim / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double th = rope_theta(i, head_dim, base);
    for (int64_t p = 0; p < n_pos; ++p) {
      const double ang = (double)p * th;
      host_out[(p * half + i) * 2] = (float)std::cos(ang);
      host_out[(p * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  }
  return KV_RING_OK;
}

size_t kv_ring_workspace_bytes(int32_t op, int32_t heads, int32_t slots, int32_t head_dim, int32_t n) {
  if (heads < 1 || heads > kvring::kMaxHeads || slots < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  switch (op) {
    case KV_RING_OP_WRITE:
      if (n < 1) return 0;
      return sizeof(float) * (size_t)kvring::write_workspace_floats(heads, n);
    case KV_RING_OP_DELTA_ROTATE:
      return sizeof(float) * (size_t)kvring::rotate_workspace_floats(heads, slots);
    case KV_RING_OP_ATTENTION:
      if (n < 0) return 0;
      if (n == 0) return 16;
      return sizeof(float) * (size_t)kvring::attention_workspace_floats(heads, slots, head_dim, n);
    case KV_RING_OP_WRITE_ATTEND:   // n = max(new tokens, queries); the write shares the
      if (n < 1) return 0;          // attention's synchronisation records
      return sizeof(float) * (size_t)kvring::attention_workspace_floats(heads, slots, head_dim, n);
    default:
      return 0;
  }
}

int kv_ring_write(const kv_ring_desc* ring, const void* k_new, const void* v_new, int32_t n,
                  int32_t start_slot, int64_t pos0, const float* rope_table, int64_t rope_n_pos,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_ring(ring);
  if (st) return st;
  if (!k_new || !v_new || !rope_table) return KV_RING_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(rope_table, 16)) return KV_RING_ERR_ALIGN;
  if (n < 1 || n > ring->slots || n > KV_RING_MAX_TOKENS || start_slot < 0 || start_slot >= ring->slots)
    return KV_RING_ERR_RANGE;
  if (pos0 < 0 || rope_n_pos < 1 || pos0 > rope_n_pos - n) return KV_RING_ERR_POSITION;
  st = check_workspace(workspace, workspace_bytes,
                       kv_ring_workspace_bytes(KV_RING_OP_WRITE, ring->heads, ring->slots, ring->head_dim, n));
  if (st) return st;
  return status_of(kvring::launch_write(*ring, static_cast<const uint16_t*>(k_new),
                                        static_cast<const uint16_t*>(v_new), n, start_slot, pos0,
                                        rope_table, static_cast<float*>(workspace),
                                        static_cast<hipStream_t>(stream)));
}

int kv_ring_write_static(const kv_ring_desc* ring, const void* k_new, const void* v_new, int32_t n,
                         int32_t start_slot, int64_t pos0, const float* rope_table, int64_t rope_n_pos,
                         void* stream) {
  int st = check_ring(ring);
  if (st) return st;
  if (!k_new || !v_new || !rope_table) return KV_RING_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(rope_table, 16)) return KV_RING_ERR_ALIGN;
  if (n < 1 || n > ring->slots || n > KV_RING_MAX_TOKENS || start_slot < 0 || start_slot >= ring->slots)
    return KV_RING_ERR_RANGE;
  if (pos0 < 0 || rope_n_pos < 1 || pos0 > rope_n_pos - n) return KV_RING_ERR_POSITION;
  if (kvring::write_workspace_floats(ring->heads, n) > kvring::kWriteStaticScratchFloats)
    return KV_RING_ERR_SCRATCH;
  float* scratch = nullptr;
  if (kvring::write_static_scratch(&scratch) != hipSuccess) return KV_RING_ERR_LAUNCH;
  return status_of(kvring::launch_write(*ring, static_cast<const uint16_t*>(k_new),
                                        static_cast<const uint16_t*>(v_new), n, start_slot, pos0,
                                        rope_table, scratch, static_cast<hipStream_t>(stream)));
}

int kv_ring_delta_rotate(const kv_ring_desc* ring, int32_t ring_head, int32_t filled, int64_t delta,
                         double rope_base, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_delta_rotate(ring, ring_head, filled, rope_base, workspace, workspace_bytes);
  if (st) return st;
  if (!delta_in_range(delta)) return KV_RING_ERR_POSITION;
  // theta_i depends only on (head_dim, base): kept per thread between calls
  thread_local int32_t theta_dim = 0;
  thread_local double theta_base = 0.0, theta[64];
  if (theta_dim != ring->head_dim || theta_base != rope_base) {
    for (int32_t i = 0; i < ring->head_dim / 2; ++i) theta[i] = rope_theta(i, ring->head_dim, rope_base);
    theta_dim = ring->head_dim;
    theta_base = rope_base;
  }
  kvring::DeltaTable tab;
  std::memset(&tab, 0, sizeof(tab));
  for (int32_t i = 0; i < ring->head_dim / 2; ++i) {
    const double ang = (double)delta * theta[i];
    tab.cs[i][0] = (float)std::cos(ang);
    tab.cs[i][1] = (float)std::sin(ang);
  }
  return status_of(kvring::launch_delta_rotate(*ring, ring_head, filled, tab, static_cast<float*>(workspace),
                                               static_cast<hipStream_t>(stream)));
}

int kv_ring_rope_table_3d(float* host_out, const int32_t* positions, int64_t n, int32_t head_dim,
                          const int32_t* band_pairs, double base) {
  if (!host_out || !positions) return KV_RING_ERR_NULL;
  if (n < 1 || (head_dim != 64 && head_dim != 128) || !(base > 0.0)) return KV_RING_ERR_SHAPE;
  int32_t axis[64];
  double theta[64];
  const int st = band_frequencies(band_pairs, head_dim, base, axis, theta);
  if (st) return st;
  const int32_t half = head_dim / 2;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* p = positions + 3 * i;
    float* row = host_out + i * half * 2;
    for (int32_t k = 0; k < half; ++k) {
      if (i > 0 && p[axis[k]] == p[axis[k] - 3]) {   // same coordinate as the previous token
        row[2 * k] = row[2 * k - 2 * half];
        row[2 * k + 1] = row[2 * k + 1 - 2 * half];
        continue;
      }
      const double ang = (double)p[axis[k]] * theta[k];
      row[2 * k] = (float)std::cos(ang);
      row[2 * k + 1] = (float)std::sin(ang);
    }
  }
  return KV_RING_OK;
}

int kv_ring_delta_rotate_3d(const kv_ring_desc* ring, int32_t ring_head, int32_t filled,
                            const int64_t* delta, const int32_t* band_pairs, double rope_base,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_delta_rotate(ring, ring_head, filled, rope_base, workspace, workspace_bytes);
  if (st) return st;
  if (!delta) return KV_RING_ERR_NULL;
  if (!delta_in_range(delta[0]) || !delta_in_range(delta[1]) || !delta_in_range(delta[2]))
    return KV_RING_ERR_POSITION;
  int32_t axis[64];
  double theta[64];
  st = band_frequencies(band_pairs, ring->head_dim, rope_base, axis, theta);
  if (st) return st;
  kvring::DeltaTable tab;
  std::memset(&tab, 0, sizeof(tab));
  for (int32_t k = 0; k < ring->head_dim / 2; ++k) {
    const double ang = (double)delta[axis[k]] * theta[k];
    tab.cs[k][0] = (float)std::cos(ang);
    tab.cs[k][1] = (float)std::sin(ang);
  }
  return status_of(kvring::launch_delta_rotate(*ring, ring_head, filled, tab, static_cast<float*>(workspace),
                                               static_cast<hipStream_t>(stream)));
}

int ring_attention(const kv_ring_desc* ring, int32_t ring_head, int32_t filled, const void* q,
                   int32_t nq, int64_t q_pos0, const float* rope_table, int64_t rope_n_pos,
                   float softmax_scale, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_ring(ring);
  if (st) return st;
  if (nq < 0 || nq > KV_RING_MAX_TOKENS || ring_head < 0 || ring_head >= ring->slots || filled < 0 ||
      filled > ring->slots)
    return KV_RING_ERR_RANGE;
  if (nq == 0) return KV_RING_OK;   // empty tensors may carry NULL data pointers
  if (!q || !rope_table || !out || !lse) return KV_RING_ERR_NULL;
  if (!aligned(q, 16) || !aligned(rope_table, 16) || !aligned(out, 8) || !aligned(lse, 4)) return KV_RING_ERR_ALIGN;
  if (q_pos0 < 0 || rope_n_pos < 1 || q_pos0 > rope_n_pos - nq) return KV_RING_ERR_POSITION;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f)) return KV_RING_ERR_RANGE;
  st = check_workspace(workspace, workspace_bytes,
                       kv_ring_workspace_bytes(KV_RING_OP_ATTENTION, ring->heads, ring->slots, ring->head_dim, nq));
  if (st) return st;
  return status_of(kvring::launch_attention(*ring, ring_head, filled, static_cast<const uint16_t*>(q), nq,
                                            q_pos0, rope_table, softmax_scale, static_cast<uint16_t*>(out),
                                            lse, static_cast<float*>(workspace), false,
                                            static_cast<hipStream_t>(stream)));
}

int kv_ring_write_attend(const kv_ring_desc* ring, const void* k_new, const void* v_new, int32_t n,
                         int32_t start_slot, int64_t pos0, int32_t ring_head, int32_t filled,
                         const void* q, int32_t nq, int64_t q_pos0, const float* rope_table,
                         int64_t rope_n_pos, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_ring(ring);
  if (st) return st;
  // the write's checks
  if (!k_new || !v_new || !rope_table) return KV_RING_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(rope_table, 16)) return KV_RING_ERR_ALIGN;
  if (n < 1 || n > ring->slots || n > KV_RING_MAX_TOKENS || start_slot < 0 || start_slot >= ring->slots)
    return KV_RING_ERR_RANGE;
  if (pos0 < 0 || rope_n_pos < 1 || pos0 > rope_n_pos - n) return KV_RING_ERR_POSITION;
  // the attention's checks
  if (nq < 0 || nq > KV_RING_MAX_TOKENS || ring_head < 0 || ring_head >= ring->slots || filled < 0 ||
      filled > ring->slots)
    return KV_RING_ERR_RANGE;
  if (nq > 0) {
    if (!q || !out || !lse) return KV_RING_ERR_NULL;
    if (!aligned(q, 16) || !aligned(out, 8) || !aligned(lse, 4)) return KV_RING_ERR_ALIGN;
    if (q_pos0 < 0 || q_pos0 > rope_n_pos - nq) return KV_RING_ERR_POSITION;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f)) return KV_RING_ERR_RANGE;
  }
  const int32_t m = n > nq ? n : nq;
  st = check_workspace(workspace, workspace_bytes,
                       kv_ring_workspace_bytes(KV_RING_OP_WRITE_ATTEND, ring->heads, ring->slots, ring->head_dim, m));
  if (st) return st;
  float* ws = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* kn = static_cast<const uint16_t*>(k_new);
  const auto* vn = static_cast<const uint16_t*>(v_new);
  if (nq == 0)
    return status_of(kvring::launch_write(*ring, kn, vn, n, start_slot, pos0, rope_table, ws, s));
  const kvring::AttnWorkspace aw =
      kvring::attention_workspace(ws, ring->heads, ring->slots, ring->head_dim, nq);
  hipError_t e = kvring::launch_write_and_q_prep(*ring, kn, vn, n, start_slot, pos0,
                                                 static_cast<const uint16_t*>(q), nq, q_pos0,
                                                 rope_table, ws, aw.q_codes, aw.q_scale, s);
  if (e != hipSuccess) return KV_RING_ERR_LAUNCH;
  return status_of(kvring::launch_attention(*ring, ring_head, filled, static_cast<const uint16_t*>(q), nq,
                                            q_pos0, rope_table, softmax_scale, static_cast<uint16_t*>(out),
                                            lse, ws, true, s));
}

int kv_ring_sync_status(const void* workspace, void* stream) {
  if (!workspace) return KV_RING_ERR_NULL;
  if (!aligned(workspace, 16)) return KV_RING_ERR_ALIGN;
  int word = 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int* src = kvring::sync_error_word(const_cast<void*>(workspace));
  if (hipMemcpyAsync(&word, src, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess) return KV_RING_ERR_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return KV_RING_ERR_LAUNCH;
  return word == 0 ? KV_RING_OK : KV_RING_ERR_SYNC;
}

int kv_ring_fp8_encode(const float* x, uint8_t* out, int64_t n, void* stream) {
  if (n < 0) return KV_RING_ERR_RANGE;
  if (n == 0) return KV_RING_OK;
  if (!x || !out) return KV_RING_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out, 16)) return KV_RING_ERR_ALIGN;
  return status_of(kvring::launch_fp8_encode(x, out, n, static_cast<hipStream_t>(stream)));
}

int kv_window_advance(const void* src, void* dst, const void* fresh, int32_t window, int32_t n,
                      int64_t row_bytes, void* stream) {
  if (window < 1 || n < 0 || n > window) return KV_RING_ERR_RANGE;
  if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > (int64_t(1) << 30)) return KV_RING_ERR_SHAPE;
  if (!dst || (n < window && !src) || (n > 0 && !fresh)) return KV_RING_ERR_NULL;
  if (!aligned(dst, 16) || (src && !aligned(src, 16)) || (fresh && !aligned(fresh, 16)))
    return KV_RING_ERR_ALIGN;
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), d1 = d0 + uintptr_t(window) * uintptr_t(row_bytes);
  auto overlaps = [&](const void* p, int64_t rows) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + uintptr_t(rows) * uintptr_t(row_bytes);
    return rows > 0 && a0 < d1 && d0 < a1;
  };
  if (overlaps(src, window - n) || overlaps(fresh, n)) return KV_RING_ERR_RANGE;
  return status_of(kvring::launch_window_advance(src, dst, fresh, window, n, row_bytes,
                                                 static_cast<hipStream_t>(stream)));
}

int kv_ring_set_attention_events(void* before, void* after) {
  if (before && after)
    kvring::set_attention_events(before, after);
  else
    kvring::set_attention_events(nullptr, nullptr);
  return KV_RING_OK;
}

const char* kv_ring_status_string(int status) {
  switch (status) {
    case KV_RING_OK: return "ok";
    case KV_RING_ERR_NULL: return "a required pointer is NULL";
    case KV_RING_ERR_ALIGN: return "a pointer is not aligned as documented";
    case KV_RING_ERR_SHAPE: return "heads, slots or head_dim unsupported";
    case KV_RING_ERR_RANGE: return "n, start_slot, ring_head, filled or nq out of range";
    case KV_RING_ERR_POSITION: return "a position falls outside the rotary table";
    case KV_RING_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_RING_ERR_LAUNCH: return "a kernel launch failed";
    case KV_RING_ERR_SCRATCH: return "the call needs more than the library's static scratch";
    case KV_RING_ERR_SYNC: return "a synchronisation wait exceeded its bound";
    default: return "unknown status";
  }
}

}  // extern "C"
