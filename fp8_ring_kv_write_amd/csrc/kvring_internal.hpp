// Internal launch interface between the C ABI (kvring_abi.hip) and the kernels.
// Arguments have been validated by the caller; every function only enqueues work on
// `stream` and returns the HIP status of the launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvring.h"

namespace kvring {

// Floats of workspace each operation needs (see kv_ring_workspace_bytes).
int64_t write_workspace_floats(int32_t heads, int32_t n);
int64_t rotate_workspace_floats(int32_t heads, int32_t slots);
int64_t attention_workspace_floats(int32_t heads, int32_t slots, int32_t head_dim, int32_t nq);

// kv_ring_write_static: the write's scratch (its synchronisation records) in a static device
// array of this many floats per GPU.
constexpr int64_t kWriteStaticScratchFloats = 196672;   // 768 KiB + 256 bytes
constexpr int kMaxDevices = 64;
// Device address of this device's copy of that array (looked up once per device).
hipError_t write_static_scratch(float** out);

hipError_t launch_write(const kv_ring_desc& r, const uint16_t* k_new, const uint16_t* v_new,
                        int32_t n, int32_t start_slot, int64_t pos0, const float* rope,
                        float* ws, hipStream_t stream);

struct DeltaTable {  // cos/sin of delta * theta_i for i < head_dim/2, float32
  float cs[64][2];
};

hipError_t launch_delta_rotate(const kv_ring_desc& r, int32_t ring_head, int32_t filled,
                               const DeltaTable& tab, float* ws, hipStream_t stream);

// Every workspace starts with the per-head synchronisation records (kSyncBytes, see head_sync):
// the write, the rotation and the query preparation meet there, and each call leaves them ready
// for the next.
// The attention's workspace follows them with the split rows' partial results and the queries
// quantised for the QK product with their per-head scales.
struct AttnWorkspace {
  float* part_o;      // [rows][8][128][head_dim] halves (the split rows' normalised outputs)
  float* part_ml;     // [rows][8][128][2]
  uint8_t* q_codes;   // [heads * ceil(nq/128)][8][64][32]
  float* q_scale;     // [heads]
};
AttnWorkspace attention_workspace(float* ws, int32_t heads, int32_t slots, int32_t head_dim,
                                  int32_t nq);

// With q_ready an earlier launch on the stream has written the quantised queries (and scales)
// into the workspace; otherwise the attention prepares them first (one more launch).
hipError_t launch_attention(const kv_ring_desc& r, int32_t ring_head, int32_t filled,
                            const uint16_t* q, int32_t nq, int64_t q_pos0, const float* rope,
                            float softmax_scale, uint16_t* out, float* lse, float* ws,
                            bool q_ready, hipStream_t stream);

// Query preparation: rotation, the per-head absmax and quantisation (one launch; sync is the
// workspace, whose records of slot 1 it uses).
hipError_t launch_q_prep(const uint16_t* q, int32_t nq, int32_t heads, int32_t head_dim,
                         int64_t q_pos0, const float* rope, void* sync, uint8_t* codes,
                         float* scale, hipStream_t stream);

// Write followed by the query preparation, in one launch (records of slots 0 and 1 of ws).
hipError_t launch_write_and_q_prep(const kv_ring_desc& r, const uint16_t* k_new,
                                   const uint16_t* v_new, int32_t n, int32_t start_slot,
                                   int64_t pos0, const uint16_t* q, int32_t nq, int64_t q_pos0,
                                   const float* rope, float* ws, uint8_t* codes,
                                   float* scale, hipStream_t stream);

void set_attention_events(void* before, void* after);

hipError_t launch_fp8_encode(const float* x, uint8_t* out, int64_t n, hipStream_t stream);

}  // namespace kvring
