// kv_ring_delta_rotate: move every cached key by `delta` positions when positions reset
// (Runway Characters abstract: a delta rotation of the cache on position reset, instead of
// rebuilding it).  Because rotation by p then by delta equals rotation by p + delta, the
// rotated keys are the keys at their new positions.
//
// Keys are dequantised (decode * slot scale, float32), rotated by the delta table (float32,
// every operation rounded), and requantised with one new per-head scale over all valid
// slots.  Two passes over the K codes (the second mostly from L2 / infinity cache), no
// atomics: pass 1 writes per-(head, chunk) absmax partials, pass 2 reduces them and rewrites
// codes and scales.  V is untouched.

#include "kvring_common.hpp"
#include "kvring_internal.hpp"

namespace kvring {

namespace {

constexpr int kThreads = 256;

struct RotGeom {
  int32_t head, filled, slots, heads, nchunks;
  int64_t tiles;
};

// Dequantise and rotate CPT channels of one slot.  `codes` holds CPT bytes.
template <int CPT>
__device__ inline void dequant_rotate(const uint32_t (&codes)[CPT / 4], float scale,
                                      const DeltaTable& tab, int pair0, float (&x)[CPT]) {
#pragma unroll
  for (int j = 0; j < CPT / 4; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * j + e] = e4m3_decode(codes[j], e) * scale;
  }
#pragma unroll
  for (int p = 0; p < CPT / 2; ++p) {
    const float c = tab.cs[pair0 + p][0], s = tab.cs[pair0 + p][1];
    const float xe = x[2 * p], xo = x[2 * p + 1];
    x[2 * p] = xe * c - xo * s;
    x[2 * p + 1] = xe * s + xo * c;
  }
}

template <int CPT>
__device__ inline void load_codes(const uint8_t* p, uint32_t (&w)[CPT / 4]) {
  if constexpr (CPT == 16) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  }
}

// grid = (chunks of 32 slots over the whole ring, heads)
template <int D>
__global__ __launch_bounds__(kThreads) void rotate_absmax_partials(
    const uint8_t* __restrict__ kc, const float* __restrict__ k_scale, RotGeom g, DeltaTable tab,
    float* __restrict__ partial) {
  constexpr int CPT = D / 8;
  __shared__ float red[4];
  const int chunk = blockIdx.x, h = blockIdx.y;
  const int slot = chunk * kChunk + (threadIdx.x >> 3), cg = threadIdx.x & 7;
  float m = 0.0f;
  if (slot_valid(slot, g.head, g.filled, g.slots)) {
    uint32_t w[CPT / 4];
    load_codes<CPT>(kc + (int64_t)h * g.tiles * kTile * D + k_code_offset(slot, (cg * CPT) & ~15, D) +
                        ((cg * CPT) & 15), w);
    float x[CPT];
    dequant_rotate<CPT>(w, k_scale[(int64_t)h * g.slots + slot], tab, cg * (CPT / 2), x);
#pragma unroll
    for (int j = 0; j < CPT; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(x[j]));
  }
  m = block_max_256(m, red);
  if (threadIdx.x == 0) partial[(int64_t)h * g.nchunks + chunk] = m;
}

template <int D>
__global__ __launch_bounds__(kThreads) void rotate_requantize(
    uint8_t* __restrict__ kc, float* __restrict__ k_scale, RotGeom g, DeltaTable tab,
    const float* __restrict__ partial) {
  constexpr int CPT = D / 8;
  __shared__ float red[4];
  const int chunk = blockIdx.x, h = blockIdx.y;
  float a = 0.0f;
  for (int j = threadIdx.x; j < g.nchunks; j += kThreads)
    a = __builtin_fmaxf(a, partial[(int64_t)h * g.nchunks + j]);
  a = block_max_256(a, red);
  float scale, inv;
  scale_from_absmax(a, scale, inv);

  const int slot = chunk * kChunk + (threadIdx.x >> 3), cg = threadIdx.x & 7;
  if (!slot_valid(slot, g.head, g.filled, g.slots)) return;
  uint8_t* p = kc + (int64_t)h * g.tiles * kTile * D + k_code_offset(slot, (cg * CPT) & ~15, D) +
               ((cg * CPT) & 15);
  uint32_t w[CPT / 4];
  load_codes<CPT>(p, w);
  float* sp = k_scale + (int64_t)h * g.slots + slot;
  float x[CPT];
  dequant_rotate<CPT>(w, *sp, tab, cg * (CPT / 2), x);
#pragma unroll
  for (int j = 0; j < CPT / 4; ++j)
    w[j] = e4m3x4(x[4 * j] * inv, x[4 * j + 1] * inv, x[4 * j + 2] * inv, x[4 * j + 3] * inv);
  // every thread of the slot has read its scale before any of them may overwrite it: the
  // 8 threads of a slot are consecutive lanes of one wavefront and execute in lock step, but
  // make the ordering explicit anyway
  __builtin_amdgcn_wave_barrier();
  if constexpr (CPT == 16) {
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  }
  if (cg == 0) *sp = scale;
}

}  // namespace

int64_t rotate_workspace_floats(int32_t heads, int32_t slots) {
  return (int64_t)heads * ((slots + kChunk - 1) / kChunk);
}

hipError_t launch_delta_rotate(const kv_ring_desc& r, int32_t ring_head, int32_t filled,
                               const DeltaTable& tab, float* ws, hipStream_t stream) {
  if (filled == 0) return hipSuccess;
  RotGeom g;
  g.head = ring_head;
  g.filled = filled;
  g.slots = r.slots;
  g.heads = r.heads;
  g.nchunks = (r.slots + kChunk - 1) / kChunk;
  g.tiles = tile_count(r.slots);
  dim3 grid(g.nchunks, r.heads);
  if (r.head_dim == 128)
    hipLaunchKernelGGL(rotate_absmax_partials<128>, grid, dim3(kThreads), 0, stream, r.k,
                       r.k_scale, g, tab, ws);
  else
    hipLaunchKernelGGL(rotate_absmax_partials<64>, grid, dim3(kThreads), 0, stream, r.k,
                       r.k_scale, g, tab, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (r.head_dim == 128)
    hipLaunchKernelGGL(rotate_requantize<128>, grid, dim3(kThreads), 0, stream, r.k, r.k_scale, g,
                       tab, ws);
  else
    hipLaunchKernelGGL(rotate_requantize<64>, grid, dim3(kThreads), 0, stream, r.k, r.k_scale, g,
                       tab, ws);
  return hipGetLastError();
}

}  // namespace kvring
