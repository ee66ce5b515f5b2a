// kv_ring_delta_rotate: move every cached key by `delta` positions when positions reset
// (Runway Characters abstract: a delta rotation of the cache on position reset, instead of
// rebuilding it).  Because rotation by p then by delta equals rotation by p + delta, the
// rotated keys are the keys at their new positions.
//
// Keys are dequantised (decode * slot scale, float32), rotated by the delta table (float32,
// every operation rounded), and requantised with one new per-head scale over all valid
// slots.  Two passes over the K codes (the second mostly from L2 / infinity cache), no
// atomics: pass 1 writes per-(head, tile) absmax partials, pass 2 reduces them and rewrites
// codes and scales.  A work-group takes one 128-slot tile of one head, each thread 4 (head_dim
// 128) or 2 (64) 16-byte units of 16 channels with all of its loads in flight at once.  V is
// untouched.

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

// Unit p (16 bytes) of a K tile -> tile slot u and channel chunk q (channels 16q .. 16q+15),
// per the tile layout (k_code_offset).
template <int D>
__device__ inline void unit_slot(int p, int& u, int& q) {
  constexpr int G = D / 32;
  const int li = p & 15, rest = p >> 4, g = rest % G, rb = rest / G;
  u = 32 * (li >> 2) + 4 * (rb >> 1) + (li & 3);
  q = 2 * g + (rb & 1);
}

// Units handled by one thread: a work-group of kThreads takes one 128-slot tile of one head.
template <int D>
constexpr int kUnitsPerThread = (kTile * D / 16) / kThreads;

// Loads of a thread's units: codes (16 bytes each) and the scale of each unit's slot, all
// issued before any is used.
template <int D>
struct Units {
  uint32_t w[kUnitsPerThread<D>][4];
  float scale[kUnitsPerThread<D>];
  int q[kUnitsPerThread<D>], slot[kUnitsPerThread<D>];
  bool ok[kUnitsPerThread<D>];
};

template <int D>
__device__ inline void load_units(const uint8_t* tile, const float* srow, int t, const RotGeom& g,
                                  Units<D>& x) {
#pragma unroll
  for (int j = 0; j < kUnitsPerThread<D>; ++j) {
    const int p = j * kThreads + int(threadIdx.x);
    int u;
    unit_slot<D>(p, u, x.q[j]);
    x.slot[j] = t * kTile + u;
    x.ok[j] = slot_valid(x.slot[j], g.head, g.filled, g.slots);
    uint4 v = make_uint4(0, 0, 0, 0);
    float sc = 0.0f;
    if (x.ok[j]) {
      v = *reinterpret_cast<const uint4*>(tile + p * 16);
      sc = srow[x.slot[j]];
    }
    x.w[j][0] = v.x; x.w[j][1] = v.y; x.w[j][2] = v.z; x.w[j][3] = v.w;
    x.scale[j] = sc;
  }
}

// grid = (tiles, heads): max |rotated key| over the valid slots of one tile of one head.
template <int D>
__global__ __launch_bounds__(kThreads) void rotate_absmax_partials(
    const uint8_t* __restrict__ kc, const float* __restrict__ k_scale, RotGeom g, DeltaTable tab,
    float* __restrict__ partial) {
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y;
  Units<D> x;
  load_units<D>(kc + ((int64_t)h * g.tiles + t) * kTile * D, k_scale + (int64_t)h * g.slots, t, g, x);
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kUnitsPerThread<D>; ++j) {
    if (!x.ok[j]) continue;
    float v[16];
    dequant_rotate<16>(x.w[j], x.scale[j], tab, 8 * x.q[j], v);
#pragma unroll
    for (int e = 0; e < 16; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
  }
  m = block_max_256(m, red);
  if (threadIdx.x == 0) partial[(int64_t)h * g.tiles + t] = m;
}

// grid = (tiles, heads): requantise one tile of one head with the head's new scale.
template <int D>
__global__ __launch_bounds__(kThreads) void rotate_requantize(
    uint8_t* __restrict__ kc, float* __restrict__ k_scale, RotGeom g, DeltaTable tab,
    const float* __restrict__ partial) {
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y;
  uint8_t* tile = kc + ((int64_t)h * g.tiles + t) * kTile * D;
  float* srow = k_scale + (int64_t)h * g.slots;
  Units<D> x;
  load_units<D>(tile, srow, t, g, x);
  // the head's new absmax from the per-tile partials (rings of up to 64 tiles: each wavefront
  // reduces them itself)
  const float a = list_max(partial + (int64_t)h * g.tiles, int(g.tiles), red);
  __syncthreads();   // every thread's reads of the old slot scales precede the writes below
  float scale, inv;
  scale_from_absmax(a, scale, inv);
#pragma unroll
  for (int j = 0; j < kUnitsPerThread<D>; ++j) {
    if (!x.ok[j]) continue;
    float v[16];
    dequant_rotate<16>(x.w[j], x.scale[j], tab, 8 * x.q[j], v);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = e4m3x4(v[4 * e] * inv, v[4 * e + 1] * inv, v[4 * e + 2] * inv, v[4 * e + 3] * inv);
    const int p = j * kThreads + int(threadIdx.x);
    *reinterpret_cast<uint4*>(tile + p * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    if (x.q[j] == 0) srow[x.slot[j]] = scale;
  }
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
  dim3 grid(g.tiles, r.heads);
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
