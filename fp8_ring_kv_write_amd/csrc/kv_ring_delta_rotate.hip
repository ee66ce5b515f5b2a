// kv_ring_delta_rotate: move every cached key by `delta` positions when positions reset
// (Runway Characters abstract: a delta rotation of the cache on position reset, instead of
// rebuilding it).  Because rotation by p then by delta equals rotation by p + delta, the
// rotated keys are the keys at their new positions.
//
// Keys are dequantised (decode * slot scale, float32), rotated by the delta table (float32,
// every operation rounded), and requantised with one new per-head scale over all valid
// slots.  One launch, one read of the K codes: a work-group takes one 128-slot tile of one head
// (each thread 4 (head_dim 128) or 2 (64) 16-byte units of 16 channels, all of its loads in
// flight at once), rotates it in registers, meets the head's other work-groups (head_sync) for
// the new absmax, and rewrites its codes and scales.  V is untouched.
// The meeting needs all of a head's work-groups on the GPU at once (head_sync), so a head takes
// at most kMaxRotGroups of them: a ring of more tiles per head gives each work-group a run of
// consecutive tiles, rotated once for the absmax and, after the meeting, read and rotated again
// to be encoded (two reads of the K codes).

#include "kvring_common.hpp"
#include "kvring_internal.hpp"

namespace kvring {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRotGroups = 1024;   // work-groups per head, at most (128 per XCD)

struct RotGeom {
  int32_t head, filled, slots, heads, nchunks;
  int32_t tpw;   // tiles per work-group: 1, or more for rings of more than kMaxRotGroups tiles
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

// grid = (work-groups per head, heads), the first varying fastest (a head's work-groups are
// consecutive, as head_sync requires): g.tpw consecutive tiles of one head (normally one),
// rotated, requantised with the head's new scale.
typedef uint32_t nt4_t __attribute__((ext_vector_type(4)));

// The rotated keys of a thread's units, and their absmax over the valid units.
template <int D>
__device__ inline float rotate_units(const Units<D>& x, const DeltaTable& tab, float (&v)[kUnitsPerThread<D>][16]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kUnitsPerThread<D>; ++j) {
    dequant_rotate<16>(x.w[j], x.scale[j], tab, 8 * x.q[j], v[j]);
    if (!x.ok[j]) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[j][e]));
  }
  return m;
}

// Codes and scales of a thread's valid units, encoded with the head's inverse scale.
template <int D>
__device__ inline void store_units(uint8_t* tile, float* srow, const Units<D>& x,
                                   const float (&v)[kUnitsPerThread<D>][16], float scale, float inv) {
#pragma unroll
  for (int j = 0; j < kUnitsPerThread<D>; ++j) {
    if (!x.ok[j]) continue;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = e4m3x4(v[j][4 * e] * inv, v[j][4 * e + 1] * inv, v[j][4 * e + 2] * inv, v[j][4 * e + 3] * inv);
    const int p = j * kThreads + int(threadIdx.x);
    // stored non-temporal: streamed to memory rather than held in L2 until the launch ends
    __builtin_nontemporal_store(nt4_t{o[0], o[1], o[2], o[3]}, reinterpret_cast<nt4_t*>(tile + p * 16));
    if (x.q[j] == 0) __builtin_nontemporal_store(scale, &srow[x.slot[j]]);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void rotate_requantize(
    uint8_t* __restrict__ kc, float* __restrict__ k_scale, RotGeom g, DeltaTable tab, void* sync) {
  __shared__ float sl[10];
  const int h = blockIdx.y;
  char* rec = sync_record(sync, 0, h);
  const unsigned gen = head_sync_generation(rec);
  uint8_t* kh = kc + (int64_t)h * g.tiles * kTile * D;
  float* srow = k_scale + (int64_t)h * g.slots;
  float unused = 0.0f;
  float v[kUnitsPerThread<D>][16];
  if (g.tpw == 1) {   // one tile, held in registers across the meeting
    const int t = blockIdx.x;
    Units<D> x;
    load_units<D>(kh + (int64_t)t * kTile * D, srow, t, g, x);
    float m = rotate_units<D>(x, tab, v);
    // the head's new absmax; every thread's reads of the old slot scales (above) precede its
    // barrier, and so the writes below
    head_sync<kThreads>(rec, gen, sync_error_word(sync), int(gridDim.x), false, m, unused, sl);
    float scale, inv;
    scale_from_absmax(m, scale, inv);
    store_units<D>(kh + (int64_t)t * kTile * D, srow, x, v, scale, inv);
    return;
  }
  // a run of tiles: the absmax over them, the meeting, then each tile read, rotated and
  // encoded again (no other work-group touches these tiles, so the second read sees the codes
  // and scales the first did)
  const int64_t t0 = (int64_t)blockIdx.x * g.tpw;
  const int64_t t1 = min<int64_t>(t0 + g.tpw, g.tiles);
  float m = 0.0f;
  for (int64_t t = t0; t < t1; ++t) {
    Units<D> x;
    load_units<D>(kh + t * kTile * D, srow, int(t), g, x);
    m = __builtin_fmaxf(m, rotate_units<D>(x, tab, v));
  }
  head_sync<kThreads>(rec, gen, sync_error_word(sync), int(gridDim.x), false, m, unused, sl);
  float scale, inv;
  scale_from_absmax(m, scale, inv);
  for (int64_t t = t0; t < t1; ++t) {
    Units<D> x;
    load_units<D>(kh + t * kTile * D, srow, int(t), g, x);
    rotate_units<D>(x, tab, v);
    store_units<D>(kh + t * kTile * D, srow, x, v, scale, inv);
  }
}

}  // namespace

int64_t rotate_workspace_floats(int32_t, int32_t) { return kSyncBytes / 4; }

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
  g.tpw = int((g.tiles + kMaxRotGroups - 1) / kMaxRotGroups);
  dim3 grid(int((g.tiles + g.tpw - 1) / g.tpw), r.heads);
  if (r.head_dim == 128)
    hipLaunchKernelGGL(rotate_requantize<128>, grid, dim3(kThreads), 0, stream, r.k, r.k_scale, g, tab, ws);
  else
    hipLaunchKernelGGL(rotate_requantize<64>, grid, dim3(kThreads), 0, stream, r.k, r.k_scale, g, tab, ws);
  return hipGetLastError();
}

}  // namespace kvring
