// kv_ring_write: write-time RoPE + per-head FP8 quantisation of new K/V tokens into the ring
// (Runway Characters abstract: RoPE and FP8 quantisation applied once per write into a ring
// cache; cpdf.ai blog, section "Como rodar 57B em tempo real com batch size 1").
//
// One bandwidth-bound launch, one read of the inputs: each write work-group takes one aligned
// 32-slot chunk of the ring x 1 head, loads its tokens, rotates K, and meets the head's other
// work-groups (head_sync) for the write's absmax of K' and V; then it encodes what it holds in
// registers and stores K and V codes into the tile layout (V transposed).  The attention's
// queries are prepared the same way (rotation, the head's absmax, quantisation in the QK
// product's operand order), in the same launch when the attention follows a write
// (kv_ring_write_attend): by the write's own work-groups when the queries are the new tokens
// (same count and positions, head_dim 128), else by query work-groups beside them.
//
// Arithmetic is float32 with every product and sum rounded separately (the translation
// unit is compiled with -ffp-contract=off) so the codes match the CPU oracle bit for bit.

#include <cstring>
#include <mutex>

#include "kvring_common.hpp"
#include "kvring_internal.hpp"

namespace kvring {

namespace {

constexpr int kThreads = 256;
// The codes and scales are stored non-temporal (streaming: written to memory rather than held
// in L2 for the end of the launch); the attention that follows reads them from memory anyway.
typedef uint32_t nt4_t __attribute__((ext_vector_type(4)));
__device__ inline void store16_nt(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store(nt4_t{a, b, c, d}, reinterpret_cast<nt4_t*>(p));
}

// Load CPT bf16 channels starting at `p` (16-byte aligned) into floats.
template <int CPT>
__device__ inline void load_bf16(const uint16_t* p, float (&x)[CPT]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int j = 0; j < CPT / 8; ++j) {
    uint4 w = q[j];
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * j + 2 * e] = __uint_as_float(ws[e] << 16);
      x[8 * j + 2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
    }
  }
}

template <int CPT>
__device__ inline float absmax(const float (&x)[CPT]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(x[j]));
  return m;
}

struct WriteGeom {
  int32_t n, start, slots, heads;
  int32_t chunk_a0, n_chunks_a;  // first chunk of the run [start, min(start+n, slots))
  int64_t tiles;
  int64_t pos0;
};

struct WriteArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  void* sync;             // the workspace: its per-head records, slot 0
  uint8_t* kc;
  uint8_t* vc;
  float* k_scale;
  float* v_scale;
  WriteGeom g;
  int32_t blocks;         // work-groups of the write (chunks touched); 0: no write
};

// The attention's queries, quantised once per call: rotated at their positions and encoded with
// the head's scale, stored in the order the attention's QK product takes them as its B operand
// (per 128-query row: wavefront w, lane 16g + li -> query 16w + li, channels 32g .. 32g+31).
struct QuantQArgs {
  const uint16_t* q;      // bfloat16 [nq][heads][D]
  void* sync;             // the workspace: its per-head records, slot 1
  uint8_t* codes;         // [heads * qtiles][8][64][32], qtiles even
  float* scale;           // [heads]
  int64_t pos0;
  int32_t nq, qtiles;
  int32_t blocks;         // 2 * qtiles (a work-group takes 64 queries of a row); 0: none (or
                          // prepared by the write's work-groups, see write_chunk)
};

// The write's work-group: one aligned 32-slot chunk of the ring x one head.  With WQ (head_dim
// 128, the queries being the new tokens themselves: same count, same positions) it also prepares
// the queries of its tokens: the rotary rows it loads serve both, and the queries' absmax joins
// the write's exchange (head_sync_pair: the write's record and the queries' record at once).
template <int D, bool WQ>
__device__ inline void write_chunk(const WriteArgs& wa, const QuantQArgs& qa_, const float* __restrict__ rope,
                                   int blk, int h) {
  constexpr int CPT = D / 8;
  static_assert(!WQ || D == 128, "queries with the write: head_dim 128");
  __shared__ float sl[16];
  __shared__ __align__(16) uint8_t vlds[kChunk][D];
  const WriteGeom& g = wa.g;
  const uint16_t* __restrict__ k_new = wa.k_new;
  const uint16_t* __restrict__ v_new = wa.v_new;
  uint8_t* __restrict__ kc = wa.kc;
  uint8_t* __restrict__ vc = wa.vc;
  float* __restrict__ k_scale = wa.k_scale;
  float* __restrict__ v_scale = wa.v_scale;
  const int chunk = blk < g.n_chunks_a ? g.chunk_a0 + blk : blk - g.n_chunks_a;
  char* rec = sync_record(wa.sync, 0, h);
  const unsigned gen = head_sync_generation(rec);
  char* rec_q = WQ ? sync_record(qa_.sync, 1, h) : nullptr;
  const unsigned gen_q = WQ ? head_sync_generation(rec_q) : 0u;

  const int t = threadIdx.x >> 3, cg = threadIdx.x & 7;
  const int slot = chunk * kChunk + t;
  int i = slot - g.start;
  i = i < 0 ? i + g.slots : i;
  const bool mine = slot < g.slots && i < g.n;
  float xk[CPT], xv[CPT], xq[WQ ? CPT : 1];
  float4 tab[CPT / 4];
  if (mine) {
    const int64_t src = ((int64_t)i * g.heads + h) * D + cg * CPT;
    load_bf16<CPT>(k_new + src, xk);
    load_bf16<CPT>(v_new + src, xv);
    if constexpr (WQ) load_bf16<CPT>(qa_.q + src, xq);
    const float4* t4 = reinterpret_cast<const float4*>(rope + ((g.pos0 + i) * (D / 2) + cg * (CPT / 2)) * 2);
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) tab[j] = t4[j];
  }

  // RoPE of K (pairs 2j, 2j+1 of this thread's channels), then the write's per-head absmax of
  // K' and V over every work-group of the head
  float mk = 0.0f, mv = 0.0f, mq = 0.0f;
  if (mine) {
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) {
      const float cs[2][2] = {{tab[j].x, tab[j].y}, {tab[j].z, tab[j].w}};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int p = 2 * j + e;
        const float xe = xk[2 * p], xo = xk[2 * p + 1];
        xk[2 * p] = xe * cs[e][0] - xo * cs[e][1];
        xk[2 * p + 1] = xe * cs[e][1] + xo * cs[e][0];
        if constexpr (WQ) {
          const float qe = xq[2 * p], qo = xq[2 * p + 1];
          xq[2 * p] = qe * cs[e][0] - qo * cs[e][1];
          xq[2 * p + 1] = qe * cs[e][1] + qo * cs[e][0];
        }
      }
    }
    mk = absmax<CPT>(xk);
    mv = absmax<CPT>(xv);
    if constexpr (WQ) mq = absmax<CPT>(xq);
  }
  if constexpr (WQ)
    head_sync_pair<kThreads>(rec, gen, wa.blocks, mk, mv, rec_q, gen_q, mq, sync_error_word(wa.sync), sl);
  else
    head_sync<kThreads>(rec, gen, sync_error_word(wa.sync), wa.blocks, true, mk, mv, sl);
  float sk, ik, sv, iv;
  scale_from_absmax(mk, sk, ik);
  scale_from_absmax(mv, sv, iv);
  if constexpr (WQ) {
    // the queries: query i = token i, channels 16cg .. 16cg + 15 are half of the 32 bytes that
    // lane (g = cg/2, li = i % 16) of wavefront (i % 128) / 16 of 128-query tile i / 128 holds
    float sq, iq;
    scale_from_absmax(mq, sq, iq);
    if (blk == 0 && threadIdx.x == 0) qa_.scale[h] = sq;
    if (mine) {
      uint32_t wq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wq[j] = e4m3x4(xq[4 * j] * iq, xq[4 * j + 1] * iq, xq[4 * j + 2] * iq, xq[4 * j + 3] * iq);
      const int qt = i >> 7, w = (i >> 4) & 7, lane = 16 * (cg >> 1) + (i & 15);
      store16_nt(qa_.codes + ((((int64_t)h * qa_.qtiles + qt) * 8 + w) * 64 + lane) * 32 + 16 * (cg & 1),
                 wq[0], wq[1], wq[2], wq[3]);
    }
    if (blk == 0) {   // the padding queries of the last tiles: zero codes
      const int pad0 = g.n, pad1 = qa_.qtiles * 128;
      for (int e = pad0 * 8 + int(threadIdx.x); e < pad1 * 8; e += kThreads) {
        const int ii = e >> 3, part = e & 7;   // 8 x 16 bytes per query
        const int qt = ii >> 7, w = (ii >> 4) & 7, lane = 16 * (part >> 1) + (ii & 15);
        *reinterpret_cast<uint4*>(qa_.codes + ((((int64_t)h * qa_.qtiles + qt) * 8 + w) * 64 + lane) * 32 +
                                  16 * (part & 1)) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  if (mine) {
    float (&x)[CPT] = xk;
    uint32_t w[CPT / 4];
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j)
      w[j] = e4m3x4(x[4 * j] * ik, x[4 * j + 1] * ik, x[4 * j + 2] * ik, x[4 * j + 3] * ik);
    // channels cg*CPT .. +CPT-1: one 16-byte unit (head_dim 128) or half of one (64)
    uint8_t* dst = kc + (int64_t)h * g.tiles * kTile * D + k_code_offset(slot, (cg * CPT) & ~15, D) +
                   ((cg * CPT) & 15);
    if constexpr (CPT == 16) {
      store16_nt(dst, w[0], w[1], w[2], w[3]);
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    }
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j)
      w[j] = e4m3x4(xv[4 * j] * iv, xv[4 * j + 1] * iv, xv[4 * j + 2] * iv, xv[4 * j + 3] * iv);
    uint32_t* vl = reinterpret_cast<uint32_t*>(&vlds[t][cg * CPT]);
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) vl[j] = w[j];
    if (cg == 0) {
      __builtin_nontemporal_store(sk, &k_scale[(int64_t)h * g.slots + slot]);
      __builtin_nontemporal_store(sv, &v_scale[(int64_t)h * g.slots + slot]);
    }
  }
  __syncthreads();

  // V: transposed.  Work item = (channel d, half r of the chunk): the chunk's slots 16r .. 16r+15
  // of channel d form one 16-byte unit of the tile.
  for (int item = threadIdx.x; item < D * 2; item += kThreads) {
    const int d = item >> 1, r = item & 1;
    const int s0 = chunk * kChunk + 16 * r;
    uint8_t* unit = vc + (int64_t)h * g.tiles * kTile * D + v_code_offset(s0, d, D);
    uint32_t word[4] = {0, 0, 0, 0};
    int nmine = 0;
    bool mine16[16];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int s = s0 + kk;
      int ii = s - g.start;
      ii = ii < 0 ? ii + g.slots : ii;
      mine16[kk] = s < g.slots && ii < g.n;
      nmine += mine16[kk];
      word[kk >> 2] |= uint32_t(vlds[16 * r + kk][d]) << (8 * (kk & 3));
    }
    if (nmine == 16) {
      store16_nt(unit, word[0], word[1], word[2], word[3]);
    } else if (nmine > 0) {   // the write's first or last chunk: only its own slots
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        if (mine16[kk]) unit[kk] = uint8_t(word[kk >> 2] >> (8 * (kk & 3)));
    }
  }
}

// Query quantisation: half a row (64 queries) of one head.  Thread -> (wavefront w of the
// attention's row, lane): the 32 bytes that lane holds as its QK operand.
template <int D>
__device__ inline void quantize_q_half(const QuantQArgs& qa_, const float* __restrict__ rope, int blk,
                                       int h, int heads) {
  __shared__ float sl[10];
  const int qt = blk >> 1, w = 4 * (blk & 1) + (int(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int i = qt * 128 + w * 16 + li;
  const bool live = i < qa_.nq && (D == 128 || g < 2);
  char* rec = sync_record(qa_.sync, 1, h);
  const unsigned gen = head_sync_generation(rec);
  uint4 raw[4];
  float4 tab[8];
  if (live) {
    const uint4* src = reinterpret_cast<const uint4*>(qa_.q + ((int64_t)i * heads + h) * D + 32 * g);
    const float4* t4 = reinterpret_cast<const float4*>(rope + ((qa_.pos0 + i) * (D / 2) + 16 * g) * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = src[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) tab[j] = t4[j];
  }
  // rotation (8 channels, 4 pairs, per step), then the head's absmax over every query
  float y[32];
  float m = 0.0f, unused = 0.0f;
  if (live) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t bw[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      const float4 t0 = tab[2 * j], t1 = tab[2 * j + 1];
      const float cs[4][2] = {{t0.x, t0.y}, {t0.z, t0.w}, {t1.x, t1.y}, {t1.z, t1.w}};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float xe = __uint_as_float(bw[p] << 16), xo = __uint_as_float(bw[p] & 0xFFFF0000u);
        y[8 * j + 2 * p] = xe * cs[p][0] - xo * cs[p][1];
        y[8 * j + 2 * p + 1] = xe * cs[p][1] + xo * cs[p][0];
      }
    }
    m = absmax<32>(y);
  }
  head_sync<kThreads>(rec, gen, sync_error_word(qa_.sync), qa_.blocks, false, m, unused, sl);
  float scale, inv;
  scale_from_absmax(m, scale, inv);
  if (blk == 0 && threadIdx.x == 0) qa_.scale[h] = scale;
  uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wd[j] = e4m3x4(y[4 * j] * inv, y[4 * j + 1] * inv, y[4 * j + 2] * inv, y[4 * j + 3] * inv);
  }
  uint4* dst = reinterpret_cast<uint4*>(qa_.codes + ((((int64_t)h * qa_.qtiles + qt) * 8 + w) * 64 + lane) * 32);
  dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
}

// Order of the work-groups (block b of head h, x blocks per head; the grid is x by heads and L is
// its flat index, x varying fastest).  Work-groups are handed to the eight XCDs in turn in flat
// index order (L to XCD L mod 8), and each XCD starts its own in that order, so XCD L mod 8
// runs the (L / 8)-th item of its own list.  Each list is head-major (all of head h's items
// before head h + 1's: head_sync's condition) and holds the same blocks for every head: block b < f (x rounded down to a multiple of 8) on XCD b mod 8, so
// an XCD loads the rotary rows of its blocks once for all heads rather than every XCD loading
// every row.  The r = x - f remaining blocks of head h go to XCDs (h r + j) mod 8, j < r, which
// evens the lists' lengths: XCD c's list then holds exactly the indices L < x * heads with
// L mod 8 = c.
struct BlockOfHead { int b, h; };
__device__ inline BlockOfHead block_of_head(int L, int x, int heads) {
  const int c = L & 7, k = L >> 3;
  const int f8 = x >> 3, r = x & 7;
  // items of XCD c before head h: h * f8 fixed ones plus the remaining blocks m < h * r with
  // m mod 8 = c
  auto before = [&](int h) {
    const int hr = h * r;
    return h * f8 + (hr > c ? (hr - c + 7) >> 3 : 0);
  };
  int h = (int)((8LL * k) / x);
  h = h < heads - 1 ? h : heads - 1;
  while (h > 0 && before(h) > k) --h;
  while (h + 1 < heads && before(h + 1) <= k) ++h;
  const int o = k - before(h);
  const int b = o < f8 ? c + 8 * o : 8 * f8 + ((c - h * r) & 7);
  return {b, h};
}

// grid = (write blocks + query blocks, heads), taken in the order of block_of_head; each
// does one or the other (WQ: the write's work-groups prepare the queries too, and there are no
// query blocks).
template <int D, bool WQ>
__global__ __launch_bounds__(kThreads) void quantize_pass(WriteArgs wa, QuantQArgs qa_,
                                                          const float* __restrict__ rope, int32_t heads) {
  const BlockOfHead bh = block_of_head(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, heads);
  if (bh.b < wa.blocks)
    write_chunk<D, WQ>(wa, qa_, rope, bh.b, bh.h);
  else
    quantize_q_half<D>(qa_, rope, bh.b - wa.blocks, bh.h, heads);
}

}  // namespace

int64_t write_workspace_floats(int32_t, int32_t) { return kSyncBytes / 4; }

namespace {

}  // namespace

namespace {

WriteArgs write_args(const kv_ring_desc& r, const uint16_t* k_new, const uint16_t* v_new, int32_t n,
                     int32_t start_slot, int64_t pos0, float* ws) {
  WriteArgs wa;
  wa.k_new = k_new;
  wa.v_new = v_new;
  wa.sync = ws;
  wa.kc = r.k;
  wa.vc = r.v;
  wa.k_scale = r.k_scale;
  wa.v_scale = r.v_scale;
  WriteGeom& g = wa.g;
  g.n = n;
  g.start = start_slot;
  g.slots = r.slots;
  g.heads = r.heads;
  g.tiles = tile_count(r.slots);
  g.pos0 = pos0;
  const int end_a = start_slot + n < r.slots ? start_slot + n : r.slots;
  g.chunk_a0 = start_slot / kChunk;
  g.n_chunks_a = (end_a - 1) / kChunk - g.chunk_a0 + 1;
  int n_chunks_b = 0;
  if (start_slot + n > r.slots) {
    const int end_b = start_slot + n - r.slots;  // run [0, end_b)
    n_chunks_b = (end_b - 1) / kChunk + 1;
    // a chunk holding both the end of the wrapped run and the start of the first run is
    // handled once, by the first run's work-group
    if ((end_b - 1) / kChunk == g.chunk_a0) n_chunks_b -= 1;
  }
  wa.blocks = g.n_chunks_a + n_chunks_b;
  return wa;
}

QuantQArgs quant_q_args(const uint16_t* q, int32_t nq, int64_t q_pos0, void* sync, uint8_t* codes,
                        float* scale) {
  QuantQArgs qa_;
  qa_.q = q;
  qa_.sync = sync;
  qa_.codes = codes;
  qa_.scale = scale;
  qa_.pos0 = q_pos0;
  qa_.nq = nq;
  // an even number of 128-query tiles per head: the attention takes its rows 256 queries at a
  // time (the padding queries of the last tile are stored as zero codes)
  qa_.qtiles = 2 * ((nq + 255) / 256);
  qa_.blocks = 2 * qa_.qtiles;
  return qa_;
}

hipError_t launch_quantize_pass(const WriteArgs& wa, const QuantQArgs& qa_, const float* rope,
                                int32_t heads, int32_t head_dim, hipStream_t stream, bool merged = false) {
  if (merged) {   // the queries with the write's work-groups (head_dim 128)
    QuantQArgs qm = qa_;
    qm.blocks = 0;
    hipLaunchKernelGGL((quantize_pass<128, true>), dim3(wa.blocks, heads), dim3(kThreads), 0, stream, wa, qm,
                       rope, heads);
    return hipGetLastError();
  }
  const dim3 g2(wa.blocks + qa_.blocks, heads);
  if (head_dim == 128)
    hipLaunchKernelGGL((quantize_pass<128, false>), g2, dim3(kThreads), 0, stream, wa, qa_, rope, heads);
  else
    hipLaunchKernelGGL((quantize_pass<64, false>), g2, dim3(kThreads), 0, stream, wa, qa_, rope, heads);
  return hipGetLastError();
}

WriteArgs no_write() {
  WriteArgs wa;
  std::memset(&wa, 0, sizeof(wa));
  return wa;
}

QuantQArgs no_queries() {
  QuantQArgs qa_;
  std::memset(&qa_, 0, sizeof(qa_));
  return qa_;
}

}  // namespace

hipError_t launch_write(const kv_ring_desc& r, const uint16_t* k_new, const uint16_t* v_new,
                        int32_t n, int32_t start_slot, int64_t pos0, const float* rope,
                        float* ws, hipStream_t stream) {
  return launch_quantize_pass(write_args(r, k_new, v_new, n, start_slot, pos0, ws), no_queries(), rope,
                              r.heads, r.head_dim, stream);
}

hipError_t launch_q_prep(const uint16_t* q, int32_t nq, int32_t heads, int32_t head_dim,
                         int64_t q_pos0, const float* rope, void* sync, uint8_t* codes,
                         float* scale, hipStream_t stream) {
  return launch_quantize_pass(no_write(), quant_q_args(q, nq, q_pos0, sync, codes, scale), rope,
                              heads, head_dim, stream);
}

hipError_t launch_write_and_q_prep(const kv_ring_desc& r, const uint16_t* k_new,
                                   const uint16_t* v_new, int32_t n, int32_t start_slot,
                                   int64_t pos0, const uint16_t* q, int32_t nq, int64_t q_pos0,
                                   const float* rope, float* ws, uint8_t* codes, float* scale,
                                   hipStream_t stream) {
  // the queries are the new tokens themselves (the layer call of the method): the write's
  // work-groups prepare them too
  const bool merged = r.head_dim == 128 && nq == n && q_pos0 == pos0 && n > 0;
  return launch_quantize_pass(write_args(r, k_new, v_new, n, start_slot, pos0, ws),
                              quant_q_args(q, nq, q_pos0, ws, codes, scale), rope, r.heads,
                              r.head_dim, stream, merged);
}

// ---- the write without a caller workspace (kv_ring_write_static) ---------------------------------
//
// Its scratch (the per-head synchronisation records of head_sync) lives in a file-scope device
// array, one copy per GPU, held until the process ends.  Host code must not pass the array's name
// to a kernel (in host code it is a host-side stand-in); its device address is looked up once per
// device, with that device current, and kept.  The array starts at zero when the code object is
// loaded and every call leaves its records ready for the next, so it needs no clearing between
// calls; calls that overlap on one GPU share it and race.

namespace {
static_assert(kSyncBytes <= kWriteStaticScratchFloats * 4, "the static scratch holds the records");
__device__ __align__(256) float g_write_scratch[kWriteStaticScratchFloats];

std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t write_static_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_write_scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kvring

