// kv_ring_write: write-time RoPE + per-head FP8 quantisation of new K/V tokens into the ring
// (Runway Characters abstract: RoPE and FP8 quantisation applied once per write into a ring
// cache; cpdf.ai blog, section "Como rodar 57B em tempo real com batch size 1").
//
// Two bandwidth-bound passes, no atomics:
//   1. rope_absmax_partials: each work-group takes 32 tokens x 1 head, rotates K, and writes
//      the max |K'| and max |V| of its rows to a per-(tensor, head, group) partial;
//   2. quantize_pass: each write work-group takes one aligned 32-slot chunk of the ring x 1
//      head, reduces the head's partials to the write's absmax, rotates and quantises again,
//      and stores K and V codes into the tile layout (V transposed).
// The attention's queries take the same two passes (their absmax partials, then rotation and
// quantisation in the QK product's operand order), in the same launches when the attention
// follows a write (kv_ring_write_attend).
// The second read of the bf16 inputs is served mostly from the L2 / infinity cache.
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

// Rotate CPT channels (CPT/2 interleaved pairs) with the table row of this position.
// `tab` points at the (cos, sin) of the first pair; 16-byte aligned.
template <int CPT>
__device__ inline void rope_pairs(float (&x)[CPT], const float* tab) {
  const float4* t4 = reinterpret_cast<const float4*>(tab);
#pragma unroll
  for (int j = 0; j < CPT / 4; ++j) {
    float4 t = t4[j];  // cos0 sin0 cos1 sin1 for pairs 2j, 2j+1
    float cs[2][2] = {{t.x, t.y}, {t.z, t.w}};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int p = 2 * j + e;
      const float xe = x[2 * p], xo = x[2 * p + 1];
      const float c = cs[e][0], s = cs[e][1];
      x[2 * p] = xe * c - xo * s;
      x[2 * p + 1] = xe * s + xo * c;
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

// Pass 1: per (tensor, head, 32-token group) max |x|, rotated tensors (K, Q) after RoPE at their
// positions.  One launch can serve up to three tensors (K and V of a write, and the queries of
// the attention that follows it): grid = (max groups, heads, jobs); job z writes its partials
// [heads][groups of job z] at its own base pointer.
struct AbsmaxJob {
  const uint16_t* x;   // bfloat16 [n][heads][D]
  float* partial;      // [heads][groups]
  int64_t pos0;        // position of token 0 (rotated jobs)
  int32_t n, groups, rotate;
};
struct AbsmaxJobs {
  AbsmaxJob job[3];
};

template <int D>
__global__ __launch_bounds__(kThreads) void rope_absmax_partials(AbsmaxJobs jobs, int32_t heads,
                                                                 const float* __restrict__ rope) {
  constexpr int CPT = D / 8;
  __shared__ float red[4];
  const AbsmaxJob& jb = jobs.job[blockIdx.z];
  const int grp = blockIdx.x, h = blockIdx.y;
  if (grp >= jb.groups) return;   // uniform per work-group: this job has fewer tokens
  const int i = grp * kChunk + (threadIdx.x >> 3);
  const int cg = threadIdx.x & 7;
  float m = 0.0f;
  if (i < jb.n) {
    const uint16_t* src = jb.x + ((int64_t)i * heads + h) * D + cg * CPT;
    float x[CPT];
    load_bf16<CPT>(src, x);
    if (jb.rotate) rope_pairs<CPT>(x, rope + ((jb.pos0 + i) * (D / 2) + cg * (CPT / 2)) * 2);
    m = absmax<CPT>(x);
  }
  m = block_max_256(m, red);
  if (threadIdx.x == 0) jb.partial[(int64_t)h * jb.groups + grp] = m;
}

struct WriteGeom {
  int32_t n, start, slots, heads;
  int32_t chunk_a0, n_chunks_a;  // first chunk of the run [start, min(start+n, slots))
  int32_t n_partial_groups;      // partial groups per (tensor, head) from pass 1
  int64_t tiles;
  int64_t pos0;
};

struct WriteArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* partial;   // pass-1 partials [2][heads][groups]
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
  const float* partial;   // [heads][groups]: the queries' absmax partials from pass 1
  uint8_t* codes;         // [heads * qtiles][8][64][32], qtiles even
  float* scale;           // [heads]
  int64_t pos0;
  int32_t nq, groups, qtiles;
  int32_t blocks;         // 2 * qtiles (a work-group takes 64 queries of a row); 0: none
};

// Pass 2 of the write: one aligned 32-slot chunk of the ring x one head.
template <int D>
__device__ inline void write_chunk(const WriteArgs& wa, const float* __restrict__ rope, int blk, int h) {
  constexpr int CPT = D / 8;
  __shared__ float red[2][4];
  __shared__ __align__(16) uint8_t vlds[kChunk][D];
  const WriteGeom& g = wa.g;
  const uint16_t* __restrict__ k_new = wa.k_new;
  const uint16_t* __restrict__ v_new = wa.v_new;
  const float* __restrict__ partial = wa.partial;
  uint8_t* __restrict__ kc = wa.kc;
  uint8_t* __restrict__ vc = wa.vc;
  float* __restrict__ k_scale = wa.k_scale;
  float* __restrict__ v_scale = wa.v_scale;
  const int chunk = blk < g.n_chunks_a ? g.chunk_a0 + blk : blk - g.n_chunks_a;

  // this thread's inputs first (they do not depend on the scales), so that their latency
  // overlaps the reduction of the partials
  const int t = threadIdx.x >> 3, cg = threadIdx.x & 7;
  const int slot = chunk * kChunk + t;
  int i = slot - g.start;
  i = i < 0 ? i + g.slots : i;
  const bool mine = slot < g.slots && i < g.n;
  float xk[CPT], xv[CPT];
  float4 tab[CPT / 4];
  if (mine) {
    const int64_t src = ((int64_t)i * g.heads + h) * D + cg * CPT;
    load_bf16<CPT>(k_new + src, xk);
    load_bf16<CPT>(v_new + src, xv);
    const float4* t4 = reinterpret_cast<const float4*>(rope + ((g.pos0 + i) * (D / 2) + cg * (CPT / 2)) * 2);
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) tab[j] = t4[j];
  }

  // the write's per-head absmax of K' and V from the pass-1 partials (up to 2,048 tokens each
  // wavefront reduces the partial lists itself, with no barrier)
  const float ak = list_max(partial + (int64_t)h * g.n_partial_groups, g.n_partial_groups, red[0]);
  const float av = list_max(partial + ((int64_t)g.heads + h) * g.n_partial_groups, g.n_partial_groups, red[1]);
  float sk, ik, sv, iv;
  scale_from_absmax(ak, sk, ik);
  scale_from_absmax(av, sv, iv);

  if (mine) {
    float (&x)[CPT] = xk;
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) {   // RoPE: pairs 2j, 2j+1 of this thread's channels
      const float cs[2][2] = {{tab[j].x, tab[j].y}, {tab[j].z, tab[j].w}};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int p = 2 * j + e;
        const float xe = x[2 * p], xo = x[2 * p + 1];
        x[2 * p] = xe * cs[e][0] - xo * cs[e][1];
        x[2 * p + 1] = xe * cs[e][1] + xo * cs[e][0];
      }
    }
    uint32_t w[CPT / 4];
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j)
      w[j] = e4m3x4(x[4 * j] * ik, x[4 * j + 1] * ik, x[4 * j + 2] * ik, x[4 * j + 3] * ik);
    // channels cg*CPT .. +CPT-1: one 16-byte unit (head_dim 128) or half of one (64)
    uint8_t* dst = kc + (int64_t)h * g.tiles * kTile * D + k_code_offset(slot, (cg * CPT) & ~15, D) +
                   ((cg * CPT) & 15);
    if constexpr (CPT == 16) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
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
      k_scale[(int64_t)h * g.slots + slot] = sk;
      v_scale[(int64_t)h * g.slots + slot] = sv;
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
      *reinterpret_cast<uint4*>(unit) = make_uint4(word[0], word[1], word[2], word[3]);
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
  __shared__ float red[4];
  const int qt = blk >> 1, w = 4 * (blk & 1) + (int(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int i = qt * 128 + w * 16 + li;
  const bool live = i < qa_.nq && (D == 128 || g < 2);
  uint4 raw[4];
  float4 tab[8];
  if (live) {   // inputs first: their latency overlaps the reduction below
    const uint4* src = reinterpret_cast<const uint4*>(qa_.q + ((int64_t)i * heads + h) * D + 32 * g);
    const float4* t4 = reinterpret_cast<const float4*>(rope + ((qa_.pos0 + i) * (D / 2) + 16 * g) * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = src[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) tab[j] = t4[j];
  }
  const float a = list_max(qa_.partial + (int64_t)h * qa_.groups, qa_.groups, red);
  float scale, inv;
  scale_from_absmax(a, scale, inv);
  if (blk == 0 && threadIdx.x == 0) qa_.scale[h] = scale;
  uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // 8 channels (4 pairs) per step
      const uint32_t bw[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      const float4 t0 = tab[2 * j], t1 = tab[2 * j + 1];
      const float cs[4][2] = {{t0.x, t0.y}, {t0.z, t0.w}, {t1.x, t1.y}, {t1.z, t1.w}};
      float y[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float xe = __uint_as_float(bw[p] << 16), xo = __uint_as_float(bw[p] & 0xFFFF0000u);
        y[2 * p] = (xe * cs[p][0] - xo * cs[p][1]) * inv;
        y[2 * p + 1] = (xe * cs[p][1] + xo * cs[p][0]) * inv;
      }
      wd[2 * j] = e4m3x4(y[0], y[1], y[2], y[3]);
      wd[2 * j + 1] = e4m3x4(y[4], y[5], y[6], y[7]);
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(qa_.codes + ((((int64_t)h * qa_.qtiles + qt) * 8 + w) * 64 + lane) * 32);
  dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
}

// Pass 2: grid = (write blocks + query blocks, heads); each work-group does one or the other.
template <int D>
__global__ __launch_bounds__(kThreads) void quantize_pass(WriteArgs wa, QuantQArgs qa_,
                                                          const float* __restrict__ rope, int32_t heads) {
  const int h = blockIdx.y;
  if ((int)blockIdx.x < wa.blocks)
    write_chunk<D>(wa, rope, blockIdx.x, h);
  else
    quantize_q_half<D>(qa_, rope, blockIdx.x - wa.blocks, h, heads);
}

}  // namespace

int64_t write_workspace_floats(int32_t heads, int32_t n) {
  return 2LL * heads * ((n + kChunk - 1) / kChunk);
}

namespace {

hipError_t launch_absmax(const AbsmaxJobs& jobs, int njobs, int32_t heads, int32_t head_dim,
                         const float* rope, hipStream_t stream) {
  int gx = 1;
  for (int j = 0; j < njobs; ++j) gx = jobs.job[j].groups > gx ? jobs.job[j].groups : gx;
  dim3 g1(gx, heads, njobs);
  if (head_dim == 128)
    hipLaunchKernelGGL(rope_absmax_partials<128>, g1, dim3(kThreads), 0, stream, jobs, heads, rope);
  else
    hipLaunchKernelGGL(rope_absmax_partials<64>, g1, dim3(kThreads), 0, stream, jobs, heads, rope);
  return hipGetLastError();
}

AbsmaxJob absmax_job(const uint16_t* x, int32_t n, bool rotate, int64_t pos0, float* partial) {
  AbsmaxJob j;
  j.x = x;
  j.partial = partial;
  j.pos0 = pos0;
  j.n = n;
  j.groups = (n + kChunk - 1) / kChunk;
  j.rotate = rotate ? 1 : 0;
  return j;
}

}  // namespace

namespace {

WriteArgs write_args(const kv_ring_desc& r, const uint16_t* k_new, const uint16_t* v_new, int32_t n,
                     int32_t start_slot, int64_t pos0, float* ws) {
  WriteArgs wa;
  wa.k_new = k_new;
  wa.v_new = v_new;
  wa.partial = ws;
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
  g.n_partial_groups = (n + kChunk - 1) / kChunk;
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

QuantQArgs quant_q_args(const uint16_t* q, int32_t nq, int64_t q_pos0, const float* q_partial,
                        uint8_t* codes, float* scale) {
  QuantQArgs qa_;
  qa_.q = q;
  qa_.partial = q_partial;
  qa_.codes = codes;
  qa_.scale = scale;
  qa_.pos0 = q_pos0;
  qa_.nq = nq;
  qa_.groups = (nq + kChunk - 1) / kChunk;
  // an even number of 128-query tiles per head: the attention takes its rows 256 queries at a
  // time (the padding queries of the last tile are stored as zero codes)
  qa_.qtiles = 2 * ((nq + 255) / 256);
  qa_.blocks = 2 * qa_.qtiles;
  return qa_;
}

hipError_t launch_quantize_pass(const WriteArgs& wa, const QuantQArgs& qa_, const float* rope,
                                int32_t heads, int32_t head_dim, hipStream_t stream) {
  dim3 g2(wa.blocks + qa_.blocks, heads);
  if (head_dim == 128)
    hipLaunchKernelGGL(quantize_pass<128>, g2, dim3(kThreads), 0, stream, wa, qa_, rope, heads);
  else
    hipLaunchKernelGGL(quantize_pass<64>, g2, dim3(kThreads), 0, stream, wa, qa_, rope, heads);
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
  const int ngroups = (n + kChunk - 1) / kChunk;
  AbsmaxJobs jobs;
  jobs.job[0] = absmax_job(k_new, n, true, pos0, ws);
  jobs.job[1] = absmax_job(v_new, n, false, 0, ws + (int64_t)r.heads * ngroups);
  jobs.job[2] = jobs.job[1];
  hipError_t e = launch_absmax(jobs, 2, r.heads, r.head_dim, rope, stream);
  if (e != hipSuccess) return e;
  return launch_quantize_pass(write_args(r, k_new, v_new, n, start_slot, pos0, ws), no_queries(), rope,
                              r.heads, r.head_dim, stream);
}

hipError_t launch_q_prep(const uint16_t* q, int32_t nq, int32_t heads, int32_t head_dim,
                         int64_t q_pos0, const float* rope, float* q_partial, uint8_t* codes,
                         float* scale, hipStream_t stream) {
  AbsmaxJobs jobs;
  jobs.job[0] = absmax_job(q, nq, true, q_pos0, q_partial);
  jobs.job[1] = jobs.job[2] = jobs.job[0];
  hipError_t e = launch_absmax(jobs, 1, heads, head_dim, rope, stream);
  if (e != hipSuccess) return e;
  return launch_quantize_pass(no_write(), quant_q_args(q, nq, q_pos0, q_partial, codes, scale), rope,
                              heads, head_dim, stream);
}

hipError_t launch_write_and_q_prep(const kv_ring_desc& r, const uint16_t* k_new,
                                   const uint16_t* v_new, int32_t n, int32_t start_slot,
                                   int64_t pos0, const uint16_t* q, int32_t nq, int64_t q_pos0,
                                   const float* rope, float* ws, float* q_partial, uint8_t* codes,
                                   float* scale, hipStream_t stream) {
  const int ngroups = (n + kChunk - 1) / kChunk;
  AbsmaxJobs jobs;
  jobs.job[0] = absmax_job(k_new, n, true, pos0, ws);
  jobs.job[1] = absmax_job(v_new, n, false, 0, ws + (int64_t)r.heads * ngroups);
  jobs.job[2] = absmax_job(q, nq, true, q_pos0, q_partial);
  hipError_t e = launch_absmax(jobs, 3, r.heads, r.head_dim, rope, stream);
  if (e != hipSuccess) return e;
  return launch_quantize_pass(write_args(r, k_new, v_new, n, start_slot, pos0, ws),
                              quant_q_args(q, nq, q_pos0, q_partial, codes, scale), rope, r.heads,
                              r.head_dim, stream);
}

// ---- the write without a caller workspace (kv_ring_write_static) ---------------------------------
//
// Its scratch (the per-(tensor, head, group) partial maxima of pass 1, read by pass 2) lives in a
// file-scope device array, one copy per GPU, held until the process ends.  Host code must not pass
// the array's name to a kernel (in host code it is a host-side stand-in); its device address is
// looked up once per device, with that device current, and kept.  Every call writes every partial
// it reads before reading it, so the array needs no clearing between calls; calls that overlap on
// one GPU share it and race.

namespace {
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

