// ring_attention: attention of the new queries over every valid slot of the FP8 ring
// (Runway Characters abstract: 757 new-token queries against a 5,788-slot cache, 240 calls
// per chunk; cpdf.ai blog, section "Blackwell, escalabilidade e limites do decodificador":
// FP8 attention with per-head scales).
//
// Launches per call:
//   1. quantize_pass (shared with the write): the queries rotated, their head's absmax agreed
//      on through the head's record in the workspace, and encoded with the head's scale in the
//      order the QK product takes them.  kv_ring_write_attend does this inside the write's own
//      launch;
//   2. attn_pp: a persistent grid of one 8-wavefront work-group per compute unit.  The work is
//      the set of units (row, tile), a row being 256 queries of one head and a tile 128 ring
//      slots; each work-group takes a contiguous range of units of equal weight (a tile weighs
//      one, the start of a row's segment kSegCost more), so a row may be split between
//      work-groups.  A row held by one work-group is finished in place.  The segments of a
//      split row store their own output, normalised by their own sum, in half precision (a
//      weighted mean of dequantised V rows: within 2^-11 relative), with their (max, sum), and
//      the last of them to finish merges the row (log-sum-exp) and writes its output (see
//      store_partial and merge_items).  When rows are short (a ring still filling up) and fit
//      the grid, each work-group takes one whole row instead, and nothing is merged.
//      Consecutive work-groups of one XCD get consecutive units, so the rows of one head share
//      that XCD's L2.
//
// Each wavefront owns 32 queries, as two groups of 16 that share every operand read from LDS:
//   S^T = K Q^T           per group 8 MFMA 16x16x128 FP8 (fp32 accumulate)
//   online softmax        log2 domain, lazily rescaled (the running max may lag the true max
//                         by up to 2^4, so P <= 16); the running max is taken over the score
//                         plus log2 of the slot's V scale, so P already carries that scale
//   O^T += V^T P^T        per group 32 MFMA 16x16x32 fp16 (fp32 accumulate): P rounded once
//                         to fp16, V widened exactly from E4M3
// Computing S^T rather than S leaves one query per lane with its keys in registers, which is
// exactly the B-operand layout of the PV product: probabilities never leave their lane.
//
// Two-phase schedule.  The 8 wavefronts form two groups, wavefronts 0-3 and 4-7, one of each on
// every SIMD.  A wavefront alternates a matrix phase M_i (PV of tile i-1, QK of tile i, widening
// its share of V tile i to fp16, its share of the copies of tiles i+2) and a vector phase V_i
// (the softmax of tile i).  The second group runs one phase behind the first, so on every SIMD
// one wavefront issues matrix products while the other computes probabilities; every phase ends
// at a work-group barrier.  K tiles (and their scale rows) go to three LDS buffers and FP8 V
// tiles to two landing buffers, copied straight from HBM with global_load_lds (the ring stores
// each tile in the order the products read it, so copies and operand reads are linear 1 KB
// wavefront accesses free of bank conflicts).  Each thread widens exactly the V units its own
// copy brought in, so its own wait for that copy suffices and the landing buffer is reused
// right after.  Per-slot factors of tile i+1 and the zeroing of its invalid K bytes are done by
// the second group during its matrix phase M_i.
//
// A tile whose 128 slots are all valid and come from one write (one K scale, one V scale) takes
// the fast path: the max runs on raw scores, one FMA forms the exponent, and the V-scale factor
// is folded into it.  Other tiles (ring edges, write boundaries, partially filled rings) take
// the general path with per-slot scales, masking, and zeroed K bytes and fp16 V values for
// invalid slots.

#include "kvring_common.hpp"
#include "kvring_internal.hpp"

namespace kvring {

namespace {

constexpr int kWaves = 8;               // 2 wavefronts per SIMD, one of each group
constexpr int kThreads = 64 * kWaves;   // 512
constexpr int kGroupQ = 16;             // queries of one MFMA group
constexpr int kRowQ = 2 * kGroupQ * kWaves;   // 256 queries per row, 32 per wavefront
constexpr int kBufs = 3;                // LDS buffers of K tiles
constexpr int kMaxGrid = 256;
constexpr int kSegCost = 2;             // weight of a segment start in tiles (UnitSplit)
constexpr int kMergeCost = 2;           // weight of splitting rows (partial stores, the merge), in tiles
constexpr int kMaxSeg = 8;              // segments of a row, at most (make_plan)
constexpr float kTau = 4.0f;            // lazy rescale threshold, log2 units
constexpr float kPmax = 4096.0f;        // bound on a lane's probability sum in the fast path
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));   // fp16 operand of the PV product
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* q_codes;  // quantised queries: per 128-query tile [8][64 lanes][32 bytes]
  const float* q_scale;    // [heads]
  uint16_t* out;
  float* lse;
  _Float16* part_o;        // per (row, segment): the segment's output normalised by its l
  float* part_ml;          // per (row, segment): [kRowQ][2] (max, sum) of each query
  int* merge_cnt;          // per split row (by its first work-group): arrival and ready counts
  int* err;                // the workspace's error word
  int64_t tiles;           // ring tiles per head
  int64_t units;           // rows * tv
  int64_t cost;            // rows * (tv + seg_cost): the partition's total weight
  int32_t seg_cost;        // weight of a segment start, in tiles (see UnitSplit)
  int32_t heads, slots, ring_head, filled, nq;
  int32_t qtiles, rows, tv, grid, max_seg;   // qtiles: rows per head
  int32_t first1, n1, first2;  // valid tiles: logical k < n1 -> first1 + k, else first2 + k - n1
  float score_scale;           // softmax_scale * log2(e)
};

// Partition of the units (row, tile) among the work-groups, by weight rather than by count: a
// work-group whose range starts a row pays a second segment start (the end of one row's
// segment, the queries and first tiles of the next), so every row start weighs seg_cost tiles on
// top of its tv tiles.  Unit u of row r at tile k sits at weight position
// r * (tv + seg_cost) + seg_cost + k; virtual work-group v takes the units whose position falls
// in [v * cost / grid, (v + 1) * cost / grid).
struct UnitSplit {
  int64_t tv, c, cost;
  int grid;
  __host__ __device__ int64_t pos(int64_t u) const { return (u / tv) * (tv + c) + c + u % tv; }
  // first unit at or after weight position x
  __host__ __device__ int64_t first_unit(int64_t x) const {
    const int64_t r = x / (tv + c), o = x % (tv + c);
    return r * tv + (o > c ? o - c : 0);
  }
  __host__ __device__ int64_t begin(int v) const { return first_unit((int64_t)v * cost / grid); }
  __host__ __device__ int owner(int64_t u) const {   // virtual work-group holding unit u
    return int(((pos(u) + 1) * grid + cost - 1) / cost) - 1;
  }
};

// LDS of a work-group.  Each array is its own LDS object, so that the compiler can tell reads of
// the factor arrays from the asynchronous tile copies landing in the tile and scale buffers.
template <int D>
struct Smem {
  uint8_t (&k)[kBufs][kTile * D];    // K tile j of a segment in k[j % 3] (with ks, vs, factors)
  uint8_t (&v8)[2][D * kTile];       // FP8 transposed V tile j lands in v8[j % 2]
  uint8_t (&v16)[2][2 * D * kTile];  // V tile j widened to fp16 in v16[j % 2] (PV operand order)
  float (&ks)[kBufs][kTile];
  float (&vs)[kBufs][kTile];
  float (&ck)[kBufs][kTile];   // per slot: c0 * k_scale (valid) or 0
  float (&nb)[kBufs][kTile];   // per slot: log2(v_scale) (valid) or -inf
  float (&iv)[kBufs][kTile];   // per slot: 1 / v_scale (valid) or 0
  int (&uni)[kBufs][4];        // per 32 slots: all valid, one K scale and one V scale (1) or not
  float (&qs)[4];              // the head's query scale
};

// QK product, FP8 x FP8 -> fp32.  Zero scale operands select the unscaled encoding
// (v_mfma_f32_16x16x128_f8f6f4): no operand scaling.
__device__ inline v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ inline v4f mfma_f16(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two floats -> two fp16 values (round to nearest even), the first in the low half.
__device__ inline uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, v2h{(_Float16)a, (_Float16)b});
}

// max over lanes l, l^16, l^32, l^48 (the four lane groups holding one query's scores)
__device__ inline float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Valid slot range(s) of tile t as u-intervals [lo1, hi1) and [lo2, hi2) within 0..127.
struct TileValid {
  int lo1, hi1, lo2, hi2;
  __device__ int count() const { return max(0, hi1 - lo1) + max(0, hi2 - lo2); }
  __device__ bool has(int u) const { return (u >= lo1 && u < hi1) || (u >= lo2 && u < hi2); }
};

__device__ inline TileValid tile_valid(int64_t t, int head, int filled, int slots) {
  const int base = int(t) * kTile;
  const int top = min(base + kTile, slots);
  int old = head - filled;
  old = old < 0 ? old + slots : old;
  const int e1 = min(old + filled, slots);        // [old, e1)
  const int e2 = old + filled - slots;            // wrapped part [0, e2)
  TileValid v;
  v.lo1 = max(base, old) - base;
  v.hi1 = min(top, e1) - base;
  v.lo2 = 0;
  v.hi2 = e2 > 0 ? min(top, e2) - base : 0;
  return v;
}

// The QK product of score block bb takes, in lane li (0..15), tile slot 32*(li/4) + 4bb + li%4
// (the K tile layout stores them in that order).  Output row 4g+r of the block is then slot
// 32g + 4bb + r: lane group g ends up holding slots 32g .. 32g+31 of its query across the 8
// blocks, in order -- the B-operand layout of the PV product.

// 16-byte copies per lane of one K or FP8 V tile (every wavefront copies its own units: unit
// (j*8 + w)*64 + lane for j < kLoads).
template <int D>
constexpr int kLoads = (kTile * D / 16) / kThreads;

// Asynchronous global -> LDS copy of 16 bytes per lane (4 for copy4): global address base + voff
// (base uniform), LDS destination lds + 16 * lane (4 * lane).  Written as inline assembly so that
// the compiler does not track these copies: it would otherwise wait for all of them before any
// LDS access that might overlap, which would cut the copy pipeline to one step.  Completion is
// tracked with wait_vm; the LDS address goes through m0, as the instruction requires.
// The compiler inserts no hazard wait states around inline assembly, so the leading s_nop 4
// provides them: 5 wait states cover an SGPR operand written just before by a vector
// instruction (v_readlane restoring a spilled base address) and the m0 write.
__device__ inline void copy16(const void* base, uint32_t voff, const void* lds) {
  const uint32_t la = uint32_t(uintptr_t((lds_ptr)lds));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(la) : "memory");
}
__device__ inline void copy4(const void* base, uint32_t voff, const void* lds) {
  const uint32_t la = uint32_t(uintptr_t((lds_ptr)lds));
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(la) : "memory");
}

// This wavefront's share of the asynchronous copies of ring tile t: its K units and one scale
// row segment into K buffer b (kLoads + 1 copies per lane; wavefronts 0-3 copy the K scales of
// 32 slots each, 4-7 the V scales), or its FP8 V units into v8[b] (kLoads copies per lane).
template <int D>
__device__ inline void issue_k(const AttnArgs& a, Smem<D>& sm, int b, int64_t t, int h, int w, int lane) {
  const uint8_t* kbase = a.kc + ((int64_t)h * a.tiles + t) * (kTile * D);   // uniform
#pragma unroll
  for (int j = 0; j < kLoads<D>; ++j)
    copy16(kbase, uint32_t(((j * kWaves + w) * 64 + lane) * 16), &sm.k[b][(j * kWaves + w) * 1024]);
  if (lane < 32) {
    // slot index clamped in bounds; padding slots are masked by the tile's validity
    const int slot = min(int(t) * kTile + (w & 3) * 32 + lane, a.slots - 1);
    const float* srow = ((w < 4) ? a.k_scale : a.v_scale) + (int64_t)h * a.slots;   // uniform
    float* dst = (w < 4) ? &sm.ks[b][(w & 3) * 32] : &sm.vs[b][(w & 3) * 32];
    copy4(srow, uint32_t(slot) * 4u, dst);
  }
}

template <int D>
__device__ inline void issue_v(const AttnArgs& a, Smem<D>& sm, int b, int64_t t, int h, int w, int lane) {
  const uint8_t* vbase = a.vc + ((int64_t)h * a.tiles + t) * (D * kTile);   // uniform
#pragma unroll
  for (int j = 0; j < kLoads<D>; ++j)
    copy16(vbase, uint32_t(((j * kWaves + w) * 64 + lane) * 16), &sm.v8[b][(j * kWaves + w) * 1024]);
}

// Wait until at most n of this wavefront's vector-memory operations are outstanding (they
// complete in issue order).  n is one of the copy counts of the schedule (0 .. 8: one K tile
// share of kLoads + 1 copies and one V share of kLoads copies, kLoads <= 2); any other count
// waits for every operation.
__device__ inline void wait_vm(int n) {
  switch (n) {   // s_waitcnt immediate: vmcnt in bits 3:0, expcnt and lgkmcnt left at their maximum
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// Work-group barrier for LDS traffic only: this thread's LDS reads and writes are complete, and
// the compiler keeps memory accesses on their side of it.  Unlike __syncthreads it does not wait
// for the asynchronous tile copies in flight (their completion is tracked with wait_vm).
__device__ inline void lds_sync() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Per-slot factors of the tile in K buffer b, by the second group (wavefronts 4-7, one per SIMD,
// 32 slots each, one per lane of their first half).  Split in two so that the LDS reads can be
// issued well before the arithmetic that needs them: factor_inputs, then tile_factors.
struct FactorIn {
  float ks, vs, ks0, vs0;
};

template <int D>
__device__ inline FactorIn factor_inputs(const Smem<D>& sm, int b, int tid) {
  FactorIn f{0.0f, 0.0f, 0.0f, 0.0f};
  const int lane = tid & 63;
  if (tid >= 4 * 64 && lane < 32) {
    const int u = ((tid >> 6) & 3) * 32 + lane;
    f.ks = sm.ks[b][u];
    f.vs = sm.vs[b][u];
    f.ks0 = sm.ks[b][0];
    f.vs0 = sm.vs[b][0];
  }
  return f;
}

template <int D>
__device__ inline void tile_factors(Smem<D>& sm, int b, const TileValid& tvd, float c0, int tid,
                                    const FactorIn& f) {
  const int lane = tid & 63;
  if (tid >= 4 * 64 && lane < 32) {
    const int u = ((tid >> 6) & 3) * 32 + lane;
    const bool ok = tvd.has(u);
    sm.ck[b][u] = ok ? c0 * f.ks : 0.0f;
    sm.nb[b][u] = ok ? __log2f(f.vs) : -INFINITY;
    sm.iv[b][u] = ok ? __builtin_amdgcn_rcpf(f.vs) : 0.0f;
    const bool same = ok && f.ks == f.ks0 && f.vs == f.vs0;
    const bool all_same = __all(same);   // over this wavefront's 32 active lanes
    if (lane == 0) sm.uni[b][u >> 5] = all_same ? 1 : 0;
  }
}

// Zeroed K bytes for the invalid slots of the tile in K buffer b (so that whatever they hold --
// NaN codes included -- never reaches a product); tiles with invalid slots only; by the second
// group (256 threads).
template <int D>
__device__ inline void zero_invalid_k(Smem<D>& sm, int b, const TileValid& tvd, int tid) {
  constexpr int NCH = D / 16;
  uint8_t* kw = sm.k[b];
  for (int c = tid - 4 * 64; c < kTile * NCH; c += 4 * 64) {   // 16-byte units of the K tile
    const int li = c & 15, bb = c / (16 * (D / 32)) / 2;
    if (!tvd.has(32 * (li >> 2) + 4 * bb + (li & 3))) *reinterpret_cast<uint4*>(kw + c * 16) = make_uint4(0, 0, 0, 0);
  }
}

// Widening of this thread's FP8 V units (loaded into x) of the tile in v8[b] to fp16 in v16[b], in the PV
// product's operand order, with the invalid slots' values zeroed when the tile is not full (a
// slot is valid exactly when its factor iv, in K buffer bf, is non-zero: 1 / v_scale is finite
// and positive for every scale a write can store).  FP8 unit ((db*2 + r)*4 + g)*16 + li holds
// slots 32g + 16r .. +15 of channel 16db + li; its first 8 slots become piece (db, kb = 2r) and
// its last 8 piece (db, 2r + 1), where piece (db, kb) of lane (g, li) -- slots 32g + 8kb .. +7
// of channel 16db + li, 8 fp16 values -- sits at byte ((db*4 + kb)*64 + g*16 + li) * 16.  Each
// thread widens the units its own tile copy brought in (unit (j*8 + w)*64 + lane), so its own
// wait for that copy suffices; the fp16 tile is read by other wavefronts only after a barrier.
template <int D>
__device__ inline void widen_store(Smem<D>& sm, int b, int bf, int w, int lane, const uint4 (&x)[kLoads<D>],
                                   bool full) {
#pragma unroll
  for (int j = 0; j < kLoads<D>; ++j) {
    const int c = (j * kWaves + w) * 64 + lane;
    const uint32_t xw[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(xw[i]), 1.0f, false));
      h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(xw[i]), 1.0f, true));
    }
    const int li = c & 15, g = (c >> 4) & 3, r = (c >> 6) & 1, db = c >> 7;
    if (!full) {
      const float* ivu = &sm.iv[bf][32 * g + 16 * r];
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        if (ivu[kk] == 0.0f) h[kk >> 1] &= (kk & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    }
    const int o0 = ((db * 4 + 2 * r) * 64 + g * 16 + li) * 16;
    *reinterpret_cast<uint4*>(&sm.v16[b][o0]) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(&sm.v16[b][o0 + 1024]) = make_uint4(h[4], h[5], h[6], h[7]);
  }
}

// Per-lane LDS byte offsets (within one buffer) of a lane's A operands: half r of score block bb
// is K unit (bb*2 + r)*(D/32)*16 + lane, piece (db, kb) of the fp16 V tile is 16-byte unit
// (db*4 + kb)*64 + lane: every operand read is one contiguous 1 KB wavefront read.
struct LaneOffs {
  int k, v;
};

template <int D>
__device__ inline LaneOffs lane_offsets(int lane) {
  LaneOffs o;
  o.k = (D == 128 ? lane : (lane & 31)) * 16;   // head_dim 64: lanes 32..63 carry zeros
  o.v = lane * 16;
  return o;
}

// A operand of score block bb (16 K rows).
template <int D>
__device__ inline v8i k_operand(const uint8_t* kt, const LaneOffs& o, int bb, int g) {
  const uint4 x0 = *reinterpret_cast<const uint4*>(kt + o.k + (bb * 2) * (D / 32) * 256);
  const uint4 x1 = *reinterpret_cast<const uint4*>(kt + o.k + (bb * 2 + 1) * (D / 32) * 256);
  if (D != 128 && g >= 2) return v8i{0, 0, 0, 0, 0, 0, 0, 0};
  return v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
}

// A operand of the PV product of channel block db over slot block kb (16 fp16 V^T rows).
__device__ inline v8h v_operand(const uint8_t* vt, const LaneOffs& o, int db, int kb) {
  return *reinterpret_cast<const v8h*>(vt + o.v + (db * 4 + kb) * 1024);
}

// State of one query group (16 queries) of a wavefront: lane (g, li) holds query li's channels
// 16*db + 4g .. +3 of every channel block db, its raw scores of tile slots 32g .. 32g+31
// (sc[bb][r]: slot 32g + 4bb + r) and their probabilities as fp16 pairs (p[2bb + h]: slots
// 32g + 4bb + 2h, +1; dwords 4kb .. 4kb+3 are the lane's B operand of PV slot block kb).
template <int D>
struct Group {
  v4f acc[D / 16];
  v4f sc[8];
  uint32_t p[16];
  float m;   // running max (log2 units), identical in the 4 lanes of a query
  float l;   // this lane's share of the running sum
  bool started;   // every lane's running max is finite (wavefront-uniform)
};

__device__ inline v8h p_operand(const uint32_t (&p)[16], int kb) {
  return __builtin_bit_cast(v8h, v4u{p[4 * kb], p[4 * kb + 1], p[4 * kb + 2], p[4 * kb + 3]});
}

// Matrix part of phase M_i: PV of the previous tile (fp16 V in vt) and QK of this tile (K in kt).
// Each operand read from LDS feeds both query groups.  PV product n takes channel block n % NDB and
// slot block n / NDB; its V operand is read kPre products ahead (PvPipe), the K operands of QK
// kPreK blocks ahead, and the scheduling
// barriers keep that distance (left to itself the compiler hoists every read to the top and runs
// out of registers).  The products run in ranges (pv_run<N0, N1>), so that the phase's side work
// can be placed between them and overlap them.
constexpr int kPre = 8;    // V operands in flight (PV)
constexpr int kPreK = 4;   // K operands in flight (QK)

template <int D>
struct PvPipe {
  v8h vo[kPre];
};

template <int D>
__device__ __forceinline__ void pv_start(PvPipe<D>& pp, const uint8_t* vt, const LaneOffs& lo) {
  constexpr int NDB = D / 16;
#pragma unroll
  for (int n = 0; n < kPre; ++n) pp.vo[n] = v_operand(vt, lo, n % NDB, n / NDB);
}

template <int N0, int N1, int D>
__device__ __forceinline__ void pv_run(PvPipe<D>& pp, const uint8_t* vt, const LaneOffs& lo, Group<D>& ga,
                                       Group<D>& gb) {
  constexpr int NDB = D / 16;
  constexpr int NPV = NDB * 4;
#pragma unroll
  for (int n = N0; n < N1; ++n) {
    const v8h x = pp.vo[n % kPre];
    if (n + kPre < NPV) pp.vo[n % kPre] = v_operand(vt, lo, (n + kPre) % NDB, (n + kPre) / NDB);
    const int db = n % NDB, kb = n / NDB;
    ga.acc[db] = mfma_f16(x, p_operand(ga.p, kb), ga.acc[db]);
    gb.acc[db] = mfma_f16(x, p_operand(gb.p, kb), gb.acc[db]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__device__ __forceinline__ void qk_run(const uint8_t* kt, const LaneOffs& lo, int g, const v8i (&qop)[2],
                                       Group<D>& ga, Group<D>& gb) {
  v8i ko[kPreK];
#pragma unroll
  for (int bb = 0; bb < kPreK; ++bb) ko[bb] = k_operand<D>(kt, lo, bb, g);
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    const v8i x = ko[bb % kPreK];
    if (bb + kPreK < 8) ko[bb % kPreK] = k_operand<D>(kt, lo, bb + kPreK, g);
    ga.sc[bb] = mfma_fp8(x, qop[0], v4f{0.0f, 0.0f, 0.0f, 0.0f});
    gb.sc[bb] = mfma_fp8(x, qop[1], v4f{0.0f, 0.0f, 0.0f, 0.0f});
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Marks a rarely taken branch: an instruction with side effects cannot be executed
// speculatively, so the compiler keeps the branch instead of flattening both paths into one
// sequence that runs every time.
__device__ inline void rare_branch() { asm volatile(""); }

// Raises the group's running max to the tile's maximum score t = raw * cf + bf (cf > 0) when it
// exceeds the running max by more than kTau (lazy rescaling), rescaling the accumulator and the
// running sum, which at this point hold the contributions of every earlier tile.
template <int D>
__device__ __forceinline__ void raise_max(Group<D>& gr, float tmax) {
  constexpr int NDB = D / 16;
  if (__any(tmax > gr.m + kTau)) {
    rare_branch();
    const float m_new = __builtin_fmaxf(gr.m, tmax);
    const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(gr.m - m_new);
    gr.m = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) gr.acc[db] *= alpha;
    gr.l *= alpha;
  }
  gr.started = __all(gr.m != -INFINITY);
}

// Probabilities of a uniform tile: P' = 2^(raw * cf + bm) into the group's fp16 operand tile;
// returns this lane's sum of the fp16 values (the dot product with ones keeps it in fp32).
template <int D>
__device__ __forceinline__ float uniform_probs(Group<D>& gr, float cf, float bm) {
  const v2h one = {(_Float16)1.0f, (_Float16)1.0f};
  float s0 = 0.0f, s1 = 0.0f;   // two chains of dependent steps
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(gr.sc[bb][r], cf, bm));
    gr.p[2 * bb] = pack_f16(p[0], p[1]);
    gr.p[2 * bb + 1] = pack_f16(p[2], p[3]);
    s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, gr.p[2 * bb]), one, s0, false);
    s1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, gr.p[2 * bb + 1]), one, s1, false);
  }
  return s0 + s1;
}

// Softmax of one query group over the tile whose factors are in K buffer bk.
// Per score (slot j, query i):  t = raw * ck_j + nb_j, the log2-domain score plus log2 of the
// slot's V scale; P' = 2^(t - m) goes to the PV product (with V decoded but not scaled) and
// P' * iv_j = 2^(score - m) to the row sum.  The running max m tracks max t, lazily.
// Uniform tile (one ck, nb, iv for all 128 slots): the probabilities are formed against the
// running max as it stands, without a max over the tile first.  Their sum bounds every one of
// them: while no lane's sum exceeds kPmax (an fp16 overflow makes it infinite), each P' <= kPmax,
// far from the fp16 range limit; otherwise the tile's max has moved up, the running max is
// raised to it and the probabilities are formed again.  The first tile of a segment raises the
// running max first.  Other tiles take per-slot factors and a max over the tile.
template <int D>
__device__ __forceinline__ void softmax_group(const Smem<D>& sm, int bk, int g, bool uniform, float cf, float bf, float ivu, Group<D>& gr) {
  if (uniform) {
    auto tile_max = [&]() __attribute__((always_inline)) {
      float rmax = gr.sc[0][0];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) rmax = __builtin_fmaxf(rmax, gr.sc[bb][r]);
      return max_over_groups(rmax) * cf + bf;
    };
    if (!gr.started) {
      rare_branch();
      raise_max(gr, tile_max());
    }
    float s2 = uniform_probs(gr, cf, bf - gr.m);
    if (!__all(s2 <= kPmax)) {
      rare_branch();
      raise_max(gr, tile_max());
      s2 = uniform_probs(gr, cf, bf - gr.m);
    }
    gr.l = __builtin_fmaf(s2, ivu, gr.l);
    return;
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    const float4 ck = *reinterpret_cast<const float4*>(&sm.ck[bk][32 * g + 4 * bb]);
    const float4 nb = *reinterpret_cast<const float4*>(&sm.nb[bk][32 * g + 4 * bb]);
    gr.sc[bb][0] = __builtin_fmaf(gr.sc[bb][0], ck.x, nb.x);
    gr.sc[bb][1] = __builtin_fmaf(gr.sc[bb][1], ck.y, nb.y);
    gr.sc[bb][2] = __builtin_fmaf(gr.sc[bb][2], ck.z, nb.z);
    gr.sc[bb][3] = __builtin_fmaf(gr.sc[bb][3], ck.w, nb.w);
#pragma unroll
    for (int r = 0; r < 4; ++r) tmax = __builtin_fmaxf(tmax, gr.sc[bb][r]);
  }
  raise_max(gr, max_over_groups(tmax));
  const float bm = -(gr.m == -INFINITY ? 0.0f : gr.m);   // P' = 2^(t + bm)
  float lsum = 0.0f;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(gr.sc[bb][r] + bm);
    const float4 iv = *reinterpret_cast<const float4*>(&sm.iv[bk][32 * g + 4 * bb]);
    lsum = __builtin_fmaf(p[0], iv.x, lsum);
    lsum = __builtin_fmaf(p[1], iv.y, lsum);
    lsum = __builtin_fmaf(p[2], iv.z, lsum);
    lsum = __builtin_fmaf(p[3], iv.w, lsum);
    gr.p[2 * bb] = pack_f16(p[0], p[1]);
    gr.p[2 * bb + 1] = pack_f16(p[2], p[3]);
  }
  gr.l += lsum;
}

// ---- Split rows: partial results and their merge inside attn_pp.
// Every segment of a split row stores its output (normalised by its own sum, half precision)
// and each query's (max, sum) with accesses of device scope (cache policy sc1: coherent between
// the XCDs without writing back or invalidating any L2), waits until those stores are complete,
// and only then counts itself in the row's arrival count.  Once its range is done, each
// work-group of the row waits until the count shows every segment stored, merges its share of
// the row with loads of the same scope, writes that share's output, and counts itself in the
// row's departure count; the last to depart sets both counts back to zero for the next launch.
// A share is a set of items, an item being half the channels of a 16-query group (32 per row):
// segment s takes the items s, s + nseg, ..., spread over all eight wavefronts.  A segment that
// opens its work-group's range and is followed by more rows counts its arrival at the next row's
// first barrier (its stores are complete by then) and merges its share after the range, in the
// same passes as the share of the work-group's closing row.
// Arrivals never wait, so a work-group only waits for work-groups that can finish: the grid never
// exceeds the compute units, so on a device running nothing else all of it is resident, and with
// other work present the wait still ends as long as every XCD can hold the work-groups of one row
// at once (they are consecutive on one XCD, and an XCD starts its work-groups in order).  The
// wait is bounded: past kSpinLimit polls a work-group sets the error word and carries on (the
// row's output is then not to be trusted).  The two counts of a row sit on their own 128-byte
// lines, picked by the row's first work-group (in one launch at most one split row starts in each
// range).
constexpr int kPolicySc1 = 16;            // cache policy operand of the buffer builtins: sc1
constexpr int kRsrcWord3 = 0x00020000;    // buffer resource: 32-bit data format, untyped access
constexpr int kCountInts = kSyncLine / 4;
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}
__device__ inline int* merge_arrivals(const AttnArgs& a, int vf) { return a.merge_cnt + vf * 2 * kCountInts; }
__device__ inline int* merge_departures(const AttnArgs& a, int vf) { return merge_arrivals(a, vf) + kCountInts; }

// Thread 0: wait until all nseg segments of the row have arrived (bounded).
__device__ inline void merge_wait(const AttnArgs& a, int vf, int nseg) {
  const int* arr = merge_arrivals(a, vf);
  int polls = 0;
  while (__hip_atomic_load(arr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nseg) {
    if (++polls > kSpinLimit) {
      __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The partial result of query group q of this wavefront into block blk (= row * max_seg +
// segment): output as [wavefront, group][piece j][lane] 16-byte pieces (one piece: channel
// blocks 2j and 2j + 1 of the lane, 8 halves; each store instruction writes 1 KB contiguous),
// and (max, sum) per query.
template <int D>
__device__ inline void store_partial(const AttnArgs& a, int64_t blk, const Group<D>& gr, float lt,
                                     int w, int q, int lane) {
  constexpr int NJ = D / 32;
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(a.part_o + blk * (kRowQ * D), kRowQ * D * 2);
  const float il = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const v4f x = gr.acc[2 * j], y = gr.acc[2 * j + 1];
    const v8h h = {(_Float16)(x[0] * il), (_Float16)(x[1] * il), (_Float16)(x[2] * il), (_Float16)(x[3] * il),
                   (_Float16)(y[0] * il), (_Float16)(y[1] * il), (_Float16)(y[2] * il), (_Float16)(y[3] * il)};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, h), ro,
                                           (((w * 2 + q) * NJ + j) * 64 + lane) * 16, 0, kPolicySc1);
  }
  if ((lane >> 4) == 0) {
    const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(a.part_ml + blk * (kRowQ * 2), kRowQ * 8);
    const v2u ml = {__float_as_uint(gr.m), __float_as_uint(lt)};
    __builtin_amdgcn_raw_buffer_store_b64(ml, rm, (32 * w + 16 * q + (lane & 15)) * 8, 0, kPolicySc1);
  }
}

// Merge of stored segments by one wavefront, for up to two items at once.  An item is half of a
// query group of a split row: queries 16 gi .. 16 gi + 15 (stored by wavefront gi / 2 as its group
// gi % 2) and half hf of the lane's channel blocks (blocks (D/32) hf .. (D/32) hf + D/32 - 1 of
// its D/16); a row has 32 items.
// Each segment weighs 2^(m_s - m) times its sum, m being the largest max (the log-sum-exp merge).
// Every load of both items is issued before any arithmetic (one memory round trip); the result
// goes to the output like a row held by one work-group.
struct MergeItem {
  int row, nseg, gi, hf;
  bool on;
};

template <int D>
__device__ inline void write_out_blocks(const AttnArgs& a, const v4f* acc, int db0, int ndb, float m,
                                        float l, int head, int qt, int ql, int g, bool with_lse);

template <int D>
__device__ inline void merge_items(const AttnArgs& a, const MergeItem (&it)[2], int lane) {
  constexpr int NJ = D / 32;   // 16-byte pieces of a lane's group (channel blocks 2j, 2j + 1)
  constexpr int NH = NJ / 2;   // pieces of one half
  float ms[2][kMaxSeg], ls[2][kMaxSeg];
  v4u o[2][kMaxSeg][NH];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (!it[k].on) continue;
    const int64_t blk0 = (int64_t)it[k].row * a.max_seg;
    // one resource per array over the row's blocks; the segment's block offset goes in soffset
    const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(a.part_ml + blk0 * (kRowQ * 2), a.max_seg * kRowQ * 8);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(a.part_o + blk0 * (kRowQ * D), a.max_seg * kRowQ * D * 2);
    const int ql = 16 * it[k].gi + (lane & 15);
#pragma unroll
    for (int s = 0; s < kMaxSeg; ++s) {
      ms[k][s] = -INFINITY;
      ls[k][s] = 0.0f;
      if (s < it[k].nseg) {
        const v2u x = __builtin_amdgcn_raw_buffer_load_b64(rm, ql * 8, s * kRowQ * 8, kPolicySc1);
        ms[k][s] = __uint_as_float(x[0]);
        ls[k][s] = __uint_as_float(x[1]);
#pragma unroll
        for (int h = 0; h < NH; ++h)
          o[k][s][h] = __builtin_amdgcn_raw_buffer_load_b128(
              ro, ((it[k].gi * NJ + it[k].hf * NH + h) * 64 + lane) * 16, s * kRowQ * D * 2, kPolicySc1);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (!it[k].on) continue;
    float mt = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSeg; ++s) mt = __builtin_fmaxf(mt, ms[k][s]);
    const float mr = mt == -INFINITY ? 0.0f : mt;   // no finite max: every weight below is 0
    float lsum = 0.0f;
    v4f acc[2 * NH];
#pragma unroll
    for (int b = 0; b < 2 * NH; ++b) acc[b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kMaxSeg; ++s) {
      if (s >= it[k].nseg) continue;
      const float ws = __builtin_amdgcn_exp2f(ms[k][s] - mr) * ls[k][s];
      lsum += ws;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const v8h x = __builtin_bit_cast(v8h, o[k][s][h]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * h][c] = __builtin_fmaf(ws, float(x[c]), acc[2 * h][c]);
          acc[2 * h + 1][c] = __builtin_fmaf(ws, float(x[4 + c]), acc[2 * h + 1][c]);
        }
      }
    }
    write_out_blocks<D>(a, acc, 2 * NH * it[k].hf, 2 * NH, mt, lsum, it[k].row / a.qtiles,
                        it[k].row % a.qtiles, 16 * it[k].gi + (lane & 15), lane >> 4, it[k].hf == 0);
  }
}

// Every vector-memory operation of this thread complete (stores included); the asm's memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ inline void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Final output of one query (ql of the row): channel blocks db0 .. db0 + ndb - 1 of this lane
// (channels 16 db + 4g .. +3) as bf16 O / l, and, with with_lse, the log-sum-exp (natural log)
// of its scores, m being in log2 units.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

template <int D>
__device__ inline void write_out_blocks(const AttnArgs& a, const v4f* acc, int db0, int ndb, float m,
                                        float l, int head, int qt, int ql, int g, bool with_lse) {
  const int i = qt * kRowQ + ql;
  if (i >= a.nq) return;
  const float il = l > 0.0f ? 1.0f / l : 0.0f;
  uint16_t* dst = a.out + ((int64_t)i * a.heads + head) * D + 4 * g;
  for (int b = 0; b < ndb; ++b) {
    const v4f o = acc[b];
    const v2bf lo = __builtin_convertvector(v2f{o[0] * il, o[1] * il}, v2bf);   // round to nearest even
    const v2bf hi = __builtin_convertvector(v2f{o[2] * il, o[3] * il}, v2bf);
    *reinterpret_cast<uint2*>(dst + 16 * (db0 + b)) =
        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  }
  if (with_lse && g == 0) a.lse[(int64_t)head * a.nq + i] = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

template <int D>
__device__ inline void write_out(const AttnArgs& a, const v4f (&acc)[D / 16], float m, float l,
                                 int head, int qt, int ql, int g) {
  write_out_blocks<D>(a, acc, 0, D / 16, m, l, head, qt, ql, g, true);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_pp(AttnArgs a) {
  constexpr int NDB = D / 16;
  __shared__ __align__(16) uint8_t s_k[kBufs][kTile * D];
  __shared__ __align__(16) uint8_t s_v8[2][D * kTile];
  __shared__ __align__(16) uint8_t s_v16[2][2 * D * kTile];
  __shared__ __align__(16) float s_ks[kBufs][kTile];
  __shared__ __align__(16) float s_vs[kBufs][kTile];
  __shared__ __align__(16) float s_ck[kBufs][kTile];
  __shared__ __align__(16) float s_nb[kBufs][kTile];
  __shared__ __align__(16) float s_iv[kBufs][kTile];
  __shared__ __align__(16) int s_uni[kBufs][4];
  __shared__ __align__(16) float s_qs[4];
  // split rows this work-group merges a share of after its range, as (row (-1: none), first
  // work-group, segment count, its segment index): [0] the row of its closing segment, [1] that
  // of its opening segment
  __shared__ int s_merge[2][4];
  Smem<D> sm{s_k, s_v8, s_v16, s_ks, s_vs, s_ck, s_nb, s_iv, s_uni, s_qs};

  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);   // wavefront (uniform)
  const int grp = w >> 2;   // 0: wavefronts 0-3 (phase ahead), 1: wavefronts 4-7

  // virtual work-group index: consecutive indices on one XCD (work-groups are dealt to the 8
  // XCDs round-robin), so that neighbouring units share an L2
  const int wg = blockIdx.x;
  const int v = (a.grid % 8 == 0) ? (wg % 8) * (a.grid / 8) + wg / 8 : wg;
  const UnitSplit split{a.tv, a.seg_cost, a.cost, a.grid};
  int64_t ub = split.begin(v);
  const int64_t ue = split.begin(v + 1);
  const int tid = int(threadIdx.x);
  const int lane = tid & 63, g = lane >> 4, li = lane & 15;
  const LaneOffs lo = lane_offsets<D>(lane);
  constexpr int nk = kLoads<D> + 1, nv = kLoads<D>;

  // The first segment may start inside a row; every later one starts the next row at tile 0
  // (and is then the row's first segment).  The 64-bit divisions happen once per work-group.
  int row = int(ub / a.tv), k0 = int(ub % a.tv);
  int seg = k0 > 0 ? v - split.owner((int64_t)row * a.tv) : 0;   // index of this segment in its row
  // A split row's segment that opens this range and is followed by more rows is described in
  // s_merge[1] (LDS rather than registers, which the tile loop needs); it counts its arrival at
  // the next row's first barrier.
  if (tid == 0) s_merge[0][0] = s_merge[1][0] = -1;
  bool open_arrive = false;
  while (ub < ue) {
    const int k1 = int(min<int64_t>(a.tv, k0 + (ue - ub)));
    const int nt = k1 - k0;
    const int head = row / a.qtiles, qt = row % a.qtiles;
    const bool row_split = nt < a.tv;   // the row has other segments (in other work-groups)
    auto phys = [&](int k) __attribute__((always_inline)) -> int64_t { return k < a.n1 ? a.first1 + k : a.first2 + (k - a.n1); };

    // ---- prologue: this wavefront's queries (group q of wavefront w: queries 32w + 16q ..
    // +15 of the row, from 128-query tile 2qt + w/4 of the head, its wavefront slot (2w + q) % 8),
    // the head's query scale, and tiles 0 and 1 (both groups' shares)
    v8i qop[2];
    {
      const int64_t qtile = (int64_t)head * (2 * a.qtiles) + 2 * qt + (w >> 2);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4* src = reinterpret_cast<const uint4*>(
            a.q_codes + ((qtile * 8 + ((2 * w + q) & 7)) * 64 + lane) * 32);
        const uint4 x0 = src[0], x1 = src[1];
        qop[q] = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      }
      if (w == 0 && lane == 0) copy4(a.q_scale, uint32_t(head) * 4u, &sm.qs[0]);
    }
    issue_k<D>(a, sm, 0, phys(k0), head, w, lane);
    issue_v<D>(a, sm, 0, phys(k0), head, w, lane);
    if (nt > 1) {
      issue_k<D>(a, sm, 1, phys(k0 + 1), head, w, lane);
      issue_v<D>(a, sm, 1, phys(k0 + 1), head, w, lane);
    }
    wait_vm(0);
    lds_sync();
    if (open_arrive) {   // every thread's partial stores of the opening segment are complete
      if (tid == 0)
        __hip_atomic_fetch_add(merge_arrivals(a, s_merge[1][1]), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      open_arrive = false;
    }
    const float c0 = a.score_scale * sm.qs[0];
    {
      const TileValid tvd = tile_valid(phys(k0), a.ring_head, a.filled, a.slots);
      tile_factors(sm, 0, tvd, c0, tid, factor_inputs(sm, 0, tid));
      if (grp == 1 && tvd.count() < kTile) zero_invalid_k(sm, 0, tvd, tid);
    }
    lds_sync();

    Group<D> ga, gb;
    ga.m = gb.m = -INFINITY;
    ga.l = gb.l = 0.0f;
    ga.started = gb.started = false;
#pragma unroll
    for (int db = 0; db < NDB; ++db) ga.acc[db] = gb.acc[db] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 16; ++i) ga.p[i] = gb.p[i] = 0u;

    // ---- the two-phase pipeline.  Slot s of the work-group: the first group runs M_{s/2} (s
    // even) or V_{s/2} (s odd), the second group one slot later; a barrier ends every slot.
    //   M_i: PV(i-1); QK(i); widen this thread's units of V tile i into v16[i % 2]; copy this
    //        wavefront's shares of tiles i+2 (V into v8[i % 2], the units just widened; K into
    //        k[(i+2) % 3], free since the barrier after the second group's QK(i-1)); the second
    //        group also prepares tile i+1 (its K copies landed by the previous slot's end);
    //   V_i: softmax of tile i.
    // Copy completion: at the end of M_i a wavefront waits for everything but the copies it has
    // just issued, at the end of V_i for everything, so each copy has two slots to land.
    // Side work of M_i, in pieces placed between the phase's products.  Loads first, at the start
    // of the phase and ahead of the product operands (LDS reads return in order): this thread's
    // FP8 units of V tile i and, in the second group, the scale rows of tile i+1.  Then, a few
    // products later, the widening of those units to fp16 and the second group's preparation of
    // tile i+1 (factors, zeroed K bytes), and last the copies of tile i+2 (so that no wait before
    // them can cover a copy just issued).  side_copies returns the number of copies issued.
    uint4 vx[kLoads<D>];
    FactorIn fin{0.0f, 0.0f, 0.0f, 0.0f};
    auto side_loads = [&](int i) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < kLoads<D>; ++j) vx[j] = *reinterpret_cast<const uint4*>(&sm.v8[i & 1][((j * kWaves + w) * 64 + lane) * 16]);
      if (grp == 1 && i + 1 < nt) fin = factor_inputs(sm, (i + 1) % kBufs, tid);
    };
    auto side_widen = [&](int i) __attribute__((always_inline)) {
      const bool vfull = tile_valid(phys(k0 + i), a.ring_head, a.filled, a.slots).count() == kTile;
      widen_store<D>(sm, i & 1, i % kBufs, w, lane, vx, vfull);
    };
    auto side_prep = [&](int i) __attribute__((always_inline)) {
      if (grp != 1 || i + 1 >= nt) return;
      const int bn = (i + 1) % kBufs;
      const TileValid tvd = tile_valid(phys(k0 + i + 1), a.ring_head, a.filled, a.slots);
      tile_factors(sm, bn, tvd, c0, tid, fin);
      if (tvd.count() < kTile) zero_invalid_k(sm, bn, tvd, tid);
    };
    auto side_copies = [&](int i) __attribute__((always_inline)) -> int {
      if (i + 2 >= nt) return 0;
      issue_v<D>(a, sm, i & 1, phys(k0 + i + 2), head, w, lane);
      issue_k<D>(a, sm, (i + 2) % kBufs, phys(k0 + i + 2), head, w, lane);
      return nv + nk;
    };
    auto vphase = [&](int i, bool uniform, float cf, float bf, float ivu) __attribute__((always_inline)) {
      const int bk = i % kBufs;
      softmax_group<D>(sm, bk, g, uniform, cf, bf, ivu, ga);
      softmax_group<D>(sm, bk, g, uniform, cf, bf, ivu, gb);
      wait_vm(0);
      lds_sync();
    };
    if (grp == 1) lds_sync();   // the first group's M_0
    {   // M_0: QK of tile 0, then its side work
      __builtin_amdgcn_s_setprio(1);
      side_loads(0);
      const int4 un = *reinterpret_cast<const int4*>(&sm.uni[0][0]);
      const float cf0 = sm.ck[0][0], bf0 = sm.nb[0][0], iv0 = sm.iv[0][0];
      qk_run<D>(sm.k[0], lo, g, qop, ga, gb);
      __builtin_amdgcn_s_setprio(0);
      const bool uniform = __builtin_amdgcn_readfirstlane(un.x & un.y & un.z & un.w) != 0;
      const float cf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cf0)));
      const float bf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bf0)));
      const float ivu = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(iv0)));
      side_widen(0);
      side_prep(0);
      const int issued = side_copies(0);
      wait_vm(issued);
      lds_sync();
      vphase(0, uniform, cf, bf, ivu);
    }
    constexpr int NPV = NDB * 4;
    for (int i = 1; i < nt; ++i) {   // M_i, V_i
      const uint8_t* vt = sm.v16[(i - 1) & 1];
      __builtin_amdgcn_s_setprio(1);   // the matrix products issue ahead of the other group's softmax
      side_loads(i);
      PvPipe<D> pp;
      pv_start<D>(pp, vt, lo);
      pv_run<0, 4, D>(pp, vt, lo, ga, gb);
      side_widen(i);
      pv_run<4, 8, D>(pp, vt, lo, ga, gb);
      side_prep(i);
      pv_run<8, 12, D>(pp, vt, lo, ga, gb);
      const int issued = side_copies(i);
      pv_run<12, NPV, D>(pp, vt, lo, ga, gb);
      const int4 un = *reinterpret_cast<const int4*>(&sm.uni[i % kBufs][0]);
      const float cf0 = sm.ck[i % kBufs][0], bf0 = sm.nb[i % kBufs][0], iv0 = sm.iv[i % kBufs][0];
      qk_run<D>(sm.k[i % kBufs], lo, g, qop, ga, gb);
      __builtin_amdgcn_s_setprio(0);
      const bool uniform = __builtin_amdgcn_readfirstlane(un.x & un.y & un.z & un.w) != 0;
      const float cf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cf0)));
      const float bf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bf0)));
      const float ivu = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(iv0)));
      wait_vm(issued);
      lds_sync();
      vphase(i, uniform, cf, bf, ivu);
    }
    {   // M_nt: PV of the last tile only
      const uint8_t* vt = sm.v16[(nt - 1) & 1];
      PvPipe<D> pp;
      __builtin_amdgcn_s_setprio(1);
      pv_start<D>(pp, vt, lo);
      pv_run<0, NPV, D>(pp, vt, lo, ga, gb);
      __builtin_amdgcn_s_setprio(0);
      wait_vm(0);
      lds_sync();
    }
    if (grp == 0) lds_sync();   // the second group's M_nt

    // ---- segment result: the row's output, or this segment's part of a split row
    float lt0 = ga.l, lt1 = gb.l;
    lt0 += __shfl_xor(lt0, 16, 64);
    lt0 += __shfl_xor(lt0, 32, 64);
    lt1 += __shfl_xor(lt1, 16, 64);
    lt1 += __shfl_xor(lt1, 32, 64);
    if (!row_split) {
      write_out<D>(a, ga.acc, ga.m, lt0, head, qt, 32 * w + li, g);
      write_out<D>(a, gb.acc, gb.m, lt1, head, qt, 32 * w + 16 + li, g);
    } else {
      const int vf = v - seg;   // the row's first work-group
      const int nseg = split.owner((int64_t)row * a.tv + a.tv - 1) - vf + 1;
      const int64_t blk = (int64_t)row * a.max_seg + seg;
      store_partial<D>(a, blk, ga, lt0, w, 0, lane);
      store_partial<D>(a, blk, gb, lt1, w, 1, lane);
      const int k = ub + nt < ue ? 1 : 0;   // 1: more rows follow in this range
      if (tid == 0) {
        s_merge[k][0] = row;
        s_merge[k][1] = vf;
        s_merge[k][2] = nseg;
        s_merge[k][3] = seg;
      }
      if (k == 1) {
        open_arrive = true;   // counted at the next row's start
      } else {                // the range ends here
        wait_memory();
        lds_sync();           // every thread's stores are complete
        if (tid == 0)
          __hip_atomic_fetch_add(merge_arrivals(a, vf), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    ub += nt;
    row += 1;
    k0 = 0;
    seg = 0;
  }
  // this work-group's share of the merge of its split rows, once all their segments are stored:
  // segment s of a row of nseg takes the row's items s, s + nseg, ..., wavefront w the items
  // s + (w + 8r) nseg for r = 0, 1, ...; a pass merges one item of each row
  lds_sync();
  MergeItem it[2];
  int seq[2];    // first item of this wavefront, per row (>= 32: none)
  int step[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    it[k].row = __builtin_amdgcn_readfirstlane(s_merge[k][0]);
    it[k].nseg = __builtin_amdgcn_readfirstlane(s_merge[k][2]);
    seq[k] = 2 * kRowQ / 16;
    step[k] = 0;
    if (it[k].row >= 0) {
      if (tid == 0) merge_wait(a, s_merge[k][1], it[k].nseg);
      seq[k] = __builtin_amdgcn_readfirstlane(s_merge[k][3]) + w * it[k].nseg;
      step[k] = kWaves * it[k].nseg;
    }
  }
  lds_sync();
  if (tid == 0) {   // done with the counts: the last to leave a row clears them
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (s_merge[k][0] < 0) continue;
      const int vf = s_merge[k][1];
      const int d = __hip_atomic_fetch_add(merge_departures(a, vf), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == s_merge[k][2] - 1) {
        __hip_atomic_store(merge_arrivals(a, vf), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(merge_departures(a, vf), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  constexpr int kItems = 2 * kRowQ / 16;   // 32 items per row
#pragma nounroll
  while (seq[0] < kItems || seq[1] < kItems) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      it[k].on = seq[k] < kItems;
      it[k].gi = seq[k] >> 1;
      it[k].hf = seq[k] & 1;
      seq[k] += step[k];
    }
    merge_items<D>(a, it, lane);
  }
}



struct Plan {
  int qtiles, rows, tv, grid, max_seg, first1, n1, first2, seg_cost;
  int64_t units, cost;
};

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kMaxGrid;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kMaxGrid;
    cached[dev] = n;
  }
  return cached[dev];
}

// Work decomposition of one call; `grid_cap` bounds the persistent grid.
Plan make_plan(int32_t heads, int32_t slots, int32_t nq, int32_t ring_head, int32_t filled, int grid_cap) {
  Plan p;
  const int64_t tiles = tile_count(slots);
  p.qtiles = (nq + kRowQ - 1) / kRowQ;   // rows per head
  p.rows = p.qtiles * heads;
  // tiles holding valid slots: the valid interval [old, old + filled) mod slots as <= 2 runs
  p.first1 = p.n1 = p.first2 = 0;
  if (filled > 0) {
    int old = ring_head - filled;
    old = old < 0 ? old + slots : old;
    const int e1 = old + filled < slots ? old + filled : slots;
    p.first1 = old / kTile;
    p.n1 = (e1 - 1) / kTile - p.first1 + 1;
    if (old + filled > slots) {
      const int e2 = old + filled - slots;
      int last2 = (e2 - 1) / kTile;
      if (last2 >= p.first1) last2 = p.first1 - 1;   // the runs meet in one tile: count it once
      p.first2 = 0;
      const int n2 = last2 + 1;
      // order the runs so that a shared tile is visited once: run 1 then run 2
      p.tv = p.n1 + (n2 > 0 ? n2 : 0);
    } else {
      p.tv = p.n1;
    }
    if (p.tv > tiles) p.tv = int(tiles);
  } else {
    p.tv = 0;
  }
  p.units = (int64_t)p.rows * p.tv;
  p.seg_cost = kSegCost;
  const int64_t span = (int64_t)p.tv + p.seg_cost;   // weight of a row
  p.cost = (int64_t)p.rows * span;
  // every work-group takes a weight of at least ceil(span / 7), so that at most 8 share a row
  int64_t g = grid_cap < kMaxGrid ? grid_cap : kMaxGrid;
  if (p.tv > 0) {
    const int64_t min_w = (span + 6) / 7;
    if (g > p.cost / min_w) g = p.cost / min_w;
    // one work-group per row (no row split, so no merge) when a whole row weighs no more than a
    // share of the split plan plus the cost of splitting, about kMergeCost tiles (the partial
    // stores, the wait for the row's other segments and the merge): the case of a ring holding
    // few tiles, as at the start of its fill-up
    const int64_t cap = grid_cap < kMaxGrid ? grid_cap : kMaxGrid;
    if (p.rows <= cap && g > 0 && span <= (p.cost + g - 1) / g + kMergeCost) g = p.rows;
  }
  p.grid = int(g < 1 ? 1 : g);
  // a row of weight span is shared by at most ceil(span / floor(cost / grid)) + 1 work-groups
  const int64_t per = p.cost / p.grid;
  p.max_seg = p.units > 0 ? int((span + per - 1) / per) + 1 : 1;
  if (p.max_seg > kMaxSeg) p.max_seg = kMaxSeg;
  return p;
}

}  // namespace

namespace {
// Profiling hook (kv_ring_set_attention_events): per host thread, so that a setting made by one
// thread never applies to calls issued by another.
thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;
}

void set_attention_events(void* before, void* after) {
  g_ev_before = static_cast<hipEvent_t>(before);
  g_ev_after = static_cast<hipEvent_t>(after);
}

namespace {

// Workspace layout (floats, each part 16-byte aligned): the per-head synchronisation records
// (kSyncBytes, head_sync; the query preparation takes slot 1) | the split rows' arrival and
// departure counts (two 128-byte lines per work-group of the largest grid; at a fixed offset,
// like the records, so that one zero-filled workspace serves calls of any shape) | split rows' partial
// outputs | their (m, l) | quantised queries | query scales.  Sized for the largest plan any
// (ring_head, filled) and any grid <= 256 can produce (<= 8 segments per row).
constexpr int64_t kMergeCountBytes = (int64_t)kMaxGrid * 2 * kSyncLine;
struct WsLayout {
  int64_t part_o, part_ml, q_codes, q_scale, total;
};

WsLayout ws_layout(int32_t heads, int32_t slots, int32_t head_dim, int32_t nq) {
  auto up4 = [](int64_t x) { return (x + 3) / 4 * 4; };
  const Plan p = make_plan(heads, slots, nq, 0, slots, kMaxGrid);
  WsLayout l;
  l.part_o = (kSyncBytes + kMergeCountBytes) / 4;
  l.part_ml = l.part_o + (int64_t)p.rows * 8 * kRowQ * head_dim / 2;   // half precision
  l.q_codes = l.part_ml + (int64_t)p.rows * 8 * kRowQ * 2;
  l.q_scale = l.q_codes + (int64_t)p.rows * (kRowQ * 128) / 4;   // 128 bytes per query
  l.total = l.q_scale + up4(heads);
  return l;
}

}  // namespace

int64_t attention_workspace_floats(int32_t heads, int32_t slots, int32_t head_dim, int32_t nq) {
  return ws_layout(heads, slots, head_dim, nq).total;
}

AttnWorkspace attention_workspace(float* ws, int32_t heads, int32_t slots, int32_t head_dim,
                                  int32_t nq) {
  const WsLayout l = ws_layout(heads, slots, head_dim, nq);
  AttnWorkspace w;
  w.part_o = ws + l.part_o;
  w.part_ml = ws + l.part_ml;
  w.q_codes = reinterpret_cast<uint8_t*>(ws + l.q_codes);
  w.q_scale = ws + l.q_scale;
  return w;
}

hipError_t launch_attention(const kv_ring_desc& r, int32_t ring_head, int32_t filled,
                            const uint16_t* q, int32_t nq, int64_t q_pos0, const float* rope,
                            float softmax_scale, uint16_t* out, float* lse, float* ws,
                            bool q_ready, hipStream_t stream) {
  const Plan p = make_plan(r.heads, r.slots, nq, ring_head, filled, device_cus());
  const AttnWorkspace aw = attention_workspace(ws, r.heads, r.slots, r.head_dim, nq);
  AttnArgs a;
  a.kc = r.k;
  a.vc = r.v;
  a.k_scale = r.k_scale;
  a.v_scale = r.v_scale;
  a.q_codes = aw.q_codes;
  a.q_scale = aw.q_scale;
  a.out = out;
  a.lse = lse;
  a.part_o = reinterpret_cast<_Float16*>(aw.part_o);
  a.part_ml = aw.part_ml;
  a.merge_cnt = reinterpret_cast<int*>(ws + kSyncBytes / 4);
  a.err = sync_error_word(ws);
  a.tiles = tile_count(r.slots);
  a.heads = r.heads;
  a.slots = r.slots;
  a.ring_head = ring_head;
  a.filled = filled;
  a.nq = nq;
  a.qtiles = p.qtiles;
  a.rows = p.rows;
  a.tv = p.tv;
  a.units = p.units;
  a.cost = p.cost;
  a.seg_cost = p.seg_cost;
  a.grid = p.grid;
  a.max_seg = p.max_seg;
  a.first1 = p.first1;
  a.n1 = p.n1;
  a.first2 = p.first2;
  a.score_scale = softmax_scale * kLog2e;

  hipError_t e = hipSuccess;
  if (!q_ready) {   // else an earlier launch on this stream wrote them
    e = launch_q_prep(q, nq, r.heads, r.head_dim, q_pos0, rope, ws, aw.q_codes, aw.q_scale, stream);
    if (e != hipSuccess) return e;
  }
  // the profiling events are recorded only outside stream capture (a captured record would
  // become a node of the caller's graph)
  bool events = g_ev_before && g_ev_after;
  if (events) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    events = hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone;
  }
  if (events) {
    e = hipEventRecord(g_ev_before, stream);
    if (e != hipSuccess) return e;
  }
  if (p.tv == 0) {
    // empty ring: every row is a single segment with no tiles -> zeros and -inf
    a.units = p.rows;
    a.cost = p.rows;
    a.seg_cost = 0;
    a.tv = 1;
    a.n1 = 0;
    a.grid = p.rows < kMaxGrid ? p.rows : kMaxGrid;
  }
  if (r.head_dim == 128)
    hipLaunchKernelGGL(attn_pp<128>, dim3(a.grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_pp<64>, dim3(a.grid), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess && events) e = hipEventRecord(g_ev_after, stream);
  return e;
}

__global__ void fp8_encode_kernel(const float* __restrict__ x, uint8_t* __restrict__ out, int64_t n) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 + 3 < n) {
    const float4 v = *reinterpret_cast<const float4*>(x + i4);
    *reinterpret_cast<uint32_t*>(out + i4) = e4m3x4(v.x, v.y, v.z, v.w);
  } else {
    for (int64_t i = i4; i < n; ++i) out[i] = uint8_t(e4m3x2(x[i], 0.0f));
  }
}

hipError_t launch_fp8_encode(const float* x, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(fp8_encode_kernel, dim3((threads + 255) / 256), dim3(256), 0, stream, x, out, n);
  return hipGetLastError();
}

}  // namespace kvring
