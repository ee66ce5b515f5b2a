// ring_attention: attention of the new queries over every valid slot of the FP8 ring
// (Runway Characters abstract: 757 new-token queries against a 5,788-slot cache, 240 calls
// per chunk; cpdf.ai blog, section "Blackwell, escalabilidade e limites do decodificador":
// FP8 attention with per-head scales).
//
// Three launches per call:
//   1. rope_absmax_partials (shared with the write): per-(head, 32-query group) max |RoPE(q)|;
//   2. attn_stream: a persistent grid of one 8-wavefront work-group per compute unit.  The work
//      is the set of units (row, tile), a row being 128 queries of one head and a tile 128 ring
//      slots; each work-group takes an equal contiguous range of units, so a row may be split
//      between work-groups.  A row held by one work-group is finished in place; the segments of
//      a split row store unnormalised partial results.  Consecutive work-groups of one XCD get
//      consecutive units, so the rows of one head share that XCD's L2;
//   3. attn_combine: log-sum-exp merge of the split rows (skipped when no row is split).  Doing
//      the merge in a kernel of its own avoids device-scope fences inside attn_stream, which on
//      this multi-XCD part write back and invalidate L2.
//
// Per tile: K tile and transposed V tile are copied straight from HBM into LDS with
// global_load_lds (16 bytes per lane, XOR-swizzled 16-byte chunks, double-buffered so the next
// tile's copy overlaps this tile's math).  Each wavefront owns 16 queries:
//   S^T = K Q^T           8 MFMA 16x16x128 FP8 (fp32 accumulate)
//   online softmax        log2 domain, lazily rescaled (the running max may lag the true max
//                         by up to 2^4, so P <= 16)
//   P = hi + lo           hi = e4m3(P), lo = e4m3((P - hi) * 2^8)
//   O^T += V^T P^T        8 x 2 MFMA 16x16x128 FP8; the B-operand exponent scale carries
//                         the tile's power-of-two V-scale factor (and 2^-8 for lo)
// Computing S^T rather than S leaves one query per lane with its keys in registers, which is
// exactly the B-operand layout of the PV product: probabilities never leave their lane.
//
// A tile whose 128 slots are all valid and come from one write (one K scale, one V scale) takes
// the fast path: the max runs on raw scores, one FMA forms the exponent, and the V-scale factor
// is folded into it.  Other tiles (ring edges, write boundaries, partially filled rings) take
// the general path with per-slot scales, masking and zeroed V bytes for invalid slots.

#include "kvring_common.hpp"
#include "kvring_internal.hpp"

namespace kvring {

hipError_t launch_q_absmax(const uint16_t* q, int32_t nq, int32_t heads, int32_t head_dim,
                           int64_t q_pos0, const float* rope, float* partial, int* zero,
                           int32_t nzero, hipStream_t stream);

namespace {

constexpr int kWaves = 8;               // 2 wavefronts per SIMD
constexpr int kQB = 1;                  // 16-query blocks per wavefront
constexpr int kThreads = 64 * kWaves;   // 512
constexpr int kRowQ = 16 * kQB * kWaves;  // 128 queries per row
constexpr int kMaxGrid = 256;
constexpr float kTau = 4.0f;            // lazy rescale threshold, log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const float* k_scale;
  const float* v_scale;
  const uint16_t* q;
  const float* rope;
  const float* q_partial;  // [heads][n_qgroups]
  uint16_t* out;
  float* lse;
  float* part_o;           // [rows][max_seg][kRowQ][D]
  float* part_ml;          // [rows][max_seg][kRowQ][2]
  int64_t tiles;           // ring tiles per head
  int64_t q_pos0;
  int64_t units;           // rows * tv
  int32_t heads, slots, ring_head, filled, nq, n_qgroups;
  int32_t qtiles, rows, tv, grid, max_seg;
  int32_t first1, n1, first2;  // valid tiles: logical k < n1 -> first1 + k, else first2 + k - n1
  float score_scale;           // softmax_scale * log2(e)
};

template <int D>
struct Smem {
  uint8_t k[2][kTile * D];
  uint8_t v[2][D * kTile];
  float ks[2][kTile];
  float vs[2][kTile];
  float ckf[kTile];   // general path: c0 * k_scale of valid slots, 0 otherwise
  float nb[kTile];    // general path: 0 for valid slots, -inf otherwise
  float vf[kTile];    // general path: v_scale of valid slots, 0 otherwise
  float red[kWaves];
};

__device__ inline v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
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

// Issue the asynchronous copies of ring tile t (K, transposed V, both scale rows) into buffer b.
// The per-lane offsets are recomputed on every call from a lane index the compiler cannot
// treat as loop-invariant, so they do not stay live in registers across the tile loop.
template <int D>
__device__ inline void issue_tile(const AttnArgs& a, Smem<D>& sm, int b, int64_t t, int h,
                                  int w, int lane_in) {
  constexpr int NCH = D / 16;                   // 16-byte chunks per K row
  constexpr int KCH = kTile * NCH;              // chunks per K tile (= per V tile)
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const uint8_t* kbase = a.kc + ((int64_t)h * a.tiles + t) * (kTile * D);   // uniform
  const uint8_t* vbase = a.vc + ((int64_t)h * a.tiles + t) * (D * kTile);   // uniform
#pragma unroll
  for (int j = 0; j < KCH / kThreads; ++j) {
    const int c0 = (j * kWaves + w) * 64;      // first chunk of this wavefront's copy
    const int c = c0 + lane;
    // K: LDS chunk c = row u, position p holds the row's chunk p ^ (u % NCH)
    const uint32_t koff = uint32_t((c / NCH) * D + (((c % NCH) ^ ((c / NCH) % NCH)) << 4));
    __builtin_amdgcn_global_load_lds(kbase + koff, (lds_ptr)&sm.k[b][c0 * 16], 16, 0, 0);
    // V: LDS chunk c = row d, position p holds the row's chunk p ^ (d % 8)
    const uint32_t voff = uint32_t((c >> 3) * kTile + (((c & 7) ^ ((c >> 3) & 7)) << 4));
    __builtin_amdgcn_global_load_lds(vbase + voff, (lds_ptr)&sm.v[b][c0 * 16], 16, 0, 0);
  }
  if (w < 4) {   // wavefronts 0,1: K scales; 2,3: V scales (64 slots each)
    const int u = (w & 1) * 64 + lane;
    const int slot = min(int(t) * kTile + u, a.slots - 1);   // in bounds; padding masked later
    const float* src = ((w < 2) ? a.k_scale : a.v_scale) + (int64_t)h * a.slots + slot;
    float* dst = (w < 2) ? &sm.ks[b][(w & 1) * 64] : &sm.vs[b][(w & 1) * 64];
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)dst, 4, 0, 0);
  }
}

// P (<= 16, non-negative) -> FP8 hi part and FP8 lo part of (P - hi) * 2^8, four values per dword.
__device__ inline int2 split_p(const float (&p)[4]) {
  int hw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
  hw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hw, true);
  const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
  const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
  v2s lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, p[0] - h01[0], p[1] - h01[1], 0x1p-8f, false);
  lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw, p[2] - h23[0], p[3] - h23[1], 0x1p-8f, true);
  return make_int2(hw, int(uint32_t(uint16_t(lw[0])) | (uint32_t(uint16_t(lw[1])) << 16)));
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_stream(AttnArgs a) {
  constexpr int NCH = D / 16;
  constexpr int NDB = D / 16;
  __shared__ __align__(16) Smem<D> sm;

  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);   // wavefront (uniform)

  // virtual work-group index: consecutive indices on one XCD (work-groups are dealt to the 8
  // XCDs round-robin), so that neighbouring units share an L2
  const int wg = blockIdx.x;
  const int v = (a.grid % 8 == 0) ? (wg % 8) * (a.grid / 8) + wg / 8 : wg;
  auto owner = [&](int64_t u) -> int {   // virtual work-group holding unit u
    return int(((u + 1) * a.grid + a.units - 1) / a.units) - 1;
  };
  int64_t ub = (int64_t)v * a.units / a.grid;
  const int64_t ue = (int64_t)(v + 1) * a.units / a.grid;

  while (ub < ue) {
    // lane-derived values are recomputed per segment from an opaque copy of the thread index, so
    // that the compiler does not hoist dozens of per-lane addresses out of this loop
    int tid = int(threadIdx.x);
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;
    const bool g_live = (D == 128) || (g < 2);
    const int row = int(ub / a.tv);
    const int k0 = int(ub % a.tv);
    const int k1 = int(min<int64_t>(a.tv, k0 + (ue - ub)));
    const int head = row / a.qtiles, qt = row % a.qtiles;
    const int seg = v - owner((int64_t)row * a.tv);
    const int nseg = owner((int64_t)row * a.tv + a.tv - 1) - owner((int64_t)row * a.tv) + 1;

    // ---- query scale of the head, then this wavefront's quantised queries
    float qa = 0.0f;
    for (int j = tid; j < a.n_qgroups; j += kThreads)
      qa = __builtin_fmaxf(qa, a.q_partial[(int64_t)head * a.n_qgroups + j]);
    for (int off = 32; off > 0; off >>= 1) qa = __builtin_fmaxf(qa, __shfl_xor(qa, off, 64));
    if (lane == 0) sm.red[w] = qa;
    __syncthreads();
    qa = sm.red[0];
#pragma unroll
    for (int j = 1; j < kWaves; ++j) qa = __builtin_fmaxf(qa, sm.red[j]);
    float q_scale, q_inv;
    scale_from_absmax(qa, q_scale, q_inv);
    const float c0 = a.score_scale * q_scale;

    v8i qop[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int i = qt * kRowQ + w * (16 * kQB) + qb * 16 + li;
      uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (i < a.nq && g_live) {
        const uint16_t* src = a.q + ((int64_t)i * a.heads + head) * D + 32 * g;
        const float* tab = a.rope + ((a.q_pos0 + i) * (D / 2) + 16 * g) * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // 8 channels (4 pairs) per step
          const uint4 bq = reinterpret_cast<const uint4*>(src)[j];
          const float4 t0 = reinterpret_cast<const float4*>(tab)[2 * j];
          const float4 t1 = reinterpret_cast<const float4*>(tab)[2 * j + 1];
          const uint32_t bw[4] = {bq.x, bq.y, bq.z, bq.w};
          const float cs[4][2] = {{t0.x, t0.y}, {t0.z, t0.w}, {t1.x, t1.y}, {t1.z, t1.w}};
          float y[8];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float xe = __uint_as_float(bw[p] << 16), xo = __uint_as_float(bw[p] & 0xFFFF0000u);
            const float c = cs[p][0], s = cs[p][1];
            y[2 * p] = (xe * c - xo * s) * q_inv;
            y[2 * p + 1] = (xe * s + xo * c) * q_inv;
          }
          wd[2 * j] = e4m3x4(y[0], y[1], y[2], y[3]);
          wd[2 * j + 1] = e4m3x4(y[4], y[5], y[6], y[7]);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) qop[qb][j] = int(wd[j]);
    }

    float m_run[kQB];
    float l_run[kQB];   // this lane's share of the row sums
    v4f acc[kQB][NDB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.0f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[qb][db] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    auto phys = [&](int k) -> int64_t { return k < a.n1 ? a.first1 + k : a.first2 + (k - a.n1); };

    issue_tile<D>(a, sm, 0, phys(k0), head, w, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int k = k0; k < k1; ++k) {
      const int b = (k - k0) & 1;
      const int64_t t = phys(k);
      if (k + 1 < k1) issue_tile<D>(a, sm, b ^ 1, phys(k + 1), head, w, lane);

      const TileValid tvd = tile_valid(t, a.ring_head, a.filled, a.slots);
      const bool full = tvd.count() == kTile;
      const float ks0 = sm.ks[b][0], vs0 = sm.vs[b][0];
      const bool same = sm.ks[b][lane] == ks0 && sm.ks[b][lane + 64] == ks0 &&
                        sm.vs[b][lane] == vs0 && sm.vs[b][lane + 64] == vs0;
      const bool fast = full && __all(same);
      if (!fast) {
        // general path (ring edges, partially filled rings, write boundaries): one cooperative
        // pass stores per-slot factors and zeroes the K/V bytes of invalid slots in LDS before
        // any product reads them, so the math below is branch-free.  `fast` is the same in
        // every wavefront (same LDS data), so the barrier is reached by all.
        for (int u = tid; u < kTile; u += kThreads) {
          const bool ok = tvd.has(u);
          sm.ckf[u] = ok ? c0 * sm.ks[b][u] : 0.0f;
          sm.nb[u] = ok ? 0.0f : -INFINITY;
          sm.vf[u] = ok ? sm.vs[b][u] : 0.0f;
        }
        if (!full) {
          uint8_t* kw = sm.k[b];
          for (int c = tid; c < kTile * NCH; c += kThreads)   // whole 16-byte chunks of K rows
            if (!tvd.has(c / NCH)) *reinterpret_cast<uint4*>(kw + c * 16) = make_uint4(0, 0, 0, 0);
          uint8_t* vw = sm.v[b];
          for (int c = tid; c < D * 8; c += kThreads) {        // 16-byte chunks of V rows
            const int pos0 = ((c & 7) ^ ((c >> 3) & 7)) * 16;   // row position of the chunk's bytes
            uint4 x = *reinterpret_cast<uint4*>(vw + c * 16);
            uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
              const int pp = pos0 + kk;
              const int u = 16 * ((pp & 31) >> 2) + 4 * (pp >> 5) + (pp & 3);   // inverse of vt_pos
              if (!tvd.has(u)) xw[kk >> 2] &= ~(0xFFu << (8 * (kk & 3)));
            }
            *reinterpret_cast<uint4*>(vw + c * 16) = make_uint4(xw[0], xw[1], xw[2], xw[3]);
          }
        }
        __syncthreads();
      }

      // ---- S^T blocks: rows = 16 slots, columns = 16 queries.  All operand reads are issued
      // before the products so that LDS latency is paid once per tile.
      v4f sacc[kQB][8];
      const uint8_t* kt = sm.k[b];
      v8i kop[8];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const int u = 16 * bb + li;
        kop[bb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        if (g_live) {
          const uint4 x0 = *reinterpret_cast<const uint4*>(kt + u * D + (((2 * g) ^ (u % NCH)) << 4));
          const uint4 x1 = *reinterpret_cast<const uint4*>(kt + u * D + (((2 * g + 1) ^ (u % NCH)) << 4));
          kop[bb] = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) sacc[qb][bb] = mfma_fp8(kop[bb], qop[qb], v4f{0, 0, 0, 0}, 127);

      __builtin_amdgcn_sched_barrier(0);
      v8i phi[kQB], plo[kQB];
      int sc_hi, sc_lo;
      if (fast) {
        // one K scale and one V scale over the tile: P' = P * f, f = vs0 * 2^-e in [0.5, 1),
        // folded into the exponent; the MFMA B-scale multiplies back by 2^e
        int e = 0;
        const float f = __builtin_frexpf(vs0, &e);
        const float lf = __log2f(f);
        const float inv_f = 1.0f / f;
        const float c = c0 * ks0;
        sc_hi = 127 + e;
        sc_lo = 127 + e - 8;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          float rmax = sacc[qb][0][0];
#pragma unroll
          for (int bb = 0; bb < 8; ++bb)
#pragma unroll
            for (int r = 0; r < 4; ++r) rmax = __builtin_fmaxf(rmax, sacc[qb][bb][r]);
          rmax = __builtin_fmaxf(rmax, __shfl_xor(rmax, 16, 64));
          rmax = __builtin_fmaxf(rmax, __shfl_xor(rmax, 32, 64));
          const float tmax = rmax * c;
          if (__any(tmax > m_run[qb] + kTau)) {
            const float m_new = __builtin_fmaxf(m_run[qb], tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
            m_run[qb] = m_new;
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[qb][db] *= alpha;
          }
          const float bias = lf - m_run[qb];
          float lsum = 0.0f;
#pragma unroll
          for (int bb = 0; bb < 8; ++bb) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][bb][r], c, bias));
              lsum += p[r];
            }
            const int2 hl = split_p(p);
            phi[qb][bb] = hl.x;
            plo[qb][bb] = hl.y;
          }
          l_run[qb] += lsum * inv_f;
        }
      } else {
        // general path: per-slot factors prepared in LDS before the QK product (see above)
        float vm = __builtin_fmaxf(sm.vf[lane], sm.vf[lane + 64]);
        for (int off = 32; off > 0; off >>= 1) vm = __builtin_fmaxf(vm, __shfl_xor(vm, off, 64));
        int e = 0;
        if (vm > 0.0f) (void)__builtin_frexpf(vm, &e);
        e = max(-120, min(120, e));
        const float finv = __builtin_ldexpf(1.0f, -e);
        sc_hi = 127 + e;
        sc_lo = 127 + e - 8;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          float tmax = -INFINITY;
#pragma unroll
          for (int bb = 0; bb < 8; ++bb) {
            const float4 ck = *reinterpret_cast<const float4*>(&sm.ckf[16 * bb + 4 * g]);
            const float4 nb = *reinterpret_cast<const float4*>(&sm.nb[16 * bb + 4 * g]);
            sacc[qb][bb][0] = __builtin_fmaf(sacc[qb][bb][0], ck.x, nb.x);
            sacc[qb][bb][1] = __builtin_fmaf(sacc[qb][bb][1], ck.y, nb.y);
            sacc[qb][bb][2] = __builtin_fmaf(sacc[qb][bb][2], ck.z, nb.z);
            sacc[qb][bb][3] = __builtin_fmaf(sacc[qb][bb][3], ck.w, nb.w);
#pragma unroll
            for (int r = 0; r < 4; ++r) tmax = __builtin_fmaxf(tmax, sacc[qb][bb][r]);
          }
          tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16, 64));
          tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64));
          if (__any(tmax > m_run[qb] + kTau)) {
            const float m_new = __builtin_fmaxf(m_run[qb], tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
            m_run[qb] = m_new;
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[qb][db] *= alpha;
          }
          const float m_use = m_run[qb] == -INFINITY ? 0.0f : m_run[qb];
#pragma unroll
          for (int bb = 0; bb < 8; ++bb) {
            const float4 vv = *reinterpret_cast<const float4*>(&sm.vf[16 * bb + 4 * g]);
            const float vr[4] = {vv.x, vv.y, vv.z, vv.w};
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float pr = __builtin_amdgcn_exp2f(sacc[qb][bb][r] - m_use);
              l_run[qb] += pr;
              p[r] = pr * (vr[r] * finv);
            }
            const int2 hl = split_p(p);
            phi[qb][bb] = hl.x;
            plo[qb][bb] = hl.y;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- O^T blocks: rows = 16 channels, columns = 16 queries.  Operand reads first; then
      // the hi products of all blocks and the lo products, so that each lo product (same
      // accumulator) follows its hi product by 8 independent ones.
      const uint8_t* vt = sm.v[b];
      v8i vop[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 16 * db + li;
        const uint4 x0 = *reinterpret_cast<const uint4*>(vt + d * kTile + (((2 * g) ^ (d & 7)) << 4));
        const uint4 x1 = *reinterpret_cast<const uint4*>(vt + d * kTile + (((2 * g + 1) ^ (d & 7)) << 4));
        vop[db] = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] = mfma_fp8(vop[db], phi[qb], acc[qb][db], sc_hi);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] = mfma_fp8(vop[db], plo[qb], acc[qb][db], sc_lo);

      __builtin_amdgcn_s_waitcnt(0);   // this thread's copies of the next tile have landed
      __syncthreads();                 // everyone's have, and buffer b is free again
    }

    // ---- segment result: direct output, or partial + merge by the last work-group of the row
    float lt[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      lt[qb] = l_run[qb];
      lt[qb] += __shfl_xor(lt[qb], 16, 64);
      lt[qb] += __shfl_xor(lt[qb], 32, 64);
    }
    if (nseg > 1) {
      // split row: unnormalised partial result; attn_combine merges the row after this kernel
      const int64_t slot0 = ((int64_t)row * a.max_seg + seg) * kRowQ;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int ql = w * (16 * kQB) + qb * 16 + li;
        float* po = a.part_o + (slot0 + ql) * D + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const v4f o = acc[qb][db];
          *reinterpret_cast<float4*>(po + 16 * db) = make_float4(o[0], o[1], o[2], o[3]);
        }
        if (g == 0) *reinterpret_cast<float2*>(a.part_ml + (slot0 + ql) * 2) = make_float2(m_run[qb], lt[qb]);
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int i = qt * kRowQ + w * (16 * kQB) + qb * 16 + li;
        if (i >= a.nq) continue;
        const float il = lt[qb] > 0.0f ? 1.0f / lt[qb] : 0.0f;
        uint16_t* dst = a.out + ((int64_t)i * a.heads + head) * D + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const v4f o = acc[qb][db];
          const uint32_t lo = uint32_t(f32_to_bf16(o[0] * il)) | (uint32_t(f32_to_bf16(o[1] * il)) << 16);
          const uint32_t hi = uint32_t(f32_to_bf16(o[2] * il)) | (uint32_t(f32_to_bf16(o[3] * il)) << 16);
          *reinterpret_cast<uint2*>(dst + 16 * db) = make_uint2(lo, hi);
        }
        if (g == 0)
          a.lse[(int64_t)head * a.nq + i] = lt[qb] > 0.0f ? (m_run[qb] + __log2f(lt[qb])) * kLn2 : -INFINITY;
      }
    }
    __syncthreads();   // LDS buffers are reused by the next segment
    ub += k1 - k0;
  }
}

// Merge of split rows: thread = (query of a row, 4 channels); rows held by one work-group were
// written directly by attn_stream and are skipped.  Segments are merged in order.
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int row = blockIdx.y;
  const auto owner = [&](int64_t u) -> int { return int(((u + 1) * a.grid + a.units - 1) / a.units) - 1; };
  const int first = owner((int64_t)row * a.tv);
  const int nseg = owner((int64_t)row * a.tv + a.tv - 1) - first + 1;
  if (nseg <= 1) return;
  const int item = blockIdx.x * 256 + threadIdx.x;
  const int ql = item / (D / 4), c4 = item % (D / 4);
  if (ql >= kRowQ) return;
  const int head = row / a.qtiles, qt = row % a.qtiles;
  const int i = qt * kRowQ + ql;
  if (i >= a.nq) return;
  const int64_t base = (int64_t)row * a.max_seg * kRowQ + ql;
  float mx = -INFINITY;
  for (int sgi = 0; sgi < nseg; ++sgi) mx = __builtin_fmaxf(mx, a.part_ml[(base + (int64_t)sgi * kRowQ) * 2]);
  float l = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (mx != -INFINITY) {
    for (int sgi = 0; sgi < nseg; ++sgi) {
      const int64_t sl = base + (int64_t)sgi * kRowQ;
      const float wz = __builtin_amdgcn_exp2f(a.part_ml[sl * 2] - mx);
      l += wz * a.part_ml[sl * 2 + 1];
      const float4 oz = *reinterpret_cast<const float4*>(a.part_o + sl * D + 4 * c4);
      o[0] += wz * oz.x;
      o[1] += wz * oz.y;
      o[2] += wz * oz.z;
      o[3] += wz * oz.w;
    }
  }
  const float il = l > 0.0f ? 1.0f / l : 0.0f;
  uint16_t* dst = a.out + ((int64_t)i * a.heads + head) * D + 4 * c4;
  const uint32_t lo = uint32_t(f32_to_bf16(o[0] * il)) | (uint32_t(f32_to_bf16(o[1] * il)) << 16);
  const uint32_t hi = uint32_t(f32_to_bf16(o[2] * il)) | (uint32_t(f32_to_bf16(o[3] * il)) << 16);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  if (c4 == 0) a.lse[(int64_t)head * a.nq + i] = l > 0.0f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
}

struct Plan {
  int qtiles, rows, tv, grid, max_seg, first1, n1, first2;
  int64_t units;
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
  p.qtiles = (nq + kRowQ - 1) / kRowQ;
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
  // every work-group takes at least ceil(tv / 7) units, so that at most 8 share a row
  int64_t g = grid_cap < kMaxGrid ? grid_cap : kMaxGrid;
  if (p.tv > 0) {
    const int64_t min_units = (p.tv + 6) / 7;
    if (g > p.units / min_units) g = p.units / min_units;
  }
  p.grid = int(g < 1 ? 1 : g);
  // a row of tv units spans at most ceil(tv / floor(units / grid)) + 1 work-groups
  const int64_t per = p.units / p.grid;
  p.max_seg = p.units > 0 ? int((p.tv + per - 1) / per) + 1 : 1;
  if (p.max_seg > 8) p.max_seg = 8;
  return p;
}

}  // namespace

namespace {
hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;
}

void set_attention_events(void* before, void* after) {
  g_ev_before = static_cast<hipEvent_t>(before);
  g_ev_after = static_cast<hipEvent_t>(after);
}

int attention_splits(int32_t heads, int32_t slots, int32_t nq) {
  return make_plan(heads, slots, nq, 0, slots, kMaxGrid).max_seg;
}

// Workspace: q partials | partial O | partial (m, l), each 16-byte aligned.  Sized for the
// largest plan any (ring_head, filled) and any grid <= 256 can produce (<= 8 segments per row).
int64_t attention_workspace_floats(int32_t heads, int32_t slots, int32_t head_dim, int32_t nq) {
  const int64_t qparts = ((int64_t)heads * ((nq + 31) / 32) + 3) / 4 * 4;
  const Plan p = make_plan(heads, slots, nq, 0, slots, kMaxGrid);
  const int64_t po = (int64_t)p.rows * 8 * kRowQ * head_dim;
  const int64_t pml = (int64_t)p.rows * 8 * kRowQ * 2;
  return qparts + po + pml;
}

hipError_t launch_attention(const kv_ring_desc& r, int32_t ring_head, int32_t filled,
                            const uint16_t* q, int32_t nq, int64_t q_pos0, const float* rope,
                            float softmax_scale, uint16_t* out, float* lse, float* ws,
                            hipStream_t stream) {
  const Plan p = make_plan(r.heads, r.slots, nq, ring_head, filled, device_cus());
  AttnArgs a;
  a.kc = r.k;
  a.vc = r.v;
  a.k_scale = r.k_scale;
  a.v_scale = r.v_scale;
  a.q = q;
  a.rope = rope;
  a.out = out;
  a.lse = lse;
  a.tiles = tile_count(r.slots);
  a.q_pos0 = q_pos0;
  a.heads = r.heads;
  a.slots = r.slots;
  a.ring_head = ring_head;
  a.filled = filled;
  a.nq = nq;
  a.n_qgroups = (nq + 31) / 32;
  a.qtiles = p.qtiles;
  a.rows = p.rows;
  a.tv = p.tv;
  a.units = p.units;
  a.grid = p.grid;
  a.max_seg = p.max_seg;
  a.first1 = p.first1;
  a.n1 = p.n1;
  a.first2 = p.first2;
  a.score_scale = softmax_scale * kLog2e;
  const int64_t qparts = ((int64_t)r.heads * a.n_qgroups + 3) / 4 * 4;
  a.q_partial = ws;
  a.part_o = ws + qparts;
  a.part_ml = a.part_o + (int64_t)p.rows * 8 * kRowQ * r.head_dim;

  hipError_t e = launch_q_absmax(q, nq, r.heads, r.head_dim, q_pos0, rope, ws, nullptr, 0, stream);
  if (e != hipSuccess) return e;
  if (g_ev_before && g_ev_after) {
    e = hipEventRecord(g_ev_before, stream);
    if (e != hipSuccess) return e;
  }
  if (p.tv == 0) {
    // empty ring: every row is a single segment with no tiles -> zeros and -inf
    a.units = p.rows;
    a.tv = 1;
    a.n1 = 0;
    a.grid = p.rows < kMaxGrid ? p.rows : kMaxGrid;
  }
  if (r.head_dim == 128)
    hipLaunchKernelGGL(attn_stream<128>, dim3(a.grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_stream<64>, dim3(a.grid), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess && g_ev_before && g_ev_after) e = hipEventRecord(g_ev_after, stream);
  if (e != hipSuccess) return e;
  bool split = false;   // does any row span more than one work-group?
  for (int row = 0; row < p.rows && !split; ++row) {
    const auto owner = [&](int64_t u) { return ((u + 1) * a.grid + a.units - 1) / a.units - 1; };
    split = owner((int64_t)row * a.tv + a.tv - 1) != owner((int64_t)row * a.tv);
  }
  if (!split) return e;
  dim3 gc((kRowQ * r.head_dim / 4 + 255) / 256, p.rows);
  if (r.head_dim == 128)
    hipLaunchKernelGGL(attn_combine<128>, gc, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_combine<64>, gc, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Exposed E4M3 encoder (the one the kernels use), for exhaustive checking.
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
