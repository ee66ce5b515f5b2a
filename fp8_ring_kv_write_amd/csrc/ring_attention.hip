// ring_attention: attention of the new queries over every valid slot of the FP8 ring
// (Runway Characters abstract: 757 new-token queries against a 5,788-slot cache, 240 calls
// per chunk; cpdf.ai blog, section "Blackwell, escalabilidade e limites do decodificador":
// FP8 attention with per-head scales).
//
// Steps of one call:
//   1. rope_absmax_partials (shared with the write): per-(head, 32-query group) max |RoPE(q)|;
//   2. attn_main: one work-group = 128 queries x 1 head x one range of 128-slot tiles.
//      Prologue: reduce the head's Q partials, rotate and quantise the work-group's queries
//      into matrix-core operand registers.  Per tile: K tile and transposed V tile staged in
//      LDS (XOR-swizzled 16-byte chunks), S^T = K Q^T with FP8 MFMA (16x16x128), per-slot K
//      scale and mask, online softmax in the log2 domain, P split into an FP8 hi part and an
//      FP8 lo part (residual x 2^8), O^T += V^T P^T with FP8 MFMA whose B-operand exponent
//      scale carries the tile's power-of-two V-scale factor (and 2^-8 for the lo part).
//   3. attn_combine (only when the key range is split): log-sum-exp merge of the partials.
//
// Computing S^T rather than S puts one query per lane with its keys in registers, which is
// exactly the B-operand layout of the PV product: probabilities never leave their lane.

#include "kvring_common.hpp"
#include "kvring_internal.hpp"

namespace kvring {

hipError_t launch_q_absmax(const uint16_t* q, int32_t nq, int32_t heads, int32_t head_dim,
                           int64_t q_pos0, const float* rope, float* partial, hipStream_t stream);

namespace {

constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kQTile = 128;     // queries per work-group (32 per wavefront)
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
  float* o_part;   // [nsplit][heads][nq_pad][D] when nsplit > 1
  float* ml_part;  // [nsplit][heads][nq_pad][2]
  int64_t tiles;
  int64_t q_pos0;
  int32_t heads, slots, ring_head, filled, nq, nq_pad, nsplit, n_qgroups;
  float score_scale;  // softmax_scale * log2(e)
};

__device__ inline v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

// Valid slots of tile t: count of [128t, min(128t+128, slots)) inside the ring's interval.
__device__ inline int tile_valid_count(int64_t t, int head, int filled, int slots) {
  const int lo = int(t) * kTile;
  const int hi = min(lo + kTile, slots);
  int old = head - filled;
  old = old < 0 ? old + slots : old;
  const int e1 = min(old + filled, slots);
  const int e2 = old + filled - slots;  // wrapped part [0, e2)
  int c = max(0, min(hi, e1) - max(lo, old));
  if (e2 > 0) c += max(0, min(hi, e2) - lo);
  return c;
}

__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_main(AttnArgs a) {
  constexpr int NCH = D / 16;   // 16-byte chunks per K row
  constexpr int NDB = D / 16;   // 16-channel blocks of the output
  __shared__ __align__(16) uint8_t kt[kTile * D];
  __shared__ __align__(16) uint8_t vt[D * kTile];
  __shared__ __align__(16) float csc[kTile];
  __shared__ __align__(16) float vsc[kTile];
  __shared__ float red[4];

  const int h = blockIdx.y, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const bool g_live = (D == 128) || (g < 2);   // lane groups that carry channels

  // ---- prologue: the head's query scale and this work-group's quantised queries
  float qa = 0.0f;
  for (int j = tid; j < a.n_qgroups; j += kThreads)
    qa = __builtin_fmaxf(qa, a.q_partial[(int64_t)h * a.n_qgroups + j]);
  qa = block_max_256(qa, red);
  float q_scale, q_inv;
  scale_from_absmax(qa, q_scale, q_inv);
  const float c0 = a.score_scale * q_scale;

  v8i qop[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = blockIdx.x * kQTile + w * 32 + qb * 16 + li;
    uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (i < a.nq && g_live) {
      const uint16_t* src = a.q + ((int64_t)i * a.heads + h) * D + 32 * g;
      const float* tab = a.rope + ((a.q_pos0 + i) * (D / 2) + 16 * g) * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {   // 8 channels (4 pairs) per step
        const uint4 b = reinterpret_cast<const uint4*>(src)[j];
        const float4 t0 = reinterpret_cast<const float4*>(tab)[2 * j];
        const float4 t1 = reinterpret_cast<const float4*>(tab)[2 * j + 1];
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
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

  // ---- main loop over this split's tiles
  const int64_t t_begin = (int64_t)z * a.tiles / a.nsplit;
  const int64_t t_end = (int64_t)(z + 1) * a.tiles / a.nsplit;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.0f, 0.0f};   // this lane's share of the row sum
  v4f acc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const uint8_t* kc_h = a.kc + (int64_t)h * a.tiles * kTile * D;
  const uint8_t* vc_h = a.vc + (int64_t)h * a.tiles * D * kTile;

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int nvalid = tile_valid_count(t, a.ring_head, a.filled, a.slots);
    if (nvalid == 0) continue;
    const bool full = nvalid == kTile;

    // K tile: 128 rows x D bytes, chunk c of row u stored at chunk c ^ (u % NCH)
    for (int c = tid; c < kTile * NCH; c += kThreads) {
      const int u = c / NCH, ch = c % NCH;
      const uint4 val = *reinterpret_cast<const uint4*>(kc_h + (t * kTile + u) * D + ch * 16);
      *reinterpret_cast<uint4*>(kt + u * D + ((ch ^ (u % NCH)) << 4)) = val;
    }
    // V tile: D rows x 128 bytes (already transposed in HBM); invalid slots zeroed so that a
    // NaN code in an unused slot cannot reach the accumulator through 0 * NaN
    for (int c = tid; c < D * 8; c += kThreads) {
      const int d = c >> 3, ch = c & 7;
      uint4 val = *reinterpret_cast<const uint4*>(vc_h + (t * D + d) * kTile + ch * 16);
      if (!full) {
        uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int p = ch * 16 + k;                              // byte position in the row
          const int u = 16 * ((p & 31) >> 2) + 4 * (p >> 5) + (p & 3);   // slot (inverse of vt_pos)
          if (!slot_valid(int(t) * kTile + u, a.ring_head, a.filled, a.slots))
            wv[k >> 2] &= ~(0xFFu << (8 * (k & 3)));
        }
        val = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
      *reinterpret_cast<uint4*>(vt + d * kTile + ((ch ^ (d & 7)) << 4)) = val;
    }
    if (tid < kTile) {
      const int s = int(t) * kTile + tid;
      const bool ok = slot_valid(s, a.ring_head, a.filled, a.slots);
      csc[tid] = ok ? c0 * a.k_scale[(int64_t)h * a.slots + s] : 0.0f;
      vsc[tid] = ok ? a.v_scale[(int64_t)h * a.slots + s] : 0.0f;
    }
    __syncthreads();

    // power-of-two exponent of the tile's largest V scale: P is multiplied by
    // v_scale * 2^-e (<= 1) before FP8 and the matrix core multiplies back by 2^e
    float vmax = __builtin_fmaxf(vsc[lane], vsc[lane + 64]);
    for (int off = 32; off > 0; off >>= 1) vmax = __builtin_fmaxf(vmax, __shfl_xor(vmax, off, 64));
    int e = 0;
    if (vmax > 0.0f) (void)__builtin_frexpf(vmax, &e);   // vmax = f * 2^e, f in [0.5, 1)
    e = max(-120, min(120, e));
    const float finv = __builtin_ldexpf(1.0f, -e);
    const int sc_hi = 127 + e, sc_lo = 127 + e - 8;

    // S^T blocks: rows = 16 slots, columns = 16 queries
    v4f sacc[2][8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int u = 16 * b + li;
      v8i kop;
      if (g_live) {
        const uint4 k0 = *reinterpret_cast<const uint4*>(kt + u * D + (((2 * g) ^ (u % NCH)) << 4));
        const uint4 k1 = *reinterpret_cast<const uint4*>(kt + u * D + (((2 * g + 1) ^ (u % NCH)) << 4));
        kop = v8i{int(k0.x), int(k0.y), int(k0.z), int(k0.w), int(k1.x), int(k1.y), int(k1.z), int(k1.w)};
      } else {
        kop = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sacc[qb][b] = mfma_fp8(kop, qop[qb], v4f{0, 0, 0, 0}, 127);
    }

    v8i phi[2], plo[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float tv[8][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const float4 cv = *reinterpret_cast<const float4*>(&csc[16 * b + 4 * g]);
        const float cr[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tv[b][r] = cr[r] > 0.0f ? sacc[qb][b][r] * cr[r] : -INFINITY;
          tmax = __builtin_fmaxf(tmax, tv[b][r]);
        }
      }
      tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = __builtin_fmaxf(m_run[qb], tmax);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
      m_run[qb] = m_new;
      l_run[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[qb][db] *= alpha;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const float4 fv = *reinterpret_cast<const float4*>(&vsc[16 * b + 4 * g]);
        const float fr[4] = {fv.x, fv.y, fv.z, fv.w};
        float pp[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(tv[b][r] - m_use);
          l_run[qb] += p;
          pp[r] = p * (fr[r] * finv);
        }
        const uint32_t hw = e4m3x4(pp[0], pp[1], pp[2], pp[3]);
        float res[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) res[r] = (pp[r] - e4m3_decode(hw, r)) * 256.0f;
        phi[qb][b] = int(hw);
        plo[qb][b] = int(e4m3x4(res[0], res[1], res[2], res[3]));
      }
    }

    // O^T blocks: rows = 16 channels, columns = 16 queries
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 16 * db + li;
      const uint4 v0 = *reinterpret_cast<const uint4*>(vt + d * kTile + (((2 * g) ^ (d & 7)) << 4));
      const uint4 v1 = *reinterpret_cast<const uint4*>(vt + d * kTile + (((2 * g + 1) ^ (d & 7)) << 4));
      const v8i vop = v8i{int(v0.x), int(v0.y), int(v0.z), int(v0.w), int(v1.x), int(v1.y), int(v1.z), int(v1.w)};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        acc[qb][db] = mfma_fp8(vop, phi[qb], acc[qb][db], sc_hi);
        acc[qb][db] = mfma_fp8(vop, plo[qb], acc[qb][db], sc_lo);
      }
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l_run[qb];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int i = blockIdx.x * kQTile + w * 32 + qb * 16 + li;
    if (i >= a.nq) continue;
    if (a.nsplit == 1) {
      const float il = lt > 0.0f ? 1.0f / lt : 0.0f;
      uint16_t* dst = a.out + ((int64_t)i * a.heads + h) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4f o = acc[qb][db];
        const uint32_t lo = uint32_t(f32_to_bf16(o[0] * il)) | (uint32_t(f32_to_bf16(o[1] * il)) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16(o[2] * il)) | (uint32_t(f32_to_bf16(o[3] * il)) << 16);
        *reinterpret_cast<uint2*>(dst + 16 * db) = make_uint2(lo, hi);
      }
      if (g == 0) a.lse[(int64_t)h * a.nq + i] = lt > 0.0f ? (m_run[qb] + __log2f(lt)) * kLn2 : -INFINITY;
    } else {
      const int64_t row = ((int64_t)z * a.heads + h) * a.nq_pad + i;
      float* dst = a.o_part + row * D + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4f o = acc[qb][db];
        *reinterpret_cast<float4*>(dst + 16 * db) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (g == 0) {
        a.ml_part[row * 2] = m_run[qb];
        a.ml_part[row * 2 + 1] = lt;
      }
    }
  }
}

// Merge of the per-split partials: thread = (query, 4 channels).
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int h = blockIdx.y;
  const int item = blockIdx.x * 256 + threadIdx.x;
  const int i = item / (D / 4), c4 = item % (D / 4);
  if (i >= a.nq) return;
  float mx = -INFINITY;
  for (int z = 0; z < a.nsplit; ++z) {
    const int64_t row = ((int64_t)z * a.heads + h) * a.nq_pad + i;
    if (a.ml_part[row * 2 + 1] > 0.0f) mx = __builtin_fmaxf(mx, a.ml_part[row * 2]);
  }
  float l = 0.0f, o[4] = {0, 0, 0, 0};
  if (mx != -INFINITY) {
    for (int z = 0; z < a.nsplit; ++z) {
      const int64_t row = ((int64_t)z * a.heads + h) * a.nq_pad + i;
      const float lz = a.ml_part[row * 2 + 1];
      if (!(lz > 0.0f)) continue;
      const float wz = __builtin_amdgcn_exp2f(a.ml_part[row * 2] - mx);
      l += wz * lz;
      const float4 oz = *reinterpret_cast<const float4*>(a.o_part + row * D + 4 * c4);
      o[0] += wz * oz.x;
      o[1] += wz * oz.y;
      o[2] += wz * oz.z;
      o[3] += wz * oz.w;
    }
  }
  const float il = l > 0.0f ? 1.0f / l : 0.0f;
  uint16_t* dst = a.out + ((int64_t)i * a.heads + h) * D + 4 * c4;
  const uint32_t lo = uint32_t(f32_to_bf16(o[0] * il)) | (uint32_t(f32_to_bf16(o[1] * il)) << 16);
  const uint32_t hi = uint32_t(f32_to_bf16(o[2] * il)) | (uint32_t(f32_to_bf16(o[3] * il)) << 16);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  if (c4 == 0) a.lse[(int64_t)h * a.nq + i] = l > 0.0f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
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
  const int64_t wgs = (int64_t)((nq + kQTile - 1) / kQTile) * heads;
  const int64_t tiles = tile_count(slots);
  int64_t s = (512 + wgs - 1) / wgs;   // aim at >= 512 work-groups (2 per compute unit)
  if (s > tiles) s = tiles;
  if (s > 64) s = 64;
  return int(s < 1 ? 1 : s);
}

int64_t attention_workspace_floats(int32_t heads, int32_t slots, int32_t head_dim, int32_t nq) {
  const int64_t qparts = (int64_t)heads * ((nq + 31) / 32);
  const int ns = attention_splits(heads, slots, nq);
  int64_t parts = 0;
  if (ns > 1) {
    const int64_t nq_pad = (int64_t)((nq + kQTile - 1) / kQTile) * kQTile;
    parts = (int64_t)ns * heads * nq_pad * (head_dim + 2);
  }
  // q partials first, then the split partials 16-byte aligned
  return ((qparts + 3) / 4) * 4 + parts;
}

hipError_t launch_attention(const kv_ring_desc& r, int32_t ring_head, int32_t filled,
                            const uint16_t* q, int32_t nq, int64_t q_pos0, const float* rope,
                            float softmax_scale, uint16_t* out, float* lse, float* ws,
                            hipStream_t stream) {
  hipError_t e = launch_q_absmax(q, nq, r.heads, r.head_dim, q_pos0, rope, ws, stream);
  if (e != hipSuccess) return e;
  AttnArgs a;
  a.kc = r.k;
  a.vc = r.v;
  a.k_scale = r.k_scale;
  a.v_scale = r.v_scale;
  a.q = q;
  a.rope = rope;
  a.q_partial = ws;
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
  a.nq_pad = ((nq + kQTile - 1) / kQTile) * kQTile;
  a.nsplit = attention_splits(r.heads, r.slots, nq);
  a.score_scale = softmax_scale * kLog2e;
  const int64_t qparts = ((int64_t)r.heads * a.n_qgroups + 3) / 4 * 4;
  a.o_part = ws + qparts;
  a.ml_part = a.o_part + (int64_t)a.nsplit * r.heads * a.nq_pad * r.head_dim;
  dim3 grid(a.nq_pad / kQTile, r.heads, a.nsplit);
  if (g_ev_before && g_ev_after) {
    e = hipEventRecord(g_ev_before, stream);
    if (e != hipSuccess) return e;
  }
  if (r.head_dim == 128)
    hipLaunchKernelGGL(attn_main<128>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_main<64>, grid, dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess && g_ev_before && g_ev_after) e = hipEventRecord(g_ev_after, stream);
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int items = nq * (r.head_dim / 4);
  dim3 g2((items + 255) / 256, r.heads);
  if (r.head_dim == 128)
    hipLaunchKernelGGL(attn_combine<128>, g2, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_combine<64>, g2, dim3(256), 0, stream, a);
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
