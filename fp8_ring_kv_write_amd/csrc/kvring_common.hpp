// Shared device helpers for the FP8 ring KV-cache kernels (gfx950).
//
// Cache layout in HBM (per ring = one layer, one GPU's share of heads), tiles of 128 slots:
//   K codes  [heads][tiles][128 * head_dim]  each tile a sequence of 16-byte units in the order
//                                            the QK matrix-core product consumes them
//                                            (k_code_offset)
//   V codes  [heads][tiles][head_dim * 128]  each tile transposed (channel-major), 16-slot
//                                            pieces in the order the attention's widening to
//                                            fp16 reads them (v_code_offset)
//   scales   [heads][slots] float32          dequantisation scale of the write that filled
//                                            each slot (k_scale, v_scale)
// tiles = ceil(slots / 128); slots past `slots` in the last tile are never valid.  With tiles in
// consumption order, a tile moves to LDS as one linear copy and every operand read of the
// attention kernel is one contiguous 1 KB wavefront read (LDS reads at full rate).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvring {

constexpr int kTile = 128;          // slots per ring tile
constexpr int kChunk = 32;          // slots per write/rotate work-group chunk
constexpr float kE4M3Max = 448.0f;
constexpr float kScaleFloor = 0x1p-100f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

__host__ __device__ inline int64_t tile_count(int32_t slots) { return (slots + kTile - 1) / kTile; }

// Byte offset, within one head's K codes, of channels c .. c+15 (c a multiple of 16) of slot s.
// Unit ((bb*2 + r) * (D/32) + g) * 16 + li of a tile holds channels 32g + 16r .. +15 of tile
// slot 32*(li/4) + 4*bb + li%4: what lane (g, li) feeds to the QK product of score block bb as
// the r-th half of its operand.
__host__ __device__ inline int64_t k_code_offset(int64_t s, int c, int D) {
  const int u = int(s % kTile);
  const int li = 4 * (u >> 5) + (u & 3), bb = (u >> 2) & 7, q = c >> 4, g = q >> 1, r = q & 1;
  return (s / kTile) * kTile * D + int64_t((((bb * 2 + r) * (D / 32) + g) * 16 + li) * 16);
}

// Byte offset, within one head's V codes, of slots s .. s+15 (s a multiple of 16) of channel d.
// Unit ((db*2 + r) * 4 + g) * 16 + li of a tile holds tile slots 32g + 16r .. +15 of channel
// 16*db + li: lane (g, li) of the attention widens it into its fp16 PV operands of channel
// block db for slot blocks 2r and 2r + 1.
__host__ __device__ inline int64_t v_code_offset(int64_t s, int d, int D) {
  const int u = int(s % kTile);
  const int g = u >> 5, r = (u >> 4) & 1, db = d >> 4, li = d & 15;
  return (s / kTile) * kTile * D + int64_t((((db * 2 + r) * 4 + g) * 16 + li) * 16);
}

// bfloat16 bit pattern -> float32 (exact).
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// E4M3 (OCP, "fn") encode of two float32 values already scaled into range: round to nearest
// even, saturate to +-448 (the clamp makes the saturation explicit), sign kept.  Returns the
// two codes in the low 16 bits (first value in bits 0..7).
__device__ inline uint32_t e4m3x2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// Four values -> four codes packed in one dword (first value in the low byte).
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  c = __builtin_fminf(__builtin_fmaxf(c, -kE4M3Max), kE4M3Max);
  d = __builtin_fminf(__builtin_fmaxf(d, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return uint32_t(w);
}

// E4M3 decode of the code in byte `sel` (0..3) of w (exact; hardware conversion).
__device__ inline float e4m3_decode(uint32_t w, int sel) {
  v2f two = __builtin_amdgcn_cvt_pk_f32_fp8(int(w >> (16 * (sel >> 1))), false);
  return (sel & 1) ? two[1] : two[0];
}

// Per-head (scale, inverse) from the absmax, both correctly rounded float32 divisions.
__device__ inline void scale_from_absmax(float amax, float& scale, float& inv) {
  const float a = __builtin_fmaxf(amax, kScaleFloor);
  scale = a / kE4M3Max;
  inv = kE4M3Max / a;
}

// Max over the 64 lanes of a wavefront, every lane receiving it, by lane moves only (DPP within
// rows of 16 lanes, then permlane swaps across rows): no LDS traffic and no barrier.  fmaxf
// semantics: a NaN operand is ignored.
__device__ inline float wave_max(float v) {
  auto dpp = [](float x, int ctrl) -> float {
    switch (ctrl) {   // the control must be a constant
      case 0: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0xB1, 0xF, 0xF, false));
      case 1: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x4E, 0xF, 0xF, false));
      case 2: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x141, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x140, 0xF, 0xF, false));
    }
  };
  v = __builtin_fmaxf(v, dpp(v, 0));   // lane ^ 1
  v = __builtin_fmaxf(v, dpp(v, 1));   // lane ^ 2
  v = __builtin_fmaxf(v, dpp(v, 2));   // 7 - lane (of 8)
  v = __builtin_fmaxf(v, dpp(v, 3));   // 15 - lane (of 16): every lane of a row holds its max
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Max over a work-group of 256 threads; `red` is LDS scratch of >= 4 floats used by this call
// only (no other call may share it).  Every thread gets the result.
__device__ inline float block_max_256(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

// Max of n floats at p (a list of partial maxima), every thread of a 256-thread work-group
// receiving it.  Lists of at most 64 entries are reduced by every wavefront on its own (one load
// per lane, lane moves, no barrier); longer ones by the work-group (`red`: LDS scratch of >= 4
// floats used by this call only).  The branch is uniform over the work-group.
__device__ inline float list_max(const float* __restrict__ p, int n, float* red) {
  if (n <= 64) {
    const int lane = threadIdx.x & 63;
    return wave_max(lane < n ? p[lane] : 0.0f);
  }
  float m = 0.0f;
  for (int j = threadIdx.x; j < n; j += 256) m = __builtin_fmaxf(m, p[j]);
  return block_max_256(m, red);
}

// ---- per-head synchronisation inside one launch ------------------------------------------------
//
// An encoding needs the absmax over every element of its head before it can encode any of them.
// The work-groups of one head meet at a record in device memory.  Each reads the record's
// generation g (its parity p selects one of two sets of maxima), adds its partial maxima to set p
// (float bits; every value is >= 0, so unsigned order is float order) and then counts itself in.
// The last one in zeroes set 1 - p and the count for the next launch and bumps the generation;
// the others wait for the generation to change.  Then every work-group reads set p.  A record is
// therefore ready for the next launch as soon as this one's work-groups are all in, with no
// clearing step (graph replays included); a zero-filled record is ready for the first.
//
// Ordering without fences: every operation on a record is an atomic at the device's coherence
// point (agent scope).  Each step depends on the value the previous one returned (the maxima's
// addresses on g, the count-in on the returned old maxima, the generation bump on the count), so
// a work-group's maxima are in before its count, and every count before the bump that releases
// the waiters.  (Acquire and release orderings would add cache write-backs and invalidations to
// every poll, with no other data to publish.)
//
// The wait cannot deadlock: work-groups start in index order on each XCD, and on each XCD a
// head's work-groups all come before the next head's (a grid whose heads are consecutive, or the
// write's XCD-aware order), so the lowest unfinished head always has all of its work-groups
// started or able to start; a head never has more work-groups than fit on one XCD at once (a
// write or query preparation takes at most KV_RING_MAX_TOKENS tokens, about 130 work-groups per
// head on each XCD; a rotation gives each head at most 1,024 work-groups, 128 per XCD).  The wait is bounded all
// the same: past kSpinLimit polls a work-group sets the error word, stops waiting and carries on
// (its output is then not to be trusted), so every launch ends.
//
// Every workspace starts with the records: slot 0 (writes, rotations) and slot 1 (queries) of
// kMaxHeads records each, then the error word; an operation's own data follows kSyncBytes.  A
// record's count, generation and four maxima each have a 128-byte line to themselves, so that
// the atomics on one do not queue behind those on another.
constexpr int kMaxHeads = 512;
constexpr int kSyncLine = 128;
constexpr int kSyncRecordBytes = 6 * kSyncLine;
constexpr int64_t kSyncRecordsBytes = 2LL * kMaxHeads * kSyncRecordBytes;
constexpr int64_t kSyncBytes = kSyncRecordsBytes + 256;
constexpr int kSpinLimit = 1 << 20;

__host__ __device__ inline char* sync_record(void* ws, int slot, int head) {
  return reinterpret_cast<char*>(ws) + ((int64_t)slot * kMaxHeads + head) * kSyncRecordBytes;
}
__host__ __device__ inline int* sync_error_word(void* ws) {
  return reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + kSyncRecordsBytes);
}

// The record's generation, read by thread 0 of a work-group as early as possible (at its start:
// the read then overlaps the work-group's loads) and passed to head_sync.  Other threads get 0.
__device__ inline unsigned head_sync_generation(const char* rec) {
  if (threadIdx.x != 0) return 0u;
  return __hip_atomic_load(reinterpret_cast<const unsigned*>(rec + kSyncLine), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of an NT-thread work-group (uniformly), with g from head_sync_generation:
// v0, v1 are this thread's partial maxima (v1 only with two = true); on return they hold the
// head's maxima over all `expected` work-groups.  `lds` is LDS scratch of >= 2 * NT/64 + 2 floats
// used by this call only.
template <int NT>
__device__ inline void head_sync(char* rec, unsigned g, int* err, int expected, bool two, float& v0,
                                 float& v1, float* lds) {
  constexpr int NW = NT / 64;
  v0 = wave_max(v0);
  if (two) v1 = wave_max(v1);
  if ((threadIdx.x & 63) == 0) {
    lds[threadIdx.x >> 6] = v0;
    lds[NW + (threadIdx.x >> 6)] = two ? v1 : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int* count = reinterpret_cast<int*>(rec);
    unsigned* gen = reinterpret_cast<unsigned*>(rec + kSyncLine);
    auto maxima = [rec](unsigned p, int k) __attribute__((always_inline)) {
      return reinterpret_cast<unsigned*>(rec + (2 + 2 * p + k) * kSyncLine);
    };
    float m0 = lds[0], m1 = lds[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      m0 = __builtin_fmaxf(m0, lds[w]);
      m1 = __builtin_fmaxf(m1, lds[NW + w]);
    }
    const unsigned p = g & 1u;
    unsigned o = __hip_atomic_fetch_max(maxima(p, 0), __float_as_uint(m0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (two) o |= __hip_atomic_fetch_max(maxima(p, 1), __float_as_uint(m1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // o is never 0xFFFFFFFF (finite or +inf bit patterns), so the increment is 1; it depends on
    // the returned old maxima, which orders it after them
    const int one = (o != 0xFFFFFFFFu) ? 1 : 2;
    const int before = __hip_atomic_fetch_add(count, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == expected - 1) {   // the last one in: ready the next launch, release the others
      __hip_atomic_store(maxima(p ^ 1u, 0), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(maxima(p ^ 1u, 1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(count, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gen, g + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      int polls = 0;
      while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
        if (++polls > kSpinLimit) {
          __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    lds[2 * NW] = __uint_as_float(__hip_atomic_load(maxima(p, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    lds[2 * NW + 1] = two ? __uint_as_float(__hip_atomic_load(maxima(p, 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) : 0.0f;
  }
  __syncthreads();
  v0 = lds[2 * NW];
  v1 = lds[2 * NW + 1];
}

// head_sync for work-groups that exchange three maxima of one head over two records (a write
// that also prepares the queries of its own tokens): record A with two maxima (v0, v1) and record
// B with one (w0), the same work-groups taking part in both.  Each work-group adds to the three
// maxima, then counts itself in at A only (the count-in depends on all three returned old
// maxima, so they are in before it); the last one in readies both records for the next launch
// (B's other set of maxima zeroed and its generation bumped as well; B's count is never used
// here and stays zero) and releases the waiters, which poll A's generation alone.  `lds` is LDS
// scratch of >= 3 * NT/64 + 3 floats used by this call only.
template <int NT>
__device__ inline void head_sync_pair(char* ra, unsigned ga, int expected, float& v0, float& v1,
                                      char* rb, unsigned gb, float& w0, int* err, float* lds) {
  constexpr int NW = NT / 64;
  v0 = wave_max(v0);
  v1 = wave_max(v1);
  w0 = wave_max(w0);
  if ((threadIdx.x & 63) == 0) {
    lds[threadIdx.x >> 6] = v0;
    lds[NW + (threadIdx.x >> 6)] = v1;
    lds[2 * NW + (threadIdx.x >> 6)] = w0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    auto maxima = [](char* rec, unsigned p, int k) __attribute__((always_inline)) {
      return reinterpret_cast<unsigned*>(rec + (2 + 2 * p + k) * kSyncLine);
    };
    float m0 = lds[0], m1 = lds[NW], m2 = lds[2 * NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      m0 = __builtin_fmaxf(m0, lds[w]);
      m1 = __builtin_fmaxf(m1, lds[NW + w]);
      m2 = __builtin_fmaxf(m2, lds[2 * NW + w]);
    }
    const unsigned pa = ga & 1u, pb = gb & 1u;
    int* ca = reinterpret_cast<int*>(ra);
    unsigned* gena = reinterpret_cast<unsigned*>(ra + kSyncLine);
    unsigned* genb = reinterpret_cast<unsigned*>(rb + kSyncLine);
    unsigned o = __hip_atomic_fetch_max(maxima(ra, pa, 0), __float_as_uint(m0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    o |= __hip_atomic_fetch_max(maxima(ra, pa, 1), __float_as_uint(m1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    o |= __hip_atomic_fetch_max(maxima(rb, pb, 0), __float_as_uint(m2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // o is never 0xFFFFFFFF (finite or +inf bit patterns), so the increment is 1; it depends on
    // the three returned old maxima, which orders it after them
    const int before = __hip_atomic_fetch_add(ca, (o != 0xFFFFFFFFu) ? 1 : 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == expected - 1) {   // the last one in: ready both records, release the others
      __hip_atomic_store(maxima(ra, pa ^ 1u, 0), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(maxima(ra, pa ^ 1u, 1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(maxima(rb, pb ^ 1u, 0), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(maxima(rb, pb ^ 1u, 1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(genb, gb + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ca, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gena, ga + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      int polls = 0;
      while (__hip_atomic_load(gena, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ga) {
        if (++polls > kSpinLimit) {
          __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    lds[3 * NW] = __uint_as_float(__hip_atomic_load(maxima(ra, pa, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    lds[3 * NW + 1] = __uint_as_float(__hip_atomic_load(maxima(ra, pa, 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    lds[3 * NW + 2] = __uint_as_float(__hip_atomic_load(maxima(rb, pb, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  }
  __syncthreads();
  v0 = lds[3 * NW];
  v1 = lds[3 * NW + 1];
  w0 = lds[3 * NW + 2];
}

// Whether `slot` holds a token of the ring whose valid interval is the `filled` slots just
// before `head` (oldest first).
__device__ inline bool slot_valid(int slot, int head, int filled, int slots) {
  if (slot < 0 || slot >= slots) return false;
  int rel = slot - (head - filled);
  rel = rel < 0 ? rel + slots : rel;
  rel = rel >= slots ? rel - slots : rel;
  return rel < filled;
}

}  // namespace kvring
