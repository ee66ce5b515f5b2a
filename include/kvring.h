/*
 * kvring.h -- C ABI of the MI355X (gfx950) FP8 ring KV cache.
 *
 * What it computes (Runway Characters: Serving a 57B Video Diffusion Transformer for
 * Real-Time Conversation, arXiv 2611.05642):
 *   - abstract: each of the 240 attention calls of a four-frame chunk reads a 5,788-slot KV
 *     cache of which 757 tokens are new; the whole-cache work that used to repeat in every
 *     call is moved to write time: a ring cache, RoPE and FP8 quantisation applied once per
 *     write, and a delta rotation of the cache when positions reset;
 *   - cpdf.ai blog, section "Como rodar 57B em tempo real com batch size 1": rotary positions
 *     and FP8 quantisation are applied as a frame enters the cache, and the ring lets the
 *     window advance without copies;
 *   - cpdf.ai blog, section "Blackwell, escalabilidade e limites do decodificador": the
 *     attention kernel reads the FP8 cache with per-head scales.
 *
 * Readings where the pages are silent (the CPU oracle states the same ones):
 *   - RoPE: 1-D positions, interleaved channel pairs (2i, 2i+1), theta_i = base^(-2i/D),
 *     x' = x cos - y sin, y' = x sin + y cos in float32 with every operation rounded; cos/sin
 *     come from a float64 C-library table rounded once to float32 (kv_ring_rope_table);
 *   - FP8 is OCP E4M3 (max 448), round to nearest even, saturating;
 *   - scales are per head and per write: A = max |x| over the write's tokens and channels of a
 *     head (K after rotation, V as is), floored at 2^-100; scale = A/448, stored for every slot
 *     the write fills; codes = e4m3(x * (448/A));
 *   - the ring's valid slots are the `filled` slots just before `ring_head`, oldest first;
 *   - attention is non-causal over all valid slots, one KV head per query head; queries are
 *     rotated at their positions and quantised to FP8 with one scale per head per call.
 *
 * Conventions for every entry point:
 *   - pointers named "device" are HIP device memory owned by the caller; the library never
 *     allocates, frees or keeps them;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *     returns without synchronising;
 *   - the return value is KV_RING_OK (0) or a negative status; arguments are checked before
 *     anything is enqueued, and on an argument error nothing is launched and nothing written;
 *   - no call allocates memory: scratch space is the caller's `workspace`, sized by
 *     kv_ring_workspace_bytes; the workspace must not be shared by calls that may overlap;
 *   - every workspace starts with the per-head synchronisation records through which the
 *     work-groups of one launch agree on a head's absmax (kv_ring_workspace_bytes counts them):
 *     the caller zero-fills a workspace once, before its first use, and every call leaves the
 *     records ready for the next (graph replays included), so one workspace serves every
 *     operation and every ring shape in turn.  An attention workspace also holds, right after
 *     the records, the counts through which the work-groups sharing a query row merge their
 *     partial results (left at zero by every call as well).  A wait that exceeds its bound (no
 *     such wait arises in correct use) sets a word of the workspace instead of hanging;
 *     kv_ring_sync_status reads it.
 */
#ifndef KVRING_H
#define KVRING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KV_RING_OK = 0,
  KV_RING_ERR_NULL = -1,       /* a required pointer is NULL                         */
  KV_RING_ERR_ALIGN = -2,      /* a pointer is not aligned as documented               */
  KV_RING_ERR_SHAPE = -3,      /* heads, slots or head_dim unsupported                 */
  KV_RING_ERR_RANGE = -4,      /* n, start_slot, ring_head, filled or nq out of range  */
  KV_RING_ERR_POSITION = -5,   /* a position falls outside the rotary table            */
  KV_RING_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than required              */
  KV_RING_ERR_LAUNCH = -7,     /* a kernel launch failed (HIP error)                   */
  KV_RING_ERR_SCRATCH = -8,    /* kv_ring_write_static: the call does not fit its scratch */
  KV_RING_ERR_SYNC = -9        /* kv_ring_sync_status: a wait exceeded its bound       */
};

/* The most new tokens one write takes, and the most queries one attention call takes.  Their
 * work-groups agree on each head's absmax inside one launch, which needs all of a head's
 * work-groups on the GPU at once; this bound keeps them within what every XCD holds together
 * (a delta rotation of any ring the library accepts stays within it by itself). */
#define KV_RING_MAX_TOKENS 16384

enum {
  KV_RING_OP_WRITE = 1,
  KV_RING_OP_DELTA_ROTATE = 2,
  KV_RING_OP_ATTENTION = 3,
  KV_RING_OP_WRITE_ATTEND = 4
};

/*
 * One ring (one layer, one GPU's share of heads).  All four buffers are device memory of the
 * caller, 16-byte aligned.  With T = ceil(slots / 128) tiles of 128 slots, the code buffers hold
 * per head T tiles of 128*head_dim bytes each, every tile a sequence of 16-byte units in the
 * order the attention's matrix-core products consume them:
 *   k        K codes.  Unit ((bb*2 + r)*(head_dim/32) + g)*16 + li of tile t holds channels
 *            32g + 16r .. +15 (in order) of slot 128t + 32*(li/4) + 4*bb + li%4
 *            (bb 0..7, r 0..1, g 0..head_dim/32-1, li 0..15);
 *   v        V codes, each tile transposed.  Unit ((db*2 + r)*4 + g)*16 + li of tile t holds
 *            channel 16*db + li of slots 128t + 32g + 16r .. +15 (in order)
 *            (db 0..head_dim/16-1, r 0..1, g 0..3, li 0..15);
 *   k_scale  float32 [heads][slots], the dequantisation scale of the write that filled a slot;
 *   v_scale  float32 [heads][slots].
 * Byte b of unit n of tile t of head h is at byte ((h*T + t)*128*head_dim + 16n + b).
 * Limits: 1 <= heads <= 512, 1 <= slots <= 1048576, head_dim in {64, 128}.
 * Bytes of the last tile for slots past `slots` are padding and never read as data.
 */
typedef struct kv_ring_desc {
  uint8_t *k;
  uint8_t *v;
  float *k_scale;
  float *v_scale;
  int32_t heads;
  int32_t slots;
  int32_t head_dim;
} kv_ring_desc;

/* Bytes of one of the two code buffers (k or v): heads * ceil(slots/128) * 128 * head_dim. */
int64_t kv_ring_codes_bytes(int32_t heads, int32_t slots, int32_t head_dim);

/* Byte offset, within one head's K codes (kv_ring_k_offset) or V codes (kv_ring_v_offset), of
 * channel `channel` of slot `slot`, per the layout above.  Host only; -1 for a negative slot, a
 * channel outside 0..head_dim-1 or an unsupported head_dim. */
int64_t kv_ring_k_offset(int64_t slot, int32_t channel, int32_t head_dim);
int64_t kv_ring_v_offset(int64_t slot, int32_t channel, int32_t head_dim);

/*
 * Fill a host float32 table [n_pos][head_dim/2][2] with cos and sin of p * theta_i for
 * positions p in 0..n_pos-1: theta_i = pow(base, -(2i)/head_dim), angle = (double)p*theta_i,
 * each value computed in double by the C library and rounded once to float.  The caller
 * copies it to the device and passes it to kv_ring_write and ring_attention.
 * Errors: NULL out, n_pos < 1, head_dim not in {64, 128}, base <= 0.
 */
int kv_ring_rope_table(float *host_out, int64_t n_pos, int32_t head_dim, double base);

/*
 * Three-axis positions for a video cache (the model of the pages is a video diffusion
 * transformer; the pages do not give its rotary variant, so this is a reading).  A token's
 * position is (t, y, x): frame, row, column.  The head_dim/2 interleaved pairs are cut into
 * three contiguous bands, frame first, then row, then column, of band_pairs[0..2] pairs (NULL:
 * row and column floor(head_dim/6) each, frame the rest: 22/21/21 at 128, 12/10/10 at 64);
 * pair j of band b turns by coordinate_b * pow(base, -(2j)/(2 * band_pairs[b])), i.e. each band
 * is kv_ring_rope_table's embedding of dimension 2 * band_pairs[b] on its own coordinate.
 * Fills a host float32 table [n][head_dim/2][2] with one row per token (cos and sin computed in
 * double by the C library, rounded once to float), for positions = host int32 [n][3].  Such a
 * table serves kv_ring_write and ring_attention unchanged: pass it with pos0 = 0 (q_pos0 = 0)
 * and rope_n_pos = n, and token i of the call is rotated by row i.
 * Errors: NULL pointers, n < 1, head_dim not in {64, 128}, base <= 0, band_pairs negative or
 * not summing to head_dim/2.
 */
int kv_ring_rope_table_3d(float *host_out, const int32_t *positions, int64_t n, int32_t head_dim,
                          const int32_t *band_pairs, double base);

/* Workspace bytes for `op` (KV_RING_OP_*) with n = new tokens (write), unused (delta
 * rotate), nq = queries (attention) or the larger of the two (write + attention).  Returns 0
 * for an unknown op or invalid shape.  Every workspace starts with the same synchronisation
 * records (786,688 bytes), zero-filled by the caller before first use; attention workspaces
 * (KV_RING_OP_ATTENTION, KV_RING_OP_WRITE_ATTEND) follow them with 65,536 bytes of split-row
 * counts. */
size_t kv_ring_workspace_bytes(int32_t op, int32_t heads, int32_t slots, int32_t head_dim,
                               int32_t n);

/* Whether any wait of the calls made with `workspace` (device memory) on another work-group of
 * the same launch (a head's record, a split row's count) has exceeded its bound: copies one word
 * of it to the host, waiting for `stream` first.  KV_RING_OK, or
 * KV_RING_ERR_SYNC (the outputs of those calls are then not to be trusted, and the workspace must
 * be zero-filled again before further use: its counts may not be back at zero), KV_RING_ERR_NULL,
 * KV_RING_ERR_ALIGN (workspace not 16-byte aligned), KV_RING_ERR_LAUNCH (a HIP error). */
int kv_ring_sync_status(const void *workspace, void *stream);

/*
 * Write n new tokens into the ring (abstract: RoPE and FP8 quantisation applied once per
 * write; cpdf.ai blog, "Como rodar 57B...": done as the frame enters the cache).
 *   k_new, v_new  device bfloat16 [n][heads][head_dim], 16-byte aligned; token i has
 *                 absolute position pos0 + i and goes to slot (start_slot + i) % slots;
 *   rope_table    device float32 table from kv_ring_rope_table with rope_n_pos positions;
 * K is rotated, K and V each get one scale per head over this write, codes and scales are
 * stored.  The caller then sets ring_head = (start_slot + n) % slots and
 * filled = min(filled + n, slots).
 * Errors: NULL pointers, misalignment, 1 <= n <= min(slots, KV_RING_MAX_TOKENS),
 * 0 <= start_slot < slots, 0 <= pos0 and pos0 + n <= rope_n_pos, workspace too small.
 */
int kv_ring_write(const kv_ring_desc *ring, const void *k_new, const void *v_new, int32_t n,
                  int32_t start_slot, int64_t pos0, const float *rope_table, int64_t rope_n_pos,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_ring_write without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same kernels,
 * arguments (less the workspace), results and errors as kv_ring_write; its scratch (the
 * per-head synchronisation records) is a static device array of the library, 768 KiB per GPU,
 * zero when the library loads and left ready for the next call by every call, held until the
 * process ends.
 * Limit: the records of 512 heads, which every ring the library accepts fits (a call that did
 * not fit would return KV_RING_ERR_SCRATCH with nothing launched).  The call allocates nothing.
 * All calls on one GPU share its scratch: calls that may overlap on one GPU (different streams,
 * or different host threads without ordering) race and must not be made.
 */
int kv_ring_write_static(const kv_ring_desc *ring, const void *k_new, const void *v_new, int32_t n,
                         int32_t start_slot, int64_t pos0, const float *rope_table,
                         int64_t rope_n_pos, void *stream);

/*
 * Delta rotation when positions reset (abstract: a delta rotation of the cache instead of
 * re-rotating it): every valid K slot is dequantised, rotated by delta positions (cos/sin of
 * delta * theta_i from the C library, in double, rounded to float) and requantised with one
 * new scale per head over all valid slots.  V and invalid slots are untouched.  One launch, one
 * read of the K codes; a ring of more than 1,024 tiles (131,072 slots) is read twice (once for
 * the absmax, once to encode).
 *   ring_head, filled  the ring's valid interval (0 <= ring_head < slots, 0 <= filled <= slots);
 *   delta              position offset, |delta| < 2^31; rope_base > 0.
 * The caller continues positions from old + delta.
 */
int kv_ring_delta_rotate(const kv_ring_desc *ring, int32_t ring_head, int32_t filled,
                         int64_t delta, double rope_base, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * The delta rotation for three-axis positions (bands as in kv_ring_rope_table_3d): every valid
 * K slot moves by the offset triple delta = host int64 [3] (dt, dy, dx), pair j of band b
 * turning by delta[b] * pow(base, -(2j)/(2 * band_pairs[b])); a band whose offset is zero turns
 * by cos 0 = 1, sin 0 = 0.  A position reset of the frame axis is (dt, 0, 0).  Otherwise the
 * same steps, results and arguments as kv_ring_delta_rotate (one new scale per head over all
 * valid slots, V untouched, same workspace).
 * Errors: those of kv_ring_delta_rotate; NULL delta; any |delta[b]| >= 2^31; band_pairs
 * negative or not summing to head_dim/2.
 */
int kv_ring_delta_rotate_3d(const kv_ring_desc *ring, int32_t ring_head, int32_t filled,
                            const int64_t *delta, const int32_t *band_pairs, double rope_base,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Attention of nq new queries over every valid slot of the ring (abstract: 757 new-token
 * queries against the 5,788-slot cache, 240 calls per chunk; cpdf.ai blog, "Blackwell...":
 * FP8 attention with per-head scales).
 *   q            device bfloat16 [nq][heads][head_dim], 16-byte aligned; query i at position
 *                q_pos0 + i (rotated, then quantised with one FP8 scale per head);
 *   softmax_scale  multiplies q.k, finite and > 0 (normally 1/sqrt(head_dim));
 *   out          device bfloat16 [nq][heads][head_dim], 8-byte aligned;
 *   lse          device float32 [heads][nq]: natural-log softmax denominator plus row max.
 * With filled == 0 the output is 0 and lse is -inf.  nq == 0 is a no-op.
 * The launch is a grid of at most one work-group per compute unit; work-groups sharing a query
 * row wait for one another to merge it, which every device running nothing else (and any on
 * which each XCD can hold the few consecutive work-groups of a row at once) lets finish.
 * Errors: NULL pointers, misalignment, nq < 0 or nq > KV_RING_MAX_TOKENS, ring_head/filled out
 * of range, softmax_scale not finite and positive, positions outside the table, workspace too
 * small.
 */
int ring_attention(const kv_ring_desc *ring, int32_t ring_head, int32_t filled, const void *q,
                   int32_t nq, int64_t q_pos0, const float *rope_table, int64_t rope_n_pos,
                   float softmax_scale, void *out, float *lse, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * One layer call of the method (abstract: in each of the 240 calls per chunk the new tokens
 * enter the cache and the new queries attend over it): exactly kv_ring_write(ring, k_new,
 * v_new, n, start_slot, pos0, ...) followed on the same stream by ring_attention(ring,
 * ring_head, filled, q, nq, q_pos0, ...), with ring_head and filled the ring's state after the
 * write.  Same results bit for bit; one launch fewer, because the queries' per-head absmax runs
 * in the same launch as the write's K and V absmax.
 *   workspace  kv_ring_workspace_bytes(KV_RING_OP_WRITE_ATTEND, heads, slots, head_dim,
 *              max(n, nq)) bytes, 16-byte aligned.
 * nq == 0 makes it the write alone (q, out, lse unused).
 * Errors: those of the two calls (all checked before anything is enqueued).
 */
int kv_ring_write_attend(const kv_ring_desc *ring, const void *k_new, const void *v_new, int32_t n,
                         int32_t start_slot, int64_t pos0, int32_t ring_head, int32_t filled,
                         const void *q, int32_t nq, int64_t q_pos0, const float *rope_table,
                         int64_t rope_n_pos, float softmax_scale, void *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The E4M3 encoder the kernels use, exposed so it can be checked exhaustively: out[i] =
 * e4m3(x[i]) with round to nearest even and saturation to +-448 (x finite).  x and out are
 * device pointers, 16-byte aligned; n >= 0.
 */
int kv_ring_fp8_encode(const float *x, uint8_t *out, int64_t n, void *stream);

/*
 * The read-time design that the ring replaces, kept as a baseline to measure against
 * (abstract: whole-cache work repeated in every attention call before it was moved to write
 * time; cpdf.ai blog, "Como rodar 57B...": the ring advances the window without copies).  That
 * design keeps the last `window` tokens as a linear bfloat16 cache and, in every call, copies it
 * forward by the n new tokens, then rotates and quantises the whole window again; with this
 * library the second part is kv_ring_write of all `window` tokens into a ring of `window`
 * slots at start_slot 0 (one per-head scale over the window), followed by ring_attention with
 * ring_head 0 and filled = window.
 *
 * kv_window_advance is the copy: dst rows 0 .. window-n-1 = src rows n .. window-1, then
 * dst rows window-n .. window-1 = fresh rows 0 .. n-1.
 *   src, dst, fresh  device memory, 16-byte aligned, rows of row_bytes bytes (for a cache of
 *                    [tokens][heads][head_dim] bfloat16, row_bytes = heads*head_dim*2);
 *                    src may be NULL when n == window, fresh when n == 0;
 *   0 <= n <= window, 1 <= window; 16 <= row_bytes <= 2^30, a multiple of 16.
 * dst must not overlap the rows read from src or fresh (callers alternate two buffers).
 * Errors: KV_RING_ERR_RANGE (window, n, or overlapping buffers), KV_RING_ERR_SHAPE (row_bytes),
 * KV_RING_ERR_NULL, KV_RING_ERR_ALIGN.
 */
int kv_window_advance(const void *src, void *dst, const void *fresh, int32_t window, int32_t n,
                      int64_t row_bytes, void *stream);

/*
 * Profiling aid.  When both handles are non-NULL, each later ring_attention call records
 * `before` (a hipEvent_t) on its stream immediately before launching its main attention kernel
 * and `after` immediately after it, so the caller can time that kernel alone with
 * hipEventElapsedTime.  Passing NULLs turns it off.  The setting is process-wide and not
 * synchronised: set it from the thread that issues the calls being timed.
 */
int kv_ring_set_attention_events(void *before, void *after);

/* Static description of a status code. */
const char *kv_ring_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVRING_H */
