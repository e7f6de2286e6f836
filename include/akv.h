/*
 * akv.h -- C ABI of libakv: the AKV state-restoration hot path on MI355X (gfx950).
 *
 * What it computes (pages about "Cache Engineering for Agents", arXiv 2610.28577v1):
 *   - the cache ops append / drop / repos and the operate-after request syntax
 *     (jaehun.me review "Cache Engineering for Agents", sections "three cache
 *     operations" (§3.3) and "AKV serving system" (§4, Fig. 6));
 *   - segment-batch attention: one restore prefill whose causal attention is cut
 *     at every drop/repos boundary; a dropped entry stays visible to the
 *     segments that used it and is hidden from later ones; with repos, per-segment
 *     KV versions are made by key rotation and value copy (same review, section
 *     "single-prefill restore with segment-batch attention", §4.2, App. A.1.1, Fig. 10);
 *   - repos: keys moved from position p to q by a RoPE rotation, values untouched
 *     (same review, section "what to keep, how to align positions", §3.3);
 *   - decode over the active cache only (same review, serving results, Fig. 12,
 *     App. A.4.1), at page size 1 (vibeprogramminglab explainer, section 4).
 *
 * Conventions for every entry point:
 *   - Return AKV_OK (0) or a negative AKV_E* status; akv_last_error() gives a
 *     thread-local message for the last failure on the calling thread.  No C++
 *     exception crosses this boundary.
 *   - Host pointers are read during the call only.  Device pointers are owned by
 *     the caller; the library never allocates device memory.  GPU entry points
 *     enqueue work on the caller's stream and return without synchronising; a
 *     launch error (hipGetLastError) is reported as AKV_EHIP.
 *   - Tensors are dense, row-major, token-major:
 *       Q / O     [tokens][Hq][d]
 *       K / V     [tokens or pool slots or version rows][Hkv][d]
 *     with element type given by `dtype` (AKV_BF16 or AKV_F32).  GQA maps query
 *     head h to kv head h / (Hq / Hkv).
 *   - RoPE: theta_i = base^(-2i/d), i < d/2; pair i is (x[i], x[i+d/2]) for
 *     AKV_ROPE_HALF or (x[2i], x[2i+1]) for AKV_ROPE_INTERLEAVED; moving a vector
 *     from position p to q rotates pair i by (q-p)*theta_i.  Angles are reduced
 *     in float64 from the exact integer position difference.
 */
#ifndef AKV_H
#define AKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define AKV_OK            0
#define AKV_EINVAL       -1   /* bad argument (null pointer, size, capacity) */
#define AKV_EOPSEQ       -2   /* invalid op sequence (drop of a future message, ...) */
#define AKV_EUNSUPPORTED -3   /* valid but not implemented (e.g. head dim != 64) */
#define AKV_EHIP         -4   /* HIP runtime / launch error */
#define AKV_ENOMEM       -5   /* host allocation failed */
#define AKV_ENOSPACE     -6   /* cache index: every slot asked for is locked */

/* Element types. */
#define AKV_F32  0
#define AKV_BF16 1

/* RoPE pair layouts. */
#define AKV_ROPE_HALF        0
#define AKV_ROPE_INTERLEAVED 1

/* Canonical cache ops. */
#define AKV_OP_APPEND 0   /* a = number of tokens appended (>= 0) */
#define AKV_OP_DROP   1   /* drop logical tokens [a, b) (already appended) */
#define AKV_OP_REPOS  2   /* renumber the active keys 0..r-1, next position r */

/* Tile classes in the plan's tile lists (tile entry = k_tile * 4 + class). */
#define AKV_TILE_PARTIAL 1
#define AKV_TILE_FULL    2

typedef struct { int32_t kind; int32_t reserved; int64_t a, b; } akv_op;

typedef struct akv_plan akv_plan;   /* opaque, host-owned, immutable once built */

typedef void* akv_stream_t;         /* a hipStream_t (NULL = the null stream) */

const char* akv_status_string(int status);
const char* akv_last_error(void);
const char* akv_version(void);

/* ---------------------------------------------------------------- A1: op compile (host)
 *
 * akv_ops_from_messages: the operate-after request -> canonical op list.
 *   msg_len[n_msgs]            tokens per message (message k is an implicit append);
 *   drop_after/drop_target[n_drop]   pairs "after message k, drop message j";
 *   repos_after[n_repos]       "after message k, repos".
 * Canonical form: for k = 0..n_msgs-1: APPEND(msg_len[k]); then one DROP per
 * distinct non-empty target of k in ascending message order (token range of the
 * target); then one REPOS if k is listed in repos_after.  Drop comes before repos
 * at the same boundary (review §4, Fig. 6; explainer section 4).
 * Errors: AKV_EOPSEQ if k or j is outside [0, n_msgs) or j > k; AKV_EINVAL for a
 * negative length, null arrays with non-zero counts, or ops_cap too small.
 * *n_ops_out always receives the number of ops required; ops_out may be NULL to
 * query it.
 */
int akv_ops_from_messages(int32_t n_msgs, const int32_t* msg_len,
                          int32_t n_drop, const int32_t* drop_after, const int32_t* drop_target,
                          int32_t n_repos, const int32_t* repos_after,
                          akv_op* ops_out, int64_t ops_cap, int64_t* n_ops_out);

/* akv_build_visibility: replay the ops and compile the restore plan (all host).
 * bq / bk: query / key tile sizes of the tile-class lists (the bf16 attention
 * kernels need bk == 64 and bq == 64 or, with hq / hkv in {1, 2, 4}, bq == 64 * 8 /
 * (hq / hkv); akv_attention_bq gives the one they run fastest with).
 * Tables (all int32, see akv_plan_tables):
 *   T1 tok_pos[T]    position of each token when appended;
 *   T2 tok_drop[T]   token index of the boundary at which it is dropped, or INT32_MAX;
 *                    query i sees key j  <=>  j <= i < tok_drop[j];
 *   T3 segments      (begin, end, stretch) per maximal run with no drop/repos inside;
 *   T4 stretches     (tok_begin, tok_end, r, ver_offset) per repos stretch that
 *                    appends tokens; r = keys active right after its repos;
 *   T5 versions      (src token, from_pos, to_pos) per version row, stretch by
 *                    stretch; to_pos = row index v in the stretch;
 *   T6 tiles         per work item (stretch, q-tile): ascending non-empty key tiles
 *                    with class FULL or PARTIAL; key tiles run over the version rows
 *                    from 0 and restart at the stretch's own tokens; a tile is FULL
 *                    only if it holds bk keys and every in-range query sees all;
 *   T7 final         active tokens ascending, their positions, p_next.
 * Errors: AKV_EOPSEQ (bad kind, negative append, drop range not yet appended),
 * AKV_EINVAL (bq/bk < 1, > 2^20, or more than 2^31-1 tokens), AKV_ENOMEM.
 */
int akv_build_visibility(const akv_op* ops, int64_t n_ops, int32_t bq, int32_t bk, akv_plan** out);

typedef struct {
  int64_t n_tokens, n_segments, n_epochs, n_versions;
  int64_t n_items, n_tiles, n_full, n_partial;
  int64_t visible_pairs;       /* exact number of (query, key) pairs attended */
  int64_t n_final, p_next;
  int32_t bq, bk;
  uint64_t device_bytes;       /* size of the device image for akv_plan_upload */
  int64_t n_runs;              /* runs of version rows that move by one shift (ver_run) */
} akv_plan_info;

typedef struct {
  const int32_t* tok_pos;      /* [n_tokens] */
  const int32_t* tok_drop;     /* [n_tokens] */
  const int32_t* segments;     /* [n_segments][3] */
  const int32_t* epochs;       /* [n_epochs][4] */
  const int32_t* versions;     /* [n_versions][3] */
  const int32_t* items;        /* [n_items][2] stretch, q-tile */
  const int32_t* tile_ptr;     /* [n_items + 1] */
  const int32_t* tiles;        /* [n_tiles] k_tile * 4 + class */
  const int32_t* item_order;   /* [n_items] launch order: stretches by descending tile count (ties by
                                  index), each stretch's items by descending tile count */
  const int32_t* final_tok;    /* [n_final] */
  const int32_t* final_pos;    /* [n_final] */
  const int32_t* ver_run;      /* [n_versions] run of each version row: a run is a maximal
                                  stretch of consecutive version rows of one repos stretch
                                  whose shift to_pos - from_pos is the same */
  const int32_t* run_delta;    /* [n_runs] that shift */
} akv_plan_tables;

int  akv_plan_info_get(const akv_plan* plan, akv_plan_info* info);
/* Read-only views into the plan (valid until akv_plan_destroy). */
int  akv_plan_tables_get(const akv_plan* plan, akv_plan_tables* views);
/* Copy the plan's device image (info.device_bytes) to caller memory `dev`,
 * asynchronously on `stream`; the plan must outlive the copy. */
int  akv_plan_upload(const akv_plan* plan, void* dev, uint64_t dev_bytes, akv_stream_t stream);
void akv_plan_destroy(akv_plan* plan);

/* ---------------------------------------------------------------- A2/A5: RoPE rotation
 *
 * akv_rope_repos: out[n] = R((pos_to[n] - pos_from[n]) theta) * in[gather ? gather[n] : n]
 * for n < n_rows; each row holds `heads` vectors of length d (d even, d <= 256,
 * d % 16 == 0).  pos_from may be NULL (all zero: "in" holds raw un-rotated vectors,
 * i.e. RoPE-apply); gather may be NULL.  pos_from / pos_to / gather are device
 * int32 arrays.  out must not overlap in unless gather is NULL and out == in.
 * This is the batched repos of the review (§3.3: rotation only, values untouched).
 */
int akv_rope_repos(void* out, const void* in, int dtype, int64_t n_rows, int32_t heads, int32_t d,
                   const int32_t* gather, const int32_t* pos_from, const int32_t* pos_to,
                   double rope_base, int rope_layout, akv_stream_t stream);

/* akv_kv_reuse: the reuse path of a cache hit ("Cache Engineering for Agents"
 * review, serving system: the extended radix tree with drop nodes, citing §4.2,
 * App. A.1.2, Fig. 8; and the request flow: a hit copies the matched KV instead of
 * re-prefilling).  A matched KV entry is copied into new rows, its key converted to
 * the position version the request needs by rotation and its value copied as is:
 *   k_out[n] = R((pos_to[n] - pos_from[n]) theta) * k_pool[gather[n]],
 *   v_out[n] = v_pool[gather[n]]                            (bit-exact copy)
 * for n < n_rows; rows hold `heads` vectors of length d (as akv_rope_repos).  A row
 * whose position is unchanged (pos_from[n] == pos_to[n]) is copied bit for bit.
 * gather, pos_from, pos_to: device int32 [n_rows], all required; gather values
 * index rows of k_pool / v_pool (not checked on the device).  Outputs must not
 * overlap the pools.  Caller-owned device memory; enqueued on `stream`.
 */
int akv_kv_reuse(void* k_out, void* v_out, const void* k_pool, const void* v_pool, int dtype, int64_t n_rows,
                 int32_t heads, int32_t d, const int32_t* gather, const int32_t* pos_from,
                 const int32_t* pos_to, double rope_base, int rope_layout, akv_stream_t stream);

/* akv_rope_apply: rotate raw Q or K rows [n_tokens][heads][d] to their append
 * positions (plan T1), out of place or in place.  dev_plan = the uploaded image. */
int akv_rope_apply(const akv_plan* plan, const void* dev_plan, void* out, const void* in,
                   int dtype, int32_t heads, int32_t d, double rope_base, int rope_layout,
                   akv_stream_t stream);

/* ---------------------------------------------------------------- A3: KV versions
 *
 * For every version row (T5): k_ver[row] = R((to_pos - from_pos) theta) * k[src],
 * v_ver[row] = v[src] (bit copy).  k must already be rotated to the append
 * positions (akv_rope_apply).  k_ver / v_ver: [n_versions][hkv][d].
 * Review §4.2 / App. A.1.1: temporary per-segment versions by key rotation and
 * value copy.
 */
int akv_build_kv_versions(const akv_plan* plan, const void* dev_plan, const void* k, const void* v,
                          void* k_ver, void* v_ver, int dtype, int32_t hkv, int32_t d,
                          double rope_base, int rope_layout, akv_stream_t stream);

/* ---------------------------------------------------------------- A4: segment attention
 *
 * out[i][h] = sum_key softmax(scale * <q[i][h], key>) value over the keys visible
 * to token i on its stretch's axis: the stretch's version rows (k_ver/v_ver) with
 * tok_drop[src] > i, then its own tokens j <= i with tok_drop[j] > i.
 * q, k: rotated to append positions; out [n_tokens][hq][d]; lse (nullable, float32
 * [n_tokens][hq]) receives the natural-log sum of exp(scale * score).
 * scale <= 0 means 1/sqrt(d).  bf16 needs d == 64, hq / hkv in {1, 2, 4, 8}, a plan
 * with bk == 64 and bq == 64 or (hq / hkv < 8) bq == 64 * 8 / (hq / hkv); f32 (a
 * vector-ALU path for small problems) needs d <= 128 and bq <= 256.  Errors:
 * AKV_EINVAL (NULL pointers, hq not a multiple of hkv, missing version buffers),
 * AKV_EUNSUPPORTED (other shapes or tile sizes), AKV_EHIP (launch failure).
 */
/* The plan query tile (bq for akv_build_visibility) with which the bf16 attention
 * runs fastest for hq query heads over hkv kv heads: 64 for 8 query heads per kv
 * head (one kv head per workgroup, eight waves of 64 query rows); 64 * 8 / (hq / hkv)
 * for 1, 2 or 4, whose eight waves then take the 8 / (hq / hkv) 64-token parts of a
 * query tile for each query head.  64 for any other shape.  Pure host function. */
int32_t akv_attention_bq(int32_t hq, int32_t hkv);

int akv_segment_attention(const akv_plan* plan, const void* dev_plan,
                          const void* q, const void* k, const void* v,
                          const void* k_ver, const void* v_ver, void* out, float* lse,
                          int dtype, int32_t hq, int32_t hkv, int32_t d, float scale,
                          akv_stream_t stream);

/* As akv_segment_attention, with the queries given raw (q_raw [n_tokens][hq][d],
 * unrotated, "at position 0"): the attention rotates each query to its append
 * position tok_pos (T1) as it loads it, in fp32 from the raw values, so no rotated
 * copy of Q is written and read back (review §3.3: a vector at position p is the
 * raw vector rotated pair by pair by p * theta_i).  k must still be rotated
 * (akv_rope_apply); k_ver / v_ver as above.  rope_base > 1 and finite; rope_layout
 * AKV_ROPE_HALF or AKV_ROPE_INTERLEAVED; d even and <= 128 (bf16: d == 64).
 * Errors as akv_segment_attention, plus AKV_EINVAL for a bad base or layout.
 */
int akv_segment_attention_rope(const akv_plan* plan, const void* dev_plan,
                               const void* q_raw, const void* k, const void* v,
                               const void* k_ver, const void* v_ver, void* out, float* lse,
                               int dtype, int32_t hq, int32_t hkv, int32_t d, float scale,
                               double rope_base, int rope_layout, akv_stream_t stream);

/* ---------------------------------------------------------------- A3 + A4 fused
 *
 * Segment attention that builds no version buffers: each version row's key and
 * value are copied from its source token into the attention's key tile, and the
 * key is rotated there.  Review "single-prefill restore with segment-batch
 * attention" (§4.2, App. A.1.1): the per-segment KV versions are temporary; key
 * rotation and value copy make them.  Version row v of a stretch is the key of
 * source token j = ver_src[v] moved from its append position tok_pos[j] to v, i.e.
 * rotated by the shift of its run (akv_plan_tables.ver_run / run_delta); every run's
 * (cos, sin) per frequency is evaluated once into the workspace, with the same
 * arithmetic as akv_build_kv_versions, so the output equals that of
 * akv_segment_attention_rope over akv_build_kv_versions buffers bit for bit.
 * q_raw: raw queries [T][hq][d] (rotated on load as in akv_segment_attention_rope);
 * k: keys rotated to their append positions (akv_rope_apply); v: values.
 * ws: caller device memory of at least akv_rot_table_bytes(plan, d) bytes (may be
 * NULL when that is 0), overwritten.  bf16 only, d == 64, hq == 8 * hkv with a plan
 * of bq == 64, or hq / hkv in {1, 2, 4} with bq == 64 * 8 / (hq / hkv) (as
 * akv_attention_bq gives), and k and v under 4 GiB each (T * hkv * d * 2 bytes <
 * 2^32, T = the plan's token count);
 * other shapes: AKV_EUNSUPPORTED, use the version-buffer path.  Other errors as
 * akv_segment_attention_rope, plus AKV_EINVAL for a short workspace.
 */
uint64_t akv_rot_table_bytes(const akv_plan* plan, int32_t d);
int akv_segment_attention_fused(const akv_plan* plan, const void* dev_plan, const void* q_raw,
                                const void* k, const void* v, void* out, float* lse, int dtype,
                                int32_t hq, int32_t hkv, int32_t d, float scale, double rope_base,
                                int rope_layout, void* ws, uint64_t ws_bytes, akv_stream_t stream);

/* ---------------------------------------------------------------- A6: decode
 *
 * One query token per request b < batch: out[b][h] = attention of q[b][h] over the
 * pool rows indices[indptr[b] .. indptr[b+1]) (its active cache plus its own new
 * slot, gathered at page size 1).  q [batch][hq][d], k_pool/v_pool [slots][hkv][d]:
 * bf16; indptr/indices: device int32, indptr nondecreasing from indptr[0] = 0
 * (indptr[batch] = total gathered keys).  out [batch][hq][d] bf16; lse [batch][hq]
 * float32 (natural log of the softmax denominator of the scaled scores), nullable.
 * max_n: host-side bound on every
 * request's key count, in [1, 2^31); it is checked but does not shape the launch,
 * which cuts all the batch's gathered keys into equal ranges, one per CU, and merges
 * each request's partials.  A request with zero keys (indptr[b+1] <= indptr[b])
 * has nothing to attend to: its output rows are written as bf16 NaN and its lse
 * entries as -inf, so the caller can detect it after the fact (the indices live on
 * the device and are not read by the host; callers that include the new token's
 * own slot never meet this).  ws: device workspace of at least
 * akv_decode_workspace_bytes(...) bytes (about (256 + batch) * hq * 264 bytes),
 * owned by the caller; its contents are scratch.  scale <= 0 means 1/sqrt(d).
 * d == 64.
 */
uint64_t akv_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int64_t max_n);
int akv_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* indptr, const int32_t* indices, int32_t batch,
                         int32_t hq, int32_t hkv, int32_t d, int64_t max_n, float scale,
                         int dtype, void* out, float* lse, void* ws, uint64_t ws_bytes,
                         akv_stream_t stream);

/* akv_decode_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, with the workspace taken from a fixed 16 MiB scratch
 * array the library holds on each device it runs on (found once per device on the
 * first call there, held until the process ends).  The call allocates nothing.
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents (the kernels need no cleared state): calls that overlap on one
 * device, on different streams or from different threads, race and must be
 * serialised by the caller.  Arguments and errors as akv_decode_attention without
 * ws / ws_bytes; AKV_EINVAL when the batch needs more than 16 MiB of scratch
 * (akv_decode_workspace_bytes(...) > 16 MiB, i.e. (256 + batch) * hq > 63,550 for
 * d == 64), AKV_EHIP when the scratch address cannot be found.
 */
int akv_decode_attention_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* indptr, const int32_t* indices, int32_t batch,
                                 int32_t hq, int32_t hkv, int32_t d, int64_t max_n, float scale,
                                 int dtype, void* out, float* lse, akv_stream_t stream);

/* ---------------------------------------------------------------------------
 * KV cache index: which rows of a request are already held, where, and at which
 * position; what has to be recomputed; which rows to give up under pressure.
 * "Cache Engineering for Agents" review, AKV serving system (§4.2, App. A.1.2,
 * Fig. 8) and the request flow (match in the extended radix tree, copy on a hit,
 * one segment-batch prefill when the state was evicted); explainer §3.4 / Fig. 5
 * (the same survivors reached by different op orders hold different KV).
 *
 * The index is host-only bookkeeping over the slots 0..n_slots-1 of a KV pool the
 * caller owns (one slot = one token's K and V rows at one position, for however
 * many layers and heads the caller stores there).  It never touches device memory.
 *
 * Sharing rule: a token's rows are identified by the canonical history up to and
 * including its append: the token ids, one drop node per op boundary holding the
 * logical ranges that boundary actually removed (drops of inactive tokens and empty
 * appends change nothing), and a repos node for every repos that moves a position
 * or the next position.  Requests share rows exactly where these histories agree.
 * A token may hold several position versions; each sits in its own slot and is
 * evicted on its own.  An evicted row leaves its tree node in place.
 *
 * Locks: every slot handed out (akv_cache_alloc, akv_cache_match with lock != 0)
 * carries one lock per hand-out; akv_cache_unlock drops them.  Locked slots are
 * never evicted; an allocated slot that never received a version goes back to the
 * free list when its last lock is dropped.
 *
 * Eviction order among unlocked rows: first those no finished request holds
 * ("dropped": not in the final state, at that position, of any completed request
 * whose history no later completed request extends), then the rest; least recently
 * used first within each class (one tick per call), then the lower slot.
 *
 * Not thread-safe: callers serialise calls on one index.  All arrays are host
 * memory owned by the caller.  Tokens: tok[0..n_tok) must be exactly the tokens
 * the op list appends (AKV_EINVAL otherwise); op errors as akv_build_visibility.
 * ------------------------------------------------------------------------- */
typedef struct akv_cache akv_cache;

typedef struct {
  int64_t n_tokens;      /* T */
  int64_t n_matched;     /* leading tokens whose history is in the tree */
  int64_t n_resident;    /* tokens with a resident version (slot_out >= 0) */
  int64_t restore_from;  /* s: recompute tokens [s, T); T means reuse only */
  int64_t n_final;       /* active tokens after the last op */
  int64_t p_next;        /* position of the next appended token */
} akv_cache_match_info;

typedef struct {
  int64_t n_slots, n_free, n_resident, n_locked;
  int64_t n_nodes;        /* tree nodes, root included */
  int64_t n_tree_tokens;  /* distinct token histories ever inserted */
  int64_t n_marks;        /* distinct completed histories */
  int64_t n_frontier;     /* of those, not extended by another */
} akv_cache_stats;

/* n_slots >= 1.  *out owned by the caller; free with akv_cache_destroy. */
int  akv_cache_create(int32_t n_slots, akv_cache** out);
void akv_cache_destroy(akv_cache* cache);

/* For every token i of the request: slot_out[i] = slot of its preferred resident
 * version (-1 if none) and pos_out[i] = that version's position.  Preferred: the
 * version at the position the request needs (final position for tokens of the
 * final state, else the append position), else the most recently used, then the
 * lowest position.  A version at another position is usable after rotating its key
 * by (needed - pos_out[i]) (akv_kv_reuse does the copy and the rotation).
 * restore_from is the largest s in [0, T] such that every key seen by a query at or
 * after s, and every final-state token below s, has a resident version.  Returned
 * slots are touched (LRU) and, if lock != 0, locked once each.  info may be NULL. */
int akv_cache_match(akv_cache* cache, const int32_t* tok, int64_t n_tok, const akv_op* ops,
                    int64_t n_ops, int32_t lock, int32_t* slot_out, int32_t* pos_out,
                    akv_cache_match_info* info);

/* n slots, each locked once: free slots in ascending order, then evicted rows in
 * eviction order.  AKV_ENOSPACE (nothing changes) if fewer than n are free or
 * evictable. */
int akv_cache_alloc(akv_cache* cache, int32_t n, int32_t* slots_out);

/* Record the request's history (creating tree nodes) and the versions it computed:
 * token ver_token[v] at position ver_pos[v] now sits in ver_slot[v], a slot from
 * akv_cache_alloc that holds no version yet; its lock is kept.  Also records the
 * request's final state as a completed request.  AKV_EINVAL (nothing changes) for an
 * index out of range, a slot that is not allocated and empty, a version given twice
 * or already resident. */
int akv_cache_insert(akv_cache* cache, const int32_t* tok, int64_t n_tok, const akv_op* ops,
                     int64_t n_ops, const int32_t* ver_token, const int32_t* ver_pos,
                     const int32_t* ver_slot, int64_t n_ver);

/* Drop one lock per listed slot (a slot may be listed as often as it is locked).
 * AKV_EINVAL (nothing changes) if a slot holds fewer locks than listed. */
int akv_cache_unlock(akv_cache* cache, const int32_t* slots, int64_t n);

int akv_cache_stats_get(const akv_cache* cache, akv_cache_stats* out);

#ifdef __cplusplus
}
#endif
#endif /* AKV_H */
