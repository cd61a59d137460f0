/*
 * kvevict.h -- C ABI of the MI355X (gfx950) KV-cache eviction hot path.
 *
 * Four calls make one eviction pass over a batch of (layer, sequence, KV
 * head) caches:
 *
 *   tri_score        score every cached key from the query centre
 *   tri_score_rotated  the same for keys stored after RoPE (dense or paged)
 *   tri_score_gqa    per-query-head scores of a GQA group, z-normalised, max over the group
 *   tri_score_gqa_rotated  the same for keys stored after RoPE (dense or paged)
 *   kv_select_topk   keep prompt + recent window + top-scoring keys per head
 *   kv_select_random keep prompt + recent window + uniformly random keys
 *   kv_compact       gather the kept K/V rows (and positions) contiguously
 *
 * and the policy variants the pages use as controls or alternatives:
 *
 *   kv_select_union          union of per-query-head top-k sets, ranked by a combined score
 *   kv_select_random_shared  one random keep-set shared by every head
 *   kv_select_recent         keep the prompt and the latest slots (no scores)
 *   kv_compact_inplace       fill evicted slots with the kept rows beyond the new length
 *
 * and a device-side check of any keep-set against the partition rules:
 *
 *   kv_audit_kept            count, per head, the entries of a kept list that break the rules
 *
 * and a measurement aid:
 *
 *   kv_stream_ceiling        tri_score's loads (and stores) without its arithmetic
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller, except
 *    where marked "host". The library allocates nothing, keeps no global
 *    state, and never synchronises the stream; every call only enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns. Calls are re-entrant given distinct workspaces.
 *  - Workspaces. tri_score, the selectors and tri_score_gqa take caller-owned
 *    device scratch memory (`workspace`, `workspace_bytes`) sized by the
 *    matching *_workspace_bytes query; a NULL, misaligned (8 bytes) or
 *    smaller workspace is rejected with KV_EWORKSPACE. Its first 256 bytes are
 *    a header: the first 4 are the device status word below, the rest is
 *    reserved. Contents beyond the header on entry do not matter and on return
 *    are unspecified. Calls that share a workspace must not overlap in time.
 *  - Device status word (first uint32 of a workspace). Preconditions on device
 *    data (valid lengths, prompt lengths, position order) cannot be checked on
 *    the host without a synchronisation. A build with device checks
 *    (kv_device_checks() == 1, libkvevict_debug.so) verifies them in an extra
 *    kernel before each call's own kernels and ORs KV_DEV_* bits into the word;
 *    the caller clears it. The release build never touches it. Either way the
 *    kernels clamp device values into the validated ranges, so memory safety
 *    never depends on them.
 *  - Cache layout is head-major: element (l, s, h, j, e) of a
 *    [n_layers, n_seq, n_kv_heads, t_cap, head_dim] tensor lives at
 *    ((((l*n_seq + s)*n_kv_heads + h)*t_cap + j)*head_dim + e). Per-slot
 *    arrays (positions, scores) are the same without the last axis.
 *  - Slot j of a head holds the token at position pos[j] (or j when the
 *    position pointer is NULL). Sequence s has seq_len[s] valid slots.
 *  - Alignment: K and V (and compaction outputs) 16 bytes; query centres
 *    8 bytes (tri_score_rotated: 4); every int32 / fp32 array 4 bytes.
 *    A misaligned pointer is rejected with KV_EINVAL.
 *  - Return value: KV_OK, or a negative kv_status for arguments rejected on
 *    the host (nothing is launched then) or a failed launch (KV_EHIP).
 *    Device-side data is never trusted for memory safety: lengths are
 *    clamped to the capacities the host validated, and out-of-range kept
 *    indices are skipped.
 *
 * Pages the operations follow (cited by title and section):
 *  [TA-sum]  "TriAttention: Efficient Long Reasoning with Trigonometric KV
 *            Compression" -- structured paper summary, section 3.4.
 *  [TA-blog] "TriAttention: Efficient Long Reasoning with Trigonometric KV
 *            Compression" -- blog walkthrough, scoring implementation and
 *            inference-time steps.
 *  [RA]      "Random Attention: Rethinking KV Cache Eviction for Efficient
 *            Reasoning" -- sections 2, 3 and Appendices D, F.
 */
#ifndef KVEVICT_H
#define KVEVICT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv_status {
  KV_OK = 0,
  KV_EINVAL = -1,   /* NULL or misaligned pointer, non-positive size, bad policy value, aliasing outputs */
  KV_EDTYPE = -2,   /* unknown element type */
  KV_ESHAPE = -3,   /* head_dim / capacity outside what the kernels support */
  KV_EWORKSPACE = -4, /* workspace NULL, not 8-byte aligned, or smaller than its query returns */
  KV_EHIP = -5      /* a kernel launch failed (hipGetLastError after the launch) */
} kv_status;

/* Bits of the device status word (debug build only; see "Device status word" above). */
#define KV_DEV_SEQ_LEN 0x1u    /* some seq_len[s] outside [0, t_cap]: clamped into it            */
#define KV_DEV_PROMPT_LEN 0x2u /* some prompt_len[s] outside [0, prompt_cap]: clamped (selectors) */
#define KV_DEV_POS_ORDER 0x4u  /* some head's positions not strictly ascending over its valid
                                  slots: slot order is then not time order, and ties break by
                                  slot, not by position (expected after kv_compact_inplace)      */
#define KV_WORKSPACE_HEADER 256 /* bytes of every workspace before any kernel scratch           */

typedef enum kv_dtype {
  KV_F32 = 0,
  KV_BF16 = 1
} kv_dtype;

/* A batch of per-(layer, sequence, KV head) caches. head_dim and dtype are
 * read by tri_score and kv_compact only; the selectors ignore them. */
typedef struct kv_shape {
  int32_t n_layers;        /* >= 1, < 65536                                   */
  int32_t n_seq;           /* >= 1                                             */
  int32_t n_kv_heads;      /* >= 1, < 65536                                   */
  int32_t head_dim;        /* even; bf16: multiple of 8, fp32: multiple of 4;
                              at most 256                                       */
  int32_t t_cap;           /* slots per head (slot stride), >= 1              */
  int32_t dtype;           /* kv_dtype of K and V                              */
  const int32_t *seq_len;  /* device [n_seq]: valid slots T_s; values outside
                              [0, t_cap] are clamped into it                     */
} kv_shape;

/* Eviction policy: a budget of entries per KV head with pinned prompt and
 * recent window. [TA-sum] 3.4 "KV Cache Pruning Procedure" (compress when
 * the cache exceeds B, keep the top B); [RA] section 2 (a recent buffer that
 * is never scored; top-K of the candidates, Eq. 2) and section 3 rule 1
 * (the prompt is never evicted); [TA-blog] (prefill kept by default). */
typedef struct kv_policy {
  int32_t budget;              /* B >= 1: entries kept per head, counting prompt
                                  and recent window                               */
  int32_t recent;              /* R >= 0: latest slots always kept (clipped so
                                  that prompt + window <= B)                      */
  int32_t prompt_cap;          /* host upper bound on every prompt_len[s] (>= 0);
                                  larger device values are clamped to it          */
  const int32_t *prompt_len;   /* device [n_seq]: prompt slots P_s (slots 0..P_s-1) */
} kv_policy;

/*
 * Per-sequence partition used by both selectors (T = seq_len[s] clamped to
 * t_cap, P = prompt_len[s] clamped to [0, min(prompt_cap, T)]):
 *   T <= B : nothing is compressed; kept = 0..T-1, n_kept = T.
 *   T >  B : R' = min(R, max(0, B-P), T-P); evictable range E = [P, T-R');
 *            n_sel = max(0, B-P-R') slots of E are selected;
 *            kept = [0,P) u selected u [T-R', T) in ascending slot order;
 *            n_kept = max(B, P)  (a prompt longer than B is kept whole and
 *            nothing else is).
 * Kept sets are written in ascending (chronological) order, [RA] Appendix F.
 */

/* Library version, (major << 16) | minor: 2.1 (2.1 added kv_stream_ceiling). */
int32_t kv_version(void);

/* Static string for a kv_status value. */
const char *kv_status_string(int32_t status);

/* 1 when this library build checks device-side preconditions into the workspace status word
 * (libkvevict_debug.so), 0 for the release build. */
int32_t kv_device_checks(void);

/*
 * tri_score -- importance of every cached key from the query centre.
 *
 * For each (l, s, h) and slot j < T_s:
 *   scores[l,s,h,j] = (1/|D|) * sum_{delta in D}
 *                     < RoPE(qbar[l,h], t_cur[s] + delta), RoPE(K[l,s,h,j], p_j) >
 * with RoPE in complex form over interleaved pairs (x[2f] + i x[2f+1]
 * rotated by omega_f * p, omega_f = rope_theta^(-2f/head_dim)) and <.,.> the
 * real dot product: the trigonometric-series term of [TA-sum] 3.4
 * ("TriAttention Key Importance Scoring: The Trigonometric Series Term")
 * with the query replaced by its centre, averaged over the future offsets D
 * ("Handling Multiple Future Positions"). No 1/sqrt(d) factor.
 * The offset average is folded into one complex coefficient per band by
 * angle addition ([TA-sum] 3.4, the a_f/b_f expansion), so each key is read
 * once. Scores are fp32 (error within 1e-4 of max(|score|, head RMS)).
 * With qabs given, the distance-free norm-based term of [TA-sum] 3.4 ("The
 * Norm-Based Term", "Adaptive Weighting via Q/K Concentration") is added:
 *   + sum_f (1 - R_f) * qabs_f * |k_f|,  R_f = |qbar_f| / qabs_f
 * (a band with qabs_f = 0 contributes nothing).
 *
 *  K        device [L,S,H,t_cap,d] of shape->dtype; pre-RoPE keys.
 *  pos      device [L,S,H,t_cap] int32 absolute positions, or NULL (p_j = j).
 *  qbar     device [L,H,d] fp32 query centre per (layer, KV head).
 *  qabs     device [L,H,d/2] fp32 mean query magnitude E|q_f| per band, or
 *           NULL for the trigonometric term alone.
 *  t_cur    device [S] int32 current position of each sequence.
 *  rope_theta  RoPE base (> 0).
 *  deltas   HOST [n_delta] int32 future offsets D, 1 <= n_delta <= 64.
 *  scores   device [L,S,H,t_cap] fp32 output; slots j >= T_s are not written.
 *  workspace  device, at least kv_score_workspace_bytes(shape, n_delta) bytes (the header:
 *           the score stream itself needs no scratch).
 * One head's rows must span less than 2 GiB (t_cap * head_dim * elem < 2^31 - 2^15).
 * Device checks (debug build): KV_DEV_SEQ_LEN, and KV_DEV_POS_ORDER when pos is given.
 */
kv_status tri_score(const kv_shape *shape, const void *K, const int32_t *pos,
                    const float *qbar, const float *qabs, const int32_t *t_cur, double rope_theta,
                    const int32_t *deltas, int32_t n_delta, float *scores,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes tri_score needs (0 for sizes it rejects: a shape outside its limits, or n_delta
 * outside 1..64). shape->seq_len is not read and may be NULL. */
size_t kv_score_workspace_bytes(const kv_shape *shape, int32_t n_delta);

/* RoPE pairing of the stored coordinates: band f is (x[2f], x[2f+1]) or (x[f], x[f+d/2]). */
typedef enum kv_rope_style {
  KV_ROPE_INTERLEAVED = 0,
  KV_ROPE_HALF = 1
} kv_rope_style;

/* A paged key pool: per layer, n_blocks blocks of block_size tokens. Token-major pools
 * (head_major = 0) keep all KV heads of a token together: the row of (layer l, physical block pb,
 * token o in the block, KV head h) starts at element
 * ((((l*n_blocks + pb)*block_size + o)*n_kv_heads + h)*head_dim). Head-major pools
 * (head_major = 1) keep each head's block contiguous: ((((l*n_blocks + pb)*n_kv_heads + h)
 * *block_size + o)*head_dim). Slot j of sequence s lives in physical block
 * block_table[s*blocks_per_seq + j/block_size], token j % block_size.
 * Block ids outside [0, n_blocks) are clamped into it (memory safety, not a result). */
typedef struct kv_paged {
  const int32_t *block_table;  /* device [n_seq][blocks_per_seq] */
  int32_t blocks_per_seq;      /* >= 1; blocks_per_seq * block_size >= t_cap */
  int32_t block_size;          /* a power of two */
  int32_t n_blocks;            /* physical blocks per layer in the pool */
  int32_t head_major;          /* 0: [L, n_blocks, block_size, H, d]; 1: [L, n_blocks, H, block_size, d] */
} kv_paged;

/*
 * tri_score_rotated -- tri_score for keys stored after RoPE, dense or paged.
 *
 * Same score as tri_score with K replaced by its rotated form: a serving
 * engine keeps k_rot = RoPE(k, p) ([TA-blog] scoring implementation), and
 *   scores[l,s,h,j] = (1/|D|) sum_{delta in D} < RoPE(qbar[l,h], t_cur[s]+delta), k_rot[j] >
 * (+ the norm-based term when qabs is given; |k_rot_f| = |k_f|). No key
 * position is needed. qbar and the keys use the pairing rope_style; with
 * KV_ROPE_HALF the two halves of a row must each fill whole 16-byte pieces
 * (bf16: head_dim a power of two >= 16; fp32: >= 8).
 *
 *  K        dense device [L,S,H,t_cap,d] (paged == NULL) or the paged pool.
 *  paged    NULL, or the host descriptor of a device block table.
 *  other arguments as for tri_score; scores are dense [L,S,H,t_cap].
 */
kv_status tri_score_rotated(const kv_shape *shape, const void *K, const kv_paged *paged,
                            int32_t rope_style, const float *qbar, const float *qabs,
                            const int32_t *t_cur, double rope_theta, const int32_t *deltas,
                            int32_t n_delta, float *scores, void *stream);

/*
 * tri_score_gqa -- the grouped-query rule of [TA-sum] 3.4 ("KV Cache Pruning
 * Procedure", GQA handling): the `group` query heads that share a KV head
 * each score the keys with their own centre (the tri_score score, with the
 * norm-based term when qabs is given), each query head's scores are
 * normalised to zero mean and unit standard deviation over the head's T_s
 * cached keys, and the final score is the maximum over the group:
 *   head_scores[l,s,h,g,j] = tri_score with qbar[l,h,g] (and qabs[l,h,g])
 *   scores[l,s,h,j] = max_g (head_scores[l,s,h,g,j] - mu_g) / sigma_g
 * mu_g and sigma_g are the mean and population standard deviation over the
 * T_s slots, accumulated in fp64 in a fixed order (the result does not
 * depend on scheduling); a query head whose scores do not vary (sigma_g = 0,
 * or T_s = 1) contributes 0. The normalised value is computed in fp64 from
 * the fp32 head scores and rounded to fp32.
 *
 *  group        G, 1 <= G <= 16 query heads per KV head; G * t_cap < 2^29.
 *  head_dim     at most 256 (bf16) or 128 (fp32).
 *  qbar         device [L,H,G,d] fp32 per-query-head centres.
 *  qabs         device [L,H,G,d/2] fp32 or NULL.
 *  head_scores  device [L,S,H,G,t_cap] fp32 output (per-query-head scores).
 *  scores       device [L,S,H,t_cap] fp32 output.
 *  workspace    device, at least kv_score_gqa_workspace_bytes(shape, group)
 *               bytes (the header, then the per-chunk partial sums).
 *  other arguments as for tri_score; slots j >= T_s are not written.
 */
kv_status tri_score_gqa(const kv_shape *shape, const void *K, const int32_t *pos, int32_t group,
                        const float *qbar, const float *qabs, const int32_t *t_cur,
                        double rope_theta, const int32_t *deltas, int32_t n_delta,
                        float *head_scores, float *scores, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Bytes of workspace tri_score_gqa needs for this shape and group (0 for sizes or a group it
 * rejects). shape->seq_len is not read and may be NULL. tri_score_gqa_rotated needs the same.
 * Device checks (debug build): KV_DEV_SEQ_LEN, and KV_DEV_POS_ORDER when pos is given. */
size_t kv_score_gqa_workspace_bytes(const kv_shape *shape, int32_t group);

/*
 * tri_score_gqa_noalloc -- tri_score_gqa for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument. Its partial sums live in a device array of kv_score_gqa_noalloc_max_bytes() bytes
 * (8 MiB, the header included) that the library keeps on every device it runs on until the
 * process ends; the first call on a device takes that array's address (hipGetSymbolAddress) and
 * no call allocates. A shape and group whose kv_score_gqa_workspace_bytes exceeds the array are
 * rejected with KV_EWORKSPACE (KV_EHIP if the address cannot be taken). Every call on one device
 * shares that device's array: calls that overlap in time on one device race and give unspecified
 * scores -- serialise them (one stream, or events). The array keeps the last call's partial sums;
 * nothing in it needs clearing. Other arguments and the results as for tri_score_gqa.
 */
kv_status tri_score_gqa_noalloc(const kv_shape *shape, const void *K, const int32_t *pos, int32_t group,
                                const float *qbar, const float *qabs, const int32_t *t_cur,
                                double rope_theta, const int32_t *deltas, int32_t n_delta,
                                float *head_scores, float *scores, void *stream);

/* Bytes of the device array behind tri_score_gqa_noalloc (the largest workspace it can stand in for). */
size_t kv_score_gqa_noalloc_max_bytes(void);

/*
 * tri_score_gqa_rotated -- the grouped-query rule (as tri_score_gqa) for keys
 * stored after RoPE, dense or through a paged block table, as a serving
 * engine keeps them ([TA-blog] implementation excerpt: the scorer works on
 * the rotated keys). Query head g's score of key j is tri_score_rotated's
 * score with qbar[l,h,g] (and qabs[l,h,g]); normalisation and the maximum as
 * for tri_score_gqa.
 *
 *  K, paged, rope_style  as for tri_score_rotated; qbar and qabs are in the
 *               same pairing as the stored keys.
 *  group        G, 1 <= G <= 8.
 *  head_dim     at most 128 (bf16) or 64 (fp32): one 16-byte piece per lane,
 *               at most 16 lanes per key.
 *  qbar, qabs, head_scores, scores, workspace  as for tri_score_gqa.
 */
kv_status tri_score_gqa_rotated(const kv_shape *shape, const void *K, const kv_paged *paged,
                                int32_t rope_style, int32_t group, const float *qbar,
                                const float *qabs, const int32_t *t_cur, double rope_theta,
                                const int32_t *deltas, int32_t n_delta, float *head_scores,
                                float *scores, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * kv_select_topk -- exact per-head top-n_sel of the evictable range.
 *
 * Ranking is (score descending, slot ascending); NaN ranks as -inf and
 * -0.0 equals +0.0. [TA-sum] 3.4 "Retention and eviction"; [RA] Eq. 2.
 *
 *  scores   device [L,S,H,t_cap] fp32 (slots j < T_s are read).
 *  kept     device [L,S,H,b_cap] int32 output: the n_kept kept slots in
 *           ascending order, then -1 up to b_cap.
 *  b_cap    must be >= max(budget, prompt_cap).
 *  n_kept   device [S] int32 output: |kept| of sequence s (same for every
 *           layer and head).
 *  workspace  device, at least kv_select_workspace_bytes(shape, b_cap) bytes.
 * Requires t_cap <= 2^26. Up to 32768 slots a head's keys stay in registers;
 * longer caches (context lengths reach 128K tokens, [TA-sum] 3.4 "Handling
 * Multiple Future Positions", on the offset range) run a kernel that
 * re-reads the scores at every step.
 * Device checks (debug build): KV_DEV_SEQ_LEN, KV_DEV_PROMPT_LEN.
 */
kv_status kv_select_topk(const kv_shape *shape, const kv_policy *policy,
                         const float *scores, int32_t *kept, int32_t b_cap,
                         int32_t *n_kept, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Workspace bytes kv_select_topk, kv_select_random and kv_select_random_shared need for this
 * shape and b_cap (0 for sizes they reject). shape->seq_len is not read and may be NULL.
 * It is the header alone, except for batches of at most 64 (layer, seq, KV head) heads with
 * 8192 < t_cap <= 32768: there the random draw is spread over several workgroups per head, which
 * hand their lists over in the workspace (8 bytes per slot and head, plus a count per 2048 slots).
 * The contents need no initialisation and are not meaningful after the call. */
size_t kv_select_workspace_bytes(const kv_shape *shape, int32_t b_cap);

/*
 * kv_select_random -- Random Attention's per-head uniform eviction.
 *
 * Every evictable slot j gets u_j = word (p_j & 3) of Philox4x32-10 (Salmon
 * et al., SC'11) with counter (p_j >> 2, (l << 16) | h, s, event) and key
 * (seed & 0xffffffff, seed >> 32) -- one block gives the draws of four
 * consecutive positions -- an i.i.d. uniform drawn independently
 * per KV head at every eviction; prompt and recent window are pinned; the
 * n_sel largest u_j are kept (ties to the lower slot). [RA] section 3,
 * Eq. 3 and Algorithm 1. No scores or keys are read.
 *
 *  pos      device [L,S,H,t_cap] int32 positions for the counter, or NULL (p_j = j).
 *  seed     64-bit key; event: eviction counter (fresh draws per event).
 *  layer_base  model index of the call's first layer: layer l of the call draws as layer
 *           layer_base + l (an engine that evicts layer by layer, or a pass split into layer
 *           chunks, gets the same draws as one call over all layers); 0 <= layer_base and
 *           layer_base + n_layers <= 65536.
 *  kept, b_cap, n_kept, workspace as for kv_select_topk (t_cap <= 2^26). From
 *  16385 slots on, with a budget of at most half of t_cap, the draws are not held
 *  in registers but drawn once per sweep (recomputed at every step when a sweep is
 *  repeated), so the call's workgroups can share CUs with a concurrent kernel such
 *  as the compaction of another layer chunk; with the split draw above, the chunk
 *  workgroups draw instead.
 * Device checks (debug build): KV_DEV_SEQ_LEN, KV_DEV_PROMPT_LEN, and
 * KV_DEV_POS_ORDER when pos is given.
 */
kv_status kv_select_random(const kv_shape *shape, const kv_policy *policy,
                           const int32_t *pos, uint64_t seed, uint32_t event, int32_t layer_base,
                           int32_t *kept, int32_t b_cap, int32_t *n_kept,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_audit_kept -- device-side audit of kept lists (for instance a caller's own selection, or a
 * selection after the cache was edited). For each (l, s, h), bad[l,s,h] is the number of
 * entries that break the partition rules above: an index r < n_kept whose slot lies outside
 * [0, T_s) or does not exceed kept[r-1]; r < P whose slot is not r (prompt); one of the last R'
 * entries that is not the matching slot of the recent window; r >= n_kept (below b_cap) that is
 * not -1; plus 1 when n_kept[s] differs from the partition's n_kept. 0 means a valid keep-set.
 * Memory safety never depends on the kept values.
 *
 *  kept, b_cap, n_kept as written by the selectors (device).
 *  bad     device [L,S,H] int32 output.
 */
kv_status kv_audit_kept(const kv_shape *shape, const kv_policy *policy, const int32_t *kept,
                        int32_t b_cap, const int32_t *n_kept, int32_t *bad, void *stream);

/*
 * kv_stream_ceiling -- a measurement aid, not part of the method: the memory system's ceiling for
 * tri_score's access pattern (bf16 keys of head_dim 128). It reads `bytes` of `buf` once as
 * tri_score does -- workgroups of 256 threads over 128 KB each, every wave two batches of sixteen
 * 16-byte pieces per lane, the second issued before the first is combined, non-temporal loads --
 * and combines each lane's pieces by XOR instead of scoring them. Timed beside tri_score over the
 * same bytes it separates the cost of the access pattern from that of the arithmetic.
 *
 *  buf     device, 16-byte aligned; bytes a positive multiple of 131072 (below 2^48).
 *  out     device uint32 words:
 *          with_stores != 0 (tri_score's score stream, non-temporal): bytes / 256 words; word
 *            (w * 128 + b * 64 + lane) is the XOR of the 64 32-bit words of lane `lane`'s 16 pieces
 *            of batch b (0, 1) of wave w, waves numbered in address order (32 KB each), a lane's
 *            pieces being the 16 bytes at lane * 16 + t * 1024 (t < 16) of its batch's 16 KB;
 *          with_stores == 0: bytes / 32768 words, word w the XOR over wave w's lanes and batches.
 * Errors: KV_EINVAL for NULL or misaligned pointers or a size that is not a whole number of 128 KB;
 * KV_ESHAPE from 2^48 bytes on.
 */
kv_status kv_stream_ceiling(const void *buf, size_t bytes, uint32_t *out, int32_t with_stores, void *stream);

/*
 * kv_select_union -- union-based selection ([TA-blog] eviction step) over the
 * `group` query heads of each KV head. Within the evictable range:
 *   1. every query head g takes its own top-k slots by head_scores[.., g, ..]
 *      (k = k_per_head, or ceil(n_sel / group) when k_per_head <= 0);
 *   2. the union U of those sets is formed;
 *   3. if |U| >= n_sel, the n_sel slots of U ranked first by `scores` (the
 *      combined score) are kept;
 *   4. otherwise all of U is kept and the rest of the evictable range tops it
 *      up in `scores` order.
 * Every ranking is (score descending, slot ascending) with NaN as -inf, as
 * for kv_select_topk; prompt and recent window are pinned as there.
 * tri_score_gqa writes both inputs: its per-query-head scores and, as the
 * combined score, the maximum over the group of the normalised scores.
 *
 *  head_scores  device [L,S,H,group,t_cap] fp32.
 *  scores       device [L,S,H,t_cap] fp32 combined score.
 *  group        1 <= group <= 64.
 *  kept, b_cap, n_kept as for kv_select_topk. Requires t_cap <= 2^18; past
 *  32768 slots the kernel re-reads the scores at every pass and holds the
 *  union as a bit per slot in LDS (t_cap / 8 bytes).
 */
kv_status kv_select_union(const kv_shape *shape, const kv_policy *policy, int32_t group,
                          int32_t k_per_head, const float *head_scores, const float *scores,
                          int32_t *kept, int32_t b_cap, int32_t *n_kept, void *stream);

/*
 * kv_select_random_shared -- the shared-draw control of [RA] sections 5.2-5.3:
 * one random keep-set that every (layer, KV head) of a sequence uses. It is
 * kv_select_random with the counter's second word fixed to 0, i.e. every head
 * draws what layer 0 / KV head 0 draws. Heads whose position arrays agree keep
 * the same slots. Arguments (workspace included) as for kv_select_random.
 */
kv_status kv_select_random_shared(const kv_shape *shape, const kv_policy *policy,
                                  const int32_t *pos, uint64_t seed, uint32_t event,
                                  int32_t *kept, int32_t b_cap, int32_t *n_kept,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_select_recent -- recency+prompt ([RA] section 4.1, the StreamingLLM-style
 * diagnostic): keep the prompt and fill the rest of the budget with the
 * contiguous latest slots. With the partition above, kept = [0, P) followed by
 * [T - (n_kept - P), T) (the evictable range's n_sel latest slots joined to the
 * recent window); slot order is taken as time order. No scores are read.
 * kept, b_cap, n_kept as for kv_select_topk (no t_cap limit beyond it).
 */
kv_status kv_select_recent(const kv_shape *shape, const kv_policy *policy,
                           int32_t *kept, int32_t b_cap, int32_t *n_kept, void *stream);

/*
 * kv_compact_inplace -- in-place hole filling: the engine compaction of [RA]
 * Appendix F without the copy of the whole cache. With n = n_kept[s] and kept
 * ascending (as the selectors write it), the kept rows below n stay where they
 * are and the i-th kept row at or beyond n (in slot order) moves into the i-th
 * evicted slot below n. Afterwards slots 0..n-1 of every head hold exactly the
 * kept rows, in an order that is no longer chronological; pos (if given) moves
 * with the rows, so later scoring and random draws use the true positions.
 * Slots >= n are left as they were. With a recent window of R slots, slot
 * order keeps naming the latest R tokens only while at least R tokens are
 * appended between evictions.
 *
 *  K, V     device [L,S,H,t_cap,d] (shape->dtype), updated in place.
 *  pos      device [L,S,H,t_cap] int32 updated in place, or NULL.
 *  kept     device [L,S,H,b_cap] int32, ascending (kept indices that do not
 *           ascend give unspecified rows, never an out-of-range access).
 *  n_kept   device [S] int32.
 */
kv_status kv_compact_inplace(const kv_shape *shape, void *K, void *V, int32_t *pos,
                             const int32_t *kept, int32_t b_cap, const int32_t *n_kept,
                             void *stream);

/*
 * kv_compact -- gather kept rows into a contiguous per-head layout.
 *
 * For r < min(n_kept[s], b_cap, out_cap):
 *   K_out[l,s,h,r,:] = K_in[l,s,h,kept[r],:], V_out likewise (bit copies),
 *   pos_out[l,s,h,r] = pos_in ? pos_in[l,s,h,kept[r]] : kept[r].
 * Rows r >= n_kept, and rows whose kept index lies outside [0, t_cap), are
 * not written. [RA] Appendix F (chronological keep-sets, gather
 * compaction); [TA-blog] (slice K/V by the kept indices).
 * Out-of-place only: K_out/V_out must not overlap K_in/V_in.
 *
 *  K_in, V_in  device [L,S,H,t_cap,d] (shape->dtype).
 *  pos_in      device [L,S,H,t_cap] int32 or NULL.
 *  kept        device [L,S,H,b_cap] int32 (from a selector).
 *  n_kept      device [S] int32.
 *  K_out, V_out device [L,S,H,out_cap,d]; pos_out device [L,S,H,out_cap] or NULL.
 */
kv_status kv_compact(const kv_shape *shape, const void *K_in, const void *V_in,
                     const int32_t *pos_in, const int32_t *kept, int32_t b_cap,
                     const int32_t *n_kept, void *K_out, void *V_out,
                     int32_t *pos_out, int32_t out_cap, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVEVICT_H */
