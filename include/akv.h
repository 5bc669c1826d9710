/*
 * akv.h -- C ABI of libakv.so: the data-parallel hot path of agent cache
 * engineering (drop / reposition of a paged bf16 KV cache, and decode
 * attention over the active KV) for AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [CE]  review of "Cache Engineering for Agents" (euisuk-chung.github.io,
 *         2026-10-29): sec. 3.3 eq. (3) append, eq. (4) drop, eq. (5)
 *         reposition; sec. 3.4 eq. (6) the state is fixed by the op history;
 *         Appendix A.1.1 / Figure 10 position walk-through.
 *   [AKV] "[Repo Review] AKV" (euisuk-chung.github.io, 2026-10-23): sec. 1
 *         drop runs before reposition at one boundary; sec. 3 / 5.3 a plan
 *         that is invalid is rejected as a whole; sec. 5.3 the layout keeps
 *         positions, a keep mask, next_position and old/new position
 *         transition arrays; sec. 5.5 the reposition kernel (un-rotate at p,
 *         rotate to q, copy when p == q, V copied, separate destination slot).
 *
 * Conventions
 *   - All tensors are DEVICE memory owned by the caller (the library never
 *     allocates device memory).  bf16 values travel as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is stream-ordered and asynchronous; the library never
 *     synchronises except inside akv_sync_status / akv_profile_read.
 *   - Page size is fixed at 16 tokens.  Pool layout (bf16, row-major):
 *         k_pool, v_pool : [n_layers][n_blocks][n_kv_heads][16][head_dim]
 *     so one (layer, page, kv head) chunk is 16*head_dim contiguous values.
 *   - Per-page metadata: positions, token_ids : int32 [n_blocks][16].
 *   - Per-sequence metadata: block_table int32 [n_seqs][max_blocks_per_seq]
 *     (-1 = unused), seq_lens int32 [n_seqs] (active entries), next_pos
 *     int32 [n_seqs].  Free pages: free_stack int32 [n_blocks] and
 *     free_count int32 [1]; pages are handed out from the top of the stack
 *     (free_stack[free_count-1] first).
 *   - Per-token argument arrays (masks, positions) have one row per sequence
 *     with row stride S = max_blocks_per_seq * 16 entries; entry i of row b
 *     refers to the i-th active entry of sequence b and entries at or beyond
 *     that sequence's length are ignored.
 *   - Errors: arguments the host can check are rejected with an error code
 *     before anything is enqueued (cache unchanged).  Checks that need device
 *     data (a decreasing new position, an old position that does not match,
 *     too few free pages, a page table overflow) are made on the device
 *     before any write; the whole operation then becomes a no-op, the first
 *     such error is latched in the device error word, and every later
 *     mutating call on the cache is a no-op until akv_sync_status() reads
 *     and clears it.  This mirrors whole-request rejection in [AKV] sec. 3
 *     and 5.3.
 *   - Free pages: a drop / reposition rebuilds survivors from the first
 *     dropped page on in fresh pages before their old pages return to the
 *     stack.  When the free pool cannot hold the fresh pages of every
 *     sequence at once, the op runs in groups of consecutive sequences, one
 *     group after another in stream order, each group's old pages freed
 *     before the next group takes fresh ones (the result is the same).  The
 *     host never reads device state, so it enqueues the rounds up front:
 *     one when the page table cannot address more than half the pool
 *     (2 * n_seqs * max_blocks_per_seq <= n_blocks: every op fits), else
 *     min(n_seqs, AKV_MAX_OP_GROUPS) (environment, read by akv_cache_init;
 *     default 8), rounds past the groups an op needs exiting at once.
 *     AKV_ERR_NO_BLOCKS comes only when one sequence alone does not fit the
 *     pages free at its turn or the op needs more groups than that.
 *   - Concurrent calls on one cache from different streams race; callers
 *     serialise them on one stream.
 *   - Environment (read by akv_cache_init): AKV_MOVE_ONESHOT_CAP=<n> caps
 *     the one-shot grid of the drop / reposition / fork move at n blocks,
 *     one per page and layer group; ops needing more use the persistent
 *     grid (0 = always persistent).  Both grids give bit-identical results.
 */
#ifndef AKV_H
#define AKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AKV_OK = 0,
  AKV_ERR_ARG = 1,          /* null pointer, bad shape, out-of-range value */
  AKV_ERR_ORDER = 2,        /* new positions negative or not strictly increasing */
  AKV_ERR_POS_MISMATCH = 3, /* old_pos differs from the stored positions */
  AKV_ERR_NO_BLOCKS = 4,    /* free pool too small for the new pages */
  AKV_ERR_CAPACITY = 5,     /* a sequence would exceed max_blocks_per_seq */
  AKV_ERR_HIP = 6,          /* a HIP runtime call failed */
  AKV_ERR_SCRATCH = 7       /* the call needs more than the library's static scratch */
} akv_status;

/* Bytes of the static decode workspace each GPU holds for
 * akv_decode_attention_noalloc (8 MiB). */
#define AKV_NOALLOC_SCRATCH_BYTES (8u << 20)

typedef struct akv_cache akv_cache; /* opaque host-side handle */

typedef struct {
  int32_t n_layers;           /* L  >= 1 */
  int32_t n_kv_heads;         /* Hkv >= 1 */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t block_size;         /* must be 16 */
  int32_t n_blocks;           /* NB pages in the pool, >= 1 */
  int32_t n_seqs;             /* B sequences, 1 .. 65535 */
  int32_t max_blocks_per_seq; /* page-table row length, >= 1 */
  double rope_base;           /* >= 1; theta_i = rope_base^(-2i/r), NeoX half split over the r rotary dims */
  uint16_t *k_pool;           /* bf16 [L][NB][Hkv][16][d] */
  uint16_t *v_pool;           /* bf16 [L][NB][Hkv][16][d] */
  int32_t *block_table;       /* [B][max_blocks_per_seq] */
  int32_t *seq_lens;          /* [B] */
  int32_t *next_pos;          /* [B] */
  int32_t *positions;         /* [NB][16] */
  int32_t *token_ids;         /* [NB][16] */
  int32_t *free_stack;        /* [NB] */
  int32_t *free_count;        /* [1] */
  void *scratch;              /* device, >= akv_scratch_bytes(desc) bytes, 256-B aligned */
  size_t scratch_bytes;
  /* RoPE variants and sliding windows ([AKV] sec. 5.5: the model binding
   * tells partial RoPE and sliding-window layers apart; the rest of K that
   * RoPE does not rotate is copied like V).  Zero / NULL = full RoPE over d
   * with rope_base frequencies and full attention in every layer. */
  int32_t rotary_dim;         /* r: 0 = head_dim, else a multiple of 16 in [16, d]; pairs
                                 (i, i + r/2) are rotated, dims [r, d) are copied */
  const double *inv_freq;     /* HOST [r/2] frequencies theta_i (e.g. a Llama 3.1 or YaRN
                                 table), in [0, 1]; NULL = rope_base^(-2i/r); copied */
  const int32_t *layer_window;/* HOST [L] sliding-window length per layer, >= 0, 0 = full
                                 attention; NULL = all full; copied.  A query at position P
                                 reads the entries whose position is >= P - W + 1 */
} akv_cache_desc;

/* Device scratch the cache needs: the compaction plan (per-survivor gather
 * map and old -> new position transitions, [AKV] sec. 5.3), the error word,
 * the RoPE frequencies.  Owned by the caller, lives as long as the cache. */
size_t akv_scratch_bytes(const akv_cache_desc *desc);

/* Validate `desc`, upload the rotation frequencies theta_i of R(p) ([CE]
 * sec. 3.3 eq. 5; [AKV] sec. 5.5 for partial RoPE and windows), computed on
 * the host in double, into the scratch and return a host handle in *out.
 * Does not touch the pools or metadata; call akv_cache_reset before first
 * use.  Errors: AKV_ERR_ARG, AKV_ERR_HIP. */
akv_status akv_cache_init(const akv_cache_desc *desc, akv_cache **out);
/* Frees the host handle only (library housekeeping; the device memory stays
 * the caller's).  NULL is a no-op. */
void akv_cache_free(akv_cache *c);

/* A resident page pool with nothing active ([CE] sec. 3.1: resident,
 * active and logical KV are separate).
 * Empty every sequence: seq_lens = next_pos = 0, block_table = -1,
 * free_count = NB, and the free stack such that pages are handed out in the
 * order page_order[0], page_order[1], ... (page_order: HOST int32 [NB], a
 * permutation of 0..NB-1; NULL = 0, 1, 2, ...).  Clears the error word.
 * With page_order the call synchronises `stream` and copies the order to the
 * device before the reset kernel (set-up only; every other call except
 * akv_sync_status / akv_profile_read is asynchronous).
 * Errors: AKV_ERR_ARG (not a permutation), AKV_ERR_HIP. */
akv_status akv_cache_reset(akv_cache *c, const int32_t *page_order, void *stream);

/* [CE] eq. (3): append counts[b] new entries to each sequence b.
 *   counts    : DEVICE int32 [B], >= 0
 *   n_new     : host copy of sum(counts) (sizes the launch)
 *   k_new     : DEVICE bf16 [L][n_new][Hkv][d], keys already rotated at
 *               their positions (the model computed them), tokens ordered by
 *               sequence then by append order
 *   v_new     : DEVICE bf16 [L][n_new][Hkv][d]
 *   token_ids : DEVICE int32 [n_new]
 * Entry j of sequence b lands at slot len_b + j with position
 * next_pos_b + j; then len_b and next_pos_b advance by counts[b].
 * Device-detected: AKV_ERR_NO_BLOCKS, AKV_ERR_CAPACITY (whole call no-op). */
akv_status akv_append(akv_cache *c, const int32_t *counts, int64_t n_new,
                      const uint16_t *k_new, const uint16_t *v_new,
                      const int32_t *token_ids, void *stream);

/* akv_append with the model's RoPE step fused in ([CE] eq. 3: the new keys
 * are rotated at the positions they take): k_raw holds the keys before RoPE,
 * same layout as k_new; entry j of sequence b is stored as
 * bf16(R(next_pos_b + j) k_raw) -- fp64 angle (next_pos_b + j) * theta_i and
 * fp64 rotation of each pair (i, i + r/2), rounded once to nearest even; the
 * non-rotary tail (partial RoPE) and V are copied.  Errors as akv_append. */
akv_status akv_append_rope(akv_cache *c, const int32_t *counts, int64_t n_new,
                           const uint16_t *k_raw, const uint16_t *v_new,
                           const int32_t *token_ids, void *stream);

/* End of a request ([CE] sec. 3.1: the request's resident KV is released):
 * every sequence b with release[b] != 0 gives up all its pages (a page
 * shared with a position version that survives stays with it; the others
 * return to the free stack) and
 * pages to the device free stack and becomes empty with next_pos = 0, ready
 * for a new request (or as the destination of akv_fork).  release: DEVICE
 * uint8 [B].  A no-op while a device error is latched. */
akv_status akv_release(akv_cache *c, const uint8_t *release, void *stream);

/* [CE] eq. (4): drop the active entries whose mask byte is non-zero.
 *   drop_mask : DEVICE uint8 [B][S]
 * Survivors keep their order, K, V, position and token id; seq_lens shrink;
 * next_pos is unchanged.  Survivors from the first dropped entry's page on
 * are moved into fresh pages (out of place); pages before it are untouched;
 * the old pages return to the free stack.  Needs up to ceil(len/16) free
 * pages per sequence while it runs; the op is split into sequence groups
 * when the pool is short (see Free pages above; AKV_ERR_NO_BLOCKS only when
 * a sequence alone does not fit).  The gather map of the call (pre-call
 * index of each survivor) is exported by akv_query_state. */
akv_status akv_drop(akv_cache *c, const uint8_t *drop_mask, void *stream);

/* [CE] eq. (5): move every active entry from its position p to q.
 *   old_pos : DEVICE int32 [B][S] or NULL.  If given it must equal the
 *             stored positions (the transition's source, [AKV] sec. 5.3);
 *             otherwise AKV_ERR_POS_MISMATCH and the call is a no-op.
 *   new_pos : DEVICE int32 [B][S] or NULL (= canonical 0..len-1).  Must be
 *             >= 0 and strictly increasing per sequence (AKV_ERR_ORDER).
 * K' = R(q - p) K with pair i = (k[i], k[i+d/2]) turned by (q - p)*theta_i,
 * computed in fp64 from bf16 and rounded once to bf16 (nearest, ties even);
 * entries with q == p are left bit-identical; V is not touched.  In place.
 * next_pos = last q + 1 (0 for an empty sequence). */
akv_status akv_reposition(akv_cache *c, const int32_t *old_pos,
                          const int32_t *new_pos, void *stream);

/* Drop then reposition at one boundary ([AKV] sec. 1), fused into one
 * compaction pass: survivors are moved and re-rotated in the same kernel.
 *   drop_mask : DEVICE uint8 [B][S]
 *   new_pos   : DEVICE int32 [B][S] indexed by SURVIVOR rank j, or NULL
 *               (= canonical 0..r-1, the next append then goes to r).
 * Result is bit-identical to akv_drop followed by akv_reposition. */
akv_status akv_drop_reposition(akv_cache *c, const uint8_t *drop_mask,
                               const int32_t *new_pos, void *stream);

/* New position versions ([CE] sec. 4.2.3, Appendix A.1.1; [AKV] sec. 5.4:
 * an existing version is reused, borrowed or allocated and copied): for
 * every source sequence b with dst_of[b] >= 0, the empty sequence dst_of[b]
 * becomes a copy of b's active entries with drop_mask applied (optional)
 * and, if reposition != 0, its positions moved to new_pos (NULL = canonical
 * 0..r-1).  The source sequence is not modified (copy on transform).
 * Pages: the version shares the source's leading full pages whose entries
 * it leaves as they are (before the first dropped entry and the first
 * changed position): those pages gain one reference each; the remaining
 * survivors are written to fresh pages (K re-rotated, V and token ids
 * copied).  A page returns to the free stack when its last holder drops or
 * releases it; a reposition never turns a page another sequence holds in
 * place, it rebuilds the sequence in fresh pages from the first changed page
 * on (copy on write), so it may need free pages.
 *   dst_of    : HOST int32 [B]; -1 = no fork.  Host-checked: destinations
 *               in range, distinct, not equal to their source, and not
 *               themselves sources.  Read during the call only (the map is
 *               passed to the device in kernel arguments), so the array may
 *               be freed or reused as soon as the call returns.
 *   drop_mask : DEVICE uint8 [B][S] (row b applies to source b) or NULL
 *   new_pos   : DEVICE int32 [B][S] by survivor rank of source b, or NULL;
 *               only with reposition != 0
 * next_pos of the copy: the source's (no reposition) or last new position
 * + 1.  Device-checked: a destination that is not empty (AKV_ERR_ARG),
 * new positions (AKV_ERR_ORDER), free pages (AKV_ERR_NO_BLOCKS: a fork
 * frees nothing, so it is never split into groups). */
akv_status akv_fork(akv_cache *c, const int32_t *dst_of, const uint8_t *drop_mask,
                    int reposition, const int32_t *new_pos, void *stream);

/* Decode attention over the active KV ([CE] sec. 3.1 and 3.3: after a drop
 * only the surviving, active entries are read; Appendix A.4.1: this is the
 * full-attention time AKV cuts) for layers [layer_begin, layer_begin +
 * n_layers):
 *   q          : DEVICE bf16 [B][n_layers][n_q_heads][d], already rotated at
 *                the query's position by the caller
 *   active_len : DEVICE int32 [B] or NULL (= seq_lens).  Values outside
 *                [0, seq_len] are clamped and AKV_ERR_ARG is latched.
 *   out        : DEVICE bf16 [B][n_layers][n_q_heads][d]
 *   workspace  : DEVICE, >= akv_decode_workspace_bytes(...) bytes
 * o = softmax(q K^T / sqrt(d)) V over the first active_len entries; query
 * head h reads kv head h / (n_q_heads / n_kv_heads); no entry beyond
 * active_len and no self token; an empty sequence gives zeros.
 * Host-checked: n_q_heads multiple of n_kv_heads with ratio <= 16, layer
 * range inside [0, L), and each launch within 2^32 work-items (splits x
 * n_kv_heads x B x n_layers workgroups of 512, B x n_layers x n_q_heads
 * combine rows of d), else AKV_ERR_ARG.
 * akv_decode_workspace_bytes: bytes of `workspace` a call with these sizes
 * needs (its split-K partials; 256 when it runs unsplit), 0 for bad sizes. */
size_t akv_decode_workspace_bytes(const akv_cache *c, int32_t n_layers,
                                  int32_t n_q_heads);
akv_status akv_decode_attention(akv_cache *c, const uint16_t *q,
                                const int32_t *active_len, int32_t layer_begin,
                                int32_t n_layers, int32_t n_q_heads,
                                uint16_t *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/* akv_decode_attention for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as akv_decode_attention
 * (bit-identical output), without the workspace: the split-K partials go to
 * a fixed array of AKV_NOALLOC_SCRATCH_BYTES in the library's code object,
 * one per GPU, held until the process ends (its address is looked up once
 * per device by akv_cache_init).  The call allocates nothing and never
 * synchronises.  Every split record is written before it is read, so the
 * array needs no clearing; it keeps the last call's contents.
 * All calls on one GPU share that GPU's array: two calls whose work overlaps
 * in time on one GPU (other streams, other caches, other threads) race and
 * give wrong results; serialise them on one stream.
 * Errors: as akv_decode_attention, plus AKV_ERR_SCRATCH (host-checked, before
 * any launch) when akv_decode_workspace_bytes(c, n_layers, n_q_heads) exceeds
 * AKV_NOALLOC_SCRATCH_BYTES. */
akv_status akv_decode_attention_noalloc(akv_cache *c, const uint16_t *q,
                                        const int32_t *active_len, int32_t layer_begin,
                                        int32_t n_layers, int32_t n_q_heads, uint16_t *out,
                                        void *stream);

/* Segment-batch attention ([CE] Appendix A.1.1, Figure 10; Section 4.2.2):
 * the queries of a restore forward, split at drop / reposition boundaries
 * into segments, each attending causally over its own sequence of the cache
 * (the original or a position version made by akv_fork), all segments in
 * one launch, for layers [layer_begin, layer_begin + n_layers).
 *   q         : DEVICE bf16 [n_q][n_layers][n_q_heads][d], rotated at each
 *               query token's own position by the caller; segment s owns
 *               rows [seg_q_off[s], seg_q_off[s+1])
 *   seg_seq   : DEVICE int32 [n_segments], the sequence segment s reads
 *   seg_q_off : DEVICE int32 [n_segments + 1], non-decreasing, from 0
 *   max_q     : HOST, >= every segment's row count n_s (sets the grid)
 *   out       : DEVICE bf16, same layout as q; q and out 16-byte aligned
 * The last n_s entries of sequence seg_seq[s] are the segment's own tokens
 * (already appended): row i of the segment attends to entries
 * [0, len - n_s + i] of that sequence.  Several segments may read one
 * sequence.  Host-checked: n_q_heads multiple of n_kv_heads with ratio
 * <= 16, layer range, 1 <= max_q.  Device-checked (AKV_ERR_ARG latched):
 * n_s > max_q or n_s < 0 (rows of that segment left unwritten), sequence
 * out of range or shorter than n_s (rows of that segment set to zero). */
akv_status akv_segment_attention(akv_cache *c, const uint16_t *q, const int32_t *seg_seq,
                                 const int32_t *seg_q_off, int32_t n_segments, int32_t max_q,
                                 int32_t layer_begin, int32_t n_layers, int32_t n_q_heads,
                                 uint16_t *out, void *stream);

/* Export of the state the server keeps per sequence ([AKV] sec. 5.3: the
 * positions of the active tokens, the next position and the transition of
 * the last plan; [CE] sec. 3.1: active index, RoPE position and token are
 * separate): one gather kernel on `stream`, outputs in active order.
 *   seq_lens  : DEVICE int32 [B] or NULL
 *   next_pos  : DEVICE int32 [B] or NULL
 *   positions : DEVICE int32 [B][S] or NULL; entry j of sequence b at
 *               [b][j], -1 past its length
 *   token_ids : DEVICE int32 [B][S] or NULL; same layout
 *   last_src  : DEVICE int32 [B][S] or NULL: the gather map of the last
 *               akv_drop / akv_reposition / akv_drop_reposition / akv_fork
 *               ([CE] eq. 4: the survivors in order): last_src[b][j] = the
 *               index, before that call, of the entry it placed at slot j of
 *               sequence b (for a fork destination, an index into its
 *               source); -1 past the call's output length of b, for rows the
 *               call did not write (fork sources and sequences not forked),
 *               before any such call, and after a rejected one.  Appends and
 *               releases leave it as it was.
 * All outputs are caller-owned; copy them to the host after the stream
 * (the call does not synchronise).  Reads only; works while an error is
 * latched.  Errors: AKV_ERR_ARG (null cache), AKV_ERR_HIP. */
akv_status akv_query_state(akv_cache *c, int32_t *seq_lens, int32_t *next_pos,
                           int32_t *positions, int32_t *token_ids, int32_t *last_src,
                           void *stream);

/* Synchronise `stream`, return the latched device error (AKV_OK if none)
 * and clear it (the error of a rejected request, [AKV] sec. 3 / 5.3). */
akv_status akv_sync_status(akv_cache *c, void *stream);
/* Static text naming a status code (library housekeeping). */
const char *akv_status_string(akv_status s);

/* Optional per-kernel timing with HIP events recorded on the launch stream
 * (measurement housekeeping, no operation of the pages).  Kernel ids: */
enum {
  AKV_KERNEL_PLAN = 0,     /* keep-scan / compaction plan */
  AKV_KERNEL_MOVE = 1,     /* fused move + re-rotation */
  AKV_KERNEL_COMMIT = 2,   /* page table / free stack commit */
  AKV_KERNEL_ATTN = 3,     /* split-K decode attention */
  AKV_KERNEL_COMBINE = 4,  /* split-K merge */
  AKV_KERNEL_APPEND = 5,   /* append plan + copy */
  AKV_KERNEL_SEGMENT = 6,  /* segment-batch attention */
  AKV_KERNEL_RELEASE = 7,  /* page release */
  AKV_KERNEL_ROUNDS = 8,   /* later (move, commit) rounds of an op split into sequence groups */
  AKV_KERNEL_COUNT = 9
};
akv_status akv_profile_enable(akv_cache *c, int on);
/* Synchronises the recorded events; *total_ms and *launches accumulate
 * since the last reset.  reset != 0 clears the accumulators afterwards. */
akv_status akv_profile_read(akv_cache *c, int kernel, double *total_ms,
                            int64_t *launches, int reset);

#ifdef __cplusplus
}
#endif
#endif /* AKV_H */
