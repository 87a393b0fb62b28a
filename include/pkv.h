/*
 * pkv.h -- C ABI of libpkv: a copy-on-write paged KV cache for
 * tree-structured decoding (beam search, MCTS, speculative draft trees,
 * agents sharing a prompt) on AMD MI355X (gfx950).
 *
 * Sources for the semantics (the pages describe the mechanism, not an API):
 *   [D1] Dendrite author's reply, "How is this different from vLLM's paged
 *        attention?": KV memory paged in fixed blocks; forking a beam or MCTS
 *        node is a shallow copy of the block table through copy-on-write,
 *        not a copy of the cache.
 *   [D2] Dendrite author's reply, "Why Rust?": a block that is being written
 *        must never be aliased.
 *   [F4] Ferrite project page, section 04 "DFlash2 verify trees and copy
 *        rows": drafted tokens are verified as best-first trees in one pass
 *        of the model; section 06: speculation never changes the text.
 *   [F7] Ferrite project page, section 07 "Prompt cache for agents":
 *        conversations snapshotted at turn boundaries resume from the
 *        longest match; a parked conversation keeps its blocks.
 *
 * Conventions (every call):
 *   - Return value: PKV_OK (0) or a negative PKV_E_* code. On error a
 *     message is available from pkv_last_error() (thread-local) and -- for
 *     every host-side call -- the pool is left exactly as it was.
 *   - No C++ exception crosses this interface.
 *   - Ownership: the caller owns every device buffer (the K/V arenas, q,
 *     out, new K/V, the attention workspace) and the stream. The library
 *     owns its host metadata, a pinned host staging ring and a small device
 *     buffer for per-call metadata (block lists, slots, copy ops), all freed
 *     by pkv_pool_destroy.
 *   - Device work is enqueued on the given stream (NULL = the null stream)
 *     and is asynchronous: kernel faults surface at the caller's next
 *     synchronisation. Use one stream per pool: a block freed on the host
 *     may be handed out again by the next append, and only stream order
 *     keeps earlier kernels from seeing the reuse.
 *   - A pool is not thread-safe; serialise calls on it.
 *
 * Device memory layout (element type = kv_dtype):
 *   K arena: [num_layers][num_blocks][num_kv_heads][block_size][head_dim]
 *   V arena: [num_layers][num_blocks][num_kv_heads][head_dim][block_size]
 *   One (layer, block, kv-head) tile is contiguous in both. V tiles are
 *   stored transposed (token index fastest) because the token index is the
 *   contracted index of P.V: the attention kernels then read V straight into
 *   matrix-core operand registers with 16-byte loads. A slot id is
 *   block * block_size + offset.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_E_INVALID (-1)     /* bad or stale handle, bad shape, double free */
#define PKV_E_OOM (-2)         /* the pool has too few free blocks */
#define PKV_E_HIP (-3)         /* a HIP runtime call failed */
#define PKV_E_UNSUPPORTED (-4) /* dtype / head_dim / block_size not built */
#define PKV_E_WORKSPACE (-5)   /* the attention workspace is too small */

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

typedef struct pkv_pool pkv_pool; /* opaque */

/* A sequence handle. A freed handle's generation no longer matches, so a
 * stale handle is rejected with PKV_E_INVALID. */
typedef struct {
  int32_t index;
  uint32_t generation;
} pkv_seq;

/* One copy-on-write copy: slots [0, n_valid) of every layer and KV head of
 * block src are copied into block dst. */
typedef struct {
  int32_t src;
  int32_t dst;
  int32_t n_valid;
} pkv_cow_op;

typedef struct {
  int32_t num_blocks;   /* blocks in the pool, > 0 */
  int32_t block_size;   /* token slots per block: 16, 32 or 64 for attention */
  int32_t num_layers;   /* layers held by the arenas, > 0 */
  int32_t num_kv_heads; /* KV heads, > 0 */
  int32_t num_q_heads;  /* query heads, a multiple of num_kv_heads */
  int32_t head_dim;     /* 64, 128 or 256 for attention */
  int32_t kv_dtype;     /* pkv_dtype; q uses the same type */
  /* Optional host array (copied at create): a permutation of
   * [0, num_blocks). Allocation hands out the free block that comes first
   * in this order. NULL = lowest free id first. */
  const int32_t* alloc_order;
  /* Device arenas, laid out as above. May be NULL for a pool used only for
   * host-side table work; device calls then fail with PKV_E_INVALID. */
  void* k_arena;
  void* v_arena;
} pkv_pool_desc;

typedef struct {
  int32_t num_blocks;
  int32_t free_blocks;
  int32_t live_seqs;
  int32_t reserved;
  int64_t total_refs; /* sum of all block reference counts */
  /* Block ids and chunk references copied into private table parts since
   * the pool was created: a fork copies none; the first change to a shared
   * table copies its list of chunks and at most one chunk of 64 ids. */
  int64_t table_ids_copied;
} pkv_stats;

/* ---------------------------------------------------------------- pool */

/* Create a pool of fixed-size blocks [D1]; all blocks start free. */
int pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out);
/* Free the host metadata, staging and metadata buffers; waits for the
 * library's own pending copies. The arenas stay the caller's. */
int pkv_pool_destroy(pkv_pool* pool);

/* Raw block verbs. alloc: take one free block (count 1) per the allocation
 * order. release: drop one reference; the block is free again at 0.
 * Releasing a free block is PKV_E_INVALID. */
int pkv_block_alloc(pkv_pool* pool, int32_t* id);
int pkv_block_release(pkv_pool* pool, int32_t id);

/* ------------------------------------------------------------ sequences */

/* A new, empty sequence. */
int pkv_seq_create(pkv_pool* pool, pkv_seq* out);
/* Fork [D1]: the child's table equals the parent's and every listed block
 * gains one reference, as seen by pkv_block_refcount. The parent is
 * unchanged and no K/V is copied. O(1): tables are persistent (a list of
 * refcounted chunks of 64 block ids), so the fork shares the parent's list
 * and bumps one count; the first change to a shared list or chunk copies
 * that part only (at most the list and one chunk per append). */
int pkv_seq_fork(pkv_pool* pool, pkv_seq parent, pkv_seq* child);
/* Drop one reference from each block of the sequence (blocks reaching 0
 * become free) and invalidate the handle. */
int pkv_seq_free(pkv_pool* pool, pkv_seq seq);

/* n forks in one call: children[i] = fork of parents[i] (host arrays).
 * All or nothing: on error no child exists. */
int pkv_seq_fork_many(pkv_pool* pool, const pkv_seq* parents, int32_t n, pkv_seq* children);
/* n frees in one call (host array); all handles are checked first, and a
 * handle listed twice is PKV_E_INVALID; on error nothing is freed. */
int pkv_seq_free_many(pkv_pool* pool, const pkv_seq* seqs, int32_t n);

/* Plan an append of n >= 0 tokens to seq [D1, D2], all or nothing:
 *  1. if the last block is partly filled and shared (count > 1), take a
 *     fresh block, record the copy {last, fresh, len % block_size}, drop one
 *     reference from the old block and point the table at the fresh one;
 *  2. for each new token, open a fresh block when the position is a
 *     multiple of block_size; the token's slot is
 *     table[pos / block_size] * block_size + pos % block_size.
 * The table and length are updated; no device work is done. slots_out
 * (host, n entries) receives the slots in token order; cow_out (host, room
 * for 1) the copy if one was taken, with *n_cow set to 0 or 1. n == 0
 * changes nothing. On PKV_E_OOM nothing changes. Never writes a block whose
 * count is above one. */
int pkv_seq_append_plan(pkv_pool* pool, pkv_seq seq, int32_t n, int64_t* slots_out,
                        pkv_cow_op* cow_out, int32_t* n_cow);

/* Device: perform copy-on-write copies [D1, D2] (host array of n ops) for
 * every layer and KV head, K and V, on the stream: the shared, partly
 * filled block is duplicated so that the appending branch writes a block
 * no other table points to. Slots at and above n_valid of
 * each destination block hold unspecified values afterwards. block_size
 * must be 16, 32 or 64 for every device call (else PKV_E_UNSUPPORTED). */
int pkv_cow_copy(pkv_pool* pool, const pkv_cow_op* ops, int32_t n, void* stream);

/* Device: scatter n tokens of new K/V into their slots [D1, D2] (slots from
 * an append plan: every one lies in a block whose count is one, so no other
 * table sees the write). slots: host array of n slot ids
 * (block * block_size + offset, each in range). k_new, v_new:
 * device, [num_layers][n][num_kv_heads][head_dim] in kv_dtype. */
int pkv_write_kv(pkv_pool* pool, const int64_t* slots, int32_t n, const void* k_new,
                 const void* v_new, void* stream);

/* Plan + copy-on-write + write for several sequences in one go: sequence
 * seqs[i] appends counts[i] tokens (each sequence at most once per call).
 * Equivalent to calling pkv_seq_append_plan for seqs[0], seqs[1], ... in
 * order and then copying and writing; all or nothing on PKV_E_OOM. k_new,
 * v_new: device [num_layers][sum(counts)][num_kv_heads][head_dim], the
 * sequences' tokens concatenated in seqs order. */
int pkv_append_kv_batch(pkv_pool* pool, const pkv_seq* seqs, const int32_t* counts,
                        int32_t n_seqs, const void* k_new, const void* v_new, void* stream);
/* One sequence: pkv_append_kv_batch with n_seqs = 1. */
int pkv_seq_append_kv(pkv_pool* pool, pkv_seq seq, int32_t n, const void* k_new,
                      const void* v_new, void* stream);

/* ----------------------------------------------------------- inspection */

int pkv_seq_info(const pkv_pool* pool, pkv_seq seq, int32_t* len, int32_t* n_blocks);
/* Copy up to cap block ids of the sequence's table into out (host). */
int pkv_seq_blocks(const pkv_pool* pool, pkv_seq seq, int32_t* out, int32_t cap);
/* References on a block: the live sequences whose table holds it, the
 * prompt-cache entries that hold it and pkv_block_alloc references. Computed
 * from the tables on each call (linear in the pool's table entries). */
int pkv_block_refcount(const pkv_pool* pool, int32_t id, int32_t* count);
/* The same for blocks 0 .. n-1 in one pass (host array, n <= num_blocks). */
int pkv_block_refcounts(const pkv_pool* pool, int32_t* counts, int32_t n);
int pkv_pool_stats(const pkv_pool* pool, pkv_stats* stats);
/* Bytes of device memory one arena (K or V) must have for this desc. */
int pkv_arena_bytes(const pkv_pool_desc* desc, size_t* bytes);

/* ------------------------------------------------------------ attention */

/* Shape of an attention plan, for inspection and accounting. */
typedef struct {
  int32_t n_segments;     /* runs of blocks with one holder set */
  int32_t n_chunks;       /* segments cut for the grid */
  int32_t n_items;        /* work items per (layer, KV head) */
  int32_t partial_rows;   /* partial states per (layer, KV head) */
  int64_t unique_tokens;  /* distinct token slots read per (layer, KV head) */
  int64_t workspace_bytes;
  int64_t plan_bytes;     /* the plan's arrays: carried in the kernel launches'
                             arguments when at most 12,288 bytes (option
                             "inline_plan"), else copied into the workspace */
  int64_t wide_tokens;    /* of unique_tokens, those in chunks served by the
                             wide-row launch (the rest: the narrow launch) */
  int64_t read_tokens;    /* token slots the work items read per (layer, KV
                             head): each item's chunk, in whole blocks; above
                             unique_tokens when short shared segments are read
                             once per branch or per group (option "fold_tokens",
                             "group_rows"); the tree launch reads unique_tokens */
  int32_t grouped_items;  /* work items that serve a group of branches
                             (option "group_rows") */
  int32_t reserved;
} pkv_plan_info;

/* Plans decode attention for these sequences (as pkv_decode_workspace_size
 * does) and describes the plan. Host only. */
int pkv_decode_plan_info(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs, int32_t n_layers,
                         pkv_plan_info* info);

/* Workspace bytes pkv_decode_attn needs for these sequences and n_layers.
 * The schedule built here is cached and reused by a following attention
 * call on the same sequences if no table has changed in between. */
int pkv_decode_workspace_size(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs,
                              int32_t n_layers, size_t* bytes);

/* Decode attention [D1]: for layer l in [layer0, layer0 + n_layers), each
 * sequence b and query head h,
 *   out[l - layer0][b][h][:] = softmax(scale * K_b q^T) V_b
 * over all tokens sequence b holds, with K_b, V_b the tokens of KV head
 * h / (num_q_heads / num_kv_heads) of layer l. Blocks that several of the
 * sequences share are read from HBM once per call and used for all of
 * them. q: device [n_layers][n_seqs][num_q_heads][head_dim] in kv_dtype;
 * out: device float32, same shape. ws: device workspace of ws_bytes >=
 * pkv_decode_workspace_size(...) bytes (256-byte aligned); it receives the
 * plan (unless the plan travels in the launch arguments, option
 * "inline_plan") and the partial states, so it must not be reused before the
 * launches on `stream` end. Every sequence must be non-empty (else
 * PKV_E_INVALID). */
int pkv_decode_attn(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs, int32_t layer0,
                    int32_t n_layers, const void* q, float* out, float scale, void* ws,
                    size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * pkv_decode_attn with the workspace taken from a static device array of
 * the library instead of a caller's buffer. Same arguments, semantics and
 * outputs as pkv_decode_attn (bit-identical: same plan, same kernels),
 * minus ws / ws_bytes. It calls no hipMalloc, hipFree, host-pinned
 * allocation or other allocating device routine: a plan too large for the
 * launch arguments is written into the array by small copy kernels whose
 * arguments carry it; the "concurrent" option's second stream and the
 * "timing" events are not used. The array holds PKV_NOALLOC_WORKSPACE_BYTES
 * (128 MiB, enough for a 32-layer decode of 64 MCTS leaves) per GPU, from the library's load until the process ends; its
 * address is looked up on the first call on each device (the device
 * current at the call; the arenas, q, out and stream must belong to it). A
 * call needing more than that (pkv_decode_workspace_size) fails with
 * PKV_E_WORKSPACE before any device work. All calls on one GPU share the
 * array: calls whose launches overlap in time (other streams, other pools,
 * other threads) race on it; calls on one stream follow each other safely.
 * Nothing in the array has to start at zero. */
#define PKV_NOALLOC_WORKSPACE_BYTES (128u << 20)
int pkv_decode_attn_noalloc(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs, int32_t layer0,
                            int32_t n_layers, const void* q, float* out, float scale,
                            void* stream);

/* Workspace bytes pkv_tree_verify_attn needs. */
int pkv_verify_workspace_size(pkv_pool* pool, const pkv_seq* reqs, int32_t n_req,
                              int32_t n_nodes, size_t* bytes);

/* Draft-tree verify attention [F4], one layer: request r's last n_nodes
 * tokens are the nodes of a draft tree, node j at position
 * len_r - n_nodes + j. Node i of request r attends, for every query head,
 * to all positions below len_r - n_nodes (the context) and to the nodes on
 * its own path to the root, itself included. parents: host int32
 * [n_req][n_nodes], parents[r][j] in {-1, 0 .. j-1}. q: device
 * [n_req][n_nodes][num_q_heads][head_dim] in kv_dtype; out: device float32,
 * same shape. 1 <= n_nodes <= 64. Requires kv_dtype == PKV_BF16 (the
 * contraction runs on the matrix cores). */
int pkv_tree_verify_attn(pkv_pool* pool, const pkv_seq* reqs, int32_t n_req,
                         const int32_t* parents, int32_t n_nodes, int32_t layer, const void* q,
                         float* out, float scale, void* ws, size_t ws_bytes, void* stream);

/* Keeps the first new_len tokens of seq (0 <= new_len <= its length):
 * blocks that then hold none of its tokens lose its reference (and are
 * freed at zero); a kept, partly filled last block keeps its count, so a
 * later append copies it if it is shared [D2]. Host only. */
int pkv_seq_truncate(pkv_pool* pool, pkv_seq seq, int32_t new_len);

/* Workspace bytes pkv_tree_commit(_batch) needs to keep n_accepted tokens
 * (for a batch: the sum over its requests). */
int pkv_tree_commit_workspace_size(const pkv_pool* pool, int32_t n_accepted, size_t* bytes);

/* Keeps the accepted path of a verified draft tree ([F4]; Ferrite page,
 * section 06: speculation never changes the text). seq's last n_nodes
 * tokens are the tree (node j at position len - n_nodes + j), parents as
 * for pkv_tree_verify_attn (host int32 [n_nodes]). accepted: host int32
 * [n_accepted], a chain from a root (parents[accepted[0]] == -1,
 * parents[accepted[i]] == accepted[i - 1]), 0 <= n_accepted <= n_nodes <=
 * 64. The sequence becomes its context followed by the accepted nodes' K/V
 * in path order, exactly as if they had been appended one by one: their
 * K/V are read into ws (device, >= pkv_tree_commit_workspace_size bytes),
 * the sequence is truncated to its context, and they are appended again
 * (copying a shared context tail on write). All or nothing on the host:
 * PKV_E_OOM (a needed copy finds no free block) or PKV_E_INVALID leave
 * the tables unchanged. Device work is queued on stream. */
int pkv_tree_commit(pkv_pool* pool, pkv_seq seq, int32_t n_nodes, const int32_t* parents,
                    const int32_t* accepted, int32_t n_accepted, void* ws, size_t ws_bytes,
                    void* stream);

/* pkv_tree_commit for n_req distinct requests of one verify step, with one
 * set of launches: parents and accepted are host int32 [n_req][n_nodes]
 * (row r of accepted holds request r's path in its first n_accepted[r]
 * entries), n_accepted host int32 [n_req]. Every request is truncated to
 * its context, then all kept paths are appended in request order as one
 * batch append; all or nothing over the batch (on PKV_E_OOM or
 * PKV_E_INVALID no table changes). ws: >= pkv_tree_commit_workspace_size
 * of the summed n_accepted. */
int pkv_tree_commit_batch(pkv_pool* pool, const pkv_seq* seqs, int32_t n_req, int32_t n_nodes,
                          const int32_t* parents, const int32_t* accepted,
                          const int32_t* n_accepted, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- prompt cache */

/* A cache of full blocks for resuming conversations from their longest
 * cached prefix (Ferrite page, section 07: snapshots at turn boundaries,
 * resume from the longest match, a system prompt shared by several agents
 * computed once, parked conversations). An entry is one full block keyed by
 * its block_size token ids and by the entry of the block before it, so a
 * chain of entries from the root spells out a whole token prefix; keys are
 * compared exactly. An entry holds one reference on its block, so a cached
 * block outlives the sequence that wrote it.
 *
 * Eviction: the next entry to go is, among entries with no child entry
 * whose block only the cache holds (reference count 1), the one walked
 * least recently by an insert or match (the deepest on a tie). An
 * allocation that finds no free block evicts one entry first; an append is
 * refused with PKV_E_OOM (and changes nothing) unless the free blocks plus
 * the entries eviction could reach cover it. Host only; no device work. */

/* Caches seq's full blocks among its first n_tokens positions, tokens[i]
 * being the id of the token at position i (n_tokens <= the sequence's
 * length). A key already present is refreshed, not duplicated. With the
 * cache at its capacity ("prefix_cache_blocks") an insert evicts as above,
 * never an entry it has walked, and stops when nothing can go. n_added
 * (may be NULL) receives the number of new entries. */
int pkv_prefix_insert(pkv_pool* pool, pkv_seq seq, const int32_t* tokens, int32_t n_tokens,
                      int32_t* n_added);

/* Creates a sequence holding the longest chain of cached blocks whose token
 * ids begin tokens[0 .. n_tokens) (whole blocks only; possibly none): each
 * block gains a reference, as in a fork. n_matched receives its length, a
 * multiple of block_size; the caller appends the rest. */
int pkv_prefix_match(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, pkv_seq* out,
                     int32_t* n_matched);

/* Drops every entry (releasing the cache's references). */
int pkv_prefix_clear(pkv_pool* pool);

/* Entries held, and how many of them eviction could remove now (either
 * pointer may be NULL). */
int pkv_prefix_info(const pkv_pool* pool, int32_t* entries, int32_t* evictable);

/* ---------------------------------------------------------------- misc */

/* Tuning knobs of the attention planner (defaults in parentheses):
 *   "path"              0 automatic (1 = vector ALUs, 2 = matrix cores)
 *   "chunk_tokens"      0 automatic: tokens per chunk of a shared segment
 *   "rows_per_item"     32: query rows a narrow work item serves (1..64)
 *   "wide"              1: chunks read by more rows use the wide-row kernel
 *   "wide_rows"         256: query rows a wide work item serves at most (16..256;
 *                       never more than one wide workgroup serves)
 *   "prefetch"          0: 1 makes each wave of the narrow kernel load its next
 *                       32-token step while the current one computes (with one
 *                       16-row block per wave)
 *   "row_blocks_per_wave" 0: 16-row blocks one wave of the narrow kernel may
 *                       own, 1 or 2; with 2 (head_dim <= 128 only) an item of
 *                       up to 32 rows loads each K/V step once, at the cost of
 *                       occupancy; 0 picks 2 when items of more than 16 rows
 *                       hold at least a quarter of the narrow launch's tokens
 *   "tokens_per_row"    0: chunk length per query row reading it (between
 *                       "min_chunk_tokens" and 8192 tokens; 1..8192), 0 for
 *                       64 up to head_dim 128 and 32 above
 *   "min_chunk_tokens"  0: shortest automatic chunk (32..8192), 0 for 1024 up
 *                       to head_dim 128 and 768 above (a 256-dim token is
 *                       twice the bytes)
 *   "short_items"       1: a narrow item of at most 16 rows and "short_tokens"
 *                       tokens runs on one wave (four such planes per workgroup)
 *                       instead of four waves that split its steps and merge
 *                       (0: always four)
 *   "short_tokens"      256: see "short_items" (32..8192)
 *   "fold_tokens"       64: a shared segment of fewer tokens is read by each
 *                       branch that holds it, together with the branch's
 *                       neighbouring short segments, instead of once for all
 *                       (its partial states would outweigh its K/V); 0: never
 *   "group_rows"        16: after folding, sibling branches whose folded paths
 *                       share blocks (the leaves under one MCTS node) are served
 *                       by one item of up to this many rows (group_rows / G
 *                       branches; at most 16 and at most "rows_per_item"), which
 *                       reads each of their blocks once and masks it for the
 *                       rows whose branch does not hold it; a group is formed
 *                       only when its blocks are at most 3/4 of its members'
 *                       (0: never; the vector path never groups)
 *   "prefix_cache_blocks" num_blocks: most entries the prompt cache holds
 *                       (0..num_blocks; applies to later inserts)
 *   "finalize"          1: when every branch has one chunk read by narrow items and
 *                       the rest by wide items (an MCTS tree: the wide root, each
 *                       leaf's folded path narrow), the narrow launch, which runs
 *                       after the wide one, merges each row's partial states and
 *                       writes the output rows itself: no combine launch; the
 *                       outputs are bit-identical to the combine's (0: always
 *                       combine; also off with "concurrent" 1)
 *   "inline_plan"       1: a decode or verify plan whose arrays fit in 12 KiB (and
 *                       whose combine lists fit in 1 KiB) travels in the kernel
 *                       launches' own arguments, so no host-to-device copy of
 *                       the plan precedes them; outputs are bit-identical either
 *                       way (0: always stage and copy the plan into the workspace)
 *   "concurrent"        0: 1 runs the wide-item launch on a second stream of the
 *                       library's, forked from and joined back into the caller's
 *                       stream, beside the narrow-item launch
 *   "wide_fill"         1: fill every wide item of a chunk but the last to the row
 *                       limit (0: split the rows evenly)
 *   "wide_waves"        0: compute waves per wide workgroup, 4, 6 or 8; 0 picks 8
 *                       up to head_dim 128 and 6 at 256 (the workgroup adds one
 *                       or two loader waves)
 *   "wide_row_blocks"   0: 16-row blocks each wide compute wave owns, 1 or 2; 0
 *                       picks 2 up to head_dim 128 and 1 at 256 (6 waves, and 8
 *                       at head_dim 256, always own one); a wide item holds at
 *                       most 16 * waves * row blocks rows
 *   "wide_spec"         0: 1 runs wide items on the kernel whose softmax and P.V
 *                       run on separate waves of each SIMD (head_dim 64 / 128,
 *                       bf16, the automatic wide shape) when every wide item
 *                       holds more than 192 rows; 2 whenever the shape allows;
 *                       the same partial states to fp32 rounding
 *   "target_workgroups" 256: chunks are shortened (down to 1024 tokens) while the
 *                       grid has fewer than 3/4 of this many workgroups
 *   "tree"              0: never; 1: a decode whose rows all fit one workgroup
 *                       (branches x query-head group <= 256) at head_dim 64 or
 *                       128 (bf16) runs as one launch with one workgroup per
 *                       (layer, KV head) that reads every chunk of the batch
 *                       once for all rows holding it and writes the outputs (no
 *                       partial states, no combine), when some segment has more
 *                       rows than a narrow item and the (layer, KV head) planes
 *                       alone fill the chip (at least 3/4 of
 *                       "target_workgroups"); 2: whenever the rows fit
 *   "tree_stages"       5: LDS ring depth of the tree launch (4, 5 or 6)
 *   "tree_piece_tokens" 512: segments of 64 or more rows are cut into pieces of
 *                       this many tokens, spread among the narrower segments
 *                       (32..8192)
 *   "timing"            0: 1 records a pair of HIP events at the start and end
 *                       of every kernel the pool launches (pkv_timing_read)
 * Unknown keys or out-of-range values are PKV_E_INVALID. */
int pkv_pool_set_option(pkv_pool* pool, const char* key, int64_t value);

/* Device time of the kernels launched since the last read (with the
 * "timing" option on): kernel is "attention" (items of few rows),
 * "attention_wide" (items of many rows; the two may overlap in time),
 * "attention_tree" (the tree launch), "attention_span" (from before the first
 * to after the last attention launch of a call, on the caller's stream), "combine", "append" (the
 * launch that performs copy-on-write copies and token writes) or
 * "commit_gather" (the read-out of a committed path's K/V). Waits for
 * the last recorded launch, returns the summed milliseconds and the launch
 * (or call) count, and resets both. */
int pkv_timing_read(pkv_pool* pool, const char* kernel, double* total_ms, int64_t* launches);

/* Device: reads `bytes` bytes of device memory at src once, with 16-byte
 * vector loads spread over every CU (8192 workgroups, each a contiguous
 * range, four loads in flight per lane), on the stream; streaming = 1 uses non-temporal loads (as the attention kernels do
 * for K/V that only one wave reads), 0 ordinary ones. A measuring aid, not
 * part of the method: it gives the practical HBM read rate of this GPU to
 * set the attention launches' rates beside. sink: device memory of at least
 * 4096 bytes that the kernel may write (its contents afterwards mean
 * nothing; it keeps the loads from being optimised away). bytes must be a
 * positive multiple of 16 and src 16-byte aligned (else PKV_E_INVALID,
 * checked before any device work). */
int pkv_stream_read(const void* src, int64_t bytes, int32_t streaming, void* sink, void* stream);

/* Last error message of this thread ("" if none). */
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
