/*
 * pagedkv.h -- C ABI of the paged KV cache and PagedAttention decode path
 * for AMD Instinct MI355X (gfx950).
 *
 * The problem, as the sources state it:
 *   - The KV cache is cut into fixed blocks of 16 tokens held in one flat
 *     physical pool; each sequence keeps a block table whose entry i names
 *     the physical block of its i-th logical block; a block is taken only
 *     when the sequence's current block is full and every block returns to
 *     the free pool when the sequence ends [KV Cache 工程学 §15.5;
 *     新一代 KV Cache 管理 §8.1].
 *   - Block tables of different sequences may point at the same physical
 *     block, counted by reference, so shared prompts and parallel samples are
 *     stored once [新一代 KV Cache 管理 §8.1; KV Cache 工程学 §15.6]; a write
 *     into a shared block copies it first [KV Cache 与 PagedAttention,
 *     first article, "PagedAttention 如何解决这个问题"].
 *   - The attention kernel takes the block table as an extra input and
 *     fetches K and V through it [KV Cache 工程学 §15.5 "PagedAttention 的代价";
 *     新一代 KV Cache 管理 §8.1].
 *   - A decode step computes only the new token's K/V, stores them, and
 *     attends once over the i cached tokens [KV Cache 工程学 §15.1].
 *   - Usage (used / total blocks) is what an engine watches to refuse work
 *     [KV Cache 工程学 §15.9].
 *
 * Conventions
 *   - Every function returns a pkv_status (0 = success, negative = error),
 *     except the size queries, which return 0 on invalid input.  On error a
 *     thread-local message is available from pkv_last_error().  Nothing
 *     aborts; a failed call leaves all host state unchanged.
 *   - The library owns host bookkeeping objects only (pkv_pool and the
 *     sequences inside it, addressed by int64 id).  Every device buffer is
 *     owned by the caller and only borrowed for the duration of the call; the
 *     library allocates no device memory at run time (its static device
 *     memory: 8 KiB of idle tiles that the decode kernels read past the end
 *     of a wave's work, and the scratch array of
 *     paged_attention_decode_noalloc).
 *   - Device calls are asynchronous on the given stream (a hipStream_t passed
 *     as void*; NULL = the legacy default stream) and never synchronize.
 *   - Host-visible arguments are validated; device-resident tables and
 *     lengths are trusted, but kernels clamp block ids into [0, num_blocks)
 *     and lengths into [0, 16 * max_blocks_per_seq] so that bad tables give
 *     wrong numbers, never out-of-bounds accesses.  pkv_validate_tables()
 *     checks host copies of them.
 *   - A pool object is not thread-safe; use one per thread or lock around it.
 *
 * Pool layout in device memory (one K pool and one V pool per layer):
 *   X = 16 bytes / element size (8 for bf16, 4 for f32)
 *   K element (blk, g, t, d) at (((blk*H + g)*(D/X) + d/X)*16 + t)*X + d%X
 *   V element (blk, g, t, d) at  ((blk*H + g)*D + d)*16 + t
 *   blk = physical block, g = kv head (H of them), t = slot in block
 *   (0..15), d = element of the head (D of them).  One (blk, g) tile is
 *   16*D elements (4 KiB for bf16 at D = 128) and contiguous in both pools.
 *   A token's slot id is blk*16 + t.  One-byte caches (int8, FP8) use X = 16,
 *   store K slot t at position p(t) (bits 2 and 3 of t exchanged) and end
 *   each tile with its 16 scales: see "Pool layout" below.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,   /* bad argument (null pointer, unsupported shape...) */
  PKV_ERR_NO_BLOCKS = -2, /* the free pool cannot satisfy the request */
  PKV_ERR_BAD_BLOCK = -3, /* block id outside [0, num_blocks) */
  PKV_ERR_REFCOUNT = -4,  /* free/incref of a block that is not allocated */
  PKV_ERR_CAPACITY = -5,  /* caller's output array is too small */
  PKV_ERR_HIP = -6,       /* a HIP runtime call failed (message has details) */
  PKV_ERR_WORKSPACE = -7, /* workspace missing or smaller than required */
  PKV_ERR_BAD_SEQ = -8    /* unknown sequence id */
};

/* Storage of the cache.  PKV_F32 and PKV_BF16 store elements as given; the
 * queries and the rows handed to paged_kv_append have the same type.
 * PKV_INT8 stores one byte per element instead of two [KV Cache 工程学
 * §15.7 (3), KV Cache 量化]: each token's row of one kv head (D values, K and
 * V separately) keeps int8 codes and one float32 scale,
 *   amax = max |x_d|, scale = amax / 127, code_d = round-half-even(x_d / scale)
 *   clamped to [-127, 127] (all codes 0 when amax = 0), value = code * scale,
 * computed in float32 when paged_kv_append stores the row.  Queries and
 * appended rows are bfloat16.
 * PKV_FP8 is the other one-byte format the same section names: the same
 * tiles and scales, with FP8 E4M3 codes as the OCP 8-bit floating point
 * format defines them (sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals m/8 * 2^-6, largest finite 448, S.1111.111 NaN):
 *   amax = max |x_d|, scale = amax / 448, code_d = the E4M3 value nearest to
 *   x_d / scale (ties to the even mantissa), saturated at 448, sign kept
 *   (all codes 0 when amax = 0), value = E4M3(code) * scale.
 * The two NaN codes are never written. */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_INT8 = 2, PKV_FP8 = 3 };

#define PKV_BLOCK_SIZE 16

/* Pool layout.  A pool is num_blocks * num_kv_heads tiles, tile (blk, g) at
 * index blk * H + g; a tile holds the 16 token slots of one block for one kv
 * head.  With X = 16 / element size (X = 16 for one-byte codes):
 *   K element (blk, g, t, d) at tile offset ((d / X) * 16 + p(t)) * X + d % X
 *   V element (blk, g, t, d) at tile offset d * 16 + t
 * (in elements; for PKV_INT8 and PKV_FP8 in bytes), where p(t) = t for f32
 * and bf16 and, for one-byte codes, t with its bits 2 and 3 exchanged (a row
 * of 16-byte K units holds slots 0-3, 8-11, 4-7, 12-15 in that order).  An
 * f32/bf16 tile is 16 * D elements.  A PKV_INT8 or PKV_FP8 tile is
 * 16 * D + 64 bytes: the codes, then the 16 float32 scales of slots 0..15 at
 * byte 16 * D + 4 * t. */
typedef struct {
  int32_t num_blocks;   /* physical blocks in the pool (> 0) */
  int32_t block_size;   /* tokens per block; must be 16 */
  int32_t num_kv_heads; /* H (> 0) */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t kv_dtype;     /* PKV_F32, PKV_BF16, PKV_INT8 or PKV_FP8 */
} pkv_layout;

/* Thread-local description of the last error raised on this thread. */
const char *pkv_last_error(void);
/* Library version string. */
const char *pkv_version(void);

/* ------------------------------------------------------------ block pool */
typedef struct pkv_pool pkv_pool;

/* Create the host block manager for a pool: the physical KV cache cut into
 * fixed 16-token blocks, all free at first [KV Cache 工程学 §15.5].
 * free_order (nullable) is a permutation of [0, num_blocks): the order in
 * which blocks are first handed out (NULL = 0, 1, 2, ...).  The free pool is a stack: a freed block is the
 * next one handed out.  *out receives the new pool. */
int pkv_pool_create(const pkv_layout *layout, const int32_t *free_order, pkv_pool **out);
/* Destroy a pool (NULL is accepted). */
int pkv_pool_destroy(pkv_pool *pool);

/* Take one free block; its reference count becomes 1.  Blocks are counted by
 * reference so that several block tables may name one physical block
 * [新一代 KV Cache 管理 §8.1; KV Cache 工程学 §15.5, "PagedAttention 的好处" 3]. */
int pkv_block_alloc(pkv_pool *pool, int32_t *block_out);
/* Add a reference to an allocated block. */
int pkv_block_incref(pkv_pool *pool, int32_t block);
/* Drop a reference; at zero the block returns to the free pool. */
int pkv_block_free(pkv_pool *pool, int32_t block);
/* Reference count of a block (0 = free) into *out. */
int pkv_block_refcount(const pkv_pool *pool, int32_t block, int32_t *out);
/* Number of blocks that can be handed out (free, or idle in the prefix cache)
 * into *out. */
int pkv_pool_num_free(const pkv_pool *pool, int32_t *out);

/* --------------------------------------------------------------- sequences */
/* New empty sequence with an empty block table [KV Cache 工程学 §15.5]; ids
 * are 0, 1, 2, ... in creation order, never reused. */
int pkv_seq_create(pkv_pool *pool, int64_t *id_out);
/* New sequence sharing every block of parent (each gains one reference): the
 * parallel samples of one prompt read its blocks through their own tables
 * [新一代 KV Cache 管理 §8.1, best-of-8]. */
int pkv_seq_fork(pkv_pool *pool, int64_t parent, int64_t *child_out);
/* Reserve slots for n more tokens at the end of a sequence, all or none:
 * a token goes into the current block while it has room, and a new block is
 * taken when it is full [KV Cache 工程学 §15.5]; a shared block is copied
 * before a write [KV Cache 与 PagedAttention, "PagedAttention 如何解决这个问题"].
 * For each token at position p: when p % 16 == 0 a block is taken and
 * appended to the table; otherwise, when the tail block is shared (count
 * > 1), a block is taken, the pair (old, new) is written to cow_pairs_out
 * for a whole-block copy (pkv_copy_blocks) that must run before the token
 * is stored, the old block loses a reference and the table points at the
 * new one.  slots_out[i] = table[p / 16] * 16 + p % 16.
 * slots_out has room for n entries; cow_pairs_out for cow_cap pairs
 * (int32 src, dst); *n_cow receives the number of pairs written.
 * Errors: PKV_ERR_NO_BLOCKS, PKV_ERR_CAPACITY (cow_cap too small). */
int pkv_seq_append_slots(pkv_pool *pool, int64_t id, int32_t n, int64_t *slots_out,
                         int32_t *cow_pairs_out, int32_t cow_cap, int32_t *n_cow);
/* The same for a batch of sequences, n tokens each, processed in batch
 * order; slots_out is [num_seqs][n].  All or none over the whole batch. */
int pkv_batch_append_slots(pkv_pool *pool, const int64_t *ids, int32_t num_seqs, int32_t n,
                           int64_t *slots_out, int32_t *cow_pairs_out, int32_t cow_cap,
                           int32_t *n_cow);
/* Release a sequence: its blocks lose a reference in table order; blocks
 * reaching zero are pushed onto the free pool in that order (a finished
 * sequence returns its blocks [KV Cache 工程学 §15.5]). */
int pkv_seq_free(pkv_pool *pool, int64_t id);
/* Number of tokens of a sequence into *len_out. */
int pkv_seq_len(const pkv_pool *pool, int64_t id, int32_t *len_out);
/* Copy a sequence's block table -- entry i names the physical block of its
 * logical block i [KV Cache 工程学 §15.5] -- into out (room for cap
 * entries); *n_out receives its length.  PKV_ERR_CAPACITY if cap is too
 * small. */
int pkv_seq_block_table(const pkv_pool *pool, int64_t id, int32_t *out, int32_t cap,
                        int32_t *n_out);
/* Block tables and lengths of a batch, as paged_attention_decode reads them
 * (the table is an extra input of the attention kernel [KV Cache 工程学
 * §15.5, "PagedAttention 的代价" 2]):
 * tables_out [num_seqs][max_blocks_per_seq] (entries past a sequence's
 * blocks are set to 0), context_lens_out [num_seqs]. */
int pkv_batch_block_tables(const pkv_pool *pool, const int64_t *ids, int32_t num_seqs,
                           int32_t max_blocks_per_seq, int32_t *tables_out,
                           int32_t *context_lens_out);

/* ------------------------------------------------------------ prefix cache */
/* Prefix caching [KV Cache 工程学 §15.6; 新一代 KV Cache 管理 §8.3]: a full
 * 16-token block is identified by a hash of the whole prefix that ends with
 * it (64-bit FNV-1a over the previous block's key and the block's 16 token
 * ids, little-endian; the block's tokens and its parent key are checked on a
 * hit), so a request whose prompt starts with a cached prefix points its
 * block table at the cached blocks and skips their prefill.  A cached block
 * whose reference count drops to zero stays cached ("idle"); idle blocks are
 * evicted least recently used first, only when the free stack is empty.
 * The blocks of one sequence that turn idle together enter the LRU deepest
 * first.  Off by default. */
typedef struct {
  int64_t lookups;      /* pkv_seq_create_from_prefix calls with the cache on */
  int64_t query_tokens; /* full-block tokens looked up */
  int64_t hit_tokens;   /* tokens found cached (prefill skipped) */
  int64_t registered;   /* blocks entered into the cache */
  int64_t evictions;    /* idle cached blocks taken for reuse */
  int32_t cached_blocks; /* blocks in the cache now (in use or idle) */
  int32_t idle_blocks;   /* cached blocks held by no sequence */
  double hit_rate;      /* hit_tokens / query_tokens */
} pkv_prefix_stats;

/* Turn the prefix cache on (enable != 0) or off (idle cached blocks return to
 * the free pool, oldest first). */
int pkv_prefix_cache_enable(pkv_pool *pool, int32_t enable);
/* New sequence whose table starts with the longest run of cached full blocks
 * matching the first tokens of token_ids[0..n) (each gains a reference);
 * *n_cached_out receives its length, a multiple of 16.  The caller appends
 * the remaining n - *n_cached_out tokens, stores their K/V, and registers
 * the prompt.  With the cache off the sequence starts empty. */
int pkv_seq_create_from_prefix(pkv_pool *pool, const int32_t *token_ids, int32_t n, int64_t *id_out,
                               int32_t *n_cached_out);
/* Enter the full blocks of a sequence's first n tokens (token_ids[0..n),
 * n <= its length, K/V already stored) into the cache; content that is
 * already cached is left as it is.  *n_registered (nullable) receives the
 * number of blocks added. */
int pkv_seq_register_prefix(pkv_pool *pool, int64_t id, const int32_t *token_ids, int32_t n,
                            int32_t *n_registered);
int pkv_prefix_cache_stats(const pkv_pool *pool, pkv_prefix_stats *out);

/* -------------------------------------------------------------- statistics */
typedef struct {
  int32_t num_blocks;
  int32_t num_free;        /* blocks that can be handed out: free, or idle cached */
  int32_t num_used;        /* blocks held by at least one reference */
  int32_t num_shared;      /* blocks with reference count > 1 */
  int64_t num_seqs;        /* live sequences */
  int64_t tokens_logical;  /* sum of live sequence lengths */
  int64_t tokens_stored;   /* distinct token slots in use (shared ones once) */
  double usage;            /* num_used / num_blocks [KV Cache 工程学 §15.9] */
  double internal_fragmentation; /* 1 - tokens_stored / (num_used * 16)
                                    [新一代 KV Cache 管理 §8.1] */
} pkv_stats;

int pkv_pool_stats(const pkv_pool *pool, pkv_stats *out);
/* K and V bytes of one token across num_layers layers:
 * num_layers * 2 * num_kv_heads * head_dim * element size
 * [KV Cache 工程学 §15.2]; for PKV_INT8 and PKV_FP8 each row also carries its 4-byte
 * scale: num_layers * 2 * num_kv_heads * (head_dim + 4).  0 on invalid input. */
int64_t pkv_kv_bytes_per_token(const pkv_layout *layout, int32_t num_layers);
/* Bytes of one pool (K or V; both have this size).  0 on invalid input. */
int64_t pkv_pool_bytes(const pkv_layout *layout);
/* Check host copies of block tables and lengths: every entry a sequence
 * uses is in [0, num_blocks) and every length is in [0, 16 * max_blocks]. */
int pkv_validate_tables(const pkv_layout *layout, const int32_t *tables, const int32_t *context_lens,
                        int32_t num_seqs, int32_t max_blocks_per_seq);

/* ------------------------------------------------- swap to host memory */
/* When device memory is short, single blocks move to host memory instead of
 * whole sequences ("fine-grained eviction" [KV Cache 与 PagedAttention,
 * summary]; offloading of KV not needed right away [KV Cache 工程学 §15.7
 * (4)]), chosen by the Clock (second chance) policy [PagedAttention：大模型KV
 * Cache内存管理革新 §3.3].  Host memory holds num_host_blocks block slots in
 * caller-owned K and V buffers of the pool's tile layout (num_host_blocks *
 * num_kv_heads tiles each; pinned memory the GPU can address).  Every device
 * block has a reference bit, set when the block is taken, when a token slot
 * in it is assigned and when pkv_batch_block_tables exports a table naming
 * it (pkv_seq_block_table only inspects).  A table entry e < 0 names
 * host slot -e-1: such a sequence is not resident, and appends and
 * pkv_batch_block_tables refuse it (PKV_ERR_INVALID) until pkv_seq_swap_in. */
typedef struct {
  int32_t host_blocks;   /* configured host slots */
  int32_t host_used;     /* slots holding a block */
  int32_t host_free;
  int32_t clock_hand;    /* next device block the hand looks at */
  int64_t swapped_out;   /* blocks moved to the host so far */
  int64_t swapped_in;    /* blocks moved back */
} pkv_swap_stats;

/* Set the number of host slots (0 .. n-1, handed out LIFO, slot 0 first).
 * Refused while a slot holds a block. */
int pkv_swap_configure(pkv_pool *pool, int32_t num_host_blocks);
/* Choose up to `want` victims with the Clock hand, which moves over device
 * block ids from where it stopped: a block held by some sequence and only
 * through block tables (a block the caller also holds by pkv_block_alloc or
 * pkv_block_incref is not), not in the prefix cache and not held by a
 * sequence of protect_ids (the batch about to run) is a candidate; a candidate whose reference bit is set has it cleared
 * and is passed over; one whose bit is clear moves to a host slot: every
 * table entry naming it becomes -(slot+1), its references move to the slot
 * and the device block returns to the free stack.  Stops after `want`
 * victims, when host slots run out, or after two turns of the hand.
 * pairs_out (cap pairs, cap >= want) receives int32 (device block, host slot)
 * pairs; *n_out their number.  The caller copies them (pkv_swap_copy, device
 * pool to host slots) before any later device call can write the freed
 * blocks: on the same stream, enqueue the copy first. */
int pkv_swap_out(pkv_pool *pool, int32_t want, const int64_t *protect_ids, int32_t n_protect, int32_t *pairs_out,
                 int32_t cap, int32_t *n_out);
/* Bring every host entry of a sequence back, in table order, all or nothing:
 * each takes a device block (free stack first, then idle cached blocks, as an
 * append does); every sequence sharing the block becomes resident for it.
 * pairs_out receives int32 (host slot, device block) pairs to copy host ->
 * device (pkv_swap_copy) before the sequence's next device call; *n_out
 * their number (also on PKV_ERR_CAPACITY).  PKV_ERR_NO_BLOCKS when the pool
 * cannot hold them (nothing changes). */
int pkv_seq_swap_in(pkv_pool *pool, int64_t id, int32_t *pairs_out, int32_t cap, int32_t *n_out);
/* 1 when every table entry of the sequence is a device block, else 0. */
int pkv_seq_resident(const pkv_pool *pool, int64_t id, int32_t *resident_out);
int pkv_swap_space_stats(const pkv_pool *pool, pkv_swap_stats *out);

/* ---------------------------------------------------------- device calls */
/* Store the new tokens' K and V into their slots [KV Cache 工程学 §15.1,
 * §15.5].  k_new, v_new: [num_tokens][H][D] of kv_dtype, bf16 for
 * PKV_INT8 and PKV_FP8 (device); d_slots: int64 [num_tokens] (device),
 * slot = blk*16 + t; a negative slot or one past the pool is skipped.  f32
 * and bf16 bits are copied unchanged; PKV_INT8 and PKV_FP8 rows are
 * quantised as described at PKV_INT8 and PKV_FP8 (rows must be finite).
 * Slots must be distinct. */
int paged_kv_append(const pkv_layout *layout, void *k_pool, void *v_pool, const void *k_new,
                    const void *v_new, const int64_t *d_slots, int32_t num_tokens, void *stream);

/* Copy whole blocks (all heads, all slots, K and V) -- the copy of a shared
 * block before a write [KV Cache 与 PagedAttention, "PagedAttention 如何解决
 * 这个问题"]: d_pairs is int32 [num_pairs][2] of (src, dst) on the device, as
 * pkv_seq_append_slots reports them for copy-on-write.  Destinations must be distinct and not
 * also sources. */
int pkv_copy_blocks(const pkv_layout *layout, void *k_pool, void *v_pool, const int32_t *d_pairs,
                    int32_t num_pairs, void *stream);

/* Copy whole blocks (all heads, K and V) from one pool to another of the
 * same layout: d_pairs is int32 [num_pairs][2] of (source block, destination
 * block), readable by the device.  Either pool may be pinned host memory
 * (the swap space of pkv_swap_out / pkv_seq_swap_in); src_blocks and
 * dst_blocks are the pools' sizes in blocks, and a pair outside them is
 * skipped.  Destinations must be distinct. */
int pkv_swap_copy(const pkv_layout *layout, void *dst_k, void *dst_v, int32_t dst_blocks, const void *src_k,
                  const void *src_v, int32_t src_blocks, const int32_t *d_pairs, int32_t num_pairs, void *stream);

/* A decode plan [balanced-split scheduling; not part of the method]: what
 * the call that recorded a plan was (opaque; all zeros = no plan yet).  See
 * pkv_decode_opts.plan. */
#define PKV_PLAN_KEY_INTS 32
typedef struct {
  int64_t opaque[PKV_PLAN_KEY_INTS];
} pkv_decode_plan;

/* Decode options (all fields may be zero / NULL for defaults). */
typedef struct {
  int32_t partition_tokens; /* a positive multiple of 32, or 0 for the default
                               (128): the fewest context tokens the balanced
                               split gives one wave, in either kernel.  Fewer
                               tokens per wave cut contexts more finely. */
  int32_t kernel;           /* 0 auto (matrix cores for int8 and FP8, and
                               for bf16 with G >= 4); 1 the wavefront-
                               reduction kernel (f32, bf16); 2 the matrix-core
                               kernel (bf16, int8, FP8) */
  int32_t waves_per_simd;   /* matrix-core kernel: resident waves per SIMD,
                               0 = default (1), 1 or 2.  One streams K/V from
                               HBM fastest (waves sharing a SIMD do not
                               progress alike); two serve batches whose blocks
                               are mostly shared (and so L2-resident) better. */
  void *ev_begin;           /* optional hipEvent_t recorded before the first kernel */
  void *ev_partition_done;  /* optional hipEvent_t recorded after the partition kernel */
  void *ev_end;             /* optional hipEvent_t recorded after the merge kernel */
  int32_t xcd_weights[8];   /* balanced split: relative work of the 8 XCDs (all 0 =
                               equal).  XCD x runs the workgroups b with b % 8 == x
                               and streams K/V at its own rate; weights from
                               pkv_xcd_weights_from_trace make them finish
                               together.  Used when all > 0 and the whole grid
                               works; results depend on the weights, never on
                               timing. */
  int32_t load_policy;      /* K/V tile loads: 0 auto (streaming for f32 and
                               bf16 caches with one wave per SIMD, cached
                               otherwise), 1 streaming: the non-temporal hint,
                               for batches that read every tile once, 2 cached:
                               tiles kept in L2 for reuse (blocks shared by
                               many sequences) */
  int32_t *trace;           /* optional device buffer of 4 * PKV_TRACE_WAVES int32:
                               the matrix-core kernel writes, per wave, its XCD,
                               chunk count and start/end clock (100 MHz, low 32
                               bits); clear it before the call (waves without
                               work write nothing) */
  pkv_decode_plan *plan;    /* optional, with plan_buffer: the split of the
                               calls of one step (see paged_attention_plan_bytes) */
  void *plan_buffer;        /* device buffer of the plan, 16-byte aligned */
  size_t plan_bytes;        /* its size, at least paged_attention_plan_bytes() */
} pkv_decode_opts;

/* Waves a decode trace buffer holds. */
#define PKV_TRACE_WAVES 8192

/* Per-XCD weights from a decode trace [balanced-split tuning; not part of
 * the method]: weight x = 1000 * (chunks per time of XCD x's waves) /
 * (mean over XCDs).  h_trace: host copy of the trace (4 int32 per wave,
 * n_waves of them; all-zero records are skipped).  Fails with
 * PKV_ERR_INVALID when some XCD has no traced wave. */
int pkv_xcd_weights_from_trace(const int32_t *h_trace, int32_t n_waves, int32_t weights_out[8]);

/* Bytes of workspace paged_attention_decode needs for these sizes and
 * options (opts may be NULL).  Layout: the partial outputs and (max, sum)
 * pairs of contexts cut between waves, two slots of G query rows per wave
 * (its first and its last context), then the merge kernel's schedule,
 *   float32 [nslots][G][D], float32 [nslots][G][2], int32 [22 + num_seqs],
 *   nslots = 2 * max(1, min(2048, num_seqs * H * ceil(max_context_len / 32)
 *                                  / fewest chunks per wave)),
 * each region padded to 16 bytes.  Its contents need not be preserved
 * between calls.  Depends on the sizes only, not on the device. */
size_t paged_attention_workspace_bytes(const pkv_layout *layout, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len,
                                       const pkv_decode_opts *opts);

/* PagedAttention decode [KV Cache 工程学 §15.5; 新一代 KV Cache 管理 §8.1]:
 * for every sequence b and query head h (kv head g = h / (Hq / H)),
 *   out[b][h] = sum_j softmax_j(scale * q[b][h] . K_j) * V_j
 * over the context_lens[b] tokens j, where token j is slot j % 16 of block
 * d_block_tables[b][j / 16].  The softmax spans the whole context.
 *   out: float32 [num_seqs][num_q_heads][D] (device, written)
 *   q:   kv_dtype [num_seqs][num_q_heads][D], bf16 for PKV_INT8 and PKV_FP8 (device)
 *   d_block_tables: int32 [num_seqs][max_blocks_per_seq] (device)
 *   d_context_lens: int32 [num_seqs] (device); a length of 0 gives zeros
 *   max_context_len: an upper bound of every context length (sizes the grid);
 *   a longer length is treated as max_context_len
 *   scale: usually 1 / sqrt(D)
 *   workspace: device scratch of paged_attention_workspace_bytes() bytes;
 *   calls that share one workspace must not overlap (keep them on one
 *   stream).
 * Requires num_q_heads % num_kv_heads == 0, G = num_q_heads / num_kv_heads
 * <= 16, D in {64, 128}, max_context_len <= min(16 * max_blocks_per_seq, 2^22).
 * Work split: a persistent partition kernel in which every wave takes an
 * equal, contiguous share of the batch's 32-token chunks whatever the mix of
 * context lengths.  A context held by one wave is written directly; a
 * context cut between waves leaves one partial maximum, sum and unnormalised
 * output per wave, combined by a merge kernel (log-sum-exp of the partials).
 * The matrix-core kernel runs the group's query heads as a 16-column tile
 * (bf16 with G >= 4, int8, FP8); the wavefront-reduction kernel serves f32
 * caches and small groups. */
int paged_attention_decode(const pkv_layout *layout, float *out, const void *q, const void *k_pool,
                           const void *v_pool, const int32_t *d_block_tables,
                           const int32_t *d_context_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                           void *workspace, size_t workspace_bytes, const pkv_decode_opts *opts,
                           void *stream);

/* Decode plans [balanced-split scheduling; not part of the method].  The
 * decode calls of one step (one per layer) share the block tables and
 * context lengths, and so the split of the work between waves.  With
 * opts->plan and opts->plan_buffer, a call whose *opts->plan is all zeros
 * schedules itself as usual and also records that split in the buffer: the
 * chunk scan and the merge kernel's schedule header, and for every wave its
 * share and the cursors and physical blocks of its first two chunks; it
 * then fills *opts->plan with what the call was.  A later call given that
 * plan takes the split from the buffer, so its waves' first K/V requests
 * wait on one memory round trip instead of three (the lengths, then the
 * block table, then the tiles).  Results are bitwise those of a call
 * without a plan.
 *   plan buffer: paged_attention_plan_bytes() bytes of device memory for
 *   the calls' num_seqs, num_q_heads, max_context_len and partition option;
 *   it must stay allocated and unchanged while calls use the plan
 * The calls may differ in out, q, pools, scale and workspace (one call per
 * layer); a call given a recorded plan whose other arguments (the table and
 * length pointers and the plan buffer included), options (but events and
 * trace) or current device differ from the recording call's fails with
 * PKV_ERR_INVALID, and a plan buffer smaller than needed with
 * PKV_ERR_WORKSPACE.  A plan buffer holds one plan: once another call
 * records into it, calls given a plan recorded there before fail with
 * PKV_ERR_INVALID (the library remembers the latest recording of up to 256
 * buffers; a plan whose buffer it has forgotten is refused as well).  The plan holds the lengths and blocks the recording call
 * read: once tables or lengths change (a new token, a new block, a swap),
 * zero *plan so that the next call records again; a call from a stale plan
 * reads the old shares and blocks (in bounds, but the results are wrong).
 * The wavefront-reduction kernel schedules itself every call (its plans
 * only check the arguments). */
size_t paged_attention_plan_bytes(const pkv_layout *layout, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, const pkv_decode_opts *opts);

/* paged_attention_decode without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * arguments, results and errors are those of paged_attention_decode; the
 * workspace is the library's own scratch, a static device array of
 * 34,111,584 bytes (the workspace of the largest call: 2 * 2048 slots of 16
 * query rows of 128 floats, their maxima and sums, and the schedule header
 * of 8192 sequences), one copy per GPU, held until the process ends; its
 * address is looked up on the first call on each device.  Every legal call
 * fits it; a call whose workspace would not fails with PKV_ERR_WORKSPACE.
 * All calls on one GPU share that GPU's scratch: calls that overlap on one
 * GPU (different streams, or different host threads without ordering)
 * race and give wrong results.  Allocates nothing: no hipMalloc, hipFree or
 * allocating library routine. */
int paged_attention_decode_noalloc(const pkv_layout *layout, float *out, const void *q, const void *k_pool,
                                   const void *v_pool, const int32_t *d_block_tables,
                                   const int32_t *d_context_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                   const pkv_decode_opts *opts, void *stream);

/* Causal prefill over a paged cache [KV Cache 工程学 §15.1: a prompt of i
 * tokens is an i x i causal attention; §15.6 and 新一代 KV Cache 管理 §8.3:
 * a cached prefix is attended to, not prefilled again].  Sequence b holds
 * d_context_lens[b] tokens in its table (slot j % 16 of block
 * d_block_tables[b][j / 16]); its last nq_b = d_query_start[b+1] -
 * d_query_start[b] tokens are new and their K and V must already be stored
 * (paged_kv_append).  New token t, at position p_b + t with
 * p_b = d_context_lens[b] - nq_b, attends to positions 0 .. p_b + t:
 *   out[r][h] = sum_{j <= p_b + t} softmax_j(scale * q[r][h] . K_j) * V_j,
 *   r = d_query_start[b] + t, kv head g = h / (num_q_heads / H).
 *   out: float32 [T][num_q_heads][D] (device, written), T = d_query_start[num_seqs]
 *   q:   bf16 [T][num_q_heads][D] (device), also for PKV_INT8 and PKV_FP8
 *   d_block_tables: int32 [num_seqs][max_blocks_per_seq] (device)
 *   d_context_lens: int32 [num_seqs] (device); d_query_start: int32 [num_seqs + 1]
 *   (device), non-decreasing from 0, with nq_b <= d_context_lens[b] (a larger
 *   nq_b is cut to d_context_lens[b]) and nq_b <= max_query_len (rows past it
 *   are not written)
 *   max_context_len: bounds every context (a longer one is treated as it)
 * Requires a bf16, int8 or FP8 cache, num_q_heads % num_kv_heads == 0,
 * G = num_q_heads / num_kv_heads <= 16, D in {64, 128},
 * max_query_len <= max_context_len <= min(16 * max_blocks_per_seq, 2^22).
 * Runs on the matrix cores: a wave takes 16 / G consecutive new tokens of one
 * (sequence, kv head) times its G query heads and walks the keys its last
 * token sees.  Needs no workspace. */
int paged_attention_prefill(const pkv_layout *layout, float *out, const void *q, const void *k_pool,
                            const void *v_pool, const int32_t *d_block_tables, const int32_t *d_context_lens,
                            const int32_t *d_query_start, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_context_len,
                            float scale, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
