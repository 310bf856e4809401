/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) batched paged-attention decode step.
 *
 * One decode step of a paged KV cache, as the nanoserve pages describe it:
 *
 *   1. pkv_kv_write: every running row's new K/V vector is scattered into its
 *      pool slot; a padding row aims at the sink slot, a legal address past every
 *      slot the allocator hands out (Day 55, "the capture list moved to startup,
 *      and the dummy batch was all padding", section "Why it matters").
 *   2. pkv_paged_attention: for every (row, query head) the row's history is read
 *      through its block table, block id times block size plus offset (Day 51,
 *      "the read rectangle stopped being built ...", section "Why it matters"),
 *      in cdiv(context_len, block) tiles folded into an online softmax (Day 59,
 *      "the rectangle the read builds, and the tile that replaces it", sections
 *      "What I added today" and "What I learned" 3-4).  The result equals the
 *      masked [rows, heads, 1, max_ctx] softmax rectangle of the reference read
 *      (same page, "What I added today").  A row whose context_len is 0 is a
 *      padding row: its output is zero and no K/V, block-table entry or pool slot
 *      of it is read.
 *
 * Conventions for every call:
 *   - Pointers named k_cache, v_cache, k, v, q, out, slot_mapping, block_tables,
 *     context_lens and workspace are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or keeps them.  The host-check entry points
 *     (pkv_check_*_host) take HOST pointers instead.
 *   - All arrays are dense, row-major, with no padding between rows.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.  Calls
 *     are asynchronous on that stream unless `validate` is non-zero.
 *   - Every entry point returns a pkv_status.  On a refusal nothing is launched
 *     and no memory is touched; pkv_last_error_detail() names the offending row,
 *     entry or argument (thread-local, valid until the next call on the thread).
 *   - Device-side safety: with validate == 0 the kernels still never read or write
 *     outside the pool: a context_len is clamped to [0, max_blocks_per_row *
 *     block_size], a live block id outside [0, num_blocks) is skipped and a write
 *     slot outside [0, sink] is skipped.  Such inputs give unspecified output values
 *     (not a fault) and raise a bit in the call's own status word, kept in its
 *     workspace (pkv_workspace_status), and in the device-wide word
 *     (pkv_device_status).
 *   - Tuning: every call reads the process-wide work split (pkv_set_tuning) once and
 *     sizes, checks and launches everything from that one copy; a concurrent
 *     pkv_set_tuning affects later calls only.  A workspace sized under one tuning can
 *     be too small under another: the call then refuses with WORKSPACE.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 4

/* Element type of q, out, the new K/V and both pools. */
typedef enum pkv_dtype {
  PKV_F32 = 0,   /* IEEE binary32 */
  PKV_BF16 = 1   /* bfloat16; accumulation is float32 */
} pkv_dtype;

/* Order of the axes of one pool block.  Both describe the same slot-indexed pool
 * [slots, kv_heads, head_dim] with slot = block * block_size + offset.
 *   HND: [num_blocks + 1][num_kv_heads][block_size][head_dim]
 *        (one block of one KV head is block_size * head_dim contiguous elements)
 *   NHD: [num_blocks + 1][block_size][num_kv_heads][head_dim]
 *        (one slot of all KV heads is num_kv_heads * head_dim contiguous elements) */
typedef enum pkv_layout {
  PKV_LAYOUT_HND = 0,
  PKV_LAYOUT_NHD = 1
} pkv_layout;

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_EMPTY = 1,          /* zero rows, or zero tokens to write */
  PKV_ERR_DTYPE = 2,          /* unknown dtype code */
  PKV_ERR_SHAPE = 3,          /* inconsistent dimensions (e.g. heads % kv_heads != 0) */
  PKV_ERR_CONTEXT_BOUNDS = 4, /* a context_len < 0, > max_blocks_per_row*block_size,
                                 or > num_blocks*block_size */
  PKV_ERR_BLOCK_ID = 5,       /* a live block-table entry outside [0, num_blocks) */
  PKV_ERR_SLOT = 6,           /* a slot_mapping entry outside [0, sink] */
  PKV_ERR_UNSUPPORTED = 7,    /* legal, but not a shape this library was built for */
  PKV_ERR_WORKSPACE = 8,      /* workspace missing or smaller than pkv_workspace_bytes */
  PKV_ERR_NULL = 9,           /* a required pointer is NULL */
  PKV_ERR_HIP = 10            /* the HIP runtime reported an error, or host memory to
                                 validate with could not be allocated (out of memory) */
} pkv_status;

/* The pool both caches share.  num_blocks counts the blocks a block table may name;
 * storage holds one more block, whose first slot is the sink. */
typedef struct pkv_pool_desc {
  int64_t num_blocks;    /* NB >= 1 */
  int32_t block_size;    /* BS: 16, 32, 64, 128 or 256 */
  int32_t num_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;      /* D: 64, 128 or 256 */
  int32_t dtype;         /* pkv_dtype */
  int32_t layout;        /* pkv_layout */
} pkv_pool_desc;

/* Device status bits raised by kernels run with validate == 0 on bad inputs. */
#define PKV_DEVERR_SLOT 1u            /* a write slot outside [0, sink], or a live read
                                         slot outside [0, sink), was skipped */
#define PKV_DEVERR_CONTEXT_BOUNDS 2u  /* a context_len was clamped */
#define PKV_DEVERR_BLOCK_ID 4u        /* a live block id outside [0, num_blocks) was skipped */

int32_t pkv_abi_version(void);
const char* pkv_status_str(pkv_status status);
const char* pkv_last_error_detail(void);

/* The sink slot, num_blocks * block_size (Day 55, "Why it matters": one past the
 * pool the allocator hands out).  Returns -1 for an invalid descriptor. */
int64_t pkv_sink_slot(const pkv_pool_desc* pool);

/* Elements of one pool (K or V): (num_blocks + 1) * block_size * num_kv_heads * head_dim.
 * Returns -1 for an invalid descriptor. */
int64_t pkv_pool_elements(const pkv_pool_desc* pool);

/* Checks a descriptor: DTYPE, SHAPE or UNSUPPORTED, else OK. */
pkv_status pkv_check_pool(const pkv_pool_desc* pool);

/* Host-side refusal checks on HOST arrays, in the order EMPTY, DTYPE, SHAPE, SLOT
 * (write) and EMPTY, DTYPE, SHAPE, CONTEXT_BOUNDS, BLOCK_ID (attention).  The first
 * offending entry is reported.  Entries of a table row past its live prefix
 * cdiv(context_len, block_size) are never checked (they may hold -1).  These are the
 * checks validate != 0 runs; they launch nothing and need no GPU. */
pkv_status pkv_check_write_host(const pkv_pool_desc* pool, const int64_t* slot_mapping,
                                int64_t num_tokens);
pkv_status pkv_check_attention_host(const pkv_pool_desc* pool, const int32_t* block_tables,
                                    int32_t max_blocks_per_row, const int32_t* context_lens,
                                    int64_t num_rows, int32_t num_heads);

/* The slot scatter (Day 55, "Why it matters": the padded batch is written with one
 * indexed assignment, pad rows into the sink).
 *   k, v          [num_tokens][num_kv_heads][head_dim], pool dtype
 *   slot_mapping  [num_tokens] int64, each in [0, sink]
 *   k_cache, v_cache  pools in the descriptor's layout, updated in place
 * Token i's vectors are copied bit-exactly into slot slot_mapping[i].  Distinct tokens
 * must name distinct slots, except that any number may name the sink (its contents
 * afterwards are one of those tokens' vectors).
 * validate != 0 copies slot_mapping to the host first (synchronising `stream`) and
 * refuses bad slots before launching. */
pkv_status pkv_kv_write(const pkv_pool_desc* pool, void* k_cache, void* v_cache,
                        const void* k, const void* v, const int64_t* slot_mapping,
                        int64_t num_tokens, int32_t validate, void* stream);

/* Device workspace bytes pkv_paged_attention needs for this batch shape under the
 * current tuning (0 for a shape the call would refuse).  Depends on the arguments and
 * the tuning's chunk range, never on the lengths.  Layout: a 256-byte counters block
 * at offset 0 (pkv_plan_info_read), the work list, and float32 partial records of the
 * rows split into several chunks, at most 16 MiB of them unless the longest chunk
 * itself splits rows into more. */
size_t pkv_workspace_bytes(const pkv_pool_desc* pool, int64_t num_rows, int32_t num_heads,
                           int32_t max_blocks_per_row);

/* The batched decode read (Day 59, "What I added today").
 *   q, out        [num_rows][num_heads][head_dim], pool dtype; query head h reads KV
 *                 head h / (num_heads / num_kv_heads)
 *   block_tables  [num_rows][max_blocks_per_row] int32; entry j of row r names the
 *                 pool block holding positions j*block_size .. j*block_size+block_size-1
 *   context_lens  [num_rows] int32; 0 marks a padding row (output zero, nothing read)
 *   scale         multiplies q.k before the softmax
 *   workspace     device scratch of at least pkv_workspace_bytes(...) bytes, owned by
 *                 the caller; its contents on entry do not matter.  On return it holds
 *                 the call's plan and status (pkv_plan_info_read, pkv_workspace_status)
 *                 until the next call that uses it.  Two calls in flight at once need
 *                 two workspaces.
 * out[r,h,:] = sum_t softmax_t(scale * q[r,h,:].K[t]) V[t] over t < context_lens[r],
 * accumulated in float32, rounded once to the pool dtype.
 * validate != 0 copies context_lens and block_tables to the host first (synchronising
 * `stream`) and refuses bad lengths and block ids before launching. */
pkv_status pkv_paged_attention(const pkv_pool_desc* pool, void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_row,
                               const int32_t* context_lens, int64_t num_rows,
                               int32_t num_heads, float scale, void* workspace,
                               size_t workspace_bytes, int32_t validate, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): pkv_paged_attention with the
 * library's own workspace, a static device array of PKV_NOALLOC_SCRATCH_BYTES on each
 * device (held from the library's load until the process ends).  The caller passes
 * the inputs and `out` as for pkv_paged_attention; the call allocates nothing, runs
 * no host checks and copies nothing to the host (validate = 0 semantics: bad lengths
 * are clamped, bad block ids skipped, each raising its bit in the device-wide status
 * word, pkv_device_status), and records no timing events.
 * Refuses (before touching anything) what pkv_paged_attention refuses from the shape,
 * and with WORKSPACE a batch whose pkv_workspace_bytes exceeds the scratch.  Every
 * call on a device shares that device's scratch: calls that overlap on one device
 * (two streams, two host threads) race and give undefined results.  The scratch keeps
 * the last call's work list; each call rewrites everything it reads. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pkv_status pkv_paged_attention_noalloc(const pkv_pool_desc* pool, void* out, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables,
                                       int32_t max_blocks_per_row,
                                       const int32_t* context_lens, int64_t num_rows,
                                       int32_t num_heads, float scale, void* stream);

/* The read with several new tokens (queries) per row: speculative decoding's draft
 * tokens, or a chunk of a prompt, over the same paged history (Day 59, "Why it
 * matters": the read's rectangle has a query_len axis beside rows and heads).
 *   q, out        [num_rows][query_len][num_heads][head_dim], pool dtype
 *   query_len     1..64 new tokens per row; query i of row r is the token at position
 *                 context_lens[r] - query_len + i (its K/V written by pkv_kv_write with
 *                 num_rows * query_len tokens before this call)
 *   context_lens  [num_rows] int32: 0 (a padding row, all outputs zero) or in
 *                 [query_len, min(max_blocks * block_size, num_blocks * block_size)]
 *   block_tables, scale, workspace, validate, stream: as in pkv_paged_attention; the
 *                 workspace is pkv_workspace_bytes_multi(...)
 * out[r,i,h,:] = sum_t softmax_t(scale * q[r,i,h,:].K[t]) V[t] over
 * t <= context_lens[r] - query_len + i (causal), accumulated in float32.  One K/V read
 * serves up to 8 query vectors (new tokens x query heads of one KV head).  Refusals:
 * those of pkv_paged_attention, in its order, with CONTEXT_BOUNDS also for a live row
 * shorter than query_len (after the range check, before BLOCK_ID); SHAPE for
 * query_len < 1, UNSUPPORTED above 64.  query_len = 1 is pkv_paged_attention. */
size_t pkv_workspace_bytes_multi(const pkv_pool_desc* pool, int64_t num_rows,
                                 int32_t query_len, int32_t num_heads,
                                 int32_t max_blocks_per_row);
pkv_status pkv_paged_attention_multi(const pkv_pool_desc* pool, void* out, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_row,
                                     const int32_t* context_lens, int64_t num_rows,
                                     int32_t query_len, int32_t num_heads, float scale,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t validate, void* stream);
/* The host checks pkv_paged_attention_multi runs with validate != 0, on HOST arrays. */
pkv_status pkv_check_attention_multi_host(const pkv_pool_desc* pool,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_row,
                                          const int32_t* context_lens, int64_t num_rows,
                                          int32_t query_len, int32_t num_heads);

/* The decode read addressed by a per-token slot rectangle instead of block tables
 * (Day 51, "What I added today": the step reads through a persistent
 * [max_batch, max_model_len] int64 slot table, handed over as the window
 * slots[:rows, :width] with the lengths beside it).
 *   slot_table     int64; cell (r, t) at slot_table[r * row_stride + t] is the slot
 *                  holding position t of row r.  row_stride >= width, so a window on a
 *                  wider table is passed as its first cell's address and the table's
 *                  row length.  Cells at or past context_lens[r] may hold anything
 *                  (a re-tenanted row keeps its old slots there) and are never read.
 *   context_lens   [num_rows] int32, each in [0, min(width, num_blocks * block_size)]
 *   q, out, k_cache, v_cache, scale, workspace, validate, stream: as in
 *                  pkv_paged_attention; the workspace is pkv_workspace_bytes_slots(...)
 * Refusals, in order: EMPTY, DTYPE, SHAPE (row_stride < width, width < 1, heads),
 * CONTEXT_BOUNDS, SLOT (a live cell outside [0, num_blocks * block_size): the sink is
 * no row's token), UNSUPPORTED (width > 2^24, rows > 65535).  validate != 0 copies
 * the lengths and the rectangle's first `width` columns to the host first.
 * out is the same function of the named tokens as pkv_paged_attention's.  Rows whose
 * live cells are block structured (cell t = B * block_size + t % block_size over each
 * block of positions, B an allocatable block) take the block-table kernels, bit for
 * bit what pkv_paged_attention gives with those blocks; other rows are read token by
 * token.  With validate = 0 a live cell outside the slots is skipped and sets
 * PKV_DEVERR_SLOT. */
size_t pkv_workspace_bytes_slots(const pkv_pool_desc* pool, int64_t num_rows,
                                 int32_t num_heads, int32_t width);
pkv_status pkv_paged_attention_slots(const pkv_pool_desc* pool, void* out, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int64_t* slot_table, int32_t width,
                                     int64_t row_stride, const int32_t* context_lens,
                                     int64_t num_rows, int32_t num_heads, float scale,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t validate, void* stream);
/* The host checks pkv_paged_attention_slots runs with validate != 0, on HOST arrays. */
pkv_status pkv_check_attention_slots_host(const pkv_pool_desc* pool,
                                          const int64_t* slot_table, int32_t width,
                                          int64_t row_stride, const int32_t* context_lens,
                                          int64_t num_rows, int32_t num_heads);

/* Which decode kernel a read with this pool, query heads and new tokens per row runs,
 * under the current tuning, as text ("decode_kernel, 1 query vector per item",
 * "decode_mfma_kernel, 8 query vectors per item", ...).  A static string; "" for a
 * shape the library refuses.  For benchmarks and profiles. */
const char* pkv_decode_kernel_for(const pkv_pool_desc* pool, int32_t num_heads,
                                  int32_t query_len);

/* Reads (and if `clear` is non-zero, resets) the current device's status word, a
 * bitwise OR of PKV_DEVERR_* raised since the last clear by every call on the device,
 * from any thread (pkv_kv_write reports its skipped slots here only).  Synchronises
 * `stream`.  A clear races with concurrent calls; for one attention call's own bits
 * use pkv_workspace_status. */
pkv_status pkv_device_status(uint32_t* flags, int32_t clear, void* stream);

/* The PKV_DEVERR_* bits raised by the kernels of the last attention call
 * (pkv_paged_attention, _multi, _slots, or a captured step's read) that used this
 * workspace, and by no other call: the call's plan kernel starts the word afresh.
 * workspace_bytes must cover the 256-byte counters block.  Synchronises `stream`,
 * which must be ordered after that call. */
pkv_status pkv_workspace_status(const void* workspace, size_t workspace_bytes,
                                uint32_t* flags, void* stream);

/* What the last attention call that used a workspace did, read back from the
 * counters at the workspace's start: the plan's choices and the decode kernel's own
 * count of the tiles it streamed (Day 59, "What I learned" 5: the host's count of
 * walked tiles and the kernel's loop are held to the same lengths).  For tests and
 * profiling.  Synchronises `stream`, which must be ordered after that call. */
typedef struct pkv_plan_info {
  int32_t chunk_tokens;     /* P: tokens per work-list chunk, chosen on the device */
  int32_t entries;          /* work-list entries: live chunks + one per padding row */
  int32_t full_chunks;      /* entries of chunks of exactly P tokens */
  int32_t live_entries;     /* entries of live chunks: sum over rows of cdiv(len, P) */
  int32_t wide_entries;     /* live entries read by a whole workgroup; the rest (chunks
                               shorter than solo_tokens) were read by one wave each */
  int32_t split_rows;       /* rows longer than P, merged over their chunks */
  int32_t records;          /* their chunks: one float32 partial record per vector */
  int32_t record_capacity;  /* chunk records the workspace holds */
  int32_t decode_groups;    /* decode workgroups that took part */
  int32_t vector_groups;    /* work items per entry: query-vector groups of a row */
  int32_t tile_tokens;      /* tokens per sub-chunk (tile) of the decode kernel that ran */
  int32_t token_rows;       /* slot input: rows read token by token */
  int64_t tiles_walked;     /* tiles the decode kernel streamed, summed over its items:
                               vector_groups x sum over block-path rows of
                               cdiv(len, tile_tokens) when every item ran once */
  int32_t token_entries;    /* slot input: the chunk entries of the token rows */
  uint32_t status;          /* PKV_DEVERR_* bits of the call (pkv_workspace_status) */
} pkv_plan_info;
pkv_status pkv_plan_info_read(const void* workspace, size_t workspace_bytes,
                              pkv_plan_info* info, void* stream);

/* A plain streaming read of `bytes` bytes at device address `src`, with the decode
 * kernels' 16-byte non-temporal loads, by groups_per_cu (1..16) workgroups of 256
 * threads per compute unit, each reading 32 KB runs dealt round robin.  For
 * benchmarks: the rate a kernel that does nothing but read reaches on this GPU, the
 * achievable reference beside the decode kernel's rate.  `sink` is a 4-byte device
 * word that is written only if the bytes read fold to one particular value (so no load
 * can be skipped).  bytes: a positive multiple of 16.  Asynchronous on `stream`. */
pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink,
                           int32_t groups_per_cu, void* stream);

/* The same loads over scattered pieces: piece i is piece_bytes bytes (a multiple of 16,
 * at most 1 MiB) at byte offset offsets[i] of both k_base and v_base (device addresses;
 * `offsets` is a device array of n_pieces int64).  groups_per_cu (1..16) workgroups of
 * waves_per_group (4 or 8) waves per compute unit; each wave reads pieces_per_wave (1, 2
 * or 4) pieces at a time, every (waves in the grid)-th piece of the list, so that the
 * grid reads one contiguous window of the list at a time.  With the offsets of the
 * (block, KV head) pieces a decode read streams, in its order, it is the rate a kernel
 * that only reads reaches on that access pattern; benchmarks take the best over these
 * shapes.  Pieces of at most 1 KB that divide 1 KB (a token's head vector in a
 * slot-major pool, or a token read through a slot window) are read by lane groups, 1024 /
 * piece_bytes pieces a wave load; larger pieces one wave each, 4 KB of each piece and
 * pool a pass.  Each piece's bytes must lie inside both allocations: the library cannot
 * check device offsets, so the caller does.  Refused (PKV_ERR_SHAPE) for other shapes.
 * Asynchronous on `stream`. */
pkv_status pkv_gather_read(const void* k_base, const void* v_base, const int64_t* offsets,
                           int64_t n_pieces, int32_t piece_bytes, uint32_t* sink,
                           int32_t groups_per_cu, int32_t waves_per_group,
                           int32_t pieces_per_wave, void* stream);

/* Work split of the decode read (process-wide).  Each call cuts every row's history
 * into chunks; one (chunk, query head) is a work item of the persistent decode kernel,
 * shared by the waves of one workgroup, and rows longer than one chunk are merged
 * afterwards in chunk order.  The chunk length is chosen on the device per call: the
 * largest power of two in [chunk_min, chunk_max] that still yields items_per_group
 * items per decode workgroup (for chunks shorter than solo_tokens, one item per wave),
 * and whose chunk holds at most a third of a workgroup's share of the batch (else the
 * largest that yields a quarter of that, else chunk_min); then the next longer one
 * while the split rows' partial records would not fit the workspace.  Setting
 * chunk_min == chunk_max pins it.
 *   chunk_min, chunk_max  powers of two in [32, 8192], chunk_max/chunk_min <= 64
 *                         (defaults 128, 8192)
 *   decode_waves          64-lane waves per workgroup: 1, 2, 4 or 8 (default 8)
 *   items_per_group       default 16 (the matrix-core fold, whose items carry 8 or 16
 *                         query vectors, aims for a quarter of it)
 *   deal                  1: whole rounds of full-length chunks are dealt to workgroups
 *                         round robin and only the rest goes through the shared work
 *                         queue; 2: every item goes through the queue (default 1)
 *   staging               1: each wave loads a sub-chunk's K/V straight into registers;
 *                         2: each wave streams its next sub-chunk into an LDS stage by
 *                         direct buffer-to-LDS loads while folding the current one
 *                         (default 2)
 *   max_query_group       1, 2, 4, 8 or 16 (default 16).  A row has query_len x heads
 *                         query vectors, and those of one KV head (query_len x
 *                         num_heads / num_kv_heads of them) can share each K/V load: one
 *                         work item covers QG of them, QG the largest power of two that
 *                         divides that count and is at most max_query_group (at most 8 on
 *                         the vector units, 4 at head_dim 256); 1 reads K/V once per
 *                         vector
 *   mfma                  1: a group of 4, 8 or 16 vectors on a bfloat16 pool of
 *                         head_dim 64 or 128 is folded on the matrix cores (default);
 *                         2: always on the vector units
 *   groups_per_cu         at most this many decode workgroups per compute unit, 1..16
 *                         (default 16: as many as fit)
 *   solo_tokens           chunks of fewer than this many tokens are read first, by one
 *                         wave each, with no merge across the waves of a workgroup,
 *                         when there is at least one such chunk per decode wave: a power
 *                         of two in [32, 1024], or 1 for none (default 512)
 * A field of 0 leaves that value unchanged.  chunk_min and chunk_max set
 * pkv_workspace_bytes: set them before sizing workspaces.  Results do not depend on
 * these values beyond float32 rounding order.  Returns UNSUPPORTED for other values,
 * changing nothing.  Safe to call while other threads run calls (each call uses the
 * values in force when it starts). */
typedef struct pkv_tuning {
  int32_t chunk_min;
  int32_t chunk_max;
  int32_t decode_waves;
  int32_t items_per_group;
  int32_t deal;
  int32_t staging;
  int32_t max_query_group;
  int32_t mfma;
  int32_t groups_per_cu;
  int32_t solo_tokens;
} pkv_tuning;

pkv_status pkv_set_tuning(const pkv_tuning* tuning);
pkv_status pkv_get_tuning(pkv_tuning* tuning);

/* Kernel timing, for benchmarks and profiling.  While enabled, every launch of the
 * phases below is bracketed by a pair of HIP events recorded on the launch stream;
 * pkv_timing_read synchronises on the recorded events and returns the summed elapsed
 * milliseconds and the number of launches of one phase.  Disabled by default; costs
 * two event records per launch when on (~10 us of device idle at each kernel boundary).
 * On this runtime the device also runs slower for a few milliseconds after hundreds of
 * event pairs: time steps before a timed loop, not after it.  Not thread-safe against
 * concurrent calls. */
typedef enum pkv_phase {
  PKV_PHASE_KV_WRITE = 0,  /* the slot scatter kernel */
  PKV_PHASE_PLAN = 1,      /* the work-list kernel of pkv_paged_attention */
  PKV_PHASE_DECODE = 2,    /* the streaming online-softmax kernel */
  PKV_PHASE_COMBINE = 3,   /* the merge of split rows */
  PKV_PHASE_TRANSLATE = 4, /* slot input: the rectangle's block-structure check */
  PKV_PHASE_TOKEN_ROWS = 5 /* slot input: the rows read token by token */
} pkv_phase;

pkv_status pkv_timing_enable(int32_t on);
pkv_status pkv_timing_read(int32_t phase, double* total_ms, int64_t* launches, int32_t reset);

/* A captured decode step: kv_write followed by paged_attention, recorded once into a
 * HIP graph over fixed buffers and replayed for every later step whose inputs are
 * written into those same buffers (Day 55, "Why it matters": a recording made over an
 * all-padding batch computes real steps because every argument it keeps is storage
 * that each step writes through).
 *   Arguments are those of pkv_kv_write and pkv_paged_attention for one decode step,
 *   one new token per row: k, v [num_rows][num_kv_heads][head_dim], slot_mapping
 *   [num_rows] int64.  Every pointer is kept by the graph and must stay valid, at the
 *   same address, until pkv_graph_destroy; the workspace too.  Nothing is read or run
 *   while capturing, so the buffers may hold anything then.
 *   Each launch reads the buffers' contents at that moment, with validate = 0
 *   semantics: no host checks; bad lengths are clamped, bad block ids and slots
 *   skipped, and each raises its bit in the device status word.  A padding row
 *   (context_lens 0, slot_mapping the sink) reads nothing and writes only the sink.
 *   The tuning in force at capture time is frozen into the graph.  The recorded step
 *   runs the slot scatter inside the work-list kernel's launch (neither reads what the
 *   other writes), so a replay is one kernel shorter than the two calls.
 * Capture uses a private stream and needs no synchronisation of the caller's streams.
 * pkv_graph_launch enqueues one replay on `stream`, which must belong to the device that
 * was current at capture; replays of graphs sharing buffers must be ordered (one
 * stream).  pkv_graph_destroy(NULL) is a no-op.  Capture fails with the same refusals
 * as the two calls' shape checks, or HIP if the runtime refuses the capture. */
typedef struct pkv_step_graph pkv_step_graph;

pkv_status pkv_graph_capture(const pkv_pool_desc* pool, void* k_cache, void* v_cache,
                             const void* k, const void* v, const int64_t* slot_mapping,
                             void* out, const void* q, const int32_t* block_tables,
                             int32_t max_blocks_per_row, const int32_t* context_lens,
                             int64_t num_rows, int32_t num_heads, float scale,
                             void* workspace, size_t workspace_bytes,
                             pkv_step_graph** graph);
/* The same, with the read addressed by a slot window (pkv_paged_attention_slots's
 * arguments): the pages record their graphs over windows on the slot table. */
pkv_status pkv_graph_capture_slots(const pkv_pool_desc* pool, void* k_cache, void* v_cache,
                                   const void* k, const void* v, const int64_t* slot_mapping,
                                   void* out, const void* q, const int64_t* slot_table,
                                   int32_t width, int64_t row_stride,
                                   const int32_t* context_lens, int64_t num_rows,
                                   int32_t num_heads, float scale, void* workspace,
                                   size_t workspace_bytes, pkv_step_graph** graph);
pkv_status pkv_graph_launch(const pkv_step_graph* graph, void* stream);
pkv_status pkv_graph_destroy(pkv_step_graph* graph);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
