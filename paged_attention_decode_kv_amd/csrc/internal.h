// Internal interface between the C ABI (capi.cpp) and the gfx950 kernels
// (kernels.hip).  Not installed; the public interface is include/pagedkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Tokens one decode work item covers for one (row, head).  The plan kernel picks a
// power of two in [chunk_min, chunk_max] per call: the largest whose item count
// reaches items_per_group items per decode workgroup.  A row of context_len tokens
// is split into cdiv(context_len, chunk) chunks; rows with more than one chunk are
// merged by the combine kernel.  pkv_set_tuning can pin the chunk length.
constexpr int kMinChunkTokens = 32;
constexpr int kMaxChunkTokens = 8192;
constexpr int kDefaultChunkMin = 128;
constexpr int kDefaultChunkMax = 8192;
constexpr int kMaxChunkRatio = 64;   // chunk_max / chunk_min: the plan's 7 candidates
constexpr int kDefaultDecodeWaves = 8;
constexpr int kDefaultItemsPerGroup = 16;
constexpr int kDefaultDealStatic = 1;
constexpr int kDefaultLdsStage = 1;
constexpr int kDefaultMaxQueryGroup = 16;
constexpr int kDefaultMfma = 1;
constexpr int kDefaultGroupsPerCu = 16;   // i.e. as many as fit
// Chunks shorter than this many tokens are read by one wave alone (they end the work
// list, and the decode kernel reads them first); at most kMaxSoloTokens.  1: none.
constexpr int kDefaultSoloTokens = 512;
constexpr int kMaxSoloTokens = 1024;
// ... and only when there are at least this many of them per decode wave
constexpr int kSoloPerWave = 1;

// Slot input: tokens of one row that one workgroup of the translation pass checks.
constexpr int kTranslateTokens = 1024;

// The work-split settings (pkv_set_tuning), process-wide.  Every library call reads
// them once, as one snapshot, and derives its workspace size, its workspace carve-up,
// its plan arguments and its kernel choice from that one copy, so a concurrent
// pkv_set_tuning can change the next call but never split one call's view.
struct Tuning {
  int32_t chunk_min;
  int32_t chunk_max;
  int32_t decode_waves;
  int32_t items_per_group;
  int32_t deal_static;       // 1: whole rounds of full chunks dealt without the queue
  int32_t lds_stage;         // 1: K/V staged through LDS
  int32_t max_query_group;
  int32_t mfma;              // 1: groups of 4-16 vectors on the matrix cores
  int32_t groups_per_cu;
  int32_t solo_tokens;
};
Tuning tuning_snapshot() noexcept;
// Raw pkv_tuning values (0 keeps a field); false, changing nothing, for unsupported ones.
bool set_tuning(int chunk_min, int chunk_max, int decode_waves, int items_per_group,
                int deal, int staging, int max_query_group, int mfma, int groups_per_cu,
                int solo_tokens) noexcept;

// Partial records (float32 m, l and acc[head_dim] per chunk of a split row and query
// vector) are kept within this many bytes unless the longest chunk itself splits rows
// into more: the plan lengthens its chunk until the records fit (record_chunks below).
constexpr int64_t kPartialBudgetBytes = int64_t{16} << 20;

// The counters block at offset 0 of every workspace (kCounterBytes).  The plan kernel
// writes every field it uses at each call, so the workspace needs no clearing.
enum Counter : int {
  kCtrEntries = 0,       // work-list entries (sections A, B and C)
  kCtrTicket = 1,        // the decode kernels' queue ticket
  kCtrChunk = 2,         // chunk length P (tokens)
  kCtrLog2Chunk = 3,     // log2 P
  kCtrSectionA = 4,      // entries of full chunks
  kCtrData = 5,          // entries of sections A and B (live chunks)
  kCtrTokenRows = 6,     // slot input: rows read token by token
  kCtrGroups = 7,        // decode workgroups that take part (the rest exit at once)
  kCtrSplitRows = 8,     // rows split into more than one chunk
  kCtrTokenEntries = 9,  // slot input: entries of the rows read token by token
  kCtrWide = 10,         // entries before the single-wave items
  kCtrTokenTicket = 11,  // slot input: the token kernel's queue ticket
  kCtrTokenWide = 12,    // slot input: token entries before the short ones
  kCtrStatus = 13,       // PKV_DEVERR_* bits raised by this call's kernels
  kCtrWalked = 14,       // 64 bits (14, 15): sub-chunks the decode kernel streamed,
                         // summed over its items
  kCtrTileTokens = 16,   // tokens per sub-chunk of the decode kernel that ran
  kCtrVectorGroups = 17, // work items per entry (query-vector groups) of that kernel
  kCtrRecords = 18,      // chunk records the plan assigned to split rows
  kCtrRecordCap = 19,    // chunk records the workspace holds
  kNumCounters = 20
};
constexpr int kCounterBytes = 256;
static_assert(kNumCounters * 4 <= kCounterBytes, "counters fit their block");

// Pool geometry in elements, derived from the descriptor.
struct PoolGeom {
  int64_t num_blocks;
  int64_t blk_stride;   // elements between consecutive blocks
  int64_t tok_stride;   // elements between consecutive slots of one block (same head)
  int64_t head_stride;  // elements between consecutive KV heads (same slot)
  int32_t block_size;
  int32_t log2_bs;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t dtype;
};

struct WriteArgs {
  PoolGeom g;
  void* k_cache;
  void* v_cache;
  const void* k;
  const void* v;
  const int64_t* slot_mapping;
  int64_t num_tokens;
};

// Workspace carve-up of one pkv_paged_attention call.
struct Workspace {
  int32_t* counters;    // [kNumCounters] at offset 0 (enum Counter)
  int4* entries;        // [max_entries]: {row, chunk (-1: pad row), record (-1: the row is
                        // one chunk, its output is written directly), context_len}
  int32_t* row_ctx;     // [rows]: each row's length as the block path reads it
  int32_t* row_rec;     // [rows]: first chunk record of a split row (slot input's token
                        // rows read it; only split rows' values are meaningful)
  int32_t* irregular;   // [rows]: the rows read token by token, counters[kCtrTokenRows]
  int4* split_rows;     // [rows]: {row, length, first record, 0} of the split rows, in row
                        // order, counters[kCtrSplitRows] of them
  int2* token_entries;  // slot input only (else null): [rows * max_chunks] {row, chunk} of
                        // the rows read token by token, longest chunk first
  float* partials;      // [record_chunks][vectors per row][head_dim + 4]: m (log2 units),
                        // l, -, -, acc; chunk c of a split row is record first + c
  int64_t max_entries;
  int32_t record_chunks;
};

struct AttnArgs {
  PoolGeom g;
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t num_rows;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t ctx_limit;    // min(max_blocks * block_size, num_blocks * block_size), or with a
                        // slot input min(width, num_blocks * block_size)
  int32_t log2_chunk_min;  // the plan's chunk length range (powers of two)
  int32_t log2_chunk_max;
  int32_t target_items;    // items the plan aims for with every workgroup (launcher)
  int32_t grid_groups;     // decode workgroups launched
  int32_t narrow_groups;   // 8 waves per compute unit, or 0 when the launch already is that
  int32_t narrow_items;    // items the plan aims for with narrow_groups workgroups
  int32_t deal_static;     // 1: whole rounds of full chunks are dealt without the queue
  int32_t query_group;     // query vectors per work item (they share one KV head)
  int32_t query_len;       // new tokens (queries) per row: 1 for decode
  int32_t solo_tokens;     // chunks shorter than this are read one wave each (0, 1: none)
  int32_t group_waves;     // waves per decode workgroup
  float scale;
  // slot input only (else null / 0): [rows][flag_stride], nonzero where a row's live
  // slots are not block structured; such rows are left to the token-by-token kernel
  const int32_t* row_flags;
  int32_t flag_stride;
  int32_t token_waves;   // slot input only: waves of the token kernels' grid
  int32_t record_chunks; // chunk records the workspace holds: the plan lengthens its chunk
                         // until the split rows' chunks fit
};

// The slot rectangle of a read addressed per token, and what the translation pass
// derives from it.
struct SlotArgs {
  const int64_t* slots;    // [rows][row_stride]; cell (r, t) is the slot of position t
  int64_t row_stride;      // elements, >= width
  int32_t width;
  int32_t max_blocks;      // cdiv(width, block_size): width of the derived block table
  int32_t flag_stride;     // cdiv(width, kTranslateTokens)
  int32_t* block_tables;   // out: [rows][max_blocks] derived block ids (live blocks only)
  int32_t* row_flags;      // out: [rows][flag_stride]
};

// Sizes and carve-ups follow one tuning snapshot; `vectors` is query vectors per row
// (query_len x heads).
int32_t record_chunks_for(int64_t num_rows, int32_t vectors, int32_t head_dim,
                          int32_t max_blocks, int32_t block_size, const Tuning& t);
size_t workspace_bytes(int64_t num_rows, int32_t vectors, int32_t head_dim,
                       int32_t max_blocks, int32_t block_size, const Tuning& t);
Workspace carve_workspace(void* base, int64_t num_rows, int32_t vectors, int32_t head_dim,
                          int32_t max_blocks, int32_t block_size, const Tuning& t);

// Slot input: the block-path workspace, then the derived table, flags and token entries.
size_t slot_workspace_bytes(int64_t num_rows, int32_t num_heads, int32_t head_dim,
                            int32_t width, int32_t block_size, const Tuning& t);
Workspace carve_slot_workspace(void* base, int64_t num_rows, int32_t num_heads,
                               int32_t head_dim, int32_t width, int32_t block_size,
                               const Tuning& t, SlotArgs* s);

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream);
// combine = false leaves split rows' partials for a later launch_combine (slot input);
// `write`, if given, is the step's slot scatter, run inside the plan kernel's launch
// (a captured step)
hipError_t launch_paged_attention(const AttnArgs& a, const Workspace& ws, const Tuning& t,
                                  hipStream_t stream, bool combine = true,
                                  const WriteArgs* write = nullptr);
hipError_t launch_paged_attention_slots(const AttnArgs& a, const SlotArgs& s,
                                        const Workspace& ws, const Tuning& t,
                                        hipStream_t stream);
hipError_t read_device_status(uint32_t* flags, int clear, hipStream_t stream);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                              int groups_per_cu, hipStream_t stream);
hipError_t launch_gather_read(const void* k_base, const void* v_base, const int64_t* offsets,
                              int64_t n_pieces, int32_t piece_bytes, uint32_t* sink,
                              int groups_per_cu, int waves_per_group, int pieces_per_wave,
                              hipStream_t stream);
// compute units of the current device (looked up once per device)
hipError_t device_cus(int* cus);

// The library's own workspace for callers that cannot allocate
// (pkv_paged_attention_noalloc): a static device array of kScratchBytes on every
// device the library runs on.  scratch_pointer gives the current device's copy: its
// device address, looked up once per device with hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t{32} << 20;
hipError_t scratch_pointer(void** ptr);
// which decode kernel (and query-vector group) a read of this shape runs under tuning t
// (uses a.g, a.num_heads, a.query_len)
const char* decode_kernel_name(const AttnArgs& a, const Tuning& t);

// Event-pair timing of kernel phases (pkv_timing_*).  begin/end bracket one launch.
void timing_begin(int phase, hipStream_t stream);
void timing_end(int phase, hipStream_t stream);
void timing_enable(bool on);
// While a TimingPause lives, this thread's launches record no events (a call that
// must not create any).
struct TimingPause {
  TimingPause();
  ~TimingPause();
};
hipError_t timing_read(int phase, double* total_ms, int64_t* launches, bool reset);

}  // namespace pkv
