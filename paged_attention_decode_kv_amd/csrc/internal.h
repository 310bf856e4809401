// Internal interface between the C ABI (capi.cpp) and the gfx950 kernels
// (kernels.hip).  Not installed; the public interface is include/pagedkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Tokens one decode work item covers for one (row, head): a power of two in
// [kMinChunkTokens, kMaxChunkTokens], kDefaultChunkTokens unless retuned with
// pkv_set_tuning.  A row of context_len tokens is split into
// cdiv(context_len, chunk_tokens) chunks; rows with more than one chunk are merged
// by the combine kernel.
constexpr int kMinChunkTokens = 32;
constexpr int kMaxChunkTokens = 1024;
constexpr int kDefaultChunkTokens = 256;
constexpr int kDefaultDecodeWaves = 4;

int tuning_chunk_tokens();
int tuning_decode_waves();
bool set_tuning(int chunk_tokens, int decode_waves);

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
  int4* entries;        // [max_entries]: {row, chunk (-1: pad row), chunks in row, context_len}
  int32_t* counters;    // [0] entries written by the plan, [1] queue ticket
  float* partials;      // [rows][heads][max_chunks][head_dim + 2]: m (log2 units), l, acc
  int64_t max_entries;
  int32_t max_chunks;
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
  int32_t ctx_limit;    // min(max_blocks * block_size, num_blocks * block_size)
  int32_t chunk_tokens; // tokens per work item
  int32_t log2_chunk;
  float scale;
};

size_t workspace_bytes(int64_t num_rows, int32_t num_heads, int32_t head_dim,
                       int32_t max_blocks, int32_t block_size);
Workspace carve_workspace(void* base, int64_t num_rows, int32_t num_heads,
                          int32_t head_dim, int32_t max_blocks, int32_t block_size);

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream);
hipError_t launch_paged_attention(const AttnArgs& a, const Workspace& ws, hipStream_t stream);
hipError_t read_device_status(uint32_t* flags, int clear, hipStream_t stream);

// Event-pair timing of kernel phases (pkv_timing_*).  begin/end bracket one launch.
void timing_begin(int phase, hipStream_t stream);
void timing_end(int phase, hipStream_t stream);
void timing_enable(bool on);
hipError_t timing_read(int phase, double* total_ms, int64_t* launches, bool reset);

}  // namespace pkv
