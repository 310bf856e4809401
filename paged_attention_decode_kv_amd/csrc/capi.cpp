// C ABI of the decode step: argument checks, host-side refusals, workspace sizing
// and the launches.  The kernels themselves are in kernels.hip.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <new>
#include <vector>

#include "internal.h"
#include "pagedkv.h"

struct pkv_step_graph {
  hipGraphExec_t exec;
};

namespace {

// the calling thread's last refusal, in a fixed buffer (nothing here allocates)
thread_local char g_detail[512];

pkv_status fail(pkv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return s;
}

pkv_status ok() {
  g_detail[0] = '\0';
  return PKV_OK;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int n = 0;
  while ((int64_t{1} << n) < x) ++n;
  return n;
}

// Descriptor checks shared by every call: DTYPE, then SHAPE, then UNSUPPORTED.
pkv_status check_pool(const pkv_pool_desc* p) {
  if (!p) return fail(PKV_ERR_NULL, "pool descriptor is NULL");
  if (p->dtype != PKV_F32 && p->dtype != PKV_BF16)
    return fail(PKV_ERR_DTYPE, "unknown dtype code %d", p->dtype);
  if (p->num_blocks < 1 || p->num_blocks > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "num_blocks %lld outside [1, 2^31)", (long long)p->num_blocks);
  if (p->block_size < 1 || p->num_kv_heads < 1 || p->head_dim < 1)
    return fail(PKV_ERR_SHAPE, "block_size, num_kv_heads and head_dim must be positive");
  if (p->layout != PKV_LAYOUT_HND && p->layout != PKV_LAYOUT_NHD)
    return fail(PKV_ERR_SHAPE, "unknown layout code %d", p->layout);
  if (!is_pow2(p->block_size) || p->block_size < 16 || p->block_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d: built for powers of two in [16, 256]",
                p->block_size);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: built for 64, 128 and 256", p->head_dim);
  return PKV_OK;
}

pkv::PoolGeom geom(const pkv_pool_desc* p) {
  pkv::PoolGeom g;
  g.num_blocks = p->num_blocks;
  g.block_size = p->block_size;
  g.log2_bs = log2i(p->block_size);
  g.kv_heads = p->num_kv_heads;
  g.head_dim = p->head_dim;
  g.dtype = p->dtype;
  const int64_t bs = p->block_size, hkv = p->num_kv_heads, d = p->head_dim;
  g.blk_stride = bs * hkv * d;
  if (p->layout == PKV_LAYOUT_HND) {
    g.head_stride = bs * d;
    g.tok_stride = d;
  } else {
    g.head_stride = d;
    g.tok_stride = hkv * d;
  }
  return g;
}

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A host buffer of a validating call.  An allocation failure is returned as a status,
// since no exception may cross the C ABI.
template <typename T>
bool host_buffer(std::vector<T>& v, size_t n) {
  try {
    v.resize(n);
    return true;
  } catch (const std::exception&) {
    return false;
  }
}

int64_t ctx_limit_of(const pkv_pool_desc* p, int32_t max_blocks) {
  const int64_t by_table = (int64_t)max_blocks * p->block_size;
  const int64_t by_pool = p->num_blocks * p->block_size;
  return by_table < by_pool ? by_table : by_pool;
}

// Attention shape checks that need no data: EMPTY, pool, SHAPE, UNSUPPORTED.
pkv_status check_attention_shape(const pkv_pool_desc* pool, int32_t max_blocks,
                                 int64_t num_rows, int32_t num_heads) {
  if (num_rows == 0) return fail(PKV_ERR_EMPTY, "no rows");
  pkv_status s = check_pool(pool);
  if (s != PKV_OK) return s;
  if (num_rows < 0) return fail(PKV_ERR_SHAPE, "num_rows %lld < 0", (long long)num_rows);
  if (num_heads < 1 || num_heads % pool->num_kv_heads != 0)
    return fail(PKV_ERR_SHAPE, "%d query heads is not a positive multiple of %d KV heads",
                num_heads, pool->num_kv_heads);
  if (max_blocks < 1) return fail(PKV_ERR_SHAPE, "max_blocks_per_row %d < 1", max_blocks);
  if (num_rows > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "num_rows %lld: built for at most 65535 rows",
                (long long)num_rows);
  if ((int64_t)max_blocks * pool->block_size > (int64_t{1} << 24))
    return fail(PKV_ERR_UNSUPPORTED, "table width %lld tokens: built for at most 2^24",
                (long long)max_blocks * pool->block_size);
  return PKV_OK;
}

// CONTEXT_BOUNDS, then (query_len > 1) live rows shorter than their new tokens, then
// BLOCK_ID.
pkv_status check_attention_data(const pkv_pool_desc* pool, const int32_t* bt,
                                int32_t max_blocks, const int32_t* ctx, int64_t num_rows,
                                int32_t query_len = 1) {
  const int64_t limit = ctx_limit_of(pool, max_blocks);
  for (int64_t r = 0; r < num_rows; ++r) {
    if (ctx[r] < 0 || ctx[r] > limit)
      return fail(PKV_ERR_CONTEXT_BOUNDS, "context_lens[%lld] = %d outside [0, %lld]",
                  (long long)r, ctx[r], (long long)limit);
  }
  for (int64_t r = 0; r < num_rows; ++r) {
    if (ctx[r] > 0 && ctx[r] < query_len)
      return fail(PKV_ERR_CONTEXT_BOUNDS,
                  "context_lens[%lld] = %d is live but shorter than query_len %d",
                  (long long)r, ctx[r], query_len);
  }
  for (int64_t r = 0; r < num_rows; ++r) {
    const int64_t live = (ctx[r] + (int64_t)pool->block_size - 1) / pool->block_size;
    for (int64_t j = 0; j < live; ++j) {
      const int32_t id = bt[r * max_blocks + j];
      if (id < 0 || id >= pool->num_blocks)
        return fail(PKV_ERR_BLOCK_ID, "block_tables[%lld, %lld] = %d outside [0, %lld)",
                    (long long)r, (long long)j, id, (long long)pool->num_blocks);
    }
  }
  return PKV_OK;
}

pkv_status check_write_data(const pkv_pool_desc* pool, const int64_t* slots, int64_t n) {
  const int64_t sink = pool->num_blocks * pool->block_size;
  for (int64_t i = 0; i < n; ++i)
    if (slots[i] < 0 || slots[i] > sink)
      return fail(PKV_ERR_SLOT, "slot_mapping[%lld] = %lld outside [0, %lld]", (long long)i,
                  (long long)slots[i], (long long)sink);
  return PKV_OK;
}


// Work items of one call at the shortest chunk; the plan indexes them in 32 bits.
// `vectors` is query vectors per row (query_len x heads).
pkv_status check_attention_items(const pkv_pool_desc* pool, int32_t max_blocks,
                                 int64_t num_rows, int32_t vectors, const pkv::Tuning& t) {
  const int64_t most_items = num_rows * ((int64_t)max_blocks * pool->block_size /
                                         t.chunk_min + 1) * vectors;
  if (most_items > (int64_t{1} << 30))
    return fail(PKV_ERR_UNSUPPORTED, "rows x heads x chunks too large for one call");
  return PKV_OK;
}

pkv::WriteArgs write_args(const pkv_pool_desc* pool, void* k_cache, void* v_cache,
                          const void* k, const void* v, const int64_t* slot_mapping,
                          int64_t num_tokens) {
  pkv::WriteArgs a;
  a.g = geom(pool);
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k = k;
  a.v = v;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  return a;
}

hipError_t launch_write(const pkv_pool_desc* pool, void* k_cache, void* v_cache, const void* k,
                        const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                        hipStream_t st) {
  return pkv::launch_kv_write(
      write_args(pool, k_cache, v_cache, k, v, slot_mapping, num_tokens), st);
}

hipError_t launch_attention(const pkv_pool_desc* pool, void* out, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, int64_t num_rows, int32_t num_heads,
                            float scale, void* workspace, const pkv::Tuning& t,
                            hipStream_t st, int32_t query_len = 1,
                            const pkv::WriteArgs* write = nullptr) {
  pkv::AttnArgs a{};
  a.g = geom(pool);
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_rows = num_rows;
  a.num_heads = num_heads;
  a.max_blocks = max_blocks;
  a.ctx_limit = (int32_t)ctx_limit_of(pool, max_blocks);
  a.log2_chunk_min = log2i(t.chunk_min);
  a.log2_chunk_max = log2i(t.chunk_max);
  a.target_items = 0;
  a.grid_groups = 0;
  a.narrow_groups = 0;
  a.narrow_items = 0;
  a.deal_static = 1;
  a.query_group = 1;
  a.query_len = query_len;
  a.scale = scale;
  a.row_flags = nullptr;
  a.flag_stride = 0;
  const pkv::Workspace ws = pkv::carve_workspace(workspace, num_rows, num_heads * query_len,
                                                 pool->head_dim, max_blocks, pool->block_size,
                                                 t);
  return pkv::launch_paged_attention(a, ws, t, st, true, write);
}

// ---- slot input ----
int64_t slot_ctx_limit(const pkv_pool_desc* p, int32_t width) {
  const int64_t by_pool = p->num_blocks * p->block_size;
  return width < by_pool ? width : by_pool;
}

// EMPTY, pool, SHAPE, UNSUPPORTED: everything that needs no data.
pkv_status check_slots_shape(const pkv_pool_desc* pool, int32_t width, int64_t row_stride,
                             int64_t num_rows, int32_t num_heads) {
  if (num_rows == 0) return fail(PKV_ERR_EMPTY, "no rows");
  pkv_status s = check_pool(pool);
  if (s != PKV_OK) return s;
  if (num_rows < 0) return fail(PKV_ERR_SHAPE, "num_rows %lld < 0", (long long)num_rows);
  if (num_heads < 1 || num_heads % pool->num_kv_heads != 0)
    return fail(PKV_ERR_SHAPE, "%d query heads is not a positive multiple of %d KV heads",
                num_heads, pool->num_kv_heads);
  if (width < 1) return fail(PKV_ERR_SHAPE, "width %d < 1", width);
  if (row_stride < width)
    return fail(PKV_ERR_SHAPE, "row_stride %lld < width %d", (long long)row_stride, width);
  if (num_rows > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "num_rows %lld: built for at most 65535 rows",
                (long long)num_rows);
  if (width > (1 << 24))
    return fail(PKV_ERR_UNSUPPORTED, "width %d tokens: built for at most 2^24", width);
  return PKV_OK;
}

// CONTEXT_BOUNDS, then SLOT; `rect` is [num_rows][width] on the host.
pkv_status check_slots_data(const pkv_pool_desc* pool, const int64_t* rect, int64_t rect_stride,
                            int32_t width, const int32_t* ctx, int64_t num_rows) {
  const int64_t limit = slot_ctx_limit(pool, width);
  for (int64_t r = 0; r < num_rows; ++r) {
    if (ctx[r] < 0 || ctx[r] > limit)
      return fail(PKV_ERR_CONTEXT_BOUNDS, "context_lens[%lld] = %d outside [0, %lld]",
                  (long long)r, ctx[r], (long long)limit);
  }
  const int64_t slots = pool->num_blocks * pool->block_size;
  for (int64_t r = 0; r < num_rows; ++r) {
    for (int64_t t = 0; t < ctx[r]; ++t) {
      const int64_t v = rect[r * rect_stride + t];
      if (v < 0 || v >= slots)
        return fail(PKV_ERR_SLOT, "slot rectangle [%lld, %lld] = %lld outside [0, %lld)",
                    (long long)r, (long long)t, (long long)v, (long long)slots);
    }
  }
  return PKV_OK;
}

hipError_t launch_attention_slots(const pkv_pool_desc* pool, void* out, const void* q,
                                  const void* k_cache, const void* v_cache,
                                  const int64_t* slot_table, int32_t width,
                                  int64_t row_stride, const int32_t* context_lens,
                                  int64_t num_rows, int32_t num_heads, float scale,
                                  void* workspace, const pkv::Tuning& t, hipStream_t st) {
  pkv::AttnArgs a{};
  a.g = geom(pool);
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = nullptr;   // the derived table, set by the launcher
  a.context_lens = context_lens;
  a.num_rows = num_rows;
  a.num_heads = num_heads;
  a.max_blocks = (int32_t)(((int64_t)width + pool->block_size - 1) / pool->block_size);
  a.ctx_limit = (int32_t)slot_ctx_limit(pool, width);
  a.log2_chunk_min = log2i(t.chunk_min);
  a.log2_chunk_max = log2i(t.chunk_max);
  a.target_items = 0;
  a.grid_groups = 0;
  a.narrow_groups = 0;
  a.narrow_items = 0;
  a.deal_static = 1;
  a.query_group = 1;
  a.query_len = 1;
  a.scale = scale;
  a.row_flags = nullptr;
  a.flag_stride = 0;
  pkv::SlotArgs sa;
  sa.slots = slot_table;
  sa.row_stride = row_stride;
  sa.width = width;
  const pkv::Workspace ws = pkv::carve_slot_workspace(workspace, num_rows, num_heads,
                                                      pool->head_dim, width,
                                                      pool->block_size, t, &sa);
  return pkv::launch_paged_attention_slots(a, sa, ws, t, st);
}

// Records what `record` enqueues on a private stream into an instantiated graph.  The
// legacy default stream cannot be captured, and the caller's streams stay free of
// capture state; nothing runs while recording.  Relaxed mode: a launcher's first use on
// a device queries occupancy, which is not a stream operation but which the stricter
// modes may refuse.
template <typename F>
pkv_status record_graph(F&& record, pkv_step_graph** graph) {
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "creating the capture stream");
  hipGraph_t g = nullptr;
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e == hipSuccess) {
    const hipError_t le = record(cs);
    e = hipStreamEndCapture(cs, &g);   // always end, so the stream leaves capture mode
    if (le != hipSuccess) e = le;
  }
  hipGraphExec_t exec = nullptr;
  if (e == hipSuccess) e = hipGraphInstantiateWithFlags(&exec, g, 0);
  if (g) (void)hipGraphDestroy(g);
  (void)hipStreamDestroy(cs);
  if (e != hipSuccess) return hip_fail(e, "capturing the decode step");
  *graph = new (std::nothrow) pkv_step_graph{exec};
  if (*graph == nullptr) {   // no exception crosses the C ABI
    (void)hipGraphExecDestroy(exec);
    return hip_fail(hipErrorOutOfMemory, "allocating the graph handle");
  }
  return ok();
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_str(pkv_status s) {
  switch (s) {
    case PKV_OK: return "OK";
    case PKV_ERR_EMPTY: return "EMPTY";
    case PKV_ERR_DTYPE: return "DTYPE";
    case PKV_ERR_SHAPE: return "SHAPE";
    case PKV_ERR_CONTEXT_BOUNDS: return "CONTEXT_BOUNDS";
    case PKV_ERR_BLOCK_ID: return "BLOCK_ID";
    case PKV_ERR_SLOT: return "SLOT";
    case PKV_ERR_UNSUPPORTED: return "UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "WORKSPACE";
    case PKV_ERR_NULL: return "NULL";
    case PKV_ERR_HIP: return "HIP";
  }
  return "UNKNOWN";
}

const char* pkv_last_error_detail(void) { return g_detail; }

int64_t pkv_sink_slot(const pkv_pool_desc* pool) {
  if (check_pool(pool) != PKV_OK) return -1;
  return pool->num_blocks * pool->block_size;
}

int64_t pkv_pool_elements(const pkv_pool_desc* pool) {
  if (check_pool(pool) != PKV_OK) return -1;
  return (pool->num_blocks + 1) * pool->block_size * (int64_t)pool->num_kv_heads *
         pool->head_dim;
}

pkv_status pkv_check_pool(const pkv_pool_desc* pool) {
  pkv_status s = check_pool(pool);
  return s == PKV_OK ? ok() : s;
}

pkv_status pkv_check_write_host(const pkv_pool_desc* pool, const int64_t* slot_mapping,
                                int64_t num_tokens) {
  if (num_tokens == 0) return fail(PKV_ERR_EMPTY, "no tokens to write");
  pkv_status s = check_pool(pool);
  if (s != PKV_OK) return s;
  if (num_tokens < 0) return fail(PKV_ERR_SHAPE, "num_tokens %lld < 0", (long long)num_tokens);
  if (!slot_mapping) return fail(PKV_ERR_NULL, "slot_mapping is NULL");
  s = check_write_data(pool, slot_mapping, num_tokens);
  return s == PKV_OK ? ok() : s;
}

pkv_status pkv_check_attention_host(const pkv_pool_desc* pool, const int32_t* block_tables,
                                    int32_t max_blocks_per_row, const int32_t* context_lens,
                                    int64_t num_rows, int32_t num_heads) {
  pkv_status s = check_attention_shape(pool, max_blocks_per_row, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (!block_tables || !context_lens) return fail(PKV_ERR_NULL, "table or lengths NULL");
  s = check_attention_data(pool, block_tables, max_blocks_per_row, context_lens, num_rows);
  return s == PKV_OK ? ok() : s;
}

pkv_status pkv_kv_write(const pkv_pool_desc* pool, void* k_cache, void* v_cache,
                        const void* k, const void* v, const int64_t* slot_mapping,
                        int64_t num_tokens, int32_t validate, void* stream) {
  if (num_tokens == 0) return fail(PKV_ERR_EMPTY, "no tokens to write");
  pkv_status s = check_pool(pool);
  if (s != PKV_OK) return s;
  if (num_tokens < 0) return fail(PKV_ERR_SHAPE, "num_tokens %lld < 0", (long long)num_tokens);
  if (!k_cache || !v_cache || !k || !v || !slot_mapping)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (validate) {
    std::vector<int64_t> host;
    if (!host_buffer(host, (size_t)num_tokens))
      return hip_fail(hipErrorOutOfMemory, "allocating host memory to validate");
    hipError_t e = hipMemcpyAsync(host.data(), slot_mapping, host.size() * sizeof(int64_t),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "copying slot_mapping to the host");
    s = check_write_data(pool, host.data(), num_tokens);
    if (s != PKV_OK) return s;
  }
  hipError_t e = launch_write(pool, k_cache, v_cache, k, v, slot_mapping, num_tokens, st);
  if (e != hipSuccess) return hip_fail(e, "launching kv_write");
  return ok();
}

size_t pkv_workspace_bytes(const pkv_pool_desc* pool, int64_t num_rows, int32_t num_heads,
                           int32_t max_blocks_per_row) {
  const pkv::Tuning t = pkv::tuning_snapshot();
  if (check_attention_shape(pool, max_blocks_per_row, num_rows, num_heads) != PKV_OK ||
      check_attention_items(pool, max_blocks_per_row, num_rows, num_heads, t) != PKV_OK)
    return 0;
  return pkv::workspace_bytes(num_rows, num_heads, pool->head_dim, max_blocks_per_row,
                              pool->block_size, t);
}

pkv_status pkv_paged_attention(const pkv_pool_desc* pool, void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_row,
                               const int32_t* context_lens, int64_t num_rows,
                               int32_t num_heads, float scale, void* workspace,
                               size_t workspace_bytes, int32_t validate, void* stream) {
  const pkv::Tuning t = pkv::tuning_snapshot();   // this call's one view of the tuning
  pkv_status s = check_attention_shape(pool, max_blocks_per_row, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  s = check_attention_items(pool, max_blocks_per_row, num_rows, num_heads, t);
  if (s != PKV_OK) return s;
  const size_t need = pkv::workspace_bytes(num_rows, num_heads, pool->head_dim,
                                           max_blocks_per_row, pool->block_size, t);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (validate) {
    std::vector<int32_t> ctx;
    if (!host_buffer(ctx, (size_t)num_rows))
      return hip_fail(hipErrorOutOfMemory, "allocating host memory to validate");
    std::vector<int32_t> bt;
    if (!host_buffer(bt, (size_t)(num_rows * max_blocks_per_row)))
      return hip_fail(hipErrorOutOfMemory, "allocating host memory to validate");
    hipError_t e = hipMemcpyAsync(ctx.data(), context_lens, ctx.size() * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(bt.data(), block_tables, bt.size() * sizeof(int32_t),
                         hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "copying lengths and tables to the host");
    s = check_attention_data(pool, bt.data(), max_blocks_per_row, ctx.data(), num_rows);
    if (s != PKV_OK) return s;
  }
  hipError_t e = launch_attention(pool, out, q, k_cache, v_cache, block_tables,
                                  max_blocks_per_row, context_lens, num_rows, num_heads, scale,
                                  workspace, t, st);
  if (e != hipSuccess) return hip_fail(e, "launching paged_attention");
  return ok();
}

pkv_status pkv_paged_attention_noalloc(const pkv_pool_desc* pool, void* out, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables,
                                       int32_t max_blocks_per_row,
                                       const int32_t* context_lens, int64_t num_rows,
                                       int32_t num_heads, float scale, void* stream) {
  static_assert(pkv::kScratchBytes == PKV_NOALLOC_SCRATCH_BYTES, "the header states it");
  const pkv::Tuning t = pkv::tuning_snapshot();   // this call's one view of the tuning
  pkv_status s = check_attention_shape(pool, max_blocks_per_row, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  s = check_attention_items(pool, max_blocks_per_row, num_rows, num_heads, t);
  if (s != PKV_OK) return s;
  const size_t need = pkv::workspace_bytes(num_rows, num_heads, pool->head_dim,
                                           max_blocks_per_row, pool->block_size, t);
  if (need > pkv::kScratchBytes)
    return fail(PKV_ERR_WORKSPACE,
                "this batch needs a workspace of %zu bytes; the static scratch holds %zu "
                "(use pkv_paged_attention with a workspace of its own)",
                need, pkv::kScratchBytes);
  void* scratch = nullptr;
  hipError_t e = pkv::scratch_pointer(&scratch);
  if (e != hipSuccess) return hip_fail(e, "looking up the static scratch");
  const pkv::TimingPause untimed;   // timing would create events
  e = launch_attention(pool, out, q, k_cache, v_cache, block_tables, max_blocks_per_row,
                       context_lens, num_rows, num_heads, scale, scratch, t,
                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching paged_attention_noalloc");
  return ok();
}

size_t pkv_workspace_bytes_slots(const pkv_pool_desc* pool, int64_t num_rows,
                                 int32_t num_heads, int32_t width) {
  const pkv::Tuning t = pkv::tuning_snapshot();
  if (check_slots_shape(pool, width, width, num_rows, num_heads) != PKV_OK) return 0;
  const int32_t max_blocks = (int32_t)(((int64_t)width + pool->block_size - 1) /
                                       pool->block_size);
  if (check_attention_items(pool, max_blocks, num_rows, num_heads, t) != PKV_OK) return 0;
  return pkv::slot_workspace_bytes(num_rows, num_heads, pool->head_dim, width,
                                   pool->block_size, t);
}

pkv_status pkv_check_attention_slots_host(const pkv_pool_desc* pool,
                                          const int64_t* slot_table, int32_t width,
                                          int64_t row_stride, const int32_t* context_lens,
                                          int64_t num_rows, int32_t num_heads) {
  pkv_status s = check_slots_shape(pool, width, row_stride, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (!slot_table || !context_lens) return fail(PKV_ERR_NULL, "rectangle or lengths NULL");
  s = check_slots_data(pool, slot_table, row_stride, width, context_lens, num_rows);
  return s == PKV_OK ? ok() : s;
}

pkv_status pkv_paged_attention_slots(const pkv_pool_desc* pool, void* out, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int64_t* slot_table, int32_t width,
                                     int64_t row_stride, const int32_t* context_lens,
                                     int64_t num_rows, int32_t num_heads, float scale,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t validate, void* stream) {
  const pkv::Tuning t = pkv::tuning_snapshot();   // this call's one view of the tuning
  pkv_status s = check_slots_shape(pool, width, row_stride, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (!out || !q || !k_cache || !v_cache || !slot_table || !context_lens)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  const int32_t max_blocks = (int32_t)(((int64_t)width + pool->block_size - 1) /
                                       pool->block_size);
  s = check_attention_items(pool, max_blocks, num_rows, num_heads, t);
  if (s != PKV_OK) return s;
  const size_t need = pkv::slot_workspace_bytes(num_rows, num_heads, pool->head_dim, width,
                                                pool->block_size, t);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (validate) {
    std::vector<int32_t> ctx;
    if (!host_buffer(ctx, (size_t)num_rows))
      return hip_fail(hipErrorOutOfMemory, "allocating host memory to validate");
    std::vector<int64_t> rect;
    if (!host_buffer(rect, (size_t)(num_rows * width)))
      return hip_fail(hipErrorOutOfMemory, "allocating host memory to validate");
    hipError_t e = hipMemcpyAsync(ctx.data(), context_lens, ctx.size() * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(rect.data(), (size_t)width * sizeof(int64_t), slot_table,
                           (size_t)row_stride * sizeof(int64_t),
                           (size_t)width * sizeof(int64_t), (size_t)num_rows,
                           hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "copying lengths and slots to the host");
    s = check_slots_data(pool, rect.data(), width, width, ctx.data(), num_rows);
    if (s != PKV_OK) return s;
  }
  hipError_t e = launch_attention_slots(pool, out, q, k_cache, v_cache, slot_table, width,
                                        row_stride, context_lens, num_rows, num_heads, scale,
                                        workspace, t, st);
  if (e != hipSuccess) return hip_fail(e, "launching paged_attention_slots");
  return ok();
}

// ---- several new tokens per row ----
static pkv_status check_multi_shape(const pkv_pool_desc* pool, int32_t max_blocks,
                                    int64_t num_rows, int32_t query_len, int32_t num_heads) {
  pkv_status s = check_attention_shape(pool, max_blocks, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (query_len < 1) return fail(PKV_ERR_SHAPE, "query_len %d < 1", query_len);
  if (query_len > 64)
    return fail(PKV_ERR_UNSUPPORTED, "query_len %d: built for at most 64", query_len);
  return PKV_OK;
}

size_t pkv_workspace_bytes_multi(const pkv_pool_desc* pool, int64_t num_rows,
                                 int32_t query_len, int32_t num_heads,
                                 int32_t max_blocks_per_row) {
  const pkv::Tuning t = pkv::tuning_snapshot();
  if (check_multi_shape(pool, max_blocks_per_row, num_rows, query_len, num_heads) != PKV_OK ||
      check_attention_items(pool, max_blocks_per_row, num_rows, num_heads * query_len, t) !=
          PKV_OK)
    return 0;
  return pkv::workspace_bytes(num_rows, num_heads * query_len, pool->head_dim,
                              max_blocks_per_row, pool->block_size, t);
}

pkv_status pkv_check_attention_multi_host(const pkv_pool_desc* pool,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_row,
                                          const int32_t* context_lens, int64_t num_rows,
                                          int32_t query_len, int32_t num_heads) {
  pkv_status s = check_multi_shape(pool, max_blocks_per_row, num_rows, query_len, num_heads);
  if (s != PKV_OK) return s;
  if (!block_tables || !context_lens) return fail(PKV_ERR_NULL, "table or lengths NULL");
  s = check_attention_data(pool, block_tables, max_blocks_per_row, context_lens, num_rows,
                           query_len);
  return s == PKV_OK ? ok() : s;
}

pkv_status pkv_paged_attention_multi(const pkv_pool_desc* pool, void* out, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_row,
                                     const int32_t* context_lens, int64_t num_rows,
                                     int32_t query_len, int32_t num_heads, float scale,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t validate, void* stream) {
  const pkv::Tuning t = pkv::tuning_snapshot();   // this call's one view of the tuning
  pkv_status s = check_multi_shape(pool, max_blocks_per_row, num_rows, query_len, num_heads);
  if (s != PKV_OK) return s;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  s = check_attention_items(pool, max_blocks_per_row, num_rows, num_heads * query_len, t);
  if (s != PKV_OK) return s;
  const size_t need = pkv::workspace_bytes(num_rows, num_heads * query_len, pool->head_dim,
                                           max_blocks_per_row, pool->block_size, t);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (validate) {
    std::vector<int32_t> ctx;
    if (!host_buffer(ctx, (size_t)num_rows))
      return hip_fail(hipErrorOutOfMemory, "allocating host memory to validate");
    std::vector<int32_t> bt;
    if (!host_buffer(bt, (size_t)(num_rows * max_blocks_per_row)))
      return hip_fail(hipErrorOutOfMemory, "allocating host memory to validate");
    hipError_t e = hipMemcpyAsync(ctx.data(), context_lens, ctx.size() * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(bt.data(), block_tables, bt.size() * sizeof(int32_t),
                         hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "copying lengths and tables to the host");
    s = check_attention_data(pool, bt.data(), max_blocks_per_row, ctx.data(), num_rows,
                             query_len);
    if (s != PKV_OK) return s;
  }
  hipError_t e = launch_attention(pool, out, q, k_cache, v_cache, block_tables,
                                  max_blocks_per_row, context_lens, num_rows, num_heads, scale,
                                  workspace, t, st, query_len);
  if (e != hipSuccess) return hip_fail(e, "launching paged_attention_multi");
  return ok();
}

const char* pkv_decode_kernel_for(const pkv_pool_desc* pool, int32_t num_heads,
                                  int32_t query_len) {
  if (check_pool(pool) != PKV_OK || num_heads < 1 || num_heads % pool->num_kv_heads != 0 ||
      query_len < 1)
    return "";
  pkv::AttnArgs a{};
  a.g = geom(pool);
  a.num_heads = num_heads;
  a.query_len = query_len;
  return pkv::decode_kernel_name(a, pkv::tuning_snapshot());
}

pkv_status pkv_device_status(uint32_t* flags, int32_t clear, void* stream) {
  if (!flags) return fail(PKV_ERR_NULL, "flags is NULL");
  hipError_t e = pkv::read_device_status(flags, clear, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reading the device status word");
  return ok();
}

// The counters block every attention call keeps at the start of its workspace.
static pkv_status read_counters(const void* workspace, size_t workspace_bytes, int32_t* c,
                                void* stream) {
  if (!workspace) return fail(PKV_ERR_NULL, "workspace is NULL");
  if (workspace_bytes < (size_t)pkv::kCounterBytes)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes holds no counters (%d bytes)",
                workspace_bytes, pkv::kCounterBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(c, workspace, pkv::kNumCounters * sizeof(int32_t),
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "reading the workspace counters");
  return PKV_OK;
}

pkv_status pkv_plan_info_read(const void* workspace, size_t workspace_bytes,
                              pkv_plan_info* info, void* stream) {
  if (!info) return fail(PKV_ERR_NULL, "info is NULL");
  int32_t c[pkv::kNumCounters];
  const pkv_status s = read_counters(workspace, workspace_bytes, c, stream);
  if (s != PKV_OK) return s;
  info->chunk_tokens = c[pkv::kCtrChunk];
  info->entries = c[pkv::kCtrEntries];
  info->full_chunks = c[pkv::kCtrSectionA];
  info->live_entries = c[pkv::kCtrData];
  info->wide_entries = c[pkv::kCtrWide];
  info->split_rows = c[pkv::kCtrSplitRows];
  info->records = c[pkv::kCtrRecords];
  info->record_capacity = c[pkv::kCtrRecordCap];
  info->decode_groups = c[pkv::kCtrGroups];
  info->vector_groups = c[pkv::kCtrVectorGroups];
  info->tile_tokens = c[pkv::kCtrTileTokens];
  uint64_t walked = 0;
  std::memcpy(&walked, &c[pkv::kCtrWalked], sizeof walked);
  info->tiles_walked = (int64_t)walked;
  info->token_rows = c[pkv::kCtrTokenRows];
  info->token_entries = c[pkv::kCtrTokenEntries];
  info->status = (uint32_t)c[pkv::kCtrStatus];
  return ok();
}

pkv_status pkv_workspace_status(const void* workspace, size_t workspace_bytes,
                                uint32_t* flags, void* stream) {
  if (!flags) return fail(PKV_ERR_NULL, "flags is NULL");
  int32_t c[pkv::kNumCounters];
  const pkv_status s = read_counters(workspace, workspace_bytes, c, stream);
  if (s != PKV_OK) return s;
  *flags = (uint32_t)c[pkv::kCtrStatus];
  return ok();
}

pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink,
                           int32_t groups_per_cu, void* stream) {
  if (!src || !sink) return fail(PKV_ERR_NULL, "src or sink is NULL");
  if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
    return fail(PKV_ERR_SHAPE, "bytes %zu: a positive multiple of 16 up to 2^40", bytes);
  if (groups_per_cu < 1 || groups_per_cu > 16)
    return fail(PKV_ERR_SHAPE, "groups_per_cu %d outside [1, 16]", groups_per_cu);
  hipError_t e = pkv::launch_stream_read(src, (int64_t)bytes, sink, groups_per_cu,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the streaming read");
  return ok();
}

pkv_status pkv_gather_read(const void* k_base, const void* v_base, const int64_t* offsets,
                           int64_t n_pieces, int32_t piece_bytes, uint32_t* sink,
                           int32_t groups_per_cu, int32_t waves_per_group,
                           int32_t pieces_per_wave, void* stream) {
  if (!k_base || !v_base || !offsets || !sink)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  if (n_pieces < 1 || piece_bytes < 16 || piece_bytes % 16 != 0 || piece_bytes > (1 << 20))
    return fail(PKV_ERR_SHAPE, "%lld pieces of %d bytes: at least one piece, each a multiple "
                "of 16 bytes up to 1 MiB", (long long)n_pieces, piece_bytes);
  if (groups_per_cu < 1 || groups_per_cu > 16)
    return fail(PKV_ERR_SHAPE, "groups_per_cu %d outside [1, 16]", groups_per_cu);
  if (waves_per_group != 4 && waves_per_group != 8)
    return fail(PKV_ERR_SHAPE, "waves_per_group %d: 4 or 8", waves_per_group);
  if (pieces_per_wave != 1 && pieces_per_wave != 2 && pieces_per_wave != 4)
    return fail(PKV_ERR_SHAPE, "pieces_per_wave %d: 1, 2 or 4", pieces_per_wave);
  hipError_t e = pkv::launch_gather_read(k_base, v_base, offsets, n_pieces, piece_bytes, sink,
                                         groups_per_cu, waves_per_group, pieces_per_wave,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the gathering read");
  return ok();
}

pkv_status pkv_set_tuning(const pkv_tuning* t) {
  if (!t) return fail(PKV_ERR_NULL, "tuning is NULL");
  if (!pkv::set_tuning(t->chunk_min, t->chunk_max, t->decode_waves, t->items_per_group,
                       t->deal, t->staging, t->max_query_group, t->mfma, t->groups_per_cu,
                       t->solo_tokens))
    return fail(PKV_ERR_UNSUPPORTED, "tuning chunk [%d, %d], waves %d, items/group %d, "
                "deal %d, staging %d, query group %d, mfma %d, groups/CU %d, solo tokens %d "
                "not supported",
                t->chunk_min, t->chunk_max, t->decode_waves, t->items_per_group, t->deal,
                t->staging, t->max_query_group, t->mfma, t->groups_per_cu, t->solo_tokens);
  return ok();
}

pkv_status pkv_get_tuning(pkv_tuning* t) {
  if (!t) return fail(PKV_ERR_NULL, "tuning is NULL");
  const pkv::Tuning c = pkv::tuning_snapshot();
  t->chunk_min = c.chunk_min;
  t->chunk_max = c.chunk_max;
  t->decode_waves = c.decode_waves;
  t->items_per_group = c.items_per_group;
  t->deal = c.deal_static ? 1 : 2;
  t->staging = c.lds_stage ? 2 : 1;
  t->max_query_group = c.max_query_group;
  t->mfma = c.mfma ? 1 : 2;
  t->groups_per_cu = c.groups_per_cu;
  t->solo_tokens = c.solo_tokens;
  return ok();
}

pkv_status pkv_timing_enable(int32_t on) {
  pkv::timing_enable(on != 0);
  return ok();
}

pkv_status pkv_timing_read(int32_t phase, double* total_ms, int64_t* launches,
                           int32_t reset) {
  if (!total_ms || !launches) return fail(PKV_ERR_NULL, "output pointer is NULL");
  if (phase < PKV_PHASE_KV_WRITE || phase > PKV_PHASE_TOKEN_ROWS)
    return fail(PKV_ERR_SHAPE, "unknown phase %d", phase);
  hipError_t e = pkv::timing_read(phase, total_ms, launches, reset != 0);
  if (e != hipSuccess) return hip_fail(e, "reading kernel timing events");
  return ok();
}

// ---------------------------------------------------------------------------------
// captured steps
// ---------------------------------------------------------------------------------
pkv_status pkv_graph_capture(const pkv_pool_desc* pool, void* k_cache, void* v_cache,
                             const void* k, const void* v, const int64_t* slot_mapping,
                             void* out, const void* q, const int32_t* block_tables,
                             int32_t max_blocks_per_row, const int32_t* context_lens,
                             int64_t num_rows, int32_t num_heads, float scale,
                             void* workspace, size_t workspace_bytes,
                             pkv_step_graph** graph) {
  if (!graph) return fail(PKV_ERR_NULL, "graph is NULL");
  *graph = nullptr;
  const pkv::Tuning t = pkv::tuning_snapshot();   // frozen into the graph
  pkv_status s = check_attention_shape(pool, max_blocks_per_row, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (!k_cache || !v_cache || !k || !v || !slot_mapping || !out || !q || !block_tables ||
      !context_lens)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  s = check_attention_items(pool, max_blocks_per_row, num_rows, num_heads, t);
  if (s != PKV_OK) return s;
  const size_t need = pkv::workspace_bytes(num_rows, num_heads, pool->head_dim,
                                           max_blocks_per_row, pool->block_size, t);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);

  // the slot scatter rides in the plan kernel's launch: one kernel fewer per replay
  const pkv::WriteArgs wa = write_args(pool, k_cache, v_cache, k, v, slot_mapping, num_rows);
  return record_graph([&](hipStream_t cs) {
    return launch_attention(pool, out, q, k_cache, v_cache, block_tables, max_blocks_per_row,
                            context_lens, num_rows, num_heads, scale, workspace, t, cs, 1, &wa);
  }, graph);
}

pkv_status pkv_graph_capture_slots(const pkv_pool_desc* pool, void* k_cache, void* v_cache,
                                   const void* k, const void* v, const int64_t* slot_mapping,
                                   void* out, const void* q, const int64_t* slot_table,
                                   int32_t width, int64_t row_stride,
                                   const int32_t* context_lens, int64_t num_rows,
                                   int32_t num_heads, float scale, void* workspace,
                                   size_t workspace_bytes, pkv_step_graph** graph) {
  if (!graph) return fail(PKV_ERR_NULL, "graph is NULL");
  *graph = nullptr;
  const pkv::Tuning t = pkv::tuning_snapshot();   // frozen into the graph
  pkv_status s = check_slots_shape(pool, width, row_stride, num_rows, num_heads);
  if (s != PKV_OK) return s;
  if (!k_cache || !v_cache || !k || !v || !slot_mapping || !out || !q || !slot_table ||
      !context_lens)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  const int32_t max_blocks = (int32_t)(((int64_t)width + pool->block_size - 1) /
                                       pool->block_size);
  s = check_attention_items(pool, max_blocks, num_rows, num_heads, t);
  if (s != PKV_OK) return s;
  const size_t need = pkv::slot_workspace_bytes(num_rows, num_heads, pool->head_dim, width,
                                                pool->block_size, t);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  return record_graph([&](hipStream_t cs) {
    hipError_t e = launch_write(pool, k_cache, v_cache, k, v, slot_mapping, num_rows, cs);
    if (e != hipSuccess) return e;
    return launch_attention_slots(pool, out, q, k_cache, v_cache, slot_table, width,
                                  row_stride, context_lens, num_rows, num_heads, scale,
                                  workspace, t, cs);
  }, graph);
}

pkv_status pkv_graph_launch(const pkv_step_graph* graph, void* stream) {
  if (!graph) return fail(PKV_ERR_NULL, "graph is NULL");
  hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching a captured step");
  return ok();
}

pkv_status pkv_graph_destroy(pkv_step_graph* graph) {
  if (!graph) return ok();
  hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  if (e != hipSuccess) return hip_fail(e, "destroying a captured step");
  return ok();
}

}  // extern "C"
