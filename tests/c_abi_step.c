/* One decode step driven from plain C through the library's boundary, with device
 * memory from the HIP C runtime and nothing else: the slot scatter (pkv_kv_write), then
 * the read (pkv_paged_attention), both validated, on the default stream.
 *
 * usage: c_abi_step <dir>
 *   <dir>/shape.txt   num_blocks block_size kv_heads head_dim dtype layout rows heads
 *                     max_blocks_per_row num_tokens  (integers, pkv_dtype / pkv_layout
 *                     codes)
 *   <dir>/scale.bin   the float32 scale
 *   <dir>/k_pool.bin, v_pool.bin, q.bin, k_new.bin, v_new.bin   pool-dtype storage
 *   <dir>/slots.bin (int64), tables.bin (int32), lens.bin (int32)
 * writes <dir>/out.bin, k_pool_out.bin, v_pool_out.bin; exits non-zero on any error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pagedkv.h"

static char path[4096];

static const char* in_dir(const char* dir, const char* name) {
  snprintf(path, sizeof path, "%s/%s", dir, name);
  return path;
}

/* the whole file, exactly `bytes` long */
static void* read_exact(const char* dir, const char* name, size_t bytes) {
  FILE* f = fopen(in_dir(dir, name), "rb");
  void* p;
  long size;
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return NULL;
  }
  fseek(f, 0, SEEK_END);
  size = ftell(f);
  fseek(f, 0, SEEK_SET);
  if (size < 0 || (size_t)size != bytes) {
    fprintf(stderr, "%s: %ld bytes, expected %zu\n", path, size, bytes);
    fclose(f);
    return NULL;
  }
  p = malloc(bytes > 0 ? bytes : 1);
  if (p && bytes > 0 && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

static int write_all(const char* dir, const char* name, const void* p, size_t bytes) {
  FILE* f = fopen(in_dir(dir, name), "wb");
  int ok;
  if (!f) return 0;
  ok = fwrite(p, 1, bytes, f) == bytes;
  return fclose(f) == 0 && ok;
}

#define HIP_CHECK(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      return 2;                                                             \
    }                                                                       \
  } while (0)

#define PKV_CHECK(x)                                                        \
  do {                                                                      \
    pkv_status s_ = (x);                                                    \
    if (s_ != PKV_OK) {                                                     \
      fprintf(stderr, "%s: %s (%s)\n", #x, pkv_status_str(s_),              \
              pkv_last_error_detail());                                     \
      return 3;                                                             \
    }                                                                       \
  } while (0)

enum { K_POOL, V_POOL, Q, K_NEW, V_NEW, SLOTS, TABLES, LENS, OUT, WS, N_BUF };

int main(int argc, char** argv) {
  const char* dir;
  FILE* f;
  long long nb, bs, hkv, d, dtype, layout, rows, heads, mb, ntok;
  pkv_pool_desc pool;
  size_t elem, bytes[N_BUF];
  void* host[N_BUF];
  void* dev[N_BUF];
  float* scale;
  uint32_t flags = 0;
  int i;
  static const char* const names[N_BUF] = {"k_pool.bin", "v_pool.bin", "q.bin",
                                           "k_new.bin", "v_new.bin", "slots.bin",
                                           "tables.bin", "lens.bin", NULL, NULL};

  if (argc != 2) {
    fprintf(stderr, "usage: %s <dir>\n", argv[0]);
    return 1;
  }
  dir = argv[1];
  f = fopen(in_dir(dir, "shape.txt"), "r");
  if (!f || fscanf(f, "%lld %lld %lld %lld %lld %lld %lld %lld %lld %lld", &nb, &bs, &hkv,
                   &d, &dtype, &layout, &rows, &heads, &mb, &ntok) != 10) {
    fprintf(stderr, "cannot read %s\n", path);
    return 1;
  }
  fclose(f);
  pool.num_blocks = nb;
  pool.block_size = (int32_t)bs;
  pool.num_kv_heads = (int32_t)hkv;
  pool.head_dim = (int32_t)d;
  pool.dtype = (int32_t)dtype;
  pool.layout = (int32_t)layout;
  PKV_CHECK(pkv_check_pool(&pool));
  elem = pool.dtype == PKV_F32 ? 4 : 2;

  bytes[K_POOL] = bytes[V_POOL] = (size_t)pkv_pool_elements(&pool) * elem;
  bytes[Q] = bytes[OUT] = (size_t)(rows * heads * d) * elem;
  bytes[K_NEW] = bytes[V_NEW] = (size_t)(ntok * hkv * d) * elem;
  bytes[SLOTS] = (size_t)ntok * sizeof(int64_t);
  bytes[TABLES] = (size_t)(rows * mb) * sizeof(int32_t);
  bytes[LENS] = (size_t)rows * sizeof(int32_t);
  bytes[WS] = pkv_workspace_bytes(&pool, rows, (int32_t)heads, (int32_t)mb);
  if (bytes[WS] == 0) {
    fprintf(stderr, "pkv_workspace_bytes: %s\n", pkv_last_error_detail());
    return 3;
  }
  scale = (float*)read_exact(dir, "scale.bin", sizeof(float));
  if (!scale) return 1;

  for (i = 0; i < N_BUF; ++i) {
    host[i] = names[i] ? read_exact(dir, names[i], bytes[i]) : calloc(1, bytes[i]);
    if (!host[i]) return 1;
    HIP_CHECK(hipMalloc(&dev[i], bytes[i] > 0 ? bytes[i] : 1));
    if (bytes[i] > 0) HIP_CHECK(hipMemcpy(dev[i], host[i], bytes[i], hipMemcpyHostToDevice));
  }

  PKV_CHECK(pkv_kv_write(&pool, dev[K_POOL], dev[V_POOL], dev[K_NEW], dev[V_NEW],
                         (const int64_t*)dev[SLOTS], ntok, 1, NULL));
  PKV_CHECK(pkv_paged_attention(&pool, dev[OUT], dev[Q], dev[K_POOL], dev[V_POOL],
                                (const int32_t*)dev[TABLES], (int32_t)mb,
                                (const int32_t*)dev[LENS], rows, (int32_t)heads, *scale,
                                dev[WS], bytes[WS], 1, NULL));
  HIP_CHECK(hipDeviceSynchronize());
  PKV_CHECK(pkv_workspace_status(dev[WS], bytes[WS], &flags, NULL));
  if (flags != 0) {
    fprintf(stderr, "device status bits %u\n", flags);
    return 4;
  }

  HIP_CHECK(hipMemcpy(host[OUT], dev[OUT], bytes[OUT], hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(host[K_POOL], dev[K_POOL], bytes[K_POOL], hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(host[V_POOL], dev[V_POOL], bytes[V_POOL], hipMemcpyDeviceToHost));
  if (!write_all(dir, "out.bin", host[OUT], bytes[OUT]) ||
      !write_all(dir, "k_pool_out.bin", host[K_POOL], bytes[K_POOL]) ||
      !write_all(dir, "v_pool_out.bin", host[V_POOL], bytes[V_POOL])) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  for (i = 0; i < N_BUF; ++i) {
    HIP_CHECK(hipFree(dev[i]));
    free(host[i]);
  }
  free(scale);
  printf("c-abi step: %lld rows x %lld heads over %lld KV heads, d %lld, workspace %zu B\n",
         rows, heads, hkv, d, bytes[WS]);
  return 0;
}
