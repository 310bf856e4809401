// gfx950 kernels of the batched paged-attention decode step.
//
//   kv_write_kernel  slot scatter of the step's new K/V (Day 55, "the capture list
//                    moved to startup, and the dummy batch was all padding", "Why it
//                    matters": pad rows write the sink slot)
//   plan_kernel      one workgroup turns context_lens into a work list of
//                    (row, chunk) entries, longest first, and resets the work queue
//   decode_kernel    persistent workgroups pull (entry, query head) items from the
//                    queue; each streams its chunk of the row's history through the
//                    block table in 16-token sub-chunks and folds them into an online
//                    softmax (Day 59, "the rectangle the read builds, and the tile
//                    that replaces it", "What I added today" and "What I learned" 3-4)
//   combine_kernel   merges the per-chunk (max, denominator, accumulator) partials of
//                    rows longer than one chunk, in chunk order
//
// Lane mapping of one wave (64 lanes) inside the decode loop: a (token, KV head)
// vector of head_dim elements is 16-byte pieces spread over LPT consecutive lanes
// (LPT = head_dim * elem_bytes / 16; 16 lanes for bf16 x 128), so one 16-byte load
// per lane moves TPS = 64 / LPT tokens and the load of one wave is a contiguous
// TPS * head_dim run in the HND layout.  Each group of LPT lanes keeps its own online
// softmax state over the tokens it loaded; the q.k partial dot is reduced inside the
// group with DPP row operations, and the groups are merged once per item.  There is
// no MFMA: with one query per head the work is a bandwidth-bound streaming read.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "pagedkv.h"

namespace pkv {

__device__ unsigned int g_status;   // PKV_DEVERR_* bits, see pkv_device_status

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------- //
// element types: float (f32) and uint16_t holding bfloat16 bits (bf16)
// ------------------------------------------------------------------------- //
template <typename T> struct Elem;

template <> struct Elem<float> {
  static constexpr int kPerLane = 4;   // elements in 16 bytes
  // acc + q.k over this lane's 4 elements
  __device__ __forceinline__ static float dot(const uint4& q, const uint4& k, float acc) {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
  __device__ __forceinline__ static void axpy(float p, const uint4& v, float* acc) {
    acc[0] = fmaf(p, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(p, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(p, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(p, __uint_as_float(v.w), acc[3]);
  }
  __device__ __forceinline__ static uint4 pack(const float* x) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  }
};

template <> struct Elem<uint16_t> {
  static constexpr int kPerLane = 8;
  __device__ __forceinline__ static float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  }
  __device__ __forceinline__ static float dot(const uint4& q, const uint4& k, float acc) {
    acc = dot2(q.x, k.x, acc);
    acc = dot2(q.y, k.y, acc);
    acc = dot2(q.z, k.z, acc);
    acc = dot2(q.w, k.w, acc);
    return acc;
  }
  // bfloat16 -> float is a 16-bit left shift of the bits
  __device__ __forceinline__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ __forceinline__ static float hi(uint32_t w) {
    return __uint_as_float(w & 0xffff0000u);
  }
  __device__ __forceinline__ static void axpy(float p, const uint4& v, float* acc) {
    acc[0] = fmaf(p, lo(v.x), acc[0]);
    acc[1] = fmaf(p, hi(v.x), acc[1]);
    acc[2] = fmaf(p, lo(v.y), acc[2]);
    acc[3] = fmaf(p, hi(v.y), acc[3]);
    acc[4] = fmaf(p, lo(v.z), acc[4]);
    acc[5] = fmaf(p, hi(v.z), acc[5]);
    acc[6] = fmaf(p, lo(v.w), acc[6]);
    acc[7] = fmaf(p, hi(v.w), acc[7]);
  }
  // float pair -> packed bfloat16 pair, round to nearest even (v_cvt_pk_bf16_f32)
  __device__ __forceinline__ static uint32_t cvt2(float a, float b) {
    float2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  }
  __device__ __forceinline__ static uint4 pack(const float* x) {
    return make_uint4(cvt2(x[0], x[1]), cvt2(x[2], x[3]), cvt2(x[4], x[5]), cvt2(x[6], x[7]));
  }
};

// ------------------------------------------------------------------------- //
// lane-group reductions
// ------------------------------------------------------------------------- //
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of N lanes (N = 8, 16, 32, 64); every lane of a group
// ends with the group's sum.  Within a 16-lane DPP row: swap neighbours, swap pairs,
// mirror halves of 8, mirror the row; across rows: cross-lane shuffles.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);   // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// ------------------------------------------------------------------------- //
// slot scatter
// ------------------------------------------------------------------------- //
template <typename T>
__global__ void __launch_bounds__(256) kv_write_kernel(WriteArgs a, int64_t sink) {
  constexpr int E = Elem<T>::kPerLane;
  const int per_head = a.g.head_dim / E;                 // 16-byte pieces per head vector
  const int64_t per_tok = (int64_t)a.g.kv_heads * per_head;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.num_tokens * per_tok) return;
  const int64_t i = idx / per_tok;
  const int c = (int)(idx - i * per_tok);
  const int h = c / per_head;
  const int d0 = (c - h * per_head) * E;
  const int64_t slot = a.slot_mapping[i];
  if (slot < 0 || slot > sink) {
    if (c == 0) atomicOr(&g_status, PKV_DEVERR_SLOT);
    return;
  }
  const int64_t blk = slot >> a.g.log2_bs;
  const int64_t off = slot & (a.g.block_size - 1);
  const int64_t dst = blk * a.g.blk_stride + h * a.g.head_stride + off * a.g.tok_stride + d0;
  const int64_t src = (i * a.g.kv_heads + h) * a.g.head_dim + d0;
  store16(static_cast<T*>(a.k_cache) + dst, load16(static_cast<const T*>(a.k) + src));
  store16(static_cast<T*>(a.v_cache) + dst, load16(static_cast<const T*>(a.v) + src));
}

// ------------------------------------------------------------------------- //
// plan: context_lens -> work list
// ------------------------------------------------------------------------- //
constexpr int kPlanThreads = 1024;

// exclusive prefix sum of one value per thread over the workgroup; returns the
// thread's prefix and writes the total to *total
__device__ int block_exclusive_scan(int x, int* s_tmp, int* total) {
  const int t = threadIdx.x;
  s_tmp[t] = x;
  __syncthreads();
  for (int d = 1; d < kPlanThreads; d <<= 1) {
    const int y = t >= d ? s_tmp[t - d] : 0;
    __syncthreads();
    s_tmp[t] += y;
    __syncthreads();
  }
  const int incl = s_tmp[t];
  *total = s_tmp[kPlanThreads - 1];
  __syncthreads();
  return incl - x;
}

__device__ __forceinline__ int clamp_ctx(int ctx, int limit) {
  if (ctx < 0 || ctx > limit) {
    atomicOr(&g_status, PKV_DEVERR_CONTEXT_BOUNDS);
    ctx = ctx < 0 ? 0 : limit;
  }
  return ctx;
}

// Entries are ordered longest first so that the queue's tail is short work:
//   A. every full chunk (kChunkTokens tokens) of every row, rows in order;
//   B. every row's trailing partial chunk, by length, longest first;
//   C. one zero-output entry per padding row.
__global__ void __launch_bounds__(kPlanThreads) plan_kernel(AttnArgs a, Workspace ws) {
  constexpr int P = kChunkTokens;
  __shared__ int s_tmp[kPlanThreads];
  __shared__ int s_bin_start[P];   // first B position of each remainder length
  __shared__ int s_bin_fill[P];
  __shared__ int s_pad_fill;
  const int t = threadIdx.x;
  for (int q = t; q < P; q += kPlanThreads) s_bin_fill[q] = 0;
  if (t == 0) s_pad_fill = 0;
  __syncthreads();

  // pass 1: section A, remainder histogram, pad count
  int total_a = 0, n_pad = 0;
  for (int64_t base = 0; base < a.num_rows; base += kPlanThreads) {
    const int64_t r = base + t;
    int ctx = 0;
    if (r < a.num_rows) ctx = clamp_ctx(a.context_lens[r], a.ctx_limit);
    const int full = ctx / P;
    const int nch = (ctx + P - 1) / P;
    int tile_a, tile_pad;
    const int at = total_a + block_exclusive_scan(full, s_tmp, &tile_a);
    block_exclusive_scan(r < a.num_rows && ctx == 0 ? 1 : 0, s_tmp, &tile_pad);
    for (int k = 0; k < full; ++k) ws.entries[at + k] = make_int4((int)r, k, nch, ctx);
    if (r < a.num_rows && (ctx % P) != 0) atomicAdd(&s_bin_fill[ctx % P], 1);
    total_a += tile_a;
    n_pad += tile_pad;
  }
  __syncthreads();
  // bins of section B in descending remainder order
  int total_b = 0;
  {
    // P <= kPlanThreads: thread q owns remainder P-1-q
    const int q = t;
    const int cnt = q < P ? s_bin_fill[P - 1 - q] : 0;
    const int start = block_exclusive_scan(cnt, s_tmp, &total_b);
    if (q < P) s_bin_start[P - 1 - q] = start;
  }
  for (int q = t; q < P; q += kPlanThreads) s_bin_fill[q] = 0;
  __syncthreads();
  // pass 2: place sections B and C
  for (int64_t r = t; r < a.num_rows; r += kPlanThreads) {
    const int ctx = clamp_ctx(a.context_lens[r], a.ctx_limit);
    const int rem = ctx % P;
    const int nch = (ctx + P - 1) / P;
    if (rem != 0) {
      const int pos = total_a + s_bin_start[rem] + atomicAdd(&s_bin_fill[rem], 1);
      ws.entries[pos] = make_int4((int)r, ctx / P, nch, ctx);
    } else if (ctx == 0) {
      const int pos = total_a + total_b + atomicAdd(&s_pad_fill, 1);
      ws.entries[pos] = make_int4((int)r, -1, 0, 0);
    }
  }
  if (t == 0) {
    ws.counters[0] = total_a + total_b + n_pad;
    ws.counters[1] = 0;
  }
}

// ------------------------------------------------------------------------- //
// decode
// ------------------------------------------------------------------------- //
template <typename T, int D>
struct Shape {
  static constexpr int E = Elem<T>::kPerLane;       // elements per lane load
  static constexpr int LPT = D / E;                 // lanes per token vector
  static constexpr int TPS = 64 / LPT;              // tokens per wave load
  static constexpr int U = (16 / TPS) < 8 ? (16 / TPS) : 8;   // loads per sub-chunk
  static constexpr int CH = TPS * U;                // tokens per sub-chunk
  static_assert(LPT >= 8 && LPT <= 64, "unsupported head_dim/dtype");
  static_assert(kChunkTokens % CH == 0, "chunk must hold whole sub-chunks");
};

template <typename T, int D, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
decode_kernel(AttnArgs a, Workspace ws, float scale_log2) {
  using S = Shape<T, D>;
  using El = Elem<T>;
  constexpr int E = S::E, LPT = S::LPT, TPS = S::TPS, U = S::U, CH = S::CH;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane / LPT;       // which token of a wave load this lane holds
  const int sub = lane % LPT;     // which 16-byte piece of the token's head vector

  __shared__ int s_ticket;
  __shared__ float s_m[WAVES], s_l[WAVES];
  __shared__ float s_acc[WAVES][D];

  const int heads = a.num_heads;
  const int group = heads / a.g.kv_heads;
  const int n_items = ws.counters[0] * heads;
  const int bs_mask = a.g.block_size - 1;

  for (;;) {
    if (threadIdx.x == 0) s_ticket = atomicAdd(&ws.counters[1], 1);
    __syncthreads();
    const int item = s_ticket;
    __syncthreads();
    if (item >= n_items) break;
    const int e = item / heads;
    const int h = item - e * heads;
    const int4 ent = ws.entries[e];
    const int r = ent.x, chunk = ent.y, nch = ent.z, ctx = ent.w;
    const int64_t rh = (int64_t)r * heads + h;
    T* outp = static_cast<T*>(a.out) + rh * D + sub * E;

    if (chunk < 0) {   // padding row: zero output, nothing read
      if (wave == 0 && g == 0) store16(outp, make_uint4(0, 0, 0, 0));
      continue;
    }
    const int t_begin = chunk * kChunkTokens;
    const int t_end = min(ctx, t_begin + kChunkTokens);
    const int hkv = h / group;
    const uint4 qv = load16(static_cast<const T*>(a.q) + rh * D + sub * E);
    const int32_t* bt = a.block_tables + (int64_t)r * a.max_blocks;
    const T* kb = static_cast<const T*>(a.k_cache) + hkv * a.g.head_stride + sub * E;
    const T* vb = static_cast<const T*>(a.v_cache) + hkv * a.g.head_stride + sub * E;

    float m = -INFINITY, l = 0.f;
    float acc[E];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = 0.f;

    const int n_sub = (t_end - t_begin + CH - 1) / CH;
    for (int s = wave; s < n_sub; s += WAVES) {
      const int t0 = t_begin + s * CH;
      int blk = bt[t0 >> a.g.log2_bs];
      const bool blk_ok = blk >= 0 && blk < a.g.num_blocks;
      if (!blk_ok) {
        if (lane == 0) atomicOr(&g_status, PKV_DEVERR_BLOCK_ID);
        blk = 0;
      }
      const int64_t boff = (int64_t)blk * a.g.blk_stride +
                           (int64_t)((t0 & bs_mask) + g) * a.g.tok_stride;
      uint4 kr[U], vr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
        if (blk_ok && t0 + u * TPS + g < t_end) {   // masked tokens are never loaded
          const int64_t off = boff + (int64_t)(u * TPS) * a.g.tok_stride;
          kr[u] = load16(kb + off);
          vr[u] = load16(vb + off);
        }
      }
      float sc[U];
      float smax = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float d = group_sum<LPT>(El::dot(qv, kr[u], 0.f));
        sc[u] = (blk_ok && t0 + u * TPS + g < t_end) ? d * scale_log2 : -INFINITY;
        smax = fmaxf(smax, sc[u]);
      }
      const float m_new = fmaxf(m, smax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = __builtin_amdgcn_exp2f(sc[u] - m_use);
        l += p;
        El::axpy(p, vr[u], acc);
      }
      m = m_new;
    }

    // merge the lane groups of this wave
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      const float m_o = __shfl_xor(m, off);
      const float l_o = __shfl_xor(l, off);
      const float mx = fmaxf(m, m_o);
      const float mu = mx == -INFINITY ? 0.f : mx;
      const float fa = __builtin_amdgcn_exp2f(m - mu);
      const float fb = __builtin_amdgcn_exp2f(m_o - mu);
      l = l * fa + l_o * fb;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] = acc[i] * fa + __shfl_xor(acc[i], off) * fb;
      m = mx;
    }
    // merge the waves of the workgroup
    if constexpr (WAVES > 1) {
      if (g == 0) {
#pragma unroll
        for (int i = 0; i < E; ++i) s_acc[wave][sub * E + i] = acc[i];
        if (sub == 0) {
          s_m[wave] = m;
          s_l[wave] = l;
        }
      }
      __syncthreads();
      if (wave != 0) continue;
      float mx = s_m[0];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) mx = fmaxf(mx, s_m[w]);
      l = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_m[w] - mx);   // mx is finite here
        l += s_l[w] * f;
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] += s_acc[w][sub * E + i] * f;
      }
      m = mx;
    }
    if (g != 0) continue;
    if (nch == 1) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] *= inv;
      store16(outp, El::pack(acc));
    } else {
      float* rec = ws.partials + (rh * ws.max_chunks + chunk) * (D + 4);
      if (sub == 0) {
        rec[0] = m;
        rec[1] = l;
      }
#pragma unroll
      for (int i = 0; i < E; i += 4)
        store16(rec + 4 + sub * E + i, make_uint4(__float_as_uint(acc[i]),
                                                  __float_as_uint(acc[i + 1]),
                                                  __float_as_uint(acc[i + 2]),
                                                  __float_as_uint(acc[i + 3])));
    }
  }
}

// ------------------------------------------------------------------------- //
// combine
// ------------------------------------------------------------------------- //
template <typename T, int D>
__global__ void __launch_bounds__(64) combine_kernel(AttnArgs a, Workspace ws) {
  constexpr int PER = D / 64;     // dims per lane
  const int h = blockIdx.x;
  const int64_t r = blockIdx.y;
  int ctx = a.context_lens[r];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_limit ? a.ctx_limit : ctx);
  const int nch = (ctx + kChunkTokens - 1) / kChunkTokens;
  if (nch <= 1) return;
  const int lane = threadIdx.x;
  const int64_t rh = r * a.num_heads + h;
  const float* rec = ws.partials + rh * ws.max_chunks * (D + 4);
  float mx = -INFINITY;
  for (int c = 0; c < nch; ++c) mx = fmaxf(mx, rec[c * (D + 4)]);
  float l = 0.f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float* p = rec + c * (D + 4);
    const float f = __builtin_amdgcn_exp2f(p[0] - mx);
    l += p[1] * f;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += p[4 + lane * PER + i] * f;
  }
  const float inv = 1.0f / l;
  T* outp = static_cast<T*>(a.out) + rh * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float y = acc[i] * inv;
    if constexpr (sizeof(T) == 4) {
      outp[i] = y;
    } else {
      outp[i] = (uint16_t)(Elem<uint16_t>::cvt2(y, 0.f) & 0xffffu);
    }
  }
}

// ------------------------------------------------------------------------- //
// launchers
// ------------------------------------------------------------------------- //
static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

static int max_chunks_for(int32_t max_blocks, int32_t block_size) {
  const int64_t width = (int64_t)max_blocks * block_size;
  return (int)((width + kChunkTokens - 1) / kChunkTokens);
}

size_t workspace_bytes(int64_t num_rows, int32_t num_heads, int32_t head_dim,
                       int32_t max_blocks, int32_t block_size) {
  const int64_t mc = max_chunks_for(max_blocks, block_size);
  const int64_t entries = num_rows * (mc > 1 ? mc : 1);
  int64_t bytes = align_up(entries * (int64_t)sizeof(int4), 256);
  bytes += 256;   // counters
  bytes += align_up(num_rows * num_heads * mc * (int64_t)(head_dim + 4) * 4, 256);
  return (size_t)bytes;
}

Workspace carve_workspace(void* base, int64_t num_rows, int32_t num_heads, int32_t head_dim,
                          int32_t max_blocks, int32_t block_size) {
  Workspace w;
  const int64_t mc = max_chunks_for(max_blocks, block_size);
  w.max_chunks = (int32_t)mc;
  w.max_entries = num_rows * (mc > 1 ? mc : 1);
  char* p = static_cast<char*>(base);
  w.entries = reinterpret_cast<int4*>(p);
  p += align_up(w.max_entries * (int64_t)sizeof(int4), 256);
  w.counters = reinterpret_cast<int32_t*>(p);
  p += 256;
  w.partials = reinterpret_cast<float*>(p);
  (void)num_heads;
  (void)head_dim;
  return w;
}

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  const int elem = a.g.dtype == PKV_F32 ? 4 : 2;
  const int64_t pieces = a.num_tokens * a.g.kv_heads * (a.g.head_dim * elem / 16);
  const int threads = 256;
  const int64_t blocks = (pieces + threads - 1) / threads;
  const int64_t sink = a.g.num_blocks * a.g.block_size;
  if (a.g.dtype == PKV_F32)
    hipLaunchKernelGGL(kv_write_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, a, sink);
  else
    hipLaunchKernelGGL(kv_write_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, a, sink);
  return hipGetLastError();
}

constexpr int kDecodeWaves = 4;

template <typename T, int D>
static hipError_t launch_decode_t(const AttnArgs& a, const Workspace& ws,
                                  hipStream_t stream) {
  auto kern = decode_kernel<T, D, kDecodeWaves>;
  static int per_cu[64] = {0};   // occupancy per device, computed once
  static int num_cu[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 64) return hipErrorInvalidDevice;
  if (per_cu[dev] == 0) {
    int n = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kDecodeWaves * 64, 0);
    if (err != hipSuccess) return err;
    int cus = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    num_cu[dev] = cus;
    per_cu[dev] = n > 0 ? n : 1;
  }
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, ws);
  int64_t grid = (int64_t)num_cu[dev] * per_cu[dev];
  const int64_t most = ws.max_entries * a.num_heads;
  if (grid > most) grid = most;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kDecodeWaves * 64), 0, stream, a, ws,
                     scale_log2);
  if (ws.max_chunks > 1)
    hipLaunchKernelGGL((combine_kernel<T, D>), dim3(a.num_heads, (unsigned)a.num_rows),
                       dim3(64), 0, stream, a, ws);
  return hipGetLastError();
}

hipError_t launch_paged_attention(const AttnArgs& a, const Workspace& ws,
                                  hipStream_t stream) {
  const bool f32 = a.g.dtype == PKV_F32;
  switch (a.g.head_dim) {
    case 64:
      return f32 ? launch_decode_t<float, 64>(a, ws, stream)
                 : launch_decode_t<uint16_t, 64>(a, ws, stream);
    case 128:
      return f32 ? launch_decode_t<float, 128>(a, ws, stream)
                 : launch_decode_t<uint16_t, 128>(a, ws, stream);
    case 256:
      return f32 ? launch_decode_t<float, 256>(a, ws, stream)
                 : launch_decode_t<uint16_t, 256>(a, ws, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t read_device_status(uint32_t* flags, int clear, hipStream_t stream) {
  hipError_t err = hipMemcpyFromSymbolAsync(flags, HIP_SYMBOL(g_status), sizeof(uint32_t), 0,
                                            hipMemcpyDeviceToHost, stream);
  if (err != hipSuccess) return err;
  err = hipStreamSynchronize(stream);
  if (err != hipSuccess || !clear) return err;
  static const uint32_t zero = 0;
  err = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_status), &zero, sizeof(uint32_t), 0,
                               hipMemcpyHostToDevice, stream);
  if (err != hipSuccess) return err;
  return hipStreamSynchronize(stream);
}

}  // namespace pkv
