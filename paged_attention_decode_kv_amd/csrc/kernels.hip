// gfx950 kernels of the batched paged-attention decode step.
//
//   kv_write_kernel     slot scatter of the step's new K/V (Day 55, "the capture list
//                       moved to startup, and the dummy batch was all padding", "Why it
//                       matters": pad rows write the sink slot)
//   plan_kernel         one workgroup turns context_lens into a work list of
//                       (row, chunk) entries, longest first, and resets the work queue;
//                       plan_write_kernel is the same with the scatter beside it (one
//                       launch for a captured step)
//   decode_kernel       persistent workgroups pull (entry, group of query vectors)
//                       items; each streams its chunk of the row's history through the
//                       block table in 16-token sub-chunks and folds them into online
//                       softmax states on the vector units (Day 59, "the rectangle the
//                       read builds, and the tile that replaces it", "What I added today"
//                       and "What I learned" 3-4); short chunks go one wave each
//   decode_mfma_kernel  the same schedule for groups of 4, 8 or 16 query vectors per
//                       KV head, whose fold is a pair of small matrix products on the
//                       matrix cores
//   combine_kernel      merges the per-chunk (max, denominator, accumulator) partials of
//                       rows longer than one chunk, in chunk order
//   translate_slots_kernel, token_rows_kernel
//                       the read through a per-token slot window (Day 51, "the read
//                       rectangle stopped being built"): block-structured rows become a
//                       derived block table, the rest are read token by token
//
// Lane mapping of one wave (64 lanes) inside the vector-unit decode loop: a (token, KV
// head) vector of head_dim elements is 16-byte pieces spread over LPT consecutive lanes
// (LPT = head_dim * elem_bytes / 16; 16 lanes for bf16 x 128), so one 16-byte load per
// lane moves TPS = 64 / LPT tokens and the load of one wave is a contiguous
// TPS * head_dim run in the HND layout.  Each group of LPT lanes keeps its own online
// softmax state over the tokens it loaded; the q.k partial dot is reduced inside the
// group with DPP row operations, and the groups are merged once per item.  With one
// query vector per KV head the work is a bandwidth-bound streaming read; the matrix
// cores take over where 4 or more vectors share each K/V load.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "internal.h"
#include "pagedkv.h"

namespace pkv {

// PKV_DEVERR_* bits raised since the last clear by any call on this device (see
// pkv_device_status); each call also keeps its own bits in its workspace's counters.
__device__ unsigned int g_status;

// The workspace of pkv_paged_attention_noalloc, one per device.  Host code never uses
// this name as an address (on the host it is a stand-in, not device memory): it uses
// the device address scratch_pointer looks up.  Calls on one device share it.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

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

// Integer sum over the wave, the same steps as group_sum<64>; every lane ends with it.
__device__ __forceinline__ int wave_sum_i(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);   // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);   // row_mirror
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// A step's attention outputs are written once and not read again by this library:
// non-temporal stores (measured: the 16-new-token step 1.261 -> 1.245 ms).  Partial
// records keep ordinary stores, as the combine kernel reads them back.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_out(void* p, const uint4& v) {
  const u32x4_nt x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_nt*>(p));
}
template <typename X>
__device__ __forceinline__ void store_out(X* p, X v) {
  __builtin_nontemporal_store(v, p);
}

// A bad input skipped by a kernel of an attention call: the bit goes to the call's own
// status word (in its workspace) and to the device-wide one.
__device__ __forceinline__ void raise_status(const Workspace& ws, unsigned bits) {
  atomicOr(&g_status, bits);
  atomicOr(reinterpret_cast<unsigned*>(ws.counters + kCtrStatus), bits);
}

// ------------------------------------------------------------------------- //
// slot scatter
// ------------------------------------------------------------------------- //
// 16-byte pieces of the scatter: num_tokens x kv_heads x (head_dim / elements per piece)
template <typename T>
__device__ __forceinline__ int64_t kv_write_pieces(const WriteArgs& a) {
  return a.num_tokens * a.g.kv_heads * (a.g.head_dim / Elem<T>::kPerLane);
}

// Piece idx of the scatter: token idx / per_tok, one KV head's 16 bytes of K and of V.
template <typename T>
__device__ __forceinline__ void kv_write_piece(const WriteArgs& a, int64_t sink, int64_t idx) {
  constexpr int E = Elem<T>::kPerLane;
  const int per_head = a.g.head_dim / E;                 // 16-byte pieces per head vector
  const int64_t per_tok = (int64_t)a.g.kv_heads * per_head;
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

template <typename T>
__global__ void __launch_bounds__(256) kv_write_kernel(WriteArgs a, int64_t sink) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < kv_write_pieces<T>(a)) kv_write_piece<T>(a, sink, idx);
}

// ------------------------------------------------------------------------- //
// plan: context_lens -> work list
// ------------------------------------------------------------------------- //
constexpr int kPlanThreads = 1024;
// Block ids of a work item.  Wave w of a workgroup streams sub-chunks w, w + WAVES,
// w + 2 WAVES, ... of the item's chunk, so lane i of wave w holds the block id of the
// wave's i-th sub-chunk (and of its 64 + i-th, ... in further registers): a chunk of
// kMaxChunkTokens tokens in sub-chunks of CH tokens needs id_regs(CH, WAVES) registers
// a lane (one for 16-token sub-chunks and 8 waves), loaded with one load a lane each.
__host__ __device__ constexpr int id_regs(int ch, int waves) {
  return (kMaxChunkTokens / ch / waves + 63) / 64;
}

// Inclusive prefix sum over the wave with DPP: within each 16-lane row shift-and-add by
// 1, 2, 4 and 8 lanes (lanes with no source add 0), then add row 0's total to row 1 and
// row 2's to row 3 (row_bcast:15), then the first two rows' total to rows 2 and 3
// (row_bcast:31).  Checked against a host prefix sum on the GPU before use.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// exclusive prefix sum of one value per thread over the workgroup (kPlanThreads
// threads); returns the thread's prefix and writes the total to *total.  Without
// sync_after the caller's own next barrier must come before s_wave is written again.
__device__ int block_exclusive_scan(int x, int* s_wave, int* total, bool sync_after = true) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kPlanThreads / 64;
  const int incl = wave_inclusive_scan(x);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int t = lane < kWaves ? s_wave[lane] : 0;
    const int ti = wave_inclusive_scan(t);
    if (lane < kWaves) s_wave[lane] = ti;
  }
  __syncthreads();
  const int prefix = (wave > 0 ? s_wave[wave - 1] : 0) + incl - x;
  *total = s_wave[kWaves - 1];
  if (sync_after) __syncthreads();
  return prefix;
}

// The same for N values per thread at once (one set of barriers): each x[k] becomes the
// thread's exclusive prefix of value k, and total[k] the workgroup's sum of it.
template <int N>
__device__ void block_exclusive_scan_n(int (&x)[N], int (*s_wave)[N], int (&total)[N],
                                       bool sync_after = true) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kPlanThreads / 64;
  int incl[N];
#pragma unroll
  for (int k = 0; k < N; ++k) incl[k] = wave_inclusive_scan(x[k]);
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < N; ++k) s_wave[wave][k] = incl[k];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int v = lane < kWaves ? s_wave[lane][k] : 0;
      const int vi = wave_inclusive_scan(v);
      if (lane < kWaves) s_wave[lane][k] = vi;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int prefix = (wave > 0 ? s_wave[wave - 1][k] : 0) + incl[k] - x[k];
    total[k] = s_wave[kWaves - 1][k];
    x[k] = prefix;
  }
  if (sync_after) __syncthreads();
}

// A row's length as the block path reads it: clamped to what the table addresses (the
// first pass reports a bad length), and 0 for a row of a slot input whose live slots
// are not block structured, which the token-by-token kernel reads instead.
// `status` (the plan's LDS word, or null) collects the bits of bad lengths.
__device__ __forceinline__ int plan_ctx(const AttnArgs& a, int64_t r, int* status,
                                        bool* irregular, int* clamped = nullptr) {
  int ctx = a.context_lens[r];
  if (ctx < 0 || ctx > a.ctx_limit) {
    if (status) atomicOr(status, (int)PKV_DEVERR_CONTEXT_BOUNDS);
    ctx = ctx < 0 ? 0 : a.ctx_limit;
  }
  // a live row shorter than its new tokens: its earliest queries see nothing (zeros)
  if (status && ctx > 0 && ctx < a.query_len) atomicOr(status, (int)PKV_DEVERR_CONTEXT_BOUNDS);
  bool irr = false;
  if (a.row_flags != nullptr && ctx > 0) {
    const int32_t* f = a.row_flags + r * a.flag_stride;
    const int n = (ctx + kTranslateTokens - 1) / kTranslateTokens;
    for (int c = 0; c < n; ++c) irr |= f[c] != 0;
  }
  if (irregular) *irregular = irr;
  if (clamped) *clamped = ctx;
  return irr ? 0 : ctx;
}

// Chooses the chunk length and writes the work list.
//
// The chunk length P is the largest power of two in [chunk_min, chunk_max] whose
// (chunk, head) item count reaches target_items (enough items per decode workgroup
// for the queue to balance) and whose chunk holds at most a third of a workgroup's
// share of the batch's tokens, else chunk_min; then the shortest at least that long
// whose split rows' chunks fit the workspace's a.record_chunks partial records.
// Longer chunks split fewer rows (fewer partial records to write and merge); the share
// bound keeps the longest item short enough for the longest-first order to balance.
// Entries are ordered longest first so that the queue's tail is short work:
//   A. every full chunk (P tokens) of every row, rows in order;
//   B. every row's trailing partial chunk, by length, longest first (in buckets of
//      P / 1024 tokens when P > 1024);
//   C. one zero-output entry per padding row.
// A row longer than P is split: its chunks c = 0, 1, ... own partial records first + c,
// the rows' records laid out in row order (ws.row_rec, ws.split_rows).  The counters
// (enum Counter) are all written here, so the workspace needs no clearing; every row's
// clamped length goes to ws.row_ctx.
__device__ void plan_body(const AttnArgs& a, const Workspace& ws) {
  constexpr int kCand = 7;                 // chunk_max / chunk_min <= kMaxChunkRatio
  static_assert((1 << (kCand - 1)) == kMaxChunkRatio, "one candidate per power of two");
  // Section B is ordered by remainder length in kBins bins (exactly when P <= kBins,
  // else in buckets of P / kBins tokens)
  constexpr int kBins = kPlanThreads;
  // the longest item may take at most 1 / kBalance of a workgroup's share of the work
  constexpr int kBalance = 3;
  __shared__ int s_wave[kPlanThreads / 64];
  __shared__ int s_scan[kPlanThreads / 64][4];
  __shared__ int s_bin_start[kBins];       // first B position of each remainder bin
  __shared__ int s_bin_fill[kBins];
  __shared__ int s_pad_fill;
  __shared__ int s_irregular;
  __shared__ int s_status;
  __shared__ int s_cand[kCand];
  __shared__ int s_spl[kCand];
  __shared__ int s_choice[2];              // chunk length's log2, narrow (8 waves per CU)
  const int t = threadIdx.x;
  const int lane = t & 63;
  if (t < kCand) {
    s_cand[t] = 0;
    s_spl[t] = 0;
  }
  if (t == 0) {
    s_pad_fill = 0;
    s_irregular = 0;
    s_status = 0;
  }
  __syncthreads();

  // pass 0: chunk count and split rows' chunk count of every candidate length; row
  // lengths; irregular rows
  const int lmin = a.log2_chunk_min;
  const int ncand = a.log2_chunk_max - lmin + 1;
  int cnt[kCand], spl[kCand];
#pragma unroll
  for (int k = 0; k < kCand; ++k) cnt[k] = spl[k] = 0;
  // the lengths of this thread's first kKeep rows stay in registers for passes 1 and 2
  constexpr int kKeep = 4;
  int kept[kKeep];
#pragma unroll
  for (int k = 0; k < kKeep; ++k) kept[k] = 0;
  for (int64_t r = t; r < a.num_rows; r += kPlanThreads) {
    bool irr;
    int full_ctx;
    const int ctx = plan_ctx(a, r, &s_status, &irr, &full_ctx);
#pragma unroll
    for (int k = 0; k < kKeep; ++k)
      if (r == t + (int64_t)k * kPlanThreads) kept[k] = ctx;
    // (a row read token by token keeps its length here: its chunks are combined too)
    ws.row_ctx[r] = full_ctx;
    if (irr) ws.irregular[atomicAdd(&s_irregular, 1)] = (int)r;
    // (the chunk length serves the rows read token by token too: counted by their full
    // length, so that a batch of them is not cut into the shortest chunks)
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
      const int n = (full_ctx + (1 << (lmin + k)) - 1) >> (lmin + k);
      cnt[k] += n;
      spl[k] += n > 1 ? n : 0;
    }
  }
  if ((t & ~63) < a.num_rows) {   // a wave without a row adds nothing
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
      if (k >= ncand) break;
      const int v = wave_sum_i(cnt[k]);
      const int vs = wave_sum_i(spl[k]);
      if (lane == 0) {
        atomicAdd(&s_cand[k], v);
        atomicAdd(&s_spl[k], vs);
      }
    }
  }
  static_assert(kBins == kPlanThreads, "one remainder bin per thread");
  s_bin_fill[t] = 0;
  __syncthreads();
  // Workgroups and chunk length.  A batch that gives 8 waves per compute unit enough
  // items of more than the shortest chunk is bandwidth-bound: then 8 waves per CU
  // (fewer concurrent streams) read it fastest.  Enough is narrow_items, or one item
  // per wave when the chunk makes every item a single-wave one (then each wave is one
  // stream).  Otherwise every workgroup takes part, with the chunk length that gives
  // them all enough items.
  const int64_t per_entry = a.query_len * a.num_heads / a.query_group;
  // Wave 0 chooses alone (the counts are workgroup-uniform: scalar registers) and
  // publishes the choice; the other waves wait at the barrier.
  if (t < 64) {
    int cand[kCand], cand_spl[kCand];   // candidates past ncand hold 0
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
      cand[k] = __builtin_amdgcn_readfirstlane(s_cand[k]);
      cand_spl[k] = __builtin_amdgcn_readfirstlane(s_spl[k]);
    }
    // Balance: with G workgroups, the largest candidate whose chunks hold at most
    // 1 / kBalance of a workgroup's share (tokens x items per entry / G); the work list
    // runs longest first, so the last items to start are short ones.  The batch's tokens
    // are taken as its chunk_min chunks x chunk_min (over by less than a chunk a row).
    const int64_t work = ((int64_t)cand[0] << lmin) * per_entry;
    auto balance_cap = [&](int64_t groups) {
      int kc = 0;
#pragma unroll
      for (int k = 1; k < kCand; ++k)
        if (k < ncand && (int64_t{1} << (lmin + k)) * kBalance * groups <= work) kc = k;
      return kc;
    };
    int lp = lmin;
    bool narrow = false;
    if (a.narrow_groups > 0) {
      const int kmax = min(ncand - 1, balance_cap(a.narrow_groups));
#pragma unroll
      for (int k = kCand - 1; k > 0; --k) {
        const int64_t items = (int64_t)cand[k] * per_entry;
        // chunks shorter than solo_tokens are all single-wave items, which need only
        // kSoloPerWave of them for each wave, not narrow_items for the workgroups
        const bool solo = a.solo_tokens > 1 && (1 << (lmin + k)) < a.solo_tokens &&
                          items >= (int64_t)kSoloPerWave * a.narrow_groups * a.group_waves;
        if (!narrow && k <= kmax && (items >= a.narrow_items || solo)) {
          lp = lmin + k;
          narrow = true;
        }
      }
    }
    if (!narrow) {
      // A batch too small to give every workgroup its share even at the shortest chunk
      // takes the longest that gives a quarter of it: each extra split of a row costs a
      // float32 partial record per vector, and the shortest chunk splits the most.
      const int kc = min(ncand - 1, balance_cap(a.grid_groups));
      int found = -1;
#pragma unroll
      for (int k = kCand - 1; k >= 0; --k)
        if (found < 0 && k <= kc && (int64_t)cand[k] * per_entry >= a.target_items) found = k;
#pragma unroll
      for (int k = kCand - 1; k >= 0; --k)
        if (found < 0 && k <= kc && (int64_t)cand[k] * per_entry >= a.target_items / 4)
          found = k;
      lp = lmin + (found > 0 ? found : 0);
    }
    // the split rows' partial records must fit the workspace (they always do at the
    // longest candidate, which the workspace is sized for)
#pragma unroll
    for (int k = 0; k < kCand - 1; ++k)
      if (k == lp - lmin && k < ncand - 1 && cand_spl[k] > a.record_chunks) ++lp;
    if (t == 0) {
      s_choice[0] = lp;
      s_choice[1] = narrow ? 1 : 0;
    }
  }
  __syncthreads();
  const int lp = s_choice[0];
  const bool narrow = s_choice[1] != 0;
  const int P = 1 << lp;
  const int bshift = lp > 10 ? lp - 10 : 0;   // remainder -> bin (kBins = 1024)
  const int nbins = P >> bshift;
  static_assert(kBins == 1024, "bin shift assumes 1024 bins");

  // a row's length as pass 0 found it
  auto row_len = [&](int64_t r) {
    const int64_t k = (r - t) / kPlanThreads;
    int v = 0;
#pragma unroll
    for (int i = 0; i < kKeep; ++i)
      if (k == i) v = kept[i];
    return k < kKeep ? v : plan_ctx(a, r, nullptr, nullptr);
  };

  // pass 1: section A; the split rows in row order, with their first partial records;
  // remainder histogram; pad count
  int total_a = 0, n_pad = 0, total_rec = 0, n_split = 0;
  int kept_rec[kKeep];
#pragma unroll
  for (int k = 0; k < kKeep; ++k) kept_rec[k] = -1;
  for (int64_t base = 0; base < a.num_rows; base += kPlanThreads) {
    const int64_t r = base + t;
    const bool in = r < a.num_rows;
    const int ctx = in ? row_len(r) : 0;
    // a row read token by token (slot input) splits by its full length
    const int fl = in ? (a.row_flags != nullptr ? ws.row_ctx[r] : ctx) : 0;
    const int fnch = (fl + P - 1) >> lp;
    const bool split = fnch > 1;
    const int full = ctx >> lp;
    int v[4] = {full, in && ctx == 0 ? 1 : 0, split ? fnch : 0, split ? 1 : 0};
    int tot[4];
    // (the last round's scan needs no closing barrier: the loop's own follows)
    block_exclusive_scan_n<4>(v, s_scan, tot, base + kPlanThreads < a.num_rows);
    const int rec0 = split ? total_rec + v[2] : -1;
    for (int k = 0; k < full; ++k)
      ws.entries[total_a + v[0] + k] = make_int4((int)r, k, split ? rec0 + k : -1, ctx);
    if (in) {
      ws.row_rec[r] = rec0;
      const int64_t kk = base / kPlanThreads;
#pragma unroll
      for (int i = 0; i < kKeep; ++i)
        if (kk == i) kept_rec[i] = rec0;
    }
    if (split) ws.split_rows[n_split + v[3]] = make_int4((int)r, fl, rec0, 0);
    if (in && (ctx & (P - 1)) != 0) atomicAdd(&s_bin_fill[(ctx & (P - 1)) >> bshift], 1);
    total_a += tot[0];
    n_pad += tot[1];
    total_rec += tot[2];
    n_split += tot[3];
  }
  __syncthreads();
  // bins of section B in descending remainder order: thread t owns the t-th from the top
  int total_b = 0;
  {
    const int bin = nbins - 1 - t;
    const int count = t < nbins ? s_bin_fill[bin] : 0;
    const int start = block_exclusive_scan(count, s_wave, &total_b, false);
    if (t < nbins) {
      s_bin_start[bin] = start;
      s_bin_fill[t] = 0;   // every count was read before the scan's first barrier
    }
  }
  __syncthreads();
  // pass 2: place sections B and C
  for (int64_t r = t; r < a.num_rows; r += kPlanThreads) {
    const int ctx = row_len(r);
    const int rem = ctx & (P - 1);
    if (rem != 0) {
      const int64_t k = (r - t) / kPlanThreads;
      int rec0 = 0;
#pragma unroll
      for (int i = 0; i < kKeep; ++i)
        if (k == i) rec0 = kept_rec[i];
      if (k >= kKeep) rec0 = ws.row_rec[r];   // written by this thread in pass 1
      const int chunk = ctx >> lp;
      const int pos = total_a + s_bin_start[rem >> bshift] +
                      atomicAdd(&s_bin_fill[rem >> bshift], 1);
      ws.entries[pos] = make_int4((int)r, chunk, rec0 >= 0 ? rec0 + chunk : -1, ctx);
    } else if (ctx == 0) {
      const int pos = total_a + total_b + atomicAdd(&s_pad_fill, 1);
      ws.entries[pos] = make_int4((int)r, -1, -1, 0);
    }
  }
  __syncthreads();
  // Entries before the single-wave items: section A if its chunks are not short, and
  // the B bins of remainders >= solo_tokens (bin b holds [b, b + 1) << bshift, and
  // solo_tokens is a multiple of 1 << bshift: a power of two >= 32 against <= 8).  Read
  // from the bins before the token rows below reuse them.
  int n_wide = total_a + total_b;
  if (a.solo_tokens > 1) {
    if (P < a.solo_tokens) {
      n_wide = 0;
    } else {
      const int tb = a.solo_tokens >> bshift;   // first bin of the long remainders
      n_wide = total_a + (tb >= nbins ? 0 : s_bin_start[tb - 1]);
    }
    // too few to keep every wave streaming: all items go wide
    const int64_t waves = (int64_t)(narrow ? a.narrow_groups : a.grid_groups) * a.group_waves;
    if ((int64_t)(total_a + total_b - n_wide) * per_entry < kSoloPerWave * waves)
      n_wide = total_a + total_b;
  }
  // The rows read token by token (slot input): their chunks, longest first, for the
  // token kernel's shared queue, as sections A and B are for the block path: every full
  // chunk, then the trailing partial chunks by length, descending (bins as for B).
  int total_ta = 0, total_tb = 0, n_tok_wide = 0;
  const int n_irr = s_irregular;
  if (n_irr > 0 && ws.token_entries != nullptr) {
    if (t < nbins) s_bin_fill[t] = 0;
    __syncthreads();
    for (int base = 0; base < n_irr; base += kPlanThreads) {
      const int i = base + t;
      const int r = i < n_irr ? ws.irregular[i] : 0;
      const int full = i < n_irr ? ws.row_ctx[r] : 0;
      const int nfull = full >> lp;
      int tile;
      const int at = total_ta + block_exclusive_scan(nfull, s_wave, &tile);
      for (int k = 0; k < nfull; ++k) ws.token_entries[at + k] = make_int2(r, k);
      if ((full & (P - 1)) != 0) atomicAdd(&s_bin_fill[(full & (P - 1)) >> bshift], 1);
      total_ta += tile;
    }
    __syncthreads();
    {
      const int bin = nbins - 1 - t;
      const int count = t < nbins ? s_bin_fill[bin] : 0;
      const int start = block_exclusive_scan(count, s_wave, &total_tb);
      if (t < nbins) s_bin_start[bin] = start;
    }
    __syncthreads();
    if (t < nbins) s_bin_fill[t] = 0;
    __syncthreads();
    for (int i = t; i < n_irr; i += kPlanThreads) {
      const int r = ws.irregular[i];
      const int full = ws.row_ctx[r];
      const int rem = full & (P - 1);
      if (rem != 0)
        ws.token_entries[total_ta + s_bin_start[rem >> bshift] +
                         atomicAdd(&s_bin_fill[rem >> bshift], 1)] = make_int2(r, full >> lp);
    }
    // entries before the chunks shorter than solo_tokens, which token_rows_short_kernel
    // reads one wave each, if there are at least kSoloPerWave for each of its waves
    n_tok_wide = total_ta + total_tb;
    if (a.solo_tokens > 1) {
      const int tb = a.solo_tokens >> bshift;
      n_tok_wide = P < a.solo_tokens ? 0 : total_ta + (tb >= nbins ? 0 : s_bin_start[tb - 1]);
      if ((int64_t)(total_ta + total_tb - n_tok_wide) * a.num_heads <
          (int64_t)kSoloPerWave * a.token_waves)
        n_tok_wide = total_ta + total_tb;
    }
    __syncthreads();
  }
  if (t == 0) {
    int* c = ws.counters;
    c[kCtrEntries] = total_a + total_b + n_pad;
    c[kCtrTicket] = 0;
    c[kCtrChunk] = P;
    c[kCtrLog2Chunk] = lp;
    c[kCtrSectionA] = total_a;
    c[kCtrData] = total_a + total_b;
    c[kCtrTokenRows] = s_irregular;
    c[kCtrGroups] = narrow ? a.narrow_groups : a.grid_groups;
    c[kCtrSplitRows] = n_split;
    c[kCtrTokenEntries] = total_ta + total_tb;
    c[kCtrWide] = n_wide;
    c[kCtrTokenTicket] = 0;
    c[kCtrTokenWide] = n_tok_wide;
    // this call's status starts with the plan's own findings
    c[kCtrStatus] = s_status;
    c[kCtrWalked] = 0;
    c[kCtrWalked + 1] = 0;
    c[kCtrTileTokens] = 0;
    c[kCtrVectorGroups] = 0;
    c[kCtrRecords] = total_rec;
    c[kCtrRecordCap] = a.record_chunks;
    if (s_status != 0) atomicOr(&g_status, (unsigned)s_status);
  }
}

__global__ void __launch_bounds__(kPlanThreads) plan_kernel(AttnArgs a, Workspace ws) {
  plan_body(a, ws);
}

// A captured step's first kernel: workgroup 0 plans the read while the others scatter
// the step's new K/V (neither reads what the other writes; the decode kernel, launched
// after it, reads both).
template <typename T>
__global__ void __launch_bounds__(kPlanThreads) plan_write_kernel(AttnArgs a, Workspace ws,
                                                                  WriteArgs w, int64_t sink) {
  if (blockIdx.x == 0) {
    plan_body(a, ws);
    return;
  }
  const int64_t n = kv_write_pieces<T>(w);
  const int64_t stride = (int64_t)(gridDim.x - 1) * kPlanThreads;
  for (int64_t idx = (int64_t)(blockIdx.x - 1) * kPlanThreads + threadIdx.x; idx < n;
       idx += stride)
    kv_write_piece<T>(w, sink, idx);
}

// ------------------------------------------------------------------------- //
// decode
// ------------------------------------------------------------------------- //
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// K/V are read once per step: non-temporal loads keep them from displacing
// anything in the caches and measurably raise the achieved HBM read rate.
__device__ __forceinline__ uint4 load16_stream(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T, int D>
struct Shape {
  static constexpr int E = Elem<T>::kPerLane;       // elements per lane load
  static constexpr int LPT = D / E;                 // lanes per token vector
  static constexpr int TPS = 64 / LPT;              // tokens per wave load
  static constexpr int U = (16 / TPS) < 4 ? (16 / TPS) : 4;   // wave loads per sub-chunk
  static constexpr int CH = TPS * U;                // tokens per sub-chunk (<= 16)
  static_assert(LPT >= 8 && LPT <= 64, "unsupported head_dim/dtype");
  static_assert(kMinChunkTokens % CH == 0 && 16 % CH == 0, "sub-chunks tile chunks and blocks");
};

// Query vectors.  A row has query_len x heads of them, one per (new token i, query
// head h), numbered v = h * query_len + i: the vectors of one KV head are consecutive
// (KV head of v = v / (query_len * heads per KV head)).  With one new token per row,
// v = h.  Vector v's q and out are [row][i][h][:]; query i sits at position
// len - query_len + i and sees positions up to its own.
__device__ __forceinline__ int64_t vec_slot(const AttnArgs& a, int64_t r, int v) {
  const int h = v / a.query_len;
  const int i = v - h * a.query_len;
  return (r * a.query_len + i) * a.num_heads + h;
}
__device__ __forceinline__ int vec_query(const AttnArgs& a, int v) {
  return v % a.query_len;
}

// Everything a work item needs before its first K/V load.  An item is (row, chunk of
// the row's history, group of QG query vectors that share one KV head).
template <int QG, int NR>
struct ItemMeta {
  // hg: vector group (vectors hg*QG .. hg*QG + QG - 1); rec: the chunk's partial record
  // (-1: the row is one chunk)
  int r, hg, chunk, rec, ctx;
  uint4 q[QG];   // this lane's 16 bytes of each vector's query
  int last[QG];  // each vector's last visible position (len - query_len + i)
  int blk[NR];   // lane i: block id of this wave's sub-chunks i, 64 + i, ...
};

// The block ids of this wave's sub-chunks of an item's chunk (see id_regs): lane i of
// register k holds the id of sub-chunk wave + WAVES (64 k + i).  Loads past the chunk's
// last sub-chunk are not issued.
template <int NR, int CH, int WAVES>
__device__ __forceinline__ void load_chunk_blocks(const AttnArgs& a, int r, int chunk, int ctx,
                                                  int lp, int log2_bs, int lane, int wave,
                                                  int (&blk)[NR]) {
  const int t_begin = chunk << lp;
  const int n_sub = (min(ctx, t_begin + (1 << lp)) - t_begin + CH - 1) / CH;
  const int32_t* bt = a.block_tables + (int64_t)r * a.max_blocks;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if (wave + WAVES * 64 * k >= n_sub) break;   // uniform
    const int s = wave + WAVES * (64 * k + lane);
    if (s < n_sub) blk[k] = bt[(t_begin + s * CH) >> log2_bs];
  }
}

// First half of fetching an item's metadata: the work-list entry load is issued and
// its value is not consumed, so no wait is inserted here.
__device__ __forceinline__ int4 issue_entry(const Workspace& ws, int item, int groups) {
  return ws.entries[item / groups];
}

// Second half: the entry becomes wave-uniform and the query and block-id loads are
// issued (they complete while the current item finishes).
template <typename T, int D, int QG, int NR, int CH, int WAVES>
__device__ __forceinline__ ItemMeta<QG, NR> finish_meta(const AttnArgs& a, int4 ent, int item,
                                                   int lp, int log2_bs, int lane, int sub,
                                                   int wave) {
  constexpr int E = Elem<T>::kPerLane;
  const int groups = a.query_len * a.num_heads / QG;
  ItemMeta<QG, NR> m;
  const int e = item / groups;
  m.hg = item - e * groups;
  m.r = __builtin_amdgcn_readfirstlane(ent.x);
  m.chunk = __builtin_amdgcn_readfirstlane(ent.y);
  m.rec = __builtin_amdgcn_readfirstlane(ent.z);
  m.ctx = __builtin_amdgcn_readfirstlane(ent.w);
#pragma unroll
  for (int j = 0; j < QG; ++j) {
    m.q[j] = make_uint4(0, 0, 0, 0);
    m.last[j] = m.ctx - a.query_len + vec_query(a, m.hg * QG + j);
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) m.blk[k] = 0;
  if (m.chunk >= 0) {
#pragma unroll
    for (int j = 0; j < QG; ++j)
      m.q[j] = load16(static_cast<const T*>(a.q) + vec_slot(a, m.r, m.hg * QG + j) * D +
                      sub * E);
    load_chunk_blocks<NR, CH, WAVES>(a, m.r, m.chunk, m.ctx, lp, log2_bs, lane, wave, m.blk);
  }
  return m;
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferFlags = 0x00020000;   // raw 32-bit buffer (gfx9 word 3)
constexpr int kLoadNonTemporal = 2;        // cache policy: nt
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0,15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int kWaitVm0 = 0x0F70;           // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;         // lgkmcnt(0)

// 16 bytes at byte `voff` of a buffer into LDS: lane i's bytes land at dst + 16 i.
// Out-of-range offsets write zeros and read no memory.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                                  uint4* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, kLoadNonTemporal);
}

// 16 bytes at byte `voff` of a buffer.  Offsets at or past the descriptor's record
// count read as zero without a memory access: that is how masked tokens are skipped.
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, 0, kLoadNonTemporal);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Sub-chunk addressing of one work item, shared by the decode kernels.  describe()
// builds the buffer descriptors of sub-chunk s's K and V; they end after its valid
// tokens, so the loads of masked tokens never reach memory.  A block id outside the
// pool is skipped (no valid tokens) and noted in `bad`.
struct ChunkAddr {
  const char* kpool;
  const char* vpool;
  int64_t head_off, blk_bytes, tok_bytes;
  int t_begin, t_end, bs_mask;
  int64_t num_blocks;

  // sub-chunk s is the calling wave's i-th; blk: the wave's ids (load_chunk_blocks)
  template <int CH, int NR>
  __device__ __forceinline__ int describe(int s, int i, __amdgpu_buffer_rsrc_t& ksrc,
                                          __amdgpu_buffer_rsrc_t& vsrc, bool& bad,
                                          const int (&blk)[NR]) const {
    const int t0 = t_begin + s * CH;
    // (i is wave-uniform: each register is read at lane i % 64 and the scalar results
    // are selected, so the id registers are never indexed)
    int raw = __builtin_amdgcn_readlane(blk[0], i & 63);
#pragma unroll
    for (int k = 1; k < NR; ++k) {
      const int rk = __builtin_amdgcn_readlane(blk[k], i & 63);
      raw = (i >> 6) == k ? rk : raw;
    }
    const bool blk_ok = raw >= 0 && raw < num_blocks;
    bad |= !blk_ok;
    const int id = blk_ok ? raw : 0;
    const int64_t off = head_off + (int64_t)id * blk_bytes + (int64_t)(t0 & bs_mask) * tok_bytes;
    const int nvalid = blk_ok ? min(CH, t_end - t0) : 0;
    const int bytes = (int)(nvalid * tok_bytes);
    ksrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kpool + off), 0, bytes,
                                             kBufferFlags);
    vsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vpool + off), 0, bytes,
                                             kBufferFlags);
    return nvalid;
  }
};

// The workgroup's place in the item order.  Workgroups are dispatched to the 8 XCDs
// round robin (workgroup b on XCD b % 8), each XCD with its own L2; numbering them XCD
// by XCD gives consecutive items, the query heads of one row chunk, to one XCD, which
// then fetches that chunk's block ids and queries once.  Measured 0.2-1.1 % faster on
// the long-gather batches; any permutation is correct.
__device__ __forceinline__ int xcd_order(int G) {
  const int b = blockIdx.x;
  if (G % 8 != 0) return b;
  return (b % 8) * (G / 8) + b / 8;
}

// Item order of the persistent decode kernels: whole rounds of the full chunks
// (section A) are dealt round robin, workgroup g taking items g, g + G, ...; the rest
// come from one shared ticket counter (n_dealt + ticket; anything at or past the data
// items ends the stream).
struct ItemOrder {
  int static_next, stride, n_dealt;
  __device__ __forceinline__ bool take(int& out) {   // true: a dealt item was taken
    if (static_next < n_dealt) {
      out = static_next;
      static_next += stride;
      return true;
    }
    return false;
  }
  // The first two items of a workgroup (all threads; may pass two barriers).
  __device__ __forceinline__ void first_two(int& item, int& next, int32_t* ticket,
                                            int* s_ticket) {
    const bool st0 = take(item);
    const bool st1 = take(next);
    if (!st0 || !st1) {
      if (threadIdx.x == 0) {
        s_ticket[0] = st0 ? 0 : atomicAdd(ticket, 1);
        s_ticket[1] = st1 ? 0 : atomicAdd(ticket, 1);
      }
      __syncthreads();
      if (!st0) item = n_dealt + __builtin_amdgcn_readfirstlane(s_ticket[0]);
      if (!st1) next = n_dealt + __builtin_amdgcn_readfirstlane(s_ticket[1]);
      __syncthreads();
    }
  }
};

// Fold one sub-chunk (this lane's 16 bytes of U wave loads of K and of V) into the
// online-softmax state of every vector of a group.  `nvalid` of its tokens are live;
// vector j sees positions up to last_rel[j] (relative to the chunk start): the causal
// limit of several new tokens.  Scores are in log2 units (scale_log2 = scale * log2 e).
template <typename T, int D, int QG>
__device__ __forceinline__ void fold_sub_chunk(const uint4 (&kr)[Shape<T, D>::U],
                                               const uint4 (&vr)[Shape<T, D>::U], int nvalid,
                                               int s, int g, const int (&last_rel)[QG],
                                               const uint4 (&q)[QG], float scale_log2,
                                               float (&m)[QG], float (&l)[QG],
                                               float (&acc)[QG][Shape<T, D>::E]) {
  using S = Shape<T, D>;
  using El = Elem<T>;
  constexpr int E = S::E, LPT = S::LPT, TPS = S::TPS, U = S::U, CH = S::CH;
#pragma unroll
  for (int j = 0; j < QG; ++j) {
    const int nv = min(nvalid, last_rel[j] - s * CH + 1);
    float sc[U];
    float smax = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float d = group_sum<LPT>(El::dot(q[j], kr[u], 0.f));
      sc[u] = u * TPS + g < nv ? d * scale_log2 : -INFINITY;
      smax = fmaxf(smax, sc[u]);
    }
    const float m_new = fmaxf(m[j], smax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m[j] - m_use);
    l[j] *= alpha;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[j][i] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = __builtin_amdgcn_exp2f(sc[u] - m_use);
      l[j] += p;
      El::axpy(p, vr[u], acc[j]);
    }
    m[j] = m_new;
  }
}

// Merge the online-softmax states of the lane groups of one wave (groups of LPT lanes
// that loaded different tokens), vector by vector; every group ends with the merge.
template <int LPT, int QG, int E>
__device__ __forceinline__ void merge_lane_groups(float (&m)[QG], float (&l)[QG],
                                                  float (&acc)[QG][E]) {
#pragma unroll
  for (int j = 0; j < QG; ++j) {
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      const float m_o = __shfl_xor(m[j], off);
      const float l_o = __shfl_xor(l[j], off);
      const float mx = fmaxf(m[j], m_o);
      const float mu = mx == -INFINITY ? 0.f : mx;
      const float fa = __builtin_amdgcn_exp2f(m[j] - mu);
      const float fb = __builtin_amdgcn_exp2f(m_o - mu);
      l[j] = l[j] * fa + l_o * fb;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[j][i] = acc[j][i] * fa + __shfl_xor(acc[j][i], off) * fb;
      m[j] = mx;
    }
  }
}

// Float offset of query vector v's partial record of chunk record `rec` (records of
// one chunk hold every vector of the row).
template <int D>
__device__ __forceinline__ int64_t record_offset(int rec, int n_vec, int v) {
  return ((int64_t)rec * n_vec + v) * (D + 4);
}

// The finished state of query vector v of row r over one chunk, written by the LPT
// lanes of one lane group (this lane's piece `sub`): the output (a row of one chunk,
// rec < 0: acc / l, zeros where nothing was visible) or the chunk's partial record
// (m, l, acc) for the combine kernel.
template <typename T, int D>
__device__ __forceinline__ void write_item_result(const AttnArgs& a, const Workspace& ws,
                                                  int r, int v, int rec, int n_vec,
                                                  int sub, float mj, float lj,
                                                  float (&aj)[Elem<T>::kPerLane]) {
  constexpr int E = Elem<T>::kPerLane;
  if (rec < 0) {
    const float inv = lj > 0.f ? 1.0f / lj : 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) aj[i] *= inv;
    store16_out(static_cast<T*>(a.out) + vec_slot(a, r, v) * D + sub * E, Elem<T>::pack(aj));
  } else {
    float* p = ws.partials + record_offset<D>(rec, n_vec, v);
    if (sub == 0) {
      p[0] = mj;
      p[1] = lj;
    }
#pragma unroll
    for (int i = 0; i < E; i += 4)
      store16(p + 4 + sub * E + i, make_uint4(__float_as_uint(aj[i]), __float_as_uint(aj[i + 1]),
                                              __float_as_uint(aj[i + 2]),
                                              __float_as_uint(aj[i + 3])));
  }
}

// The sub-chunks a workgroup streamed (each wave's count in s_walk[wave]), added to the
// call's counter once per workgroup: the kernel's own loop count, which the tests hold
// against the host's tile accounting.  All waves of the workgroup call this.
template <int WAVES>
__device__ __forceinline__ void report_walked(const Workspace& ws, int* s_walk, int walked) {
  if ((threadIdx.x & 63) == 0) s_walk[threadIdx.x >> 6] = walked;
  __syncthreads();
  if (threadIdx.x == 0) {
    int sum = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += s_walk[w];
    if (sum != 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(ws.counters + kCtrWalked),
                (unsigned long long)sum);
  }
}

// Block-id registers of a single-wave item (its chunk has fewer than kMaxSoloTokens
// tokens, all of its sub-chunks read by one wave).
__host__ __device__ constexpr int solo_id_regs(int ch) {
  return (kMaxSoloTokens / ch + 63) / 64;
}

// The decode read.  Persistent workgroups process work items; an item is (chunk of a
// row's history, group of QG query heads sharing one KV head).
//
// Wide items: the waves of a workgroup share the item, wave w folding sub-chunks w,
// w + WAVES, ... into its own online-softmax state of every head of the group before
// the waves are merged through LDS.  With grouped-query attention one K/V load serves
// QG query heads.  Whole rounds of the full chunks (section A, all the same length)
// are dealt round robin, workgroup g taking items g, g + G, g + 2G, ...; the rest of A
// and the trailing partial chunks (section B, longest first) come from one shared
// ticket counter, so the uneven tail is balanced dynamically with few atomics.  The
// next item's metadata and the ticket after it are fetched while the current item
// streams.
//
// Single-wave items: chunks shorter than a.solo_tokens (the tail of section B, or every
// item when the chunk length itself is shorter; the plan keeps them only when there are
// at least kSoloPerWave for every wave) are read first, by one wave each, dealt round
// robin over every wave of the launch.  A short chunk shared by 8 waves leaves most of
// them idle at its last round and pays a workgroup merge and barrier per few
// sub-chunks; alone, a wave streams its items back to back: the next item's metadata
// loads while the current one streams, and its first sub-chunk is staged while the
// current item's last one is folded.  A single wave takes ~8x as long over one item, so
// these go before the wide items, whose shared queue evens out the workgroups'
// finishing times.
//
// Padding rows (section C) are zeroed round robin at the end.
template <typename T, int D, int WAVES, bool LDS_STAGE, int QG>
__global__ void __launch_bounds__(WAVES * 64)
decode_kernel(AttnArgs a, Workspace ws, float scale_log2) {
  using S = Shape<T, D>;
  constexpr int E = S::E, LPT = S::LPT, TPS = S::TPS, U = S::U, CH = S::CH;
  constexpr int NR = id_regs(CH, WAVES);
  constexpr int NRS = solo_id_regs(CH);
  using Meta = ItemMeta<QG, NR>;
  using MetaS = ItemMeta<QG, NRS>;
  constexpr int ES = sizeof(T);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane / LPT;       // which token of a wave load this lane holds
  const int sub = lane % LPT;     // which 16-byte piece of the token's head vector

  // LDS staging: each wave owns one sub-chunk stage (its U K loads, then its U V loads,
  // 64 lanes x 16 bytes each); the next sub-chunk streams into it by direct
  // buffer-to-LDS loads while the current one is folded from registers.
  constexpr int kStageWaves = LDS_STAGE ? WAVES : 1;
  constexpr int kStageLoads = LDS_STAGE ? 2 * U : 1;
  __shared__ __attribute__((aligned(16))) uint4 s_stage[kStageWaves][kStageLoads][64];
  __shared__ int s_ticket[2];
  __shared__ float s_m[2][QG][WAVES], s_l[2][QG][WAVES];
  __shared__ float s_acc[2][QG][WAVES][D];
  __shared__ int s_walk[WAVES];

  const int n_vec = a.query_len * a.num_heads;   // query vectors per row
  const int groups = n_vec / QG;                 // items per work-list entry
  const int vpkv = n_vec / a.g.kv_heads;         // query vectors per KV head
  const int lp = ws.counters[3];
  const int P = 1 << lp;
  const int n_wide = ws.counters[10] * groups;    // items before the single-wave ones
  const int n_data = ws.counters[5] * groups;     // sections A and B
  const int n_items = ws.counters[0] * groups;
  const int G = ws.counters[7];                  // workgroups taking part
  if ((int)blockIdx.x >= G) return;
  if (blockIdx.x == 0 && threadIdx.x == 0) {     // what the walk count is counted in
    ws.counters[kCtrTileTokens] = CH;
    ws.counters[kCtrVectorGroups] = groups;
  }
  const int n_static = min(ws.counters[4] * groups, n_wide);   // section A items
  const int n_dealt = a.deal_static ? n_static / G * G : 0;
  const int log2_bs = a.g.log2_bs;
  const int bs_mask = a.g.block_size - 1;
  const int64_t tok_bytes = a.g.tok_stride * ES;
  const int64_t blk_bytes = a.g.blk_stride * ES;
  const int64_t head_bytes = a.g.head_stride * ES;
  int walked = 0;   // sub-chunks this wave streamed (wide items: wave 0 counts each once)
  // byte offset of this lane's 16 bytes in the u-th wave load of a sub-chunk
  uint32_t voff[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    voff[u] = (uint32_t)((u * TPS + g) * tok_bytes + sub * E * ES);
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  bool bad_block = false;   // a live block id outside [0, num_blocks) was skipped

  // addressing of an item's sub-chunks (its fields are wave-uniform; saying so keeps the
  // load descriptors scalar)
  auto chunk_addr = [&](int chunk, int hg, int ctx) {
    const int t_begin = chunk * P;
    return ChunkAddr{kpool, vpool, (int64_t)(hg * QG / vpkv) * head_bytes, blk_bytes,
                     tok_bytes, t_begin, min(ctx, t_begin + P), bs_mask, a.g.num_blocks};
  };
  // this wave's LDS stage <- sub-chunk s of an item
  auto stage_from = [&](const ChunkAddr& ca, int s, int i, auto& blk) {
    __amdgpu_buffer_rsrc_t ksrc, vsrc;
    ca.describe<CH>(s, i, ksrc, vsrc, bad_block, blk);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      buffer_load16_lds(ksrc, voff[u], &s_stage[wave][u][0]);
      buffer_load16_lds(vsrc, voff[u], &s_stage[wave][U + u][0]);
    }
  };
  // sub-chunk s of an item into registers: from the stage (then the stage is free), or
  // straight from memory; returns its live tokens
  auto fetch = [&](const ChunkAddr& ca, int s, int i, auto& blk, uint4 (&kr)[U],
                   uint4 (&vr)[U]) {
    __amdgpu_buffer_rsrc_t ksrc, vsrc;
    const int nvalid = ca.describe<CH>(s, i, ksrc, vsrc, bad_block, blk);
    if constexpr (LDS_STAGE) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);          // this wave's stage has landed
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = s_stage[wave][u][lane];
        vr[u] = s_stage[wave][U + u][lane];
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);        // stage read before it is refilled
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = buffer_load16(ksrc, voff[u]);
        vr[u] = buffer_load16(vsrc, voff[u]);
      }
    }
    return nvalid;
  };

  // ---- single-wave items first: [n_wide, n_data), wave k of the launch takes n_wide + k,
  // n_wide + k + G * WAVES, ...; the wide items' shared queue then evens out the
  // workgroups' finishing times ----
  {
    const int stride = G * WAVES;
    int it = n_wide + xcd_order(G) * WAVES + wave;
    MetaS sc;
    int4 ent_nx = make_int4(0, -1, 0, 0);
    if (it < n_data) {
      sc = finish_meta<T, D, QG, NRS, CH, 1>(a, issue_entry(ws, it, groups), it, lp, log2_bs,
                                             lane, sub, 0);
      if (it + stride < n_data) ent_nx = issue_entry(ws, it + stride, groups);
    }
    bool staged = false;   // the item's first sub-chunk is already in the stage
    while (it < n_data) {
      const int nx = it + stride;
      // the next item's query and block ids, and the entry after it, load while this
      // item streams
      MetaS sn = finish_meta<T, D, QG, NRS, CH, 1>(a, ent_nx, nx, lp, log2_bs, lane, sub, 0);
      ent_nx = nx + stride < n_data ? issue_entry(ws, nx + stride, groups)
                                    : make_int4(0, -1, 0, 0);

      const int chunk = __builtin_amdgcn_readfirstlane(sc.chunk);
      const int hg = __builtin_amdgcn_readfirstlane(sc.hg);
      const ChunkAddr ca = chunk_addr(chunk, hg, __builtin_amdgcn_readfirstlane(sc.ctx));
      float m[QG], l[QG], acc[QG][E];
#pragma unroll
      for (int j = 0; j < QG; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) acc[j][i] = 0.f;
      }
      int last_rel[QG];
#pragma unroll
      for (int j = 0; j < QG; ++j)
        last_rel[j] = __builtin_amdgcn_readfirstlane(sc.last[j]) - ca.t_begin;

      const int n_sub = (ca.t_end - ca.t_begin + CH - 1) / CH;
      walked += n_sub;
      if constexpr (LDS_STAGE) {
        if (!staged) stage_from(ca, 0, 0, sc.blk);
      }
      staged = false;
      for (int s = 0; s < n_sub; ++s) {
        uint4 kr[U], vr[U];
        const int nvalid = fetch(ca, s, s, sc.blk, kr, vr);
        if constexpr (LDS_STAGE) {
          if (s + 1 < n_sub) {
            stage_from(ca, s + 1, s + 1, sc.blk);
          } else if (nx < n_data) {   // the next item's first sub-chunk
            const ChunkAddr cn = chunk_addr(__builtin_amdgcn_readfirstlane(sn.chunk),
                                            __builtin_amdgcn_readfirstlane(sn.hg),
                                            __builtin_amdgcn_readfirstlane(sn.ctx));
            stage_from(cn, 0, 0, sn.blk);
            staged = true;
          }
        }
        fold_sub_chunk<T, D, QG>(kr, vr, nvalid, s, g, last_rel, sc.q, scale_log2, m, l, acc);
      }
      merge_lane_groups<LPT, QG, E>(m, l, acc);
      if (g == 0) {
#pragma unroll
        for (int j = 0; j < QG; ++j)
          write_item_result<T, D>(a, ws, sc.r, hg * QG + j, sc.rec, n_vec, sub, m[j], l[j],
                                  acc[j]);
      }
      it = nx;
      sc = sn;
    }
  }

  // ---- wide items: the workgroup's waves share each one ----
  ItemOrder order{xcd_order(G), G, n_dealt};
  // A batch with no wide items takes no tickets: at the end of a kernel that has
  // only single-wave items, one shared counter taking two returning atomics from every
  // workgroup was the last thing each waited for.  n_wide is the same for every
  // workgroup, so all of them skip the barriers together.
  int item = n_wide, next = n_wide;
  if (n_wide > 0) order.first_two(item, next, &ws.counters[1], s_ticket);
  int buf = 0;
  Meta cur;
  if (item < n_wide)
    cur = finish_meta<T, D, QG, NR, CH, WAVES>(a, issue_entry(ws, item, groups), item, lp,
                                               log2_bs, lane, sub, wave);

  while (item < n_wide) {
    // the item after next: static, or a ticket whose value is needed only at the end
    int after = 0;
    const bool after_static = order.take(after);
    if (!after_static && threadIdx.x == 0) after = atomicAdd(&ws.counters[1], 1);
    int4 next_ent = make_int4(0, -1, 0, 0);
    if (next < n_wide) next_ent = issue_entry(ws, next, groups);

    const int chunk = __builtin_amdgcn_readfirstlane(cur.chunk);
    const int hg = __builtin_amdgcn_readfirstlane(cur.hg);
    const ChunkAddr ca = chunk_addr(chunk, hg, __builtin_amdgcn_readfirstlane(cur.ctx));

    float m[QG], l[QG], acc[QG][E];
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[j][i] = 0.f;
    }
    int last_rel[QG];
#pragma unroll
    for (int j = 0; j < QG; ++j)
      last_rel[j] = __builtin_amdgcn_readfirstlane(cur.last[j]) - ca.t_begin;

    const int n_sub = (ca.t_end - ca.t_begin + CH - 1) / CH;
    if (wave == 0) walked += n_sub;
    if constexpr (LDS_STAGE) {
      if (wave < n_sub) stage_from(ca, wave, 0, cur.blk);
    }
    for (int s = wave; s < n_sub; s += WAVES) {
      uint4 kr[U], vr[U];
      const int i = (s - wave) / WAVES;   // the wave's i-th sub-chunk of the item
      const int nvalid = fetch(ca, s, i, cur.blk, kr, vr);
      if constexpr (LDS_STAGE) {
        if (s + WAVES < n_sub) stage_from(ca, s + WAVES, i + 1, cur.blk);
      }
      fold_sub_chunk<T, D, QG>(kr, vr, nvalid, s, g, last_rel, cur.q, scale_log2, m, l, acc);
    }

    // the next item's query and block ids load while this item's state is merged
    const Meta nxt = finish_meta<T, D, QG, NR, CH, WAVES>(a, next_ent, next, lp, log2_bs, lane,
                                                          sub, wave);
    merge_lane_groups<LPT, QG, E>(m, l, acc);
    // merge the waves (LDS double-buffered by item parity: one barrier); wave w merges
    // and writes heads w, w + WAVES, ... of the group
    if constexpr (WAVES > 1) {
      if (g == 0) {
#pragma unroll
        for (int j = 0; j < QG; ++j) {
#pragma unroll
          for (int i = 0; i < E; ++i) s_acc[buf][j][wave][sub * E + i] = acc[j][i];
          if (sub == 0) {
            s_m[buf][j][wave] = m[j];
            s_l[buf][j][wave] = l[j];
          }
        }
      }
    }
    if (!after_static && threadIdx.x == 0) s_ticket[buf] = after;
    __syncthreads();
    if (!after_static) after = n_dealt + __builtin_amdgcn_readfirstlane(s_ticket[buf]);
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < QG; ++j) {
        if (j % WAVES != wave) continue;
        float mj = m[j], lj = l[j], aj[E];
#pragma unroll
        for (int i = 0; i < E; ++i) aj[i] = acc[j][i];
        if constexpr (WAVES > 1) {
          float mx = s_m[buf][j][0];
#pragma unroll
          for (int w = 1; w < WAVES; ++w) mx = fmaxf(mx, s_m[buf][j][w]);
          // -inf only for a vector whose causal limit precedes this whole chunk
          const float mu = mx == -INFINITY ? 0.f : mx;
          lj = 0.f;
#pragma unroll
          for (int i = 0; i < E; ++i) aj[i] = 0.f;
#pragma unroll
          for (int w = 0; w < WAVES; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[buf][j][w] - mu);
            lj += s_l[buf][j][w] * f;
#pragma unroll
            for (int i = 0; i < E; ++i) aj[i] += s_acc[buf][j][w][sub * E + i] * f;
          }
          mj = mx;
        }
        write_item_result<T, D>(a, ws, cur.r, hg * QG + j, cur.rec, n_vec, sub, mj, lj, aj);
      }
    }
    buf ^= 1;
    item = next;
    cur = nxt;
    next = after;
  }

  if (bad_block && lane == 0) raise_status(ws, PKV_DEVERR_BLOCK_ID);
  report_walked<WAVES>(ws, s_walk, walked);
  // padding rows: zero output, nothing read
  for (int it = n_data + (int)blockIdx.x; it < n_items; it += G) {
    const int e = it / groups;
    const int hgp = it - e * groups;
    const int r = ws.entries[e].x;
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < QG; ++j)
        if (j % WAVES == wave)
          store16(static_cast<T*>(a.out) + vec_slot(a, r, hgp * QG + j) * D + sub * E,
                  make_uint4(0, 0, 0, 0));
    }
  }
}

// ------------------------------------------------------------------------- //
// decode on the matrix cores
// ------------------------------------------------------------------------- //
// With 4, 8 or 16 query vectors per KV head (grouped heads x new tokens), the fold of a
// 16-token sub-chunk is two small dense products per item:
//   S^T[16 tokens x 16 vectors]  = K[16 x d] . Q^T[d x 16]   (v_mfma_f32_16x16x32_bf16)
//   O^T[d x 16 vectors]         += V^T[d x 16] . P^T[16 x 16] (v_mfma_f32_16x16x16_bf16)
// K comes from the LDS stage row by row; V^T by transposing LDS reads
// (ds_read_b64_tr_b16); the scores' result layout (lane: one vector, four tokens) is
// already the P^T operand, so nothing moves between lanes but the running maxima.
// P goes in as two bfloat16 parts (hi + the rounding residue), keeping the weights at
// float precision.  Lane l owns vector l % 16 and rows 4 (l / 16) .. +3 of each tile.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 4 bf16 of a transposing LDS read: within each 16-lane group the four rows addressed by
// lanes 4r .. 4r + 3 (8 bytes each) come back one column per lane.
__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
}

// Bank spread of a parked vector: its column index XORed into dim bits 0-1 and 4-5
// (a permutation of the vector's D dims for D >= 64).
__device__ __forceinline__ int park_swizzle(int c) { return (c & 3) | ((c >> 2) << 4); }

// XOR mask on the 16-byte piece index of token g of stage chunk u (bfloat16 head
// vectors: 16 pieces, 4 tokens a chunk, 4 chunks at head_dim 128; 8 pieces, 8 tokens,
// 2 chunks at 64).  At 128 the mask takes every value 0..15 once over the 16 tokens and
// differs in bits 1..2 between the tokens of a chunk and in bit 3 between chunks 2k and
// 2k + 1; at 64 it takes every value 0..7 once over (u, g / 2).
template <int D>
__device__ __forceinline__ constexpr int piece_mask(int u, int g) {
  return D == 128 ? 2 * g + 8 * (u & 1) + (u >> 1) : 2 * (g >> 1) + u;
}

template <int D, int NR>
struct MfmaMeta {
  int r, hg, chunk, rec, ctx;   // rec: the chunk's partial record (-1: one-chunk row)
  int last;           // lane: last visible position of vector hg*QG + l%16 (-1: none)
  uint4 q[D / 32];    // lane: 8 dims (32 s + 8 (l/16) ..) of that vector's query
  int blk[NR];   // lane i: block id of this wave's sub-chunks i, 64 + i, ...
};

template <int D, int QG, int NR, int WAVES>
__device__ __forceinline__ MfmaMeta<D, NR> finish_meta_mfma(const AttnArgs& a, int4 ent, int item,
                                                        int lp, int log2_bs, int lane, int wave) {
  const int groups = a.query_len * a.num_heads / QG;
  const int col = lane & 15, grp = lane >> 4;
  MfmaMeta<D, NR> m;
  const int e = item / groups;
  m.hg = item - e * groups;
  m.r = __builtin_amdgcn_readfirstlane(ent.x);
  m.chunk = __builtin_amdgcn_readfirstlane(ent.y);
  m.rec = __builtin_amdgcn_readfirstlane(ent.z);
  m.ctx = __builtin_amdgcn_readfirstlane(ent.w);
  const int v = m.hg * QG + col;
  m.last = col < QG ? m.ctx - a.query_len + vec_query(a, v) : -1;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) m.q[s] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int k = 0; k < NR; ++k) m.blk[k] = 0;
  if (m.chunk >= 0) {
    if (col < QG) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + vec_slot(a, m.r, v) * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) m.q[s] = load16(qp + 32 * s);
    }
    load_chunk_blocks<NR, 16, WAVES>(a, m.r, m.chunk, m.ctx, lp, log2_bs, lane, wave, m.blk);
  }
  return m;
}

// Scores of one staged 16-token tile for the lane's vector (S^T = K . Q^T: lane
// (col, grp) gets tokens 4 grp .. 4 grp + 3 of vector col) and the tile's V^T operands,
// both read from a wave's stage.
template <int D>
__device__ __forceinline__ f32x4_t mfma_tile_scores(const char* st_k, const char* st_v,
                                                    const int (&k_off)[D / 32],
                                                    const int (&v_off)[D / 16],
                                                    const uint4 (&q)[D / 32],
                                                    i16x4_t (&vt)[D / 16]) {
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    const bf16x8_t kk = *reinterpret_cast<const bf16x8_t*>(st_k + k_off[ds]);
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, __builtin_bit_cast(bf16x8_t, q[ds]), sc,
                                                 0, 0, 0);
  }
#pragma unroll
  for (int o = 0; o < D / 16; ++o) vt[o] = lds_read_tr16(st_v + v_off[o]);
  return sc;
}

// Online-softmax fold of one tile into the lane's vector state: `vis` of the tile's
// tokens are visible to it; the row groups share the tile's maximum, and each keeps its
// own share of the denominator.  P goes in as two bfloat16 parts (hi + the rounding
// residue).
template <int NO>
__device__ __forceinline__ void mfma_tile_fold(f32x4_t sc, const i16x4_t (&vt)[NO], int vis,
                                               int grp, float scale_log2, float& m, float& l,
                                               f32x4_t (&acc)[NO]) {
  float x[4], tmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = 4 * grp + e < vis ? sc[e] * scale_log2 : -INFINITY;
    tmax = fmaxf(tmax, x[e]);
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(m, tmax);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - m_use);
  l *= alpha;
#pragma unroll
  for (int o = 0; o < NO; ++o) acc[o] *= alpha;
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
    l += p[e];
  }
  const uint32_t h01 = Elem<uint16_t>::cvt2(p[0], p[1]);
  const uint32_t h23 = Elem<uint16_t>::cvt2(p[2], p[3]);
  const uint32_t l01 = Elem<uint16_t>::cvt2(p[0] - __uint_as_float(h01 << 16),
                                            p[1] - __uint_as_float(h01 & 0xffff0000u));
  const uint32_t l23 = Elem<uint16_t>::cvt2(p[2] - __uint_as_float(h23 << 16),
                                            p[3] - __uint_as_float(h23 & 0xffff0000u));
  const i16x4_t ph = __builtin_bit_cast(i16x4_t, make_uint2(h01, h23));
  const i16x4_t pl = __builtin_bit_cast(i16x4_t, make_uint2(l01, l23));
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    acc[o] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[o], ph, acc[o], 0, 0, 0);
    acc[o] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[o], pl, acc[o], 0, 0, 0);
  }
  m = m_new;
}

typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));

// Same schedule, staging and partial records as decode_kernel (bfloat16 pools, head_dim
// 64 or 128, sub-chunks of 16 tokens), single-wave items first.  A single wave's tiles
// hold whole vectors (lane (col, grp): dims 16 o + 4 grp .. + 3 of vector col), so it
// writes its item's result from registers.  After its last fold of a wide item a wave
// parks its state, [QG][D] floats, in a park area of its own, and the waves are merged
// from there; its stage is free by then, so the next item's first sub-chunk streams in
// while the waves meet and merge.  (At head_dim 128 these kernels hold one workgroup per
// compute unit by registers, so the park area costs no occupancy.)
template <int D, int WAVES, int QG>
__global__ void __launch_bounds__(WAVES * 64)
decode_mfma_kernel(AttnArgs a, Workspace ws, float scale_log2) {
  using T = uint16_t;
  using S = Shape<T, D>;
  constexpr int NR = id_regs(16, WAVES);
  using Meta = MfmaMeta<D, NR>;
  constexpr int TPS = S::TPS, U = S::U, CH = S::CH, LPT = S::LPT;
  constexpr int ES = sizeof(T);
  static_assert(CH == 16, "one 16-token tile per sub-chunk");
  static_assert(QG == 4 || QG == 8 || QG == 16, "4, 8 or 16 query vectors per item");
  static_assert(D == 64 || D == 128, "piece_mask covers head_dim 64 and 128");
  constexpr int NS = D / 32;      // score products (32 dims each)
  constexpr int NO = D / 16;      // output tiles (16 dims each)
  constexpr int PER = D / 64;     // dims per lane in the merge
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;      // matrix cores: vector (and K row) of this lane
  const int grp = lane >> 4;      // matrix cores: row group of this lane

  // Stage layout.  A sub-chunk's K (then V) arrives as U chunks of 1 KB, one per
  // buffer-to-LDS load of TPS tokens x LPT 16-byte pieces, lane i landing at byte 16 i.
  // Lane g * LPT + j fetches piece j ^ piece_mask<D>(u, g) of token g: every quad of
  // lanes still reads one aligned 64-byte run of the pool, and the masks spread the
  // 16 tokens of one K read pass, and the 4 tokens x 32 bytes of one transposing V read
  // (or two of them), over distinct LDS banks.  With plain token rows the 16 tokens of a
  // 256-byte head vector all sit in the same 4 banks.
  constexpr int STAGE = 2 * U * 1024;      // K chunks, then V chunks
  __shared__ __attribute__((aligned(16))) char s_stage[WAVES][STAGE];
  __shared__ __attribute__((aligned(16))) float s_park[WAVES][QG * D];
  __shared__ int s_ticket[2];
  __shared__ float s_m[2][QG][WAVES], s_l[2][QG][WAVES];
  __shared__ int s_walk[WAVES];

  const int n_vec = a.query_len * a.num_heads;
  const int groups = n_vec / QG;
  const int vpkv = n_vec / a.g.kv_heads;
  const int lp = ws.counters[3];
  const int P = 1 << lp;
  const int n_wide = ws.counters[10] * groups;    // items before the single-wave ones
  const int n_data = ws.counters[5] * groups;
  const int n_items = ws.counters[0] * groups;
  const int G = ws.counters[7];                  // workgroups taking part
  if ((int)blockIdx.x >= G) return;
  if (blockIdx.x == 0 && threadIdx.x == 0) {     // what the walk count is counted in
    ws.counters[kCtrTileTokens] = CH;
    ws.counters[kCtrVectorGroups] = groups;
  }
  int walked = 0;   // sub-chunks this wave streamed (wide items: wave 0 counts each once)
  const int n_static = min(ws.counters[4] * groups, n_wide);
  const int n_dealt = a.deal_static ? n_static / G * G : 0;
  const int log2_bs = a.g.log2_bs;
  const int bs_mask = a.g.block_size - 1;
  const int64_t tok_bytes = a.g.tok_stride * ES;
  const int64_t blk_bytes = a.g.blk_stride * ES;
  const int64_t head_bytes = a.g.head_stride * ES;
  uint32_t voff[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = lane / LPT;
    voff[u] = (uint32_t)((u * TPS + g) * tok_bytes + ((lane % LPT) ^ piece_mask<D>(u, g)) * 16);
  }
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  const char* st_k = &s_stage[wave][0];
  const char* st_v = &s_stage[wave][U * 1024];
  // byte offset in a stage half of token t's dims d .. d + 3 (d a multiple of 4)
  auto at = [](int t, int d) {
    const int u = t / TPS, g = t % TPS;
    return u * 1024 + (g * LPT + ((d / 8) ^ piece_mask<D>(u, g))) * 16 + ((d / 4) & 1) * 8;
  };
  // this lane's K operands (token col, dims 32 ds + 8 grp ..) and V^T operands (token
  // 4 grp + col / 4, dims 16 o + 4 (col % 4) ..)
  int k_off[NS], v_off[NO];
#pragma unroll
  for (int ds = 0; ds < NS; ++ds) k_off[ds] = at(col, 32 * ds + 8 * grp);
#pragma unroll
  for (int o = 0; o < NO; ++o) v_off[o] = at(4 * grp + (col >> 2), 16 * o + 4 * (col & 3));

  bool bad_block = false;
  // addressing of an item's sub-chunks (fields wave-uniform: scalar descriptors)
  auto chunk_addr = [&](int chunk, int hg, int ctx) {
    const int t_begin = chunk * P;
    return ChunkAddr{kpool, vpool, (int64_t)(hg * QG / vpkv) * head_bytes, blk_bytes,
                     tok_bytes, t_begin, min(ctx, t_begin + P), bs_mask, a.g.num_blocks};
  };
  // this wave's stage <- sub-chunk s (the wave's i-th) of an item
  auto stage_in = [&](const ChunkAddr& c, int s, int i, const auto& blk) {
    __amdgpu_buffer_rsrc_t ksrc, vsrc;
    c.describe<CH>(s, i, ksrc, vsrc, bad_block, blk);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      buffer_load16_lds(ksrc, voff[u], reinterpret_cast<uint4*>(&s_stage[wave][u * 1024]));
      buffer_load16_lds(vsrc, voff[u], reinterpret_cast<uint4*>(&s_stage[wave][(U + u) * 1024]));
    }
  };

  // ---- single-wave items first (see decode_kernel) ----
  {
    constexpr int NRS = solo_id_regs(16);
    using MetaS = MfmaMeta<D, NRS>;
    const int stride = G * WAVES;
    int it = n_wide + xcd_order(G) * WAVES + wave;
    MetaS sc_m;
    int4 ent_nx = make_int4(0, -1, 0, 0);
    if (it < n_data) {
      sc_m = finish_meta_mfma<D, QG, NRS, 1>(a, issue_entry(ws, it, groups), it, lp, log2_bs,
                                             lane, 0);
      if (it + stride < n_data) ent_nx = issue_entry(ws, it + stride, groups);
    }
    bool staged = false;   // the item's first sub-chunk is already in the stage
    while (it < n_data) {
      const int nx = it + stride;
      // the next item's query and block ids, and the entry after it, load while this
      // item streams
      MetaS sn = finish_meta_mfma<D, QG, NRS, 1>(a, ent_nx, nx, lp, log2_bs, lane, 0);
      ent_nx = nx + stride < n_data ? issue_entry(ws, nx + stride, groups)
                                    : make_int4(0, -1, 0, 0);
      const int chunk = __builtin_amdgcn_readfirstlane(sc_m.chunk);
      const int hg = __builtin_amdgcn_readfirstlane(sc_m.hg);
      const ChunkAddr ca = chunk_addr(chunk, hg, __builtin_amdgcn_readfirstlane(sc_m.ctx));
      const int last_rel = sc_m.last - ca.t_begin;
      f32x4_t acc[NO];
#pragma unroll
      for (int o = 0; o < NO; ++o) acc[o] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float m = -INFINITY, l = 0.f;
      const int n_sub = (ca.t_end - ca.t_begin + CH - 1) / CH;
      walked += n_sub;
      if (!staged) stage_in(ca, 0, 0, sc_m.blk);
      staged = false;
      for (int s = 0; s < n_sub; ++s) {
        __amdgpu_buffer_rsrc_t ksrc, vsrc;
        const int nvalid = ca.describe<CH>(s, s, ksrc, vsrc, bad_block, sc_m.blk);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);          // the stage has landed
        i16x4_t vt[NO];
        const f32x4_t sc = mfma_tile_scores<D>(st_k, st_v, k_off, v_off, sc_m.q, vt);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);        // stage read before it is refilled
        if (s + 1 < n_sub) {
          stage_in(ca, s + 1, s + 1, sc_m.blk);
        } else if (nx < n_data) {   // the next item's first sub-chunk
          stage_in(chunk_addr(__builtin_amdgcn_readfirstlane(sn.chunk),
                              __builtin_amdgcn_readfirstlane(sn.hg),
                              __builtin_amdgcn_readfirstlane(sn.ctx)),
                   0, 0, sn.blk);
          staged = true;
        }
        mfma_tile_fold<NO>(sc, vt, min(nvalid, last_rel - s * CH + 1), grp, scale_log2, m, l,
                           acc);
      }
      l += __shfl_xor(l, 16);        // the four row groups' denominators
      l += __shfl_xor(l, 32);
      if (col < QG) {
        const int v = hg * QG + col;
        if (sc_m.rec < 0) {
          const float inv = l > 0.f ? 1.0f / l : 0.f;
          T* op = static_cast<T*>(a.out) + vec_slot(a, sc_m.r, v) * D + 4 * grp;
#pragma unroll
          for (int o = 0; o < NO; ++o)
            store_out(reinterpret_cast<u32x2_nt*>(op + 16 * o),
                      u32x2_nt{Elem<uint16_t>::cvt2(acc[o][0] * inv, acc[o][1] * inv),
                               Elem<uint16_t>::cvt2(acc[o][2] * inv, acc[o][3] * inv)});
        } else {
          float* rec = ws.partials + record_offset<D>(sc_m.rec, n_vec, v);
          if (grp == 0) {
            rec[0] = m;
            rec[1] = l;
          }
#pragma unroll
          for (int o = 0; o < NO; ++o)
            store16(rec + 4 + 16 * o + 4 * grp,
                    make_uint4(__float_as_uint(acc[o][0]), __float_as_uint(acc[o][1]),
                               __float_as_uint(acc[o][2]), __float_as_uint(acc[o][3])));
        }
      }
      it = nx;
      sc_m = sn;
    }
  }

  // ---- wide items: the workgroup's waves share each one ----
  ItemOrder order{xcd_order(G), G, n_dealt};
  // A batch with no wide items takes no tickets: at the end of a kernel that has
  // only single-wave items, one shared counter taking two returning atomics from every
  // workgroup was the last thing each waited for.  n_wide is the same for every
  // workgroup, so all of them skip the barriers together.
  int item = n_wide, next = n_wide;
  if (n_wide > 0) order.first_two(item, next, &ws.counters[1], s_ticket);
  int buf = 0;
  bool first_staged = false;   // the item's first sub-chunk is already in this wave's stage
  Meta cur;
  if (item < n_wide)
    cur = finish_meta_mfma<D, QG, NR, WAVES>(a, issue_entry(ws, item, groups), item, lp,
                                             log2_bs, lane, wave);

  while (item < n_wide) {
    int after = 0;
    const bool after_static = order.take(after);
    if (!after_static && threadIdx.x == 0) after = atomicAdd(&ws.counters[1], 1);
    int4 next_ent = make_int4(0, -1, 0, 0);
    if (next < n_wide) next_ent = issue_entry(ws, next, groups);

    const int chunk = __builtin_amdgcn_readfirstlane(cur.chunk);
    const int hg = __builtin_amdgcn_readfirstlane(cur.hg);
    const ChunkAddr ca = chunk_addr(chunk, hg, __builtin_amdgcn_readfirstlane(cur.ctx));
    const int last_rel = cur.last - ca.t_begin;      // this lane's vector

    f32x4_t acc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) acc[o] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    const int n_sub = (ca.t_end - ca.t_begin + CH - 1) / CH;
    if (wave == 0) walked += n_sub;
    if (wave < n_sub && !first_staged) stage_in(ca, wave, 0, cur.blk);
    first_staged = false;
    // the next item's query and block ids load after this wave's first fold (its entry
    // has landed by then), in time for its first sub-chunk to be staged below
    Meta nxt;
    bool nxt_issued = false;
    for (int s = wave; s < n_sub; s += WAVES) {
      __amdgpu_buffer_rsrc_t ksrc, vsrc;
      const int i = (s - wave) / WAVES;
      const int nvalid = ca.describe<CH>(s, i, ksrc, vsrc, bad_block, cur.blk);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);          // this wave's stage has landed
      i16x4_t vt[NO];
      const f32x4_t sc = mfma_tile_scores<D>(st_k, st_v, k_off, v_off, cur.q, vt);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);        // stage read before it is refilled
      if (s + WAVES < n_sub) stage_in(ca, s + WAVES, i + 1, cur.blk);
      mfma_tile_fold<NO>(sc, vt, min(nvalid, last_rel - s * CH + 1), grp, scale_log2, m, l,
                         acc);
      if (!nxt_issued) {
        nxt = finish_meta_mfma<D, QG, NR, WAVES>(a, next_ent, next, lp, log2_bs, lane, wave);
        nxt_issued = true;
      }
    }
    if (!nxt_issued)
      nxt = finish_meta_mfma<D, QG, NR, WAVES>(a, next_ent, next, lp, log2_bs, lane, wave);
    // the next item's first sub-chunk into this wave's stage (its last read of this
    // item's stage has completed), to land while the waves merge this item
    if (next < n_wide) {
      const ChunkAddr cn = chunk_addr(__builtin_amdgcn_readfirstlane(nxt.chunk),
                                      __builtin_amdgcn_readfirstlane(nxt.hg),
                                      __builtin_amdgcn_readfirstlane(nxt.ctx));
      if (wave < (cn.t_end - cn.t_begin + CH - 1) / CH) {
        stage_in(cn, wave, 0, nxt.blk);
        first_staged = true;
      }
    }
    l += __shfl_xor(l, 16);        // the four row groups' denominators
    l += __shfl_xor(l, 32);
    // park this wave's state: vector c's dim d at c * D + (d ^ park_swizzle(c)), so
    // that the 64 lanes of one write (16 vectors x 4 row groups) fall in distinct LDS
    // banks
    float* park = &s_park[wave][0];
    if (col < QG) {
      const int sw = park_swizzle(col);
#pragma unroll
      for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int e = 0; e < 4; ++e) park[col * D + ((16 * o + 4 * grp + e) ^ sw)] = acc[o][e];
      if (grp == 0) {
        s_m[buf][col][wave] = m;
        s_l[buf][col][wave] = l;
      }
    }
    if (!after_static && threadIdx.x == 0) s_ticket[buf] = after;
    __syncthreads();
    if (!after_static) after = n_dealt + __builtin_amdgcn_readfirstlane(s_ticket[buf]);
    // merge the waves: wave w finishes vectors w, w + WAVES, ...
    for (int j = wave; j < QG; j += WAVES) {
      float mx = s_m[buf][j][0];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) mx = fmaxf(mx, s_m[buf][j][w]);
      const float mu = mx == -INFINITY ? 0.f : mx;
      float lj = 0.f, y[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) y[i] = 0.f;
      const int sw = park_swizzle(j);
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_m[buf][j][w] - mu);
        lj += s_l[buf][j][w] * f;
        const float* pw = &s_park[w][0] + j * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) y[i] += pw[(lane * PER + i) ^ sw] * f;
      }
      const int v = hg * QG + j;
      if (cur.rec < 0) {
        const float inv = lj > 0.f ? 1.0f / lj : 0.f;
        T* op = static_cast<T*>(a.out) + vec_slot(a, cur.r, v) * D + lane * PER;
        if constexpr (PER == 1) {
          store_out(op, (uint16_t)(Elem<uint16_t>::cvt2(y[0] * inv, 0.f) & 0xffffu));
        } else {
#pragma unroll
          for (int i = 0; i < PER; i += 2)
            store_out(reinterpret_cast<uint32_t*>(op + i),
                      Elem<uint16_t>::cvt2(y[i] * inv, y[i + 1] * inv));
        }
      } else {
        float* rec = ws.partials + record_offset<D>(cur.rec, n_vec, v);
        if (lane == 0) {
          rec[0] = mx;
          rec[1] = lj;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) rec[4 + lane * PER + i] = y[i];
      }
    }
    __syncthreads();     // every park area is free again before the next item parks
    buf ^= 1;
    item = next;
    cur = nxt;
    next = after;
  }
  if (bad_block && lane == 0) raise_status(ws, PKV_DEVERR_BLOCK_ID);
  report_walked<WAVES>(ws, s_walk, walked);
  for (int it = n_data + (int)blockIdx.x; it < n_items; it += G) {
    const int e = it / groups;
    const int hgp = it - e * groups;
    const int r = ws.entries[e].x;
    for (int j = wave; j < QG; j += WAVES) {
      T* op = static_cast<T*>(a.out) + vec_slot(a, r, hgp * QG + j) * D + lane * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i) op[i] = 0;
    }
  }
}

// ------------------------------------------------------------------------- //
// combine
// ------------------------------------------------------------------------- //
constexpr int kCombineThreads = 256;
constexpr int kCombineGroups = 1024;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// One wave per (split row, query vector) at a time, four waves to a workgroup, over
// the plan's list of split rows (a grid of a fixed size strides over the pairs, so a
// batch with no split row costs one load per wave).  Chunk c of the row carries
// (m_c, l_c, acc_c); the result is
// sum_c 2^(m_c - M) acc_c divided by sum_c 2^(m_c - M) l_c with M = max_c m_c, summed in
// chunk order, so it does not depend on scheduling.  Lane i holds dims i * D/64 .. of
// the vector.  A chunk wholly past a vector's causal limit carries m = -inf and l = 0
// and adds nothing.
template <typename T, int D>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(AttnArgs a, Workspace ws) {
  constexpr int PER = D / 64;     // dims per lane
  constexpr int W = kCombineThreads / 64;
  constexpr int kHeld = 8;        // a row of at most this many chunks: one round of loads
  const int lane = threadIdx.x & 63;
  const int n_vec = a.query_len * a.num_heads;
  const int64_t pairs = (int64_t)ws.counters[8] * n_vec;
  const int lp = ws.counters[3];
  for (int64_t pair = (int64_t)blockIdx.x * W + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       pair < pairs; pair += (int64_t)gridDim.x * W) {
    const int4 sr = ws.split_rows[pair / n_vec];
    const int64_t r = sr.x;
    const int v = (int)(pair % n_vec);
    const int ctx = sr.y;
    const int nch = (ctx + (1 << lp) - 1) >> lp;
    if (nch <= 1) continue;
    // chunk c's record of vector v, c = 0 .. nch - 1
    const float* rec = ws.partials + record_offset<D>(sr.z, n_vec, v);
    const int64_t stride = (int64_t)n_vec * (D + 4);

    float mx = -INFINITY;
    float l = 0.f, acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    if (nch <= kHeld) {
      // every chunk's (m, l, acc) at once, then the same sums in chunk order
      float m[kHeld], lc[kHeld], y[kHeld][PER];
#pragma unroll
      for (int c = 0; c < kHeld; ++c) {
        m[c] = -INFINITY;
        lc[c] = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) y[c][i] = 0.f;
        if (c < nch) {
          const float* p = rec + c * stride;
          m[c] = p[0];
          lc[c] = p[1];
#pragma unroll
          for (int i = 0; i < PER; ++i) y[c][i] = p[4 + lane * PER + i];
        }
      }
#pragma unroll
      for (int c = 0; c < kHeld; ++c) mx = fmaxf(mx, m[c]);
      if (mx == -INFINITY) mx = 0.f;   // only a row whose length was out of bounds
#pragma unroll
      for (int c = 0; c < kHeld; ++c) {
        if (c < nch) {
          const float f = __builtin_amdgcn_exp2f(m[c] - mx);
          l += lc[c] * f;
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] += y[c][i] * f;
        }
      }
    } else {
      for (int c = lane; c < nch; c += 64) mx = fmaxf(mx, rec[c * stride]);
      mx = wave_max(mx);
      if (mx == -INFINITY) mx = 0.f;   // only a row whose length was out of bounds
#pragma unroll 4
      for (int c = 0; c < nch; ++c) {
        const float* p = rec + c * stride;
        const float f = __builtin_amdgcn_exp2f(p[0] - mx);
        l += p[1] * f;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += p[4 + lane * PER + i] * f;
      }
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    T* outp = static_cast<T*>(a.out) + vec_slot(a, r, v) * D + lane * PER;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int i = 0; i < PER; ++i) store_out(outp + i, (T)(acc[i] * inv));
    } else if constexpr (PER == 1) {
      store_out(outp, (uint16_t)(Elem<uint16_t>::cvt2(acc[0] * inv, 0.f) & 0xffffu));
    } else {
#pragma unroll
      for (int i = 0; i < PER; i += 2)
        store_out(reinterpret_cast<uint32_t*>(outp + i),
                  Elem<uint16_t>::cvt2(acc[i] * inv, acc[i + 1] * inv));
    }
  }
}

// ------------------------------------------------------------------------- //
// slot input
// ------------------------------------------------------------------------- //
// The translation pass of a read addressed by a slot rectangle.  A row whose live
// cells are block structured (cell t = B * block_size + t % block_size for every t of
// block t / block_size, B an allocatable block) is exactly a block-table row: its block
// ids go to a derived table and the block path reads it.  Any other row is flagged and
// read token by token.  One workgroup per (row, kTranslateTokens positions); each
// writes its flag whether or not it found anything, so nothing needs clearing first.
constexpr int kTranslateThreads = 256;

__global__ void __launch_bounds__(kTranslateThreads) translate_slots_kernel(AttnArgs a,
                                                                           SlotArgs sa) {
  const int64_t r = blockIdx.y;
  int ctx = a.context_lens[r];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_limit ? a.ctx_limit : ctx);
  const int64_t* row = sa.slots + r * sa.row_stride;
  const int bs_mask = a.g.block_size - 1;
  const int64_t n_slots = a.g.num_blocks * a.g.block_size;
  const int t_base = blockIdx.x * kTranslateTokens;
  const int t_end = min(ctx, t_base + kTranslateTokens);
  bool bad = false;
  for (int t = t_base + threadIdx.x; t < t_end; t += kTranslateThreads) {
    const int off = t & bs_mask;
    const int64_t slot = row[t];
    const int64_t first = off == 0 ? slot : row[t - off];   // the block's first cell
    const bool ok = first >= 0 && first < n_slots && (first & bs_mask) == 0 &&
                    slot == first + off;
    bad |= !ok;
    if (off == 0 && ok)
      sa.block_tables[r * sa.max_blocks + (t >> a.g.log2_bs)] =
          (int32_t)(first >> a.g.log2_bs);
  }
  const int any = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) sa.row_flags[r * sa.flag_stride + blockIdx.x] = any;
}

// The rows of a slot input that are not block structured.  An item is (chunk of a row,
// query head): the plan lists these rows' chunks longest first (the decode kernel's
// chunk length; a split row leaves partial records for the combine kernel just as the
// decode kernel does).  This kernel reads the chunks of at least a.solo_tokens tokens:
// each workgroup takes the item of its own index first, then items from one shared
// ticket counter; token_rows_short_kernel reads the rest.  Each
// 16-lane group (bf16 x 128) takes one token, loads its slot, then the token's K and V
// through that slot, and folds it into its own online softmax; the groups and the waves
// are merged at the end of the item.  A live slot outside the allocatable slots is
// skipped and reported.  Runs after the decode kernel (which wrote zeros for these rows)
// and before the combine kernel.
constexpr int kTokenRowThreads = 256;

template <typename T, int D>
__global__ void __launch_bounds__(kTokenRowThreads)
token_rows_kernel(AttnArgs a, SlotArgs sa, Workspace ws, float scale_log2) {
  using Sh = Shape<T, D>;
  using El = Elem<T>;
  constexpr int E = Sh::E, LPT = Sh::LPT, TPS = Sh::TPS, U = Sh::U;
  constexpr int ES = sizeof(T);
  constexpr int WAVES = kTokenRowThreads / 64;
  constexpr int STEP = WAVES * TPS * U;
  __shared__ float s_m[WAVES], s_l[WAVES];
  __shared__ float s_acc[WAVES][D];
  __shared__ int s_item[2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane / LPT;
  const int sub = lane % LPT;
  const int heads = a.num_heads;
  const int qpkv = heads / a.g.kv_heads;
  const int lp = ws.counters[3];
  const int n_items = ws.counters[12] * heads;  // (token entry, query head), long ones
  const int64_t n_slots = a.g.num_blocks * a.g.block_size;
  const int log2_bs = a.g.log2_bs;
  const int bs_mask = a.g.block_size - 1;
  const int64_t tok_bytes = a.g.tok_stride * ES;
  const int64_t blk_bytes = a.g.blk_stride * ES;
  const int64_t head_bytes = a.g.head_stride * ES;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  bool bad = false;
  // workgroup b's first item is b (one a workgroup across the grid), later ones come
  // from the ticket counter, past the first round
  int item = blockIdx.x;
  int buf = 0;
  while (item < n_items) {
    // the next ticket, whose value is needed only at the end of this item
    int next = 0;
    if (threadIdx.x == 0) next = (int)gridDim.x + atomicAdd(&ws.counters[11], 1);
    const int e = item / heads;
    const int h = item - e * heads;
    const int2 ent = ws.token_entries[e];
    const int r = __builtin_amdgcn_readfirstlane(ent.x);
    const int chunk = __builtin_amdgcn_readfirstlane(ent.y);
    const int ctx = __builtin_amdgcn_readfirstlane(ws.row_ctx[r]);
    const int nch = (ctx + (1 << lp) - 1) >> lp;
    const int t_begin = chunk << lp;
    const int t_end = min(ctx, t_begin + (1 << lp));
    const int64_t rh = (int64_t)r * heads + h;
    const uint4 qv = load16(static_cast<const T*>(a.q) + rh * D + sub * E);
    const int64_t lane_off = (int64_t)(h / qpkv) * head_bytes + sub * E * ES;
    const int64_t* row = sa.slots + (int64_t)r * sa.row_stride;
    float m = -INFINITY, l = 0.f, acc[E];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = 0.f;
    // Software pipeline over this wave's steps of TPS * U tokens: the slots two steps
    // ahead and the K/V one step ahead are in flight while a step is folded (a slot
    // is needed before its K/V can be addressed).  A slot outside the allocatable
    // slots (or a position past the chunk) loads nothing and scores -inf.
    auto slots_of = [&](int t0, int64_t (&sl)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * TPS + g;
        sl[u] = t < t_end ? row[t] : -1;
      }
    };
    auto kv_of = [&](const int64_t (&sl)[U], uint4 (&kr)[U], uint4 (&vr)[U], bool (&ok)[U],
                     int t0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * TPS + g;
        const int64_t slot = sl[u];
        ok[u] = t < t_end && slot >= 0 && slot < n_slots;
        bad |= t < t_end && !ok[u];
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
        if (ok[u]) {
          const int64_t off = (slot >> log2_bs) * blk_bytes + (slot & bs_mask) * tok_bytes +
                              lane_off;
          kr[u] = load16_stream(kpool + off);
          vr[u] = load16_stream(vpool + off);
        }
      }
    };
    const int t_first = t_begin + wave * TPS * U;
    int64_t sl_next[U];
    uint4 kr[U], vr[U];
    bool ok[U];
    {
      int64_t sl[U];
      slots_of(t_first, sl);
      kv_of(sl, kr, vr, ok, t_first);
      slots_of(t_first + STEP, sl_next);
    }
    for (int t0 = t_first; t0 < t_end; t0 += STEP) {
      // the next step's K/V (its slots have landed) and the slots of the one after
      uint4 kr_n[U], vr_n[U];
      bool ok_n[U];
      kv_of(sl_next, kr_n, vr_n, ok_n, t0 + STEP);
      slots_of(t0 + 2 * STEP, sl_next);

      float sc[U];
      float smax = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float d = group_sum<LPT>(El::dot(qv, kr[u], 0.f));
        sc[u] = ok[u] ? d * scale_log2 : -INFINITY;
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
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = kr_n[u];
        vr[u] = vr_n[u];
        ok[u] = ok_n[u];
      }
    }
    // merge the lane groups, then the waves
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
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < E; ++i) s_acc[wave][sub * E + i] = acc[i];
      if (sub == 0) {
        s_m[wave] = m;
        s_l[wave] = l;
      }
    }
    if (threadIdx.x == 0) s_item[buf] = next;
    __syncthreads();
    if (wave == 0 && g == 0) {
      float mx = s_m[0];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) mx = fmaxf(mx, s_m[w]);
      const float mu = mx == -INFINITY ? 0.f : mx;
      float lt = 0.f, y[E];
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_m[w] - mu);
        lt += s_l[w] * f;
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] += s_acc[w][sub * E + i] * f;
      }
      if (nch == 1) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;   // every live slot skipped: zeros
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] *= inv;
        store16_out(static_cast<T*>(a.out) + rh * D + sub * E, El::pack(y));
      } else {
        float* rec = ws.partials + record_offset<D>(ws.row_rec[r] + chunk, heads, h);
        if (sub == 0) {
          rec[0] = mx;
          rec[1] = lt;
        }
#pragma unroll
        for (int i = 0; i < E; i += 4)
          store16(rec + 4 + sub * E + i, make_uint4(__float_as_uint(y[i]), __float_as_uint(y[i + 1]),
                                                    __float_as_uint(y[i + 2]),
                                                    __float_as_uint(y[i + 3])));
      }
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item[buf]);
    buf ^= 1;
  }
  if (bad) raise_status(ws, PKV_DEVERR_SLOT);
}

// The token rows' chunks shorter than a.solo_tokens (the end of their list), one wave
// each, dealt round robin over every wave of the grid (the list runs longest first; a
// shared ticket counter cost ~50 us of serialized atomics over 4096 waves), with no
// merge across waves: a wave streams all of an item's steps through the same pipeline
// as token_rows_kernel (slots two steps ahead, K/V one).  A kernel of its own: the same
// loop inside token_rows_kernel slowed that kernel's shared items.  Runs right after it.
template <typename T, int D>
__global__ void __launch_bounds__(kTokenRowThreads)
token_rows_short_kernel(AttnArgs a, SlotArgs sa, Workspace ws, float scale_log2) {
  using Sh = Shape<T, D>;
  using El = Elem<T>;
  constexpr int E = Sh::E, LPT = Sh::LPT, TPS = Sh::TPS, U = Sh::U;
  constexpr int ES = sizeof(T);
  constexpr int WSTEP = TPS * U;
  const int lane = threadIdx.x & 63;
  const int g = lane / LPT;
  const int sub = lane % LPT;
  const int heads = a.num_heads;
  const int qpkv = heads / a.g.kv_heads;
  const int lp = ws.counters[3];
  const int n_items = ws.counters[9] * heads;
  const int n_wide = ws.counters[12] * heads;
  const int64_t n_slots = a.g.num_blocks * a.g.block_size;
  const int log2_bs = a.g.log2_bs;
  const int bs_mask = a.g.block_size - 1;
  const int64_t tok_bytes = a.g.tok_stride * ES;
  const int64_t blk_bytes = a.g.blk_stride * ES;
  const int64_t head_bytes = a.g.head_stride * ES;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  bool bad = false;
  const int waves = gridDim.x * (kTokenRowThreads / 64);
  for (int item = n_wide + blockIdx.x * (kTokenRowThreads / 64) +
                  __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       item < n_items; item += waves) {
    const int e = item / heads;
    const int h = item - e * heads;
    const int2 ent = ws.token_entries[e];
    const int r = __builtin_amdgcn_readfirstlane(ent.x);
    const int chunk = __builtin_amdgcn_readfirstlane(ent.y);
    const int ctx = __builtin_amdgcn_readfirstlane(ws.row_ctx[r]);
    const int nch = (ctx + (1 << lp) - 1) >> lp;
    const int t_begin = chunk << lp;
    const int t_end = min(ctx, t_begin + (1 << lp));
    const uint4 qv = load16(static_cast<const T*>(a.q) + ((int64_t)r * heads + h) * D + sub * E);
    const int64_t lane_off = (int64_t)(h / qpkv) * head_bytes + sub * E * ES;
    const int64_t* row = sa.slots + (int64_t)r * sa.row_stride;
    float m[1] = {-INFINITY}, l[1] = {0.f}, acc[1][E];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[0][i] = 0.f;
    // step 0's slots and K/V, step 1's slots
    int64_t sl_next[U];
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t_begin + u * TPS + g;
      const int64_t slot = t < t_end ? row[t] : -1;
      sl_next[u] = t + WSTEP < t_end ? row[t + WSTEP] : -1;
      ok[u] = t < t_end && slot >= 0 && slot < n_slots;
      bad |= t < t_end && !ok[u];
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (ok[u]) {
        const int64_t off = (slot >> log2_bs) * blk_bytes + (slot & bs_mask) * tok_bytes +
                            lane_off;
        kr[u] = load16_stream(kpool + off);
        vr[u] = load16_stream(vpool + off);
      }
    }
    for (int t0 = t_begin; t0 < t_end; t0 += WSTEP) {
      // the next step's K/V (its slots have landed) and the slots of the one after
      uint4 kr_n[U], vr_n[U];
      bool ok_n[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + WSTEP + u * TPS + g;
        ok_n[u] = t < t_end && sl_next[u] >= 0 && sl_next[u] < n_slots;
        bad |= t < t_end && !ok_n[u];
        kr_n[u] = make_uint4(0, 0, 0, 0);
        vr_n[u] = make_uint4(0, 0, 0, 0);
        if (ok_n[u]) {
          const int64_t off = (sl_next[u] >> log2_bs) * blk_bytes +
                              (sl_next[u] & bs_mask) * tok_bytes + lane_off;
          kr_n[u] = load16_stream(kpool + off);
          vr_n[u] = load16_stream(vpool + off);
        }
        sl_next[u] = t + WSTEP < t_end ? row[t + WSTEP] : -1;
      }
      float sc[U];
      float smax = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float d = group_sum<LPT>(El::dot(qv, kr[u], 0.f));
        sc[u] = ok[u] ? d * scale_log2 : -INFINITY;
        smax = fmaxf(smax, sc[u]);
      }
      const float m_new = fmaxf(m[0], smax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[0] - m_use);
      l[0] *= alpha;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[0][i] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = __builtin_amdgcn_exp2f(sc[u] - m_use);
        l[0] += p;
        El::axpy(p, vr[u], acc[0]);
      }
      m[0] = m_new;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = kr_n[u];
        vr[u] = vr_n[u];
        ok[u] = ok_n[u];
      }
    }
    merge_lane_groups<LPT, 1, E>(m, l, acc);
    if (g == 0)
      write_item_result<T, D>(a, ws, r, h, nch > 1 ? ws.row_rec[r] + chunk : -1, heads, sub,
                              m[0], l[0], acc[0]);
  }
  if (bad) raise_status(ws, PKV_DEVERR_SLOT);
}

// ------------------------------------------------------------------------- //
// launchers
// ------------------------------------------------------------------------- //
static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

static int64_t cdiv64(int64_t x, int64_t y) { return (x + y - 1) / y; }

// Chunk records (each one record of head_dim + 4 floats per query vector) the partials
// area holds.  The plan splits a row into cdiv(length, P) chunks only when that is
// more than one, so at P = chunk_max at most rows x cdiv(width, chunk_max) chunks have
// records (none when a chunk covers the table), and at P = chunk_min at most rows x
// cdiv(width, chunk_min).  Between the two the area is kPartialBudgetBytes: the plan
// lengthens P until its split rows' chunks fit.
int32_t record_chunks_for(int64_t num_rows, int32_t vectors, int32_t head_dim,
                          int32_t max_blocks, int32_t block_size, const Tuning& t) {
  const int64_t width = (int64_t)max_blocks * block_size;
  const int64_t mc_min = cdiv64(width, t.chunk_min);
  const int64_t mc_max = cdiv64(width, t.chunk_max);
  const int64_t at_min = mc_min > 1 ? num_rows * mc_min : 0;
  const int64_t at_max = mc_max > 1 ? num_rows * mc_max : 0;
  const int64_t budget = kPartialBudgetBytes / ((int64_t)(head_dim + 4) * 4 * vectors);
  const int64_t chunks = at_min < (at_max > budget ? at_max : budget)
                             ? at_min
                             : (at_max > budget ? at_max : budget);
  return (int32_t)chunks;   // <= rows x cdiv(width, chunk_min), bounded by the item check
}

// Work-list entries: at most every row's chunks at the shortest chunk (pad rows: one).
static int64_t max_entries_for(int64_t num_rows, int32_t max_blocks, int32_t block_size,
                               const Tuning& t) {
  const int64_t mc = cdiv64((int64_t)max_blocks * block_size, t.chunk_min);
  return num_rows * (mc > 1 ? mc : 1);
}

size_t workspace_bytes(int64_t num_rows, int32_t vectors, int32_t head_dim,
                       int32_t max_blocks, int32_t block_size, const Tuning& t) {
  const int64_t recs = record_chunks_for(num_rows, vectors, head_dim, max_blocks, block_size, t);
  int64_t bytes = kCounterBytes;
  bytes += align_up(max_entries_for(num_rows, max_blocks, block_size, t) * 16, 256);
  bytes += 3 * align_up(num_rows * 4, 256);        // row lengths, first records, irregular
  bytes += align_up(num_rows * 16, 256);           // split rows
  bytes += align_up(recs * vectors * (int64_t)(head_dim + 4) * 4, 256);
  return (size_t)bytes;
}

Workspace carve_workspace(void* base, int64_t num_rows, int32_t vectors, int32_t head_dim,
                          int32_t max_blocks, int32_t block_size, const Tuning& t) {
  Workspace w;
  w.record_chunks = record_chunks_for(num_rows, vectors, head_dim, max_blocks, block_size, t);
  w.max_entries = max_entries_for(num_rows, max_blocks, block_size, t);
  char* p = static_cast<char*>(base);
  w.counters = reinterpret_cast<int32_t*>(p);
  p += kCounterBytes;
  w.entries = reinterpret_cast<int4*>(p);
  p += align_up(w.max_entries * 16, 256);
  w.row_ctx = reinterpret_cast<int32_t*>(p);
  p += align_up(num_rows * 4, 256);
  w.row_rec = reinterpret_cast<int32_t*>(p);
  p += align_up(num_rows * 4, 256);
  w.irregular = reinterpret_cast<int32_t*>(p);
  p += align_up(num_rows * 4, 256);
  w.split_rows = reinterpret_cast<int4*>(p);
  p += align_up(num_rows * 16, 256);
  w.token_entries = nullptr;
  w.partials = reinterpret_cast<float*>(p);
  return w;
}

static int32_t slot_table_blocks(int32_t width, int32_t block_size) {
  return (int32_t)(((int64_t)width + block_size - 1) / block_size);
}
static int32_t slot_flag_stride(int32_t width) {
  return (int32_t)(((int64_t)width + kTranslateTokens - 1) / kTranslateTokens);
}

// token entries of a slot input: at most every row's chunks
static int64_t token_entry_bytes(int64_t num_rows, int32_t mb, int32_t block_size,
                                 const Tuning& t) {
  return align_up(max_entries_for(num_rows, mb, block_size, t) * 8, 256);
}

size_t slot_workspace_bytes(int64_t num_rows, int32_t num_heads, int32_t head_dim,
                            int32_t width, int32_t block_size, const Tuning& t) {
  const int32_t mb = slot_table_blocks(width, block_size);
  int64_t bytes = (int64_t)workspace_bytes(num_rows, num_heads, head_dim, mb, block_size, t);
  bytes += align_up(num_rows * mb * 4, 256);
  bytes += align_up(num_rows * slot_flag_stride(width) * 4, 256);
  bytes += token_entry_bytes(num_rows, mb, block_size, t);
  return (size_t)bytes;
}

Workspace carve_slot_workspace(void* base, int64_t num_rows, int32_t num_heads,
                               int32_t head_dim, int32_t width, int32_t block_size,
                               const Tuning& t, SlotArgs* sa) {
  const int32_t mb = slot_table_blocks(width, block_size);
  Workspace w = carve_workspace(base, num_rows, num_heads, head_dim, mb, block_size, t);
  sa->max_blocks = mb;
  sa->flag_stride = slot_flag_stride(width);
  char* p = static_cast<char*>(base) +
            workspace_bytes(num_rows, num_heads, head_dim, mb, block_size, t);
  sa->block_tables = reinterpret_cast<int32_t*>(p);
  p += align_up(num_rows * mb * 4, 256);
  sa->row_flags = reinterpret_cast<int32_t*>(p);
  p += align_up(num_rows * sa->flag_stride * 4, 256);
  w.token_entries = reinterpret_cast<int2*>(p);
  return w;
}

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  const int elem = a.g.dtype == PKV_F32 ? 4 : 2;
  const int64_t pieces = a.num_tokens * a.g.kv_heads * (a.g.head_dim * elem / 16);
  const int threads = 256;
  const int64_t blocks = (pieces + threads - 1) / threads;
  const int64_t sink = a.g.num_blocks * a.g.block_size;
  timing_begin(PKV_PHASE_KV_WRITE, stream);
  if (a.g.dtype == PKV_F32)
    hipLaunchKernelGGL(kv_write_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, a, sink);
  else
    hipLaunchKernelGGL(kv_write_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0,
                       stream, a, sink);
  timing_end(PKV_PHASE_KV_WRITE, stream);
  return hipGetLastError();
}

// the merge of split rows (nothing to do when no row can split)
template <typename T, int D>
static void launch_combine_t(const AttnArgs& a, const Workspace& ws, hipStream_t stream) {
  if (ws.record_chunks <= 0) return;
  timing_begin(PKV_PHASE_COMBINE, stream);
  // a grid fixed by the shape (graph replays keep it): one wave per (row, vector) pair,
  // at most kCombineGroups workgroups, striding over the split rows' pairs
  const int waves = kCombineThreads / 64;
  const int64_t most = ((int64_t)a.num_rows * a.query_len * a.num_heads + waves - 1) / waves;
  const unsigned grid = (unsigned)(most < kCombineGroups ? most : kCombineGroups);
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(grid), dim3(kCombineThreads), 0, stream, a, ws);
  timing_end(PKV_PHASE_COMBINE, stream);
}

template <typename T, int D, int WAVES, bool LDS_STAGE, int QG, bool MFMA = false>
static hipError_t launch_decode_w(const AttnArgs& a, const Workspace& ws, const Tuning& t,
                                  hipStream_t stream, bool combine, const WriteArgs* write) {
  void (*kern)(AttnArgs, Workspace, float);
  if constexpr (MFMA) kern = decode_mfma_kernel<D, WAVES, QG>;
  else kern = decode_kernel<T, D, WAVES, LDS_STAGE, QG>;
  // occupancy and compute units per device, computed once (host threads that race to
  // fill them store the same values; the occupancy is published last)
  static std::atomic<int> per_cu[64];
  static std::atomic<int> num_cu[64];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 64) return hipErrorInvalidDevice;
  int occ = per_cu[dev].load(std::memory_order_acquire);
  if (occ == 0) {
    int n = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, WAVES * 64, 0);
    if (err != hipSuccess) return err;
    int cus = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    occ = n > 0 ? n : 1;
    num_cu[dev].store(cus, std::memory_order_relaxed);
    per_cu[dev].store(occ, std::memory_order_release);
  }
  const int cus = num_cu[dev].load(std::memory_order_relaxed);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int wpc = occ < t.groups_per_cu ? occ : t.groups_per_cu;
  int64_t grid = (int64_t)cus * wpc;
  const int64_t most = ws.max_entries * (a.query_len * a.num_heads / QG);
  if (grid > most) grid = most;
  AttnArgs pa = a;
  pa.query_group = QG;
  // an item on the matrix cores carries 8 or 16 query vectors: a quarter as many items
  // keep the workgroups as busy (measured best at the full-width batch's lengths)
  const int per_group = MFMA ? (t.items_per_group + 3) / 4 : t.items_per_group;
  pa.target_items = (int32_t)(grid * per_group);
  pa.grid_groups = (int32_t)grid;
  // the plan may keep 8 waves per CU (one workgroup of 8, two of 4, ...)
  const int64_t narrow = (int64_t)cus * (WAVES < 8 ? 8 / WAVES : 1);
  pa.narrow_groups = grid > narrow ? (int32_t)narrow : 0;
  pa.narrow_items = pa.narrow_groups * per_group;
  pa.deal_static = t.deal_static;
  pa.solo_tokens = t.solo_tokens;
  pa.group_waves = WAVES;
  pa.record_chunks = ws.record_chunks;
  timing_begin(PKV_PHASE_PLAN, stream);
  if (write) {   // the step's scatter rides along with the plan
    const int64_t pieces = write->num_tokens * write->g.kv_heads *
                           (write->g.head_dim * (int64_t)sizeof(T) / 16);
    int64_t blocks = (pieces + kPlanThreads - 1) / kPlanThreads;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(plan_write_kernel<T>, dim3((unsigned)(1 + blocks)), dim3(kPlanThreads), 0,
                       stream, pa, ws, *write, write->g.num_blocks * write->g.block_size);
  } else {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, pa, ws);
  }
  timing_end(PKV_PHASE_PLAN, stream);
  timing_begin(PKV_PHASE_DECODE, stream);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * 64), 0, stream, pa, ws,
                     scale_log2);
  timing_end(PKV_PHASE_DECODE, stream);
  if (combine) launch_combine_t<T, D>(a, ws, stream);
  return hipGetLastError();
}

// query vectors per work item: the largest of 8, 4, 2, 1 that divides the number of
// query vectors per KV head (query heads per KV head x new tokens per row) and is at
// most the tuning cap (4 for head_dim 256, whose per-vector merge buffers would not fit
// in LDS beside the K/V stages at 8)
static int query_group_of(const AttnArgs& a, const Tuning& t) {
  const int vpkv = a.query_len * (a.num_heads / a.g.kv_heads);
  int cap = t.max_query_group;
  if (cap > 8) cap = 8;
  if (a.g.head_dim >= 256 && cap > 4) cap = 4;
  for (int qg = 8; qg > 1; qg >>= 1)
    if (qg <= cap && vpkv % qg == 0) return qg;
  return 1;
}

// query vectors per item on the matrix cores: 16, 8 or 4 when that many share a KV head
// (and the tuning allows it), else 0 (the vector units take the call; with 1 or 2 they
// measured as fast or faster)
static int mfma_group_of(const AttnArgs& a, const Tuning& t) {
  if (!t.mfma || a.g.dtype != PKV_BF16 || a.g.head_dim > 128) return 0;
  const int vpkv = a.query_len * (a.num_heads / a.g.kv_heads);
  const int cap = t.max_query_group;
  for (int qg = 16; qg >= 4; qg >>= 1)
    if (qg <= cap && vpkv % qg == 0) return qg;
  return 0;
}

template <typename T, int D>
static hipError_t launch_decode_t(const AttnArgs& a, const Workspace& ws, const Tuning& t,
                                  hipStream_t stream, bool combine, const WriteArgs* write) {
  if constexpr (sizeof(T) == 2 && D <= 128) {
    switch (mfma_group_of(a, t)) {
      case 16: return launch_decode_w<T, D, 8, true, 16, true>(a, ws, t, stream, combine, write);
      case 8: return launch_decode_w<T, D, 8, true, 8, true>(a, ws, t, stream, combine, write);
      case 4: return launch_decode_w<T, D, 8, true, 4, true>(a, ws, t, stream, combine, write);
      default: break;
    }
  }
  switch (query_group_of(a, t)) {
    case 8:
      if constexpr (D < 256) return launch_decode_w<T, D, 8, true, 8>(a, ws, t, stream, combine, write);
      break;
    case 4: return launch_decode_w<T, D, 8, true, 4>(a, ws, t, stream, combine, write);
    case 2: return launch_decode_w<T, D, 8, true, 2>(a, ws, t, stream, combine, write);
    default: break;
  }
  if (t.lds_stage) {
    switch (t.decode_waves) {
      case 1: return launch_decode_w<T, D, 1, true, 1>(a, ws, t, stream, combine, write);
      case 2: return launch_decode_w<T, D, 2, true, 1>(a, ws, t, stream, combine, write);
      case 8: return launch_decode_w<T, D, 8, true, 1>(a, ws, t, stream, combine, write);
      default: return launch_decode_w<T, D, 4, true, 1>(a, ws, t, stream, combine, write);
    }
  }
  switch (t.decode_waves) {
    case 1: return launch_decode_w<T, D, 1, false, 1>(a, ws, t, stream, combine, write);
    case 2: return launch_decode_w<T, D, 2, false, 1>(a, ws, t, stream, combine, write);
    case 8: return launch_decode_w<T, D, 8, false, 1>(a, ws, t, stream, combine, write);
    default: return launch_decode_w<T, D, 4, false, 1>(a, ws, t, stream, combine, write);
  }
}

hipError_t launch_paged_attention(const AttnArgs& a, const Workspace& ws, const Tuning& t,
                                  hipStream_t stream, bool combine, const WriteArgs* write) {
  const bool f32 = a.g.dtype == PKV_F32;
  switch (a.g.head_dim) {
    case 64:
      return f32 ? launch_decode_t<float, 64>(a, ws, t, stream, combine, write)
                 : launch_decode_t<uint16_t, 64>(a, ws, t, stream, combine, write);
    case 128:
      return f32 ? launch_decode_t<float, 128>(a, ws, t, stream, combine, write)
                 : launch_decode_t<uint16_t, 128>(a, ws, t, stream, combine, write);
    case 256:
      return f32 ? launch_decode_t<float, 256>(a, ws, t, stream, combine, write)
                 : launch_decode_t<uint16_t, 256>(a, ws, t, stream, combine, write);
    default:
      return hipErrorInvalidValue;
  }
}


static void launch_combine(const AttnArgs& a, const Workspace& ws, hipStream_t stream) {
  const bool f32 = a.g.dtype == PKV_F32;
  switch (a.g.head_dim) {
    case 64:
      f32 ? launch_combine_t<float, 64>(a, ws, stream) : launch_combine_t<uint16_t, 64>(a, ws, stream);
      break;
    case 128:
      f32 ? launch_combine_t<float, 128>(a, ws, stream)
          : launch_combine_t<uint16_t, 128>(a, ws, stream);
      break;
    default:
      f32 ? launch_combine_t<float, 256>(a, ws, stream)
          : launch_combine_t<uint16_t, 256>(a, ws, stream);
      break;
  }
}

hipError_t device_cus(int* cus) {
  static std::atomic<int> count[64];   // per device, computed once
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 64) return hipErrorInvalidDevice;
  int c = count[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    c = n > 0 ? n : 1;
    count[dev].store(c, std::memory_order_relaxed);
  }
  *cus = c;
  return hipSuccess;
}

template <typename T, int D>
static void launch_token_rows(const AttnArgs& a, const SlotArgs& sa, const Workspace& ws,
                              int grid, hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((token_rows_kernel<T, D>), dim3(grid), dim3(kTokenRowThreads), 0,
                     stream, a, sa, ws, scale_log2);
  hipLaunchKernelGGL((token_rows_short_kernel<T, D>), dim3(grid), dim3(kTokenRowThreads), 0,
                     stream, a, sa, ws, scale_log2);
}

hipError_t launch_paged_attention_slots(const AttnArgs& a, const SlotArgs& sa,
                                        const Workspace& ws, const Tuning& t,
                                        hipStream_t stream) {
  // the token kernels: two 4-wave workgroups per CU (measured against one and four)
  int cus = 0;
  hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  const int token_groups = cus * 2;
  AttnArgs b = a;
  b.block_tables = sa.block_tables;
  b.max_blocks = sa.max_blocks;
  b.row_flags = sa.row_flags;
  b.flag_stride = sa.flag_stride;
  b.token_waves = token_groups * (kTokenRowThreads / 64);
  timing_begin(PKV_PHASE_TRANSLATE, stream);
  hipLaunchKernelGGL(translate_slots_kernel, dim3((unsigned)sa.flag_stride, (unsigned)a.num_rows),
                     dim3(kTranslateThreads), 0, stream, b, sa);
  timing_end(PKV_PHASE_TRANSLATE, stream);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_paged_attention(b, ws, t, stream, /*combine=*/false);
  if (err != hipSuccess) return err;
  // the rows the block path could not take, then the merge of every split row: the
  // count is on the device, and with none every workgroup exits at once
  timing_begin(PKV_PHASE_TOKEN_ROWS, stream);
  const bool f32 = a.g.dtype == PKV_F32;
  switch (a.g.head_dim) {
    case 64:
      f32 ? launch_token_rows<float, 64>(b, sa, ws, token_groups, stream)
          : launch_token_rows<uint16_t, 64>(b, sa, ws, token_groups, stream);
      break;
    case 128:
      f32 ? launch_token_rows<float, 128>(b, sa, ws, token_groups, stream)
          : launch_token_rows<uint16_t, 128>(b, sa, ws, token_groups, stream);
      break;
    case 256:
      f32 ? launch_token_rows<float, 256>(b, sa, ws, token_groups, stream)
          : launch_token_rows<uint16_t, 256>(b, sa, ws, token_groups, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  timing_end(PKV_PHASE_TOKEN_ROWS, stream);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  launch_combine(b, ws, stream);
  return hipGetLastError();
}

const char* decode_kernel_name(const AttnArgs& a, const Tuning& t) {
  static const char* const kMfma[] = {"decode_mfma_kernel, 4 query vectors per item",
                                      "decode_mfma_kernel, 8 query vectors per item",
                                      "decode_mfma_kernel, 16 query vectors per item"};
  static const char* const kVec[] = {"decode_kernel, 1 query vector per item",
                                     "decode_kernel, 2 query vectors per item",
                                     "decode_kernel, 4 query vectors per item",
                                     "decode_kernel, 8 query vectors per item"};
  switch (mfma_group_of(a, t)) {
    case 4: return kMfma[0];
    case 8: return kMfma[1];
    case 16: return kMfma[2];
    default: break;
  }
  switch (query_group_of(a, t)) {
    case 2: return kVec[1];
    case 4: return kVec[2];
    case 8: return kVec[3];
    default: return kVec[0];
  }
}

hipError_t scratch_pointer(void** ptr) {
  static std::atomic<void*> addr[64];   // per device, looked up once
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with the device current: its own copy of the array
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);   // racing threads store the same
  }
  *ptr = p;
  return hipSuccess;
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
