// Read-only reference kernels for benchmarks: the rate a kernel that does nothing but
// read reaches on this GPU, over a contiguous range (stream_read_kernel) and over the
// scattered pieces a decode read streams (gather_read_kernel for (block, KV head) pieces
// of a few KB, gather_small_kernel for token pieces of at most 1 KB).  They
// touch no decode state and sit in a file of their own, so that changing them leaves the
// decode kernels' source unchanged.
//
// Both use the decode kernels' 16-byte non-temporal loads and fold every word they load
// into one per-thread word; a store that depends on that word (taken only when it
// equals one particular value) keeps every load.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t load16_nt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ uint32_t fold4(u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

constexpr uint32_t kSinkValue = 0x5EED5EEDu;

// ------------------------------------------------------------------------- //
// contiguous
// ------------------------------------------------------------------------- //
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

// Each thread reads 16-byte pieces i, i + 256, ... of its workgroup's runs of
// 256 x kStreamUnroll pieces (32 KB), runs dealt round robin over the grid.
__global__ void __launch_bounds__(kStreamThreads)
stream_read_kernel(const char* src, int64_t pieces, uint32_t* sink) {
  constexpr int64_t kRun = (int64_t)kStreamThreads * kStreamUnroll;
  uint32_t acc = 0;
  for (int64_t run = (int64_t)blockIdx.x * kRun; run < pieces; run += (int64_t)gridDim.x * kRun) {
    u32x4_t v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = run + u * kStreamThreads + threadIdx.x;
      v[u] = i < pieces ? load16_nt(src + i * 16) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= fold4(v[u]);
  }
  if (acc == kSinkValue) sink[0] = acc;   // almost never taken; the loads must happen
}

// ------------------------------------------------------------------------- //
// scattered pieces
// ------------------------------------------------------------------------- //
// The same loads over pieces scattered in two pools.  Wave w of the grid's `waves`
// takes, in pass k, pieces w + (NP k + j) waves (j = 0 .. NP - 1) of the offset list:
// at any moment the grid reads one contiguous window of the list.  Each piece is
// `piece16` 16-byte words at its byte offset of both pools, read in steps of 4 KB per
// piece and pool, every load of a step issued before any is folded (NP x 8 KB a wave
// in flight); the next pass's offsets load while a pass is read.
template <int WAVES, int NP>
__global__ void __launch_bounds__(WAVES * 64)
gather_read_kernel(const char* kb, const char* vb, const int64_t* offsets, int64_t n,
                   int piece16, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * WAVES;
  int64_t p = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  uint32_t acc = 0;
  int64_t off[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) off[j] = p + j * waves < n ? offsets[p + j * waves] : 0;
  for (; p < n; p += NP * waves) {
    int64_t o[NP];
    bool live[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      o[j] = off[j];
      live[j] = p + j * waves < n;
      const int64_t q = p + (NP + j) * waves;
      off[j] = q < n ? offsets[q] : 0;
    }
    for (int base = 0; base < piece16; base += 4 * 64) {
      u32x4_t v[NP][2][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * 64 + lane;
        const int64_t b = (int64_t)i * 16;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          const bool in = live[j] && i < piece16;
          v[j][0][u] = in ? load16_nt(kb + o[j] + b) : u32x4_t{0, 0, 0, 0};
          v[j][1][u] = in ? load16_nt(vb + o[j] + b) : u32x4_t{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int u = 0; u < 4; ++u) acc ^= fold4(v[j][s][u]);
    }
  }
  if (acc == kSinkValue) sink[0] = acc;   // almost never taken; the loads must happen
}

// Pieces of at most 64 16-byte words that divide a wave's 64 lanes (piece16 = 1, 2, 4,
// ..., 64): lane l reads word l % piece16 of piece l / piece16 of its group, so one
// wave load covers 64 / piece16 whole pieces (a one-wave-a-piece read of a 256-byte
// piece would leave 48 of 64 lanes idle).  Group q of the list is pieces
// q * per .. q * per + per - 1 (per = 64 / piece16); wave w of the grid's `waves` takes,
// in pass k, groups w + (NP k + j) waves (j = 0 .. NP - 1), all NP loads of a pass issued
// before any is folded, and the next pass's offsets load while a pass is read.
template <int WAVES, int NP>
__global__ void __launch_bounds__(WAVES * 64)
gather_small_kernel(const char* kb, const char* vb, const int64_t* offsets, int64_t n,
                    int piece16, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int per = 64 / piece16;
  const int64_t part = lane / piece16;             // this lane's piece within a group
  const int64_t word = (int64_t)(lane % piece16) * 16;
  const int64_t waves = (int64_t)gridDim.x * WAVES;
  const int64_t groups = (n + per - 1) / per;
  int64_t q = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  uint32_t acc = 0;
  int64_t off[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int64_t p = (q + j * waves) * per + part;
    off[j] = p < n ? offsets[p] : -1;
  }
  for (; q < groups; q += NP * waves) {
    int64_t o[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      o[j] = off[j];
      const int64_t p = (q + (NP + j) * waves) * per + part;
      off[j] = p < n ? offsets[p] : -1;
    }
    u32x4_t v[NP][2];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const bool in = o[j] >= 0;
      v[j][0] = in ? load16_nt(kb + o[j] + word) : u32x4_t{0, 0, 0, 0};
      v[j][1] = in ? load16_nt(vb + o[j] + word) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) acc ^= fold4(v[j][0]) ^ fold4(v[j][1]);
  }
  if (acc == kSinkValue) sink[0] = acc;   // almost never taken; the loads must happen
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                              int groups_per_cu, hipStream_t stream) {
  int cus = 0;
  hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)(cus * groups_per_cu)),
                     dim3(kStreamThreads), 0, stream, static_cast<const char*>(src), bytes / 16,
                     sink);
  return hipGetLastError();
}

template <int WAVES, int NP>
static void launch_gather(const char* kb, const char* vb, const int64_t* offsets, int64_t n,
                          int piece16, uint32_t* sink, unsigned grid, hipStream_t stream) {
  if (piece16 <= 64 && 64 % piece16 == 0)
    hipLaunchKernelGGL((gather_small_kernel<WAVES, NP>), dim3(grid), dim3(WAVES * 64), 0,
                       stream, kb, vb, offsets, n, piece16, sink);
  else
    hipLaunchKernelGGL((gather_read_kernel<WAVES, NP>), dim3(grid), dim3(WAVES * 64), 0,
                       stream, kb, vb, offsets, n, piece16, sink);
}

hipError_t launch_gather_read(const void* k_base, const void* v_base, const int64_t* offsets,
                              int64_t n_pieces, int32_t piece_bytes, uint32_t* sink,
                              int groups_per_cu, int waves_per_group, int pieces_per_wave,
                              hipStream_t stream) {
  int cus = 0;
  hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  const char* kb = static_cast<const char*>(k_base);
  const char* vb = static_cast<const char*>(v_base);
  const unsigned grid = (unsigned)(cus * groups_per_cu);
  const int p16 = piece_bytes / 16;
  switch (waves_per_group * 8 + pieces_per_wave) {
    case 4 * 8 + 1: launch_gather<4, 1>(kb, vb, offsets, n_pieces, p16, sink, grid, stream); break;
    case 4 * 8 + 2: launch_gather<4, 2>(kb, vb, offsets, n_pieces, p16, sink, grid, stream); break;
    case 4 * 8 + 4: launch_gather<4, 4>(kb, vb, offsets, n_pieces, p16, sink, grid, stream); break;
    case 8 * 8 + 1: launch_gather<8, 1>(kb, vb, offsets, n_pieces, p16, sink, grid, stream); break;
    case 8 * 8 + 2: launch_gather<8, 2>(kb, vb, offsets, n_pieces, p16, sink, grid, stream); break;
    case 8 * 8 + 4: launch_gather<8, 4>(kb, vb, offsets, n_pieces, p16, sink, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
