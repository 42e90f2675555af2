// Device-side building blocks for the verify kernels (gfx950, wave64).
//
// Logit values are compared as integer keys: a bf16 (or fp32) bit pattern in
// sign-magnitude form is turned into a two's-complement integer and biased to
// an unsigned key, so integer order equals float order, -0 and +0 share one
// key, -inf is the smallest valid key, and NaN / +inf land outside the valid
// range.  Key 0 never occurs and means "no element".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int NT = 1024;         // threads per finisher workgroup (16 wavefronts)
constexpr int NWAVE = NT / 64;
constexpr int KMAX_SPARSE = 512; // largest top-k handled by the streaming select
constexpr uint32_t NONE = 0xFFFFFFFFu;

template <typename ET> struct Key;

// bf16 stored as its 16-bit pattern.
template <> struct Key<uint16_t> {
  static constexpr int VEC = 8;             // elements per 16-byte vector
  static constexpr int LEVELS = 2;          // 8-bit radix digits in a key
  static constexpr uint32_t NEG_INF = 0x8000u - 0x7F80u;
  static constexpr uint32_t POS_INF = 0x8000u + 0x7F80u;
  __device__ __forceinline__ static uint32_t of_bits(uint32_t h) {
    uint32_t mag = h & 0x7FFFu;
    return (h & 0x8000u) ? (0x8000u - mag) : (0x8000u + mag);
  }
  __device__ __forceinline__ static float value(uint32_t uk) {
    uint32_t bits = uk >= 0x8000u ? (uk - 0x8000u) : (0x8000u | (0x8000u - uk));
    return __uint_as_float(bits << 16);
  }
  __device__ __forceinline__ static uint32_t load_key(const uint16_t* row, int i) {
    return of_bits(row[i]);
  }
};

// fp32.
template <> struct Key<float> {
  static constexpr int VEC = 4;
  static constexpr int LEVELS = 4;
  static constexpr uint32_t NEG_INF = 0x80000000u - 0x7F800000u;
  static constexpr uint32_t POS_INF = 0x80000000u + 0x7F800000u;
  __device__ __forceinline__ static uint32_t of_bits(uint32_t b) {
    uint32_t mag = b & 0x7FFFFFFFu;
    return (b & 0x80000000u) ? (0x80000000u - mag) : (0x80000000u + mag);
  }
  __device__ __forceinline__ static float value(uint32_t uk) {
    uint32_t bits = uk >= 0x80000000u ? (uk - 0x80000000u) : (0x80000000u | (0x80000000u - uk));
    return __uint_as_float(bits);
  }
  __device__ __forceinline__ static uint32_t load_key(const float* row, int i) {
    return of_bits(__float_as_uint(row[i]));
  }
};

template <typename ET>
__device__ __forceinline__ bool key_valid(uint32_t uk) {
  return uk >= Key<ET>::NEG_INF && uk < Key<ET>::POS_INF;
}

// ---------------------------------------------------------------------------
// Wave / block reductions (wave64).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
// Inclusive prefix sum across the wave (lane order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Inclusive prefix sum of a 32-bit value across the wave with DPP row shifts
// and row broadcasts (no LDS round trip): within each 16-lane row by
// shifts of 1, 2, 4, 8, then lane 15 of each row added to the next row and
// lane 31 to the upper half.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return (uint32_t)x;
}

// Whole-wave reductions with the same DPP pattern (an inclusive scan whose
// lane 63 holds the result, read back uniformly).  The neutral element fills
// the lanes a shift or broadcast does not reach.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_dpp_u32(uint32_t v, uint32_t neutral, Op op) {
  const int nu = (int)neutral;
  int x = (int)v;
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(nu, x, 0x111, 0xF, 0xF, false));
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(nu, x, 0x112, 0xF, 0xF, false));
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(nu, x, 0x114, 0xF, 0xF, false));
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(nu, x, 0x118, 0xF, 0xF, false));
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(nu, x, 0x142, 0xA, 0xF, false));
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(nu, x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  return wave_reduce_dpp_u32(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  return wave_reduce_dpp_u32(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
// One DPP step of a double: v + (v moved by CTRL within ROWMASK), the 64-bit
// value moving as two halves; unreached lanes add +0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_add_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFFll), CTRL, ROWMASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROWMASK, 0xF, false);
  return v + __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
// Sum of a double over the wave.
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v = dpp_add_f64<0x111, 0xF>(v);
  v = dpp_add_f64<0x112, 0xF>(v);
  v = dpp_add_f64<0x114, 0xF>(v);
  v = dpp_add_f64<0x118, 0xF>(v);
  v = dpp_add_f64<0x142, 0xA>(v);
  v = dpp_add_f64<0x143, 0xC>(v);
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Inclusive prefix sum of a double over the wave (lane order).
__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  v = dpp_add_f64<0x111, 0xF>(v);
  v = dpp_add_f64<0x112, 0xF>(v);
  v = dpp_add_f64<0x114, 0xF>(v);
  v = dpp_add_f64<0x118, 0xF>(v);
  v = dpp_add_f64<0x142, 0xA>(v);
  v = dpp_add_f64<0x143, 0xC>(v);
  return v;
}
// Lane l's double, read uniformly by the whole wave (l wave-uniform).
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Block-wide reductions through a small LDS scratch of NWAVE entries.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T r = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) r += scratch[i];
  __syncthreads();
  return r;
}
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* scratch) {
  v = wave_max_u32(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) r = max(r, scratch[i]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* scratch) {
  v = wave_min_u32(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  uint32_t r = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) r = min(r, scratch[i]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ uint32_t block_or_u32(uint32_t v, uint32_t* scratch) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, 64);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) r |= scratch[i];
  __syncthreads();
  return r;
}

// Block exclusive scan of one value per thread (thread order); returns the
// exclusive prefix and writes the block total to *total.
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* scratch, T* total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  T incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) {
    T s = scratch[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------------------
// Block radix select: the k-th largest key (1-based) of a multiset spread
// over the block's threads.  `feed(fn)` must call fn(key) for every key the
// calling thread holds (keys of 0 are ignored).  Every thread of the block
// calls this with the same k.  Returns the exact k-th largest key, or 0 when
// fewer than k keys exist.  hist: 256 words of LDS; bc: 2 words of LDS.
// ---------------------------------------------------------------------------
template <int LEVELS, int NTHR = NT, class Feed>
__device__ __forceinline__ uint32_t block_kth_largest(Feed feed, uint32_t k, uint32_t* hist, uint32_t* bc) {
  uint32_t prefix = 0, pmask = 0, krem = k;
  for (int lvl = 0; lvl < LEVELS; ++lvl) {
    const int shift = 8 * (LEVELS - 1 - lvl);
    for (int i = threadIdx.x; i < 256; i += NTHR) hist[i] = 0;
    __syncthreads();
    feed([&](uint32_t key) {
      if (key != 0 && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int top = 255 - 4 * lane;
      uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
      uint32_t s = c0 + c1 + c2 + c3;
      uint32_t incl = wave_incl_scan_dpp(s);
      uint32_t excl = incl - s;
      bool hit = excl < krem && incl >= krem;
      unsigned long long any = __ballot(hit);
      if (hit) {
        uint32_t r = krem - excl, d;
        if (c0 >= r) {
          d = top;
        } else if (c0 + c1 >= r) {
          d = top - 1; r -= c0;
        } else if (c0 + c1 + c2 >= r) {
          d = top - 2; r -= c0 + c1;
        } else {
          d = top - 3; r -= c0 + c1 + c2;
        }
        bc[0] = d;
        bc[1] = r;
      }
      if (lane == 0 && any == 0ull) bc[0] = NONE;
    }
    __syncthreads();
    const uint32_t d = bc[0], r = bc[1];
    __syncthreads();
    if (d == NONE) return 0;
    prefix |= d << shift;
    pmask |= 255u << shift;
    krem = r;
  }
  return prefix;
}

// ---------------------------------------------------------------------------
// Wavefront radix select: like block_kth_largest, for the keys the calling
// wavefront's lanes feed; hist is the wavefront's private 256-word LDS
// histogram.  No block barrier.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int LEVELS, class Feed>
__device__ __forceinline__ uint32_t wave_kth(Feed feed, uint32_t k, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0, krem = k;
  for (int lvl = 0; lvl < LEVELS; ++lvl) {
    const int shift = 8 * (LEVELS - 1 - lvl);
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0;
    wave_sync_lds();
    feed([&](uint32_t key) {
      if (key != 0 && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    });
    wave_sync_lds();
    const int top = 255 - 4 * lane;
    const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
    const uint32_t sum = c0 + c1 + c2 + c3;
    const uint32_t incl = wave_incl_scan_dpp(sum);
    const uint32_t excl = incl - sum;
    const bool hit = excl < krem && incl >= krem;
    const unsigned long long any = __ballot(hit);
    wave_sync_lds();
    if (any == 0ull) return 0;
    uint32_t d = 0, r = 0;
    if (hit) {
      r = krem - excl;
      if (c0 >= r) {
        d = top;
      } else if (c0 + c1 >= r) {
        d = top - 1; r -= c0;
      } else if (c0 + c1 + c2 >= r) {
        d = top - 2; r -= c0 + c1;
      } else {
        d = top - 3; r -= c0 + c1 + c2;
      }
    }
    const int src = __ffsll((long long)any) - 1;
    d = (uint32_t)__builtin_amdgcn_readlane((int)d, src);
    r = (uint32_t)__builtin_amdgcn_readlane((int)r, src);
    prefix |= d << shift;
    pmask |= 255u << shift;
    krem = r;
  }
  return prefix;
}

}  // namespace sv
