// Device-side building blocks shared by the kernels of libvce (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Vocabulary shards of one table: shard k owns rows [row[k], row[k+1]) of the
// table (contiguous, in order, possibly empty), and its GEMM tiles are
// tile[k] .. tile[k+1]-1 (tiles never cross a shard end). Passed by value to
// the kernels (launch arguments), so the library keeps no state.
constexpr int kMaxShards = 128;
struct SegTable {
  int64_t row[kMaxShards + 1];
  int32_t tile[kMaxShards + 1];
  int32_t n;
};

// Shard of a row r (0 <= r < row[n]) by binary search over the offsets: the
// last k with row[k] <= r (empty shards are skipped).
__device__ __forceinline__ int shard_of_row(const SegTable& sg, int64_t r) {
  int lo = 0, hi = sg.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sg.row[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Shard of a tile t (0 <= t < tile[n]): the last k with tile[k] <= t.
__device__ __forceinline__ int shard_of_tile(const SegTable& sg, int64_t t) {
  int lo = 0, hi = sg.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sg.tile[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bits <-> float
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two (max, sum of exp(z - max)) pairs into (m, s). A pair with
// m == -inf carries s == 0 and contributes nothing.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = (m == -INFINITY ? 0.0f : s * fast_exp2((m - m2) * kLog2e)) + s2;
    m = m2;
  } else if (m2 != -INFINITY) {
    s += s2 * fast_exp2((m2 - m) * kLog2e);
  }
}

// Blocks are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Renumber so that each XCD walks a contiguous range of logical tiles, which
// then share operand tiles in that XCD's L2.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t b, int64_t total) {
  const int64_t x = b & 7, i = b >> 3;
  const int64_t q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + i;
}

// Wave-wide helpers
__device__ __forceinline__ float wave_shfl_xor(float v, int mask) { return __shfl_xor(v, mask); }

}  // namespace vce
