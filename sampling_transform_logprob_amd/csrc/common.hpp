// Shared device/host definitions of the scoring-core library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stce {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Row flags kept in the per-row state and in the forward's flag array.
enum : uint32_t {
  ROW_VALID = 1u,      // metadata passed validation
  ROW_FILTERED = 2u,   // at least one of top-k / top-p / min-p is active
  ROW_IN_SUPPORT = 4u, // the target lies in the row's support
  ROW_IGNORED = 8u     // inactive row (target equals the problem's ignore_index)
};

// Per-row state written by the forward, read by the backward (32 bytes).
// Field order is the one of stce_row_info in stce.h.
struct RowState {
  uint32_t key_thr;  // key of the last support token (0 on unfiltered rows)
  int32_t id_thr;    // its token id (V - 1 on unfiltered rows)
  int32_t n;         // support size
  uint32_t flags;
  float lse_s;       // log-sum-exp of the keys over the support
  float lse_full;    // log-sum-exp of the keys over the full row
  float m;           // row maximum of the keys
  float s_y;         // key of the target
};
static_assert(sizeof(RowState) == 32, "row state must be 32 bytes");

// Partial statistics of one (row, 256-wide vocabulary tile) block, written by
// the projection epilogue: tile maximum, sum of exp(s - tile max), tile
// minimum, and (when entropies are requested, else 0) the sum of
// exp(s - tile max) * (s - tile max).
struct TilePart {
  float mx;
  float sum;
  float mn;
  float ent;
};

constexpr int VTILE = 256;  // vocabulary columns per partial

// Order-preserving map of an fp32 key to uint32: a larger float gives a
// larger unsigned integer; -0 and +0 map to the same value.
__device__ __host__ inline uint32_t order_key(float s) {
  uint32_t b = __builtin_bit_cast(uint32_t, s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of order_key (for keys of finite values).
__device__ __host__ inline float key_value(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, b);
}

// Composite sort key of (key, token id): a larger composite comes first in
// the support order (larger key, then lower id).
__device__ inline uint64_t composite(uint32_t key, uint32_t id) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ inline uint32_t comp_key(uint64_t c) { return (uint32_t)(c >> 32); }
__device__ inline uint32_t comp_id(uint64_t c) { return 0xffffffffu - (uint32_t)c; }

__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace stce
