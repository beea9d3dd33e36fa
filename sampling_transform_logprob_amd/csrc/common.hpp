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

// operand dtypes (stce_dtype): hidden and weight bf16, both fp32, or bf16
// hidden with an e4m3 weight and per-row weight scales (the fp8 lane)
enum : int { DT_BF16 = 1, DT_F32 = 2, DT_FP8 = 3 };

// Row flags kept in the per-row state and in the forward's flag array.
enum : uint32_t {
  ROW_VALID = 1u,      // metadata passed validation
  ROW_FILTERED = 2u,   // at least one of top-k / top-p / min-p is active
  ROW_IN_SUPPORT = 4u, // the target lies in the row's support
  ROW_IGNORED = 8u,    // inactive row (target equals the problem's ignore_index)
  // forward flag only (never in the state): a row bounded by top-k whose
  // projection keeps candidates instead of its fp32 keys (KCAND)
  ROW_CAND = 16u,
  // state flag: the row's support is stored in the state with its keys
  // (RowState's support list, below)
  ROW_LISTED = 32u
};

// Top-k-bounded rows with 0 < k <= KCAND (and at least k vocabulary tiles, at
// most 2 CAP of them: the selection's tile-maximum bound search) keep, per
// (row, 256-token tile), the two largest keys of each of the 8 lanes that
// hold the tile's 256 logits (16 candidates) and the largest key that is
// not a candidate, instead of the row's fp32 keys.
constexpr int KCAND = 256;

// Per-row record of the state written by the forward, read by the backward
// (32 bytes; the tile lists and then the support lists follow the T
// records).
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

// The vocabulary tiles (VTILE columns each) that can hold a row's support
// tokens: every tile whose maximum key reaches the row's last support key,
// in increasing order, when there are at most NTILE of them (n = 0 otherwise,
// and on unfiltered or invalid rows).  Written by the selection after the
// per-row records (the state holds T RowState records, then T RowTiles), read
// by the backward, which recomputes such a row's keys on these tiles only.
constexpr int NTILE = 31;
struct RowTiles {
  uint16_t n;
  uint16_t t[NTILE];
};
static_assert(sizeof(RowTiles) == 64, "tile list must be 64 bytes");

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

// The backward's row classes.  dz = c (1[j == y] - q) is nonzero only on the
// row's support, so a row whose support holds at most NSP tokens ("sparse")
// has at most NSP nonzero dz entries: the recompute emits them as
// (vocabulary row, value) entries and the two gradient products take them
// one by one.  A sparse row whose support the state lists ("listed") takes
// its entries from the stored keys; one with a tile list ("tiled") has its
// keys recomputed on those tiles only.  Rows with a larger support ("dense") go
// through the matrix-core products; rows with no gradient (target out of
// support, invalid or ignored metadata, zero upstream gradient) are "empty".
constexpr int NSP = 128;
enum : int { GRAD_DENSE = 0, GRAD_SPARSE = 1, GRAD_LISTED = 2, GRAD_TILED = 3, GRAD_EMPTY = 4, GRAD_CLASSES = 5 };

// Row counts of the classes, written on the device by the classification:
// rows are placed in the order dense, sparse, listed, tiled, empty, each in
// row order, so dense rows take permuted positions [0, dense), sparse ones
// [dense, full), listed ones [full, listed) and tiled ones [listed, active).
// The whole-vocabulary recompute covers [0, full), the tile recompute
// [listed, active); listed rows need no recompute.
struct GradCounts {
  int dense, full, listed, active;
};

// One nonzero dz entry: a vocabulary row (or, in a weight-gradient bucket,
// a permuted token position) and its fp32 value.
struct SpEntry {
  int32_t idx;
  float v;
};

// A filtered row's support of at most NSP tokens as (token id, key) pairs, in
// decreasing key order (increasing id among equal keys): the selection's
// window when it starts at the top of the order (a top-k row decided from
// its candidates), else gathered from the row's stored keys.  The row is
// then flagged ROW_LISTED and the backward forms its dz entries from these
// keys, recomputing none.
// Entries past the support, and every entry of other rows, are zero.  The
// state holds T RowState records, then T RowTiles, then T support lists.
struct RowSupport {
  SpEntry e[NSP];
};
static_assert(sizeof(RowSupport) == 1024, "support list must be 1 KB");
// bytes of state per row: the record, the tile list and the support list
constexpr int STATE_BYTES_PER_ROW = (int)(sizeof(RowState) + sizeof(RowTiles) + sizeof(RowSupport));

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

// The OCP e4m3 format ("e4m3fn": sign, 4 exponent bits with bias 7, 3
// mantissa bits, subnormals m 2^-9, largest finite value 448, no
// infinities), written from its definition.  Encoding rounds to nearest
// with ties to even and takes |x| <= 448; the matrix cores read the same
// codes.
constexpr float E4M3_MAX = 448.0f;

__device__ inline uint32_t e4m3_encode(float x) {
  const uint32_t s = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
  const float a = __builtin_fabsf(x);
  if (a < 0x1p-6f) return s | (uint32_t)__builtin_rintf(a * 512.0f);  // 0 .. 8 (8: the smallest normal)
  int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xffu) - 127;
  float q = __builtin_rintf(__builtin_ldexpf(a, 3 - e));                // 8 .. 16, exact scaling
  if (q == 16.0f) {
    ++e;
    q = 8.0f;
  }
  return s | (uint32_t)((e + 7) << 3) | ((uint32_t)q - 8u);
}

__device__ inline float e4m3_decode(uint32_t c) {
  const int e = (int)((c >> 3) & 15u);
  const float m = (float)(c & 7u);
  const float v = e ? __builtin_ldexpf(1.0f + m * 0.125f, e - 7) : m * 0x1p-9f;
  return (c & 0x80u) ? -v : v;
}

__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace stce
