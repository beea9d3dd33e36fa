// Launchers of the library's kernels (host side).
#pragma once

#include "common.hpp"
#include "select.hpp"

namespace stce {

// Launch-timing hook (no-op unless a profile is attached to this thread).
void prof_begin(int kind, hipStream_t s);
void prof_end(hipStream_t s);
struct ProfScope {
  hipStream_t s;
  ProfScope(int kind, hipStream_t st) : s(st) { prof_begin(kind, st); }
  ~ProfScope() { prof_end(s); }
};

// Per-row metadata validation: flags[t] = ROW_VALID | ROW_FILTERED or 0, and
// the first bad (row << 8 | field) into *status with an atomic min.
hipError_t launch_validate(int64_t T, int64_t V, int ignore, int64_t ignore_index, const float* temp,
                           const int32_t* top_k, const float* top_p,
                           const float* min_p, const int64_t* target, uint32_t* flags, int64_t* status,
                           hipStream_t s);
hipError_t launch_fill_i64(int64_t* p, int64_t v, hipStream_t s);

// out[c][r] = in[r][c] for r < R, c < Cc; zeros for R <= r < R_pad.
hipError_t launch_transpose_bf16(const bf16* in, int64_t ld_in, int64_t R, int64_t Cc, bf16* out,
                                 int64_t ld_out, int64_t R_pad, hipStream_t s);
hipError_t launch_transpose_f32(const float* in, int64_t ld_in, int64_t R, int64_t Cc, float* out,
                                int64_t ld_out, int64_t R_pad, hipStream_t s);

// out = in / t for n elements (n a multiple of 8, 16-byte aligned buffers):
// the fp32 quotient rounded to the operand type (dtype 1 bf16, 2 fp32).
hipError_t launch_prescale(int dtype, const void* in, int64_t n, float t, void* out, hipStream_t s);

// (max, sum exp, min) of every (row, 256-wide tile) of given keys, and the
// target key of every row.
hipError_t launch_tile_partials(const float* s, int64_t ld, int64_t R, int64_t V, int ntv,
                                const int64_t* target, TilePart* part, float* s_y, hipStream_t st);

// Forward projection of one chunk of rows with the keys epilogue.
struct FwdArgs {
  int dtype;  // 1 bf16, 2 fp32
  const void* W;
  const void* h;  // first row of the chunk
  int64_t H, V, rows;
  float* tile;
  int64_t ld;
  const float* temp;
  const int64_t* target;
  const uint32_t* flags;
  int store_all;
  TilePart* part;
  int ntv;
  float* s_y;
  int want_ent;  // tile partials carry the entropy sums
  int bf16_lane; // keys of the bf16 value lane
};
hipError_t launch_fwd_projection(const FwdArgs& a, hipStream_t s);

// Per-row policy-gradient loss: objective 1 = CISPO, 2 = clipped surrogate.
hipError_t launch_policy_loss(int objective, float eps_low, float eps_high, float scale, const float* adv,
                              const float* old_lp, const RowState* st, int64_t T, const float* lp, float* loss,
                              float* grad, float* ratio, hipStream_t s);

// One vocabulary slice of the backward.
struct BwdSliceArgs {
  int dtype;
  const void* W;       // full weight [V][H]
  const void* h;       // [T][H]
  const void* hT;      // [H][Tp]
  void* WT;            // [H][ld_WT] scratch
  void* d;             // [Tp][ld_d] scratch
  void* dT;            // [ld_d rows][Tp] scratch
  float* dh_sum;       // [T][H] fp32 running sum (bf16 path) or the fp32 output
  void* grad_hidden;   // [T][H] or null
  float* grad_weight;  // [V][H] or null
  int accumulate_w;
  const float* temp;
  const int64_t* target;
  const RowState* st;
  const float* g;
  int64_t T, Tp, H, V, v0, vs, vsp, ld_d;
  int first, last;
  float dh_div;        // the hidden gradient's final value is divided by it (1 = none)
  int bf16_lane;       // keys of the bf16 value lane
};
hipError_t launch_bwd_slice(const BwdSliceArgs& a, hipStream_t s);

// Gradients of one chunk of the fused policy step, from the chunk's stored
// keys (no recompute product): dz token-major and vocab-major, the chunk's
// hidden-gradient rows as a split-K product over the vocabulary (fp32
// partials summed in split order), and, at the end of a group of chunks whose
// vocab-major dz is kept, the weight gradient with the group's rows as the
// reduction.
struct FusedGradArgs {
  int dtype;
  const float* keys;    // [rows][ld_keys] fp32 keys of the chunk
  int64_t ld_keys;
  const float* temp;    // chunk rows, or null
  const int64_t* target;
  const RowState* st;
  const float* g;       // [rows] d loss / d logprob
  void* d;              // [rows_pad][V_pad] scratch
  void* dT;             // [V_pad][ld_dT] scratch: the group's vocab-major dz; this chunk's at column dT_col
  int64_t ld_dT, dT_col;
  const void* WT;       // [H][V_pad] transposed weight (zero columns V .. V_pad)
  const void* h;        // [T][H] hidden (bf16: read MN-major)
  const void* hT;       // [H][Tp] transposed hidden (fp32)
  int64_t T;
  float* dh_part;       // [splits][rows][H] scratch
  int splits;
  int64_t ks;           // vocabulary columns per split (multiple of 64)
  void* grad_hidden;    // chunk rows [rows][H] or null
  float* grad_weight;   // [V][H] or null
  int accumulate_w;
  // the weight-gradient product of the group ends with this chunk: rows
  // dw_c0 .. dw_c0 + dw_k of hT against dT columns 0 .. dw_k
  int dw;
  int64_t dw_c0, dw_k;
  int64_t rows, rows_pad, Tp, H, V, V_pad;
  float dh_div;         // the hidden-gradient rows are divided by it (1 = none)
};
hipError_t launch_fused_chunk_grads(const FusedGradArgs& a, hipStream_t s);

}  // namespace stce
