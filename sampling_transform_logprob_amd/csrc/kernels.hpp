// Launchers of the library's kernels (host side).
#pragma once

#include "common.hpp"
#include "select.hpp"

namespace stce {

// Launch kinds of the timing hook (the STCE_KERNEL_* values of stce.h).
enum : int {
  KIND_VALIDATE = 1, KIND_PROJECTION = 2, KIND_SELECT = 3, KIND_DLOGITS = 4, KIND_GRAD_WEIGHT = 5,
  KIND_GRAD_HIDDEN = 6, KIND_TRANSPOSE = 7, KIND_PARTIALS = 8, KIND_POLICY_LOSS = 9, KIND_DZ_KEYS = 10,
  KIND_SPLIT_SUM = 11, KIND_PRESCALE = 12, KIND_CLASSIFY = 13, KIND_SPARSE_DW = 14, KIND_SPARSE_DH = 15,
  KIND_REPROJECT = 16, KIND_QUANTIZE = 17, KIND_TILE_LISTS = 18, KIND_TILE_RECOMPUTE = 19,
  KIND_LISTED_ENTRIES = 20
};

// Launch-timing hook (no-op unless a profile is attached to this thread).
void prof_begin(int kind, hipStream_t s);
void prof_end(hipStream_t s);
struct ProfScope {
  hipStream_t s;
  ProfScope(int kind, hipStream_t st) : s(st) { prof_begin(kind, st); }
  ~ProfScope() { prof_end(s); }
};

// Per-row metadata validation: flags[t] = ROW_VALID | ROW_FILTERED | ... or
// 0, and the first bad (row << 8 | field) into *status with an atomic min.
// cand_ok: mark top-k-bounded rows ROW_CAND (the forward keeps candidates for
// them instead of their keys).
hipError_t launch_validate(int64_t T, int64_t V, int ignore, int64_t ignore_index, const float* temp,
                           const int32_t* top_k, const float* top_p,
                           const float* min_p, const int64_t* target, uint32_t* flags, int64_t* status,
                           hipStream_t s, int cand_ok = 0);
hipError_t launch_fill_i64(int64_t* p, int64_t v, hipStream_t s);

// out[c][r] = in[r][c] for r < R, c < Cc; zeros for R <= r < R_pad.
// skip: when not null and *skip == 0 on the device, nothing is written.
hipError_t launch_transpose_bf16(const bf16* in, int64_t ld_in, int64_t R, int64_t Cc, bf16* out,
                                 int64_t ld_out, int64_t R_pad, hipStream_t s, const int* skip = nullptr);
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
  // candidates of ROW_CAND rows (null: none kept), token stride cld
  float* ckey;
  uint8_t* cid;
  float* cbound;
  int64_t cld;
  // re-projection of chosen rows: column n is row rowmap[n] (its metadata),
  // columns from *n_dev on do nothing
  const int* rowmap;
  const int* n_dev;
  // fp8 lane (dtype 3): W holds e4m3 codes, h the chunk's quantized hidden
  // rows; weight scales [V] and the chunk's row scales (indexed like temp)
  const float* row_scale;
  const float* col_scale;
};
hipError_t launch_fwd_projection(const FwdArgs& a, hipStream_t s);

// fp8 lane: for n < T, row t = perm[n] (t = n without perm) of the bf16
// hidden states h (H a multiple of 16): a[t] = fl32(max_k |h[t, k]| / 448)
// (1 for a zero row), q[n, k] = e4m3(clamp(fl32(h[t, k] / a[t]), -448, 448))
// and, when deq is not null, deq[n, k] = bf16(fl32(a[t] e4m3(q[n, k]))).
hipError_t launch_fp8_quantize_rows(const bf16* h, const int* perm, int64_t T, int64_t H, uint8_t* q, float* a,
                                    bf16* deq, hipStream_t s);
// out[c][r] = bf16(fl32(scale[r] * e4m3(in[r][c]))) for r < R, zeros for
// R <= r < R_pad (the transposed dequantized weight of a slice); nothing when
// skip is not null and *skip == 0.
hipError_t launch_fp8_dequant_transpose(const uint8_t* in, const float* scale, int64_t ld_in, int64_t R, int64_t Cc,
                                        bf16* out, int64_t ld_out, int64_t R_pad, const int* skip, hipStream_t s);

// out[r] = in[rowmap[r]] for r < *n_dev (rows of H elements of the dtype, 1
// bf16, 2 fp32 or 3 e4m3 codes, 16-byte rows); rows up to nmax are covered
// by the launch.
hipError_t launch_gather_rows_dev(int dtype, const void* in, const int* rowmap, const int* n_dev, int64_t nmax,
                                  int64_t H, void* out, hipStream_t s);

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
  // parity export: when set, only the recompute product runs, and it also
  // writes the keys it recomputes to keys_out [T][ld_keys] (columns v0 ..)
  float* keys_out;
  int64_t ld_keys;
};
hipError_t launch_bwd_slice(const BwdSliceArgs& a, hipStream_t s);

// ---- the backward with row classes (bf16 operands; sparse.hip) ----------
// Classification: counts of the classes into *cnt, the permutation perm
// (permuted position -> row: dense rows, then sparse, listed, tiled and
// empty ones, each in row order) and a cleared entry counter per position.
// tl: the rows' tile lists (null: no row is tiled); use_lists 0: no row is
// listed (their support lists are ignored).  blk: scratch of
// grad_class_blk_ints(T) ints.
size_t grad_class_blk_ints(int64_t T);
hipError_t launch_grad_classes(const RowState* st, const RowTiles* tl, const float* g, int64_t T, int use_lists,
                               int* blk,
                               GradCounts* cnt, int* perm, int* rowcnt, hipStream_t s);

// The listed rows' dz entries (positions [full, listed)) from the support
// lists of the state, into list / rowcnt by position and, when cntj is not
// null, the per-vocabulary-row counts.  g [T]: upstream gradients by row.
hipError_t launch_listed_entries(const int* perm, const GradCounts* cnt, const RowState* st, const RowSupport* sup,
                                 const float* g, const float* temp, const int64_t* target, int64_t V, int* rowcnt,
                                 SpEntry* list, int* cntj, int64_t T, hipStream_t s);

// Work lists of the tile recompute: per vocabulary tile j < ntv, the tiled
// positions listing it (bucket[toff[j] .. toff[j] + tcnt[j])) and its work
// items (twoff: exclusive scan of ceil(tcnt / TILE_COLS), twoff[ntv] the
// total).  tfill: scratch [ntv]; sums: scratch of scan_sums_ints(ntv).
constexpr int TILE_COLS = 256;  // positions per work item: the product's N tile
struct TileListArgs {
  const int* perm;
  const GradCounts* cnt;
  const RowTiles* tiles;  // [T] by row
  int64_t T, ntv;
  int* tcnt;              // [ntv]
  int* tfill;             // [ntv]
  int* toff;              // [ntv + 1]
  int* twork;             // [ntv]
  int* twoff;             // [ntv + 1]
  int* sums;
  int* bucket;            // [NTILE * T]
};
hipError_t launch_tile_lists(const TileListArgs& a, hipStream_t s);
// out[n] = in[perm[n]] for rows of H elements of the dtype (1 bf16, 2 fp32).
hipError_t launch_gather_rows(int dtype, const void* in, const int* perm, int64_t T, int64_t H, void* out,
                              hipStream_t s);
hipError_t launch_fill_i32(int* p, int64_t n, int v, hipStream_t s);
// Exclusive scan of x[0, n) into y[0, n] (y[n] = the total); sums: scratch
// of scan_sums_ints(n) ints.
size_t scan_sums_ints(int64_t n);
hipError_t launch_exclusive_scan(const int* x, int64_t n, int* sums, int* y, hipStream_t s);

// One vocabulary slice of the classed backward: the recompute product (dense
// rows' dz^T, sparse rows' entries) and the dense rows' two products.
struct ClassSliceArgs {
  const bf16* W;        // full weight [V][H] (bf16)
  // fp8 lane: the weight's e4m3 codes [V][H] and scales [V], the hidden
  // rows' codes in permuted order [T][H] and their scales [rows] (h_perm then
  // holds the dequantized hidden rows, the weight gradient's operand)
  const uint8_t* W8;
  const float* w_scale;
  const uint8_t* h8_perm;
  const float* h_scale;
  const bf16* h_perm;   // [T][H] hidden rows in permuted order
  const int* perm;
  const GradCounts* cnt;
  bf16* WT;             // [H][ld_d] scratch
  bf16* dT;             // [ld_d rows][Tp] scratch: dense rows' dz^T, columns = permuted positions
  float* dh_sum;        // [T][H] fp32 running sum of the dense rows (permuted positions)
  void* grad_hidden;    // [T][H] or null
  float* grad_weight;   // [V][H] or null
  int accumulate_w;
  const float* temp;
  const int64_t* target;
  const RowState* st;
  const float* g;
  int* rowcnt;          // [T]
  SpEntry* list;        // [T][NSP]
  int* cntj;            // [V] (null without grad_weight)
  int64_t T, Tp, H, V, v0, vs, vsp, ld_d;
  int first, last;
  float dh_div;
  int bf16_lane;
  float* keys_out;      // parity export (only the recompute runs), [T][ld_keys]
  int64_t ld_keys;
};
hipError_t launch_class_slice(const ClassSliceArgs& a, hipStream_t s);

// The tile recompute: the keys of the tiled rows (positions [full, active))
// on the vocabulary tiles their lists name, gathered GN positions at a time
// per tile, with the recompute epilogue of the whole-vocabulary product
// (their dz entries and per-vocabulary-row counts).  The hidden rows are
// read by permuted position: the product addresses them with 32-bit offsets,
// so T H bytes (fp8 codes) or 2 T H bytes (bf16) must stay below 2^31 - 2^22.
struct TiledArgs {
  const bf16* W;          // [V][H] bf16, or null with W8
  const uint8_t* W8;      // fp8 lane: [V][H] codes
  const float* w_scale;   // fp8 lane: [V]
  const bf16* h_perm;     // [T][H] permuted hidden rows (bf16)
  const uint8_t* h8_perm; // fp8 lane: their codes
  const float* h_scale;   // fp8 lane: [rows] by row
  const int* perm;
  const GradCounts* cnt;
  const float* temp;
  const int64_t* target;
  const RowState* st;
  const float* g;
  int* rowcnt;
  SpEntry* list;
  int* cntj;              // [V] or null
  int64_t T, H, V;
  int bf16_lane;
  float* keys_out;        // parity export (their listed tiles only), or null
  int64_t ld_keys;
  TileListArgs lists;
};
hipError_t launch_tiled_recompute(const TiledArgs& a, hipStream_t s);

// The sparse rows' products after the last slice: the weight gradient from
// per-vocabulary-row buckets of the entries, the hidden gradient of every
// sparse and empty position.
struct SparseGradArgs {
  int dtype;            // 1 bf16, 2 fp32, 3 fp8 lane (W e4m3 codes with w_scale)
  const void* W;        // [V][H]
  const float* w_scale; // [V] (fp8 lane)
  const void* h_perm;   // [T][H] permuted rows
  const int* perm;
  const GradCounts* cnt;
  const int* rowcnt;
  const SpEntry* list;
  int* cntj;            // [V] entry counts (consumed)
  int* offj;            // [V + 1] scratch: bucket offsets
  int* scan_sums;       // scratch of scan_sums_ints(V)
  SpEntry* bucket;      // [T][NSP] scratch
  void* grad_hidden;    // [T][H] or null
  float* grad_weight;   // [V][H] or null
  int accumulate_w;
  int64_t T, H, V;
  float dh_div;
};
hipError_t launch_sparse_grads(const SparseGradArgs& a, hipStream_t s);

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
