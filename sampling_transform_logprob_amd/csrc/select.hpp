// Support program and selected logprob, one workgroup per row.
//
// Inputs per row: the fp32 keys s[0, V) of the row (stored by the projection
// epilogue), the (max, sum exp, min) partials of its 256-wide vocabulary
// tiles, the target key, and the metadata.  Decisions are exact functions of
// the fp32 keys: counts are integers, masses exp(s - m) are fp64, min-p is the
// fp64 comparison s - m >= ln(min_p) with m the unfiltered row maximum.
//
// Every filter keeps a prefix of one order (key descending, lower token id
// first among equal keys).  The row's support is the shortest prefix; its
// last token is found inside a "window" of at most CAP consecutive tokens of
// that order, which is gathered into LDS, sorted by composite (key, ~id) and
// scanned, with the count and the mass of everything ahead of the window
// known.  The window is found by one of:
//   * whole row, when V <= CAP;
//   * bounded candidates: tokens >= the k-th largest tile maximum (a lower
//     bound of the k-th largest key, since the tile maxima are distinct
//     tokens) and passing min-p -- a prefix that contains the support; for a
//     top-k row whose keys were not stored, from the projection's per-tile
//     candidates when every candidate tile's bound (its largest key that is
//     not a candidate) lies below the k-th largest tile maximum, so that the
//     candidates hold every token of that prefix (else the row is re-projected
//     with its keys stored and selected again);
//   * value histogram: NB bins of (m - s) over the row with per-bin counts and
//     fp64 masses; the first bin where a filter crosses is the window;
//   * radix refinement of that bin on the 64-bit composite (key, ~id), 8 bits
//     per pass, when the bin holds more than CAP tokens (ties or very peaked
//     rows).
#pragma once

#include "common.hpp"

namespace stce {

constexpr int ST = 256;     // threads per row
constexpr int CAP = 3712;   // window capacity (composites in LDS); with the
                            // rest of the shared state the kernel stays under
                            // 32 KB, so it fits beside a projection workgroup
constexpr int NB = 512;     // value-histogram bins
constexpr int RB = 256;     // radix bins (8-bit digits)

struct SelParams {
  const float* tile;        // [R][ld] keys
  int64_t ld;
  const TilePart* part;     // [R][ntv]
  int ntv;
  const float* s_y;         // [R] target keys
  const uint32_t* flags;    // [R] ROW_VALID / ROW_FILTERED
  const int64_t* target;    // [R]
  const int32_t* top_k;     // [R] or null
  const float* top_p;       // [R] or null
  const float* min_p;       // [R] or null
  float* logprob;           // [R]
  RowState* state;          // [R]
  RowTiles* tiles;          // [R] or null (more than 65,535 vocabulary tiles)
  RowSupport* support;      // [R] support lists (every row's written), or null
  int V;
  // side outputs, each [R] or null; the entropies need the partials' sums
  float* lse_full;          // log-sum-exp of the keys over the row
  float* ent_full;          // entropy of softmax(s) over the row
  float* ent_supp;          // entropy of the filtered distribution on the support
  int round_lp_bf16;        // the bf16 value lane: logprob rounded to bf16
  // candidates of ROW_CAND rows (the projection's layout; null: every
  // filtered row's keys are in `tile`): a row decides its support from them
  // when they provably hold every token its window needs, else it is added to
  // fail_rows (fail_cnt counts them) and writes nothing
  const float* ckey;
  const uint8_t* cid;
  const float* cbound;
  int64_t cld;
  int* fail_rows;
  int* fail_cnt;
  // re-selection of chosen rows: row r reads keys, partials and target key
  // at r but takes the metadata of row rowmap[r] and writes its outputs
  // there; rows from *n_dev on do nothing (null: identity, all rows)
  const int* rowmap;
  const int* n_dev;
};

void launch_select(const SelParams& p, int rows, hipStream_t stream);

}  // namespace stce
