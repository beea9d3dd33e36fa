// Epilogues of the block-tiled product (accumulator layout in gemm.hpp).
#pragma once

#include "gemm.hpp"

namespace stce {

#define STCE_INF __builtin_huge_valf()

// Merge of two (max, sum of exp(x - max), sum of exp(x - max) (x - max))
// partials; max = -inf means "empty".  Re-based on the new maximum M, a
// part's entropy sum gains (max - M) times its mass; an empty part adds
// nothing.
__device__ inline void lse_ent_merge(float& mx, float& sm, float& en, float omx, float osm, float oen) {
  const float M = fmaxf(mx, omx);
  if (M == -STCE_INF) {
    sm = 0.f;
    en = 0.f;
  } else {
    float e = 0.f;
    if (mx != -STCE_INF) e += (en + (mx - M) * sm) * __expf(mx - M);
    if (omx != -STCE_INF) e += (oen + (omx - M) * osm) * __expf(omx - M);
    en = e;
    sm = __builtin_fmaf(sm, __expf(mx - M), osm * __expf(omx - M));
  }
  mx = M;
}

// The same merge of (max, mass) alone; its mass arithmetic is lse_ent_merge's.
__device__ inline void lse_merge(float& mx, float& sm, float omx, float osm) {
  const float M = fmaxf(mx, omx);
  sm = M == -STCE_INF ? 0.f : __builtin_fmaf(sm, __expf(mx - M), osm * __expf(omx - M));
  mx = M;
}

// Per-row temperature: s = fl32(z / T), correctly rounded.  With the row's
// correctly rounded reciprocal r = fl32(1 / T), q0 = fl32(z r) is within one
// ulp of z / T, an fma gives the remainder z - q0 T exactly, and one more fma
// rounds q0 + (z - q0 T) r to the correctly rounded quotient (Markstein's
// correction step, as used for IA-64 division).  That needs the remainder and
// the quotient to stay normal numbers, which holds when 2^-90 <= |z| <= 2^90
// and 2^-30 <= T <= 2^30; a lane column with any value outside that range
// (zeros included) takes the IEEE division instead.  Both give the same bits,
// so the choice cannot make the forward and the backward disagree.
__device__ inline float quot_fast(float z, float t, float r) {
  const float q0 = z * r;
  return __builtin_fmaf(__builtin_fmaf(-q0, t, z), r, q0);
}

// Scales the lane's accumulators of column j (one token) by 1 / t in place.
__device__ inline void scale_column(AccTile& acc, int j, float t) {
  if (t == 1.0f) return;  // exact
  float lo = STCE_INF, hi = 0.f;
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int r = 0; r < ACC_R; ++r) {
      lo = fminf(lo, __builtin_fabsf(acc[i][j][r]));
      hi = fmaxf(hi, __builtin_fabsf(acc[i][j][r]));
    }
  if (lo >= 0x1p-90f && hi <= 0x1p+90f && t >= 0x1p-30f && t <= 0x1p+30f) {
    const float r = 1.0f / t;
#pragma unroll
    for (int i = 0; i < ACC_I; ++i)
#pragma unroll
      for (int q = 0; q < ACC_R; ++q) acc[i][j][q] = quot_fast(acc[i][j][q], t, r);
  } else {
#pragma unroll
    for (int i = 0; i < ACC_I; ++i)
#pragma unroll
      for (int q = 0; q < ACC_R; ++q) acc[i][j][q] = acc[i][j][q] / t;
  }
}

// The keys of column j from its fp32 products: s = fl32(z / t), or in the
// bf16 value lane s = bf16(fl32(bf16(z) / t)) (both roundings to nearest,
// ties to even).
__device__ inline void round_column_bf16(AccTile& acc, int j) {
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int r = 0; r < ACC_R; ++r) acc[i][j][r] = (float)(bf16)acc[i][j][r];
}
__device__ inline void keys_column(AccTile& acc, int j, float t, bool bf16_lane) {
  if (bf16_lane) round_column_bf16(acc, j);
  scale_column(acc, j, t);
  if (bf16_lane && t != 1.0f) round_column_bf16(acc, j);
}

constexpr float LOG2E = 1.4426950408889634f;

// fp8 lane: the products of e4m3 codes scaled back, z = fl32(fl32(acc sW[m])
// a[n]), for the lane's rows of column j; sw[i][r] holds sW of row
// acc_row(wm, i, r, quad) (no contraction: each product is rounded).
__device__ inline void load_row_scales(const float* row_scale, int mb, int quad, int rows, float (&sw)[ACC_I][ACC_R]) {
#pragma unroll
  for (int i = 0; i < ACC_I; ++i) {
    const int m = mb + i * 16 + quad * 4;
#pragma unroll
    for (int r = 0; r < ACC_R; ++r) sw[i][r] = m + r < rows ? row_scale[m + r] : 0.0f;
  }
}
__device__ inline void scale_column_fp8(AccTile& acc, int j, const float (&sw)[ACC_I][ACC_R], float a) {
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int r = 0; r < ACC_R; ++r) acc[i][j][r] = __fmul_rn(__fmul_rn(acc[i][j][r], sw[i][r]), a);
}

// ---------------------------------------------------------------------------
// Forward projection epilogue.  M = vocabulary, N = tokens of the chunk.
// For each (token, 256-wide vocabulary tile): applies the temperature,
// stores the fp32 keys (rows flagged ROW_FILTERED but not ROW_CAND, or all
// rows with store_all), or, for ROW_CAND rows, the tile's candidates: each
// of the 8 lanes holding the token's 256 logits of the tile keeps its two
// largest keys (the lower token id first among equal keys) and the largest
// of the rest; the 16 keys and their tile-local ids are stored, and the
// largest non-candidate key over the 8 lanes as the tile's bound (every key
// above the bound is a candidate).  Writes the tile's (max, sum exp(s - max),
// min) and captures the target key.
// ---------------------------------------------------------------------------
template <bool Ent>
struct EpiLogits {
  float* tile;             // [N][ld] keys, row = token
  int64_t ld;
  const float* temp;       // [N] or null (= 1)
  const int64_t* target;   // [N] or null
  const uint32_t* flags;   // [N] or null (with store_all)
  int store_all;
  int vec;                 // ld and the tile base allow 16-byte stores
  TilePart* part;          // [N][ntv]
  int ntv;
  float* s_y;              // [N] or null
  int V;                   // valid vocabulary rows
  int N;                   // valid tokens
  int bf16_lane;           // keys of the bf16 value lane
  // candidates of ROW_CAND rows: ckey / cid [ntv][2][cld][8] (tile, half of
  // the tile held by wave row wm, token, lane quad * 2 + rank), cbound
  // [cld][ntv]; null when no row is a candidate row
  float* ckey = nullptr;
  uint8_t* cid = nullptr;
  float* cbound = nullptr;
  int64_t cld = 0;
  // re-projection of chosen rows: column n carries row rowmap[n]'s metadata
  // and only columns below *n_dev exist (null: identity, N)
  const int* rowmap = nullptr;
  const int* n_dev = nullptr;
  // fp8 lane: per vocabulary row weight scales [V] and per token row scales
  // (indexed like the metadata), or null
  const float* row_scale = nullptr;
  const float* col_scale = nullptr;
  static constexpr int LDS_BYTES = 2 * GN * 5 * 4;  // cross-wave merge

  __device__ inline void operator()(AccTile& acc, int m0, int n0, char* smem, char*) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3, quad = lane >> 4, col = lane & 15;
    const int mb = m0 + wm * 128;
    const bool full = m0 + GM <= V;
    const int Nn = n_dev ? min(N, *n_dev) : N;
    float pmx[ACC_J], psm[ACC_J], pmn[ACC_J], pen[ACC_J], pbd[ACC_J];
    // Every per-token load comes first: loads and stores share one in-order
    // counter, so a load issued after a column's key stores would make the
    // wave wait for all of them to complete before the next column.
    float tv[ACC_J], av[ACC_J];
    bool stv[ACC_J], cnd[ACC_J];
    int64_t tgv[ACC_J];
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int n = n0 + acc_col(wn, j, col);
      const bool nv = n < Nn;
      const int rn = (nv && rowmap) ? rowmap[n] : n;
      const uint32_t f = (nv && flags) ? flags[rn] : 0u;
      tv[j] = (nv && temp) ? temp[rn] : 1.0f;
      av[j] = (nv && col_scale) ? col_scale[rn] : 1.0f;
      cnd[j] = nv && !store_all && ckey && (f & ROW_CAND);
      stv[j] = nv && (store_all || ((f & ROW_FILTERED) && !cnd[j]));
      tgv[j] = (nv && target && s_y) ? target[rn] : -1;
    }
    float sw[ACC_I][ACC_R];
    if (row_scale) load_row_scales(row_scale, mb, quad, V, sw);
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int n = n0 + acc_col(wn, j, col);
      if (row_scale) scale_column_fp8(acc, j, sw, av[j]);
      keys_column(acc, j, tv[j], bf16_lane);
      float mx = -STCE_INF, mn = STCE_INF;
      if (full) {
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int r = 0; r < ACC_R; ++r) {
            mx = fmaxf(mx, acc[i][j][r]);
            mn = fminf(mn, acc[i][j][r]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int r = 0; r < ACC_R; ++r)
            if (m0 + acc_row(wm, i, r, quad) < V) {
              mx = fmaxf(mx, acc[i][j][r]);
              mn = fminf(mn, acc[i][j][r]);
            }
      }
      float bnd = -STCE_INF;  // the lane's largest non-candidate key
      if (cnd[j]) {
        // the lane's two largest keys, visited in increasing token id (a
        // later equal key does not displace an earlier one)
        float a = -STCE_INF, b = -STCE_INF, c = -STCE_INF;
        int ia = 0, ib = 0;
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int r = 0; r < ACC_R; ++r) {
            const int ml = wm * 128 + i * 16 + quad * 4 + r;
            const float v = (full || m0 + ml < V) ? acc[i][j][r] : -STCE_INF;
            const bool ga = v > a, gb = v > b;
            c = gb ? b : fmaxf(c, v);
            b = ga ? a : (gb ? v : b);
            ib = ga ? ia : (gb ? ml : ib);
            a = ga ? v : a;
            ia = ga ? ml : ia;
          }
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const int64_t rec = ((int64_t)(m0 / VTILE) * 2 + wm) * cld + n;
        *(f32x2*)(ckey + rec * 8 + quad * 2) = f32x2{a, b};
        *(uint16_t*)(cid + rec * 8 + quad * 2) = (uint16_t)(ia | (ib << 8));
        bnd = c;
      }
      if (stv[j]) {
        float* rowp = tile + (int64_t)n * ld;
        const int mbu = __builtin_amdgcn_readfirstlane(mb);
#pragma unroll
        for (int i = 0; i < ACC_I; ++i) {
          const int base = mbu + i * 16;  // the wave's 16 rows (uniform)
          const int mm = base + quad * 4;
          if (vec && base + 16 <= V) {
            *(f32x4*)(rowp + mm) = acc[i][j];
          } else {
#pragma unroll
            for (int e = 0; e < ACC_R; ++e)
              if (mm + e < V) rowp[mm + e] = acc[i][j][e];
          }
        }
      }
      if (tgv[j] >= 0) {
        const int64_t off = tgv[j] - mb;
        if (off >= 0 && off < 128) {
          const int oi = (int)off >> 4, ow = (int)off & 15;
          if ((ow >> 2) == quad) {
            const int orr = ow & 3;
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < ACC_I; ++i)
#pragma unroll
              for (int r = 0; r < ACC_R; ++r)
                if (i == oi && r == orr) v = acc[i][j][r];
            s_y[n] = v;
          }
        }
      }
      // the tile's mass and, with Ent, its entropy sum, in a separate
      // accumulator: the mass arithmetic is the same in both instances, so
      // the mass (and every decision and logprob that uses it) does not
      // depend on whether the entropy is requested
      float sm = 0.f, en = 0.f;
      if (mx != -STCE_INF) {
        const float nmx = -mx * LOG2E;
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int r = 0; r < ACC_R; ++r)
            if (full || m0 + acc_row(wm, i, r, quad) < V) {
              const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][r], LOG2E, nmx));
              sm += e;
              if (Ent) en = __builtin_fmaf(e, acc[i][j][r] - mx, en);
            }
      }
      // merge the four lanes that hold this column (quads 0..3)
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float omx = __shfl_xor(mx, o), osm = __shfl_xor(sm, o), omn = __shfl_xor(mn, o);
        if (Ent) {
          lse_ent_merge(mx, sm, en, omx, osm, __shfl_xor(en, o));
        } else {
          lse_merge(mx, sm, omx, osm);
        }
        mn = fminf(mn, omn);
        bnd = fmaxf(bnd, __shfl_xor(bnd, o));
      }
      pmx[j] = mx;
      psm[j] = sm;
      pmn[j] = mn;
      pen[j] = en;
      pbd[j] = bnd;
    }
    // merge the two waves that share these tokens (wm = 0 and 1)
    __syncthreads();
    float* red = (float*)smem;  // [2][256][5]
    if (quad == 0) {
#pragma unroll
      for (int j = 0; j < ACC_J; ++j) {
        const int tok = acc_col(wn, j, col);
        red[(wm * 256 + tok) * 5 + 0] = pmx[j];
        red[(wm * 256 + tok) * 5 + 1] = psm[j];
        red[(wm * 256 + tok) * 5 + 2] = pmn[j];
        if (Ent) red[(wm * 256 + tok) * 5 + 3] = pen[j];
        red[(wm * 256 + tok) * 5 + 4] = pbd[j];
      }
    }
    __syncthreads();
    if (wm == 0 && quad == 0) {
#pragma unroll
      for (int j = 0; j < ACC_J; ++j) {
        const int tok = acc_col(wn, j, col);
        const int n = n0 + tok;
        if (n < Nn) {
          float mx = red[tok * 5 + 0], sm = red[tok * 5 + 1], en = 0.f;
          if (Ent) {
            en = red[tok * 5 + 3];
            lse_ent_merge(mx, sm, en, red[(256 + tok) * 5 + 0], red[(256 + tok) * 5 + 1], red[(256 + tok) * 5 + 3]);
          } else {
            lse_merge(mx, sm, red[(256 + tok) * 5 + 0], red[(256 + tok) * 5 + 1]);
          }
          TilePart tp;
          tp.mx = mx;
          tp.sum = sm;
          tp.mn = fminf(red[tok * 5 + 2], red[(256 + tok) * 5 + 2]);
          tp.ent = en;
          part[(int64_t)n * ntv + m0 / VTILE] = tp;
          if (cnd[j]) cbound[(int64_t)n * ntv + m0 / VTILE] = fmaxf(red[tok * 5 + 4], red[(256 + tok) * 5 + 4]);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Backward recompute epilogue.  M = vocabulary rows of one slice (local index
// m, global v0 + m), N = tokens.  Recomputes the keys exactly as EpiLogits
// does, re-derives support membership from the saved boundary, and writes
//   dz[t, v] = c_t * (1[v == y_t] - exp(s - lse_S) * 1[v in S_t]),
//   c_t = g_t / T_t on rows whose target is in support, else 0,
// rounded to the operand type, vocab-major (dT [v][t]: the weight gradient
// reads it K-major, the hidden gradient MN-major).  The fp32 path, whose
// products take K-major operands only, also writes it token-major (d).
// Padding rows/columns (m >= Vs, n >= N, up to the padded sizes) get zeros.
// ---------------------------------------------------------------------------
template <class OutT>
struct EpiDlogits {
  const float* temp;       // [N] or null
  const int64_t* target;   // [N]
  const RowState* st;      // [N]
  const float* g;          // [N]
  OutT* d;                 // [N_pad][ld_d] (fp32 only)
  int64_t ld_d;
  OutT* dT;                // [Vs_pad][ld_dT]
  int64_t ld_dT;
  int v0, Vs, Vs_pad, N, N_pad;
  int bf16_lane = 0;       // keys of the bf16 value lane
  // parity export (null in every production launch): the recomputed keys of
  // the tile, keys_out[n * ld_keys + v0 + m], for n < N and m < Vs
  float* keys_out = nullptr;
  int64_t ld_keys = 0;
  // bf16: the vocab-major tile leaves through LDS, 128 rows in each of the
  // two epilogue buffers
  static constexpr int LDS_BYTES = sizeof(OutT) == 2 ? 128 * GN * 2 : 0;

  // fn(i, j, n, mm, v): the dz values v[0..3] of rows mm .. mm + 3 (block i)
  // of column n (j), for the lane's columns below N_pad and rows below Vs_pad
  template <class Fn>
  __device__ inline void each(AccTile& acc, int m0, int n0, int wmu, int wn, int quad, int col, Fn&& fn) const {
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int n = n0 + acc_col(wn, j, col);
      const bool nv = n < N;
      const float t = (nv && temp) ? temp[n] : 1.0f;
      RowState rs{};
      float c = 0.f;
      int yy = -1;
      if (nv) {
        rs = st[n];
        yy = (int)target[n];
        if ((rs.flags & (ROW_VALID | ROW_IN_SUPPORT)) == (ROW_VALID | ROW_IN_SUPPORT)) c = g[n] / t;
      }
      if (n >= N_pad) continue;
      keys_column(acc, j, t, bf16_lane);
      if (keys_out && nv) {
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int e = 0; e < ACC_R; ++e) {
            const int m = m0 + wmu * 128 + i * 16 + quad * 4 + e;
            if (m < Vs) keys_out[(int64_t)n * ld_keys + v0 + m] = acc[i][j][e];
          }
      }
      // support membership as a float compare against the boundary key's
      // value (-0 == +0 like the canonical keys); unfiltered rows keep all
      const float sthr = (rs.flags & ROW_FILTERED) ? key_value(rs.key_thr) : -STCE_INF;
      const int idt = rs.id_thr;
      const float nl = -rs.lse_s * LOG2E;
      const bool live = c != 0.f;  // rows with c == 0 give exact zeros
#pragma unroll
      for (int i = 0; i < ACC_I; ++i) {
        // the wave's 16 rows base .. base + 15 (Vs_pad is a multiple of 64,
        // so they are all in or all out): a uniform test
        const int base = m0 + wmu * 128 + i * 16;
        if (base >= Vs_pad) continue;
        const int mm = base + quad * 4;  // this lane's 4 consecutive rows
        OutT v[ACC_R];
#pragma unroll
        for (int e = 0; e < ACC_R; ++e) {
          const int m = mm + e;
          const int vg = v0 + m;
          const float s = acc[i][j][e];
          const bool in = (s > sthr) | ((s == sthr) & (vg <= idt));
          const float q = in ? __builtin_amdgcn_exp2f(__builtin_fmaf(s, LOG2E, nl)) : 0.f;
          const float dv = c * ((vg == yy ? 1.f : 0.f) - q);
          v[e] = (OutT)((live && m < Vs) ? dv : 0.f);
        }
        fn(i, j, n, mm, v);
      }
    }
  }

  __device__ inline void operator()(AccTile& acc, int m0, int n0, char* smem, char* smem1) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3, quad = lane >> 4, col = lane & 15;
    const int wmu = __builtin_amdgcn_readfirstlane(wm);
    if constexpr (sizeof(OutT) == 2) {
      // rows 0 .. 127 of the tile (the waves with wm == 0) are staged in the
      // first buffer, rows 128 .. 255 in the second, as 512-byte rows whose
      // 16-byte chunk c sits at c ^ 2 ((r >> 2) & 3): the four quads of a
      // wave's store (rows 4 apart) then hit distinct banks; then every
      // thread copies out 16-byte row segments
      OutT* stg = (OutT*)(wmu ? smem1 : smem);
      each(acc, m0, n0, wmu, wn, quad, col, [&](int, int, int n, int mm, OutT(&v)[ACC_R]) {
        const int nl = n - n0, r0 = mm - m0 - wmu * 128;  // r0 = i*16 + quad*4
        const int pc = (nl >> 3) ^ (2 * quad);
#pragma unroll
        for (int e = 0; e < ACC_R; ++e) stg[(r0 + e) * GN + pc * 8 + (nl & 7)] = v[e];
      });
      __syncthreads();
      const int rows = min(GM, Vs_pad - m0), cols = min(GN, N_pad - n0);
      for (int q = tid; q < GM * (GN / 8); q += GTHREADS) {
        const int r = q / (GN / 8), cc = q % (GN / 8);
        const OutT* src = (const OutT*)(r < 128 ? smem : smem1) + (r & 127) * GN;
        if (r < rows && cc * 8 < cols)
          *(u32x4*)(dT + (int64_t)(m0 + r) * ld_dT + n0 + cc * 8) =
              *(const u32x4*)(src + ((cc ^ (2 * ((r >> 2) & 3))) * 8));
      }
    } else {
      each(acc, m0, n0, wmu, wn, quad, col, [&](int, int, int n, int mm, OutT(&v)[ACC_R]) {
        OutT* dr = d + (int64_t)n * ld_d;
#pragma unroll
        for (int e = 0; e < ACC_R; ++e) dr[mm + e] = v[e];
#pragma unroll
        for (int e = 0; e < ACC_R; ++e) dT[(int64_t)(mm + e) * ld_dT + n] = v[e];
      });
    }
  }
};

// ---------------------------------------------------------------------------
// Backward recompute epilogue with row classes (bf16 operands).  M =
// vocabulary rows of one slice (local m, global v0 + m), N = permuted token
// positions: position n holds row perm[n]; positions [0, dense) are dense
// rows, [dense, full) sparse rows, [full, active) tiled rows, the rest empty
// (GradCounts).  The whole-vocabulary recompute leaves the tiled rows alone;
// the tile recompute (colpos set) takes its columns' positions from colpos
// and treats them as the sparse rows.  Recomputes
// the keys exactly as EpiLogits does and re-derives support membership from
// the saved boundary, as EpiDlogits does, with the same dz arithmetic
//   dz[t, v] = c_t (1[v == y_t] - exp(s - lse_S) 1[v in S_t]),  c_t = g_t / T_t.
// Dense rows: dz rounded to bf16, vocab-major into dT [v][n] (a tile holding
// any dense position writes all its columns, zeros past the dense ones, so
// the products reading dT over k = n < dense see zeros in the padding).
// Sparse rows: every dz of a support token (the only nonzero ones), rounded
// to bf16 as the dense rows' are, is appended to the position's entry list
// (list[n * NSP + slot], slot from rowcnt[n]), and counted per vocabulary row
// in cntj for the weight gradient's buckets.
// ---------------------------------------------------------------------------
// FP8: the fp8 lane's scalings (row_scale, col_scale); TILED: the tile
// recompute's column positions (colpos).  Both are compile-time so that the
// bf16 whole-vocabulary instance carries neither.
template <bool FP8, bool TILED>
struct EpiGradT {
  const int* perm;          // [N] permuted position -> row
  const GradCounts* cnt;
  const float* temp;        // [rows] or null
  const int64_t* target;
  const RowState* st;
  const float* g;
  bf16* dT;                 // [Vs_pad][ld_dT]
  int64_t ld_dT;
  int v0, Vs, Vs_pad, N, N_pad;
  int bf16_lane;
  int* rowcnt;              // [N]
  SpEntry* list;            // [N][NSP]
  int* cntj;                // [V] or null (no weight gradient)
  float* keys_out = nullptr;  // parity export of the keys, [rows][ld_keys] (null in production)
  int64_t ld_keys = 0;
  // fp8 lane: weight scales of the slice's rows [Vs] and per-row hidden
  // scales [rows] (indexed by row, not position), or null
  const float* row_scale = nullptr;
  const float* col_scale = nullptr;
  // tile recompute: column c < ncols is position colpos[c] (a tiled row)
  const int* colpos = nullptr;
  int ncols = 0;
  static constexpr int LDS_BYTES = 128 * GN * 2;

  __device__ inline void operator()(AccTile& acc, int m0, int n0, char* smem, char* smem1) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3, quad = lane >> 4, col = lane & 15;
    const int wmu = __builtin_amdgcn_readfirstlane(wm);
    // rows with a gradient this product forms: dense and sparse ones, or the
    // tiled ones of colpos; the whole-vocabulary product exports no keys of
    // the tiled rows (the tile recompute exports theirs)
    const int nd = cnt->dense, nf = cnt->full, na = TILED ? cnt->active : nf, nt = cnt->active;
    const bool any_dense = !TILED && n0 < nd;  // uniform over the workgroup
    bf16* stg = (bf16*)(wmu ? smem1 : smem);
    // every per-token load first (loads and stores share one in-order counter)
    float tv[ACC_J], cv[ACC_J], thr[ACC_J], nlv[ACC_J], av[ACC_J];
    int idt[ACC_J], yv[ACC_J], rowv[ACC_J], nv[ACC_J];
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int cc = n0 + acc_col(wn, j, col);
      const int n = TILED ? (cc < ncols ? colpos[cc] : N) : cc;
      nv[j] = n;
      const int t = n < N ? perm[n] : -1;  // the row at this position
      RowState rs{};
      float tt = 1.0f, c = 0.f;
      int y = -1;
      if (t >= 0 && temp) tt = temp[t];
      if (n < na) {  // a row with a gradient (dense or sparse)
        rs = st[t];
        y = (int)target[t];
        if ((rs.flags & (ROW_VALID | ROW_IN_SUPPORT)) == (ROW_VALID | ROW_IN_SUPPORT)) c = g[t] / tt;
      }
      rowv[j] = t;
      tv[j] = tt;
      if constexpr (FP8) av[j] = t >= 0 ? col_scale[t] : 1.0f;
      cv[j] = c;
      thr[j] = (rs.flags & ROW_FILTERED) ? key_value(rs.key_thr) : -STCE_INF;
      idt[j] = rs.id_thr;
      nlv[j] = -rs.lse_s * LOG2E;
      yv[j] = y;
    }
    float sw[ACC_I][ACC_R];
    if constexpr (FP8) load_row_scales(row_scale, m0 + wmu * 128, quad, Vs, sw);
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int n = nv[j];
      if constexpr (FP8) scale_column_fp8(acc, j, sw, av[j]);
      keys_column(acc, j, tv[j], bf16_lane);
      if (keys_out && rowv[j] >= 0 && (TILED || n < nf || n >= nt)) {
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int e = 0; e < ACC_R; ++e) {
            const int m = m0 + wmu * 128 + i * 16 + quad * 4 + e;
            if (m < Vs) keys_out[(int64_t)rowv[j] * ld_keys + v0 + m] = acc[i][j][e];
          }
      }
      const float c = cv[j], sthr = thr[j], nl = nlv[j];
      const int it = idt[j], y = yv[j];
      const bool live = c != 0.f;
      const bool dense = n < nd, sparse = live && !dense && n < na;
      const int nl_ = n - n0;  // (the dense staging column: whole-vocabulary product only)
#pragma unroll
      for (int i = 0; i < ACC_I; ++i) {
        const int base = m0 + wmu * 128 + i * 16;  // the wave's 16 rows (uniform)
        if (base >= Vs_pad) continue;
        const int mm = base + quad * 4;
        float dv[ACC_R];
        bool in[ACC_R];
#pragma unroll
        for (int e = 0; e < ACC_R; ++e) {
          const int m = mm + e;
          const int vg = v0 + m;
          const float s = acc[i][j][e];
          in[e] = ((s > sthr) | ((s == sthr) & (vg <= it))) && m < Vs;
          const float q = in[e] ? __builtin_amdgcn_exp2f(__builtin_fmaf(s, LOG2E, nl)) : 0.f;
          dv[e] = c * ((vg == y ? 1.f : 0.f) - q);
        }
        if (any_dense) {
          const int r0 = mm - m0 - wmu * 128;  // i*16 + quad*4
          const int pc = (nl_ >> 3) ^ (2 * quad);
#pragma unroll
          for (int e = 0; e < ACC_R; ++e)
            stg[(r0 + e) * GN + pc * 8 + (nl_ & 7)] = (bf16)((dense && live && mm + e < Vs) ? dv[e] : 0.f);
        }
        if (sparse) {
#pragma unroll
          for (int e = 0; e < ACC_R; ++e) {
            if (in[e]) {
              const int slot = atomicAdd(rowcnt + n, 1);
              if (slot < NSP) {
                // rounded to bf16 like the dense rows' dz: a row's gradient
                // does not depend on its class beyond fp32 summation order
                list[(int64_t)n * NSP + slot] = SpEntry{v0 + mm + e, (float)(bf16)dv[e]};
                if (cntj) atomicAdd(cntj + v0 + mm + e, 1);
              }
            }
          }
        }
      }
    }
    if (any_dense) {
      __syncthreads();
      const int rows = min(GM, Vs_pad - m0), cols = min(GN, N_pad - n0);
      for (int q = tid; q < GM * (GN / 8); q += GTHREADS) {
        const int r = q / (GN / 8), cc = q % (GN / 8);
        const bf16* src = (const bf16*)(r < 128 ? smem : smem1) + (r & 127) * GN;
        if (r < rows && cc * 8 < cols)
          *(u32x4*)(dT + (int64_t)(m0 + r) * ld_dT + n0 + cc * 8) =
              *(const u32x4*)(src + ((cc ^ (2 * ((r >> 2) & 3))) * 8));
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Plain fp32 store (weight gradient slice): out[m, n] (+)= acc.
// ---------------------------------------------------------------------------
struct EpiStore {
  float* out;
  int64_t ld;
  int M, N;
  int accumulate;
  static constexpr int LDS_BYTES = 0;

  __device__ inline void operator()(AccTile& acc, int m0, int n0, char*, char*) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3, quad = lane >> 4, col = lane & 15;
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int n = n0 + acc_col(wn, j, col);
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < ACC_I; ++i)
#pragma unroll
        for (int r = 0; r < ACC_R; ++r) {
          const int m = m0 + acc_row(wm, i, r, quad);
          if (m < M) {
            float* p = out + (int64_t)m * ld + n;
            *p = accumulate ? *p + acc[i][j][r] : acc[i][j][r];
          }
        }
    }
  }
};

// ---------------------------------------------------------------------------
// Hidden-gradient accumulation over vocabulary slices: sum[m, n] = (first ? 0 :
// sum[m, n]) + acc; on the last slice the result goes to `out` (OutT) instead.
// The slices are visited in a fixed order, so the sum is deterministic.
// ---------------------------------------------------------------------------
template <class OutT>
struct EpiAccum {
  float* sum;  // [M][ld] fp32 running sum (may alias out when OutT is float)
  int64_t ld;
  OutT* out;   // [M][ld]
  int M, N;
  int first, last;
  float div = 1.f;  // the last slice writes (sum + acc) / div
  static constexpr int LDS_BYTES = 0;

  __device__ inline void operator()(AccTile& acc, int m0, int n0, char*, char*) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3, quad = lane >> 4, col = lane & 15;
    const bool scaled = last && div != 1.f;
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int n = n0 + acc_col(wn, j, col);
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < ACC_I; ++i)
#pragma unroll
        for (int r = 0; r < ACC_R; ++r) {
          const int m = m0 + acc_row(wm, i, r, quad);
          if (m < M) {
            const int64_t o = (int64_t)m * ld + n;
            float v = first ? acc[i][j][r] : sum[o] + acc[i][j][r];
            if (scaled) v = v / div;
            if (last)
              out[o] = (OutT)v;
            else
              sum[o] = v;
          }
        }
    }
  }
};

// ---------------------------------------------------------------------------
// Transposed forms, for products computed as C^T: C[m, n] goes to
// out[n * ld + m].  The lane's 4 consecutive m of one n are contiguous there,
// so every store is 16 bytes (8 for bf16).  M is a multiple of 4.
// ---------------------------------------------------------------------------
// Hidden-gradient accumulation (dH^T = W^T dz^T): sum[n, m] = (first ? 0 :
// sum[n, m]) + acc; on the last slice the result goes to `out` (OutT).  With
// first = last = 1 and OutT = float it is a plain transposed fp32 store (the
// split-K partials of the fused step).
template <class OutT>
struct EpiAccumT {
  float* sum;  // [N][ld] fp32 running sum (may alias out when OutT is float)
  int64_t ld;
  OutT* out;   // [N][ld]
  int M, N;
  int first, last;
  float div = 1.f;  // the last slice writes (sum + acc) / div
  // columns n are permuted token positions: the result of column n goes to
  // out row rowmap[n] (the running sum keeps position n), and only columns
  // below *n_dev exist (null: identity, N)
  const int* rowmap = nullptr;
  const int* n_dev = nullptr;
  static constexpr int LDS_BYTES = 0;

  __device__ inline void operator()(AccTile& acc, int m0, int n0, char*, char*) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3, quad = lane >> 4, col = lane & 15;
    const bool scaled = last && div != 1.f;
    const int Nn = n_dev ? min(N, *n_dev) : N;
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) {
      const int n = n0 + acc_col(wn, j, col);
      if (n >= Nn) continue;
      const int64_t orow = rowmap ? rowmap[n] : n;
#pragma unroll
      for (int i = 0; i < ACC_I; ++i) {
        const int m = m0 + acc_row(wm, i, 0, quad);
        if (m >= M) continue;
        const int64_t o = (int64_t)n * ld + m, oo = orow * ld + m;
        f32x4 v = acc[i][j];
        if (!first) {
          const f32x4 s0 = *(const f32x4*)(sum + o);
          v[0] += s0[0];
          v[1] += s0[1];
          v[2] += s0[2];
          v[3] += s0[3];
        }
        if (scaled) {
          v[0] = v[0] / div;
          v[1] = v[1] / div;
          v[2] = v[2] / div;
          v[3] = v[3] / div;
        }
        if (last) {
          if constexpr (sizeof(OutT) == 2) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const uint32_t p0 = (uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[0]) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[1]) << 16);
            const uint32_t p1 = (uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[2]) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[3]) << 16);
            *(u32x2*)(out + oo) = u32x2{p0, p1};
          } else {
            *(f32x4*)(out + oo) = v;
          }
        } else {
          *(f32x4*)(sum + o) = v;
        }
      }
    }
  }
};

}  // namespace stce
