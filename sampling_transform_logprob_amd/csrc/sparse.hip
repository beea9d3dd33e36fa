// The backward's row classes and its products over sparse dz.
//
// dz = c (1[j == y] - q) / T is nonzero only on a row's support, so for a
// row bounded by top-k (or a small min-p / top-p support) the two gradient
// products dH = dz W and dW = dz^T h are sums over a handful of vocabulary
// rows.  Rows whose support holds at most NSP tokens take these sums
// directly; the others go through the matrix-core products (kernels.hip).
//
//   1. classification: every row is dense, sparse, tiled (sparse, with a
//      list of the vocabulary tiles that can hold its support) or empty (no
//      gradient); the rows are placed in that class order, each class in row
//      order (a block count, one scan, a placement pass), and the hidden
//      states are gathered into that order;
//   2. the recompute product (EpiGrad) writes the dense rows' dz and appends
//      each sparse row's nonzero dz to its entry list, counting the entries
//      of every vocabulary row; the tiled rows' keys are recomputed on their
//      listed tiles only (a product over (tile, rows) work items: per tile
//      the positions listing it, filed by a count, a scan and a fill pass),
//      with the same epilogue;
//   3. weight gradient: an exclusive scan of the per-vocabulary-row counts,
//      a pass that files each entry into its vocabulary row's bucket, and one
//      workgroup per vocabulary row that sums its bucket's dz h[t] terms in
//      increasing token position (a fixed order), onto the dense product's
//      result or the caller's dW when there is one, else onto zero;
//   4. hidden gradient: one workgroup per sparse row that sums its entries'
//      dz W[j] terms in increasing vocabulary order; empty rows get zeros.
//
// Every order of summation is fixed (entries are ordered by their index
// before they are summed), so the results are deterministic although the
// entry lists are filled with atomics.
#include "epilogues.hpp"
#include "kernels.hpp"

namespace stce {
namespace {

constexpr int CB = 1024;  // rows per classification block (256 threads x 4)

// ntile: the row's tile-list length (0: none, or tile recompute off);
// lists 0: the row's support list is not used
__device__ inline int grad_class(const RowState& rs, float g, int ntile, int lists) {
  if ((rs.flags & (ROW_VALID | ROW_IN_SUPPORT)) != (ROW_VALID | ROW_IN_SUPPORT) || g == 0.f) return GRAD_EMPTY;
  if (!(rs.flags & ROW_FILTERED) || rs.n > NSP) return GRAD_DENSE;
  if (lists && (rs.flags & ROW_LISTED)) return GRAD_LISTED;
  return ntile > 0 ? GRAD_TILED : GRAD_SPARSE;
}

// Inclusive scan over the 256 threads of a workgroup (4 waves): wave scans
// by shuffles, then the wave totals through LDS.  All threads must call it.
__device__ inline int block_incl_scan(int v, int* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  __syncthreads();
  if (lane == 63) scratch[w] = v;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += scratch[i];
  return v + off;
}

// Per block of CB rows: how many rows of each class.
__global__ __launch_bounds__(256) void class_count_kernel(const RowState* st, const RowTiles* tl, const float* g,
                                                          int64_t T, int lists, int* blk) {
  __shared__ int scr[4];
  const int64_t r0 = (int64_t)blockIdx.x * CB + threadIdx.x * 4;
  int c[GRAD_CLASSES] = {};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (r0 + i < T) ++c[grad_class(st[r0 + i], g[r0 + i], tl ? tl[r0 + i].n : 0, lists)];
#pragma unroll
  for (int k = 0; k < GRAD_CLASSES; ++k) {
    const int s = block_incl_scan(c[k], scr);
    if (threadIdx.x == 255) blk[blockIdx.x * GRAD_CLASSES + k] = s;
  }
}

// One workgroup: exclusive scan of the block counts (in place, per class)
// and the class totals.
__global__ __launch_bounds__(1024) void class_scan_kernel(int* blk, int nblk, GradCounts* cnt) {
  constexpr int NC = GRAD_CLASSES;
  __shared__ int part[1024 * NC];
  __shared__ int tot[NC];
  const int t = threadIdx.x;
  // thread t scans blocks [t * per, (t + 1) * per)
  const int per = (nblk + 1023) / 1024;
  int s[NC] = {};
  for (int b = t * per; b < min(nblk, (t + 1) * per); ++b)
#pragma unroll
    for (int k = 0; k < NC; ++k) s[k] += blk[b * NC + k];
#pragma unroll
  for (int k = 0; k < NC; ++k) part[t * NC + k] = s[k];
  __syncthreads();
  if (t < NC) {
    int run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int x = part[i * NC + t];
      part[i * NC + t] = run;
      run += x;
    }
    tot[t] = run;
  }
  __syncthreads();
  int run[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) run[k] = part[t * NC + k];
  for (int b = t * per; b < min(nblk, (t + 1) * per); ++b)
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int x = blk[b * NC + k];
      blk[b * NC + k] = run[k];
      run[k] += x;
    }
  if (t == 0) {
    GradCounts c;
    c.dense = tot[GRAD_DENSE];
    c.full = c.dense + tot[GRAD_SPARSE];
    c.listed = c.full + tot[GRAD_LISTED];
    c.active = c.listed + tot[GRAD_TILED];
    *cnt = c;
  }
}

// Places every row at its permuted position (dense, sparse, listed, tiled,
// then empty; row order within a class) and clears the position's entry
// counter.
__global__ __launch_bounds__(256) void class_place_kernel(const RowState* st, const RowTiles* tl, const float* g,
                                                          int64_t T, int lists, const int* blk, const GradCounts* cnt,
                                                          int* perm, int* rowcnt) {
  __shared__ int scr[4];
  const int64_t r0 = (int64_t)blockIdx.x * CB + threadIdx.x * 4;
  int cls[4];
  int c[GRAD_CLASSES] = {};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cls[i] = r0 + i < T ? grad_class(st[r0 + i], g[r0 + i], tl ? tl[r0 + i].n : 0, lists) : -1;
    if (cls[i] >= 0) ++c[cls[i]];
  }
  const GradCounts n = *cnt;
  const int cls_base[GRAD_CLASSES] = {0, n.dense, n.full, n.listed, n.active};
  int pos[GRAD_CLASSES];
#pragma unroll
  for (int k = 0; k < GRAD_CLASSES; ++k)
    pos[k] = cls_base[k] + blk[blockIdx.x * GRAD_CLASSES + k] + block_incl_scan(c[k], scr) - c[k];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (cls[i] >= 0) {
      const int p = pos[cls[i]]++;
      perm[p] = (int)(r0 + i);
      rowcnt[p] = 0;
    }
}

// The listed rows' dz entries from the support the forward stored with its
// keys (no key is recomputed): position n in [full, listed), row t =
// perm[n], one entry per support token j with the recompute epilogue's
// arithmetic, bf16(c (1[j == y] - exp2(s_j log2 e - lse_S log2 e))),
// c = g / T; the per-vocabulary-row counts into cntj when it is not null.
// (A list entry naming no token of [0, V) is skipped, so that no state can
// index past the vocabulary.)  One wave per position, a lane per support
// token (n <= NSP).
__global__ __launch_bounds__(256) void listed_entries_kernel(const int* perm, const GradCounts* cnt,
                                                             const RowState* st, const RowSupport* sup,
                                                             const float* g, const float* temp,
                                                             const int64_t* target, int V, int* rowcnt,
                                                             SpEntry* list, int* cntj, int64_t T) {
  const int lane = threadIdx.x & 63;
  const GradCounts c = *cnt;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t n = c.full + (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       n < c.listed && n < T; n += nw) {
    const int64_t t = perm[n];
    const RowState rs = st[t];
    const int ns = min(rs.n, NSP);
    const float cf = g[t] / (temp ? temp[t] : 1.0f), nl = -rs.lse_s * LOG2E;
    const int y = (int)target[t];
    int k = 0;
    for (int i0 = 0; i0 < ns; i0 += 64) {  // (uniform: every lane runs each pass)
      const int i = i0 + lane;
      const SpEntry e = i < ns ? sup[t].e[i] : SpEntry{-1, 0.0f};
      const bool in = (uint32_t)e.idx < (uint32_t)V;
      const uint64_t b = __ballot(in);
      const int slot = k + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
      if (in) {
        const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(e.v, LOG2E, nl));
        const float dv = cf * ((e.idx == y ? 1.f : 0.f) - q);
        list[n * NSP + slot] = SpEntry{e.idx, (float)(bf16)dv};
        if (cntj) atomicAdd(cntj + e.idx, 1);
      }
      k += __builtin_popcountll(b);
    }
    if (lane == 0) rowcnt[n] = k;
  }
}

// out[n] = in[perm[n]], rows of H elements (H a multiple of 8, 16-byte rows).
template <class E>
__global__ __launch_bounds__(256) void gather_rows_kernel(const E* in, const int* perm, int64_t T, int64_t H,
                                                          E* out) {
  constexpr int EPV = 16 / (int)sizeof(E);
  const int64_t per_row = H / EPV;
  const int64_t total = T * per_row;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int64_t n = i / per_row, c = i - n * per_row;
    ((u32x4*)(out + n * H))[c] = ((const u32x4*)(in + (int64_t)perm[n] * H))[c];
  }
}

__global__ void fill_i32_kernel(int* p, int64_t n, int v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// Exclusive scan of x[0, n) into y[0, n] (y[n] = total) in three launches:
// per-block sums (SB elements a block), one workgroup scanning them, and a
// pass that scans each block from its base.
constexpr int SB = 4096;

__global__ __launch_bounds__(256) void scan_sums_kernel(const int* x, int64_t n, int* sums) {
  __shared__ int scr[4];
  const int64_t b0 = (int64_t)blockIdx.x * SB + threadIdx.x * 16;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (b0 + i < n) s += x[b0 + i];
  s = block_incl_scan(s, scr);
  if (threadIdx.x == 255) sums[blockIdx.x] = s;
}

__global__ __launch_bounds__(1024) void scan_top_kernel(int* sums, int nb, int* total) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (nb + 1023) / 1024;
  int s = 0;
  for (int b = t * per; b < min(nb, (t + 1) * per); ++b) s += sums[b];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
    *total = run;
  }
  __syncthreads();
  int run = part[t];
  for (int b = t * per; b < min(nb, (t + 1) * per); ++b) {
    const int v = sums[b];
    sums[b] = run;
    run += v;
  }
}

__global__ __launch_bounds__(256) void scan_apply_kernel(const int* x, int64_t n, const int* sums, int* y) {
  __shared__ int scr[4];
  const int64_t b0 = (int64_t)blockIdx.x * SB + threadIdx.x * 16;
  int v[16];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = b0 + i < n ? x[b0 + i] : 0;
    s += v[i];
  }
  int run = sums[blockIdx.x] + block_incl_scan(s, scr) - s;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (b0 + i < n) {
      y[b0 + i] = run;
      run += v[i];
    }
}

// Files the entries of the sparse positions into their vocabulary rows'
// buckets: bucket[off[j] + slot] = (position, dz), the slot taken by counting
// cntj[j] back down to zero (the order inside a bucket is arbitrary here and
// fixed by the summing kernel).  One wave per position.
__global__ __launch_bounds__(256) void bucket_fill_kernel(const GradCounts* cnt, int64_t T, const int* rowcnt,
                                                          const SpEntry* list, const int* off, int* cntj,
                                                          SpEntry* bucket) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const GradCounts c = *cnt;
  if (n < c.dense || n >= c.active || n >= T) return;
  const int ne = min(rowcnt[n], NSP);
  for (int i = lane; i < ne; i += 64) {
    const SpEntry e = list[n * NSP + i];
    const int slot = atomicSub(cntj + e.idx, 1) - 1;
    bucket[off[e.idx] + slot] = SpEntry{(int32_t)n, e.v};
  }
}

// Orders the ne entries of src (distinct indices) by increasing index into
// dst, both in LDS: entry i goes to the number of entries with a smaller
// index.  256 threads; the caller synchronizes before and after.
__device__ inline void rank_order(const SpEntry* src, int ne, SpEntry* dst) {
  for (int i = threadIdx.x; i < ne; i += 256) {
    const SpEntry e = src[i];
    int r = 0;
    for (int k = 0; k < ne; ++k) r += src[k].idx < e.idx ? 1 : 0;
    dst[r] = e;
  }
}

template <class E>
__device__ inline void load8(const E* p, float (&x)[8]) {
  if constexpr (sizeof(E) == 2) {
    const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)v[k];
  } else {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a[k];
      x[4 + k] = b[k];
    }
  }
}

// fp8 lane: x[k] = fl32(sc * e4m3(p[k])), the dequantized weight element.
__device__ inline void load8(const uint8_t* p, float sc, float (&x)[8]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = *(const u32x2*)p;
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = __fmul_rn(sc, e4m3_decode((w[k >> 2] >> (8 * (k & 3))) & 0xffu));
}

template <class E>
__device__ inline void load8_row(const E* X, const float* xs, int64_t row, int64_t H, int64_t c0, float (&x)[8]) {
  if constexpr (sizeof(E) == 1)
    load8(X + row * H + c0, xs[row], x);
  else
    load8(X + row * H + c0, x);
}

// acc[k] += e.v * X[e.idx, c0 + k] over the ordered entries e = ord[0 .. ne),
// in that order, fp32 fmas; the rows of eight entries are loaded before their
// fmas so that the loads overlap (the order of the sums is unchanged).
// X of e4m3 codes takes the per-row scales xs.
template <class E>
__device__ inline void ordered_sum(const SpEntry* ord, int ne, const E* X, int64_t H, int64_t c0, float (&acc)[8],
                                   const float* xs = nullptr) {
  int r = 0;
  for (; r + 8 <= ne; r += 8) {
    float x[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8_row(X, xs, (int64_t)ord[r + u].idx, H, c0, x[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float v = ord[r + u].v;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(v, x[u][k], acc[k]);
    }
  }
  for (; r < ne; ++r) {
    float x[8];
    load8_row(X, xs, (int64_t)ord[r].idx, H, c0, x);
    const float v = ord[r].v;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(v, x[k], acc[k]);
  }
}

constexpr int ORDER_CAP = 1024;   // entries a weight-gradient bucket orders in LDS
constexpr int WAVE_MAX = 64;      // entries a row summed by one wave orders in its lanes

// One wave's up to WAVE_MAX entries (lane l < ne holds entry l; distinct
// indices), placed in increasing index order: lane s gets the entry of rank
// s (its rank by comparison with every other, then a lane permute).
__device__ inline void wave_order(int ne, int& idx, float& v) {
  const int lane = threadIdx.x & 63;
  int r = lane;
  if (lane < ne) {
    r = 0;
    for (int k = 0; k < ne; ++k) r += __builtin_amdgcn_readlane(idx, k) < idx ? 1 : 0;
  }
  idx = __builtin_amdgcn_ds_permute(r * 4, idx);
  v = __int_as_float(__builtin_amdgcn_ds_permute(r * 4, __float_as_int(v)));
}

// acc[k] += v_s * X[idx_s, c0 + k] for the ordered entries s = 0 .. ne of a
// wave (lane s holds entry s), in that order: ordered_sum's arithmetic.  The
// entries are read with readlane (a uniform lane index, whatever the exec
// mask: the last column pass may leave lanes idle).
template <class E>
__device__ inline void wave_ordered_sum(int ne, int idx, float v, const E* X, const float* xs, int64_t H, int64_t c0,
                                        float (&acc)[8]) {
  int s = 0;
  for (; s + 4 <= ne; s += 4) {
    float x[4][8], vs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = __builtin_amdgcn_readlane(idx, s + u);
      vs[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s + u));
      load8_row(X, xs, (int64_t)row, H, c0, x[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(vs[u], x[u][k], acc[k]);
  }
  for (; s < ne; ++s) {
    float x[8];
    const int row = __builtin_amdgcn_readlane(idx, s);
    const float vv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s));
    load8_row(X, xs, (int64_t)row, H, c0, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(vv, x[k], acc[k]);
  }
}
// Four consecutive elements of a hidden row as fp32 (8-byte bf16 or 16-byte
// fp32 loads).
template <class E>
__device__ inline void load4(const E* p, float (&x)[4]) {
  if constexpr (sizeof(E) == 2) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = *(const bf16x4*)p;
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (float)v[k];
  } else {
    const f32x4 a = *(const f32x4*)p;
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = a[k];
  }
}

// wave_ordered_sum's arithmetic on the columns ca .. ca + 4 (acc[0..4)) and
// cb .. cb + 4 (acc[4..8)) of each entry's row: the same sums, each element
// over the entries in order.
template <class E>
__device__ inline void wave_ordered_sum_split(int ne, int idx, float v, const E* X, int64_t H, int64_t ca,
                                              int64_t cb, float (&acc)[8]) {
  int s = 0;
  for (; s + 4 <= ne; s += 4) {
    float x[4][8], vs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t row = __builtin_amdgcn_readlane(idx, s + u);
      vs[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s + u));
      float a[4], b[4];
      load4(X + row * H + ca, a);
      load4(X + row * H + cb, b);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[u][k] = a[k];
        x[u][4 + k] = b[k];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(vs[u], x[u][k], acc[k]);
  }
  for (; s < ne; ++s) {
    const int64_t row = __builtin_amdgcn_readlane(idx, s);
    const float vv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s));
    float a[4], b[4];
    load4(X + row * H + ca, a);
    load4(X + row * H + cb, b);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[k] = __builtin_fmaf(vv, a[k], acc[k]);
      acc[4 + k] = __builtin_fmaf(vv, b[k], acc[4 + k]);
    }
  }
}
constexpr int WIN = 4096;         // token positions per window beyond that

// Weight gradient rows from the buckets: one workgroup per vocabulary row j,
//   dW[j, :] = base + sum over the bucket's entries, in increasing token
//              position n, of dz * h_perm[n, :]  (fp32),
// base = dW[j, :] when the dense product wrote it or the caller accumulates,
// else 0.  Rows with an empty bucket are left alone, or zeroed when nothing
// else writes them.  Buckets larger than ORDER_CAP entries are summed window
// by window of WIN positions, each entry placed at its position in LDS.
template <class E>
__device__ inline void sparse_dw_row(int64_t j, const int* off, const SpEntry* bucket, const E* h, int64_t H,
                                     bool from_mem, float* dW, int64_t T, SpEntry* ord, SpEntry* raw, float* win) {
  const int o0 = off[j], ne = off[j + 1] - o0;
  float* row = dW + j * H;
  if (ne == 0) {
    if (!from_mem)
      for (int64_t c = threadIdx.x * 4; c < H; c += 256 * 4) *(f32x4*)(row + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  if (ne <= ORDER_CAP) {
    for (int i = threadIdx.x; i < ne; i += 256) raw[i] = bucket[o0 + i];
    __syncthreads();
    rank_order(raw, ne, ord);
    __syncthreads();
    for (int64_t c0 = threadIdx.x * 8; c0 < H; c0 += 256 * 8) {
      float acc[8];
      if (from_mem) {
        const f32x4 a = *(const f32x4*)(row + c0), b = *(const f32x4*)(row + c0 + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[k] = a[k];
          acc[4 + k] = b[k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.f;
      }
      ordered_sum(ord, ne, h, H, c0, acc);
      *(f32x4*)(row + c0) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)(row + c0 + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
    return;
  }
  // a large bucket (a token in many rows' supports): windows of positions
  for (int64_t c0 = threadIdx.x * 8; c0 - threadIdx.x * 8 < H; c0 += 256 * 8) {
    const bool mine = c0 < H;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    if (mine && from_mem) {
      const f32x4 a = *(const f32x4*)(row + c0), b = *(const f32x4*)(row + c0 + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[k] = a[k];
        acc[4 + k] = b[k];
      }
    }
    for (int64_t w0 = 0; w0 < T; w0 += WIN) {
      __syncthreads();
      for (int i = threadIdx.x; i < WIN; i += 256) win[i] = 0.f;
      __syncthreads();
      for (int i = threadIdx.x; i < ne; i += 256) {
        const SpEntry e = bucket[o0 + i];
        if (e.idx >= w0 && e.idx < w0 + WIN) win[e.idx - w0] = e.v;
      }
      __syncthreads();
      if (mine) {
        const int lim = (int)min((int64_t)WIN, T - w0);
        for (int r = 0; r < lim; ++r) {
          const float v = win[r];
          if (v == 0.f) continue;  // no entry (a zero entry adds nothing)
          float x[8];
          load8(h + (w0 + r) * H + c0, x);
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(v, x[k], acc[k]);
        }
      }
    }
    if (mine) {
      *(f32x4*)(row + c0) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)(row + c0 + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

// Weight-gradient rows j = blockIdx.x, + gridDim.x, ... (sparse_dw_row) whose
// bucket holds more than WAVE_MAX entries.
template <class E>
__global__ __launch_bounds__(256) void sparse_dw_kernel(const int* off, const SpEntry* bucket, const E* h, int64_t H,
                                                        const GradCounts* cnt, int accumulate, float* dW, int64_t T,
                                                        int64_t V) {
  // the ordering buffers and the window are never used by the same row: one
  // 16 KB region (more workgroups per compute unit to hide the row loads)
  __shared__ union {
    struct {
      SpEntry ord[ORDER_CAP];
      SpEntry raw[ORDER_CAP];
    } o;
    float win[WIN];
  } L;
  const bool from_mem = accumulate || cnt->dense > 0;
  for (int64_t j = blockIdx.x; j < V; j += gridDim.x) {
    if (off[j + 1] - off[j] <= WAVE_MAX) continue;  // (sparse_dw_wave_kernel's rows; uniform)
    sparse_dw_row(j, off, bucket, h, H, from_mem, dW, T, L.o.ord, L.o.raw, L.win);
    __syncthreads();  // the row's LDS before the next row's
  }
}

// Hidden gradient rows of the sparse and empty positions: one workgroup per
// permuted position n >= dense (row t = perm[n]):
//   dH[t, :] = (sum over the entries, in increasing vocabulary row j, of
//              dz * W[j, :]) / div   in the hidden dtype; zeros for empty rows.
// An e4m3 weight (E = uint8_t) is read dequantized, fl32(w_scale[j] code),
// and the hidden gradient is bf16.
template <class E, class O>
__global__ __launch_bounds__(256) void sparse_dh_kernel(const int* perm, const GradCounts* cnt, const int* rowcnt,
                                                        const SpEntry* list, const E* W, const float* w_scale,
                                                        int64_t H, float div, O* dH, int64_t T) {
  __shared__ SpEntry raw[NSP];
  __shared__ SpEntry ord[NSP];
  const int64_t n = blockIdx.x;
  const GradCounts c = *cnt;
  if (n < c.dense || n >= T) return;
  const int ne = n < c.active ? min(rowcnt[n], NSP) : 0;
  if (ne <= WAVE_MAX) return;  // (sparse_dh_wave_kernel's rows)
  const int64_t t = perm[n];
  O* out = dH + t * H;
  for (int i = threadIdx.x; i < ne; i += 256) raw[i] = list[n * NSP + i];
  __syncthreads();
  rank_order(raw, ne, ord);
  __syncthreads();
  for (int64_t c0 = threadIdx.x * 8; c0 < H; c0 += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    ordered_sum(ord, ne, W, H, c0, acc, w_scale);
    if (div != 1.f)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = acc[k] / div;
    if constexpr (sizeof(O) == 2) {
      bf16x8 o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = (bf16)acc[k];
      *(bf16x8*)(out + c0) = o;
    } else {
      *(f32x4*)(out + c0) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)(out + c0 + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

// The rows with at most WAVE_MAX entries, one wave per row (the common case:
// a top-k row's support, a vocabulary row reached by a few supports), with
// no workgroup barrier, so that many rows' load chains are in flight at once.
// Same order of summation, hence the same results, as the workgroup kernels.
template <class E>
__global__ __launch_bounds__(256) void sparse_dw_wave_kernel(const int* off, const SpEntry* bucket, const E* h,
                                                             int64_t H, const GradCounts* cnt, int accumulate,
                                                             float* dW, int64_t V) {
  const int lane = threadIdx.x & 63;
  const bool from_mem = accumulate || cnt->dense > 0;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); j < V; j += nw) {
    const int o0 = off[j], ne = off[j + 1] - o0;
    if (ne > WAVE_MAX || (ne == 0 && from_mem)) continue;
    int idx = 0;
    float v = 0.f;
    if (lane < ne) {
      const SpEntry e = bucket[o0 + lane];
      idx = e.idx;
      v = e.v;
    }
    wave_order(ne, idx, v);
    float* row = dW + j * H;
    // a pass covers 512 columns: lane l the groups of four at 4 l and
    // 256 + 4 l, so that each fp32 store instruction writes 1 KB of the row
    // contiguously (whole cache lines) and each row load reads 512 B
    for (int64_t c0 = 0; c0 < H; c0 += 512) {
      const int64_t ca = c0 + 4 * lane, cb = ca + 256;
      const bool ia = ca < H, ib = cb < H;  // (H is a multiple of 8)
      float acc[8];
      if (from_mem) {
        const f32x4 a = ia ? *(const f32x4*)(row + ca) : f32x4{}, b = ib ? *(const f32x4*)(row + cb) : f32x4{};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[k] = a[k];
          acc[4 + k] = b[k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.f;
      }
      wave_ordered_sum_split(ne, idx, v, h, H, ia ? ca : 0, ib ? cb : 0, acc);
      // (nontemporal: nothing here reads dW again, and the stream of it
      // should not displace the hidden rows the gathers hit in the cache)
      if (ia) __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)(row + ca));
      if (ib) __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, (f32x4*)(row + cb));
    }
  }
}

template <class E, class O>
__global__ __launch_bounds__(256) void sparse_dh_wave_kernel(const int* perm, const GradCounts* cnt, const int* rowcnt,
                                                             const SpEntry* list, const E* W, const float* w_scale,
                                                             int64_t H, float div, O* dH, int64_t T) {
  const int lane = threadIdx.x & 63;
  const GradCounts c = *cnt;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t n = c.dense + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); n < T; n += nw) {
    const int ne = n < c.active ? min(rowcnt[n], NSP) : 0;
    if (ne > WAVE_MAX) continue;
    int idx = 0;
    float v = 0.f;
    if (lane < ne) {
      const SpEntry e = list[n * NSP + lane];
      idx = e.idx;
      v = e.v;
    }
    wave_order(ne, idx, v);
    O* out = dH + (int64_t)perm[n] * H;
    for (int64_t c0 = lane * 8; c0 < H; c0 += 64 * 8) {
      float acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = 0.f;
      wave_ordered_sum(ne, idx, v, W, w_scale, H, c0, acc);
      if (div != 1.f)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = acc[k] / div;
      if constexpr (sizeof(O) == 2) {
        bf16x8 o;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = (bf16)acc[k];
        __builtin_nontemporal_store(o, (bf16x8*)(out + c0));  // (written once, read by the caller)
      } else {
        __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)(out + c0));
        __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, (f32x4*)(out + c0 + 4));
      }
    }
  }
}

// Tile recompute work lists.  tile_count: per vocabulary tile, how many tiled
// positions list it; tile_fill: each listing position appended to its tile's
// bucket (order within a bucket is free: a key does not depend on its
// column); tile_work: product work items per tile (GN positions each).
// (a list is at most NTILE long and names tiles below ntv when the forward
// wrote it; both are enforced so that no other state can index past them).
// With at most TH_LDS tiles a workgroup counts its rows' tiles in LDS and
// adds each nonzero count to the global one once (the lists of thousands of
// rows name the same few hundred tiles), and the fill reserves each tile's
// range of slots once per workgroup the same way.
constexpr int TH_LDS = 8192;
constexpr int TROWS = 1024;  // positions per workgroup of the count and the fill

__global__ __launch_bounds__(256) void tile_count_kernel(const int* perm, const GradCounts* cnt, const RowTiles* tl,
                                                         int64_t T, int64_t ntv, int* tcnt) {
  __shared__ int hist[TH_LDS];
  const GradCounts c = *cnt;
  const bool lds = ntv <= TH_LDS;
  if (lds)
    for (int j = threadIdx.x; j < ntv; j += 256) hist[j] = 0;
  __syncthreads();
  const int64_t n0 = c.listed + (int64_t)blockIdx.x * TROWS;
  for (int64_t n = n0 + threadIdx.x; n < n0 + TROWS && n < c.active && n < T; n += 256) {
    const RowTiles& r = tl[perm[n]];
    const int nt = min((int)r.n, NTILE);
    for (int i = 0; i < nt; ++i) {
      const int j = r.t[i];
      if (j < ntv) atomicAdd(lds ? hist + j : tcnt + j, 1);
    }
  }
  __syncthreads();
  if (lds)
    for (int j = threadIdx.x; j < ntv; j += 256)
      if (hist[j]) atomicAdd(tcnt + j, hist[j]);
}

__global__ __launch_bounds__(256) void tile_fill_kernel(const int* perm, const GradCounts* cnt, const RowTiles* tl,
                                                        int64_t T, int64_t ntv, const int* toff, int* tfill,
                                                        int* bucket) {
  __shared__ int hist[TH_LDS];
  const GradCounts c = *cnt;
  const bool lds = ntv <= TH_LDS;
  const int64_t n0 = c.listed + (int64_t)blockIdx.x * TROWS;
  if (lds) {
    for (int j = threadIdx.x; j < ntv; j += 256) hist[j] = 0;
    __syncthreads();
    for (int64_t n = n0 + threadIdx.x; n < n0 + TROWS && n < c.active && n < T; n += 256) {
      const RowTiles& r = tl[perm[n]];
      const int nt = min((int)r.n, NTILE);
      for (int i = 0; i < nt; ++i)
        if (r.t[i] < ntv) atomicAdd(hist + r.t[i], 1);
    }
    __syncthreads();
    // this workgroup's range of each tile's bucket
    for (int j = threadIdx.x; j < ntv; j += 256)
      if (hist[j]) hist[j] = toff[j] + atomicAdd(tfill + j, hist[j]);
    __syncthreads();
  }
  for (int64_t n = n0 + threadIdx.x; n < n0 + TROWS && n < c.active && n < T; n += 256) {
    const RowTiles& r = tl[perm[n]];
    const int nt = min((int)r.n, NTILE);
    for (int i = 0; i < nt; ++i) {
      const int j = r.t[i];
      if (j < ntv) bucket[lds ? atomicAdd(hist + j, 1) : toff[j] + atomicAdd(tfill + j, 1)] = (int)n;
    }
  }
}

__global__ __launch_bounds__(256) void tile_work_kernel(const int* tcnt, int64_t ntv, int* twork) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < ntv) twork[j] = (tcnt[j] + TILE_COLS - 1) / TILE_COLS;
}

}  // namespace

hipError_t launch_tile_lists(const TileListArgs& a, hipStream_t s) {
  hipError_t e;
  if ((e = launch_fill_i32(a.tcnt, a.ntv, 0, s)) || (e = launch_fill_i32(a.tfill, a.ntv, 0, s))) return e;
  // one workgroup per TROWS positions of the whole row range (those past the
  // tiled ones return at once)
  const unsigned g = (unsigned)ceil_div(a.T, TROWS);
  hipLaunchKernelGGL(tile_count_kernel, dim3(g), dim3(256), 0, s, a.perm, a.cnt, a.tiles, a.T, a.ntv, a.tcnt);
  if ((e = launch_exclusive_scan(a.tcnt, a.ntv, a.sums, a.toff, s))) return e;
  hipLaunchKernelGGL(tile_work_kernel, dim3((unsigned)ceil_div(a.ntv, 256)), dim3(256), 0, s, a.tcnt, a.ntv,
                     a.twork);
  if ((e = launch_exclusive_scan(a.twork, a.ntv, a.sums, a.twoff, s))) return e;
  hipLaunchKernelGGL(tile_fill_kernel, dim3(g), dim3(256), 0, s, a.perm, a.cnt, a.tiles, a.T, a.ntv, a.toff,
                     a.tfill, a.bucket);
  return hipGetLastError();
}

hipError_t launch_grad_classes(const RowState* st, const RowTiles* tl, const float* g, int64_t T, int use_lists,
                               int* blk, GradCounts* cnt, int* perm, int* rowcnt, hipStream_t s) {
  ProfScope ps(KIND_CLASSIFY, s);
  const unsigned nb = (unsigned)ceil_div(T, CB);
  hipLaunchKernelGGL(class_count_kernel, dim3(nb), dim3(256), 0, s, st, tl, g, T, use_lists, blk);
  hipLaunchKernelGGL(class_scan_kernel, dim3(1), dim3(1024), 0, s, blk, (int)nb, cnt);
  hipLaunchKernelGGL(class_place_kernel, dim3(nb), dim3(256), 0, s, st, tl, g, T, use_lists, blk, cnt, perm,
                     rowcnt);
  return hipGetLastError();
}

size_t grad_class_blk_ints(int64_t T) { return GRAD_CLASSES * (size_t)ceil_div(T, CB); }

hipError_t launch_gather_rows(int dtype, const void* in, const int* perm, int64_t T, int64_t H, void* out,
                              hipStream_t s) {
  const int64_t total = T * H / (dtype == 1 ? 8 : 4);
  const unsigned blocks = (unsigned)(ceil_div(total, 256) < 8192 ? ceil_div(total, 256) : 8192);
  if (dtype == 1)
    hipLaunchKernelGGL(gather_rows_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)in, perm, T, H,
                       (bf16*)out);
  else
    hipLaunchKernelGGL(gather_rows_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)in, perm, T, H,
                       (float*)out);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int64_t n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(ceil_div(n, 256) < 4096 ? ceil_div(n, 256) : 4096);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

size_t scan_sums_ints(int64_t n) { return (size_t)ceil_div(n, SB) + 1; }

hipError_t launch_exclusive_scan(const int* x, int64_t n, int* sums, int* y, hipStream_t s) {
  const unsigned nb = (unsigned)ceil_div(n, SB);
  hipLaunchKernelGGL(scan_sums_kernel, dim3(nb), dim3(256), 0, s, x, n, sums);
  hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(1024), 0, s, sums, (int)nb, y + n);
  hipLaunchKernelGGL(scan_apply_kernel, dim3(nb), dim3(256), 0, s, x, n, sums, y);
  return hipGetLastError();
}

hipError_t launch_listed_entries(const int* perm, const GradCounts* cnt, const RowState* st, const RowSupport* sup,
                                 const float* g, const float* temp, const int64_t* target, int64_t V, int* rowcnt,
                                 SpEntry* list, int* cntj, int64_t T, hipStream_t s) {
  ProfScope ps(KIND_LISTED_ENTRIES, s);
  const unsigned blocks = (unsigned)(ceil_div(T, 4) < 8192 ? ceil_div(T, 4) : 8192);
  hipLaunchKernelGGL(listed_entries_kernel, dim3(blocks), dim3(256), 0, s, perm, cnt, st, sup, g, temp, target,
                     (int)V, rowcnt, list, cntj, T);
  return hipGetLastError();
}

hipError_t launch_sparse_grads(const SparseGradArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.grad_weight) {
    {
      ProfScope ps(KIND_SPARSE_DW, s);
      if ((e = launch_exclusive_scan(a.cntj, a.V, a.scan_sums, a.offj, s))) return e;
      hipLaunchKernelGGL(bucket_fill_kernel, dim3((unsigned)ceil_div(a.T, 4)), dim3(256), 0, s, a.cnt, a.T, a.rowcnt,
                         a.list, a.offj, a.cntj, a.bucket);
      // rows with few entries one wave each, then the rest one workgroup
      // each; both loop over the vocabulary rows, each taking its own
      const unsigned gw = (unsigned)(ceil_div(a.V, 4) < 8192 ? ceil_div(a.V, 4) : 8192);
      const unsigned g = (unsigned)(a.V < 4096 ? a.V : 4096);
      if (a.dtype != DT_F32) {  // bf16 rows (the fp8 lane's are the dequantized hidden rows)
        hipLaunchKernelGGL(sparse_dw_wave_kernel<bf16>, dim3(gw), dim3(256), 0, s, a.offj, a.bucket,
                           (const bf16*)a.h_perm, a.H, a.cnt, a.accumulate_w, a.grad_weight, a.V);
        hipLaunchKernelGGL(sparse_dw_kernel<bf16>, dim3(g), dim3(256), 0, s, a.offj, a.bucket, (const bf16*)a.h_perm,
                           a.H, a.cnt, a.accumulate_w, a.grad_weight, a.T, a.V);
      } else {
        hipLaunchKernelGGL(sparse_dw_wave_kernel<float>, dim3(gw), dim3(256), 0, s, a.offj, a.bucket,
                           (const float*)a.h_perm, a.H, a.cnt, a.accumulate_w, a.grad_weight, a.V);
        hipLaunchKernelGGL(sparse_dw_kernel<float>, dim3(g), dim3(256), 0, s, a.offj, a.bucket,
                           (const float*)a.h_perm, a.H, a.cnt, a.accumulate_w, a.grad_weight, a.T, a.V);
      }
    }
    if ((e = hipGetLastError())) return e;
  }
  if (a.grad_hidden) {
    ProfScope ps(KIND_SPARSE_DH, s);
    const unsigned gw = (unsigned)(ceil_div(a.T, 4) < 8192 ? ceil_div(a.T, 4) : 8192);
    if (a.dtype == DT_FP8)
      hipLaunchKernelGGL((sparse_dh_wave_kernel<uint8_t, bf16>), dim3(gw), dim3(256), 0, s, a.perm, a.cnt,
                         a.rowcnt, a.list, (const uint8_t*)a.W, a.w_scale, a.H, a.dh_div, (bf16*)a.grad_hidden, a.T);
    else if (a.dtype == DT_BF16)
      hipLaunchKernelGGL((sparse_dh_wave_kernel<bf16, bf16>), dim3(gw), dim3(256), 0, s, a.perm, a.cnt,
                         a.rowcnt, a.list, (const bf16*)a.W, nullptr, a.H, a.dh_div, (bf16*)a.grad_hidden, a.T);
    else
      hipLaunchKernelGGL((sparse_dh_wave_kernel<float, float>), dim3(gw), dim3(256), 0, s, a.perm, a.cnt,
                         a.rowcnt, a.list, (const float*)a.W, nullptr, a.H, a.dh_div, (float*)a.grad_hidden, a.T);
    if (a.dtype == DT_FP8)
      hipLaunchKernelGGL((sparse_dh_kernel<uint8_t, bf16>), dim3((unsigned)a.T), dim3(256), 0, s, a.perm, a.cnt,
                         a.rowcnt, a.list, (const uint8_t*)a.W, a.w_scale, a.H, a.dh_div, (bf16*)a.grad_hidden, a.T);
    else if (a.dtype == DT_BF16)
      hipLaunchKernelGGL((sparse_dh_kernel<bf16, bf16>), dim3((unsigned)a.T), dim3(256), 0, s, a.perm, a.cnt,
                         a.rowcnt, a.list, (const bf16*)a.W, nullptr, a.H, a.dh_div, (bf16*)a.grad_hidden, a.T);
    else
      hipLaunchKernelGGL((sparse_dh_kernel<float, float>), dim3((unsigned)a.T), dim3(256), 0, s, a.perm, a.cnt,
                         a.rowcnt, a.list, (const float*)a.W, nullptr, a.H, a.dh_div, (float*)a.grad_hidden, a.T);
    if ((e = hipGetLastError())) return e;
  }
  return hipSuccess;
}

}  // namespace stce
