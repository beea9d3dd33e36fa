// Small kernels (validation, transposes, tile partials) and the launchers of
// the block-tiled products with their epilogues.
#include "epilogues.hpp"
#include "kernels.hpp"

namespace stce {
namespace {

// ---------------------------------------------------------------------------
__global__ void validate_kernel(int64_t T, int64_t V, int ignore, int64_t ignore_index, const float* temp,
                                const int32_t* top_k, const float* top_p, const float* min_p,
                                const int64_t* target, uint32_t* flags, int64_t* status, int cand_ok) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float tt = temp ? temp[t] : 1.0f;
  const int32_t k = top_k ? top_k[t] : 0;
  const float p = top_p ? top_p[t] : 1.0f;
  const float mp = min_p ? min_p[t] : 0.0f;
  const int64_t y = target[t];
  const bool ign = ignore && y == ignore_index;
  int field = 0;
  if (!(__builtin_isfinite(tt) && tt > 0.0f)) field = 1;
  else if (k < 0) field = 2;
  else if (!(p > 0.0f && p <= 1.0f)) field = 3;
  else if (!(mp >= 0.0f && mp <= 1.0f)) field = 4;
  else if (!ign && (y < 0 || y >= V)) field = 5;
  const bool filtered = (k > 0 && (int64_t)k < V) || p < 1.0f || mp > 0.0f;
  const int64_t ntv = (V + VTILE - 1) / VTILE;
  const bool cand = cand_ok && k > 0 && (int64_t)k < V && k <= KCAND && k <= ntv && ntv <= 2 * CAP;
  flags[t] = field ? 0u
                   : (ROW_VALID | (filtered ? ROW_FILTERED : 0u) | (ign ? ROW_IGNORED : 0u) | (cand ? ROW_CAND : 0u));
  if (field && status) atomicMin((unsigned long long*)status, (unsigned long long)((t << 8) | field));
}

__global__ void fill_i64_kernel(int64_t* p, int64_t v) { *p = v; }

// One thread per row.  The loss sign: CISPO's token loss is
// -A sg(min(r, 1 + eh)) lp, the clipped surrogate's -min(r A, clip(r) A);
// grad is d loss / d lp with the CISPO weight held constant.
__global__ void policy_loss_kernel(int objective, float el, float eh, float scale, const float* adv,
                                   const float* old_lp, const RowState* st, int64_t T, const float* lp,
                                   float* loss, float* grad, float* ratio) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float x = lp[t];
  float l = 0.f, g = 0.f, r = 0.f;
  if (st && (st[t].flags & ROW_IGNORED)) {
    // inactive row: nothing
  } else if (x != x) {
    l = x;  // invalid row: NaN loss, no gradient
  } else if (x != -__builtin_huge_valf()) {
    const float a = adv[t];
    r = expf(x - old_lp[t]);
    if (objective == 1) {
      const float w = fminf(r, 1.0f + eh);
      l = -a * w * x;
      g = -a * w;
    } else {
      const float unclipped = r * a;
      const float clipped = fminf(fmaxf(r, 1.0f - el), 1.0f + eh) * a;
      if (unclipped <= clipped) {
        l = -unclipped;
        g = -a * r;
      } else {
        l = -clipped;
      }
    }
  }
  loss[t] = l * scale;
  grad[t] = g * scale;
  if (ratio) ratio[t] = r;
}

template <class T>
__global__ void transpose_kernel(const T* in, int64_t ld_in, int64_t R, int64_t Cc, T* out, int64_t ld_out,
                                 int64_t R_pad, const int* skip) {
  if (skip && *skip == 0) return;
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < Cc) ? in[r * ld_in + c] : (T)0.0f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < Cc && r < R_pad) out[c * ld_out + r] = tile[tx][i];
  }
}

// bf16 transpose with 16-byte accesses only: each wave moves one 64 x 64
// tile; lane (rb, cb) = (lane / 8, lane % 8) loads rows rb*8 .. +8 at columns
// cb*8 .. +8 (8 lanes cover 128 contiguous bytes of a row), transposes the
// 8 x 8 block in registers and stores output rows cb*8 + e at columns
// rb*8 .. +8 (again 128 contiguous bytes per 8 lanes).  Needs Cc, ld_in,
// ld_out and R_pad multiples of 8, 8, 8 and 64 and 16-byte aligned bases;
// rows R .. R_pad - 1 of the output columns are zero-filled.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* in, int64_t ld_in, int64_t R, int64_t Cc,
                                                             bf16* out, int64_t ld_out, const int* skip) {
  if (skip && *skip == 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = ((int64_t)blockIdx.y * 4 + w) * 64;
  if (c0 >= Cc) return;
  const int rb = lane >> 3, cb = lane & 7;
  const int64_t c = c0 + cb * 8;
  if (c >= Cc) return;  // whole 8-column block out of range (Cc % 8 == 0)
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = r0 + rb * 8 + j;
    v[j] = r < R ? *(const u32x4*)(in + r * ld_in + c) : u32x4{0u, 0u, 0u, 0u};
  }
  // element e of row j is the 16-bit half (e & 1) of word e >> 1 of v[j]
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = (v[2 * k][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
      const uint32_t hi = (v[2 * k + 1][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
      o[k] = lo | (hi << 16);
    }
    *(u32x4*)(out + (c + e) * ld_out + r0 + rb * 8) = o;
  }
}

// fp8 lane: one workgroup per hidden row t = perm[n] (n without perm): its
// absolute maximum, the row scale a[t] = fl32(amax / 448) (1 for a zero row),
// the e4m3 codes q[n, :] of clamp(fl32(h[t, :] / a[t]), +-448) and, with deq,
// the dequantized row deq[n, :] = bf16(fl32(a[t] e4m3(q[n, :]))); 8 elements
// per thread at a time.
__global__ __launch_bounds__(256) void fp8_quantize_rows_kernel(const bf16* h, int64_t H, const int* perm,
                                                                uint8_t* q, float* scale, bf16* deq) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __shared__ float red[4];
  const int64_t n = blockIdx.x;
  const int64_t t = perm ? perm[n] : n;
  const bf16* hr = h + t * H;
  float mx = 0.0f;
  for (int64_t c = threadIdx.x * 8; c < H; c += 256 * 8) {
    const bf16x8 v = *(const bf16x8*)(hr + c);
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmaxf(mx, __builtin_fabsf((float)v[k]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float a = mx > 0.0f ? mx / E4M3_MAX : 1.0f;
  if (threadIdx.x == 0) scale[t] = a;
  // fl32(h / a) by the correction step of quot_fast where it is exact (the
  // eight values and a inside its range; zeros, which would lose the sign
  // of -0, and tiny or huge values take the IEEE division)
  const float r = 1.0f / a;
  const bool a_ok = a >= 0x1p-30f && a <= 0x1p+30f;
  uint8_t* qr = q + n * H;
  for (int64_t c = threadIdx.x * 8; c < H; c += 256 * 8) {
    const bf16x8 v = *(const bf16x8*)(hr + c);
    float lo = STCE_INF, hi = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      lo = fminf(lo, __builtin_fabsf((float)v[k]));
      hi = fmaxf(hi, __builtin_fabsf((float)v[k]));
    }
    const bool fast = a_ok && lo >= 0x1p-90f && hi <= 0x1p+90f;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float hv = (float)v[k];
      const float x = fminf(fmaxf(fast ? quot_fast(hv, a, r) : hv / a, -E4M3_MAX), E4M3_MAX);
      w[k >> 2] |= e4m3_encode(x) << (8 * (k & 3));
    }
    *(u32x2*)(qr + c) = u32x2{w[0], w[1]};
    if (deq) {
      bf16x8 o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = (bf16)__fmul_rn(a, e4m3_decode((w[k >> 2] >> (8 * (k & 3))) & 0xffu));
      *(bf16x8*)(deq + n * H + c) = o;
    }
  }
}

// out[c][r] = bf16(fl32(scale[r] e4m3(in[r][c]))) through a 64 x 64 LDS tile;
// zeros for R <= r < R_pad.
__global__ void fp8_dequant_transpose_kernel(const uint8_t* in, const float* scale, int64_t ld_in, int64_t R,
                                             int64_t Cc, bf16* out, int64_t ld_out, int64_t R_pad, const int* skip) {
  if (skip && *skip == 0) return;
  __shared__ bf16 tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < Cc) ? (bf16)__fmul_rn(scale[r], e4m3_decode(in[r * ld_in + c])) : (bf16)0.0f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < Cc && r < R_pad) out[c * ld_out + r] = tile[tx][i];
  }
}

// out[r] = in[rowmap[r]] for r < *n_dev: rows of H elements, 16-byte rows;
// a grid-stride loop over nmax rows.
template <class E>
__global__ __launch_bounds__(256) void gather_rows_dev_kernel(const E* in, const int* rowmap, const int* n_dev,
                                                              int64_t nmax, int64_t H, E* out) {
  constexpr int EPV = 16 / (int)sizeof(E);
  const int64_t per_row = H / EPV;
  const int64_t n = min(nmax, (int64_t)*n_dev);
  const int64_t total = n * per_row;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / per_row, c = i - r * per_row;
    ((u32x4*)(out + r * H))[c] = ((const u32x4*)(in + (int64_t)rowmap[r] * H))[c];
  }
}

// out = in / t element by element: the fp32 quotient (IEEE division,
// correctly rounded) rounded to the operand type, nearest with ties to even.
// n8 groups of 8 elements, 16-byte aligned; a grid-stride loop.
template <class E>
__global__ __launch_bounds__(256) void prescale_kernel(const E* in, int64_t n8, float t, E* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    if constexpr (sizeof(E) == 2) {
      const bf16x8 v = ((const bf16x8*)in)[i];
      bf16x8 o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = (bf16)((float)v[k] / t);
      ((bf16x8*)out)[i] = o;
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 v = ((const f32x4*)in)[2 * i + h];
        v[0] = v[0] / t;
        v[1] = v[1] / t;
        v[2] = v[2] / t;
        v[3] = v[3] / t;
        ((f32x4*)out)[2 * i + h] = v;
      }
    }
  }
}

// One wave per (row, 256-wide tile).
__global__ void tile_partials_kernel(const float* s, int64_t ld, int64_t R, int64_t V, int ntv,
                                     const int64_t* target, TilePart* part, float* s_y) {
  const int64_t row = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.y * 4 + w;
  const float* rp = s + row * ld;
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    const int64_t y = target[row];
    s_y[row] = (y >= 0 && y < V) ? rp[y] : 0.0f;
  }
  if (t >= ntv) return;
  float v[4];
  float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t c = (int64_t)t * VTILE + lane + 64 * e;
    v[e] = c < V ? rp[c] : -__builtin_huge_valf();
    if (c < V) {
      mx = fmaxf(mx, v[e]);
      mn = fminf(mn, v[e]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    mn = fminf(mn, __shfl_xor(mn, o));
  }
  float sm = 0.f, en = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if ((int64_t)t * VTILE + lane + 64 * e < V) {
      const float x = __expf(v[e] - mx);
      sm += x;
      en = __builtin_fmaf(x, v[e] - mx, en);
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sm += __shfl_xor(sm, o);
    en += __shfl_xor(en, o);
  }
  if (lane == 0) {
    TilePart tp;
    tp.mx = mx;
    tp.sum = sm;
    tp.mn = mn;
    tp.ent = en;
    part[row * ntv + t] = tp;
  }
}

// dz of one chunk from its stored fp32 keys, with the arithmetic of the
// recompute epilogue (the same membership test against the boundary key's
// value, exp2 argument, coefficient and rounding), so every value is the one
// the recompute backward forms from the same keys.  Block: TT rows x 256
// columns; lane l of a wave takes columns 4l .. 4l+3 of 8 rows at a time,
// writes them token-major when d is not null (the fp32 path) and stages
// them in LDS, from where the vocab-major copy leaves as 16-byte row
// segments.  Rows rows .. rows_pad and columns V .. V_pad get zeros.
template <class OutT>
__global__ __launch_bounds__(256) void dz_keys_kernel(const float* keys, int64_t ld, const float* temp,
                                                      const int64_t* target, const RowState* st, const float* g,
                                                      int rows, int rows_pad, int V, int V_pad, OutT* d,
                                                      int64_t ld_d, OutT* dT, int64_t ld_dT) {
  constexpr int TT = sizeof(OutT) == 2 ? 64 : 32, TV = 256, SP = TT + 16 / (int)sizeof(OutT);
  __shared__ __attribute__((aligned(16))) OutT stage[TV * SP];
  __shared__ float r_c[TT], r_thr[TT], r_nl[TT];
  __shared__ int r_idt[TT], r_y[TT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: the row resources stay scalar
  const int t0 = blockIdx.y * TT, v0 = blockIdx.x * TV;
  if (tid < TT) {
    const int t = t0 + tid;
    float c = 0.f, thr = -__builtin_huge_valf(), nl = 0.f;
    int idt = 0, y = -1;
    if (t < rows) {
      const RowState rs = st[t];
      const float tt = temp ? temp[t] : 1.0f;
      if ((rs.flags & (ROW_VALID | ROW_IN_SUPPORT)) == (ROW_VALID | ROW_IN_SUPPORT)) c = g[t] / tt;
      thr = (rs.flags & ROW_FILTERED) ? key_value(rs.key_thr) : -__builtin_huge_valf();
      idt = rs.id_thr;
      nl = -rs.lse_s * LOG2E;
      y = (int)target[t];
    }
    r_c[tid] = c;
    r_thr[tid] = thr;
    r_nl[tid] = nl;
    r_idt[tid] = idt;
    r_y[tid] = y;
  }
  __syncthreads();
  const int v = v0 + 4 * lane;
  for (int grp = w; grp < TT / 8; grp += 4) {
    // the 8 rows' keys, all loaded before any store: one range-checked
    // resource per row spanning its ld keys (a dead row's range is empty, so
    // its loads return zeros; columns V .. ld are masked below)
    f32x4 xs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tl = grp * 8 + i;
      const int nrec = __builtin_amdgcn_readfirstlane(r_c[tl] != 0.f ? (int)(ld * 4) : 0);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(keys + (int64_t)(t0 + tl) * ld), (short)0, nrec, RSRC_WORD3);
      xs[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, v * 4, 0, 0));
    }
    OutT o[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tl = grp * 8 + i, t = t0 + tl;
      const float c = r_c[tl], thr = r_thr[tl], nl = r_nl[tl];
      const int idt = r_idt[tl], y = r_y[tl];
      const f32x4 x = xs[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int vg = v + e;
        const float sv = x[e];
        const bool in = (sv > thr) | ((sv == thr) & (vg <= idt));
        const float q = in ? __builtin_amdgcn_exp2f(__builtin_fmaf(sv, LOG2E, nl)) : 0.f;
        const float dv = c * ((vg == y ? 1.f : 0.f) - q);
        o[i][e] = (OutT)((c != 0.f && vg < V) ? dv : 0.f);
      }
      if (d && t < rows_pad && v < V_pad) {
        OutT* dp = d + (int64_t)t * ld_d + v;
        if constexpr (sizeof(OutT) == 2) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          const uint32_t p0 = (uint32_t)__builtin_bit_cast(uint16_t, o[i][0]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, o[i][1]) << 16);
          const uint32_t p1 = (uint32_t)__builtin_bit_cast(uint16_t, o[i][2]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, o[i][3]) << 16);
          *(u32x2*)dp = u32x2{p0, p1};
        } else {
          *(f32x4*)dp = f32x4{(float)o[i][0], (float)o[i][1], (float)o[i][2], (float)o[i][3]};
        }
      }
    }
    // staged as [column][row]: 8 consecutive rows of each of the 4 columns
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      OutT* sp = stage + (4 * lane + e) * SP + grp * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) sp[i] = o[i][e];
    }
  }
  __syncthreads();
  constexpr int EPC = 16 / (int)sizeof(OutT);  // elements per 16-byte chunk
  constexpr int CPR = TT / EPC;                // chunks per staged row
  for (int q = tid; q < TV * CPR; q += 256) {
    const int r = q / CPR, cc = (q % CPR) * EPC;
    const int vv = v0 + r, tt = t0 + cc;
    if (vv < V_pad && tt < rows_pad)
      *(u32x4*)(dT + (int64_t)vv * ld_dT + tt) = *(const u32x4*)(stage + r * SP + cc);
  }
}

// Split-K product: workgroup (b, split) computes tile b over the reduction
// range [split * ks, min(K, (split + 1) * ks)) and stores it (fp32, through
// the epilogue) into partial buffer `split`.
template <class Main, class Epi>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_splitk_kernel(Main mainloop, Epi epi, TileMap map, int tiles,
                                                                 int64_t ks, int64_t pstride) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int split = blockIdx.y;
  int tm, tn;
  map.get(blockIdx.x, tm, tn);
  Main mn = mainloop;
  mn.shift_k(split * ks);
  if (mn.K > ks) mn.K = (int)ks;
  Epi ep = epi;
  ep.out += split * pstride;
  AccTile acc;
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) acc[i][j] = f32x4{};
  hold_in_sgprs(ep);
  mn.run(acc, tm * GM, tn * GN, smem);
  ep(acc, tm * GM, tn * GN, Main::epilogue_lds(smem), Main::epilogue_lds1(smem));
}

// out[i] = (part[0][i] + part[1][i] + ...) / div, summed in split order, 4
// elements a thread.
template <class OutT>
__global__ void sum_splits_kernel(const float* part, int splits, int64_t pstride, int64_t n4, float div, OutT* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  f32x4 v = ((const f32x4*)part)[i];
  for (int s = 1; s < splits; ++s) {
    const f32x4 x = ((const f32x4*)(part + s * pstride))[i];
    v[0] += x[0];
    v[1] += x[1];
    v[2] += x[2];
    v[3] += x[3];
  }
  if (div != 1.f) {
    v[0] = v[0] / div;
    v[1] = v[1] / div;
    v[2] = v[2] / div;
    v[3] = v[3] / div;
  }
  if constexpr (sizeof(OutT) == 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t p0 = (uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[1]) << 16);
    const uint32_t p1 = (uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (OutT)v[3]) << 16);
    ((u32x2*)out)[i] = u32x2{p0, p1};
  } else {
    ((f32x4*)out)[i] = v;
  }
}

// ---------------------------------------------------------------------------
template <class Main, class Epi>
hipError_t launch_gemm(const Main& mn, const Epi& ep, int64_t tiles_m, int64_t tiles_n, hipStream_t s,
                       DynLimits dyn = {}) {
  if (tiles_m <= 0 || tiles_n <= 0) return hipSuccess;
  auto kern = gemm_kernel<Main, Epi>;
  constexpr int lds = gemm_dyn_lds<Main, Epi>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  static const hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  TileMap map{(int)tiles_m, (int)tiles_n, 4};
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(GTHREADS), lds, s, mn, ep, map, dyn);
  return hipGetLastError();
}

template <class Main, class Epi>
hipError_t launch_gemm_splitk(const Main& mn, const Epi& ep, int64_t tiles_m, int64_t tiles_n, int splits,
                              int64_t ks, int64_t pstride, hipStream_t s) {
  if (tiles_m <= 0 || tiles_n <= 0 || splits <= 0) return hipSuccess;
  auto kern = gemm_splitk_kernel<Main, Epi>;
  constexpr int lds = gemm_dyn_lds<Main, Epi>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  static const hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  TileMap map{(int)tiles_m, (int)tiles_n, 4};
  const int tiles = (int)(tiles_m * tiles_n);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles, (unsigned)splits), dim3(GTHREADS), lds, s, mn, ep, map, tiles, ks,
                     pstride);
  return hipGetLastError();
}

template <class Main, class Epi>
hipError_t launch_gemm_worklist(const Main& mn, const Epi& ep, const WorkList& wl, int64_t max_items, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  auto kern = gemm_worklist_kernel<Main, Epi>;
  static_assert(gemm_dyn_lds<Main, Epi>() == 0, "the work-list product takes no dynamic LDS");
  hipLaunchKernelGGL(kern, dim3((unsigned)max_items), dim3(GTHREADS), 0, s, mn, ep, wl);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_validate(int64_t T, int64_t V, int ignore, int64_t ignore_index, const float* temp,
                           const int32_t* top_k, const float* top_p,
                           const float* min_p, const int64_t* target, uint32_t* flags, int64_t* status,
                           hipStream_t s, int cand_ok) {
  ProfScope ps(1, s);
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0, s, T, V, ignore,
                     ignore_index, temp, top_k, top_p, min_p, target, flags, status, cand_ok);
  return hipGetLastError();
}

hipError_t launch_policy_loss(int objective, float eps_low, float eps_high, float scale, const float* adv,
                              const float* old_lp, const RowState* st, int64_t T, const float* lp, float* loss,
                              float* grad, float* ratio, hipStream_t s) {
  ProfScope ps(9, s);
  hipLaunchKernelGGL(policy_loss_kernel, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0, s, objective, eps_low,
                     eps_high, scale, adv, old_lp, st, T, lp, loss, grad, ratio);
  return hipGetLastError();
}

hipError_t launch_fill_i64(int64_t* p, int64_t v, hipStream_t s) {
  hipLaunchKernelGGL(fill_i64_kernel, dim3(1), dim3(1), 0, s, p, v);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const bf16* in, int64_t ld_in, int64_t R, int64_t Cc, bf16* out,
                                 int64_t ld_out, int64_t R_pad, hipStream_t s, const int* skip) {
  ProfScope ps(7, s);
  if (Cc % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0 && R_pad % 64 == 0 && (uintptr_t)in % 16 == 0 &&
      (uintptr_t)out % 16 == 0) {
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(R_pad / 64), (unsigned)ceil_div(Cc, 256)), dim3(256), 0,
                       s, in, ld_in, R, Cc, out, ld_out, skip);
  } else {
    hipLaunchKernelGGL(transpose_kernel<bf16>, dim3((unsigned)ceil_div(R_pad, 64), (unsigned)ceil_div(Cc, 64)),
                       dim3(256), 0, s, in, ld_in, R, Cc, out, ld_out, R_pad, skip);
  }
  return hipGetLastError();
}

hipError_t launch_prescale(int dtype, const void* in, int64_t n, float t, void* out, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(ceil_div(n8, 256) < 16384 ? ceil_div(n8, 256) : 16384);
  ProfScope ps(12, s);
  if (dtype == 1)
    hipLaunchKernelGGL(prescale_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)in, n8, t, (bf16*)out);
  else
    hipLaunchKernelGGL(prescale_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)in, n8, t, (float*)out);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_rows(const bf16* h, const int* perm, int64_t T, int64_t H, uint8_t* q, float* a,
                                    bf16* deq, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope ps(KIND_QUANTIZE, s);
  hipLaunchKernelGGL(fp8_quantize_rows_kernel, dim3((unsigned)T), dim3(256), 0, s, h, H, perm, q, a, deq);
  return hipGetLastError();
}

hipError_t launch_fp8_dequant_transpose(const uint8_t* in, const float* scale, int64_t ld_in, int64_t R, int64_t Cc,
                                        bf16* out, int64_t ld_out, int64_t R_pad, const int* skip, hipStream_t s) {
  ProfScope ps(KIND_TRANSPOSE, s);
  hipLaunchKernelGGL(fp8_dequant_transpose_kernel, dim3((unsigned)ceil_div(R_pad, 64), (unsigned)ceil_div(Cc, 64)),
                     dim3(256), 0, s, in, scale, ld_in, R, Cc, out, ld_out, R_pad, skip);
  return hipGetLastError();
}

hipError_t launch_gather_rows_dev(int dtype, const void* in, const int* rowmap, const int* n_dev, int64_t nmax,
                                  int64_t H, void* out, hipStream_t s) {
  const int64_t total = nmax * H / (dtype == 1 ? 8 : dtype == 3 ? 16 : 4);
  const unsigned blocks = (unsigned)(ceil_div(total, 256) < 2048 ? ceil_div(total, 256) : 2048);
  if (blocks == 0) return hipSuccess;
  if (dtype == 3)
    hipLaunchKernelGGL(gather_rows_dev_kernel<uint8_t>, dim3(blocks), dim3(256), 0, s, (const uint8_t*)in, rowmap,
                       n_dev, nmax, H, (uint8_t*)out);
  else if (dtype == 1)
    hipLaunchKernelGGL(gather_rows_dev_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)in, rowmap, n_dev,
                       nmax, H, (bf16*)out);
  else
    hipLaunchKernelGGL(gather_rows_dev_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)in, rowmap, n_dev,
                       nmax, H, (float*)out);
  return hipGetLastError();
}

hipError_t launch_transpose_f32(const float* in, int64_t ld_in, int64_t R, int64_t Cc, float* out,
                                int64_t ld_out, int64_t R_pad, hipStream_t s) {
  ProfScope ps(7, s);
  hipLaunchKernelGGL(transpose_kernel<float>, dim3((unsigned)ceil_div(R_pad, 64), (unsigned)ceil_div(Cc, 64)),
                     dim3(256), 0, s, in, ld_in, R, Cc, out, ld_out, R_pad, (const int*)nullptr);
  return hipGetLastError();
}

hipError_t launch_tile_partials(const float* sk, int64_t ld, int64_t R, int64_t V, int ntv,
                                const int64_t* target, TilePart* part, float* s_y, hipStream_t st) {
  ProfScope ps(8, st);
  hipLaunchKernelGGL(tile_partials_kernel, dim3((unsigned)R, (unsigned)ceil_div(ntv, 4)), dim3(256), 0, st, sk,
                     ld, R, V, ntv, target, part, s_y);
  return hipGetLastError();
}

namespace {
template <bool Ent>
hipError_t fwd_projection_impl(const FwdArgs& a, hipStream_t s) {
  EpiLogits<Ent> ep{};
  ep.tile = a.tile;
  ep.ld = a.ld;
  ep.temp = a.temp;
  ep.target = a.target;
  ep.flags = a.flags;
  ep.store_all = a.store_all;
  ep.vec = (a.ld % 4 == 0) && ((uintptr_t)a.tile % 16 == 0);
  ep.part = a.part;
  ep.ntv = a.ntv;
  ep.s_y = a.s_y;
  ep.bf16_lane = a.bf16_lane;
  ep.V = (int)a.V;
  ep.N = (int)a.rows;
  ep.ckey = a.ckey;
  ep.cid = a.cid;
  ep.cbound = a.cbound;
  ep.cld = a.cld;
  ep.rowmap = a.rowmap;
  ep.n_dev = a.n_dev;
  // a re-projection's column tiles past the device count of its rows do
  // nothing (an empty launch: every workgroup returns at once)
  DynLimits dyn{};
  dyn.n_lim = a.n_dev;
  const int64_t tm = ceil_div(a.V, GM), tn = ceil_div(a.rows, GN);
  ep.row_scale = a.row_scale;
  ep.col_scale = a.col_scale;
  ProfScope ps(a.n_dev ? KIND_REPROJECT : KIND_PROJECTION, s);
  if (a.dtype == DT_FP8) {
    MainFp8 mn{(const uint8_t*)a.W, a.H, (int)a.V, (const uint8_t*)a.h, a.H, (int)a.rows, (int)a.H};
    return launch_gemm(mn, ep, tm, tn, s, dyn);
  }
  if (a.dtype == 1) {
    MainBf16 mn{(const bf16*)a.W, a.H, (int)a.V, (const bf16*)a.h, a.H, (int)a.rows, (int)a.H};
    return launch_gemm(mn, ep, tm, tn, s, dyn);
  }
  MainF32 mn{(const float*)a.W, a.H, (int)a.V, (const float*)a.h, a.H, (int)a.rows, (int)a.H};
  return launch_gemm(mn, ep, tm, tn, s, dyn);
}
}  // namespace

// the entropy sums are formed only when requested (a separate instance)
hipError_t launch_fwd_projection(const FwdArgs& a, hipStream_t s) {
  return a.want_ent ? fwd_projection_impl<true>(a, s) : fwd_projection_impl<false>(a, s);
}

namespace {
template <class E, class Main>
hipError_t bwd_slice_impl(const BwdSliceArgs& a, hipStream_t s) {
  hipError_t e;
  const E* W = (const E*)a.W;
  // 1. recompute the slice's keys and form dz (token- and vocab-major)
  {
    EpiDlogits<E> ep{a.temp, a.target, a.st, a.g, (E*)a.d, a.ld_d, (E*)a.dT, a.Tp,
                     (int)a.v0, (int)a.vs, (int)a.vsp, (int)a.T, (int)a.Tp};
    ep.bf16_lane = a.bf16_lane;
    ep.keys_out = a.keys_out;
    ep.ld_keys = a.ld_keys;
    Main mn{W + a.v0 * a.H, a.H, (int)a.vs, (const E*)a.h, a.H, (int)a.T, (int)a.H};
    ProfScope ps(4, s);
    e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.Tp, GN), s);
    if (e != hipSuccess) return e;
  }
  if (a.keys_out) return hipSuccess;
  // 2. weight gradient of the slice: dW[v0 + m, :] = dz^T[m, :] . h^T
  if (a.grad_weight) {
    EpiStore ep{a.grad_weight + a.v0 * a.H, a.H, (int)a.vs, (int)a.H, a.accumulate_w};
    Main mn{(const E*)a.dT, a.Tp, (int)a.vsp, (const E*)a.hT, a.Tp, (int)a.H, (int)a.Tp};
    ProfScope ps(5, s);
    e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.H, GN), s);
    if (e != hipSuccess) return e;
  }
  // 3. hidden gradient, summed over slices in order: dH += dz . W_slice
  if (a.grad_hidden) {
    if constexpr (sizeof(E) == 2)
      e = launch_transpose_bf16((const bf16*)(W + a.v0 * a.H), a.H, a.vs, a.H, (bf16*)a.WT, a.ld_d, a.vsp, s);
    else
      e = launch_transpose_f32((const float*)(W + a.v0 * a.H), a.H, a.vs, a.H, (float*)a.WT, a.ld_d, a.vsp, s);
    if (e != hipSuccess) return e;
    EpiAccum<E> ep{a.dh_sum, a.H, (E*)a.grad_hidden, (int)a.T, (int)a.H, a.first, a.last, a.dh_div};
    Main mn{(const E*)a.d, a.ld_d, (int)a.T, (const E*)a.WT, a.ld_d, (int)a.H, (int)a.vsp};
    ProfScope ps(6, s);
    e = launch_gemm(mn, ep, ceil_div(a.T, GM), ceil_div(a.H, GN), s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

// bf16 slice: dz is kept vocab-major only; the weight gradient reads it
// K-major (and h MN-major), the hidden gradient is formed transposed
// (dH^T = W^T dz^T) and reads it MN-major, so neither a token-major copy of
// dz nor a transposed h is written.
hipError_t bwd_slice_bf16(const BwdSliceArgs& a, hipStream_t s) {
  hipError_t e;
  const bf16* W = (const bf16*)a.W;
  const bf16* dT = (const bf16*)a.dT;
  // 1. recompute the slice's keys and form dz^T [vsp][Tp]
  {
    EpiDlogits<bf16> ep{a.temp, a.target, a.st, a.g, nullptr, 0, (bf16*)a.dT, a.Tp,
                        (int)a.v0, (int)a.vs, (int)a.vsp, (int)a.T, (int)a.Tp};
    ep.bf16_lane = a.bf16_lane;
    ep.keys_out = a.keys_out;
    ep.ld_keys = a.ld_keys;
    MainBf16 mn{W + a.v0 * a.H, a.H, (int)a.vs, (const bf16*)a.h, a.H, (int)a.T, (int)a.H};
    ProfScope ps(4, s);
    e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.Tp, GN), s);
    if (e != hipSuccess) return e;
  }
  if (a.keys_out) return hipSuccess;
  // 2. weight gradient of the slice: dW[v0 + m, :] = sum_t dz^T[m, t] h[t, :],
  //    h read as it is (MN-major, k = token; rows past T read 0)
  if (a.grad_weight) {
    EpiStore ep{a.grad_weight + a.v0 * a.H, a.H, (int)a.vs, (int)a.H, a.accumulate_w};
    MainBf16T<false, true> mn{dT, a.Tp, (int)a.vsp, (const bf16*)a.h, a.H, (int)a.H, (int)a.Tp, 0, (int)a.T};
    ProfScope ps(5, s);
    e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.H, GN), s);
    if (e != hipSuccess) return e;
  }
  // 3. hidden gradient, summed over slices in order: dH^T += W_slice^T . dz_slice^T,
  //    with dz^T as an MN-major operand (k = vocabulary rows of the slice)
  if (a.grad_hidden) {
    e = launch_transpose_bf16(W + a.v0 * a.H, a.H, a.vs, a.H, (bf16*)a.WT, a.ld_d, a.vsp, s);
    if (e != hipSuccess) return e;
    EpiAccumT<bf16> ep{a.dh_sum, a.H, (bf16*)a.grad_hidden, (int)a.H, (int)a.T, a.first, a.last, a.dh_div};
    MainBf16T<false, true> mn{(const bf16*)a.WT, a.ld_d, (int)a.H, dT, a.Tp, (int)a.T, (int)a.vsp, 0, (int)a.vs};
    ProfScope ps(6, s);
    e = launch_gemm(mn, ep, ceil_div(a.H, GM), ceil_div(a.T, GN), s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_slice(const BwdSliceArgs& a, hipStream_t s) {
  if (a.dtype == 1) return bwd_slice_bf16(a, s);
  return bwd_slice_impl<float, MainF32>(a, s);
}

// One slice of the classed backward (bf16).  Columns of every product are
// permuted token positions; the products of the dense rows run over the
// dense prefix only (its length is a device count).
hipError_t launch_class_slice(const ClassSliceArgs& a, hipStream_t s) {
  hipError_t e;
  // 1. recompute the slice's keys: dense rows' dz^T, sparse rows' entries
  {
    auto fill = [&](auto& ep) {
      ep.perm = a.perm;
      ep.cnt = a.cnt;
      ep.temp = a.temp;
      ep.target = a.target;
      ep.st = a.st;
      ep.g = a.g;
      ep.dT = a.dT;
      ep.ld_dT = a.Tp;
      ep.v0 = (int)a.v0;
      ep.Vs = (int)a.vs;
      ep.Vs_pad = (int)a.vsp;
      ep.N = (int)a.T;
      ep.N_pad = (int)a.Tp;
      ep.bf16_lane = a.bf16_lane;
      ep.rowcnt = a.rowcnt;
      ep.list = a.list;
      ep.cntj = a.keys_out ? nullptr : a.cntj;
      ep.keys_out = a.keys_out;
      ep.ld_keys = a.ld_keys;
    };
    DynLimits dyn{};
    dyn.n_lim = a.keys_out ? nullptr : &a.cnt->full;  // dense and sparse rows (tiled ones: the tile recompute)
    ProfScope ps(KIND_DLOGITS, s);
    if (a.W8) {  // fp8 lane: the forward's e4m3 product and scaling
      EpiGradT<true, false> ep{};
      fill(ep);
      ep.row_scale = a.w_scale + a.v0;
      ep.col_scale = a.h_scale;
      MainFp8 mn{a.W8 + a.v0 * a.H, a.H, (int)a.vs, a.h8_perm, a.H, (int)a.T, (int)a.H};
      e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.Tp, GN), s, dyn);
    } else {
      EpiGradT<false, false> ep{};
      fill(ep);
      MainBf16 mn{a.W + a.v0 * a.H, a.H, (int)a.vs, a.h_perm, a.H, (int)a.T, (int)a.H};
      e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.Tp, GN), s, dyn);
    }
    if (e != hipSuccess) return e;
  }
  if (a.keys_out) return hipSuccess;
  // 2. dense rows' weight gradient of the slice: dW[v0 + m, :] (+)= sum over
  //    dense positions n of dz^T[m, n] h_perm[n, :] (no tile runs without dense rows)
  if (a.grad_weight) {
    EpiStore ep{a.grad_weight + a.v0 * a.H, a.H, (int)a.vs, (int)a.H, a.accumulate_w};
    MainBf16T<false, true> mn{a.dT, a.Tp, (int)a.vsp, a.h_perm, a.H, (int)a.H, (int)a.Tp, 0, (int)a.T};
    DynLimits dyn{};
    dyn.k_lim = &a.cnt->dense;
    ProfScope ps(KIND_GRAD_WEIGHT, s);
    e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.H, GN), s, dyn);
    if (e != hipSuccess) return e;
  }
  // 3. dense rows' hidden gradient, summed over slices in order:
  //    dH^T[:, n] += W_slice^T . dz^T[:, n] for dense positions n, written to row perm[n]
  if (a.grad_hidden) {
    if (a.W8)  // fp8 lane: the dequantized weight, rounded to bf16, as the product's operand
      e = launch_fp8_dequant_transpose(a.W8 + a.v0 * a.H, a.w_scale + a.v0, a.H, a.vs, a.H, a.WT, a.ld_d, a.vsp,
                                       &a.cnt->dense, s);
    else
      e = launch_transpose_bf16(a.W + a.v0 * a.H, a.H, a.vs, a.H, a.WT, a.ld_d, a.vsp, s, &a.cnt->dense);
    if (e != hipSuccess) return e;
    EpiAccumT<bf16> ep{a.dh_sum, a.H, (bf16*)a.grad_hidden, (int)a.H, (int)a.T, a.first, a.last, a.dh_div};
    ep.rowmap = a.perm;
    ep.n_dev = &a.cnt->dense;
    MainBf16T<false, true> mn{a.WT, a.ld_d, (int)a.H, a.dT, a.Tp, (int)a.T, (int)a.vsp, 0, (int)a.vs};
    DynLimits dyn{};
    dyn.n_lim = &a.cnt->dense;
    ProfScope ps(KIND_GRAD_HIDDEN, s);
    e = launch_gemm(mn, ep, ceil_div(a.H, GM), ceil_div(a.T, GN), s, dyn);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {
template <class E, class Main>
hipError_t fused_grads_impl(const FusedGradArgs& a, hipStream_t s) {
  hipError_t e;
  // 1. dz of the chunk, vocab-major into the group's dT [V_pad][ld_dT] and
  //    (fp32 only) token-major d [rows_pad][V_pad]
  {
    constexpr int TT = sizeof(E) == 2 ? 64 : 32;
    ProfScope ps(10, s);
    hipLaunchKernelGGL(dz_keys_kernel<E>, dim3((unsigned)ceil_div(a.V_pad, 256), (unsigned)ceil_div(a.rows_pad, TT)),
                       dim3(256), 0, s, a.keys, a.ld_keys, a.temp, a.target, a.st, a.g, (int)a.rows, (int)a.rows_pad,
                       (int)a.V, (int)a.V_pad, sizeof(E) == 2 ? nullptr : (E*)a.d, a.V_pad, (E*)a.dT + a.dT_col,
                       a.ld_dT);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 2. the chunk's hidden-gradient rows over vocabulary splits, fp32
  //    partials, then their sum in split order; bf16 forms them transposed,
  //    dH^T = W^T . dz^T, reading the chunk's columns of dT MN-major
  if (a.grad_hidden) {
    if constexpr (sizeof(E) == 2) {
      MainBf16T<false, true> mn{(const bf16*)a.WT, a.V_pad, (int)a.H, (const bf16*)a.dT + a.dT_col, a.ld_dT,
                                (int)a.rows, (int)a.V_pad, 0, (int)a.V_pad};
      EpiAccumT<float> ep{a.dh_part, a.H, a.dh_part, (int)a.H, (int)a.rows, 1, 1};
      ProfScope ps(6, s);
      e = launch_gemm_splitk(mn, ep, ceil_div(a.H, GM), ceil_div(a.rows, GN), a.splits, a.ks, a.rows * a.H, s);
    } else {
      Main mn{(const E*)a.d, a.V_pad, (int)a.rows, (const E*)a.WT, a.V_pad, (int)a.H, (int)a.V_pad};
      EpiStore ep{a.dh_part, a.H, (int)a.rows, (int)a.H, 0};
      ProfScope ps(6, s);
      e = launch_gemm_splitk(mn, ep, ceil_div(a.rows, GM), ceil_div(a.H, GN), a.splits, a.ks, a.rows * a.H, s);
    }
    if (e != hipSuccess) return e;
    const int64_t n4 = a.rows * a.H / 4;
    ProfScope ps(11, s);
    hipLaunchKernelGGL(sum_splits_kernel<E>, dim3((unsigned)ceil_div(n4, 256)), dim3(256), 0, s, a.dh_part, a.splits,
                       a.rows * a.H, n4, a.dh_div, (E*)a.grad_hidden);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 3. weight gradient of a finished group: dW (+)= dz^T . h over the
  //    group's rows (zero dT columns for the padding rows)
  if (a.grad_weight && a.dw) {
    EpiStore ep{a.grad_weight, a.H, (int)a.V, (int)a.H, a.accumulate_w};
    ProfScope ps(5, s);
    if constexpr (sizeof(E) == 2) {
      // h read as it is (MN-major): rows dw_c0 .. of the T that exist
      MainBf16T<false, true> mn{(const bf16*)a.dT, a.ld_dT, (int)a.V, (const bf16*)a.h + a.dw_c0 * a.H, a.H,
                                (int)a.H, (int)a.dw_k, 0, (int)(a.T - a.dw_c0)};
      e = launch_gemm(mn, ep, ceil_div(a.V, GM), ceil_div(a.H, GN), s);
    } else {
      Main mn{(const E*)a.dT, a.ld_dT, (int)a.V, (const E*)a.hT + a.dw_c0, a.Tp, (int)a.H, (int)a.dw_k};
      e = launch_gemm(mn, ep, ceil_div(a.V, GM), ceil_div(a.H, GN), s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_fused_chunk_grads(const FusedGradArgs& a, hipStream_t s) {
  if (a.dtype == 1) return fused_grads_impl<bf16, MainBf16>(a, s);
  return fused_grads_impl<float, MainF32>(a, s);
}


hipError_t launch_tiled_recompute(const TiledArgs& a, hipStream_t s) {
  static_assert(TILE_COLS == GN, "a work item is one N tile of the product");
  hipError_t e;
  {
    ProfScope ps(KIND_TILE_LISTS, s);
    if ((e = launch_tile_lists(a.lists, s))) return e;
  }
  auto fill = [&](auto& ep) {
    ep.perm = a.perm;
    ep.cnt = a.cnt;
    ep.temp = a.temp;
    ep.target = a.target;
    ep.st = a.st;
    ep.g = a.g;
    ep.dT = nullptr;  // no dense row here
    ep.ld_dT = 0;
    ep.v0 = 0;
    ep.Vs = (int)a.V;
    ep.Vs_pad = (int)round_up(a.V, 64);
    ep.N = (int)a.T;
    ep.N_pad = (int)round_up(a.T, 64);
    ep.bf16_lane = a.bf16_lane;
    ep.rowcnt = a.rowcnt;
    ep.list = a.list;
    ep.cntj = a.keys_out ? nullptr : a.cntj;
    ep.keys_out = a.keys_out;
    ep.ld_keys = a.ld_keys;
  };
  const WorkList wl{a.lists.twoff, a.lists.tcnt, a.lists.toff, a.lists.bucket, (int)a.lists.ntv};
  // most work items: a tile's items are ceil(count / GN) <= count / GN + 1
  const int64_t items = a.lists.ntv + ceil_div(NTILE * a.T, GN);
  ProfScope ps(KIND_TILE_RECOMPUTE, s);
  if (a.W8) {
    EpiGradT<true, true> ep{};
    fill(ep);
    ep.row_scale = a.w_scale;
    ep.col_scale = a.h_scale;
    MainFp8G mn{a.W8, a.H, (int)a.V, a.h8_perm, a.H, 0, (int)a.H};
    mn.nrecB = (int)(a.T * a.H);
    return launch_gemm_worklist(mn, ep, wl, items, s);
  }
  EpiGradT<false, true> ep{};
  fill(ep);
  MainBf16G mn{a.W, a.H, (int)a.V, a.h_perm, a.H, 0, (int)a.H};
  mn.nrecB = (int)(a.T * a.H * 2);
  return launch_gemm_worklist(mn, ep, wl, items, s);
}

}  // namespace stce
