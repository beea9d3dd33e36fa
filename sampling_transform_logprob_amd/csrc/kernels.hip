// Small kernels (validation, transposes, tile partials) and the launchers of
// the block-tiled products with their epilogues.
#include "epilogues.hpp"
#include "kernels.hpp"

namespace stce {
namespace {

// ---------------------------------------------------------------------------
__global__ void validate_kernel(int64_t T, int64_t V, int ignore, int64_t ignore_index, const float* temp,
                                const int32_t* top_k, const float* top_p, const float* min_p,
                                const int64_t* target, uint32_t* flags, int64_t* status) {
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
  flags[t] = field ? 0u : (ROW_VALID | (filtered ? ROW_FILTERED : 0u) | (ign ? ROW_IGNORED : 0u));
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
                                 int64_t R_pad) {
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
                                                             bf16* out, int64_t ld_out) {
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

// ---------------------------------------------------------------------------
template <class Main, class Epi>
hipError_t launch_gemm(const Main& mn, const Epi& ep, int64_t tiles_m, int64_t tiles_n, hipStream_t s) {
  if (tiles_m <= 0 || tiles_n <= 0) return hipSuccess;
  auto kern = gemm_kernel<Main, Epi>;
  constexpr int lds = Main::LDS_BYTES > Epi::LDS_BYTES ? Main::LDS_BYTES : Epi::LDS_BYTES;
  static_assert(lds <= 160 * 1024, "LDS budget");
  static const hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  TileMap map{(int)tiles_m, (int)tiles_n, 4};
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(GTHREADS), lds, s, mn, ep, map);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_validate(int64_t T, int64_t V, int ignore, int64_t ignore_index, const float* temp,
                           const int32_t* top_k, const float* top_p,
                           const float* min_p, const int64_t* target, uint32_t* flags, int64_t* status,
                           hipStream_t s) {
  ProfScope ps(1, s);
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0, s, T, V, ignore,
                     ignore_index, temp, top_k, top_p, min_p, target, flags, status);
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
                                 int64_t ld_out, int64_t R_pad, hipStream_t s) {
  ProfScope ps(7, s);
  if (Cc % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0 && R_pad % 64 == 0 && (uintptr_t)in % 16 == 0 &&
      (uintptr_t)out % 16 == 0) {
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(R_pad / 64), (unsigned)ceil_div(Cc, 256)), dim3(256), 0,
                       s, in, ld_in, R, Cc, out, ld_out);
  } else {
    hipLaunchKernelGGL(transpose_kernel<bf16>, dim3((unsigned)ceil_div(R_pad, 64), (unsigned)ceil_div(Cc, 64)),
                       dim3(256), 0, s, in, ld_in, R, Cc, out, ld_out, R_pad);
  }
  return hipGetLastError();
}

hipError_t launch_transpose_f32(const float* in, int64_t ld_in, int64_t R, int64_t Cc, float* out,
                                int64_t ld_out, int64_t R_pad, hipStream_t s) {
  ProfScope ps(7, s);
  hipLaunchKernelGGL(transpose_kernel<float>, dim3((unsigned)ceil_div(R_pad, 64), (unsigned)ceil_div(Cc, 64)),
                     dim3(256), 0, s, in, ld_in, R, Cc, out, ld_out, R_pad);
  return hipGetLastError();
}

hipError_t launch_tile_partials(const float* sk, int64_t ld, int64_t R, int64_t V, int ntv,
                                const int64_t* target, TilePart* part, float* s_y, hipStream_t st) {
  ProfScope ps(8, st);
  hipLaunchKernelGGL(tile_partials_kernel, dim3((unsigned)R, (unsigned)ceil_div(ntv, 4)), dim3(256), 0, st, sk,
                     ld, R, V, ntv, target, part, s_y);
  return hipGetLastError();
}

hipError_t launch_fwd_projection(const FwdArgs& a, hipStream_t s) {
  EpiLogits ep{};
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
  ep.want_ent = a.want_ent;
  ep.V = (int)a.V;
  ep.N = (int)a.rows;
  const int64_t tm = ceil_div(a.V, GM), tn = ceil_div(a.rows, GN);
  ProfScope ps(2, s);
  if (a.dtype == 1) {
    MainBf16 mn{(const bf16*)a.W, a.H, (int)a.V, (const bf16*)a.h, a.H, (int)a.rows, (int)a.H};
    return launch_gemm(mn, ep, tm, tn, s);
  }
  MainF32 mn{(const float*)a.W, a.H, (int)a.V, (const float*)a.h, a.H, (int)a.rows, (int)a.H};
  return launch_gemm(mn, ep, tm, tn, s);
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
    Main mn{W + a.v0 * a.H, a.H, (int)a.vs, (const E*)a.h, a.H, (int)a.T, (int)a.H};
    ProfScope ps(4, s);
    e = launch_gemm(mn, ep, ceil_div(a.vsp, GM), ceil_div(a.Tp, GN), s);
    if (e != hipSuccess) return e;
  }
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
    EpiAccum<E> ep{a.dh_sum, a.H, (E*)a.grad_hidden, (int)a.T, (int)a.H, a.first, a.last};
    Main mn{(const E*)a.d, a.ld_d, (int)a.T, (const E*)a.WT, a.ld_d, (int)a.H, (int)a.vsp};
    ProfScope ps(6, s);
    e = launch_gemm(mn, ep, ceil_div(a.T, GM), ceil_div(a.H, GN), s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_bwd_slice(const BwdSliceArgs& a, hipStream_t s) {
  if (a.dtype == 1) return bwd_slice_impl<bf16, MainBf16>(a, s);
  return bwd_slice_impl<float, MainF32>(a, s);
}

}  // namespace stce
