// Block-tiled "NT" matrix product for gfx950: C[m, n] = sum_k A[m, k] * B[n, k]
// with both operands row-major and contiguous along k.  Every product of the
// scoring core has this form once the backward keeps transposed copies of its
// operands (h^T, a W^T slice, dz^T):
//   projection   z^T[v, t] = W[v, :] . h[t, :]       (M = vocab, N = tokens, K = H)
//   weight grad  dW[v, :] = dz^T[v, :] . h^T[:, :]   (M = vocab, N = H,      K = tokens)
//   hidden grad  dH[t, :] = dz[t, :] . W^T[:, :]     (M = tokens, N = H,     K = vocab)
//
// Block tile 256 x 256, k-step 64, 256 threads = 4 waves in a 2 x 2 grid, each
// wave owning a 128 x 128 sub-tile = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16.
// Operands are staged through registers into double-buffered LDS tiles whose
// 16-byte chunks are XOR-swizzled by row, so the fragment reads (32 rows at
// one k offset) spread over all banks.  An output element's k order is the
// same in every launch (no split-k), so the projection is bitwise identical
// wherever a row or vocabulary slice falls; the backward relies on it.
//
// Accumulator layout, shared by both main loops and read by the epilogues:
// acc[i][j][r] of lane l in wave (wm, wn) holds
//   m = m0 + wm*128 + i*32 + (r/4)*8 + (l/32)*4 + (r%4)
//   n = n0 + wn*128 + j*32 + (l%32).
#pragma once

#include "common.hpp"

namespace stce {

constexpr int GM = 256, GN = 256, GK = 64;
constexpr int GTHREADS = 256;

// Linear workgroup id -> output tile.  Workgroups are dispatched round-robin
// over the 8 XCDs (id % 8); the remap gives each XCD a contiguous range of
// logical tiles, and the logical order sweeps groups of `group_m` tile rows
// across all tile columns so that the tiles one XCD runs together share
// operand panels in its L2.
struct TileMap {
  int tiles_m, tiles_n, group_m;
  __device__ inline void get(int bid, int& tm, int& tn) const {
    const int total = tiles_m * tiles_n;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    const int lid = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
    const int gsz = group_m * tiles_n;
    const int g = lid / gsz;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in = lid - g * gsz;
    tm = first_m + in % gm;
    tn = in / gm;
  }
};

__device__ inline int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------
// bf16 main loop (MFMA)
// ---------------------------------------------------------------------------
struct MainBf16 {
  static constexpr int LDS_BYTES = 2 * 2 * GM * GK * 2;  // 2 stages x (A, B) x 32 KB
  const bf16* A;
  int64_t lda;
  int M;  // rows of A that exist (loads clamp to M - 1)
  const bf16* B;
  int64_t ldb;
  int N;
  int K;  // multiple of 8

  __device__ inline void run(f32x16 (&acc)[4][4], int m0, int n0, char* smem) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int lr = tid >> 3, lch = tid & 7;          // load: rows lr + 32 i, chunk lch
    const int soff = (lr * 8 + (lch ^ (lr & 7))) * 16;  // byte offset of that chunk in LDS

    const bf16* ga[8];
    const bf16* gb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ga[i] = A + (int64_t)min(m0 + lr + 32 * i, M - 1) * lda + lch * 8;
      gb[i] = B + (int64_t)min(n0 + lr + 32 * i, N - 1) * ldb + lch * 8;
    }
    u32x4 ra[8], rb[8];
    auto load = [&](int k0) {
      if (k0 + GK <= K) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ra[i] = *(const u32x4*)(ga[i] + k0);
          rb[i] = *(const u32x4*)(gb[i] + k0);
        }
      } else {
        const bool in = k0 + lch * 8 < K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ra[i] = in ? *(const u32x4*)(ga[i] + k0) : u32x4{0, 0, 0, 0};
          rb[i] = in ? *(const u32x4*)(gb[i] + k0) : u32x4{0, 0, 0, 0};
        }
      }
    };
    auto store = [&](int stage) {
      char* sa = smem + stage * 65536;
      char* sb = sa + 32768;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *(u32x4*)(sa + soff + i * 32 * 128) = ra[i];
        *(u32x4*)(sb + soff + i * 32 * 128) = rb[i];
      }
    };

    // fragment read offsets: row = wm*128 + i*32 + lane%32 (row & 7 == lane & 7)
    const int frow = lane & 31, fsw = lane & 7, fhalf = lane >> 5;
    const int nk = (K + GK - 1) / GK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load((kt + 1) * GK);
      const char* sa = smem + cur * 65536;
      const char* sb = sa + 32768;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = ((kk * 2 + fhalf) ^ fsw) * 16;
        bf16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = *(const bf16x8*)(sa + (wm * 128 + i * 32 + frow) * 128 + ch);
          b[i] = *(const bf16x8*)(sb + (wn * 128 + i * 32 + frow) * 128 + ch);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store(cur ^ 1);
      __syncthreads();
    }
  }
};

// ---------------------------------------------------------------------------
// fp32 main loop (plain fused multiply-adds, same accumulator layout).  Used
// for fp32 operands, where shapes are small; each output element accumulates
// its k terms in order with one fma each.
// ---------------------------------------------------------------------------
struct MainF32 {
  static constexpr int BK = 16;
  static constexpr int LDS_BYTES = 2 * GM * (BK + 1) * 4;
  const float* A;
  int64_t lda;
  int M;
  const float* B;
  int64_t ldb;
  int N;
  int K;  // multiple of 4

  __device__ inline void run(f32x16 (&acc)[4][4], int m0, int n0, char* smem) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    float* sa = (float*)smem;              // [256][17]
    float* sb = sa + GM * (BK + 1);         // [256][17]
    const float* ga = A + (int64_t)min(m0 + tid, M - 1) * lda;
    const float* gb = B + (int64_t)min(n0 + tid, N - 1) * ldb;
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
      for (int c = 0; c < BK; c += 4) {
        const bool in = k0 + c < K;
        f32x4 va = in ? *(const f32x4*)(ga + k0 + c) : f32x4{0, 0, 0, 0};
        f32x4 vb = in ? *(const f32x4*)(gb + k0 + c) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sa[tid * (BK + 1) + c + e] = va[e];
          sb[tid * (BK + 1) + c + e] = vb[e];
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int kk = 0; kk < BK; ++kk) {
        float bv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = sb[(wn * 128 + j * 32 + (lane & 31)) * (BK + 1) + kk];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float av = sa[(wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * (BK + 1) + kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j][r] = __builtin_fmaf(av, bv[j], acc[i][j][r]);
          }
      }
      __syncthreads();
    }
  }
};

template <class Main, class Epi>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_kernel(Main mainloop, Epi epi, TileMap map) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int tm, tn;
  map.get(blockIdx.x, tm, tn);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  mainloop.run(acc, tm * GM, tn * GN, smem);
  epi(acc, tm * GM, tn * GN, smem);
}

}  // namespace stce
