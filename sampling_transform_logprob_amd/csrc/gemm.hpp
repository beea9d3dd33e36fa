// Block-tiled "NT" matrix product for gfx950: C[m, n] = sum_k A[m, k] * B[n, k]
// with both operands row-major and contiguous along k.  Every product of the
// scoring core has this form once the backward keeps transposed copies of its
// operands (h^T, a W^T slice, dz^T):
//   projection   z^T[v, t] = W[v, :] . h[t, :]       (M = vocab, N = tokens, K = H)
//   weight grad  dW[v, :] = dz^T[v, :] . h^T[:, :]   (M = vocab, N = H,      K = tokens)
//   hidden grad  dH[t, :] = dz[t, :] . W^T[:, :]     (M = tokens, N = H,     K = vocab)
//
// Block tile 256 x 256, k-step 64, 512 threads = 8 waves (2 per SIMD) in a
// 2 (m) x 4 (n) grid, each wave owning a 128 x 64 sub-tile = 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16.  Operand tiles go straight from global memory to
// LDS with buffer loads (buffer_load_dwordx4 ... lds): each instruction fills
// 1 KB of LDS, lane l writing bytes [16 l, 16 l + 16) of it, so the lane ->
// global address mapping realizes the LDS layout.  Rows are 128 bytes; the
// 16-byte chunks of a row are XOR-permuted by (row >> 1) & 7, which makes
// the fragment reads (16 lanes = 16 consecutive rows at one k offset per
// LDS cycle on the 64-bank LDS) conflict-free.  Two LDS stages: the loads of
// k-tile t + 2 are issued right after the barrier that frees stage t % 2,
// which sits before the last k-step of tile t, so they, and the first
// fragment reads of tile t + 1, overlap that k-step's MFMAs.  Fragment reads
// of k-step s + 1 are interleaved one per MFMA with the MFMAs of k-step s.
// Out-of-range rows and k-columns read as zeros (buffer range checking).
// An output element's k order is the same in every launch (no split-k), so
// the projection is bitwise identical wherever a row or vocabulary slice
// falls; the backward relies on it.
//
// Accumulator layout, shared by both main loops and read by the epilogues:
// acc[i][j][r] (i < 4, j < 2, r < 16) of lane l in wave w (wm = w / 4,
// wn = w % 4) holds
//   m = m0 + wm*128 + i*32 + (r/4)*8 + (l/32)*4 + (r%4)
//   n = n0 + wn*64 + j*32 + (l%32).
#pragma once

#include "common.hpp"

namespace stce {

constexpr int GM = 256, GN = 256, GK = 64;
constexpr int GTHREADS = 512;
constexpr int ACC_I = 4, ACC_J = 2;

typedef f32x16 AccTile[ACC_I][ACC_J];

__device__ inline int acc_row(int wm, int i, int r, int half) { return wm * 128 + i * 32 + (r >> 2) * 8 + half * 4 + (r & 3); }
__device__ inline int acc_col(int wn, int j, int col) { return wn * 64 + j * 32 + col; }

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

#define STCE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// range checking on): used for all operand loads.
constexpr int RSRC_WORD3 = 0x00020000;

__device__ inline int lds_swz(int row) { return (row >> 1) & 7; }

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits 3:0 and 15:14,
// expcnt in 6:4, lgkmcnt in 11:8.
constexpr int WAIT_VM0_LGKM0 = 0x0070;

// ---------------------------------------------------------------------------
// bf16 main loop (MFMA)
// ---------------------------------------------------------------------------
struct MainBf16 {
  static constexpr int LDS_BYTES = 2 * 2 * GM * GK * 2;  // 2 stages x (A, B) x 32 KB
  static constexpr int ROWB = GK * 2;                     // 128-byte tile rows
  static constexpr int TILEB = GM * ROWB;                 // one operand tile
  static constexpr int STAGEB = 2 * TILEB;
  static constexpr int LPW = 4;                           // 1 KB loads per wave per operand per k-tile
  const bf16* A;
  int64_t lda;
  int M;  // rows of A that exist
  const bf16* B;
  int64_t ldb;
  int N;
  int K;  // multiple of 8

  __device__ inline void run(AccTile& acc, int m0, int n0, char* smem) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3;
    // each resource spans only this tile's (at most 256) rows, so offsets
    // stay far below 2^31 and the tail sentinel below is always out of range
    const int rowsA = min(M - m0, GM), rowsB = min(N - n0, GN);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * lda), (short)0,
                                                                        rowsA * (int)lda * 2, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)n0 * ldb), (short)0,
                                                                        rowsB * (int)ldb * 2, RSRC_WORD3);
    // load instruction i of wave w fills rows (w*LPW + i)*8 .. +8 of a tile;
    // lane l covers row + l/8, physical chunk l%8
    const int lrow = lane >> 3, lpc = lane & 7;
    int voffA[LPW], voffB[LPW], lchunk[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row = (w * LPW + i) * 8 + lrow;
      lchunk[i] = lpc ^ lds_swz(row);
      voffA[i] = row * (int)lda * 2 + lchunk[i] * 16;
      voffB[i] = row * (int)ldb * 2 + lchunk[i] * 16;
    }
    const int nk = (K + GK - 1) / GK;
    auto issue = [&](int kt) {
      char* st = smem + (kt & 1) * STAGEB;
      const int k0 = kt * GK;
      const int so = k0 * 2;
      if (k0 + GK <= K) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, STCE_LDS(st + (w * LPW + i) * 1024), 16, voffA[i], so, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, STCE_LDS(st + TILEB + (w * LPW + i) * 1024), 16, voffB[i], so,
                                                   0, 0);
        }
      } else {
        // k tail: chunks at or past K get an offset beyond the buffer's
        // range, which the hardware turns into zeros
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
          const bool in = k0 + lchunk[i] * 8 < K;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, STCE_LDS(st + (w * LPW + i) * 1024), 16,
                                                   in ? voffA[i] : 0x7ffffff0, so, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, STCE_LDS(st + TILEB + (w * LPW + i) * 1024), 16,
                                                   in ? voffB[i] : 0x7ffffff0, so, 0, 0);
        }
      }
    };
    const int frow = lane & 31, fhalf = lane >> 5, sw = lds_swz(frow);
    int offA[4], offB[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) offA[i] = (wm * 128 + i * 32 + frow) * ROWB;
#pragma unroll
    for (int j = 0; j < 2; ++j) offB[j] = TILEB + (wn * 64 + j * 32 + frow) * ROWB;
    auto rd = [&](bf16x8 (&a)[4], bf16x8 (&b)[2], int kt, int kk) {
      const char* st = smem + (kt & 1) * STAGEB;
      const int ch = ((kk * 2 + fhalf) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(st + offA[i] + ch);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)(st + offB[j] + ch);
    };

    issue(0);
    __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
    __syncthreads();
    bf16x8 fa[2][4], fb[2][2];
    rd(fa[0], fb[0], 0, 0);
    if (1 < nk) issue(1);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int cur = kk & 1, nxt = cur ^ 1;
        if (kk < 3) {
          rd(fa[nxt], fb[nxt], kt, kk + 1);
        } else if (kt + 1 < nk) {
          // tile kt + 1 has landed (every wave waits for its own loads) and
          // every wave is done reading stage kt & 1 before it is refilled
          __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
          __syncthreads();
          rd(fa[nxt], fb[nxt], kt + 1, 0);
          if (kt + 2 < nk) issue(kt + 2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        // one LDS read (or operand load) issued after each MFMA
#pragma unroll
        for (int q = 0; q < 6; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, LPW, 0);
        }
      }
    }
    __syncthreads();  // the epilogue may reuse the LDS
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

  __device__ inline void run(AccTile& acc, int m0, int n0, char* smem) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3;
    float* sa = (float*)smem;              // [256][17]
    float* sb = sa + GM * (BK + 1);         // [256][17]
    // thread t loads half a row: row t / 2, columns (t & 1) * 8 .. + 8
    const int lr = tid >> 1, lc = (tid & 1) * 8;
    const float* ga = A + (int64_t)min(m0 + lr, M - 1) * lda + lc;
    const float* gb = B + (int64_t)min(n0 + lr, N - 1) * ldb + lc;
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
      for (int c = 0; c < 8; c += 4) {
        const bool in = k0 + lc + c < K;
        f32x4 va = in ? *(const f32x4*)(ga + k0 + c) : f32x4{0, 0, 0, 0};
        f32x4 vb = in ? *(const f32x4*)(gb + k0 + c) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sa[lr * (BK + 1) + lc + c + e] = va[e];
          sb[lr * (BK + 1) + lc + c + e] = vb[e];
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int kk = 0; kk < BK; ++kk) {
        float bv[ACC_J];
#pragma unroll
        for (int j = 0; j < ACC_J; ++j) bv[j] = sb[acc_col(wn, j, lane & 31) * (BK + 1) + kk];
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float av = sa[acc_row(wm, i, r, lane >> 5) * (BK + 1) + kk];
#pragma unroll
            for (int j = 0; j < ACC_J; ++j) acc[i][j][r] = __builtin_fmaf(av, bv[j], acc[i][j][r]);
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
  AccTile acc;
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) acc[i][j] = f32x16{};
  mainloop.run(acc, tm * GM, tn * GN, smem);
  epi(acc, tm * GM, tn * GN, smem);
}

}  // namespace stce
