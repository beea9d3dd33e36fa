// Block-tiled "NT" matrix product for gfx950: C[m, n] = sum_k A[m, k] * B[n, k]
// with both operands row-major and contiguous along k.  Every product of the
// scoring core has this form once the backward keeps transposed copies of its
// operands (h^T, a W^T slice, dz^T):
//   projection   z^T[v, t] = W[v, :] . h[t, :]       (M = vocab, N = tokens, K = H)
//   weight grad  dW[v, :] = dz^T[v, :] . h^T[:, :]   (M = vocab, N = H,      K = tokens)
//   hidden grad  dH[t, :] = dz[t, :] . W^T[:, :]     (M = tokens, N = H,     K = vocab)
//
// Block tile 256 x 256, k-tile 64, 512 threads = 8 waves (2 per SIMD) in a
// 2 (m) x 4 (n) grid, each wave owning a 128 x 64 sub-tile = 8 x 4 blocks of
// v_mfma_f32_16x16x32_bf16.  (On this part the 16x16x32 form sustains a
// higher clock under full load than the 32x32x16 form, for the same work per
// cycle.)  Operand tiles go straight from global memory to LDS with buffer
// loads (buffer_load_dwordx4 ... lds): each instruction fills 1 KB of LDS,
// lane l writing bytes [16 l, 16 l + 16) of it, so the lane -> global address
// mapping realizes the LDS layout.  Rows are 128 bytes; the 16-byte chunks of
// a row are XOR-permuted by (row >> 1) & 7, which makes the fragment reads
// (16 lanes = 16 consecutive rows at one k offset per LDS cycle on the
// 64-bank LDS) conflict-free.  Two LDS stages.  A k-tile is two k-steps of
// 32; the fragments of k-step s + 1 are read (one LDS read per two MFMAs)
// while the MFMAs of k-step s run.  Halfway through the last k-step of tile t
// sits the one barrier of the tile: it waits for tile t + 1 to land and frees
// stage t % 2; right after it the first fragments of tile t + 1 are read and
// the loads of tile t + 2 are issued, interleaved with the remaining MFMAs,
// so the matrix pipe keeps work queued across the barrier.  The steady-state
// tile is one basic block (no branches), which keeps that interleaving
// intact.  Out-of-range rows and k-columns read as zeros (buffer range
// checking).  An output element's k order is the same in every launch (no
// split-k), so the projection is bitwise identical wherever a row or
// vocabulary slice falls; the backward relies on it.
//
// Accumulator layout, shared by both main loops and read by the epilogues:
// acc[i][j][r] (i < 8, j < 4, r < 4) of lane l in wave w (wm = w / 4,
// wn = w % 4) holds
//   m = m0 + wm*128 + i*16 + (l/16)*4 + r
//   n = n0 + wn*64 + j*16 + (l%16).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace stce {

constexpr int GM = 256, GN = 256, GK = 64;
constexpr int GTHREADS = 512;
constexpr int ACC_I = 8, ACC_J = 4, ACC_R = 4;

typedef f32x4 AccTile[ACC_I][ACC_J];

// quad = lane / 16, col = lane % 16
__device__ inline int acc_row(int wm, int i, int r, int quad) { return wm * 128 + i * 16 + quad * 4 + r; }
__device__ inline int acc_col(int wn, int j, int col) { return wn * 64 + j * 16 + col; }

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
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
    const int wm = w >> 2, wn = w & 3;
    // each resource spans only this tile's (at most 256) rows, so offsets
    // stay far below 2^31 and the tail sentinel below is always out of range
    const int rowsA = min(M - m0, GM), rowsB = min(N - n0, GN);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * lda), (short)0,
                                                                        rowsA * (int)lda * 2, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)n0 * ldb), (short)0,
                                                                        rowsB * (int)ldb * 2, RSRC_WORD3);
    // load instruction i of wave w fills rows (w*LPW + i)*8 .. +8 of a tile;
    // lane l covers row + l/8 and physical chunk l%8, i.e. logical chunk
    // (l%8) ^ swz(row); the swizzle uses row bits 1..3, bit 3 being the
    // parity of i
    const int lrow = lane >> 3, lpc = lane & 7;
    const int ce = lpc ^ lds_swz(lrow), co = lpc ^ lds_swz(lrow + 8);
    const int rA = (w * LPW * 8 + lrow) * (int)lda * 2, rB = (w * LPW * 8 + lrow) * (int)ldb * 2;
    const int stepA = 8 * (int)lda * 2, stepB = 8 * (int)ldb * 2;
    const int nk = (K + GK - 1) / GK;
    // loads of k-tile kt into stage kt % 2; 16-byte chunks at or past K get
    // an offset beyond the buffer's range, which the hardware turns into zeros
    auto issue = [&](int kt) __attribute__((always_inline)) {
      char* st = smem + (kt & 1) * STAGEB + w * LPW * 1024;
      const int k0 = kt * GK, so = k0 * 2;
      const bool ine = k0 + ce * 8 < K, ino = k0 + co * 8 < K;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const bool in = (i & 1) ? ino : ine;
        const int c16 = ((i & 1) ? co : ce) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, STCE_LDS(st + i * 1024), 16, in ? rA + i * stepA + c16 : 0x7ffffff0,
                                                 so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, STCE_LDS(st + TILEB + i * 1024), 16,
                                                 in ? rB + i * stepB + c16 : 0x7ffffff0, so, 0, 0);
      }
    };
    // fragment of a 16 x 32 (rows x k) block: lane l reads row l % 16, the
    // 16-byte chunk l / 16 of the k-step's 32 columns
    const int frow = lane & 15, fq = lane >> 4, sw = lds_swz(frow);
    const int offA = (wm * 128 + frow) * ROWB, offB = TILEB + (wn * 64 + frow) * ROWB;
    bf16x8 fa[2][ACC_I], fb[2][ACC_J];
    auto rd = [&](bf16x8 (&a)[ACC_I], bf16x8 (&b)[ACC_J], int kt, int kk) __attribute__((always_inline)) {
      const char* st = smem + (kt & 1) * STAGEB;
      const int ch = ((kk * 4 + fq) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < ACC_I; ++i) a[i] = *(const bf16x8*)(st + offA + i * 16 * ROWB + ch);
#pragma unroll
      for (int j = 0; j < ACC_J; ++j) b[j] = *(const bf16x8*)(st + offB + j * 16 * ROWB + ch);
    };
    auto mma = [&](int cur, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
      for (int i = i0; i < i1; ++i)
#pragma unroll
        for (int j = 0; j < ACC_J; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    };
    // one k-tile; NEXT: a tile follows (barrier + its first fragments),
    // ISSUE: the tile after that is loaded into the stage this one frees
    auto tile = [&](int kt, auto next_c, auto issue_c) __attribute__((always_inline)) {
      constexpr bool NEXT = decltype(next_c)::value, ISSUE = decltype(issue_c)::value;
      rd(fa[1], fb[1], kt, 1);
      mma(0, 0, ACC_I);
#pragma unroll
      for (int q = 0; q < ACC_I + ACC_J; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, ACC_I * ACC_J - 2 * (ACC_I + ACC_J), 0);
      mma(1, 0, 2);
      __builtin_amdgcn_sched_barrier(0);
      if (NEXT) {
        // tile kt + 1 has landed (every wave waits for its own loads) and
        // every wave is done reading stage kt % 2 before it is refilled
        __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        rd(fa[0], fb[0], kt + 1, 0);
        if (ISSUE) issue(kt + 2);
      }
      mma(1, 2, ACC_I);
      if (NEXT) {
#pragma unroll
        for (int q = 0; q < ACC_I + ACC_J; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (ISSUE && q < 2 * LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    issue(0);
    __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
    __syncthreads();
    rd(fa[0], fb[0], 0, 0);
    if (1 < nk) issue(1);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) tile(kt, std::true_type{}, std::true_type{});
    if (kt + 1 < nk) {
      tile(kt, std::true_type{}, std::false_type{});
      ++kt;
    }
    tile(kt, std::false_type{}, std::false_type{});
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
        for (int j = 0; j < ACC_J; ++j) bv[j] = sb[acc_col(wn, j, lane & 15) * (BK + 1) + kk];
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int r = 0; r < ACC_R; ++r) {
            const float av = sa[acc_row(wm, i, r, lane >> 4) * (BK + 1) + kk];
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
    for (int j = 0; j < ACC_J; ++j) acc[i][j] = f32x4{};
  mainloop.run(acc, tm * GM, tn * GN, smem);
  epi(acc, tm * GM, tn * GN, smem);
}

}  // namespace stce
