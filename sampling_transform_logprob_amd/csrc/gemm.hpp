// Block-tiled matrix product for gfx950: C[m, n] = sum_k A[m, k] * B[n, k].
// Each operand is read either K-major (row-major along k) or MN-major
// (row-major along m or n, through transposing LDS reads; see the bf16 main
// loop below), so the products of the scoring core read their operands as
// they lie in memory:
//   projection   z^T[v, t] = W[v, :] . h[t, :]       (M = vocab, N = tokens, K = H; both K-major)
//   weight grad  dW[v, :] = dz^T[v, :] . h[:, :]     (M = vocab, N = H, K = tokens; h MN-major)
//   hidden grad  dH^T[:, t] = W^T[:, :] . dz^T[:, t] (M = H, N = tokens, K = vocab; dz^T MN-major,
//                                                     W^T a transposed copy)
// The fp32 main loop (16x16x4 fp32 matrix instruction) takes K-major operands only.
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
// bf16 main loop (MFMA).  Each operand is stored either K-major (X[r * ld + k],
// the form above) or MN-major (X[k * ld + r]: rows of the tile along k).  An
// MN-major operand spares the products of the backward a transposed copy:
// the weight gradient reads dz and h as they are, the hidden gradient reads W.
//
// MN-major tile in LDS: 64 k-rows of 512 bytes (256 rows of the operand).
// Its 32-byte chunks are XOR-permuted by f(k) = (k & 3) | ((k >> 3) & 1) << 2,
// applied on the global side of the LDS loads (lane l of a load writes bytes
// [16 l, 16 l + 16) of two consecutive k-rows).  Fragments come from the
// transposing LDS read ds_read_b64_tr_b16: within a 16-lane group, lane L
// receives element L % 4 of the 8-byte chunks addressed by lanes L / 4 + 4 j,
// j < 4.  Lane c of group g addresses k-row kk*32 + g*8 + 4 r + c / 4 at
// operand rows 4 (c % 4) .. +4 of the 16-row block, so lane L gets
// rows L, k-rows kk*32 + g*8 + 4 r .. +4; the reads r = 0, 1 make the 8
// k values of the MFMA operand.  Every 32 lanes of a read cover the 8 bank
// groups of 32 bytes once (no conflicts).  Each k-tile builds a fresh buffer
// resource at its first k-row, so offsets stay below 64 rows and rows past
// the operand's k extent read as zeros; rows past M (N) read values whose
// products land only in output rows the epilogues drop.
// ---------------------------------------------------------------------------
__device__ inline int mn_swz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// B_GATHER (K-major B only): B row r of the tile is row brow[r] of B (r < N),
// through one buffer resource over nrecB bytes of B (< 2^31 - 2^22, so row
// offsets and the tail sentinel stay in 32 bits): the tile recompute's
// gathered hidden rows.
template <bool A_MN, bool B_MN, bool B_GATHER = false>
struct MainBf16T {
  static constexpr int LDS_BYTES = 2 * 2 * GM * GK * 2;  // 2 stages x (A, B) x 32 KB
  static constexpr int ROWB = GK * 2;                     // 128-byte K-major tile rows
  static constexpr int MNROWB = GM * 2;                   // 512-byte MN-major tile rows
  static constexpr int TILEB = GM * ROWB;                 // one operand tile
  static constexpr int STAGEB = 2 * TILEB;
  static constexpr int LPW = 4;                           // 1 KB loads per wave per operand per k-tile
  // LDS reads per k-step of 32: a K-major fragment is one 16-byte read, an
  // MN-major one two transposing 8-byte reads
  static constexpr int NRD = (A_MN ? 2 : 1) * ACC_I + (B_MN ? 2 : 1) * ACC_J;
  const bf16* A;
  int64_t lda;
  int M;  // rows of A that exist
  const bf16* B;
  int64_t ldb;
  int N;
  int K;  // K-major operands: multiple of 8
  int ka = 0, kb = 0;  // MN-major operands: k-rows that exist (0: K); lda, ldb < 2^24
  const int* brow = nullptr;  // B_GATHER: the tile's B rows
  int nrecB = 0;              // B_GATHER: bytes of B

  // the same product over k-columns dk .. K of this one (split-K)
  __device__ inline void shift_k(int64_t dk) {
    A += A_MN ? dk * lda : dk;
    B += B_MN ? dk * ldb : dk;
    const int ka0 = ka ? ka : K, kb0 = kb ? kb : K;
    ka = max(ka0 - (int)dk, 0);
    kb = max(kb0 - (int)dk, 0);
    K -= (int)dk;
    if (ka == 0) ka = -1;  // nothing left (0 would mean "K")
    if (kb == 0) kb = -1;
  }

  // the same product over k-columns 0 .. k only (k > 0; a reduction length
  // known on the device)
  __device__ inline void limit_k(int k) {
    if (ka > 0) ka = min(ka, k);
    if (kb > 0) kb = min(kb, k);
    K = min(K, k);
  }

  // The two stages are distinct __shared__ objects (see the loop at the end
  // of run for why).  Stage 0 doubles as the epilogue's LDS (at most 64 KB),
  // so the product launches with no dynamic LDS.
  static constexpr int DYN_LDS = 0;
  static constexpr int EPI_LDS_MAX = STAGEB;
  __device__ static char* stage0() {
    __shared__ __attribute__((aligned(16))) char s0[STAGEB];
    return s0;
  }
  __device__ static char* stage1() {
    __shared__ __attribute__((aligned(16))) char s1[STAGEB];
    return s1;
  }
  // the epilogue's two LDS buffers (up to EPI_LDS_MAX bytes each): the stages
  __device__ static char* epilogue_lds(char*) { return stage0(); }
  __device__ static char* epilogue_lds1(char*) { return stage1(); }

  __device__ inline void run(AccTile& acc, int m0, int n0, char*) const {
    char* const S0 = stage0();
    char* const S1 = stage1();
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
    const int wm = w >> 2, wn = w & 3;
    const int kxa = ka ? ka : K, kxb = kb ? kb : K;
    // K-major: each resource spans only this tile's (at most 256) rows, so
    // offsets stay far below 2^31 and the tail sentinel below is always out
    // of range
    const int rowsA = min(M - m0, GM), rowsB = min(N - n0, GN);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * lda), (short)0,
                                                                        A_MN ? 0 : rowsA * (int)lda * 2, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rb =
        B_GATHER ? __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, nrecB, RSRC_WORD3)
                 : __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)n0 * ldb), (short)0,
                                                     B_MN ? 0 : rowsB * (int)ldb * 2, RSRC_WORD3);
    // K-major loads: instruction i of wave w fills rows (w*LPW + i)*8 .. +8
    // of a tile; lane l covers row + l/8 and physical chunk l%8, i.e.
    // logical chunk (l%8) ^ swz(row); the swizzle uses row bits 1..3, bit 3
    // being the parity of i
    const int lrow = lane >> 3, lpc = lane & 7;
    const int ce = lpc ^ lds_swz(lrow), co = lpc ^ lds_swz(lrow + 8);
    const int rA = (w * LPW * 8 + lrow) * (int)lda * 2, rB = (w * LPW * 8 + lrow) * (int)ldb * 2;
    const int stepA = 8 * (int)lda * 2, stepB = 8 * (int)ldb * 2;
    // B_GATHER: byte offset of each load's row (-1: past the tile's rows)
    int rBg[LPW];
    if constexpr (B_GATHER) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = n0 + w * LPW * 8 + i * 8 + lrow;
        rBg[i] = r < N ? brow[r] * (int)ldb * 2 : -1;
      }
    }
    // MN-major loads: instruction i of wave w fills k-rows (w*LPW + i)*2 .. +2;
    // lane l covers k-row + l/32, physical 32-byte chunk (l%32)/2, half l%2.
    // The swizzle of those rows depends on i only through its parity, so
    // instruction i takes the even or odd lane offset plus the scalar offset
    // of rows (i & ~1) * 2
    int mnoA[2], mnoB[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = (w * LPW + i) * 2 + (lane >> 5);
      const int col = ((((lane & 31) >> 1) ^ mn_swz(kr)) * 16 + (lane & 1) * 8) * 2;
      mnoA[i] = kr * (int)lda * 2 + col;
      mnoB[i] = kr * (int)ldb * 2 + col;
    }
    const int nk = (K + GK - 1) / GK;
    // loads of k-tile kt into stage kt % 2; K-major 16-byte chunks at or past
    // K get an offset beyond the buffer's range, which the hardware turns
    // into zeros
    auto issue = [&](int sg, int kt) __attribute__((always_inline)) {
      char* st = (sg ? S1 : S0) + w * LPW * 1024;
      const int k0 = kt * GK, so = k0 * 2;
      const bool ine = k0 + ce * 8 < K, ino = k0 + co * 8 < K;
      __amdgpu_buffer_rsrc_t rak = ra, rbk = rb;
      // (the record counts are wave-uniform; readfirstlane keeps the
      // resources in scalar registers)
      if constexpr (A_MN)
        rak = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(A + (int64_t)k0 * lda + m0), (short)0,
            __builtin_amdgcn_readfirstlane(max(min(GK, kxa - k0), 0) * (int)lda * 2), RSRC_WORD3);
      if constexpr (B_MN)
        rbk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(B + (int64_t)k0 * ldb + n0), (short)0,
            __builtin_amdgcn_readfirstlane(max(min(GK, kxb - k0), 0) * (int)ldb * 2), RSRC_WORD3);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const bool in = (i & 1) ? ino : ine;
        const int c16 = ((i & 1) ? co : ce) * 16;
        if constexpr (A_MN)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rak, STCE_LDS(st + i * 1024), 16, mnoA[i & 1],
                                                   (i & ~1) * 4 * (int)lda, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, STCE_LDS(st + i * 1024), 16,
                                                   in ? rA + i * stepA + c16 : 0x7ffffff0, so, 0, 0);
        if constexpr (B_MN)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rbk, STCE_LDS(st + TILEB + i * 1024), 16, mnoB[i & 1],
                                                   (i & ~1) * 4 * (int)ldb, 0, 0);
        else if constexpr (B_GATHER)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, STCE_LDS(st + TILEB + i * 1024), 16,
                                                   (in && rBg[i] >= 0) ? rBg[i] + c16 : 0x7ffffff0, so, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, STCE_LDS(st + TILEB + i * 1024), 16,
                                                   in ? rB + i * stepB + c16 : 0x7ffffff0, so, 0, 0);
      }
    };
    // K-major fragment of a 16 x 32 (rows x k) block: lane l reads row
    // l % 16, the 16-byte chunk l / 16 of the k-step's 32 columns
    const int frow = lane & 15, fq = lane >> 4, sw = lds_swz(frow);
    const int offA = (wm * 128 + frow) * ROWB, offB = TILEB + (wn * 64 + frow) * ROWB;
    // MN-major fragment: lane (g, c) = (lane / 16, lane % 16) reads k-row
    // g*8 + c/4 (+ 32 kk + 4 r) at chunk (block ^ f), byte 8 (c % 4)
    const int fz = (frow >> 2) | ((fq & 1) << 2);
    const int mnrow = (fq * 8 + (frow >> 2)) * MNROWB + (frow & 3) * 8;
    const int xbA = wm * 8, xbB = wn * 4;  // first 32-byte chunk of the wave's rows
    auto rd_mn = [&](const char* base, int x, int kk) __attribute__((always_inline)) {
      const char* p = base + mnrow + kk * 32 * MNROWB + ((x ^ fz) * 32);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)STCE_LDS(p));
      const s16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)STCE_LDS(p + 4 * MNROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 fa[2][ACC_I], fb[2][ACC_J];
    auto rd = [&](int sg, bf16x8 (&a)[ACC_I], bf16x8 (&b)[ACC_J], int kk) __attribute__((always_inline)) {
      const char* st = sg ? S1 : S0;
      const int ch = ((kk * 4 + fq) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < ACC_I; ++i) {
        if constexpr (A_MN)
          a[i] = rd_mn(st, xbA + i, kk);
        else
          a[i] = *(const bf16x8*)(st + offA + i * 16 * ROWB + ch);
      }
#pragma unroll
      for (int j = 0; j < ACC_J; ++j) {
        if constexpr (B_MN)
          b[j] = rd_mn(st + TILEB, xbB + j, kk);
        else
          b[j] = *(const bf16x8*)(st + offB + j * 16 * ROWB + ch);
      }
    };
    auto mma = [&](int cur, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
      for (int i = i0; i < i1; ++i)
#pragma unroll
        for (int j = 0; j < ACC_J; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    };
    // MFMAs per LDS read in the two interleaved stretches (24 MFMAs each,
    // then 8 more in the first), and the number of reads they interleave
    constexpr int P = NRD <= 12 ? 2 : 1;
    constexpr int Q = NRD < 24 / P ? NRD : 24 / P;
    // one k-tile, held in stage sg; NEXT: a tile follows (barrier + its
    // first fragments, from the other stage), ISSUE: the tile after that is
    // loaded into the stage this one frees
    auto tile = [&](int sg, int kt, auto next_c, auto issue_c) __attribute__((always_inline)) {
      constexpr bool NEXT = decltype(next_c)::value, ISSUE = decltype(issue_c)::value;
      rd(sg, fa[1], fb[1], 1);
      mma(0, 0, ACC_I);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, P, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, ACC_I * ACC_J - P * Q, 0);
      mma(1, 0, 2);
      __builtin_amdgcn_sched_barrier(0);
      if (NEXT) {
        // tile kt + 1 has landed (every wave waits for its own loads) and
        // every wave is done reading stage kt % 2 before it is refilled
        __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        rd(1 - sg, fa[0], fb[0], 0);
        if (ISSUE) issue(sg, kt + 2);
      }
      mma(1, 2, ACC_I);
      if (NEXT) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, P, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (ISSUE && q < 2 * LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        if constexpr ((ACC_I - 2) * ACC_J > P * Q)
          __builtin_amdgcn_sched_group_barrier(0x008, (ACC_I - 2) * ACC_J - P * Q, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    using T_ = std::true_type;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
    __syncthreads();
    rd(0, fa[0], fb[0], 0);
    // An even number of k-tiles (an odd count gets one more, all zeros: its
    // loads fall past K), so that tile kt's stage kt % 2 is a constant at
    // every read and load.  The compiler then sees that the transposing reads
    // of one stage do not alias the loads in flight into the other and adds
    // no wait for them; K-major operands gain too (3% at K = 5120, measured
    // against a single-tile loop with the stage chosen at run time).  Every
    // pair runs the steady-state form: the last pair's loads (two tiles past
    // the end) fall past K and fill stages nobody reads with zeros, and its
    // last barrier reads fragments nobody uses, so there is no tail code
    // whose addresses would stay live across the loop.  The barrier after
    // the loop waits for those loads before the epilogue reuses the stages.
    const int nk2 = (nk + 1) & ~1;
    issue(1, 1);
    for (int kt = 0; kt < nk2; kt += 2) {
      tile(0, kt, T_{}, T_{});
      tile(1, kt + 1, T_{}, T_{});
    }
    __syncthreads();  // the epilogue may reuse the LDS
  }
};
using MainBf16 = MainBf16T<false, false>;
using MainBf16G = MainBf16T<false, false, true>;

// ---------------------------------------------------------------------------
// fp8 main loop (MFMA): e4m3 operands, both K-major, C[m, n] = sum_k A[m, k]
// B[n, k] with the 16x16x128 fp8 matrix instruction (twice the bf16 rate).
// A k-tile is 128 elements = 128 bytes of a row, the bf16 loop's tile row
// size, so the loads, the LDS layout and its swizzle are the bf16 loop's; a
// k-tile is one k-step, whose fragment per 16-row block is 32 bytes a lane
// (chunks 2q and 2q + 1 of the row, q = lane / 16).  Both operands take the
// same byte-to-lane mapping, so every product pairs equal k.  The 32 MFMAs
// of a k-tile (each 4 times the work of a bf16 16x16x32) cover the next
// tile's fragment reads of the other wave of the SIMD; the loads of tile
// kt + 2 go out right after the barrier that frees the stage of tile kt.
// K (bytes) is a multiple of 16; chunks past K read as zeros.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <bool B_GATHER = false>
struct MainFp8T {
  static constexpr int ROWB = 128;
  static constexpr int TILEB = GM * ROWB;
  static constexpr int STAGEB = 2 * TILEB;
  static constexpr int LPW = 4;
  static constexpr int DYN_LDS = 0;
  static constexpr int EPI_LDS_MAX = STAGEB;
  const uint8_t* A;
  int64_t lda;  // bytes
  int M;
  const uint8_t* B;
  int64_t ldb;
  int N;
  int K;        // bytes (elements)
  const int* brow = nullptr;  // B_GATHER: the tile's B rows (as MainBf16T)
  int nrecB = 0;              // B_GATHER: bytes of B

  __device__ inline void limit_k(int k) { K = min(K, k); }
  __device__ static char* stage0() { return MainBf16::stage0(); }
  __device__ static char* stage1() { return MainBf16::stage1(); }
  __device__ static char* epilogue_lds(char*) { return stage0(); }
  __device__ static char* epilogue_lds1(char*) { return stage1(); }

  __device__ inline void run(AccTile& acc, int m0, int n0, char*) const {
    char* const S0 = stage0();
    char* const S1 = stage1();
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 2, wn = w & 3;
    const int rowsA = min(M - m0, GM), rowsB = min(N - n0, GN);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * lda), (short)0, rowsA * (int)lda, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rb =
        B_GATHER ? __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, nrecB, RSRC_WORD3)
                 : __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)n0 * ldb), (short)0, rowsB * (int)ldb,
                                                     RSRC_WORD3);
    const int lrow = lane >> 3, lpc = lane & 7;
    const int ce = lpc ^ lds_swz(lrow), co = lpc ^ lds_swz(lrow + 8);
    const int rA = (w * LPW * 8 + lrow) * (int)lda, rB = (w * LPW * 8 + lrow) * (int)ldb;
    const int stepA = 8 * (int)lda, stepB = 8 * (int)ldb;
    int rBg[LPW];
    if constexpr (B_GATHER) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = n0 + w * LPW * 8 + i * 8 + lrow;
        rBg[i] = r < N ? brow[r] * (int)ldb : -1;
      }
    }
    const int nk = (K + ROWB - 1) / ROWB;
    auto issue = [&](int sg, int kt) __attribute__((always_inline)) {
      char* st = (sg ? S1 : S0) + w * LPW * 1024;
      const int k0 = kt * ROWB;
      const bool ine = k0 + ce * 16 < K, ino = k0 + co * 16 < K;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const bool in = (i & 1) ? ino : ine;
        const int c16 = ((i & 1) ? co : ce) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, STCE_LDS(st + i * 1024), 16, in ? rA + i * stepA + c16 : 0x7ffffff0,
                                                 k0, 0, 0);
        if constexpr (B_GATHER)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, STCE_LDS(st + TILEB + i * 1024), 16,
                                                   (in && rBg[i] >= 0) ? rBg[i] + c16 : 0x7ffffff0, k0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, STCE_LDS(st + TILEB + i * 1024), 16,
                                                   in ? rB + i * stepB + c16 : 0x7ffffff0, k0, 0, 0);
      }
    };
    const int frow = lane & 15, fq = lane >> 4, sw = lds_swz(frow);
    const int offA = (wm * 128 + frow) * ROWB, offB = TILEB + (wn * 64 + frow) * ROWB;
    const int c0 = ((2 * fq) ^ sw) * 16, c1 = ((2 * fq + 1) ^ sw) * 16;
    auto frag = [&](const char* base) __attribute__((always_inline)) {
      const u32x4 lo = *(const u32x4*)(base + c0), hi = *(const u32x4*)(base + c1);
      return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // Fragments: B's four of a tile double-buffered by stage (fb[sg]); A's
    // eight through a ring of four, read three ahead (A fragment i of a tile
    // in slot i % 4, so every slot index is a compile-time constant).  A
    // k-tile: before MFMA block i (four MFMAs), A fragment i + 3 is read;
    // fragments 8.. are the next tile's, in the other stage, so the barrier
    // sits before block 5, once every read of this stage has landed (A
    // fragment 7 was read before block 4) and this wave's loads of the next
    // tile are in.  After it the freed stage is refilled with tile kt + 2 and
    // the next tile's B fragments and A fragments 0..2 are read while blocks
    // 5..7 (12 MFMAs) run.
    i32x8 fb[2][ACC_J], fa[4];
    auto rdA = [&](const char* st, int i) __attribute__((always_inline)) {
      return frag(st + offA + i * 16 * ROWB);
    };
    auto mma = [&](const i32x8& a, const i32x8 (&b)[ACC_J], int i) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < ACC_J; ++j)
        // (constant zero scale operands: the compiler emits the unscaled
        // v_mfma_f32_16x16x128_f8f6f4, plain e4m3 products, 1% faster here
        // than the scaled form with unit scales)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    };
    auto tile = [&](auto sg_c, int kt) __attribute__((always_inline)) {
      constexpr int sg = decltype(sg_c)::value;
      const char* st = sg ? S1 : S0;
      const char* nx = sg ? S0 : S1;
#pragma unroll
      for (int i = 0; i < ACC_I; ++i) {
        if (i == 5) {
          __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
          __syncthreads();
          __builtin_amdgcn_sched_barrier(0);
          issue(sg, kt + 2);
#pragma unroll
          for (int j = 0; j < ACC_J; ++j) fb[1 - sg][j] = frag(nx + offB + j * 16 * ROWB);
        }
        if (i + 3 < ACC_I)
          fa[(i + 3) & 3] = rdA(st, i + 3);
        else
          fa[(i + 3) & 3] = rdA(nx, i + 3 - ACC_I);
        mma(fa[i & 3], fb[sg], i);
        if (i == 4) {
          // blocks 0..4: one A read (16 bytes) after every two MFMAs, so
          // no read sits next to the MFMA that consumes it
#pragma unroll
          for (int q = 0; q < 10; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // blocks 5..7: the next tile's 14 fragment reads and the 8 loads of
      // tile kt + 2 between the 12 MFMAs
#pragma unroll
      for (int q = 0; q < 12; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (q < 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (q < 2 * LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global->LDS load
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    issue(0, 0);
    issue(1, 1);
    __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) fb[0][j] = frag(S0 + offB + j * 16 * ROWB);
    // (in the loop's order, B then A 0, 1, 2, so that the wait at the
    // loop's head is for B and A fragment 0 only)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      fa[i] = rdA(S0, i);
    }
    __builtin_amdgcn_sched_barrier(0);
    // an even number of k-tiles (an odd count gets one all-zero tile) so that
    // every read and load names its stage at compile time; the last pair's
    // loads and next-tile reads fall past K or read a stage nobody uses
    const int nk2 = (nk + 1) & ~1;
    using Z_ = std::integral_constant<int, 0>;
    using O_ = std::integral_constant<int, 1>;
    for (int kt = 0; kt < nk2; kt += 2) {
      tile(Z_{}, kt);
      tile(O_{}, kt + 1);
    }
    __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
    __syncthreads();  // the epilogue may reuse the LDS
  }
};

using MainFp8 = MainFp8T<false>;
using MainFp8G = MainFp8T<true>;

// ---------------------------------------------------------------------------
// fp32 main loop (MFMA): fp32 operands, both K-major, on the 16x16x4 fp32
// matrix instruction, same accumulator layout as the bf16 loop.  A k-slab of
// BK = 16 columns goes through registers into LDS rows of 20 floats (80
// bytes: 16-byte aligned, and the 16 rows of a fragment read fall on 16
// distinct groups of four banks).  Lane l of a wave reads the four
// consecutive columns 4 (l / 16) .. +4 of its fragment row with one 16-byte
// read; matrix step s (s < 4) of the slab then multiplies column 4 g + s of
// lane group g = l / 16, which the instruction takes as its k index g.  So an
// output element sums its k terms four per instruction, in an order fixed by
// k alone (every tile position, chunk and launch gives the same bits).
// K is a multiple of 4; columns at or past K read as zeros, rows past M (N)
// repeat the last row (their outputs are dropped by the epilogues).
// ---------------------------------------------------------------------------
struct MainF32 {
  static constexpr int BK = 16;
  static constexpr int LDR = 20;  // floats per LDS row
  static constexpr int LDS_BYTES = 2 * GM * LDR * 4;
  static constexpr int DYN_LDS = LDS_BYTES;  // dynamic LDS, shared with the epilogue
  static constexpr int EPI_LDS_MAX = 160 * 1024;
  // one epilogue LDS buffer, shared with the main loop (no second one)
  __device__ static char* epilogue_lds(char* dyn) { return dyn; }
  __device__ static char* epilogue_lds1(char*) { return nullptr; }
  const float* A;
  int64_t lda;
  int M;
  const float* B;
  int64_t ldb;
  int N;
  int K;  // multiple of 4

  // the same product over k-columns dk .. K of this one (split-K)
  __device__ inline void shift_k(int64_t dk) {
    A += dk;
    B += dk;
    K -= (int)dk;
  }
  __device__ inline void limit_k(int k) { K = min(K, k); }

  __device__ inline void run(AccTile& acc, int m0, int n0, char* smem) const {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3;
    float* sa = (float*)smem;  // [256][LDR]
    float* sb = sa + GM * LDR;  // [256][LDR]
    // thread t loads half a row: row t / 2, columns (t & 1) * 8 .. + 8
    const int lr = tid >> 1, lc = (tid & 1) * 8;
    const float* ga = A + (int64_t)min(m0 + lr, M - 1) * lda + lc;
    const float* gb = B + (int64_t)min(n0 + lr, N - 1) * ldb + lc;
    // fragment reads: row lane % 16 of each 16-row block, columns 4 (lane / 16) .. +4
    const float* fra = sa + (wm * 128 + (lane & 15)) * LDR + 4 * (lane >> 4);
    const float* frb = sb + (wn * 64 + (lane & 15)) * LDR + 4 * (lane >> 4);
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
      for (int c = 0; c < 8; c += 4) {
        const bool in = k0 + lc + c < K;
        const f32x4 va = in ? *(const f32x4*)(ga + k0 + c) : f32x4{0, 0, 0, 0};
        const f32x4 vb = in ? *(const f32x4*)(gb + k0 + c) : f32x4{0, 0, 0, 0};
        *(f32x4*)(sa + lr * LDR + lc + c) = va;
        *(f32x4*)(sb + lr * LDR + lc + c) = vb;
      }
      __syncthreads();
      f32x4 fa[ACC_I], fb[ACC_J];
#pragma unroll
      for (int i = 0; i < ACC_I; ++i) fa[i] = *(const f32x4*)(fra + i * 16 * LDR);
#pragma unroll
      for (int j = 0; j < ACC_J; ++j) fb[j] = *(const f32x4*)(frb + j * 16 * LDR);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < ACC_I; ++i)
#pragma unroll
          for (int j = 0; j < ACC_J; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i][st], fb[j][st], acc[i][j], 0, 0, 0);
      __syncthreads();
    }
  }
};

// Dynamic LDS of a product: the main loop's when it takes dynamic LDS (the
// epilogue then shares it), else the epilogue reuses the main loop's stage 0.
template <class Main, class Epi>
constexpr int gemm_dyn_lds() {
  static_assert(Epi::LDS_BYTES <= Main::EPI_LDS_MAX, "epilogue LDS exceeds what the main loop leaves it");
  return Main::DYN_LDS ? (Main::DYN_LDS > Epi::LDS_BYTES ? Main::DYN_LDS : Epi::LDS_BYTES) : 0;
}

// Extents of a product known only on the device (counts a previous kernel
// wrote): output tiles whose first column reaches *n_lim do nothing, and the
// reduction runs over k-columns 0 .. *k_lim (no tile does anything when it
// is 0).  Null pointers: the launch's own extents.
struct DynLimits {
  const int* n_lim = nullptr;
  const int* k_lim = nullptr;
};

// Holds every 32-bit word of a kernel argument in scalar registers from this
// point on, so the argument's scalar loads have completed here.  Scalar-cache
// loads share the LDS wait counter but complete out of order: while one is in
// flight, a wait for an LDS read can only be a wait for everything.  With the
// epilogue's argument loads still in flight at the main loop, the compiler
// makes the loop's first fragment wait (at every iteration) a wait for all of
// the previous tile's reads.
template <int N>
struct ArgWords {
  uint32_t w[N];
};
template <class T>
__device__ inline void hold_in_sgprs(const T& x) {
  static_assert(sizeof(T) % 4 == 0, "argument of whole words");
  const auto a = __builtin_bit_cast(ArgWords<sizeof(T) / 4>, x);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"s"(a.w[i]));
}

template <class Main, class Epi>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_kernel(Main mainloop, Epi epi, TileMap map, DynLimits dyn) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int tm, tn;
  map.get(blockIdx.x, tm, tn);
  if (dyn.n_lim && tn * GN >= *dyn.n_lim) return;
  if (dyn.k_lim) {
    const int k = *dyn.k_lim;
    if (k <= 0) return;
    mainloop.limit_k(k);
  }
  AccTile acc;
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int j = 0; j < ACC_J; ++j) acc[i][j] = f32x4{};
  hold_in_sgprs(epi);
  mainloop.run(acc, tm * GM, tn * GN, smem);
  epi(acc, tm * GM, tn * GN, Main::epilogue_lds(smem), Main::epilogue_lds1(smem));
}

// A product over work items whose B rows are gathered: A tile j (rows j GM ..)
// pairs with the B rows listed for it, GN at a time.  woff: exclusive scan of
// the tiles' work-item counts (woff[ntiles] = the total); item w of tile j
// takes rows[boff[j] + (w - woff[j]) GN ..] up to cnt[j] rows.  Workgroups
// past the total return at once (the grid is sized for the most items).
struct WorkList {
  const int* woff;   // [ntiles + 1]
  const int* cnt;    // [ntiles]
  const int* boff;   // [ntiles]
  const int* rows;
  int ntiles;
};

template <class Main, class Epi>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_worklist_kernel(Main mainloop, Epi epi, WorkList wl) {
  const int w = blockIdx.x;
  if (w >= wl.woff[wl.ntiles]) return;
  int lo = 0, hi = wl.ntiles - 1;  // the largest j with woff[j] <= w
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wl.woff[mid] <= w)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int j = lo, it = w - wl.woff[j];
  const int* rows = wl.rows + wl.boff[j] + it * GN;
  const int ncol = min(GN, wl.cnt[j] - it * GN);
  mainloop.brow = rows;
  mainloop.N = ncol;
  epi.colpos = rows;
  epi.ncols = ncol;
  AccTile acc;
#pragma unroll
  for (int i = 0; i < ACC_I; ++i)
#pragma unroll
    for (int jj = 0; jj < ACC_J; ++jj) acc[i][jj] = f32x4{};
  hold_in_sgprs(epi);
  mainloop.run(acc, j * GM, 0, nullptr);
  epi(acc, j * GM, 0, Main::epilogue_lds(nullptr), Main::epilogue_lds1(nullptr));
}

}  // namespace stce
