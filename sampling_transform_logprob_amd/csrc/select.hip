// Support program + selected logprob, one workgroup of 256 threads per row.
// The algorithm is described in select.hpp.
#include "kernels.hpp"
#include "select.hpp"

namespace stce {
namespace {

// The selected logprob in the lane's dtype: the fp32 value, or its bf16
// rounding (nearest, ties to even) in the bf16 value lane.
__device__ inline float lane_logprob(const SelParams& P, float lp) {
  return P.round_lp_bf16 ? (float)(bf16)lp : lp;
}


#define F_INF __builtin_huge_valf()
#define D_INF __builtin_huge_val()

struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct MinF { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct AddD { __device__ double operator()(double a, double b) const { return a + b; } };
struct MinI { __device__ int operator()(int a, int b) const { return min(a, b); } };
struct MaxI { __device__ int operator()(int a, int b) const { return max(a, b); } };

// Deterministic block reduction: xor butterfly inside each wave (every lane
// ends with the same value since each step combines a commutative pair),
// then waves 0..3 in order.  All threads must call it.
template <class T, class Op>
__device__ inline T block_reduce(T v, Op op, T* scratch) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T r = scratch[0];
#pragma unroll
  for (int i = 1; i < ST / 64; ++i) r = op(r, scratch[i]);
  return r;
}

// Exclusive prefix sum of one double per thread (thread order).
__device__ inline double block_excl_scan(double v, double* scratch) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  double ex = __shfl_up(x, 1);
  if (lane == 0) ex = 0.0;
  __syncthreads();
  if (lane == 63) scratch[w] = x;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += scratch[i];
  return off + ex;
}

// Bitonic sort, descending, of x[0, n) for any n: the network of the next
// power of two in the form where every compare-exchange puts the larger value
// at the lower index (each merge starts with a mirrored half-cleaner).
// Positions >= n stand for minimum values that never move, so they are
// neither read nor written.
template <class T>
__device__ inline void bitonic_desc(T* x, int n) {
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int size = 2; size <= n2; size <<= 1) {
    const int half = size >> 1;
    for (int i = threadIdx.x; i < (n2 >> 1); i += ST) {
      const int base = (i / half) * size, off = i % half;
      const int lo = base + off, hi = base + size - 1 - off;
      if (hi < n) {
        const T a = x[lo], b = x[hi];
        if (a < b) {
          x[lo] = b;
          x[hi] = a;
        }
      }
    }
    __syncthreads();
    for (int stride = half >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n2 >> 1); i += ST) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        if (hi < n) {
          const T a = x[lo], b = x[hi];
          if (a < b) {
            x[lo] = b;
            x[hi] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

constexpr int TLIST = 512;  // candidate-tile list capacity

struct Shared {
  union {
    uint64_t cand[CAP];
    uint32_t k32[2 * CAP];
    struct {
      uint32_t cnt[ST / 64][NB];
      double mass[ST / 64][NB];
    } h;
  } u;
  double sd[ST / 64];
  float sf[ST / 64];
  int si[ST / 64];
  uint32_t tiles[TLIST];   // vocabulary tiles that can hold window tokens (V < 2^31: up to 2^23 tiles)
  int ntiles;
  uint32_t bkey;
  double mass_o;           // mass of the first n_other window tokens
  int cnt;
  int c;             // chosen bin
  int c_p;           // bin where top-p crosses (NB if not found)
  uint32_t nbin;     // tokens in the chosen bin
  int fail;          // the row's candidates cannot decide its support
  uint32_t above;    // tokens ahead of the window
  double mabove;     // their mass
  double Z;          // full-row mass
  double mass_s;     // mass of the support
};

// The projection's two LDS stages take 128 KB of a compute unit's 160 KB, so
// a selection workgroup fits beside a projection workgroup only within 32 KB.
static_assert(sizeof(Shared) <= 32 * 1024, "selection LDS must fit beside a projection workgroup");

// A row with no support list: all of its entries zero, so that the state's
// bytes are a function of the inputs.
__device__ inline void clear_support(const SelParams& P, int orow) {
  if (!P.support) return;
  for (int i = threadIdx.x; i < NSP; i += ST) P.support[orow].e[i] = SpEntry{0, 0.0f};
}

// At most 96 VGPRs (5 waves per SIMD): one of these waves fits beside the
// two projection waves of a SIMD.
__global__ __launch_bounds__(ST, 5) void select_kernel(SelParams P) {
  __shared__ Shared S;
  // row: where the keys, partials and target key are; orow: whose metadata
  // and outputs (the same row unless re-selecting chosen rows)
  const int row = blockIdx.x, tid = threadIdx.x, w = tid >> 6;
  if (P.n_dev && row >= *P.n_dev) return;
  const int orow = P.rowmap ? P.rowmap[row] : row;
  const int V = P.V;
  const uint32_t fl = P.flags[orow];
  if (!(fl & ROW_VALID)) {
    clear_support(P, orow);
    if (tid == 0) {
      const float nan = __builtin_nanf("");
      P.logprob[orow] = nan;
      RowState rs{};
      P.state[orow] = rs;
      if (P.tiles) P.tiles[orow] = RowTiles{};
      if (P.lse_full) P.lse_full[orow] = nan;
      if (P.ent_full) P.ent_full[orow] = nan;
      if (P.ent_supp) P.ent_supp[orow] = nan;
    }
    return;
  }
  // a top-k row whose keys were not stored: its support comes from the
  // projection's candidates, or the row is handed to the re-projection
  const bool cand = P.ckey && (fl & ROW_CAND);
  auto fail_row = [&]() {
    if (tid == 0) P.fail_rows[atomicAdd(P.fail_cnt, 1)] = row;
  };

  // ---- row maximum, minimum and full log-sum-exp from the tile partials
  const TilePart* pp = P.part + (int64_t)row * P.ntv;
  float mx = -F_INF, mn = F_INF;
  for (int t = tid; t < P.ntv; t += ST) {
    mx = fmaxf(mx, pp[t].mx);
    mn = fminf(mn, pp[t].mn);
  }
  const float m = block_reduce(mx, MaxF{}, S.sf);
  const float smin = block_reduce(mn, MinF{}, S.sf);
  const double m64 = (double)m;
  double zs = 0.0;
  for (int t = tid; t < P.ntv; t += ST) zs += (double)pp[t].sum * exp((double)pp[t].mx - m64);
  const double zfull = block_reduce(zs, AddD{}, S.sd);
  const double lse_full = m64 + log(zfull);
  // entropy of softmax(s) over the row from the tiles' sums of
  // e^(s - mx) (s - mx): sum_j e^(s_j - m) (s_j - m) re-bases each tile on m
  const bool want_ent = P.ent_full || P.ent_supp;
  double h_full = 0.0;
  if (want_ent) {
    double es = 0.0;
    for (int t = tid; t < P.ntv; t += ST) {
      const double d = (double)pp[t].mx - m64;
      if (pp[t].mx != -F_INF) es += exp(d) * ((double)pp[t].ent + d * (double)pp[t].sum);
    }
    h_full = log(zfull) - block_reduce(es, AddD{}, S.sd) / zfull;
    if (tid == 0 && P.ent_full) P.ent_full[orow] = (float)h_full;
  }
  if (tid == 0 && P.lse_full) P.lse_full[orow] = (float)lse_full;

  // an inactive row's target is no token, so the projection left no key
  // for it: its state records 0
  const float sy = (fl & ROW_IGNORED) ? 0.0f : P.s_y[row];
  const int64_t y = P.target[orow];
  RowState rs;
  rs.m = m;
  rs.lse_full = (float)lse_full;
  rs.s_y = sy;

  if (!(fl & ROW_FILTERED)) {  // identity program: the support is the whole row
    clear_support(P, orow);
    if (tid == 0) {
      rs.key_thr = 0u;
      rs.id_thr = V - 1;
      rs.n = V;
      rs.flags = ROW_VALID | ROW_IN_SUPPORT;
      rs.lse_s = rs.lse_full;
      if (fl & ROW_IGNORED) rs.flags = ROW_VALID | ROW_IGNORED;
      P.logprob[orow] = lane_logprob(P, (fl & ROW_IGNORED) ? 0.0f : (float)fmin((double)sy - lse_full, 0.0));
      P.state[orow] = rs;
      if (P.tiles) P.tiles[orow] = RowTiles{};
      if (P.ent_supp) P.ent_supp[orow] = (float)h_full;
    }
    return;
  }

  const int k = P.top_k ? P.top_k[orow] : 0;
  const float p = P.top_p ? P.top_p[orow] : 1.0f;
  const float mp = P.min_p ? P.min_p[orow] : 0.0f;
  const bool k_on = k > 0 && k < V, p_on = p < 1.0f, m_on = mp > 0.0f;
  const double thr = m_on ? log((double)mp) : -D_INF;
  const float* rp = P.tile + (int64_t)row * P.ld;
  const int nv4 = (V + 3) >> 2;

  // One pass over the row: gathers the tokens `pred` accepts into the window
  // (up to CAP) and, if want_z, sums the fp64 masses of the whole row.
  auto collect = [&](auto pred, bool want_z, double& Z) -> int {
    if (tid == 0) S.cnt = 0;
    __syncthreads();
    double zl = 0.0;
    for (int q = tid; q < nv4; q += ST) {
      const f32x4 x = *(const f32x4*)(rp + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * q + e;
        if (v < V) {
          const float s = x[e];
          if (want_z) zl += exp((double)s - m64);
          const uint32_t key = order_key(s);
          if (pred(s, key, v)) {
            const int i = atomicAdd(&S.cnt, 1);
            if (i < CAP) S.u.cand[i] = composite(key, (uint32_t)v);
          }
        }
      }
    }
    Z = want_z ? block_reduce(zl, AddD{}, S.sd) : 0.0;
    __syncthreads();
    return S.cnt;
  };

  // Full-row mass relative to m from the fp32 tile partials: within 1e-4
  // relative of the exact value (each exp carries ~|x| 2^-24 relative error,
  // each 256-term fp32 sum at most 256 ulps), used only to certify that
  // top-p cannot bind before another filter does.
  const double z32 = exp(lse_full - m64);

  int nw = -1;              // window size; -1 until a window is found
  uint32_t above = 0;       // tokens ahead of the window in the order
  double mabove = 0.0;      // their fp64 mass
  double Z = 0.0;           // full-row fp64 mass (top-p only)
  int zmode = 0;            // 0: Z exact; 1: Z = window total; 2: only z32 known
  bool p_here = false;      // top-p is known to cross inside the window

  if (V <= CAP) {
    double dummy;
    nw = collect([](float, uint32_t, int) { return true; }, false, dummy);
    zmode = 1;
    p_here = p_on;
  } else {
    // lower bound of the k-th largest key: the k-th largest tile maximum
    // (the tile maxima are distinct tokens), found bit by bit by wave 0
    bool kb = false;
    if (k_on && k <= P.ntv && P.ntv <= 2 * CAP) {
      for (int t = tid; t < P.ntv; t += ST) S.u.k32[t] = order_key(pp[t].mx);
      __syncthreads();
      if (w == 0) {
        const int lane = tid & 63;
        uint32_t tau = 0u;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t c = tau | (1u << bit);
          int cnt = 0;
          for (int t = lane; t < P.ntv; t += 64) cnt += S.u.k32[t] >= c ? 1 : 0;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
          if (cnt >= k) tau = c;
        }
        if (lane == 0) S.bkey = tau;
      }
      kb = true;
      __syncthreads();
    }
    const uint32_t bkey = kb ? S.bkey : 0u;
    if (kb || m_on) {
      // tiles whose maximum passes the bound can hold window tokens
      if (tid == 0) S.ntiles = 0;
      __syncthreads();
      for (int t = tid; t < P.ntv; t += ST) {
        const float tm = pp[t].mx;
        if ((!kb || order_key(tm) >= bkey) && (!m_on || (double)tm - m64 >= thr)) {
          const int i = atomicAdd(&S.ntiles, 1);
          if (i < TLIST) S.tiles[i] = (uint32_t)t;
        }
      }
      __syncthreads();
      const int nt = S.ntiles;
      auto pred = [&](float s, uint32_t key, int) { return (!kb || key >= bkey) && (!m_on || (double)s - m64 >= thr); };
      int n;
      if (cand) {
        // the candidates of the candidate tiles; every token at or above the
        // bound is among them when each tile's largest non-candidate key is
        // below it (ROW_CAND rows always have the bound: kb)
        if (tid == 0) {
          S.cnt = 0;
          S.fail = nt > TLIST;
        }
        __syncthreads();
        const int ntl = min(nt, TLIST);
        for (int q = tid; q < ntl; q += ST)
          if (order_key(P.cbound[(int64_t)row * P.ntv + S.tiles[q]]) >= bkey) S.fail = 1;
        for (int q = tid; q < ntl * 16; q += ST) {
          const int t = (int)S.tiles[q >> 4], e = q & 15;
          const int64_t rec = ((int64_t)t * 2 + (e >> 3)) * P.cld + row;
          const float sv = P.ckey[rec * 8 + (e & 7)];
          const int v = t * VTILE + P.cid[rec * 8 + (e & 7)];
          const uint32_t key = order_key(sv);
          if (v < V && pred(sv, key, v)) {
            const int i = atomicAdd(&S.cnt, 1);
            if (i < CAP) S.u.cand[i] = composite(key, (uint32_t)v);
          }
        }
        __syncthreads();
        n = S.fail ? CAP + 1 : S.cnt;
        __syncthreads();
      } else if (nt <= TLIST) {
        if (tid == 0) S.cnt = 0;
        __syncthreads();
        for (int q = tid; q < nt * (VTILE / 4); q += ST) {
          const int v0 = (int)S.tiles[q / (VTILE / 4)] * VTILE + (q % (VTILE / 4)) * 4;
          if (v0 >= V) continue;
          const f32x4 x = *(const f32x4*)(rp + v0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = v0 + e;
            if (v < V) {
              const float sv = x[e];
              const uint32_t key = order_key(sv);
              if (pred(sv, key, v)) {
                const int i = atomicAdd(&S.cnt, 1);
                if (i < CAP) S.u.cand[i] = composite(key, (uint32_t)v);
              }
            }
          }
        }
        __syncthreads();
        n = S.cnt;
        __syncthreads();
      } else {
        double dummy;
        n = collect(pred, false, dummy);
      }
      if (n <= CAP) {
        nw = n;
        zmode = 2;
      }
    }
  }

  if (nw < 0 && cand) {  // no bounded window from the candidates
    fail_row();
    return;
  }
  if (nw < 0) {
    // ---- value histogram of (m - s): counts and fp64 masses per bin
    const float range = m - smin;
    const float scale = (range > 1e-30f && range < 3.0e38f) ? (float)NB / range : 0.0f;
    auto vbin = [&](float s) -> int {
      const float d = (m - s) * scale;
      return d >= (float)(NB - 1) ? NB - 1 : (d > 0.0f ? (int)d : 0);
    };
    for (int b = tid; b < (ST / 64) * NB; b += ST) {
      S.u.h.cnt[b / NB][b % NB] = 0u;
      S.u.h.mass[b / NB][b % NB] = 0.0;
    }
    __syncthreads();
    int cm_loc = -1;
    for (int q = tid; q < nv4; q += ST) {
      const f32x4 x = *(const f32x4*)(rp + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * q + e;
        if (v < V) {
          const float s = x[e];
          const int b = vbin(s);
          const double dm = (double)s - m64;
          atomicAdd(&S.u.h.cnt[w][b], 1u);
          atomicAdd(&S.u.h.mass[w][b], exp(dm));
          if (m_on && dm >= thr) cm_loc = max(cm_loc, b);
        }
      }
    }
    const int cm = m_on ? block_reduce(cm_loc, MaxI{}, S.si) : NB;
    __syncthreads();
    for (int b = tid; b < NB; b += ST) {
      uint32_t c = S.u.h.cnt[0][b];
      double ms = S.u.h.mass[0][b];
      for (int i = 1; i < ST / 64; ++i) {
        c += S.u.h.cnt[i][b];
        ms += S.u.h.mass[i][b];
      }
      S.u.h.cnt[0][b] = c;
      S.u.h.mass[0][b] = ms;
    }
    __syncthreads();
    if (tid == 0) {
      double Zt = 0.0;
      for (int b = 0; b < NB; ++b) Zt += S.u.h.mass[0][b];
      const double pz = (double)p * Zt;
      uint32_t cc = 0;
      double cms = 0.0;
      int ck = NB, cp = NB;
      for (int b = 0; b < NB; ++b) {
        cc += S.u.h.cnt[0][b];
        cms += S.u.h.mass[0][b];
        if (k_on && ck == NB && cc >= (uint32_t)k) ck = b;
        if (p_on && cp == NB && cms >= pz) cp = b;
      }
      const int c = min(min(ck, cp), cm);
      uint32_t ab = 0;
      double mab = 0.0;
      for (int b = 0; b < c; ++b) {
        ab += S.u.h.cnt[0][b];
        mab += S.u.h.mass[0][b];
      }
      S.c = c;
      S.c_p = cp;
      S.nbin = S.u.h.cnt[0][c];
      S.above = ab;
      S.mabove = mab;
      S.Z = Zt;
    }
    __syncthreads();
    const int c = S.c;
    above = S.above;
    mabove = S.mabove;
    Z = S.Z;
    p_here = p_on && S.c_p == c;
    const uint32_t nbin = S.nbin;
    __syncthreads();

    if (nbin <= (uint32_t)CAP) {
      double dummy;
      nw = collect([&](float s, uint32_t, int) { return vbin(s) == c; }, false, dummy);
    } else {
      // ---- radix refinement of bin c on the composite (key, ~id)
      uint64_t prefix = 0, pmask = 0;
      for (int shift = 56;; shift -= 8) {
        for (int b = tid; b < (ST / 64) * RB; b += ST) {
          S.u.h.cnt[b / RB][b % RB] = 0u;
          S.u.h.mass[b / RB][b % RB] = 0.0;
        }
        __syncthreads();
        int cml = -1;
        for (int q = tid; q < nv4; q += ST) {
          const f32x4 x = *(const f32x4*)(rp + 4 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * q + e;
            if (v < V) {
              const float s = x[e];
              if (vbin(s) != c) continue;
              const uint64_t comp = composite(order_key(s), (uint32_t)v);
              if ((comp & pmask) != prefix) continue;
              const int b = 255 - (int)((comp >> shift) & 255u);
              const double dm = (double)s - m64;
              atomicAdd(&S.u.h.cnt[w][b], 1u);
              atomicAdd(&S.u.h.mass[w][b], exp(dm));
              if (m_on && dm >= thr) cml = max(cml, b);
            }
          }
        }
        const int cm2 = m_on ? block_reduce(cml, MaxI{}, S.si) : RB;
        __syncthreads();
        for (int b = tid; b < RB; b += ST) {
          uint32_t cc = S.u.h.cnt[0][b];
          double ms = S.u.h.mass[0][b];
          for (int i = 1; i < ST / 64; ++i) {
            cc += S.u.h.cnt[i][b];
            ms += S.u.h.mass[i][b];
          }
          S.u.h.cnt[0][b] = cc;
          S.u.h.mass[0][b] = ms;
        }
        __syncthreads();
        if (tid == 0) {
          const double pz = (double)p * Z;
          uint32_t cc = above;
          double cms = mabove;
          int ck = RB, cp = RB, last = 0;
          for (int b = 0; b < RB; ++b) {
            cc += S.u.h.cnt[0][b];
            cms += S.u.h.mass[0][b];
            if (S.u.h.cnt[0][b]) last = b;
            if (k_on && ck == RB && cc >= (uint32_t)k) ck = b;
            if (p_on && cp == RB && cms >= pz) cp = b;
          }
          // rounding may leave top-p just short inside the bin it crossed in
          if (p_here && cp == RB) cp = last;
          const int c2 = min(min(ck, cp), cm2);
          uint32_t ab = above;
          double mab = mabove;
          for (int b = 0; b < c2; ++b) {
            ab += S.u.h.cnt[0][b];
            mab += S.u.h.mass[0][b];
          }
          S.c = c2;
          S.c_p = cp;
          S.nbin = S.u.h.cnt[0][c2];
          S.above = ab;
          S.mabove = mab;
        }
        __syncthreads();
        const int c2 = S.c;
        p_here = p_here && S.c_p == c2;
        above = S.above;
        mabove = S.mabove;
        prefix |= (uint64_t)(255 - c2) << shift;
        pmask |= (uint64_t)0xff << shift;
        const uint32_t nsub = S.nbin;
        __syncthreads();
        if (nsub <= (uint32_t)CAP || shift == 0) break;
      }
      double dummy;
      nw = collect(
          [&](float s, uint32_t key, int v) {
            return vbin(s) == c && (composite(key, (uint32_t)v) & pmask) == prefix;
          },
          false, dummy);
    }
  }

  // ---- resolve the boundary inside the window
  __syncthreads();
  bitonic_desc(S.u.cand, nw);
  const int E = (nw + ST - 1) / ST;
  const int lo = tid * E, hi = min(lo + E, nw);
  double seg = 0.0;
  for (int i = lo; i < hi; ++i) seg += exp((double)key_value(comp_key(S.u.cand[i])) - m64);
  if (zmode == 1) Z = block_reduce(seg, AddD{}, S.sd);   // the window is the whole row
  const double base = mabove + block_excl_scan(seg, S.sd);
  // min-p: the passing tokens are a prefix of the window
  int nm_loc = INT32_MAX;
  if (m_on)
    for (int i = lo; i < hi; ++i)
      if ((double)key_value(comp_key(S.u.cand[i])) - m64 < thr) {
        nm_loc = i;
        break;
      }
  const int nm_idx = block_reduce(nm_loc, MinI{}, S.si);
  int n_loc = nw;
  if (k_on) {
    const int64_t nk = (int64_t)k - (int64_t)above;
    if (nk >= 1 && nk < n_loc) n_loc = (int)nk;
  }
  if (m_on) {
    const int nm = nm_idx != INT32_MAX ? nm_idx : nw;
    if (nm < n_loc) n_loc = nm;
  }
  if (n_loc < 1) n_loc = 1;
  // number of window tokens up to and including the first at which the
  // running mass (from the thread's base, in window order, as the top-p scan
  // below sums it) reaches pz; INT32_MAX if no window token does
  auto crossing = [&](double b0, double pz) -> int {
    int loc = INT32_MAX;
    double run = b0;
    for (int i = lo; i < hi; ++i) {
      run += exp((double)key_value(comp_key(S.u.cand[i])) - m64);
      if (run >= pz) {
        loc = i;
        break;
      }
    }
    const int idx = block_reduce(loc, MinI{}, S.si);
    return idx != INT32_MAX ? idx + 1 : INT32_MAX;
  };
  // mass of the first `upto` window tokens, summed in the same order as the
  // top-p scan below
  auto mass_upto = [&](int upto, double* dst) {
    const int b = upto - 1;
    if (b >= lo && b < hi) {
      double run = base;
      for (int i = lo; i <= b; ++i) run += exp((double)key_value(comp_key(S.u.cand[i])) - m64);
      *dst = run;
    }
    __syncthreads();
  };
  bool need_p = p_on;
  if (p_on && zmode == 2) {
    // top-p cannot bind before n_loc if even the first n_loc tokens hold
    // clearly less than p of the row mass; otherwise take the exact fp64
    // full-row mass (one more pass) and decide exactly
    mass_upto(n_loc, &S.mass_o);
    if (S.mass_o < (double)p * z32 * (1.0 - 1e-3)) {
      need_p = false;
    } else if (cand) {
      // no keys to sum the exact row mass from: the crossing must be the
      // same for every row mass within the partials' error of z32
      const int np_lo = crossing(base, (double)p * z32 * (1.0 - 1e-3));
      const int np_hi = crossing(base, (double)p * z32 * (1.0 + 1e-3));
      if (np_lo != np_hi || np_lo == INT32_MAX) {
        fail_row();
        return;
      }
      need_p = false;
      if (np_lo < n_loc) n_loc = np_lo;
    } else {
      double zl = 0.0;
      for (int q = tid; q < nv4; q += ST) {
        const f32x4 x = *(const f32x4*)(rp + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q + e < V) zl += exp((double)x[e] - m64);
      }
      Z = block_reduce(zl, AddD{}, S.sd);
    }
  }
  if (need_p) {
    const double pz = (double)p * Z;
    int np_loc = INT32_MAX;
    double run = base;
    for (int i = lo; i < hi; ++i) {
      run += exp((double)key_value(comp_key(S.u.cand[i])) - m64);
      if (run >= pz) {
        np_loc = i;
        break;
      }
    }
    const int np_idx = block_reduce(np_loc, MinI{}, S.si);
    const int np = np_idx != INT32_MAX ? np_idx + 1 : (p_here ? nw : INT32_MAX);
    if (np < n_loc) n_loc = np;
  }
  mass_upto(n_loc, &S.mass_s);
  // (past this point the row is decided; everything below reads the window)
  if (P.ent_supp) {
    // sum over the support of e^(s - m) (s - m): from the window when the
    // support starts at the top of the order, else one membership pass
    double es = 0.0;
    if (above == 0) {
      for (int i = lo; i < min(hi, n_loc); ++i) {
        const double d = (double)key_value(comp_key(S.u.cand[i])) - m64;
        es += exp(d) * d;
      }
    } else {
      const uint64_t bc = S.u.cand[n_loc - 1];
      const uint32_t kt = comp_key(bc), it = comp_id(bc);
      for (int q = tid; q < nv4; q += ST) {
        const f32x4 x = *(const f32x4*)(rp + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * q + e;
          if (v < V) {
            const uint32_t key = order_key(x[e]);
            if (key > kt || (key == kt && (uint32_t)v <= it)) {
              const double d = (double)x[e] - m64;
              es += exp(d) * d;
            }
          }
        }
      }
    }
    const double E = block_reduce(es, AddD{}, S.sd);
    if (tid == 0) P.ent_supp[orow] = (float)(log(S.mass_s) - E / S.mass_s);
  }
  // The vocabulary tiles that can hold a support token: those whose maximum
  // reaches the last support key (a superset of the support's tiles, from the
  // partials), in increasing order; kept when there are at most NTILE.
  if (P.tiles) {
    const float kv = key_value(comp_key(S.u.cand[n_loc - 1]));
    RowTiles* rt = P.tiles + orow;
    const int lane = tid & 63;
    int base = 0;
    __syncthreads();
    for (int t0 = 0; t0 < P.ntv && base <= NTILE; t0 += ST) {
      const int t = t0 + tid;
      const bool hit = t < P.ntv && pp[t].mx >= kv;
      const uint64_t bal = __ballot(hit);
      if (lane == 0) S.si[w] = __popcll(bal);
      __syncthreads();
      int off = base, tot = 0;
#pragma unroll
      for (int q = 0; q < ST / 64; ++q) {
        off += q < w ? S.si[q] : 0;
        tot += S.si[q];
      }
      const int at = off + __popcll(bal & ((1ull << lane) - 1ull));
      if (hit && at < NTILE) rt->t[at] = (uint16_t)t;
      __syncthreads();  // S.si is rewritten by the next pass
      base += tot;
    }
    // unused entries (all of them when there are too many tiles) are zero, so
    // the state's bytes are a function of the inputs
    const int keep = base <= NTILE ? base : 0;
    if (tid >= keep && tid < NTILE) rt->t[tid] = 0;
    if (tid == 0) rt->n = (uint16_t)keep;
  }
  // The support with its keys when it has at most NSP tokens: the window's
  // first n_loc tokens, already in decreasing (key, -id) order, when no
  // token lies ahead of the window; else (a row decided from a histogram,
  // whose keys are stored) one membership pass gathers every token at or
  // above the boundary into the window's space, and they are sorted.
  const uint64_t bcomp = S.u.cand[n_loc - 1];  // the boundary: the last support token
  const int n_sup = (int)above + n_loc;
  bool listed = P.support && n_sup <= NSP && (above == 0 || !cand);
  if (listed && above > 0) {
    __syncthreads();  // (every read of the window is done)
    if (tid == 0) S.cnt = 0;
    __syncthreads();
    for (int q = tid; q < nv4; q += ST) {
      const f32x4 x = *(const f32x4*)(rp + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * q + e;
        if (v < V) {
          const uint64_t c = composite(order_key(x[e]), (uint32_t)v);
          if (c >= bcomp) {
            const int i = atomicAdd(&S.cnt, 1);
            if (i < NSP) S.u.cand[i] = c;
          }
        }
      }
    }
    __syncthreads();
    const int got = S.cnt;
    bitonic_desc(S.u.cand, min(got, NSP));
    listed = got == n_sup;  // (always, as the boundary is a composite of the row's own keys)
  }
  if (P.support) {
    SpEntry* sl = P.support[orow].e;
    for (int i = tid; i < NSP; i += ST) {
      SpEntry e{0, 0.0f};
      if (listed && i < n_sup) {
        const uint64_t c = S.u.cand[i];
        e = SpEntry{(int32_t)comp_id(c), key_value(comp_key(c))};
      }
      sl[i] = e;
    }
  }
  if (tid == 0) {
    const uint64_t bc = bcomp;
    rs.key_thr = comp_key(bc);
    rs.id_thr = (int32_t)comp_id(bc);
    rs.n = (int32_t)n_sup;
    const double lse_s = m64 + log(S.mass_s);
    rs.lse_s = (float)lse_s;
    const uint32_t ky = order_key(sy);
    const bool ign = (fl & ROW_IGNORED) != 0;
    const bool in = !ign && (ky > rs.key_thr || (ky == rs.key_thr && y <= (int64_t)rs.id_thr));
    rs.flags = ROW_VALID | ROW_FILTERED | (in ? ROW_IN_SUPPORT : 0u) | (ign ? ROW_IGNORED : 0u) |
               (listed ? ROW_LISTED : 0u);
    P.logprob[orow] = lane_logprob(P, ign ? 0.0f : (in ? (float)fmin((double)sy - lse_s, 0.0) : -F_INF));
    P.state[orow] = rs;
  }
}

}  // namespace

void launch_select(const SelParams& p, int rows, hipStream_t stream) {
  if (rows <= 0) return;
  ProfScope ps(3, stream);
  hipLaunchKernelGGL(select_kernel, dim3(rows), dim3(ST), 0, stream, p);
}

}  // namespace stce
