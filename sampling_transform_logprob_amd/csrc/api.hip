// Host side of the C ABI declared in include/stce.h: argument checks,
// workspace layout, chunk / slice schedule and kernel launches.  No call
// allocates device memory or synchronizes the stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <unordered_map>

#include "../../include/stce.h"
#include "kernels.hpp"

using namespace stce;

namespace {

thread_local char g_err[512] = "";
thread_local stce_profile* g_prof = nullptr;
thread_local int g_prof_open = -1;

stce_status fail(stce_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

stce_status hip_fail(hipError_t e, const char* what) {
  return fail(STCE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kDefaultChunk = 4096;   // forward rows per chunk
// Default backward slice: the widest (multiple of 256) whose dz (T x V_s
// elements for bf16 operands; twice that for fp32, which also keeps it
// vocab-major) fits in this many bytes.  Wider slices mean fewer
// read-modify-write passes over the fp32 dH sum.
constexpr double kSliceBudgetBytes = 8e9;
constexpr int64_t kMaxSlice = (1 << 22) - 256;  // vocabulary columns of a slice
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  int64_t C, ldt, ntv, nbuf;                               // forward
  size_t f_flags, f_tile, f_part, f_sy, f_hs, fwd;
  size_t buf_tile, buf_part, buf_sy;                       // bytes per chunk buffer
  int64_t Vs, Vsp, Tp;                                      // backward
  size_t b_flags, b_hT, b_WT, b_d, b_dT, b_dh, b_hs, bwd;
};

// The scalar pre-GEMM temperature: the problem's hidden states are replaced
// by h' = h / Ts (rounded to the operand type), written to the workspace.
bool pre_gemm(const stce_problem* p) { return (p->flags & STCE_PROBLEM_PRE_GEMM_TEMPERATURE) != 0; }
// The bf16 value lane: bf16 keys and a bf16 logprob.
int bf16_lane(const stce_problem* p) { return (p->flags & STCE_PROBLEM_BF16_LANE) ? 1 : 0; }

size_t elt_size(int dtype) { return dtype == STCE_DT_BF16 ? 2 : 4; }
size_t hs_bytes(const stce_problem* p) {
  return pre_gemm(p) ? align_up(elt_size(p->dtype) * (size_t)p->T * (size_t)p->H) : 0;
}

stce_status check_shapes(const stce_problem* p) {
  if (!p) return fail(STCE_E_ARG, "problem is NULL");
  if (p->flags & ~(STCE_PROBLEM_IGNORE_INDEX | STCE_PROBLEM_PRE_GEMM_TEMPERATURE | STCE_PROBLEM_BF16_LANE))
    return fail(STCE_E_ARG, "problem.flags=%d has unknown bits", (int)p->flags);
  if (pre_gemm(p) && !(__builtin_isfinite(p->pre_gemm_temperature) && p->pre_gemm_temperature > 0.0f))
    return fail(STCE_E_ARG, "pre_gemm_temperature=%g must be finite and > 0", (double)p->pre_gemm_temperature);
  if ((p->flags & STCE_PROBLEM_IGNORE_INDEX) && p->ignore_index >= 0 && p->ignore_index < p->V)
    return fail(STCE_E_ARG, "ignore_index=%lld is a token id of [0, V)", (long long)p->ignore_index);
  if (p->dtype != STCE_DT_BF16 && p->dtype != STCE_DT_F32)
    return fail(STCE_E_UNSUPPORTED,
                "unsupported operand dtype %d: hidden and weight must both be bf16 (STCE_DT_BF16) or fp32 "
                "(STCE_DT_F32); quantized (e.g. fp8) LM heads are not scored -- keep an fp32/bf16 copy of "
                "lm_head.weight for scoring",
                (int)p->dtype);
  if (bf16_lane(p) && p->dtype != STCE_DT_BF16)
    return fail(STCE_E_UNSUPPORTED, "the bf16 value lane (STCE_PROBLEM_BF16_LANE) takes bf16 hidden and weight");
  if (p->T < 1 || p->T > INT32_MAX - 512) return fail(STCE_E_ARG, "T=%lld out of range [1, 2^31-513]", (long long)p->T);
  if (p->H < 8 || p->H % 8 != 0 || p->H > (1 << 20))
    return fail(STCE_E_ARG, "H=%lld must be a positive multiple of 8 (<= 2^20)", (long long)p->H);
  if (p->V < 1 || p->V > INT32_MAX - 512) return fail(STCE_E_ARG, "V=%lld out of range [1, 2^31-513]", (long long)p->V);
  if (p->chunk_rows < 0 || p->vocab_slice < 0) return fail(STCE_E_ARG, "chunk_rows / vocab_slice must be >= 0");
  return STCE_OK;
}

Layout plan(const stce_problem* p) {
  Layout L{};
  const int64_t T = p->T, V = p->V, H = p->H;
  const size_t es = elt_size(p->dtype);
  L.C = p->chunk_rows > 0 ? p->chunk_rows : kDefaultChunk;
  if (L.C > T) L.C = T;
  L.ldt = round_up(V, 4);
  L.ntv = ceil_div(V, VTILE);
  // two chunk buffers when there is more than one chunk: the selection of
  // chunk c (side stream) reads one while the projection of chunk c + 1
  // writes the other
  L.nbuf = T > L.C ? 2 : 1;
  L.buf_tile = align_up(4 * (size_t)L.C * L.ldt);
  L.buf_part = align_up(sizeof(TilePart) * (size_t)L.C * L.ntv);
  L.buf_sy = align_up(4 * (size_t)L.C);
  size_t o = 0;
  L.f_flags = o; o = align_up(o + 4 * (size_t)T);
  L.f_tile = o;  o += L.nbuf * L.buf_tile;
  L.f_part = o;  o += L.nbuf * L.buf_part;
  L.f_sy = o;    o += L.nbuf * L.buf_sy;
  L.f_hs = o;    o += hs_bytes(p);
  L.fwd = o;

  // bf16 keeps dz vocab-major only (the hidden gradient reads it MN-major);
  // fp32, whose products take K-major operands only, keeps it both ways
  const bool bf = p->dtype == STCE_DT_BF16;
  if (p->vocab_slice > 0) {
    L.Vs = p->vocab_slice;
  } else {
    const double per_col = (bf ? 1.0 : 2.0) * (double)round_up(T, 64) * (double)es;
    int64_t fit = (int64_t)(kSliceBudgetBytes / per_col) / 256 * 256;
    if (fit < 4096) fit = 4096;
    // equal slices: ceil(V / fit) of them
    const int64_t n = ceil_div(V, fit);
    L.Vs = round_up(ceil_div(V, n), 256);
  }
  if (L.Vs > V) L.Vs = V;
  // a product's operand resource spans 256 rows of dz: keep them below 2^31 bytes
  if (L.Vs > kMaxSlice) L.Vs = kMaxSlice;
  L.Vsp = round_up(L.Vs, 64);
  L.Tp = round_up(T, 64);
  o = 0;
  L.b_flags = o; o = align_up(o + 4 * (size_t)T);
  L.b_hT = o;    o = align_up(o + (bf ? 0 : es * (size_t)H * L.Tp));
  L.b_WT = o;    o = align_up(o + es * (size_t)H * L.Vsp);
  L.b_d = o;     o = align_up(o + (bf ? 0 : es * (size_t)L.Tp * L.Vsp));
  L.b_dT = o;    o = align_up(o + es * (size_t)L.Vsp * L.Tp);
  L.b_dh = o;    o = align_up(o + (p->dtype == STCE_DT_BF16 ? 4 * (size_t)T * H : 0));
  L.b_hs = o;    o += hs_bytes(p);
  L.bwd = o;
  return L;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// Scalar parameters of the policy-gradient loss.
stce_status check_pg(const stce_pg_params* pg) {
  if (!pg) return fail(STCE_E_ARG, "pg parameters are NULL");
  if (pg->objective != STCE_PG_CISPO && pg->objective != STCE_PG_CLIP)
    return fail(STCE_E_ARG, "objective=%d: expected STCE_PG_CISPO (1) or STCE_PG_CLIP (2)", (int)pg->objective);
  if (!(pg->eps_low >= 0.0f && pg->eps_low < 1.0f))
    return fail(STCE_E_ARG, "eps_low=%g outside [0, 1)", (double)pg->eps_low);
  if (!(pg->eps_high >= 0.0f && __builtin_isfinite(pg->eps_high)))
    return fail(STCE_E_ARG, "eps_high=%g must be finite and >= 0", (double)pg->eps_high);
  if (!__builtin_isfinite(pg->scale)) return fail(STCE_E_ARG, "scale must be finite");
  return STCE_OK;
}

// Workspace of the fused policy step: two sets of chunk key buffers when
// there is more than one chunk (chunk c's selection, on the side stream,
// overlaps chunk c + 1's projection), the chunk's token-major dz, the
// group's vocab-major dz, the transposed weight and hidden, and the fp32
// split partials of the chunk's hidden gradient.
struct FusedLayout {
  int64_t C, ldt, ntv, Vp, Tp, S, ks, G, nbuf;
  size_t flags, tile, part, sy, g, d, dT, WT, hT, dhp, hs, total;
  size_t buf_tile, buf_part, buf_sy;
};

FusedLayout plan_fused(const stce_problem* p, int64_t gmax = INT64_MAX) {
  FusedLayout L{};
  const int64_t T = p->T, V = p->V, H = p->H;
  const size_t es = elt_size(p->dtype);
  L.Tp = round_up(T, 64);
  L.C = round_up(p->chunk_rows > 0 ? p->chunk_rows : kDefaultChunk, 64);
  if (L.C > L.Tp) L.C = L.Tp;
  L.ldt = round_up(V, 4);
  L.ntv = ceil_div(V, VTILE);
  L.Vp = round_up(V, 64);
  // split-K of the chunk's hidden-gradient product (a chunk has few output
  // tiles): about four workgroups per compute unit, splits at least 512
  // vocabulary columns wide
  const int64_t tiles = ceil_div(L.C, 256) * ceil_div(H, 256);
  int64_t S = ceil_div(4 * 256, tiles);
  if (S > 16) S = 16;
  int64_t ks = round_up(ceil_div(L.Vp, S), 64);
  if (ks < 512) ks = 512;
  if (ks > L.Vp) ks = L.Vp;
  L.ks = ks;
  L.S = ceil_div(L.Vp, ks);
  // the vocab-major dz of G consecutive chunks is kept, so dW is one product
  // per group with the group's rows as its reduction: as many chunks as the
  // slice budget holds (fewer fp32 read-modify-write passes over dW)
  const int64_t nch = ceil_div(T, L.C);
  L.G = (int64_t)(kSliceBudgetBytes / ((double)es * (double)L.Vp * (double)L.C));
  if (L.G > nch) L.G = nch;
  if (L.G > gmax) L.G = gmax;
  if (L.G < 1) L.G = 1;
  size_t o = 0;
  L.flags = o; o = align_up(o + 4 * (size_t)T);
  L.nbuf = nch > 1 ? 2 : 1;
  L.buf_tile = align_up(4 * (size_t)L.C * L.ldt);
  L.buf_part = align_up(sizeof(TilePart) * (size_t)L.C * L.ntv);
  L.buf_sy = align_up(4 * (size_t)L.C);
  L.tile = o;  o += L.nbuf * L.buf_tile;
  L.part = o;  o += L.nbuf * L.buf_part;
  L.sy = o;    o += L.nbuf * L.buf_sy;
  L.g = o;     o = align_up(o + 4 * (size_t)L.C);
  L.d = o;     o = align_up(o + (p->dtype == STCE_DT_BF16 ? 0 : es * (size_t)L.C * L.Vp));
  L.dT = o;    o = align_up(o + es * (size_t)L.Vp * L.C * L.G);
  L.WT = o;    o = align_up(o + es * (size_t)H * L.Vp);
  L.hT = o;    o = align_up(o + (p->dtype == STCE_DT_BF16 ? 0 : es * (size_t)H * L.Tp));
  L.dhp = o;   o = align_up(o + 4 * (size_t)L.S * L.C * H);
  L.hs = o;    o += hs_bytes(p);
  L.total = o;
  return L;
}

stce_status check_inputs(const stce_problem* p) {
  if (!p->hidden || !p->weight || !p->target) return fail(STCE_E_ARG, "hidden, weight and target are required");
  if (!aligned(p->hidden, 16) || !aligned(p->weight, 16))
    return fail(STCE_E_ARG, "hidden and weight must be 16-byte aligned");
  if (!aligned(p->target, 8)) return fail(STCE_E_ARG, "target must be 8-byte aligned");
  if ((p->temperature && !aligned(p->temperature, 4)) || (p->top_k && !aligned(p->top_k, 4)) ||
      (p->top_p && !aligned(p->top_p, 4)) || (p->min_p && !aligned(p->min_p, 4)))
    return fail(STCE_E_ARG, "metadata arrays must be 4-byte aligned");
  if (pre_gemm(p) && p->temperature)
    return fail(STCE_E_ARG,
                "a per-row temperature array and the scalar pre-GEMM temperature do not combine: pass one of them");
  return STCE_OK;
}

// The hidden states the products read: the caller's, or h' = h / Ts written
// into the workspace at `off` (rows row0 .. row0 + nrows; the rows keep their
// offsets).  *dh_div receives the divisor of the hidden gradient.
hipError_t hidden_for_products(const stce_problem* p, void* ws, size_t off, int64_t row0, int64_t nrows,
                               const void** h, float* dh_div, hipStream_t st) {
  *h = p->hidden;
  if (dh_div) *dh_div = 1.0f;
  if (!pre_gemm(p)) return hipSuccess;
  if (dh_div) *dh_div = p->pre_gemm_temperature;
  const size_t es = elt_size(p->dtype);
  char* hs = (char*)ws + off;
  *h = hs;
  return launch_prescale(p->dtype, (const char*)p->hidden + es * (size_t)row0 * p->H, nrows * p->H,
                         p->pre_gemm_temperature, hs + es * (size_t)row0 * p->H, st);
}

stce_status check_ws(void* ws, size_t have, size_t need) {
  if (need && !ws) return fail(STCE_E_WORKSPACE, "workspace is NULL (needs %zu bytes)", need);
  if (have < need) return fail(STCE_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", have, need);
  if (ws && !aligned(ws, kAlign)) return fail(STCE_E_ARG, "workspace must be 256-byte aligned");
  return STCE_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

// Per-thread, per-device side stream (default priority) and four
// timing-free events, created on first use and kept for the thread's life.
// The forward runs each chunk's selection on the side stream, ordered
// against the projections on the caller's stream by event waits only, so
// the pattern is a plain fork/join that stream capture records as graph
// dependencies.  Chunk c uses the fork and done events of its buffer c % 2;
// a wait takes the event's record current at the time of the call, and every
// wait on chunk c's records is enqueued before chunk c + 2 records them
// again, so the four events serve any number of chunks.
struct SideCtx {
  hipStream_t stream = nullptr;
  hipEvent_t ev[4] = {};
  hipEvent_t fork(int64_t c) const { return ev[2 * (c & 1)]; }
  hipEvent_t done(int64_t c) const { return ev[2 * (c & 1) + 1]; }
};
thread_local std::unordered_map<int, SideCtx> g_side;

hipError_t side_ctx(SideCtx** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  SideCtx& c = g_side[dev];
  if (!c.stream && (e = hipStreamCreateWithFlags(&c.stream, hipStreamNonBlocking)) != hipSuccess) return e;
  for (hipEvent_t& ev : c.ev)
    if (!ev && (e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return e;
  *out = &c;
  return hipSuccess;
}

}  // namespace

namespace stce {
void prof_begin(int kind, hipStream_t s) {
  stce_profile* p = g_prof;
  if (!p || p->count >= p->capacity) {
    g_prof_open = -1;
    return;
  }
  g_prof_open = p->count++;
  p->kind[g_prof_open] = kind;
  (void)hipEventRecord((hipEvent_t)p->start[g_prof_open], s);  // diagnostics: a failure only loses a timing
}
void prof_end(hipStream_t s) {
  if (g_prof && g_prof_open >= 0) (void)hipEventRecord((hipEvent_t)g_prof->stop[g_prof_open], s);
  g_prof_open = -1;
}
}  // namespace stce

extern "C" {

stce_status stce_profile_attach(stce_profile* prof) {
  g_prof = prof;
  g_prof_open = -1;
  return STCE_OK;
}


size_t stce_state_bytes(int64_t T) { return T > 0 ? (size_t)T * STCE_STATE_BYTES_PER_ROW : 0; }

stce_status stce_workspace_bytes(const stce_problem* prob, size_t* fwd, size_t* bwd) {
  stce_status s = check_shapes(prob);
  if (s) return s;
  const Layout L = plan(prob);
  if (fwd) *fwd = L.fwd;
  if (bwd) *bwd = L.bwd;
  return STCE_OK;
}

stce_status stce_schedule(const stce_problem* prob, int64_t* chunk_rows, int64_t* vocab_slice) {
  stce_status s = check_shapes(prob);
  if (s) return s;
  const Layout L = plan(prob);
  if (chunk_rows) *chunk_rows = L.C;
  if (vocab_slice) *vocab_slice = L.Vs;
  return STCE_OK;
}

stce_status stce_forward(const stce_problem* p, float* logprob, void* state, int64_t* dev_status, void* ws,
                         size_t ws_bytes, void* stream) {
  return stce_forward_with_side(p, logprob, state, nullptr, dev_status, ws, ws_bytes, stream);
}

stce_status stce_forward_with_side(const stce_problem* p, float* logprob, void* state,
                                   const stce_side_outputs* side_out, int64_t* dev_status, void* ws,
                                   size_t ws_bytes, void* stream) {
  stce_status s = check_shapes(p);
  if (s) return s;
  if ((s = check_inputs(p))) return s;
  if (!logprob || !state) return fail(STCE_E_ARG, "logprob and state are required");
  float* so_lse = side_out ? side_out->lse_full : nullptr;
  float* so_hf = side_out ? side_out->entropy_full : nullptr;
  float* so_hs = side_out ? side_out->entropy_support : nullptr;
  if ((so_lse && !aligned(so_lse, 4)) || (so_hf && !aligned(so_hf, 4)) || (so_hs && !aligned(so_hs, 4)))
    return fail(STCE_E_ARG, "side outputs must be 4-byte aligned");
  const int want_ent = (so_hf || so_hs) ? 1 : 0;
  const Layout L = plan(p);
  if ((s = check_ws(ws, ws_bytes, L.fwd))) return s;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  uint32_t* flags = at<uint32_t>(ws, L.f_flags);
  if (dev_status && (e = launch_fill_i64(dev_status, STCE_STATUS_NONE, st))) return hip_fail(e, "status fill");
  if ((e = launch_validate(p->T, p->V, p->flags & STCE_PROBLEM_IGNORE_INDEX, p->ignore_index, p->temperature,
                           p->top_k, p->top_p, p->min_p, p->target, flags, dev_status,
                           st)))
    return hip_fail(e, "validate");
  const size_t es = elt_size(p->dtype);
  const void* hid = nullptr;
  if ((e = hidden_for_products(p, ws, L.f_hs, 0, p->T, &hid, nullptr, st))) return hip_fail(e, "prescale hidden");
  const int64_t nch = ceil_div(p->T, L.C);
  SideCtx* side = nullptr;
  if (L.nbuf == 2 && (e = side_ctx(&side))) return hip_fail(e, "side stream");
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t c0 = c * L.C;
    const int64_t nc = p->T - c0 < L.C ? p->T - c0 : L.C;
    const int64_t b = c % L.nbuf;
    if (side && c >= 2 && (e = hipStreamWaitEvent(st, side->done(c - 2), 0)))
      return hip_fail(e, "wait for selection");  // chunk c - 2 released this buffer
    FwdArgs a{};
    a.dtype = p->dtype;
    a.W = p->weight;
    a.h = (const char*)hid + es * (size_t)c0 * p->H;
    a.H = p->H;
    a.V = p->V;
    a.rows = nc;
    a.tile = at<float>(ws, L.f_tile + b * L.buf_tile);
    a.ld = L.ldt;
    a.temp = p->temperature ? p->temperature + c0 : nullptr;
    a.target = p->target + c0;
    a.flags = flags + c0;
    a.store_all = 0;
    a.part = at<TilePart>(ws, L.f_part + b * L.buf_part);
    a.ntv = (int)L.ntv;
    a.s_y = at<float>(ws, L.f_sy + b * L.buf_sy);
    a.want_ent = want_ent;
    a.bf16_lane = bf16_lane(p);
    if ((e = launch_fwd_projection(a, st))) return hip_fail(e, "projection");
    hipStream_t ss = st;
    if (side) {
      ss = side->stream;
      if ((e = hipEventRecord(side->fork(c), st)) || (e = hipStreamWaitEvent(ss, side->fork(c), 0)))
        return hip_fail(e, "fork to the side stream");
    }
    SelParams sp{};
    sp.tile = a.tile;
    sp.ld = L.ldt;
    sp.part = a.part;
    sp.ntv = (int)L.ntv;
    sp.s_y = a.s_y;
    sp.flags = flags + c0;
    sp.target = p->target + c0;
    sp.top_k = p->top_k ? p->top_k + c0 : nullptr;
    sp.top_p = p->top_p ? p->top_p + c0 : nullptr;
    sp.min_p = p->min_p ? p->min_p + c0 : nullptr;
    sp.logprob = logprob + c0;
    sp.state = (RowState*)state + c0;
    sp.V = (int)p->V;
    sp.lse_full = so_lse ? so_lse + c0 : nullptr;
    sp.ent_full = so_hf ? so_hf + c0 : nullptr;
    sp.ent_supp = so_hs ? so_hs + c0 : nullptr;
    sp.round_lp_bf16 = bf16_lane(p);
    launch_select(sp, (int)nc, ss);
    if ((e = hipGetLastError())) return hip_fail(e, "select");
    if (side && (e = hipEventRecord(side->done(c), ss))) return hip_fail(e, "selection event");
  }
  // join: the caller's stream waits for the last selection (the side stream
  // runs them in order)
  if (side && (e = hipStreamWaitEvent(st, side->done(nch - 1), 0))) return hip_fail(e, "join");
  return STCE_OK;
}

stce_status stce_backward(const stce_problem* p, const float* grad_logprob, const void* state, void* grad_hidden,
                          float* grad_weight, int32_t accumulate_grad_weight, int64_t* dev_status, void* ws,
                          size_t ws_bytes, void* stream) {
  stce_status s = check_shapes(p);
  if (s) return s;
  if ((s = check_inputs(p))) return s;
  if (!grad_logprob || !state) return fail(STCE_E_ARG, "grad_logprob and state are required");
  if ((grad_hidden && !aligned(grad_hidden, 16)) || (grad_weight && !aligned(grad_weight, 16)))
    return fail(STCE_E_ARG, "gradient outputs must be 16-byte aligned");
  const Layout L = plan(p);
  if ((s = check_ws(ws, ws_bytes, L.bwd))) return s;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dev_status) {
    if ((e = launch_fill_i64(dev_status, STCE_STATUS_NONE, st))) return hip_fail(e, "status fill");
    if ((e = launch_validate(p->T, p->V, p->flags & STCE_PROBLEM_IGNORE_INDEX, p->ignore_index, p->temperature,
                             p->top_k, p->top_p, p->min_p, p->target,
                             at<uint32_t>(ws, L.b_flags), dev_status, st)))
      return hip_fail(e, "validate");
  }
  if (!grad_hidden && !grad_weight) return STCE_OK;
  const void* hid = nullptr;
  float dh_div = 1.0f;
  if ((e = hidden_for_products(p, ws, L.b_hs, 0, p->T, &hid, &dh_div, st))) return hip_fail(e, "prescale hidden");
  if (grad_weight && p->dtype != STCE_DT_BF16) {
    // the fp32 products take K-major operands only (bf16 reads h as it is)
    if ((e = launch_transpose_f32((const float*)hid, p->H, p->T, p->H, at<float>(ws, L.b_hT), L.Tp, L.Tp, st)))
      return hip_fail(e, "transpose hidden");
  }
  const int64_t nsl = ceil_div(p->V, L.Vs);
  for (int64_t si = 0; si < nsl; ++si) {
    BwdSliceArgs a{};
    a.dtype = p->dtype;
    a.W = p->weight;
    a.h = hid;
    a.hT = at<char>(ws, L.b_hT);
    a.WT = at<char>(ws, L.b_WT);
    a.d = at<char>(ws, L.b_d);
    a.dT = at<char>(ws, L.b_dT);
    a.dh_sum = p->dtype == STCE_DT_BF16 ? at<float>(ws, L.b_dh) : (float*)grad_hidden;
    a.grad_hidden = grad_hidden;
    a.grad_weight = grad_weight;
    a.accumulate_w = accumulate_grad_weight ? 1 : 0;
    a.temp = p->temperature;
    a.target = p->target;
    a.st = (const RowState*)state;
    a.g = grad_logprob;
    a.T = p->T;
    a.Tp = L.Tp;
    a.H = p->H;
    a.V = p->V;
    a.v0 = si * L.Vs;
    a.vs = p->V - a.v0 < L.Vs ? p->V - a.v0 : L.Vs;
    a.vsp = round_up(a.vs, 64);
    a.ld_d = L.Vsp;
    a.first = si == 0;
    a.last = si == nsl - 1;
    a.dh_div = dh_div;
    a.bf16_lane = bf16_lane(p);
    if ((e = launch_bwd_slice(a, st))) return hip_fail(e, "backward slice");
  }
  return STCE_OK;
}

stce_status stce_scaled_logits(const stce_problem* p, int64_t row0, int64_t nrows, float* s_out, void* ws,
                               size_t ws_bytes, void* stream) {
  stce_status s = check_shapes(p);
  if (s) return s;
  if ((s = check_inputs(p))) return s;
  if (!s_out) return fail(STCE_E_ARG, "s_out is required");
  if (row0 < 0 || nrows < 0 || row0 + nrows > p->T) return fail(STCE_E_ARG, "rows [%lld, %lld) outside [0, T)",
                                                                 (long long)row0, (long long)(row0 + nrows));
  const Layout L = plan(p);
  if ((s = check_ws(ws, ws_bytes, L.fwd))) return s;
  hipStream_t st = (hipStream_t)stream;
  const size_t es = elt_size(p->dtype);
  const void* hid = nullptr;
  hipError_t e0 = hidden_for_products(p, ws, L.f_hs, row0, nrows, &hid, nullptr, st);
  if (e0) return hip_fail(e0, "prescale hidden");
  for (int64_t c0 = row0; c0 < row0 + nrows; c0 += L.C) {
    const int64_t nc = row0 + nrows - c0 < L.C ? row0 + nrows - c0 : L.C;
    FwdArgs a{};
    a.dtype = p->dtype;
    a.W = p->weight;
    a.h = (const char*)hid + es * (size_t)c0 * p->H;
    a.H = p->H;
    a.V = p->V;
    a.rows = nc;
    a.tile = s_out + (c0 - row0) * p->V;
    a.ld = p->V;
    a.temp = p->temperature ? p->temperature + c0 : nullptr;
    a.target = nullptr;
    a.flags = nullptr;
    a.store_all = 1;
    a.part = at<TilePart>(ws, L.f_part);
    a.ntv = (int)L.ntv;
    a.s_y = nullptr;
    a.bf16_lane = bf16_lane(p);
    hipError_t e = launch_fwd_projection(a, st);
    if (e) return hip_fail(e, "projection");
  }
  return STCE_OK;
}

size_t stce_support_workspace_bytes(int64_t R, int64_t V) {
  if (R < 1 || V < 1) return 0;
  const int64_t ntv = ceil_div(V, VTILE);
  return align_up(4 * (size_t)R) + align_up(sizeof(TilePart) * (size_t)R * ntv) + align_up(4 * (size_t)R);
}

stce_status stce_support_from_logits(const float* sk, int64_t R, int64_t V, const int32_t* top_k, const float* top_p,
                                     const float* min_p, const int64_t* target, float* logprob, void* state,
                                     int64_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  if (!sk || !target || !logprob || !state) return fail(STCE_E_ARG, "s, target, logprob and state are required");
  if (R < 1 || R > INT32_MAX - 512 || V < 1 || V > INT32_MAX - 512)
    return fail(STCE_E_ARG, "R=%lld, V=%lld out of range", (long long)R, (long long)V);
  if (!aligned(sk, 16) || V % 4 != 0) return fail(STCE_E_ARG, "s must be 16-byte aligned with V a multiple of 4");
  stce_status s = check_ws(ws, ws_bytes, stce_support_workspace_bytes(R, V));
  if (s) return s;
  const int64_t ntv = ceil_div(V, VTILE);
  size_t o = 0;
  uint32_t* flags = at<uint32_t>(ws, o);
  o = align_up(o + 4 * (size_t)R);
  TilePart* part = at<TilePart>(ws, o);
  o = align_up(o + sizeof(TilePart) * (size_t)R * ntv);
  float* s_y = at<float>(ws, o);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dev_status && (e = launch_fill_i64(dev_status, STCE_STATUS_NONE, st))) return hip_fail(e, "status fill");
  if ((e = launch_validate(R, V, 0, 0, nullptr, top_k, top_p, min_p, target, flags, dev_status, st)))
    return hip_fail(e, "validate");
  if ((e = launch_tile_partials(sk, V, R, V, (int)ntv, target, part, s_y, st))) return hip_fail(e, "partials");
  SelParams sp{};
  sp.tile = sk;
  sp.ld = V;
  sp.part = part;
  sp.ntv = (int)ntv;
  sp.s_y = s_y;
  sp.flags = flags;
  sp.target = target;
  sp.top_k = top_k;
  sp.top_p = top_p;
  sp.min_p = min_p;
  sp.logprob = logprob;
  sp.state = (RowState*)state;
  sp.V = (int)V;
  launch_select(sp, (int)R, st);
  if ((e = hipGetLastError())) return hip_fail(e, "select");
  return STCE_OK;
}

stce_status stce_decode_state(const void* host_state, int64_t nrows, stce_row_info* out) {
  if (!host_state || !out || nrows < 0) return fail(STCE_E_ARG, "bad arguments");
  static_assert(sizeof(stce_row_info) == sizeof(RowState), "state layout");
  memcpy(out, host_state, (size_t)nrows * sizeof(RowState));
  return STCE_OK;
}

stce_status stce_fused_workspace_bytes(const stce_problem* p, size_t* bytes, size_t* min_bytes) {
  stce_status s = check_shapes(p);
  if (s) return s;
  if (!bytes) return fail(STCE_E_ARG, "bytes is NULL");
  *bytes = plan_fused(p).total;
  if (min_bytes) *min_bytes = plan_fused(p, 1).total;
  return STCE_OK;
}

stce_status stce_fused_policy_step(const stce_problem* p, const stce_pg_params* pg, float* logprob, void* state,
                                   float* loss, float* ratio, const stce_side_outputs* side_out, void* grad_hidden,
                                   float* grad_weight, int32_t accumulate_grad_weight, int64_t* dev_status, void* ws,
                                   size_t ws_bytes, void* stream) {
  stce_status s = check_shapes(p);
  if (s) return s;
  if ((s = check_inputs(p))) return s;
  if ((s = check_pg(pg))) return s;
  if (!pg->advantages || !pg->old_logprob || !logprob || !state || !loss)
    return fail(STCE_E_ARG, "advantages, old_logprob, logprob, state and loss are required");
  if (!aligned(pg->advantages, 4) || !aligned(pg->old_logprob, 4) || !aligned(logprob, 4) || !aligned(loss, 4) ||
      (ratio && !aligned(ratio, 4)) || !aligned(state, 16))
    return fail(STCE_E_ARG, "arrays must be 4-byte aligned (state 16-byte)");
  if ((grad_hidden && !aligned(grad_hidden, 16)) || (grad_weight && !aligned(grad_weight, 16)))
    return fail(STCE_E_ARG, "gradient outputs must be 16-byte aligned");
  float* so_lse = side_out ? side_out->lse_full : nullptr;
  float* so_hf = side_out ? side_out->entropy_full : nullptr;
  float* so_hs = side_out ? side_out->entropy_support : nullptr;
  if ((so_lse && !aligned(so_lse, 4)) || (so_hf && !aligned(so_hf, 4)) || (so_hs && !aligned(so_hs, 4)))
    return fail(STCE_E_ARG, "side outputs must be 4-byte aligned");
  // a workspace below the default keeps fewer chunks per weight-gradient
  // group: each further chunk of a group adds exactly G1.Vp * G1.C elements
  if (4 * round_up(p->V, 4) >= (int64_t)INT32_MAX)
    return fail(STCE_E_ARG, "V=%lld: the fused step takes V < 2^29", (long long)p->V);
  const FusedLayout G1 = plan_fused(p, 1);
  if ((s = check_ws(ws, ws_bytes, G1.total))) return s;
  const size_t per_chunk = elt_size(p->dtype) * (size_t)G1.Vp * (size_t)G1.C;
  const FusedLayout L = plan_fused(p, 1 + (int64_t)((ws_bytes - G1.total) / per_chunk));
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  if (dev_status && (e = launch_fill_i64(dev_status, STCE_STATUS_NONE, st))) return hip_fail(e, "status fill");
  if ((e = launch_validate(p->T, p->V, p->flags & STCE_PROBLEM_IGNORE_INDEX, p->ignore_index, p->temperature,
                           p->top_k, p->top_p, p->min_p, p->target, flags, dev_status, st)))
    return hip_fail(e, "validate");
  const size_t es = elt_size(p->dtype);
  const void* hid = nullptr;
  float dh_div = 1.0f;
  if ((e = hidden_for_products(p, ws, L.hs, 0, p->T, &hid, &dh_div, st))) return hip_fail(e, "prescale hidden");
  if (grad_hidden) {
    if (p->dtype == STCE_DT_BF16)
      e = launch_transpose_bf16((const bf16*)p->weight, p->H, p->V, p->H, at<bf16>(ws, L.WT), L.Vp, L.Vp, st);
    else
      e = launch_transpose_f32((const float*)p->weight, p->H, p->V, p->H, at<float>(ws, L.WT), L.Vp, L.Vp, st);
    if (e) return hip_fail(e, "transpose weight");
  }
  if (grad_weight && p->dtype != STCE_DT_BF16) {
    // fp32 products take K-major operands only (bf16 reads h as it is)
    if ((e = launch_transpose_f32((const float*)hid, p->H, p->T, p->H, at<float>(ws, L.hT), L.Tp, L.Tp, st)))
      return hip_fail(e, "transpose hidden");
  }
  const int64_t nch = ceil_div(p->T, L.C);
  SideCtx* side = nullptr;
  if (L.nbuf == 2 && (e = side_ctx(&side))) return hip_fail(e, "side stream");
  auto rows_of = [&](int64_t c) { return p->T - c * L.C < L.C ? p->T - c * L.C : L.C; };
  // the chunk's keys (every row: the gradient needs them all), then its
  // selection and selected logprob, on the side stream when there is one
  auto project_select = [&](int64_t c) -> stce_status {
    const int64_t c0 = c * L.C, nc = rows_of(c), b = c % L.nbuf;
    FwdArgs a{};
    a.dtype = p->dtype;
    a.W = p->weight;
    a.h = (const char*)hid + es * (size_t)c0 * p->H;
    a.H = p->H;
    a.V = p->V;
    a.rows = nc;
    a.tile = at<float>(ws, L.tile + b * L.buf_tile);
    a.ld = L.ldt;
    a.temp = p->temperature ? p->temperature + c0 : nullptr;
    a.target = p->target + c0;
    a.flags = flags + c0;
    a.store_all = 1;
    a.part = at<TilePart>(ws, L.part + b * L.buf_part);
    a.ntv = (int)L.ntv;
    a.s_y = at<float>(ws, L.sy + b * L.buf_sy);
    a.want_ent = (so_hf || so_hs) ? 1 : 0;
    a.bf16_lane = bf16_lane(p);
    hipError_t e2;
    if ((e2 = launch_fwd_projection(a, st))) return hip_fail(e2, "projection");
    hipStream_t ss = st;
    if (side) {
      ss = side->stream;
      if ((e2 = hipEventRecord(side->fork(c), st)) || (e2 = hipStreamWaitEvent(ss, side->fork(c), 0)))
        return hip_fail(e2, "fork to the side stream");
    }
    SelParams sp{};
    sp.tile = a.tile;
    sp.ld = L.ldt;
    sp.part = a.part;
    sp.ntv = (int)L.ntv;
    sp.s_y = a.s_y;
    sp.flags = flags + c0;
    sp.target = p->target + c0;
    sp.top_k = p->top_k ? p->top_k + c0 : nullptr;
    sp.top_p = p->top_p ? p->top_p + c0 : nullptr;
    sp.min_p = p->min_p ? p->min_p + c0 : nullptr;
    sp.logprob = logprob + c0;
    sp.state = (RowState*)state + c0;
    sp.V = (int)p->V;
    sp.lse_full = so_lse ? so_lse + c0 : nullptr;
    sp.ent_full = so_hf ? so_hf + c0 : nullptr;
    sp.ent_supp = so_hs ? so_hs + c0 : nullptr;
    sp.round_lp_bf16 = bf16_lane(p);
    launch_select(sp, (int)nc, ss);
    if ((e2 = hipGetLastError())) return hip_fail(e2, "select");
    if (side && (e2 = hipEventRecord(side->done(c), ss))) return hip_fail(e2, "selection event");
    return STCE_OK;
  };
  if ((s = project_select(0))) return s;
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t c0 = c * L.C, nc = rows_of(c), b = c % L.nbuf;
    // the next chunk's projection overlaps this chunk's selection; it writes
    // the other buffer, whose readers (chunk c - 1's selection and dz) are
    // done: the first is waited for below, the second is earlier on `st`
    if (c + 1 < nch && (s = project_select(c + 1))) return s;
    if (side && (e = hipStreamWaitEvent(st, side->done(c), 0))) return hip_fail(e, "join");
    // the token loss of the chunk's rows
    RowState* stc = (RowState*)state + c0;
    float* g = at<float>(ws, L.g);
    if ((e = launch_policy_loss(pg->objective, pg->eps_low, pg->eps_high, pg->scale, pg->advantages + c0,
                                pg->old_logprob + c0, stc, nc, logprob + c0, loss + c0, g,
                                ratio ? ratio + c0 : nullptr, st)))
      return hip_fail(e, "policy loss");
    if (!grad_hidden && !grad_weight) continue;
    // dlogits formed from the chunk's keys, then its dH rows and its share
    // of dW
    FusedGradArgs ga{};
    ga.dtype = p->dtype;
    ga.keys = at<float>(ws, L.tile + b * L.buf_tile);
    ga.ld_keys = L.ldt;
    ga.temp = p->temperature ? p->temperature + c0 : nullptr;
    ga.target = p->target + c0;
    ga.st = stc;
    ga.g = g;
    ga.d = at<char>(ws, L.d);
    ga.dT = at<char>(ws, L.dT);
    ga.ld_dT = L.G * L.C;
    ga.dT_col = (c % L.G) * L.C;
    ga.WT = at<char>(ws, L.WT);
    ga.hT = at<char>(ws, L.hT);
    ga.h = hid;
    ga.T = p->T;
    ga.dh_part = at<float>(ws, L.dhp);
    ga.splits = (int)L.S;
    ga.ks = L.ks;
    ga.grad_hidden = grad_hidden ? (char*)grad_hidden + es * (size_t)c0 * p->H : nullptr;
    ga.grad_weight = grad_weight;
    ga.accumulate_w = (c >= L.G || accumulate_grad_weight) ? 1 : 0;
    ga.rows = nc;
    ga.rows_pad = round_up(nc, 64);
    ga.dw = (c % L.G == L.G - 1 || c == nch - 1) ? 1 : 0;
    ga.dw_c0 = (c / L.G) * L.G * L.C;
    ga.dw_k = c0 - ga.dw_c0 + ga.rows_pad;
    ga.Tp = L.Tp;
    ga.H = p->H;
    ga.V = p->V;
    ga.V_pad = L.Vp;
    ga.dh_div = dh_div;
    if ((e = launch_fused_chunk_grads(ga, st))) return hip_fail(e, "fused gradients");
  }
  return STCE_OK;
}

stce_status stce_policy_loss(const stce_pg_params* pg, int64_t T, const float* logprob, float* loss,
                             float* grad_logprob, float* ratio, void* stream) {
  stce_status s = check_pg(pg);
  if (s) return s;
  if (T < 1 || T > INT32_MAX - 512) return fail(STCE_E_ARG, "T=%lld out of range", (long long)T);
  if (!pg->advantages || !pg->old_logprob || !logprob || !loss || !grad_logprob)
    return fail(STCE_E_ARG, "advantages, old_logprob, logprob, loss and grad_logprob are required");
  if (!aligned(pg->advantages, 4) || !aligned(pg->old_logprob, 4) || !aligned(logprob, 4) || !aligned(loss, 4) ||
      !aligned(grad_logprob, 4) || (ratio && !aligned(ratio, 4)) || (pg->state && !aligned(pg->state, 16)))
    return fail(STCE_E_ARG, "arrays must be 4-byte aligned (state 16-byte)");
  hipError_t e = launch_policy_loss(pg->objective, pg->eps_low, pg->eps_high, pg->scale, pg->advantages,
                                    pg->old_logprob, (const RowState*)pg->state, T, logprob, loss, grad_logprob,
                                    ratio, (hipStream_t)stream);
  if (e) return hip_fail(e, "policy loss");
  return STCE_OK;
}

const char* stce_status_string(stce_status status) {
  switch (status) {
    case STCE_OK: return "STCE_OK";
    case STCE_E_ARG: return "STCE_E_ARG: invalid argument";
    case STCE_E_UNSUPPORTED: return "STCE_E_UNSUPPORTED: unsupported dtype or shape";
    case STCE_E_WORKSPACE: return "STCE_E_WORKSPACE: workspace too small";
    case STCE_E_HIP: return "STCE_E_HIP: HIP runtime error";
  }
  return "unknown stce_status";
}

const char* stce_last_error(void) { return g_err; }

}  // extern "C"
