// C ABI of libgdn: argument checks, workspace layout and launch sequencing.
// Every check runs on the host before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "gdn.h"
#include "gdn_common.h"

// Device scratch of gdn_step_noalloc (one copy per GPU). Host code never uses
// this name as an address: it holds a host-side stand-in; the device address
// comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

using gdn::Shape;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p % 16) == 0; }

// Every launch must hold fewer than 2^32 work-items (the limit of a dispatch).
// Conservative bounds of the grids a call on sh can launch, `chunks` being its
// largest count of time chunks or reverse-scan chunks: the per-frame-head
// kernels (phase 1 with up to 5 splits of 512 threads, the readout, the
// backward's passes) at most 4096 work-items per frame-head; the fp32 and
// small-D kernels at most S D + 4096 per frame-head; the scans and the
// combine at most 32 blocks of 256 threads per (head, chunk) job.
bool grids_fit(const gdn::Shape& sh, int64_t chunks) {
  const long double limit = (long double)gdn::kGridLimit;
  const long double fh = (long double)sh.FH();
  if (fh * 4096.0L > limit) return false;
  if (!(sh.io == 1 && sh.D == 128) && fh * ((long double)sh.S * sh.D + 4096.0L) > limit) return false;
  const long double jobs = (long double)sh.BH() * (long double)(chunks > 1 ? chunks : 1);
  return (jobs + 8.0L) * 32.0L * 256.0L <= limit;
}

gdn_status check_desc(const gdn_desc* d, Shape* sh) {
  if (d == nullptr) return GDN_EINVAL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->S < 1 || d->D < 1) return GDN_EINVAL;
  if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) return GDN_EINVAL;
  if ((d->flags & ~(GDN_KEYS_PREPARED | GDN_QK_RMSNORM | GDN_REUSE_FWD_TERMS)) != 0)
    return GDN_EINVAL;
  if (!(std::isfinite(d->key_scale))) return GDN_EINVAL;
  if (d->D != 16 && d->D != 32 && d->D != 64 && d->D != 128) return GDN_EUNSUPPORTED;
  // element counts must stay far from 64-bit overflow
  const double elems = (double)d->B * d->H * d->T * d->S * d->D;
  if (elems > 4.0e18) return GDN_EINVAL;
  sh->B = d->B;
  sh->H = d->H;
  sh->T = d->T;
  sh->S = d->S;
  sh->D = d->D;
  sh->io = d->io_dtype;
  sh->prepared = (d->flags & GDN_KEYS_PREPARED) ? 1 : 0;
  sh->qk_norm = (d->flags & GDN_QK_RMSNORM) ? 1 : 0;
  sh->reuse_terms = (d->flags & GDN_REUSE_FWD_TERMS) ? 1 : 0;
  if (!grids_fit(*sh, 1)) return GDN_EUNSUPPORTED;
  if (sh->prepared) {
    sh->c = 1.0f;
  } else if (d->key_scale > 0.f) {
    sh->c = d->key_scale;
  } else {
    sh->c = (float)(1.0 / std::sqrt((double)d->D * (double)d->S));
  }
  return GDN_OK;
}

struct Layout {
  size_t terms = 0, partial = 0, states = 0, rev = 0, compC = 0, compH = 0, start = 0;
  size_t total = 0;
  int n_split = 1;
};

Layout layout(const Shape& sh, int P) {
  Layout L;
  const size_t DD = (size_t)sh.D * sh.D * sizeof(float);
  const size_t FH = (size_t)sh.FH();
  const size_t BH = (size_t)sh.BH();
  L.n_split = gdn::terms_split(sh);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.terms = take(FH * 2 * DD);
  L.partial = take(L.n_split > 1 ? FH * L.n_split * 2 * DD : 0);
  L.states = take(FH * DD);
  L.rev = take(FH * DD);
  const size_t Pn = (size_t)(P > 1 ? P : 1);
  L.compC = take(BH * Pn * DD);
  L.compH = take(BH * Pn * DD);
  L.start = take(BH * Pn * DD);
  L.total = off;
  return L;
}

// Workspace of the backward pass: phase-1 terms (A; the same offset and size
// as in the forward layout, so a forward call's workspace can hand its terms
// over), split partials, E_t,
// the adjoint states G, the per-frame P_t, G_{T-1} per head and a ones gate;
// for the chunk-causal scan (n_rev chunks) also the reverse-state adjoint F
// and its value at every chunk start.
struct BwdLayout {
  size_t terms = 0, partial = 0, E = 0, G = 0, P = 0, ginit = 0, ones = 0, F = 0, finit = 0;
  size_t total = 0;
  int n_split = 1;
};

BwdLayout bwd_layout(const Shape& sh, int64_t n_rev = 0) {
  BwdLayout L;
  const size_t DD = (size_t)sh.D * sh.D * sizeof(float);
  const size_t FH = (size_t)sh.FH();
  L.n_split = gdn::terms_split(sh);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.terms = take(FH * 2 * DD);
  L.partial = take(L.n_split > 1 ? FH * L.n_split * 2 * DD : 0);
  L.E = take(FH * DD);
  L.G = take(FH * DD);
  L.P = take(FH * DD);
  L.ginit = take((size_t)sh.BH() * DD);
  L.ones = take(FH * (size_t)sh.S * sizeof(float));
  L.F = take(n_rev > 0 ? FH * DD : 0);
  L.finit = take((size_t)sh.BH() * (size_t)n_rev * DD);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

#define GDN_HIP(x)                                 \
  do {                                             \
    if ((x) != hipSuccess) return GDN_EHIP;        \
  } while (0)

// The calling thread's phase trace (gdn_trace_set), or NULL.
thread_local gdn_trace* t_trace = nullptr;

// Records the next event of the thread's trace on `st`, tagged with `phase`.
hipError_t mark(int phase, hipStream_t st) {
  gdn_trace* t = t_trace;
  if (t == nullptr || t->count < 0 || t->count >= t->capacity) return hipSuccess;
  const hipError_t e = hipEventRecord((hipEvent_t)t->events[t->count], st);
  if (e != hipSuccess) return e;
  t->phases[t->count++] = phase;
  return hipSuccess;
}
#define GDN_MARK(phase, st) GDN_HIP(mark(phase, st))

// Device pointers of one call.
struct Slice {
  const char* q;
  const char* k;
  const char* v;
  const float* beta;
  const float* gamma;
  const float* s0;
  float* fwd;        // per-frame forward states (nullable)
  float* rev;        // per-frame reverse states (nullable)
  float* s_final;    // nullable
  char* o;           // nullable
  float* terms;      // workspace [FH][2D][D]
  float* partial;    // workspace [FH][n_split][2D][D] (n_split > 1 only)
  float* compC;      // workspace [BH][P][D][D]
  float* compH;
  float* start;

};

Slice work_slice(const Layout& L, void* ws) {
  Slice w;
  memset(&w, 0, sizeof(w));
  w.terms = at<float>(ws, L.terms);
  w.partial = at<float>(ws, L.partial);
  w.compC = at<float>(ws, L.compC);
  w.compH = at<float>(ws, L.compH);
  w.start = at<float>(ws, L.start);
  return w;
}

// Phase 1 into the terms buffer [FH][2D][D].
gdn_status run_terms(const Shape& sh, int n_split, const Slice& x, hipStream_t st) {
  const int64_t DD = (int64_t)sh.D * sh.D;
  gdn::TermsOut direct{x.terms, x.terms + DD, 2 * DD, 0};
  const bool scan_layout = gdn::scan_uses_mfma(sh);
  if (n_split == 1) {
    GDN_HIP(gdn::launch_terms(sh, x.k, x.v, x.beta, 1, direct, scan_layout, st));
    GDN_MARK(GDN_PHASE_TERMS, st);
  } else {
    gdn::TermsOut po{x.partial, x.partial + DD, (int64_t)n_split * 2 * DD, 2 * DD};
    GDN_HIP(gdn::launch_terms(sh, x.k, x.v, x.beta, n_split, po, false, st));
    GDN_MARK(GDN_PHASE_TERMS, st);
    GDN_HIP(gdn::launch_reduce_partials(sh, x.partial, n_split, direct, scan_layout, st));
    GDN_MARK(GDN_PHASE_TERMS_REDUCE, st);
  }
  return GDN_OK;
}

void uniform_offsets(int* offs, int T, int P) {
  for (int p = 0; p <= P; ++p) offs[p] = (int)(((int64_t)p * T) / P);
}

// Parameters of the scan launches over the terms buffer.
// Sequential forward scan into x.fwd (nullable) and x.s_final (nullable).
gdn::ScanParams seq_params(const Shape& sh, const Slice& x) {
  const int64_t DD = (int64_t)sh.D * sh.D;
  gdn::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.terms = x.terms;
  p.gamma = x.gamma;
  p.T = sh.T;
  p.nchunk = 1;
  p.mode = gdn::SCAN_FORWARD;
  p.init = x.s0;
  p.init_bh_stride = DD;
  p.init_c_stride = 0;
  p.states = x.fwd;
  p.finA = x.s_final;
  p.fin_bh_stride = DD;
  p.fin_last_only = 1;
  p.offsets[0] = 0;
  p.offsets[1] = sh.T;
  return p;
}

// Composites (C_p, H_p) of P time chunks into x.compC, x.compH.
gdn::ScanParams compose_params(const Shape& sh, int P, const Slice& x) {
  const int64_t DD = (int64_t)sh.D * sh.D;
  gdn::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.terms = x.terms;
  p.gamma = x.gamma;
  p.T = sh.T;
  p.nchunk = P;
  p.mode = gdn::SCAN_COMPOSE;
  p.finA = x.compC;
  p.finB = x.compH;
  p.fin_bh_stride = (int64_t)P * DD;
  p.fin_c_stride = DD;
  uniform_offsets(p.offsets, sh.T, P);
  return p;
}

// Every chunk replayed from its start state x.start into x.fwd / x.s_final.
gdn::ScanParams replay_params(const Shape& sh, int P, const Slice& x) {
  const int64_t DD = (int64_t)sh.D * sh.D;
  gdn::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.terms = x.terms;
  p.gamma = x.gamma;
  p.T = sh.T;
  p.nchunk = P;
  p.mode = gdn::SCAN_FORWARD;
  p.init = x.start;
  p.init_bh_stride = (int64_t)P * DD;
  p.init_c_stride = DD;
  p.states = x.fwd;
  p.finA = x.s_final;
  p.fin_bh_stride = DD;
  p.fin_last_only = 1;
  uniform_offsets(p.offsets, sh.T, P);
  return p;
}

// Reverse scan restarted at every chunk_len-frame boundary into x.rev.
gdn::ScanParams reverse_params(const Shape& sh, int chunk_len, const Slice& x) {
  const int64_t n_rev = ((int64_t)sh.T + chunk_len - 1) / chunk_len;
  gdn::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.terms = x.terms;
  p.gamma = x.gamma;
  p.T = sh.T;
  p.nchunk = (int)n_rev;
  p.mode = gdn::SCAN_REVERSE;
  p.states = x.rev;
  for (int c = 0; c <= (int)n_rev; ++c) {
    int64_t off = (int64_t)c * chunk_len;
    p.offsets[c] = (int)(off < sh.T ? off : sh.T);
  }
  return p;
}

// Everything after phase 1 except the readout: forward scan (when per-frame
// forward states or the final state are wanted; sequential for P <= 1, else
// compose, combine and replay) and the chunk-reset reverse scan (chunk_len >
// 0, when reverse states are wanted). The reverse scan needs only the terms,
// so on the MFMA path it shares a launch with the first forward one (the
// compose of several chunks, or a sequential scan that leaves most CUs idle).
gdn_status run_scans(const Shape& sh, int P, int chunk_len, const Slice& x, hipStream_t st) {
  const bool fwd = x.fwd || x.s_final;
  const bool rev = chunk_len > 0 && x.rev;
  const gdn::ScanParams first = P <= 1 ? seq_params(sh, x) : compose_params(sh, P, x);
  const gdn::ScanParams second = rev ? reverse_params(sh, chunk_len, x) : first;
  const bool pair = fwd && rev && gdn::scan_pairs(sh);
  if (fwd) {
    if (pair)
      GDN_HIP(gdn::launch_scan_pair(sh, first, second, st));
    else
      GDN_HIP(gdn::launch_scan(sh, first, st));
    GDN_MARK(GDN_PHASE_SCAN, st);
    if (P > 1) {
      gdn::CombineParams cp{x.compC, x.compH, x.s0, x.start, P};
      GDN_HIP(gdn::launch_combine(sh, cp, st));
      GDN_MARK(GDN_PHASE_COMBINE, st);
      GDN_HIP(gdn::launch_scan(sh, replay_params(sh, P, x), st));
      GDN_MARK(GDN_PHASE_REPLAY, st);
    }
  }
  if (rev && !pair) {
    GDN_HIP(gdn::launch_scan(sh, second, st));
    GDN_MARK(GDN_PHASE_REVERSE, st);
  }
  return GDN_OK;
}

gdn_status run_readout(const Shape& sh, const Slice& x, hipStream_t st) {
  if (x.o) {
    GDN_HIP(gdn::launch_readout(sh, x.q, x.fwd, x.rev, x.o, st));
    GDN_MARK(GDN_PHASE_READOUT, st);
  }
  return GDN_OK;
}

// Phase 1, scans and readout of a whole call, in stream order.
gdn_status run_path(const Shape& sh, int n_split, int P, int chunk_len, const Slice& x,
                    hipStream_t st) {
  gdn_status s;
  GDN_MARK(GDN_PHASE_CALL_BEGIN, st);
  if ((s = run_terms(sh, n_split, x, st)) != GDN_OK) return s;
  if ((s = run_scans(sh, P, chunk_len, x, st)) != GDN_OK) return s;
  return run_readout(sh, x, st);
}

// No frames: the final state is the initial state.
gdn_status run_empty(const Shape& sh, const float* s0, float* s_final, hipStream_t st) {
  if (s_final == nullptr) return GDN_OK;
  GDN_MARK(GDN_PHASE_CALL_BEGIN, st);
  const int64_t n = sh.BH() * sh.D * sh.D;
  if (s0)
    GDN_HIP(gdn::launch_copy_f32(s0, s_final, n, st));
  else
    GDN_HIP(gdn::launch_zero_f32(s_final, n, st));
  GDN_MARK(GDN_PHASE_OTHER, st);
  return GDN_OK;
}

gdn_status check_ws(const Layout& L, const void* ws, size_t ws_bytes) {
  if (ws_bytes < L.total) return GDN_EWORKSPACE;
  if (L.total > 0 && ws == nullptr) return GDN_EINVAL;
  if (((uintptr_t)ws % kAlign) != 0) return GDN_EINVAL;
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_str(int32_t s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_EINVAL: return "GDN_EINVAL: invalid argument";
    case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED: unsupported configuration";
    case GDN_EWORKSPACE: return "GDN_EWORKSPACE: workspace too small";
    case GDN_EHIP: return "GDN_EHIP: HIP launch failed";
    default: return "GDN: unknown status";
  }
}

gdn_status gdn_trace_set(gdn_trace* trace) {
  if (trace != nullptr &&
      (trace->events == nullptr || trace->phases == nullptr || trace->capacity < 0 || trace->count < 0))
    return GDN_EINVAL;
  t_trace = trace;
  return GDN_OK;
}

gdn_status gdn_workspace_bytes(const gdn_desc* desc, int32_t n_time_chunks, size_t* bytes) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (!grids_fit(sh, n_time_chunks)) return GDN_EUNSUPPORTED;
  if (bytes == nullptr || n_time_chunks < 1 || n_time_chunks > GDN_MAX_TIME_CHUNKS)
    return GDN_EINVAL;
  *bytes = layout(sh, n_time_chunks).total;
  return GDN_OK;
}

gdn_status gdn_prepare(const gdn_desc* desc, const void* k, void* k_hat, void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (sh.prepared) return GDN_EINVAL;
  if (sh.FH() == 0) return GDN_OK;
  if (k == nullptr || k_hat == nullptr || !aligned16(k) || !aligned16(k_hat)) return GDN_EINVAL;
  GDN_MARK(GDN_PHASE_CALL_BEGIN, (hipStream_t)stream);
  GDN_HIP(gdn::launch_prepare(sh, k, k_hat, (hipStream_t)stream));
  GDN_MARK(GDN_PHASE_OTHER, (hipStream_t)stream);
  return GDN_OK;
}

gdn_status gdn_frame_terms(const gdn_desc* desc, const void* k, const void* v, const float* beta,
                           float* A, float* U, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (sh.FH() == 0 || (A == nullptr && U == nullptr)) return GDN_OK;
  if (!k || !v || !beta) return GDN_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(A) || !aligned16(U)) return GDN_EINVAL;
  Layout L = layout(sh, 1);
  if ((s = check_ws(L, ws, ws_bytes)) != GDN_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int64_t DD = (int64_t)sh.D * sh.D;
  gdn::TermsOut direct{A, U, DD, 0};
  GDN_MARK(GDN_PHASE_CALL_BEGIN, st);
  if (L.n_split == 1) {
    GDN_HIP(gdn::launch_terms(sh, k, v, beta, 1, direct, false, st));
    GDN_MARK(GDN_PHASE_TERMS, st);
  } else {
    float* part = at<float>(ws, L.partial);
    gdn::TermsOut po{part, part + DD, (int64_t)L.n_split * 2 * DD, 2 * DD};
    GDN_HIP(gdn::launch_terms(sh, k, v, beta, L.n_split, po, false, st));
    GDN_MARK(GDN_PHASE_TERMS, st);
    GDN_HIP(gdn::launch_reduce_partials(sh, part, L.n_split, direct, false, st));
    GDN_MARK(GDN_PHASE_TERMS_REDUCE, st);
  }
  return GDN_OK;
}

gdn_status gdn_scan_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                        const float* beta, const float* gamma, const float* s0, float* states,
                        float* s_final, void* o, int32_t n_time_chunks, void* ws, size_t ws_bytes,
                        void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (n_time_chunks < 1 || n_time_chunks > GDN_MAX_TIME_CHUNKS) return GDN_EINVAL;
  if (sh.T > 0 && n_time_chunks > sh.T) return GDN_EINVAL;
  if (!grids_fit(sh, n_time_chunks)) return GDN_EUNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(s0) || !aligned16(states) ||
      !aligned16(s_final) || !aligned16(o))
    return GDN_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (sh.BH() == 0) return GDN_OK;
  if (sh.T == 0) return run_empty(sh, s0, s_final, st);
  if (states == nullptr && s_final == nullptr && o == nullptr) return GDN_OK;
  if (!k || !v || !beta || !gamma || (o && !q)) return GDN_EINVAL;
  Layout L = layout(sh, n_time_chunks);
  if ((s = check_ws(L, ws, ws_bytes)) != GDN_OK) return s;
  Slice x = work_slice(L, ws);
  x.q = (const char*)q;
  x.k = (const char*)k;
  x.v = (const char*)v;
  x.beta = beta;
  x.gamma = gamma;
  x.s0 = s0;
  x.fwd = states ? states : (o ? at<float>(ws, L.states) : nullptr);
  x.s_final = s_final;
  x.o = (char*)o;
  return run_path(sh, L.n_split, n_time_chunks, 0, x, st);
}

gdn_status gdn_scan_bidir_chunked(const gdn_desc* desc, const void* q, const void* k,
                                  const void* v, const float* beta, const float* gamma,
                                  const float* s0, int32_t chunk_len, float* states_fwd,
                                  float* states_rev, float* s_final, void* o,
                                  int32_t n_time_chunks, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (chunk_len < 1) return GDN_EINVAL;
  if (n_time_chunks < 1 || n_time_chunks > GDN_MAX_TIME_CHUNKS) return GDN_EINVAL;
  if (sh.T > 0 && n_time_chunks > sh.T) return GDN_EINVAL;
  const int64_t n_rev = sh.T > 0 ? ((int64_t)sh.T + chunk_len - 1) / chunk_len : 0;
  if (n_rev > gdn::kMaxChunks) return GDN_EUNSUPPORTED;
  if (!grids_fit(sh, n_rev > n_time_chunks ? n_rev : n_time_chunks)) return GDN_EUNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(s0) ||
      !aligned16(states_fwd) || !aligned16(states_rev) || !aligned16(s_final) || !aligned16(o))
    return GDN_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (sh.BH() == 0) return GDN_OK;
  if (sh.T == 0) return run_empty(sh, s0, s_final, st);
  if (!states_fwd && !states_rev && !s_final && !o) return GDN_OK;
  if (!k || !v || !beta || !gamma || (o && !q)) return GDN_EINVAL;
  Layout L = layout(sh, n_time_chunks);
  if ((s = check_ws(L, ws, ws_bytes)) != GDN_OK) return s;
  Slice x = work_slice(L, ws);
  x.q = (const char*)q;
  x.k = (const char*)k;
  x.v = (const char*)v;
  x.beta = beta;
  x.gamma = gamma;
  x.s0 = s0;
  x.fwd = states_fwd ? states_fwd : (o ? at<float>(ws, L.states) : nullptr);
  x.rev = states_rev ? states_rev : (o ? at<float>(ws, L.rev) : nullptr);
  x.s_final = s_final;
  x.o = (char*)o;
  return run_path(sh, L.n_split, n_time_chunks, chunk_len, x, st);
}

gdn_status gdn_step(const gdn_desc* desc, const void* q, const void* k, const void* v,
                    const float* beta, const float* gamma, const float* carry_in,
                    float* carry_out, void* o, float* states_fwd, float* states_rev, void* ws,
                    size_t ws_bytes, void* stream) {
  if (desc == nullptr) return GDN_EINVAL;
  // the block is one reverse chunk; T = 0 passes the carry through
  const int32_t chunk_len = desc->T > 0 ? desc->T : 1;
  return gdn_scan_bidir_chunked(desc, q, k, v, beta, gamma, carry_in, chunk_len, states_fwd,
                                states_rev, carry_out, o, 1, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the device of `st`, which must be the
// current device; looked up on the device's first call and kept.
gdn_status scratch_address(hipStream_t st, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GDN_EHIP;
  int dev = cur;
  if (st != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(st, &d) != hipSuccess) return GDN_EINVAL;
    dev = d;
  }
  if (dev != cur) return GDN_EINVAL;
  if (dev < 0 || dev >= kMaxDevices) return GDN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GDN_EHIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_step_noalloc(const gdn_desc* desc, const void* q, const void* k, const void* v,
                            const float* beta, const float* gamma, const float* carry_in,
                            float* carry_out, void* o, float* states_fwd, float* states_rev,
                            void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (layout(sh, 1).total > GDN_NOALLOC_SCRATCH_BYTES) return GDN_EWORKSPACE;
  void* ws = nullptr;
  if ((s = scratch_address((hipStream_t)stream, &ws)) != GDN_OK) return s;
  return gdn_step(desc, q, k, v, beta, gamma, carry_in, carry_out, o, states_fwd, states_rev, ws,
                  GDN_NOALLOC_SCRATCH_BYTES, stream);
}

gdn_status gdn_compose(const gdn_desc* desc, const void* k, const void* v, const float* beta,
                       const float* gamma, const int32_t* chunk_offsets, int32_t P, float* C,
                       float* Hc, const float* s0, float* s_start, void* ws, size_t ws_bytes,
                       void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (P < 1 || P > GDN_MAX_TIME_CHUNKS || chunk_offsets == nullptr) return GDN_EINVAL;
  if (!grids_fit(sh, P)) return GDN_EUNSUPPORTED;
  if (chunk_offsets[0] != 0 || chunk_offsets[P] != sh.T) return GDN_EINVAL;
  for (int p = 0; p < P; ++p)
    if (chunk_offsets[p + 1] < chunk_offsets[p]) return GDN_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(C) || !aligned16(Hc) || !aligned16(s0) ||
      !aligned16(s_start))
    return GDN_EINVAL;
  if (sh.BH() == 0 || (!C && !Hc && !s_start)) return GDN_OK;
  if (sh.T > 0 && (!k || !v || !beta || !gamma)) return GDN_EINVAL;
  Layout L = layout(sh, P);
  if ((s = check_ws(L, ws, ws_bytes)) != GDN_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int64_t DD = (int64_t)sh.D * sh.D;
  float* Cb = C ? C : at<float>(ws, L.compC);
  float* Hb = Hc ? Hc : at<float>(ws, L.compH);
  GDN_MARK(GDN_PHASE_CALL_BEGIN, st);
  if (sh.T > 0) {
    Slice x = work_slice(L, ws);
    x.k = (const char*)k;
    x.v = (const char*)v;
    x.beta = beta;
    if ((s = run_terms(sh, L.n_split, x, st)) != GDN_OK) return s;
  }
  gdn::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.terms = at<float>(ws, L.terms);
  p.gamma = gamma;
  p.T = sh.T;
  p.nchunk = P;
  p.mode = gdn::SCAN_COMPOSE;
  p.finA = Cb;
  p.finB = Hb;
  p.fin_bh_stride = (int64_t)P * DD;
  p.fin_c_stride = DD;
  for (int c = 0; c <= P; ++c) p.offsets[c] = chunk_offsets[c];
  GDN_HIP(gdn::launch_scan(sh, p, st));
  GDN_MARK(GDN_PHASE_SCAN, st);
  if (s_start) {
    gdn::CombineParams cp{Cb, Hb, s0, s_start, P};
    GDN_HIP(gdn::launch_combine(sh, cp, st));
    GDN_MARK(GDN_PHASE_COMBINE, st);
  }
  return GDN_OK;
}

gdn_status gdn_bwd_workspace_bytes(const gdn_desc* desc, size_t* bytes) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (bytes == nullptr) return GDN_EINVAL;
  *bytes = bwd_layout(sh).total;
  return GDN_OK;
}

gdn_status gdn_bidir_bwd_workspace_bytes(const gdn_desc* desc, int32_t chunk_len, size_t* bytes) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (bytes == nullptr || chunk_len < 1) return GDN_EINVAL;
  const int64_t n_rev = sh.T > 0 ? ((int64_t)sh.T + chunk_len - 1) / chunk_len : 0;
  if (n_rev > gdn::kMaxChunks) return GDN_EUNSUPPORTED;
  if (!grids_fit(sh, n_rev)) return GDN_EUNSUPPORTED;
  *bytes = bwd_layout(sh, n_rev).total;
  return GDN_OK;
}

}  // extern "C"

namespace {

// Both backward passes. chunk_len == 0: the causal scan; otherwise the
// chunk-causal bidirectional scan with reverse states `rev`.
gdn_status run_bwd(const gdn_desc* desc, int32_t chunk_len, const void* q, const void* k,
                   const void* v, const float* beta, const float* gamma, const float* s0,
                   const float* states, const float* rev, const void* d_o, const float* ds_final,
                   void* dq, void* dk, void* dv, float* dbeta, float* dgamma, float* ds0, void* ws,
                   size_t ws_bytes, void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  const bool bidir = chunk_len > 0;
  if (chunk_len < 0) return GDN_EINVAL;
  const int64_t n_rev = bidir && sh.T > 0 ? ((int64_t)sh.T + chunk_len - 1) / chunk_len : 0;
  if (n_rev > gdn::kMaxChunks) return GDN_EUNSUPPORTED;
  if (!grids_fit(sh, n_rev)) return GDN_EUNSUPPORTED;
  for (const void* p : {q, k, v, (const void*)s0, (const void*)states, (const void*)rev, d_o,
                        (const void*)ds_final, (const void*)dq, (const void*)dk, (const void*)dv,
                        (const void*)ds0})
    if (!aligned16(p)) return GDN_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (sh.BH() == 0) return GDN_OK;
  const int64_t DD = (int64_t)sh.D * sh.D;
  if (sh.T == 0) {
    // no frames: L depends on s0 only through S_{-1} = s0 = S_{T-1}
    if (ds0 == nullptr) return GDN_OK;
    GDN_MARK(GDN_PHASE_CALL_BEGIN, st);
    if (ds_final) GDN_HIP(gdn::launch_copy_f32(ds_final, ds0, sh.BH() * DD, st));
    else GDN_HIP(gdn::launch_zero_f32(ds0, sh.BH() * DD, st));
    GDN_MARK(GDN_PHASE_OTHER, st);
    return GDN_OK;
  }
  if (!q || !k || !v || !beta || !gamma || !states || !d_o) return GDN_EINVAL;
  if (bidir && !rev) return GDN_EINVAL;
  const BwdLayout L = bwd_layout(sh, n_rev);
  if (ws_bytes < L.total) return GDN_EWORKSPACE;
  if (ws == nullptr || ((uintptr_t)ws % kAlign) != 0) return GDN_EINVAL;
  const bool mfma = gdn::scan_uses_mfma(sh);  // layout of the internal terms and E
  float* terms = at<float>(ws, L.terms);
  float* part = at<float>(ws, L.partial);
  float* E = at<float>(ws, L.E);
  float* G = at<float>(ws, L.G);
  float* P = at<float>(ws, L.P);
  float* ginit = at<float>(ws, L.ginit);
  float* ones = at<float>(ws, L.ones);
  GDN_MARK(GDN_PHASE_CALL_BEGIN, st);
  // A_t of every frame (the U half is not needed), unless the workspace
  // still holds the forward call's terms: both layouts put them first, in the
  // same internal format, and nothing below writes there
  if (!sh.reuse_terms) {
    gdn::TermsOut direct{terms, nullptr, 2 * DD, 0};
    if (L.n_split == 1) {
      GDN_HIP(gdn::launch_terms(sh, k, v, beta, 1, direct, mfma, st));
    } else {
      gdn::TermsOut po{part, part + DD, (int64_t)L.n_split * 2 * DD, 2 * DD};
      GDN_HIP(gdn::launch_terms(sh, k, v, beta, L.n_split, po, false, st));
      GDN_HIP(gdn::launch_reduce_partials(sh, part, L.n_split, direct, mfma, st));
    }
    GDN_MARK(GDN_PHASE_BWD_TERMS, st);
  }
  // E_t = d_o_t^T q_t: the phase-1 contraction with q as prepared keys, d_o
  // as values and unit gates (the U half of its output)
  bool fused_dq = false;
  {
    Shape shq = sh;
    shq.prepared = 1;
    shq.c = 1.f;
    // with the RMSNorm of q, E_t uses the normalised queries (the generic
    // phase-1 kernel's mode 2: prepared keys normalised, no ReLU)
    shq.qk_norm = sh.qk_norm ? 2 : 0;
    gdn::TermsOut eout{nullptr, E, DD, 0};
    if ((dq != nullptr || sh.qk_norm) && gdn::edq_fused(shq)) {
      // one pass over q and d_o forms E_t and dq = (S_t [+ R_t])^T do together
      // (one workgroup per frame-head, whatever split phase 1 uses)
      GDN_HIP(gdn::launch_edq(shq, q, d_o, states, bidir ? rev : nullptr, dq, E, sh.qk_norm != 0, st));
      fused_dq = dq != nullptr;
    } else if (L.n_split == 1) {
      GDN_HIP(gdn::launch_fill_f32(ones, sh.FH() * sh.S, 1.f, st));
      GDN_HIP(gdn::launch_terms(shq, q, d_o, ones, 1, eout, mfma, st));
    } else {
      GDN_HIP(gdn::launch_fill_f32(ones, sh.FH() * sh.S, 1.f, st));
      gdn::TermsOut po{part, part + DD, (int64_t)L.n_split * 2 * DD, 2 * DD};
      GDN_HIP(gdn::launch_terms(shq, q, d_o, ones, L.n_split, po, false, st));
      GDN_HIP(gdn::launch_reduce_partials(shq, part, L.n_split, eout, mfma, st));
    }
    GDN_MARK(GDN_PHASE_BWD_EDQ, st);
  }
  GDN_HIP(gdn::launch_grad_init(sh, E, ds_final, ginit, mfma, st));
  // adjoint recurrence: frames T-1 .. 0 from G_{T-1}, adding E_{f-1} after
  // frame f's transition, so the state after frame f is G_{f-1} (stored in
  // slot f) and after frame 0 it is dL/dS0
  gdn::ScanParams pg;
  memset(&pg, 0, sizeof(pg));
  pg.terms = terms;
  pg.gamma = gamma;
  pg.T = sh.T;
  pg.nchunk = 1;
  pg.mode = gdn::SCAN_REVERSE;
  pg.usrc = E;
  pg.ushift = -1;
  pg.init = ginit;
  pg.init_bh_stride = DD;
  pg.states = G;
  pg.finA = ds0;
  pg.fin_bh_stride = DD;
  pg.fin_last_only = 1;
  pg.offsets[0] = 0;
  pg.offsets[1] = sh.T;
  gdn::RevGrad rg;
  if (bidir) {
    // adjoint of the reverse states, forward inside every chunk [a, e):
    // F_a = E_a and F_{t+1} = F_t M_t + E_{t+1}. The scan starts each chunk
    // from E_a, steps frames a .. e-1 adding E_{f+1} after frame f's
    // transition and stores F_{f+1} in slot f (the last step of a chunk
    // leaves a value nobody reads). Both adjoints need only E_t and the
    // terms: on the MFMA path they share one launch, the short chunks
    // running beside the long sequential chain of G.
    float* F = at<float>(ws, L.F);
    float* finit = at<float>(ws, L.finit);
    GDN_HIP(gdn::launch_chunk_init(sh, E, chunk_len, (int)n_rev, finit, mfma, st));
    GDN_MARK(GDN_PHASE_BWD_INIT, st);
    gdn::ScanParams pf;
    memset(&pf, 0, sizeof(pf));
    pf.terms = terms;
    pf.gamma = gamma;
    pf.T = sh.T;
    pf.nchunk = (int)n_rev;
    pf.mode = gdn::SCAN_FORWARD;
    pf.usrc = E;
    pf.ushift = 1;
    pf.init = finit;
    pf.init_bh_stride = n_rev * DD;
    pf.init_c_stride = DD;
    pf.states = F;
    for (int c = 0; c <= (int)n_rev; ++c)
      pf.offsets[c] = (int)std::min<int64_t>((int64_t)c * chunk_len, sh.T);
    if (gdn::scan_pairs(sh)) {
      GDN_HIP(gdn::launch_scan_pair(sh, pg, pf, st));
    } else {
      GDN_HIP(gdn::launch_scan(sh, pg, st));
      GDN_HIP(gdn::launch_scan(sh, pf, st));
    }
    GDN_MARK(GDN_PHASE_BWD_ADJOINT, st);
    rg.rev = rev;
    rg.fbuf = F;
    rg.finit = finit;
    rg.L = chunk_len;
    rg.nchunk = (int)n_rev;
  } else {
    GDN_MARK(GDN_PHASE_BWD_INIT, st);
    GDN_HIP(gdn::launch_scan(sh, pg, st));
    GDN_MARK(GDN_PHASE_BWD_ADJOINT, st);
  }
  GDN_HIP(gdn::launch_frame_grad(sh, states, s0, G, ginit, terms, mfma, gamma, P, dgamma, rg, st));
  GDN_MARK(GDN_PHASE_BWD_FRAME, st);
  if (dq || dk || dv || dbeta) {
    GDN_HIP(gdn::launch_token_grad(sh, q, k, v, beta, d_o, states, bidir ? rev : nullptr, G, ginit,
                                   P, fused_dq ? nullptr : dq, dk, dv, dbeta, st));
    GDN_MARK(GDN_PHASE_BWD_TOKEN, st);
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_scan_bwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                        const float* beta, const float* gamma, const float* s0,
                        const float* states, const void* d_o, const float* ds_final, void* dq,
                        void* dk, void* dv, float* dbeta, float* dgamma, float* ds0, void* ws,
                        size_t ws_bytes, void* stream) {
  return run_bwd(desc, 0, q, k, v, beta, gamma, s0, states, nullptr, d_o, ds_final, dq, dk, dv,
                 dbeta, dgamma, ds0, ws, ws_bytes, stream);
}

gdn_status gdn_scan_bidir_chunked_bwd(const gdn_desc* desc, int32_t chunk_len, const void* q,
                                      const void* k, const void* v, const float* beta,
                                      const float* gamma, const float* s0,
                                      const float* states_fwd, const float* states_rev,
                                      const void* d_o, const float* ds_final, void* dq, void* dk,
                                      void* dv, float* dbeta, float* dgamma, float* ds0, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (chunk_len < 1) return GDN_EINVAL;
  return run_bwd(desc, chunk_len, q, k, v, beta, gamma, s0, states_fwd, states_rev, d_o, ds_final,
                 dq, dk, dv, dbeta, dgamma, ds0, ws, ws_bytes, stream);
}

gdn_status gdn_readout(const gdn_desc* desc, const void* q, const float* states,
                       const float* states_add, void* o, void* stream) {
  Shape sh;
  gdn_status s = check_desc(desc, &sh);
  if (s != GDN_OK) return s;
  if (sh.FH() == 0) return GDN_OK;
  if (!q || !states || !o) return GDN_EINVAL;
  if (!aligned16(q) || !aligned16(states) || !aligned16(states_add) || !aligned16(o))
    return GDN_EINVAL;
  GDN_MARK(GDN_PHASE_CALL_BEGIN, (hipStream_t)stream);
  GDN_HIP(gdn::launch_readout(sh, q, states, states_add, o, (hipStream_t)stream));
  GDN_MARK(GDN_PHASE_READOUT, (hipStream_t)stream);
  return GDN_OK;
}

}  // extern "C"
