/*
 * gdn.h -- C ABI of libgdn, the frame-wise Gated DeltaNet (GDN) frame scan for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (blog.hotdry.top SANA-WM post, section "混合线性注意力", the
 * three equations; xiejiayun.github.io "好文共赏 | SANA-WM", section 2.1):
 *
 *   K_hat = ReLU(k) * c,            c = 1/sqrt(D*S) unless given
 *   A_t   = K_t beta_t K_t^T         (D x D; K_t has the frame's S tokens as columns)
 *   U_t   = V_t beta_t K_t^T         (D x D; rows = value dim, cols = key dim)
 *   M_t   = gamma_t (I - A_t)
 *   S_t   = S_{t-1} M_t + U_t,       S_{-1} = s0 (zero when s0 is NULL)
 *   o_{t,s} = S_t q_{t,s}            (readout with the state after frame t)
 *
 * Memory layouts (row-major, last index fastest; all device memory unless
 * marked "host"):
 *   q, k, v, o, k_hat : [B, H, T, S, D]  element type io_dtype (fp32 or bf16)
 *   beta              : [B, H, T, S]     fp32, per-token gate
 *   gamma             : [B, H, T]        fp32, per-frame decay gate
 *   s0, s_final       : [B, H, D, D]     fp32, entry (i, j) = (value dim, key dim)
 *   states, states_*  : [B, H, T, D, D]  fp32, the state after each frame
 *   A, U              : [B, H, T, D, D]  fp32
 *   C, Hc, s_start    : [B, H, P, D, D]  fp32
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every buffer, the workspace included. The
 *     library allocates and frees no device memory and keeps no global state
 *     (apart from the opt-in per-thread phase trace, gdn_trace_set); calls are
 *     re-entrant.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream). Work is
 *     only enqueued on it; no call synchronises.
 *   - Errors: arguments are checked on the host before anything is enqueued.
 *     On any status other than GDN_OK nothing has been enqueued, except for
 *     GDN_EHIP (a launch failed; earlier launches of the same call may have
 *     been enqueued). Device faults surface at the caller's next
 *     synchronisation, as usual in HIP.
 *   - Outputs are overwritten, never accumulated into. A NULL optional output
 *     is not computed. Output buffers must not alias inputs.
 *   - Determinism: the same call on the same device gives bitwise-identical
 *     results (no atomics, fixed reduction orders).
 *   - Supported shapes: B, H, T >= 0, S >= 1. D = 128 with bf16 runs the MFMA
 *     path; D in {16, 32, 64} (bf16 or fp32) and D = 128 with fp32 run the
 *     fp32 vector path. Other D give GDN_EUNSUPPORTED. Every kernel launch
 *     must stay below 2^32 work-items, which bounds a call to about
 *     B*H*T < 2^20 frame-heads (and B*H*T*S*D < 2^32 on the fp32 vector path)
 *     and B*H times the number of time or reverse chunks below 2^19; larger
 *     calls give GDN_EUNSUPPORTED before anything is enqueued (split them
 *     over batch, heads or calls).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

typedef enum {
  GDN_OK = 0,
  GDN_EINVAL = 1,        /* NULL required pointer, bad size, bad dtype, bad chunking */
  GDN_EUNSUPPORTED = 2,  /* valid request the library does not implement (e.g. D) */
  GDN_EWORKSPACE = 3,    /* ws_bytes smaller than gdn_workspace_bytes() asks for */
  GDN_EHIP = 4           /* a HIP launch failed */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* flags (may be combined with |) */
#define GDN_KEYS_RAW 0u       /* kernels apply ReLU and the key scale to k */
#define GDN_KEYS_PREPARED 1u  /* k already holds K_hat; no ReLU, no scale */
/* RMS-normalise every token of q, and of k unless GDN_KEYS_PREPARED, over the
 * head dim before use: x / sqrt(mean_d x_d^2 + 1e-6), unit weight, ahead of
 * the key's ReLU and scale. The RMSNorm of the fused operator in
 * blog.hotdry.top SANA-WM post, section "显存分片: Context-Parallel 的工程实现";
 * the pages give no axis, epsilon or weight, so these are this library's
 * reading. Fused into the kernels' load paths (no extra HBM pass). */
#define GDN_QK_RMSNORM 2u
/* Backward calls only (forward calls ignore it): the workspace passed to the
 * backward already holds the phase-1 terms of the forward call that produced
 * its states, and A_t is read from there instead of being recomputed (one
 * pass over k and beta less). That forward call (gdn_scan_fwd,
 * gdn_scan_bidir_chunked or gdn_step) must have used this same workspace
 * buffer, the same k and beta, and a descriptor that differs from the
 * backward's in this bit alone, and nothing may have written to the buffer
 * since. Size it for both calls: the larger of gdn_workspace_bytes(desc, P)
 * and the backward's own query. The phase-1 terms occupy the same leading
 * bytes in both layouts. If the buffer does not hold those terms, the
 * gradients are wrong (every access still stays inside the workspace). */
#define GDN_REUSE_FWD_TERMS 4u

#define GDN_MAX_TIME_CHUNKS 256

typedef struct {
  int32_t B, H, T, S, D;  /* batch, heads, frames, tokens per frame, head dim (Dk = Dv) */
  int32_t io_dtype;       /* gdn_dtype of q, k, v, o, k_hat */
  float key_scale;        /* <= 0 selects 1/sqrt(D*S) */
  uint32_t flags;         /* GDN_KEYS_RAW or GDN_KEYS_PREPARED, optionally | GDN_QK_RMSNORM,
                           * | GDN_REUSE_FWD_TERMS (backward calls) */
} gdn_desc;

/* Human-readable name of a status code (static string; never NULL). */
GDN_API const char* gdn_status_str(int32_t status);

/* Workspace size in bytes that every entry point below needs for `desc` and
 * `n_time_chunks` (1 = sequential scan). Host-only; enqueues nothing.
 * Returns GDN_EINVAL / GDN_EUNSUPPORTED for a bad descriptor (then *bytes is
 * left unchanged). */
GDN_API gdn_status gdn_workspace_bytes(const gdn_desc* desc, int32_t n_time_chunks, size_t* bytes);

/* K_hat = ReLU(k) * c (with GDN_QK_RMSNORM: ReLU(k / rms(k)) * c, per token),
 * written in io_dtype (bf16: round to nearest even of the fp32 product). Key scaling: blog.hotdry.top SANA-WM post,
 * section "混合线性注意力", paragraph on the 1/sqrt(D*S) factor. Requires
 * flags = GDN_KEYS_RAW. k and k_hat: [B,H,T,S,D]; may not overlap. */
GDN_API gdn_status gdn_prepare(const gdn_desc* desc, const void* k, void* k_hat, void* stream);

/* Phase 1 alone: A_t = K_t beta_t K_t^T and U_t = V_t beta_t K_t^T for every
 * frame of every head (same section, the M_t and U_t equations). A and U are
 * [B,H,T,D,D] fp32; either may be NULL. */
GDN_API gdn_status gdn_frame_terms(const gdn_desc* desc, const void* k, const void* v, const float* beta,
                           float* A, float* U, void* ws, size_t ws_bytes, void* stream);

/* Causal frame scan S_t = S_{t-1} M_t + U_t with readout o = S_t q (same
 * section). n_time_chunks = 1 scans frames one after another; P > 1 splits
 * the frames into P chunks at offsets floor(p*T/P), forms each chunk's affine
 * composite (C_p, H_p) in parallel, combines them into exact chunk start states
 * and replays the chunks in parallel (blog.hotdry.top SANA-WM post, section
 * "显存分片: Context-Parallel 的工程实现", S_end = S_start C_p + H_p). Requires
 * 1 <= P <= max(T, 1) and P <= GDN_MAX_TIME_CHUNKS.
 * q may be NULL when o is NULL. s0 NULL = zero initial state. states,
 * s_final, o may each be NULL. */
GDN_API gdn_status gdn_scan_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                        const float* beta, const float* gamma, const float* s0, float* states,
                        float* s_final, void* o, int32_t n_time_chunks, void* ws, size_t ws_bytes,
                        void* stream);

/* Chunk-causal bidirectional scan (hyper.ai page 2605.15178, method section:
 * the reverse temporal scan restarts at every chunk boundary). Forward states
 * as gdn_scan_fwd; reverse states R_t = R_{t+1} M_t + U_t inside each chunk
 * [a, a+L) (chunks start at frame 0, the last one may be short), starting from
 * zero after the chunk's last frame; readout o = (S_t + R_t) q.
 * chunk_len >= T gives the full-sequence bidirectional scan. chunk_len >= 1.
 * states_fwd, states_rev, s_final, o may each be NULL. */
GDN_API gdn_status gdn_scan_bidir_chunked(const gdn_desc* desc, const void* q, const void* k,
                                  const void* v, const float* beta, const float* gamma,
                                  const float* s0, int32_t chunk_len, float* states_fwd,
                                  float* states_rev, float* s_final, void* o,
                                  int32_t n_time_chunks, void* ws, size_t ws_bytes, void* stream);

/* Streaming chunk step: one block of desc->T frames, bidirectional inside the
 * block (the reverse scan covers the whole block), with the causal forward
 * state carried from block to block. This is how the released chunk-causal
 * model runs (trdm.cn SANA-WM guide, sections 四.3 and 七: blocks of
 * num_frame_per_block = 3 latent frames, chunk_size 3). S_{-1} = carry_in
 * (NULL = zero state); carry_out receives S_{T-1} of the block; o, states_fwd
 * and states_rev are the block's outputs as in gdn_scan_bidir_chunked.
 * Equivalent to gdn_scan_bidir_chunked(chunk_len = T, n_time_chunks = 1,
 * s0 = carry_in, s_final = carry_out): cutting a sequence into blocks of L
 * frames and stepping through them gives the chunk-causal scan with
 * chunk_len = L. carry_in and carry_out may be the same buffer (each state
 * row is read before it is rewritten); no other output may alias an input.
 * Workspace: gdn_workspace_bytes(desc, 1). */
GDN_API gdn_status gdn_step(const gdn_desc* desc, const void* q, const void* k, const void* v,
                            const float* beta, const float* gamma, const float* carry_in,
                            float* carry_out, void* o, float* states_fwd, float* states_rev,
                            void* ws, size_t ws_bytes, void* stream);

/* Size of the device scratch array that gdn_step_noalloc uses in place of a
 * workspace: one copy per GPU the library runs on, held until the process
 * ends. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_step without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as gdn_step
 * (bitwise the same outputs), but the workspace is the library's own static
 * device array of GDN_NOALLOC_SCRATCH_BYTES: shapes whose
 * gdn_workspace_bytes(desc, 1) exceeds it give GDN_EWORKSPACE before anything
 * is enqueued (16 heads at S = 3600, D = 128, bf16: blocks of up to 6 frames fit).
 * The call allocates nothing; the array's device address is looked up once
 * per device, on that device's first call. `stream` must belong to the
 * current device (else GDN_EINVAL). Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other host threads, or streams that
 * are not ordered with each other) race and give wrong results; calls
 * ordered on one stream are safe. */
GDN_API gdn_status gdn_step_noalloc(const gdn_desc* desc, const void* q, const void* k,
                                    const void* v, const float* beta, const float* gamma,
                                    const float* carry_in, float* carry_out, void* o,
                                    float* states_fwd, float* states_rev, void* stream);

/* Affine composites of explicit time chunks (blog.hotdry.top SANA-WM post,
 * section "显存分片: Context-Parallel 的工程实现"): for chunk p = [a_p, a_{p+1}),
 * C_p = M_{a_p} ... M_{a_{p+1}-1} (ordered product) and H_p = the chunk scanned
 * from a zero state, so that S_end = S_start C_p + H_p. chunk_offsets is a
 * HOST array of P+1 ascending ints with [0] = 0 and [P] = T (empty chunks
 * allowed: C = I, H = 0). 1 <= P <= GDN_MAX_TIME_CHUNKS. When s_start is not
 * NULL it receives the exact chunk start states s_start[0] = s0 (or zero),
 * s_start[p+1] = s_start[p] C_p + H_p. C and Hc may each be NULL. */
GDN_API gdn_status gdn_compose(const gdn_desc* desc, const void* k, const void* v, const float* beta,
                       const float* gamma, const int32_t* chunk_offsets, int32_t P, float* C,
                       float* Hc, const float* s0, float* s_start, void* ws, size_t ws_bytes,
                       void* stream);

/* Workspace in bytes that gdn_scan_bwd needs for `desc`. Host-only. */
GDN_API gdn_status gdn_bwd_workspace_bytes(const gdn_desc* desc, size_t* bytes);

/* Backward pass of the causal frame scan (gdn_scan_fwd): reverse-mode
 * gradients of L = sum <d_o, o> + <ds_final, S_{T-1}> through the rule of
 * blog.hotdry.top SANA-WM post, section "混合线性注意力". With
 * G_t = dL/dS_t: G_{T-1} = E_{T-1} + ds_final, G_t = E_t + G_{t+1} M_{t+1}
 * (E_t = d_o_t^T q_t, M symmetric), and per frame dM_t = S_{t-1}^T G_t,
 * dgamma_t = <dM_t, I - A_t>; per token dq = S_t^T do,
 * dk_hat = beta ((dA + dA^T) k_hat + G_t^T v) with dA = -gamma_t dM_t,
 * dv = beta G_t k_hat, dbeta = k_hat^T dA k_hat + v^T G_t k_hat; raw keys
 * then get the key scale and the ReLU mask (zero where k <= 0).
 * Inputs: the forward's q, k, v, beta, gamma, s0 (NULL = zero) and its
 * per-frame states [B,H,T,D,D] (required), d_o [B,H,T,S,D] (io dtype,
 * required), ds_final [B,H,D,D] (NULL = zero). Outputs (each may be NULL):
 * dq, dk, dv [B,H,T,S,D] (io dtype), dbeta [B,H,T,S], dgamma [B,H,T],
 * ds0 [B,H,D,D] (fp32). The adjoint recurrence runs sequentially over the
 * frames. With GDN_QK_RMSNORM, E_t and the readout use the normalised
 * queries and the raw keys are normalised before their ReLU (as in the
 * forward call); dq and dk then pass back through the norm, dx =
 * r (dy - (y . dy) y / D) with y = x r, r = 1 / rms(x).
 * Workspace: gdn_bwd_workspace_bytes; with GDN_REUSE_FWD_TERMS, the forward
 * call's workspace (see that flag). */
GDN_API gdn_status gdn_scan_bwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                const float* beta, const float* gamma, const float* s0,
                                const float* states, const void* d_o, const float* ds_final,
                                void* dq, void* dk, void* dv, float* dbeta, float* dgamma,
                                float* ds0, void* ws, size_t ws_bytes, void* stream);

/* Workspace in bytes that gdn_scan_bidir_chunked_bwd needs for `desc` and
 * `chunk_len` (>= 1). Host-only. */
GDN_API gdn_status gdn_bidir_bwd_workspace_bytes(const gdn_desc* desc, int32_t chunk_len,
                                                 size_t* bytes);

/* Backward pass of the chunk-causal bidirectional scan
 * (gdn_scan_bidir_chunked; hyper.ai paper page 2605.15178, method section:
 * the reverse scan restarts at every chunk boundary): gradients of
 * L = sum <d_o, o> + <ds_final, S_{T-1}> with o = (S_t + R_t) q. The causal
 * adjoint G is that of gdn_scan_bwd; the reverse states R get their own
 * adjoint, forward in time inside each chunk [a, e): F_a = E_a,
 * F_t = E_t + F_{t-1} M_{t-1}. Then dU_t = G_t + F_t,
 * dM_t = S_{t-1}^T G_t + R_{t+1}^T F_t (the second term only when t + 1 < e),
 * dq = (S_t + R_t)^T do, and the per-frame and per-token rules of
 * gdn_scan_bwd with dU_t in place of G_t.
 * Inputs: as gdn_scan_bwd plus chunk_len (>= 1, as in the forward call) and
 * the forward's states_fwd and states_rev [B,H,T,D,D] (both required).
 * Outputs as gdn_scan_bwd (each may be NULL). More than 256 chunks:
 * GDN_EUNSUPPORTED. GDN_QK_RMSNORM as in gdn_scan_bwd.
 * Workspace: gdn_bidir_bwd_workspace_bytes; with GDN_REUSE_FWD_TERMS, the
 * forward call's workspace (see that flag). */
GDN_API gdn_status gdn_scan_bidir_chunked_bwd(const gdn_desc* desc, int32_t chunk_len,
                                              const void* q, const void* k, const void* v,
                                              const float* beta, const float* gamma,
                                              const float* s0, const float* states_fwd,
                                              const float* states_rev, const void* d_o,
                                              const float* ds_final, void* dq, void* dk, void* dv,
                                              float* dbeta, float* dgamma, float* ds0, void* ws,
                                              size_t ws_bytes, void* stream);

/* Phase 3 alone: o_{t,s} = (states_t + states_add_t) q_{t,s} for every token
 * of every frame (states_add may be NULL). The readout with the state after
 * frame t is this library's reading of the frame-wise rule (the pages give the
 * token-level Gated DeltaNet of xiejiayun.github.io "好文共赏 | SANA-WM",
 * section 2.1, whose output uses the updated state). bf16 io: the summed state
 * is rounded to bf16 once and products accumulate in fp32. q, o: [B,H,T,S,D];
 * states, states_add: [B,H,T,D,D] fp32. */
GDN_API gdn_status gdn_readout(const gdn_desc* desc, const void* q, const float* states,
                               const float* states_add, void* o, void* stream);

/* Phase timing (tracing). A caller that wants per-phase device times sets a
 * trace on its host thread; from then on every call made on that thread
 * records, on the call's own stream, one caller-created hipEvent_t when it
 * starts enqueueing (phase GDN_PHASE_CALL_BEGIN) and one after each launch
 * group, tagged with the phase that group ran, so that the elapsed time
 * between events[i-1] and events[i] is the device time of phases[i]. The
 * events must have been created with timing enabled; the library only
 * records them. When `capacity` events have been recorded, further marks are
 * dropped (the call itself is unaffected). A call that fails its argument
 * checks records nothing. gdn_trace_set(NULL) stops tracing on the thread.
 * This per-thread pointer is the only state the library keeps; the trace
 * struct and its arrays belong to the caller and must outlive the traced
 * calls. A call inside HIP graph capture records its events into the graph
 * like any other work (do not trace such calls). */
typedef enum {
  GDN_PHASE_CALL_BEGIN = 0,   /* a call started enqueueing */
  GDN_PHASE_TERMS = 1,        /* phase 1: A_t and U_t of every frame */
  GDN_PHASE_TERMS_REDUCE = 2, /* sum of phase 1's split partials (calls with few frame-heads) */
  GDN_PHASE_SCAN = 3,         /* first scan launch: the sequential scan or the composites
                               * (with the reverse chunk scan when they share the launch) */
  GDN_PHASE_COMBINE = 4,      /* chunk start states from the composites */
  GDN_PHASE_REPLAY = 5,       /* every time chunk replayed from its start state */
  GDN_PHASE_REVERSE = 6,      /* the reverse chunk scan in a launch of its own */
  GDN_PHASE_READOUT = 7,      /* o = (S_t [+ R_t]) q */
  GDN_PHASE_BWD_TERMS = 8,    /* backward: A_t recomputed */
  GDN_PHASE_BWD_EDQ = 9,      /* backward: E_t = d_o^T q (and dq in the same pass) */
  GDN_PHASE_BWD_INIT = 10,    /* backward: adjoint start values */
  GDN_PHASE_BWD_ADJOINT = 11, /* backward: adjoint recurrences */
  GDN_PHASE_BWD_FRAME = 12,   /* backward: per-frame gradients dM_t, dgamma, P_t */
  GDN_PHASE_BWD_TOKEN = 13,   /* backward: per-token gradients dk, dv, dbeta (dq) */
  GDN_PHASE_OTHER = 14        /* copies and fills */
} gdn_phase;

typedef struct {
  void** events;      /* capacity hipEvent_t handles, created by the caller */
  int32_t* phases;    /* capacity entries, written: phases[i] = gdn_phase of events[i] */
  int32_t capacity;
  int32_t count;      /* events recorded so far (the caller may reset it to 0) */
} gdn_trace;

/* Sets (or with NULL clears) the trace of the calling host thread. Returns
 * GDN_EINVAL for a trace with NULL arrays or a negative capacity or count. */
GDN_API gdn_status gdn_trace_set(gdn_trace* trace);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
