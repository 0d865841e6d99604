// Phase 1: per-frame terms A_t = K_t beta_t K_t^T and U_t = V_t beta_t K_t^T.
//
// Source: blog.hotdry.top SANA-WM post, section "混合线性注意力" (the M_t and U_t
// equations); keys K_hat = ReLU(k) / sqrt(D*S) from the same section.
//
// With tokens as rows (k, v are [S, D] per frame), both products contract over
// the S tokens of a frame:
//   [A; U] (2D x D) = [R^T; V^T] (2D x S) * (beta . R) (S x D),  R = ReLU(k)
// followed by the scales c^2 (A rows) and c (U rows) in fp32. Every frame-head
// is independent, so the grid is frame-parallel.
//
// MFMA path (bf16, D = 128): terms_dma_bf16_d128 below; any other shape runs
// the fp32 vector path terms_generic.
#include <algorithm>
#include <type_traits>

#include "gdn_common.h"
#include "gdn_dma.h"

namespace gdn {

namespace {

// MFMA path. Phase 1 is bound by the HBM reads of k and v. With the loads
// staged through registers (two workgroups per CU, about 64 KB outstanding)
// the stream reached about 5 TB/s, while a plain read stream with more in
// flight reaches about 7 TB/s. Here the loads bypass registers: global_load_lds_dwordx4
// copies 16 bytes per lane straight into a ring of kNst LDS stages (32 tokens
// of k and v each), so kNst - 1 stages stay in flight while one is consumed.
// MFMA fragments (eight consecutive tokens of one feature) are read with
// ds_read_b64_tr_b16, which returns, for each 16-lane group, the columns of
// the 4 x 16 block its lanes address: two reads give a lane its eight tokens.
// A per-stage transform pass forms ReLU(k) in place and bf16(beta . ReLU(k))
// (beta rides along in the same ring). 8 waves: wave w owns output columns
// 32(w%4)..+32 and the 128 rows of A (w < 4) or of U (w >= 4), as four
// 32 x 32 tiles.
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Three stages (two in flight while one is consumed) keep two workgroups per
// CU within the LDS (2 x 65920 B); on MI355X phase 1 ran 8 % faster than with
// two stages, and four stages (one workgroup per CU) were no faster than two.
#ifndef GDN_TERMS_NST
#define GDN_TERMS_NST 3
#endif
constexpr int kTsd = 32;                        // tokens per stage
constexpr int kNst = GDN_TERMS_NST;             // stages in the ring
constexpr int kKvBytes = kTsd * 256;            // one stage of k (or v): 32 rows x 256 B

// LDS layout of a stage tensor: token block b (tokens 4b..4b+3) occupies
// bytes [1024 b, 1024 b + 1024), chunk-major inside: 16-byte chunk c (features
// 8c..8c+7) of token 4b+e sits at 1024 b + 64 c + 16 e. One DMA instruction
// fills one block from four contiguous 256-byte token rows; a transposed read
// by a 16-lane group (4 tokens x 16 features) covers 128 contiguous bytes, and
// every fragment address is a per-lane base plus a compile-time offset.
__device__ __forceinline__ int tr_lane_base(int lane) {
  const int G = lane >> 4;
  const int j = lane & 15;
  return 2048 * (G >> 1) + 64 * (2 * (G & 1) + ((j & 3) >> 1)) + 16 * (j >> 2) + 8 * (j & 1);
}



// One MFMA operand fragment: lane gets the 8 consecutive tokens
// k0 + 8*(lane/32) + 0..7 of feature f0 + (lane % 32) (k0 % 16 == 0,
// f0 % 32 == 0), from the stage tensor at `base`, `lb` = tr_lane_base(lane).
__device__ __forceinline__ uint4 tr_frag(const uint8_t* base, int lb, int k0, int f0) {
  const uint8_t* p = base + lb + 256 * k0 + 8 * f0;
  const v4i16_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDN_LDS v4i16_t*)(p));
  const v4i16_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDN_LDS v4i16_t*)(p + 1024));
  const uint2 a = __builtin_bit_cast(uint2, r0);
  const uint2 b = __builtin_bit_cast(uint2, r1);
  return make_uint4(a.x, a.y, b.x, b.y);
}

#if GDN_TERMS_NST <= 3
#define GDN_TERMS_WAVES_PER_EU 4  // two 8-wave workgroups per CU: at most 128 VGPRs
#else
#define GDN_TERMS_WAVES_PER_EU 2  // one workgroup per CU (its ring fills the LDS)
#endif
// kAOnly: only A_t is wanted (U_t is not written), so v is never read: the
// copies move k and the gates only and the U waves skip the products.
//
// kDq (backward pass): k holds the queries, v the output gradients d_o, and
// the gates are 1, so U = d_o^T q is E_t; the A waves instead form the query
// gradient dq_s = S_t^T do_s of every token of the stage from S_t^T staged
// in LDS, so d_o is read once for both. Waves 4-7 issue all copies (their
// vmcnt then counts copies only and the explicit waits stay exact) and
// waves 0-3 issue all dq stores; wbuf (unused without gates) stages each
// stage's dq tile so that the stores are whole 256-byte rows.
#ifndef GDN_EDQ_NST
#define GDN_EDQ_NST 6
#endif
// Ring stages of the A-only mode (k alone: half-size slots). On MI355X the
// 60 s 720p layer's recompute took 371-374 us with 4 stages, 376-378 us with
// 6, 379 us with 7 and 453-460 us with 8 (one workgroup per CU); 4 stages at
// three workgroups per CU spilled registers and took 825 us.
#ifndef GDN_AONLY_NST
#define GDN_AONLY_NST 4
#endif
template <bool kScanLayout, bool kPrepared, bool kNorm, bool kAOnly, bool kDq>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(kDq ? 2 : GDN_TERMS_WAVES_PER_EU, kDq ? 2 : GDN_TERMS_WAVES_PER_EU)))
terms_dma_bf16_d128(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const float* __restrict__ beta, int S, int n_split, float c,
                    TermsOut out, const float* __restrict__ sdq, const float* __restrict__ sdq2,
                    uint16_t* __restrict__ dq) {
  constexpr int D = 128;
  static_assert(!kDq || (kScanLayout && kPrepared && !kAOnly), "dq mode of the E pass");
  // ring slot: k block, v block, then the stage's 32 gates; wbuf[st % 2]
  // holds the second operand bf16(beta . ReLU(k)) of stage st
  // Without v a slot is half as large, and the same LDS holds twice the stages.
  constexpr int kNs = kDq ? (kNorm ? GDN_EDQ_NST - 1 : GDN_EDQ_NST) : (kAOnly ? GDN_AONLY_NST : kNst);
  constexpr int kGateOff = (kAOnly ? 1 : 2) * kKvBytes;
  constexpr int kSlot = kGateOff + 4 * kTsd;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kNs][kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf[2][kKvBytes];
  __shared__ uint4 Sl[kDq ? D * 16 : 1];  // kDq: S_t^T in bf16, row i = column i of S_t
  // kDq with the RMSNorm of q: the stage's normalised queries in the staging
  // layout of dq (for the norm's backward) and 1 / rms per token
  __shared__ __attribute__((aligned(16))) uint8_t qstg[kDq && kNorm ? 2 : 1][kDq && kNorm ? kKvBytes : 16];
  __shared__ float rqs[kDq && kNorm ? 3 : 1][kTsd];

  const int64_t fh = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int stages = (S + kTsd - 1) / kTsd;
  const int st_begin = (int)(((int64_t)split * stages) / n_split);
  const int st_end = (int)(((int64_t)(split + 1) * stages) / n_split);
  // last token the copies may touch: the ring's prefetch past this
  // workgroup's range re-reads it instead of the next range's tokens
  const int tok_last = max(min(st_end * kTsd, S) - 1, 0);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const uint16_t* kf = k + fh * (int64_t)S * D;
  const uint16_t* vf = v + fh * (int64_t)S * D;
  const float* bf = kDq ? nullptr : beta + fh * (int64_t)S;

  // S_t^T -> LDS (kDq; S_t + R_t with the reverse states of the bidirectional
  // scan), 16-byte chunk ch of row i at chunk position ch ^ (i % 8)
  if (kDq) {
    const float* s1 = sdq + fh * D * D;
    const float* s2 = sdq2 ? sdq2 + fh * D * D : nullptr;
#pragma unroll
    for (int u = 0; u < D * 16 / 512; ++u) {
      const int cidx = tid + 512 * u;
      const int i = cidx >> 4, ch = cidx & 15;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = s1[(int64_t)(8 * ch + e) * D + i] + (s2 ? s2[(int64_t)(8 * ch + e) * D + i] : 0.f);
      Sl[i * 16 + (ch ^ (i & 7))] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
    }
  }

  // DMA of stage `st` into its ring slot: wave w copies tokens 4w..4w+3 of
  // k and of v (one 1 KB instruction each; k only when kAOnly) and their 4
  // gates. Lane L of a
  // copy instruction fills LDS slot L of its block: chunk L/4 of token
  // 4w + L%4. Tokens past the end of the range are clamped to its last
  // token (valid memory); past the frame's end their gate is zeroed by the
  // transform pass, and stages past the range are never consumed.
  const int dtok = 4 * wave + (lane & 3);            // token within the stage
  const int dchunk = lane >> 2;
  constexpr int kOps = kDq ? 4 : (kAOnly ? 2 : 3);  // copy instructions per (copying) wave and stage
  auto issue = [&](int st) {
    uint8_t* slot = ring[st % kNs];
    if (kDq) {  // waves 4-7: token blocks 2 (w - 4) and 2 (w - 4) + 1 of q and d_o
      if (wave >= 4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int blk = 2 * (wave - 4) + h;
          const int t = min(st * kTsd + 4 * blk + (lane & 3), S - 1);
          const int64_t off = (int64_t)t * D + 8 * dchunk;
          dma16(kf + off, slot + 1024 * blk);
          dma16(vf + off, slot + kKvBytes + 1024 * blk);
        }
      }
      return;
    }
    const int t = min(st * kTsd + dtok, tok_last);
    const int64_t off = (int64_t)t * D + 8 * dchunk;
    dma16(kf + off, slot + 1024 * wave);
    if (!kAOnly) dma16(vf + off, slot + kKvBytes + 1024 * wave);
    dma4(bf + t, slot + kGateOff + 16 * wave, lane < 4);
  };
  const int lb = tr_lane_base(lane);

  // Transform pass: thread i owns bytes [16 i, 16 i + 16) of the k block,
  // i.e. chunk (i % 64) / 4 of token 4 (i / 64) + i % 4: exactly the bytes
  // (and the gate) that lane i % 64 of its own wave copied, so it needs only
  // its own wave's copies to have landed. It applies ReLU in place (the first
  // operand of the A rows) and writes bf16(beta . ReLU(k)) to wbuf[st % 2]
  // (the second operand of every row).
  const int ttok = 4 * (tid >> 6) + (tid & 3);       // == dtok
  auto transform = [&](int st) {
    uint8_t* Ks = ring[st % kNs];
    const float* gates = (const float*)(Ks + kGateOff);
    uint4 x = *(const uint4*)(Ks + 16 * tid);
    const float b = (st * kTsd + ttok < S) ? gates[ttok] : 0.f;
    if (kNorm && !kPrepared) {
      // RMSNorm of the raw key over its 128 features: the token's 16 chunks
      // sit in the lanes congruent to this one mod 4 of the same wave
      const uint32_t w0[4] = {x.x, x.y, x.z, x.w};
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) ss = sumsq_bf16x2(w0[q], ss);
      const float r = rms_inv(sum_lanes_mod4(ss), D);
      uint32_t kq[4], o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t z = relu_bf16x2_pk(w0[q]);
        const float lo = __uint_as_float(z << 16) * r, hi = __uint_as_float(z & 0xFFFF0000u) * r;
        kq[q] = pack_bf16x2(lo, hi);         // first operand of the A rows: ReLU(k) / rms(k)
        o[q] = pack_bf16x2(lo * b, hi * b);  // beta . ReLU(k) / rms(k), rounded once
      }
      *(uint4*)(Ks + 16 * tid) = make_uint4(kq[0], kq[1], kq[2], kq[3]);
      *(uint4*)(wbuf[st & 1] + 16 * tid) = make_uint4(o[0], o[1], o[2], o[3]);
      return;
    }
    if (!kPrepared) {
      x.x = relu_bf16x2_pk(x.x);
      x.y = relu_bf16x2_pk(x.y);
      x.z = relu_bf16x2_pk(x.z);
      x.w = relu_bf16x2_pk(x.w);
      *(uint4*)(Ks + 16 * tid) = x;
    }
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(__uint_as_float(w[q] << 16) * b, __uint_as_float(w[q] & 0xFFFF0000u) * b);
    *(uint4*)(wbuf[st & 1] + 16 * tid) = make_uint4(o[0], o[1], o[2], o[3]);
  };

  // Wave w: output column tile nt = w % 4 (columns 32nt..32nt+31) and the four
  // 32-row tiles of A (waves 0-3, first operand ReLU(k)) or of U (waves 4-7,
  // first operand v).
  const int nt = wave & 3;
  const bool rowsK = wave < 4;
  // the v block sits kKvBytes = 1024 eight-byte feature slots after the k block
  const int aoff = rowsK ? 0 : kKvBytes / 8;
  f32x16_t acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[mt][q] = 0.f;

  auto compute = [&](int st) {
    const uint8_t* Ks = ring[st % kNs];
#pragma unroll
    for (int kk = 0; kk < kTsd / 16; ++kk) {
      const int k0 = 16 * kk;
      uint4 fa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) fa[mt] = tr_frag(Ks, lb, k0, aoff + 32 * mt);
      // kDq: the gates are 1 and the keys prepared, so the second operand is q itself
      const uint4 fb = tr_frag(kDq ? Ks : wbuf[st & 1], lb, k0, 32 * nt);
      const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, fb);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[mt]), bw,
                                                          acc[mt], 0, 0, 0);
    }
  };

  // kDq, waves 0-3: the dq tile of stage st (its 32 tokens x features
  // 32 w .. 32 w + 31) as (dq^T) = S_t^T . do^T on MFMA: the first operand is
  // row i of S_t^T, the second token l32's d_o chunk, both 16-byte LDS reads.
  // Lane (half, l32) ends with features 32 w + 8 jg + 4 half + 0..3 of token
  // l32 and drops them, in bf16, into wbuf[st % 2] as row-major [token][feature]
  // (16-byte chunk c of row r at position c ^ (r % 16)).
  const int half = (lane >> 5) & 1;
  const int l32 = lane & 31;
  auto compute_dq = [&](int st) {
    const uint8_t* Vs = ring[st % kNs] + kKvBytes;
    const int i = 32 * wave + l32;
    f32x16_t dacc;
#pragma unroll
    for (int q = 0; q < 16; ++q) dacc[q] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int ch = 2 * kk + half;
      const uint4 fa = Sl[i * 16 + (ch ^ (i & 7))];
      const uint4 fb = *(const uint4*)(Vs + 1024 * (l32 >> 2) + 64 * ch + 16 * (l32 & 3));
      dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa),
                                                     __builtin_bit_cast(bf16x8_t, fb), dacc, 0, 0, 0);
    }
    uint8_t* stg = wbuf[st & 1];
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int cc = 4 * wave + jg;
      *(uint2*)(stg + l32 * 256 + ((cc ^ (l32 & 15)) << 4) + 8 * half) =
          make_uint2(pack_bf16x2(dacc[4 * jg], dacc[4 * jg + 1]),
                     pack_bf16x2(dacc[4 * jg + 2], dacc[4 * jg + 3]));
    }
    if (kNorm) {  // this wave's 32 features of the stage's normalised queries
      const uint8_t* Qs = ring[st % kNs];
      uint8_t* qd = qstg[kNorm ? (st & 1) : 0];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int i = lane + 64 * m;
        const int tq = i >> 2, cq = 4 * wave + (i & 3);
        *(uint4*)(qd + tq * 256 + ((cq ^ (tq & 15)) << 4)) =
            *(const uint4*)(Qs + 1024 * (tq >> 2) + 64 * cq + 16 * (tq & 3));
      }
    }
  };
  // Stores of the staged dq tile of stage st by waves 0-3 (two 16-byte row
  // pieces per thread). Rows past the frame's end are not stored: with the
  // RMSNorm their staged queries are zero (they were silenced for E_t), so
  // the norm's backward would give them a value that is not row S - 1's.
  // Waves 0-3 issue no loads in the stage loop, so the exec-masked store
  // holds back no prefetch.
  uint16_t* dqf = (kDq && dq) ? dq + fh * (int64_t)S * D : nullptr;
  // With the RMSNorm of q the staged tile is the gradient dqh for the
  // normalised query qh = q r, and dq = r (dqh - (qh . dqh) qh / D); the 16
  // chunks of a row sit in one DPP row of 16 lanes.
  auto store_dq = [&](int st) {
    const uint8_t* stg = wbuf[st & 1];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + 256 * r;
      const int row = idx >> 4, ch = idx & 15;
      const int at = row * 256 + ((ch ^ (row & 15)) << 4);
      uint4 x = *(const uint4*)(stg + at);
      if (kNorm) {
        const uint4 qv = *(const uint4*)(qstg[kNorm ? (st & 1) : 0] + at);
        const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, qw[4] = {qv.x, qv.y, qv.z, qv.w};
        float dv8[8], qv8[8], dot = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dv8[2 * e] = __uint_as_float(xw[e] << 16);
          dv8[2 * e + 1] = __uint_as_float(xw[e] & 0xFFFF0000u);
          qv8[2 * e] = __uint_as_float(qw[e] << 16);
          qv8[2 * e + 1] = __uint_as_float(qw[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += qv8[e] * dv8[e];
        dot = sum_row16(dot) / (float)D;
        const float rr = rqs[kNorm ? st % 3 : 0][row];
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16x2(rr * (dv8[2 * e] - dot * qv8[2 * e]), rr * (dv8[2 * e + 1] - dot * qv8[2 * e + 1]));
        x = make_uint4(o[0], o[1], o[2], o[3]);
      }
      const int sr = st * kTsd + row;
      if (dqf && sr < S) *(uint4*)(dqf + (int64_t)sr * D + 8 * ch) = x;
    }
  };

  // Pipeline: kNs - 1 stages in flight, one barrier per stage. Each step
  // waits for this wave's copies of stage st (and its own LDS reads of the
  // step before), transforms its share of stage st, waits for those LDS
  // writes, and meets every other wave: then all of stage st is transformed,
  // and every wave has finished consuming stage st - 1, so its ring slot can
  // be refilled with stage st + kNs - 1 (past the end the copy re-reads the
  // last token: harmless) and wbuf[(st + 1) % 2] rewritten in the next step.
  // Then the wave consumes stage st.
#pragma unroll
  for (int i = 0; i < kNs - 1; ++i) issue(st_begin + i);
  if (kDq) {
    for (int st = st_begin; st < st_end; ++st) {
      if (wave >= 4 && kNorm) {
        wait_vmcnt_lgkm0<(kNs - 2) * kOps>();  // this wave's copies of stage st
        // RMSNorm of this wave's own query copies, in place: the 16 chunks of
        // a token sit in the lanes congruent to this one mod 4. Tokens past
        // the end are zeroed (they add nothing to E_t).
        uint8_t* slot = ring[st % kNs];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int blk = 2 * (wave - 4) + h;
          uint4* p = (uint4*)(slot + 1024 * blk + 16 * lane);
          const uint4 x = *p;
          const uint32_t w0[4] = {x.x, x.y, x.z, x.w};
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = sumsq_bf16x2(w0[e], ss);
          const float r = rms_inv(sum_lanes_mod4(ss), D);
          const bool past = st * kTsd + 4 * blk + (lane & 3) >= S;
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = past ? 0u
                        : pack_bf16x2(__uint_as_float(w0[e] << 16) * r, __uint_as_float(w0[e] & 0xFFFF0000u) * r);
          *p = make_uint4(o[0], o[1], o[2], o[3]);
          if ((lane >> 2) == 0) rqs[kNorm ? st % 3 : 0][4 * blk + (lane & 3)] = r;
        }
        wait_vmcnt_lgkm0<63>();
      } else if (wave >= 4) {
        wait_vmcnt_lgkm0<(kNs - 2) * kOps>();  // this wave's copies of stage st
        if ((st + 1) * kTsd > S) {
          // tokens past the end hold copies of row S - 1 and have no gate
          // to silence them: zero their q bytes (this lane's own copies) so
          // that they add nothing to E_t (their dq is row S - 1's, see below)
          uint8_t* slot = ring[st % kNs];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int blk = 2 * (wave - 4) + h;
            if (st * kTsd + 4 * blk + (lane & 3) >= S) *(uint4*)(slot + 1024 * blk + 16 * lane) = make_uint4(0, 0, 0, 0);
          }
          wait_vmcnt_lgkm0<63>();
        }
      } else {
        wait_vmcnt_lgkm0<63>();  // lgkmcnt(0): staged dq is written
      }
      bare_barrier();
      if (wave >= 4) {
        issue(st + kNs - 1);
        compute(st);
      } else {
        if (st > st_begin) store_dq(st - 1);
        compute_dq(st);
      }
    }
    wait_vmcnt_lgkm0<0>();
    bare_barrier();
    if (wave < 4 && st_end > st_begin) store_dq(st_end - 1);
  }
  for (int st = st_begin; !kDq && st < st_end; ++st) {
    wait_vmcnt_lgkm0<(kNs - 2) * kOps>();
    transform(st);
    wait_vmcnt_lgkm0<(kNs - 2) * kOps>();  // lgkmcnt(0): this wave's transform writes are done
    bare_barrier();
    issue(st + kNs - 1);
    if (!kAOnly || rowsK) compute(st);
  }
  wait_vmcnt_lgkm0<0>();  // no copy may still be landing in LDS when the workgroup retires

  // Epilogue, staged through the idle ring so that every global store
  // instruction writes 1 KB of consecutive bytes: block by block (32 KB each:
  // bf16(A) in the scan's layout, or 64 rows of an fp32 result), the
  // owning waves drop their values into LDS, the workgroup meets, and all 512
  // threads copy the block out with 16-byte stores. Scattered 8-byte stores
  // straight from the MFMA accumulators cost phase 1 about a seventh of its
  // time on MI355X.
  static_assert(kNs * kSlot >= 32768, "epilogue staging needs 32 KB of ring");
  uint8_t* const stage = &ring[0][0];
  bare_barrier();  // every wave has finished reading the ring
  const float scale = rowsK ? c * c : c;
  const int n = 32 * nt + (lane & 31);
  const int64_t obase = fh * out.fstride + (int64_t)split * out.sstride;

  // 32 KB staged block -> dst: 16-byte granule ci of dst comes from LDS byte
  // offset lds_of(ci).
  auto flush = [&](void* dst, auto lds_of) {
    wait_vmcnt_lgkm0<63>();  // lgkmcnt(0): this wave's LDS writes are done
    bare_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = 512 * i + tid;
      __builtin_nontemporal_store(*(const u32x4_t*)(stage + lds_of(ci)), (u32x4_t*)dst + ci);
    }
    wait_vmcnt_lgkm0<63>();  // this wave's LDS reads are done before the block is refilled
    bare_barrier();
  };
  // LDS placements: fp32 rows plain (row-major) or swizzled (row m: 16-byte
  // chunk c at position c ^ (m % 16)); A^T rows n of 256 bytes, chunk kc at
  // kc ^ (n % 16). The swizzles keep both the owners' writes and the
  // granule-order reads free of bank conflicts.
  auto plain = [](int ci) { return 16 * ci; };
  auto u_frag = [](int ci) {  // granule ci of a 64-row half of U
    const int m = 16 * (ci >> 9) + (ci & 15);
    const int nc = 4 * ((ci >> 6) & 7) + ((ci >> 4) & 3);
    return m * 512 + ((nc ^ (m & 15)) << 4);
  };
  auto a_frag = [](int ci) {  // granule ci of bf16(A)
    const int n = 16 * (ci >> 8) + (ci & 15);
    const int kc = 4 * ((ci >> 6) & 3) + ((ci >> 4) & 3);
    return n * 256 + ((kc ^ (n & 15)) << 4);
  };
  // Owning waves: rows 64 hh .. 64 hh + 63 of their (scaled) fp32 result.
  auto put_rows = [&](int hh, bool swz) {
    float* Sf = (float*)stage;
#pragma unroll
    for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = 32 * mt2 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const int col = swz ? ((((n >> 2) ^ (m & 15)) << 2) | (n & 3)) : n;
        Sf[m * D + col] = acc[2 * hh + mt2][q] * scale;
      }
  };
  // A waves: bf16(A) transposed (row n holds A[0..D)[n]) for the scan.
  auto put_a_bf16 = [&]() {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int m = 32 * mt + 8 * jg + 4 * (lane >> 5);
        const uint32_t w0 = pack_bf16x2(acc[mt][4 * jg] * scale, acc[mt][4 * jg + 1] * scale);
        const uint32_t w1 = pack_bf16x2(acc[mt][4 * jg + 2] * scale, acc[mt][4 * jg + 3] * scale);
        *(uint2*)(stage + n * 256 + (((m >> 3) ^ (n & 15)) << 4) + 2 * (m & 7)) = make_uint2(w0, w1);
      }
  };

  // The output pointers are kernel arguments, so every wave takes the same
  // branches and meets the same barriers. kScanLayout: A in bf16 and U in
  // fp32, both in the scan's granule layout; otherwise fp32 row-major A and U.
  if (out.outA != nullptr) {
    if (kScanLayout) {
      if (rowsK) put_a_bf16();
      flush(out.outA + obase, a_frag);
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if (rowsK) put_rows(hh, false);
        flush(out.outA + obase + hh * 64 * D, plain);
      }
    }
  }
  if (!kAOnly && out.outU != nullptr) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (!rowsK) put_rows(hh, kScanLayout);
      if (kScanLayout)
        flush(out.outU + obase + hh * 64 * D, u_frag);
      else
        flush(out.outU + obase + hh * 64 * D, plain);
    }
  }
}

// fp32 vector path: any io type, D in {16, 32, 64, 128}. One workgroup per
// frame-head (or token range); tokens staged through LDS 16 at a time.
template <typename TIn>
__device__ __forceinline__ float ld(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <typename TIn, int D>
__global__ void __launch_bounds__(256)
terms_generic(const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ beta,
              int S, int n_split, float c, int prepared, int norm, TermsOut out) {
  constexpr int TSG = 16;
  constexpr int OPT = 2 * D * D / 256;
  __shared__ float Ls[TSG][2 * D];
  __shared__ float Ws[TSG][D];
  __shared__ float rn[TSG];  // per-token key factor c (times 1/rms(k) with norm)

  const int64_t fh = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int s_begin = (int)(((int64_t)split * S) / n_split);
  const int s_end = (int)(((int64_t)(split + 1) * S) / n_split);
  const TIn* kf = k + fh * (int64_t)S * D;
  const TIn* vf = v + fh * (int64_t)S * D;
  const float* bf = beta + fh * (int64_t)S;
  const int tid = threadIdx.x;

  float acc[OPT];
#pragma unroll
  for (int r = 0; r < OPT; ++r) acc[r] = 0.f;

  for (int s0 = s_begin; s0 < s_end; s0 += TSG) {
    __syncthreads();
    if (tid < TSG) {
      float f = c;
      // norm == 2: prepared keys normalised without ReLU (queries of the
      // backward's E pass)
      if (norm && (!prepared || norm == 2) && s0 + tid < s_end) {
        float ss = 0.f;
        for (int j = 0; j < D; ++j) {
          const float kv = ld<TIn>(kf, (int64_t)(s0 + tid) * D + j);
          ss += kv * kv;
        }
        f = c * rms_inv(ss, D);
      }
      rn[tid] = f;
    }
    __syncthreads();
    for (int idx = tid; idx < TSG * 2 * D; idx += 256) {
      const int s = idx / (2 * D);
      const int m = idx % (2 * D);
      const int tok = s0 + s;
      float val = 0.f;
      if (tok < s_end) {
        if (m < D) {
          float kv = ld<TIn>(kf, (int64_t)tok * D + m);
          val = prepared ? (norm == 2 ? kv * rn[s] : kv) : (kv > 0.f ? kv : 0.f) * rn[s];
        } else {
          val = ld<TIn>(vf, (int64_t)tok * D + (m - D));
        }
      }
      Ls[s][m] = val;
    }
    for (int idx = tid; idx < TSG * D; idx += 256) {
      const int s = idx / D;
      const int n = idx % D;
      const int tok = s0 + s;
      float val = 0.f;
      if (tok < s_end) {
        float kv = ld<TIn>(kf, (int64_t)tok * D + n);
        val = bf[tok] * (prepared ? (norm == 2 ? kv * rn[s] : kv) : (kv > 0.f ? kv : 0.f) * rn[s]);
      }
      Ws[s][n] = val;
    }
    __syncthreads();
#pragma unroll 4
    for (int s = 0; s < TSG; ++s) {
#pragma unroll
      for (int r = 0; r < OPT; ++r) {
        const int o = tid + 256 * r;
        acc[r] = fmaf(Ls[s][o / D], Ws[s][o % D], acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < OPT; ++r) {
    const int o = tid + 256 * r;
    const int m = o / D;
    const int n = o % D;
    float* dst = m < D ? out.outA : out.outU;
    if (dst == nullptr) continue;
    dst[fh * out.fstride + (int64_t)split * out.sstride + (m % D) * D + n] = acc[r];
  }
}

// p[0] + p[stride] + ... + p[(n - 1) stride] as four-float groups, added in
// index order. With the split count known at compile time (kN > 0) every
// load is issued before the first addition, so a thread waits for one round
// trip rather than one per split.
template <int kN>
__device__ __forceinline__ float4 sum_splits(const float* p, int n, int64_t stride) {
  if (kN > 0) {
    float4 t[kN > 0 ? kN : 1];
#pragma unroll
    for (int b = 0; b < kN; ++b) t[b] = *(const float4*)(p + (int64_t)b * stride);
    float4 acc = t[0];
#pragma unroll
    for (int b = 1; b < kN; ++b) {
      acc.x += t[b].x;
      acc.y += t[b].y;
      acc.z += t[b].z;
      acc.w += t[b].w;
    }
    return acc;
  }
  float4 acc = *(const float4*)p;
  for (int b = 1; b < n; ++b) {
    const float4 t = *(const float4*)(p + (int64_t)b * stride);
    acc.x += t.x;
    acc.y += t.y;
    acc.z += t.z;
    acc.w += t.w;
  }
  return acc;
}

// Sum of the token-range partials in a fixed order (deterministic), as fp32
// row-major A_t and U_t (the scan's granule layout: reduce_partials_granules).
// kN: the split count when it is a compile-time constant (0: n_split).
template <int kN>
__global__ void __launch_bounds__(256)
reduce_partials_kernel(const float* __restrict__ partial, int n_split, int D, int64_t FH,
                       TermsOut out) {
  const int64_t per = (int64_t)2 * D * D / 4;  // four-element groups per frame-head
  const int64_t n = FH * per;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    const int64_t f = i / per;
    const int64_t e = (i % per) * 4;
    const float* base = partial + (f * n_split) * 2 * D * D;
    const float4 s = sum_splits<kN>(base + e, n_split, (int64_t)2 * D * D);
    const int64_t row = e / D;
    const int64_t col = e % D;
    float* dst = row < D ? out.outA : out.outU;
    if (dst == nullptr) continue;
    *(float4*)(dst + f * out.fstride + (row % D) * D + col) = s;
  }
}

// The same sum written in the scan's granule layout (D = 128), one 16-byte
// granule per thread in granule order, so that every wave's stores are 1 KB
// of consecutive bytes: per frame-head the 2048 granules of bf16(A) (8 rows m
// of column n, read as row n, columns m.. by the symmetry of A_t, two 16-byte
// loads per split), then the 4096 granules of U (4 columns of row m). The
// additions run in split order, as in reduce_partials_kernel.
template <int kN>
__global__ void __launch_bounds__(256)
reduce_partials_granules(const float* __restrict__ partial, int n_split, int64_t FH, TermsOut out) {
  constexpr int D = 128;
  constexpr int64_t DD = (int64_t)D * D;
  constexpr int kAG = D * D / 8, kUG = D * D / 4;  // granules of A (bf16) and of U (fp32)
  const int64_t n = FH * (kAG + kUG);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t f = i / (kAG + kUG);
    const int g = (int)(i % (kAG + kUG));
    const float* base = partial + (f * n_split) * 2 * DD;
    if (g < kAG) {
      const int blk = g >> 6, r = g & 63;
      const int nn = (blk >> 2) * 16 + (r & 15);  // inverse of a_granule
      const int kc = (blk & 3) * 4 + (r >> 4);
      const float* src = base + (int64_t)nn * D + 8 * kc;
      const float4 lo = sum_splits<kN>(src, n_split, 2 * DD);
      const float4 hi = sum_splits<kN>(src + 4, n_split, 2 * DD);
      if (out.outA == nullptr) continue;
      uint4* At = (uint4*)(out.outA + f * out.fstride);
      At[g] = make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                         pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w));
    } else {
      const int gu = g - kAG;
      const int blk = gu >> 6, r = gu & 63;
      const int m = (blk >> 3) * 16 + (r & 15);  // inverse of u_granule
      const int nc = (blk & 7) * 4 + (r >> 4);
      const float4 v = sum_splits<kN>(base + DD + (int64_t)m * D + 4 * nc, n_split, 2 * DD);
      if (out.outU == nullptr) continue;
      ((float4*)(out.outU + f * out.fstride))[gu] = v;
    }
  }
}

template <typename TIn>
hipError_t launch_generic(const Shape& sh, const void* k, const void* v, const float* beta,
                          int n_split, TermsOut out, hipStream_t st) {
  if (!grid_fits(sh.FH() * n_split, 256)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(sh.FH() * n_split));
  const TIn* kk = (const TIn*)k;
  const TIn* vv = (const TIn*)v;
  switch (sh.D) {
    case 16:
      terms_generic<TIn, 16><<<grid, 256, 0, st>>>(kk, vv, beta, sh.S, n_split, sh.c, sh.prepared,
                                                  sh.qk_norm, out);
      break;
    case 32:
      terms_generic<TIn, 32><<<grid, 256, 0, st>>>(kk, vv, beta, sh.S, n_split, sh.c, sh.prepared,
                                                  sh.qk_norm, out);
      break;
    case 64:
      terms_generic<TIn, 64><<<grid, 256, 0, st>>>(kk, vv, beta, sh.S, n_split, sh.c, sh.prepared,
                                                  sh.qk_norm, out);
      break;
    case 128:
      terms_generic<TIn, 128><<<grid, 256, 0, st>>>(kk, vv, beta, sh.S, n_split, sh.c, sh.prepared,
                                                  sh.qk_norm, out);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool terms_use_mfma(const Shape& sh) { return sh.io == 1 && sh.D == 128; }

#ifndef GDN_TERMS_SPLIT_MAX
#define GDN_TERMS_SPLIT_MAX 5
#endif
int terms_split(const Shape& sh) {
  const int64_t fh = sh.FH();
  // A workgroup streams a frame-head at the rate of its CU's pipeline, so a
  // call with at least half as many frame-heads as CUs runs them whole: on
  // MI355X the 16-head 5 s layer (176 frame-heads) took 94 us unsplit against
  // 98 and 115 us (reduction included) with 2 and 3 splits. Fewer frame-heads
  // are split to about one workgroup per CU (the split partials cost a
  // reduction launch and their traffic).
  if (fh <= 0 || fh >= 128) return 1;
  const int64_t want = (256 + fh - 1) / fh;
  int64_t cap = sh.S / 512;                   // keep at least 512 tokens per split
  // at most GDN_TERMS_SPLIT_MAX splits: a 3-frame streaming block of the
  // 16-head layer (48 frame-heads of 3600 tokens) took 74.7 us with 7 splits
  // against 71 us with 4; 5 splits (240 workgroups, one round) cut its
  // phase 1 and reduction from 38.7 to 37.4 us, while 6 (288 workgroups)
  // took 45.6 us
  cap = std::min<int64_t>(std::max<int64_t>(cap, 1), GDN_TERMS_SPLIT_MAX);
  return (int)std::max<int64_t>(1, std::min(want, cap));
}

hipError_t launch_terms(const Shape& sh, const void* k, const void* v, const float* beta,
                        int n_split, TermsOut out, bool scan_layout, hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  if (terms_use_mfma(sh)) {
    if (!grid_fits(sh.FH() * n_split, 512)) return hipErrorInvalidValue;
    dim3 grid((unsigned)(sh.FH() * n_split));
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    const bool norm = sh.qk_norm && !sh.prepared;  // prepared keys are used as given
#define GDN_TERMS_DMA(L, P, N, AO)                                                           \
  terms_dma_bf16_d128<L, P, N, AO, false><<<grid, 512, 0, st>>>(kk, vv, beta, sh.S, n_split, sh.c, \
                                                                out, nullptr, nullptr, nullptr)
    if (sh.qk_norm == 2) return hipErrorInvalidValue;  // the generic path's E mode only
    if (scan_layout && out.outU == nullptr) {  // A_t alone (the backward's recompute)
      if (sh.prepared) GDN_TERMS_DMA(true, true, false, true);
      else if (norm) GDN_TERMS_DMA(true, false, true, true);
      else GDN_TERMS_DMA(true, false, false, true);
    } else if (scan_layout) {
      if (sh.prepared) GDN_TERMS_DMA(true, true, false, false);
      else if (norm) GDN_TERMS_DMA(true, false, true, false);
      else GDN_TERMS_DMA(true, false, false, false);
    } else {
      if (sh.prepared) GDN_TERMS_DMA(false, true, false, false);
      else if (norm) GDN_TERMS_DMA(false, false, true, false);
      else GDN_TERMS_DMA(false, false, false, false);
    }
#undef GDN_TERMS_DMA
    return hipGetLastError();
  }
  if (sh.io == 1) return launch_generic<uint16_t>(sh, k, v, beta, n_split, out, st);
  return launch_generic<float>(sh, k, v, beta, n_split, out, st);
}

bool edq_fused(const Shape& sh) { return terms_use_mfma(sh); }

hipError_t launch_edq(const Shape& sh, const void* q, const void* d_o, const float* states,
                      const float* states2, void* dq, float* E, bool norm, hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  if (!edq_fused(sh) || !grid_fits(sh.FH(), 512)) return hipErrorInvalidValue;
  TermsOut out{nullptr, E, (int64_t)sh.D * sh.D, 0};
  if (norm)
    terms_dma_bf16_d128<true, true, true, false, true><<<dim3((unsigned)sh.FH()), 512, 0, st>>>(
        (const uint16_t*)q, (const uint16_t*)d_o, nullptr, sh.S, 1, 1.f, out, states, states2,
        (uint16_t*)dq);
  else
    terms_dma_bf16_d128<true, true, false, false, true><<<dim3((unsigned)sh.FH()), 512, 0, st>>>(
        (const uint16_t*)q, (const uint16_t*)d_o, nullptr, sh.S, 1, 1.f, out, states, states2,
        (uint16_t*)dq);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const Shape& sh, const float* partial, int n_split, TermsOut out,
                                  bool scan_layout, hipStream_t st) {
  const int64_t n = sh.FH() * 2 * sh.D * sh.D / 4;
  if (n == 0) return hipSuccess;
  int64_t g = std::min<int64_t>((n + 255) / 256, 8192);
  if (scan_layout) {
    if (sh.D != 128) return hipErrorInvalidValue;  // the granule layout is D = 128's
    const int64_t ng = sh.FH() * (sh.D * sh.D / 8 + sh.D * sh.D / 4);
    const int64_t gg = std::min<int64_t>((ng + 255) / 256, 8192);
    switch (n_split) {
      case 2: reduce_partials_granules<2><<<(unsigned)gg, 256, 0, st>>>(partial, n_split, sh.FH(), out); break;
      case 3: reduce_partials_granules<3><<<(unsigned)gg, 256, 0, st>>>(partial, n_split, sh.FH(), out); break;
      case 4: reduce_partials_granules<4><<<(unsigned)gg, 256, 0, st>>>(partial, n_split, sh.FH(), out); break;
      case 5: reduce_partials_granules<5><<<(unsigned)gg, 256, 0, st>>>(partial, n_split, sh.FH(), out); break;
      default: reduce_partials_granules<0><<<(unsigned)gg, 256, 0, st>>>(partial, n_split, sh.FH(), out); break;
    }
    return hipGetLastError();
  }
  switch (n_split) {
    case 2: reduce_partials_kernel<2><<<(unsigned)g, 256, 0, st>>>(partial, n_split, sh.D, sh.FH(), out); break;
    case 3: reduce_partials_kernel<3><<<(unsigned)g, 256, 0, st>>>(partial, n_split, sh.D, sh.FH(), out); break;
    case 4: reduce_partials_kernel<4><<<(unsigned)g, 256, 0, st>>>(partial, n_split, sh.D, sh.FH(), out); break;
    case 5: reduce_partials_kernel<5><<<(unsigned)g, 256, 0, st>>>(partial, n_split, sh.D, sh.FH(), out); break;
    default: reduce_partials_kernel<0><<<(unsigned)g, 256, 0, st>>>(partial, n_split, sh.D, sh.FH(), out); break;
  }
  return hipGetLastError();
}

}  // namespace gdn
