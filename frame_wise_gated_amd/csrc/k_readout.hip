// Phase 3: per-token readout o_{t,s} = S_t q_{t,s} (or (S_t + R_t) q_{t,s} for
// the chunk-causal bidirectional scan), frame-parallel.
//
// The readout with the post-update state S_t is the usual Gated DeltaNet
// output rule (xiejiayun.github.io "好文共赏 | SANA-WM", section 2.1 recalls the
// token-level rule); the pages do not spell the frame-wise readout out, and
// this library takes o = S_t q with the state after frame t.
//
// MFMA path (bf16, D = 128): O_t^T = S_t Q_t^T, so the MFMA "A" operand is the
// state (rows = value dim i, contraction = key dim j, contiguous in memory) and
// the "B" operand is q (columns = tokens, contraction j contiguous): q
// fragments are plain 16-byte loads, no transpose. A workgroup stages the
// state once in LDS as bf16 and its four waves stream 32-token tiles of q;
// each output tile goes through a per-wave LDS buffer so that the 8 KB tile
// (contiguous in HBM) is written with fully coalesced 16-byte stores. The
// workgroup -> frame-head mapping keeps all workgroups of a frame-head on one
// XCD, so the state comes from HBM once.
#include "gdn_common.h"

namespace gdn {

namespace {

constexpr int kTokPerWave = 32;
constexpr int kWavesPerBlock = 4;
// Workgroups per frame-head (their tiles interleave). HBM serves a mixed
// read/write stream faster when the concurrently active workgroups touch a
// narrower address window, which more workgroups per frame-head give, while
// every workgroup stages the state once. On MI355X, the 60 s 720p layer's
// readout (one state) took 706 / 678-686 / 671-675 / 674-684 / 682-684 /
// 693-698 / 703-710 us with 4 / 8 / 9 / 10 / 11 / 12 / 16 workgroups per
// frame-head, and its chunk-causal readout (two states staged) 734 / 723 /
// 732 / 755-759 us with 4 / 8 / 10 / 12; the 16-head 5 s layer's 81 us with 4
// and 70-72 us with 8 to 16.
#ifndef GDN_READOUT_NB
#define GDN_READOUT_NB 9
#endif
#ifndef GDN_READOUT_NB2
#define GDN_READOUT_NB2 8
#endif
constexpr int kMaxBlocksPerFrameHead = 16;
constexpr int kXcd = 8;

__device__ __forceinline__ uint4 ld_q(const uint16_t* q, int s, int S, int j) {
  return (s < S) ? *(const uint4*)(q + (int64_t)s * 128 + j) : make_uint4(0, 0, 0, 0);
}

// 16-byte chunk swizzle inside a 256-byte LDS row (16 chunks): eight
// consecutive rows read at the same logical chunk hit eight distinct bank groups.
__device__ __forceinline__ int rswz(int row, int chunk) { return chunk ^ (row & 7); }

template <bool kNorm>
__global__ void __launch_bounds__(256, 2)
readout_mfma_bf16_d128(const uint16_t* __restrict__ q, const float* __restrict__ sa,
                       const float* __restrict__ sb, uint16_t* __restrict__ o, int S, int64_t FH,
                       int nb) {
  constexpr int D = 128;
  __shared__ uint4 Sl[D * 16];                              // state, bf16, row i = value dim
  __shared__ uint4 Ol[kWavesPerBlock][kTokPerWave * 16];    // per-wave output tile staging

  const int xcd = blockIdx.x % kXcd;
  const int slot = blockIdx.x / kXcd;
  const int64_t fh = (int64_t)(slot / nb) * kXcd + xcd;
  const int b = slot % nb;
  if (fh >= FH) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Stage the (summed) state once per workgroup: fp32 -> bf16, coalesced.
  // Thread t handles the 8-column chunks t + 256 it (row c / 16, columns
  // 8 (c % 16) ..). Every load is issued before the first one is used: as a
  // plain loop the eight chunks cost eight round trips one after the other
  // (the chunk-causal 60 s layer's readout took 749 us that way, against
  // 707 us with no staging at all).
  constexpr int kStageIt = D * 16 / 256;
  const float* s1 = sa + fh * D * D;
  const float* s2 = sb ? sb + fh * D * D : nullptr;
  float4 xs[kStageIt][2];
#pragma unroll
  for (int it = 0; it < kStageIt; ++it) {
    const int c = tid + 256 * it;
    const int64_t off = (int64_t)(c >> 4) * D + 8 * (c & 15);
    xs[it][0] = *(const float4*)(s1 + off);
    xs[it][1] = *(const float4*)(s1 + off + 4);
  }
  if (s2) {
    float4 ys[kStageIt][2];
#pragma unroll
    for (int it = 0; it < kStageIt; ++it) {
      const int c = tid + 256 * it;
      const int64_t off = (int64_t)(c >> 4) * D + 8 * (c & 15);
      ys[it][0] = *(const float4*)(s2 + off);
      ys[it][1] = *(const float4*)(s2 + off + 4);
    }
#pragma unroll
    for (int it = 0; it < kStageIt; ++it)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        xs[it][h2].x += ys[it][h2].x;
        xs[it][h2].y += ys[it][h2].y;
        xs[it][h2].z += ys[it][h2].z;
        xs[it][h2].w += ys[it][h2].w;
      }
  }
#pragma unroll
  for (int it = 0; it < kStageIt; ++it) {
    const int c = tid + 256 * it;
    const int i = c >> 4;
    const float4 x0 = xs[it][0], x1 = xs[it][1];
    Sl[i * 16 + rswz(i, c & 15)] = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w),
                                              pack_bf16x2(x1.x, x1.y), pack_bf16x2(x1.z, x1.w));
  }
  __syncthreads();

  const uint16_t* qf = q + fh * (int64_t)S * D;
  uint16_t* of = o + fh * (int64_t)S * D;
  const int ntiles = (S + kTokPerWave - 1) / kTokPerWave;
  const int wstride = nb * kWavesPerBlock;
  int tile = b * kWavesPerBlock + wave;
  if (tile >= ntiles) return;
  uint4* stage = Ol[wave];

  uint4 qb[8];
  {
    const int s = tile * kTokPerWave + l32;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[kk] = ld_q(qf, s, S, 16 * kk + 8 * half);
  }
  for (; tile < ntiles; tile += wstride) {
    bf16x8_t bq[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) bq[kk] = __builtin_bit_cast(bf16x8_t, qb[kk]);
    // RMSNorm of q: this lane holds 64 of token l32's 128 features, the
    // other 64 sit in lane l32 + 32 of the other half
    float rq = 1.f;
    if (kNorm) {
      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        ss = sumsq_bf16x2(qb[kk].x, ss);
        ss = sumsq_bf16x2(qb[kk].y, ss);
        ss = sumsq_bf16x2(qb[kk].z, ss);
        ss = sumsq_bf16x2(qb[kk].w, ss);
      }
      rq = rms_inv(sum_lane_xor32(ss), D);
    }
    const int nxt = tile + wstride;
    if (nxt < ntiles) {
      const int sn = nxt * kTokPerWave + l32;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) qb[kk] = ld_q(qf, sn, S, 16 * kk + 8 * half);
    }
    f32x16_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mt][j] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = 32 * mt + l32;
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, Sl[row * 16 + rswz(row, 2 * kk + half)]);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[kk], acc[mt], 0, 0, 0);
      }
    if (kNorm) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] *= rq;  // o = S (q / rms(q)) = (S q) / rms(q)
    }
    // Accumulator (i, s): lane holds token s = l32 and value dims
    // 32mt + 8jg + 4half + (0..3). Stage as rows of tokens, then write the
    // 32 x 256-byte tile (contiguous in HBM) with 16-byte stores.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const uint2 w = make_uint2(pack_bf16x2(acc[mt][4 * jg + 0], acc[mt][4 * jg + 1]),
                                   pack_bf16x2(acc[mt][4 * jg + 2], acc[mt][4 * jg + 3]));
        uint2* dst = (uint2*)&stage[l32 * 16 + rswz(l32, 4 * mt + jg)];
        dst[half] = w;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int s0 = tile * kTokPerWave;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = 4 * it + (lane >> 4);
      const int ch = lane & 15;
      const uint4 val = stage[row * 16 + rswz(row, ch)];
      if (s0 + row < S) *(uint4*)(of + (int64_t)(s0 + row) * D + 8 * ch) = val;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// fp32 vector path, D in {16, 32, 64, 128}: the summed state is staged
// transposed in LDS (St[j][i]); each thread forms whole dot products.
template <typename TIn, int D>
__global__ void __launch_bounds__(256)
readout_generic(const TIn* __restrict__ q, const float* __restrict__ sa,
                const float* __restrict__ sb, TIn* __restrict__ o, int S, int ntile, int norm) {
  constexpr int TT = 2048 / D;        // tokens per tile
  constexpr int OPT = TT * D / 256;   // outputs per thread
  __shared__ float St[D][D];
  __shared__ float Qs[TT][D];
  __shared__ float rq[TT];  // per-token factor 1/rms(q) (1 without norm)
  const int64_t fh = blockIdx.x / ntile;
  const int tile = blockIdx.x % ntile;
  const int tid = threadIdx.x;
  const float* s1 = sa + fh * D * D;
  const float* s2 = sb ? sb + fh * D * D : nullptr;
  for (int idx = tid; idx < D * D; idx += 256) {
    const int i = idx / D;
    const int j = idx % D;
    float x = s1[idx];
    if (s2) x += s2[idx];
    St[j][i] = x;
  }
  const int s0 = tile * TT;
  const TIn* qf = q + fh * (int64_t)S * D;
  for (int idx = tid; idx < TT * D; idx += 256) {
    const int s = idx / D;
    const int j = idx % D;
    float x = 0.f;
    if (s0 + s < S) {
      if constexpr (sizeof(TIn) == 2) x = bf16_to_f32(((const uint16_t*)qf)[(int64_t)(s0 + s) * D + j]);
      else x = ((const float*)qf)[(int64_t)(s0 + s) * D + j];
    }
    Qs[s][j] = x;
  }
  __syncthreads();
  if (tid < TT) {
    float f = 1.f;
    if (norm) {
      float ss = 0.f;
      for (int j = 0; j < D; ++j) ss += Qs[tid][j] * Qs[tid][j];
      f = rms_inv(ss, D);
    }
    rq[tid] = f;
  }
  __syncthreads();
  TIn* of = o + fh * (int64_t)S * D;
#pragma unroll
  for (int r = 0; r < OPT; ++r) {
    const int idx = tid + 256 * r;
    const int s = idx / D;
    const int i = idx % D;
    float acc = 0.f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) acc = fmaf(St[j][i], Qs[s][j], acc);
    acc *= rq[s];
    if (s0 + s < S) {
      if constexpr (sizeof(TIn) == 2)
        ((uint16_t*)of)[(int64_t)(s0 + s) * D + i] = (uint16_t)(pack_bf16x2(acc, 0.f) & 0xFFFFu);
      else
        ((float*)of)[(int64_t)(s0 + s) * D + i] = acc;
    }
  }
}

template <typename TIn>
hipError_t launch_readout_generic(const Shape& sh, const void* q, const float* sa, const float* sb,
                                  void* o, hipStream_t st) {
  const int TT = 2048 / sh.D;
  const int ntile = (sh.S + TT - 1) / TT;
  if (!grid_fits(sh.FH() * ntile, 256)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(sh.FH() * ntile));
  const TIn* qq = (const TIn*)q;
  TIn* oo = (TIn*)o;
  switch (sh.D) {
    case 16: readout_generic<TIn, 16><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile, sh.qk_norm); break;
    case 32: readout_generic<TIn, 32><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile, sh.qk_norm); break;
    case 64: readout_generic<TIn, 64><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile, sh.qk_norm); break;
    case 128: readout_generic<TIn, 128><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile, sh.qk_norm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_readout(const Shape& sh, const void* q, const float* sa, const float* sb, void* o,
                          hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  if (sh.io == 1 && sh.D == 128) {
    const int ntiles = (sh.S + kTokPerWave - 1) / kTokPerWave;
    // calls with few frame-heads (a streaming block) take more workgroups per
    // frame-head, up to two per CU in one round (512: more would start a
    // second round of workgroups)
    const int64_t base = sb ? GDN_READOUT_NB2 : GDN_READOUT_NB;
    int64_t want = 512 / sh.FH();
    want = want < base ? base : (want > kMaxBlocksPerFrameHead ? kMaxBlocksPerFrameHead : want);
    int nb = (ntiles + kWavesPerBlock - 1) / kWavesPerBlock;
    if (nb > want) nb = (int)want;
    const int64_t groups = (sh.FH() + kXcd - 1) / kXcd;
    if (!grid_fits(groups * kXcd * nb, 256)) return hipErrorInvalidValue;
    dim3 grid((unsigned)(groups * kXcd * nb));
    if (sh.qk_norm)
      readout_mfma_bf16_d128<true><<<grid, 256, 0, st>>>((const uint16_t*)q, sa, sb, (uint16_t*)o,
                                                         sh.S, sh.FH(), nb);
    else
      readout_mfma_bf16_d128<false><<<grid, 256, 0, st>>>((const uint16_t*)q, sa, sb, (uint16_t*)o,
                                                          sh.S, sh.FH(), nb);
    return hipGetLastError();
  }
  if (sh.io == 1) return launch_readout_generic<uint16_t>(sh, q, sa, sb, o, st);
  return launch_readout_generic<float>(sh, q, sa, sb, o, st);
}

}  // namespace gdn
