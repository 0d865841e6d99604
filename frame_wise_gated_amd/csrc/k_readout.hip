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
// the "B" operand is q (columns = tokens, contraction j contiguous): both
// fragments are plain 16-byte loads, no transpose. Each wave keeps the whole
// state as bf16 fragments in registers and streams 32-token tiles of q; the
// 32x32 accumulator gives every lane four consecutive value dims of one token,
// stored as one 8-byte write. The workgroup -> frame-head mapping keeps all
// workgroups of a frame-head on one XCD, so the state is fetched from HBM once.
#include "gdn_common.h"

namespace gdn {

namespace {

constexpr int kTokPerWave = 32;
constexpr int kWavesPerBlock = 4;
constexpr int kXcd = 8;

__device__ __forceinline__ uint4 ld_q(const uint16_t* q, int s, int S, int j) {
  return (s < S) ? *(const uint4*)(q + (int64_t)s * 128 + j) : make_uint4(0, 0, 0, 0);
}

__global__ void __launch_bounds__(256)
readout_mfma_bf16_d128(const uint16_t* __restrict__ q, const float* __restrict__ sa,
                       const float* __restrict__ sb, uint16_t* __restrict__ o, int S, int64_t FH,
                       int nb) {
  constexpr int D = 128;
  const int xcd = blockIdx.x % kXcd;
  const int slot = blockIdx.x / kXcd;
  const int64_t fh = (int64_t)(slot / nb) * kXcd + xcd;
  const int b = slot % nb;
  if (fh >= FH) return;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // State fragments: a[mt][kk] = S[32mt + l32][16kk + 8half .. +8] as bf16.
  bf16x8_t a[4][8];
  {
    const float* s1 = sa + fh * D * D;
    const float* s2 = sb ? sb + fh * D * D : nullptr;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int64_t off = (int64_t)(32 * mt + l32) * D + 16 * kk + 8 * half;
        float4 x0 = *(const float4*)(s1 + off);
        float4 x1 = *(const float4*)(s1 + off + 4);
        if (s2) {
          float4 y0 = *(const float4*)(s2 + off);
          float4 y1 = *(const float4*)(s2 + off + 4);
          x0.x += y0.x; x0.y += y0.y; x0.z += y0.z; x0.w += y0.w;
          x1.x += y1.x; x1.y += y1.y; x1.z += y1.z; x1.w += y1.w;
        }
        uint4 pk = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w),
                              pack_bf16x2(x1.x, x1.y), pack_bf16x2(x1.z, x1.w));
        a[mt][kk] = __builtin_bit_cast(bf16x8_t, pk);
      }
  }

  const uint16_t* qf = q + fh * (int64_t)S * D;
  uint16_t* of = o + fh * (int64_t)S * D;
  const int ntiles = (S + kTokPerWave - 1) / kTokPerWave;
  const int wstride = nb * kWavesPerBlock;
  int tile = b * kWavesPerBlock + wave;
  if (tile >= ntiles) return;

  uint4 qb[8];
  {
    const int s = tile * kTokPerWave + l32;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[kk] = ld_q(qf, s, S, 16 * kk + 8 * half);
  }
  for (; tile < ntiles; tile += wstride) {
    const int s = tile * kTokPerWave + l32;
    bf16x8_t bq[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) bq[kk] = __builtin_bit_cast(bf16x8_t, qb[kk]);
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
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][kk], bq[kk], acc[mt], 0, 0, 0);
    if (s < S) {
      uint16_t* orow = of + (int64_t)s * D;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int i0 = 32 * mt + 8 * jg + 4 * half;
          uint2 w = make_uint2(pack_bf16x2(acc[mt][4 * jg + 0], acc[mt][4 * jg + 1]),
                               pack_bf16x2(acc[mt][4 * jg + 2], acc[mt][4 * jg + 3]));
          *(uint2*)(orow + i0) = w;
        }
    }
  }
}

// fp32 vector path, D in {16, 32, 64, 128}: the summed state is staged
// transposed in LDS (St[j][i]); each thread forms whole dot products.
template <typename TIn, int D>
__global__ void __launch_bounds__(256)
readout_generic(const TIn* __restrict__ q, const float* __restrict__ sa,
                const float* __restrict__ sb, TIn* __restrict__ o, int S, int ntile) {
  constexpr int TT = 2048 / D;        // tokens per tile
  constexpr int OPT = TT * D / 256;   // outputs per thread
  __shared__ float St[D][D];
  __shared__ float Qs[TT][D];
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
  TIn* of = o + fh * (int64_t)S * D;
#pragma unroll
  for (int r = 0; r < OPT; ++r) {
    const int idx = tid + 256 * r;
    const int s = idx / D;
    const int i = idx % D;
    float acc = 0.f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) acc = fmaf(St[j][i], Qs[s][j], acc);
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
  dim3 grid((unsigned)(sh.FH() * ntile));
  const TIn* qq = (const TIn*)q;
  TIn* oo = (TIn*)o;
  switch (sh.D) {
    case 16: readout_generic<TIn, 16><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile); break;
    case 32: readout_generic<TIn, 32><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile); break;
    case 64: readout_generic<TIn, 64><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile); break;
    case 128: readout_generic<TIn, 128><<<grid, 256, 0, st>>>(qq, sa, sb, oo, sh.S, ntile); break;
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
    int nb = (ntiles + 4 * kWavesPerBlock - 1) / (4 * kWavesPerBlock);  // ~4 tiles per wave
    if (nb < 1) nb = 1;
    const int64_t groups = (sh.FH() + kXcd - 1) / kXcd;
    dim3 grid((unsigned)(groups * kXcd * nb));
    readout_mfma_bf16_d128<<<grid, 256, 0, st>>>((const uint16_t*)q, sa, sb, (uint16_t*)o, sh.S,
                                                 sh.FH(), nb);
    return hipGetLastError();
  }
  if (sh.io == 1) return launch_readout_generic<uint16_t>(sh, q, sa, sb, o, st);
  return launch_readout_generic<float>(sh, q, sa, sb, o, st);
}

}  // namespace gdn
