// Backward pass of the causal frame scan: the per-frame and per-token
// gradient kernels. The adjoint recurrence itself runs on the scan kernels
// (k_scan.hip, REVERSE mode with a shifted U source); phase 1 supplies A_t and
// E_t = dO_t^T Q_t.
//
// Forward rule (blog.hotdry.top SANA-WM post, section "混合线性注意力"):
// S_t = S_{t-1} M_t + U_t, M_t = gamma_t (I - A_t), o = S_t q. With
// G_t = dL/dS_t (G_{T-1} = E_{T-1} + dS_final, G_t = E_t + G_{t+1} M_{t+1},
// M symmetric) the gradients are, per frame,
//   dM_t = S_{t-1}^T G_t,  dgamma_t = <dM_t, I - A_t>,
//   P_t  = dA_t + dA_t^T = -gamma_t (dM_t + dM_t^T),
// and per token (k the prepared key, beta its gate)
//   dq = S_t^T do,   dk = beta (P_t k + G_t^T v),   dv = beta G_t k,
//   dbeta = 1/2 k^T P_t k + v^T G_t k,
// followed by the key scale and the ReLU mask for raw keys.
#include "gdn_common.h"

namespace gdn {

namespace {

// G_{T-1} = E_{T-1} + dS_final for every head (row-major output). E is in the
// scan's granule layout when `granule`, fp32 row-major otherwise.
__global__ void __launch_bounds__(256) grad_init_kernel(const float* __restrict__ E,
                                                        const float* __restrict__ ds_final,
                                                        float* __restrict__ ginit, int T, int D,
                                                        int64_t BH, int granule) {
  const int64_t DD = (int64_t)D * D;
  const int64_t n_all = BH * DD;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_all;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bh = i / DD;
    const int e = (int)(i % DD);
    const int m = e / D, n = e % D;
    const float* Et = E + (bh * T + (T - 1)) * DD;
    const float ev = granule ? Et[(int64_t)u_granule(m, n >> 2) * 4 + (n & 3)] : Et[e];
    ginit[i] = ev + (ds_final ? ds_final[i] : 0.f);
  }
}

// F at the first frame of every chunk of the bidirectional backward:
// finit[bh][c] = E_{c L} (row-major output; E in the scan's granule layout
// when `granule`).
__global__ void __launch_bounds__(256) chunk_init_kernel(const float* __restrict__ E,
                                                         float* __restrict__ finit, int T, int D,
                                                         int L, int nchunk, int64_t BH,
                                                         int granule) {
  const int64_t DD = (int64_t)D * D;
  const int64_t n_all = BH * nchunk * DD;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_all;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bc = i / DD;
    const int64_t bh = bc / nchunk;
    const int c = (int)(bc % nchunk);
    const int e = (int)(i % DD);
    const int m = e / D, n = e % D;
    const float* Ea = E + (bh * T + (int64_t)c * L) * DD;
    finit[i] = granule ? Ea[(int64_t)u_granule(m, n >> 2) * 4 + (n & 3)] : Ea[e];
  }
}

// Chunk-causal backward, per frame t of chunk [a, e): F_t (first frame: the
// chunk's start value; later frames: slot f - 1 of the F scan), and whether a
// reverse state R_{t+1} of the same chunk exists.
__device__ __forceinline__ const float* rev_adjoint(const RevGrad& rg, int64_t f, int64_t bh,
                                                    int t, int T, int64_t DD, bool* more) {
  const int c = t / rg.L;
  const int a = c * rg.L;
  *more = t + 1 < min(a + rg.L, T);
  return t == a ? rg.finit + (bh * rg.nchunk + c) * DD : rg.fbuf + (f - 1) * DD;
}

// Per frame-head: dM = S_prev^T G (fp32), dgamma = tr(dM) - <dM, A>,
// P = -gamma (dM + dM^T). 256 threads as a 16 x 16 grid, each owning a
// B x B block of dM (B = D / 16); S_prev and G staged in LDS.
// Chunk-causal scan (rg.rev set): dM also gets R_{t+1}^T F_t, and G_t is
// replaced in place by G_t + F_t (the gradient reaching U_t) for the token
// kernel; no other workgroup reads frame t's slot.
template <int D>
__global__ void __launch_bounds__(256) frame_grad_kernel(
    const float* __restrict__ states, const float* __restrict__ s0, float* __restrict__ gbuf,
    float* __restrict__ ginit, const float* __restrict__ terms, int a_granule_bf16,
    const float* __restrict__ gamma, float* __restrict__ P, float* __restrict__ dgamma, int T,
    RevGrad rg) {
  constexpr int B = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  __shared__ float Ss[D][D];
  __shared__ float Gs[D][D];
  __shared__ float red[256];
  const int64_t f = blockIdx.x;
  const int64_t bh = f / T;
  const int t = (int)(f % T);
  const int tid = threadIdx.x;
  const float* Sp = t > 0 ? states + (f - 1) * DD : (s0 ? s0 + bh * DD : nullptr);
  float* Gt = t == T - 1 ? ginit + bh * DD : gbuf + (f + 1) * DD;
  for (int e = tid; e < D * D; e += 256) {
    Ss[e / D][e % D] = Sp ? Sp[e] : 0.f;
    Gs[e / D][e % D] = Gt[e];
  }
  __syncthreads();
  const int a0 = B * (tid / 16), b0 = B * (tid % 16);
  float acc[B][B];
#pragma unroll
  for (int x = 0; x < B; ++x)
#pragma unroll
    for (int y = 0; y < B; ++y) acc[x][y] = 0.f;
  auto product = [&]() {  // acc += Ss^T Gs
    for (int i = 0; i < D; ++i) {
      float sa[B], gb[B];
#pragma unroll
      for (int x = 0; x < B; ++x) sa[x] = Ss[i][a0 + x];
#pragma unroll
      for (int y = 0; y < B; ++y) gb[y] = Gs[i][b0 + y];
#pragma unroll
      for (int x = 0; x < B; ++x)
#pragma unroll
        for (int y = 0; y < B; ++y) acc[x][y] = fmaf(sa[x], gb[y], acc[x][y]);
    }
  };
  product();
  if (rg.rev != nullptr) {
    bool more;
    const float* Ft = rev_adjoint(rg, f, bh, t, T, DD, &more);
    const float* Rn = rg.rev + (f + 1) * DD;
    __syncthreads();  // every thread is done with Ss and Gs
    for (int e = tid; e < D * D; e += 256) {
      const float fv = Ft[e];
      Gt[e] = Gs[e / D][e % D] + fv;
      Gs[e / D][e % D] = fv;
      if (more) Ss[e / D][e % D] = Rn[e];
    }
    __syncthreads();
    if (more) product();
  }
  // <dM, I - A>
  const float* At = terms + f * 2 * DD;
  float part = 0.f;
#pragma unroll
  for (int x = 0; x < B; ++x)
#pragma unroll
    for (int y = 0; y < B; ++y) {
      const int a = a0 + x, b = b0 + y;
      float av;
      if (a_granule_bf16) {
        const uint16_t* Ab = (const uint16_t*)At;  // A[a][b] = granule (n = b, kc = a / 8), entry a % 8
        av = bf16_to_f32(Ab[(int64_t)a_granule(b, a >> 3) * 8 + (a & 7)]);
      } else {
        av = At[(int64_t)a * D + b];
      }
      part += acc[x][y] * ((a == b ? 1.f : 0.f) - av);
    }
  red[tid] = part;
  __syncthreads();  // also: every thread is done reading Ss, reused below for dM
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float g = gamma[f];
  if (tid == 0 && dgamma != nullptr) dgamma[f] = red[0];
#pragma unroll
  for (int x = 0; x < B; ++x)
#pragma unroll
    for (int y = 0; y < B; ++y) Ss[a0 + x][b0 + y] = acc[x][y];
  __syncthreads();
  float* Pf = P + f * DD;
#pragma unroll
  for (int x = 0; x < B; ++x)
#pragma unroll
    for (int y = 0; y < B; ++y) {
      const int a = a0 + x, b = b0 + y;
      Pf[(int64_t)a * D + b] = -g * (acc[x][y] + Ss[b][a]);
    }
}

// Per-token gradients, fp32 vector path (any io type, D <= 128). A workgroup
// handles 256 / D tokens of one frame-head; thread (token, i) forms entry i
// of the four products, dbeta is reduced over the token's D threads.
template <typename TIn, int D>
__global__ void __launch_bounds__(256) token_grad_generic(
    const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ beta,
    const TIn* __restrict__ dout, const float* __restrict__ states,
    const float* __restrict__ states2, const float* __restrict__ gbuf,
    const float* __restrict__ ginit, const float* __restrict__ P, TIn* __restrict__ dq,
    TIn* __restrict__ dk, TIn* __restrict__ dv, float* __restrict__ dbeta, int S, int T,
    int ntile, float c, int prepared) {
  constexpr int TPW = 256 / D;
  constexpr int64_t DD = (int64_t)D * D;
  __shared__ float kh[TPW][D], vs[TPW][D], ds[TPW][D], red[TPW][D];
  const int64_t f = blockIdx.x / ntile;
  const int tile = blockIdx.x % ntile;
  const int64_t bh = f / T;
  const int t = (int)(f % T);
  const int tl = threadIdx.x / D, i = threadIdx.x % D;
  const int s = tile * TPW + tl;
  const bool on = s < S;
  const int64_t row = (f * S + (on ? s : 0)) * D;
  auto ld = [&](const TIn* p, int64_t idx) -> float {
    if constexpr (sizeof(TIn) == 2) return bf16_to_f32(((const uint16_t*)p)[idx]);
    else return ((const float*)p)[idx];
  };
  auto st = [&](TIn* p, int64_t idx, float x) {
    if constexpr (sizeof(TIn) == 2) ((uint16_t*)p)[idx] = (uint16_t)(pack_bf16x2(x, 0.f) & 0xFFFFu);
    else ((float*)p)[idx] = x;
  };
  const float kraw = on ? ld(k, row + i) : 0.f;
  kh[tl][i] = prepared ? kraw : (kraw > 0.f ? kraw : 0.f) * c;
  vs[tl][i] = on ? ld(v, row + i) : 0.f;
  ds[tl][i] = on ? ld(dout, row + i) : 0.f;
  __syncthreads();
  const float* St = states + f * DD;
  const float* S2t = states2 ? states2 + f * DD : nullptr;
  const float* Gt = t == T - 1 ? ginit + bh * DD : gbuf + (f + 1) * DD;
  const float* Pt = P + f * DD;
  float dqv = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
  for (int j = 0; j < D; ++j) {
    const float sji = St[(int64_t)j * D + i] + (S2t ? S2t[(int64_t)j * D + i] : 0.f);
    dqv = fmaf(sji, ds[tl][j], dqv);
    y1 = fmaf(Pt[(int64_t)i * D + j], kh[tl][j], y1);
    y2 = fmaf(Gt[(int64_t)j * D + i], vs[tl][j], y2);
    y3 = fmaf(Gt[(int64_t)i * D + j], kh[tl][j], y3);
  }
  const float b = on ? beta[f * S + s] : 0.f;
  red[tl][i] = 0.5f * kh[tl][i] * y1 + vs[tl][i] * y3;
  if (on) {
    if (dq) st(dq, row + i, dqv);
    const float dkh = b * (y1 + y2);
    if (dk) st(dk, row + i, prepared ? dkh : (kraw > 0.f ? dkh * c : 0.f));
    if (dv) st(dv, row + i, b * y3);
  }
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (i < w) red[tl][i] += red[tl][i + w];
    __syncthreads();
  }
  if (on && i == 0 && dbeta != nullptr) dbeta[f * S + s] = red[tl][0];
}

// MFMA path of the per-token gradients (bf16, D = 128), dq excluded (it is
// the readout with the state transposed). Per frame-head, P_t, G_t and
// G_t^T are staged once in LDS as bf16 MFMA "A" operands (rows i,
// contraction j contiguous, chunk-swizzled like the readout's state); each
// wave streams 32-token tiles of k and v as "B" operands:
//   pass 1: Y1 = P ReLU(k) c, Y2 = G^T v  ->  dk = beta c [k > 0] (Y1 + Y2),
//           dbeta = k_hat . (Y1 / 2 + Y2)   (v^T G k_hat = k_hat . G^T v);
//   pass 2: Y3 = G ReLU(k) c              ->  dv = beta Y3.
// The accumulators hold tokens as columns; each result tile goes through a
// per-wave LDS buffer so that a row pass can combine it with the token's raw
// key (mask, dbeta) and write 16-byte chunks of contiguous token rows.
constexpr int kTgTok = 32;    // tokens per wave tile
constexpr int kTgWaves = 4;
constexpr int kTgXcd = 8;

__device__ __forceinline__ int tswz(int row, int chunk) { return chunk ^ (row & 7); }

// 16 bytes of token row min(s, S - 1) (features j .. j + 7). Rows past the
// end repeat the last token: an MFMA output column depends only on its own
// token and those columns are never stored, so no zeroing is needed, and the
// load stays unconditional (a select on it becomes an exec-masked load, which
// makes the compiler drain every prefetch at the loop's back edge).
__device__ __forceinline__ uint4 ld_row16(const uint16_t* base, int s, int S, int j) {
  return *(const uint4*)(base + (int64_t)min(s, S - 1) * 128 + j);
}

// Sum over the 16 lanes of a DPP row (rotations by 1, 2, 4, 8).
__device__ __forceinline__ float sum_row16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  return x;
}

// kAll: dk, dv and dbeta are all wanted, so no store sits behind a pointer
// test (on a path without stores the prefetch loads would be the youngest
// memory operations, and the loop's back edge would wait for all of them).
template <bool kPrepared, bool kAll>
__global__ void __launch_bounds__(256, 1)
token_grad_mfma_bf16_d128(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                          const float* __restrict__ beta, const float* __restrict__ gbuf,
                          const float* __restrict__ ginit, const float* __restrict__ P,
                          uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                          float* __restrict__ dbeta, int S, int T,
                          int64_t FH, int nb, float c) {
  constexpr int D = 128;
  constexpr int64_t DD = (int64_t)D * D;
  __shared__ uint4 Pl[D * 16], Gl[D * 16], GTl[D * 16];           // 3 x 32 KB
  __shared__ uint4 Zs[kTgWaves][kTgTok * 16], Ws[kTgWaves][kTgTok * 16];  // 2 x 4 x 8 KB

  const int xcd = blockIdx.x % kTgXcd;
  const int slot = blockIdx.x / kTgXcd;
  const int64_t fh = (int64_t)(slot / nb) * kTgXcd + xcd;
  const int b = slot % nb;
  if (fh >= FH) return;
  const int64_t bh = fh / T;
  const int t = (int)(fh % T);
  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: read it into a scalar so that
  // the tile loop below is uniform control flow (no exec-masked loads)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  {
    const float* Pt = P + fh * DD;
    const float* Gt = t == T - 1 ? ginit + bh * DD : gbuf + (fh + 1) * DD;
    for (int cc = tid; cc < D * 16; cc += 256) {
      const int i = cc >> 4;
      const int ch = cc & 15;
      const int64_t off = (int64_t)i * D + 8 * ch;
      const float4 p0 = *(const float4*)(Pt + off), p1 = *(const float4*)(Pt + off + 4);
      const float4 g0 = *(const float4*)(Gt + off), g1 = *(const float4*)(Gt + off + 4);
      Pl[i * 16 + tswz(i, ch)] = make_uint4(pack_bf16x2(p0.x, p0.y), pack_bf16x2(p0.z, p0.w),
                                            pack_bf16x2(p1.x, p1.y), pack_bf16x2(p1.z, p1.w));
      Gl[i * 16 + tswz(i, ch)] = make_uint4(pack_bf16x2(g0.x, g0.y), pack_bf16x2(g0.z, g0.w),
                                            pack_bf16x2(g1.x, g1.y), pack_bf16x2(g1.z, g1.w));
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = Gt[(int64_t)(8 * ch + e) * D + i];
      GTl[i * 16 + tswz(i, ch)] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                             pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
    }
  }
  __syncthreads();

  const uint16_t* kf = k + fh * (int64_t)S * D;
  const uint16_t* vf = v + fh * (int64_t)S * D;
  const float* bf = beta + fh * (int64_t)S;
  uint16_t* dkf = dk ? dk + fh * (int64_t)S * D : nullptr;
  uint16_t* dvf = dv ? dv + fh * (int64_t)S * D : nullptr;
  float* dbf = dbeta ? dbeta + fh * (int64_t)S : nullptr;
  const int ntiles = (S + kTgTok - 1) / kTgTok;
  const int wstride = nb * kTgWaves;
  int tile = b * kTgWaves + wave;
  if (tile >= ntiles) return;
  uint4* zs = Zs[wave];
  uint4* ws = Ws[wave];
  const float ck = kPrepared ? 1.f : c;  // key scale carried by the products of ReLU(k)

  // B operands of the tile (token l32, features 16 kk + 8 half ..) and, for
  // the row passes, the raw key chunk (8 ch ..) and gate of rows 4 it + lane/16;
  // all prefetched one tile ahead
  const int rch = lane & 15;
  const int rrow = lane >> 4;
  uint4 kb[8], vb[8], kr[8];
  float br[8], bl;
  auto fetch = [&](int tl) {
    const int s = tl * kTgTok + l32;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      kb[kk] = ld_row16(kf, s, S, 16 * kk + 8 * half);
      vb[kk] = ld_row16(vf, s, S, 16 * kk + 8 * half);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int sr = tl * kTgTok + 4 * it + rrow;
      kr[it] = ld_row16(kf, sr, S, 8 * rch);
      br[it] = bf[min(sr, S - 1)];  // rows past the end are never stored
    }
    bl = bf[min(tl * kTgTok + l32, S - 1)];  // gate of this lane's token column
  };
  fetch(tile);
  // staged tile -> per-row pass over the 32 tokens: lane handles 16-byte
  // chunk (lane & 15) of rows 4 it + lane / 16
  for (; tile < ntiles; tile += wstride) {
    bf16x8_t bk[8], bv[8];
    uint4 krc[8];
    float brc[8];
    const float blc = bl;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      krc[it] = kr[it];
      brc[it] = br[it];
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 x = kb[kk];
      if (!kPrepared) {
        x.x = relu_bf16x2_pk(x.x);
        x.y = relu_bf16x2_pk(x.y);
        x.z = relu_bf16x2_pk(x.z);
        x.w = relu_bf16x2_pk(x.w);
      }
      bk[kk] = __builtin_bit_cast(bf16x8_t, x);
      bv[kk] = __builtin_bit_cast(bf16x8_t, vb[kk]);
    }
    const int s0 = tile * kTgTok;
    const int nxt = tile + wstride;
    if (nxt < ntiles) fetch(nxt);
    // ---- pass 1: Y1 = P k_hat, Y2 = G^T v
    {
      f32x16_t y1[4], y2[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) y1[mt][j] = y2[mt][j] = 0.f;
      uint4 pa[2][4], ga[2][4];
      auto frag1 = [&](int buf, int kk) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = 32 * mt + l32;
          const int at = row * 16 + tswz(row, 2 * kk + half);
          pa[buf][mt] = Pl[at];
          ga[buf][mt] = GTl[at];
        }
      };
      frag1(0, 0);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (kk + 1 < 8) frag1((kk + 1) & 1, kk + 1);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          y1[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, pa[kk & 1][mt]),
                                                           bk[kk], y1[mt], 0, 0, 0);
          y2[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ga[kk & 1][mt]),
                                                           bv[kk], y2[mt], 0, 0, 0);
        }
      }
      // accumulator (i, s): token s = l32, rows i = 32 mt + 8 jg + 4 half + (0..3)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          float z[4], w[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a1 = y1[mt][4 * jg + r] * ck, a2 = y2[mt][4 * jg + r];
            z[r] = a1 + a2;
            w[r] = 0.5f * a1 + a2;
          }
          const int at = l32 * 16 + tswz(l32, 4 * mt + jg);
          ((uint2*)&zs[at])[half] = make_uint2(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]));
          ((uint2*)&ws[at])[half] = make_uint2(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = 4 * it + rrow;
      const int ch = rch;
      const int s = s0 + row;
      const uint4 zc = zs[row * 16 + tswz(row, ch)];
      const uint4 wc = ws[row * 16 + tswz(row, ch)];
      const uint4 kc = krc[it];
      const float bt = brc[it];
      const uint32_t zw[4] = {zc.x, zc.y, zc.z, zc.w};
      const uint32_t ww[4] = {wc.x, wc.y, wc.z, wc.w};
      const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
      uint32_t out[4];
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float k0 = __uint_as_float(kw[q] << 16), k1 = __uint_as_float(kw[q] & 0xFFFF0000u);
        const float z0 = __uint_as_float(zw[q] << 16), z1 = __uint_as_float(zw[q] & 0xFFFF0000u);
        const float w0 = __uint_as_float(ww[q] << 16), w1 = __uint_as_float(ww[q] & 0xFFFF0000u);
        float h0, h1, m0, m1;
        if (kPrepared) {
          h0 = k0; h1 = k1; m0 = m1 = 1.f;
        } else {
          h0 = (k0 > 0.f ? k0 : 0.f) * c; h1 = (k1 > 0.f ? k1 : 0.f) * c;
          m0 = k0 > 0.f ? c : 0.f; m1 = k1 > 0.f ? c : 0.f;
        }
        part += h0 * w0 + h1 * w1;
        out[q] = pack_bf16x2(bt * m0 * z0, bt * m1 * z1);
      }
      part = sum_row16(part);  // the 16 lanes of this token row
      // Every store is issued (a store under a per-lane condition makes the
      // compiler drain the prefetch). A row past the end was computed from
      // clamped copies of row S - 1, so it holds exactly row S - 1's values
      // and is written there again.
      const int sc = min(s, S - 1);
      if (kAll || dkf) *(uint4*)(dkf + (int64_t)sc * D + 8 * ch) = make_uint4(out[0], out[1], out[2], out[3]);
      if (kAll || dbf) dbf[sc] = part;  // the row's 16 lanes agree
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- pass 2: Y3 = G k_hat, dv = beta Y3
    if (kAll || dvf) {
      f32x16_t y3[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) y3[mt][j] = 0.f;
      uint4 gf[2][4];
      auto frag3 = [&](int buf, int kk) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = 32 * mt + l32;
          gf[buf][mt] = Gl[row * 16 + tswz(row, 2 * kk + half)];
        }
      };
      frag3(0, 0);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (kk + 1 < 8) frag3((kk + 1) & 1, kk + 1);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          y3[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, gf[kk & 1][mt]),
                                                           bk[kk], y3[mt], 0, 0, 0);
      }
      const float bt = blc * ck;  // columns past the end are never stored
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int at = l32 * 16 + tswz(l32, 4 * mt + jg);
          ((uint2*)&zs[at])[half] =
              make_uint2(pack_bf16x2(bt * y3[mt][4 * jg], bt * y3[mt][4 * jg + 1]),
                         pack_bf16x2(bt * y3[mt][4 * jg + 2], bt * y3[mt][4 * jg + 3]));
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = 4 * it + (lane >> 4);
        const int ch = lane & 15;
        const int sc = min(s0 + row, S - 1);  // see the dk store
        *(uint4*)(dvf + (int64_t)sc * D + 8 * ch) = zs[row * 16 + tswz(row, ch)];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// MFMA path of the per-frame gradients (D = 128): dM = S_prev^T G on fp32
// MFMA (v_mfma_f32_32x32x2_f32: exact fp32 products), wave w owns rows
// 32w .. 32w + 31 of dM as four 32 x 32 tiles. The A operand of lane l is
// S_prev[i][32w + l % 32] with i = 2 ks + l / 32, the B operand
// G[i][32 nb + l % 32]; both are conflict-free row reads of the staged
// matrices.
__global__ void __launch_bounds__(256, 1)
frame_grad_mfma_d128(const float* __restrict__ states, const float* __restrict__ s0,
                     float* __restrict__ gbuf, float* __restrict__ ginit,
                     const float* __restrict__ terms, int a_granule_bf16,
                     const float* __restrict__ gamma, float* __restrict__ P,
                     float* __restrict__ dgamma, int T, RevGrad rg) {
  constexpr int D = 128;
  constexpr int LDT = D + 4;  // padded row for the transposed read of dM
  constexpr int64_t DD = (int64_t)D * D;
  __shared__ float Ss[D][LDT];
  __shared__ float Gs[D][D];
  __shared__ float red[4];
  const int64_t f = blockIdx.x;
  const int64_t bh = f / T;
  const int t = (int)(f % T);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hk = lane >> 5;
  const float* Sp = t > 0 ? states + (f - 1) * DD : (s0 ? s0 + bh * DD : nullptr);
  float* Gt = t == T - 1 ? ginit + bh * DD : gbuf + (f + 1) * DD;
  const float* At = terms + f * 2 * DD;
  // A_t entries of this lane's accumulators (see the epilogue), loaded before
  // the products so that their latency is hidden: in the bf16 granule layout
  // the four entries a = 32 w + 8 jg + 4 hk + 0..3 of column b = 32 nb + l32
  // are one 8-byte piece of granule (b, 4 w + jg)
  uint2 ag[4][4];
  if (a_granule_bf16) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg)
        ag[nb][jg] = *(const uint2*)((const uint16_t*)At +
                                     (int64_t)a_granule(32 * nb + l32, 4 * wave + jg) * 8 + 4 * hk);
  }
  // S_prev and G_t into LDS: all 32 loads of a thread are issued before the
  // first LDS write, so the staging costs one memory round trip
  {
    constexpr int kPer = D * D / 4 / 256;
    float4 sv[kPer], gv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      const int r = e / (D / 4), c4 = 4 * (e % (D / 4));
      sv[u] = Sp ? *(const float4*)(Sp + (int64_t)r * D + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
      gv[u] = *(const float4*)(Gt + (int64_t)r * D + c4);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      const int r = e / (D / 4), c4 = 4 * (e % (D / 4));
      Ss[r][c4] = sv[u].x; Ss[r][c4 + 1] = sv[u].y; Ss[r][c4 + 2] = sv[u].z; Ss[r][c4 + 3] = sv[u].w;
      *(float4*)&Gs[r][c4] = gv[u];
    }
  }
  __syncthreads();
  f32x16_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[nb][j] = 0.f;
  auto product = [&]() {  // acc += Ss^T Gs
#pragma unroll 4
    for (int ks = 0; ks < D / 2; ++ks) {
      const int i = 2 * ks + hk;
      const float a = Ss[i][32 * wave + l32];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Gs[i][32 * nb + l32], acc[nb], 0, 0, 0);
    }
  };
  product();
  // chunk-causal scan: + R_{t+1}^T F_t, and G_t + F_t written over G_t
  if (rg.rev != nullptr) {
    bool more;
    const float* Ft = rev_adjoint(rg, f, bh, t, T, DD, &more);
    const float* Rn = rg.rev + (f + 1) * DD;
    constexpr int kPer = D * D / 4 / 256;
    float4 fv[kPer], rv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      fv[u] = *(const float4*)(Ft + 4 * (int64_t)e);
      rv[u] = more ? *(const float4*)(Rn + 4 * (int64_t)e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();  // every wave is done with Ss and Gs
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      const int r = e / (D / 4), c4 = 4 * (e % (D / 4));
      const float4 g4 = *(const float4*)&Gs[r][c4];
      *(float4*)(Gt + 4 * (int64_t)e) =
          make_float4(g4.x + fv[u].x, g4.y + fv[u].y, g4.z + fv[u].z, g4.w + fv[u].w);
      *(float4*)&Gs[r][c4] = fv[u];
      Ss[r][c4] = rv[u].x; Ss[r][c4 + 1] = rv[u].y; Ss[r][c4 + 2] = rv[u].z; Ss[r][c4 + 3] = rv[u].w;
    }
    __syncthreads();
    if (more) product();
  }
  // acc[nb][j] = dM[a][b], a = 32 wave + 8 (j / 4) + 4 hk + j % 4, b = 32 nb + l32
  float part = 0.f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int a = 32 * wave + 8 * (j >> 2) + 4 * hk + (j & 3), b = 32 * nb + l32;
      const uint2 w = ag[nb][j >> 2];
      const uint32_t pair = (j & 2) ? w.y : w.x;
      const float av = a_granule_bf16 ? bf16_to_f32((j & 1) ? (pair >> 16) : (pair & 0xFFFFu))
                                      : At[(int64_t)a * D + b];
      part += acc[nb][j] * ((a == b ? 1.f : 0.f) - av);
    }
  part = sum_lane_xor32(sum_lane_xor16(sum_row16(part)));
  if (lane == 0) red[wave] = part;
  __syncthreads();  // every wave is done reading Ss
  const float g = gamma[f];
  if (tid == 0 && dgamma != nullptr) dgamma[f] = red[0] + red[1] + red[2] + red[3];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      Ss[32 * wave + 8 * (j >> 2) + 4 * hk + (j & 3)][32 * nb + l32] = acc[nb][j];
  __syncthreads();
  float* Pf = P + f * DD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int a = 32 * wave + 8 * (j >> 2) + 4 * hk + (j & 3), b = 32 * nb + l32;
      Pf[(int64_t)a * D + b] = -g * (acc[nb][j] + Ss[b][a]);
    }
}

int grid_cap(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

hipError_t launch_grad_init(const Shape& sh, const float* E, const float* ds_final, float* ginit,
                            bool granule, hipStream_t st) {
  const int64_t n = sh.BH() * sh.D * sh.D;
  if (n == 0) return hipSuccess;
  grad_init_kernel<<<grid_cap(n), 256, 0, st>>>(E, ds_final, ginit, sh.T, sh.D, sh.BH(),
                                                granule ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_chunk_init(const Shape& sh, const float* E, int L, int nchunk, float* finit,
                             bool granule, hipStream_t st) {
  const int64_t n = sh.BH() * nchunk * sh.D * sh.D;
  if (n == 0) return hipSuccess;
  if (L < 1 || (int64_t)(nchunk - 1) * L >= sh.T) return hipErrorInvalidValue;
  chunk_init_kernel<<<grid_cap(n), 256, 0, st>>>(E, finit, sh.T, sh.D, L, nchunk, sh.BH(),
                                                 granule ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_frame_grad(const Shape& sh, const float* states, const float* s0, float* gbuf,
                             float* ginit, const float* terms, bool a_granule_bf16,
                             const float* gamma, float* P, float* dgamma, const RevGrad& rg,
                             hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  if (rg.rev != nullptr && (rg.L < 1 || rg.fbuf == nullptr || rg.finit == nullptr ||
                            (int64_t)rg.nchunk * rg.L < sh.T))
    return hipErrorInvalidValue;
  dim3 grid((unsigned)sh.FH());
  const int ag = a_granule_bf16 ? 1 : 0;
  if (sh.D == 128) {
    frame_grad_mfma_d128<<<grid, 256, 0, st>>>(states, s0, gbuf, ginit, terms, ag, gamma, P, dgamma,
                                               sh.T, rg);
    return hipGetLastError();
  }
#define GDN_FG(DV)                                                                              \
  frame_grad_kernel<DV><<<grid, 256, 0, st>>>(states, s0, gbuf, ginit, terms, ag, gamma, P, \
                                              dgamma, sh.T, rg)
  switch (sh.D) {
    case 16: GDN_FG(16); break;
    case 32: GDN_FG(32); break;
    case 64: GDN_FG(64); break;
    case 128: GDN_FG(128); break;
    default: return hipErrorInvalidValue;
  }
#undef GDN_FG
  return hipGetLastError();
}

// Workgroups per frame-head in the token-gradient kernel (each stages P_t and
// G_t once).
#ifndef GDN_TG_NB
#define GDN_TG_NB 1
#endif

bool token_grad_uses_mfma(const Shape& sh) { return sh.io == 1 && sh.D == 128; }

hipError_t launch_token_grad(const Shape& sh, const void* k, const void* v, const float* beta,
                             const void* dout, const float* states, const float* states2,
                             const float* gbuf, const float* ginit, const float* P, void* dq,
                             void* dk, void* dv, float* dbeta, hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  if (token_grad_uses_mfma(sh)) {
    // dq = states^T do: the readout with the state staged transposed (the
    // summed states of the bidirectional scan go through the fused E pass)
    if (dq && states2) return hipErrorInvalidValue;
    if (dq) {
      hipError_t e = launch_readout(sh, dout, states, nullptr, dq, st, true);
      if (e != hipSuccess) return e;
    }
    if (!dk && !dv && !dbeta) return hipSuccess;
    const int ntiles = (sh.S + kTgTok - 1) / kTgTok;
    int nb = (ntiles + kTgWaves - 1) / kTgWaves;
    if (nb > GDN_TG_NB) nb = GDN_TG_NB;
    const int64_t groups = (sh.FH() + kTgXcd - 1) / kTgXcd;
    dim3 grid((unsigned)(groups * kTgXcd * nb));
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    const bool all = dk && dv && dbeta;
#define GDN_TOKEN_GRAD(PR, ALL)                                                                \
  token_grad_mfma_bf16_d128<PR, ALL><<<grid, 256, 0, st>>>(kk, vv, beta, gbuf, ginit, P,       \
                                                           (uint16_t*)dk, (uint16_t*)dv, dbeta, \
                                                           sh.S, sh.T, sh.FH(), nb, sh.c)
    if (sh.prepared) {
      if (all) GDN_TOKEN_GRAD(true, true);
      else GDN_TOKEN_GRAD(true, false);
    } else {
      if (all) GDN_TOKEN_GRAD(false, true);
      else GDN_TOKEN_GRAD(false, false);
    }
#undef GDN_TOKEN_GRAD
    return hipGetLastError();
  }
  const int tpw = 256 / sh.D;
  const int ntile = (sh.S + tpw - 1) / tpw;
  dim3 grid((unsigned)(sh.FH() * ntile));
#define GDN_TG(TT, DV)                                                                        \
  token_grad_generic<TT, DV><<<grid, 256, 0, st>>>(                                          \
      (const TT*)k, (const TT*)v, beta, (const TT*)dout, states, states2, gbuf, ginit, P, (TT*)dq, \
      (TT*)dk, (TT*)dv, dbeta, sh.S, sh.T, ntile, sh.c, sh.prepared)
  if (sh.io == 1) {
    switch (sh.D) {
      case 16: GDN_TG(uint16_t, 16); break;
      case 32: GDN_TG(uint16_t, 32); break;
      case 64: GDN_TG(uint16_t, 64); break;
      case 128: GDN_TG(uint16_t, 128); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (sh.D) {
      case 16: GDN_TG(float, 16); break;
      case 32: GDN_TG(float, 32); break;
      case 64: GDN_TG(float, 64); break;
      case 128: GDN_TG(float, 128); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef GDN_TG
  return hipGetLastError();
}

}  // namespace gdn
