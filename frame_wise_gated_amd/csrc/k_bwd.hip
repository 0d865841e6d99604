// Backward pass of the causal and the chunk-causal frame scan: the per-frame
// and per-token gradient kernels. The adjoint recurrences themselves run on
// the scan kernels (k_scan.hip: REVERSE mode with a shifted U source for G,
// and per chunk FORWARD for the reverse states' adjoint F); phase 1 supplies
// A_t and E_t = dO_t^T Q_t.
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
#include "gdn_dma.h"

namespace gdn {

namespace {

// Granule g of a D = 128 matrix in the scan's layout holds row m, columns
// 4 nc .. 4 nc + 3 (the inverse of u_granule). The granule-layout kernels
// below walk the granules in order, one per thread: their granule-side loads
// are contiguous, and the four lanes that share a row's 16-row group write (or
// read) its row-major side as one 64-byte piece. In row-major order instead,
// every 16-byte granule read fetched a 64-byte sector (4x the bytes).
__device__ __forceinline__ void granule_rc(int g, int* m, int* nc) {
  const int blk = g >> 6, r = g & 63;
  *m = (blk >> 3) * 16 + (r & 15);
  *nc = (blk & 7) * 4 + (r >> 4);
}

// G_{T-1} = E_{T-1} + dS_final for every head (row-major output). E is in the
// scan's granule layout when `granule` (D = 128), fp32 row-major otherwise.
__global__ void __launch_bounds__(256) grad_init_kernel(const float* __restrict__ E,
                                                        const float* __restrict__ ds_final,
                                                        float* __restrict__ ginit, int T, int D,
                                                        int64_t BH, int granule) {
  const int64_t DD = (int64_t)D * D;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (granule) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < BH * (DD / 4); i += stride) {
      const int64_t bh = i / (DD / 4);
      const int g = (int)(i % (DD / 4));
      int m, nc;
      granule_rc(g, &m, &nc);
      float4 x = ((const float4*)(E + (bh * T + (T - 1)) * DD))[g];
      const int64_t o = bh * DD + (int64_t)m * D + 4 * nc;
      const float4 d = ds_final ? *(const float4*)(ds_final + o) : make_float4(0.f, 0.f, 0.f, 0.f);
      x.x += d.x;
      x.y += d.y;
      x.z += d.z;
      x.w += d.w;
      *(float4*)(ginit + o) = x;
    }
    return;
  }
  const int64_t n_all = BH * DD;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_all; i += stride) {
    const int64_t bh = i / DD;
    const int e = (int)(i % DD);
    const float* Et = E + (bh * T + (T - 1)) * DD;
    ginit[i] = Et[e] + (ds_final ? ds_final[i] : 0.f);
  }
}

// F at the first frame of every chunk of the bidirectional backward:
// finit[bh][c] = E_{c L} (row-major output; E in the scan's granule layout
// when `granule`, D = 128).
__global__ void __launch_bounds__(256) chunk_init_kernel(const float* __restrict__ E,
                                                         float* __restrict__ finit, int T, int D,
                                                         int L, int nchunk, int64_t BH,
                                                         int granule) {
  const int64_t DD = (int64_t)D * D;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (granule) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < BH * nchunk * (DD / 4);
         i += stride) {
      const int64_t bc = i / (DD / 4);
      const int64_t bh = bc / nchunk;
      const int c = (int)(bc % nchunk);
      const int g = (int)(i % (DD / 4));
      int m, nc;
      granule_rc(g, &m, &nc);
      const float4 x = ((const float4*)(E + (bh * T + (int64_t)c * L) * DD))[g];
      *(float4*)(finit + bc * DD + (int64_t)m * D + 4 * nc) = x;
    }
    return;
  }
  const int64_t n_all = BH * nchunk * DD;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_all; i += stride) {
    const int64_t bc = i / DD;
    const int64_t bh = bc / nchunk;
    const int c = (int)(bc % nchunk);
    const int e = (int)(i % DD);
    finit[i] = E[(bh * T + (int64_t)c * L) * DD + e];
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
// of the four products, per-token sums run over the token's D threads.
// With `norm` (the RMSNorm of q and k, raw keys only for k): the keys enter
// the products as c ReLU(k r_k), and dq, dk pass back through the norm,
// dx = r (dy - (y . dy) y / D) with y = x r.
template <typename TIn, int D>
__global__ void __launch_bounds__(256) token_grad_generic(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ beta, const TIn* __restrict__ dout, const float* __restrict__ states,
    const float* __restrict__ states2, const float* __restrict__ gbuf,
    const float* __restrict__ ginit, const float* __restrict__ P, TIn* __restrict__ dq,
    TIn* __restrict__ dk, TIn* __restrict__ dv, float* __restrict__ dbeta, int S, int T,
    int ntile, float c, int prepared, int norm) {
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
  // sum over the D threads of this token (every thread of the block calls it)
  auto rowsum = [&](float x) -> float {
    __syncthreads();
    red[tl][i] = x;
    __syncthreads();
    for (int w = D / 2; w > 0; w >>= 1) {
      if (i < w) red[tl][i] += red[tl][i + w];
      __syncthreads();
    }
    return red[tl][0];
  };
  const bool knorm = norm && !prepared;  // prepared keys are used as given
  const float kraw = on ? ld(k, row + i) : 0.f;
  const float rk = knorm ? rms_inv(rowsum(kraw * kraw), D) : 1.f;
  const float kt = kraw * rk;  // the key before its ReLU
  kh[tl][i] = prepared ? kraw : (kt > 0.f ? kt : 0.f) * c;
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
  const float dbsum = rowsum(0.5f * kh[tl][i] * y1 + vs[tl][i] * y3);
  // dk: through the ReLU and the key scale, then through the norm
  const float dkh = b * (y1 + y2);
  float dkv = prepared ? dkh : (kt > 0.f ? dkh * c : 0.f);
  if (knorm) dkv = rk * (dkv - rowsum(kt * dkv) * kt / (float)D);
  // dq: through the norm of the query
  if (norm && dq) {
    const float qraw = on ? ld(q, row + i) : 0.f;
    const float rq = rms_inv(rowsum(qraw * qraw), D);
    const float qh = qraw * rq;
    dqv = rq * (dqv - rowsum(qh * dqv) * qh / (float)D);
  }
  if (on) {
    if (dq) st(dq, row + i, dqv);
    if (dk) st(dk, row + i, dkv);
    if (dv) st(dv, row + i, b * y3);
    if (i == 0 && dbeta != nullptr) dbeta[f * S + s] = dbsum;
  }
}


// Weights-stationary MFMA path of the per-token gradients (bf16, D = 128).
// Wave w keeps rows 32 w .. 32 w + 31 of P_t, G_t^T and G_t as bf16 MFMA
// "A" fragments in registers (96 VGPRs) for the whole frame, and the frame's
// tokens stream through a ring of 32-token LDS stages filled by direct
// global -> LDS copies, so no register holds a prefetch and k is read once for
// both the MFMA operand and the gradients. Per stage every wave forms its 32
// rows of Y1 = P relu(k), Y2 = G^T v and Y3 = G relu(k) for the 32 tokens and,
// still in fp32 registers, with Z = c Y1 + Y2 and W = c Y1 / 2 + Y2, its
// features of dk = beta c [k > 0] Z (prepared keys: beta Z) and dv = beta c Y3
// and its part of dbeta = k_hat . W; it drops dk and dv into LDS (bf16, token
// rows) and one partial dbeta per token. A store pass then writes whole
// 16-byte row chunks. Waves 0-1 issue every copy (their vmcnt counts copies
// only, so the explicit waits are exact) and waves 2-3 issue every store. Two
// workgroups fit a CU (66 KB of LDS each).
constexpr int kWsTok = 32;                       // tokens per stage
constexpr int kWsNst = 3;                        // ring stages
constexpr int kWsKv = kWsTok * 256;              // one stage of k (or v): 32 rows x 256 B
constexpr int kWsSlot = 2 * kWsKv + 4 * kWsTok;  // k, v, the stage's gates

// byte offset of 16-byte chunk ch of token row r in a stage tensor: row r at
// 256 r, chunk ch at position ch ^ (r % 16), so 16 consecutive rows read at
// one chunk, or one row read at 16 chunks, hit distinct banks
__device__ __forceinline__ int ws_at(int r, int ch) { return r * 256 + ((ch ^ (r & 15)) << 4); }

__device__ __forceinline__ bf16x8_t pack8(float4 a, float4 b) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w),
                                                 pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)));
}

// kNorm (the RMSNorm of the raw keys): the copying waves normalise their own
// key copies in place (k r, r = 1 / rms(k); the 16 chunks of a token sit in
// one DPP row) and keep r per token; the waves form dkt, the gradient for
// kt = k r, and their parts of kt . dkt, and the store pass takes dk through
// the norm, dk = r (dkt - (kt . dkt) kt / D).
template <bool kPrepared, bool kNorm>
__global__ void __launch_bounds__(256, 2)
token_grad_ws_bf16_d128(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                        const float* __restrict__ beta, const float* __restrict__ gbuf,
                        const float* __restrict__ ginit, const float* __restrict__ P,
                        uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                        float* __restrict__ dbeta, int S, int T, int64_t FH, int nb, float c) {
  constexpr int D = 128;
  constexpr int64_t DD = (int64_t)D * D;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWsNst][kWsSlot];
  __shared__ __attribute__((aligned(16))) uint8_t Zs[kWsKv];   // dk (kNorm: dkt) of the stage
  __shared__ __attribute__((aligned(16))) uint8_t Vsb[kWsKv];  // dv of the stage
  __shared__ float dbp[4][kWsTok];                              // per-wave parts of dbeta
  __shared__ float dkp[kNorm ? 4 : 1][kWsTok];                  // per-wave parts of kt . dkt
  __shared__ float rks[kNorm ? kWsNst : 1][kWsTok];  // 1 / rms of each token's key

  // nb workgroups per frame-head, all on one XCD (consecutive workgroups go
  // to consecutive XCDs); part p takes stages p, p + nb, p + 2 nb, .. so the
  // frame-head's workgroups sweep it together
  const int xcd = blockIdx.x % 8;
  const int slot_id = blockIdx.x / 8;
  const int64_t f = (int64_t)(slot_id / nb) * 8 + xcd;  // frame-head
  const int part = slot_id % nb;
  if (f >= FH) return;
  const int64_t bh = f / T;
  const int t = (int)(f % T);
  const int stages = (S + kWsTok - 1) / kWsTok;
  const int nmine = stages > part ? (stages - part + nb - 1) / nb : 0;  // stages of this part
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const uint16_t* kf = k + f * (int64_t)S * D;
  const uint16_t* vf = v + f * (int64_t)S * D;
  const float* bf = beta + f * (int64_t)S;
  const float ck = kPrepared ? 1.f : c;  // key scale carried by the products of relu(k)

  // this wave's rows of P_t, G_t^T, G_t: fragment kk holds columns
  // 16 kk + 8 h .. + 7 of row 32 w + l32
  const float* Pt = P + f * DD;
  const float* Gt = t == T - 1 ? ginit + bh * DD : gbuf + (f + 1) * DD;
  const int row = 32 * wave + l32;
  bf16x8_t pa[8], gta[8], ga[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int j0 = 16 * kk + 8 * h;
    pa[kk] = pack8(*(const float4*)(Pt + row * D + j0), *(const float4*)(Pt + row * D + j0 + 4));
    ga[kk] = pack8(*(const float4*)(Gt + row * D + j0), *(const float4*)(Gt + row * D + j0 + 4));
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = Gt[(j0 + e) * D + row];
    gta[kk] = pack8(make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7]));
  }

  // copies of stage st (waves 0-1): wave w fills 4-token blocks 4 w .. 4 w + 3
  // of k and v (lane i of a block's instruction lands at byte 16 i of the
  // block, i.e. row 4 blk + i / 16 at chunk position i % 16, so it loads the
  // chunk (i % 16) ^ (row % 16)) and the gates of tokens 16 w .. 16 w + 15.
  // Tokens past the end copy row S - 1.
  constexpr int kOps = 9;  // copy instructions per copying wave and stage
  // j-th stage of this part: tokens 32 (part + j nb) ..; ring slot j % kWsNst
  auto issue = [&](int j) {
    const int st = part + j * nb;
    uint8_t* slot = ring[j % kWsNst];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int blk = 4 * wave + b;
      const int r = 4 * blk + (lane >> 4);
      const int ch = (lane & 15) ^ (r & 15);
      const int64_t off = (int64_t)min(st * kWsTok + r, S - 1) * D + 8 * ch;
      dma16(kf + off, slot + 1024 * blk);
      dma16(vf + off, slot + kWsKv + 1024 * blk);
    }
    dma4(bf + min(st * kWsTok + 16 * wave + (lane & 15), S - 1), slot + 2 * kWsKv + 64 * wave,
         lane < 16);
  };
  if (wave < 2) {
#pragma unroll
    for (int i = 0; i < kWsNst - 1; ++i) issue(i);
  }
  uint16_t* dkf = dk ? dk + f * (int64_t)S * D : nullptr;
  uint16_t* dvf = dv ? dv + f * (int64_t)S * D : nullptr;
  float* dbf = dbeta ? dbeta + f * (int64_t)S : nullptr;

  for (int j = 0; j < nmine; ++j) {
    const int st = part + j * nb;
    if (wave < 2) {
      wait_vmcnt_lgkm0<(kWsNst - 2) * kOps>();  // this wave's copies of stage j
      if (kNorm) {
        uint8_t* slot_w = ring[j % kWsNst];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int blk = 4 * wave + b;
          uint4* pk = (uint4*)(slot_w + 1024 * blk + 16 * lane);
          const uint4 x = *pk;
          const uint32_t w0[4] = {x.x, x.y, x.z, x.w};
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = sumsq_bf16x2(w0[e], ss);
          const float r = rms_inv(sum_row16(ss), D);
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16x2(__uint_as_float(w0[e] << 16) * r, __uint_as_float(w0[e] & 0xFFFF0000u) * r);
          *pk = make_uint4(o[0], o[1], o[2], o[3]);
          if ((lane & 15) == 0) rks[kNorm ? j % kWsNst : 0][4 * blk + (lane >> 4)] = r;
        }
        wait_vmcnt_lgkm0<63>();  // lgkmcnt(0): the normalised keys are written
      }
    } else {
      wait_vmcnt_lgkm0<63>();  // lgkmcnt(0)
    }
    bare_barrier();  // stage j has landed; stage j - 1's slot and the staging are free
    if (wave < 2) issue(j + kWsNst - 1);
    const uint8_t* slot = ring[j % kWsNst];
    const float* gates = (const float*)(slot + 2 * kWsKv);
    f32x16_t y1, y2, y3;
#pragma unroll
    for (int j = 0; j < 16; ++j) y1[j] = y2[j] = y3[j] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int at = ws_at(l32, 2 * kk + h);
      uint4 kb = *(const uint4*)(slot + at);
      const uint4 vb = *(const uint4*)(slot + kWsKv + at);
      if (!kPrepared) {
        kb.x = relu_bf16x2_pk(kb.x);
        kb.y = relu_bf16x2_pk(kb.y);
        kb.z = relu_bf16x2_pk(kb.z);
        kb.w = relu_bf16x2_pk(kb.w);
      }
      const bf16x8_t kv8 = __builtin_bit_cast(bf16x8_t, kb);
      y1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], kv8, y1, 0, 0, 0);
      y2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gta[kk], __builtin_bit_cast(bf16x8_t, vb), y2, 0, 0, 0);
      y3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[kk], kv8, y3, 0, 0, 0);
    }
    // lane (h, l32): token l32, features 32 w + 8 jg + 4 h + 0..3, and the
    // key's same four features (kNorm: normalised) at the same place of its row
    const float bt = gates[l32];
    const float bc = bt * ck;
    float pb = 0.f, pk = 0.f;  // this lane's parts of dbeta and (kNorm) kt . dkt
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int at = ws_at(l32, 4 * wave + jg) + 8 * h;
      const uint2 kq = *(const uint2*)(slot + at);
      const float kv[4] = {__uint_as_float(kq.x << 16), __uint_as_float(kq.x & 0xFFFF0000u),
                           __uint_as_float(kq.y << 16), __uint_as_float(kq.y & 0xFFFF0000u)};
      float dk4[4], d[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a1 = y1[4 * jg + r] * ck, a2 = y2[4 * jg + r];
        const float z = a1 + a2, wv = 0.5f * a1 + a2;
        float kh, m;
        if (kPrepared) {
          kh = kv[r];
          m = 1.f;
        } else {
          kh = (kv[r] > 0.f ? kv[r] : 0.f) * c;
          m = kv[r] > 0.f ? c : 0.f;
        }
        pb += kh * wv;
        dk4[r] = bt * m * z;
        if (kNorm) pk += kv[r] * dk4[r];
        d[r] = bc * y3[4 * jg + r];
      }
      *(uint2*)(Zs + at) = make_uint2(pack_bf16x2(dk4[0], dk4[1]), pack_bf16x2(dk4[2], dk4[3]));
      *(uint2*)(Vsb + at) = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
    }
    // lanes l32 and l32 + 32 hold different features of one token
    pb = sum_lane_xor32(pb);
    if (kNorm) pk = sum_lane_xor32(pk);
    if (h == 0) {
      dbp[wave][l32] = pb;
      if (kNorm) dkp[kNorm ? wave : 0][l32] = pk;
    }
    wait_vmcnt_lgkm0<63>();  // lgkmcnt(0): the staged tiles are written
    bare_barrier();
    if (wave >= 2) {
      // store pass: thread u handles chunk u % 16 of rows u / 16 + 8 m. Rows
      // past the end were computed from copies of row S - 1, hold its values
      // and are written there again.
      const int u = tid - 128;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = u + 128 * m;
        const int r = i >> 4, ch = i & 15;
        const int at = ws_at(r, ch);
        uint4 dkc = *(const uint4*)(Zs + at);
        if (kNorm) {  // through the norm of the key
          const uint4 kc = *(const uint4*)(slot + at);
          const float proj =
              (dkp[0][r] + dkp[kNorm ? 1 : 0][r] + dkp[kNorm ? 2 : 0][r] + dkp[kNorm ? 3 : 0][r]) / (float)D;
          const float rr = rks[kNorm ? j % kWsNst : 0][r];
          const uint32_t dw[4] = {dkc.x, dkc.y, dkc.z, dkc.w};
          const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
          uint32_t out[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float d0 = __uint_as_float(dw[q] << 16), d1 = __uint_as_float(dw[q] & 0xFFFF0000u);
            const float k0 = __uint_as_float(kw[q] << 16), k1 = __uint_as_float(kw[q] & 0xFFFF0000u);
            out[q] = pack_bf16x2(rr * (d0 - proj * k0), rr * (d1 - proj * k1));
          }
          dkc = make_uint4(out[0], out[1], out[2], out[3]);
        }
        const int64_t sr = min(st * kWsTok + r, S - 1);
        if (dkf) *(uint4*)(dkf + sr * D + 8 * ch) = dkc;
        if (dvf) *(uint4*)(dvf + sr * D + 8 * ch) = *(const uint4*)(Vsb + at);
        if (dbf && ch == 0) dbf[sr] = dbp[0][r] + dbp[1][r] + dbp[2][r] + dbp[3][r];
      }
    }
  }
  wait_vmcnt_lgkm0<0>();  // no copy may still be landing in LDS when the workgroup retires
}

// MFMA path of the per-frame gradients (D = 128): dM = S_prev^T G on bf16
// MFMA with both operands split into hi/lo bf16 pairs (Sh Gh + Sl Gh + Sh Gl,
// fp32 accumulation; |X - Xh - Xl| <= 2^-17 |X|), about 16 significant bits
// per product as in the scan's own steps, while P_t leaves for the token
// kernel rounded to bf16. Wave w owns rows 32w .. 32w + 31 of dM as four
// 32 x 32 tiles. The first operand of lane l is S_prev[i][32w + l % 32] for
// the eight i = 16 ks + 8 (l / 32) + 0..7 of step ks: the wave's 64 values
// per lane are loaded straight into registers (coalesced 128-byte row
// pieces) and split there. The second operand, G[i][32 nb + l % 32] for the
// same i, is shared by the four waves: G_t sits in LDS transposed as a hi/lo
// pair (row b holds column b, 16-byte chunk c = rows 8c .. 8c + 7 at position
// c ^ (b % 16)), one 16-byte read per fragment. The same 66 KB then hold the
// chunk-causal scan's F_t, and finally dM for its transposed read: two
// workgroups per CU, so that one's loads overlap the other's products.
__global__ void __launch_bounds__(256, 2)
frame_grad_mfma_d128(const float* __restrict__ states, const float* __restrict__ s0,
                     float* __restrict__ gbuf, float* __restrict__ ginit,
                     const float* __restrict__ terms, int a_granule_bf16,
                     const float* __restrict__ gamma, float* __restrict__ P,
                     float* __restrict__ dgamma, int T, RevGrad rg) {
  constexpr int D = 128;
  constexpr int LDT = D + 4;  // padded row for the transposed read of dM
  constexpr int64_t DD = (int64_t)D * D;
  __shared__ __attribute__((aligned(16))) float Ws[D][LDT];
  static_assert(sizeof(Ws) >= 2 * D * 16 * sizeof(uint4), "the hi/lo operand pair fits the dM buffer");
  uint4* const Bh = (uint4*)&Ws[0][0];  // second operand, hi
  uint4* const Bl = Bh + D * 16;        // second operand, lo
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
  auto split8 = [](const float* x, uint4* hi, uint4* lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
      l[q] = pack_bf16x2(x[2 * q] - bf16_to_f32(h[q] & 0xFFFFu), x[2 * q + 1] - bf16_to_f32(h[q] >> 16));
    }
    *hi = make_uint4(h[0], h[1], h[2], h[3]);
    *lo = make_uint4(l[0], l[1], l[2], l[3]);
  };
  // this lane's first operands (S_prev, or zero), split in registers
  uint4 sh[D / 16], sl[D / 16];
  auto load_a_operands = [&](const float* X) {
    const float* col = X ? X + 32 * wave + l32 : nullptr;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = col ? col[(int64_t)(16 * ks + 8 * hk + e) * D] : 0.f;
      split8(x, &sh[ks], &sl[ks]);
    }
  };
  // X (row-major D x D fp32) into LDS as the transposed hi/lo pair: thread t
  // takes column t % 128 and the chunks 8 (t / 128) .. + 7 (rows 64 (t / 128) ..)
  auto stage_b = [&](const float* X) {
    const int bc = tid & 127, c0 = 8 * (tid >> 7);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int c = c0 + cc;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = X[(int64_t)(8 * c + e) * D + bc];
      split8(x, &Bh[bc * 16 + (c ^ (bc & 15))], &Bl[bc * 16 + (c ^ (bc & 15))]);
    }
  };
  load_a_operands(Sp);
  stage_b(Gt);
  __syncthreads();
  f32x16_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[nb][j] = 0.f;
  auto product = [&]() {  // acc += X^T B, X^T's operands in sh / sl, B in LDS
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c = 2 * ks + hk;
      const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, sh[ks]);
      const bf16x8_t al = __builtin_bit_cast(bf16x8_t, sl[ks]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int bcol = 32 * nb + l32;
        const bf16x8_t bhv = __builtin_bit_cast(bf16x8_t, Bh[bcol * 16 + (c ^ (bcol & 15))]);
        const bf16x8_t blv = __builtin_bit_cast(bf16x8_t, Bl[bcol * 16 + (c ^ (bcol & 15))]);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bhv, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bhv, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, blv, acc[nb], 0, 0, 0);
      }
    }
  };
  product();
  // chunk-causal scan: + R_{t+1}^T F_t, and G_t + F_t written over G_t
  if (rg.rev != nullptr) {
    bool more;
    const float* Ft = rev_adjoint(rg, f, bh, t, T, DD, &more);
    const float* Rn = rg.rev + (f + 1) * DD;
    __syncthreads();  // every wave is done with G_t's operands, and every thread has read G_t
    constexpr int kPer = D * D / 4 / 256;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int64_t e = 4 * (int64_t)(tid + 256 * u);
      const float4 g4 = *(const float4*)(Gt + e);
      const float4 f4 = *(const float4*)(Ft + e);
      *(float4*)(Gt + e) = make_float4(g4.x + f4.x, g4.y + f4.y, g4.z + f4.z, g4.w + f4.w);
    }
    if (more) {
      load_a_operands(Rn);
      stage_b(Ft);
      __syncthreads();
      product();
    }
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
  __syncthreads();  // every wave is done reading Ws
  const float g = gamma[f];
  if (tid == 0 && dgamma != nullptr) dgamma[f] = red[0] + red[1] + red[2] + red[3];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      Ws[32 * wave + 8 * (j >> 2) + 4 * hk + (j & 3)][32 * nb + l32] = acc[nb][j];
  __syncthreads();
  float* Pf = P + f * DD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int a = 32 * wave + 8 * (j >> 2) + 4 * hk + (j & 3), b = 32 * nb + l32;
      Pf[(int64_t)a * D + b] = -g * (acc[nb][j] + Ws[b][a]);
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
  if (granule && sh.D != 128) return hipErrorInvalidValue;  // the granule layout is D = 128's
  grad_init_kernel<<<grid_cap(granule ? n / 4 : n), 256, 0, st>>>(E, ds_final, ginit, sh.T, sh.D,
                                                                  sh.BH(), granule ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_chunk_init(const Shape& sh, const float* E, int L, int nchunk, float* finit,
                             bool granule, hipStream_t st) {
  const int64_t n = sh.BH() * nchunk * sh.D * sh.D;
  if (n == 0) return hipSuccess;
  if (L < 1 || (int64_t)(nchunk - 1) * L >= sh.T) return hipErrorInvalidValue;
  if (granule && sh.D != 128) return hipErrorInvalidValue;  // the granule layout is D = 128's
  chunk_init_kernel<<<grid_cap(granule ? n / 4 : n), 256, 0, st>>>(E, finit, sh.T, sh.D, L, nchunk,
                                                                   sh.BH(), granule ? 1 : 0);
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
  if (!grid_fits(sh.FH(), 256)) return hipErrorInvalidValue;
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


// Workgroups per frame-head of the token-gradient kernel. More than one
// narrows the window of active addresses but reloads the P and G fragments
// per workgroup. On MI355X, 60 s 720p layer: 1524-1551 / 1535-1537 /
// 1502-1505 / 1516 us with 1 / 2 / 3 / 4 (an earlier version of the kernel,
// at 1.73 ms, had run fastest with 1).
#ifndef GDN_TG_NB
#define GDN_TG_NB 3
#endif

bool token_grad_uses_mfma(const Shape& sh) { return sh.io == 1 && sh.D == 128; }

hipError_t launch_token_grad(const Shape& sh, const void* q, const void* k, const void* v,
                             const float* beta,
                             const void* dout, const float* states, const float* states2,
                             const float* gbuf, const float* ginit, const float* P, void* dq,
                             void* dk, void* dv, float* dbeta, hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  if (token_grad_uses_mfma(sh)) {
    // on this path dq comes from the fused E_t pass over q and d_o
    if (dq) return hipErrorInvalidValue;
    if (!dk && !dv && !dbeta) return hipSuccess;
    // GDN_TG_NB workgroups per frame-head on one XCD; two fit a CU
    const int nb = GDN_TG_NB;
    const int64_t groups = (sh.FH() + 7) / 8;
    if (!grid_fits(groups * 8 * nb, 256)) return hipErrorInvalidValue;
    dim3 grid((unsigned)(groups * 8 * nb));
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
#define GDN_TOKEN_WS(PR, NM)                                                                    \
  token_grad_ws_bf16_d128<PR, NM><<<grid, 256, 0, st>>>(kk, vv, beta, gbuf, ginit, P, (uint16_t*)dk, \
                                                        (uint16_t*)dv, dbeta, sh.S, sh.T, sh.FH(), nb,  \
                                                        sh.c)
    if (sh.prepared) GDN_TOKEN_WS(true, false);  // prepared keys are used as given
    else if (sh.qk_norm) GDN_TOKEN_WS(false, true);
    else GDN_TOKEN_WS(false, false);
#undef GDN_TOKEN_WS
    return hipGetLastError();
  }
  const int tpw = 256 / sh.D;
  const int ntile = (sh.S + tpw - 1) / tpw;
  if (!grid_fits(sh.FH() * ntile, 256)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(sh.FH() * ntile));
#define GDN_TG(TT, DV)                                                                        \
  token_grad_generic<TT, DV><<<grid, 256, 0, st>>>(                                          \
      (const TT*)q, (const TT*)k, (const TT*)v, beta, (const TT*)dout, states, states2, gbuf,    \
      ginit, P, (TT*)dq, (TT*)dk, (TT*)dv, dbeta, sh.S, sh.T, ntile, sh.c, sh.prepared, sh.qk_norm)
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
