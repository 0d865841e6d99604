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

// Per frame-head: dM = S_prev^T G (fp32), dgamma = tr(dM) - <dM, A>,
// P = -gamma (dM + dM^T). 256 threads as a 16 x 16 grid, each owning a
// B x B block of dM (B = D / 16); S_prev and G staged in LDS.
template <int D>
__global__ void __launch_bounds__(256) frame_grad_kernel(
    const float* __restrict__ states, const float* __restrict__ s0, const float* __restrict__ gbuf,
    const float* __restrict__ ginit, const float* __restrict__ terms, int a_granule_bf16,
    const float* __restrict__ gamma, float* __restrict__ P, float* __restrict__ dgamma, int T) {
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
  const float* Gt = t == T - 1 ? ginit + bh * DD : gbuf + (f + 1) * DD;
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
    const TIn* __restrict__ dout, const float* __restrict__ states, const float* __restrict__ gbuf,
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
  const float* Gt = t == T - 1 ? ginit + bh * DD : gbuf + (f + 1) * DD;
  const float* Pt = P + f * DD;
  float dqv = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
  for (int j = 0; j < D; ++j) {
    dqv = fmaf(St[(int64_t)j * D + i], ds[tl][j], dqv);
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

hipError_t launch_frame_grad(const Shape& sh, const float* states, const float* s0,
                             const float* gbuf, const float* ginit, const float* terms,
                             bool a_granule_bf16, const float* gamma, float* P, float* dgamma,
                             hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  dim3 grid((unsigned)sh.FH());
  const int ag = a_granule_bf16 ? 1 : 0;
#define GDN_FG(DV)                                                                              \
  frame_grad_kernel<DV><<<grid, 256, 0, st>>>(states, s0, gbuf, ginit, terms, ag, gamma, P, \
                                              dgamma, sh.T)
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

hipError_t launch_token_grad(const Shape& sh, const void* k, const void* v, const float* beta,
                             const void* dout, const float* states, const float* gbuf,
                             const float* ginit, const float* P, void* dq, void* dk, void* dv,
                             float* dbeta, hipStream_t st) {
  if (sh.FH() == 0) return hipSuccess;
  const int tpw = 256 / sh.D;
  const int ntile = (sh.S + tpw - 1) / tpw;
  dim3 grid((unsigned)(sh.FH() * ntile));
#define GDN_TG(TT, DV)                                                                        \
  token_grad_generic<TT, DV><<<grid, 256, 0, st>>>(                                          \
      (const TT*)k, (const TT*)v, beta, (const TT*)dout, states, gbuf, ginit, P, (TT*)dq, \
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
