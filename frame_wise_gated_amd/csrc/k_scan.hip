// Phase 2: the short sequential D x D affine scan over frames, in fp32.
//
//   forward  S_t = S_{t-1} M_t + U_t = gamma_t (S_{t-1} - S_{t-1} A_t) + U_t
//            (blog.hotdry.top SANA-WM post, section "混合线性注意力");
//   compose  per time chunk p: the same recurrence run on the 2D x D state
//            [C; H] from [I; 0], with U added to the H rows only, giving
//            S_end = S_start C_p + H_p (same post, section
//            "显存分片: Context-Parallel 的工程实现");
//   reverse  R_t = R_{t+1} M_t + U_t inside each chunk, from zero after the
//            chunk's last frame (hyper.ai page 2605.15178, method section:
//            the reverse temporal scan restarts at chunk boundaries);
//   combine  s_start[p+1] = s_start[p] C_p + H_p, chunk after chunk.
//
// Rows of the state are independent given M_t (row i of S_{t-1} M_t only needs
// row i of S_{t-1}), so a workgroup owns a 16-row block of one head's state and
// steps it through the frames of one chunk; the grid covers heads x chunks x
// row blocks. A_t and U_t do not depend on the state, so they stream from HBM/L2
// while the row block stays in LDS.
#include "gdn_common.h"

namespace gdn {

namespace {

constexpr int kR = 16;  // state rows per workgroup

template <int D>
__global__ void __launch_bounds__(256) scan_rows_kernel(ScanParams p) {
  constexpr int RG = 256 / D;       // row groups (threads sharing a column)
  constexpr int RPT = kR / RG;      // rows per thread
  __shared__ float Xs[2][kR][D];

  const int rows_total = (p.mode == SCAN_COMPOSE) ? 2 * D : D;
  const int nrb = rows_total / kR;
  const int rb = blockIdx.x % nrb;
  const int c = (blockIdx.x / nrb) % p.nchunk;
  const int64_t bh = blockIdx.x / (nrb * p.nchunk);
  const int row0 = rb * kR;                    // first row of this block in [0, rows_total)
  const bool c_rows = (p.mode == SCAN_COMPOSE) && row0 < D;  // composite transition rows
  const bool use_u = !c_rows;
  const int srow0 = row0 % D;                  // first row inside its D x D matrix

  const int tid = threadIdx.x;
  const int n = tid % D;
  const int ig = tid / D;

  // initial rows
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = ig + RG * r;
    float x0 = 0.f;
    if (p.mode == SCAN_COMPOSE) {
      x0 = (c_rows && (srow0 + i) == n) ? 1.f : 0.f;
    } else if (p.mode == SCAN_FORWARD && p.init != nullptr) {
      x0 = p.init[bh * p.init_bh_stride + (int64_t)c * p.init_c_stride + (int64_t)(srow0 + i) * D + n];
    }
    Xs[0][i][n] = x0;
  }
  __syncthreads();

  const int a = p.offsets[c];
  const int e = p.offsets[c + 1];
  const int nsteps = e - a;
  const int64_t DD = (int64_t)D * D;
  int cur = 0;
  for (int step = 0; step < nsteps; ++step) {
    const int t = (p.mode == SCAN_REVERSE) ? (e - 1 - step) : (a + step);
    const int64_t f = bh * p.T + t;
    const float* At = p.terms + f * 2 * DD;
    const float* Ut = At + DD;
    const float g = p.gamma[f];
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = 0.f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) {
      const float av = At[(int64_t)j * D + n];
#pragma unroll
      for (int r = 0; r < RPT; ++r) acc[r] = fmaf(Xs[cur][ig + RG * r][j], av, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = ig + RG * r;
      float xn = g * (Xs[cur][i][n] - acc[r]);
      if (use_u) xn += Ut[(int64_t)(srow0 + i) * D + n];
      Xs[cur ^ 1][i][n] = xn;
      if (p.states != nullptr) p.states[f * DD + (int64_t)(srow0 + i) * D + n] = xn;
    }
    cur ^= 1;
    __syncthreads();
  }

  if (p.fin_last_only && c != p.nchunk - 1) return;
  float* fin = (p.mode == SCAN_COMPOSE && !c_rows) ? p.finB : p.finA;
  if (fin == nullptr) return;
  fin += bh * p.fin_bh_stride + (p.fin_last_only ? 0 : (int64_t)c * p.fin_c_stride);
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = ig + RG * r;
    fin[(int64_t)(srow0 + i) * D + n] = Xs[cur][i][n];
  }
}

template <int D>
__global__ void __launch_bounds__(256) combine_rows_kernel(CombineParams p) {
  constexpr int RG = 256 / D;
  constexpr int RPT = kR / RG;
  __shared__ float Xs[2][kR][D];
  constexpr int nrb = D / kR;
  const int rb = blockIdx.x % nrb;
  const int64_t bh = blockIdx.x / nrb;
  const int row0 = rb * kR;
  const int tid = threadIdx.x;
  const int n = tid % D;
  const int ig = tid / D;
  const int64_t DD = (int64_t)D * D;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = ig + RG * r;
    Xs[0][i][n] = p.s0 ? p.s0[bh * DD + (int64_t)(row0 + i) * D + n] : 0.f;
  }
  __syncthreads();
  int cur = 0;
  for (int q = 0; q < p.P; ++q) {
    const float* Cq = p.C + (bh * p.P + q) * DD;
    const float* Hq = p.Hc + (bh * p.P + q) * DD;
    float* out = p.s_start + (bh * p.P + q) * DD;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = ig + RG * r;
      out[(int64_t)(row0 + i) * D + n] = Xs[cur][i][n];
    }
    if (q == p.P - 1) break;
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = 0.f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) {
      const float cv = Cq[(int64_t)j * D + n];
#pragma unroll
      for (int r = 0; r < RPT; ++r) acc[r] = fmaf(Xs[cur][ig + RG * r][j], cv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = ig + RG * r;
      Xs[cur ^ 1][i][n] = acc[r] + Hq[(int64_t)(row0 + i) * D + n];
    }
    cur ^= 1;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_scan(const Shape& sh, const ScanParams& p, hipStream_t st) {
  const int64_t rows_total = (p.mode == SCAN_COMPOSE) ? 2 * sh.D : sh.D;
  const int64_t blocks = sh.BH() * p.nchunk * (rows_total / kR);
  if (blocks == 0) return hipSuccess;
  dim3 grid((unsigned)blocks);
  switch (sh.D) {
    case 16: scan_rows_kernel<16><<<grid, 256, 0, st>>>(p); break;
    case 32: scan_rows_kernel<32><<<grid, 256, 0, st>>>(p); break;
    case 64: scan_rows_kernel<64><<<grid, 256, 0, st>>>(p); break;
    case 128: scan_rows_kernel<128><<<grid, 256, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& sh, const CombineParams& p, hipStream_t st) {
  const int64_t blocks = sh.BH() * (sh.D / kR);
  if (blocks == 0 || p.P == 0) return hipSuccess;
  dim3 grid((unsigned)blocks);
  switch (sh.D) {
    case 16: combine_rows_kernel<16><<<grid, 256, 0, st>>>(p); break;
    case 32: combine_rows_kernel<32><<<grid, 256, 0, st>>>(p); break;
    case 64: combine_rows_kernel<64><<<grid, 256, 0, st>>>(p); break;
    case 128: combine_rows_kernel<128><<<grid, 256, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
