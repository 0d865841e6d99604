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

// Build-time tuning knobs of the MFMA scan: the row block in 16-row MFMA
// tiles of launches that fill the chip, that of launches which would have
// fewer workgroups than CUs at that size (the sequential scans of a few
// heads), and the frames of A_t / U_t prefetched in registers. Measured on
// MI355X for the 60 s 720p layer: the sequential 121-frame scan of 16 heads
// took 159 us with 16-row blocks against 223-236 us with 32-row blocks, while
// the compose and the replay of 8 chunks took 101 and 83 us with 16-row
// blocks against 81 and 67 us with 32-row blocks.
#ifndef GDN_SCAN_MT
#define GDN_SCAN_MT 2
#endif
#ifndef GDN_SCAN_MT_SMALL
#define GDN_SCAN_MT_SMALL 1
#endif
#ifndef GDN_SCAN_F
#define GDN_SCAN_F 2
#endif
// A compose launch of its own (not sharing a launch with a reverse scan) that
// fills the chip takes 64-row blocks with a one-frame ring (168 registers,
// two workgroups per CU): each workgroup reads A_t once for twice the rows.
// 60 s 720p layer, 8 chunks: 64-66 us against 73-75 us with 32-row blocks
// and a two-frame ring; the replay stays faster with 32-row blocks (63 us
// against 64-65 us).
#ifndef GDN_COMPOSE_MT
#define GDN_COMPOSE_MT 4
#endif
#ifndef GDN_COMPOSE_F
#define GDN_COMPOSE_F 1
#endif
// bf16 D = 128: the combine on MFMA (1) or on fp32 vector FMAs (0)
#ifndef GDN_COMBINE_MFMA
#define GDN_COMBINE_MFMA 1
#endif

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
  int64_t job;
  int rb;
  xcd_job(blockIdx.x, nrb, &job, &rb);
  if (job >= p.njobs) return;
  const int c = (int)(job % p.nchunk);
  const int64_t bh = job / p.nchunk;
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
    } else if (p.init != nullptr) {
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
    bool u_on = use_u;
    if (p.usrc != nullptr) {
      const int fs = t + p.ushift;
      u_on = use_u && fs >= 0 && fs < p.T;
      Ut = p.usrc + (bh * p.T + (u_on ? fs : 0)) * DD;
    }
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
      // one rounding of g (X - XA) + U (an explicit fma, so that the result
      // does not depend on how the compiler contracts the expression)
      const float dx = Xs[cur][i][n] - acc[r];
      const float xn = u_on ? fmaf(g, dx, Ut[(int64_t)(srow0 + i) * D + n]) : g * dx;
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
constexpr int combine_rows() { return (256 / D) > 4 ? (256 / D) : 4; }

// combine: s_start[q+1] = s_start[q] C_q + H_q, for one head's CR-row block.
// Thread (n, ig) forms column n of its rows. Column n of C_q is read from
// global memory (L2) in blocks of kCJ entries whose loads are all issued before
// the first use, so a step waits for D / kCJ round trips rather than one per
// few entries; the state rows come from LDS.
#ifndef GDN_COMBINE_J
#define GDN_COMBINE_J 64
#endif
template <int D>
__global__ void __launch_bounds__(256) combine_rows_kernel(CombineParams p) {
  constexpr int CR = combine_rows<D>();  // state rows per workgroup
  constexpr int RG = 256 / D;
  constexpr int RPT = CR / RG;
  constexpr int kCJ = D < GDN_COMBINE_J ? D : GDN_COMBINE_J;
  __shared__ float Xs[2][CR][D];
  constexpr int nrb = D / CR;
  int64_t bh;
  int rb;
  xcd_job(blockIdx.x, nrb, &bh, &rb);
  if (bh >= p.BH) return;
  const int row0 = rb * CR;
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
    for (int r = 0; r < RPT; ++r) acc[r] = Hq[(int64_t)(row0 + ig + RG * r) * D + n];
    for (int j0 = 0; j0 < D; j0 += kCJ) {
      float cv[kCJ];
#pragma unroll
      for (int jj = 0; jj < kCJ; ++jj) cv[jj] = Cq[(int64_t)(j0 + jj) * D + n];
#pragma unroll
      for (int jj = 0; jj < kCJ; ++jj)
#pragma unroll
        for (int r = 0; r < RPT; ++r) acc[r] = fmaf(Xs[cur][ig + RG * r][j0 + jj], cv[jj], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) Xs[cur ^ 1][ig + RG * r][n] = acc[r];
    cur ^= 1;
    __syncthreads();
  }
}

// MFMA combine for bf16 workloads (D = 128): the same recurrence
// s_start[q+1] = s_start[q] C_q + H_q with the products on bf16 MFMA as three
// terms of hi/lo splits (Xh Ch + Xl Ch + Xh Cl; |X - Xh - Xl| <= 2^-17 |X|,
// likewise C), fp32 accumulation: about 16 significant bits per product, as
// in the scan's own steps. A workgroup owns a 32-row block of one head's
// start states (four per head) and wave w forms columns 32 w .. 32 w + 31.
// C_q sits in LDS transposed (row n holds column n of C_q, 16-byte chunk c at
// position c ^ (n % 16)) so that the second operand is a row read; C_{q+1}
// and this lane's entries of H_{q+1} are loaded into registers while step q
// computes, so a step costs LDS staging, 24 MFMAs per wave and two barriers.
__global__ void __launch_bounds__(256, 1) combine_mfma_d128(CombineParams p) {
  constexpr int D = 128;
  constexpr int64_t DD = (int64_t)D * D;
  constexpr int R = 32;
  __shared__ uint4 Cth[D * 16], Ctl[D * 16];
  __shared__ uint4 Xh[R * 16], Xl[R * 16];
  int64_t bh;
  int rb;
  xcd_job(blockIdx.x, D / R, &bh, &rb);
  if (bh >= p.BH) return;
  const int row0 = rb * R;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int n = 32 * wave + l32;  // this lane's output column
  auto at = [](int r, int c) { return r * 16 + (c ^ (r & 15)); };
  auto hi_lo = [](float a, float b, uint32_t* hi, uint32_t* lo) {
    *hi = pack_bf16x2(a, b);
    *lo = pack_bf16x2(a - bf16_to_f32(*hi & 0xFFFFu), b - bf16_to_f32(*hi >> 16));
  };
  // X_0 = s0 (or 0): thread t holds row t / 8, columns 16 (t % 8) .. + 15
  {
    const int i = tid >> 3, c0 = 2 * (tid & 7);
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      x[e] = p.s0 ? p.s0[bh * DD + (int64_t)(row0 + i) * D + 8 * c0 + e] : 0.f;
    float* out0 = p.s_start + (bh * p.P) * DD + (int64_t)(row0 + i) * D + 8 * c0;
#pragma unroll
    for (int e = 0; e < 16; e += 4) *(float4*)(out0 + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hi_lo(x[8 * cc + 2 * q], x[8 * cc + 2 * q + 1], &hw[q], &lw[q]);
      Xh[at(i, c0 + cc)] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      Xl[at(i, c0 + cc)] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
  if (p.P < 2) return;
  // C_q in registers: thread t holds column t % 128, rows 64 (t / 128) .. + 63;
  // H_q: this lane's output entries (rows 8 jg + 4 h + r, column n)
  const int cn = tid & 127, cj0 = 64 * (tid >> 7);
  float cv[64], hq[16], hn[16];
  auto fetch = [&](int q, float* hdst) {
    const float* Cq = p.C + (bh * p.P + q) * DD;
#pragma unroll
    for (int e = 0; e < 64; ++e) cv[e] = Cq[(int64_t)(cj0 + e) * D + cn];
    const float* Hq = p.Hc + (bh * p.P + q) * DD;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      hdst[j] = Hq[(int64_t)(row0 + 8 * (j >> 2) + 4 * h + (j & 3)) * D + n];
  };
  fetch(0, hq);
  for (int q = 0; q + 1 < p.P; ++q) {
    // C_q^T (hi, lo) into LDS from the registers
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hi_lo(cv[8 * c + 2 * e], cv[8 * c + 2 * e + 1], &hw[e], &lw[e]);
      Cth[at(cn, cj0 / 8 + c)] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      Ctl[at(cn, cj0 / 8 + c)] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    if (q + 2 < p.P) fetch(q + 1, hn);
    __syncthreads();  // C_q^T and X_q are in LDS
    f32x16_t acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int c = 2 * kk + h;
      const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, Xh[at(l32, c)]);
      const bf16x8_t al = __builtin_bit_cast(bf16x8_t, Xl[at(l32, c)]);
      const bf16x8_t bh8 = __builtin_bit_cast(bf16x8_t, Cth[at(n, c)]);
      const bf16x8_t bl8 = __builtin_bit_cast(bf16x8_t, Ctl[at(n, c)]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh8, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh8, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl8, acc, 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading C_q^T and X_q
    // X_{q+1} = acc + H_q: to s_start[q+1] and, split, to LDS
    float* outq = p.s_start + (bh * p.P + q + 1) * DD;
    uint16_t* xh16 = (uint16_t*)Xh;
    uint16_t* xl16 = (uint16_t*)Xl;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = 8 * (j >> 2) + 4 * h + (j & 3);
      const float x = acc[j] + hq[j];
      outq[(int64_t)(row0 + i) * D + n] = x;
      const uint32_t hw = pack_bf16x2(x, 0.f) & 0xFFFFu;
      const uint32_t lw = pack_bf16x2(x - bf16_to_f32(hw), 0.f) & 0xFFFFu;
      const int e = at(i, n >> 3) * 8 + (n & 7);
      xh16[e] = (uint16_t)hw;
      xl16[e] = (uint16_t)lw;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) hq[j] = hn[j];
  }
}

// MFMA scan step for bf16 workloads with D = 128: the product X A_t of the
// fp32 row block X (R = 16*MT rows) with A_t runs on bf16 MFMA, the state
// split into a hi/lo bf16 pair and A_t rounded to bf16 once by phase 1:
//   X A ~= Xh A' + Xl A',     |X - Xh - Xl| <= 2^-17 |X|,  A' = bf16(A).
// The state therefore keeps about 16 significant bits through every step
// (rounding the state itself to bf16 each frame would compound over the
// frames), at twice the bf16 MFMA cost. A' perturbs the transition by at most
// 2^-9 |A| elementwise, and since the transition is contractive
// (tr A <= 1), that error stays at the 1e-4 level over a 121-frame scan
// (measured with the float64 oracle: 6.5e-5 relative on the states of the
// 60 s 720p layer). Accumulation, the decay and the U_t update are fp32, and
// U_t stays fp32.
//
// The MFMA computes (X A)^T tiles: bf16(A_t)^T (from phase 1, in the granule
// layout described with a_granule) is the first operand, one 16-byte
// load per fragment and 1 KB per wave, and the state rows are the second. A lane then owns
// four consecutive columns n of one state row m, so its U_t entries, its
// per-frame state store and its share of the split bf16 copy in LDS are
// single 16- or 8-byte accesses. Each lane keeps its fp32 state entries in
// registers for the whole scan; LDS holds the split copy that the MFMA reads
// (double-buffered, one barrier per frame) and, for row blocks of up to 32
// rows, a copy of the new fp32 rows that the per-frame state store reads back
// after the barrier: a lane's own entries cover only 64 bytes of each
// 128-byte line, and stores of whole 512-byte rows (two per wave
// instruction) took the sequential 121-frame scan of 16 heads from 152 to
// 132 us and the replay of 8 chunks from 66 to 61 us.
//
// The per-frame step is short (64 MFMAs per wave for MT = 4) next to the
// latency of a global load, so the A_t fragments and U_t entries of the next
// kF frames live in a register ring: the loads of frame s + kF are issued as
// soon as frame s has consumed the slot. Slot indices are compile-time (the
// frame loop is unrolled by kF); loads past the last frame re-read it, so
// the outstanding-load bookkeeping is identical in every step. Wave w owns
// output columns [32w, 32w + 32) as two 16-column MFMA tiles.
// Rows of one workgroup's job: row block rb of job `job`. kC: the composite C
// rows of a COMPOSE job (start I, no U term), which load no U entries. kMix
// (COMPOSE, MT even): tiles [0, MT/2) hold C rows and tiles [MT/2, MT) the H
// rows of the same indices, so that every workgroup of a job reads A_t and
// the same amount of U_t per frame: the workgroups of a job then step
// together and share each A_t through L2. With whole C and whole H row
// blocks the C blocks ran ahead and the H blocks, which set the compose's
// time, fetched A_t again from HBM (the compose read 1.2 times its bytes).
constexpr int kScanLdb = 128 + 8;  // bf16 row stride 272 B: 8 lanes reading 16 B at one column are conflict-free
constexpr int kSstLd = 128 + 4;   // fp32 row stride 528 B: the 16 rows of a lane group start 4 banks apart
template <int MT, int kF, bool kC, bool kMix = false>
__device__ __forceinline__ void scan_rows(const ScanParams& p, int64_t job, int rb,
                                          uint16_t (*Xh)[16 * MT][kScanLdb],
                                          uint16_t (*Xl)[16 * MT][kScanLdb],
                                          float (*Sst)[MT <= 2 ? 16 * MT : 1][kSstLd]) {
  constexpr int D = 128;
  constexpr int R = 16 * MT;
  constexpr int64_t DD = (int64_t)D * D;
  const int c = (int)(job % p.nchunk);
  const int64_t bh = job / p.nchunk;
  const int row0 = rb * R;
  static_assert(!kMix || (!kC && MT % 2 == 0), "mixed C/H row blocks");
  constexpr bool c_rows = kC;
  const float umul = c_rows ? 0.f : 1.f;
  const int srow0 = kMix ? rb * (R / 2) : row0 % D;
  // tile mt: C rows or not, and its first row inside its D x D matrix
  auto is_c = [&](int mt) { return kC || (kMix && mt < MT / 2); };
  auto trow = [&](int mt) { return srow0 + 16 * (kMix ? mt % (MT / 2) : mt); };

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int n0 = 32 * wave;
  // this lane's state entries: rows m = 16 mt + l16, columns ncol(nt) .. + 3
  auto ncol = [&](int nt) { return n0 + 16 * nt + 4 * g; };

  f32x4_t xr[MT][2];
  auto put_split = [&](int buf, int m, int n, const f32x4_t& x) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      h[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
      l[q] = pack_bf16x2(x[2 * q] - bf16_to_f32(h[q] & 0xFFFFu), x[2 * q + 1] - bf16_to_f32(h[q] >> 16));
    }
    *(uint2*)&Xh[buf][m][n] = make_uint2(h[0], h[1]);
    *(uint2*)&Xl[buf][m][n] = make_uint2(l[0], l[1]);
  };
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int m = 16 * mt + l16;
      const int n = ncol(nt);
      f32x4_t x0 = {0.f, 0.f, 0.f, 0.f};
      if (p.mode == SCAN_COMPOSE) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x0[r] = (is_c(mt) && trow(mt) + l16 == n + r) ? 1.f : 0.f;
      } else if (p.init != nullptr) {
        x0 = *(const f32x4_t*)(p.init + bh * p.init_bh_stride + (int64_t)c * p.init_c_stride +
                              (int64_t)(trow(mt) + l16) * D + n);
      }
      xr[mt][nt] = x0;
      put_split(0, m, n, x0);
    }
  __syncthreads();

  const int a = p.offsets[c];
  const int e = p.offsets[c + 1];
  const int nsteps = e - a;
  auto frame_of = [&](int step) {
    step = step < nsteps ? step : nsteps - 1;
    return (p.mode == SCAN_REVERSE) ? (e - 1 - step) : (a + step);
  };
  auto terms_of = [&](int step) { return p.terms + (bh * p.T + frame_of(step)) * 2 * DD; };

  // register ring: A_t^T fragments, U_t entries and gamma_t of kF
  // frames. gamma rides with U_t: waiting for a load issued later than the
  // prefetches would wait for all of them (vmcnt counts in order).
  uint4 af[kF][2][4];
  f32x4_t u[kF][MT][2];
  float gmr[kF];
  float umr[kF];  // 1 when the frame's U term applies, 0 otherwise
  // granule layout of the terms (a_granule / u_granule): each load below is
  // 1 KB of consecutive bytes per wave
  auto load_a = [&](int j, int step) {
    const uint4* At = (const uint4*)terms_of(step);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)  // a_granule(n0 + 16nt + l16, 4ks + g)
        af[j][nt][ks] = At[((2 * wave + nt) * 4 + ks) * 64 + lane];
  };
  // Composite C rows have no U term: they load only gamma (their load
  // sequence differs from the other rows', so they are a separate
  // instantiation with exact waits of its own).
  auto load_u = [&](int j, int step) {
    umr[j] = umul;
    if (kC) {
      gmr[j] = p.gamma[bh * p.T + frame_of(step)];
      return;
    }
    const f32x4_t* Ug = (const f32x4_t*)(terms_of(step) + DD);
    if (p.usrc != nullptr && !c_rows) {
      // U of frame f from the shifted source slot (zero outside [0, T))
      const int fs = frame_of(step) + p.ushift;
      const bool on = fs >= 0 && fs < p.T;
      umr[j] = on ? 1.f : 0.f;
      Ug = (const f32x4_t*)(p.usrc + (bh * p.T + (on ? fs : 0)) * DD);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)  // u_granule(trow(mt) + l16, ncol(nt) / 4)
        if (!is_c(mt)) u[j][mt][nt] = Ug[((trow(mt) / 16) * 8 + 2 * wave + nt) * 64 + lane];
    gmr[j] = p.gamma[bh * p.T + frame_of(step)];
  };
  if (nsteps > 0) {
#pragma unroll
    for (int j = 0; j < kF; ++j) {
      load_a(j, j);
      load_u(j, j);
    }
  }

  int cur = 0;
  for (int s0 = 0; s0 < nsteps; s0 += kF) {
#pragma unroll
    for (int j = 0; j < kF; ++j) {
      const int step = s0 + j;
      const bool active = step < nsteps;
      const int64_t f = bh * p.T + frame_of(step);
      const float gm = gmr[j];
      f32x4_t acc[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // per k-slice: the state fragments of every row tile first, then the
      // two products in an order that puts 2*MT independent MFMAs between two
      // that accumulate into the same tile
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t xh[MT], xl[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + l16;
          xh[mt] = __builtin_bit_cast(bf16x8_t, *(const uint4*)&Xh[cur][m][32 * ks + 8 * g]);
          xl[mt] = __builtin_bit_cast(bf16x8_t, *(const uint4*)&Xl[cur][m][32 * ks + 8 * g]);
        }
#pragma unroll
        for (int prod = 0; prod < 2; ++prod)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
              const bf16x8_t a_ = __builtin_bit_cast(bf16x8_t, af[j][nt][ks]);
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_, prod == 0 ? xh[mt] : xl[mt],
                                                                    acc[mt][nt], 0, 0, 0);
            }
      }
      load_a(j, step + kF);  // the slot's fragments are consumed: refill with frame step + kF

      // acc[mt][nt][r] = (X A_t)[m][ncol(nt) + r] with m = 16 mt + l16
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int m = 16 * mt + l16;
          f32x4_t xn;
#pragma unroll
          for (int r = 0; r < 4; ++r)  // one rounding: umr is 0 or 1, so umr u is exact
            xn[r] = __builtin_fmaf(gm, xr[mt][nt][r] - acc[mt][nt][r], is_c(mt) ? 0.f : umr[j] * u[j][mt][nt][r]);
          if (active) xr[mt][nt] = xn;
          put_split(cur ^ 1, m, ncol(nt), xr[mt][nt]);
        }
      // per-frame state: staged rows (stored whole after the barrier), or
      // each lane's own entries for the 64-row blocks
      constexpr bool kStage = MT <= 2;
      const int sb = step & 1;
      if (kStage) {
        if (p.states != nullptr) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
              *(f32x4_t*)&Sst[sb][16 * mt + l16][ncol(nt)] = xr[mt][nt];
        }
      } else if (active && p.states != nullptr) {
        float* st = p.states + f * DD + (int64_t)srow0 * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            *(f32x4_t*)(st + (16 * mt + l16) * D + ncol(nt)) = xr[mt][nt];
      }
      load_u(j, step + kF);
      cur ^= 1;
      lds_barrier();  // a plain __syncthreads() would also wait for the prefetched frames
      // wave w stores rows 4 MT w .. 4 MT w + 4 MT - 1, two whole rows per
      // instruction. Sst[sb] is written again two frames later, after the
      // next barrier, which this wave reaches only once these reads are done.
      if (kStage && active && p.states != nullptr) {
        float* st = p.states + f * DD + (int64_t)srow0 * D;
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i) {
          const int row = wave * (4 * MT) + 2 * i + (lane >> 5);
          const f32x4_t x = *(const f32x4_t*)&Sst[sb][row][4 * (lane & 31)];
          *(f32x4_t*)(st + row * D + 4 * (lane & 31)) = x;
        }
      }
    }
  }

  if (p.fin_last_only && c != p.nchunk - 1) return;
  const int64_t fin_off = bh * p.fin_bh_stride + (p.fin_last_only ? 0 : (int64_t)c * p.fin_c_stride);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float* fin = (p.mode == SCAN_COMPOSE && !is_c(mt)) ? p.finB : p.finA;
    if (fin == nullptr) continue;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      *(f32x4_t*)(fin + fin_off + (int64_t)(trow(mt) + l16) * D + ncol(nt)) = xr[mt][nt];
  }
}

// One workgroup's job; `blk` is its block index within the launch of p. The
// split state copy lives here, once per kernel, for both row kinds.
template <int MT, int kF>
__device__ __forceinline__ void scan_block(const ScanParams& p, int64_t blk) {
  constexpr int D = 128;
  constexpr int R = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t Xh[2][R][kScanLdb];
  __shared__ __attribute__((aligned(16))) uint16_t Xl[2][R][kScanLdb];
  __shared__ __attribute__((aligned(16))) float Sst[MT <= 2 ? 2 : 1][MT <= 2 ? R : 1][kSstLd];
  const int rows_total = (p.mode == SCAN_COMPOSE) ? 2 * D : D;
  int64_t job;
  int rb;
  xcd_job(blk, rows_total / R, &job, &rb);
  if (job >= p.njobs) return;
  if constexpr (MT % 2 == 0) {
    if (p.mode == SCAN_COMPOSE) {
      scan_rows<MT, kF, false, true>(p, job, rb, Xh, Xl, Sst);
      return;
    }
  }
  if (p.mode == SCAN_COMPOSE && rb * R < D)
    scan_rows<MT, kF, true>(p, job, rb, Xh, Xl, Sst);
  else
    scan_rows<MT, kF, false>(p, job, rb, Xh, Xl, Sst);
}

// Blocks [0, split) run the jobs of p0 and blocks [split, grid) those of p1:
// two independent scans over the same terms can share one launch (split is a
// multiple of the XCD count, so both keep their XCD mapping). Each branch
// reads its own kernel argument (a runtime choice between the two would copy
// them to scratch memory).
template <int MT, int kF>
__global__ void __launch_bounds__(256) scan_mfma_d128(ScanParams p0, ScanParams p1,
                                                      int64_t split) {
  if ((int64_t)blockIdx.x < split)
    scan_block<MT, kF>(p0, (int64_t)blockIdx.x);
  else
    scan_block<MT, kF>(p1, (int64_t)blockIdx.x - split);
}

}  // namespace

bool scan_uses_mfma(const Shape& sh) { return sh.io == 1 && sh.D == 128; }

namespace {

constexpr int kCUs = 256;

// Workgroups of one MFMA scan launch with MT-tile row blocks (0 without jobs).
int64_t mfma_blocks(const Shape& sh, const ScanParams& q, int MT) {
  const int rows = q.mode == SCAN_COMPOSE ? 2 * sh.D : sh.D;
  return q.njobs ? xcd_grid(q.njobs, rows / (16 * MT)) : 0;
}

// Row block of a launch: the small one when the large one leaves CUs idle.
int mfma_mt(const Shape& sh, const ScanParams& q) {
  return mfma_blocks(sh, q, GDN_SCAN_MT) < kCUs ? GDN_SCAN_MT_SMALL : GDN_SCAN_MT;
}

ScanParams with_jobs(const Shape& sh, const ScanParams& p) {
  ScanParams q = p;
  q.njobs = sh.BH() * p.nchunk;
  return q;
}

// One launch running the jobs of a and then those of b (b may be null).
template <int MT, int kF = GDN_SCAN_F>
hipError_t launch_mfma(const Shape& sh, const ScanParams& a, const ScanParams* b, hipStream_t st) {
  const int64_t na = mfma_blocks(sh, a, MT);
  const int64_t nb = b ? mfma_blocks(sh, *b, MT) : 0;
  if (na + nb == 0) return hipSuccess;
  if (!grid_fits(na + nb, 256)) return hipErrorInvalidValue;
  scan_mfma_d128<MT, kF><<<dim3((unsigned)(na + nb)), 256, 0, st>>>(
      a, b ? *b : a, b ? na : INT64_MAX);
  return hipGetLastError();
}

hipError_t launch_mfma(const Shape& sh, const ScanParams& a, const ScanParams* b, int mt,
                       hipStream_t st) {
  return mt == GDN_SCAN_MT ? launch_mfma<GDN_SCAN_MT>(sh, a, b, st)
                           : launch_mfma<GDN_SCAN_MT_SMALL>(sh, a, b, st);
}

}  // namespace

bool scan_pairs(const Shape& sh) { return scan_uses_mfma(sh); }

// Both job lists take the smaller of their two row blocks: a short scan that
// shares the launch of a long chain of few blocks (a sequential scan) fills
// the CUs that chain leaves idle.
hipError_t launch_scan_pair(const Shape& sh, const ScanParams& a, const ScanParams& b,
                            hipStream_t st) {
  if (!scan_pairs(sh)) return hipErrorInvalidValue;
  const ScanParams qa = with_jobs(sh, a), qb = with_jobs(sh, b);
  const int mta = mfma_mt(sh, qa), mtb = mfma_mt(sh, qb);
  return launch_mfma(sh, qa, &qb, mta < mtb ? mta : mtb, st);
}

hipError_t launch_scan(const Shape& sh, const ScanParams& p, hipStream_t st) {
  const int64_t rows_total = (p.mode == SCAN_COMPOSE) ? 2 * sh.D : sh.D;
  const ScanParams q = with_jobs(sh, p);
  if (q.njobs == 0) return hipSuccess;
  if (scan_uses_mfma(sh)) {
    if (q.mode == SCAN_COMPOSE && mfma_blocks(sh, q, GDN_COMPOSE_MT) >= kCUs)
      return launch_mfma<GDN_COMPOSE_MT, GDN_COMPOSE_F>(sh, q, nullptr, st);
    return launch_mfma(sh, q, nullptr, mfma_mt(sh, q), st);
  }
  if (!grid_fits(xcd_grid(q.njobs, (int)(rows_total / kR)), 256)) return hipErrorInvalidValue;
  dim3 grid((unsigned)xcd_grid(q.njobs, (int)(rows_total / kR)));
  switch (sh.D) {
    case 16: scan_rows_kernel<16><<<grid, 256, 0, st>>>(q); break;
    case 32: scan_rows_kernel<32><<<grid, 256, 0, st>>>(q); break;
    case 64: scan_rows_kernel<64><<<grid, 256, 0, st>>>(q); break;
    case 128: scan_rows_kernel<128><<<grid, 256, 0, st>>>(q); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& sh, const CombineParams& p, hipStream_t st) {
  int rows = 4;
  switch (sh.D) {
    case 16: rows = combine_rows<16>(); break;
    case 32: rows = combine_rows<32>(); break;
    case 64: rows = combine_rows<64>(); break;
    default: rows = combine_rows<128>(); break;
  }
  if (sh.BH() == 0 || p.P == 0) return hipSuccess;
  CombineParams q = p;
  q.BH = sh.BH();
  if (GDN_COMBINE_MFMA && scan_uses_mfma(sh)) {
    if (!grid_fits(xcd_grid(q.BH, 4), 256)) return hipErrorInvalidValue;
    combine_mfma_d128<<<dim3((unsigned)xcd_grid(q.BH, 4)), 256, 0, st>>>(q);
    return hipGetLastError();
  }
  if (!grid_fits(xcd_grid(q.BH, sh.D / rows), 256)) return hipErrorInvalidValue;
  dim3 grid((unsigned)xcd_grid(q.BH, sh.D / rows));
  switch (sh.D) {
    case 16: combine_rows_kernel<16><<<grid, 256, 0, st>>>(q); break;
    case 32: combine_rows_kernel<32><<<grid, 256, 0, st>>>(q); break;
    case 64: combine_rows_kernel<64><<<grid, 256, 0, st>>>(q); break;
    case 128: combine_rows_kernel<128><<<grid, 256, 0, st>>>(q); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
