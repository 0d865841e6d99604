// Key preparation K_hat = ReLU(k) * c (optionally after a per-token RMSNorm),
// fp32 copy and fill.
//
// Key scaling: blog.hotdry.top SANA-WM post, section "混合线性注意力" (keys are
// scaled by 1/sqrt(D*S) so that the frame transition cannot expand the state).
// HBM-bound streams: 16-byte loads and stores, grid-stride loops.
#include "gdn_common.h"

namespace gdn {

namespace {

// x * c for x >= 0, c > 0, rounded to odd in fp32: the product rounded to
// nearest, then, when it is inexact (the fma residual is nonzero), the
// truncated value with its last bit set. A later round-to-nearest-even to bf16
// (8 significant bits, far fewer than 24 - 2) then rounds the exact product
// once, as if it were converted directly (Boldo and Melquiond, "When double
// rounding is odd", 2005).
__device__ __forceinline__ float mul_round_odd(float x, float c) {
  const float p = x * c;
  const float e = __builtin_fmaf(x, c, -p);
  uint32_t b = __float_as_uint(p);
  if (e != 0.f) b = (e < 0.f ? b - 1u : b) | 1u;
  return __uint_as_float(b);
}

__global__ void __launch_bounds__(256) prepare_bf16_kernel(const uint4* __restrict__ k,
                                                           uint4* __restrict__ out, int64_t n8,
                                                           float c) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n8; i += stride) {
    uint4 x = k[i];
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t r[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t z = relu_bf16x2(w[p]);
      r[p] = pack_bf16x2(mul_round_odd(bf16_to_f32(z & 0xFFFFu), c),
                         mul_round_odd(bf16_to_f32(z >> 16), c));
    }
    out[i] = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

__global__ void __launch_bounds__(256) prepare_f32_kernel(const float* __restrict__ k,
                                                          float* __restrict__ out, int64_t n,
                                                          float c) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    float x = k[i];
    out[i] = (x > 0.f ? x : 0.f) * c;  // ReLU; -0 and negatives give +0
  }
}

__global__ void __launch_bounds__(256) copy_f32_kernel(const float* __restrict__ s,
                                                       float* __restrict__ d, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) d[i] = s[i];
}

__global__ void __launch_bounds__(256) fill_f32_kernel(float* __restrict__ d, int64_t n, float x) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) d[i] = x;
}

// K_hat = ReLU(k / rms(k)) * c with the per-token RMSNorm over D: each lane
// handles one 16-byte chunk, the kL lanes of a token are consecutive (kL
// divides 64, so a token never straddles two waves, and a token's lanes are
// active together), and the sum of squares is reduced with lane swaps.
template <bool kBf16, int kL>
__global__ void __launch_bounds__(256) prepare_norm_kernel(const uint4* __restrict__ k,
                                                           uint4* __restrict__ out, int64_t n16,
                                                           int D, float c) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) {
    const uint4 x = k[i];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float f[8];
    constexpr int kN = kBf16 ? 8 : 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (kBf16) {
        f[2 * p] = bf16_to_f32(w[p] & 0xFFFFu);
        f[2 * p + 1] = bf16_to_f32(w[p] >> 16);
      } else {
        f[p] = __uint_as_float(w[p]);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < kN; ++e) ss += f[e] * f[e];
#pragma unroll
    for (int off = 1; off < kL; off <<= 1) ss += __shfl_xor(ss, off);
    const float rc = rms_inv(ss, D) * c;
#pragma unroll
    for (int e = 0; e < kN; ++e) f[e] = (f[e] > 0.f ? f[e] : 0.f) * rc;
    uint32_t r[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      r[p] = kBf16 ? pack_bf16x2(f[2 * p], f[2 * p + 1]) : __float_as_uint(f[p]);
    out[i] = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_prepare(const Shape& sh, const void* k, void* k_hat, hipStream_t st) {
  int64_t n = sh.FH() * sh.S * sh.D;
  if (n == 0) return hipSuccess;
  if (sh.qk_norm) {
    // 16-byte chunks: D * (2 or 4) / 16 lanes per token, a power of two <= 32
    const int64_t n16 = n * (sh.io == 1 ? 2 : 4) / 16;
    const int lanes = sh.D * (sh.io == 1 ? 2 : 4) / 16;
    const uint4* src = (const uint4*)k;
    uint4* dst = (uint4*)k_hat;
    const int g = grid_for(n16);
#define GDN_PREP_NORM(BF, L) \
  prepare_norm_kernel<BF, L><<<g, 256, 0, st>>>(src, dst, n16, sh.D, sh.c)
    if (sh.io == 1) {
      switch (lanes) {
        case 2: GDN_PREP_NORM(true, 2); break;
        case 4: GDN_PREP_NORM(true, 4); break;
        case 8: GDN_PREP_NORM(true, 8); break;
        case 16: GDN_PREP_NORM(true, 16); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (lanes) {
        case 4: GDN_PREP_NORM(false, 4); break;
        case 8: GDN_PREP_NORM(false, 8); break;
        case 16: GDN_PREP_NORM(false, 16); break;
        case 32: GDN_PREP_NORM(false, 32); break;
        default: return hipErrorInvalidValue;
      }
    }
#undef GDN_PREP_NORM
    return hipGetLastError();
  }
  if (sh.io == 1) {
    // D is a multiple of 16, so n is a multiple of 8 and rows are 16-byte aligned.
    int64_t n8 = n / 8;
    prepare_bf16_kernel<<<grid_for(n8), 256, 0, st>>>((const uint4*)k, (uint4*)k_hat, n8, sh.c);
  } else {
    prepare_f32_kernel<<<grid_for(n), 256, 0, st>>>((const float*)k, (float*)k_hat, n, sh.c);
  }
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  copy_f32_kernel<<<grid_for(n), 256, 0, st>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* dst, int64_t n, float value, hipStream_t st) {
  if (n == 0) return hipSuccess;
  fill_f32_kernel<<<grid_for(n), 256, 0, st>>>(dst, n, value);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* dst, int64_t n, hipStream_t st) {
  return launch_fill_f32(dst, n, 0.f, st);
}

}  // namespace gdn
