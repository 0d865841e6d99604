// Elementwise kernels: key preparation K_hat = ReLU(k) * c, fp32 copy and fill.
//
// Key scaling: blog.hotdry.top SANA-WM post, section "混合线性注意力" (keys are
// scaled by 1/sqrt(D*S) so that the frame transition cannot expand the state).
// HBM-bound streams: 16-byte loads and stores, grid-stride loops.
#include "gdn_common.h"

namespace gdn {

namespace {

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
      r[p] = pack_bf16x2(bf16_to_f32(z & 0xFFFFu) * c, bf16_to_f32(z >> 16) * c);
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

__global__ void __launch_bounds__(256) zero_f32_kernel(float* __restrict__ d, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) d[i] = 0.f;
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

hipError_t launch_zero_f32(float* dst, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  zero_f32_kernel<<<grid_for(n), 256, 0, st>>>(dst, n);
  return hipGetLastError();
}

}  // namespace gdn
