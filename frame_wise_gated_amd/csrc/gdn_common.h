// Shared device helpers and launch interfaces of libgdn (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kMaxChunks = 256;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two floats -> packed bf16 pair (lo = a, hi = b), round to nearest even
// (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r.x = (__bf16)a;
  r.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// ReLU on two packed bf16 values with one packed 16-bit integer max: a bf16
// with the sign bit set is a negative int16 (-0 included), so max(x, 0) as
// int16 maps it to +0 and keeps every non-negative value.
typedef short i16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t relu_bf16x2_pk(uint32_t w) {
  const i16x2_t x = __builtin_bit_cast(i16x2_t, w);
  const i16x2_t z = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, z));
}

// ReLU on two packed bf16 values: a half whose sign bit is set becomes +0.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  uint32_t neg = (w >> 15) & 0x00010001u;
  return w & ~(neg * 0xFFFFu);
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding): this wave's global loads
// except the n youngest have completed and its own LDS accesses are done.
// n = 63 leaves every global load in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | 0x70 | (((N >> 4) & 3) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads(), which waits
// for every global load in flight (vmcnt(0)) and so drains any prefetch; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier for data exchanged through LDS only: this wave's LDS accesses
// complete, then the workgroup meets; global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  wait_vmcnt_lgkm0<63>();
  bare_barrier();
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2. Kernels whose workgroups come in groups of `per` that
// read the same data (e.g. the row blocks of one head's scan, which all read
// A_t) map linear id -> (job, member) so that a job's members share one XCD.
constexpr int kNumXcd = 8;

// Work-items one dispatch can hold (its grid size is a 32-bit count).
constexpr int64_t kGridLimit = 0xFFFFFFFFLL;
inline bool grid_fits(int64_t blocks, int threads) {
  return blocks >= 0 && blocks <= kGridLimit / threads;
}

__host__ __device__ inline int64_t xcd_grid(int64_t njobs, int per) {
  return (njobs + kNumXcd - 1) / kNumXcd * kNumXcd * per;
}

__device__ __forceinline__ void xcd_job(int64_t linear, int per, int64_t* job, int* member) {
  const int64_t xcd = linear % kNumXcd;
  const int64_t slot = linear / kNumXcd;
  *job = (slot / per) * kNumXcd + xcd;
  *member = (int)(slot % per);
}

// Epsilon of the optional per-token RMSNorm of q and k.
constexpr float kRmsEps = 1e-6f;

// 1 / sqrt(mean square + eps) from a sum of squares over D entries
// (v_rsq_f32: about one ulp; the argument is at least eps, never denormal).
__device__ __forceinline__ float rms_inv(float sum_sq, int D) {
  return __builtin_amdgcn_rsqf(sum_sq * (1.0f / (float)D) + kRmsEps);
}

// Sum of squares of two packed bf16 values added to acc (v_dot2_f32_bf16;
// the bf16 products are exact in fp32).
__device__ __forceinline__ float sumsq_bf16x2(uint32_t w, float acc) {
  const bf16x2_t a = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(a, a, acc, false);
}

// Cross-lane sums in VALU (no LDS round trip). The gfx950 swaps exchange
// rows (permlane16_swap: 16-lane rows 0<->1 and 2<->3 between its two
// operands) or halves (permlane32_swap: lanes 0..31 <-> 32..63); called with
// the same value twice, the two results hold a lane's value and its partner's,
// so their sum is the pair sum in every lane.
__device__ __forceinline__ float sum_lane_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float sum_lane_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
// Sum over the 16 lanes of a DPP row (rotations by 1, 2, 4, 8).
__device__ __forceinline__ float sum_row16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  return x;
}
// Sum over the 16 lanes of the wave congruent to this one mod 4: DPP row
// rotations by 4 and 8 sum the four such lanes of each 16-lane row, then the
// row swaps add the other rows.
__device__ __forceinline__ float sum_lanes_mod4(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  return sum_lane_xor32(sum_lane_xor16(x));
}

// Internal layout of the phase-1 terms read by the MFMA scan (bf16 inputs,
// D = 128), per frame-head slot of 2*D*D floats: bf16(A) (32 KB), 32 KB not
// used, U (64 KB, fp32).
// Both are stored as 16-byte granules in the order in which the scan's MFMA
// lanes load them, so every 64-lane load instruction reads 1 KB of
// consecutive bytes:
//   A granule (n, kc): A[8kc .. 8kc+7][n] (bf16), at granule
//     index ((n/16)*4 + kc/4)*64 + (kc%4)*16 + n%16;
//   U granule (m, nc): U[m][4nc .. 4nc+3] (fp32), at granule index
//     ((m/16)*8 + nc/4)*64 + (nc%4)*16 + m%16.
// Lane l of the scan's wave w, tile nt, k-slice ks reads A granule
// (32w + 16nt + l%16, 4ks + l/16): index ((2w + nt)*4 + ks)*64 + l.
__host__ __device__ constexpr int a_granule(int n, int kc) {
  return ((n >> 4) * 4 + (kc >> 2)) * 64 + (kc & 3) * 16 + (n & 15);
}
__host__ __device__ constexpr int u_granule(int m, int nc) {
  return ((m >> 4) * 8 + (nc >> 2)) * 64 + (nc & 3) * 16 + (m & 15);
}

// Geometry shared by the host dispatcher and the kernels.
struct Shape {
  int B, H, T, S, D;
  int io;          // 0 = fp32, 1 = bf16
  float c;         // key scale applied to ReLU(k) (1 for prepared keys)
  int prepared;    // keys already hold K_hat: no ReLU
  int qk_norm;     // RMS-normalise q (and k unless prepared) per token over D
  int reuse_terms; // backward: the workspace already holds the forward's terms
  int64_t BH() const { return (int64_t)B * H; }
  int64_t FH() const { return (int64_t)B * H * T; }
};

// Frame-term outputs: for frame-head f and split p, A rows go to
// outA + f*fstride + p*sstride and U rows to outU + f*fstride + p*sstride.
struct TermsOut {
  float* outA;
  float* outU;
  int64_t fstride;
  int64_t sstride;
};

enum ScanMode : int {
  SCAN_FORWARD = 0,  // rows = D, frames ascending, U added
  SCAN_COMPOSE = 1,  // rows = 2D: C rows (identity start, no U) then H rows (zero start, U)
  SCAN_REVERSE = 2,  // rows = D, frames descending, U added, start from init (or zero)
};

struct ScanParams {
  const float* terms;   // [FH][2D][D]: A then U of every frame (granule layout of
                        // a_granule / u_granule on the MFMA path, fp32 row-major otherwise)
  const float* gamma;   // [FH]
  int T;
  int nchunk;           // chunks per head
  int mode;             // ScanMode
  const float* usrc;    // nullable: U of frame f comes from usrc slot bh*T + f + ushift
                        // (same layout as the terms' U, slots of DD floats) and is zero
                        // when f + ushift < 0; NULL = the terms' own U
  int ushift;
  const float* init;    // nullable start states (FORWARD and REVERSE):
                        // base + bh*init_bh_stride + c*init_c_stride
  int64_t init_bh_stride;
  int64_t init_c_stride;
  float* states;        // nullable [FH][D][D] per-frame states
  float* finA;          // nullable final rows < D: base + bh*fin_bh_stride + c*fin_c_stride
  float* finB;          // nullable final rows >= D (compose H rows)
  int64_t fin_bh_stride;
  int64_t fin_c_stride;
  int fin_last_only;    // write finals only for the last chunk of each head
  int64_t njobs;        // heads x chunks (set by launch_scan)
  int offsets[kMaxChunks + 1];
};

struct CombineParams {
  const float* C;       // [BH][P][D][D]
  const float* Hc;      // [BH][P][D][D]
  const float* s0;      // nullable [BH][D][D]
  float* s_start;       // [BH][P][D][D]
  int P;
  int64_t BH;           // set by launch_combine
};

// Reverse-state adjoint of the chunk-causal bidirectional scan for the
// per-frame gradients; rev == nullptr means the causal scan alone.
struct RevGrad {
  const float* rev = nullptr;    // [FH][D][D] reverse states R_t
  const float* fbuf = nullptr;   // [FH][D][D]: slot f holds F_{t+1} (unused at chunk ends)
  const float* finit = nullptr;  // [BH][nchunk][D][D]: F at each chunk's first frame
  int L = 0;                     // chunk length
  int nchunk = 0;
};

// Launchers (defined in the k_*.hip files). Each returns hipGetLastError().
hipError_t launch_prepare(const Shape& sh, const void* k, void* k_hat, hipStream_t st);
bool terms_use_mfma(const Shape& sh);
int terms_split(const Shape& sh);
// scan_layout: write A in bf16 and U in fp32, both in the granule layout the
// MFMA scan reads (MFMA path only); otherwise A and U are fp32 row-major.
hipError_t launch_terms(const Shape& sh, const void* k, const void* v, const float* beta,
                        int n_split, TermsOut out, bool scan_layout, hipStream_t st);
// Backward pass: E_t = d_o_t^T q_t (into E, the scan's granule layout) and
// dq = S_t^T do (bf16) in one pass over q and d_o (bf16, D = 128 only).
bool edq_fused(const Shape& sh);
// states2 (nullable): reverse states summed into the state of dq.
// norm: q is RMS-normalised for E and dq passes back through the norm; dq may
// be NULL (E alone).
hipError_t launch_edq(const Shape& sh, const void* q, const void* d_o, const float* states,
                      const float* states2, void* dq, float* E, bool norm, hipStream_t st);
hipError_t launch_reduce_partials(const Shape& sh, const float* partial, int n_split,
                                  TermsOut out, bool scan_layout, hipStream_t st);
bool scan_uses_mfma(const Shape& sh);
hipError_t launch_scan(const Shape& sh, const ScanParams& p, hipStream_t st);
// Two independent scans over the same terms in one launch (MFMA path only:
// scan_pairs must hold, else hipErrorInvalidValue and nothing launched).
bool scan_pairs(const Shape& sh);
hipError_t launch_scan_pair(const Shape& sh, const ScanParams& a, const ScanParams& b,
                            hipStream_t st);
hipError_t launch_combine(const Shape& sh, const CombineParams& p, hipStream_t st);
hipError_t launch_readout(const Shape& sh, const void* q, const float* st_a, const float* st_b,
                          void* o, hipStream_t st);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t st);
hipError_t launch_zero_f32(float* dst, int64_t n, hipStream_t st);
hipError_t launch_fill_f32(float* dst, int64_t n, float value, hipStream_t st);
// Backward pass (k_bwd.hip).
hipError_t launch_grad_init(const Shape& sh, const float* E, const float* ds_final, float* ginit,
                            bool granule, hipStream_t st);
// F_t at every chunk start (= E of the chunk's first frame), row-major.
hipError_t launch_chunk_init(const Shape& sh, const float* E, int L, int nchunk, float* finit,
                             bool granule, hipStream_t st);
// With rg.rev set, G_t (in gbuf / ginit) is replaced in place by G_t + F_t.
hipError_t launch_frame_grad(const Shape& sh, const float* states, const float* s0, float* gbuf,
                             float* ginit, const float* terms, bool a_granule_bf16,
                             const float* gamma, float* P, float* dgamma, const RevGrad& rg,
                             hipStream_t st);
// states2 (nullable): reverse states summed into the state of dq.
// q is read only with the RMSNorm of q (sh.qk_norm) for dq.
hipError_t launch_token_grad(const Shape& sh, const void* q, const void* k, const void* v,
                             const float* beta,
                             const void* dout, const float* states, const float* states2,
                             const float* gbuf, const float* ginit, const float* P, void* dq,
                             void* dk, void* dv, float* dbeta, hipStream_t st);
bool token_grad_uses_mfma(const Shape& sh);

}  // namespace gdn
