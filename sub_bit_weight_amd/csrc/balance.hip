// Magnitude balancing and scale extraction (research.samsung.com NanoQuant
// blog, section 3, "Magnitude Balancing and Scale Extraction").  The latent
// factors U_hat [d_out][r] and V_hat [d_in][r] left by the ADMM step can be
// rescaled inversely without changing U_hat V_hat^T; the method fixes that
// freedom with eta = sqrt(||V_hat||_F / ||U_hat||_F), U = eta U_hat,
// V = V_hat / eta, and takes s1 (s2) as the mean absolute value of each row of
// U (V).  Where a norm is 0 there is no ratio: eta is then 1.
//
// HBM-bound: one read of both latents for the row statistics, then (when the
// balanced latents are wanted) one read and one write to scale them.
//   balance_rows_kernel   one wave per row: sum |.| in fp32, sum (.)^2 in fp64
//                         (fp32 squares would overflow above |v| ~ 1.8e19 and
//                         vanish below ~1e-23; squares of fp32 values are
//                         exact in fp64)
//   balance_eta_kernel    one workgroup: the squared norms in fp64, eta
//   balance_apply_kernel  one wave per row: s, and the scaled row
// Rows 0..d_out-1 are U's, d_out..d_out+d_in-1 are V's.  Every sum has a
// fixed order, so results do not depend on scheduling.
#include "nq_internal.h"

namespace nq {

namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row, 256 threads

template <typename F>
__device__ inline F wave_sum(F v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// the row's first element and its stride
__device__ inline const float* row_ptr(const float* uh, int64_t ldu, const float* vh, int64_t ldv, int64_t d_out,
                                       int64_t row) {
  return row < d_out ? uh + row * ldu : vh + (row - d_out) * ldv;
}

// Vec4: every row (of the inputs and, in balance_apply_kernel, the outputs)
// starts 16-byte aligned (checked on the host); lane l takes float4 l, l + 64,
// ...; the tail past the last whole float4 goes one float per lane.
template <bool Vec4>
__global__ __launch_bounds__(256) void balance_rows_kernel(const float* __restrict__ uh, int64_t ldu,
                                                           const float* __restrict__ vh, int64_t ldv, int64_t d_out,
                                                           int64_t rows, int64_t r, float* __restrict__ abs_sum,
                                                           double* __restrict__ sq_sum) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves
  const float* p = row_ptr(uh, ldu, vh, ldv, d_out, row);
  float a = 0.0f;
  double q = 0.0;
  int64_t k0 = 0;
  if (Vec4) {
    const int64_t n4 = r / 4;
    const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll 4
    for (int64_t i = lane; i < n4; i += 64) {
      const float4 v = p4[i];
      a += fabsf(v.x) + fabsf(v.y) + fabsf(v.z) + fabsf(v.w);
      const double x = v.x, y = v.y, z = v.z, w = v.w;
      q = fma(x, x, fma(y, y, fma(z, z, fma(w, w, q))));
    }
    k0 = n4 * 4;
  }
  for (int64_t k = k0 + lane; k < r; k += 64) {
    const float v = p[k];
    a += fabsf(v);
    q = fma((double)v, (double)v, q);
  }
  a = wave_sum(a);
  q = wave_sum(q);
  if (lane == 0) {
    abs_sum[row] = a;
    sq_sum[row] = q;
  }
}

// eta from the rows' squared sums; one workgroup of 1024 threads, thread i
// adds rows i, i + 1024, ... in fp64, then a fixed tree over the threads.
__global__ __launch_bounds__(1024) void balance_eta_kernel(const double* __restrict__ sq_sum, int64_t d_out,
                                                           int64_t d_in, float* __restrict__ eta) {
  __shared__ double su[1024], sv[1024];
  const int tid = threadIdx.x;
  double a = 0.0, b = 0.0;
#pragma unroll 8
  for (int64_t i = tid; i < d_out; i += 1024) a += sq_sum[i];
#pragma unroll 8
  for (int64_t i = tid; i < d_in; i += 1024) b += sq_sum[d_out + i];
  su[tid] = a;
  sv[tid] = b;
  __syncthreads();
  for (int h = 512; h >= 1; h >>= 1) {
    if (tid < h) {
      su[tid] += su[tid + h];
      sv[tid] += sv[tid + h];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double nu = su[0], nv = sv[0];
    // sqrt(||V|| / ||U||) = (||V||^2 / ||U||^2)^(1/4); no ratio when a norm is 0
    eta[0] = (nu > 0.0 && nv > 0.0) ? (float)sqrt(sqrt(nv / nu)) : 1.0f;
  }
}

// s1[i] = eta * mean_k |U_hat[i][k]|, s2[j] = mean_k |V_hat[j][k]| / eta; with
// outputs, U = eta U_hat and V = V_hat / eta row by row (each element read and
// written by the same lane: the outputs may be the inputs).
template <bool Vec4>
__global__ __launch_bounds__(256) void balance_apply_kernel(const float* uh, int64_t ldu, const float* vh,
                                                            int64_t ldv, int64_t d_out, int64_t rows, int64_t r,
                                                            const float* __restrict__ abs_sum,
                                                            const float* __restrict__ eta_p, float* uo, float* vo,
                                                            float* __restrict__ s1, float* __restrict__ s2) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float eta = *eta_p;
  const bool is_u = row < d_out;
  if (lane == 0) {
    const float mean = abs_sum[row] / (float)r;
    if (is_u)
      s1[row] = eta * mean;
    else
      s2[row - d_out] = mean / eta;
  }
  if (!uo) return;
  const float* p = row_ptr(uh, ldu, vh, ldv, d_out, row);
  float* o = is_u ? uo + row * ldu : vo + (row - d_out) * ldv;
  int64_t k0 = 0;
  if (Vec4) {
    const int64_t n4 = r / 4;
    const float4* p4 = reinterpret_cast<const float4*>(p);
    float4* o4 = reinterpret_cast<float4*>(o);
    if (is_u) {
#pragma unroll 4
      for (int64_t i = lane; i < n4; i += 64) {
        const float4 v = p4[i];
        o4[i] = make_float4(eta * v.x, eta * v.y, eta * v.z, eta * v.w);
      }
    } else {
#pragma unroll 4
      for (int64_t i = lane; i < n4; i += 64) {
        const float4 v = p4[i];
        o4[i] = make_float4(v.x / eta, v.y / eta, v.z / eta, v.w / eta);
      }
    }
    k0 = n4 * 4;
  }
  if (is_u) {
    for (int64_t k = k0 + lane; k < r; k += 64) o[k] = eta * p[k];
  } else {
    for (int64_t k = k0 + lane; k < r; k += 64) o[k] = p[k] / eta;
  }
}

}  // namespace

size_t balance_workspace_bytes(int64_t d_out, int64_t d_in) {
  return align_up((size_t)(d_out + d_in) * sizeof(float)) + align_up((size_t)(d_out + d_in) * sizeof(double));
}

hipError_t launch_balance(const float* uh, int64_t ldu, const float* vh, int64_t ldv, int64_t d_out, int64_t d_in,
                          int64_t r, float* uo, float* vo, float* s1, float* s2, float* eta, void* workspace,
                          hipStream_t s) {
  const int64_t rows = d_out + d_in;
  float* abs_sum = static_cast<float*>(workspace);
  double* sq_sum = reinterpret_cast<double*>(static_cast<char*>(workspace) + align_up((size_t)rows * sizeof(float)));
  const bool vec4 = ((uintptr_t)uh % 16 == 0) && ((uintptr_t)vh % 16 == 0) && ldu % 4 == 0 && ldv % 4 == 0;
  const dim3 grid((unsigned)cdiv(rows, kRowsPerBlock));
  if (vec4)
    hipLaunchKernelGGL(balance_rows_kernel<true>, grid, dim3(256), 0, s, uh, ldu, vh, ldv, d_out, rows, r, abs_sum,
                       sq_sum);
  else
    hipLaunchKernelGGL(balance_rows_kernel<false>, grid, dim3(256), 0, s, uh, ldu, vh, ldv, d_out, rows, r, abs_sum,
                       sq_sum);
  hipLaunchKernelGGL(balance_eta_kernel, dim3(1), dim3(1024), 0, s, sq_sum, d_out, d_in, eta);
  const bool vec4_out = vec4 && (!uo || ((uintptr_t)uo % 16 == 0 && (uintptr_t)vo % 16 == 0));
  if (vec4_out)
    hipLaunchKernelGGL(balance_apply_kernel<true>, grid, dim3(256), 0, s, uh, ldu, vh, ldv, d_out, rows, r, abs_sum,
                       eta, uo, vo, s1, s2);
  else
    hipLaunchKernelGGL(balance_apply_kernel<false>, grid, dim3(256), 0, s, uh, ldu, vh, ldv, d_out, rows, r, abs_sum,
                       eta, uo, vo, s1, s2);
  return hipGetLastError();
}

}  // namespace nq
