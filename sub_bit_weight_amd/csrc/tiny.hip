// Small layers at decode sizes (T <= 8) in one workgroup.
//
// The multi-workgroup decode path runs one layer as a chain of dependent tiles
// (input pieces, stage 1, pieces of t, stage 2), each waiting on the previous
// one's counter after a counter-clearing launch: about ten global round trips,
// ~16 us for a 256 x 256 rank-64 layer whose 4 KB of sign words stream in a
// fraction of a microsecond.  Here one workgroup evaluates the factored form
// of the layer (research.samsung.com NanoQuant blog, section 2 "Low-Rank
// Binary Factorization": y = s1 (.) U (V^T (s2 (.) x)), U and V of +-1):
// z = s2 (.) x into LDS, t = V^T z into LDS, y = s1 (.) U t.  Each output is
// an fp32 sum over its reduction in index order with the exact +-1 signs
// (bit set: -1), so the result is deterministic and its error is that of one
// rounding of s2 * x and of the sequential fp32 additions.
#include "nq_internal.h"

namespace nq {
namespace {

constexpr int kTinyThreads = 256;
constexpr int64_t kTinyMaxT = 8;

__device__ inline float tiny_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// LDS: z [T][in_p] then t [T][r_p]; in_p and r_p are d_in and r rounded up to
// whole words, the tails zero, so each word's 32 positions are summed without
// a bound check (their sign bits are 0).
template <int T>
__global__ __launch_bounds__(kTinyThreads) void tiny_linear_kernel(const nq_lrb L, const void* __restrict__ x,
                                                                   int x_bf16, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int d_in = (int)L.d_in, r = (int)L.r, d_out = (int)L.d_out;
  const int in_p = (d_in + 31) & ~31, r_p = (r + 31) & ~31;
  float* z = sm;
  float* t = sm + T * in_p;
  const int tid = threadIdx.x;
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
    for (int j = tid; j < in_p; j += kTinyThreads) {
      float v = 0.0f;
      if (j < d_in) {
        const int64_t i = (int64_t)tt * d_in + j;
        const float xv = x_bf16 ? tiny_bf16(static_cast<const uint16_t*>(x)[i]) : static_cast<const float*>(x)[i];
        v = L.s2 ? L.s2[j] * xv : xv;
      }
      z[tt * in_p + j] = v;
    }
  __syncthreads();
  // t[k] = sum_j sign(V[j][k]) z[j]: thread k, words of output k in order
  for (int k = tid; k < r_p; k += kTinyThreads) {
    float acc[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) acc[tt] = 0.0f;
    if (k < r) {
      for (int w = 0; w < in_p / 32; ++w) {
        const uint32_t word = L.vt_bits[(int64_t)w * L.ldv + k];
#pragma unroll 8
        for (int b = 0; b < 32; ++b) {
          const bool neg = (word >> b) & 1u;
#pragma unroll
          for (int tt = 0; tt < T; ++tt) {
            const float v = z[tt * in_p + 32 * w + b];
            acc[tt] += neg ? -v : v;
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < T; ++tt) t[tt * r_p + k] = acc[tt];  // zero past r
  }
  __syncthreads();
  // y[i] = s1[i] sum_k sign(U[i][k]) t[k]: thread i, words of output i in order
  for (int i = tid; i < d_out; i += kTinyThreads) {
    float acc[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) acc[tt] = 0.0f;
    for (int w = 0; w < r_p / 32; ++w) {
      const uint32_t word = L.u_bits[(int64_t)w * L.ldu + i];
#pragma unroll 8
      for (int b = 0; b < 32; ++b) {
        const bool neg = (word >> b) & 1u;
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          const float v = t[tt * r_p + 32 * w + b];
          acc[tt] += neg ? -v : v;
        }
      }
    }
    const float sc = L.s1 ? L.s1[i] : 1.0f;
#pragma unroll
    for (int tt = 0; tt < T; ++tt) y[(int64_t)tt * d_out + i] = sc * acc[tt];
  }
}

size_t tiny_lds_bytes(const nq_lrb& L, int64_t T) {
  return (size_t)T * (round_up(L.d_in, kWordBits) + round_up(L.r, kWordBits)) * sizeof(float);
}

}  // namespace

// One workgroup serves the layer when its work per thread stays short: at
// most 2048 input values and 512 values of t over all tokens, and 1024
// outputs (four per thread).
bool tiny_fits(const nq_lrb& L, int64_t T) {
  return T >= 1 && T <= kTinyMaxT && T * round_up(L.d_in, kWordBits) <= 2048 &&
         T * round_up(L.r, kWordBits) <= 512 && L.d_out <= 1024;
}

hipError_t launch_tiny_linear(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, hipStream_t s) {
  const size_t lds = tiny_lds_bytes(L, T);
  switch (T) {
#define NQ_CASE(TT)                                                                                            \
  case TT:                                                                                                     \
    hipLaunchKernelGGL(tiny_linear_kernel<TT>, dim3(1), dim3(kTinyThreads), lds, s, L, x, (int)(xd == NQ_BF16), y); \
    break;
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
#undef NQ_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nq
