// Dense reconstruction of W for checking:
//   W[i,j] = s1[i] * m[i,j] * s2[j],  m[i,j] = sum_k U[i,k] V[j,k]
// (research.samsung.com NanoQuant blog, section 2, subsection "Low-Rank Binary
// Factorization", the factorization equation).
//
// m is computed exactly as r - 2*popcount(u_i xor v_j), where u_i are the signs
// of U row i along r (the stored U words) and v_j the signs of V row j along r.
// The stored V^T words run along d_in, so each block transposes a 32(j) x 32(k)
// bit tile in LDS to get v_j.  Both products are rounded to nearest even
// (__fmul_rn), so the result is unique bit for bit.
#include "nq_internal.h"

namespace nq {
namespace {

constexpr int kTi = 64;      // outputs i per block
constexpr int kTj = 32;      // inputs j per block (one V^T word row)
constexpr int kChunk = 32;   // words of r per LDS chunk (1024 ranks)
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void reconstruct_kernel(nq_lrb L, float* __restrict__ w) {
  __shared__ uint32_t ush[kTi][kChunk + 1];
  __shared__ uint32_t vtsh[kChunk * kWordBits];
  __shared__ uint32_t vsh[kTj][kChunk + 1];

  const int t = threadIdx.x;
  const int jj = t % kTj;
  const int ig = t / kTj;  // 0..7, owns 8 rows
  const int64_t jw = blockIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * kTi;
  const int64_t j = jw * kWordBits + jj;
  const int64_t nwr = cdiv(L.r, kWordBits);
  const int rem = (int)(L.r % kWordBits);
  const uint32_t last_mask = rem ? ((1u << rem) - 1u) : 0xFFFFFFFFu;

  int pc[8] = {0, 0, 0, 0, 0, 0, 0, 0};

  for (int64_t kw0 = 0; kw0 < nwr; kw0 += kChunk) {
    for (int idx = t; idx < kTi * kChunk; idx += kThreads) {
      const int kwi = idx / kTi, ii = idx % kTi;
      const int64_t kw = kw0 + kwi, i = i0 + ii;
      ush[ii][kwi] = (kw < nwr && i < L.d_out) ? L.u_bits[kw * L.ldu + i] : 0u;
    }
    for (int idx = t; idx < kChunk * kWordBits; idx += kThreads) {
      const int64_t k = kw0 * kWordBits + idx;
      vtsh[idx] = (k < L.r) ? L.vt_bits[jw * L.ldv + k] : 0u;
    }
    __syncthreads();
    for (int idx = t; idx < kTj * kChunk; idx += kThreads) {
      const int jx = idx % kTj, kwi = idx / kTj;
      uint32_t v = 0;
      for (int kb = 0; kb < kWordBits; ++kb) v |= ((vtsh[kwi * kWordBits + kb] >> jx) & 1u) << kb;
      vsh[jx][kwi] = v;
    }
    __syncthreads();
    const int nk = (int)imin(kChunk, nwr - kw0);
    for (int kwi = 0; kwi < nk; ++kwi) {
      const uint32_t mask = (kw0 + kwi == nwr - 1) ? last_mask : 0xFFFFFFFFu;
      const uint32_t v = vsh[jj][kwi];
#pragma unroll
      for (int q = 0; q < 8; ++q) pc[q] += __popc((ush[ig * 8 + q][kwi] ^ v) & mask);
    }
    __syncthreads();
  }

  if (j >= L.d_in) return;
  const float s2j = L.s2[j];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t i = i0 + ig * 8 + q;
    if (i >= L.d_out) break;
    const int m = (int)L.r - 2 * pc[q];
    w[i * L.d_in + j] = __fmul_rn(__fmul_rn(L.s1[i], (float)m), s2j);
  }
}

}  // namespace

hipError_t launch_reconstruct(const nq_lrb& L, float* w, hipStream_t s) {
  dim3 grid((unsigned)cdiv(L.d_in, kTj), (unsigned)cdiv(L.d_out, kTi));
  hipLaunchKernelGGL(reconstruct_kernel, grid, dim3(kThreads), 0, s, L, w);
  return hipGetLastError();
}

}  // namespace nq
