// Matrix-core regime (T > 8): the two stages of y = s1 (.) U (V^T (s2 (.) x))
// as binary GEMMs (research.samsung.com NanoQuant blog, section 4, subsection
// "Inference Performance": binary GEMM kernels for batch processing).
//
// C[m][n] = sum_k A[m][k] * S[k][n] with A the activations of the stage
// (stage 1: x*s2, stage 2: t) and S = +-1 from the sign words of the stage.
// +-1 is exact in bf16, so the only rounding of the product is the conversion
// of A to bf16.  A is written as a sum of NT bf16 terms (hi, lo, ...), each
// multiplied on the matrix cores with fp32 accumulation
// (v_mfma_f32_16x16x32_bf16).  NT = 1 rounds A once, NT = 2 keeps ~16
// significant bits, NT = 3 keeps fp32's 24.
#include "nq_internal.h"

namespace nq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileM = 64;
constexpr int kTileN = 64;

enum ASrc { kAF32Scaled = 0, kABF16Scaled = 1, kAF32 = 2 };

template <int SRC>
__device__ inline float load_a(const void* __restrict__ a, const float* __restrict__ cs, int64_t M,
                               int64_t K, int64_t m, int64_t k) {
  if (m >= M || k >= K) return 0.0f;
  const int64_t g = m * K + k;
  if (SRC == kAF32Scaled) return static_cast<const float*>(a)[g] * cs[k];
  if (SRC == kABF16Scaled)
    return __uint_as_float((uint32_t) static_cast<const uint16_t*>(a)[g] << 16) * cs[k];
  return static_cast<const float*>(a)[g];
}

// +-1 bf16 operand for 8 consecutive reduction elements starting at bit `b0`
// of `word`: bf16 1.0 = 0x3F80, the sign bit (bit 15) set for a stored 1.
__device__ inline bf16x8 signs_to_bf16(uint32_t word, int b0) {
  const uint32_t s = word >> b0;
  u32x4 v;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = (s >> (2 * d)) & 1u, hi = (s >> (2 * d + 1)) & 1u;
    v[d] = 0x3F803F80u | (lo << 15) | (hi << 31);
  }
  return __builtin_bit_cast(bf16x8, v);
}

// One workgroup = 4 waves = a 64x64 tile of C; a wave owns a 32x32 quarter
// as 2x2 MFMA tiles of 16x16.  Lane l of a 16x16x32 MFMA holds A row l%16 and
// B column l%16 for the 8 reduction elements of group l/16; A and B use the
// same element order, so the pairing of reduction indices is consistent.
template <int NT, int SRC>
__global__ __launch_bounds__(kThreads) void sign_gemm_kernel(const void* __restrict__ a,
                                                             const float* __restrict__ colscale,
                                                             const uint32_t* __restrict__ bits,
                                                             int64_t ld, int64_t M, int64_t N, int64_t K,
                                                             const float* __restrict__ rowscale,
                                                             float* __restrict__ out) {
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int64_t m_base = (int64_t)blockIdx.y * kTileM + (wave / 2) * 32;
  const int64_t n_base = (int64_t)blockIdx.x * kTileN + (wave % 2) * 32;
  const int r16 = lane % 16, grp = lane / 16;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < K; k0 += 32) {
    bf16x8 bfrag[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n_base + j * 16 + r16;
      const uint32_t word = (n < N) ? bits[(k0 / 32) * ld + n] : 0u;
      bfrag[j] = signs_to_bf16(word, 8 * grp);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t m = m_base + i * 16 + r16;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = load_a<SRC>(a, colscale, M, K, m, k0 + 8 * grp + e);
#pragma unroll
      for (int term = 0; term < NT; ++term) {
        bf16x8 af;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 h = static_cast<__bf16>(v[e]);
          af[e] = h;
          v[e] = v[e] - static_cast<float>(h);  // exact residual
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfrag[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // C/D layout of a 16x16 MFMA: lane l, register q -> row 4*(l/16)+q, column l%16.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n_base + j * 16 + r16;
      if (n >= N) continue;
      const float sc = rowscale ? rowscale[n] : 1.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m_base + i * 16 + 4 * grp + q;
        if (m < M) out[m * N + n] = sc * acc[i][j][q];
      }
    }
}

template <int SRC>
hipError_t launch_gemm(int nt, const void* a, const float* cs, const uint32_t* bits, int64_t ld, int64_t M,
                       int64_t N, int64_t K, const float* rs, float* out, hipStream_t s) {
  dim3 grid((unsigned)cdiv(N, kTileN), (unsigned)cdiv(M, kTileM));
  switch (nt) {
    case 1: hipLaunchKernelGGL((sign_gemm_kernel<1, SRC>), grid, dim3(kThreads), 0, s, a, cs, bits, ld, M, N, K, rs, out); break;
    case 2: hipLaunchKernelGGL((sign_gemm_kernel<2, SRC>), grid, dim3(kThreads), 0, s, a, cs, bits, ld, M, N, K, rs, out); break;
    case 3: hipLaunchKernelGGL((sign_gemm_kernel<3, SRC>), grid, dim3(kThreads), 0, s, a, cs, bits, ld, M, N, K, rs, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(const nq_lrb& L, int64_t T) {
  return align_up((size_t)T * L.r * sizeof(float));
}

hipError_t launch_prefill(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                          hipStream_t s) {
  float* t = static_cast<float*>(ws);
  // bf16 x: split the cheaper stage's activations into two bf16 terms, round
  // the other stage's once.  fp32 x: three terms on both stages.
  int nt1, nt2;
  if (xd == NQ_F32) {
    nt1 = nt2 = 3;
  } else if (L.d_in <= L.d_out) {
    nt1 = 2, nt2 = 1;
  } else {
    nt1 = 1, nt2 = 2;
  }
  hipError_t e;
  if (xd == NQ_BF16)
    e = launch_gemm<kABF16Scaled>(nt1, x, L.s2, L.vt_bits, L.ldv, T, L.r, L.d_in, nullptr, t, s);
  else
    e = launch_gemm<kAF32Scaled>(nt1, x, L.s2, L.vt_bits, L.ldv, T, L.r, L.d_in, nullptr, t, s);
  if (e != hipSuccess) return e;
  return launch_gemm<kAF32>(nt2, t, nullptr, L.u_bits, L.ldu, T, L.d_out, L.r, L.s1, y, s);
}

}  // namespace nq
