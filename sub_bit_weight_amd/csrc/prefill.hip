// Matrix-core regime (T > 8): the two stages of y = s1 (.) U (V^T (s2 (.) x))
// as binary GEMMs (research.samsung.com NanoQuant blog, section 4, subsection
// "Inference Performance": binary GEMM kernels for batch processing; the
// stages follow the factorization equation of section 2).
//
// Each stage is C[m][n] = sum_k A[m][k] * S[k][n] with A the stage's
// activations (stage 1: x (.) s2, stage 2: t) and S = +-1 from the stage's
// sign words, words[k/32][n] bit k%32.
//
// Numerics.  +-1 is exact in fp16 and fp32 accumulation is used throughout, so
// the only rounding of a product is the conversion of A to fp16.  Each token
// row of A is first scaled by an exact power of two 2^e (chosen from the row's
// largest magnitude so that it lands in [2^13, 2^14)); the fp16 rounding then
// has relative error <= 2^-11 for every element above 2^-28 of the row maximum,
// independent of the data's range.  The epilogue multiplies by 2^-e (exact).
// For fp32 activations A is kept as two fp16 terms (hi + lo), ~22 bits.
//
// Kernels per stage: a prep kernel (row maxima, exponents, fp16 terms) and the
// GEMM.  GEMM tiles are 128 (tokens) x 256 (outputs) x 64 (reduction) per
// workgroup of 8 waves, each wave 64 x 64 as 2 x 2 v_mfma_f32_32x32x16_f16
// tiles; two workgroups fit a CU (four waves per SIMD).  A streams into a ring of LDS stages with direct global->LDS loads
// issued several 64-deep steps ahead; the +-1 operand is built in registers
// straight from the sign words: a 32x32x16 MFMA lane needs 8 signs
// of one column, and with the reduction order below two signs 16 bits apart
// become one fp16 pair with a shift and a v_and_or_b32:
//   pair q (0..15) of each 32-element block holds elements (q, q+16);
//   the prep kernel writes A in that interleaved order.
#include "nq_internal.h"

namespace nq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 256, kBK = 64;
constexpr int kWaves = 8;                 // 2 (tokens) x 4 (outputs); each wave owns 64 x 64
constexpr int kThreads = 64 * kWaves;
constexpr int kPrepThreads = 256;

enum ASrc { kAF32Scaled = 0, kABF16Scaled = 1, kAF32 = 2 };

template <int SRC>
__device__ inline float act(const void* a, const float* cs, int64_t m, int64_t K, int64_t k) {
  const int64_t g = m * K + k;
  if (SRC == kAF32Scaled) return static_cast<const float*>(a)[g] * cs[k];
  if (SRC == kABF16Scaled) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(a)[g] << 16) * cs[k];
  return static_cast<const float*>(a)[g];
}

// One workgroup per token row m:
//   e[m] = 14 - exponent(max_k |a[m][k]|)  (0 for an all-zero row)
//   out[term][m][2p], out[term][m][2p+1] = fp16 terms of a[m][k]*2^e for the
//   element pair p (block p/16, elements q and q+16 with q = p%16); zero past K.
template <int SRC>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const void* __restrict__ a,
                                                            const float* __restrict__ cs, int64_t M,
                                                            int64_t K, int64_t Kpad, int nt,
                                                            _Float16* __restrict__ out, int* __restrict__ e_out) {
  __shared__ float red[kPrepThreads / 64];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  float mx = 0.0f;
  for (int64_t k = tid; k < K; k += kPrepThreads) mx = fmaxf(mx, fabsf(act<SRC>(a, cs, m, K, k)));
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (tid % 64 == 0) red[tid / 64] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (mx > 0.0f && isfinite(mx)) {
    int ex;
    frexpf(mx, &ex);  // mx = f * 2^ex, f in [0.5, 1)
    e = 14 - ex;      // mx * 2^e in [2^13, 2^14)
  }
  if (tid == 0) e_out[m] = e;
  const int64_t npairs = Kpad / 2;
  uint32_t* hi = reinterpret_cast<uint32_t*>(out + m * Kpad);
  uint32_t* lo = reinterpret_cast<uint32_t*>(out + (M + m) * Kpad);
  for (int64_t p = tid; p < npairs; p += kPrepThreads) {
    const int64_t k0 = (p / 16) * 32 + (p % 16);
    const int64_t k1 = k0 + 16;
    const float v0 = k0 < K ? ldexpf(act<SRC>(a, cs, m, K, k0), e) : 0.0f;
    const float v1 = k1 < K ? ldexpf(act<SRC>(a, cs, m, K, k1), e) : 0.0f;
    const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
    hi[p] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    if (nt == 2) {
      const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
      lo[p] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
  }
}

// +-1 fp16 operand of a 32x32x16 MFMA lane: 8 signs of one column, the pairs
// (b+d, b+d+16) for d = 0..3 of sign word w; fp16 1.0 = 0x3C00, sign bit 15.
__device__ inline f16x8 signs_f16(uint32_t w, int b) {
  u32x4 v;
#pragma unroll
  for (int d = 0; d < 4; ++d) v[d] = ((w << (15 - b - d)) & 0x80008000u) | 0x3C003C00u;
  return __builtin_bit_cast(f16x8, v);
}

// s_waitcnt that waits until at most n vector-memory operations of this wave
// are outstanding (lgkmcnt and expcnt left alone).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int NT>
struct Pipe {
  static constexpr int S = NT == 1 ? 4 : 2;                       // LDS stages
  static constexpr int A_BYTES = NT * kBM * kBK * 2;              // A tile(s) of one stage
  static constexpr int B_BYTES = kWaves * 2 * 64 * 4;             // per wave: 2 word rows x 64 columns
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int ROWS_PER_WAVE = kBM / kWaves;              // A rows each wave moves
  static constexpr int DMA_PER_WAVE = NT * ROWS_PER_WAVE / 8;     // 8 rows (1 KiB) per 16-byte DMA
  static constexpr int PER_STAGE = DMA_PER_WAVE + 2;              // + 2 sign-word DMA instructions
};

// A stage holds NT tiles of kBM rows x kBK fp16 (128 bytes per row) written by
// direct global->LDS loads: one instruction moves 64 lanes x 16 bytes = 8 rows.
// The 16-byte chunk c of row r is stored at chunk c ^ ((r >> 1) & 7): any 16
// consecutive rows read at the same logical chunk hit 16 distinct 16-byte bank
// groups, so the 32-row fragment reads below are conflict-free.
template <int NT>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const _Float16* __restrict__ A, const int* __restrict__ erow,
                                                           const uint32_t* __restrict__ bits, int64_t ldb,
                                                           int64_t M, int64_t N, int64_t K, int64_t Kpad,
                                                           int tiles_m, int tiles_n, const float* __restrict__ colscale,
                                                           float* __restrict__ out) {
  using P = Pipe<NT>;
  extern __shared__ __attribute__((aligned(16))) char lds[];  // [S][NT][kBM][128 bytes]
  const int tid = threadIdx.x;
  const int lane = tid % 64, wave = tid / 64;
  const int wm = wave / 4, wn = wave % 4;  // wave tile: rows 64*wm .., columns 64*wn ..
  const int l32 = lane % 32, h = lane / 32;

  // XCD-aware tile order: workgroup i runs on XCD i % 8; give each XCD a
  // contiguous range of tiles (N fastest) so concurrent tiles share A rows in L2.
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (t >= ntiles) return;
  const int64_t m0 = (int64_t)(t / tiles_n) * kBM;
  const int64_t n0 = (int64_t)(t % tiles_n) * kBN;
  const int64_t nwords = cdiv(K, kWordBits);
  const int nk = (int)(Kpad / kBK);

  // this lane's DMA source rows: wave w fills rows ROWS_PER_WAVE*w .., 8 per instruction
  const int drow = lane / 8, dchunk = lane % 8;
  // Every global read is a direct global->LDS load, so no register waits on a
  // global load and the explicit vmcnt waits below are the only ones.  A stage
  // is exactly PER_STAGE such instructions per wave.  Sign words past the last
  // word row or column are clamped: they only ever meet zero-padded A columns
  // or produce outputs that are not stored.
  auto issue = [&](int kt, int st) {
    char* stage = lds + (int64_t)st * P::STAGE_BYTES;
#pragma unroll
    for (int term = 0; term < NT; ++term)
#pragma unroll
      for (int j = 0; j < P::ROWS_PER_WAVE / 8; ++j) {
        const int r = wave * P::ROWS_PER_WAVE + j * 8 + drow;
        const int64_t m = m0 + r < M ? m0 + r : M - 1;  // rows past M load row M-1 (never stored)
        const int c = dchunk ^ ((r >> 1) & 7);
        const _Float16* src = A + ((int64_t)term * M + m) * Kpad + (int64_t)kt * kBK + c * 8;
        char* dst = stage + ((int64_t)term * kBM + wave * P::ROWS_PER_WAVE + j * 8) * 128;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      }
    const int64_t n = imin(n0 + wn * 64 + lane, N - 1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t kw = imin((int64_t)kt * 2 + q, nwords - 1);
      char* dst = stage + P::A_BYTES + (wave * 2 + q) * 64 * 4;
      __builtin_amdgcn_global_load_lds(bits + kw * ldb + n, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int kt = 0; kt < P::S - 1; ++kt)
    if (kt < nk) issue(kt, kt);

  // the ring index is kept compile-time (kt = kt0 + st, st < S) so the sign
  // words stay in registers
  for (int kt0 = 0; kt0 < nk; kt0 += P::S) {
#pragma unroll
    for (int st = 0; st < P::S; ++st) {
      const int kt = kt0 + st;
      if (kt >= nk) break;
      // wait for stage kt: later stages (up to S-2 of them) may stay in flight
      const int ahead = nk - 1 - kt;
      if (ahead >= P::S - 2) {
        wait_vmcnt<(P::S - 2) * P::PER_STAGE>();
      } else if (P::S > 3 && ahead == 1) {
        wait_vmcnt<P::PER_STAGE>();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();  // every wave's DMA for stage kt landed; stage kt-1 fully consumed
      if (kt + P::S - 1 < nk) issue(kt + P::S - 1, (st + P::S - 1) % P::S);

      // 16-deep MFMA steps within the 64-deep tile; the A fragments of step
      // s+1 are read from LDS while the MFMAs of step s run
      const char* stage = lds + (int64_t)st * P::STAGE_BYTES;
      const uint32_t* bws = reinterpret_cast<const uint32_t*>(stage + P::A_BYTES) + wave * 2 * 64;
      f16x8 af[2][NT][2];
      auto read_a = [&](int s, f16x8 (&dst)[NT][2]) {
        const int chunk = (4 * (s / 2) + 2 * (s % 2) + h) ^ ((l32 >> 1) & 7);
#pragma unroll
        for (int term = 0; term < NT; ++term)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            dst[term][mb] = *reinterpret_cast<const f16x8*>(
                stage + ((int64_t)term * kBM + wm * 64 + mb * 32 + l32) * 128 + chunk * 16);
      };
      read_a(0, af[0]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s + 1 < 4) read_a(s + 1, af[(s + 1) & 1]);
        const int q = s / 2, b = 8 * (s % 2) + 4 * h;
        f16x8 bf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bf[nb] = signs_f16(bws[q * 64 + nb * 32 + l32], b);
#pragma unroll
        for (int term = 0; term < NT; ++term)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][term][mb], bf[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // 32x32 MFMA result layout: lane l, register 4a+c -> row 8a + 4(l/32) + c, column l%32.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t n = n0 + wn * 64 + nb * 32 + l32;
      const float sc = (n < N && colscale) ? colscale[n] : 1.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t m = m0 + wm * 64 + mb * 32 + 8 * a + 4 * h + c;
          if (m < M && n < N) out[m * N + n] = sc * ldexpf(acc[mb][nb][4 * a + c], -erow[m]);
        }
    }
}

size_t gemm_lds_bytes(int nt) {
  return nt == 1 ? (size_t)Pipe<1>::S * Pipe<1>::STAGE_BYTES : (size_t)Pipe<2>::S * Pipe<2>::STAGE_BYTES;
}

template <int SRC>
hipError_t launch_prep(const void* a, const float* cs, int64_t M, int64_t K, int64_t Kpad, int nt, _Float16* out,
                       int* e, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel<SRC>, dim3((unsigned)M), dim3(kPrepThreads), 0, s, a, cs, M, K, Kpad, nt, out, e);
  return hipGetLastError();
}

hipError_t launch_gemm(int nt, const _Float16* A, const int* e, const uint32_t* bits, int64_t ldb, int64_t M,
                       int64_t N, int64_t K, int64_t Kpad, const float* colscale, float* out, hipStream_t s) {
  const int tiles_m = (int)cdiv(M, kBM), tiles_n = (int)cdiv(N, kBN);
  const unsigned grid = (unsigned)(8 * ((tiles_m * tiles_n + 7) / 8));
  if (nt == 1)
    hipLaunchKernelGGL(gemm_kernel<1>, dim3(grid), dim3(kThreads), gemm_lds_bytes(1), s, A, e, bits, ldb, M, N, K,
                       Kpad, tiles_m, tiles_n, colscale, out);
  else
    hipLaunchKernelGGL(gemm_kernel<2>, dim3(grid), dim3(kThreads), gemm_lds_bytes(2), s, A, e, bits, ldb, M, N, K,
                       Kpad, tiles_m, tiles_n, colscale, out);
  return hipGetLastError();
}

struct PrefillLayout {
  int nt;
  int64_t kpad1, kpad2;
  size_t off_z, off_e1, off_t, off_t16, off_e2, total;
};

PrefillLayout prefill_layout(const nq_lrb& L, int64_t T, nq_dtype xd) {
  PrefillLayout d;
  d.nt = xd == NQ_F32 ? 2 : 1;
  d.kpad1 = round_up(L.d_in, kBK);
  d.kpad2 = round_up(L.r, kBK);
  size_t off = 0;
  d.off_z = off;
  off = align_up(off + (size_t)d.nt * T * d.kpad1 * sizeof(_Float16));
  d.off_e1 = off;
  off = align_up(off + (size_t)T * sizeof(int));
  d.off_t = off;
  off = align_up(off + (size_t)T * L.r * sizeof(float));
  d.off_t16 = off;
  off = align_up(off + (size_t)d.nt * T * d.kpad2 * sizeof(_Float16));
  d.off_e2 = off;
  off = align_up(off + (size_t)T * sizeof(int));
  d.total = off;
  return d;
}

bool lds_configured = false;

}  // namespace

size_t prefill_workspace_bytes(const nq_lrb& L, int64_t T) {
  // sized for the larger (fp32 activation) plan so one size serves both dtypes
  return prefill_layout(L, T, NQ_F32).total;
}

hipError_t launch_prefill(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                          hipStream_t s) {
  if (!lds_configured) {
    hipError_t e1 = hipFuncSetAttribute((const void*)gemm_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)gemm_lds_bytes(1));
    hipError_t e2 = hipFuncSetAttribute((const void*)gemm_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)gemm_lds_bytes(2));
    if (e1 != hipSuccess) return e1;
    if (e2 != hipSuccess) return e2;
    lds_configured = true;
  }
  const PrefillLayout d = prefill_layout(L, T, xd);
  char* base = static_cast<char*>(ws);
  _Float16* z = reinterpret_cast<_Float16*>(base + d.off_z);
  int* e1 = reinterpret_cast<int*>(base + d.off_e1);
  float* t = reinterpret_cast<float*>(base + d.off_t);
  _Float16* t16 = reinterpret_cast<_Float16*>(base + d.off_t16);
  int* e2 = reinterpret_cast<int*>(base + d.off_e2);
  hipError_t e;
  if (xd == NQ_BF16)
    e = launch_prep<kABF16Scaled>(x, L.s2, T, L.d_in, d.kpad1, d.nt, z, e1, s);
  else
    e = launch_prep<kAF32Scaled>(x, L.s2, T, L.d_in, d.kpad1, d.nt, z, e1, s);
  if (e != hipSuccess) return e;
  if ((e = launch_gemm(d.nt, z, e1, L.vt_bits, L.ldv, T, L.r, L.d_in, d.kpad1, nullptr, t, s)) != hipSuccess) return e;
  if ((e = launch_prep<kAF32>(t, nullptr, T, L.r, d.kpad2, d.nt, t16, e2, s)) != hipSuccess) return e;
  return launch_gemm(d.nt, t16, e2, L.u_bits, L.ldu, T, L.d_out, L.r, d.kpad2, L.s1, y, s);
}

}  // namespace nq
