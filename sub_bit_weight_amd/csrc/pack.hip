// Sign packing, unpacking and the synthetic-word generator.
//
// Packing freezes sign(U) and sign(V) of the latent factors into 32-bit words
// (research.samsung.com NanoQuant blog, section 3 "Step 3: Factorized Component
// Refinement" for sign(U), sign(V); section 3 "Phase 3: Scale-Only Model
// Reconstruction" for packing the frozen factors into integer formats).
// Word layout: words[w*ld + o], bit b <-> element (o, 32w+b), 1 = -1.
#include "nq_internal.h"

namespace nq {
namespace {

constexpr int kBlock = 256;
constexpr int64_t kMaxGridY = 65535;

// One thread builds one word: 32 compares of consecutive reduction elements.
// For V (stride_out = 1) neighbouring threads read neighbouring floats.
__global__ __launch_bounds__(kBlock) void pack_kernel(const float* __restrict__ src, int64_t n_out,
                                                      int64_t n_red, int64_t so, int64_t sr,
                                                      uint32_t* __restrict__ dst, int64_t ld) {
  const int64_t o = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (o >= n_out) return;
  const int64_t nw = cdiv(n_red, kWordBits);
  for (int64_t w = blockIdx.y; w < nw; w += gridDim.y) {
    const int64_t e0 = w * kWordBits;
    const int nb = (int)imin(kWordBits, n_red - e0);
    const float* p = src + o * so + e0 * sr;
    uint32_t word = 0;
    for (int b = 0; b < nb; ++b) {
      // IEEE compare: NaN, +0 and -0 are not < 0 and pack as +1.
      word |= (uint32_t)(p[b * sr] < 0.0f) << b;
    }
    dst[w * ld + o] = word;
  }
}

// dst[o][e] = +-1 from bit e%32 of words[e/32][o].
__global__ __launch_bounds__(kBlock) void unpack_kernel(const uint32_t* __restrict__ bits, int64_t n_out,
                                                        int64_t n_red, int64_t ld,
                                                        float* __restrict__ dst) {
  const int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (e >= n_red) return;
  for (int64_t o = blockIdx.y; o < n_out; o += gridDim.y) {
    const uint32_t word = bits[(e / kWordBits) * ld + o];
    const uint32_t bit = (word >> (e % kWordBits)) & 1u;
    dst[o * n_red + e] = bit ? -1.0f : 1.0f;
  }
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014; Vigna's constants):
// output i of the stream started at `seed` is mix(seed + (i+1)*gamma).
__device__ inline uint64_t splitmix64(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(kBlock) void fill_words_kernel(uint32_t* __restrict__ dst, int64_t n,
                                                            uint64_t seed) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
    dst[i] = (uint32_t)splitmix64(seed, (uint64_t)i);
  }
}

}  // namespace

hipError_t launch_pack(const float* src, int64_t n_out, int64_t n_red, int64_t so, int64_t sr,
                       uint32_t* dst, int64_t ld, hipStream_t s) {
  const int64_t nw = cdiv(n_red, kWordBits);
  dim3 grid((unsigned)cdiv(n_out, kBlock), (unsigned)min(nw, kMaxGridY));
  hipLaunchKernelGGL(pack_kernel, grid, dim3(kBlock), 0, s, src, n_out, n_red, so, sr, dst, ld);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* bits, int64_t n_out, int64_t n_red, int64_t ld, float* dst,
                         hipStream_t s) {
  dim3 grid((unsigned)cdiv(n_red, kBlock), (unsigned)min(n_out, kMaxGridY));
  hipLaunchKernelGGL(unpack_kernel, grid, dim3(kBlock), 0, s, bits, n_out, n_red, ld, dst);
  return hipGetLastError();
}

hipError_t launch_fill_words(uint32_t* dst, int64_t n, uint64_t seed, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = imin(cdiv(n, kBlock), 65536);
  hipLaunchKernelGGL(fill_words_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, dst, n, seed);
  return hipGetLastError();
}

}  // namespace nq
