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

// Reduction elements contiguous (stride_red = 1: the U latent [d_out][r]):
// a workgroup takes 16 outputs x 32 words.  Wave q builds the words of
// outputs 4q..4q+3, one 1024-element run of a latent row each: lane l reads
// the float4 at element 32w0 + 256j + 4l (j < 4; whole float4s with Vec4,
// rows 16-byte aligned, checked on the host), turns it into a nibble of sign
// bits, and three shuffles gather the nibbles of lanes 8m..8m+7 into word
// w0 + 8j + m at lane 8m.  The words go through LDS so that each word row is
// stored as 16 consecutive outputs.  blockIdx.x walks the word tiles of the
// same outputs, so the workgroups that run together read a contiguous band
// of whole latent rows.
constexpr int kRowTile = 16, kRowTileWords = 32;

template <bool Vec4>
__global__ __launch_bounds__(kBlock) void pack_rows_kernel(const float* __restrict__ src, int64_t n_out,
                                                           int64_t n_red, int64_t so, uint32_t* __restrict__ dst,
                                                           int64_t ld) {
  __shared__ uint32_t words[kRowTileWords][kRowTile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nw = cdiv(n_red, kWordBits);
  const int64_t w0 = (int64_t)blockIdx.x * kRowTileWords;
  for (int64_t o0 = (int64_t)blockIdx.y * kRowTile; o0 < n_out; o0 += (int64_t)gridDim.y * kRowTile) {
    for (int i = 0; i < kRowTile / 4; ++i) {
      const int row = wave * (kRowTile / 4) + i;
      const int64_t o = o0 + row;
      if (o >= n_out) break;  // uniform over the wave
      const float* p = src + o * so;
      float4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t e = w0 * kWordBits + 256 * j + 4 * lane;
        // elements past n_red are not read and give 0 bits
        if (Vec4 && e + 3 < n_red) {
          v[j] = *reinterpret_cast<const float4*>(p + e);
        } else {
          v[j].x = e < n_red ? p[e] : 0.0f;
          v[j].y = e + 1 < n_red ? p[e + 1] : 0.0f;
          v[j].z = e + 2 < n_red ? p[e + 2] : 0.0f;
          v[j].w = e + 3 < n_red ? p[e + 3] : 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // IEEE compare: NaN, +0 and -0 are not < 0 and pack as +1
        uint32_t x = (uint32_t)(v[j].x < 0.0f) | (uint32_t)(v[j].y < 0.0f) << 1 | (uint32_t)(v[j].z < 0.0f) << 2 |
                     (uint32_t)(v[j].w < 0.0f) << 3;
        x |= (uint32_t)__shfl_down((int)x, 1, 64) << 4;
        x |= (uint32_t)__shfl_down((int)x, 2, 64) << 8;
        x |= (uint32_t)__shfl_down((int)x, 4, 64) << 16;
        if ((lane & 7) == 0) words[8 * j + (lane >> 3)][row] = x;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int w = h * (kBlock / kRowTile) + threadIdx.x / kRowTile, row = threadIdx.x % kRowTile;
      if (o0 + row < n_out && w0 + w < nw) dst[(w0 + w) * ld + o0 + row] = words[w][row];
    }
    __syncthreads();
  }
}

// Outputs contiguous (stride_out = 1: the V latent [d_in][r]) with 16-byte
// aligned rows and n_out % 4 == 0 (checked on the host): one thread builds
// the words of outputs 4t..4t+3, reading one float4 per reduction element, so
// a wave reads 1 KB of one latent row per load.
__global__ __launch_bounds__(kBlock) void pack_cols4_kernel(const float* __restrict__ src, int64_t n_out,
                                                            int64_t n_red, int64_t sr, uint32_t* __restrict__ dst,
                                                            int64_t ld) {
  const int64_t o = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4;
  if (o >= n_out) return;
  const int64_t nw = cdiv(n_red, kWordBits);
  for (int64_t w = blockIdx.y; w < nw; w += gridDim.y) {
    const int64_t e0 = w * kWordBits;
    const int nb = (int)imin(kWordBits, n_red - e0);
    const float* p = src + e0 * sr + o;
    uint32_t a = 0, b = 0, c = 0, d = 0;
#pragma unroll 8
    for (int k = 0; k < nb; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(p + k * sr);
      a |= (uint32_t)(v.x < 0.0f) << k;
      b |= (uint32_t)(v.y < 0.0f) << k;
      c |= (uint32_t)(v.z < 0.0f) << k;
      d |= (uint32_t)(v.w < 0.0f) << k;
    }
    uint32_t* q = dst + w * ld + o;
    q[0] = a;
    q[1] = b;
    q[2] = c;
    q[3] = d;
  }
}

}  // namespace

hipError_t launch_pack(const float* src, int64_t n_out, int64_t n_red, int64_t so, int64_t sr,
                       uint32_t* dst, int64_t ld, hipStream_t s) {
  const int64_t nw = cdiv(n_red, kWordBits);
  if (sr == 1) {
    dim3 grid((unsigned)cdiv(nw, kRowTileWords), (unsigned)min(cdiv(n_out, kRowTile), kMaxGridY));
    if ((uintptr_t)src % 16 == 0 && so % 4 == 0)
      hipLaunchKernelGGL(pack_rows_kernel<true>, grid, dim3(kBlock), 0, s, src, n_out, n_red, so, dst, ld);
    else
      hipLaunchKernelGGL(pack_rows_kernel<false>, grid, dim3(kBlock), 0, s, src, n_out, n_red, so, dst, ld);
    return hipGetLastError();
  }
  if (so == 1 && n_out % 4 == 0 && sr % 4 == 0 && (uintptr_t)src % 16 == 0) {
    dim3 grid((unsigned)cdiv(n_out / 4, kBlock), (unsigned)min(nw, kMaxGridY));
    hipLaunchKernelGGL(pack_cols4_kernel, grid, dim3(kBlock), 0, s, src, n_out, n_red, sr, dst, ld);
    return hipGetLastError();
  }
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
