// Scale-only reconstruction (research.samsung.com NanoQuant blog, section 3,
// "Phase 3: Scale-Only Model Reconstruction"): with the binary factors frozen,
// only s1 and s2 are tuned, and the loss reaches earlier layers through the
// input gradient.  For y = W x, W = s1 (.) U V^T (.) s2 (section 2, the
// factorization equation) and an output gradient g, by the chain rule:
//     u = U (V^T (s2 (.) x)),   b = V (U^T (s1 (.) g)),
//     dx = s2 (.) b,   ds1 = sum_t g (.) u,   ds2 = sum_t x (.) b.
// u is the layer's forward product without the row scale; b is the transposed
// layer's (W^T = s2 (.) V U^T (.) s1 is again a low-rank binary matrix, with
// the roles of U and V exchanged) without its row scale.  Both run through
// the forward kernels; the transposed layer's sign words come from
// transpose_signs_kernel.  This file holds the transposition and the token
// reductions.
#include "nq_internal.h"

namespace nq {

namespace {

// Sign words of the transposed sign matrix.  The source holds an n_out x n_red
// sign matrix as words[w][o] (bit b: element (o, 32w+b)); the result holds its
// transpose as words_t[w'][e] (bit b': element (e, 32w'+b') of the transpose,
// i.e. (32w'+b', e) of the source).  A wave transposes two 32 x 32 blocks: lane
// l holds source word (w, 32*(wt + l/32) + l%32); the ballot of bit b over the
// wave gives, in its low and high halves, the transposed words of element
// 32w + b for both blocks, and lane b (resp. 32 + b) keeps them.
__global__ __launch_bounds__(256) void transpose_signs_kernel(const uint32_t* __restrict__ src, int64_t n_out,
                                                              int64_t n_red, int64_t ld, uint32_t* __restrict__ dst,
                                                              int64_t ldt, int64_t nwt_pairs) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nw = (n_red + 31) / 32, nwt = (n_out + 31) / 32;
  if (wave >= nw * nwt_pairs) return;  // whole waves exit together
  const int64_t w = wave / nwt_pairs;
  const int64_t wt = (wave % nwt_pairs) * 2 + (lane >> 5);  // this lane's block of the transpose
  const int64_t o = wt * 32 + (lane & 31);
  const uint32_t word = o < n_out ? src[w * ld + o] : 0u;
  uint32_t mine = 0;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const unsigned long long m = __ballot((word >> b) & 1u);
    if ((lane & 31) == b) mine = lane < 32 ? (uint32_t)m : (uint32_t)(m >> 32);
  }
  const int64_t e = w * 32 + (lane & 31);
  if (wt < nwt && e < n_red) dst[wt * ldt + e] = mine;
}

__device__ inline float load_act(const void* p, int bf16, int64_t i) {
  return bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16) : static_cast<const float*>(p)[i];
}

// dx[t][j] = s2[j] b[t][j],  ds2[j] = sum_t x[t][j] b[t][j]  (columns j < d_in)
// ds1[i] = sum_t g[t][i] u[t][i]                            (columns d_in + i)
// Work item (column tile of 256, token chunk of tc): one thread per
// column walks the chunk's tokens in order; rows are read as whole 256- or
// 1024-byte segments per wave.  A single chunk writes ds1 / ds2 itself; else
// each chunk writes its partial sums, part[chunk][column], and
// scale_grads_sum_kernel adds them in chunk order.  Both orders are fixed:
// the sums do not depend on scheduling.  A launch covers columns
// [c_begin, c_end), so the two halves (from b, from u) can run apart.
__global__ __launch_bounds__(256) void scale_grads_partial_kernel(
    const void* __restrict__ x, int x_bf16, const void* __restrict__ g, int g_bf16, const float* __restrict__ u,
    const float* __restrict__ b, const float* __restrict__ s2, int64_t T, int64_t tc, int64_t d_in, int64_t d_out,
    float* __restrict__ dx, float* __restrict__ part, float* __restrict__ ds1, float* __restrict__ ds2,
    int64_t c_begin, int64_t c_end) {
  const int64_t c = c_begin + (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= c_end) return;
  const int64_t t0 = (int64_t)blockIdx.y * tc;
  const int64_t t1 = t0 + tc < T ? t0 + tc : T;
  const int64_t ncols = d_in + d_out;
  float acc = 0.0f;
  if (c < d_in) {
    const float sc = s2[c];
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t i = t * d_in + c;
      const float bv = b[i];
      dx[i] = sc * bv;
      acc = fmaf(load_act(x, x_bf16, i), bv, acc);
    }
  } else if (c < ncols) {
    const int64_t k = c - d_in;
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) acc = fmaf(load_act(g, g_bf16, t * d_out + k), u[t * d_out + k], acc);
  } else {
    return;
  }
  if (gridDim.y > 1)
    part[(int64_t)blockIdx.y * ncols + c] = acc;
  else if (c < d_in)
    ds2[c] = acc;
  else
    ds1[c - d_in] = acc;
}

// Four adjacent columns per thread (d_in, d_out multiples of 4; x, g, dx
// aligned for 16-byte fp32 / 8-byte bf16 vectors, checked on the host): the
// same per-column sums in the same order as scale_grads_partial_kernel, read
// and written as vectors.
__device__ inline float4 load_act4(const void* p, int bf16, int64_t i) {
  if (bf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}

__global__ __launch_bounds__(256) void scale_grads_partial4_kernel(
    const void* __restrict__ x, int x_bf16, const void* __restrict__ g, int g_bf16, const float* __restrict__ u,
    const float* __restrict__ b, const float* __restrict__ s2, int64_t T, int64_t tc, int64_t d_in, int64_t d_out,
    float* __restrict__ dx, float* __restrict__ part, float* __restrict__ ds1, float* __restrict__ ds2,
    int64_t c_begin, int64_t c_end) {
  const int64_t c = c_begin + ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= c_end) return;
  const int64_t t0 = (int64_t)blockIdx.y * tc;
  const int64_t t1 = t0 + tc < T ? t0 + tc : T;
  const int64_t ncols = d_in + d_out;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (c < d_in) {
    const float4 sc = make_float4(s2[c], s2[c + 1], s2[c + 2], s2[c + 3]);
#pragma unroll 4
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t i = t * d_in + c;
      const float4 bv = *reinterpret_cast<const float4*>(b + i);
      *reinterpret_cast<float4*>(dx + i) = make_float4(sc.x * bv.x, sc.y * bv.y, sc.z * bv.z, sc.w * bv.w);
      const float4 xv = load_act4(x, x_bf16, i);
      acc.x = fmaf(xv.x, bv.x, acc.x);
      acc.y = fmaf(xv.y, bv.y, acc.y);
      acc.z = fmaf(xv.z, bv.z, acc.z);
      acc.w = fmaf(xv.w, bv.w, acc.w);
    }
  } else if (c < ncols) {
    const int64_t k = c - d_in;
#pragma unroll 4
    for (int64_t t = t0; t < t1; ++t) {
      const float4 gv = load_act4(g, g_bf16, t * d_out + k);
      const float4 uv = *reinterpret_cast<const float4*>(u + t * d_out + k);
      acc.x = fmaf(gv.x, uv.x, acc.x);
      acc.y = fmaf(gv.y, uv.y, acc.y);
      acc.z = fmaf(gv.z, uv.z, acc.z);
      acc.w = fmaf(gv.w, uv.w, acc.w);
    }
  } else {
    return;
  }
  if (gridDim.y > 1) {
    *reinterpret_cast<float4*>(part + (int64_t)blockIdx.y * ncols + c) = acc;
  } else {
    float* d = c < d_in ? ds2 + c : ds1 + (c - d_in);
    d[0] = acc.x;
    d[1] = acc.y;
    d[2] = acc.z;
    d[3] = acc.w;
  }
}

__global__ __launch_bounds__(256) void scale_grads_sum_kernel(const float* __restrict__ part, int nchunks,
                                                              int64_t d_in, int64_t d_out, float* __restrict__ ds1,
                                                              float* __restrict__ ds2, int64_t c_begin,
                                                              int64_t c_end) {
  const int64_t c = c_begin + (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ncols = d_in + d_out;
  if (c >= c_end) return;
  float acc = 0.0f;
  for (int q = 0; q < nchunks; ++q) acc += part[(int64_t)q * ncols + c];
  if (c < d_in)
    ds2[c] = acc;
  else
    ds1[c - d_in] = acc;
}

}  // namespace

hipError_t launch_transpose_signs(const uint32_t* src, int64_t n_out, int64_t n_red, int64_t ld, uint32_t* dst,
                                  int64_t ldt, hipStream_t s) {
  const int64_t nw = cdiv(n_red, kWordBits), nwt = cdiv(n_out, kWordBits);
  const int64_t pairs = cdiv(nwt, 2);
  const int64_t blocks = cdiv(nw * pairs, 4);
  hipLaunchKernelGGL(transpose_signs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, n_out, n_red, ld, dst, ldt,
                     pairs);
  return hipGetLastError();
}

namespace {
// tokens per chunk: kGradTokens, grown so that there are at most kGradChunks
int64_t grad_chunk_tokens(int64_t T) { return std::max(kGradTokens, cdiv(T, kGradChunks)); }
}  // namespace

hipError_t launch_scale_grads_sums(const float* part, int64_t nchunks, int64_t d_in, int64_t d_out, float* ds1,
                                   float* ds2, int64_t c_begin, int64_t c_end, hipStream_t s) {
  if (c_end <= c_begin) return hipSuccess;
  hipLaunchKernelGGL(scale_grads_sum_kernel, dim3((unsigned)cdiv(c_end - c_begin, 256)), dim3(256), 0, s, part,
                     (int)nchunks, d_in, d_out, ds1, ds2, c_begin, c_end);
  return hipGetLastError();
}

size_t scale_grads_partial_bytes(int64_t T, int64_t d_in, int64_t d_out) {
  const int64_t nchunks = cdiv(T, grad_chunk_tokens(T));
  return nchunks > 1 ? (size_t)nchunks * (size_t)(d_in + d_out) * sizeof(float) : 0;
}

hipError_t launch_scale_grads_finish(const void* x, nq_dtype xd, const void* g, nq_dtype gd, const float* u,
                                     const float* b, const float* s2, int64_t T, int64_t d_in, int64_t d_out, float* dx,
                                     float* part, float* ds1, float* ds2, int64_t c_begin, int64_t c_end,
                                     hipStream_t s) {
  if (c_end <= c_begin) return hipSuccess;
  const int64_t col_tiles = cdiv(c_end - c_begin, 256);
  const int64_t tc = grad_chunk_tokens(T), nchunks = cdiv(T, tc);
  const auto vec_ok = [](const void* p, nq_dtype d) { return (uintptr_t)p % (d == NQ_BF16 ? 8 : 16) == 0; };
  if (d_in % 4 == 0 && d_out % 4 == 0 && vec_ok(x, xd) && vec_ok(g, gd) && (uintptr_t)dx % 16 == 0 &&
      (uintptr_t)u % 16 == 0 && (uintptr_t)b % 16 == 0 && (uintptr_t)part % 16 == 0)
    hipLaunchKernelGGL(scale_grads_partial4_kernel, dim3((unsigned)cdiv((c_end - c_begin) / 4, 256), (unsigned)nchunks),
                       dim3(256), 0, s, x, (int)(xd == NQ_BF16), g, (int)(gd == NQ_BF16), u, b, s2, T, tc, d_in,
                       d_out, dx, part, ds1, ds2, c_begin, c_end);
  else
    hipLaunchKernelGGL(scale_grads_partial_kernel, dim3((unsigned)col_tiles, (unsigned)nchunks), dim3(256), 0, s, x,
                       (int)(xd == NQ_BF16), g, (int)(gd == NQ_BF16), u, b, s2, T, tc, d_in, d_out, dx, part, ds1,
                       ds2, c_begin, c_end);
  if (nchunks > 1)
    hipLaunchKernelGGL(scale_grads_sum_kernel, dim3((unsigned)col_tiles), dim3(256), 0, s, part, (int)nchunks, d_in,
                       d_out, ds1, ds2, c_begin, c_end);
  return hipGetLastError();
}

}  // namespace nq
