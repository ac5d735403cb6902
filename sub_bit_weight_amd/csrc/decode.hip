// Decode regime (T <= 8): the factored product y = s1 (.) U (V^T (s2 (.) x))
// as two binary GEMV stages (research.samsung.com NanoQuant blog, section 4,
// subsection "Inference Performance": binary GEMV kernels for token-by-token
// decoding; the stages follow the factorization equation of section 2).
//
// Each stage computes out[t][o] = sum_e sign(o,e) * v[t][e] for outputs o and
// reduction elements e, from words[e/32][o].  Lanes own outputs, so a wave
// reads 64 consecutive words of one word row (coalesced) and every lane needs
// the same v[t][e]: v is staged once per workgroup in LDS and read as a
// broadcast.  A sign is applied exactly by XOR-ing its bit into the float's
// sign bit before the fp32 add.  The reduction is split over workgroups;
// partial sums land in the workspace and are added in a fixed order, so the
// result is deterministic.
#include "nq_internal.h"

namespace nq {
namespace {

constexpr int kBlock = 256;
constexpr int kMaxLdsFloats = 8192;  // 32 KiB of staged activations per workgroup

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

enum Src { kSrcF32 = 0, kSrcBF16 = 1, kSrcF32NoScale = 2 };

// out_part[ks][t][o] = sum over e in chunk ks of sign(o,e) * v[t][e]
//   SRC kSrcF32 / kSrcBF16: v[t][e] = x[t][e] * s2[e]   (stage 1)
//   SRC kSrcF32NoScale:     v[t][e] = x[t][e]           (stage 2, x = t)
template <int T, int SRC>
__global__ __launch_bounds__(kBlock) void sign_gemv_kernel(const uint32_t* __restrict__ bits, int64_t ld,
                                                           int64_t n_out, int64_t n_red,
                                                           const void* __restrict__ xv,
                                                           const float* __restrict__ s2, int kchunk,
                                                           float* __restrict__ out_part) {
  extern __shared__ float vz[];  // [T][kchunk]
  const int ks = blockIdx.y;
  const int64_t e0 = (int64_t)ks * kchunk;
  const int klen = (int)imin(kchunk, n_red - e0);
  const int kpad = (int)round_up(klen, kWordBits);

  for (int idx = threadIdx.x; idx < T * kpad; idx += kBlock) {
    const int t = idx / kpad, e = idx - t * kpad;
    float v = 0.0f;
    if (e < klen) {
      const int64_t g = (int64_t)t * n_red + e0 + e;
      if (SRC == kSrcF32) v = static_cast<const float*>(xv)[g] * s2[e0 + e];
      if (SRC == kSrcBF16) v = bf16_to_f32(static_cast<const uint16_t*>(xv)[g]) * s2[e0 + e];
      if (SRC == kSrcF32NoScale) v = static_cast<const float*>(xv)[g];
    }
    vz[t * kchunk + e] = v;
  }
  __syncthreads();

  const int64_t o = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (o >= n_out) return;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;

  const int64_t w0 = e0 / kWordBits;
  const int nw = kpad / kWordBits;
  const uint32_t* wp = bits + w0 * ld + o;
  for (int wi = 0; wi < nw; ++wi) {
    const uint32_t word = wp[(int64_t)wi * ld];
    const float* vb = vz + wi * kWordBits;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const uint32_t sgn = (word << (31 - b)) & 0x80000000u;
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] += __uint_as_float(__float_as_uint(vb[t * kchunk + b]) ^ sgn);
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) out_part[((int64_t)ks * T + t) * n_out + o] = acc[t];
}

// out[t][o] = scale[o] * sum_ks part[ks][t][o]   (scale may be null)
__global__ __launch_bounds__(kBlock) void reduce_parts_kernel(const float* __restrict__ part, int nks,
                                                              int64_t T, int64_t n_out,
                                                              const float* __restrict__ scale,
                                                              float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= T * n_out) return;
  const int64_t o = idx % n_out;
  float acc = 0.0f;
  for (int ks = 0; ks < nks; ++ks) acc += part[(int64_t)ks * T * n_out + idx];
  out[idx] = scale ? scale[o] * acc : acc;
}

template <int SRC>
hipError_t launch_stage_t(int64_t T, const uint32_t* bits, int64_t ld, const DecodePlan& p,
                          const void* xv, const float* s2, float* part, hipStream_t s) {
  dim3 grid((unsigned)cdiv(p.n_out, kBlock), (unsigned)p.nks);
  const size_t lds = (size_t)T * p.kchunk * sizeof(float);
#define NQ_CASE(TT)                                                                               \
  case TT:                                                                                        \
    hipLaunchKernelGGL((sign_gemv_kernel<TT, SRC>), grid, dim3(kBlock), lds, s, bits, ld, p.n_out, \
                       p.n_red, xv, s2, p.kchunk, part);                                          \
    break;
  switch (T) {
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef NQ_CASE
  return hipGetLastError();
}

hipError_t launch_reduce(const float* part, int nks, int64_t T, int64_t n_out, const float* scale,
                         float* out, hipStream_t s) {
  const int64_t n = T * n_out;
  hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)cdiv(n, kBlock)), dim3(kBlock), 0, s, part, nks,
                     T, n_out, scale, out);
  return hipGetLastError();
}

struct DecodeLayout {
  DecodePlan p1, p2;
  size_t off_part1, off_t, off_part2, total;
};

DecodeLayout decode_layout(const nq_lrb& L, int64_t T) {
  DecodeLayout d;
  d.p1 = decode_plan(L.r, L.d_in, T);
  d.p2 = decode_plan(L.d_out, L.r, T);
  size_t off = 0;
  d.off_part1 = off;
  off = align_up(off + (size_t)d.p1.nks * T * L.r * sizeof(float));
  d.off_t = off;
  off = align_up(off + (size_t)T * L.r * sizeof(float));
  d.off_part2 = off;
  off = align_up(off + (size_t)d.p2.nks * T * L.d_out * sizeof(float));
  d.total = off;
  return d;
}

}  // namespace

DecodePlan decode_plan(int64_t n_out, int64_t n_red, int64_t T) {
  DecodePlan p;
  p.n_out = n_out;
  p.n_red = n_red;
  const int64_t nblk = cdiv(n_out, kBlock);
  const int64_t target = cdiv(1024, nblk);
  int64_t kc = round_up(cdiv(n_red, target), kWordBits);
  kc = imax(kc, 256);
  kc = imin(kc, (kMaxLdsFloats / T) / kWordBits * kWordBits);
  kc = imin(kc, round_up(n_red, kWordBits));
  p.kchunk = (int)kc;
  p.nks = (int)cdiv(n_red, kc);
  return p;
}

size_t decode_workspace_bytes(const nq_lrb& L, int64_t T) { return decode_layout(L, T).total; }

hipError_t launch_decode(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                         hipStream_t s) {
  const DecodeLayout d = decode_layout(L, T);
  char* base = static_cast<char*>(ws);
  float* part1 = reinterpret_cast<float*>(base + d.off_part1);
  float* tbuf = reinterpret_cast<float*>(base + d.off_t);
  float* part2 = reinterpret_cast<float*>(base + d.off_part2);
  hipError_t e;
  if (xd == NQ_BF16)
    e = launch_stage_t<kSrcBF16>(T, L.vt_bits, L.ldv, d.p1, x, L.s2, part1, s);
  else
    e = launch_stage_t<kSrcF32>(T, L.vt_bits, L.ldv, d.p1, x, L.s2, part1, s);
  if (e != hipSuccess) return e;
  if ((e = launch_reduce(part1, d.p1.nks, T, L.r, nullptr, tbuf, s)) != hipSuccess) return e;
  if ((e = launch_stage_t<kSrcF32NoScale>(T, L.u_bits, L.ldu, d.p2, tbuf, nullptr, part2, s)) != hipSuccess)
    return e;
  return launch_reduce(part2, d.p2.nks, T, L.d_out, L.s1, y, s);
}

}  // namespace nq
