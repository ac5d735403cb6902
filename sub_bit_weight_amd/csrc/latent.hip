// The refinement forward at decode sizes (T <= 8) with the signs taken from
// the fp32 latent factors as they load: y = s1 (.) sign(U)(sign(V)^T (s2 (.) x))
// (research.samsung.com NanoQuant blog, section 3 "Step 3: Factorized
// Component Refinement": the forward pass uses sign(U) and sign(V) of latents
// that the refinement keeps updating).  sign() is the packing rule: -1 only for
// values < 0 (NaN, +0 and -0 give +1).
//
// At T <= 8 the latents are the bytes (4 per weight, against T*(...) of
// activations), so the two stages are plain HBM-bound products over the fp32
// matrices, each latent read once, with the sign applied to the activation it
// multiplies.  Packing first would read the latents just the same, then write
// and re-read the words and launch the packed layer: this reads them once.
//
//  * Stage 1, t = sign(V)^T z with z = s2 (.) x, V latent [d_in][ldv]: a
//    workgroup takes 256 consecutive outputs k (a float4 of one latent row per
//    lane, so a wave reads 1 KB of a row per load) over a span of rows j, wave
//    w taking rows j0 + w, j0 + w + 4, ...; z of the span sits in LDS.  The
//    waves' sums are added in wave order in LDS, the spans' partial sums in
//    span order by the last workgroup of the column tile to finish.
//  * Stage 2, y = s1 (.) sign(U) t, U latent [d_out][ldu]: a wave takes four
//    rows, its lanes 256 consecutive reduction elements at a time (1 KB of a
//    row per load), t of the workgroup's span in LDS; lane sums are added
//    across the wave, spans in order by the last workgroup of the row block.
// Everything is fp32 and deterministic (fixed summation orders).
#include "nq_internal.h"

namespace nq {
namespace {

constexpr int kLatThreads = 256;
constexpr int kS1Waves = kLatThreads / 64;
constexpr int kS1Cols = 4 * 64;           // stage-1 outputs per workgroup (a float4 per lane)
constexpr int kS1MaxSpan = 1024;          // stage-1 rows per workgroup, at most
constexpr int kS1MinSpan = 64;
constexpr int kS1Target = 512;            // stage-1 workgroups to aim for (two per CU)
constexpr int kS2RowsPerWave = 4;
constexpr int kS2Rows = kS2RowsPerWave * (kLatThreads / 64);  // 16 rows per workgroup
constexpr int kS2Span = 2048;             // stage-2 reduction elements per workgroup, at most
constexpr int kS2MinSpan = 256;
constexpr int kS2Target = 2048;           // stage-2 workgroups to aim for at T = 1 (divided by T)

__device__ inline float signed_by(float lat, float v) { return lat < 0.0f ? -v : v; }

// Partial sums read by another workgroup of the same launch: agent-scope
// stores, then (after every thread's stores completed and a barrier) a relaxed
// counter increment; the last workgroup acquires before it reads them.
__device__ inline void store_agent(float* p, float v) {
  typedef __attribute__((address_space(1))) float* gptr;
  __hip_atomic_store((gptr)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline bool last_to_arrive(int* ctr, int n, int* s_last) {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): this thread's stores are out
  __syncthreads();
  if (threadIdx.x == 0) {
    typedef __attribute__((address_space(1))) int* gptr;
    *s_last = __hip_atomic_fetch_add((gptr)ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
    if (*s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return *s_last != 0;
}

__global__ void lat_zero_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// VEC: the latent is 16-byte aligned with a row stride that is a multiple of
// 4, so every float4 that starts before the row's end lies inside the row's
// stride; threads past the last column read the last float4 again (results
// dropped), and the loop has no branch.
template <int T, bool VEC>
__global__ __launch_bounds__(kLatThreads) void lat_stage1_kernel(const float* __restrict__ v_lat, int64_t ldv,
                                                                 int64_t d_in, int64_t r, const void* __restrict__ x,
                                                                 int x_bf16, const float* __restrict__ s2, int span,
                                                                 float* __restrict__ part, int* __restrict__ ctr,
                                                                 float* __restrict__ t) {
  __shared__ float zs[T][kS1MaxSpan];
  __shared__ __attribute__((aligned(16))) float red[kS1Waves][T][kS1Cols];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nsp = (int)gridDim.y, sp = (int)blockIdx.y;
  const int64_t j0 = (int64_t)sp * span;
  const int n = (int)imin(span, d_in - j0);
  for (int i = tid; i < T * span; i += kLatThreads) {
    const int tt = i / span, jj = i % span;
    float z = 0.0f;
    if (jj < n) {
      const int64_t j = j0 + jj, idx = (int64_t)tt * d_in + j;
      const float xv = x_bf16 ? __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[idx] << 16)
                              : static_cast<const float*>(x)[idx];
      z = xv * s2[j];
    }
    zs[tt][jj] = z;
  }
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kS1Cols;  // the tile's first output
  const int64_t k0 = c0 + 4 * lane;
  float acc[T][4];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) acc[tt][0] = acc[tt][1] = acc[tt][2] = acc[tt][3] = 0.0f;
  const float* col = v_lat + j0 * ldv + (VEC ? imin(k0, (r - 1) & ~int64_t{3}) : k0);
  constexpr int kUnroll = T <= 4 ? 8 : 4;  // rows in flight per lane
#pragma unroll kUnroll
  for (int jj = wv; jj < n; jj += kS1Waves) {
    const float* p = col + (int64_t)jj * ldv;
    float v[4];
    if constexpr (VEC) {
      const float4 q = *reinterpret_cast<const float4*>(p);
      v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = k0 + c < r ? p[c] : 0.0f;
    }
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const float z = zs[tt][jj];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[tt][c] += signed_by(v[c], z);
    }
  }
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
    *reinterpret_cast<float4*>(&red[wv][tt][4 * lane]) = make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
  __syncthreads();
  // (output, token) pairs of the tile, spread over the workgroup: the waves'
  // sums in wave order
  constexpr int kPairs = (T * kS1Cols + kLatThreads - 1) / kLatThreads;
  float sum[kPairs];
#pragma unroll
  for (int q = 0; q < kPairs; ++q) {
    const int pi = tid + q * kLatThreads;  // pair: token pi / kS1Cols, output pi % kS1Cols
    sum[q] = 0.0f;
    if (pi < T * kS1Cols) {
#pragma unroll
      for (int w = 0; w < kS1Waves; ++w) sum[q] += red[w][pi / kS1Cols][pi % kS1Cols];
    }
  }
  if (nsp == 1) {
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      const int pi = tid + q * kLatThreads;
      const int64_t k = c0 + pi % kS1Cols;
      if (pi < T * kS1Cols && k < r) t[(int64_t)(pi / kS1Cols) * r + k] = sum[q];
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < kPairs; ++q) {
    const int pi = tid + q * kLatThreads;
    const int64_t k = c0 + pi % kS1Cols;
    if (pi < T * kS1Cols && k < r) store_agent(part + ((int64_t)sp * T + pi / kS1Cols) * r + k, sum[q]);
  }
  if (!last_to_arrive(ctr + blockIdx.x, nsp, &s_last)) return;
#pragma unroll
  for (int q = 0; q < kPairs; ++q) {
    const int pi = tid + q * kLatThreads;
    const int tt = pi / kS1Cols;
    const int64_t k = c0 + pi % kS1Cols;
    if (pi >= T * kS1Cols || k >= r) continue;
    float total = 0.0f;
#pragma unroll 8
    for (int s = 0; s < nsp; ++s) total += part[((int64_t)s * T + tt) * r + k];
    t[(int64_t)tt * r + k] = total;
  }
}

// VEC as for stage 1: lanes past the span's end and rows past the last read
// the last float4 of the span and the last row again (their t is 0, their
// sums dropped), so the loop has no branch.
template <int T, bool VEC>
__global__ __launch_bounds__(kLatThreads) void lat_stage2_kernel(const float* __restrict__ u_lat, int64_t ldu,
                                                                 int64_t d_out, int64_t r, const float* __restrict__ t,
                                                                 const float* __restrict__ s1,
                                                                 float* __restrict__ part, int* __restrict__ ctr,
                                                                 float* __restrict__ y, int span) {
  __shared__ __attribute__((aligned(16))) float ts[T][kS2Span];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nsp = (int)gridDim.y, sp = (int)blockIdx.y;
  const int64_t k0 = (int64_t)sp * span;
  const int n = (int)imin(span, r - k0);
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
    for (int kk = tid; kk < span; kk += kLatThreads)  // span: a multiple of 256, at most kS2Span
      ts[tt][kk] = kk < n ? t[(int64_t)tt * r + k0 + kk] : 0.0f;
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * kS2Rows + wv * kS2RowsPerWave;
  float acc[kS2RowsPerWave][T];
#pragma unroll
  for (int rr = 0; rr < kS2RowsPerWave; ++rr)
#pragma unroll
    for (int tt = 0; tt < T; ++tt) acc[rr][tt] = 0.0f;
  for (int kb = 0; kb < n; kb += 256) {  // (unrolled twice: slower)
    const int kk = kb + 4 * lane;  // < span; t is zero past n
    float tv[T][4];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const float4 q = *reinterpret_cast<const float4*>(&ts[tt][kk]);
      tv[tt][0] = q.x, tv[tt][1] = q.y, tv[tt][2] = q.z, tv[tt][3] = q.w;
    }
#pragma unroll
    for (int rr = 0; rr < kS2RowsPerWave; ++rr) {
      const int64_t i = imin(i0 + rr, d_out - 1);
      float u[4];
      if constexpr (VEC) {
        const float4 q = *reinterpret_cast<const float4*>(u_lat + i * ldu + k0 + imin(kk, (n - 1) & ~3));
        u[0] = q.x, u[1] = q.y, u[2] = q.z, u[3] = q.w;
      } else {
        const float* p = u_lat + i * ldu + k0 + kk;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = kk + c < n ? p[c] : 0.0f;
      }
#pragma unroll
      for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[rr][tt] += signed_by(u[c], tv[tt][c]);
    }
  }
  // sums over the wave's lanes (every lane ends with the totals); lane
  // rr * T + tt keeps row rr's total for token tt
  float mine = 0.0f;
#pragma unroll
  for (int rr = 0; rr < kS2RowsPerWave; ++rr)
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      float v = acc[rr][tt];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == rr * T + tt) mine = v;
    }
  const int rr = lane / T, tt = lane % T;
  const int64_t i = i0 + rr;
  const bool owner = lane < kS2RowsPerWave * T && i < d_out;
  if (nsp == 1) {
    if (owner) y[(int64_t)tt * d_out + i] = s1[i] * mine;
    return;
  }
  if (owner) store_agent(part + ((int64_t)sp * T + tt) * d_out + i, mine);
  if (!last_to_arrive(ctr + blockIdx.x, nsp, &s_last)) return;
  if (tid < kS2Rows * T) {
    const int64_t row = (int64_t)blockIdx.x * kS2Rows + tid / T;
    const int tk = tid % T;
    if (row < d_out) {
      float sum = 0.0f;
#pragma unroll 8
      for (int s = 0; s < nsp; ++s) sum += part[((int64_t)s * T + tk) * d_out + row];
      y[(int64_t)tk * d_out + row] = s1[row] * sum;
    }
  }
}

struct LatPlan {
  int ncol, nsp1, span1;  // stage 1: column tiles, row spans, rows per span
  int nrb, nsp2, span2;   // stage 2: row blocks, reduction spans, elements per span
  size_t off_t, off_p1, off_p2, off_c, bytes;
};

LatPlan lat_plan(int64_t d_out, int64_t d_in, int64_t r, int64_t T) {
  LatPlan p;
  p.ncol = (int)cdiv(r, kS1Cols);
  int nsp = (int)imax(1, imin(cdiv(kS1Target, p.ncol), cdiv(d_in, kS1MinSpan)));
  p.span1 = (int)imin(kS1MaxSpan, round_up(cdiv(d_in, nsp), 4));
  p.nsp1 = (int)cdiv(d_in, p.span1);
  p.nrb = (int)cdiv(d_out, kS2Rows);
  // reduction spans: enough workgroups for the chip, each span a whole number
  // of the waves' 256-element steps; a workgroup's work per loaded element
  // grows with T, so fewer are needed (more spans at T = 8 measured 5 % slower)
  const int64_t want2 = imax(1, cdiv(kS2Target / T, p.nrb));
  p.span2 = (int)imin(kS2Span, imax(kS2MinSpan, round_up(cdiv(r, want2), kS2MinSpan)));
  p.nsp2 = (int)cdiv(r, p.span2);
  size_t off = 0;
  p.off_t = off;
  off = align_up(off + (size_t)T * r * sizeof(float));
  p.off_p1 = off;
  off = align_up(off + (p.nsp1 > 1 ? (size_t)p.nsp1 * T * r * sizeof(float) : 0));
  p.off_p2 = off;
  off = align_up(off + (p.nsp2 > 1 ? (size_t)p.nsp2 * T * d_out * sizeof(float) : 0));
  p.off_c = off;
  off = align_up(off + (size_t)(p.ncol + p.nrb) * sizeof(int));
  p.bytes = off;
  return p;
}

template <int T>
hipError_t launch_lat_t(const float* u_lat, int64_t ldu, const float* v_lat, int64_t ldv, int64_t d_out, int64_t d_in,
                        int64_t r, const float* s1, const float* s2, const void* x, bool x_bf16, float* y, char* ws,
                        hipStream_t s) {
  const LatPlan p = lat_plan(d_out, d_in, r, T);
  float* t = reinterpret_cast<float*>(ws + p.off_t);
  float* p1 = reinterpret_cast<float*>(ws + p.off_p1);
  float* p2 = reinterpret_cast<float*>(ws + p.off_p2);
  int* ctr = reinterpret_cast<int*>(ws + p.off_c);
  const int nctr = p.ncol + p.nrb;
  hipLaunchKernelGGL(lat_zero_kernel, dim3((unsigned)imin(cdiv(nctr, 256), 64)), dim3(256), 0, s, ctr, nctr);
  const dim3 g1((unsigned)p.ncol, (unsigned)p.nsp1), g2((unsigned)p.nrb, (unsigned)p.nsp2);
  if (ldv % 4 == 0 && reinterpret_cast<uintptr_t>(v_lat) % 16 == 0)
    hipLaunchKernelGGL((lat_stage1_kernel<T, true>), g1, dim3(kLatThreads), 0, s, v_lat, ldv, d_in, r, x,
                       x_bf16 ? 1 : 0, s2, p.span1, p1, ctr, t);
  else
    hipLaunchKernelGGL((lat_stage1_kernel<T, false>), g1, dim3(kLatThreads), 0, s, v_lat, ldv, d_in, r, x,
                       x_bf16 ? 1 : 0, s2, p.span1, p1, ctr, t);
  if (ldu % 4 == 0 && reinterpret_cast<uintptr_t>(u_lat) % 16 == 0)
    hipLaunchKernelGGL((lat_stage2_kernel<T, true>), g2, dim3(kLatThreads), 0, s, u_lat, ldu, d_out, r, t, s1, p2,
                       ctr + p.ncol, y, p.span2);
  else
    hipLaunchKernelGGL((lat_stage2_kernel<T, false>), g2, dim3(kLatThreads), 0, s, u_lat, ldu, d_out, r, t, s1, p2,
                       ctr + p.ncol, y, p.span2);
  return hipGetLastError();
}

}  // namespace

size_t lat_forward_bytes(int64_t d_out, int64_t d_in, int64_t r, int64_t T) {
  return lat_plan(d_out, d_in, r, T).bytes;
}

bool lat_forward_fits(int64_t d_out, int64_t d_in, int64_t r, int64_t T) {
  const LatPlan p = lat_plan(d_out, d_in, r, T);
  return T >= 1 && T <= kLatMaxT && p.nsp1 <= 65535 && p.nsp2 <= 65535 && p.ncol <= 65535 &&
         (int64_t)p.nrb <= 0x7fffffff;
}

hipError_t launch_lat_forward(const float* u_lat, int64_t ldu, const float* v_lat, int64_t ldv, int64_t d_out,
                              int64_t d_in, int64_t r, const float* s1, const float* s2, const void* x, bool x_bf16,
                              int64_t T, float* y, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  switch (T) {
#define NQ_CASE(TT) \
  case TT: return launch_lat_t<TT>(u_lat, ldu, v_lat, ldv, d_out, d_in, r, s1, s2, x, x_bf16, y, w, s);
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
#undef NQ_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nq
