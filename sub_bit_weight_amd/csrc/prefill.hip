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
// GEMM.  GEMM workgroups are 8 waves over an output tile of 64*MB tokens x 256
// outputs (2 x 4 waves, each 32*MB x 64 as MB x 2 v_mfma_f32_32x32x16_f16
// tiles), stepping through the reduction 64 deep.  A streams into a ring of
// LDS stages with direct global->LDS loads issued several steps ahead; the
// +-1 operand is built in registers straight from the sign words: a 32x32x16
// MFMA lane needs 8 signs of one column, and with the reduction order below
// two signs 16 bits apart become one fp16 pair with a shift and a v_and_or_b32:
//   pair q (0..15) of each 32-element block holds elements (q, q+16);
//   the prep kernel writes A in that interleaved order.
// A GEMM with too few output tiles to fill the chip splits its reduction;
// the partial sums are added in fixed order by the next kernel.
#include "nq_internal.h"

namespace nq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBN = 256, kBK = 64;
constexpr int kWaves = 8;                 // 2 (tokens) x 4 (outputs); each wave owns 64 x 64
constexpr int kThreads = 64 * kWaves;
constexpr int kPrepThreads = 256;
constexpr uint32_t kSignMask = 0x80008000u, kOnePair = 0x3C003C00u;  // fp16 pair: sign bits, +1.0

enum ASrc { kAF32Scaled = 0, kABF16Scaled = 1, kAF32 = 2 };

// Activations of one 32-element block of row m, already multiplied by the
// column scale (zero past K).  Stage 2 may hold `nsplit` partial sums of t,
// added here in split order.
template <int SRC>
__device__ inline void load_block(const void* __restrict__ a, const float* __restrict__ cs, int64_t M, int64_t K,
                                  int nsplit, bool vec, int64_t m, int64_t blk, float (&v)[32]) {
  const int64_t k0 = blk * 32;
  const bool full = vec && k0 + 32 <= K;
  if (SRC == kABF16Scaled && full) {
    const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a) + m * K + k0);
    const float4* sp = reinterpret_cast<const float4*>(cs + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = xp[i];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
      const float4 s0 = sp[2 * i], s1 = sp[2 * i + 1];
      const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(u[j] << 16) * sc[2 * j];
        v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u) * sc[2 * j + 1];
      }
    }
    return;
  }
  if (SRC != kABF16Scaled && full) {
    const float4* base = reinterpret_cast<const float4*>(static_cast<const float*>(a) + m * K + k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 p = base[i];
      v[4 * i] = p.x;
      v[4 * i + 1] = p.y;
      v[4 * i + 2] = p.z;
      v[4 * i + 3] = p.w;
    }
#pragma unroll 1
    for (int sp = 1; sp < nsplit; ++sp) {  // partial sums of a split reduction, in order
      const float4* ps = base + (int64_t)sp * M * K / 4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 p = ps[i];
        v[4 * i] += p.x;
        v[4 * i + 1] += p.y;
        v[4 * i + 2] += p.z;
        v[4 * i + 3] += p.w;
      }
    }
    if (SRC == kAF32Scaled) {
      const float4* sp4 = reinterpret_cast<const float4*>(cs + k0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 c = sp4[i];
        v[4 * i] *= c.x;
        v[4 * i + 1] *= c.y;
        v[4 * i + 2] *= c.z;
        v[4 * i + 3] *= c.w;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {  // ragged tail or unaligned data: element by element
    const int64_t k = k0 + i;
    float x = 0.0f;
    if (k < K) {
      if (SRC == kABF16Scaled) {
        x = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a)[m * K + k] << 16) * cs[k];
      } else {
        for (int sp = 0; sp < nsplit; ++sp) x += static_cast<const float*>(a)[(int64_t)sp * M * K + m * K + k];
        if (SRC == kAF32Scaled) x *= cs[k];
      }
    }
    v[i] = x;
  }
}

// Reduction order within a 32-element block (one sign word) for the two
// operand encodings of the GEMM.
//  * Pair order (fp32 activations): k-slot j holds element j/2 + 16*(j%2).
//  * Rotated order (bf16 activations): k-slot j = 16*sg + 8*h + 2*d + half
//    (sg: which 16-deep step of the word, h: lane half of the 32x32x16 MFMA,
//    d: dword of the lane's operand, half: fp16 within it) holds element
//    (kPos[d] + 16*half + 8*h + 4*sg) mod 32.  The GEMM rotates the sign word
//    right by 8*h + 4*sg and takes bit kPos[d] (and kPos[d]+16) of it: bit 15
//    is the fp16 sign (value -1 or +1), bits 10, 9, 8 turn 1.0 into 0.5, 1.5
//    or 1.25.  So slot j's operand is 1 + c*bit with c = -2, -1/2, +1/2, +1/4,
//    and with A prescaled by f = 1, 4, -4, -8 (exact powers of two) the MFMA
//    sums a*sign + (f - 1)*a per slot; the prep kernel returns the second
//    part, C = sum (f - 1)*a, per row and reduction piece, and the GEMM
//    subtracts it.  One rotation and four v_bitop3_b32 build a 16-deep step's
//    operand instead of four shifts and four v_and_or_b32.
constexpr int kPos[4] = {15, 10, 9, 8};
constexpr int kPre[4] = {1, 4, -4, -8};

__device__ constexpr int rot_element(int j) {
  return (kPos[(j / 2) % 4] + 16 * (j % 2) + 8 * ((j / 8) % 2) + 4 * (j / 16)) % 32;
}

// One workgroup per (token row m, reduction piece sp); the piece covers
// blocks [sp*bps, min((sp+1)*bps, nblk)) of 32 elements.
//   e[sp][m] = E_TOP - exponent(max |a[m][k]| over the piece)  (0 if all zero);
//   E_TOP = 14 puts the maximum in [2^13, 2^14), 11 leaves room for the x8
//   prescale of the rotated order.
//   out[term][m][slot] = fp16 terms of a[m][k]*2^e in the block's slot order
//   (zero past K); fp32 activations get two terms (hi + lo).
//   c[sp][m] = sum over the piece of (f - 1) * (fp16 of a*2^e)  (rotated order).
//   e_next[m] (when not null; one piece, rotated order) = 14 + e - exponent(sum
//   over the row of |fp16 of a*2^e|): the sum bounds every output of the GEMM
//   that takes this operand (one row of t), so 2^e_next puts all of that row
//   below 2^14, the exponent of the next stage's operand written by the GEMM
//   itself (see gemm_kernel, FUSE).
// A thread handles whole 32-element blocks: 16-byte loads when `vec` (rows and
// scales 16-byte aligned), 16 output dwords.  Pieces of up to 256 blocks stay
// in registers between the two passes; longer ones are read twice.
// Convert one 32-element block (values v, already in registers) to its fp16
// terms in the block's slot order and store them; returns the block's part of
// the correction sum (rotated order).
template <bool ROT>
__device__ inline float convert_block(const float (&v)[32], int e, int64_t M, int64_t Kpad, int nt, int64_t m,
                                      int64_t blk, _Float16* __restrict__ out, float& l1) {
  float csum = 0.0f;
  uint32_t hi[16], lo[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    _Float16 h2[2], l2[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = 2 * p + half;
      const float x = ldexpf(v[ROT ? rot_element(j) : p + 16 * half], e);
      const _Float16 hx = (_Float16)x;
      if (ROT) {
        h2[half] = (_Float16)(kPre[p % 4] * (float)hx);
        l2[half] = (_Float16)0.0f;
        csum += (float)(kPre[p % 4] - 1) * (float)hx;
        l1 += fabsf((float)hx);
      } else {
        h2[half] = hx;
        l2[half] = (_Float16)(x - (float)hx);
      }
    }
    hi[p] = (uint32_t)__builtin_bit_cast(uint16_t, h2[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h2[1]) << 16);
    lo[p] = (uint32_t)__builtin_bit_cast(uint16_t, l2[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, l2[1]) << 16);
  }
  uint4* dh = reinterpret_cast<uint4*>(out + m * Kpad + blk * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) dh[i] = make_uint4(hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]);
  if (!ROT && nt == 2) {
    uint4* dl = reinterpret_cast<uint4*>(out + (M + m) * Kpad + blk * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) dl[i] = make_uint4(lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]);
  }
  return csum;
}

// Workgroup-wide reduction (max or sum) in a fixed order.
template <int NW, bool MAX>
__device__ inline float wg_reduce(float x, float* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(x, off);
    x = MAX ? fmaxf(x, o) : x + o;
  }
  if (NW > 1) {
    __syncthreads();  // red may still be read by an earlier reduction
    if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = x;
    __syncthreads();
    x = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) x = MAX ? fmaxf(x, red[w]) : x + red[w];
  }
  return x;
}

template <int SRC, bool ROT, int NTH, int BPT>
__global__ __launch_bounds__(NTH) void prep_kernel(const void* __restrict__ a, const float* __restrict__ cs,
                                                   int64_t M, int64_t K, int64_t Kpad, int nt, int nsum, int vec,
                                                   int bps, _Float16* __restrict__ out, int* __restrict__ e_out,
                                                   float* __restrict__ c_out, int* __restrict__ e_next) {
  constexpr int NW = NTH / 64;
  __shared__ float red[NW];
  const int64_t m = blockIdx.x;
  const int sp = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t nblk = Kpad / 32;
  const int64_t b0 = (int64_t)sp * bps, b1 = imin(b0 + bps, nblk);
  // this thread's blocks: b0 + tid + i*NTH; up to BPT of them stay in registers,
  // longer pieces are read a second time for the conversion
  const bool in_regs = b1 - b0 <= (int64_t)NTH * BPT;
  float v[BPT][32];
  float mx = 0.0f;
  for (int64_t base = b0 + tid; base < b1; base += (int64_t)NTH * BPT) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int64_t blk = base + (int64_t)i * NTH;
      if (blk < b1) load_block<SRC>(a, cs, M, K, nsum, vec != 0, m, blk, v[i]);
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i)
      if (base + (int64_t)i * NTH < b1)
#pragma unroll
        for (int k = 0; k < 32; ++k) mx = fmaxf(mx, fabsf(v[i][k]));
  }
  mx = wg_reduce<NW, true>(mx, red);
  int e = 0;
  if (mx > 0.0f && isfinite(mx)) {
    int ex;
    frexpf(mx, &ex);  // mx = f * 2^ex, f in [0.5, 1)
    e = (ROT ? 11 : 14) - ex;
  }
  if (tid == 0) e_out[(int64_t)sp * M + m] = e;
  float csum = 0.0f, l1 = 0.0f;
  for (int64_t base = b0 + tid; base < b1; base += (int64_t)NTH * BPT) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int64_t blk = base + (int64_t)i * NTH;
      if (blk < b1) {
        if (!in_regs) load_block<SRC>(a, cs, M, K, nsum, vec != 0, m, blk, v[i]);
        csum += convert_block<ROT>(v[i], e, M, Kpad, nt, m, blk, out, l1);
      }
    }
  }
  if (ROT) {
    csum = wg_reduce<NW, false>(csum, red);
    if (tid == 0) c_out[(int64_t)sp * M + m] = csum;
    if (e_next) {
      l1 = wg_reduce<NW, false>(l1, red);
      int en = 0;
      if (l1 > 0.0f && isfinite(l1)) {
        int ex;
        frexpf(l1, &ex);  // l1 = f * 2^ex, f in [0.5, 1): the row's outputs stay below 2^(ex - e)
        en = 14 + e - ex;
      }
      if (tid == 0) e_next[m] = en;
    }
  }
}

// prep_kernel for bf16 activations in the rotated encoding with the row in one
// reduction piece (every entry of a sequence), with coalesced memory access:
// thread tid takes the 8-element chunks tid + i*NTH (i < CPT) of the row, so a
// wave's loads of x and s2 and its stores cover contiguous bytes (the general
// kernel's thread takes whole 32-element blocks, and its 16-byte accesses at a
// 64- or 128-byte lane stride cost the address unit four times the cache-line
// visits).  A block's four chunks sit in four neighbouring threads of one round;
// the values go through LDS in element order and each thread reads back its
// chunk's slots in the rotated order.  Values, exponents, correction sums and
// the next stage's exponent are those of prep_kernel (the sums over the row
// are taken in another order).
template <int NTH, int CPT>
__global__ __launch_bounds__(NTH) void prep_rot_bf16_kernel(const uint16_t* __restrict__ x, const float* __restrict__ cs,
                                                            int64_t M, int64_t K, int64_t Kpad,
                                                            _Float16* __restrict__ out, int* __restrict__ e_out,
                                                            float* __restrict__ c_out, int* __restrict__ e_next) {
  constexpr int NW = NTH / 64;
  __shared__ float red[NW];
  __shared__ uint16_t stage[NTH * 8];  // one round's fp16 values, element order
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nch = Kpad / 8;
  float v[CPT][8];
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t c = tid + (int64_t)i * NTH;
    if (c * 8 < K) {  // K % 8 == 0: a chunk is wholly inside or past the row
      const uint4 w = *reinterpret_cast<const uint4*>(x + m * K + c * 8);
      const float4 s0 = *reinterpret_cast<const float4*>(cs + c * 8);
      const float4 s1 = *reinterpret_cast<const float4*>(cs + c * 8 + 4);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
      const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[i][2 * k] = __uint_as_float(u[k] << 16) * sc[2 * k];
        v[i][2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u) * sc[2 * k + 1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[i][k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(v[i][k]));
  }
  mx = wg_reduce<NW, true>(mx, red);
  int e = 0;
  if (mx > 0.0f && isfinite(mx)) {
    int ex;
    frexpf(mx, &ex);
    e = 11 - ex;  // room for the x8 prescale of the rotated order
  }
  if (tid == 0) e_out[m] = e;
  float csum = 0.0f, l1 = 0.0f;
  const int q = tid % 4;              // this chunk's place in its 32-element block
  const int bt = (tid - q) * 8;       // the block's first element in `stage`
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t c = tid + (int64_t)i * NTH;
    if (i > 0) __syncthreads();  // the previous round's reads are done
#pragma unroll
    for (int k = 0; k < 8; ++k)
      stage[tid * 8 + k] = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(v[i][k], e));
    __syncthreads();
    if (c < nch) {
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        _Float16 h2[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          // slot j = 8q + 2d + half of the block; its pair index j/2 = 4q + d
          const int j = 8 * q + 2 * d + half;
          const float hx = (float)__builtin_bit_cast(_Float16, stage[bt + rot_element(j)]);
          h2[half] = (_Float16)(kPre[d] * hx);
          csum += (float)(kPre[d] - 1) * hx;
          l1 += fabsf(hx);
        }
        o[d] = (uint32_t)__builtin_bit_cast(uint16_t, h2[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h2[1]) << 16);
      }
      *reinterpret_cast<uint4*>(out + m * Kpad + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  csum = wg_reduce<NW, false>(csum, red);
  if (tid == 0) c_out[m] = csum;
  if (e_next) {
    l1 = wg_reduce<NW, false>(l1, red);
    int en = 0;
    if (l1 > 0.0f && isfinite(l1)) {
      int ex;
      frexpf(l1, &ex);
      en = 14 + e - ex;
    }
    if (tid == 0) e_next[m] = en;
  }
}

// +-1 fp16 operand of a 32x32x16 MFMA lane: 8 signs of one column, the pairs
// (b+d, b+d+16) for d = 0..3 of sign word w; fp16 1.0 = 0x3C00, sign bit 15.
// `mask` (0x80008000) and `one` (0x3C003C00) arrive as kernel arguments: held
// in registers they let each dword compile to a shift and one v_and_or_b32
// (a VOP3 operand cannot be a literal).  Plain C is used rather than inline
// asm so the compiler's MFMA hazard tracking sees every VGPR write.
__device__ inline f16x8 signs_f16(uint32_t w, int b, uint32_t mask, uint32_t one) {
  u32x4 v;
#pragma unroll
  for (int d = 0; d < 4; ++d) v[d] = ((w << (15 - b - d)) & mask) | one;
  return __builtin_bit_cast(f16x8, v);
}

// The same operand in the rotated order (see rot_element): rotate the sign
// word right by 8*h + 4*sg, then dword d = (x & (bit kPos[d] | bit kPos[d]+16))
// ^ 1.0 pair, one v_bitop3_b32 each.
__device__ inline f16x8 signs_rot(uint32_t w, uint32_t rot, uint32_t one) {
  const uint32_t x = __builtin_amdgcn_alignbit(w, w, rot);
  u32x4 v;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t mask = __builtin_amdgcn_readfirstlane((1u << kPos[d]) | (1u << (kPos[d] + 16)));
    v[d] = __builtin_amdgcn_bitop3_b32(x, mask, one, (0xF0 & 0xCC) ^ 0xAA);  // (x & mask) ^ one
  }
  return __builtin_bit_cast(f16x8, v);
}

// Workgroup barrier without a memory fence.  __syncthreads() (and any
// workgroup fence) waits for every outstanding global->LDS load of the wave,
// which would drain the loads issued for later pipeline stages.  Here the
// stage being consumed is waited for explicitly (wait_vmcnt) before the
// barrier, and every LDS read of the previous stage has been consumed by an
// MFMA (so has completed) before it; the empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ inline void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// An element of the product operand of the stage-2 epilogue (fp32 or bf16).
__device__ inline float load_prod(const void* p, int bf16, int64_t i) {
  return bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16) : static_cast<const float*>(p)[i];
}
constexpr int kTileRowsFixed = 128;  // output rows per workgroup tile (64 * kTileMB), per product block

// s_waitcnt that waits until at most n vector-memory operations of this wave
// are outstanding (lgkmcnt and expcnt left alone).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup tile BM x kBN x kBK: 8 waves as 2 (rows) x 4 (columns), each wave
// 32*MB rows x 64 columns as MB x 2 v_mfma_f32_32x32x16_f16 tiles.
template <int NT, int MB>
struct Pipe {
  static constexpr int BM = 2 * 32 * MB;                          // tile rows (tokens)
  static constexpr int S = NT == 1 ? 4 : 2;                       // LDS stages
  static constexpr int A_BYTES = NT * BM * kBK * 2;               // A tile(s) of one stage
  static constexpr int B_BYTES = 2 * kBN * 4;                     // 2 sign-word rows x kBN columns
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int ROWS_PER_WAVE = BM / kWaves;               // A rows each wave moves
  static constexpr int A_DMA = NT * ROWS_PER_WAVE / 8;            // 8 rows (1 KiB) per 16-byte DMA
  static constexpr int PER_STAGE = A_DMA + 1;                     // + 1 sign-word DMA instruction
  static constexpr int LDS = S * STAGE_BYTES;
};

// A stage holds NT tiles of BM rows x kBK fp16 (128 bytes per row) written by
// direct global->LDS loads: one instruction moves 64 lanes x 16 bytes = 8 rows.
// The 16-byte chunk c of row r is stored at chunk c ^ ((r >> 1) & 7): any 16
// consecutive rows read at the same logical chunk hit 16 distinct 16-byte bank
// groups, so the 32-row fragment reads below are conflict-free.  The stage's
// sign words follow: word row q (of the tile's two) at [q][kBN columns].
// PROD: the epilogue also takes the column products of ProdEpilogue (a kernel
// of its own, so that the plain GEMM keeps its registers and LDS).
// ROT: A in the rotated encoding (one fp16 term only); otherwise pair order.
// FUSE (stage 1, no split, no column scale): the output is written as the next
// GEMM's A operand instead of fp32: row m times 2^en[m], one fp16 term in pair
// order, row stride kpad_next, zero in columns [N, kpad_next).  en comes from
// the prep kernel's bound, so no value reaches 2^14 and fp16 keeps 2^-11
// relative accuracy for every value above 2^-14 (2^-28 of the bound).
template <int NT, int MB, bool PROD, bool ROT, bool FUSE>
__global__ __launch_bounds__(kThreads, MB == 2 ? 4 : 2) void gemm_kernel(
    const _Float16* __restrict__ A, const int* __restrict__ erow, const float* __restrict__ crow,
    const uint32_t* __restrict__ bits, int64_t ldb,
    int64_t M, int64_t N, int64_t K, int64_t Kpad, int tiles_m, int tiles_n, int nsplit, int kts,
    uint32_t sign_mask, uint32_t one, const float* __restrict__ colscale, float* __restrict__ out,
    const void* __restrict__ pm, int pm_bf16, float* __restrict__ psum, int64_t ldp,
    _Float16* __restrict__ out16, const int* __restrict__ en, int64_t kpad_next) {
  using P = Pipe<NT, MB>;
  static_assert(!ROT || NT == 1, "the rotated encoding takes one fp16 term");
  static_assert(!(FUSE && PROD), "a fused stage-1 output has no column products");
  extern __shared__ __attribute__((aligned(16))) char lds[];  // [S][A tiles | sign words]
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wave / 4, wn = wave % 4;  // wave tile: rows 32*MB*wm .., columns 64*wn ..
  const int l32 = lane % 32, h = lane / 32;

  // XCD-aware tile order: workgroup i runs on XCD i % 8; give each XCD a
  // contiguous range of tiles (N fastest, then M, then the reduction split) so
  // concurrent tiles share A rows in L2.
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles * nsplit + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (t >= ntiles * nsplit) return;
  const int split = t / ntiles, tt = t % ntiles;
  const int64_t m0 = (int64_t)(tt / tiles_n) * P::BM;
  const int64_t n0 = (int64_t)(tt % tiles_n) * kBN;
  const int64_t nwords = cdiv(K, kWordBits);
  // this workgroup's reduction tiles: [kt_base, kt_base + nk) of the 64-deep tiles
  const int kt_base = split * kts;
  const int nk = imin((int)(Kpad / kBK) - kt_base, kts);

  // Per-lane DMA source offsets, fixed over the reduction: A rows past M load
  // row M-1 and sign-word columns past N load column N-1 (neither is stored).
  const int drow = lane / 8, dchunk = lane % 8;
  uint32_t a_off[P::ROWS_PER_WAVE / 8];
#pragma unroll
  for (int j = 0; j < P::ROWS_PER_WAVE / 8; ++j) {
    const int r = wave * P::ROWS_PER_WAVE + j * 8 + drow;
    const int64_t m = imin(m0 + r, M - 1);
    a_off[j] = (uint32_t)((m - m0) * Kpad + ((dchunk ^ ((r >> 1) & 7)) * 8));
  }
  const uint32_t b_off = (uint32_t)imin(n0 + wn * 64 + lane, N - 1);
  const _Float16* a_tile = A + m0 * Kpad;

  // Every global read is a direct global->LDS load, so no register waits on a
  // global load and the explicit vmcnt waits below are the only ones.  A stage
  // is exactly PER_STAGE such instructions per wave.  Sign-word rows past the
  // last are clamped: they only ever meet zero-padded A columns.
  auto issue = [&](int ktl, int st) {
    const int kt = kt_base + ktl;
    char* stage = lds + st * P::STAGE_BYTES;
#pragma unroll
    for (int term = 0; term < NT; ++term) {
      const _Float16* base = a_tile + (int64_t)term * M * Kpad + (int64_t)kt * kBK;
#pragma unroll
      for (int j = 0; j < P::ROWS_PER_WAVE / 8; ++j) {
        char* dst = stage + (term * P::BM + wave * P::ROWS_PER_WAVE + j * 8) * 128;
        __builtin_amdgcn_global_load_lds((const void*)(base + a_off[j]), (__attribute__((address_space(3))) void*)dst, 16,
                                         0, 0);
      }
    }
    const int64_t kw = imin((int64_t)kt * 2 + wm, nwords - 1);
    char* dst = stage + P::A_BYTES + (wm * kBN + wn * 64) * 4;
    __builtin_amdgcn_global_load_lds((const void*)(bits + kw * ldb + b_off), (__attribute__((address_space(3))) void*)dst,
                                     4, 0, 0);
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int kt = 0; kt < P::S - 1; ++kt)
    if (kt < nk) issue(kt, kt);

  asm volatile("" : "+v"(one));  // keep `one` in a VGPR: one SGPR operand per VOP3 (sign_mask)

  // lane offsets of the A fragments for the four 16-deep steps of a tile
  uint32_t frag_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    frag_off[s] = (uint32_t)((wm * 32 * MB + l32) * 128 + (((4 * (s / 2) + 2 * (s % 2) + h) ^ ((l32 >> 1) & 7)) * 16));

  // the ring index is kept compile-time (kt = kt0 + st, st < S)
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
      stage_barrier();  // every wave's DMA for stage kt landed; stage kt-1 fully consumed
      if (kt + P::S - 1 < nk) issue(kt + P::S - 1, (st + P::S - 1) % P::S);

      // 16-deep MFMA steps within the 64-deep tile, one fp16 term at a time
      // (j = NT*step + term), software-pipelined by hand: the A fragments of
      // j+1 are read from LDS and the +-1 operands of the next step are built
      // between the MFMAs of j (scheduling-group barriers fix the interleave:
      // one MFMA, one fragment read, a share of the sign expansion).
      const char* stage = lds + st * P::STAGE_BYTES;
      const uint32_t* bws = reinterpret_cast<const uint32_t*>(stage + P::A_BYTES) + wn * 64 + l32;
      uint32_t words[2][2];  // [q][nb]: this lane's sign words of the tile
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) words[q][nb] = bws[q * kBN + nb * 32];
      f16x8 af[2][MB];
      auto read_a = [&](int j, f16x8 (&dst)[MB]) {
        const int s = j / NT, term = j % NT;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          dst[mb] = *reinterpret_cast<const f16x8*>(stage + frag_off[s] + (term * P::BM + mb * 32) * 128);
      };
      auto build_b = [&](int s, f16x8 (&dst)[2]) {
        const int q = s / 2;
        if constexpr (ROT) {
          const uint32_t rot = 8 * h + 4 * (s % 2);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) dst[nb] = signs_rot(words[q][nb], rot, one);
        } else {
          const int b = 8 * (s % 2) + 4 * h;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) dst[nb] = signs_f16(words[q][nb], b, sign_mask, one);
        }
      };
      read_a(0, af[0]);
      f16x8 bf[2][2];
      build_b(0, bf[0]);
#pragma unroll
      for (int j = 0; j < 4 * NT; ++j) {
        const int s = j / NT;
        __builtin_amdgcn_sched_barrier(0);
        const bool rd = j + 1 < 4 * NT, bld = j % NT == NT - 1 && s + 1 < 4;
        if (rd) read_a(j + 1, af[(j + 1) & 1]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][mb], bf[s & 1][nb], acc[mb][nb], 0, 0, 0);
        if (bld) build_b(s + 1, bf[(s + 1) & 1]);
        // one MFMA, then (first MB of them) one A-fragment read, then a share of
        // the sign expansion for the next step
#pragma unroll
        for (int i = 0; i < 2 * MB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (rd && i < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (bld) __builtin_amdgcn_sched_group_barrier(0x002, 16 / (2 * MB), 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // 32x32 MFMA result layout: lane l, register 4a+c -> row 8a + 4(l/32) + c, column l%32.
  // A split reduction writes its partial sums to out[split] (colscale is then
  // applied by whoever adds the partials).
  // Exponents (and, in the rotated encoding, the correction sums) are per
  // reduction piece and row.
  // With psum (only without a split), each column's products pm * v over the
  // tile's rows are summed: per lane over its 16 rows of each 32-row block in
  // order, then the two lane halves, then the two wave rows through LDS.
  const int* ep = erow + (int64_t)split * M;
  const float* cp = crow + (int64_t)split * M;
  if constexpr (FUSE) {
    // column n is element l32 of its 32-element block, pair-order slot
    // 2*(l32 % 16) + l32/16; lanes l32 = 0..31 of a row write one 64-byte run
    const int slot = 2 * (l32 % 16) + l32 / 16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int64_t n = n0 + wn * 64 + nb * 32 + l32;
        if (n >= kpad_next) continue;
        const int64_t col = n - l32 + slot;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int64_t m = m0 + wm * 32 * MB + mb * 32 + 8 * a + 4 * h + c;
            if (m < M) {
              const float v = ROT ? acc[mb][nb][4 * a + c] - cp[m] : acc[mb][nb][4 * a + c];
              out16[m * kpad_next + col] = n < N ? (_Float16)ldexpf(v, en[m] - ep[m]) : (_Float16)0.0f;
            }
          }
      }
    return;
  }
  float* dst = (!PROD || out) ? out + (int64_t)split * M * N : nullptr;
  float colsum[2] = {0.0f, 0.0f};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t n = n0 + wn * 64 + nb * 32 + l32;
      const float sc = (n < N && colscale) ? colscale[n] : 1.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t m = m0 + wm * 32 * MB + mb * 32 + 8 * a + 4 * h + c;
          if (m < M && n < N) {
            const float v = ldexpf(ROT ? acc[mb][nb][4 * a + c] - cp[m] : acc[mb][nb][4 * a + c], -ep[m]);
            if (!PROD || dst) dst[m * N + n] = sc * v;
            if constexpr (PROD) colsum[nb] = fmaf(load_prod(pm, pm_bf16, m * N + n), v, colsum[nb]);
          }
        }
    }
  if constexpr (PROD) {
    __shared__ float s_col[2][kBN];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      colsum[nb] += __shfl_xor(colsum[nb], 32);  // lanes l and l+32 hold rows of one column
      if (h == 0) s_col[wm][wn * 64 + nb * 32 + l32] = colsum[nb];
    }
    __syncthreads();
    if (wm == 0 && h == 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int c = wn * 64 + nb * 32 + l32;
        if (n0 + c < N) psum[(int64_t)(tt / tiles_n) * ldp + n0 + c] = s_col[0][c] + s_col[1][c];
      }
    }
  }
}

// The same outputs and column products when the reduction was split:
// v[m][n] = sum over splits of part[split][m][n] in split order, y[m][n] =
// colscale[n] * v (y may be null), psum[q * ldp + n] = sum over the rows of
// 128-row block q, in order, of pm[m][n] * v.  Grid: (column tiles of 256,
// row blocks).
__global__ __launch_bounds__(256) void split_sum_prod_kernel(const float* __restrict__ part, int nsplit, int64_t M,
                                                             int64_t N, const float* __restrict__ colscale,
                                                             float* __restrict__ y, const void* __restrict__ pm,
                                                             int pm_bf16, float* __restrict__ psum, int64_t ldp) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int64_t MN = M * N;
  const int64_t m0 = (int64_t)blockIdx.y * kTileRowsFixed, m1 = imin(m0 + kTileRowsFixed, M);
  const float sc = colscale ? colscale[n] : 1.0f;
  float acc = 0.0f;
  for (int64_t m = m0; m < m1; ++m) {
    const int64_t i = m * N + n;
    float v = part[i];
    for (int sp = 1; sp < nsplit; ++sp) v += part[(int64_t)sp * MN + i];
    if (y) y[i] = sc * v;
    acc = fmaf(load_prod(pm, pm_bf16, i), v, acc);
  }
  psum[(int64_t)blockIdx.y * ldp + n] = acc;
}

// y[m][n] = colscale[n] * sum over splits of part[split][m][n], in split order
// (colscale may be null: no scale).
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int nsplit, int64_t MN,
                                                        int64_t N, const float* __restrict__ colscale,
                                                        float* __restrict__ y) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += (int64_t)gridDim.x * 256) {
    float acc = part[i];
    for (int sp = 1; sp < nsplit; ++sp) acc += part[(int64_t)sp * MN + i];
    y[i] = colscale ? colscale[i % N] * acc : acc;
  }
}

// Prep of one GEMM operand: grid (rows, reduction pieces); bps = blocks of 32
// per piece.  nt == 1 uses the rotated encoding (with correction sums in c).
template <int SRC>
hipError_t launch_prep(const void* a, const float* cs, int64_t M, int64_t K, int64_t Kpad, int nt, int nsum,
                       int npieces, int bps, _Float16* out, int* e, float* c, hipStream_t s, int* e_next = nullptr) {
  const int esize = SRC == kABF16Scaled ? 2 : 4;
  const int vec = (reinterpret_cast<uintptr_t>(a) % 16 == 0) && (reinterpret_cast<uintptr_t>(cs) % 16 == 0) &&
                  ((K * esize) % 16 == 0);
  const dim3 grid((unsigned)M, (unsigned)npieces);
  if (SRC == kABF16Scaled && nt == 1 && npieces == 1 && vec) {  // coalesced variant, rows up to 32768
    const int64_t nch = Kpad / 8;
#define NQ_PREP_ROT(NTH, CPT)                                                                                 \
  hipLaunchKernelGGL((prep_rot_bf16_kernel<NTH, CPT>), dim3((unsigned)M), dim3(NTH), 0, s,                    \
                     static_cast<const uint16_t*>(a), cs, M, K, Kpad, out, e, c, e_next)
    if (nch <= 256)
      NQ_PREP_ROT(256, 1);
    else if (nch <= 512)
      NQ_PREP_ROT(256, 2);
    else if (nch <= 1024)
      NQ_PREP_ROT(256, 4);
    else if (nch <= 2048)
      NQ_PREP_ROT(256, 8);
    else if (nch <= 4096)
      NQ_PREP_ROT(512, 8);
#undef NQ_PREP_ROT
    if (nch <= 4096) return hipGetLastError();
  }
  // 1 to 8 waves per (row, piece), the fewest that hold the piece in registers
  const int64_t pblk = imin((int64_t)bps, Kpad / 32);
#define NQ_PREP(ROT, NTH, BPT)                                                                                    \
  hipLaunchKernelGGL((prep_kernel<SRC, ROT, NTH, BPT>), grid, dim3(NTH), 0, s, a, cs, M, K, Kpad, nt, nsum, vec, bps, \
                     out, e, c, e_next)
  // bf16 sources: two blocks per thread in registers; fp32 sources (whose
  // loads need more registers): one
  constexpr int BPT = SRC == kABF16Scaled ? 2 : 1;
  if (nt == 1) {
    if (pblk <= 64 * BPT)
      NQ_PREP(true, 64, BPT);
    else if (pblk <= 128 * BPT)
      NQ_PREP(true, 128, BPT);
    else if (pblk <= 256 * BPT)
      NQ_PREP(true, 256, BPT);
    else
      NQ_PREP(true, 512, BPT);
  } else {
    if (pblk <= 64 * BPT)
      NQ_PREP(false, 64, BPT);
    else if (pblk <= 128 * BPT)
      NQ_PREP(false, 128, BPT);
    else if (pblk <= 256 * BPT)
      NQ_PREP(false, 256, BPT);
    else
      NQ_PREP(false, 512, BPT);
  }
#undef NQ_PREP
  return hipGetLastError();
}

// MFMA tiles per wave along the rows.  2: 128 x 256 workgroup tiles, two
// workgroups (16 waves) per CU.  4 (256 x 256, one workgroup of 8 waves per
// CU) halves the sign expansion per MFMA but measured slower on the 70B
// shapes: two waves per SIMD hide too little LDS and barrier latency.
constexpr int kTileMB = 2;
constexpr int kTileRows = 64 * kTileMB;
static_assert(kTileRows == kTileRowsFixed, "product blocks are the GEMM's row tiles");
constexpr int kWgSlots = kTileMB == 2 ? 512 : 256;  // resident workgroups on 256 CUs

// Reduction split of one GEMM: a GEMM with fewer output tiles than resident
// workgroup slots leaves CUs idle; its reduction is then cut into up to
// kMaxSplit pieces of at least kMinSplitTiles 64-deep tiles, the partial sums
// going through the workspace.
constexpr int kMaxSplit = 8, kMinSplitTiles = 4;

struct Split {
  int n;    // number of pieces
  int kts;  // 64-deep reduction tiles per piece
};

Split split_plan(int64_t M, int64_t N, int64_t Kpad, bool allow) {
  const int64_t tiles = cdiv(M, kTileRows) * cdiv(N, kBN);
  const int nk = (int)(Kpad / kBK);
  int n = 1;
  while (allow && n < kMaxSplit && tiles * n * 2 <= kWgSlots && nk / (n * 2) >= kMinSplitTiles) n *= 2;
  const int kts = (int)cdiv(nk, n);
  return {(int)cdiv(nk, kts), kts};
}

// A fused stage-1 output (gemm_kernel, FUSE): the next GEMM's operand, its
// row exponents and its row stride.
struct FuseOut {
  _Float16* out16;
  const int* en;
  int64_t kpad;
};

template <int NT, int MB, bool PROD, bool ROT, bool FUSE>
hipError_t launch_gemm_t(const _Float16* A, const int* e, const float* c, const uint32_t* bits, int64_t ldb, int64_t M,
                         int64_t N, int64_t K, int64_t Kpad, Split sp, const float* colscale, float* out,
                         const ProdEpilogue* pe, const FuseOut* fo, hipStream_t s) {
  using P = Pipe<NT, MB>;
  const auto kernel = gemm_kernel<NT, MB, PROD, ROT, FUSE>;
  static bool configured = false;
  if (!configured) {
    const hipError_t err =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, P::LDS);
    if (err != hipSuccess) return err;
    configured = true;
  }
  const int tiles_m = (int)cdiv(M, P::BM), tiles_n = (int)cdiv(N, kBN);
  const unsigned grid = (unsigned)(8 * ((tiles_m * tiles_n * sp.n + 7) / 8));
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), P::LDS, s, A, e, c, bits, ldb, M, N, K, Kpad, tiles_m,
                     tiles_n, sp.n, sp.kts, kSignMask, kOnePair, colscale, out, pe ? pe->pm : nullptr,
                     pe ? (int)pe->pm_bf16 : 0, pe ? pe->psum : nullptr, pe ? pe->ldp : (int64_t)0,
                     fo ? fo->out16 : nullptr, fo ? fo->en : nullptr, fo ? fo->kpad : (int64_t)0);
  return hipGetLastError();
}

// nt fp16 terms of A (2: pair order); with nt == 1, rot selects the rotated
// encoding (A from a prep kernel) or pair order (A from a fused stage 1).
hipError_t launch_gemm(int nt, bool rot, const _Float16* A, const int* e, const float* c, const uint32_t* bits,
                       int64_t ldb, int64_t M, int64_t N, int64_t K, int64_t Kpad, Split sp, const float* colscale,
                       float* out, hipStream_t s, const ProdEpilogue* pe = nullptr, const FuseOut* fo = nullptr) {
  constexpr int MB = kTileMB;
#define NQ_GEMM(NT, PROD, ROT, FUSE) \
  launch_gemm_t<NT, MB, PROD, ROT, FUSE>(A, e, c, bits, ldb, M, N, K, Kpad, sp, colscale, out, pe, fo, s)
  if (fo) return rot ? NQ_GEMM(1, false, true, true) : hipErrorInvalidValue;  // stage 1 of bf16 activations
  if (nt == 2) return pe ? NQ_GEMM(2, true, false, false) : NQ_GEMM(2, false, false, false);
  if (rot) return pe ? NQ_GEMM(1, true, true, false) : NQ_GEMM(1, false, true, false);
  return pe ? NQ_GEMM(1, true, false, false) : NQ_GEMM(1, false, false, false);
#undef NQ_GEMM
}

struct PrefillLayout {
  int nt;
  int64_t kpad1, kpad2;
  Split sp1, sp2;
  size_t off_z, off_e1, off_c1, off_t, off_t16, off_e2, off_c2, off_y2, total;
};

// Workspace: fp16 terms of stage 1's activations, their exponents and
// correction sums (per reduction piece and row), t (one copy per reduction
// piece of stage 1), the same three for t, and the partial outputs of stage 2
// when its reduction is split.
PrefillLayout prefill_layout(const nq_lrb& L, int64_t T, nq_dtype xd, bool split) {
  PrefillLayout d;
  d.nt = xd == NQ_F32 ? 2 : 1;
  d.kpad1 = round_up(L.d_in, kBK);
  d.kpad2 = round_up(L.r, kBK);
  d.sp1 = split_plan(T, L.r, d.kpad1, split);
  d.sp2 = split_plan(T, L.d_out, d.kpad2, split);
  size_t off = 0;
  d.off_z = off;
  off = align_up(off + (size_t)d.nt * T * d.kpad1 * sizeof(_Float16));
  d.off_e1 = off;
  off = align_up(off + (size_t)d.sp1.n * T * sizeof(int));
  d.off_c1 = off;
  off = align_up(off + (size_t)d.sp1.n * T * sizeof(float));
  d.off_t = off;
  off = align_up(off + (size_t)d.sp1.n * T * L.r * sizeof(float));
  d.off_t16 = off;
  off = align_up(off + (size_t)d.nt * T * d.kpad2 * sizeof(_Float16));
  d.off_e2 = off;
  off = align_up(off + (size_t)d.sp2.n * T * sizeof(int));
  d.off_c2 = off;
  off = align_up(off + (size_t)d.sp2.n * T * sizeof(float));
  d.off_y2 = off;
  if (d.sp2.n > 1) off = align_up(off + (size_t)d.sp2.n * T * L.d_out * sizeof(float));
  d.total = off;
  return d;
}

}  // namespace

size_t prefill_workspace_bytes(const nq_lrb& L, int64_t T, bool split) {
  // sized for the larger (fp32 activation) plan so one size serves both dtypes
  return prefill_layout(L, T, NQ_F32, split).total;
}

int64_t prefill_row_blocks(int64_t T) { return cdiv(T, kTileRows); }

hipError_t launch_prefill(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                          hipStream_t s, bool split, const ProdEpilogue* pe) {
  const PrefillLayout d = prefill_layout(L, T, xd, split);
  char* base = static_cast<char*>(ws);
  _Float16* z = reinterpret_cast<_Float16*>(base + d.off_z);
  int* e1 = reinterpret_cast<int*>(base + d.off_e1);
  float* c1 = reinterpret_cast<float*>(base + d.off_c1);
  float* t = reinterpret_cast<float*>(base + d.off_t);
  _Float16* t16 = reinterpret_cast<_Float16*>(base + d.off_t16);
  int* e2 = reinterpret_cast<int*>(base + d.off_e2);
  float* c2 = reinterpret_cast<float*>(base + d.off_c2);
  float* y2 = reinterpret_cast<float*>(base + d.off_y2);
  const int bps1 = 2 * d.sp1.kts, bps2 = 2 * d.sp2.kts;  // 32-element blocks per reduction piece
  hipError_t e;
  // bf16 activations with neither reduction split: stage 1 writes stage 2's
  // fp16 operand itself (row exponents from the stage-1 prep's bound), so t
  // makes no fp32 round trip and has no prep kernel; stage 2 takes pair order
  const bool fuse = xd == NQ_BF16 && d.sp1.n == 1 && d.sp2.n == 1;
  if (xd == NQ_BF16)
    e = launch_prep<kABF16Scaled>(x, L.s2, T, L.d_in, d.kpad1, d.nt, 1, d.sp1.n, bps1, z, e1, c1, s,
                                  fuse ? e2 : nullptr);
  else
    e = launch_prep<kAF32Scaled>(x, L.s2, T, L.d_in, d.kpad1, d.nt, 1, d.sp1.n, bps1, z, e1, c1, s);
  if (e != hipSuccess) return e;
  if (fuse) {
    const FuseOut fo{t16, e2, d.kpad2};
    if ((e = launch_gemm(1, true, z, e1, c1, L.vt_bits, L.ldv, T, L.r, L.d_in, d.kpad1, d.sp1, nullptr, nullptr, s,
                         nullptr, &fo)) != hipSuccess)
      return e;
    return launch_gemm(1, false, t16, e2, c2, L.u_bits, L.ldu, T, L.d_out, L.r, d.kpad2, d.sp2, L.s1, y, s, pe);
  }
  const bool rot = d.nt == 1;
  if ((e = launch_gemm(d.nt, rot, z, e1, c1, L.vt_bits, L.ldv, T, L.r, L.d_in, d.kpad1, d.sp1, nullptr, t, s)) !=
      hipSuccess)
    return e;
  // the stage-2 prep adds stage 1's partial sums while it reads t
  if ((e = launch_prep<kAF32>(t, nullptr, T, L.r, d.kpad2, d.nt, d.sp1.n, d.sp2.n, bps2, t16, e2, c2, s)) !=
      hipSuccess)
    return e;
  if (d.sp2.n == 1)
    return launch_gemm(d.nt, rot, t16, e2, c2, L.u_bits, L.ldu, T, L.d_out, L.r, d.kpad2, d.sp2, L.s1, y, s, pe);
  if ((e = launch_gemm(d.nt, rot, t16, e2, c2, L.u_bits, L.ldu, T, L.d_out, L.r, d.kpad2, d.sp2, nullptr, y2, s)) !=
      hipSuccess)
    return e;
  if (pe) {
    const dim3 grid((unsigned)cdiv(L.d_out, 256), (unsigned)cdiv(T, kTileRows));
    hipLaunchKernelGGL(split_sum_prod_kernel, grid, dim3(256), 0, s, y2, d.sp2.n, T, L.d_out, L.s1, y, pe->pm,
                       (int)pe->pm_bf16, pe->psum, pe->ldp);
    return hipGetLastError();
  }
  const int64_t MN = T * L.d_out;
  const unsigned grid = (unsigned)imin(cdiv(MN, 256), (int64_t)4096);
  hipLaunchKernelGGL(split_sum_kernel, dim3(grid), dim3(256), 0, s, y2, d.sp2.n, MN, L.d_out, L.s1, y);
  return hipGetLastError();
}

}  // namespace nq
