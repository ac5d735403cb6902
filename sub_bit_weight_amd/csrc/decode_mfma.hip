// Decode regime (T <= 8): matrix-core tiles for the low-rank binary linear.
//
// The layer is evaluated in factored form, stage 1 t = V^T (s2 (.) x) and
// stage 2 y = s1 (.) (U t) (research.samsung.com NanoQuant blog, section 2,
// subsection "Low-Rank Binary Factorization", the factorization equation; the
// GEMV regime for token-by-token decoding is section 4, "Inference
// Performance").  Both stages have the form
//     out[t][o] = sum_e sign(o,e) * v[t][e],   sign from words[e/32][o] bit e%32.
// The regime is bound by the sign-word bytes streamed from HBM.
//
// Structure:
//  * A tile is a block of 512 output rows over a reduction span (single calls
//    split the reduction; sequences give a tile the whole reduction).  Partial
//    sums of split spans go to the workspace; the last span of a row block to
//    finish (arrival counter) adds them in span order, so results are
//    deterministic, then applies s1 for stage 2.
//  * Each stage input is first cut into fp8 pieces by input-piece tiles; the
//    row-block tiles multiply fp4 +-1 sign operands by those pieces on the
//    matrix cores (details before mfma_tile below).
//  * A persistent kernel runs a whole sequence of linears from one launch:
//    tiles are taken in schedule order from an atomic counter, and a tile
//    whose input is produced by other tiles first waits for them.  Waits only
//    target earlier tiles, which are already running, so the queue always
//    drains; each wait also has a spin limit that records an error and exits.
#include "nq_internal.h"

namespace nq {

namespace {

constexpr unsigned kSpinLimit = 1u << 21;  // ~1 s of polling, then give up and flag


__device__ inline float bf16_bits(uint32_t h) { return __uint_as_float(h << 16); }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Loads through pointers held in a descriptor: tell the compiler they are
// global memory (plain global_load, not flat).
template <typename V>
__device__ inline V gload(const V* p) {
  typedef const __attribute__((address_space(1))) V* gptr;
  return *(gptr)(p);
}

template <typename V>
__device__ inline void gstore(V* p, V v) {
  typedef __attribute__((address_space(1))) V* gptr;
  *(gptr)p = v;
}
// Counter accesses through global (not flat) instructions: a pending flat
// access makes the compiler wait for every outstanding load at the next
// s_waitcnt, as flat accesses may complete out of order.
__device__ inline int load_relaxed(const int* p) {
  typedef const __attribute__((address_space(1))) int* gptr;
  return __hip_atomic_load((gptr)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int add_relaxed(int* p, int v) {
  typedef __attribute__((address_space(1))) int* gptr;
  return __hip_atomic_fetch_add((gptr)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void or_relaxed(int* p, int v) {
  typedef __attribute__((address_space(1))) int* gptr;
  __hip_atomic_fetch_or((gptr)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Values that other workgroups read during the same launch (partial sums and
// the stage-1 result t) are written with agent-scope stores (sc1).  Such a
// store writes through to the device coherence point by itself, so once every
// thread's stores have completed (vmcnt 0) and the workgroup has met at a
// barrier, a relaxed counter increment hands them over; the readers still
// acquire (invalidate) before reading.  An agent-scope release fence would
// instead write back every dirty line of the XCD's L2 on each tile.
__device__ inline void store_agent(float* p, float v) {
  typedef __attribute__((address_space(1))) float* gptr;
  __hip_atomic_store((gptr)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this thread's stores have completed, then meet the workgroup.
__device__ inline void stores_done_barrier() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  __syncthreads();
}

// Sign words are read with buffer loads: the word row's byte offset is a scalar
// (uniform) operand and the lane's column a 32-bit vector offset, so a load
// costs no vector ALU work.  Sign-word buffers are below 2 GiB (checked by the
// host), so both offsets fit.
// Sign words are read once: their loads carry the non-temporal hint (cache
// policy bit 1, "nt"), so they do not push the input pieces, which every row
// block re-reads, out of the L2 (measured: 5.3 -> 5.6 TB/s on the 70B stack).
constexpr int kStreamLoad = 2;
constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past every sign-word buffer (< 2 GiB)

// A tile whose input is made by other tiles of the same launch (a stage by
// its input-piece tiles, the pieces of t by the stage-1 row blocks) waits
// until their counter reaches its target.  Thread 0 polls with relaxed loads
// (an acquire per poll would invalidate caches that streaming workgroups are
// using), then acquires once; the barrier releases the workgroup.
__device__ inline void wait_input(const StageDesc& S, int* err) {
  if (!S.wait_ctr) return;
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (load_relaxed(S.wait_ctr) < S.wait_target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        if (err) or_relaxed(err, 1);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// End of a tile, one output row per thread (acc[t] = this tile's sum for row o,
// token t): store the row (times the row scale), or publish the span's partial
// sums and let the last span of the row block add them in span order.  Every
// thread of the workgroup must call it; it ends with a barrier.
template <int T>
__device__ void finish_rows(const StageDesc& S, int rb, int ks, int64_t o, bool valid, const float* acc, int* s_flag) {
  const int tid = threadIdx.x;
  if (S.nks == 1) {
    if (valid) {
      const float sc = S.rowscale ? gload(S.rowscale + o) : 1.0f;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float* dst = S.out + (int64_t)t * S.n_rows + o;
        if (S.signal)
          store_agent(dst, sc * acc[t]);
        else
          gstore(dst, sc * acc[t]);
      }
    }
  } else {
    if (valid) {
#pragma unroll
      for (int t = 0; t < T; ++t) store_agent(S.part + ((int64_t)ks * T + t) * S.n_rows + o, acc[t]);
    }
    stores_done_barrier();  // this workgroup's partial sums are at the coherence point
    if (tid == 0) {
      *s_flag = (add_relaxed(S.rb_count + rb, 1) == S.nks - 1);
      if (*s_flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // see the other spans' sums
    }
    __syncthreads();
    if (!*s_flag) {
      __syncthreads();  // s_flag is reused by the next tile
      return;
    }
    if (valid) {
      const float sc = S.rowscale ? gload(S.rowscale + o) : 1.0f;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float sum = 0.0f;
        for (int c = 0; c < S.nks; ++c) sum += gload(S.part + ((int64_t)c * T + t) * S.n_rows + o);
        float* dst = S.out + (int64_t)t * S.n_rows + o;
        if (S.signal)
          store_agent(dst, sc * sum);
        else
          gstore(dst, sc * sum);
      }
    }
    if (tid == 0) gstore(S.rb_count + rb, 0);  // all arrivals happened: ready for the next run
  }
  if (S.signal) {
    stores_done_barrier();  // the final row block is at the coherence point
    if (tid == 0) add_relaxed(S.signal, 1);
  }
  __syncthreads();
}


// ------------------------------------------------------- matrix-core tiles
//
// Evaluating the sign sums on the vector ALU costs an instruction or more per
// weight bit, several times what HBM delivers per instruction slot (and table
// lookups per 4-bit nibble are bound by the LDS instruction rate).  These
// tiles run the sign matrix through the matrix cores instead:
//  * A sign word becomes four dwords of fp4 (e2m1) values: dword j holds, in
//    nibble i, element 4i+3-j as +1.0 (0x2) or -1.0 (0xA): the word doubled j
//    times, masked to bit 3 of every nibble, ORed with 0x2 in every nibble.
//    That is eleven full-rate VALU operations per word.
//  * The inputs v = colscale (.) x are cut into fp8 (e4m3) pieces:
//    v * 2^s = q0 + q1/16 + q2/256 + ... (each q the round-to-nearest fp8 of
//    the scaled remainder), kPieces per token, each piece a matrix column.
//    2^s brings the chunk's largest |v| into [64, 128), so no piece saturates;
//    five pieces carry v to about 2^-20 of that largest value.
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 (fp4 A, fp8 B; the B scale of a
//    column is the 2^-(s+4p) of its piece) then gives, for 16 rows and 128
//    reduction elements, the signed sums of 16 piece columns (one column
//    group; up to three groups for T <= 8).  Products of +-1 and fp8 values
//    are exact and accumulate in fp32 across the chunks of the span; the
//    pieces of a token are added across lanes at the end of the tile.
// Operand layouts of the 16x16x128 fp4 x fp8 form (measured on the device):
// lane l holds A row l%16, reduction elements 32*(l/16) + [0, 32) as nibbles
// (dword d, nibble i = element 8d+i); B column l%16, elements 16*(l/16) +
// [0, 16) in bytes 0..15 and 64 + 16*(l/16) + [0, 16) in bytes 16..31; C
// column l%16, rows 4*(l/16) + [0, 4).  The expansion above permutes the
// elements within each lane's 32, and the B pieces follow the same order.
//
// The pieces of a stage's input are made once per stage, by input-piece
// tiles (eight chunks of 1024 elements each), and stored in the workspace in
// a compact form (only the 16-byte fragment blocks of the T*kPieces used
// columns); every row-block tile of the stage copies them into LDS chunk by
// chunk.  (Making them in every row-block tile took about a fifth of the
// stream rate: the loads of x and s2, the chunk maxima and the conversions.)
//
// A workgroup covers 512 rows: each of 8 waves 64 rows as four sets of 16, set q
// holding rows 4m + q (m = 0..15) of the wave's 64.  For MFMA step k (128
// elements) lane l reads the words of rows 4*(l%16) + [0, 4) in word row
// 4k + l/16 (one 16-byte load; 16 lanes cover 256 contiguous bytes of a word
// row), and component q feeds the MFMAs of set q.

constexpr int kMfmaMaxT = 8;
constexpr int kMRows = 512;                            // rows per tile = threads per workgroup (8 waves)
constexpr int kPieces = 5;                            // fp8 pieces per token
constexpr int kStepWords = 4;                         // word rows per MFMA step
constexpr int kChunkSteps = 8;                        // steps per staged chunk
constexpr int kChunkWords = kChunkSteps * kStepWords;  // 32 word rows
constexpr int kRingSteps = 8;                         // steps of sign words in flight per lane
static_assert(kChunkSteps % kRingSteps == 0, "ring slots are compile-time within a chunk");
constexpr int kStepInts = 64 * 8;                     // B fragments of one step and MFMA (64 lanes x 32 bytes)
constexpr int kPrepGroups = kMRows / 256;            // chunks per round of an input-piece tile
// B columns are (token t, piece p) -> t*kPieces + p; every 16 of them form
// one MFMA column group (T*kPieces columns: 1 group up to T = 3, 2 up to 6,
// 3 up to 8).
template <int T>
constexpr int col_groups() { return (T * kPieces + 15) / 16; }
// Steps of sign words in flight per lane: with two column groups the ring is
// half as deep, so that two workgroups fit a CU (their registers); the CU
// then keeps as many bytes in flight as one workgroup with the full ring.
template <int T>
constexpr int ring_steps() { return col_groups<T>() == 2 ? kRingSteps / 2 : kRingSteps; }
// LDS of a workgroup, in 4-byte words: [B fragments, two chunk buffers of
// kChunkSteps x col_groups x kStepInts] [chunk scale exponents, two buffers of
// T] [per-chunk maxima of an input-piece tile] [row sums [T][kMRows]]
template <int T>
constexpr int b_ints() { return kChunkSteps * col_groups<T>() * kStepInts; }
template <int T>
constexpr int sig_off() { return 2 * b_ints<T>(); }
template <int T>
constexpr int slot_off() { return sig_off<T>() + 2 * T; }
template <int T>
constexpr int sum_off() { return slot_off<T>() + 2 * kPrepGroups * T; }
template <int T>
constexpr int mfma_lds() { return sum_off<T>() + T * kMRows; }

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int T>
struct MfmaIn {
  uint32_t x[T][4];  // raw bf16 / fp32 bits of this thread's 4 elements
  float cs[4];
};

// This thread's build task within a chunk: word row wr (0..31), dword j of
// the A expansion, half ih of the nibbles: elements 32*wr + 4*(4*ih + k) +
// 3 - j, k = 0..3, i.e. one B dword (4 consecutive reduction positions).
__device__ inline int task_element(int task, int k) {
  const int wr = task >> 3, j = (task >> 1) & 3, ih = task & 1;
  return 32 * wr + 4 * (4 * ih + k) + 3 - j;
}

// Loads of a chunk's inputs.  Elements at or past cend read element `safe`
// (any in-bounds index) and are dropped later, so chunks past the span can be
// loaded too: the loads keep a fixed count and position in the pipeline.
template <int T>
__device__ inline void mfma_load_inputs(const StageDesc& S, int task, int64_t c0, int64_t cend, int64_t safe,
                                        MfmaIn<T>& in) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t e = c0 + task_element(task, k);
    const int64_t ec = e < cend ? e : safe;
    in.cs[k] = S.colscale ? gload(S.colscale + ec) : 1.0f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t idx = (int64_t)t * S.n_red + ec;
      in.x[t][k] = S.x_bf16 ? (uint32_t)gload(static_cast<const uint16_t*>(S.xin) + idx)
                            : gload(static_cast<const uint32_t*>(S.xin) + idx);
    }
  }
}

template <int T>
__device__ inline float mfma_value(const StageDesc& S, const MfmaIn<T>& in, int task, int64_t c0, int64_t cend, int t,
                                  int k) {
  const float x = S.x_bf16 ? bf16_bits(in.x[t][k]) : __uint_as_float(in.x[t][k]);
  return c0 + task_element(task, k) < cend ? x * in.cs[k] : 0.0f;
}

// Largest |v| of the chunk per token into slot[t] (float bits of a
// non-negative value order like unsigned integers; NaN orders above inf).
template <int T>
__device__ inline void mfma_chunk_max(const StageDesc& S, const MfmaIn<T>& in, int task, int64_t c0, int64_t cend,
                                      unsigned* slot) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
    unsigned m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, __float_as_uint(fabsf(mfma_value<T>(S, in, task, c0, cend, t, k))));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) atomicMax(slot + t, m);
  }
}

// Scale exponent s for a chunk maximum (float bits): max * 2^s in [64, 128).
// s is capped at 107 so that the MFMA scale of the last piece, 2^-(s+20),
// stays within the E8M0 range; only chunks whose largest |v| is below 2^-81
// start below 64 and so keep fewer significant bits.  A non-finite maximum
// gives kShiftNaN: the chunk's pieces are NaN.
constexpr int kShiftNaN = 1 << 20;
__device__ inline int chunk_shift(unsigned mbits) {
  const int e = (int)((mbits >> 23) & 0xFF);
  return e == 255 ? kShiftNaN : min(133 - e, 107);
}

// The 16x16x128 fp4 x fp8 MFMA adds each group of 8 consecutive products
// (reduction positions 8m..8m+7) in a window of about 13 binades below the
// group's leading bit, truncating what lies below it (measured on the device:
// 128 + 7 * 1.875*2^-4 comes out 128.765625).  So a piece keeps, per group,
// only values whose exponent is within 7 of the group's largest (their last
// bit then lies inside the window even after the group sum carries 3 binades
// up), and no subnormals; what it leaves stays in the remainder and reaches a
// later piece, scaled by 16 per piece.
// Bytes of four packed e4m3 values with exponent field < lo (1 <= lo <= 15)
// become 0.
__device__ inline int keep_fp8_exponents(int d, int lo) {
  const uint32_t u = (uint32_t)d;
  const uint32_t bias = (uint32_t)(0x80 - 8 * lo) * 0x01010101u;  // bit 7 of (field*8 + bias): field >= lo
  const uint32_t keep = ((u & 0x78787878u) + bias) & 0x80808080u;
  return (int)(u & (keep | (keep - (keep >> 7))));
}
// Largest exponent field among the four bytes of d.
__device__ inline int max_fp8_exponent(int d) {
  const uint32_t u = (uint32_t)d & 0x78787878u;
  return (int)(max(max(u & 0xFFu, (u >> 8) & 0xFFu), max((u >> 16) & 0xFFu, u >> 24)) >> 3);
}

// Compact piece layout of one chunk: 16-byte blocks, block
// ((step*2 + half)*4 + group)*NC + column holds half `half` of the B fragment
// of lane (column % 16) + 16*group in column group column / 16, MFMA step
// `step` (NC = T*kPieces used columns; column t*kPieces + p is piece p of
// token t).
template <int T>
constexpr int chunk_blocks() { return kChunkSteps * 2 * 4 * T * kPieces; }

// One input-piece tile: chunks [kPrepChunks*tile, ...) of the stage input
// (fewer tiles, each with its own latency, fences and barriers, cost less
// than one tile per chunk).  Each group of 256 threads of the workgroup takes
// a chunk per round; per chunk each thread makes one B dword
// (4 consecutive reduction positions) per piece and token; the next round's
// inputs load while the current ones are converted.
constexpr int kPrepChunks = 8;

template <int T>
__device__ void mfma_prep_tile(const StageDesc& S, int tile, float* ldsf, int* err) {
  constexpr int NC = T * kPieces;
  constexpr int64_t kChunkElems = kChunkWords * kWordBits;
  unsigned* slots = reinterpret_cast<unsigned*>(reinterpret_cast<int*>(ldsf) + slot_off<T>());  // [round&1][group][T]
  const int tid = threadIdx.x, half = tid >> 8, task = tid & 255;  // half: this thread's group
  const int ch0 = tile * kPrepChunks;
  const int ch1 = min(ch0 + kPrepChunks, (int)cdiv(S.n_red, kChunkElems));
  wait_input(S, err);
  const int wr = task >> 3, j = (task >> 1) & 3, ih = task & 1;
  const int kk = wr >> 2, gw = wr & 3;
  const int gp = 2 * (gw & 1) + (j >> 1);
  const int64_t task_off = (int64_t)(((kk * 2 + (gw >> 1)) * 4 + gp) * NC) * 4 + 2 * (j & 1) + ih;
  if (tid < 2 * kPrepGroups * T) slots[tid] = 0;
  MfmaIn<T> in, nxt;
  mfma_load_inputs<T>(S, task, (ch0 + half) * kChunkElems, S.n_red, 0, in);
  __syncthreads();
  for (int r0 = ch0, round = 0; r0 < ch1; r0 += kPrepGroups, ++round) {
    const int ch = r0 + half;  // this group's chunk (past ch1: loads clamp, nothing is stored)
    const int64_t c0 = ch * kChunkElems;
    unsigned* slot = slots + ((round & 1) * kPrepGroups + half) * T;
    mfma_chunk_max<T>(S, in, task, c0, S.n_red, slot);
    mfma_load_inputs<T>(S, task, c0 + kPrepGroups * kChunkElems, S.n_red, 0, nxt);  // next round (or none)
    __syncthreads();  // the chunks' maxima are complete
    if (ch < ch1) {   // wave-uniform: a group is 4 whole waves
      uint32_t* dst = S.bfrag + (int64_t)ch * chunk_blocks<T>() * 4 + task_off;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int shift = chunk_shift(slot[t]);
        float r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          r[k] = shift == kShiftNaN ? __int_as_float(0x7FC00000)
                                    : ldexpf(mfma_value<T>(S, in, task, c0, S.n_red, t, k), shift);
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
          int d = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
          d = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], d, true);
          // this dword and the partner thread's (task ^ 1, same wave) form one group of 8
          int emax = max_fp8_exponent(d);
          emax = max(emax, __shfl_xor(emax, 1));
          d = keep_fp8_exponents(d, max(1, emax - 7));
          store_agent(reinterpret_cast<float*>(dst + (t * kPieces + p) * 4), __int_as_float(d));
          if (p + 1 < kPieces) {
            typedef float v2f __attribute__((ext_vector_type(2)));
            const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(d, false);
            const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(d, true);
            r[0] = (r[0] - lo.x) * 16.0f;
            r[1] = (r[1] - lo.y) * 16.0f;
            r[2] = (r[2] - hi.x) * 16.0f;
            r[3] = (r[3] - hi.y) * 16.0f;
          }
        }
        if (task == 0) store_agent(reinterpret_cast<float*>(S.bsig + (int64_t)ch * T + t), __int_as_float(shift));
      }
    }
    __syncthreads();  // every thread has read this round's maxima
    if (task < T) slot[task] = 0;  // reused two rounds on (its maxima come after the next barrier)
    in = nxt;
  }
  if (S.signal) {
    stores_done_barrier();  // the tile's pieces are at the coherence point
    if (tid == 0) add_relaxed(S.signal, 1);
  }
  __syncthreads();  // the slots are reused by the next tile
}

// B columns past the last piece of the last token stay zero for the life of
// the kernel (the chunk copies never write them): clear them once.
template <int T>
__device__ inline void mfma_lds_init(int* lds) {
  constexpr int NC = T * kPieces, G = col_groups<T>();
  if constexpr (NC < 16 * G) {
    // per step and column group, per half: 64 lanes x 4 dwords; lane = column + 16 * lane group
    for (int i = threadIdx.x; i < 2 * b_ints<T>(); i += kMRows) {  // both chunk buffers
      const int lane = (i >> 2) & 63, cg = (i / kStepInts) % G;
      if (16 * cg + (lane & 15) >= NC) lds[i] = 0;
    }
  }
}

// Four fp4 dwords of one sign word (see above).
// x + x as an add (the compiler would turn it into a shift, which issues at
// half the rate of an add on this chip).
__device__ inline uint32_t twice(uint32_t x) {
  uint32_t y;
  asm("v_add_u32_e32 %0, %1, %1" : "=v"(y) : "v"(x));
  return y;
}

__device__ inline v8i expand_word(uint32_t x) {
  const uint32_t x1 = twice(x), x2 = twice(x1), x3 = twice(x2);
  v8i a;
  a[0] = (int)((x & 0x88888888u) | 0x22222222u);
  a[1] = (int)((x1 & 0x88888888u) | 0x22222222u);
  a[2] = (int)((x2 & 0x88888888u) | 0x22222222u);
  a[3] = (int)((x3 & 0x88888888u) | 0x22222222u);
  a[4] = a[5] = a[6] = a[7] = 0;
  return a;
}

// Sum over the 16 lanes of a row of the wavefront (DPP rotations).
__device__ inline float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

// W4: sign words are read 4 rows at a time (16-byte loads); otherwise one
// word per load (row counts or strides that are not multiples of 4).
template <int T, bool W4>
__device__ void mfma_tile(const StageDesc& S, int local, float* ldsf, int* s_flag, int* err) {
  static_assert(T <= kMfmaMaxT, "tokens");
  constexpr int G = col_groups<T>();
  int* lds = reinterpret_cast<int*>(ldsf);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int rb = local % S.nrb;
  const int ks = local / S.nrb;
  const int64_t span0 = (int64_t)ks * S.kc;
  const int64_t span1 = imin(span0 + S.kc, S.n_red);
  const int w0 = __builtin_amdgcn_readfirstlane((int)(span0 / kWordBits));
  const uint32_t ld4 = __builtin_amdgcn_readfirstlane((uint32_t)(S.ld * 4));
  const int nw = (int)cdiv(span1 - span0, kWordBits);
  const int nk = (nw + kStepWords - 1) / kStepWords;
  const int nchunks = (nw + kChunkWords - 1) / kChunkWords;

  // byte offset of this lane's q-th word from word row 4k; rows at or past
  // n_rows (in the last row block) get an offset past any buffer (sign-word
  // buffers are below 2 GiB), so their loads read 0 without memory traffic
  // instead of words of the next word row
  const int row0 = rb * kMRows + wv * 64 + 4 * col;
  const uint32_t voff = 4u * (uint32_t)row0 + (uint32_t)grp * ld4;
  uint32_t qoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) qoff[q] = row0 + q < S.n_rows ? voff + 4u * q : kOutOfRange;
  // Step k reads word row 4k + grp of the span through a buffer resource that
  // starts at word row 4k and ends with row n_rows-1 of the span's last word
  // row: words past the span (a partial last step, steps past the last) or
  // past the last row are out of range and read as 0 without touching memory
  // (with W4, n_rows is a multiple of 4, so a 16-byte load is entirely in or
  // out of range).  Everything but the lane offset is scalar.
  auto load_step = [&](int k, u32x4& dst) {
    const int wb = kStepWords * k;  // from the span start
    const int rows_left = max(nw - wb, 0);
    const uint32_t nrec = rows_left > 0 ? (uint32_t)(rows_left - 1) * ld4 + 4u * (uint32_t)S.n_rows : 0u;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(S.bits) + (int64_t)(w0 + wb) * S.ld, (short)0, (int)nrec, 0x00020000);
    if constexpr (W4) {  // n_rows % 4 == 0: the lane's 4 rows are all valid or all past the end
      dst = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)qoff[0], 0, kStreamLoad));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)qoff[q], 0, kStreamLoad);
    }
  };

  // This thread's compact blocks of a chunk (see mfma_prep_tile) and their
  // LDS places.  Every thread loads NBT blocks (past the chunk's last block:
  // the last one again, written to the row-sum area, unused until the tile's
  // end) and the chunk's scale exponents, so no branch surrounds the
  // loads.  Chunk c+1 is loaded during chunk c and written to the other LDS
  // buffer half-way through it (the loads are then waited for with the sign
  // words issued after them still in flight); one barrier per chunk.  A chunk
  // past the stage's last loads the last one again.
  constexpr int NB = chunk_blocks<T>();
  constexpr int NBT = (NB + kMRows - 1) / kMRows;  // blocks per thread
  constexpr int NC = T * kPieces;
  int lds_at[NBT], blk_at[NBT];
#pragma unroll
  for (int m = 0; m < NBT; ++m) {
    const int bi = tid + m * kMRows;
    const int n = bi % NC, rest = bi / NC;
    const int g = rest % 4, h = (rest / 4) % 2, kk = rest / 8;
    lds_at[m] = bi < NB ? (kk * G + n / 16) * kStepInts + h * 256 + (n % 16 + 16 * g) * 4 : sum_off<T>();
    blk_at[m] = min(bi, NB - 1);
  }
  const int chunk0 = (int)(span0 / (kChunkWords * kWordBits));
  const int last_chunk = (int)((S.n_red - 1) / (kChunkWords * kWordBits));
  const u32x4* bsrc = reinterpret_cast<const u32x4*>(S.bfrag);
  u32x4 blk[NBT];
  int sig;
  auto load_chunk = [&](int ch) {
    ch = min(ch, last_chunk);
#pragma unroll
    for (int m = 0; m < NBT; ++m) blk[m] = gload(bsrc + (int64_t)ch * NB + blk_at[m]);
    sig = gload(S.bsig + (int64_t)ch * T + min(tid, T - 1));
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int m = 0; m < NBT; ++m) *reinterpret_cast<u32x4*>(lds + buf * b_ints<T>() + lds_at[m]) = blk[m];
    // every thread stores (threads past T into the row-sum area, unused until
    // the tile's end), so the compiler cannot move the load into a branch
    // behind later sign-word loads
    lds[tid < T ? sig_off<T>() + buf * T + tid : sum_off<T>() + tid] = sig;
  };
  // the first sign words do not depend on the stage input: in flight while
  // the wait and the first chunk's pieces complete (loads complete in issue
  // order for s_waitcnt, so the acquire and chunk 0's pieces wait for them;
  // issuing them after the wait measured slightly slower)
  constexpr int R = ring_steps<T>();
  u32x4 ring[R];
#pragma unroll
  for (int k = 0; k < R; ++k) load_step(k, ring[k]);
  wait_input(S, err);  // the stage's pieces are final
  load_chunk(chunk0);
  store_chunk(0);
  __syncthreads();  // chunk 0's fragments are in LDS buffer 0

  // the sums of all chunks accumulate in acc: each chunk's B column (token t,
  // piece p) carries the MFMA scale 2^-(s_t + 4p) of that chunk
  v4f acc[4][G];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int cg = 0; cg < G; ++cg) acc[q][cg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    // E8M0 scale of this lane's column in every group (2^0 for columns past
    // the last piece, whose B entries are 0; a NaN chunk has NaN pieces)
    int bscale[G];
#pragma unroll
    for (int cg = 0; cg < G; ++cg) {
      const int n = 16 * cg + col, tc = n / kPieces, pc = n % kPieces;
      const int sg = lds[sig_off<T>() + buf * T + min(tc, T - 1)];
      bscale[cg] = tc < T ? 127 - (sg == kShiftNaN ? 0 : sg) - 4 * pc : 127;
    }
    load_chunk(chunk0 + c + 1);  // next chunk's pieces (or none)

    const u32x4* bfrag = reinterpret_cast<const u32x4*>(lds + buf * b_ints<T>()) + lane;
    // B fragments: with one column group the next step's are read a step ahead;
    // with two, at their own step (the registers a step ahead would cost the
    // second workgroup per CU)
    constexpr bool kAhead = G == 1;
    u32x4 blo[G], bhi[G];
    if constexpr (kAhead) {
#pragma unroll
      for (int cg = 0; cg < G; ++cg) {
        blo[cg] = bfrag[cg * (kStepInts / 4)];
        bhi[cg] = bfrag[cg * (kStepInts / 4) + 64];
      }
    }
#pragma unroll
    for (int kk = 0; kk < kChunkSteps; ++kk) {
      const int k = c * kChunkSteps + kk;
      v8i b[G];
#pragma unroll
      for (int cg = 0; cg < G; ++cg) {
        if constexpr (!kAhead) {
          blo[cg] = bfrag[(kk * G + cg) * (kStepInts / 4)];
          bhi[cg] = bfrag[(kk * G + cg) * (kStepInts / 4) + 64];
        }
        b[cg][0] = (int)blo[cg].x; b[cg][1] = (int)blo[cg].y; b[cg][2] = (int)blo[cg].z; b[cg][3] = (int)blo[cg].w;
        b[cg][4] = (int)bhi[cg].x; b[cg][5] = (int)bhi[cg].y; b[cg][6] = (int)bhi[cg].z; b[cg][7] = (int)bhi[cg].w;
        if (kAhead && kk + 1 < kChunkSteps) {  // next step's fragments (stale past the span; then unused)
          blo[cg] = bfrag[((kk + 1) * G + cg) * (kStepInts / 4)];
          bhi[cg] = bfrag[((kk + 1) * G + cg) * (kStepInts / 4) + 64];
        }
      }
      if (k < nk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v8i a = expand_word(ring[kk % R][q]);
#pragma unroll
          for (int cg = 0; cg < G; ++cg)
            acc[q][cg] =
                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[cg], acc[q][cg], 4, 0, 0, 127, 0, bscale[cg]);
        }
      }
      load_step(k + R, ring[kk % R]);  // past the span: out of range, no memory access
      if (kk == kChunkSteps / 2) store_chunk(buf ^ 1);    // the other buffer was last read in chunk c-1
    }
    __syncthreads();  // chunk c+1's fragments are in LDS; every wave is done with chunk c's
  }

  // add the pieces of each token across the lanes of a row (and the column
  // groups); lane col == 0 of every row group writes its 4 rows of every set
  float* sums = ldsf + sum_off<T>();
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // C row 4*grp + r of set q is row 16*grp + 4r + q of the wave
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float u = 0.0f;
#pragma unroll
        for (int cg = 0; cg < G; ++cg)
          if ((16 * cg + 15) / kPieces >= t && (16 * cg) / kPieces <= t)  // the group holds columns of token t
            u += (16 * cg + col) / kPieces == t ? acc[q][cg][r] : 0.0f;
        v[q] = row16_sum(u);
      }
      if (col == 0)
        *reinterpret_cast<float4*>(sums + t * kMRows + wv * 64 + grp * 16 + 4 * r) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  __syncthreads();
  float accr[T];
#pragma unroll
  for (int t = 0; t < T; ++t) accr[t] = sums[t * kMRows + tid];
  const int64_t o = (int64_t)rb * kMRows + tid;
  finish_rows<T>(S, rb, ks, o, o < S.n_rows, accr, s_flag);
}

// With one or two column groups: 4 waves per SIMD (at most 128 VGPRs) and 2
// workgroups per CU (two groups: a half-deep ring and B fragments read at
// their step make room for the second group's accumulators); with three
// (74-115 KB of LDS) 2 waves per SIMD, one workgroup per CU.
template <int T>
constexpr int min_waves() { return col_groups<T>() <= 2 ? 4 : 2; }

// The workgroup's two shared flag words live in the first entries of LDS (B
// fragments of column 0 in chunk buffer 0): every write to them follows the
// barrier after a tile's last fragment read, and the next tile's first chunk
// copy follows the barrier after their last read.
template <int T>
__device__ inline void stage_tile(const StageDesc& S, int local, float* lds, int* s_flag, int* err) {
  if (S.kind == 1)
    mfma_prep_tile<T>(S, local, lds, err);
  else if (S.w_vec)
    mfma_tile<T, true>(S, local, lds, s_flag, err);
  else
    mfma_tile<T, false>(S, local, lds, s_flag, err);
}

template <int T>
__global__ __launch_bounds__(kMRows) __attribute__((amdgpu_waves_per_eu(min_waves<T>())))
void dec_stage_kernel(StageDesc S, int* err) {
  __shared__ __attribute__((aligned(16))) float lds[mfma_lds<T>()];
  int* s_flag = reinterpret_cast<int*>(lds);
  mfma_lds_init<T>(reinterpret_cast<int*>(lds));
  __syncthreads();
  stage_tile<T>(S, blockIdx.x, lds, s_flag, err);
}

// ints: [0] error flag (sticky), [1] next tile, [2] workgroups exited,
// [3 .. n_ints) per-linear counters.  The last workgroup to exit zeroes
// [1 .. n_ints), so consecutive runs need no separate reset launch.
template <int T>
__global__ __launch_bounds__(kMRows) __attribute__((amdgpu_waves_per_eu(min_waves<T>())))
void dec_persistent_kernel(const StageDesc* __restrict__ segs, const int* __restrict__ tile_seg, int ntiles, int* ints,
                           int n_ints) {
  __shared__ __attribute__((aligned(16))) float lds[mfma_lds<T>()];
  int& s_flag = reinterpret_cast<int*>(lds)[0];  // aliases B fragments (see stage_tile)
  int& s_tile = reinterpret_cast<int*>(lds)[1];
  int* err = ints;
  int* next_tile = ints + 1;
  mfma_lds_init<T>(reinterpret_cast<int*>(lds));
  if (threadIdx.x == 0) s_tile = add_relaxed(next_tile, 1);
  __syncthreads();
  int tile = __builtin_amdgcn_readfirstlane(s_tile);
  while (tile < ntiles) {
    int nxt;  // thread 0's (no initial value: a write would wait for loads in flight)
    if (threadIdx.x == 0) nxt = add_relaxed(next_tile, 1);  // prefetch the next tile id
    const StageDesc S = segs[tile_seg[tile]];  // one lookup (a scan over the segments stalled for microseconds)
    stage_tile<T>(S, tile - S.tile0, lds, &s_flag, err);
    if (threadIdx.x == 0) s_tile = nxt;
    __syncthreads();
    tile = __builtin_amdgcn_readfirstlane(s_tile);
    __syncthreads();
  }
  // every counter access of this workgroup is done: count the exit; the last
  // workgroup out resets the counters for the next run
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    s_flag = atomicAdd(ints + 2, 1) == (int)gridDim.x - 1;
    if (s_flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (s_flag)
    for (int i = 1 + threadIdx.x; i < n_ints; i += blockDim.x) ints[i] = 0;
}

__global__ void zero_ints_kernel(int* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

int64_t dec_tile_rows(int64_t) { return kMRows; }

// Reduction spans per row block: `kspan_max` bounds a span (0 = whole reduction).
StagePlan dec_stage_plan(int64_t n_rows, int64_t n_red, int64_t T, int64_t kspan_max) {
  StagePlan p;
  p.n_rows = n_rows;
  p.n_red = n_red;
  p.nrb = (int)cdiv(n_rows, dec_tile_rows(T));
  const int64_t span = kspan_max > 0 ? imin(kspan_max, n_red) : n_red;
  p.nks = (int)cdiv(n_red, span);
  // balanced spans in whole chunks of input pieces (a span starts at a chunk)
  const int64_t grain = kChunkWords * kWordBits;
  p.kc = (int)round_up(cdiv(n_red, p.nks), grain);
  p.nks = (int)cdiv(n_red, p.kc);
  return p;
}

// Single calls split the reduction until the two stages have enough tiles to
// fill the GPU; sequences keep whole reductions (no partial sums).
int64_t dec_single_span(int64_t n_rows, int64_t n_red, int64_t T) {
  const int64_t nrb = cdiv(n_rows, dec_tile_rows(T));
  const int64_t want = cdiv(512, nrb);
  const int64_t span = round_up(cdiv(n_red, want), 1024);
  return span;
}

hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = imin(cdiv(n, 256), 1024);
  hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_dec_stage(const StageDesc& S, int64_t T, int* err, hipStream_t s) {
  const unsigned grid = (unsigned)(S.nrb * S.nks);
  switch (T) {
#define NQ_CASE(TT) \
  case TT: hipLaunchKernelGGL(dec_stage_kernel<TT>, dim3(grid), dim3(kMRows), 0, s, S, err); break;
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
#undef NQ_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int dec_persistent_grid(int64_t T) {
  int dev = 0, cus = 256, per = 1;
  if (hipGetDevice(&dev) == hipSuccess) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  hipError_t e = hipErrorInvalidValue;
  switch (T) {
#define NQ_CASE(TT) \
  case TT: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, dec_persistent_kernel<TT>, kMRows, 0); break;
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
#undef NQ_CASE
  }
  if (e != hipSuccess || per < 1) per = 1;
  return cus * per;
}

hipError_t launch_dec_persistent(const StageDesc* segs, const int* tile_seg, int ntiles, int* ints, int n_ints,
                                 int64_t T, int grid, hipStream_t s) {
  switch (T) {
#define NQ_CASE(TT)                                                                                     \
  case TT:                                                                                              \
    hipLaunchKernelGGL(dec_persistent_kernel<TT>, dim3(grid), dim3(kMRows), 0, s, segs, tile_seg, ntiles, \
                       ints, n_ints);                                                                   \
    break;
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
#undef NQ_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ layouts

namespace {

// Sequences give each tile its row block's whole reduction: no partial sums
// and one release per row block.  (Capping the span at 8K or 16K elements to
// shorten the longest tiles measured slower: the extra fixups cost more than
// the shorter dependency waits they buy.)
constexpr int64_t kSeqSpan = 0;

void plans(const nq_lrb& L, int64_t T, bool split, StagePlan* p1, StagePlan* p2) {
  *p1 = dec_stage_plan(L.r, L.d_in, T, split ? dec_single_span(L.r, L.d_in, T) : kSeqSpan);
  *p2 = dec_stage_plan(L.d_out, L.r, T, split ? dec_single_span(L.d_out, L.r, T) : kSeqSpan);
}

size_t part_bytes(const StagePlan& p, int64_t T) {
  return p.nks > 1 ? (size_t)p.nks * T * p.n_rows * sizeof(float) : 0;
}

}  // namespace

namespace {

// Matrix-core pieces of a stage input of n_red elements: compact blocks and
// per-chunk scale exponents.
int64_t piece_chunks(int64_t n_red) { return cdiv(n_red, kChunkWords * kWordBits); }
size_t piece_bytes(int64_t n_red, int64_t T) {
  const int64_t nch = piece_chunks(n_red);
  return align_up((size_t)nch * 64 * T * kPieces * 16) + align_up((size_t)nch * T * sizeof(int));
}

}  // namespace

// Per-linear device buffers: [part1][t][part2][pieces of x][pieces of t].
size_t dec_linear_bytes(const nq_lrb& L, int64_t T, bool split) {
  StagePlan p1, p2;
  plans(L, T, split, &p1, &p2);
  size_t off = align_up(part_bytes(p1, T));
  off = align_up(off + (size_t)T * L.r * sizeof(float));
  off = align_up(off + part_bytes(p2, T));
  return off + piece_bytes(L.d_in, T) + piece_bytes(L.r, T);
}

// Per-linear counters: [stage-1 row blocks][stage-2 row blocks][t ready]
// [pieces of x ready][pieces of t ready].
int dec_linear_counters(const nq_lrb& L, int64_t T, bool split) {
  StagePlan p1, p2;
  plans(L, T, split, &p1, &p2);
  return p1.nrb + p2.nrb + 3;
}


// Sign words of a stage can be read 4 rows at a time (16-byte loads).
bool words_vec(const uint32_t* bits, int64_t ld, int64_t n_rows) {
  return reinterpret_cast<uintptr_t>(bits) % 16 == 0 && ld % 4 == 0 && n_rows % 4 == 0;
}

int dec_stage_descs(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, bool split,
                    char* ws_linear, int* ctr_base, StageDesc* d) {
  StagePlan p1, p2;
  plans(L, T, split, &p1, &p2);
  size_t off = 0;
  float* part1 = reinterpret_cast<float*>(ws_linear + off);
  off = align_up(off + part_bytes(p1, T));
  float* tbuf = reinterpret_cast<float*>(ws_linear + off);
  off = align_up(off + (size_t)T * L.r * sizeof(float));
  float* part2 = reinterpret_cast<float*>(ws_linear + off);
  off = align_up(off + part_bytes(p2, T));
  char* pieces1 = ws_linear + off;
  off += piece_bytes(L.d_in, T);
  char* pieces2 = ws_linear + off;
  int* t_ready = ctr_base + p1.nrb + p2.nrb;

  StageDesc a{};
  a.bits = L.vt_bits;
  a.ld = L.ldv;
  a.xin = x;
  a.colscale = L.s2;
  a.rowscale = nullptr;
  a.out = tbuf;
  a.part = part1;
  a.rb_count = ctr_base;
  a.signal = t_ready;
  a.wait_ctr = nullptr;
  a.wait_target = 0;
  a.n_rows = (int)L.r;
  a.n_red = (int)L.d_in;
  a.kc = p1.kc;
  a.nks = p1.nks;
  a.nrb = p1.nrb;
  a.x_bf16 = xd == NQ_BF16;
  a.w_vec = words_vec(L.vt_bits, L.ldv, L.r);
  a.kind = 0;
  a.tile0 = 0;
  StageDesc b = a;
  b.bits = L.u_bits;
  b.ld = L.ldu;
  b.xin = tbuf;
  b.colscale = nullptr;
  b.rowscale = L.s1;
  b.out = y;
  b.part = part2;
  b.rb_count = ctr_base + p1.nrb;
  b.signal = nullptr;
  b.wait_ctr = t_ready;
  b.wait_target = p1.nrb;
  b.n_rows = (int)L.d_out;
  b.n_red = (int)L.r;
  b.kc = p2.kc;
  b.nks = p2.nks;
  b.nrb = p2.nrb;
  b.x_bf16 = 0;
  b.w_vec = words_vec(L.u_bits, L.ldu, L.d_out);
  // input-piece tiles before each stage; each stage waits for its pieces,
  // the pieces of t wait for stage 1
  auto pieces = [&](const StageDesc& st, char* buf, int* ready) {
    StageDesc pc = st;
    const int64_t nch = piece_chunks(st.n_red);
    pc.kind = 1;
    pc.bfrag = reinterpret_cast<uint32_t*>(buf);
    pc.bsig = reinterpret_cast<int*>(buf + align_up((size_t)nch * 64 * T * kPieces * 16));
    pc.nrb = (int)cdiv(nch, kPrepChunks);  // tiles
    pc.nks = 1;
    pc.signal = ready;
    return pc;
  };
  int* x_ready = t_ready + 1;
  int* tp_ready = t_ready + 2;
  d[0] = pieces(a, pieces1, x_ready);  // no wait
  d[2] = pieces(b, pieces2, tp_ready);  // waits for t (b's wait)
  a.bfrag = d[0].bfrag;
  a.bsig = d[0].bsig;
  a.wait_ctr = x_ready;
  a.wait_target = d[0].nrb;
  b.bfrag = d[2].bfrag;
  b.bsig = d[2].bsig;
  b.wait_ctr = tp_ready;
  b.wait_target = d[2].nrb;
  d[1] = a;
  d[3] = b;
  return 4;
}

size_t dec_workspace_bytes(const nq_lrb& L, int64_t T) {
  return align_up((size_t)(1 + dec_linear_counters(L, T, true)) * sizeof(int)) + dec_linear_bytes(L, T, true);
}

hipError_t launch_dec_linear(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                             hipStream_t s) {
  char* base = static_cast<char*>(ws);
  int* err = reinterpret_cast<int*>(base);
  int* ctr = err + 1;
  const int nctr = dec_linear_counters(L, T, true);
  char* lin = base + align_up((size_t)(1 + nctr) * sizeof(int));
  StageDesc d[kMaxLinearDescs];
  const int nd = dec_stage_descs(L, x, xd, T, y, true, lin, ctr, d);
  hipError_t e;
  if ((e = launch_zero_ints(err, 1 + nctr, s)) != hipSuccess) return e;
  for (int i = 0; i < nd; ++i) {
    d[i].signal = nullptr;  // stream order separates the launches
    d[i].wait_ctr = nullptr;
    if ((e = launch_dec_stage(d[i], T, err, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nq
