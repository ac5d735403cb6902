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
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "nq_internal.h"

namespace nq {

namespace {

constexpr unsigned kSpinLimit = 1u << 21;  // ~1 s of polling, then give up and flag


__device__ inline float bf16_bits(uint32_t h) { return __uint_as_float(h << 16); }

// Cross-lane moves within a row of 16 lanes (DPP: no LDS round trip, unlike
// __shfl_xor, which becomes ds_bpermute).  Every lane of the wave must be active.
__device__ inline unsigned lane_xor1(unsigned v) {  // quad_perm [1,0,3,2]
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
// Largest of v over the 64 lanes, in every lane: quad, half-row and row steps
// by DPP, then the four row maxima through scalar registers.
__device__ inline unsigned wave_max_u32(unsigned v) {
  v = max(v, lane_xor1(v));
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)v, 0), r1 = (unsigned)__builtin_amdgcn_readlane((int)v, 16);
  const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)v, 32), r3 = (unsigned)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

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

// The next tile id of a persistent workgroup is taken from the queue counter
// by thread 0 once the current tile enters its last chunk (or last round):
// early enough that the atomic's latency is hidden, late enough that a tile
// another stage waits for is not held behind a long tile that this workgroup
// has yet to finish.  (Taking it when the current tile started kept, e.g.,
// the t pieces of a linear behind a 224-step stage-1 tile while that
// linear's stage-2 tiles spun.)  Tiles outside a persistent loop pass none.
struct NextTile {
  int* counter;         // queue counter (null: no claim)
  int id = 0x7fffffff;  // thread 0: the claimed id (past every queue until claimed)
  __device__ inline void claim() {
    if (counter && threadIdx.x == 0) id = add_relaxed(counter, 1);
  }
};

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
      // the spans' sums in span order, loaded kBatch spans at a time (a load
      // per add would wait out one memory latency per span)
      constexpr int kBatch = 4;
      float sum[T];
#pragma unroll
      for (int t = 0; t < T; ++t) sum[t] = 0.0f;
      for (int c0 = 0; c0 < S.nks; c0 += kBatch) {
        float v[kBatch][T];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
#pragma unroll
          for (int t = 0; t < T; ++t)
            v[i][t] = c0 + i < S.nks ? gload(S.part + ((int64_t)(c0 + i) * T + t) * S.n_rows + o) : 0.0f;
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (c0 + i < S.nks)
#pragma unroll
            for (int t = 0; t < T; ++t) sum[t] += v[i][t];
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float* dst = S.out + (int64_t)t * S.n_rows + o;
        if (S.signal)
          store_agent(dst, sc * sum[t]);
        else
          gstore(dst, sc * sum[t]);
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
//    That is seven full-rate VALU operations per word.
//  * The inputs v = colscale (.) x are cut into fp8 (e4m3) pieces:
//    v * 2^s = q0 + q1/16 + q2/256 + ... (each q the round-to-nearest fp8 of
//    the scaled remainder), kPieces per token, each piece a matrix column.
//    2^s brings the chunk's largest |v| into [64, 128), so no piece saturates;
//    four pieces carry v to within 2^-16 of that largest value (the worst
//    case; round-to-nearest remainders alternate in sign, and a model of the
//    split measures about 2^-20, a relative error of ~4e-7 per stage).  A
//    fifth piece (~3e-9) added nothing next to the fp32 sums (~1e-7) but a
//    column per token: with four, T <= 4 fits one 16-column group and T <= 8
//    two.
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 (fp4 A, fp8 B; the B scale of a
//    column is the 2^-(s+4p) of its piece) then gives, for 16 rows and 128
//    reduction elements, the signed sums of 16 piece columns (one column
//    group; two for T = 5..8).  Products of +-1 and fp8 values
//    are exact and accumulate in fp32 across the chunks of the span; the
//    pieces of a token are added across lanes at the end of the tile.
// Operand layouts of the 16x16x128 fp4 x fp8 form (measured on the device):
// lane l holds A row l%16, reduction elements 32*(l/16) + [0, 32) as nibbles
// (dword d, nibble i = element 8d+i); B column l%16, elements 16*(l/16) +
// [0, 16) in bytes 0..15 and 64 + 16*(l/16) + [0, 16) in bytes 16..31; C
// column l%16, rows 4*(l/16) + [0, 4).  The expansion above permutes the
// elements within each lane's 32, and the B pieces follow the same order.
//
// In sequences the pieces of a stage's input are made once per stage, by
// input-piece tiles (eight chunks of 1024 elements each), and stored in the
// workspace in a compact form (only the 16-byte fragment blocks of the
// T*kPieces used columns); every row-block tile of the stage copies them into
// LDS chunk by chunk.  (Making them in every row-block tile took about a fifth
// of the stream rate: the loads of x and s2, the chunk maxima and the
// conversions.)  A single call, bound by its chain of dependent steps rather
// than by bytes, has each tile make its one chunk's pieces (tile_pieces).
//
// A workgroup covers 512 rows: each of 8 waves 64 rows as four sets of 16, set q
// holding rows 4m + q (m = 0..15) of the wave's 64.  For MFMA step k (128
// elements) lane l reads the words of rows 4*(l%16) + [0, 4) in word row
// 4k + l/16 (one 16-byte load; 16 lanes cover 256 contiguous bytes of a word
// row), and component q feeds the MFMAs of set q.

constexpr int kMfmaMaxT = 8;
constexpr int kMaxGroupT = 4;                          // largest T whose tiles take groups of row blocks
constexpr int kMRows = 512;                            // rows per tile = threads per workgroup (8 waves)
constexpr int kPieces = 4;                            // fp8 pieces per token
constexpr int kStepWords = 4;                         // word rows per MFMA step
constexpr int kChunkSteps = 8;                        // steps per staged chunk
constexpr int kChunkWords = kChunkSteps * kStepWords;  // 32 word rows
constexpr int kRingSteps = 4;                         // steps of sign words in flight per lane
static_assert(kChunkSteps % kRingSteps == 0, "ring slots are compile-time within a chunk");
constexpr int kStepInts = 64 * 8;                     // B fragments of one step and MFMA (64 lanes x 32 bytes)
constexpr int kPrepGroups = kMRows / 256;            // chunks per round of an input-piece tile
// B columns are (token t, piece p) -> t*kPieces + p; every 16 of them form
// one MFMA column group (T*kPieces columns: 1 group up to T = 4, 2 up to 8).
template <int T>
constexpr int col_groups() { return (T * kPieces + 15) / 16; }
// Steps of sign words in flight per lane: 4 (16 KB per wave).  8 kept twice
// the bytes in flight and measured 1-4 % slower (same box; 70B stacks and 7B
// attention sequences): the deeper queues lengthen every other global access
// of a tile (input counters, pieces, descriptors), which wait behind them.
template <int T>
constexpr int ring_steps() { return kRingSteps; }
// LDS of a workgroup, in 4-byte words: [B fragments, two chunk buffers of
// kChunkSteps x col_groups x kStepInts] [chunk scale exponents, two buffers of
// T] [per-round maxima of an input-piece tile, [2][kPrepGroups][T]] [row sums
// [T][kMRows], 16-byte aligned] [two shared flag words].  Stores that only keep loads out of branches (blocks
// past a chunk's last, scale exponents of threads past T) go to the row sums,
// which are unused until a row block's end.
// T = 8 (kSumsInB) keeps its row sums in the first chunk buffer instead and
// those stores in a region of their own: two workgroups then fit a CU's
// 160 KB.  That buffer is free at a tile's end (one row block per tile, the
// last chunk read before the barrier that ends the loop) and, with all 32
// columns used, has no zero columns to keep (see mfma_lds_init).
template <int T>
constexpr int b_ints() { return kChunkSteps * col_groups<T>() * kStepInts; }
template <int T>
constexpr bool sums_in_b() { return T > kMaxGroupT && T * kPieces == 16 * col_groups<T>(); }
template <int T>
constexpr int sig_off() { return 2 * b_ints<T>(); }
template <int T>
constexpr int slot_off() { return sig_off<T>() + 2 * T; }
constexpr int align4(int x) { return (x + 3) & ~3; }
template <int T>
constexpr int sum_off() { return sums_in_b<T>() ? 0 : align4(slot_off<T>() + 2 * kPrepGroups * T); }
template <int T>
constexpr int dummy_off() { return sums_in_b<T>() ? align4(slot_off<T>() + 2 * kPrepGroups * T) : sum_off<T>(); }
template <int T>
constexpr int flag_off() { return dummy_off<T>() + kMRows * (sums_in_b<T>() ? 1 : T); }  // s_flag, s_tile
template <int T>
constexpr int mfma_lds() { return flag_off<T>() + 4; }

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Every token's inputs for this thread's 4 elements of a chunk.
template <int T>
struct PieceIn {
  uint32_t x[T][4];  // raw bf16 / fp32 bits
  float cs[4];
};

// This thread's build task within a chunk: word row wr (0..31), dword j of
// the A expansion, half ih of the nibbles: elements 32*wr + 4*(4*ih + k) +
// 3 - j, k = 0..3, i.e. one B dword (4 consecutive reduction positions).
__device__ inline int task_element(int task, int k) {
  const int wr = task >> 3, j = (task >> 1) & 3, ih = task & 1;
  return 32 * wr + 4 * (4 * ih + k) + 3 - j;
}

// Loads of tokens tok0 .. tok0+NT-1 of a chunk's inputs (the column scales
// once).  Elements at or past cend read element 0 of the token (always in
// bounds) and are dropped later, so the loads keep a fixed count and position
// in the pipeline.
template <int NT>
__device__ inline void piece_load_inputs(const StageDesc& S, int task, int tok0, int64_t c0, int64_t cend,
                                         PieceIn<NT>& in) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t e = c0 + task_element(task, k);
    const int64_t ec = e < cend ? e : 0;
    in.cs[k] = S.colscale ? gload(S.colscale + ec) : 1.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t idx = (int64_t)(tok0 + t) * S.n_red + ec;
      in.x[t][k] = S.x_bf16 ? (uint32_t)gload(static_cast<const uint16_t*>(S.xin) + idx)
                            : gload(static_cast<const uint32_t*>(S.xin) + idx);
    }
  }
}

template <int T>
__device__ inline float piece_value(const StageDesc& S, const PieceIn<T>& in, int t, int task, int64_t c0,
                                    int64_t cend, int k) {
  const float x = S.x_bf16 ? bf16_bits(in.x[t][k]) : __uint_as_float(in.x[t][k]);
  return c0 + task_element(task, k) < cend ? x * in.cs[k] : 0.0f;
}

// Largest |v| of the chunk for every token into slot[t] (float bits of a
// non-negative value order like unsigned integers; NaN orders above inf).
template <int T>
__device__ inline void piece_chunk_max(const StageDesc& S, const PieceIn<T>& in, int task, int64_t c0, int64_t cend,
                                       unsigned* slot) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
    unsigned m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, __float_as_uint(fabsf(piece_value(S, in, t, task, c0, cend, k))));
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) atomicMax(slot + t, m);
  }
}

// Scale exponent s for a chunk maximum (float bits): max * 2^s in [64, 128).
// s is capped at 115 so that the MFMA scale of the last piece,
// 2^-(s+4(kPieces-1)), stays within the E8M0 range; only chunks whose largest
// |v| is below 2^-89 start below 64 and so keep fewer significant bits.  A non-finite maximum
// gives kShiftNaN: the chunk's pieces are NaN.
constexpr int kShiftNaN = 1 << 20;
constexpr int kMaxShift = 127 - 4 * (kPieces - 1);
__device__ inline int chunk_shift(unsigned mbits) {
  const int e = (int)((mbits >> 23) & 0xFF);
  return e == 255 ? kShiftNaN : min(133 - e, kMaxShift);
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

// The kPieces fp8 pieces of four consecutive reduction positions, for NT
// tokens at once: r[i] holds token i's four values (already times 2^shift);
// emit(i, p, dword) receives piece p of token i as one packed dword.  The
// pieces of a token depend on one another (each is cut from the remainder of
// the last), so the tokens' chains are interleaved piece by piece.  The
// partner thread (lane ^ 1, the other half of each group of 8) must run it
// too.
template <int NT, typename Emit>
__device__ inline void cut_pieces(float (&r)[NT][4], Emit emit) {
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    int d[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      d[i] = __builtin_amdgcn_cvt_pk_fp8_f32(r[i][0], r[i][1], 0, false);
      d[i] = __builtin_amdgcn_cvt_pk_fp8_f32(r[i][2], r[i][3], d[i], true);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      int emax = max_fp8_exponent(d[i]);  // with the partner thread: one group of 8
      emax = max(emax, (int)lane_xor1((unsigned)emax));
      d[i] = keep_fp8_exponents(d[i], max(1, emax - 7));
      emit(i, p, d[i]);
    }
    if (p + 1 < kPieces) {
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        typedef float v2f __attribute__((ext_vector_type(2)));
        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(d[i], false);
        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(d[i], true);
        r[i][0] = (r[i][0] - lo.x) * 16.0f;
        r[i][1] = (r[i][1] - lo.y) * 16.0f;
        r[i][2] = (r[i][2] - hi.x) * 16.0f;
        r[i][3] = (r[i][3] - hi.y) * 16.0f;
      }
    }
  }
}

// Compact piece layout of one chunk: 16-byte blocks, block
// ((step*2 + half)*4 + group)*NC + column holds half `half` of the B fragment
// of lane (column % 16) + 16*group in column group column / 16, MFMA step
// `step` (NC = T*kPieces used columns; column t*kPieces + p is piece p of
// token t).
template <int T>
constexpr int chunk_blocks() { return kChunkSteps * 2 * 4 * T * kPieces; }

// Input-piece work items: (chunk, group of TG tokens), two per round (one per
// group of 256 threads).  Sequences take every token of a chunk in one item
// (TG = T: the column scales load once, all of the chunk's loads are in flight
// together, fewer items) and up to four rounds per tile at T = 1 (eight
// chunks), one from T = 3 on.  Single calls take one token per item (TG = 1)
// and one round per tile: the pieces are ready one item's latency after the
// launch, on as many workgroups as there are (chunk, token) pairs.
__host__ __device__ inline int prep_items(int64_t T, bool single) {
  return single || T >= 3 ? kPrepGroups : (int)(8 / T);
}

// One input-piece tile: items [S.prep_items * tile, ...) of the stage input,
// item i being chunk i / (T / TG) with tokens TG * (i % (T / TG)) ...  Each
// group of 256 threads takes an item per round; per chunk and token each
// thread makes one B dword (4 consecutive reduction positions) per piece; the
// next round's inputs load while the current ones are converted.
template <int T, int TG>
__device__ void mfma_prep_tile(const StageDesc& S, int tile, float* ldsf, int* err, NextTile& next) {
  static_assert(T % TG == 0, "whole token groups");
  constexpr int NTG = T / TG;  // token groups per chunk
  constexpr int NC = T * kPieces;
  constexpr int64_t kChunkElems = kChunkWords * kWordBits;
  unsigned* slots = reinterpret_cast<unsigned*>(reinterpret_cast<int*>(ldsf) + slot_off<T>());  // [round&1][group][T]
  const int tid = threadIdx.x, half = tid >> 8, task = tid & 255;  // half: this thread's group
  const int nit = (int)cdiv(S.n_red, kChunkElems) * NTG;
  const int it0 = tile * S.prep_items;
  const int it1 = min(it0 + S.prep_items, nit);
  wait_input(S, err);
  const int wr = task >> 3, j = (task >> 1) & 3, ih = task & 1;
  const int kk = wr >> 2, gw = wr & 3;
  const int gp = 2 * (gw & 1) + (j >> 1);
  const int64_t task_off = (int64_t)(((kk * 2 + (gw >> 1)) * 4 + gp) * NC) * 4 + 2 * (j & 1) + ih;
  if (tid < 2 * kPrepGroups * TG) slots[tid] = 0;
  // the item this group takes in a round (past the tile's last: the last item
  // again for the loads, nothing stored)
  auto item_of = [&](int r0) { return min(r0 + half, nit - 1); };
  PieceIn<TG> in, nxt;
  {
    const int it = item_of(it0);
    piece_load_inputs<TG>(S, task, TG * (it % NTG), (int64_t)(it / NTG) * kChunkElems, S.n_red, in);
  }
  __syncthreads();
  for (int r0 = it0, round = 0; r0 < it1; r0 += kPrepGroups, ++round) {
    const bool last = r0 + kPrepGroups >= it1;
    if (last) next.claim();  // the tile's last round
    const bool mine = r0 + half < it1;  // wave-uniform: a group is 4 whole waves
    const int it = item_of(r0);
    const int ch = it / NTG, tok0 = TG * (it % NTG);
    const int64_t c0 = ch * kChunkElems;
    unsigned* slot = slots + ((round & 1) * kPrepGroups + half) * TG;
    piece_chunk_max<TG>(S, in, task, c0, S.n_red, slot);
    if (!last) {
      const int itn = item_of(r0 + kPrepGroups);
      piece_load_inputs<TG>(S, task, TG * (itn % NTG), (int64_t)(itn / NTG) * kChunkElems, S.n_red, nxt);
    }
    __syncthreads();  // the items' maxima are complete
    if (mine) {
      uint32_t* dst = S.bfrag + (int64_t)ch * chunk_blocks<T>() * 4 + task_off;
      // tokens in pairs (all TG at once costs the sequence kernel registers)
      constexpr int NP = TG > 1 ? 2 : 1;
#pragma unroll
      for (int tg0 = 0; tg0 < TG; tg0 += NP) {
        float r[NP][4];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int tg = min(tg0 + i, TG - 1);
          const int shift = chunk_shift(slot[tg]);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            r[i][k] = shift == kShiftNaN ? __int_as_float(0x7FC00000)
                                         : ldexpf(piece_value(S, in, tg, task, c0, S.n_red, k), shift);
          if (task == 0 && tg0 + i < TG)
            store_agent(reinterpret_cast<float*>(S.bsig + (int64_t)ch * T + tok0 + tg), __int_as_float(shift));
        }
        // each dword and the partner thread's (task ^ 1, same wave) form one group of 8
        cut_pieces<NP>(r, [&](int i, int p, int d) {
          if (tg0 + i < TG)
            store_agent(reinterpret_cast<float*>(dst + ((tok0 + tg0 + i) * kPieces + p) * 4), __int_as_float(d));
        });
      }
    }
    __syncthreads();  // every thread has read this round's maxima
    if (task < TG) slot[task] = 0;  // reused two rounds on (its maxima come after the next barrier)
    if (!last) in = nxt;
  }
  if (S.signal) {
    stores_done_barrier();  // the tile's pieces are at the coherence point
    if (tid == 0) add_relaxed(S.signal, 1);
  }
  __syncthreads();  // the slots are reused by the next tile
}

// Single calls: a stage tile spans one chunk and makes that chunk's input
// pieces itself, straight into LDS buffer 0 (no input-piece tiles and no hand
// over through the workspace: for one linear the chain of dependent steps,
// not the bytes, sets the time).  Thread task = tid & 255 makes the B dword of
// each piece for 4 reduction positions, as an input-piece tile does, for
// tokens (tid >> 8) + 2i; the dword goes where the chunk copy of a sequence
// tile would put it.  Ends with the chunk's fragments and scale exponents in
// LDS (after a barrier).
template <int T>
__device__ inline void tile_pieces(const StageDesc& S, int64_t c0, int* lds) {
  constexpr int TH = (T + 1) / 2;  // tokens per half of the workgroup
  constexpr int G = col_groups<T>();
  const int tid = threadIdx.x, task = tid & 255;
  const int half = __builtin_amdgcn_readfirstlane(tid >> 8);  // uniform over a wave
  unsigned* slot = reinterpret_cast<unsigned*>(lds + slot_off<T>());  // [T] chunk maxima
  const int64_t cend = S.n_red;
  PieceIn<TH> in;
  uint32_t eo[4];  // element offsets in a token row (past the end: element 0, dropped later)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t e = c0 + task_element(task, k);
    eo[k] = e < cend ? (uint32_t)e : 0u;
    in.cs[k] = S.colscale ? gload(S.colscale + eo[k]) : 1.0f;
  }
  // token half + 2i (past T: token T-1 again, dropped below)
  auto idx = [&](int i, int k) { return (int64_t)min(half + 2 * i, T - 1) * S.n_red + eo[k]; };
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < TH; ++i)
      in.x[i][k] = S.x_bf16 ? (uint32_t)gload(static_cast<const uint16_t*>(S.xin) + idx(i, k))
                            : gload(static_cast<const uint32_t*>(S.xin) + idx(i, k));
  if (tid < T) slot[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TH; ++i) {
    unsigned m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, __float_as_uint(fabsf(piece_value(S, in, i, task, c0, cend, k))));
    m = wave_max_u32(m);
    if ((tid & 63) == 0 && half + 2 * i < T) atomicMax(slot + half + 2 * i, m);
  }
  __syncthreads();  // the chunk's maxima are complete
  const int wr = task >> 3, j = (task >> 1) & 3, ih = task & 1;
  const int kk = wr >> 2, gw = wr & 3;
  const int gp = 2 * (gw & 1) + (j >> 1);
  // LDS place of column n's dword: block (kk, group gp, half gw >> 1) of
  // column n in column group n / 16, dword 2 * (j & 1) + ih
  const int base = kk * G * kStepInts + (gw >> 1) * 256 + 16 * gp * 4 + 2 * (j & 1) + ih;
  float r[TH][4];
#pragma unroll
  for (int i = 0; i < TH; ++i) {
    const int t = min(half + 2 * i, T - 1);  // past T: a copy of token T-1, not stored
    const int shift = chunk_shift(slot[t]);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r[i][k] = shift == kShiftNaN ? __int_as_float(0x7FC00000) : ldexpf(piece_value(S, in, i, task, c0, cend, k), shift);
    if (task == 0 && half + 2 * i < T) lds[sig_off<T>() + t] = shift;
  }
  cut_pieces<TH>(r, [&](int i, int p, int d) {  // the partner thread is task ^ 1, same wave
    const int t = half + 2 * i;  // uniform over a wave
    if (t < T) {
      const int n = t * kPieces + p;
      lds[base + (n / 16) * kStepInts + (n % 16) * 4] = d;
    }
  });
  __syncthreads();  // the chunk's fragments are in LDS buffer 0
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

// The two constants of the expansion, held in registers for the whole tile:
// as literals the mask and the OR cannot share one instruction (a three-operand
// VALU instruction takes no literal here), and the compiler would issue them
// as two.  Made by asm so that they are not rematerialised at every use.
struct ExpandConsts {
  uint32_t mask;  // SGPR: 0x88888888, the sign bit of every nibble
  uint32_t one;   // VGPR: 0x22222222, +1.0 in every nibble
};
__device__ inline ExpandConsts expand_consts() {
  ExpandConsts c;
  asm volatile("s_mov_b32 %0, 0x88888888" : "=s"(c.mask));
  asm volatile("v_mov_b32 %0, 0x22222222" : "=v"(c.one));
  return c;
}
__device__ inline uint32_t and_or(uint32_t x, const ExpandConsts& c) {
  uint32_t y;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(y) : "v"(x), "s"(c.mask), "v"(c.one));
  return y;
}

// Seven full-rate VALU instructions per word: three doublings, four AND-ORs.
__device__ inline v8i expand_word(uint32_t x, const ExpandConsts& c) {
  const uint32_t x1 = twice(x), x2 = twice(x1), x3 = twice(x2);
  v8i a;
  a[0] = (int)and_or(x, c);
  a[1] = (int)and_or(x1, c);
  a[2] = (int)and_or(x2, c);
  a[3] = (int)and_or(x3, c);
  a[4] = a[5] = a[6] = a[7] = 0;
  return a;
}

// Sum over the 4 lanes of a quad (DPP quad permutations), in every lane of it.
__device__ inline float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  return v;
}

// W4: sign words are read 4 rows at a time (16-byte loads); otherwise one
// word per load (row counts or strides that are not multiples of 4).
// FUSE (single calls): the span is one chunk whose pieces the tile makes
// itself (tile_pieces); otherwise they are copied from the stage's
// input-piece blocks chunk by chunk.
template <int T, bool W4, bool FUSE>
__device__ void mfma_tile(const StageDesc& S, int local, float* ldsf, int* s_flag, int* err, NextTile& next) {
  static_assert(T <= kMfmaMaxT, "tokens");
  constexpr int G = col_groups<T>();
  int* lds = reinterpret_cast<int*>(ldsf);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, col = lane & 15, grp = lane >> 4;
  // a tile is rb_group consecutive row blocks (rb0 ..) of one reduction span;
  // for T > 3 always one (the host plans it so): the loop over row blocks
  // costs those tiles registers they do not have
  constexpr bool kGroups = T <= kMaxGroupT;
  const int group = kGroups ? S.rb_group : 1;
  const int nrbt = (S.nrb + group - 1) / group;
  const int rbt = local % nrbt;
  const int ks = local / nrbt;
  const int rb0 = rbt * group;
  const int nrbs = kGroups ? min(group, S.nrb - rb0) : 1;
  const int64_t span0 = (int64_t)ks * S.kc;
  const int64_t span1 = imin(span0 + S.kc, S.n_red);
  const int w0 = __builtin_amdgcn_readfirstlane((int)(span0 / kWordBits));
  const uint32_t ld4 = __builtin_amdgcn_readfirstlane((uint32_t)(S.ld * 4));
  const int nw = (int)cdiv(span1 - span0, kWordBits);
  const int nk = (nw + kStepWords - 1) / kStepWords;
  const int nchunks = (nw + kChunkWords - 1) / kChunkWords;

  // this lane's first row in the tile's first row block (row block i adds
  // i * kMRows) and its byte offset in a word row
  const int lrow = rb0 * kMRows + wv * 64 + 4 * col;
  const uint32_t lane_off = 4u * (uint32_t)lrow + (uint32_t)grp * ld4;
  // Step k of row block i reads word row 4k + grp of the span through a buffer
  // resource that starts at word row 4k and ends with row n_rows-1 of the
  // span's last word row: words past the span (a partial last step, steps past
  // the last) or past the last row are out of range and read as 0 without
  // touching memory (with W4, n_rows is a multiple of 4, so a 16-byte load is
  // entirely in or out of range).  Rows at or past n_rows (in the last row
  // block) get an offset past any buffer (sign-word buffers are below 2 GiB)
  // instead of words of the next word row; row blocks past the tile's last
  // read nothing.  Everything but the lane offset is scalar.
  auto load_step = [&](int i, int k, u32x4& dst) {
    const int wb = kStepWords * k;  // from the span start
    const int rows_left = i < nrbs ? max(nw - wb, 0) : 0;
    const uint32_t nrec = rows_left > 0 ? (uint32_t)(rows_left - 1) * ld4 + 4u * (uint32_t)S.n_rows : 0u;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(S.bits) + (int64_t)(w0 + wb) * S.ld, (short)0, (int)nrec, 0x00020000);
    const int row = lrow + i * kMRows;
    const uint32_t off = lane_off + 4u * (uint32_t)(i * kMRows);
    if constexpr (W4) {  // n_rows % 4 == 0: the lane's 4 rows are all valid or all past the end
      const uint32_t o = row < S.n_rows ? off : kOutOfRange;
      dst = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, kStreamLoad));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[q] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(row + q < S.n_rows ? off + 4u * q : kOutOfRange), 0,
                                                      kStreamLoad);
    }
  };

  // This thread's compact blocks of a chunk (see mfma_prep_tile) and their
  // LDS places.  Every thread loads NBT blocks (past the chunk's last block:
  // the last one again, written to the dummy region of the LDS layout) and
  // the chunk's scale exponents, so no branch surrounds the loads.  Chunk c+1
  // is copied into the other LDS buffer during chunk c in two halves of the
  // blocks: the first loaded at the chunk's start and written at step 2, the
  // second loaded then and written at step 6 (the loads are waited for with
  // the sign words issued after them still in flight); one barrier per chunk.
  // Half the blocks in registers at a time leaves T >= 7 fewer spills (measured
  // +2 % at T = 7, 8; one half at the chunk's middle measured the same for
  // T <= 6).  A chunk past the stage's last loads the last one again.
  constexpr int NB = chunk_blocks<T>();
  constexpr int NBT = (NB + kMRows - 1) / kMRows;  // blocks per thread
  constexpr int NC = T * kPieces;
  int lds_at[NBT], blk_at[NBT];
#pragma unroll
  for (int m = 0; m < NBT; ++m) {
    const int bi = tid + m * kMRows;
    const int n = bi % NC, rest = bi / NC;
    const int g = rest % 4, h = (rest / 4) % 2, kk = rest / 8;
    lds_at[m] = bi < NB ? (kk * G + n / 16) * kStepInts + h * 256 + (n % 16 + 16 * g) * 4 : dummy_off<T>();
    blk_at[m] = min(bi, NB - 1);
  }
  const int chunk0 = (int)(span0 / (kChunkWords * kWordBits));
  const int last_chunk = (int)((S.n_red - 1) / (kChunkWords * kWordBits));
  const u32x4* bsrc = reinterpret_cast<const u32x4*>(S.bfrag);
  constexpr int NH = (NBT + 1) / 2;  // blocks per thread and half
  u32x4 blk[NH];
  int sig;
  auto load_half = [&](int ch, int hh) {
    ch = min(ch, last_chunk);
#pragma unroll
    for (int m = 0; m < NH; ++m)
      if (hh * NH + m < NBT) blk[m] = gload(bsrc + (int64_t)ch * NB + blk_at[hh * NH + m]);
    if (hh == 0) sig = gload(S.bsig + (int64_t)ch * T + min(tid, T - 1));
  };
  auto store_half = [&](int buf, int hh) {
#pragma unroll
    for (int m = 0; m < NH; ++m)
      if (hh * NH + m < NBT) *reinterpret_cast<u32x4*>(lds + buf * b_ints<T>() + lds_at[hh * NH + m]) = blk[m];
    if (hh != 0) return;
    // every thread stores (threads past T into the dummy region), so the
    // compiler cannot move the load into a branch behind later sign-word loads
    lds[tid < T ? sig_off<T>() + buf * T + tid : dummy_off<T>() + tid] = sig;
  };
  // the first sign words do not depend on the stage input: in flight while
  // the wait and the first chunk's pieces complete (loads complete in issue
  // order for s_waitcnt, so the acquire and chunk 0's pieces wait for them;
  // issuing them after the wait measured slightly slower)
  constexpr int R = ring_steps<T>();
  u32x4 ring[R];
#pragma unroll
  for (int k = 0; k < R; ++k) load_step(0, k, ring[k]);
  wait_input(S, err);  // the stage's input (or its pieces) is final
  if constexpr (FUSE) {
    tile_pieces<T>(S, span0, lds);
  } else {
    load_half(chunk0, 0);
    store_half(0, 0);
    load_half(chunk0, 1);
    store_half(0, 1);
    __syncthreads();  // chunk 0's fragments are in LDS buffer 0
  }

  const ExpandConsts xc = expand_consts();
  // the sums of all chunks accumulate in acc: each chunk's B column (token t,
  // piece p) carries the MFMA scale 2^-(s_t + 4p) of that chunk
  v4f acc[4][G];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int cg = 0; cg < G; ++cg) acc[q][cg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // row block ri is complete: add the pieces of each token across the quad
  // of lanes that holds its columns (lane col = 4 t' + p holds piece p of
  // token 4 cg + t'), then lane 4 t' of every row group writes its 4 rows of
  // every set; then the rows' results, and a clear start for the next row
  // block
  auto finish_rb = [&](int ri) {
    float* sums = ldsf + sum_off<T>();
    static_assert(kPieces == 4, "a token's pieces are one quad of lanes");
#pragma unroll
    for (int cg = 0; cg < G; ++cg) {
      const int t = 4 * cg + col / 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // C row 4*grp + r of set q is row 16*grp + 4r + q of the wave
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = quad_sum(acc[q][cg][r]);
        if ((col & 3) == 0 && t < T)
          *reinterpret_cast<float4*>(sums + t * kMRows + wv * 64 + grp * 16 + 4 * r) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
    float accr[T];
#pragma unroll
    for (int t = 0; t < T; ++t) accr[t] = sums[t * kMRows + tid];
    const int rb = rb0 + ri;
    const int64_t o = (int64_t)rb * kMRows + tid;
    finish_rows<T>(S, rb, ks, o, o < S.n_rows, accr, s_flag);  // ends with a barrier: sums are free again
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int cg = 0; cg < G; ++cg) acc[q][cg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // the tile's row blocks run back to back: virtual chunk vc is chunk c of row
  // block ri; the ring's loads R steps ahead cross into the next row block, so
  // its first sign words are in flight while this one finishes
  const int nvc = nrbs * nchunks;
  int ri = 0, c = 0;
  for (int vc = 0; vc < nvc; ++vc) {
    if (vc + 1 == nvc) next.claim();  // the tile's last chunk
    const int buf = vc & 1;
    // E8M0 scale of this lane's column in every group (2^0 for columns past
    // the last piece, whose B entries are 0; a NaN chunk has NaN pieces)
    int bscale[G];
#pragma unroll
    for (int cg = 0; cg < G; ++cg) {
      const int n = 16 * cg + col, tc = n / kPieces, pc = n % kPieces;
      const int sg = lds[sig_off<T>() + buf * T + min(tc, T - 1)];
      bscale[cg] = tc < T ? 127 - (sg == kShiftNaN ? 0 : sg) - 4 * pc : 127;
    }
    const int nxt_chunk = chunk0 + (c + 1 < nchunks ? c + 1 : 0);
    if constexpr (!FUSE) load_half(nxt_chunk, 0);  // next chunk's pieces (the next row block's first)

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
          const v8i a = expand_word(ring[kk % R][q], xc);
#pragma unroll
          for (int cg = 0; cg < G; ++cg)
            acc[q][cg] =
                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[cg], acc[q][cg], 4, 0, 0, 127, 0, bscale[cg]);
        }
      }
      // the load R steps ahead: this row block's step k + R, or, past its last
      // chunk, the next row block's step kk + R - 8 (past the tile's last row
      // block: out of range, no memory access); no branch around the load
      const bool next_rb = kk + R >= kChunkSteps && c + 1 == nchunks;
      load_step(next_rb ? ri + 1 : ri, next_rb ? kk + R - kChunkSteps : k + R, ring[kk % R]);
      if constexpr (!FUSE) {
        if (kk == 2) {  // the other buffer was last read in chunk vc-1
          store_half(buf ^ 1, 0);
          load_half(nxt_chunk, 1);
        }
        if (kk == 6) store_half(buf ^ 1, 1);
      }
    }
    __syncthreads();  // chunk vc+1's fragments are in LDS; every wave is done with chunk vc's
    if (c + 1 < nchunks) {
      ++c;
      continue;
    }
    if constexpr (!kGroups) break;  // one row block: its finish follows the loop
    finish_rb(ri);
    ++ri;
    c = 0;
  }
  if constexpr (!kGroups) finish_rb(0);
}

// 4 waves per SIMD (at most 128 VGPRs) and 2 workgroups per CU for every T
// (with two column groups B fragments are read at their own step, to make
// room for the second group's accumulators).
template <int T>
constexpr int min_waves() { return 4; }
static_assert(col_groups<kMfmaMaxT>() <= 2, "T <= 8 in two column groups");

// SINGLE: a single call's tiles (kind 2 only); otherwise a sequence's (kinds
// 0 and 1).  Kept apart so that neither kernel carries the other's code and
// registers.
template <int T, bool SINGLE>
__device__ inline void stage_tile(const StageDesc& S, int local, float* lds, int* s_flag, int* err, NextTile& next) {
  if constexpr (SINGLE) {
    if (S.w_vec)
      mfma_tile<T, true, true>(S, local, lds, s_flag, err, next);
    else
      mfma_tile<T, false, true>(S, local, lds, s_flag, err, next);
  } else {
    if (S.kind == 1 && S.prep_tg == 1)
      mfma_prep_tile<T, 1>(S, local, lds, err, next);
    else if (S.kind == 1)
      mfma_prep_tile<T, T>(S, local, lds, err, next);
    else if (S.w_vec)
      mfma_tile<T, true, false>(S, local, lds, s_flag, err, next);
    else
      mfma_tile<T, false, false>(S, local, lds, s_flag, err, next);
  }
}

// ints: [0] error flag (sticky), [1] next tile, [2] workgroups exited,
// [3 .. n_ints) per-linear counters.  Workgroups take tiles in schedule order
// from the counter at [1]; `lookup(tile, S, local)` gives a tile's descriptor
// and its index within its stage.  The last workgroup to exit zeroes
// [1 .. n_ints), so consecutive runs need no separate reset launch.
template <int T, bool SINGLE, typename Lookup>
__device__ inline void persistent_tiles(Lookup lookup, int ntiles, int* ints, int n_ints, float* lds) {
  int& s_flag = reinterpret_cast<int*>(lds)[flag_off<T>()];
  int& s_tile = reinterpret_cast<int*>(lds)[flag_off<T>() + 1];
  int* err = ints;
  int* next_tile = ints + 1;
  mfma_lds_init<T>(reinterpret_cast<int*>(lds));
  if (threadIdx.x == 0) s_tile = add_relaxed(next_tile, 1);
  __syncthreads();
  int tile = __builtin_amdgcn_readfirstlane(s_tile);
  while (tile < ntiles) {
    NextTile next;  // thread 0 claims the next tile id during the tile's last chunk
    next.counter = next_tile;
    StageDesc S;
    int local;
    lookup(tile, S, local);
    stage_tile<T, SINGLE>(S, local, lds, &s_flag, err, next);
    if (threadIdx.x == 0) s_tile = next.id;
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

// A sequence plan: descriptors and the per-tile descriptor table in the
// workspace (uploaded once per plan).
template <int T>
__global__ __launch_bounds__(kMRows) __attribute__((amdgpu_waves_per_eu(min_waves<T>())))
void dec_persistent_kernel(const StageDesc* __restrict__ segs, const int* __restrict__ tile_seg, int ntiles, int* ints,
                           int n_ints) {
  __shared__ __attribute__((aligned(16))) float lds[mfma_lds<T>()];
  persistent_tiles<T, false>(
      [&](int tile, StageDesc& S, int& local) {
        S = segs[tile_seg[tile]];  // one lookup (a scan over the segments stalled for microseconds)
        local = tile - S.tile0;
      },
      ntiles, ints, n_ints, lds);
}

// One linear (a single call): its descriptors travel in the kernel arguments.
struct LinearSched {
  StageDesc d[kMaxLinearDescs];
  int end[kMaxLinearDescs];  // cumulative tile counts
};

template <int T>
__global__ __launch_bounds__(kMRows) __attribute__((amdgpu_waves_per_eu(min_waves<T>())))
void dec_linear_kernel(LinearSched L, int* ints, int n_ints) {
  __shared__ __attribute__((aligned(16))) float lds[mfma_lds<T>()];
  persistent_tiles<T, true>(
      [&](int tile, StageDesc& S, int& local) {
        // the stage is uniform across the workgroup: select a pointer into the
        // argument segment (scalar loads), not a copy of each descriptor
        const int k = (tile >= L.end[0]) + (tile >= L.end[1]) + (tile >= L.end[2]);
        const StageDesc* P = &L.d[k];
        S = *P;
        local = tile - P->tile0;
      },
      L.end[kMaxLinearDescs - 1], ints, n_ints, lds);
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

// Single calls split the reduction into spans of one chunk, whose input
// pieces each tile makes itself (tile_pieces); sequences keep whole
// reductions (no partial sums).
int64_t dec_single_span(int64_t, int64_t, int64_t) { return kChunkWords * kWordBits; }

hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = imin(cdiv(n, 256), 1024);
  hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

namespace {
int persistent_grid_query(int64_t T) {
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
}  // namespace

// Resident workgroups of the persistent kernel, per device and T: queried once
// (the property and occupancy queries cost microseconds of host time, which a
// single call would otherwise pay every time).
int dec_persistent_grid(int64_t T) {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][kMfmaMaxT + 1];
  int dev = 0;
  if (T < 1 || T > kMfmaMaxT || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs)
    return persistent_grid_query(T);
  int g = cache[dev][T].load(std::memory_order_relaxed);
  if (g == 0) {
    g = persistent_grid_query(T);
    cache[dev][T].store(g, std::memory_order_relaxed);
  }
  return g;
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
int64_t seq_span() {
  static const int64_t v = [] {
    const char* e = getenv("NQ_SEQ_SPAN");
    const long long x = e ? atoll(e) : 0;
    return (int64_t)(x < 0 ? 0 : x);
  }();
  return v;
}

void plans(const nq_lrb& L, int64_t T, bool split, StagePlan* p1, StagePlan* p2) {
  *p1 = dec_stage_plan(L.r, L.d_in, T, split ? dec_single_span(L.r, L.d_in, T) : seq_span());
  *p2 = dec_stage_plan(L.d_out, L.r, T, split ? dec_single_span(L.d_out, L.r, T) : seq_span());
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

// Per-linear device buffers: [part1][t][part2], then for sequences [pieces of
// x][pieces of t] (single calls make their pieces in LDS).
size_t dec_linear_bytes(const nq_lrb& L, int64_t T, bool split) {
  StagePlan p1, p2;
  plans(L, T, split, &p1, &p2);
  size_t off = align_up(part_bytes(p1, T));
  off = align_up(off + (size_t)T * L.r * sizeof(float));
  off = align_up(off + part_bytes(p2, T));
  return split ? off : off + piece_bytes(L.d_in, T) + piece_bytes(L.r, T);
}

// Per-linear counters: [stage-1 row blocks][stage-2 row blocks][t ready]
// [pieces of x ready][pieces of t ready].
int dec_linear_counters(const nq_lrb& L, int64_t T, bool split) {
  StagePlan p1, p2;
  plans(L, T, split, &p1, &p2);
  return p1.nrb + p2.nrb + 3;
}


// Sequences: row blocks per stage tile (T <= kMaxGroupT only), so that a tile streams about 32
// MFMA steps (256 KB of sign words) however short the stage's reduction is;
// the per-tile costs (descriptor lookup, input wait, first pieces, the ring's
// start) are then paid once per group.  Measured (same box, ms per step or
// GB/s; 1 = one row block per tile / 32 / 64): 70B 0.55 bit 0.945 / 0.940 /
// 0.929, 0.25x ranks 0.544 / 0.523 / 0.519, 1 bit flat; 7B attention over 505
// copies 4231 / 4535 / 4075 GB/s, 7B MLP set 3912 / 4105 / 4194 GB/s
// (NQ_SEQ_TILE_STEPS: tuning knob).
int seq_rb_group(const StagePlan& p, int64_t T) {
  if (T > kMaxGroupT) return 1;
  static const int steps = [] {
    const char* e = getenv("NQ_SEQ_TILE_STEPS");
    const int v = e ? atoi(e) : 32;
    return v < 1 ? 1 : v;
  }();
  const int per_rb = (int)cdiv(p.kc, kChunkWords * kWordBits) * kChunkSteps;  // whole chunks
  return (int)imax(1, imin(p.nrb, steps / per_rb));
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
  a.rb_group = split ? 1 : seq_rb_group(p1, T);
  a.x_bf16 = xd == NQ_BF16;
  a.w_vec = words_vec(L.vt_bits, L.ldv, L.r);
  a.kind = split ? 2 : 0;
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
  b.rb_group = split ? 1 : seq_rb_group(p2, T);
  b.x_bf16 = 0;
  b.w_vec = words_vec(L.u_bits, L.ldu, L.d_out);
  if (split) {  // single call: each tile makes its chunk's pieces; stage 2 waits for t
    d[0] = a;
    d[1] = b;
    return 2;
  }
  // input-piece tiles before each stage; each stage waits for its pieces,
  // the pieces of t wait for stage 1
  auto pieces = [&](const StageDesc& st, char* buf, int* ready) {
    StageDesc pc = st;
    const int64_t nch = piece_chunks(st.n_red);
    pc.kind = 1;
    pc.bfrag = reinterpret_cast<uint32_t*>(buf);
    pc.bsig = reinterpret_cast<int*>(buf + align_up((size_t)nch * 64 * T * kPieces * 16));
    pc.prep_tg = split ? 1 : (int)T;
    pc.prep_items = prep_items(T, split);
    pc.nrb = (int)cdiv(nch * (T / pc.prep_tg), pc.prep_items);  // tiles
    pc.rb_group = 1;
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

// Single calls: [error flag][next tile][exited][the linear's counters] (used
// only when the stream has no counter slot) then the linear's buffers; one
// persistent launch runs the two stages, each tile making its chunk's input
// pieces, the stage-2 tiles waiting for t.
size_t dec_workspace_bytes(const nq_lrb& L, int64_t T) {
  return align_up((size_t)(3 + dec_linear_counters(L, T, true)) * sizeof(int)) + dec_linear_bytes(L, T, true);
}

namespace {

// Counters of single calls, one slot per (device, stream).  Every launch
// leaves its counters at zero when it ends (the last workgroup out clears
// them), and the launches on one stream run one after another, so a stream's
// slot is zero whenever its next call starts: no clearing launch per call.
// The array is zero when the code object loads; each GPU has its own copy,
// whose address is looked up once per device.  A stream is given a slot on
// its first call and keeps it; past kSlots streams on a device, or for a layer
// with more counters than a slot holds, the counters live in the workspace and
// are cleared by a launch before the call.
constexpr int kSlots = 64, kSlotInts = 1024, kSlotDevices = 64;
static __device__ __align__(256) int g_slots[kSlots][kSlotInts];

struct SlotTable {
  int* base = nullptr;  // this device's copy of g_slots
  hipStream_t stream[kSlots] = {};
  int used = 0;
};
std::mutex g_slot_mu;
SlotTable g_slot_tab[kSlotDevices];

int* stream_slot(hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSlotDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_slot_mu);
  SlotTable& tab = g_slot_tab[dev];
  if (!tab.base) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_slots)) != hipSuccess || !p) return nullptr;
    tab.base = static_cast<int*>(p);
  }
  for (int i = 0; i < tab.used; ++i)
    if (tab.stream[i] == s) return tab.base + (size_t)i * kSlotInts;
  if (tab.used == kSlots) return nullptr;
  tab.stream[tab.used] = s;
  return tab.base + (size_t)(tab.used++) * kSlotInts;
}

}  // namespace

hipError_t launch_dec_linear(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                             hipStream_t s) {
  char* base = static_cast<char*>(ws);
  const int n_ints = 3 + dec_linear_counters(L, T, true);
  int* slot = n_ints <= kSlotInts ? stream_slot(s) : nullptr;
  int* ints = slot ? slot : reinterpret_cast<int*>(base);
  char* lin = base + align_up((size_t)n_ints * sizeof(int));
  LinearSched sched;
  const int nd = dec_stage_descs(L, x, xd, T, y, true, lin, ints + 3, sched.d);
  if (nd != 2) return hipErrorInvalidValue;
  int tiles = 0;
  for (int i = 0; i < kMaxLinearDescs; ++i) {  // entries past nd: empty (end = the last end)
    if (i < nd) {
      sched.d[i].tile0 = tiles;
      tiles += stage_tiles(sched.d[i]);
    } else {
      sched.d[i] = sched.d[nd - 1];
    }
    sched.end[i] = tiles;
  }
  hipError_t e;
  if (!slot && (e = launch_zero_ints(ints, n_ints, s)) != hipSuccess) return e;
  const int grid = (int)imin(tiles, dec_persistent_grid(T));
  switch (T) {
#define NQ_CASE(TT)                                                                                        \
  case TT: hipLaunchKernelGGL(dec_linear_kernel<TT>, dim3(grid), dim3(kMRows), 0, s, sched, ints, n_ints); break;
    NQ_CASE(1) NQ_CASE(2) NQ_CASE(3) NQ_CASE(4) NQ_CASE(5) NQ_CASE(6) NQ_CASE(7) NQ_CASE(8)
#undef NQ_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nq
