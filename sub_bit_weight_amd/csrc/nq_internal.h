// Internal declarations shared by the libnq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nq.h"

namespace nq {

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();
nq_status hip_status(hipError_t e, const char* what);

// ---------------------------------------------------------------- helpers
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
__host__ __device__ inline int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ inline int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }
constexpr int64_t kWordBits = 32;
constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------- validation and dispatch (nq_api.hip)
// Host-side argument checks of a packed layer and of a call's x, T, y; each
// sets the thread-local message and returns a non-OK status on failure.
nq_status check_lrb(const char* who, const nq_lrb* L);
nq_status check_io(const char* who, const nq_lrb* L, const void* x, nq_dtype xd, int64_t T, const float* y);
// Workspace and launch of one linear in the regime T selects (in_seq: an entry
// of a sequence plan, whose GEMMs never split their reductions).
size_t linear_workspace(const nq_lrb& L, int64_t T, bool in_seq = false);
hipError_t launch_linear(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                         hipStream_t s, bool in_seq = false);

// ---------------------------------------------------------------- launchers
// Each returns the hipError_t of its launch (hipGetLastError after the launch).

// Decode of a small layer (T <= 8) in one workgroup, no workspace (tiny.hip);
// tiny_fits says which layers take it.
bool tiny_fits(const nq_lrb& L, int64_t T);
hipError_t launch_tiny_linear(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, hipStream_t s);
hipError_t launch_pack(const float* src, int64_t n_out, int64_t n_red, int64_t so, int64_t sr,
                       uint32_t* dst, int64_t ld, hipStream_t s);
hipError_t launch_unpack(const uint32_t* bits, int64_t n_out, int64_t n_red, int64_t ld, float* dst,
                         hipStream_t s);
hipError_t launch_fill_words(uint32_t* dst, int64_t n, uint64_t seed, hipStream_t s);
hipError_t launch_reconstruct(const nq_lrb& L, float* w, hipStream_t s);

// Decode regime (T <= 8): split-reduction plan for one stage.
struct DecodePlan {
  int64_t n_out, n_red;
  int kchunk;   // reduction elements per workgroup (multiple of 32)
  int nks;      // number of reduction chunks
};
DecodePlan decode_plan(int64_t n_out, int64_t n_red, int64_t T);
size_t decode_workspace_bytes(const nq_lrb& L, int64_t T);
hipError_t launch_decode(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y,
                         void* ws, hipStream_t s);

// Decode regime, matrix-core kernels.  One stage of one linear:
//   out[t][o] = rowscale[o] * sum_e sign(o,e) * xin[t][e] * colscale[e]
struct StageDesc {
  const uint32_t* bits;   // words[e/32][o], row stride ld
  int64_t ld;
  const void* xin;        // [T][n_red], fp32 or bf16 (x_bf16)
  const float* colscale;  // [n_red] or null
  const float* rowscale;  // [n_rows] or null
  float* out;             // [T][n_rows]
  float* part;            // [nks][T][n_rows] partial sums (nks > 1)
  int* rb_count;          // [nrb] arrival counters (nks > 1)
  int* signal;            // incremented once per final row block (or null)
  const int* wait_ctr;    // wait for *wait_ctr >= wait_target before reading xin (or null)
  int wait_target;
  int n_rows, n_red;
  int kc, nks, nrb;       // reduction span per tile (elements), spans, row blocks
  int rb_group;           // kind 0: consecutive row blocks per tile (one span); kind 1: 1
  int x_bf16;
  int w_vec;              // bits 16-byte aligned, ld and n_rows multiples of 4: 16-byte word loads
  int kind;               // 0: stage tiles (nrb x nks); 1: input-piece tiles (nrb = tiles, nks = 1);
                          // 2: stage tiles of one chunk that make their own pieces (single calls)
  uint32_t* bfrag;        // matrix-core operand pieces of the stage input (written by kind 1, read by kind 0)
  int* bsig;              // per chunk and token: scale exponent of the pieces
  int prep_items;         // kind 1: (chunk, token group) work items per tile
  int prep_tg;            // kind 1: tokens per work item (1 or T)
  int tile0;              // first tile of this stage in a persistent schedule
};
// Tiles of a stage: kind 0, groups of rb_group row blocks per span; kind 1,
// nrb input-piece tiles (rb_group 1, nks 1).
__host__ __device__ inline int stage_tiles(const StageDesc& d) {
  return (d.nrb + d.rb_group - 1) / d.rb_group * d.nks;
}
struct StagePlan {
  int64_t n_rows, n_red;
  int kc, nks, nrb;
};
StagePlan dec_stage_plan(int64_t n_rows, int64_t n_red, int64_t T, int64_t kspan_max);
int64_t dec_single_span(int64_t n_rows, int64_t n_red, int64_t T);
size_t dec_workspace_bytes(const nq_lrb& L, int64_t T);
// split = true: single-call plan (reduction split over workgroups); false: sequence plan
size_t dec_linear_bytes(const nq_lrb& L, int64_t T, bool split);
int dec_linear_counters(const nq_lrb& L, int64_t T, bool split);
// Descriptors of one linear in dependency order (each waits only on earlier
// ones): sequences (split = false) pieces of x, stage 1, pieces of t, stage 2;
// single calls (split = true) stage 1, stage 2.  Returns their number.
constexpr int kMaxLinearDescs = 4;
int dec_stage_descs(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, bool split,
                    char* ws_linear, int* ctr_base, StageDesc* d);
hipError_t launch_dec_linear(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                             hipStream_t s);
hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t s);
int dec_persistent_grid(int64_t T);
// ints: [0] error flag, [1] next tile, [2] exited workgroups, [3..n_ints) counters;
// [1..n_ints) must be zero before the first run and are left zero by each run.
// tile_seg[i] (device) is the index in segs of the descriptor of tile i.
hipError_t launch_dec_persistent(const StageDesc* segs, const int* tile_seg, int ntiles, int* ints, int n_ints,
                                 int64_t T, int grid, hipStream_t s);

// Scale-only reconstruction: transposed sign words and the token reductions
// of the scale gradients (grads.hip).
hipError_t launch_transpose_signs(const uint32_t* src, int64_t n_out, int64_t n_red, int64_t ld, uint32_t* dst,
                                  int64_t ldt, hipStream_t s);
// Token chunks of the scale gradients' sums: kGradTokens tokens each, more
// when T > kGradTokens * kGradChunks.  T > kGradTokens needs
// scale_grads_partial_bytes of scratch (part) for the per-chunk sums.
constexpr int64_t kGradTokens = 64, kGradChunks = 1024;
size_t scale_grads_partial_bytes(int64_t T, int64_t d_in, int64_t d_out);
// ds2[j] (columns j < d_in) and ds1[i] (columns d_in + i) of columns
// [c_begin, c_end): the sum of part[q][column] over q < nchunks in order.
hipError_t launch_scale_grads_sums(const float* part, int64_t nchunks, int64_t d_in, int64_t d_out, float* ds1,
                                   float* ds2, int64_t c_begin, int64_t c_end, hipStream_t s);
hipError_t launch_scale_grads_finish(const void* x, nq_dtype xd, const void* g, nq_dtype gd, const float* u,
                                     const float* b, const float* s2, int64_t T, int64_t d_in, int64_t d_out, float* dx,
                                     float* part, float* ds1, float* ds2, int64_t c_begin, int64_t c_end,
                                     hipStream_t s);

// Magnitude balancing and scale extraction (balance.hip).  workspace: at
// least balance_workspace_bytes(d_out, d_in), 256-byte aligned.
// Refinement forward with the signs taken from the fp32 latents as they load
// (latent.hip), for T <= kLatMaxT: workspace bytes, whether the launch grid
// fits, and the launch (zeroes its counters, then the two stages).
constexpr int kLatMaxT = 8;
size_t lat_forward_bytes(int64_t d_out, int64_t d_in, int64_t r, int64_t T);
bool lat_forward_fits(int64_t d_out, int64_t d_in, int64_t r, int64_t T);
hipError_t launch_lat_forward(const float* u_lat, int64_t ldu, const float* v_lat, int64_t ldv, int64_t d_out,
                              int64_t d_in, int64_t r, const float* s1, const float* s2, const void* x, bool x_bf16,
                              int64_t T, float* y, void* ws, hipStream_t s);

size_t balance_workspace_bytes(int64_t d_out, int64_t d_in);
hipError_t launch_balance(const float* uh, int64_t ldu, const float* vh, int64_t ldv, int64_t d_out, int64_t d_in,
                          int64_t r, float* uo, float* vo, float* s1, float* s2, float* eta, void* workspace,
                          hipStream_t s);

// Matrix-core regime (T > 8).
// split = false: never split a GEMM's reduction (entries of a sequence run
// concurrently and fill the chip together).
size_t prefill_workspace_bytes(const nq_lrb& L, int64_t T, bool split = true);
// A product with the stage-2 output: for every 128-row block q of the output
// (tokens 128q ..) and column n, psum[q * ldp + n] = sum over the block's rows
// m of pm[m][n] * v[m][n], v the output before the row scale s1 (pm: [T][d_out],
// fp32 or bf16).  The output itself is written only when y is not null.
struct ProdEpilogue {
  const void* pm;
  bool pm_bf16;
  float* psum;
  int64_t ldp;
};
int64_t prefill_row_blocks(int64_t T);  // the 128-row blocks of a T-token output
hipError_t launch_prefill(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y,
                          void* ws, hipStream_t s, bool split = true, const ProdEpilogue* pe = nullptr);

}  // namespace nq
