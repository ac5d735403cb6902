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

// ---------------------------------------------------------------- launchers
// Each returns the hipError_t of its launch (hipGetLastError after the launch).
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

// Matrix-core regime (T > 8).
size_t prefill_workspace_bytes(const nq_lrb& L, int64_t T);
hipError_t launch_prefill(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y,
                          void* ws, hipStream_t s);

}  // namespace nq
