/*
 * nq.h -- C ABI of libnq, the MI355X (gfx950) library for NanoQuant's
 * low-rank binary (LRB) linear layer.
 *
 * The layer (research.samsung.com blog "NanoQuant: Efficient Sub-1-Bit
 * Quantization of Large Language Models", section 2 "Problem Formulation and
 * Background", subsection "Low-Rank Binary Factorization", the factorization
 * equation) approximates a weight matrix W (d_out x d_in) by
 *
 *     W[i,j] = s1[i] * (sum_k U[i,k] * V[j,k]) * s2[j],
 *
 * with U in {-1,+1}^(d_out x r), V in {-1,+1}^(d_in x r) and real scale vectors
 * s1 (d_out) and s2 (d_in).  The library evaluates y = W x for T tokens in the
 * factored order y = s1 (.) U (V^T (s2 (.) x)) without forming W.
 *
 * Conventions shared by every call:
 *  - Every pointer argument except `const nq_lrb*`, `nq_seq*` and the arrays of
 *    nq_seq_create is DEVICE memory of the current HIP device.  The caller
 *    allocates and frees all device buffers; libnq keeps no device allocation.
 *  - Every call that launches work enqueues it on `stream` (a hipStream_t
 *    passed as void*; NULL is the default stream) and returns without waiting.
 *    Device faults surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call.  A failed check
 *    returns a non-zero status, launches nothing, and sets a thread-local
 *    message readable with nq_last_error().  No C++ exception crosses the ABI.
 *  - Buffers passed to one call must not overlap unless stated.
 *  - Calls are re-entrant; different streams may be used concurrently.
 *
 * Sign-word layout (the "packed integer format"; the pages say only that the
 * frozen binary factors are packed into integer formats, section 3 "Phase 3:
 * Scale-Only Model Reconstruction"):
 *  A stage with n_out outputs and a reduction of length n_red is stored as
 *  words[w][o], w < ceil(n_red/32), o < n_out, with row stride ld >= n_out
 *  (in 32-bit words).  Bit b of words[w][o] is 1 exactly when the sign of
 *  element (o, 32w+b) is -1.  Bits for 32w+b >= n_red are 0.
 *    U   is stored with outputs i < d_out and reduction k < r    (words along r),
 *    V^T is stored with outputs k < r     and reduction j < d_in (words along d_in).
 *  With dimensions that are multiples of 32 and ld = n_out the two buffers hold
 *  exactly r(d_out+d_in) bits, the storage the pages give for the signs
 *  (section 2, the sentence after the factorization equation).
 */
#ifndef NQ_H
#define NQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NQ_OK = 0,
  NQ_ERR_ARG = 1,         /* invalid argument (null pointer, bad size, bad stride) */
  NQ_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. a shape limit)        */
  NQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required           */
  NQ_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed           */
} nq_status;

/* Element type of an activation buffer: NQ_F32 or NQ_BF16.  A plain 32-bit
   integer rather than an enum type, so that any value a caller passes is
   well defined in the library (anything else is rejected with NQ_ERR_ARG). */
typedef int32_t nq_dtype;
enum { NQ_F32 = 0, NQ_BF16 = 1 };

/* One packed LRB matrix.  A host struct, read only during a call. */
typedef struct {
  int64_t d_out, d_in, r;   /* all >= 1 */
  const uint32_t* u_bits;   /* [ceil(r/32)][ldu] words, ldu >= d_out   */
  int64_t ldu;
  const uint32_t* vt_bits;  /* [ceil(d_in/32)][ldv] words, ldv >= r    */
  int64_t ldv;
  const float* s1;          /* [d_out] fp32 */
  const float* s2;          /* [d_in]  fp32 */
} nq_lrb;

/*
 * nq_pack_signs -- pack the signs of a real matrix into sign words.
 * The binary factors are sign(U) and sign(V) of real latent factors (section 3
 * "Step 3: Factorized Component Refinement"); once frozen they are packed into
 * integer formats (section 3 "Phase 3").
 *   dst[w*ld + o] bit b = (src[o*stride_out + (32w+b)*stride_red] < 0.0f)
 * for o < n_out, 32w+b < n_red; padding bits are 0; dst columns n_out..ld-1 are
 * not written.  sign() reads -1 only for values < 0 under IEEE comparison:
 * +0, -0 and NaN pack as +1.
 *   U latent [d_out][r]:  n_out=d_out, n_red=r,    stride_out=r, stride_red=1
 *   V latent [d_in][r]:   n_out=r,     n_red=d_in, stride_out=1, stride_red=r
 * Errors: NQ_ERR_ARG for null pointers, n_out or n_red < 1, strides < 1,
 * ld < n_out.
 */
nq_status nq_pack_signs(const float* src, int64_t n_out, int64_t n_red,
                        int64_t stride_out, int64_t stride_red,
                        uint32_t* dst, int64_t ld, void* stream);

/*
 * nq_unpack_signs -- inverse of nq_pack_signs for checking the layout.
 *   dst[o*n_red + e] = bit(words[e/32][o], e%32) ? -1.0f : +1.0f
 * dst is [n_out][n_red] fp32, row-major.  Padding bits are ignored.
 * Errors: NQ_ERR_ARG as for nq_pack_signs.
 */
nq_status nq_unpack_signs(const uint32_t* bits, int64_t n_out, int64_t n_red, int64_t ld,
                          float* dst, void* stream);

/*
 * nq_lrb_workspace_bytes -- device workspace nq_lrb_linear needs for T tokens
 * (the rank-r intermediate t and split-reduction partial sums).  Returns 0 if
 * the arguments are invalid (see nq_lrb_linear).
 */
size_t nq_lrb_workspace_bytes(const nq_lrb* L, int64_t T);

/*
 * nq_lrb_linear -- y = s1 (.) U (V^T (s2 (.) x)) for T tokens.
 * The pages run binary GEMV kernels for token-by-token decoding and binary GEMM
 * kernels for batches (section 4 "Results", subsection "Inference Performance").
 *   x: [T][d_in] row-major, fp32 or bf16 (x_dtype);  y: [T][d_out] fp32.
 *   workspace: at least nq_lrb_workspace_bytes(L, T) bytes, 256-byte aligned.
 * Regimes: T <= 8 runs the decode kernels: each token's stage input is scaled
 * per chunk of 1024 elements by a power of two and split into four fp8 pieces
 * that carry it to within 2^-16 of the chunk's largest value (about 2^-20 in
 * practice, ~4e-7 relative per stage), multiplied by
 * the exact +-1 signs on the matrix cores with fp32 accumulation;
 * T > 8 runs the GEMM kernels: each token row of a stage's activations
 * is scaled by an exact power of two and rounded to fp16 (two fp16 terms for
 * fp32 x), multiplied by the exact +-1 signs with fp32 accumulation, and
 * scaled back.
 * Small layers at T <= 8 (T*d_in <= 2048 and T*r <= 512 with both rounded up
 * to whole words, d_out <= 1024) run in one workgroup instead: z, t and y as
 * fp32 sums in index order with the exact signs (set NQ_DECODE_TINY=0 in the
 * environment to keep them on the decode kernels above; sequence plans always
 * use those, so a sequence entry and a single call of such a layer may differ
 * in the last bits).
 * y is fully overwritten.  Summation order is fixed: results are run-to-run
 * deterministic, but not bitwise equal across regimes.
 * The decode kernels of a single call keep their dependency counters in a
 * small array of the library, one slot per stream (up to 64 streams per
 * device; each launch leaves its slot cleared, so calls need no clearing
 * launch): calls on different streams may overlap, and a call captured into a
 * graph keeps the slot of the stream it was captured on, so its replays must
 * not overlap other calls made on that stream.
 * Errors: NQ_ERR_ARG for null pointers, dims < 1, ldu < d_out, ldv < r, T < 1,
 * an unknown dtype or a misaligned pointer (x, y: 4 bytes; bits, scales: 4
 * bytes); NQ_ERR_UNSUPPORTED when r > 2^24, d_out or d_in > 2^31, or a
 * sign-word buffer exceeds 2 GiB; NQ_ERR_WORKSPACE when workspace_bytes is too
 * small; NQ_ERR_HIP when a launch fails.
 */
nq_status nq_lrb_linear(const nq_lrb* L, const void* x, nq_dtype x_dtype, int64_t T,
                        float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nq_reconstruct -- the dense W for checking (the factorization equation):
 *   w[i*d_in + j] = fl32( fl32(s1[i] * m) * s2[j] ),  m = sum_k U[i,k] V[j,k]
 * with m an exact integer and both products rounded to nearest even, so the
 * result is unique bit for bit.  w is [d_out][d_in] fp32.
 * Errors: NQ_ERR_ARG as for nq_lrb_linear; NQ_ERR_UNSUPPORTED for r > 2^24.
 */
nq_status nq_reconstruct(const nq_lrb* L, float* w, void* stream);

/*
 * nq_storage_bits -- storage of one LRB matrix in bits: r(d_out+d_in) signs
 * plus (d_out+d_in) fp32 scales (section 2, the sentence after the
 * factorization equation).  Returns 0 for non-positive arguments.  Host only.
 */
uint64_t nq_storage_bits(int64_t d_out, int64_t d_in, int64_t r);

/*
 * Sequences of independent LRB linears (e.g. every linear of a decoder stack)
 * run as one schedule.  Running the sequence is equivalent to calling
 * nq_lrb_linear on each entry in order, except that entries may run
 * concurrently (no entry's input may be another entry's output, and no two
 * entries' outputs may overlap) and that in the matrix-core regime an entry
 * never splits its reduction, so its sums may be ordered differently from a
 * single call (equal up to rounding; each plan is run-to-run deterministic).
 *
 * nq_seq_create: host-only planning.  `layers`, `xs`, `ys` are host arrays of
 *   n entries (the nq_lrb structs are copied; xs[i], ys[i] are device
 *   pointers).  All entries share T and x_dtype.  The decode regime (T <= 8)
 *   runs as one persistent kernel; T > 8 runs the per-entry kernels
 *   round-robin on three streams owned by the plan (created on the first run
 *   on the device current then), each entry with its own part of the
 *   workspace.  Errors: as for nq_lrb_linear, per entry.
 * nq_seq_workspace_bytes: device workspace the plan needs.
 * nq_seq_run: runs the whole sequence, ordered after the work already on
 *   `stream`; work queued on `stream` afterwards waits for all of it.  The
 *   workspace must stay the same buffer across runs of one plan (the first
 *   decode-regime run uploads the schedule into it, synchronising `stream`
 *   once) and must not be shared by plans running concurrently.  In the decode
 *   regime the first 4 bytes of the workspace are a device error word: 0, or
 *   non-zero (sticky) if a dependency wait inside the kernel gave up; read it
 *   after synchronising.
 * nq_seq_destroy: frees the plan (and its streams).
 */
typedef struct nq_seq nq_seq;
nq_status nq_seq_create(const nq_lrb* layers, const void* const* xs, float* const* ys, int64_t n,
                        nq_dtype x_dtype, int64_t T, nq_seq** out);
size_t nq_seq_workspace_bytes(const nq_seq* s);
nq_status nq_seq_run(nq_seq* s, void* workspace, size_t workspace_bytes, void* stream);
void nq_seq_destroy(nq_seq* s);

/*
 * Scale-only reconstruction (section 3 "Phase 3: Scale-Only Model
 * Reconstruction": with the binary factors frozen only s1 and s2 are tuned).
 *
 * nq_transpose_signs -- sign words of the transposed sign matrix.  src holds an
 *   n_out x n_red sign matrix S in the layout above (row stride ld); dst
 *   receives S^T, i.e. n_red outputs with a reduction over n_out:
 *     bit b of dst[w*ldt + e] = bit (e%32) of src[(e/32)*ld + 32w+b]
 *   for e < n_red, 32w+b < n_out; padding bits are 0; columns n_red..ldt-1 are
 *   not written.  dst is [ceil(n_out/32)][ldt] words, ldt >= n_red, and must
 *   not overlap src.  The transposed layer's words are
 *     ut_bits = nq_transpose_signs(u_bits,  n_out=d_out, n_red=r,    ld=ldu)  [ceil(d_out/32)][ldut >= r]
 *     v_bits  = nq_transpose_signs(vt_bits, n_out=r,     n_red=d_in, ld=ldv)  [ceil(r/32)][ldvv >= d_in]
 *   Errors: NQ_ERR_ARG for null pointers, sizes < 1, ld < n_out, ldt < n_red,
 *   misaligned pointers; NQ_ERR_UNSUPPORTED if a buffer exceeds 2 GiB.
 *
 * nq_lrb_scale_grads -- for y = W x (W as in nq_lrb_linear) and the gradient
 *   g = dL/dy of a loss, the gradients with respect to the input and the scales:
 *     dx[t][j] = sum_i W[i][j] g[t][i]
 *     ds1[i]   = sum_t g[t][i] * (U V^T (s2 (.) x_t))_i
 *     ds2[j]   = sum_t x[t][j] * (V U^T (s1 (.) g_t))_j
 *   x: [T][d_in] fp32 or bf16 (x_dtype); g: [T][d_out] fp32 or bf16
 *   (g_dtype); dx: [T][d_in] fp32; ds1: [d_out] fp32; ds2: [d_in] fp32
 *   (overwritten, not accumulated).
 *   ut_bits/v_bits: the transposed layer's words from nq_transpose_signs.
 *   Both products run through the kernels of nq_lrb_linear (decode regime for
 *   T <= 8, GEMM regime above, with the same arithmetic); the token sums are
 *   fp32 in token order (deterministic).  The two products run concurrently:
 *   the transposed one on a second stream that the library makes on a
 *   device's first call and keeps, forked from and joined back to `stream`
 *   (all of the call's work is ordered after what `stream` holds at the call,
 *   and what is queued on `stream` afterwards is ordered after all of it).
 *   workspace: at least nq_lrb_scale_grads_workspace_bytes(L, T) bytes,
 *   256-byte aligned.  Errors: as for nq_lrb_linear, for L and for the
 *   transposed layer's words; NQ_ERR_ARG for an unknown g_dtype or a null or
 *   misaligned g, ds1 or ds2.
 */
nq_status nq_transpose_signs(const uint32_t* src, int64_t n_out, int64_t n_red, int64_t ld,
                             uint32_t* dst, int64_t ldt, void* stream);
size_t nq_lrb_scale_grads_workspace_bytes(const nq_lrb* L, int64_t T);
nq_status nq_lrb_scale_grads(const nq_lrb* L, const uint32_t* ut_bits, int64_t ldut,
                             const uint32_t* v_bits, int64_t ldvv, const void* x, nq_dtype x_dtype,
                             const void* g, nq_dtype g_dtype, int64_t T, float* dx, float* ds1,
                             float* ds2, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nq_lrb_scale_grads_batch -- nq_lrb_scale_grads for n independent linears in
 * one call (the linears of a decoder layer, say: section 3 "Phase 3: Scale-Only
 * Model Reconstruction" tunes every layer's scales against the model's
 * outputs).  Linear i takes L[i], ut_bits[i]/ldut[i], v_bits[i]/ldvv[i], x[i],
 * g[i] and writes dx[i], ds1[i], ds2[i], each as in nq_lrb_scale_grads; all
 * share T, x_dtype and g_dtype.  The results equal n calls of
 * nq_lrb_scale_grads bit for bit.  With T > 8 the 2n products (forward and
 * transposed of each linear) run round-robin on three streams that the library
 * makes on a device's first such call and keeps, forked from and joined back
 * to `stream`, so that one product's prep kernels and partly filled GEMM waves
 * run beside another's GEMMs; with T <= 8 the linears run one after another.
 *   workspace: at least nq_lrb_scale_grads_batch_workspace_bytes(n, L, T)
 *   bytes, 256-byte aligned; the query returns 0 for invalid arguments.
 * Errors: as for nq_lrb_scale_grads, for each linear (the message names it);
 * NQ_ERR_ARG for n < 1 or a null array.
 */
size_t nq_lrb_scale_grads_batch_workspace_bytes(int64_t n, const nq_lrb* L, int64_t T);
nq_status nq_lrb_scale_grads_batch(int64_t n, const nq_lrb* L, const uint32_t* const* ut_bits,
                                   const int64_t* ldut, const uint32_t* const* v_bits, const int64_t* ldvv,
                                   const void* const* x, nq_dtype x_dtype, const void* const* g,
                                   nq_dtype g_dtype, int64_t T, float* const* dx, float* const* ds1,
                                   float* const* ds2, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nq_lrb_linear_latent -- the layer with the signs taken from real latent
 *   factors at the call: y = s1 (.) sign(U)(sign(V)^T (s2 (.) x)), the forward
 *   pass of the factorized component refinement (section 3 "Step 3:
 *   Factorized Component Refinement", where the binary factors are sign(U) and
 *   sign(V) of latents that the refinement keeps updating).  sign() as in
 *   nq_pack_signs (-1 only for values < 0).  T <= 8: the two stages read the
 *   fp32 latents once and apply sign() as they load (no packed words), fp32
 *   sums in a fixed order.  T > 8: the latents are packed into the workspace,
 *   then the packed layer runs as in nq_lrb_linear: y equals nq_pack_signs
 *   followed by nq_lrb_linear bit for bit.
 *   u_lat: [d_out][ldu_lat] fp32 (row i's r entries first), v_lat:
 *   [d_in][ldv_lat] fp32; s1, s2, x, x_dtype, T, y as for nq_lrb_linear.
 *   workspace: at least nq_lrb_latent_workspace_bytes(d_out, d_in, r, T)
 *   bytes, 256-byte aligned.  Errors: NQ_ERR_ARG for null or misaligned
 *   latents, sizes < 1, ldu_lat or ldv_lat < r; NQ_ERR_UNSUPPORTED at T <= 8
 *   for shapes whose launch grid would exceed 65535 reduction spans;
 *   otherwise as nq_lrb_linear.
 */
size_t nq_lrb_latent_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r, int64_t T);
nq_status nq_lrb_linear_latent(const float* u_lat, int64_t ldu_lat, const float* v_lat,
                               int64_t ldv_lat, int64_t d_out, int64_t d_in, int64_t r,
                               const float* s1, const float* s2, const void* x, nq_dtype x_dtype,
                               int64_t T, float* y, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Magnitude balancing and scale extraction (section 3, "Magnitude Balancing
 * and Scale Extraction"): the step between the ADMM factorization and the
 * sign packing.  The latent factors can be rescaled inversely without
 * changing their product; balancing equalises their Frobenius norms and the
 * scale vectors are the balanced factors' per-row mean absolute values.
 *
 * nq_balance_factors --
 *     eta = sqrt(||V_hat||_F / ||U_hat||_F)      (1 if either norm is 0)
 *     U = eta * U_hat,   V = V_hat / eta
 *     s1[i] = mean_k |U[i][k]|,   s2[j] = mean_k |V[j][k]|
 *   u_hat: [d_out][ldu] fp32, row i's r entries first (the U latent layout of
 *   nq_pack_signs when ldu = r); v_hat: [d_in][ldv] likewise.  u_out, v_out:
 *   both null (scales only) or both given, with the inputs' strides; each may
 *   be its input (in place) but must not otherwise overlap anything.  s1:
 *   [d_out], s2: [d_in], eta: [1] fp32 device.  Sums of |.| are fp32, sums of
 *   squares and the norms fp64 (every finite fp32 latent), all in a fixed order
 *   (deterministic).  Signs are unchanged (eta > 0), so
 *   nq_pack_signs may read either the latents or the balanced factors.
 *   workspace: at least nq_balance_workspace_bytes(d_out, d_in) bytes,
 *   256-byte aligned.  Errors: NQ_ERR_ARG for null inputs, scales or eta,
 *   sizes < 1, ldu or ldv < r, only one of u_out / v_out, pointers not 4-byte
 *   aligned; NQ_ERR_WORKSPACE for a missing or short workspace.
 */
size_t nq_balance_workspace_bytes(int64_t d_out, int64_t d_in);
nq_status nq_balance_factors(const float* u_hat, int64_t d_out, int64_t ldu, const float* v_hat,
                             int64_t d_in, int64_t ldv, int64_t r, float* u_out, float* v_out,
                             float* s1, float* s2, float* eta, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * nq_fill_random_words -- synthetic sign words for large benchmark matrices:
 *   dst[i] = low 32 bits of SplitMix64(seed, i), i < n, where SplitMix64(seed,
 *   i) is output number i+1 of the SplitMix64 stream started at `seed`
 *   (Steele, Lea, Flood 2014).  Uniform words give iid +-1 signs.  This is an
 *   input generator, not part of the layer.  Errors: NQ_ERR_ARG for a null
 *   dst or n < 0.
 */
nq_status nq_fill_random_words(uint32_t* dst, int64_t n, uint64_t seed, void* stream);

/*
 * nq_lrb_linear_noalloc -- nq_lrb_linear without a caller workspace and
 *   without any device allocation, for callers that cannot allocate device
 *   memory: code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc.  The caller still passes x and y; the workspace is a
 *   fixed array of NQ_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy
 *   per GPU, held from the first use on that GPU until the process ends.
 *   Arguments, results and regimes are those of nq_lrb_linear (same kernels,
 *   bit-identical y).  Every call on one GPU uses that GPU's one array, so
 *   calls on one GPU whose executions overlap (different streams or threads
 *   without ordering between them) race and give wrong results; order them.
 *   The decode regime clears the array's counters with a fill kernel at the
 *   start of each call (no memset).  16 MiB covers the decode regime (T <= 8)
 *   at every Llama-2-70B linear shape up to 2 bits/weight and small GEMM
 *   batches.  Errors: as for nq_lrb_linear; NQ_ERR_UNSUPPORTED when the call
 *   needs more workspace than the array holds (nq_lrb_workspace_bytes(L, T) >
 *   NQ_NOALLOC_SCRATCH_BYTES), checked before any HIP call.
 */
#define NQ_NOALLOC_SCRATCH_BYTES (16u << 20)
nq_status nq_lrb_linear_noalloc(const nq_lrb* L, const void* x, nq_dtype x_dtype, int64_t T, float* y,
                                void* stream);

/* Thread-local message for the last non-OK status of this thread ("" if none). */
const char* nq_last_error(void);

/* Library version string. */
const char* nq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NQ_H */
