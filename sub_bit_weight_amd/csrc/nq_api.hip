// C ABI of libnq: argument validation, status codes and dispatch.
// Every check runs on the host before any HIP call; no exception crosses the ABI.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <array>
#include <vector>

#include "nq_internal.h"

namespace nq {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

nq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return NQ_OK;
  set_error("%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return NQ_ERR_HIP;
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

nq_status check_words(const char* who, const void* p, int64_t n_out, int64_t n_red, int64_t ld) {
  if (!p) return set_error("%s: null pointer", who), NQ_ERR_ARG;
  if (n_out < 1 || n_red < 1) return set_error("%s: n_out=%lld n_red=%lld must be >= 1", who, (long long)n_out, (long long)n_red), NQ_ERR_ARG;
  if (ld < n_out) return set_error("%s: ld=%lld < n_out=%lld", who, (long long)ld, (long long)n_out), NQ_ERR_ARG;
  if (!aligned(p, 4)) return set_error("%s: pointer not 4-byte aligned", who), NQ_ERR_ARG;
  return NQ_OK;
}

}  // namespace

nq_status check_lrb(const char* who, const nq_lrb* L) {
  if (!L) return set_error("%s: null layer", who), NQ_ERR_ARG;
  if (L->d_out < 1 || L->d_in < 1 || L->r < 1)
    return set_error("%s: d_out=%lld d_in=%lld r=%lld must be >= 1", who, (long long)L->d_out,
                     (long long)L->d_in, (long long)L->r), NQ_ERR_ARG;
  if (L->r > (int64_t(1) << 24))
    return set_error("%s: r=%lld exceeds 2^24", who, (long long)L->r), NQ_ERR_UNSUPPORTED;
  if (L->d_out > (int64_t(1) << 31) || L->d_in > (int64_t(1) << 31))
    return set_error("%s: dimension exceeds 2^31", who), NQ_ERR_UNSUPPORTED;
  // sign-word buffers are addressed with 32-bit byte offsets inside the kernels
  if (cdiv(L->r, kWordBits) * L->ldu >= (int64_t(1) << 29) || cdiv(L->d_in, kWordBits) * L->ldv >= (int64_t(1) << 29))
    return set_error("%s: a sign-word buffer exceeds 2 GiB", who), NQ_ERR_UNSUPPORTED;
  nq_status st;
  if ((st = check_words(who, L->u_bits, L->d_out, L->r, L->ldu)) != NQ_OK) return st;
  if ((st = check_words(who, L->vt_bits, L->r, L->d_in, L->ldv)) != NQ_OK) return st;
  if (!L->s1 || !L->s2) return set_error("%s: null scale vector", who), NQ_ERR_ARG;
  if (!aligned(L->s1, 4) || !aligned(L->s2, 4)) return set_error("%s: scale vector not 4-byte aligned", who), NQ_ERR_ARG;
  return NQ_OK;
}

nq_status check_io(const char* who, const nq_lrb* L, const void* x, nq_dtype xd, int64_t T, const float* y) {
  if (T < 1) return set_error("%s: T=%lld must be >= 1", who, (long long)T), NQ_ERR_ARG;
  if (T > (int64_t(1) << 24)) return set_error("%s: T=%lld too large", who, (long long)T), NQ_ERR_UNSUPPORTED;
  if (xd != NQ_F32 && xd != NQ_BF16) return set_error("%s: unknown x dtype %d", who, (int)xd), NQ_ERR_ARG;
  if (!x || !y) return set_error("%s: null x or y", who), NQ_ERR_ARG;
  if (!aligned(x, xd == NQ_F32 ? 4 : 2) || !aligned(y, 4))
    return set_error("%s: x or y misaligned", who), NQ_ERR_ARG;
  (void)L;
  return NQ_OK;
}

constexpr int64_t kDecodeMaxT = 8;
constexpr int64_t kSeqLanes = 3;  // streams of a sequence plan in the matrix-core regime

// NQ_DECODE_VARIANT=xor selects the per-weight sign-XOR decode kernels (kept
// for comparison); the default is the table-lookup kernels.
bool decode_xor() {
  const char* e = getenv("NQ_DECODE_VARIANT");
  return e && strcmp(e, "xor") == 0;
}

// NQ_DECODE_TINY=0 keeps small layers on the multi-workgroup decode kernels
// (read at each call, like NQ_DECODE_VARIANT: tests compare the two paths).
bool tiny_enabled() {
  const char* e = getenv("NQ_DECODE_TINY");
  return !(e && strcmp(e, "0") == 0);
}

// in_seq: the linear is an entry of a sequence plan, whose entries run
// concurrently; the matrix-core regime then never splits a reduction (the
// entries fill the chip together, and a split only adds partial-sum traffic).
size_t linear_workspace(const nq_lrb& L, int64_t T, bool in_seq) {
  if (T > kDecodeMaxT) return prefill_workspace_bytes(L, T, !in_seq);
  return decode_xor() ? decode_workspace_bytes(L, T) : dec_workspace_bytes(L, T);
}

hipError_t launch_linear(const nq_lrb& L, const void* x, nq_dtype xd, int64_t T, float* y, void* ws,
                         hipStream_t s, bool in_seq) {
  if (T > kDecodeMaxT) return launch_prefill(L, x, xd, T, y, ws, s, !in_seq);
  if (decode_xor()) return launch_decode(L, x, xd, T, y, ws, s);
  if (tiny_enabled() && tiny_fits(L, T)) return launch_tiny_linear(L, x, xd, T, y, s);  // one workgroup

  return launch_dec_linear(L, x, xd, T, y, ws, s);
}

namespace {

// The transposed layer W^T = s2 (.) V U^T (.) s1 as an LRB matrix.
nq_lrb adjoint_layer(const nq_lrb& L, const uint32_t* ut_bits, int64_t ldut, const uint32_t* v_bits, int64_t ldvv) {
  nq_lrb A;
  A.d_out = L.d_in;
  A.d_in = L.d_out;
  A.r = L.r;
  A.u_bits = v_bits;  // outputs j < d_in, words along r
  A.ldu = ldvv;
  A.vt_bits = ut_bits;  // outputs k < r, words along d_out
  A.ldv = ldut;
  A.s1 = L.s2;
  A.s2 = L.s1;
  return A;
}

// Workspace of nq_lrb_scale_grads: [u: T x d_out][b: T x d_in][per-chunk
// partial sums][the forward product's linear workspace][the transposed
// product's] (the two products run concurrently).  In the matrix-core regime
// the partial sums are per 128-row block of the GEMM outputs and u, b are
// not stored.
struct ScaleGradsLayout {
  size_t off_u, off_b, off_part, off_lin, off_lin_t, bytes;
};
ScaleGradsLayout scale_grads_layout(const nq_lrb& L, int64_t T) {
  ScaleGradsLayout g;
  g.off_u = 0;
  g.off_b = align_up((size_t)T * L.d_out * sizeof(float));
  g.off_part = g.off_b + align_up((size_t)T * L.d_in * sizeof(float));
  const size_t part = std::max(scale_grads_partial_bytes(T, L.d_in, L.d_out),
                               T > kDecodeMaxT ? (size_t)prefill_row_blocks(T) * (L.d_in + L.d_out) * sizeof(float)
                                               : (size_t)0);
  g.off_lin = g.off_part + align_up(part);
  const nq_lrb A = adjoint_layer(L, L.vt_bits, L.r, L.u_bits, L.d_in);  // sizes only
  g.off_lin_t = g.off_lin + align_up(linear_workspace(L, T));
  g.bytes = g.off_lin_t + linear_workspace(A, T);
  return g;
}

// A second stream per device for calls made of two independent products,
// with the events that fork it from and join it back to the caller's stream.
// Made on a device's first such call and kept until the process ends; the
// mutex keeps one call's fork, launches and join together.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::vector<SideStream> g_side;

hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)g_side.size() <= dev) g_side.resize(dev + 1);
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);  // default priority
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    ss.s = s, ss.fork = f, ss.join = j;
  }
  *out = &ss;
  return hipSuccess;
}

// Streams per device for batched calls (entries round-robin on them), with a
// fork event and one join event per stream; made on first use and kept, under
// the same mutex as the side stream.
constexpr int kBatchLanes = 3;
struct LaneSet {
  hipStream_t s[kBatchLanes] = {};
  hipEvent_t fork = nullptr, join[kBatchLanes] = {};
};
std::vector<LaneSet> g_lanes;

hipError_t lane_set(LaneSet** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)g_lanes.size() <= dev) g_lanes.resize(dev + 1);
  LaneSet& ls = g_lanes[dev];
  if (!ls.fork) {
    LaneSet n;
    for (int l = 0; l < kBatchLanes && e == hipSuccess; ++l) {
      e = hipStreamCreateWithFlags(&n.s[l], hipStreamNonBlocking);  // default priority
      if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join[l], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    ls = n;
  }
  *out = &ls;
  return hipSuccess;
}

// Workspace of nq_lrb_scale_grads_batch in the matrix-core regime: per stream
// [block partial sums][one linear workspace], each sized for the largest of
// the batch's linears.
struct BatchGradsLayout {
  size_t off_part, off_lin, lane, bytes;
};
BatchGradsLayout batch_grads_layout(const nq_lrb* L, int64_t n, int64_t T) {
  size_t part = 0, lin = 0;
  for (int64_t i = 0; i < n; ++i) {
    part = std::max(part, (size_t)prefill_row_blocks(T) * (L[i].d_in + L[i].d_out) * sizeof(float));
    const nq_lrb A = adjoint_layer(L[i], L[i].vt_bits, L[i].r, L[i].u_bits, L[i].d_in);  // sizes only
    lin = std::max(lin, std::max(linear_workspace(L[i], T), linear_workspace(A, T)));
  }
  BatchGradsLayout b;
  b.off_part = 0;
  b.off_lin = align_up(part);
  b.lane = align_up(b.off_lin + lin);
  b.bytes = kBatchLanes * b.lane;
  return b;
}

// Checks of one linear's scale-gradient arguments; the transposed layer into A.
nq_status check_grads(const char* who, const nq_lrb* L, const uint32_t* ut_bits, int64_t ldut, const uint32_t* v_bits,
                      int64_t ldvv, const void* x, nq_dtype x_dtype, const void* g, nq_dtype g_dtype, int64_t T,
                      const float* dx, const float* ds1, const float* ds2, nq_lrb* A) {
  nq_status st = check_lrb(who, L);
  if (st != NQ_OK) return st;
  // the transposed layer W^T: outputs d_in, reduction d_out; its U is V (words
  // along r), its V^T is U^T (words along d_out); its scales are s2 and s1
  *A = adjoint_layer(*L, ut_bits, ldut, v_bits, ldvv);
  if ((st = check_lrb("nq_lrb_scale_grads (transposed sign words)", A)) != NQ_OK) return st;
  if ((st = check_io(who, L, x, x_dtype, T, dx)) != NQ_OK) return st;
  if (g_dtype != NQ_F32 && g_dtype != NQ_BF16) return set_error("%s: unknown g dtype %d", who, (int)g_dtype), NQ_ERR_ARG;
  if (!g || !ds1 || !ds2) return set_error("%s: null g, ds1 or ds2", who), NQ_ERR_ARG;
  if (!aligned(g, g_dtype == NQ_F32 ? 4 : 2) || !aligned(ds1, 4) || !aligned(ds2, 4))
    return set_error("%s: g, ds1 or ds2 misaligned", who), NQ_ERR_ARG;
  return NQ_OK;
}

// One product chain of the matrix-core regime on stream s: the forward product
// (transposed = false: u only summed against g into ds1) or the transposed one
// (dx written, x (.) b summed into ds2), then its blocks added in order.
hipError_t enqueue_grads_chain(const nq_lrb& L, const nq_lrb& A, bool transposed, const void* x, nq_dtype x_dtype,
                               const void* g, nq_dtype g_dtype, int64_t T, float* dx, float* ds1, float* ds2,
                               float* part, char* lin, hipStream_t s) {
  const int64_t nb = prefill_row_blocks(T), ldp = L.d_in + L.d_out;
  if (transposed) {
    const ProdEpilogue pb{x, x_dtype == NQ_BF16, part, ldp};
    hipError_t e = launch_prefill(A, g, g_dtype, T, dx, lin, s, true, &pb);
    return e == hipSuccess ? launch_scale_grads_sums(part, nb, L.d_in, L.d_out, ds1, ds2, 0, L.d_in, s) : e;
  }
  nq_lrb Lu = L;  // u = U (V^T (s2 (.) x)): the forward product without s1
  Lu.s1 = nullptr;
  const ProdEpilogue pu{g, g_dtype == NQ_BF16, part + L.d_in, ldp};
  hipError_t e = launch_prefill(Lu, x, x_dtype, T, nullptr, lin, s, true, &pu);
  return e == hipSuccess ? launch_scale_grads_sums(part, nb, L.d_in, L.d_out, ds1, ds2, L.d_in, L.d_in + L.d_out, s)
                         : e;
}


}  // namespace
}  // namespace nq

struct nq_seq {
  std::vector<nq_lrb> layers;
  std::vector<const void*> xs;
  std::vector<float*> ys;
  nq_dtype xd;
  int64_t T;
  size_t ws_bytes;
  // persistent decode schedule (T <= 8)
  bool persistent = false;
  int grid = 0, ntiles = 0;
  int64_t n_ints = 0;                 // [error flag][next tile][exited][per-linear counters]
  std::vector<int64_t> ctr_off;       // per linear, in ints from the start of the workspace
  std::vector<size_t> buf_off;        // per linear, in bytes
  std::vector<std::pair<int, int>> order;  // (linear, stage) in schedule order
  size_t off_sched = 0;                // descriptors in schedule order
  size_t off_tseg = 0;                 // per tile: index of its descriptor
  std::vector<nq::StageDesc> segs;    // host copies of the uploaded schedule
  std::vector<int> tile_seg;
  void* uploaded_for = nullptr;
  bool needs_zero = true;
  // per-entry kernels (T > 8): entries run round-robin on `nlanes` streams of
  // the plan, each with its own slice of the workspace, so that one entry's
  // memory-bound prep kernels and partly filled last GEMM waves overlap the
  // next entries' GEMMs.  The streams and events are created on the first run.
  int nlanes = 0;
  size_t lane_ws = 0;
  std::vector<hipStream_t> lanes;
  std::vector<hipEvent_t> lane_done;
  hipEvent_t start = nullptr;
  ~nq_seq() {
    for (hipStream_t l : lanes) (void)hipStreamDestroy(l);
    for (hipEvent_t e : lane_done) (void)hipEventDestroy(e);
    if (start) (void)hipEventDestroy(start);
  }
};

namespace {

// Stage 2 of linear i is scheduled after stage 1 of linear i+lag, so that its
// inputs are usually final by the time a workgroup takes its first tile and
// enough independent tiles are ready to keep every workgroup streaming.  The
// input-piece tiles of linear i's stage 1 come lag/2 linears ahead of its
// stage 1 (its stage-1 tiles then find them final), those
// of its stage 2 3*lag/4 linears after it (late enough that stage 1, whose
// tiles can be long, has usually finished, early enough to be done before
// stage 2).
int seq_lag() {
  const char* e = getenv("NQ_SEQ_LAG");
  const int v = e ? atoi(e) : 320;
  return v < 0 ? 0 : v;
}

void plan_persistent(nq_seq* s) {
  using namespace nq;
  const int64_t n = (int64_t)s->layers.size();
  s->persistent = true;
  int64_t ints = 3;
  size_t bufs = 0;
  for (int64_t i = 0; i < n; ++i) {
    s->ctr_off.push_back(ints);
    ints += dec_linear_counters(s->layers[i], s->T, false);
    s->buf_off.push_back(bufs);
    bufs = align_up(bufs + dec_linear_bytes(s->layers[i], s->T, false));
  }
  s->n_ints = ints;
  const int64_t lag = seq_lag();
  // descriptors: pieces of x, stage 1, pieces of t, stage 2
  // how far ahead of its stage 1 a linear's x pieces are made, and how far
  // behind it its t pieces (NQ_SEQ_PRE, NQ_SEQ_LAG2: linears; tuning knobs)
  const char* ep = getenv("NQ_SEQ_PRE");
  const char* e2 = getenv("NQ_SEQ_LAG2");
  const int64_t pre = std::max<int64_t>(ep ? atoi(ep) : lag / 2, 1);
  const int64_t lag2 = std::min<int64_t>(std::max<int64_t>(e2 ? atoi(e2) : lag * 3 / 4, 0), lag);
  auto E = [](int64_t i) { return (int)i; };
  for (int64_t i = 0; i < std::min(pre, n); ++i) s->order.push_back({E(i), 0});
  for (int64_t i = 0; i < n; ++i) {
    if (i + pre < n) s->order.push_back({E(i + pre), 0});
    s->order.push_back({E(i), 1});
    if (i >= lag2) s->order.push_back({E(i - lag2), 2});
    if (i >= lag) s->order.push_back({E(i - lag), 3});
  }
  for (int64_t i = std::max<int64_t>(0, n - lag2); i < n; ++i) s->order.push_back({E(i), 2});
  for (int64_t i = std::max<int64_t>(0, n - lag); i < n; ++i) s->order.push_back({E(i), 3});
  // tile counts do not depend on where the buffers are: count them with the
  // descriptors of a stand-in workspace address
  s->ntiles = 0;
  char* const stand_in = reinterpret_cast<char*>(uintptr_t{1} << 40);
  for (auto& o : s->order) {
    StageDesc d[kMaxLinearDescs];
    dec_stage_descs(s->layers[o.first], s->xs[o.first], s->xd, s->T, s->ys[o.first], false, stand_in,
                    reinterpret_cast<int*>(stand_in), d);
    s->ntiles += stage_tiles(d[o.second]);
  }
  s->off_sched = align_up((size_t)ints * sizeof(int));
  s->off_tseg = align_up(s->off_sched + s->order.size() * sizeof(StageDesc));
  const size_t off_bufs = align_up(s->off_tseg + (size_t)s->ntiles * sizeof(int));
  for (auto& b : s->buf_off) b += off_bufs;
  s->ws_bytes = off_bufs + bufs;
  s->grid = 0;
}

nq_status build_and_upload(nq_seq* s, void* ws, hipStream_t stream) {
  using namespace nq;
  char* base = static_cast<char*>(ws);
  int* ints = reinterpret_cast<int*>(base);
  std::vector<std::array<StageDesc, kMaxLinearDescs>> st(s->layers.size());
  for (size_t i = 0; i < s->layers.size(); ++i)
    dec_stage_descs(s->layers[i], s->xs[i], s->xd, s->T, s->ys[i], false, base + s->buf_off[i], ints + s->ctr_off[i],
                    st[i].data());
  s->segs.clear();
  s->tile_seg.clear();
  for (auto& o : s->order) {
    StageDesc d = st[o.first][o.second];
    d.tile0 = (int)s->tile_seg.size();
    s->tile_seg.insert(s->tile_seg.end(), (size_t)stage_tiles(d), (int)s->segs.size());
    s->segs.push_back(d);
  }
  if ((int64_t)s->tile_seg.size() != s->ntiles) return set_error("nq_seq_run: tile count changed"), NQ_ERR_ARG;
  if (s->grid == 0) s->grid = dec_persistent_grid(s->T);
  hipError_t e = hipMemcpyAsync(base + s->off_sched, s->segs.data(), s->segs.size() * sizeof(StageDesc),
                                hipMemcpyHostToDevice, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(base + s->off_tseg, s->tile_seg.data(), s->tile_seg.size() * sizeof(int),
                       hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "nq_seq_run schedule upload");
  s->uploaded_for = ws;
  s->needs_zero = true;
  return NQ_OK;
}

}  // namespace

using namespace nq;

extern "C" {

const char* nq_last_error(void) { return g_err; }

const char* nq_version(void) { return "libnq 0.1 (gfx950)"; }

uint64_t nq_storage_bits(int64_t d_out, int64_t d_in, int64_t r) {
  if (d_out < 1 || d_in < 1 || r < 1) return 0;
  return (uint64_t)r * (uint64_t)(d_out + d_in) + 32ull * (uint64_t)(d_out + d_in);
}

nq_status nq_pack_signs(const float* src, int64_t n_out, int64_t n_red, int64_t stride_out,
                        int64_t stride_red, uint32_t* dst, int64_t ld, void* stream) {
  clear_error();
  if (!src) return set_error("nq_pack_signs: null src"), NQ_ERR_ARG;
  if (stride_out < 1 || stride_red < 1) return set_error("nq_pack_signs: strides must be >= 1"), NQ_ERR_ARG;
  if (!aligned(src, 4)) return set_error("nq_pack_signs: src not 4-byte aligned"), NQ_ERR_ARG;
  nq_status st = check_words("nq_pack_signs", dst, n_out, n_red, ld);
  if (st != NQ_OK) return st;
  return hip_status(launch_pack(src, n_out, n_red, stride_out, stride_red, dst, ld, (hipStream_t)stream),
                    "nq_pack_signs launch");
}

nq_status nq_unpack_signs(const uint32_t* bits, int64_t n_out, int64_t n_red, int64_t ld, float* dst,
                          void* stream) {
  clear_error();
  nq_status st = check_words("nq_unpack_signs", bits, n_out, n_red, ld);
  if (st != NQ_OK) return st;
  if (!dst) return set_error("nq_unpack_signs: null dst"), NQ_ERR_ARG;
  if (!aligned(dst, 4)) return set_error("nq_unpack_signs: dst not 4-byte aligned"), NQ_ERR_ARG;
  return hip_status(launch_unpack(bits, n_out, n_red, ld, dst, (hipStream_t)stream), "nq_unpack_signs launch");
}

size_t nq_lrb_workspace_bytes(const nq_lrb* L, int64_t T) {
  if (check_lrb("nq_lrb_workspace_bytes", L) != NQ_OK || T < 1 || T > (int64_t(1) << 24)) return 0;
  return linear_workspace(*L, T);
}

nq_status nq_lrb_linear(const nq_lrb* L, const void* x, nq_dtype x_dtype, int64_t T, float* y,
                        void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  nq_status st = check_lrb("nq_lrb_linear", L);
  if (st != NQ_OK) return st;
  if ((st = check_io("nq_lrb_linear", L, x, x_dtype, T, y)) != NQ_OK) return st;
  const size_t need = linear_workspace(*L, T);
  if (!workspace || workspace_bytes < need)
    return set_error("nq_lrb_linear: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0, need),
           NQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return set_error("nq_lrb_linear: workspace not 256-byte aligned"), NQ_ERR_ARG;
  return hip_status(launch_linear(*L, x, x_dtype, T, y, workspace, (hipStream_t)stream), "nq_lrb_linear launch");
}

namespace {
// Workspace of nq_lrb_linear_latent: [U words][V^T words][the linear's].
struct LatentLayout {
  nq_lrb L;  // sign-word pointers relative to the workspace start
  size_t off_u, off_v, off_lin, bytes;
};
LatentLayout latent_layout(int64_t d_out, int64_t d_in, int64_t r, const float* s1, const float* s2, int64_t T) {
  LatentLayout g;
  g.L = nq_lrb{d_out, d_in, r, nullptr, d_out, nullptr, r, s1, s2};
  g.off_u = 0;
  g.off_v = align_up((size_t)cdiv(r, kWordBits) * d_out * sizeof(uint32_t));
  g.off_lin = g.off_v + align_up((size_t)cdiv(d_in, kWordBits) * r * sizeof(uint32_t));
  g.L.u_bits = reinterpret_cast<const uint32_t*>(uintptr_t{1} << 40);  // stand-ins for sizing
  g.L.vt_bits = g.L.u_bits;
  g.bytes = g.off_lin + linear_workspace(g.L, T);
  return g;
}
}  // namespace

size_t nq_lrb_latent_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r, int64_t T) {
  if (d_out < 1 || d_in < 1 || r < 1 || T < 1 || T > (int64_t(1) << 24)) return 0;
  static const float one = 1.0f;
  const LatentLayout g = latent_layout(d_out, d_in, r, &one, &one, T);
  if (check_lrb("nq_lrb_latent_workspace_bytes", &g.L) != NQ_OK) return 0;
  if (T <= kLatMaxT) return lat_forward_fits(d_out, d_in, r, T) ? lat_forward_bytes(d_out, d_in, r, T) : 0;
  return g.bytes;
}

nq_status nq_lrb_linear_latent(const float* u_lat, int64_t ldu_lat, const float* v_lat, int64_t ldv_lat,
                               int64_t d_out, int64_t d_in, int64_t r, const float* s1, const float* s2, const void* x,
                               nq_dtype x_dtype, int64_t T, float* y, void* workspace, size_t workspace_bytes,
                               void* stream) {
  clear_error();
  const char* who = "nq_lrb_linear_latent";
  if (!u_lat || !v_lat) return set_error("%s: null latent", who), NQ_ERR_ARG;
  if (d_out < 1 || d_in < 1 || r < 1) return set_error("%s: sizes must be >= 1", who), NQ_ERR_ARG;
  if (ldu_lat < r || ldv_lat < r)
    return set_error("%s: latent row strides %lld / %lld below r=%lld", who, (long long)ldu_lat, (long long)ldv_lat,
                     (long long)r),
           NQ_ERR_ARG;
  if (!aligned(u_lat, 4) || !aligned(v_lat, 4)) return set_error("%s: latent not 4-byte aligned", who), NQ_ERR_ARG;
  LatentLayout g = latent_layout(d_out, d_in, r, s1, s2, T);
  nq_status st = check_lrb(who, &g.L);
  if (st != NQ_OK) return st;
  if ((st = check_io(who, &g.L, x, x_dtype, T, y)) != NQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (T <= kLatMaxT) {  // decode sizes: the signs are taken as the latents load
    if (!lat_forward_fits(d_out, d_in, r, T))
      return set_error("%s: shape exceeds the launch grid", who), NQ_ERR_UNSUPPORTED;
    const size_t need = lat_forward_bytes(d_out, d_in, r, T);
    if (!workspace || workspace_bytes < need)
      return set_error("%s: workspace %zu bytes, need %zu", who, workspace ? workspace_bytes : 0, need),
             NQ_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return set_error("%s: workspace not 256-byte aligned", who), NQ_ERR_ARG;
    return hip_status(launch_lat_forward(u_lat, ldu_lat, v_lat, ldv_lat, d_out, d_in, r, s1, s2, x,
                                         x_dtype == NQ_BF16, T, y, workspace, s),
                      "nq_lrb_linear_latent launch");
  }
  if (!workspace || workspace_bytes < g.bytes)
    return set_error("%s: workspace %zu bytes, need %zu", who, workspace ? workspace_bytes : 0, g.bytes),
           NQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return set_error("%s: workspace not 256-byte aligned", who), NQ_ERR_ARG;
  char* ws = static_cast<char*>(workspace);
  uint32_t* ub = reinterpret_cast<uint32_t*>(ws + g.off_u);
  uint32_t* vb = reinterpret_cast<uint32_t*>(ws + g.off_v);
  g.L.u_bits = ub;
  g.L.vt_bits = vb;
  // U latent [d_out][ldu_lat]: outputs d_out, reduction r; V latent [d_in][ldv_lat]: outputs r, reduction d_in
  hipError_t e = launch_pack(u_lat, d_out, r, ldu_lat, 1, ub, d_out, s);
  if (e == hipSuccess) e = launch_pack(v_lat, r, d_in, 1, ldv_lat, vb, r, s);
  if (e == hipSuccess) e = launch_linear(g.L, x, x_dtype, T, y, ws + g.off_lin, s);
  return hip_status(e, "nq_lrb_linear_latent launch");
}

nq_status nq_reconstruct(const nq_lrb* L, float* w, void* stream) {
  clear_error();
  nq_status st = check_lrb("nq_reconstruct", L);
  if (st != NQ_OK) return st;
  if (!w) return set_error("nq_reconstruct: null w"), NQ_ERR_ARG;
  if (!aligned(w, 4)) return set_error("nq_reconstruct: w not 4-byte aligned"), NQ_ERR_ARG;
  return hip_status(launch_reconstruct(*L, w, (hipStream_t)stream), "nq_reconstruct launch");
}

nq_status nq_transpose_signs(const uint32_t* src, int64_t n_out, int64_t n_red, int64_t ld, uint32_t* dst,
                             int64_t ldt, void* stream) {
  clear_error();
  nq_status st = check_words("nq_transpose_signs", src, n_out, n_red, ld);
  if (st != NQ_OK) return st;
  if ((st = check_words("nq_transpose_signs", dst, n_red, n_out, ldt)) != NQ_OK) return st;
  if (cdiv(n_red, kWordBits) * ld >= (int64_t(1) << 29) || cdiv(n_out, kWordBits) * ldt >= (int64_t(1) << 29))
    return set_error("nq_transpose_signs: a sign-word buffer exceeds 2 GiB"), NQ_ERR_UNSUPPORTED;
  return hip_status(launch_transpose_signs(src, n_out, n_red, ld, dst, ldt, (hipStream_t)stream),
                    "nq_transpose_signs launch");
}

size_t nq_lrb_scale_grads_workspace_bytes(const nq_lrb* L, int64_t T) {
  if (check_lrb("nq_lrb_scale_grads_workspace_bytes", L) != NQ_OK || T < 1 || T > (int64_t(1) << 24)) return 0;
  return scale_grads_layout(*L, T).bytes;
}

nq_status nq_lrb_scale_grads(const nq_lrb* L, const uint32_t* ut_bits, int64_t ldut, const uint32_t* v_bits,
                             int64_t ldvv, const void* x, nq_dtype x_dtype, const void* g, nq_dtype g_dtype,
                             int64_t T, float* dx, float* ds1, float* ds2, void* workspace, size_t workspace_bytes,
                             void* stream) {
  clear_error();
  const char* who = "nq_lrb_scale_grads";
  nq_lrb A;
  nq_status st = check_grads(who, L, ut_bits, ldut, v_bits, ldvv, x, x_dtype, g, g_dtype, T, dx, ds1, ds2, &A);
  if (st != NQ_OK) return st;
  const ScaleGradsLayout lay = scale_grads_layout(*L, T);
  if (!workspace || workspace_bytes < lay.bytes)
    return set_error("%s: workspace %zu bytes, need %zu", who, workspace ? workspace_bytes : 0, lay.bytes),
           NQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return set_error("%s: workspace not 256-byte aligned", who), NQ_ERR_ARG;
  char* ws = static_cast<char*>(workspace);
  float* u = reinterpret_cast<float*>(ws + lay.off_u);
  float* b = reinterpret_cast<float*>(ws + lay.off_b);
  hipStream_t s = (hipStream_t)stream;
  nq_lrb Lu = *L;  // u = U (V^T (s2 (.) x)): the forward product without s1
  Lu.s1 = nullptr;
  float* part = reinterpret_cast<float*>(ws + lay.off_part);
  if (T > kDecodeMaxT) {
    // matrix-core regime: the GEMMs' epilogues take the token sums per 128-row
    // block (ds1 from g (.) u with u never stored; ds2 from x (.) b while the
    // transposed product, its row scale s2 kept, writes dx), and each stream
    // adds its blocks in order
    hipError_t e;
    {
      std::lock_guard<std::mutex> lock(g_side_mu);
      SideStream* side = nullptr;
      e = side_stream(&side);
      if (e == hipSuccess) e = hipEventRecord(side->fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
      if (e == hipSuccess)
        e = enqueue_grads_chain(*L, A, true, x, x_dtype, g, g_dtype, T, dx, ds1, ds2, part, ws + lay.off_lin_t,
                                side->s);
      if (e == hipSuccess)
        e = enqueue_grads_chain(*L, A, false, x, x_dtype, g, g_dtype, T, dx, ds1, ds2, part, ws + lay.off_lin, s);
      if (e == hipSuccess) e = hipEventRecord(side->join, side->s);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
    }
    return hip_status(e, "nq_lrb_scale_grads launch");
  }
  A.s1 = nullptr;  // b = V (U^T (s1 (.) g)): the transposed product without s2
  // the two products on two streams: one's prep kernels and last, partly
  // filled wave of tiles run beside the other's GEMMs
  hipError_t e;
  {
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* side = nullptr;
    e = side_stream(&side);
    if (e == hipSuccess) e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    // each stream then takes the token sums of its own product: columns
    // [0, d_in) (dx and ds2, from b) and [d_in, d_in + d_out) (ds1, from u)
    if (e == hipSuccess) e = launch_linear(A, g, g_dtype, T, b, ws + lay.off_lin_t, side->s);
    if (e == hipSuccess)
      e = launch_scale_grads_finish(x, x_dtype, g, g_dtype, u, b, L->s2, T, L->d_in, L->d_out, dx, part, ds1, ds2,
                                    0, L->d_in, side->s);
    if (e == hipSuccess) e = launch_linear(Lu, x, x_dtype, T, u, ws + lay.off_lin, s);
    if (e == hipSuccess)
      e = launch_scale_grads_finish(x, x_dtype, g, g_dtype, u, b, L->s2, T, L->d_in, L->d_out, dx, part, ds1, ds2,
                                    L->d_in, L->d_in + L->d_out, s);
    if (e == hipSuccess) e = hipEventRecord(side->join, side->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
  }
  return hip_status(e, "nq_lrb_scale_grads launch");
}

size_t nq_lrb_scale_grads_batch_workspace_bytes(int64_t n, const nq_lrb* L, int64_t T) {
  if (n < 1 || n > (int64_t(1) << 20) || !L || T < 1 || T > (int64_t(1) << 24)) return 0;
  size_t single = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (check_lrb("nq_lrb_scale_grads_batch_workspace_bytes", &L[i]) != NQ_OK) return 0;
    single = std::max(single, scale_grads_layout(L[i], T).bytes);
  }
  return T > kDecodeMaxT ? batch_grads_layout(L, n, T).bytes : single;
}

nq_status nq_lrb_scale_grads_batch(int64_t n, const nq_lrb* L, const uint32_t* const* ut_bits, const int64_t* ldut,
                                   const uint32_t* const* v_bits, const int64_t* ldvv, const void* const* x,
                                   nq_dtype x_dtype, const void* const* g, nq_dtype g_dtype, int64_t T,
                                   float* const* dx, float* const* ds1, float* const* ds2, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  clear_error();
  const char* who = "nq_lrb_scale_grads_batch";
  if (n < 1 || n > (int64_t(1) << 20)) return set_error("%s: n = %lld", who, (long long)n), NQ_ERR_ARG;
  if (!L || !ut_bits || !ldut || !v_bits || !ldvv || !x || !g || !dx || !ds1 || !ds2)
    return set_error("%s: null array", who), NQ_ERR_ARG;
  std::vector<nq_lrb> A((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    nq_status st = check_grads(who, &L[i], ut_bits[i], ldut[i], v_bits[i], ldvv[i], x[i], x_dtype, g[i], g_dtype, T,
                               dx[i], ds1[i], ds2[i], &A[(size_t)i]);
    if (st != NQ_OK) {
      const std::string why = nq_last_error();  // the message buffer is rewritten below
      return set_error("%s: linear %lld: %s", who, (long long)i, why.c_str()), st;
    }
  }
  const size_t need = nq_lrb_scale_grads_batch_workspace_bytes(n, L, T);
  if (!workspace || workspace_bytes < need)
    return set_error("%s: workspace %zu bytes, need %zu", who, workspace ? workspace_bytes : 0, need),
           NQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return set_error("%s: workspace not 256-byte aligned", who), NQ_ERR_ARG;
  if (T <= kDecodeMaxT) {  // the decode regime: the linears one after another
    for (int64_t i = 0; i < n; ++i) {
      nq_status st = nq_lrb_scale_grads(&L[i], ut_bits[i], ldut[i], v_bits[i], ldvv[i], x[i], x_dtype, g[i], g_dtype,
                                        T, dx[i], ds1[i], ds2[i], workspace, workspace_bytes, stream);
      if (st != NQ_OK) return st;
    }
    return NQ_OK;
  }
  // matrix-core regime: the 2n product chains (transposed and forward of each
  // linear) round-robin on the library's streams, each with its own slice of
  // the workspace; forked from and joined back to the caller's stream
  const BatchGradsLayout lay = batch_grads_layout(L, n, T);
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  {
    std::lock_guard<std::mutex> lock(g_side_mu);
    LaneSet* ls = nullptr;
    e = lane_set(&ls);
    if (e == hipSuccess) e = hipEventRecord(ls->fork, s);
    for (int l = 0; l < kBatchLanes && e == hipSuccess; ++l) e = hipStreamWaitEvent(ls->s[l], ls->fork, 0);
    for (int64_t c = 0; c < 2 * n && e == hipSuccess; ++c) {
      const int64_t i = c / 2;
      const int l = (int)(c % kBatchLanes);
      char* lane = ws + (size_t)l * lay.lane;
      e = enqueue_grads_chain(L[i], A[(size_t)i], c % 2 == 0, x[i], x_dtype, g[i], g_dtype, T, dx[i], ds1[i], ds2[i],
                              reinterpret_cast<float*>(lane + lay.off_part), lane + lay.off_lin, ls->s[l]);
    }
    for (int l = 0; l < kBatchLanes && e == hipSuccess; ++l) {
      e = hipEventRecord(ls->join[l], ls->s[l]);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, ls->join[l], 0);
    }
  }
  return hip_status(e, "nq_lrb_scale_grads_batch launch");
}

size_t nq_balance_workspace_bytes(int64_t d_out, int64_t d_in) {
  if (d_out < 1 || d_in < 1 || d_out > (int64_t(1) << 30) || d_in > (int64_t(1) << 30)) return 0;
  return balance_workspace_bytes(d_out, d_in);
}

nq_status nq_balance_factors(const float* u_hat, int64_t d_out, int64_t ldu, const float* v_hat, int64_t d_in,
                             int64_t ldv, int64_t r, float* u_out, float* v_out, float* s1, float* s2, float* eta,
                             void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const char* who = "nq_balance_factors";
  if (!u_hat || !v_hat || !s1 || !s2 || !eta) return set_error("%s: null input, scale or eta", who), NQ_ERR_ARG;
  if (d_out < 1 || d_in < 1 || r < 1 || d_out > (int64_t(1) << 30) || d_in > (int64_t(1) << 30))
    return set_error("%s: bad sizes d_out=%lld d_in=%lld r=%lld", who, (long long)d_out, (long long)d_in,
                     (long long)r),
           NQ_ERR_ARG;
  if (ldu < r || ldv < r)
    return set_error("%s: ldu=%lld / ldv=%lld below r=%lld", who, (long long)ldu, (long long)ldv, (long long)r),
           NQ_ERR_ARG;
  if ((u_out == nullptr) != (v_out == nullptr)) return set_error("%s: give both u_out and v_out or neither", who), NQ_ERR_ARG;
  if (!aligned(u_hat, 4) || !aligned(v_hat, 4) || !aligned(u_out, 4) || !aligned(v_out, 4) || !aligned(s1, 4) ||
      !aligned(s2, 4) || !aligned(eta, 4))
    return set_error("%s: a pointer is not 4-byte aligned", who), NQ_ERR_ARG;
  const size_t need = balance_workspace_bytes(d_out, d_in);
  if (!workspace || workspace_bytes < need)
    return set_error("%s: workspace %zu bytes, need %zu", who, workspace ? workspace_bytes : 0, need),
           NQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return set_error("%s: workspace not 256-byte aligned", who), NQ_ERR_ARG;
  return hip_status(launch_balance(u_hat, ldu, v_hat, ldv, d_out, d_in, r, u_out, v_out, s1, s2, eta, workspace,
                                   (hipStream_t)stream),
                    "nq_balance_factors launch");
}

nq_status nq_fill_random_words(uint32_t* dst, int64_t n, uint64_t seed, void* stream) {
  clear_error();
  if (!dst || n < 0) return set_error("nq_fill_random_words: null dst or n < 0"), NQ_ERR_ARG;
  if (!aligned(dst, 4)) return set_error("nq_fill_random_words: dst not 4-byte aligned"), NQ_ERR_ARG;
  return hip_status(launch_fill_words(dst, n, seed, (hipStream_t)stream), "nq_fill_random_words launch");
}

nq_status nq_seq_create(const nq_lrb* layers, const void* const* xs, float* const* ys, int64_t n,
                        nq_dtype x_dtype, int64_t T, nq_seq** out) {
  clear_error();
  if (!out) return set_error("nq_seq_create: null out"), NQ_ERR_ARG;
  *out = nullptr;
  if (!layers || !xs || !ys || n < 1) return set_error("nq_seq_create: empty or null arrays"), NQ_ERR_ARG;
  nq_seq* s = new (std::nothrow) nq_seq;
  if (!s) return set_error("nq_seq_create: out of host memory"), NQ_ERR_ARG;
  s->xd = x_dtype;
  s->T = T;
  s->ws_bytes = 0;
  for (int64_t i = 0; i < n; ++i) {
    char who[64];
    snprintf(who, sizeof(who), "nq_seq_create[%lld]", (long long)i);
    nq_status st = check_lrb(who, &layers[i]);
    if (st == NQ_OK) st = check_io(who, &layers[i], xs[i], x_dtype, T, ys[i]);
    if (st != NQ_OK) {
      delete s;
      return st;
    }
    s->layers.push_back(layers[i]);
    s->xs.push_back(xs[i]);
    s->ys.push_back(ys[i]);
    s->ws_bytes = std::max<size_t>(s->ws_bytes, linear_workspace(layers[i], T, true));
  }
  if (T <= kDecodeMaxT && !decode_xor()) {
    plan_persistent(s);
  } else {
    s->nlanes = (int)std::min<int64_t>(kSeqLanes, n);
    s->lane_ws = align_up(s->ws_bytes);
    s->ws_bytes = s->lane_ws * s->nlanes;
  }
  *out = s;
  return NQ_OK;
}

size_t nq_seq_workspace_bytes(const nq_seq* s) { return s ? s->ws_bytes : 0; }

nq_status nq_seq_run(nq_seq* s, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (!s) return set_error("nq_seq_run: null plan"), NQ_ERR_ARG;
  if (!workspace || workspace_bytes < s->ws_bytes)
    return set_error("nq_seq_run: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0, s->ws_bytes),
           NQ_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return set_error("nq_seq_run: workspace not 256-byte aligned"), NQ_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (s->persistent) {
    if (s->uploaded_for != workspace) {
      nq_status r = build_and_upload(s, workspace, st);
      if (r != NQ_OK) return r;
    }
    int* ints = static_cast<int*>(workspace);
    hipError_t e = hipSuccess;
    if (s->needs_zero) {  // first run on this workspace; later runs leave the counters zeroed
      e = launch_zero_ints(ints, s->n_ints, st);
      s->needs_zero = false;
    }
    if (e == hipSuccess)
      e = launch_dec_persistent(reinterpret_cast<const StageDesc*>(static_cast<char*>(workspace) + s->off_sched),
                                reinterpret_cast<const int*>(static_cast<char*>(workspace) + s->off_tseg), s->ntiles,
                                ints, (int)s->n_ints, s->T, s->grid, st);
    return hip_status(e, "nq_seq_run launch");
  }
  if (s->lanes.empty()) {  // first run: the plan's streams (default priority) and events
    for (int l = 0; l < s->nlanes; ++l) {
      hipStream_t ls = nullptr;
      hipEvent_t ev = nullptr;
      hipError_t e = hipStreamCreateWithFlags(&ls, hipStreamNonBlocking);
      if (e == hipSuccess) s->lanes.push_back(ls);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e == hipSuccess) s->lane_done.push_back(ev);
      if (e != hipSuccess) return hip_status(e, "nq_seq_run stream setup");
    }
    hipError_t e = hipEventCreateWithFlags(&s->start, hipEventDisableTiming);
    if (e != hipSuccess) return hip_status(e, "nq_seq_run stream setup");
  }
  // fork: every lane waits for the work already queued on the caller's stream
  hipError_t e = hipEventRecord(s->start, st);
  for (int l = 0; l < s->nlanes && e == hipSuccess; ++l) e = hipStreamWaitEvent(s->lanes[l], s->start, 0);
  for (size_t i = 0; i < s->layers.size() && e == hipSuccess; ++i) {
    const int l = (int)(i % s->nlanes);
    e = launch_linear(s->layers[i], s->xs[i], s->xd, s->T, s->ys[i], static_cast<char*>(workspace) + l * s->lane_ws,
                      s->lanes[l], true);
  }
  // join: the caller's stream waits for every lane
  for (int l = 0; l < s->nlanes && e == hipSuccess; ++l) {
    e = hipEventRecord(s->lane_done[l], s->lanes[l]);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, s->lane_done[l], 0);
  }
  return hip_status(e, "nq_seq_run launch");
}

void nq_seq_destroy(nq_seq* s) { delete s; }

}  // extern "C"
