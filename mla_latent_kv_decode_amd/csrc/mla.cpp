// Host layer of the MLA library: the C ABI of include/mla.h.
//
// Validation of every argument happens here, on the host, before anything is
// launched.  Ragged metadata arrive as host arrays; the decode work list is
// built here and copied into the caller's workspace from pinned staging
// memory the handle owns (a small ring, so a call never overwrites staging
// data an earlier asynchronous copy may still be reading).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "mla.h"
#include "kernels.h"

// rows-equivalent cost of a segment start in the split-S work list
#ifndef MLA_SEG_ROWS
#define MLA_SEG_ROWS 64
#endif

using mla::bf16;
using mla::DecodeMeta;
using mla::DecodeSeg;
using mla::Dims;

namespace {

constexpr size_t kAlign = 256;
constexpr int kRing = 4;
// Pinned bytes every staging slot gets at mla_create, so that the
// no-allocation decode step finds its metadata room already there.
constexpr size_t kStageInit = (size_t)256 << 10;

size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

}  // namespace

struct mla_ctx {
  mla_config cfg{};
  Dims d{};
  mla::RopeTab rope{};
  hipStream_t stream = nullptr;
  int device = 0;
  int n_cu = 256;
  size_t esz = 2;
  bool absorbed = false;
  bool mfma = false;  // bf16 MFMA kernels apply to these shapes
  bool kv8 = false;   // the latent cache holds FP8 rows (mla_config.kv_storage)
  // owned device weights
  void* w_q = nullptr;
  void* w_qa = nullptr;
  void* q_norm_g = nullptr;
  void* w_qb = nullptr;
  void* w_kva = nullptr;
  void* kv_norm_g = nullptr;
  void* w_kvb = nullptr;
  void* w_ukT = nullptr;  // (H, dc, dn): q_abs = q_nope . W_ukT^T per head
  void* w_uv = nullptr;   // (H, dv, dc)
  void* w_o = nullptr;
  void* w_in = nullptr;   // [W_kva ; W_q] (or [W_kva ; W_qa]) rows: one in-projection GEMM
  // fragment-tiled copies of the weights the large-tile GEMM reads (bf16
  // layers with aligned dimensions; null where the width is not a multiple
  // of 32)
  void* t_in = nullptr;
  void* t_q = nullptr;   // w_q or w_qa
  void* t_qb = nullptr;
  void* t_kva = nullptr;
  void* t_kvb = nullptr;
  void* t_o = nullptr;
  int n_in = 0;           // rows of w_in
  // materialised absorption (mla_config.absorb): per head [W^KQ_h ; W_q,rope_h]
  // query rows (behind the W_kva rows without a query LoRA, as w_in), and
  // W^OV (D, H * dc)
  bool mat = false;
  void* m_in = nullptr;   // [W_kva ; per head (W^KQ_h ; W_q,rope_h)] (no query LoRA)
  void* m_qb = nullptr;   // per head (W^KQ_h ; W_qb,rope_h) (query LoRA)
  void* m_ov = nullptr;
  Staging ring[kRing];
  int ring_next = 0;
  std::vector<void*> captured;  // pinned staging owned by captured graphs
  // timing ring of the attention-core launches: events 2i, 2i+1 bracket slot i
  std::vector<hipEvent_t> tev;
  int t_next = 0;
  int64_t t_count = 0;
  // every dimension that strides a GEMM operand or output is a multiple of 8
  // elements (16-byte rows for the large-tile GEMM)
  bool dims_aligned = false;
  // the no-allocation decode step: device address of this device's static
  // scratch array, and set while such a call runs (the staging ring must not
  // grow then)
  void* noalloc_ws = nullptr;
  bool no_alloc = false;
  std::string err;
};

namespace {

int fail(mla_ctx* h, int code, const char* fmt, ...) {
  if (h) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    h->err = buf;
  }
  return code;
}

// MLA_LOG=1 (read once per process): one line per call on stderr with the
// call's shape, the work plan and the kernels chosen.
bool log_on() {
  static const bool on = [] {
    const char* e = getenv("MLA_LOG");
    return e && *e && strcmp(e, "0") != 0;
  }();
  return on;
}

void mlog(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[mla] %s\n", buf);
}

#define HIP_TRY(h, call)                                                              \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail((h), MLA_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));  \
  } while (0)

// Makes the handle's device current for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

int check_launch(mla_ctx* h, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(h, MLA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

// Put `bytes` of host data into pinned staging memory the GPU can read: a
// slot of the handle's ring (reusable once the event *ev, to be recorded after
// the call's last reader is enqueued, has passed), or, while the stream is
// being captured into a graph, a buffer kept for the life of the handle (the
// graph reads it at every replay).  Staging memory is allocated coherent, so a
// kernel may read it directly over the bus; sizes are padded to 256 bytes.
int stage_host(mla_ctx* h, const void* src, size_t bytes, const void** pinned,
               hipEvent_t* ev) {
  *pinned = nullptr;
  *ev = nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  HIP_TRY(h, hipStreamIsCapturing(h->stream, &cap));
  if (cap == hipStreamCaptureStatusActive) {
    void* p = nullptr;
    HIP_TRY(h, hipHostMalloc(&p, align_up(bytes), hipHostMallocCoherent));
    h->captured.push_back(p);
    memcpy(p, src, bytes);
    *pinned = p;
    return MLA_OK;
  }
  Staging& s = h->ring[h->ring_next];
  h->ring_next = (h->ring_next + 1) % kRing;
  if (s.pending) {
    HIP_TRY(h, hipEventSynchronize(s.ev));
    s.pending = false;
  }
  if (s.cap < bytes && h->no_alloc)
    return fail(h, MLA_ERR_WORKSPACE,
                "metadata of %zu bytes exceed the %zu pinned bytes staged at mla_create", bytes,
                s.cap);
  if (s.cap < bytes) {
    if (s.host) HIP_TRY(h, hipHostFree(s.host));
    s.host = nullptr;
    s.cap = 0;
    const size_t cap = std::max(align_up(bytes, 1 << 16), (size_t)1 << 16);
    HIP_TRY(h, hipHostMalloc(&s.host, cap, hipHostMallocCoherent));
    s.cap = cap;
  }
  if (!s.ev) HIP_TRY(h, hipEventCreateWithFlags(&s.ev, hipEventDisableTiming));
  memcpy(s.host, src, bytes);
  s.pending = true;
  *pinned = s.host;
  *ev = s.ev;
  return MLA_OK;
}

// Copy `bytes` of host data to device `dst` on the handle's stream through the
// pinned staging memory.
int stage_upload(mla_ctx* h, void* dst, const void* src, size_t bytes) {
  if (bytes == 0) return MLA_OK;
  const void* p = nullptr;
  hipEvent_t ev = nullptr;
  int rc = stage_host(h, src, bytes, &p, &ev);
  if (rc) return rc;
  HIP_TRY(h, hipMemcpyAsync(dst, p, bytes, hipMemcpyHostToDevice, h->stream));
  if (ev) HIP_TRY(h, hipEventRecord(ev, h->stream));
  return MLA_OK;
}

// Workspace carving: regions are 256-byte aligned offsets from the base.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

bool is_f32(const mla_ctx* h) { return h->cfg.dtype == MLA_F32; }

bool mfma_gemm(const mla_ctx* h, int N, int K) {
  // every one of the 4 K-slices of a block needs whole 32-wide k-steps
  return h->cfg.dtype == MLA_BF16 && N % 16 == 0 && K % 128 == 0;
}

// Projections with many rows (prefill, bulk appends) are plain GEMMs with
// enough work for the large-tile kernel: at least 256 rows and enough tiles to
// fill half the compute units.
constexpr int kBigGemmMinM = 256;
bool big_gemm(const mla_ctx* h, int M, int N, int K, int batch) {
  if (h->cfg.dtype != MLA_BF16 || !h->dims_aligned || batch != 1 || M < kBigGemmMinM ||
      K % 32 != 0 || N % 4 != 0)
    return false;
  const int bn = mla::gemm_big_bn(M, N, h->n_cu);
  const long tiles = (long)((M + 255) / 256) * ((N + bn - 1) / bn);
  return tiles * 2 >= h->n_cu;
}

int gemm_ks(const mla_ctx* h, int M, int N, int K, int batch) {
  if (big_gemm(h, M, N, K, batch)) return 1;
  return mfma_gemm(h, N, K) ? mla::gemm_bf16_ksplit(M, N, K, batch, h->n_cu) : 1;
}

// floats that hold A in the fragment-tiled layout of the large-tile GEMM
size_t tiled_floats(int M, int K) { return align_up(mla::tiled_bytes(M, K)) / 4; }

// fp32 scratch floats of gemm_out (split-K partials, the VALU path's C, or A
// tiled for the large-tile GEMM)
size_t out_scratch(const mla_ctx* h, int M, int N, int K, int batch) {
  if (big_gemm(h, M, N, K, batch)) return tiled_floats(M, K);
  const int ks = gemm_ks(h, M, N, K, batch);
  if (mfma_gemm(h, N, K) && ks == 1) return 0;
  return (size_t)ks * batch * M * N;
}
// fp32 floats of gemm_part's partial buffer (then A tiled for the large-tile
// GEMM)
size_t part_floats(const mla_ctx* h, int M, int N, int K) {
  const size_t c = (size_t)gemm_ks(h, M, N, K, 1) * M * N;
  return big_gemm(h, M, N, K, 1) ? align_up(c * 4) / 4 + tiled_floats(M, K) : c;
}

// out = alpha * A W^T (batched, strided).  MFMA path: epilogue fused when K is
// not split, else partials in `scratch` and a store kernel sums them.
// Wt: W's fragment-tiled copy (batch 1), which lets the large-tile GEMM run;
// A is then tiled into `scratch` first.
template <typename T>
void gemm_out(mla_ctx* h, const T* A, int64_t lda, int64_t sA, const T* W, int64_t ldw,
              int64_t sW, int M, int N, int K, int batch, const mla::GemmOut& out,
              float* scratch, const void* Wt = nullptr) {
  if constexpr (sizeof(T) == 2) {
    if (Wt && big_gemm(h, M, N, K, batch)) {
      bf16* At = reinterpret_cast<bf16*>(scratch);
      mla::tile_rows(A, lda, M, K, At, h->stream);
      mla::gemm_big(At, static_cast<const bf16*>(Wt), M, N, K, out, h->n_cu, h->stream);
      return;
    }
    if (mfma_gemm(h, N, K)) {
      const int ks = gemm_ks(h, M, N, K, batch);
      mla::gemm_bf16_mfma(A, lda, sA, W, ldw, sW, M, N, K, batch, ks, scratch, out, h->stream);
      if (ks > 1) mla::gemm_store(scratch, ks, M, N, batch, out, h->stream);
      return;
    }
  }
  mla::gemm_generic<T>(A, lda, sA, W, ldw, sW, scratch, M, N, K, batch, 1, h->stream);
  mla::gemm_store(scratch, 1, M, N, batch, out, h->stream);
}

// A W^T (batch 1) left as fp32 split-K partials in `part` for the consuming
// kernel to sum (part_floats() floats).
template <typename T>
mla::Part gemm_part(mla_ctx* h, const T* A, int64_t lda, const T* W, int64_t ldw, int M,
                    int N, int K, float* part, const void* Wt = nullptr) {
  if constexpr (sizeof(T) == 2) {
    if (Wt && big_gemm(h, M, N, K, 1)) {
      bf16* At = reinterpret_cast<bf16*>(part + align_up((size_t)M * N * 4) / 4);
      mla::tile_rows(A, lda, M, K, At, h->stream);
      mla::gemm_big(At, static_cast<const bf16*>(Wt), M, N, K,
                    mla::GemmOut{part, nullptr, N, 0, 1.f}, h->n_cu, h->stream);
      return mla::Part{part, 1, N, (int64_t)M * N};
    }
    if (mfma_gemm(h, N, K)) {
      const int ks = gemm_ks(h, M, N, K, 1);
      mla::gemm_bf16_mfma(A, lda, 0, W, ldw, 0, M, N, K, 1, ks, part,
                          mla::GemmOut{part, nullptr, N, 0, 1.f}, h->stream);
      return mla::Part{part, ks, N, (int64_t)M * N};
    }
  }
  mla::gemm_generic<T>(A, lda, 0, W, ldw, 0, part, M, N, K, 1, 1, h->stream);
  return mla::Part{part, 1, N, (int64_t)M * N};
}

mla::GemmOut out_f32(float* p, int64_t ldo, int64_t so = 0, float alpha = 1.f) {
  return mla::GemmOut{p, nullptr, ldo, so, alpha};
}
template <typename T>
mla::GemmOut out_t(T* p, int64_t ldo, int64_t so = 0, float alpha = 1.f) {
  if constexpr (sizeof(T) == 4) return mla::GemmOut{(float*)p, nullptr, ldo, so, alpha};
  else return mla::GemmOut{nullptr, (bf16*)p, ldo, so, alpha};
}

// ------------------------------------------------------------------------
// decode plan
// ------------------------------------------------------------------------
struct DecodeLayout {
  int max_segs = 0;
  bool step = false;  // fused append (mla_decode_step)
  int max_cslots = 0;  // chunk slots of the two-pass combine
  size_t meta, scratch, pin, pq, cq, q_nope, q_cat, acc, ml, cacc, cml, o_lat, o;
  size_t rpart;  // split-K partials of the resident-activation stream GEMMs
  size_t total = 0;
};

// layers with many heads use the shared-tile core (bf16 or FP8 rows)
bool wide_core(const mla_ctx* h) {
  return h->mfma && h->d.H % mla::decode_core_wide_heads() == 0;
}
// other MFMA layers use the ring core
bool ring_core(const mla_ctx* h) { return h->mfma && !wide_core(h); }
// the attention core a decode call of this layer runs
const char* core_name(const mla_ctx* h) {
  if (!h->mfma) return "decode_core_generic_k";
  if (wide_core(h)) return h->kv8 ? "decode_core_wide8_k" : "decode_core_wide_k";
  return h->kv8 ? "decode_core_ring8_k" : "decode_core_ring_k";
}
// the split combine fused with the value un-absorb (MFMA layers with dv = 128)
bool combine_uv(const mla_ctx* h) { return h->mfma && h->d.dv == 128; }

int max_parts(const mla_ctx* h, int64_t total_rows, int q_len = 1) {
  // at least 64 rows per part; 256 for the many-head core, whose partial of a
  // segment (128 heads x 512 fp32 sums, 262 KB) weighs as much as ~230 rows
  // of cache: at one sequence of 32,768 rows, 256 parts wrote 67 MB of
  // partials for 38 MB of rows and needed the combine's first pass
  // (rounded down there: 32,768 cached rows plus the new one make 128 parts,
  // whose partials the combine merges without its first pass, not 129)
  int64_t p = wide_core(h) ? total_rows / 256 : (total_rows + 63) / 64;
  // the MFMA cores run one workgroup per compute unit: per 16-head group (or
  // per 128 heads for the many-head core) and new token of a part
  const int64_t wgs = !h->mfma ? h->n_cu
                      : wide_core(h)
                          ? std::max<int64_t>(1, (int64_t)h->n_cu /
                                                     (h->d.H / mla::decode_core_wide_heads() *
                                                      q_len))
                          : std::max<int64_t>(1, (int64_t)h->n_cu /
                                                     (h->d.H / 16 * q_len /
                                                      (h->kv8 ? 1 : mla::decode_core_ring_tokens(
                                                                        q_len))));
  if (p > wgs) p = wgs;
  if (p < 1) p = 1;
  return (int)p;
}

// page lists of a paged cache: at most total_rows / 32 + B pages (pages hold
// 32 rows or more)
size_t page_list_bytes(int B, int64_t total_rows) {
  return align_up((size_t)B * 4) + align_up((size_t)(total_rows / 32 + B) * 4);
}

// per sequence: seq_off, seq_len, pstart, nseg, cstart; per query row (B *
// q_len): slot, pos and the combine's pstart, nseg, cstart
size_t meta_bytes(int B, int parts, int max_segs, int64_t total_rows, int q_len = 1) {
  const size_t Bq = (size_t)B * q_len;
  return align_up((size_t)B * 8) + align_up(Bq * 8) + 4 * align_up((size_t)B * 4) +
         4 * align_up(Bq * 4) + align_up((size_t)(parts + 1) * 4) +
         align_up((size_t)max_segs * sizeof(DecodeSeg)) +
         align_up((size_t)max_segs * sizeof(mla::DecodeWork)) + page_list_bytes(B, total_rows);
}

int qw_of(const Dims& d) { return d.H * (d.dn + d.dr); }

// B sequences with q_len new tokens each: the query path, the combine and the
// output projections run over B * q_len rows; the core keeps one partial per
// segment and token.
DecodeLayout decode_layout(const mla_ctx* h, int Bs, int64_t total_rows, bool step,
                           int q_len = 1) {
  const Dims& d = h->d;
  DecodeLayout L;
  L.step = step;
  const int parts = max_parts(h, total_rows, q_len);
  L.max_segs = parts + Bs;
  const int B = Bs * q_len;  // query rows
  // only sequences with more than kCombineChunk slots use chunk slots: there are
  // at most max_segs / (kCombineChunk + 1) of them, each with at most
  // nseg / kCombineChunk + 1 chunks (per token)
  L.max_cslots = (2 * (L.max_segs / mla::kCombineChunk) + 2) * q_len;
  const int qw = qw_of(d);
  const size_t scr = std::max({out_scratch(h, B, d.dc, d.dn, d.H),
                               out_scratch(h, B, d.dv, d.dc, d.H),
                               out_scratch(h, B, d.D, d.H * d.dv, 1)});
  // partials of the first projection (in-projection for a step, else q or q_a)
  size_t pin = 0, pq = 0;
  if (step) pin = part_floats(h, B, h->n_in, d.D);
  else pin = part_floats(h, B, d.dq ? d.dq : qw, d.D);
  if (d.dq) pq = part_floats(h, B, qw, d.dq);
  const size_t e = h->esz;
  Carve c;
  L.meta = c.take(meta_bytes(Bs, parts, L.max_segs, total_rows, q_len));
  L.scratch = c.take(scr * 4);
  L.pin = c.take(pin * 4);
  L.pq = c.take(pq * 4);
  L.cq = c.take(d.dq ? (size_t)B * d.dq * e : 0);
  L.q_nope = c.take((size_t)B * d.H * d.dn * e);
  L.q_cat = c.take((size_t)B * d.H * d.R * e);
  L.acc = c.take((size_t)L.max_segs * q_len * d.H * d.dc * 4);
  L.ml = c.take((size_t)L.max_segs * q_len * d.H * 2 * 4);
  L.cacc = c.take((size_t)L.max_cslots * d.H * d.dc * 4);
  L.cml = c.take((size_t)L.max_cslots * d.H * 2 * 4);
  L.o_lat = c.take((size_t)B * d.H * d.dc * e);
  L.o = c.take((size_t)B * d.H * d.dv * e);
  // the fused path's few-row products over the tiled weights (W_o, q_b, the
  // first projection) may split K
  size_t rp = 0;
  if (h->mfma) {
    auto res = [&](int N, int K) {
      const int ns = mla::res_slices(B, N, K);
      rp = std::max(rp, ns > 1 ? (size_t)ns * B * N : (size_t)0);
    };
    res(d.D, d.H * d.dv);
    res(step ? h->n_in : (d.dq ? d.dq : qw), d.D);
    if (d.dq) res(qw, d.dq);
  }
  L.rpart = c.take(rp * 4);
  L.total = c.off;
  return L;
}

struct MetaOffsets {
  size_t seq_off, seq_len, pos, pstart, nseg, cstart, part, segs, work, slot, pg_off, pages;
  size_t vpstart, vnseg, vcstart;  // the combine's view: one virtual sequence per query row
};

// A paged cache view (NULL for a contiguous cache): block_table (B x max_pages,
// host) lists the pages of each sequence, pages hold page_rows = 2^shift rows.
struct PageArgs {
  const int32_t* table;
  int32_t max_pages, page_rows, shift;
};

int64_t paged_row(const PageArgs& pg, int b, int64_t t) {
  return (int64_t)pg.table[(int64_t)b * pg.max_pages + (t >> pg.shift)] * pg.page_rows +
         (t & (pg.page_rows - 1));
}

// Host-side work list.  The concatenated rows of all sequences are cut into
// at most `max_parts(total)` contiguous spans, one persistent workgroup each,
// and every span is split at sequence boundaries into segments.  A segment
// start costs its workgroup about kSegRows rows' worth of time (pipeline
// restart, query load, wave merge and partial write), so spans are balanced
// on rows + kSegRows * segments: the smallest per-part budget for which a
// greedy left-to-right fill needs no more than the available parts is found by
// bisection.  Cuts inside a sequence fall on 32-row tile boundaries (kCutAlign).
constexpr int64_t kSegRows = MLA_SEG_ROWS;
constexpr int64_t kCutAlign = 32;  // rows per tile of the MFMA cores

struct SpanPlan {
  std::vector<DecodeSeg> segs;
  std::vector<int32_t> part_begin;
};

// Greedy fill with per-part budget `budget`; returns the parts used.
// min_tail: the last segment of every sequence keeps at least this many rows
// (its q_len new tokens mask their last rows there; no segment is left empty
// for any of them).
int fill_spans(int B, const int32_t* seq_len, int64_t budget, SpanPlan* plan, int min_tail = 1) {
  if (plan) {
    plan->segs.clear();
    plan->part_begin.assign(1, 0);
  }
  int used = 0;
  int64_t cost = 0;  // cost of the open part; 0 = no part open
  for (int b = 0; b < B; ++b) {
    int32_t in_b = 0;
    while (in_b < seq_len[b]) {
      const int64_t rem = seq_len[b] - in_b;
      int64_t room = budget - cost - kSegRows;
      if (cost > 0 && room < std::min<int64_t>(rem, kCutAlign)) {
        if (plan) plan->part_begin.push_back((int32_t)plan->segs.size());
        cost = 0;  // close the part, open a new one below
        continue;
      }
      if (cost == 0) ++used;
      int64_t take = rem;
      if (take > room) take = std::max<int64_t>(kCutAlign, room / kCutAlign * kCutAlign);
      if (take > rem) take = rem;
      if (take < rem && rem - take < min_tail) {  // leave a long enough last segment
        const int64_t t2 = (rem - min_tail) / kCutAlign * kCutAlign;
        take = t2 >= kCutAlign ? t2 : rem;
      }
      if (plan)
        plan->segs.push_back(
            DecodeSeg{b, in_b, (int32_t)(in_b + take), (int32_t)plan->segs.size()});
      cost += kSegRows + take;
      in_b += (int32_t)take;
    }
  }
  if (plan && cost > 0) plan->part_begin.push_back((int32_t)plan->segs.size());
  return used;
}

// Balanced plan over at most max_p parts; returns the parts used.
int plan_spans(int B, const int32_t* seq_len, int max_p, SpanPlan* plan, int min_tail = 1) {
  int64_t total = 0;
  for (int b = 0; b < B; ++b) total += seq_len[b];
  int64_t lo = (total + max_p - 1) / max_p, hi = lo + kSegRows * 2 + kCutAlign;
  while (fill_spans(B, seq_len, hi, nullptr, min_tail) > max_p) hi *= 2;
  while (lo < hi) {  // smallest budget that fits
    const int64_t mid = lo + (hi - lo) / 2;
    if (fill_spans(B, seq_len, mid, nullptr, min_tail) <= max_p) hi = mid;
    else lo = mid + 1;
  }
  return fill_spans(B, seq_len, hi, plan, min_tail);
}

// Query row b * q_len + j is token j of sequence b, at position
// seq_len[b] - q_len + j.
int build_decode_meta(const mla_ctx* h, int B, const int64_t* seq_off, const int32_t* seq_len,
                      int q_len, int64_t total, bool with_slot, const PageArgs* pg,
                      std::vector<char>& blob, MetaOffsets* mo, int* nseg_total, int* max_chunks,
                      int* cslots) {
  SpanPlan plan;
  const int parts = plan_spans(B, seq_len, max_parts(h, total, q_len), &plan, q_len);
  const int Bq = B * q_len;
  std::vector<DecodeSeg>& segs = plan.segs;
  std::vector<int32_t>& part_begin = plan.part_begin;
  std::vector<int32_t> pstart(B, 0), nseg(B, 0);
  for (const DecodeSeg& sg : segs) {
    if (sg.r0 == 0) pstart[sg.b] = sg.pidx;
    nseg[sg.b]++;
  }
  // chunk slots of the combine's second pass, for sequences with several chunks
  std::vector<int32_t> cstart(B, 0);
  *max_chunks = 1;
  *cslots = 0;
  for (int b = 0; b < B; ++b) {
    const int nch = (nseg[b] + mla::kCombineChunk - 1) / mla::kCombineChunk;
    *max_chunks = std::max(*max_chunks, nch);
    if (nch > 1) {
      cstart[b] = *cslots;
      *cslots += nch;
    }
  }
  // the combine's view: query row b * q_len + j is a sequence of its own whose
  // partials are slots j * nseg_total + pstart[b] ..; chunk slots likewise
  const int cs_real = *cslots;
  const int nsegs = (int)segs.size();
  std::vector<int32_t> vpstart(Bq), vnseg(Bq), vcstart(Bq), qpos(Bq);
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < q_len; ++j) {
      const int i = b * q_len + j;
      vpstart[i] = j * nsegs + pstart[b];
      vnseg[i] = nseg[b];
      vcstart[i] = j * cs_real + cstart[b];
      qpos[i] = seq_len[b] - q_len + j;
    }
  *cslots = cs_real * q_len;
  Carve c;
  mo->seq_off = c.take((size_t)B * 8);
  mo->slot = c.take(with_slot ? (size_t)Bq * 8 : 0);
  mo->seq_len = c.take((size_t)B * 4);
  mo->pos = c.take((size_t)Bq * 4);
  mo->pstart = c.take((size_t)B * 4);
  mo->nseg = c.take((size_t)B * 4);
  mo->cstart = c.take((size_t)B * 4);
  mo->vpstart = c.take((size_t)Bq * 4);
  mo->vnseg = c.take((size_t)Bq * 4);
  mo->vcstart = c.take((size_t)Bq * 4);
  mo->part = c.take((size_t)(parts + 1) * 4);
  mo->segs = c.take(segs.size() * sizeof(DecodeSeg));
  mo->work = c.take(segs.size() * sizeof(mla::DecodeWork));
  // paged: each sequence's used pages, back to back (pg_off[b]: its first)
  std::vector<int32_t> pg_off;
  int64_t npages = 0;
  if (pg) {
    pg_off.resize(B);
    for (int b = 0; b < B; ++b) {
      pg_off[b] = (int32_t)npages;
      npages += (seq_len[b] + pg->page_rows - 1) / pg->page_rows;
    }
  }
  mo->pg_off = c.take(pg ? (size_t)B * 4 : 0);
  mo->pages = c.take((size_t)npages * 4);
  blob.assign(c.off, 0);
  if (pg) {
    memcpy(blob.data() + mo->pg_off, pg_off.data(), (size_t)B * 4);
    int32_t* pl = reinterpret_cast<int32_t*>(blob.data() + mo->pages);
    for (int b = 0; b < B; ++b) {
      const int np = (seq_len[b] + pg->page_rows - 1) / pg->page_rows;
      memcpy(pl + pg_off[b], pg->table + (int64_t)b * pg->max_pages, (size_t)np * 4);
    }
  } else {
    memcpy(blob.data() + mo->seq_off, seq_off, (size_t)B * 8);
  }
  if (with_slot) {
    int64_t* sl = reinterpret_cast<int64_t*>(blob.data() + mo->slot);
    for (int i = 0; i < Bq; ++i) {
      const int b = i / q_len;
      sl[i] = pg ? paged_row(*pg, b, qpos[i]) : seq_off[b] + qpos[i];
    }
  }
  memcpy(blob.data() + mo->seq_len, seq_len, (size_t)B * 4);
  memcpy(blob.data() + mo->pos, qpos.data(), (size_t)Bq * 4);
  memcpy(blob.data() + mo->vpstart, vpstart.data(), (size_t)Bq * 4);
  memcpy(blob.data() + mo->vnseg, vnseg.data(), (size_t)Bq * 4);
  memcpy(blob.data() + mo->vcstart, vcstart.data(), (size_t)Bq * 4);
  memcpy(blob.data() + mo->pstart, pstart.data(), (size_t)B * 4);
  memcpy(blob.data() + mo->nseg, nseg.data(), (size_t)B * 4);
  memcpy(blob.data() + mo->cstart, cstart.data(), (size_t)B * 4);
  memcpy(blob.data() + mo->part, part_begin.data(), part_begin.size() * 4);
  memcpy(blob.data() + mo->segs, segs.data(), segs.size() * sizeof(DecodeSeg));
  {
    // work records: part p's first segment at p, the rest chained after the parts
    std::vector<mla::DecodeWork> work(segs.size());
    int extra = parts;
    for (int p = 0; p < parts; ++p) {
      int slot = p;
      for (int si = part_begin[p]; si < part_begin[p + 1]; ++si) {
        const DecodeSeg& sg = segs[si];
        mla::DecodeWork& w = work[slot];
        w.row = pg ? ((int64_t)pg_off[sg.b] << 32) | sg.r0 : seq_off[sg.b] + sg.r0;
        w.n = sg.r1 - sg.r0;
        w.b = sg.b;
        w.pidx = sg.pidx;
        w.next = -1;
        w.nseg = nseg[sg.b];
        w.pstart = pstart[sg.b];
        if (si + 1 < part_begin[p + 1]) {
          w.next = extra;
          slot = extra++;
        }
      }
    }
    memcpy(blob.data() + mo->work, work.data(), work.size() * sizeof(mla::DecodeWork));
  }
  *nseg_total = (int)segs.size();
  return parts;
}

// Slot of the timing ring for the next core launch, or -1 (timing off, or the
// stream is being captured into a graph, where event records do not time).
int timing_slot(mla_ctx* h) {
  if (h->tev.empty()) return -1;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(h->stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return -1;
  const int slot = h->t_next;
  h->t_next = (h->t_next + 1) % (int)(h->tev.size() / 2);
  h->t_count++;
  return slot;
}

int check_ws(mla_ctx* h, void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MLA_OK;
  if (!ws) return fail(h, MLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (((uintptr_t)ws) % kAlign)
    return fail(h, MLA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(h, MLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return MLA_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

// ==========================================================================
// C ABI (linkage comes from the extern "C" declarations in mla.h)
// ==========================================================================

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_SHAPE: return "unsupported shape";
    case MLA_ERR_CAPACITY: return "cache capacity exceeded";
    case MLA_ERR_STATE: return "call out of order";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_WORKSPACE: return "workspace too small or misaligned";
    default: return "unknown status";
  }
}

const char* mla_last_error(mla_handle h) { return h ? h->err.c_str() : "null handle"; }

int mla_config_check(const mla_config* c) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->n_heads <= 0 || c->qk_nope <= 0 || c->v_head <= 0 || c->kv_lora <= 0)
    return MLA_ERR_INVALID_ARG;
  if (c->qk_rope < 0 || c->q_lora < 0) return MLA_ERR_INVALID_ARG;
  if (c->dtype != MLA_BF16 && c->dtype != MLA_F32) return MLA_ERR_INVALID_ARG;
  if (!(c->rope_base > 0.f) || !isfinite(c->rope_base)) return MLA_ERR_INVALID_ARG;
  if (!(c->rms_eps > 0.f) || !isfinite(c->rms_eps)) return MLA_ERR_INVALID_ARG;
  if (!(c->softmax_scale >= 0.f) || !isfinite(c->softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (c->qk_rope % 2) return MLA_ERR_SHAPE;  // RoPE rotates pairs
  // kernel limits of the VALU paths: latent width and v_head per thread block
  if (c->kv_lora > 1024 || c->v_head > 256) return MLA_ERR_SHAPE;
  if (c->qk_rope > 2 * mla::kMaxRopePairs) return MLA_ERR_SHAPE;
  if (c->kv_storage != MLA_KV_DTYPE && c->kv_storage != MLA_KV_FP8_E4M3)
    return MLA_ERR_INVALID_ARG;
  if (c->absorb != MLA_ABSORB_FACTORED && c->absorb != MLA_ABSORB_MATERIALIZED)
    return MLA_ERR_INVALID_ARG;
  if (!isfinite(c->rope_scale)) return MLA_ERR_INVALID_ARG;
  if (c->rope_scale > 1.f &&
      (c->rope_orig_max < 1 || !isfinite(c->yarn_beta_fast) || !isfinite(c->yarn_beta_slow) ||
       !(c->yarn_beta_slow > 0.f) || !(c->yarn_beta_fast > c->yarn_beta_slow) ||
       !isfinite(c->yarn_mscale) || !(c->yarn_mscale >= 0.f)))
    return MLA_ERR_INVALID_ARG;
  // materialised weights are read by the fused decode path of bf16 MFMA layers
  if (c->absorb == MLA_ABSORB_MATERIALIZED && (c->dtype != MLA_BF16 || c->kv_lora != 512))
    return MLA_ERR_SHAPE;
  if (c->kv_storage == MLA_KV_FP8_E4M3) {
    // the FP8 rows are read by the 16-head-group MFMA core only
    if (c->dtype != MLA_BF16 || c->kv_lora != 512 || c->qk_rope != 64 || c->n_heads % 16)
      return MLA_ERR_SHAPE;
  }
  return MLA_OK;
}

size_t mla_cache_row_bytes(const mla_config* c) {
  if (mla_config_check(c) != MLA_OK) return 0;
  if (c->kv_storage == MLA_KV_FP8_E4M3) return (size_t)mla::fp8_row_bytes(c->kv_lora, c->qk_rope);
  return (size_t)(c->kv_lora + c->qk_rope) * (c->dtype == MLA_F32 ? 4 : 2);
}

static int check_slots_pure(const int64_t* slot, int32_t T, int64_t cache_rows, int32_t* bad) {
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)T * 2);
  for (int32_t t = 0; t < T; ++t) {
    *bad = t;
    if (slot[t] < 0 || slot[t] >= cache_rows) return MLA_ERR_CAPACITY;
    if (!seen.insert(slot[t]).second) return MLA_ERR_INVALID_ARG;
  }
  return MLA_OK;
}

int mla_append_check(const mla_config* cfg, const int32_t* pos, const int64_t* slot, int32_t T,
                     int64_t cache_rows) {
  int rc = mla_config_check(cfg);
  if (rc) return rc;
  if (T <= 0 || !pos || !slot || cache_rows <= 0) return MLA_ERR_INVALID_ARG;
  for (int32_t t = 0; t < T; ++t)
    if (pos[t] < 0) return MLA_ERR_INVALID_ARG;
  int32_t bad = 0;
  return check_slots_pure(slot, T, cache_rows, &bad);
}

int mla_decode_check(const mla_config* cfg, const int32_t* pos, const int64_t* seq_off,
                     const int32_t* seq_len, int32_t B, int64_t cache_rows) {
  int rc = mla_config_check(cfg);
  if (rc) return rc;
  if (B <= 0 || !pos || !seq_off || !seq_len || cache_rows <= 0) return MLA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_len[b] < 1 || pos[b] != seq_len[b] - 1) return MLA_ERR_INVALID_ARG;
    if (seq_off[b] < 0 || seq_off[b] > cache_rows - seq_len[b]) return MLA_ERR_CAPACITY;
  }
  return MLA_OK;
}

// Rows a step writes (sorted in place) against the rows it reads: every
// written row is distinct, and none lies inside a half-open range of rows
// some sequence reads as already cached -- that row would be overwritten
// before the attention core reads it.  `cached(visit)` calls visit(r0, r1)
// for every such range.
template <typename Ranges>
static int write_read_check(std::vector<int64_t>& w, Ranges cached) {
  std::sort(w.begin(), w.end());
  if (std::adjacent_find(w.begin(), w.end()) != w.end()) return MLA_ERR_INVALID_ARG;
  bool clash = false;
  cached([&](int64_t r0, int64_t r1) {
    auto it = std::lower_bound(w.begin(), w.end(), r0);
    if (it != w.end() && *it < r1) clash = true;
  });
  return clash ? MLA_ERR_INVALID_ARG : MLA_OK;
}

// The new rows of a step on a contiguous cache: q_len rows at the end of
// every sequence's range.
static int contig_write_check(const int64_t* seq_off, const int32_t* seq_len, int32_t B,
                              int q_len) {
  std::vector<int64_t> w;
  w.reserve((size_t)B * q_len);
  for (int32_t b = 0; b < B; ++b)
    for (int j = 0; j < q_len; ++j) w.push_back(seq_off[b] + seq_len[b] - q_len + j);
  return write_read_check(w, [&](auto visit) {
    for (int32_t b = 0; b < B; ++b)
      if (seq_len[b] > q_len) visit(seq_off[b], seq_off[b] + seq_len[b] - q_len);
  });
}

// The block table of a paged decode: page size, table width, every used page
// in range; with `writes`, the q_len new rows of every sequence land on
// distinct cache rows, none of them on a row any sequence reads as cached
// (pages may be shared between sequences).
static int paged_table_check(const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                             const int32_t* seq_len, int32_t B, int64_t cache_rows, int q_len,
                             int32_t writes) {
  if (!block_table || max_pages <= 0) return MLA_ERR_INVALID_ARG;
  if (page_rows < 32 || page_rows > (1 << 30) || (page_rows & (page_rows - 1)))
    return MLA_ERR_INVALID_ARG;
  const int64_t n_pages = cache_rows / page_rows;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t np = ((int64_t)seq_len[b] + page_rows - 1) / page_rows;
    if (np > max_pages) return MLA_ERR_CAPACITY;
    const int32_t* row = block_table + (int64_t)b * max_pages;
    for (int64_t i = 0; i < np; ++i)
      if (row[i] < 0 || row[i] >= n_pages) return MLA_ERR_CAPACITY;
  }
  if (writes) {  // the new rows of a step: one cache row each
    std::vector<int64_t> w;
    w.reserve((size_t)B * q_len);
    for (int32_t b = 0; b < B; ++b)
      for (int j = 0; j < q_len; ++j) {
        const int32_t t = seq_len[b] - q_len + j;
        w.push_back((int64_t)block_table[(int64_t)b * max_pages + t / page_rows] * page_rows +
                    t % page_rows);
      }
    return write_read_check(w, [&](auto visit) {
      for (int32_t b = 0; b < B; ++b) {
        const int64_t cached = (int64_t)seq_len[b] - q_len;  // positions read, not written
        const int32_t* row = block_table + (int64_t)b * max_pages;
        for (int64_t t0 = 0; t0 < cached; t0 += page_rows)
          visit((int64_t)row[t0 / page_rows] * page_rows,
                (int64_t)row[t0 / page_rows] * page_rows + std::min<int64_t>(page_rows, cached - t0));
      }
    });
  }
  return MLA_OK;
}

int mla_decode_paged_check(const mla_config* cfg, const int32_t* pos, const int32_t* block_table,
                           int32_t max_pages, int32_t page_rows, const int32_t* seq_len, int32_t B,
                           int64_t cache_rows, int32_t writes) {
  int rc = mla_config_check(cfg);
  if (rc) return rc;
  if (B <= 0 || !pos || !block_table || !seq_len || cache_rows <= 0 || max_pages <= 0)
    return MLA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b)
    if (seq_len[b] < 1 || pos[b] != seq_len[b] - 1) return MLA_ERR_INVALID_ARG;
  return paged_table_check(block_table, max_pages, page_rows, seq_len, B, cache_rows, 1, writes);
}

int mla_decode_ex_check(const mla_config* cfg, const mla_decode_args* a) {
  int rc = mla_config_check(cfg);
  if (rc) return rc;
  if (!a || a->B <= 0 || !a->seq_len || a->cache_rows <= 0) return MLA_ERR_INVALID_ARG;
  if (a->q_len < 1 || a->q_len > MLA_MAX_Q_LEN) return MLA_ERR_INVALID_ARG;
  if ((a->seq_off != nullptr) == (a->block_table != nullptr)) return MLA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < a->B; ++b)
    if (a->seq_len[b] < a->q_len) return MLA_ERR_INVALID_ARG;
  if (a->block_table)
    return paged_table_check(a->block_table, a->max_pages, a->page_rows, a->seq_len, a->B,
                             a->cache_rows, a->q_len, a->append);
  for (int32_t b = 0; b < a->B; ++b)
    if (a->seq_off[b] < 0 || a->seq_off[b] > a->cache_rows - a->seq_len[b])
      return MLA_ERR_CAPACITY;
  return a->append ? contig_write_check(a->seq_off, a->seq_len, a->B, a->q_len) : MLA_OK;
}

int mla_prefill_check(const mla_config* cfg, const int32_t* cu_new, const int32_t* prior_len,
                      const int64_t* seq_off, int32_t B, int64_t cache_rows) {
  int rc = mla_config_check(cfg);
  if (rc) return rc;
  if (B <= 0 || !cu_new || !prior_len || !seq_off || cache_rows <= 0) return MLA_ERR_INVALID_ARG;
  if (cu_new[0] != 0) return MLA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b) {
    if (cu_new[b + 1] < cu_new[b] || prior_len[b] < 0) return MLA_ERR_INVALID_ARG;
    const int64_t len = (int64_t)prior_len[b] + (cu_new[b + 1] - cu_new[b]);
    if (len > INT32_MAX) return MLA_ERR_INVALID_ARG;  // positions are int32
    if (seq_off[b] < 0 || seq_off[b] > cache_rows - len) return MLA_ERR_CAPACITY;
  }
  if (cu_new[B] <= 0) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// The new rows of a prefill step on a contiguous cache: rows prior_len[b] ..
// prior_len[b] + n_b - 1 of every sequence, distinct, none of them a row any
// sequence reads as already cached.
int mla_prefill_step_check(const mla_config* cfg, const int32_t* cu_new, const int32_t* prior_len,
                           const int64_t* seq_off, int32_t B, int64_t cache_rows) {
  const int rc = mla_prefill_check(cfg, cu_new, prior_len, seq_off, B, cache_rows);
  if (rc) return rc;
  std::vector<int64_t> w;
  w.reserve((size_t)cu_new[B]);
  for (int32_t b = 0; b < B; ++b)
    for (int32_t i = 0; i < cu_new[b + 1] - cu_new[b]; ++i)
      w.push_back(seq_off[b] + prior_len[b] + i);
  return write_read_check(w, [&](auto visit) {
    for (int32_t b = 0; b < B; ++b)
      if (prior_len[b] > 0) visit(seq_off[b], seq_off[b] + prior_len[b]);
  });
}

int mla_prefill_paged_check(const mla_config* cfg, const int32_t* cu_new,
                            const int32_t* prior_len, const int32_t* block_table,
                            int32_t max_pages, int32_t page_rows, int32_t B, int64_t cache_rows) {
  int rc = mla_config_check(cfg);
  if (rc) return rc;
  if (B <= 0 || !cu_new || !prior_len || !block_table || cache_rows <= 0 || max_pages <= 0)
    return MLA_ERR_INVALID_ARG;
  if (cu_new[0] != 0) return MLA_ERR_INVALID_ARG;
  std::vector<int32_t> len(B);
  for (int32_t b = 0; b < B; ++b) {
    if (cu_new[b + 1] < cu_new[b] || prior_len[b] < 0) return MLA_ERR_INVALID_ARG;
    const int64_t l = (int64_t)prior_len[b] + (cu_new[b + 1] - cu_new[b]);
    if (l > INT32_MAX) return MLA_ERR_INVALID_ARG;
    len[b] = (int32_t)l;
  }
  if (cu_new[B] <= 0) return MLA_ERR_INVALID_ARG;
  // the prefill only reads the cache: the caller appends the new rows first
  return paged_table_check(block_table, max_pages, page_rows, len.data(), B, cache_rows, 1, 0);
}

// RoPE frequency of every pair (dr / 2 of them), YaRN-interpolated for
// rope_scale > 1: plain theta_i below the blend band, theta_i / s above it,
// linear in the pair index across it (band ends: the pair indices that turn
// yarn_beta_fast and yarn_beta_slow times over the original context, floored
// and ceiled).
static void yarn_table(const mla_config* cfg, double* theta) {
  const int half = cfg->qk_rope / 2;
  const double base = cfg->rope_base;
  double lo = 0.0, hi = 1.0;
  if (cfg->rope_scale > 1.f) {
    auto pair_at = [&](double turns) {
      return cfg->qk_rope * log(cfg->rope_orig_max / (2.0 * M_PI * turns)) / (2.0 * log(base));
    };
    lo = std::max(floor(pair_at(cfg->yarn_beta_fast)), 0.0);
    hi = std::min(ceil(pair_at(cfg->yarn_beta_slow)), (double)(half - 1));
    if (hi <= lo) hi = lo + 0.001;
  }
  for (int i = 0; i < half; ++i) {
    const double th = pow(base, -2.0 * i / (double)cfg->qk_rope);
    double f = th;
    if (cfg->rope_scale > 1.f) {
      const double w = std::min(1.0, std::max(0.0, (i - lo) / (hi - lo)));
      f = (1.0 - w) * th + w * th / cfg->rope_scale;
    }
    theta[i] = f;
  }
}

// Device address of each device's static scratch array (scratch.hip), taken
// once per device with that device current.
static std::mutex g_scratch_mu;
static void* g_scratch[256];

static hipError_t noalloc_setup(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = mla::noalloc_scratch_address(&p);
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

int mla_create(const mla_config* cfg, void* stream, mla_handle* out) {
  if (!out) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  int rc = mla_config_check(cfg);
  if (rc != MLA_OK) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  mla_ctx* h = new mla_ctx();
  h->cfg = *cfg;
  h->device = dev;
  h->stream = (hipStream_t)stream;
  h->esz = cfg->dtype == MLA_F32 ? 4 : 2;
  Dims& d = h->d;
  d.D = cfg->hidden; d.H = cfg->n_heads; d.dn = cfg->qk_nope; d.dr = cfg->qk_rope;
  d.dv = cfg->v_head; d.dc = cfg->kv_lora; d.dq = cfg->q_lora; d.R = d.dc + d.dr;
  d.rope_base = cfg->rope_base; d.eps = cfg->rms_eps;
  d.scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / sqrtf((float)(d.dn + d.dr));
  yarn_table(cfg, h->rope.theta);
  if (cfg->softmax_scale <= 0.f && cfg->rope_scale > 1.f) {
    // YaRN's attention factor on the default scale
    const double m = 0.1 * cfg->yarn_mscale * log((double)cfg->rope_scale) + 1.0;
    d.scale = (float)(m * m / sqrt((double)(d.dn + d.dr)));
  }
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      ncu > 0)
    h->n_cu = ncu;
  h->mfma = cfg->dtype == MLA_BF16 && d.dc == 512 && d.dr == 64 && d.H % 16 == 0;
  h->kv8 = cfg->kv_storage == MLA_KV_FP8_E4M3;
  h->n_in = d.R + (d.dq ? d.dq : qw_of(d));
  h->mat = cfg->absorb == MLA_ABSORB_MATERIALIZED;
  h->dims_aligned = d.D % 8 == 0 && d.dc % 8 == 0 && d.R % 8 == 0 && d.dq % 8 == 0 &&
                    qw_of(d) % 8 == 0 && (d.H * d.dv) % 8 == 0 &&
                    (d.H * (d.dn + d.dv)) % 8 == 0;
  // set-up of the no-allocation decode step: the scratch address and a
  // staging ring that already holds its pinned memory and events
  hipError_t e = noalloc_setup(dev, &h->noalloc_ws);
  for (auto& sl : h->ring) {
    if (e == hipSuccess) e = hipHostMalloc(&sl.host, kStageInit, hipHostMallocCoherent);
    if (e == hipSuccess) sl.cap = kStageInit;
    if (e == hipSuccess) e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    (void)mla_destroy(h);
    return MLA_ERR_HIP;
  }
  *out = h;
  mlog("create: device %d (%d CUs), H=%d D=%d dc=%d dr=%d dn=%d dv=%d q_lora=%d, %s, cache %s, "
       "absorption %s, decode core %s", h->device, h->n_cu, h->d.H, h->d.D, h->d.dc, h->d.dr,
       h->d.dn, h->d.dv, h->d.dq, is_f32(h) ? "fp32" : "bf16", h->kv8 ? "FP8 rows" : "dtype rows",
       h->cfg.absorb ? "materialised" : "factored", core_name(h));
  return MLA_OK;
}

static void free_weights(mla_ctx* h) {
  void** ws[] = {&h->w_q,  &h->w_qa, &h->q_norm_g, &h->w_qb,  &h->w_kva, &h->kv_norm_g,
                 &h->w_kvb, &h->w_ukT, &h->w_uv,   &h->w_o,   &h->w_in,  &h->t_in,
                 &h->t_q,   &h->t_qb,  &h->t_kva,  &h->t_kvb, &h->t_o,   &h->m_in,
                 &h->m_qb,  &h->m_ov};
  for (void** p : ws) {
    if (*p) (void)hipFree(*p);
    *p = nullptr;
  }
  h->absorbed = false;
}

static void drop_timing(mla_ctx* h);

int mla_destroy(mla_handle h) {
  if (!h) return MLA_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  (void)hipStreamSynchronize(h->stream);
  free_weights(h);
  for (auto& s : h->ring) {
    if (s.ev) (void)hipEventDestroy(s.ev);
    if (s.host) (void)hipHostFree(s.host);
  }
  for (void* p : h->captured) (void)hipHostFree(p);
  drop_timing(h);
  delete h;
  return MLA_OK;
}

static void drop_timing(mla_ctx* h) {
  for (hipEvent_t e : h->tev) (void)hipEventDestroy(e);
  h->tev.clear();
  h->t_next = 0;
  h->t_count = 0;
}

int mla_core_timing(mla_handle h, int32_t n_slots) {
  if (!h || n_slots < 0) return MLA_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  (void)hipStreamSynchronize(h->stream);
  drop_timing(h);
  for (int i = 0; i < 2 * n_slots; ++i) {
    hipEvent_t e;
    // no system-scope fence: recording must not write back or invalidate caches
    HIP_TRY(h, hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    h->tev.push_back(e);
  }
  return MLA_OK;
}

int mla_core_timing_read(mla_handle h, float* ms, int32_t n, int32_t* n_out) {
  if (!h || !ms || !n_out || n < 0) return MLA_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  const int slots = (int)h->tev.size() / 2;
  const int avail = (int)std::min<int64_t>(h->t_count, slots);
  const int k = std::min(n, avail);
  for (int i = 0; i < k; ++i) {
    const int slot = ((h->t_next - k + i) % slots + slots) % slots;
    HIP_TRY(h, hipEventSynchronize(h->tev[2 * slot + 1]));
    HIP_TRY(h, hipEventElapsedTime(&ms[i], h->tev[2 * slot], h->tev[2 * slot + 1]));
  }
  *n_out = k;
  return MLA_OK;
}

int mla_set_stream(mla_handle h, void* stream) {
  if (!h) return MLA_ERR_INVALID_ARG;
  h->stream = (hipStream_t)stream;
  return MLA_OK;
}

// Materialised absorption ("Multi-Head Latent Attention" post, section 3.5):
// per head W^KQ_h = W_UK_h^T W_q,nope_h (dc x K, K = D or q_lora) stacked with
// the head's rope rows of W_q (or W_qb), and W^OV_h = W_o,h W_UV_h (D x dc),
// formed once on the device in fp32 and stored in bf16.  Runs after the
// factored copies exist (w_ukT, w_uv, w_o, w_q / w_qb, w_kva).
static int materialize(mla_ctx* h) {
  const Dims& d = h->d;
  const int K = d.dq ? d.dq : d.D, qrow = d.dc + d.dr;
  const bf16* wq = static_cast<const bf16*>(d.dq ? h->w_qb : h->w_q);  // (H (dn + dr), K)
  void* wqT = nullptr;
  void* wuvT = nullptr;
  void* scr = nullptr;
  auto done = [&](int rc) {
    (void)hipStreamSynchronize(h->stream);
    for (void* p : {wqT, wuvT, scr})
      if (p) (void)hipFree(p);
    return rc;
  };
  const size_t sf = std::max(out_scratch(h, d.dc, K, d.dn, d.H), out_scratch(h, d.D, d.dc, d.dv, d.H));
  if (hipMalloc(&wqT, (size_t)d.H * K * d.dn * 2) != hipSuccess ||
      hipMalloc(&wuvT, (size_t)d.H * d.dc * d.dv * 2) != hipSuccess ||
      (sf && hipMalloc(&scr, sf * 4) != hipSuccess))
    return done(fail(h, MLA_ERR_HIP, "materialised absorption: out of device memory"));
  bf16* qdst;
  if (!d.dq) {
    if (hipMalloc(&h->m_in, ((size_t)d.R + (size_t)d.H * qrow) * d.D * 2) != hipSuccess)
      return done(fail(h, MLA_ERR_HIP, "materialised absorption: out of device memory"));
    if (hipMemcpyAsync(h->m_in, h->w_kva, (size_t)d.R * d.D * 2, hipMemcpyDeviceToDevice,
                       h->stream) != hipSuccess)
      return done(fail(h, MLA_ERR_HIP, "materialised absorption: copy"));
    qdst = static_cast<bf16*>(h->m_in) + (size_t)d.R * d.D;
  } else {
    if (hipMalloc(&h->m_qb, (size_t)d.H * qrow * d.dq * 2) != hipSuccess)
      return done(fail(h, MLA_ERR_HIP, "materialised absorption: out of device memory"));
    qdst = static_cast<bf16*>(h->m_qb);
  }
  // W_q,nope_h^T (H, K, dn), then W^KQ_h = W_UK_h^T (dc x dn) . (W_q,nope_h^T)^T
  mla::transpose_heads<bf16>(wq, static_cast<bf16*>(wqT), d.H, d.dn, K, (int64_t)(d.dn + d.dr) * K,
                             h->stream);
  gemm_out<bf16>(h, static_cast<const bf16*>(h->w_ukT), d.dn, (int64_t)d.dc * d.dn,
                 static_cast<const bf16*>(wqT), d.dn, (int64_t)K * d.dn, d.dc, K, d.dn, d.H,
                 out_t<bf16>(qdst, K, (int64_t)qrow * K), static_cast<float*>(scr));
  // the head's rope rows follow its W^KQ rows
  if (d.dr &&
      hipMemcpy2DAsync(qdst + (size_t)d.dc * K, (size_t)qrow * K * 2, wq + (size_t)d.dn * K,
                       (size_t)(d.dn + d.dr) * K * 2, (size_t)d.dr * K * 2, d.H,
                       hipMemcpyDeviceToDevice, h->stream) != hipSuccess)
    return done(fail(h, MLA_ERR_HIP, "materialised absorption: copy"));
  // W_UV_h^T (H, dc, dv), then W^OV_h = W_o,h (D x dv) . (W_UV_h^T)^T into
  // columns h dc .. of (D, H dc)
  mla::transpose_heads<bf16>(static_cast<const bf16*>(h->w_uv), static_cast<bf16*>(wuvT), d.H,
                             d.dv, d.dc, (int64_t)d.dv * d.dc, h->stream);
  if (hipMalloc(&h->m_ov, (size_t)d.D * d.H * d.dc * 2) != hipSuccess)
    return done(fail(h, MLA_ERR_HIP, "materialised absorption: out of device memory"));
  gemm_out<bf16>(h, static_cast<const bf16*>(h->w_o), (int64_t)d.H * d.dv, d.dv,
                 static_cast<const bf16*>(wuvT), d.dv, (int64_t)d.dc * d.dv, d.D, d.dc, d.dv,
                 d.H, out_t<bf16>(static_cast<bf16*>(h->m_ov), (int64_t)d.H * d.dc, d.dc),
                 static_cast<float*>(scr));
  return done(check_launch(h, "materialised absorption"));
}

int mla_absorb_weights(mla_handle h, const void* w_q, const void* w_qa, const void* q_norm_g,
                       const void* w_qb, const void* w_kva, const void* kv_norm_g,
                       const void* w_kvb, const void* w_o) {
  if (!h) return MLA_ERR_INVALID_ARG;
  const Dims& d = h->d;
  if (d.dq) {
    if (!w_qa || !q_norm_g || !w_qb || w_q)
      return fail(h, MLA_ERR_INVALID_ARG, "q_lora > 0 needs w_qa, q_norm_g, w_qb and no w_q");
  } else if (!w_q || w_qa || q_norm_g || w_qb) {
    return fail(h, MLA_ERR_INVALID_ARG, "q_lora == 0 needs w_q and no w_qa/q_norm_g/w_qb");
  }
  if (!w_kva || !w_kvb || !w_o) return fail(h, MLA_ERR_INVALID_ARG, "missing weight pointer");
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  free_weights(h);
  const size_t e = h->esz;
  auto dup = [&](void** dst, const void* src, size_t n) -> int {
    HIP_TRY(h, hipMalloc(dst, n * e));
    HIP_TRY(h, hipMemcpyAsync(*dst, src, n * e, hipMemcpyDeviceToDevice, h->stream));
    return MLA_OK;
  };
  int rc;
  const size_t qw = (size_t)qw_of(d);
  if (d.dq) {
    if ((rc = dup(&h->w_qa, w_qa, (size_t)d.dq * d.D))) return rc;
    if ((rc = dup(&h->q_norm_g, q_norm_g, (size_t)d.dq))) return rc;
    if ((rc = dup(&h->w_qb, w_qb, qw * d.dq))) return rc;
  } else if ((rc = dup(&h->w_q, w_q, qw * d.D))) {
    return rc;
  }
  if ((rc = dup(&h->w_kva, w_kva, (size_t)d.R * d.D))) return rc;
  if (kv_norm_g) {
    if ((rc = dup(&h->kv_norm_g, kv_norm_g, (size_t)d.dc))) return rc;
  }
  if ((rc = dup(&h->w_kvb, w_kvb, (size_t)d.H * (d.dn + d.dv) * d.dc))) return rc;
  if ((rc = dup(&h->w_o, w_o, (size_t)d.D * d.H * d.dv))) return rc;
  // in-projection rows [W_kva ; W_q] (or [W_kva ; W_qa]): both read the hidden state
  HIP_TRY(h, hipMalloc(&h->w_in, (size_t)h->n_in * d.D * e));
  HIP_TRY(h, hipMemcpyAsync(h->w_in, w_kva, (size_t)d.R * d.D * e, hipMemcpyDeviceToDevice,
                            h->stream));
  HIP_TRY(h, hipMemcpyAsync(static_cast<char*>(h->w_in) + (size_t)d.R * d.D * e,
                            d.dq ? w_qa : w_q, (size_t)(h->n_in - d.R) * d.D * e,
                            hipMemcpyDeviceToDevice, h->stream));
  // W_UV per head: rows dn .. dn+dv of each head's kv_b block, packed (H, dv, dc)
  HIP_TRY(h, hipMalloc(&h->w_uv, (size_t)d.H * d.dv * d.dc * e));
  HIP_TRY(h, hipMemcpy2DAsync(h->w_uv, (size_t)d.dv * d.dc * e,
                              static_cast<const char*>(w_kvb) + (size_t)d.dn * d.dc * e,
                              (size_t)(d.dn + d.dv) * d.dc * e, (size_t)d.dv * d.dc * e, d.H,
                              hipMemcpyDeviceToDevice, h->stream));
  // W_UK^T per head (H, dc, dn) through a transposing copy
  HIP_TRY(h, hipMalloc(&h->w_ukT, (size_t)d.H * d.dc * d.dn * e));
  if (is_f32(h))
    mla::transpose_heads<float>((const float*)w_kvb, (float*)h->w_ukT, d.H, d.dn, d.dc,
                                (int64_t)(d.dn + d.dv) * d.dc, h->stream);
  else
    mla::transpose_heads<bf16>((const bf16*)w_kvb, (bf16*)h->w_ukT, d.H, d.dn, d.dc,
                               (int64_t)(d.dn + d.dv) * d.dc, h->stream);
  if ((rc = check_launch(h, "transpose_heads"))) return rc;
  if (h->mat && !is_f32(h) && (rc = materialize(h))) return rc;
  // tiled copies for the large-tile GEMM (prefill, bulk appends, wide steps)
  if (!is_f32(h) && h->dims_aligned) {
    auto tile = [&](void** dst, const void* src, int rows, int K) -> int {
      if (K % 32) return MLA_OK;
      HIP_TRY(h, hipMalloc(dst, mla::tiled_bytes(rows, K)));
      mla::tile_rows(static_cast<const bf16*>(src), K, rows, K, static_cast<bf16*>(*dst),
                     h->stream);
      return check_launch(h, "tile_rows");
    };
    if ((rc = tile(&h->t_in, h->w_in, h->n_in, d.D))) return rc;
    if ((rc = tile(&h->t_q, d.dq ? h->w_qa : h->w_q, d.dq ? d.dq : (int)qw, d.D))) return rc;
    if (d.dq && (rc = tile(&h->t_qb, h->w_qb, (int)qw, d.dq))) return rc;
    if ((rc = tile(&h->t_kva, h->w_kva, d.R, d.D))) return rc;
    if ((rc = tile(&h->t_kvb, h->w_kvb, d.H * (d.dn + d.dv), d.dc))) return rc;
    if ((rc = tile(&h->t_o, h->w_o, d.D, d.H * d.dv))) return rc;
  }
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  h->absorbed = true;
  return MLA_OK;
}

// ------------------------------------------------------------------------
// append
// ------------------------------------------------------------------------
namespace {
struct AppendLayout {
  size_t pos, slot, part, total;
};
AppendLayout append_layout(const mla_ctx* h, int T) {
  AppendLayout L;
  Carve c;
  L.pos = c.take((size_t)T * 4);
  L.slot = c.take((size_t)T * 8);
  L.part = c.take(part_floats(h, T, h->d.R, h->d.D) * 4);
  L.total = c.off;
  return L;
}
}  // namespace

size_t mla_append_workspace_bytes(mla_handle h, int32_t T) {
  if (!h || T <= 0) return 0;
  return append_layout(h, T).total;
}

template <typename T>
static void run_append(mla_ctx* h, const T* hidden, int ntok, T* cache, void* ws,
                       const AppendLayout& L) {
  const Dims& d = h->d;
  const mla::Part a =
      gemm_part<T>(h, hidden, d.D, (const T*)h->w_kva, d.D, ntok, d.R, d.D, at<float>(ws, L.part),
                   h->t_kva);
  mla::append_rows<T>(a, ntok, at<int32_t>(ws, L.pos), at<int64_t>(ws, L.slot),
                      (const T*)h->kv_norm_g, cache, d, h->rope, h->stream);
}

int mla_append_latent(mla_handle h, const void* hidden, const int32_t* pos, const int64_t* slot,
                      int32_t T, void* cache, int64_t cache_rows, void* ws, size_t ws_bytes) {
  if (!h) return MLA_ERR_INVALID_ARG;
  if (!hidden || !cache) return fail(h, MLA_ERR_INVALID_ARG, "append: NULL tensor");
  int rc = mla_append_check(&h->cfg, pos, slot, T, cache_rows);
  if (rc) return fail(h, rc, "append: %s (T=%d, cache_rows=%lld)", mla_status_string(rc), T,
                      (long long)cache_rows);
  if (!h->absorbed) return fail(h, MLA_ERR_STATE, "append before mla_absorb_weights");
  const AppendLayout L = append_layout(h, T);
  if ((rc = check_ws(h, ws, ws_bytes, L.total))) return rc;
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  std::vector<char> blob(L.part, 0);
  memcpy(blob.data() + L.pos, pos, (size_t)T * 4);
  memcpy(blob.data() + L.slot, slot, (size_t)T * 8);
  if ((rc = stage_upload(h, ws, blob.data(), blob.size()))) return rc;
  if (is_f32(h)) {
    run_append<float>(h, (const float*)hidden, T, (float*)cache, ws, L);
  } else if (h->kv8) {
    const Dims& d = h->d;
    const mla::Part a = gemm_part<bf16>(h, (const bf16*)hidden, d.D, (const bf16*)h->w_kva, d.D, T,
                                        d.R, d.D, at<float>(ws, L.part), h->t_kva);
    mla::append_rows_fp8(a, T, at<int32_t>(ws, L.pos), at<int64_t>(ws, L.slot),
                         (const bf16*)h->kv_norm_g, (uint8_t*)cache, d, h->rope, h->stream);
  } else {
    run_append<bf16>(h, (const bf16*)hidden, T, (bf16*)cache, ws, L);
  }
  return check_launch(h, "append");
}

size_t mla_cache_write_workspace_bytes(mla_handle h, int32_t T) {
  if (!h || T <= 0) return 0;
  return align_up((size_t)T * 8);
}

int mla_cache_write(mla_handle h, const void* rows, const int64_t* slot, int32_t T, void* cache,
                    int64_t cache_rows, void* ws, size_t ws_bytes) {
  if (!h) return MLA_ERR_INVALID_ARG;
  if (T <= 0 || !rows || !slot || !cache || cache_rows <= 0)
    return fail(h, MLA_ERR_INVALID_ARG, "cache_write: bad argument (T=%d)", T);
  int32_t bad = 0;
  int rc = check_slots_pure(slot, T, cache_rows, &bad);
  if (rc) return fail(h, rc, "cache_write: slot[%d] = %lld is out of range or repeated", bad,
                      (long long)slot[bad]);
  if ((rc = check_ws(h, ws, ws_bytes, mla_cache_write_workspace_bytes(h, T)))) return rc;
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  if ((rc = stage_upload(h, ws, slot, (size_t)T * 8))) return rc;
  if (h->kv8)
    mla::cache_write_bytes((const uint8_t*)rows, (const int64_t*)ws, T,
                           (int)mla_cache_row_bytes(&h->cfg), (uint8_t*)cache, h->stream);
  else if (is_f32(h))
    mla::cache_write<float>((const float*)rows, (const int64_t*)ws, T, h->d.R, (float*)cache,
                            h->stream);
  else
    mla::cache_write<bf16>((const bf16*)rows, (const int64_t*)ws, T, h->d.R, (bf16*)cache,
                           h->stream);
  return check_launch(h, "cache_write");
}

int mla_cache_store(mla_handle h, const void* rows, const int64_t* slot, int32_t T, void* cache,
                    int64_t cache_rows, void* ws, size_t ws_bytes) {
  if (!h) return MLA_ERR_INVALID_ARG;
  if (!h->kv8) return mla_cache_write(h, rows, slot, T, cache, cache_rows, ws, ws_bytes);
  if (T <= 0 || !rows || !slot || !cache || cache_rows <= 0)
    return fail(h, MLA_ERR_INVALID_ARG, "cache_store: bad argument (T=%d)", T);
  int32_t bad = 0;
  int rc = check_slots_pure(slot, T, cache_rows, &bad);
  if (rc) return fail(h, rc, "cache_store: slot[%d] = %lld is out of range or repeated", bad,
                      (long long)slot[bad]);
  if ((rc = check_ws(h, ws, ws_bytes, mla_cache_write_workspace_bytes(h, T)))) return rc;
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  if ((rc = stage_upload(h, ws, slot, (size_t)T * 8))) return rc;
  mla::cache_store_fp8((const bf16*)rows, (const int64_t*)ws, T, (uint8_t*)cache, h->d,
                       h->stream);
  return check_launch(h, "cache_store");
}

// ------------------------------------------------------------------------
// decode
// ------------------------------------------------------------------------
size_t mla_decode_workspace_bytes(mla_handle h, int32_t B, int64_t total_rows) {
  if (!h || B <= 0 || total_rows <= 0) return 0;
  return decode_layout(h, B, total_rows, false).total;
}

size_t mla_decode_step_workspace_bytes(mla_handle h, int32_t B, int64_t total_rows) {
  if (!h || B <= 0 || total_rows <= 0) return 0;
  return decode_layout(h, B, total_rows, true).total;
}

int mla_decode_plan(int32_t B, const int32_t* seq_len, int32_t max_parts, int32_t* part_begin,
                    int32_t* seg_b, int32_t* seg_r0, int32_t* seg_r1, int32_t* n_parts,
                    int32_t* n_segs) {
  return mla_decode_plan_tokens(B, seq_len, 1, max_parts, part_begin, seg_b, seg_r0, seg_r1,
                                n_parts, n_segs);
}

int mla_decode_plan_tokens(int32_t B, const int32_t* seq_len, int32_t q_len, int32_t max_parts,
                           int32_t* part_begin, int32_t* seg_b, int32_t* seg_r0, int32_t* seg_r1,
                           int32_t* n_parts, int32_t* n_segs) {
  if (B <= 0 || max_parts <= 0 || !seq_len || !part_begin || !seg_b || !seg_r0 || !seg_r1 ||
      !n_parts || !n_segs || q_len < 1 || q_len > MLA_MAX_Q_LEN)
    return MLA_ERR_INVALID_ARG;
  for (int b = 0; b < B; ++b)
    if (seq_len[b] < q_len) return MLA_ERR_INVALID_ARG;
  SpanPlan plan;
  const int parts = plan_spans(B, seq_len, max_parts, &plan, q_len);
  for (int p = 0; p <= parts; ++p) part_begin[p] = plan.part_begin[p];
  for (size_t i = 0; i < plan.segs.size(); ++i) {
    seg_b[i] = plan.segs[i].b;
    seg_r0[i] = plan.segs[i].r0;
    seg_r1[i] = plan.segs[i].r1;
  }
  *n_parts = parts;
  *n_segs = (int32_t)plan.segs.size();
  return MLA_OK;
}

int mla_decode_stage_offsets(mla_handle h, int32_t B, int64_t total_rows, size_t* q_cat_off,
                             size_t* o_lat_off) {
  if (!h || B <= 0 || total_rows <= 0 || !q_cat_off || !o_lat_off) return MLA_ERR_INVALID_ARG;
  const DecodeLayout L = decode_layout(h, B, total_rows, false);
  *q_cat_off = L.q_cat;
  *o_lat_off = L.o_lat;
  return MLA_OK;
}

// A3 (+ A2 for a step): query projection, RoPE of the rope part (scaled into
// q_cat) and, for a step, the new latent rows.
template <typename T>
static void run_q_and_append(mla_ctx* h, const T* x, int B, void* ws, const DecodeLayout& L,
                             const DecodeMeta& mt, const int64_t* slot_dev, T* cache) {
  const Dims& d = h->d;
  const int qw = qw_of(d);
  T* q_nope = at<T>(ws, L.q_nope);
  T* q_rope = at<T>(ws, L.q_cat) + d.dc;
  const int64_t tok_stride = (int64_t)d.H * d.R;
  mla::Part pq;
  if (L.step) {
    // one GEMM for [kv_a | q (or q_a)] over the same hidden states
    const mla::Part pin = gemm_part<T>(h, x, d.D, (const T*)h->w_in, d.D, B, h->n_in, d.D,
                                       at<float>(ws, L.pin), h->t_in);
    if (!d.dq) {
      mla::step_finish<T>(pin, B, mt.pos, slot_dev, (const T*)h->kv_norm_g, cache, q_nope, q_rope,
                          tok_stride, d.R, d.scale, d, h->rope, h->stream, h->kv8);
      return;
    }
    if (h->kv8)
      mla::append_rows_fp8(pin, B, mt.pos, slot_dev, (const bf16*)h->kv_norm_g,
                           (uint8_t*)(void*)cache, d, h->rope, h->stream);
    else
      mla::append_rows<T>(pin, B, mt.pos, slot_dev, (const T*)h->kv_norm_g, cache, d, h->rope,
                          h->stream);
    mla::Part pa = pin;
    pa.p += d.R;
    mla::rmsnorm_rows<T>(pa, B, d.dq, (const T*)h->q_norm_g, d.eps, at<T>(ws, L.cq), h->stream);
    pq = gemm_part<T>(h, at<T>(ws, L.cq), d.dq, (const T*)h->w_qb, d.dq, B, qw, d.dq,
                      at<float>(ws, L.pq), h->t_qb);
  } else if (d.dq) {
    const mla::Part pa = gemm_part<T>(h, x, d.D, (const T*)h->w_qa, d.D, B, d.dq, d.D,
                                      at<float>(ws, L.pin), h->t_q);
    mla::rmsnorm_rows<T>(pa, B, d.dq, (const T*)h->q_norm_g, d.eps, at<T>(ws, L.cq), h->stream);
    pq = gemm_part<T>(h, at<T>(ws, L.cq), d.dq, (const T*)h->w_qb, d.dq, B, qw, d.dq,
                      at<float>(ws, L.pq), h->t_qb);
  } else {
    pq = gemm_part<T>(h, x, d.D, (const T*)h->w_q, d.D, B, qw, d.D, at<float>(ws, L.pin),
                      h->t_q);
  }
  mla::q_finish<T>(pq, B, mt.pos, q_nope, q_rope, tok_stride, d.R, d.scale, d, h->rope,
                   h->stream);
}

// A2-A4 through the decode-step GEMMs with in-place epilogues (bf16 MFMA
// layers, B <= 128 query rows): the first projection leaves the kv_a columns (and q_a) in
// fp32 and finishes the query heads itself; one more launch appends the latent
// rows, normalises q_a and / or forms the absorbed query.
// the tiled weight and partial buffer for the resident-activation stream GEMMs
static mla::StreamRes stream_res(const mla_ctx* h, const void* wt, void* ws,
                                 const DecodeLayout& L) {
  mla::StreamRes r;
  r.wt = static_cast<const bf16*>(wt);
  r.part = at<float>(ws, L.rpart);
  return r;
}

static bool q_skinny_fits(const mla_ctx* h, int B, const DecodeLayout& L) {
  const Dims& d = h->d;
  if (!h->mfma || d.dc != 512 || d.dn % 32 != 0 || d.dr % 2 != 0) return false;
  const int qw = qw_of(d);
  const int n1 = L.step ? h->n_in : (d.dq ? d.dq : qw);
  return mla::skinny_ok(B, n1, d.D) && (!d.dq || mla::skinny_ok(B, qw, d.dq));
}

// the first projection (positions come by value)
static void q_skinny_first(mla_ctx* h, const bf16* x, int B, void* ws, const DecodeLayout& L,
                           const int32_t* pos_host, const mla::HostCopy& hc) {
  const Dims& d = h->d;
  const int qw = qw_of(d);
  const int n1 = L.step ? h->n_in : (d.dq ? d.dq : qw);
  float* a = at<float>(ws, L.pin);  // fp32 rows of the first GEMM's non-query columns
  const bf16* w1 = (const bf16*)(L.step ? h->w_in : (d.dq ? h->w_qa : h->w_q));
  if (!d.dq && h->mat) {
    // materialised: [W_kva ;] per head [W^KQ_h ; W_q,rope_h] straight into q_cat
    const int nq = d.H * (d.dc + d.dr);
    const bf16* wm = static_cast<const bf16*>(h->m_in) + (L.step ? 0 : (size_t)d.R * d.D);
    mla::skinny_query(x, d.D, wm, d.D, B, (L.step ? d.R : 0) + nq, d.D, a, L.step ? d.R : 0,
                      nullptr, at<bf16>(ws, L.q_cat), pos_host, d, h->rope, h->stream, hc);
  } else if (!d.dq) {
    mla::skinny_query(x, d.D, w1, d.D, B, n1, d.D, a, L.step ? d.R : 0, at<bf16>(ws, L.q_nope),
                      at<bf16>(ws, L.q_cat), pos_host, d, h->rope, h->stream, hc,
                      stream_res(h, L.step ? h->t_in : h->t_q, ws, L));
  } else {
    mla::skinny_f32(x, d.D, w1, d.D, B, n1, d.D, a, n1, h->stream, hc,
                    stream_res(h, L.step ? h->t_in : h->t_q, ws, L));
  }
}

static void q_skinny_rest(mla_ctx* h, int B, void* ws, const DecodeLayout& L,
                          const DecodeMeta& mt, const int64_t* slot_dev, bf16* cache,
                          const int32_t* pos_host) {
  const Dims& d = h->d;
  const int qw = qw_of(d);
  const int n1 = L.step ? h->n_in : (d.dq ? d.dq : qw);
  bf16* q_nope = at<bf16>(ws, L.q_nope);
  bf16* q_cat = at<bf16>(ws, L.q_cat);
  float* a = at<float>(ws, L.pin);
  const bf16* w_ukT = (const bf16*)h->w_ukT;
  const bf16* kv_g = (const bf16*)h->kv_norm_g;
  const int R = L.step ? d.R : 0;  // kv_a columns in front of the query columns
  if (!d.dq) {
    // (materialised: the projection already formed q_abs; only the append)
    mla::decode_finish(q_nope, w_ukT, q_cat, B, !h->mat, L.step, false, a, R, 0, mt.pos,
                       slot_dev, kv_g, cache, nullptr, nullptr, d, h->rope, h->stream, h->kv8);
    return;
  }
  bf16* cq = at<bf16>(ws, L.cq);
  mla::decode_finish(q_nope, w_ukT, q_cat, B, false, L.step, true, a, n1, R, mt.pos, slot_dev,
                     kv_g, cache, (const bf16*)h->q_norm_g, cq, d, h->rope, h->stream, h->kv8);
  if (h->mat) {
    mla::skinny_query(cq, d.dq, (const bf16*)h->m_qb, d.dq, B, d.H * (d.dc + d.dr), d.dq,
                      nullptr, 0, nullptr, q_cat, pos_host, d, h->rope, h->stream);
    return;
  }
  mla::skinny_query(cq, d.dq, (const bf16*)h->w_qb, d.dq, B, qw, d.dq, nullptr, 0, q_nope, q_cat,
                    pos_host, d, h->rope, h->stream, mla::HostCopy{},
                    stream_res(h, h->t_qb, ws, L));
  mla::decode_finish(q_nope, w_ukT, q_cat, B, true, false, false, nullptr, 0, 0, mt.pos,
                     slot_dev, kv_g, cache, nullptr, nullptr, d, h->rope, h->stream);
}

// B query rows (q_len per sequence); mt: the core's metadata, mc: the
// combine's (one virtual sequence per query row)
template <typename T>
static int run_decode(mla_ctx* h, const T* hidden, int B, int q_len, T* cache, T* out, void* ws,
                      const DecodeLayout& L, const DecodeMeta& mt, const DecodeMeta& mc,
                      int parts, int nseg_total, int max_chunks, const int64_t* slot_dev,
                      const int32_t* pos_host, const mla::HostCopy& hc) {
  const Dims& d = h->d;
  float* scratch = at<float>(ws, L.scratch);
  T* q_nope = at<T>(ws, L.q_nope);
  T* q_cat = at<T>(ws, L.q_cat);
  bool fast = false;
  if constexpr (sizeof(T) == 2) {
    fast = q_skinny_fits(h, B, L);
    if (fast) q_skinny_first(h, (const bf16*)hidden, B, ws, L, pos_host, hc);
  }
  if constexpr (sizeof(T) == 2) {
    if (fast) q_skinny_rest(h, B, ws, L, mt, slot_dev, (bf16*)cache, pos_host);
  }
  if (!fast) {
    run_q_and_append<T>(h, hidden, B, ws, L, mt, slot_dev, cache);
    // A4: absorbed query q_abs_h = W_UK_h^T q_nope_h, scaled into q_cat[:, :, :dc]
    gemm_out<T>(h, q_nope, (int64_t)d.H * d.dn, d.dn, (const T*)h->w_ukT, d.dn,
                (int64_t)d.dc * d.dn, B, d.dc, d.dn, d.H,
                out_t<T>(q_cat, (int64_t)d.H * d.R, d.R, d.scale), scratch);
  }
  // A5: split-S latent attention core
  float* acc = at<float>(ws, L.acc);
  float* ml = at<float>(ws, L.ml);
  T* o_lat = at<T>(ws, L.o_lat);
  bool mfma_core = false;
  const int ts = timing_slot(h);
  if (ts >= 0) HIP_TRY(h, hipEventRecord(h->tev[2 * ts], h->stream));
  if constexpr (sizeof(T) == 2) {
    if (h->mfma) {
      const mla::TokenSplit tk{q_len, nseg_total};
      if (wide_core(h) && h->kv8)
        mla::decode_core_wide8(q_cat, (const uint8_t*)(const void*)cache, mt, parts, tk, acc, ml,
                               d, h->stream);
      else if (wide_core(h))
        mla::decode_core_wide(q_cat, cache, mt, parts, tk, acc, ml, d, h->stream);
      else if (h->kv8)  // FP8 rows; otherwise as the bf16 ring core
        mla::decode_core_ring8(q_cat, (const uint8_t*)(const void*)cache, mt, parts, tk, acc, ml,
                               (bf16*)o_lat, d, h->stream);
      else  // sequences inside one segment are finished into o_lat by the core
        mla::decode_core_ring(q_cat, cache, mt, parts, tk, acc, ml, (bf16*)o_lat, d, h->stream);
      mfma_core = true;
    }
  }
  if (!mfma_core)
    mla::decode_core_generic<T>(q_cat, cache, mt, nseg_total, q_len, acc, ml, d, h->stream);
  if (ts >= 0) HIP_TRY(h, hipEventRecord(h->tev[2 * ts + 1], h->stream));
  T* o = at<T>(ws, L.o);
  bool uv_done = false;
  if constexpr (sizeof(T) == 2) {
    if (fast && h->mat && mfma_core && mla::skinny_ok(B, d.D, d.H * d.dc)) {
      // materialised: merged latent sums, then y = W^OV [o_lat_h]_h in one product
      mla::decode_combine_512(acc, ml, mc, B, d.H, max_chunks, at<float>(ws, L.cacc),
                              at<float>(ws, L.cml), ring_core(h), (bf16*)o_lat, h->stream);
      mla::skinny_store((const bf16*)o_lat, (int64_t)d.H * d.dc, (const bf16*)h->m_ov,
                        (int64_t)d.H * d.dc, B, d.D, d.H * d.dc, (bf16*)out, d.D, 1.f,
                        h->stream);
      return check_launch(h, "decode");
    }
    if (combine_uv(h)) {
      // A6 + A7: combine the partials of each sequence (fixed slot order) and
      // apply W_UV_h to the merged latent sums
      mla::decode_combine_uv(acc, ml, mc, B, d.H, max_chunks, at<float>(ws, L.cacc),
                             at<float>(ws, L.cml), ring_core(h), (const bf16*)h->w_uv,
                             (bf16*)o_lat, (bf16*)o, h->stream);
      uv_done = true;
    } else if (mfma_core) {
      mla::decode_combine_512(acc, ml, mc, B, d.H, max_chunks, at<float>(ws, L.cacc),
                              at<float>(ws, L.cml), ring_core(h), (bf16*)o_lat, h->stream);
    }
  }
  if (!mfma_core) mla::decode_combine<T>(acc, ml, mc, B, o_lat, d, h->stream);
  // A7: o_h = W_UV_h o_lat_h
  if (!uv_done)
    gemm_out<T>(h, o_lat, (int64_t)d.H * d.dc, d.dc, (const T*)h->w_uv, d.dc,
                (int64_t)d.dv * d.dc, B, d.dv, d.dc, d.H, out_t<T>(o, (int64_t)d.H * d.dv, d.dv),
                scratch);
  // A8: y = W_o o
  const int ko = d.H * d.dv;
  bool o_done = false;
  if constexpr (sizeof(T) == 2) {
    if (h->mfma && mla::skinny_ok(B, d.D, ko)) {
      mla::skinny_store((const bf16*)o, ko, (const bf16*)h->w_o, ko, B, d.D, ko, (bf16*)out, d.D,
                        1.f, h->stream, stream_res(h, h->t_o, ws, L));
      o_done = true;
    }
  }
  if (!o_done)
    gemm_out<T>(h, o, ko, 0, (const T*)h->w_o, ko, 0, B, d.D, ko, 1, out_t<T>(out, d.D), scratch,
                h->t_o);
  return check_launch(h, "decode");
}

// One decode call after its arguments have been checked: B sequences with
// q_len new tokens each (query row b * q_len + j), a contiguous cache
// (seq_off) or a paged one (pg), appending the new rows first for a step.
struct DecodeCall {
  const void* hidden;
  void* out;
  int B, q_len;
  const int32_t* seq_len;
  const int64_t* seq_off;
  const PageArgs* pg;
  void* cache;
  bool step;
  void* ws;
  size_t ws_bytes;
};

static int decode_exec(mla_ctx* h, const DecodeCall& c, const char* what) {
  if (!h->absorbed) return fail(h, MLA_ERR_STATE, "%s before mla_absorb_weights", what);
  const int B = c.B, q_len = c.q_len, Bq = B * q_len;
  int64_t total = 0;
  for (int32_t b = 0; b < B; ++b) total += c.seq_len[b];
  const DecodeLayout L = decode_layout(h, B, total, c.step, q_len);
  int rc;
  if ((rc = check_ws(h, c.ws, c.ws_bytes, L.total))) return rc;
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  std::vector<char> blob;
  MetaOffsets mo;
  int nseg_total = 0, max_chunks = 1, cslots = 0;
  const int parts = build_decode_meta(h, B, c.seq_off, c.seq_len, q_len, total, c.step, c.pg,
                                      blob, &mo, &nseg_total, &max_chunks, &cslots);
  if (cslots > L.max_cslots)
    return fail(h, MLA_ERR_WORKSPACE, "internal: combine chunk slots larger than planned");
  if (blob.size() > meta_bytes(B, max_parts(h, total, q_len), L.max_segs, total, q_len))
    return fail(h, MLA_ERR_WORKSPACE, "internal: decode metadata larger than planned");
  void* ws = c.ws;
  void* meta = at<char>(ws, L.meta);
  // The metadata is first read by the kernel after the first projection, so
  // when that projection is a stream GEMM, extra blocks of its launch copy the
  // metadata from pinned memory (saving the separate copy); else a copy.
  mla::HostCopy hc;
  hipEvent_t stage_ev = nullptr;
  if (!is_f32(h) && q_skinny_fits(h, Bq, L)) {
    const void* pinned = nullptr;
    if ((rc = stage_host(h, blob.data(), blob.size(), &pinned, &stage_ev))) return rc;
    hc.src = pinned;
    hc.dst = meta;
    hc.n16 = (int)((blob.size() + 15) / 16);
    hc.blocks = mla::host_copy_blocks(hc.n16);
  } else if ((rc = stage_upload(h, meta, blob.data(), blob.size()))) {
    return rc;
  }
  DecodeMeta mt;
  mt.seq_off = at<int64_t>(meta, mo.seq_off);
  mt.seq_len = at<int32_t>(meta, mo.seq_len);
  mt.pos = at<int32_t>(meta, mo.pos);
  mt.pstart = at<int32_t>(meta, mo.pstart);
  mt.nseg = at<int32_t>(meta, mo.nseg);
  mt.cstart = at<int32_t>(meta, mo.cstart);
  mt.work = at<mla::DecodeWork>(meta, mo.work);
  mt.part_begin = at<int32_t>(meta, mo.part);
  mt.segs = at<DecodeSeg>(meta, mo.segs);
  mt.pages = c.pg ? at<int32_t>(meta, mo.pages) : nullptr;
  mt.pg_off = c.pg ? at<int32_t>(meta, mo.pg_off) : nullptr;
  mt.page_shift = c.pg ? c.pg->shift : 0;
  mlog("%s: B=%d q_len=%d rows=%lld, %d parts, %d segments, combine chunks %d, workspace %zu B, "
       "core %s, projections %s", what, B, q_len, (long long)total, parts, nseg_total, max_chunks,
       L.total, core_name(h), hc.n16 > 0 ? "stream GEMMs (metadata copied by the first)"
                                          : "tile GEMMs (metadata copied first)");
  DecodeMeta mc = mt;  // the combine's view: one sequence per query row
  mc.pstart = at<int32_t>(meta, mo.vpstart);
  mc.nseg = at<int32_t>(meta, mo.vnseg);
  mc.cstart = at<int32_t>(meta, mo.vcstart);
  std::vector<int32_t> qpos(Bq);
  for (int i = 0; i < Bq; ++i) qpos[i] = c.seq_len[i / q_len] - q_len + i % q_len;
  const int64_t* slot_dev = c.step ? at<int64_t>(meta, mo.slot) : nullptr;
  if (is_f32(h))
    return run_decode<float>(h, (const float*)c.hidden, Bq, q_len, (float*)c.cache,
                             (float*)c.out, ws, L, mt, mc, parts, nseg_total, max_chunks,
                             slot_dev, qpos.data(), hc);
  rc = run_decode<bf16>(h, (const bf16*)c.hidden, Bq, q_len, (bf16*)c.cache, (bf16*)c.out, ws, L,
                        mt, mc, parts, nseg_total, max_chunks, slot_dev, qpos.data(), hc);
  if (stage_ev) HIP_TRY(h, hipEventRecord(stage_ev, h->stream));  // the staging slot's last reader
  return rc;
}

static int decode_common(mla_handle h, const void* hidden, const int32_t* pos,
                         const int64_t* seq_off, const int32_t* seq_len, int32_t B, void* cache,
                         int64_t cache_rows, void* out, void* ws, size_t ws_bytes, bool step,
                         const PageArgs* pg = nullptr) {
  if (!h) return MLA_ERR_INVALID_ARG;
  const char* what = pg ? (step ? "decode_step_paged" : "decode_paged")
                        : (step ? "decode_step" : "decode");
  if (!hidden || !cache || !out) return fail(h, MLA_ERR_INVALID_ARG, "%s: NULL tensor", what);
  int rc = pg ? mla_decode_paged_check(&h->cfg, pos, pg ? pg->table : nullptr,
                                       pg ? pg->max_pages : 0, pg ? pg->page_rows : 0, seq_len,
                                       B, cache_rows, step ? 1 : 0)
              : mla_decode_check(&h->cfg, pos, seq_off, seq_len, B, cache_rows);
  if (!rc && !pg && step) rc = contig_write_check(seq_off, seq_len, B, 1);
  if (rc) return fail(h, rc, "%s: %s (B=%d, cache_rows=%lld)", what, mla_status_string(rc), B,
                      (long long)cache_rows);
  const DecodeCall c{hidden, out, B, 1, seq_len, seq_off, pg, cache, step, ws, ws_bytes};
  return decode_exec(h, c, what);
}

int mla_decode(mla_handle h, const void* hidden, const int32_t* pos, const int64_t* seq_off,
               const int32_t* seq_len, int32_t B, const void* cache, int64_t cache_rows, void* out,
               void* ws, size_t ws_bytes) {
  return decode_common(h, hidden, pos, seq_off, seq_len, B, const_cast<void*>(cache), cache_rows,
                       out, ws, ws_bytes, false);
}

int mla_decode_step(mla_handle h, const void* hidden, const int32_t* pos, const int64_t* seq_off,
                    const int32_t* seq_len, int32_t B, void* cache, int64_t cache_rows, void* out,
                    void* ws, size_t ws_bytes) {
  return decode_common(h, hidden, pos, seq_off, seq_len, B, cache, cache_rows, out, ws, ws_bytes,
                       true);
}

int mla_decode_step_noalloc(mla_handle h, const void* hidden, const int32_t* pos,
                            const int64_t* seq_off, const int32_t* seq_len, int32_t B, void* cache,
                            int64_t cache_rows, void* out) {
  if (!h) return MLA_ERR_INVALID_ARG;
  const char* what = "decode_step_noalloc";
  int rc = mla_decode_check(&h->cfg, pos, seq_off, seq_len, B, cache_rows);
  if (!rc) rc = contig_write_check(seq_off, seq_len, B, 1);
  if (rc) return fail(h, rc, "%s: %s (B=%d, cache_rows=%lld)", what, mla_status_string(rc), B,
                      (long long)cache_rows);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIP_TRY(h, hipStreamIsCapturing(h->stream, &cs));
  if (cs != hipStreamCaptureStatusNone)
    return fail(h, MLA_ERR_STATE, "%s: the stream is being captured (the step's metadata "
                "would need pinned memory of their own)", what);
  int64_t total = 0;
  for (int32_t b = 0; b < B; ++b) total += seq_len[b];
  const size_t need = mla_decode_step_workspace_bytes(h, B, total);
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return fail(h, MLA_ERR_WORKSPACE,
                "%s: B=%d with %lld cache rows needs %zu bytes of scratch; the static scratch "
                "holds %zu", what, B, (long long)total, need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  if (!h->noalloc_ws) return fail(h, MLA_ERR_STATE, "%s: no scratch address", what);
  h->no_alloc = true;
  rc = decode_common(h, hidden, pos, seq_off, seq_len, B, cache, cache_rows, out, h->noalloc_ws,
                     (size_t)MLA_NOALLOC_SCRATCH_BYTES, true);
  h->no_alloc = false;
  return rc;
}

size_t mla_decode_ex_workspace_bytes(mla_handle h, int32_t B, int32_t q_len, int64_t total_rows,
                                     int32_t append) {
  if (!h || B <= 0 || q_len < 1 || q_len > MLA_MAX_Q_LEN || total_rows <= 0) return 0;
  return decode_layout(h, B, total_rows, append != 0, q_len).total;
}

static int page_shift_of(int32_t page_rows);

int mla_decode_ex(mla_handle h, const mla_decode_args* a) {
  if (!h) return MLA_ERR_INVALID_ARG;
  const char* what = "decode_ex";
  if (!a || !a->hidden || !a->cache || !a->out)
    return fail(h, MLA_ERR_INVALID_ARG, "%s: NULL argument or tensor", what);
  const int rc = mla_decode_ex_check(&h->cfg, a);
  if (rc) return fail(h, rc, "%s: %s (B=%d, q_len=%d, cache_rows=%lld)", what,
                      mla_status_string(rc), a->B, a->q_len, (long long)a->cache_rows);
  PageArgs pg{a->block_table, a->max_pages, a->page_rows, 0};
  if (a->block_table) pg.shift = page_shift_of(a->page_rows);
  const DecodeCall c{a->hidden, a->out,   a->B,           a->q_len,  a->seq_len,
                     a->seq_off, a->block_table ? &pg : nullptr, a->cache, a->append != 0,
                     a->ws,     a->ws_bytes};
  return decode_exec(h, c, what);
}

static int page_shift_of(int32_t page_rows) {
  int k = 0;
  while ((1 << k) < page_rows && k < 30) ++k;
  return k;
}

int mla_decode_paged(mla_handle h, const void* hidden, const int32_t* pos,
                     const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                     const int32_t* seq_len, int32_t B, const void* cache, int64_t cache_rows,
                     void* out, void* ws, size_t ws_bytes) {
  const PageArgs pg{block_table, max_pages, page_rows, page_shift_of(page_rows)};
  return decode_common(h, hidden, pos, nullptr, seq_len, B, const_cast<void*>(cache), cache_rows,
                       out, ws, ws_bytes, false, &pg);
}

int mla_decode_step_paged(mla_handle h, const void* hidden, const int32_t* pos,
                          const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                          const int32_t* seq_len, int32_t B, void* cache, int64_t cache_rows,
                          void* out, void* ws, size_t ws_bytes) {
  const PageArgs pg{block_table, max_pages, page_rows, page_shift_of(page_rows)};
  return decode_common(h, hidden, pos, nullptr, seq_len, B, cache, cache_rows, out, ws, ws_bytes,
                       true, &pg);
}

// ------------------------------------------------------------------------
// prefill
// ------------------------------------------------------------------------
namespace {
struct PrefillLayout {
  size_t meta, scratch, pin, pq, cq, q_nope, q_rope, kv, o, keys, total;
  size_t meta_bytes, tiles_off;  // blob size and offset of the MFMA query tiles
  size_t slot_off;               // prefill step: the new rows' cache rows (int64, T)
  // gathered key rows (FP8 or paged caches): offsets in the blob of the per-
  // sequence row counts, source offsets (contiguous) or page list starts
  // (paged), and the page list
  size_t nrows_off, gsrc_off, pstart_off, pages_off;
};

// the MFMA prefill attention applies (bf16, 128 + 64 query/key dims, 128 values)
bool prefill_mfma(const mla_ctx* h) {
  const Dims& d = h->d;
  return h->cfg.dtype == MLA_BF16 && d.dn == 128 && d.dr == 64 && d.dv == 128;
}

int max_prefill_tiles(int T, int B) { return T / mla::prefill_tile_queries() + B; }

// pages of a paged prefill's key rows: at most rows / 32 + B (pages hold 32
// rows or more)
int64_t max_prefill_pages(int B, int64_t rows) { return rows / 32 + B; }

// staged: the key rows are gathered into the workspace first (FP8 or paged
// caches)
// Columns of the in-projection a prefill step runs: [W_kva ; W_qa] for a
// query LoRA (one product for the append and the query's first half), else
// W_kva alone (the query projection then reads the hidden states itself).
int step_in_cols(const mla_ctx* h) { return h->d.dq ? h->n_in : h->d.R; }

PrefillLayout prefill_layout(const mla_ctx* h, int T, int B, int64_t rows, int max_rows,
                             bool staged, bool paged, bool step = false) {
  const Dims& d = h->d;
  PrefillLayout L;
  const int qw = qw_of(d);
  const size_t scr = std::max({out_scratch(h, T, d.D, d.H * d.dv, 1),
                               out_scratch(h, max_rows, d.H * (d.dn + d.dv), d.dc, 1),
                               out_scratch(h, T, qw, d.dq ? d.dq : d.D, 1)});
  const size_t pin = std::max(part_floats(h, T, d.dq ? d.dq : qw, d.D),
                              step ? part_floats(h, T, step_in_cols(h), d.D) : (size_t)0);
  const size_t pq = d.dq ? part_floats(h, T, qw, d.dq) : 0;
  const size_t e = h->esz;
  Carve c;
  L.tiles_off = align_up((size_t)T * 4) * 2 + align_up((size_t)B * 8) * 2;
  L.nrows_off = align_up(L.tiles_off + (size_t)max_prefill_tiles(T, B) * sizeof(mla::PrefillTile));
  L.gsrc_off = L.nrows_off + align_up((size_t)B * 4);
  L.pstart_off = L.gsrc_off + align_up((size_t)B * 8);
  L.pages_off = L.pstart_off + align_up((size_t)B * 4);
  L.meta_bytes = !staged ? L.nrows_off
                 : L.pages_off + (paged ? align_up((size_t)max_prefill_pages(B, rows) * 4) : 0);
  L.slot_off = L.meta_bytes;
  if (step) L.meta_bytes += align_up((size_t)T * 8);
  L.meta = c.take(L.meta_bytes);
  L.scratch = c.take(scr * 4);
  L.pin = c.take(pin * 4);
  L.pq = c.take(pq * 4);
  L.cq = c.take(d.dq ? (size_t)T * d.dq * e : 0);
  // q_nope (generic path), or the whole (T, H, dn + dr) query (MFMA path)
  L.q_nope = c.take((size_t)T * d.H * (d.dn + d.dr) * e);
  L.q_rope = c.take((size_t)T * d.H * std::max(d.dr, 1) * e);
  L.kv = c.take((size_t)rows * d.H * (d.dn + d.dv) * 4);
  // attention output: rows, or the output projection's tiled operand
  L.o = c.take(std::max((size_t)T * d.H * d.dv * e,
                        is_f32(h) ? (size_t)0 : mla::tiled_bytes(T, d.H * d.dv)));
  L.keys = c.take(staged ? (size_t)rows * d.R * e : 0);
  L.total = c.off;
  return L;
}
}  // namespace

size_t mla_prefill_workspace_bytes(mla_handle h, int32_t T, int32_t B, int64_t total_key_rows) {
  if (!h || T <= 0 || B <= 0 || total_key_rows <= 0) return 0;
  const int max_rows = (int)std::min<int64_t>(total_key_rows, INT32_MAX);
  return prefill_layout(h, T, B, total_key_rows, max_rows, h->kv8, false).total;
}

size_t mla_prefill_paged_workspace_bytes(mla_handle h, int32_t T, int32_t B,
                                         int64_t total_key_rows) {
  if (!h || T <= 0 || B <= 0 || total_key_rows <= 0) return 0;
  const int max_rows = (int)std::min<int64_t>(total_key_rows, INT32_MAX);
  return prefill_layout(h, T, B, total_key_rows, max_rows, true, true).total;
}

template <typename T>
static int run_prefill(mla_ctx* h, const T* hidden, int ntok, int B, const int32_t* cu_new,
                       const int32_t* prior, const int64_t* seq_off, const T* cache, T* out,
                       void* ws, const PrefillLayout& L, const int64_t* kv_off_h,
                       int ntiles, const mla::Part* qa_done = nullptr) {
  const Dims& d = h->d;
  const int qw = qw_of(d);
  char* meta = at<char>(ws, L.meta);
  const int32_t* tok_seq = reinterpret_cast<const int32_t*>(meta);
  const int32_t* tok_pos = reinterpret_cast<const int32_t*>(meta + align_up((size_t)ntok * 4));
  const int64_t* kv_off =
      reinterpret_cast<const int64_t*>(meta + 2 * align_up((size_t)ntok * 4));
  const int64_t* seq_off_d = kv_off + align_up((size_t)B * 8) / 8;
  float* scratch = at<float>(ws, L.scratch);
  T* q_nope = at<T>(ws, L.q_nope);
  T* q_rope = at<T>(ws, L.q_rope);
  bool mfma_attn = false;
  if constexpr (sizeof(T) == 2) mfma_attn = prefill_mfma(h);
  // query (A3): c_q = RMSNorm(W_qa x) for a query LoRA
  const T* qin = hidden;
  int qk = d.D;
  const T* wq = (const T*)h->w_q;
  const void* wqt = h->t_q;  // its tiled copy
  if (d.dq) {
    // (a prefill step has W_qa x already, beside the append's columns)
    const mla::Part pa = qa_done ? *qa_done
                                 : gemm_part<T>(h, hidden, d.D, (const T*)h->w_qa, d.D, ntok, d.dq,
                                                d.D, at<float>(ws, L.pin), h->t_q);
    mla::rmsnorm_rows<T>(pa, ntok, d.dq, (const T*)h->q_norm_g, d.eps, at<T>(ws, L.cq),
                         h->stream);
    qin = at<T>(ws, L.cq);
    qk = d.dq;
    wq = (const T*)h->w_qb;
    wqt = h->t_qb;
  }
  if (mfma_attn) {
    // the projection writes the bf16 query rows (T, H, dn + dr) directly; the
    // attention kernel rotates the rope parts as it loads them
    gemm_out<T>(h, qin, qk, 0, wq, qk, 0, ntok, qw, qk, 1, out_t<T>(q_nope, qw), scratch, wqt);
  } else {
    const mla::Part pq = gemm_part<T>(h, qin, qk, wq, qk, ntok, qw, qk,
                                      at<float>(ws, d.dq ? L.pq : L.pin), wqt);
    mla::q_finish<T>(pq, ntok, tok_pos, q_nope, q_rope, (int64_t)d.H * d.dr, d.dr, 1.f, d,
                     h->rope, h->stream);
  }
  // expansion of every key row: [K_nope_h | V_h] = W_kvb c_t (bf16 for the
  // MFMA attention, fp32 for the generic one)
  // Sequences whose cache rows and expanded rows both follow each other
  // directly are expanded by one GEMM.
  const int wkv = d.H * (d.dn + d.dv);
  for (int b = 0; b < B;) {
    int64_t rows = prior[b] + (cu_new[b + 1] - cu_new[b]);
    int e = b + 1;
    while (e < B && seq_off[e] == seq_off[b] + rows && kv_off_h[e] == kv_off_h[b] + rows &&
           rows + prior[e] + (cu_new[e + 1] - cu_new[e]) <= INT32_MAX) {
      rows += prior[e] + (cu_new[e + 1] - cu_new[e]);
      ++e;
    }
    if (rows > 0) {
      const int64_t o0 = kv_off_h[b] * (int64_t)wkv;
      const mla::GemmOut go = mfma_attn ? out_t<T>(at<T>(ws, L.kv) + o0, wkv)
                                        : out_f32(at<float>(ws, L.kv) + o0, wkv);
      gemm_out<T>(h, cache + seq_off[b] * d.R, d.R, 0, (const T*)h->w_kvb, d.dc, 0, (int)rows,
                  wkv, d.dc, 1, go, scratch, h->t_kvb);
    }
    b = e;
  }
  T* o = at<T>(ws, L.o);
  // the attention writes its output straight into the output projection's
  // tiled operand when that product runs on the large-tile GEMM
  const bool o_tiled = mfma_attn && h->t_o && big_gemm(h, ntok, d.D, d.H * d.dv, 1);
  const int ts = timing_slot(h);
  if (ts >= 0) HIP_TRY(h, hipEventRecord(h->tev[2 * ts], h->stream));
  if constexpr (sizeof(T) == 2) {
    if (mfma_attn)
      mla::prefill_attn_mfma(q_nope, at<bf16>(ws, L.kv), cache,
                             reinterpret_cast<const mla::PrefillTile*>(meta + L.tiles_off),
                             ntiles, d.H, d.scale, o, o_tiled, h->rope, h->stream);
  }
  if (!mfma_attn)
    mla::prefill_attn_generic<T>(q_nope, q_rope, at<float>(ws, L.kv), cache, tok_seq, tok_pos,
                                 kv_off, seq_off_d, ntok, o, d, h->stream);
  if (ts >= 0) HIP_TRY(h, hipEventRecord(h->tev[2 * ts + 1], h->stream));
  if (o_tiled) {
    if constexpr (sizeof(T) == 2)
      mla::gemm_big(o, static_cast<const bf16*>(h->t_o), ntok, d.D, d.H * d.dv,
                    out_t<T>(out, d.D), h->n_cu, h->stream);
  } else {
    gemm_out<T>(h, o, (int64_t)d.H * d.dv, 0, (const T*)h->w_o, (int64_t)d.H * d.dv, 0, ntok,
                d.D, d.H * d.dv, 1, out_t<T>(out, d.D), scratch, h->t_o);
  }
  return check_launch(h, "prefill");
}

// A chunked prefill over a contiguous (seq_off) or a paged (pg) cache.  The
// expansion and the attention read the key rows in place from a contiguous
// cache in the storage type; FP8 and paged caches have their key rows
// gathered into the workspace first, at kv_off (the expanded rows' order).
static int prefill_common(mla_ctx* h, const void* hidden, const int32_t* cu_new,
                          const int32_t* prior_len, const int64_t* seq_off, const PageArgs* pg,
                          int32_t B, const void* cache, int64_t cache_rows, void* out, void* ws,
                          size_t ws_bytes, bool step = false) {
  const char* what = pg ? "prefill_paged" : step ? "prefill_step" : "prefill";
  if (!h) return MLA_ERR_INVALID_ARG;
  if (!hidden || !cache || !out) return fail(h, MLA_ERR_INVALID_ARG, "%s: NULL tensor", what);
  const int rc0 = pg ? mla_prefill_paged_check(&h->cfg, cu_new, prior_len, pg->table,
                                               pg->max_pages, pg->page_rows, B, cache_rows)
                  : step ? mla_prefill_step_check(&h->cfg, cu_new, prior_len, seq_off, B, cache_rows)
                         : mla_prefill_check(&h->cfg, cu_new, prior_len, seq_off, B, cache_rows);
  if (rc0) return fail(h, rc0, "%s: %s (B=%d, cache_rows=%lld)", what, mla_status_string(rc0), B,
                       (long long)cache_rows);
  if (!h->absorbed) return fail(h, MLA_ERR_STATE, "%s before mla_absorb_weights", what);
  const bool staged = h->kv8 || pg;
  int64_t rows = 0;
  int32_t max_n = 0;
  std::vector<int64_t> kv_off(B);
  for (int32_t b = 0; b < B; ++b) {
    kv_off[b] = rows;
    const int32_t n = prior_len[b] + (cu_new[b + 1] - cu_new[b]);
    rows += n;
    max_n = std::max(max_n, n);
  }
  // where the expansion and the attention read sequence b's key rows
  const int64_t* key_off = staged ? kv_off.data() : seq_off;
  const int32_t T = cu_new[B];
  const PrefillLayout L = prefill_layout(h, T, B, rows, (int)std::min<int64_t>(rows, INT32_MAX),
                                         staged, pg != nullptr, step);
  int rc = check_ws(h, ws, ws_bytes, L.total);
  if (rc) return rc;
  DeviceGuard g(h->device);
  if (!g.ok) return fail(h, MLA_ERR_HIP, "cannot select device %d", h->device);
  std::vector<char> blob(L.meta_bytes, 0);
  int32_t* tok_seq = reinterpret_cast<int32_t*>(blob.data());
  int32_t* tok_pos = reinterpret_cast<int32_t*>(blob.data() + align_up((size_t)T * 4));
  int64_t* kvo = reinterpret_cast<int64_t*>(blob.data() + 2 * align_up((size_t)T * 4));
  int64_t* so = kvo + align_up((size_t)B * 8) / 8;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t i = cu_new[b]; i < cu_new[b + 1]; ++i) {
      tok_seq[i] = b;
      tok_pos[i] = prior_len[b] + (i - cu_new[b]);
    }
    kvo[b] = kv_off[b];
    so[b] = key_off[b];
  }
  if (step) {  // the new rows' cache rows
    int64_t* slot = reinterpret_cast<int64_t*>(blob.data() + L.slot_off);
    for (int32_t i = 0; i < T; ++i) slot[i] = seq_off[tok_seq[i]] + tok_pos[i];
  }
  // query tiles of the MFMA attention, longest key range first
  std::vector<mla::PrefillTile> tiles;
  const int tq = mla::prefill_tile_queries();
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = cu_new[b + 1] - cu_new[b];
    for (int32_t i = 0; i < n; i += tq) {
      mla::PrefillTile t;
      t.kv_row0 = kv_off[b];
      t.cache_row0 = key_off[b];
      t.t0 = cu_new[b] + i;
      t.nq = std::min(tq, n - i);
      t.pos0 = prior_len[b] + i;
      t.pad = 0;
      tiles.push_back(t);
    }
  }
  std::stable_sort(tiles.begin(), tiles.end(), [](const mla::PrefillTile& a,
                                                  const mla::PrefillTile& b) {
    return a.pos0 + a.nq > b.pos0 + b.nq;
  });
  if ((int)tiles.size() > max_prefill_tiles(T, B))
    return fail(h, MLA_ERR_WORKSPACE, "internal: more prefill tiles than planned");
  memcpy(blob.data() + L.tiles_off, tiles.data(), tiles.size() * sizeof(mla::PrefillTile));
  if (staged) {
    int32_t* nrows = reinterpret_cast<int32_t*>(blob.data() + L.nrows_off);
    int64_t* gsrc = reinterpret_cast<int64_t*>(blob.data() + L.gsrc_off);
    int32_t* pstart = reinterpret_cast<int32_t*>(blob.data() + L.pstart_off);
    int32_t* pages = reinterpret_cast<int32_t*>(blob.data() + L.pages_off);
    int64_t np = 0;
    for (int32_t b = 0; b < B; ++b) {
      nrows[b] = prior_len[b] + (cu_new[b + 1] - cu_new[b]);
      gsrc[b] = seq_off ? seq_off[b] : 0;
      if (pg) {
        const int64_t n = ((int64_t)nrows[b] + pg->page_rows - 1) / pg->page_rows;
        if (np + n > max_prefill_pages(B, rows))
          return fail(h, MLA_ERR_WORKSPACE, "internal: more prefill pages than planned");
        pstart[b] = (int32_t)np;
        for (int64_t i = 0; i < n; ++i) pages[np++] = pg->table[(int64_t)b * pg->max_pages + i];
      }
    }
  }
  mlog("%s: B=%d new tokens %d, key rows %lld (longest %d), %zu attention tiles of %d queries "
       "x %d heads, key rows %s, workspace %zu B", what, B, T, (long long)rows, max_n,
       tiles.size(), tq, h->d.H, staged ? "gathered into the workspace" : "read in place",
       L.total);
  if ((rc = stage_upload(h, at<char>(ws, L.meta), blob.data(), blob.size()))) return rc;
  // a prefill step first appends the new tokens' latent rows (c and k_rope
  // of every new position, "Multi-Head Latent Attention" post, section 3.1),
  // reading the hidden states once for the append and, with a query LoRA,
  // the query's first projection (both take the same hidden state in the
  // DeepSeek code quoted in section 3.4)
  mla::Part qa{};
  bool qa_done = false;
  if (step) {
    const Dims& d = h->d;
    const char* meta = at<char>(ws, L.meta);
    const int32_t* pos_d = reinterpret_cast<const int32_t*>(meta + align_up((size_t)T * 4));
    const int64_t* slot_d = reinterpret_cast<const int64_t*>(meta + L.slot_off);
    const int n = step_in_cols(h);
    const bool fuse = d.dq > 0;
    if (is_f32(h)) {
      const mla::Part a = gemm_part<float>(h, (const float*)hidden, d.D,
                                           (const float*)(fuse ? h->w_in : h->w_kva), d.D, T, n,
                                           d.D, at<float>(ws, L.pin), fuse ? h->t_in : h->t_kva);
      mla::append_rows<float>(a, T, pos_d, slot_d, (const float*)h->kv_norm_g, (float*)cache, d,
                              h->rope, h->stream);
      qa = mla::Part{a.p + d.R, a.ks, a.ld, a.zs};
    } else {
      mla::Part a;
      if (fuse && h->t_kva && h->t_q && big_gemm(h, T, n, d.D, 1) &&
          big_gemm(h, T, d.R, d.D, 1) && big_gemm(h, T, d.dq, d.D, 1)) {
        // the hidden states tiled once for both products, which write adjacent
        // columns of one output: as two launches the products fill the compute
        // units better than one over 576 + dq columns does (its 128-wide
        // column tiles leave a quarter-full last wave at 16,384 rows)
        float* pin = at<float>(ws, L.pin);
        bf16* At = reinterpret_cast<bf16*>(pin + align_up((size_t)T * n * 4) / 4);
        mla::tile_rows((const bf16*)hidden, d.D, T, d.D, At, h->stream);
        mla::gemm_big(At, (const bf16*)h->t_kva, T, d.R, d.D,
                      mla::GemmOut{pin, nullptr, n, 0, 1.f}, h->n_cu, h->stream);
        mla::gemm_big(At, (const bf16*)h->t_q, T, d.dq, d.D,
                      mla::GemmOut{pin + d.R, nullptr, n, 0, 1.f}, h->n_cu, h->stream);
        a = mla::Part{pin, 1, n, (int64_t)T * n};
      } else {
        a = gemm_part<bf16>(h, (const bf16*)hidden, d.D, (const bf16*)(fuse ? h->w_in : h->w_kva),
                            d.D, T, n, d.D, at<float>(ws, L.pin), fuse ? h->t_in : h->t_kva);
      }
      if (h->kv8)
        mla::append_rows_fp8(a, T, pos_d, slot_d, (const bf16*)h->kv_norm_g, (uint8_t*)cache, d,
                             h->rope, h->stream);
      else
        mla::append_rows<bf16>(a, T, pos_d, slot_d, (const bf16*)h->kv_norm_g, (bf16*)cache, d,
                               h->rope, h->stream);
      qa = mla::Part{a.p + d.R, a.ks, a.ld, a.zs};
    }
    qa_done = fuse;
  }
  const void* keys = cache;
  if (staged) {
    const char* meta = at<char>(ws, L.meta);
    mla::KeyRowSrc src;
    src.cache = cache;
    src.seq_off = reinterpret_cast<const int64_t*>(meta + L.gsrc_off);
    src.page_start = reinterpret_cast<const int32_t*>(meta + L.pstart_off);
    src.pages = pg ? reinterpret_cast<const int32_t*>(meta + L.pages_off) : nullptr;
    src.page_shift = pg ? pg->shift : 0;
    const int64_t* kvo_d = reinterpret_cast<const int64_t*>(meta + 2 * align_up((size_t)T * 4));
    if (mla::gather_key_rows(src, h->kv8, kvo_d,
                             reinterpret_cast<const int32_t*>(meta + L.nrows_off), B, max_n,
                             h->d.R * (int)h->esz, at<char>(ws, L.keys), h->stream))
      return fail(h, MLA_ERR_SHAPE, "%s: FP8 rows need kv_lora 512 and qk_rope 64", what);
    keys = at<char>(ws, L.keys);
  }
  if (is_f32(h))
    return run_prefill<float>(h, (const float*)hidden, T, B, cu_new, prior_len, key_off,
                              (const float*)keys, (float*)out, ws, L, kv_off.data(),
                              (int)tiles.size(), qa_done ? &qa : nullptr);
  return run_prefill<bf16>(h, (const bf16*)hidden, T, B, cu_new, prior_len, key_off,
                           (const bf16*)keys, (bf16*)out, ws, L, kv_off.data(),
                           (int)tiles.size(), qa_done ? &qa : nullptr);
}

int mla_prefill(mla_handle h, const void* hidden, const int32_t* cu_new, const int32_t* prior_len,
                const int64_t* seq_off, int32_t B, const void* cache, int64_t cache_rows,
                void* out, void* ws, size_t ws_bytes) {
  return prefill_common(h, hidden, cu_new, prior_len, seq_off, nullptr, B, cache, cache_rows,
                        out, ws, ws_bytes);
}

size_t mla_prefill_step_workspace_bytes(mla_handle h, int32_t T, int32_t B,
                                        int64_t total_key_rows) {
  if (!h || T <= 0 || B <= 0 || total_key_rows <= 0) return 0;
  const int max_rows = (int)std::min<int64_t>(total_key_rows, INT32_MAX);
  return prefill_layout(h, T, B, total_key_rows, max_rows, h->kv8, false, true).total;
}

int mla_prefill_step(mla_handle h, const void* hidden, const int32_t* cu_new,
                     const int32_t* prior_len, const int64_t* seq_off, int32_t B, void* cache,
                     int64_t cache_rows, void* out, void* ws, size_t ws_bytes) {
  return prefill_common(h, hidden, cu_new, prior_len, seq_off, nullptr, B, cache, cache_rows,
                        out, ws, ws_bytes, true);
}

int mla_prefill_paged(mla_handle h, const void* hidden, const int32_t* cu_new,
                      const int32_t* prior_len, const int32_t* block_table, int32_t max_pages,
                      int32_t page_rows, int32_t B, const void* cache, int64_t cache_rows,
                      void* out, void* ws, size_t ws_bytes) {
  const PageArgs pg{block_table, max_pages, page_rows, page_shift_of(page_rows)};
  return prefill_common(h, hidden, cu_new, prior_len, nullptr, &pg, B, cache, cache_rows, out,
                        ws, ws_bytes);
}
