// Internal launcher interface between the host layer (mla.cpp) and the HIP
// kernels.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace mla {

// RoPE frequencies theta_i = base^(-2i/dr), computed once on the host in
// double precision (dr <= 2 * kMaxRopePairs).
constexpr int kMaxRopePairs = 64;

// Shapes the kernels need, copied from the public config.
struct Dims {
  int D, H, dn, dr, dv, dc, dq, R;
  float rope_base, eps, scale;
};

struct RopeTab {
  double theta[kMaxRopePairs];
};

// Bytes per cached row of an FP8 latent cache: dc OCP E4M3 codes, dr bf16
// rope values, the fp32 row scale, zero-padded to a multiple of 16.
__host__ __device__ constexpr int fp8_row_bytes(int dc, int dr) {
  return (dc + 2 * dr + 4 + 15) / 16 * 16;
}

// One decode work segment: rows [r0, r1) of sequence b (row indices relative
// to the sequence start), whose partial result goes to slot pidx.
struct DecodeSeg {
  int32_t b, r0, r1, pidx;
};

// The same segment as the persistent cores read it: one self-contained record
// (absolute first cache row, row count, sequence, partial slot, and the
// sequence's partial slots [pstart, pstart + nseg)).  Record p < parts is the
// first segment of part p; `next` chains the part's further segments (-1 ends
// the chain).
struct DecodeWork {
  int64_t row;
  int32_t n, b, pidx, next;
  int32_t nseg, pstart;
};
static_assert(sizeof(DecodeWork) == 32, "work records are read as 32-byte scalar loads");

// Per-sequence decode metadata on the device.
struct DecodeMeta {
  const int64_t* seq_off;   // (B)
  const int32_t* seq_len;   // (B)
  const int32_t* pos;       // (B)
  const int32_t* pstart;    // (B) first partial slot of sequence b
  const int32_t* nseg;      // (B) number of partial slots of sequence b
  const DecodeSeg* segs;    // (nseg_total)
  const int32_t* part_begin;  // (parts + 1) segment range of each persistent part
  const int32_t* cstart;    // (B) first chunk slot of sequence b (two-stage combine)
  const DecodeWork* work;   // (nseg_total) work records of the MFMA core
  // Paged cache (page_shift > 0): pages of 2^page_shift rows; position t of
  // sequence b is cache row pages[pg_off[b] + (t >> page_shift)] *
  // 2^page_shift + t % 2^page_shift, and a work record's `row` holds
  // pg_off[b] << 32 | (the segment's first position).  page_shift == 0: rows
  // of sequence b are contiguous from seq_off[b] and `row` is the segment's
  // first cache row.
  const int32_t* pages;     // (sum_b ceil(seq_len[b] / page_rows))
  const int32_t* pg_off;    // (B)
  int32_t page_shift;
};

// The 512-wide combine merges the partials of a sequence in chunks of
// kCombineChunk slots; a sequence with more than one chunk gets a second pass.
constexpr int kCombineChunk = 16;

// ---- GEMM: Cpart[z][bt][m][n] = sum_{k in split z} A[bt][m][k] * W[bt][n][k]
// A row m of batch bt at A + bt*sA + m*lda; W row n at W + bt*sW + n*ldw.
// The K range is cut into ksplit equal chunks (kchunk = K / ksplit).
template <typename T>
void gemm_generic(const T* A, int64_t lda, int64_t sA, const T* W, int64_t ldw, int64_t sW,
                  float* C, int M, int N, int K, int batch, int ksplit, hipStream_t st);
// Fused GEMM epilogue: out[bt*so + m*ldo + n] = alpha * C (fp32 if f32 is set,
// else rounded to bf16 into b16).
// Host-to-device copy folded into a kernel launch: `blocks` extra blocks,
// numbered from `first_block`, copy n16 16-byte words from pinned host memory
// (read over the bus, zero-copy) to device memory while the kernel's other
// blocks run.  n16 = 0: none.
struct HostCopy {
  const void* src = nullptr;
  void* dst = nullptr;
  int n16 = 0;
  int first_block = 0;
  int blocks = 0;
};

struct GemmOut {
  float* f32;
  bf16* b16;
  int64_t ldo, so;
  float alpha;
};
// MFMA bf16 GEMM (decode shapes): needs N % 16 == 0, K % 128 == 0 and
// (K/32) % (4*ksplit) == 0.  ksplit == 1: the result goes through `out`.
// ksplit > 1: fp32 partials part[((z * batch + bt) * M + m) * N + n] are left
// for the consumer to sum over z (the epilogue is not applied).
void gemm_bf16_mfma(const bf16* A, int64_t lda, int64_t sA, const bf16* W, int64_t ldw,
                    int64_t sW, int M, int N, int K, int batch, int ksplit, float* part,
                    const GemmOut& out, hipStream_t st);
int gemm_bf16_ksplit(int M, int N, int K, int batch, int n_cu);

// Large-tile GEMM (k_gemm_big.hip) for many rows: C = alpha A W^T, batch 1,
// K a multiple of 32, out.ldo a multiple of 4.  A and W are in the
// fragment-tiled layout tile_rows writes (tiled_bytes(rows, K) bytes each).
// gemm_big_bn: the tile width (256 or 128) it picks for an M x N product.
int gemm_big_bn(int M, int N, int n_cu);
void gemm_big(const bf16* A, const bf16* W, int M, int N, int K, const GemmOut& out, int n_cu,
              hipStream_t st);
// Row-major rows x (rows, K) with row stride ld (a multiple of 8) -> the
// fragment-tiled layout: 16-row block b, k step s (32 wide) at byte (b * K /
// 32 + s) * 1024, lanes in MFMA operand order; rows past `rows` are zero.
size_t tiled_bytes(int rows, int K);
void tile_rows(const bf16* x, int64_t ld, int rows, int K, bf16* t, hipStream_t st);

// Split-K partial sums as a consumer sees them: element (z, row, col) at
// p[z * zs + row * ld + col], summed over z = 0..ks-1 in order.
struct Part {
  const float* p;
  int ks;
  int64_t ld, zs;
};

// out = alpha * sum_z C[z] (layout [z][bt][m][n]) with GemmOut's strides and type
void gemm_store(const float* C, int ks, int M, int N, int batch, const GemmOut& out,
                hipStream_t st);

// ---- epilogues over split-K partials
// out[row] = T(RMSNorm(sum_z x[z][row][0:n]) * gamma)
template <typename T>
void rmsnorm_rows(const Part& x, int rows, int n, const T* gamma, float eps, T* out,
                  hipStream_t st);
// latent rows: cache[slot[t]] = [RMSNorm(a[:dc])*gamma | RoPE(a[dc:R], pos[t])]
template <typename T>
void append_rows(const Part& a, int ntok, const int32_t* pos, const int64_t* slot,
                 const T* gamma, T* cache, const Dims& d, const RopeTab& rt, hipStream_t st);
// query heads: q_nope[t][h][:] = T(q_nope); rope_out[t*tok_stride + h*head_stride + i] =
// T(scale * RoPE(q_rope)[i])
template <typename T>
void q_finish(const Part& q, int ntok, const int32_t* pos, T* q_nope, T* rope_out,
              int64_t tok_stride, int64_t head_stride, float scale, const Dims& d,
              const RopeTab& rt, hipStream_t st);
// append_rows on columns [0, R) and q_finish on columns [R, R + H(dn+dr)) of
// one fused in-projection, one block per token
template <typename T>
void step_finish(const Part& a, int ntok, const int32_t* pos, const int64_t* slot,
                 const T* gamma, T* cache, T* q_nope, T* rope_out, int64_t tok_stride,
                 int64_t head_stride, float scale, const Dims& d, const RopeTab& rt,
                 hipStream_t st, bool kv8 = false);  // kv8: `cache` holds FP8 rows (bf16 only)
// per-head transpose: out[h][c][n] = in[h*stride + n*cols + c], n < rows, c < cols
template <typename T>
void transpose_heads(const T* in, T* out, int H, int rows, int cols, int64_t stride,
                     hipStream_t st);
// raw row scatter
template <typename T>
void cache_write(const T* rows, const int64_t* slot, int ntok, int R, T* cache, hipStream_t st);

// ---- decode-step GEMMs with in-place epilogues (no split over blocks):
// C = A W^T for M <= 128 rows and K % 256 == 0 (skinny_ok), bf16 operands.
bool skinny_ok(int M, int N, int K);
// compute units of the current device (cached per device)
int device_cu_count();
// For few rows against large weights (M <= 32, N K >= 8 Mi elements,
// K % 128 == 0, N % 4 == 0) the same products run split-K with the activation
// slice resident in LDS, over W's fragment-tiled copy (tile_rows layout);
// res_slices: the K slices that path uses (0: it does not apply).  With more
// than one slice it needs res_slices * M * N fp32 of partials.
int res_slices(int M, int N, int K);
struct StreamRes {
  const bf16* wt = nullptr;  // W fragment-tiled, or null: the 32-column tiles
  float* part = nullptr;     // split-K partials
};
// out (bf16, row stride ldo) = alpha C
void skinny_store(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K,
                  bf16* out, int64_t ldo, float alpha, hipStream_t st,
                  const StreamRes& r = StreamRes{});
// out (fp32, row stride ldo) = C
void skinny_f32(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K,
                float* out, int64_t ldo, hipStream_t st, const HostCopy& hc = HostCopy{},
                const StreamRes& r = StreamRes{});
// columns [0, R) of C to a (fp32, row stride R); the remaining columns are
// query heads [nope (dn) | rope (dr)]: nope to q_nope (M, H, dn), rope rotated
// at pos_host[row] (a host array, passed to the kernel by value) and scaled by
// d.scale into q_cat[row][h][dc ..] (row stride H R).  With q_nope null the
// heads are [q_abs (dc) | rope (dr)] (materialised W^KQ rows) and q_abs goes
// scaled into q_cat[row][h][0 .. dc).
void skinny_query(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K,
                  float* a, int R, bf16* q_nope, bf16* q_cat, const int32_t* pos_host,
                  const Dims& d, const RopeTab& rt, hipStream_t st,
                  const HostCopy& hc = HostCopy{}, const StreamRes& r = StreamRes{});
// Blocks (of 256 threads) a HostCopy of n16 words takes.
int host_copy_blocks(int n16);
// One launch finishing the projections of B tokens, each part optional:
// absorb: q_cat[t][h][0:dc] = scale * W_ukT_h q_nope[t][h] (dc = 512);
// append: cache[slot[t]] = [RMSNorm(a[t][0:dc]) * kv_gamma | RoPE(a[t][dc:R], pos[t])];
// qnorm:  cq[t] = RMSNorm(a[t][qa_col : qa_col + dq]) * q_gamma (bf16).
void decode_finish(const bf16* q_nope, const bf16* w_ukT, bf16* q_cat, int B, bool absorb,
                   bool append, bool qnorm, const float* a, int lda, int qa_col,
                   const int32_t* pos, const int64_t* slot, const bf16* kv_gamma, void* cache,
                   const bf16* q_gamma, bf16* cq, const Dims& d, const RopeTab& rt,
                   hipStream_t st, bool kv8 = false);  // kv8: `cache` holds FP8 rows

// ---- decode core (split-S) and combine
// q_len new tokens per sequence: query row b * q_len + j (q_cat, o_lat) is
// token j of sequence b, at position seq_len[b] - q_len + j; on the
// sequence's last segment it sees q_len - 1 - j rows fewer.  Partial layout:
// acc[j * nseg_total + pidx][h][dc] fp32, ml[...][h][2] = (max in log2 units,
// sum).
struct TokenSplit {
  int q_len, nseg_total;
};
template <typename T>
void decode_core_generic(const T* q_cat, const T* cache, const DecodeMeta& m, int nseg_total,
                         int q_len, float* acc, float* ml, const Dims& d, hipStream_t st);
// MFMA core for head counts that are a multiple of decode_core_wide_heads()
// (128): each workgroup covers that many heads of a part over shared row
// tiles; the H / 128 workgroups of a part run on one XCD.
int decode_core_wide_heads();
void decode_core_wide(const bf16* q_cat, const bf16* cache, const DecodeMeta& m, int parts,
                      const TokenSplit& tk, float* acc, float* ml, const Dims& d,
                      hipStream_t st);
// The same over FP8 rows (fp8_row_bytes(512, 64) bytes): each tile of raw rows
// is decoded once into the shared bf16 tile (code values, exact) with the row
// scales applied in fp32 to the scores and the latent sum's operand.
void decode_core_wide8(const bf16* q_cat, const uint8_t* cache, const DecodeMeta& m, int parts,
                       const TokenSplit& tk, float* acc, float* ml, const Dims& d,
                       hipStream_t st);
// FP8 latent cache (rows of fp8_row_bytes(dc, dr) bytes, dc == 512, dr == 64):
// the latent row append (as append_rows, into FP8 rows), the store of rows
// given in bf16 (T x R) into FP8 rows, a raw row-byte scatter, and the ring
// core reading FP8 rows (otherwise as decode_core_ring).
void append_rows_fp8(const Part& a, int ntok, const int32_t* pos, const int64_t* slot,
                     const bf16* gamma, uint8_t* cache, const Dims& d, const RopeTab& rt,
                     hipStream_t st);
void cache_store_fp8(const bf16* rows, const int64_t* slot, int ntok, uint8_t* cache,
                     const Dims& d, hipStream_t st);
void cache_write_bytes(const uint8_t* rows, const int64_t* slot, int ntok, int row_bytes,
                       uint8_t* cache, hipStream_t st);
void decode_core_ring8(const bf16* q_cat, const uint8_t* cache, const DecodeMeta& m, int parts,
                       const TokenSplit& tk, float* acc, float* ml, bf16* o_lat, const Dims& d,
                       hipStream_t st);
// MFMA core over a ring of shared row tiles (bf16, dc == 512, dr == 64,
// H % 16 == 0): one workgroup per (part, token, 16-head group), parts =
// persistent workgroups per (token, head group).  Partials as for the generic
// core, except that a sequence contained in one segment is normalised and
// written to o_lat (B * q_len, H, 512) directly.
// tokens of a sequence one workgroup of the ring core covers (2 for an even
// q_len: the part's rows then stream once per token pair)
int decode_core_ring_tokens(int q_len);
void decode_core_ring(const bf16* q_cat, const bf16* cache, const DecodeMeta& m, int parts,
                      const TokenSplit& tk, float* acc, float* ml, bf16* o_lat, const Dims& d,
                      hipStream_t st);
// combine for dc == 512, bf16 output.  max_chunks = max over sequences of
// ceil(nseg / kCombineChunk); cacc (chunk slots x H x 512) and cml (chunk slots
// x H x 2) hold the chunk partials of sequences with more than one chunk.
// direct_single: sequences with one partial were finished into o_lat by the
// core (the ring core does that) and are left alone.
void decode_combine_512(const float* acc, const float* ml, const DecodeMeta& m, int B, int H,
                        int max_chunks, float* cacc, float* cml, bool direct_single,
                        bf16* o_lat, hipStream_t st);
template <typename T>
void decode_combine(const float* acc, const float* ml, const DecodeMeta& m, int B, T* o_lat,
                    const Dims& d, hipStream_t st);
// combine fused with the value un-absorb for dc == 512, dv == 128 (bf16):
// o_lat (B, H, 512) = merged latent sums (read back instead for sequences with
// one partial when direct_single: the core wrote them), o (B, H * 128) =
// per head W_UV_h o_lat_h; w_uv is (H, 128, 512).
void decode_combine_uv(const float* acc, const float* ml, const DecodeMeta& m, int B, int H,
                       int max_chunks, float* cacc, float* cml, bool direct_single,
                       const bf16* w_uv, bf16* o_lat, bf16* o, hipStream_t st);

// ---- prefill attention (non-absorbed, causal)
// One query tile of the MFMA prefill kernel: new tokens t0 .. t0+nq-1 of one
// sequence at positions pos0 .. pos0+nq-1; the sequence's expanded rows start
// at kv_row0 and its cache rows at cache_row0.
struct PrefillTile {
  int64_t kv_row0, cache_row0;
  int32_t t0, nq, pos0, pad;
};
// Where the key rows of prefill sequence b live: contiguous rows from
// seq_off[b], or row t at pages[page_start[b] + t / 2^page_shift] *
// 2^page_shift + t % 2^page_shift (a paged cache).
struct KeyRowSrc {
  const void* cache;
  const int64_t* seq_off;     // (B) device; unused for a paged cache
  const int32_t* page_start;  // (B) device; paged cache only
  const int32_t* pages;       // device page list, or null for a contiguous cache
  int page_shift;
};
// Copies the nrows[b] key rows of every sequence b to out + kv_off[b] rows
// (row_bytes per output row); fp8: decodes 656-byte FP8 rows (dc 512, dr 64)
// into bf16 rows of 576.  Returns nonzero if fp8 rows do not fit row_bytes.
int gather_key_rows(const KeyRowSrc& s, bool fp8, const int64_t* kv_off, const int32_t* nrows,
                    int B, int max_rows, int row_bytes, void* out, hipStream_t st);
// queries per tile of prefill_attn_mfma
int prefill_tile_queries();
// MFMA version: bf16, qk_nope = v_head = 128, qk_rope = 64.  q: (T, H, 192)
// rows [q_nope | q_rope] (the rope part is rotated by the kernel at each
// query's position); kv: expanded rows (H x [K_nope | V]) in bf16;
// o: (T, H, 128) rows, or with o_tiled the fragment-tiled layout of the
// (T, H * 128) output-projection operand (tiled_bytes(T, H * 128) bytes);
// scale: softmax scale.
void prefill_attn_mfma(const bf16* q, const bf16* kv, const bf16* cache,
                       const PrefillTile* tiles, int ntiles, int H, float scale, bf16* o,
                       bool o_tiled, const RopeTab& rt, hipStream_t st);
// kv: per sequence the expanded rows [K_nope_h | V_h] (fp32, row width H*(dn+dv)),
// sequence b at row kv_off[b]; q_nope (T,H,dn), q_rope (T,H,dr) already rotated.
template <typename T>
void prefill_attn_generic(const T* q_nope, const T* q_rope, const float* kv, const T* cache,
                          const int32_t* tok_seq, const int32_t* tok_pos,
                          const int64_t* kv_off, const int64_t* seq_off, int ntok, T* o,
                          const Dims& d, hipStream_t st);

// Device address of the current device's copy of the static scratch array of
// mla_decode_step_noalloc (scratch.hip).
hipError_t noalloc_scratch_address(void** out);

}  // namespace mla
