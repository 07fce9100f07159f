// Internal launcher interface between the host layer (mla.cpp) and the HIP
// kernels.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace mla {

// Shapes the kernels need, copied from the public config.
struct Dims {
  int D, H, dn, dr, dv, dc, dq, R;
  float rope_base, eps, scale;
};

// One decode work segment: rows [r0, r1) of sequence b (row indices relative
// to the sequence start), whose partial result goes to slot pidx.
struct DecodeSeg {
  int32_t b, r0, r1, pidx;
};

// Per-sequence decode metadata on the device.
struct DecodeMeta {
  const int64_t* seq_off;   // (B)
  const int32_t* seq_len;   // (B)
  const int32_t* pos;       // (B)
  const int32_t* pstart;    // (B) first partial slot of sequence b
  const int32_t* nseg;      // (B) number of partial slots of sequence b
  const DecodeSeg* segs;    // (nseg_total)
  const int32_t* part_begin;  // (parts + 1) segment range of each persistent part
};

// ---- GEMM: Cpart[z][bt][m][n] = sum_{k in split z} A[bt][m][k] * W[bt][n][k]
// A row m of batch bt at A + bt*sA + m*lda; W row n at W + bt*sW + n*ldw.
// The K range is cut into ksplit equal chunks (kchunk = K / ksplit).
template <typename T>
void gemm_generic(const T* A, int64_t lda, int64_t sA, const T* W, int64_t ldw, int64_t sW,
                  float* C, int M, int N, int K, int batch, int ksplit, hipStream_t st);
// MFMA bf16 version; needs K % (32*ksplit) == 0 and N % 16 == 0.
void gemm_bf16_mfma(const bf16* A, int64_t lda, int64_t sA, const bf16* W, int64_t ldw,
                    int64_t sW, float* C, int M, int N, int K, int batch, int ksplit,
                    hipStream_t st);

// ---- epilogues over split-K partials
// out[bt*so + m*ldo + n] = T(alpha * sum_z part[z][bt][m][n])
template <typename T>
void sum_store(const float* part, int ksplit, int M, int N, int batch, T* out, int64_t ldo,
               int64_t so, float alpha, hipStream_t st);
// out[row] = T(RMSNorm(sum_z part[z][row]) * gamma)   (row width n)
template <typename T>
void rmsnorm_rows(const float* part, int ksplit, int rows, int n, const T* gamma, float eps,
                  T* out, hipStream_t st);
// latent rows: cache[slot[t]] = [RMSNorm(a[:dc])*gamma | RoPE(a[dc:], pos[t])]
template <typename T>
void append_rows(const float* apart, int ksplit, int ntok, const int32_t* pos,
                 const int64_t* slot, const T* gamma, T* cache, const Dims& d, hipStream_t st);
// query heads: q_nope[t][h][:] = T(q_nope); rope_out[t*tok_stride + h*head_stride + i] =
// T(scale * RoPE(q_rope)[i])
template <typename T>
void q_finish(const float* qpart, int ksplit, int ntok, const int32_t* pos, T* q_nope,
              T* rope_out, int64_t tok_stride, int64_t head_stride, float scale,
              const Dims& d, hipStream_t st);
// per-head transpose: out[h][c][n] = in[h*stride + n*cols + c], n < rows, c < cols
template <typename T>
void transpose_heads(const T* in, T* out, int H, int rows, int cols, int64_t stride,
                     hipStream_t st);
// raw row scatter
template <typename T>
void cache_write(const T* rows, const int64_t* slot, int ntok, int R, T* cache, hipStream_t st);

// ---- decode core (split-S) and combine
// partial layout: acc[pidx][h][dc] fp32, ml[pidx][h][2] = (max in log2 units, sum)
template <typename T>
void decode_core_generic(const T* q_cat, const T* cache, const DecodeMeta& m, int nseg_total,
                         float* acc, float* ml, const Dims& d, hipStream_t st);
// MFMA version: bf16, dc == 512, dr == 64, H % 16 == 0.  parts = persistent groups.
void decode_core_mfma(const bf16* q_cat, const bf16* cache, const DecodeMeta& m, int parts,
                      int B, float* acc, float* ml, const Dims& d, hipStream_t st);
template <typename T>
void decode_combine(const float* acc, const float* ml, const DecodeMeta& m, int B, T* o_lat,
                    const Dims& d, hipStream_t st);

// ---- prefill attention (non-absorbed, causal)
// kv: per sequence the expanded rows [K_nope_h | V_h] (fp32, row width H*(dn+dv)),
// sequence b at row kv_off[b]; q_nope (T,H,dn), q_rope (T,H,dr) already rotated.
template <typename T>
void prefill_attn_generic(const T* q_nope, const T* q_rope, const float* kv, const T* cache,
                          const int32_t* tok_seq, const int32_t* tok_pos,
                          const int64_t* kv_off, const int64_t* seq_off, int ntok, T* o,
                          const Dims& d, hipStream_t st);

}  // namespace mla
