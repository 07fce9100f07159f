// Shape-generic kernels (fp32 or bf16 storage, fp32 arithmetic): the GEMM
// used when the MFMA tiling does not apply, the split-K epilogues, latent-row
// append, the query finish, the raw cache scatter, the VALU split-S decode
// core, the split combine and the non-absorbed prefill attention.
#include "kernels.h"
#include "row_dev.h"

#include <math.h>

namespace mla {

// ---------------------------------------------------------------------------
// GEMM (VALU, 16x16 LDS tiles): Cpart[z][bt][m][n] = sum_k A[m][k] * W[n][k]
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
gemm_generic_k(const T* __restrict__ A, int64_t lda, int64_t sA, const T* __restrict__ W,
               int64_t ldw, int64_t sW, float* __restrict__ C, int M, int N, int K,
               int batch, int kchunk) {
  __shared__ float As[16][17];
  __shared__ float Ws[16][17];
  const int bt = blockIdx.z % batch, z = blockIdx.z / batch;
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 16;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const T* Ab = A + bt * sA;
  const T* Wb = W + bt * sW;
  const int kb = z * kchunk, ke = min(K, kb + kchunk);
  float acc = 0.f;
  for (int k0 = kb; k0 < ke; k0 += 16) {
    const int k = k0 + tx;
    As[ty][tx] = (m0 + ty < M && k < ke) ? ldf(Ab + (int64_t)(m0 + ty) * lda + k) : 0.f;
    Ws[ty][tx] = (n0 + ty < N && k < ke) ? ldf(Wb + (int64_t)(n0 + ty) * ldw + k) : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(As[ty][kk], Ws[tx][kk], acc);
    __syncthreads();
  }
  if (m0 + ty < M && n0 + tx < N)
    C[((int64_t)(z * batch + bt) * M + m0 + ty) * N + n0 + tx] = acc;
}

template <typename T>
void gemm_generic(const T* A, int64_t lda, int64_t sA, const T* W, int64_t ldw, int64_t sW,
                  float* C, int M, int N, int K, int batch, int ksplit, hipStream_t st) {
  const int kchunk = (K + ksplit - 1) / ksplit;
  dim3 grid((N + 15) / 16, (M + 15) / 16, batch * ksplit);
  gemm_generic_k<T><<<grid, 256, 0, st>>>(A, lda, sA, W, ldw, sW, C, M, N, K, batch, kchunk);
}

// ---------------------------------------------------------------------------
// epilogues over split-K partials (summed in split order z = 0..ks-1)
// ---------------------------------------------------------------------------
__global__ void gemm_store_k(const float* __restrict__ C, int ks, int M, int N, int batch,
                             GemmOut out) {
  const int64_t total = (int64_t)batch * M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = C[i];
    for (int z = 1; z < ks; ++z) v += C[z * total + i];
    const int n = (int)(i % N);
    const int64_t r = i / N;
    const int m = (int)(r % M);
    const int bt = (int)(r / M);
    const int64_t o = bt * out.so + (int64_t)m * out.ldo + n;
    if (out.f32)
      out.f32[o] = out.alpha * v;
    else
      out.b16[o] = f32_to_bf16(out.alpha * v);
  }
}

void gemm_store(const float* C, int ks, int M, int N, int batch, const GemmOut& out,
                hipStream_t st) {
  const int64_t total = (int64_t)batch * M * N;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  gemm_store_k<<<blocks, 256, 0, st>>>(C, ks, M, N, batch, out);
}

template <typename T>
__global__ void __launch_bounds__(256)
rmsnorm_rows_k(Part x, int n, const T* __restrict__ gamma, float eps, T* __restrict__ out) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  float ss = 0.f;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const float a = part_at(x, r, j);
    ss += a * a;
  }
  const float inv = rsqrtf(block_sum_256(ss, red) / (float)n + eps);
  for (int j = threadIdx.x; j < n; j += blockDim.x)
    stf(out + (int64_t)r * n + j, part_at(x, r, j) * inv * ldf(gamma + j));
}

template <typename T>
void rmsnorm_rows(const Part& x, int rows, int n, const T* gamma, float eps, T* out,
                  hipStream_t st) {
  rmsnorm_rows_k<T><<<rows, 256, 0, st>>>(x, n, gamma, eps, out);
}

template <typename T>
__device__ __forceinline__ void q_finish_block(const Part& q, int t, int p, int h0, int h1,
                                               T* __restrict__ q_nope, T* __restrict__ rope_out,
                                               int64_t tok_stride, int64_t head_stride,
                                               float scale, const Dims& d, const RopeTab& rt) {
  const int w = d.dn + d.dr;
  for (int i = threadIdx.x; i < (h1 - h0) * d.dn; i += blockDim.x) {
    const int h = h0 + i / d.dn, j = i % d.dn;
    stf(q_nope + ((int64_t)t * d.H + h) * d.dn + j, part_at(q, t, h * w + j));
  }
  const int hp = d.dr / 2;
  for (int i = threadIdx.x; i < (h1 - h0) * hp; i += blockDim.x) {
    const int h = h0 + i / hp, k = i % hp;
    float ou, ov;
    rope_pair(part_at(q, t, h * w + d.dn + 2 * k), part_at(q, t, h * w + d.dn + 2 * k + 1), p,
              rt.theta[k], &ou, &ov);
    T* o = rope_out + t * tok_stride + h * head_stride;
    stf(o + 2 * k, ou * scale);
    stf(o + 2 * k + 1, ov * scale);
  }
}

// heads per q_finish block: ~4 KB of partial columns per block
__host__ __device__ inline int q_heads_per_block(const Dims& d) {
  int g = 1024 / (d.dn + d.dr);
  return g < 1 ? 1 : g;
}

template <typename T>
__global__ void __launch_bounds__(256)
append_rows_k(Part a, const int32_t* __restrict__ pos, const int64_t* __restrict__ slot,
              const T* __restrict__ gamma, T* __restrict__ cache, Dims d, RopeTab rt) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  append_row_block<T>(a, t, pos[t], slot[t], gamma, cache, d, rt, red);
}

template <typename T>
void append_rows(const Part& a, int ntok, const int32_t* pos, const int64_t* slot,
                 const T* gamma, T* cache, const Dims& d, const RopeTab& rt, hipStream_t st) {
  append_rows_k<T><<<ntok, 256, 0, st>>>(a, pos, slot, gamma, cache, d, rt);
}

template <typename T>
__global__ void __launch_bounds__(256)
q_finish_k(Part q, const int32_t* __restrict__ pos, T* __restrict__ q_nope,
           T* __restrict__ rope_out, int64_t tok_stride, int64_t head_stride, float scale, Dims d,
           RopeTab rt) {
  const int t = blockIdx.x, g = q_heads_per_block(d);
  const int h0 = blockIdx.y * g, h1 = min(d.H, h0 + g);
  q_finish_block<T>(q, t, pos[t], h0, h1, q_nope, rope_out, tok_stride, head_stride, scale, d,
                    rt);
}

template <typename T>
void q_finish(const Part& q, int ntok, const int32_t* pos, T* q_nope, T* rope_out,
              int64_t tok_stride, int64_t head_stride, float scale, const Dims& d,
              const RopeTab& rt, hipStream_t st) {
  const int g = q_heads_per_block(d);
  dim3 grid(ntok, (d.H + g - 1) / g);
  q_finish_k<T><<<grid, 256, 0, st>>>(q, pos, q_nope, rope_out, tok_stride, head_stride, scale,
                                       d, rt);
}

// blockIdx.y == 0: the token's latent row; blockIdx.y >= 1: a group of query
// heads (one launch finishes the fused in-projection)
template <typename T>
__global__ void __launch_bounds__(256)
step_finish_k(Part a, const int32_t* __restrict__ pos, const int64_t* __restrict__ slot,
              const T* __restrict__ gamma, T* __restrict__ cache, T* __restrict__ q_nope,
              T* __restrict__ rope_out, int64_t tok_stride, int64_t head_stride, float scale,
              Dims d, RopeTab rt, int kv8) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  if (blockIdx.y == 0) {
    if constexpr (sizeof(T) == 2) {
      if (kv8) {  // the cache holds FP8 rows
        append_row_block_fp8(a, t, pos[t], slot[t], gamma, reinterpret_cast<uint8_t*>(cache), d,
                             rt, red);
        return;
      }
    }
    append_row_block<T>(a, t, pos[t], slot[t], gamma, cache, d, rt, red);
    return;
  }
  Part q = a;
  q.p += d.R;
  const int g = q_heads_per_block(d);
  const int h0 = (blockIdx.y - 1) * g, h1 = min(d.H, h0 + g);
  q_finish_block<T>(q, t, pos[t], h0, h1, q_nope, rope_out, tok_stride, head_stride, scale, d,
                    rt);
}

template <typename T>
void step_finish(const Part& a, int ntok, const int32_t* pos, const int64_t* slot,
                 const T* gamma, T* cache, T* q_nope, T* rope_out, int64_t tok_stride,
                 int64_t head_stride, float scale, const Dims& d, const RopeTab& rt,
                 hipStream_t st, bool kv8) {
  const int g = q_heads_per_block(d);
  dim3 grid(ntok, 1 + (d.H + g - 1) / g);
  step_finish_k<T><<<grid, 256, 0, st>>>(a, pos, slot, gamma, cache, q_nope, rope_out,
                                          tok_stride, head_stride, scale, d, rt, kv8 ? 1 : 0);
}

template <typename T>
__global__ void transpose_heads_k(const T* __restrict__ in, T* __restrict__ out, int rows,
                                  int cols, int64_t stride) {
  const int h = blockIdx.y;
  const int64_t total = (int64_t)rows * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i / rows), n = (int)(i % rows);
    out[(int64_t)h * total + i] = in[h * stride + (int64_t)n * cols + c];
  }
}

template <typename T>
void transpose_heads(const T* in, T* out, int H, int rows, int cols, int64_t stride,
                     hipStream_t st) {
  dim3 grid((unsigned)(((int64_t)rows * cols + 255) / 256), H);
  transpose_heads_k<T><<<grid, 256, 0, st>>>(in, out, rows, cols, stride);
}

__global__ void __launch_bounds__(256)
append_rows_fp8_k(Part a, const int32_t* __restrict__ pos, const int64_t* __restrict__ slot,
                  const bf16* __restrict__ gamma, uint8_t* __restrict__ cache, Dims d, RopeTab rt) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  append_row_block_fp8(a, t, pos[t], slot[t], gamma, cache, d, rt, red);
}

void append_rows_fp8(const Part& a, int ntok, const int32_t* pos, const int64_t* slot,
                     const bf16* gamma, uint8_t* cache, const Dims& d, const RopeTab& rt,
                     hipStream_t st) {
  append_rows_fp8_k<<<ntok, 256, 0, st>>>(a, pos, slot, gamma, cache, d, rt);
}

// rows (T x R, bf16) -> FP8 rows: the latent part quantised as the append
// does, the rope part copied
__global__ void __launch_bounds__(256)
cache_store_fp8_k(const bf16* __restrict__ rows, const int64_t* __restrict__ slot,
                  uint8_t* __restrict__ cache, Dims d) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const bf16* src = rows + (int64_t)t * d.R;
  uint8_t* row = cache + slot[t] * (int64_t)fp8_row_bytes(d.dc, d.dr);
  store_latent_fp8([&](int j) { return bf16_to_f32(src[j]); }, row, d, red);
  bf16* rope = reinterpret_cast<bf16*>(row + d.dc);
  for (int i = threadIdx.x; i < d.dr; i += blockDim.x) rope[i] = src[d.dc + i];
}

void cache_store_fp8(const bf16* rows, const int64_t* slot, int ntok, uint8_t* cache,
                     const Dims& d, hipStream_t st) {
  cache_store_fp8_k<<<ntok, 256, 0, st>>>(rows, slot, cache, d);
}

// raw scatter of whole rows (row_bytes a multiple of 16)
__global__ void cache_write_bytes_k(const uint8_t* __restrict__ rows,
                                    const int64_t* __restrict__ slot, int row_bytes,
                                    uint8_t* __restrict__ cache) {
  const int t = blockIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(rows + (int64_t)t * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(cache + slot[t] * (int64_t)row_bytes);
  for (int j = threadIdx.x; j < row_bytes / 16; j += blockDim.x) dst[j] = src[j];
}

void cache_write_bytes(const uint8_t* rows, const int64_t* slot, int ntok, int row_bytes,
                       uint8_t* cache, hipStream_t st) {
  cache_write_bytes_k<<<ntok, 64, 0, st>>>(rows, slot, row_bytes, cache);
}

template <typename T>
__global__ void cache_write_k(const T* __restrict__ rows, const int64_t* __restrict__ slot,
                              int ntok, int R, T* __restrict__ cache) {
  const int t = blockIdx.x;
  const int64_t s = slot[t];
  for (int j = threadIdx.x; j < R; j += blockDim.x) cache[s * R + j] = rows[(int64_t)t * R + j];
}

template <typename T>
void cache_write(const T* rows, const int64_t* slot, int ntok, int R, T* cache, hipStream_t st) {
  cache_write_k<T><<<ntok, 256, 0, st>>>(rows, slot, ntok, R, cache);
}

// ---------------------------------------------------------------------------
// Split-S decode core, VALU version: one block per (segment, head).  Scores
// are kept in log2 units (s * log2 e) so the softmax uses exp2.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
decode_core_generic_k(const T* __restrict__ q_cat, const T* __restrict__ cache, DecodeMeta mt,
                      float* __restrict__ acc_out, float* __restrict__ ml_out, Dims d, int q_len,
                      int nseg_total) {
  extern __shared__ float sm[];
  float* q = sm;              // R
  float* p = q + d.R;         // 256
  float* red = p + 256;       // 4
  const DecodeSeg sg = mt.segs[blockIdx.x];
  const int h = blockIdx.y % d.H, tok = blockIdx.y / d.H;  // head, new token
  const int R = d.R;
  for (int j = threadIdx.x; j < R; j += blockDim.x)
    q[j] = ldf(q_cat + ((int64_t)(sg.b * q_len + tok) * d.H + h) * R + j);
  __syncthreads();
  // rows token tok sees: on the sequence's last segment, not the later tokens'
  const int n = sg.r1 - sg.r0 - (sg.r1 == mt.seq_len[sg.b] ? q_len - 1 - tok : 0);
  // cache row of the segment's position t (contiguous, or through the page list)
  auto row_of = [&](int t) -> const T* {
    int64_t r;
    if (mt.page_shift) {
      const int pos = sg.r0 + t;
      r = ((int64_t)mt.pages[mt.pg_off[sg.b] + (pos >> mt.page_shift)] << mt.page_shift) +
          (pos & ((1 << mt.page_shift) - 1));
    } else {
      r = mt.seq_off[sg.b] + sg.r0 + t;
    }
    return cache + r * (int64_t)R;
  };
  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // dc <= 1024
  for (int t0 = 0; t0 < n; t0 += 256) {
    const int t = t0 + threadIdx.x;
    float s = -INFINITY;
    if (t < n) {
      const T* r = row_of(t);
      float dot = 0.f;
      for (int j = 0; j < R; ++j) dot = fmaf(q[j], ldf(r + j), dot);
      s = dot * kLog2e;
    }
    // block max
    float bm = warp_max(s);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = bm;
    __syncthreads();
    bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float mn = fmaxf(m, bm);
    const float alpha = exp2f(m - mn);
    const float pt = (t < n) ? exp2f(s - mn) : 0.f;
    p[threadIdx.x] = pt;
    const float ps = block_sum_256(pt, red);  // contains the barrier that publishes p
    l = l * alpha + ps;
    m = mn;
    const int cnt = min(256, n - t0);
    for (int c4 = 0; c4 < 4; ++c4) {
      const int c = threadIdx.x + c4 * 256;
      if (c < d.dc) {
        float a = acc[c4] * alpha;
        for (int k = 0; k < cnt; ++k) a = fmaf(p[k], ldf(row_of(t0 + k) + c), a);
        acc[c4] = a;
      }
    }
    __syncthreads();
  }
  const int64_t slot = (int64_t)tok * nseg_total + sg.pidx;
  float* ao = acc_out + (slot * d.H + h) * d.dc;
  for (int c4 = 0; c4 < 4; ++c4) {
    const int c = threadIdx.x + c4 * 256;
    if (c < d.dc) ao[c] = acc[c4];
  }
  if (threadIdx.x == 0) {
    ml_out[(slot * d.H + h) * 2] = m;
    ml_out[(slot * d.H + h) * 2 + 1] = l;
  }
}

template <typename T>
void decode_core_generic(const T* q_cat, const T* cache, const DecodeMeta& m, int nseg_total,
                         int q_len, float* acc, float* ml, const Dims& d, hipStream_t st) {
  dim3 grid(nseg_total, d.H * q_len);
  const size_t smem = (size_t)(d.R + 256 + 4) * sizeof(float);
  decode_core_generic_k<T><<<grid, 256, smem, st>>>(q_cat, cache, m, acc, ml, d, q_len,
                                                    nseg_total);
}

// Split combine: o_lat[b][h] = sum_j e^(m_j - M) acc_j / sum_j e^(m_j - M) l_j,
// summed in the fixed slot order (deterministic).
template <typename T>
__global__ void __launch_bounds__(256)
decode_combine_k(const float* __restrict__ acc, const float* __restrict__ ml, DecodeMeta mt,
                 T* __restrict__ o_lat, Dims d) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int j0 = mt.pstart[b], nj = mt.nseg[b];
  float M = -INFINITY;
  for (int j = 0; j < nj; ++j) M = fmaxf(M, ml[((int64_t)(j0 + j) * d.H + h) * 2]);
  float L = 0.f;
  for (int j = 0; j < nj; ++j) {
    const float* e = ml + ((int64_t)(j0 + j) * d.H + h) * 2;
    L += exp2f(e[0] - M) * e[1];
  }
  const float invL = 1.f / L;
  for (int c = threadIdx.x; c < d.dc; c += blockDim.x) {
    float s = 0.f;
    for (int j = 0; j < nj; ++j) {
      const float w = exp2f(ml[((int64_t)(j0 + j) * d.H + h) * 2] - M);
      s = fmaf(w, acc[((int64_t)(j0 + j) * d.H + h) * d.dc + c], s);
    }
    stf(o_lat + ((int64_t)b * d.H + h) * d.dc + c, s * invL);
  }
}

template <typename T>
void decode_combine(const float* acc, const float* ml, const DecodeMeta& m, int B, T* o_lat,
                    const Dims& d, hipStream_t st) {
  dim3 grid(B, d.H);
  decode_combine_k<T><<<grid, 256, 0, st>>>(acc, ml, m, o_lat, d);
}

// ---------------------------------------------------------------------------
// Prefill attention, non-absorbed, VALU: one block per (token, head).
// Keys: [K_nope_h ; k_rope] (k_rope from the cache row), values V_h, visible
// rows 0..pos ("Transformer and KV Cache Basics", mask design).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
prefill_attn_generic_k(const T* __restrict__ q_nope, const T* __restrict__ q_rope,
                       const float* __restrict__ kv, const T* __restrict__ cache,
                       const int32_t* __restrict__ tok_seq, const int32_t* __restrict__ tok_pos,
                       const int64_t* __restrict__ kv_off, const int64_t* __restrict__ seq_off,
                       T* __restrict__ o, Dims d) {
  extern __shared__ float sm[];
  const int dq = d.dn + d.dr;
  float* q = sm;           // dq
  float* p = q + dq;       // 256
  float* red = p + 256;    // 4
  const int t = blockIdx.x, h = blockIdx.y;
  const int b = tok_seq[t], pos = tok_pos[t];
  for (int j = threadIdx.x; j < dq; j += blockDim.x)
    q[j] = j < d.dn ? ldf(q_nope + ((int64_t)t * d.H + h) * d.dn + j)
                    : ldf(q_rope + ((int64_t)t * d.H + h) * d.dr + (j - d.dn));
  __syncthreads();
  const int wkv = d.H * (d.dn + d.dv);
  const float* kvb = kv + kv_off[b] * (int64_t)wkv + h * (d.dn + d.dv);
  const T* cb = cache + seq_off[b] * (int64_t)d.R + d.dc;
  const int n = pos + 1;
  float m = -INFINITY, l = 0.f;
  float acc = 0.f;  // thread j < dv owns output j (dv <= 256)
  for (int t0 = 0; t0 < n; t0 += 256) {
    const int k = t0 + threadIdx.x;
    float s = -INFINITY;
    if (k < n) {
      float dot = 0.f;
      const float* kr = kvb + (int64_t)k * wkv;
      for (int j = 0; j < d.dn; ++j) dot = fmaf(q[j], kr[j], dot);
      const T* rr = cb + (int64_t)k * d.R;
      for (int j = 0; j < d.dr; ++j) dot = fmaf(q[d.dn + j], ldf(rr + j), dot);
      s = dot * d.scale * kLog2e;
    }
    float bm = warp_max(s);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = bm;
    __syncthreads();
    bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float mn = fmaxf(m, bm);
    const float alpha = exp2f(m - mn);
    const float pt = (k < n) ? exp2f(s - mn) : 0.f;
    p[threadIdx.x] = pt;
    const float ps = block_sum_256(pt, red);
    l = l * alpha + ps;
    m = mn;
    const int cnt = min(256, n - t0);
    if (threadIdx.x < d.dv) {
      float a = acc * alpha;
      for (int kk = 0; kk < cnt; ++kk)
        a = fmaf(p[kk], kvb[(int64_t)(t0 + kk) * wkv + d.dn + threadIdx.x], a);
      acc = a;
    }
    __syncthreads();
  }
  if (threadIdx.x < d.dv) stf(o + ((int64_t)t * d.H + h) * d.dv + threadIdx.x, acc / l);
}

template <typename T>
void prefill_attn_generic(const T* q_nope, const T* q_rope, const float* kv, const T* cache,
                          const int32_t* tok_seq, const int32_t* tok_pos,
                          const int64_t* kv_off, const int64_t* seq_off, int ntok, T* o,
                          const Dims& d, hipStream_t st) {
  dim3 grid(ntok, d.H);
  const size_t smem = (size_t)(d.dn + d.dr + 256 + 4) * sizeof(float);
  prefill_attn_generic_k<T><<<grid, 256, smem, st>>>(q_nope, q_rope, kv, cache, tok_seq,
                                                      tok_pos, kv_off, seq_off, o, d);
}

// explicit instantiations
#define MLA_INST(T)                                                                          \
  template void gemm_generic<T>(const T*, int64_t, int64_t, const T*, int64_t, int64_t,     \
                                float*, int, int, int, int, int, hipStream_t);              \
  template void rmsnorm_rows<T>(const Part&, int, int, const T*, float, T*, hipStream_t);    \
  template void append_rows<T>(const Part&, int, const int32_t*, const int64_t*, const T*,   \
                               T*, const Dims&, const RopeTab&, hipStream_t);                \
  template void q_finish<T>(const Part&, int, const int32_t*, T*, T*, int64_t, int64_t,      \
                            float, const Dims&, const RopeTab&, hipStream_t);                \
  template void step_finish<T>(const Part&, int, const int32_t*, const int64_t*, const T*,   \
                               T*, T*, T*, int64_t, int64_t, float, const Dims&,             \
                               const RopeTab&, hipStream_t, bool);                           \
  template void cache_write<T>(const T*, const int64_t*, int, int, T*, hipStream_t);         \
  template void transpose_heads<T>(const T*, T*, int, int, int, int64_t, hipStream_t);        \
  template void decode_core_generic<T>(const T*, const T*, const DecodeMeta&, int, int,      \
                                       float*, float*, const Dims&, hipStream_t);            \
  template void decode_combine<T>(const float*, const float*, const DecodeMeta&, int, T*,    \
                                  const Dims&, hipStream_t);                                 \
  template void prefill_attn_generic<T>(const T*, const T*, const float*, const T*,          \
                                        const int32_t*, const int32_t*, const int64_t*,      \
                                        const int64_t*, int, T*, const Dims&, hipStream_t);
MLA_INST(float)
MLA_INST(bf16)
#undef MLA_INST

}  // namespace mla
