// Device helpers for row-wise epilogues shared by the kernel files: split-K
// partial sums, a 256-thread block sum, RoPE of one pair and the latent-row
// append.
#pragma once

#include <math.h>

#include "kernels.h"

namespace mla {

// Sum over the ks split slices; the loads of 4 slices are independent (issued
// together), the adds follow a fixed order (deterministic).
__device__ __forceinline__ float part_at(const Part& a, int64_t row, int col) {
  const float* p = a.p + row * a.ld + col;
  if (a.ks == 1) return p[0];
  float s = 0.f;
  int z = 0;
  for (; z + 4 <= a.ks; z += 4) {
    const float v0 = p[(int64_t)z * a.zs], v1 = p[(int64_t)(z + 1) * a.zs];
    const float v2 = p[(int64_t)(z + 2) * a.zs], v3 = p[(int64_t)(z + 3) * a.zs];
    s += (v0 + v1) + (v2 + v3);
  }
  for (; z < a.ks; ++z) s += p[(int64_t)z * a.zs];
  return s;
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

// RoPE of one pair (u, v) at position pos with frequency theta ("Multi-Head
// Latent Attention" post, section 3.7: adjacent pairs as complex numbers times
// cos + i sin of pos * theta).  The angle is formed and reduced to [-pi, pi]
// in double precision (positions reach 10^4..10^5 radians), then sin/cos are
// taken in fp32.
__device__ __forceinline__ void rope_pair(float u, float v, int pos, double theta, float* ou,
                                          float* ov) {
  const double ang = (double)pos * theta;
  const double k = rint(ang * 0.15915494309189535);       // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, ang);             // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);                 // 2 pi, low part
  float sf, cf;
  sincosf((float)r, &sf, &cf);
  *ou = u * cf - v * sf;
  *ov = u * sf + v * cf;
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float m = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
  return m;
}

// FP8 storage of one latent row (the "Multi-Head Latent Attention" post lists
// low-precision storage among DeepSeek's ideas and sizes an FP8 cache element
// at one byte, section 3.1): the dc latent values c_j = cval(j) (fp32) become
// OCP E4M3 codes of c_j / s with s = max_j |c_j| / 448 (1 for an all-zero
// row), rounded to nearest-even by the hardware conversion after clamping to
// +-448; the row keeps s as fp32 at byte dc + 2 dr.  Row layout: [codes (dc)
// | rope (dr bf16) | s | zero pad to fp8_row_bytes].  One block of 256
// threads per row; dc even.
template <class CVal>
__device__ __forceinline__ void store_latent_fp8(CVal cval, uint8_t* row, const Dims& d,
                                                 float* red) {
  float amax = 0.f;
  for (int j = 2 * threadIdx.x; j < d.dc; j += 2 * blockDim.x)
    amax = fmaxf(amax, fmaxf(fabsf(cval(j)), fabsf(cval(j + 1))));
  amax = block_max_256(amax, red);
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  for (int j = 2 * threadIdx.x; j < d.dc; j += 2 * blockDim.x) {
    const float q0 = fminf(fmaxf(__fdiv_rn(cval(j), s), -448.f), 448.f);
    const float q1 = fminf(fmaxf(__fdiv_rn(cval(j + 1), s), -448.f), 448.f);
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    *reinterpret_cast<uint16_t*>(row + j) = (uint16_t)(pk & 0xffff);
  }
  if (threadIdx.x == 0) {
    uint8_t* tail = row + d.dc + 2 * d.dr;
    *reinterpret_cast<float*>(tail) = s;
    for (int k = 4; k < fp8_row_bytes(d.dc, d.dr) - d.dc - 2 * d.dr; ++k) tail[k] = 0;
  }
}

// Latent row of token t ("Deepseek V2 Lite Inference Engine in C", MLA notes:
// kv_a_proj gives [latent | rope key]; the latent is RMS-normalised and the key
// rotated; then the row is written to its cache slot).  One block per token.
template <typename T>
__device__ __forceinline__ void append_row_block(const Part& a, int t, int p, int64_t slot,
                                                 const T* __restrict__ gamma,
                                                 T* __restrict__ cache, const Dims& d,
                                                 const RopeTab& rt, float* red) {
  float ss = 0.f;
  for (int j = threadIdx.x; j < d.dc; j += blockDim.x) {
    const float v = part_at(a, t, j);
    ss += v * v;
  }
  const float inv = rsqrtf(block_sum_256(ss, red) / (float)d.dc + d.eps);
  T* row = cache + slot * (int64_t)d.R;
  for (int j = threadIdx.x; j < d.dc; j += blockDim.x)
    stf(row + j, part_at(a, t, j) * inv * (gamma ? ldf(gamma + j) : 1.f));
  for (int i = threadIdx.x; i < d.dr / 2; i += blockDim.x) {
    float ou, ov;
    rope_pair(part_at(a, t, d.dc + 2 * i), part_at(a, t, d.dc + 2 * i + 1), p, rt.theta[i], &ou,
              &ov);
    stf(row + d.dc + 2 * i, ou);
    stf(row + d.dc + 2 * i + 1, ov);
  }
}

// The same row into an FP8 cache (row stride fp8_row_bytes(dc, dr) bytes).
__device__ __forceinline__ void append_row_block_fp8(const Part& a, int t, int p, int64_t slot,
                                                     const bf16* __restrict__ gamma,
                                                     uint8_t* __restrict__ cache, const Dims& d,
                                                     const RopeTab& rt, float* red) {
  float ss = 0.f;
  for (int j = threadIdx.x; j < d.dc; j += blockDim.x) {
    const float v = part_at(a, t, j);
    ss += v * v;
  }
  const float inv = rsqrtf(block_sum_256(ss, red) / (float)d.dc + d.eps);
  uint8_t* row = cache + slot * (int64_t)fp8_row_bytes(d.dc, d.dr);
  store_latent_fp8(
      [&](int j) { return part_at(a, t, j) * inv * (gamma ? ldf(gamma + j) : 1.f); }, row, d, red);
  bf16* rope = reinterpret_cast<bf16*>(row + d.dc);
  for (int i = threadIdx.x; i < d.dr / 2; i += blockDim.x) {
    float ou, ov;
    rope_pair(part_at(a, t, d.dc + 2 * i), part_at(a, t, d.dc + 2 * i + 1), p, rt.theta[i], &ou,
              &ov);
    stf(rope + 2 * i, ou);
    stf(rope + 2 * i + 1, ov);
  }
}

}  // namespace mla
