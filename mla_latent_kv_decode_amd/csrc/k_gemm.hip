// bf16 MFMA GEMM for the projections: C = A W^T, both operands K-contiguous
// (activations row-major (M, K), weights row-major (N, K) like a linear
// layer), fp32 accumulation, split-K partials written as fp32.
//
// gfx950 v_mfma_f32_16x16x32_bf16 operand layout (64 lanes):
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + 0..7]
//   B (32 x 16): lane l holds B[8 * (l / 16) + 0..7][l % 16]
//   D (16 x 16): lane l holds D[4 * (l / 16) + 0..3][l % 16]
// so a 16-byte load of 8 consecutive K elements of one row feeds either
// operand directly: no LDS is needed for the small-M (decode) shapes.
#include "kernels.h"

namespace mla {

// Block: 4 waves.  Block tile 64 (M) x 64 (N); wave w owns the 16 columns
// [16w, 16w + 16) for all 64 rows (4 accumulators).  Every wave streams its own
// weight rows once; the activation fragments are shared through L1/L2.
__global__ void __launch_bounds__(256)
gemm_bf16_mfma_k(const bf16* __restrict__ A, int64_t lda, int64_t sA, const bf16* __restrict__ W,
                 int64_t ldw, int64_t sW, float* __restrict__ C, int M, int N, int K, int batch,
                 int kchunk) {
  const int bt = blockIdx.z % batch, z = blockIdx.z / batch;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 64 + wave * 16;
  if (n0 >= N) return;
  const int m0 = blockIdx.y * 64;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const bf16* Ab = A + bt * sA;
  const bf16* Wrow = W + bt * sW + (int64_t)(n0 + lr) * ldw + lk;
  const bf16* Arow[4];
  bool aval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 16 * i + lr;
    aval[i] = m < M;
    Arow[i] = Ab + (int64_t)(aval[i] ? m : 0) * lda + lk;
  }
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int kb = z * kchunk, ke = kb + kchunk;
  const bf16x8_t zero8 = (bf16x8_t){};
#pragma unroll 4
  for (int k = kb; k < ke; k += 32) {
    const bf16x8_t wf = *reinterpret_cast<const bf16x8_t*>(Wrow + k);
    bf16x8_t af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = aval[i] ? *reinterpret_cast<const bf16x8_t*>(Arow[i] + k) : zero8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], wf, acc[i], 0, 0, 0);
  }
  float* Cb = C + (int64_t)(z * batch + bt) * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * i + (lane >> 4) * 4 + r;
      if (m < M) Cb[(int64_t)m * N + n0 + lr] = acc[i][r];
    }
  }
}

void gemm_bf16_mfma(const bf16* A, int64_t lda, int64_t sA, const bf16* W, int64_t ldw,
                    int64_t sW, float* C, int M, int N, int K, int batch, int ksplit,
                    hipStream_t st) {
  const int kchunk = K / ksplit;
  dim3 grid((N + 63) / 64, (M + 63) / 64, batch * ksplit);
  gemm_bf16_mfma_k<<<grid, 256, 0, st>>>(A, lda, sA, W, ldw, sW, C, M, N, K, batch, kchunk);
}

}  // namespace mla
