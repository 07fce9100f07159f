// bf16 MFMA GEMM for the projections: C = A W^T, both operands K-contiguous
// (activations row-major (M, K), weights row-major (N, K) like a linear
// layer), fp32 accumulation.
//
// gfx950 v_mfma_f32_16x16x32_bf16 operand layout (64 lanes):
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + 0..7]
//   B (32 x 16): lane l holds B[8 * (l / 16) + 0..7][l % 16]
//   D (16 x 16): lane l holds D[4 * (l / 16) + 0..3][l % 16]
// so a 16-byte load of 8 consecutive K elements of one row feeds either
// operand straight from global memory.
//
// Decode projections are weight-streaming GEMMs with M = batch <= 64 per
// tile, so their cost is load latency.  Each wave computes a whole 64 x 64
// output tile over its K-slice: per 32-wide k-step it loads 4 weight and 4
// activation fragments (8 x 16 B per lane) and runs 16 MFMAs; loads come in
// groups of two k-steps, double-buffered.  The 4 waves of a block take 4 consecutive
// K-slices and are summed through LDS (64 KB).  K may further be split over
// `ksplit` blocks: each block then writes its fp32 partial tile and the
// consumer of the result sums the ksplit slices in order z = 0..ksplit-1
// (deterministic; no cross-block synchronisation inside the kernel).
#include "kernels.h"

namespace mla {

namespace {
constexpr int kMaxSplit = 16;
constexpr int KSL = 4;  // K-slices (waves) per block
}  // namespace

__global__ void __launch_bounds__(256)
gemm_bf16_tile_k(const bf16* __restrict__ A, int64_t lda, int64_t sA, const bf16* __restrict__ W,
                 int64_t ldw, int64_t sW, int M, int N, int K, int batch, int ksplit,
                 float* __restrict__ part, GemmOut out) {
  __shared__ float red[KSL][4][16][64];  // [K-slice][row block][value][lane]
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int bt = blockIdx.z % batch, z = blockIdx.z / batch;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int n0 = nt * 64, m0 = mt * 64;
  const int wsteps = (K / 32) / (ksplit * KSL);
  const int kbeg = (z * KSL + wave) * wsteps * 32;
  const bf16* Ab = A + bt * sA;
  // rows past M / N read row 0 instead: an MFMA output row (column) depends
  // only on its own A row (W row) and those outputs are never stored, so the
  // loads stay unconditional and straight-line
  const bf16* wrow[4];
  const bf16* arow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + lr;
    wrow[j] = W + bt * sW + (int64_t)(n < N ? n : 0) * ldw + lk;
    const int m = m0 + 16 * j + lr;
    arow[j] = Ab + (int64_t)(m < M ? m : 0) * lda + lk;
  }
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  // two k-steps per load group, double-buffered: the next group's 16 loads
  // are in flight while the current group's 32 MFMAs run
  bf16x8_t wf[2][2][4], af[2][2][4];
  auto load = [&](int buf, int s0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = kbeg + (s0 + (u < wsteps - s0 ? u : 0)) * 32;  // a lone last step reloads
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wf[buf][u][j] = *reinterpret_cast<const bf16x8_t*>(wrow[j] + k);
        af[buf][u][j] = *reinterpret_cast<const bf16x8_t*>(arow[j] + k);
      }
    }
  };
  auto mma = [&](int buf, int nu) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (u < nu)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[buf][u][i], wf[buf][u][j],
                                                                acc[i][j], 0, 0, 0);
  };
  if (wsteps > 0) load(0, 0);
  for (int s0 = 0; s0 < wsteps; s0 += 4) {
    if (s0 + 2 < wsteps) load(1, s0 + 2);
    mma(0, wsteps - s0 >= 2 ? 2 : 1);
    if (s0 + 2 < wsteps) {
      if (s0 + 4 < wsteps) load(0, s0 + 4);
      mma(1, wsteps - s0 - 2 >= 2 ? 2 : 1);
    }
  }
  // every wave writes its tile; wave w then sums row block w over the K-slices
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][i][j * 4 + r][lane] = acc[i][j][r];
  __syncthreads();
  float v[16];  // v[4j + r]: row m0 + 16 wave + 4(l/16) + r, column n0 + 16 j + l%16
#pragma unroll
  for (int q = 0; q < 16; ++q)
    v[q] = red[0][wave][q][lane] + red[1][wave][q][lane] + red[2][wave][q][lane] +
           red[3][wave][q][lane];
  if (ksplit > 1) {
    float* pz = part + (int64_t)(z * batch + bt) * M * N;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * wave + 4 * (lane >> 4) + r, n = n0 + 16 * j + lr;
        if (m < M && n < N) pz[(int64_t)m * N + n] = v[j * 4 + r];
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * wave + 4 * (lane >> 4) + r, n = n0 + 16 * j + lr;
      if (m >= M || n >= N) continue;
      const int64_t o = bt * out.so + (int64_t)m * out.ldo + n;
      if (out.f32)
        out.f32[o] = out.alpha * v[j * 4 + r];
      else
        out.b16[o] = f32_to_bf16(out.alpha * v[j * 4 + r]);
    }
}

#ifndef MLA_NOSPLIT_KB
#define MLA_NOSPLIT_KB 0
#endif

int gemm_bf16_ksplit(int M, int N, int K, int batch, int n_cu) {
  const long tiles = (long)((N + 63) / 64) * ((M + 63) / 64) * batch;
  int ks = 1;
  // a block whose whole weight tile is small streams it faster than a split
  // costs (the split needs a second kernel to sum the partials)
  if ((long)64 * K * 2 <= (long)MLA_NOSPLIT_KB * 1024) return 1;
  // split K over blocks while the grid stays within one block per CU; each
  // wave keeps >= 1 whole k-step
  while (tiles * ks * 2 <= (long)n_cu && (K / 32) % (ks * 2 * KSL) == 0 && ks < kMaxSplit) ks *= 2;
  return ks;
}

void gemm_bf16_mfma(const bf16* A, int64_t lda, int64_t sA, const bf16* W, int64_t ldw,
                    int64_t sW, int M, int N, int K, int batch, int ksplit, float* part,
                    const GemmOut& out, hipStream_t st) {
  dim3 grid((N + 63) / 64, (M + 63) / 64, batch * ksplit);
  gemm_bf16_tile_k<<<grid, 256, 0, st>>>(A, lda, sA, W, ldw, sW, M, N, K, batch, ksplit, part,
                                          out);
}

}  // namespace mla
