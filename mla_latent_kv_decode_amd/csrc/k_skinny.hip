// The decode step's weight-streaming GEMMs (M = query rows <= 128) with their
// epilogues applied in place, the split-K variant with LDS-resident
// activations for at most 32 rows against large weights (gemm_res_k, below),
// and the kernel that finishes the projections (latent-row append, query
// RMSNorm, absorbed query).
//
// C (M x N) = A (M x K) W^T with A row-major activations and W a row-major
// (N, K) weight (a linear layer), bf16 in, fp32 accumulation, on
// v_mfma_f32_16x16x32_bf16:
//   A (16 x 32): lane l holds A[l % 16][8 (l / 16) .. + 7]
//   B (32 x 16): lane l holds B[8 (l / 16) .. + 7][l % 16]
//   D (16 x 16): lane l holds D[4 (l / 16) .. + 3][l % 16]
// A block computes a 16 (32, 64) x 32 tile over all of K, streaming 256-wide
// K chunks of its 32 weight rows and 16 (32, 64) activation rows into a
// 3-stage LDS ring with global_load_lds_dwordx4 (each copy is 1 KB: two
// 512-byte row pieces, so the weights are read in long contiguous runs and
// the copies hold no registers), two chunks in flight (16-row tiles: two
// blocks per compute unit).  Eight waves issue the copies: L2-to-LDS copy
// throughput per compute unit grows with the waves issuing them (measured
// ~46 GB/s with 4 waves, ~62 with 8, on L2-resident data).  Inside a row
// piece the 16-byte chunk c of row r is stored at c ^ (r % 16): the operand
// reads (16 lanes = 16 rows at one K offset) then hit distinct banks.  Wave w
// takes k-step w of every chunk; the eight waves' sums are added through LDS
// in wave order (deterministic).  Nothing is split over blocks, so the epilogue sees final
// sums and is applied right there, on adjacent column pairs: a bf16 store, an
// fp32 store, or the query finish (per head: the nope part stored, the rope
// part rotated and scaled into q_cat).  The 16-row blocks of a column tile are
// numbered 8 apart, so they run on one XCD and share its L2 for the weights.
#include <algorithm>
#include <atomic>

#include "decode_dev.h"
#include "row_dev.h"

namespace mla {
namespace skn {

using ddev::dma16;
using ddev::dma16_nt;
using ddev::lds_u32;
using ddev::wait_vmcnt;

constexpr int NWV = 4;                    // waves of the split-K products
constexpr int SWV = 8;                    // waves of the column-tile stream products
constexpr int NT = 32;                    // output columns per block
constexpr int KC = 256;                   // K per chunk
constexpr int ROWB = KC * 2;              // 512 bytes per row piece
constexpr int W_OFF = 0, A_OFF = NT * ROWB;
constexpr int NST = 3;                    // stages
constexpr int kXcds = 8;
constexpr int kMaxStreamRows = 128;  // rows (query rows of a step) the stream GEMMs take
// MR activation rows per block (16: 24 KB stages, two blocks per compute
// unit; 32: 32 KB stages, 64: 48 KB stages, one block).  A block copies
// (NT + MR) rows over all of K, so the copy volume of a launch is
// (N / NT) (M / MR) (NT + MR) K 2
// bytes: taller tiles re-read the weights fewer times.
template <int MR>
struct Tile {
  static constexpr int ST_BYTES = (NT + MR) * ROWB;
  static constexpr int NCOPY = (NT + MR) / 2;  // one-KB copies per chunk
  static constexpr int CPW = NCOPY / SWV;
  static_assert(NCOPY % SWV == 0, "copies split evenly over the waves");
  static_assert((NST - 2) * CPW <= 63, "copies in flight fit the vmcnt field");
};

// copy i of chunk k0 (rows 2i, 2i + 1 of the stage: weight rows first, then
// activation rows), lanes 0-31 on the first row, 32-63 on the second
__device__ __forceinline__ void chunk_copy(int i, const bf16* W, int64_t ldw, int n0, int N,
                                           const bf16* A, int64_t lda, int m0, int M, int k0,
                                           uint32_t stage, int lane) {
  const int r = 2 * i + (lane >> 5);
  const int c = (lane & 31) ^ (r & 15);  // source chunk stored at position lane & 31
  const bf16* src = r < NT ? W + (int64_t)min(n0 + r, N - 1) * ldw
                           : A + (int64_t)min(m0 + r - NT, M - 1) * lda;
  dma16(src + k0 + 8 * c, stage + (uint32_t)i * 1024);
}

// The extra blocks of a launch that carries a HostCopy: block `blk` of them
// (NTH threads) copies words blk * NTH + threadIdx.x, then every
// (blocks * NTH)-th, four loads in flight per thread.
template <int NTH>
__device__ __forceinline__ void host_copy(const HostCopy& hc, int blk) {
  const uint4* src = static_cast<const uint4*>(hc.src);
  uint4* dst = static_cast<uint4*>(hc.dst);
  const int stride = hc.blocks * NTH;
  for (int i0 = blk * NTH + (int)threadIdx.x; i0 < hc.n16; i0 += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * stride < hc.n16) v[u] = src[i0 + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * stride < hc.n16) dst[i0 + u * stride] = v[u];
  }
}

template <int MR, class Epi>
__global__ void __launch_bounds__(SWV * 64)
gemm_stream_k(const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ W, int64_t ldw,
              int M, int N, int K, int mtiles, Epi epi, HostCopy hc) {
  constexpr int ST_BYTES = Tile<MR>::ST_BYTES, CPW = Tile<MR>::CPW, NMB = MR / 16;
  __shared__ __attribute__((aligned(1024))) char lds[NST * ST_BYTES];
  // block -> (column tile, row tile); the row tiles of a column tile share an XCD
  const int bid = blockIdx.x;
  if (hc.n16 > 0 && bid >= hc.first_block) {
    host_copy<SWV * 64>(hc, bid - hc.first_block);
    return;
  }
  const int mt = (bid / kXcds) % mtiles;
  const int ntile = (bid / (kXcds * mtiles)) * kXcds + bid % kXcds;
  const int n0 = ntile * NT, m0 = MR * mt;
  if (n0 >= N) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const uint32_t lds0 = lds_u32(lds);
  const int nchunk = K / KC;
  auto issue = [&](int ch) {
    const uint32_t stage = lds0 + (uint32_t)(ch % NST) * ST_BYTES;
#pragma unroll
    for (int j = 0; j < CPW; ++j)
      chunk_copy(wave * CPW + j, W, ldw, n0, N, A, lda, m0, M, ch * KC, stage, lane);
  };
#pragma unroll 1
  for (int ch = 0; ch < NST - 1 && ch < nchunk; ++ch) issue(ch);

  f32x4_t acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  static_assert(NST == 3, "the waits below assume at most one chunk issued after the awaited one");
#pragma unroll 1
  for (int ch = 0; ch < nchunk; ++ch) {
    if (ch + 1 < nchunk) wait_vmcnt<CPW>();
    else wait_vmcnt<0>();
    __syncthreads();  // chunk ch is in LDS; every wave is done with chunk ch - 1
    if (ch + NST - 1 < nchunk) issue(ch + NST - 1);
    const char* st = lds + (ch % NST) * ST_BYTES;
#pragma unroll
    for (int u = 0; u < KC / 32 / SWV; ++u) {
      const int c = 4 * (wave + SWV * u) + lg;  // 16-byte chunk of this lane's operands
      bf16x8_t af[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8_t*>(st + A_OFF + (16 * mb + lr) * ROWB +
                                                    16 * (c ^ lr));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bf16x8_t wf = *reinterpret_cast<const bf16x8_t*>(
            st + W_OFF + (16 * nb + lr) * ROWB + 16 * (c ^ lr));
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], wf, acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // sum the waves' tiles: red[w][row][col]
  static_assert(SWV * MR * NT * 4 <= NST * ST_BYTES, "the wave sums fit in the ring");
  __syncthreads();  // the ring is free
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * MR + 16 * mb + 4 * lg + i) * NT + 16 * nb + lr] = acc[mb][nb][i];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < (MR * 16 + SWV * 64 - 1) / (SWV * 64); ++e) {
    const int t = threadIdx.x + SWV * 64 * e;  // row t / 16, columns 2 (t % 16), + 1
    if (t >= MR * 16) break;
    const int row = t >> 4, col = 2 * (t & 15);
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int w = 0; w < SWV; ++w) {
      const float2 p = *reinterpret_cast<const float2*>(red + (w * MR + row) * NT + col);
      v0 += p.x;
      v1 += p.y;
    }
    if (m0 + row < M && n0 + col < N) epi(m0 + row, n0 + col, v0, v1);
  }
}

// epilogues on the column pair (c, c + 1) of row r (c even; c + 1 < N)
struct EpiStore {
  bf16* out;
  int64_t ldo;
  float alpha;
  __device__ void operator()(int r, int c, float v0, float v1) const {
    *reinterpret_cast<uint32_t*>(out + (int64_t)r * ldo + c) = pack_bf16x2(alpha * v0, alpha * v1);
  }
};

struct EpiF32 {
  float* out;
  int64_t ldo;
  __device__ void operator()(int r, int c, float v0, float v1) const {
    *reinterpret_cast<float2*>(out + (int64_t)r * ldo + c) = make_float2(v0, v1);
  }
};

// Columns [0, R) go to `a` (fp32, row stride R); the rest are query heads of
// dn + dr columns: the first dn to q_nope (T, H, dn) or, with q_nope null
// (materialised absorption: these columns already are W^KQ_h x, dn = dc),
// scaled into q_cat[t][h][0 .. dc); the rope part rotated at the row's
// position ("Multi-Head Latent Attention" post, section 3.7: RoPE per head on
// the decoupled query part) and scaled into q_cat[t][h][dc + i].
struct EpiQuery {
  float* a;
  int R;
  bf16* q_nope;
  bf16* q_cat;
  int H, dn, dr, dc;
  float scale;
  RopeTab rt;
  int32_t pos[kMaxStreamRows];  // positions of the rows, passed by value
  __device__ void operator()(int r, int c, float v0, float v1) const {
    if (c < R) {
      *reinterpret_cast<float2*>(a + (int64_t)r * R + c) = make_float2(v0, v1);
      return;
    }
    const int cc = c - R, w = dn + dr, h = cc / w, j = cc - h * w;
    if (j < dn) {
      if (q_nope)
        *reinterpret_cast<uint32_t*>(q_nope + ((int64_t)r * H + h) * dn + j) = pack_bf16x2(v0, v1);
      else
        *reinterpret_cast<uint32_t*>(q_cat + ((int64_t)r * H + h) * (dc + dr) + j) =
            pack_bf16x2(scale * v0, scale * v1);
      return;
    }
    const int i = j - dn;
    float ou, ov;
    rope_pair(v0, v1, pos[r], rt.theta[i >> 1], &ou, &ov);
    *reinterpret_cast<uint32_t*>(q_cat + ((int64_t)r * H + h) * (dc + dr) + dc + i) =
        pack_bf16x2(scale * ou, scale * ov);
  }
};

}  // namespace skn

// compute units of the current device, looked up once per device
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool slot = dev >= 0 && dev < 64;
  int n = slot ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  if (slot) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace skn {

// ---- few rows (M <= 32) against large weights: split-K with the activation
// slice resident in LDS.  The 32-column tiles above re-copy all M x K
// activations per tile, as many bytes as their weights when M = 32 (V3's W_o:
// 235 MB of weights, 470 MB of copies).  Here block (slice s, column group g)
// copies the activations of K slice s once (32 rows x 1024 k = 64 KB, in MFMA
// fragment order) and each wave streams the fragment-tiled weight blocks of
// its share (R 16-row blocks; a block's fragments of one slice are 32
// contiguous KB) through a 3-stage ring of its own in LDS, two batches of
// 2 R one-KB fragments in flight while one multiplies: each k-step's two
// activation fragments feed 2 R MFMAs.  All copies are LDS-DMA with explicit
// waits; the weights are read non-temporally (once), so each weight byte
// crosses HBM -> CU once.  With one slice the epilogue is applied in place;
// with more, fp32 partials go to `part` (slice s at s M N) and res_reduce_k
// sums them in slice order (deterministic).  The product is taken transposed
// (D = W_frag . A_frag^T), so a lane ends with four adjacent columns of one
// activation row.
constexpr int RS_MT = 2;      // 16-row activation blocks (M <= 32)
constexpr int RS_KS = 1024;   // largest k per slice
constexpr int RS_KB = 2;      // k-steps per batch
constexpr int RS_NST = 3;     // ring stages per wave
constexpr int RS_RMAX = 4;    // weight blocks per wave at most
constexpr int RS_A_BYTES = RS_MT * (RS_KS / 32) * 1024;              // 64 KB
constexpr int RS_WST = RS_RMAX * RS_KB * 1024;                       // 8 KB per stage
constexpr int RS_LDS = RS_A_BYTES + NWV * RS_NST * RS_WST;           // 160 KB

template <int R, class Epi>
__global__ void __launch_bounds__(256)
gemm_res_k(const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ Wt, int M, int N,
           int K, int KS, int nslice, float* __restrict__ part, Epi epi, HostCopy hc) {
  static_assert(R <= RS_RMAX, "ring stages hold RS_RMAX weight blocks");
  constexpr int CPB = R * RS_KB;  // copies per batch and wave
  __shared__ __attribute__((aligned(1024))) char lds[RS_LDS];
  const int bid = blockIdx.x;
  if (hc.n16 > 0 && bid >= hc.first_block) {
    host_copy<NWV * 64>(hc, bid - hc.first_block);
    return;
  }
  const int s = bid % nslice, g = bid / nslice;  // slice s on XCD s % 8
  const int k0 = s * KS, nks = K / 32, sks = min(KS, K - k0) / 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t lds0 = lds_u32(lds);
  // the slice's activations: fragment (ks, m) at (ks RS_MT + m) KB, lane l
  // holding row 16 m + l % 16 (rows past M repeat the last), k = 8 (l / 16)
  for (int f = wave; f < sks * RS_MT; f += NWV) {
    const int ks = f / RS_MT, m = f % RS_MT;
    const int row = min(16 * m + (lane & 15), M - 1);
    dma16(A + (int64_t)row * lda + k0 + 32 * ks + 8 * (lane >> 4), lds0 + (uint32_t)f * 1024);
  }
  // this wave's weight blocks rb0 + 4 r (past the last one the copies repeat
  // it and nothing is stored), batch b = k-steps 2 b, 2 b + 1 of the slice
  const int NB = (N + 15) / 16;
  const int rb0 = g * NWV * R + wave;
  const char* wsrc[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wsrc[r] = reinterpret_cast<const char*>(Wt) +
              ((int64_t)min(rb0 + NWV * r, NB - 1) * nks + k0 / 32) * 1024 + lane * 16;
  const uint32_t ring = lds0 + RS_A_BYTES + (uint32_t)wave * RS_NST * RS_WST;
  auto issue = [&](int b) {
    const uint32_t st = ring + (uint32_t)(b % RS_NST) * RS_WST;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < RS_KB; ++j)
        dma16_nt(wsrc[r] + (int64_t)(RS_KB * b + j) * 1024, st + (uint32_t)(r * RS_KB + j) * 1024);
  };
  const int nb = sks / RS_KB;  // batches per slice (>= 2: K % 256 == 0)
  issue(0);
  issue(1);
  wait_vmcnt<2 * CPB>();  // this wave's activation copies (issued first) are done
  __syncthreads();        // every wave's activation copies are visible
  f32x4_t acc[R][RS_MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < RS_MT; ++m) acc[r][m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const char* al = lds + lane * 16;
  const char* wl = lds + RS_A_BYTES + wave * RS_NST * RS_WST + lane * 16;
  for (int b = 0; b < nb; ++b) {
    // the stage of batch b + 2 held batch b - 1, whose reads ended before
    // the products of the previous iteration
    if (b + 2 < nb) issue(b + 2);
    const int later = min(2, nb - 1 - b);  // batches issued after b
    if (later == 2) wait_vmcnt<2 * CPB>();
    else if (later == 1) wait_vmcnt<CPB>();
    else wait_vmcnt<0>();
    const char* st = wl + (b % RS_NST) * RS_WST;
#pragma unroll
    for (int j = 0; j < RS_KB; ++j) {
      const int ks = RS_KB * b + j;
      bf16x8_t a[RS_MT], w[R];
#pragma unroll
      for (int m = 0; m < RS_MT; ++m)
        a[m] = *reinterpret_cast<const bf16x8_t*>(al + (ks * RS_MT + m) * 1024);
#pragma unroll
      for (int r = 0; r < R; ++r)
        w[r] = *reinterpret_cast<const bf16x8_t*>(st + (r * RS_KB + j) * 1024);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < RS_MT; ++m)
          acc[r][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[r], a[m], acc[r][m], 0, 0, 0);
    }
  }
  // lane: C[row = 16 m + l % 16][col = 16 rb + 4 (l / 16) .. + 3]
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (rb0 + NWV * r >= NB) continue;
    const int col = 16 * (rb0 + NWV * r) + 4 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < RS_MT; ++m) {
      const int row = 16 * m + (lane & 15);
      if (row >= M || col >= N) continue;
      if (nslice == 1) {
        epi(row, col, acc[r][m][0], acc[r][m][1]);
        if (col + 2 < N) epi(row, col + 2, acc[r][m][2], acc[r][m][3]);
      } else {
        float* dst = part + ((int64_t)s * M + row) * N + col;
        if (col + 3 < N) {
          *reinterpret_cast<float4*>(dst) =
              make_float4(acc[r][m][0], acc[r][m][1], acc[r][m][2], acc[r][m][3]);
        } else {
          dst[0] = acc[r][m][0];
          dst[1] = acc[r][m][1];
          if (col + 2 < N) {
            dst[2] = acc[r][m][2];
            dst[3] = acc[r][m][3];
          }
        }
      }
    }
  }
}

// The partials of gemm_res_k summed, then the epilogue.  A block covers one
// row and 4 (256 / G) columns: each of G thread groups sums every G-th slice
// (four adjacent columns per thread, all its loads independent), then the G
// group sums are added in group order, so the result does not depend on
// timing.
template <int G, class Epi>
__global__ void __launch_bounds__(256)
res_reduce_k(const float* __restrict__ part, int nslice, int M, int N, Epi epi) {
  constexpr int QN = 256 / G;  // column quads per block
  __shared__ float4 red[256];
  const int g = threadIdx.x / QN, q = threadIdx.x % QN;
  const int row = blockIdx.y, col = 4 * (blockIdx.x * QN + q);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col < N) {
    const int64_t step = (int64_t)G * M * N;
    const float* p = part + ((int64_t)g * M + row) * N + col;
#pragma unroll 4
    for (int s = g; s < nslice; s += G, p += step) {
      const float4 x = *reinterpret_cast<const float4*>(p);
      v.x += x.x;
      v.y += x.y;
      v.z += x.z;
      v.w += x.w;
    }
  }
  red[threadIdx.x] = v;
  __syncthreads();
  if (g != 0 || col >= N) return;
#pragma unroll
  for (int i = 1; i < G; ++i) {
    const float4 x = red[i * QN + q];
    v.x += x.x;
    v.y += x.y;
    v.z += x.z;
    v.w += x.w;
  }
  epi(row, col, v.x, v.y);
  epi(row, col + 2, v.z, v.w);
}

template <int G, class Epi>
void launch_reduce(const float* part, int nslice, int M, int N, const Epi& epi, hipStream_t st) {
  constexpr int QN = 256 / G;
  res_reduce_k<G, Epi><<<dim3((N / 4 + QN - 1) / QN, M), 256, 0, st>>>(part, nslice, M, N, epi);
}

// The split: whole K in one slice with the most weight blocks per wave that
// still give three quarters of the compute units a block; else the largest
// slice that does, with four, two, then one weight block per wave.
struct ResPlan {
  int R = 0, KS = 0, nslice = 0, blocks = 0;
};
inline ResPlan res_plan(int M, int N, int K, int ncu) {
  ResPlan p;
  const int NB = (N + 15) / 16;
  auto fits = [&](int R, int KS) {
    const int ns = (K + KS - 1) / KS, groups = (NB + NWV * R - 1) / (NWV * R);
    if (ns * groups * 4 < ncu * 3) return false;
    p.R = R;
    p.KS = KS;
    p.nslice = ns;
    p.blocks = ns * groups;
    return true;
  };
  if (K <= RS_KS)
    for (int R : {4, 2, 1})
      if (fits(R, K)) return p;
  for (int R : {4, 2, 1})
    for (int KS : {RS_KS, RS_KS / 2, RS_KS / 4})
      if (KS < K && fits(R, KS)) return p;
  // nothing fills the chip: one weight block per wave, the smallest slices
  p.R = 1;
  p.KS = std::min(K, RS_KS / 4);
  p.nslice = (K + p.KS - 1) / p.KS;
  p.blocks = p.nslice * ((NB + NWV - 1) / NWV);
  return p;
}

template <class Epi>
void launch_res(const bf16* A, int64_t lda, const bf16* Wt, int M, int N, int K, float* part,
                const Epi& epi, hipStream_t st, HostCopy hc) {
  const ResPlan p = res_plan(M, N, K, device_cu_count());
  hc.first_block = p.blocks;
  const int grid = p.blocks + (hc.n16 > 0 ? hc.blocks : 0);
  if (p.R == 4)
    gemm_res_k<4, Epi><<<grid, NWV * 64, 0, st>>>(A, lda, Wt, M, N, K, p.KS, p.nslice, part, epi, hc);
  else if (p.R == 2)
    gemm_res_k<2, Epi><<<grid, NWV * 64, 0, st>>>(A, lda, Wt, M, N, K, p.KS, p.nslice, part, epi, hc);
  else
    gemm_res_k<1, Epi><<<grid, NWV * 64, 0, st>>>(A, lda, Wt, M, N, K, p.KS, p.nslice, part, epi, hc);
  if (p.nslice > 4)
    launch_reduce<8>(part, p.nslice, M, N, epi, st);
  else if (p.nslice > 2)
    launch_reduce<4>(part, p.nslice, M, N, epi, st);
  else if (p.nslice == 2)
    launch_reduce<2>(part, p.nslice, M, N, epi, st);
}

// The tallest row blocks (64 or 32 rows: one block per compute unit; 16 rows:
// two) whose grid still occupies three quarters of the compute units: taller
// blocks re-read the weights fewer times.
template <class Epi>
void launch_stream(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K,
                   const Epi& epi, hipStream_t st, HostCopy hc = HostCopy{}) {
  const int ntiles = (N + NT - 1) / NT;
  const int nt8 = (ntiles + kXcds - 1) / kXcds * kXcds;
  const int m64 = (M + 63) / 64, m32 = (M + 31) / 32;
  if (M > 32 && ntiles * m64 * 4 >= device_cu_count() * 3) {
    hc.first_block = nt8 * m64;
    gemm_stream_k<64, Epi><<<nt8 * m64 + (hc.n16 > 0 ? hc.blocks : 0), SWV * 64, 0, st>>>(
        A, lda, W, ldw, M, N, K, m64, epi, hc);
    return;
  }
  if (M > 16 && ntiles * m32 * 4 >= device_cu_count() * 3) {
    hc.first_block = nt8 * m32;
    gemm_stream_k<32, Epi><<<nt8 * m32 + (hc.n16 > 0 ? hc.blocks : 0), SWV * 64, 0, st>>>(
        A, lda, W, ldw, M, N, K, m32, epi, hc);
    return;
  }
  const int mtiles = (M + 15) / 16;
  hc.first_block = nt8 * mtiles;
  gemm_stream_k<16, Epi><<<nt8 * mtiles + (hc.n16 > 0 ? hc.blocks : 0), SWV * 64, 0, st>>>(
      A, lda, W, ldw, M, N, K, mtiles, epi, hc);
}

// ---- projection finish: blocks [0, nab) absorbed query tiles, then nap
// latent-row appends, then nqn query RMSNorm rows.
//
// Absorbed query ("Multi-Head Latent Attention" post, section 3.3): for head h
// q_cat[t][h][c] = scale * sum_k q_nope[t][h][k] W_ukT[h][c][k] (c < 512,
// K = dn), one block per (32-row group, head, 128 columns), wave w on 32 of
// them.  (Groups of 64 rows took ~7 us at 64 query rows, 32 ~5 us: twice the
// blocks and half the loads per wave before the first product.)
template <int MT>
__global__ void __launch_bounds__(256)
finish_k(const bf16* __restrict__ q_nope, const bf16* __restrict__ w_ukT,
         bf16* __restrict__ q_cat, int B, int nab, int nap, const float* __restrict__ a, int lda,
         int qa_col, const int32_t* __restrict__ pos, const int64_t* __restrict__ slot,
         const bf16* __restrict__ kv_gamma, void* __restrict__ cache, const bf16* q_gamma,
         bf16* __restrict__ cq, Dims d, RopeTab rt, int kv8) {
  __shared__ float red[4];
  const int blk = blockIdx.x;
  if (blk >= nab + nap) {  // RMSNorm of the query down-projection row
    const int t = blk - nab - nap;
    const float* x = a + (int64_t)t * lda + qa_col;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d.dq; j += blockDim.x) ss += x[j] * x[j];
    const float inv = rsqrtf(block_sum_256(ss, red) / (float)d.dq + d.eps);
    for (int j = threadIdx.x; j < d.dq; j += blockDim.x)
      cq[(int64_t)t * d.dq + j] = f32_to_bf16(x[j] * inv * bf16_to_f32(q_gamma[j]));
    return;
  }
  if (blk >= nab) {  // latent row of token t
    const int t = blk - nab;
    Part p;
    p.p = a;
    p.ks = 1;
    p.ld = lda;
    p.zs = 0;
    if (kv8)
      append_row_block_fp8(p, t, pos[t], slot[t], kv_gamma, static_cast<uint8_t*>(cache), d, rt,
                           red);
    else
      append_row_block<bf16>(p, t, pos[t], slot[t], kv_gamma, static_cast<bf16*>(cache), d, rt,
                             red);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // block = (32-row group, head, 128 columns)
  static_assert(MT <= 2, "32-row groups");
  const int r0 = 32 * (blk / (d.H * 4)), hb = blk % (d.H * 4);
  const int h = hb >> 2, c0 = (hb & 3) * 128 + 32 * wave;
  const int nks = d.dn / 32;
  f32x4_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mt][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const bf16* wb = w_ukT + ((int64_t)h * d.dc + c0 + lr) * d.dn + 8 * lg;
  // four k-steps per round, all their loads issued before the MFMAs
  for (int ks0 = 0; ks0 < nks; ks0 += 4) {
    bf16x8_t fa[4][MT], fw[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ks = min(ks0 + u, nks - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        fa[u][mt] = *reinterpret_cast<const bf16x8_t*>(
            q_nope + ((int64_t)min(r0 + 16 * mt + lr, B - 1) * d.H + h) * d.dn + 32 * ks + 8 * lg);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        fw[u][nb] = *reinterpret_cast<const bf16x8_t*>(wb + (int64_t)16 * nb * d.dn + 32 * ks);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ks0 + u < nks)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mt][nb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[u][mt], fw[u][nb], acc[mt][nb], 0, 0, 0);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = r0 + 16 * mt + 4 * lg + i;
        if (t < B)
          q_cat[((int64_t)t * d.H + h) * d.R + c0 + 16 * nb + lr] = f32_to_bf16(d.scale * acc[mt][nb][i]);
      }
}

}  // namespace skn

bool skinny_ok(int M, int N, int K) {
  return M >= 1 && M <= skn::kMaxStreamRows && N >= 2 && N % 2 == 0 && K % skn::KC == 0;
}

int res_slices(int M, int N, int K) {
  if (M < 1 || M > 16 * skn::RS_MT || K % (64 * skn::RS_KB) != 0 || N % 4 != 0) return 0;
  // weights under 80 MiB: the column tiles (eight-wave stream products), whose
  // re-copied activations cost less than the split-K reduction's launch (V3
  // in-projection, [W_kva; W_qa] 30 MB at 32 rows: step 239-243 -> 234-235
  // us; V3 q_b, 75 MB: B = 1 step 135 -> 127 us, B = 32 unchanged); above
  // (V3 W_o, 235 MB) the resident-activation split-K wins
  if ((size_t)N * K * 2 < (size_t(80) << 20)) return 0;
  return skn::res_plan(M, N, K, device_cu_count()).nslice;
}

// the resident-activation path applies (and has its partial buffer if it splits K)
static bool use_res(const StreamRes& r, int M, int N, int K) {
  const int ns = r.wt ? res_slices(M, N, K) : 0;
  return ns == 1 || (ns > 1 && r.part);
}

void skinny_store(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K,
                  bf16* out, int64_t ldo, float alpha, hipStream_t st, const StreamRes& r) {
  if (use_res(r, M, N, K))
    skn::launch_res(A, lda, r.wt, M, N, K, r.part, skn::EpiStore{out, ldo, alpha}, st, HostCopy{});
  else
    skn::launch_stream(A, lda, W, ldw, M, N, K, skn::EpiStore{out, ldo, alpha}, st);
}

void skinny_f32(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K,
                float* out, int64_t ldo, hipStream_t st, const HostCopy& hc, const StreamRes& r) {
  if (use_res(r, M, N, K))
    skn::launch_res(A, lda, r.wt, M, N, K, r.part, skn::EpiF32{out, ldo}, st, hc);
  else
    skn::launch_stream(A, lda, W, ldw, M, N, K, skn::EpiF32{out, ldo}, st, hc);
}

int host_copy_blocks(int n16) { return std::min(16, std::max(1, (n16 + 1023) / 1024)); }

void skinny_query(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K,
                  float* a, int R, bf16* q_nope, bf16* q_cat, const int32_t* pos_host,
                  const Dims& d, const RopeTab& rt, hipStream_t st, const HostCopy& hc,
                  const StreamRes& r) {
  skn::EpiQuery e;
  e.a = a;
  e.R = R;
  e.q_nope = q_nope;
  e.q_cat = q_cat;
  for (int i = 0; i < skn::kMaxStreamRows; ++i) e.pos[i] = i < M ? pos_host[i] : 0;
  e.H = d.H;
  e.dn = q_nope ? d.dn : d.dc;
  e.dr = d.dr;
  e.dc = d.dc;
  e.scale = d.scale;
  e.rt = rt;
  if (use_res(r, M, N, K))
    skn::launch_res(A, lda, r.wt, M, N, K, r.part, e, st, hc);
  else
    skn::launch_stream(A, lda, W, ldw, M, N, K, e, st, hc);
}

void decode_finish(const bf16* q_nope, const bf16* w_ukT, bf16* q_cat, int B, bool absorb,
                   bool append, bool qnorm, const float* a, int lda, int qa_col, const int32_t* pos,
                   const int64_t* slot, const bf16* kv_gamma, void* cache, const bf16* q_gamma,
                   bf16* cq, const Dims& d, const RopeTab& rt, hipStream_t st, bool kv8) {
  // the absorbed query in groups of up to 32 rows
  const int nab = absorb ? d.H * 4 * ((B + 31) / 32) : 0, nap = append ? B : 0,
            nqn = qnorm ? B : 0;
  const int blocks = nab + nap + nqn;
  if (blocks == 0) return;
#define MLA_FIN(MT)                                                                          \
  skn::finish_k<MT><<<blocks, 256, 0, st>>>(q_nope, w_ukT, q_cat, B, nab, nap, a, lda, qa_col, pos, \
                                            slot, kv_gamma, cache, q_gamma, cq, d, rt, kv8 ? 1 : 0)
  if (B <= 16) MLA_FIN(1);
  else MLA_FIN(2);
#undef MLA_FIN
}

}  // namespace mla
