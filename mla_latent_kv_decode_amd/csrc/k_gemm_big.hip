// Large-tile bf16 MFMA GEMM for projections with many rows (prefill, bulk
// appends): C = alpha A W^T with A (M, K) and W (N, K), fp32 accumulation, C
// stored as bf16 or fp32 with its own row stride.  These are the
// compute-bound, GEMM-shaped steps of prefill ("Transformer and KV Cache
// Basics", KV Cache -- Conceptually).
//
// Operand layout ("fragment-tiled"): both operands are stored as a list of
// 1 KB fragments, fragment (b, s) = rows 16 b .. 16 b + 15, k = 32 s .. 32 s
// + 31 at byte (b * K / 32 + s) * 1024, in the lane order of a
// v_mfma_f32_16x16x32_bf16 operand (lane l holds row l % 16, k = 8 (l / 16)
// .. + 7, 16 bytes at l * 16).  A row block's fragments follow each other in
// k, so a tile's operand stream is a sequential read of 1 KB blocks: against
// the same GEMM reading row-major rows (16 rows x 64 bytes per copy) the copy
// stream alone runs twice as fast (measured) and the GEMM ~20-35 % faster.
// Weights are tiled once when they are absorbed; activations by tile_rows
// just before the product (one extra pass over A).
//
// Block = 512 threads (8 waves, two per SIMD, so one wave's fragment reads
// overlap the other's products) computing a 256 x BN tile of C (BN = 256 or
// 128); wave (wm, wn) owns rows 128 wm .. +127 and columns (BN / 4) wn .. +
// BN / 4 - 1.  K advances in steps of 32 through a 4-stage LDS ring filled by
// global_load_lds_dwordx4 (three steps in flight; one barrier per step both
// publishes a stage and frees the one the next copy overwrites).  A copy
// instruction moves one fragment (lane l fetches the 16 bytes it deposits at
// l * 16) and an operand read is one contiguous 1 KB ds_read per wave, so
// neither side has bank conflicts.
//
// The product is taken transposed, D = W_frag . A_frag^T (C^T tile), so lane
// l ends with C[m = l % 16][n = 4 (l / 16) .. + 3]: four adjacent columns of
// one row, stored as one 8-byte (bf16) or 16-byte (fp32) write.
//
// Tiles are numbered so that the blocks the hardware sends to one XCD (block
// b runs on XCD b % 8) take a contiguous range of tiles, walked in groups of
// 8 row tiles, so blocks running together on one XCD share A rows and W rows
// in that XCD's L2.
#include <algorithm>

#include "kernels.h"

namespace mla {
namespace bg {

constexpr int BM = 256;     // rows of A per tile
constexpr int BK = 32;      // k per stage
constexpr int NST = 4;      // LDS stages
constexpr int NWAVE = 8;
constexpr int GROUP_M = 8;  // row tiles walked together
constexpr int kXcds = 8;

template <int BN>
struct Cfg {
  static constexpr int WN = BN / 4;           // columns per wave
  static constexpr int NJ = WN / 16;          // 16-column blocks per wave
  static constexpr int NI = 8;                // 16-row blocks per wave (128 rows)
  static constexpr int A_FR = BM / 16;        // A fragments per stage
  static constexpr int W_FR = BN / 16;        // W fragments per stage
  static constexpr int FR = A_FR + W_FR;      // copy instructions per stage
  static constexpr int PER_WAVE = FR / NWAVE; // ... per wave
  static constexpr int ST = FR * 1024;        // bytes per stage
  static_assert(FR % NWAVE == 0, "copies split evenly over the waves");
};

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Tile (tm, tn) of linear block b: XCD x = b % 8 takes the contiguous tile
// range of its share (the first `r` XCDs one tile more), walked in groups of
// GROUP_M row tiles, column tile by column tile.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / kXcds, r = total % kXcds;
  const int x = b % kXcds, i = b / kXcds;
  const int t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
  const int per_group = GROUP_M * tiles_n;
  const int g = t / per_group, in = t % per_group;
  const int gm = min(GROUP_M, tiles_m - g * GROUP_M);  // row tiles in this group
  *tm = g * GROUP_M + in % gm;
  *tn = in / gm;
}

// Row stride of the bf16 output tile staged in LDS: 16 bytes past the row, so
// that the 16 rows x 32 bytes a fragment store covers fall on distinct banks
// (stride / 4 = 4 mod 64), and the 16-byte reads of 16 consecutive chunks of
// a row as well.
template <int BN>
constexpr int out_row_bytes() { return BN * 2 + 16; }
template <int BN>
constexpr int lds_bytes(bool staged) {
  return staged && BM * out_row_bytes<BN>() > NST * Cfg<BN>::ST ? BM * out_row_bytes<BN>()
                                                                  : NST * Cfg<BN>::ST;
}

// STAGED (bf16 output, N and the row stride multiples of 8, 16-byte aligned
// output): the tile goes through LDS and leaves in 16-byte row chunks, 1 KB
// of contiguous rows per wave store, instead of 32-byte pieces of 16 rows.
template <int BN, bool STAGED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_big_k(const bf16* __restrict__ A, const bf16* __restrict__ W, int M, int N, int K,
           int tiles_m, int tiles_n, GemmOut out) {
  using C = Cfg<BN>;
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<BN>(STAGED)];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const uint32_t lds0 = lds_u32(lds);

  // the PER_WAVE fragments this wave copies each stage: fragment f = wave *
  // PER_WAVE + u of the stage; row blocks past M / N re-read the last one
  // (never stored)
  const int nk = K / BK;
  const int rbA = (M + 15) / 16, rbW = (N + 15) / 16;
  const char* src[C::PER_WAVE];
#pragma unroll
  for (int u = 0; u < C::PER_WAVE; ++u) {
    const int f = wave * C::PER_WAVE + u;
    if (f < C::A_FR) {
      const int rb = min(m0 / 16 + f, rbA - 1);
      src[u] = reinterpret_cast<const char*>(A) + (int64_t)rb * nk * 1024 + lane * 16;
    } else {
      const int rb = min(n0 / 16 + f - C::A_FR, rbW - 1);
      src[u] = reinterpret_cast<const char*>(W) + (int64_t)rb * nk * 1024 + lane * 16;
    }
  }
  auto issue = [&](int kb) {
    const uint32_t st = lds0 + (uint32_t)((kb % NST) * C::ST + wave * C::PER_WAVE * 1024);
#pragma unroll
    for (int u = 0; u < C::PER_WAVE; ++u) dma16(src[u] + (int64_t)kb * 1024, st + u * 1024);
  };
  // this wave's copies of step kb are done once at most `later` steps issued
  // after it are still outstanding
  auto wait_step = [&](int later) {
    if (later >= 2) wait_vmcnt<2 * C::PER_WAVE>();
    else if (later == 1) wait_vmcnt<C::PER_WAVE>();
    else wait_vmcnt<0>();
  };

  f32x4_t acc[C::NI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) issue(s);
  for (int kb = 0; kb < nk; ++kb) {
    wait_step(min(NST - 2, nk - 1 - kb));
    __syncthreads();  // stage kb visible to all; stage kb - 1 (refilled next) free
    if (kb + NST - 1 < nk) issue(kb + NST - 1);
    // all 16 fragment reads go out first, in the order the products use
    // them (a0, then every w, then a1 ..), so the products start after two
    // reads and each later read only has to beat eight products
    const char* sb = lds + (kb % NST) * C::ST + lane * 16;
    bf16x8_t a[C::NI], w[C::NJ];
    a[0] = *reinterpret_cast<const bf16x8_t*>(sb + (wm * C::NI) * 1024);
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
      w[j] = *reinterpret_cast<const bf16x8_t*>(sb + (C::A_FR + wn * C::NJ + j) * 1024);
#pragma unroll
    for (int i = 1; i < C::NI; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(sb + (wm * C::NI + i) * 1024);
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[j], a[i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, C::NI + C::NJ, 0);  // the DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, C::NI * C::NJ, 0);  // then the products
  }

  if constexpr (STAGED) {
    constexpr int S = out_row_bytes<BN>();
    __syncthreads();  // every wave is done with the ring
    // lane holds tile rows wm 128 + 16 i + lane % 16, columns wn WN + 16 j +
    // 4 (lane / 16) .. + 3
    const int rw = wm * 128 + (lane & 15), cw = wn * C::WN + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const f32x4_t v = acc[i][j] * out.alpha;
        *reinterpret_cast<uint2*>(lds + (rw + 16 * i) * S + (cw + 16 * j) * 2) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    __syncthreads();
    constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
#pragma unroll 4
    for (int c = threadIdx.x; c < BM * CPR; c += 512) {
      const int r = c / CPR, cc = c % CPR;
      const int m = m0 + r, n = n0 + 8 * cc;
      if (m < M && n < N)
        *reinterpret_cast<uint4*>(out.b16 + (int64_t)m * out.ldo + n) =
            *reinterpret_cast<const uint4*>(lds + r * S + 16 * cc);
    }
    return;
  }

  // lane holds C[m][n .. n + 3] of every (i, j) block
  const int mw = m0 + wm * 128 + (lane & 15);
  const int nw = n0 + wn * C::WN + 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    __builtin_amdgcn_sched_barrier(0);  // one row block's values live at a time
    const int m = mw + 16 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int n = nw + 16 * j;
      if (n >= N) continue;
      const f32x4_t v = acc[i][j] * out.alpha;
      const int64_t o = (int64_t)m * out.ldo + n;
      if (n + 3 < N) {
        if (out.f32) {
          *reinterpret_cast<f32x4_t*>(out.f32 + o) = v;
        } else {
          const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(out.b16 + o) = make_uint2(lo, hi);
        }
      } else {
        for (int r = 0; r < 4 && n + r < N; ++r) {
          if (out.f32) out.f32[o + r] = v[r];
          else out.b16[o + r] = f32_to_bf16(v[r]);
        }
      }
    }
  }
}

// Row-major rows (stride ld) -> fragment-tiled layout.  Block = 256 threads
// for one 16-row block and four 32-k steps: thread t reads 16 bytes of row t /
// 16 (256 contiguous bytes per row and block) and stores them at their lane
// position in one of the four fragments (4 KB contiguous per block).  Rows
// past M are stored as zeros.
__global__ void __launch_bounds__(256)
tile_rows_k(const bf16* __restrict__ x, int64_t ld, int M, int nks, bf16* __restrict__ t) {
  const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int ks = 4 * blockIdx.x + (c >> 2);
  if (ks >= nks) return;
  const int nrb = (M + 15) / 16;
  for (int rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
    const int row = 16 * rb + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < M)
      v = *reinterpret_cast<const uint4*>(x + (int64_t)row * ld + 32 * ks + 8 * (c & 3));
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(t) + ((int64_t)rb * nks + ks) * 1024 +
                              (r + 16 * (c & 3)) * 16) = v;
  }
}

}  // namespace bg

size_t tiled_bytes(int rows, int K) { return (size_t)((rows + 15) / 16) * 16 * K * 2; }

void tile_rows(const bf16* x, int64_t ld, int rows, int K, bf16* t, hipStream_t st) {
  const int nks = K / 32;
  const dim3 grid((nks + 3) / 4, std::min((rows + 15) / 16, 65535));
  bg::tile_rows_k<<<grid, 256, 0, st>>>(x, ld, rows, nks, t);
}

int gemm_big_bn(int M, int N, int n_cu) {
  // the wider tile unless its grid leaves part of the last wave of tiles idle
  // where the narrower one fills the chip better
  const long tm = (M + bg::BM - 1) / bg::BM;
  auto eff = [&](int bn) {
    const long tiles = tm * ((N + bn - 1) / bn);
    const long waves = (tiles + n_cu - 1) / n_cu;
    const double useful = (double)M * N / ((double)tm * bg::BM * ((N + bn - 1) / bn) * bn);
    return useful * (double)tiles / (double)(waves * n_cu) * (bn == 256 ? 1.0 : 0.9);
  };
  return eff(256) >= eff(128) ? 256 : 128;
}

void gemm_big(const bf16* A, const bf16* W, int M, int N, int K, const GemmOut& out, int n_cu,
              hipStream_t st) {
  const int bn = gemm_big_bn(M, N, n_cu);
  const int tiles_m = (M + bg::BM - 1) / bg::BM, tiles_n = (N + bn - 1) / bn;
  const dim3 grid(tiles_m * tiles_n);
  const bool staged = !out.f32 && out.b16 && N % 8 == 0 && out.ldo % 8 == 0 &&
                      (uintptr_t)out.b16 % 16 == 0;
  if (bn == 256 && staged)
    bg::gemm_big_k<256, true><<<grid, 512, 0, st>>>(A, W, M, N, K, tiles_m, tiles_n, out);
  else if (bn == 256)
    bg::gemm_big_k<256, false><<<grid, 512, 0, st>>>(A, W, M, N, K, tiles_m, tiles_n, out);
  else if (staged)
    bg::gemm_big_k<128, true><<<grid, 512, 0, st>>>(A, W, M, N, K, tiles_m, tiles_n, out);
  else
    bg::gemm_big_k<128, false><<<grid, 512, 0, st>>>(A, W, M, N, K, tiles_m, tiles_n, out);
}

}  // namespace mla
