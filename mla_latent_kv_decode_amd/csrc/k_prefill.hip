// Causal chunked-prefill attention on CDNA4 MFMA (bf16 in, fp32 accumulate),
// expanded (non-absorbed) form: per head h and new token at position p,
//   s_t = q_h . [K_nope_h,t ; k_rope_t] * scale  for cached rows t <= p,
//   o_h = softmax_t(s) . V_h,t
// ("Multi-Head Latent Attention" post, sections 3.2 and 3.6: keys are the
// expanded K_nope with the shared rope key appended, values the expanded V;
// "Transformer and KV Cache Basics", mask design: a query at position p sees
// rows 0..p of its sequence).  K_nope and V come from the expansion GEMM
// (rows x H x [K_nope | V], bf16); k_rope is read from the latent cache row.
//
// Block = (tile of up to 256 new tokens of one sequence, head), 8 waves.  Wave
// w owns queries 32w .. 32w+31 of the tile as 2 blocks of 16.  Every value of
// a wave fits in 256 VGPRs (no accumulation registers), so two waves share each
// SIMD and one's softmax can overlap the other's MFMAs.  Keys stream in tiles
// of 32 through a 4-stage LDS ring filled by global_load_lds_dwordx4 (waves 0-3
// each issue a quarter of every tile; one barrier per tile both publishes the
// tile and frees the stage the next prefetch overwrites).  Per 32-key tile:
//   S^T (16 keys x 16 queries) = K . Q^T  -- 6 x mfma 16x16x32 per 16-key
//       block and query block, each K fragment (LDS) reused for the wave's
//       query blocks;
//   online softmax per query with a lazily moved reference maximum;
//   O (16 queries x 128 dims) += P . V -- mfma 16x16x32 over all 32 keys: P is
//       the A operand exactly as the two S^T blocks left it (k index = keys
//       4g..4g+3 of block 0, then of block 1, for lane group g), V the B
//       operand from two transposing reads (ds_read_b64_tr_b16) per 16-dim
//       block, each V fragment reused for the wave's query blocks.
// Key tiles past a wave's last query are skipped (the causal diagonal).
#include <utility>

#include "kernels.h"
#include "row_dev.h"

namespace mla {
namespace pf {

constexpr int DN = 128, DR = 64, DV = 128;
constexpr int KT = 32;                       // keys per tile
constexpr int NW = 8;                        // waves per block (two per SIMD)
constexpr int LOADERS = 4;                   // waves that issue the tile loads
constexpr int QW = 32;                       // queries per wave
constexpr int NQB = QW / 16;                 // 16-query blocks per wave
constexpr int NST = 4;                       // LDS stages
constexpr int KR_OFF = KT * DN * 2;          // K_nope: 256 B per key
constexpr int V_OFF = KR_OFF + KT * DR * 2;  // k_rope: 128 B per key
constexpr int ST_BYTES = V_OFF + KT * DV * 2;  // V: 256 B per key; 20 KB per stage
constexpr int NLOAD = ST_BYTES / 1024;       // 20 wave-wide 16-byte loads per tile
constexpr int LPW = NLOAD / LOADERS;         // 5 per loading wave
constexpr int KN_LOADS = KR_OFF / 1024, KR_LOADS = (V_OFF - KR_OFF) / 1024;
constexpr float kRescale = 8.0f;             // lazy-rescale threshold, log2 units
constexpr int kXcds = 8;
static_assert(NLOAD % LOADERS == 0 && LOADERS == 4 && LOADERS <= NW,
              "tile loads split evenly over 4 waves");
static_assert(NW * QW * (DV * 2 + 16) <= NST * ST_BYTES, "output tiles fit in the ring");

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// LDS layout of one stage, 16-byte chunks XOR-swizzled per key so the reads
// of both products spread over all banks:
//   K_nope chunk c (0..15) of key r at r*256 + 16*(c ^ (r & 15));
//   k_rope chunk c (0..7)  at KR_OFF + r*128 + 16*(c ^ ((r >> 1) & 7));
//   V      chunk c (0..15) at V_OFF  + r*256 + 16*(c ^ (2 * (r & 7))).
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

typedef const __attribute__((address_space(4))) PrefillTile* ConstTilePtr;

// Load I (0..NLOAD-1) of key tile [k0, k0 + KT): first K_nope (4 keys per
// load), then k_rope (8 keys per load), then V (4 keys per load).  In a full
// tile every key exists: the per-lane row offsets (lrow4 = (lane / 16) rows of
// the expanded K/V, lrow8 = (lane / 8) cache rows) are loop invariants and
// the tile's base addresses are uniform, so an address costs one add.  In the
// last tile keys at or past kend re-read the last key (their scores are
// masked).
template <int I, bool FULL>
__device__ __forceinline__ void issue_load(const char* kvh, const char* rope, int64_t kv_stride,
                                           int k0, int kend, uint32_t stage, int lane,
                                           int64_t lrow4, int64_t lrow8) {
  if constexpr (I < KN_LOADS) {
    const int r = 4 * I + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    if constexpr (FULL)
      dma16(kvh + (k0 + 4 * I) * kv_stride + lrow4 + c * 16, stage + I * 1024);
    else
      dma16(kvh + min(k0 + r, kend - 1) * kv_stride + c * 16, stage + I * 1024);
  } else if constexpr (I < KN_LOADS + KR_LOADS) {
    constexpr int J = I - KN_LOADS;
    const int r = 8 * J + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    if constexpr (FULL)
      dma16(rope + (int64_t)(k0 + 8 * J) * 1152 + lrow8 + c * 16, stage + KR_OFF + J * 1024);
    else
      dma16(rope + (int64_t)min(k0 + r, kend - 1) * 1152 + c * 16, stage + KR_OFF + J * 1024);
  } else {
    constexpr int J = I - KN_LOADS - KR_LOADS;
    const int r = 4 * J + (lane >> 4);
    const int c = (lane & 15) ^ (2 * (r & 7));
    if constexpr (FULL)
      dma16(kvh + (k0 + 4 * J) * kv_stride + lrow4 + 256 + c * 16, stage + V_OFF + J * 1024);
    else
      dma16(kvh + min(k0 + r, kend - 1) * kv_stride + 256 + c * 16, stage + V_OFF + J * 1024);
  }
}

template <int W, bool FULL, int... U>
__device__ __forceinline__ void issue_wave(const char* kvh, const char* rope, int64_t kv_stride,
                                           int k0, int kend, uint32_t stage, int lane,
                                           int64_t lrow4, int64_t lrow8,
                                           std::integer_sequence<int, U...>) {
  (issue_load<W * LPW + U, FULL>(kvh, rope, kv_stride, k0, kend, stage, lane, lrow4, lrow8), ...);
}

// This wave's LPW loads of the tile: straight-line code per wave.
template <bool FULL>
__device__ __forceinline__ void issue_tile_w(const char* kvh, const char* rope, int64_t kv_stride,
                                             int k0, int kend, uint32_t stage, int wave, int lane,
                                             int64_t lrow4, int64_t lrow8) {
  const auto seq = std::make_integer_sequence<int, LPW>{};
  switch (wave) {
    case 0: issue_wave<0, FULL>(kvh, rope, kv_stride, k0, kend, stage, lane, lrow4, lrow8, seq); break;
    case 1: issue_wave<1, FULL>(kvh, rope, kv_stride, k0, kend, stage, lane, lrow4, lrow8, seq); break;
    case 2: issue_wave<2, FULL>(kvh, rope, kv_stride, k0, kend, stage, lane, lrow4, lrow8, seq); break;
    case 3: issue_wave<3, FULL>(kvh, rope, kv_stride, k0, kend, stage, lane, lrow4, lrow8, seq); break;
    default: break;
  }
}

__device__ __forceinline__ void issue_tile(const char* kvh, const char* rope, int64_t kv_stride,
                                           int k0, int kend, uint32_t stage, int wave, int lane,
                                           int64_t lrow4, int64_t lrow8) {
  if (k0 + KT <= kend)
    issue_tile_w<true>(kvh, rope, kv_stride, k0, kend, stage, wave, lane, lrow4, lrow8);
  else
    issue_tile_w<false>(kvh, rope, kv_stride, k0, kend, stage, wave, lane, lrow4, lrow8);
}

__global__ void __launch_bounds__(NW * 64, 1)
prefill_attn_mfma_k(const bf16* __restrict__ q, const bf16* __restrict__ kv,
                    const bf16* __restrict__ cache,
                    const PrefillTile* tiles, int ntiles, int H, float qk_scale,
                    bf16* __restrict__ o_out, int o_tiled, RopeTab rt) {
  __shared__ __attribute__((aligned(1024))) char lds[NST * ST_BYTES];
  // Block -> (tile, head): every block of head h runs on XCD h % 8, so the
  // tiles of one head share that XCD's L2 for their keys and values.
  const int bid = blockIdx.x;
  const int r8 = bid / kXcds;
  const int h = (r8 / ntiles) * kXcds + bid % kXcds;
  const int tix = r8 % ntiles;
  if (h >= H) return;
  const ConstTilePtr tp = reinterpret_cast<ConstTilePtr>((uintptr_t)tiles) + tix;
  const int64_t kv_row0 = tp->kv_row0, cache_row0 = tp->cache_row0;
  const int t0 = tp->t0, nq = tp->nq, pos0 = tp->pos0;
  const int kend = pos0 + nq;  // keys 0 .. kend-1
  const int nkt = (kend + KT - 1) / KT;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const uint32_t lds0 = lds_u32(lds);
  const int64_t kv_stride = (int64_t)H * (DN + DV) * 2;  // bytes per expanded row
  const char* kvh = reinterpret_cast<const char*>(kv) + kv_row0 * kv_stride + h * (DN + DV) * 2;
  const char* rope = reinterpret_cast<const char*>(cache) + cache_row0 * 1152 + 1024;
  const int64_t lrow4 = (int64_t)(lane >> 4) * kv_stride, lrow8 = (int64_t)(lane >> 3) * 1152;

  // prologue: tiles 0 .. NST-2 in flight
#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
    if (t < nkt)
      issue_tile(kvh, rope, kv_stride, t * KT, kend, lds0 + t * ST_BYTES, wave, lane, lrow4, lrow8);

  // this wave's queries; lanes past the tile's last query repeat it
  const int qw0 = wave * QW;
  const bool wave_active = qw0 < nq;
  const int wmax_pos = pos0 + min(qw0 + QW, nq) - 1;
  const int wmin_pos = pos0 + qw0;
  bf16x8_t qf[NQB][6];
  int qpos[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int qi = min(qw0 + 16 * nb + lr, nq - 1);
    qpos[nb] = pos0 + qi;
    const bf16* qn = q + ((int64_t)(t0 + qi) * H + h) * (DN + DR) + 8 * lg;
    const bf16* qr = qn + DN;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[nb][s] = *reinterpret_cast<const bf16x8_t*>(qn + 32 * s);
    // the rope part is rotated here, at the query's position ("Multi-Head
    // Latent Attention" post, section 3.7): elements 32 s + 8 lg + 2 j, + 1
    // form pair 16 s + 4 lg + j; the rotated pair is rounded to bf16
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qr + 32 * s);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      uint32_t rw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float ou, ov;
        rope_pair(bf16_to_f32((bf16)(w[j] & 0xffff)), bf16_to_f32((bf16)(w[j] >> 16)), qpos[nb],
                  rt.theta[16 * s + 4 * lg + j], &ou, &ov);
        rw[j] = pack_bf16x2(ou, ov);
      }
      qf[nb][4 + s] = __builtin_bit_cast(bf16x8_t, rw);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
    for (int s = 0; s < 6; ++s) asm volatile("" ::"v"(qf[nb][s]));

  // K fragment of key row lr, 16-byte chunk c of k-step s: byte offsets
  const int kn_off = lr * 256;
  const int kr_off = KR_OFF + lr * 128;
  const int kn_x = lr & 15, kr_x = (lr >> 1) & 7;
  // V^T fragment (transposing read): lane (g = lg, s = lr) addresses key
  // 4g + s/4, dims 16 db + 4(s % 4): chunk 2 db + (s % 4)/2, byte 8(s & 1)
  const int vr = 4 * lg + (lr >> 2);
  const int v_base = V_OFF + vr * 256 + 8 * (lr & 1);
  const int v_h = (lr & 3) >> 1, v_x = 2 * (vr & 7);

  // o[db][nb][i]: query 16 nb + 4 lg + i, dim 16 db + lr; block db = 8 multiplies
  // P by a block of ones, so every lane holds the row sums of its queries
  float m_run[NQB];
  f32x4_t o[9][NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    m_run[nb] = -INFINITY;
#pragma unroll
    for (int db = 0; db < 9; ++db) o[db][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }
  bf16x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;

  for (int kt = 0; kt < nkt; ++kt) {
    // tiles kt+1 .. kt+NST-2 may stay in flight
    static_assert(NST == 4, "wait counts below assume 4 stages");
    if (wave >= LOADERS) {
    } else if (kt + 2 < nkt) wait_vmcnt<2 * LPW>();
    else if (kt + 1 < nkt) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    __syncthreads();  // tile kt is in LDS; every wave is done with tile kt-1
    if (kt + NST - 1 < nkt)
      issue_tile(kvh, rope, kv_stride, (kt + NST - 1) * KT, kend,
                 lds0 + ((kt + NST - 1) % NST) * ST_BYTES, wave, lane, lrow4, lrow8);
    if (!wave_active) continue;
    const char* st = lds + (kt % NST) * ST_BYTES;
    const int k0 = kt * KT;
    if (k0 > wmax_pos) continue;  // every key of the tile is masked for this wave
    // ---- S^T (16 keys x 16 queries) = K . Q^T for both 16-key blocks of the tile
    f32x4_t sacc[2][NQB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const char* sb = st + mb * 16 * 256;  // K_nope rows of this block
      const char* sr = st + mb * 16 * 128;  // k_rope rows of this block
      bf16x8_t kf[6];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[s] = *reinterpret_cast<const bf16x8_t*>(sb + kn_off + (((4 * s + lg) ^ kn_x) << 4));
#pragma unroll
      for (int s = 0; s < 2; ++s)
        kf[4 + s] = *reinterpret_cast<const bf16x8_t*>(sr + kr_off + (((4 * s + lg) ^ kr_x) << 4));
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        sacc[mb][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 6; ++s)
          sacc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[nb][s], sacc[mb][nb], 0, 0, 0);
      }
    }
    // softmax: lane holds keys k0 + 16 mb + 4 lg + i of query 16 nb + lr.  In
    // log2 units t = s * scale - m_run; the reference maximum m_run only moves
    // when some t exceeds kRescale (a wave vote), so p = 2^t <= 2^kRescale.
    // The causal mask is applied only to tiles that reach past the wave's
    // first query.
    const bool diag = k0 + KT - 1 > wmin_pos;
    bf16x8_t pf[NQB];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
      float t[8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = fmaf(sacc[mb][nb][i], qk_scale, -m_run[nb]);
          if (diag && k0 + 16 * mb + 4 * lg + i > qpos[nb]) v = -INFINITY;
          t[4 * mb + i] = v;
        }
      float tmax = t[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, t[i]);
      if (__any(tmax > kRescale)) {
        float sv[8];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool valid = !diag || k0 + 16 * mb + 4 * lg + i <= qpos[nb];
            sv[4 * mb + i] = valid ? sacc[mb][nb][i] * qk_scale : -INFINITY;
          }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[nb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_new);
        m_run[nb] = m_new;
#pragma unroll
        for (int db = 0; db < 9; ++db) o[db][nb] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = sv[i] - m_new;
      }
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = __builtin_amdgcn_exp2f(t[i]);
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
      pf[nb] = __builtin_bit_cast(bf16x8_t, pk);
    }
    // ---- O += P . V over the 32 keys: mfma 16x16x32 whose k index runs over
    // keys 4g..4g+3 of block 0, then of block 1, for lane group g (how the
    // lanes hold P); V comes from two transposing reads per 16-dim block.
    const char* sv_base = st + v_base;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int c = (2 * db + v_h) ^ v_x;
      typedef __attribute__((address_space(3))) s16x4_t* lptr;
      const s16x4_t c0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(sv_base + (c << 4)));
      const s16x4_t c1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(sv_base + 16 * 256 + (c << 4)));
      const s16x8_t c8 = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8_t cf = __builtin_bit_cast(bf16x8_t, c8);
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb)
        o[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[nb], cf, o[db][nb], 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb)
      o[8][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[nb], ones, o[8][nb], 0, 0, 0);
  }

  // epilogue through LDS: every wave is done with the ring, which now holds
  // each wave's normalised 32 x 128 output tile (rows padded to 272 bytes so
  // the four rows a store instruction touches fall on different banks); the
  // tile then leaves in 16-byte chunks of 8 dims, row-major or in the output
  // projection's fragment-tiled layout
  __syncthreads();
  if (!wave_active) return;
  constexpr int OROW = DV * 2 + 16;
  char* ot = lds + wave * (QW * OROW);
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv = 1.f / o[8][nb][i];  // row sum of query 16 nb + 4 lg + i
      bf16* row = reinterpret_cast<bf16*>(ot + (16 * nb + 4 * lg + i) * OROW) + lr;
#pragma unroll
      for (int db = 0; db < 8; ++db) row[16 * db] = f32_to_bf16(o[db][nb][i] * inv);
    }
  }
#pragma unroll
  for (int k = 0; k < QW * DV / 8 / 64; ++k) {
    const int c = lane + 64 * k, r = c >> 4, c8 = c & 15;
    const int qi = qw0 + r;
    if (qi >= nq) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(ot + r * OROW + 16 * c8);
    const int64_t t = t0 + qi;
    bf16* dst;
    if (o_tiled)  // dims 8 c8 .. of head h: fragment (t / 16, 4 h + c8 / 4), lane slot
      dst = o_out + ((t >> 4) * (H * DV / 32) + h * (DV / 32) + (c8 >> 2)) * 512 +
            ((t & 15) + 16 * (c8 & 3)) * 8;
    else
      dst = o_out + (t * H + h) * DV + 8 * c8;
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

}  // namespace pf

int prefill_tile_queries() { return pf::NW * pf::QW; }

void prefill_attn_mfma(const bf16* q, const bf16* kv, const bf16* cache,
                       const PrefillTile* tiles, int ntiles, int H, float scale, bf16* o,
                       bool o_tiled, const RopeTab& rt, hipStream_t st) {
  const int blocks = ntiles * ((H + pf::kXcds - 1) / pf::kXcds) * pf::kXcds;
  pf::prefill_attn_mfma_k<<<blocks, pf::NW * 64, 0, st>>>(q, kv, cache, tiles, ntiles, H,
                                                  scale * kLog2e, o, o_tiled ? 1 : 0, rt);
}

}  // namespace mla
