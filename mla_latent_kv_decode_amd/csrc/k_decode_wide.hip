// Split-S latent attention core for many heads: 128 heads per workgroup.
//
// Same computation as the 16-head core (absorbed decode, "Multi-Head Latent
// Attention" post, sections 3.3 and 3.6: scores of every head against the
// whole 576-wide latent row, softmax, latent sum of the 512 c_kv columns), for
// layers with many heads (DeepSeek-V3: 128), where the work per latent row is
// 8x larger and the 16-head kernel's per-head-group workgroups would stream
// every row 8 times from L2.  One workgroup of 8 waves (two per SIMD) covers
// 128 heads.  The rows of a segment stream once per workgroup through a
// 4-stage ring of 32-row tiles shared by the waves (global_load_lds_dwordx4;
// waves 0-3 each issue a quarter of every tile; one barrier per tile
// publishes it and frees the stage the next prefetch overwrites).
//
// Per tile, two phases split the work two ways so that no wave reads the whole
// tile twice:
//  - scores and softmax by head: wave w takes heads 16w .. 16w + 15 (36
//    mfma 16x16x32 over the 576 columns, K fragments read from LDS, Q^T in
//    VGPRs; lazy reference maximum) and publishes its P fragment (1 KB, in
//    the lane order of the latent sum's B operand), the heads' rescale
//    factors and whether the group rescaled;
//  - after a second barrier, the latent sum by column: wave w takes columns
//    64w .. 64w + 63 for all 128 heads (4 transposing C^T fragments, read
//    once, times the 8 groups' P: 32 mfma), rescaling its accumulators of a
//    group only when that group's maximum moved.
// Per tile and wave the LDS reads are 18 KB of K fragments, 4 KB of C^T and
// 8 KB of P (30 KB, against 50 KB when every wave summed all 512 columns for
// its own heads).  A segment's partial is the softmax waves' (max, sum) per
// head and the column waves' latent sums, written through the idle tile ring
// in whole rows.  MFMA operand layouts and the LDS swizzle of a 16-row block
// are those of the 16-head core.
//
// decode_core_wide8_k (below) is the same kernel over FP8 rows: each raw tile
// is copied once and decoded once into the shared bf16 tile, and the row
// scales enter the scores and the latent sum's probabilities in fp32.
#include <utility>

#include "decode_dev.h"

namespace mla {
namespace decw {

using namespace ddev;

constexpr int DC = 512;
constexpr int RW = 576;
constexpr int NW = 8;                         // waves (two per SIMD)
constexpr int HEADS = 16 * NW;                // heads per workgroup
constexpr int TR = 32;                        // rows per tile
constexpr int NST = 4;                        // stages
constexpr int ROPE_OFF = TR * 1024;           // latent of row r at r*1024, rope after
constexpr int ST_BYTES = TR * RW * 2;         // 36 KB
constexpr int NLOAD = TR + TR / 8;            // 36 wave-wide 16-byte loads per tile
constexpr int LOADERS = 4;                    // waves that issue the tile loads
constexpr int LPW = NLOAD / LOADERS;          // 9 per loading wave
static_assert(NLOAD % LOADERS == 0 && LOADERS <= NW, "tile loads split evenly");
// exchange area after the ring: every head group's P fragment (1 KB, lane
// order), the per-head rescale factors and the per-group rescale flags
constexpr int XP_OFF = NST * ST_BYTES;
// inside the exchange area: P fragments, rescale factors, rescale flags
constexpr int X_P = 0, X_A = NW * 1024, X_F = X_A + HEADS * 4, X_BYTES = X_F + NW * 4;
constexpr int LDS_BYTES = XP_OFF + X_BYTES;
constexpr int CB_W = 32 / NW;                  // 16-column blocks of the latent sum per wave
constexpr float kRescale = 8.0f;
constexpr int kXcds = 8;

static_assert(ROPE_OFF + TR * 128 == ST_BYTES, "stage layout");

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
// Load I of a tile whose first row is at `base` and whose last valid row is
// `last`: I < 32 copies the latent part of row I (source chunk lane ^ lat_swz(I & 15)),
// I >= 32 the rope parts of rows 8j .. 8j+7.  Rows past `last` re-read it.
template <int I, bool NT>
__device__ __forceinline__ void tile_load(const char* base, int last, uint32_t stage, int lane) {
  if constexpr (I < TR) {
    const int r = I <= last ? I : last;
    dma16h<NT>(base + r * (RW * 2) + ((lane ^ lat_swz(I & 15)) << 4), stage + I * 1024);
  } else {
    constexpr int J = I - TR;
    int r = 8 * J + (lane >> 3);
    const int cc = (lane & 7) ^ rope_swz(r & 15);
    r = r <= last ? r : last;
    dma16h<NT>(base + r * (RW * 2) + 1024 + (cc << 4), stage + ROPE_OFF + J * 1024);
  }
}

template <int W, bool NT, int... U>
__device__ __forceinline__ void wave_loads(const char* base, int last, uint32_t stage, int lane,
                                           std::integer_sequence<int, U...>) {
  (tile_load<W * LPW + U, NT>(base, last, stage, lane), ...);
}

// The lane index is re-read through an opaque instruction so the per-lane load
// addresses are recomputed per tile instead of being hoisted out of the tile
// loop (where they would take registers the accumulators need).
__device__ __forceinline__ int lane_id_opaque() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// NT: the non-temporal copy (cache rows no other workgroup of the part reads)
template <bool NT>
__device__ __forceinline__ void issue_tile(const char* base, int last, uint32_t stage, int wave) {
  const int lane = lane_id_opaque();
  const auto seq = std::make_integer_sequence<int, LPW>{};
  switch (wave) {
    case 0: wave_loads<0, NT>(base, last, stage, lane, seq); break;
    case 1: wave_loads<1, NT>(base, last, stage, lane, seq); break;
    case 2: wave_loads<2, NT>(base, last, stage, lane, seq); break;
    case 3: wave_loads<3, NT>(base, last, stage, lane, seq); break;
    default: break;
  }
}

// Per-lane LDS offsets of the MFMA operands inside a tile (as in the 16-head
// core).  Row-wise operand of k-step s < 16: row lr, chunk 4s + lg, i.e. at
// qk_off[s & 3] + 256 (s >> 2); rope chunk 4(s - 16) + lg at qk_rope[s - 16].
// Transposing operand of column block cb = 4q + t: lane (g = lg, s = lr)
// addresses row r = 4g + s/4, columns 16 cb + 4(s % 4): chunk 2cb + h with
// h = (s % 4) / 2, byte 8(s & 1).  Its position 2(cb ^ a) + (h ^ b) (a = r & 7,
// b = r >> 3) puts it at pv_e[t] + 128q for even q and pv_e[t] - pv_d + 128q
// for odd q.
struct TileOffsets {
  int qk_off[4], qk_rope0, qk_rope1, pv_e[4], pv_d;
  __device__ __forceinline__ explicit TileOffsets(int lane) {
    const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) qk_off[k] = lr * 1024 + 16 * ((4 * k + lg) ^ lat_swz(lr));
    qk_rope0 = ROPE_OFF + lr * 128 + 16 * (lg ^ rope_swz(lr));
    qk_rope1 = ROPE_OFF + lr * 128 + 16 * ((4 + lg) ^ rope_swz(lr));
    const int r = 4 * lg + (lr >> 2);
    const int a = r & 7, b = (r >> 3) & 1, h = (lr & 3) >> 1;
    pv_d = 256 * (a >> 2);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      pv_e[t] = r * 1024 + 16 * (h ^ b) + 8 * (lr & 1) + 32 * (t ^ (a & 3)) + 128 * (a >> 2);
  }
};

// Scores of this wave's 16 heads against the tile at `st` (S^T = K . Q^T for
// both 16-row blocks), the online softmax (lazy reference maximum; lane holds
// rows row0 + 16 rb + 4 lg + i of head h0 + lr), and the publication of P (the
// B operand of the latent sum, in lane order), the rescale factor of each
// head and whether this group rescaled, in the exchange area at `xch`.
// F8: the tile holds the rows' codes (exact in bf16) and `scl` their scales
// s_r; a score is s_r (q_abs . code) + q_rope . k_rope, and the latent sum's
// operand is p s_r (the softmax sum takes p).
template <bool F8>
__device__ __forceinline__ void tile_scores(const char* st, char* xch, const TileOffsets& to,
                                            const bf16x8_t (&qf)[18], int row0, int nv,
                                            int wave, int lane, float& m_run, float& l_run,
                                            const float* scl = nullptr) {
  const int lr = lane & 15, lg = lane >> 4;
  f32x4_t sc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const char* sl = st + rb * 16 * 1024;  // latent rows of this block
    const char* sr = st + rb * 16 * 128;   // rope rows (offsets include ROPE_OFF)
    f32x4_t sa = (f32x4_t){0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
    for (int part = 0; part < 6; ++part) {
      bf16x8_t kf[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int s = 3 * part + u;
        if (s < 16)
          kf[u] = *reinterpret_cast<const bf16x8_t*>(sl + to.qk_off[s & 3] + 256 * (s >> 2));
        else
          kf[u] = *reinterpret_cast<const bf16x8_t*>(sr + (s == 16 ? to.qk_rope0 : to.qk_rope1));
      }
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int s = 3 * part + u;
        if (F8 && s == 16) {
          // the latent part complete: scale it by the rows' s_r, then add
          // the rope products to it
          const float4 r4 = *reinterpret_cast<const float4*>(scl + 16 * rb + 4 * lg);
          const f32x4_t lat = sa + sb;
          sa = (f32x4_t){r4.x * lat[0], r4.y * lat[1], r4.z * lat[2], r4.w * lat[3]};
          sb = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
        if (s & 1) sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u], qf[s], sb, 0, 0, 0);
        else sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u], qf[s], sa, 0, 0, 0);
      }
    }
    sc[rb] = sa + sb;
  }
  float sv[8];
  bool grow = false;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = row0 + 16 * rb + 4 * lg + i < nv;
      sv[4 * rb + i] = valid ? sc[rb][i] * kLog2e : -INFINITY;
      grow |= sv[4 * rb + i] > m_run + kRescale;
    }
  float alpha = 1.f;
  const bool resc = __any(grow);
  if (resc) {
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
  }
  float pv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_run);
    l_run += pv[i];
  }
  if constexpr (F8) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float4 r4 = *reinterpret_cast<const float4*>(scl + 16 * rb + 4 * lg);
      pv[4 * rb] *= r4.x;
      pv[4 * rb + 1] *= r4.y;
      pv[4 * rb + 2] *= r4.z;
      pv[4 * rb + 3] *= r4.w;
    }
  }
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
  // (store addresses from the opaque lane index: nothing per lane stays live
  // across the tile loop for them)
  const int ln = lane_id_opaque();
  *reinterpret_cast<bf16x8_t*>(xch + X_P + wave * 1024 + ln * 16) =
      __builtin_bit_cast(bf16x8_t, pk);
  if (ln < 16) reinterpret_cast<float*>(xch + X_A)[16 * wave + ln] = alpha;
  if (ln == 0) reinterpret_cast<unsigned char*>(xch + X_F)[wave] = resc ? 1 : 0;
}

// O^T += C^T . P^T for this wave's columns and every head group: mfma
// 16x16x32 whose k index runs over rows 4g..4g+3 of row block 0, then of row
// block 1, for lane group g (the order the softmax lanes hold P in); C^T from
// two transposing reads per 16-column block, read once.
__device__ __forceinline__ void tile_latent_sum(const char* st, const char* xch,
                                                const TileOffsets& to, int wave, int lane,
                                                f32x4_t (&o)[NW][CB_W]) {
  const int lr = lane & 15;
  bf16x8_t cf[CB_W];
#pragma unroll
  for (int c = 0; c < CB_W; ++c) {
    typedef __attribute__((address_space(3))) s16x4_t* lptr;
    const int q = (CB_W * wave + c) >> 2, tt = (CB_W * wave + c) & 3;
    const int off = to.pv_e[tt] - (q & 1) * to.pv_d + 128 * q;
    const s16x4_t c0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(st + off));
    const s16x4_t c1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(st + 16 * 1024 + off));
    const s16x8_t c8 = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
    cf[c] = __builtin_bit_cast(bf16x8_t, c8);
  }
  // the eight groups' rescale flags (one byte each) in one read, the P
  // fragments one group ahead of their products
  static_assert(NW == 8, "eight flag bytes");
  const uint2 fl = *reinterpret_cast<const uint2*>(xch + X_F);
  const uint32_t flo = __builtin_amdgcn_readfirstlane(fl.x), fhi = __builtin_amdgcn_readfirstlane(fl.y);
  const float* xa = reinterpret_cast<const float*>(xch + X_A);
  bf16x8_t pg[NW];
  pg[0] = *reinterpret_cast<const bf16x8_t*>(xch + X_P + lane * 16);
#pragma unroll
  for (int g = 0; g < NW; ++g) {
    if (g + 1 < NW)
      pg[g + 1] = *reinterpret_cast<const bf16x8_t*>(xch + X_P + (g + 1) * 1024 + lane * 16);
    if (((g < 4 ? flo : fhi) >> (8 * (g & 3))) & 0xff) {
      // (the rescale factor's address from the opaque lane index: nothing
      // per lane stays live across the tile loop for it)
      const float a = xa[16 * g + (lane_id_opaque() & 15)];
#pragma unroll
      for (int c = 0; c < CB_W; ++c) o[g][c] *= a;
    }
#pragma unroll
    for (int c = 0; c < CB_W; ++c)
      o[g][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cf[c], pg[g], o[g][c], 0, 0, 0);
  }
}

// Q^T fragments of head h0 + lr of query row qrow_idx: columns 32 s + 8 lg .. + 7
__device__ __forceinline__ void load_query(const bf16* q_cat, int64_t qrow_idx, int H, int h0,
                                           int lane, bf16x8_t (&qf)[18]) {
  const bf16* qrow = q_cat + (qrow_idx * H + h0 + (lane & 15)) * RW + (lane >> 4) * 8;
#pragma unroll
  for (int s = 0; s < 18; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * s);
#pragma unroll
  for (int s = 0; s < 18; ++s) asm volatile("" ::"v"(qf[s]));
}

// The segment's partial: (max, sum) of this wave's heads; the latent sums of
// every head (fp32, 2 KB per head), staged through `stage` (the idle tile ring,
// at least 64 x XR_BYTES) 64 heads at a time so that they leave in 16-byte
// chunks of whole rows (1 KB of a row per wave store) rather than 64-byte
// pieces of 16 rows.  Starts with a barrier (the ring's last readers) and
// leaves the stage in use.
constexpr int XR_BYTES = DC * 4 + 16;  // staged row: the 16-byte pad spreads 16 rows over the banks
__device__ __forceinline__ void store_partial(float* __restrict__ acc_out,
                                              float* __restrict__ ml_out, int64_t slot, int H,
                                              int hbase, int wave, int lane, float m_run,
                                              float l_run, const f32x4_t (&o)[NW][CB_W],
                                              char* stage) {
  const int lr = lane & 15, lg = lane >> 4;
  const int h0 = hbase + wave * 16;
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (lg == 0) {
    ml_out[(slot * H + h0 + lr) * 2] = m_run;
    ml_out[(slot * H + h0 + lr) * 2 + 1] = l;
  }
  constexpr int GH = NW / 2;  // head groups per half
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // the stage is free
#pragma unroll
    for (int gg = 0; gg < GH; ++gg)
#pragma unroll
      for (int c = 0; c < CB_W; ++c)
        *reinterpret_cast<f32x4_t*>(stage + (16 * gg + lr) * XR_BYTES +
                                    (16 * CB_W * wave + 16 * c + 4 * lg) * 4) = o[GH * half + gg][c];
    __syncthreads();
    float* dst = acc_out + (slot * H + hbase + 16 * GH * half) * DC;
#pragma unroll 4
    for (int k = threadIdx.x; k < 16 * GH * (DC / 4); k += 64 * NW) {
      const int r = k / (DC / 4), cc = k % (DC / 4);
      *reinterpret_cast<float4*>(dst + r * DC + 4 * cc) =
          *reinterpret_cast<const float4*>(stage + r * XR_BYTES + 16 * cc);
    }
  }
}

__global__ void __launch_bounds__(512, 1)
decode_core_wide_k(const bf16* __restrict__ q_cat, const bf16* __restrict__ cache, DecodeMeta mt,
                   float* __restrict__ acc_out, float* __restrict__ ml_out, int H, int nparts,
                   int q_len, int nseg_total) {
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  // block -> (part, token, 128-head block), the blocks of a part on one XCD
  const int WG = H / HEADS;
  const int bid = blockIdx.x;
  const int part = (bid / (kXcds * WG * q_len)) * kXcds + bid % kXcds;
  const int hbq = (bid / kXcds) % (WG * q_len);
  const int tok = hbq / WG, hblk = hbq % WG;
  if (part >= nparts) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hbase = hblk * HEADS;
  const int h0 = hbase + wave * 16;  // this wave's softmax heads h0 .. h0 + 15
  const uint32_t lds0 = lds_u32(lds);
  const TileOffsets to(lane);

  const ConstWorkPtr works = reinterpret_cast<ConstWorkPtr>((uintptr_t)mt.work);
  DecodeWork wk = load_work(works + part);
  for (;;) {
    const int n = wk.n;                         // rows streamed
    const int nv = token_rows(wk, q_len, tok);  // rows this token sees
    const int ntile = (n + TR - 1) / TR;
    const int64_t wrow = wk.row;
    // rows no other workgroup of the part streams take the non-temporal copy
    const bool once = WG * q_len == 1;
    auto issue = [&](int t) {
      const char* base = reinterpret_cast<const char*>(cache + seg_row(mt, wrow, t * TR) * RW);
      const uint32_t stage = lds0 + (t % NST) * ST_BYTES;
      if (once) issue_tile<true>(base, n - t * TR - 1, stage, wave);
      else issue_tile<false>(base, n - t * TR - 1, stage, wave);
    };
#pragma unroll
    for (int t = 0; t < NST - 1; ++t)
      if (t < ntile) issue(t);
    DecodeWork nx = wk;
    if (wk.next >= 0) nx = load_work(works + wk.next);

    bf16x8_t qf[18];
    load_query(q_cat, (int64_t)wk.b * q_len + tok, H, h0, lane, qf);

    float m_run = -INFINITY, l_run = 0.f;
    // o[g][c][i]: latent sum of head hbase + 16 g + lr, column 16 (CB_W wave + c) + 4 lg + i
    f32x4_t o[NW][CB_W];
#pragma unroll
    for (int g = 0; g < NW; ++g)
#pragma unroll
      for (int c = 0; c < CB_W; ++c) o[g][c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < ntile; ++t) {
      static_assert(NST == 4, "wait counts below assume 4 stages");
      if (wave >= LOADERS) {
      } else if (t + 2 < ntile) wait_vmcnt<2 * LPW>();
      else if (t + 1 < ntile) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      __syncthreads();  // tile t is in LDS; every wave is done with tile t-1
      if (t + NST - 1 < ntile) issue(t + NST - 1);
      const char* st = lds + (t % NST) * ST_BYTES;
      tile_scores<false>(st, lds + XP_OFF, to, qf, t * TR, nv, wave, lane, m_run, l_run);
      __syncthreads();  // every group's P of tile t is published
      tile_latent_sum(st, lds + XP_OFF, to, wave, lane, o);
    }

    store_partial(acc_out, ml_out, (int64_t)tok * nseg_total + wk.pidx, H, hbase, wave, lane,
                  m_run, l_run, o, lds);
    __syncthreads();  // the stages are refilled by the next segment
    if (wk.next < 0) break;
    wk = nx;
  }
}

// ---- FP8 rows (656 bytes: 512 E4M3 codes, 64 bf16 rope values, the fp32
// row scale s).  The raw rows of a 32-row tile stream into a 3-stage ring of
// 21 KB stages (21 one-KB LDS-DMA copies per tile from waves 0-6, rows laid
// end to end at r * 656; past the tile's last row the copies re-read it); all
// eight waves then decode the tile once into a bf16 tile of the layout above
// (the codes' values, exact in bf16, and the rope values) plus the 32 row
// scales, which the scores and the latent sum's operand take in fp32 as the
// 16-head FP8 core does.  Two bf16 tiles alternate, so the decode of tile
// t + 1 runs beside the scores of tile t:
//   raw tile t + 1 arrived -> barrier Y(t): tile t decoded, the other bf16
//   tile, the P area and raw stage of tile t free
//   -> copy raw tile t + 3; decode raw tile t + 1 into the other bf16 tile;
//      scores and softmax of tile t
//   -> barrier X(t): P published -> latent sum of tile t.
constexpr int F8_RB = 656;                      // bytes per FP8 row
constexpr int F8_SCALE = 640;                   // byte of the row scale
constexpr int F8_NR = 3;                        // raw stages
constexpr int F8_NLOAD = 21;                    // one-KB copies per raw tile (32 x 656 B <= 21 KB)
constexpr int F8_LOADERS = 7;
constexpr int F8_LPW = F8_NLOAD / F8_LOADERS;   // 3 per loading wave
constexpr int F8_RAW_BYTES = F8_NLOAD * 1024;
constexpr int F8_RAW_OFF = 2 * ST_BYTES;
constexpr int F8_SC_OFF = F8_RAW_OFF + F8_NR * F8_RAW_BYTES;  // row scales of the two tiles
constexpr int F8_XP_OFF = F8_SC_OFF + 2 * TR * 4;
constexpr int F8_LDS_BYTES = F8_XP_OFF + X_BYTES;
static_assert(F8_NLOAD % F8_LOADERS == 0 && F8_LOADERS <= NW, "raw tile copies split evenly");
static_assert(TR * F8_RB <= F8_RAW_BYTES, "raw stage holds a tile");
static_assert(F8_LDS_BYTES <= 160 * 1024, "LDS");
static_assert(16 * (NW / 2) * XR_BYTES <= XP_OFF && 16 * (NW / 2) * XR_BYTES <= F8_SC_OFF,
              "a staged half of the partial fits in the tile ring");

// Copies I = LPW wave .. + LPW - 1 of a raw tile: 16-byte chunk j = 64 I +
// lane is chunk j % 41 of row j / 41 (rows past `last` re-read it).
template <bool NT>
__device__ __forceinline__ void issue_raw_tile(const char* base, int last, uint32_t stage,
                                               int wave) {
  const int lane = lane_id_opaque();
#pragma unroll
  for (int u = 0; u < F8_LPW; ++u) {
    const int I = F8_LPW * wave + u;
    const int j = 64 * I + lane;
    int r = j / (F8_RB / 16);
    const int c = j - r * (F8_RB / 16);
    r = r <= last ? r : last;
    dma16h<NT>(base + (int64_t)r * F8_RB + 16 * c, stage + I * 1024);
  }
}

// Rows 4 wave .. 4 wave + 3 of a raw tile decoded into a bf16 tile: lane l
// turns codes 8 l .. 8 l + 7 of each row into bf16 chunk l (at
// l ^ lat_swz(r)); lanes 0..31 copy rope chunk l & 7 of row 4 wave + l / 8;
// lanes 0..3 copy the rows' scales to `scl`.  (The lane index is re-read
// opaquely so that the per-lane offsets are not kept live across the tile
// loop.)
__device__ __forceinline__ void decode_raw_rows(const char* raw, char* dst, float* scl, int wave) {
  const int lane = lane_id_opaque();
  constexpr int RPW = TR / NW;  // rows per wave
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = RPW * wave + k;
    const uint2 v = *reinterpret_cast<const uint2*>(raw + r * F8_RB + 8 * lane);
    const uint32_t w[2] = {v.x, v.y};
    uint32_t out[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      out[2 * h] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, false));
      out[2 * h + 1] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, true));
    }
    *reinterpret_cast<uint4*>(dst + r * 1024 + 16 * (lane ^ lat_swz(r & 15))) =
        make_uint4(out[0], out[1], out[2], out[3]);
  }
  if (lane < 8 * RPW) {
    const int r = RPW * wave + (lane >> 3), c = lane & 7;
    *reinterpret_cast<uint4*>(dst + ROPE_OFF + r * 128 + 16 * (c ^ rope_swz(r & 15))) =
        *reinterpret_cast<const uint4*>(raw + r * F8_RB + 512 + 16 * c);
  }
  if (lane < RPW) {
    const int r = RPW * wave + lane;
    scl[r] = *reinterpret_cast<const float*>(raw + r * F8_RB + F8_SCALE);
  }
}

__global__ void __launch_bounds__(512, 1)
decode_core_wide8_k(const bf16* __restrict__ q_cat, const uint8_t* __restrict__ cache,
                    DecodeMeta mt, float* __restrict__ acc_out, float* __restrict__ ml_out, int H,
                    int nparts, int q_len, int nseg_total) {
  __shared__ __attribute__((aligned(1024))) char lds_all[F8_LDS_BYTES];
  char* xch = lds_all + F8_XP_OFF;  // the exchange area, behind the raw ring
  const int WG = H / HEADS;
  const int bid = blockIdx.x;
  const int part = (bid / (kXcds * WG * q_len)) * kXcds + bid % kXcds;
  const int hbq = (bid / kXcds) % (WG * q_len);
  const int tok = hbq / WG, hblk = hbq % WG;
  if (part >= nparts) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hbase = hblk * HEADS;
  const int h0 = hbase + wave * 16;
  const uint32_t raw0 = lds_u32(lds_all) + F8_RAW_OFF;
  const TileOffsets to(lane);

  const ConstWorkPtr works = reinterpret_cast<ConstWorkPtr>((uintptr_t)mt.work);
  DecodeWork wk = load_work(works + part);
  for (;;) {
    const int n = wk.n;
    const int nv = token_rows(wk, q_len, tok);
    const int ntile = (n + TR - 1) / TR;
    const int64_t wrow = wk.row;
    const bool once = WG * q_len == 1;
    auto issue = [&](int t) {
      if (wave >= F8_LOADERS) return;
      const char* base =
          reinterpret_cast<const char*>(cache) + seg_row(mt, wrow, t * TR) * F8_RB;
      const uint32_t stage = raw0 + (t % F8_NR) * F8_RAW_BYTES;
      if (once) issue_raw_tile<true>(base, n - t * TR - 1, stage, wave);
      else issue_raw_tile<false>(base, n - t * TR - 1, stage, wave);
    };
#pragma unroll
    for (int t = 0; t < F8_NR; ++t)
      if (t < ntile) issue(t);
    DecodeWork nx = wk;
    if (wk.next >= 0) nx = load_work(works + wk.next);

    bf16x8_t qf[18];
    load_query(q_cat, (int64_t)wk.b * q_len + tok, H, h0, lane, qf);

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t o[NW][CB_W];
#pragma unroll
    for (int g = 0; g < NW; ++g)
#pragma unroll
      for (int c = 0; c < CB_W; ++c) o[g][c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    wait_vmcnt<0>();
    __syncthreads();  // raw tile 0 arrived
    float* scl = reinterpret_cast<float*>(lds_all + F8_SC_OFF);  // [tile & 1][row]
    if (ntile > 0) decode_raw_rows(lds_all + F8_RAW_OFF, lds_all, scl, wave);

    for (int t = 0; t < ntile; ++t) {
      static_assert(F8_NR == 3, "wait counts below assume 3 raw stages");
      if (wave < F8_LOADERS && t + 1 < ntile) {
        if (t + 2 < ntile) wait_vmcnt<F8_LPW>();
        else wait_vmcnt<0>();
      }
      __syncthreads();  // Y(t)
      if (t + F8_NR < ntile) issue(t + F8_NR);
      if (t + 1 < ntile)
        decode_raw_rows(lds_all + F8_RAW_OFF + ((t + 1) % F8_NR) * F8_RAW_BYTES,
                        lds_all + ((t + 1) & 1) * ST_BYTES, scl + ((t + 1) & 1) * TR, wave);
      const char* st = lds_all + (t & 1) * ST_BYTES;
      tile_scores<true>(st, xch, to, qf, t * TR, nv, wave, lane, m_run, l_run, scl + (t & 1) * TR);
      __syncthreads();  // X(t)
      tile_latent_sum(st, xch, to, wave, lane, o);
    }

    store_partial(acc_out, ml_out, (int64_t)tok * nseg_total + wk.pidx, H, hbase, wave, lane,
                  m_run, l_run, o, lds_all);
    __syncthreads();  // the stages are refilled by the next segment
    if (wk.next < 0) break;
    wk = nx;
  }
}

}  // namespace decw

int decode_core_wide_heads() { return decw::HEADS; }

void decode_core_wide8(const bf16* q_cat, const uint8_t* cache, const DecodeMeta& m, int parts,
                       const TokenSplit& tk, float* acc, float* ml, const Dims& d,
                       hipStream_t st) {
  const int wg = d.H / decw::HEADS * tk.q_len;
  const int blocks = (parts + decw::kXcds - 1) / decw::kXcds * decw::kXcds * wg;
  decw::decode_core_wide8_k<<<blocks, 64 * decw::NW, 0, st>>>(q_cat, cache, m, acc, ml, d.H,
                                                              parts, tk.q_len, tk.nseg_total);
}

void decode_core_wide(const bf16* q_cat, const bf16* cache, const DecodeMeta& m, int parts,
                      const TokenSplit& tk, float* acc, float* ml, const Dims& d,
                      hipStream_t st) {
  const int wg = d.H / decw::HEADS * tk.q_len;
  const int blocks = (parts + decw::kXcds - 1) / decw::kXcds * decw::kXcds * wg;
  decw::decode_core_wide_k<<<blocks, 64 * decw::NW, 0, st>>>(q_cat, cache, m, acc, ml, d.H, parts,
                                                             tk.q_len, tk.nseg_total);
}

}  // namespace mla
