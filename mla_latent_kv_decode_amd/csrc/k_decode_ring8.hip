// Split-S latent attention core over an FP8 latent cache, for layers whose
// heads come in a few 16-head groups (DeepSeek-V2-Lite shapes: d_c = 512,
// d_r = 64).
//
// Same computation as the bf16 ring core ("Multi-Head Latent Attention" post,
// sections 3.3 and 3.6: per head, scores against the whole cached row, a
// softmax over the rows, the probability-weighted latent sum), reading rows
// stored in low precision (the post's introduction lists low-precision
// storage; section 3.1 sizes a cache element at 1 byte for FP8).  A cached row
// is 656 bytes:
//   [0, 512)    c as OCP FP8 E4M3 codes, c_i ~= s * value(code_i)
//   [512, 640)  k_rope as 64 bf16
//   [640, 644)  the row's scale s (fp32), then 12 zero bytes
// E4M3 values convert to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale
// 1), so the MFMA products are those of the stored values; the row scale is
// applied in fp32 to the latent part of each score, s_t = s_r (q_abs . code_t)
// + q_rope . k_rope_t, and folded into the probabilities of the latent sum,
// sum_t (p_t s_t) code_t.
//
// Work and waves as in the bf16 ring core: the host cuts the concatenated rows
// into one contiguous span per persistent workgroup, split at sequence
// boundaries into segments; two producer waves stream every position (the
// segment's query tile, then its 32-row tiles) into a 7-stage LDS ring with
// global_load_lds_dwordx4 (22 one-KB copies per position), four consumer
// waves compute, one barrier per position.  (Measured: with the consumers'
// math removed the stream takes 93 % of the kernel's time, and a deeper ring
// - six positions in flight, bought with a second barrier per tile - does
// not speed the stream up: its in-loop rate is that of the bf16 core, and
// launch and tail make up the rest.)
//
// The per-row work is larger than in the bf16 core (every code is converted
// before each of the two MFMA products that use it, and the conversion issues
// at about two thirds of an MFMA's rate), so the score product is not
// repeated in every consumer wave: wave w computes, for row block w >> 1 and
// half w & 1 of the query dimensions (256 latent + 32 rope), the partial
// score s_r (q_lat . code) + q_rope . k_rope over its half and writes it to
// LDS (1 KB per wave and tile, two buffers).  The softmax and the latent sum
// of a tile run one position later, after the barrier that makes the four
// partials visible, so a tile's stage stays in use for two positions: the
// producers refill the stage of position gt - 2 after barrier gt (four
// positions in flight), and both sides pass one extra barrier at the end.
//
// LDS stage of a row tile (21 KB):
//   latent codes  row r at r * 512, 16-byte chunk c at c ^ f8(r),
//                 f8(r) = (r & 15) ^ 8 ((r >> 4) & 1)
//   rope (bf16)   row r at 16384 + r * 128, chunk c at c ^ rope_swz(r)
//   scales        row r at 20480 + 16 r (the spare copy writes the same bytes)
// f8 makes both reads conflict-free on 64 four-byte banks (32 lanes per
// cycle for 8-byte reads): the score operand (16 rows, one chunk) and the
// transposing read of the latent sum (rows 4g .. 4g + 3 of both 16-row blocks
// for lane groups g = 0, 1 and g = 2, 3) each hit 16 distinct chunks.
// A query tile keeps the bf16 ring core's layout: 16 rows of 1 KB (latent
// part, chunk c at c ^ lat_swz(r)) and the rope parts at 16384; its spare
// copies fill 18432 .. 21503 (the last one twice).
// After the 7 stages: the partial scores, [buffer][wave][lane] as f32x4.
//
// Per 32-row tile and consumer wave w:
//   partial S^T over rows 16 (w >> 1) .. + 15 and dimension half w & 1:
//     8 mfma 16x16x32 on converted codes (8 codes per lane from one
//     ds_read_b64) + 1 mfma on the bf16 rope part, scaled by s_r in fp32;
//   next position: S^T = sum of the two partials of each row block, online
//     softmax in log2 units with a lazily moved reference maximum (as the
//     bf16 core, repeated in every wave), p' = p * s_r;
//   O^T += C8^T . P'^T over column quarter w: 8 mfma 16x16x32; one
//     ds_read_b64_tr_b8 per 16-column block gives each lane 8 codes of one
//     column (rows 4g .. 4g + 3 of both row blocks for lane group g: the k
//     order the score layout holds P in).
// Outputs are those of the bf16 core (normalised o_lat rows for sequences in
// one segment, else fp32 partials for the combine).
#include <utility>

#include "decode_dev.h"

namespace mla {
namespace decr8 {

using namespace ddev;

constexpr int DC = 512;
constexpr int QRW = 576;                     // q_cat row width (bf16 elements)
constexpr int RB = 656;                      // FP8 cache row bytes
constexpr int TR = 32;                       // rows per tile
constexpr int NST = 7;                       // ring stages
constexpr int ROPE_OFF = 16384;              // rope rows (data and query tiles)
constexpr int SC_OFF = 20480;                // row scales
constexpr int QSPARE_OFF = 18432;            // query tiles: after 16 rope rows
constexpr int ST_BYTES = 21504;              // 21 KB
constexpr int PS_OFF = NST * ST_BYTES;       // partial scores: 2 buffers x 4 waves x 1 KB
constexpr int PS_BYTES = 2 * 4096;
constexpr int NCOPY = 22;                    // one-KB copies per position
constexpr int NPROD = 2;
constexpr int LPW = NCOPY / NPROD;           // 11
constexpr int NCONS = 4;
constexpr int NCB = 32 / NCONS;              // 16-column blocks per consumer wave
constexpr int NTHR = 64 * (NCONS + NPROD);
constexpr float kRescale = 8.0f;
constexpr int kXcds = 8;
static_assert(NCOPY % NPROD == 0, "copies split evenly over the producers");
static_assert((NST - 3) * LPW <= 63, "copies in flight fit the vmcnt field");
static_assert(PS_OFF + PS_BYTES <= 160 * 1024, "ring and partial scores fit the LDS");
static_assert(QSPARE_OFF + 3 * 1024 == ST_BYTES, "query spares fill the stage");

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ constexpr int f8(int r) { return (r & 15) ^ (((r >> 4) & 1) << 3); }

// Copy I of a row tile whose first row is at `base` (byte address) and whose
// last valid row is `last`; rows past `last` re-read it (their scores are
// masked).
template <int I, bool NT>
__device__ __forceinline__ void row_copy(const char* base, int last, uint32_t stage, int lane) {
  if constexpr (I < 16) {  // latent codes of rows 2I (lanes 0-31) and 2I + 1
    const int r = 2 * I + (lane >> 5);
    const int rs = r <= last ? r : last;
    dma16h<NT>(base + rs * RB + (((lane & 31) ^ f8(r)) << 4), stage + I * 1024);
  } else if constexpr (I < 20) {  // rope of rows 8J .. 8J + 7
    constexpr int J = I - 16;
    const int r = 8 * J + (lane >> 3);
    const int cc = (lane & 7) ^ rope_swz(r & 15);
    const int rs = r <= last ? r : last;
    dma16h<NT>(base + rs * RB + 512 + (cc << 4), stage + ROPE_OFF + J * 1024);
  } else {  // scales of rows 0 .. 31 (twice); the spare copy I = 21 repeats it
    const int r = lane & 31;
    const int rs = r <= last ? r : last;
    dma16h<NT>(base + rs * RB + 640, stage + SC_OFF);
  }
}

// Copy I of a query tile (the group's 16 q_cat rows, bf16, 1152 bytes each)
template <int I>
__device__ __forceinline__ void query_copy(const char* qb, uint32_t stage, int lane) {
  if constexpr (I < 16) {
    dma16(qb + I * (QRW * 2) + ((lane ^ lat_swz(I & 15)) << 4), stage + I * 1024);
  } else if constexpr (I < 18) {
    constexpr int J = I - 16;
    const int r = 8 * J + (lane >> 3);
    const int cc = (lane & 7) ^ rope_swz(r & 15);
    dma16(qb + r * (QRW * 2) + 1024 + (cc << 4), stage + ROPE_OFF + J * 1024);
  } else {  // spares: the first KB of row 0, into 18432 .. 21503 (I = 21 repeats I = 20)
    constexpr int J = I < 21 ? I - 18 : 2;
    dma16(qb + (lane << 4), stage + QSPARE_OFF + J * 1024);
  }
}

template <int P, bool NT, int... U>
__device__ __forceinline__ void producer_rows(const char* base, int last, uint32_t stage, int lane,
                                              std::integer_sequence<int, U...>) {
  (row_copy<P * LPW + U, NT>(base, last, stage, lane), ...);
}

template <int P, int... U>
__device__ __forceinline__ void producer_query(const char* qb, uint32_t stage, int lane,
                                               std::integer_sequence<int, U...>) {
  (query_copy<P * LPW + U>(qb, stage, lane), ...);
}

// NT: the non-temporal copy (rows no other workgroup of the part reads)
template <bool NT>
__device__ __forceinline__ void issue_rows(const char* base, int last, uint32_t stage, int p,
                                           int lane) {
  const auto seq = std::make_integer_sequence<int, LPW>{};
  if (p == 0) producer_rows<0, NT>(base, last, stage, lane, seq);
  else producer_rows<1, NT>(base, last, stage, lane, seq);
}

__device__ __forceinline__ void issue_query(const char* qb, uint32_t stage, int p, int lane) {
  const auto seq = std::make_integer_sequence<int, LPW>{};
  if (p == 0) producer_query<0>(qb, stage, lane, seq);
  else producer_query<1>(qb, stage, lane, seq);
}

// wait until at most `ahead` positions (LPW copies each) are in flight
template <int A>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A) wait_vmcnt<A * LPW>();
    else wait_ahead<A - 1>(ahead);
  }
}

// 8 E4M3 codes -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8_t codes_to_bf16(i32x2_t v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return (bf16x8_t){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__global__ void __launch_bounds__(NTHR, 1)
decode_core_ring8_k(const bf16* __restrict__ q_cat, const uint8_t* __restrict__ cache,
                    DecodeMeta mt, float* __restrict__ acc, float* __restrict__ ml,
                    bf16* __restrict__ o_lat, int H, int nparts, int q_len, int nseg_total) {
  __shared__ __attribute__((aligned(1024))) char lds[PS_OFF + PS_BYTES];
  const int HG = H / 16;
  const int bid = blockIdx.x;
  const int part = (bid / (kXcds * HG * q_len)) * kXcds + bid % kXcds;
  const int hgq = (bid / kXcds) % (HG * q_len);
  const int tok = hgq / HG, hg = hgq % HG;  // new token and 16-head group
  if (part >= nparts) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t lds0 = lds_u32(lds);
  const ConstWorkPtr works = reinterpret_cast<ConstWorkPtr>((uintptr_t)mt.work);
  const DecodeWork first = load_work(works + part);

  if (wave >= NCONS) {
    // ------------------------------------------------------------ producers
    const int p = wave - NCONS;
    DecodeWork iw = first, inx = first;
    if (iw.next >= 0) inx = load_work(works + iw.next);
    int ik = 0, intl = 1 + (iw.n + TR - 1) / TR;  // next position of segment iw, its count
    int issued = 0;
    int64_t next_row = 0;
    auto issue_next = [&]() {
      if (ik == intl) {
        if (iw.next < 0) return;
        iw = inx;
        if (iw.next >= 0) inx = load_work(works + iw.next);
        ik = 0;
        intl = 1 + (iw.n + TR - 1) / TR;
      }
      const uint32_t stage = lds0 + (uint32_t)(issued % NST) * ST_BYTES;
      if (ik == 0) {
        issue_query(reinterpret_cast<const char*>(
                        q_cat + ((int64_t)(iw.b * q_len + tok) * H + hg * 16) * QRW),
                    stage, p, lane);
      } else {
        const int t = ik - 1;
        const char* rb = reinterpret_cast<const char*>(cache) + next_row * RB;
        if (HG * q_len == 1) issue_rows<true>(rb, iw.n - t * TR - 1, stage, p, lane);
        else issue_rows<false>(rb, iw.n - t * TR - 1, stage, p, lane);
      }
      // the cache row of the segment's next tile, one issue ahead (a paged
      // cache's page lookup is a load)
      if (ik + 1 < intl) next_row = seg_row(mt, iw.row, ik * TR);
      ++ik;
      ++issued;
    };
#pragma unroll 1
    for (int i = 0; i < NST - 2; ++i) issue_next();
#pragma unroll 1
    for (int gt = 0; gt < issued; ++gt) {
      wait_ahead<NST - 3>(issued - gt - 1);  // positions issued after position gt
      __syncthreads();  // position gt is in LDS; the consumers are done with gt - 2
      if (issued == gt + NST - 2) issue_next();  // refills the stage of position gt - 2
    }
    __syncthreads();  // the consumers' last exchange of partial scores
    return;
  }

  // -------------------------------------------------------------- consumers
  const int cq = wave;                    // latent-sum column quarter: 128 cq .. 128 cq + 127
  const int rbq = cq >> 1, hq = cq & 1;   // score row block and dimension half
  const int lr = lane & 15, lg = lane >> 4;
  // score operand of latent k-step s = 8 hq + j (row 16 rbq + lr, codes
  // 32 s + 8 lg .. + 7): half (lg & 1) of chunk c = 2 s + (lg >> 1), stored at
  // c ^ f8(row) = 2 (s ^ x1) + h1 with x1, h1 from lr ^ 8 rbq
  int qk8[8];
  {
    const int x = lr ^ (8 * rbq);
    const int h1 = (lg >> 1) ^ (x & 1);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      qk8[j] = (16 * rbq + lr) * 512 + 32 * (j ^ (x >> 1)) + 16 * h1 + 8 * (lg & 1) + 256 * hq;
  }
  // rope operand: row 16 rbq + lr, rope dims 32 hq + 8 lg .. + 7
  const int qk_rope = ROPE_OFF + (16 * rbq + lr) * 128 + 16 * ((4 * hq + lg) ^ rope_swz(lr));
  // transposing read of column block cb for lane (g = lg, i = lr): row
  // j < 4 ? 4g + j : 16 + 4g + j - 4 with j = i / 2, bytes 8 (i & 1) of chunk
  // cb ^ f8(row); cb = 8 cq + k: pv8[k] = base + 16 (k ^ (f8 & 7))
  int pv8[NCB];
  {
    const int j = lr >> 1;
    const int row = j < 4 ? 4 * lg + j : 16 + 4 * lg + (j - 4);
    const int fr = f8(row);
    const int base = row * 512 + 16 * ((8 * cq) ^ (fr & 8)) + 8 * (lr & 1);
#pragma unroll
    for (int k = 0; k < NCB; ++k) pv8[k] = base + 16 * (k ^ (fr & 7));
  }
  const int gh = hg * 16 + lr;  // this lane's head in the score and sum layouts
  const int sc0 = SC_OFF + 16 * 4 * lg;  // scale of row 16 rb + 4 lg + i at sc0 + 256 rb + 16 i
  char* const ps = lds + PS_OFF + 16 * lane;  // + 4096 buffer + 1024 wave

  // LDS reads of a position's two computations, issued together before either
  // (the partial scores of the new tile, the softmax and latent sum of the
  // previous one), so that one wave per SIMD keeps many reads in flight
  struct PartIn {
    i32x2_t c[8];
    bf16x8_t kr;
    float scale[4];
  };
  struct FinIn {
    f32x4_t pa[4];
    float rs[8];
    i32x2_t cr[NCB];
  };
  auto part_load = [&](const char* st, PartIn& in) {
#pragma unroll
    for (int j = 0; j < 8; ++j) in.c[j] = *reinterpret_cast<const i32x2_t*>(st + qk8[j]);
    in.kr = *reinterpret_cast<const bf16x8_t*>(st + qk_rope);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      in.scale[i] = *reinterpret_cast<const float*>(st + sc0 + 256 * rbq + 16 * i);
  };
  auto fin_load = [&](const char* st, int par, FinIn& in) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      in.pa[i] = *reinterpret_cast<const f32x4_t*>(ps + par * 4096 + i * 1024);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      in.rs[i] = *reinterpret_cast<const float*>(st + sc0 + 256 * (i >> 2) + 16 * (i & 3));
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      typedef __attribute__((address_space(3))) i32x2_t* lptr;
      in.cr[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lptr)(st + pv8[j]));
    }
  };

  // partial scores of a tile -> buffer par
  auto partial = [&](const PartIn& in, int par, const bf16x8_t (&ql)[8], const bf16x8_t& qr) {
    f32x4_t sa = (f32x4_t){0.f, 0.f, 0.f, 0.f}, sb = sa, sr = sa;
    sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(in.kr, qr, sr, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(in.c[j]), ql[j], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(in.c[j + 1]), ql[j + 1], sb, 0, 0,
                                                   0);
    }
    const f32x4_t sl = sa + sb;
    f32x4_t out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = fmaf(in.scale[i], sl[i], sr[i]);
    *reinterpret_cast<f32x4_t*>(ps + par * 4096 + cq * 1024) = out;
  };

  DecodeWork wk = first, nx = first;
  if (wk.next >= 0) nx = load_work(works + wk.next);
  int gt = 0;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[NCB];

  // softmax and latent sum of a tile; only a segment's last tile (finished on
  // the pending path) can hold rows past the segment's end, so only that call
  // masks
  auto finish = [&](const FinIn& in, int row0, int n, bool last) {
    bf16x8_t cf[NCB];
#pragma unroll
    for (int j = 0; j < NCB; ++j) cf[j] = codes_to_bf16(in.cr[j]);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sv[i] = (in.pa[2 * (i >> 2)][i & 3] + in.pa[2 * (i >> 2) + 1][i & 3]) * kLog2e;
    if (last) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (row0 + 16 * (i >> 2) + 4 * lg + (i & 3) >= n) sv[i] = -INFINITY;
    }
    // ---- online softmax: lane holds rows row0 + 16 rb + 4 lg + i of head gh
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) grow |= sv[i] > m_run + kRescale;
    if (__any(grow)) {
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < NCB; ++j) o[j] *= alpha;
    }
    bf16x8_t pf;
    {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_run);
        l_run += pv[i];
      }
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk[i] = pack_bf16x2(pv[2 * i] * in.rs[2 * i], pv[2 * i + 1] * in.rs[2 * i + 1]);
      pf = __builtin_bit_cast(bf16x8_t, pk);
    }
    // ---- O^T += C8^T . P'^T over this wave's column blocks 8 cq .. 8 cq + 7
#pragma unroll
    for (int j = 0; j < NCB; ++j)
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cf[j], pf, o[j], 0, 0, 0);
  };
  // finish of the tile in stage st with partials in buffer par, on its own
  auto finish_alone = [&](const char* st, int par, int row0, int n) {
    FinIn in;
    fin_load(st, par, in);
    finish(in, row0, n, true);
  };

  // ---- end of a segment: lane holds columns 128 cq + 16 j + 4 lg .. +3 of head gh
  auto store = [&](const DecodeWork& w) {
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (w.nseg == 1) {
      const float inv = 1.f / l;
      bf16* dst = o_lat + ((int64_t)(w.b * q_len + tok) * H + gh) * DC + 128 * cq + 4 * lg;
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        uint2 pk;
        pk.x = pack_bf16x2(o[j][0] * inv, o[j][1] * inv);
        pk.y = pack_bf16x2(o[j][2] * inv, o[j][3] * inv);
        *reinterpret_cast<uint2*>(dst + 16 * j) = pk;
      }
    } else {
      const int64_t slot = (int64_t)tok * nseg_total + w.pidx;
      float* pacc = acc + (slot * H + gh) * DC + 128 * cq + 4 * lg;
#pragma unroll
      for (int j = 0; j < NCB; ++j)
        *reinterpret_cast<float4*>(pacc + 16 * j) = make_float4(o[j][0], o[j][1], o[j][2], o[j][3]);
      if (cq == 0 && lg == 0)
        *reinterpret_cast<float2*>(ml + (slot * H + gh) * 2) = make_float2(m_run, l);
    }
  };

  // The tile of position gt - 1 (the segment's last) is finished after the
  // barrier of the next segment's query position, or after the final barrier.
  DecodeWork done = first;  // segment of the pending last tile
  bool pending = false;
#pragma unroll 1
  for (;;) {
    bf16x8_t ql[8], qr;
    const int ntile = (wk.n + TR - 1) / TR;  // the producers' count
    const int n = token_rows(wk, q_len, tok);  // rows this token sees
    {
      __syncthreads();  // the query tile is in LDS; the partials of gt - 1 are visible
      const char* st = lds + (gt % NST) * ST_BYTES;
      if (pending) {
        finish_alone(lds + ((gt - 1) % NST) * ST_BYTES, (gt - 1) & 1, (done.n - 1) / TR * TR,
                     token_rows(done, q_len, tok));
        store(done);
      }
      // Q^T fragments of head gh, columns 32 s + 8 lg .. + 7 for s = 8 hq + j
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = 8 * hq + j;
        const int off = lr * 1024 + 16 * ((4 * (s & 3) + lg) ^ lat_swz(lr)) + 256 * (s >> 2);
        ql[j] = *reinterpret_cast<const bf16x8_t*>(st + off);
      }
      qr = *reinterpret_cast<const bf16x8_t*>(st + ROPE_OFF + lr * 128 +
                                               16 * ((4 * hq + lg) ^ rope_swz(lr)));
      ++gt;
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int j = 0; j < NCB; ++j) o[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    __syncthreads();  // first row tile
    {
      PartIn pin;
      part_load(lds + (gt % NST) * ST_BYTES, pin);
      partial(pin, gt & 1, ql, qr);
    }
    ++gt;
#pragma unroll 1
    for (int k = 1; k < ntile; ++k, ++gt) {
      __syncthreads();  // tile gt is in LDS; the partials of tile gt - 1 are visible
      PartIn pin;
      FinIn fin;
      part_load(lds + (gt % NST) * ST_BYTES, pin);
      fin_load(lds + ((gt - 1) % NST) * ST_BYTES, (gt - 1) & 1, fin);
      __builtin_amdgcn_sched_barrier(0);  // keep every read of the position ahead of the math
      partial(pin, gt & 1, ql, qr);
      finish(fin, (k - 1) * TR, n, k * TR > n);  // a tile past the token's last row masks
    }
    pending = true;
    done = wk;
    if (wk.next < 0) break;
    wk = nx;
    if (wk.next >= 0) nx = load_work(works + wk.next);
  }
  __syncthreads();  // the partials of the last tile are visible
  finish_alone(lds + ((gt - 1) % NST) * ST_BYTES, (gt - 1) & 1, (done.n - 1) / TR * TR,
               token_rows(done, q_len, tok));
  store(done);
}

}  // namespace decr8

void decode_core_ring8(const bf16* q_cat, const uint8_t* cache, const DecodeMeta& m, int parts,
                       const TokenSplit& tk, float* acc, float* ml, bf16* o_lat, const Dims& d,
                       hipStream_t st) {
  const int hg = d.H / 16 * tk.q_len;
  const int blocks = (parts + decr8::kXcds - 1) / decr8::kXcds * decr8::kXcds * hg;
  decr8::decode_core_ring8_k<<<blocks, decr8::NTHR, 0, st>>>(q_cat, cache, m, acc, ml, o_lat,
                                                             d.H, parts, tk.q_len, tk.nseg_total);
}

}  // namespace mla
