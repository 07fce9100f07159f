// Split-S latent attention core for layers whose heads come in a few 16-head
// groups (DeepSeek-V2-Lite: 16 heads).
//
// Absorbed decode ("Multi-Head Latent Attention" post, sections 3.3 and 3.6):
// per head h, s_h,t = q_cat_h . row_t over all 576 columns of the cached row
// [c_kv (512) | k_rope (64)], a softmax over t, and the latent sum
// sum_t p_h,t c_t over the 512 c_kv columns.
//
// Work: the host cuts the concatenated rows of the batch into one contiguous
// span per persistent workgroup and splits spans at sequence boundaries into
// segments (chained work records).  A workgroup covers one 16-head group; the
// workgroups of the other groups of a span run on the same XCD and stream the
// same rows through its L2.
//
// Waves: two producer waves issue every tile copy (global_load_lds_dwordx4,
// 18 of the 36 one-KB copies of a 32-row tile each) into a 4-stage LDS ring
// and keep three tiles in flight, across segment boundaries too: a segment's
// stream is a query tile (the group's 16 q_cat rows, copied like cache rows)
// followed by its row tiles.  Four consumer waves compute.  One barrier per
// tile publishes it and frees the stage the next copy refills.
//
// Each consumer wave computes the scores and the softmax of all 16 heads (the
// same in the four waves) and the latent sum of its quarter of the 512
// columns, so a segment needs no cross-wave merge.  Per 32-row tile and wave:
//   S^T (rows x heads) = K . Q^T: 2 x 18 mfma 16x16x32 (one per 16-row block
//     and 32 columns), K fragments read from LDS (row l%16, 8 columns per
//     lane), Q^T in VGPRs.  Lane l ends with rows 4(l/16)..+3 of both row
//     blocks for head l%16.
//   softmax in log2 units with a lazy reference maximum (it moves only when a
//     score exceeds it by 2^8), running sums per lane.
//   O^T (128 columns x 16 heads) += C^T . P^T: 8 mfma 16x16x32.  Their k index
//     runs over rows 4g..4g+3 of row block 0, then of row block 1, for lane
//     group g, which is exactly how the lanes hold P; C^T comes from two
//     transposing LDS reads (ds_read_b64_tr_b16) per 16-column block.
//
// Outputs: a sequence that fits one segment is normalised and written to o_lat
// directly; otherwise the segment leaves a partial (reference max in log2
// units, sum, unnormalised latent sum) for the combine, which rescales the
// partials of a sequence to their common maximum and so recovers the single
// softmax the pages take over all rows.
#include <utility>

#include "decode_dev.h"

namespace mla {
namespace decr {

using namespace ddev;

constexpr int DC = 512;
constexpr int RW = 576;                      // row width in elements
constexpr int TR = 32;                       // rows per tile
constexpr int NST = 4;                       // ring stages
constexpr int ROPE_OFF = TR * 1024;          // latent of row r at r*1024, rope after
constexpr int ST_BYTES = TR * RW * 2;        // 36 KB
constexpr int NLOAD = TR + TR / 8;           // one-KB copies per tile
constexpr int NPROD = 2;                     // producer waves
constexpr int LPW = NLOAD / NPROD;           // copies per producer wave and tile
constexpr int NCONS = 4;                     // consumer waves = column quarters
constexpr int NCB1 = 32 / NCONS;             // 16-column blocks per consumer wave (one token)
constexpr int NTHR = 64 * (NCONS + NPROD);
constexpr float kRescale = 8.0f;
constexpr int kXcds = 8;
static_assert(NLOAD % NPROD == 0, "tile copies split evenly over the producers");
static_assert((NST - 2) * LPW <= 63, "copies in flight fit the vmcnt field");
static_assert(ROPE_OFF + TR * 128 == ST_BYTES, "stage layout");

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// Copy I of a tile whose first row is at `base` and whose last valid row is
// `last`: I < 32 copies the latent part of row I, I >= 32 the rope parts of
// rows 8(I-32) .. +7.  Rows past `last` re-read it (their scores are masked).
// jump16: bytes added to the address of rows 16 .. 31 (a query tile holding
// two tokens' 16 heads: their q_cat rows are H rows apart; 0 for cache tiles)
template <int I, bool NT>
__device__ __forceinline__ void tile_copy(const char* base, int last, uint32_t stage, int lane,
                                          int jump16) {
  if constexpr (I < TR) {
    const int r = I <= last ? I : last;
    dma16h<NT>(base + r * (RW * 2) + (r >= 16 ? jump16 : 0) + ((lane ^ lat_swz(I & 15)) << 4),
          stage + I * 1024);
  } else {
    constexpr int J = I - TR;
    int r = 8 * J + (lane >> 3);
    const int cc = (lane & 7) ^ rope_swz(r & 15);
    r = r <= last ? r : last;
    dma16h<NT>(base + r * (RW * 2) + (r >= 16 ? jump16 : 0) + 1024 + (cc << 4),
          stage + ROPE_OFF + J * 1024);
  }
}

template <int P, bool NT, int... U>
__device__ __forceinline__ void producer_copies(const char* base, int last, uint32_t stage,
                                                int lane, int jump16,
                                                std::integer_sequence<int, U...>) {
  (tile_copy<P * LPW + U, NT>(base, last, stage, lane, jump16), ...);
}

// NT: the non-temporal copy (cache rows no other workgroup of the part reads)
template <bool NT>
__device__ __forceinline__ void issue_tile(const char* base, int last, uint32_t stage, int p,
                                           int lane, int jump16 = 0) {
  const auto seq = std::make_integer_sequence<int, LPW>{};
  if (p == 0) producer_copies<0, NT>(base, last, stage, lane, jump16, seq);
  else producer_copies<1, NT>(base, last, stage, lane, jump16, seq);
}

__device__ __forceinline__ bf16x8_t cat_bf16(s16x4_t lo, s16x4_t hi) {
  const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// TOK tokens per workgroup: 1, or 2 (a pair of a sequence's new tokens: the
// query tile holds both tokens' 16 heads, consumer wave w takes token w >> 1
// and half w & 1 of the latent columns, so the part's rows stream once for
// both)
template <int TOK>
__global__ void __launch_bounds__(NTHR, 1)
decode_core_ring_k(const bf16* __restrict__ q_cat, const bf16* __restrict__ cache, DecodeMeta mt,
                   float* __restrict__ acc, float* __restrict__ ml, bf16* __restrict__ o_lat,
                   int H, int nparts, int q_len, int nseg_total) {
  __shared__ __attribute__((aligned(1024))) char lds[NST * ST_BYTES];
  // block -> (part, token group, head group); the groups of a part are
  // numbered part % 8 modulo 8, so they share an XCD (blocks go to XCDs round
  // robin)
  constexpr int NCB = NCB1 * TOK;  // 16-column blocks per consumer wave
  const int HG = H / 16;
  const int NG = HG * q_len / TOK;
  const int bid = blockIdx.x;
  const int part = (bid / (kXcds * NG)) * kXcds + bid % kXcds;
  const int g = (bid / kXcds) % NG;
  const int tok0 = TOK * (g / HG), hg = g % HG;  // first token of the group
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
    int ik = 0, intl = 1 + (iw.n + TR - 1) / TR;  // next tile of segment iw, its tile count
    int issued = 0;
    int64_t next_row = 0;
    // issue the next tile of the part's stream (query tile, then row tiles,
    // segment after segment) into stage issued % NST
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
        const char* qb = reinterpret_cast<const char*>(
            q_cat + ((int64_t)(iw.b * q_len + tok0) * H + hg * 16) * RW);
        issue_tile<false>(qb, 16 * TOK - 1, stage, p, lane, (H - 16) * RW * 2);
      } else {
        const int t = ik - 1;
        const char* rb = reinterpret_cast<const char*>(cache + next_row * RW);
        if (NG == 1) issue_tile<true>(rb, iw.n - t * TR - 1, stage, p, lane);
        else issue_tile<false>(rb, iw.n - t * TR - 1, stage, p, lane);
      }
      // the cache row of the segment's next tile, one issue ahead (a paged
      // cache's page lookup is a load)
      if (ik + 1 < intl) next_row = seg_row(mt, iw.row, ik * TR);
      ++ik;
      ++issued;
    };
#pragma unroll 1
    for (int i = 0; i < NST - 1; ++i) issue_next();
    static_assert(NST == 4, "the waits below assume at most two tiles issued after the awaited one");
#pragma unroll 1
    for (int gt = 0; gt < issued; ++gt) {
      const int ahead = issued - gt - 1;  // tiles issued after tile gt
      if (ahead >= 2) wait_vmcnt<2 * LPW>();
      else if (ahead == 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      __syncthreads();  // tile gt is in LDS; the consumers are done with tile gt - 1
      if (issued == gt + NST - 1) issue_next();  // refills the stage of tile gt - 1
    }
    return;
  }

  // -------------------------------------------------------------- consumers
  // this wave's token and columns: 16 NCB cq .. 16 NCB (cq + 1) - 1
  const int tw = TOK == 2 ? wave >> 1 : 0, cq = TOK == 2 ? wave & 1 : wave;
  const int tok = tok0 + tw;
  const int qrow = 16 * tw;  // the token's rows in the query tile
  const int lr = lane & 15, lg = lane >> 4;
  // row-wise operand of k-step s < 16 in a 16-row block: row lr, chunk 4s + lg,
  // at qk_off[s & 3] + 256 (s >> 2); rope chunk 4(s - 16) + lg at qk_rope[s - 16]
  int qk_off[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) qk_off[k] = lr * 1024 + 16 * ((4 * k + lg) ^ lat_swz(lr));
  const int qk_rope0 = ROPE_OFF + lr * 128 + 16 * (lg ^ rope_swz(lr));
  const int qk_rope1 = ROPE_OFF + lr * 128 + 16 * ((4 + lg) ^ rope_swz(lr));
  // transposing operand of column block cb = 4q + t in a 16-row block: lane
  // (g = lg, s = lr) addresses row r = 4g + s/4, columns 16 cb + 4(s % 4):
  // chunk 2cb + h with h = (s % 4) / 2, byte 8(s & 1).  Its position
  // 2(cb ^ a) + (h ^ b) (a = r & 7, b = r >> 3) puts it at pv_e[t] + 128q for
  // even q and pv_e[t] - pv_d + 128q for odd q.
  int pv_e[4], pv_d;
  {
    const int r = 4 * lg + (lr >> 2);
    const int a = r & 7, b = (r >> 3) & 1, h = (lr & 3) >> 1;
    pv_d = 256 * (a >> 2);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      pv_e[t] = r * 1024 + 16 * (h ^ b) + 8 * (lr & 1) + 32 * (t ^ (a & 3)) + 128 * (a >> 2);
  }
  const int gh = hg * 16 + lr;  // this lane's head in the score and sum layouts

  DecodeWork wk = first, nx = first;
  if (wk.next >= 0) nx = load_work(works + wk.next);
  int gt = 0;
#pragma unroll 1
  for (;;) {
    bf16x8_t qf[18];
    float m_run, l_run;
    f32x4_t o[NCB];
    const int ntile = (wk.n + TR - 1) / TR;  // the producers' count
    const int n = token_rows(wk, q_len, tok);  // rows this token sees
    {
      // the segment's query tile: Q^T fragments of head gh, columns 32 s + 8 lg .. + 7
      __syncthreads();
      const char* st = lds + (gt % NST) * ST_BYTES;
#pragma unroll
      for (int s = 0; s < 16; ++s)
        qf[s] = *reinterpret_cast<const bf16x8_t*>(st + qrow * 1024 + qk_off[s & 3] +
                                                    256 * (s >> 2));
      qf[16] = *reinterpret_cast<const bf16x8_t*>(st + qrow * 128 + qk_rope0);
      qf[17] = *reinterpret_cast<const bf16x8_t*>(st + qrow * 128 + qk_rope1);
      ++gt;
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int j = 0; j < NCB; ++j) o[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int k = 0; k < ntile; ++k, ++gt) {
      __syncthreads();  // tile gt is in LDS
      const char* st = lds + (gt % NST) * ST_BYTES;
      const int row0 = k * TR;
      // ---- S^T = K . Q^T for both 16-row blocks
      f32x4_t sc[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const char* sl = st + rb * 16 * 1024;
        const char* sr = st + rb * 16 * 128;  // rope offsets include ROPE_OFF
        bf16x8_t kf[18];
#pragma unroll
        for (int s = 0; s < 16; ++s)
          kf[s] = *reinterpret_cast<const bf16x8_t*>(sl + qk_off[s & 3] + 256 * (s >> 2));
        kf[16] = *reinterpret_cast<const bf16x8_t*>(sr + qk_rope0);
        kf[17] = *reinterpret_cast<const bf16x8_t*>(sr + qk_rope1);
        f32x4_t sa = (f32x4_t){0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
        for (int s = 0; s < 18; s += 2) {
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s + 1], qf[s + 1], sb, 0, 0, 0);
        }
        sc[rb] = sa + sb;
      }
      // ---- online softmax: lane holds rows row0 + 16 rb + 4 lg + i of head gh
      float sv[8];
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = row0 + 16 * rb + 4 * lg + i < n;
          sv[4 * rb + i] = valid ? sc[rb][i] * kLog2e : -INFINITY;
          grow |= sv[4 * rb + i] > m_run + kRescale;
        }
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
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_run);
        l_run += pv[i];
      }
      bf16x8_t pf;
      {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
        pf = __builtin_bit_cast(bf16x8_t, pk);
      }
      // ---- O^T += C^T . P^T over this wave's column blocks 8 cq .. 8 cq + 7
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        const int q = NCB / 4 * cq + j / 4, t = j % 4;
        const int off = pv_e[t] - (q & 1) * pv_d + 128 * q;
        typedef __attribute__((address_space(3))) s16x4_t* lptr;
        const s16x4_t c0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(st + off));
        const s16x4_t c1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(st + 16 * 1024 + off));
        o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat_bf16(c0, c1), pf, o[j], 0, 0, 0);
      }
    }

    // ---- end of the segment: lane holds columns 128 cq + 16 j + 4 lg .. +3 of head gh
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int b = wk.b;
    if (wk.nseg == 1) {
      const float inv = 1.f / l;
      bf16* dst = o_lat + ((int64_t)(b * q_len + tok) * H + gh) * DC + 16 * NCB * cq + 4 * lg;
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        uint2 pk;
        pk.x = pack_bf16x2(o[j][0] * inv, o[j][1] * inv);
        pk.y = pack_bf16x2(o[j][2] * inv, o[j][3] * inv);
        *reinterpret_cast<uint2*>(dst + 16 * j) = pk;
      }
    } else {
      // partial of this segment: unnormalised sums (this wave's quarter) and,
      // from the first wave, the (max, sum) pair of each head
      const int64_t slot = (int64_t)tok * nseg_total + wk.pidx;
      float* pacc = acc + (slot * H + gh) * DC + 16 * NCB * cq + 4 * lg;
#pragma unroll
      for (int j = 0; j < NCB; ++j)
        *reinterpret_cast<float4*>(pacc + 16 * j) = make_float4(o[j][0], o[j][1], o[j][2], o[j][3]);
      if (cq == 0 && lg == 0)
        *reinterpret_cast<float2*>(ml + (slot * H + gh) * 2) = make_float2(m_run, l);
    }
    if (wk.next < 0) break;
    wk = nx;
    if (wk.next >= 0) nx = load_work(works + wk.next);
  }
}

}  // namespace decr

int decode_core_ring_tokens(int q_len) { return q_len % 2 == 0 ? 2 : 1; }

void decode_core_ring(const bf16* q_cat, const bf16* cache, const DecodeMeta& m, int parts,
                      const TokenSplit& tk, float* acc, float* ml, bf16* o_lat, const Dims& d,
                      hipStream_t st) {
  const int tok = decode_core_ring_tokens(tk.q_len);
  const int ng = d.H / 16 * tk.q_len / tok;
  const int blocks = (parts + decr::kXcds - 1) / decr::kXcds * decr::kXcds * ng;
  if (tok == 2)
    decr::decode_core_ring_k<2><<<blocks, decr::NTHR, 0, st>>>(q_cat, cache, m, acc, ml, o_lat,
                                                               d.H, parts, tk.q_len, tk.nseg_total);
  else
    decr::decode_core_ring_k<1><<<blocks, decr::NTHR, 0, st>>>(q_cat, cache, m, acc, ml, o_lat,
                                                               d.H, parts, tk.q_len, tk.nseg_total);
}

}  // namespace mla
