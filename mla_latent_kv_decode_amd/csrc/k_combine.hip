// Split combine for a 512-wide latent (bf16 output).
//
// Each split j of sequence b left (m_j, l_j, acc_j) per head, with m_j the
// reference maximum in log2 units, l_j = sum_t 2^(s_t - m_j) and acc_j the
// matching unnormalised sum of latent rows.  The pages take one softmax over
// all cached rows ("Multi-Head Latent Attention" post, section 3.3
// Absorption); splitting the rows is this library's, and rescaling every split
// to the common maximum M recovers that softmax exactly:
//   o_lat = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j.
// Splits are summed in slot order, so the result does not depend on timing.
//
// Pass 1: one block per (sequence, head, chunk of kCombineChunk slots); its 4
// waves take every 4th slot of the chunk (all loads issued before the adds)
// and are summed through LDS in wave order.  A sequence whose slots fit one
// chunk is finished here; otherwise the chunk's (M, L, acc) goes to a chunk
// slot.  Pass 2 (only launched if some sequence has several chunks) merges the
// chunk slots of those sequences the same way.
#include "kernels.h"

namespace mla {
namespace cmb {

constexpr int DC = 512;
constexpr int JC = kCombineChunk;
constexpr int NW = 4;
constexpr int PER_WAVE = JC / NW;
static_assert(JC % NW == 0, "chunk must split evenly over the waves");

__device__ __forceinline__ void store_bf16x8(bf16* dst, const float* r, float inv) {
  uint4 pk;
  pk.x = pack_bf16x2(r[0] * inv, r[1] * inv);
  pk.y = pack_bf16x2(r[2] * inv, r[3] * inv);
  pk.z = pack_bf16x2(r[4] * inv, r[5] * inv);
  pk.w = pack_bf16x2(r[6] * inv, r[7] * inv);
  *reinterpret_cast<uint4*>(dst) = pk;
}

// lane owns columns 8 lane .. 8 lane + 7
__global__ void __launch_bounds__(256)
combine_chunks_512_k(const float* __restrict__ acc, const float* __restrict__ ml, DecodeMeta mt,
                     int H, float* __restrict__ cacc, float* __restrict__ cml,
                     bf16* __restrict__ o_lat, int chunked_only, int direct_single) {
  const int b = blockIdx.x, h = blockIdx.y, c = blockIdx.z;
  const int ns = mt.nseg[b];
  const int nch = (ns + JC - 1) / JC;
  // chunked_only = c: sequences of at most c chunks are merged by the consumer;
  // direct_single: the core wrote o_lat of one-segment sequences itself
  if (c >= nch || nch <= chunked_only || (direct_single && ns == 1)) return;
  const int j0 = mt.pstart[b] + c * JC;
  const int nj = min(JC, ns - c * JC);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ float4 red[NW][64][2];
  __shared__ float redl[NW];

  float M = -INFINITY;
  for (int j = 0; j < nj; ++j) M = fmaxf(M, ml[((int64_t)(j0 + j) * H + h) * 2]);
  float4 v[PER_WAVE][2];
  float w[PER_WAVE], l[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int jj = wave + NW * u;
    const int64_t idx = (int64_t)(j0 + min(jj, nj - 1)) * H + h;
    const float* p = acc + idx * DC + 8 * lane;
    v[u][0] = *reinterpret_cast<const float4*>(p);
    v[u][1] = *reinterpret_cast<const float4*>(p + 4);
    w[u] = jj < nj ? ml[idx * 2] : -INFINITY;
    l[u] = ml[idx * 2 + 1];
  }
  float r[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const float s = exp2f(w[u] - M);  // 0 for slots past the chunk
    L = fmaf(s, l[u], L);
    r[0] = fmaf(s, v[u][0].x, r[0]); r[1] = fmaf(s, v[u][0].y, r[1]);
    r[2] = fmaf(s, v[u][0].z, r[2]); r[3] = fmaf(s, v[u][0].w, r[3]);
    r[4] = fmaf(s, v[u][1].x, r[4]); r[5] = fmaf(s, v[u][1].y, r[5]);
    r[6] = fmaf(s, v[u][1].z, r[6]); r[7] = fmaf(s, v[u][1].w, r[7]);
  }
  red[wave][lane][0] = make_float4(r[0], r[1], r[2], r[3]);
  red[wave][lane][1] = make_float4(r[4], r[5], r[6], r[7]);
  if (lane == 0) redl[wave] = L;
  __syncthreads();
  if (wave != 0) return;
  L = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = 0.f;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    const float4 a = red[u][lane][0], e = red[u][lane][1];
    r[0] += a.x; r[1] += a.y; r[2] += a.z; r[3] += a.w;
    r[4] += e.x; r[5] += e.y; r[6] += e.z; r[7] += e.w;
    L += redl[u];
  }
  if (nch == 1) {
    store_bf16x8(o_lat + ((int64_t)b * H + h) * DC + 8 * lane, r, 1.f / L);
    return;
  }
  const int64_t k = (int64_t)(mt.cstart[b] + c) * H + h;
  float* q = cacc + k * DC + 8 * lane;
  *reinterpret_cast<float4*>(q) = make_float4(r[0], r[1], r[2], r[3]);
  *reinterpret_cast<float4*>(q + 4) = make_float4(r[4], r[5], r[6], r[7]);
  if (lane == 0) {
    cml[k * 2] = M;
    cml[k * 2 + 1] = L;
  }
}

// one wave per (sequence, head) with several chunks; lane owns 8 columns
__global__ void __launch_bounds__(64)
combine_final_512_k(const float* __restrict__ cacc, const float* __restrict__ cml, DecodeMeta mt,
                    int H, bf16* __restrict__ o_lat) {
  const int b = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int nch = (mt.nseg[b] + JC - 1) / JC;
  if (nch <= 1) return;
  const int k0 = mt.cstart[b];
  float M = -INFINITY;
  for (int k = 0; k < nch; ++k) M = fmaxf(M, cml[((int64_t)(k0 + k) * H + h) * 2]);
  float r[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int k = 0; k < nch; k += 4) {
    float4 v[4][2];
    float w[4], l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t idx = (int64_t)(k0 + min(k + u, nch - 1)) * H + h;
      const float* p = cacc + idx * DC + 8 * lane;
      v[u][0] = *reinterpret_cast<const float4*>(p);
      v[u][1] = *reinterpret_cast<const float4*>(p + 4);
      w[u] = k + u < nch ? cml[idx * 2] : -INFINITY;
      l[u] = cml[idx * 2 + 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float s = exp2f(w[u] - M);
      L = fmaf(s, l[u], L);
      r[0] = fmaf(s, v[u][0].x, r[0]); r[1] = fmaf(s, v[u][0].y, r[1]);
      r[2] = fmaf(s, v[u][0].z, r[2]); r[3] = fmaf(s, v[u][0].w, r[3]);
      r[4] = fmaf(s, v[u][1].x, r[4]); r[5] = fmaf(s, v[u][1].y, r[5]);
      r[6] = fmaf(s, v[u][1].z, r[6]); r[7] = fmaf(s, v[u][1].w, r[7]);
    }
  }
  store_bf16x8(o_lat + ((int64_t)b * H + h) * DC + 8 * lane, r, 1.f / L);
}

// ---- combine fused with the value un-absorb (dc = 512, dv = 128)
//
// Block (head h, group of SB sequences), 8 waves.  Phase 1: the partials of
// each sequence of the group are merged by WPS waves (1, or 8 / SB; lane:
// columns 8 lane .. + 7); sub-wave k takes slots k, k + WPS, .. (up to 8 slots
// per round with all their loads in flight), and the sub-waves' (max, sum,
// latent sum) are then merged in sub-wave order through LDS.  A sequence is
// merged from the core's slots when it has at most JC * WPS of them, else from
// the chunk slots the first pass left.  Sequences the core finished itself are
// read back from o_lat.  The rows o_lat_h (bf16) go to LDS and to o_lat.
// Phase 2 ("Multi-Head Latent Attention" post, eq. 3.3.3: W_UV after the
// softmax-weighted latent sum): o_h (SB x 128) = o_lat_h (SB x 512) W_UV_h^T
// with mfma 16x16x32, A from LDS, B = W_UV_h rows (K-contiguous) fetched into
// VGPRs at kernel start, while phase 1 runs (rows SB .. 15 of the MFMA row
// block are zero).  Wave w owns output columns 16 w .. 16 w + 15; o is rounded
// to bf16.
constexpr int SB_MAX = 16;             // sequences per block: 16, 8 or 4 to fill the compute units
constexpr int UV_NW = 8;               // waves
constexpr int UV_DV = 128;
constexpr int OROW = DC * 2 + 16;      // LDS row stride in bytes (padding: no bank conflicts)
constexpr int MB = 8;                  // slots merged per round

// merged (unnormalised) sums r over slots j0, j0 + js, .., j0 + (nj - 1) js,
// their total L and common reference maximum M (-inf, 0, 0 for no slots)
__device__ __forceinline__ void merge_slots(const float* __restrict__ a, const float* __restrict__ m,
                                            int j0, int js, int nj, int H, int h, int lane, float* r,
                                            float* Lout, float* Mout) {
  float M = -INFINITY, L = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = 0.f;
  for (int j = 0; j < nj; j += MB) {
    float4 v[MB][2];
    float2 w[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int64_t idx = (int64_t)(j0 + js * min(j + u, nj - 1)) * H + h;
      const float* p = a + idx * DC + 8 * lane;
      v[u][0] = *reinterpret_cast<const float4*>(p);
      v[u][1] = *reinterpret_cast<const float4*>(p + 4);
      w[u] = *reinterpret_cast<const float2*>(m + idx * 2);
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < MB; ++u) Mn = fmaxf(Mn, w[u].x);  // repeats of the last slot change nothing
    const float g = exp2f(M - Mn);  // 0 on the first round
    L *= g;
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] *= g;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const float s = j + u < nj ? exp2f(w[u].x - Mn) : 0.f;
      L = fmaf(s, w[u].y, L);
      r[0] = fmaf(s, v[u][0].x, r[0]); r[1] = fmaf(s, v[u][0].y, r[1]);
      r[2] = fmaf(s, v[u][0].z, r[2]); r[3] = fmaf(s, v[u][0].w, r[3]);
      r[4] = fmaf(s, v[u][1].x, r[4]); r[5] = fmaf(s, v[u][1].y, r[5]);
      r[6] = fmaf(s, v[u][1].z, r[6]); r[7] = fmaf(s, v[u][1].w, r[7]);
    }
    M = Mn;
  }
  *Lout = L;
  *Mout = M;
}

// MULTI: UV_NW / SB waves per sequence (SB < UV_NW), else one
template <bool MULTI>
__global__ void __launch_bounds__(UV_NW * 64)
combine_uv_k(const float* __restrict__ acc, const float* __restrict__ ml,
             const float* __restrict__ cacc, const float* __restrict__ cml, DecodeMeta mt,
             int direct_single, const bf16* __restrict__ w_uv, int B, int H,
             bf16* __restrict__ o_lat, bf16* __restrict__ o, int SB) {
  __shared__ __attribute__((aligned(16))) char rows[16 * OROW];
  __shared__ float4 xr[MULTI ? UV_NW : 1][64][2];  // sub-waves' latent sums
  __shared__ float2 xml[UV_NW];                    // and their (max, sum)
  const int h = blockIdx.x, b0 = blockIdx.y * SB;  // SB <= SB_MAX sequences
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;

  // W_UV_h fragments of this wave's column block, all 16 k-steps
  bf16x8_t wf[16];
  {
    const bf16* wb = w_uv + ((int64_t)h * UV_DV + 16 * wave + lr) * DC + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) wf[ks] = *reinterpret_cast<const bf16x8_t*>(wb + 32 * ks);
  }

  if constexpr (MULTI) {
    // rows SB .. 15 of the product's row block are zero
    for (int e = threadIdx.x; e < (16 - SB) * 64; e += UV_NW * 64)
      *reinterpret_cast<uint4*>(rows + (SB + e / 64) * OROW + 16 * (e % 64)) = make_uint4(0u, 0u, 0u, 0u);

    // phase 1: o_lat rows of the group's sequences, wps = UV_NW / SB waves per
    // sequence
    const int wps = UV_NW / SB;
    const int k = wave % wps;
    for (int i = wave / wps; i < SB; i += UV_NW / wps) {  // the same trip count in every wave
      const int b = b0 + i;
      bf16* og = o_lat + ((int64_t)b * H + h) * DC + 8 * lane;
      const int ns = b < B ? mt.nseg[b] : 0;
      const bool copy = direct_single && ns == 1;  // the core wrote this row
      float r[8], L = 0.f, M = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = 0.f;
      if (b < B && !copy) {
        if (ns <= JC * wps)
          merge_slots(acc, ml, mt.pstart[b] + k, wps, (ns - k + wps - 1) / wps, H, h, lane, r, &L, &M);
        else {
          const int nch = (ns + JC - 1) / JC;
          merge_slots(cacc, cml, mt.cstart[b] + k, wps, (nch - k + wps - 1) / wps, H, h, lane, r, &L,
                      &M);
        }
      }
      xr[wave][lane][0] = make_float4(r[0], r[1], r[2], r[3]);
      xr[wave][lane][1] = make_float4(r[4], r[5], r[6], r[7]);
      if (lane == 0) xml[wave] = make_float2(M, L);
      __syncthreads();
      if (k == 0 && b < B && !copy) {
        float Mt = -INFINITY;
        for (int q = 0; q < wps; ++q) Mt = fmaxf(Mt, xml[wave + q].x);
        L = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = 0.f;
        for (int q = 0; q < wps; ++q) {  // sub-wave order
          const float2 mlq = xml[wave + q];
          const float s = mlq.x == -INFINITY ? 0.f : exp2f(mlq.x - Mt);
          L = fmaf(s, mlq.y, L);
          const float4 a0 = xr[wave + q][lane][0], a1 = xr[wave + q][lane][1];
          r[0] = fmaf(s, a0.x, r[0]); r[1] = fmaf(s, a0.y, r[1]);
          r[2] = fmaf(s, a0.z, r[2]); r[3] = fmaf(s, a0.w, r[3]);
          r[4] = fmaf(s, a1.x, r[4]); r[5] = fmaf(s, a1.y, r[5]);
          r[6] = fmaf(s, a1.z, r[6]); r[7] = fmaf(s, a1.w, r[7]);
        }
      }
      if (k != 0) continue;
      uint4* dst = reinterpret_cast<uint4*>(rows + i * OROW + 16 * lane);
      if (b >= B) {
        *dst = make_uint4(0u, 0u, 0u, 0u);
      } else if (copy) {
        *dst = *reinterpret_cast<const uint4*>(og);
      } else {
        const float inv = 1.f / L;
        uint4 pk;
        pk.x = pack_bf16x2(r[0] * inv, r[1] * inv);
        pk.y = pack_bf16x2(r[2] * inv, r[3] * inv);
        pk.z = pack_bf16x2(r[4] * inv, r[5] * inv);
        pk.w = pack_bf16x2(r[6] * inv, r[7] * inv);
        *dst = pk;
        *reinterpret_cast<uint4*>(og) = pk;
      }
    }
    __syncthreads();
  } else {
    // phase 1: o_lat rows of the group's sequences
    for (int i = wave; i < 16; i += UV_NW) {
      const int b = b0 + i;
      uint4* dst = reinterpret_cast<uint4*>(rows + i * OROW + 16 * lane);
      if (i >= SB || b >= B) {
        *dst = make_uint4(0u, 0u, 0u, 0u);
        continue;
      }
      bf16* og = o_lat + ((int64_t)b * H + h) * DC + 8 * lane;
      const int ns = mt.nseg[b];
      if (direct_single && ns == 1) {
        *dst = *reinterpret_cast<const uint4*>(og);
        continue;
      }
      float r[8], L, M;
      if (ns <= JC) merge_slots(acc, ml, mt.pstart[b], 1, ns, H, h, lane, r, &L, &M);
      else merge_slots(cacc, cml, mt.cstart[b], 1, (ns + JC - 1) / JC, H, h, lane, r, &L, &M);
      const float inv = 1.f / L;
      uint4 pk;
      pk.x = pack_bf16x2(r[0] * inv, r[1] * inv);
      pk.y = pack_bf16x2(r[2] * inv, r[3] * inv);
      pk.z = pack_bf16x2(r[4] * inv, r[5] * inv);
      pk.w = pack_bf16x2(r[6] * inv, r[7] * inv);
      *dst = pk;
      *reinterpret_cast<uint4*>(og) = pk;
    }
    __syncthreads();
  }

  // phase 2: o (SB x 128) = o_lat_h (SB x 512) . W_UV_h^T, this wave's 16 columns
  f32x4_t d0 = (f32x4_t){0.f, 0.f, 0.f, 0.f}, d1 = d0;
  const char* arow = rows + lr * OROW + 16 * lg;
#pragma unroll
  for (int ks = 0; ks < 16; ks += 2) {
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(arow + 64 * ks),
                                                 wf[ks], d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        *reinterpret_cast<const bf16x8_t*>(arow + 64 * (ks + 1)), wf[ks + 1], d1, 0, 0, 0);
  }
  const f32x4_t d = d0 + d1;
  // lane holds rows 4 lg + i of column 16 wave + lr
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = b0 + 4 * lg + i;
    if (4 * lg + i < SB && b < B) o[(int64_t)b * H * UV_DV + h * UV_DV + 16 * wave + lr] = f32_to_bf16(d[i]);
  }
}

}  // namespace cmb

void decode_combine_512(const float* acc, const float* ml, const DecodeMeta& m, int B, int H,
                        int max_chunks, float* cacc, float* cml, bool direct_single,
                        bf16* o_lat, hipStream_t st) {
  cmb::combine_chunks_512_k<<<dim3(B, H, max_chunks), 256, 0, st>>>(acc, ml, m, H, cacc, cml,
                                                                      o_lat, 0, direct_single);
  if (max_chunks > 1)
    cmb::combine_final_512_k<<<dim3(B, H), 64, 0, st>>>(cacc, cml, m, H, o_lat);
}

// A6 + A7 with the split combine's first pass only for sequences with more
// than kCombineChunk partials.
void decode_combine_uv(const float* acc, const float* ml, const DecodeMeta& m, int B, int H,
                       int max_chunks, float* cacc, float* cml, bool direct_single,
                       const bf16* w_uv, bf16* o_lat, bf16* o, hipStream_t st) {
  // the most sequences per block (16, 8, 4, 2, else 1) that still give a
  // block per compute unit: each block reads its head's whole W_UV, so fewer,
  // taller blocks read less (and fill more of the 16-row product); more
  // blocks spread the reads over more compute units.  With fewer than 8
  // sequences per block and some sequence with more than 16 partials, 8 / sb
  // waves merge each sequence's partials, so a sequence of up to 16 * 8 / sb
  // partials needs no first pass (with at most 16 partials one wave per
  // sequence is faster: measured 7.0 against 9.4 us at 64 sequences of ~5).
  int sb = cmb::SB_MAX;
  while (sb > 1 && (int64_t)H * ((B + sb - 1) / sb) < device_cu_count()) sb /= 2;
  const int wps = sb >= cmb::UV_NW || max_chunks <= 1 ? 1 : cmb::UV_NW / sb;
  if (max_chunks > wps)
    cmb::combine_chunks_512_k<<<dim3(B, H, max_chunks), 256, 0, st>>>(acc, ml, m, H, cacc, cml,
                                                                        o_lat, wps, 0);
  if (wps > 1)
    cmb::combine_uv_k<true><<<dim3(H, (B + sb - 1) / sb), cmb::UV_NW * 64, 0, st>>>(
        acc, ml, cacc, cml, m, direct_single ? 1 : 0, w_uv, B, H, o_lat, o, sb);
  else
    cmb::combine_uv_k<false><<<dim3(H, (B + sb - 1) / sb), cmb::UV_NW * 64, 0, st>>>(
        acc, ml, cacc, cml, m, direct_single ? 1 : 0, w_uv, B, H, o_lat, o, sb);
}

}  // namespace mla
