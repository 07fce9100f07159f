// Split-S latent attention core on CDNA4 MFMA (bf16 in, fp32 accumulate).
//
// Absorbed decode ("Multi-Head Latent Attention" post, section 3.3 and 3.6):
// per head h, s_h,t = q_cat_h . row_t over all 576 columns of the cached row
// [c_kv (512) | k_rope (64)], online softmax over t, and the latent sum
// acc_h += p_h,t * c_t (512 columns).  Each latent row is read from HBM once
// and used by all 16 heads of a head group: the head dimension is the M = 16
// side of one MFMA, so one wave covers a whole head group.
//
// Work decomposition: the host cuts the concatenated rows of all sequences
// into `parts` equal spans (one persistent workgroup each) and splits spans at
// sequence boundaries into segments.  Inside a workgroup the 4 waves take
// 16-row sub-tiles of the segment round-robin, each with its own online
// softmax state and a private double-buffered LDS stage filled by
// global_load_lds_dwordx4 (no VGPRs held by loads in flight).  At the end of a
// segment the 4 wave states are merged through LDS and one partial
// (max, sum, unnormalised acc) is written; the combine kernel merges partials
// of a sequence in a fixed order.
//
// Per 16-row sub-tile and wave:
//   S^T (16 rows x 16 heads) = K (16 x 576) . Q^T   -- 18 x mfma 16x16x32,
//       A = K fragments read from LDS (row l%16, 8 columns), B = Q in VGPRs;
//       lane l ends with rows 4(l/16)..+3 of head l%16.
//   softmax: per head = per lane column; max/sum across the 4 lane groups by
//       two xor-shuffles.
//   O^T (512 cols x 16 heads) += C^T (512 x 16 rows) . P^T (16 rows x 16 heads)
//       -- 32 x mfma 16x16x16; B = P exactly as S^T left it; A = C^T built from
//       4 x 16-byte LDS reads (4 rows x 8 columns) and a 4x8 bf16 transpose
//       in registers, giving fragments for 8 MFMAs (column 8c + j of chunk c).
#include "kernels.h"

namespace mla {
namespace dec {

constexpr int DC = 512;
constexpr int RW = 576;                      // row width in elements
constexpr int SUB = 16;                      // rows per sub-tile
constexpr int SUB_BYTES = SUB * RW * 2;      // 18432
constexpr int LOADS = SUB + 2;               // 18 wave-wide 16-byte loads per sub-tile
constexpr int NWAVE = 4;
constexpr int NSTAGE = 2;
constexpr int LDS_BYTES = NWAVE * NSTAGE * SUB_BYTES;  // 147456
static_assert(NWAVE * 16 * DC * 4 + NWAVE * 16 * 2 * 4 <= LDS_BYTES, "merge space");

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Stage layout (18 KB for 16 rows): the latent part of row r (64 chunks of 16
// bytes) at byte r*1024, the rope part (8 chunks) at 16384 + r*128.  Chunk c
// of a row is stored at position c ^ (r & 7) inside its aligned group of 8:
// 8 consecutive rows read at one column hit 8 different bank groups.
constexpr int ROPE_OFF = SUB * 1024;
static_assert(ROPE_OFF + SUB * 128 == SUB_BYTES, "stage layout");

// One wave-wide 16-byte-per-lane copy global -> LDS.  The LDS destination is
// M0 + 16 * lane (a 1 KB block per instruction).  Issued from inline asm so the
// compiler neither reorders it nor adds its own (conservative) waits; the
// kernel waits with explicit s_waitcnt vmcnt.  SALU write of M0 needs one wait
// state before an LDS-DMA load.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// 18 loads per 16-row sub-tile: load i < 16 copies the latent part of row i
// (lane = physical chunk, source chunk lane ^ (i & 7)); loads 16 and 17 copy
// the rope parts of rows 8j + lane/8.  Rows at or past `nvalid` re-read the
// last valid row (their scores are masked).
__device__ __forceinline__ void issue_subtile(const bf16* rows, int row0, int n,
                                              uint32_t stage_addr, int lane) {
  const char* base = reinterpret_cast<const char*>(rows + (int64_t)row0 * RW);
  const int last = n - row0 - 1;
#pragma unroll
  for (int i = 0; i < SUB; ++i) {
    const int r = i <= last ? i : last;
    dma16(base + r * (RW * 2) + ((lane ^ (i & 7)) << 4), stage_addr + i * 1024);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int r = 8 * j + (lane >> 3);
    const int cc = (lane & 7) ^ (lane >> 3);
    r = r <= last ? r : last;
    dma16(base + r * (RW * 2) + 1024 + (cc << 4), stage_addr + ROPE_OFF + j * 1024);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__global__ void __launch_bounds__(256, 1)
decode_core_mfma_k(const bf16* __restrict__ q_cat, const bf16* __restrict__ cache, DecodeMeta mt,
                   float* __restrict__ acc_out, float* __restrict__ ml_out, int H) {
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  const int part = blockIdx.x;
  const int hg = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  char* my = lds + wave * NSTAGE * SUB_BYTES;
  const uint32_t my_addr = lds_u32(my);
  // QK operand of k-step s: row lr, columns 32s + 8lg .. +7.  Latent chunk
  // 4s + lg (s < 16) sits at lr*1024 + 16*((4s + lg) ^ (lr & 7)) =
  // base(s & 1) + 128*(s >> 1) with b = bit 2 of lr selecting the order of each
  // even/odd pair; rope chunk 4(s-16) + lg at ROPE_OFF + lr*128 + 16*((...) ^ (lr & 7)).
  const int qk_b = (lr >> 2) & 1;
  const int qk_lo = (lg ^ (lr & 3)) * 16;
  const int qk_base0 = lr * 1024 + 64 * qk_b + qk_lo;          // even s
  const int qk_base1 = lr * 1024 + 64 * (qk_b ^ 1) + qk_lo;    // odd s
  const int qk_rope0 = ROPE_OFF + lr * 128 + 64 * qk_b + qk_lo;        // s = 16
  const int qk_rope1 = ROPE_OFF + lr * 128 + 64 * (qk_b ^ 1) + qk_lo;  // s = 17
  // PV operand: row r = 4lg + i, latent chunk 16cb + lr at r*1024 + 256cb + 16(lr ^ (r & 7))
  int pv_base[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * lg + i;
    pv_base[i] = r * 1024 + 16 * (lr ^ (r & 7));
  }

  const int sbeg = mt.part_begin[part], send = mt.part_begin[part + 1];
  for (int si = sbeg; si < send; ++si) {
    const DecodeSeg sg = mt.segs[si];
    const int n = sg.r1 - sg.r0;
    const int nsub = (n + SUB - 1) / SUB;
    const bf16* rows = cache + (mt.seq_off[sg.b] + sg.r0) * (int64_t)RW;

    // this wave's sub-tiles: wave, wave + 4, ...
    const int my_n = wave < nsub ? (nsub - 1 - wave) / NWAVE + 1 : 0;
    if (my_n > 0) issue_subtile(rows, wave * SUB, n, my_addr, lane);
    if (my_n > 1) issue_subtile(rows, (wave + NWAVE) * SUB, n, my_addr + SUB_BYTES, lane);

    // Q^T fragments of head (hg*16 + lr): columns 32 s + 8 lg .. + 7
    bf16x8_t qf[18];
    {
      const bf16* qrow = q_cat + ((int64_t)sg.b * H + hg * 16 + lr) * RW + lg * 8;
#pragma unroll
      for (int s = 0; s < 18; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * s);
      // Consume the Q loads here so the compiler's own waits for them sit before
      // the loop: inside it the only loads in flight are the stage prefetches,
      // which are waited for explicitly.
#pragma unroll
      for (int s = 0; s < 18; ++s) asm volatile("" ::"v"(qf[s]));
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t o[4][8];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[cb][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    for (int it = 0; it < my_n; ++it) {
      char* stage = my + (it & 1) * SUB_BYTES;
      const int row0 = (wave + NWAVE * it) * SUB;
      if (it + 1 < my_n) wait_vmcnt<LOADS>(); else wait_vmcnt<0>();

      // ---- S^T = K . Q^T
      // all 18 K fragments are read before the MFMAs (no read->use stalls), and
      // even/odd k-steps accumulate separately to halve the dependency chain
      bf16x8_t kf[18];
#pragma unroll
      for (int s = 0; s < 16; ++s)
        kf[s] = *reinterpret_cast<const bf16x8_t*>(stage + ((s & 1) ? qk_base1 : qk_base0) +
                                                   128 * (s >> 1));
      kf[16] = *reinterpret_cast<const bf16x8_t*>(stage + qk_rope0);
      kf[17] = *reinterpret_cast<const bf16x8_t*>(stage + qk_rope1);
      f32x4_t sa = (f32x4_t){0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
      for (int s = 0; s < 18; s += 2) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s + 1], qf[s + 1], sb, 0, 0, 0);
      }
      const f32x4_t sacc = sa + sb;

      // ---- online softmax (log2 units); lane owns rows row0 + 4 lg + i of head lr
      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = row0 + 4 * lg + i < n;
        sv[i] = valid ? sacc[i] * kLog2e : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float pv[4], rs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_new);
        rs += pv[i];
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (!__all(alpha == 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int j = 0; j < 8; ++j) o[cb][j] *= alpha;
      }
      s16x4_t pf;
      {
        const uint32_t p01 = pack_bf16x2(pv[0], pv[1]);
        const uint32_t p23 = pack_bf16x2(pv[2], pv[3]);
        pf[0] = (short)(p01 & 0xffff);
        pf[1] = (short)(p01 >> 16);
        pf[2] = (short)(p23 & 0xffff);
        pf[3] = (short)(p23 >> 16);
      }

      // ---- O^T += C^T . P^T
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        uint32_t d[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = *reinterpret_cast<const uint4*>(stage + pv_base[i] + 256 * cb);
          d[i][0] = v.x; d[i][1] = v.y; d[i][2] = v.z; d[i][3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s16x4_t a0, a1;  // column 2q and 2q + 1 of this lane's chunk, rows 4lg..4lg+3
          a0[0] = (short)(d[0][q] & 0xffff); a0[1] = (short)(d[1][q] & 0xffff);
          a0[2] = (short)(d[2][q] & 0xffff); a0[3] = (short)(d[3][q] & 0xffff);
          a1[0] = (short)(d[0][q] >> 16);    a1[1] = (short)(d[1][q] >> 16);
          a1[2] = (short)(d[2][q] >> 16);    a1[3] = (short)(d[3][q] >> 16);
          o[cb][2 * q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, pf, o[cb][2 * q], 0, 0, 0);
          o[cb][2 * q + 1] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, pf, o[cb][2 * q + 1], 0, 0, 0);
        }
      }

      // refill this stage with the sub-tile two steps ahead
      if (it + 2 < my_n) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_subtile(rows, (wave + NWAVE * (it + 2)) * SUB, n, my_addr + (it & 1) * SUB_BYTES,
                      lane);
      }
    }

    // ---- merge the 4 wave states through LDS (staging buffers are free now)
    __syncthreads();
    float* om = reinterpret_cast<float*>(lds);             // [wave][16 heads][512]
    float* mlm = om + NWAVE * 16 * DC;                      // [wave][16][2]
    {
      float* ow = om + (wave * 16 + lr) * DC;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 8 * (16 * cb + 4 * lg + i);
          float4 lo = make_float4(o[cb][0][i], o[cb][1][i], o[cb][2][i], o[cb][3][i]);
          float4 hi = make_float4(o[cb][4][i], o[cb][5][i], o[cb][6][i], o[cb][7][i]);
          *reinterpret_cast<float4*>(ow + col) = lo;
          *reinterpret_cast<float4*>(ow + col + 4) = hi;
        }
      if (lg == 0) {
        mlm[(wave * 16 + lr) * 2] = m_run;
        mlm[(wave * 16 + lr) * 2 + 1] = l_run;
      }
    }
    __syncthreads();
    {
      // thread t: head t / 16, columns (t % 16) * 32 .. + 31
      const int h = threadIdx.x >> 4;
      const int c0 = (threadIdx.x & 15) * 32;
      float mw[NWAVE], M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        mw[w] = mlm[(w * 16 + h) * 2];
        M = fmaxf(M, mw[w]);
      }
      float L = 0.f, sc[NWAVE];
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        sc[w] = exp2f(mw[w] - M);
        L += sc[w] * mlm[(w * 16 + h) * 2 + 1];
      }
      float* dst = acc_out + ((int64_t)sg.pidx * H + hg * 16 + h) * DC + c0;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
          const float4 v = *reinterpret_cast<const float4*>(om + (w * 16 + h) * DC + c0 + c);
          r.x = fmaf(sc[w], v.x, r.x);
          r.y = fmaf(sc[w], v.y, r.y);
          r.z = fmaf(sc[w], v.z, r.z);
          r.w = fmaf(sc[w], v.w, r.w);
        }
        *reinterpret_cast<float4*>(dst + c) = r;
      }
      if ((threadIdx.x & 15) == 0) {
        ml_out[((int64_t)sg.pidx * H + hg * 16 + h) * 2] = M;
        ml_out[((int64_t)sg.pidx * H + hg * 16 + h) * 2 + 1] = L;
      }
    }
    __syncthreads();
  }
}

}  // namespace dec

void decode_core_mfma(const bf16* q_cat, const bf16* cache, const DecodeMeta& m, int parts,
                      int B, float* acc, float* ml, const Dims& d, hipStream_t st) {
  (void)B;
  dim3 grid(parts, d.H / 16);
  dec::decode_core_mfma_k<<<grid, 256, 0, st>>>(q_cat, cache, m, acc, ml, d.H);
}

}  // namespace mla
