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
// sequence boundaries into segments.  Inside a workgroup the waves take
// 16-row sub-tiles of the segment round-robin, each with its own online
// softmax state and a private double-buffered LDS stage filled by
// global_load_lds_dwordx4 (no VGPRs held by loads in flight).  At the end of a
// segment the wave states are merged through LDS and one partial
// (max, sum, unnormalised acc) is written; the combine kernels merge the
// partials of each sequence in a fixed order.
//
// Per 16-row sub-tile and wave:
//   S^T (16 rows x 16 heads) = K (16 x 576) . Q^T   -- 18 x mfma 16x16x32,
//       A = K fragments read from LDS (row l%16, 8 columns), B = Q in VGPRs;
//       lane l ends with rows 4(l/16)..+3 of head l%16.
//   softmax: per head = per lane column; max/sum across the 4 lane groups by
//       two xor-shuffles.
//   O^T (512 cols x 16 heads) += C^T (512 x 16 rows) . P^T (16 rows x 16 heads)
//       -- 32 x mfma 16x16x16; B = P exactly as S^T left it; A = C^T read
//       straight into operand layout by ds_read_b64_tr_b16 (gfx950 transposing
//       LDS read: inside each 16-lane group, output lane i element k is element
//       i % 4 of source lane 4k + i/4; source lane s of group g addresses row
//       4g + s/4, columns c0 + 4(s % 4), so lane i receives rows 4g..4g+3 of
//       column c0 + i).  Lane l accumulates columns c0 + 4(l/16) .. +3 of head
//       l % 16 for every 16-column block c0.
#include "kernels.h"
#include "stage_layout.h"

namespace mla {
namespace dec {

constexpr int DC = 512;
constexpr int RW = 576;                      // row width in elements
constexpr int SUB = 16;                      // rows per sub-tile
constexpr int SUB_BYTES = SUB * RW * 2;      // 18432
constexpr int LOADS = SUB + 2;               // 18 wave-wide 16-byte loads per sub-tile
#ifndef MLA_DEC_NWAVE
#define MLA_DEC_NWAVE 4
#endif
constexpr int NWAVE = MLA_DEC_NWAVE;         // waves per workgroup
constexpr int NTHR = 64 * NWAVE;
constexpr int NSTAGE = 2;
constexpr float kRescale = 8.0f;
constexpr int kXcds = 8;                     // XCDs of an MI355X             // lazy-rescale threshold, log2 units
constexpr int LDS_BYTES = NWAVE * NSTAGE * SUB_BYTES;  // 36 KB per wave
// merge: each wave finalises CB_PER_WAVE of the 32 16-column blocks; the
// exchange area holds every wave's value of every block (1 KB each)
constexpr int CB_PER_WAVE = 32 / NWAVE;
constexpr int XO_BYTES = NWAVE * 32 * 1024;
static_assert(32 % NWAVE == 0, "column blocks must split evenly over the waves");
static_assert(XO_BYTES + NWAVE * 16 * 2 * 4 <= LDS_BYTES, "merge space");


typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Stage layout (18 KB for 16 rows): the latent part of row r (64 chunks of 16
// bytes) at byte r*1024, the rope part (8 chunks) at 16384 + r*128, chunks
// swizzled per row as described in stage_layout.h.
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
// (lane = physical chunk, source chunk lane ^ lat_swz(i)); loads 16 and 17 copy
// the rope parts of rows 8j + lane/8.  Rows at or past `nvalid` re-read the
// last valid row (their scores are masked).
__device__ __forceinline__ void issue_subtile(const bf16* rows, int row0, int n,
                                              uint32_t stage_addr, int lane) {
  const char* base = reinterpret_cast<const char*>(rows + (int64_t)row0 * RW);
  const int last = n - row0 - 1;
#pragma unroll
  for (int i = 0; i < SUB; ++i) {
    const int r = i <= last ? i : last;
    dma16(base + r * (RW * 2) + ((lane ^ lat_swz(i)) << 4), stage_addr + i * 1024);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int r = 8 * j + (lane >> 3);
    const int cc = (lane & 7) ^ rope_swz(r);
    r = r <= last ? r : last;
    dma16(base + r * (RW * 2) + 1024 + (cc << 4), stage_addr + ROPE_OFF + j * 1024);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef const __attribute__((address_space(4))) DecodeWork* ConstWorkPtr;

// Field by field: a constant-address-space object cannot bind to the implicit
// copy constructor.
__device__ __forceinline__ DecodeWork load_work(ConstWorkPtr p) {
  DecodeWork w;
  w.row = p->row;
  w.n = p->n;
  w.b = p->b;
  w.pidx = p->pidx;
  w.next = p->next;
  return w;
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__global__ void __launch_bounds__(NTHR, 1)
decode_core_mfma_k(const bf16* __restrict__ q_cat, const bf16* __restrict__ cache, DecodeMeta mt,
                   float* __restrict__ acc_out, float* __restrict__ ml_out, int H, int nparts) {
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  // Block -> (part, head group).  Workgroups are handed to the XCDs round
  // robin (block i to XCD i % 8), so the HG head-group blocks of part p are
  // numbered p % 8 modulo 8: they share an XCD and its L2, start together and
  // stream the same rows, which HBM then delivers once.
  const int HG = H / 16;
  const int bid = blockIdx.x;
  const int part = (bid / (kXcds * HG)) * kXcds + bid % kXcds;
  const int hg = (bid / kXcds) % HG;
  if (part >= nparts) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  char* my = lds + wave * NSTAGE * SUB_BYTES;
  const uint32_t my_addr = lds_u32(my);
  // QK operand of k-step s: row lr, columns 32s + 8lg .. +7.  Latent chunk
  // 4s + lg (s < 16) sits at lr*1024 + 16*((4s + lg) ^ (lr & 7)) =
  // base(s & 1) + 128*(s >> 1) with b = bit 2 of lr selecting the order of each
  // even/odd pair; rope chunk 4(s-16) + lg at ROPE_OFF + lr*128 + 16*((...) ^ (lr & 7)).
  // row-wise operand of k-step s < 16: row lr, chunk 4s + lg, i.e. at
  // qk_off[s & 3] + 256 (s >> 2); rope chunk 4(s - 16) + lg at qk_rope[s - 16]
  int qk_off[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) qk_off[k] = lr * 1024 + 16 * ((4 * k + lg) ^ lat_swz(lr));
  const int qk_rope0 = ROPE_OFF + lr * 128 + 16 * (lg ^ rope_swz(lr));
  const int qk_rope1 = ROPE_OFF + lr * 128 + 16 * ((4 + lg) ^ rope_swz(lr));
  // transposing operand of column block cb = 4q + t: lane (g = lg, s = lr)
  // addresses row r = 4g + s/4, columns 16 cb + 4(s % 4): chunk 2cb + h with
  // h = (s % 4) / 2, byte 8(s & 1).  Its position 2(cb ^ a) + (h ^ b) (a = r & 7,
  // b = r >> 3) puts it at pv_e[t] + 128q for even q and pv_e[t] - pv_d + 128q
  // for odd q.
  int pv_e[4], pv_d;
  {
    const int r = 4 * lg + (lr >> 2);
    const int a = r & 7, b = (r >> 3) & 1, h = (lr & 3) >> 1;
    pv_d = 256 * (a >> 2);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      pv_e[t] = r * 1024 + 16 * (h ^ b) + 8 * (lr & 1) + 32 * (t ^ (a & 3)) + 128 * (a >> 2);
  }

  // the part's first work record is work[part]; further ones are chained.  The
  // records are read through the constant address space: the kernel never
  // writes them, and this keeps them on scalar loads (the inline-asm memory
  // clobbers would otherwise turn them into vector loads plus waits that also
  // drain the stage prefetches).
  const ConstWorkPtr works = reinterpret_cast<ConstWorkPtr>((uintptr_t)mt.work);
  DecodeWork wk = load_work(works + part);
  for (;;) {
    const int n = wk.n;
    const int nsub = (n + SUB - 1) / SUB;
    const bf16* rows = cache + wk.row * (int64_t)RW;

    // this wave's sub-tiles: wave, wave + NWAVE, ...
    const int my_n = wave < nsub ? (nsub - 1 - wave) / NWAVE + 1 : 0;
    if (my_n > 0) issue_subtile(rows, wave * SUB, n, my_addr, lane);
    if (my_n > 1) issue_subtile(rows, (wave + NWAVE) * SUB, n, my_addr + SUB_BYTES, lane);
    // the next record is fetched now and used after this segment
    DecodeWork nx = wk;
    if (wk.next >= 0) nx = load_work(works + wk.next);

    // Q^T fragments of head (hg*16 + lr): columns 32 s + 8 lg .. + 7
    bf16x8_t qf[18];
    {
      const bf16* qrow = q_cat + ((int64_t)wk.b * H + hg * 16 + lr) * RW + lg * 8;
#pragma unroll
      for (int s = 0; s < 18; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * s);
      // Consume the Q loads here so the compiler's own waits for them sit before
      // the loop: inside it the only loads in flight are the stage prefetches,
      // which are waited for explicitly.
#pragma unroll
      for (int s = 0; s < 18; ++s) asm volatile("" ::"v"(qf[s]));
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t o[32];  // o[cb][i]: head lr, column 16 cb + 4 lg + i
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) o[cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

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
        kf[s] = *reinterpret_cast<const bf16x8_t*>(stage + qk_off[s & 3] + 256 * (s >> 2));
      kf[16] = *reinterpret_cast<const bf16x8_t*>(stage + qk_rope0);
      kf[17] = *reinterpret_cast<const bf16x8_t*>(stage + qk_rope1);
      f32x4_t sa = (f32x4_t){0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
      for (int s = 0; s < 18; s += 2) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s + 1], qf[s + 1], sb, 0, 0, 0);
      }
      const f32x4_t sacc = sa + sb;
      // schedule: all 18 LDS reads first, then the 18 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 18, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 18, 0);

      // ---- online softmax (log2 units); lane owns rows row0 + 4 lg + i of head lr.
      // No cross-lane work in the common case: the reference max m_run only
      // moves when some score exceeds it by more than kRescale (a wave vote),
      // so p stays <= 2^kRescale; the running sum is kept per lane and reduced
      // over the 4 lane groups once per segment.  On a (rare) move, the head's
      // tile max is formed with two xor-shuffles and O and the sums rescaled.
      // The same reference enters l and acc, so their ratio is exact math.
      float sv[4];
      bool grow = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = row0 + 4 * lg + i < n;
        sv[i] = valid ? sacc[i] * kLog2e : -INFINITY;
        grow |= sv[i] > m_run + kRescale;
      }
      if (__any(grow)) {
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) o[cb] *= alpha;
      }
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_run);
        l_run += pv[i];
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
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const s16x4_t cf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(stage + pv_e[t] -
                                                          (q & 1) * pv_d + 128 * q));
          o[4 * q + t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cf, pf, o[4 * q + t], 0, 0, 0);
        }

      // refill this stage with the sub-tile two steps ahead
      if (it + 2 < my_n) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_subtile(rows, (wave + NWAVE * (it + 2)) * SUB, n, my_addr + (it & 1) * SUB_BYTES,
                      lane);
      }
    }

    // ---- merge the wave states through LDS (staging buffers are free now).
    // Every wave holds (head lr, columns 16 cb + 4 lg .. +3) for all 32 column
    // blocks cb; wave w finalises the blocks of its own range, reading the
    // other waves' values of those blocks from lane-contiguous 1 KB slots
    // (conflict-free), and sums the waves in order 0..NWAVE-1.
    __syncthreads();
    float4* xo = reinterpret_cast<float4*>(lds);              // [src wave][cb][64 lanes]
    float* mlx = reinterpret_cast<float*>(lds + XO_BYTES);    // [wave][16 heads][2]
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
      if (cb / CB_PER_WAVE != wave)
        xo[(wave * 32 + cb) * 64 + lane] = make_float4(o[cb][0], o[cb][1], o[cb][2], o[cb][3]);
    // per-lane partial sums -> per-head sum over the 4 lane groups
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (lg == 0) {
      mlx[(wave * 16 + lr) * 2] = m_run;
      mlx[(wave * 16 + lr) * 2 + 1] = l_run;
    }
    __syncthreads();
    {
      float mw[NWAVE], sc[NWAVE];
      float M = -INFINITY, L = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        mw[w] = mlx[(w * 16 + lr) * 2];
        M = fmaxf(M, mw[w]);
      }
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        sc[w] = exp2f(mw[w] - M);
        L += sc[w] * mlx[(w * 16 + lr) * 2 + 1];
      }
      const int gh = hg * 16 + lr;  // global head index
      float* pacc = acc_out + ((int64_t)wk.pidx * H + gh) * DC + 4 * lg;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        if (cb / CB_PER_WAVE != wave) continue;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
          const float4 v = w == wave ? make_float4(o[cb][0], o[cb][1], o[cb][2], o[cb][3])
                                     : xo[(w * 32 + cb) * 64 + lane];
          a.x = fmaf(sc[w], v.x, a.x);
          a.y = fmaf(sc[w], v.y, a.y);
          a.z = fmaf(sc[w], v.z, a.z);
          a.w = fmaf(sc[w], v.w, a.w);
        }
        *reinterpret_cast<float4*>(pacc + 16 * cb) = a;
      }
      if (wave == 0 && lg == 0) {
        ml_out[((int64_t)wk.pidx * H + gh) * 2] = M;
        ml_out[((int64_t)wk.pidx * H + gh) * 2 + 1] = L;
      }
    }
    __syncthreads();  // the stages are refilled by the next segment
    if (wk.next < 0) break;
    wk = nx;
  }
}

}  // namespace dec

int decode_core_wg_per_cu() { return dec::NWAVE >= 4 ? 1 : 4 / dec::NWAVE; }

void decode_core_mfma(const bf16* q_cat, const bf16* cache, const DecodeMeta& m, int parts,
                      int B, float* acc, float* ml, const Dims& d, hipStream_t st) {
  (void)B;
  const int hg = d.H / 16;
  const int blocks = (parts + dec::kXcds - 1) / dec::kXcds * dec::kXcds * hg;
  dec::decode_core_mfma_k<<<blocks, dec::NTHR, 0, st>>>(q_cat, cache, m, acc, ml, d.H, parts);
}

}  // namespace mla
