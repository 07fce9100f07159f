// Key rows of a chunked prefill gathered into one contiguous block in the
// layer's storage type, for caches that the K/V expansion and the attention do
// not read in place:
//   * a paged cache, whose rows are reached through a page list (the pool of
//     pages that "Transformer and KV Cache Basics" grows its cache from,
//     Engineering section);
//   * an FP8 cache (E4M3 codes of the latent part with one fp32 scale per
//     row, the low-precision storage of the "Multi-Head Latent Attention"
//     post, introduction and section 3.1), decoded to c_i = s * value(code_i)
//     rounded to bf16.
// Prefill is bound by its matrix products; one extra pass over its key rows
// (about 1.2 KB per row in bf16) costs microseconds against milliseconds of
// products, and the rest of the prefill then runs unchanged on the gathered
// rows.
//
// One wave per key row, four waves per block; blockIdx.y walks sequences.
#include <algorithm>

#include "kernels.h"

namespace mla {
namespace gat {

constexpr int kWaves = 4;
constexpr int kFp8Dc = 512, kFp8Dr = 64;
constexpr int kFp8Rb = fp8_row_bytes(kFp8Dc, kFp8Dr);  // 656
constexpr int kFp8Scale = kFp8Dc + 2 * kFp8Dr;          // byte offset of the row scale

__device__ __forceinline__ int64_t src_row(const KeyRowSrc& s, int b, int r) {
  if (s.pages) {
    const int64_t page = s.pages[s.page_start[b] + (r >> s.page_shift)];
    return (page << s.page_shift) + (r & ((1 << s.page_shift) - 1));
  }
  return s.seq_off[b] + r;
}

// Rows in the storage type: a plain copy of row_bytes / sizeof(V) words.
template <typename V>
__global__ void __launch_bounds__(64 * kWaves)
gather_rows_k(KeyRowSrc s, const int64_t* __restrict__ kv_off, const int32_t* __restrict__ nrows,
              int B, int row_bytes, char* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nv = row_bytes / (int)sizeof(V);
  for (int b = blockIdx.y; b < B; b += gridDim.y) {
    const int n = nrows[b];
    for (int r = blockIdx.x * kWaves + wave; r < n; r += gridDim.x * kWaves) {
      const V* src = reinterpret_cast<const V*>(static_cast<const char*>(s.cache) +
                                                src_row(s, b, r) * row_bytes);
      V* dst = reinterpret_cast<V*>(out + (kv_off[b] + r) * row_bytes);
      for (int i = lane; i < nv; i += 64) dst[i] = src[i];
    }
  }
}

// FP8 rows (656 bytes: 512 codes, 64 bf16 rope values, the fp32 scale) ->
// bf16 rows of 576.  Lane l < 32 decodes codes 16 l .. 16 l + 15 (the E4M3 ->
// bf16 conversion is exact; the product with the scale is rounded once, to
// nearest even); lanes 32 .. 39 copy the rope values.
__global__ void __launch_bounds__(64 * kWaves)
gather_fp8_k(KeyRowSrc s, const int64_t* __restrict__ kv_off, const int32_t* __restrict__ nrows,
             int B, bf16* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int R = kFp8Dc + kFp8Dr;
  for (int b = blockIdx.y; b < B; b += gridDim.y) {
    const int n = nrows[b];
    for (int r = blockIdx.x * kWaves + wave; r < n; r += gridDim.x * kWaves) {
      const uint8_t* row = static_cast<const uint8_t*>(s.cache) + src_row(s, b, r) * kFp8Rb;
      bf16* dst = out + (kv_off[b] + r) * R;
      if (lane < 32) {
        const float sc = *reinterpret_cast<const float*>(row + kFp8Scale);
        const uint4 v = *reinterpret_cast<const uint4*>(row + lane * 16);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[8];
        // two decoded codes (bf16 pair), times the scale, rounded to bf16
        auto pair = [sc](uint32_t bits) {
          return pack_bf16x2(__uint_as_float(bits << 16) * sc,
                             __uint_as_float(bits & 0xffff0000u) * sc);
        };
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.0f, false);
          const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.0f, true);
          o[2 * k] = pair(__builtin_bit_cast(uint32_t, lo));
          o[2 * k + 1] = pair(__builtin_bit_cast(uint32_t, hi));
        }
        uint4* d = reinterpret_cast<uint4*>(dst + lane * 16);
        d[0] = make_uint4(o[0], o[1], o[2], o[3]);
        d[1] = make_uint4(o[4], o[5], o[6], o[7]);
      } else if (lane < 32 + 2 * kFp8Dr / 16) {
        const int i = lane - 32;
        *reinterpret_cast<uint4*>(dst + kFp8Dc + 8 * i) =
            *reinterpret_cast<const uint4*>(row + kFp8Dc + 16 * i);
      }
    }
  }
}

}  // namespace gat

int gather_key_rows(const KeyRowSrc& s, bool fp8, const int64_t* kv_off, const int32_t* nrows,
                    int B, int max_rows, int row_bytes, void* out, hipStream_t st) {
  if (B <= 0 || max_rows <= 0) return 0;
  const dim3 grid((unsigned)std::min<int64_t>(((int64_t)max_rows + gat::kWaves - 1) / gat::kWaves,
                                              4096),
                  (unsigned)std::min(B, 65535));
  const int threads = 64 * gat::kWaves;
  if (fp8) {
    if (row_bytes != 2 * (gat::kFp8Dc + gat::kFp8Dr)) return -1;
    gat::gather_fp8_k<<<grid, threads, 0, st>>>(s, kv_off, nrows, B, static_cast<bf16*>(out));
  } else if (row_bytes % 16 == 0 && (uintptr_t)s.cache % 16 == 0 && (uintptr_t)out % 16 == 0) {
    gat::gather_rows_k<uint4><<<grid, threads, 0, st>>>(s, kv_off, nrows, B, row_bytes,
                                                        static_cast<char*>(out));
  } else if (row_bytes % 4 == 0 && (uintptr_t)s.cache % 4 == 0 && (uintptr_t)out % 4 == 0) {
    gat::gather_rows_k<uint32_t><<<grid, threads, 0, st>>>(s, kv_off, nrows, B, row_bytes,
                                                           static_cast<char*>(out));
  } else {
    gat::gather_rows_k<uint16_t><<<grid, threads, 0, st>>>(s, kv_off, nrows, B, row_bytes,
                                                           static_cast<char*>(out));
  }
  return 0;
}

}  // namespace mla
