// fa_mask.hip -- packing a byte mask into the bit layout the attention kernel reads, and the
// per-tile summary of a packed mask (C ABI declared in include/fa.h).
//
// Pages followed (cited by URL and section heading):
//   https://yunpan.plus/t/19526-1-1, section "AI生成的代码质量如何？": excerpt 2 fixes the bit
//   layout (key j is bit j % 32 of word j / 32, least significant bit first, a set bit keeps,
//   keys at or past seq_len are never kept); excerpt 1 skips a tile whose mask bits are all
//   clear, which the summary lets a caller (or a later pass) see per 64 x 64 block.
//
// Both kernels are bound by HBM bandwidth (a byte per (query, key) read once, an eighth of that
// written; the summary reads the words once), so they are written for full-line coalesced
// traffic and little else: one thread per output word, consecutive threads on consecutive
// words of a row.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;  // summary block: 64 query rows x 64 keys (the attention key tile)

// Bit k (k < 4) set iff byte k of d is nonzero.  Bit 7 of each byte of m is (byte != 0): the
// low seven bits plus 0x7f carry into bit 7 exactly when they are not all zero, and the OR
// adds the byte's own bit 7; no carry leaves a byte (0x7f + 0x7f < 0x100).
__device__ __forceinline__ u32 nonzero_bytes(u32 d) {
  const u32 m = ((d & 0x7f7f7f7fu) + 0x7f7f7f7fu) | d;
  return ((m >> 7) & 1u) | ((m >> 14) & 2u) | ((m >> 21) & 4u) | ((m >> 28) & 8u);
}

__device__ __forceinline__ u32 low_bits(int n) {
  return n >= 32 ? ~0u : (n <= 0 ? 0u : ((1u << n) - 1u));
}

// words[row, wi] for every row of the [B*H*S, S] byte matrix.  V = bytes per load (16, 8, 4, 1):
// the row length and the base address are multiples of V, so full words load in V-byte pieces;
// the last, partial word of a row (S % 32 != 0) reads only its own bytes.
template <int V>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ bytes,
                                                   u32* __restrict__ words, int S, int W,
                                                   long long n_words) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= n_words) return;
  const long long row = gid / W;
  const int wi = (int)(gid - row * W);
  const uint8_t* src = bytes + row * (long long)S + 32 * wi;
  const int n = min(32, S - 32 * wi);
  u32 w = 0u;
  if (n == 32) {
    if constexpr (V == 16) {
      const u32x4 a = *(const u32x4*)src;
      const u32x4 b = *(const u32x4*)(src + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w |= (nonzero_bytes(a[e]) << (4 * e)) | (nonzero_bytes(b[e]) << (16 + 4 * e));
    } else if constexpr (V == 8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32x2 a = *(const u32x2*)(src + 8 * e);
        w |= (nonzero_bytes(a[0]) << (8 * e)) | (nonzero_bytes(a[1]) << (8 * e + 4));
      }
    } else if constexpr (V == 4) {
#pragma unroll
      for (int e = 0; e < 8; ++e) w |= nonzero_bytes(*(const u32*)(src + 4 * e)) << (4 * e);
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) w |= (u32)(src[e] != 0) << e;
    }
  } else {
    for (int e = 0; e < n; ++e) w |= (u32)(src[e] != 0) << e;
  }
  words[gid] = w;
}

// tiles[bh, r, t / 32] bit t % 32 = any kept bit in rows [64r, 64r+64) x keys [64t, 64t+64) of
// head bh, bits at keys >= S ignored.  One thread per (bh, r, t) with t over TW * 32 slots, so
// each aligned 32-lane half of a wave owns one summary word, assembled with a ballot.
__global__ __launch_bounds__(256) void tiles_kernel(const u32* __restrict__ words,
                                                    u32* __restrict__ tiles, int S, int W,
                                                    int n_rb, int TW, long long n_items) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  bool any = false;
  if (gid < n_items) {
    const int slots = TW * 32;
    const long long rbh = gid / slots;
    const int t = (int)(gid - rbh * slots);
    const int r = (int)(rbh % n_rb);
    const long long bh = rbh / n_rb;
    if (t < n_rb) {  // (as many key tiles as row blocks: the mask is square)
      const u32* base = words + (bh * S + (long long)kTile * r) * W + 2 * t;
      const int rows = min(kTile, S - kTile * r);
      const u32 m0 = low_bits(S - kTile * t), m1 = low_bits(S - kTile * t - 32);
      u32 acc = 0u;
      if (m1) {
        for (int i = 0; i < rows; ++i) acc |= (base[(long long)i * W] & m0) | (base[(long long)i * W + 1] & m1);
      } else {
        for (int i = 0; i < rows; ++i) acc |= base[(long long)i * W] & m0;
      }
      any = acc != 0u;
    }
  }
  const unsigned long long bal = __ballot(any);
  if (gid < n_items && (threadIdx.x & 31) == 0) tiles[gid >> 5] = (u32)(bal >> (threadIdx.x & 32));
}

bool shape_ok(int batch, int n_heads, int seq_len) {
  return batch > 0 && n_heads > 0 && seq_len > 0;
}

}  // namespace

extern "C" {

fa_status fa_pack_mask(int batch, int n_heads, int seq_len, const uint8_t* mask_bytes,
                       uint32_t* mask_words, void* stream) {
  if (!mask_bytes || !mask_words) return FA_ERR_NULL_PTR;
  if (!shape_ok(batch, n_heads, seq_len)) return FA_ERR_BAD_SHAPE;
  if ((uintptr_t)mask_words & 3u) return FA_ERR_UNSUPPORTED;
  const int W = (seq_len + 31) / 32;
  const long long n_words = (long long)batch * n_heads * seq_len * W;
  const long long blocks = (n_words + 255) / 256;
  if (blocks >= ((long long)1 << 31)) return FA_ERR_BAD_SHAPE;
  const uintptr_t a = (uintptr_t)mask_bytes;
  const int v = (seq_len % 16 == 0 && a % 16 == 0) ? 16
                : (seq_len % 8 == 0 && a % 8 == 0) ? 8
                : (seq_len % 4 == 0 && a % 4 == 0) ? 4 : 1;
  const void* k = v == 16 ? (const void*)pack_kernel<16>
                  : v == 8 ? (const void*)pack_kernel<8>
                  : v == 4 ? (const void*)pack_kernel<4>
                           : (const void*)pack_kernel<1>;
  int S = seq_len, Wa = W;
  long long nw = n_words;
  void* args[] = {(void*)&mask_bytes, (void*)&mask_words, (void*)&S, (void*)&Wa, (void*)&nw};
  const hipError_t e = hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_mask_tiles(int batch, int n_heads, int seq_len, const uint32_t* mask_words,
                        uint32_t* tiles, void* stream) {
  if (!mask_words || !tiles) return FA_ERR_NULL_PTR;
  if (!shape_ok(batch, n_heads, seq_len)) return FA_ERR_BAD_SHAPE;
  if (((uintptr_t)mask_words | (uintptr_t)tiles) & 3u) return FA_ERR_UNSUPPORTED;
  const int W = (seq_len + 31) / 32;
  const int n_rb = (seq_len + kTile - 1) / kTile;
  const int TW = (n_rb + 31) / 32;
  const long long n_items = (long long)batch * n_heads * n_rb * TW * 32;
  const long long blocks = (n_items + 255) / 256;
  if (blocks >= ((long long)1 << 31)) return FA_ERR_BAD_SHAPE;
  int S = seq_len, Wa = W, nrb = n_rb, tw = TW;
  long long ni = n_items;
  void* args[] = {(void*)&mask_words, (void*)&tiles, (void*)&S, (void*)&Wa, (void*)&nrb, (void*)&tw, (void*)&ni};
  const hipError_t e = hipLaunchKernel((const void*)tiles_kernel, dim3((unsigned)blocks), dim3(256),
                                       args, 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
