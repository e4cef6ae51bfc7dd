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
// written; the summary reads the words once), so they are written for coalesced traffic: one
// wave per run of 64 words of a row, each load instruction covering 512 B - 1 KiB of
// consecutive bytes, and the words assembled across lanes with shuffles.

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

// Each wave takes IPW consecutive items, an item being one (row, run of 64 words).  Load e of
// lane l reads the V (16 or 8) bytes at row offset 2048 seg + 64 V e + V l, so every load
// instruction covers 64 V consecutive bytes; all loads of the wave's items are issued before
// any result is used.  Those bytes are part l % (32 / V) of word 64 seg + (64 V / 32) e +
// l / (32 / V); the lane keeps the piece's V bits at bit V e of its value, and lane j then
// gathers the 32 / V parts of word 64 seg + j from the lanes that loaded them.  The row length
// S and the base address are multiples of V, so a piece never straddles the row end; pieces
// past it are 0 (padding bits).
constexpr int kItemsPerWave = 4;
template <int V>
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint8_t* __restrict__ bytes,
                                                        u32* __restrict__ words, int S, int W,
                                                        int n_seg, long long n_items) {
  static_assert(V == 16 || V == 8, "piece size");
  constexpr int PARTS = 32 / V;   // pieces per word
  constexpr int LOADS = 32 / V;   // load instructions per 2 KiB run (64 words)
  constexpr int IPW = kItemsPerWave;
  // (wave-uniform indices: the row and run arithmetic stays on the scalar unit)
  const long long item0 =
      ((long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * IPW;
  const int lane = threadIdx.x & 63;
  if (item0 >= n_items) return;  // (whole waves)
  u32 v[IPW];
  long long rows_[IPW];
  int segs[IPW];
#pragma unroll
  for (int it = 0; it < IPW; ++it) {
    const long long item = item0 + it;
    rows_[it] = n_seg == 1 ? item : item / n_seg;
    segs[it] = (int)(item - rows_[it] * n_seg);
  }
#pragma unroll
  for (int it = 0; it < IPW; ++it) {
    v[it] = 0u;
    const long long item = item0 + it;
    if (item < n_items) {
      const long long row = rows_[it];
      const int seg = segs[it];
      const uint8_t* rb = bytes + row * (long long)S;
#pragma unroll
      for (int e = 0; e < LOADS; ++e) {
        const int col = 2048 * seg + 64 * V * e + V * lane;
        if (col < S) {
          if constexpr (V == 16) {
            const u32x4 a = *(const u32x4*)(rb + col);
            v[it] |= (nonzero_bytes(a[0]) | (nonzero_bytes(a[1]) << 4) |
                      (nonzero_bytes(a[2]) << 8) | (nonzero_bytes(a[3]) << 12)) << (16 * e);
          } else {
            const u32x2 a = *(const u32x2*)(rb + col);
            v[it] |= (nonzero_bytes(a[0]) | (nonzero_bytes(a[1]) << 4)) << (8 * e);
          }
        }
      }
    }
  }
  // word 64 seg + j: load e = j / (64 / PARTS), parts from lanes PARTS (j % (64 / PARTS)) + k
  const int j = lane, e = j / (64 / PARTS), src = PARTS * (j % (64 / PARTS));
#pragma unroll
  for (int it = 0; it < IPW; ++it) {
    u32 w = 0u;
#pragma unroll
    for (int k = 0; k < PARTS; ++k)
      w |= ((__shfl((int)v[it], src + k) >> (V * e)) & ((1u << V) - 1u)) << (V * k);
    const long long item = item0 + it;
    if (item < n_items) {
      const int wi = 64 * segs[it] + j;
      if (wi < W) words[rows_[it] * W + wi] = w;
    }
  }
}

// Fallback (row length or base not a multiple of 8): one thread per word.
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

// tiles[bh, r, c] bit i = any kept bit in rows [64r, 64r+64) x keys [64t, 64t+64) of head bh,
// t = 32 c + i, bits at keys >= S ignored.  One wave per (bh, r, c): lane l ORs word 64 c + l of
// the block's rows (one 256-byte load instruction per row), a ballot marks the nonzero words,
// and tile t is the OR of the bits of its two words 2t, 2t+1.
__global__ __launch_bounds__(256) void tiles_kernel(const u32* __restrict__ words,
                                                    u32* __restrict__ tiles, int S, int W,
                                                    int n_rb, int TW, long long n_waves) {
  const long long wv = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wv >= n_waves) return;  // (whole waves)
  const long long rbh = wv / TW;
  const int c = (int)(wv - rbh * TW);
  const int r = (int)(rbh % n_rb);
  const long long bh = rbh / n_rb;
  const int wi = 64 * c + lane;
  u32 acc = 0u;
  if (wi < W) {
    const u32 valid = low_bits(S - 32 * wi);
    const u32* col = words + (bh * S + (long long)kTile * r) * W + wi;
    const int rows = min(kTile, S - kTile * r);
    int i = 0;
    for (; i + 8 <= rows; i += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc |= col[(long long)(i + u) * W];
    }
    for (; i < rows; ++i) acc |= col[(long long)i * W];
    acc &= valid;
  }
  unsigned long long x = __ballot(acc != 0u);
  // tile i of the run = word bits 2i | 2i+1, compacted to bit i
  x = (x | (x >> 1)) & 0x5555555555555555ull;
  x = (x | (x >> 1)) & 0x3333333333333333ull;
  x = (x | (x >> 2)) & 0x0f0f0f0f0f0f0f0full;
  x = (x | (x >> 4)) & 0x00ff00ff00ff00ffull;
  x = (x | (x >> 8)) & 0x0000ffff0000ffffull;
  x = (x | (x >> 16)) & 0x00000000ffffffffull;
  if (lane == 0) tiles[rbh * TW + c] = (u32)x;
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
  int S = seq_len, Wa = W;
  hipError_t e;
  if (seq_len % 8 == 0 && a % 8 == 0) {  // wave per 64-word run, contiguous loads
    int n_seg = (W + 63) / 64;
    long long n_items = (long long)batch * n_heads * seq_len * n_seg;
    const long long wblocks = (n_items + 4 * kItemsPerWave - 1) / (4 * kItemsPerWave);
    if (wblocks >= ((long long)1 << 31)) return FA_ERR_BAD_SHAPE;
    const void* k = (seq_len % 16 == 0 && a % 16 == 0) ? (const void*)pack_rows_kernel<16>
                                                        : (const void*)pack_rows_kernel<8>;
    void* args[] = {(void*)&mask_bytes, (void*)&mask_words, (void*)&S, (void*)&Wa, (void*)&n_seg,
                    (void*)&n_items};
    e = hipLaunchKernel(k, dim3((unsigned)wblocks), dim3(256), args, 0, (hipStream_t)stream);
  } else {
    const void* k = (seq_len % 4 == 0 && a % 4 == 0) ? (const void*)pack_kernel<4>
                                                      : (const void*)pack_kernel<1>;
    long long nw = n_words;
    void* args[] = {(void*)&mask_bytes, (void*)&mask_words, (void*)&S, (void*)&Wa, (void*)&nw};
    e = hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream);
  }
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
  const long long n_waves = (long long)batch * n_heads * n_rb * TW;
  const long long blocks = (n_waves + 3) / 4;
  if (blocks >= ((long long)1 << 31)) return FA_ERR_BAD_SHAPE;
  int S = seq_len, Wa = W, nrb = n_rb, tw = TW;
  long long nwv = n_waves;
  void* args[] = {(void*)&mask_words, (void*)&tiles, (void*)&S, (void*)&Wa, (void*)&nrb, (void*)&tw, (void*)&nwv};
  const hipError_t e = hipLaunchKernel((const void*)tiles_kernel, dim3((unsigned)blocks), dim3(256),
                                       args, 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
