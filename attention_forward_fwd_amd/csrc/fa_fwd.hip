// fa_fwd.hip -- FlashAttention forward pass for AMD MI355X (gfx950, CDNA4) and the C ABI
// declared in include/fa.h.
//
// Pages followed (cited by URL and section heading):
//   [avo]    https://yetianai.com/news/16520
//            "传统进化搜索的天花板": block-wise attention that never stores the score matrix; the
//            FA4 design with a correction step that rescales the accumulator of the single-pass
//            softmax.  "进化轨迹与AI发现的优化手法": interleaving QK^T with PV, causal masking
//            expressed as bit masks, branch-free accumulator rescaling with lighter barriers,
//            overlap of correction with matrix work.  "七天跑出的成绩单": the prefill grid and
//            the GQA head groups.
//   [mask]   https://yunpan.plus/t/19526-1-1
//            "迭代历程": mask preloaded from global to shared memory, bank-conflict removal,
//            vectorised loads, P V accumulated from registers without a shared-memory P tile.
//            "AI生成的代码质量如何？" excerpt 1: skip a tile when a warp vote finds no kept bit;
//            excerpt 2: scale and mask applied in registers, row max reduced across the lanes
//            that share a row, bit key%32 of word key/32 keeps the score, out-of-range rows and
//            keys are never kept.
//
// Design for gfx950 (what differs from the pages' NVIDIA kernels is deliberate):
//   * Work: one workgroup = 4 waves x 32 rows.  A "row" is a (position, query head) pair; the
//     rows of one KV head are ordered position-major, head-minor (row r -> position r / G,
//     head hk*G + r % G), so a workgroup covers every query head of a GQA group at the same
//     positions and each K/V tile staged in LDS feeds G heads.
//   * Matrix cores: v_mfma_f32_32x32x16_{bf16,f16}.  S^T = K Q^T puts one query in each lane
//     column (lane l holds query l%32 and 16 keys per 32-key block), so the row max and row sum
//     are in-lane reductions plus one v_permlane32_swap, and the rescale of O^T += V^T P^T
//     touches only the lane's own query.  P never leaves registers: the S^T accumulator layout
//     is re-used directly as the B operand of the P V product (keys permuted consistently on
//     both operands).
//   * LDS: K tiles are copied global -> LDS by the DMA path (global_load_lds_dwordx4, no
//     registers) into 1 KiB regions of whole rows, padded so the 128-bit operand reads are
//     conflict-free (layout below).  V tiles are read with coalesced 128-bit loads into
//     registers one tile ahead, transposed in registers with byte permutes and written as V^T
//     in a layout where every P V operand (8 keys of one head_dim column, in the key order of
//     the P registers) is a single 128-bit read.  Q is staged once through the same LDS.  K, V
//     and mask tiles are double-buffered, one workgroup barrier per tile.  Key rows past the
//     sequence end are loaded from the last valid row (address clamp) and masked, so their
//     probabilities are exactly 0.
//   * Softmax: exp2 with log2(e) folded into the scale, running max floored at -1e30 so a
//     fully masked row never makes NaN, unconditional (branch-free) rescale of O and l every
//     tile, masked scores set to -inf with one bit-field extract and one bit-field insert.
//   * Skips: per wave and tile, the keep bits of the wave's rows are voted with a 64-lane
//     ballot; a tile with no kept bit costs no matrix or softmax work (causal tiles above the
//     diagonal, empty blocks of a custom mask).  Causal workgroups stop at their last live tile.
//   * Scheduling: workgroups are remapped so each of the 8 XCDs gets a contiguous range of
//     tiles (tiles of one KV head share that XCD's L2); causal row tiles run longest first.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

enum { kNone = 0, kCausal = 1, kBitmask = 2 };

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const u32* mask;
  uint16_t* o;
  int S, Hq, Hkv, G, W;
  int n_rt;   // row tiles per (batch, kv head)
  int n_wg;   // workgroups in the grid
  float c;    // |scale| * log2(e), floored at 2^-100
  u32 qflip;  // 0x80008000 when scale < 0 (moves the sign onto Q exactly), else 0
};

// Tile shape shared by every instance: 4 waves of 32 rows, 64 keys per tile; two workgroups
// share a CU (two waves per SIMD, from different workgroups, so one wave's vector work can run
// while the other's matrix work occupies the matrix cores).
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // rows per workgroup
constexpr int kBN = 64;           // keys per tile

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack8(f32x8 x) {  // round to nearest even
  if constexpr (BF16)
    return __builtin_bit_cast(u32x4, __builtin_convertvector(x, bf16x8));
  else
    return __builtin_bit_cast(u32x4, __builtin_convertvector(x, f16x8));
}

template <bool BF16>
__device__ __forceinline__ u32x2 pack4(f32x4 x) {
  if constexpr (BF16)
    return __builtin_bit_cast(u32x2, __builtin_convertvector(x, bf16x4));
  else
    return __builtin_bit_cast(u32x2, __builtin_convertvector(x, f16x4));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// acc + x.lo + x.hi for a packed pair of 16-bit floats (v_dot2 against (1, 1)).
template <bool BF16>
__device__ __forceinline__ float dot2_ones(u32 x, float acc) {
  if constexpr (BF16) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
  }
}

// Both lane halves (l and l^32) hold the same query: combine their partial values.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keep-bits of `n` keys starting at bit 0 (n clamped to [0, 32]).
__device__ __forceinline__ u32 low_bits(int n) {
  return n >= 32 ? ~0u : (n <= 0 ? 0u : ((1u << n) - 1u));
}

// LDS layout of a K or Q tile (rows = keys or query rows, 16-byte chunks of head_dim).
// A "region" is the 1 KiB one wave-wide DMA instruction writes (lane i -> byte 16 i): it holds
// RPR whole rows (4 at d=128, 8 at d=64), chunk c of row rr at slot c*RPR + (rr ^ x(c)), and
// regions are padded to a stride of RS bytes.  Why:
//   * a DMA instruction reads RPR complete rows, 1 KiB contiguous per row group (coalesced);
//   * every operand address is a per-lane base plus compile-time offsets for the k-step, the
//     32-key block and the buffer, so no per-read address registers;
//   * with 64 banks x 4 B, a 128-bit operand read (16 lanes per LDS cycle: one chunk of 16
//     consecutive rows) touches every bank once: the RPR rows of a region sit in consecutive
//     slots and the padding shifts consecutive regions by 16 (d=128) or 32 (d=64) banks.  At
//     d=64 the row index within the region is also XORed with bit 1 of the chunk (x(c) =
//     4 * ((c >> 1) & 1)); that only permutes the slots of one row group and is neutral for
//     these reads.
template <int D>
struct Lds {
  static constexpr int RB = D * 2;              // bytes of one row's data
  static constexpr int RPR = 1024 / RB;         // rows per region
  static constexpr int RS = D == 128 ? 1088 : 1152;
  static constexpr int KC = D / 8;              // chunks per row
  __device__ static constexpr int x(int c) { return D == 64 ? 4 * ((c >> 1) & 1) : 0; }
  // byte offset of (row r, chunk c) within a tile
  __device__ static constexpr int off(int r, int c) {
    return (r / RPR) * RS + (c * RPR + ((r % RPR) ^ x(c))) * 16;
  }
};

// LDS layout of a transposed V tile: row d (one head_dim index) holds the BN = 64 keys of the
// tile, 128 bytes, as 8 "units" of 16 bytes.  Unit u = 2ks + hl holds keys 16ks + 4hl + 0..3
// (first 8 bytes) and 16ks + 8 + 4hl + 0..3 (last 8 bytes): exactly the 8 keys, in register
// order, that lane half hl of an MFMA needs at k-step ks of P V, so each V^T operand is one
// 128-bit read.  Rows d and d ^ 8 share the 256-byte line ((d/16) * 8 + d % 8); unit u of row d
// sits at 16-byte slot u ^ g(d), g(d) = (d % 16) ^ ((d / 16) % 8) (bit 3 of the slot is bit 3
// of d).  With 64 banks x 4 B, the operand reads (16 lanes: one unit of 16 consecutive rows)
// and the staging writes (32 lanes: one half-unit of 16 rows spaced 8 apart, both halves) touch
// every bank once.  The read address of k-step ks is a per-(lane, 32-row block) base XOR 32*ks.
struct VtLds {
  __device__ static constexpr int off(int d, int u, int half) {
    return ((((d >> 4) << 3) | (d & 7)) * 256) + ((u ^ ((d & 15) ^ ((d >> 4) & 7))) & 15) * 16 +
           half * 8;
  }
};

typedef __attribute__((address_space(3))) void lds_void;

template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(Params p) {
  constexpr int BM = kBM, BN = kBN, NT = kThreads, NW = kWaves;
  constexpr int KC = D / 8;        // 16-byte chunks per row
  constexpr int NKB = BN / 32;     // 32-key blocks per tile (one MFMA output block each)
  constexpr int QKS = D / 16;      // MFMA k-steps of Q K^T
  constexpr int NDB = D / 32;      // 32-wide blocks of head_dim in O
  constexpr int PKS = BN / 16;     // MFMA k-steps of P V
  using L = Lds<D>;
  constexpr int RPR = L::RPR, RS = L::RS;
  constexpr int NREG = BN / RPR;     // regions per tile
  constexpr int T_BYTES = NREG * RS; // one K tile (BN rows)
  constexpr int VT_BYTES = D * 128;  // one transposed V tile (D rows of BN = 64 keys)
  constexpr int NDQ = D / 8;         // 16-byte column chunks of a V row
  constexpr int VS_THREADS = 16 * NDQ;  // V staging: one key quad x one column chunk each
  constexpr int M_WORDS = MODE == kBitmask ? BM * NKB : 1;
  constexpr int DMA_PER_WAVE = NREG / NW;             // one region per DMA instruction
  constexpr int QL = BM * KC / NT;                    // Q chunks staged per thread
  static_assert(BM == 2 * BN, "Q staging uses the two K buffers, BN rows each");
  static_assert(DMA_PER_WAVE * NW == NREG && QL * NT == BM * KC, "load split");
  static_assert(BN == 64 && VS_THREADS <= NT, "V staging covers a 64-key tile");

  // Separate arrays (not one array indexed by buffer) so the compiler can tell the DMA into one
  // buffer from LDS reads of another and does not wait for the DMA before those reads.
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[T_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[T_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[VT_BYTES];  // V^T tiles
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[VT_BYTES];
  __shared__ __attribute__((aligned(16))) u32 m_lds0[M_WORDS];
  __shared__ __attribute__((aligned(16))) u32 m_lds1[M_WORDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;   // lane column and lane half
  const int S = p.S, G = p.G, Hq = p.Hq, Hkv = p.Hkv;

  // XCD-aware remap: the hardware deals workgroup i to XCD i % 8.  Give XCD x the contiguous
  // logical range so that row tiles of one KV head (which read the same K/V) share an L2.
  int wg = blockIdx.x;
  {
    const int x = wg & 7, idx = wg >> 3, q8 = p.n_wg >> 3, r8 = p.n_wg & 7;
    wg = x * q8 + min(x, r8) + idx;
  }
  const int bh = wg / p.n_rt;
  int rt = wg - bh * p.n_rt;
  if (MODE == kCausal) rt = p.n_rt - 1 - rt;  // longest causal rows first
  const int b = bh / Hkv, hk = bh - b * Hkv;
  const int row0 = rt * BM;

  const size_t q_batch = (size_t)b * S * Hq * D;
  const uint16_t* __restrict__ kg = p.k + ((size_t)b * S * Hkv + hk) * D;
  const uint16_t* __restrict__ vg = p.v + ((size_t)b * S * Hkv + hk) * D;
  const int kv_stride = Hkv * D;

  // This lane's query row.
  const int my_row = row0 + wave * 32 + l32;
  const int my_pos = my_row / G;
  const int my_head = hk * G + (my_row - my_pos * G);
  const int w_pmin = (row0 + wave * 32) / G;
  const bool wave_live = w_pmin < S;

  int n_tiles;
  if (MODE == kCausal) {
    const int pmax = min((row0 + BM - 1) / G, S - 1);
    n_tiles = pmax / BN + 1;
  } else {
    n_tiles = (S + BN - 1) / BN;
  }

  // Lane bases of the 128-bit operand reads (Q and K): row l32 of a 32-row block, chunk
  // 2ks + hl.  At d=64 the row XOR depends on ks & 1, hence two bases.
  int op_base[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) op_base[e] = L::off(l32, 2 * e + hl);
  // (row 32*blk + l32, chunk 2ks + hl) = op_base[ks & 1] + blk*BLK_OFF + (ks >> 1)*2*KS2_OFF
  constexpr int BLK_OFF = (32 / RPR) * RS;
  constexpr int KS2_OFF = 2 * RPR * 16;  // two chunks
  auto op_addr = [&](int ks, int blk) __attribute__((always_inline)) {
    return op_base[ks & 1] + blk * BLK_OFF + (ks >> 1) * 2 * KS2_OFF;
  };

  // ---- Q: coalesced 128-bit loads -> LDS (rows 0..63 in k_lds0, 64..127 in k_lds1) -> MFMA B
  // operands held in registers for the whole key loop.
#pragma unroll
  for (int i = 0; i < QL; ++i) {
    const int id = tid + NT * i, r = id / KC, c = id % KC;
    const int grow = row0 + r, pos = grow / G, h = hk * G + (grow - pos * G);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (pos < S) x = *(const u32x4*)(p.q + q_batch + ((size_t)pos * Hq + h) * D + c * 8);
    *(u32x4*)((r < BN ? k_lds0 : k_lds1) + L::off(r % BN, c)) = x;
  }
  __syncthreads();
  u32x4 qreg[QKS];
#pragma unroll
  for (int ks = 0; ks < QKS; ++ks) {
    const u32x4 x = *(const u32x4*)((wave < 2 ? k_lds0 : k_lds1) + op_addr(ks, wave & 1));
    qreg[ks] = x ^ p.qflip;
  }
  __syncthreads();

  // ---- K/V staging by DMA: instruction i of this wave fills region n = i*NW + wave; lane = slot
  // s holds chunk s / RPR of row n*RPR + ((s % RPR) ^ x(chunk)).
  const int dma_c = lane / RPR;
  const int dma_rr = (lane % RPR) ^ L::x(dma_c);
  auto dma_tile = [&](const uint16_t* __restrict__ src, int j, unsigned char* dst)
                      __attribute__((always_inline)) {
    const int k0 = j * BN;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int n = i * NW + wave;
      const int key = min(k0 + n * RPR + dma_rr, S - 1);
      __builtin_amdgcn_global_load_lds((const void*)(src + key * kv_stride + dma_c * 8),
                                       (lds_void*)(dst + n * RS), 16, 0, 0);
    }
  };

  // ---- V staging (transposed).  Thread t < VS_THREADS owns column chunk dq (head_dim
  // 8dq..8dq+7) of key quad q (keys 4q..4q+3).  Consecutive lanes take consecutive column
  // chunks of one key row, so every load instruction reads whole rows.  Lanes 16-31 take quad
  // q+2 (same V^T unit, other half) so the two 16-lane halves of a write never share a bank.
  // The four 16-byte pieces (one per key) are loaded into registers early, then transposed with
  // byte permutes into eight 8-byte pieces (one per column) and written at their V^T unit:
  // unit 2(q/4) + (q%2), half (q/2)%2.
  const int vs_dq = D == 128 ? (tid & 15) : (tid & 7);
  const int vs_qi = D == 128 ? (tid >> 4) : (tid >> 3);
  const int vs_q = 4 * (vs_qi >> 2) + ((vs_qi >> 1) & 1) + 2 * (vs_qi & 1);
  u32x4 vstage[4];
  auto v_load = [&](int j) __attribute__((always_inline)) {
    if (tid < VS_THREADS) {
      const int k0 = j * BN;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = min(k0 + 4 * vs_q + kk, S - 1);
        vstage[kk] = *(const u32x4*)(vg + key * kv_stride + 8 * vs_dq);
      }
    }
  };
  auto v_store = [&](unsigned char* vt) __attribute__((always_inline)) {
    if (tid < VS_THREADS) {
      const int u = 2 * (vs_q >> 2) + (vs_q & 1), half = (vs_q >> 1) & 1;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int m = jj >> 1;
        const u32 sel = (jj & 1) ? 0x07060302u : 0x05040100u;  // high / low 16-bit halves
        const u32x2 col = {__builtin_amdgcn_perm(vstage[1][m], vstage[0][m], sel),
                           __builtin_amdgcn_perm(vstage[3][m], vstage[2][m], sel)};
        *(u32x2*)(vt + VtLds::off(8 * vs_dq + jj, u, half)) = col;
      }
    }
  };

  // Mask words (bitmask mode): thread t < BM stages the NKB words of row t for a tile.
  u32 mreg[NKB];
  const u32* mrow = nullptr;
  bool mrow_ok = false;
  if (MODE == kBitmask && tid < BM) {
    const int grow = row0 + tid, pos = grow / G, h = hk * G + (grow - pos * G);
    mrow_ok = pos < S;
    if (mrow_ok) mrow = p.mask + (((size_t)b * Hq + h) * S + pos) * (size_t)p.W;
  }
  auto mask_load = [&](int j) __attribute__((always_inline)) {
    if (MODE == kBitmask && tid < BM) {
#pragma unroll
      for (int w = 0; w < NKB; ++w) {
        const int word = j * NKB + w;
        mreg[w] = (mrow_ok && word < p.W) ? mrow[word] : 0u;
      }
    }
  };
  auto mask_store = [&](u32* mb) __attribute__((always_inline)) {
    if (MODE == kBitmask && tid < BM) {
#pragma unroll
      for (int w = 0; w < NKB; ++w) mb[tid * NKB + w] = mreg[w];
    }
  };

  // Tile class of tile j for this wave: full (no masking), skip (a 64-lane ballot finds no kept
  // bit), or partial with per-lane keep words.  Lane half hl holds keys 8*(r/4) + 4*hl + r%4 of
  // each 32-key block, so the word is pre-shifted by 4*hl and register r tests the constant bit
  // 8*(r/4) + r%4.
  struct Cls {
    u32 wsh[NKB];
    bool full, skip;
  };
  auto classify = [&](int j, const u32* mb) __attribute__((always_inline)) {
    Cls cl;
    const int k0 = j * BN;
    if (MODE == kNone) cl.full = k0 + BN <= S;
    else if (MODE == kCausal) cl.full = k0 + BN - 1 <= w_pmin;
    else cl.full = false;
    cl.skip = false;
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) cl.wsh[kb32] = ~0u;
    if (!cl.full) {
      u32 any = 0;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) {
        const int kbase = k0 + 32 * kb32;
        u32 w = low_bits(S - kbase);
        if (MODE == kCausal) w = my_pos < S ? (w & low_bits(my_pos - kbase + 1)) : 0u;
        if (MODE == kBitmask) w &= mb[(wave * 32 + l32) * NKB + kb32];
        any |= w;
        cl.wsh[kb32] = w >> (4 * hl);
      }
      cl.skip = __ballot(any != 0u) == 0ull;
    }
    return cl;
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -1e30f;  // finite floor: a fully masked row keeps alpha = 1 and p = 0
  float l_run = 0.f;     // this lane's partial row sum (its 16 keys of each 32-key block)
  const float c = p.c;

  // V^T operand (A of O^T += V^T P^T): lane l reads head_dim row 32*db + l%32, unit 2ks + hl,
  // at a per-block base XOR 32*ks.
  int vt_base[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) vt_base[db] = VtLds::off(32 * db + l32, hl, 0);
  auto v_operand = [&](const unsigned char* vb, int ks, int db) __attribute__((always_inline)) {
    return *(const u32x4*)(vb + (vt_base[db] ^ (32 * ks)));
  };

  // One tile's compute: S^T = K Q^T (operands read one k-step ahead), masked online softmax,
  // O = alpha O + V^T P^T (branch-free rescale, P straight from registers; P slots 0..3 of lane
  // half hl hold keys 16ks + 4hl + 0..3 and slots 4..7 keys 16ks + 8 + 4hl + 0..3, the key order
  // of a V^T unit).
  auto compute = [&](const Cls& cls, const unsigned char* kb, const unsigned char* vb)
                     __attribute__((always_inline)) {
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb32][r] = 0.f;
    u32x4 ka[2][NKB];
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) ka[0][kb32] = *(const u32x4*)(kb + op_addr(0, kb32));
#pragma unroll
    for (int ks = 0; ks < QKS; ++ks) {
      if (ks + 1 < QKS) {
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32)
          ka[(ks + 1) & 1][kb32] = *(const u32x4*)(kb + op_addr(ks + 1, kb32));
      }
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
        sacc[kb32] = mfma32<BF16>(ka[ks & 1][kb32], qreg[ks], sacc[kb32]);
    }

    if (!cls.full) {  // masked scores -> -inf: bit-field extract of the keep bit + bit-field insert
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int bit = 8 * (r >> 2) + (r & 3);
          const int keep = ((int)(cls.wsh[kb32] << (31 - bit))) >> 31;
          sacc[kb32][r] = __int_as_float((__float_as_int(sacc[kb32][r]) & keep) |
                                         (~keep & (int)0xff800000));
        }
    }
    // Row max: four independent in-lane chains of 3-input maxima (v_max3_f32) over 8 scores
    // each, then across the two lane halves.
    float mx4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x16& v = sacc[(q >> 1) % NKB];
      const int b0 = 8 * (q & 1);
      float m = __builtin_fmaxf(__builtin_fmaxf(v[b0], v[b0 + 1]), v[b0 + 2]);
      m = __builtin_fmaxf(__builtin_fmaxf(m, v[b0 + 3]), v[b0 + 4]);
      m = __builtin_fmaxf(__builtin_fmaxf(m, v[b0 + 5]), v[b0 + 6]);
      mx4[q] = __builtin_fmaxf(m, v[b0 + 7]);
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(mx4[0], mx4[1]), __builtin_fmaxf(mx4[2], mx4[3]));
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    // p = 2^(s*c - m), rounded to the input dtype; the row sum adds the rounded values
    // (v_dot2 against (1, 1)) so numerator and denominator see the same P.
    u32x4 pk[PKS];
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          t[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kb32][8 * h + e], c, -m_new));
        const u32x4 pw = pack8<BF16>(t);
        pk[2 * kb32 + h] = pw;
#pragma unroll
        for (int e = 0; e < 4; ++e) ps[e & 1] = dot2_ones<BF16>(pw[e], ps[e & 1]);
      }
    l_run = l_run * alpha + (ps[0] + ps[1]);

#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    u32x4 va[2][NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) va[0][db] = v_operand(vb, 0, db);
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
      if (ks + 1 < PKS) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          va[(ks + 1) & 1][db] = v_operand(vb, ks + 1, db);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32<BF16>(va[ks & 1][db], pk[ks], oacc[db]);
    }
  };

  // One tile: prefetch tile j+1 (K by DMA, V and mask words into registers), compute tile j,
  // then wait for this wave's loads, write V^T and the mask words and meet the other waves at
  // the barrier.
  auto tile = [&](int j, const unsigned char* k_cur, const unsigned char* v_cur,
                  const u32* m_cur, unsigned char* k_fill, unsigned char* v_fill, u32* m_fill)
                  __attribute__((always_inline)) {
    const bool more = j + 1 < n_tiles;
    if (more) {
      dma_tile(kg, j + 1, k_fill);
      v_load(j + 1);
      mask_load(j + 1);
    }
    const Cls cls = classify(j, m_cur);
    if (wave_live && !cls.skip) compute(cls, k_cur, v_cur);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA and loads have landed
    if (more) {
      v_store(v_fill);
      mask_store(m_fill);
    }
    __syncthreads();
  };

  // Prologue: tile 0.
  dma_tile(kg, 0, k_lds0);
  v_load(0);
  mask_load(0);
  mask_store(m_lds0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  v_store(v_lds0);
  __syncthreads();
  for (int j = 0; j < n_tiles; j += 2) {
    tile(j, k_lds0, v_lds0, m_lds0, k_lds1, v_lds1, m_lds1);
    if (j + 1 < n_tiles) tile(j + 1, k_lds1, v_lds1, m_lds1, k_lds0, v_lds0, m_lds0);
  }

  // ---- Epilogue: O / l (0 for a row with no kept key), rounded, 8-byte stores.
  const float lt = sum_halves(l_run);
  const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
  if (wave_live && my_pos < S) {
    uint16_t* orow = p.o + q_batch + ((size_t)my_pos * Hq + my_head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[db][4 * t4 + e] * inv;
        *(u32x2*)(orow + 32 * db + 8 * t4 + 4 * hl) = pack4<BF16>(x);
      }
  }
}

template <bool BF16, int D, int MODE>
hipError_t launch(const Params& p, hipStream_t s) {
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)fa_fwd_kernel<BF16, D, MODE>, dim3(p.n_wg),
                         dim3(kThreads), args, 0, s);
}

template <bool BF16, int D>
hipError_t launch_mode(int mode, const Params& p, hipStream_t s) {
  switch (mode) {
    case kNone: return launch<BF16, D, kNone>(p, s);
    case kCausal: return launch<BF16, D, kCausal>(p, s);
    default: return launch<BF16, D, kBitmask>(p, s);
  }
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_PTR: return "null q, k, v or o pointer";
    case FA_ERR_BAD_SHAPE: return "bad shape (non-positive size, heads not divisible, or too large)";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype or head_dim, or misaligned pointer";
    case FA_ERR_BAD_MASK_MODE: return "unknown mask mode, or bitmask mode without a mask";
    case FA_ERR_BAD_SCALE: return "scale is not finite";
    case FA_ERR_HIP: return "HIP runtime rejected the kernel launch";
    default: return "unknown status";
  }
}

fa_status fa_fwd(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                 int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                 const void* k, const void* v, const uint32_t* mask, void* o, void* stream) {
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (mask_mode != FA_MASK_NONE && mask_mode != FA_MASK_CAUSAL && mask_mode != FA_MASK_BITMASK)
    return FA_ERR_BAD_MASK_MODE;
  if (!q || !k || !v || !o) return FA_ERR_NULL_PTR;
  if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || seq_len <= 0 ||
      n_q_heads % n_kv_heads != 0)
    return FA_ERR_BAD_SHAPE;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  // Offsets inside one batch are 32-bit; the grid is a 32-bit count.
  if ((int64_t)seq_len * n_q_heads * head_dim >= ((int64_t)1 << 31)) return FA_ERR_BAD_SHAPE;
  const int G = n_q_heads / n_kv_heads;
  const int64_t rows = (int64_t)seq_len * G;
  const int64_t n_rt = (rows + kBM - 1) / kBM;
  const int64_t n_wg = n_rt * n_kv_heads * batch;
  if (n_wg >= ((int64_t)1 << 31)) return FA_ERR_BAD_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_UNSUPPORTED;
  if (mask_mode == FA_MASK_BITMASK && (!mask || ((uintptr_t)mask & 3u))) return FA_ERR_BAD_MASK_MODE;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;

  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.mask = mask_mode == FA_MASK_BITMASK ? mask : nullptr;
  p.o = (uint16_t*)o;
  p.S = seq_len;
  p.Hq = n_q_heads;
  p.Hkv = n_kv_heads;
  p.G = G;
  p.W = (seq_len + 31) / 32;
  p.n_rt = (int)n_rt;
  p.n_wg = (int)n_wg;
  // exp(x) = 2^(x log2 e): fold log2(e) into the scale.  A zero scale becomes a tiny positive
  // one (2^-100): every 2^(s*c - m) is then 1 to fp32 precision, the uniform average the zero
  // scale defines, without 0 * inf on masked scores.
  const float c = fabsf(scale) * 1.4426950408889634f;
  p.c = c > 0x1p-100f ? c : 0x1p-100f;
  p.qflip = scale < 0.f ? 0x80008000u : 0u;

  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dtype == FA_DTYPE_BF16;
  hipError_t e;
  if (bf16)
    e = head_dim == 128 ? launch_mode<true, 128>(mask_mode, p, s) : launch_mode<true, 64>(mask_mode, p, s);
  else
    e = head_dim == 128 ? launch_mode<false, 128>(mask_mode, p, s) : launch_mode<false, 64>(mask_mode, p, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
