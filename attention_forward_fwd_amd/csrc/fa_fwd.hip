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
//   * Work: one workgroup = 4 or 8 waves x 32 rows (8 when a KV head has many rows: each K/V
//     tile staged in LDS then serves 256 rows).  A "row" is a (position, query head) pair; the
//     rows of one KV head are ordered position-major, head-minor (row r -> position r / G,
//     head hk*G + r % G), so a workgroup covers every query head of a GQA group at the same
//     positions and each K/V tile staged in LDS feeds G heads.  Two waves per SIMD either way.
//   * Matrix cores: v_mfma_f32_32x32x16_{bf16,f16}.  S^T = K Q^T puts one query in each lane
//     column (lane l holds query l%32 and 16 keys per 32-key block), so the row max and row sum
//     are in-lane reductions plus one v_permlane32_swap, and the rescale of O^T += V^T P^T
//     touches only the lane's own query.  P never leaves registers: the S^T accumulator layout
//     is re-used directly as the B operand of the P V product (keys permuted consistently on
//     both operands).
//   * Pipeline: per 64-key tile, one instruction stream runs O += V_{j-1}^T P_{j-1}^T and
//     S_{j+1} = K_{j+1} Q^T on the matrix cores while the vector units run the softmax of S_j,
//     each matrix instruction with a share of the vector work and of the tile's loads; one
//     workgroup barrier per tile.
//   * Memory: K tiles go global -> LDS by buffer-load DMA (no registers) into 1 KiB regions of
//     whole rows, padded so the 128-bit operand reads are conflict-free.  V reaches the P V
//     product either as V^T tiles packed once per call by vt_pack_kernel (8 keys of one head_dim
//     column per 128-bit operand, in the key order of the P registers), copied the same way, or,
//     when few workgroups share a KV head, as V's own rows copied like K and transposed by the
//     operand reads (two ds_read_b64_tr_b16 per operand).  Buffer resources end at the sequence:
//     key rows past it read as zeros and are masked, so their probabilities are exactly 0.  Q is
//     staged once through LDS into registers.
//   * Softmax: exp2 with log2(e) folded into the scale, running max floored at -1e30 so a
//     fully masked row never makes NaN.  Causal and ragged tiles set masked scores to -inf (one
//     bit-field extract and one 3-input bit operation per score); with a bit mask the keep bits
//     clear the packed weights after the exp (1.5 instructions per key).  The running max
//     starts at the first tile's row max and is lazy, checked after the fact: a tile's weights
//     are formed against the max as it stands, and only when some lane's sum of them exceeds
//     2^15 (which bounds every weight) does the wave take the tile's row max and redo the tile,
//     rescaling O and the row sum (every lane multiplies: no per-lane branch).  With it the
//     common tile needs no row max and no rescale.
//   * Skips: per wave and tile, the keep bits of the wave's rows are voted with a 64-lane
//     ballot.  A skipped tile's weights are exactly 0.  Causal workgroups stop at their last
//     live tile, and on the diagonal tail (and in the walk over a mask summary) a wave whose
//     tiles j-1 and j+1 are both dead skips the iteration's matrix work.
//   * Scheduling: workgroups are remapped so each of the 8 XCDs gets a contiguous range of
//     tiles (tiles of one KV head share that XCD's L2); causal row tiles run longest first,
//     ordered so each XCD's four shader engines get equal work.
//   * Optional outputs and schedules (fa_fwd_ex): each row's log-sum-exp from the running
//     softmax state; in bitmask mode a walk over only the key tiles a per-block mask summary
//     marks live (no loads for the others); split-KV, where shares of a row tile's key range
//     run in separate workgroups and merge_kernel combines their (max, sum, O) states.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

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
  const uint16_t* vt;  // packed V^T tiles (see VtPack), when the kernel reads V that way
  uint16_t* o;
  float* lse;  // [B, Hq, S] log-sum-exp of each row's kept scores, or null
  const u32* tiles;  // bitmask mode: [B, Hq, n_rb, TW] summary of 64x64 blocks with a kept bit,
                     // or null (then every key tile is visited)
  int n_rb, TW;      // 64-row blocks per head, summary words per block
  int n_split;       // key ranges each row tile is split into (1 = none)
  float* o_part;     // n_split > 1: [n_split, B*S*Hq, D] unnormalised fp32 O of each key range
  float* ml_part;    // n_split > 1: [n_split, B*S*Hq, 2] running max and row sum of each range
  size_t part_rows;  // B*S*Hq
  int S, Hq, Hkv, G, W;
  int n_kt;   // 64-key tiles per sequence
  int n_rt;   // row tiles per (batch, kv head)
  int n_wg;   // workgroups in the grid
  int xsplit; // XCDs sharing one (batch, KV head) of causal row tiles, or 0
  float c;    // |scale| * log2(e), floored at 2^-100
  u32 qflip;  // 0x80008000 when scale < 0 (moves the sign onto Q exactly), else 0
};

// Tile shape: NW waves of 32 rows each per workgroup, 64 keys per tile, two waves per SIMD
// either way: NW = 4 with two workgroups per CU (the two waves of a SIMD come from different
// workgroups, so one wave's vector work runs while the other's matrix work occupies the matrix
// cores), or NW = 8 with one workgroup per CU (each K and V tile staged in LDS then serves 256
// rows: half the global->LDS traffic per FLOP), used when a KV head has many rows.
constexpr int kBN = 64;           // keys per tile
constexpr int kWide = 8;          // waves of the 256-row workgroup
#ifndef FA_WIDE_ROWS
#define FA_WIDE_ROWS 2048
#endif
#ifndef FA_WIDE_ROWS_D128
#define FA_WIDE_ROWS_D128 512
#endif
#ifndef FA_WIDE_ROWS_CAUSAL
#define FA_WIDE_ROWS_CAUSAL 8192
#endif
constexpr int kWideRows = FA_WIDE_ROWS;   // rows per KV head (S x G) from which it is used (d=64)
constexpr int kWideRows128 = FA_WIDE_ROWS_D128;  // (d=128: its tiles cost twice the matrix work)
constexpr int kWideRowsCausal = FA_WIDE_ROWS_CAUSAL;   // (causal at d=64: its short tiles favour 128 rows below)
#ifndef FA_WIDE_ROWS_CAUSAL_D128
#define FA_WIDE_ROWS_CAUSAL_D128 2048
#endif
constexpr int kWideRowsCausal128 = FA_WIDE_ROWS_CAUSAL_D128;  // causal at d=128
// Row tiles per KV head from which V is packed once per call (below it, each workgroup reads V's
// rows through transposing LDS reads: the pre-pass costs more than those reads save).
#ifndef FA_PACK_ROW_TILES
#define FA_PACK_ROW_TILES 32
#endif
constexpr int kPackRowTiles = FA_PACK_ROW_TILES;
// (causal at d=128 does half the work per row tile, so the pre-pass pays off only from 64)
#ifndef FA_PACK_ROW_TILES_CAUSAL_D128
#define FA_PACK_ROW_TILES_CAUSAL_D128 64
#endif
constexpr int kPackRowTilesCausal128 = FA_PACK_ROW_TILES_CAUSAL_D128;
constexpr int kMaxListTiles = 2048;  // key tiles a workgroup can list from a tile summary
constexpr int kMaxSplits = 16;       // key ranges per row tile (split-KV)
constexpr int kNumCUs = 256;         // MI355X compute units (automatic split-KV sizing)
#ifndef FA_QK_AHEAD
#define FA_QK_AHEAD 3
#endif

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

// LDS layout of a transposed V tile in the packing pre-pass.  Row d (one head_dim index) holds
// the tile's BN = 64 keys as 8 "units" of 16 bytes: unit (ks, hl) holds keys 16ks + 4hl + 0..3
// (first 8 bytes) and 16ks + 8 + 4hl + 0..3 (last 8 bytes), exactly the 8 keys, in register
// order, that lane half hl of an MFMA needs at k-step ks of P V (the packed tile keeps the
// units, so each V^T operand of the attention kernel is one 128-bit read).  Units of one
// k-step and one 32-row block of d form a 1 KiB region (4 lines of 8 rows x 2 units), padded
// to RGS bytes; within a line, unit hl of row d sits at 16-byte slot
// (2 (d % 8) + hl) ^ ((d / 8) % 4) ^ x(hl).  With 64 banks x 4 B:
//   * an operand read (16 lanes: one unit of 16 consecutive rows) touches every bank once, and
//     its address is one per-lane base plus the compile-time offset ks*KSS + block*RGS;
//   * a staging write (32 lanes: column 8dq + jj of 16 column chunks dq, both halves; at d=64
//     8 chunks x both lane halves) touches every bank once: the padding shifts the regions of
//     consecutive 32-row blocks by 16 (d=128) or 32 (d=64) banks, and x(hl) = 4 hl at d=64
//     moves the two lane halves to different slot quads.  The write addresses of one thread
//     are two (d=128) or four (d=64) bases plus multiples of 64 bytes.
template <int D>
struct Vt {
  static constexpr int RGS = D == 128 ? 1088 : 1152;
  static constexpr int KSS = (D / 32) * RGS;  // one k-step: D/32 regions
  static constexpr int BYTES = 4 * KSS;
  __device__ static constexpr int x(int hl) { return D == 64 ? 4 * hl : 0; }
  __device__ static constexpr int off(int d, int ks, int hl, int half) {
    return ks * KSS + (d >> 5) * RGS + ((d >> 3) & 3) * 256 +
           (((2 * (d & 7) + hl) ^ ((d >> 3) & 3) ^ x(hl)) * 16) + half * 8;
  }
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// DMA of one 16-byte chunk per lane from a buffer resource into LDS: lane i writes dst + 16 i.
// Compiled in the device pass only: with this builtin in a kernel body, the host pass of the
// compiler omits the kernel's launch stub.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_void* dst, unsigned voff,
                                      unsigned soff = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
#endif
}

// s_waitcnt immediate: vmcnt(vm) with expcnt and lgkmcnt at `lgkm` (15 = no wait).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// Workgroup barrier of the tile pipeline.  The caller first waits (s_waitcnt) for the memory
// operations that other waves must see: its LDS writes and all of its global->LDS copies.  A
// vector load it issues after that wait (a register load that no other wave reads) may stay in
// flight, which a partial wait could not express safely: the compiler is free to issue a tile's
// loads in any order.  (__syncthreads would also drain that load: its workgroup-scope fence
// waits for every outstanding load.)  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void pipeline_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer resource over rows [key0, S) of a [S, row_elems]-strided tensor slice starting at
// `base`: rows at or past S lie outside it, their reads return zeros and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int key0, int S,
                                                            int row_elems) {
  const unsigned rows = (unsigned)max(S - key0, 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)key0 * row_elems), (short)0,
                                           (int)(rows * (unsigned)row_elems * 2u), 0x00020000);
}

// Per-thread V transpose for one 64-key tile (the packing pre-pass): thread t < THREADS owns column chunk dq (head_dim
// 8dq..8dq+7) of key quad q (keys 4q..4q+3).  Consecutive lanes take consecutive column chunks
// of one key row, so every load instruction reads whole rows.  Lanes 16-31 take quad q+2 (same
// V^T unit, other half) so the two 16-lane halves of a write never share a bank.  The four
// 16-byte pieces (one per key) are loaded into registers, then transposed with byte permutes
// into eight 8-byte pieces (one per column) and written at their V^T unit: unit (q/4, q%2),
// half (q/2)%2.
template <int D, int NT>
struct VStage {
  static constexpr int THREADS = 16 * (D / 8);
  static constexpr int VP = D == 128 ? 2 : 4;  // write address bases (see Vt)
  bool active;
  unsigned off;  // byte offset of this thread's first key row and column chunk
  int base[VP];  // LDS offset of column 8dq + r, r < VP
  __device__ VStage(int tid, unsigned row_bytes) {
    const int dq = D == 128 ? (tid & 15) : (tid & 7);
    const int qi = D == 128 ? (tid >> 4) : (tid >> 3);
    const int q = 4 * (qi >> 2) + ((qi >> 1) & 1) + 2 * (qi & 1);
    active = THREADS >= NT || tid < THREADS;
    off = (unsigned)(4 * q) * row_bytes + 16u * dq;
#pragma unroll
    for (int r = 0; r < VP; ++r) base[r] = Vt<D>::off(8 * dq + r, q >> 2, q & 1, (q >> 1) & 1);
  }
  // Keys key0 + 4q + kk of the V slice at `v` (rows of row_elems elements, S valid rows).
  __device__ __forceinline__ void load(u32x4 (&st)[4], const uint16_t* v, int key0, int S,
                                       int row_elems) const {
    if (active) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        st[kk] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rows_rsrc(v, key0 + kk, S, row_elems), off, 0, 0));
    }
  }
  // Column 8dq + jj at base[jj % VP] + 32 (jj - jj % VP).
  __device__ __forceinline__ void store(const u32x4 (&st)[4], unsigned char* vt) const {
    if (active) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int m = jj >> 1;
        const u32 sel = (jj & 1) ? 0x07060302u : 0x05040100u;  // high / low 16-bit halves
        const u32x2 col = {__builtin_amdgcn_perm(st[1][m], st[0][m], sel),
                           __builtin_amdgcn_perm(st[3][m], st[2][m], sel)};
        *(u32x2*)(vt + base[jj % VP] + (jj - jj % VP) * 32) = col;
      }
    }
  }
};

// Packed V^T tiles in device memory, and their LDS image: for each (batch, KV head, 64-key
// tile), 4 * D/32 regions of 1 KiB, region r = ks * D/32 + db for k-step ks and 32-row block db
// of head_dim.  Slot t (16 bytes) of a region holds unit (ks, hl = t / 32) of row 32 db + t % 32
// (the units of Vt).  An MFMA operand read of region r is then lane l -> slot l: 64 lanes read
// 1 KiB of consecutive slots, which touches every LDS bank the same number of times whatever
// the number of lanes served per cycle; and one DMA instruction copies one region (lane i ->
// 16 i).
template <int D>
struct VtPack {
  static constexpr int NREG = 4 * (D / 32);
  static constexpr int TILE = NREG * 1024;
};

// Packs V [B, S, Hkv, D] into VtPack tiles: one workgroup per (batch, KV head, key tile), a
// register transpose (VStage) into LDS, then a linear copy LDS -> memory.  Keys at or past S
// are zeros.
template <int D>
__global__ __launch_bounds__(256) void vt_pack_kernel(const uint16_t* __restrict__ v,
                                                      uint16_t* __restrict__ vt, int S, int Hkv,
                                                      int n_kt) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[Vt<D>::BYTES];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int kt = tile % n_kt, bh = tile / n_kt, hk = bh % Hkv, b = bh / Hkv;
  const int row_elems = Hkv * D;
  const uint16_t* vg = v + ((size_t)b * S * Hkv + hk) * D;
  const VStage<D, 256> st(tid, (unsigned)row_elems * 2u);
  u32x4 x[4];
  st.load(x, vg, kt * 64, S, row_elems);
  st.store(x, lds);
  __syncthreads();
  unsigned char* out = (unsigned char*)vt + (size_t)tile * VtPack<D>::TILE;
#pragma unroll
  for (int i = 0; i < VtPack<D>::TILE / 16 / 256; ++i) {
    const int c = tid + 256 * i, r = c >> 6, t = c & 63;
    const int ks = r / (D / 32), db = r % (D / 32);
    *(u32x4*)(out + (size_t)c * 16) =
        *(const u32x4*)(lds + Vt<D>::off(32 * db + (t & 31), ks, t >> 5, 0));
  }
}

template <bool BF16, int D, int MODE, bool VPACK, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void fa_fwd_kernel(Params p) {
  // VPACK: V arrives as packed V^T tiles (vt_pack_kernel) by DMA; otherwise V's rows arrive by
  // DMA like K and the operand reads transpose them.
  constexpr int BM = NW * 32, BN = kBN, NT = NW * 64;
  static_assert(NW == 4 || NW == 8, "workgroup shape");
  constexpr int KC = D / 8;        // 16-byte chunks per row
  constexpr int NKB = BN / 32;     // 32-key blocks per tile (one MFMA output block each)
  constexpr int QKS = D / 16;      // MFMA k-steps of Q K^T
  constexpr int NDB = D / 32;      // 32-wide blocks of head_dim in O
  constexpr int PKS = BN / 16;     // MFMA k-steps of P V
  using L = Lds<D>;
  constexpr int RPR = L::RPR, RS = L::RS;
  constexpr int NREG = BN / RPR;     // regions per tile
  constexpr int T_BYTES = NREG * RS; // one K tile (BN rows)
  constexpr int VT_BYTES = VPACK ? VtPack<D>::TILE : T_BYTES;  // one packed V^T tile, or V rows
  constexpr int M_WORDS = MODE == kBitmask ? BM * NKB : 1;
  constexpr int DMA_PER_WAVE = NREG / NW;             // one region per DMA instruction
  constexpr int QROWS = 2 * BN;                       // Q rows staged per pass (two K buffers)
  constexpr int QPASS = BM / QROWS;                   // passes
  constexpr int QL = QROWS * KC / NT;                 // Q chunks staged per thread and pass
  static_assert(BM % QROWS == 0 && QL >= 1, "Q staging uses the two K buffers, BN rows each");
  static_assert(DMA_PER_WAVE * NW == NREG && QL * NT == QROWS * KC, "load split");
  static_assert(BN == 64, "64-key tiles");

  // Separate arrays (not one array indexed by buffer) so the compiler can tell the DMA into one
  // buffer from LDS reads of another and does not wait for the DMA before those reads.
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[T_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[T_BYTES];
  // V^T tiles (also the Q staging area, hence at least one K tile's size)
  constexpr int VBUF_BYTES = VT_BYTES > T_BYTES ? VT_BYTES : T_BYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[VBUF_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[VBUF_BYTES];
  __shared__ __attribute__((aligned(16))) u32 m_lds0[M_WORDS];
  __shared__ __attribute__((aligned(16))) u32 m_lds1[M_WORDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;   // lane column and lane half
  const int S = p.S, G = p.G, Hq = p.Hq, Hkv = p.Hkv;

  // XCD-aware remap: the hardware deals workgroup i to XCD i % 8.  Give XCD x the contiguous
  // logical range so that row tiles of one KV head (which read the same K/V) share an L2.
  // Causal row tiles of a (batch, KV head) run longest first.  When one head's row tiles are
  // shared by xsplit > 1 XCDs (a long sequence with few heads), its tiles are dealt round-robin
  // among them instead, so that those XCDs get equal causal work.
  int wg = blockIdx.x;
  {
    const int x = wg & 7;
    int idx = wg >> 3;
    // Within an XCD the hardware deals workgroup idx to shader engine idx % 4 (a fixed order of
    // its four engines) and starts workgroups in index order, so an engine whose next workgroup
    // cannot start yet holds back the others.  Causal row tiles shorten along the order, so
    // every second aligned group of four runs reversed: over each pair of groups every engine
    // then gets the same number of key tiles.  (A last, incomplete group keeps its order.)  With
    // fewer than four rounds of resident workgroups per XCD the plain longest-first order
    // measured better, so the reversal starts from four.
#ifndef FA_SE_SNAKE
#define FA_SE_SNAKE 1
#endif
    if (MODE == kCausal && FA_SE_SNAKE) {
      const int share = (p.n_wg >> 3) + (x < (p.n_wg & 7) ? 1 : 0);
      constexpr int kResident = (kNumCUs / 8) * (NW == kWide ? 1 : 2);  // per XCD
      if (share >= 4 * kResident && ((idx >> 2) & 1) && (idx | 3) < share) idx ^= 3;
    }
    if (MODE == kCausal && p.xsplit > 1) {
      wg = (x / p.xsplit) * p.n_rt + (x % p.xsplit) + p.xsplit * idx;
    } else {
      const int q8 = p.n_wg >> 3, r8 = p.n_wg & 7;
      wg = x * q8 + min(x, r8) + idx;
    }
  }
  // Split-KV: the key ranges of one row tile are consecutive logical workgroups (same XCD).
  int split = 0;
  if (p.n_split > 1) {
    split = wg % p.n_split;
    wg /= p.n_split;
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

  // Bitmask mode with a tile summary: the workgroup visits only the key tiles in which some row
  // of its positions and heads keeps a key (the OR of the summary words of its G heads and the
  // 64-row blocks its positions touch; a superset of the live tiles, so nothing kept is
  // dropped), listed in LDS in increasing order.  Waves still skip the listed tiles they have
  // no kept bit in by the ballot.  Tile j of the walk is tix(j).
  __shared__ uint16_t tlist[MODE == kBitmask ? kMaxListTiles : 1];
  __shared__ int tcount;
  bool sparse = false;
  if constexpr (MODE == kBitmask) {
    if (p.tiles) {
      sparse = true;
      if (wave == 0) {
        const int rb0 = (row0 / G) / 64, rb1 = min((row0 + BM - 1) / G, S - 1) / 64;
        u32 word = 0u;
        if (lane < p.TW) {  // TW <= 64 words of 32 tiles
          for (int g = 0; g < G; ++g)
            for (int rb = rb0; rb <= rb1; ++rb)
              word |= p.tiles[(((size_t)b * Hq + hk * G + g) * p.n_rb + rb) * p.TW + lane];
        }
        // exclusive prefix sum of the popcounts over the 64 lanes, then each lane lists its bits
        const int pc = __popc(word);
        int incl = pc;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(incl, d);
          if (lane >= d) incl += y;
        }
        int pos = incl - pc;
        while (word) {
          const int bit = __ffs((int)word) - 1;
          tlist[pos++] = (uint16_t)(lane * 32 + bit);
          word &= word - 1u;
        }
        if (lane == 63) tcount = incl;
      }
      __syncthreads();
      n_tiles = __builtin_amdgcn_readfirstlane(tcount);
    }
  }
  // Split-KV (never with a tile summary): key range `split` of n_split equal shares of this
  // workgroup's tiles.
  int kt0 = 0;
  if (p.n_split > 1) {
    const int chunk = (n_tiles + p.n_split - 1) / p.n_split;
    kt0 = split * chunk;
    n_tiles = max(0, min(n_tiles - kt0, chunk));
  }
  auto tix = [&](int j) __attribute__((always_inline)) {
    const int jj = min(j, n_tiles - 1);
    if constexpr (MODE == kBitmask) {
      if (sparse) return __builtin_amdgcn_readfirstlane((int)tlist[jj]);
    }
    return kt0 + jj;
  };
  // Row index of O (and of the split partials): (b, position, query head), token-major.
  const size_t orow_idx = ((size_t)b * S + my_pos) * Hq + my_head;
  if (n_tiles == 0) {  // (tile summary or an empty key range) no key of these rows is visited
    if (wave_live && my_pos < S) {
      if (p.n_split > 1) {  // empty partial: max at the floor, sum 0, O 0
        float* op = p.o_part + ((size_t)split * p.part_rows + orow_idx) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) *(f32x4*)(op + 32 * db + 8 * t4 + 4 * hl) = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (hl == 0)
          *(float2*)(p.ml_part + ((size_t)split * p.part_rows + orow_idx) * 2) = make_float2(-1e30f, 0.f);
      } else {
        uint16_t* orow = p.o + q_batch + ((size_t)my_pos * Hq + my_head) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) *(u32x2*)(orow + 32 * db + 8 * t4 + 4 * hl) = (u32x2){0u, 0u};
        if (p.lse && hl == 0) p.lse[((size_t)b * Hq + my_head) * S + my_pos] = -INFINITY;
      }
    }
    return;
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

  // ---- Q: coalesced 128-bit loads -> LDS (2 BN rows per pass, through the two V^T buffers:
  // rows 0..63 of the pass in v_lds0, 64..127 in v_lds1, K layout) -> MFMA B operands held in
  // registers for the whole key loop.  Staged in the prologue below.
  u32x4 qreg[QKS];
  auto q_load = [&](int pass, u32x4 (&qx)[QL]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int id = tid + NT * i, r = id / KC, c = id % KC;
      const int grow = row0 + pass * QROWS + r, pos = grow / G, h = hk * G + (grow - pos * G);
      qx[i] = (u32x4){0u, 0u, 0u, 0u};
      if (pos < S) qx[i] = *(const u32x4*)(p.q + q_batch + ((size_t)pos * Hq + h) * D + c * 8);
    }
  };

  const unsigned row_bytes = (unsigned)kv_stride * 2u;

  // ---- K staging by DMA (buffer load into LDS): instruction i of this wave fills region
  // n = i*NW + wave; lane = slot s holds chunk s / RPR of row n*RPR + ((s % RPR) ^ x(chunk)).
  // One buffer resource over this (batch, KV head)'s S key rows: a row at or past S is outside
  // it and reads as zeros (its scores are masked in any case); the tile's first row is a scalar
  // offset, clamped to S so it stays below 2^32.
  const int dma_c = lane / RPR;
  const unsigned dma_off = (unsigned)((lane % RPR) ^ L::x(dma_c)) * row_bytes + dma_c * 16u;
  const __amdgpu_buffer_rsrc_t k_rsrc = rows_rsrc(kg, 0, S, kv_stride);
  auto dma_rows = [&](__amdgpu_buffer_rsrc_t rsrc, int j, unsigned char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int n = i * NW + wave;
      const unsigned row = (unsigned)min(j * BN + n * RPR, S);
      dma16(rsrc, (lds_void*)(dst + n * RS), dma_off, row * row_bytes);
    }
  };
  auto dma_tile = [&](int j, unsigned char* dst) __attribute__((always_inline)) { dma_rows(k_rsrc, j, dst); };

  // ---- V staging.  VPACK: one DMA instruction per 1 KiB region of a packed V^T tile (lane i
  // -> 16 i), instruction i of this wave taking region i*NW + wave.  Otherwise V's rows by DMA
  // into the K layout, like K (the operand reads transpose them).
  constexpr int VDMA_PER_WAVE = VPACK ? VtPack<D>::NREG / NW : DMA_PER_WAVE;
  static_assert(!VPACK || VDMA_PER_WAVE * NW == VtPack<D>::NREG, "packed V^T regions split over waves");
  const __amdgpu_buffer_rsrc_t v_rsrc =
      VPACK ? __builtin_amdgcn_make_buffer_rsrc(
                  (void*)(p.vt + (size_t)bh * p.n_kt * (VtPack<D>::TILE / 2)), (short)0,
                  p.n_kt * VtPack<D>::TILE, 0x00020000)
            : rows_rsrc(vg, 0, S, kv_stride);
  auto v_dma = [&](int j, unsigned char* dst) __attribute__((always_inline)) {
    if constexpr (VPACK) {
#pragma unroll
      for (int i = 0; i < VDMA_PER_WAVE; ++i) {
        const int n = i * NW + wave;
        dma16(v_rsrc, (lds_void*)(dst + n * 1024), lane * 16u + n * 1024u,
              (unsigned)(j * VtPack<D>::TILE));
      }
    } else {
      dma_rows(v_rsrc, j, dst);
    }
  };

  // Mask words (bitmask mode): thread t stages word t / BM of row t % BM for a tile (NKB = 2
  // words per row, so the BM x NKB words of a tile take one load per thread).  The row pointer
  // is clamped to a valid row and the word index to the row length, so the load needs no
  // branch; words of rows >= S or past the row end are then replaced by 0.  A tile's words are
  // loaded into a register at the end of the iteration two before the one that stores them to
  // LDS, after that iteration's wait for all of its loads: the load (from HBM: every word is
  // read once) then has a whole iteration to arrive, and it is the only vector load a wave has
  // in flight at the barrier, so no wait ever depends on the order in which the compiler issues
  // the tile's loads.
  static_assert(MODE != kBitmask || BM * NKB == NT, "one mask word per thread and tile");
  u32 mreg = 0u;        // the word most recently loaded ...
  bool mvalid = false;  // ... and whether it is a real word of a valid row (applied at the store,
                        // so no wait for the load is forced where it is issued)
  const u32* mrow = nullptr;
  bool mrow_ok = false;
  const int m_row = tid % BM, m_word = tid / BM;
  if (MODE == kBitmask) {
    const int grow = row0 + m_row, pos = grow / G, h = hk * G + (grow - pos * G);
    mrow_ok = pos < S;
    mrow = p.mask + (((size_t)b * Hq + h) * S + min(pos, S - 1)) * (size_t)p.W;
  }
  auto mask_load = [&](int j) __attribute__((always_inline)) {
    if (MODE == kBitmask) {
      const int word = j * NKB + m_word;
      mreg = mrow[min(word, p.W - 1)];
      mvalid = mrow_ok && word < p.W;
    }
  };
  auto mask_store = [&](u32* mb) __attribute__((always_inline)) {
    if (MODE == kBitmask) mb[m_row * NKB + m_word] = mvalid ? mreg : 0u;
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

  // V^T operand (A of O^T += V^T P^T): head_dim row 32*db + l%32 of the 32-row block, the 8 keys
  // of k-step ks that lane half hl multiplies (16ks + 4hl + 0..3, then 16ks + 8 + 4hl + 0..3).
  // VPACK: region ks * D/32 + db of the packed tile, slot = lane, one 128-bit read.  Otherwise
  // two ds_read_b64_tr_b16 of the V rows: that instruction transposes 16-bit elements within
  // each 16-lane group, lane j receiving element j%4 of the 8 bytes addressed by lane j/4 + 4t
  // as its element t (t = 0..3).  Lane l (index i = l%16 in its group) therefore addresses key
  // row 16ks + 4hl + i/4 (+8 for the second read), head_dim columns 32db + 16((l/16)%2) +
  // 4(i%4) + 0..3, and receives keys 16ks + 4hl + 0..3 of column 32db + l%32.
  const int vt_base = lane * 16;
  const int tr_base = L::off(4 * hl + ((lane & 15) >> 2), (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) >> 3) +
                      8 * (lane & 1);
  constexpr int TR_KS = (16 / RPR) * RS, TR_H = (8 / RPR) * RS, TR_DB = 4 * RPR * 16;
  auto v_operand = [&](const unsigned char* vb, int ks, int db) __attribute__((always_inline)) {
    if constexpr (VPACK) {
      return *(const u32x4*)(vb + vt_base + (ks * (D / 32) + db) * 1024);
    } else {
      const int oa = tr_base + ks * TR_KS + db * TR_DB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + oa));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + oa + TR_H));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      return (u32x4){lo2[0], lo2[1], hi2[0], hi2[1]};
    }
  };

  // ---- Tile pipeline ("tile j" is the j-th tile of the walk: tix(j)).  Iteration j holds S_j
  // (computed one iteration earlier) and P_{j-1} (its softmax, one iteration old), and runs one
  // instruction stream in which three independent pieces of work are interleaved:
  //   * S_{j+1} = K_{j+1} Q^T                 (matrix cores, K operands from LDS),
  //   * O += V_{j-1}^T P_{j-1}^T              (matrix cores, V^T operands from LDS, P in registers),
  //   * the masked online softmax of S_j -> P_j and its row sums (vector units),
  // so every matrix instruction of the tile has vector work of the softmax beside it; then the
  // sum check (softmax_finish), which in the rare case redoes the tile against its row max and
  // rescales O before the next iteration adds V_j^T P_j^T.  The iteration also issues the loads
  // of K_{j+2} and V_j (DMA into LDS), waits for them, stores the mask words of tile j+2 (loaded
  // at the end of the previous iteration) to LDS, issues the load of those of tile j+3 (into a
  // register), and ends at the one workgroup barrier of the tile.  The keep words of tile j are carried in registers
  // from iteration j-1, so the mask buffer of tile j can be refilled during iteration j.  After
  // the last iteration one more V^T P^T product remains.  Loads past the last tile re-read the
  // last tile (in bounds, never used).

  // The matrix instructions of one iteration, in one index space: i < NPV are O^T += V^T P^T
  // (k-step i / NDB, head_dim block i % NDB: k-step major, so each P register is dead after its
  // NDB instructions), the next NQK are S^T = K Q^T (k-step t / NKB, 32-key block t % NKB, t =
  // i - NPV).  Each LDS operand is read AH matrix instructions ahead into a ring of AH + 1
  // registers indexed by i, across the boundary of the two products.
  constexpr int NQK = QKS * NKB, NPV = PKS * NDB, NMM = NPV + NQK;
  constexpr int AH = FA_QK_AHEAD;
  auto mm_operand = [&](int i, const unsigned char* kb, const unsigned char* vb)
                        __attribute__((always_inline)) {
    if (i < NPV) return v_operand(vb, i / NDB, i % NDB);
    const int t = i - NPV;
    return *(const u32x4*)(kb + op_addr(t / NKB, t % NKB));
  };
  // Operands of instructions i0 .. i0 + AH - 1 (those below iend).
  auto mm_prefetch = [&](int i0, int iend, u32x4 (&op)[AH + 1], const unsigned char* kb,
                         const unsigned char* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < AH; ++a)
      if (i0 + a < iend) op[(i0 + a) % (AH + 1)] = mm_operand(i0 + a, kb, vb);
  };
  // Instructions i0 .. i1 - 1, reading the operand of i + AH (below iend) before each.
  auto mm_run = [&](int i0, int i1, int iend, u32x4 (&op)[AH + 1], const unsigned char* kb,
                    f32x16 (&s)[NKB], const unsigned char* vb, const u32x4 (&pk)[PKS])
                    __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMM; ++i) {
      if (i < i0 || i >= i1) continue;
      if (i + AH < iend) op[(i + AH) % (AH + 1)] = mm_operand(i + AH, kb, vb);
      const u32x4 a = op[i % (AH + 1)];
      if (i < NPV) {
        oacc[i % NDB] = mfma32<BF16>(a, pk[i / NDB], oacc[i % NDB]);
      } else {
        const int t = i - NPV;
        if (t < NKB) {  // first k-step of a 32-key block: accumulate onto zero
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          s[t % NKB] = mfma32<BF16>(a, qreg[t / NKB], z);
        } else {
          s[t % NKB] = mfma32<BF16>(a, qreg[t / NKB], s[t % NKB]);
        }
      }
    }
  };

  // Masked scores -> -inf (a bit-field extract of the keep bit, then one 3-input bit operation
  // that selects s or -inf), for tiles that are not full (with a bit mask: only for a row max,
  // in the prologue and the redo).  A tile with all-zero keep words becomes all -inf, whatever
  // s held.
  auto mask_block = [&](const Cls& cls, f32x16 (&s)[NKB], int kb32) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bit = 8 * (r >> 2) + (r & 3);
      const int keep = ((int)(cls.wsh[kb32] << (31 - bit))) >> 31;
      s[kb32][r] = __int_as_float((__float_as_int(s[kb32][r]) & keep) | (~keep & (int)0xff800000));
    }
  };
  auto mask_scores = [&](const Cls& cls, f32x16 (&s)[NKB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) mask_block(cls, s, kb32);
  };

  // Online softmax of one tile's (masked) scores with a lazy running max that is checked after
  // the fact.  Each 32-key block's P = 2^(s c - m) is formed with the running max m as it stands
  // (softmax_block, one block beside each of the iteration's two products), rounded to the input
  // dtype into pk (slots 0..3 of lane half hl: keys 16ks + 4hl + 0..3, slots 4..7: keys
  // 16ks + 8 + 4hl + 0..3, the key order of a V^T unit), and summed per lane from the rounded
  // values (v_dot2 against (1, 1)), so numerator and denominator see the same P.  The weights
  // are >= 0, so a lane's sum bounds each of its weights: when no lane's sum exceeds kSumBound
  // (the common case) the tile is done with alpha = 1 and no row max at all.  Otherwise -- a
  // row's first kept key past its first tile (m still at its -1e30 floor, set from the first
  // tile's row max before the loop, makes the weights infinite), or scores that rose far above
  // m -- the wave recomputes the tile (softmax_finish): the row max, m_new,
  // alpha = 2^(m_old - m_new), P and the sums.  Every weight therefore stays below kSumBound
  // (finite in fp16, far from overflow in the fp32 sums), and O / l and the LSE are the same
  // function of (m, l) whatever m is.  An all -inf tile gives P = 0 and leaves m and l alone.
  constexpr float kSumBound = 32768.f;  // 2^15
  float ps_sm[2];
  // Bitmask mode applies the keep bits to the packed weights (masked = true, w = the block's
  // pre-shifted keep word): a register of P holds two consecutive keys of the lane, bits b and
  // b+1 of w for the block's first 16 keys (b = 0, 2, 8, 10) and b+16, b+17 for the last 16.
  // w << (15 - k) puts bit k at bit 15 and bit k+16 at bit 31, the bits v_perm_b32's selectors
  // 8..11 replicate into a byte, so one permute of two such words gives a register's mask
  // (0xffff per kept half): 1.5 vector instructions per key instead of the 2 of mask_block.
  // The weights of masked keys are computed and then cleared (an infinite one included; s is
  // finite), and the row sums add the cleared values.
  auto exp_block = [&](f32x16 (&s)[NKB], u32x4 (&pk)[PKS], int kb32, auto masked, u32 w)
                       __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    u32 a[8];
    if constexpr (MASKED) {
      constexpr int kq[8] = {0, 1, 2, 3, 8, 9, 10, 11};
#pragma unroll
      for (int q = 0; q < 8; ++q) a[q] = w << (15 - kq[q]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x8 t;
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = __builtin_amdgcn_exp2f(fmaf(s[kb32][8 * h + e], c, -m_run));
      u32x4 pw = pack8<BF16>(t);
      if constexpr (MASKED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q0 = 2 * (e & 1) + 4 * (e >> 1);
          pw[e] &= __builtin_amdgcn_perm(a[q0 + 1], a[q0], h ? 0x0B0B0909u : 0x0A0A0808u);
        }
      }
      pk[2 * kb32 + h] = pw;
#pragma unroll
      for (int e = 0; e < 4; ++e) ps_sm[e & 1] = dot2_ones<BF16>(pw[e], ps_sm[e & 1]);
    }
  };
  constexpr bool PAIR_MASK = MODE == kBitmask;  // keep bits applied to the packed weights
  auto softmax_block = [&](const Cls& cls, f32x16 (&s)[NKB], u32x4 (&pk)[PKS], int kb32)
                           __attribute__((always_inline)) {
    if (kb32 == 0) ps_sm[0] = ps_sm[1] = 0.f;
    if constexpr (PAIR_MASK) exp_block(s, pk, kb32, std::true_type{}, cls.wsh[kb32]);
    else exp_block(s, pk, kb32, std::false_type{}, 0u);
  };
  // Row max of a tile's (masked) scores: two in-lane chains of 3-input maxima (v_max3_f32), one
  // per 32-key block, then across the two lane halves.
  auto row_max = [&](const f32x16 (&s)[NKB]) __attribute__((always_inline)) {
    float mx2[NKB];
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) {
      const f32x16& v = s[kb32];
      float m = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, v[e]), v[e + 1]);
      mx2[kb32] = __builtin_fmaxf(m, v[15]);
    }
    static_assert(NKB == 2, "two 32-key blocks per tile");
    return max_halves(__builtin_fmaxf(mx2[0], mx2[1]));
  };
  auto softmax_finish = [&](const Cls& cls, f32x16 (&s)[NKB], u32x4 (&pk)[PKS]) __attribute__((always_inline)) {
    float ps = ps_sm[0] + ps_sm[1];
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(!(ps <= kSumBound))) {  // (a NaN or infinite sum included)
      // (the weights were masked after the exp: mask the scores themselves for the row max)
      if constexpr (PAIR_MASK) mask_scores(cls, s);
      // The max moves straight to the tile's max.
      const float mx = row_max(s);
      const float m_new = __builtin_fmaxf(m_run, mx * c);
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      ps_sm[0] = ps_sm[1] = 0.f;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) exp_block(s, pk, kb32, std::false_type{}, 0u);
      ps = ps_sm[0] + ps_sm[1];
      // O (all tiles before this one) onto the new max before this tile's V^T P^T is added;
      // every lane multiplies (no per-lane branch).
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    l_run = l_run * alpha + ps;
  };

  // Scheduling pattern of the interleaved stream, per part: each matrix instruction with the
  // operand read of a later one, a share of the tile's global loads and V^T writes (part a),
  // and VP vector instructions of the softmax (transcendentals included).
  constexpr int NVMEM = VDMA_PER_WAVE + DMA_PER_WAVE;
  constexpr int VALU_A = 52 + (PAIR_MASK ? 24 : 0);  // one block: mask, P, sums
  constexpr int VALU_B = VALU_A;
  constexpr int VPA = (VALU_A + NPV - 1) / NPV, VPB = (VALU_B + NQK - 1) / NQK;
  auto stream_pattern = [&](int i0, int i1, auto vp, bool with_loads, bool first)
                            __attribute__((always_inline)) {
    // (a V^T operand of the unpacked path is two reads)
    if (first) __builtin_amdgcn_sched_group_barrier(0x100, VPACK ? AH : 2 * AH, 0);  // first operands
#pragma unroll
    for (int i = 0; i < NMM; ++i) {
      if (i < i0 || i >= i1) continue;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
      if (i + AH < NMM) {  // a later operand
        if (!VPACK && i + AH < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (with_loads && i - i0 < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, decltype(vp)::value, 0);  // softmax (VALU, transcendental)
    }
  };

  // A tile that is not computed (skipped by the ballot, past the last tile, or a wave with no
  // valid rows) gets all-zero keep words: its softmax is then an exact no-op.
  auto retire = [&](Cls& cl, bool live) __attribute__((always_inline)) {
    if (!live) {
      cl.full = false;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) cl.wsh[kb32] = 0u;
    }
  };

  // One pipelined iteration (see above).  s_cur holds S_j, s_nxt receives S_{j+1}; pk_prev holds
  // P_{j-1} (live_prev: it has a kept key) and receives P_j; k_nxt holds K_{j+1}, k_fill
  // receives K_{j+2}; v_prev holds V_{j-1}^T, v_fill receives V_j^T; m_nxt holds the mask words
  // of tile j+1, m_fill receives those of tile j+2.
  auto iter = [&](auto skip, int j, Cls& cls_cur, bool& live_cur, bool& live_prev,
                  f32x16 (&s_cur)[NKB], f32x16 (&s_nxt)[NKB], u32x4 (&pk_prev)[PKS],
                  const unsigned char* k_nxt, unsigned char* k_fill, const unsigned char* v_prev,
                  unsigned char* v_fill, const u32* m_nxt, u32* m_fill)
                  __attribute__((always_inline)) {
    // skip: 0 = branch-free, 1 = skipping (a wave with both neighbouring tiles dead does no
    // matrix work), 2 = the first iteration of the branch-free loop (no P_{-1}: part a has no
    // matrix work).  (The branch-free loop never walks a tile summary: its tile j is kt0 + j.)
    constexpr int KIND = decltype(skip)::value;
    auto tx = [&](int jj) __attribute__((always_inline)) {
      return KIND == 1 ? tix(jj) : kt0 + min(jj, n_tiles - 1);
    };
    const int j0 = tx(j), j1 = tx(j + 1), j2 = tx(j + 2);
    auto issue_loads = [&]() __attribute__((always_inline)) {
      dma_tile(j2, k_fill);
      v_dma(j0, v_fill);      // V_j (packed V^T, or rows) straight into LDS
    };
    Cls cls_nxt = classify(j1, m_nxt);
    const bool live_nxt = wave_live && j + 1 < n_tiles && !cls_nxt.skip;
    retire(cls_nxt, live_nxt);
    // (bitmask tiles are never full: their masking is part of the interleaved stream below)
    if (MODE != kBitmask && !cls_cur.full) mask_scores(cls_cur, s_cur);
    u32x4 pk[PKS];
    u32x4 op[AH + 1];
    if constexpr (KIND == 2) {
      issue_loads();
      mm_prefetch(NPV, NMM, op, k_nxt, v_prev);
      softmax_block(cls_cur, s_cur, pk, 0);
      __builtin_amdgcn_sched_barrier(0);
      mm_run(NPV, NMM, NMM, op, k_nxt, s_nxt, v_prev, pk_prev);
      softmax_block(cls_cur, s_cur, pk, 1);
      stream_pattern(NPV, NMM, std::integral_constant<int, VPB>{}, true, true);
    } else if (KIND == 0 || live_nxt || live_prev) {
      issue_loads();  // (in the stream's scheduling region, spread over its first instructions)
      // One interleaved stream in two parts.  Both products run: when one of the two tiles is
      // skipped, its P is exactly 0 (so O += V^T P^T adds zeros; V^T in LDS is always finite
      // data) or its S is never used (its keep words are all zero), and the code keeps one path.
      // part a: O += V_{j-1}^T P_{j-1}^T beside P of keys 0..31 of tile j
      mm_prefetch(0, NMM, op, k_nxt, v_prev);
      mm_run(0, NPV, NMM, op, k_nxt, s_nxt, v_prev, pk_prev);
      softmax_block(cls_cur, s_cur, pk, 0);
      stream_pattern(0, NPV, std::integral_constant<int, VPA>{}, true, true);
      __builtin_amdgcn_sched_barrier(0);
      // part b: S_{j+1} = K_{j+1} Q^T beside P of keys 32..63
      mm_run(NPV, NMM, NMM, op, k_nxt, s_nxt, v_prev, pk_prev);
      softmax_block(cls_cur, s_cur, pk, 1);
      stream_pattern(NPV, NMM, std::integral_constant<int, VPB>{}, false, false);
    } else {
      // Both neighbouring tiles are skipped by the wave's ballot (no kept key: causal-dead, an
      // empty mask block, past the end, or a wave with no valid rows): no matrix work.  (S_{j+1}
      // is not used; define it anyway, so the old contents of its registers are dead here.)
      issue_loads();
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) s_nxt[kb32][r] = 0.f;
      softmax_block(cls_cur, s_cur, pk, 0);
      softmax_block(cls_cur, s_cur, pk, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    softmax_finish(cls_cur, s_cur, pk);
#pragma unroll
    for (int t = 0; t < PKS; ++t) pk_prev[t] = pk[t];
    // This wave's K and V DMA and the mask words of tile j+2 (loaded at the end of the previous
    // iteration) have landed; the words of tile j+3 go out only now, so they are the one load
    // in flight past the barrier.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    mask_store(m_fill);
    if constexpr (MODE == kBitmask) {
      __builtin_amdgcn_sched_barrier(0);
      mask_load(tx(j + 3));
    }
    // This wave's LDS writes (mask words, V^T) are complete; then meet the other waves.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    pipeline_barrier();
    cls_cur = cls_nxt;
    live_prev = live_cur;
    live_cur = live_nxt;
  };

  Cls cls_cur;
  bool live_cur, live_prev = false;
  f32x16 sA[NKB], sB[NKB];
  u32x4 pk_prev[PKS];
#pragma unroll
  for (int t = 0; t < PKS; ++t) pk_prev[t] = (u32x4){0u, 0u, 0u, 0u};
  // Prologue: Q in registers; masks 0 and 1, K_0 and K_1 staged; S_0 computed.  The Q loads of
  // every staging pass go out first, then the K_0 / K_1 DMA and the first mask loads, so all
  // their latencies overlap the Q staging; the staging barriers wait only for the Q loads and
  // LDS accesses (not for those DMAs).
  u32 mw0 = 0u, mw1 = 0u;  // mask words of tiles 0 and 1 (bitmask mode)
  bool mv0 = false, mv1 = false;
  {
    u32x4 qx[QPASS][QL];   // every pass's Q chunks loaded at once (one memory latency)
#pragma unroll
    for (int pass = 0; pass < QPASS; ++pass) q_load(pass, qx[pass]);
    dma_tile(tix(0), k_lds0);
    dma_tile(tix(1), k_lds1);
    // The mask words of tiles 0, 1 and 2 go out together (one memory latency for the three).
    mask_load(tix(0));
    mw0 = mreg;
    mv0 = mvalid;
    mask_load(tix(1));
    mw1 = mreg;
    mv1 = mvalid;
    mask_load(tix(2));  // (stored at the end of iteration 0)
#pragma unroll
    for (int pass = 0; pass < QPASS; ++pass) {
      // (Buffer choices are static, so the compiler can tell these LDS accesses from the DMA
      // into the K buffers and does not wait for it.)  Chunk i of a thread is in the first
      // 64 rows iff i < BN * KC / NT.
      constexpr int QHALF = BN * KC / NT;
      static_assert(QHALF * NT == BN * KC && 2 * QHALF == QL, "Q chunk split");
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const int id = tid + NT * i, r = id / KC, c = id % KC;
        if (i < QHALF) *(u32x4*)(v_lds0 + L::off(r, c)) = qx[pass][i];
        else *(u32x4*)(v_lds1 + L::off(r - BN, c)) = qx[pass][i];
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      pipeline_barrier();
      if (wave / 4 == pass) {  // waves 4 pass .. 4 pass + 3 own these 128 rows
        if ((wave & 3) < 2) {
#pragma unroll
          for (int ks = 0; ks < QKS; ++ks) qreg[ks] = *(const u32x4*)(v_lds0 + op_addr(ks, wave & 1)) ^ p.qflip;
        } else {
#pragma unroll
          for (int ks = 0; ks < QKS; ++ks) qreg[ks] = *(const u32x4*)(v_lds1 + op_addr(ks, wave & 1)) ^ p.qflip;
        }
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      pipeline_barrier();
    }
  }
  // Iteration 0 multiplies the V^T buffer v_lds1 (still holding the Q staging, and unwritten
  // padding) by P_{-1} = 0: fill it with zeros so the product is exactly 0.
#pragma unroll
  for (int i = 0; i < (VBUF_BYTES / 16 + NT - 1) / NT; ++i) {
    const int c = tid + NT * i;
    if (c < VBUF_BYTES / 16) *(u32x4*)(v_lds1 + 16 * c) = (u32x4){0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // K_0, K_1 DMA and the mask words
  if (MODE == kBitmask) {
    m_lds0[m_row * NKB + m_word] = mv0 ? mw0 : 0u;
    m_lds1[m_row * NKB + m_word] = mv1 ? mw1 : 0u;
  }
  __syncthreads();
  cls_cur = classify(tix(0), m_lds0);
  live_cur = wave_live && !cls_cur.skip;
  retire(cls_cur, live_cur);
  if (live_cur) {
    u32x4 op[AH + 1];
    mm_prefetch(NPV, NMM, op, k_lds0, v_lds1);
    mm_run(NPV, NMM, NMM, op, k_lds0, sA, v_lds1, pk_prev);
    // The running max starts at the first tile's row max (its masked scores), so that tile
    // passes the sum check instead of being computed twice: the same m the check's redo would
    // set (from the -1e30 floor, alpha = 0 with O still 0), so results are unchanged.  (A row
    // whose first tile keeps no key keeps the floor.)
    if (!cls_cur.full) mask_scores(cls_cur, sA);
    m_run = __builtin_fmaxf(m_run, row_max(sA) * c);
  }
  __syncthreads();  // every wave has read K_0 before iteration 0 refills its buffer
  // Two loops over the walk: iterations in which every wave keeps a key in tiles j-1, j and j+1
  // run without any branch around the matrix work (its cheapest form); the rest skip the matrix
  // work of a wave whose two neighbouring tiles are both dead by its ballot.  Causal: the tiles
  // up to the last one wave 0 (the workgroup's first rows) keeps, then the diagonal tail; with a
  // tile summary (a structured mask): all skipping; otherwise (random masks have no empty tile)
  // none.
  int n_fast = n_tiles;
  if (MODE == kCausal) n_fast = min(n_tiles, min((row0 + 31) / G, S - 1) / BN);
  if (sparse) n_fast = 0;
  n_fast &= ~1;
  const std::integral_constant<int, 0> fast{};
  const std::integral_constant<int, 1> skipping{};
  const std::integral_constant<int, 2> first{};
#ifndef FA_PEEL
#define FA_PEEL 1
#endif
  // With a bit mask the extra copy of the iteration's code measured slower than the product it
  // saves, so only the other modes peel iteration 0.
  constexpr bool kPeel = FA_PEEL && MODE != kBitmask;
  if (kPeel && n_fast >= 2) {
    // Iteration 0 without the product of P_{-1} = 0, then pairs from iteration 1, then the last
    // branch-free iteration (n_fast is even).
    iter(first, 0, cls_cur, live_cur, live_prev, sA, sB, pk_prev, k_lds1, k_lds0, v_lds1, v_lds0,
         m_lds1, m_lds0);
    for (int j = 1; j + 1 < n_fast; j += 2) {
      iter(fast, j, cls_cur, live_cur, live_prev, sB, sA, pk_prev, k_lds0, k_lds1, v_lds0, v_lds1,
           m_lds0, m_lds1);
      iter(fast, j + 1, cls_cur, live_cur, live_prev, sA, sB, pk_prev, k_lds1, k_lds0, v_lds1,
           v_lds0, m_lds1, m_lds0);
    }
    iter(fast, n_fast - 1, cls_cur, live_cur, live_prev, sB, sA, pk_prev, k_lds0, k_lds1, v_lds0,
         v_lds1, m_lds0, m_lds1);
  } else {
    for (int j = 0; j < n_fast; j += 2) {
      iter(fast, j, cls_cur, live_cur, live_prev, sA, sB, pk_prev, k_lds1, k_lds0, v_lds1, v_lds0,
           m_lds1, m_lds0);
      iter(fast, j + 1, cls_cur, live_cur, live_prev, sB, sA, pk_prev, k_lds0, k_lds1, v_lds0,
           v_lds1, m_lds0, m_lds1);
    }
  }
  for (int j = n_fast; j < n_tiles; j += 2) {
    iter(skipping, j, cls_cur, live_cur, live_prev, sA, sB, pk_prev, k_lds1, k_lds0, v_lds1,
         v_lds0, m_lds1, m_lds0);
    if (j + 1 < n_tiles)
      iter(skipping, j + 1, cls_cur, live_cur, live_prev, sB, sA, pk_prev, k_lds0, k_lds1,
           v_lds0, v_lds1, m_lds0, m_lds1);
  }
  // The last tile's O += V^T P^T (V_{n-1}^T is in the buffer the last iteration filled).
  if (live_prev) {
    u32x4 op[AH + 1];
    const unsigned char* vb = ((n_tiles - 1) & 1) ? v_lds1 : v_lds0;
    mm_prefetch(0, NPV, op, k_lds0, vb);
    mm_run(0, NPV, NPV, op, k_lds0, sA, vb, pk_prev);
  }

  // ---- Epilogue: O / l (0 for a row with no kept key), rounded, stored row-major through LDS.
  const float lt = sum_halves(l_run);
  if (p.n_split > 1) {  // split-KV: this key range's unnormalised O, running max and row sum
    if (wave_live && my_pos < S) {
      float* op = p.o_part + ((size_t)split * p.part_rows + orow_idx) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[db][4 * t4 + e];
          *(f32x4*)(op + 32 * db + 8 * t4 + 4 * hl) = x;
        }
      if (hl == 0)
        *(float2*)(p.ml_part + ((size_t)split * p.part_rows + orow_idx) * 2) = make_float2(m_run, lt);
    }
    return;
  }
  const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
  // O rows through LDS.  A lane holds 8-byte pieces of its own row, so storing from registers
  // writes 16 bytes of each of 32 rows per instruction; instead each wave writes its rows, one
  // half of the columns at a time (OW bytes a row, rows OW + 8 bytes apart), into a region of
  // its own in the K buffers (no wave reads them once the key loop has ended), reads them
  // back row-major, 16 bytes a lane, and stores whole row halves: 128-byte lines at d=128.
  // (A wave's LDS accesses complete in order, so no barrier is needed around its region.)
  constexpr int OW = D;               // bytes of one half of a row
  constexpr int ORS = OW + 8;         // row stride of a region
  constexpr int OLR = OW / 16;        // lanes per row half
  constexpr int ORI = 64 / OLR;       // rows per store instruction
  static_assert((NW / 2) * 32 * ORS <= T_BYTES, "O staging regions fit the K buffers");
  if (wave_live) {
    unsigned char* ost = (wave < NW / 2 ? k_lds0 : k_lds1) + (wave % (NW / 2)) * (32 * ORS);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int dbl = 0; dbl < NDB / 2; ++dbl)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[h * (NDB / 2) + dbl][4 * t4 + e] * inv;
          *(u32x2*)(ost + l32 * ORS + (32 * dbl + 8 * t4 + 4 * hl) * 2) = pack4<BF16>(x);
        }
#pragma unroll
      for (int i = 0; i < 32 / ORI; ++i) {
        const int r = lane / OLR + ORI * i, c = lane % OLR;
        const u32x4 x = *(const u32x4*)(ost + r * ORS + 16 * c);
        const int grow = row0 + wave * 32 + r, pos = grow / G, head = hk * G + (grow - pos * G);
        // (non-temporal: O is not read again here, so it need not displace K/V tiles in L2)
        if (pos < S)
          __builtin_nontemporal_store(x, (u32x4*)(p.o + q_batch + ((size_t)pos * Hq + head) * D + h * (D / 2) + 8 * c));
      }
    }
  }
  if (wave_live && my_pos < S) {
    // Log-sum-exp of the row's kept scores (natural log), from the running softmax state: the
    // max m_run is of s*c with c = |scale| log2(e) (Q carries the sign of the scale), and lt
    // is the sum of 2^(s*c - m_run), so ln(sum exp(scale s)) = (m_run + log2 lt) ln 2.  A row
    // with no kept key gets -inf.
    if (p.lse && hl == 0)
      p.lse[((size_t)b * Hq + my_head) * S + my_pos] =
          lt > 0.f ? (m_run + __builtin_amdgcn_logf(lt)) * 0.693147180559945f : -INFINITY;
  }
}

// Split-KV merge: for each row, the key ranges' states (m_s, l_s, O_s), with O_s summed from
// weights 2^(s c - m_s), combine exactly as the online softmax combines tiles:
// m = max m_s, l = sum 2^(m_s - m) l_s, O = sum 2^(m_s - m) O_s / l (0 when l = 0), and
// lse = (m + log2 l) ln 2.  One thread per 4 consecutive elements of a row.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ ml_part,
                                                    uint16_t* __restrict__ o, float* __restrict__ lse,
                                                    int n_split, size_t rows, int S, int Hq) {
  constexpr int TPR = D / 4;  // threads per row
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / TPR;
  const int c = (int)(gid - row * TPR);
  if (row >= rows) return;
  float m = -1e30f;
  for (int s = 0; s < n_split; ++s) m = fmaxf(m, ml_part[((size_t)s * rows + row) * 2]);
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_split; ++s) {
    const float2 ml = *(const float2*)(ml_part + ((size_t)s * rows + row) * 2);
    const float w = __builtin_amdgcn_exp2f(ml.x - m);
    l += w * ml.y;
    const f32x4 x = *(const f32x4*)(o_part + ((size_t)s * rows + row) * D + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += w * x[e];
  }
  const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = acc[e] * inv;
  *(u32x2*)(o + row * D + 4 * c) = pack4<BF16>(y);
  if (lse && c == 0) {
    const size_t sh = (size_t)S * Hq;
    const size_t bb = row / sh, rem = row - bb * sh;
    const size_t pos = rem / Hq, h = rem - pos * Hq;
    lse[(bb * Hq + h) * S + pos] =
        l > 0.f ? (m + __builtin_amdgcn_logf(l)) * 0.693147180559945f : -INFINITY;
  }
}

template <bool BF16, int D>
hipError_t launch_merge(const Params& p, float* lse, hipStream_t s) {
  const float* op = p.o_part;
  const float* ml = p.ml_part;
  uint16_t* o = p.o;
  int n_split = p.n_split, S = p.S, Hq = p.Hq;
  size_t rows = p.part_rows;
  void* args[] = {(void*)&op, (void*)&ml, (void*)&o, (void*)&lse, (void*)&n_split, (void*)&rows,
                  (void*)&S, (void*)&Hq};
  const size_t blocks = (rows * (D / 4) + 255) / 256;
  return hipLaunchKernel((const void*)merge_kernel<BF16, D>, dim3((unsigned)blocks), dim3(256),
                         args, 0, s);
}

// Instances: 4 or 8 waves, each with packed V^T or with V's rows.
template <bool BF16, int D, int MODE>
hipError_t launch(const Params& p, bool vpack, int nw, hipStream_t s) {
  void* args[] = {(void*)&p};
  if (vpack && !p.vt) return hipErrorInvalidValue;  // (the packed kernels read p.vt)
  const void* k = nw == kWide ? (vpack ? (const void*)fa_fwd_kernel<BF16, D, MODE, true, kWide>
                                       : (const void*)fa_fwd_kernel<BF16, D, MODE, false, kWide>)
                              : (vpack ? (const void*)fa_fwd_kernel<BF16, D, MODE, true, 4>
                                       : (const void*)fa_fwd_kernel<BF16, D, MODE, false, 4>);
  return hipLaunchKernel(k, dim3(p.n_wg), dim3(nw * 64), args, 0, s);
}

template <bool BF16, int D>
hipError_t launch_mode(int mode, const Params& p, bool vpack, int nw, hipStream_t s) {
  switch (mode) {
    case kNone: return launch<BF16, D, kNone>(p, vpack, nw, s);
    case kCausal: return launch<BF16, D, kCausal>(p, vpack, nw, s);
    default: return launch<BF16, D, kBitmask>(p, vpack, nw, s);
  }
}

template <int D>
hipError_t launch_pack(const Params& p, int batch, hipStream_t s) {
  const uint16_t* v = p.v;
  uint16_t* vt = const_cast<uint16_t*>(p.vt);
  int S = p.S, Hkv = p.Hkv, n_kt = p.n_kt;
  void* args[] = {(void*)&v, (void*)&vt, (void*)&S, (void*)&Hkv, (void*)&n_kt};
  return hipLaunchKernel((const void*)vt_pack_kernel<D>, dim3(batch * Hkv * n_kt), dim3(256), args,
                         0, s);
}

// The packed V^T workspace comes from one memory pool per device, created on first use and
// kept for the life of the process (memory freed back to it is retained for the next call).
constexpr int kMaxDevices = 64;
std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxDevices];

hipError_t workspace_pool(hipMemPool_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mutex);
  if (!g_pools[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pools[dev] = pool;
  }
  *out = g_pools[dev];
  return hipSuccess;
}

// Device scratch of fa_fwd_noalloc: a file-scope array in every device's copy of this code
// object (held until the process ends), so that entry point allocates nothing.  Host code never
// passes `scratch` itself to a kernel (on the host it names a stand-in, not device memory): it
// resolves each device's address once, with that device current, and uses that pointer.
constexpr size_t kStaticScratchBytes = (size_t)FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(fa_status s) {
  switch ((int)s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_PTR: return "null q, k, v, o or lse pointer";
    case FA_ERR_BAD_SHAPE: return "bad shape (non-positive size, heads not divisible, or too large)";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype or head_dim, or misaligned pointer";
    case FA_ERR_BAD_MASK_MODE: return "unknown mask mode, or bitmask mode without a mask";
    case FA_ERR_BAD_SCALE: return "scale is not finite";
    case FA_ERR_HIP: return "HIP runtime rejected a kernel launch or the workspace allocation";
    case FA_ERR_WORKSPACE: return "caller workspace smaller than the plan's workspace_bytes or not 256-byte aligned";
    case FA_ERR_SCRATCH_LIMIT: return "the call needs more device scratch than fa_fwd_noalloc's static array holds";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// The launch plan of a call: workgroup shape, V packing, split-KV shares and workspace, from the
// sizes alone (shared by fa_fwd_plan and the launches, so the two always agree).
struct Plan {
  int nw;             // waves per workgroup (4: 128 rows, 8: 256 rows)
  bool vpack;         // V^T packed by a pre-pass
  int n_split;        // split-KV shares per row tile
  int n_kt, n_rb, G;  // 64-key tiles, 64-row blocks, query heads per KV head
  int64_t n_rt, n_wg; // row tiles per (batch, KV head); workgroups before splitting
  size_t vt_bytes, part_bytes;  // packed V^T workspace, split-KV partials
  size_t part_off, ws_bytes;    // workspace layout: V^T at 0, partials at part_off (256-aligned)
};

fa_status make_plan(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                    int n_kv_heads, int seq_len, int head_dim, bool with_tiles, int kv_splits,
                    Plan* pl) {
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (mask_mode != FA_MASK_NONE && mask_mode != FA_MASK_CAUSAL && mask_mode != FA_MASK_BITMASK)
    return FA_ERR_BAD_MASK_MODE;
  if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || seq_len <= 0 ||
      n_q_heads % n_kv_heads != 0)
    return FA_ERR_BAD_SHAPE;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  // Offsets inside one batch are 32-bit; the grid is a 32-bit count.
  if ((int64_t)seq_len * n_q_heads * head_dim >= ((int64_t)1 << 31)) return FA_ERR_BAD_SHAPE;
  const int G = n_q_heads / n_kv_heads;
  const int64_t rows = (int64_t)seq_len * G;
  // Packed V^T offsets must stay 31-bit.
  const int n_kt = (seq_len + kBN - 1) / kBN;
  const int64_t tile_bytes = head_dim == 128 ? VtPack<128>::TILE : VtPack<64>::TILE;
  const bool pack_ok = (int64_t)n_kt * tile_bytes < ((int64_t)1 << 31);
  const int64_t wide_rows = mask_mode != FA_MASK_CAUSAL ? (head_dim == 128 ? kWideRows128 : kWideRows)
                            : head_dim == 128 ? kWideRowsCausal128 : kWideRowsCausal;
  const int nw = rows >= wide_rows ? kWide : 4;
  const int64_t n_rt = (rows + nw * 32 - 1) / (nw * 32);
  const int64_t n_wg = n_rt * n_kv_heads * batch;
  if (n_wg >= ((int64_t)1 << 31)) return FA_ERR_BAD_SHAPE;
  const int n_rb = (seq_len + 63) / 64;
  if (with_tiles) {
    if (mask_mode != FA_MASK_BITMASK) return FA_ERR_BAD_MASK_MODE;
    if (n_rb > kMaxListTiles) return FA_ERR_UNSUPPORTED;
  }
  if (kv_splits < 0 || kv_splits > kMaxSplits || (with_tiles && kv_splits > 1))
    return FA_ERR_UNSUPPORTED;
  // Split-KV: explicit, or (kv_splits == 0, no tile summary) when the grid fills at most half
  // of the chip's workgroup slots (one 256-row or two 128-row workgroups per CU): enough key
  // ranges per row tile to fill it, each at least 8 tiles long.
  int n_split = kv_splits > 1 ? min(kv_splits, n_kt) : 1;
  if (kv_splits == 0 && !with_tiles) {
    const int64_t slots = nw == kWide ? kNumCUs : 2 * kNumCUs;
    if (2 * n_wg <= slots)
      n_split = (int)std::min<int64_t>({(int64_t)kMaxSplits, (slots + n_wg - 1) / n_wg,
                                        std::max<int64_t>(1, n_kt / 8)});
  }
  if (n_wg * n_split >= ((int64_t)1 << 31)) return FA_ERR_BAD_SHAPE;
  // Packed V^T (one pre-pass over V) when kPackRowTiles or more row-tile workgroups would
  // otherwise each transpose a KV head's V in their operand reads.
  pl->nw = nw;
  pl->vpack = pack_ok && n_rt >= (mask_mode == FA_MASK_CAUSAL && head_dim == 128 ? kPackRowTilesCausal128
                                                                                : kPackRowTiles);
  pl->n_split = n_split;
  pl->n_kt = n_kt;
  pl->n_rb = n_rb;
  pl->G = G;
  pl->n_rt = n_rt;
  pl->n_wg = n_wg;
  pl->vt_bytes = pl->vpack ? (size_t)batch * n_kv_heads * n_kt * tile_bytes : 0;
  pl->part_bytes = n_split > 1 ? (size_t)n_split * batch * seq_len * n_q_heads * (head_dim + 2) * 4 : 0;
  pl->part_off = (pl->vt_bytes + 255) & ~(size_t)255;
  pl->ws_bytes = pl->part_bytes ? pl->part_off + pl->part_bytes : pl->vt_bytes;
  return FA_OK;
}

// Measurement hook (fa_set_kernel_events): HIP events to record around the attention kernel of
// this thread's next call.
thread_local hipEvent_t t_kernel_events[2] = {nullptr, nullptr};

// fa_fwd, fa_fwd_lse and fa_fwd_ex: validation first (no HIP call), then the launches.
fa_status run_fwd(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                  int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                  const void* k, const void* v, const uint32_t* mask, const uint32_t* tiles,
                  int kv_splits, void* o, float* lse, void* user_ws, uint64_t user_ws_bytes,
                  bool use_static_scratch, void* stream) {
  // (the hook's events serve this call only, whatever its outcome)
  const hipEvent_t ev_start = t_kernel_events[0], ev_stop = t_kernel_events[1];
  t_kernel_events[0] = t_kernel_events[1] = nullptr;
  if (!q || !k || !v || !o) {
    // (an unknown dtype or mode is reported first, as the plan would)
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (mask_mode != FA_MASK_NONE && mask_mode != FA_MASK_CAUSAL && mask_mode != FA_MASK_BITMASK)
      return FA_ERR_BAD_MASK_MODE;
    return FA_ERR_NULL_PTR;
  }
  Plan pl;
  const fa_status ps = make_plan(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len,
                                 head_dim, tiles != nullptr, kv_splits, &pl);
  if (ps != FA_OK) return ps;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_UNSUPPORTED;
  if (mask_mode == FA_MASK_BITMASK && (!mask || ((uintptr_t)mask & 3u))) return FA_ERR_BAD_MASK_MODE;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (lse && ((uintptr_t)lse & 3u)) return FA_ERR_UNSUPPORTED;
  if (tiles && ((uintptr_t)tiles & 3u)) return FA_ERR_UNSUPPORTED;
  // A caller's workspace must hold the plan's layout (packed V^T at 0, partials at part_off).
  if (user_ws && pl.ws_bytes && (((uintptr_t)user_ws & 255u) || user_ws_bytes < pl.ws_bytes))
    return FA_ERR_WORKSPACE;
  if (use_static_scratch) {  // (every argument is valid by now: the first HIP call follows)
    if (pl.ws_bytes > kStaticScratchBytes) return FA_ERR_SCRATCH_LIMIT;
    if (static_scratch(&user_ws) != hipSuccess) return FA_ERR_HIP;
    user_ws_bytes = kStaticScratchBytes;
  }
  const int nw = pl.nw, n_split = pl.n_split, n_kt = pl.n_kt, n_rb = pl.n_rb, G = pl.G;
  const int64_t n_rt = pl.n_rt, n_wg = pl.n_wg;

  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.mask = mask_mode == FA_MASK_BITMASK ? mask : nullptr;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.tiles = tiles;
  p.n_rb = n_rb;
  p.TW = (n_rb + 31) / 32;
  p.S = seq_len;
  p.Hq = n_q_heads;
  p.Hkv = n_kv_heads;
  p.G = G;
  p.W = (seq_len + 31) / 32;
  p.n_rt = (int)n_rt;
  p.n_wg = (int)(n_wg * n_split);  // the grid (key ranges of one row tile are adjacent)
  p.n_split = n_split;
  p.part_rows = (size_t)batch * seq_len * n_q_heads;
  p.o_part = nullptr;
  p.ml_part = nullptr;
  p.n_kt = n_kt;
  p.vt = nullptr;
  // Causal balance across the 8 XCDs: when the grid is a multiple of 8 and one head's row tiles
  // fill exactly k > 1 XCDs' shares, the kernel deals each head's tiles over its k XCDs.
  p.xsplit = 0;
  if (n_split == 1 && n_wg % 8 == 0 && n_rt % (n_wg / 8) == 0 && n_rt > n_wg / 8)
    p.xsplit = (int)(n_rt / (n_wg / 8));
  // exp(x) = 2^(x log2 e): fold log2(e) into the scale.  A zero scale becomes a tiny positive
  // one (2^-100): every 2^(s*c - m) is then 1 to fp32 precision, the uniform average the zero
  // scale defines, without 0 * inf on masked scores.
  const float c = fabsf(scale) * 1.4426950408889634f;
  p.c = c > 0x1p-100f ? c : 0x1p-100f;
  p.qflip = scale < 0.f ? 0x80008000u : 0u;

  hipStream_t s = (hipStream_t)stream;
  const bool vpack = pl.vpack;
  hipError_t e = hipSuccess;
  void* ws = nullptr;  // the pool's workspace, when the caller passes none (freed below)
  if (pl.ws_bytes && !user_ws) {
    hipMemPool_t pool = nullptr;
    e = workspace_pool(&pool);
    if (e != hipSuccess) return FA_ERR_HIP;
    e = hipMallocFromPoolAsync(&ws, pl.ws_bytes, pool, s);
    if (e != hipSuccess) return FA_ERR_HIP;
  }
  unsigned char* base = (unsigned char*)(user_ws ? user_ws : ws);
  if (n_split > 1) {
    p.o_part = (float*)(base + pl.part_off);
    p.ml_part = p.o_part + (size_t)n_split * p.part_rows * head_dim;
    p.lse = nullptr;  // (written by the merge)
  }
  if (vpack) {
    p.vt = (const uint16_t*)base;
    e = head_dim == 128 ? launch_pack<128>(p, batch, s) : launch_pack<64>(p, batch, s);
  }
  const bool bf16 = dtype == FA_DTYPE_BF16;
  if (e == hipSuccess && ev_start) e = hipEventRecord(ev_start, s);
  if (e == hipSuccess) {
    if (bf16)
      e = head_dim == 128 ? launch_mode<true, 128>(mask_mode, p, vpack, nw, s)
                          : launch_mode<true, 64>(mask_mode, p, vpack, nw, s);
    else
      e = head_dim == 128 ? launch_mode<false, 128>(mask_mode, p, vpack, nw, s)
                          : launch_mode<false, 64>(mask_mode, p, vpack, nw, s);
  }
  if (e == hipSuccess && ev_stop) e = hipEventRecord(ev_stop, s);
  if (e == hipSuccess && n_split > 1) {
    if (bf16)
      e = head_dim == 128 ? launch_merge<true, 128>(p, lse, s) : launch_merge<true, 64>(p, lse, s);
    else
      e = head_dim == 128 ? launch_merge<false, 128>(p, lse, s) : launch_merge<false, 64>(p, lse, s);
  }
  if (ws) {
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = ef;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_set_kernel_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return FA_ERR_NULL_PTR;
  t_kernel_events[0] = (hipEvent_t)start;
  t_kernel_events[1] = (hipEvent_t)stop;
  return FA_OK;
}

fa_status fa_fwd(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                 int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                 const void* k, const void* v, const uint32_t* mask, void* o, void* stream) {
  return run_fwd(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim, scale, q, k,
                 v, mask, nullptr, 1, o, nullptr, nullptr, 0, false, stream);
}

fa_status fa_fwd_lse(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                     int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                     const void* k, const void* v, const uint32_t* mask, void* o, float* lse,
                     void* stream) {
  if (!lse) return FA_ERR_NULL_PTR;
  return run_fwd(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim, scale, q, k,
                 v, mask, nullptr, 1, o, lse, nullptr, 0, false, stream);
}

fa_status fa_fwd_plan(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                      int n_kv_heads, int seq_len, int head_dim, int with_tiles, int kv_splits,
                      fa_plan* plan) {
  if (!plan) return FA_ERR_NULL_PTR;
  Plan pl;
  const fa_status st = make_plan(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len,
                                 head_dim, with_tiles != 0, kv_splits, &pl);
  if (st != FA_OK) return st;
  plan->rows_per_workgroup = pl.nw * 32;
  plan->packed_v = pl.vpack ? 1 : 0;
  plan->kv_splits = pl.n_split;
  plan->workgroups = pl.n_wg * pl.n_split;
  plan->workspace_bytes = (uint64_t)pl.ws_bytes;
  plan->kernels = 1 + (pl.vpack ? 1 : 0) + (pl.n_split > 1 ? 1 : 0);
  return FA_OK;
}

fa_status fa_fwd_ex(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                    int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                    const void* k, const void* v, const uint32_t* mask, const uint32_t* tiles,
                    int kv_splits, void* o, float* lse, void* workspace,
                    uint64_t workspace_bytes, void* stream) {
  return run_fwd(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim, scale, q, k,
                 v, mask, tiles, kv_splits, o, lse, workspace, workspace_bytes, false, stream);
}

fa_status fa_fwd_noalloc(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                         int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                         const void* k, const void* v, const uint32_t* mask, const uint32_t* tiles,
                         int kv_splits, void* o, float* lse, void* stream) {
  return run_fwd(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim, scale, q, k,
                 v, mask, tiles, kv_splits, o, lse, nullptr, 0, true, stream);
}

}  // extern "C"
