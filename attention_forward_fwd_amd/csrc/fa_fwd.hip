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
//   * LDS: K tile [BN][D] and the Q staging tile with 16-byte chunks XOR-swizzled by row; V is
//     written transposed ([D][BN]) with the key order permuted to match the P register layout,
//     so every MFMA operand is one 128-bit ds_read.  K/V/mask tiles are double-buffered with
//     one workgroup barrier per tile.
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

// Tile shape shared by every instance.
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

template <bool BF16, int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(Params p) {
  constexpr int BM = kBM, BN = kBN, NT = kThreads;
  constexpr int KC = D / 8;      // 16-byte chunks in a K/Q row
  constexpr int VC = BN / 8;     // 16-byte chunks in a transposed-V row
  constexpr int NKB = BN / 32;   // 32-key blocks per tile (one MFMA output block each)
  constexpr int QKS = D / 16;    // MFMA k-steps of Q K^T
  constexpr int NDB = D / 32;    // 32-wide blocks of head_dim in O
  constexpr int PKS = BN / 16;   // MFMA k-steps of P V
  constexpr int K_BYTES = BN * D * 2;
  constexpr int V_BYTES = D * BN * 2;
  constexpr int M_BYTES = MODE == kBitmask ? BM * NKB * 4 : 0;
  constexpr int BUF = K_BYTES + V_BYTES + M_BYTES;
  constexpr int KL = BN * KC / NT;                   // K chunks loaded per thread
  constexpr int VPAIRS = (BN / 4) * KC;              // (key quad, d chunk) pairs per V tile
  constexpr int VL = (VPAIRS + NT - 1) / NT;
  constexpr int QL = BM * KC / NT;                   // Q chunks staged per thread
  static_assert(BM * D * 2 <= 2 * BUF, "Q staging must fit in the K/V buffers");
  static_assert(KL * NT == BN * KC && QL * NT == BM * KC, "load split");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;  // lane column and lane half
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
  const int w_row0 = row0 + wave * 32;
  const int w_pmin = w_row0 / G;
  const bool wave_live = w_pmin < S;

  int n_tiles;
  if (MODE == kCausal) {
    const int pmax = min((row0 + BM - 1) / G, S - 1);
    n_tiles = pmax / BN + 1;
  } else {
    n_tiles = (S + BN - 1) / BN;
  }

  // ---- Q: coalesced 128-bit loads -> swizzled LDS -> MFMA B operands held in registers.
#pragma unroll
  for (int i = 0; i < QL; ++i) {
    const int id = tid + NT * i, r = id / KC, c = id % KC;
    const int grow = row0 + r, pos = grow / G, h = hk * G + (grow - pos * G);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (pos < S) x = *(const u32x4*)(p.q + q_batch + ((size_t)pos * Hq + h) * D + c * 8);
    *(u32x4*)(smem + r * D * 2 + ((c ^ (r % KC)) * 16)) = x;
  }
  __syncthreads();
  u32x4 qreg[QKS];
#pragma unroll
  for (int ks = 0; ks < QKS; ++ks) {
    const int r = wave * 32 + l32, c = 2 * ks + hl;
    u32x4 x = *(const u32x4*)(smem + r * D * 2 + ((c ^ (r % KC)) * 16));
    qreg[ks] = x ^ p.qflip;
  }
  __syncthreads();

  // ---- K/V/mask staging: global -> registers (prefetch) -> LDS.
  u32x4 kreg[KL];
  u32x4 vreg[VL][4];
  u32 mreg[NKB];
  const u32* mrow = nullptr;  // mask row of the row this thread stages (bitmask mode)
  bool mrow_ok = false;
  if (MODE == kBitmask && tid < BM) {
    const int grow = row0 + tid, pos = grow / G, h = hk * G + (grow - pos * G);
    mrow_ok = pos < S;
    if (mrow_ok) mrow = p.mask + (((size_t)b * Hq + h) * S + pos) * (size_t)p.W;
  }

  auto gload = [&](int j) {
    const int k0 = j * BN;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int id = tid + NT * i, r = id / KC, c = id % KC, key = k0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < S) x = *(const u32x4*)(kg + key * kv_stride + c * 8);
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int id = tid + NT * i;
      if (VPAIRS % NT == 0 || id < VPAIRS) {
        const int quad = id / KC, c = id % KC;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = k0 + 4 * quad + kk;
          u32x4 x = {0u, 0u, 0u, 0u};
          if (key < S) x = *(const u32x4*)(vg + key * kv_stride + c * 8);
          vreg[i][kk] = x;
        }
      }
    }
    if (MODE == kBitmask && tid < BM) {
#pragma unroll
      for (int w = 0; w < NKB; ++w) {
        const int word = j * NKB + w;
        mreg[w] = (mrow_ok && word < p.W) ? mrow[word] : 0u;
      }
    }
  };

  auto lstore = [&](int buf) {
    unsigned char* kb = smem + buf * BUF;
    unsigned char* vb = kb + K_BYTES;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int id = tid + NT * i, r = id / KC, c = id % KC;
      *(u32x4*)(kb + r * D * 2 + ((c ^ (r % KC)) * 16)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int id = tid + NT * i;
      if (VPAIRS % NT == 0 || id < VPAIRS) {
        const int quad = id / KC, c = id % KC;
        // Key quad -> position in the transposed row.  Within every 16 keys the quads are
        // stored in the order 0, 2, 1, 3 so that the 8 keys one MFMA lane half needs for P V
        // (keys 4h..4h+3 and 8+4h..8+4h+3) are 16 contiguous bytes.
        const int qq = quad & 3;
        const int pos0 = 16 * (quad >> 2) + ((qq & 1) << 3) + ((qq & 2) << 1);
        const int cc = pos0 >> 3, off = (pos0 & 7) * 2;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32 x0 = vreg[i][0][m], x1 = vreg[i][1][m], x2 = vreg[i][2][m], x3 = vreg[i][3][m];
          const u32x2 lo = {__builtin_amdgcn_perm(x1, x0, 0x05040100u),
                            __builtin_amdgcn_perm(x3, x2, 0x05040100u)};
          const u32x2 hi = {__builtin_amdgcn_perm(x1, x0, 0x07060302u),
                            __builtin_amdgcn_perm(x3, x2, 0x07060302u)};
          const int d0 = 8 * c + 2 * m, d1 = d0 + 1;
          *(u32x2*)(vb + d0 * BN * 2 + ((cc ^ (d0 % VC)) * 16) + off) = lo;
          *(u32x2*)(vb + d1 * BN * 2 + ((cc ^ (d1 % VC)) * 16) + off) = hi;
        }
      }
    }
    if (MODE == kBitmask && tid < BM) {
      u32* mb = (u32*)(vb + V_BYTES);
#pragma unroll
      for (int w = 0; w < NKB; ++w) mb[tid * NKB + w] = mreg[w];
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -1e30f;  // finite floor: a fully masked row keeps alpha = 1 and p = 0
  float l_run = 0.f;     // this lane's partial row sum (its 16 keys of each 32-key block)
  const float c = p.c;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) gload(j + 1);

    if (wave_live) {
      const unsigned char* kb = smem + buf * BUF;
      const unsigned char* vb = kb + K_BYTES;
      const int k0 = j * BN;

      // Tile class for this wave: full (no masking), partial (per-element keep bits) or
      // empty (ballot finds no kept bit: skipped).
      bool full;
      if (MODE == kNone) full = k0 + BN <= S;
      else if (MODE == kCausal) full = k0 + BN - 1 <= w_pmin;
      else full = false;

      u32 wsh[NKB];
      bool skip = false;
      if (!full) {
        u32 any = 0;
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32) {
          const int kbase = k0 + 32 * kb32;
          u32 w = low_bits(S - kbase);
          if (MODE == kCausal) w = my_pos < S ? (w & low_bits(my_pos - kbase + 1)) : 0u;
          if (MODE == kBitmask) w &= ((const u32*)(vb + V_BYTES))[(wave * 32 + l32) * NKB + kb32];
          any |= w;
          // Lane half hl holds keys 8*(r/4) + 4*hl + r%4 of the block: pre-shift by 4*hl so
          // register r tests the constant bit 8*(r/4) + r%4.
          wsh[kb32] = w >> (4 * hl);
        }
        skip = __ballot(any != 0u) == 0ull;
      }

      if (!skip) {
        // S^T = K Q^T on the matrix cores.
        f32x16 sacc[NKB];
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb32][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < QKS; ++ks) {
#pragma unroll
          for (int kb32 = 0; kb32 < NKB; ++kb32) {
            const int r = 32 * kb32 + l32, cch = 2 * ks + hl;
            const u32x4 a = *(const u32x4*)(kb + r * D * 2 + ((cch ^ (r % KC)) * 16));
            sacc[kb32] = mfma32<BF16>(a, qreg[ks], sacc[kb32]);
          }
        }

        // Masked scores -> -inf (bit-field extract of the keep bit, bit-field insert).
        if (!full) {
#pragma unroll
          for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int bit = 8 * (r >> 2) + (r & 3);
              const int keep = ((int)(wsh[kb32] << (31 - bit))) >> 31;
              sacc[kb32][r] = __int_as_float((__float_as_int(sacc[kb32][r]) & keep) |
                                             (~keep & (int)0xff800000));
            }
        }

        // Row max: in-lane, then across the two lane halves.
        float mx = -INFINITY;
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb32][r]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx * c);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;

        // p = 2^(s*c - m); partial row sum; P rounded to the input dtype for P V.
        float psum = 0.f;
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb32][r], c, -m_new));
            sacc[kb32][r] = e;
            psum += e;
          }
        l_run = l_run * alpha + psum;

        // Branch-free rescale of the O accumulator.
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

        u32x4 pk[PKS];
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x8 t;
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = sacc[kb32][8 * h + e];
            pk[2 * kb32 + h] = pack8<BF16>(t);
          }

        // O^T += V^T P^T on the matrix cores; P comes straight from registers.
#pragma unroll
        for (int ks = 0; ks < PKS; ++ks) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int r = 32 * db + l32, cch = 2 * ks + hl;
            const u32x4 a = *(const u32x4*)(vb + r * BN * 2 + ((cch ^ (r % VC)) * 16));
            oacc[db] = mfma32<BF16>(a, pk[ks], oacc[db]);
          }
        }
      }
    }

    if (j + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
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
