// HIP kernels (gfx950 / CDNA4) for the weight stream of the speculative-decoding
// verify pass: a one-time weight pack, NVFP4, FP8 E4M3 and affine 4-bit
// skinny GEMMs (M <= 32 rows) with a stream-K schedule and a fixed-order
// split-K reduction, the vocabulary-head argmax + greedy-accept epilogue, and
// two HBM probes.
//
// Method: "lithos-metal: per-layer megakernels for Qwen3.8-27B on an M5 Max ..."
// (sections "What one token costs the bus", "How DSpark is wired in",
// "Formats, and what runs where", and "The control experiment the blog leaves
// out" for the idea of a weight layout packed for the bus); "144 tok/s needs
// 502 GB/s ..." (section "Why Apple silicon, and why not the M5": the verify
// rows form a real GEMM); "Beating Splash on an M5 Max ..." (sections "The
// kernels were not the gap": split-K on narrow projections; "What actually
// moved the needle": acceptance on the GPU).
//
// Design (MI355X-first, not the pages' Metal tiles):
//  * Packed weights. A tile is 64 weight rows (four sub-tiles of 16), an
//    iteration 128 K. The weights of one (tile, iteration) are one contiguous
//    block, tiles in order, iterations in order inside a tile, arranged so that
//    every wave load instruction reads 1 KB contiguous and lands exactly in the
//    lanes that feed the MFMA (NVFP4: 4 KB of codes + 512 B of scales per
//    block; FP8: 8 KB). A worker's stream is one linear read.
//  * The matrix unit is v_mfma_f32_16x16x32_bf16: lane l gives A row l % 16
//    and B column l % 16, both for k-group l / 16 (8 consecutive k); MFMA j of
//    an iteration covers k [32j, 32j+32).
//  * NVFP4: the E4M3 block scale is applied after the MFMA. The A operand holds
//    each group of 8 activation rows twice: rows 0-7 carry X only on k-groups
//    0,1 (= scale block 2j) and rows 8-15 only on k-groups 2,3 (= block 2j+1),
//    zeros elsewhere. D rows 0-7 are then block 2j's partial sums and rows 8-15
//    block 2j+1's, so every accumulator lane multiplies by exactly one block
//    scale (one fp32 FMA) and lanes l, l+32 are added once per tile piece.
//    gfx950's packed fp4 -> bf16 convert applies only the exponent of its
//    scale operand, so a non-power-of-two E4M3 scale cannot be folded into it.
//  * NVFP4 with more than 8 rows: the same weights scaled in registers (exact
//    in bf16), 16 activation rows per MFMA.
//  * FP8: the MFMA accumulates directly; the per-tensor scale is applied in
//    the epilogue.
//  * Affine 4-bit (scale * q + bias per 64 K, "144 tok/s needs 502 GB/s ...",
//    section "The engine hard-codes the model"): nibbles decode to bf16
//    128 + q with one mask-and-or per two weights; the group sums of X come
//    from MFMAs against ones, and s * (x . (128+q)) + (b - 128 s) * sum(x) is
//    accumulated in fp32.
//  * Weights stream with non-temporal 16-byte loads, 3 iterations in flight
//    per wave; one workgroup of 4 waves per CU, registers budgeted for one
//    wave per SIMD. The activation rows of an iteration are read as whole
//    128-byte lines (8 rows x 128 B per load) in the same ring and put in
//    A-operand order through a small LDS area of the wave; at M <= 8 only
//    rows 0-7 are read (an 8-row instance of the 16-row FP8 and affine
//    kernels).
//  * Stream-K over 4-wave workgroups: workgroup g owns iterations
//    [g*W/G, (g+1)*W/G) of the (tile, iteration) space and each wave a
//    contiguous quarter of that. Tiles shared by waves of one workgroup are
//    summed through LDS; tiles shared by workgroups are reduced by the
//    last-arriving workgroup in workgroup order (deterministic, independent of
//    M). Cross-workgroup data moves only through agent-scope atomics, so no
//    L2 write-back/invalidate is issued.
//  * Accumulating FP8 epilogue (fp32 output, zero on entry): the units are
//    half tiles (two sub-tiles, the first or second half of every block) and
//    the schedule gives each unit at most two workgroup shares; every share
//    is added into the output with one fp32 atomic add per element. From
//    zero, 0 + a + b = 0 + b + a, so the result does not depend on the order
//    in which the shares arrive, and no workgroup waits on another (no piece
//    exchange, no counter, no final store after a round trip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "vq_internal.h"
#include "vq_keys.h"

namespace vq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// 8 E2M1 codes (one dword, low nibble first) -> 8 bf16 in k order.
__device__ __forceinline__ bf16x8_t dec_fp4x8(uint32_t w) {
  auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, a);
  r.y = __builtin_bit_cast(uint32_t, b);
  r.z = __builtin_bit_cast(uint32_t, c);
  r.w = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 E2M1 codes (one dword, low nibble first) times one E4M3 block scale ->
// 8 bf16 in k order. Every E2M1 x E4M3 product has at most 6 significant bits
// and lies inside bf16's normal range, so each product is exact in bf16.
__device__ __forceinline__ bf16x8_t dec_fp4x8_scaled(uint32_t w, float sc) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  u32x4_t r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x2_t v = b == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
              : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
              : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                       : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v.x = v.x * sc;
    v.y = v.y * sc;
    r[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 unsigned 4-bit codes in the packed affine order (the even-k nibbles in
// bits 0-15, the odd-k nibbles in bits 16-31, k ascending within each half)
// -> 8 bf16 holding 128 + q in k order. bf16 0x43nn is 128 + nn exactly for
// nn < 128, so each output dword is one mask-and-or of a shifted word.
__device__ __forceinline__ bf16x8_t dec_q4x8_offset(uint32_t w) {
  u32x4_t r;
#pragma unroll
  for (int b = 0; b < 4; ++b) r[b] = ((w >> (4 * b)) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 E4M3FN codes (two dwords, byte order = k order) -> 8 bf16.
__device__ __forceinline__ bf16x8_t dec_fp8x8(uint32_t lo, uint32_t hi) {
  auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, a);
  r.y = __builtin_bit_cast(uint32_t, b);
  r.z = __builtin_bit_cast(uint32_t, c);
  r.w = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(bf16x8_t, r);
}

// The four E4M3 block scales of one dword (byte j = block j) as fp32, two per
// convert: 8 instead of 16 scale converts per iteration, the same values
// (M = 16 [gate; up] 26.4 -> 25.0 us, the 4-lane pass 5.94 -> 5.86 ms).
__device__ __forceinline__ void scales4(uint32_t w, float (&s)[4]) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  s[0] = lo[0];
  s[1] = lo[1];
  s[2] = hi[0];
  s[3] = hi[1];
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x0040u;
  return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? quiet : rounded);
}

__device__ __forceinline__ void store_out(void* y, int f32, size_t idx, float v) {
  if (f32)
    reinterpret_cast<float*>(y)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
}

// ------------------------------------------------------------- weight pack
//
// Canonical row of sub-tile t, sub-tile row n, of tile `tile` (-1: past the
// matrix, packed as zeros). Plain: tile rows 64*tile .. +63. Gate/up pairs:
// sub-tiles 0,1 hold gate rows 32*tile + 16t + n, sub-tiles 2,3 the up rows
// half + 32*tile + 16(t-2) + n, half = rows / 2.
__device__ __forceinline__ int pack_row(const PackParams& p, int tile, int t, int n) {
  if (p.gate_up) {
    const int half = p.rows / 2;
    const int r = tile * 32 + (t & 1) * 16 + n;
    return r < half ? r + (t >> 1) * half : -1;
  }
  const int r = tile * kTileRows + t * kSub + n;
  return r < p.rows ? r : -1;
}

// One thread per 16-byte chunk of a packed NVFP4 block (288 chunks: 256 of
// codes, 32 of scales). Codes chunk (t, l): lane l = 16g + n gets, for MFMA
// j = 0..3, the 4 code bytes of k [128*it + 32j + 8g, +8) of row (t, n).
// Scales chunk (h, n): byte 4t + j = scale of block 8*it + 2j + h of row (t, n).
__device__ __forceinline__ void pack_nvfp4_chunk(const PackParams& p, int64_t gid) {
  const int64_t blk = gid / 288;
  const int c = (int)(gid - blk * 288);
  const int tile = (int)(blk / p.iters), it = (int)(blk - (int64_t)tile * p.iters);
  const size_t K = (size_t)p.K;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (c < 256) {
    const int t = c >> 6, l = c & 63, n = l & 15, g = l >> 4;
    const int r = pack_row(p, tile, t, n);
    if (r >= 0) {
      const uint8_t* row = p.codes + (size_t)r * (K / 2) + (size_t)it * 64 + g * 4;
      v.x = *reinterpret_cast<const uint32_t*>(row);
      v.y = *reinterpret_cast<const uint32_t*>(row + 16);
      v.z = *reinterpret_cast<const uint32_t*>(row + 32);
      v.w = *reinterpret_cast<const uint32_t*>(row + 48);
    }
  } else {
    const int h = (c - 256) >> 4, n = (c - 256) & 15;
    uint32_t words[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = pack_row(p, tile, t, n);
      uint32_t wv = 0u;
      if (r >= 0) {
        const uint8_t* srow = p.scales + (size_t)r * (K / 16) + (size_t)it * 8 + h;
        wv = (uint32_t)srow[0] | ((uint32_t)srow[2] << 8) | ((uint32_t)srow[4] << 16) | ((uint32_t)srow[6] << 24);
      }
      words[t] = wv;
    }
    v = u32x4_t{words[0], words[1], words[2], words[3]};
  }
  *reinterpret_cast<u32x4_t*>(p.out + blk * kBlockF4 + (size_t)c * 16) = v;
}

__global__ __launch_bounds__(256) void pack_nvfp4_kernel(PackParams p) {
  const int64_t nchunks = (int64_t)p.tiles * p.iters * 288;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < nchunks;
       gid += (int64_t)gridDim.x * blockDim.x)
    pack_nvfp4_chunk(p, gid);
}

// Canonical code dword (byte j = k 2j low nibble, k 2j+1 high nibble) -> the
// packed affine order: even-k nibbles in bits 0-15, odd-k nibbles in 16-31.
__device__ __forceinline__ uint32_t affine_nibble_order(uint32_t w) {
  auto squeeze = [](uint32_t x) {  // low nibbles of the 4 bytes -> bits 0-15
    x = (x | (x >> 4)) & 0x00FF00FFu;
    return (x | (x >> 8)) & 0x0000FFFFu;
  };
  return squeeze(w & 0x0F0F0F0Fu) | (squeeze((w >> 4) & 0x0F0F0F0Fu) << 16);
}

// One thread per 16-byte chunk of a packed affine block (288 chunks): the 256
// code chunks as for NVFP4 (each dword in the affine nibble order), then 32
// chunks of (scale, bias) pairs. Chunk
// (n, part) holds, for sub-tiles t = 2 part, 2 part + 1 of row n and groups
// h = 0, 1 of the iteration, the bf16 pairs (scale, bias) as two 16-bit
// halves of one dword: t, then h.
__device__ __forceinline__ void pack_affine_chunk(const PackParams& p, int64_t gid) {
  const int64_t blk = gid / 288;
  const int c = (int)(gid - blk * 288);
  const int tile = (int)(blk / p.iters), it = (int)(blk - (int64_t)tile * p.iters);
  if (c < 256) {
    const int t = c >> 6, l = c & 63, n = l & 15, g = l >> 4;
    const int r = pack_row(p, tile, t, n);
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r >= 0) {
      const uint8_t* row = p.codes + (size_t)r * ((size_t)p.K / 2) + (size_t)it * 64 + g * 4;
      v.x = affine_nibble_order(*reinterpret_cast<const uint32_t*>(row));
      v.y = affine_nibble_order(*reinterpret_cast<const uint32_t*>(row + 16));
      v.z = affine_nibble_order(*reinterpret_cast<const uint32_t*>(row + 32));
      v.w = affine_nibble_order(*reinterpret_cast<const uint32_t*>(row + 48));
    }
    *reinterpret_cast<u32x4_t*>(p.out + blk * kBlockF4 + (size_t)c * 16) = v;
    return;
  }
  const size_t G = (size_t)p.K / 64;
  const int n = (c - 256) >> 1, part = (c - 256) & 1;
  uint32_t words[4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int r = pack_row(p, tile, 2 * part + tt, n);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t wv = 0u;
      if (r >= 0) {
        const size_t gi = (size_t)r * G + (size_t)it * 2 + h;
        wv = (uint32_t)reinterpret_cast<const uint16_t*>(p.scales)[gi] |
             ((uint32_t)reinterpret_cast<const uint16_t*>(p.biases)[gi] << 16);
      }
      words[2 * tt + h] = wv;
    }
  }
  *reinterpret_cast<u32x4_t*>(p.out + blk * kBlockF4 + (size_t)c * 16) = u32x4_t{words[0], words[1], words[2], words[3]};
}

__global__ __launch_bounds__(256) void pack_affine_kernel(PackParams p) {
  const int64_t nchunks = (int64_t)p.tiles * p.iters * 288;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < nchunks;
       gid += (int64_t)gridDim.x * blockDim.x)
    pack_affine_chunk(p, gid);
}

// One thread per 16-byte chunk of a packed FP8 block (512 chunks). Chunk
// (t, h, l): lane l = 16g + n gets the 8 weights of k [128*it + 32j + 8g, +8)
// for j = 2h and j = 2h+1 of row (t, n).
__device__ __forceinline__ void pack_fp8_chunk(const PackParams& p, int64_t gid) {
  const int64_t blk = gid / 512;
  const int c = (int)(gid - blk * 512);
  const int tile = (int)(blk / p.iters), it = (int)(blk - (int64_t)tile * p.iters);
  const int t = c >> 7, h = (c >> 6) & 1, l = c & 63, n = l & 15, g = l >> 4;
  const int r = pack_row(p, tile, t, n);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (r >= 0) {
    const uint8_t* row = p.codes + (size_t)r * p.K + (size_t)it * kIterK + 64 * h + 8 * g;
    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(row);
    const u32x2_t b = *reinterpret_cast<const u32x2_t*>(row + 32);
    v = u32x4_t{a.x, a.y, b.x, b.y};
  }
  *reinterpret_cast<u32x4_t*>(p.out + blk * kBlockF8 + (size_t)c * 16) = v;
}

__global__ __launch_bounds__(256) void pack_fp8_kernel(PackParams p) {
  const int64_t nchunks = (int64_t)p.tiles * p.iters * 512;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < nchunks;
       gid += (int64_t)gridDim.x * blockDim.x)
    pack_fp8_chunk(p, gid);
}

// ------------------------------------------------------------ kernel traits
//
// RG row groups: NVFP4 groups of 8 activation rows (each group's A operand is
// the 16-row "two blocks" arrangement above), FP8 groups of 16 rows.

template <int FMT, int RG>
struct Traits {
  static constexpr int REGS = 4 * RG;  // accumulator registers per sub-tile
  static constexpr int RED = 16;       // lanes holding the same output rows
  static __device__ __forceinline__ bool out_lane(int lane) { return FMT != FMT_NVFP4 || lane < 32; }
  // output row of accumulator register (rg, r) of this lane
  static __device__ __forceinline__ int row(int lane, int rg, int r) {
    if (FMT == FMT_NVFP4) return 8 * rg + 4 * ((lane >> 4) & 1) + r;
    return 16 * rg + 4 * (lane >> 4) + r;
  }
};

template <int EPI>
__device__ __forceinline__ int out_col(int tile, int t, int n) {
  if (EPI == EPI_SILU) return tile * (kTileRows / 2) + (t & 1) * kSub + n;
  if (EPI == EPI_ACC) return tile * (kTileRows / 2) + t * kSub + n;  // tile = half-tile unit
  return tile * kTileRows + t * kSub + n;
}

// Sub-tiles per unit of the (unit, iteration) space (the kernel's NT): a
// whole 64-row tile (4), half of one for the accumulating epilogue (2), or a
// pair of tiles for the scaled NVFP4 family on wide outputs (8).

// ---------------------------------------------------------- per-iteration data

template <int FMT, int NT = kNT>
struct WBuf;
template <>
struct WBuf<FMT_NVFP4, kNT> {
  u32x4_t c[kNT];  // per sub-tile: code dwords of MFMA steps 0..3
  u32x4_t s;       // per sub-tile: the 4 block scales of this lane's half
  __device__ __forceinline__ uint32_t scales(int t) const { return s[t]; }
};
template <>
struct WBuf<FMT_NVFP4S, kNT> : WBuf<FMT_NVFP4, kNT> {};
// A tile pair (scaled NVFP4 at M > 8 on wide outputs): the two tiles' blocks
// of one iteration, sub-tiles 0-3 from the first tile and 4-7 from the second.
template <>
struct WBuf<FMT_NVFP4S, 2 * kNT> {
  u32x4_t c[2 * kNT];
  u32x4_t s[2];
  __device__ __forceinline__ uint32_t scales(int t) const { return s[t >> 2][t & 3]; }
};
template <>
struct WBuf<FMT_AFFINE, kNT> {
  u32x4_t c[kNT];   // per sub-tile: code dwords of MFMA steps 0..3
  u32x4_t sb[2];    // (scale, bias) of this lane's row: sub-tiles 0,1 then 2,3; groups 0,1
};
template <int NT>
struct WBuf<FMT_FP8, NT> {
  u32x4_t c[NT][2];  // per sub-tile: weights of MFMA steps (0,1) and (2,3)
};
template <int RG>
struct XBuf {
  u32x4_t xa[RG][4];  // X fragments of MFMA steps 0..3 per row group
};

// Weights are read once per pass: non-temporal loads stream them without
// displacing the activations, partial sums and counters from L2 and the MALL
// (measured 5 % faster over the whole pass than ordinary loads). They are
// buffer loads off a resource per block: the block's address sits in SGPRs
// and each lane supplies a 32-bit offset, so the ring's loads cost no 64-bit
// address arithmetic (M = 8 pass 0.3-0.5 % faster than global loads on three
// boxes; adding the scope bits to the non-temporal hint changed nothing).
// The resource's range is the bytes the unit reads from that base, so an
// offset past it reads zeros instead of another block.
constexpr int kBufNT = 2;           // cache-policy operand: non-temporal
constexpr int kBufWord3 = 0x00020000;  // resource word 3 for raw dword access
struct WRes {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ WRes(const uint8_t* base, int bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, kBufWord3)) {}
  __device__ __forceinline__ u32x4_t ld(int off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNT);
  }
};

// blk: the block, or for a half-tile unit (NT = 2, FP8 only) the start of the
// half's two sub-tiles inside its block; blk2: a tile pair's second block.
template <int FMT, int NT>
__device__ __forceinline__ void load_w(WBuf<FMT, NT>& b, const uint8_t* blk, const uint8_t* blk2, int lane) {
  static_assert(NT == kNT || (NT < kNT && FMT == FMT_FP8) || (NT > kNT && FMT == FMT_NVFP4S),
                "half-tile units are FP8 only, tile pairs scaled NVFP4 only");
  if constexpr (NT > kNT) {
    const WRes w(blk, kBlockF4), w2(blk2, kBlockF4);
#pragma unroll
    for (int t = 0; t < kNT; ++t) b.c[t] = w.ld(t * 1024 + lane * 16);
#pragma unroll
    for (int t = 0; t < kNT; ++t) b.c[kNT + t] = w2.ld(t * 1024 + lane * 16);
    b.s[0] = w.ld(4096 + (((lane >> 5) * 16) + (lane & 15)) * 16);
    b.s[1] = w2.ld(4096 + (((lane >> 5) * 16) + (lane & 15)) * 16);
  } else if constexpr (FMT == FMT_AFFINE) {
    const WRes w(blk, kBlockF4);
#pragma unroll
    for (int t = 0; t < kNT; ++t) b.c[t] = w.ld(t * 1024 + lane * 16);
    b.sb[0] = w.ld(4096 + (lane & 15) * 32);
    b.sb[1] = w.ld(4096 + (lane & 15) * 32 + 16);
  } else if constexpr (FMT != FMT_FP8) {
    const WRes w(blk, kBlockF4);
#pragma unroll
    for (int t = 0; t < kNT; ++t) b.c[t] = w.ld(t * 1024 + lane * 16);
    b.s = w.ld(4096 + (((lane >> 5) * 16) + (lane & 15)) * 16);
  } else {
    const WRes w(blk, NT * 2048);  // a half-tile unit reads half of its block
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      b.c[t][0] = w.ld((t * 2 + 0) * 1024 + lane * 16);
      b.c[t][1] = w.ld((t * 2 + 1) * 1024 + lane * 16);
    }
  }
}

// X cursor: each iteration's activation rows are read as whole 128-byte
// lines (8 rows x 128 B per load instruction, two lines per row and
// iteration) and put in MFMA A-operand order through the wave's LDS area
// (stage_x). An A operand for one 32-K step is 16 rows x 64 B: loaded
// directly it would touch half of 16 lines per instruction, twice the line
// requests per byte.
//  A full 16-row group: 4 loads per iteration, rows 0-7 and 8-15 of each
//    half of the iteration's k range.
//  A half group (LAST8: the last group holds at most 8 rows -- M <= 8 for the
//    16-row kernels, M = 17-24 for two groups -- and the NVFP4 M <= 8
//    family): 2 loads, rows 0-7. The NVFP4 A operand holds the rows twice
//    with zeros in between (rows 0-7 on k-groups 0,1, rows 8-15 on k-groups
//    2,3; see compute_iter); the 16-row kernels' rows 8-15 of a half group
//    are padding. Lanes that hold zeros read a zeroed slot.
// Lane l reads row l >> 3 (+ 8 for the second half of a 16-row group),
// 16-byte segment (l & 7) ^ (l >> 3) of the line, and its 16 bytes land at
// position l & 7 of that row in LDS: the swizzle keeps the fragment reads
// free of bank conflicts.
template <int FMT, int RG, bool LAST8 = false>
struct XCursor {
  // the last row group is a half group
  static constexpr bool kHalf = FMT == FMT_NVFP4 || LAST8;
  static_assert(FMT != FMT_NVFP4 || RG == 1, "the NVFP4 M <= 8 family has one row group");
  static constexpr bool half_group(int rg) { return kHalf && rg == RG - 1; }
  const uint16_t* row[RG];   // rows 0-7 of each row group
  const uint16_t* half[RG];  // full groups: rows 8-15
  __device__ __forceinline__ void init(const GemmParams& p, int lane) {
    const int r = lane >> 3, seg = (lane & 7) ^ r;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      int m0 = 16 * rg + r, m1 = m0 + 8;
      m0 = m0 < p.M ? m0 : p.M - 1;  // rows past M are padding: any valid row will do
      m1 = m1 < p.M ? m1 : p.M - 1;
      row[rg] = p.x + (size_t)m0 * p.K + 8 * seg;
      half[rg] = p.x + (size_t)m1 * p.K + 8 * seg;
    }
  }
  // Full group: b.xa[rg][c] holds rows 8 (c & 1) .. +7 of k 64 (c >> 1) ..
  // +63. Half group: b.xa[rg][c], c = 0, 1, holds rows 0-7 of k 64 c .. +63.
  __device__ __forceinline__ void load(XBuf<RG>& b, int kit) const {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const uint16_t* lo = row[rg] + (size_t)(kit * kIterK);
      if (half_group(rg)) {
        b.xa[rg][0] = ld16(lo);
        b.xa[rg][1] = ld16(lo + 64);
      } else {
        const uint16_t* hi = half[rg] + (size_t)(kit * kIterK);
        b.xa[rg][0] = ld16(lo);
        b.xa[rg][1] = ld16(hi);
        b.xa[rg][2] = ld16(lo + 64);
        b.xa[rg][3] = ld16(hi + 64);
      }
    }
  }
};

// Activation staging: one chunk per (row group, load) holds 8 rows x 128 B;
// 1152 B per chunk rather than 1024 puts the two row halves of a fragment
// read on different banks. Full groups come first (4 chunks each), then a
// half group's 2 chunks and one zeroed 16-byte slot.
constexpr int kXChunk = 72;  // u32x4 per chunk
template <int RG, bool HALF>
struct XStage {
  static constexpr int kChunks = HALF ? 4 * (RG - 1) + 2 : 4 * RG;
  static constexpr int kZero = kChunks * kXChunk;  // HALF: the zero slot
  static constexpr int kSize = kChunks * kXChunk + (HALF ? 8 : 0);
};

// Whole-line registers (see XCursor::load) -> MFMA A operands, through this
// wave's LDS area xs. The wave barriers keep the compiler from moving the LDS
// reads above the writes, or the next call's writes above this call's reads;
// a wave's LDS operations execute in order.
template <typename XC, int RG, int FMT>
__device__ __forceinline__ void stage_x(const XBuf<RG>& in, XBuf<RG>& out, u32x4_t* xs, int lane) {
  using XS = XStage<RG, XC::kHalf>;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    if (XC::half_group(rg)) {
#pragma unroll
      for (int c = 0; c < 2; ++c) xs[(4 * rg + c) * kXChunk + lane] = in.xa[rg][c];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) xs[(4 * rg + c) * kXChunk + lane] = in.xa[rg][c];
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int i = lane & 15, g = lane >> 4;  // MFMA A operand: row i, k 8 g .. +7 of the step
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    if (XC::half_group(rg)) {
      const bool carries = FMT == FMT_NVFP4 ? (i >> 3) == (g >> 1) : i < 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int seg = 4 * (j & 1) + g;
        const int at = carries ? (4 * rg + (j >> 1)) * kXChunk + (i & 7) * 8 + (seg ^ (i & 7)) : XS::kZero;
        out.xa[rg][j] = xs[at];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 2 * (j >> 1) + (i >> 3);
        const int seg = 4 * (j & 1) + g;
        out.xa[rg][j] = xs[(4 * rg + c) * kXChunk + (i & 7) * 8 + (seg ^ (i & 7))];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
}

template <int FMT, int RG, int NT = kNT>
struct Acc {
  float v[NT][4 * RG];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4 * RG; ++r) v[t][r] = 0.0f;
  }
  __device__ __forceinline__ float get(int t, int r) const { return v[t][r]; }
  // NVFP4: lanes l and l^32 hold the even- and odd-block halves of the sums.
  __device__ __forceinline__ void combine() {
    if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4 * RG; ++r) v[t][r] = v[t][r] + __shfl_xor(v[t][r], 32);
    }
  }
};

template <int FMT, int RG, int NT>
__device__ __forceinline__ void compute_iter(const WBuf<FMT, NT>& b, const XBuf<RG>& x, Acc<FMT, RG, NT>& acc) {
  if constexpr (FMT == FMT_NVFP4) {
    // All 16 MFMAs of the block first, each into its own result registers,
    // then the block-scale FMAs: the matrix unit's latency is covered by the
    // other MFMAs and the decodes instead of stalling every FMA chain (the
    // summation order per accumulator is unchanged: j = 0..3 within t).
    static_assert(RG == 1, "the block-scale-after-MFMA family serves M <= 8 (one row group)");
    f32x4_t d[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        d[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.xa[0][j]),
                                                          dec_fp4x8(b.c[t][j]), f32x4_t{}, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float s4[4];
      scales4(b.scales(t), s4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = s4[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc.v[t][r] = __builtin_fmaf(sc, d[t][j][r], acc.v[t][r]);
      }
    }
  } else if constexpr (FMT == FMT_NVFP4S) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float s4[4];
      scales4(b.scales(t), s4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t wv = dec_fp4x8_scaled(b.c[t][j], s4[j]);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          f32x4_t a = {acc.v[t][4 * rg], acc.v[t][4 * rg + 1], acc.v[t][4 * rg + 2], acc.v[t][4 * rg + 3]};
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.xa[rg][j]), wv, a, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc.v[t][4 * rg + r] = a[r];
        }
      }
    }
  } else if constexpr (FMT == FMT_AFFINE) {
    // sum_k x (s q + b) over a group of 64 = s * (x . (128 + q)) +
    // (b - 128 s) * (sum of x): per group and sub-tile two MFMAs give
    // x . (128 + q) for the lane's row; the group sums of x come from two
    // MFMAs against ones (shared by the sub-tiles), in the same accumulator
    // layout.
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    f32x4_t sx[RG][2];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sx[rg][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.xa[rg][2 * h]), ones,
                                                            f32x4_t{}, 0, 0, 0);
        sx[rg][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.xa[rg][2 * h + 1]), ones,
                                                            sx[rg][h], 0, 0, 0);
      }
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8_t w0 = dec_q4x8_offset(b.c[t][2 * h]);
        const bf16x8_t w1 = dec_q4x8_offset(b.c[t][2 * h + 1]);
        const uint32_t pair = b.sb[t >> 1][2 * (t & 1) + h];
        const float sc = __uint_as_float(pair << 16);
        const float bi = __builtin_fmaf(-128.0f, sc, __uint_as_float(pair & 0xFFFF0000u));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.xa[rg][2 * h]), w0,
                                                              f32x4_t{}, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.xa[rg][2 * h + 1]), w1, d, 0,
                                                      0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc.v[t][4 * rg + r] = __builtin_fmaf(sc, d[r], __builtin_fmaf(bi, sx[rg][h][r], acc.v[t][4 * rg + r]));
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t c = b.c[t][j >> 1];
        const bf16x8_t wv = (j & 1) ? dec_fp8x8(c.z, c.w) : dec_fp8x8(c.x, c.y);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          f32x4_t a = {acc.v[t][4 * rg], acc.v[t][4 * rg + 1], acc.v[t][4 * rg + 2], acc.v[t][4 * rg + 3]};
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.xa[rg][j]), wv, a, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc.v[t][4 * rg + r] = a[r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- epilogues

// Final step of the head: reduce the bucketed candidates, write argmax / max,
// run the greedy accept per lane and reset the workspace. One wave.
__device__ __forceinline__ void head_final(const GemmParams& p, int lane) {
  int idx = -1;
  if (lane < p.M) {
    unsigned long long best = 0ull;
    for (int b = 0; b < kBuckets; ++b) {
      unsigned long long k = __hip_atomic_load(&p.best[b * kMaxRows + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      best = k > best ? k : best;
    }
    idx = best ? (int)(0xFFFFFFFFu - (uint32_t)best) : -1;
    p.argmax_out[lane] = idx;
    if (p.maxlogit_out) p.maxlogit_out[lane] = key_value(best);
    for (int b = 0; b < kBuckets; ++b)
      __hip_atomic_store(&p.best[b * kMaxRows + lane], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Greedy accept: lane L < lanes scans its R rows.
  const int L = lane < p.lanes ? lane : 0;
  int a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int src = L * p.R + (j < p.R ? j : 0);
    a[j] = __shfl(idx, src);
  }
  if (lane < p.lanes) {
    int acc = 0;
    bool go = true;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      if (go && j < p.R - 1 && a[j] >= 0 && a[j] == p.draft[lane * (p.R - 1) + j]) ++acc;
      else go = false;
    }
    p.accept_len_out[lane] = acc + 1;
    if (p.commit_out) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < p.R) p.commit_out[lane * p.R + j] = j <= acc ? a[j] : -1;
    }
  }
  if (lane == 0) __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Running per-lane argmax candidates of a worker (vocabulary head only).
template <int REGS>
struct Best {
  unsigned long long k[REGS];
};

// Epilogue of a finished tile. NONE / SILU store the outputs; ARGMAX stores
// the optional logits and folds the tile into the lane's running candidates.
template <int FMT, int EPI, int RG, typename GetF>
__device__ __forceinline__ void epilogue(const GemmParams& p, int tile, int lane, GetF get, Best<4 * RG>& best) {
  using T = Traits<FMT, RG>;
  if (!T::out_lane(lane)) return;
  const int n = lane & 15;
  const float sc = p.out_scale;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = T::row(lane, rg, r);
      const int q = 4 * rg + r;
      if constexpr (EPI == EPI_ACC) {
        // a workgroup's share of a half-tile unit (the whole unit, or one of
        // its two shares) is added into the fp32 output: from zero, 0 + a and
        // 0 + a + b = 0 + b + a are exact in any order of arrival
        if (m < p.M) {
          float* y = static_cast<float*>(p.y);
#pragma unroll
          for (int t = 0; t < kNT / 2; ++t) {
            const int col = out_col<EPI>(tile, t, n);
            if (col < p.N)
              __hip_atomic_fetch_add(y + (size_t)m * p.N + col, get(t, q) * sc, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      } else if constexpr (EPI == EPI_NONE) {
        if (m < p.M) {
#pragma unroll
          for (int t = 0; t < kNT; ++t) {
            const int col = out_col<EPI>(tile, t, n);
            if (col < p.N) store_out(p.y, p.y_f32, (size_t)m * p.N + col, get(t, q) * sc);
          }
        }
      } else if constexpr (EPI == EPI_SILU) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int col = out_col<EPI>(tile, t, n);
          if (m < p.M && col < p.N) {
            const float gv = get(t, q) * sc;
            const float uv = get(t + 2, q) * sc;
            const float h = gv / (1.0f + expf(-gv)) * uv;
            store_out(p.y, p.y_f32, (size_t)m * p.N + col, h);
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          const int col = out_col<EPI>(tile, t, n);
          const float v = get(t, q) * sc;
          if (m < p.M && col < p.N) {
            if (p.y) store_out(p.y, p.y_f32, (size_t)m * p.N + col, v);
            const unsigned long long k = argmax_key(v, (uint32_t)col);
            best.k[q] = k > best.k[q] ? k : best.k[q];
          }
        }
      }
    }
  }
}

// Epilogue of a finished unit: its tile, its half tile (accumulating), or both
// tiles of a pair. A pair's second tile past the last one (an odd tile count)
// has only columns >= N, which the epilogue skips.
template <int FMT, int EPI, int RG, int NT, typename GetF>
__device__ __forceinline__ void unit_epilogue(const GemmParams& p, int unit, int lane, GetF get, Best<4 * RG>& best) {
  if constexpr (NT > kNT) {
    epilogue<FMT, EPI, RG>(p, 2 * unit, lane, get, best);
    epilogue<FMT, EPI, RG>(p, 2 * unit + 1, lane, [&](int t, int r) { return get(kNT + t, r); }, best);
  } else {
    epilogue<FMT, EPI, RG>(p, unit, lane, get, best);
  }
}

// Cross-workgroup data (partial sums, counters, argmax candidates) only moves
// through agent-scope atomics, which gfx950 performs with the SC1 bit: stores
// write through to the memory side (the level all eight XCDs share) and loads
// and read-modify-writes are served there, so they are coherent across XCDs
// without any L2 write-back or invalidate. The ordering a piece needs --
// "every store of my piece is visible before my counter increment" -- comes
// from s_waitcnt vmcnt(0): on gfx9 a vector store decrements vmcnt only when
// the memory system acknowledges it, and an SC1 store is acknowledged once it
// is written at that shared level. So after the wait, any agent that observes
// the increment and then issues SC1 loads sees the piece. The reader side
// needs no wait of its own: its loads are issued after the counter value they
// depend on has returned. The compiler does not model s_waitcnt as touching
// memory, so compiler-only fences on both sides keep it from moving the atomic
// stores or the counter operation across the wait (no instruction is emitted
// for them). The formally ordered alternative -- a release on the counter
// increment -- costs an L2 write-back (buffer_wbl2) per piece.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Stream-K over workgroups: workgroup g owns iterations [g*W/G, (g+1)*W/G).
__device__ __forceinline__ int64_t wg_start(int64_t g, const GemmParams& p) { return g * p.total / p.wgs; }
// The workgroup whose range contains iteration `it`.
__device__ __forceinline__ int64_t wg_of(int64_t it, const GemmParams& p) {
  return ((it + 1) * p.wgs - 1) / p.total;
}

// Lanes whose accumulators hold distinct sums (NVFP4: after the l / l^32
// combine, lanes 32..63 repeat lanes 0..31 and are neither stored nor loaded).
template <int FMT>
__device__ __forceinline__ bool holds_sum(int lane) {
  return FMT != FMT_NVFP4 || lane < 32;
}

// A piece (one wave's or one workgroup's share of a tile) is stored as value
// (t, r) of lane l at float index (t * REGS + r) * 64 + l.
template <int FMT, int REGS, int NT>
__device__ __forceinline__ void lds_put(float* slot, int lane, const float (&v)[NT][REGS]) {
  if (!holds_sum<FMT>(lane)) return;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < REGS; ++r) slot[(t * REGS + r) * 64 + lane] = v[t][r];
}
template <int FMT, int REGS, int NT>
__device__ __forceinline__ void lds_add(const float* slot, int lane, float (&v)[NT][REGS]) {
  if (!holds_sum<FMT>(lane)) return;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < REGS; ++r) v[t][r] += slot[(t * REGS + r) * 64 + lane];
}

template <int FMT, int REGS, int NT>
__device__ __forceinline__ void store_piece(const GemmParams& p, int64_t slot, int lane, const float (&v)[NT][REGS]) {
  static_assert(NT * REGS * 64 <= kSlotFloats, "slot too small");
  if (!holds_sum<FMT>(lane)) return;
  float* dst = p.partials + slot * kSlotFloats;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < REGS; ++r)
      __hip_atomic_store(&dst[(t * REGS + r) * 64 + lane], v[t][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup piece of `tile` has been published; true when it was the last
// one, i.e. the caller must reduce the pieces and finish the tile.
__device__ __forceinline__ bool arrive(const GemmParams& p, int tile, int lane) {
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the pieces' loads stay after the counter value
  const int64_t t0 = (int64_t)tile * p.iters;
  return old == (uint32_t)(wg_of(t0 + p.iters - 1, p) - wg_of(t0, p));
}

// Sum of the workgroup pieces of `tile` in workgroup order (deterministic).
// Workgroups after the first start inside the tile (their slot 0); the first
// one holds the tile in slot 0 only if it starts exactly at the tile's start.
// Up to B pieces are loaded per step (one round trip for the usual 2-4).
template <int FMT, int REGS, int NT>
__device__ __forceinline__ void reduce_tile(const GemmParams& p, int tile, int lane, float (&sum)[NT][REGS]) {
  const int64_t t0 = (int64_t)tile * p.iters;
  const int64_t g0 = wg_of(t0, p), g1 = wg_of(t0 + p.iters - 1, p);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < REGS; ++r) sum[t][r] = 0.0f;
  if (holds_sum<FMT>(lane)) {
    const int64_t first_slot = 2 * g0 + (wg_start(g0, p) == t0 ? 0 : 1);
    constexpr int B = NT * REGS <= 16 ? 4 : 2;
    for (int64_t gb = g0; gb <= g1; gb += B) {
      float v[B][NT][REGS];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (gb + b <= g1) {  // uniform
          const int64_t gg = gb + b;
          const float* a = p.partials + (gg == g0 ? first_slot : 2 * gg) * kSlotFloats;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < REGS; ++r)
              v[b][t][r] = __hip_atomic_load(&a[(t * REGS + r) * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (gb + b <= g1) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < REGS; ++r) sum[t][r] += v[b][t][r];
        }
      }
    }
  }
  if (lane == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------------- main kernel

// Iterations in flight per wave. The vector-memory counter retires loads in
// issue order, so the activation lines share the weights' ring (a shallower
// activation ring would cap the weight prefetch at its depth).
template <int FMT, int RG, int NT = kNT>
struct PipeDepth {
  // Measured with the whole-line activation loads (interleaved pass replays;
  // deeper rings and refilling a slot before its compute were slower, so more
  // bytes in flight per wave do not help): NVFP4, both families, 2 (3 and 4
  // slower; 2 took the M = 8 pass 4.18 -> 4.14 ms and the 2-lane pass
  // 4.69 -> 4.55 ms); FP8 3 at one row group (2 and 4 slower), 2 at two;
  // half-tile units 3 at one row group (2, 4 and 5 slower), 2 at two; affine
  // 3.
  static constexpr int value = NT < kNT ? (RG == 1 ? 3 : 2)
                               : (FMT == FMT_NVFP4 || FMT == FMT_NVFP4S) ? 2
                               : (FMT == FMT_FP8 && RG == 2) ? 2 : 3;
};
// Workgroups per CU the register budget is sized for. Every launch has at
// most one workgroup per CU (at most 256 workgroups of 4 waves), so one wave
// per SIMD is all that ever runs: the bound only lets the compiler keep the
// MFMA results, the prefetch ring and the accumulators in registers (measured
// 2 % faster over the pass than budgeting for two waves per SIMD).
template <int FMT, int RG>
struct Occupancy {
  static constexpr int value = 1;
};

// Schedule. Workgroup g (4 waves) owns the iteration range [S, E) of the
// (tile, iteration) space, and wave q the q-th quarter of it. A wave finishes
// every tile that lies inside its own range. A tile shared by several waves of
// the workgroup is summed through LDS, in wave order, by the lowest wave that
// touches it; if the tile also extends past [S, E), that sum is the
// workgroup's piece of the tile and goes through the global stream-K fixup,
// whose last-arriving workgroup sums the pieces in workgroup order.
//
// The values the prologue needs before the first weight load come first in
// the argument list, so the dispatcher preloads them into SGPRs (kernel
// arguments preloaded at wave launch, -amdgpu-kernarg-preload-count): the
// first loads are issued without waiting on a kernel-argument fetch
// (measured 1 % over the pass). The rest of the parameters follow in p.
//
// RGX: the row groups (1, 2), or a count whose last 16-row group holds at
// most 8 rows, so its activation loads read only those: 0 = one such group
// (FP8 and affine at M <= 8), 3 = two groups, the second of them such a
// group (16-row kernels at M = 17-24). NT: sub-tiles per unit of the schedule
// (2: half tiles of the accumulating epilogue; 4: tiles; 8: tile pairs,
// scaled NVFP4 only).
template <int FMT, int EPI, int RGX, int NT>
__global__ __launch_bounds__(256, (Occupancy<FMT, RGX>::value)) void vq_gemm_kernel(
    const uint8_t* a_w, const uint16_t* a_x, int64_t a_total, int32_t a_wgs,
    int32_t a_iters, int32_t a_K, int32_t a_M, GemmParams p) {
  constexpr int RG = RGX == 0 ? 1 : RGX == 3 ? 2 : RGX;
  p.w = a_w;
  p.x = a_x;
  p.total = a_total;
  p.wgs = a_wgs;
  p.iters = a_iters;
  p.K = a_K;
  p.M = a_M;
  using T = Traits<FMT, RG>;
  constexpr bool ACC = EPI == EPI_ACC;
  static_assert(ACC == (NT < kNT), "half-tile units are the accumulating epilogue's");
  constexpr bool JUMP = NT != kNT;  // a unit's stream is not the next run of blocks
  constexpr int PD = PipeDepth<FMT, RG, NT>::value;
  constexpr int REGS = T::REGS;
  constexpr int SLOT = NT * REGS * 64;
  constexpr size_t BLOCK = FMT == FMT_FP8 ? kBlockF8 : kBlockF4;
  __shared__ float lds[4 * SLOT];
  using XC = XCursor<FMT, RG, RGX == 0 || RGX == 3>;
  using XST = XStage<RG, XC::kHalf>;
  constexpr int XS = XST::kSize;  // activation staging per wave
  __shared__ u32x4_t xstage[4 * XS];

  const int lane = threadIdx.x & 63;
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = blockIdx.x;
  const int64_t S = wg_start(g, p), E = wg_start(g + 1, p);
  const int64_t span = E - S;
  const int64_t s = S + q * span / 4, e = S + (q + 1) * span / 4;
  const int I = p.iters;
  const int first_tile = (int)(s / I);

  Best<REGS> best;
#pragma unroll
  for (int r = 0; r < REGS; ++r) best.k[r] = 0ull;
  int finished = 0;       // tiles this wave finished (vocabulary head)
  bool lds_piece = false; // this wave's share of first_tile (entered mid-way) is in its LDS slot
  bool reg_piece = false; // acc holds this wave's share of ctile, which starts inside [s, e)
  int ctile = first_tile;
  Acc<FMT, RG, NT> acc;
  acc.zero();

  if (s < e) {
    // The wave's weight stream is the contiguous run of blocks [s, e). With
    // half-tile units, unit u is half u & 1 of tile u >> 1 and its stream the
    // first or second half of each of that tile's blocks; with tile pairs,
    // unit u is tiles 2u and 2u + 1, streamed side by side (the second one
    // re-reads the first where the tile count is odd and 2u + 1 is past it).
    constexpr size_t HALF = BLOCK / 2;  // FP8: sub-tiles 2 and 3 fill the second half of a block
    auto unit_base = [&](int64_t u) {
      if constexpr (NT < kNT) return p.w + (size_t)((u >> 1) * I) * BLOCK + (size_t)(u & 1) * HALF;
      else return p.w + (size_t)(u * (NT / kNT) * I) * BLOCK;
    };
    const int ptiles = EPI == EPI_SILU ? (p.N + kSub * 2 - 1) / (kSub * 2) : (p.N + kTileRows - 1) / kTileRows;
    int64_t lu = first_tile;  // unit of the next load
    const uint8_t* wnext = unit_base(lu) + (size_t)(s - lu * I) * BLOCK;
    XC xc;
    xc.init(p, lane);
    if constexpr (XC::kHalf) xstage[q * XS + XST::kZero] = u32x4_t{0u, 0u, 0u, 0u};
    int xkit = (int)(s - (int64_t)first_tile * I);
    int64_t lit = s;  // next iteration to load

    WBuf<FMT, NT> wb[PD];
    XBuf<RG> xb[PD];
    auto load_next = [&](int qq) {
      const uint8_t* wpair = wnext;
      if constexpr (NT > kNT) wpair = 2 * lu + 1 < ptiles ? wnext + (size_t)I * BLOCK : wnext;
      load_w<FMT, NT>(wb[qq], wnext, wpair, lane);
      xc.load(xb[qq], xkit);
      if (lit + 1 < e) {  // loads past the range re-read the last iteration
        ++lit;
        if constexpr (JUMP) {
          if (++xkit == I) {
            xkit = 0;
            wnext = unit_base(++lu);
          } else {
            wnext += BLOCK;
          }
        } else {
          wnext += BLOCK;
          if (++xkit == I) xkit = 0;
        }
      }
    };
#pragma unroll
    for (int qq = 0; qq < PD; ++qq) load_next(qq);

    int ckit = (int)(s - (int64_t)first_tile * I);
    bool started_inside = ckit != 0;

    auto compute = [&](int qq) {
      XBuf<RG> xt;
      stage_x<XC, RG, FMT>(xb[qq], xt, xstage + q * XS, lane);
      compute_iter<FMT, RG, NT>(wb[qq], xt, acc);
    };

    auto tile_end = [&]() {
      acc.combine();
      if (!started_inside) {
        unit_epilogue<FMT, EPI, RG, NT>(p, ctile, lane, [&](int t, int r) { return acc.get(t, r); }, best);
        ++finished;
      } else {
        lds_put<FMT, REGS, NT>(lds + q * SLOT, lane, acc.v);
        lds_piece = true;
      }
      acc.zero();
      started_inside = false;
      ckit = 0;
      ++ctile;
    };

    const int64_t count = e - s;
    const int64_t blocks = count / PD;
    for (int64_t bl = 0; bl < blocks; ++bl) {
#pragma unroll
      for (int qq = 0; qq < PD; ++qq) {
        compute(qq);
        load_next(qq);
        if (++ckit == I) tile_end();
      }
    }
    const int rem = (int)(count - blocks * PD);
#pragma unroll
    for (int qq = 0; qq < PD; ++qq) {
      if (qq < rem) {
        compute(qq);
        if (++ckit == I) tile_end();
      }
    }
    if (ckit != 0) {  // the range ends inside ctile
      acc.combine();
      if (started_inside) {  // ... which is first_tile, entered mid-way
        lds_put<FMT, REGS, NT>(lds + q * SLOT, lane, acc.v);
        lds_piece = true;
      } else {
        reg_piece = true;
      }
    }
  }
  __syncthreads();

  // Adds the LDS shares of the later waves that start inside `tile`.
  auto add_later_waves = [&](int tile, float (&sum)[NT][REGS]) {
    const int64_t tend = (int64_t)(tile + 1) * I;
    for (int q2 = q + 1; q2 < 4; ++q2) {
      const int64_t s2 = S + q2 * span / 4, e2 = S + (q2 + 1) * span / 4;
      if (s2 >= tend) break;
      if (s2 < e2) lds_add<FMT, REGS, NT>(lds + q2 * SLOT, lane, sum);
    }
  };
  // Finishes `tile` from this workgroup's share: directly when the tile lies
  // inside [S, E), else through the global fixup; a half-tile unit's share is
  // always added into the output.
  auto finish = [&](int tile, float (&sum)[NT][REGS]) {
    const int64_t t0 = (int64_t)tile * I;
    if (ACC || (t0 >= S && t0 + I <= E)) {  // accumulating: every share is added, no exchange
      unit_epilogue<FMT, EPI, RG, NT>(p, tile, lane, [&](int t, int r) { return sum[t][r]; }, best);
      ++finished;
      return;
    }
    if constexpr (!ACC) {
    store_piece<FMT, REGS, NT>(p, 2 * g + (tile == S / I ? 0 : 1), lane, sum);
    wait_stores();
    if (arrive(p, tile, lane)) {
      float tot[NT][REGS];
      reduce_tile<FMT, REGS, NT>(p, tile, lane, tot);
      unit_epilogue<FMT, EPI, RG, NT>(p, tile, lane, [&](int t, int r) { return tot[t][r]; }, best);
      ++finished;
    }
    }
  };

  if (reg_piece) {  // this wave is the lowest one touching ctile
    add_later_waves(ctile, acc.v);
    finish(ctile, acc.v);
  }
  if (lds_piece && s == S) {  // the workgroup starts inside first_tile: its first wave collects the share
    float sum[NT][REGS];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < REGS; ++r) sum[t][r] = 0.0f;
    lds_add<FMT, REGS, NT>(lds + q * SLOT, lane, sum);
    add_later_waves(first_tile, sum);
    finish(first_tile, sum);
  }

  if constexpr (EPI == EPI_ARGMAX) {
    if (finished > 0) {
#pragma unroll
      for (int qq = 0; qq < REGS; ++qq) {
        unsigned long long k = T::out_lane(lane) ? best.k[qq] : 0ull;
#pragma unroll
        for (int off = T::RED / 2; off >= 1; off >>= 1) {
          const unsigned long long o = __shfl_xor(k, off);
          k = o > k ? o : k;
        }
        const int m = T::row(lane, qq >> 2, qq & 3);
        if (T::out_lane(lane) && (lane % T::RED) == 0 && m < p.M && k != 0ull) {
          const int bucket = (int)((g * 4 + q) % kBuckets);
          const unsigned long long prev = __hip_atomic_fetch_max(&p.best[bucket * kMaxRows + m], k,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          asm volatile("" ::"v"(prev));  // keep the returning form: it completes before the wait below
        }
      }
      wait_stores();
      uint32_t old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(p.done, (uint32_t)finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __shfl(old, 0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // head_final's bucket loads stay after the count
      if (old + (uint32_t)finished == (uint32_t)p.tiles) head_final(p, lane);
    }
  }
}

// ------------------------------------------------------------------- probes

// Copy: each thread moves 4 x 16 bytes per step (4 loads in flight before the
// stores), non-temporal both ways, over 8192 workgroups; the fastest of the
// copy forms measured on MI355X (grid-stride 1 x 16 B, 4 x 16 B, 8 x 16 B,
// plain or non-temporal, 1,024-8,192 workgroups, and hipMemcpy device to
// device), so the copy denominator is not flattered by a weak probe.
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst, size_t n) {
  constexpr size_t chunk = (size_t)256 * kCopyUnroll;
  const size_t full = n / chunk * chunk;
  for (size_t base = (size_t)blockIdx.x * chunk; base < full; base += (size_t)gridDim.x * chunk) {
    u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + base + u * 256 + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], dst + base + u * 256 + threadIdx.x);
  }
  if (blockIdx.x == 0)  // the last n % chunk elements
    for (size_t i = full + threadIdx.x; i < n; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4_t* __restrict__ src, size_t n, u32x4_t* sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t st = (size_t)gridDim.x * blockDim.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i < n; i += st) acc ^= __builtin_nontemporal_load(src + i);
  // Never true for the probe's data in practice, but the compiler cannot know.
  if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u) sink[0] = acc;
}

// ------------------------------------------------------------------ scratch
//
// Device memory of the allocation-free GEMM entry point (the layout is in
// vq_internal.h). In host code `scratch` names a host-side stand-in, never the
// device address: hipGetSymbolAddress gives each device's own copy, and only
// that pointer is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
}  // namespace

int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxScratchDevices) return (int)hipErrorInvalidDevice;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return 0;
}

// ---------------------------------------------------------------- launchers

template <int FMT, int EPI, int NT>
static int launch_rg(const GemmParams& p, hipStream_t st) {
  const int rows = FMT == FMT_NVFP4 ? 8 : 16;
  const int rg = (p.M + rows - 1) / rows;
  const dim3 grid((unsigned)p.wgs), block(256);
  if constexpr (FMT == FMT_NVFP4) {
    (void)rg;  // launch_gemm sends M > 8 to the scaled family
    hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 1, NT>), grid, block, 0, st, p.w, p.x, p.total, p.wgs,
                       p.iters, p.K, p.M, p);
  } else {
    // 16-row groups; a last group of at most 8 rows gets the instance that
    // reads only those (M <= 8 for FP8 and affine; M = 17-24)
    if constexpr (FMT != FMT_NVFP4S) {
      if (p.M <= 8) {
        hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 0, NT>), grid, block, 0, st, p.w, p.x, p.total, p.wgs,
                           p.iters, p.K, p.M, p);
        return (int)hipGetLastError();
      }
    }
    if (rg == 1)
      hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 1, NT>), grid, block, 0, st, p.w, p.x, p.total, p.wgs,
                         p.iters, p.K, p.M, p);
    else if (p.M <= 24)
      hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 3, NT>), grid, block, 0, st, p.w, p.x, p.total, p.wgs,
                         p.iters, p.K, p.M, p);
    else
      hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 2, NT>), grid, block, 0, st, p.w, p.x, p.total, p.wgs,
                         p.iters, p.K, p.M, p);
  }
  return (int)hipGetLastError();
}

int launch_gemm(int fmt, int epi, const GemmParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (fmt == FMT_NVFP4 && p.M > 8) {
    // more than 8 rows: scale in registers, 16 activation rows per MFMA; the
    // schedule's units are tiles or, on wide outputs, tile pairs
    if (p.unit_subs != kNT && p.unit_subs != 2 * kNT) return (int)hipErrorInvalidValue;
    const bool pair = p.unit_subs == 2 * kNT;
    if (epi == EPI_NONE)
      return pair ? launch_rg<FMT_NVFP4S, EPI_NONE, 2 * kNT>(p, st) : launch_rg<FMT_NVFP4S, EPI_NONE, kNT>(p, st);
    if (epi == EPI_SILU)
      return pair ? launch_rg<FMT_NVFP4S, EPI_SILU, 2 * kNT>(p, st) : launch_rg<FMT_NVFP4S, EPI_SILU, kNT>(p, st);
    return pair ? launch_rg<FMT_NVFP4S, EPI_ARGMAX, 2 * kNT>(p, st) : launch_rg<FMT_NVFP4S, EPI_ARGMAX, kNT>(p, st);
  }
  if (p.unit_subs != (epi == EPI_ACC ? kNT / 2 : kNT)) return (int)hipErrorInvalidValue;
  if (fmt == FMT_NVFP4) {
    if (epi == EPI_NONE) return launch_rg<FMT_NVFP4, EPI_NONE, kNT>(p, st);
    if (epi == EPI_SILU) return launch_rg<FMT_NVFP4, EPI_SILU, kNT>(p, st);
    return launch_rg<FMT_NVFP4, EPI_ARGMAX, kNT>(p, st);
  }
  if (fmt == FMT_AFFINE) {
    if (epi == EPI_SILU) return launch_rg<FMT_AFFINE, EPI_SILU, kNT>(p, st);
    return launch_rg<FMT_AFFINE, EPI_NONE, kNT>(p, st);
  }
  if (epi == EPI_ACC) return launch_rg<FMT_FP8, EPI_ACC, kNT / 2>(p, st);
  return launch_rg<FMT_FP8, EPI_NONE, kNT>(p, st);
}

int launch_pack(int fmt, const PackParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t chunks = (int64_t)p.tiles * p.iters * (fmt == FMT_FP8 ? 512 : 288);
  int64_t groups = (chunks + 255) / 256;
  if (groups > 65536) groups = 65536;  // grid-stride beyond this
  const dim3 grid((unsigned)groups), block(256);
  if (fmt == FMT_NVFP4) hipLaunchKernelGGL(pack_nvfp4_kernel, grid, block, 0, st, p);
  else if (fmt == FMT_AFFINE) hipLaunchKernelGGL(pack_affine_kernel, grid, block, 0, st, p);
  else hipLaunchKernelGGL(pack_fp8_kernel, grid, block, 0, st, p);
  return (int)hipGetLastError();
}

int launch_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t chunks = bytes / 16 / (256 * kCopyUnroll);
  const unsigned groups = chunks >= 8192 ? 8192u : (chunks < 1 ? 1u : (unsigned)chunks);
  hipLaunchKernelGGL(probe_copy_kernel, dim3(groups), dim3(256), 0, st,
                     reinterpret_cast<const u32x4_t*>(src), reinterpret_cast<u32x4_t*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

int launch_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(probe_read_kernel, dim3(2048), dim3(256), 0, st,
                     reinterpret_cast<const u32x4_t*>(src), bytes / 16, reinterpret_cast<u32x4_t*>(sink));
  return (int)hipGetLastError();
}

}  // namespace vq
