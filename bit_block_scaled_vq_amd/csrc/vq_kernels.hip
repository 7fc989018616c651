// HIP kernels (gfx950 / CDNA4) for the weight stream of the speculative-decoding
// verify pass: NVFP4 and FP8 E4M3 skinny GEMMs (M <= 32 rows) with a stream-K
// schedule and a fixed-order split-K reduction, plus the vocabulary-head argmax
// and greedy-accept epilogue, and two HBM probes.
//
// Method: "lithos-metal: per-layer megakernels for Qwen3.8-27B on an M5 Max ..."
// (sections "What one token costs the bus", "How DSpark is wired in",
// "Formats, and what runs where"); "144 tok/s needs 502 GB/s ..." (section
// "Why Apple silicon, and why not the M5": the verify rows form a real GEMM);
// "Beating Splash on an M5 Max ..." (sections "The kernels were not the gap":
// split-K on narrow projections; "What actually moved the needle": acceptance on
// the GPU).
//
// Design (MI355X-first, not the pages' Metal tiles):
//  * Every wave is an independent stream-K worker. The work space is
//    (tile, k-iteration); a tile is 2 x 32 weight rows, an iteration is 64 K.
//    Worker w owns iterations [w*W/P, (w+1)*W/P), so all workers carry the same
//    number of bytes and a GEMM has no tail wave. A tile split between workers
//    is reduced by its last-arriving piece, in worker order (deterministic).
//  * Weights stream straight from HBM into VGPRs with 16-byte non-temporal
//    loads, several iterations in flight per wave.
//  * The matrix unit is v_mfma_f32_32x32x16_bf16 with X as the A operand (rows
//    = verify rows, padded to 32) and the decoded weights as B (32 columns).
//    Its K of 16 is exactly one NVFP4 scale block, so each MFMA produces the
//    unscaled block partial of 32 columns and the E4M3 block scale is applied
//    after it with one fp32 FMA per useful accumulator. gfx950's packed fp4 ->
//    bf16 convert only honours the exponent of its scale operand, so the scale
//    cannot be folded into the decode; doing it after the MFMA costs about one
//    VALU op per eight weights at M = 8.
//  * Lanes load contiguous 16 bytes (32 codes = 2 blocks) of a row; one
//    v_permlane32_swap per register pair regroups them so the two lanes that
//    feed one MFMA column hold the two halves of the same block.
//  * E2M1 and E4M3 decode use the hardware converts with a unit scale; both
//    are exact in bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_internal.h"

namespace vq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ u32x4_t ld16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ uint32_t ld4_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

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

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void* y, int f32, size_t idx, float v) {
  if (f32)
    reinterpret_cast<float*>(y)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
}

// Monotone 64-bit argmax key: (orderable fp32 << 32) | (~index). Larger key =
// larger value, and on equal values the lower index. NaN -> 0 (never wins);
// -0 is treated as +0. 0 also means "no candidate".
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  if (v != v) return 0ull;
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)k << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ float key_value(unsigned long long key) {
  uint32_t k = (uint32_t)(key >> 32);
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return key ? __uint_as_float(u) : __builtin_nanf("");
}

__device__ __forceinline__ int64_t worker_start(int64_t w, int64_t total, int64_t workers) {
  return w * total / workers;
}
// The worker whose range contains iteration `it`.
__device__ __forceinline__ int64_t worker_of(int64_t it, int64_t total, int64_t workers) {
  return ((it + 1) * workers - 1) / total;
}

// ---------------------------------------------------------- per-iteration data

template <int FMT>
struct Buf;

template <>
struct Buf<FMT_NVFP4> {
  u32x4_t c[kNT];   // 16 code bytes per sub-tile row
  uint32_t s[kNT];  // 4 block scales per sub-tile row
  u32x4_t xa[4];    // X fragments of the 4 blocks (8 bf16 each)
};

template <>
struct Buf<FMT_FP8> {
  u32x4_t c[kNT][2];  // 2 x 16 weight bytes per sub-tile row
  u32x4_t xa[4];
};

// Weight row of sub-tile t of tile `tile` for the lane's column n.
template <int EPI>
__device__ __forceinline__ int weight_row(const GemmParams& p, int tile, int t, int n) {
  if (EPI == EPI_SILU) {
    int col = tile * kSubRows + n;
    col = col < p.N ? col : p.N - 1;
    return col + t * p.N;
  } else {
    int row = tile * (kSubRows * kNT) + t * kSubRows + n;
    return row < p.N ? row : p.N - 1;
  }
}

template <int FMT, int EPI>
__device__ __forceinline__ void load_iter(Buf<FMT>& b, const GemmParams& p, int tile, int kit,
                                          int n, int g, bool xrow, int m) {
  const size_t K = (size_t)p.K;
  if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const size_t row = (size_t)weight_row<EPI>(p, tile, t, n);
      b.c[t] = ld16_stream(p.codes + row * (K / 2) + (size_t)kit * 32 + g * 16);
      b.s[t] = ld4_stream(p.scales + row * (K / 16) + (size_t)kit * 4);
    }
    if (xrow) {
      const uint16_t* xr = p.x + (size_t)m * K + (size_t)kit * kIterK + g * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) b.xa[j] = ld16(xr + 16 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) b.xa[j] = u32x4_t{0u, 0u, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const size_t row = (size_t)weight_row<EPI>(p, tile, t, n);
      const uint8_t* base = p.codes + row * K + (size_t)kit * kIterK + g * 16;
      b.c[t][0] = ld16_stream(base);
      b.c[t][1] = ld16_stream(base + 32);
    }
    if (xrow) {
      const uint16_t* xr = p.x + (size_t)m * K + (size_t)kit * kIterK + g * 16;
      b.xa[0] = ld16(xr);
      b.xa[1] = ld16(xr + 8);
      b.xa[2] = ld16(xr + 32);
      b.xa[3] = ld16(xr + 40);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) b.xa[j] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

// Accumulators: NVFP4 keeps the scaled sums in plain VGPRs (the MFMA output is
// only a per-block temporary); FP8 accumulates inside the MFMA.
template <int FMT, int MB>
struct Acc;
template <int MB>
struct Acc<FMT_NVFP4, MB> {
  float v[kNT][4 * MB];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int r = 0; r < 4 * MB; ++r) v[t][r] = 0.0f;
  }
  __device__ __forceinline__ float get(int t, int r) const { return v[t][r]; }
};
template <int MB>
struct Acc<FMT_FP8, MB> {
  f32x16_t v[kNT];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int t = 0; t < kNT; ++t) v[t] = f32x16_t{};
  }
  __device__ __forceinline__ float get(int t, int r) const { return v[t][r]; }
};

template <int FMT, int MB>
__device__ __forceinline__ void compute_iter(const Buf<FMT>& b, Acc<FMT, MB>& acc) {
  if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      // Lanes 0-31 hold blocks 0,1 of this iteration, lanes 32-63 blocks 2,3
      // (each as two 8-code halves). The swap pairs half 0 (lanes 0-31) with
      // half 1 (lanes 32-63) of the same block.
      auto s02 = __builtin_amdgcn_permlane32_swap(b.c[t].x, b.c[t].y, false, false);
      auto s13 = __builtin_amdgcn_permlane32_swap(b.c[t].z, b.c[t].w, false, false);
      const uint32_t op[4] = {(uint32_t)s02[0], (uint32_t)s13[0], (uint32_t)s02[1], (uint32_t)s13[1]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t wv = dec_fp4x8(op[j]);
        const bf16x8_t xv = __builtin_bit_cast(bf16x8_t, b.xa[j]);
        const f32x16_t d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xv, wv, f32x16_t{}, 0, 0, 0);
        float sc;
        if (j == 0) sc = __builtin_amdgcn_cvt_f32_fp8(b.s[t], 0);
        else if (j == 1) sc = __builtin_amdgcn_cvt_f32_fp8(b.s[t], 1);
        else if (j == 2) sc = __builtin_amdgcn_cvt_f32_fp8(b.s[t], 2);
        else sc = __builtin_amdgcn_cvt_f32_fp8(b.s[t], 3);
#pragma unroll
        for (int r = 0; r < 4 * MB; ++r) acc.v[t][r] = __builtin_fmaf(sc, d[r], acc.v[t][r]);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const bf16x8_t w0 = dec_fp8x8(b.c[t][0].x, b.c[t][0].y);
      acc.v[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b.xa[0]), w0, acc.v[t], 0, 0, 0);
      const bf16x8_t w1 = dec_fp8x8(b.c[t][0].z, b.c[t][0].w);
      acc.v[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b.xa[1]), w1, acc.v[t], 0, 0, 0);
      const bf16x8_t w2 = dec_fp8x8(b.c[t][1].x, b.c[t][1].y);
      acc.v[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b.xa[2]), w2, acc.v[t], 0, 0, 0);
      const bf16x8_t w3 = dec_fp8x8(b.c[t][1].z, b.c[t][1].w);
      acc.v[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b.xa[3]), w3, acc.v[t], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------- epilogues

// Row of the output held by accumulator register r of a lane in half g.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Final step of the head: reduce the bucketed candidates, write argmax / max,
// run the greedy accept per lane and reset the workspace. One wave.
__device__ __noinline__ void head_final(const GemmParams& p, int lane) {
  __threadfence();
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

template <int EPI, int MB, typename GetF>
__device__ __forceinline__ void epilogue(const GemmParams& p, int tile, int lane, GetF get) {
  const int n = lane & 31, g = lane >> 5;
  const float sc = p.out_scale;
  if constexpr (EPI == EPI_NONE) {
#pragma unroll
    for (int r = 0; r < 4 * MB; ++r) {
      const int m = acc_row(r, g);
      if (m < p.M) {
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          const int col = tile * (kSubRows * kNT) + t * kSubRows + n;
          if (col < p.N) store_out(p.y, p.y_f32, (size_t)m * p.N + col, get(t, r) * sc);
        }
      }
    }
  } else if constexpr (EPI == EPI_SILU) {
#pragma unroll
    for (int r = 0; r < 4 * MB; ++r) {
      const int m = acc_row(r, g);
      const int col = tile * kSubRows + n;
      if (m < p.M && col < p.N) {
        const float gv = get(0, r) * sc;
        const float uv = get(1, r) * sc;
        const float h = gv / (1.0f + expf(-gv)) * uv;
        store_out(p.y, p.y_f32, (size_t)m * p.N + col, h);
      }
    }
  } else {
    // Vocabulary head: optional logits, per-row candidate over this tile.
#pragma unroll
    for (int r = 0; r < 4 * MB; ++r) {
      const int m = acc_row(r, g);
      unsigned long long best = 0ull;
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int col = tile * (kSubRows * kNT) + t * kSubRows + n;
        const float v = get(t, r) * sc;
        if (m < p.M && col < p.N) {
          if (p.y) store_out(p.y, p.y_f32, (size_t)m * p.N + col, v);
          const unsigned long long k = argmax_key(v, (uint32_t)col);
          best = k > best ? k : best;
        }
      }
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off);
        best = o > best ? o : best;
      }
      if (n == 0 && m < p.M && best != 0ull)
        atomicMax(&p.best[(tile % kBuckets) * kMaxRows + m], best);
    }
    __threadfence();
    uint32_t old = 0;
    if (lane == 0) old = atomicAdd(p.done, 1u);
    old = __shfl(old, 0);
    if (old == (uint32_t)(p.tiles - 1)) head_final(p, lane);
  }
}

// End of a piece of tile `tile` held in `acc`. A tile covered by one worker is
// finished directly; otherwise the piece is parked in its slot and the last
// piece to arrive sums all pieces in worker order and finishes the tile.
template <int FMT, int EPI, int MB>
__device__ __forceinline__ void finish_piece(const GemmParams& p, int tile, bool full, int64_t w,
                                             bool first, const Acc<FMT, MB>& acc, int lane) {
  if (full) {
    epilogue<EPI, MB>(p, tile, lane, [&](int t, int r) { return acc.get(t, r); });
    return;
  }
  const int64_t slot = 2 * w + (first ? 0 : 1);
  float* dst = p.partials + slot * kSlotFloats;
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int r = 0; r < 4 * MB; ++r) dst[(t * 16 + r) * 64 + lane] = acc.get(t, r);
  __threadfence();
  uint32_t old = 0;
  if (lane == 0) old = atomicAdd(&p.counters[tile], 1u);
  old = __shfl(old, 0);
  const int64_t I = p.iters;
  const int64_t w0 = worker_of((int64_t)tile * I, p.total, p.workers);
  const int64_t w1 = worker_of((int64_t)(tile + 1) * I - 1, p.total, p.workers);
  if (old != (uint32_t)(w1 - w0)) return;
  __threadfence();
  if (lane == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float sum[kNT][4 * MB];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int r = 0; r < 4 * MB; ++r) sum[t][r] = 0.0f;
  for (int64_t v = w0; v <= w1; ++v) {
    const bool vfirst = (worker_start(v, p.total, p.workers) / I) == tile;
    const float* src = p.partials + (2 * v + (vfirst ? 0 : 1)) * kSlotFloats;
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int r = 0; r < 4 * MB; ++r) sum[t][r] += src[(t * 16 + r) * 64 + lane];
  }
  epilogue<EPI, MB>(p, tile, lane, [&](int t, int r) { return sum[t][r]; });
}

// --------------------------------------------------------------- main kernel

template <int FMT>
struct PipeDepth {
  static constexpr int value = 4;
};

// M <= 8 fits two waves per SIMD without spills; larger M keeps one wave per
// SIMD so the extra accumulators stay in registers (AGPRs included).
template <int FMT, int EPI, int MB>
__global__ __launch_bounds__(256, MB == 1 ? 2 : 1) void vq_gemm_kernel(GemmParams p) {
  constexpr int PD = PipeDepth<FMT>::value;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= p.workers) return;
  const int64_t s = worker_start(w, p.total, p.workers);
  const int64_t e = worker_start(w + 1, p.total, p.workers);
  if (s >= e) return;
  const int n = lane & 31, g = lane >> 5;
  const int m = n;  // A-operand row of this lane
  const bool xrow = m < p.M;
  const int I = p.iters;

  Buf<FMT> buf[PD];
  int ltile = (int)(s / I), lkit = (int)(s % I);
  int64_t lit = s;
#pragma unroll
  for (int q = 0; q < PD; ++q) {
    if (lit < e) {
      load_iter<FMT, EPI>(buf[q], p, ltile, lkit, n, g, xrow, m);
      ++lit;
      if (++lkit == I) { lkit = 0; ++ltile; }
    }
  }

  int ctile = (int)(s / I), ckit = (int)(s % I);
  const int first_tile = ctile;
  int pstart = ckit;
  int64_t cit = s;
  Acc<FMT, MB> acc;
  acc.zero();
  while (cit < e) {
#pragma unroll
    for (int q = 0; q < PD; ++q) {
      if (cit < e) {
        compute_iter<FMT, MB>(buf[q], acc);
        if (lit < e) {
          load_iter<FMT, EPI>(buf[q], p, ltile, lkit, n, g, xrow, m);
          ++lit;
          if (++lkit == I) { lkit = 0; ++ltile; }
        }
        ++cit;
        if (++ckit == I) {
          finish_piece<FMT, EPI, MB>(p, ctile, pstart == 0, w, ctile == first_tile, acc, lane);
          acc.zero();
          ckit = 0;
          pstart = 0;
          ++ctile;
        }
      }
    }
  }
  if (ckit != 0) finish_piece<FMT, EPI, MB>(p, ctile, false, w, ctile == first_tile, acc, lane);
}

// ------------------------------------------------------------------- probes

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t st = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += st) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4_t* __restrict__ src, size_t n, u32x4_t* sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t st = (size_t)gridDim.x * blockDim.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i < n; i += st) acc ^= __builtin_nontemporal_load(src + i);
  // Never true for the probe's data in practice, but the compiler cannot know.
  if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u) sink[0] = acc;
}

// ---------------------------------------------------------------- launchers

template <int FMT, int EPI>
static int launch_mb(const GemmParams& p, hipStream_t st) {
  const int mb = (p.M + 7) / 8;
  const dim3 grid((unsigned)((p.workers + 3) / 4)), block(256);
  switch (mb) {
    case 1: hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 3>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((vq_gemm_kernel<FMT, EPI, 4>), grid, block, 0, st, p); break;
  }
  return (int)hipGetLastError();
}

int launch_gemm(int fmt, int epi, const GemmParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (fmt == FMT_NVFP4) {
    if (epi == EPI_NONE) return launch_mb<FMT_NVFP4, EPI_NONE>(p, st);
    if (epi == EPI_SILU) return launch_mb<FMT_NVFP4, EPI_SILU>(p, st);
    return launch_mb<FMT_NVFP4, EPI_ARGMAX>(p, st);
  }
  return launch_mb<FMT_FP8, EPI_NONE>(p, st);
}

int launch_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(probe_copy_kernel, dim3(2048), dim3(256), 0, st,
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
