// HIP kernel (gfx950) for the Gated DeltaNet state stream of the verify pass:
// the gated delta rule over a lane's verify rows, read from one parity slot of
// the fp32 state and written out of place to the other, and the commit re-scan
// of the accepted rows from the slot the verify read.
//
// Method: "Beating Splash on an M5 Max ..." (section "What actually moved the
// needle": double-buffered GatedDeltaNet state, partial rejections re-scan the
// committed rows from the intact parity); "lithos-metal ..." (section "What one
// token costs the bus": fp32 state (v_heads, dk, dv) = (48, 128, 128) per
// layer, read and written once per pass; section "How DSpark is wired in":
// verify reads one slot and writes the other, the commit pass recomputes the
// recurrence over the committed tokens only). The recurrence is the gated
// delta rule of Yang, Kautz and Hatamizadeh, "Gated Delta Networks: Improving
// Mamba2 with Delta Rule" (ICLR 2025), per value head in the (dk, dv) layout:
//   S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
//
// Design (MI355X-first):
//  * Columns of S are independent: column j only needs u_j = k^T S[:, j] and
//    v_j. A workgroup owns 32 columns (one 128-byte line of every state row)
//    of one value head, 4 workgroups per head. It reads its 128 x 32 chunk
//    with whole 128-byte row segments per wave instruction (non-temporal:
//    the state is read once and written once per pass) into a padded LDS
//    tile, together with the rows' keys, queries, values and gates, behind
//    one barrier.
//  * Each column's 128 rows are then held by one 16-lane DPP row of a wave
//    (lane 16c + g: column c of the wave's 4, rows 8g .. 8g + 7), 8 waves per
//    workgroup. Per row t: u_j = the lane's 8 products (two interleaved
//    sums) summed over the 16 lanes by a DPP butterfly (pairs l ^ 1, l ^ 2,
//    then the half-row and row mirrors), so every lane of the column holds
//    the same bits; then S[i][j] = a S[i][j] + k_i (b (v_j - a u_j)), and the
//    output q^T S[:, j] by the same butterfly. A row step has no LDS exchange
//    and no barrier.
//  * The updated chunk goes back through the LDS tile and out with whole row
//    segments per instruction; the outputs leave from LDS once per call.
//  * The split of the rows over lanes is fixed, so the result of a scan does
//    not depend on how many entries a call carries: a commit re-scan of c
//    rows is bitwise the state a verify of those c rows wrote.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_internal.h"

namespace vq {

namespace {

constexpr int kCols = 32;                       // state columns per workgroup
constexpr int kChunks = kGdnDv / kCols;         // 4 workgroups per value head
constexpr int kColsPerWave = 4;                 // one column per 16-lane DPP row
constexpr int kWaves = kCols / kColsPerWave;    // 8
constexpr int kThreads = 64 * kWaves;           // 512
constexpr int kGroupRows = kGdnDk / 16;         // 8 state rows per lane
constexpr int kPitch = kCols + 1;               // padded LDS row of the state tile

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row by a butterfly (lane pairs l ^ 1, l ^ 2,
// then the half-row and row mirrors): every lane ends with the same bits.
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// this lane's 8 rows of a staged 128-vector
__device__ __forceinline__ void group_rows(float (&dst)[kGroupRows], const f32x4_t* src, int g) {
  const f32x4_t a = src[2 * g], b = src[2 * g + 1];
  dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
  dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
}

__device__ __forceinline__ float group_dot(const float (&x)[kGroupRows], const float (&S)[kGroupRows]) {
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int r = 0; r < kGroupRows; r += 2) {
    a0 = __builtin_fmaf(x[r], S[r], a0);
    a1 = __builtin_fmaf(x[r + 1], S[r + 1], a1);
  }
  return a0 + a1;
}

__global__ __launch_bounds__(kThreads) void gdn_scan_kernel(GdnParams p) {
  __shared__ float s_tile[kGdnDk * kPitch];  // the workgroup's 128 x 32 state chunk
  __shared__ f32x4_t k_s[kGdnMaxT][kGdnDk / 4];
  __shared__ f32x4_t q_s[kGdnMaxT][kGdnDk / 4];
  __shared__ float v_s[kGdnMaxT][kCols];
  __shared__ float a_s[kGdnMaxT], b_s[kGdnMaxT];
  __shared__ float o_s[kGdnMaxT][kCols];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int chunk = blockIdx.x % kChunks;
  const int h = (blockIdx.x / kChunks) % p.H;
  const int e = blockIdx.x / (kChunks * p.H);
  const int kh = h / (p.H / p.Hk);
  const int jc = w * kColsPerWave + (lane >> 4);  // this lane's column in the chunk
  const int g = lane & 15;                          // its row group: rows 8g .. 8g + 7

  int n = p.T;
  if (p.count) {
    // commit: the lane's accepted rows, clamped to [0, T]; a fully accepted
    // entry keeps the verify's output slot as it is
    const int c = p.count[e % p.lanes];
    n = c < 0 ? 0 : (c > p.T ? p.T : c);
    if (n == p.T) return;  // uniform over the workgroup
  }
  // state chunk: 128 rows x 128 bytes, two 16-byte pieces per thread, each
  // wave instruction covering whole 128-byte row segments
  const size_t sbase = ((size_t)e * p.H + h) * kGdnDk * kGdnDv + chunk * kCols;
  constexpr int kPieces = kGdnDk * kCols / 4 / kThreads;  // 2
  f32x4_t sreg[kPieces];
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int i = threadIdx.x + u * kThreads;
    const int row = i >> 3, c4 = (i & 7) * 4;
    sreg[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p.state_in + sbase + (size_t)row * kGdnDv + c4));
  }

  // the rows' inputs of this head and chunk
  const bool want_o = p.o != nullptr;
  constexpr int kQKSlots = (kGdnMaxT * (kGdnDk / 4) + kThreads - 1) / kThreads;
  constexpr int kVSlots = (kGdnMaxT * kCols + kThreads - 1) / kThreads;
  f32x4_t kreg[kQKSlots], qreg[kQKSlots];
  float vreg[kVSlots];
  float areg = 0.0f, breg = 0.0f;
#pragma unroll
  for (int u = 0; u < kQKSlots; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < n * (kGdnDk / 4)) {
      const int t = i / (kGdnDk / 4), c4 = i % (kGdnDk / 4);
      const size_t src = (((size_t)e * p.T + t) * p.Hk + kh) * kGdnDk + 4 * c4;
      kreg[u] = *reinterpret_cast<const f32x4_t*>(p.k + src);
      if (want_o) qreg[u] = *reinterpret_cast<const f32x4_t*>(p.q + src);
    }
  }
#pragma unroll
  for (int u = 0; u < kVSlots; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < n * kCols) {
      const int t = i / kCols, c = i % kCols;
      vreg[u] = p.v[(((size_t)e * p.T + t) * p.H + h) * kGdnDv + chunk * kCols + c];
    }
  }
  if (threadIdx.x < n) {
    const size_t et = (size_t)e * p.T + threadIdx.x;
    areg = p.a[et * p.H + h];
    breg = p.b[et * p.H + h];
  }
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int i = threadIdx.x + u * kThreads;
    float* d = s_tile + (i >> 3) * kPitch + (i & 7) * 4;
    d[0] = sreg[u].x; d[1] = sreg[u].y; d[2] = sreg[u].z; d[3] = sreg[u].w;
  }
#pragma unroll
  for (int u = 0; u < kQKSlots; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < n * (kGdnDk / 4)) {
      k_s[i / (kGdnDk / 4)][i % (kGdnDk / 4)] = kreg[u];
      if (want_o) q_s[i / (kGdnDk / 4)][i % (kGdnDk / 4)] = qreg[u];
    }
  }
#pragma unroll
  for (int u = 0; u < kVSlots; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < n * kCols) v_s[i / kCols][i % kCols] = vreg[u];
  }
  if (threadIdx.x < n) {
    a_s[threadIdx.x] = areg;
    b_s[threadIdx.x] = breg;
  }
  __syncthreads();

  float S[kGroupRows];
#pragma unroll
  for (int r = 0; r < kGroupRows; ++r) S[r] = s_tile[(8 * g + r) * kPitch + jc];

  // the rows: each column's 128 rows live in one 16-lane DPP row, so a row
  // step needs no LDS exchange and no barrier
  for (int t = 0; t < n; ++t) {
    float kr[kGroupRows];
    group_rows(kr, k_s[t], g);
    const float u = row_sum(group_dot(kr, S));
    const float at = a_s[t];
    const float wj = b_s[t] * (v_s[t][jc] - at * u);
#pragma unroll
    for (int r = 0; r < kGroupRows; ++r) S[r] = __builtin_fmaf(kr[r], wj, at * S[r]);
    if (want_o) {
      float qr[kGroupRows];
      group_rows(qr, q_s[t], g);
      const float o = row_sum(group_dot(qr, S));
      if (g == 0) o_s[t][jc] = o;
    }
  }

#pragma unroll
  for (int r = 0; r < kGroupRows; ++r) s_tile[(8 * g + r) * kPitch + jc] = S[r];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int i = threadIdx.x + u * kThreads;
    const float* d = s_tile + (i >> 3) * kPitch + (i & 7) * 4;
    const f32x4_t v = {d[0], d[1], d[2], d[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p.state_out + sbase + (size_t)(i >> 3) * kGdnDv + (i & 7) * 4));
  }
  if (want_o) {
    for (int idx = threadIdx.x; idx < n * kCols; idx += kThreads) {
      const int t = idx / kCols, jj = idx % kCols;
      p.o[(((size_t)e * p.T + t) * p.H + h) * kGdnDv + chunk * kCols + jj] = o_s[t][jj];
    }
  }
}

}  // namespace

int launch_gdn(const GdnParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t groups = (int64_t)p.B * p.H * kChunks;
  hipLaunchKernelGGL(gdn_scan_kernel, dim3((unsigned)groups), dim3(64 * kWaves), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace vq

