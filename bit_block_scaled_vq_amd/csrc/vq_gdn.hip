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
//    of one value head; its 4 waves split the 128 key rows, 32 each; within a
//    wave lane l holds column l >> 1 and rows (l & 1) * 16 + r, r < 16, so a
//    state load instruction reads two whole 128-byte row segments.
//  * The rows' keys, queries, values and gates are staged in LDS once, behind
//    one barrier, so no row waits on a global load.
//  * Per row t: u_j = the lane's 16 products (two interleaved sums), a DPP add
//    with the lane holding the other 16 rows of that wave, then the 4 waves'
//    sums through a double-buffered LDS slot (one barrier per row), added in
//    wave order by every lane, so all lanes hold the same bits. Then
//    S[i][j] = a S[i][j] + k_i * (b (v_j - a u_j)); the output partials
//    q^T S[:, j] go to LDS and are summed in wave order after the last row.
//  * The split of the rows over waves and lanes is fixed, so the result of a
//    scan does not depend on how many entries a call carries: a commit
//    re-scan of c rows is bitwise the state a verify of those c rows wrote.
//  * The state is streamed with non-temporal loads and stores (read once and
//    written once per pass).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_internal.h"

namespace vq {

namespace {

constexpr int kWaves = 4;                       // waves per workgroup (row split)
constexpr int kRowsPerWave = kGdnDk / kWaves;   // 32
constexpr int kRowsPerLane = kRowsPerWave / 2;  // 16
constexpr int kCols = 32;                       // state columns per workgroup
constexpr int kChunks = kGdnDv / kCols;         // 4 workgroups per value head

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// value of the lane l ^ 1 (DPP quad permutation [1, 0, 3, 2])
__device__ __forceinline__ float swap_pair(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}

__global__ __launch_bounds__(256) void gdn_scan_kernel(GdnParams p) {
  __shared__ f32x4_t k_s[kGdnMaxT][kGdnDk / 4];
  __shared__ f32x4_t q_s[kGdnMaxT][kGdnDk / 4];
  __shared__ float v_s[kGdnMaxT][kCols];
  __shared__ float a_s[kGdnMaxT], b_s[kGdnMaxT];
  __shared__ float lds_u[2][kWaves][kCols];
  __shared__ float lds_o[kGdnMaxT][kWaves][kCols];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int chunk = blockIdx.x % kChunks;
  const int h = (blockIdx.x / kChunks) % p.H;
  const int e = blockIdx.x / (kChunks * p.H);
  const int kh = h / (p.H / p.Hk);
  const int j = lane >> 1;
  const int col = chunk * kCols + j;
  const int row0 = w * kRowsPerWave + (lane & 1) * kRowsPerLane;

  int n = p.T;
  if (p.count) {
    // commit: the lane's accepted rows, clamped to [0, T]; a fully accepted
    // entry keeps the verify's output slot as it is
    const int c = p.count[e % p.lanes];
    n = c < 0 ? 0 : (c > p.T ? p.T : c);
    if (n == p.T) return;  // uniform over the workgroup
  }
  const size_t sbase = ((size_t)e * p.H + h) * kGdnDk * kGdnDv;
  const float* sin = p.state_in + sbase + (size_t)row0 * kGdnDv + col;
  float S[kRowsPerLane];
#pragma unroll
  for (int r = 0; r < kRowsPerLane; ++r) S[r] = __builtin_nontemporal_load(sin + (size_t)r * kGdnDv);

  // stage the n rows' inputs of this head and chunk: every global load is
  // issued before the first LDS write, so staging costs one round trip (and
  // overlaps the state loads above)
  const bool want_o = p.o != nullptr;
  constexpr int kThreads = 64 * kWaves;
  constexpr int kQKSlots = kGdnMaxT * (kGdnDk / 4) / kThreads;  // float4s per thread
  constexpr int kVSlots = kGdnMaxT * kCols / kThreads;          // values per thread
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

  for (int t = 0; t < n; ++t) {
    float kr[kRowsPerLane];
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r += 4) {
      const f32x4_t k4 = k_s[t][(row0 + r) / 4];
      kr[r] = k4.x; kr[r + 1] = k4.y; kr[r + 2] = k4.z; kr[r + 3] = k4.w;
    }
    float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r += 2) {
      u0 = __builtin_fmaf(kr[r], S[r], u0);
      u1 = __builtin_fmaf(kr[r + 1], S[r + 1], u1);
    }
    float u = u0 + u1;
    u += swap_pair(u);
    if ((lane & 1) == 0) lds_u[t & 1][w][j] = u;
    __syncthreads();
    u = lds_u[t & 1][0][j];
#pragma unroll
    for (int w2 = 1; w2 < kWaves; ++w2) u += lds_u[t & 1][w2][j];
    const float at = a_s[t];
    const float wj = b_s[t] * (v_s[t][j] - at * u);
#pragma unroll
    for (int r = 0; r < kRowsPerLane; ++r) S[r] = __builtin_fmaf(kr[r], wj, at * S[r]);
    if (want_o) {
      float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
      for (int r = 0; r < kRowsPerLane; r += 4) {
        const f32x4_t q4 = q_s[t][(row0 + r) / 4];
        o0 = __builtin_fmaf(q4.x, S[r], o0);
        o1 = __builtin_fmaf(q4.y, S[r + 1], o1);
        o0 = __builtin_fmaf(q4.z, S[r + 2], o0);
        o1 = __builtin_fmaf(q4.w, S[r + 3], o1);
      }
      float op = o0 + o1;
      op += swap_pair(op);
      if ((lane & 1) == 0) lds_o[t][w][j] = op;
    }
  }
  float* sout = p.state_out + sbase + (size_t)row0 * kGdnDv + col;
#pragma unroll
  for (int r = 0; r < kRowsPerLane; ++r) __builtin_nontemporal_store(S[r], sout + (size_t)r * kGdnDv);
  if (want_o && n > 0) {
    __syncthreads();
    // one thread per (row, column): the wave partials in wave order
    for (int idx = threadIdx.x; idx < n * kCols; idx += blockDim.x) {
      const int t = idx / kCols, jj = idx % kCols;
      float s = lds_o[t][0][jj];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) s += lds_o[t][w2][jj];
      p.o[(((size_t)e * p.T + t) * p.H + h) * kGdnDv + chunk * kCols + jj] = s;
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
