// HIP kernels (gfx950) of the sampled verify: over the fp32 verify logits,
// each row's target distribution (temperature over its top_k <= 32 logits,
// truncated by top_p, renormalised), a draw from it, and the accept scan of
// each lane -- the point-mass rule (the draft token is accepted when it equals
// the target's draw) or the speculative-sampling rule (accept when
// u * q(d) < p(d), else draw from max(p - q, 0)).
//
// Method: "144 tok/s needs 502 GB/s, and Apple sells two M5 Max chips",
// section "Exact, up to top-32" (the truncated distribution, the accept test
// and the residual draw, 32 target and 16 draft candidates per row);
// "Beating Splash on an M5 Max ...", section "What actually moved the needle"
// (top-k, top-p, sampling and acceptance in one pass on the GPU, writing a
// small result block); "lithos-metal ...", section "How DSpark is wired in"
// (the point-mass case).
//
// Design:
//  * Candidates are the monotone 64-bit keys of the GEMM's argmax (value bits,
//    then the lower token id), so the order is total and ties break by id.
//  * Top-32 of a row in two launches. A chunk workgroup (8192 logits, 32 per
//    lane) reduces each wave's 2048 logits to its 32 largest keys; a row
//    workgroup merges the chunks' lists. Inside a wave: the 32nd largest of
//    the 64 lane maxima bounds the wave's 32nd largest key from below, so
//    only keys at or above it can matter; they are fed to a running list, one
//    per lane per round (a 64-key bitonic sort across lanes and a bitonic
//    merge with the list). Random logits take one or two rounds.
//  * The distribution, the draw and the accept scan run on one wave with the
//    32 candidates in lanes 0..31; sums and prefix sums use a fixed shuffle
//    order, so results do not depend on timing.
//  * The rows of a lane meet through agent-scope atomics: each row workgroup
//    publishes its candidates, then counts itself in; the last row of a lane
//    runs the scan and resets the count.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_internal.h"
#include "vq_keys.h"

namespace vq {

typedef unsigned long long u64;

__device__ __forceinline__ u64 kmax(u64 a, u64 b) { return a > b ? a : b; }
__device__ __forceinline__ u64 kmin(u64 a, u64 b) { return a < b ? a : b; }

// Bitonic sort of one key per lane across the wave, descending in lane order.
__device__ __forceinline__ u64 wave_sort_desc(u64 v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const u64 o = __shfl_xor(v, j);
      const bool desc = (lane & k) == 0;
      const bool low = (lane & j) == 0;
      v = (low == desc) ? kmax(v, o) : kmin(v, o);
    }
  }
  return v;
}

// `list`: a descending list in lanes 0..31; `s`: 64 keys sorted descending.
// Returns the 32 largest of list and s[0..31], descending in lanes 0..31
// (lanes 32..63: the rest, descending). The list followed by s[31..0] is a
// bitonic sequence; one bitonic merge sorts it.
__device__ __forceinline__ u64 merge_top32(u64 list, u64 s, int lane) {
  const u64 rev = __shfl(s, 63 - lane);
  u64 x = lane < 32 ? list : rev;
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    const u64 o = __shfl_xor(x, j);
    x = (lane & j) == 0 ? kmax(x, o) : kmin(x, o);
  }
  return x;
}

// The wave's 32 largest keys among N per lane (0 = no key), descending in
// lanes 0..31; lanes 32..63 return 0.
template <int N>
__device__ __forceinline__ u64 wave_top32(const u64 (&k)[N], int lane) {
  static_assert(N <= 64, "one survivor bit per key");
  u64 mx = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) mx = kmax(mx, k[i]);
  // The lane maxima are 64 of the wave's keys, so their 32nd largest is at
  // most the wave's 32nd largest: every key of the answer is >= theta.
  const u64 theta = __shfl(wave_sort_desc(mx, lane), 31);
  u64 live = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (k[i] != 0ull && k[i] >= theta) live |= 1ull << i;
  u64 list = 0;
  while (__ballot(live != 0ull)) {
    u64 c = 0;
    if (live) {
      const int b = __builtin_ctzll(live);
      live &= live - 1;
#pragma unroll
      for (int i = 0; i < N; ++i) c = i == b ? k[i] : c;
    }
    list = merge_top32(list, wave_sort_desc(c, lane), lane);
  }
  return lane < 32 ? list : 0ull;
}

// Wave sum and inclusive prefix sum, fixed order (lanes 0..31 carry values).
__device__ __forceinline__ float wave_sum32(float v) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 32);
  return v;
}
__device__ __forceinline__ float wave_scan32(float v, int lane) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const float o = __shfl_up(v, off, 32);
    if ((lane & 31) >= off) v += o;
  }
  return v;
}

// First lane i < count with cum_i > t (cum ascending over lanes), else
// count - 1.
__device__ __forceinline__ int first_above(float cum, float t, int lane, int count) {
  const u64 m = __ballot(lane < count && cum > t);
  return m ? __builtin_ctzll(m) : count - 1;
}

// ------------------------------------------------------------ chunk top-32

__global__ __launch_bounds__(256) void sample_chunk_kernel(SampleParams p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x, m = blockIdx.y;
  const float* row = p.logits + (size_t)m * p.V;
  const int64_t base = (int64_t)c * kSampleChunk + w * (kSampleChunk / 4);
  u64 k[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t idx = base + i * 64 + lane;
    k[i] = idx < p.V ? argmax_key(row[idx], (uint32_t)idx) : 0ull;
  }
  const u64 top = wave_top32<32>(k, lane);
  if (lane < 32) p.cand[(((size_t)m * p.chunks + c) * 4 + w) * 32 + lane] = top;
}

// ------------------------------------------------- row distribution + scan

// Accept scan of lane l (one wave; every row of the lane is published).
__device__ void lane_scan(const SampleParams& p, int l, int lane) {
  const int R = p.R;
  auto ld_i = [](const int32_t* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto ld_f = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  int acc_len = R;
  int commit = -1;  // lane j < R holds committed token j
  int j = 0;
  for (; j < R - 1; ++j) {
    const int m = l * R + j;
    const int count = ld_i(&p.row_meta[2 * m]);
    const int tok = ld_i(&p.row_meta[2 * m + 1]);
    const int d = p.draft[l * (R - 1) + j];
    if (count == 0) break;  // no distribution: the scan stops, committing nothing here
    if (!p.q_ids) {         // point-mass: the draft must equal the target's draw
      if (tok == d) {
        if (lane == j) commit = d;
        continue;
      }
      if (lane == j) commit = tok;
      break;
    }
    const int id = lane < count ? ld_i(&p.row_ids[m * 32 + lane]) : -1;
    const float pr = lane < count ? ld_f(&p.row_probs[m * 32 + lane]) : 0.0f;
    const int qbase = (l * (R - 1) + j) * kDraftCands;
    const int qid = lane < kDraftCands ? p.q_ids[qbase + lane] : -1;
    const float qp = lane < kDraftCands ? p.q_probs[qbase + lane] : 0.0f;
    const u64 pm = __ballot(lane < count && id == d);
    const float pd = pm ? __shfl(pr, __builtin_ctzll(pm)) : 0.0f;
    const u64 qm = __ballot(lane < kDraftCands && qid >= 0 && qid == d);
    const float qd = qm ? __shfl(qp, __builtin_ctzll(qm)) : 0.0f;
    if (p.u_accept[m] * qd < pd) {
      if (lane == j) commit = d;
      continue;
    }
    // rejected: draw from max(p - q, 0) over the kept candidates
    float qi = 0.0f;
    bool found = false;
#pragma unroll
    for (int e = 0; e < kDraftCands; ++e) {
      const int qe = __shfl(qid, e);
      const float pe = __shfl(qp, e);
      if (!found && qe >= 0 && qe == id) {
        qi = pe;
        found = true;
      }
    }
    const float r = lane < count ? fmaxf(pr - qi, 0.0f) : 0.0f;
    const float rs = wave_sum32(r);
    int pick;
    if (rs > 0.0f) {
      pick = __shfl(id, first_above(wave_scan32(r, lane), p.u_draw[m] * rs, lane, count));
    } else {
      pick = tok;  // no residual mass: the draw from p itself
    }
    if (lane == j) commit = pick;
    break;
  }
  if (j == R - 1) {  // every draft accepted: the bonus is the last row's draw
    const int tok = ld_i(&p.row_meta[2 * (l * R + j) + 1]);
    if (lane == j) commit = tok;
  }
  acc_len = j + 1;
  if (lane == 0) p.accept_len_out[l] = acc_len;
  if (p.commit_out && lane < R) p.commit_out[l * R + lane] = lane < acc_len ? commit : -1;
}

template <int NL>
__global__ __launch_bounds__(256) void sample_row_kernel(SampleParams p) {
  __shared__ u64 lists[4][32];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = blockIdx.x;
  // wave w merges chunk lists [w*C, (w+1)*C) of this row: C * 32 keys
  const int n = p.chunks * 32;
  const u64* src = p.cand + ((size_t)m * p.chunks * 4 + (size_t)w * p.chunks) * 32;
  u64 k[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int idx = i * 64 + lane;
    k[i] = idx < n ? src[idx] : 0ull;
  }
  const u64 top = wave_top32<NL>(k, lane);
  if (lane < 32) lists[w][lane] = top;
  __syncthreads();
  if (w != 0) return;

  u64 list = lane < 32 ? lists[0][lane] : 0ull;
#pragma unroll
  for (int v = 1; v < 4; ++v) list = merge_top32(list, lane < 32 ? lists[v][lane] : 0ull, lane);

  // The truncated target distribution over the first top_k candidates.
  const bool cand = lane < p.top_k && list != 0ull;
  const float z = cand ? key_value(list) : 0.0f;
  const float z0 = __shfl(z, 0);
  const bool has0 = __shfl((int)cand, 0) != 0;
  int count = 0, tok = -1, id = cand ? key_index(list) : -1;
  float prob = 0.0f;
  if (has0 && __builtin_isfinite(z0)) {
    const float wgt = cand ? expf((z - z0) / p.temperature) : 0.0f;
    const float cum = wave_scan32(wgt, lane);
    const float total = __shfl(cum, 31);
    // shortest prefix reaching top_p of the mass, then without zero weights
    const u64 reach = __ballot(cand && cum >= p.top_p * total);
    count = reach ? __builtin_ctzll(reach) + 1 : (int)__popcll(__ballot(cand));
    const u64 pos = __ballot(lane < count && wgt > 0.0f);
    count = pos ? 64 - __builtin_clzll(pos) : 1;
    const float kept = __shfl(cum, count - 1);
    prob = lane < count ? wgt / kept : 0.0f;
    tok = __shfl(id, first_above(cum, p.u_draw[m] * kept, lane, count));
  }
  if (lane >= count) {
    id = -1;
    prob = 0.0f;
  }
  if (p.token_out && lane == 0) p.token_out[m] = tok;
  if (p.cand_out && lane < 32) p.cand_out[m * 32 + lane] = id;
  if (p.prob_out && lane < 32) p.prob_out[m * 32 + lane] = prob;

  // Publish the row, then count it in; the lane's last row runs the scan.
  if (lane < 32) {
    __hip_atomic_store(&p.row_ids[m * 32 + lane], id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.row_probs[m * 32 + lane], prob, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (lane == 0) {
    __hip_atomic_store(&p.row_meta[2 * m], count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.row_meta[2 * m + 1], tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const int l = m / p.R;
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&p.lane_count[l], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != (uint32_t)(p.R - 1)) return;
  lane_scan(p, l, lane);
  if (lane == 0) __hip_atomic_store(&p.lane_count[l], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int launch_sample(const SampleParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(sample_chunk_kernel, dim3(p.chunks, p.M), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  // C * 32 keys per wave, 64 lanes: C / 2 keys per lane
  if (p.chunks <= 32)
    hipLaunchKernelGGL(sample_row_kernel<16>, dim3(p.M), dim3(256), 0, st, p);
  else if (p.chunks <= 64)
    hipLaunchKernelGGL(sample_row_kernel<32>, dim3(p.M), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(sample_row_kernel<64>, dim3(p.M), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace vq
