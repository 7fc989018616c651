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
//    workgroup merges the chunks' sorted lists, one list per lane. Inside a
//    wave, the 32nd largest lane maximum bounds the answer from below; the
//    keys above it are packed into LDS and sorted 64 at a time (usually
//    once).
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

// The need-th largest of the wave's J * 64 values v (the largest t with at
// least `need` values >= t), by a bitwise search on ballots.
template <int J>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&v)[J], int need) {
  uint32_t t = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) n += (int)__popcll(__ballot(v[j] >= c));
    if (n >= need) t = c;
  }
  return t;
}

// The wave's 32 largest keys among N per lane (0 = no key), descending in
// lanes 0..31; lanes 32..63 return 0. `buf` is this wave's LDS area of 64 * N
// keys. Every wave of the workgroup must call it (it holds a barrier).
//
// theta = the 32nd largest value among a sample of the keys: each lane's
// maximum (SORTED = false), or the first four keys of each lane (SORTED =
// true: each lane holds a descending list). At least 32 keys have value bits
// >= theta, so every key of the answer does too; keys below it are dropped.
// The survivors are packed into LDS and reduced 64 at a time: a bitonic sort
// across the lanes and a bitonic merge into the running list. Random logits
// leave 40-50 survivors: one sort.
template <int N, bool SORTED>
__device__ __forceinline__ u64 wave_top32(const u64 (&k)[N], int lane, u64* buf) {
  uint32_t theta;
  if constexpr (SORTED) {
    const uint32_t v[4] = {(uint32_t)(k[0] >> 32), (uint32_t)(k[1] >> 32), (uint32_t)(k[2] >> 32),
                           (uint32_t)(k[3] >> 32)};
    theta = kth_largest<4>(v, 32);
  } else {
    uint32_t mh[1] = {0};
#pragma unroll
    for (int i = 0; i < N; ++i) mh[0] = max(mh[0], (uint32_t)(k[i] >> 32));
    theta = kth_largest<1>(mh, 32);
  }
  u64 live = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (k[i] != 0ull && (uint32_t)(k[i] >> 32) >= theta) live |= 1ull << i;
  int total = 0;
  while (true) {
    const u64 has = __ballot(live != 0ull);
    if (!has) break;
    if (live) {
      const int b = __builtin_ctzll(live);
      live &= live - 1;
      u64 c = 0;
#pragma unroll
      for (int i = 0; i < N; ++i) c = i == b ? k[i] : c;
      buf[total + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(has >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)has, 0u))] = c;
    }
    total += (int)__popcll(has);
  }
  __syncthreads();
  u64 list = 0;
  for (int base = 0; base < total; base += 64) {
    const u64 c = base + lane < total ? buf[base + lane] : 0ull;
    const u64 sorted = wave_sort_desc(c, lane);
    list = base == 0 ? sorted : merge_top32(list, sorted, lane);
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

// Chunk lists of a row: 4C lists of 32 keys (list L = 4 * chunk + wave). Row
// wave w reads lists [wC, (w+1)C), one per lane; key i of list wC + l is
// stored at i * C + l of that wave's block, so each of its loads is one
// contiguous run.
__device__ __forceinline__ size_t cand_index(int C, int m, int L, int i) {
  return (size_t)m * 4 * C * 32 + (size_t)(L / C) * 32 * C + (size_t)i * C + (L % C);
}

// VEC = 4: 16-byte loads (rows 16-byte aligned, V % 4 == 0), lane l holding
// logits 4(64i + l) .. +3 of its wave's 2048; VEC = 1: 4-byte loads.
template <int VEC>
__global__ __launch_bounds__(256) void sample_chunk_kernel(SampleParams p) {
  __shared__ u64 buf[4][64 * 32];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x, m = blockIdx.y;
  const float* row = p.logits + (size_t)m * p.V;
  const int64_t base = (int64_t)c * kSampleChunk + w * (kSampleChunk / 4);
  u64 k[32];
  if constexpr (VEC == 4) {
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t idx = base + 4 * (i * 64 + lane);
      v[i] = idx < p.V ? *reinterpret_cast<const float4*>(row + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t idx = base + 4 * (i * 64 + lane);
      const bool in = idx < p.V;
      k[4 * i + 0] = in ? argmax_key(v[i].x, (uint32_t)idx) : 0ull;
      k[4 * i + 1] = in ? argmax_key(v[i].y, (uint32_t)(idx + 1)) : 0ull;
      k[4 * i + 2] = in ? argmax_key(v[i].z, (uint32_t)(idx + 2)) : 0ull;
      k[4 * i + 3] = in ? argmax_key(v[i].w, (uint32_t)(idx + 3)) : 0ull;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int64_t idx = base + i * 64 + lane;
      k[i] = idx < p.V ? argmax_key(row[idx], (uint32_t)idx) : 0ull;
    }
  }
  const u64 top = wave_top32<32, false>(k, lane, buf[w]);
  if (lane < 32) p.cand[cand_index(p.chunks, m, c * 4 + w, lane)] = top;
}

// ------------------------------------------------- row distribution + scan

// Accept scan of lane l (one wave; every row of the lane is published). All
// loads are issued up front (one round trip): lane j < R reads row j's kept
// count and draw; for the speculative rule lane i also reads candidate i of
// rows 0..R-2 and lane e < 16 the draft pair e of those rows.
__device__ void lane_scan(const SampleParams& p, int l, int lane) {
  const int R = p.R;
  const bool spec = p.q_ids != nullptr;
  auto ld_i = [](const int32_t* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto ld_f = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  int cnt_l = 0, tok_l = -1;
  if (lane < R) {
    cnt_l = ld_i(&p.row_meta[2 * (l * R + lane)]);
    tok_l = ld_i(&p.row_meta[2 * (l * R + lane) + 1]);
  }
  int ids[7], qids[7], drafts[7];
  float prs[7], qps[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const bool row = j < R - 1;
    drafts[j] = row ? p.draft[l * (R - 1) + j] : -1;
    ids[j] = -1;
    prs[j] = 0.0f;
    qids[j] = -1;
    qps[j] = 0.0f;
    if (spec && row) {
      const int m = l * R + j;
      if (lane < 32) {
        ids[j] = ld_i(&p.row_ids[m * 32 + lane]);
        prs[j] = ld_f(&p.row_probs[m * 32 + lane]);
      }
      if (lane < kDraftCands) {
        qids[j] = p.q_ids[(l * (R - 1) + j) * kDraftCands + lane];
        qps[j] = p.q_probs[(l * (R - 1) + j) * kDraftCands + lane];
      }
    }
  }
  int commit = -1;  // lane j < R holds committed token j
  int stop = R - 1; // the row where the scan ends
  bool done = false;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    if (done || j >= R - 1) continue;
    const int m = l * R + j;
    const int count = __shfl(cnt_l, j);
    const int tok = __shfl(tok_l, j);
    const int d = drafts[j];
    if (count == 0) {  // no distribution: the scan stops, committing nothing here
      stop = j;
      done = true;
      continue;
    }
    if (!spec) {  // point-mass: the draft must equal the target's draw
      if (lane == j) commit = tok;
      if (tok != d) {
        stop = j;
        done = true;
      }
      continue;
    }
    const u64 pm = __ballot(lane < count && ids[j] == d);
    const float pd = pm ? __shfl(prs[j], __builtin_ctzll(pm)) : 0.0f;
    const u64 qm = __ballot(lane < kDraftCands && qids[j] >= 0 && qids[j] == d);
    const float qd = qm ? __shfl(qps[j], __builtin_ctzll(qm)) : 0.0f;
    if (p.u_accept[m] * qd < pd) {
      if (lane == j) commit = d;
      continue;
    }
    // rejected: draw from max(p - q, 0) over the kept candidates
    float qi = 0.0f;
    bool found = false;
#pragma unroll
    for (int e = 0; e < kDraftCands; ++e) {
      const int qe = __shfl(qids[j], e);
      const float pe = __shfl(qps[j], e);
      if (!found && qe >= 0 && qe == ids[j]) {
        qi = pe;
        found = true;
      }
    }
    const float r = lane < count ? fmaxf(prs[j] - qi, 0.0f) : 0.0f;
    const float rs = wave_sum32(r);
    const int pick = rs > 0.0f ? __shfl(ids[j], first_above(wave_scan32(r, lane), p.u_draw[m] * rs, lane, count))
                               : tok;  // no residual mass: the draw from p itself
    if (lane == j) commit = pick;
    stop = j;
    done = true;
  }
  if (!done && lane == R - 1) commit = tok_l;  // every draft accepted: the last row's draw is the bonus
  const int acc_len = stop + 1;
  if (lane == 0) p.accept_len_out[l] = acc_len;
  if (p.commit_out && lane < R) p.commit_out[l * R + lane] = lane < acc_len ? commit : -1;
}

// Row workgroup: the 4C chunk lists of row m (sorted, 32 keys each); wave w
// takes lists [w*C, (w+1)*C), one whole list per lane (two when C > 64).
template <int NL>
__global__ __launch_bounds__(256) void sample_row_kernel(SampleParams p) {
  __shared__ u64 buf[4][64 * NL];
  __shared__ u64 lists[4][32];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = blockIdx.x;
  const int C = p.chunks;
  u64 k[NL];
#pragma unroll
  for (int h = 0; h < NL / 32; ++h) {
    const int l = lane + 64 * h;
#pragma unroll
    for (int i = 0; i < 32; ++i) k[32 * h + i] = l < C ? p.cand[cand_index(C, m, w * C + l, i)] : 0ull;
  }
  const u64 top = wave_top32<NL, true>(k, lane, buf[w]);
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
  // The agent-scope (SC1) stores above are acknowledged by the shared memory
  // level before vmcnt drops, so after this wait the row is visible to any
  // agent that sees the count below; compiler-only fences keep the compiler
  // from moving the stores or the count across the wait (s_waitcnt is not
  // modelled as a memory operation).
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int l = m / p.R;
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&p.lane_count[l], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // lane_scan's loads stay after the count
  if (old != (uint32_t)(p.R - 1)) return;
  lane_scan(p, l, lane);
  if (lane == 0) __hip_atomic_store(&p.lane_count[l], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int launch_sample(const SampleParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.V % 4 == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0)
    hipLaunchKernelGGL(sample_chunk_kernel<4>, dim3(p.chunks, p.M), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(sample_chunk_kernel<1>, dim3(p.chunks, p.M), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  // C lists per wave: one list (32 keys) per lane up to C = 64, two beyond
  if (p.chunks <= 64)
    hipLaunchKernelGGL(sample_row_kernel<32>, dim3(p.M), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(sample_row_kernel<64>, dim3(p.M), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace vq
