// Internal interface between the C-ABI layer (libverify.cpp) and the HIP
// kernels (vq_kernels.hip). Not installed; not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace vq {

enum Fmt : int { FMT_NVFP4 = 0, FMT_FP8 = 1 };
enum Epi : int { EPI_NONE = 0, EPI_SILU = 1, EPI_ARGMAX = 2 };

// Output columns handled by one tile: NT sub-tiles of 32 weight rows.
constexpr int kSubRows = 32;
constexpr int kNT = 2;
// K consumed by one pipeline iteration of one wave.
constexpr int kIterK = 64;
// Stream-K workers (waves) per launch at most, and the minimum iterations a
// worker gets before the worker count is reduced.
constexpr int kMaxWorkers = 2048;
constexpr int kMinItersPerWorker = 4;
// Partial-sum slot: NT sub-tiles x 16 accumulator registers x 64 lanes (fp32).
constexpr int kSlotFloats = kNT * 16 * 64;
// Argmax candidate buckets per row (spread the cross-tile atomics).
constexpr int kBuckets = 64;
constexpr int kMaxRows = 32;

struct Schedule {
  int32_t tiles;      // T
  int32_t iters;      // I = K / kIterK
  int64_t total;      // T * I
  int32_t workers;    // P
  size_t off_partials, off_counters, off_best, off_done, bytes;
};

// The schedule depends only on (epilogue kind, N, K) -- never on M.
Schedule make_schedule(int epi, int32_t n_out, int32_t k);

struct GemmParams {
  const uint16_t* x;
  const uint8_t* codes;   // NVFP4 codes, or FP8 weights
  const uint8_t* scales;  // NVFP4 block scales
  float out_scale;        // NVFP4 tensor scale or FP8 per-tensor scale
  void* y;
  int32_t M, N, K;        // N: output columns
  int32_t y_f32;
  int32_t tiles, iters, workers;
  int64_t total;
  float* partials;
  uint32_t* counters;
  unsigned long long* best;
  uint32_t* done;
  const int32_t* draft;
  int32_t lanes, R;
  int32_t* argmax_out;
  float* maxlogit_out;
  int32_t* accept_len_out;
  int32_t* commit_out;
};

// Launchers: return 0 on success, else the hipError_t of the launch.
int launch_gemm(int fmt, int epi, const GemmParams& p, void* stream);
int launch_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int launch_probe_read(const void* src, size_t bytes, void* sink, void* stream);

}  // namespace vq
