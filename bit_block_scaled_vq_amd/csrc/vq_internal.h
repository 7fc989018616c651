// Internal interface between the C-ABI layer (libverify.cpp) and the HIP
// kernels (vq_kernels.hip: GEMMs, packing, probes; vq_sample.hip: sampled
// verify; vq_gdn.hip: GDN state stream). Not installed; not part of the
// public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace vq {

// FMT_NVFP4: block scale applied to the fp32 partial after the MFMA (two
// scale blocks per MFMA through zero-padded activation rows; up to 8 rows per
// row group). FMT_NVFP4S: the same packed weights scaled in registers before
// the MFMA (exact in bf16), 16 activation rows per row group.
// FMT_AFFINE: affine 4-bit, w = scale * q + bias per group of 64 K (bf16 scale
// and bias), 16 activation rows per row group; the packed block has the NVFP4
// code layout and 512 B of (scale, bias) pairs.
enum Fmt : int { FMT_NVFP4 = 0, FMT_FP8 = 1, FMT_NVFP4S = 2, FMT_AFFINE = 3 };
enum Epi : int { EPI_NONE = 0, EPI_SILU = 1, EPI_ARGMAX = 2, EPI_ACC = 3 };

// Packed weights are laid out in blocks of one tile (64 weight rows, four
// sub-tiles of 16) by one k-iteration (128 K). NVFP4 block: 4 KB of codes +
// 512 B of block scales; FP8 block: 8 KB.
constexpr int kTileRows = 64;
constexpr int kSub = 16;
constexpr int kNT = 4;
constexpr int kIterK = 128;
constexpr int kBlockF4 = 4096 + 512;
constexpr int kBlockF8 = 8192;

// Minimum iterations per wave before the workgroup count is reduced.
constexpr int kCUs = 256;  // MI355X compute units
// Unaligned stream-K splits use one CU per XCD fewer than the chip has
// (measured faster than all 256 for the 34816 x 5120 projection).
constexpr int kMaxWgs = kCUs - 8;
constexpr int kMinItersPerWave = 4;
// Partial-sum slot: 4 sub-tiles x up to 16 accumulator registers x 64 lanes.
constexpr int kSlotFloats = kNT * 16 * 64;
// Argmax candidate buckets per row (spread the cross-worker atomics).
constexpr int kBuckets = 64;
constexpr int kMaxRows = 32;

struct Schedule {
  int32_t tiles;      // T: units of the schedule (tiles, half tiles or tile pairs)
  int32_t iters;      // I = K / kIterK
  int64_t total;      // T * I
  int32_t wgs;        // G: stream-K workgroups
  int32_t unit_subs;  // sub-tiles per unit: 2 (half tiles), 4 (tiles), 8 (tile pairs)
  size_t off_partials, off_counters, off_best, off_done, bytes;
};

// Tiles of an output of n_out columns: 64 columns per tile, or 32 with the
// SiLU epilogue (whose tiles carry 32 gate + 32 up rows).
inline int32_t tiles_for(int epi, int32_t n_out) {
  // accumulating epilogue: both halves of every 64-row weight tile
  if (epi == EPI_ACC) return 2 * ((n_out + kTileRows - 1) / kTileRows);
  const int32_t cols = epi == EPI_SILU ? kTileRows / 2 : kTileRows;
  return (n_out + cols - 1) / cols;
}

// Tile pairs as units for the scaled NVFP4 family (M > 8) from this many
// tiles on: one activation load then feeds 128 output columns. Only where a
// workgroup gets many units: the vocabulary head (3,880 tiles) at M = 32
// 160 against 180 us per launch, but [gate; up] (544 tiles, 1.1 pairs per
// workgroup, nearly every pair then split between two) 38.3 against 34.2 us.
constexpr int32_t kPairMinTiles = 8 * kCUs;

// The schedule depends only on (epilogue kind, N, K) and on wide_rows, the
// scaled NVFP4 family (NVFP4 at M > 8), never on M otherwise.
Schedule make_schedule(int epi, int32_t n_out, int32_t k, bool wide_rows = false);

struct GemmParams {
  const uint16_t* x;
  const uint8_t* w;       // packed weights
  float out_scale;        // NVFP4 tensor scale or FP8 per-tensor scale
  void* y;
  int32_t M, N, K;        // N: output columns
  int32_t y_f32;
  int32_t tiles, iters, wgs;  // tiles: units of the schedule
  int32_t unit_subs;          // sub-tiles per unit (the kernel instance's NT)
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

struct PackParams {
  const uint8_t* codes;   // NVFP4 codes [rows][K/2] or FP8 weights [rows][K]
  const uint8_t* scales;  // NVFP4 scales [rows][K/16]; affine: bf16 scales [rows][K/64]
  const uint8_t* biases;  // affine: bf16 biases [rows][K/64]
  uint8_t* out;
  int32_t rows, K;        // rows of the canonical matrix
  int32_t gate_up;        // NVFP4: tiles pair gate row r with up row r + rows/2
  int32_t tiles, iters;
};

// Sampled verify over fp32 logits [M][V]: per row the top-32 candidates, the
// truncated target distribution, a draw, and the accept scan per lane.
constexpr int kSampleChunk = 8192;   // logits per chunk workgroup (32 per thread)
constexpr int kTopK = 32;            // largest top_k
constexpr int kDraftCands = 16;      // draft (id, prob) pairs per verify row
constexpr int kMaxSampleV = 1 << 20; // at most 128 chunks per row

struct SampleLayout {
  int32_t chunks;                    // C = ceil(V / kSampleChunk)
  size_t off_cand, off_ids, off_probs, off_meta, off_count, bytes;
};
SampleLayout make_sample_layout(int32_t M, int32_t V);

struct SampleParams {
  const float* logits;               // [M][V]
  int32_t M, V, lanes, R, chunks;
  float temperature, top_p;
  int32_t top_k;
  const int32_t* draft;              // [lanes][R-1]
  const int32_t* q_ids;              // [lanes][R-1][16] or null (point-mass)
  const float* q_probs;
  const float* u_accept;             // [M]
  const float* u_draw;               // [M]
  int32_t* token_out;                // [M] or null
  int32_t* accept_len_out;           // [lanes]
  int32_t* commit_out;               // [lanes][R] or null
  int32_t* cand_out;                 // [M][32] or null
  float* prob_out;                   // [M][32] or null
  unsigned long long* cand;          // workspace: [M][C][4][32] chunk candidates
  int32_t* row_ids;                  // workspace: [M][32]
  float* row_probs;                  // workspace: [M][32]
  int32_t* row_meta;                 // workspace: [M][2] (kept count, draw)
  uint32_t* lane_count;              // workspace: [4] rows finished per lane
};

// Gated DeltaNet state stream: fp32 state per value head, dk x dv.
constexpr int kGdnDk = 128;
constexpr int kGdnDv = 128;
constexpr int kGdnMaxT = 16;         // rows per entry and call

struct GdnParams {
  const float* state_in;             // [B][H][dk][dv]
  float* state_out;                  // [B][H][dk][dv], disjoint from state_in
  const float* q;                    // [B][T][Hk][dk]
  const float* k;                    // [B][T][Hk][dk]
  const float* v;                    // [B][T][H][dv]
  const float* a;                    // [B][T][H] decays
  const float* b;                    // [B][T][H] write strengths
  float* o;                          // [B][T][H][dv] or null
  const int32_t* count;              // [lanes] rows to re-scan (commit) or null (verify)
  int32_t B, T, H, Hk, lanes;
};

// Device scratch of the allocation-free GEMM entry point: one fixed layout
// for every shape, so calls of different (N, K, epilogue) can follow each
// other on it: [per-tile counters][partial-sum slots].
// Counters start at zero (static storage) and every call leaves the ones it
// used at zero; the slots need no initial value.
constexpr int kScratchTiles = 1 << 16;                 // N <= 4,194,304 (2,097,152 with SILU_MUL)
constexpr size_t kScratchCounters = 0;
constexpr size_t kScratchPartials = kScratchCounters + (size_t)kScratchTiles * sizeof(uint32_t);
constexpr size_t kScratchBytes = kScratchPartials + (size_t)2 * kCUs * kSlotFloats * sizeof(float);
// This device's copy of the scratch array (looked up once per device); 0 on
// success, else the hipError_t of the lookup.
int scratch_ptr(void** out);

// Launchers: return 0 on success, else the hipError_t of the launch.
int launch_gemm(int fmt, int epi, const GemmParams& p, void* stream);
int launch_pack(int fmt, const PackParams& p, void* stream);
int launch_sample(const SampleParams& p, void* stream);
int launch_gdn(const GdnParams& p, void* stream);
int launch_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int launch_probe_read(const void* src, size_t bytes, void* sink, void* stream);

}  // namespace vq
