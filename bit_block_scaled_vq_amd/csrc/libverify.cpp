// libverify C ABI: argument validation, the gfx950 gate, the stream-K schedule
// and workspace layout, and dispatch to the HIP kernels. See include/libverify.h
// for the contract of every entry point.
#include "libverify.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <string>

#include "vq_internal.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int32_t check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(VQ_ERR_DEVICE, "no HIP device is available");
  }
  if (dev >= kMaxDevices) return fail(VQ_ERR_DEVICE, "device index %d out of range", dev);
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(VQ_ERR_DEVICE, "hipGetDeviceProperties failed on device %d", dev);
    }
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(VQ_ERR_DEVICE, "device %d is %s, libverify is built for gfx950", dev, prop.gcnArchName);
  }
  return st == 1 ? VQ_OK : fail(VQ_ERR_DEVICE, "device %d is not gfx950", dev);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool shape_ok(int32_t M, int32_t N, int32_t K) {
  return M >= 1 && M <= vq::kMaxRows && N >= 1 && N <= (1 << 30) && K >= vq::kIterK && K % vq::kIterK == 0 &&
         K <= (1 << 24);
}

int32_t check_shape(int32_t M, int32_t N, int32_t K) {
  if (M < 1 || M > vq::kMaxRows) return fail(VQ_ERR_SHAPE, "M = %d outside [1, %d]", M, vq::kMaxRows);
  if (N < 1 || N > (1 << 30)) return fail(VQ_ERR_SHAPE, "N = %d outside [1, 2^30]", N);
  if (K < vq::kIterK || K % vq::kIterK != 0 || K > (1 << 24))
    return fail(VQ_ERR_SHAPE, "K = %d must be a positive multiple of %d (at most 2^24)", K, vq::kIterK);
  return VQ_OK;
}

int32_t check_ws(const vq::Schedule& s, void* ws, size_t ws_bytes) {
  if (!ws) return fail(VQ_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", s.bytes);
  if (!aligned(ws, 16)) return fail(VQ_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (ws_bytes < s.bytes) return fail(VQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, s.bytes);
  return VQ_OK;
}

// Bytes of a packed matrix: kind VQ_PACK_*, `rows` canonical rows.
size_t packed_bytes(int32_t kind, int64_t rows, int64_t k) {
  if (rows < 1 || k < vq::kIterK || k % vq::kIterK != 0) return 0;
  const int64_t iters = k / vq::kIterK;
  if (kind == VQ_PACK_NVFP4) return (size_t)((rows + 63) / 64 * iters) * vq::kBlockF4;
  if (kind == VQ_PACK_NVFP4_GATE_UP) return rows % 2 ? 0 : (size_t)((rows / 2 + 31) / 32 * iters) * vq::kBlockF4;
  if (kind == VQ_PACK_FP8) return (size_t)((rows + 63) / 64 * iters) * vq::kBlockF8;
  if (kind == VQ_PACK_AFFINE_Q4) return (size_t)((rows + 63) / 64 * iters) * vq::kBlockF4;
  if (kind == VQ_PACK_AFFINE_Q4_GATE_UP) return rows % 2 ? 0 : (size_t)((rows / 2 + 31) / 32 * iters) * vq::kBlockF4;
  return 0;
}

int32_t check_w(const uint8_t* w, size_t w_bytes, size_t need) {
  if (!aligned(w, 16)) return fail(VQ_ERR_ALIGN, "packed weights must be 16-byte aligned");
  if (w_bytes < need) return fail(VQ_ERR_SHAPE, "packed weights have %zu bytes, this shape needs %zu", w_bytes, need);
  return VQ_OK;
}

void bind_workspace(vq::GemmParams& p, const vq::Schedule& s, void* ws) {
  char* base = static_cast<char*>(ws);
  p.partials = reinterpret_cast<float*>(base + s.off_partials);
  p.counters = reinterpret_cast<uint32_t*>(base + s.off_counters);
  p.best = s.off_best ? reinterpret_cast<unsigned long long*>(base + s.off_best) : nullptr;
  p.done = s.off_done ? reinterpret_cast<uint32_t*>(base + s.off_done) : nullptr;
  p.tiles = s.tiles;
  p.unit_subs = s.unit_subs;
  p.iters = s.iters;
  p.total = s.total;
  p.wgs = s.wgs;
}

int32_t launch(int fmt, int epi, const vq::GemmParams& p, void* stream) {
  const int err = vq::launch_gemm(fmt, epi, p, stream);
  if (err != 0) return fail(VQ_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

}  // namespace

namespace vq {

Schedule make_schedule(int epi, int32_t n_out, int32_t k, bool wide_rows) {
  Schedule s{};
  const int32_t tiles = tiles_for(epi, n_out);
  const bool pairs = wide_rows && epi != EPI_ACC && tiles >= kPairMinTiles;
  s.unit_subs = epi == EPI_ACC ? kNT / 2 : (pairs ? 2 * kNT : kNT);
  s.tiles = pairs ? (tiles + 1) / 2 : tiles;
  s.iters = k / kIterK;
  s.total = (int64_t)s.tiles * s.iters;
  // Stream-K over at most kMaxWgs 4-wave workgroups, each wave with at least
  // kMinItersPerWave iterations; never more workgroups than iterations.
  int64_t g = (s.total + 4 * kMinItersPerWave - 1) / (4 * kMinItersPerWave);
  if (g > kMaxWgs) g = kMaxWgs;
  if (g > s.total) g = s.total;
  if (g < 1) g = 1;
  // Prefer a tile-aligned split that keeps at least 7/8 of the CUs busy with
  // one workgroup each: k workgroups per tile (narrow outputs) or k tiles per
  // workgroup (wide ones). Then no workgroup holds parts of two tiles, and a
  // tile's shares come from whole workgroups.
  const int64_t lo = kCUs * 7 / 8;
  if (s.tiles <= kCUs) {
    const int64_t k = kCUs / s.tiles;
    if (k >= 1 && s.tiles * k >= lo && s.iters / k >= 4 * kMinItersPerWave) g = s.tiles * k;
  } else {
    for (int64_t k = (s.tiles + kCUs - 1) / kCUs; k <= 64; ++k) {
      if (s.tiles % k) continue;
      if (s.tiles / k < lo) break;
      g = s.tiles / k;
      break;
    }
  }
  if (epi == EPI_ACC) {
    // Every half-tile unit must be shared by at most two workgroups. Three
    // workgroups per tile (stream-K over the tile's two units, boundaries at
    // 2/3 and 4/3 of a unit) when that fits the CUs, else at most one
    // workgroup per unit.
    const int64_t pairs = s.tiles / 2;
    g = 3 * pairs <= kCUs ? 3 * pairs : (s.tiles < kMaxWgs ? s.tiles : kMaxWgs);
  }
  s.wgs = (int32_t)g;
  size_t off = 0;
  s.off_partials = off;
  off = align_up(off + (size_t)2 * s.wgs * kSlotFloats * sizeof(float), 256);
  s.off_counters = off;
  // one counter per tile, whatever the unit: both NVFP4 families lay out a
  // workspace of (op, N, K) the same way when their workgroup counts agree
  off = align_up(off + (size_t)tiles * sizeof(uint32_t), 256);
  if (epi == EPI_ARGMAX) {
    s.off_best = off;
    off = align_up(off + (size_t)kBuckets * kMaxRows * sizeof(unsigned long long), 256);
    s.off_done = off;
    off = align_up(off + sizeof(uint32_t), 256);
  }
  s.bytes = off;
  return s;
}

SampleLayout make_sample_layout(int32_t M, int32_t V) {
  SampleLayout L{};
  L.chunks = (V + kSampleChunk - 1) / kSampleChunk;
  size_t off = 0;
  L.off_cand = off;
  off = align_up(off + (size_t)M * L.chunks * 4 * kTopK * sizeof(unsigned long long), 256);
  L.off_ids = off;
  off = align_up(off + (size_t)M * kTopK * sizeof(int32_t), 256);
  L.off_probs = off;
  off = align_up(off + (size_t)M * kTopK * sizeof(float), 256);
  L.off_meta = off;
  off = align_up(off + (size_t)M * 2 * sizeof(int32_t), 256);
  L.off_count = off;
  off = align_up(off + 4 * sizeof(uint32_t), 256);
  L.bytes = off;
  return L;
}

}  // namespace vq

extern "C" {

int32_t vq_abi_version(void) { return VQ_ABI_VERSION; }

const char* vq_last_error(void) { return g_last_error.c_str(); }

const char* vq_status_str(int32_t s) {
  switch (s) {
    case VQ_OK: return "VQ_OK";
    case VQ_ERR_NULL: return "VQ_ERR_NULL";
    case VQ_ERR_SHAPE: return "VQ_ERR_SHAPE";
    case VQ_ERR_ALIGN: return "VQ_ERR_ALIGN";
    case VQ_ERR_WORKSPACE: return "VQ_ERR_WORKSPACE";
    case VQ_ERR_DEVICE: return "VQ_ERR_DEVICE";
    case VQ_ERR_LAUNCH: return "VQ_ERR_LAUNCH";
    case VQ_ERR_VALUE: return "VQ_ERR_VALUE";
    default: return "VQ_ERR_UNKNOWN";
  }
}

size_t vq_workspace_bytes(int32_t op, int32_t M, int32_t N, int32_t K) {
  if (op == VQ_OP_SAMPLE) {
    if (M < 1 || M > vq::kMaxRows || N < 1 || N > vq::kMaxSampleV) return 0;
    return vq::make_sample_layout(M, N).bytes;
  }
  if (!shape_ok(M, N, K)) return 0;
  // NVFP4 ops: large enough for both families (M <= 8 and M > 8), so one
  // workspace of (op, N, K) serves every M
  auto both = [&](int epi) {
    const size_t a = vq::make_schedule(epi, N, K, false).bytes, b = vq::make_schedule(epi, N, K, true).bytes;
    return a > b ? a : b;
  };
  switch (op) {
    case VQ_OP_NVFP4: return both(vq::EPI_NONE);
    case VQ_OP_NVFP4_SILU_MUL:
      if (N > (1 << 29)) return 0;
      return both(vq::EPI_SILU);
    case VQ_OP_FP8: return vq::make_schedule(vq::EPI_NONE, N, K).bytes;
    case VQ_OP_LMHEAD: return both(vq::EPI_ARGMAX);
    case VQ_OP_AFFINE_Q4: return vq::make_schedule(vq::EPI_NONE, N, K).bytes;
    case VQ_OP_AFFINE_Q4_SILU_MUL:
      if (N > (1 << 29)) return 0;
      return vq::make_schedule(vq::EPI_SILU, N, K).bytes;
    default: return 0;
  }
}

size_t vq_packed_bytes(int32_t kind, int32_t rows, int32_t K) { return packed_bytes(kind, rows, K); }

int32_t vq_schedule_info(int32_t op, int32_t M, int32_t N, int32_t K, int32_t* units, int32_t* iters,
                         int32_t* workgroups) {
  if (!units || !iters || !workgroups) return fail(VQ_ERR_NULL, "vq_schedule_info: outputs are required");
  if (!shape_ok(M, N, K)) return fail(VQ_ERR_SHAPE, "vq_schedule_info: M = %d, N = %d, K = %d out of range", M, N, K);
  int epi;
  bool nvfp4 = false;
  switch (op) {
    case VQ_OP_NVFP4: nvfp4 = true; epi = vq::EPI_NONE; break;
    case VQ_OP_FP8: case VQ_OP_AFFINE_Q4: epi = vq::EPI_NONE; break;
    case VQ_OP_NVFP4_SILU_MUL: nvfp4 = true; epi = vq::EPI_SILU; break;
    case VQ_OP_AFFINE_Q4_SILU_MUL: epi = vq::EPI_SILU; break;
    case VQ_OP_LMHEAD: nvfp4 = true; epi = vq::EPI_ARGMAX; break;
    case VQ_OP_FP8_ACCUMULATE: epi = vq::EPI_ACC; break;
    default: return fail(VQ_ERR_VALUE, "vq_schedule_info: op %d has no GEMM schedule", op);
  }
  const vq::Schedule s = vq::make_schedule(epi, N, K, nvfp4 && M > 8);
  *units = s.tiles;
  *iters = s.iters;
  *workgroups = s.wgs;
  return VQ_OK;
}

int32_t vq_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, int32_t rows, int32_t K, int32_t gate_up,
                      uint8_t* packed, size_t packed_bytes_avail, void* stream) {
  if (!codes || !scales || !packed) return fail(VQ_ERR_NULL, "vq_pack_nvfp4: codes, scales and packed are required");
  if (gate_up != 0 && gate_up != 1) return fail(VQ_ERR_VALUE, "gate_up must be 0 or 1");
  const int32_t kind = gate_up ? VQ_PACK_NVFP4_GATE_UP : VQ_PACK_NVFP4;
  if (rows < 1 || rows > (1 << 30) || (gate_up && rows % 2)) return fail(VQ_ERR_SHAPE, "rows = %d invalid", rows);
  if (K < vq::kIterK || K % vq::kIterK != 0 || K > (1 << 24))
    return fail(VQ_ERR_SHAPE, "K = %d must be a positive multiple of %d (at most 2^24)", K, vq::kIterK);
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(packed, 16))
    return fail(VQ_ERR_ALIGN, "codes, scales and packed must be 16-byte aligned");
  const size_t need = packed_bytes(kind, rows, K);
  if (packed_bytes_avail < need) return fail(VQ_ERR_SHAPE, "packed buffer has %zu bytes, %zu needed", packed_bytes_avail, need);
  int32_t st = check_device();
  if (st) return st;
  vq::PackParams p{};
  p.codes = codes;
  p.scales = scales;
  p.out = packed;
  p.rows = rows;
  p.K = K;
  p.gate_up = gate_up;
  p.tiles = gate_up ? (rows / 2 + 31) / 32 : (rows + 63) / 64;
  p.iters = K / vq::kIterK;
  const int err = vq::launch_pack(vq::FMT_NVFP4, p, stream);
  if (err) return fail(VQ_ERR_LAUNCH, "pack launch failed: %s", hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

int32_t vq_pack_fp8(const uint8_t* w, int32_t rows, int32_t K, uint8_t* packed, size_t packed_bytes_avail,
                    void* stream) {
  if (!w || !packed) return fail(VQ_ERR_NULL, "vq_pack_fp8: w and packed are required");
  if (rows < 1 || rows > (1 << 30)) return fail(VQ_ERR_SHAPE, "rows = %d invalid", rows);
  if (K < vq::kIterK || K % vq::kIterK != 0 || K > (1 << 24))
    return fail(VQ_ERR_SHAPE, "K = %d must be a positive multiple of %d (at most 2^24)", K, vq::kIterK);
  if (!aligned(w, 16) || !aligned(packed, 16)) return fail(VQ_ERR_ALIGN, "w and packed must be 16-byte aligned");
  const size_t need = packed_bytes(VQ_PACK_FP8, rows, K);
  if (packed_bytes_avail < need) return fail(VQ_ERR_SHAPE, "packed buffer has %zu bytes, %zu needed", packed_bytes_avail, need);
  int32_t st = check_device();
  if (st) return st;
  vq::PackParams p{};
  p.codes = w;
  p.out = packed;
  p.rows = rows;
  p.K = K;
  p.tiles = (rows + 63) / 64;
  p.iters = K / vq::kIterK;
  const int err = vq::launch_pack(vq::FMT_FP8, p, stream);
  if (err) return fail(VQ_ERR_LAUNCH, "pack launch failed: %s", hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

int32_t vq_gemm_nvfp4(const uint16_t* x, const uint8_t* w, size_t w_bytes, float tensor_scale, void* y,
                      int32_t y_dtype, int32_t M, int32_t N, int32_t K, int32_t epilogue, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!x || !w || !y) return fail(VQ_ERR_NULL, "vq_gemm_nvfp4: x, w and y are required");
  if (y_dtype != VQ_OUT_BF16 && y_dtype != VQ_OUT_F32) return fail(VQ_ERR_VALUE, "unknown y_dtype %d", y_dtype);
  if (epilogue != VQ_EPI_NONE && epilogue != VQ_EPI_SILU_MUL) return fail(VQ_ERR_VALUE, "unknown epilogue %d", epilogue);
  int32_t st = check_shape(M, N, K);
  if (st) return st;
  if (epilogue == VQ_EPI_SILU_MUL && N > (1 << 29)) return fail(VQ_ERR_SHAPE, "N = %d too large for SILU_MUL", N);
  if (!aligned(x, 16)) return fail(VQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, y_dtype == VQ_OUT_F32 ? 4 : 2)) return fail(VQ_ERR_ALIGN, "y is not aligned to its element size");
  const bool silu = epilogue == VQ_EPI_SILU_MUL;
  st = check_w(w, w_bytes, silu ? packed_bytes(VQ_PACK_NVFP4_GATE_UP, 2 * (int64_t)N, K)
                                 : packed_bytes(VQ_PACK_NVFP4, N, K));
  if (st) return st;
  const int epi = silu ? vq::EPI_SILU : vq::EPI_NONE;
  const vq::Schedule s = vq::make_schedule(epi, N, K, M > 8);
  st = check_ws(s, workspace, workspace_bytes);
  if (st) return st;
  st = check_device();
  if (st) return st;
  vq::GemmParams p{};
  p.x = x;
  p.w = w;
  p.out_scale = tensor_scale;
  p.y = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.y_f32 = y_dtype == VQ_OUT_F32;
  bind_workspace(p, s, workspace);
  return launch(vq::FMT_NVFP4, epi, p, stream);
}

int32_t vq_gemm_nvfp4_noalloc(const uint16_t* x, const uint8_t* w, size_t w_bytes, float tensor_scale, void* y,
                              int32_t y_dtype, int32_t M, int32_t N, int32_t K, int32_t epilogue, void* stream) {
  if (!x || !w || !y) return fail(VQ_ERR_NULL, "vq_gemm_nvfp4_noalloc: x, w and y are required");
  if (y_dtype != VQ_OUT_BF16 && y_dtype != VQ_OUT_F32) return fail(VQ_ERR_VALUE, "unknown y_dtype %d", y_dtype);
  if (epilogue != VQ_EPI_NONE && epilogue != VQ_EPI_SILU_MUL) return fail(VQ_ERR_VALUE, "unknown epilogue %d", epilogue);
  int32_t st = check_shape(M, N, K);
  if (st) return st;
  const bool silu = epilogue == VQ_EPI_SILU_MUL;
  const int epi = silu ? vq::EPI_SILU : vq::EPI_NONE;
  if (vq::tiles_for(epi, N) > vq::kScratchTiles)
    return fail(VQ_ERR_SHAPE, "vq_gemm_nvfp4_noalloc: N = %d needs %d tiles, the device scratch holds %d (N <= %d%s)",
                N, vq::tiles_for(epi, N), vq::kScratchTiles, silu ? vq::kScratchTiles * 32 : vq::kScratchTiles * 64,
                silu ? " with SILU_MUL" : "");
  if (!aligned(x, 16)) return fail(VQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, y_dtype == VQ_OUT_F32 ? 4 : 2)) return fail(VQ_ERR_ALIGN, "y is not aligned to its element size");
  st = check_w(w, w_bytes, silu ? packed_bytes(VQ_PACK_NVFP4_GATE_UP, 2 * (int64_t)N, K)
                                 : packed_bytes(VQ_PACK_NVFP4, N, K));
  if (st) return st;
  const vq::Schedule s = vq::make_schedule(epi, N, K, M > 8);
  if (s.wgs > vq::kCUs) return fail(VQ_ERR_SHAPE, "schedule of %d workgroups exceeds the scratch's %d", s.wgs, vq::kCUs);
  st = check_device();
  if (st) return st;
  void* base = nullptr;
  const int err = vq::scratch_ptr(&base);
  if (err != 0)
    return fail(VQ_ERR_DEVICE, "device scratch lookup failed: %s", hipGetErrorString((hipError_t)err));
  char* sc = static_cast<char*>(base);
  vq::GemmParams p{};
  p.x = x;
  p.w = w;
  p.out_scale = tensor_scale;
  p.y = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.y_f32 = y_dtype == VQ_OUT_F32;
  p.counters = reinterpret_cast<uint32_t*>(sc + vq::kScratchCounters);
  p.partials = reinterpret_cast<float*>(sc + vq::kScratchPartials);
  p.tiles = s.tiles;
  p.unit_subs = s.unit_subs;
  p.iters = s.iters;
  p.total = s.total;
  p.wgs = s.wgs;
  return launch(vq::FMT_NVFP4, epi, p, stream);
}

int32_t vq_pack_affine_q4(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int32_t rows,
                          int32_t K, int32_t gate_up, uint8_t* packed, size_t packed_bytes_avail, void* stream) {
  if (!codes || !scales || !biases || !packed)
    return fail(VQ_ERR_NULL, "vq_pack_affine_q4: codes, scales, biases and packed are required");
  if (gate_up != 0 && gate_up != 1) return fail(VQ_ERR_VALUE, "gate_up must be 0 or 1");
  const int32_t kind = gate_up ? VQ_PACK_AFFINE_Q4_GATE_UP : VQ_PACK_AFFINE_Q4;
  if (rows < 1 || rows > (1 << 30) || (gate_up && rows % 2)) return fail(VQ_ERR_SHAPE, "rows = %d invalid", rows);
  if (K < vq::kIterK || K % vq::kIterK != 0 || K > (1 << 24))
    return fail(VQ_ERR_SHAPE, "K = %d must be a positive multiple of %d (at most 2^24)", K, vq::kIterK);
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(biases, 16) || !aligned(packed, 16))
    return fail(VQ_ERR_ALIGN, "codes, scales, biases and packed must be 16-byte aligned");
  const size_t need = packed_bytes(kind, rows, K);
  if (packed_bytes_avail < need) return fail(VQ_ERR_SHAPE, "packed buffer has %zu bytes, %zu needed", packed_bytes_avail, need);
  int32_t st = check_device();
  if (st) return st;
  vq::PackParams p{};
  p.codes = codes;
  p.scales = reinterpret_cast<const uint8_t*>(scales);
  p.biases = reinterpret_cast<const uint8_t*>(biases);
  p.out = packed;
  p.rows = rows;
  p.K = K;
  p.gate_up = gate_up;
  p.tiles = gate_up ? (rows / 2 + 31) / 32 : (rows + 63) / 64;
  p.iters = K / vq::kIterK;
  const int err = vq::launch_pack(vq::FMT_AFFINE, p, stream);
  if (err) return fail(VQ_ERR_LAUNCH, "pack launch failed: %s", hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

int32_t vq_gemm_affine_q4(const uint16_t* x, const uint8_t* w, size_t w_bytes, void* y, int32_t y_dtype, int32_t M,
                          int32_t N, int32_t K, int32_t epilogue, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!x || !w || !y) return fail(VQ_ERR_NULL, "vq_gemm_affine_q4: x, w and y are required");
  if (y_dtype != VQ_OUT_BF16 && y_dtype != VQ_OUT_F32) return fail(VQ_ERR_VALUE, "unknown y_dtype %d", y_dtype);
  if (epilogue != VQ_EPI_NONE && epilogue != VQ_EPI_SILU_MUL) return fail(VQ_ERR_VALUE, "unknown epilogue %d", epilogue);
  int32_t st = check_shape(M, N, K);
  if (st) return st;
  if (epilogue == VQ_EPI_SILU_MUL && N > (1 << 29)) return fail(VQ_ERR_SHAPE, "N = %d too large for SILU_MUL", N);
  if (!aligned(x, 16)) return fail(VQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, y_dtype == VQ_OUT_F32 ? 4 : 2)) return fail(VQ_ERR_ALIGN, "y is not aligned to its element size");
  const bool silu = epilogue == VQ_EPI_SILU_MUL;
  st = check_w(w, w_bytes, silu ? packed_bytes(VQ_PACK_AFFINE_Q4_GATE_UP, 2 * (int64_t)N, K)
                                 : packed_bytes(VQ_PACK_AFFINE_Q4, N, K));
  if (st) return st;
  const int epi = silu ? vq::EPI_SILU : vq::EPI_NONE;
  const vq::Schedule s = vq::make_schedule(epi, N, K);
  st = check_ws(s, workspace, workspace_bytes);
  if (st) return st;
  st = check_device();
  if (st) return st;
  vq::GemmParams p{};
  p.x = x;
  p.w = w;
  p.out_scale = 1.0f;
  p.y = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.y_f32 = y_dtype == VQ_OUT_F32;
  bind_workspace(p, s, workspace);
  return launch(vq::FMT_AFFINE, epi, p, stream);
}

int32_t vq_gemm_fp8(const uint16_t* x, const uint8_t* w, size_t w_bytes, float w_scale, void* y, int32_t y_dtype,
                    int32_t M, int32_t N, int32_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w || !y) return fail(VQ_ERR_NULL, "vq_gemm_fp8: x, w and y are required");
  if (y_dtype != VQ_OUT_BF16 && y_dtype != VQ_OUT_F32) return fail(VQ_ERR_VALUE, "unknown y_dtype %d", y_dtype);
  int32_t st = check_shape(M, N, K);
  if (st) return st;
  if (!aligned(x, 16)) return fail(VQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, y_dtype == VQ_OUT_F32 ? 4 : 2)) return fail(VQ_ERR_ALIGN, "y is not aligned to its element size");
  st = check_w(w, w_bytes, packed_bytes(VQ_PACK_FP8, N, K));
  if (st) return st;
  const vq::Schedule s = vq::make_schedule(vq::EPI_NONE, N, K);
  st = check_ws(s, workspace, workspace_bytes);
  if (st) return st;
  st = check_device();
  if (st) return st;
  vq::GemmParams p{};
  p.x = x;
  p.w = w;
  p.out_scale = w_scale;
  p.y = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.y_f32 = y_dtype == VQ_OUT_F32;
  bind_workspace(p, s, workspace);
  return launch(vq::FMT_FP8, vq::EPI_NONE, p, stream);
}

int32_t vq_gemm_fp8_accumulate(const uint16_t* x, const uint8_t* w, size_t w_bytes, float w_scale, float* y,
                               int32_t M, int32_t N, int32_t K, void* stream) {
  if (!x || !w || !y) return fail(VQ_ERR_NULL, "vq_gemm_fp8_accumulate: x, w and y are required");
  int32_t st = check_shape(M, N, K);
  if (st) return st;
  if (!aligned(x, 16)) return fail(VQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, 4)) return fail(VQ_ERR_ALIGN, "y must be 4-byte aligned");
  st = check_w(w, w_bytes, packed_bytes(VQ_PACK_FP8, N, K));
  if (st) return st;
  st = check_device();
  if (st) return st;
  const vq::Schedule s = vq::make_schedule(vq::EPI_ACC, N, K);
  vq::GemmParams p{};
  p.x = x;
  p.w = w;
  p.out_scale = w_scale;
  p.y = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.y_f32 = 1;
  p.tiles = s.tiles;
  p.unit_subs = s.unit_subs;
  p.iters = s.iters;
  p.total = s.total;
  p.wgs = s.wgs;  // no workspace: the shares are added into y, none is exchanged
  return launch(vq::FMT_FP8, vq::EPI_ACC, p, stream);
}

int32_t vq_lmhead_argmax_accept(const uint16_t* h, const uint8_t* w, size_t w_bytes, float tensor_scale,
                                const int32_t* draft, int32_t lanes, int32_t R, int32_t V, int32_t K,
                                int32_t* argmax_out, float* maxlogit_out, int32_t* accept_len_out,
                                int32_t* commit_out, void* logits_out, int32_t logits_dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!h || !w || !argmax_out || !accept_len_out)
    return fail(VQ_ERR_NULL, "vq_lmhead_argmax_accept: h, w, argmax_out and accept_len_out are required");
  if (R > 1 && !draft) return fail(VQ_ERR_NULL, "draft is required when R > 1");
  if (lanes < 1 || lanes > 4) return fail(VQ_ERR_SHAPE, "lanes = %d outside [1, 4]", lanes);
  if (R < 1 || R > 8) return fail(VQ_ERR_SHAPE, "R = %d outside [1, 8]", R);
  if (logits_out && logits_dtype != VQ_OUT_BF16 && logits_dtype != VQ_OUT_F32)
    return fail(VQ_ERR_VALUE, "unknown logits_dtype %d", logits_dtype);
  const int32_t M = lanes * R;
  int32_t st = check_shape(M, V, K);
  if (st) return st;
  if (!aligned(h, 16)) return fail(VQ_ERR_ALIGN, "h must be 16-byte aligned");
  if (!aligned(argmax_out, 4) || !aligned(accept_len_out, 4) || (maxlogit_out && !aligned(maxlogit_out, 4)) ||
      (commit_out && !aligned(commit_out, 4)) || (draft && !aligned(draft, 4)))
    return fail(VQ_ERR_ALIGN, "int32/float arrays must be 4-byte aligned");
  if (logits_out && !aligned(logits_out, logits_dtype == VQ_OUT_F32 ? 4 : 2))
    return fail(VQ_ERR_ALIGN, "logits_out is not aligned to its element size");
  st = check_w(w, w_bytes, packed_bytes(VQ_PACK_NVFP4, V, K));
  if (st) return st;
  const vq::Schedule s = vq::make_schedule(vq::EPI_ARGMAX, V, K, M > 8);
  st = check_ws(s, workspace, workspace_bytes);
  if (st) return st;
  st = check_device();
  if (st) return st;
  vq::GemmParams p{};
  p.x = h;
  p.w = w;
  p.out_scale = tensor_scale;
  p.y = logits_out;
  p.y_f32 = logits_dtype == VQ_OUT_F32;
  p.M = M;
  p.N = V;
  p.K = K;
  p.draft = draft;
  p.lanes = lanes;
  p.R = R;
  p.argmax_out = argmax_out;
  p.maxlogit_out = maxlogit_out;
  p.accept_len_out = accept_len_out;
  p.commit_out = commit_out;
  bind_workspace(p, s, workspace);
  return launch(vq::FMT_NVFP4, vq::EPI_ARGMAX, p, stream);
}

int32_t vq_sample_accept(const float* logits, int32_t lanes, int32_t R, int32_t V, float temperature, int32_t top_k,
                         float top_p, const int32_t* draft, const int32_t* draft_ids, const float* draft_probs,
                         const float* u_accept, const float* u_draw, int32_t* token_out, int32_t* accept_len_out,
                         int32_t* commit_out, int32_t* cand_out, float* prob_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!logits || !u_draw || !accept_len_out)
    return fail(VQ_ERR_NULL, "vq_sample_accept: logits, u_draw and accept_len_out are required");
  if (lanes < 1 || lanes > 4) return fail(VQ_ERR_SHAPE, "lanes = %d outside [1, 4]", lanes);
  if (R < 1 || R > 8) return fail(VQ_ERR_SHAPE, "R = %d outside [1, 8]", R);
  if (V < 1 || V > vq::kMaxSampleV) return fail(VQ_ERR_SHAPE, "V = %d outside [1, %d]", V, vq::kMaxSampleV);
  if (R > 1 && !draft) return fail(VQ_ERR_NULL, "draft is required when R > 1");
  if ((draft_ids == nullptr) != (draft_probs == nullptr))
    return fail(VQ_ERR_NULL, "draft_ids and draft_probs go together (both or neither)");
  if (draft_ids && !u_accept) return fail(VQ_ERR_NULL, "u_accept is required with draft distributions");
  if (!(temperature > 0.0f) || !std::isfinite(temperature))
    return fail(VQ_ERR_VALUE, "temperature must be finite and > 0 (greedy verify is vq_lmhead_argmax_accept)");
  if (top_k < 1 || top_k > vq::kTopK) return fail(VQ_ERR_VALUE, "top_k = %d outside [1, %d]", top_k, vq::kTopK);
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(VQ_ERR_VALUE, "top_p must lie in (0, 1]");
  const void* arrays[] = {logits, draft, draft_ids, draft_probs, u_accept, u_draw,
                          token_out, accept_len_out, commit_out, cand_out, prob_out};
  for (const void* a : arrays)
    if (a && !aligned(a, 4)) return fail(VQ_ERR_ALIGN, "int32/float arrays must be 4-byte aligned");
  const int32_t M = lanes * R;
  const vq::SampleLayout L = vq::make_sample_layout(M, V);
  if (!workspace) return fail(VQ_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.bytes);
  if (!aligned(workspace, 16)) return fail(VQ_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < L.bytes)
    return fail(VQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.bytes);
  int32_t st = check_device();
  if (st) return st;
  char* base = static_cast<char*>(workspace);
  vq::SampleParams p{};
  p.logits = logits;
  p.M = M;
  p.V = V;
  p.lanes = lanes;
  p.R = R;
  p.chunks = L.chunks;
  p.temperature = temperature;
  p.top_k = top_k;
  p.top_p = top_p;
  p.draft = draft;
  p.q_ids = draft_ids;
  p.q_probs = draft_probs;
  p.u_accept = u_accept;
  p.u_draw = u_draw;
  p.token_out = token_out;
  p.accept_len_out = accept_len_out;
  p.commit_out = commit_out;
  p.cand_out = cand_out;
  p.prob_out = prob_out;
  p.cand = reinterpret_cast<unsigned long long*>(base + L.off_cand);
  p.row_ids = reinterpret_cast<int32_t*>(base + L.off_ids);
  p.row_probs = reinterpret_cast<float*>(base + L.off_probs);
  p.row_meta = reinterpret_cast<int32_t*>(base + L.off_meta);
  p.lane_count = reinterpret_cast<uint32_t*>(base + L.off_count);
  const int err = vq::launch_sample(p, stream);
  if (err != 0) return fail(VQ_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

}  // extern "C"

namespace {

int32_t gdn_call(const char* fn, const float* state_in, float* state_out, const float* q, const float* k,
                 const float* v, const float* a, const float* b, float* o, const int32_t* count, int32_t lanes,
                 int32_t B, int32_t T, int32_t H, int32_t Hk, void* stream) {
  if (!state_in || !state_out || !q || !k || !v || !a || !b)
    return fail(VQ_ERR_NULL, "%s: state_in, state_out, q, k, v, a and b are required", fn);
  if (B < 1 || T < 1 || T > vq::kGdnMaxT || H < 1 || Hk < 1 || Hk > H || H % Hk != 0 ||
      (int64_t)B * H > (1 << 24))
    return fail(VQ_ERR_SHAPE, "%s: B = %d, T = %d, H = %d, Hk = %d out of range (1 <= T <= %d, Hk divides H)", fn,
                B, T, H, Hk, vq::kGdnMaxT);
  if (lanes < 1 || lanes > 4 || B % lanes != 0)
    return fail(VQ_ERR_SHAPE, "%s: lanes = %d must lie in [1, 4] and divide B = %d", fn, lanes, B);
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(VQ_ERR_ALIGN, "%s: q and k must be 16-byte aligned", fn);
  const void* arrays[] = {state_in, state_out, v, a, b, o, count};
  for (const void* x : arrays)
    if (x && !aligned(x, 4)) return fail(VQ_ERR_ALIGN, "%s: fp32/int32 arrays must be 4-byte aligned", fn);
  const size_t sbytes = (size_t)B * H * vq::kGdnDk * vq::kGdnDv * sizeof(float);
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(state_in), o0 = reinterpret_cast<uintptr_t>(state_out);
  if (i0 < o0 + sbytes && o0 < i0 + sbytes) return fail(VQ_ERR_VALUE, "%s: state_in and state_out overlap", fn);
  int32_t st = check_device();
  if (st) return st;
  vq::GdnParams p{};
  p.state_in = state_in;
  p.state_out = state_out;
  p.q = q;
  p.k = k;
  p.v = v;
  p.a = a;
  p.b = b;
  p.o = o;
  p.count = count;
  p.B = B;
  p.T = T;
  p.H = H;
  p.Hk = Hk;
  p.lanes = lanes;
  const int err = vq::launch_gdn(p, stream);
  if (err) return fail(VQ_ERR_LAUNCH, "%s: kernel launch failed: %s", fn, hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

}  // namespace

extern "C" {

int32_t vq_gdn_verify(const float* state_in, float* state_out, const float* q, const float* k, const float* v,
                      const float* a, const float* b, float* o, int32_t B, int32_t T, int32_t H, int32_t Hk,
                      void* stream) {
  return gdn_call("vq_gdn_verify", state_in, state_out, q, k, v, a, b, o, nullptr, 1, B, T, H, Hk, stream);
}

int32_t vq_gdn_commit(const float* state_in, float* state_out, const float* q, const float* k, const float* v,
                      const float* a, const float* b, const int32_t* accept_len, int32_t lanes, int32_t B,
                      int32_t T, int32_t H, int32_t Hk, void* stream) {
  if (!accept_len) return fail(VQ_ERR_NULL, "vq_gdn_commit: accept_len is required");
  return gdn_call("vq_gdn_commit", state_in, state_out, q, k, v, a, b, nullptr, accept_len, lanes, B, T, H, Hk,
                  stream);
}

int32_t vq_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return fail(VQ_ERR_NULL, "vq_probe_copy: src and dst are required");
  if (bytes == 0 || bytes % 16) return fail(VQ_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(VQ_ERR_ALIGN, "src and dst must be 16-byte aligned");
  int32_t st = check_device();
  if (st) return st;
  const int err = vq::launch_probe_copy(src, dst, bytes, stream);
  if (err) return fail(VQ_ERR_LAUNCH, "probe launch failed: %s", hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

int32_t vq_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return fail(VQ_ERR_NULL, "vq_probe_read: src and sink are required");
  if (bytes == 0 || bytes % 16) return fail(VQ_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (!aligned(src, 16) || !aligned(sink, 16)) return fail(VQ_ERR_ALIGN, "src and sink must be 16-byte aligned");
  int32_t st = check_device();
  if (st) return st;
  const int err = vq::launch_probe_read(src, bytes, sink, stream);
  if (err) return fail(VQ_ERR_LAUNCH, "probe launch failed: %s", hipGetErrorString((hipError_t)err));
  return VQ_OK;
}

}  // extern "C"
