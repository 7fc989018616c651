/* libverify -- weight stream of the speculative-decoding verify pass on MI355X (gfx950).
 *
 * The verify pass runs the target model once over the anchor plus the drafted
 * tokens of each lane: an M x K activation block (M = 8 rows per lane, up to 4
 * lanes) against every projection of the model, which makes each projection a
 * skinny M x K x N GEMM rather than a GEMV ("144 tok/s needs 502 GB/s, and
 * Apple sells two M5 Max chips", sections "The decode step is one command
 * buffer" and "Why Apple silicon, and why not the M5"). The weights come in two
 * formats ("lithos-metal: per-layer megakernels ...", sections "What one token
 * costs the bus" and "Formats, and what runs where"):
 *   - NVFP4: 4-bit E2M1 codes, one E4M3 block scale per 16 consecutive K
 *     elements and one FP32 tensor scale that multiplies (9 bytes per 16
 *     weights) -- the MLP projections and the vocabulary head;
 *   - FP8 E4M3 codes with one FP32 per-tensor scale -- the Gated DeltaNet and
 *     attention projections.
 * Activations are bf16, accumulation is fp32 (weight-only quantisation).
 * The pass ends in the vocabulary head, a per-row argmax and the greedy accept
 * length ("lithos-metal ...", section "How DSpark is wired in").
 *
 * Weights are consumed in a packed layout that the library builds once from
 * the canonical layout (vq_pack_nvfp4 / vq_pack_fp8, at weight-load time; the
 * lithos-metal page, section "The control experiment the blog leaves out",
 * credits a weight layout packed for the memory bus).
 * Canonical layout: NVFP4 codes uint8 [rows][K/2], byte j of a row holds
 * element k = 2j in its low nibble and k = 2j+1 in its high nibble; scales
 * uint8 [rows][K/16] (E4M3FN: no infinities, NaN = S.1111.111, max 448), scale
 * byte b covers k in [16b, 16b+16). FP8 weights uint8 [rows][K] (E4M3FN).
 * Packed layout (bytes are moved, never changed): rows are cut into tiles of
 * 64 (four sub-tiles of 16 rows; for a fused SwiGLU [gate; up] matrix a tile
 * holds 32 gate rows and the 32 up rows of the same output columns), K into
 * iterations of 128, and each (tile, iteration) is one contiguous block, tiles
 * in order and iterations in order inside a tile.
 *   NVFP4 block, 4608 B: for sub-tile t and lane l = 16g + n, the 16 bytes at
 *   1024t + 16l are the code bytes of k 32j + 8g .. 32j + 8g + 7 (j = 0..3) of
 *   the sub-tile's row n; then for half h and row n, the 16 bytes at
 *   4096 + 16(16h + n) hold for each sub-tile t (4 bytes) the scales of blocks
 *   2j + h, j = 0..3 (block index inside the iteration).
 *   FP8 block, 8192 B: for sub-tile t, half h and lane l = 16g + n, the 16
 *   bytes at 1024(2t + h) + 16l are the weights of k 64h + 8g .. +7 and
 *   64h + 32 + 8g .. +7 of row n.
 * Rows past the matrix are zero. Sizes come from vq_packed_bytes().
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller; arrays are
 *     dense and row-major. The library never allocates, frees, synchronises or
 *     reads device memory on the host. Calls are asynchronous on `stream`
 *     (a hipStream_t; NULL is the default stream) and can be captured into a
 *     HIP graph.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Every argument is validated on the host before any HIP call; on error
 *     nothing is launched and a non-zero vq_status is returned, with detail in
 *     vq_last_error(). Shapes: 1 <= M <= 32, N >= 1, K >= 128 and K % 128 == 0.
 *     x, h, canonical and packed weights must be 16-byte aligned (every row
 *     then is); y and logits must be aligned to their element size; int32/f32
 *     arrays 4-byte aligned; the workspace 16-byte aligned. A packed size
 *     (w_bytes) smaller than the shape needs returns VQ_ERR_SHAPE.
 *   - workspace: device memory of at least vq_workspace_bytes(op, M, N, K)
 *     bytes, zero-filled by the caller ONCE before its first use. A workspace
 *     is BOUND to one (op, N, K): its layout (partial-sum slots, per-tile
 *     counters, argmax buckets, done counter) is placed from those three
 *     values, and a call with another op, N or K would find its counters on
 *     the previous shape's non-zero partial sums. Within that binding it
 *     serves every M (the size does not depend on M; the NVFP4 ops at M > 8
 *     may use a schedule of tile pairs, laid out in the same size, and every
 *     call leaves the counters zeroed). Kernels leave
 *     every counter in it at zero again, so a bound workspace can be reused
 *     by any number of stream-ordered calls (and graph replays); reusing it
 *     for another (op, N, K) requires zero-filling it again first. Two calls
 *     that may run concurrently need distinct workspaces. A NULL or short
 *     workspace returns VQ_ERR_WORKSPACE; the schedule never changes
 *     silently.
 *   - Results are deterministic: the K partition and the order of the fixed
 *     split-K reduction depend only on (N, K) and the epilogue, and for NVFP4
 *     on the family below, never on M otherwise. FP8 and affine 4-bit: row r
 *     of an M-row call equals row r of any other M bit for bit.
 *     NVFP4 has two compute families with different rounding (M <= 8: the
 *     block scale multiplies each block's fp32 partial sum; M > 8: the weights
 *     are scaled before the MFMA, exactly, and summed in fp32), and rows agree
 *     bit for bit within a family.
 *   - The first call on a device checks that it is gfx950 (VQ_ERR_DEVICE).
 *     A failed launch returns VQ_ERR_LAUNCH.
 *   - Thread-safe; vq_last_error() is per host thread.
 */
#ifndef LIBVERIFY_H
#define LIBVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQ_ABI_VERSION 8

typedef enum {
  VQ_OK = 0,
  VQ_ERR_NULL = 1,      /* a required pointer is NULL */
  VQ_ERR_SHAPE = 2,     /* M, N, K, lanes, R, V or a size out of range */
  VQ_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  VQ_ERR_WORKSPACE = 4, /* workspace NULL or smaller than vq_workspace_bytes() */
  VQ_ERR_DEVICE = 5,    /* no HIP device, or the current device is not gfx950 */
  VQ_ERR_LAUNCH = 6,    /* the kernel launch failed */
  VQ_ERR_VALUE = 7      /* an enum argument is unknown, or a sampling parameter
                           (temperature, top_k, top_p) is out of range */
} vq_status;

typedef enum { VQ_OUT_BF16 = 0, VQ_OUT_F32 = 1 } vq_out_dtype;
typedef enum { VQ_EPI_NONE = 0, VQ_EPI_SILU_MUL = 1 } vq_epilogue;
typedef enum {
  VQ_OP_NVFP4 = 0, VQ_OP_NVFP4_SILU_MUL = 1, VQ_OP_FP8 = 2, VQ_OP_LMHEAD = 3, VQ_OP_SAMPLE = 4,
  VQ_OP_AFFINE_Q4 = 5, VQ_OP_AFFINE_Q4_SILU_MUL = 6,
  VQ_OP_FP8_ACCUMULATE = 7 /* vq_gemm_fp8_accumulate: no workspace (schedule query only) */
} vq_op;
typedef enum {
  VQ_PACK_NVFP4 = 0, VQ_PACK_NVFP4_GATE_UP = 1, VQ_PACK_FP8 = 2,
  VQ_PACK_AFFINE_Q4 = 3, VQ_PACK_AFFINE_Q4_GATE_UP = 4
} vq_pack_kind;

/* Bytes of the packed form of a canonical matrix of `rows` rows and K columns
 * (VQ_PACK_NVFP4_GATE_UP: the fused [gate; up] matrix, rows = 2N, even).
 * Returns 0 for an invalid kind or shape. */
size_t vq_packed_bytes(int32_t kind, int32_t rows, int32_t K);

/* Pack a canonical NVFP4 matrix (codes [rows][K/2], scales [rows][K/16]) into
 * `packed` (at least vq_packed_bytes() bytes). gate_up = 1 packs a fused
 * SwiGLU [gate; up] matrix (rows = 2N) for VQ_EPI_SILU_MUL; 0 packs plain rows
 * (VQ_EPI_NONE and the vocabulary head). A one-time, bandwidth-bound copy on
 * `stream`; `packed` must not overlap the inputs. Returns a vq_status. */
int32_t vq_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, int32_t rows, int32_t K,
                      int32_t gate_up, uint8_t* packed, size_t packed_bytes, void* stream);

/* Pack a canonical FP8 E4M3 matrix w [rows][K] into `packed`. */
int32_t vq_pack_fp8(const uint8_t* w, int32_t rows, int32_t K, uint8_t* packed, size_t packed_bytes,
                    void* stream);

/* NVFP4 skinny GEMM: Y[M][N] = X[M][K] . W^T with
 *   W[n][k] = E2M1(code[n][k]) * E4M3(scale[n][k/16]) * tensor_scale
 * (formats: "lithos-metal ...", sections "What one token costs the bus" and
 * "Formats, and what runs where"; 9 bytes per 16 weights).
 *   x       bf16 [M][K]
 *   w       packed weights, w_bytes bytes
 *   epilogue VQ_EPI_NONE:     w = vq_pack_nvfp4(gate_up = 0) of W [N][K]
 *            VQ_EPI_SILU_MUL: w = vq_pack_nvfp4(gate_up = 1) of the fused
 *            [2N][K] matrix whose rows [0,N) are the SwiGLU gate and rows
 *            [N,2N) the up projection; Y = silu(gate) * up with silu(g) =
 *            g / (1 + exp(-g)), computed in fp32 before the single rounding of
 *            the store ("144 tok/s ...", section "The engine hard-codes the
 *            model": SwiGLU gate, up, down).
 *   y       [M][N], bf16 (round to nearest even) or fp32 per y_dtype.
 * Returns a vq_status. */
int32_t vq_gemm_nvfp4(const uint16_t* x, const uint8_t* w, size_t w_bytes,
                      float tensor_scale, void* y, int32_t y_dtype,
                      int32_t M, int32_t N, int32_t K, int32_t epilogue,
                      void* workspace, size_t workspace_bytes, void* stream);

/* vq_gemm_nvfp4 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Arguments, results and rounding are those
 * of vq_gemm_nvfp4 (the same kernels and split-K schedule, so the outputs are
 * bitwise equal); the partial sums and per-tile counters live in a static
 * device array of the library, one per device, 256 KiB + 8 MiB
 * (8,650,752 bytes), allocated when the library's code is loaded on the device
 * and held until the process ends. Limits: N <= 4,194,304 output columns
 * (2,097,152 with VQ_EPI_SILU_MUL); larger N returns VQ_ERR_SHAPE. Every call
 * on a device shares that device's array and leaves its counters at zero, so
 * stream-ordered calls of any shape may follow each other, but calls that may
 * overlap on one device (concurrent streams, graph branches) race on it and
 * must use vq_gemm_nvfp4 with distinct workspaces instead. The call never
 * allocates, frees or synchronises. */
int32_t vq_gemm_nvfp4_noalloc(const uint16_t* x, const uint8_t* w, size_t w_bytes,
                              float tensor_scale, void* y, int32_t y_dtype,
                              int32_t M, int32_t N, int32_t K, int32_t epilogue, void* stream);

/* Affine 4-bit weights ("144 tok/s needs 502 GB/s ...", section "The engine
 * hard-codes the model": per group of 64 inputs, 32 bytes of nibbles plus a
 * bf16 scale and a bf16 bias, 9 bytes per 16 weights; "lithos-metal ...",
 * section "Formats, and what runs where": the MLX/AWQ/GPTQ affine INT4
 * layout):  W[n][k] = scale[n][k/64] * q[n][k] + bias[n][k/64], q the unsigned
 * nibble 0..15.
 * Canonical layout: codes uint8 [rows][K/2] (low nibble = even k, as for
 * NVFP4); scales and biases bf16 bit patterns uint16 [rows][K/64].
 * Packed layout: the NVFP4 block (4608 B per 64 rows x 128 K) with the same
 * 4096 B of code dwords, each holding its 8 codes (k0..k7) as k0 k2 k4 k6 in
 * bits 0-15 and k1 k3 k5 k7 in bits 16-31 (4 bits each, ascending), then for
 * row n of the tile the 32 bytes at 4096 + 32n:
 * for sub-tile t = 0..3 and group h = 0, 1 of the iteration one dword
 * holding scale (low half) and bias (high half). gate_up = 1 pairs gate and
 * up rows exactly as vq_pack_nvfp4 does. */
int32_t vq_pack_affine_q4(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                          int32_t rows, int32_t K, int32_t gate_up, uint8_t* packed,
                          size_t packed_bytes, void* stream);

/* Affine 4-bit skinny GEMM: Y[M][N] = X . W^T, with epilogue VQ_EPI_NONE or
 * VQ_EPI_SILU_MUL (w from vq_pack_affine_q4 with gate_up = 0 / 1, as for
 * vq_gemm_nvfp4). The bias term uses the per-group sums of X, formed by the
 * matrix unit next to the products ("Beating Splash on an M5 Max ...",
 * section "What actually moved the needle": the Q4 tiles need per-group
 * input sums). y [M][N] bf16 or fp32. Workspace:
 * vq_workspace_bytes(VQ_OP_AFFINE_Q4[_SILU_MUL], M, N, K). */
int32_t vq_gemm_affine_q4(const uint16_t* x, const uint8_t* w, size_t w_bytes, void* y,
                          int32_t y_dtype, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                          void* workspace, size_t workspace_bytes, void* stream);

/* FP8 skinny GEMM: Y[M][N] = (X[M][K] . E4M3(w)^T) * w_scale
 * ("lithos-metal ...", section "What one token costs the bus": every Gated
 * DeltaNet and attention projection is FP8 with a scalar scale).
 *   x bf16 [M][K]; w = vq_pack_fp8 of the E4M3FN codes [N][K] (w_bytes
 *   bytes); y [M][N] bf16 or fp32. */
int32_t vq_gemm_fp8(const uint16_t* x, const uint8_t* w, size_t w_bytes, float w_scale,
                    void* y, int32_t y_dtype, int32_t M, int32_t N, int32_t K,
                    void* workspace, size_t workspace_bytes, void* stream);

/* FP8 skinny GEMM added into an fp32 output: Y[M][N] += (X . E4M3(w)^T) *
 * w_scale. Same operands and shapes as vq_gemm_fp8 (x bf16 [M][K], 16-byte
 * aligned; w from vq_pack_fp8 of [N][K]); y fp32 [M][N], 4-byte aligned. No
 * workspace. The split-K reduction is done by the additions themselves: the
 * output columns are worked in units of 32, the schedule gives every unit
 * at most two workgroup shares, and each share is added with one fp32
 * atomic add per element, so no workgroup waits for another ("Beating
 * Splash on an M5 Max ...", section "The kernels were not the gap": split-K
 * on the narrow projections, here with a reduction whose result does not
 * depend on arrival order). With y zero on entry the result is
 * deterministic (0 + a + b = 0 + b + a: bitwise the same on every call);
 * a nonzero y is added to, but the order of a unit's two shares is then not
 * fixed. Meant for the narrow projections (N <= 5,440 fills the CUs with
 * three workgroups per 64 columns); any N up to the vq_gemm_fp8 limits is
 * accepted. */
int32_t vq_gemm_fp8_accumulate(const uint16_t* x, const uint8_t* w, size_t w_bytes, float w_scale,
                               float* y, int32_t M, int32_t N, int32_t K, void* stream);

/* Vocabulary head + per-row argmax + greedy accept, all on the device
 * ("Beating Splash on an M5 Max ...", section "What actually moved the
 * needle": acceptance runs on the GPU and writes a small result block;
 * "lithos-metal ...", section "How DSpark is wired in": the accept scan).
 *   h       bf16 [M][K] hidden rows, M = lanes * R; rows l*R .. l*R+R-1
 *           belong to lane l (row 0 of a lane follows its anchor token)
 *   w, w_bytes, tensor_scale: the NVFP4 head W_head [V][K], packed with
 *           vq_pack_nvfp4(gate_up = 0)
 *   draft   int32 [lanes][R-1]: draft j of lane l is compared with the argmax
 *           of row l*R + j. Ids are not validated; an id outside [0,V) never
 *           matches, and a row whose argmax is -1 matches no draft.
 *   argmax_out     int32 [M]: lowest index among the equal maximal fp32 logits
 *                  (-0 equals +0; NaN is never selected; -1 if a row has no
 *                  non-NaN logit)
 *   maxlogit_out   float [M] or NULL: the maximal logit (NaN for a -1 row)
 *   accept_len_out int32 [lanes]: 1 + length of the matched draft prefix, in [1, R]
 *   commit_out     int32 [lanes][R] or NULL: committed tokens (the argmax of
 *                  rows 0..accept_len-1 of the lane), -1 after them
 *   logits_out     [M][V] bf16 or fp32 per logits_dtype, or NULL
 * Shapes: 1 <= lanes <= 4, 1 <= R <= 8, 1 <= V <= 2^30, K as above. */
int32_t vq_lmhead_argmax_accept(const uint16_t* h, const uint8_t* w, size_t w_bytes,
                                float tensor_scale, const int32_t* draft,
                                int32_t lanes, int32_t R, int32_t V, int32_t K,
                                int32_t* argmax_out, float* maxlogit_out,
                                int32_t* accept_len_out, int32_t* commit_out,
                                void* logits_out, int32_t logits_dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Sampled verify over the fp32 verify logits (nonzero temperature): per row
 * the target's distribution, a draw from it, and the accept scan per lane.
 * ("144 tok/s needs 502 GB/s ...", section "Exact, up to top-32": the
 * distribution is temperature over the row's first top_k <= 32 logits,
 * truncated by top_p and renormalised, and acceptance is the speculative-
 * sampling test u*q < p with a draw from max(p - q, 0) on rejection;
 * "Beating Splash on an M5 Max ...", section "What actually moved the
 * needle": top-k, top-p, sampling and acceptance run on the GPU and write a
 * small result block; "lithos-metal ...", section "How DSpark is wired in":
 * the point-mass case, where the draft token is accepted only when it equals
 * the target's draw.)
 *   logits   fp32 [M][V], M = lanes * R, rows grouped by lane as in
 *            vq_lmhead_argmax_accept (its logits_out in VQ_OUT_F32)
 *   temperature > 0 and finite; 1 <= top_k <= 32; 0 < top_p <= 1
 *   Per row: candidates in logit order (equal logits by lower id, -0 == +0,
 *   NaN never a candidate); w_i = exp((z_i - z_0) / temperature) over the
 *   first top_k; kept = the shortest prefix whose weight reaches top_p of the
 *   total (zero weights dropped); probabilities w_i / sum(kept). A row whose
 *   top logit is not finite has no distribution (draw -1, kept count 0).
 *   u_draw   fp32 [M] uniforms in [0, 1): row r's draw is the first kept
 *            candidate whose cumulative weight exceeds u_draw[r] of the kept
 *            weight (the last kept one if none)
 *   draft    int32 [lanes][R-1] drafted tokens (draft j of lane l is checked
 *            at row l*R + j); required when R > 1
 *   draft_ids, draft_probs  int32 / fp32 [lanes][R-1][16], or both NULL.
 *            NULL selects the point-mass rule: draft j is accepted when it
 *            equals row j's draw, and the first differing draw is the bonus.
 *            Given, they are the draft's distribution q_j for row j (id -1 =
 *            empty slot; the first pair with a matching id counts; other
 *            tokens have q = 0) and the speculative-sampling rule applies:
 *            accept draft j when u_accept[row] * q_j(d_j) < p_j(d_j); on the
 *            first rejection the token is drawn with u_draw[row] from
 *            max(p_j - q_j, 0) over the kept candidates (from p_j when that
 *            has no mass). With every draft accepted the bonus is the last
 *            row's draw.
 *   u_accept fp32 [M] uniforms (speculative-sampling rule only; entries of
 *            the last row of a lane are not read)
 *   token_out      int32 [M] or NULL: each row's draw (-1: no distribution)
 *   accept_len_out int32 [lanes]: committed tokens, in [1, R]
 *   commit_out     int32 [lanes][R] or NULL: committed tokens, -1 after them
 *                  (and for a row without a distribution, which ends the scan)
 *   cand_out, prob_out int32 / fp32 [M][32] or NULL: the kept candidates and
 *                  their probabilities per row, -1 / 0 after the kept count
 * Uniforms outside [0, 1) give unspecified tokens (never a fault). Shapes:
 * 1 <= lanes <= 4, 1 <= R <= 8, 1 <= V <= 2^20. Workspace:
 * vq_workspace_bytes(VQ_OP_SAMPLE, M, V, 0). Two launches on `stream`;
 * arithmetic is fp32 with sums in a fixed order (deterministic). */
int32_t vq_sample_accept(const float* logits, int32_t lanes, int32_t R, int32_t V,
                         float temperature, int32_t top_k, float top_p,
                         const int32_t* draft, const int32_t* draft_ids, const float* draft_probs,
                         const float* u_accept, const float* u_draw,
                         int32_t* token_out, int32_t* accept_len_out, int32_t* commit_out,
                         int32_t* cand_out, float* prob_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Gated DeltaNet state stream of the verify pass, out of place between two
 * parity slots of the fp32 recurrent state ("Beating Splash on an M5 Max
 * ...", section "What actually moved the needle": the fused GDN step writes
 * from parity buffer A to B, a fully accepted round flips the parity, a
 * partly rejected one re-scans only the committed rows from the intact
 * previous parity; "lithos-metal ...", section "What one token costs the
 * bus": the state is fp32 (v_heads, dk, dv) = (48, 128, 128) per GDN layer,
 * read and written once per pass; section "How DSpark is wired in": the
 * commit pass recomputes the recurrence from the slot the verify read over
 * the committed tokens, whose count the accept scan wrote). The pages print
 * no recurrence; it is the gated delta rule of Yang, Kautz and Hatamizadeh,
 * "Gated Delta Networks: Improving Mamba2 with Delta Rule" (ICLR 2025), per
 * value head in the (dk, dv) layout:
 *     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t
 * Queries, keys and values arrive already convolved and normalised, and the
 * decays a_t and write strengths b_t already computed: the 4-tap
 * convolution, the Q/K norm and the gate formulas are not part of this call.
 *
 * B entries (e.g. layers x lanes, entry-major with entry e = layer * lanes +
 * lane) of T rows each; dk = dv = 128; H value heads share Hk key heads
 * (Hk divides H; value head h reads key head h / (H / Hk)).
 *   state_in   fp32 [B][H][128][128]: the slot read (never written)
 *   state_out  fp32 [B][H][128][128]: the slot written; must not overlap
 *              state_in
 *   q, k       fp32 [B][T][Hk][128], 16-byte aligned
 *   v          fp32 [B][T][H][128]
 *   a, b       fp32 [B][T][H]: decay and write strength of each row and head
 *   o          fp32 [B][T][H][128] or NULL: the output of every row; must
 *              not overlap any other array of the call
 * Shapes: 1 <= B, 1 <= T <= 16, 1 <= Hk <= H, H % Hk == 0, B * H <= 2^24.
 * All arrays 4-byte aligned (q, k 16-byte). One launch on `stream`, no
 * workspace; fp32 arithmetic with every sum in a fixed order, and the row
 * partition does not depend on B, so an entry's result is bitwise the same
 * whatever B is.
 *
 * vq_gdn_verify: every entry scans all T rows from state_in, writes the
 * final state to state_out and, when o is given, the T outputs. */
int32_t vq_gdn_verify(const float* state_in, float* state_out, const float* q, const float* k,
                      const float* v, const float* a, const float* b, float* o,
                      int32_t B, int32_t T, int32_t H, int32_t Hk, void* stream);

/* vq_gdn_commit: the commit pass after the accept scan. Entry e belongs to
 * lane e % lanes and c = accept_len[lane] (device int32 [lanes], as written
 * by vq_lmhead_argmax_accept or vq_sample_accept), clamped to [0, T]. An
 * entry with c = T is left alone (state_out already holds what
 * vq_gdn_verify wrote); any other entry gets the scan of its first c rows
 * from state_in (c = 0 copies it). The inputs are the same arrays the verify
 * call read. For each entry the result is bitwise what vq_gdn_verify over
 * those c rows writes (the rollback identity). 1 <= lanes <= 4, B % lanes
 * == 0; other shapes as above. */
int32_t vq_gdn_commit(const float* state_in, float* state_out, const float* q, const float* k,
                      const float* v, const float* a, const float* b, const int32_t* accept_len,
                      int32_t lanes, int32_t B, int32_t T, int32_t H, int32_t Hk, void* stream);

/* Workspace bytes needed by `op` at this shape (for VQ_OP_NVFP4_SILU_MUL, N is
 * the output width, i.e. half the weight rows; for VQ_OP_LMHEAD, N = V and
 * M = lanes * R). Returns 0 for an invalid shape. The size does not depend
 * on M beyond the M <= 32 bound, so a workspace bound to one (op, N, K)
 * serves every M; for VQ_OP_SAMPLE, N = V, K is ignored, the size grows
 * with M, and the per-lane counters sit at an offset placed from (M, V), so a
 * sampling workspace is bound to one (M, V). */
size_t vq_workspace_bytes(int32_t op, int32_t M, int32_t N, int32_t K);

/* The split-K / stream-K schedule a call of `op` (not VQ_OP_SAMPLE) uses at
 * (M, N, K), for inspection and host-side checks ("Beating Splash on an M5
 * Max ...", section "The kernels were not the gap": split-K on the narrow
 * projections). The iteration space is units x iterations, W = units * (K /
 * 128); workgroup g of G owns iterations [g W / G, (g + 1) W / G), unit-major.
 * A unit is a 64-row tile of the packed weights (64 output columns, 32 with
 * SILU_MUL); for VQ_OP_FP8_ACCUMULATE half a tile (32 output columns), and
 * then no unit is shared by more than two workgroups; for the NVFP4 ops
 * (VQ_OP_NVFP4, VQ_OP_NVFP4_SILU_MUL, VQ_OP_LMHEAD) at M > 8 on outputs of
 * at least 2,048 tiles, a pair of adjacent tiles (the last one alone when the
 * tile count is odd). M enters only through that choice (M <= 8 or
 * M > 8). Writes units, iterations per unit and G; returns VQ_OK, or
 * VQ_ERR_NULL / VQ_ERR_SHAPE / VQ_ERR_VALUE. */
int32_t vq_schedule_info(int32_t op, int32_t M, int32_t N, int32_t K, int32_t* units, int32_t* iters,
                         int32_t* workgroups);

const char* vq_status_str(int32_t status);
const char* vq_last_error(void);
int32_t vq_abi_version(void);

/* HBM probes used as the measured bandwidth denominator.
 * vq_probe_copy: dst[i] = src[i] for `bytes` bytes (multiple of 16, both
 * 16-byte aligned). vq_probe_read: reads `bytes` bytes of src and writes one
 * 16-byte value derived from them to sink (keeps the reads live). */
int32_t vq_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int32_t vq_probe_read(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBVERIFY_H */
