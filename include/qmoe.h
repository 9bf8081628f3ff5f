/*
 * qmoe.h — C ABI of libqmoe: ROCmFPX block-quantized MoE layers on MI355X (gfx950).
 *
 * Page citations:
 *   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
 *                AMD Ryzen AI MAX+ 395", sections "ROCmFPX: fitting 284B weights
 *                into 128 GB" and "Decode: up to 32 tok/s".
 *   [0731-Strix] lucebox.com, "Lucebox × Geometric: DeepSeek V4 Flash 0731
 *                reaches 32.7 tok/s on AMD Strix Halo", sections "How the model
 *                fits on AMD Strix Halo", "Lucebox Engine integration with
 *                Geometric" and "Run with Lucebox Engine".
 *   [evox3]      soothill.io, "DeepSeek V4 Flash 0731 on evox3", introduction and
 *                table "The optimization ladder".
 *
 * Data formats (normative for both this library and its CPU checker):
 *   A block is 32 consecutive weights of one row ([Strix-284B], ROCmFPX section).
 *   FP2: 8 B of 2-bit codes + fp16 scale = 10 B (2.50 bpw).
 *        Code of weight j: byte 4*(j>>4) + (j&3), bits 2*((j>>2)&3)..+1.
 *   FP3: FP2-style plane of the low 2 code bits (8 B) + 4 B plane of bit 2
 *        (weight j: byte j&3, bit j>>2) + fp16 scale = 14 B (3.50 bpw).
 *   FP4: 16 B of nibbles (weight j: byte 4*(j>>3) + (j&3), bits 4*((j>>2)&1)..+3)
 *        + E8M0 scale byte e (value 2^(e-127), e = 255 invalid) = 17 B (4.25 bpw).
 *   Rows are row-planar: all code planes of the row (block-major), then the FP3
 *   high planes, then the scales (little-endian fp16 or E8M0 bytes).
 *   Codebooks: int8, 2^bits entries per (tensor, expert); dequantized weight =
 *   scale * C[code] ([0731-Strix]: learned per-expert codebooks).
 *   Activations: per 32-block, optional H32 (Sylvester FWHT, butterflies
 *   h = 1..16, then * fp32(1/sqrt(32))), d = amax/127 (zero or subnormal d:
 *   block stored as zero), q = clamp(rint(v * (1/d)), -127, 127).
 *
 * Conventions:
 *   - Every pointer argument of a launch entry point is a DEVICE pointer unless
 *     the comment says host. The caller owns all memory; the library never
 *     allocates, frees or keeps a pointer after the call returns, and never
 *     synchronises the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Launch entry points are asynchronous on that stream.
 *   - Every entry point returns a qmoe_status. Argument errors are detected on the
 *     host before any launch ([0731-Strix] integration section: codebooks are
 *     validated before serving starts; [evox3] introduction: an unsupported
 *     rotation must fail at load, not mid-run). A message naming the argument is
 *     available from qmoe_last_error() (thread-local).
 *   - No C++ exception crosses this ABI.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMOE_OK = 0,
  QMOE_E_INVAL = -1,     /* NULL pointer, bad enum value, bad flag            */
  QMOE_E_SHAPE = -2,     /* K % 32 != 0, q not in 1..4, topk not in 1..min(E,8),
                            E > 512, hidden > 8192, rows not 16-byte multiples */
  QMOE_E_FORMAT = -3,    /* unknown format or unsupported format/rotation pair */
  QMOE_E_CODEBOOK = -4,  /* missing / truncated / mismatched codebook bytes     */
  QMOE_E_SCALE = -5,     /* non-finite fp16 scale or E8M0 0xFF (pack)           */
  QMOE_E_WORKSPACE = -6, /* workspace missing or smaller than required          */
  QMOE_E_HIP = -7,       /* a HIP runtime call or launch failed                 */
  QMOE_E_SIZE = -8       /* a weight buffer is smaller than its shape requires  */
} qmoe_status;

typedef enum { QMOE_FP2 = 2, QMOE_FP3 = 3, QMOE_FP4 = 4 } qmoe_format;

/* Human-readable name of a status code (static string). */
const char* qmoe_strerror(int status);
/* Detail of the last error on this thread (static thread-local buffer). */
const char* qmoe_last_error(void);
/* ABI version (major * 100 + minor). */
int qmoe_version(void);

/* Bytes per 32-weight block: 10, 14, 17; 0 for an unknown format
 * ([Strix-284B] ROCmFPX section: 2.50 / 3.50 / 4.25 bits per weight). */
size_t qmoe_block_bytes(int fmt);
/* rows * (k/32) * block bytes; 0 if k % 32 != 0 or the format is unknown. */
size_t qmoe_packed_bytes(int fmt, int64_t rows, int64_t k);

/* HOST (CPU only). Packs codes (host uint8 [rows*k], each < 2^bits) and scales
 * (host; uint16 fp16 bits [rows*k/32] for FP2/FP3, uint8 E8M0 [rows*k/32] for
 * FP4) into `out` (host, out_bytes >= qmoe_packed_bytes), in the row-planar
 * block layout above. The pages fix only the block: 32 weights as packed
 * low-bit codes plus a small scale in 10, 14 or 17 bytes, with a file layout
 * designed together with the kernel that reads it ([Strix-284B], ROCmFPX
 * section); the bit positions are this library's. Rejects codes out of range
 * (QMOE_E_INVAL), non-finite fp16 or E8M0 0xFF scales (QMOE_E_SCALE), k not a
 * multiple of 32 (QMOE_E_SHAPE), out_bytes too small (QMOE_E_SIZE). */
int qmoe_pack(int fmt, int64_t rows, int64_t k, const uint8_t* codes,
              const void* scales, void* out, size_t out_bytes);
/* HOST. Inverse of qmoe_pack (same passage): codes (host uint8 [rows*k]) and
 * scales (host, as for qmoe_pack) from packed rows (host, packed_bytes >=
 * qmoe_packed_bytes). Errors as qmoe_pack; the scales are not re-validated. */
int qmoe_unpack(int fmt, int64_t rows, int64_t k, const void* packed,
                size_t packed_bytes, uint8_t* codes, void* scales);

/* One top-k SwiGLU MoE layer ([Strix-284B] ROCmFPX section: routed gate/up in
 * the 2.5-bit format, down in the 3.5-bit format; [0731-Strix] run section:
 * 256 experts, 6 routed). All pointers are device pointers.
 *   gate, up: [E][inter][row_bytes(fmt, hidden)];  down: [E][hidden][row_bytes(fmt, inter)]
 *   cb_*:     [E][2^bits(fmt)] int8
 *   w_router: fp16 bits [E][hidden];  router_bias: fp64 [E] or NULL (= 0)
 *   rot_gateup / rot_down: 0 = none, 1 = H32 on the input blocks of gate/up
 *   (the token) or of down (the SwiGLU output). */
typedef struct {
  int32_t hidden, inter, n_experts, topk;
  int32_t fmt_gate, fmt_up, fmt_down;
  int32_t rot_gateup, rot_down;
  const uint16_t* w_router; size_t w_router_bytes;
  const double* router_bias;
  const void* gate; size_t gate_bytes;
  const void* up;   size_t up_bytes;
  const void* down; size_t down_bytes;
  const int8_t* cb_gate; size_t cb_gate_bytes;
  const int8_t* cb_up;   size_t cb_up_bytes;
  const int8_t* cb_down; size_t cb_down_bytes;
} qmoe_layer;

/* HOST check of a layer descriptor (no device access), the load-time
 * validation of [0731-Strix], integration section (codebooks that are missing,
 * truncated or mismatched are refused before serving starts) and of [evox3],
 * introduction (a rotation the kernels do not implement must be refused at
 * load, not at layer 3, expert 7 of a running server). Checks: shapes and
 * limits (QMOE_E_SHAPE); format and rotation values, gate/up format equality
 * (QMOE_E_FORMAT); NULL weights, weights or router not 16-byte aligned,
 * codebooks not 4-byte aligned, bias not 8-byte aligned (QMOE_E_INVAL); weight
 * or router buffers shorter than their shapes (QMOE_E_SIZE); codebooks NULL
 * (missing), shorter (truncated) or longer (mismatched) than E * 2^bits bytes
 * (QMOE_E_CODEBOOK). Each expert's codebook is a separate array slot, so a
 * duplicated entry cannot arise in this descriptor. */
int qmoe_layer_check(const qmoe_layer* L);

/* Bytes of device workspace needed by qmoe_route / qmoe_decode_layer /
 * qmoe_prefill_layer for up to `max_tokens` tokens (0 on an invalid layer).
 * The workspace needs no initialisation: every call writes each region before
 * it reads it, and its contents are scratch between calls. Calls that share a
 * workspace must be ordered (same stream or synchronised). */
size_t qmoe_workspace_bytes(const qmoe_layer* L, int32_t max_tokens);

/* Router only: logits in fp64 in a fixed order (per block sequential, then a
 * stride-halving tree over blocks, + bias), top-k with ties to the lower id,
 * ids ascending, softmax over the k selected logits. x: fp32 [ntok][hidden];
 * idx: int32 [ntok][topk]; gate_w: fp32 [ntok][topk].
 * ([Strix-284B] decode section: dedicated top-k / argsort routing kernels.) */
int qmoe_route(const qmoe_layer* L, const float* x, int32_t ntok, int32_t* idx,
               float* gate_w, void* ws, size_t ws_bytes, void* stream);

/* Decode: q = 1..4 independent tokens (verification columns). Each packed
 * block of every expert selected by any of the q tokens is read and expanded
 * once and applied to each column routed to it ([Strix-284B] decode section).
 * x: fp32 [q][hidden]; out: fp32 [q][hidden]. No host synchronisation. */
int qmoe_decode_layer(const qmoe_layer* L, const float* x, int32_t q, float* out,
                      void* ws, size_t ws_bytes, void* stream);

/* The same decode with the expert products on the int8 matrix cores
 * (v_mfma_i32_4x4x4_16b_i8: the q <= 4 tokens are the instruction's 4
 * columns, 4 weight rows its rows, 16 consecutive 32-weight blocks its 16
 * blocks), each packed block still read and expanded once for all q columns
 * ([Strix-284B] decode section; the routed experts' products with q padded to
 * the matrix core's width). Per-block int32 sums are exact as on the dot4 path;
 * the fp32 accumulation runs in an order of its own, so results agree with
 * qmoe_decode_layer within the layer tolerance, not bit for bit, and column t
 * of a q-token call equals a one-token call of this function bit for bit.
 * Arguments, workspace and errors as qmoe_decode_layer; in addition hidden and
 * inter must be multiples of 512 with hidden <= 8192 and inter <= 2048, and
 * q * topk routed slots of inter/32 blocks must fit the down kernel's 64 KB of
 * staged activations, else QMOE_E_SHAPE before any launch. */
int qmoe_decode_layer_mfma(const qmoe_layer* L, const float* x, int32_t q, float* out,
                           void* ws, size_t ws_bytes, void* stream);

/* Decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * computation and kernels as qmoe_decode_layer, but the workspace is a fixed
 * device array inside the library, qmoe_decode_noalloc_max_bytes() (4 MiB) on
 * each GPU, held until the process ends; no call allocates or frees anything.
 * Its device address is looked up once per device (hipGetSymbolAddress, with
 * that device current). Every call on one GPU shares that GPU's array and
 * leaves its contents behind (nothing in it needs clearing between calls):
 * calls that overlap on one GPU (unordered streams, several host threads)
 * race on it and give undefined results. x, out, q, stream and errors as
 * qmoe_decode_layer; a layer whose decode workspace at q tokens exceeds the
 * array is refused before any launch (QMOE_E_WORKSPACE). */
size_t qmoe_decode_noalloc_max_bytes(void);
int qmoe_decode_layer_noalloc(const qmoe_layer* L, const float* x, int32_t q, float* out,
                              void* stream);

/* Prefill: ntok tokens through the layer, grouped by expert on the device
 * ([evox3] ladder: layer-major prefill batching). x: fp32 [ntok][hidden];
 * out: fp32 [ntok][hidden]. Deterministic: per token the expert outputs are
 * combined in ascending expert id. hidden and inter must be multiples of 256
 * (the GEMM tiles: 128 rows, K in stages of 256), else QMOE_E_SHAPE.
 * Experts are multiplied in 64-pair tiles on the int8 matrix cores; experts
 * with at most QMOE_PREFILL_SMALL_DEFAULT pairs in the batch take the matvec
 * path instead (see qmoe_prefill_layer_ex). */
int qmoe_prefill_layer(const qmoe_layer* L, const float* x, int32_t ntok, float* out,
                       void* ws, size_t ws_bytes, void* stream);

/* qmoe_prefill_layer with the expert split as an argument: experts that 1 ..
 * small_pairs (0..4) pairs of the batch route to go through the decode path's
 * matvec arithmetic (each block expanded once by byte permutes, sdot4 against
 * every pair) instead of a 64-pair MFMA tile that would be mostly padding
 * ([evox3] ladder: the multi-token expert path next to the layer-major batch).
 * 0 sends every expert to the tiles. The default (2) was the best or near it
 * over batches of 32 .. 8192 tokens on MI355X, with and without Zipf-skewed
 * routing: where every expert gets a handful of pairs the matvec path is up to
 * 18% faster, at 8K it is within the run-to-run spread (the MFMA GEMMs are
 * vector-ALU bound, so a padded tile's weight stream costs little there).
 * Within a path a pair's result does not
 * depend on the other tokens of the batch; the two paths round differently, so
 * a token whose expert changes path between two batches can differ in the last
 * bits (both within the layer's parity bar). small_pairs outside 0..4:
 * QMOE_E_INVAL; other arguments and errors as qmoe_prefill_layer. */
#define QMOE_PREFILL_SMALL_DEFAULT 2
int qmoe_prefill_layer_ex(const qmoe_layer* L, const float* x, int32_t ntok, float* out,
                          void* ws, size_t ws_bytes, int32_t small_pairs, void* stream);

/* Expand-then-multiply form of qmoe_matvec, the comparison path for the fused
 * kernel ([0731-Strix], section "Lucebox Engine integration with Geometric":
 * the fused 3.5-bit matrix-vector kernel against the generic expand-then-
 * multiply fallback). It first writes every block of w as 32 int8 weights and
 * an fp32 scale into the workspace, then multiplies the expanded matrix with
 * the same lane mapping and accumulation order as qmoe_matvec, so y equals
 * qmoe_matvec's output bit for bit. Arguments and errors as qmoe_matvec; ws:
 * qmoe_matvec_expanded_workspace_bytes(rows, k, ncols) bytes, 16-byte aligned,
 * caller-owned, scratch after the call. */
size_t qmoe_matvec_expanded_workspace_bytes(int64_t rows, int64_t k, int32_t ncols);
int qmoe_matvec_expanded(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes,
                         const int8_t* cb, int32_t rot, const float* x, int32_t ncols, float* y,
                         void* ws, size_t ws_bytes, void* stream);

/* One matrix of qmoe_matvec_group: arguments as qmoe_matvec's. */
typedef struct {
  int32_t fmt, rot;
  int64_t rows, k;
  const void* w; size_t w_bytes;
  const int8_t* cb;
  const float* x;   /* fp32 [ncols][k], 16-byte aligned */
  float* y;         /* fp32 [ncols][rows] */
} qmoe_matvec_item;

/* The matrix-vector products of n (1..4) matrices with the same number of
 * columns in one launch when ncols <= 2 and every input holds at most 512
 * blocks per call (ncols x k / 32; each workgroup quantizes its matrix's input
 * into LDS, then multiplies), else in two launches (all inputs quantized, then
 * all rows multiplied, each workgroup reading its matrix's quantized input from
 * LDS when every input holds at most 2048 blocks per call):
 * the dense projections of a decode step ([Strix-284B], decode section: the
 * dense 4-bit weights of a step decoded once for all of its columns; [evox3],
 * table "The optimization ladder": the fused H32 matrix-vector path), where
 * one qmoe_matvec per matrix pays a launch per matrix and one more for each
 * long input's quantization. Each y equals qmoe_matvec's output for the same
 * item bit for bit. ws:
 * qmoe_matvec_group_workspace_bytes bytes, 16-byte aligned, caller-owned,
 * scratch after the call (it holds the quantized inputs, item after item, each
 * as qmoe_matvec's workspace does). Errors before any launch: as qmoe_matvec
 * per item, n or ncols outside their ranges (QMOE_E_SHAPE). */
size_t qmoe_matvec_group_workspace_bytes(const qmoe_matvec_item* m, int32_t n, int32_t ncols);
int qmoe_matvec_group(const qmoe_matvec_item* m, int32_t n, int32_t ncols, void* ws,
                      size_t ws_bytes, void* stream);

/* Workspace bytes of qmoe_matvec for K = k and ncols columns. */
size_t qmoe_matvec_workspace_bytes(int64_t k, int32_t ncols);

/* Dense block-quantized matvec / small matmul: y[c][r] = sum_b s[r][b] d_c[b] P_c[r][b]
 * for columns c < ncols (1..4), with x quantized per 32-block (rot 0 or 1).
 * The packed blocks are read directly and their codebook expanded in registers
 * for integer dot products ([Strix-284B], ROCmFPX section); up to four columns
 * share each decoded block, the q = 4 weight reuse of the dense ROCmFP4 path
 * ([Strix-284B], decode section); rot = 1 is the H32 input rotation of the
 * fused H32 matvec ([evox3], table "The optimization ladder").
 * w: packed [rows][row_bytes] (w_bytes >= qmoe_packed_bytes, 16-byte aligned);
 * cb: int8 [2^bits]; x: fp32 [ncols][k] (16-byte aligned); y: fp32
 * [ncols][rows]; ws: qmoe_matvec_workspace_bytes(k, ncols) bytes, scratch.
 * Errors before any launch: QMOE_E_FORMAT (format, rot), QMOE_E_SHAPE (k, rows,
 * ncols), QMOE_E_INVAL (NULL or misaligned), QMOE_E_SIZE, QMOE_E_WORKSPACE. */
int qmoe_matvec(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes,
                const int8_t* cb, int32_t rot, const float* x, int32_t ncols,
                float* y, void* ws, size_t ws_bytes, void* stream);

/* Activation quantization only: x fp32 [n_vec][k] -> xq int8 [n_vec][k],
 * dx fp32 [n_vec][k/32] (all device). The int8 per-32-block activations that
 * the integer dot products consume ([Strix-284B], ROCmFPX section), with the
 * optional H32 rotation of each input block ([evox3], table "The optimization
 * ladder": H32 support and the shared H32 input); the arithmetic is the one in
 * the preamble above. Errors: QMOE_E_SHAPE (k % 32), QMOE_E_FORMAT (rot),
 * QMOE_E_INVAL (NULL). */
int qmoe_quant_act(const float* x, int64_t n_vec, int64_t k, int32_t rot,
                   int8_t* xq, float* dx, void* stream);

/* Per-block exact integer sums P[r][b] = sum_j C[code] * xq[32b+j] (int32),
 * the integer dot product of an expanded block with int8 activations
 * ([Strix-284B], ROCmFPX section), through the same expansion and sdot4 code
 * as the decode and matvec kernels. xq: int8 [k]; P: int32 [rows][k/32] (both
 * device). Errors as qmoe_matvec. */
int qmoe_block_dots(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes,
                    const int8_t* cb, const int8_t* xq, int32_t* P, void* stream);

/* The same per-block sums for ncols (1..64) int8 columns through the prefill
 * kernels' matrix-core path: the A operand expanded from the packed codes by
 * byte permutes, one int8 MFMA (v_mfma_i32_32x32x32_i8) per 32-block and
 * 32 x 32 tile, as the prefill expert GEMMs compute them ([evox3], table "The
 * optimization ladder": the batched multi-token prefill). xq: int8
 * [ncols][k]; P: int32 [ncols][rows][k/32] (device). rows: a multiple of 128;
 * k: a multiple of 256.
 * Errors as qmoe_matvec (ncols outside 1..64: QMOE_E_SHAPE). */
int qmoe_block_dots_mfma(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes,
                         const int8_t* cb, const int8_t* xq, int32_t ncols, int32_t* P,
                         void* stream);

/* Byte offsets of the internal buffers inside a layer workspace, so that a caller
 * can inspect intermediate results (int8 activations, routing, SwiGLU outputs).
 * Fields are byte offsets from the workspace start. */
typedef struct {
  size_t xq;          /* int8  [max_tokens][hidden]                        */
  size_t dx;          /* fp32  [max_tokens][hidden/32]                     */
  size_t idx;         /* int32 [max_tokens][topk]                          */
  size_t gw;          /* fp32  [max_tokens][topk]                          */
  size_t logits;      /* fp64  [max_tokens][E]                             */
  size_t plan;        /* decode plan: int32 U, ids[32], masks[32], fp32 w[32][4] */
  size_t hq;          /* int8  [slots][inter]  (decode: slot = u*4 + t; prefill: pair) */
  size_t dh;          /* fp32  [slots][inter/32]                           */
  size_t group;       /* prefill grouping (counts, offsets, pairs, tiles)  */
  size_t ypair;       /* fp32  [max_tokens][topk][hidden] (prefill)        */
  size_t total;       /* == qmoe_workspace_bytes                           */
} qmoe_ws_layout;

int qmoe_workspace_layout(const qmoe_layer* L, int32_t max_tokens, qmoe_ws_layout* out);

/* Measurement probes: the denominators that the path's kernels are compared
 * with. They are not steps of the layer; each is asynchronous on `stream` and
 * allocates nothing.
 *   qmoe_probe_read: a read-only stream of `bytes` (a multiple of 16) from
 *     `buf` (device, 16-byte aligned) by `grid` workgroups of 256 threads (0 =
 *     4 per compute unit), each reading a contiguous share with 16-byte loads
 *     and writing one word of a checksum to sink[blockIdx] (device, grid
 *     words), so that no load is dead.
 *   qmoe_probe_mfma: `iters` rounds of back-to-back int8 MFMAs on registers
 *     only; `kind` 0 = v_mfma_i32_16x16x32_i8 (the form the prefill GEMMs use),
 *     1 = v_mfma_i32_32x32x32_i8 (the gfx950 form at the full int8 rate);
 *     grid workgroups of 256 threads (0 = 4 per compute unit); each lane adds
 *     its results into sink[global thread id] (device, grid*256 words). The
 *     int8 ops are grid * 4 waves * iters * 4 MFMAs * 2*M*N*K.
 *   qmoe_probe_valu: `iters` rounds of the per-block fp32 epilogue of the
 *     prefill GEMMs (an int32 -> fp32 convert and a fused multiply-add per
 *     element and block) on 16 independent values per lane, registers only;
 *     grid and sink as qmoe_probe_mfma. Epilogue element-blocks =
 *     grid * 256 * iters * 16.
 * Errors: QMOE_E_INVAL (NULL, misaligned, bytes % 16, kind), QMOE_E_SHAPE
 * (iters < 1). */
int qmoe_probe_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, void* stream);
int qmoe_probe_mfma(int32_t kind, int32_t iters, int32_t grid, uint32_t* sink, void* stream);
int qmoe_probe_valu(int32_t iters, int32_t grid, uint32_t* sink, void* stream);

/* Weight quantizer: n fp32 matrices w [n][rows][k] (device, 16-byte aligned,
 * finite) -> packed ROCmFPX rows out [n][rows][row_bytes] (device) and one int8
 * codebook per matrix cb [n][2^bits] (device). The pages say the expert
 * weights carry learned codebooks, one per expert ([0731-Strix], section "How
 * the model fits on AMD Strix Halo"), in 32-weight blocks with a small scale
 * ([Strix-284B], ROCmFPX section); the procedure is the format specification's
 * weight-quantization section: per block an absmax scale (fp16 for FP2/FP3, a
 * power of two E8M0 for FP4), the weights normalized to integers in units of
 * scale/256, `iters` (0..64) Lloyd iterations of a 1-D k-means per matrix in
 * integer arithmetic (results independent of reduction order), then the
 * nearest codebook entry of each weight (ties to the lower entry).
 * k: a multiple of 256 (FP2/FP3) or 512 (FP4); n <= 65535; n*rows*k <= 2^34.
 * ws: caller-owned device
 * workspace of qmoe_quantize_workspace_bytes(n, rows, k) bytes, 256-byte
 * aligned; its contents need no initialisation and are scratch afterwards.
 * Asynchronous on `stream`; never allocates or synchronises. Errors (checked
 * before any launch): QMOE_E_FORMAT, QMOE_E_SHAPE (k, iters, sizes),
 * QMOE_E_INVAL (NULL or misaligned pointers), QMOE_E_SIZE (out too small),
 * QMOE_E_WORKSPACE. */
size_t qmoe_quantize_workspace_bytes(int32_t n, int64_t rows, int64_t k);
int qmoe_quantize(qmoe_format f, int32_t n, int64_t rows, int64_t k, const float* w,
                  int32_t iters, void* out, size_t out_bytes, int8_t* cb, void* ws,
                  size_t ws_bytes, void* stream);

/* Kernel timing (instrumentation). qmoe_timing_enable(1) starts recording, for
 * every kernel that an entry point launches afterwards, a pair of HIP events
 * carried by the kernel's own dispatch (so the elapsed time is the kernel's
 * execution); (0) stops; either call discards earlier records.
 * qmoe_timing_read waits for the recorded kernels named `name` and returns
 * their summed time in ms and their count. Names: "quant_act", "router",
 * "topk", "matvec", "expand", "matvec_x" (shared); "route", "gateup", "down" (decode);
 * "group_count", "group_scan", "group_scatter", "gateup_mfma", "down_mfma",
 * "combine" (prefill); "qz_norm", "qz_assign", "qz_update", "qz_pack"
 * (quantizer). */
int qmoe_timing_enable(int on);
int qmoe_timing_read(const char* name, double* total_ms, int* count);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
