/*
 * fc_gguf.h -- fully-connected layer computed directly on GGUF K-quant
 * weight blocks (Q4_K, Q5_K, Q6_K) on an AMD Instinct MI355X (gfx950).
 *
 *   Y[M,N] = A[M,K] . W[N,K]^T (+ R[M,N])
 *
 * W is never materialised as an f16 matrix: the kernels read the raw
 * super-blocks.  The operation and its paths follow OpenVINO PR #39119
 * ("FullyConnectedGGUF"):
 *   - section "Why a new primitive": GGUF weights are byte rows of
 *     K/256 * block_bytes, so K must be a multiple of 256;
 *   - section "Transformation": the weights are converted once; Q6_K blocks
 *     are regrouped into the planes QL|QH|SC|D (done on the device at create
 *     time here, where every plane, and the Q4_K / Q5_K blocks, are also
 *     cut into tiles of 16 rows x 4 blocks for coalesced wave64 loads);
 *   - section "Implementation": the path is chosen from the number of
 *     activation rows M: M < 8 -> per-32 int8 activation quantisation and an
 *     int8 GEMV; M >= 8 -> each 256-value block decoded once into on-chip
 *     memory and reused across rows on f16 matrix cores, with a tile that
 *     grows with M; a same-shape residual Add is fused into the store;
 *     GPU_GGUF_PREFILL_PATH-style forcing of a path for testing.
 * Q4_K, which that PR leaves on its converted path, is taken on the same
 * paths here; its 144-byte block is the struct printed in the
 * onnxruntime-mobius "GGUF Support Proposal", section 7.3.
 * The grouped (MoE) entry points follow llama.cpp PR #28301 (Metal
 * mul_mm_id), section Overview: each expert's routed rows are multiplied by
 * that expert's weights in one launch, and under-filled row tiles skip their
 * empty half.
 *
 * Conventions for every call:
 *   - Return value: 0 on success, a negative FC_GGUF_E* code on failure;
 *     fc_gguf_strerror() describes it.  Nothing is launched on failure.
 *   - "device" pointers are HIP device memory of the current device;
 *     "host" pointers are ordinary host memory.  A handle lives on the device
 *     that was current at its creation: every call that launches work on it
 *     (run, run_f32, run_grouped, debug_int_dots, debug_weights) needs that
 *     device current and returns FC_GGUF_EDEVICE otherwise.
 *   - f16 is IEEE binary16; all matrices are row-major and contiguous.
 *   - `stream` is a hipStream_t (NULL = the null stream).  run calls are
 *     asynchronous and stream-ordered; kernel faults surface at the caller's
 *     next synchronisation.  A handle owns a workspace, so one handle must not
 *     be run concurrently on two streams.  The workspace grows (and moves)
 *     when a call needs more than earlier calls did; the growth is
 *     stream-ordered (hipFreeAsync / hipMallocAsync on the call's stream), so
 *     it waits for no other stream.  A HIP graph that captured earlier calls
 *     of the handle must then be captured again, so capture after a call at
 *     the largest row count and path.
 *   - Testing switch: the environment variable FC_GGUF_TEST_FAIL_ALLOC =
 *     create | workspace | all makes the named device allocations fail
 *     (FC_GGUF_ENOMEM), read at every allocation.
 *   - Prefill kernel: three f16 matrix-core kernels serve the prefill path:
 *     a tile whose compute waves decode the weights into their matrix-core
 *     operand registers (16 .. 128 activation rows, growing with M; "dma"),
 *     a 128 x 128 tile whose producer waves decode each block once into an
 *     f16 tile in LDS that consumer waves multiply ("lds"), and a few-row
 *     kernel that streams the weights like the decode GEMV, one workgroup
 *     per 16 weight rows over all of K, with the activation rows in LDS
 *     ("skinny": M <= 32 when M * (K + 8) * 2 bytes plus the partial sums
 *     fit the 160 KB of LDS).  The default takes the few-row kernel where it
 *     fits, else the first tile.  The environment variable
 *     FC_GGUF_PREFILL_KERNEL = dma | lds | skinny, read when a handle is
 *     created, forces one (testing; skinny only where it fits).  The first
 *     tile's height and its split of K come from an estimate of the launch
 *     time; FC_GGUF_TILE = <mt>,<splits> (mt in 1, 2, 4, 8: 16*mt rows;
 *     splits a power of two up to 64), read when a handle is created, forces
 *     that tile and them (tuning; ignored for a call whose K it would leave
 *     a part of).
 */
#ifndef FC_GGUF_H
#define FC_GGUF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fc_gguf* fc_gguf_t;

/* Quantisation types (this library's own numbering). */
#define FC_GGUF_Q4_K 4   /* 144 B per 256 values: d, dmin, 12 B scales/mins, qs[128] */
#define FC_GGUF_Q5_K 5   /* 176 B per 256 values: d, dmin, 12 B scales/mins, qh[32], qs[128] */
#define FC_GGUF_Q6_K 6   /* 210 B per 256 values: ql[128], qh[64], sc[16] (int8), d */

/* Path override (fc_gguf_set_path; default from env
   FC_GGUF_PATH=auto|decode|prefill|scratch|int8). */
#define FC_GGUF_PATH_AUTO    0   /* M < D -> decode, else prefill; D = 8 (the page's row
                                    threshold) unless the environment variable
                                    FC_GGUF_DECODE_ROWS held another integer >= 0 when the
                                    handle was created (on MI355X the prefill path is the
                                    faster one from about 5 rows for most shapes) */
#define FC_GGUF_PATH_DECODE  1   /* int8 GEMV for any M (rows taken in chunks of at most 7) */
#define FC_GGUF_PATH_PREFILL 2   /* f16 matrix-core path for any M >= 1 */
#define FC_GGUF_PATH_SCRATCH 3   /* comparison only: weights dequantised to an f16 buffer in the
                                    handle's workspace (N*K*2 bytes), then a rocBLAS GEMM with the
                                    residual as beta*C (the page's path for devices without the
                                    decode-once kernel; never chosen by AUTO) */
#define FC_GGUF_PATH_INT8    4   /* variant: per-32 int8 activations (the decode path's
                                    quantisation, a pass of its own) times the integer codes on
                                    int8 matrix cores, scales applied per 32-value group in f32;
                                    computes what the decode path computes, at any M (its
                                    results are checked against the int8 emulation, not the
                                    fp64 FC); workspace: M rounded up to 128 times (K + K/4)
                                    bytes plus the split-K partials; never chosen by AUTO */

/* Error codes. */
#define FC_GGUF_OK            0
#define FC_GGUF_EINVAL       -1  /* NULL handle/pointer, N<=0, K<=0, K%256!=0, M<0, bad top_k ... */
#define FC_GGUF_EUNSUPPORTED -2  /* unknown qtype or path */
#define FC_GGUF_ENOMEM       -3  /* device allocation failed */
#define FC_GGUF_EHIP         -4  /* a HIP runtime call or kernel launch failed */
#define FC_GGUF_ERANGE       -5  /* a size exceeds an internal limit (e.g. 32-bit indexing) */
#define FC_GGUF_EDEVICE      -6  /* the current device is not the one the handle was created on */

/*
 * Create a handle for one weight matrix W[N,K].
 *   blocks           u8[N][K/256 * block_bytes] in canonical GGUF AoS order
 *                    (row n holds its K/256 super-blocks in order).
 *   blocks_on_device 0: `blocks` is host memory; 1: device memory.
 * The bytes are copied into library-owned device memory and converted there
 * to the device layout (see fc_gguf_debug_weights), so the caller may free
 * `blocks` as soon as the call returns.  Synchronous.  *out receives the
 * handle.
 */
int fc_gguf_create(int64_t N, int64_t K, int qtype, const void* blocks,
                   int blocks_on_device, fc_gguf_t* out);

/*
 * Y = A . W^T (+ R).
 *   A  device f16[M,K]; R device f16[M,N] or NULL; Y device f16[M,N].
 *   Y may be the same pointer as R (in-place residual); Y must not overlap A.
 *   M == 0 is a no-op.  Path per fc_gguf_set_path (default: M<8 -> decode).
 */
int fc_gguf_run(fc_gguf_t h, const void* A, int64_t M, const void* R, void* Y, void* stream);

/*
 * Y = A . W^T (+ R) with f32 activations, residual and output.
 *   A  device f32[M,K] (16-byte aligned); R device f32[M,N] or NULL;
 *   Y device f32[M,N].  Y may be the same pointer as R; Y must not overlap A.
 * OpenVINO PR #39119, section Implementation: f32 activations take the int8
 * quantisation + GEMV path at every row count, so this call ignores
 * fc_gguf_set_path and runs the decode path (rows in chunks of at most 7,
 * one launch each).  The per-32 quantisation reads the f32 values directly
 * (no f16 rounding); the result is stored in f32 without rounding to f16.
 * Single-matrix handles only.  M == 0 is a no-op.
 */
int fc_gguf_run_f32(fc_gguf_t h, const float* A, int64_t M, const float* R, float* Y,
                    void* stream);

/* Force a path (FC_GGUF_PATH_*); the testing switch of the FC primitive.  The
 * environment variable FC_GGUF_PATH (auto | decode | prefill | scratch | int8),
 * read at create, sets a handle's initial path. */
int fc_gguf_set_path(fc_gguf_t h, int path);

/* Frees the handle and its device memory; NULL is accepted.  Synchronises the
 * handle's device (made current for the call if another one is). */
int fc_gguf_destroy(fc_gguf_t h);

/* N, K, qtype, and the byte size of the device weights of a handle (any may be
 * NULL); the size includes the padding of the device layout (see
 * fc_gguf_debug_weights). */
int fc_gguf_info(fc_gguf_t h, int64_t* N, int64_t* K, int* qtype, int64_t* weight_bytes);

/*
 * Grouped (MoE expert) FC: E weight matrices W_e[N,K] of one qtype.
 *   blocks u8[E][N][K/256 * block_bytes], host or device as in fc_gguf_create.
 *   1 <= E <= 4096, else FC_GGUF_ERANGE.
 */
int fc_gguf_create_grouped(int64_t E, int64_t N, int64_t K, int qtype, const void* blocks,
                           int blocks_on_device, fc_gguf_t* out);

/*
 * Y[t, j, :] = A_row(t, j) . W_{ids[t,j]}^T for every token t < T and slot j < top_k.
 *   ids  device i32[T, top_k]: expert ids in [0, E), distinct within a row.
 *   A    device f16[T, K] when a_per_slot == 0 (row t shared by its slots),
 *        device f16[T, top_k, K] when a_per_slot == 1 (one row per pair).
 *   Y    device f16[T, top_k, N], one output row per (token, slot) pair.
 * No routing weights are applied and nothing is combined.  Ids outside
 * [0, E) produce zero rows.  T == 0 is a no-op.  Matrix-core numerics
 * (f16 weights, f32 accumulation) for every expert, whatever its row count.
 * Two kernels on `stream`: the bucketing of the pairs by expert (into the
 * handle's workspace, grown stream-ordered on first use) and the grouped FC.
 * T * top_k <= 2^24.
 */
int fc_gguf_run_grouped(fc_gguf_t h, const void* A, int64_t T, int a_per_slot,
                        const int32_t* ids, int top_k, void* Y, void* stream);

/*
 * fc_gguf_run_grouped on the expert bucketing that the last
 * fc_gguf_run_grouped call on `routed` computed, without sorting the routing
 * again: for a second grouped FC with the same routing, such as the down
 * projection after gate/up (llama.cpp PR #28301, section Overview: the rows
 * are grouped by expert once per routing).  `routed` is a grouped handle
 * with the same expert count on the same device whose last
 * fc_gguf_run_grouped call had these same `ids` (the same pointer, holding
 * the same values), T and top_k; otherwise FC_GGUF_EINVAL.  The bucketing is
 * read from `routed`'s workspace, so this call must be ordered after that
 * one (the same stream) and before the next grouped call on `routed`.  h may
 * be `routed` itself.  Other arguments and results as fc_gguf_run_grouped.
 */
int fc_gguf_run_grouped_reuse(fc_gguf_t h, fc_gguf_t routed, const void* A, int64_t T,
                              int a_per_slot, const int32_t* ids, int top_k, void* Y,
                              void* stream);

/*
 * fc_gguf_run_grouped without any allocation, for callers that cannot
 * allocate device memory (code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments, kernels and
 * results as fc_gguf_run_grouped, but the bucketing workspace is a static
 * 512 KB device array of the library (one per GPU, held until the process
 * ends) instead of the handle's workspace; no hipMalloc, hipFree or other
 * allocating call is made.  Calls whose bucketing needs more than 512 KB
 * (about E*12 + T*top_k*4.25 bytes) return FC_GGUF_ERANGE.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, or two host threads) race and must not be issued; calls ordered on
 * one stream are safe.
 */
int fc_gguf_run_grouped_noalloc(fc_gguf_t h, const void* A, int64_t T, int a_per_slot,
                                const int32_t* ids, int top_k, void* Y, void* stream);

/*
 * Test exports: they run the same device code as the decode path.
 *
 * fc_gguf_debug_quantize: the per-32 int8 activation quantisation of the
 *   decode path.  A device f16[M,K] (K % 32 == 0); qa device i8[M,K];
 *   s device f32[M,K/32]; T device i32[M,K/32] (sum of qa per group);
 *   H device i32[M,K/16] or NULL: the sum of qa over each 16-value half of
 *   a group, as the quantisation hands it to the Q6_K GEMV (whose sub-blocks
 *   are 16 values: the -32 offset enters as -32 times this sum).
 * fc_gguf_debug_quantize_f32: the same for f32 activations, A device
 *   f32[M,K] (the quantisation fc_gguf_run_f32 runs).
 *
 * fc_gguf_debug_int_dots: the integer sub-block dot sums of the decode path,
 *   from given int8 activations qa device i8[M,K].  S device i32:
 *   Q4_K, Q5_K [M, N, K/32] (sum of qa*q over each 32-value sub-block,
 *   q in [0,15] / [0,31]);
 *   Q6_K [M, N, K/16] (sum of qa*(q-32) over each 16-value sub-block).
 *
 * fc_gguf_debug_bucketing: the grouped path's expert bucketing alone
 *   (llama.cpp PR #28301, Overview: routed rows grouped by expert, then cut
 *   into row tiles), as fc_gguf_run_grouped runs it before the grouped FC.
 *   ids device i32[P] (pair p = t*top_k + j); E experts; BM rows per tile
 *   (the grouped FC uses 32, 64 or 128).  Outputs, all device i32:
 *   offsets[E+2] (bucket b's pairs are pairs[offsets[b] .. offsets[b+1]);
 *   bucket E holds the pairs whose id is outside [0, E)); pairs[P], the pair
 *   indices grouped by bucket (in no fixed order within a bucket); tiles[2*n]
 *   (bucket, first row within the bucket) for every BM rows of a bucket,
 *   buckets in order, with n <= ceil(P/BM) + min(E+1, P) and tiles 8-byte
 *   aligned; ntiles[1] = n.  EINVAL for NULL buffers, P < 0, E < 1 or BM
 *   outside [1, 4096]; ERANGE for E above 4096 or P above 2^30.
 *
 * fc_gguf_debug_weights: copies the handle's device weight bytes to device
 *   memory `dst` (fc_gguf_info's weight_bytes long).  Device layout, per
 *   matrix (experts one after another), block (n, kb) being the kb-th
 *   super-block of row n, cut into 16-byte pieces.  Q4_K / Q5_K: one plane
 *   of P = 9 / 11 pieces per block.  Q6_K: planes QL (P = 8) | QH (P = 4) |
 *   SC (P = 1) | D (2 bytes per block), each over the same padded block count.
 *   Every matrix is tiled: rows padded with zero bytes to a multiple of 16
 *   and blocks per row to a multiple of 4 (KBp); tile t = (n/16)*(KBp/4) +
 *   kb/4 holds 16 rows x 4 blocks, piece p of block (n, kb) at
 *   (t*P + p)*1024 + l*16 within its plane, l = (kb%4)*16 + n%16; D at
 *   t*128 + l*2.  Grouped handles hold their experts' matrices one after
 *   another.
 */
int fc_gguf_debug_quantize(const void* A, int64_t M, int64_t K, int8_t* qa, float* s,
                           int32_t* T, int32_t* H, void* stream);
int fc_gguf_debug_quantize_f32(const float* A, int64_t M, int64_t K, int8_t* qa, float* s,
                               int32_t* T, int32_t* H, void* stream);
int fc_gguf_debug_int_dots(fc_gguf_t h, const int8_t* qa, int64_t M, int32_t* S, void* stream);
int fc_gguf_debug_bucketing(const int32_t* ids, int64_t P, int64_t E, int64_t BM, int32_t* offsets,
                            int32_t* pairs, int32_t* tiles, int32_t* ntiles, void* stream);
int fc_gguf_debug_weights(fc_gguf_t h, void* dst, void* stream);

/* Static description of an error code. */
const char* fc_gguf_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FC_GGUF_H */
