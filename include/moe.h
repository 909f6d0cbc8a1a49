/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE expert-forward library.
 *
 * One MoE layer of a batch-1 (or small-batch) decode step, as the Flash-MoE
 * pages describe for Qwen3.5-397B-A17B:
 *   router GEMV -> softmax -> top-K -> renormalise            (moe_route)
 *   dequantised gate/up GEMVs -> SwiGLU -> dequantised down GEMV
 *   for the K routed experts plus one shared expert -> weighted combine
 *                                                               (moe_expert_forward)
 *   both, back to back on one stream                            (moe_layer_decode)
 *   RMS norm of the residual, the layer, residual add   (moe_layer_decode_residual)
 *   experts held in host memory behind a device cache            (moe_tier_*)
 *
 * Sources for the method (web pages; cited by title and section):
 *   [HL] "Flash-MoE: Running a 397B Parameter Model on a Laptop" (hysenlabs.com),
 *        section "How the SSD expert streaming pipeline works": 60 layers, 512
 *        experts per layer, K=4 routed plus one shared expert, hidden size 4096,
 *        4-bit experts of about 6.75 MB; routing is a softmax followed by a
 *        top-K; the expert forward pass is followed by a combine.
 *   [MC] "Flash-MoE: Running a 400 Billion Parameter Model on a MacBook"
 *        (mattcullerton.com), section "The Architecture": experts are 4-bit,
 *        about 6.75 MB each, and the inner loop is a dequantising FMA kernel.
 *   [WK] "Flash-MoE" (wiki.edouardfoussier.com), section "Performance Results"
 *        (table): 4-bit and 2-bit expert configurations.
 * The pages state neither the quantisation form, the group size, the
 * intermediate size, the activation nor the renormalisation; the readings
 * taken here are written next to each item below.
 *
 * ---------------------------------------------------------------------------
 * Expert blob format (one contiguous byte range per expert)
 * ---------------------------------------------------------------------------
 * Parameters: hidden H, intermediate I, bits b in {2,4}, group g = 64.
 * cpw = 32/b codes per 32-bit little-endian word.
 * Sections, in this order, each starting at a 256-byte aligned offset from
 * the start of the blob (with H, I multiples of 256 no padding occurs):
 *   0 GATE_Q  I rows x H/cpw words   codes of Gate [I][H]
 *   1 UP_Q    I rows x H/cpw words   codes of Up   [I][H]
 *   2 DOWN_Q  H rows x I/cpw words   codes of Down [H][I]
 *   3 GATE_SB I rows x H/g words     (scale, bias) of Gate
 *   4 UP_SB   I rows x H/g words     (scale, bias) of Up
 *   5 DOWN_SB H rows x I/g words     (scale, bias) of Down
 * Code c of row r of a matrix with C columns lives in word r*(C/cpw) + c/cpw
 * at bit offset b*(c % cpw), lowest bits first; it is an unsigned integer
 * q in [0, 2^b - 1].
 * An SB word [r][j] holds two bf16 values: bits 0..15 the scale s, bits
 * 16..31 the bias z, both applying to columns j*g .. j*g+g-1 of row r.
 * The dequantised weight is the affine map
 *     W[r][c] = s[r][c/g] * q[r][c] + z[r][c/g].
 * With H=4096, I=1024, b=4 a blob is 7,077,888 bytes = 6.75 MiB, the expert
 * size [HL] and [MC] give; with b=2 it is 3,932,160 bytes.
 * Readings ([MC] names only a "4-bit" "dequant" with FMAs): affine form with
 * unsigned codes, groups of 64 along the input dimension, bf16 scale and
 * bias; the nibble order and section order are this library's own choice.
 *
 * The shared expert uses the same format and the same I.
 * The router is a bf16 matrix [E][H] (row e = expert e), no bias.
 *
 * ---------------------------------------------------------------------------
 * Conventions for every entry point
 * ---------------------------------------------------------------------------
 * - All tensor pointers are DEVICE pointers (hipMalloc / torch allocations on
 *   the current device) unless stated otherwise; the caller owns them.  The
 *   library never allocates device or pinned memory (a tier object holds
 *   host heap memory and two HIP events).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Every compute call only enqueues work on `stream` and returns; none of
 *   them synchronises the host, except moe_get_device_error.
 * - Arguments are validated on the host before anything is enqueued; on any
 *   error nothing is enqueued and the status says why.
 * - bf16 tensors are passed as uint16_t bit patterns.
 * - x is bf16 [T][H], row-major, and is expected to be RMS-normalised by the
 *   caller (the pages place a norm before routing, [HL]);
 *   moe_layer_decode_residual forms it from the residual itself.
 * - y is fp32 [T][H] row-major.  ids int32 [T][K], w fp32 [T][K], per token
 *   in descending-logit order.
 * - Results are deterministic: identical inputs give bitwise-identical
 *   outputs (no floating-point atomics; fixed reduction orders).
 * - The workspace `ws` (device memory, caller-owned, moe_workspace_bytes
 *   bytes, 256-byte aligned) must be initialised once before its first use:
 *   with moe_workspace_init, or by allocating it zero-filled (a workspace
 *   whose bytes are all zero is initialised; moe_workspace_init zeroes its
 *   control words).  Every call leaves it initialised again.  Two calls that
 *   overlap in time must not share a workspace.
 * - A call of 1 to 3 tokens on a GPU with 256 compute units, hidden 4096,
 *   intermediate 1024 and top-4 runs as one launch per token of 256
 *   workgroups, one per compute unit, that exchange data while running: it
 *   needs the whole GPU.  Do not run it concurrently with other kernels
 *   (such as a second such call on another stream): workgroups that cannot
 *   become resident make the others' waits time out, which sets bit 1 of the
 *   sticky error flags and leaves the outputs invalid (nothing hangs).  Calls
 *   on one stream, or captured in one graph, are always safe.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  MOE_ERR_UNSUPPORTED = -3, /* a valid but unimplemented configuration */
  MOE_ERR_ALIGN = -4,       /* a pointer or stride is misaligned */
  MOE_ERR_WORKSPACE = -5,   /* workspace too small */
  MOE_ERR_HIP = -6,         /* a HIP runtime call failed */
  MOE_ERR_DEVICE = -7       /* the device reported an invalid input */
} moe_status;

/* Layer dimensions.
 *   hidden      H: power of two, 256 <= H <= 16384
 *   inter       I: power of two, 256 <= I <= 16384
 *   n_experts   E: 1 <= E <= 1024
 *   top_k       K: 1 <= K <= min(E, 8)
 *   group       g: must be 64
 *   bits        b: 2 or 4
 *   has_shared  0 or 1 (one shared expert, added with weight 1.0) */
typedef struct {
  int32_t hidden, inter, n_experts, top_k, group, bits, has_shared;
} moe_dims;

/* One layer's weights (device pointers).
 *   router         bf16 [E][H]; 16-byte aligned
 *   experts        expert e's blob starts at experts + e * expert_stride;
 *                  256-byte aligned
 *   expert_stride  bytes; >= moe_expert_bytes(dims), multiple of 256
 *   shared         the shared expert's blob (256-byte aligned), NULL iff
 *                  has_shared == 0 */
typedef struct {
  const uint16_t *router;
  const uint8_t *experts;
  int64_t expert_stride;
  const uint8_t *shared;
} moe_layer;

/* Blob sections, in storage order (see the format above). */
enum {
  MOE_SEC_GATE_Q = 0, MOE_SEC_UP_Q = 1, MOE_SEC_DOWN_Q = 2,
  MOE_SEC_GATE_SB = 3, MOE_SEC_UP_SB = 4, MOE_SEC_DOWN_SB = 5
};

/* Library ABI version (MOE_ABI_VERSION). */
int32_t moe_abi_version(void);

/* Human-readable name of a status code (static string, never NULL).  Takes
 * any int, so a value outside moe_status yields "unknown status". */
const char *moe_status_str(int32_t s);

/* Checks dims against the constraints above.  Host only. */
moe_status moe_check_dims(const moe_dims *dims);

/* Bytes of one expert blob for dims (0 if dims are invalid).  Host only. */
size_t moe_expert_bytes(const moe_dims *dims);

/* Byte offsets of the six sections (out[6]); returns MOE_ERR_* for bad dims.
 * Host only. */
moe_status moe_blob_layout(const moe_dims *dims, size_t out_offsets[6]);

/* Workspace bytes needed for calls with T tokens (0 if invalid).  Host only. */
size_t moe_workspace_bytes(const moe_dims *dims, int32_t T);

/* Enqueues the one-time initialisation of a workspace of ws_bytes bytes
 * (zeroes its control words; not needed for a zero-filled workspace). */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Routing ([HL], "How the SSD expert streaming pipeline works": the router
 * scores feed a softmax and a top-K selection).
 *   logits[t][e] = sum_c router[e][c] * x[t][c]    (bf16 products, fp32 sums)
 *   ids[t][0..K-1] = the K largest logits in descending order; equal logits
 *                    are ordered by lower expert index (a reading: the pages
 *                    do not say)
 *   w[t][k] = exp(logit_k) / sum over the K selected of exp(logit)
 *           = softmax over all E, restricted to the selected K, renormalised
 *             to sum to 1 (a reading: the pages do not say whether they
 *             renormalise; here they do).
 * Arguments: x bf16 [T][H] (16-byte aligned); ids int32 [T][K]; w fp32 [T][K];
 * logits fp32 [T][E] or NULL.  1 <= T <= 4096 (every entry point). */
moe_status moe_route(const moe_dims *dims, const uint16_t *router,
                     const uint16_t *x, int32_t T, int32_t *ids, float *w,
                     float *logits, void *ws, size_t ws_bytes, void *stream);

/* Expert forward and combine ([HL], same section: the expert forward pass
 * for the K routed experts, then the combine; the shared expert runs beside
 * them).  For each token t:
 *   for each selected expert e and for the shared expert:
 *     g = Gate_e x_t, u = Up_e x_t            (dequantised weights)
 *     h = silu(g) * u,  silu(v) = v / (1 + exp(-v))   (SwiGLU: a reading)
 *     d_e = Down_e h
 *   y[t] = sum_k w[t][k] * d_{ids[t][k]} + d_shared
 * (the shared expert enters with weight 1: a reading.)
 * ids/w: device int32/fp32 [T][K] (e.g. from moe_route).  An id outside
 * [0, E) makes that slot contribute 0 and sets the workspace's sticky error
 * flag (see moe_get_device_error).  y fp32 [T][H], 16-byte aligned. */
moe_status moe_expert_forward(const moe_dims *dims, const moe_layer *layer,
                              const uint16_t *x, int32_t T,
                              const int32_t *ids, const float *w, float *y,
                              void *ws, size_t ws_bytes, void *stream);

/* moe_route followed by moe_expert_forward on the same stream, with ids/w
 * kept on the device.  ids and w may be NULL (then they stay in the
 * workspace); if given they receive the routing. */
moe_status moe_layer_decode(const moe_dims *dims, const moe_layer *layer,
                            const uint16_t *x, int32_t T, float *y,
                            int32_t *ids, float *w, void *ws, size_t ws_bytes,
                            void *stream);

/* One MoE block on the residual stream ([HL], "How the SSD expert streaming
 * pipeline works": each layer ends with the combine and a norm, so the next
 * layer's router sees the normalised sum).  For each token t:
 *   x[t] = bf16( r[t] / sqrt(mean_c r[t][c]^2 + 1e-6) )   (RMS norm)
 *   y[t] = the MoE layer of x[t], exactly as moe_layer_decode
 *   r[t] = r[t] + y[t]                                   (fp32, in place)
 * Readings (the pages name the norm but not its form): RMS norm without a
 * learned gain (a gain folds into the next matrices), epsilon 1e-6, the
 * residual kept in fp32, the sum of squares accumulated in fp32 and x
 * rounded to bf16 to nearest-even.  Calling this once per layer with the
 * same r chains layers: x of layer l+1 = norm(r after layer l).
 * Arguments: resid fp32 [T][H], 16-byte aligned, read and written (the
 * caller owns it; it must not alias any other argument).  x_out bf16 [T][H]
 * (16-byte aligned) receives x, or NULL.  y fp32 [T][H] (16-byte aligned)
 * receives the layer output, or NULL.  ids/w as in moe_layer_decode.
 * After a call that leaves a device error (moe_get_device_error) resid is
 * undefined. */
moe_status moe_layer_decode_residual(const moe_dims *dims, const moe_layer *layer,
                                     float *resid, int32_t T, uint16_t *x_out, float *y,
                                     int32_t *ids, float *w, void *ws, size_t ws_bytes,
                                     void *stream);

/* Consecutive layers of one decode token ([HL], "How the SSD expert
 * streaming pipeline works": a token runs the layers in sequence, each one
 * router -> top-K -> expert forward -> combine; the pages keep the next
 * layer's command queued so that the GPU does not wait between layers).
 * For l = 0 .. n_layers - 1, exactly as moe_layer_decode of one token:
 *   y[l] = the MoE layer `layers[l]` of x[l];  ids[l], w[l] its routing.
 * layers: HOST array of n_layers layer descriptors (device pointers inside,
 * each as for moe_layer_decode).  x bf16 [n_layers][H], y fp32
 * [n_layers][H] (16-byte aligned); ids int32 [n_layers][K] and w fp32
 * [n_layers][K], each optional (NULL).  ws: at least moe_workspace_bytes(
 * dims, 1) bytes, initialised.  Where the single-token kernel covers the
 * dims (see the conventions), up to 64 layers run in one launch that keeps
 * all 256 compute units (same condition: nothing may run beside it); the
 * routing-independent bytes of each layer (router, shared expert) are read
 * while the layer before it routes.  Results are bitwise those of
 * n_layers moe_layer_decode calls; other dims run exactly those calls. */
moe_status moe_stack_decode(const moe_dims *dims, const moe_layer *layers, int32_t n_layers,
                            const uint16_t *x, float *y, int32_t *ids, float *w, void *ws,
                            size_t ws_bytes, void *stream);

/* The same on the residual stream: for l = 0 .. n_layers - 1, exactly as
 * moe_layer_decode_residual of one token,
 *   x[l] = bf16(rmsnorm(r)),  y[l] = layer l of x[l],  r = r + y[l],
 * so each layer's routing depends on the layer before it.  resid fp32 [H]
 * (16-byte aligned), read and written (r after the last layer); x_out bf16
 * [n_layers][H], y fp32 [n_layers][H], ids, w: each optional.  Results are
 * bitwise those of n_layers moe_layer_decode_residual calls.  After a call
 * that leaves a device error resid is undefined. */
moe_status moe_stack_decode_residual(const moe_dims *dims, const moe_layer *layers,
                                     int32_t n_layers, float *resid, uint16_t *x_out, float *y,
                                     int32_t *ids, float *w, void *ws, size_t ws_bytes,
                                     void *stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * serving loops that must not call an allocator): moe_stack_decode_residual
 * with no workspace argument.  Its workspace is an array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library's device memory, one per GPU,
 * held until the process ends; this call allocates nothing.  Arguments,
 * results and errors are those of moe_stack_decode_residual, plus
 * MOE_ERR_WORKSPACE when the dims need a larger workspace than the array
 * (moe_workspace_bytes(dims, 1) > MOE_NOALLOC_SCRATCH_BYTES; no valid dims
 * do today).  The first call on a GPU looks up the array's address and
 * enqueues its initialisation on `stream`, so it must not be made under
 * graph capture (MOE_ERR_UNSUPPORTED if it is); later calls may be.  All
 * calls on one GPU share the array and carry state from one call to the
 * next: calls whose kernels overlap on one GPU (on different streams,
 * or from different threads) race and give undefined results.  The GPU is
 * the current device of the calling thread. */
#define MOE_NOALLOC_SCRATCH_BYTES (2u * 1024u * 1024u)
moe_status moe_stack_decode_residual_noalloc(const moe_dims *dims, const moe_layer *layers,
                                             int32_t n_layers, float *resid, uint16_t *x_out,
                                             float *y, int32_t *ids, float *w, void *stream);

/* ---------------------------------------------------------------------------
 * Off-HBM expert tier ([HL], "How the SSD expert streaming pipeline works":
 * per token only the K routed experts of a layer are read from the slow tier,
 * once the routing of that layer is known, and a least-recently-used page
 * cache absorbs the reuse between tokens).  Here the slow tier is host memory
 * (pinned, so that copies are asynchronous) and the cache is n_slots expert
 * blobs in device memory, shared by all layers with least-recently-used
 * replacement.  For GPUs, or expert sets, whose experts do not all fit in
 * device memory; results are identical to moe_route + moe_expert_forward on
 * resident experts (the same kernels run over the slots).
 * A tier object holds host-side state only (allocated with the C++ heap); it
 * is not thread-safe, and all calls on one tier must be issued on one compute
 * stream (a slot is overwritten only after every kernel enqueued before the
 * call's routing on that stream has finished).
 * ------------------------------------------------------------------------- */
typedef struct moe_tier moe_tier;

typedef struct {
  int32_t n_layers;                   /* layers served by this tier */
  int32_t t_max;                      /* most tokens per call (t_max K <= n_slots) */
  const uint8_t *const *host_experts; /* host array of n_layers host pointers:
                                         layer l's expert e at
                                         host_experts[l] + e * host_stride */
  int64_t host_stride;                /* bytes, >= moe_expert_bytes */
  void *slots;                        /* device: n_slots blobs, 256-byte aligned */
  int64_t slot_stride;                /* bytes, >= moe_expert_bytes, multiple of 256 */
  int32_t n_slots;                    /* t_max * K <= n_slots <= 1024 */
  void *copy_stream;                  /* hipStream_t of the host-to-device copies */
  void *staging;                      /* pinned host, moe_tier_staging_bytes, 16-byte aligned */
  void *dev_scratch;                  /* device, moe_tier_device_bytes, 256-byte aligned */
} moe_tier_config;

/* Sizes of the caller-owned buffers of a tier (0 if invalid).  Host only. */
size_t moe_tier_staging_bytes(const moe_dims *dims, int32_t t_max);
size_t moe_tier_device_bytes(const moe_dims *dims, int32_t t_max);
/* Workspace bytes for tier calls of T tokens (covers the routing with E
 * experts and the expert forward over n_slots slots).  Host only. */
size_t moe_tier_workspace_bytes(const moe_dims *dims, int32_t n_slots, int32_t T);

/* Creates a tier with every slot empty.  Validates the configuration; makes
 * no HIP call.  *out receives the object (NULL on error). */
moe_status moe_tier_create(const moe_dims *dims, const moe_tier_config *cfg, moe_tier **out);

/* One layer for T tokens through the tier: moe_route on `stream` (router,
 * x as in moe_route), the host waits for the ids (this call synchronises
 * with `stream` once), missing experts are copied into least-recently-used
 * slots on the copy stream, then the expert forward over the slots runs on
 * `stream` after the copies.  shared: the layer's shared expert blob in
 * device memory (NULL iff has_shared == 0).  y as in moe_layer_decode;
 * ids/w (device, optional) receive the routing (real expert ids).  ws: at
 * least moe_tier_workspace_bytes. */
moe_status moe_tier_decode(moe_tier *tier, int32_t layer, const uint16_t *router,
                           const uint8_t *shared, const uint16_t *x, int32_t T, float *y,
                           int32_t *ids, float *w, void *ws, size_t ws_bytes, void *stream);

/* Host-only test hook: the slot plan of one call for host expert ids
 * [T][K] of `layer`, applied to the tier's state as moe_tier_decode would
 * (no copy is made).  slot_ids (host) receive the slot of each id (-1 for an
 * id outside [0, E)); copy_expert (host, optional) the expert copied into
 * that slot by this call, or -1 for a hit. */
moe_status moe_tier_plan(moe_tier *tier, int32_t layer, const int32_t *ids, int32_t T,
                         int32_t *slot_ids, int32_t *copy_expert);

/* Counters since creation: out[0] hits, out[1] misses (copies), out[2] bytes
 * copied, out[3] evictions.  A repeat of an expert inside one call counts
 * once.  Host only. */
moe_status moe_tier_stats(const moe_tier *tier, int64_t out[4]);

/* Frees the tier object (not the caller's buffers).  NULL is ignored. */
void moe_tier_destroy(moe_tier *tier);

/* Code decoders of the kernels, for moe_dequantize_as.  Each turns the codes
 * of a 32-bit word into numbers the way one kernel path does before its
 * products ([MC], "The Architecture": the dequantisation sits inside the
 * matrix-vector inner loop, so each path has its own unpack):
 *   MOE_DEQ_SCALAR      mask and shift per code (the format read directly)
 *   MOE_DEQ_FP16_PAIR   fp16 pairs 1024 + m q from one AND-OR with 0x6400:
 *                       gate/up of the single-token and unfused paths
 *   MOE_DEQ_FP8_PAIR    masked code bytes converted two at a time as fp8:
 *                       down of the single-token path
 *   MOE_DEQ_BF16_PAIR   bf16 pairs 128 + q from one AND-OR with 0x4300: down
 *                       of the unfused path
 *   MOE_DEQ_BF16_SLICE  bf16 slices 128 + q of the matrix-core A operand:
 *                       gate/up and down of the grouped path (T >= 2) */
enum {
  MOE_DEQ_SCALAR = 0, MOE_DEQ_FP16_PAIR = 1, MOE_DEQ_FP8_PAIR = 2,
  MOE_DEQ_BF16_PAIR = 3, MOE_DEQ_BF16_SLICE = 4
};

/* Test hook: writes the dequantised fp32 matrix `which` (0 Gate [I][H],
 * 1 Up [I][H], 2 Down [H][I]) of one blob to out (row-major), each code
 * decoded by `decoder` (any of the MOE_DEQ_* values, for any matrix).  Each
 * element is s*q + z rounded once to fp32 (s*q is exact in fp32), so every
 * correct decoder gives the same bits.  blob 256-byte aligned, out 16-byte
 * aligned.  MOE_ERR_SHAPE for `which` or `decoder` out of range. */
moe_status moe_dequantize_as(const moe_dims *dims, const uint8_t *blob,
                             int32_t which, int32_t decoder, float *out, void *stream);

/* moe_dequantize_as with the decoders of the single-token kernel:
 * MOE_DEQ_FP16_PAIR for gate and up, MOE_DEQ_FP8_PAIR for down. */
moe_status moe_dequantize(const moe_dims *dims, const uint8_t *blob,
                          int32_t which, float *out, void *stream);

/* Synchronises `stream`, returns the workspace's sticky device error flags in
 * *err (0 = none; bit 0 = an expert id was out of range; bit 1 = a wait of
 * the single-token kernel timed out, see the conventions) and clears them.
 * `err` is a host pointer.  Returns MOE_ERR_DEVICE when *err != 0. */
moe_status moe_get_device_error(void *ws, void *stream, int32_t *err);

/* ---------------------------------------------------------------------------
 * Measurement helpers (beside the method, for benchmarks)
 * ------------------------------------------------------------------------- */

/* Words of `sink` that moe_stream_read writes for a read of `bytes` (one per
 * workgroup).  Host only. */
size_t moe_stream_read_sink_words(size_t bytes);

/* Enqueues one launch that reads `bytes` of device memory at `src` with
 * 16-byte loads spread over up to 2048 workgroups and writes an XOR of what
 * each workgroup read to sink[0 .. moe_stream_read_sink_words(bytes) - 1]:
 * the streaming read rate a single launch reaches at that size, the
 * achievable counterpart of the HBM peak for the layer's byte counts.  From
 * 256 MiB on the loads carry the non-temporal hint (faster there on this GPU),
 * below it they are plain loads (faster there).
 * src 16-byte aligned, bytes a nonzero multiple of 16, sink device uint32. */
moe_status moe_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Enqueues a launch that overwrites `bytes` of device memory at `dst`
 * (16-byte aligned, nonzero multiple of 16) with stores: with a size above
 * the last-level cache (256 MB) the next launch finds none of its bytes
 * cached. */
moe_status moe_flush(void *dst, size_t bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Per-stage timing: the per-layer breakdown that the pages' timing flag
 * prints ("Flash-MoE: Running a 397B Parameter Model on a Laptop",
 * hysenlabs.com, section "Install"; the stage times of section "How the SSD
 * expert streaming pipeline works"), taken with HIP events.
 *
 * While timing is on, every decode entry point (moe_route,
 * moe_expert_forward, moe_layer_decode, moe_layer_decode_residual,
 * moe_stack_decode, moe_stack_decode_residual) records an event on its
 * stream before each of its stages and one after its last; moe_timing_read
 * waits for the events recorded so far and adds each stage's elapsed time
 * to the stage's total.  Timing starts on when the environment variable
 * MOE_TIMING is set to anything but "0" at the library's first timed call,
 * and moe_timing_set switches it.  A call whose stream is being captured
 * into a graph records nothing.  Recorded events are held until the next
 * moe_timing_read, so a long run reads from time to time.  The events add a
 * few microseconds of host work per stage; the numbers are for breakdowns,
 * not for the benchmark's figures.
 * ------------------------------------------------------------------------- */
enum {
  MOE_ST_NORM = 0,    /* RMS norm of the residual (moe_layer_decode_residual) */
  MOE_ST_ROUTE = 1,   /* router logits, top-K and weights */
  MOE_ST_BUCKET = 2,  /* pairs grouped by expert, x staged (T >= 4) */
  MOE_ST_GATEUP = 3,  /* gate and up products, SwiGLU (unfused kernels) */
  MOE_ST_DOWN = 4,    /* down products (unfused kernels; T <= 3: and combine) */
  MOE_ST_COMBINE = 5, /* weighted combine (T >= 4) */
  MOE_ST_RESID = 6,   /* residual add (moe_layer_decode_residual) */
  MOE_ST_LAYER = 7,   /* the whole layer in one kernel (single-token path) */
  MOE_ST_STACK = 8,   /* layers of one token in one kernel (per launch) */
  MOE_TIMING_STAGES = 9
};

typedef struct {
  double ms[MOE_TIMING_STAGES];    /* total time per stage, milliseconds */
  int64_t count[MOE_TIMING_STAGES]; /* times each stage ran */
} moe_timing;

/* Switches timing on (on != 0) or off.  Host only; always MOE_OK. */
moe_status moe_timing_set(int32_t on);

/* Waits for the events recorded so far (synchronises the host with them),
 * writes the totals since the last reset to *out and, if reset != 0, sets
 * them to zero.  MOE_ERR_NULL for out == NULL; MOE_ERR_HIP if an event call
 * failed since the last read (the totals then miss those stages). */
moe_status moe_timing_read(moe_timing *out, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
