/*
 * nvfp4kv.h -- C ABI of the MI355X (gfx950) NVFP4 KV-cache chunk-attention library.
 *
 * Sources of the operations (pages: "LongLive-2.0: An NVFP4 Parallel Infrastructure
 * for Long Video Generation", the paper text and a reading note on it):
 *   - NVFP4 format: paper section 2.2 "NVFP4 Training" (16-element blocks, E4M3 block
 *     scale with max 448, E2M1 elements with max 6) and the reading note, section II
 *     "The NVFP4 quantization format" (one FP32 tensor scale x one E4M3 scale per 16
 *     elements x the E2M1 element).
 *   - Per-chunk KV quantization and in-kernel dequantization: paper section 1 and the
 *     reading note, "The inference infrastructure" (frame-chunk granularity,
 *     9/8 T_c H d bytes for K and V, dequantization inside the attention kernel).
 *   - Sink + window cache: paper section 4.2 "Inference with Multi-Shot Attention Sink"
 *     (sliding window of W chunks, global sink of the first S_g frames, effective key
 *     set = sink U window with duplicates removed).
 *   - Chunk attention: paper section 2.1 (a noisy chunk attends to the clean history
 *     and to its own tokens) with section 4.2's cache as the history.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers owned by the caller unless marked "host".  The
 *     library never allocates device memory (no hipMalloc); callers bring inputs,
 *     outputs, cache storage and workspace.
 *   - bf16 tensors are passed as their uint16 bit patterns; all tensors are dense and
 *     row-major in the order of their stated shape.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *     call validates its arguments on the host first, then enqueues work on `stream`
 *     and returns without synchronizing.  An argument error returns a negative status
 *     before anything is enqueued.  A HIP launch error returns NVFP4KV_EHIP; a device
 *     fault shows at the caller's next synchronization.
 *   - Return value: 0 (NVFP4KV_OK) or a negative nvfp4kv_status.  No exceptions, no
 *     abort, no printing.
 *   - A kvcache handle must not be used by two threads, or from two streams whose work
 *     may overlap, at the same time.
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4KV_OK = 0,
  NVFP4KV_EINVAL = -1,    /* null pointer, non-positive or unsupported size        */
  NVFP4KV_ESHAPE = -2,    /* shapes inconsistent with the cache configuration      */
  NVFP4KV_ECAPACITY = -3, /* request does not fit (workspace, window, frame count) */
  NVFP4KV_ESTATE = -4,    /* e.g. evicting more frames than the window holds       */
  NVFP4KV_EHIP = -5       /* HIP runtime / launch error                            */
} nvfp4kv_status;

/* Static, NUL-terminated description of a status code (host). */
const char *nvfp4kv_strerror(int status);

/* Library version as "major.minor.patch" (host, static string). */
const char *nvfp4kv_version(void);

/* Testing hook for the two bounded waits between workgroups; either way the results
 * are the same.  kvcache_append's single-pass quantizer: workgroups exchange their
 * maxima through the cache's workspace; a workgroup that has polled `limit` times
 * without finding every other workgroup's maxima helps instead, computing one missing
 * workgroup's tile maxima per further poll and publishing them in its place (bounded
 * extra work: about one more read of the chunk in all).  With K-smoothing the K
 * workgroups also exchange their tiles' channel sums and their max |K - mean| the same
 * way (a helper computes a missing tile's sums, or its maximum after the means of its
 * head: at most about two more reads of K).
 * chunk_attention: a query block cut between workgroups is finished by the one that
 * holds its LAST key tiles: the workgroups holding its earlier tiles each publish the
 * partial result of their part, and the last one waits for them for at most `limit`
 * polls per partial, merges them in workgroup order, or, when one is still missing,
 * processes the block's earlier tiles itself.
 * Default 65536; a small limit exercises the fallbacks.  Process-wide, read at each
 * call.  Errors: EINVAL (limit < 0). */
int nvfp4kv_set_wait_limit(int32_t limit);

/* ------------------------------------------------------------------------------
 * Standalone NVFP4 codec of one tensor (paper section 2.2; reading note section II).
 *
 *   x            bf16 [H, T, D], D % 16 == 0 (16 <= D <= 4096), H, T >= 1 (T may be odd).
 *   codes        uint8 [H, T, D/2]: element 2i in the low nibble, 2i+1 in the high
 *                nibble; nibble = sign << 3 | E2M1 magnitude code.
 *   scales       uint8 [H, T, D/16]: raw E4M3FN bytes of the block scales.
 *   tensor_scale float[1]: s_t = amax(|x|) / (6 * 448) over the whole tensor.
 * Recipe (fp32, round-to-nearest-even, no fast math): block scale
 *   bs = (block amax / 6) / s_t rounded to E4M3 (saturating at 448), element code =
 *   E2M1(|x| / (E4M3(bs) * s_t)) (saturating at 6); a block whose E4M3(bs) * s_t is 0
 *   gets all-zero magnitudes with the element signs kept.  x must be finite.
 *   workspace    device scratch of >= nvfp4_quantize_workspace_bytes() bytes (per-
 *                workgroup partial maxima; needs no initialization).  Calls that
 *                share a workspace must not run concurrently.
 * Alignment: x 16 bytes, codes 8 bytes, tensor_scale 4 bytes.
 * Errors: EINVAL (null or misaligned pointer, H/T/D out of range, D % 16 != 0), ECAPACITY (workspace
 * too small), EHIP.
 * ------------------------------------------------------------------------------ */
size_t nvfp4_quantize_workspace_bytes(void);
int nvfp4_quantize_kv(const uint16_t *x, int64_t H, int64_t T, int64_t D, uint8_t *codes,
                      uint8_t *scales, float *tensor_scale, void *workspace,
                      size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------
 * The same codec for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results and errors are those of nvfp4_quantize_kv (minus
 * the workspace); the result is bit-identical to it.
 * Scratch: a file-scope device array of nvfp4_quantize_noalloc_scratch_bytes()
 * (32 KiB) inside the library, one per GPU, held until the process ends; its address
 * is resolved on the first call on each device.  The codec's scratch need does not
 * grow with the input (one partial maximum per workgroup of its first pass, at most
 * 256), so every input nvfp4_quantize_kv accepts fits; a need beyond the array would
 * return NVFP4KV_ECAPACITY.  The call allocates nothing (no hipMalloc, no allocating
 * library routine).  Every call on a GPU shares that GPU's array: calls that may
 * overlap on one GPU (two streams, two threads) race and must be serialized by the
 * caller.  Errors: as nvfp4_quantize_kv; EHIP also if the array's device address
 * cannot be resolved.
 * ------------------------------------------------------------------------------ */
size_t nvfp4_quantize_noalloc_scratch_bytes(void);
int nvfp4_quantize_kv_noalloc(const uint16_t *x, int64_t H, int64_t T, int64_t D, uint8_t *codes,
                              uint8_t *scales, float *tensor_scale, void *stream);

/* Measurement hook: the bytes of a two-tensor NVFP4 codec call (2 bytes read, 1/2 + 1/16
 * byte written per element) moved with the quantizer's tiling, no exchange between
 * workgroups and almost no arithmetic -- the time this transfer size allows on the GPU.
 * x0, x1 bf16 [H, T, D]; codes0/1 uint8 [H, T, D/2] and scales0/1 uint8 [H, T, D/16]
 * receive bytes derived from the inputs that are NOT an NVFP4 encoding.
 * Errors: EINVAL (null or misaligned pointer, sizes as for nvfp4_quantize_kv), EHIP. */
int nvfp4kv_stream_reference(const uint16_t *x0, const uint16_t *x1, int64_t H, int64_t T, int64_t D,
                             uint8_t *codes0, uint8_t *scales0, uint8_t *codes1, uint8_t *scales1,
                             void *stream);

/* ------------------------------------------------------------------------------
 * Standalone MXFP4 codec of one tensor: the block-scaled FP4 format the paper text's
 * appendix A.2 ("FP4 Quantization") sets against NVFP4, as defined by the OCP
 * Microscaling Formats (MX) specification v1.0 it cites.
 *
 *   x       bf16 [H, T, D], D % 32 == 0 (32 <= D <= 4096), H, T >= 1; finite.
 *   codes   uint8 [H, T, D/2]: as for NVFP4 (element 2i in the low nibble, nibble =
 *           sign << 3 | E2M1 magnitude code).
 *   scales  uint8 [H, T, D/32]: E8M0 bytes E + 127 of the block scales 2^E.
 * Recipe: per block of 32 along D, E = floor(log2(block max |x|)) - 2 clamped to
 *   [-127, 127] (-127 for an all-zero block); code = E2M1(|x| / 2^E) rounded to
 *   nearest-even, saturating at 6, with x's sign.  No tensor scale; one pass, no
 *   workspace.
 * Alignment: x 16 bytes, codes 8 bytes.
 * Errors: EINVAL (null or misaligned pointer, H/T/D out of range, D % 32 != 0), EHIP.
 * ------------------------------------------------------------------------------ */
int mxfp4_quantize_kv(const uint16_t *x, int64_t H, int64_t T, int64_t D, uint8_t *codes,
                      uint8_t *scales, void *stream);

/* ------------------------------------------------------------------------------
 * Paged sink + window KV cache (paper section 4.2; reading note "The inference
 * infrastructure").
 *
 * A frame slot holds one latent frame (tokens_per_frame tokens, all heads) of K and V
 * in NVFP4.  Slots [0, sink_frames) hold the global sink: the first sink_frames frames
 * ever appended, kept for the life of the cache.  The window is a FIFO of the
 * window_frames most recent other frames.  The shot-level sink (paper section 4.2,
 * "Multi-Shot Attention Sink") is the first shot_frames frames of the current shot:
 * such a frame stays in the cache when the window rolls past it, until the next
 * scene cut (kvcache_begin_shot), and is never stored or attended twice.  The first
 * shot starts at the first frame.  The effective key set is global sink U shot-level
 * sink U window.  Frames are never copied; eviction only changes host metadata.
 *
 * Options (reading note, "The inference infrastructure": within each chunk,
 * K-smoothing for K and adaptive scale selection for V):
 *   NVFP4KV_K_SMOOTH    each appended chunk's K has its per-head channel means
 *                       (over the chunk's tokens) subtracted before quantization;
 *                       the means are kept in fp32 and attention adds q . mean back
 *                       to every logit of that chunk's keys.  The mean is a pairwise
 *                       fp32 tree over the tokens padded with +0.0 to a power of two,
 *                       divided by the token count.
 *   NVFP4KV_V_ADAPTIVE  each V block is encoded with its maximum mapped to 6 and to 4
 *                       (same tensor scale) and keeps the encoding with the smaller
 *                       fp32 squared error (ties: 6).  Decoding is unchanged.
 * Appends with options run their own single-pass quantizer when its grid fits on the
 *                       GPU at once (kvcache_append_schedule), else the channel-mean
 *                       reduction and the two-pass quantizer; the results are the same.
 *   NVFP4KV_MXFP4       the cache holds MXFP4 instead (see mxfp4_quantize_kv: 32-element
 *                       blocks, E8M0 scales, no tensor scale; the paper text's appendix
 *                       A.2 contrasts the two formats).  Appends run one single-pass
 *                       kernel; attention dequantizes these tiles to bf16 and runs their
 *                       QK^T and PV on the bf16 matrix cores with plain bf16 Q and P
 *                       rounded to nearest-even.  Not combinable with the two options
 *                       above (steps of the NVFP4 recipe).
 *   NVFP4KV_MX_SCALED_QK  (with NVFP4KV_MXFP4) QK^T of the cache tiles runs on gfx950's
 *                       MX-scaled matrix cores straight from the E2M1 codes and E8M0
 *                       scales: the queries enter that product quantized to MXFP8
 *                       (E4M3 elements, E8M0 scale per 32 along head_dim with exponent
 *                       floor(log2 block max) - 8, nearest-even, saturating at 448).
 *                       The own-segment logits keep the bf16 queries.  This changes the
 *                       results beyond the cache format (the queries are quantized).
 *
 * Supported: n_heads >= 1; head_dim 64 or 128; tokens_per_frame >= 8 and a multiple
 * of 8; sink_frames >= 0; window_frames >= 1; shot_frames >= 0 (0: no shot-level
 * sink); sink_frames + window_frames + shot_frames <= 64; options a combination of
 * the flags above.
 * Every bf16 / fp32 tensor argument must be 16-byte aligned.
 * ------------------------------------------------------------------------------ */
#define NVFP4KV_K_SMOOTH 1
#define NVFP4KV_V_ADAPTIVE 2
#define NVFP4KV_MXFP4 4
#define NVFP4KV_MX_SCALED_QK 8

typedef struct {
  int32_t n_heads;
  int32_t head_dim;
  int32_t tokens_per_frame;
  int32_t sink_frames;
  int32_t window_frames;
  int32_t shot_frames;
  int32_t options;   /* NVFP4KV_K_SMOOTH | NVFP4KV_V_ADAPTIVE, or NVFP4KV_MXFP4 [| NVFP4KV_MX_SCALED_QK], or 0 */
} kvcache_config;

typedef struct kvcache kvcache; /* opaque host object */

/* Device bytes the cache needs: 9/16 byte per cached K or V element (codes + block
 * scales, i.e. 9/8 T H d for K and V together; 17/32 byte for MXFP4), plus scratch of a
 * fixed size that does not grow with the cache: a per-chunk tensor-scale table, the quantizer's workspace
 * and chunk_attention's load-balancing slots (one partial query-block result per
 * workgroup of a full-GPU launch: about 34.6 MB for head_dim 128, 17.8 MB for 64).
 * Returns 0 for an unsupported configuration. */
size_t kvcache_storage_bytes(const kvcache_config *cfg);

/* Creates the host object over caller-owned device storage (>= kvcache_storage_bytes,
 * 256-byte aligned).  Zero-fills the storage's control words with a blocking copy on
 * the current device.  Errors: EINVAL, ECAPACITY (storage too small), EHIP. */
int kvcache_create(const kvcache_config *cfg, void *storage, size_t storage_bytes,
                   kvcache **out /* host */);

/* Frees the host object only; the storage stays the caller's.  NULL is accepted. */
int kvcache_destroy(kvcache *c);

/* Appends one chunk of n_frames frames.  k, v: bf16 [H, n_frames * tokens_per_frame, D]
 * (finite).  K and V each get one FP32 tensor scale computed over the whole chunk (all
 * heads), then are quantized straight into their frame slots in one kernel.  The first
 * sink_frames frames ever appended become sinks; each later frame enters the window,
 * and when the window is full the oldest window frame is evicted first (FIFO).
 * Errors: EINVAL (null or misaligned, n_frames < 1), ECAPACITY (more than window_frames frames of
 * this chunk would enter the window), ESTATE (2^31 - 1 chunks already appended to this
 * cache: chunk numbers and the kernels' epoch tags would repeat), EHIP. */
int kvcache_append(kvcache *c, const uint16_t *k, const uint16_t *v, int32_t n_frames,
                   void *stream);

/* The kernel schedule an append of n_frames frames takes on the current device (host
 * output): 1 = the single-pass quantizer (one kernel, each chunk element read once),
 * 2 = the two-pass quantizer (a grid that would not fit on the GPU at once; with
 * K-smoothing, after the channel-mean reduction), 3 = the MXFP4 quantizer (one kernel,
 * no exchange between workgroups), 4 = the single-pass quantizer with the cache's
 * K-smoothing and/or adaptive V scales (one kernel; K workgroups also exchange their
 * tiles' channel sums and their max |K - mean|).  Errors: EINVAL, EHIP. */
int kvcache_append_schedule(const kvcache *c, int32_t n_frames, int32_t *schedule);

/* Drops the oldest n_frames window frames (never sinks); metadata only.
 * Errors: EINVAL (n_frames < 0), ESTATE (fewer than n_frames window frames). */
int kvcache_evict(kvcache *c, int32_t n_frames);

/* Number of cached tokens in the global sink and in the window (host outputs). */
int kvcache_tokens(const kvcache *c, int64_t *sink_tokens, int64_t *window_tokens);

/* Scene cut: the next appended frame starts a new shot, whose first shot_frames
 * frames form the new shot-level sink.  The old shot's sink frames that are no
 * longer in the window leave the cache (metadata only).  Errors: EINVAL (null). */
int kvcache_begin_shot(kvcache *c);

/* The shot-level sink as its two pointers (host outputs): start_frame, the index of
 * the current shot's first frame among all frames ever appended, and n_frames, how
 * many of its first shot_frames frames have been appended; extra_tokens, the tokens
 * of those frames that are in neither the global sink nor the window (attended in
 * addition to kvcache_tokens' two counts).  Errors: EINVAL (null). */
int kvcache_shot_sink(const kvcache *c, int64_t *start_frame, int32_t *n_frames,
                      int64_t *extra_tokens);

/* Number of chunks appended so far (the next chunk's index) (host output). */
int kvcache_chunk_count(const kvcache *c, int32_t *n_chunks);

/* Noisy-chunk attention (paper sections 2.1 and 4.2): for every head,
 *   out = softmax(q K^T * softmax_scale) V,  K = [cache K ; k_own],  V = [cache V ; v_own]
 * over all cached tokens (global sink, shot-level sink and window; NVFP4, or MXFP4 with
 * NVFP4KV_MXFP4, dequantized inside the kernel) and
 * the chunk's own n_q bf16 tokens, with no mask (bidirectional inside the chunk).
 *   q, k_own, v_own  bf16 [H, n_q, D] (finite);
 *   out              fp32 [H, n_q, D];  n_q >= 1;  softmax_scale > 0 and finite.
 * The work (query blocks x key tiles) is spread evenly over every CU; query blocks
 * cut between workgroups are merged through the cache's scratch, so attention calls
 * on one cache must not run concurrently (calls on different caches may).
 * Errors: EINVAL (null or misaligned pointer, bad size or scale), EHIP. */
int chunk_attention(const kvcache *c, const uint16_t *q, const uint16_t *k_own,
                    const uint16_t *v_own, int64_t n_q, float softmax_scale, float *out,
                    void *stream);

/* Copies chunk `chunk_index` (0-based append order), which must be fully resident,
 * out of the cache in the codec's layout: k_codes / v_codes uint8 [H, n*T_f, D/2],
 * k_scales / v_scales uint8 [H, n*T_f, D/16] (MXFP4: E8M0 bytes [H, n*T_f, D/32]),
 * k_scale / v_scale float[1] (device; 1 for MXFP4), with n the chunk's frame count.
 * Device-to-device, on `stream`.
 * Errors: EINVAL (null), ESTATE (chunk unknown or not fully resident), EHIP. */
int kvcache_export_chunk(const kvcache *c, int32_t chunk_index, uint8_t *k_codes,
                         uint8_t *k_scales, uint8_t *v_codes, uint8_t *v_scales,
                         float *k_scale, float *v_scale, void *stream);

/* K-smoothing means of a resident chunk: k_mean fp32 [H, D] (device), the values
 * subtracted from its K before quantization.  Device-to-device, on `stream`.
 * Errors: EINVAL (null, or the cache has no NVFP4KV_K_SMOOTH), ESTATE (chunk not
 * resident), EHIP. */
int kvcache_export_k_mean(const kvcache *c, int32_t chunk_index, float *k_mean, void *stream);

/* Frame count of a resident chunk (host output); ESTATE if not resident. */
int kvcache_chunk_frames(const kvcache *c, int32_t chunk_index, int32_t *n_frames);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4KV_H */
