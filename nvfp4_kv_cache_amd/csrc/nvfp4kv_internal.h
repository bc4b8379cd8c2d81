// Internal interface between the host library (cache manager, argument checks)
// and the gfx950 kernels.  Plain C++ types only: the host side also builds with g++
// (for CPU tests of the cache metadata) against a recording stand-in of these
// launch functions.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace nvfp4kv {

constexpr int kMaxFrames = 64;            // sink + window frame slots
constexpr int kScaleSlots = kMaxFrames + 1;
constexpr int kMaxSegments = kMaxFrames;  // one per resident frame at worst
constexpr int kMaxQuantGrid = 2048;       // workgroups of one quantize launch
constexpr int kQuantThreads = 256;

// Quantizer scratch.  partial: per-workgroup maxima of |x| (fp32 bit patterns)
// written by the amax pass and read by the encode pass of the same call.  slot:
// one word per workgroup of the single-pass kernel, (epoch << 30) | (K max << 15) |
// V max with the maxima as |bf16| bit patterns; a slot is current only when it holds
// the launch's epoch, so the words must start zeroed and epochs never repeat.
struct QuantWorkspace {
  uint32_t partial[2][kMaxQuantGrid];
  uint64_t slot[kMaxQuantGrid];
};

// One tensor of a quantize launch.  Source: bf16 [H][T][D].  Destination, canonical
// layout: codes [H][rows][D/2], scales [H][rows][D/16]; transposed layout (V in the
// cache): codes [H][D][rows/2] (token 2i in the low nibble), scales [H][D/16][rows].
struct QuantTensor {
  const uint16_t *src;
  uint8_t *codes;
  uint8_t *scales;
  float *tensor_scale;   // receives s_t
  int32_t transposed;
  int32_t adaptive;      // choose each block's scale between the 6- and 4-candidates
  const float *mean;     // K-smoothing: channel means [H][D] subtracted first, or null
};

struct QuantArgs {
  QuantTensor t[2];
  int32_t n_tensors;
  int32_t H, T, D;
  int32_t tokens_per_frame;   // T_f; source token t is frame t / T_f
  int32_t n_frames;
  int64_t rows;               // destination tokens per head
  int32_t tile_tokens;        // tokens per workgroup tile (set by the launcher)
  int32_t tiles_per_head;     // set by the launcher
  int32_t total_tiles;        // set by the launcher
  int32_t spin_limit;         // polls of the single-pass wait before its fallback scan
  uint64_t epoch;             // > 0: the single-pass kernel may be used with this epoch
  QuantWorkspace *ws;
  // Single pass with K-smoothing (null: the options take the two passes).  Words
  // (low 32 bits of the epoch) << 32 | fp32 bits, current only when the tag matches
  // the launch's epoch, so they start zeroed and the low half of an epoch is never 0.
  uint64_t *sum_slots;        // [2][H][tiles_per_head][D]: each K tile's channel sums, then
                              // its channel extremes (bf16 bits of the largest << 16 | smallest)
  uint64_t *cmax_slots;       // [16 x kMaxQuantGrid]: each head's max |K - mean|, one word
                              // per 128-byte line (every K workgroup of the head writes it)
  float *k_mean_out;          // receives the channel means [H][D]
  int32_t frame_slot[kMaxFrames];   // destination slot of each source frame
};

// Tokens of one quantizer tile for the cache's head_dim (one octet of tokens per
// thread, 256 threads, D/16 threads per octet).
inline int64_t quant_tile_tokens(int D) { return int64_t(8) * kQuantThreads / (D / 16); }
// Words of the K-smoothing single pass's slots for chunks of up to t_max tokens: the
// head words, the tile statistics, and slack for the reads of the statistics past a
// head's last tile (at most max(tiles_per_head, 16) nodes of 64 words).
inline size_t option_slot_words(int H, int64_t t_max, int D) {
  const int64_t tt = quant_tile_tokens(D);
  const int64_t tiles = (t_max + tt - 1) / tt;
  return size_t(16 * kMaxQuantGrid + 2 * int64_t(H) * tiles * D + (tiles + 16) * 64);
}

// One level of the K-smoothing channel sums: a pairwise tree over each channel's
// tokens (padded with +0.0 to a power of two), `group` leaves per workgroup.
struct MeanLevel {
  const uint16_t *src16;      // first level: bf16 K [H][T][D]; leaves past T are +0.0
  const float *src32;         // later levels: node sums [H][n_in][D]
  float *dst;                 // node sums [H][n_in / group][D]; at the last level the
                              // means [H][D] (root / T)
  int32_t H, D, T;
  int32_t n_in;               // leaves per head at this level (a power of two)
  int32_t group;              // leaves per workgroup (a power of two, at most 256)
  int32_t last;
};
constexpr int kMeanGroup = 256;

struct Segment {
  int32_t tok0;        // first token (slot * T_f) in the cache rows
  int32_t ntok;
  int32_t scale_slot;  // index into the tensor-scale table
  int32_t pad;
};

// Attention load balancing.  The key tiles of all (head, query block) pairs form one
// list of work units that is cut into equal ranges, one per workgroup.  A query block
// cut between workgroups gf < gf+1 < ... < g is finished by g, which holds its LAST
// tiles and processes them last (each workgroup walks its share from the end): every
// earlier workgroup holds an earlier part of the block as the first range it
// processes, publishes that partial result in its slot and tags its flag with the
// launch's epoch; g waits for those flags (bounded), merges the partials in
// workgroup order, and on a timeout processes the block's earlier tiles itself.
// Scratch (in the cache's storage): one slot and one flag per workgroup (flags
// start zeroed; epochs never repeat).
constexpr int kAttnMaxCus = 256;
constexpr int attn_wg_per_cu(int D) { return D >= 128 ? 1 : 2; }
constexpr int attn_max_grid(int D) { return kAttnMaxCus * attn_wg_per_cu(D); }
constexpr int attn_block_queries(int D) { return (D >= 128 ? 8 : 4) * 32; }
constexpr int attn_threads(int D) { return (D >= 128 ? 8 : 4) * 64; }
// one partial: the query block's unnormalized output (fp32) + per-lane max and sum
constexpr size_t attn_slot_bytes(int D) {
  return size_t(attn_block_queries(D)) * D * 4 + size_t(attn_threads(D)) * 8;
}

struct AttnArgs {
  const uint16_t *q, *k_own, *v_own;
  float *out;
  const uint8_t *kcodes, *kscales, *vcodes, *vscales;   // cache planes
  const float *scale_table;                               // [slot][2] = {s_K, s_V}
  int64_t rows;                                           // cache tokens per head
  int32_t H, D, n_q;
  float sm_scale_log2;                                    // softmax_scale * log2(e)
  int32_t n_seg;
  // set by the launcher: key tiles per query block, by kind (cache full tiles, cache
  // ragged tails, own full tiles, own ragged tail), and the total work
  int32_t n_cfull, n_ctail, n_ofull, n_otail, tiles;
  // cost weights of a cache full tile, a ragged tail and an own full tile; a block's
  // total weight; the work list is cut by weight
  int32_t w_cfull, w_tail, w_ofull, w_block;
  int32_t mx;                 // 0: NVFP4 cache; 1: MXFP4 (E8M0 scales per 32); 2: MXFP4 with MX-scaled QK^T
  int64_t work;               // query blocks x block weight
  const float *k_mean;        // K-smoothing means [scale slot][H][D], or null
  float *partials;            // [max grid][slot]
  uint64_t *flags;            // [max grid]: epoch of the last partial published in the slot
  uint64_t epoch;             // > 0, never repeated for one scratch area
  int32_t spin_limit;         // polls before a workgroup stops waiting for a partial
  int32_t pad2;
  Segment seg[kMaxSegments];
};

struct ExportArgs {
  const uint8_t *kcodes, *kscales, *vcodes, *vscales;
  const float *scale_table;
  int32_t scale_slot;
  int32_t H, D, T_f, n_frames;
  int32_t block;              // elements per block scale: 16 (NVFP4) or 32 (MXFP4)
  int64_t rows;
  uint8_t *k_codes_out, *k_scales_out, *v_codes_out, *v_scales_out;
  float *k_scale_out, *v_scale_out;
  int32_t frame_slot[kMaxFrames];
};

// Launchers: return 0 or a negative nvfp4kv_status (EHIP).  `stream` is hipStream_t.
int launch_quantize(const QuantArgs &a, void *stream);
// 1 if launch_quantize would take the single-pass kernel for these arguments on the
// current device, 0 for the two passes, or a negative status.
int quantize_single_pass(const QuantArgs &a);
// Appends with K-smoothing (k_mean: the chunk's means [H][D], written) and/or adaptive
// V scales (a.t[1].adaptive): the single pass with the options when it fits on the
// device at once (a.epoch > 0, and the slots given for K-smoothing), else the channel
// means (kmean_ws: channel_mean_ws_floats(H, T, D) floats) and the two passes.
int launch_quantize_options(const QuantArgs &a, float *k_mean, float *kmean_ws, void *stream);
// 1 if launch_quantize_options would take its single pass, 0 if not, or a negative status.
int quantize_options_single_pass(const QuantArgs &a, bool k_smooth, bool v_adaptive);
// Same-size streaming reference of a two-tensor codec launch (measurement hook).
int launch_stream_reference(const QuantArgs &a, void *stream);
// The standalone codec with its workspace in the library's per-device scratch array
// (a.ws is ignored): no allocation.  EHIP if the array's address cannot be resolved.
constexpr size_t kNoAllocScratchBytes = sizeof(QuantWorkspace);
int launch_quantize_noalloc(const QuantArgs &a, void *stream);
// MXFP4 (32-element blocks, E8M0 scales, no tensor scale): one pass
int launch_quantize_mx(const QuantArgs &a, void *stream);
int launch_attention(const AttnArgs &a, void *stream);
int launch_export(const ExportArgs &a, void *stream);
// K-smoothing channel means of one chunk tensor k [H][T][D] into mean [H][D]; ws holds
// at least channel_mean_ws_floats(H, T, D) floats (two buffers of level node sums).
inline size_t channel_mean_ws_floats(int H, int T, int D) {
  int64_t P = 1;
  while (P < T) P *= 2;
  const int64_t nodes = P > kMeanGroup ? P / kMeanGroup : 1;
  return size_t(2 * int64_t(H) * nodes * D);
}
int launch_channel_mean(const uint16_t *k, int H, int T, int D, float *mean, float *ws, void *stream);
int copy_device_floats(float *dst, const float *src, size_t n, void *stream);
int zero_device_bytes_blocking(void *ptr, size_t bytes);

}  // namespace nvfp4kv
