// C ABI of libnvfp4kv: argument checks, the sink + window cache metadata, and the
// hand-off to the gfx950 kernels.  Declared in include/nvfp4kv.h.
//
// Cache semantics follow the paper text, section 4.2 "Inference with Multi-Shot
// Attention Sink": a sliding window of recent frames plus a global sink made of
// the first S_g frames, kept permanently; the effective key set is their union,
// each frame stored once.  The reading note's "The inference infrastructure"
// fixes the per-chunk NVFP4 quantization of K and V (one tensor scale each).

#include <string.h>

#include <atomic>
#include <map>
#include <new>

#include "../../include/nvfp4kv.h"
#include "nvfp4kv_internal.h"

using namespace nvfp4kv;

namespace {

constexpr size_t kAlign = 256;
constexpr int32_t kDefaultSpinLimit = 1 << 16;
std::atomic<int32_t> g_spin_limit{kDefaultSpinLimit};

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Layout {
  int64_t rows;   // token capacity per head
  size_t kcodes, kscales, vcodes, vscales, table, ws, opt_slots, attn_flags, attn_part, kmean, kmean_ws, total;
};

bool config_ok(const kvcache_config *c) {
  if (!c) return false;
  if (c->n_heads < 1 || c->n_heads > 4096) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->tokens_per_frame < 8 || c->tokens_per_frame % 8 != 0 ||
      c->tokens_per_frame > (1 << 20))
    return false;
  if (c->sink_frames < 0 || c->window_frames < 1 || c->shot_frames < 0) return false;
  if (c->options & ~(NVFP4KV_K_SMOOTH | NVFP4KV_V_ADAPTIVE | NVFP4KV_MXFP4 | NVFP4KV_MX_SCALED_QK)) return false;
  if ((c->options & NVFP4KV_MX_SCALED_QK) && !(c->options & NVFP4KV_MXFP4)) return false;
  // smoothing and adaptive 4/6 scales are steps of the NVFP4 recipe
  if ((c->options & NVFP4KV_MXFP4) && (c->options & (NVFP4KV_K_SMOOTH | NVFP4KV_V_ADAPTIVE))) return false;
  if (c->sink_frames + c->window_frames + c->shot_frames > kMaxFrames) return false;
  // per-head planes are addressed with 32-bit offsets
  if (int64_t(c->sink_frames + c->window_frames + c->shot_frames) * c->tokens_per_frame * c->head_dim >=
      (int64_t(1) << 31))
    return false;
  return true;
}

bool make_layout(const kvcache_config *c, Layout *L) {
  if (!config_ok(c)) return false;
  const int64_t H = c->n_heads, D = c->head_dim;
  L->rows = int64_t(c->sink_frames + c->window_frames + c->shot_frames) * c->tokens_per_frame;
  if (H * L->rows * D > (int64_t(1) << 40)) return false;
  size_t off = 0;
  L->kcodes = off;  off = round_up(off + size_t(H * L->rows * D / 2));
  const int64_t block = (c->options & NVFP4KV_MXFP4) ? 32 : 16;   // elements per block scale
  L->kscales = off; off = round_up(off + size_t(H * L->rows * D / block));
  L->vcodes = off;  off = round_up(off + size_t(H * L->rows * D / 2));
  L->vscales = off; off = round_up(off + size_t(H * L->rows * D / block));
  L->table = off;   off = round_up(off + sizeof(float) * 2 * kScaleSlots);
  L->ws = off;      off = round_up(off + sizeof(QuantWorkspace));
  const int64_t t_max = int64_t(c->sink_frames + c->window_frames) * c->tokens_per_frame;
  L->opt_slots = off;
  if (c->options & NVFP4KV_K_SMOOTH)   // the smoothing single pass's exchange words (zeroed)
    off = round_up(off + sizeof(uint64_t) * option_slot_words(int(H), t_max, int(D)));
  L->attn_flags = off; off = round_up(off + sizeof(uint64_t) * attn_max_grid(int(D)));
  L->attn_part = off; off = round_up(off + attn_max_grid(int(D)) * attn_slot_bytes(int(D)));
  L->kmean = off;
  L->kmean_ws = off;
  if (c->options & NVFP4KV_K_SMOOTH) {
    // per scale slot, the K channel means of its chunk; and the reduction's workspace
    // for the longest chunk an append accepts (sink + window frames)
    off = round_up(off + sizeof(float) * kScaleSlots * H * D);
    L->kmean_ws = off;
    off = round_up(off + sizeof(float) * channel_mean_ws_floats(int(H), int(t_max), int(D)));
  }
  L->total = off;
  return true;
}

struct FrameRec {
  int32_t chunk;
  int32_t frame_in_chunk;
  int64_t frame;              // index among all frames ever appended
};

struct ChunkRec {
  int32_t scale_slot;
  int32_t n_frames;
  int32_t resident;
  int32_t slot[kMaxFrames];   // slot of each frame, -1 once evicted
};

// Slots [0, sink_frames) hold the global sink.  The other slots form a pool shared by
// the window (a FIFO of at most window_frames frames) and the shot-level sink: a
// frame among the first shot_frames frames of the current shot keeps its slot after
// it leaves the window, until the next scene cut.  The pool has window_frames +
// shot_frames slots, which is always enough.
struct State {
  int32_t sink_used = 0;
  int32_t win[kMaxFrames];    // window slots, oldest first, as a ring
  int32_t win_head = 0;
  int32_t win_count = 0;
  int64_t next_frame = 0;     // frames appended so far
  int64_t shot_start = 0;     // first frame of the current shot
  int32_t next_chunk = 0;
  FrameRec slot_frame[kMaxFrames];
  bool slot_used[kMaxFrames] = {false};   // pool slots holding a resident frame
  int32_t scale_ref[kScaleSlots] = {0};
  std::map<int32_t, ChunkRec> chunks;   // resident chunks only
};

}  // namespace

struct kvcache {
  kvcache_config cfg;
  Layout L;
  uint8_t *base;
  State st;
  uint64_t epoch = 0;   // last epoch given to the single-pass quantizer (workspace zeroed at create)
  mutable uint64_t attn_epoch = 0;   // last epoch given to an attention launch (flags zeroed at create)

  uint8_t *kcodes() const { return base + L.kcodes; }
  uint8_t *kscales() const { return base + L.kscales; }
  uint8_t *vcodes() const { return base + L.vcodes; }
  uint8_t *vscales() const { return base + L.vscales; }
  float *table() const { return reinterpret_cast<float *>(base + L.table); }
  QuantWorkspace *ws() const { return reinterpret_cast<QuantWorkspace *>(base + L.ws); }
  uint64_t *attn_flags() const { return reinterpret_cast<uint64_t *>(base + L.attn_flags); }
  float *attn_partials() const { return reinterpret_cast<float *>(base + L.attn_part); }
  bool k_smooth() const { return (cfg.options & NVFP4KV_K_SMOOTH) != 0; }
  bool mx() const { return (cfg.options & NVFP4KV_MXFP4) != 0; }
  float *kmean(int32_t scale_slot) const {
    return reinterpret_cast<float *>(base + L.kmean) + int64_t(scale_slot) * cfg.n_heads * cfg.head_dim;
  }
  float *kmean_ws() const { return reinterpret_cast<float *>(base + L.kmean_ws); }
  uint64_t *cmax_slots() const { return reinterpret_cast<uint64_t *>(base + L.opt_slots); }
  uint64_t *sum_slots() const { return cmax_slots() + 16 * kMaxQuantGrid; }
  int32_t window_slot(const State &s, int32_t i) const { return s.win[(s.win_head + i) % kMaxFrames]; }
  bool in_shot_sink(const State &s, int64_t frame) const {
    return frame >= s.shot_start && frame < s.shot_start + cfg.shot_frames;
  }
  bool in_window(const State &s, int32_t slot) const {
    for (int32_t i = 0; i < s.win_count; ++i)
      if (window_slot(s, i) == slot) return true;
    return false;
  }
};

namespace {

// Frees a pool slot: its frame leaves the cache (metadata only).
void release_slot(State &s, int32_t slot) {
  const FrameRec fr = s.slot_frame[slot];
  auto it = s.chunks.find(fr.chunk);
  if (it != s.chunks.end()) {
    ChunkRec &rec = it->second;
    rec.slot[fr.frame_in_chunk] = -1;
    rec.resident -= 1;
    s.scale_ref[rec.scale_slot] -= 1;
    if (rec.resident == 0) s.chunks.erase(it);
  }
  s.slot_used[slot] = false;
}

// Drops the oldest n window frames of `s`; a frame of the current shot-level sink
// keeps its slot (it stays in the effective key set).
void evict_oldest(const kvcache *c, State &s, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    const int32_t slot = c->window_slot(s, 0);
    s.win_head = (s.win_head + 1) % kMaxFrames;
    s.win_count -= 1;
    if (!c->in_shot_sink(s, s.slot_frame[slot].frame)) release_slot(s, slot);
  }
}

// Pool slots of shot-level-sink frames that are no longer in the window, in frame
// order.
int pinned_frames(const kvcache *c, const State &s, int32_t *slots) {
  int n = 0;
  const int32_t lo = c->cfg.sink_frames, hi = lo + c->cfg.window_frames + c->cfg.shot_frames;
  for (int32_t sl = lo; sl < hi; ++sl)
    if (s.slot_used[sl] && !c->in_window(s, sl)) slots[n++] = sl;
  for (int i = 1; i < n; ++i)   // insertion sort by frame index (n <= 64)
    for (int j = i; j > 0 && s.slot_frame[slots[j]].frame < s.slot_frame[slots[j - 1]].frame; --j) {
      const int32_t t = slots[j];
      slots[j] = slots[j - 1];
      slots[j - 1] = t;
    }
  return n;
}

// Resident frames in effective-key order: global sink, shot-level-sink frames that
// left the window (virtually prepended to it), then the window oldest first.  Each
// frame appears once.
int collect_frames(const kvcache *c, int32_t *slots) {
  int n = 0;
  for (int32_t i = 0; i < c->st.sink_used; ++i) slots[n++] = i;
  n += pinned_frames(c, c->st, slots + n);
  for (int32_t i = 0; i < c->st.win_count; ++i) slots[n++] = c->window_slot(c->st, i);
  return n;
}

}  // namespace

extern "C" {

const char *nvfp4kv_strerror(int status) {
  switch (status) {
    case NVFP4KV_OK: return "ok";
    case NVFP4KV_EINVAL: return "invalid argument (null pointer or unsupported size)";
    case NVFP4KV_ESHAPE: return "shape inconsistent with the cache configuration";
    case NVFP4KV_ECAPACITY: return "request exceeds capacity (workspace, window or frame count)";
    case NVFP4KV_ESTATE: return "operation not valid in the current cache state";
    case NVFP4KV_EHIP: return "HIP runtime or kernel launch error";
    default: return "unknown status";
  }
}

const char *nvfp4kv_version(void) { return "0.1.0"; }

size_t nvfp4_quantize_workspace_bytes(void) { return sizeof(QuantWorkspace); }

namespace {
// Argument checks and launch arguments of the standalone codec (workspace apart).
int codec_args(const uint16_t *x, int64_t H, int64_t T, int64_t D, uint8_t *codes, uint8_t *scales,
               float *tensor_scale, QuantArgs *a) {
  if (!x || !codes || !scales || !tensor_scale) return NVFP4KV_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4)) return NVFP4KV_EINVAL;
  if (H < 1 || T < 1 || D < 16 || D % 16 != 0 || D > 4096) return NVFP4KV_EINVAL;
  if (H * T * D >= (int64_t(1) << 40) || T > (int64_t(1) << 30) || H > (1 << 20))
    return NVFP4KV_EINVAL;
  memset(a, 0, sizeof(*a));
  a->t[0].src = x;
  a->t[0].codes = codes;
  a->t[0].scales = scales;
  a->t[0].tensor_scale = tensor_scale;
  a->t[0].transposed = 0;
  a->n_tensors = 1;
  a->H = int32_t(H);
  a->T = int32_t(T);
  a->D = int32_t(D);
  a->tokens_per_frame = int32_t(T);
  a->n_frames = 1;
  a->rows = T;
  a->frame_slot[0] = 0;
  return NVFP4KV_OK;
}
}  // namespace

int nvfp4_quantize_kv(const uint16_t *x, int64_t H, int64_t T, int64_t D, uint8_t *codes,
                      uint8_t *scales, float *tensor_scale, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!workspace || !aligned(workspace, 4)) return NVFP4KV_EINVAL;
  QuantArgs a;
  if (int rc = codec_args(x, H, T, D, codes, scales, tensor_scale, &a)) return rc;
  if (workspace_bytes < sizeof(QuantWorkspace)) return NVFP4KV_ECAPACITY;
  a.ws = reinterpret_cast<QuantWorkspace *>(workspace);
  return launch_quantize(a, stream);
}

int nvfp4kv_stream_reference(const uint16_t *x0, const uint16_t *x1, int64_t H, int64_t T, int64_t D,
                             uint8_t *codes0, uint8_t *scales0, uint8_t *codes1, uint8_t *scales1,
                             void *stream) {
  if (!x0 || !x1 || !codes0 || !scales0 || !codes1 || !scales1) return NVFP4KV_EINVAL;
  if (!aligned(x0, 16) || !aligned(x1, 16) || !aligned(codes0, 8) || !aligned(codes1, 8)) return NVFP4KV_EINVAL;
  if (H < 1 || T < 1 || D < 16 || D % 16 != 0 || D > 4096) return NVFP4KV_EINVAL;
  if (H * T * D >= (int64_t(1) << 40) || T > (int64_t(1) << 30) || H > (1 << 20)) return NVFP4KV_EINVAL;
  QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.t[0] = QuantTensor{x0, codes0, scales0, nullptr, 0, 0, nullptr};
  a.t[1] = QuantTensor{x1, codes1, scales1, nullptr, 0, 0, nullptr};
  a.n_tensors = 2;
  a.H = int32_t(H);
  a.T = int32_t(T);
  a.D = int32_t(D);
  a.tokens_per_frame = int32_t(T);
  a.n_frames = 1;
  a.rows = T;
  return launch_stream_reference(a, stream);
}

size_t nvfp4_quantize_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int nvfp4_quantize_kv_noalloc(const uint16_t *x, int64_t H, int64_t T, int64_t D, uint8_t *codes,
                              uint8_t *scales, float *tensor_scale, void *stream) {
  QuantArgs a;
  if (int rc = codec_args(x, H, T, D, codes, scales, tensor_scale, &a)) return rc;
  return launch_quantize_noalloc(a, stream);
}

int mxfp4_quantize_kv(const uint16_t *x, int64_t H, int64_t T, int64_t D, uint8_t *codes,
                      uint8_t *scales, void *stream) {
  if (!x || !codes || !scales) return NVFP4KV_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8)) return NVFP4KV_EINVAL;
  if (H < 1 || T < 1 || D < 32 || D % 32 != 0 || D > 4096) return NVFP4KV_EINVAL;
  if (H * T * D >= (int64_t(1) << 40) || T > (int64_t(1) << 30) || H > (1 << 20))
    return NVFP4KV_EINVAL;
  QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.t[0].src = x;
  a.t[0].codes = codes;
  a.t[0].scales = scales;
  a.t[0].tensor_scale = nullptr;
  a.t[0].transposed = 0;
  a.n_tensors = 1;
  a.H = int32_t(H);
  a.T = int32_t(T);
  a.D = int32_t(D);
  a.tokens_per_frame = int32_t(T);
  a.n_frames = 1;
  a.rows = T;
  a.frame_slot[0] = 0;
  return launch_quantize_mx(a, stream);
}

size_t kvcache_storage_bytes(const kvcache_config *cfg) {
  Layout L;
  if (!make_layout(cfg, &L)) return 0;
  return L.total;
}

int kvcache_create(const kvcache_config *cfg, void *storage, size_t storage_bytes,
                   kvcache **out) {
  if (!out) return NVFP4KV_EINVAL;
  *out = nullptr;
  Layout L;
  if (!storage || !make_layout(cfg, &L)) return NVFP4KV_EINVAL;
  if (reinterpret_cast<uintptr_t>(storage) % kAlign != 0) return NVFP4KV_EINVAL;
  if (storage_bytes < L.total) return NVFP4KV_ECAPACITY;
  kvcache *c = new (std::nothrow) kvcache;
  if (!c) return NVFP4KV_ECAPACITY;
  c->cfg = *cfg;
  c->L = L;
  c->base = static_cast<uint8_t *>(storage);
  // tensor-scale table, quantizer workspace and attention flags start zeroed (the
  // attention partial slots need no initialization)
  int rc = zero_device_bytes_blocking(c->base + L.table, L.attn_part - L.table);
  if (rc != NVFP4KV_OK) {
    delete c;
    return rc;
  }
  *out = c;
  return NVFP4KV_OK;
}

int kvcache_destroy(kvcache *c) {
  delete c;
  return NVFP4KV_OK;
}

int kvcache_append(kvcache *c, const uint16_t *k, const uint16_t *v, int32_t n_frames,
                   void *stream) {
  if (!c || !k || !v) return NVFP4KV_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16)) return NVFP4KV_EINVAL;
  if (n_frames < 1 || n_frames > kMaxFrames) return NVFP4KV_EINVAL;
  const kvcache_config &cfg = c->cfg;
  if (int64_t(n_frames) * cfg.tokens_per_frame > (int64_t(1) << 30)) return NVFP4KV_EINVAL;
  // chunk numbers are int32, and the quantizers' epoch tags hold the epoch's low 32
  // bits: both stay unique below 2^31 appends
  if (c->st.next_chunk == INT32_MAX) return NVFP4KV_ESTATE;
  State s = c->st;   // planned state, committed only if the launch succeeds
  const int32_t to_sink = n_frames < cfg.sink_frames - s.sink_used
                              ? n_frames
                              : cfg.sink_frames - s.sink_used;
  const int32_t to_win = n_frames - to_sink;
  if (to_win > cfg.window_frames) return NVFP4KV_ECAPACITY;
  const int32_t overflow = s.win_count + to_win - cfg.window_frames;
  if (overflow > 0) evict_oldest(c, s, overflow);

  int32_t sslot = -1;
  for (int32_t i = 0; i < kScaleSlots; ++i)
    if (s.scale_ref[i] == 0) {
      sslot = i;
      break;
    }
  if (sslot < 0) return NVFP4KV_ESTATE;   // unreachable: slots > frames

  const int32_t cid = s.next_chunk;
  ChunkRec rec;
  rec.scale_slot = sslot;
  rec.n_frames = n_frames;
  rec.resident = n_frames;
  QuantArgs a;
  memset(&a, 0, sizeof(a));
  const int32_t pool_lo = cfg.sink_frames, pool_hi = pool_lo + cfg.window_frames + cfg.shot_frames;
  for (int32_t f = 0; f < n_frames; ++f) {
    int32_t slot;
    if (f < to_sink) {
      slot = s.sink_used++;
    } else {
      slot = pool_lo;
      while (slot < pool_hi && s.slot_used[slot]) ++slot;
      if (slot == pool_hi) return NVFP4KV_ESTATE;   // unreachable: the pool is large enough
      s.slot_used[slot] = true;
      s.win[(s.win_head + s.win_count) % kMaxFrames] = slot;
      s.win_count += 1;
    }
    s.slot_frame[slot] = FrameRec{cid, f, s.next_frame + f};
    rec.slot[f] = slot;
    a.frame_slot[f] = slot;
  }
  s.scale_ref[sslot] = n_frames;
  s.chunks[cid] = rec;
  s.next_chunk = cid + 1;
  s.next_frame += n_frames;

  float *tab = c->table();
  const bool v_adaptive = (cfg.options & NVFP4KV_V_ADAPTIVE) != 0;
  a.t[0] = QuantTensor{k, c->kcodes(), c->kscales(), tab + 2 * sslot, 0, 0,
                       c->k_smooth() ? c->kmean(sslot) : nullptr};
  a.t[1] = QuantTensor{v, c->vcodes(), c->vscales(), tab + 2 * sslot + 1, 1, v_adaptive ? 1 : 0, nullptr};
  a.n_tensors = 2;
  a.H = cfg.n_heads;
  a.T = n_frames * cfg.tokens_per_frame;
  a.D = cfg.head_dim;
  a.tokens_per_frame = cfg.tokens_per_frame;
  a.n_frames = n_frames;
  a.rows = c->L.rows;
  a.ws = c->ws();
  a.epoch = ++c->epoch;   // never reused, even if the launch fails
  if (uint32_t(a.epoch) == 0) a.epoch = ++c->epoch;   // tagged words use the low half; 0 = never written
  a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  int rc;
  if (c->mx()) {
    rc = launch_quantize_mx(a, stream);
  } else if (cfg.options) {
    if (c->k_smooth()) {
      a.sum_slots = c->sum_slots();
      a.cmax_slots = c->cmax_slots();
    }
    rc = launch_quantize_options(a, c->k_smooth() ? c->kmean(sslot) : nullptr, c->kmean_ws(), stream);
  } else {
    rc = launch_quantize(a, stream);
  }
  if (rc != NVFP4KV_OK) return rc;
  c->st = s;
  return NVFP4KV_OK;
}

int kvcache_append_schedule(const kvcache *c, int32_t n_frames, int32_t *schedule) {
  if (!c || !schedule || n_frames < 1 || n_frames > kMaxFrames) return NVFP4KV_EINVAL;
  const kvcache_config &cfg = c->cfg;
  if (int64_t(n_frames) * cfg.tokens_per_frame > (int64_t(1) << 30)) return NVFP4KV_EINVAL;
  if (c->mx()) {
    *schedule = 3;
    return NVFP4KV_OK;
  }
  QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.n_tensors = 2;
  a.H = cfg.n_heads;
  a.T = n_frames * cfg.tokens_per_frame;
  a.D = cfg.head_dim;
  a.tokens_per_frame = cfg.tokens_per_frame;
  a.n_frames = n_frames;
  a.epoch = 1;
  if (cfg.options) {   // the slots are part of every K-smoothing cache
    const int rc = quantize_options_single_pass(a, c->k_smooth(), (cfg.options & NVFP4KV_V_ADAPTIVE) != 0);
    if (rc < 0) return rc;
    *schedule = rc ? 4 : 2;
    return NVFP4KV_OK;
  }
  const int rc = quantize_single_pass(a);
  if (rc < 0) return rc;
  *schedule = rc ? 1 : 2;
  return NVFP4KV_OK;
}

int kvcache_evict(kvcache *c, int32_t n_frames) {
  if (!c || n_frames < 0) return NVFP4KV_EINVAL;
  if (n_frames > c->st.win_count) return NVFP4KV_ESTATE;
  evict_oldest(c, c->st, n_frames);
  return NVFP4KV_OK;
}

int kvcache_tokens(const kvcache *c, int64_t *sink_tokens, int64_t *window_tokens) {
  if (!c || !sink_tokens || !window_tokens) return NVFP4KV_EINVAL;
  *sink_tokens = int64_t(c->st.sink_used) * c->cfg.tokens_per_frame;
  *window_tokens = int64_t(c->st.win_count) * c->cfg.tokens_per_frame;
  return NVFP4KV_OK;
}

int kvcache_begin_shot(kvcache *c) {
  if (!c) return NVFP4KV_EINVAL;
  State &s = c->st;
  // the old shot's sink frames that already left the window leave the cache
  int32_t pinned[kMaxFrames];
  const int n = pinned_frames(c, s, pinned);
  for (int i = 0; i < n; ++i) release_slot(s, pinned[i]);
  s.shot_start = s.next_frame;
  return NVFP4KV_OK;
}

int kvcache_shot_sink(const kvcache *c, int64_t *start_frame, int32_t *n_frames,
                      int64_t *extra_tokens) {
  if (!c || !start_frame || !n_frames || !extra_tokens) return NVFP4KV_EINVAL;
  const State &s = c->st;
  *start_frame = s.shot_start;
  const int64_t seen = s.next_frame - s.shot_start;
  *n_frames = int32_t(seen < c->cfg.shot_frames ? seen : c->cfg.shot_frames);
  int32_t pinned[kMaxFrames];
  *extra_tokens = int64_t(pinned_frames(c, s, pinned)) * c->cfg.tokens_per_frame;
  return NVFP4KV_OK;
}

int kvcache_chunk_count(const kvcache *c, int32_t *n_chunks) {
  if (!c || !n_chunks) return NVFP4KV_EINVAL;
  *n_chunks = c->st.next_chunk;
  return NVFP4KV_OK;
}

int kvcache_export_k_mean(const kvcache *c, int32_t chunk_index, float *k_mean, void *stream) {
  if (!c || !k_mean) return NVFP4KV_EINVAL;
  if (!c->k_smooth()) return NVFP4KV_EINVAL;
  auto it = c->st.chunks.find(chunk_index);
  if (it == c->st.chunks.end()) return NVFP4KV_ESTATE;
  return copy_device_floats(k_mean, c->kmean(it->second.scale_slot),
                            size_t(c->cfg.n_heads) * c->cfg.head_dim, stream);
}

int kvcache_chunk_frames(const kvcache *c, int32_t chunk_index, int32_t *n_frames) {
  if (!c || !n_frames) return NVFP4KV_EINVAL;
  auto it = c->st.chunks.find(chunk_index);
  if (it == c->st.chunks.end()) return NVFP4KV_ESTATE;
  *n_frames = it->second.n_frames;
  return NVFP4KV_OK;
}

int chunk_attention(const kvcache *c, const uint16_t *q, const uint16_t *k_own,
                    const uint16_t *v_own, int64_t n_q, float softmax_scale, float *out,
                    void *stream) {
  if (!c || !q || !k_own || !v_own || !out) return NVFP4KV_EINVAL;
  if (!aligned(q, 16) || !aligned(k_own, 16) || !aligned(v_own, 16) || !aligned(out, 16))
    return NVFP4KV_EINVAL;
  if (n_q < 1 || n_q > (int64_t(1) << 24)) return NVFP4KV_EINVAL;
  if (!(softmax_scale > 0.0f) || softmax_scale > 3.0e38f) return NVFP4KV_EINVAL;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_own = k_own;
  a.v_own = v_own;
  a.out = out;
  a.kcodes = c->kcodes();
  a.kscales = c->kscales();
  a.vcodes = c->vcodes();
  a.vscales = c->vscales();
  a.scale_table = c->table();
  a.rows = c->L.rows;
  a.H = c->cfg.n_heads;
  a.D = c->cfg.head_dim;
  a.n_q = int32_t(n_q);
  a.sm_scale_log2 = softmax_scale * 1.4426950408889634f;
  a.k_mean = c->k_smooth() ? c->kmean(0) : nullptr;
  a.mx = c->mx() ? ((c->cfg.options & NVFP4KV_MX_SCALED_QK) ? 2 : 1) : 0;
  a.partials = c->attn_partials();
  a.flags = c->attn_flags();
  a.epoch = ++c->attn_epoch;   // never reused, even if the launch fails
  a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  int32_t slots[kMaxFrames];
  const int nf = collect_frames(c, slots);
  const int32_t T_f = c->cfg.tokens_per_frame;
  int ns = 0;
  for (int i = 0; i < nf; ++i) {
    const FrameRec fr = c->st.slot_frame[slots[i]];
    const int32_t ss = c->st.chunks.at(fr.chunk).scale_slot;
    const int32_t tok0 = slots[i] * T_f;
    if (ns > 0 && a.seg[ns - 1].scale_slot == ss &&
        a.seg[ns - 1].tok0 + a.seg[ns - 1].ntok == tok0) {
      a.seg[ns - 1].ntok += T_f;
    } else {
      a.seg[ns] = Segment{tok0, T_f, ss, 0};
      ++ns;
    }
  }
  a.n_seg = ns;
  return launch_attention(a, stream);
}

int kvcache_export_chunk(const kvcache *c, int32_t chunk_index, uint8_t *k_codes,
                         uint8_t *k_scales, uint8_t *v_codes, uint8_t *v_scales,
                         float *k_scale, float *v_scale, void *stream) {
  if (!c || !k_codes || !k_scales || !v_codes || !v_scales || !k_scale || !v_scale)
    return NVFP4KV_EINVAL;
  auto it = c->st.chunks.find(chunk_index);
  if (it == c->st.chunks.end()) return NVFP4KV_ESTATE;
  const ChunkRec &rec = it->second;
  if (rec.resident != rec.n_frames) return NVFP4KV_ESTATE;
  ExportArgs a;
  memset(&a, 0, sizeof(a));
  a.kcodes = c->kcodes();
  a.kscales = c->kscales();
  a.vcodes = c->vcodes();
  a.vscales = c->vscales();
  a.scale_table = c->table();
  a.scale_slot = rec.scale_slot;
  a.H = c->cfg.n_heads;
  a.D = c->cfg.head_dim;
  a.T_f = c->cfg.tokens_per_frame;
  a.n_frames = rec.n_frames;
  a.block = c->mx() ? 32 : 16;
  a.rows = c->L.rows;
  a.k_codes_out = k_codes;
  a.k_scales_out = k_scales;
  a.v_codes_out = v_codes;
  a.v_scales_out = v_scales;
  a.k_scale_out = k_scale;
  a.v_scale_out = v_scale;
  for (int32_t f = 0; f < rec.n_frames; ++f) a.frame_slot[f] = rec.slot[f];
  return launch_export(a, stream);
}

int nvfp4kv_set_wait_limit(int32_t limit) {
  if (limit < 0) return NVFP4KV_EINVAL;
  g_spin_limit.store(limit, std::memory_order_relaxed);
  return NVFP4KV_OK;
}

}  // extern "C"
