// Test-only stand-in for the kernel launchers of libnvfp4kv: records the
// arguments the host library would launch with, so the cache metadata (slot
// assignment, eviction, segment lists) can be checked on a machine without a GPU.
// Built with g++ together with the library's api.cpp; never part of the product.
#include <string.h>

#include "../../nvfp4_kv_cache_amd/csrc/nvfp4kv_internal.h"

namespace nvfp4kv {
namespace {
QuantArgs g_q;
AttnArgs g_a;
ExportArgs g_e;
int g_calls[3];
int g_fail_next = 0;
int take_fail() {
  const int rc = g_fail_next;
  g_fail_next = 0;
  return rc;
}
}  // namespace

int launch_quantize(const QuantArgs &a, void *) {
  if (int rc = take_fail()) return rc;
  g_q = a;
  ++g_calls[0];
  return 0;
}
int launch_quantize_noalloc(const QuantArgs &a, void *) {
  if (int rc = take_fail()) return rc;
  g_q = a;
  ++g_calls[0];
  return 0;
}
int quantize_single_pass(const QuantArgs &a) { return a.epoch > 0 ? 1 : 0; }
int g_opt_calls = 0;
// as the library: the options' single pass when given an epoch, which appends always
// give; the K means are then written by the quantizer itself
int launch_quantize_options(const QuantArgs &a, float *k_mean, float *, void *) {
  if (int rc = take_fail()) return rc;
  g_q = a;
  g_q.t[0].mean = k_mean;
  ++g_opt_calls;
  return 0;
}
int quantize_options_single_pass(const QuantArgs &a, bool, bool) { return a.epoch > 0 ? 1 : 0; }
int launch_stream_reference(const QuantArgs &, void *) { return take_fail(); }
int g_mx_calls = 0;
int launch_quantize_mx(const QuantArgs &a, void *) {
  if (int rc = take_fail()) return rc;
  g_q = a;
  ++g_mx_calls;
  return 0;
}
int launch_attention(const AttnArgs &a, void *) {
  if (int rc = take_fail()) return rc;
  g_a = a;
  ++g_calls[1];
  return 0;
}
int launch_export(const ExportArgs &a, void *) {
  if (int rc = take_fail()) return rc;
  g_e = a;
  ++g_calls[2];
  return 0;
}
int g_mean_calls = 0;
int launch_channel_mean(const uint16_t *, int, int, int, float *, float *, void *) {
  if (int rc = take_fail()) return rc;
  ++g_mean_calls;
  return 0;
}
int copy_device_floats(float *, const float *, size_t, void *) { return take_fail(); }
int zero_device_bytes_blocking(void *, size_t) { return 0; }
}  // namespace nvfp4kv

using namespace nvfp4kv;

extern "C" {
int stub_calls(int kind) {
  return kind == 5 ? g_opt_calls : kind == 4 ? g_mx_calls : kind == 3 ? g_mean_calls : g_calls[kind];
}
// slots of the last quantize launch (K-smoothing single pass), as offsets from the
// storage base, or -1 when null
int64_t stub_last_quant_slots_ptr(int which) {
  const void *p = which ? static_cast<const void *>(g_q.sum_slots) : static_cast<const void *>(g_q.cmax_slots);
  return p ? reinterpret_cast<int64_t>(p) : -1;
}
// format seen by the last attention and export launches: 1 / 32 for MXFP4
int stub_last_attn_mx(void) { return g_a.mx; }
int stub_last_export_block(void) { return g_e.block; }
// options of the last quantize launch: bit 0 K mean given, bit 1 V adaptive
int stub_last_quant_options(void) {
  return (g_q.t[0].mean ? 1 : 0) | (g_q.n_tensors > 1 && g_q.t[1].adaptive ? 2 : 0);
}
int64_t stub_last_attn_k_mean(void) { return reinterpret_cast<int64_t>(g_a.k_mean); }
// epoch of the last quantize launch: > 0 lets the launcher take the single-pass kernel
int64_t stub_last_quant_epoch(void) { return int64_t(g_q.epoch); }
void stub_fail_next(int rc) { g_fail_next = rc; }
// segments of the last attention launch: out[3i..3i+2] = tok0, ntok, scale_slot
int stub_last_segments(int32_t *out, int max) {
  for (int i = 0; i < g_a.n_seg && i < max; ++i) {
    out[3 * i] = g_a.seg[i].tok0;
    out[3 * i + 1] = g_a.seg[i].ntok;
    out[3 * i + 2] = g_a.seg[i].scale_slot;
  }
  return g_a.n_seg;
}
// destination slots of the last quantize launch; returns the frame count
int stub_last_quant_slots(int32_t *out, int max, int32_t *n_tensors, int64_t *rows) {
  for (int i = 0; i < g_q.n_frames && i < max; ++i) out[i] = g_q.frame_slot[i];
  *n_tensors = g_q.n_tensors;
  *rows = g_q.rows;
  return g_q.n_frames;
}
// table offsets (bytes from the storage base) the last quantize launch writes its two
// tensor scales to, and the scale slot the last export reads
int64_t stub_last_scale_ptr(int i) { return reinterpret_cast<int64_t>(g_q.t[i].tensor_scale); }
int stub_last_export_slot(int32_t *slots, int max) {
  for (int i = 0; i < g_e.n_frames && i < max; ++i) slots[i] = g_e.frame_slot[i];
  return g_e.scale_slot;
}
}
