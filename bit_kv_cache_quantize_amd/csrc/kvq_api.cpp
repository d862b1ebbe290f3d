// The kvq C ABI: host-side validation, split sizing and kernel dispatch.
// Declarations, argument meaning, layout and error behaviour: include/kvq.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>

#include "kvq_device.h"

namespace kvq {
namespace {

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

Splits splits_for(const Geometry& g, int32_t batch, int32_t num_q_heads, int32_t max_seq_len, int32_t requested,
                  SplitKernel kernel = SplitKernel::kMatrix) {
  return choose_splits(g, batch, num_q_heads, max_seq_len, requested, device_cus(), kernel);
}

// Workspace for either decode kernel with these arguments.
size_t workspace_for(const Geometry& g, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                     int32_t requested) {
  const size_t a = workspace_bytes(g, batch, num_q_heads, splits_for(g, batch, num_q_heads, max_seq_len, requested));
  const size_t b = workspace_bytes(
      g, batch, num_q_heads, splits_for(g, batch, num_q_heads, max_seq_len, requested, SplitKernel::kReference));
  return a > b ? a : b;
}

DecodeArgs decode_args(const kvq_cache* cache, const Geometry& g, const void* q, int32_t batch, int32_t num_q_heads,
                       const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                       int32_t max_seq_len, float softmax_scale, const Splits& sp, void* workspace, float* out) {
  DecodeArgs a;
  a.c = dev_cache(cache, g);
  a.q = static_cast<const uint16_t*>(q);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.partials = static_cast<float*>(workspace);
  a.out = out;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.ratio = num_q_heads / g.hkv;
  a.max_pages = max_pages_per_seq;
  a.split_len = sp.split_len;
  a.num_splits = sp.num_splits;
  a.tok_begin = 0;
  a.tok_tail = 0;
  a.tail_mod = 0;
  a.balanced = sp.balanced;
  a.units_per_head = sp.units_per_head;
  a.unit_slots = sp.unit_slots;
  a.seq_plan = sp.balanced ? reinterpret_cast<int2*>(static_cast<char*>(workspace) +
                                                     balanced_partials_bytes(g, num_q_heads, sp))
                           : nullptr;
  a.max_len = max_seq_len;
  a.win_partials = nullptr;
  a.window = 0;
  a.keep_chunks = 0;
  a.chunk_mask = nullptr;
  a.hblock = g.hblock;
  a.rot_c = g.hblock > 0 ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(g.hblock))) : 1.0f;
  const double scale = softmax_scale > 0.f ? softmax_scale : 1.0 / std::sqrt(static_cast<double>(g.d));
  a.qscale = static_cast<float>(scale * 1.4426950408889634);  // log2(e)
  a.k_new = nullptr;
  a.v_new = nullptr;
  return a;
}

// the matrix-core split kernel for this cache's value grouping
hipError_t split_kernel(const DecodeArgs& a, const Geometry& g, hipStream_t s, void* t0 = nullptr,
                        void* t1 = nullptr) {
  const auto e0 = static_cast<hipEvent_t>(t0), e1 = static_cast<hipEvent_t>(t1);
  return g.v_grouping ? launch_decode_split_vgroup(a, g, s, e0, e1) : launch_decode_split(a, g, s, e0, e1);
}

DevWindow dev_window(const kvq_window* w) {
  DevWindow d;
  d.k = static_cast<uint16_t*>(w->k);
  d.v = static_cast<uint16_t*>(w->v);
  d.sink = w->sink;
  d.recent = w->recent;
  d.residual = w->residual;
  return d;
}

}  // namespace

kvq_status decode_run(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                       const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                       int32_t max_seq_len, float softmax_scale, int32_t num_splits, void* workspace,
                       size_t workspace_bytes_given, float* out, void* stream, void* ev_begin, void* ev_end,
                       bool reference, const void* k_new, const void* v_new) {
  Geometry g;
  kvq_status st = check_decode(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                               max_seq_len, num_splits, workspace, out, &g);
  if (st == KVQ_OK && (k_new || v_new)) st = check_step_rows(g, k_new, v_new, reference);
  if (st != KVQ_OK || batch == 0) return st;
  const Splits sp = splits_for(g, batch, num_q_heads, max_seq_len, num_splits,
                               reference ? SplitKernel::kReference : SplitKernel::kMatrix);
  const size_t need = workspace_bytes(g, batch, num_q_heads, sp);
  if (need == SIZE_MAX) return KVQ_ERR_INVALID;  // no such workspace can exist
  if (workspace_bytes_given < need) return KVQ_ERR_WORKSPACE;
  if (reference && sp.split_len > 2048) return KVQ_ERR_UNSUPPORTED;
  DecodeArgs a = decode_args(cache, g, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                             max_seq_len, softmax_scale, sp, workspace, out);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (reference) {
    if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), s) != hipSuccess) return KVQ_ERR_HIP;
    e = launch_decode_split_reference(a, g, s);
    if (e == hipSuccess && ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), s) != hipSuccess)
      return KVQ_ERR_HIP;
  } else {
    e = split_kernel(a, g, s, ev_begin, ev_end);
  }
  if (e != hipSuccess) return KVQ_ERR_HIP;
  e = launch_combine(a, g, s);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

int64_t kvq_cache_plane_bytes(const kvq_cache* cache, int32_t plane) { return cache_plane_bytes(cache, plane); }

kvq_status kvq_quantize_append(const kvq_cache* cache, const void* k_new, const void* v_new, const int64_t* slots,
                               int64_t n_new, void* stream) {
  Geometry g;
  kvq_status st = check_append(cache, k_new, v_new, slots, n_new, &g);
  if (st != KVQ_OK || n_new == 0) return st;
  const hipError_t e =
      launch_quantize_append(dev_cache(cache, g), g, k_new, v_new, slots, n_new, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                                  int32_t num_splits) {
  Geometry g;
  if (check_cache(cache, false, &g) != KVQ_OK) return 0;
  if (check_decode_sizes(batch, num_q_heads, max_seq_len, num_splits) != KVQ_OK) return 0;
  const size_t n = workspace_for(g, batch, num_q_heads, max_seq_len, num_splits);
  return n == SIZE_MAX ? 0 : n;
}

int32_t kvq_decode_num_splits(const kvq_cache* cache, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                              int32_t num_splits) {
  Geometry g;
  if (check_cache(cache, false, &g) != KVQ_OK) return 0;
  if (check_decode_sizes(batch, num_q_heads, max_seq_len, num_splits) != KVQ_OK) return 0;
  return splits_for(g, batch, num_q_heads, max_seq_len, num_splits).num_splits;
}

kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                                const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                int32_t max_seq_len, float softmax_scale, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, float* out, void* stream) {
  return decode_run(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens, max_seq_len,
                     softmax_scale, num_splits, workspace, workspace_bytes, out, stream, nullptr, nullptr, false);
}

kvq_status kvq_decode_attention_timed(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                                      const int32_t* block_table, int32_t max_pages_per_seq,
                                      const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                      int32_t num_splits, void* workspace, size_t workspace_bytes, float* out,
                                      void* stream, void* split_begin, void* split_end) {
  return decode_run(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens, max_seq_len,
                     softmax_scale, num_splits, workspace, workspace_bytes, out, stream, split_begin, split_end,
                     false);
}

kvq_status kvq_decode_step(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                           int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                           float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                           float* out, void* stream) {
  if (!k_new || !v_new) return KVQ_ERR_INVALID;
  return decode_run(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens, max_seq_len,
                     softmax_scale, num_splits, workspace, workspace_bytes, out, stream, nullptr, nullptr, false,
                     k_new, v_new);
}

kvq_status kvq_decode_step_timed(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                 float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                                 float* out, void* stream, void* split_begin, void* split_end) {
  if (!k_new || !v_new) return KVQ_ERR_INVALID;
  return decode_run(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens, max_seq_len,
                     softmax_scale, num_splits, workspace, workspace_bytes, out, stream, split_begin, split_end,
                     false, k_new, v_new);
}

kvq_status kvq_decode_attention_reference(const kvq_cache* cache, const void* q, int32_t batch,
                                          int32_t num_q_heads, const int32_t* block_table,
                                          int32_t max_pages_per_seq, const int32_t* seq_lens,
                                          int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                          void* workspace, size_t workspace_bytes, float* out, void* stream) {
  return decode_run(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens, max_seq_len,
                     softmax_scale, num_splits, workspace, workspace_bytes, out, stream, nullptr, nullptr, true);
}

int64_t kvq_window_plane_bytes(const kvq_cache* cache, const kvq_window* window) {
  Geometry g;
  if (check_cache(cache, false, &g) != KVQ_OK || check_window(cache, window, false) != KVQ_OK) return -1;
  return window_plane_bytes(g, window);
}

kvq_status kvq_window_append(const kvq_cache* cache, const kvq_window* window, const void* k_new, const void* v_new,
                             const int32_t* seqs, const int32_t* positions, const int64_t* evict_slots,
                             int64_t n_new, void* stream) {
  Geometry g;
  kvq_status st = check_window_append(cache, window, k_new, v_new, seqs, positions, evict_slots, n_new, &g);
  if (st != KVQ_OK || n_new == 0) return st;
  const hipError_t e = launch_window_append(dev_cache(cache, g), dev_window(window), g, k_new, v_new, seqs,
                                            positions, evict_slots, n_new, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

size_t kvq_decode_window_workspace_bytes(const kvq_cache* cache, const kvq_window* window, int32_t batch,
                                         int32_t num_q_heads, int32_t max_seq_len, int32_t num_splits) {
  Geometry g;
  if (check_cache(cache, false, &g) != KVQ_OK || check_window(cache, window, false) != KVQ_OK) return 0;
  if (check_decode_sizes(batch, num_q_heads, max_seq_len, num_splits) != KVQ_OK) return 0;
  const Splits sp = splits_for(g, batch, num_q_heads, window_span(window, max_seq_len), num_splits);
  const size_t n = window_workspace_bytes(g, batch, num_q_heads, sp);
  return n == SIZE_MAX ? 0 : n;
}

kvq_status kvq_decode_attention_window_timed(const kvq_cache* cache, const kvq_window* window, const void* q,
                                             int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                                             int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                             void* workspace, size_t workspace_bytes_given, float* out,
                                             void* stream, void* split_begin, void* split_end) {
  Geometry g;
  kvq_status st = check_decode(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                               max_seq_len, num_splits, workspace, out, &g);
  if (st != KVQ_OK) return st;
  st = check_window(cache, window, true);
  if (st != KVQ_OK) return st;
  if (batch > window->batch) return KVQ_ERR_INVALID;
  if (batch == 0) return KVQ_OK;
  const Splits sp = splits_for(g, batch, num_q_heads, window_span(window, max_seq_len), num_splits);
  const size_t need = window_workspace_bytes(g, batch, num_q_heads, sp);
  if (need == SIZE_MAX) return KVQ_ERR_INVALID;
  if (workspace_bytes_given < need) return KVQ_ERR_WORKSPACE;
  DecodeArgs a = decode_args(cache, g, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                             max_seq_len, softmax_scale, sp, workspace, out);
  a.tok_begin = window->sink;
  a.tok_tail = window->residual ? 0 : window->recent;
  a.tail_mod = window->residual ? window->recent : 0;
  a.win_partials = a.partials + workspace_bytes(g, batch, num_q_heads, sp) / sizeof(float);
  a.window = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (split_kernel(a, g, s, split_begin, split_end) != hipSuccess) return KVQ_ERR_HIP;
  if (launch_decode_window(a, dev_window(window), g, s) != hipSuccess) return KVQ_ERR_HIP;
  return launch_combine(a, g, s) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_decode_attention_window(const kvq_cache* cache, const kvq_window* window, const void* q,
                                       int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                       int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                       float softmax_scale, int32_t num_splits, void* workspace,
                                       size_t workspace_bytes_given, float* out, void* stream) {
  return kvq_decode_attention_window_timed(cache, window, q, batch, num_q_heads, block_table, max_pages_per_seq,
                                           seq_lens, max_seq_len, softmax_scale, num_splits, workspace,
                                           workspace_bytes_given, out, stream, nullptr, nullptr);
}

kvq_status kvq_decode_attention_pruned(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                                       const int32_t* block_table, int32_t max_pages_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                       int32_t num_splits, int32_t keep_chunks, int32_t* chunk_mask,
                                       void* workspace, size_t workspace_bytes_given, float* out, void* stream,
                                       void* split_begin, void* split_end) {
  Geometry g;
  kvq_status st = check_decode(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                               max_seq_len, num_splits, workspace, out, &g);
  if (st != KVQ_OK) return st;
  if (keep_chunks < 1 || keep_chunks > g.row_bytes / 16) return KVQ_ERR_INVALID;
  if (g.v_grouping) return KVQ_ERR_UNSUPPORTED;  // the pruned kernel reads value groups per token
  if (chunk_mask && !aligned(chunk_mask, 4)) return KVQ_ERR_INVALID;
  if (batch == 0) return KVQ_OK;
  const Splits sp = splits_for(g, batch, num_q_heads, max_seq_len, num_splits);
  const size_t need = workspace_bytes(g, batch, num_q_heads, sp);
  if (need == SIZE_MAX) return KVQ_ERR_INVALID;
  if (workspace_bytes_given < need) return KVQ_ERR_WORKSPACE;
  DecodeArgs a = decode_args(cache, g, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                             max_seq_len, softmax_scale, sp, workspace, out);
  a.keep_chunks = keep_chunks;
  a.chunk_mask = chunk_mask;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_decode_split_pruned(a, g, s, static_cast<hipEvent_t>(split_begin), static_cast<hipEvent_t>(split_end)) !=
      hipSuccess)
    return KVQ_ERR_HIP;
  return launch_combine(a, g, s) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_dequantize(const kvq_cache* cache, int32_t which, const int64_t* slots, int64_t n, float* out,
                          void* stream) {
  Geometry g;
  kvq_status st = check_dequantize(cache, which, slots, n, out, &g);
  if (st != KVQ_OK || n == 0) return st;
  const hipError_t e = launch_dequantize(dev_cache(cache, g), g, which, slots, n, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t nontemporal,
                           int32_t workgroups_per_cu, void* stream, void* ev_begin, void* ev_end) {
  if (!src || !aligned(src, 16) || bytes % 16 != 0 || !sink || !aligned(sink, 4)) return KVQ_ERR_INVALID;
  if ((nontemporal != 0 && nontemporal != 1) || workgroups_per_cu < 1 || workgroups_per_cu > 32)
    return KVQ_ERR_INVALID;
  if (bytes == 0) return KVQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t wgs = static_cast<int64_t>(device_cus()) * workgroups_per_cu;
  if (launch_stream_read(src, static_cast<int64_t>(bytes / 16), sink, nontemporal, wgs, s,
                         static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end)) != hipSuccess)
    return KVQ_ERR_HIP;
  return KVQ_OK;
}

const char* kvq_status_string(kvq_status status) {
  switch (status) {
    case KVQ_OK:
      return "ok";
    case KVQ_ERR_INVALID:
      return "invalid argument";
    case KVQ_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case KVQ_ERR_WORKSPACE:
      return "workspace too small";
    case KVQ_ERR_HIP:
      return "HIP runtime error";
  }
  return "unknown status";
}

const char* kvq_version(void) { return "kvq 0.1.0 (gfx950)"; }

}  // extern "C"
