// Decode attention with a workspace the library owns, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): kvq_decode_attention_noalloc.
//
// The decode kernels' workspace (split partials and the balanced plan's table) lives in
// a file-scope device array. Its device address is looked up once per device with
// hipGetSymbolAddress (each device holds its own copy of the array) and only that
// address is handed to the kernels and compared against sizes; the array's name is a
// host-side stand-in that no host code here dereferences or passes on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_device.h"

namespace kvq {
namespace {

constexpr size_t kScratchBytes = KVQ_NOALLOC_WORKSPACE_BYTES;  // per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's `scratch`, or nullptr if it cannot be found.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace kvq

extern "C" {

kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                                        const int32_t* block_table, int32_t max_pages_per_seq,
                                        const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                        int32_t num_splits, float* out, void* stream) {
  // the argument checks run before the address lookup (which allocates nothing); the
  // workspace size is checked against the array's inside decode_run
  kvq::Geometry g;
  const kvq_status st = kvq::check_decode_args(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                                          max_seq_len, num_splits, out, &g);
  if (st != KVQ_OK || batch == 0) return st;
  void* ws = kvq::scratch_on_current_device();
  if (!ws) return KVQ_ERR_HIP;
  return kvq::decode_run(cache, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens, max_seq_len,
                         softmax_scale, num_splits, ws, kvq::kScratchBytes, out, stream, nullptr, nullptr, false);
}

}  // extern "C"
