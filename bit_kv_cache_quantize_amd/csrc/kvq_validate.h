// Host-side argument checking for the kvq C ABI. No HIP dependency: this
// translation unit also builds with a plain host compiler for CPU-only tests.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/kvq.h"

namespace kvq {

// Kernel granularity: the decode kernels walk the cache in 32-token blocks made of
// two 16-token tiles; split-K partitions are whole blocks.
constexpr int kTile = 16;
constexpr int kBlock = 32;
// Size limits of well-formed descriptions: larger values return KVQ_ERR_UNSUPPORTED, so
// token positions and partition lengths stay far inside 32 bits and per-row sizes too.
constexpr int32_t kMaxSeqLen = 1 << 30;
constexpr int32_t kMaxHeadDim = 1 << 16;

struct Geometry {
  int d, hkv, bits, group, ngroups, hblock, page, row_bytes, quant_mode, v_grouping;
  int64_t num_pages;
};

// Structural checks of a cache description. `planes` also checks the four device
// pointers (non-null, 16-byte aligned).
kvq_status check_cache(const kvq_cache* c, bool planes, Geometry* g);

// Description is well formed but outside what the kernels are built for.
bool cache_supported(const Geometry& g);

bool aligned(const void* p, size_t a);

// Bytes of one cache plane (-1 for a plane index outside 0..3 or a size beyond int64).
int64_t plane_bytes(const Geometry& g, int plane);
// kvq_cache_plane_bytes: -1 for an invalid description, a width without a packing
// (bits other than 2, 4) or a head beyond kMaxHeadDim; sizes also for other unsupported ones.
int64_t cache_plane_bytes(const kvq_cache* c, int32_t plane);

// Split-K sizing. `cus` is the device's compute-unit count (256 on MI355X).
// Fixed partitions: every sequence is cut into split_len-token partitions (a caller's
// num_splits, the reference kernel, a batch of one). Balanced partitions (the matrix
// kernels' automatic choice): one length for the whole batch, chosen on the device from the
// total covered span so that every kv head gets about units_per_head partitions of equal
// length whatever the mix of sequence lengths; num_splits and split_len then describe a
// batch whose sequences all have max_seq_len tokens.
struct Splits {
  int32_t num_splits;  // partitions of a max_seq_len sequence
  int32_t split_len;   // tokens per partition, a multiple of kBlock
  int32_t balanced;
  int32_t units_per_head;  // balanced: target partitions per kv head
  int32_t unit_slots;      // balanced: bound on the partitions of one kv head (grid units)
};
constexpr int kBalancedMinLen = 256;     // 8 blocks
constexpr int kBalancedMaxK = 64;        // longest balanced partition: 64 * 256 tokens
constexpr int kWavesPerCU = 8;           // the matrix kernels' occupancy: 2 waves per SIMD
// Every split and combine workgroup recomputes the plan from all of seq_lens (64 per
// step); past this many sequences the batch alone gives enough partitions to balance,
// and fixed partitions are used.
constexpr int kBalancedMaxBatch = 256;
// Automatic choices differ per decode kernel: the matrix-core kernel takes balanced
// partitions (batch > 1) or fixed ones of up to 128 blocks (one sequence); the plain
// reference kernel keeps a partition's scores in LDS and takes at most 64 blocks.
enum class SplitKernel { kMatrix, kReference };
Splits choose_splits(const Geometry& g, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                     int32_t requested, int cus, SplitKernel kernel);

// Workspace sizes saturate at SIZE_MAX (no configuration that large can be allocated).
size_t workspace_bytes(const Geometry& g, int32_t batch, int32_t num_q_heads, const Splits& s);
// Balanced layout: the partials [Hq][unit_slots][d + 2] fp32, then a table of int32 pairs
// {first unit, partitions} per sequence (written by the split kernel, read by the combine).
size_t balanced_partials_bytes(const Geometry& g, int32_t num_q_heads, const Splits& s);

// Sizes of a decode call: INVALID for negative counts or no query heads, UNSUPPORTED for
// max_seq_len beyond kMaxSeqLen.
kvq_status check_decode_sizes(int32_t batch, int32_t num_q_heads, int32_t max_seq_len, int32_t num_splits);

// Decode arguments other than the workspace (for calls whose workspace is the library's).
kvq_status check_decode_args(const kvq_cache* c, const void* q, int32_t batch, int32_t num_q_heads,
                             const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                             int32_t max_seq_len, int32_t num_splits, const float* out, Geometry* g);

// Full check of decode arguments (everything but the workspace size).
kvq_status check_decode(const kvq_cache* c, const void* q, int32_t batch, int32_t num_q_heads,
                        const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                        int32_t max_seq_len, int32_t num_splits, const void* workspace, const float* out,
                        Geometry* g);

kvq_status check_append(const kvq_cache* c, const void* k_new, const void* v_new, const int64_t* slots,
                        int64_t n_new, Geometry* g);

// The new-token rows of a fused step (kvq_decode_step) for a cache that passed
// check_decode: INVALID for a null or misaligned row pointer, UNSUPPORTED for value
// token groups or the reference kernel.
kvq_status check_step_rows(const Geometry& g, const void* k_new, const void* v_new, bool reference);

// Window description against the cache (sizes only; `planes` also checks k and v).
// Plane sizes are -1 when they exceed int64.
constexpr int kMaxWindow = 1024;  // sink + recent
kvq_status check_window(const kvq_cache* c, const kvq_window* w, bool planes);
int64_t window_plane_bytes(const Geometry& g, const kvq_window* w);

kvq_status check_window_append(const kvq_cache* c, const kvq_window* w, const void* k_new, const void* v_new,
                               const int32_t* seqs, const int32_t* positions, const int64_t* evict_slots,
                               int64_t n_new, Geometry* g);

// Splits of the quantized span of a max_seq_len sequence (max_seq_len - sink - recent).
int32_t window_span(const kvq_window* w, int32_t max_seq_len);
size_t window_workspace_bytes(const Geometry& g, int32_t batch, int32_t num_q_heads, const Splits& s);

kvq_status check_dequantize(const kvq_cache* c, int32_t which, const int64_t* slots, int64_t n,
                            const float* out, Geometry* g);

}  // namespace kvq
