// Device-side helpers and the launch interface shared by the kvq kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvq_validate.h"

namespace kvq {

// The cache as the kernels see it (plane pointers plus the few sizes they index with).
// u = page * Hkv + kv head; tokens live in 16-token tiles (see the byte helpers below).
struct DevCache {
  uint8_t* kc;   // K codes  [u][P/16][RB/16][16][16 B]  tile rows in 16-byte chunks, chunk-major
  uint32_t* km;  // K meta   [u][P][NG]                  {scale | zero << 16}
  uint8_t* vc;   // V codes  [u][P/16][RB/2][8][2][2]    16-bit words, token pairs byte-interleaved
  uint32_t* vm;  // V meta   [u][P/16][2][NG][2][4]      {scale | zero << 16}
  int hkv;
  int page;
  int row_bytes;
  int ngroups;
  int quant_mode;  // 0 = asymmetric min/max, 1 = hybrid symmetric/asymmetric per group
  int v_grouping;  // 0 = value groups of G channels per token, 1 = of G tokens per channel
};

inline DevCache dev_cache(const kvq_cache* c, const Geometry& g) {
  DevCache d;
  d.kc = static_cast<uint8_t*>(c->k_codes);
  d.km = static_cast<uint32_t*>(c->k_meta);
  d.vc = static_cast<uint8_t*>(c->v_codes);
  d.vm = static_cast<uint32_t*>(c->v_meta);
  d.hkv = g.hkv;
  d.page = g.page;
  d.row_bytes = g.row_bytes;
  d.ngroups = g.ngroups;
  d.quant_mode = g.quant_mode;
  d.v_grouping = g.v_grouping;
  return d;
}

// Byte of the K code plane holding byte `k` of the packed row of token o (0..15) of the
// tile whose first token is row `tile_row` (= u * P + 16 * tile).
__host__ __device__ __forceinline__ int64_t k_code_byte(int64_t tile_row, int row_bytes, int o, int k) {
  return tile_row * row_bytes + ((k >> 4) * 16 + o) * 16 + (k & 15);
}
// Byte of the V code plane holding byte `k` of the packed row of token o of that tile.
__host__ __device__ __forceinline__ int64_t v_code_byte(int64_t tile_row, int row_bytes, int o, int k) {
  return tile_row * row_bytes + (k >> 1) * 32 + (o >> 1) * 4 + (k & 1) * 2 + (o & 1);
}
// Entry of the V meta plane for group g of token o of tile `tile` (= u * P / 16 + tile
// index): token o = 8 half + 4 part + i at ((part * NG + g) * 2 + half) * 4 + i.
__host__ __device__ __forceinline__ int64_t v_meta_entry(int64_t tile, int ngroups, int g, int o) {
  return tile * ngroups * 16 + ((((o >> 2) & 1) * ngroups + g) * 2 + (o >> 3)) * 4 + (o & 3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16_bits_to_float(uint32_t h16) {
  _Float16 h;
  const uint16_t b = static_cast<uint16_t>(h16);
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

__device__ __forceinline__ uint32_t float_to_f16_bits(float x) {
  const _Float16 h = static_cast<_Float16>(x);  // v_cvt_f16_f32, round to nearest even
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// bf16 windows: row w of sequence b, kv head h at ((b * (sink + recent) + w) * Hkv + h) * 128.
struct DevWindow {
  uint16_t* k;
  uint16_t* v;
  int sink;
  int recent;
  int residual;  // 1: sink 0 and the ring holds the incomplete last group of `recent` tokens
};

// ---- host launchers (defined in the .hip files) ----
hipError_t launch_quantize_append(const DevCache& c, const Geometry& g, const void* k_new,
                                  const void* v_new, const int64_t* slots, int64_t n_new,
                                  hipStream_t stream);
hipError_t launch_window_append(const DevCache& c, const DevWindow& w, const Geometry& g, const void* k_new,
                                const void* v_new, const int32_t* seqs, const int32_t* positions,
                                const int64_t* evict_slots, int64_t n_new, hipStream_t stream);
hipError_t launch_dequantize(const DevCache& c, const Geometry& g, int which, const int64_t* slots,
                             int64_t n, float* out, hipStream_t stream);

struct DecodeArgs {
  DevCache c;
  const uint16_t* q;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* partials;
  float* out;
  int batch;
  int num_q_heads;
  int ratio;
  int max_pages;
  int split_len;
  int num_splits;
  // The split kernels cover tokens [tok_begin, max(tok_begin, T - tok_tail)) of each
  // sequence (0, 0 without windows); partition p starts at tok_begin + p * split_len.
  int tok_begin;
  int tok_tail;
  // with a residual of whole groups of tail_mod tokens (else 0): the span ends at
  // T - T % tail_mod instead
  int tail_mod;
  // partial slots per (sequence, query head): num_splits, plus one for the window
  // partial (slot num_splits) when `window` is set
  int part_stride;
  int window;
  // query-channel pruning (pruned kernel only): key chunks kept per (sequence, kv head),
  // and where the chosen masks go ([batch][Hkv], may be null)
  int keep_chunks;
  int32_t* chunk_mask;
  int hblock;
  float rot_c;    // float nearest 1/sqrt(hblock)
  float qscale;   // softmax scale * log2(e): logits are kept in the exp2 domain
};

hipError_t launch_decode_split(const DecodeArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_decode_split_pruned(const DecodeArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_decode_split_vgroup(const DecodeArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_decode_split_reference(const DecodeArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_decode_window(const DecodeArgs& a, const DevWindow& w, const Geometry& g, hipStream_t stream);

}  // namespace kvq
