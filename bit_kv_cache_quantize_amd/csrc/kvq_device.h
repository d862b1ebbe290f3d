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
// read probe (stream_probe.hip): n16 16-byte pieces at src, `workgroups` of 256 threads;
// t0 / t1 (may be null) recorded as part of the dispatch, as for the split launches
hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* sink, int nontemporal, int64_t workgroups,
                              hipStream_t stream, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

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
  // Where partials go. Fixed partitions (split_len from the host): partition p of
  // sequence b, query head j at partials[((b * Hq + j) * num_splits + p) * (d + 2)].
  // Balanced partitions (balanced = 1): the length L comes from the batch's total
  // covered span on the device (the balanced plan below); units u = 0, 1, ... number the
  // partitions of sequence 0, then sequence 1, ...; workgroups run them in the order
  // (sequence, kv head, partition), and unit u of kv head hk writes
  // partials[(j * unit_slots + u) * (d + 2)] for its query heads j.
  int balanced;
  int units_per_head;  // balanced: target partitions per kv head
  int unit_slots;      // balanced: units per kv head in the grid, partial slots per query head
  // balanced: per sequence {first unit, partitions}, written by the split kernel's unit
  // (kv head 0, partition 0) of each sequence with tokens, read by the combine
  int2* seq_plan;
  // the host's max_seq_len: the split kernels and their plan take longer sequences as this
  // long, which keeps every partition within the block table's row and the host's sizing
  int max_len;
  // window partials [batch][Hq][d + 2], when `window` is set
  float* win_partials;
  int window;
  // query-channel pruning (pruned kernel only): key chunks kept per (sequence, kv head),
  // and where the chosen masks go ([batch][Hkv], may be null)
  int keep_chunks;
  int32_t* chunk_mask;
  int hblock;
  float rot_c;    // float nearest 1/sqrt(hblock)
  float qscale;   // softmax scale * log2(e): logits are kept in the exp2 domain
  // Fused step (kvq_decode_step; null otherwise): the new token of each sequence, K and V
  // rows [batch][Hkv][128] bf16, quantized into position seq_lens[b] - 1 by the split
  // kernel's unit whose partition holds that position, before that unit's first load.
  const uint16_t* k_new;
  const uint16_t* v_new;
};

// ---- partition plan ----

// Tokens of sequence b (seq_len T) the split kernels cover: [tok_begin, qend).
__device__ __forceinline__ int covered_end(const DecodeArgs& a, int T) {
  return a.tail_mod ? T - T % a.tail_mod : max(a.tok_begin, T - a.tok_tail);
}
__device__ __forceinline__ int covered_span(const DecodeArgs& a, int T) {
  return T > 0 ? max(0, covered_end(a, T) - a.tok_begin) : 0;
}

// Balanced plan, in units of 256 tokens (kBalancedMinLen): c_b = ceil(span_b / 256),
// C = sum_b c_b, U = units_per_head (one round of waves over the kv heads). The
// partition length is L = 256 k: k starts at ceil(C / U) and grows until the partitions,
// sum_b ceil(c_b / k), fit in U (at most kBalancedMaxK; past that, several rounds);
// sequence b gets ceil(c_b / k) partitions, the same as ceil(span_b / L). Every function
// below runs on a full wavefront (lane = 0..63, all active) and returns wave-uniform
// values (made visibly uniform, so what derives from them stays scalar); every workgroup
// and kernel gets the same plan from the same seq_lens. Lane l keeps seq_lens[l] (the
// first 64 sequences) from a single load.

// Inclusive prefix sum over the 64 lanes: DPP row shifts (zeros shifted in) within each
// row of 16 lanes, then the totals of the rows below.
template <int CTRL>
__device__ __forceinline__ int dpp_shifted(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  x += dpp_shifted<0x111>(x);  // row_shr:1
  x += dpp_shifted<0x112>(x);  // row_shr:2
  x += dpp_shifted<0x114>(x);  // row_shr:4
  x += dpp_shifted<0x118>(x);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
__device__ __forceinline__ int wave_sum(int x, int lane) {
  return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(wave_incl_scan(x, lane), 63));
}

__device__ __forceinline__ int span_units(const DecodeArgs& a, int T) {
  return (covered_span(a, min(T, a.max_len)) + kBalancedMinLen - 1) / kBalancedMinLen;
}

__device__ __forceinline__ int first_lens(const DecodeArgs& a, int lane) {
  return lane < a.batch ? a.seq_lens[lane] : 0;
}

// Partitions of all sequences for a given k.
__device__ __forceinline__ int balanced_count(const DecodeArgs& a, int lane, int c0, int k) {
  int n = (c0 + k - 1) / k;
  for (int b = 64 + lane; b < a.batch; b += 64) n += (span_units(a, a.seq_lens[b]) + k - 1) / k;
  return wave_sum(n, lane);
}

// k of the plan (L = 256 k). Lane sums of C saturate at 2^24 (>= kBalancedMaxK * U, so
// the result is unchanged) to keep the 64-lane total within 32 bits.
__device__ __forceinline__ int balanced_k(const DecodeArgs& a, int lane, int T0) {
  constexpr int kCap = 1 << 24;
  const int c0 = span_units(a, T0);
  int c = c0;
  for (int b = 64 + lane; b < a.batch; b += 64) c = min(kCap, c + span_units(a, a.seq_lens[b]));
  const int C = wave_sum(c, lane);
  const int U = a.units_per_head;
  if (C >= kBalancedMaxK * U) return kBalancedMaxK;
  int k = C > U ? (C + U - 1) / U : 1;
  while (k < kBalancedMaxK && balanced_count(a, lane, c0, k) > U) ++k;
  return k;
}

// Workgroup g of the split launch in the order (sequence, kv head, partition) — each
// sequence's n_b partitions for kv head 0, then for kv head 1, ... — as the fixed
// partitions are ordered: its sequence b (-1 past the last partition), kv head hk,
// partition index p within the sequence, the plan's length L, seq_lens[b], and its unit
// u = (first unit of b) + p, the partial slot shared by all kv heads' layouts.
struct PlanUnit {
  int b, hk, p, u, L, T, n;
};
__device__ __forceinline__ PlanUnit balanced_unit(const DecodeArgs& a, int g, int hkv, int lane) {
  const int T0 = first_lens(a, lane);
  const int k = balanced_k(a, lane, T0);
  int base = 0;  // partitions of the sequences before this group of 64
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int Tl = b0 == 0 ? T0 : (b0 + lane < a.batch ? a.seq_lens[b0 + lane] : 0);
    const int n = (span_units(a, Tl) + k - 1) / k;
    const int incl = wave_incl_scan(n, lane);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (g < (base + total) * hkv) {
      const unsigned long long hit = __ballot((base + incl) * hkv > g);  // lane 63 is set
      const int l = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(hit)));
      const int first = base + __builtin_amdgcn_readlane(incl - n, l);
      const int nb = __builtin_amdgcn_readlane(n, l);  // >= 1: workgroup g falls in it
      const int r = g - first * hkv;
      const int hk = r / nb, p = r - hk * nb;
      return {b0 + l, hk, p, first + p, kBalancedMinLen * k, __builtin_amdgcn_readlane(Tl, l), nb};
    }
    base += total;
  }
  return {-1, 0, 0, 0, kBalancedMinLen * k, 0, 0};
}

// Workgroups of a split-K launch.
inline int64_t split_units(const DecodeArgs& a, const Geometry& g) {
  return a.balanced ? static_cast<int64_t>(g.hkv) * a.unit_slots
                    : static_cast<int64_t>(a.batch) * g.hkv * a.num_splits;
}

// The split launches record t0 / t1 (may be null) as part of the kernel's dispatch
// (hipExtLaunchKernel): their elapsed time is the kernel's own, without the dispatch
// around it that separately recorded events would also time.
hipError_t launch_decode_split(const DecodeArgs& a, const Geometry& g, hipStream_t stream, hipEvent_t t0 = nullptr,
                               hipEvent_t t1 = nullptr);
hipError_t launch_decode_split_paged(const DecodeArgs& a, const Geometry& g, hipStream_t stream,
                                     hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_decode_split_pruned(const DecodeArgs& a, const Geometry& g, hipStream_t stream,
                                      hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_decode_split_vgroup(const DecodeArgs& a, const Geometry& g, hipStream_t stream,
                                      hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_decode_split_reference(const DecodeArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs& a, const Geometry& g, hipStream_t stream);
hipError_t launch_decode_window(const DecodeArgs& a, const DevWindow& w, const Geometry& g, hipStream_t stream);

// kvq_decode_attention and its timed and reference variants, and the fused step
// (kvq_api.cpp): every host check, the split kernel (matrix or reference; with k_new and
// v_new, the matrix kernel appends each sequence's new token first) and the combine, with
// the given workspace.
kvq_status decode_run(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                      const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                      int32_t max_seq_len, float softmax_scale, int32_t num_splits, void* workspace,
                      size_t workspace_bytes_given, float* out, void* stream, void* ev_begin, void* ev_end,
                      bool reference, const void* k_new = nullptr, const void* v_new = nullptr);

}  // namespace kvq
