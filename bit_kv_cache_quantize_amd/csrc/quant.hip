// Fused rotation + low-bit group quantization on cache append, and dequantization.
//
// SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving,
// Abstract: token-wise INT4 with a block-diagonal Hadamard rotation, done by one fused
// rotation-quantization kernel that writes straight into the paged KV layout.
// InnerQ (Abstract): asymmetric groups with a scale and a zero point.
//
// Mapping: one 128-channel token row per 16 lanes, 8 consecutive channels per lane,
// loaded with one 16-byte load. The Walsh-Hadamard butterfly (Sylvester order) runs
// in registers: strides 1, 2, 4 inside a lane, 8..64 across lanes of the row. Group
// min/max are reduced across the 4/8/16 lanes of a 32/64/128-channel group. Every fp32
// step is a separate IEEE round-to-nearest-even operation in the order the library
// documents, so the codes and fp16 scale/zero are bit-exact functions of the input.
#include <cmath>
#include <type_traits>

#include "kvq_device.h"
#include "quant_row.h"

// Every fp32 operation of the quantizer is its own rounding: never fuse.
#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kRowsPerBlock = 16;  // 256 threads, 16 lanes per row
constexpr int64_t kTileAppendMin = 256;  // appends of at least this many tokens go tile by tile

// rows_per_token 2: the K and V rows of every token; 1: K rows only (values in token
// groups are quantized per group, vgroup_append_kernel).
template <int BITS, int G>
__global__ __launch_bounds__(256) void quantize_append_kernel(DevCache c, const uint16_t* __restrict__ k_new,
                                                              const uint16_t* __restrict__ v_new,
                                                              const int64_t* __restrict__ slots, int64_t n_rows,
                                                              int rows_per_token, int hblock, float rot_c) {
  const int lane = threadIdx.x & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 4);
  if (row >= n_rows) return;  // whole 16-lane rows retire together
  const int which = rows_per_token == 2 ? static_cast<int>(row & 1) : 0;  // 0 = K, 1 = V
  const int64_t rh = rows_per_token == 2 ? row >> 1 : row;                 // token * Hkv + head
  const int h = static_cast<int>(rh % c.hkv);
  const int64_t r = rh / c.hkv;
  const uint4 raw = *reinterpret_cast<const uint4*>((which ? v_new : k_new) + rh * 128 + lane * 8);
  float x[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  quantize_store_row<BITS, G>(c, which, h, slots[r], x, lane, hblock, rot_c);
}

// Bulk appends: a workgroup takes rows 16j .. 16j+15 of one kv head and one kind (K or V;
// kinds 1 = keys only). When those rows are one whole 16-token tile (consecutive slots
// from a tile boundary), the tile is assembled in LDS in its cache layout and written
// with whole-line 16-byte stores; otherwise every row is stored on its own, as the
// per-row kernel does. The codes are the same either way.
template <int BITS, int G>
__global__ __launch_bounds__(256) void quantize_tiles_kernel(DevCache c, const uint16_t* __restrict__ k_new,
                                                             const uint16_t* __restrict__ v_new,
                                                             const int64_t* __restrict__ slots, int64_t n_new,
                                                             int kinds, int hblock, float rot_c) {
  constexpr int RB = 128 * BITS / 8;
  constexpr int NG = 128 / G;
  constexpr int kLanesPerGroup = G / 8;
  constexpr int kBytes = BITS;  // packed bytes per lane (8 channels)
  __shared__ uint32_t codes_s[16 * RB / 4];
  __shared__ uint32_t meta_s[16 * NG];
  const int which = kinds == 2 ? static_cast<int>(blockIdx.x & 1) : 0;
  const int64_t jh = kinds == 2 ? blockIdx.x >> 1 : blockIdx.x;
  const int h = static_cast<int>(jh % c.hkv);
  const int64_t j = jh / c.hkv;
  const int lane = threadIdx.x & 15, o = threadIdx.x >> 4;
  const int64_t r = 16 * j + o;
  const bool valid = r < n_new;
  // the row's data and the slots are independent loads: both in flight before the check
  uint4 raw = {0u, 0u, 0u, 0u};
  if (valid) raw = *reinterpret_cast<const uint4*>((which ? v_new : k_new) + (r * c.hkv + h) * 128 + lane * 8);
  const int64_t slot = valid ? slots[r] : 0;
  const int64_t s0 = slots[16 * j];
  const bool tile = __syncthreads_and(valid && slot == s0 + o && (s0 & 15) == 0 && (s0 % c.page) + 15 < c.page);
  if (!valid) return;  // only when not a whole tile: no barrier follows then
  float x[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  if (!tile) {
    quantize_store_row<BITS, G>(c, which, h, slot, x, lane, hblock, rot_c);
    return;
  }
  uint32_t packed, meta;
  quantize_row_codes<BITS, G>(c, which, x, lane, hblock, rot_c, packed, meta);
  uint8_t* cs = reinterpret_cast<uint8_t*>(codes_s);
  const int g = lane / kLanesPerGroup;
  const bool group_leader = (lane % kLanesPerGroup) == 0;
  if (which == 0) {
    uint8_t* dst = cs + k_code_byte(0, RB, o, lane * kBytes);
    if (BITS == 4)
      *reinterpret_cast<uint32_t*>(dst) = packed;
    else
      *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(packed);
    if (group_leader) meta_s[o * NG + g] = meta;
  } else {
#pragma unroll
    for (int k = 0; k < kBytes; ++k) cs[v_code_byte(0, RB, o, lane * kBytes + k)] = static_cast<uint8_t>(packed >> (8 * k));
    if (group_leader) meta_s[v_meta_entry(0, NG, g, o)] = meta;
  }
  __syncthreads();
  const int64_t page = s0 / c.page;
  const int64_t tile_row = (page * c.hkv + h) * c.page + (s0 - page * c.page);
  const int t = threadIdx.x;
  if (t < 16 * RB / 16) {
    uint4* dst = reinterpret_cast<uint4*>((which ? c.vc : c.kc) + tile_row * RB);
    dst[t] = reinterpret_cast<const uint4*>(codes_s)[t];
  } else if (t - 16 * RB / 16 < 16 * NG / 4) {
    const int m = t - 16 * RB / 16;
    // K meta is token-major [u][P][NG]; V meta is tile-major: both are this tile's
    // 16 NG consecutive entries
    uint32_t* mdst = which ? c.vm + (tile_row >> 4) * NG * 16 : c.km + tile_row * NG;
    reinterpret_cast<uint4*>(mdst)[m] = reinterpret_cast<const uint4*>(meta_s)[m];
  }
}

// High-precision windows (InnerQ, Abstract): one new token per row of (seqs, positions).
// The token at position t goes to window slot t (t < sink) or to the recent ring slot
// sink + (t - sink) % recent. A full ring first hands the token it holds there, position
// t - recent, to the quantizer, which stores it at evict_slots[r]. Each lane reads its
// 16 bytes of the evicted row before it writes the same 16 bytes of the new row.
template <int BITS, int G>
__global__ __launch_bounds__(256) void window_append_kernel(DevCache c, DevWindow w, const uint16_t* __restrict__ k_new,
                                                            const uint16_t* __restrict__ v_new,
                                                            const int32_t* __restrict__ seqs,
                                                            const int32_t* __restrict__ positions,
                                                            const int64_t* __restrict__ evict_slots, int64_t n_rows,
                                                            int hblock, float rot_c) {
  const int lane = threadIdx.x & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 4);
  if (row >= n_rows) return;
  const int which = static_cast<int>(row & 1);
  const int64_t rh = row >> 1;
  const int h = static_cast<int>(rh % c.hkv);
  const int64_t r = rh / c.hkv;
  const int b = seqs[r], t = positions[r];
  const int ws = t < w.sink ? t : w.sink + (t - w.sink) % w.recent;
  uint16_t* wrow = (which ? w.v : w.k) + ((static_cast<int64_t>(b) * (w.sink + w.recent) + ws) * c.hkv + h) * 128;
  uint4* mine = reinterpret_cast<uint4*>(wrow + lane * 8);
  if (!w.residual && t >= w.sink && t - w.recent >= w.sink) {  // uniform over the row's 16 lanes
    const uint4 old = *mine;
    float x[8] = {bf16_lo(old.x), bf16_hi(old.x), bf16_lo(old.y), bf16_hi(old.y),
                  bf16_lo(old.z), bf16_hi(old.z), bf16_lo(old.w), bf16_hi(old.w)};
    quantize_store_row<BITS, G>(c, which, h, evict_slots[r], x, lane, hblock, rot_c);
  }
  *mine = *reinterpret_cast<const uint4*>((which ? v_new : k_new) + rh * 128 + lane * 8);
}

// Residual (a window with sink 0 whose ring of `recent` rows holds the incomplete last
// group): when row r's token completes its group (position + 1 a multiple of recent),
// the group's ring rows are quantized into the cache at evict_slots[r] + 0 .. recent - 1.
// One 16-lane row per (row r, ring row i, kv head, K/V); rows_per_token 1 = keys only.
template <int BITS, int G>
__global__ __launch_bounds__(256) void residual_flush_kernel(DevCache c, DevWindow w, const int32_t* __restrict__ seqs,
                                                             const int32_t* __restrict__ positions,
                                                             const int64_t* __restrict__ evict_slots, int64_t n_rows,
                                                             int rows_per_token, int hblock, float rot_c) {
  const int lane = threadIdx.x & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 4);
  if (row >= n_rows) return;
  const int which = rows_per_token == 2 ? static_cast<int>(row & 1) : 0;
  const int64_t rih = rows_per_token == 2 ? row >> 1 : row;  // (r * recent + i) * Hkv + h
  const int h = static_cast<int>(rih % c.hkv);
  const int64_t ri = rih / c.hkv;
  const int i = static_cast<int>(ri % w.recent);
  const int64_t r = ri / w.recent;
  if ((positions[r] + 1) % w.recent != 0) return;  // uniform over the row's 16 lanes
  const int b = seqs[r];
  const uint16_t* src = (which ? w.v : w.k) + ((static_cast<int64_t>(b) * w.recent + i) * c.hkv + h) * 128;
  const uint4 raw = *reinterpret_cast<const uint4*>(src + lane * 8);
  float x[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  quantize_store_row<BITS, G>(c, which, h, evict_slots[r] + i, x, lane, hblock, rot_c);
}

// Entry of channel ch among the 128 {scale, zero} entries of a value token group: channel
// c = 4(n + 16(t >> 2)) + 2(t & 1) + ((t >> 1) & 1) (INT4) or 8n + (t >> 1) + 4(t & 1)
// (INT2) at 8n + t, the order in which the decode kernel's lanes hold channels.
template <int BITS>
__host__ __device__ __forceinline__ int vt_entry(int ch) {
  if (BITS == 4) return 8 * ((ch >> 2) & 15) + 4 * (ch >> 6) + 2 * (ch & 1) + ((ch >> 1) & 1);
  return 8 * (ch >> 3) + 2 * (ch & 3) + ((ch >> 2) & 1);
}

// One value token group (InnerQ, Abstract: groups along the inner dimension of the value
// product): channel ch = threadIdx.x (128 threads) of the G bf16 rows src[i * row_stride],
// i = 0..G-1, quantized by the row quantizer's formula (min/max, or hybrid) and stored for
// the tokens slot0 .. slot0 + G - 1 (one page; slot0 a multiple of G). Codes of 8 / BITS
// neighbouring channels share a byte: the lane holding the byte's first channel gathers
// them by shuffles and stores it.
template <int BITS, int G>
__device__ __forceinline__ void vgroup_quantize(const DevCache& c, const uint16_t* src, int64_t row_stride,
                                                int64_t slot0, int h) {
  constexpr int kQmax = (1 << BITS) - 1;
  constexpr int kPerByte = 8 / BITS;
  const int ch = threadIdx.x;
  // the group's G values of this channel, all loads in flight together
  float xs[G];
#pragma unroll
  for (int i = 0; i < G; ++i) xs[i] = __uint_as_float(static_cast<uint32_t>(src[i * row_stride + ch]) << 16);
  auto val = [&](int i) { return xs[i]; };
  float mn = val(0), mx = mn;
#pragma unroll
  for (int i = 1; i < G; ++i) {
    const float v = val(i);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  const float range = (mx - mn) + 0.0f;
  uint32_t s16 = float_to_f16_bits(range / static_cast<float>(kQmax));
  uint32_t z16 = float_to_f16_bits(mn + 0.0f);
  auto code_of = [&](float x, float s, float z, float inv) -> uint32_t {
    if (s == 0.0f) return 0u;
    const float diff = x - z;
    const float u = diff * inv;
    return static_cast<uint32_t>(fminf(fmaxf(__builtin_rintf(u), 0.0f), static_cast<float>(kQmax)));
  };
  if (c.quant_mode == 1) {  // hybrid: as for row groups (largest error, asymmetric on a tie)
    constexpr int kMid = 1 << (BITS - 1);
    const float amax = fmaxf(fabsf(mn), fabsf(mx));
    const uint32_t ss16 = float_to_f16_bits(amax / static_cast<float>(kMid - 1));
    const uint32_t sz16 = float_to_f16_bits(-(static_cast<float>(kMid) * f16_bits_to_float(ss16)) + 0.0f);
    auto group_err = [&](uint32_t sb, uint32_t zb) {
      const float s = f16_bits_to_float(sb), z = f16_bits_to_float(zb);
      const float inv = s != 0.0f ? 1.0f / s : 0.0f;
      float err = 0.0f;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float x = val(i);
        err = fmaxf(err, fabsf(x - __builtin_fmaf(static_cast<float>(code_of(x, s, z, inv)), s, z)));
      }
      return err;
    };
    if (group_err(ss16, sz16) < group_err(s16, z16)) {
      s16 = ss16;
      z16 = sz16;
    }
  }
  const int64_t page = slot0 / c.page;
  const int off0 = static_cast<int>(slot0 - page * c.page);
  const int64_t u = page * c.hkv + h;
  c.vm[(u * (c.page / G) + off0 / G) * 128 + vt_entry<BITS>(ch)] = s16 | (z16 << 16);
  const float s = f16_bits_to_float(s16), z = f16_bits_to_float(z16);
  const float inv = s != 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    uint32_t byte = code_of(val(i), s, z, inv);
#pragma unroll
    for (int k = 1; k < kPerByte; ++k) byte |= static_cast<uint32_t>(__shfl_down(static_cast<int>(byte & kQmax), k, 64))
                                                << (BITS * k);
    if (ch % kPerByte == 0) {
      const int off = off0 + i;
      c.vc[v_code_byte(u * c.page + (off & ~15), c.row_bytes, off & 15, ch / kPerByte)] = static_cast<uint8_t>(byte);
    }
  }
}

// Value token groups of an append: group j = rows j*G .. j*G+G-1 of v_new, kv head h.
template <int BITS, int G>
__global__ __launch_bounds__(128) void vgroup_append_kernel(DevCache c, const uint16_t* __restrict__ v_new,
                                                            const int64_t* __restrict__ slots) {
  const int h = static_cast<int>(blockIdx.x % c.hkv);
  const int64_t j = blockIdx.x / c.hkv;
  vgroup_quantize<BITS, G>(c, v_new + (j * G * c.hkv + h) * 128, static_cast<int64_t>(c.hkv) * 128, slots[j * G], h);
}

// Value token groups completed by a residual append: row r, kv head h.
template <int BITS, int G>
__global__ __launch_bounds__(128) void vgroup_flush_kernel(DevCache c, DevWindow w, const int32_t* __restrict__ seqs,
                                                           const int32_t* __restrict__ positions,
                                                           const int64_t* __restrict__ evict_slots) {
  const int h = static_cast<int>(blockIdx.x % c.hkv);
  const int64_t r = blockIdx.x / c.hkv;
  if ((positions[r] + 1) % G != 0) return;
  const int b = seqs[r];
  vgroup_quantize<BITS, G>(c, w.v + (static_cast<int64_t>(b) * G * c.hkv + h) * 128, static_cast<int64_t>(c.hkv) * 128,
                           evict_slots[r], h);
}

template <int BITS, int G>
__global__ __launch_bounds__(256) void dequantize_kernel(DevCache c, int which, const int64_t* __restrict__ slots,
                                                         int64_t n_rows, float* __restrict__ out) {
  constexpr int kLanesPerGroup = G / 8;
  const int lane = threadIdx.x & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 4);
  if (row >= n_rows) return;
  const int h = static_cast<int>(row % c.hkv);
  const int64_t r = row / c.hkv;
  const int64_t slot = slots[r];
  const int64_t page = slot / c.page;
  const int off = static_cast<int>(slot - page * c.page);
  const int64_t u = page * c.hkv + h;
  const int g = lane / kLanesPerGroup;

  const int64_t tile_row = u * c.page + (off & ~15);
  const int o = off & 15;
  constexpr int kBytes = BITS * 8 / 8;
  uint32_t packed = 0, meta;
  if (which == 0) {
    const uint8_t* src = c.kc + k_code_byte(tile_row, c.row_bytes, o, lane * kBytes);
    packed = BITS == 4 ? *reinterpret_cast<const uint32_t*>(src) : *reinterpret_cast<const uint16_t*>(src);
    meta = c.km[(u * c.page + off) * c.ngroups + g];
  } else {
#pragma unroll
    for (int k = 0; k < kBytes; ++k)
      packed |= static_cast<uint32_t>(c.vc[v_code_byte(tile_row, c.row_bytes, o, lane * kBytes + k)]) << (8 * k);
    meta = c.v_grouping ? 0u : c.vm[v_meta_entry(tile_row >> 4, c.ngroups, g, o)];
  }
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t m = (which == 1 && c.v_grouping)
                           ? c.vm[(u * (c.page / G) + off / G) * 128 + vt_entry<BITS>(lane * 8 + e)]
                           : meta;
    const uint32_t code = (packed >> (BITS * e)) & ((1u << BITS) - 1u);
    y[e] = __builtin_fmaf(static_cast<float>(code), f16_bits_to_float(m & 0xFFFFu), f16_bits_to_float(m >> 16));
  }
  float4* dst = reinterpret_cast<float4*>(out + row * 128 + lane * 8);
  dst[0] = make_float4(y[0], y[1], y[2], y[3]);
  dst[1] = make_float4(y[4], y[5], y[6], y[7]);
}

}  // namespace

hipError_t launch_quantize_append(const DevCache& c, const Geometry& g, const void* k_new, const void* v_new,
                                  const int64_t* slots, int64_t n_new, hipStream_t stream) {
  const int rows_per_token = c.v_grouping ? 1 : 2;
  const int64_t n_rows = n_new * g.hkv * rows_per_token;
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float rot_c = g.hblock > 0 ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(g.hblock))) : 1.0f;
  const auto* k = static_cast<const uint16_t*>(k_new);
  const auto* v = static_cast<const uint16_t*>(v_new);
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  // bulk appends (prefill): whole tiles at a time
  const bool tiles = n_new >= kTileAppendMin;
  const int64_t tile_blocks = (n_new + 15) / 16 * g.hkv * rows_per_token;
  if (tiles && tile_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
#define KVQ_QA(B, GS)                                                                                      \
  if (g.bits == B && g.group == GS) {                                                                      \
    if (tiles)                                                                                             \
      hipLaunchKernelGGL((quantize_tiles_kernel<B, GS>), dim3(static_cast<unsigned>(tile_blocks)), block, 0, \
                         stream, c, k, v, slots, n_new, rows_per_token, g.hblock, rot_c);                  \
    else                                                                                                   \
      hipLaunchKernelGGL((quantize_append_kernel<B, GS>), grid, block, 0, stream, c, k, v, slots, n_rows, \
                         rows_per_token, g.hblock, rot_c);                                                  \
    if (c.v_grouping) {                                                                                    \
      const int64_t units = n_new / GS * g.hkv;                                                            \
      if (units > 0)                                                                                       \
        hipLaunchKernelGGL((vgroup_append_kernel<B, GS>), dim3(static_cast<unsigned>(units)), dim3(128), 0, \
                           stream, c, v, slots);                                                           \
    }                                                                                                      \
    return hipGetLastError();                                                                              \
  }
  KVQ_QA(4, 32) KVQ_QA(4, 64) KVQ_QA(4, 128) KVQ_QA(2, 32) KVQ_QA(2, 64) KVQ_QA(2, 128)
#undef KVQ_QA
  return hipErrorInvalidValue;
}

hipError_t launch_window_append(const DevCache& c, const DevWindow& w, const Geometry& g, const void* k_new,
                                const void* v_new, const int32_t* seqs, const int32_t* positions,
                                const int64_t* evict_slots, int64_t n_new, hipStream_t stream) {
  const int64_t n_rows = n_new * g.hkv * 2;
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float rot_c = g.hblock > 0 ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(g.hblock))) : 1.0f;
  const auto* k = static_cast<const uint16_t*>(k_new);
  const auto* v = static_cast<const uint16_t*>(v_new);
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int rows_per_token = c.v_grouping ? 1 : 2;
  const int64_t flush_rows = n_new * w.recent * g.hkv * rows_per_token;
  const int64_t flush_blocks = (flush_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (w.residual && flush_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
#define KVQ_WA(B, GS)                                                                                      \
  if (g.bits == B && g.group == GS) {                                                                      \
    hipLaunchKernelGGL((window_append_kernel<B, GS>), grid, block, 0, stream, c, w, k, v, seqs, positions, \
                       evict_slots, n_rows, g.hblock, rot_c);                                              \
    if (w.residual) {                                                                                      \
      hipLaunchKernelGGL((residual_flush_kernel<B, GS>), dim3(static_cast<unsigned>(flush_blocks)), block, 0, \
                         stream, c, w, seqs, positions, evict_slots, flush_rows, rows_per_token, g.hblock,  \
                         rot_c);                                                                           \
      if (c.v_grouping)                                                                                    \
        hipLaunchKernelGGL((vgroup_flush_kernel<B, GS>), dim3(static_cast<unsigned>(n_new * g.hkv)), dim3(128), \
                           0, stream, c, w, seqs, positions, evict_slots);                                 \
    }                                                                                                      \
    return hipGetLastError();                                                                              \
  }
  KVQ_WA(4, 32) KVQ_WA(4, 64) KVQ_WA(4, 128) KVQ_WA(2, 32) KVQ_WA(2, 64) KVQ_WA(2, 128)
#undef KVQ_WA
  return hipErrorInvalidValue;
}

hipError_t launch_dequantize(const DevCache& c, const Geometry& g, int which, const int64_t* slots, int64_t n,
                             float* out, hipStream_t stream) {
  const int64_t n_rows = n * g.hkv;
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
#define KVQ_DQ(B, GS)                                                                                      \
  if (g.bits == B && g.group == GS) {                                                                      \
    hipLaunchKernelGGL((dequantize_kernel<B, GS>), grid, block, 0, stream, c, which, slots, n_rows, out); \
    return hipGetLastError();                                                                              \
  }
  KVQ_DQ(4, 32) KVQ_DQ(4, 64) KVQ_DQ(4, 128) KVQ_DQ(2, 32) KVQ_DQ(2, 64) KVQ_DQ(2, 128)
#undef KVQ_DQ
  return hipErrorInvalidValue;
}

}  // namespace kvq
