// The row quantizer shared by the append kernels and the fused append + decode step:
// one 128-channel K or V row per 16 lanes, 8 consecutive channels per lane.
//
// SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving,
// Abstract: token-wise INT4 with a block-diagonal Hadamard rotation, done by one fused
// rotation-quantization kernel that writes straight into the paged KV layout.
// InnerQ (Abstract): asymmetric groups with a scale and a zero point.
//
// Every fp32 step is a separate IEEE round-to-nearest-even operation in the order the
// library documents (each function body turns contraction off), so the codes and fp16
// scale/zero are bit-exact functions of the input, whichever kernel includes this.
#pragma once

#include <type_traits>

#include "kvq_device.h"

namespace kvq {

// The value of lane (lane ^ M) of the same 16-lane row, by DPP row permutes instead of
// LDS-routed shuffles: quad swaps for M = 1, 2; a rotation by 8 of the row for M = 8;
// for M = 4 the rotations by 4 and by 12, one of which holds lane ^ 4 for each lane.
template <int M>
__device__ __forceinline__ float lane_xor16(float v, int lane) {
#pragma clang fp contract(off)
  const int iv = __float_as_int(v);
  if (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  if (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  if (M == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false));  // row_ror:8
  const int a = __builtin_amdgcn_update_dpp(0, iv, 0x124, 0xF, 0xF, false);  // row_ror:4, lane i <- i - 4
  const int b = __builtin_amdgcn_update_dpp(0, iv, 0x12C, 0xF, 0xF, false);  // row_ror:12, lane i <- i + 4
  return __int_as_float((lane & 4) ? a : b);
}

// One 128-channel K (which = 0, rotated first) or V row, 8 channels per lane in x, 16
// lanes per row: group parameters and codes. packed = the lane's packed codes (8 channels,
// BITS * 8 bits), meta = its group's {scale | zero << 16}.
template <int BITS, int G>
__device__ __forceinline__ void quantize_row_codes(const DevCache& c, int which, float (&x)[8], int lane, int hblock,
                                                   float rot_c, uint32_t& packed_out, uint32_t& meta_out) {
#pragma clang fp contract(off)
  const bool hybrid = c.quant_mode == 1;
  constexpr int kQmax = (1 << BITS) - 1;
  constexpr int kLanesPerGroup = G / 8;
  if (which == 0 && hblock > 0) {
    // in-lane strides 1, 2, 4
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
      if (s < hblock) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!(e & s)) {
            const float a = x[e], b = x[e + s];
            x[e] = a + b;
            x[e + s] = a - b;
          }
        }
      }
    }
    // cross-lane strides 8..64: partner lane = lane ^ (stride / 8)
    auto stage = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if (8 * m < hblock) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = lane_xor16<m>(x[e], lane);
          x[e] = upper ? (y - x[e]) : (x[e] + y);
        }
      }
    };
    stage(std::integral_constant<int, 1>{});
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 4>{});
    stage(std::integral_constant<int, 8>{});
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * rot_c;
  }

  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    mn = fminf(mn, x[e]);
    mx = fmaxf(mx, x[e]);
  }
  // over the group's lanes (4, 8 or 16)
  mn = fminf(mn, lane_xor16<1>(mn, lane));
  mx = fmaxf(mx, lane_xor16<1>(mx, lane));
  mn = fminf(mn, lane_xor16<2>(mn, lane));
  mx = fmaxf(mx, lane_xor16<2>(mx, lane));
  if (kLanesPerGroup > 4) {
    mn = fminf(mn, lane_xor16<4>(mn, lane));
    mx = fmaxf(mx, lane_xor16<4>(mx, lane));
  }
  if (kLanesPerGroup > 8) {
    mn = fminf(mn, lane_xor16<8>(mn, lane));
    mx = fmaxf(mx, lane_xor16<8>(mx, lane));
  }
  const float range = (mx - mn) + 0.0f;  // +0.0f: a -0 range (mixed-sign zeros) becomes +0
  const float s32 = range / static_cast<float>(kQmax);
  uint32_t s16 = float_to_f16_bits(s32);
  uint32_t z16 = float_to_f16_bits(mn + 0.0f);  // -0 minimum stored as +0

  // codes of the lane's 8 channels for the stored pair (s16, z16)
  auto group_codes = [&](uint32_t sb, uint32_t zb, uint32_t (&cd)[8]) {
    const float s = f16_bits_to_float(sb), z = f16_bits_to_float(zb);
    if (s == 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) cd[e] = 0;
      return;
    }
    const float inv = 1.0f / s;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float diff = x[e] - z;
      const float u = diff * inv;
      cd[e] = static_cast<uint32_t>(fminf(fmaxf(__builtin_rintf(u), 0.0f), static_cast<float>(kQmax)));
    }
  };
  uint32_t cd[8];
  group_codes(s16, z16, cd);

  if (hybrid) {
    // InnerQ (Abstract): per group, symmetric or asymmetric. The symmetric pair is
    // scale = fp16(max|x| / (2^(b-1) - 1)), zero = -2^(b-1) * scale (exact in fp16); the
    // group keeps the pair with the smaller largest |x - fma(code, scale, zero)| (max is
    // exact and order-free, so every lane of the group decides alike), asymmetric on a tie.
    constexpr int kMid = 1 << (BITS - 1);
    auto group_err = [&](uint32_t sb, uint32_t zb, const uint32_t (&c8)[8]) {
      const float s = f16_bits_to_float(sb), z = f16_bits_to_float(zb);
      float err = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) err = fmaxf(err, fabsf(x[e] - __builtin_fmaf(static_cast<float>(c8[e]), s, z)));
      err = fmaxf(err, lane_xor16<1>(err, lane));
      err = fmaxf(err, lane_xor16<2>(err, lane));
      if (kLanesPerGroup > 4) err = fmaxf(err, lane_xor16<4>(err, lane));
      if (kLanesPerGroup > 8) err = fmaxf(err, lane_xor16<8>(err, lane));
      return err;
    };
    const float amax = fmaxf(fabsf(mn), fabsf(mx));
    const uint32_t ss16 = float_to_f16_bits(amax / static_cast<float>(kMid - 1));
    const uint32_t sz16 = float_to_f16_bits(-(static_cast<float>(kMid) * f16_bits_to_float(ss16)) + 0.0f);
    uint32_t cs[8];
    group_codes(ss16, sz16, cs);
    if (group_err(ss16, sz16, cs) < group_err(s16, z16, cd)) {
      s16 = ss16;
      z16 = sz16;
#pragma unroll
      for (int e = 0; e < 8; ++e) cd[e] = cs[e];
    }
  }

  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) packed |= cd[e] << (BITS * e);
  packed_out = packed;
  meta_out = s16 | (z16 << 16);
}

// The row quantizer plus its stores at `slot` (kv head h).
template <int BITS, int G>
__device__ __forceinline__ void quantize_store_row(const DevCache& c, int which, int h, int64_t slot, float (&x)[8],
                                                   int lane, int hblock, float rot_c) {
#pragma clang fp contract(off)
  constexpr int kLanesPerGroup = G / 8;
  uint32_t packed, meta;
  quantize_row_codes<BITS, G>(c, which, x, lane, hblock, rot_c, packed, meta);
  const int64_t page = slot / c.page;
  const int off = static_cast<int>(slot - page * c.page);
  const int64_t u = page * c.hkv + h;
  const int g = lane / kLanesPerGroup;
  const bool group_leader = (lane % kLanesPerGroup) == 0;

  const int64_t tile_row = u * c.page + (off & ~15);  // first token row of the 16-token tile
  const int o = off & 15;
  constexpr int kBytes = BITS * 8 / 8;  // packed bytes held by this lane (8 channels)
  if (which == 0) {
    // K tiles: rows cut into 16-byte chunks, chunk-major, so the decode kernel's loads of
    // one channel range of a tile's tokens are whole cache lines. The lane's bytes sit
    // in one chunk.
    uint8_t* dst = c.kc + k_code_byte(tile_row, c.row_bytes, o, lane * kBytes);
    if (BITS == 4)
      *reinterpret_cast<uint32_t*>(dst) = packed;
    else
      *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(packed);
    if (group_leader) c.km[(u * c.page + off) * c.ngroups + g] = meta;
  } else {
    // V tiles: rows cut into 16-bit words, each word's token pairs byte-interleaved, so
    // the decode kernel's one mask turns a token pair's same-channel codes into adjacent
    // bytes. Every token owns whole bytes: appends never share a byte.
#pragma unroll
    for (int k = 0; k < kBytes; ++k)
      c.vc[v_code_byte(tile_row, c.row_bytes, o, lane * kBytes + k)] = static_cast<uint8_t>(packed >> (8 * k));
    if (group_leader) c.vm[v_meta_entry(tile_row >> 4, c.ngroups, g, o)] = meta;
  }
}

}  // namespace kvq
