// Split-K decode attention over the packed low-bit cache, on the CDNA4 matrix cores.
//
// SAW-INT4 (Abstract): attention runs straight over the paged INT4 cache.
// InnerQ (Abstract): dequantization is aligned with the decode vector-matrix
//   products, so the per-group scale multiplies a partial dot product instead of
//   every element.
// Dual-QK (Abstract): the query receives the keys' rotation, so q.k is preserved.
//
// One wavefront (one 64-thread workgroup) owns one (sequence, kv head, partition)
// and walks it in 32-token blocks (two 16-token tiles), grouped in super-blocks of 8.
//
// Scores, v_mfma_f32_32x32x16_f16, 8 per block: C[row][token] = sum_ch A[row][ch] B[ch][token]
//   A rows = (query head jj, digit d, group g): the rotated, pre-scaled query of head jj
//     split into two f16 parts (hi = f16(x), lo = f16(x - hi)), zero outside group g.
//   B = the codes as exact f16 integers: a mask spreads the 4-bit (2-bit) codes into
//     bytes, and bytes 0..15 read as fp8-e4m3 are exactly c * 2^-9, which the scaled
//     fp8->f16 conversion turns into c. Every product is exact. (Codes could also be
//     fed as f16 subnormals c * 2^-24 with a mask alone, but the matrix core sums
//     products of subnormal operands with visibly less precision.)
//   logit = sum_g scale_g * (C[jj,hi,g] + C[jj,lo,g]) + sum_g zero_g * Qsum[jj][g].
// Softmax: exp2 domain (the query carries softmax_scale * log2 e). A super-block first
//   computes the logits of all its blocks (kept in registers), then updates the running
//   max once and rescales the state once, then runs the values: no data-dependent
//   branch touches the accumulators.
// Values, v_mfma_f32_16x16x32_f16, 16 per block: O[row][ch] += sum_t W[row][t] V[t][ch]
//   A rows = (query head jj, group g), W = 2^8 p * scale_g(t) split into f16 hi (W
//     rounded toward zero to f16: its top 11 bits) and lo (the exact remainder, rounded
//     toward zero), two MFMAs into the same accumulator; the 2^8 keeps lo out of the f16
//     subnormal range. A value scale >= 128 could push W past the f16 maximum: the
//     partition is then recomputed with W = p * scale.
//   B = value codes as exact f16 integers, from one 16-byte load per lane of the cache's
//     16-token tiles, where each word's token pairs are byte-interleaved so one mask
//     yields both tokens' codes for a channel side by side;
//   the zero term sum_t p * zero_g(t) is accumulated separately in fp32.
// Partials (unnormalised o, reference max m, sum l) go to the workspace for the combine.
//
// Groups of 64 or 128 channels (two or one per head) take a leaner form of both passes:
// Scores, v_mfma_i32_16x16x64_i8, 4 per block: C[row][token] over 64 channels per K-step
//   A rows = (query head jj, digit d): the rotated, pre-scaled query of head jj as four
//     signed int8 digits (base 128, first digit within +-64: 2^-28 of the head's largest
//     element), so one i32 sum per digit is exact; the lane holding a head's four digit
//     sums combines them.
//   B = the codes as int8 bytes, from masks alone. Each K-step lies inside one group; the
//     two 16-token tiles of a block are the two N-tiles. Lane (head q, token n) receives
//     the logits of head q for token n of both tiles. A stays in registers.
// Values: one 16x16x32 product per N-tile: the hi and lo digits of W take separate A rows
//   (head, digit, group), summed after the partition. Each lane forms W = p * scale for two
//   tokens of one head only (no lane repeats another's), and the A rows are gathered from
//   a small wave-local LDS table.
#pragma once

#include <type_traits>

#include "kvq_device.h"
#include "quant_row.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

// Two fp8-e4m3 bytes (values c * 2^-9, c = 0..15) of `bytes` -> f16x2 holding the
// integers c exactly (word 0 = bytes 0,1; word 1 = bytes 2,3).
template <bool HI_WORD>
__device__ __forceinline__ uint32_t codes_f16x2(uint32_t bytes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 512.0f, HI_WORD));
}

// Two 2-bit codes c (0..3), the low and high nibble of byte SEL of `nibbles`, -> f16x2
// holding them exactly: nibbles 0..3 read as fp4-e2m1 are c / 2 (0, 0.5, 1, 1.5), which
// the scaled fp4->f16 conversion with scale 2 turns into c.
template <int SEL>
__device__ __forceinline__ uint32_t crumbs_f16x2(uint32_t nibbles) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nibbles, 2.0f, SEL));
}

// Score MFMA p, lane half h covers the 8 channels 64h + 8p .. 64h + 8p + 7; its K-slot
// kappa (0..7) holds the channel at this position within them, the order in which
// unpack_k() below lays codes into the B operand.
template <int BITS>
__device__ __forceinline__ int qk_slot_channel(int kappa) {
  if (BITS == 4) return 2 * (kappa & 3) + (kappa >> 2);
  return 2 * (kappa & 1) + 4 * ((kappa >> 1) & 1) + (kappa >> 2);
}

// B operand of score MFMA p from the lane's packed key codes (kc: 8 dwords at INT4 =
// channels 64h..64h+63 of its token, 4 dwords at INT2).
template <int BITS>
__device__ __forceinline__ half8 unpack_k(const uint32_t* kc, int p) {
  if (BITS == 4) {
    const uint32_t w = kc[p];
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // nibbles 0,2,4,6 / 1,3,5,7
    return as_half8(codes_f16x2<false>(lo), codes_f16x2<true>(lo), codes_f16x2<false>(hi), codes_f16x2<true>(hi));
  }
  // byte j of w holds channels 4j .. 4j + 3 (crumb i = channel 4j + i); m0 keeps crumbs
  // 0 and 2 of every byte in its nibbles, m1 crumbs 1 and 3: two masks feed all four bytes
  const uint32_t w = kc[p >> 1];
  const uint32_t m0 = w & 0x33333333u, m1 = (w >> 2) & 0x33333333u;
  if (p & 1)
    return as_half8(crumbs_f16x2<2>(m0), crumbs_f16x2<3>(m0), crumbs_f16x2<2>(m1), crumbs_f16x2<3>(m1));
  return as_half8(crumbs_f16x2<0>(m0), crumbs_f16x2<1>(m0), crumbs_f16x2<0>(m1), crumbs_f16x2<1>(m1));
}

// Channel of column n (0..15) of value N-tile nt (0..7), matching unpack_v().
template <int BITS>
__device__ __forceinline__ int pv_channel(int nt, int n) {
  if (BITS == 4) return 4 * (n + 16 * (nt >> 2)) + 2 * (nt & 1) + ((nt >> 1) & 1);
  return 8 * n + (nt >> 1) + 4 * (nt & 1);
}

// B operand of value N-tile nt: vc holds, for 8 tokens (4 token pairs, one dword each),
// one 16-bit code word with the pair's bytes interleaved: [t0 byte0, t1 byte0, t0 byte1,
// t1 byte1]. INT4: words n and n+16 in vc[0..3] and vc[4..7].
template <int BITS>
__device__ __forceinline__ half8 unpack_v(const uint32_t* vc, int nt) {
  uint32_t x[4];
  if (BITS == 4) {
    const uint32_t* w = vc + 4 * (nt >> 2);
    const int sh = 4 * ((nt >> 1) & 1);  // low or high nibbles
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (w[k] >> sh) & 0x0F0F0F0Fu;
  } else {
    const int sh = 2 * (nt >> 1);  // crumb j of each byte
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (vc[k] >> sh) & 0x03030303u;
  }
  if (nt & 1)
    return as_half8(codes_f16x2<true>(x[0]), codes_f16x2<true>(x[1]), codes_f16x2<true>(x[2]), codes_f16x2<true>(x[3]));
  return as_half8(codes_f16x2<false>(x[0]), codes_f16x2<false>(x[1]), codes_f16x2<false>(x[2]),
                  codes_f16x2<false>(x[3]));
}

// Narrow groups (G = 64, 128). Channel held by K-slot s (0..15) of K-step k (0, 1) in lane
// group q (0..3, the lanes 16q..16q+15) of the int8 score MFMAs: the order in which
// unpack_k_i8() lays a K-step's codes into the B operand (and the prologue the query digits
// into A). A K-step's 16 channels of lane group q are 2 * BITS contiguous code bytes of the
// packed row; at G = 64 K-step k covers group k.
template <int BITS, int G>
__device__ __forceinline__ int narrow_channel(int k, int q, int s) {
  const int base = G == 128 ? 32 * q + 16 * k : 64 * k + 16 * q;
  if (BITS == 4) {
    const int w = s >> 2, j = s & 3;  // dword w of the operand: low / high nibbles of two dwords
    return base + 8 * (w >> 1) + 2 * j + (w & 1);
  }
  return base + 4 * (s & 3) + (s >> 2);  // dword s / 4 holds crumb s / 4 of the 4 bytes
}
// Its inverse: the position 32 q + 16 k + s of channel c in a row of A operands.
template <int BITS, int G>
__device__ __forceinline__ int narrow_position(int c) {
  const int q = G == 128 ? c >> 5 : (c >> 4) & 3;
  const int k = G == 128 ? (c >> 4) & 1 : c >> 6;
  const int off = c & 15;
  const int s = BITS == 4 ? 4 * (2 * (off >> 3) + (off & 1)) + ((off >> 1) & 3) : 4 * (off & 3) + (off >> 2);
  return 32 * q + 16 * k + s;
}
// B operand of one K-step: its BITS / 2 dwords of packed codes spread into 16 int8 codes.
template <int BITS>
__device__ __forceinline__ i32x4 unpack_k_i8(const uint32_t* d) {
  if (BITS == 4)
    return i32x4{static_cast<int>(d[0] & 0x0F0F0F0Fu), static_cast<int>((d[0] >> 4) & 0x0F0F0F0Fu),
                 static_cast<int>(d[1] & 0x0F0F0F0Fu), static_cast<int>((d[1] >> 4) & 0x0F0F0F0Fu)};
  return i32x4{static_cast<int>(d[0] & 0x03030303u), static_cast<int>((d[0] >> 2) & 0x03030303u),
               static_cast<int>((d[0] >> 4) & 0x03030303u), static_cast<int>((d[0] >> 6) & 0x03030303u)};
}

__device__ __forceinline__ float lo_f16(uint32_t m) { return f16_bits_to_float(m & 0xFFFFu); }
__device__ __forceinline__ float hi_f16(uint32_t m) { return f16_bits_to_float(m >> 16); }

template <int BITS, int NG, bool NARROW>
struct KBlock {
  uint32_t kc[BITS == 4 ? 8 : 4];  // key codes of the lane's token, channels 64h..64h+63
  uint32_t km[NG];                 // key {scale, zero} of the lane's token
};
// narrow groups: per 16-token tile t, the lane's code dwords of both K-steps (BITS / 2 each)
// and the {scale, zero} of its token in that tile
template <int BITS, int NG>
struct KBlock<BITS, NG, true> {
  uint32_t kc[2][BITS];
  uint32_t km[2][NG];
};

template <int BITS, bool NARROW = false, int NG = 4>
struct VBlock {
  uint32_t vc[BITS == 4 ? 8 : 4];  // value code words, 8 tokens
  uint32_t vm[8];                  // value {scale, zero} of group g, 8 tokens
};
// narrow groups: the {scale, zero} of the lane's two tokens (below) in every group
template <int BITS, int NG>
struct VBlock<BITS, true, NG> {
  uint32_t vc[BITS == 4 ? 8 : 4];
  uint32_t vm[NG][2];
};

__device__ __forceinline__ _Float16 f16_lo(uint32_t m) {
  return __builtin_bit_cast(_Float16, static_cast<uint16_t>(m & 0xFFFFu));
}

constexpr int NBS = 8;  // blocks per super-block
constexpr int PF = 3;   // blocks loaded ahead

// PRUNE: query-channel pruning of key reads (Dual-QK, Abstract: dynamic query-channel
// pruning further cuts key-cache reads). Per (sequence, kv head) the rotated query keeps
// the a.keep_chunks 16-byte chunks of the packed key row (128 / BITS channels each) with
// the largest summed squared query over the kv head's query heads (ties: lower chunk);
// the other channels are zeroed in the query and their key chunks are never loaded
// (the first PF blocks, loaded before the query is known, read every chunk).
// VT: value token groups (InnerQ, Abstract: dequantization aligned with the value
// vector-matrix product). A block's 32 tokens lie in one group of G tokens, whose
// {scale, zero} is per channel: the value MFMAs take p itself (A rows = (head, f16 digit
// of p), B = the codes), and each block's product C is folded per channel as
// o += scale * (C_hi + C_lo) + zero * sum_t p, so the scale multiplies a finished partial
// sum instead of every element.
// PAGED (caches whose sequences span pages): the tiles of a whole super-block are looked up
// at once into a small LDS table that both kinds' loads read (SBT below), instead of a
// block-table lookup per block and kind.
template <int BITS, int G, int R, bool PRUNE, bool VT, bool PAGED = false>
__global__ __launch_bounds__(64) void decode_split_mfma_kernel(DecodeArgs a) {
  constexpr int NG = 128 / G;
  constexpr int RB = 128 * BITS / 8;
  // one or two groups per head: int8 score MFMAs and merged value digits (see the top)
  constexpr bool NARROW = NG <= 2 && !PRUNE && !VT;
  // paged instances take their tiles a super-block at a time (SBT below)
  constexpr bool SBT = PAGED;
  using VB = std::conditional_t<NARROW, VBlock<BITS, true, NG>, VBlock<BITS>>;
  const DevCache& c = a.c;
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  // this unit's (sequence, kv head, partition); `slot` indexes its partials
  int b, hk, split, split_len, T;
  int64_t slot;
  if (a.balanced) {
    const PlanUnit pu = balanced_unit(a, unit, c.hkv, lane);
    if (pu.b < 0) return;  // past the batch's last partition
    if (pu.hk == 0 && pu.p == 0 && lane == 0) a.seq_plan[pu.b] = make_int2(pu.u, pu.n);
    b = pu.b;
    hk = pu.hk;
    split = pu.p;
    split_len = pu.L;
    T = pu.T;
    slot = static_cast<int64_t>(hk) * R * a.unit_slots + pu.u;
  } else {
    split = unit % a.num_splits;
    const int bh = unit / a.num_splits;
    hk = bh % c.hkv;
    b = bh / c.hkv;
    split_len = a.split_len;
    T = a.seq_lens[b];
    slot = (static_cast<int64_t>(b) * a.num_q_heads + hk * R) * a.num_splits + split;
  }
  // the span this kernel covers ends here (with a residual: at the last whole group);
  // a sequence longer than max_seq_len is taken as max_seq_len long
  const int qend = covered_end(a, min(T, a.max_len));
  const int start = a.tok_begin + split * split_len;
  if (start >= qend) return;
  const int end = min(qend, start + split_len);
  // This lane's 8 query channels (head lane / 16 < R), loaded ahead of the first key
  // blocks: a wave's loads complete in issue order, so a query load issued after them
  // would hold the query's preparation until the whole first fill had arrived.
  uint4 qraw = {0u, 0u, 0u, 0u};
  if ((lane >> 4) < R)
    qraw = *reinterpret_cast<const uint4*>(
        a.q + (static_cast<int64_t>(b) * a.num_q_heads + hk * R + (lane >> 4)) * 128 + 8 * (lane & 15));

  // Fused step (kvq_decode_step): the unit whose partition holds the sequence's last
  // position quantizes that token's key row (lanes 0-15) and value row (lanes 16-31) into
  // the cache, with the append kernels' row quantizer, and waits for its stores to
  // complete before it loads the block that holds them (a wave's own stores, read back by
  // the same wave). The rows are loaded here; the quantizer runs after the first blocks'
  // loads are issued and the query is prepared, unless the new token lies in one of those
  // blocks. (A position past the block table's row, seq_lens above max_seq_len: no append.)
  constexpr bool FUSE = !PRUNE && !VT;
  const bool appends =
      FUSE && a.k_new != nullptr && T - 1 >= start && T - 1 < end && (T - 1) / c.page < a.max_pages;
  uint4 new_raw = {0u, 0u, 0u, 0u};
  int64_t new_slot = 0;
  if (appends) {
    if (lane < 32) {
      const int64_t rh = static_cast<int64_t>(b) * c.hkv + hk;
      new_raw = *reinterpret_cast<const uint4*>((lane >= 16 ? a.v_new : a.k_new) + rh * 128 + (lane & 15) * 8);
    }
    const int pos = T - 1;
    new_slot = static_cast<int64_t>(a.block_table[static_cast<int64_t>(b) * a.max_pages + pos / c.page]) * c.page +
               pos % c.page;
  }
  auto append_new = [&]() {
    if constexpr (FUSE) {
      if (lane < 32) {
        float x[8] = {bf16_lo(new_raw.x), bf16_hi(new_raw.x), bf16_lo(new_raw.y), bf16_hi(new_raw.y),
                      bf16_lo(new_raw.z), bf16_hi(new_raw.z), bf16_lo(new_raw.w), bf16_hi(new_raw.w)};
        quantize_store_row<BITS, G>(c, lane >> 4, hk, new_slot, x, lane & 15, a.hblock, a.rot_c);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  };

  __shared__ float o_s[4][128];  // partial outputs, staged for the workspace stores
  __shared__ float p_s[NBS][4][32];  // p of a super-block's blocks, per head and token
  __shared__ float qsum_s[4][4];
  __shared__ int qexp_s[4];       // per head: the query carries 2^-qexp in the score MFMAs
  __shared__ half8 aqk_s[8][64];  // score A operands, re-read from LDS for every block
  __shared__ __align__(16) int8_t dig_s[4][4][128];  // narrow: query digits in A-operand order
  __shared__ __align__(16) uint32_t w_s[2][2][4][16];  // narrow: W digit pairs [digit][group][head][token pair]

  // lane roles: scores use (hQ, nQ) = (lane / 32, lane % 32): heads 2hQ, 2hQ+1 of token nQ;
  // values use (q4, r16) = (lane / 16, lane % 16): A row r16 = 4g + jj, tokens 8q4..8q4+7,
  // B column r16.
  // Narrow groups: scores use (qS, nS) = (lane / 16, lane % 16): head qS, token nS of each
  // tile; value A row r16 = 8g + 4d + jj (d = the digit of W).
  const int hQ = lane >> 5, nQ = lane & 31;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int qS = q4, nS = r16;
  const int jjV = r16 & 3, gV = NARROW ? r16 >> 3 : r16 >> 2;
  const int dV = (r16 >> 2) & 1;
  const int gVc = gV < NG ? gV : NG - 1;
  // -1 the compiler cannot see: keeps fma(f16 -> f32 x, -1, y) a single mixed-precision FMA
  float neg1 = -1.0f;
  asm("" : "+s"(neg1));

  // ---- where the partition's blocks live ----
  // nfull full 32-token blocks, then possibly one partial block
  const int nblk = (end - start + 31) >> 5;
  const int nfull = (end - start) >> 5;
  const int P = c.page;
  const int pg_first = start / P;
  const int pg_last = (end - 1) / P;
  // contiguous case: the whole partition in one page, token t in row row_base + t
  const bool one_page = pg_last == pg_first;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages;
  const int64_t row_base =
      (static_cast<int64_t>(bt[pg_first]) * c.hkv + hk) * P - static_cast<int64_t>(pg_first) * P;
  // Blocks are loaded in order, each kind through its own cursor: block index, the
  // page and in-page offset of its first token, and (paged case) a window of 64
  // block-table entries in a register, lane i holding phys * Hkv + hk for logical page
  // wbase + i (the page's tile-row block of this kv head: fewer than 2^32, checked on the
  // host), so a lookup is one readlane and one 32 x 32-bit multiply. A cursor stops at
  // the last block (no load is issued past it).
  struct Cursor {
    int blk, pg, off, wbase;
    uint32_t bt_w;
  };
  // The refill is consumed where it is loaded: a load still pending where a refilled and a
  // kept window meet would make every later lookup wait for all loads in flight (the
  // prefetched blocks included), not just for this one.
  auto window = [&](int first) -> uint32_t {
    int32_t w = (first + lane <= pg_last) ? bt[first + lane] : 0;
    asm volatile("" : "+v"(w));
    return static_cast<uint32_t>(w) * static_cast<uint32_t>(c.hkv) + static_cast<uint32_t>(hk);
  };
  const Cursor cur0 = {0, pg_first, start - pg_first * P, pg_first, one_page ? 0u : window(pg_first)};
  // contiguous full blocks need only the block index (step_blk); the paged lookup the page
  // and offset too (advance)
  auto step_blk = [&](Cursor& cu) { cu.blk = min(cu.blk + 1, nblk - 1); };
  auto advance = [&](Cursor& cu) {
    if (cu.blk + 1 < nblk) {
      ++cu.blk;
      cu.off += 32;
      while (cu.off >= P) {
        cu.off -= P;
        ++cu.pg;
      }
    }
  };
  // The cursor block's two 16-token tiles as tile indices: a tile of one kv head starts at
  // row 16 t, and t stays below 2^32 (num_pages * Hkv * page / 16, checked on the host), so
  // the first tile t0 and the step d to the second (t0 + d; d = 0 when the second lies past
  // the partition end: the first tile again) are 32-bit. One window check per block keeps
  // both of its pages in the window.
  const uint32_t p16 = static_cast<uint32_t>(P >> 4);  // tiles per page
  auto tile_ids = [&](Cursor& cu, uint32_t& t0, uint32_t& d) {
    const int tok = start + 32 * cu.blk;
    if (one_page || SBT) {  // (SBT: only one-page partitions get here)
      t0 = static_cast<uint32_t>((row_base + tok) >> 4);
      d = tok + 16 < end ? 1u : 0u;
      return;
    }
    if (cu.pg + 1 - cu.wbase >= 64) {  // a cursor visits pages in increasing order
      cu.wbase = cu.pg;
      cu.bt_w = window(cu.pg);
    }
    const int i0 = cu.pg - cu.wbase;  // 0 .. 62
    t0 = __builtin_amdgcn_readlane(cu.bt_w, i0) * p16 + static_cast<uint32_t>(cu.off >> 4);
    if (tok + 16 >= end)
      d = 0u;
    else if (cu.off + 16 < P)
      d = 1u;
    else  // the second tile opens the next page (off = P - 16)
      d = __builtin_amdgcn_readlane(cu.bt_w, i0 + 1) * p16 - t0;
  };

  // the same as token rows (narrow groups)
  auto tile_rows = [&](Cursor& cu, int64_t& row0, int64_t& row1) {
    uint32_t t0, d;
    tile_ids(cu, t0, d);
    row0 = static_cast<int64_t>(t0) << 4;
    row1 = static_cast<int64_t>(t0 + d) << 4;
  };
  // SBT (paged instances): the tiles of a whole super-block at a time. Lanes 0..15
  // take the 16 tiles of its 8 blocks (lane 2j + h: tile h of block j; a block past the
  // partition's last repeats the last, a tile past the partition end its block's first),
  // divide their offset from the walk's page by the tiles per page, fetch the page's entry
  // from the window of block-table entries with one cross-lane permute, and write the tile
  // indices to a two-slot LDS table (slot = super-block mod 2) that both kinds' loads read
  // per lane; lane 16 finds the next super-block's page and offset. A super-block's table
  // is written before its first key load (the previous super-block's value pass, or the
  // prologue) and read until the next one's value pass rewrites the other slot.
  __shared__ __align__(8) uint32_t sbid_s[SBT ? 2 : 1][16];
  struct SbWalk {
    int blk, pg, off16, wbase;  // the super-block's first block, its page, tile offset in it
    uint32_t bt_w;              // window of block-table entries from page wbase
  };
  const SbWalk walk0 = {0, pg_first, (start - pg_first * P) >> 4, pg_first, cur0.bt_w};
  SbWalk walk = walk0;
  // 1 / p16, for the lanes' quotients below: their offsets stay below p16 + 2 NBS + 1, so
  // the fp32 estimate is within one of the quotient and one correction makes it exact
  const float p16_rcp =
      __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, 1.0f / static_cast<float>(p16))));
  auto sb_ids = [&](SbWalk& w) {
    // the lane index is re-read here, so that nothing derived from it stays live in a
    // register between super-blocks
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int x16;
    if (ln < 16) {
      const int j = min(ln >> 1, nblk - 1 - w.blk);
      const int h = start + 32 * (w.blk + j) + 16 < end ? (ln & 1) : 0;
      x16 = w.off16 + 2 * j + h;
    } else {
      x16 = w.off16 + 2 * NBS;
    }
    uint32_t q = static_cast<uint32_t>(static_cast<float>(x16) * p16_rcp);
    int r = x16 - static_cast<int>(q * p16);
    if (r < 0) {
      --q;
      r += static_cast<int>(p16);
    } else if (r >= static_cast<int>(p16)) {
      ++q;
      r -= static_cast<int>(p16);
    }
    // pages w.pg .. w.pg + q(lane 15) hold the super-block (a cursor visits pages in
    // increasing order; the window reaches at most pg_last)
    const int qlast = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(static_cast<int>(q), 15));
    if (w.pg + qlast - w.wbase >= 64) {
      w.wbase = w.pg;
      w.bt_w = window(w.pg);
    }
    const int wi = (w.pg + static_cast<int>(q) - w.wbase) & 63;
    const uint32_t u = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * wi, static_cast<int>(w.bt_w)));
    if (ln < 16) sbid_s[(w.blk >> 3) & 1][ln] = u * p16 + static_cast<uint32_t>(r);
    w.blk += NBS;
    w.pg += __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(static_cast<int>(q), 16));
    w.off16 = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(static_cast<int>(r), 16));
  };
  // this lane's tile of the cursor block from the table (both tiles in one read; `second`:
  // the lane reads the block's second tile)
  auto sb_tile = [&](const Cursor& cu, bool second) -> uint32_t {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = *reinterpret_cast<const u32x2*>(&sbid_s[(cu.blk >> 3) & 1][2 * (cu.blk & 7)]);
    return second ? t[1] : t[0];
  };
  // both tiles of the cursor block from the table, as token rows (a wave-uniform pair:
  // the narrow-group key loads address one tile per instruction)
  auto sb_rows = [&](const Cursor& cu, int64_t& row0, int64_t& row1) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = *reinterpret_cast<const u32x2*>(&sbid_s[(cu.blk >> 3) & 1][2 * (cu.blk & 7)]);
    row0 = static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(t[0])))) << 4;
    row1 = static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(t[1])))) << 4;
  };
  auto value_next = [&](Cursor& cu) {
    if constexpr (PAGED)
      step_blk(cu);  // only one-page partitions get here (the table serves the others)
    else
      advance(cu);
  };

  // This lane's pieces of a block, relative to the first token row (tile_row) of its
  // tile: key codes, the 16-byte chunk(s) of channels 64 hQ .. 64 hQ + 63 of token nQ
  // (tiles are chunk-major, so one load instruction reads whole cache lines); value code
  // words r16 and r16 + 16 of tokens 8 (q4 % 2) ..; value {scale, zero} of group gVc,
  // tokens 8 (q4 % 2) + 0..3 (part 0) and + 4..7 (part 1).
  constexpr int KCH = BITS == 4 ? 2 : 1;  // key code chunks per lane
  const uint32_t kc_lane = static_cast<uint32_t>((KCH * hQ * 16 + (nQ & 15)) * 16);
  const uint32_t vc_lane = static_cast<uint32_t>((r16 * 16 + 8 * (q4 & 1)) * 2);
  const uint32_t vm_lane = static_cast<uint32_t>((gVc * 2 + (q4 & 1)) * 4 * 4);
  // the same for a full block of a contiguous partition, relative to the block's first row
  const uint32_t koff = static_cast<uint32_t>((nQ >> 4) * 16 * RB) + kc_lane;
  const uint32_t kmoff = static_cast<uint32_t>(nQ * NG * 4);
  const uint32_t voff = static_cast<uint32_t>(q4 < 2 ? 0 : 16 * RB) + vc_lane;
  const uint32_t vmoff = static_cast<uint32_t>(q4 < 2 ? 0 : NG * 64) + vm_lane;
  // Off the contiguous fast path a lane's tile is t0 + (mask & d), its second-tile lanes
  // taking the mask: its address is one multiply-add from these per-lane bases.
  const uint32_t hmK = nQ < 16 ? 0u : ~0u;  // key loads: token nQ lies in the second tile
  const uint32_t hmV = q4 < 2 ? 0u : ~0u;   // value loads: tokens 8 q4 .. lie in the second tile
  const uint8_t* const kc_l = c.kc + kc_lane;
  const uint8_t* const km_l = reinterpret_cast<const uint8_t*>(c.km) + (nQ & 15) * NG * 4;
  const uint8_t* const vc_l = c.vc + vc_lane;
  const uint8_t* const vm_l = reinterpret_cast<const uint8_t*>(c.vm) + vm_lane;
  // Key and value streams are read once: non-temporal loads. V meta loads cover whole
  // cache lines only with 4 groups; with fewer they read half lines and stay cached.
  auto ld16 = [](const uint8_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); };

  // kept key chunks (bit j = chunk j); every chunk until the query has been ranked
  constexpr int NCH = RB / 16;
  int kmask = (1 << NCH) - 1;

  // narrow: lane group qS's code bytes of K-step k start at byte knb[k] of the packed row
  // (G = 128: both K-steps in one piece of 4 BITS bytes)
  int knoff[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int bk = G == 128 ? 4 * qS * BITS + 2 * k * BITS : 8 * k * BITS + 2 * qS * BITS;
    knoff[k] = ((bk >> 4) * 16 + nS) * 16 + (bk & 15);
  }
  auto load_k_narrow = [&](Cursor& cu, auto full) {
    KBlock<BITS, NG, true> kb;
    int64_t row0, row1;
    if (one_page && (decltype(full)::value || start + 32 * cu.blk + 32 <= end)) {
      row0 = row_base + start + 32 * cu.blk;  // a multiple of 16
      row1 = row0 + 16;
      step_blk(cu);
    } else if (SBT && !one_page) {
      sb_rows(cu, row0, row1);
      step_blk(cu);
    } else {
      tile_rows(cu, row0, row1);
      advance(cu);
    }
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t row = t ? row1 : row0;
      const uint8_t* tile = c.kc + row * RB;
      if (G == 128 && BITS == 4) {
        const u32x4 x = ld16(tile + knoff[0]);
        kb.kc[t][0] = x[0]; kb.kc[t][1] = x[1]; kb.kc[t][2] = x[2]; kb.kc[t][3] = x[3];
      } else if (G == 128) {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tile + knoff[0]));
        kb.kc[t][0] = x[0]; kb.kc[t][1 % BITS] = x[1];
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (BITS == 4) {
            const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tile + knoff[k]));
            kb.kc[t][2 * k] = x[0]; kb.kc[t][(2 * k + 1) % BITS] = x[1];
          } else {
            kb.kc[t][k % BITS] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(tile + knoff[k]));
          }
        }
      }
      const uint32_t* m = c.km + (row + nS) * NG;
      if (NG == 2) {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(m));
        kb.km[t][0] = x[0]; kb.km[t][1 % NG] = x[1];
      } else {
        kb.km[t][0] = __builtin_nontemporal_load(m);
      }
    }
    return kb;
  };
  auto load_k_wide = [&](Cursor& cu, auto full) {
    KBlock<BITS, NG, false> kb;
    const uint8_t* src;
    const uint8_t* msrc;
    if (one_page && (decltype(full)::value || start + 32 * cu.blk + 32 <= end)) {
      const int64_t r0 = row_base + start + 32 * cu.blk;  // a multiple of 16
      src = c.kc + r0 * RB + koff;
      msrc = reinterpret_cast<const uint8_t*>(c.km) + r0 * (NG * 4) + kmoff;
      step_blk(cu);
    } else if (SBT && !one_page) {
      const uint32_t ts = sb_tile(cu, nQ >= 16);
      src = kc_l + static_cast<uint64_t>(ts) * (16 * RB);
      msrc = km_l + static_cast<uint64_t>(ts) * (16 * NG * 4);
      step_blk(cu);
    } else {
      uint32_t t0, d;
      tile_ids(cu, t0, d);
      const uint32_t ts = t0 + (hmK & d);  // this lane's tile
      src = kc_l + static_cast<uint64_t>(ts) * (16 * RB);
      msrc = km_l + static_cast<uint64_t>(ts) * (16 * NG * 4);
      advance(cu);
    }
    u32x4 x0 = {0u, 0u, 0u, 0u};
    if (!PRUNE || ((kmask >> (KCH * hQ)) & 1)) x0 = ld16(src);
    kb.kc[0] = x0[0]; kb.kc[1] = x0[1]; kb.kc[2] = x0[2]; kb.kc[3] = x0[3];
    if (BITS == 4) {
      u32x4 x1 = {0u, 0u, 0u, 0u};
      if (!PRUNE || ((kmask >> (KCH * hQ + 1)) & 1)) x1 = ld16(src + 16 * 16);  // the next chunk of the token
      kb.kc[4] = x1[0]; kb.kc[5] = x1[1]; kb.kc[6] = x1[2]; kb.kc[7] = x1[3];
    }
    if (NG == 4) {
      const u32x4 mm = ld16(msrc);
      kb.km[0] = mm[0]; kb.km[1] = mm[1]; kb.km[2 % NG] = mm[2]; kb.km[3 % NG] = mm[3];
    } else if (NG == 2) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 mm = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(msrc));
      kb.km[0] = mm[0]; kb.km[1 % NG] = mm[1];
    } else {
      kb.km[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(msrc));
    }
    return kb;
  };
  // `full`: the block is known to be a full one (inside an unguarded super-block)
  auto load_k = [&](Cursor& cu, auto full) {
    if constexpr (NARROW)
      return load_k_narrow(cu, full);
    else
      return load_k_wide(cu, full);
  };
  // narrow: this lane's two tokens 8 (q4 % 2) + 2 i4 + e (e = 0, 1) of tile q4 / 2, i4 = r16 / 4;
  // their {scale, zero} entries of group g are adjacent in the tile's meta, part i4 / 2
  const int i4 = r16 >> 2;
  const uint32_t vmn_lane = static_cast<uint32_t>((((i4 >> 1) * NG) * 2 + (q4 & 1)) * 16 + 8 * (i4 & 1));
  auto load_v_narrow = [&](Cursor& cu, auto full) {
    VBlock<BITS, true, NG> vb;
    const uint8_t* src;
    const uint8_t* msrc;
    if (one_page && (decltype(full)::value || start + 32 * cu.blk + 32 <= end)) {
      const int64_t r0 = row_base + start + 32 * cu.blk;  // a multiple of 16
      src = c.vc + r0 * RB + voff;
      msrc = reinterpret_cast<const uint8_t*>(c.vm) + (r0 / 16 + (q4 >> 1)) * (NG * 64) + vmn_lane;
      step_blk(cu);
    } else if (SBT && !one_page) {
      const uint32_t ts = sb_tile(cu, q4 >= 2);  // value tile of tokens 8q4..8q4+7
      src = vc_l + static_cast<uint64_t>(ts) * (16 * RB);
      msrc = reinterpret_cast<const uint8_t*>(c.vm) + vmn_lane + static_cast<uint64_t>(ts) * (NG * 64);
      step_blk(cu);
    } else {
      int64_t row0, row1;
      tile_rows(cu, row0, row1);
      const int64_t trow = (q4 < 2) ? row0 : row1;
      src = c.vc + trow * RB + vc_lane;
      msrc = reinterpret_cast<const uint8_t*>(c.vm) + (trow / 16) * (NG * 64) + vmn_lane;
      value_next(cu);
    }
    const u32x4 w0 = ld16(src);
    vb.vc[0] = w0[0]; vb.vc[1] = w0[1]; vb.vc[2] = w0[2]; vb.vc[3] = w0[3];
    if (BITS == 4) {
      const u32x4 w1 = ld16(src + 16 * 16 * 2);
      vb.vc[4] = w1[0]; vb.vc[5] = w1[1]; vb.vc[6] = w1[2]; vb.vc[7] = w1[3];
    }
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int g = 0; g < NG; ++g) {  // group g's entries sit 32 bytes after group g - 1's
      const u32x2 m = *reinterpret_cast<const u32x2*>(msrc + 32 * g);
      vb.vm[g][0] = m[0];
      vb.vm[g][1] = m[1];
    }
    return vb;
  };
  auto load_v_wide = [&](Cursor& cu, auto full) {
    VBlock<BITS> vb;
    const uint8_t* src;   // this lane's first code word of its 8 tokens
    const uint8_t* msrc;  // this lane's value {scale, zero}, part 0
    int64_t brow;         // row of the block's first token
    if (one_page && (decltype(full)::value || start + 32 * cu.blk + 32 <= end)) {
      const int64_t r0 = row_base + start + 32 * cu.blk;  // a multiple of 16
      src = c.vc + r0 * RB + voff;
      msrc = reinterpret_cast<const uint8_t*>(c.vm) + (r0 / 16) * (NG * 64) + vmoff;
      brow = r0;
      step_blk(cu);
    } else if (SBT && !one_page) {
      const uint32_t ts = sb_tile(cu, q4 >= 2);  // value tile of tokens 8q4..8q4+7
      src = vc_l + static_cast<uint64_t>(ts) * (16 * RB);
      msrc = vm_l + static_cast<uint64_t>(ts) * (NG * 64);
      brow = 0;  // (value token groups have no paged instances)
      step_blk(cu);
    } else {
      uint32_t t0, d;
      tile_ids(cu, t0, d);
      const uint32_t ts = t0 + (hmV & d);  // value tile of tokens 8q4..8q4+7
      src = vc_l + static_cast<uint64_t>(ts) * (16 * RB);
      msrc = vm_l + static_cast<uint64_t>(ts) * (NG * 64);
      brow = static_cast<int64_t>(t0) << 4;
      value_next(cu);
    }
    if (VT) {
      // {scale, zero} of channels pv_channel(0..7, r16): entries 8 r16 .. 8 r16 + 7 of the
      // block's token group (row / G: pages hold whole groups); re-read by the group's
      // blocks, so ordinary cached loads
      const u32x4* gm = reinterpret_cast<const u32x4*>(c.vm + (brow / G) * 128 + 8 * r16);
      const u32x4 g0 = gm[0], g1 = gm[1];
      vb.vm[0] = g0[0]; vb.vm[1] = g0[1]; vb.vm[2] = g0[2]; vb.vm[3] = g0[3];
      vb.vm[4] = g1[0]; vb.vm[5] = g1[1]; vb.vm[6] = g1[2]; vb.vm[7] = g1[3];
      const u32x4 w0 = ld16(src);
      vb.vc[0] = w0[0]; vb.vc[1] = w0[1]; vb.vc[2] = w0[2]; vb.vc[3] = w0[3];
      if (BITS == 4) {
        const u32x4 w1 = ld16(src + 16 * 16 * 2);
        vb.vc[4] = w1[0]; vb.vc[5] = w1[1]; vb.vc[6] = w1[2]; vb.vc[7] = w1[3];
      }
      return vb;
    }
    const u32x4 w0 = ld16(src);
    vb.vc[0] = w0[0]; vb.vc[1] = w0[1]; vb.vc[2] = w0[2]; vb.vc[3] = w0[3];
    if (BITS == 4) {
      const u32x4 w1 = ld16(src + 16 * 16 * 2);
      vb.vc[4] = w1[0]; vb.vc[5] = w1[1]; vb.vc[6] = w1[2]; vb.vc[7] = w1[3];
    }
    const uint8_t* msrc1 = msrc + NG * 8 * 4;  // part 1
    const u32x4 m0 = NG == 4 ? ld16(msrc) : *reinterpret_cast<const u32x4*>(msrc);
    const u32x4 m1 = NG == 4 ? ld16(msrc1) : *reinterpret_cast<const u32x4*>(msrc1);
    vb.vm[0] = m0[0]; vb.vm[1] = m0[1]; vb.vm[2] = m0[2]; vb.vm[3] = m0[3];
    vb.vm[4] = m1[0]; vb.vm[5] = m1[1]; vb.vm[6] = m1[2]; vb.vm[7] = m1[3];
    return vb;
  };
  auto load_v = [&](Cursor& cu, auto full) {
    if constexpr (NARROW)
      return load_v_narrow(cu, full);
    else
      return load_v_wide(cu, full);
  };

  // the new token in one of the first PF blocks: appended before they are loaded
  const bool append_early = appends && (T - 1 - start) / 32 < PF;
  if (append_early) append_new();

  // the first key blocks are in flight while the query is prepared
  // a buffer whose block lies past the partition's end is zeroed instead of loaded (so
  // the old contents die at their last use)
  using KBT = KBlock<BITS, NG, NARROW>;
  KBT kb[PF + 1];
  VB vb[PF + 1];
  Cursor kcur = cur0, vcur = cur0;
  if constexpr (SBT) {
    if (!one_page) sb_ids(walk);
  }
#pragma unroll
  for (int j = 0; j < PF; ++j) kb[j] = j < nblk ? load_k(kcur, std::false_type{}) : KBT{};

  // ---- rotated, scaled query of the R heads: score A operands and group sums ----
  // Lane (head jq = lane / 16, chunk c16 = lane % 16) holds channels 8 c16 .. 8 c16 + 7.
  // The Walsh-Hadamard butterfly runs in registers: strides 1, 2, 4 in the lane, 8..64
  // across the 16 lanes of the head. A chunk is exactly the channel set of score MFMA
  // p = c16 % 8 in lane half c16 / 8, so each lane writes its own two A rows (hi and lo
  // digit of head jq, group of the chunk); every other row of an A operand is zero.
  {
    const int jq = lane >> 4, c16 = lane & 15;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (jq < R) {
      const uint4 raw = qraw;
      x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x); x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
      x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z); x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
    }
    const int hb = a.hblock;
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
      if (s < hb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!(e & s)) {
            const float u = x[e], v = x[e + s];
            x[e] = u + v;
            x[e + s] = u - v;
          }
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      if (8 * m < hb) {
        const bool upper = (c16 & m) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = __shfl_xor(x[e], m, 64);
          x[e] = upper ? (y - x[e]) : (x[e] + y);
        }
      }
    }
    if (PRUNE) {
      // chunk energies: the lane's squared channels, summed over the chunk's lanes and the
      // heads, then read from the lanes of head 0 that open each chunk
      constexpr int LPC = 128 / BITS / 8;  // lanes per chunk
      float e2 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) e2 = __builtin_fmaf(x[e], x[e], e2);
#pragma unroll
      for (int m = 1; m < LPC; m <<= 1) e2 += __shfl_xor(e2, m, 64);
      e2 += __shfl_xor(e2, 16, 64);
      e2 += __shfl_xor(e2, 32, 64);
      float en[NCH];
#pragma unroll
      for (int j = 0; j < NCH; ++j) en[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e2), j * LPC));
      int keep = 0;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        int rank = 0;
#pragma unroll
        for (int i = 0; i < NCH; ++i) rank += (en[i] > en[j] || (en[i] == en[j] && i < j)) ? 1 : 0;
        if (rank < a.keep_chunks) keep |= 1 << j;
      }
      kmask = keep;
      if (!((kmask >> (c16 / LPC)) & 1)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      if (split == 0 && lane == 0 && a.chunk_mask != nullptr) a.chunk_mask[static_cast<int64_t>(b) * c.hkv + hk] = kmask;
    }
    const float qmul = (hb > 0 ? a.rot_c : 1.0f) * a.qscale;
    // Each head's scaled query is brought to a largest magnitude in [2^13, 2^14) by a
    // power of two 2^-qe (exact) before the f16 split: no finite query overflows the f16
    // range, and the lo digit stays clear of the f16 subnormals. The scores multiply the
    // logits back by 2^qe.
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = x[e] * qmul;
      amax = fmaxf(amax, fabsf(v[e]));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));  // the head's 16 lanes
    const int qe = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 14 : 0;
    if constexpr (NARROW) {
      // Four int8 digits per channel, base 128: x = v 2^-ne lies in (-64, 64); d0 = rint(x),
      // then each next digit is rint(128 r) of the previous remainder r (|r| <= 1/2), every
      // step exact in fp32, so x = d0 + d1 2^-7 + d2 2^-14 + d3 2^-21 up to 2^-22. The score
      // MFMAs sum each digit against the codes in int32 (exact); the sums are recombined as
      // D = 2^21 d0 + 2^14 d1 + 2^7 d2 + d3 per channel, and the logits carry 2^(ne - 21).
      const int ne = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 6 : 0;
      float part = 0.f;  // the lane's sum of D 2^-21 over its 8 channels
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float r = __builtin_amdgcn_ldexpf(v[e], -ne);
        float dg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dg[i] = __builtin_rintf(r);
          r = (r - dg[i]) * 128.0f;
        }
        if (jq < R) {
          const int pos = narrow_position<BITS, G>(8 * c16 + e);
#pragma unroll
          for (int i = 0; i < 4; ++i) dig_s[jq][i][pos] = static_cast<int8_t>(dg[i]);
        }
        part += dg[0] + dg[1] * 0x1p-7f + dg[2] * 0x1p-14f + dg[3] * 0x1p-21f;
      }
#pragma unroll
      for (int m = 1; m < G / 8; m <<= 1) part += __shfl_xor(part, m, 64);
      if (jq < R && (c16 % (G / 8)) == 0) qsum_s[jq][(8 * c16) / G] = part * 0x1p21f;
      if (c16 == 0 && jq < R) qexp_s[jq] = ne - 21;
    } else {
    _Float16 hi[8], lo[8];
    float part = 0.f;  // group sum of the query as the MFMA sees it (hi + lo)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = __builtin_amdgcn_ldexpf(v[e], -qe);
      hi[e] = static_cast<_Float16>(s);
      lo[e] = static_cast<_Float16>(s - static_cast<float>(hi[e]));
      part += static_cast<float>(hi[e]) + static_cast<float>(lo[e]);
    }
    if (c16 == 0 && jq < R) qexp_s[jq] = qe;
#pragma unroll
    for (int p = 0; p < 8; ++p) aqk_s[p][lane] = half8{};
    __syncthreads();
    if (jq < R) {
      const int p = c16 & 7, hA = c16 >> 3, g = (8 * c16) / G;
      const int rho = 8 * g + 4 * (jq >> 1) + 2 * (jq & 1);
      half8 vh, vl;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        vh[k] = hi[qk_slot_channel<BITS>(k)];
        vl[k] = lo[qk_slot_channel<BITS>(k)];
      }
      aqk_s[p][32 * hA + rho] = vh;
      aqk_s[p][32 * hA + rho + 1] = vl;
    }
#pragma unroll
    for (int m = 1; m < G / 8; m <<= 1) part += __shfl_xor(part, m, 64);
    if (jq < R && (c16 % (G / 8)) == 0) qsum_s[jq][(8 * c16) / G] = part;
    }
  }
  __syncthreads();

  // narrow: the score A operands of both K-steps, held in registers (lane: row r16 = 4 jj + d
  // of A, K-slots 16 q4 ..; rows of heads beyond R are zero)
  i32x4 aq[2] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
  if constexpr (NARROW) {
    const int jjA = r16 >> 2, dA = r16 & 3;
    if (jjA < R) {
#pragma unroll
      for (int k = 0; k < 2; ++k) aq[k] = *reinterpret_cast<const i32x4*>(&dig_s[jjA][dA][32 * q4 + 16 * k]);
    }
  }

  // the query sums and the power of two of the lane's heads: 2hQ + j2 (narrow: qS only)
  float qsum[2][NG];
  int qexp[2];
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2) {
    const int jh = NARROW ? qS : 2 * hQ + j2;
    qexp[j2] = (jh < R) ? qexp_s[jh] : 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) qsum[j2][g] = (jh < R) ? qsum_s[jh][g] : 0.f;
  }

  if (appends && !append_early) append_new();

  // ---- state (exp2 domain) ----
  // p = 2^(logit - mref) with mref = mrun - shift, mrun the running max: the value
  // weights carry 2^shift (shift = 8), which keeps the f16 split of p * scale clear of the
  // f16 subnormal range; written partials hold mref, so the factor cancels in the
  // combine. A value scale >= 128 could push the weights past the f16 maximum: the
  // partition is then recomputed with shift = 0.
  float mrun[2], mref[2], lsum[2], zacc;
  float zaccN[2];  // narrow: the lane's share of sum_t p * zero for head jjV, groups 0 / 1
  floatx4 acc[8];

  // scores of one block, narrow groups: logits of head qS for token nS of tiles 0 and 1
  auto qk_narrow = [&](const KBlock<BITS, NG, true>& kb, int t0, auto tail, float (&logit)[2]) {
    constexpr bool TAIL = decltype(tail)::value;
    i32x4 C[2][NG];
    __builtin_amdgcn_s_setprio(1);  // the matrix-core cluster (see below)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        const i32x4 bk = unpack_k_i8<BITS>(&kb.kc[t][k * (BITS / 2)]);
        const i32x4 zero = {0, 0, 0, 0};
        if (NG == 1)
          C[t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[k], bk, k == 0 ? zero : C[t][0], 0, 0, 0);
        else
          C[t][k % NG] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[k], bk, zero, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        // rows 4 qS + d of C: head qS, digit d. Pairs of digit sums recombine exactly in
        // integers below 2^24 (|sum| <= 64 * 15 * 128 per digit), then one fp32 FMA.
        const int hi = static_cast<int>((static_cast<uint32_t>(C[t][g][0]) << 7) + static_cast<uint32_t>(C[t][g][1]));
        const int lo = static_cast<int>((static_cast<uint32_t>(C[t][g][2]) << 7) + static_cast<uint32_t>(C[t][g][3]));
        const float sum = __builtin_fmaf(static_cast<float>(hi), 16384.0f, static_cast<float>(lo));
        acc = __builtin_fmaf(lo_f16(kb.km[t][g]), sum, acc);
        acc = __builtin_fmaf(hi_f16(kb.km[t][g]), qsum[0][g], acc);
      }
      logit[t] = __builtin_amdgcn_ldexpf(acc, qexp[0]);
      if (TAIL) logit[t] = (t0 + 16 * t + nS < end) ? logit[t] : -INFINITY;
    }
    asm volatile("" : "+v"(logit[0]), "+v"(logit[1]));
  };

  // scores of one block: logits of heads 2hQ, 2hQ+1 for token nQ
  auto qk_wide = [&](const KBlock<BITS, NG, false>& kb, int t0, auto tail, float (&logit)[2]) {
    constexpr bool TAIL = decltype(tail)::value;
    half8 a_next[2] = {aqk_s[0][lane], aqk_s[1][lane]};
    floatx16 cs;
    // The matrix-core clusters run at raised wave priority: when both waves of a SIMD are
    // ready, the one feeding the matrix core issues first and the other's VALU work fills
    // in behind it (H1: ~2 % faster than equal priorities; raising it around the loads
    // instead gained nothing).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      // keep each unpack next to its MFMA (bounds the live operand registers); the A
      // operand is read from LDS two MFMAs ahead
      __builtin_amdgcn_sched_barrier(0);
      const half8 ap = a_next[p & 1];
      if (p + 2 < 8) a_next[p & 1] = aqk_s[p + 2][lane];
      cs = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap, unpack_k<BITS>(kb.kc, p), p == 0 ? floatx16{} : cs, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      float sa = 0.f, zb = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        // fp16 scale/zero feed the fused mixed-precision FMAs directly
        sa = __builtin_fmaf(lo_f16(kb.km[g]), cs[4 * g + 2 * j2], sa);
        sa = __builtin_fmaf(lo_f16(kb.km[g]), cs[4 * g + 2 * j2 + 1], sa);
        zb = __builtin_fmaf(hi_f16(kb.km[g]), qsum[j2][g], zb);
      }
      logit[j2] = __builtin_amdgcn_ldexpf(sa + zb, qexp[j2]);
      if (TAIL) logit[j2] = (t0 + nQ < end) ? logit[j2] : -INFINITY;
    }
    // materialise the logits here: left to the compiler, the fold sinks to the logits'
    // later use and every block's 16 score registers stay live until then
    asm volatile("" : "+v"(logit[0]), "+v"(logit[1]));
  };
  auto qk = [&](const KBlock<BITS, NG, NARROW>& kb, int t0, auto tail, float (&logit)[2]) {
    if constexpr (NARROW)
      qk_narrow(kb, t0, tail, logit);
    else
      qk_wide(kb, t0, tail, logit);
  };

  // new running max from the lane-local maxima bm of a group of blocks; rescales the
  // state to the new reference (unconditionally: alpha = 1 when the max is unchanged)
  auto advance_max = [&](float bm0, float bm1, float shift) {
    if constexpr (NARROW) {
      // both logit slots belong to head qS: one max over the slots and the head's 16 lanes
      float bm = fmaxf(bm0, bm1);
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) bm = fmaxf(bm, __shfl_xor(bm, m, 64));
      const float n0 = fmaxf(mrun[0], bm);
      const float r0 = n0 - shift;
      const float al = __builtin_amdgcn_exp2f(mref[0] - r0);
      mrun[0] = n0;
      mref[0] = r0;
      lsum[0] *= al;
      const float alpha[4] = {__shfl(al, 0, 64), __shfl(al, 16, 64), __shfl(al, 32, 64), __shfl(al, 48, 64)};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] *= alpha[r];
      zaccN[0] *= alpha[jjV];
      zaccN[1] *= alpha[jjV];
      return;
    }
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) {
      bm0 = fmaxf(bm0, __shfl_xor(bm0, m, 64));
      bm1 = fmaxf(bm1, __shfl_xor(bm1, m, 64));
    }
    const float n0 = fmaxf(mrun[0], bm0), n1 = fmaxf(mrun[1], bm1);
    const float r0 = n0 - shift, r1 = n1 - shift;
    const float al0 = __builtin_amdgcn_exp2f(mref[0] - r0), al1 = __builtin_amdgcn_exp2f(mref[1] - r1);
    mrun[0] = n0;
    mrun[1] = n1;
    mref[0] = r0;
    mref[1] = r1;
    lsum[0] *= al0;
    lsum[1] *= al1;
    // scale factors of all four heads, everywhere (heads 0,1 live in lanes 0..31)
    const float alpha[4] = {__shfl(al0, 0, 64), __shfl(al1, 0, 64), __shfl(al0, 32, 64), __shfl(al1, 32, 64)};
    if (VT) {  // lane (q4 < 2) holds heads 2 q4, 2 q4 + 1 in acc[nt][0], acc[nt][1]
      const float a0 = alpha[2 * (q4 & 1)], a1 = alpha[2 * (q4 & 1) + 1];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        acc[nt][0] *= a0;
        acc[nt][1] *= a1;
      }
      return;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nt][r] *= alpha[r];
    zacc *= alpha[jjV];
  };

  // p = 2^(logit - mref) of the super-block's first n blocks: summed into l and published
  // in LDS for the value steps (lane (hQ, nQ) holds heads 2hQ, 2hQ + 1 of token nQ; a
  // value lane needs 8 tokens of one head)
  auto publish_p = [&](const float (&lg)[NBS][2], int n, auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    // A single wavefront owns this LDS: its DS instructions complete in program order,
    // so reads of the previous super-block's p are done before these writes land, and
    // the exchange needs no barrier, only compiler fences.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < NBS; ++j) {
      if (!GUARD || j < n) {
        if constexpr (NARROW) {  // head qS, tokens nS and 16 + nS
          const float p0 = __builtin_amdgcn_exp2f(lg[j][0] - mref[0]);
          const float p1 = __builtin_amdgcn_exp2f(lg[j][1] - mref[0]);
          lsum[0] += p0 + p1;
          p_s[j][qS][nS] = p0;
          p_s[j][qS][16 + nS] = p1;
        } else {
          const float p0 = __builtin_amdgcn_exp2f(lg[j][0] - mref[0]);
          const float p1 = __builtin_amdgcn_exp2f(lg[j][1] - mref[1]);
          lsum[0] += p0;
          lsum[1] += p1;
          p_s[j][2 * hQ][nQ] = p0;
          p_s[j][2 * hQ + 1][nQ] = p1;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // values of block j, narrow groups: the lane forms the W digits of head jjV for its two
  // tokens in each group and publishes them; it then reads back its A row (digit dV, group
  // gVc, head jjV) for tokens 8 q4 .. 8 q4 + 7 and runs one MFMA per N-tile
  auto pv_narrow = [&](const VBlock<BITS, true, NG>& vb, int j, int t0, auto tail, bool check_big) -> bool {
    constexpr bool TAIL = decltype(tail)::value;
    if (check_big) {
      _Float16 smax = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 2; ++e) smax = __builtin_fmaxf16(smax, f16_lo(vb.vm[g][e]));
      if (__any(smax >= static_cast<_Float16>(128.0f))) return false;
    }
    typedef float floatx2 __attribute__((ext_vector_type(2)));
    const floatx2 pp = *reinterpret_cast<const floatx2*>(&p_s[j][jjV][8 * q4 + 2 * i4]);
    // the previous block's reads of w_s are issued before these writes (one wavefront: its
    // DS instructions complete in program order), so compiler fences suffice
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float w[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        w[e] = __builtin_fmaf(lo_f16(vb.vm[g][e]), pp[e], 0.f);
        float zp = hi_f16(vb.vm[g][e]);
        if (TAIL && t0 + 8 * q4 + 2 * i4 + e >= end) {  // slots past the end may hold anything
          w[e] = 0.f;
          zp = 0.f;
        }
        zaccN[g] = __builtin_fmaf(zp, pp[e], zaccN[g]);
      }
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w[0], w[1]));
      const float lo0 = __builtin_fmaf(lo_f16(hi), neg1, w[0]);
      const float lo1 = __builtin_fmaf(hi_f16(hi), neg1, w[1]);
      w_s[0][g][jjV][4 * q4 + i4] = hi;
      w_s[1][g][jjV][4 * q4 + i4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo0, lo1));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const half8 A = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(&w_s[dV][gVc][jjV][4 * q4]));
    __builtin_amdgcn_s_setprio(1);  // the matrix-core cluster (see qk)
#pragma unroll
    for (int nt = 0; nt < 8; nt += 2) {
      __builtin_amdgcn_sched_barrier(0);
      const half8 bv0 = unpack_v<BITS>(vb.vc, nt);
      const half8 bv1 = unpack_v<BITS>(vb.vc, nt + 1);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bv0, acc[nt], 0, 0, 0);
      acc[nt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bv1, acc[nt + 1], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    return true;
  };

  // values of block j of the super-block; false if a value scale is too large for the
  // f16 weights at this shift (nothing is accumulated then)
  auto pv_wide = [&](const VBlock<BITS>& vb, int j, int t0, auto tail, bool check_big) -> bool {
    constexpr bool TAIL = decltype(tail)::value;
    if (check_big) {
      _Float16 smax = 0;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) smax = __builtin_fmaxf16(smax, f16_lo(vb.vm[kk]));
      if (__any(smax >= static_cast<_Float16>(128.0f))) return false;
    }
    float pv[8];
    {
      const floatx4* src = reinterpret_cast<const floatx4*>(&p_s[j][jjV][8 * q4]);
      const floatx4 x0 = src[0], x1 = src[1];
      pv[0] = x0[0]; pv[1] = x0[1]; pv[2] = x0[2]; pv[3] = x0[3];
      pv[4] = x1[0]; pv[5] = x1[1]; pv[6] = x1[2]; pv[7] = x1[3];
    }
    // w = p * scale (masked tokens have p = 0 exactly); w = hi + lo with hi = w's top 11
    // significant bits (exact in f16) and lo the exact remainder, rounded toward zero to f16
    uint32_t ahi[4], alo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float w[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kk = 2 * k + e;
        w[e] = __builtin_fmaf(lo_f16(vb.vm[kk]), pv[kk], 0.f);
        float zp = hi_f16(vb.vm[kk]);
        if (TAIL && t0 + 8 * q4 + kk >= end) {  // slots past the end may hold anything
          w[e] = 0.f;
          zp = 0.f;
        }
        zacc = __builtin_fmaf(zp, pv[kk], zacc);
      }
      // hi = w rounded toward zero to f16 (w's top 11 significant bits), lo = the exact
      // remainder w - hi, rounded toward zero to f16
      ahi[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w[0], w[1]));
      const float lo0 = __builtin_fmaf(lo_f16(ahi[k]), neg1, w[0]);
      const float lo1 = __builtin_fmaf(hi_f16(ahi[k]), neg1, w[1]);
      alo[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo0, lo1));
    }
    const half8 Ahi = as_half8(ahi[0], ahi[1], ahi[2], ahi[3]);
    const half8 Alo = as_half8(alo[0], alo[1], alo[2], alo[3]);
    __builtin_amdgcn_s_setprio(1);  // the matrix-core cluster (see qk)
#pragma unroll
    for (int nt = 0; nt < 8; nt += 2) {
      // two N-tiles at a time: the hi and lo products of one tile are not back to back
      __builtin_amdgcn_sched_barrier(0);
      const half8 bv0 = unpack_v<BITS>(vb.vc, nt);
      const half8 bv1 = unpack_v<BITS>(vb.vc, nt + 1);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, bv0, acc[nt], 0, 0, 0);
      acc[nt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, bv1, acc[nt + 1], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, bv0, acc[nt], 0, 0, 0);
      acc[nt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, bv1, acc[nt + 1], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    return true;
  };
  auto pv = [&](const VB& vb, int j, int t0, auto tail, bool check_big) -> bool {
    if constexpr (NARROW)
      return pv_narrow(vb, j, t0, tail, check_big);
    else
      return pv_wide(vb, j, t0, tail, check_big);
  };

  // values of block j with value token groups: A rows 2 jj + digit hold the f16 hi / lo
  // parts of head jj's p (rows >= 2R zero), one MFMA per N-tile; lane (q4 < 2, r16) then
  // folds rows 4 q4 .. 4 q4 + 3 (heads 2 q4, 2 q4 + 1, both digits) of channel
  // pv_channel(nt, r16) with that channel's scale and zero
  auto pv_vt = [&](const auto& vb, int j) {  // generic: instantiated only where called (VT)
    const int jjA = r16 >> 1;
    float pv[8];
    {
      const floatx4* src = reinterpret_cast<const floatx4*>(&p_s[j][jjA < R ? jjA : 0][8 * q4]);
      const floatx4 x0 = src[0], x1 = src[1];
      pv[0] = x0[0]; pv[1] = x0[1]; pv[2] = x0[2]; pv[3] = x0[3];
      pv[4] = x1[0]; pv[5] = x1[1]; pv[6] = x1[2]; pv[7] = x1[3];
    }
    uint32_t ad[4];
    float ps = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ps += pv[2 * k] + pv[2 * k + 1];
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[2 * k], pv[2 * k + 1]));
      const float lo0 = __builtin_fmaf(lo_f16(hi), neg1, pv[2 * k]);
      const float lo1 = __builtin_fmaf(hi_f16(hi), neg1, pv[2 * k + 1]);
      const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo0, lo1));
      ad[k] = jjA < R ? ((r16 & 1) ? lo : hi) : 0u;
    }
    const half8 A = as_half8(ad[0], ad[1], ad[2], ad[3]);
    // sum of the block's p per head: the lane's 8 tokens, then the 4 token quarters
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    const float P0 = __shfl(ps, 4 * (q4 & 1), 64), P1 = __shfl(ps, 4 * (q4 & 1) + 2, 64);
    __builtin_amdgcn_s_setprio(1);  // the matrix-core cluster (see qk)
#pragma unroll
    for (int nt = 0; nt < 8; nt += 2) {
      __builtin_amdgcn_sched_barrier(0);
      // the products start from zeros that depend on the running sums: each block's MFMAs
      // stay behind the previous block's fold (from constant zeros the scheduler hoists
      // every block's products and holds them all, past 400 registers)
      const floatx4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, unpack_v<BITS>(vb.vc, nt), acc[nt] * 0.0f, 0, 0, 0);
      const floatx4 c1 =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(A, unpack_v<BITS>(vb.vc, nt + 1), acc[nt + 1] * 0.0f, 0, 0, 0);
      const float s0 = lo_f16(vb.vm[nt]), z0 = hi_f16(vb.vm[nt]);
      const float s1 = lo_f16(vb.vm[nt + 1]), z1 = hi_f16(vb.vm[nt + 1]);
      acc[nt][0] = __builtin_fmaf(s0, c0[0] + c0[1], __builtin_fmaf(z0, P0, acc[nt][0]));
      acc[nt][1] = __builtin_fmaf(s0, c0[2] + c0[3], __builtin_fmaf(z0, P1, acc[nt][1]));
      acc[nt + 1][0] = __builtin_fmaf(s1, c1[0] + c1[1], __builtin_fmaf(z1, P0, acc[nt + 1][0]));
      acc[nt + 1][1] = __builtin_fmaf(s1, c1[2] + c1[3], __builtin_fmaf(z1, P1, acc[nt + 1][1]));
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // The partition in super-blocks of NBS blocks, each in two passes: the scores of all
  // its blocks (logits stay in registers), one max update, then the values. Loads run
  // two blocks ahead through the sequence K(0..NBS-1), V(0..NBS-1), K of the next
  // super-block, ... into three rotating buffers per kind (static slots: the super-block
  // body is fully unrolled). Super-blocks of NBS full blocks run without guards or
  // masks; the rest of the partition (fewer than NBS full blocks and a partial block)
  // forms one last, guarded and masked super-block. Loads past the partition's last
  // block: the last super-block (LASTC when unguarded, any guarded one) prefetches no
  // keys, and a guarded one loads none of its blocks at or past n. The one left: when the
  // guarded super-block holds fewer than PF blocks, the key prefetches before it read up
  // to PF - 1 blocks past the end. (A run-time test on the prefetch instead of a second
  // unguarded body splits the body into basic blocks and costs the issue-bound INT2
  // kernels 4 %.)
  auto super_block = [&](int base, int n, auto guard, auto lastc, bool check_big) -> bool {
    constexpr bool GUARD = decltype(guard)::value;
    constexpr bool LASTC = decltype(lastc)::value;
    float lg[NBS][2];
    float bm0 = -INFINITY, bm1 = -INFINITY;
#pragma unroll
    for (int j = 0; j < NBS; ++j) {
      if (j + PF < NBS)
        kb[(j + PF) % (PF + 1)] = (!GUARD || j + PF < n) ? load_k(kcur, std::bool_constant<!GUARD>{}) : KBT{};
      else
        vb[(j + PF - NBS) % (PF + 1)] = (!GUARD || j + PF - NBS < n) ? load_v(vcur, std::bool_constant<!GUARD>{}) : VB{};
      if (!GUARD || j < n) {
        qk(kb[j % (PF + 1)], start + 32 * (base + j), guard, lg[j]);
        bm0 = fmaxf(bm0, lg[j][0]);
        bm1 = fmaxf(bm1, lg[j][1]);
      }
    }
    advance_max(bm0, bm1, check_big ? 8.0f : 0.0f);
    publish_p(lg, n, guard);
    if constexpr (SBT && !GUARD && !LASTC) {  // the next super-block's tiles
      if (!one_page) sb_ids(walk);
    }
#pragma unroll
    for (int j = 0; j < NBS; ++j) {
      if (j + PF < NBS)
        vb[(j + PF) % (PF + 1)] = (!GUARD || j + PF < n) ? load_v(vcur, std::bool_constant<!GUARD>{}) : VB{};
      else if constexpr (!GUARD && !LASTC)  // the next super-block's keys
        kb[(j + PF - NBS) % (PF + 1)] = load_k(kcur, std::false_type{});
      if (!GUARD || j < n) {
        if constexpr (VT)
          pv_vt(vb[j % (PF + 1)], j);
        else if (!pv(vb[j % (PF + 1)], j, start + 32 * (base + j), guard, check_big))
          return false;
      }
    }
    return true;
  };
  // p carries 2^8 (check_big) unless a value scale >= 128 shows up: the partition is
  // then recomputed with p unscaled
  for (int attempt = 0; attempt < 2; ++attempt) {
    const bool check_big = attempt == 0;
    mrun[0] = mrun[1] = -INFINITY;
    mref[0] = mref[1] = -INFINITY;
    lsum[0] = lsum[1] = 0.f;
    zacc = 0.f;
    zaccN[0] = zaccN[1] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (attempt > 0) {
      kcur = cur0;
      vcur = cur0;
      if constexpr (SBT) {
        walk = walk0;
        if (!one_page) sb_ids(walk);
      }
#pragma unroll
      for (int j = 0; j < PF; ++j) kb[j] = j < nblk ? load_k(kcur, std::false_type{}) : KBT{};
    }
    const int nsbf = nfull / NBS;
    const int rem = nblk - nsbf * NBS;
    bool ok = true;
    // (value token groups: no LASTC body, whose registers would cost them a wave per SIMD;
    // their last super-block prefetches PF key blocks past the end)
    const int nplain = nsbf - (rem == 0 && !VT ? 1 : 0);
    for (int sb = 0; sb < nplain && ok; ++sb)
      ok = super_block(sb * NBS, NBS, std::false_type{}, std::false_type{}, check_big);
    if constexpr (!VT) {
      if (ok && rem == 0 && nsbf > 0)
        ok = super_block((nsbf - 1) * NBS, NBS, std::false_type{}, std::true_type{}, check_big);
    }
    if (ok && rem > 0) ok = super_block(nsbf * NBS, rem, std::true_type{}, std::false_type{}, check_big);
    if (ok) break;
  }

  // ---- partials: o[jj][ch] = acc + Z[jj][g(ch)], m = mref, l ----
  if constexpr (NARROW) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) lsum[0] += __shfl_xor(lsum[0], m, 64);  // head qS's 16 lanes
  } else {
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) {
      lsum[0] += __shfl_xor(lsum[0], m, 64);
      lsum[1] += __shfl_xor(lsum[1], m, 64);
    }
  }
  zacc += __shfl_xor(zacc, 16, 64);
  zacc += __shfl_xor(zacc, 32, 64);  // every lane r16 now holds Z of row (jjV, gV)
  float* part = a.partials + slot * 130;
  const int64_t head_stride = static_cast<int64_t>(a.balanced ? a.unit_slots : a.num_splits) * 130;
  // lane (q4, r16) owns accumulator rows 4*q4 + r = (jj = r, g = q4) at column r16; the
  // rows of group q4 hold head jj's output for the channels of that group. Staged in LDS
  // so the workspace is written with 8-byte stores.
  if (VT) {
    if (q4 < 2) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int ch = pv_channel<BITS>(nt, r16);
        if (2 * q4 < R) o_s[2 * q4][ch] = acc[nt][0];
        if (2 * q4 + 1 < R) o_s[2 * q4 + 1][ch] = acc[nt][1];
      }
    }
  } else if (NARROW) {
    // lane (q4, r16) holds rows 4 q4 + r = (group q4 / 2, digit q4 % 2, head r): the digits
    // are summed across lanes q4 and q4 ^ 1. Z of (head r, group g): the sum of zaccN[g]
    // over the lanes of head r (after the reduction, lane r holds it)
    const int g = q4 >> 1;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int m = 4; m <= 32; m <<= 1) zaccN[gg] += __shfl_xor(zaccN[gg], m, 64);
    float zrow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float z0 = __shfl(zaccN[0], r, 64), z1 = __shfl(zaccN[1], r, 64);
      zrow[r] = (g == 1 && NG == 2) ? z1 : z0;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = pv_channel<BITS>(nt, r16);
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = acc[nt][r] + __shfl_xor(acc[nt][r], 16, 64);
      if ((q4 & 1) == 0 && ch / G == g) {
#pragma unroll
        for (int r = 0; r < R; ++r) o_s[r][ch] = o4[r] + zrow[r];
      }
    }
  } else {
    float zrow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) zrow[r] = __shfl(zacc, 4 * (q4 < NG ? q4 : 0) + r, 64);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = pv_channel<BITS>(nt, r16);
      if (ch / G == q4) {
#pragma unroll
        for (int r = 0; r < R; ++r) o_s[r][ch] = acc[nt][r] + zrow[r];
      }
    }
  }
  __syncthreads();
  {
    const int jo = lane >> 4, c8 = 8 * (lane & 15);
    if (jo < R) {
      float2* dst = reinterpret_cast<float2*>(part + jo * head_stride + c8);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = make_float2(o_s[jo][c8 + 2 * e], o_s[jo][c8 + 2 * e + 1]);
    }
  }
  if (NARROW) {
    if (nS == 0 && qS < R) {
      part[qS * head_stride + 128] = mref[0];
      part[qS * head_stride + 129] = lsum[0];
    }
  } else if (nQ == 0) {
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const int jj = 2 * hQ + j2;
      if (jj < R) {
        part[jj * head_stride + 128] = mref[j2];
        part[jj * head_stride + 129] = lsum[j2];
      }
    }
  }
}

}  // namespace

}  // namespace kvq
