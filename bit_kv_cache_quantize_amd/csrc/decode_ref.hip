// Split-K decode attention, plain VALU formulation, and the split combine.
//
// SAW-INT4 (Abstract): attention runs directly over the paged low-bit cache.
// Dual-QK (Abstract): the query gets the keys' rotation so q.k is unchanged.
// The split-K / log-sum-exp combine structure is the standard flash-decoding
// arrangement; partials are (unnormalised o[d], running max m, running sum l) with
// logits in the exp2 domain (the query is pre-scaled by softmax_scale * log2 e).
//
// This kernel is the straightforward one: one workgroup per (sequence, kv head,
// partition), fp32 dequantization fma(code, scale, zero) per element, fp32 dot
// products, scores staged in LDS. It is kept as an independent GPU formulation that
// the tests compare the MFMA kernel against; the library's decode call uses the MFMA
// kernel for every supported configuration.
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kMaxSplit = 2048;  // tokens per partition this kernel stages in LDS

// Entry of channel ch among a value token group's 128 {scale, zero} entries (caches with
// value token groups): 8n + t for ch = 4(n + 16(t>>2)) + 2(t&1) + ((t>>1)&1) at INT4,
// 8n + (t>>1) + 4(t&1) at INT2; found here by searching the documented forward map.
__device__ __forceinline__ int vt_entry_ref(int bits, int ch) {
  for (int n = 0; n < 16; ++n)
    for (int t = 0; t < 8; ++t) {
      const int c = bits == 4 ? 4 * (n + 16 * (t >> 2)) + 2 * (t & 1) + ((t >> 1) & 1) : 8 * n + (t >> 1) + 4 * (t & 1);
      if (c == ch) return 8 * n + t;
    }
  return 0;
}
constexpr int kThreads = 256;

template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void decode_split_reference_kernel(DecodeArgs a) {
  constexpr int kD = 128;
  constexpr int kMask = (1 << BITS) - 1;
  const DevCache& c = a.c;
  const int unit = blockIdx.x;
  const int split = unit % a.num_splits;
  const int bh = unit / a.num_splits;
  const int h = bh % c.hkv;
  const int b = bh / c.hkv;
  const int T = a.seq_lens[b];
  // the span this kernel covers ends here (with a residual: at the last whole group)
  const int qend = covered_end(a, min(T, a.max_len));  // longer sequences: taken as max_len long
  const int start = a.tok_begin + split * a.split_len;
  if (start >= qend) return;
  const int end = min(qend, start + a.split_len);
  const int n = end - start;
  const int R = a.ratio;
  const int tid = threadIdx.x;

  __shared__ float qs[4][kD];
  __shared__ float sc[4][kMaxSplit];
  __shared__ float red[4][kThreads];
  __shared__ float stat[2][4];

  for (int idx = tid; idx < R * kD; idx += kThreads) {
    const int j = idx / kD, i = idx % kD;
    const uint16_t bits = a.q[(static_cast<int64_t>(b) * a.num_q_heads + h * R + j) * kD + i];
    qs[j][i] = __uint_as_float(static_cast<uint32_t>(bits) << 16);
  }
  __syncthreads();
  if (a.hblock > 0) {
    for (int s = 1; s < a.hblock; s <<= 1) {
      for (int idx = tid; idx < R * (kD / 2); idx += kThreads) {
        const int j = idx / (kD / 2), p = idx % (kD / 2);
        const int i = (p / s) * 2 * s + (p % s);
        const float x0 = qs[j][i], x1 = qs[j][i + s];
        qs[j][i] = x0 + x1;
        qs[j][i + s] = x0 - x1;
      }
      __syncthreads();
    }
  }
  for (int idx = tid; idx < R * kD; idx += kThreads) {
    const int j = idx / kD, i = idx % kD;
    qs[j][i] = qs[j][i] * (a.hblock > 0 ? a.rot_c : 1.0f) * a.qscale;
  }
  __syncthreads();

  // scores: one token per thread
  for (int t = start + tid; t < end; t += kThreads) {
    const int64_t page = a.block_table[static_cast<int64_t>(b) * a.max_pages + t / c.page];
    const int off = t % c.page;
    const int64_t u = page * c.hkv + h;
    const int64_t tile_row = u * c.page + (off & ~15);
    const uint32_t* meta = c.km + (u * c.page + off) * c.ngroups;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < kD; ++i) {
      const uint32_t byte = c.kc[k_code_byte(tile_row, c.row_bytes, off & 15, i * BITS / 8)];
      const uint32_t code = (byte >> ((i * BITS) % 8)) & kMask;
      const uint32_t m = meta[i / G];
      const float khat = __builtin_fmaf(static_cast<float>(code), f16_bits_to_float(m & 0xFFFFu),
                                        f16_bits_to_float(m >> 16));
      for (int j = 0; j < R; ++j) acc[j] = __builtin_fmaf(qs[j][i], khat, acc[j]);
    }
    for (int j = 0; j < R; ++j) sc[j][t - start] = acc[j];
  }
  __syncthreads();

  // max and sum per head
  for (int j = 0; j < R; ++j) {
    float m = -INFINITY;
    for (int t = tid; t < n; t += kThreads) m = fmaxf(m, sc[j][t]);
    red[j][tid] = m;
  }
  __syncthreads();
  if (tid < R) {
    float m = -INFINITY;
    for (int k = 0; k < kThreads; ++k) m = fmaxf(m, red[tid][k]);
    stat[0][tid] = m;
  }
  __syncthreads();
  for (int j = 0; j < R; ++j) {
    float l = 0.f;
    for (int t = tid; t < n; t += kThreads) {
      const float p = exp2f(sc[j][t] - stat[0][j]);
      sc[j][t] = p;
      l += p;
    }
    red[j][tid] = l;
  }
  __syncthreads();
  if (tid < R) {
    float l = 0.f;
    for (int k = 0; k < kThreads; ++k) l += red[tid][k];
    stat[1][tid] = l;
  }
  __syncthreads();

  // p . vhat: each thread owns (head, channel) pairs
  for (int idx = tid; idx < R * kD; idx += kThreads) {
    const int j = idx / kD, i = idx % kD;
    const int byte = i * BITS / 8;          // byte of the packed row holding channel i
    const int sh = (i * BITS) % 8;
    const int vte = c.v_grouping ? vt_entry_ref(BITS, i) : 0;  // channel i's entry in a token group
    float o = 0.f;
    for (int t = start; t < end; ++t) {
      const int64_t page = a.block_table[static_cast<int64_t>(b) * a.max_pages + t / c.page];
      const int off = t % c.page;
      const int64_t u = page * c.hkv + h;
      const int64_t tile_row = u * c.page + (off & ~15);
      const uint32_t code = (static_cast<uint32_t>(c.vc[v_code_byte(tile_row, c.row_bytes, off & 15, byte)]) >> sh) & kMask;
      const uint32_t m = c.v_grouping ? c.vm[((u * c.page + off) / G) * 128 + vte]
                                      : c.vm[v_meta_entry(tile_row >> 4, c.ngroups, i / G, off & 15)];
      const float vhat = __builtin_fmaf(static_cast<float>(code), f16_bits_to_float(m & 0xFFFFu),
                                        f16_bits_to_float(m >> 16));
      o = __builtin_fmaf(sc[j][t - start], vhat, o);
    }
    float* part = a.partials + ((static_cast<int64_t>(b) * a.num_q_heads + h * R + j) * a.num_splits + split) * (kD + 2);
    part[i] = o;
    if (i == 0) {
      part[kD] = stat[0][j];
      part[kD + 1] = stat[1][j];
    }
  }
}

// Log-sum-exp merge of the partials of one (sequence, query head), or of CW of its 128
// channels (the grid then holds 128 / CW workgroups per pair). The workgroup has CW * NGRP
// threads: group gp (threads CW gp .. CW gp + CW - 1, thread = channel) merges partials gp,
// gp + NGRP, ... 16 at a time (one pass, every load of a chunk issued together: the
// running reference M moves up chunk by chunk and rescales (L, o) like the online softmax
// inside a partition); the groups' (M, L, o) are then merged through LDS. Many partials
// take many groups of fewer channels, so the loads spread over more CUs in one pass.
// The partials present are the split kernel's partitions that hold tokens of the covered
// span (fixed partitions: slots 0.. of the sequence's row; balanced: the sequence's units,
// from the table the split kernel wrote), then (with windows) the window partial.
template <int NGRP, int CW>
__global__ __launch_bounds__(CW * NGRP) void combine_kernel(DecodeArgs a) {
  constexpr int kD = 128;
  constexpr int kChunk = 16;
  constexpr int kParts = kD / CW;
  static_assert(CW * NGRP >= 64 && CW * NGRP <= 1024, "one to sixteen wavefronts");
  __shared__ float o_s[NGRP][CW];
  __shared__ float ml_s[NGRP][2];
  const int bj = blockIdx.x / kParts;
  const int b = bj / a.num_q_heads, j = bj % a.num_q_heads;
  const int gp = threadIdx.x / CW;
  const int i = (blockIdx.x % kParts) * CW + threadIdx.x % CW;  // channel
  const int T = a.seq_lens[b];
  // the split kernel's table entry (in bounds for every b), loaded alongside T; used only
  // for a sequence with tokens to cover, whose entry this call's split kernel wrote
  const int2 plan = a.balanced ? a.seq_plan[b] : make_int2(0, 0);
  if (T <= 0) {
    if (gp == 0) a.out[static_cast<int64_t>(bj) * kD + i] = 0.f;
    return;
  }
  const int span = covered_span(a, min(T, a.max_len));  // as the split kernels take it
  const float* base;
  int nq;
  if (a.balanced) {
    // clamped to the grid's units, so seq_lens above max_seq_len cannot read outside it
    int first = 0;
    nq = 0;
    if (span > 0) {
      first = min(max(plan.x, 0), a.unit_slots);
      nq = max(0, min(plan.y, a.unit_slots - first));
    }
    base = a.partials + (static_cast<int64_t>(j) * a.unit_slots + first) * (kD + 2);
  } else {
    nq = min(a.num_splits, (span + a.split_len - 1) / a.split_len);
    base = a.partials + static_cast<int64_t>(bj) * a.num_splits * (kD + 2);
  }
  const int ns = nq + a.window;  // >= 1: a sequence with T > 0 has a split or window token
  const float* win = a.window ? a.win_partials + static_cast<int64_t>(bj) * (kD + 2) : base;
  float M = -INFINITY, L = 0.f, o = 0.f;
  for (int s0 = gp; s0 < ns; s0 += kChunk * NGRP) {
    float m[kChunk], l[kChunk], v[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const int idx = s0 + k * NGRP;
      const bool ok = idx < ns;
      const float* p = idx < nq ? base + idx * (kD + 2) : win;
      m[k] = ok ? p[kD] : -INFINITY;
      l[k] = ok ? p[kD + 1] : 0.f;
      v[k] = ok ? p[i] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) Mn = fmaxf(Mn, m[k]);
    if (Mn == -INFINITY) continue;  // only empty partials so far (an empty window residual)
    const float r = exp2f(M - Mn);  // 0 on the first chunk (M = -inf), 1 when M holds
    L *= r;
    o *= r;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float w = exp2f(m[k] - Mn);  // 0 for padding (m = -inf)
      L = __builtin_fmaf(l[k], w, L);
      o = __builtin_fmaf(v[k], w, o);
    }
    M = Mn;
  }
  if (NGRP == 1) {
    a.out[static_cast<int64_t>(bj) * kD + i] = o / L;
    return;
  }
  o_s[gp][threadIdx.x % CW] = o;
  if (threadIdx.x % CW == 0) {
    ml_s[gp][0] = M;
    ml_s[gp][1] = L;
  }
  __syncthreads();
  if (gp == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < NGRP; ++g) Mt = fmaxf(Mt, ml_s[g][0]);
    float Lt = 0.f, ot = 0.f;
#pragma unroll
    for (int g = 0; g < NGRP; ++g) {
      const float w = exp2f(ml_s[g][0] - Mt);  // 0 for a group without partials
      Lt = __builtin_fmaf(ml_s[g][1], w, Lt);
      ot = __builtin_fmaf(o_s[g][threadIdx.x], w, ot);
    }
    a.out[static_cast<int64_t>(bj) * kD + i] = ot / Lt;
  }
}

}  // namespace

hipError_t launch_decode_split_reference(const DecodeArgs& a, const Geometry& g, hipStream_t stream) {
  if (a.split_len > kMaxSplit) return hipErrorInvalidValue;
  const int64_t units = static_cast<int64_t>(a.batch) * g.hkv * a.num_splits;
  if (units > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(units)), block(kThreads);
#define KVQ_DR(B, GS)                                                                                  \
  if (g.bits == B && g.group == GS) {                                                                  \
    hipLaunchKernelGGL((decode_split_reference_kernel<B, GS>), grid, block, 0, stream, a);            \
    return hipGetLastError();                                                                          \
  }
  KVQ_DR(4, 32) KVQ_DR(4, 64) KVQ_DR(4, 128) KVQ_DR(2, 32) KVQ_DR(2, 64) KVQ_DR(2, 128)
#undef KVQ_DR
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const DecodeArgs& a, const Geometry& g, hipStream_t stream) {
  (void)g;
  // One group of threads per up to 16 partials, each thread one channel; a pair's partials
  // beyond 128 are spread over 32 groups of 32 channels (four workgroups per pair), so
  // long sequences in many partitions merge in one pass over more CUs. Balanced plans are
  // sized for max_seq_len-long sequences (longer partition lists of a ragged batch take
  // more passes).
  const int parts = a.num_splits + a.window;
  const unsigned pairs = static_cast<unsigned>(a.batch * a.num_q_heads);
#define KVQ_CB(NG, CW)                                                                          \
  {                                                                                             \
    hipLaunchKernelGGL((combine_kernel<NG, CW>), dim3(pairs * (128 / CW)), dim3(NG * CW), 0, stream, a); \
    return hipGetLastError();                                                                   \
  }
  if (parts > 128) KVQ_CB(32, 32)
  if (parts > 64) KVQ_CB(8, 128)
  if (parts > 32) KVQ_CB(4, 128)
  if (parts > 16) KVQ_CB(2, 128)
  KVQ_CB(1, 128)
#undef KVQ_CB
}

}  // namespace kvq
