// Decode attention over the high-precision windows: one partial per query head.
//
// InnerQ (Abstract): the attention-sink tokens and a window of recent tokens stay in
// high precision. Here they are bf16 rows in the original basis, so the query takes no
// rotation; its scale is the split kernels' (softmax scale * log2 e, exp2 domain), and
// the partial (o, m, l) is merged with the quantized partitions' by the combine kernel.
//
// One workgroup of 256 threads per (sequence, kv head). Rows are read by 16-lane
// groups, 8 channels (16 bytes) per lane: scores reduce across the group, the value
// sums across the 16 groups through LDS. Each wave turns one head's scores into
// probabilities on its own (max, exp2, sum).
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kWThreads = 256;
constexpr int kGroups = kWThreads / 16;

template <int R>
__global__ __launch_bounds__(kWThreads) void decode_window_kernel(DecodeArgs a, DevWindow w) {
  constexpr int kD = 128;
  const int hkv = a.c.hkv;
  const int hk = blockIdx.x % hkv;
  const int b = blockIdx.x / hkv;
  const int T = a.seq_lens[b];
  if (T <= 0) return;
  const int S = w.sink, RW = w.recent;
  // window tokens: sink 0..ns-1, then recent rbeg..T-1
  const int ns = min(S, T);
  const int rbeg = max(S, T - RW);
  const int n = ns + max(0, T - rbeg);  // 1 .. S + RW

  __shared__ float sc[R][kMaxWindow];
  __shared__ float red[kGroups][R][kD];
  __shared__ float stat[2][R];

  const int tid = threadIdx.x;
  const int lane16 = tid & 15, grp = tid >> 4;
  const int64_t rows = static_cast<int64_t>(b) * (S + RW);
  auto row_of = [&](int i) -> int64_t {  // window row of the i-th window token
    const int wr = i < ns ? i : S + (rbeg + (i - ns) - S) % RW;
    return ((rows + wr) * hkv + hk) * kD + 8 * lane16;
  };

  // the R query heads, channels 8 lane16 .. 8 lane16 + 7, scaled
  float q[R][8];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint4 raw =
        *reinterpret_cast<const uint4*>(a.q + (static_cast<int64_t>(b) * a.num_q_heads + hk * R + j) * kD + 8 * lane16);
    const float x[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                        bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) q[j][e] = x[e] * a.qscale;
  }

  // scores
  for (int i = grp; i < n; i += kGroups) {
    const uint4 raw = *reinterpret_cast<const uint4*>(w.k + row_of(i));
    const float k[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                        bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = __builtin_fmaf(q[j][e], k[e], s);
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
      if (lane16 == 0) sc[j][i] = s;
    }
  }
  __syncthreads();

  // wave j: probabilities of head j, p = exp2(s - max), and their sum
  {
    const int j = tid >> 6, l64 = tid & 63;
    if (j < R) {
      float m = -INFINITY;
      for (int i = l64; i < n; i += 64) m = fmaxf(m, sc[j][i]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float l = 0.f;
      for (int i = l64; i < n; i += 64) {
        const float p = exp2f(sc[j][i] - m);
        sc[j][i] = p;
        l += p;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
      if (l64 == 0) {
        stat[0][j] = m;
        stat[1][j] = l;
      }
    }
  }
  __syncthreads();

  // p . v: group grp sums its tokens, then the groups are added through LDS
  float acc[R][8];
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  for (int i = grp; i < n; i += kGroups) {
    const uint4 raw = *reinterpret_cast<const uint4*>(w.v + row_of(i));
    const float v[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                        bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float p = sc[j][i];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = __builtin_fmaf(p, v[e], acc[j][e]);
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[grp][j][8 * lane16 + e] = acc[j][e];
  __syncthreads();

  for (int idx = tid; idx < R * kD; idx += kWThreads) {
    const int j = idx / kD, ch = idx % kD;
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) o += red[g][j][ch];
    float* part = a.partials +
                  ((static_cast<int64_t>(b) * a.num_q_heads + hk * R + j) * a.part_stride + a.num_splits) * (kD + 2);
    part[ch] = o;
    if (ch == 0) {
      part[kD] = stat[0][j];
      part[kD + 1] = stat[1][j];
    }
  }
}

}  // namespace

hipError_t launch_decode_window(const DecodeArgs& a, const DevWindow& w, const Geometry& g, hipStream_t stream) {
  if (w.sink + w.recent > kMaxWindow || w.recent < 1) return hipErrorInvalidValue;
  const int64_t units = static_cast<int64_t>(a.batch) * g.hkv;
  if (units > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(units)), block(kWThreads);
  switch (a.ratio) {
    case 1:
      hipLaunchKernelGGL((decode_window_kernel<1>), grid, block, 0, stream, a, w);
      break;
    case 2:
      hipLaunchKernelGGL((decode_window_kernel<2>), grid, block, 0, stream, a, w);
      break;
    case 4:
      hipLaunchKernelGGL((decode_window_kernel<4>), grid, block, 0, stream, a, w);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
