// Decode attention over the high-precision windows: one partial per query head.
//
// InnerQ (Abstract): the attention-sink tokens and a window of recent tokens stay in
// high precision. Here they are bf16 rows in the original basis, so the query takes no
// rotation; its scale is the split kernels' (softmax scale * log2 e, exp2 domain), and
// the partial (o, m, l) goes to the window partials, merged with the quantized partitions'
// by the combine kernel.
//
// One workgroup of 256 threads per (sequence, kv head), 16 groups of 16 lanes, 8
// channels (16 bytes of a row) per lane. Group g takes window tokens g, g + 16, ...,
// kNB at a time: the K and V rows of all kNB tokens are loaded together, then the
// scores (reduced across the group's lanes) update the group's online softmax. The 16
// groups' (m, l, o) are merged through LDS at the end.
#include <type_traits>

#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kWThreads = 256;
constexpr int kGroups = kWThreads / 16;
constexpr int kNB = 8;  // tokens per group per round

// Sum over the 16 lanes of a row, in every lane: DPP quad swaps (lane ^ 1, lane ^ 2), then
// the half-row mirror (lane i <-> 7 - i) and the row mirror (i <-> 15 - i); each step adds
// a partner holding a disjoint partial sum.
__device__ __forceinline__ float dpp_sum16(float x) {
  auto step = [](float v, auto ctrl) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, true);
    return v + __int_as_float(y);
  };
  x = step(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  x = step(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  x = step(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  x = step(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

__device__ __forceinline__ void bf16x8(const uint4 raw, float (&x)[8]) {
  x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x); x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
  x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z); x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
}

template <int R>
__global__ __launch_bounds__(kWThreads) void decode_window_kernel(DecodeArgs a, DevWindow w) {
  constexpr int kD = 128;
  const int hkv = a.c.hkv;
  const int hk = blockIdx.x % hkv;
  const int b = blockIdx.x / hkv;
  const int T = a.seq_lens[b];
  if (T <= 0) return;
  const int S = w.sink, RW = w.recent;
  // window tokens: sink 0..ns-1, then recent rbeg..T-1 (a residual: the incomplete last
  // group rbeg..T-1, possibly empty)
  const int ns = w.residual ? 0 : min(S, T);
  const int rbeg = w.residual ? T - T % RW : max(S, T - RW);
  const int n = ns + max(0, T - rbeg);  // 1 .. S + RW; 0 for an empty residual
  if (n == 0) {  // an empty partial: m = -inf, l = 0, o = 0
    for (int idx = threadIdx.x; idx < R * (kD + 2); idx += kWThreads) {
      const int j = idx / (kD + 2), e = idx % (kD + 2);
      a.win_partials[(static_cast<int64_t>(b) * a.num_q_heads + hk * R + j) * (kD + 2) + e] = e == kD ? -INFINITY : 0.f;
    }
    return;
  }

  __shared__ float red_o[kGroups][R][kD];
  __shared__ float red_ml[kGroups][R][2];

  const int tid = threadIdx.x;
  const int lane16 = tid & 15, grp = tid >> 4;
  const int64_t rows = static_cast<int64_t>(b) * (S + RW);
  // window row of every window token, computed once (the ring index is a modulo)
  __shared__ uint16_t wrow_s[kMaxWindow];
  for (int i = tid; i < n; i += kWThreads) wrow_s[i] = static_cast<uint16_t>(i < ns ? i : S + (rbeg + (i - ns) - S) % RW);
  __syncthreads();
  auto row_of = [&](int i) -> int64_t {  // element offset of this lane's 8 channels
    return ((rows + wrow_s[i]) * hkv + hk) * kD + 8 * lane16;
  };

  // the R query heads, channels 8 lane16 .. 8 lane16 + 7, scaled
  float q[R][8];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint4 raw =
        *reinterpret_cast<const uint4*>(a.q + (static_cast<int64_t>(b) * a.num_q_heads + hk * R + j) * kD + 8 * lane16);
    bf16x8(raw, q[j]);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[j][e] *= a.qscale;
  }

  float m[R], l[R], acc[R][8];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }

  // rounds of NB tokens per group: kNB while at least kNB remain, then pairs, so that at
  // most one token slot per group is idle
  auto round = [&](int i0, auto nb) {
    constexpr int NB = decltype(nb)::value;
    uint4 kr[NB], vr[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {  // every load of the round in flight together
      const int i = i0 + kGroups * u;
      const int64_t off = row_of(i < n ? i : i0);
      kr[u] = *reinterpret_cast<const uint4*>(w.k + off);
      vr[u] = *reinterpret_cast<const uint4*>(w.v + off);
    }
    float s[R][NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      float k[8];
      bf16x8(kr[u], k);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = __builtin_fmaf(q[j][e], k[e], d);
        d = dpp_sum16(d);
        s[j][u] = (i0 + kGroups * u < n) ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float mn = m[j];
#pragma unroll
      for (int u = 0; u < NB; ++u) mn = fmaxf(mn, s[j][u]);  // finite: token i0 is valid
      const float alpha = exp2f(m[j] - mn);                   // 0 on the first round
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= alpha;
      m[j] = mn;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      float v[8];
      bf16x8(vr[u], v);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float p = exp2f(s[j][u] - m[j]);  // 0 for tokens past the end
        l[j] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = __builtin_fmaf(p, v[e], acc[j][e]);
      }
    }
  };
  int i0 = grp;
  for (; i0 + kGroups * (kNB - 1) < n; i0 += kGroups * kNB) round(i0, std::integral_constant<int, kNB>{});
  for (; i0 < n; i0 += kGroups * 2) round(i0, std::integral_constant<int, 2>{});

  // merge the groups (a group without tokens has m = -inf, l = 0, o = 0)
#pragma unroll
  for (int j = 0; j < R; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[grp][j][8 * lane16 + e] = acc[j][e];
    if (lane16 == 0) {
      red_ml[grp][j][0] = m[j];
      red_ml[grp][j][1] = l[j];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < R * kD; idx += kWThreads) {
    const int j = idx / kD, ch = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) M = fmaxf(M, red_ml[g][j][0]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const float f = exp2f(red_ml[g][j][0] - M);  // M is finite: group 0 holds window token 0
      o = __builtin_fmaf(red_o[g][j][ch], f, o);
      L = __builtin_fmaf(red_ml[g][j][1], f, L);
    }
    float* part = a.win_partials + (static_cast<int64_t>(b) * a.num_q_heads + hk * R + j) * (kD + 2);
    part[ch] = o;
    if (ch == 0) {
      part[kD] = M;
      part[kD + 1] = L;
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
