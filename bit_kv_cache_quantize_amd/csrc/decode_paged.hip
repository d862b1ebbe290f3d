// Split-K decode attention on the matrix cores for caches whose sequences span several
// pages: the kernel (decode_mfma.h) with its PAGED form, which looks up the tiles of a
// whole super-block at once into an LDS table, for every supported (bits, group, GQA
// ratio).
#include "decode_mfma.h"

namespace kvq {

hipError_t launch_decode_split_paged(const DecodeArgs& a, const Geometry& g, hipStream_t stream, hipEvent_t t0,
                                     hipEvent_t t1) {
  const int64_t units = split_units(a, g);
  if (units > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(units)), block(64);
#define KVQ_DP(B, GS, RR)                                                                               \
  if (g.bits == B && g.group == GS && a.ratio == RR) {                                                  \
    void* args[] = {const_cast<DecodeArgs*>(&a)};                                                       \
    return hipExtLaunchKernel(                                                                          \
        reinterpret_cast<const void*>(&decode_split_mfma_kernel<B, GS, RR, false, false, true>), grid, \
        block, args, 0, stream, t0, t1, 0);                                                             \
  }
#define KVQ_DP_R(B, GS) KVQ_DP(B, GS, 1) KVQ_DP(B, GS, 2) KVQ_DP(B, GS, 4)
  KVQ_DP_R(4, 32) KVQ_DP_R(4, 64) KVQ_DP_R(4, 128) KVQ_DP_R(2, 32) KVQ_DP_R(2, 64) KVQ_DP_R(2, 128)
#undef KVQ_DP_R
#undef KVQ_DP
  return hipErrorInvalidValue;
}

}  // namespace kvq
