// Split-K decode attention on the matrix cores with query-channel pruning of key reads:
// the kernel of decode_mfma.h with PRUNE set, for every supported (bits, group, GQA ratio).
#include "decode_mfma.h"

namespace kvq {

hipError_t launch_decode_split_pruned(const DecodeArgs& a, const Geometry& g, hipStream_t stream) {
  const int64_t units = split_units(a, g);
  if (units > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(units)), block(64);
#define KVQ_DM(B, GS, RR)                                                                              \
  if (g.bits == B && g.group == GS && a.ratio == RR) {                                                 \
    hipLaunchKernelGGL((decode_split_mfma_kernel<B, GS, RR, true, false>), grid, block, 0, stream, a);       \
    return hipGetLastError();                                                                          \
  }
#define KVQ_DM_R(B, GS) KVQ_DM(B, GS, 1) KVQ_DM(B, GS, 2) KVQ_DM(B, GS, 4)
  KVQ_DM_R(4, 32) KVQ_DM_R(4, 64) KVQ_DM_R(4, 128) KVQ_DM_R(2, 32) KVQ_DM_R(2, 64) KVQ_DM_R(2, 128)
#undef KVQ_DM_R
#undef KVQ_DM
  return hipErrorInvalidValue;
}

}  // namespace kvq
