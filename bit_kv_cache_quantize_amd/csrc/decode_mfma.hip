// Split-K decode attention on the matrix cores: the kernel (decode_mfma.h) without
// query-channel pruning, for every supported (bits, group, GQA ratio); caches whose
// sequences may span several pages go to decode_paged.hip's instances.
#include "decode_mfma.h"

namespace kvq {

hipError_t launch_decode_split(const DecodeArgs& a, const Geometry& g, hipStream_t stream, hipEvent_t t0,
                               hipEvent_t t1) {
  // sequences that may span pages: the instance whose value loads reuse the key lookups
  if (g.page < a.max_len) return launch_decode_split_paged(a, g, stream, t0, t1);
  const int64_t units = split_units(a, g);
  if (units > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(units)), block(64);
#define KVQ_DM(B, GS, RR)                                                                              \
  if (g.bits == B && g.group == GS && a.ratio == RR) {                                                 \
    void* args[] = {const_cast<DecodeArgs*>(&a)};                                                 \
    return hipExtLaunchKernel(reinterpret_cast<const void*>(&decode_split_mfma_kernel<B, GS, RR, false, false>), grid, \
                              block, args, 0, stream, t0, t1, 0);                                       \
  }
#define KVQ_DM_R(B, GS) KVQ_DM(B, GS, 1) KVQ_DM(B, GS, 2) KVQ_DM(B, GS, 4)
  KVQ_DM_R(4, 32) KVQ_DM_R(4, 64) KVQ_DM_R(4, 128) KVQ_DM_R(2, 32) KVQ_DM_R(2, 64) KVQ_DM_R(2, 128)
#undef KVQ_DM_R
#undef KVQ_DM
  return hipErrorInvalidValue;
}

}  // namespace kvq
