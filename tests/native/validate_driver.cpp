// The host-side checks and sizing of the kvq C ABI (kvq_validate.cpp), built on its own
// with the address and undefined-behaviour sanitizers: every documented status of a
// malformed description, the closed forms of the plane and workspace sizes, and a sweep
// of extreme sizes (huge page pools, heads, batches and context lengths) in which no size
// may wrap and no signed arithmetic may overflow. Prints "ok <cases>" and exits 0 when
// every expectation holds; a sanitizer finding aborts the run.
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../bit_kv_cache_quantize_amd/csrc/kvq_validate.h"

using namespace kvq;

static int g_fail = 0;
static long g_cases = 0;

#define EXPECT(cond)                                                           \
  do {                                                                         \
    ++g_cases;                                                                 \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);             \
      ++g_fail;                                                                \
    }                                                                          \
  } while (0)

static char g_planes[4][64] __attribute__((aligned(16)));

static kvq_cache desc(int d = 128, int hkv = 8, int bits = 4, int G = 32, int hb = 128, int P = 16,
                      int64_t pages = 64, int mode = 0, int vg = 0) {
  kvq_cache c;
  c.head_dim = d;
  c.num_kv_heads = hkv;
  c.bits = bits;
  c.group_size = G;
  c.hadamard_block = hb;
  c.page_size = P;
  c.num_pages = pages;
  c.k_codes = g_planes[0];
  c.k_meta = g_planes[1];
  c.v_codes = g_planes[2];
  c.v_meta = g_planes[3];
  c.quant_mode = mode;
  c.v_grouping = vg;
  return c;
}

// The statuses the header documents for malformed or unsupported descriptions.
static void documented_statuses() {
  struct Case {
    kvq_cache c;
    kvq_status want;
  };
  std::vector<Case> cases = {
      {desc(), KVQ_OK},
      {desc(0), KVQ_ERR_INVALID},
      {desc(128, 0), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, 128, 16, 0), KVQ_ERR_INVALID},
      {desc(128, 8, 3), KVQ_ERR_UNSUPPORTED},
      {desc(128, 8, 0), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 48), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 16), KVQ_ERR_UNSUPPORTED},
      {desc(128, 8, 4, 32, 96), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, -1), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, 256), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, 128, 0), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, 128, 24), KVQ_ERR_INVALID},
      {desc(64, 8, 4, 32, 64), KVQ_ERR_UNSUPPORTED},
      {desc(128, 8, 4, 32, 128, 16, 64, 2), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, 128, 16, 64, 0, 2), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, 128, 16, 64, 0, 1), KVQ_ERR_INVALID},
      {desc(128, 8, 4, 32, 128, 32, 64, 0, 1), KVQ_OK},
      {desc(128, 8, 4, 32, 128, 16, (INT64_C(1) << 29) - 1), KVQ_OK},
      {desc(128, 8, 4, 32, 128, 16, INT64_C(1) << 29), KVQ_ERR_UNSUPPORTED},  // pages * Hkv = 2^32
      {desc(128, 8, 4, 32, 128, 16, INT64_MAX), KVQ_ERR_UNSUPPORTED},
      {desc(1 << 20, 8, 4, 32, 0), KVQ_ERR_UNSUPPORTED},
  };
  for (const Case& k : cases) {
    Geometry g;
    EXPECT(check_cache(&k.c, true, &g) == k.want);
  }
  kvq_cache c = desc();
  c.k_codes = nullptr;
  EXPECT(check_cache(&c, true, nullptr) == KVQ_ERR_INVALID);
  EXPECT(check_cache(&c, false, nullptr) == KVQ_OK);
  c = desc();
  c.v_meta = g_planes[3] + 4;
  EXPECT(check_cache(&c, true, nullptr) == KVQ_ERR_INVALID);
  EXPECT(check_cache(nullptr, false, nullptr) == KVQ_ERR_INVALID);

  // decode sizes
  EXPECT(check_decode_sizes(2, 32, 1000, 0) == KVQ_OK);
  EXPECT(check_decode_sizes(-1, 32, 1000, 0) == KVQ_ERR_INVALID);
  EXPECT(check_decode_sizes(2, 0, 1000, 0) == KVQ_ERR_INVALID);
  EXPECT(check_decode_sizes(2, 32, -5, 0) == KVQ_ERR_INVALID);
  EXPECT(check_decode_sizes(2, 32, 1000, -1) == KVQ_ERR_INVALID);
  EXPECT(check_decode_sizes(2, 32, kMaxSeqLen, 0) == KVQ_OK);
  EXPECT(check_decode_sizes(2, 32, kMaxSeqLen + 1, 0) == KVQ_ERR_UNSUPPORTED);
  const kvq_cache ok = desc();
  const char* p = g_planes[0];
  EXPECT(check_decode(&ok, p, 2, 12, reinterpret_cast<const int32_t*>(p), 64, reinterpret_cast<const int32_t*>(p),
                      1000, 0, p, reinterpret_cast<const float*>(p), nullptr) == KVQ_ERR_INVALID);
  EXPECT(check_decode(&ok, p, 2, 64, reinterpret_cast<const int32_t*>(p), 64, reinterpret_cast<const int32_t*>(p),
                      1000, 0, p, reinterpret_cast<const float*>(p), nullptr) == KVQ_ERR_UNSUPPORTED);
  EXPECT(check_decode(&ok, p, 2, 32, reinterpret_cast<const int32_t*>(p), 10, reinterpret_cast<const int32_t*>(p),
                      1000, 0, p, reinterpret_cast<const float*>(p), nullptr) == KVQ_ERR_INVALID);
  EXPECT(check_decode(&ok, p + 2, 2, 32, reinterpret_cast<const int32_t*>(p), 64,
                      reinterpret_cast<const int32_t*>(p), 1000, 0, p, reinterpret_cast<const float*>(p),
                      nullptr) == KVQ_ERR_INVALID);
  EXPECT(check_decode(&ok, p, 2, 32, reinterpret_cast<const int32_t*>(p), 64, reinterpret_cast<const int32_t*>(p),
                      1000, 0, p, reinterpret_cast<const float*>(p), nullptr) == KVQ_OK);
  // append, dequantize
  EXPECT(check_append(&ok, p, p, reinterpret_cast<const int64_t*>(p), -1, nullptr) == KVQ_ERR_INVALID);
  EXPECT(check_append(&ok, nullptr, nullptr, nullptr, 0, nullptr) == KVQ_OK);
  EXPECT(check_append(&ok, p + 2, p, reinterpret_cast<const int64_t*>(p), 1, nullptr) == KVQ_ERR_INVALID);
  // the fused step's new-token rows
  {
    Geometry g{};
    EXPECT(check_cache(&ok, true, &g) == KVQ_OK);
    EXPECT(check_step_rows(g, p, p, false) == KVQ_OK);
    EXPECT(check_step_rows(g, nullptr, p, false) == KVQ_ERR_INVALID);
    EXPECT(check_step_rows(g, p, p + 8, false) == KVQ_ERR_INVALID);
    EXPECT(check_step_rows(g, p, p, true) == KVQ_ERR_UNSUPPORTED);
    const kvq_cache vg = desc(128, 8, 4, 32, 128, 32, 64, 0, 1);
    Geometry gv{};
    EXPECT(check_cache(&vg, true, &gv) == KVQ_OK);
    EXPECT(check_step_rows(gv, p, p, false) == KVQ_ERR_UNSUPPORTED);
  }
  EXPECT(check_dequantize(&ok, 2, reinterpret_cast<const int64_t*>(p), 1, reinterpret_cast<const float*>(p),
                          nullptr) == KVQ_ERR_INVALID);
  EXPECT(check_dequantize(&ok, 1, reinterpret_cast<const int64_t*>(p), 1, reinterpret_cast<const float*>(p),
                          nullptr) == KVQ_OK);
  // windows
  kvq_window w{32, 128, 4, g_planes[0], g_planes[1], 0};
  EXPECT(check_window(&ok, &w, true) == KVQ_OK);
  w.sink = 8;
  EXPECT(check_window(&ok, &w, true) == KVQ_ERR_UNSUPPORTED);  // sink off the 16-token tile
  w.sink = 512;
  w.recent = 513;
  EXPECT(check_window(&ok, &w, true) == KVQ_ERR_UNSUPPORTED);  // sink + recent beyond 1024
  w = kvq_window{0, 16, 4, g_planes[0], g_planes[1], 1};
  EXPECT(check_window(&ok, &w, true) == KVQ_OK);
  w.sink = 16;
  EXPECT(check_window(&ok, &w, true) == KVQ_ERR_INVALID);  // a residual has no sink
}

// Sizes against their closed forms for supported caches.
static void closed_forms() {
  for (int bits : {2, 4})
    for (int G : {32, 64, 128})
      for (int P : {16, 48, 1024})
        for (int64_t pages : {int64_t(1), int64_t(3), int64_t(1000)}) {
          const kvq_cache c = desc(128, 8, bits, G, 128, P, pages);
          const int64_t tokens = pages * 8 * P;
          EXPECT(cache_plane_bytes(&c, 0) == tokens * 128 * bits / 8);
          EXPECT(cache_plane_bytes(&c, 2) == tokens * 128 * bits / 8);
          EXPECT(cache_plane_bytes(&c, 1) == tokens * (128 / G) * 4);
          EXPECT(cache_plane_bytes(&c, 3) == tokens * (128 / G) * 4);
          EXPECT(cache_plane_bytes(&c, 4) == -1);
          EXPECT(cache_plane_bytes(&c, -1) == -1);
        }
  // an unsupported but well-formed description still has sizes; one without a packing
  // has none
  const kvq_cache d64 = desc(64, 8, 4, 32, 64);
  EXPECT(cache_plane_bytes(&d64, 0) == 64 * 8 * 16 * 32);
  const kvq_cache b3 = desc(128, 8, 3);
  EXPECT(cache_plane_bytes(&b3, 0) == -1);
}

// Split-K sizing: partitions cover the context in whole blocks; workspace holds them.
static void split_sizing(const Geometry& g, int32_t batch, int32_t hq, int32_t maxlen, int32_t req, int cus,
                         SplitKernel kern) {
  const Splits s = choose_splits(g, batch, hq, maxlen, req, cus, kern);
  EXPECT(s.split_len > 0 && s.split_len % kBlock == 0);
  EXPECT(s.num_splits >= 1);
  EXPECT(static_cast<int64_t>(s.num_splits) * s.split_len >= (maxlen > 0 ? maxlen : 1));
  if (s.balanced) {
    EXPECT(s.unit_slots >= 1 && s.units_per_head >= 1);
    // one kv head's partitions, sum_b ceil(c_b / k) with every c_b <= ceil(maxlen / 256),
    // fit the slots
    const int64_t k = s.split_len / kBalancedMinLen;
    const int64_t cu = (static_cast<int64_t>(maxlen > 0 ? maxlen : 1) + kBalancedMinLen - 1) / kBalancedMinLen;
    EXPECT(static_cast<int64_t>(batch) * ((cu + k - 1) / k) <= s.unit_slots);
  } else if (req > 0) {
    EXPECT(s.num_splits <= req);
  }
  const size_t ws = workspace_bytes(g, batch, hq, s);
  if (ws != SIZE_MAX && !s.balanced)
    EXPECT(ws == static_cast<size_t>(batch) * hq * s.num_splits * (g.d + 2) * sizeof(float));
}

static void sweep() {
  const int ds[] = {1, 2, 16, 64, 128, 256, 1 << 16, (1 << 16) + 2, INT32_MAX};
  const int hkvs[] = {1, 8, 1 << 16, INT32_MAX};
  const int bitss[] = {-1, 0, 1, 2, 3, 4, 8, 9, INT32_MAX};
  const int Gs[] = {-32, 0, 1, 32, 64, 128, INT32_MAX};
  const int hbs[] = {-1, 0, 2, 3, 64, 128, 1 << 30, INT32_MAX};
  const int Ps[] = {-16, 0, 16, 48, 1 << 20, INT32_MAX - 15};
  const int64_t pagess[] = {-1, 0, 1, INT64_C(1) << 32, INT64_MAX};
  for (int d : ds)
    for (int hkv : hkvs)
      for (int bits : bitss)
        for (int G : Gs)
          for (int hb : hbs)
            for (int P : Ps)
              for (int64_t pages : pagess)
                for (int vg : {0, 1}) {
                  const kvq_cache c = desc(d, hkv, bits, G, hb, P, pages, 0, vg);
                  Geometry g;
                  const kvq_status st = check_cache(&c, true, &g);
                  EXPECT(st == KVQ_OK || st == KVQ_ERR_INVALID || st == KVQ_ERR_UNSUPPORTED);
                  for (int pl = 0; pl < 4; ++pl) {
                    const int64_t n = cache_plane_bytes(&c, pl);
                    EXPECT(n >= -1);
                    if (st == KVQ_ERR_INVALID) EXPECT(n == -1);
                  }
                  if (st != KVQ_OK) continue;
                  for (int32_t batch : {0, 1, 2, 64, 256, 257, 100000, INT32_MAX})
                    for (int64_t hq64 : {static_cast<int64_t>(hkv), 4 * static_cast<int64_t>(hkv)})
                      for (int32_t maxlen : {0, 1, 31, 33, 32768, 131072, kMaxSeqLen})
                        for (int32_t req : {0, 1, 7, 1 << 20, INT32_MAX})
                          for (SplitKernel kern : {SplitKernel::kMatrix, SplitKernel::kReference}) {
                            if (hq64 > INT32_MAX) continue;  // not an int32 head count
                            const int32_t hq = static_cast<int32_t>(hq64);
                            split_sizing(g, batch, hq, maxlen, req, 256, kern);
                            split_sizing(g, batch, hq, maxlen, req, 0, kern);
                            kvq_window w{16, 128, batch, g_planes[0], g_planes[1], 0};
                            if (check_window(&c, &w, true) == KVQ_OK) {
                              EXPECT(window_plane_bytes(g, &w) >= -1);
                              const int32_t span = window_span(&w, maxlen);
                              EXPECT(span >= 0 && span <= maxlen);
                              const Splits s = choose_splits(g, batch, hq, span, req, 256, kern);
                              EXPECT(window_workspace_bytes(g, batch, hq, s) >= workspace_bytes(g, batch, hq, s));
                            }
                          }
                }
}

int main() {
  documented_statuses();
  closed_forms();
  sweep();
  if (g_fail) {
    std::fprintf(stderr, "%d of %ld expectations failed\n", g_fail, g_cases);
    return 1;
  }
  std::printf("ok %ld\n", g_cases);
  return 0;
}
