// Host-side argument checking for the kvq C ABI (no HIP dependency).
#include "kvq_validate.h"

namespace kvq {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Products of non-negative sizes: -1 (int64) or SIZE_MAX (size_t) when the exact product
// does not fit, so no size computed here ever wraps.
static int64_t mul64(int64_t a, int64_t b) {
  int64_t r;
  return (a < 0 || b < 0 || __builtin_mul_overflow(a, b, &r)) ? -1 : r;
}
static size_t mulsz(size_t a, size_t b) {
  size_t r;
  return __builtin_mul_overflow(a, b, &r) ? SIZE_MAX : r;
}
static size_t addsz(size_t a, size_t b) {
  size_t r;
  return __builtin_add_overflow(a, b, &r) ? SIZE_MAX : r;
}

kvq_status check_cache(const kvq_cache* c, bool planes, Geometry* g) {
  if (!c) return KVQ_ERR_INVALID;
  if (c->head_dim <= 0 || c->num_kv_heads <= 0 || c->num_pages <= 0) return KVQ_ERR_INVALID;
  // far beyond any head; keeps every per-row size below in 32 bits
  if (c->head_dim > kMaxHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (c->bits != 2 && c->bits != 4) {
    // other widths are well formed integers but not a packing this library defines
    return (c->bits > 0 && c->bits <= 8) ? KVQ_ERR_UNSUPPORTED : KVQ_ERR_INVALID;
  }
  if (c->group_size <= 0 || c->head_dim % c->group_size != 0) return KVQ_ERR_INVALID;
  if (c->hadamard_block < 0) return KVQ_ERR_INVALID;
  if (c->hadamard_block > 0 && (!pow2(c->hadamard_block) || c->head_dim % c->hadamard_block != 0))
    return KVQ_ERR_INVALID;
  if (c->page_size <= 0 || c->page_size % kTile != 0) return KVQ_ERR_INVALID;
  if ((static_cast<int64_t>(c->head_dim) * c->bits) % 16 != 0) return KVQ_ERR_INVALID;
  if (c->quant_mode != 0 && c->quant_mode != 1) return KVQ_ERR_INVALID;
  if (c->v_grouping != 0 && c->v_grouping != 1) return KVQ_ERR_INVALID;
  // value token groups live inside one page
  if (c->v_grouping == 1 && c->page_size % c->group_size != 0) return KVQ_ERR_INVALID;
  if (planes) {
    const void* p[4] = {c->k_codes, c->k_meta, c->v_codes, c->v_meta};
    for (const void* x : p)
      if (!x || !aligned(x, 16)) return KVQ_ERR_INVALID;
  }
  Geometry t;
  t.d = c->head_dim;
  t.hkv = c->num_kv_heads;
  t.bits = c->bits;
  t.group = c->group_size;
  t.ngroups = c->head_dim / c->group_size;
  t.hblock = c->hadamard_block;
  t.page = c->page_size;
  t.row_bytes = c->head_dim * c->bits / 8;
  t.num_pages = c->num_pages;
  t.quant_mode = c->quant_mode;
  t.v_grouping = c->v_grouping;
  if (g) *g = t;
  return cache_supported(t) ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
}

bool cache_supported(const Geometry& g) {
  if (g.d != 128) return false;
  // the decode kernels index a page's rows of one kv head as page * Hkv + head, and a
  // 16-token tile of one kv head as (page * Hkv + head) * page_size / 16 + offset / 16, in
  // 32 bits: fewer than 2^32 tiles (2^32 tiles of INT2 codes alone would be 2 TiB)
  if (g.num_pages > 0xFFFFFFFFLL / g.hkv) return false;
  if (g.num_pages * g.hkv > 0xFFFFFFFFLL / (g.page / kTile)) return false;
  if (g.group != 32 && g.group != 64 && g.group != 128) return false;
  if (g.hblock != 0 && (g.hblock < 2 || g.hblock > 128)) return false;
  return true;
}

int64_t plane_bytes(const Geometry& g, int plane) {
  const int64_t tokens = mul64(mul64(g.num_pages, g.hkv), g.page);
  if (tokens < 0) return -1;
  switch (plane) {
    case 0:
    case 2:
      return mul64(tokens, g.row_bytes);
    case 1:
    case 3:
      return mul64(tokens, static_cast<int64_t>(g.ngroups) * 4);
    default:
      return -1;
  }
}

int64_t cache_plane_bytes(const kvq_cache* c, int32_t plane) {
  Geometry g;
  const kvq_status st = check_cache(c, false, &g);
  // well-formed descriptions have sizes whether or not a kernel is built for them; a
  // width other than 2 or 4 bits has no packing, and an oversized head no geometry
  if (st == KVQ_ERR_INVALID || !c) return -1;
  if (st == KVQ_ERR_UNSUPPORTED && ((c->bits != 2 && c->bits != 4) || c->head_dim > kMaxHeadDim)) return -1;
  return plane_bytes(g, plane);
}

Splits choose_splits(const Geometry& g, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                     int32_t requested, int cus, SplitKernel kernel) {
  (void)num_q_heads;
  Splits s{1, kBlock, 0, 0, 0};
  const int64_t len = max_seq_len > 0 ? max_seq_len : 1;
  const int64_t blocks = (len + kBlock - 1) / kBlock;
  const bool matrix = kernel == SplitKernel::kMatrix;
  if (requested == 0 && matrix && batch > 1 && batch <= kBalancedMaxBatch) {
    // Balanced: one round of equal partitions, as many as the GPU holds waves (kWavesPerCU
    // per CU, over all kv heads), of one length from the total span in 256-token units;
    // the device recomputes the plan from seq_lens (here every sequence is taken as
    // max_seq_len long).
    const int64_t nb = batch;
    const int64_t uph = (static_cast<int64_t>(kWavesPerCU) * (cus > 0 ? cus : 256) + g.hkv - 1) / g.hkv;
    const int64_t cu = (len + kBalancedMinLen - 1) / kBalancedMinLen;  // units of one sequence
    const int64_t C = nb * cu;
    int64_t k = C >= kBalancedMaxK * uph ? kBalancedMaxK : C > uph ? (C + uph - 1) / uph : 1;
    while (k < kBalancedMaxK && nb * ((cu + k - 1) / k) > uph) ++k;  // the device's fitting search
    s.split_len = static_cast<int32_t>(kBalancedMinLen * k);
    s.num_splits = static_cast<int32_t>((cu + k - 1) / k);
    s.balanced = 1;
    s.units_per_head = static_cast<int32_t>(uph);
    // partitions of one kv head: sum_b ceil(c_b / k) <= C / k + batch, where C / k <= uph
    // unless k is held at kBalancedMaxK, and every c_b <= cu
    const int64_t most = (C + kBalancedMaxK - 1) / kBalancedMaxK;
    int64_t slots = (most > uph ? most : uph) + nb;
    if (slots > C) slots = C;
    s.unit_slots = static_cast<int32_t>(slots);
    return s;
  }
  int64_t n;
  int64_t per;  // blocks per partition
  if (requested > 0) {
    n = requested < blocks ? requested : blocks;
    per = (blocks + n - 1) / n;
  } else {
    // Enough independent work units to fill every CU: one round of the matrix kernel's
    // waves (kWavesPerCU per CU; fewer, longer partitions measured faster than two
    // rounds), 16 per CU for the reference kernel; without partitions shorter than 8
    // blocks (256 tokens), whose partial results would cost more than they balance, nor
    // longer than 128 blocks (the reference kernel: 64, its LDS limit).
    const int64_t units = static_cast<int64_t>(batch) * g.hkv;
    const int64_t target = static_cast<int64_t>(matrix ? kWavesPerCU : 16) * (cus > 0 ? cus : 256);
    n = (target + units - 1) / (units > 0 ? units : 1);
    int64_t cap = blocks / 8;
    if (cap < 1) cap = 1;
    if (n > cap) n = cap;
    const int64_t max_per = matrix ? 128 : 64;
    const int64_t floor_n = (blocks + max_per - 1) / max_per;
    if (n < floor_n) n = floor_n;
    per = (blocks + n - 1) / n;
    // the matrix kernel walks whole 8-block super-blocks: the nearest multiple of 8
    if (matrix && per > 8) per = (per + 4) / 8 * 8;
  }
  s.split_len = static_cast<int32_t>(per * kBlock);
  s.num_splits = static_cast<int32_t>((blocks + per - 1) / per);
  return s;
}

size_t workspace_bytes(const Geometry& g, int32_t batch, int32_t num_q_heads, const Splits& s) {
  if (s.balanced)
    return addsz(balanced_partials_bytes(g, num_q_heads, s), (static_cast<size_t>(batch) * 8 + 255) / 256 * 256);
  return mulsz(mulsz(mulsz(static_cast<size_t>(batch), static_cast<size_t>(num_q_heads)),
                     static_cast<size_t>(s.num_splits)),
               static_cast<size_t>(g.d + 2) * sizeof(float));
}

size_t balanced_partials_bytes(const Geometry& g, int32_t num_q_heads, const Splits& s) {
  return mulsz(mulsz(static_cast<size_t>(num_q_heads), static_cast<size_t>(s.unit_slots)),
               static_cast<size_t>(g.d + 2) * sizeof(float));
}

kvq_status check_decode_sizes(int32_t batch, int32_t num_q_heads, int32_t max_seq_len, int32_t num_splits) {
  if (batch < 0 || num_q_heads <= 0 || max_seq_len < 0 || num_splits < 0) return KVQ_ERR_INVALID;
  if (max_seq_len > kMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status check_decode_args(const kvq_cache* c, const void* q, int32_t batch, int32_t num_q_heads,
                             const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                             int32_t max_seq_len, int32_t num_splits, const float* out, Geometry* g) {
  kvq_status st = check_cache(c, true, g);
  if (st != KVQ_OK) return st;
  st = check_decode_sizes(batch, num_q_heads, max_seq_len, num_splits);
  if (st != KVQ_OK) return st;
  if (num_q_heads % c->num_kv_heads != 0) return KVQ_ERR_INVALID;
  const int ratio = num_q_heads / c->num_kv_heads;
  if (ratio != 1 && ratio != 2 && ratio != 4) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  if (max_pages_per_seq <= 0) return KVQ_ERR_INVALID;
  if (static_cast<int64_t>(max_pages_per_seq) * c->page_size < max_seq_len) return KVQ_ERR_INVALID;
  if (!q || !aligned(q, 16)) return KVQ_ERR_INVALID;
  if (!block_table || !aligned(block_table, 4)) return KVQ_ERR_INVALID;
  if (!seq_lens || !aligned(seq_lens, 4)) return KVQ_ERR_INVALID;
  if (!out || !aligned(out, 16)) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

kvq_status check_decode(const kvq_cache* c, const void* q, int32_t batch, int32_t num_q_heads,
                        const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                        int32_t max_seq_len, int32_t num_splits, const void* workspace, const float* out,
                        Geometry* g) {
  const kvq_status st = check_decode_args(c, q, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                                          max_seq_len, num_splits, out, g);
  if (st != KVQ_OK || batch == 0) return st;
  if (!workspace || !aligned(workspace, 16)) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

kvq_status check_append(const kvq_cache* c, const void* k_new, const void* v_new, const int64_t* slots,
                        int64_t n_new, Geometry* g) {
  kvq_status st = check_cache(c, true, g);
  if (st != KVQ_OK) return st;
  if (n_new < 0) return KVQ_ERR_INVALID;
  if (c->v_grouping == 1 && n_new % c->group_size != 0) return KVQ_ERR_INVALID;  // whole token groups
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new || !slots) return KVQ_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slots, 8)) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

kvq_status check_step_rows(const Geometry& g, const void* k_new, const void* v_new, bool reference) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return KVQ_ERR_INVALID;
  if (reference || g.v_grouping != 0) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status check_window(const kvq_cache* c, const kvq_window* w, bool planes) {
  if (!c || !w) return KVQ_ERR_INVALID;
  if (w->sink < 0 || w->recent < 1 || w->batch < 0) return KVQ_ERR_INVALID;
  if (w->residual != 0 && w->residual != 1) return KVQ_ERR_INVALID;
  if (w->residual == 1 && w->sink != 0) return KVQ_ERR_INVALID;
  // a completed group goes to its tokens' consecutive slots: groups must not cross pages
  if (w->residual == 1 && c->page_size % w->recent != 0) return KVQ_ERR_INVALID;
  // value token groups come whole out of a residual of one group
  if (c->v_grouping == 1 && (w->residual != 1 || w->recent != c->group_size)) return KVQ_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(w->sink) + w->recent > kMaxWindow) return KVQ_ERR_UNSUPPORTED;
  // the quantized span starts at `sink`, which the decode kernels need on a tile boundary
  if (w->sink % kTile != 0) return KVQ_ERR_UNSUPPORTED;
  if (planes && (!w->k || !w->v || !aligned(w->k, 16) || !aligned(w->v, 16))) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

int64_t window_plane_bytes(const Geometry& g, const kvq_window* w) {
  return mul64(mul64(mul64(w->batch, static_cast<int64_t>(w->sink) + w->recent), g.hkv), static_cast<int64_t>(g.d) * 2);
}

kvq_status check_window_append(const kvq_cache* c, const kvq_window* w, const void* k_new, const void* v_new,
                               const int32_t* seqs, const int32_t* positions, const int64_t* evict_slots,
                               int64_t n_new, Geometry* g) {
  kvq_status st = check_cache(c, true, g);
  if (st != KVQ_OK) return st;
  st = check_window(c, w, true);
  if (st != KVQ_OK) return st;
  if (n_new < 0) return KVQ_ERR_INVALID;
  if (n_new == 0) return KVQ_OK;
  if (n_new > w->batch) return KVQ_ERR_INVALID;  // at most one token per sequence
  if (!k_new || !v_new || !seqs || !positions || !evict_slots) return KVQ_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(seqs, 4) || !aligned(positions, 4) ||
      !aligned(evict_slots, 8))
    return KVQ_ERR_INVALID;
  return KVQ_OK;
}

int32_t window_span(const kvq_window* w, int32_t max_seq_len) {
  if (w->residual) return max_seq_len;  // up to max_seq_len - (max_seq_len % recent)
  const int64_t n = static_cast<int64_t>(max_seq_len) - w->sink - w->recent;
  return n > 0 ? static_cast<int32_t>(n) : 0;
}

size_t window_workspace_bytes(const Geometry& g, int32_t batch, int32_t num_q_heads, const Splits& s) {
  return addsz(workspace_bytes(g, batch, num_q_heads, s),
               mulsz(mulsz(static_cast<size_t>(batch), static_cast<size_t>(num_q_heads)),
                     static_cast<size_t>(g.d + 2) * sizeof(float)));
}

kvq_status check_dequantize(const kvq_cache* c, int32_t which, const int64_t* slots, int64_t n,
                            const float* out, Geometry* g) {
  kvq_status st = check_cache(c, true, g);
  if (st != KVQ_OK) return st;
  if (which != 0 && which != 1) return KVQ_ERR_INVALID;
  if (n < 0) return KVQ_ERR_INVALID;
  if (n == 0) return KVQ_OK;
  if (!slots || !aligned(slots, 8) || !out || !aligned(out, 16)) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

}  // namespace kvq
