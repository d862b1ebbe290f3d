/*
 * kvq oracle: plain CPU reference. TEST INFRASTRUCTURE ONLY (see kvq_oracle.h).
 *
 * Build: g++ -std=c++17 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared kvq_oracle.cpp -lm
 * (C-style C++: plain loops and arrays; the exported functions have C linkage.)
 * -ffp-contract=off keeps every fp32 operation a separate IEEE rounding, which the
 * arithmetic contract in kvq_oracle.h requires.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats, written from the IEEE 754 binary16 and bfloat16 definitions. */

float orc_bf16_to_f32(uint16_t b) {
  /* bfloat16 is the top half of a binary32 pattern: widening is exact. */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static int bit_length_u32(uint32_t m) {
  int n = 0;
  while (m) {
    ++n;
    m >>= 1;
  }
  return n;
}

uint16_t orc_f32_to_f16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t ex = (u >> 23) & 0xFFu;
  uint32_t man = u & 0x7FFFFFu;
  if (ex == 0xFFu) {
    if (man == 0) return sign | 0x7C00u;                      /* infinity */
    return (uint16_t)(sign | 0x7E00u | (man >> 13));          /* quiet NaN */
  }
  /* |x| = m * 2^e with m an integer of at most 24 bits */
  uint32_t m;
  int e;
  if (ex == 0) {
    m = man;
    e = -149;
  } else {
    m = man | 0x800000u;
    e = (int)ex - 150;
  }
  if (m == 0) return sign; /* signed zero */
  /* binary16 keeps 11 significant bits; its smallest quantum is 2^-24 */
  int top = bit_length_u32(m) - 1 + e; /* floor(log2 |x|) */
  int q = top - 10;
  if (q < -24) q = -24;
  /* N = round_half_even(m * 2^(e - q)) */
  uint64_t N;
  int sh = q - e;
  if (sh <= 0) {
    N = (uint64_t)m << (-sh); /* exact; only when the value is already coarse */
  } else if (sh > 40) {
    N = 0;
  } else {
    uint64_t mm = m;
    uint64_t whole = mm >> sh;
    uint64_t rem = mm - (whole << sh);
    uint64_t half = (uint64_t)1 << (sh - 1);
    if (rem > half || (rem == half && (whole & 1u))) whole += 1;
    N = whole;
  }
  if (N == 0) return sign;
  /* re-normalise: a round-up can carry into the next binade */
  while (N >= 2048) {
    N >>= 1; /* N is even here: 2048 exactly */
    q += 1;
  }
  if (N >= 1024) {
    int biased = q + 25; /* value = N * 2^q = (N/1024) * 2^(q+10), exponent field q+10+15 */
    if (biased >= 31) return sign | 0x7C00u;
    return (uint16_t)(sign | ((uint32_t)biased << 10) | (uint32_t)(N - 1024));
  }
  /* subnormal: q == -24 */
  return (uint16_t)(sign | (uint32_t)N);
}

float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = (h & 0x8000u) ? 1u : 0u;
  uint32_t ex = (h >> 10) & 31u;
  uint32_t f = h & 1023u;
  float v;
  if (ex == 0) {
    v = ldexpf((float)f, -24);
  } else if (ex == 31) {
    if (f == 0) {
      v = INFINITY;
    } else {
      uint32_t u = 0x7FC00000u | (f << 13);
      memcpy(&v, &u, 4);
      return sign ? -v : v;
    }
  } else {
    v = ldexpf((float)(1024u + f), (int)ex - 25);
  }
  return sign ? -v : v;
}

void orc_f32_to_f16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_array(const uint16_t* h, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(h[i]);
}

float orc_fmaf(float a, float b, float c) { return fmaf(a, b, c); }

/* ------------------------------------------------------------------------- */
/* Walsh-Hadamard rotation (SAW-INT4, Abstract: block-diagonal Hadamard rotation;
   Dual-QK, Abstract: the same orthogonal transform on queries and keys). */

static int popcount_u32(uint32_t v) {
  int c = 0;
  while (v) {
    c += (int)(v & 1u);
    v >>= 1;
  }
  return c;
}

void orc_hadamard_sylvester(int n, int32_t* H) {
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) H[i * n + j] = (popcount_u32((uint32_t)(i & j)) & 1) ? -1 : 1;
}

void orc_fwht_unnormalized(float* x, int n) {
  for (int h = 1; h < n; h <<= 1)
    for (int i = 0; i < n; ++i)
      if (!(i & h)) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
}

float orc_rotation_constant(int n) {
  /* 1/sqrt(2^k) = 2^(-k/2); for odd k it is sqrt(2) * 2^(-(k+1)/2), and scaling the
     correctly rounded sqrt(2) by a power of two keeps it the nearest float. */
  int k = 0;
  while ((1 << k) < n) ++k;
  if ((k & 1) == 0) return ldexpf(1.0f, -k / 2);
  return ldexpf(sqrtf(2.0f), -(k + 1) / 2);
}

void orc_rotate(float* x, int d, int block) {
  if (block <= 0) return;
  float c = orc_rotation_constant(block);
  for (int b = 0; b < d; b += block) {
    orc_fwht_unnormalized(x + b, block);
    for (int i = 0; i < block; ++i) x[b + i] = x[b + i] * c;
  }
}

void orc_rotate_dense_f64(const double* x, double* y, int d, int block) {
  if (block <= 0) {
    for (int i = 0; i < d; ++i) y[i] = x[i];
    return;
  }
  int32_t* H = (int32_t*)malloc(sizeof(int32_t) * (size_t)block * (size_t)block);
  orc_hadamard_sylvester(block, H);
  double inv = 1.0 / sqrt((double)block);
  for (int b = 0; b < d; b += block)
    for (int i = 0; i < block; ++i) {
      double acc = 0.0;
      for (int k = 0; k < block; ++k) acc += (double)H[i * block + k] * x[b + k];
      y[b + i] = acc * inv;
    }
  free(H);
}

/* ------------------------------------------------------------------------- */
/* Asymmetric min/max group quantizer (InnerQ, Abstract: group-wise quantization with
   asymmetric groups; SAW-INT4, Abstract: token-wise groups; the fp32 formula itself is
   this library's reading, spelled out in kvq_oracle.h). */

/* codes of one group for the stored pair (s16, z16) */
static void group_codes(const float* xg, int group, int qmax, uint16_t s16, uint16_t z16, uint8_t* codes) {
  float s = orc_f16_to_f32(s16), z = orc_f16_to_f32(z16);
  if (s == 0.0f) {
    for (int i = 0; i < group; ++i) codes[i] = 0;
    return;
  }
  float inv = 1.0f / s;
  for (int i = 0; i < group; ++i) {
    float diff = xg[i] - z;
    float u = diff * inv;
    float r = rintf(u);
    int c = (int)r;
    if (r < 0.0f) c = 0;
    if (r > (float)qmax) c = qmax;
    codes[i] = (uint8_t)c;
  }
}

/* largest |x - fmaf(code, s, z)| of one group, in fp32 */
static float group_max_error(const float* xg, int group, const uint8_t* codes, uint16_t s16, uint16_t z16) {
  float s = orc_f16_to_f32(s16), z = orc_f16_to_f32(z16);
  float e = 0.0f;
  for (int i = 0; i < group; ++i) {
    float d = fabsf(xg[i] - fmaf((float)codes[i], s, z));
    if (d > e) e = d;
  }
  return e;
}

static void quantize_row_mode(const float* x, int d, int bits, int group, int hybrid, uint8_t* codes,
                              uint16_t* scale, uint16_t* zero) {
  const int qmax = (1 << bits) - 1;
  uint8_t* alt = (uint8_t*)malloc((size_t)group);
  for (int g = 0; g < d / group; ++g) {
    const float* xg = x + g * group;
    float mn = xg[0], mx = xg[0];
    for (int i = 1; i < group; ++i) {
      if (xg[i] < mn) mn = xg[i];
      if (xg[i] > mx) mx = xg[i];
    }
    float range = mx - mn;
    float s32 = range / (float)qmax;
    uint16_t s16 = orc_f32_to_f16(s32);
    uint16_t z16 = orc_f32_to_f16(mn + 0.0f); /* +0.0f turns -0 into +0 */
    group_codes(xg, group, qmax, s16, z16, codes + g * group);
    if (hybrid) {
      /* InnerQ, Abstract: each group takes the symmetric or the asymmetric quantizer
         from its own statistics. Reading: symmetric = scale max|x| / (2^(b-1) - 1) with
         codes centred on 2^(b-1), stored as the pair {scale, zero = -2^(b-1) scale}
         (exact in fp16); the group keeps the candidate with the smaller largest
         reconstruction error, the asymmetric one on a tie. */
      const int mid = 1 << (bits - 1);
      float a = fabsf(mn) > fabsf(mx) ? fabsf(mn) : fabsf(mx);
      uint16_t ss16 = orc_f32_to_f16(a / (float)(mid - 1));
      uint16_t sz16 = orc_f32_to_f16(-((float)mid * orc_f16_to_f32(ss16)) + 0.0f);
      group_codes(xg, group, qmax, ss16, sz16, alt);
      float err_a = group_max_error(xg, group, codes + g * group, s16, z16);
      float err_s = group_max_error(xg, group, alt, ss16, sz16);
      if (err_s < err_a) {
        s16 = ss16;
        z16 = sz16;
        for (int i = 0; i < group; ++i) codes[g * group + i] = alt[i];
      }
    }
    scale[g] = s16;
    zero[g] = z16;
  }
  free(alt);
}

void orc_quantize_row(const float* x, int d, int bits, int group, uint8_t* codes, uint16_t* scale,
                      uint16_t* zero) {
  quantize_row_mode(x, d, bits, group, 0, codes, scale, zero);
}

void orc_quantize_row_hybrid(const float* x, int d, int bits, int group, uint8_t* codes, uint16_t* scale,
                             uint16_t* zero) {
  quantize_row_mode(x, d, bits, group, 1, codes, scale, zero);
}

void orc_pack_row(const uint8_t* codes, int d, int bits, uint8_t* packed) {
  int per_byte = 8 / bits;
  memset(packed, 0, (size_t)(d * bits / 8));
  for (int k = 0; k < d; ++k) packed[k / per_byte] |= (uint8_t)(codes[k] << (bits * (k % per_byte)));
}

void orc_unpack_row(const uint8_t* packed, int d, int bits, uint8_t* codes) {
  int per_byte = 8 / bits;
  uint8_t mask = (uint8_t)((1 << bits) - 1);
  for (int k = 0; k < d; ++k) codes[k] = (packed[k / per_byte] >> (bits * (k % per_byte))) & mask;
}

/* ------------------------------------------------------------------------- */
/* Cache layout (SAW-INT4, Abstract: quantized rows go straight into a paged KV layout;
   the byte layout itself is this library's reading, spelled out in kvq_oracle.h). */

static int64_t row_bytes(const orc_cache* c) { return (int64_t)c->head_dim * c->bits / 8; }
static int64_t n_groups(const orc_cache* c) { return c->head_dim / c->group_size; }

int64_t orc_plane_bytes(const orc_cache* c, int plane) {
  int64_t tokens = c->num_pages * c->num_kv_heads * (int64_t)c->page_size;
  if (plane == 0 || plane == 2) return tokens * row_bytes(c);
  return tokens * n_groups(c) * 4;
}

int orc_check_cache(const orc_cache* c) {
  if (c->head_dim <= 0 || c->head_dim > 4096 || c->num_kv_heads <= 0 || c->num_pages <= 0) return 1;
  if (c->bits != 2 && c->bits != 4) return 2;
  if (c->group_size <= 0 || c->head_dim % c->group_size) return 3;
  if (c->hadamard_block < 0) return 4;
  if (c->hadamard_block > 0) {
    if (c->hadamard_block & (c->hadamard_block - 1)) return 4;
    if (c->head_dim % c->hadamard_block) return 4;
  }
  if (c->page_size <= 0 || c->page_size % 16) return 5;
  if ((c->head_dim * c->bits) % 128) return 6; /* whole 16-byte chunks per row */
  if (c->quant_mode != 0 && c->quant_mode != 1) return 7;
  if (c->v_grouping != 0 && c->v_grouping != 1) return 8;
  if (c->v_grouping == 1 && (c->head_dim != 128 || c->group_size % 32 || c->page_size % c->group_size)) return 8;
  return 0;
}

/* byte k (0..RB-1) of the packed K row of token `off`: 16-token tiles; inside a tile the
   rows are cut into 16-byte chunks stored chunk-major: chunk j of tokens 0..15, then chunk
   j+1: chunk k/16, token o, byte k%16 -> ((k/16)*16 + o)*16 + k%16 */
static int64_t k_byte_off(const orc_cache* c, int64_t page, int h, int off, int k) {
  int64_t base = (page * c->num_kv_heads + h) * c->page_size * row_bytes(c);
  int64_t tile = (off / 16) * 16 * row_bytes(c);
  int o = off % 16;
  return base + tile + ((int64_t)(k / 16) * 16 + o) * 16 + k % 16;
}
static int64_t k_meta_off(const orc_cache* c, int64_t page, int h, int off, int g) {
  return (((page * c->num_kv_heads + h) * c->page_size + off) * n_groups(c) + g) * 4;
}
/* byte k (0..RB-1) of the packed V row of token `off`: 16-token tiles; inside a tile the
   row is cut into 16-bit words and each word holds its 16 tokens as 8 token pairs, the
   pair's low bytes then its high bytes, byte-interleaved by token:
   word w, token o, byte b -> w*32 + (o/2)*4 + b*2 + (o%2) */
static int64_t v_byte_off(const orc_cache* c, int64_t page, int h, int off, int k) {
  int64_t base = (page * c->num_kv_heads + h) * c->page_size * row_bytes(c);
  int64_t tile = (off / 16) * 16 * row_bytes(c);
  int o = off % 16, w = k / 2, b = k % 2;
  return base + tile + (int64_t)w * 32 + (o / 2) * 4 + b * 2 + (o % 2);
}
/* V {scale, zero} of token `off`, group g: 16-token tiles of NG*16 entries; token
   o = 8*half + 4*part + i sits at entry ((part*NG + g)*2 + half)*4 + i */
static int64_t v_meta_off(const orc_cache* c, int64_t page, int h, int off, int g) {
  int64_t tiles = c->page_size / 16;
  int64_t t = (page * c->num_kv_heads + h) * tiles + off / 16;
  int o = off % 16, half = o / 8, part = (o % 8) / 4, i = o % 4;
  return (t * n_groups(c) * 16 + (((int64_t)part * n_groups(c) + g) * 2 + half) * 4 + i) * 4;
}

/* V token groups (v_grouping 1): {scale, zero} per (group of G tokens of a page, channel),
   128 entries per group; channel c sits at entry 8n + t with
   c = 4(n + 16(t >> 2)) + 2(t & 1) + ((t >> 1) & 1) at INT4 and c = 8n + (t >> 1) + 4(t & 1)
   at INT2 (n = 0..15, t = 0..7), so that the 8 channels one decode lane needs are
   adjacent. */
static int vt_entry(int bits, int ch) {
  int n, t;
  if (bits == 4) {
    n = (ch / 4) % 16;
    t = 4 * (ch / 64) + 2 * (ch % 2) + (ch % 4) / 2;
  } else {
    n = ch / 8;
    t = 2 * (ch % 4) + (ch % 8) / 4;
  }
  return 8 * n + t;
}
static int64_t vt_meta_off(const orc_cache* c, int64_t page, int h, int gi, int ch) {
  int64_t groups = c->page_size / c->group_size;
  return (((page * c->num_kv_heads + h) * groups + gi) * 128 + vt_entry(c->bits, ch)) * 4;
}

static void put_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)(v >> 8);
}
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static void store_row(const orc_cache* c, int which, int64_t page, int h, int off, const uint8_t* packed,
                      const uint16_t* scale, const uint16_t* zero) {
  int64_t rb = row_bytes(c);
  if (which == 0) {
    for (int k = 0; k < rb; ++k) c->k_codes[k_byte_off(c, page, h, off, k)] = packed[k];
    for (int g = 0; g < n_groups(c); ++g) {
      uint8_t* m = c->k_meta + k_meta_off(c, page, h, off, g);
      put_u16(m, scale[g]);
      put_u16(m + 2, zero[g]);
    }
  } else {
    for (int k = 0; k < rb; ++k) c->v_codes[v_byte_off(c, page, h, off, k)] = packed[k];
    if (c->v_grouping == 1) return; /* token groups store their {scale, zero} per group */
    for (int g = 0; g < n_groups(c); ++g) {
      uint8_t* m = c->v_meta + v_meta_off(c, page, h, off, g);
      put_u16(m, scale[g]);
      put_u16(m + 2, zero[g]);
    }
  }
}

static void load_row(const orc_cache* c, int which, int64_t page, int h, int off, uint8_t* packed,
                     uint16_t* scale, uint16_t* zero) {
  int64_t rb = row_bytes(c);
  if (which == 0) {
    for (int k = 0; k < rb; ++k) packed[k] = c->k_codes[k_byte_off(c, page, h, off, k)];
    for (int g = 0; g < n_groups(c); ++g) {
      const uint8_t* m = c->k_meta + k_meta_off(c, page, h, off, g);
      scale[g] = get_u16(m);
      zero[g] = get_u16(m + 2);
    }
  } else {
    for (int k = 0; k < rb; ++k) packed[k] = c->v_codes[v_byte_off(c, page, h, off, k)];
    if (c->v_grouping == 1) { /* per channel: scale[i], zero[i] for channel i */
      for (int i = 0; i < c->head_dim; ++i) {
        const uint8_t* m = c->v_meta + vt_meta_off(c, page, h, off / c->group_size, i);
        scale[i] = get_u16(m);
        zero[i] = get_u16(m + 2);
      }
      return;
    }
    for (int g = 0; g < n_groups(c); ++g) {
      const uint8_t* m = c->v_meta + v_meta_off(c, page, h, off, g);
      scale[g] = get_u16(m);
      zero[g] = get_u16(m + 2);
    }
  }
}

/* Dequantize one stored row into fp32: xhat = fmaf(code, scale, zero). */
static void dequant_row(const orc_cache* c, int which, int64_t page, int h, int off, float* out) {
  int d = c->head_dim;
  int G = c->group_size;
  uint8_t packed[4096];
  uint8_t codes[4096];
  uint16_t sc[4096], ze[4096];
  load_row(c, which, page, h, off, packed, sc, ze);
  orc_unpack_row(packed, d, c->bits, codes);
  int per_channel = which == 1 && c->v_grouping == 1;
  for (int i = 0; i < d; ++i) {
    float s = orc_f16_to_f32(sc[per_channel ? i : i / G]);
    float z = orc_f16_to_f32(ze[per_channel ? i : i / G]);
    out[i] = fmaf((float)codes[i], s, z);
  }
}

/* Quantize one bf16 row of kv head h (K rotated first, or V with channel groups) and
   store it at `slot`. */
static void quantize_store_row_one(const orc_cache* c, int which, const uint16_t* row, int64_t slot, int h) {
  int d = c->head_dim;
  float* x = (float*)malloc(sizeof(float) * (size_t)d);
  uint8_t* codes = (uint8_t*)malloc((size_t)d);
  uint8_t* packed = (uint8_t*)malloc((size_t)d);
  uint16_t* sc = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
  uint16_t* ze = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
  for (int i = 0; i < d; ++i) x[i] = orc_bf16_to_f32(row[i]);
  if (which == 0) orc_rotate(x, d, c->hadamard_block); /* keys only */
  quantize_row_mode(x, d, c->bits, c->group_size, c->quant_mode == 1, codes, sc, ze);
  orc_pack_row(codes, d, c->bits, packed);
  store_row(c, which, slot / c->page_size, h, (int)(slot % c->page_size), packed, sc, ze);
  free(x);
  free(codes);
  free(packed);
  free(sc);
  free(ze);
}

/* V token groups (InnerQ, Abstract: groups along the inner dimension of the value
   product). Reading: channel ch of the G tokens slot0 .. slot0 + G - 1 (one page,
   slot0 a multiple of G) forms one group, quantized by the same formula as a row group
   (min/max, or hybrid); rows[i] is the bf16 V row of token slot0 + i. */
static void quantize_store_v_group(const orc_cache* c, const uint16_t* const* rows, int64_t slot0, int h) {
  int d = c->head_dim, G = c->group_size;
  int64_t page = slot0 / c->page_size;
  int off0 = (int)(slot0 % c->page_size);
  float* col = (float*)malloc(sizeof(float) * (size_t)G);
  uint8_t* ccodes = (uint8_t*)malloc((size_t)G);
  uint8_t* codes = (uint8_t*)malloc((size_t)G * (size_t)d); /* [token][channel] */
  uint8_t* packed = (uint8_t*)malloc((size_t)d);
  for (int ch = 0; ch < d; ++ch) {
    uint16_t sc, ze;
    for (int i = 0; i < G; ++i) col[i] = orc_bf16_to_f32(rows[i][ch]);
    quantize_row_mode(col, G, c->bits, G, c->quant_mode == 1, ccodes, &sc, &ze);
    uint8_t* m = c->v_meta + vt_meta_off(c, page, h, off0 / G, ch);
    put_u16(m, sc);
    put_u16(m + 2, ze);
    for (int i = 0; i < G; ++i) codes[(size_t)i * d + ch] = ccodes[i];
  }
  for (int i = 0; i < G; ++i) {
    orc_pack_row(codes + (size_t)i * d, d, c->bits, packed);
    for (int k = 0; k < row_bytes(c); ++k) c->v_codes[v_byte_off(c, page, h, off0 + i, k)] = packed[k];
  }
  free(col);
  free(ccodes);
  free(codes);
  free(packed);
}

/* Quantize the bf16 K and V rows of kv head h and store them at `slot` (channel groups). */
static void quantize_store_pair(const orc_cache* c, const uint16_t* krow, const uint16_t* vrow, int64_t slot, int h) {
  quantize_store_row_one(c, 0, krow, slot, h);
  quantize_store_row_one(c, 1, vrow, slot, h);
}

/* G tokens whose V rows form token groups: keys row by row at slots[i], values as one
   group per kv head at slots[0] .. slots[0] + G - 1. k, v: bf16 [G][Hkv][d]. */
static void quantize_store_token_group(const orc_cache* c, const uint16_t* k, const uint16_t* v, const int64_t* slots,
                                       int64_t krow_stride, int64_t vrow_stride) {
  int d = c->head_dim, H = c->num_kv_heads, G = c->group_size;
  const uint16_t** rows = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)G);
  for (int h = 0; h < H; ++h) {
    for (int i = 0; i < G; ++i) {
      quantize_store_row_one(c, 0, k + i * krow_stride + (int64_t)h * d, slots[i], h);
      rows[i] = v + i * vrow_stride + (int64_t)h * d;
    }
    quantize_store_v_group(c, rows, slots[0], h);
  }
  free(rows);
}

void orc_quantize_append(const orc_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                         const int64_t* slots, int64_t n) {
  int d = c->head_dim;
  if (c->v_grouping == 1) { /* whole token groups of G consecutive rows */
    int G = c->group_size;
    int64_t stride = (int64_t)c->num_kv_heads * d;
    for (int64_t r = 0; r + G <= n; r += G)
      quantize_store_token_group(c, k_new + r * stride, v_new + r * stride, slots + r, stride, stride);
    return;
  }
  for (int64_t r = 0; r < n; ++r)
    for (int h = 0; h < c->num_kv_heads; ++h)
      quantize_store_pair(c, k_new + (r * c->num_kv_heads + h) * d, v_new + (r * c->num_kv_heads + h) * d, slots[r],
                          h);
}

void orc_dequantize(const orc_cache* c, int which, const int64_t* slots, int64_t n, float* out) {
  int d = c->head_dim;
  for (int64_t r = 0; r < n; ++r) {
    int64_t page = slots[r] / c->page_size;
    int off = (int)(slots[r] % c->page_size);
    for (int h = 0; h < c->num_kv_heads; ++h)
      dequant_row(c, which, page, h, off, out + (r * c->num_kv_heads + h) * d);
  }
}

/* ------------------------------------------------------------------------- */
/* Decode attention over the quantized cache, in fp64 (SAW-INT4, Abstract: attention runs
   over the INT4 paged cache; Dual-QK, Abstract: queries get the keys' rotation so q.k is
   preserved). Query head j reads KV head j / (Hq / Hkv). */

static void decode_attention_masked(const orc_cache* c, const uint16_t* q, int32_t batch, int32_t num_q_heads,
                                    const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                    double softmax_scale, const int32_t* keep_mask, double* out) {
  int width = 128 / c->bits; /* channels of one 16-byte chunk of a packed key row */
  int d = c->head_dim;
  int P = c->page_size;
  int ratio = num_q_heads / c->num_kv_heads;
  double sigma = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)d);
  double* qv = (double*)malloc(sizeof(double) * (size_t)d);
  double* qr = (double*)malloc(sizeof(double) * (size_t)d);
  float* row = (float*)malloc(sizeof(float) * (size_t)d);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  for (int b = 0; b < batch; ++b) {
    int T = seq_lens[b];
    double* logit = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int j = 0; j < num_q_heads; ++j) {
      int h = j / ratio;
      double* o = out + ((int64_t)b * num_q_heads + j) * d;
      if (T <= 0) {
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        continue;
      }
      for (int i = 0; i < d; ++i) qv[i] = (double)orc_bf16_to_f32(q[((int64_t)b * num_q_heads + j) * d + i]);
      orc_rotate_dense_f64(qv, qr, d, c->hadamard_block);
      if (keep_mask) { /* pruned query channels take no part in the scores */
        int32_t mask = keep_mask[(int64_t)b * c->num_kv_heads + h];
        for (int i = 0; i < d; ++i)
          if (!((mask >> (i / width)) & 1)) qr[i] = 0.0;
      }
      double m = -INFINITY;
      for (int t = 0; t < T; ++t) {
        int64_t page = block_table[(int64_t)b * max_pages + t / P];
        dequant_row(c, 0, page, h, t % P, row);
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += qr[i] * (double)row[i];
        logit[t] = sigma * dot;
        if (logit[t] > m) m = logit[t];
      }
      double den = 0.0;
      for (int i = 0; i < d; ++i) acc[i] = 0.0;
      for (int t = 0; t < T; ++t) {
        double w = exp(logit[t] - m);
        den += w;
        int64_t page = block_table[(int64_t)b * max_pages + t / P];
        dequant_row(c, 1, page, h, t % P, row);
        for (int i = 0; i < d; ++i) acc[i] += w * (double)row[i];
      }
      for (int i = 0; i < d; ++i) o[i] = acc[i] / den;
    }
    free(logit);
  }
  free(qv);
  free(qr);
  free(row);
  free(acc);
}

void orc_decode_attention(const orc_cache* c, const uint16_t* q, int32_t batch, int32_t num_q_heads,
                          const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                          double softmax_scale, double* out) {
  decode_attention_masked(c, q, batch, num_q_heads, block_table, max_pages, seq_lens, softmax_scale, NULL, out);
}

/* Query-channel pruning of key reads (Dual-QK, Abstract: dynamic query-channel pruning
   further reduces key-cache reads). Reading: per (sequence, kv head) the rotated query
   keeps whole 16-byte chunks of the packed key row (128 / bits channels each, the unit in
   which key codes are read); bit j of keep_mask[b * Hkv + h] keeps chunk j, the other
   channels count as zero in every score. Values are not pruned. */
void orc_decode_attention_pruned(const orc_cache* c, const uint16_t* q, int32_t batch, int32_t num_q_heads,
                                 const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                 double softmax_scale, const int32_t* keep_mask, double* out) {
  decode_attention_masked(c, q, batch, num_q_heads, block_table, max_pages, seq_lens, softmax_scale, keep_mask,
                          out);
}

/* Energy of each chunk of the rotated query, summed over the query heads of each kv head:
   energy[(b * Hkv + h) * n_chunks + j] = sum over heads of h, channels of chunk j, of qr^2
   (fp64), n_chunks = head_dim * bits / 128. The pruning keeps the largest. */
void orc_prune_energy(const orc_cache* c, const uint16_t* q, int32_t batch, int32_t num_q_heads, double* energy) {
  int d = c->head_dim, H = c->num_kv_heads, width = 128 / c->bits, nch = d / width;
  int ratio = num_q_heads / H;
  double* qv = (double*)malloc(sizeof(double) * (size_t)d);
  double* qr = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t i = 0; i < (int64_t)batch * H * nch; ++i) energy[i] = 0.0;
  for (int b = 0; b < batch; ++b)
    for (int j = 0; j < num_q_heads; ++j) {
      for (int i = 0; i < d; ++i) qv[i] = (double)orc_bf16_to_f32(q[((int64_t)b * num_q_heads + j) * d + i]);
      orc_rotate_dense_f64(qv, qr, d, c->hadamard_block);
      for (int i = 0; i < d; ++i) energy[((int64_t)b * H + j / ratio) * nch + i / width] += qr[i] * qr[i];
    }
  free(qv);
  free(qr);
}

/* ------------------------------------------------------------------------- */
/* High-precision windows (InnerQ, Abstract: windows of recent tokens and of attention
   sink tokens stay in high precision). Reading: the first `sink` tokens and the last
   `recent` tokens of every sequence stay in bf16, keys in the original (unrotated)
   basis; a token leaving the recent window is quantized into the cache at its own slot;
   the tokens between are the quantized cache. */

int orc_window_slot(const orc_window* w, int t) { return t < w->sink ? t : w->sink + (t - w->sink) % w->recent; }

/* is token t of a sequence of T tokens a window token? */
static int in_window(const orc_window* w, int t, int T) {
  if (w->residual) return t >= T - T % w->recent; /* the incomplete last group */
  return t < w->sink || t >= T - w->recent;
}

void orc_window_append(const orc_cache* c, const orc_window* w, const uint16_t* k_new, const uint16_t* v_new,
                       const int32_t* seqs, const int32_t* positions, const int64_t* evict_slots, int64_t n) {
  int d = w->head_dim, H = w->num_kv_heads, S = w->sink, R = w->recent;
  for (int64_t r = 0; r < n; ++r) {
    int b = seqs[r], t = positions[r];
    int ws = orc_window_slot(w, t);
    for (int h = 0; h < H; ++h) {
      uint16_t* kw = w->k + (((int64_t)b * (S + R) + ws) * H + h) * d;
      uint16_t* vw = w->v + (((int64_t)b * (S + R) + ws) * H + h) * d;
      /* the recent ring is full: its slot holds token t - R, which now leaves the window */
      if (!w->residual && t >= S && t - R >= S) quantize_store_pair(c, kw, vw, evict_slots[r], h);
      memcpy(kw, k_new + (r * H + h) * d, sizeof(uint16_t) * (size_t)d);
      memcpy(vw, v_new + (r * H + h) * d, sizeof(uint16_t) * (size_t)d);
    }
    /* residual: token t completes the group t - R + 1 .. t (ring rows 0 .. R-1), which is
       quantized into the cache at evict_slots[r] .. evict_slots[r] + R - 1 */
    if (w->residual && (t + 1) % R == 0) {
      const uint16_t* kg = w->k + (int64_t)b * R * H * d;
      const uint16_t* vg = w->v + (int64_t)b * R * H * d;
      int64_t* gs = (int64_t*)malloc(sizeof(int64_t) * (size_t)R);
      for (int i = 0; i < R; ++i) gs[i] = evict_slots[r] + i;
      if (c->v_grouping == 1) {
        quantize_store_token_group(c, kg, vg, gs, (int64_t)H * d, (int64_t)H * d);
      } else {
        for (int i = 0; i < R; ++i)
          for (int h = 0; h < H; ++h)
            quantize_store_pair(c, kg + ((int64_t)i * H + h) * d, vg + ((int64_t)i * H + h) * d, gs[i], h);
      }
      free(gs);
    }
  }
}

void orc_decode_attention_window(const orc_cache* c, const orc_window* w, const uint16_t* q, int32_t batch,
                                 int32_t num_q_heads, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seq_lens, double softmax_scale, double* out) {
  int d = c->head_dim, P = c->page_size, H = w->num_kv_heads, S = w->sink, R = w->recent;
  int ratio = num_q_heads / c->num_kv_heads;
  double sigma = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)d);
  double* qv = (double*)malloc(sizeof(double) * (size_t)d);
  double* qr = (double*)malloc(sizeof(double) * (size_t)d);
  float* row = (float*)malloc(sizeof(float) * (size_t)d);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  for (int b = 0; b < batch; ++b) {
    int T = seq_lens[b];
    double* logit = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int j = 0; j < num_q_heads; ++j) {
      int h = j / ratio;
      double* o = out + ((int64_t)b * num_q_heads + j) * d;
      if (T <= 0) {
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        continue;
      }
      for (int i = 0; i < d; ++i) qv[i] = (double)orc_bf16_to_f32(q[((int64_t)b * num_q_heads + j) * d + i]);
      orc_rotate_dense_f64(qv, qr, d, c->hadamard_block);
      double m = -INFINITY;
      for (int t = 0; t < T; ++t) {
        double dot = 0.0;
        if (in_window(w, t, T)) { /* window token: original bf16 key, original query */
          const uint16_t* kw = w->k + (((int64_t)b * (S + R) + orc_window_slot(w, t)) * H + h) * d;
          for (int i = 0; i < d; ++i) dot += qv[i] * (double)orc_bf16_to_f32(kw[i]);
        } else {
          int64_t page = block_table[(int64_t)b * max_pages + t / P];
          dequant_row(c, 0, page, h, t % P, row);
          for (int i = 0; i < d; ++i) dot += qr[i] * (double)row[i];
        }
        logit[t] = sigma * dot;
        if (logit[t] > m) m = logit[t];
      }
      double den = 0.0;
      for (int i = 0; i < d; ++i) acc[i] = 0.0;
      for (int t = 0; t < T; ++t) {
        double wt = exp(logit[t] - m);
        den += wt;
        if (in_window(w, t, T)) {
          const uint16_t* vw = w->v + (((int64_t)b * (S + R) + orc_window_slot(w, t)) * H + h) * d;
          for (int i = 0; i < d; ++i) acc[i] += wt * (double)orc_bf16_to_f32(vw[i]);
        } else {
          int64_t page = block_table[(int64_t)b * max_pages + t / P];
          dequant_row(c, 1, page, h, t % P, row);
          for (int i = 0; i < d; ++i) acc[i] += wt * (double)row[i];
        }
      }
      for (int i = 0; i < d; ++i) o[i] = acc[i] / den;
    }
    free(logit);
  }
  free(qv);
  free(qr);
  free(row);
  free(acc);
}

void orc_attention_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t batch,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t seq_len,
                        double softmax_scale, double* out) {
  int d = head_dim;
  int ratio = num_q_heads / num_kv_heads;
  double sigma = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)d);
  double* logit = (double*)malloc(sizeof(double) * (size_t)(seq_len > 0 ? seq_len : 1));
  for (int b = 0; b < batch; ++b)
    for (int j = 0; j < num_q_heads; ++j) {
      int h = j / ratio;
      double* o = out + ((int64_t)b * num_q_heads + j) * d;
      const uint16_t* qq = q + ((int64_t)b * num_q_heads + j) * d;
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      if (seq_len <= 0) continue;
      double m = -INFINITY;
      for (int t = 0; t < seq_len; ++t) {
        const uint16_t* kk = k + (((int64_t)b * seq_len + t) * num_kv_heads + h) * d;
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += (double)orc_bf16_to_f32(qq[i]) * (double)orc_bf16_to_f32(kk[i]);
        logit[t] = sigma * dot;
        if (logit[t] > m) m = logit[t];
      }
      double den = 0.0;
      for (int t = 0; t < seq_len; ++t) {
        double w = exp(logit[t] - m);
        den += w;
        const uint16_t* vv = v + (((int64_t)b * seq_len + t) * num_kv_heads + h) * d;
        for (int i = 0; i < d; ++i) o[i] += w * (double)orc_bf16_to_f32(vv[i]);
      }
      for (int i = 0; i < d; ++i) o[i] /= den;
    }
  free(logit);
}
