/*
 * kvq oracle: a plain, slow, obviously-correct CPU reference for rotated low-bit
 * KV-cache quantization and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. The product path
 * (libkvq.so and its Python binding) never links, imports or executes it, and it
 * shares no code, header, table or constant with that path.
 *
 * What it follows (no page prints formulas or code; the readings are fixed here):
 *  - SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving,
 *    Abstract: keys and values are quantized token-wise to 4 bits after a
 *    block-diagonal Hadamard rotation, written straight into a paged KV layout.
 *  - Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, Abstract:
 *    the orthogonal transform applied to keys is applied to queries too, so
 *    query-key dot products are unchanged; 2-bit caches are in scope.
 *  - InnerQ: Hardware-Aware Tuning-Free Quantization of KV Cache for Large
 *    Language Models, Abstract: group-wise quantization with asymmetric
 *    (scale + zero) groups.
 *  - "Is QuaRot superseded?" (scholarfeed), critique quotes: INT2 has four levels;
 *    the INT2 methods compared sit at about 2.25 bits per element with group 128.
 *
 * Arithmetic contract (fp32, round-to-nearest-even everywhere, no fused ops
 * except the single fmaf of dequantization):
 *   rotate  : per block of n channels, butterfly with strides 1,2,4,..,n/2 in that
 *             order, (a,b) -> (a+b, a-b); then multiply by c_n = fp32 nearest 1/sqrt(n).
 *   group   : mn = min, mx = max; s32 = (mx - mn) / (2^bits - 1);
 *             scale = fp16(s32); zero = fp16(mn + 0.0f).
 *   codes   : s = float(scale), z = float(zero); s == 0 -> all 0; else
 *             inv = 1/s; u = (x - z) * inv (two roundings); code = clamp(rint(u), 0, 2^bits-1).
 *   hybrid  : (quant_mode 1) per group also the symmetric pair scale = fp16(max|x| /
 *             (2^(bits-1) - 1)), zero = -2^(bits-1) * scale, codes by the same formula;
 *             the pair with the smaller largest |x - xhat| is stored (asymmetric on a tie).
 *   dequant : xhat = fmaf(code, s, z).
 *   attention (fp64): qr = dense (H/sqrt(n)) q per block; logit_t = sigma * qr . khat_t;
 *             o = sum_t exp(logit_t - max) vhat_t / sum_t exp(logit_t - max).
 *
 * Cache layout (all byte offsets; RB = head_dim*bits/8 bytes per token row, a multiple
 * of 16, NG = head_dim/group_size groups, P = page_size, a multiple of 16; tokens are
 * stored in 16-token tiles):
 *   row base      u = page*Hkv + h
 *   packed row    byte k holds channels (INT4) 2k at bits 0-3, 2k+1 at 4-7;
 *                 (INT2) 4k+e at bits 2e.
 *   K codes       [u][P/16][RB/16][16][16]    each tile's rows cut into 16-byte chunks,
 *                                             chunk-major: chunk j, token o, byte b at
 *                                             (j*16 + o)*16 + b.
 *   K meta        [u][P][NG] x {u16 scale, u16 zero}  (scale in the low half)
 *   V codes       [u][P/16][RB/2][8][2][2]    the row cut into 16-bit words; per tile and
 *                                             word, the 8 token pairs each store both
 *                                             tokens' low bytes then both high bytes:
 *                                             word w, token o, byte b at
 *                                             w*32 + (o/2)*4 + b*2 + o%2.
 *   V meta        [u][P/16][2][NG][2][4] x {u16 scale, u16 zero}: token
 *                                             o = 8*half + 4*part + i of group g at
 *                                             entry ((part*NG + g)*2 + half)*4 + i.
 *   V meta, token groups (v_grouping 1, head_dim 128, P a multiple of G):
 *                 [u][P/G][128] x {u16 scale, u16 zero}: channel c of token group j of
 *                 the page at entry 8n + t, c = 4(n + 16(t>>2)) + 2(t&1) + ((t>>1)&1)
 *                 (INT4) or 8n + (t>>1) + 4(t&1) (INT2).
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats (IEEE 754 binary16 / bfloat16, written from the definitions) ---- */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_f16(float x); /* round to nearest, ties to even; subnormals; inf; nan */
float orc_f16_to_f32(uint16_t h);
void orc_f32_to_f16_array(const float* x, uint16_t* out, int64_t n);
void orc_f16_to_f32_array(const uint16_t* h, float* out, int64_t n);
float orc_fmaf(float a, float b, float c);

/* ---- Walsh-Hadamard ---- */
void orc_hadamard_sylvester(int n, int32_t* H);      /* H[i*n+j] = (-1)^popcount(i&j) */
void orc_fwht_unnormalized(float* x, int n);         /* butterfly, ascending strides */
float orc_rotation_constant(int n);                  /* fp32 nearest to 1/sqrt(n) */
void orc_rotate(float* x, int d, int block);         /* block-diagonal rotation of d channels */
void orc_rotate_dense_f64(const double* x, double* y, int d, int block);

/* ---- quantizer (one token row of d channels, already rotated when needed) ---- */
void orc_quantize_row(const float* x, int d, int bits, int group,
                      uint8_t* codes, uint16_t* scale, uint16_t* zero);
/* hybrid (InnerQ, Abstract): per group the asymmetric pair above or the symmetric pair
   scale = fp16(max|x| / (2^(bits-1) - 1)), zero = -2^(bits-1) * scale, whichever has the
   smaller largest |x - fmaf(code, scale, zero)| (asymmetric on a tie); codes by the same
   formula from the chosen pair */
void orc_quantize_row_hybrid(const float* x, int d, int bits, int group,
                             uint8_t* codes, uint16_t* scale, uint16_t* zero);
void orc_pack_row(const uint8_t* codes, int d, int bits, uint8_t* packed);
void orc_unpack_row(const uint8_t* packed, int d, int bits, uint8_t* codes);

/* ---- cache ---- */
typedef struct {
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t bits;
  int32_t group_size;
  int32_t hadamard_block; /* 0 = none */
  int32_t page_size;
  int64_t num_pages;
  uint8_t* k_codes;
  uint8_t* k_meta;
  uint8_t* v_codes;
  uint8_t* v_meta;
  int32_t quant_mode; /* 0 = asymmetric min/max, 1 = hybrid symmetric/asymmetric */
  int32_t v_grouping; /* 0 = V groups of G channels of a token; 1 = of G tokens of a channel */
} orc_cache;

/* bytes of each plane: 0 = K codes, 1 = K meta, 2 = V codes, 3 = V meta */
int64_t orc_plane_bytes(const orc_cache* c, int plane);
/* returns 0 on success, nonzero when the description is outside the oracle's domain */
int orc_check_cache(const orc_cache* c);

/* k_new, v_new: bf16 [n][Hkv][d]; slots[r] = page*P + offset. With v_grouping 1, rows come
   in whole groups of G consecutive tokens (slots[r..r+G-1] = slots[r] + 0..G-1, slots[r] a
   multiple of G): keys per token, values per (group, channel). */
void orc_quantize_append(const orc_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                         const int64_t* slots, int64_t n);
/* which: 0 = K, 1 = V; out: float [n][Hkv][d] */
void orc_dequantize(const orc_cache* c, int which, const int64_t* slots, int64_t n, float* out);
/* q: bf16 [B][Hq][d]; block_table [B][max_pages]; out: double [B][Hq][d].
   softmax_scale <= 0 means 1/sqrt(d). */
void orc_decode_attention(const orc_cache* c, const uint16_t* q, int32_t batch, int32_t num_q_heads,
                          const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                          double softmax_scale, double* out);
/* Query-channel pruning (Dual-QK, Abstract): as orc_decode_attention, with bit j of
   keep_mask[b * Hkv + h] keeping channels j*W .. j*W + W - 1 of the rotated query,
   W = 128 / bits (one 16-byte chunk of a packed key row); other channels are zero. */
void orc_decode_attention_pruned(const orc_cache* c, const uint16_t* q, int32_t batch, int32_t num_q_heads,
                                 const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                 double softmax_scale, const int32_t* keep_mask, double* out);
/* energy [B][Hkv][d*bits/128]: per chunk, sum over the kv head's query heads of qr^2 */
void orc_prune_energy(const orc_cache* c, const uint16_t* q, int32_t batch, int32_t num_q_heads, double* energy);
/* ---- high-precision windows (InnerQ, Abstract) ----
   The first `sink` and the last `recent` tokens of every sequence stay in bf16 (keys in
   the original basis); token t sits in window slot t (t < sink) or
   sink + (t - sink) % recent. Tokens sink <= t < T - recent are in the quantized cache,
   at their own slots. */
typedef struct {
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t sink;
  int32_t recent; /* >= 1 */
  int32_t batch;
  uint16_t* k; /* bf16 [batch][sink + recent][Hkv][d] */
  uint16_t* v;
  int32_t residual; /* 1: sink 0, a ring of `recent` rows holding the incomplete last group
                       of `recent` tokens (T mod recent of them); a group is quantized when
                       its last token arrives */
} orc_window;

int orc_window_slot(const orc_window* w, int t);
/* One new token per row r: sequence seqs[r], position positions[r] (= tokens before it).
   A full recent window first moves its oldest token (position t - recent) into the cache
   at evict_slots[r]. */
void orc_window_append(const orc_cache* c, const orc_window* w, const uint16_t* k_new, const uint16_t* v_new,
                       const int32_t* seqs, const int32_t* positions, const int64_t* evict_slots, int64_t n);
/* Attention over window tokens (bf16, original query) and cache tokens (as
   orc_decode_attention) together; seq_lens counts all tokens. */
void orc_decode_attention_window(const orc_cache* c, const orc_window* w, const uint16_t* q, int32_t batch,
                                 int32_t num_q_heads, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seq_lens, double softmax_scale, double* out);
/* fp64 attention over unquantized bf16 K/V ([B][T][Hkv][d] contiguous), no rotation:
   the loss-free reference the quantized cache approximates (information only). */
void orc_attention_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t batch,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t seq_len,
                        double softmax_scale, double* out);

#ifdef __cplusplus
}
#endif
#endif
