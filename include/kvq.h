/*
 * kvq: rotated low-bit (INT4 / INT2) KV-cache quantize-append and split-K decode
 * attention for AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The method:
 *  - SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving,
 *    Abstract: keys and values are quantized token-wise to 4 bits after a
 *    block-diagonal Hadamard rotation, by a fused rotation-quantization kernel that
 *    writes straight into a paged KV layout; attention then runs over that cache.
 *  - Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, Abstract:
 *    the transform applied to keys is applied to queries as well, which leaves every
 *    query-key dot product unchanged; 2-bit caches are in scope.
 *  - InnerQ: Hardware-Aware Tuning-Free Quantization of KV Cache for Large Language
 *    Models, Abstract: group-wise asymmetric quantization whose dequantization is
 *    folded into the decode-time vector-matrix products.
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers the caller owns (e.g. torch tensors'
 *    data_ptr()); the library never allocates, frees or retains them. `stream` is a
 *    hipStream_t (NULL = the null stream). Calls are asynchronous on that stream and
 *    return before the work finishes; buffers must stay alive until it does.
 *  - The library holds no state between calls and is safe to call from several host
 *    threads (kernels on one stream run in order; concurrent calls that write the
 *    same cache memory race, as any two kernels would).
 *  - Every argument check is done on the host before any launch. On any status other
 *    than KVQ_OK nothing was launched, except KVQ_ERR_HIP, which reports a failed
 *    launch. Device-side contents are not checked: a slot outside the page pool,
 *    duplicate slots in one append, seq_len beyond the pages of its block-table row,
 *    or non-finite inputs give undefined results. Finite queries of any magnitude are
 *    in the domain as long as the logits softmax_scale * (R q) . khat are finite in fp32.
 *  - Supported today: head_dim 128; bits 4 or 2; group_size 32, 64 or 128;
 *    hadamard_block 0 (off) or a power of two from 2 to 128; GQA ratio
 *    num_q_heads / num_kv_heads of 1, 2 or 4; page_size a multiple of 16;
 *    num_pages * num_kv_heads * page_size / 16 below 2^32 (the decode kernels index
 *    the 16-token tiles of one kv head in 32 bits); max_seq_len up to 2^30. Other
 *    well-formed descriptions return KVQ_ERR_UNSUPPORTED.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = 1,     /* null/misaligned pointer, inconsistent sizes */
  KVQ_ERR_UNSUPPORTED = 2, /* well-formed but not built (see the list above) */
  KVQ_ERR_WORKSPACE = 3,   /* workspace smaller than kvq_decode_workspace_bytes() */
  KVQ_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} kvq_status;

/*
 * A quantized KV cache: four device planes the caller allocates (sizes from
 * kvq_cache_plane_bytes) and zero-fills once. Rows are addressed by slot =
 * page * page_size + offset. With u = page * num_kv_heads + kv_head, RB =
 * head_dim * bits / 8 bytes of codes per token and NG = head_dim / group_size:
 *
 * Tokens are grouped in 16-token tiles (page_size is a multiple of 16):
 *   k_codes  uint8 [u][page_size/16][RB/16][16][16] each tile's packed rows cut into
 *            16-byte chunks, chunk-major (byte b of chunk j of token o at
 *            (j*16 + o)*16 + b of the tile), so a load of one channel range of a
 *            tile's tokens reads whole cache lines
 *   k_meta   half2 [u][page_size][NG]          {scale (low 16 bits), zero (high)}
 *   v_codes  uint8 [u][page_size/16][RB/2][8][2][2] each tile's packed rows cut into
 *            16-bit words, word-major; within a word the 8 token pairs keep both
 *            tokens' low bytes, then both high bytes (byte b of word w of token o at
 *            w*32 + (o/2)*4 + b*2 + o%2 of the tile)
 *   v_meta   half2 [u][page_size/16][2][NG][2][4] {scale, zero}; token
 *            o = 8*half + 4*part + i of group g at entry ((part*NG + g)*2 + half)*4 + i
 *            of the tile
 *
 * With v_grouping 1 (InnerQ, Abstract: groups along the inner dimension of the value
 * product) the value codes keep the layout above and v_meta holds one {scale, zero} per
 * (group of G tokens of a page, channel):
 *   v_meta   half2 [u][page_size/G][128]: channel c of token group j at entry 8n + t,
 *            c = 4(n + 16(t>>2)) + 2(t&1) + ((t>>1)&1) at INT4, 8n + (t>>1) + 4(t&1) at
 *            INT2 (n = 0..15, t = 0..7); the plane has the same size.
 * Keys keep their per-token groups.
 *
 * Packed rows are little-endian: INT4 channel 2k in the low nibble of byte k and
 * 2k+1 in the high nibble; INT2 channel 4k+e in bits 2e..2e+1 of byte k.
 * A contiguous cache is the special case of one page of capacity tokens per
 * sequence. Keys are stored in the rotated basis; values are not rotated.
 * All four planes must be 16-byte aligned.
 */
typedef struct kvq_cache {
  int32_t head_dim;       /* d */
  int32_t num_kv_heads;   /* Hkv */
  int32_t bits;           /* 4 or 2 */
  int32_t group_size;     /* G: channels sharing one scale/zero, divides d */
  int32_t hadamard_block; /* 0 = no rotation; else power of two dividing d */
  int32_t page_size;      /* P tokens per page, multiple of 16 */
  int64_t num_pages;      /* pages in the pool */
  void* k_codes;
  void* k_meta;
  void* v_codes;
  void* v_meta;
  int32_t quant_mode;     /* 0 = asymmetric min/max groups; 1 = hybrid (below) */
  int32_t v_grouping;     /* 0 = value groups of G channels of a token; 1 = of G tokens of a
                             channel (InnerQ, below; page_size a multiple of G) */
} kvq_cache;

/* Bytes of one plane: 0 = k_codes, 1 = k_meta, 2 = v_codes, 3 = v_meta.
   Host-only; returns -1 for an invalid description or plane index. */
int64_t kvq_cache_plane_bytes(const kvq_cache* cache, int32_t plane);

/*
 * Quantize and append n_new tokens (SAW-INT4, Abstract: fused rotation +
 * quantization into the paged layout).
 *   k_new, v_new : bf16 [n_new][Hkv][d], 16-byte aligned, contiguous.
 *   slots        : int64 [n_new] device array, slot of each token (page*P + offset).
 * For every (token, kv head): K is rotated by the block-diagonal Walsh-Hadamard
 * matrix (Sylvester order, fp32 butterfly with strides 1,2,..,n/2 then a multiply
 * by the float nearest 1/sqrt(n)); then K and V are quantized per group of G
 * channels: scale = fp16((max-min)/(2^bits-1)), zero = fp16(min) (a -0 zero is
 * stored as +0), code = clamp(rint((x-zero)*(1/scale)), 0, 2^bits-1) (all codes 0
 * when scale is 0), all in fp32 with round-to-nearest-even. Results are bit-exact
 * functions of the inputs. n_new == 0 is a no-op returning KVQ_OK.
 */
kvq_status kvq_quantize_append(const kvq_cache* cache, const void* k_new, const void* v_new,
                               const int64_t* slots, int64_t n_new, void* stream);
/*
 * v_grouping 1: n_new must be a multiple of G (else KVQ_ERR_INVALID); rows come in whole
 * token groups, rows j*G .. j*G+G-1 at the consecutive slots slots[j*G] + 0 .. G-1 of one
 * page, slots[j*G] a multiple of G (device contents, not checked). Keys are quantized per
 * token; each channel of a group's values forms one group, by the same formula.
 *
 * quant_mode 1, hybrid groups (InnerQ, Abstract: each group chooses symmetric or
 * asymmetric quantization from its own statistics): besides the pair above, a symmetric
 * pair scale = fp16(fl32(max|x| / (2^(bits-1) - 1))), zero = -2^(bits-1) * scale (exact)
 * with codes by the same formula; the group stores the pair whose largest
 * |x - fmaf(code, scale, zero)| (fp32) is smaller, the asymmetric one on a tie. Both
 * are stored as {scale, zero}, so decode and dequantize read either alike. Applies to
 * every append into the cache (kvq_quantize_append and the window append).
 */

/*
 * Workspace bytes kvq_decode_attention (and kvq_decode_attention_reference) need for
 * these sizes. num_splits > 0 (fixed partitions): fp32 split partials
 * [batch][num_q_heads][splits][d + 2]. num_splits 0 = the library's choice, made the
 * same way for the same arguments on the same device: kvq_decode_attention then plans
 * balanced partitions on the device (below), partials [num_q_heads][U][d + 2] with U a
 * bound on one kv head's partitions, then two int32 per sequence (the split kernel's
 * record of where each sequence's partials start, for the combine); the reference
 * kernel takes fixed partitions of up
 * to 2048 tokens; the size covers both. Returns 0 for an invalid description and for
 * sizes that do not fit in size_t (the decode calls then return KVQ_ERR_INVALID).
 *
 * Balanced partitions (kvq_decode_attention, _timed, _pruned and _window with
 * num_splits 0 and 2 <= batch <= 256): one partition length L for the whole call, computed on
 * the device from seq_lens: with c_b = ceil(span_b / 256) (span_b = the tokens of
 * sequence b the split kernel covers), C = sum_b c_b and U = ceil(8 * CUs / Hkv) (one
 * round of the kernel's waves per kv head), L = 256 k where k starts at ceil(C / U)
 * (at least 1) and grows until sum_b ceil(c_b / k) <= U, at most 64; sequence b gets
 * ceil(span_b / L) partitions. Equal-length partitions keep the GPU evenly loaded
 * whatever the mix of sequence lengths, with no host-side knowledge of the lengths.
 */
size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                  int32_t max_seq_len, int32_t num_splits);

/* The number of split-K partitions (per sequence of max_seq_len tokens) that
   kvq_decode_attention uses with these arguments; with num_splits 0, the count for a
   batch whose sequences all have max_seq_len tokens (a ragged batch's long sequences
   get more, shorter partitions). 0 for an invalid description. */
int32_t kvq_decode_num_splits(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                              int32_t max_seq_len, int32_t num_splits);

/*
 * Decode-phase GQA attention over the quantized cache (one query token per
 * sequence). Query head j reads kv head j / (num_q_heads / Hkv).
 *   q           : bf16 [batch][num_q_heads][d] in the ORIGINAL basis (post-RoPE); the
 *                 kernel applies the keys' rotation to it (Dual-QK, Abstract).
 *   block_table : int32 [batch][max_pages_per_seq], physical page of each logical page.
 *   seq_lens    : int32 [batch] on the device: tokens to attend (0 gives a zero row).
 *   max_seq_len : host upper bound of seq_lens, used to size the split-K grid
 *                 (seq_lens above it give undefined output rows, but no access outside
 *                 the buffers).
 *   softmax_scale: 0 means 1/sqrt(d).
 *   num_splits  : 0 = automatic (balanced partitions planned on the device, see
 *                 kvq_decode_workspace_bytes); otherwise the number of token partitions
 *                 of a max_seq_len sequence (rounded to the kernel's 32-token
 *                 granularity), the same length for every sequence.
 *   workspace   : device scratch of at least kvq_decode_workspace_bytes() bytes,
 *                 16-byte aligned; overwritten.
 *   out         : fp32 [batch][num_q_heads][d]:
 *                 softmax(scale * (R q) . khat_t) weighted sum of vhat_t, where khat/vhat
 *                 are the dequantized rows fma(code, scale, zero).
 * Two kernels run: split-K partial attention (online softmax, exp2 domain), then a
 * log-sum-exp combine of the partials.
 */
kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                int32_t num_splits, void* workspace, size_t workspace_bytes, float* out,
                                void* stream);

/*
 * Same as kvq_decode_attention, and additionally records the hipEvent_t
 * `split_begin` at the start and `split_end` at the end of the split-K kernel on
 * `stream` (either may be NULL), as part of that kernel's dispatch (hipExtLaunchKernel),
 * so a caller can time that kernel alone with hipEventElapsedTime. For benchmarking.
 */
kvq_status kvq_decode_attention_timed(const kvq_cache* cache, const void* q, int32_t batch,
                                      int32_t num_q_heads, const int32_t* block_table,
                                      int32_t max_pages_per_seq, const int32_t* seq_lens,
                                      int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                      void* workspace, size_t workspace_bytes, float* out, void* stream,
                                      void* split_begin, void* split_end);

/*
 * One decode step with the append fused into the split-K kernel (SAW-INT4, Abstract:
 * rotation and quantization fused into one kernel that writes the paged layout): the
 * same results as kvq_quantize_append of each sequence's new token at the slot of its
 * position seq_lens[b] - 1 (page block_table[b][pos / P], offset pos % P), followed by
 * kvq_decode_attention with the same arguments, in one split-K launch and the combine.
 *   k_new, v_new : bf16 [batch][Hkv][d], 16-byte aligned, contiguous: row b is the new
 *                  token of sequence b (sequences with seq_lens[b] <= 0 append nothing).
 * The unit whose partition holds position seq_lens[b] - 1 quantizes those rows before it
 * reads its blocks, so the rows are bit-identical to kvq_quantize_append's and the
 * output bit-identical to the two calls'. Every other argument, the workspace and the
 * errors are those of kvq_decode_attention; in addition KVQ_ERR_INVALID for a null or
 * misaligned k_new / v_new, KVQ_ERR_UNSUPPORTED for a cache with v_grouping 1 (value
 * token groups are appended a group at a time). Requires seq_lens[b] <= max_seq_len for
 * the append to happen (above it the row is undefined, as is the output).
 */
kvq_status kvq_decode_step(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                           int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                           float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                           float* out, void* stream);

/* kvq_decode_step with hipEvent_t records around its split-K kernel, as
   kvq_decode_attention_timed. For benchmarking. */
kvq_status kvq_decode_step_timed(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                 float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                                 float* out, void* stream, void* split_begin, void* split_end);

/*
 * The same computation through a second, plain-VALU split-K kernel (fp32
 * dequantization and dot products, scores staged in LDS) instead of the MFMA
 * kernel. For cross-checking the fast path; partitions longer than 2048 tokens
 * return KVQ_ERR_UNSUPPORTED.
 */
kvq_status kvq_decode_attention_reference(const kvq_cache* cache, const void* q, int32_t batch,
                                          int32_t num_q_heads, const int32_t* block_table,
                                          int32_t max_pages_per_seq, const int32_t* seq_lens,
                                          int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                          void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): kvq_decode_attention without the
 * workspace arguments. The split partials and the balanced plan's table go to a device
 * array the library owns, KVQ_NOALLOC_WORKSPACE_BYTES (32 MiB) per device, held from the
 * first call on a device until the process ends; the call allocates nothing. A call
 * whose matrix-kernel workspace would exceed it returns KVQ_ERR_WORKSPACE before any
 * launch (kvq_decode_workspace_bytes() is an upper bound of that size). Every call on a
 * device shares the one array: calls that overlap on one GPU (other streams or host
 * threads) race and must be serialised by the caller. Nothing in the array needs to
 * start at zero: every byte the combine reads is written by the same call's split kernel.
 * Same arguments and the same result, bit for bit, as kvq_decode_attention otherwise.
 */
#define KVQ_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                                        const int32_t* block_table, int32_t max_pages_per_seq,
                                        const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                        int32_t num_splits, float* out, void* stream);

/*
 * Decode attention with dynamic query-channel pruning of key reads (Dual-QK, Abstract:
 * query-channel pruning further reduces key-cache reads). Arguments as
 * kvq_decode_attention (same workspace size), plus:
 *   keep_chunks : 1 .. head_dim * bits / 128 (4 at INT4, 2 at INT2). Packed key rows are
 *                 read in 16-byte chunks of 128 / bits channels (32 at INT4, 64 at INT2).
 *                 Per (sequence, kv head) the rotated query keeps the keep_chunks chunks
 *                 with the largest sum of squared rotated-query channels over the kv
 *                 head's query heads (fp32; ties keep the lower chunk); every other
 *                 channel counts as zero in the scores, and those key chunks are not read
 *                 (except in the first three 32-token blocks of each partition, read
 *                 before the query is ranked). Values are not pruned.
 *   chunk_mask  : int32 [batch][Hkv] device array or NULL; receives the kept chunks
 *                 (bit j = chunk j) of every sequence with seq_len > 0.
 *   split_begin, split_end : hipEvent_t recorded at the start and end of the split-K
 *                            kernel (as kvq_decode_attention_timed), or NULL.
 * out = softmax(scale * (R q restricted to the kept channels) . khat_t) weighted sum of
 * vhat_t. keep_chunks equal to the number of chunks gives kvq_decode_attention's result.
 */
kvq_status kvq_decode_attention_pruned(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                                       const int32_t* block_table, int32_t max_pages_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                       int32_t num_splits, int32_t keep_chunks, int32_t* chunk_mask,
                                       void* workspace, size_t workspace_bytes, float* out, void* stream,
                                       void* split_begin, void* split_end);

/*
 * Dequantize n stored rows (InnerQ, Abstract: asymmetric group quantization with a scale
 * and a zero point per group; SAW-INT4, Abstract: token-wise INT4 keys and values):
 * out fp32 [n][Hkv][d] = fma(code, scale, zero) per element, one fp32 rounding, read from
 * the rows at `slots` (int64 device array, page * P + offset, not checked). which = 0
 * reads K (in the rotated basis), 1 reads V (value token groups: each channel's
 * {scale, zero} of its token group). Bit-exact. For checks and export.
 */
kvq_status kvq_dequantize(const kvq_cache* cache, int32_t which, const int64_t* slots, int64_t n,
                          float* out, void* stream);

/*
 * High-precision windows (InnerQ, Abstract: the tokens of a recent window and the
 * attention-sink tokens are kept in high precision). The first `sink` tokens and the
 * last `recent` tokens of every sequence stay in bf16, keys in the ORIGINAL basis
 * (not rotated); tokens sink <= t < T - recent live quantized in the cache at their own
 * slots. Token t of sequence b sits in window row
 *   w = t                               (t < sink)
 *   w = sink + (t - sink) % recent      (t >= sink, a ring of `recent` rows)
 * of the planes k, v: bf16 [batch][sink + recent][Hkv][d], 16-byte aligned, owned and
 * zero-filled (or written directly) by the caller, sizes from kvq_window_plane_bytes.
 * Supported: sink a multiple of 16 (the cache's tile), recent >= 1,
 * sink + recent <= 1024.
 */
typedef struct kvq_window {
  int32_t sink;   /* S */
  int32_t recent; /* R */
  int32_t batch;  /* sequences the planes hold */
  void* k;
  void* v;
  int32_t residual; /* 0 = sink and recent windows as above; 1 = residual (below) */
} kvq_window;

/*
 * residual 1 (sink must be 0, page_size a multiple of R): the ring of R rows holds the incomplete last group of R
 * tokens in bf16, token t in row t % R, T % R tokens of them; the tokens before are in
 * the cache. Appending token t with (t + 1) % R == 0 completes the group t-R+1 .. t,
 * which is then quantized from the ring into the cache at evict_slots[r] + 0 .. R-1
 * (its tokens' consecutive slots); no token is evicted otherwise. Decode scores the
 * residual tokens like window tokens. A cache with v_grouping 1 needs a residual window
 * with R == group_size (other windows return KVQ_ERR_UNSUPPORTED).
 */

/* Bytes of one window plane (k or v) for this cache's d and Hkv; -1 if invalid. */
int64_t kvq_window_plane_bytes(const kvq_cache* cache, const kvq_window* window);

/*
 * Append one new token to each of n_new sequences through the windows.
 *   k_new, v_new : bf16 [n_new][Hkv][d] in the original basis, 16-byte aligned.
 *   seqs         : int32 [n_new] device array, sequence (row of the window planes);
 *                  at most one row per sequence in one call.
 *   positions    : int32 [n_new] device array, position t of the token (= tokens the
 *                  sequence held before it).
 *   evict_slots  : int64 [n_new] device array, cache slot of token t - recent.
 * The token is written to its window row. When t >= sink + recent the ring row already
 * holds token t - recent, which leaves the window: before being overwritten it is
 * rotated and quantized (exactly as kvq_quantize_append does) into evict_slots[r];
 * otherwise evict_slots[r] is not read. n_new == 0 is a no-op returning KVQ_OK.
 */
kvq_status kvq_window_append(const kvq_cache* cache, const kvq_window* window, const void* k_new,
                             const void* v_new, const int32_t* seqs, const int32_t* positions,
                             const int64_t* evict_slots, int64_t n_new, void* stream);

/* Workspace bytes of kvq_decode_attention_window: the split partials of the quantized
   span (as kvq_decode_workspace_bytes describes, for the matrix kernel), then the window
   partials [batch][num_q_heads][d + 2] fp32; 0 for an invalid description. */
size_t kvq_decode_window_workspace_bytes(const kvq_cache* cache, const kvq_window* window, int32_t batch,
                                         int32_t num_q_heads, int32_t max_seq_len, int32_t num_splits);

/*
 * Decode attention over the windows and the cache together: one softmax over all
 * seq_lens[b] tokens, window tokens scored with the original query against their bf16
 * keys, cache tokens with the rotated query against the dequantized keys (Dual-QK,
 * Abstract), values likewise. Arguments as kvq_decode_attention, plus the window
 * (batch <= window->batch; sequence b uses window row b). num_splits partitions the
 * quantized span of a max_seq_len sequence (max_seq_len - sink - recent tokens).
 * Three kernels: the split-K kernel over the quantized span, one partial over the
 * window tokens, the combine.
 */
kvq_status kvq_decode_attention_window(const kvq_cache* cache, const kvq_window* window, const void* q,
                                       int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                       int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                       float softmax_scale, int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, float* out, void* stream);

/*
 * Same as kvq_decode_attention_window, and additionally records the hipEvent_t
 * `split_begin` at the start and `split_end` at the end of the split-K kernel over the
 * quantized span on `stream` (either may be NULL), as kvq_decode_attention_timed does.
 * For benchmarking.
 */
kvq_status kvq_decode_attention_window_timed(const kvq_cache* cache, const kvq_window* window, const void* q,
                                             int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                                             int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                             void* workspace, size_t workspace_bytes, float* out,
                                             void* stream, void* split_begin, void* split_end);

/*
 * Read-bandwidth probe, a measurement aid (InnerQ, Abstract, and SAW-INT4, Abstract: the
 * cost of decode lies in reading the KV cache from memory, so the decode kernel is
 * measured against the read rate the device sustains). Reads the `bytes` bytes at `src`
 * (device memory, 16-byte aligned, bytes a multiple of 16) once, with 16-byte loads laid
 * out as the decode kernel's (consecutive lanes on consecutive 16-byte pieces, so each
 * wave-wide load covers whole cache lines), non-temporal when `nontemporal` is 1, from
 * workgroups_per_cu (1..32) workgroups of 256 threads per compute unit. Nothing is
 * written except, with negligible probability, the first dword of `sink` (a device
 * word the caller provides). Records the hipEvent_t `ev_begin` / `ev_end` (either may be
 * NULL) at the start and end of the probe kernel on `stream`, as part of its dispatch.
 * bytes == 0 is a no-op returning KVQ_OK.
 */
kvq_status kvq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t nontemporal,
                           int32_t workgroups_per_cu, void* stream, void* ev_begin, void* ev_end);

/* Static description of a status code. */
const char* kvq_status_string(kvq_status status);

/* Library version string. */
const char* kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
