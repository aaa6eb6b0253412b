/*
 * rq.h -- ResidualQuant decode attention over a looped Transformer's packed,
 * paged INT4/INT2 KV cache, on AMD Instinct MI355X (gfx950).
 *
 * The method (ResidualQuant: KV Cache Quantization for Looped Transformers
 * with 2-Bit Residuals, arXiv 2610.10381, abstract; rit.work summary of the
 * paper, section on how each pass's KV cache is restored):
 *   - the final loop's K/V of every token is the reference, stored as
 *     asymmetric INT4;
 *   - every other loop l stores r_l = R * (x_l - alpha_l * x_ref), with alpha_l
 *     the least-squares scale of the reference and R an orthogonal rotation
 *     per (layer, head, K|V) shared by all tokens and loops, quantized to INT2
 *     (INT4 under loop-wise mixed precision) with a tunable step and offset;
 *   - a token is compressed once, after its final loop; until then its K/V of
 *     every loop stay uncompressed (bf16) and are attended as a "tail";
 *   - attention rebuilds the reference and the loop's own residual on chip and
 *     never writes decompressed K/V back to memory.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or synchronizes; scratch comes from the caller's
 *     workspace. Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns at once.
 *   - On any validation failure the call returns a negative rq_status before
 *     touching memory or enqueuing work. RQ_ERR_HIP reports a failed launch.
 *   - Calls only enqueue kernels, so a sequence of them can be captured into a
 *     HIP graph (stream capture) and replayed. The first call on a device also
 *     queries device attributes (compute units, LDS per CU, kernel occupancy)
 *     and caches them: make one call on the device before capturing.
 *   - Tensor layouts are C-contiguous (row-major) in the stated index order.
 *   - Device-side indices (block ids, slots, sequence lengths) are clamped
 *     against the pool and table sizes: an out-of-range id never causes an
 *     out-of-bounds access. In the decode calls a block-table entry < 0 or
 *     >= num_blocks masks its page: that page's tokens are not attended (the
 *     output is attention over the remaining tokens). Elsewhere the affected
 *     output is unspecified.
 *
 * Packed pool format (one layer). The pool is num_blocks * num_heads slabs,
 * slab (block, head) at byte (block * num_heads + head) * slab_bytes. A slab
 * holds, for l = 0 .. num_loops-1 in order and inside each loop K (kv=0) then
 * V (kv=1), one page record of block_size tokens:
 *     codes   block_size * head_dim * b_l / 8 bytes. K records: token-major;
 *             channel i of a token sits in byte i*b_l/8 at bit
 *             (i mod (8/b_l)) * b_l. V records: ordered for the B operand of
 *             a 16x16x16 matrix instruction (tokens along k). Token t is
 *             position v = t%4 of quad u = t/4; channel c is column j = c%16
 *             of group m = c/16. "Lane" 16u + j (0..63) holds the codes
 *             (t = 4u+v, c = 16m+j) for every m and v. W = 8/b_l groups
 *             share a 32-bit word: word p holds groups W*p .. W*p+W_p-1
 *             (W_p = min(W, head_dim/16 - W*p)), with code (m = W*p+i, v) in
 *             bits [f*b_l, (f+1)*b_l), f = 2*W_p*(v%2) + W_p*(v/2) + i.
 *             Word p of all 64 lanes forms plane p (lane order,
 *             W_p*b_l/2 bytes per lane); the planes follow one another.
 *             Every plane is 256 bytes except the last one of
 *             head_dim = 96 INT2, which has 16-bit units (128 bytes).
 *     meta    block_size * (head_dim/group_size) pairs (scale, zero), token-
 *             major, meta dtype
 *     alpha   block_size values, meta dtype (only for loops l < num_loops-1)
 *     pad     zero bytes up to a multiple of 16
 * with b_l = loop_bits[l] for l < num_loops-1 and 4 for the reference loop.
 * A value decodes as code * scale + zero (per group of group_size channels);
 * loop l reconstructs as alpha * ref_hat + R^T * residual_hat.
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rq_status;
#define RQ_OK               0
#define RQ_ERR_NULL        -1   /* a required pointer is NULL */
#define RQ_ERR_SHAPE       -2   /* inconsistent or out-of-range sizes / indices */
#define RQ_ERR_UNSUPPORTED -3   /* a valid request the library has no kernel for */
#define RQ_ERR_WORKSPACE   -4   /* workspace smaller than the *_workspace_bytes figure */
#define RQ_ERR_HIP         -5   /* a HIP runtime call or kernel launch failed */
#define RQ_ERR_SCRATCH     -6   /* request needs more than RQ_NOALLOC_SCRATCH_BYTES */

/* Size of the fixed device scratch of rq_decode_attention_noalloc (one array
 * per GPU the library runs on, held until the process ends). */
#define RQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

#define RQ_DTYPE_BF16 0
#define RQ_DTYPE_F16  1
#define RQ_DTYPE_F32  2

#define RQ_MAX_LOOPS 16

#define RQ_MODE_RESIDUAL 0   /* ResidualQuant: INT4 reference + rotated residuals (default) */
#define RQ_MODE_DIRECT   1   /* baseline: every loop quantized on its own */

/* Geometry of one layer's packed cache.
 *   num_heads   H >= 1
 *   head_dim    D in {64, 96, 128}
 *   group_size  G: channels per (scale, zero) group, contiguous inside a head.
 *               Supported: D=128: 32, 64, 128; D=96: 96; D=64: 16, 32, 64.
 *   num_loops   L in [1, 16]; loop L-1 is the reference
 *   block_size  tokens per page; must be 16
 *   num_blocks  pages in the pool (>= 1)
 *   meta_dtype  RQ_DTYPE_F16 or RQ_DTYPE_F32 (scale, zero, alpha)
 *   kv_dtype    RQ_DTYPE_BF16 or RQ_DTYPE_F32 (new K/V, queries, tails)
 *   loop_bits   loop_bits[l] in {2, 4} for l < L-1 (the residual of loop l);
 *               entries from L-1 on are ignored (the reference is INT4).
 *   mode        RQ_MODE_RESIDUAL (0), or RQ_MODE_DIRECT (1): the per-loop
 *               quantization the pages compare against (arXiv 2610.10381
 *               abstract: quantizing each loop's cache separately). Every loop
 *               l < L, the last included, stores its own K/V at loop_bits[l]
 *               bits with the same quantizer and record format but no alpha
 *               field; there is no reference, alpha or rotation (rot may be
 *               NULL), and loop l's decode reads loop l's records only. */
typedef struct rq_layout {
    int32_t num_heads;
    int32_t head_dim;
    int32_t group_size;
    int32_t num_loops;
    int32_t block_size;
    int32_t num_blocks;
    int32_t meta_dtype;
    int32_t kv_dtype;
    uint8_t loop_bits[RQ_MAX_LOOPS];
    int32_t mode;
} rq_layout;

/* Tuning and instrumentation for the decode calls (all fields optional).
 *   split_pages       pages per split-K wave, 1..64 (packed decode; larger is
 *                     RQ_ERR_UNSUPPORTED); 0 = chosen by the library
 *   event_main_begin  hipEvent_t stamped when the split-K kernel starts, or NULL
 *   event_main_end    hipEvent_t stamped when it completes, or NULL
 * The events are recorded by the kernel's own dispatch (hipExtLaunchKernel),
 * so they add no separate packets to `stream`. With several loops decoded one
 * kernel per loop they bracket the last loop's kernel; in multi-loop mode,
 * the last group's kernel. */
typedef struct rq_decode_opts {
    int32_t split_pages;
    int32_t reserved;
    void   *event_main_begin;
    void   *event_main_end;
} rq_decode_opts;

/* Human-readable name of a status code (static string). */
const char *rq_status_string(rq_status status);

/* RQ_OK if `layout` is one the kernels support, else the reason. */
rq_status rq_layout_check(const rq_layout *layout);

/* Bytes of the packed pool of one layer (0 if the layout is invalid). */
size_t rq_pool_bytes(const rq_layout *layout);

/* Bytes of one page record of loop `loop` (0 if invalid). */
size_t rq_record_bytes(const rq_layout *layout, int32_t loop);

/* Byte offset of the record (block, head, loop, kv) inside the pool, or -1. */
int64_t rq_record_offset(const rq_layout *layout, int32_t block, int32_t head,
                         int32_t loop, int32_t kv);

/* Compress new tokens once their final loop has run and write them into the
 * paged pool (rit.work summary: deferred write after the final pass).
 *   pool          packed pool of this layer (rq_pool_bytes), written in place
 *   kv_new        [L][2][T][H][D] kv_dtype: every loop's K (kv=0) and V (kv=1)
 *                 of the T tokens
 *   rot           [H][2][D][D] fp32: R of (head, K|V), row-major, r = R * d.
 *                 May be NULL when L == 1.
 *   slot_mapping  [T] int64: page * 16 + offset of each token; a negative slot
 *                 skips the token
 * Per token-head and K|V, in float64: alpha = <x_l,x_ref>/<x_ref,x_ref>
 * (0 if x_ref = 0) rounded to meta_dtype; d = x_l - alpha*x_ref;
 * r = R*d; per group: scale = (max-min)/(2^b-1) and zero = min rounded to
 * meta_dtype (nearest even); code = clamp(rint((y-zero)/scale), 0, 2^b-1),
 * all codes 0 when scale == 0. Tokens of one call must have distinct slots.
 * V codes of the four tokens of a quad share 32-bit words; each token's codes
 * are written with atomic and/or on those words, so writes of different
 * tokens of one page (in one call or in calls running at once) never clobber
 * each other. */
rq_status rq_encode_pack(const rq_layout *layout, void *pool, const void *kv_new,
                         const float *rot, const int64_t *slot_mapping,
                         int32_t num_tokens, void *stream);

/* Device workspace bytes rq_encode_pack needs for num_tokens tokens: 0 for a
 * valid layout and num_tokens >= 0 (the encoder keeps its scratch in LDS, so
 * rq_encode_pack takes no workspace argument); SIZE_MAX for an invalid
 * layout or a negative num_tokens. */
size_t rq_encode_workspace_bytes(const rq_layout *layout, int32_t num_tokens);

/* Workspace bytes for rq_decode_attention(_ex) with these sizes. */
size_t rq_decode_workspace_bytes(const rq_layout *layout, int32_t n_loops,
                                 int32_t batch, int32_t max_blocks_per_seq,
                                 int32_t split_pages);

/* Pages per split that rq_decode_attention(_ex) uses when split_pages is 0,
 * for these sizes on the current device: enough split workgroups for several
 * rounds of resident workgroups on the device's compute units, the pages
 * spread evenly over the splits (per-loop calls: about 8 rounds of 4-split
 * workgroups; several non-direct loops in one call: about 14 rounds of
 * one-split workgroups), clamped to 16..64 before the even spread. The same
 * rule sizes rq_decode_workspace_bytes(..., 0), so a workspace sized on one
 * device may be too small on a device with more compute units
 * (RQ_ERR_WORKSPACE). Returns 0 for invalid arguments. */
int32_t rq_decode_auto_split_pages(const rq_layout *layout, int32_t n_loops,
                                   int32_t batch, int32_t max_blocks_per_seq);

/* Decode attention of one query per (loop, sequence, head) over the packed
 * cache plus the uncompressed current token (arXiv 2610.10381 abstract: the
 * reduced KV traffic is what speeds up decoding; rit.work summary: reference
 * and residual are rebuilt in small blocks inside attention).
 *   loops        HOST array [n_loops] of loop indices in [0, L); each entry i
 *                attends loop loops[i]'s cache with query q[i]
 *   q            [n_loops][B][H][D] kv_dtype
 *   rot          [H][2][D][D] fp32 (as in rq_encode_pack); may be NULL if every
 *                requested loop is the reference
 *   block_table  [B][max_blocks_per_seq] int32 physical page ids
 *   seq_lens     [B] int32 cached tokens per sequence
 *   tail_k/v     [n_loops][B][H][D] kv_dtype, the current token's K/V of that
 *                loop, or both NULL
 *   out          [n_loops][B][H][D] fp32
 * out = softmax(tau * q.k_hat) v_hat over the seq_len cached tokens and the
 * tail, with k_hat, v_hat the reconstruction above (tau = softmax_scale). A
 * sequence with no cached token and no tail gets a zero row. */
rq_status rq_decode_attention(const rq_layout *layout, const void *pool,
                              const int32_t *loops, int32_t n_loops, const void *q,
                              const float *rot, const int32_t *block_table,
                              const int32_t *seq_lens, int32_t batch,
                              int32_t max_blocks_per_seq, const void *tail_k,
                              const void *tail_v, float softmax_scale, float *out,
                              void *workspace, size_t workspace_bytes, void *stream);

rq_status rq_decode_attention_ex(const rq_layout *layout, const void *pool,
                                 const int32_t *loops, int32_t n_loops, const void *q,
                                 const float *rot, const int32_t *block_table,
                                 const int32_t *seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, const void *tail_k,
                                 const void *tail_v, float softmax_scale, float *out,
                                 void *workspace, size_t workspace_bytes,
                                 const rq_decode_opts *opts, void *stream);

/* Bandwidth reference of the decode call of one loop: runs the per-loop split
 * kernel's grid, ring, block-table walk and direct-to-LDS loads over the same
 * page records (reference and, for a residual loop, the loop's own records)
 * with no attention arithmetic -- every landed stage is folded into a
 * per-workgroup checksum -- so its duration is the rate at which this access
 * pattern streams the packed cache from HBM (the ceiling of the decode
 * kernel's bandwidth, ResidualQuant being bound by the bytes it reads: arXiv
 * 2610.10381 abstract). No query prep, merge or output. The checksums go to
 * the start of the workspace as uint32 [batch][H][workgroups per sequence][4
 * waves] (workgroups per sequence = ceil(max_blocks_per_seq / (4 *
 * split_pages))); the workspace is sized as for rq_decode_attention_ex with
 * one loop (rq_decode_workspace_bytes(layout, 1, batch, max_blocks_per_seq,
 * opts->split_pages)); opts as in rq_decode_attention_ex (split_pages, timing
 * events around the kernel). Nothing is written to the pool. */
rq_status rq_decode_stream_probe(const rq_layout *layout, const void *pool, int32_t loop,
                                 const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, void *workspace, size_t workspace_bytes,
                                 const rq_decode_opts *opts, void *stream);

/* Bandwidth reference of a plain contiguous read: streams `bytes` bytes of
 * device memory at `buf` (16-byte aligned, bytes a multiple of 16) with
 * 16-byte non-temporal vector loads, eight in flight per lane, over eight
 * 256-thread workgroups per compute unit, and folds them into checksum words:
 * `sink` is a device array of `sink_words` uint32 that the caller zeroes
 * first; each wave XORs its share into one word, so that on completion the
 * XOR of all sink words is the XOR of all 32-bit words of the buffer (every
 * byte read once). Give one word per wave, 32 per compute unit (fewer words
 * are allowed; waves then share them and their atomics queue). Its duration
 * is the rate at which HBM streams contiguous reads, the roof against which
 * the decode kernels and their page pattern (rq_decode_stream_probe) are
 * compared, ResidualQuant decode being bound by the bytes it reads (arXiv
 * 2610.10381, abstract). opts may be NULL; its timing events bracket the
 * kernel when set (split_pages is ignored). RQ_ERR_NULL for a null sink (or a
 * null buf with bytes > 0), RQ_ERR_SHAPE for a misaligned buffer or size or
 * sink_words < 1. */
rq_status rq_read_probe(const void *buf, size_t bytes, uint32_t *sink, int32_t sink_words,
                        const rq_decode_opts *opts, void *stream);

/* rq_decode_attention_ex without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The query records and split partials go
 * to a fixed library-owned device array of RQ_NOALLOC_SCRATCH_BYTES per GPU;
 * the call itself allocates nothing. A request whose workspace
 * (rq_decode_workspace_bytes with the same arguments and opts->split_pages)
 * exceeds that size returns RQ_ERR_SCRATCH before touching memory; larger
 * splits (opts->split_pages) or fewer loops per call shrink it. Every call on
 * one GPU uses that GPU's one array: calls that can overlap on a GPU (several
 * streams, several host threads) race on it and must be ordered by the
 * caller. The array keeps the last call's contents; nothing in it needs to
 * start at zero. The first call on a device looks up the array's address on
 * that device (make one call before capturing a graph). Arguments otherwise as
 * in rq_decode_attention_ex. */
rq_status rq_decode_attention_noalloc(const rq_layout *layout, const void *pool,
                                      const int32_t *loops, int32_t n_loops, const void *q,
                                      const float *rot, const int32_t *block_table,
                                      const int32_t *seq_lens, int32_t batch,
                                      int32_t max_blocks_per_seq, const void *tail_k,
                                      const void *tail_v, float softmax_scale, float *out,
                                      const rq_decode_opts *opts, void *stream);

/* Decode attention and the deferred compression of the current tokens in the
 * same launches (rit.work summary: a token is compressed once, after its final
 * pass; here that write runs beside the final-loop attention instead of after
 * it). Equivalent to rq_decode_attention_ex(...) followed by
 * rq_encode_pack(layout, pool, kv_new, rot, slot_mapping, num_tokens, stream),
 * with bit-identical outputs and pool bytes, provided that no new token's slot
 * holds one of the cached tokens this call attends (the new tokens are the
 * current ones, attended through tail_k/tail_v; a slot at position seq_len of
 * its sequence satisfies this). The encode's workgroups join the launch of the
 * reference loop's split kernel (per-loop calls) or of the last multi-loop
 * kernel; without a reference-loop call and with n_loops == 1 they get a launch
 * of their own after it.
 *   pool, kv_new, slot_mapping, num_tokens  as in rq_encode_pack (pool is
 *                written); num_tokens == 0 makes this rq_decode_attention_ex
 *   other arguments as in rq_decode_attention_ex. */
rq_status rq_decode_attention_encode(const rq_layout *layout, void *pool, const int32_t *loops,
                                     int32_t n_loops, const void *q, const float *rot,
                                     const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                                     int32_t max_blocks_per_seq, const void *tail_k, const void *tail_v,
                                     float softmax_scale, float *out, void *workspace,
                                     size_t workspace_bytes, const void *kv_new,
                                     const int64_t *slot_mapping, int32_t num_tokens,
                                     const rq_decode_opts *opts, void *stream);

/* Fit a residual rotation on calibration samples (HOST memory; runs on the
 * host, not on the decode path). The pages give the rotation's role (a channel
 * rotation of each loop's residual before its low-bit quantization, per
 * layer, head and K|V: arXiv 2610.10381 abstract; rit.work summary, section on
 * how each pass is restored) but no fitting rule; this one alternates the
 * method's group quantization of the rotated samples with an orthogonal
 * Procrustes step (R = U V^T for M = sum_i yhat_i d_i^T = U S V^T) and returns
 * the rotation with the lowest mean squared quantization error seen, the
 * starting one included. All arithmetic in float64.
 *   samples     [n][head_dim] float32: residual rows d = x_l - alpha * x_ref
 *   bits, group_size, meta_dtype  the quantizer (as in rq_layout)
 *   rot0        [head_dim][head_dim] float32 starting rotation (row-major, r = R d)
 *   iters       alternations, >= 0
 *   rot_out     [head_dim][head_dim] float32: the fitted rotation (may alias rot0)
 *   objective   [iters + 1] float64 or NULL: the mean squared error of rot0
 *               and of every iterate
 * head_dim <= 128 and a multiple of group_size; bits 2 or 4. */
rq_status rq_fit_rotation(const float *samples, int64_t n, int32_t head_dim, int32_t bits,
                          int32_t group_size, int32_t meta_dtype, const float *rot0, int32_t iters,
                          float *rot_out, double *objective);

/* The same fit with the calibration rows in DEVICE memory: every pass of the
 * alternation (rotate each row, quantize it with the group quantizer,
 * accumulate the squared error and M = sum_i yhat_i d_i^T) runs in float64 on
 * the GPU with a fixed summation order (deterministic); the polar factor of M
 * is taken on the host as in rq_fit_rotation. Unlike the decode calls this
 * one synchronizes `stream` once per pass (it reads M back each iteration);
 * it is a calibration step, not part of the decode path.
 *   samples     [n][head_dim] float32, DEVICE, 4-byte aligned
 *   rot0, iters, rot_out, objective: HOST, as in rq_fit_rotation
 *   workspace   DEVICE, 256-byte aligned, rq_fit_workspace_bytes(head_dim)
 *               bytes (RQ_ERR_WORKSPACE if smaller)
 * head_dim 64, 96 or 128 (RQ_ERR_UNSUPPORTED otherwise), a multiple of
 * group_size; bits 2 or 4; meta_dtype RQ_DTYPE_F16 or RQ_DTYPE_F32. Results
 * equal rq_fit_rotation's up to the summation order of float64 sums. */
rq_status rq_fit_rotation_device(const float *samples, int64_t n, int32_t head_dim, int32_t bits,
                                 int32_t group_size, int32_t meta_dtype, const float *rot0,
                                 int32_t iters, float *rot_out, double *objective, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Workspace bytes of rq_fit_rotation_device for a head dim (0 if unsupported). */
size_t rq_fit_workspace_bytes(int32_t head_dim);

/* Chunked prefill over the packed cache: a chunk of `chunk` new tokens per
 * sequence, for one loop, attends every cached token of that loop and,
 * causally, the chunk's own uncompressed K/V (query i sees chunk tokens
 * 0..i). This is the serving setting in which a prefill chunk reads the
 * compressed cache (rit.work summary, section on the infrastructure plan;
 * arXiv 2610.10381 abstract on reduced KV traffic). The queries of a chunk
 * share every page read, and both products run on the matrix cores.
 *   loop          loop index in [0, L); loop L-1 attends the reference alone
 *   chunk         queries per sequence, 1..256 (RQ_ERR_UNSUPPORTED above)
 *   q             [B][chunk][H][D] bf16
 *   rot           as in rq_decode_attention (may be NULL for the reference loop)
 *   block_table, seq_lens, batch, max_blocks_per_seq: as in rq_decode_attention;
 *                 seq_lens[b] counts the cached tokens, without the chunk
 *   chunk_k/v     [B][chunk][H][D] bf16: the chunk's own K/V of this loop, or
 *                 both NULL (then only the cache is attended)
 *   out           [B][chunk][H][D] fp32
 * Supported layouts: RQ_MODE_RESIDUAL, group_size == head_dim, kv_dtype bf16;
 * others return RQ_ERR_UNSUPPORTED, and so do calls whose launch grids would
 * exceed 65535 in a dimension (splits per sequence; batch * ceil(chunk/64);
 * ceil(batch * chunk / 16)). opts: split_pages (1..1024, larger is
 * RQ_ERR_UNSUPPORTED; 0 = the library's choice) and timing events bracketing
 * the split kernel.
 * q, chunk_k, chunk_v and the workspace must be 16-byte aligned. */
size_t rq_chunk_workspace_bytes(const rq_layout *layout, int32_t chunk, int32_t batch,
                                int32_t max_blocks_per_seq, int32_t split_pages);

rq_status rq_chunk_attention(const rq_layout *layout, const void *pool, int32_t loop,
                             int32_t chunk, const void *q, const float *rot,
                             const int32_t *block_table, const int32_t *seq_lens,
                             int32_t batch, int32_t max_blocks_per_seq,
                             const void *chunk_k, const void *chunk_v,
                             float softmax_scale, float *out, void *workspace,
                             size_t workspace_bytes, const rq_decode_opts *opts,
                             void *stream);

/* Uncompressed baseline (for the speed ratio): the same decode attention over
 * a paged bf16 cache of ONE loop, the cache against which the arXiv
 * 2610.10381 abstract states the method's accuracy (close to BF16) and its
 * fixed-batch and peak decode throughput gains.
 *   k_cache, v_cache  [num_blocks][H][16][D] bf16; num_blocks bounds the
 *                     block ids as in the packed path (an id < 0 or >=
 *                     num_blocks masks its page)
 *   q, tail_k, tail_v [B][H][D] bf16 (tails may both be NULL); out [B][H][D] fp32
 * head_dim in {64, 96, 128}; block_size must be 16. */
size_t rq_bf16_workspace_bytes(int32_t num_heads, int32_t head_dim, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t split_pages);

/* Pages per split of the bf16 baseline when split_pages is 0. Its split
 * kernel writes one partial per split, so it takes the multi-loop rule of
 * rq_decode_auto_split_pages (about 14 rounds of one-split units). Returns 0
 * for invalid arguments. */
int32_t rq_bf16_auto_split_pages(int32_t num_heads, int32_t batch,
                                 int32_t max_blocks_per_seq);

rq_status rq_bf16_decode_attention(int32_t num_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   const void *k_cache, const void *v_cache,
                                   const void *q, const int32_t *block_table,
                                   const int32_t *seq_lens, int32_t batch,
                                   int32_t max_blocks_per_seq, const void *tail_k,
                                   const void *tail_v, float softmax_scale, float *out,
                                   void *workspace, size_t workspace_bytes, void *stream);

rq_status rq_bf16_decode_attention_ex(int32_t num_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks,
                                      const void *k_cache, const void *v_cache,
                                      const void *q, const int32_t *block_table,
                                      const int32_t *seq_lens, int32_t batch,
                                      int32_t max_blocks_per_seq, const void *tail_k,
                                      const void *tail_v, float softmax_scale, float *out,
                                      void *workspace, size_t workspace_bytes,
                                      const rq_decode_opts *opts, void *stream);

/* Append tokens to a paged bf16 cache (the baseline's write step).
 *   kv_new [2][T][H][D] bf16 (K then V of one loop); slot_mapping [T] int64,
 *   negative = skip. */
rq_status rq_bf16_write(int32_t num_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, void *k_cache, void *v_cache,
                        const void *kv_new, const int64_t *slot_mapping,
                        int32_t num_tokens, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */
