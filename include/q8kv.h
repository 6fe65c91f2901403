/*
 * q8kv -- single-query decode attention over a paged int8 ("q8") KV cache,
 * one online-softmax pass, for AMD Instinct MI355X (gfx950).
 *
 * The computation is the one walked through on the page "Day 9-2:
 * flash_attn_single_q_q8_neon" (trdm.cn), section 2:
 *   segment 1  each query head is quantised once to int8 in 32-element
 *              blocks, scale = absmax * fp32(1/127), codes = truncate(clamp(
 *              q * (127 / absmax), -128, 127)), absmax < 1e-6 treated as 1;
 *   segment 2  every cached token is scored with int8 x int8 -> int32 dot
 *              products, one per 32-block, rescaled in fp32 by the block's q
 *              scale, the token's K scale and the softmax scale; a running
 *              maximum M and exp-sum S rescale the accumulated
 *              V_int8 * (weight * v_scale) whenever M grows, so each K/V row
 *              is read once;
 *   segment 3  the output is the accumulator divided by S.
 * The page's per-token rule is applied per tile of tokens and per partition
 * of the context (the same rescale rule on whole groups), which changes the
 * fp32 rounding but not the mathematics.
 *
 * Memory layouts (all tensors are caller-owned device memory, densely
 * packed, naturally aligned -- 16 bytes for pages and scales):
 *   q, out        fp32  [batch][n_q_heads][hd] row-major
 *   k_pages,
 *   v_pages       int8  [num_blocks][n_kv_heads][kv_bs / 16][16 * hp]: each
 *                       page (block, kv head) is a run of 16-row sub-tiles,
 *                       and a sub-tile's 16 x hp bytes are stored in the
 *                       matrix-core operand order below, so that one 16-byte
 *                       load per lane of a 64-lane wave reads 1 KB of
 *                       consecutive bytes;
 *   k_scale,
 *   v_scale       fp32  [num_blocks][n_kv_heads][kv_bs]  dequantisation
 *                       factor absmax * fp32(1/127) of that row
 *   block_table   int32 [batch][max_blocks_per_seq]  physical block of each
 *                       logical block of a sequence; entries past a
 *                       sequence's last block may be read (the whole row
 *                       must be readable) but never address a page (-1 by
 *                       convention)
 *   seq_lens      int32 [batch]  tokens cached for each sequence
 * Token t of sequence b lives in physical block block_table[b][t / kv_bs] at
 * row t % kv_bs.  Query head h reads kv head h / (n_q_heads / n_kv_heads).
 *
 * Page width.  hp, the bytes of one page row, is the head size hd rounded
 * up to 64, 128 or 256 (hd 32 -> 64, 96 -> 128, 160 / 192 / 224 -> 256):
 * the matrix-core steps contract 64 bytes at a time.  Columns hd .. hp - 1
 * of every written row hold zero codes, which add nothing to a dot product
 * and leave each row's absmax unchanged; q8kv_append and q8kv_import_pages
 * write them.  q and out rows stay hd floats long.
 *
 * Sub-tile byte order.  A sub-tile is hp / 64 chunks of 1024 bytes; byte
 * 16 * l + i of chunk c belongs to lane slot l = 16 * r + n (r in 0..3, n in
 * 0..15) and is, for row t (0..15) and column x (0..hp-1) of the sub-tile:
 *   K: t = n, x = 64 * c + 16 * r + i;
 *   V: with BPL = hp / 16, slot l holds rows 4r..4r+3, columns
 *      BPL*n .. BPL*n + BPL - 1, as 4 * BPL bytes in (row, column) order;
 *      byte j * BPL + e of that run (row 4r + j, column BPL*n + e) is byte
 *      i of chunk c where c * 16 + i = j * BPL + e.
 * q8kv_append writes this order; a caller that fills pages itself must too.
 *
 * Every entry point checks its arguments on the host before it makes any HIP
 * call, launches asynchronously on `stream` (a hipStream_t passed as void*,
 * NULL = the null stream of the current device) and never synchronises.
 * Faults inside a kernel surface at the caller's next synchronisation.  On a
 * non-zero return nothing was launched and q8kv_last_error() says why.
 */
#ifndef Q8KV_H
#define Q8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    Q8KV_OK = 0,
    Q8KV_EINVAL = -1, /* a size, shape or value argument is out of range */
    Q8KV_ENULL = -2,  /* a required pointer is NULL */
    Q8KV_EHIP = -3,   /* a HIP call failed; the message holds its error string */
    Q8KV_ENOMEM = -4  /* the split-context workspace could not be allocated */
};

/*
 * Decode attention for one query token per sequence.
 *
 * out          [batch][n_q_heads][hd] fp32, written in full.  A sequence with
 *              seq_lens[b] <= 0 gets an all-zero row.  A row whose sequence
 *              reaches a block_table entry outside [0, num_blocks), or whose
 *              seq_lens[b] exceeds max_blocks_per_seq * kv_bs, is written as
 *              NaN (the kernel never reads outside the page pool).
 * q            [batch][n_q_heads][hd] fp32 query (already rotated).
 * max_blocks_per_seq  row stride of block_table; bounds every sequence.
 * num_blocks   physical blocks in the page pool (bounds table entries).
 * hd           head size: a multiple of 32 from 32 to 256 (pages are hp
 *              wide, see "Page width").
 * kv_bs        tokens per page: 16, 32, 64, 128 or 256.
 * n_q_heads / n_kv_heads must be a positive integer G.  The query heads of
 *              a kv head are taken in head groups of g heads, g the largest
 *              divisor of G that is at most 8 (the matrix cores' column
 *              set); each head group is its own work item and reads the kv
 *              head's K/V itself, so G above 8 costs G/g reads of the cache.
 * batch        1 to 2048 sequences per call.
 * scale        softmax scale (normally 1/sqrt(hd)), finite.
 * K and V scales are any finite non-negative fp32 values (q8kv_append
 *              writes absmax/127).  The P.V weights carry a power-of-two
 *              offset that follows the largest V scale seen so far (up to
 *              2^126), so scales far above 1 do not overflow the f16 weight
 *              operands and scales far below 1 do not sink into their
 *              subnormals; outputs are checked for V amplitudes from 1e-6 to
 *              1e6.
 *
 * Contexts longer than one partition are split into fixed ranges of tokens
 * whose (max, sum, accumulator) states are merged in range order: inside the
 * decode kernel, by the workgroup that stores a (sequence, head group)'s
 * last state, when there are at most 64 states (partitions x query heads),
 * else by a second kernel (one workgroup per 16 output floats of a query
 * head, over every partition).  The plan depends only on the shapes, so results are
 * deterministic.  Split contexts use a library-owned device workspace (grown
 * on demand with hipMalloc, one per device and stream, freed by
 * q8kv_release, which waits for the device first).  Calls on one stream run
 * in order; calls on different streams use different workspaces.  The
 * workspace holds per-(sequence, head group) arrival counters that each call
 * leaves at zero, so a call that is aborted mid-kernel leaves the workspace
 * unusable until q8kv_release.
 */
int q8kv_decode_attn(float* out, const float* q,
                     const int8_t* k_pages, const int8_t* v_pages,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int max_blocks_per_seq, int num_blocks,
                     int batch, int n_q_heads, int n_kv_heads, int hd, int kv_bs,
                     float scale, void* stream);

/*
 * q8kv_decode_attn with an explicit partition length in tokens (a positive
 * multiple of 32), or 0 for the automatic plan.  Same contract otherwise.
 */
int q8kv_decode_attn_split(float* out, const float* q,
                           const int8_t* k_pages, const int8_t* v_pages,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int max_blocks_per_seq, int num_blocks,
                           int batch, int n_q_heads, int n_kv_heads, int hd, int kv_bs,
                           float scale, int part_tokens, void* stream);

/*
 * q8kv_decode_attn_split for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results (bit for bit); it never
 * calls hipMalloc or hipFree.  Its partition states, merge counters and
 * work ticket live in one library-owned 32 MiB device array (a file-scope
 * __device__ variable, one copy per device, held until the process ends),
 * whose counters it clears with a kernel at the start of every call.
 * Every call on a device shares that array: calls that overlap on one
 * device (on different streams, or from different threads) race and give
 * undefined results.  A call needs 256 bytes, plus 4 bytes per (sequence,
 * group of at most 8 query heads of one kv head) rounded up to a multiple of
 * 256, plus, when contexts are split into n_parts > 1 partitions (the
 * q8kv_plan count, or the one part_tokens gives), S = batch * n_q_heads *
 * n_parts states of 4 * hp bytes (all S rounded up to a multiple of 256) and
 * 8 bytes each.  A shape that needs more than 32 MiB is rejected with
 * Q8KV_EINVAL before any HIP call; q8kv_last_error() gives the bytes needed.
 * (Every one of the five benchmark workloads fits: the largest, 64
 * sequences of 64 query heads split in 8, needs about 17 MB.)  After one
 * call on a device (which looks up the array and the kernels' launch
 * limits), the call can be captured into a HIP graph and replayed: it
 * records kernels only.
 */
int q8kv_decode_attn_noalloc(float* out, const float* q,
                             const int8_t* k_pages, const int8_t* v_pages,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int max_blocks_per_seq, int num_blocks,
                             int batch, int n_q_heads, int n_kv_heads, int hd, int kv_bs,
                             float scale, int part_tokens, void* stream);

/*
 * Append the step's new token and attend to it in one launch: for every
 * sequence b with 1 <= seq_lens[b] <= max_blocks_per_seq * kv_bs, the new
 * token's K and V rows are quantised exactly as q8kv_append does and written
 * at position seq_lens[b] - 1, i.e. slot block_table[b][(L-1) / kv_bs] * kv_bs
 * + (L-1) % kv_bs with L = seq_lens[b] (the page-table slot rule of the page
 * "deepseek-attention-div64" (beaiera.top), section on top-k indices and slot
 * mapping); then out is what q8kv_decode_attn_split returns over positions
 * 0 .. L-1 of the updated cache, the new token included.  The fused-kernel
 * idea follows the same page's section on its fused quantise-and-cache-write
 * kernel.  The result equals q8kv_append with that slot mapping followed by
 * q8kv_decode_attn_split, bit for bit (cache and output).
 *
 * k_new, v_new [batch][n_kv_heads][hd], fp32 (src_dtype 0) or bf16
 *              (src_dtype 1), the new token's rows (q's token).
 * Sequences with seq_lens[b] <= 0 get a zero row and nothing is written; a
 * sequence whose new slot's table entry lies outside [0, num_blocks), or
 * whose length exceeds max_blocks_per_seq * kv_bs, gets a NaN row and
 * nothing is written.  The new slots of different sequences must be
 * distinct.  Other arguments as for q8kv_decode_attn_split.
 */
int q8kv_append_decode_attn(float* out, const float* q, const void* k_new, const void* v_new,
                            int src_dtype, int8_t* k_pages, int8_t* v_pages, float* k_scale,
                            float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                            int max_blocks_per_seq, int num_blocks, int batch, int n_q_heads,
                            int n_kv_heads, int hd, int kv_bs, float scale, int part_tokens,
                            void* stream);

/*
 * The automatic partition plan for a decode shape (host only, no HIP call):
 * *part_tokens = tokens per partition, *n_parts = partitions of the longest
 * possible sequence (max_blocks_per_seq * kv_bs tokens).
 */
int q8kv_plan(int batch, int n_q_heads, int n_kv_heads, int hd, int kv_bs,
              int max_blocks_per_seq, int* part_tokens, int* n_parts);

/*
 * Quantise new K and V rows into the paged cache (page "Day 9-2", section 1
 * and the kscale argument of section 2: one scale per token and kv head,
 * computed with the same absmax rule as the query, over the whole hd row).
 *
 * k_src, v_src [n_tokens][n_kv_heads][hd], fp32 (src_dtype 0) or bf16
 *              (src_dtype 1, widened exactly to fp32).
 * slot_mapping [n_tokens] int32: destination slot block * kv_bs + row of each
 *              token; a negative slot skips the token, as does a slot at or
 *              beyond num_blocks * kv_bs.
 * Row `row` of page (block, kh) is written in the sub-tile byte order above
 * (sub-tile row / 16, row row % 16 of it) and its dequantisation factors to
 * k_scale/v_scale[block][kh][row].
 */
int q8kv_append(int8_t* k_pages, int8_t* v_pages, float* k_scale, float* v_scale,
                const void* k_src, const void* v_src, int src_dtype,
                const int32_t* slot_mapping, int n_tokens, int num_blocks,
                int n_kv_heads, int hd, int kv_bs, void* stream);

/*
 * Rewrite an int8 cache held in row order into the layout above, on the
 * device, bit for bit.  Row order is the addressing of the int8 K/V blocks
 * on the page "Day 9-2: flash_attn_single_q_q8_neon" (trdm.cn), section 2
 * (the function signature and the per-token K row pointer): a block holds
 * kv_bs token rows, each row the hd bytes of every kv head in turn (row
 * stride n_kv_heads * hd; no padding), and the per-row scales sit beside them, one fp32
 * per (row, kv head).  (The page indexes its scales by sequence position;
 * here they are laid out per block, which is the same array when each
 * sequence owns consecutive blocks.)
 *
 * k_rows, v_rows           int8 [num_blocks][kv_bs][n_kv_heads][hd]
 * k_row_scale, v_row_scale fp32 [num_blocks][kv_bs][n_kv_heads]
 * k_pages, v_pages, k_scale, v_scale  the destination cache, as for
 *              q8kv_append; every byte and scale of it is written (the
 *              pad columns of a head size below hp with zeros).
 * All eight buffers are caller-owned device memory, 16-byte aligned; the
 * destination must not overlap the source (Q8KV_EINVAL otherwise, checked
 * on the host from the pointers and sizes).  Shape limits as for
 * q8kv_append.  The scales are copied as bit patterns, NaN included.
 */
int q8kv_import_pages(int8_t* k_pages, int8_t* v_pages, float* k_scale, float* v_scale,
                      const int8_t* k_rows, const int8_t* v_rows,
                      const float* k_row_scale, const float* v_row_scale,
                      int num_blocks, int n_kv_heads, int hd, int kv_bs, void* stream);

/*
 * FP8 KV codec (page "deepseek-attention-div64" (beaiera.top), section on the
 * FP8 quantisation scaling): every K and V row is stored as E4M3 codes (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; largest finite value 448; no
 * infinity), and every 64 consecutive elements of a row share one UE8M0
 * scale byte s, the exponent of the power-of-two scale 2^(s - 127).  A
 * block's absolute maximum a fixes e = ceil(log2(a / 448)) -- the exact
 * ceiling for the fp32 quotient a / 448, clamped to [-126, 127], and 0 for
 * an all-zero block -- and the codes are E4M3(clamp(x * 2^-e, -448, 448)),
 * rounded to nearest, ties to even; s = e + 127.  An element's value is
 * code value * 2^e.
 *
 * Layouts (caller-owned device memory):
 *   k_pages,
 *   v_pages   uint8 [num_blocks][n_kv_heads][kv_bs / 16][16 * hd]: E4M3
 *             codes in 16-row sub-tiles of hd / 64 chunks of 1024 bytes
 *             (lane slot l = 16 r + n owns bytes [16 l, 16 l + 16) of each);
 *             K in the int8 codec's K order (chunk c, slot l: row n,
 *             columns 64 c + 16 r .. + 16); V: slot l holds rows 4r .. 4r+3
 *             of the columns 16 s + n (s = 0 .. hd/16 - 1) as hd / 16
 *             dwords, dword s = those four rows of column 16 s + n in row
 *             order, dword s lying in chunk s / 4 at bytes 4 (s % 4) ..;
 *   k_scale,
 *   v_scale   uint8 [num_blocks][n_kv_heads][kv_bs][hd / 64] UE8M0 bytes.
 * hd is 64, 128 or 256 (no padded widths: Q8KV_EINVAL otherwise).  Other
 * arguments, errors and behaviour as for q8kv_append and
 * q8kv_decode_attn_split.
 */
int q8kv_fp8_append(uint8_t* k_pages, uint8_t* v_pages, uint8_t* k_scale, uint8_t* v_scale,
                    const void* k_src, const void* v_src, int src_dtype,
                    const int32_t* slot_mapping, int n_tokens, int num_blocks,
                    int n_kv_heads, int hd, int kv_bs, void* stream);

/*
 * Decode attention over an FP8 cache: out[b][h] = softmax(scale * q[b][h] .
 * K) V over tokens 0 .. seq_lens[b] - 1, with K and V the dequantised
 * values above and q used as given (carried as two f16 parts, about 22
 * significant bits).  One pass with the same online-softmax recurrence,
 * partitions and merges as q8kv_decode_attn_split.
 */
int q8kv_fp8_decode_attn(float* out, const float* q, const uint8_t* k_pages,
                         const uint8_t* v_pages, const uint8_t* k_scale,
                         const uint8_t* v_scale, const int32_t* block_table,
                         const int32_t* seq_lens, int max_blocks_per_seq, int num_blocks,
                         int batch, int n_q_heads, int n_kv_heads, int hd, int kv_bs,
                         float scale, int part_tokens, void* stream);

/*
 * q4_0 KV codec.  The pages name it only (page "FlashAttention" tag
 * (baguaai.com), news item on llama.cpp's SYCL decode path for q4_0 / q8_0
 * KV caches); this is llama.cpp's block format: every 32 consecutive
 * elements of a K or V row share one fp16 scale d and are stored as 4-bit
 * codes c, element value (c - 8) * d.  Quantisation of a block: m = its
 * element of largest magnitude (sign kept, the first on ties), d = m / -8
 * in fp32, id = 1 / d (0 when d = 0), c = min(15, trunc(x * id + 8.5)) with
 * two fp32 roundings (no fused multiply-add), stored d = fp16(d).
 *
 * Layouts (caller-owned device memory):
 *   k_pages,
 *   v_pages   uint8 [num_blocks][n_kv_heads][kv_bs / 16][8 * hd]: 16-row
 *             sub-tiles of 8 hd bytes; lane slot l = 16 r + n (r in 0..3, n in
 *             0..15) owns hd / 8 bytes at byte (hd / 8) * l:
 *             K: byte 8 c + i of the slot holds row n, column 64 c + 16 r + i
 *                in its low nibble and column 64 c + 16 r + 8 + i in its high
 *                nibble (c < hd / 64, i < 8);
 *             V: byte 4 (s / 2) + j holds row 4 r + j of column 16 s + n, the
 *                even s in the low nibble and the odd s in the high one
 *                (s < hd / 16, j < 4);
 *   k_scale,
 *   v_scale   fp16 bits, uint16 [num_blocks][n_kv_heads][kv_bs][hd / 32].
 * Decode: the query is quantised per 32-block to int8 as for the int8 cache
 * (codes qi, scales qsc); a token's score is scale * sum over blocks b of
 * qsc[b] * d_K[b] * sum_{i in b} qi[i] * (c_K[i] - 8), and the output is the
 * softmax-weighted sum of the dequantised V rows, one pass as in
 * q8kv_decode_attn_split.  hd is 64, 128 or 256 (Q8KV_EINVAL otherwise).
 * Other arguments, errors and behaviour as for q8kv_append and
 * q8kv_decode_attn_split.
 */
int q8kv_q40_append(uint8_t* k_pages, uint8_t* v_pages, uint16_t* k_scale, uint16_t* v_scale,
                    const void* k_src, const void* v_src, int src_dtype,
                    const int32_t* slot_mapping, int n_tokens, int num_blocks,
                    int n_kv_heads, int hd, int kv_bs, void* stream);
int q8kv_q40_decode_attn(float* out, const float* q, const uint8_t* k_pages,
                         const uint8_t* v_pages, const uint16_t* k_scale,
                         const uint16_t* v_scale, const int32_t* block_table,
                         const int32_t* seq_lens, int max_blocks_per_seq, int num_blocks,
                         int batch, int n_q_heads, int n_kv_heads, int hd, int kv_bs,
                         float scale, int part_tokens, void* stream);

/*
 * QUEST block metadata (page "CANN ops-transformer Quest Prefill Metadata"
 * (xdnf.cn), section on the experiment background: for every KV block, the
 * per-channel maximum and minimum over the block's tokens of the K cache).
 *
 * kmax, kmin  fp32 [num_blocks][n_kv_heads][hd], caller-owned.  For every
 *             sequence b and logical block j < ceil(L / kv_bs) with
 *             L = seq_lens[b], physical block p = block_table[b][j]:
 *             kmax[p][kh][c] / kmin[p][kh][c] = max / min over the block's
 *             rows r < min(kv_bs, L - j kv_bs) of float(k code) * k_scale
 *             of that row (an fp32 product).  Other blocks, and table entries
 *             outside [0, num_blocks), are left untouched.
 * Other arguments as for q8kv_decode_attn, except that hd is 64, 128 or
 * 256 (for both QUEST calls).  A block shared by several sequences must
 * cover the same rows in each.
 */
int q8kv_quest_metadata(float* kmax, float* kmin, const int8_t* k_pages, const float* k_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        int max_blocks_per_seq, int num_blocks, int batch, int n_kv_heads,
                        int hd, int kv_bs, void* stream);

/*
 * Query-aware block selection over that metadata (same page: at decode the
 * query is matched against each block's metadata and the top-k blocks take
 * part in attention).  The bound of block j for query head h is the largest
 * dot product any vector inside the block's [kmin, kmax] box can have with
 * q_h: sum over c of max(q_h[c] kmax[c], q_h[c] kmin[c]), computed in fp32;
 * a kv head takes the largest bound over its query heads.  For each
 * sequence with nblk = ceil(L / kv_bs) blocks: if nblk <= top_k every block
 * is kept; else the last block (which holds the newest token) plus the
 * top_k - 1 blocks of largest bound among the others, ties to the lower
 * logical index.
 *
 * sel_table  int32 [batch][n_kv_heads][top_k]: the kept physical blocks of
 *            each kv head in logical order, -1 past the kept count.
 * sel_lens   int32 [batch]: tokens the kept blocks hold
 *            ((kept - 1) * kv_bs + the last block's rows), the same for every
 *            kv head; 0 for an empty sequence.
 * max_blocks_per_seq may be at most 4097.  The bounds go through a
 * library-owned workspace (grown on demand, freed by q8kv_release).
 * q8kv_decode_attn_heads(sel_table, sel_lens, max_blocks_per_seq = top_k)
 * then attends over the kept tokens only.
 */
int q8kv_quest_select(int32_t* sel_table, int32_t* sel_lens, const float* q, const float* kmax,
                      const float* kmin, const int32_t* block_table, const int32_t* seq_lens,
                      int max_blocks_per_seq, int num_blocks, int batch, int n_q_heads,
                      int n_kv_heads, int hd, int kv_bs, int top_k, void* stream);

/*
 * q8kv_decode_attn_split with one block list per kv head: head_table is
 * int32 [batch][n_kv_heads][max_blocks_per_seq]; kv head kh of sequence b
 * reads token t from block head_table[b][kh][t / kv_bs].  seq_lens[b] is the
 * token count of every kv head's list.  Same contract otherwise.
 */
int q8kv_decode_attn_heads(float* out, const float* q, const int8_t* k_pages,
                           const int8_t* v_pages, const float* k_scale, const float* v_scale,
                           const int32_t* head_table, const int32_t* seq_lens,
                           int max_blocks_per_seq, int num_blocks, int batch, int n_q_heads,
                           int n_kv_heads, int hd, int kv_bs, float scale, int part_tokens,
                           void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* q8kv_last_error(void);

/* Free every library-owned workspace on every device (synchronising first). */
int q8kv_release(void);

/*
 * Test exports: the decode kernel's own device functions, so that the int8
 * parts can be compared bit for bit.
 *
 * q8kv_debug_quantize_q: qi [rows][hd] int8 and qsc [rows][hd/32] fp32 from
 * q [rows][hd] fp32, through the decode kernel's query prologue.
 *
 * q8kv_debug_block_dots: dots [batch][n_q_heads][max_tok][hd/32] int32, the
 * per-32-block int32 dot of the quantised query with each K row, computed by
 * the decode kernel's matrix-core scoring step, for t < min(seq_lens[b],
 * max_tok); other entries are left untouched.
 */
int q8kv_debug_quantize_q(int8_t* qi, float* qsc, const float* q, int rows, int hd,
                          void* stream);
int q8kv_debug_block_dots(int32_t* dots, int max_tok, const float* q, const int8_t* k_pages,
                          const int32_t* block_table, const int32_t* seq_lens,
                          int max_blocks_per_seq, int num_blocks, int batch, int n_q_heads,
                          int n_kv_heads, int hd, int kv_bs, void* stream);

/*
 * Test export: enable (1, the default) or disable (0) the 8-wave workgroups
 * that the decode entry points use for a static grid of at most one
 * workgroup per CU at hd 64 and 128.  With 0 such grids run the 4-wave
 * kernel, as larger grids do, so that tests can compare the two.  Applies to
 * every later call in the process; Q8KV_EINVAL for other values.  The two
 * kernels merge their waves' states in different orders, so their outputs
 * agree to rounding, not bit for bit.
 */
int q8kv_debug_set_wide(int enable);

/*
 * Test and measurement export: enable (1) or disable (0, the default) the
 * LDS-staged variant of the int8 decode kernels for static grids at hd 64
 * and 128 (q8kv_decode_attn, _split, _noalloc and q8kv_append_decode_attn).
 * Each wave then keeps two tiles in flight in an LDS ring, loaded with
 * global_load_lds, and reads a tile into registers only to compute it; the
 * arithmetic is unchanged, so outputs are bit for bit those of the default
 * kernels.  A static grid of more than two workgroups per CU runs the
 * persistent kernel instead.  Applies to every later call in the process;
 * Q8KV_EINVAL for other values.
 */
int q8kv_debug_set_stage(int enable);

/*
 * Measurement export: read a_bytes of device buffer a and b_bytes of device
 * buffer b (both multiples of 16) in one launch with plain linear
 * non-temporal loads and discard the data.  A benchmark times it over a
 * decode call's page pools to state the decode's rate against a plain
 * streaming read of the same bytes on the same device.  No output; never
 * writes either buffer.
 */
int q8kv_debug_stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes, void* stream);

/*
 * Measurement export: the int8 decode kernel's loads without its arithmetic,
 * over the first num_pages pages (block, kv head) of a page pool taken as
 * one flat array, to compare load orders on the same device.  Items of
 * item_pages consecutive pages, one per workgroup of four waves (at most
 * two per CU), each wave loading 32-token tiles as the decode kernel does.
 * pattern 0: the page layout above (one 16-byte load per lane per 1 KB
 * chunk of K and V) plus the per-row K and V scale loads; 1: the same
 * without the scale loads; 2: the same bytes taken as row-major pages
 * ([row][hd] bytes per page, the token-major order of a row cache) loaded
 * into the same matrix-core operands (K 16-byte pieces of 16 rows, V
 * hd/16-byte pieces of four rows per lane) plus the scale loads.  hd 64,
 * 128 or 256; item_pages * kv_bs a multiple of 128; num_pages a multiple of
 * item_pages.  No output; never writes the pool.
 */
int q8kv_debug_load_probe(const int8_t* k_pages, const int8_t* v_pages, const float* k_scale,
                          const float* v_scale, int num_pages, int hd, int kv_bs, int item_pages,
                          int pattern, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8KV_H */
