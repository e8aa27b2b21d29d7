/*
 * xs/xs.h - C ABI of libxs.so: paged-KV decode attention for AMD MI355X (gfx950).
 *
 * One decode step of an LLM serving engine over a paged KV cache:
 *   1. xs_kv_append          writes each running sequence's new K/V row into its block.
 *   2. xs_paged_attn_decode  computes GQA softmax(q K^T * scale) V for every (sequence,
 *                            query head), optionally per split-K partition of the context.
 *   3. xs_paged_attn_reduce  merges the partitions with a log-sum-exp rule.
 *
 * Sources: the xserv pages (gitea compare views of the xserv engine).
 *   - Pool layout, block table, context_lens, q/out shapes, the append and decode
 *     contracts: xserv compare phase10...cf1e9e41, crates/xserv-kernels/src/attention.rs,
 *     FFI block and doc comments of `reshape_and_cache_bf16`,
 *     `reshape_and_cache_batched_bf16` and `paged_decode_attention`.
 *   - GQA mapping (query head h reads kv head h / n_rep, n_rep = Hq / Hkv): xserv compare
 *     phase8...phase13, `repeat_kv` in the Qwen3 model and the `repeat_kv_bf16` kernel.
 *   - Split-K partitions and the log-sum-exp merge are not on the pages. They are this
 *     library's way to spread long contexts over the GPU. The merge is an exact identity of
 *     the unsplit softmax.
 *
 * Common conventions
 *   - Every pointer is a device pointer on the current HIP device, except where stated.
 *     The caller owns every buffer. The library allocates nothing, never synchronizes,
 *     and enqueues all work on `stream` (a hipStream_t passed as void*; NULL = null stream).
 *   - Shapes are row-major (C-contiguous):
 *       q, out          [batch, num_q_heads, head_dim]          (one query token per sequence)
 *       k_new, v_new    [batch, num_kv_heads, head_dim]
 *       k_cache/v_cache [num_blocks, num_kv_heads, block_size, head_dim]
 *       block_tables    int32 [batch, max_blocks_per_seq]; entry j of row b is the physical
 *                       block holding tokens [j*block_size, (j+1)*block_size) of sequence b.
 *       context_lens    int32 [batch]; L_b = the context length of sequence b AFTER this
 *                       step's append, i.e. the index of the just-written token + 1.
 *   - dtype: q, k_new, v_new, the pools and out all have the same dtype (XS_F32 or XS_BF16).
 *     Parameters named dtype are plain ints carrying an xs_dtype value: any other value is
 *     rejected with XS_EUNSUPPORTED (an enum-typed parameter would make such a value undefined
 *     behaviour in C++ instead of an error).
 *     Arithmetic is fp32. bf16 results are rounded to nearest-even.
 *   - Supported: head_dim in {64, 128}; block_size in {8, 16, 32}; num_q_heads a multiple
 *     of num_kv_heads; q, pools, k_new/v_new, out and part_o 16-byte aligned.
 *   - Return value: XS_OK (0) or an xs_status. A nonzero status sets a message that
 *     xs_last_error() returns. Host-checkable argument errors are reported before any HIP
 *     call is made. A failed launch gives XS_ELAUNCH.
 *   - Device-resident preconditions cannot be checked on the host: 0 <= L_b <= max_blocks_per_seq
 *     * block_size, and the block ids in use lie in [0, num_blocks). Violating them gives
 *     undefined results but no out-of-bounds access. The kernels clamp L_b to
 *     max_blocks_per_seq * block_size, skip blocks whose id lies outside [0, num_blocks),
 *     and treat L_b <= 0 as an empty context. The slot an append writes (position L_b - 1 of
 *     sequence b) must lie neither inside another sequence's context nor be another sequence's
 *     slot, or the results of both are undefined (a read races the write). The Python package's
 *     check_device_inputs checks these conditions on a host copy of the tables.
 */
#ifndef XS_H
#define XS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { XS_F32 = 0, XS_BF16 = 1 } xs_dtype;

typedef enum {
  XS_OK = 0,
  XS_EINVAL = 1,       /* a null pointer, a bad size, a misaligned pointer */
  XS_EUNSUPPORTED = 2, /* a valid request this library does not implement (head_dim, block_size, dtype) */
  XS_ELAUNCH = 3       /* the HIP runtime rejected a kernel launch */
} xs_status;

/*
 * Decode-step KV append (xserv compare phase10...cf1e9e41, attention.rs,
 * `reshape_and_cache_batched_bf16` and its doc comment).
 *
 * For every sequence b with L = context_lens[b] >= 1, position p = L - 1 lies in physical
 * block blk = block_tables[b, p / block_size] at slot off = p % block_size. For every kv
 * head g, row k_cache[blk, g, off, :] becomes k_new[b, g, :], and v_cache likewise. This is
 * a bit-exact copy, and no other byte of the pools changes.
 * Arguments: k_new, v_new [batch, num_kv_heads, head_dim] (read); k_cache, v_cache (written
 * in place); block_tables, context_lens (read).
 * Two sequences must not map the same slot; otherwise the last write wins in no fixed order.
 * batch == 0 is a no-op.
 */
int xs_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens,
                 int batch, int num_kv_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int num_blocks, int dtype, void* stream);

/*
 * Single-token GQA decode attention over the paged pool (xserv compare phase10...cf1e9e41,
 * attention.rs, `paged_decode_attention` and its FFI `launch_paged_decode_attention_bf16`).
 *
 * For sequence b, query head h, g = h / (num_q_heads / num_kv_heads), tokens t in [0, L_b):
 *   K_t = k_cache[block_tables[b, t / block_size], g, t % block_size, :], V_t likewise,
 *   s_t = scale * dot(q[b, h, :], K_t),
 *   out[b, h, :] = sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s).
 * The single query sits at the last position, so the causal mask lets it see all L_b keys.
 * Pool slots at t >= L_b are never used, and may hold anything, NaN included.
 * L_b = 0 gives out[b, h, :] = 0.
 *
 * partition_size == 0: no split. `out` is written. part_o/part_m/part_l must be NULL and
 *   max_partitions is ignored.
 * partition_size  > 0: split-K. It must be a multiple of block_size. Partition j of sequence b
 *   covers tokens [j*P, min((j+1)*P, L_b)) for j < n_b = ceil(L_b / P). For each (b, h, j)
 *   the call writes, in fp32:
 *     part_m[b, h, j]     = m_j = max_t s_t                          [batch, num_q_heads, NP]
 *     part_l[b, h, j]     = l_j = sum_t exp(s_t - m_j)               [batch, num_q_heads, NP]
 *     part_o[b, h, j, :]  = sum_t exp(s_t - m_j) V_t / l_j           [batch, num_q_heads, NP, head_dim]
 *   with NP = max_partitions. `out` is not touched (it may be NULL); xs_paged_attn_reduce
 *   produces it. Entries j >= n_b are not written. Partitions at j >= max_partitions are
 *   not computed, so the caller must give max_partitions >= max_b ceil(L_b / P); the reduce
 *   writes NaN rows for a sequence where that does not hold.
 */
int xs_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         float scale, void* out,
                         float* part_o, float* part_m, float* part_l,
                         int batch, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int num_blocks,
                         int partition_size, int max_partitions, int dtype, void* stream);

/*
 * xs_kv_append followed by xs_paged_attn_decode, in one launch (the decode step without the
 * append's separate kernel). Same arguments as xs_paged_attn_decode plus k_new, v_new
 * [batch, num_kv_heads, head_dim] (read), and the pools are written: for each sequence with
 * 1 <= L_b <= max_blocks_per_seq * block_size, row (block_tables[b, (L_b-1) / block_size], g,
 * (L_b-1) % block_size, :) of k_cache/v_cache becomes k_new[b, g, :] / v_new[b, g, :], as in
 * xs_kv_append. The attention result is bit-identical to the two separate calls: the kernel
 * takes token L_b - 1 straight from k_new/v_new, which are the bits the append stores.
 * Sources: the batched append and the decode attention of xserv compare phase10...cf1e9e41,
 * attention.rs (`reshape_and_cache_batched_bf16`, `paged_decode_attention`), issued back to
 * back by the decode step.
 */
int xs_paged_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                float scale, void* out,
                                float* part_o, float* part_m, float* part_l,
                                int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_blocks_per_seq, int num_blocks,
                                int partition_size, int max_partitions, int dtype, void* stream);

/* Bytes of the device-resident scratch behind xs_paged_attn_decode_append_noalloc (per device). */
#define XS_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * xs_paged_attn_decode_append followed by xs_paged_attn_reduce, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the split-K partials live in a scratch array inside the library
 * (XS_NOALLOC_SCRATCH_BYTES per device, held from the first call on that device until the process
 * ends) instead of in part_o/part_m/part_l. Nothing is allocated, by this call or the library.
 * Arguments, results and the append are those of xs_paged_attn_decode_append and
 * xs_paged_attn_reduce with the same partition_size and max_partitions; `out` [batch,
 * num_q_heads, head_dim] (16-byte aligned) is always written, k_new and v_new are required.
 * partition_size == 0 is the unsplit call (no scratch used). With split-K the partials take
 * batch * num_q_heads * max_partitions * (head_dim + 2) * 4 bytes (each array rounded up to 256);
 * more than XS_NOALLOC_SCRATCH_BYTES is XS_EINVAL, before any device work.
 * Every call on a device shares that device's scratch and leaves its contents behind: two calls
 * that may run at the same time on one device (other streams, other threads) race and give wrong
 * results; calls on one stream are ordered and safe.
 */
int xs_paged_attn_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                        void* k_cache, void* v_cache,
                                        const int32_t* block_tables, const int32_t* context_lens,
                                        float scale, void* out,
                                        int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                        int block_size, int max_blocks_per_seq, int num_blocks,
                                        int partition_size, int max_partitions, int dtype, void* stream);

/*
 * Decode attention with attention sinks and a sliding window (xserv compare
 * phase10...cf1e9e41, attention.rs, `paged_decode_attention_sinks` and its FFI
 * `launch_paged_decode_attention_sinks_bf16`), optionally with the fused append.
 *
 * sinks: NULL, or bf16 [num_q_heads] (device, read): one logit sigma_h per query head in the
 *   units of the scaled scores. It joins the softmax as an entry without a value row.
 * window_size: 0 keeps all positions; W > 0 keeps positions t in [max(0, L_b - W), L_b), the
 *   query's own position L_b - 1 included.
 * Result, for t0 = max(0, L_b - W) (or 0) and M = max(sigma_h, max_t s_t):
 *   out[b, h, :] = sum_{t >= t0} exp(s_t - M) V_t / (exp(sigma_h - M) + sum_{t >= t0} exp(s_t - M)).
 * L_b = 0 gives zeros. k_new/v_new: both NULL (no append) or both given, as in
 * xs_paged_attn_decode_append. Other arguments, layouts and partitions as in
 * xs_paged_attn_decode, except that with split-K partitions wholly before t0 are not written
 * and the partials carry no sink: xs_paged_attn_reduce_sinks, with the same sinks and window,
 * produces `out`.
 * Supported: bf16, head_dim 64 or 128, block_size 16 or 32 (XS_EUNSUPPORTED otherwise).
 * Readings where the pages are silent (sink units, window bounds, empty context) are the
 * plainest ones the pages support; the oracle states them.
 */
int xs_paged_attn_decode_sinks(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               const void* sinks, int window_size, float scale, void* out,
                               float* part_o, float* part_m, float* part_l,
                               int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq, int num_blocks,
                               int partition_size, int max_partitions, int dtype, void* stream);

/*
 * The merge of xs_paged_attn_decode_sinks' partials (same sinks and window_size): partitions
 * j in [t0 / P, ceil(L_b / P)) with t0 the window start, and
 *   M = max(sigma_h, max_j m_j),
 *   out = sum_j l_j e^(m_j - M) o_j / (e^(sigma_h - M) + sum_j l_j e^(m_j - M)).
 * bf16 output only. Other arguments as in xs_paged_attn_reduce.
 */
int xs_paged_attn_reduce_sinks(const float* part_o, const float* part_m, const float* part_l,
                               const int32_t* context_lens, const void* sinks, int window_size,
                               void* out, int batch, int num_q_heads, int head_dim,
                               int partition_size, int max_partitions, int dtype, void* stream);

/*
 * Decode steps as one HIP graph: captured once, then replayed (xserv compare
 * phase10...cf1e9e41, crates/xserv-cuda/src/graph.rs: capture a fixed sequence of launches and
 * replay it without per-launch host work; shapes and addresses fixed at capture, no host
 * branching inside; the decode loop there captures the whole forward of a token, every layer).
 * A graph holds num_steps steps in order, e.g. one per layer of a model. Each step is the append of k_new/v_new (fused into the decode when `fused` != 0,
 * otherwise xs_kv_append's kernel first), the decode (xs_paged_attn_decode_sinks when sinks or
 * window_size are given, else xs_paged_attn_decode), and, when partition_size > 0, the matching
 * reduce into `out`. Fields mean what the arguments of those calls mean; all pointers are
 * device pointers that must stay valid while the graph exists. Their contents (q, k_new,
 * v_new, block_tables, context_lens, sinks) may change between replays: a decode loop updates
 * them in place and replays. Sizes (batch, max_partitions, ...) are fixed at capture.
 */
typedef struct {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* sinks;  /* NULL: no sinks */
  int window_size;    /* 0: no window */
  float scale;
  void* out;
  float* part_o;      /* split-K partials: NULL when partition_size == 0 */
  float* part_m;
  float* part_l;
  int batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks;
  int partition_size, max_partitions, dtype;
  int fused;          /* != 0: append fused into the decode launch */
} xs_step_desc;

typedef struct xs_step_graph xs_step_graph;

/*
 * Checks descs[0 .. num_steps-1] (1 <= num_steps <= 4096), each as the entry points above check
 * their arguments, plus: batch >= 1, k_new and v_new given; then captures the steps in order on a
 * private stream and instantiates the graph. On success
 * *out_graph owns a HIP graph and its executable instance (host-side runtime objects; no device
 * memory is allocated by this library). On failure *out_graph is NULL. Capture runs in
 * thread-local mode: other threads may keep using HIP meanwhile.
 */
int xs_step_graph_create(const xs_step_desc* descs, int num_steps, xs_step_graph** out_graph);

/* Replays the captured steps on `stream` (asynchronous, like the calls above). */
int xs_step_graph_launch(xs_step_graph* graph, void* stream);

/* Releases the graph (NULL is a no-op). The caller must not destroy a graph that is still
 * running on a stream. */
int xs_step_graph_destroy(xs_step_graph* graph);

/*
 * Log-sum-exp merge of split-K partitions (not on the pages: the exact identity of the
 * unsplit softmax). For each (b, h), with n = min(ceil(L_b / P), max_partitions),
 *   M = max_j m_j,  w_j = l_j exp(m_j - M),  out[b, h, :] = sum_j w_j o_j / sum_j w_j.
 * Reads part_o/part_m/part_l as written by xs_paged_attn_decode with the same partition_size
 * and max_partitions (part_o and out 16-byte aligned). Writes out [batch, num_q_heads, head_dim]
 * in `dtype`. L_b <= 0, or a
 * sequence whose partitions all have l_j = 0, gives zeros. A sequence with ceil(L_b / P) >
 * max_partitions (the decode did not compute its last partitions) gives NaN rows, so that a
 * truncated context cannot pass for a result.
 */
int xs_paged_attn_reduce(const float* part_o, const float* part_m, const float* part_l,
                         const int32_t* context_lens, void* out,
                         int batch, int num_q_heads, int head_dim,
                         int partition_size, int max_partitions, int dtype, void* stream);

/*
 * KV block swap between the paged pools and a swap space in pinned host memory (the xserv
 * README, xserv compare phase10...cf1e9e41: CPU swap-out / swap-in of the paged KV cache into
 * pinned host memory, `--swap-space-gb`).
 * The swap space is k_host, v_host: [num_slots, num_kv_heads, block_size, head_dim] in `dtype`,
 * allocated pinned (hipHostMalloc, or torch pin_memory=True) by the caller; anything else is
 * rejected with XS_EINVAL before any launch. One slot holds one pool block (all kv heads).
 * xs_kv_swap_out: for i < num_pairs, slot dst_slots[i] becomes a bit copy of pool block
 *   src_blocks[i] (K and V).
 * xs_kv_swap_in:  for i < num_pairs, pool block dst_blocks[i] becomes a bit copy of slot
 *   src_slots[i] (K and V).
 * The index lists are int32 device arrays of num_pairs entries. A pair with an index outside
 * [0, num_blocks) or [0, num_slots) is skipped. Two pairs must not share a destination (their
 * order is not fixed). One launch moves the whole list; the GPU reads or writes the host memory
 * directly over the host link. Asynchronous on `stream`, like the calls above: host memory is
 * complete only once the stream has been synchronized.
 */
int xs_kv_swap_out(const void* k_cache, const void* v_cache, void* k_host, void* v_host,
                   const int32_t* src_blocks, const int32_t* dst_slots, int num_pairs,
                   int num_blocks, int num_slots, int num_kv_heads, int block_size, int head_dim,
                   int dtype, void* stream);
int xs_kv_swap_in(const void* k_host, const void* v_host, void* k_cache, void* v_cache,
                  const int32_t* src_slots, const int32_t* dst_blocks, int num_pairs,
                  int num_blocks, int num_slots, int num_kv_heads, int block_size, int head_dim,
                  int dtype, void* stream);

/*
 * Chunked prefill, step 1: multi-token paged append (xserv compare phase10...cf1e9e41,
 * attention.rs, `reshape_and_cache_bf16` / `launch_reshape_and_cache_bf16`: a run of tokens of
 * one sequence written from start_pos on through its block ids; here batched over sequences).
 *
 * For every sequence b with 0 <= start_pos[b], 0 <= n_b = chunk_lens[b] <= chunk_size and
 * start_pos[b] + n_b <= max_blocks_per_seq * block_size, and every i < n_b: position
 * p = start_pos[b] + i lies in block blk = block_tables[b, p / block_size] at slot
 * p % block_size, and for every kv head g row k_cache[blk, g, p % block_size, :] becomes
 * k_src[b, g, i, :] (v_cache likewise). A bit copy; nothing else in the pools changes. Rows
 * i >= n_b of k_src/v_src are not read, sequences outside the conditions above are skipped, and
 * so are positions whose block id is outside [0, num_blocks).
 * Arguments: k_src, v_src [batch, num_kv_heads, chunk_size, head_dim] (read); k_cache, v_cache
 * (written in place); block_tables [batch, max_blocks_per_seq], start_pos [batch], chunk_lens
 * [batch] (int32, device, read). XS_BF16 or XS_F32. Two positions must not map the same slot,
 * and no appended slot may lie inside another sequence's context (a read would race the write);
 * the Python package's check_prefill_inputs checks these conditions on a host copy of the tables.
 * batch == 0 or chunk_size == 0 is a no-op.
 */
int xs_kv_append_chunk(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                       const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                       int batch, int num_kv_heads, int head_dim, int chunk_size, int block_size,
                       int max_blocks_per_seq, int num_blocks, int dtype, void* stream);

/*
 * Chunked prefill, step 2: causal GQA attention of a chunk of queries over the paged pool
 * (xserv compare phase10...cf1e9e41, attention.rs, `flash_attention(q, k, v, causal)`, GQA
 * native, with its K/V read through the block table as the decode attention reads them).
 *
 * Row i < n_b = chunk_lens[b] of sequence b sits at position p = start_pos[b] + i and sees the
 * keys at positions t = 0 .. p (the causal mask aligned to the end of the cached range; with
 * start_pos = 0 it is the plain causal mask). With g = h / (num_q_heads / num_kv_heads):
 *   s_t = scale * dot(q[b, h, i, :], K_t),  K_t = k_cache[block_tables[b, t / block_size], g,
 *         t % block_size, :], V_t likewise,
 *   out[b, h, i, :] = sum_{t <= p} exp(s_t - max s) V_t / sum_{t <= p} exp(s_t - max s).
 * The chunk's own K/V must already be in the pool (xs_kv_append_chunk). Rows i >= n_b are
 * written as zeros, and so are all rows of a sequence outside the conditions of
 * xs_kv_append_chunk. Positions whose block id is outside [0, num_blocks) are skipped.
 * Arguments: q, out [batch, num_q_heads, chunk_size, head_dim] bf16 (q read, out written);
 * pools and index arrays as above (read). XS_BF16 only (XS_EUNSUPPORTED otherwise); products in
 * fp32 from bf16 inputs, the probabilities rounded to bf16 for the P.V product, fp32 softmax
 * statistics, out rounded to bf16. batch == 0 or chunk_size == 0 is a no-op.
 */
int xs_paged_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                          float scale, void* out, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                          int chunk_size, int block_size, int max_blocks_per_seq, int num_blocks, int dtype,
                          void* stream);

/*
 * Chunked prefill attention with split-K over the key range: the same result as
 * xs_paged_attn_prefill (the same passage), computed in pieces so that the row blocks with the
 * most keys (the chunks that start deepest into their sequence) are spread over more compute
 * units. Row blocks of 256 (chunk row, query head) pairs of one kv head cut their keys into
 * pieces of `partition_size` positions (piece j: positions [j P, (j+1) P)); a row block with a
 * single piece writes `out` directly, the others leave, for every row and piece, the row's
 * output over the piece's keys o_j (fp32) and (m_j, l_j) (m_j the reference max in scaled log2
 * units, l_j the sum of 2^(s log2e - m_j) over those keys; m_j = -inf, l_j = 0, o_j = 0 for a
 * piece with none of the row's keys). A second kernel, launched by this call on the same
 * stream, merges them with the log-sum-exp identity (not on the pages: exact up to rounding):
 *   M = max_j m_j,  w_j = l_j 2^(m_j - M),  out = sum_j w_j o_j / sum_j w_j.
 * Arguments as xs_paged_attn_prefill, plus: part_o [batch, num_q_heads, chunk_size,
 * max_partitions, head_dim] fp32 and part_ml [batch, num_q_heads, chunk_size, max_partitions, 2]
 * fp32, device scratch owned by the caller (16- and 8-byte aligned; contents on entry are not
 * read, on exit unspecified); partition_size a positive multiple of 64; max_partitions >=
 * ceil(max_blocks_per_seq * block_size / partition_size) (XS_EINVAL otherwise). batch == 0 or
 * chunk_size == 0 is a no-op.
 */
int xs_paged_attn_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                                float scale, void* out, float* part_o, float* part_ml, int batch, int num_q_heads,
                                int num_kv_heads, int head_dim, int chunk_size, int block_size,
                                int max_blocks_per_seq, int num_blocks, int partition_size, int max_partitions,
                                int dtype, void* stream);

/*
 * Chunked prefill attention with attention sinks and a sliding window, the prefill of the
 * gpt-oss layers (xserv compare phase10...cf1e9e41, attention.rs, `flash_attention_sinks` and
 * its FFI `launch_flash_attention_sinks_bf16`: always causal, one sink per query head folded
 * into the softmax denominator, window_size 0 for full causal attention), over the paged pool
 * as xs_paged_attn_prefill reads it.
 *   sinks: NULL, or bf16 [num_q_heads] (device, read, 2-byte aligned): one logit sigma_h per
 *          query head in the units of the scaled scores.
 *   window_size: 0 keeps keys 0 .. p; W > 0 keeps keys max(0, p + 1 - W) .. p (the query's own
 *          position and the W - 1 before it).
 * Row i < chunk_lens[b] at position p = start_pos[b] + i, with t0 its first key, gets
 *   out[b, h, i, :] = sum_{t0 <= t <= p} exp(s_t - M) V_t
 *                     / (exp(sigma_h - M) + sum_{t0 <= t <= p} exp(s_t - M)),  M = max(sigma_h, max s_t)
 * (no sigma term when sinks is NULL); other rows, invalid sequences and bad block ids as in
 * xs_paged_attn_prefill. partition_size 0 computes each row block's keys in one workgroup
 * (part_o and part_ml are not used and may be NULL); partition_size > 0 is the split-K of
 * xs_paged_attn_prefill_split with the same partials and conditions, where the pieces carry no
 * sink and the merge adds it once (M = max(sigma_h, max_j m_j), the sink a term of weight
 * 2^(sigma_h log2e - M) with no value row), starting at the piece of the row's first window key.
 * Readings where the pages are silent (window bounds, sink units, paged layout) are those of
 * xs_paged_attn_decode_sinks. XS_BF16 only; window_size < 0 is XS_EINVAL. With sinks NULL and
 * window_size 0 the result is that of xs_paged_attn_prefill / _split.
 */
int xs_paged_attn_prefill_sinks(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                                const void* sinks, int window_size, float scale, void* out, float* part_o,
                                float* part_ml, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                int chunk_size, int block_size, int max_blocks_per_seq, int num_blocks,
                                int partition_size, int max_partitions, int dtype, void* stream);

/*
 * Measurement aid, not part of the decode step: reads `bytes` (a multiple of 16) at `buf` with
 * 16-byte loads (nontemporal if `nontemporal` != 0) and writes at most one word to `sink` (device
 * memory, 4 bytes). Workgroups take chunks of the buffer in turn: shape 0 runs 16 workgroups per
 * CU on 256 KiB chunks, shape 1 two workgroups per CU on 16 KiB chunks (any other shape is
 * XS_EINVAL). Timing both and taking the faster gives the read rate that contiguous streaming
 * reaches on the device, the reference the decode kernel's bandwidth is compared with. `buf` must
 * be 16-byte aligned.
 */
int xs_stream_read_probe(const void* buf, size_t bytes, unsigned* sink, int nontemporal, int shape, void* stream);

/* Message for the last nonzero status returned on this thread ("" if none). Host memory owned
 * by the library, valid until the next call on this thread. */
const char* xs_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int xs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* XS_H */
