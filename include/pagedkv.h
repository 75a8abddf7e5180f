/*
 * pagedkv.h - PagedAttention decode on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpagedkv.so.  Three operations of the decode step (cache write,
 * decode attention, split-K reduce), multi-query attention over the same
 * pool, a workspace query and a status string.  All kernels are hand-written
 * HIP for CDNA4.
 *
 * Sources (by page title and section):
 *   [P4] "vLLM 推理引擎源码级拆解：PagedAttention 显存虚拟化、Continuous
 *        Batching 调度与量化落地全指南" (chenxutan.com/d/5333)
 *   [P2] "vLLM 深度实战" (chenxutan.com/d/3332)
 *   [P1] "vLLM 0.5 深度拆解" (chenxutan.com/d/4924)
 *   [P3] "vLLM 深度剖析：PagedAttention 与连续批处理如何撑起大模型推理"
 *        (pgsm.cn/news/372185)
 *
 * Conventions for every call
 *   - Pointers are device pointers owned by the caller, except where noted.
 *     The library allocates, frees and synchronises nothing: each call
 *     validates its arguments on the host, enqueues kernels on `stream` and
 *     returns.  The only state it keeps across calls is per-device facts
 *     asked once and cached (compute-unit count, a kernel's occupancy) and
 *     a counter that numbers balanced-split calls; both are atomics, so
 *     calls are thread-safe.
 *   - Tensors are dense, row-major (C order), with the shapes given below.
 *     Device pointers must be 16-byte aligned.
 *   - Argument errors are reported by a negative pkv_status before anything
 *     is enqueued.  PKV_ERR_HIP means the kernel launch itself failed.
 *   - Device-side contents (block ids, lengths, slots) are not validated on
 *     the host; the kernels clamp them so that no access leaves the
 *     buffers described here, and the documented preconditions say when the
 *     result is meaningful.
 *
 * Pool layout ([P4] §2.3 declares [num_blocks, block_size, num_heads,
 * head_dim]; the head axis is read as KV heads):
 *   k_cache, v_cache : [num_blocks][block_size][num_kv_heads][head_dim]
 *   element (b, o, h, d) sits at ((b*block_size + o)*num_kv_heads + h)*head_dim + d
 *   Token t of sequence s lives in physical block block_tables[s][t / block_size]
 *   at offset t % block_size ([P4] §2.2-2.3).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_NULL = -1,        /* a required pointer is NULL */
    PKV_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    PKV_ERR_DTYPE = -3,       /* unknown dtype or an invalid dtype pairing */
    PKV_ERR_UNSUPPORTED = -4, /* valid, but no kernel for this combination */
    PKV_ERR_WORKSPACE = -5,   /* workspace missing or too small */
    PKV_ERR_ALIGN = -6,       /* a device pointer is not 16-byte aligned */
    PKV_ERR_HIP = -7,         /* the HIP runtime reported a launch error */
    PKV_ERR_NO_BLOCKS = -8,   /* block manager: the pool has no block to give */
    PKV_ERR_SCRATCH = -9      /* the call needs more than the fixed scratch array */
} pkv_status;

typedef enum {
    PKV_F32 = 0,
    PKV_F16 = 1,
    PKV_BF16 = 2,
    PKV_FP8_E4M3 = 3          /* OCP E4M3 (no inf, 0x7F/0xFF NaN, max 448) */
} pkv_dtype;

/* partition_size value selecting the balanced split (see
 * pkv_paged_attention_decode). */
#define PKV_PARTITION_BALANCED (-1)

/* Kernel choice for pkv_paged_attention_decode. */
typedef enum {
    PKV_ALGO_AUTO = 0,        /* fastest kernel that supports the arguments */
    PKV_ALGO_VALU = 1,        /* vector-ALU kernel: every supported combination */
    PKV_ALGO_MFMA = 2         /* matrix-core kernel: f16/bf16 query, f16/bf16/fp8 cache */
} pkv_algo;

/*
 * pkv_reshape_and_cache - store new tokens' K and V in their cache slots.
 *
 * [P4] §2.2: the next token goes into the free slot of the sequence's last
 * block, or into a fresh block appended to its table; the caller's block
 * bookkeeping turns that into one slot number per token,
 * slot = physical_block * block_size + offset.  For every token i with
 * 0 <= slot_mapping[i] < num_blocks*block_size and every KV head h:
 *     k_cache[slot / block_size][slot % block_size][h][:] = conv(key[i][h][:])
 *     v_cache[...same...]                                  = conv(value[i][h][:])
 * Other slots are skipped.  conv is a bit copy when cache_dtype == src_dtype;
 * for cache_dtype PKV_FP8_E4M3 it is e4m3(x / scale) with x the exact fp32
 * value of the source element, an IEEE fp32 division, round to nearest even
 * and saturation of finite overflow to +-448 (NaN stays NaN).  The pages give
 * only an fp8 cache flag ([P1] §4.2, [P3] §6.1, [P4] §6.4); OCP E4M3 with
 * one scale per tensor is this library's reading.
 *
 *   key, value    [num_tokens][num_kv_heads][head_dim], src_dtype
 *                 (PKV_F32, PKV_F16 or PKV_BF16)
 *   k_cache, v_cache  pool as above, cache_dtype == src_dtype or PKV_FP8_E4M3
 *   slot_mapping  [num_tokens] int64
 *   k_scale, v_scale  fp8 scales (> 0, finite); ignored otherwise
 * Precondition: slots are distinct (two tokens writing one slot race).
 * num_tokens == 0 is a no-op.
 */
int pkv_reshape_and_cache(const void* key, const void* value, pkv_dtype src_dtype,
                          void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                          const int64_t* slot_mapping, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, float k_scale,
                          float v_scale, hipStream_t stream);

/*
 * pkv_paged_attention_decode - one query token per sequence against its
 * paged K/V ([P4] §2.3).
 *
 * For sequence s, query head hq and G = num_q_heads / num_kv_heads, with
 * h = hq / G (consecutive query heads share a KV head; [P4] §2.3 names GQA
 * and MQA) and L = seq_lens[s]:
 *     z_t = scale * k_scale' * sum_d query[s][hq][d] * K[t][d],  t < L
 *     out[s][hq][:] = sum_t softmax(z)_t * v_scale' * V[t][:]
 * where K[t], V[t] are the stored rows of token t of (s, h), read through the
 * block table, and k_scale' = k_scale, v_scale' = v_scale for an fp8 cache
 * (1 otherwise).  Tokens t >= L never contribute, whatever the memory holds.
 * The softmax is evaluated online (running max and running sum, as in the
 * [P4] §2.3 kernel sketch), in fp32.  L <= 0 gives a zero row.
 *
 *   out           [num_seqs][num_q_heads][head_dim], dtype = q_dtype
 *   query         [num_seqs][num_q_heads][head_dim], q_dtype
 *   k_cache, v_cache  pool as above, cache_dtype
 *   block_tables  [num_seqs][max_blocks_per_seq] int32 physical block ids;
 *                 only the first ceil(L / block_size) entries of a row are read
 *   seq_lens      [num_seqs] int32
 *   max_seq_len   host-side bound on seq_lens (sizes the split-K grid)
 *
 * Supported: (q_dtype, cache_dtype) in {(F32,F32), (F16,F16), (BF16,BF16),
 * (F16,FP8), (BF16,FP8)}; head_dim 64 or 128; block_size 8, 16 or 32;
 * num_q_heads % num_kv_heads == 0 with G <= 8 (PKV_ALGO_VALU) or G <= 16
 * (PKV_ALGO_MFMA).
 *
 * Split-K (not on the pages; the merge follows from the running max/sum of
 * the online softmax).  Three modes, chosen by partition_size:
 *
 *   0      one pass: `out` is written and workspace may be NULL.
 *
 *   P > 0  fixed partitions (P a multiple of 16 and of block_size): the
 *          tokens of each sequence are cut into partitions
 *          [k*P, min(L, (k+1)*P)); a sequence with at most one partition is
 *          finished here and its `out` rows written; for every other sequence
 *          the per-partition partials go to `workspace` and
 *          pkv_paged_attention_reduce must run next on the same stream.
 *          Workspace layout, with P_max = ceil(max_seq_len / P) and
 *          n = num_seqs * num_q_heads * P_max:
 *            offset 0             float max_logit[num_seqs][num_q_heads][P_max]
 *            offset A = round_up(4n, 256)
 *                                 float exp_sum[num_seqs][num_q_heads][P_max]
 *            offset 2A            float partial_out[num_seqs][num_q_heads][P_max][head_dim]
 *          For partition k: m_k is a reference logit (natural-log units, at
 *          most the partition's largest z_t and within 8 ln 2 of it),
 *          l_k = sum over the partition of exp(z_t - m_k) and
 *          o_k = sum of exp(z_t - m_k) * v_scale' * V[t] (not normalised).
 *          Entries of partitions k >= ceil(L/P), and of single-partition
 *          sequences, are not written.
 *
 *   PKV_PARTITION_BALANCED (-1)
 *          balanced split (matrix-core kernel only, so f16/bf16 queries;
 *          num_seqs <= 8192): the whole batch's work -- every (sequence, KV
 *          head) pair's tokens in 16-token tiles, laid end to end -- is cut
 *          into chunks by a guided schedule (large chunks first, small ones
 *          last) and spread over a persistent grid of one wavefront per
 *          SIMD (at most 2048); each wavefront starts on a
 *          chunk of its own and then takes chunks in order from a counter,
 *          so that ragged lengths and uneven wavefront speeds cost no load
 *          balance.  One kernel is enqueued.  A
 *          (sequence, KV head) pair that falls into one chunk is finished
 *          here; for every other pair each chunk's piece leaves its partials
 *          in `workspace` (layout private to the library: a header, the tile
 *          prefix of the sequences, the first and last chunk of every
 *          (sequence, KV head) pair, then (m, l, o) entries as above, two
 *          per query head of the group per chunk), and pkv_paged_attention_reduce
 *          must run next on the same stream with partition_size =
 *          PKV_PARTITION_BALANCED; it also writes the zero rows of sequences
 *          with L <= 0.  The workspace needs no initialisation: its chunk
 *          counter carries the number of the call that last used it, and
 *          each call takes it over at its first request, whatever it held;
 *          the reduce returns it to zero, so a graph holding the decode and
 *          its reduce replays correctly although the call number is frozen
 *          in the graph.  Calls sharing one workspace must not overlap in
 *          time (use one stream).  Requires
 *          num_seqs * num_kv_heads * ceil(max_seq_len / 16) < 2^31.
 *
 * pkv_decode_workspace_bytes gives the workspace size for either split mode.
 *
 * Preconditions for a meaningful result: 0 <= block ids < num_blocks and
 * seq_lens[s] <= min(max_seq_len, max_blocks_per_seq * block_size).  Block
 * ids outside the pool are clamped to num_blocks - 1 and lengths to that
 * bound, so a bad table gives a wrong row but no stray access.
 *
 * algo selects the kernel (pkv_algo); an explicit choice that cannot serve
 * the arguments returns PKV_ERR_UNSUPPORTED.
 */
int pkv_paged_attention_decode(void* out, const void* query, pkv_dtype q_dtype,
                               const void* k_cache, const void* v_cache,
                               pkv_dtype cache_dtype, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_seq_len, float scale, float k_scale,
                               float v_scale, int32_t partition_size,
                               void* workspace, size_t workspace_bytes,
                               int32_t algo, hipStream_t stream);

/*
 * pkv_paged_attention_decode_noalloc - for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the balanced split of
 * pkv_paged_attention_decode and its pkv_paged_attention_reduce in one
 * call, with the workspace taken from a fixed array inside the library
 * instead of from the caller.
 *
 * Arguments, what is computed and the errors are those of
 * pkv_paged_attention_decode with partition_size = PKV_PARTITION_BALANCED
 * and algo = PKV_ALGO_MFMA (f16/bf16 queries; f16/bf16/fp8 caches; head_dim
 * 64 or 128; num_q_heads / num_kv_heads <= 16; num_seqs <= 8192), followed
 * by the reduce on the same stream; `out` is complete when both kernels are
 * done.  The results equal those of that decode + reduce pair bit for bit.
 *
 * The array is 64 MiB of device memory per GPU the library runs on, held
 * until the process ends.  It needs, for a grid of nW = one wavefront per
 * SIMD (1024 on MI355X), 256 B + 4 (num_seqs + 1) B rounded up to 256, then
 * 2 (5 nW + 8) G entries of (head_dim + 2) floats (G = num_q_heads /
 * num_kv_heads): about 21 MB at G = 4 and 43 MB at G = 8 for head_dim 128.
 * A call that needs more returns PKV_ERR_SCRATCH with nothing enqueued.
 * The call allocates and frees nothing: the array's device address is
 * looked up once per device (PKV_ERR_HIP if HIP cannot give it).
 *
 * Every call on one GPU uses that GPU's one array and leaves its contents
 * behind; no call needs it cleared (the balanced chunk counter takes over
 * whatever it finds, and the reduce returns it to zero).  Calls that
 * overlap in time on one GPU, e.g. from two streams, race on the array and
 * give wrong results: serialise them.
 */
int pkv_paged_attention_decode_noalloc(void* out, const void* query, pkv_dtype q_dtype,
                                       const void* k_cache, const void* v_cache,
                                       pkv_dtype cache_dtype, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks,
                                       int32_t max_seq_len, float scale, float k_scale,
                                       float v_scale, hipStream_t stream);

/*
 * pkv_paged_attention_decode_mixed - decode over a pool whose sequences use
 * different block sizes: "vLLM 0.5 深度拆解" §1.3 picks 8, 16 or 32
 * tokens per block per request (short requests small blocks, long ones
 * large).  The pages do not say how blocks of several sizes share memory;
 * this library's reading:
 *
 *   The pool is kept in pages of page_size tokens, laid out as a pool of
 *   page_size-token blocks: k_cache, v_cache [num_pages][page_size]
 *   [num_kv_heads][head_dim].  Sequence s has blocks of bs_s =
 *   seq_block_sizes[s] tokens (8, 16 or 32, a multiple of page_size); a
 *   block is bs_s / page_size consecutive pages, and block_tables[s][j] is
 *   the first page of its block j.  Token t of sequence s is therefore row
 *       block_tables[s][t / bs_s] * page_size + t % bs_s
 *   of the pool (the slot pkv_reshape_and_cache takes, with block_size =
 *   page_size and num_blocks = num_pages).
 *
 * What is computed, the other arguments, partition_size (P > 0: a multiple
 * of 32; PKV_PARTITION_BALANCED: the balanced split, each sequence walked
 * over its own block size, 8-token blocks in 8-token tiles; either way the
 * partials go to the workspace of pkv_decode_workspace_bytes with the same
 * sizes and partition_size, and pkv_paged_attention_reduce with that
 * partition_size merges them) and the errors are as for
 * pkv_paged_attention_decode with block_size = page_size and num_blocks =
 * num_pages, for the matrix-core type combinations (f16/bf16 query;
 * f16/bf16/fp8 cache; head_dim 64 or 128; G <= 16).
 * Also PKV_ERR_NULL for a NULL seq_block_sizes ([num_seqs] int32, device);
 * PKV_ERR_SHAPE for a pool smaller than 32 tokens or P not a multiple of 32.
 * Preconditions: each bs_s is 8, 16 or 32 and at least page_size (other
 * values are read as the nearest of page_size and 32); a block's pages lie
 * in the pool; seq_lens[s] <= max_blocks_per_seq * bs_s.
 */
int pkv_paged_attention_decode_mixed(void* out, const void* query, pkv_dtype q_dtype,
                                     const void* k_cache, const void* v_cache,
                                     pkv_dtype cache_dtype, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     const int32_t* seq_block_sizes, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size, int32_t num_pages,
                                     int32_t max_seq_len, float scale, float k_scale,
                                     float v_scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_paged_attention_multi - several new query tokens per sequence against
 * the paged K/V: chunked prefill ([P4] §6.3: a long prompt's prefill cut
 * into chunks that run between decode steps; [P1] §2.3) and speculative
 * verification ([P4] §6.5: the large model checks several drafted tokens in
 * one pass).
 *
 * Sequence s brings Qn = query_start[s+1] - query_start[s] query tokens,
 * rows query_start[s] .. query_start[s+1]-1 of `query`.  They are the last
 * Qn of its L = seq_lens[s] cached tokens (stored by pkv_reshape_and_cache
 * before this call, as in decode), so query token i sits at position
 * L - Qn + i and attends to tokens 0 .. L - Qn + i (causal among the new
 * tokens, every earlier token visible):
 *     z_t = scale * k_scale' * sum_d query[r][hq][d] * K[t][d],  t <= L - Qn + i
 *     out[r][hq][:] = sum_t softmax(z)_t * v_scale' * V[t][:]
 * with r = query_start[s] + i, h = hq / G, K/V and the scales as in
 * pkv_paged_attention_decode.  A query token whose position is negative
 * (Qn > L) gets a zero row.  The pages give no kernel for this step; the
 * definition above is this library's reading of theirs.
 *
 *   out, query    [total_q][num_q_heads][head_dim], dtype q_dtype, where
 *                 total_q = query_start[num_seqs]
 *   query_start   [num_seqs + 1] int32, query_start[0] = 0, non-decreasing
 *   max_query_len host-side bound on every Qn (sizes the grid); rows of
 *                 tokens past it are not written
 *   other arguments as for pkv_paged_attention_decode
 *
 * Supported: the matrix-core combinations of pkv_paged_attention_decode
 * (f16/bf16 query; f16/bf16/fp8 cache; head_dim 64 or 128; block_size 8, 16
 * or 32; G <= 16).  One wavefront serves 16 / G consecutive query tokens of
 * one sequence and one KV head, so K/V is read once per 16 / G query tokens.
 * Preconditions for a meaningful result as for decode, and
 * Qn <= max_query_len.
 *
 *   partition_size 0: each wavefront walks its query tokens' whole context
 *                 (no workspace).  P > 0 (a multiple of 16 and of
 *                 block_size): split-K as in decode - the context is cut
 *                 into P-token partitions, one wavefront per (partition,
 *                 group of query tokens, KV head), and a second kernel on
 *                 the same stream merges the partials of every row (query
 *                 token, query head) whose token sees more than P tokens;
 *                 rows that see at most P are written by the first kernel.
 *                 Partitions wholly after a query token's last visible
 *                 token are skipped for it.
 *   PKV_PARTITION_BALANCED (-1), for speculative verification with
 *                 max_query_len <= 16 / G (else PKV_ERR_UNSUPPORTED): the
 *                 balanced split of pkv_paged_attention_decode over the
 *                 (sequence, KV head) streams, whose last query token sees
 *                 all L tokens; the B operand's columns are the (query
 *                 token, head) pairs, each dropping the tokens past its own
 *                 position.  The call enqueues the decode kernel and its
 *                 reduce over the rows (query token, head); calls on one
 *                 workspace must not overlap (its chunk counter, as for
 *                 decode).
 *   workspace     device memory of at least pkv_multi_workspace_bytes(...)
 *                 bytes for the same num_seqs, max_query_len, num_q_heads,
 *                 head_dim, max_seq_len and partition_size, 16-byte aligned,
 *                 owned by the caller; its contents on entry do not matter.
 *                 Ignored (may be NULL) for partition_size 0.  Calls that
 *                 share a workspace must be ordered on one stream.
 *
 * Errors (nothing launched): as for decode; PKV_ERR_SHAPE also for a
 * negative partition_size other than PKV_PARTITION_BALANCED or one that is
 * not a multiple of 16 and of block_size; PKV_ERR_WORKSPACE for a missing
 * or short workspace.
 */
int pkv_paged_attention_multi(void* out, const void* query, pkv_dtype q_dtype,
                              const void* k_cache, const void* v_cache,
                              pkv_dtype cache_dtype, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              const int32_t* query_start, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                              int32_t max_query_len, float scale, float k_scale,
                              float v_scale, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_multi_workspace_bytes - bytes of workspace pkv_paged_attention_multi
 * needs.  PKV_PARTITION_BALANCED: a 256-byte header, num_seqs + 1 words
 * and 2 * num_seqs * num_q_heads words (the chunk ranges of the streams),
 * then m, l [2 * (5 * 2048 + 8) * 16] float32 and room for o [same][head_dim]
 * float32 (each part on a 256-byte boundary), whatever the lengths.  The o
 * rows are stored compactly in the first half of that room: head_dim f16
 * values per row, the row's mean scaled by a power of two whose exponent
 * the low byte of the row's l carries.  P > 0: with rows = num_seqs * max_query_len *
 * num_q_heads and P_max = ceil(max_seq_len / P), m and l [rows][P_max] and
 * o [rows][P_max][head_dim] float32, then [num_seqs * max_query_len] int32
 * context lengths, each part starting on a 256-byte boundary.  0 for
 * partition_size 0 or a size that is not positive.  Host-only.
 */
size_t pkv_multi_workspace_bytes(int32_t num_seqs, int32_t max_query_len,
                                 int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t partition_size);

/*
 * pkv_decode_workspace_bytes - bytes of workspace split-K decode needs
 * (layouts above) for partition_size > 0 or PKV_PARTITION_BALANCED; 0 when
 * partition_size == 0, a size is not positive or num_q_heads is not a
 * multiple of num_kv_heads.  The balanced size does not depend on the
 * lengths: a header, num_seqs + 1 + 2 * num_seqs * num_kv_heads words, and
 * 2 * (5 * 2048 + 8) entries of head_dim + 2 floats per query head of the
 * group.  Host-only, touches no device.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t partition_size);

/*
 * pkv_paged_attention_reduce - merge split-K partials (the second kernel of
 * long-context decode).
 *
 * For every row (sequence s, query head hq) whose work was split, from the
 * workspace written by pkv_paged_attention_decode with the same
 * partition_size, seq_lens and sizes:
 *     M = max_k m_k
 *     out[s][hq][:] = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k
 * over the row's entries k (fixed partitions: k < ceil(L/P); balanced: the
 * pieces of the row's KV-head stream).  Rows that decode finished are left
 * untouched.  Fixed partitions: the workspace may also come from any other
 * producer of the documented layout.  Balanced: the workspace must hold what
 * the decode call wrote (for the same num_kv_heads); if its header does not
 * match, nothing is written.  out_dtype is F32, F16 or BF16.
 */
int pkv_paged_attention_reduce(void* out, pkv_dtype out_dtype,
                               const void* workspace, size_t workspace_bytes,
                               const int32_t* seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_seq_len,
                               int32_t partition_size, hipStream_t stream);

/*
 * pkv_copy_blocks - copy whole blocks of the K and V pools: for i <
 * num_pairs, block block_pairs[2i] of (src_k, src_v) is copied over block
 * block_pairs[2i+1] of (dst_k, dst_v).
 *  - Inside one pool (dst == src) it is the data movement of copy on write
 *    ([P4] §2.1: a sequence about to write into a block that other block
 *    tables still reference gets its own copy); pkv_bm_append reports the
 *    pairs.
 *  - Between the device pool and a pool in pinned host memory (allocated
 *    with hipHostMalloc, which the GPU reads and writes directly over the
 *    host link) it is swapping ([P4] §3.2: a preempted sequence's blocks move
 *    to host memory and back, bound by the host link's bandwidth).
 * Pairs with a block id outside its pool (src_blocks / dst_blocks blocks), or
 * copying a block onto itself, are skipped.
 *   pools         [*_blocks][block_size][num_kv_heads][head_dim], cache_dtype
 *                 (any pkv_dtype); K and V are both same-pool or both not
 *   block_pairs   [num_pairs][2] int32, device or pinned host memory
 * Precondition: within one pool, no block is both a destination and a
 * source, or a destination twice, in one call.  num_pairs == 0 is a no-op.
 */
int pkv_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                    pkv_dtype cache_dtype, const int32_t* block_pairs, int32_t num_pairs,
                    int32_t src_blocks, int32_t dst_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, hipStream_t stream);

/*
 * pkv_host_device_pointer - the address under which the GPU reaches pinned
 * host memory (allocated with hipHostMalloc, e.g. a host pool for swapping),
 * for use as a pkv_copy_blocks pool.  PKV_ERR_HIP if host_ptr is not pinned,
 * mapped host memory (then *device_ptr is NULL).  Host-only.
 */
int pkv_host_device_pointer(const void* host_ptr, void** device_ptr);

/*
 * Block manager - host-side books of one pool ([P4] §3.3: it records who
 * holds which physical block, the reference counts and the free blocks, and
 * never touches the data).  It hands out the block tables and slot numbers
 * the calls above consume.  Host memory only; no call touches the GPU; one
 * manager is not safe to use from several threads at once.
 *
 *  - Blocks are taken on demand ([P4] §2.1-2.2): a sequence's next token
 *    goes into the free slot of its last block, or into a fresh block.
 *  - Sharing: pkv_bm_fork gives a new sequence the same table (reference
 *    counts + 1).  Writing into a block that another table still references
 *    first moves the writer onto a fresh copy (copy on write); the caller
 *    performs the copy with pkv_copy_blocks before writing the token.
 *  - Prefix caching ([P4] §4.2), when enabled: each full block is registered
 *    under a hash of its token ids and of the block before it; a new
 *    sequence whose leading full blocks match registered ones points its
 *    table at them (their K/V is reused, and the caller writes only the
 *    tokens after them).  A registered block nobody references stays
 *    registered until its block is needed.
 *  - Order (the pages leave it open; fixed so that tables are
 *    reproducible): the lowest-numbered free block is taken first; when no
 *    block is free, the registered unreferenced block released longest ago
 *    is taken (and unregistered).  A sequence's blocks are released last
 *    block first.  A partial last block is never registered.
 *  - A call that needs more blocks than the pool can give returns
 *    PKV_ERR_NO_BLOCKS and changes nothing (the caller preempts a sequence:
 *    frees it and recomputes it later, or swaps it out, [P4] §3.2).
 */
typedef struct pkv_block_manager pkv_block_manager;

/* New manager for a pool of num_blocks blocks of block_size tokens; NULL on
 * bad sizes or out of memory. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t enable_prefix_cache);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Registers sequence seq_id with num_tokens tokens (its prompt) and takes its
 * blocks.  slots[t] (host, [num_tokens]) receives the slot of token t; the
 * first *num_cached tokens (a multiple of block_size) are held by reused
 * prefix-cache blocks and need no writing.  Errors: the id exists
 * (PKV_ERR_SHAPE), not enough blocks (PKV_ERR_NO_BLOCKS). */
int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                        int32_t num_tokens, int64_t* slots, int32_t* num_cached);

/* Appends one token: *slot receives its slot.  If the sequence's last block
 * was shared, *copy_src / *copy_dst receive the block to copy and its new
 * copy (pass them to pkv_copy_blocks before writing the token), else -1. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int32_t token_id, int64_t* slot,
                  int32_t* copy_src, int32_t* copy_dst);

/* New sequence child sharing every block of parent (e.g. parallel samples). */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Releases a sequence's blocks. */
int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id);

/* Blocks the pool can still give (free plus registered unreferenced). */
int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);

/* Tokens of a sequence (negative status if unknown). */
int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id);

/* Copies up to max_entries entries of a sequence's block table into out
 * (host) and returns its length (negative status if unknown). */
int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* out,
                           int32_t max_entries);

/* Reference count of a block (negative status if out of range). */
int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);

/* Static, human-readable name of a pkv_status value. */
const char* pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
