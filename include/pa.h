/*
 * pa.h -- C ABI of libpagedattn.so: paged KV cache and decode-step paged attention on MI355X
 * (gfx950).
 *
 * Sources, cited by page title and section:
 *   [Ultralytics] "PagedAttention", Ultralytics glossary (Japanese):
 *       "ページングの仕組み" (how paging works) -- fixed-size blocks (16 tokens by default) in one
 *       shared pool, a per-request block table recording the order of the blocks, the attention
 *       kernel fetching keys and values block by block through that table; its PyTorch example
 *       writes each key into slot (pos mod B) of the block at table index (pos div B) and reads
 *       the request back through the table.
 *       "シーケンス間でのブロック共有" (sharing blocks between sequences) -- refcounted shared
 *       blocks and copy-on-write of a block another sequence still uses.
 *       "関連手法" (related methods) -- grouped-query attention and an 8-bit (FP8) KV cache.
 *   [Wikipedia] "PagedAttention", Wikipedia article, section "Математическая формулировка"
 *       (mathematical formulation) -- causal attention of query token i with the 1/sqrt(d)
 *       scaling, and its blockwise form over blocks K_j, V_j of B tokens, j = 1..ceil(i/B).
 *
 * Data layout (all arrays row-major, C order):
 *   k_cache  [num_blocks][num_kv_heads][block_size][head_dim]  key of slot o of block b, head g
 *   v_cache  [num_blocks][num_kv_heads][head_dim][block_size]  value of that slot, dim-major
 *   k_scale, v_scale  float [num_blocks][num_kv_heads]          fp8 caches only: real value of a
 *                                                                stored code c is e4m3(c) * scale
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]          physical block of logical block j
 *   context_lens  int32 [num_seqs]                              tokens a sequence attends (L)
 *   slot_mapping  int32 [num_tokens]                            block * block_size + offset
 *   q, out        [num_seqs][num_heads][head_dim]
 *   query head h reads kv head h / (num_heads / num_kv_heads).
 *
 * Where this interface goes beyond the plain statement of the problem (a query, the shared K/V
 * block pools, per-sequence block tables, context lengths, the block size and the scale):
 *   - values are stored dim-major inside a block (v_cache above); the pages fix only a one-head
 *     [block][slot][dim] key pool, and keys keep that order;
 *   - pa_decode takes three more ints: partition_tokens (split length, 0 = the library's plan),
 *     variant (kernel choice) and flags (a cache hint); pa_decode_workspace_bytes takes
 *     num_kv_heads and partition_tokens, on which the plan depends;
 *   - streams are passed as void* (a hipStream_t), so this header needs no HIP include.
 *
 * Element types: PA_F32 (IEEE binary32), PA_F16 (binary16), PA_BF16 (bfloat16 bit patterns),
 * PA_FP8_E4M3 (OCP E4M3: bias 7, max 448, no infinities, S.1111.111 = NaN).
 *
 * Ownership: every pointer is caller-owned memory; device pointers are HIP device memory of the
 * current device. The library never allocates or frees device memory; pa_decode takes a
 * caller-supplied workspace. Calls only enqueue work on `stream` (a hipStream_t; NULL = the
 * null stream) and return without synchronising.
 *
 * Errors: every scalar argument is checked on the host before any HIP call, so a bad call
 * returns an error code and touches neither the device nor the stream. Device array *contents*
 * (block ids, slots, lengths) are not validated; the kernels clamp them so that a bad entry can
 * never make them read or write outside the arrays described above, but the result is then
 * undefined. After the launches, a HIP launch error is reported as PA_ERR_HIP.
 *
 * Thread safety: the compute entry points hold no state and may be called concurrently; the
 * profiling counters (pa_profile_*) are process-global and not synchronised.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent shapes        */
  PA_ERR_UNSUPPORTED = -2, /* head_dim / block_size / dtype combination not built         */
  PA_ERR_WORKSPACE = -3,   /* workspace smaller than pa_decode_workspace_bytes() asks for  */
  PA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed                   */
} pa_status;

typedef enum {
  PA_VARIANT_AUTO = 0, /* MFMA when num_heads > num_kv_heads and the cache is 16-bit or fp8   */
  PA_VARIANT_VALU = 1, /* one work-group per query head: DPP dot products, any head grouping  */
  PA_VARIANT_MFMA = 2  /* one work-group per kv head: the query group x block on MFMA        */
} pa_variant;

/* pa_decode flags. */
enum { PA_DECODE_SHARED_BLOCKS = 1 };

/* Human-readable name of a pa_status value (static string, never NULL). */
const char* pa_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int pa_version(void);

/*
 * pa_write_kv -- slot-mapped write of new tokens' keys and values into their blocks
 * ([Ultralytics] "ページングの仕組み": the slot arithmetic of the example).
 *
 *   k_new, v_new  device, in_dtype  [num_tokens][num_kv_heads][head_dim]
 *   k_cache, v_cache  device, cache_dtype, layout above (written)
 *   slot_mapping  device int32 [num_tokens]; slot < 0 skips the token. Slots must be distinct.
 *   cache_dtype == in_dtype (PA_F32 / PA_F16 / PA_BF16): the stored bits are the input bits.
 *   cache_dtype == PA_FP8_E4M3 (in_dtype any 16/32-bit type): stored code = round-to-nearest-
 *     even E4M3 of (float)x / scale[block][head] (one IEEE fp32 divide; scales must be positive),
 *     magnitudes >= 448 saturate to 448, NaN stays NaN; the code's sign bit is x's sign bit.
 *     k_scale / v_scale are read, not written.
 *   head_dim in {64, 128}; block_size in {8, 16, 32}; num_blocks * block_size < 2^31.
 */
int pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                int block_size, int num_blocks, pa_dtype in_dtype, pa_dtype cache_dtype,
                const float* k_scale, const float* v_scale, void* stream);

/*
 * pa_copy_blocks -- copy whole blocks for copy-on-write ([Ultralytics]
 * "シーケンス間でのブロック共有": a block still used by another sequence is copied before a
 * write).
 *
 *   block_pairs  device int32 [num_pairs][2] = (src, dst). For each pair the dst block's keys
 *   and values of every kv head (and, for fp8 caches, both scales) become a copy of src's.
 *   The dsts must be distinct and no dst may also be a src in the same call (pairs are then
 *   independent and run in parallel). num_pairs == 0 is a no-op.
 *   k_scale / v_scale: required for PA_FP8_E4M3 caches, ignored otherwise.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   const int32_t* block_pairs, int num_pairs, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, pa_dtype cache_dtype, void* stream);

/*
 * pa_gather_kv -- read sequences back through their block tables into contiguous arrays
 * ([Ultralytics] "ページングの仕組み": the example's read-back through the table).
 *
 *   k_out, v_out  device, cache_dtype, [num_seqs][max_tokens][num_kv_heads][head_dim]
 *   Row t of sequence s is written for t < min(context_lens[s], max_tokens) with the stored
 *   bits of token t (values transposed back to dim-minor); other rows are left untouched.
 *   max_tokens <= max_blocks_per_seq * block_size.
 */
int pa_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                 int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                 int num_blocks, int max_tokens, pa_dtype cache_dtype, void* stream);

/*
 * pa_decode_workspace_bytes -- bytes of workspace pa_decode needs for these sizes. With an
 * explicit partition_tokens this is exactly the fixed-partition need (0 when no sequence can span
 * more than one partition); with partition_tokens = 0 it is an upper bound that covers whichever
 * default plan pa_decode picks (fixed partitions, or the balanced split of the work over one
 * resident grid, whose partial results take at most 2 * 2048 slots of Hq / Hkv heads).
 * Returns 0 as well for invalid sizes; pa_decode then reports the error.
 */
size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int max_blocks_per_seq, int block_size, int partition_tokens);

/*
 * pa_decode -- decode-step paged attention ([Wikipedia] "Математическая формулировка"):
 * for every sequence s and query head h,
 *     out[s][h] = sum_{t < L} a_t v_t,   a_t = exp(scale q.k_t) / sum_{u < L} exp(scale q.k_u)
 * with L = context_lens[s], keys/values of logical token t read from block
 * block_tables[s][t / block_size] at slot t % block_size. Slots at or beyond L in the last block
 * are excluded (their contents, NaN included, never reach the output); table entries at index
 * >= ceil(L / block_size) are never read. L == 0 gives a zero output.
 *
 * Work is split into partitions of partition_tokens tokens (0 = library default; else a positive
 * multiple of block_size); a sequence longer than one partition is combined by an exact
 * log-sum-exp merge in a second kernel, using the workspace.
 *
 *   (q_dtype, cache_dtype): (F32, F32), (F16, F16), (BF16, BF16), (F16 | BF16, FP8_E4M3).
 *   out_dtype: q_dtype or PA_F32. Accumulation is fp32 throughout.
 *   k_scale / v_scale: required for fp8 caches (one scale per block and kv head).
 *   num_heads % num_kv_heads == 0; head_dim in {64, 128}; block_size in {8, 16, 32}.
 *   variant: pa_variant; PA_VARIANT_MFMA needs a 16-bit or fp8 cache and at most 16 query heads
 *   per kv head (any supported block size).
 *   flags: 0 or PA_DECODE_SHARED_BLOCKS (a hint, never a change of result): several sequences of
 *   the batch reference the same physical blocks (shared prefixes, parallel samples), so K/V are
 *   read through the caches and a shared block fetched for one sequence is reused by the others.
 *   Without it K/V are streamed non-temporally, which is faster when every block is read once.
 *   workspace: device memory of at least pa_decode_workspace_bytes(...) bytes (may be NULL when
 *   that is 0). Results are deterministic: the same inputs give the same bits, whatever the
 *   physical placement of the blocks.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int num_blocks, float scale, pa_dtype q_dtype,
              pa_dtype cache_dtype, pa_dtype out_dtype, const float* k_scale,
              const float* v_scale, int partition_tokens, int variant, int flags,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid hipMalloc): the same arguments, plan,
 * kernels and result bits as pa_decode, but the partial results of split sequences go to a
 * fixed device array of the library's own (PA_NOALLOC_SCRATCH_BYTES on every GPU the library runs
 * on, held until the process ends) instead of a caller workspace. The call allocates nothing.
 *   Returns PA_ERR_WORKSPACE, before any device work, when the plan pa_decode would pick needs more
 *   than PA_NOALLOC_SCRATCH_BYTES of partial results (pa_decode_workspace_bytes with the same
 *   partition_tokens bounds the need; a smaller partition count or an explicit partition_tokens
 *   that keeps the need below the limit avoids it). Otherwise as pa_decode.
 *   The array is shared by every call on one GPU and nothing in it needs clearing between calls
 *   (every partial result the merge reads is written by the same call). Calls that overlap on one
 *   GPU (on different streams, or from different threads without ordering) race on it.
 *   The array used is the current HIP device's: `stream` must be NULL or a stream of that device
 *   (another device's stream returns PA_ERR_INVALID_ARG).
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int max_blocks_per_seq, int num_blocks, float scale, pa_dtype q_dtype,
                      pa_dtype cache_dtype, pa_dtype out_dtype, const float* k_scale,
                      const float* v_scale, int partition_tokens, int variant, int flags,
                      void* stream);

/*
 * pa_decode_grouped -- pa_decode for a batch whose sequences share prefix blocks (parallel
 * samples of one prompt: [Ultralytics] "シーケンス間でのブロック共有"; [Transcript] the paragraph
 * on shared prefixes), with the shared blocks read once per group instead of once per sequence.
 * The result is pa_decode's, up to the order of the floating-point sums (the prefix and the rest
 * of a sequence are two parts combined by the same log-sum-exp merge as pa_decode's partitions).
 *
 *   group_start    device int32 [num_groups + 1]: sequences group_start[i] .. group_start[i+1]-1
 *                  form group i (consecutive, non-decreasing, group_start[num_groups] = num_seqs).
 *   prefix_blocks  device int32 [num_seqs]: the number of leading table entries sequence s shares
 *                  with the other members of its group -- the same value for every member, the
 *                  entries identical, and at most floor(context_lens[s] / block_size) (whole
 *                  blocks every member attends; 0 = nothing shared). Values that break this give
 *                  undefined results (never a fault), like duplicate slots elsewhere.
 *   max_group_size host int: the largest group; max_group_size * (num_heads / num_kv_heads) <= 16
 *                  (each member's query heads become rows of the matrix-core tile).
 *   workspace      at least pa_decode_grouped_workspace_bytes(...) bytes (never NULL).
 *   flags: PA_DECODE_SHARED_BLOCKS only when blocks are also shared between different groups;
 *                  the kernel itself reads each group's shared blocks once, and streams them
 *                  faster without the hint.
 *   everything else as for pa_decode; the cache must be 16-bit or fp8 (matrix-core kernel).
 */
size_t pa_decode_grouped_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                         int max_blocks_per_seq, int block_size,
                                         int partition_tokens);
int pa_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* group_start, const int32_t* prefix_blocks, int num_groups,
                      int max_group_size, int num_seqs, int num_heads, int num_kv_heads,
                      int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                      float scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                      const float* k_scale, const float* v_scale, int partition_tokens, int flags,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_grouped_append -- pa_decode_grouped with the step's slot write taken along, as
 * pa_decode_append takes it along with pa_decode ([Ultralytics] "ページングの仕組み": the new
 * token goes to its slot): the same result, in the cache and in `out`, as pa_write_kv(k_new,
 * v_new, ..., slot_mapping, num_tokens = num_seqs) followed by pa_decode_grouped, bit for bit.
 * The work-group holding a sequence's own last block (never a shared one: copy-on-write gives the
 * block the step writes into to one sequence) puts the new key and value into its loaded tile
 * and stores the key row and the block's value tile back.
 *
 *   k_new, v_new, slot_mapping, new_dtype  as for pa_decode_append.
 *   everything else as for pa_decode_grouped (same workspace size).
 */
int pa_decode_grouped_append(void* out, const void* q, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const void* k_new, const void* v_new, const int32_t* slot_mapping,
                             pa_dtype new_dtype, const int32_t* group_start,
                             const int32_t* prefix_blocks, int num_groups, int max_group_size,
                             int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                             pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                             const float* k_scale, const float* v_scale, int partition_tokens,
                             int flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_append -- the slot write and the decode of one step in one pass: the same result, in
 * the cache and in `out`, as pa_write_kv(k_new, v_new, ..., slot_mapping, num_tokens = num_seqs)
 * followed by pa_decode ([Ultralytics] "ページングの仕組み": the new token goes to its slot;
 * [Wikipedia] "Математическая формулировка": the query attends every cached token including its
 * own), bit for bit. The new token of sequence s is its position context_lens[s] - 1: the
 * work-group that loads that position's block puts the new key and value (fp8: quantised with the
 * block's scale exactly as pa_write_kv stores them) into the loaded tile in its registers, so no
 * separate write launch precedes the attention. Who stores the token into the cache: with the
 * vector-ALU kernel on its ordered 1-D grid, extra work-groups at the end of the grid, which the
 * hardware dispatches after all the attention's (they run in its drain and store each token as
 * pa_write_kv does); otherwise (the matrix-core kernel, or a 3-D grid: partitions shorter than
 * 1024 tokens, more sequences than the ordered list holds, or PA_DECODE_SHARED_BLOCKS) the
 * work-group holding the block, which stores the key row and the block's whole value tile back.
 *
 *   k_new, v_new  device [num_seqs][num_kv_heads][head_dim] in new_dtype: the cache dtype for a
 *                 16/32-bit cache, q_dtype for an fp8 cache.
 *   slot_mapping  device int32 [num_seqs]: slot of sequence s's new token; it must be the slot of
 *                 position context_lens[s] - 1 of block_tables[s] (that block owned by s alone,
 *                 as copy-on-write guarantees). A negative slot, or one that is not that
 *                 position's, is skipped: nothing is written and the cache is attended as it is.
 *   everything else as for pa_decode (same workspace size).
 */
int pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, const void* k_new,
                     const void* v_new, const int32_t* slot_mapping, pa_dtype new_dtype,
                     int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int num_blocks, float scale, pa_dtype q_dtype,
                     pa_dtype cache_dtype, pa_dtype out_dtype, const float* k_scale,
                     const float* v_scale, int partition_tokens, int variant, int flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill -- causal paged attention of a chunk of new tokens per sequence, each query token
 * attending the cached tokens up to and including its own position ([Wikipedia]
 * "Математическая формулировка": the equations for a query at any position i, the last block cut
 * at i). This is the step before decoding -- a prompt, or a chunk of one, over what is already
 * cached -- and pa_decode is its one-token case.
 *
 *   q, out        device [num_tokens][num_heads][head_dim]; sequence s owns rows
 *                 query_start[s] .. query_start[s+1]-1 (n_s rows, possibly 0).
 *   query_start   device int32 [num_seqs + 1], non-decreasing, query_start[num_seqs] <= num_tokens.
 *   context_lens  device int32 [num_seqs]: tokens cached for s *including* its n_s new ones,
 *                 whose keys and values must already be written (pa_write_kv); query row k of s
 *                 (0-based) sits at position context_lens[s] - n_s + k.
 *   max_query_len host int >= every n_s (rows beyond it are not computed).
 *   block_tables, k_cache, v_cache, scales, dtypes: as for pa_decode (block_size 8, 16 or 32);
 *   the cache 16-bit or fp8 (matrix-core kernel). Rows of a sequence with n_s > context_lens[s]
 *   are cut to the last context_lens[s]. num_tokens == 0 is a no-op. No workspace.
 *   PA_ERR_UNSUPPORTED when ceil(max_query_len * num_heads / num_kv_heads / 64) * num_kv_heads
 *   * num_seqs reaches 2^31 (one work-group per 64-row tile, kv head and sequence).
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
               int num_seqs, int num_tokens, int max_query_len, int num_heads, int num_kv_heads,
               int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
               pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
               const float* k_scale, const float* v_scale, void* stream);

/*
 * pa_swap_blocks -- move whole blocks between the device pool and a host pool in pinned memory,
 * to preempt a group of sequences and resume it later ("vLLM и PagedAttention" (podcast
 * transcript), paragraph on preemption: a group's KV data can be moved to CPU memory and brought
 * back, at the speed of the host link).
 *
 *   k_cache, v_cache (+ k_scale, v_scale): the device pool, num_blocks blocks, layout above.
 *   host_k, host_v (+ host_k_scale, host_v_scale): a host pool of num_host_blocks blocks in the
 *     same layout, in pinned host memory (hipHostMalloc, or a pinned torch tensor).
 *   block_pairs: int32 [num_pairs][2] = (src, dst), in device memory or pinned host memory.
 *     PA_SWAP_OUT: device block src -> host block dst. PA_SWAP_IN: host block src -> device
 *     block dst. Both caches, every kv head, and for fp8 caches both scales. The dsts must be
 *     distinct; a pair naming a block outside its pool is skipped.
 *   Scales: required on both sides for PA_FP8_E4M3 caches, ignored otherwise.
 * Every pointer's kind is checked with hipPointerGetAttributes before the launch: a device
 * pointer that is not device memory, or a host pointer that is not pinned, returns
 * PA_ERR_INVALID_ARG (pageable host memory cannot be read by the kernel). The kernel accesses the
 * host pool directly over the host link; the host pool must stay allocated until the stream has
 * passed the call. num_pairs == 0 is a no-op.
 */
typedef enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 } pa_swap_direction;

int pa_swap_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int num_blocks,
                   void* host_k, void* host_v, float* host_k_scale, float* host_v_scale,
                   int num_host_blocks, const int32_t* block_pairs, int num_pairs, int direction,
                   int num_kv_heads, int head_dim, int block_size, pa_dtype cache_dtype,
                   void* stream);

/*
 * Profiling: when enabled, every pa_* call's kernel launch carries a pair of HIP events that the
 * runtime stamps at that kernel's own start and end (hipExtLaunchKernel). pa_profile_read
 * synchronises on those events and returns, for one kernel kind, the summed kernel time in
 * milliseconds and the number of launches since the last reset.
 */
typedef enum {
  PA_KERNEL_DECODE_PARTITION = 0, /* the attention kernel (VALU or MFMA variant)      */
  PA_KERNEL_DECODE_MERGE = 1,     /* the log-sum-exp merge of partitions              */
  PA_KERNEL_WRITE_KV = 2,
  PA_KERNEL_COPY_BLOCKS = 3,
  PA_KERNEL_GATHER_KV = 4,
  PA_KERNEL_SWAP_BLOCKS = 5,
  PA_KERNEL_PREFILL = 6
} pa_kernel_kind;

int pa_profile_enable(int on);  /* also resets the counters */
int pa_profile_read(int kernel_kind, double* total_ms, long long* launches);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
