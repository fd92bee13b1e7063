/*
 * gqa_decode.h - C ABI of the MI355X (gfx950) incremental-decoding attention
 * library for multi-head, grouped-query and multi-query attention.
 *
 * One decoding step of one attention layer, with the projections left to the
 * caller, is:
 *
 *   gqa_kv_append(...)          store the new token's K and V rows in the cache
 *   gqa_decode_attention(...)   let the new token's h query heads attend over
 *                               every cached position, the new one included
 *
 * in that order on one stream, or both at once with gqa_decode_step (one
 * launch). Around that core the library also offers: the same three calls on
 * paged caches (*_paged), n new tokens per sequence with a causal mask
 * (*_multi, and *_multi_paged over paged caches), the layer's projections
 * and the whole layer step (gqa_pack_weight, gqa_linear, gqa_decode_layer),
 * the mean-fold of KV heads that turns an MHA cache into a GQA one
 * (gqa_fold_kv_heads), and a streaming read that measures the bandwidth the
 * decode kernels are held to (gqa_read_bandwidth).
 * The step is the per-layer decode loop of the
 * "LLM inference 05" notes (albangk): push K, push V, then attend; and the
 * incremental attention of the "Fast Transformer Decoding: One Write-Head is
 * All You Need" review (velog), §2.4 Multi-head Attention (Incremental) and
 * §3 Multi Query Attention, with the projections removed.
 *
 * Grouping (the "TF2 GQA" lesson, ttlab: the g-knob table and the lab): h
 * query heads share g KV heads; g = h is MHA, g = 1 is MQA, and h must be a
 * multiple of g. Query head i reads KV head floor(i / (h/g)), i.e. query heads
 * form contiguous groups.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer on the current HIP device, owned
 *   by the caller. The library never allocates, frees or keeps device memory
 *   and keeps no state between calls apart from host-side caches of device
 *   attributes and kernel occupancy (safe to fill from several threads) and
 *   the calling thread's last error message. The workspace of the attention
 *   calls is the caller's too; a call leaves its counters at zero.
 * - All tensors are dense and row-major (C-contiguous) with the shapes given
 *   below; element type is one of GQA_DTYPE_*; q, caches, new rows and out
 *   share it.
 * - Caches: K is [b][g][cap][d_k], V is [b][g][cap][d_v]. Position t of
 *   sequence s, KV head j starts at element ((s*g + j)*cap + t)*d.
 * - lens is an int32 [b] device array: the number of valid cache positions
 *   of each sequence.
 * - max_len is the caller's host-side upper bound of lens (see each call).
 *   It sizes the launch; positions at or beyond min(lens[s], max_len) are
 *   never read.
 * - stream is a hipStream_t passed as void* (NULL: the null stream). Calls
 *   are asynchronous on it: a return of GQA_OK means "enqueued".
 * - All argument checks run on the host before anything is enqueued, so an
 *   error return leaves every buffer untouched and enqueues nothing.
 *   gqa_last_error() then describes the failure.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. bf16 is stored as the upper 16 bits of an IEEE fp32. */
#define GQA_DTYPE_F32 0
#define GQA_DTYPE_BF16 1

/* Status codes. */
#define GQA_OK 0
#define GQA_ERR_ARG (-1)         /* null pointer, or a size <= 0 / too large     */
#define GQA_ERR_GROUPS (-2)      /* h is not a multiple of g                     */
#define GQA_ERR_UNSUPPORTED (-3) /* dtype, head dims or options not supported    */
#define GQA_ERR_CAPACITY (-4)    /* max_len (plus the appended token) > cap      */
#define GQA_ERR_WORKSPACE (-5)   /* workspace missing or smaller than required   */
#define GQA_ERR_HIP (-6)         /* the HIP runtime refused a launch or a query  */

/* Path selection for gqa_decode_attention_ex. */
#define GQA_PATH_AUTO 0
#define GQA_PATH_VECTOR 1 /* vector-ALU kernel: every supported shape and dtype   */
#define GQA_PATH_MATRIX 2 /* MFMA kernel: bf16, d_k = d_v = 128, up to 64 heads/KV */

/* How segments split over several workgroups are merged; OR one into path. */
#define GQA_MERGE_INLINE 0x10 /* by the segment's last workgroup, inside the decode launch */
#define GQA_MERGE_KERNEL 0x20 /* by a second launch, one workgroup per (segment, head)  */
/* By the segment's parts themselves at the end of the decode launch, each
   merging a slice of the heads (the stream kernel only: bf16, d = 128, 3-64
   heads per KV head, b <= 64, through gqa_decode_attention_ex and
   gqa_decode_step_ex; GQA_ERR_UNSUPPORTED elsewhere). */
#define GQA_MERGE_SPREAD 0x80
/* Reported by gqa_decode_plan only: the matrix path runs its streaming
   kernel (3-64 query heads, or virtual heads of several tokens, per KV
   head, b <= 64). */
#define GQA_PLAN_STREAM 0x40

/*
 * Append one token per sequence ("LLM inference 05": push K, push V;
 * MQA review §2.4 / §3: the new row is concatenated on the position axis).
 *
 * For every sequence s and KV head j < g, with p = lens[s]:
 *   K[s][j][p][:] = k_new[s][j][:]   (d_k elements, copied bit for bit)
 *   V[s][j][p][:] = v_new[s][j][:]   (d_v elements)
 * then lens[s] = p + 1.
 *
 * k_new: [b][g][d_k], v_new: [b][g][d_v] (device, read only).
 * k_cache, v_cache, lens: device, updated in place.
 * max_len: host upper bound of lens[s] BEFORE the call; max_len + 1 <= cap is
 *   checked (GQA_ERR_CAPACITY).
 * Device-side precondition: 0 <= lens[s] <= max_len. A sequence whose lens[s]
 *   is outside [0, cap) is left untouched (nothing written, lens unchanged).
 * Errors: GQA_ERR_ARG (null pointer, b/g/d/cap <= 0, b > 65535),
 *   GQA_ERR_UNSUPPORTED (dtype), GQA_ERR_CAPACITY, GQA_ERR_HIP.
 */
int gqa_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  int32_t* lens, int b, int g, int d_k, int d_v, int cap, int max_len,
                  int dtype, void* stream);

/*
 * Bytes of device workspace gqa_decode_attention needs for this shape; the
 * value covers every path and launch size, so one buffer serves all calls
 * with b, h/g and d_v no larger than these (it does not grow with max_len).
 * Returns 0 for invalid arguments.
 *
 * The workspace (256-byte aligned) holds the split-softmax partial states of
 * the persistent workgroups from its start, and int32 counters and flags at
 * its end: the last 36864 + 65792 + c bytes (of the buffer's size rounded
 * down to 256), where c = 4*n rounded up to a multiple of 256, with n = 32*b*h
 * if b*h <= 8192, else max(b*h, 262144). Those bytes must be ZERO before the
 * first call that uses a buffer (e.g. allocate it zero-filled). Every call
 * leaves the first 36864 + c of them zero again; the last 65792 hold launch
 * stamps (a generation count and flags tagged with it) that calls merging
 * split segments with GQA_MERGE_SPREAD update and never reset: leave them as
 * they are between calls, or zero them together with the rest. Because the counters are
 * placed from the end, a buffer sized for one shape serves any sequence of
 * calls with b, h, h/g and d_v no larger. Two calls that share a workspace
 * must be ordered (same stream or synchronised); calls with distinct
 * workspaces may run concurrently.
 */
size_t gqa_decode_workspace_size(int b, int h, int g, int d_k, int d_v, int max_len, int dtype);

/*
 * Attention of one query token per sequence over its cache (MQA review §2.1
 * Dot-Product Attention applied per query head, §2.4 / §3 for the cache):
 *
 *   for s < b, i < h, j = floor(i / (h/g)), L = min(lens[s], max_len):
 *     w_t = softmax_t( scale * sum_k q[s][i][k] * K[s][j][t][k] ),  t < L
 *     out[s][i][v] = sum_t w_t * V[s][j][t][v]
 *
 * q: [b][h][d_k], out: [b][h][d_v], in the input element type (bf16 outputs
 * are rounded to nearest even from fp32 accumulation). A sequence with L = 0
 * gets an all-zero output row.
 * lens: attended lengths (AFTER this step's append). max_len: host upper bound
 *   of lens, 0 <= max_len <= cap (GQA_ERR_CAPACITY otherwise).
 * scale: multiplies every logit (1/sqrt(d_k) for the usual scaled attention;
 *   1 reproduces the pages' unscaled einsum).
 * workspace / workspace_bytes: see gqa_decode_workspace_size.
 * Supported: dtype F32 or BF16; d_k == d_v in {16, 32, 64, 128, 256};
 *   b <= 65535; h <= 4096.
 * Errors: GQA_ERR_ARG, GQA_ERR_GROUPS, GQA_ERR_UNSUPPORTED, GQA_ERR_CAPACITY,
 *   GQA_ERR_WORKSPACE, GQA_ERR_HIP.
 */
int gqa_decode_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap,
                         int max_len, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * gqa_decode_attention with explicit launch choices, for tests and tuning.
 * path: GQA_PATH_AUTO / GQA_PATH_VECTOR / GQA_PATH_MATRIX (MATRIX on an
 *   unsupported shape gives GQA_ERR_UNSUPPORTED), optionally OR-ed with one
 *   of GQA_MERGE_INLINE, GQA_MERGE_KERNEL or GQA_MERGE_SPREAD to fix how
 *   split segments are merged (default: a second launch once a segment's
 *   partial states exceed 64 KiB, e.g. few long sequences with many heads
 *   per KV head, else inside the launch). The second launch goes to the
 *   same stream. GQA_MERGE_SPREAD keeps the call to one launch; it uses the
 *   workspace's stamp region (see gqa_decode_workspace_size).
 * workgroups: size of the persistent grid that splits the work evenly;
 *   0 = automatic (compute units x resident workgroups per unit), otherwise
 *   1 .. 2048 (GQA_ERR_UNSUPPORTED outside that range).
 * Results equal gqa_decode_attention's up to floating-point summation order.
 */
int gqa_decode_attention_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap,
                            int max_len, float scale, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream, int path, int workgroups);

/*
 * One whole decoding step in one launch: gqa_kv_append followed by
 * gqa_decode_attention ("LLM inference 05": push K, push V, then attend;
 * the new position attends to every earlier one and to itself).
 *
 * For every sequence s, with p = lens[s] (clamped to [0, max_len]):
 *   K[s][j][p] = k_new[s][j], V[s][j][p] = v_new[s][j]   (bit for bit)
 *   out[s][i]  = attention of q[s][i] over positions [0, p + 1)
 *   lens[s]    = p + 1
 * The appended row is taken straight from k_new / v_new for the attention
 * and stored into the cache by the same kernel; lens is updated by the last
 * workgroup to finish, after every workgroup has read it.
 * max_len: host upper bound of lens BEFORE the call; max_len + 1 <= cap
 *   (GQA_ERR_CAPACITY). Results equal the two-call sequence up to
 *   floating-point summation order; caches and lens equal it bit for bit.
 * Same shapes, workspace rules and errors as gqa_decode_attention (the
 * workspace's counters include the step's finish counter).
 */
int gqa_decode_step(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap, int max_len,
                    float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* gqa_decode_step with the launch choices of gqa_decode_attention_ex. */
int gqa_decode_step_ex(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap,
                       int max_len, float scale, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream, int path, int workgroups);

/*
 * Projection weights are used in a packed layout: gqa_pack_weight reads a
 * bf16 matrix w [n_out][n_in] (row o holds output feature o's weights,
 * PyTorch's Linear layout) and writes gqa_packed_weight_bytes(n_out, n_in)
 * bytes to dst (16-byte aligned, caller-owned, must not overlap src): the
 * matrix cut into tiles of 16 rows x 32 columns, zero-padded at the edges,
 * each tile in the order the matrix cores read it, the tiles of 16 rows
 * consecutive. Pack once per weight matrix, reuse for every step.
 * gqa_packed_weight_bytes returns 0 for non-positive sizes.
 */
size_t gqa_packed_weight_bytes(int n_out, int n_in);
int gqa_pack_weight(void* dst, const void* src, int n_out, int n_in, int dtype, void* stream);

/*
 * A linear projection of the decode batch: y[r][o] = sum_k x[r][k] * w[o][k]
 * for r < rows, o < n_out (the token's vector times a projection matrix, as
 * in the MQA review, §2.4: q = x P_q, k = x P_k, v = x P_v, and the output
 * y = o P_o). All arrays are bf16 (GQA_DTYPE_BF16 only; anything else gives
 * GQA_ERR_UNSUPPORTED): x [rows][n_in] and y [rows][n_out] row-major and
 * contiguous, w packed by gqa_pack_weight from its [n_out][n_in] form.
 * Accumulation in fp32, y rounded to bf16 (nearest even).
 * rows in [1, 64] (a decode batch) and n_in a multiple of 8, else
 * GQA_ERR_UNSUPPORTED; x and w 16-byte aligned, else GQA_ERR_ARG. y must not
 * overlap x or w. Asynchronous on stream.
 */
int gqa_linear(void* y, const void* x, const void* w, int rows, int n_in, int n_out, int dtype, void* stream);

/*
 * One attention step of a decoder layer for the new token of each of b
 * sequences (the MQA review, §2.4 incremental multi-head attention, with the
 * K/V head axis of size g as in §3 for g = 1 and the TF2 GQA lesson for
 * 1 < g < h):
 *   q     = x W_q^T   -> [b][h][d_k]      (query projection)
 *   k_new = x W_k^T   -> [b][g][d_k]      (key projection)
 *   v_new = x W_v^T   -> [b][g][d_v]      (value projection)
 *   gqa_decode_step(attn, q, k_new, v_new, caches, lens, ...)  -> attn [b][h][d_v]
 *   y     = attn W_o^T -> [b][d_model]    (output projection)
 * x [b][d_model]; the weights packed by gqa_pack_weight from
 * W_q [h*d_k][d_model] (row i*d_k + c holds the pages' P_q[i][:][c]),
 * W_k [g*d_k][d_model], W_v [g*d_v][d_model] and W_o [d_model][h*d_v]
 * (row m, column i*d_v + c holds P_o[i][m][c]).
 * q, k_new, v_new and attn are caller-owned scratch of the sizes above; they
 * hold the intermediate results when the call completes. The projections'
 * outputs are stored in bf16 before the append and attention use them.
 * bf16 only; b <= 64; d_model and h*d_v multiples of 8; caches, lens, cap,
 * max_len, scale and workspace as in gqa_decode_step (lens grows by one).
 * Every check runs before anything is enqueued; three launches on stream
 * (one for the three input projections, the step, the output projection),
 * four when the step merges split segments in a second launch.
 */
int gqa_decode_layer(void* y, const void* x, const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                     void* q, void* k_new, void* v_new, void* attn, void* k_cache, void* v_cache, int32_t* lens,
                     int b, int h, int g, int d_model, int d_k, int d_v, int cap, int max_len, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-token decode: n new tokens per sequence in one step (speculative or
 * chunked decoding), the batched form of the MQA review (§2.3: n query
 * positions of each sequence at once, with an additive mask) with the causal
 * mask: the new tokens sit at positions L .. L + n - 1 after the cache's L
 * rows, and token r attends every cached position and the new tokens up to
 * and including itself (the "LLM inference 05" notes: under the causal mask
 * a position's K and V depend only on the positions up to it).
 *   q, out      [b][n][h][d]   (token-major; out same dtype as q)
 *   k_new, v_new [b][n][g][d]
 * gqa_kv_append_multi writes token r of sequence s at position lens[s] + r
 * and adds n to lens[s] (max_len + n <= cap, else GQA_ERR_CAPACITY; a device
 * length with lens[s] + n > cap leaves that sequence untouched).
 * gqa_decode_attention_multi: lens[s] is the attended length of the LAST
 * new token (the cache already holds the n new rows); token r attends
 * positions t < lens[s] - (n - 1 - r). max_len bounds lens on the host.
 * gqa_decode_step_multi = append, then attention, with the same result as
 * the two calls: one launch where the tiles holding the new positions store
 * the new rows before reading them (bf16, d = 128, n * h/g <= 64, b <= 64),
 * else two launches; every check runs before anything is enqueued; max_len
 * bounds the lengths before the append.
 * All n tokens of a KV group share each K/V tile: the n * h/g query rows of a
 * group run together (on the matrix cores for bf16, d = 128 and
 * n * h/g <= 64; otherwise on the vector path, a head block at a time), so
 * the bytes read do not grow with n. Element types and head dims as for
 * gqa_decode_attention; 1 <= n <= 64 and n * h <= 4096 (GQA_ERR_ARG). The
 * workspace is gqa_decode_multi_workspace_size bytes (that of a one-token
 * call with n * h query heads), same rules as gqa_decode_attention.
 */
size_t gqa_decode_multi_workspace_size(int b, int n, int h, int g, int d_k, int d_v, int dtype);
int gqa_kv_append_multi(void* k_cache, void* v_cache, const void* k_new, const void* v_new, int32_t* lens, int b,
                        int n, int g, int d_k, int d_v, int cap, int max_len, int dtype, void* stream);
int gqa_decode_attention_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* lens, int b, int n, int h, int g, int d_k, int d_v, int cap,
                               int max_len, float scale, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream);
int gqa_decode_step_multi(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                          void* v_cache, int32_t* lens, int b, int n, int h, int g, int d_k, int d_v, int cap,
                          int max_len, float scale, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Paged caches. The "LLM inference 05" notes name block-table (vLLM-style)
 * caches without fixing a layout; this library reads them as follows. K and
 * V live in pools of blocks of block_size positions:
 *   k_pool [num_blocks][g][block_size][d_k], v_pool [num_blocks][g][block_size][d_v]
 * and block_table int32 [b][max_blocks] (row stride max_blocks) names, for
 * sequence s, the pool block holding its positions n*block_size ..
 * (n+1)*block_size - 1 in entry [s][n]. Position t of KV head j of sequence
 * s is k_pool[block_table[s][t / block_size]][j][t % block_size]. A sequence
 * holds at most max_blocks * block_size positions (its "cap").
 * block_size is a power of two in [32, 2^20]: a 32-position tile of the
 * decode kernels then never straddles two blocks. b * max_blocks < 2^31.
 * Table entries the call needs (positions < the attended length, and the
 * append position) must be valid ids; the kernels clamp any id into
 * [0, num_blocks), so a bad id reads or writes the wrong block of the pool
 * but never memory outside it. Entries past a sequence's last needed block
 * are never read. All pointers are caller-owned device memory. Results are
 * exactly those of the contiguous entry points on the cache the pool stands
 * for (same kernels, same schedule, same arithmetic).
 */

/* gqa_kv_append on a paged cache: the new rows go to position lens[s]. */
int gqa_kv_append_paged(void* k_pool, void* v_pool, const void* k_new, const void* v_new, int32_t* lens,
                        const int32_t* block_table, int b, int g, int d_k, int d_v, int block_size, int max_blocks,
                        int num_blocks, int max_len, int dtype, void* stream);

/* gqa_decode_attention on paged caches (workspace as for the contiguous call). */
int gqa_decode_attention_paged(void* out, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* lens, const int32_t* block_table, int b, int h, int g, int d_k,
                               int d_v, int block_size, int max_blocks, int num_blocks, int max_len, float scale,
                               int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* gqa_decode_step (append + attention in one launch) on paged caches. */
int gqa_decode_step_paged(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                          void* v_pool, int32_t* lens, const int32_t* block_table, int b, int h, int g, int d_k,
                          int d_v, int block_size, int max_blocks, int num_blocks, int max_len, float scale,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-token decode over paged caches: the *_multi calls above with the
 * caches replaced by block pools and a block table, laid out as for the paged
 * calls (pools [num_blocks][g][block_size][d], table int32 [b][max_blocks],
 * ids clamped into the pool). A sequence holds max_blocks * block_size
 * positions; an append of n tokens needs max_len + n of them (else
 * GQA_ERR_CAPACITY, nothing enqueued) and may cross into a new block, whose
 * table entry must then be valid. q, out, k_new, v_new, n, the causal limits,
 * the workspace (gqa_decode_multi_workspace_size) and the error rules are
 * those of the contiguous *_multi calls, and so are the results, bit for bit,
 * on the cache the pool stands for.
 */
int gqa_kv_append_multi_paged(void* k_pool, void* v_pool, const void* k_new, const void* v_new, int32_t* lens,
                              const int32_t* block_table, int b, int n, int g, int d_k, int d_v, int block_size,
                              int max_blocks, int num_blocks, int max_len, int dtype, void* stream);
int gqa_decode_attention_multi_paged(void* out, const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* lens, const int32_t* block_table, int b, int n, int h, int g,
                                     int d_k, int d_v, int block_size, int max_blocks, int num_blocks, int max_len,
                                     float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);
int gqa_decode_step_multi_paged(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                void* v_pool, int32_t* lens, const int32_t* block_table, int b, int n, int h, int g,
                                int d_k, int d_v, int block_size, int max_blocks, int num_blocks, int max_len,
                                float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mean-fold of KV heads ("TF2 GQA" lesson, on moving a trained multi-head
 * model to grouped-query attention: each contiguous group of key/value heads
 * is replaced by its average; the lesson's lab folds them that way and
 * compares the outputs at the same weights). With F = g_src / g_dst:
 *   dst[s][j][t][c] = (sum_{f<F} src[s][j*F + f][t][c]) / F
 * for s < b, j < g_dst, t < rows_s, c < d, where rows_s = lens[s] (device
 * int32, clamped to [0, max_rows]) or max_rows for every s when lens is
 * NULL. The sum runs in head order in double precision and the mean is
 * rounded once to the element type (nearest even; a NaN becomes bf16
 * 0x7fc0), so the result is bitwise reproducible.
 * src [b][g_src][cap_src][d] and dst [b][g_dst][cap_dst][d], contiguous,
 * 16-byte aligned, caller-owned device memory that must not overlap; rows of
 * dst at or beyond rows_s are not written. Fold the K and the V cache with
 * one call each. A key or value projection W [g*d_k][d_model] folds as b = 1,
 * cap = max_rows = d_k, d = d_model, lens = NULL.
 * Errors: null pointers, sizes <= 0 (max_rows < 0), misalignment or overlap
 * GQA_ERR_ARG; g_src % g_dst != 0 GQA_ERR_GROUPS; d % 8 != 0 or another
 * dtype GQA_ERR_UNSUPPORTED; max_rows > cap_src or cap_dst GQA_ERR_CAPACITY.
 * max_rows = 0 enqueues nothing. Asynchronous on stream.
 */
int gqa_fold_kv_heads(void* dst, const void* src, const int32_t* lens, int b, int g_src, int g_dst, int cap_src,
                      int cap_dst, int d, int max_rows, int dtype, void* stream);

/*
 * Read bandwidth of this part, for stating the decode kernels' roofline
 * against what the memory system sustains as well as against the nominal
 * peak (decode is memory-bound: "LLM inference 05", the decode phase).
 * Reads the `bytes` bytes at src (device memory, 16-byte aligned, bytes a
 * multiple of 16) once, with a persistent grid of `workgroups` 512-thread
 * workgroups (1 .. 2048; one per compute unit is the decode kernels' grid)
 * and the decode kernels' non-temporal 16-byte loads: workgroup w reads the
 * contiguous chunks [w n / P, (w + 1) n / P) of the n = bytes / 16 chunks and
 * writes the sum of their 32-bit words (mod 2^32) to sink[w] (device
 * uint32 [workgroups]), so the sink's total is the sum of every word of the
 * buffer. Errors: GQA_ERR_ARG (null pointers, alignment, workgroups out of
 * range, more than 2 GiB per workgroup), GQA_ERR_HIP. Asynchronous on stream.
 */
int gqa_read_bandwidth(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream);

/*
 * Describe the launch gqa_decode_attention_ex would make on the current
 * device, without enqueueing anything: writes the chosen path
 * (GQA_PATH_VECTOR or GQA_PATH_MATRIX, OR-ed with the GQA_MERGE_* flag in
 * effect and with GQA_PLAN_STREAM when the matrix path runs its one-block
 * streaming kernel) and persistent grid size. Same argument checks as the real call,
 * minus pointers.
 */
int gqa_decode_plan(int b, int h, int g, int d_k, int d_v, int cap, int max_len, int dtype,
                    int path, int workgroups, int* chosen_path, int* chosen_workgroups);

/*
 * gqa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The workspace is an 8 MiB array inside
 * the library, one per GPU, kept for the life of the process; the call
 * allocates nothing. Same arguments, results (bit for bit), ordering and
 * errors as gqa_decode_step, plus GQA_ERR_WORKSPACE when the shape needs
 * more than the 8 MiB (partial slots are reserved only for the planned grid:
 * the Llama-3-70B-shaped step, b = 16, h = 64, g = 8, d = 128, needs about
 * 2.3 MB) and GQA_ERR_HIP if the array's device address cannot be obtained.
 * All calls on one GPU share the array: calls that overlap on one GPU
 * (different streams, not synchronised) race and must be serialised.
 */
int gqa_decode_step_static(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                           void* v_cache, int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap, int max_len,
                           float scale, int dtype, void* stream);

/* Message for the calling thread's last non-OK return ("" if none). */
const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
