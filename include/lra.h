/*
 * lra.h - C ABI of the Flash-LoRA-Attention library for AMD Instinct MI355X (gfx950).
 *
 * What it computes (LRAgent: "Efficient KV Cache Sharing for Multi-LoRA LLM
 * Agents", core method and method steps (2)-(4); PReCache, PreLRShared):
 * agents share one key cache K_base and one base value cache V_base = X W0.
 * Each agent k keeps only a rank-r value cache V_lr = X A_k. Attention for
 * agent a streams K/V_base/V_lr tiles with an online softmax, accumulates the
 * base output O and a rank-r output O_lr, and after the last tile applies one
 * up-projection O += O_lr B_a, then normalises. V_base + V_lr B_a is never
 * built. The LR precompute produces X [A_1 .. A_N] for all agents at once.
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are device pointers on the current HIP device;
 *    pointers marked (host) are host pointers. Scalars are host values.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the null
 *    stream). A return of LRA_OK means the work was enqueued.
 *  - The caller allocates and owns every buffer, including workspaces. The
 *    library allocates nothing, keeps no pointer after it returns, and holds no
 *    state between calls, so calls on different streams with different
 *    workspaces may run concurrently.
 *  - All tensors are dense and row-major; one element type (`dtype`) per call:
 *    LRA_F32 (IEEE float) or LRA_BF16 (bfloat16 bits). Accumulation is fp32;
 *    bf16 outputs are rounded to nearest, ties to even.
 *  - The softmax scale must be positive and finite (the workloads use 1/sqrt(d_head)).
 *  - Scalar arguments are validated on the host before anything is enqueued;
 *    a failing call enqueues nothing and returns a negative lra_status.
 *    lra_last_error() gives a message for the calling thread's last failure.
 *    Errors reported by the HIP runtime at launch come back as LRA_ERR_HIP.
 *  - Device-side index arrays (kv_start, kv_len, agent, out_rows) cannot be
 *    checked on the host. The kernels check them against the sizes passed in
 *    and never access memory outside the buffers those sizes describe: a
 *    decode request with an invalid range or agent gets NaN in every output
 *    element; a precompute row whose out_rows entry is out of range is not
 *    written.
 *  - Agent index -1 (LRA_ADAPTER_FREE) selects the adapter-free view of double
 *    batching (PReCache paper, section 3, ReBaseShared: the adapter-free path
 *    processes the same tokens and attends only to the neutral base cache):
 *    O is attention over K_base and V_base alone, with no LR term. Adapted and
 *    adapter-free decode requests can share one launch.
 *  - Supported: d_head in {64, 128}; rank in {8, 16}; n_q % n_kv == 0 with
 *    group size n_q / n_kv in 1..8. Anything else returns LRA_ERR_UNSUPPORTED.
 *  - The LR cache V_lr holds, for cache row t, agent k and rank column j, the
 *    element at t * ld_vlr + k * vlr_agent_stride + j. Two layouts are accepted
 *    where an entry point takes vlr_agent_stride: interleaved rows (each row
 *    holds every agent's columns: vlr_agent_stride = rank, ld_vlr >= N*rank),
 *    or agent-major (each agent's cache contiguous, [N x rows x ld_vlr] with
 *    ld_vlr >= rank and vlr_agent_stride >= rows * ld_vlr). Both strides are
 *    multiples of 8; anything else returns LRA_ERR_SHAPE. In the agent-major
 *    layout a request reads only its own agent's bytes of each row. Entry
 *    points without vlr_agent_stride (paged caches, lra_expand_values) take
 *    interleaved rows.
 *
 * Names follow the pages: Q, K_base, V_base, V_lr, B_i, agent i, L_P (tokens
 * already cached), L_C (new tokens of the chunk), r (rank), N (agents).
 */
#ifndef LRA_H
#define LRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LRA_ABI_VERSION 8   /* 2: agent index -1 selects the adapter-free view; 3: lra_expand_values;
                                4: lra_attn_decode_strided; 5: lra_attn_decode_paged_strided;
                                6: finite inputs beyond the fp16 range accepted everywhere (range-safe
                                   recomputation); the qkvo decode workspace holds fp32 key scores;
                                   lra_attn_decode_noalloc;
                                7: stream-K decode slices and a new record layout (workspace sizes
                                   changed); the LR precompute needs no workspace;
                                   lra_attn_decode_step;
                                8: one round of decode workgroups, each streaming its slice as
                                   one sequence of tiles (workspace sizes changed);
                                   lra_stream_read; the LR cache's agent stride (vlr_agent_stride)
                                   on every entry point over contiguous caches: agent-major caches;
                                   small batches of lra_attn_decode in 128/256-key chunks */

typedef enum {
    LRA_OK = 0,
    LRA_ERR_NULL = -1,        /* a required pointer is NULL */
    LRA_ERR_SHAPE = -2,       /* sizes, strides or ranges are inconsistent */
    LRA_ERR_UNSUPPORTED = -3, /* a dtype / d_head / rank / group size the kernels do not cover */
    LRA_ERR_INDEX = -4,       /* a host-side index (agent) is out of range */
    LRA_ERR_WORKSPACE = -5,   /* workspace missing, too small or misaligned */
    LRA_ERR_HIP = -6          /* the HIP runtime reported an error */
} lra_status;

typedef enum { LRA_F32 = 0, LRA_BF16 = 1 } lra_dtype;

/* agent index of the adapter-free view (attention over the base cache alone, no LR term) */
#define LRA_ADAPTER_FREE (-1)

/* ABI version of the loaded library (LRA_ABI_VERSION at build time). */
int lra_abi_version(void);

/* Static string naming a status code; never NULL. */
const char* lra_status_str(int status);

/* Message describing the calling thread's most recent failed call ("" if none). */
const char* lra_last_error(void);

/* ------------------------------------------------------------------------------------------------
 * LR precompute (PReCache, PreLRShared: when a segment is first processed, every agent's
 * down-projection is applied to its hidden states; LRAgent method step (2): V_lr = X A, L x r).
 *
 *   V_lr(row out_rows[t], agent k, column j) = sum_c X[t, c] * A[k*rank + j, c]    t < T, k < N, j < rank
 *
 * X        (device) [T x d_model], row stride ldx elements (ldx >= d_model, multiple of 8)
 * A        (device) [n_agents*rank x d_model] row-major: row k*rank + j holds column j of A_k,
 *          i.e. the agents' LoRA down-projection weights (each r x d_model) stacked. This is the
 *          transpose of the pages' side-by-side [A_1 .. A_N] ([d_model x n_agents*rank]): stored
 *          this way, both matrix-core operands (X rows and A rows) are contiguous along d_model,
 *          and it is the usual storage of LoRA down-projection weights.
 * V_lr     (device) output cache of vlr_rows rows in either layout (conventions above; with the
 *          agent-major one, vlr_agent_stride >= vlr_rows * ld_vlr); only the n_agents*rank
 *          entries of the addressed rows are written
 * out_rows (device) [T] int64 destination row of each X row, or NULL for row t -> row t
 *          (then vlr_rows >= T is required)
 * workspace(device) lra_lr_precompute_workspace_bytes() bytes, which is 0: the reduction over
 *          d_model finishes inside one launch. workspace may be NULL; the argument is kept so
 *          that a later kernel may use scratch without changing the call.
 * T = 0 is allowed and enqueues nothing. d_model must be a multiple of 32.
 * Every tensor pointer must be 16-byte aligned.
 */
size_t lra_lr_precompute_workspace_bytes(int64_t T, int32_t d_model, int32_t n_agents, int32_t rank);

int lra_lr_precompute(int dtype, const void* X, int64_t T, int32_t d_model, int64_t ldx,
                      const void* A, int32_t n_agents, int32_t rank,
                      void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride, int64_t vlr_rows,
                      const int64_t* out_rows, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Causal chunked prefill for one agent (LRAgent method steps (3)-(4); PReCache: the new chunk of
 * L_C tokens follows L_P reused tokens). Query i (0 <= i < L_C) sits at absolute position L_P + i
 * and attends keys 0 .. L_P + i. Query head h reads KV head g = h / (n_q / n_kv).
 *
 *   O[i, h] = ( sum_j p_ij V_base[j, g] + (sum_j p_ij V_lr[j, agent*rank : agent*rank+rank]) B_agent[:, g*d : g*d+d] )
 *             / sum_j p_ij,        p_ij = exp(scale * <Q[i, h], K_base[j, g]> - m_i)
 *
 * Q        (device) [L_C x n_q x d_head]
 * K_base   (device) [L_P+L_C x n_kv x d_head]    (rows 0 .. L_P+L_C-1 are read)
 * V_base   (device) [L_P+L_C x n_kv x d_head]
 * V_lr     (device) L_P+L_C rows in either layout (conventions above; rows = L_P+L_C)
 * B        (device) [n_agents x rank x n_kv*d_head]: B_a, one r x (n_kv*d_head) matrix per agent
 * agent    (host) in [0, n_agents), or -1 for the adapter-free view (V_lr and B are not read);
 *          anything else returns LRA_ERR_INDEX
 * O        (device) [L_C x n_q x d_head] output
 * bf16 inputs: Q.K products are exact (bf16 operands, fp32 accumulation). For P.V the
 * probabilities are rounded to fp16 and V_base / V_lr converted exactly to fp16; a workgroup (256
 * query rows of one KV head) whose sums come out non-finite (it staged an entry beyond the fp16
 * range, |v| > 65504, or its fp32 sums overflowed near the bf16 maximum) recomputes its rows with
 * bf16 V_base / V_lr (scaled by a power of two when huge) and the probabilities split into two bf16
 * parts, so every finite input is accepted. l, m, O and O_lr are fp32; scores must stay finite in
 * fp32.
 * Every tensor pointer must be 16-byte aligned. n_kv*d_head and ld_vlr must not exceed 2^22 (the
 * kernel reads 64-row tiles through 32-bit offsets); larger values return LRA_ERR_SHAPE. L_C = 0
 * enqueues nothing.
 */
int lra_attn_prefill(int dtype, const void* Q, int64_t L_C, int64_t L_P,
                     const void* K_base, const void* V_base, const void* V_lr, int64_t ld_vlr,
                     int64_t vlr_agent_stride, const void* B, int32_t n_agents, int32_t agent,
                     int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                     void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * lra_attn_prefill with LoRA on the key projection as well (the qkvo configuration; LRAgent page,
 * limitations, and PReCache summary page, which adapt q and v by default): the agent's keys are
 *
 *   K_a[j, g] = K_base[j, g] + RoPE_j( (K_lr[j, agent*rank : agent*rank+rank] B_k[agent])[g*d : g*d+d] )
 *
 * where RoPE_j turns the pair (y_i, y_{i+d/2}) (i < d/2) by the angle whose cosine and sine are
 * rope_cos[j, i] and rope_sin[j, i]: (y_i c - y_{i+d/2} s, y_{i+d/2} c + y_i s). K_base is stored
 * after its own rotation. The rotation sits between the up-projection and the dot product, so the
 * rank-r key part cannot be deferred like the value side: the call first expands the agent's
 * L_P+L_C keys into the workspace (one pass), then runs the attention over them.
 *
 * K_lr     (device) [L_P+L_C x ld_klr], agent a owns columns a*rank .. a*rank+rank-1
 * B_k      (device) [n_agents x rank x n_kv*d_head]
 * rope_cos, rope_sin (device, fp32) [L_P+L_C x d_head/2], row j = position j
 * workspace(device) lra_attn_prefill_qkvo_workspace_bytes(L_P+L_C, n_kv, d_head) bytes, 256-byte
 *          aligned, no initialisation needed; calls sharing one workspace must be ordered (same
 *          stream). It holds the expanded keys (fp16) and the largest |key| of each 64-key tile.
 * Every other argument is as for lra_attn_prefill. Agent -1 (adapter-free view) runs
 * lra_attn_prefill's kernel on K_base: none of V_lr, B, K_lr, B_k, the tables or the workspace is
 * read. bf16 only (LRA_F32 returns LRA_ERR_UNSUPPORTED). The Q.K products take fp16 operands with
 * fp32 accumulation: Q is converted exactly (up to fp16 subnormals) and K_a is summed in fp32 and
 * rounded to fp16 once. A workgroup whose queries or keys leave the fp16 range, or whose largest
 * |query entry| times largest |key entry| exceeds 1024 (where fp16 rounding of the keys could move
 * a score noticeably), recomputes its rows with bf16 queries against the keys rebuilt in fp32 and
 * split into three bf16 parts (and the value side as for lra_attn_prefill). ld_klr must be
 * >= n_agents*rank and a multiple of 8; every tensor pointer 16-byte aligned.
 */
size_t lra_attn_prefill_qkvo_workspace_bytes(int64_t n_rows, int32_t n_kv, int32_t d_head);

int lra_attn_prefill_qkvo(int dtype, const void* Q, int64_t L_C, int64_t L_P,
                          const void* K_base, const void* V_base, const void* V_lr, int64_t ld_vlr,
                          int64_t vlr_agent_stride, const void* K_lr, int64_t ld_klr, const void* B, const void* B_k,
                          const float* rope_cos, const float* rope_sin, int32_t n_agents, int32_t agent,
                          int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                          void* workspace, size_t workspace_bytes, void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Batched variable-length prefill: several causal chunked prefills (each as lra_attn_prefill) in
 * one launch, for concurrent serving (PReCache summary page: each new chunk L_C follows its reused
 * context L_P; requests are batched together). Request b owns
 *   queries   rows q_start[b] .. q_start[b]+q_len[b]-1 of Q (and the same rows of O),
 *             at absolute positions kv_prefix[b] .. kv_prefix[b]+q_len[b]-1,
 *   cache     rows kv_start[b] .. kv_start[b]+kv_prefix[b]+q_len[b]-1 of K_base, V_base, V_lr
 *             (its own L_P cached tokens followed by its chunk; requests may share cache rows),
 *   agent     agent[b] in [0, n_agents), or -1 for the adapter-free view.
 * Query i of request b attends its cache rows 0 .. kv_prefix[b]+i (relative to kv_start[b]).
 *
 * Q, O     (device) [q_rows x n_q x d_head]; rows no request covers are not written
 * q_start  (device) [batch] int64, q_len (device) [batch] int32
 * max_q_len (host) an upper bound on every q_len[b]; it sizes the launch
 * K_base, V_base (device) [kv_rows x n_kv x d_head]; V_lr (device) kv_rows rows in either layout
 * kv_start (device) [batch] int64, kv_prefix (device) [batch] int32, agent (device) [batch] int32
 * B        (device) [n_agents x rank x n_kv*d_head]
 * A request with q_len[b] = 0 writes nothing; one whose query rows fall outside [0, q_rows) is
 * skipped. One with q_len[b] > max_q_len, a cache range outside [0, kv_rows), kv_prefix[b]+q_len[b]
 * >= 2^31 or an agent outside [-1, n_agents) gets NaN in all its output rows. Precision (with the
 * range-safe recomputation), alignment and the 2^22 bounds are as for lra_attn_prefill.
 * batch = 0 or max_q_len = 0 enqueues nothing.
 */
int lra_attn_prefill_varlen(int dtype, const void* Q, int64_t q_rows, int32_t batch,
                            const int64_t* q_start, const int32_t* q_len, int64_t max_q_len,
                            const void* K_base, const void* V_base, int64_t kv_rows,
                            const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                            const int64_t* kv_start, const int32_t* kv_prefix,
                            const void* B, int32_t n_agents, const int32_t* agent,
                            int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                            void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Batched variable-length prefill over a paged cache: lra_attn_prefill_varlen with request b's
 * cache rows 0 .. kv_prefix[b]+q_len[b]-1 spread over fixed-size pages (the layout of concurrent
 * serving). Cache row j of request b is row j % P of page block_table[b * max_blocks + j / P];
 * requests may name the same pages (a shared prefix). Queries and outputs are rows of Q and O as in
 * lra_attn_prefill_varlen.
 *
 * K_pages, V_pages (device) [n_pages x P x n_kv x d_head]; Vlr_pages (device) [n_pages x P x ld_vlr]
 * page_size P: a power of two in [64, 65536]
 * block_table (device) [batch x max_blocks] int32; kv_prefix, q_len, agent (device) [batch] int32
 * A request whose kv_prefix[b]+q_len[b] exceeds max_blocks * P is invalid (NaN rows, as in
 * lra_attn_prefill_varlen). A page id outside [0, n_pages) reads page 0 in its place and turns the
 * rows of every workgroup that met it to NaN.
 */
int lra_attn_prefill_paged(int dtype, const void* Q, int64_t q_rows, int32_t batch,
                           const int64_t* q_start, const int32_t* q_len, int64_t max_q_len,
                           const void* K_pages, const void* V_pages, const void* Vlr_pages,
                           int64_t n_pages, int32_t page_size, int64_t ld_vlr,
                           const int32_t* block_table, int32_t max_blocks, const int32_t* kv_prefix,
                           const void* B, int32_t n_agents, const int32_t* agent,
                           int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                           void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Batched decode, one new query token per request, split along the key axis (LRAgent method steps
 * (3)-(4) with L_C = 1). The batch's keys, counted in 32-key tiles request after request, are cut
 * into equal contiguous slices, one per workgroup; each (slice, KV head) writes one fp32 partial
 * (m, l, O, O_lr) per request piece it covers to the workspace, and a second kernel merges the
 * partials of each (request, KV head) with the log-sum-exp rule, applies B_agent once and
 * normalises. Request b attends all rows
 * kv_start[b] .. kv_start[b]+kv_len[b]-1 of the shared caches; requests may share rows.
 * kv_len[b] = 0 gives a zero output row.
 *
 * Q        (device) [batch x n_q x d_head]
 * K_base, V_base (device) [kv_rows x n_kv x d_head]
 * V_lr     (device) kv_rows rows in either layout (conventions above)
 * kv_start (device) [batch] int64, kv_len (device) [batch] int32, agent (device) [batch] int32:
 *          agent[b] in [0, n_agents), or -1 for the adapter-free view (B is not read; the split
 *          kernel streams agent 0's V_lr columns of the range and the merge drops that product)
 * max_kv_len (host) an upper bound on every kv_len[b]; it sizes the launch
 * B        (device) [n_agents x rank x n_kv*d_head]
 * keys_per_split  keys per slice at full lengths (batch * max_kv_len / keys_per_split slices,
 *          rounded up to a multiple of 8; keys_per_split a multiple of 64), or 0 for the library's
 *          choice (one round of 8-wave workgroups on 15/16 of the chip's CUs: 240 slices per
 *          group of 8 KV heads, fewer when the batch's actual lengths hold fewer tiles). With 0
 *          and a small batch (batch x n_kv x ceil(max_kv_len / 128) <= 256, else with 256-key
 *          chunks <= 512) lra_attn_decode and its strided and no-allocation forms instead give
 *          each (request, KV head, 128- or 256-key chunk) one workgroup, which merges its tiles
 *          in LDS; requests of one chunk finish in that launch, longer ones in a merge launch over
 *          their chunk records. The slicing changes the rounding of the result only.
 * workspace(device) lra_attn_decode_workspace_bytes() bytes, 256-byte aligned; its contents need
 *          no initialisation. Calls that share one workspace must be ordered (same stream).
 * O        (device) [batch x n_q x d_head] output
 * Every tensor pointer must be 16-byte aligned. batch = 0 enqueues
 * nothing. The workspace size is 0 when no request can have a key (max_kv_len = 0); the call then
 * only writes the zero and NaN rows.
 */
size_t lra_attn_decode_workspace_bytes(int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_head,
                                       int32_t rank, int64_t max_kv_len, int32_t keys_per_split);

int lra_attn_decode(int dtype, const void* Q, int32_t batch,
                    const void* K_base, const void* V_base, int64_t kv_rows,
                    const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                    const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                    const void* B, int32_t n_agents, const int32_t* agent,
                    int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                    int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                    void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * One decode step with the LR rows of the step's newest tokens formed in the same launch
 * (PReCache paper page §3, PreLRShared: each new token's hidden state goes through every agent's
 * down-projection once; LRAgent method steps (2)-(4)). For every request b with kv_len[b] > 0 and a
 * valid range and agent, the newest key is cache row n_b = kv_start[b] + kv_len[b] - 1, and
 *
 *   V_lr(row n_b, agent k, column j) = sum_c X_new[b, c] * A[k*rank + j, c]      (k < n_agents, j < rank)
 *
 * is written into the cache (rounded once to the element type), then the decode runs as
 * lra_attn_decode over all kv_len[b] keys, that row included. This is lra_lr_precompute with
 * out_rows = n_b followed by lra_attn_decode, in one launch plus the merge kernel: the rows are
 * formed by extra workgroups of the split launch while the others stream the caches, the split
 * kernel leaves the newest key out of O_lr and records its score, and the merge kernel adds that
 * key's LR term from the written row. Results agree with the two calls within the decode's
 * tolerance (the newest key's LR term is summed in fp32 instead of on the matrix cores).
 *
 * X_new    (device) [batch x d_model], row stride ldx elements (ldx >= d_model, multiple of 8)
 * A        (device) [n_agents*rank x d_model], the stacked down-projections (as lra_lr_precompute)
 * d_model  a positive multiple of 64
 * V_lr     (device) the cache, written at the rows n_b (all n_agents*rank columns); the newest rows
 *          of different requests must be distinct
 * Every other argument, the workspace (lra_attn_decode_workspace_bytes) and the errors are those
 * of lra_attn_decode.
 */
int lra_attn_decode_step(int dtype, const void* Q, int32_t batch,
                         const void* K_base, const void* V_base, int64_t kv_rows,
                         void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                         const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                         const void* B, int32_t n_agents, const int32_t* agent,
                         int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                         const void* X_new, int64_t ldx, const void* A, int32_t d_model,
                         int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                         void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * lra_attn_decode over K and V caches with explicit strides, for caches kept head-major
 * ([n_kv x rows x d_head], each KV head's rows contiguous) or in any other layout whose
 * (row, KV head) vectors of d_head elements are contiguous. Element (row j, KV head g, dim c) of K
 * and of V is at offset  j * kv_row_stride + g * kv_head_stride + c  (elements). Token-major
 * ([rows x n_kv x d_head], what lra_attn_decode reads) is kv_row_stride = n_kv*d_head,
 * kv_head_stride = d_head; head-major is kv_row_stride = d_head, kv_head_stride = rows*d_head. In the
 * head-major layout each workgroup of the split kernel streams one contiguous range of memory.
 * Both strides must be positive multiples of 8, kv_row_stride at most 2^24; the caller's K and V
 * buffers must hold every element addressed for rows 0 .. kv_rows-1 (the row ranges are checked
 * against kv_rows as in lra_attn_decode). Every other argument, the workspace
 * (lra_attn_decode_workspace_bytes) and the results are as for lra_attn_decode: with the same
 * values the outputs are bit-identical in either layout.
 */
int lra_attn_decode_strided(int dtype, const void* Q, int32_t batch,
                            const void* K_base, const void* V_base, int64_t kv_rows,
                            int64_t kv_row_stride, int64_t kv_head_stride,
                            const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                            const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                            const void* B, int32_t n_agents, const int32_t* agent,
                            int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                            int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                            void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * lra_attn_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, and harnesses that forbid allocation. It takes no workspace: the split
 * partials live in a static device array of the library, LRA_NOALLOC_SCRATCH_BYTES bytes, of which
 * each GPU the library runs on holds its own copy until the process ends. The call allocates
 * nothing (no hipMalloc, no allocating library routine); it looks the array's address up once per
 * device, on its first call there.
 *
 * Arguments, results and errors are those of lra_attn_decode with the same keys_per_split (same
 * kernels, same output bits). A call whose lra_attn_decode_workspace_bytes() exceeds
 * LRA_NOALLOC_SCRATCH_BYTES returns LRA_ERR_WORKSPACE and enqueues nothing. The array keeps the
 * last call's contents, which no call needs cleared. Every call on one GPU uses the same array, so
 * calls on one GPU that overlap in time (different streams, or host threads without ordering)
 * race: order them, e.g. on one stream.
 */
#define LRA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int lra_attn_decode_noalloc(int dtype, const void* Q, int32_t batch,
                            const void* K_base, const void* V_base, int64_t kv_rows,
                            const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                            const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                            const void* B, int32_t n_agents, const int32_t* agent,
                            int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                            int32_t keys_per_split, void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * lra_attn_decode with LoRA on the key projection as well (the qkvo configuration; LRAgent page,
 * limitations): request b's key t (cache row kv_start[b] + t) is
 *
 *   K_a[t, g] = K_base[kv_start[b] + t, g] + RoPE_t( (K_lr[kv_start[b] + t, a*rank : a*rank+rank] B_k[a])[g*d : g*d+d] )
 *
 * with a = agent[b] and RoPE_t as for lra_attn_prefill_qkvo, at table row t (a request's keys sit at
 * positions 0 .. kv_len[b]-1). The call first computes the rank-r part of every score,
 * Q . RoPE_t(K_lr B_k), for all query heads and writes it as fp32 into the workspace, then runs the
 * decode kernels, which add it to the base scores Q . K_base.
 *
 * K_lr     (device) [kv_rows x ld_klr], agent a owns columns a*rank .. a*rank+rank-1
 * B_k      (device) [n_agents x rank x n_kv*d_head]
 * rope_cos, rope_sin (device, fp32) [>= max_kv_len x d_head/2], row t = position t
 * workspace(device) lra_attn_decode_qkvo_workspace_bytes() bytes (same arguments), 256-byte
 *          aligned, no initialisation needed; calls sharing one workspace must be ordered.
 * Every other argument is as for lra_attn_decode. Adapter-free requests (agent -1) attend K_base
 * alone and read none of the key-side operands. bf16 only (LRA_F32 returns LRA_ERR_UNSUPPORTED);
 * max_kv_len <= 2^24. Precision: the base part of a score is as in lra_attn_decode; the rank-r
 * part is computed from fp16 operands (per-head weights from B_k and the query, and K_lr times the
 * rotary entries) with fp32 accumulation. A block of 512 keys whose rank-r parts come out
 * non-finite (an operand beyond the fp16 range) or larger than 16 in the exponent (scale * |part|)
 * is recomputed in fp32 from Q, K_lr, B_k and the tables, so every finite input is accepted.
 */
size_t lra_attn_decode_qkvo_workspace_bytes(int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_head,
                                            int32_t rank, int64_t max_kv_len, int32_t keys_per_split);

int lra_attn_decode_qkvo(int dtype, const void* Q, int32_t batch,
                         const void* K_base, const void* V_base, int64_t kv_rows,
                         const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                         const void* K_lr, int64_t ld_klr,
                         const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                         const void* B, const void* B_k, const float* rope_cos, const float* rope_sin,
                         int32_t n_agents, const int32_t* agent,
                         int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                         int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                         void* O, void* stream);

/* Keys per slice of the library's choice for the split launch (keys_per_split = 0) when every
 * request has max_kv_len keys, rounded up to a multiple of 64 (passing it may round the slice count
 * differently). Passing it explicitly always selects the split launch; with 0, small batches take the
 * chunked launch described at lra_attn_decode instead. */
int32_t lra_attn_decode_default_split(int32_t batch, int32_t n_kv, int64_t max_kv_len);

/* ------------------------------------------------------------------------------------------------
 * Batched decode over a paged cache, for concurrent serving (the pages' serving experiments run
 * under vLLM, whose KV cache is paged): lra_attn_decode with request b's logical rows
 * 0 .. kv_len[b]-1 spread over fixed-size pages. Logical row j of request b is row j % P of page
 * block_table[b * max_blocks + j / P]. Requests may name the same pages (a shared prefix).
 *
 * K_pages, V_pages (device) [n_pages x P x n_kv x d_head]
 * Vlr_pages (device) [n_pages x P x ld_vlr], the LR cache rows of the same tokens
 * page_size P: a power of two in [32, 65536]
 * block_table (device) [batch x max_blocks] int32; entries past a request's last page are unread
 * kv_len, agent (device) [batch] int32; agent[b] in [0, n_agents) or -1 (adapter-free view)
 * max_kv_len (host) an upper bound on every kv_len[b], at most max_blocks * P
 * keys_per_split  as for lra_attn_decode (0: the library's choice, the same as for contiguous
 *          caches); a slice may span any number of pages
 * workspace(device) lra_attn_decode_workspace_bytes(..., keys_per_split) bytes; no initialisation
 *          needed
 * A request whose pages include an id outside [0, n_pages) gets NaN in every output element and
 * reads page 0 in place of the bad ones. Everything else is as for lra_attn_decode.
 */
int lra_attn_decode_paged(int dtype, const void* Q, int32_t batch,
                          const void* K_pages, const void* V_pages, const void* Vlr_pages,
                          int64_t n_pages, int32_t page_size, int64_t ld_vlr,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* kv_len, int64_t max_kv_len,
                          const void* B, int32_t n_agents, const int32_t* agent,
                          int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                          int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                          void* O, void* stream);

/* ------------------------------------------------------------------------------------------------
 * lra_attn_decode_paged with explicit strides for the K and V pages: element (page, row j of the
 * page, KV head g, dim c) of K_pages and of V_pages is at offset
 *   page * kv_page_stride + j * kv_row_stride + g * kv_head_stride + c      (elements).
 * Token-major pages [n_pages x P x n_kv x d_head] (what lra_attn_decode_paged reads) are
 * (P*n_kv*d_head, n_kv*d_head, d_head); head-major pages [n_pages x n_kv x P x d_head] are
 * (n_kv*P*d_head, d_head, P*d_head), where each KV head's slice of a page is one contiguous run.
 * Vlr_pages keeps its layout [n_pages x P x ld_vlr]. The strides must be positive multiples of 8,
 * kv_row_stride at most 2^24; the caller's buffers must hold every element addressed for pages
 * 0 .. n_pages-1. Every other argument, the workspace and the results are as for
 * lra_attn_decode_paged: with the same values the outputs are bit-identical in either layout.
 */
int lra_attn_decode_paged_strided(int dtype, const void* Q, int32_t batch,
                                  const void* K_pages, const void* V_pages, const void* Vlr_pages,
                                  int64_t n_pages, int32_t page_size, int64_t ld_vlr,
                                  int64_t kv_page_stride, int64_t kv_row_stride, int64_t kv_head_stride,
                                  const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* kv_len, int64_t max_kv_len,
                                  const void* B, int32_t n_agents, const int32_t* agent,
                                  int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                  int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                                  void* O, void* stream);

/* lra_attn_decode_default_split for a supported page size P, else 0. */
int32_t lra_attn_decode_paged_default_split(int32_t batch, int32_t n_kv, int64_t max_kv_len, int32_t page_size);

/* ------------------------------------------------------------------------------------------------
 * Value expansion: the expand-then-attend baseline (LRAgent page, Flash-LoRA-Attention: without the
 * reordering, each agent's full value cache V_a = V_base + V_lr B_a is built before attention).
 * Flash-LoRA-Attention never needs this call; it exists so the two orders can be compared on the same
 * attention kernels: expand, then run lra_attn_prefill / lra_attn_decode with the adapter-free agent
 * (-1) over K_base and V_out. For request b with a = agent[b], rows t < len[b]:
 *
 *   V_out[dst_start[b] + t, c] = V_base[src_start[b] + t, c]
 *                                + sum_j V_lr[src_start[b] + t, a*rank + j] * B[a, j, c]     c < n_kv*d_head
 *
 * summed in fp32 and rounded once to the element type. Agent -1 copies V_base rows unchanged.
 *
 * V_base   (device) [kv_rows x n_kv x d_head];  V_lr (device) [kv_rows x ld_vlr]
 * B        (device) [n_agents x rank x n_kv*d_head]
 * src_start, dst_start (device) [batch] int64; len, agent (device) [batch] int32
 * max_len  (host) an upper bound on every len[b]; it sizes the launch
 * V_out    (device) [out_rows x n_kv x d_head] output; rows no request covers are not written.
 *          Requests whose destination ranges overlap race.
 * A request with len[b] <= 0 or a destination range outside [0, out_rows) is skipped. One with
 * len[b] > max_len, a source range outside [0, kv_rows) or an agent outside [-1, n_agents) gets NaN
 * in its destination rows dst_start[b] .. dst_start[b] + min(len[b], max_len) - 1.
 * ld_vlr must be a multiple of 8 and every tensor pointer 16-byte aligned. batch = 0 or max_len = 0
 * enqueues nothing; batch * ceil(max_len / 256) must not exceed 2^24.
 */
int lra_expand_values(int dtype, const void* V_base, int64_t kv_rows, const void* V_lr, int64_t ld_vlr,
                      const void* B, int32_t n_agents, int32_t n_kv, int32_t d_head, int32_t rank,
                      int32_t batch, const int64_t* src_start, const int32_t* len,
                      const int32_t* agent, int64_t max_len,
                      void* V_out, int64_t out_rows, const int64_t* dst_start, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Measurement helper: reads bytes of device memory at x with 16-byte loads, one contiguous chunk of
 * bytes / n_workgroups per 8-wave workgroup, and writes the XOR fold of chunk w's 32-bit words to
 * out[w]. Timed, it gives the read bandwidth a plain streaming kernel reaches on this GPU: the
 * practical ceiling for the decode, whose work is a read-only stream of the caches.
 *
 * x        (device) bytes bytes, 16-byte aligned; bytes a positive multiple of 16 * n_workgroups
 * out      (device) [n_workgroups] uint32
 * n_workgroups in [1, 2^20]. Errors: LRA_ERR_NULL, LRA_ERR_SHAPE; nothing is enqueued then.
 */
int lra_stream_read(const void* x, int64_t bytes, int32_t n_workgroups, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LRA_H */
