// Internal interface between the C ABI layer (api.hip) and the kernel launchers.
// Arguments reaching these launchers have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace lra {

// agent index of the adapter-free view (double batching: attends the base cache alone, no LR term)
constexpr int kAdapterFree = -1;

struct DecodeParams {
    const void* Q;
    const void* K;
    const void* V;
    const void* Vlr;
    const void* B;
    const int64_t* kv_start;
    const int32_t* kv_len;
    const int32_t* agent;
    // partial records of the pieces: (slices + batch) * n_kv blocks of decode_record_slots()
    // 16-byte slots (unnormalised O and O_lr, running max in base-2 units and sum), record_bytes
    // in all (below 2^31)
    float* records;
    uint32_t record_bytes;
    void* O;
    // V_lr: row r, agent a, rank column j at r * ld_vlr + a * vlr_agent_stride + j (the rows'
    // layout: vlr_agent_stride = rank; agent-major: ld_vlr = rank, vlr_agent_stride >= rows * rank)
    int64_t ld_vlr, vlr_agent_stride;
    int64_t kv_rows;
    int64_t max_kv_len;
    // elements between consecutive rows of one KV head, and between the KV heads of one row, of K
    // and V (token-major [rows x n_kv x d]: n_kv*d and d; head-major [n_kv x rows x d]: d and rows*d)
    int64_t kv_row_stride, kv_head_stride;
    int64_t kv_page_stride;     // paged cache: elements between consecutive pages of K and V
    int batch, n_q, n_kv, G, n_agents, d_head, rank;
    // workgroup slots per group of 8 KV heads (a multiple of 8): the batch's units are cut into
    // min(n_slots, units) slices of equal size, one per slot (decode_slices)
    int n_slots;
    float scale;
    bool bf16;
    // paged cache (null block_table: contiguous rows addressed by kv_start). Request b's logical row
    // j lives in page block_table[b*max_blocks + j/P], at row j%P of that page; P = 2^page_shift.
    const int32_t* block_table;
    int64_t n_pages;
    int max_blocks;
    int page_shift;
    // LoRA on the keys (null: none): key_scores[(b*n_q + h)*ks_stride + j] = Q_bh . RoPE_j(K_lr B_k)
    // of request b's key j, fp32 (bf16 only; ks_stride a multiple of 64)
    const float* key_scores;
    int64_t ks_stride;
    // decode step (null X_new: none): the newest key of request b (row kv_start[b] + kv_len[b] - 1)
    // gets its LR row V_lr[row, 0 .. n_agents*rank) = X_new[b] . A_new^T, computed by the first
    // n_pre workgroups of the split launch (a multiple of 8, two requests each); the split kernel
    // leaves that key out of O_lr and records its score, and the merge kernel adds its LR term
    const void* X_new;
    const void* A_new;   // [n_agents*rank x d_model], stacked like the precompute's A
    int64_t ldx;
    int d_model;
    int n_pre;
    // small batches (n_chunks 0: the split launch above): one workgroup per (request, KV head, chunk
    // of chunk_keys = 128 or 256 keys), n_chunks chunks per request at max_kv_len; the records are
    // then decode_small_record_slots() 16-byte slots per (request, KV head, chunk), merged by a
    // second launch when n_chunks > 1
    int n_chunks, chunk_keys;
};

struct PrecomputeParams {
    const void* X;
    const void* A;
    void* Vlr;
    const int64_t* out_rows;
    int64_t T;
    int64_t ldx;
    int64_t ld_vlr, vlr_agent_stride;   // output column a * rank + j at row * ld_vlr + a * vlr_agent_stride + j
    int64_t vlr_rows;
    int d_model;
    int rank;
    int NR;               // n_agents * rank
    int n_rg;             // row ranges (one per workgroup and column group)
    int n_cg;             // column groups
    int cols_per_group;   // 16 or 32
    bool bf16;
};

struct PrefillParams {
    const void* Q;
    const void* K;
    const void* V;
    const void* Vlr;
    const void* B;
    void* O;
    int64_t L_C;
    int64_t L_P;
    int64_t ld_vlr, vlr_agent_stride;   // as in DecodeParams
    int n_q, n_kv, G, d_head, rank, agent, n_agents;
    float scale;
    bool bf16;
    // batched variable-length prefill: per-request tables (all null for one request given by
    // L_C, L_P and agent above)
    const int64_t* q_start;     // [batch] first row of the request's queries in Q and O
    const int32_t* q_len;       // [batch] its L_C
    const int64_t* kv_start;    // [batch] first row of its cache range in K, V and V_lr
    const int32_t* kv_prefix;   // [batch] its L_P
    const int32_t* agents;      // [batch] its agent (or kAdapterFree)
    int64_t q_rows;             // rows of Q and O
    int64_t kv_rows;            // rows of K, V and V_lr
    int64_t max_q_len;          // bound on every q_len[b] (host value that sized the grid)
    int batch;                  // requests in the grid
    int max_pairs;              // workgroups per (request, KV head): enough for the longest chunk
    // paged cache (null block_table: rows from kv_start). Request b's logical cache row j lives in
    // page block_table[b*max_blocks + j/P], at row j%P of that page; P = 2^page_shift >= 64.
    const int32_t* block_table;
    int64_t n_pages;
    int max_blocks;
    int page_shift;
    // LoRA on the keys too: non-null key_flags means K holds the agent's keys as fp16 bit patterns
    // (the key expansion pass's output) and key_flags[t*n_kv + g] holds the largest |key| of 64-key
    // tile t of KV head g as fp32 bits. The range-safe pass rebuilds the keys in fp32 from K_src
    // (K_base), K_lr, B_k and the rotary tables.
    const int32_t* key_flags;
    const void* K_src;
    const void* Klr;
    int64_t ld_klr;
    const void* Bk;
    const float* rope_cos;
    const float* rope_sin;
};

// keys per tile of the key expansion pass's range flags (the prefill's LDS key tile)
constexpr int kKeyTile = 64;

// Key expansion of the qkvo configuration: Ka[j, g] = fp16(K_base[j, g] + RoPE_j(K_lr[j, agent] B_k)),
// with the largest |value| of each (64-key tile, KV head) as fp32 bits in flags.
struct KeyExpandParams {
    const void* K;              // bf16 [n_rows x n_kv x d_head]
    const void* Klr;            // bf16 [n_rows x ld_klr]
    const void* Bk;             // bf16 [n_agents x rank x n_kv*d_head]
    const float* rope_cos;      // [n_rows x d_head/2]
    const float* rope_sin;
    void* Ka;                   // fp16 [n_rows x n_kv x d_head]
    int32_t* flags;             // [ceil(n_rows/64) x n_kv]
    int64_t n_rows, ld_klr;
    int n_kv, d_head, rank, agent;
};
hipError_t launch_key_expand(const KeyExpandParams& p, hipStream_t stream);

// Value expansion of the expand-then-attend baseline: request b's rows t < len[b] become
// V_out[dst_start[b] + t] = V_base[src_start[b] + t] + V_lr[src_start[b] + t, agent cols] B_agent
// (a copy of V_base for the adapter-free agent). Invalid requests as documented in lra.h.
struct ValueExpandParams {
    const void* V;              // [kv_rows x row_elems]
    const void* Vlr;            // [kv_rows x ld_vlr]
    const void* B;              // [n_agents x rank x row_elems]
    void* Vout;                 // [out_rows x row_elems]
    const int64_t* src_start;   // [batch]
    const int32_t* len;         // [batch]
    const int32_t* agent;       // [batch]
    const int64_t* dst_start;   // [batch]
    int64_t kv_rows, out_rows, ld_vlr, max_len, n_chunks;
    int batch, n_agents, row_elems, rank, rows_per_wg;
    bool bf16;
};
hipError_t launch_value_expand(const ValueExpandParams& p, hipStream_t stream);
// rows of one request per workgroup for these sizes: 256, halved (down to 16) until the grid holds
// about 2048 workgroups
int value_expand_rows(int batch, int64_t max_len);

// Decode with LoRA on the keys: the rank-r part of every score,
// S[(b*n_q + h)*ks_stride + j] = Q[b, h] . RoPE_j(K_lr[kv_start[b] + j, agent_b] B_k[agent_b][:, g]) (fp32),
// for keys j < round_up(kv_len[b], 32) (later keys repeat the last row). Requests that are invalid
// or adapter-free are skipped. W holds the per-head weights of the features K_lr (x) [cos, sin]
// (d_head*rank fp16 per request and query head); flags marks the score workgroups (request, key
// block, head block) whose fp16 pass produced a non-finite or very large value and were
// recomputed in fp32.
struct KeyScoreParams {
    const void* Q;              // bf16 [batch x n_q x d_head]
    const void* Klr;            // bf16 [kv_rows x ld_klr]
    const void* Bk;             // bf16 [n_agents x rank x n_kv*d_head]
    const float* rope_cos;      // [>= max_kv_len x d_head/2]
    const float* rope_sin;
    const int64_t* kv_start;
    const int32_t* kv_len;
    const int32_t* agent;
    float* S;                   // fp32 [batch x n_q x ks_stride]
    int32_t* flags;             // [batch x key blocks x head blocks] (the score kernel's grid)
    uint16_t* W;                // fp16 [batch x n_q x d_head*rank]
    uint16_t* Tp;               // fp16 rotary tables in the score kernel's lane order, key_score_table_bytes()
    int64_t kv_rows, max_kv_len, ld_klr, ks_stride;
    int batch, n_q, n_kv, G, n_agents, d_head, rank;
    float scale;                // the softmax scale (decides when the fp32 recomputation runs)
};
hipError_t launch_key_scores(const KeyScoreParams& p, hipStream_t stream);
// tiles of 16 keys of the repacked rotary tables: the score pass reads keys up to round_up(len, 32)
__host__ __device__ inline int64_t key_score_table_tiles(int64_t max_kv_len) { return (max_kv_len + 31) / 32 * 2; }
// bytes of the repacked rotary tables: per 16-key tile, d_head*rank/32 steps x 64 lanes x 2 bytes
inline size_t key_score_table_bytes(int64_t max_kv_len, int d_head, int rank) {
    return size_t(key_score_table_tiles(max_kv_len)) * size_t(d_head * rank / 32) * 128;
}
constexpr int kKeyScoreBlock = 512;   // keys per workgroup of the key score pass
// query heads per workgroup of the key score pass
inline int key_score_heads(int d_head, int rank) { return d_head * rank <= 1024 ? 32 : 16; }

// workgroups per (request, KV head) of the prefill grid for a chunk of L_C queries
int prefill_pairs(int64_t L_C, int G);

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// streaming-read probe: n_workgroups chunks of bytes / n_workgroups bytes, one XOR fold per chunk
hipError_t launch_read_probe(const void* x, int64_t bytes, int n_workgroups, uint32_t* out, hipStream_t stream);
hipError_t launch_precompute(const PrecomputeParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Host-side launch geometry of the LR precompute.
struct PrecomputePlan {
    int n_rg, n_cg, cols_per_group;
    int chunks_per_wave;  // 32-element reduction chunks per wave
    int cb;               // chunks a wave holds in registers (the kernel's limit)
};
PrecomputePlan plan_precompute(int64_t T, int d_model, int NR, bool bf16);

// workgroup slots of a decode launch per group of 8 KV heads: one per about keys_per_split keys at
// full lengths, or (0) the library's choice (one 8-wave workgroup per CU on 15/16 of the chip); 0
// when there is nothing to do, -1 when the sizes are too large
int decode_slots(int batch, int n_kv, int64_t max_kv_len, int keys_per_split);
// 16-byte slots of one decode record block (one piece, one KV head, GP query heads; GP = the
// group size rounded up to 4 or 8): O (d_head/16 * 4GP), O_lr (GP * rank/4), (m, l) (GP), padded to
// a multiple of 16 slots (256 bytes)
inline int decode_record_slots(int G, int d_head, int rank) {
    const int GP = G <= 4 ? 4 : 8;
    return (GP * (d_head / 4 + rank / 4 + 1) + 15) / 16 * 16;
}

// Small-batch decode: requests are cut into chunks of 128 or 256 keys, one workgroup of 4 or 8 waves
// (a 32-key tile each) per (request, KV head, chunk). Used for the library's default split when
// few such workgroups cover the batch at max_kv_len (the split launch would give each of its slots
// a tile or two): 128-key chunks while they fit one workgroup per CU, else 256-key chunks up to
// two per CU (measured on MI355X: 64-key chunks, one per CU, cost more in the merge than they save
// in the streaming). Returns the chunks per request (and their keys), or 0 for the split launch.
constexpr int kDecodeSmallCUs = 256;
inline int decode_small_chunks(int batch, int n_kv, int64_t max_kv_len, int keys_per_split, int* chunk_keys = nullptr) {
    if (keys_per_split != 0 || batch <= 0 || n_kv <= 0 || max_kv_len <= 0) return 0;
    const int64_t bg = int64_t(batch) * n_kv;
    const int64_t c128 = (max_kv_len + 127) / 128, c256 = (max_kv_len + 255) / 256;
    int keys = 0;
    int64_t chunks = 0;
    if (bg * c128 <= kDecodeSmallCUs) keys = 128, chunks = c128;
    else if (bg * c256 <= 2 * kDecodeSmallCUs) keys = 256, chunks = c256;
    if (chunk_keys) *chunk_keys = keys;
    return int(chunks);
}
// 16-byte slots of one small-batch record (one request, KV head and chunk): the merged O^T and
// O_lr^T fragments of the GP heads (d_head/16 + 1 tiles of 4*GP slots), then m and l of the GP
// heads as floats
inline int decode_small_record_slots(int G, int d_head) {
    const int GP = G <= 4 ? 4 : 8;
    return (d_head / 16 + 1) * 4 * GP + (2 * GP + 3) / 4;
}

// The slices of a decode launch over the batch's U units (32-key tiles, request after request):
// min(n_slots, U) slices, slice k starting at unit U*k/n (equal to within a unit), so every slice
// holds at least one unit. A function of U and the slots alone, so the split kernel, the merge
// kernel and the host agree. A slice holds at most one piece of each request it touches, and the
// piece of request b in slice k has record block k + b.
__host__ __device__ inline int decode_slices(int U, int n_slots) { return U < n_slots ? (U > 0 ? U : 0) : n_slots; }
__host__ __device__ inline int slice_begin(int U, int k, int n) { return int(int64_t(U) * k / n); }
__host__ __device__ inline int slice_owner(int U, int u, int n) { return int((int64_t(u + 1) * n - 1) / U); }

}  // namespace lra
