// C ABI of liblra: host-side validation, workspace layout and dispatch to the gfx950 kernels.
// Every failing check returns before anything is enqueued; see include/lra.h for the contract.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/lra.h"
#include "lra_kernels.h"

static_assert(lra::kAdapterFree == LRA_ADAPTER_FREE, "adapter-free agent index");

#define LRA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return LRA_OK;
    return fail(LRA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// V_lr layouts: row r, agent a, rank column j at r * ld_vlr + a * vlr_agent_stride + j, either
// interleaved (each row holds every agent's columns: vlr_agent_stride = rank, ld_vlr >=
// n_agents * rank) or agent-major (each agent's rows contiguous: ld_vlr >= rank, vlr_agent_stride >=
// rows * ld_vlr). Both strides are multiples of 8 elements (16-byte aligned runs).
int check_vlr(int64_t ld_vlr, int64_t agent_stride, int64_t rows, int32_t n_agents, int32_t rank) {
    const bool aligned8 = ld_vlr > 0 && agent_stride > 0 && ld_vlr % 8 == 0 && agent_stride % 8 == 0;
    const bool interleaved = agent_stride == rank && ld_vlr >= int64_t(n_agents) * rank;
    const bool agent_major = ld_vlr >= rank && agent_stride >= std::max<int64_t>(rows, 1) * ld_vlr;
    if (!aligned8 || !(interleaved || agent_major))
        return fail(LRA_ERR_SHAPE, "V_lr strides (ld_vlr=%lld, vlr_agent_stride=%lld) are neither interleaved (agent "
                    "stride = rank, ld_vlr >= n_agents*rank) nor agent-major (ld_vlr >= rank, agent stride >= %lld "
                    "rows x ld_vlr), or not multiples of 8", (long long)ld_vlr, (long long)agent_stride, (long long)rows);
    return LRA_OK;
}

// -------------------------------------------------------------------------- decode workspace
struct DecodeLayout {
    int n_slots;
    size_t rec_off, rec_bytes, total;
};

// records: (slices + batch) * n_kv blocks of decode_record_slots() 16-byte slots, with the most
// slices the sizes allow, min(n_slots, units at max_kv_len) (a slice holds at most one piece of
// each request it touches, and its pieces' blocks (k + b) * n_kv + g are distinct). n_slots < 0:
// the sizes are too large for one launch.
DecodeLayout decode_layout(int batch, int n_q, int n_kv, int d_head, int rank, int64_t max_kv_len, int keys_per_split) {
    DecodeLayout L{};
    L.n_slots = lra::decode_slots(batch, n_kv, max_kv_len, keys_per_split);
    if (L.n_slots <= 0 || n_kv <= 0 || n_q % n_kv != 0) return L;
    const int64_t units_max = int64_t(batch) * ((max_kv_len + 31) / 32);   // below 2^31 (decode_slots)
    const int slices = lra::decode_slices(int(units_max), L.n_slots);
    const size_t blocks = (size_t(slices) + size_t(batch)) * size_t(n_kv);
    L.rec_off = 0;
    L.rec_bytes = blocks * size_t(lra::decode_record_slots(n_q / n_kv, d_head, rank)) * 16;
    // the small-batch launch's chunk records, when the sizes select it (plain decodes only, but the
    // workspace query serves every decode entry point)
    const int chunks = lra::decode_small_chunks(batch, n_kv, max_kv_len, keys_per_split);
    if (chunks > 1)
        L.rec_bytes = std::max(L.rec_bytes, size_t(batch) * size_t(n_kv) * size_t(chunks) *
                                                size_t(lra::decode_small_record_slots(n_q / n_kv, d_head)) * 16);
    if (L.rec_bytes >= (size_t(1) << 31)) L.n_slots = -1;   // 32-bit record offsets
    L.total = L.rec_off + L.rec_bytes;
    return L;
}

int check_heads(int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank) {
    if (n_q <= 0 || n_kv <= 0) return fail(LRA_ERR_SHAPE, "n_q=%d and n_kv=%d must be positive", n_q, n_kv);
    if (n_q % n_kv != 0) return fail(LRA_ERR_SHAPE, "n_q=%d is not a multiple of n_kv=%d", n_q, n_kv);
    if (n_q / n_kv > 8) return fail(LRA_ERR_UNSUPPORTED, "group size n_q/n_kv=%d exceeds 8", n_q / n_kv);
    if (d_head != 64 && d_head != 128) return fail(LRA_ERR_UNSUPPORTED, "d_head=%d (supported: 64, 128)", d_head);
    if (rank != 8 && rank != 16) return fail(LRA_ERR_UNSUPPORTED, "rank=%d (supported: 8, 16)", rank);
    return LRA_OK;
}

// contiguous prefill caches are read through 32-bit buffer offsets over 64-row tiles
int check_prefill_rows(int32_t n_kv, int32_t d_head, int64_t ld_vlr) {
    if (int64_t(n_kv) * d_head > (int64_t(1) << 22)) return fail(LRA_ERR_SHAPE, "n_kv*d_head exceeds 2^22");
    if (ld_vlr > (int64_t(1) << 22)) return fail(LRA_ERR_SHAPE, "ld_vlr=%lld exceeds 2^22", (long long)ld_vlr);
    return LRA_OK;
}

int check_dtype(int dtype) {
    if (dtype != LRA_F32 && dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "dtype=%d", dtype);
    return LRA_OK;
}

}  // namespace

LRA_EXPORT int lra_abi_version(void) { return LRA_ABI_VERSION; }

LRA_EXPORT const char* lra_status_str(int status) {
    switch (status) {
        case LRA_OK: return "LRA_OK";
        case LRA_ERR_NULL: return "LRA_ERR_NULL";
        case LRA_ERR_SHAPE: return "LRA_ERR_SHAPE";
        case LRA_ERR_UNSUPPORTED: return "LRA_ERR_UNSUPPORTED";
        case LRA_ERR_INDEX: return "LRA_ERR_INDEX";
        case LRA_ERR_WORKSPACE: return "LRA_ERR_WORKSPACE";
        case LRA_ERR_HIP: return "LRA_ERR_HIP";
        default: return "LRA_ERR_UNKNOWN";
    }
}

LRA_EXPORT const char* lra_last_error(void) { return g_last_error.c_str(); }

// ============================================================================ LR precompute
LRA_EXPORT size_t lra_lr_precompute_workspace_bytes(int64_t T, int32_t d_model, int32_t n_agents, int32_t rank) {
    (void)T; (void)d_model; (void)n_agents; (void)rank;
    return 0;   // one launch, no partials
}

LRA_EXPORT int lra_lr_precompute(int dtype, const void* X, int64_t T, int32_t d_model, int64_t ldx,
                                 const void* A, int32_t n_agents, int32_t rank,
                                 void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride, int64_t vlr_rows,
                                 const int64_t* out_rows, void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace; (void)workspace_bytes;
    if (int s = check_dtype(dtype)) return s;
    if (T < 0) return fail(LRA_ERR_SHAPE, "T=%lld is negative", (long long)T);
    if (n_agents <= 0 || rank <= 0) return fail(LRA_ERR_SHAPE, "n_agents=%d, rank=%d must be positive", n_agents, rank);
    const int64_t NR = int64_t(n_agents) * rank;
    if (NR % 8 != 0 || NR > (1 << 20)) return fail(LRA_ERR_UNSUPPORTED, "n_agents*rank=%lld must be a multiple of 8", (long long)NR);
    if (d_model <= 0 || d_model % 32 != 0) return fail(LRA_ERR_UNSUPPORTED, "d_model=%d must be a positive multiple of 32", d_model);
    if (ldx < d_model || ldx % 8 != 0) return fail(LRA_ERR_SHAPE, "ldx=%lld must be >= d_model and a multiple of 8", (long long)ldx);
    if (vlr_rows < 0) return fail(LRA_ERR_SHAPE, "vlr_rows is negative");
    if (int s = check_vlr(ld_vlr, vlr_agent_stride, vlr_rows, n_agents, rank)) return s;
    if (!out_rows && vlr_rows < T) return fail(LRA_ERR_SHAPE, "vlr_rows=%lld < T=%lld with identity row map", (long long)vlr_rows, (long long)T);
    const lra::PrecomputePlan pl = lra::plan_precompute(T, d_model, int(NR), dtype == LRA_BF16);
    if (int64_t(pl.n_rg + 7) / 8 * 8 * pl.n_cg > INT32_MAX) return fail(LRA_ERR_SHAPE, "n_agents*rank too large for one launch");
    if (T == 0) return LRA_OK;
    if (!X || !A || !V_lr) return fail(LRA_ERR_NULL, "X, A and V_lr must not be NULL");
    if (!aligned(X, 16) || !aligned(A, 16) || !aligned(V_lr, 16)) return fail(LRA_ERR_SHAPE, "X, A and V_lr must be 16-byte aligned");

    lra::PrecomputeParams p{};
    p.X = X; p.A = A; p.Vlr = V_lr; p.out_rows = out_rows;
    p.T = T; p.ldx = ldx; p.ld_vlr = ld_vlr; p.vlr_agent_stride = vlr_agent_stride; p.vlr_rows = vlr_rows;
    p.d_model = d_model; p.rank = rank; p.NR = int(NR);
    p.n_rg = pl.n_rg; p.n_cg = pl.n_cg; p.cols_per_group = pl.cols_per_group;
    p.bf16 = dtype == LRA_BF16;
    return hip_status(lra::launch_precompute(p, static_cast<hipStream_t>(stream)), "lra_lr_precompute launch");
}

// ============================================================================ prefill
namespace {

// key-side LoRA operands of the qkvo configuration (null: keys are K_base)
struct KeyLora {
    const void* K_lr;
    int64_t ld_klr;
    const void* B_k;
    const float* cos;
    const float* sin;
    void* workspace;
    size_t workspace_bytes;
};

// qkvo workspace: [expanded keys: n_rows x n_kv x d_head fp16][largest |key| per (64-key tile, KV
// head): tiles x n_kv fp32]
struct KeyExpandLayout {
    size_t flags_off, total;
};

KeyExpandLayout key_expand_layout(int64_t n_rows, int n_kv, int d_head) {
    KeyExpandLayout L{};
    const int64_t tiles = (n_rows + lra::kKeyTile - 1) / lra::kKeyTile;
    L.flags_off = align_up(size_t(n_rows) * size_t(n_kv) * size_t(d_head) * 2, 256);
    L.total = n_rows > 0 ? L.flags_off + size_t(tiles) * size_t(n_kv) * sizeof(int32_t) : 0;
    return L;
}

int prefill_single(const char* name, int dtype, const void* Q, int64_t L_C, int64_t L_P,
                   const void* K_base, const void* V_base, const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                   const void* B, int32_t n_agents, int32_t agent,
                   int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                   void* O, void* stream, const KeyLora* kl) {
    if (int s = check_dtype(dtype)) return s;
    if (kl && dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "%s: bf16 only", name);
    if (int s = check_heads(n_q, n_kv, d_head, rank)) return s;
    if (int s = check_prefill_rows(n_kv, d_head, ld_vlr)) return s;
    if (L_C < 0 || L_P < 0) return fail(LRA_ERR_SHAPE, "L_C=%lld and L_P=%lld must be >= 0", (long long)L_C, (long long)L_P);
    if (L_P + L_C > (int64_t(1) << 31) - 1) return fail(LRA_ERR_SHAPE, "L_P + L_C exceeds 2^31 - 1");
    if (n_agents <= 0) return fail(LRA_ERR_SHAPE, "n_agents=%d must be positive", n_agents);
    if (agent < lra::kAdapterFree || agent >= n_agents)
        return fail(LRA_ERR_INDEX, "agent=%d outside [-1, %d)", agent, n_agents);
    if (int s = check_vlr(ld_vlr, vlr_agent_stride, L_P + L_C, n_agents, rank)) return s;
    if (kl && (kl->ld_klr < int64_t(n_agents) * rank || kl->ld_klr % 8 != 0))
        return fail(LRA_ERR_SHAPE, "ld_klr=%lld must be >= n_agents*rank and a multiple of 8", (long long)kl->ld_klr);
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(LRA_ERR_SHAPE, "scale must be positive and finite");
    if (L_C == 0) return LRA_OK;
    if (!Q || !K_base || !V_base || !V_lr || !B || !O) return fail(LRA_ERR_NULL, "Q, K_base, V_base, V_lr, B and O must not be NULL");
    if (!aligned(Q, 16) || !aligned(K_base, 16) || !aligned(V_base, 16) || !aligned(V_lr, 16) || !aligned(B, 16) || !aligned(O, 16))
        return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    if (kl && agent == lra::kAdapterFree) kl = nullptr;   // the keys are K_base: the plain kernel
    KeyExpandLayout kx{};
    if (kl) {
        if (!kl->K_lr || !kl->B_k || !kl->cos || !kl->sin) return fail(LRA_ERR_NULL, "K_lr, B_k, rope_cos and rope_sin must not be NULL");
        if (!aligned(kl->K_lr, 16) || !aligned(kl->B_k, 16) || !aligned(kl->cos, 16) || !aligned(kl->sin, 16))
            return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
        kx = key_expand_layout(L_P + L_C, n_kv, d_head);
        if (!kl->workspace) return fail(LRA_ERR_WORKSPACE, "workspace of %zu bytes required", kx.total);
        if (!aligned(kl->workspace, 256)) return fail(LRA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (kl->workspace_bytes < kx.total)
            return fail(LRA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", kl->workspace_bytes, kx.total);
    }
    lra::PrefillParams p{};
    p.Q = Q; p.K = K_base; p.V = V_base; p.Vlr = V_lr; p.B = B; p.O = O;
    p.L_C = L_C; p.L_P = L_P; p.ld_vlr = ld_vlr; p.vlr_agent_stride = vlr_agent_stride;
    p.n_q = n_q; p.n_kv = n_kv; p.G = n_q / n_kv; p.d_head = d_head; p.rank = rank;
    p.agent = agent; p.n_agents = n_agents; p.scale = scale; p.bf16 = dtype == LRA_BF16;
    p.batch = 1;
    p.max_pairs = lra::prefill_pairs(L_C, p.G);
    if (int64_t(p.max_pairs) * n_kv > (int64_t(1) << 31) - 1) return fail(LRA_ERR_SHAPE, "L_C too large for one launch");
    if (kl) {
        // the agent's keys, expanded once per call, then the attention over them
        char* ws = static_cast<char*>(kl->workspace);
        lra::KeyExpandParams e{};
        e.K = K_base; e.Klr = kl->K_lr; e.Bk = kl->B_k; e.rope_cos = kl->cos; e.rope_sin = kl->sin;
        e.Ka = ws; e.flags = reinterpret_cast<int32_t*>(ws + kx.flags_off);
        e.n_rows = L_P + L_C; e.ld_klr = kl->ld_klr;
        e.n_kv = n_kv; e.d_head = d_head; e.rank = rank; e.agent = agent;
        if (int s = hip_status(lra::launch_key_expand(e, static_cast<hipStream_t>(stream)), "lra_attn_prefill_qkvo key expansion"))
            return s;
        p.K = e.Ka;
        p.key_flags = e.flags;
        // the range-safe pass rebuilds the agent's keys in fp32 from these
        p.K_src = K_base; p.Klr = kl->K_lr; p.ld_klr = kl->ld_klr; p.Bk = kl->B_k;
        p.rope_cos = kl->cos; p.rope_sin = kl->sin;
    }
    return hip_status(lra::launch_prefill(p, static_cast<hipStream_t>(stream)), name);
}

}  // namespace

LRA_EXPORT int lra_attn_prefill(int dtype, const void* Q, int64_t L_C, int64_t L_P,
                                const void* K_base, const void* V_base, const void* V_lr, int64_t ld_vlr,
                                int64_t vlr_agent_stride, const void* B, int32_t n_agents, int32_t agent,
                                int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                void* O, void* stream) {
    return prefill_single("lra_attn_prefill launch", dtype, Q, L_C, L_P, K_base, V_base, V_lr, ld_vlr, vlr_agent_stride, B,
                          n_agents, agent, n_q, n_kv, d_head, rank, scale, O, stream, nullptr);
}

LRA_EXPORT size_t lra_attn_prefill_qkvo_workspace_bytes(int64_t n_rows, int32_t n_kv, int32_t d_head) {
    if (n_rows <= 0 || n_kv <= 0 || d_head <= 0) return 0;
    return key_expand_layout(n_rows, n_kv, d_head).total;
}

LRA_EXPORT int lra_attn_prefill_qkvo(int dtype, const void* Q, int64_t L_C, int64_t L_P,
                                     const void* K_base, const void* V_base, const void* V_lr, int64_t ld_vlr,
                                     int64_t vlr_agent_stride, const void* K_lr, int64_t ld_klr, const void* B, const void* B_k,
                                     const float* rope_cos, const float* rope_sin, int32_t n_agents, int32_t agent,
                                     int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                     void* workspace, size_t workspace_bytes, void* O, void* stream) {
    const KeyLora kl{K_lr, ld_klr, B_k, rope_cos, rope_sin, workspace, workspace_bytes};
    return prefill_single("lra_attn_prefill_qkvo launch", dtype, Q, L_C, L_P, K_base, V_base, V_lr, ld_vlr,
                          vlr_agent_stride, B,
                          n_agents, agent, n_q, n_kv, d_head, rank, scale, O, stream, &kl);
}

LRA_EXPORT int lra_attn_prefill_varlen(int dtype, const void* Q, int64_t q_rows, int32_t batch,
                                       const int64_t* q_start, const int32_t* q_len, int64_t max_q_len,
                                       const void* K_base, const void* V_base, int64_t kv_rows,
                                       const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                                       const int64_t* kv_start, const int32_t* kv_prefix,
                                       const void* B, int32_t n_agents, const int32_t* agent,
                                       int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                       void* O, void* stream) {
    if (int s = check_dtype(dtype)) return s;
    if (int s = check_heads(n_q, n_kv, d_head, rank)) return s;
    if (int s = check_prefill_rows(n_kv, d_head, ld_vlr)) return s;
    if (batch < 0 || q_rows < 0 || kv_rows < 0 || max_q_len < 0)
        return fail(LRA_ERR_SHAPE, "batch, q_rows, kv_rows and max_q_len must be >= 0");
    if (max_q_len > (int64_t(1) << 31) - 1) return fail(LRA_ERR_SHAPE, "max_q_len exceeds 2^31 - 1");
    if (n_agents <= 0) return fail(LRA_ERR_SHAPE, "n_agents=%d must be positive", n_agents);
    if (int s = check_vlr(ld_vlr, vlr_agent_stride, kv_rows, n_agents, rank)) return s;
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(LRA_ERR_SHAPE, "scale must be positive and finite");
    if (batch == 0 || max_q_len == 0) return LRA_OK;
    if (!Q || !K_base || !V_base || !V_lr || !B || !O || !q_start || !q_len || !kv_start || !kv_prefix || !agent)
        return fail(LRA_ERR_NULL, "tensor and index pointers must not be NULL");
    if (!aligned(Q, 16) || !aligned(K_base, 16) || !aligned(V_base, 16) || !aligned(V_lr, 16) || !aligned(B, 16) || !aligned(O, 16))
        return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    lra::PrefillParams p{};
    p.Q = Q; p.K = K_base; p.V = V_base; p.Vlr = V_lr; p.B = B; p.O = O;
    p.ld_vlr = ld_vlr; p.vlr_agent_stride = vlr_agent_stride;
    p.n_q = n_q; p.n_kv = n_kv; p.G = n_q / n_kv; p.d_head = d_head; p.rank = rank;
    p.n_agents = n_agents; p.scale = scale; p.bf16 = dtype == LRA_BF16;
    p.q_start = q_start; p.q_len = q_len; p.kv_start = kv_start; p.kv_prefix = kv_prefix; p.agents = agent;
    p.q_rows = q_rows; p.kv_rows = kv_rows; p.batch = batch; p.max_q_len = max_q_len;
    p.max_pairs = lra::prefill_pairs(max_q_len, p.G);
    if (int64_t(batch) * p.max_pairs * n_kv > (int64_t(1) << 31) - 1)
        return fail(LRA_ERR_SHAPE, "batch x max_q_len too large for one launch");
    return hip_status(lra::launch_prefill(p, static_cast<hipStream_t>(stream)), "lra_attn_prefill_varlen launch");
}

LRA_EXPORT int lra_attn_prefill_paged(int dtype, const void* Q, int64_t q_rows, int32_t batch,
                                      const int64_t* q_start, const int32_t* q_len, int64_t max_q_len,
                                      const void* K_pages, const void* V_pages, const void* Vlr_pages,
                                      int64_t n_pages, int32_t page_size, int64_t ld_vlr,
                                      const int32_t* block_table, int32_t max_blocks, const int32_t* kv_prefix,
                                      const void* B, int32_t n_agents, const int32_t* agent,
                                      int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                      void* O, void* stream) {
    if (int s = check_dtype(dtype)) return s;
    if (int s = check_heads(n_q, n_kv, d_head, rank)) return s;
    if (batch < 0 || q_rows < 0 || max_q_len < 0) return fail(LRA_ERR_SHAPE, "batch, q_rows and max_q_len must be >= 0");
    if (max_q_len > (int64_t(1) << 31) - 1) return fail(LRA_ERR_SHAPE, "max_q_len exceeds 2^31 - 1");
    if (page_size < 64 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0)
        return fail(LRA_ERR_UNSUPPORTED, "page_size=%d must be a power of two in [64, 65536]", page_size);
    if (n_pages <= 0 || max_blocks <= 0) return fail(LRA_ERR_SHAPE, "n_pages and max_blocks must be positive");
    if (n_agents <= 0) return fail(LRA_ERR_SHAPE, "n_agents=%d must be positive", n_agents);
    if (ld_vlr < int64_t(n_agents) * rank || ld_vlr % 8 != 0)
        return fail(LRA_ERR_SHAPE, "ld_vlr=%lld must be >= n_agents*rank and a multiple of 8", (long long)ld_vlr);
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(LRA_ERR_SHAPE, "scale must be positive and finite");
    if (batch == 0 || max_q_len == 0) return LRA_OK;
    if (!Q || !K_pages || !V_pages || !Vlr_pages || !B || !O || !q_start || !q_len || !block_table || !kv_prefix || !agent)
        return fail(LRA_ERR_NULL, "tensor and index pointers must not be NULL");
    if (!aligned(Q, 16) || !aligned(K_pages, 16) || !aligned(V_pages, 16) || !aligned(Vlr_pages, 16) || !aligned(B, 16) ||
        !aligned(O, 16))
        return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    lra::PrefillParams p{};
    p.Q = Q; p.K = K_pages; p.V = V_pages; p.Vlr = Vlr_pages; p.B = B; p.O = O;
    p.ld_vlr = ld_vlr; p.vlr_agent_stride = rank;   // pages hold interleaved rows
    p.n_q = n_q; p.n_kv = n_kv; p.G = n_q / n_kv; p.d_head = d_head; p.rank = rank;
    p.n_agents = n_agents; p.scale = scale; p.bf16 = dtype == LRA_BF16;
    p.q_start = q_start; p.q_len = q_len; p.kv_start = nullptr; p.kv_prefix = kv_prefix; p.agents = agent;
    p.q_rows = q_rows; p.kv_rows = int64_t(max_blocks) * page_size; p.batch = batch; p.max_q_len = max_q_len;
    p.block_table = block_table; p.n_pages = n_pages; p.max_blocks = max_blocks;
    p.page_shift = __builtin_ctz(unsigned(page_size));
    p.max_pairs = lra::prefill_pairs(max_q_len, p.G);
    if (int64_t(batch) * p.max_pairs * n_kv > (int64_t(1) << 31) - 1)
        return fail(LRA_ERR_SHAPE, "batch x max_q_len too large for one launch");
    return hip_status(lra::launch_prefill(p, static_cast<hipStream_t>(stream)), "lra_attn_prefill_paged launch");
}

// ============================================================================ decode
LRA_EXPORT int32_t lra_attn_decode_default_split(int32_t batch, int32_t n_kv, int64_t max_kv_len) {
    // keys per slice of the library's choice when every request has max_kv_len keys
    const int n = lra::decode_slots(batch, n_kv, max_kv_len, 0);
    if (n <= 0) return 0;
    const int64_t units = int64_t(batch) * ((max_kv_len + 31) / 32);
    const int64_t n_act = std::min<int64_t>(n, units);
    const int64_t keys = (int64_t(batch) * max_kv_len + n_act - 1) / n_act;   // a valid keys_per_split: multiple of 64
    return int32_t(std::min<int64_t>((keys + 63) / 64 * 64, INT32_MAX / 64 * 64));
}

LRA_EXPORT size_t lra_attn_decode_workspace_bytes(int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_head,
                                                  int32_t rank, int64_t max_kv_len, int32_t keys_per_split) {
    if (batch <= 0 || n_q <= 0 || n_kv <= 0 || max_kv_len <= 0 || d_head <= 0 || rank <= 0) return 0;
    if (keys_per_split < 0 || keys_per_split % 64 != 0) return 0;
    return decode_layout(batch, n_q, n_kv, d_head, rank, max_kv_len, keys_per_split).total;
}

LRA_EXPORT int32_t lra_attn_decode_paged_default_split(int32_t batch, int32_t n_kv, int64_t max_kv_len, int32_t page_size) {
    if (page_size < 32 || (page_size & (page_size - 1)) != 0) return 0;
    return lra_attn_decode_default_split(batch, n_kv, max_kv_len);
}

namespace {
// paged decode with K / V element (page, row in page, KV head, c) at
// page * page_stride + row * row_stride + head * head_stride + c
int decode_paged_call(const char* name, int dtype, const void* Q, int32_t batch,
                      const void* K_pages, const void* V_pages, const void* Vlr_pages,
                      int64_t n_pages, int32_t page_size, int64_t ld_vlr,
                      int64_t page_stride, int64_t row_stride, int64_t head_stride,
                      const int32_t* block_table, int32_t max_blocks,
                      const int32_t* kv_len, int64_t max_kv_len,
                      const void* B, int32_t n_agents, const int32_t* agent,
                      int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                      int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                      void* O, void* stream) {
    if (int s = check_dtype(dtype)) return s;
    if (int s = check_heads(n_q, n_kv, d_head, rank)) return s;
    if (batch < 0) return fail(LRA_ERR_SHAPE, "batch=%d is negative", batch);
    if (page_size < 32 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0)
        return fail(LRA_ERR_UNSUPPORTED, "page_size=%d must be a power of two in [32, 65536]", page_size);
    if (n_pages <= 0 || max_blocks <= 0) return fail(LRA_ERR_SHAPE, "n_pages and max_blocks must be positive");
    if (max_kv_len < 0 || max_kv_len > int64_t(max_blocks) * page_size)
        return fail(LRA_ERR_SHAPE, "max_kv_len=%lld must be in [0, max_blocks * page_size]", (long long)max_kv_len);
    if (max_kv_len > (int64_t(1) << 31) - 1) return fail(LRA_ERR_SHAPE, "max_kv_len exceeds 2^31 - 1");
    if (n_agents <= 0) return fail(LRA_ERR_SHAPE, "n_agents=%d must be positive", n_agents);
    if (ld_vlr < int64_t(n_agents) * rank || ld_vlr % 8 != 0)
        return fail(LRA_ERR_SHAPE, "ld_vlr=%lld must be >= n_agents*rank and a multiple of 8", (long long)ld_vlr);
    if (keys_per_split < 0 || keys_per_split % 64 != 0)
        return fail(LRA_ERR_SHAPE, "keys_per_split=%d must be 0 or a positive multiple of 64", keys_per_split);
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(LRA_ERR_SHAPE, "scale must be positive and finite");
    if (page_stride <= 0 || row_stride <= 0 || head_stride <= 0 || page_stride % 8 != 0 || row_stride % 8 != 0 ||
        head_stride % 8 != 0)
        return fail(LRA_ERR_SHAPE, "K/V strides (%lld, %lld, %lld) must be positive multiples of 8",
                    (long long)page_stride, (long long)row_stride, (long long)head_stride);
    if (row_stride > (int64_t(1) << 24)) return fail(LRA_ERR_SHAPE, "K/V row stride exceeds 2^24 elements");
    if (batch == 0) return LRA_OK;
    if (!Q || !K_pages || !V_pages || !Vlr_pages || !B || !O || !block_table || !kv_len || !agent)
        return fail(LRA_ERR_NULL, "tensor and index pointers must not be NULL");
    if (!aligned(Q, 16) || !aligned(K_pages, 16) || !aligned(V_pages, 16) || !aligned(Vlr_pages, 16) || !aligned(B, 16) ||
        !aligned(O, 16))
        return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    const DecodeLayout L = decode_layout(batch, n_q, n_kv, d_head, rank, max_kv_len, keys_per_split);
    if (L.n_slots < 0) return fail(LRA_ERR_SHAPE, "batch x max_kv_len too large for one launch");
    if (L.total) {
        if (!workspace) return fail(LRA_ERR_WORKSPACE, "workspace of %zu bytes required", L.total);
        if (!aligned(workspace, 256)) return fail(LRA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (workspace_bytes < L.total) return fail(LRA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, L.total);
    }
    lra::DecodeParams p{};
    p.Q = Q; p.K = K_pages; p.V = V_pages; p.Vlr = Vlr_pages; p.B = B;
    p.kv_start = nullptr; p.kv_len = kv_len; p.agent = agent;
    p.records = L.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.rec_off) : nullptr;
    p.record_bytes = uint32_t(L.rec_bytes);
    p.O = O; p.ld_vlr = ld_vlr; p.vlr_agent_stride = rank; p.kv_rows = int64_t(max_blocks) * page_size; p.max_kv_len = max_kv_len;
    p.kv_row_stride = row_stride; p.kv_head_stride = head_stride; p.kv_page_stride = page_stride;
    p.batch = batch; p.n_q = n_q; p.n_kv = n_kv; p.G = n_q / n_kv; p.n_agents = n_agents;
    p.d_head = d_head; p.rank = rank; p.n_slots = std::max(L.n_slots, 0); p.scale = scale;
    p.bf16 = dtype == LRA_BF16;
    p.block_table = block_table; p.n_pages = n_pages; p.max_blocks = max_blocks;
    p.page_shift = __builtin_ctz(unsigned(page_size));
    return hip_status(lra::launch_decode(p, static_cast<hipStream_t>(stream)), name);
}
}  // namespace

LRA_EXPORT int lra_attn_decode_paged(int dtype, const void* Q, int32_t batch,
                                     const void* K_pages, const void* V_pages, const void* Vlr_pages,
                                     int64_t n_pages, int32_t page_size, int64_t ld_vlr,
                                     const int32_t* block_table, int32_t max_blocks,
                                     const int32_t* kv_len, int64_t max_kv_len,
                                     const void* B, int32_t n_agents, const int32_t* agent,
                                     int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                     int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                                     void* O, void* stream) {
    // token-major pages [n_pages x P x n_kv x d_head]
    const int64_t row = int64_t(n_kv) * d_head;
    return decode_paged_call("lra_attn_decode_paged launch", dtype, Q, batch, K_pages, V_pages, Vlr_pages, n_pages,
                             page_size, ld_vlr, row * page_size, row, d_head, block_table, max_blocks, kv_len,
                             max_kv_len, B, n_agents, agent, n_q, n_kv, d_head, rank, scale, keys_per_split,
                             workspace, workspace_bytes, O, stream);
}

LRA_EXPORT int lra_attn_decode_paged_strided(int dtype, const void* Q, int32_t batch,
                                             const void* K_pages, const void* V_pages, const void* Vlr_pages,
                                             int64_t n_pages, int32_t page_size, int64_t ld_vlr,
                                             int64_t kv_page_stride, int64_t kv_row_stride, int64_t kv_head_stride,
                                             const int32_t* block_table, int32_t max_blocks,
                                             const int32_t* kv_len, int64_t max_kv_len,
                                             const void* B, int32_t n_agents, const int32_t* agent,
                                             int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                             int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                                             void* O, void* stream) {
    return decode_paged_call("lra_attn_decode_paged_strided launch", dtype, Q, batch, K_pages, V_pages, Vlr_pages,
                             n_pages, page_size, ld_vlr, kv_page_stride, kv_row_stride, kv_head_stride, block_table,
                             max_blocks, kv_len, max_kv_len, B, n_agents, agent, n_q, n_kv, d_head, rank, scale,
                             keys_per_split, workspace, workspace_bytes, O, stream);
}

namespace {

// key-side LoRA operands of a decode (null: keys are K_base)
struct DecodeKeyLora {
    const void* K_lr;
    int64_t ld_klr;
    const void* B_k;
    const float* cos;
    const float* sin;
};

int64_t key_score_stride(int64_t max_kv_len) { return (max_kv_len + 63) / 64 * 64; }

// decode workspace, then (LoRA on the keys) the fp32 key scores [batch x n_q x stride], the fp16
// score weights [batch x n_q x d_head*rank], the repacked rotary tables and the score pass's range
// flags [batch x key blocks x head blocks], each part 256-aligned
size_t decode_qkvo_bytes(const DecodeLayout& L, int batch, int n_q, int d_head, int rank, int64_t max_kv_len,
                         size_t* ks_off, size_t* w_off, size_t* t_off, size_t* f_off) {
    *ks_off = align_up(L.total, 256);
    *w_off = align_up(*ks_off + size_t(batch) * size_t(n_q) * size_t(key_score_stride(max_kv_len)) * 4, 256);
    *t_off = align_up(*w_off + size_t(batch) * size_t(n_q) * size_t(d_head) * size_t(rank) * 2, 256);
    *f_off = align_up(*t_off + lra::key_score_table_bytes(max_kv_len, d_head, rank), 256);
    const int hpb = lra::key_score_heads(d_head, rank);
    const size_t blocks = size_t((max_kv_len + lra::kKeyScoreBlock - 1) / lra::kKeyScoreBlock);
    return *f_off + size_t(batch) * blocks * size_t((n_q + hpb - 1) / hpb) * sizeof(int32_t);
}

// the newest tokens' hidden states of a decode step (null: a plain decode)
struct DecodeStep {
    const void* X_new;
    int64_t ldx;
    const void* A;
    int32_t d_model;
};

int decode_call(const char* name, int dtype, const void* Q, int32_t batch,
                const void* K_base, const void* V_base, int64_t kv_rows, int64_t kv_row_stride, int64_t kv_head_stride,
                const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                const void* B, int32_t n_agents, const int32_t* agent,
                int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                void* O, void* stream, const DecodeKeyLora* kl, const DecodeStep* st = nullptr) {
    if (int s = check_dtype(dtype)) return s;
    if (st) {
        if (st->d_model <= 0 || st->d_model % 64 != 0)
            return fail(LRA_ERR_SHAPE, "d_model=%d must be a positive multiple of 64", st->d_model);
        if (st->ldx < st->d_model || st->ldx % 8 != 0)
            return fail(LRA_ERR_SHAPE, "ldx=%lld must be >= d_model and a multiple of 8", (long long)st->ldx);
    }
    if (kl && dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "%s: bf16 only", name);
    if (int s = check_heads(n_q, n_kv, d_head, rank)) return s;
    if (batch < 0) return fail(LRA_ERR_SHAPE, "batch=%d is negative", batch);
    if (kv_rows < 0 || max_kv_len < 0) return fail(LRA_ERR_SHAPE, "kv_rows and max_kv_len must be >= 0");
    if (max_kv_len > (int64_t(1) << 31) - 1) return fail(LRA_ERR_SHAPE, "max_kv_len exceeds 2^31 - 1");
    // key-score grid: one workgroup row per 512-key block (at most 32,768)
    if (kl && max_kv_len > (int64_t(1) << 24)) return fail(LRA_ERR_SHAPE, "max_kv_len exceeds 2^24 with LoRA on the keys");
    if (n_agents <= 0) return fail(LRA_ERR_SHAPE, "n_agents=%d must be positive", n_agents);
    if (int s = check_vlr(ld_vlr, vlr_agent_stride, kv_rows, n_agents, rank)) return s;
    if (kl && (kl->ld_klr < int64_t(n_agents) * rank || kl->ld_klr % 8 != 0))
        return fail(LRA_ERR_SHAPE, "ld_klr=%lld must be >= n_agents*rank and a multiple of 8", (long long)kl->ld_klr);
    if (keys_per_split < 0 || keys_per_split % 64 != 0)
        return fail(LRA_ERR_SHAPE, "keys_per_split=%d must be 0 or a positive multiple of 64", keys_per_split);
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(LRA_ERR_SHAPE, "scale must be positive and finite");
    // strides: 16-byte aligned rows of d elements; a 32-key tile spans less than 2^31 bytes
    if (kv_row_stride <= 0 || kv_head_stride <= 0 || kv_row_stride % 8 != 0 || kv_head_stride % 8 != 0)
        return fail(LRA_ERR_SHAPE, "K/V strides (%lld, %lld) must be positive multiples of 8",
                    (long long)kv_row_stride, (long long)kv_head_stride);
    if (kv_row_stride > (int64_t(1) << 24)) return fail(LRA_ERR_SHAPE, "K/V row stride exceeds 2^24 elements");
    if (batch == 0) return LRA_OK;
    if (!Q || !K_base || !V_base || !V_lr || !B || !O || !kv_start || !kv_len || !agent)
        return fail(LRA_ERR_NULL, "tensor and index pointers must not be NULL");
    if (!aligned(Q, 16) || !aligned(K_base, 16) || !aligned(V_base, 16) || !aligned(V_lr, 16) || !aligned(B, 16) || !aligned(O, 16))
        return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    if (st) {
        if (!st->X_new || !st->A) return fail(LRA_ERR_NULL, "X_new and A must not be NULL");
        if (!aligned(st->X_new, 16) || !aligned(st->A, 16)) return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    }
    if (kl) {
        if (!kl->K_lr || !kl->B_k || !kl->cos || !kl->sin) return fail(LRA_ERR_NULL, "K_lr, B_k, rope_cos and rope_sin must not be NULL");
        if (!aligned(kl->K_lr, 16) || !aligned(kl->B_k, 16) || !aligned(kl->cos, 16) || !aligned(kl->sin, 16))
            return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    }
    const DecodeLayout L = decode_layout(batch, n_q, n_kv, d_head, rank, max_kv_len, keys_per_split);
    if (L.n_slots < 0) return fail(LRA_ERR_SHAPE, "batch x max_kv_len too large for one launch");
    size_t ks_off = 0, w_off = 0, t_off = 0, f_off = 0;
    const size_t need = kl ? (max_kv_len > 0 ? decode_qkvo_bytes(L, batch, n_q, d_head, rank, max_kv_len, &ks_off, &w_off, &t_off, &f_off) : 0)
                           : L.total;
    if (need) {
        if (!workspace) return fail(LRA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
        if (!aligned(workspace, 256)) return fail(LRA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (workspace_bytes < need) return fail(LRA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, need);
    }
    lra::DecodeParams p{};
    p.Q = Q; p.K = K_base; p.V = V_base; p.Vlr = V_lr; p.B = B;
    p.kv_start = kv_start; p.kv_len = kv_len; p.agent = agent;
    p.records = L.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.rec_off) : nullptr;
    p.record_bytes = uint32_t(L.rec_bytes);
    p.O = O; p.ld_vlr = ld_vlr; p.vlr_agent_stride = vlr_agent_stride; p.kv_rows = kv_rows; p.max_kv_len = max_kv_len;
    p.kv_row_stride = kv_row_stride; p.kv_head_stride = kv_head_stride; p.kv_page_stride = 0;
    p.batch = batch; p.n_q = n_q; p.n_kv = n_kv; p.G = n_q / n_kv; p.n_agents = n_agents;
    p.d_head = d_head; p.rank = rank; p.n_slots = std::max(L.n_slots, 0); p.scale = scale;
    p.bf16 = dtype == LRA_BF16;
    // small batches of plain decodes: one workgroup per (request, KV head, 256-key chunk)
    if (!st && !kl) p.n_chunks = lra::decode_small_chunks(batch, n_kv, max_kv_len, keys_per_split, &p.chunk_keys);
    if (st) {
        p.X_new = st->X_new;
        p.A_new = st->A;
        p.ldx = st->ldx;
        p.d_model = st->d_model;
        p.n_pre = (batch + 1) / 2;
        p.n_pre = (p.n_pre + 7) / 8 * 8;
        if (int64_t(p.n_pre) + int64_t(p.n_slots) * ((n_kv + 7) / 8) > INT32_MAX)
            return fail(LRA_ERR_SHAPE, "batch too large for one launch");
    }
    if (kl && max_kv_len > 0) {
        // the rank-r part of every score first, then the attention adds it to the base scores
        lra::KeyScoreParams e{};
        e.Q = Q; e.Klr = kl->K_lr; e.Bk = kl->B_k; e.rope_cos = kl->cos; e.rope_sin = kl->sin;
        e.kv_start = kv_start; e.kv_len = kv_len; e.agent = agent;
        e.S = reinterpret_cast<float*>(static_cast<char*>(workspace) + ks_off);
        e.flags = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + f_off);
        e.W = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + w_off);
        e.Tp = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + t_off);
        e.kv_rows = kv_rows; e.max_kv_len = max_kv_len; e.ld_klr = kl->ld_klr; e.ks_stride = key_score_stride(max_kv_len);
        e.batch = batch; e.n_q = n_q; e.n_kv = n_kv; e.G = n_q / n_kv; e.n_agents = n_agents; e.d_head = d_head; e.rank = rank;
        e.scale = scale;
        if (int s = hip_status(lra::launch_key_scores(e, static_cast<hipStream_t>(stream)), "lra_attn_decode_qkvo key scores"))
            return s;
        p.key_scores = e.S;
        p.ks_stride = e.ks_stride;
    }
    return hip_status(lra::launch_decode(p, static_cast<hipStream_t>(stream)), name);
}

}  // namespace

LRA_EXPORT int lra_attn_decode(int dtype, const void* Q, int32_t batch,
                               const void* K_base, const void* V_base, int64_t kv_rows,
                               const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                               const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                               const void* B, int32_t n_agents, const int32_t* agent,
                               int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                               int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                               void* O, void* stream) {
    return decode_call("lra_attn_decode launch", dtype, Q, batch, K_base, V_base, kv_rows, int64_t(n_kv) * d_head, d_head,
                       V_lr, ld_vlr, vlr_agent_stride, kv_start,
                       kv_len, max_kv_len, B, n_agents, agent, n_q, n_kv, d_head, rank, scale, keys_per_split,
                       workspace, workspace_bytes, O, stream, nullptr);
}

LRA_EXPORT int lra_attn_decode_strided(int dtype, const void* Q, int32_t batch,
                                       const void* K_base, const void* V_base, int64_t kv_rows,
                                       int64_t kv_row_stride, int64_t kv_head_stride,
                                       const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                                       const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                                       const void* B, int32_t n_agents, const int32_t* agent,
                                       int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                       int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                                       void* O, void* stream) {
    return decode_call("lra_attn_decode_strided launch", dtype, Q, batch, K_base, V_base, kv_rows, kv_row_stride,
                       kv_head_stride, V_lr, ld_vlr, vlr_agent_stride, kv_start, kv_len, max_kv_len, B, n_agents, agent, n_q, n_kv,
                       d_head, rank, scale, keys_per_split, workspace, workspace_bytes, O, stream, nullptr);
}

LRA_EXPORT int lra_attn_decode_step(int dtype, const void* Q, int32_t batch,
                                    const void* K_base, const void* V_base, int64_t kv_rows,
                                    void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                                    const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                                    const void* B, int32_t n_agents, const int32_t* agent,
                                    int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                    const void* X_new, int64_t ldx, const void* A, int32_t d_model,
                                    int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                                    void* O, void* stream) {
    const DecodeStep st{X_new, ldx, A, d_model};
    return decode_call("lra_attn_decode_step launch", dtype, Q, batch, K_base, V_base, kv_rows, int64_t(n_kv) * d_head,
                       d_head, V_lr, ld_vlr, vlr_agent_stride, kv_start, kv_len, max_kv_len, B, n_agents, agent, n_q, n_kv, d_head, rank,
                       scale, keys_per_split, workspace, workspace_bytes, O, stream, nullptr, &st);
}

// ============================================================================ decode without allocation
// The split partials of lra_attn_decode_noalloc live here. In host code this name is only a stand-in
// for the symbol: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[LRA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// device address of `scratch` on the current device (looked up on the first call there)
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (int s = hip_status(hipGetDevice(&dev), "hipGetDevice")) return s;
    if (dev < 0 || dev >= kMaxDevices) return fail(LRA_ERR_UNSUPPORTED, "device %d: the library tracks devices 0..%d", dev, kMaxDevices - 1);
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (int s = hip_status(g_scratch_err[dev], "hipGetSymbolAddress(scratch)")) return s;
    *out = g_scratch_ptr[dev];
    return LRA_OK;
}

}  // namespace

LRA_EXPORT int lra_stream_read(const void* x, int64_t bytes, int32_t n_workgroups, uint32_t* out, void* stream) {
    if (!x || !out) return fail(LRA_ERR_NULL, "x and out must not be NULL");
    if (!aligned(x, 16)) return fail(LRA_ERR_SHAPE, "x must be 16-byte aligned");
    if (n_workgroups < 1 || n_workgroups > (1 << 20))
        return fail(LRA_ERR_SHAPE, "n_workgroups=%d must be in [1, 2^20]", n_workgroups);
    if (bytes <= 0 || bytes % (int64_t(16) * n_workgroups) != 0)
        return fail(LRA_ERR_SHAPE, "bytes=%lld must be a positive multiple of 16 x n_workgroups", (long long)bytes);
    return hip_status(lra::launch_read_probe(x, bytes, n_workgroups, out, static_cast<hipStream_t>(stream)), "lra_stream_read launch");
}

LRA_EXPORT int lra_attn_decode_noalloc(int dtype, const void* Q, int32_t batch,
                                       const void* K_base, const void* V_base, int64_t kv_rows,
                                       const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                                       const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                                       const void* B, int32_t n_agents, const int32_t* agent,
                                       int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                       int32_t keys_per_split, void* O, void* stream) {
    const size_t need = lra_attn_decode_workspace_bytes(batch, n_q, n_kv, d_head, rank, max_kv_len, keys_per_split);
    if (need > LRA_NOALLOC_SCRATCH_BYTES)
        return fail(LRA_ERR_WORKSPACE, "lra_attn_decode_noalloc: these sizes need %zu bytes of partials, the static "
                    "array holds %zu (use lra_attn_decode with a workspace)", need, size_t(LRA_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    if (need && batch > 0) {
        if (int s = scratch_on_current_device(&ws)) return s;
    }
    return decode_call("lra_attn_decode_noalloc launch", dtype, Q, batch, K_base, V_base, kv_rows, int64_t(n_kv) * d_head,
                       d_head, V_lr, ld_vlr, vlr_agent_stride, kv_start, kv_len, max_kv_len, B, n_agents, agent, n_q, n_kv, d_head, rank,
                       scale, keys_per_split, ws, ws ? size_t(LRA_NOALLOC_SCRATCH_BYTES) : 0, O, stream, nullptr);
}

LRA_EXPORT size_t lra_attn_decode_qkvo_workspace_bytes(int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_head,
                                                       int32_t rank, int64_t max_kv_len, int32_t keys_per_split) {
    if (batch <= 0 || n_q <= 0 || n_kv <= 0 || d_head <= 0 || rank <= 0 || max_kv_len <= 0 || keys_per_split < 0) return 0;
    if (keys_per_split % 64 != 0) return 0;
    size_t ks_off = 0, w_off = 0, t_off = 0, f_off = 0;
    return decode_qkvo_bytes(decode_layout(batch, n_q, n_kv, d_head, rank, max_kv_len, keys_per_split), batch, n_q,
                             d_head, rank, max_kv_len, &ks_off, &w_off, &t_off, &f_off);
}

LRA_EXPORT int lra_attn_decode_qkvo(int dtype, const void* Q, int32_t batch,
                                    const void* K_base, const void* V_base, int64_t kv_rows,
                                    const void* V_lr, int64_t ld_vlr, int64_t vlr_agent_stride,
                                    const void* K_lr, int64_t ld_klr,
                                    const int64_t* kv_start, const int32_t* kv_len, int64_t max_kv_len,
                                    const void* B, const void* B_k, const float* rope_cos, const float* rope_sin,
                                    int32_t n_agents, const int32_t* agent,
                                    int32_t n_q, int32_t n_kv, int32_t d_head, int32_t rank, float scale,
                                    int32_t keys_per_split, void* workspace, size_t workspace_bytes,
                                    void* O, void* stream) {
    const DecodeKeyLora kl{K_lr, ld_klr, B_k, rope_cos, rope_sin};
    return decode_call("lra_attn_decode_qkvo launch", dtype, Q, batch, K_base, V_base, kv_rows, int64_t(n_kv) * d_head,
                       d_head, V_lr, ld_vlr, vlr_agent_stride, kv_start,
                       kv_len, max_kv_len, B, n_agents, agent, n_q, n_kv, d_head, rank, scale, keys_per_split,
                       workspace, workspace_bytes, O, stream, &kl);
}

namespace lra {

int decode_slots(int batch, int n_kv, int64_t max_kv_len, int keys_per_split) {
    if (batch <= 0 || n_kv <= 0 || max_kv_len <= 0) return 0;
    const int64_t units_max = int64_t(batch) * ((max_kv_len + 31) / 32);   // 32-key tiles
    const int64_t n_hg = (n_kv + 7) / 8;                                   // workgroups per slot
    int64_t n;
    if (keys_per_split > 0) {
        n = (int64_t(batch) * max_kv_len + keys_per_split - 1) / keys_per_split;
    } else {
        // One 8-wave workgroup per CU on 15/16 of the 256 CUs of MI355X, each streaming its slice
        // as one sequence of tiles. Measured on MI355X: 16 x 66,400 keys take 0.722 ms this way
        // against 0.740 with two rounds of half-size slices (the previous kernel's best), and
        // counter-fed slices for the stragglers cost more in merge pieces than they saved.
        n = std::max<int64_t>(8, 256 * 15 / 16 / n_hg / 8 * 8);
        n = std::min(n, units_max);   // down to one tile per slice for small batches
    }
    n = (std::max<int64_t>(n, 1) + 7) / 8 * 8;
    // the grid (n x n_hg workgroups) and the 32-bit unit counts of the kernels stay in range
    if (n > (int64_t(1) << 24) || n * n_hg > INT32_MAX || units_max > INT32_MAX) return -1;
    return int(n);
}

}  // namespace lra

// ============================================================================ value expansion
LRA_EXPORT int lra_expand_values(int dtype, const void* V_base, int64_t kv_rows, const void* V_lr, int64_t ld_vlr,
                                 const void* B, int32_t n_agents, int32_t n_kv, int32_t d_head, int32_t rank,
                                 int32_t batch, const int64_t* src_start, const int32_t* len,
                                 const int32_t* agent, int64_t max_len,
                                 void* V_out, int64_t out_rows, const int64_t* dst_start, void* stream) {
    if (int s = check_dtype(dtype)) return s;
    if (n_kv <= 0) return fail(LRA_ERR_SHAPE, "n_kv=%d must be positive", n_kv);
    if (d_head != 64 && d_head != 128) return fail(LRA_ERR_UNSUPPORTED, "d_head=%d (supported: 64, 128)", d_head);
    if (rank != 8 && rank != 16) return fail(LRA_ERR_UNSUPPORTED, "rank=%d (supported: 8, 16)", rank);
    if (int64_t(n_kv) * d_head > (int64_t(1) << 24)) return fail(LRA_ERR_SHAPE, "n_kv*d_head exceeds 2^24");
    if (n_agents <= 0) return fail(LRA_ERR_SHAPE, "n_agents=%d must be positive", n_agents);
    if (batch < 0 || kv_rows < 0 || out_rows < 0 || max_len < 0)
        return fail(LRA_ERR_SHAPE, "batch, kv_rows, out_rows and max_len must be >= 0");
    if (max_len > (int64_t(1) << 31) - 1) return fail(LRA_ERR_SHAPE, "max_len exceeds 2^31 - 1");
    if (ld_vlr < int64_t(n_agents) * rank || ld_vlr % 8 != 0)
        return fail(LRA_ERR_SHAPE, "ld_vlr=%lld must be >= n_agents*rank and a multiple of 8", (long long)ld_vlr);
    const int rows_per_wg = lra::value_expand_rows(batch, max_len);
    const int64_t n_chunks = (max_len + rows_per_wg - 1) / rows_per_wg;
    // one-dimensional grid of (request, chunk) workgroups of 256 threads
    if (int64_t(batch) * n_chunks > (int64_t(1) << 24))
        return fail(LRA_ERR_SHAPE, "batch x ceil(max_len/256) exceeds 2^24 workgroups");
    if (batch == 0 || max_len == 0) return LRA_OK;
    if (!V_base || !V_lr || !B || !V_out || !src_start || !len || !agent || !dst_start)
        return fail(LRA_ERR_NULL, "tensor and index pointers must not be NULL");
    if (!aligned(V_base, 16) || !aligned(V_lr, 16) || !aligned(B, 16) || !aligned(V_out, 16))
        return fail(LRA_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    lra::ValueExpandParams p{};
    p.V = V_base; p.Vlr = V_lr; p.B = B; p.Vout = V_out;
    p.src_start = src_start; p.len = len; p.agent = agent; p.dst_start = dst_start;
    p.kv_rows = kv_rows; p.out_rows = out_rows; p.ld_vlr = ld_vlr; p.max_len = max_len; p.n_chunks = n_chunks;
    p.batch = batch; p.n_agents = n_agents; p.row_elems = n_kv * d_head; p.rank = rank;
    p.rows_per_wg = rows_per_wg;
    p.bf16 = dtype == LRA_BF16;
    return hip_status(lra::launch_value_expand(p, static_cast<hipStream_t>(stream)), "lra_expand_values launch");
}
