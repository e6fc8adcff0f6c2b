// Flash-LoRA-Attention decode for gfx950: split along the key axis, merged by log-sum-exp.
//
// Method (LRAgent page, "method steps" (3)-(4)): stream key/value tiles, keep the online-softmax
// statistics, accumulate the base output O and the rank-r output O_lr from the agent's LR cache,
// and only after the last tile apply O <- O + O_lr B_agent and normalise. The rank-r accumulation
// is what makes the reordering pay: the per-key work of the LR path is r multiply-adds instead of
// d_head (LRAgent page, "core method" / "technical novelty": associativity moves the d_out-wide
// product out of the key loop).
//
// Work split: the batch's keys, counted in 32-key tiles (units) per request, are cut into equal
// contiguous slices (stream-K style), one per workgroup slot: 15/16 of the chip's CUs, so the
// whole launch is one round of workgroups; one workgroup of 8 waves takes a slice for 8 KV heads,
// one wave per head. Every workgroup streams the same number of bytes whatever the request
// lengths; a slice covers the end of one request and the start of the next as two pieces, each
// with its own partial. The 8 waves read the same keys of 8 heads, i.e. whole 2 KB token rows of
// a token-major cache, and the V_lr rows they share come into the CU once. Workgroup w runs on
// XCD w % 8. A wave streams its head's 32-key tiles: the K registers of the next tile are refilled
// as soon as the scores are computed and the V registers as soon as P.V is done, also when the
// next tile starts the next piece, so one tile's loads are always in flight behind the
// arithmetic. Everything per key runs on the matrix cores; the vector ALUs only do the
// softmax and an in-register transpose.
//   * S^T = K Q^T (16x16x32 steps): A = 16 keys x 8 d-elements (128-bit loads of K rows),
//     B = the G query heads of the group as columns (columns >= G are zero). Lane (n, q) then
//     holds the scores of head n for keys 4q..4q+3 of each 16-key half: the lane's 8 keys of the
//     tile are key(q, e) = 16*(e/4) + 4q + e%4, e = 0..7.
//   * O^T = V^T P^T: the same 8 keys are the reduction slots, so P never leaves the lane. Output
//     row r of O^T tile t is d = VEC*r + t (VEC = d_head/16), which lets lane (n, q) fetch its V
//     operand as one 128-bit load per key (V[key][VEC*n .. VEC*n+VEC-1]); an 8 x VEC transpose of
//     16-bit values in registers (byte permutes) turns the 8 loaded rows into the VEC operands.
//   * P enters the bf16 step as a hi + lo pair (two steps), so the product keeps ~16 bits of P.
//   * O_lr^T = V_lr^T P^T on one more step: row n is column n of the agent's V_lr slice.
//   * fp32 inputs run the same loads on 16x16x4 fp32 steps (one key per slot, no transpose).
//   * keys past the piece's end are clamped to its last row (finite data) and get P = 0, so no row
//     outside [kv_start, kv_start+kv_len) is read
//   * each wave writes one fp32 partial (m, l, O, O_lr) per query head of its group and piece
//   * a second kernel, one workgroup per (request, KV head), merges the request's partials with
//     weights 2^(m_s - max m), applies O = (O + O_lr B_agent[:, g*d..]) / l once per query row and
//     rounds to the output type. Empty requests get zeros and requests with an invalid range or
//     agent NaN. The kernel boundary orders the partial writes before the merge: a device-scope
//     fence per workgroup (to let the last piece merge in place) writes back and invalidates an
//     XCD's L2, which cost more than the whole merge at thousands of workgroups.
// Small batches (few tiles in all) take a chunked launch instead, defined further down: one
// workgroup per (request, KV head, 128- or 256-key chunk), its tiles merged in LDS.
#include <algorithm>
#include <type_traits>

#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kCombineWaves = 8;
constexpr int kCombineThreads = 64 * kCombineWaves;
constexpr int kSplitWaves = 8;                 // split kernel: one wave per KV head of a group of 8
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kTile = 32;   // keys per wave tile

__device__ __forceinline__ bool decode_request_ok(int64_t start, int32_t len, int32_t a, const DecodeParams& p) {
    return len >= 0 && int64_t(len) <= p.max_kv_len && start >= 0 && start + int64_t(len) <= p.kv_rows &&
           a >= kAdapterFree && a < p.n_agents;
}

// key of the tile held by lane group q in slot e
__device__ __forceinline__ int tile_key(int q, int e) { return 16 * (e >> 2) + 4 * q + (e & 3); }

// One wave's loads of a 32-key tile: K (consumed by the scores) and V / V_lr (consumed by P.V) are
// fetched in two groups so each group's registers are refilled as soon as they have been used.
template <typename T, int D> struct DecodeTile {
    static constexpr int VEC = D / 16;
    static constexpr int KCH = D / 32;
    Vec<T, 8> k[2][KCH];   // K rows 16u + n, d = 32i + 8q .. +7
    Vec<T, VEC> v[8];      // V rows key(q, e), d = VEC*n .. +VEC-1
    Vec<T, 8> lr;          // V_lr[key(q, e)][agent*R + n % R] in slot e
    float4 ks[2];          // rank-r key scores (fp32) of head n, keys 16u + 4q .. +3 (LoRA on the keys)
};

// A operand of O^T tile t from the 8 loaded V rows: slot e <- v[e][t] (16-bit transpose).
template <int VEC>
__device__ __forceinline__ Vec<bf16, 8> v_operand(const Vec<bf16, VEC> (&v)[8], int t) {
    Vec<bf16, 8> a;
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) a.w[pp] = __builtin_amdgcn_perm(v[2 * pp + 1].w[t >> 1], v[2 * pp].w[t >> 1], sel);
    return a;
}

// Units of work: 32-key tiles. A request's units (0 when it is empty or invalid); the slices of the
// batch's units and the slice that owns a unit come from decode_schedule, the same integer formulas
// in both kernels, so the merge finds exactly the partials the split kernel wrote.
// The host bounds batch x tiles(max_kv_len) below 2^31, so unit counts are 32-bit.
template <bool PAGED>
__device__ __forceinline__ int request_units(const DecodeParams& p, int b) {
    const int64_t start = PAGED ? 0 : p.kv_start[b];
    const int32_t len = p.kv_len[b];
    return decode_request_ok(start, len, p.agent[b], p) ? (len + kTile - 1) / kTile : 0;
}

// Partial records. A piece of request b in slice k writes, per KV head g, one block of 16-byte
// slots at block (k + b) * n_kv + g (GP = the group size rounded up to 4 or 8; n < G, q < 4):
//   O:   slot c * 4GP + 4n + q, c < VEC  <- O^T of head n, d = VEC*(4q + c/(VEC/4)) + 4*(c%(VEC/4)) + 0..3
//   O_lr: slot VEC*4GP + n*(R/4) + q, q < R/4  <- O_lr of head n, ranks 4q .. 4q+3
//   m, l: slot VEC*4GP + GP*R/4 + n  <- (m, l, 0, 0) of head n
// padded to a multiple of 16 slots, so a wave's store instructions write contiguous runs of
// 16 * 4G bytes (measured on MI355X: faster than the strided stores of one record per head). The records are
// written and read with the device-coherent cache policy (sc1, the one the compiler uses for
// agent-scope atomic stores and loads): the stores write through this XCD's L2, and the merging
// wave's loads do not take a stale copy from its own. Measured on MI355X, these stores cost less
// than plain write-back ones, and no whole-L2 write-back or invalidate is needed.
template <int D, int R, int GP> struct RecordFormat {
    static constexpr int VEC = D / 16;
    static constexpr int O_SLOTS = VEC * 4 * GP;
    static constexpr int LR_SLOT = O_SLOTS;
    static constexpr int ML_SLOT = O_SLOTS + GP * R / 4;
    static constexpr int SLOTS = (ML_SLOT + GP + 15) / 16 * 16;   // blocks of whole 256-byte runs
    static constexpr int REGS = (SLOTS + 63) / 64;      // slots per lane in the merge
    static constexpr int LR_REG = O_SLOTS / 64;          // the register holding the O_lr and (m, l) slots
    static_assert(O_SLOTS % 64 == 0 || O_SLOTS < 64, "O slots fill whole registers");
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCoherent = 16;   // sc1: device-coherent cache policy of a buffer access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, int(bytes), 0x00020000);
}
__device__ __forceinline__ void record_store(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<u32x4_t*>(&v), rs, off, 0, kCoherent);
}
__device__ __forceinline__ f32x4 record_load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherent);
    return *reinterpret_cast<const f32x4*>(&v);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// Decode step: workgroup i of the first n_pre forms the LR rows of the newest tokens of requests
// 2i and 2i+1 (PReCache paper page, PreLRShared: every agent's columns of a new token's row, from its
// hidden state). Wave w takes d_model elements [w*d_model/8, (w+1)*d_model/8); lane c takes column
// c0 + c of the stacked A (one 16-byte run per 8 elements; X rows are broadcast loads). The eight
// wave sums are added in wave order through LDS (deterministic) and rounded once to the cache type.
template <typename T>
__device__ void newest_lr_rows(const DecodeParams& p, int i, float (*red)[2][64]) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int NR = p.n_agents * p.rank;
    const int ks = p.d_model / kSplitWaves;
    int64_t row[2];
    bool live[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int b = 2 * i + h;
        live[h] = false;
        row[h] = 0;
        if (b < p.batch) {
            const int64_t start = p.kv_start[b];
            const int32_t len = p.kv_len[b];
            live[h] = len > 0 && decode_request_ok(start, len, p.agent[b], p);
            row[h] = start + len - 1;
        }
    }
    const T* __restrict__ X0 = static_cast<const T*>(p.X_new) + int64_t(min(2 * i, p.batch - 1)) * p.ldx;
    const T* __restrict__ X1 = static_cast<const T*>(p.X_new) + int64_t(min(2 * i + 1, p.batch - 1)) * p.ldx;
    for (int c0 = 0; c0 < NR; c0 += 64) {
        const int c = min(c0 + lane, NR - 1);
        const T* __restrict__ Ac = static_cast<const T*>(p.A_new) + int64_t(c) * p.d_model;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 4
        for (int k = wv * ks; k < (wv + 1) * ks; k += 8) {
            Vec<T, 8> av, x0, x1;
            av.load(Ac + k);
            x0.load(X0 + k);
            x1.load(X1 + k);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc0 = fmaf(av.get(e), x0.get(e), acc0);
                acc1 = fmaf(av.get(e), x1.get(e), acc1);
            }
        }
        red[wv][0][lane] = acc0;
        red[wv][1][lane] = acc1;
        __syncthreads();
        if (threadIdx.x < 128) {
            const int h = threadIdx.x >> 6, cc = c0 + (threadIdx.x & 63);
            if (cc < NR && live[h]) {
                float v = 0.f;
#pragma unroll
                for (int ww = 0; ww < kSplitWaves; ++ww) v += red[ww][h][threadIdx.x & 63];
                const int ka = cc / p.rank;   // agent of column cc
                static_cast<T*>(const_cast<void*>(p.Vlr))[row[h] * p.ld_vlr + ka * p.vlr_agent_stride + (cc - ka * p.rank)] = from_f32<T>(v);
            }
        }
        __syncthreads();
    }
}

template <typename T, int D, int R, int GP, bool PAGED, bool KSC>
__global__ __launch_bounds__(kSplitThreads, 2) void decode_split_kernel(DecodeParams p) {
    using Tile = DecodeTile<T, D>;
    constexpr int VEC = Tile::VEC, KCH = Tile::KCH;
    static_assert(R <= 16 && GP <= 16, "one 16-wide matrix-core tile covers the rank and the group");

    // decode step: the first n_pre workgroups form the newest LR rows (n_pre is a multiple of 8,
    // so the XCD of every slot's workgroup stays w % 8)
    int w = blockIdx.x;
    if constexpr (!PAGED && !KSC) {
        if (p.X_new) {
            __shared__ float red[kSplitWaves][2][64];
            if (w < p.n_pre) {
                newest_lr_rows<T>(p, w, red);
                return;
            }
            w -= p.n_pre;
        }
    }
    // workgroup w = (slot, group hg of 8 KV heads); wave wv takes KV head g. Workgroup w runs on
    // XCD w % 8, and the head groups of one slot get the same w % 8.
    const int xcd = w & 7;
    const int rest = w >> 3;
    const int n_hg = (p.n_kv + kSplitWaves - 1) / kSplitWaves;
    const int slot = (rest / n_hg) * 8 + xcd;
    const int hg = rest % n_hg;
    if (slot >= p.n_slots) return;   // the whole workgroup
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // a wave past the last KV head (n_kv not a multiple of 8) follows its workgroup through the
    // same tiles on head n_kv - 1, so that it meets the same barriers, and stores nothing
    const bool live = hg * kSplitWaves + wv < p.n_kv;
    const int g = min(hg * kSplitWaves + wv, p.n_kv - 1);
    const int lane = threadIdx.x & 63;
    const int G = p.G;

    // ---- the request table, 64 requests at a time: lane l holds request wb + l's range, agent and
    // units, and the units' inclusive prefix sum in the window; wP = units before request wb. Every
    // wave reads it; pieces then take their request's entries by readlane, with no memory access.
    int wb = 0, wP = 0;
    int64_t w_start = 0;
    int w_len = 0, w_agent = 0, w_ub = 0, w_incl = 0;
    auto load_window = [&]() {
        const int bb = wb + lane;
        w_start = 0;
        w_len = w_agent = w_ub = 0;
        if (bb < p.batch) {
            w_start = PAGED ? 0 : p.kv_start[bb];
            w_len = p.kv_len[bb];
            w_agent = p.agent[bb];
            w_ub = decode_request_ok(w_start, w_len, w_agent, p) ? (w_len + kTile - 1) / kTile : 0;
        }
        // consumed here, so that no later read of the window waits for the loads (a piece's
        // request always has units)
        w_start = w_ub > 0 ? w_start : 0;
        w_len = w_ub > 0 ? w_len : 0;
        w_agent = w_ub > 0 ? w_agent : 0;
        w_incl = wave_incl_scan(w_ub, lane);
    };
    load_window();
    int U = __builtin_amdgcn_readlane(w_incl, 63);
    for (int c0 = 64; c0 < p.batch; c0 += 64) {
        const int bb = c0 + lane;
        U += wave_sum(bb < p.batch ? request_units<PAGED>(p, bb) : 0);
    }
    U = __builtin_amdgcn_readfirstlane(U);
    const int n_act = decode_slices(U, p.n_slots);
    if (slot >= n_act) return;   // the whole workgroup (U is the same in every wave)
    const int s0 = slice_begin(U, slot, n_act), s1 = slice_begin(U, slot + 1, n_act);   // this slice's units

    // ---- pieces: the part of one request's units in the slice
    struct Piece {
        int b;          // request
        int u0, pe;     // units [u0, pe) of the batch
        int k0, k1;     // keys [k0, k1) of the request
        int len, a;
        int64_t start;
    };
    // the piece that starts at unit u (s0 <= u < s1)
    auto piece_at = [&](int u, Piece& pc) {
        int l = 0;
        for (;;) {   // the request holding u, never before the window: units only increase
            const uint64_t past = __ballot(wb + lane < p.batch && wP + w_incl > u);
            if (past) {
                l = __builtin_ctzll(past);
                break;
            }
            if (wb + 64 >= p.batch) {   // not reached (u < U); ends the search on a valid request
                l = p.batch - 1 - wb;
                break;
            }
            wP += __builtin_amdgcn_readlane(w_incl, 63);
            wb += 64;
            load_window();
        }
        const int ub = __builtin_amdgcn_readlane(w_ub, l);
        const int Pb = wP + __builtin_amdgcn_readlane(w_incl, l) - ub;   // units before the request
        pc.b = wb + l;
        pc.u0 = u;
        pc.pe = min(Pb + ub, s1);
        pc.start = PAGED ? 0 : int64_t(__builtin_amdgcn_readlane(int(uint64_t(w_start) >> 32), l)) << 32 |
                                   uint32_t(__builtin_amdgcn_readlane(int(w_start), l));
        pc.len = __builtin_amdgcn_readlane(w_len, l);
        pc.a = __builtin_amdgcn_readlane(w_agent, l);
        pc.k0 = (u - Pb) * kTile;
        pc.k1 = min((pc.pe - Pb) * kTile, pc.len);
    };

    const int n = lane & 15;   // key row of K, head column of Q^T / P^T, O^T row
    const int q = lane >> 4;   // reduction slot group
    const int64_t row_bytes = p.kv_row_stride * int64_t(sizeof(T));
    const int64_t lr_bytes = p.ld_vlr * int64_t(sizeof(T));
    const int64_t head_bytes = int64_t(g) * p.kv_head_stride * int64_t(sizeof(T));
    const float sl2 = p.scale * kLog2e;

    // Paged cache: each wave keeps the page ids of 64 consecutive blocks of one request, one per
    // lane, and reloads that window when a tile moves past it or to another request; a tile never
    // crosses a page (P is a power of two >= 32 and tiles are 32-aligned), so its page is one
    // readlane away. Out-of-range page ids read page 0 instead and poison the piece with NaN.
    int page_vec = 0, pg_base = 0, pg_req = -1;
    bool pg_bad = false;
    auto page_of = [&](const Piece& pc, int kt, bool& bad) -> int {
        const int blk = kt >> p.page_shift;   // wave-uniform
        if (pc.b != pg_req || blk - pg_base >= 64 || blk < pg_base) {
            pg_req = pc.b;
            pg_base = blk;
            const int n_blk = ((pc.len - 1) >> p.page_shift) + 1;
            int id = 0;
            if (pg_base + lane < n_blk) id = p.block_table[int64_t(pc.b) * p.max_blocks + pg_base + lane];
            const bool lane_bad = pg_base + lane < n_blk && (id < 0 || int64_t(id) >= p.n_pages);
            pg_bad = __ballot(lane_bad) != 0;
            page_vec = lane_bad ? 0 : id;
        }
        bad = bad || pg_bad;
        return __builtin_amdgcn_readlane(page_vec, blk - pg_base);
    };
    // first cache row of the 32-key tile starting at key kt of the piece's request (V_lr rows), and
    // the byte offset of that row from the request's first row in K / V (a page's rows are
    // adjacent; pages sit kv_page_stride elements apart)
    auto tile_row = [&](const Piece& pc, int kt, bool& bad) -> int64_t {
        if constexpr (PAGED) return (int64_t(page_of(pc, kt, bad)) << p.page_shift) + (kt & ((1 << p.page_shift) - 1));
        else return kt;
    };
    auto tile_kv_off = [&](const Piece& pc, int kt, bool& bad) -> int64_t {
        if constexpr (PAGED) {
            return int64_t(page_of(pc, kt, bad)) * p.kv_page_stride * int64_t(sizeof(T)) +
                   int64_t(kt & ((1 << p.page_shift) - 1)) * row_bytes;
        } else {
            return int64_t(kt) * row_bytes;
        }
    };

    // Addresses: a wave-uniform base per tile and slot (scalar registers) plus one 32-bit lane
    // offset per operand, so the loads use the scalar-base + vector-offset form. An adapter-free
    // request streams agent 0's columns of V_lr (same rows, valid memory) through the same
    // instructions; the merge drops that product.
    const uint32_t k_lane = uint32_t(n * row_bytes + 8 * q * sizeof(T));
    const uint32_t v_lane = uint32_t(4 * q * row_bytes + VEC * n * sizeof(T));
    const uint32_t l_lane = uint32_t(4 * q * lr_bytes + (n % R) * sizeof(T));
    auto kv_base = [&](const void* X, const Piece& pc) -> const char* {
        return static_cast<const char*>(X) + pc.start * row_bytes + head_bytes;
    };
    auto lr_base = [&](const Piece& pc) -> const char* {
        return static_cast<const char*>(p.Vlr) + (pc.start * p.ld_vlr + int64_t(max(pc.a, 0)) * p.vlr_agent_stride) * int64_t(sizeof(T));
    };

    // the group's queries as the B operand (columns >= G are zero)
    const T* __restrict__ Qp = static_cast<const T*>(p.Q);
    Vec<T, 8> qf[KCH];
    auto load_q = [&](const Piece& pc) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            if (n < G) qf[i].load(Qp + (int64_t(pc.b) * p.n_q + int64_t(g) * G + n) * D + 32 * i + 8 * q);
            else qf[i].zero();
        }
    };

    // LoRA on the keys: the rank-r part of the scores, Q . RoPE(K_lr B_k), comes from the key
    // score pass as fp32 [request][query head][key]; lane (n, q) adds keys 16u + 4q .. +3 of head
    // n (a wave-uniform base per request and KV head plus one 32-bit lane offset)
    bool ks_live = false;
    const char* __restrict__ ksg = nullptr;
    const uint32_t ks_lane = uint32_t((min(n, G - 1) * p.ks_stride + 4 * q) * 4);
    auto load_ks = [&](Tile& t, int kt) {
        if constexpr (KSC) {
            if (ks_live) {   // request-uniform; rows are padded to whole 64-key blocks
                t.ks[0] = *reinterpret_cast<const float4*>(ksg + ks_lane + 4 * kt);
                t.ks[1] = *reinterpret_cast<const float4*>(ksg + ks_lane + 4 * (kt + 16));
            } else {
                t.ks[0] = t.ks[1] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };
    // Tile loads of the tile at key kt of a piece. A full tile addresses each operand as a
    // wave-uniform base plus one 32-bit lane offset. Only a piece's last tile can run past k1: its
    // rows are clamped to k1 - 1 (finite data; those keys get P = 0). Both forms issue the same
    // loads into the same registers, so the choice is a uniform branch around address arithmetic.
    auto load_k = [&](Tile& t, const Piece& pc, int kt, bool& bad) {
        const char* kb = kv_base(p.K, pc) + tile_kv_off(pc, kt, bad);
        if (kt + kTile <= pc.k1) {
#pragma unroll
            for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                for (int i = 0; i < KCH; ++i)
                    t.k[uu][i].load(reinterpret_cast<const T*>(kb + 16 * uu * row_bytes + k_lane) + 32 * i);
        } else {
            const int lim = pc.k1 - 1 - kt;
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
                const uint32_t o = uint32_t(min(16 * uu + n, lim) * row_bytes + 8 * q * sizeof(T));
#pragma unroll
                for (int i = 0; i < KCH; ++i) t.k[uu][i].load(reinterpret_cast<const T*>(kb + o) + 32 * i);
            }
        }
    };
    auto load_v = [&](Tile& t, const Piece& pc, int kt, bool& bad) {
        const char* vb = kv_base(p.V, pc) + tile_kv_off(pc, kt, bad);
        const char* lb = lr_base(pc) + tile_row(pc, kt, bad) * lr_bytes;
        // every lane loads V_lr (lanes n >= R repeat a column; their O_lr^T rows are never used),
        // so no load sits behind a lane mask
        uint32_t h[8];
        if (kt + kTile <= pc.k1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                t.v[e].load(reinterpret_cast<const T*>(vb + tile_key(0, e) * row_bytes + v_lane));
                if constexpr (sizeof(T) == 2) h[e] = *reinterpret_cast<const uint16_t*>(lb + tile_key(0, e) * lr_bytes + l_lane);
                else t.lr.v[e] = *reinterpret_cast<const float*>(lb + tile_key(0, e) * lr_bytes + l_lane);
            }
        } else {
            const int lim = pc.k1 - 1 - kt;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = min(tile_key(q, e), lim);
                t.v[e].load(reinterpret_cast<const T*>(vb + uint32_t(key * row_bytes + VEC * n * sizeof(T))));
                const uint32_t lo = uint32_t(key * lr_bytes + (n % R) * sizeof(T));
                if constexpr (sizeof(T) == 2) h[e] = *reinterpret_cast<const uint16_t*>(lb + lo);
                else t.lr.v[e] = *reinterpret_cast<const float*>(lb + lo);
            }
        }
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) t.lr.w[qq] = h[2 * qq] | (h[2 * qq + 1] << 16);
        }
    };

    f32x4 acc[VEC];
    f32x4 acc_lr;
    float m_run, l_run, s_new;

    // One tile of piece pc at key kt: scores, online softmax, P.V. With pf, the tile's registers
    // are refilled with tile nkt of piece np (the next tile of pc, or the first tile of the next
    // piece, whose queries are then loaded too: new_q) as soon as they have been read: K after the
    // scores, V after P.V, so one tile's loads are always in flight behind the arithmetic, also
    // across pieces and slices. Returns whether a page id of those loads was out of range.
    auto tile_step = [&](Tile& t, const Piece& pc, int kt, bool pf, const Piece& np, int nkt, bool new_q) -> bool {
        bool nbad = false;
        // the key scores are loaded here, not a tile ahead: prefetched, they overflow the registers
        load_ks(t, kt);
        f32x4 sacc[2];
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            sacc[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KCH; ++i) sacc[uu] = mma16x16x32(t.k[uu][i], qf[i], sacc[uu]);
        }
        if constexpr (KSC) {
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
                sacc[uu][0] += t.ks[uu].x;
                sacc[uu][1] += t.ks[uu].y;
                sacc[uu][2] += t.ks[uu].z;
                sacc[uu][3] += t.ks[uu].w;
            }
        }
        if (pf) load_k(t, np, nkt, nbad);
        if (new_q) load_q(np);
        float sc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[e] = sacc[e >> 2][e & 3] * sl2;
        if (kt + kTile > pc.k1) {   // a partial last tile
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (kt + tile_key(q, e) >= pc.k1) sc[e] = -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // online softmax (base 2); key kt is live, so mnew is finite
        const float mnew = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - mnew);
        m_run = mnew;
        float pr[8], ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pr[e] = fast_exp2(sc[e] - mnew);
            ls += pr[e];
        }
        l_run = fmaf(l_run, alpha, ls);
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int tt = 0; tt < VEC; ++tt) acc[tt] *= alpha;
            acc_lr *= alpha;
        }
        // decode step: the piece holding the request's newest key, whose LR row is formed in this
        // launch, leaves that key out of O_lr and records its score
        const bool has_new = !PAGED && !KSC && p.X_new != nullptr && pc.k1 == pc.len;
        if (has_new && kt + kTile >= pc.len) {   // the newest key (len - 1) is in this tile
            const int kk = pc.len - 1 - kt;
            const int qk = (kk & 15) >> 2, ek = 4 * (kk >> 4) + (kk & 3);
            float v = sc[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) v = e == ek ? sc[e] : v;
            s_new = __shfl(v, n + 16 * qk);
            // its V_lr entries (and those of the clamped keys past it, which have P = 0) drop out
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (kt + tile_key(q, e) >= pc.len - 1) {
                    if constexpr (sizeof(T) == 2) t.lr.w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                    else t.lr.v[e] = 0.f;
                }
            }
        }
        // O^T += V^T P^T, O_lr^T += V_lr^T P^T
        if constexpr (sizeof(T) == 2) {
            Vec<bf16, 8> phi, plo;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                phi.w[qq] = pack_bf16x2(pr[2 * qq], pr[2 * qq + 1]);
                plo.w[qq] = pack_bf16x2(pr[2 * qq] - bf16_lo(phi.w[qq]), pr[2 * qq + 1] - bf16_hi(phi.w[qq]));
            }
#pragma unroll
            for (int tt = 0; tt < VEC; ++tt) {
                const Vec<bf16, 8> va = v_operand<VEC>(t.v, tt);
                acc[tt] = mma16x16x32(va, phi, acc[tt]);
                acc[tt] = mma16x16x32(va, plo, acc[tt]);
            }
            acc_lr = mma16x16x32(t.lr, phi, acc_lr);
            acc_lr = mma16x16x32(t.lr, plo, acc_lr);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
#pragma unroll
                for (int tt = 0; tt < VEC; ++tt)
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[e].v[tt], pr[e], acc[tt], 0, 0, 0);
                acc_lr = __builtin_amdgcn_mfma_f32_16x16x4f32(t.lr.v[e], pr[e], acc_lr, 0, 0, 0);
            }
        }
        if (pf) load_v(t, np, nkt, nbad);
        return nbad;
    };

    // ---- the piece's record block (lanes n < G; see RecordFormat): lane (n, q) holds O^T rows
    // 4q+j of each tile tt, i.e. d = VEC*(4q+j) + tt, and O_lr rows 4q .. 4q+3
    using F = RecordFormat<D, R, GP>;
    const __amdgpu_buffer_rsrc_t rs = record_rsrc(p.records, p.record_bytes);
    auto write_record = [&](const Piece& pc, bool bad) {
        const uint32_t blk = uint32_t((int64_t(slot) + pc.b) * p.n_kv + g) * (F::SLOTS * 16);
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        if (n < G) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int tt = 0; tt < VEC; tt += 4) {
                    const int c = j * (VEC / 4) + tt / 4;
                    record_store(rs, blk + (c * 4 * GP + 4 * n + q) * 16, f32x4{acc[tt][j], acc[tt + 1][j], acc[tt + 2][j], acc[tt + 3][j]});
                }
            if (4 * q < R) record_store(rs, blk + (F::LR_SLOT + n * (R / 4) + q) * 16, acc_lr);
            if (q == 0)
                record_store(rs, blk + (F::ML_SLOT + n) * 16,
                             f32x4{bad ? __builtin_nanf("") : m_run, l_run, s_new, 0.f});
        }
    };

    // ---- the slice's pieces, each tile prefetched during the one before it
    Piece cur{}, nxt{};
    piece_at(s0, cur);
    bool cur_bad = false, nxt_bad = false;
    Tile t;
    load_q(cur);
    load_k(t, cur, cur.k0, cur_bad);
    load_v(t, cur, cur.k0, cur_bad);
    for (;;) {   // workgroup-uniform
        const bool has_nxt = cur.pe < s1;
        if (has_nxt) piece_at(cur.pe, nxt);
        if constexpr (KSC) {
            ks_live = cur.a != kAdapterFree;
            ksg = reinterpret_cast<const char*>(p.key_scores + (int64_t(cur.b) * p.n_q + int64_t(g) * G) * p.ks_stride);
        }
#pragma unroll
        for (int tt = 0; tt < VEC; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_lr = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        s_new = -INFINITY;
        // the piece's tiles kt = k0 + 32 j, j < nt (at least one); only the last one can be partial
        const int nt = (cur.k1 - cur.k0 + kTile - 1) / kTile;
        int kt = cur.k0;
        for (int j = 0; j < nt; ++j, kt += kTile) {
            // one instance of the tile code: the next tile's piece is picked by scalar selects
            const bool more = j + 1 < nt;
            const Piece np = more ? cur : nxt;
            const bool pb = tile_step(t, cur, kt, more || has_nxt, np, more ? kt + kTile : nxt.k0, !more && has_nxt);
            if (more) cur_bad = cur_bad || pb;
            else nxt_bad = nxt_bad || pb;
        }
        if (live) write_record(cur, cur_bad);
        if (!has_nxt) break;
        cur = nxt;
        cur_bad = nxt_bad;
        nxt_bad = false;
    }
}

// Merge of the pieces of one (request b, KV head g), one 8-wave workgroup each: the request's units
// [P_b, P_b + units) lie in slices kf = slice_owner(P_b) .. slice_owner(P_b + units - 1), which
// wrote record blocks (kk + b) * n_kv + g. Wave w takes the pieces w, w+8, ...; lane L takes slots
// L + 64t of each block (RecordFormat: its O slots all belong to head n = (L % 4GP) / 4, and lanes
// L < GP*R/4 hold the O_lr slots of head L / (R/4) in register LR_REG). Every slot keeps its own
// running maximum and sum (the log-sum-exp rule with weights 2^(m_s - max m)); the slots of one head
// see the same (m, l) sequence, so they agree. A wave issues the loads of up to 8 pieces at once;
// the eight wave states are merged in LDS. Wave 0 then applies the up-projection
// O = (O + O_lr B_agent[:, g*d .. g*d+d-1]) / l (O / l for an adapter-free request), rounded to the
// output type; NaN when a piece had a bad page id. Requests without a key get zeros, invalid
// requests NaN.
template <typename T, int D, int R, int GP, bool PAGED>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeParams p) {
    using F = RecordFormat<D, R, GP>;
    constexpr int VEC = F::VEC;
    constexpr int NO = F::LR_REG;   // registers of O slots
    constexpr int PB = 8;           // pieces per batch of loads of a wave
    __shared__ f32x4 st_acc[kCombineWaves][NO + 1][64];
    __shared__ float st_m[kCombineWaves][2][64], st_l[kCombineWaves][64];
    __shared__ int st_bad[kCombineWaves];
    __shared__ int red_u[2][kCombineWaves];
    const int b = blockIdx.x / p.n_kv;
    const int g = blockIdx.x - b * p.n_kv;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // the request's range and agent, and the units of the requests before b and of the whole batch,
    // read in one round
    const int64_t start = PAGED ? 0 : p.kv_start[b];
    const int32_t len = p.kv_len[b];
    const int32_t a = p.agent[b];
    // units of the requests before b and of the batch
    int before = 0, total = 0;
    for (int bb = threadIdx.x; bb < p.batch; bb += kCombineThreads) {
        const int ub = request_units<PAGED>(p, bb);
        total += ub;
        if (bb < b) before += ub;
    }
    const bool ok = decode_request_ok(start, len, a, p);
    if (!ok || len == 0) {
        const T fill = from_f32<T>(ok ? 0.f : __builtin_nanf(""));
        T* Op = static_cast<T*>(p.O) + (int64_t(b) * p.n_q + int64_t(g) * p.G) * D;
        for (int i = threadIdx.x; i < p.G * D; i += kCombineThreads) Op[i] = fill;
        return;
    }
    // wave 0 fetches its B values now, while the partials are read: B[rr][g*d + d0 .. d0+3] of
    // each of its O slots (see below)
    const int64_t d_kv = int64_t(p.n_kv) * D;
    const bool adapted = a != kAdapterFree;
    const int q = lane & 3;
    Vec<T, 4> bv[NO][R];
    // decode step: the newest key's V_lr entries (ranks 4(L % (R/4)) .. +3 of the agent, for lanes
    // holding O_lr slots), formed by the split launch; its recorded score follows the merge
    Vec<T, 4> vnew;
    vnew.zero();
    const bool step_new = !PAGED && p.X_new != nullptr && adapted;
    if (wv == 0 && step_new)
        vnew.load(static_cast<const T*>(p.Vlr) + (start + len - 1) * p.ld_vlr + int64_t(a) * p.vlr_agent_stride + 4 * (lane % (R / 4)));
    if (wv == 0 && adapted) {
        const T* __restrict__ Bp = static_cast<const T*>(p.B) + int64_t(a) * R * d_kv + int64_t(g) * D;
#pragma unroll
        for (int t = 0; t < NO; ++t) {
            const int c = (64 * t + lane) / (4 * GP);
            const int d0 = VEC * (4 * q + c / (VEC / 4)) + 4 * (c % (VEC / 4));
#pragma unroll
            for (int rr = 0; rr < R; ++rr) bv[t][rr].load(Bp + int64_t(rr) * d_kv + d0);
        }
    }
    before = wave_sum(before);
    total = wave_sum(total);
    if (lane == 0) {
        red_u[0][wv] = before;
        red_u[1][wv] = total;
    }
    __syncthreads();
    int Pb = 0, U = 0;
#pragma unroll
    for (int v = 0; v < kCombineWaves; ++v) {
        Pb += red_u[0][v];
        U += red_u[1][v];
    }
    // the request's pieces: slices kf .. kf + n_pieces - 1, piece i in record block kf + i + b
    const int n_act = decode_slices(U, p.n_slots);
    const int kf = slice_owner(U, Pb, n_act);
    const int n_pieces = slice_owner(U, Pb + (len + kTile - 1) / kTile - 1, n_act) - kf + 1;
    auto piece_block = [&](int i) -> int64_t { return int64_t(kf) + i + b; };

    const __amdgpu_buffer_rsrc_t rs = record_rsrc(p.records, p.record_bytes);
    const int n_o = (lane % (4 * GP)) / 4;
    const int n_lr = min(lane / (R / 4), GP - 1);
    const uint32_t block = F::SLOTS * 16;
    // decode step: the newest key's recorded score, from the last piece, read beside the partials
    float s_new = -INFINITY;
    if (wv == 0 && step_new) {
        const uint32_t last = uint32_t(piece_block(n_pieces - 1) * p.n_kv + g) * (F::SLOTS * 16);
        s_new = record_load(rs, last + (F::ML_SLOT + n_lr) * 16)[2];
    }
    float M = -INFINITY, L = 0.f, M2 = -INFINITY;
    bool bad = false;
    f32x4 acc[NO + 1];
#pragma unroll
    for (int t = 0; t <= NO; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = wv; i0 < n_pieces; i0 += PB * kCombineWaves) {
        f32x4 v[PB][NO + 1], ml[PB], ml2[PB];
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int i = min(i0 + u * kCombineWaves, n_pieces - 1);
            const uint32_t base = uint32_t(piece_block(i) * p.n_kv + g) * block;
#pragma unroll
            for (int t = 0; t <= NO; ++t) v[u][t] = record_load(rs, base + (64 * t + lane) * 16);
            ml[u] = record_load(rs, base + (F::ML_SLOT + n_o) * 16);
            ml2[u] = record_load(rs, base + (F::ML_SLOT + n_lr) * 16);
        }
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            if (i0 + u * kCombineWaves >= n_pieces) break;
            bad = bad || ml[u][0] != ml[u][0];
            const float mn = fmaxf(M, ml[u][0]), mn2 = fmaxf(M2, ml2[u][0]);
            const float keep = fast_exp2(M - mn), w = fast_exp2(ml[u][0] - mn);
            const float keep2 = fast_exp2(M2 - mn2), w2 = fast_exp2(ml2[u][0] - mn2);
            L = fmaf(L, keep, w * ml[u][1]);
#pragma unroll
            for (int t = 0; t < NO; ++t) acc[t] = acc[t] * keep + v[u][t] * w;
            acc[NO] = acc[NO] * keep2 + v[u][NO] * w2;
            M = mn;
            M2 = mn2;
        }
    }
    // the eight wave states (a wave without pieces has M = -inf and weight 0)
#pragma unroll
    for (int t = 0; t <= NO; ++t) st_acc[wv][t][lane] = acc[t];
    st_m[wv][0][lane] = M;
    st_m[wv][1][lane] = M2;
    st_l[wv][lane] = L;
    const uint64_t any_bad = __ballot(bad);
    if (lane == 0) st_bad[wv] = any_bad != 0;
    __syncthreads();
    if (wv != 0) return;
    float Ms = -INFINITY, Ms2 = -INFINITY;
    bad = false;
#pragma unroll
    for (int w = 0; w < kCombineWaves; ++w) {
        Ms = fmaxf(Ms, st_m[w][0][lane]);
        Ms2 = fmaxf(Ms2, st_m[w][1][lane]);
        bad = bad || st_bad[w];
    }
    L = 0.f;
#pragma unroll
    for (int t = 0; t <= NO; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kCombineWaves; ++w) {
        const float e = fast_exp2(st_m[w][0][lane] - Ms), e2 = fast_exp2(st_m[w][1][lane] - Ms2);
        L = fmaf(e, st_l[w][lane], L);
#pragma unroll
        for (int t = 0; t < NO; ++t) acc[t] += st_acc[w][t][lane] * e;
        acc[NO] += st_acc[w][NO][lane] * e2;
    }
    if (step_new) {
        // the newest key's LR term: weight 2^(s_new - M) against the merged maximum of the head
        const float w_new = fast_exp2(s_new - Ms2);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[NO][e] = fmaf(w_new, vnew.get(e), acc[NO][e]);
    }
    // O_lr column rr of head n_o: lane n_o*(R/4) + rr/4, component rr%4 of register LR_REG
    float lr[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) lr[rr] = __shfl(acc[NO][rr & 3], n_o * (R / 4) + (rr >> 2));
    const float inv = bad ? __builtin_nanf("") : 1.f / L;
#pragma unroll
    for (int t = 0; t < NO; ++t) {
        const int c = (64 * t + lane) / (4 * GP);
        const int d0 = VEC * (4 * q + c / (VEC / 4)) + 4 * (c % (VEC / 4));
        f32x4 o = acc[t];
        if (adapted) {
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = fmaf(lr[rr], bv[t][rr].get(e), o[e]);
        }
        if (n_o < p.G) {
            T* dst = static_cast<T*>(p.O) + (int64_t(b) * p.n_q + int64_t(g) * p.G + n_o) * D + d0;
            if constexpr (sizeof(T) == 2)
                *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
            else
                *reinterpret_cast<float4*>(dst) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
        }
    }
}

// ---- small batches ---------------------------------------------------------------------------
// When the batch holds few tiles, the split launch above gives each of its slots a tile or two of
// eight heads, and the merge reads one record per 32-key tile and head. Here workgroup (b, g, c)
// instead takes chunk c (32*CW keys) of request b on KV head g, wave w its 32-key tile w, with the same matrix-core tile as the split kernel (one tile per wave: its softmax maximum is
// the tile's). The wave partials are merged in LDS with weights 2^(m_w - max m), so a chunk leaves
// one record; a request of one chunk is finished in the same launch, otherwise a second launch
// merges its chunk records the same way and applies the up-projection. Both kernels issue every
// load that does not need the request's range before that range arrives (the queries, the
// records, the B values of every agent when there are few), so each is about one memory round
// trip more than its launch.
template <int D, int GP, int CW> struct SmallRecord {
    static constexpr int VEC = D / 16;
    static constexpr int ENT = VEC + 1;      // fragments per lane: the O^T tiles, then O_lr^T
    static constexpr int FR = 4 * GP;        // lanes (n, q) with n < GP, at index q * GP + n
    static constexpr int ML = ENT * FR;      // then m[GP], l[GP] as floats
    static constexpr int SLOTS = ML + (2 * GP + 3) / 4;
    static constexpr int FPT = (ENT * FR + 64 * CW - 1) / (64 * CW);   // fragments per thread
};

// merged state of one (request, KV head) in LDS: O[n][d], O_lr[n][r] (unnormalised) and l[n]
template <int D, int R, int GP> struct SmallOut {
    float o[GP][D];
    float lr[GP][R];
    float l[GP];
};

// fragment tt of lane index i = q * GP + n (n < GP) into the LDS state: O^T tile tt, lane (n, q),
// register j is O[n][VEC*(4q + j) + tt]; the O_lr^T fragment (tt = VEC) register j is O_lr[n][4q + j]
template <int D, int R, int GP>
__device__ __forceinline__ void small_put(SmallOut<D, R, GP>& so, int tt, int i, f32x4 v) {
    constexpr int VEC = D / 16;
    const int n = i % GP, q = i / GP;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (tt < VEC) so.o[n][VEC * (4 * q + j) + tt] = v[j];
        else if (4 * q + j < R) so.lr[n][4 * q + j] = v[j];
    }
}

// The epilogue thread i < G*D/4 takes 4 consecutive elements d0 .. d0+3 of head n = i / (D/4) and
// needs B_a[r][g*D + d0 .. +3], r < R. With at most kSpecAgents agents (bf16) every agent's values
// are loaded before the request's agent is known; otherwise they are loaded once it is.
template <typename T, int D, int R> struct SmallB {
    static constexpr int kSpecAgents = sizeof(T) == 2 ? 4 : 0;
    Vec<T, 4> bs[kSpecAgents > 0 ? kSpecAgents : 1][R];
    __device__ __forceinline__ const T* at(const DecodeParams& p, int g, int a, int d0) const {
        const int64_t d_kv = int64_t(p.n_kv) * D;
        return static_cast<const T*>(p.B) + int64_t(a) * R * d_kv + int64_t(g) * D + d0;
    }
    __device__ __forceinline__ void prefetch(const DecodeParams& p, int g) {
        if constexpr (kSpecAgents > 0) {
            const int i = threadIdx.x;
            if (p.n_agents > kSpecAgents || i >= p.G * (D / 4)) return;
            const int d0 = 4 * (i % (D / 4));
            const int64_t d_kv = int64_t(p.n_kv) * D;
#pragma unroll
            for (int k = 0; k < kSpecAgents; ++k)
                if (k < p.n_agents) {
                    const T* Bp = at(p, g, k, d0);
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) bs[k][rr].load(Bp + rr * d_kv);
                }
        }
    }
    // agent a's values (a >= 0)
    __device__ __forceinline__ void get(const DecodeParams& p, int g, int a, int d0, Vec<T, 4> (&bv)[R]) const {
        if (kSpecAgents > 0 && p.n_agents <= kSpecAgents) {
#pragma unroll
            for (int rr = 0; rr < R; ++rr) bv[rr] = bs[0][rr];
#pragma unroll
            for (int k = 1; k < (kSpecAgents > 0 ? kSpecAgents : 1); ++k)
                if (a == k) {
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) bv[rr] = bs[k][rr];
                }
        } else {
            const int64_t d_kv = int64_t(p.n_kv) * D;
            const T* Bp = at(p, g, a, d0);
#pragma unroll
            for (int rr = 0; rr < R; ++rr) bv[rr].load(Bp + rr * d_kv);
        }
    }
};

// O rows of (b, g) from the LDS state: (O + O_lr B_a[:, g*d .. g*d + d)) / l, rounded to T
template <typename T, int D, int R, int GP>
__device__ __forceinline__ void small_epilogue(const DecodeParams& p, int b, int g, int a, const SmallOut<D, R, GP>& so,
                                               const SmallB<T, D, R>& sb) {
    const int i = threadIdx.x;
    if (i >= p.G * (D / 4)) return;
    const int n = i / (D / 4), d0 = 4 * (i % (D / 4));
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = so.o[n][d0 + e];
    if (a != kAdapterFree) {
        Vec<T, 4> bv[R];
        sb.get(p, g, a, d0, bv);
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = fmaf(so.lr[n][rr], bv[rr].get(e), o[e]);
    }
    const float inv = 1.f / so.l[n];
    T* dst = static_cast<T*>(p.O) + (int64_t(b) * p.n_q + int64_t(g) * p.G + n) * D + d0;
    if constexpr (sizeof(T) == 2)
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
    else
        *reinterpret_cast<float4*>(dst) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
}

// O rows of (b, g) for a request without keys (zeros) or with an invalid range or agent (NaN)
template <typename T, int D>
__device__ __forceinline__ void small_fill(const DecodeParams& p, int b, int g, bool ok) {
    const T fill = from_f32<T>(ok ? 0.f : __builtin_nanf(""));
    T* Op = static_cast<T*>(p.O) + (int64_t(b) * p.n_q + int64_t(g) * p.G) * D;
    for (int i = threadIdx.x; i < p.G * D; i += blockDim.x) Op[i] = fill;
}

template <typename T, int D, int R, int GP, int CW, bool FINAL>
__global__ __launch_bounds__(64 * CW, 2) void decode_small_kernel(DecodeParams p) {
    constexpr int kSmallWaves = CW, kSmallThreads = 64 * CW, kChunk = kTile * CW;
    using Tile = DecodeTile<T, D>;
    using F = SmallRecord<D, GP, CW>;
    constexpr int VEC = Tile::VEC, KCH = Tile::KCH, ENT = F::ENT, FR = F::FR;
    __shared__ f32x4 st[kSmallWaves][ENT][FR];
    __shared__ float st_m[kSmallWaves][GP], st_l[kSmallWaves][GP];
    __shared__ SmallOut<D, R, GP> so;

    const int c = blockIdx.x % p.n_chunks;
    const int bg = blockIdx.x / p.n_chunks;
    const int b = bg / p.n_kv, g = bg - b * p.n_kv;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const int G = p.G;
    // the group's queries as the B operand (columns >= G are zero), and with one chunk the B values,
    // requested together with the request's range
    Vec<T, 8> qf[KCH];
    {
        const T* __restrict__ Qp = static_cast<const T*>(p.Q) + (int64_t(b) * p.n_q + int64_t(g) * G + min(n, G - 1)) * D + 8 * q;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            if (n < G) qf[i].load(Qp + 32 * i);
            else qf[i].zero();
        }
    }
    SmallB<T, D, R> sb;
    if constexpr (FINAL) sb.prefetch(p, g);
    const int64_t start = p.kv_start[b];
    const int32_t len = p.kv_len[b];
    const int32_t a = p.agent[b];
    const bool ok = decode_request_ok(start, len, a, p);
    if (!ok || int64_t(len) <= int64_t(c) * kChunk) {   // workgroup-uniform
        if (FINAL && c == 0) small_fill<T, D>(p, b, g, ok);
        return;
    }
    const int kt = c * kChunk + wv * kTile;   // this wave's tile (wave 0's is never empty)
    const bool live = kt < len;

    f32x4 acc[VEC];
#pragma unroll
    for (int tt = 0; tt < VEC; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 acc_lr = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    if (live) {   // wave-uniform
        const int lim = len - 1 - kt;   // keys past it read row len - 1 and get P = 0
        const int64_t row0 = start + kt;
        const T* __restrict__ Kp = static_cast<const T*>(p.K) + row0 * p.kv_row_stride + int64_t(g) * p.kv_head_stride;
        const T* __restrict__ Vp = static_cast<const T*>(p.V) + row0 * p.kv_row_stride + int64_t(g) * p.kv_head_stride;
        const T* __restrict__ Lp = static_cast<const T*>(p.Vlr) + row0 * p.ld_vlr + int64_t(max(a, 0)) * p.vlr_agent_stride + n % R;
        Tile t;
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const int64_t o = int64_t(min(16 * uu + n, lim)) * p.kv_row_stride + 8 * q;
#pragma unroll
            for (int i = 0; i < KCH; ++i) t.k[uu][i].load(Kp + o + 32 * i);
        }
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = min(tile_key(q, e), lim);
            t.v[e].load(Vp + int64_t(key) * p.kv_row_stride + VEC * n);
            if constexpr (sizeof(T) == 2) h[e] = *reinterpret_cast<const uint16_t*>(Lp + int64_t(key) * p.ld_vlr);
            else t.lr.v[e] = Lp[int64_t(key) * p.ld_vlr];
        }
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) t.lr.w[qq] = h[2 * qq] | (h[2 * qq + 1] << 16);
        }
        // S^T = K Q^T; lane (n, q) holds head n's scores of keys tile_key(q, e)
        f32x4 sacc[2];
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            sacc[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KCH; ++i) sacc[uu] = mma16x16x32(t.k[uu][i], qf[i], sacc[uu]);
        }
        const float sl2 = p.scale * kLog2e;
        float sc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[e] = tile_key(q, e) <= lim ? sacc[e >> 2][e & 3] * sl2 : -INFINITY;
        float mx = sc[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        m = mx;   // key kt is live: finite
        float pr[8], ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pr[e] = fast_exp2(sc[e] - m);
            ls += pr[e];
        }
        ls += __shfl_xor(ls, 16);
        l = ls + __shfl_xor(ls, 32);
        if constexpr (sizeof(T) == 2) {
            Vec<bf16, 8> phi, plo;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                phi.w[qq] = pack_bf16x2(pr[2 * qq], pr[2 * qq + 1]);
                plo.w[qq] = pack_bf16x2(pr[2 * qq] - bf16_lo(phi.w[qq]), pr[2 * qq + 1] - bf16_hi(phi.w[qq]));
            }
#pragma unroll
            for (int tt = 0; tt < VEC; ++tt) {
                const Vec<bf16, 8> va = v_operand<VEC>(t.v, tt);
                acc[tt] = mma16x16x32(va, phi, acc[tt]);
                acc[tt] = mma16x16x32(va, plo, acc[tt]);
            }
            acc_lr = mma16x16x32(t.lr, phi, acc_lr);
            acc_lr = mma16x16x32(t.lr, plo, acc_lr);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
#pragma unroll
                for (int tt = 0; tt < VEC; ++tt)
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[e].v[tt], pr[e], acc[tt], 0, 0, 0);
                acc_lr = __builtin_amdgcn_mfma_f32_16x16x4f32(t.lr.v[e], pr[e], acc_lr, 0, 0, 0);
            }
        }
    }
    // the wave partials (an empty wave: m = -inf, zeros) -> LDS
    if (n < GP) {
        const int i = q * GP + n;
#pragma unroll
        for (int tt = 0; tt < VEC; ++tt) st[wv][tt][i] = acc[tt];
        st[wv][VEC][i] = acc_lr;
        if (q == 0) {
            st_m[wv][n] = m;
            st_l[wv][n] = l;
        }
    }
    __syncthreads();
    // fragment (tt, i) summed over the waves in order with weights 2^(m_w - max m)
    float* rec = p.records + (int64_t(bg) * p.n_chunks + c) * (F::SLOTS * 4);
#pragma unroll
    for (int u = 0; u < F::FPT; ++u) {
        const int fi = threadIdx.x + u * kSmallThreads;
        if (fi < ENT * FR) {
            const int tt = fi / FR, i = fi % FR, hn = i % GP;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kSmallWaves; ++w) M = fmaxf(M, st_m[w][hn]);
            f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < kSmallWaves; ++w) {
                const float e = fast_exp2(st_m[w][hn] - M);
                v += st[w][tt][i] * e;
                L = fmaf(st_l[w][hn], e, L);
            }
            if constexpr (FINAL) {
                small_put<D, R, GP>(so, tt, i, v);
                if (fi < GP) so.l[fi] = L;
            } else {
                reinterpret_cast<f32x4*>(rec)[fi] = v;
                if (fi < GP) {
                    rec[F::ML * 4 + fi] = M;
                    rec[F::ML * 4 + GP + fi] = L;
                }
            }
        }
    }
    if constexpr (FINAL) {
        __syncthreads();
        small_epilogue<T, D, R, GP>(p, b, g, a, so, sb);
    }
}

// merge of the chunk records of one (request b, KV head g): thread (tt, i) keeps its fragment's
// running maximum and sum over the chunks (the log-sum-exp rule). The first CB chunks' records are
// requested before the request's length is known (chunks past it hold stale values and are not used).
template <typename T, int D, int R, int GP, int CW>
__global__ __launch_bounds__(kCombineThreads) void decode_small_combine_kernel(DecodeParams p) {
    constexpr int kSmallThreads = kCombineThreads, kChunk = kTile * CW;
    using F = SmallRecord<D, GP, kCombineWaves>;
    constexpr int ENT = F::ENT, FR = F::FR, FPT = F::FPT, CB = 16;
    __shared__ SmallOut<D, R, GP> so;
    const int bg = blockIdx.x;
    const int b = bg / p.n_kv, g = bg - b * p.n_kv;
    const float* rec = p.records + int64_t(bg) * p.n_chunks * (F::SLOTS * 4);
    f32x4 x[FPT][CB];
    float mc[FPT][CB], lc[FPT][CB];
    auto load_batch = [&](int c0, int nc) {
#pragma unroll
        for (int u = 0; u < FPT; ++u) {
            const int fi = min(int(threadIdx.x) + u * kSmallThreads, ENT * FR - 1);
            const int hn = (fi % FR) % GP;
#pragma unroll
            for (int k = 0; k < CB; ++k) {
                const float* r = rec + int64_t(min(c0 + k, nc - 1)) * (F::SLOTS * 4);
                x[u][k] = reinterpret_cast<const f32x4*>(r)[fi];
                mc[u][k] = r[F::ML * 4 + hn];
                lc[u][k] = r[F::ML * 4 + GP + hn];
            }
        }
    };
    load_batch(0, p.n_chunks);
    SmallB<T, D, R> sb;
    sb.prefetch(p, g);
    const int64_t start = p.kv_start[b];
    const int32_t len = p.kv_len[b];
    const int32_t a = p.agent[b];
    const bool ok = decode_request_ok(start, len, a, p);
    if (!ok || len == 0) {
        small_fill<T, D>(p, b, g, ok);
        return;
    }
    const int nc = (len + kChunk - 1) / kChunk;   // <= n_chunks
    float M[FPT], L[FPT];
    f32x4 v[FPT];
#pragma unroll
    for (int u = 0; u < FPT; ++u) {
        M[u] = -INFINITY;
        L[u] = 0.f;
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int c0 = 0; c0 < nc; c0 += CB) {
        if (c0 > 0) load_batch(c0, nc);
#pragma unroll
        for (int u = 0; u < FPT; ++u)
#pragma unroll
            for (int k = 0; k < CB; ++k) {
                if (c0 + k < nc) {
                    const float mn = fmaxf(M[u], mc[u][k]);
                    const float keep = fast_exp2(M[u] - mn), w = fast_exp2(mc[u][k] - mn);
                    v[u] = v[u] * keep + x[u][k] * w;
                    L[u] = fmaf(L[u], keep, lc[u][k] * w);
                    M[u] = mn;
                }
            }
    }
#pragma unroll
    for (int u = 0; u < FPT; ++u) {
        const int fi = threadIdx.x + u * kSmallThreads;
        if (fi < ENT * FR) {
            small_put<D, R, GP>(so, fi / FR, fi % FR, v[u]);
            if (fi < GP) so.l[fi] = L[u];
        }
    }
    __syncthreads();
    small_epilogue<T, D, R, GP>(p, b, g, a, so, sb);
}

template <typename T, int D, int R, int GP, int CW>
hipError_t launch_small(const DecodeParams& p, hipStream_t stream) {
    const dim3 block{unsigned(64 * CW)};
    const unsigned n_bg = unsigned(p.batch * p.n_kv);
    if (p.n_chunks == 1) {
        hipLaunchKernelGGL((decode_small_kernel<T, D, R, GP, CW, true>), dim3(n_bg), block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((decode_small_kernel<T, D, R, GP, CW, false>), dim3(n_bg * unsigned(p.n_chunks)), block, 0, stream, p);
        hipLaunchKernelGGL((decode_small_combine_kernel<T, D, R, GP, CW>), dim3(n_bg), dim3(kCombineThreads), 0, stream, p);
    }
    return hipGetLastError();
}

template <typename T, int D, int R, int GP>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
    if (p.n_chunks > 0)
        return p.chunk_keys == 128 ? launch_small<T, D, R, GP, 4>(p, stream) : launch_small<T, D, R, GP, 8>(p, stream);
    // slots x head groups of 8 (n_slots is a multiple of 8)
    const int64_t n_wg = int64_t(p.n_slots) * ((p.n_kv + kSplitWaves - 1) / kSplitWaves) + (p.X_new ? p.n_pre : 0);
    if (n_wg > 0) {
        const dim3 grid{unsigned(n_wg)}, block{unsigned(kSplitThreads)};
        if (p.key_scores) {
            if constexpr (sizeof(T) == 2)
                hipLaunchKernelGGL((decode_split_kernel<T, D, R, GP, false, true>), grid, block, 0, stream, p);
        } else if (p.block_table) {
            hipLaunchKernelGGL((decode_split_kernel<T, D, R, GP, true, false>), grid, block, 0, stream, p);
        } else {
            hipLaunchKernelGGL((decode_split_kernel<T, D, R, GP, false, false>), grid, block, 0, stream, p);
        }
    }
    if (p.block_table)
        hipLaunchKernelGGL((decode_combine_kernel<T, D, R, GP, true>), dim3(unsigned(p.batch * p.n_kv)), dim3(kCombineThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_combine_kernel<T, D, R, GP, false>), dim3(unsigned(p.batch * p.n_kv)), dim3(kCombineThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, int R>
hipError_t dispatch_gp(const DecodeParams& p, hipStream_t s) {
    return p.G <= 4 ? launch_decode_t<T, D, R, 4>(p, s) : launch_decode_t<T, D, R, 8>(p, s);
}
template <typename T, int D>
hipError_t dispatch_r(const DecodeParams& p, hipStream_t s) {
    return p.rank == 8 ? dispatch_gp<T, D, 8>(p, s) : dispatch_gp<T, D, 16>(p, s);
}
template <typename T>
hipError_t dispatch_d(const DecodeParams& p, hipStream_t s) {
    return p.d_head == 64 ? dispatch_r<T, 64>(p, s) : dispatch_r<T, 128>(p, s);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
    return p.bf16 ? dispatch_d<bf16>(p, stream) : dispatch_d<float>(p, stream);
}

}  // namespace lra
