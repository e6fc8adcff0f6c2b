// Flash-LoRA-Attention causal chunked prefill for gfx950.
//
// Method (LRAgent page, "method steps" (3)-(4) and "core method"): stream key/value tiles with an
// online softmax; next to the base output O accumulate the rank-r output O_lr = P V_lr (the agent's
// column slice of the LR cache) from the same probability tile; after the last tile apply the
// up-projection O <- O + O_lr B_agent once per query row and normalise. The chunk's L_C queries sit
// at positions L_P .. L_P+L_C-1 after the reused context (PReCache summary page), causal mask
// bottom-right aligned.
//
// gfx950 mapping (16x16x32 matrix-core steps, fp32 accumulation; fp32 inputs run the same template
// on 16x16x4 fp32 steps):
//   * one workgroup = 8 waves (two per SIMD) = 256 "query rows" of one KV head; a query row is one
//     (query, head) pair of the head's group, so all G heads of a group share every K/V tile
//     (grouped-query). Each wave owns 2 tiles of 16 rows; their queries stay in registers as MFMA B
//     operands. The two halves of a workgroup take 128-row pieces from the two ends of the chunk,
//     one with a short causal key range and one with a long one, which evens out the work per
//     workgroup and per SIMD; a wave stops multiplying after its own last visible key.
//   * 64-key tiles are staged in LDS in their natural row layout with 128-bit stores, double
//     buffered; two register sets keep the next two tiles' global loads in flight while the
//     current one is multiplied (a tile's loads have two tile steps to arrive),
//     one barrier per tile. A wave takes the whole tile in one softmax step when it sees both of its
//     32-key blocks (one block on its diagonal), which halves the per-step bookkeeping.
//   * S^T = K Q^T: A operand = 16 keys x 8 d-elements of the K tile; output lane (q, n) holds keys
//     4q..4q+3 of each 16-key group for query row n. The two groups of a block give the lane the 8
//     keys it feeds as the B operand of O^T = V^T P^T, so P never leaves the lane.
//   * V^T operand: LDS transpose reads (ds_read_b64_tr_b16) turn the row-major V tile into the
//     operand directly: two per 16-d tile give lane n column d0+n of the lane group's 8 keys.
//   * bf16 inputs: Q.K runs on bf16 steps; P.V on fp16 steps, with V and V_lr converted bf16 ->
//     fp16 once while they are staged (exact for |v| <= 65504) and P rounded to fp16. A workgroup
//     whose fp32 sums left the finite range (a value beyond the fp16 range became inf) or whose
//     scores are too large for the folded exponent runs a second, range-safe pass over its tiles
//     (workgroup-uniform, so the fast pass never pays for it): bf16 V and V_lr, scaled by a power
//     of two when huge, exact differences to the row max, and P split into bf16 hi + lo parts (two
//     steps, ~16 bits of P).
//   * one more 16-column tile holds the agent's V_lr slice (columns 0..r-1) and a column of ones:
//     O_lr^T and the softmax normaliser l come out of the same matrix-core product as O (l is the
//     sum of exactly the rounded P the products used). For r = 16 the ones column is a second tile.
//   * online softmax per query row and softmax step in base 2, scale*log2(e) folded into one fma
//     per score. The reference max m only moves (and O, O_lr, l are rescaled) when a score of the
//     step exceeds it by more than a factor 2^8 in P; otherwise P may reach 2^8, well inside fp16.
//     Each lane tests its own 8 or 16 scores against that threshold; only when some lane of the wave
//     crosses it is the row max reduced over the 4 lanes sharing a row (permlane swaps).
//   * epilogue: gather O_lr and l of the row across its 4 lanes, add O_lr B_agent (B slice in LDS),
//     divide by l, store in the input type (bf16 round-to-nearest-even)
#include <type_traits>

#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

typedef uint32_t pf_u32x4 __attribute__((ext_vector_type(4)));
// 8 elements at byte offset off of a buffer (zeros past its range)
template <typename T>
__device__ __forceinline__ void buffer_load8(Vec<T, 8>& v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    if constexpr (sizeof(T) == 2) {
        const pf_u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) v.w[i] = x[i];
    } else {
        const pf_u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        const pf_u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v.v[i] = __uint_as_float(x0[i]);
            v.v[4 + i] = __uint_as_float(x1[i]);
        }
    }
}

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMT = 2;                          // 16-row tiles per wave
constexpr int kRowsPerWG = 16 * kMT * kWaves;   // 256 query rows
constexpr int kPieceRows = kRowsPerWG / 2;      // rows of one half of a workgroup
constexpr int kBK = 64;                         // keys per LDS tile
static_assert(kBK == kKeyTile, "the key expansion flags one LDS tile each");
constexpr float kRescaleLog2 = 8.f;             // m moves when P would exceed 2^8

template <typename T> struct PrefillTypes {
    // element type of the P.V operands in LDS: fp16 bits (fast pass) or bf16 bits (range-safe pass)
    // for bf16 inputs, fp32 for fp32 inputs
    using TV = typename std::conditional<sizeof(T) == 2, uint16_t, float>::type;
    // P as an MFMA B operand: 8 fp16 values (4 dwords) or 8 fp32 values (one per 16x16x4 step)
    using PF = typename std::conditional<sizeof(T) == 2, H8, Vec<float, 8>>::type;
};

template <typename T, int D, int R, bool KLORA>
struct PrefillShared {
    using TV = typename PrefillTypes<T>::TV;
    static constexpr int NAUX = R < 16 ? 1 : 2;        // V_lr + ones tiles
    static constexpr int LDK = D + 16 / sizeof(T);     // K row (elements), padded by 16 bytes
    static constexpr int LDV = D + 32 / sizeof(TV);    // V row, padded by 32 bytes (transpose reads)
    static constexpr int LDX = 16 * NAUX;              // aux row: V_lr columns, then the ones column
    // every tile starts on a 16-byte boundary: the 128-bit LDS reads and writes depend on it
    alignas(16) T k[2][kBK * LDK];
    alignas(16) TV v[2][kBK * LDV];
    alignas(16) TV aux[2][kBK * LDX];
    alignas(16) float b[R * D];   // B_agent[:, g*D .. g*D+D-1]
    // LoRA on the keys, range-safe pass (single-buffered): the keys as three bf16 parts, high in
    // k[0], middle in k[1], low here; and the agent's B_k slice of this KV head
    alignas(16) T klo[KLORA ? kBK * LDK : 1];
    alignas(16) float bk[KLORA ? R * D : 1];
    int range_bad;    // bit 1: a bad page id; bit 2: a row max too large for the fast pass's fma;
                      // bit 3: a non-finite accumulator after the fast pass
    uint32_t vmax_bits, qmax_bits, kmax_bits;   // largest |V|, |Q|, |expanded key| met (fp32 bits)
};

// hi + lo bf16 parts of two fp32 values (about 16 significant bits together)
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}
// three bf16 parts of two fp32 values (all 24 significant bits)
__device__ __forceinline__ void split3_bf16x2(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = pack_bf16x2(a, b);
    const float ra = a - bf16_lo(hi), rb = b - bf16_hi(hi);
    mid = pack_bf16x2(ra, rb);
    lo = pack_bf16x2(ra - bf16_lo(mid), rb - bf16_hi(mid));
}
// the fast pass's fp16 keys and fp16 queries keep every score within about 2^-10 * max|q| * max|k|
// of its value; past this product (or past the fp16 range) a workgroup takes the range-safe pass
constexpr float kKeyQueryProductMax = 1024.f;
// largest |row max * scale * log2 e| the fast pass's folded fma handles to within 2^-10
constexpr float kFoldedMaxLog2 = 16384.f;

template <typename T, int D, int R, bool PAGED, bool KLORA>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
    using TV = typename PrefillTypes<T>::TV;
    using PF = typename PrefillTypes<T>::PF;
    using SH = PrefillShared<T, D, R, KLORA>;
    static_assert(!KLORA || (sizeof(T) == 2 && !PAGED), "key LoRA: bf16, contiguous cache");
    constexpr int KCH = D / 32;      // Q.K reduction chunks
    constexpr int NKB = kBK / 32;    // 32-key blocks of a tile
    constexpr int NDT = D / 16;      // O^T tiles: tile t holds d = 16t .. 16t+15
    constexpr int NAUX = SH::NAUX;
    constexpr int LDK = SH::LDK, LDV = SH::LDV, LDX = SH::LDX;
    constexpr int MT = kMT;
    constexpr int KF = kBK * D / 8 / kThreads;   // 8-element fragments per thread of K (and of V)
    static_assert(KF >= 1 && kBK * D / 8 % kThreads == 0, "tile split");
    constexpr int LF = kBK * R / 8;              // 8-element fragments of the V_lr tile
    static_assert(LF <= kThreads, "V_lr tile split");
    constexpr int LROW = R < 16 ? R : 16;        // aux column holding the ones (l)

    __shared__ __align__(16) SH sh;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int G = p.G;
    const int n_kv = p.n_kv;
    // workgroup -> (request, pair of row pieces, KV head); KV head = w mod n_kv keeps one head per
    // XCD when n_kv = 8
    const int per_req = p.max_pairs * n_kv;
    const int req = int(blockIdx.x) / per_req;
    const int wrem = int(blockIdx.x) - req * per_req;
    const int g = wrem % n_kv;
    const int pair = wrem / n_kv;
    // The request's chunk: L_C queries (rows q0 .. of Q and O) at positions L_P .. L_P+L_C-1, over
    // cache rows k0 .. k0+L_P+L_C-1. A batched request is checked here: one without rows that can
    // be written is skipped; one with a bad cache range or agent, or longer than max_q_len, gets
    // NaN in all its rows (spread over its workgroups) and nothing is read.
    const int64_t kv_stride = int64_t(n_kv) * D;
    const int64_t q_stride = int64_t(p.n_q) * D;
    int64_t L_C = p.L_C, L_P = p.L_P, q0 = 0, k0 = 0;
    int agent = p.agent;
    if (p.q_len) {
        L_C = p.q_len[req];
        L_P = p.kv_prefix[req];
        q0 = p.q_start[req];
        k0 = PAGED ? 0 : p.kv_start[req];   // a paged request starts at its page 0
        agent = p.agents[req];
        if (L_C <= 0 || q0 < 0 || q0 + L_C > p.q_rows) return;
        const bool req_bad = L_C > p.max_q_len || L_P < 0 || k0 < 0 || k0 + L_P + L_C > p.kv_rows ||
                             L_P + L_C > int64_t(INT32_MAX) || agent < kAdapterFree || agent >= p.n_agents;
        if (req_bad) {   // workgroup-uniform
            T* Ob = static_cast<T*>(p.O) + q0 * q_stride;
            const int64_t n_el = L_C * G * D;   // this KV head's query rows of the request
            for (int64_t idx = int64_t(pair) * kThreads + tid; idx < n_el; idx += int64_t(p.max_pairs) * kThreads) {
                const int64_t r = idx / D;
                const int c = int(idx - r * D);
                const int64_t qi = r / G;
                Ob[qi * q_stride + (int64_t(g) * G + (r - qi * G)) * D + c] = from_f32<T>(__uint_as_float(0x7fc00000u));
            }
            return;
        }
    }
    const int64_t rows_total = L_C * G;
    // The rows of one KV head are cut into pieces of kPieceRows; the two halves of workgroup `pair`
    // take pieces pair and n_pieces-1-pair, a short and a long causal key range, so workgroups
    // (and SIMDs, each of which runs one wave of each half) get about the same number of
    // query-key pairs. With an odd count the middle workgroup's second half has no rows.
    const int n_pieces = int((rows_total + kPieceRows - 1) / kPieceRows);
    if (pair >= (n_pieces + 1) / 2) return;   // a shorter chunk than the longest in the batch
    const int half = wv / (kWaves / 2);
    const int piece = half ? n_pieces - 1 - pair : pair;
    const bool half_empty = half && piece == pair;
    const int64_t R0 = int64_t(piece) * kPieceRows + (wv % (kWaves / 2)) * (16 * MT);   // wave's first row
    const bool wave_rows = !half_empty && R0 < rows_total;

    const T* __restrict__ Qp = static_cast<const T*>(p.Q) + q0 * q_stride;
    const T* __restrict__ Kp = static_cast<const T*>(p.K) + k0 * kv_stride;
    const T* __restrict__ Vp = static_cast<const T*>(p.V) + k0 * kv_stride;
    const T* __restrict__ Lp = static_cast<const T*>(p.Vlr) + k0 * p.ld_vlr;
    const T* __restrict__ Bp = static_cast<const T*>(p.B);
    T* __restrict__ Op = static_cast<T*>(p.O) + q0 * q_stride;

    // ---- this lane's query rows (B operand column n of each 16-row tile): absolute positions
    // (< 2^31, checked on the host) and source addresses
    int qpos[MT];
    bool qok[MT];
    const T* qsrc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t r = R0 + mt * 16 + n;
        qok[mt] = wave_rows && r < rows_total;
        const int64_t rc = min(r, rows_total - 1);
        const int64_t qi = rc / G;
        const int qh = int(rc - qi * G);
        qpos[mt] = int(L_P + qi);
        qsrc[mt] = Qp + qi * q_stride + (int64_t(g) * G + qh) * D + 8 * q;
    }

    // ---- key ranges: the workgroup stages keys [0, kv_end) (visible to some row of its long
    // piece); a wave computes the blocks below its own end and masks from its full_end on
    const int64_t heavy_last = min<int64_t>(rows_total, int64_t(n_pieces - pair) * kPieceRows) - 1;
    const int kv_end = int(L_P + heavy_last / G + 1);
    const int n_tiles = (kv_end + kBK - 1) / kBK;
    const int64_t i_min = min(R0, rows_total - 1) / G;
    const int64_t i_max = min<int64_t>(L_C - 1, (R0 + 16 * MT - 1) / G);
    const int wave_end = wave_rows ? int(L_P + i_max + 1) : 0;   // keys [0, wave_end) visible to some row
    const int full_end = int(L_P + i_min + 1);                   // keys [0, full_end) visible to every row

    // ---- B_agent slice in LDS (fp32; zero for the adapter-free view, which has no LR term)
    const bool adapted = agent != kAdapterFree;
    for (int idx = tid; idx < R * D; idx += kThreads) {
        const int rr = idx / D, c = idx - rr * D;
        sh.b[idx] = adapted ? to_f32<T>(Bp[(int64_t(agent) * R + rr) * kv_stride + int64_t(g) * D + c]) : 0.f;
    }
    if (tid == 0) {
        sh.range_bad = 0;
        sh.vmax_bits = sh.qmax_bits = sh.kmax_bits = 0u;
    }
    // expanded keys: the largest |key| of the tiles this workgroup stages, read once up front
    float kmax = 0.f;
    if constexpr (KLORA) {
        for (int t = tid; t < n_tiles; t += kThreads) kmax = fmaxf(kmax, __int_as_float(p.key_flags[int64_t(t) * n_kv + g]));
    }

    float qmax = 0.f;     // largest |Q| entry of this lane's rows (LoRA on the keys)
    float vscale = 1.f;   // power of two the range-safe pass applies to V and V_lr as it stages them
    float unscale = 1.f;  // its inverse, applied to the outputs
    const float sl2 = p.scale * kLog2e;
    const float thr_gap = kRescaleLog2 / sl2;   // scale > 0
    // Paged cache: each wave keeps the page ids of 64 consecutive blocks of the request, one per
    // lane, and reloads that window when a tile moves past it (once per 64 pages). A 64-key tile
    // never crosses a page (P >= 64, a power of two). A page id outside [0, n_pages) reads page 0
    // instead and turns the workgroup's rows to NaN.
    int pg_vec = 0, pg_base = 0;
    bool pg_bad = false;
    const int n_blk = PAGED ? int((L_P + L_C + (int64_t(1) << p.page_shift) - 1) >> p.page_shift) : 0;

    // One pass over the key tiles, then the epilogue. The fast pass (WIDE = false) takes P.V on fp16
    // steps (and, with LoRA on the keys, the scores on fp16 steps over the expanded fp16 keys), with
    // double-buffered tiles. A workgroup whose fp32 sums left the finite range (a staged value
    // beyond the fp16 range), whose scores are too large for the folded exponent (or, with LoRA on
    // the keys, whose queries and keys are too large for fp16 precision) runs the range-safe pass
    // (WIDE = true) after it, which rewrites the same rows; it stages one tile at a time: bf16 V and
    // V_lr (scaled by vscale, a power of two, when they are huge), P as a bf16 hi + lo pair, and with
    // LoRA on the keys bf16 queries against the keys rebuilt in fp32 and split into three bf16
    // parts. Each pass holds its own accumulators (captured from outside, the arrays cost about 30
    // registers).
    auto pass = [&](auto wide_tag) {
        constexpr bool WIDE = decltype(wide_tag)::value;
        static_assert(!WIDE || sizeof(T) == 2, "the range-safe pass is for bf16 inputs");
        constexpr bool F16S = KLORA && !WIDE;   // scores on fp16 steps
        constexpr bool KREBUILD = KLORA && WIDE;  // keys rebuilt in fp32, three bf16 parts

        Vec<T, 8> qf[MT][KCH];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                if (qok[mt]) qf[mt][i].load(qsrc[mt] + 32 * i);
                else qf[mt][i].zero();
            }
        if constexpr (KLORA) {
            if constexpr (F16S) {
                // the fast pass with LoRA on the keys converts the queries to fp16 (exact within its range)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < KCH; ++i)
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) {
                            const float lo = bf16_lo(qf[mt][i].w[e2]), hi = bf16_hi(qf[mt][i].w[e2]);
                            qmax = fmaxf(qmax, fmaxf(fabsf(lo), fabsf(hi)));
                            qf[mt][i].w[e2] = pack_f16x2(lo, hi);
                        }
                // take the maximum here: sunk to its use after the pass it would keep the bf16 rows live
                asm volatile("" : "+v"(qmax));
            }
        }

        // the ones / zero columns of the aux tiles, in the pass's P.V element type
        for (int idx = tid; idx < 2 * kBK * (LDX - R); idx += kThreads) {
            const int buf = idx / (kBK * (LDX - R));
            const int rem = idx - buf * (kBK * (LDX - R));
            const int key = rem / (LDX - R);
            const int col = R + rem % (LDX - R);
            const float v = col == LROW ? 1.f : 0.f;
            TV tv;
            if constexpr (sizeof(T) == 2) tv = TV((WIDE ? pack_bf16x2(v, 0.f) : pack_f16x2(v, 0.f)) & 0xffffu);
            else tv = v;
            sh.aux[buf][key * LDX + col] = tv;
        }
        if constexpr (KREBUILD) {   // the agent's B_k slice of this KV head (ordered by the loop's first barrier)
            for (int idx = tid; idx < R * D; idx += kThreads) {
                const int rr = idx / D, c = idx - rr * D;
                sh.bk[idx] = to_f32<T>(static_cast<const T*>(p.Bk)[(int64_t(agent) * R + rr) * kv_stride + int64_t(g) * D + c]);
            }
        }

        // ---- tile fetch (registers) and store (LDS). A contiguous cache is read through a buffer
        // at the tile's first row whose range ends at row kv_end, with this thread's byte offsets in
        // a tile fixed for the pass: the loads take no vector address arithmetic, and keys past
        // kv_end read zeros. A paged cache reads row kv_end-1 for them. Either way they get P = 0.
        // two register sets: the fast pass keeps two tiles' loads in flight where they fit
        Vec<T, 8> kpre[2][KF], vpre[2][KF], lpre[2];
        lpre[0].zero();   // the adapter-free view stages zero V_lr columns
        lpre[1].zero();
        pg_base = -(1 << 30);
        uint32_t koff[KF];
#pragma unroll
        for (int c = 0; c < KF; ++c) {
            const int f = tid + kThreads * c;
            const int key = f / (D / 8);
            koff[c] = uint32_t((int64_t(key) * kv_stride + int64_t(g) * D + (f - key * (D / 8)) * 8) * int64_t(sizeof(T)));
        }
        const uint32_t loff = uint32_t((int64_t(tid / (R / 8)) * p.ld_vlr + (tid % (R / 8)) * 8) * int64_t(sizeof(T)));
        auto fetch = [&](int t, auto set_tag) {
            constexpr int S = decltype(set_tag)::value;
            const int kb = t * kBK;
            if constexpr (!PAGED) {
                const uint32_t rows = uint32_t(min(kBK, kv_end - kb));   // >= 1
                const uint32_t kv_bytes = rows * uint32_t(kv_stride * int64_t(sizeof(T)));   // < 2^31 (host bound)
                const __amdgpu_buffer_rsrc_t rk =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Kp + int64_t(kb) * kv_stride), 0, int(kv_bytes), 0x00020000);
                const __amdgpu_buffer_rsrc_t rv =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Vp + int64_t(kb) * kv_stride), 0, int(kv_bytes), 0x00020000);
#pragma unroll
                for (int c = 0; c < KF; ++c) {
                    if constexpr (!KREBUILD) buffer_load8(kpre[S][c], rk, koff[c]);
                    buffer_load8(vpre[S][c], rv, koff[c]);
                }
                if (tid < LF && adapted) {
                    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<T*>(Lp + int64_t(kb) * p.ld_vlr + int64_t(agent) * p.vlr_agent_stride), 0,
                        int(rows * uint32_t(p.ld_vlr * int64_t(sizeof(T)))), 0x00020000);
                    buffer_load8(lpre[S], rl, loff);
                }
                return;
            }
            int64_t page_off = 0;   // cache row of key j = j + page_off for every key j of the tile
            if constexpr (PAGED) {
                const int pi = kb >> p.page_shift;
                if (pi - pg_base >= 64) {
                    pg_base = pi;
                    int id = 0;
                    if (pg_base + lane < n_blk) id = p.block_table[int64_t(req) * p.max_blocks + pg_base + lane];
                    const bool bad = pg_base + lane < n_blk && (id < 0 || int64_t(id) >= p.n_pages);
                    pg_bad = pg_bad || bad;
                    pg_vec = bad ? 0 : id;
                }
                const int page = __builtin_amdgcn_readlane(pg_vec, pi - pg_base);
                page_off = (int64_t(page) - pi) << p.page_shift;
            }
#pragma unroll
            for (int c = 0; c < KF; ++c) {
                const int f = tid + kThreads * c;
                const int key = f / (D / 8);
                const int d0 = (f - key * (D / 8)) * 8;
                const int64_t j = min(kb + key, kv_end - 1) + page_off;
                if constexpr (!KREBUILD) kpre[S][c].load(Kp + j * kv_stride + int64_t(g) * D + d0);
                vpre[S][c].load(Vp + j * kv_stride + int64_t(g) * D + d0);
            }
            if (tid < LF && adapted) {
                const int key = tid / (R / 8);
                const int r0 = (tid - key * (R / 8)) * 8;
                const int64_t j = min(kb + key, kv_end - 1) + page_off;
                lpre[S].load(Lp + j * p.ld_vlr + int64_t(agent) * p.vlr_agent_stride + r0);
            }
        };
        // 8 values of one key's row in the pass's P.V element type: fp16 (exact within its range),
        // bf16 times vscale (range-safe pass), or fp32
        auto put8 = [&](TV* dst, const Vec<T, 8>& src) {
            if constexpr (sizeof(T) == 2) {
                uint32_t hv[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float lo = bf16_lo(src.w[e2]), hi = bf16_hi(src.w[e2]);
                    if constexpr (WIDE) hv[e2] = pack_bf16x2(lo * vscale, hi * vscale);
                    else hv[e2] = pack_f16x2(lo, hi);   // beyond the fp16 range: inf (checked after the pass)
                }
                *reinterpret_cast<uint4*>(dst) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(src.v[0], src.v[1], src.v[2], src.v[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(src.v[4], src.v[5], src.v[6], src.v[7]);
            }
        };
        auto store = [&](int buf, auto set_tag) {
            constexpr int S = decltype(set_tag)::value;
#pragma unroll
            for (int c = 0; c < KF; ++c) {
                const int f = tid + kThreads * c;
                const int key = f / (D / 8);
                const int d0 = (f - key * (D / 8)) * 8;
                if constexpr (sizeof(T) == 2) {
                    if constexpr (!KREBUILD)
                        *reinterpret_cast<uint4*>(&sh.k[buf][key * LDK + d0]) = *reinterpret_cast<const uint4*>(kpre[S][c].w);
                } else {
                    float* kd = &sh.k[buf][key * LDK + d0];
                    *reinterpret_cast<float4*>(kd) = make_float4(kpre[S][c].v[0], kpre[S][c].v[1], kpre[S][c].v[2], kpre[S][c].v[3]);
                    *reinterpret_cast<float4*>(kd + 4) = make_float4(kpre[S][c].v[4], kpre[S][c].v[5], kpre[S][c].v[6], kpre[S][c].v[7]);
                }
                put8(&sh.v[buf][key * LDV + d0], vpre[S][c]);
            }
            if (tid < LF) {
                const int key = tid / (R / 8);
                const int r0 = (tid - key * (R / 8)) * 8;
                put8(&sh.aux[buf][key * LDX + r0], lpre[S]);
            }
        };
        // range-safe pass with LoRA on the keys: key j of the tile rebuilt in fp32 from K_base, K_lr,
        // B_k and the rotary tables (rotate-half pairing, the same sum as the key expansion pass:
        // element i < d/2 gets y_i cos_i - y_{i+d/2} sin_i, element i + d/2 gets
        // y_{i+d/2} cos_i + y_i sin_i, y = K_lr[j] B_k), then split into three bf16 parts
        auto stage_keys_wide = [&](int t) {
            if constexpr (KREBUILD) {
                const T* __restrict__ Ks = static_cast<const T*>(p.K_src) + k0 * kv_stride;
                const T* __restrict__ Kl = static_cast<const T*>(p.Klr) + k0 * p.ld_klr;
                // rolled loops: this pass is rare, and unrolled it would spill registers
#pragma unroll 1
                for (int c = 0; c < KF; ++c) {
                    const int f = tid + kThreads * c;
                    const int key = f / (D / 8);
                    const int d0 = (f - key * (D / 8)) * 8;
                    const int64_t j = min(t * kBK + key, kv_end - 1);
                    const bool low = d0 < D / 2;
                    const int i0 = low ? d0 : d0 - D / 2;
                    const int dp0 = low ? d0 + D / 2 : d0 - D / 2;   // rotation partners
                    const uint32_t* kb2 = reinterpret_cast<const uint32_t*>(Ks + j * kv_stride + int64_t(g) * D + d0);
                    const T* lr = Kl + j * p.ld_klr + int64_t(agent) * R;
                    const float* cs = p.rope_cos + (k0 + j) * (D / 2) + i0;
                    const float* sn = p.rope_sin + (k0 + j) * (D / 2) + i0;
#pragma unroll 1
                    for (int e2 = 0; e2 < 4; ++e2) {
                        float ka[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int x = 2 * e2 + h;
                            float yo = 0.f, yp = 0.f;
#pragma unroll
                            for (int rr = 0; rr < R; ++rr) {
                                const float kr = to_f32<T>(lr[rr]);
                                yo = fmaf(kr, sh.bk[rr * D + d0 + x], yo);
                                yp = fmaf(kr, sh.bk[rr * D + dp0 + x], yp);
                            }
                            const float kbase = h ? bf16_hi(kb2[e2]) : bf16_lo(kb2[e2]);
                            ka[h] = kbase + (low ? (yo * cs[x] - yp * sn[x]) : (yo * cs[x] + yp * sn[x]));
                        }
                        uint32_t hi, mid, lo;
                        split3_bf16x2(ka[0], ka[1], hi, mid, lo);
                        *reinterpret_cast<uint32_t*>(&sh.k[0][key * LDK + d0 + 2 * e2]) = hi;
                        *reinterpret_cast<uint32_t*>(&sh.k[1][key * LDK + d0 + 2 * e2]) = mid;
                        *reinterpret_cast<uint32_t*>(&sh.klo[key * LDK + d0 + 2 * e2]) = lo;
                    }
                }
            }
        };

        // accumulators: O^T tiles (tile t holds d = 16t .. 16t+15), aux tiles (O_lr^T rows
        // 0..R-1, l in row LROW). Lane (q, n) holds rows 4q..4q+3 of each tile for query row n.
        f32x4 oacc[MT][NDT];
        f32x4 xacc[MT][NAUX];
        float m_run[MT];   // raw-score reference maximum of the exponentials
        float m_thr[MT];   // raw score at which P would exceed 2^kRescaleLog2
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            m_run[mt] = -INFINITY;
            m_thr[mt] = -INFINITY;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[mt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < NAUX; ++x) xacc[mt][x] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        // a lane's transpose reads start at key 4q + n/4 of a 32-key block, columns 4(n%4) ..
        const int tr_v = (4 * q + (n >> 2)) * LDV + 4 * (n & 3);
        const int tr_x = (4 * q + (n >> 2)) * LDX + 4 * (n & 3);
        // scores, softmax and P.V of tile t staged in buffer buf
        auto tile_step = [&](int t, int buf) {
            const T* ks = sh.k[buf];
            const T* kms = sh.k[1];   // range-safe pass with LoRA on the keys: middle part
            const T* kls = sh.klo;    // and low part
            const TV* vs = sh.v[buf];
            const TV* xs = sh.aux[buf];

            // blocks of this tile holding a key visible to the wave (wave-uniform); both blocks of a
            // tile go through one softmax step when the wave sees them both
            const int nkb = min(NKB, max(0, (wave_end - t * kBK + 31) / 32));
            auto step = [&](auto nb_tag) {
                constexpr int NB = decltype(nb_tag)::value;   // 32-key blocks in this step
                const int kblk = t * kBK;
                // scores: lane (q, n) holds keys kblk + 16u + 4q + j (u < 2NB; j = 0..3) of query row n
                f32x4 sacc[MT][2 * NB];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int u = 0; u < 2 * NB; ++u) sacc[mt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 2 * NB; ++u)
#pragma unroll
                    for (int i = 0; i < KCH; ++i) {
                        Vec<T, 8> ka;
                        ka.load(&ks[(16 * u + n) * LDK + 32 * i + 8 * q]);
                        if constexpr (KREBUILD) {
                            Vec<T, 8> km, kl;
                            km.load(&kms[(16 * u + n) * LDK + 32 * i + 8 * q]);
                            kl.load(&kls[(16 * u + n) * LDK + 32 * i + 8 * q]);
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                sacc[mt][u] = mma16x16x32(kl, qf[mt][i], sacc[mt][u]);
                                sacc[mt][u] = mma16x16x32(km, qf[mt][i], sacc[mt][u]);
                                sacc[mt][u] = mma16x16x32(ka, qf[mt][i], sacc[mt][u]);
                            }
                        } else {
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                if constexpr (KLORA) {
                                    if constexpr (F16S) sacc[mt][u] = mma16x16x32_f16(ka, qf[mt][i], sacc[mt][u]);
                                    else sacc[mt][u] = mma16x16x32(ka, qf[mt][i], sacc[mt][u]);
                                } else {
                                    sacc[mt][u] = mma16x16x32(ka, qf[mt][i], sacc[mt][u]);
                                }
                            }
                        }
                    }

                // online softmax per query row (raw scores; scale folded into the exponent)
                if (kblk + 32 * NB > full_end) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int u = 0; u < 2 * NB; ++u)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                if (kblk + 16 * u + 4 * q + j > qpos[mt]) sacc[mt][u][j] = -INFINITY;
                }
                float lmx[MT];
                bool any_grow = false;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    // a chain of three-input maxima (the row tiles' chains are independent)
                    float m = fmaxf(sacc[mt][0][0], sacc[mt][0][1]);
                    m = fmaxf(fmaxf(m, sacc[mt][0][2]), sacc[mt][0][3]);
#pragma unroll
                    for (int u = 1; u < 2 * NB; ++u) {
                        m = fmaxf(fmaxf(m, sacc[mt][u][0]), sacc[mt][u][1]);
                        m = fmaxf(fmaxf(m, sacc[mt][u][2]), sacc[mt][u][3]);
                    }
                    lmx[mt] = m;
                    any_grow |= lmx[mt] > m_thr[mt];
                }
                if (__builtin_expect(__ballot(any_grow) != 0, 0)) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const float mx = xor32_max(xor16_max(lmx[mt]));
                        const bool grow = mx > m_thr[mt];
                        const float mnew = grow ? mx : m_run[mt];
                        const float alpha = fast_exp2((m_run[mt] - mnew) * sl2);
                        m_run[mt] = mnew;
                        m_thr[mt] = mnew + thr_gap;
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) oacc[mt][dt] *= alpha;
#pragma unroll
                        for (int x = 0; x < NAUX; ++x) xacc[mt][x] *= alpha;
                    }
                }
                float mbs[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mbs[mt] = -m_run[mt] * sl2;
                // per 32-key block: its probabilities, then its P.V steps (the next block's
                // exponentials can fill the matrix-core shadow of this block's steps)
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    if constexpr (sizeof(T) == 2 && WIDE) {
                        Vec<bf16, 8> phi[MT], plo[MT];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            // exact differences to the row max: any score magnitude works here
                            float pv[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) pv[e] = fast_exp2((sacc[mt][2 * bb + (e >> 2)][e & 3] - m_run[mt]) * sl2);
#pragma unroll
                            for (int w2 = 0; w2 < 4; ++w2) split_bf16x2(pv[2 * w2], pv[2 * w2 + 1], phi[mt].w[w2], plo[mt].w[w2]);
                        }
                        const int rkey = 32 * bb + 4 * q + (n >> 2);
                        const int rcol = 4 * (n & 3);
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) {
                            const uint2 lo = lds_read_tr16(&vs[rkey * LDV + 16 * dt + rcol]);
                            const uint2 hi = lds_read_tr16(&vs[(rkey + 16) * LDV + 16 * dt + rcol]);
                            Vec<bf16, 8> va;
                            va.w[0] = lo.x; va.w[1] = lo.y; va.w[2] = hi.x; va.w[3] = hi.y;
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                oacc[mt][dt] = mma16x16x32(va, plo[mt], oacc[mt][dt]);
                                oacc[mt][dt] = mma16x16x32(va, phi[mt], oacc[mt][dt]);
                            }
                        }
#pragma unroll
                        for (int x = 0; x < NAUX; ++x) {
                            const uint2 lo = lds_read_tr16(&xs[rkey * LDX + 16 * x + rcol]);
                            const uint2 hi = lds_read_tr16(&xs[(rkey + 16) * LDX + 16 * x + rcol]);
                            Vec<bf16, 8> xa;
                            xa.w[0] = lo.x; xa.w[1] = lo.y; xa.w[2] = hi.x; xa.w[3] = hi.y;
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                xacc[mt][x] = mma16x16x32(xa, plo[mt], xacc[mt][x]);
                                xacc[mt][x] = mma16x16x32(xa, phi[mt], xacc[mt][x]);
                            }
                        }
                    } else {
                        PF pf[MT];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            float pv[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(sacc[mt][2 * bb + (e >> 2)][e & 3], sl2, mbs[mt]));
                            if constexpr (sizeof(T) == 2) {
#pragma unroll
                                for (int w2 = 0; w2 < 4; ++w2) pf[mt].w[w2] = pack_f16x2(pv[2 * w2], pv[2 * w2 + 1]);
                            } else {
#pragma unroll
                                for (int e = 0; e < 8; ++e) pf[mt].v[e] = pv[e];
                            }
                        }
                        if constexpr (sizeof(T) == 2) {
                            // this lane's transpose-read addresses: one add per buffer, the rest immediates
                            const TV* vrow = vs + tr_v + 32 * bb * LDV;
                            const TV* xrow = xs + tr_x + 32 * bb * LDX;
#pragma unroll
                            for (int dt = 0; dt < NDT; ++dt) {
                                const uint2 lo = lds_read_tr16(vrow + 16 * dt);
                                const uint2 hi = lds_read_tr16(vrow + 16 * LDV + 16 * dt);
                                H8 va;
                                va.w[0] = lo.x; va.w[1] = lo.y; va.w[2] = hi.x; va.w[3] = hi.y;
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt) oacc[mt][dt] = mma16x16x32_f16(va, pf[mt], oacc[mt][dt]);
                            }
#pragma unroll
                            for (int x = 0; x < NAUX; ++x) {
                                const uint2 lo = lds_read_tr16(xrow + 16 * x);
                                const uint2 hi = lds_read_tr16(xrow + 16 * LDX + 16 * x);
                                H8 xa;
                                xa.w[0] = lo.x; xa.w[1] = lo.y; xa.w[2] = hi.x; xa.w[3] = hi.y;
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt) xacc[mt][x] = mma16x16x32_f16(xa, pf[mt], xacc[mt][x]);
                            }
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int key = 32 * bb + 16 * (e >> 2) + 4 * q + (e & 3);
#pragma unroll
                                for (int dt = 0; dt < NDT; ++dt) {
                                    const float vv = vs[key * LDV + 16 * dt + n];
#pragma unroll
                                    for (int mt = 0; mt < MT; ++mt)
                                        oacc[mt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, pf[mt].v[e], oacc[mt][dt], 0, 0, 0);
                                }
#pragma unroll
                                for (int x = 0; x < NAUX; ++x) {
                                    const float xv = xs[key * LDX + 16 * x + n];
#pragma unroll
                                    for (int mt = 0; mt < MT; ++mt)
                                        xacc[mt][x] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, pf[mt].v[e], xacc[mt][x], 0, 0, 0);
                                }
                            }
                        }
                    }
                }
            };
            if (nkb == 2) step(std::integral_constant<int, 2>{});
            else if (nkb == 1) step(std::integral_constant<int, 1>{});
        };

        if constexpr (!WIDE) {
            // double-buffered LDS tiles, two tiles' loads in flight: tile t is multiplied while the
            // loads of t+1 (issued a tile earlier) and t+2 are outstanding. Where the second register
            // set would not fit beside the accumulators (fp32 inputs; paged rank-16 bf16 with
            // d_head 128) one tile's loads are in flight instead.
            constexpr std::integral_constant<int, 0> s0{};
            constexpr std::integral_constant<int, 1> s1{};
            constexpr bool DEEP = sizeof(T) == 2 && !(PAGED && R == 16 && D == 128);
            if constexpr (!DEEP) {
                fetch(0, s0);
                store(0, s0);
                __syncthreads();
                for (int t = 0; t < n_tiles; ++t) {
                    const int buf = t & 1;
                    if (t + 1 < n_tiles) fetch(t + 1, s0);
                    tile_step(t, buf);
                    if (t + 1 < n_tiles) store(buf ^ 1, s0);
                    __syncthreads();
                }
            } else {
                fetch(0, s0);
                if (1 < n_tiles) fetch(1, s1);
                store(0, s0);
                __syncthreads();
                for (int t = 0; t < n_tiles; t += 2) {
                    if (t + 2 < n_tiles) fetch(t + 2, s0);
                    tile_step(t, 0);
                    if (t + 1 < n_tiles) store(1, s1);
                    __syncthreads();
                    if (t + 1 >= n_tiles) break;
                    if (t + 3 < n_tiles) fetch(t + 3, s1);
                    tile_step(t + 1, 1);
                    if (t + 2 < n_tiles) store(0, s0);
                    __syncthreads();
                }
            }
        } else {
            // the largest |V| / |V_lr| of the staged keys (read once more) brings them to at most 2^64
            // by a power of two, so the unnormalised fp32 sums (at most 2^31 keys, P < 2^9) cannot
            // overflow; the outputs are multiplied back
            if constexpr (sizeof(T) == 2) {
                float vm = 0.f;
                for (int t = 0; t < n_tiles; ++t) {
                    fetch(t, std::integral_constant<int, 0>{});
#pragma unroll
                    for (int c = 0; c < KF; ++c)
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2)
                            vm = fmaxf(fmaxf(vm, fabsf(bf16_lo(vpre[0][c].w[e2]))), fabsf(bf16_hi(vpre[0][c].w[e2])));
                    if (tid < LF && adapted) {
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2)
                            vm = fmaxf(fmaxf(vm, fabsf(bf16_lo(lpre[0].w[e2]))), fabsf(bf16_hi(lpre[0].w[e2])));
                    }
                }
                atomicMax(&sh.vmax_bits, __float_as_uint(vm));   // |v| >= 0: the bits order like the values
                __syncthreads();
                const int ex = int((sh.vmax_bits >> 23) & 0xffu) - 127;
                const int e = max(0, ex - 63);   // <= 65
                vscale = __uint_as_float(uint32_t(127 - e) << 23);
                unscale = __uint_as_float(uint32_t(127 + e) << 23);
            }
            // one tile at a time (the key parts use both K buffers)
            for (int t = 0; t < n_tiles; ++t) {
                fetch(t, std::integral_constant<int, 0>{});
                __syncthreads();   // the previous tile's readers are done
                store(0, std::integral_constant<int, 0>{});
                stage_keys_wide(t);
                __syncthreads();
                tile_step(t, 0);
            }
        }

        // ---- after the fast pass: non-finite sums (a staged value beyond the fp16 range), a row max
        // too large for the folded exponent (and, with LoRA on the keys, the largest |Q| and
        // |expanded key|) decide whether the range-safe pass runs next; a bad page id poisons the rows
        if constexpr (!WIDE) {
            // The fast pass folds the row max m into one fma per score; that fma's rounding, 2^-24 of
            // |m| scale log2(e), must stay negligible in the exponent. m only grows, and an earlier
            // m more than ~150 below the final one has had its terms scaled to zero by the rescale
            // factor, so checking the final m (with that margin) covers every term that counts.
            bool big_scores = false;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) big_scores = big_scores || !(fabsf(m_run[mt] * sl2) <= kFoldedMaxLog2 - 256.f);
            if constexpr (sizeof(T) == 2) {
                // A staged V / V_lr entry beyond the fp16 range became inf, and every staged key is
                // multiplied by some row's probability (inf x 0 is NaN on the matrix cores), so it
                // leaves a non-finite accumulator; so does a non-finite input. Either sends the
                // workgroup to the range-safe pass.
                // (Exponent bits, hidden from the optimiser, not a float compare: this file is built
                // without NaN semantics, which would let a NaN test fold away.)
                auto inf_or_nan = [](float x) {
                    uint32_t b = __float_as_uint(x);
                    asm("" : "+v"(b));
                    return uint32_t((b & 0x7f800000u) == 0x7f800000u);
                };
                uint32_t nonfinite = 0u;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) nonfinite |= inf_or_nan(oacc[mt][dt][j]);
#pragma unroll
                    for (int x = 0; x < NAUX; ++x)
#pragma unroll
                        for (int j = 0; j < 4; ++j) nonfinite |= inf_or_nan(xacc[mt][x][j]);
                }
                if (nonfinite) atomicOr(&sh.range_bad, 8);
            }
            if constexpr (KLORA) {
                atomicMax(&sh.qmax_bits, __float_as_uint(qmax));
                atomicMax(&sh.kmax_bits, __float_as_uint(kmax));
            }
            if (PAGED && pg_bad) atomicOr(&sh.range_bad, 2);
            if (big_scores) atomicOr(&sh.range_bad, 4);
            __syncthreads();
        }
        const bool poison = (sh.range_bad & 2) != 0;

        // ---- epilogue: O_lr and l of the row from its 4 lanes, O += O_lr B_agent, normalise, store
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            // aux row 4q'+j of tile x lives in lane (q', n), register j: gather them for row n
            float olr[R];
#pragma unroll
            for (int rr = 0; rr < R; ++rr) olr[rr] = __shfl(xacc[mt][rr / 16][rr & 3], n + 16 * ((rr & 15) >> 2));
            const float l = __shfl(xacc[mt][LROW / 16][LROW & 3], n + 16 * ((LROW & 15) >> 2));
            const int64_t r = R0 + mt * 16 + n;
            if (!wave_rows || r >= rows_total) continue;
            const int64_t qi = r / G;
            const int qh = int(r - qi * G);
            T* orow = Op + qi * q_stride + (int64_t(g) * G + qh) * D;
            const float inv = poison ? __uint_as_float(0x7fc00000u) : unscale / l;   // quiet NaN by its bits
            // lane (q, n) holds O^T rows 4q+j of tile dt: d = 16dt + 4q + j
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                float o4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = 16 * dt + 4 * q + j;
                    float acc = oacc[mt][dt][j];
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) acc = fmaf(olr[rr], sh.b[rr * D + d], acc);
                    o4[j] = acc * inv;
                }
                T* dst = orow + 16 * dt + 4 * q;
                if constexpr (sizeof(T) == 2)
                    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3]));
                else
                    *reinterpret_cast<float4*>(dst) = make_float4(o4[0], o4[1], o4[2], o4[3]);
            }
        }
    };

    pass(std::false_type{});
    if constexpr (sizeof(T) == 2) {
        bool wide = (sh.range_bad & (4 | 8)) != 0;
        if constexpr (KLORA) {
            const float qm = __uint_as_float(sh.qmax_bits), km = __uint_as_float(sh.kmax_bits);
            wide = wide || !(qm <= kF16Max) || !(km <= kF16Max) || !(qm * km <= kKeyQueryProductMax);
        }
        if (wide) pass(std::true_type{});   // workgroup-uniform
    }
}

template <typename T, int D, int R>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
    const int64_t grid = int64_t(p.batch) * p.max_pairs * p.n_kv;
    if constexpr (sizeof(T) == 2) {
        if (p.key_flags) {
            hipLaunchKernelGGL((prefill_kernel<T, D, R, false, true>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p);
            return hipGetLastError();
        }
    }
    if (p.block_table)
        hipLaunchKernelGGL((prefill_kernel<T, D, R, true, false>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<T, D, R, false, false>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_r(const PrefillParams& p, hipStream_t s) {
    return p.rank == 8 ? launch_t<T, D, 8>(p, s) : launch_t<T, D, 16>(p, s);
}
template <typename T>
hipError_t dispatch_d(const PrefillParams& p, hipStream_t s) {
    return p.d_head == 64 ? dispatch_r<T, 64>(p, s) : dispatch_r<T, 128>(p, s);
}

}  // namespace

int prefill_pairs(int64_t L_C, int G) {
    const int64_t n_pieces = (L_C * G + kPieceRows - 1) / kPieceRows;
    return int((n_pieces + 1) / 2);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    return p.bf16 ? dispatch_d<bf16>(p, stream) : dispatch_d<float>(p, stream);
}

}  // namespace lra
