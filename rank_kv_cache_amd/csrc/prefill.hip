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
//   * one workgroup = 4 waves = 256 "query rows" of one KV head; a query row is one (query, head)
//     pair of that head's group, so all G heads of a group share every K/V tile (grouped-query).
//     Each wave owns 4 tiles of 16 rows; their queries stay in registers as MFMA B operands.
//   * 64-key tiles are staged in LDS in their natural row layout with 128-bit stores, double
//     buffered: the next tile's global loads are in flight while the current one is multiplied,
//     one barrier per tile.
//   * S^T = K Q^T: A operand = 16 keys x 8 d-elements of the K tile; output lane (r, n) holds keys
//     4r..4r+3 of each 16-key group for query row n. Two groups give the lane the 8 keys it feeds
//     as the B operand of O^T = V^T P^T, so P never leaves the lane.
//   * V^T operand: row s of O^T tile t is d = NDT*s + t (NDT = d_head/16 tiles), so a lane reads
//     its 8 keys' V[key][NDT*n .. NDT*n+NDT-1] as one LDS load each and an 8 x NDT 16-bit transpose
//     in registers (byte permutes) yields the NDT operands, shared by the wave's 4 row tiles.
//   * bf16 inputs: Q.K runs on bf16 steps; P.V on fp16 steps, with V and V_lr converted bf16 ->
//     fp16 once while they are staged (exact for |v| <= 65504) and P rounded to fp16. A workgroup
//     that meets a value beyond the fp16 range writes NaN for its rows.
//   * one more 16-row tile of V^T holds the agent's V_lr slice (rows 0..r-1) and a row of ones:
//     O_lr^T and the softmax normaliser l come out of the same matrix-core product as O (l is the
//     sum of exactly the rounded P the products used). For r = 16 the ones row is a second tile.
//   * online softmax per query row and 32-key block in base 2, scale*log2(e) folded into one fma
//     per score; the row max is reduced over the 4 lanes sharing a row
//   * epilogue: gather O_lr of the row across its 4 lanes, add O_lr B_agent (B slice in LDS),
//     divide by l, store in the input type (bf16 round-to-nearest-even)
#include <type_traits>

#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMT = 4;                          // 16-row tiles per wave
constexpr int kRowsPerWG = 16 * kMT * kWaves;   // 256 query rows
constexpr int kBK = 64;                         // keys per tile

template <typename T> struct PrefillTypes {
    // element type of the P.V operands in LDS: fp16 bits for bf16 inputs, fp32 for fp32 inputs
    using TV = typename std::conditional<sizeof(T) == 2, uint16_t, float>::type;
    // P as an MFMA B operand: 8 fp16 values (4 dwords) or 8 fp32 values (one per 16x16x4 step)
    using PF = typename std::conditional<sizeof(T) == 2, H8, Vec<float, 8>>::type;
};

template <typename T, int D, int R>
struct PrefillShared {
    using TV = typename PrefillTypes<T>::TV;
    static constexpr int LDK = D + 16 / sizeof(T);    // K row (elements), padded by 16 bytes
    static constexpr int LDV = D + 16 / sizeof(TV);   // V row
    static constexpr int NAUX = R < 16 ? 1 : 2;       // V_lr + ones tiles
    static constexpr int LDA = kBK + 16 / sizeof(TV); // aux row (keys)
    T k[2][kBK * LDK];
    TV v[2][kBK * LDV];
    TV aux[2][NAUX * 16 * LDA];   // [tile row][key]: rows < R = V_lr columns, row R (or 16) = ones
    float b[R * D];               // B_agent[:, g*D .. g*D+D-1]
    int range_bad;
};

// fp32 -> fp16 bits (round to nearest even) of two values
__device__ __forceinline__ uint32_t h2(float lo, float hi) { return pack_f16x2(lo, hi); }

template <typename T, int D, int R>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
    using TV = typename PrefillTypes<T>::TV;
    using PF = typename PrefillTypes<T>::PF;
    using SH = PrefillShared<T, D, R>;
    constexpr int KCH = D / 32;           // Q.K reduction chunks
    constexpr int NKB = kBK / 32;         // 32-key blocks of P.V
    constexpr int NDT = D / 16;           // O^T tiles of 16 d-rows (d = NDT*s + t)
    constexpr int NAUX = SH::NAUX;
    constexpr int LDK = SH::LDK, LDV = SH::LDV, LDA = SH::LDA;
    constexpr int MT = kMT;
    constexpr int KF = kBK * D / 8 / kThreads;      // 8-element fragments per thread of K (and of V)
    static_assert(KF >= 1 && kBK * D / 8 % kThreads == 0, "tile split");
    constexpr int LF = kBK * R / 8;                 // 8-element fragments of the V_lr tile
    static_assert(LF <= kThreads, "V_lr tile split");

    __shared__ __align__(16) SH sh;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int G = p.G;
    const int n_kv = p.n_kv;
    const int64_t rows_total = p.L_C * G;
    const int nblk = int((rows_total + kRowsPerWG - 1) / kRowsPerWG);
    // KV head = w mod n_kv keeps one head per XCD when n_kv = 8; heavier (later) blocks start first
    const int g = blockIdx.x % n_kv;
    const int blk = nblk - 1 - int(blockIdx.x / n_kv);
    const int64_t R0 = int64_t(blk) * kRowsPerWG;

    const T* __restrict__ Qp = static_cast<const T*>(p.Q);
    const T* __restrict__ Kp = static_cast<const T*>(p.K);
    const T* __restrict__ Vp = static_cast<const T*>(p.V);
    const T* __restrict__ Lp = static_cast<const T*>(p.Vlr);
    const T* __restrict__ Bp = static_cast<const T*>(p.B);
    const int64_t kv_stride = int64_t(n_kv) * D;

    // ---- this lane's query rows (B operand column n of each 16-row tile)
    int qpos[MT];   // absolute positions (< 2^31, checked on the host)
    Vec<T, 8> qf[MT][KCH];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t r = R0 + (wv * MT + mt) * 16 + n;
        const bool ok = r < rows_total;
        const int64_t rc = ok ? r : rows_total - 1;
        const int64_t qi = rc / G;
        const int qh = int(rc - qi * G);
        qpos[mt] = int(p.L_P + qi);
        const T* qp = Qp + (qi * p.n_q + int64_t(g) * G + qh) * D + 8 * q;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            if (ok) qf[mt][i].load(qp + 32 * i);
            else qf[mt][i].zero();
        }
    }

    // ---- key range of the workgroup
    const int64_t i_min = R0 / G;
    const int64_t i_max = min<int64_t>(p.L_C - 1, (R0 + kRowsPerWG - 1) / G);
    const int64_t kv_end = p.L_P + i_max + 1;     // keys [0, kv_end) are visible to some row
    const int64_t full_end = p.L_P + i_min + 1;   // keys [0, full_end) are visible to every row
    const int n_tiles = int((kv_end + kBK - 1) / kBK);

    // ---- constants in LDS: B_agent slice (fp32), the ones / zero rows of the aux tiles
    for (int idx = tid; idx < R * D; idx += kThreads) {
        const int rr = idx / D, c = idx - rr * D;
        sh.b[idx] = to_f32<T>(Bp[(int64_t(p.agent) * R + rr) * kv_stride + int64_t(g) * D + c]);
    }
    for (int idx = tid; idx < 2 * (NAUX * 16 - R) * LDA; idx += kThreads) {
        const int buf = idx / ((NAUX * 16 - R) * LDA);
        const int rem = idx - buf * ((NAUX * 16 - R) * LDA);
        const int row = R + rem / LDA;
        float v = row == (R < 16 ? R : 16) ? 1.f : 0.f;
        TV tv;
        if constexpr (sizeof(T) == 2) tv = TV(h2(v, 0.f) & 0xffffu);
        else tv = v;
        sh.aux[buf][row * LDA + (rem % LDA)] = tv;
    }
    if (tid == 0) sh.range_bad = 0;
    float vmax = 0.f;   // largest |V| / |V_lr| staged by this thread (fp16 range check)

    // ---- tile fetch (registers) and store (LDS)
    Vec<T, 8> kpre[KF], vpre[KF], lpre;
    auto fetch = [&](int t) {
        const int64_t kb = int64_t(t) * kBK;
#pragma unroll
        for (int c = 0; c < KF; ++c) {
            const int f = tid + kThreads * c;
            const int key = f / (D / 8);
            const int d0 = (f - key * (D / 8)) * 8;
            const int64_t j = min<int64_t>(kb + key, kv_end - 1);   // rows past kv_end: a valid row, P = 0
            kpre[c].load(Kp + j * kv_stride + int64_t(g) * D + d0);
            vpre[c].load(Vp + j * kv_stride + int64_t(g) * D + d0);
        }
        if (tid < LF) {
            const int key = tid / (R / 8);
            const int r0 = (tid - key * (R / 8)) * 8;
            const int64_t j = min<int64_t>(kb + key, kv_end - 1);
            lpre.load(Lp + j * p.ld_vlr + int64_t(p.agent) * R + r0);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int c = 0; c < KF; ++c) {
            const int f = tid + kThreads * c;
            const int key = f / (D / 8);
            const int d0 = (f - key * (D / 8)) * 8;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint4*>(&sh.k[buf][key * LDK + d0]) = *reinterpret_cast<const uint4*>(kpre[c].w);
                uint32_t hv[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float lo = bf16_lo(vpre[c].w[e2]), hi = bf16_hi(vpre[c].w[e2]);
                    vmax = fmaxf(vmax, fmaxf(fabsf(lo), fabsf(hi)));
                    hv[e2] = h2(lo, hi);
                }
                *reinterpret_cast<uint4*>(&sh.v[buf][key * LDV + d0]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
            } else {
                float* kd = &sh.k[buf][key * LDK + d0];
                float* vd = &sh.v[buf][key * LDV + d0];
                *reinterpret_cast<float4*>(kd) = make_float4(kpre[c].v[0], kpre[c].v[1], kpre[c].v[2], kpre[c].v[3]);
                *reinterpret_cast<float4*>(kd + 4) = make_float4(kpre[c].v[4], kpre[c].v[5], kpre[c].v[6], kpre[c].v[7]);
                *reinterpret_cast<float4*>(vd) = make_float4(vpre[c].v[0], vpre[c].v[1], vpre[c].v[2], vpre[c].v[3]);
                *reinterpret_cast<float4*>(vd + 4) = make_float4(vpre[c].v[4], vpre[c].v[5], vpre[c].v[6], vpre[c].v[7]);
            }
        }
        if (tid < LF) {
            // the agent's V_lr slice goes to the aux tile transposed: row = rank column, column = key
            const int key = tid / (R / 8);
            const int r0 = (tid - key * (R / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = lpre.get(e);
                if constexpr (sizeof(T) == 2) {
                    vmax = fmaxf(vmax, fabsf(v));
                    sh.aux[buf][(r0 + e) * LDA + key] = TV(h2(v, 0.f) & 0xffffu);
                } else {
                    sh.aux[buf][(r0 + e) * LDA + key] = v;
                }
            }
        }
    };

    // ---- accumulators: O^T tiles 0..NDT-1 (row s of tile t is d = NDT*s + t), aux tiles (O_lr^T
    // rows 0..R-1, l in row R or in the second aux tile). Lane (q, n) holds rows 4q..4q+3 of each
    // tile for query row n.
    f32x4 oacc[MT][NDT];
    f32x4 xacc[MT][NAUX];
    float m_run[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m_run[mt] = -INFINITY;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[mt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < NAUX; ++x) xacc[mt][x] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = p.scale * kLog2e;

    fetch(0);
    store(0);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < n_tiles) fetch(t + 1);
        const int64_t kbase = int64_t(t) * kBK;
        const T* ks = sh.k[buf];
        const TV* vs = sh.v[buf];
        const TV* xs = sh.aux[buf];

        // the tile in two 32-key blocks, each: S^T = K Q^T, online softmax, O^T += V^T P^T
#pragma unroll 1
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
            const int64_t kblk = kbase + 32 * kb2;
            // scores: lane (q, n) holds keys 32kb2 + 16u + 4q + j (u = 0, 1; j = 0..3) of query row n
            f32x4 sacc[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int u = 0; u < 2; ++u) sacc[mt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < KCH; ++i) {
                    Vec<T, 8> ka;
                    ka.load(&ks[(32 * kb2 + 16 * u + n) * LDK + 32 * i + 8 * q]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) sacc[mt][u] = mma16x16x32(ka, qf[mt][i], sacc[mt][u]);
                }

            // online softmax per query row (raw scores; scale folded into the exponent)
            PF pf[MT];
            const bool need_mask = kblk + 32 > full_end;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (need_mask) {
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (kblk + 16 * u + 4 * q + j > qpos[mt]) sacc[mt][u][j] = -INFINITY;
                }
                float mx = -INFINITY;
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sacc[mt][u][j]);
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                // mnew is finite: key 0 (in the first block) is visible to every row
                const float mnew = fmaxf(m_run[mt], mx);
                const float alpha = fast_exp2((m_run[mt] - mnew) * sl2);
                m_run[mt] = mnew;
                const float mb = -mnew * sl2;
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(sacc[mt][e >> 2][e & 3], sl2, mb));
                if (__ballot(alpha != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) oacc[mt][dt] *= alpha;
#pragma unroll
                    for (int x = 0; x < NAUX; ++x) xacc[mt][x] *= alpha;
                }
                if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) pf[mt].w[w2] = h2(pv[2 * w2], pv[2 * w2 + 1]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pf[mt].v[e] = pv[e];
                }
            }

            // O^T += V^T P^T; the lane's 8 keys of the block are key(e) = 32kb2 + 16(e/4) + 4q + e%4
            if constexpr (sizeof(T) == 2) {
                // V rows of the lane's keys, d = NDT*n .. (fp16), then the 8 x NDT 16-bit transpose
                uint32_t vr[8][NDT / 2];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = 32 * kb2 + 16 * (e >> 2) + 4 * q + (e & 3);
                    const TV* src = &vs[key * LDV + NDT * n];
                    if constexpr (NDT == 8) {
                        const uint4 w4 = *reinterpret_cast<const uint4*>(src);
                        vr[e][0] = w4.x; vr[e][1] = w4.y; vr[e][2] = w4.z; vr[e][3] = w4.w;
                    } else {
                        const uint2 w2 = *reinterpret_cast<const uint2*>(src);
                        vr[e][0] = w2.x; vr[e][1] = w2.y;
                    }
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    H8 va;
                    const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) va.w[pp] = __builtin_amdgcn_perm(vr[2 * pp + 1][dt >> 1], vr[2 * pp][dt >> 1], sel);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) oacc[mt][dt] = mma16x16x32_f16(va, pf[mt], oacc[mt][dt]);
                }
#pragma unroll
                for (int x = 0; x < NAUX; ++x) {
                    H8 xa;
                    const TV* xr = &xs[(16 * x + n) * LDA + 32 * kb2 + 4 * q];
                    const uint2 lo = *reinterpret_cast<const uint2*>(xr);
                    const uint2 hi = *reinterpret_cast<const uint2*>(xr + 16);
                    xa.w[0] = lo.x; xa.w[1] = lo.y; xa.w[2] = hi.x; xa.w[3] = hi.y;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) xacc[mt][x] = mma16x16x32_f16(xa, pf[mt], xacc[mt][x]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = 32 * kb2 + 16 * (e >> 2) + 4 * q + (e & 3);
                    Vec<float, NDT> vv;
                    vv.load(&vs[key * LDV + NDT * n]);
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            oacc[mt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.v[dt], pf[mt].v[e], oacc[mt][dt], 0, 0, 0);
#pragma unroll
                    for (int x = 0; x < NAUX; ++x) {
                        const float xv = xs[(16 * x + n) * LDA + key];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            xacc[mt][x] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, pf[mt].v[e], xacc[mt][x], 0, 0, 0);
                    }
                }
            }
        }

        if (t + 1 < n_tiles) store(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O_lr and l of the row from its 4 lanes, O += O_lr B_agent, normalise, store
    if (sizeof(T) == 2 && !(vmax <= kF16Max)) sh.range_bad = 1;
    __syncthreads();
    const bool poison = sh.range_bad != 0;
    T* __restrict__ Op = static_cast<T*>(p.O);
    constexpr int LROW = R < 16 ? R : 16;   // aux row holding l (in the second tile when R = 16)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        // aux tile rows 4q'+j live in lane (q', n): gather all of them for row n
        float olr[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) olr[rr] = __shfl(xacc[mt][0][rr & 3], n + 16 * (rr >> 2));
        const float l = __shfl(xacc[mt][LROW / 16][LROW % 16 & 3], n + 16 * ((LROW % 16) >> 2));
        const int64_t r = R0 + (wv * MT + mt) * 16 + n;
        if (r >= rows_total) continue;
        const int64_t qi = r / G;
        const int qh = int(r - qi * G);
        T* orow = Op + (qi * p.n_q + int64_t(g) * G + qh) * D;
        const float inv = poison ? __builtin_nanf("") : 1.f / l;
        // lane (q, n) holds O^T rows 4q+j of tile dt, i.e. d = NDT*(4q+j) + dt: the 4*NDT contiguous
        // values d = 4*NDT*q .. 4*NDT*q + 4*NDT - 1
        float o[4 * NDT];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int d = NDT * (4 * q + j) + dt;
                float acc = oacc[mt][dt][j];
#pragma unroll
                for (int rr = 0; rr < R; ++rr) acc = fmaf(olr[rr], sh.b[rr * D + d], acc);
                o[NDT * j + dt] = acc * inv;
            }
        T* dst = orow + 4 * NDT * q;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int c = 0; c < NDT / 2; ++c) {
                uint4 w;
                w.x = pack_bf16x2(o[8 * c + 0], o[8 * c + 1]);
                w.y = pack_bf16x2(o[8 * c + 2], o[8 * c + 3]);
                w.z = pack_bf16x2(o[8 * c + 4], o[8 * c + 5]);
                w.w = pack_bf16x2(o[8 * c + 6], o[8 * c + 7]);
                *reinterpret_cast<uint4*>(dst + 8 * c) = w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < NDT; ++c)
                *reinterpret_cast<float4*>(dst + 4 * c) = make_float4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
        }
    }
}

template <typename T, int D, int R>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
    const int64_t rows = p.L_C * p.G;
    const int64_t nblk = (rows + kRowsPerWG - 1) / kRowsPerWG;
    hipLaunchKernelGGL((prefill_kernel<T, D, R>), dim3(unsigned(nblk * p.n_kv)), dim3(kThreads), 0, stream, p);
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

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    return p.bf16 ? dispatch_d<bf16>(p, stream) : dispatch_d<float>(p, stream);
}

}  // namespace lra
