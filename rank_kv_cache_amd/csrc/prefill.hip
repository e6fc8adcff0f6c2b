// Flash-LoRA-Attention causal chunked prefill for gfx950.
//
// Method (LRAgent page, "method steps" (3)-(4) and "core method"): stream key/value tiles with an
// online softmax; next to the base output O accumulate the rank-r output O_lr = P V_lr (the agent's
// column slice of the LR cache) from the same probability tile; after the last tile apply the
// up-projection O <- O + O_lr B_agent once per query row and normalise. The chunk's L_C queries sit
// at positions L_P .. L_P+L_C-1 after the reused context (PReCache summary page), causal mask
// bottom-right aligned.
//
// gfx950 mapping (16x16x32 matrix-core steps with fp32 accumulation; fp32 inputs run the same
// template on 16x16x4 fp32 steps):
//   * one workgroup = 4 waves = 128 "query rows" of one KV head; a query row is one (query, head)
//     pair of that head's group, so all G heads of a group share every K/V tile (grouped-query)
//   * each wave owns MT tiles of 16 query rows; its queries stay in registers as MFMA B operands
//   * S^T = K Q^T: A operand = 16 keys x 8 d-elements from the K tile in LDS; output lane (r, n)
//     holds keys 4r..4r+3 (of each 16) for query row n
//   * that layout is already the B operand of O^T = V^T P^T: two 16-key groups give each lane the
//     8 keys of its reduction slot, so P never leaves the lane; V is staged transposed in LDS
//   * bf16 inputs: Q.K runs on bf16 steps; P.V runs on fp16 steps, with V and V_lr converted
//     bf16 -> fp16 while they are staged (exact for |v| <= 65504) and P rounded to fp16, whose 11
//     significant bits keep the product within the bf16 tolerance even when a row attends only a
//     few keys. A workgroup that meets a value beyond the fp16 range writes NaN for its rows.
//   * the agent's V_lr slice is staged as 16 extra rows of V^T (rows >= r are zero): O_lr^T comes
//     out of the same P tile as one more 16-row output tile
//   * online softmax per query row in base 2 (scale*log2(e) folded in): row max over the 4 lanes
//     sharing a row, running sum kept per lane and reduced once at the end
//   * the next K/V/V_lr tile is fetched into registers while the current one is multiplied
//   * epilogue: gather O_lr of the row across its 4 lanes, add O_lr B_agent (B slice in LDS),
//     divide by l, store in the input type (bf16 round-to-nearest-even)
#include <type_traits>

#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWG = 128;   // query rows per workgroup
constexpr int kMT = 2;            // 16-row tiles per wave

template <typename T> struct PrefillTile {
    static constexpr int BK = sizeof(T) == 2 ? 64 : 32;   // keys per tile
    using TV = typename std::conditional<sizeof(T) == 2, uint16_t, float>::type;
};

template <typename T, int D, int R>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
    constexpr int BK = PrefillTile<T>::BK;
    constexpr int KCH = D / 32;         // Q.K reduction chunks
    constexpr int NU = BK / 16;         // 16-key subtiles
    constexpr int NKB = BK / 32;        // 32-key blocks of P.V
    constexpr int NDT = D / 16;         // 16-column output tiles of O^T (plus one for O_lr^T)
    constexpr int LDK = D + 8;          // K tile row (elements), padded
    constexpr int LDV = BK + 8;         // V^T row (elements), padded
    constexpr int MT = kMT;
    constexpr int FK = BK * D / 8 / kThreads;   // 8-element fragments per thread per K (or V) tile
    static_assert(FK >= 1 && BK * D / 8 % kThreads == 0, "tile split");
    constexpr int FL = BK * R / 8;              // 8-element fragments of the V_lr tile

    using TV = typename PrefillTile<T>::TV;   // P.V operand type in LDS (fp16 bits for bf16 inputs)
    __shared__ __align__(16) T k_s[BK * LDK];
    __shared__ __align__(16) TV vt_s[(D + 16) * LDV];
    __shared__ float b_s[R * D];
    __shared__ int range_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, n = lane & 15, rg = lane >> 4;
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
    int64_t qpos[MT];
    Vec<T, 8> qf[MT][KCH];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t r = R0 + (wv * MT + mt) * 16 + n;
        const bool ok = r < rows_total;
        const int64_t rc = ok ? r : rows_total - 1;
        const int64_t qi = rc / G;
        const int qh = int(rc - qi * G);
        qpos[mt] = p.L_P + qi;
        const T* qp = Qp + (qi * p.n_q + int64_t(g) * G + qh) * D + 8 * rg;
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
    const int n_tiles = int((kv_end + BK - 1) / BK);

    // ---- B_agent[:, g*D : g*D+D] as fp32 in LDS
    for (int idx = tid; idx < R * D; idx += kThreads) {
        const int rr = idx / D, c = idx - rr * D;
        b_s[idx] = to_f32<T>(Bp[(int64_t(p.agent) * R + rr) * kv_stride + int64_t(g) * D + c]);
    }
    // rows D+R .. D+15 of V^T stay zero
    for (int idx = tid; idx < (16 - R) * LDV; idx += kThreads) vt_s[(D + R) * LDV + idx] = TV(0);
    if (tid == 0) range_bad = 0;
    float vmax = 0.f;   // largest |V| / |V_lr| staged by this thread (fp16 range check)

    // ---- tile fetch (registers) and store (LDS)
    Vec<T, 8> kpre[FK], vpre[FK], lpre;
    auto fetch = [&](int t) {
        const int64_t kb = int64_t(t) * BK;
#pragma unroll
        for (int c = 0; c < FK; ++c) {
            const int f = tid + kThreads * c;
            const int key = f / (D / 8);
            const int d0 = (f - key * (D / 8)) * 8;
            const int64_t j = kb + key;
            if (j < kv_end) {
                kpre[c].load(Kp + j * kv_stride + int64_t(g) * D + d0);
                vpre[c].load(Vp + j * kv_stride + int64_t(g) * D + d0);
            } else {
                kpre[c].zero();
                vpre[c].zero();
            }
        }
        if (tid < FL) {
            const int key = tid / (R / 8);
            const int r0 = (tid - key * (R / 8)) * 8;
            const int64_t j = kb + key;
            if (j < kv_end) lpre.load(Lp + j * p.ld_vlr + int64_t(p.agent) * R + r0);
            else lpre.zero();
        }
    };
    // write 8 consecutive elements of one key as 8 rows of the transposed tile (fp16 for bf16 inputs)
    auto store_col = [&](const Vec<T, 8>& v, int row0, int key) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float lo = bf16_lo(v.w[e2]), hi = bf16_hi(v.w[e2]);
                vmax = fmaxf(vmax, fmaxf(fabsf(lo), fabsf(hi)));
                const uint32_t h2 = pack_f16x2(lo, hi);
                vt_s[(row0 + 2 * e2) * LDV + key] = uint16_t(h2 & 0xffffu);
                vt_s[(row0 + 2 * e2 + 1) * LDV + key] = uint16_t(h2 >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vt_s[(row0 + e) * LDV + key] = v.v[e];
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int c = 0; c < FK; ++c) {
            const int f = tid + kThreads * c;
            const int key = f / (D / 8);
            const int d0 = (f - key * (D / 8)) * 8;
            if constexpr (sizeof(T) == 2) *reinterpret_cast<uint4*>(&k_s[key * LDK + d0]) = *reinterpret_cast<const uint4*>(kpre[c].w);
            else {
                *reinterpret_cast<float4*>(&k_s[key * LDK + d0]) = make_float4(kpre[c].v[0], kpre[c].v[1], kpre[c].v[2], kpre[c].v[3]);
                *reinterpret_cast<float4*>(&k_s[key * LDK + d0 + 4]) = make_float4(kpre[c].v[4], kpre[c].v[5], kpre[c].v[6], kpre[c].v[7]);
            }
            store_col(vpre[c], d0, key);
        }
        if (tid < FL) {
            const int key = tid / (R / 8);
            const int r0 = (tid - key * (R / 8)) * 8;
            store_col(lpre, D + r0, key);
        }
    };

    // ---- accumulators: O^T tiles 0..NDT-1, O_lr^T tile NDT; lane (rg, n) holds rows 4rg+j of each
    f32x4 oacc[MT][NDT + 1];
    float m_run[MT], l_run[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m_run[mt] = -INFINITY;
        l_run[mt] = 0.f;
#pragma unroll
        for (int dt = 0; dt <= NDT; ++dt) oacc[mt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = p.scale * kLog2e;

    fetch(0);
    store();
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        if (t + 1 < n_tiles) fetch(t + 1);
        const int64_t kbase = int64_t(t) * BK;
        const bool need_mask = kbase + BK > full_end;

        // S^T = K Q^T for the wave's query rows
        f32x4 sacc[MT][NU];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int u = 0; u < NU; ++u) sacc[mt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                Vec<T, 8> ka;
                ka.load(&k_s[(16 * u + n) * LDK + 32 * i + 8 * rg]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) sacc[mt][u] = mma16x16x32(ka, qf[mt][i], sacc[mt][u]);
            }

        // online softmax per query row; P packed as the B operand of O^T = V^T P^T
        using PF = typename std::conditional<sizeof(T) == 2, H8, Vec<float, 8>>::type;
        PF pf[MT][NKB];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float sv[NU][4];
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float s = sacc[mt][u][j] * sl2;
                    if (need_mask && kbase + 16 * u + 4 * rg + j > qpos[mt]) s = -INFINITY;
                    sv[u][j] = s;
                    mx = fmaxf(mx, s);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m_run[mt], mx);   // finite: key 0 is visible to every row
            const float alpha = fast_exp2(m_run[mt] - mnew);
            m_run[mt] = mnew;
            float ls = 0.f;
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float e = fast_exp2(sv[u][j] - mnew);
                    sv[u][j] = e;
                    ls += e;
                }
            l_run[mt] = alpha * l_run[mt] + ls;
#pragma unroll
            for (int dt = 0; dt <= NDT; ++dt) oacc[mt][dt] *= alpha;
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2) {
                if constexpr (sizeof(T) == 2) {
                    pf[mt][kb2].w[0] = pack_f16x2(sv[2 * kb2][0], sv[2 * kb2][1]);
                    pf[mt][kb2].w[1] = pack_f16x2(sv[2 * kb2][2], sv[2 * kb2][3]);
                    pf[mt][kb2].w[2] = pack_f16x2(sv[2 * kb2 + 1][0], sv[2 * kb2 + 1][1]);
                    pf[mt][kb2].w[3] = pack_f16x2(sv[2 * kb2 + 1][2], sv[2 * kb2 + 1][3]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pf[mt][kb2].v[j] = sv[2 * kb2][j];
                        pf[mt][kb2].v[4 + j] = sv[2 * kb2 + 1][j];
                    }
                }
            }
        }

        // O^T += V^T P^T and O_lr^T += V_lr^T P^T: slot rg of a 32-key block = keys 4rg..4rg+3, 16+4rg..16+4rg+3
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
            for (int dt = 0; dt <= NDT; ++dt) {
                PF va;
                const TV* vrow = &vt_s[(16 * dt + n) * LDV + 32 * kb2 + 4 * rg];
                if constexpr (sizeof(T) == 2) {
                    const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
                    va.w[0] = lo.x; va.w[1] = lo.y; va.w[2] = hi.x; va.w[3] = hi.y;
                } else {
                    const float4 lo = *reinterpret_cast<const float4*>(vrow);
                    const float4 hi = *reinterpret_cast<const float4*>(vrow + 16);
                    va.v[0] = lo.x; va.v[1] = lo.y; va.v[2] = lo.z; va.v[3] = lo.w;
                    va.v[4] = hi.x; va.v[5] = hi.y; va.v[6] = hi.z; va.v[7] = hi.w;
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if constexpr (sizeof(T) == 2) oacc[mt][dt] = mma16x16x32_f16(va, pf[mt][kb2], oacc[mt][dt]);
                    else oacc[mt][dt] = mma16x16x32(va, pf[mt][kb2], oacc[mt][dt]);
                }
            }

        __syncthreads();
        if (t + 1 < n_tiles) {
            store();
            __syncthreads();
        }
    }

    // ---- epilogue: l over the row's 4 lanes, O += O_lr B_agent, normalise, store
    if (sizeof(T) == 2 && !(vmax <= kF16Max)) range_bad = 1;
    __syncthreads();
    const bool poison = range_bad != 0;
    T* __restrict__ Op = static_cast<T*>(p.O);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        float l = l_run[mt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        float olr[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) olr[rr] = __shfl(oacc[mt][NDT][rr & 3], n + 16 * (rr >> 2));
        const int64_t r = R0 + (wv * MT + mt) * 16 + n;
        if (r >= rows_total) continue;
        const int64_t qi = r / G;
        const int qh = int(r - qi * G);
        T* orow = Op + (qi * p.n_q + int64_t(g) * G + qh) * D;
        const float inv = poison ? __builtin_nanf("") : 1.f / l;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            float o4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = 16 * dt + 4 * rg + j;
                float acc = oacc[mt][dt][j];
#pragma unroll
                for (int rr = 0; rr < R; ++rr) acc = fmaf(olr[rr], b_s[rr * D + col], acc);
                o4[j] = acc * inv;
            }
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * rg) = make_uint2(pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3]));
            } else {
                *reinterpret_cast<float4*>(orow + 16 * dt + 4 * rg) = make_float4(o4[0], o4[1], o4[2], o4[3]);
            }
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
