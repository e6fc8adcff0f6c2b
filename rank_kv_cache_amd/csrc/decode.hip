// Flash-LoRA-Attention decode for gfx950: split along the key axis, then a log-sum-exp combine.
//
// Method (LRAgent page, "method steps" (3)-(4)): stream key/value tiles, keep the online-softmax
// statistics, accumulate the base output O and the rank-r output O_lr from the agent's LR cache,
// and only after the last tile apply O <- O + O_lr B_agent and normalise. The rank-r accumulation
// is what makes the reordering pay: the per-key work of the LR path is r multiply-adds instead of
// d_head (LRAgent page, "core method" / "technical novelty": associativity moves the d_out-wide
// product out of the key loop).
//
// One kernel, one workgroup per (request b, KV head g, key split s), 4 waves.
//   * the G query heads of KV head g share every K/V/V_lr load (grouped-query attention)
//   * S = Q K^T on the matrix cores: A operand = the G queries (rows padded to 16), B operand =
//     16 keys, 8 contiguous d-elements per lane (128-bit loads)
//   * online softmax per 64-key tile in the base-2 domain (log2(e) folded into the scale),
//     row maxima/sums with DPP inside 16-lane rows
//   * P.V_base and P.V_lr on the vector ALUs: lane (slot, c) owns d-columns c*VEC.. of one key out
//     of every 4, with P broadcast through LDS; keys past the split end are clamped to a valid row
//     (finite data) and get P = 0, so no row outside [kv_start, kv_start+kv_len) is ever read
//   * the 4 waves merge their states in LDS and write one fp32 partial (m, l, O, O_lr) per query head
//   * the split that arrives last for its (request, KV head) (release fence + arrival counter) merges
//     the partials with weights 2^(m_s - max m), applies O = (O + O_lr B_agent[:, g*d:(g+1)*d]) / l
//     once per query row, rounds to the output type and zeroes the counter for the next call.
//     Empty requests get zeros and requests with an invalid range or agent get NaN (split 0 writes them).
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <typename T, int D, int R, int GP>
struct DecodeCfg {
    static constexpr int VEC = D / 16;        // d-columns per lane in the P.V step
    static constexpr int KCH = D / 32;        // 32-wide reduction chunks of Q.K
    static constexpr int NU = 4;              // 16-key subtiles per wave tile
    static constexpr int TK = 16 * NU;        // keys per wave tile
    static constexpr int NP = GP * R / 16;    // O_lr elements per lane
    static_assert(GP == 4 || GP == 8, "padded group");
    static_assert(NP >= 2 && R % NP == 0, "O_lr lane split");
};

__device__ __forceinline__ bool decode_request_ok(int64_t start, int32_t len, int32_t a, const DecodeParams& p) {
    return len >= 0 && int64_t(len) <= p.max_kv_len && start >= 0 && start + int64_t(len) <= p.kv_rows &&
           a >= 0 && a < p.n_agents;
}

template <typename T, int D, int R, int GP>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
    using C = DecodeCfg<T, D, R, GP>;
    constexpr int VEC = C::VEC, KCH = C::KCH, NU = C::NU, TK = C::TK, NP = C::NP;

    __shared__ float plds[kWaves][TK][16];          // probabilities of the current tile, per wave
    __shared__ float red_o[kWaves][GP][D + R];      // per-wave O | O_lr after the slot reduction
    __shared__ float red_m[kWaves][GP], red_l[kWaves][GP];

    // XCD-aware order: workgroup w runs on XCD w % 8. All KV heads of one (request, split) get the
    // same w % 8, so the LR rows they all read stay in one L2.
    const int w = blockIdx.x;
    const int xcd = w & 7;
    const int rest = w >> 3;
    const int g = rest % p.n_kv;
    const int bs = (rest / p.n_kv) * 8 + xcd;
    if (bs >= p.batch * p.n_split) return;
    const int b = bs / p.n_split;
    const int s = bs - b * p.n_split;

    const int64_t start = p.kv_start[b];
    const int32_t len = p.kv_len[b];
    const int32_t a = p.agent[b];
    const int G = p.G;
    const bool ok = decode_request_ok(start, len, a, p);
    if (!ok || len == 0) {
        // no key to attend: zeros for an empty range, NaN for an invalid request (split 0 writes them)
        if (s == 0) {
            T* Op = static_cast<T*>(p.O) + (int64_t(b) * p.n_q + int64_t(g) * G) * D;
            const T fill = from_f32<T>(ok ? 0.f : __builtin_nanf(""));
            for (int idx = threadIdx.x; idx < G * D; idx += kThreads) Op[idx] = fill;
        }
        return;
    }
    const int k0 = s * p.chunk;
    if (k0 >= len) return;                                   // splits past the request's end do nothing
    const int k1 = min(k0 + p.chunk, len);
    const int ns = (len + p.chunk - 1) / p.chunk;            // live splits of this request

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n = lane & 15;   // MFMA row/column; P.V column group
    const int rg = lane >> 4;  // MFMA reduction group; P.V key slot

    const T* __restrict__ Kp = static_cast<const T*>(p.K);
    const T* __restrict__ Vp = static_cast<const T*>(p.V);
    const T* __restrict__ Lp = static_cast<const T*>(p.Vlr);
    const T* __restrict__ Qp = static_cast<const T*>(p.Q);
    const int64_t row_stride = int64_t(p.n_kv) * D;

    // queries of the group as the MFMA A operand (rows >= G are zero)
    Vec<T, 8> qf[KCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        if (n < G) qf[i].load(Qp + (int64_t(b) * p.n_q + int64_t(g) * G + n) * D + 32 * i + 8 * rg);
        else qf[i].zero();
    }

    const int lr_p0 = n * NP;
    const int h_lr = lr_p0 / R;   // head of this lane's O_lr elements
    const int rr0 = lr_p0 % R;    // first rank column of them
    const int64_t lr_col = int64_t(a) * R + rr0;

    float m_run[4], l_run[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.f; }
    float o[GP][VEC];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = 0.f;
    float olr[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) olr[i] = 0.f;

    const float sl2 = p.scale * kLog2e;

    for (int kt = k0 + wv * TK; kt < k1; kt += kWaves * TK) {
        // ---- loads: K as MFMA B operands, V and V_lr in the P.V layout; rows past k1 clamp to k1-1
        Vec<T, 8> kf[NU][KCH];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int kr = min(kt + 16 * u + n, k1 - 1);
            const T* kp = Kp + (start + kr) * row_stride + int64_t(g) * D + 8 * rg;
#pragma unroll
            for (int i = 0; i < KCH; ++i) kf[u][i].load(kp + 32 * i);
        }
        Vec<T, VEC> vf[TK / 4];
        Vec<T, NP> lf[TK / 4];
#pragma unroll
        for (int t = 0; t < TK / 4; ++t) {
            const int64_t row = start + min(kt + 4 * t + rg, k1 - 1);
            vf[t].load(Vp + row * row_stride + int64_t(g) * D + VEC * n);
            lf[t].load(Lp + row * p.ld_vlr + lr_col);
        }

        // ---- scores on the matrix cores: lane holds S[head 4*rg+j][key kt+16u+n]
        float sc[NU][4];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KCH; ++i) acc = mma16x16x32(qf[i], kf[u][i], acc);
            const bool live = (kt + 16 * u + n) < k1;
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[u][j] = live ? acc[j] * sl2 : -INFINITY;
        }

        // ---- online softmax (base 2)
        float alpha[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float mt = sc[0][j];
#pragma unroll
            for (int u = 1; u < NU; ++u) mt = fmaxf(mt, sc[u][j]);
            mt = row16_max(mt);
            const float mnew = fmaxf(m_run[j], mt);  // finite: key kt is live
            alpha[j] = fast_exp2(m_run[j] - mnew);
            float ls = 0.f;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                sc[u][j] = fast_exp2(sc[u][j] - mnew);
                ls += sc[u][j];
            }
            l_run[j] = alpha[j] * l_run[j] + ls;
            m_run[j] = mnew;
        }

        wave_sync();
#pragma unroll
        for (int u = 0; u < NU; ++u)
            *reinterpret_cast<float4*>(&plds[wv][16 * u + n][4 * rg]) = make_float4(sc[u][0], sc[u][1], sc[u][2], sc[u][3]);
        wave_sync();

        // ---- rescale the accumulators by 2^(m_old - m_new) of each head (wave-uniform values)
        float ah[GP];
        bool any = false;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            ah[h] = readlane_f(alpha[h & 3], 16 * (h >> 2));
            any |= ah[h] != 1.f;
        }
        if (any) {
            float alr = ah[0];
#pragma unroll
            for (int h = 1; h < GP; ++h) alr = (h_lr == h) ? ah[h] : alr;
#pragma unroll
            for (int h = 0; h < GP; ++h)
#pragma unroll
                for (int e = 0; e < VEC; ++e) o[h][e] *= ah[h];
#pragma unroll
            for (int i = 0; i < NP; ++i) olr[i] *= alr;
        }

        // ---- P.V_base and P.V_lr: slot rg takes keys 4t+rg
#pragma unroll
        for (int t = 0; t < TK / 4; ++t) {
            const int kl = 4 * t + rg;
            float ph[GP];
            const float4 p0 = *reinterpret_cast<const float4*>(&plds[wv][kl][0]);
            ph[0] = p0.x; ph[1] = p0.y; ph[2] = p0.z; ph[3] = p0.w;
            if constexpr (GP == 8) {
                const float4 p1 = *reinterpret_cast<const float4*>(&plds[wv][kl][4]);
                ph[4] = p1.x; ph[5] = p1.y; ph[6] = p1.z; ph[7] = p1.w;
            }
            const float plr = plds[wv][kl][h_lr];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float v = vf[t].get(e);
#pragma unroll
                for (int h = 0; h < GP; ++h) o[h][e] = fmaf(ph[h], v, o[h][e]);
            }
#pragma unroll
            for (int i = 0; i < NP; ++i) olr[i] = fmaf(plr, lf[t].get(i), olr[i]);
        }
    }

    // ---- per-wave reduction: l over the 16 lanes of a row, O / O_lr over the 4 key slots
#pragma unroll
    for (int j = 0; j < 4; ++j) l_run[j] = row16_sum(l_run[j]);
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float v = o[h][e];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            o[h][e] = v;
        }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        float v = olr[i];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        olr[i] = v;
    }
    if (rg == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < VEC; ++e) red_o[wv][h][VEC * n + e] = o[h][e];
#pragma unroll
        for (int i = 0; i < NP; ++i) red_o[wv][h_lr][D + rr0 + i] = olr[i];
    }
    if (n == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = 4 * rg + j;
            if (h < GP) { red_m[wv][h] = m_run[j]; red_l[wv][h] = l_run[j]; }
        }
    }
    __syncthreads();

    // ---- merge the 4 waves (weights 2^(m_w - M)) and write this split's partial per query head
    const int64_t bh0 = int64_t(b) * p.n_q + int64_t(g) * G;
    for (int idx = threadIdx.x; idx < G * (D + R); idx += kThreads) {
        const int h = idx / (D + R);
        const int col = idx - h * (D + R);
        float M = red_m[0][h];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) M = fmaxf(M, red_m[v][h]);
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float mv = red_m[v][h];
            const float wgt = (mv == -INFINITY) ? 0.f : fast_exp2(mv - M);
            acc = fmaf(wgt, red_o[v][h][col], acc);
            L = fmaf(wgt, red_l[v][h], L);
        }
        const int64_t rec = (bh0 + h) * p.n_split + s;
        p.ws_o[rec * (D + R) + col] = acc;
        if (col == 0) {
            p.ws_ml[rec * 2 + 0] = M;
            p.ws_ml[rec * 2 + 1] = L;
        }
    }

    // ---- the last split of (b, g) to arrive merges all splits of the group's query heads
    __shared__ int last_s;
    __threadfence();
    __syncthreads();
    uint32_t* counter = p.ws_count + int64_t(b) * p.n_kv + g;
    if (threadIdx.x == 0) last_s = atomicAdd(counter, 1u) == uint32_t(ns - 1);
    __syncthreads();
    if (!last_s) return;
    __threadfence();

    // per-head maximum and normaliser over the live splits (one wave per head)
    for (int h = wv; h < G; h += kWaves) {
        const int64_t rec0 = (bh0 + h) * p.n_split;
        float M = -INFINITY;
        for (int sidx = lane; sidx < ns; sidx += 64) M = fmaxf(M, p.ws_ml[(rec0 + sidx) * 2]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        float L = 0.f;
        for (int sidx = lane; sidx < ns; sidx += 64) {
            const float* ml = p.ws_ml + (rec0 + sidx) * 2;
            L = fmaf(fast_exp2(ml[0] - M), ml[1], L);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
        if (lane == 0) { red_m[0][h] = M; red_l[0][h] = L; }
    }
    __syncthreads();
    // weighted sums of O | O_lr over the splits
    for (int idx = threadIdx.x; idx < G * (D + R); idx += kThreads) {
        const int h = idx / (D + R);
        const int col = idx - h * (D + R);
        const int64_t rec0 = (bh0 + h) * p.n_split;
        const float M = red_m[0][h];
        float acc = 0.f;
        for (int sidx = 0; sidx < ns; ++sidx)
            acc = fmaf(fast_exp2(p.ws_ml[(rec0 + sidx) * 2] - M), p.ws_o[(rec0 + sidx) * (D + R) + col], acc);
        red_o[1][h][col] = acc;
    }
    __syncthreads();
    // up-projection once per query row: O += O_lr B_agent[:, g*D + col], then normalise and store
    T* __restrict__ Op = static_cast<T*>(p.O);
    const T* __restrict__ Bp = static_cast<const T*>(p.B) + int64_t(a) * R * row_stride + int64_t(g) * D;
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int h = idx / D;
        const int col = idx - h * D;
        float acc = red_o[1][h][col];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) acc = fmaf(red_o[1][h][D + rr], to_f32<T>(Bp[int64_t(rr) * row_stride + col]), acc);
        Op[(bh0 + h) * D + col] = from_f32<T>(acc / red_l[0][h]);
    }
    if (threadIdx.x == 0) *counter = 0u;
}

template <typename T, int D, int R, int GP>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
    const int64_t bs = int64_t(p.batch) * p.n_split;
    const int64_t groups = (bs + 7) / 8;
    const int64_t n_wg = groups * 8 * p.n_kv;
    hipLaunchKernelGGL((decode_split_kernel<T, D, R, GP>), dim3(unsigned(n_wg)), dim3(kThreads), 0, stream, p);
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
