// Key expansion for LoRA on the key projection (the qkvo configuration) on gfx950.
//
// LRAgent page (limitations) and PReCache summary page (which adapt only q and v by default): when
// the key projection carries LoRA too, an agent's key is K_base + RoPE(K_lr B_k). The rotation
// sits between the up-projection and the dot product with the query, so the rank-r part cannot be
// folded behind the softmax the way the value side is; each key has to be expanded and rotated at
// its own position before the scores. A causal prefill reads every key once per 128-row piece of
// queries, so the expansion runs once per call in this pass and the attention kernel reads the
// result: Ka[j, g] = fp16(K_base[j, g] + RoPE_j(K_lr[j, agent] B_k[agent][:, g])).
//
// Rotation (rotate-half pairing): element i < d/2 pairs with i + d/2; with c = cos[j, i] and
// s = sin[j, i], (y_i, y_{i+d/2}) -> (y_i c - y_{i+d/2} s, y_{i+d/2} c + y_i s).
//
// Mapping: one workgroup = one 64-key tile of one KV head, 256 threads; a thread owns 8 consecutive
// dims i .. i+7 of the low half and their partners i+d/2 .. of one key (d/16 threads per key), so
// every K_base, table and output access is a 16-byte run and the threads of a key cover its row
// contiguously. The rank-r product (r = 8 or 16 multiply-adds per element) runs on the vector ALU
// from the key's K_lr row (one broadcast load) and the B_k slice staged in LDS. The sum is taken in
// fp32 and rounded once to fp16; a tile that meets |value| > 65504 or a NaN sets its flag.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kThreads = 256;
constexpr int kRankPad = 16;   // the 16x16x16 steps' reduction depth
constexpr int kHeads = 8;      // KV heads per workgroup of the key score pass

template <int D, int R>
__global__ __launch_bounds__(kThreads) void key_expand_kernel(KeyExpandParams p) {
    constexpr int TPK = D / 16;                  // threads per key
    constexpr int KPI = kThreads / TPK;          // keys per pass
    static_assert(kKeyTile % KPI == 0, "tile split");
    __shared__ float bk[R][D];                   // the agent's B_k slice of this head, fp32

    const int tile = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t kv_stride = int64_t(p.n_kv) * D;
    const uint16_t* __restrict__ Bk = static_cast<const uint16_t*>(p.Bk) + int64_t(p.agent) * R * kv_stride + int64_t(g) * D;
    for (int idx = tid; idx < R * D; idx += kThreads) {
        const int r = idx / D, d = idx - r * D;
        bk[r][d] = bf16_to_f32(Bk[int64_t(r) * kv_stride + d]);
    }
    __syncthreads();

    const int i0 = 8 * (tid % TPK);              // first dim of the low half
    bool out_of_range = false;                   // |value| > 65504 or NaN (which compares false)
#pragma unroll
    for (int pass = 0; pass < kKeyTile / KPI; ++pass) {
        const int64_t j = int64_t(tile) * kKeyTile + pass * KPI + tid / TPK;
        if (j >= p.n_rows) break;
        const uint16_t* krow = static_cast<const uint16_t*>(p.K) + j * kv_stride + int64_t(g) * D;
        Vec<bf16, 8> lr[R / 8];   // the key's K_lr columns of the agent (same address for all its threads)
#pragma unroll
        for (int h = 0; h < R / 8; ++h) lr[h].load(static_cast<const bf16*>(p.Klr) + j * p.ld_klr + int64_t(p.agent) * R + 8 * h);
        float klr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) klr[r] = lr[r / 8].get(r % 8);
        const uint4 klo = *reinterpret_cast<const uint4*>(krow + i0);
        const uint4 khi = *reinterpret_cast<const uint4*>(krow + i0 + D / 2);
        const float4 c0 = *reinterpret_cast<const float4*>(p.rope_cos + j * (D / 2) + i0);
        const float4 c1 = *reinterpret_cast<const float4*>(p.rope_cos + j * (D / 2) + i0 + 4);
        const float4 s0 = *reinterpret_cast<const float4*>(p.rope_sin + j * (D / 2) + i0);
        const float4 s1 = *reinterpret_cast<const float4*>(p.rope_sin + j * (D / 2) + i0 + 4);
        const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const uint32_t wl[4] = {klo.x, klo.y, klo.z, klo.w}, wh[4] = {khi.x, khi.y, khi.z, khi.w};
        uint32_t ol[4], oh[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float lo[2], hi[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int x = 2 * w + e;
                float ylo = 0.f, yhi = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    ylo = fmaf(klr[r], bk[r][i0 + x], ylo);
                    yhi = fmaf(klr[r], bk[r][i0 + x + D / 2], yhi);
                }
                const float kl0 = e ? bf16_hi(wl[w]) : bf16_lo(wl[w]);
                const float kh0 = e ? bf16_hi(wh[w]) : bf16_lo(wh[w]);
                lo[e] = kl0 + (ylo * cv[x] - yhi * sv[x]);
                hi[e] = kh0 + (yhi * cv[x] + ylo * sv[x]);
                out_of_range = out_of_range || !(fabsf(lo[e]) <= kF16Max) || !(fabsf(hi[e]) <= kF16Max);
            }
            ol[w] = pack_f16x2(lo[0], lo[1]);
            oh[w] = pack_f16x2(hi[0], hi[1]);
        }
        uint16_t* orow = static_cast<uint16_t*>(p.Ka) + j * kv_stride + int64_t(g) * D;
        *reinterpret_cast<uint4*>(orow + i0) = make_uint4(ol[0], ol[1], ol[2], ol[3]);
        *reinterpret_cast<uint4*>(orow + i0 + D / 2) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
    }
    const int any_bad = __syncthreads_or(out_of_range);
    if (tid == 0) p.flags[int64_t(tile) * p.n_kv + g] = any_bad;
}

template <int D>
void launch_d(const KeyExpandParams& p, hipStream_t stream) {
    const dim3 grid(unsigned((p.n_rows + kKeyTile - 1) / kKeyTile), unsigned(p.n_kv));
    if (p.rank == 8) hipLaunchKernelGGL((key_expand_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((key_expand_kernel<D, 16>), grid, dim3(kThreads), 0, stream, p);
}

// ---- decode: the rank-r part of the scores, one pass over every request's keys
//
// A decode reads each key once, so the attention kernel could expand keys as it streams them, but
// the rotary tables (2 x d/2 floats per position) would then be read once per KV head and the
// extra registers do not fit the decode kernel. This pass computes, per request and 256-key
// block, S = Q . RoPE(K_lr B_k) for all query heads and writes it as fp16 (2 bytes per score);
// the decode kernel adds it to the base scores. One workgroup = 4 waves = one 256-key block of
// one request and up to 8 KV heads; a wave takes 16 keys at a time. For each head and pair of
// 16-dim tiles (t, t + d/32): two 16x16x16 bf16 steps Y^T = B_k^T K_lr^T (rank padded to 16) give
// lane (key n, group q) dims 16t + 4q .. +3 of key n in both halves; the rotation is lane-local;
// rounded to fp16, those registers are already the A operand (keys x dims) of the score step
// S^T += Y_rot Q^T on 16x16x16 fp16 steps, whose B operand is the group's queries (fp16).
template <int D, int R>
__global__ __launch_bounds__(kThreads) void key_scores_kernel(KeyScoreParams p) {
    constexpr int NDT = D / 16, NPAIR = NDT / 2;
    __shared__ uint16_t bkt[kHeads][D][kRankPad + 4];   // B_k slices transposed, rows padded by 8 bytes

    const int blk = blockIdx.x, b = blockIdx.y, g0 = blockIdx.z * kHeads;
    const int nh = min(kHeads, p.n_kv - g0);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int64_t start = p.kv_start[b];
    const int32_t len = p.kv_len[b];
    const int32_t a = p.agent[b];
    const bool ok = len > 0 && int64_t(len) <= p.max_kv_len && start >= 0 && start + int64_t(len) <= p.kv_rows &&
                    a >= 0 && a < p.n_agents;   // adapter-free and invalid requests need no scores
    const int32_t len32 = ok ? (len + 31) / 32 * 32 : 0;   // keys the decode reads
    if (int64_t(blk) * kKeyScoreBlock >= len32) return;  // workgroup-uniform

    const int64_t kv_stride = int64_t(p.n_kv) * D;
    const uint16_t* __restrict__ Bk = static_cast<const uint16_t*>(p.Bk) + int64_t(a) * R * kv_stride;
    for (int idx = tid; idx < nh * D * kRankPad; idx += kThreads) {
        const int h = idx / (D * kRankPad), rem = idx - h * (D * kRankPad);
        const int d = rem / kRankPad, r = rem - d * kRankPad;
        bkt[h][d][r] = r < R ? Bk[int64_t(r) * kv_stride + int64_t(g0 + h) * D + d] : uint16_t(0);
    }
    __syncthreads();

    const uint16_t* __restrict__ Klr = static_cast<const uint16_t*>(p.Klr);
    const uint16_t* __restrict__ Qb = static_cast<const uint16_t*>(p.Q) + int64_t(b) * p.n_q * D;
    for (int j0 = blk * kKeyScoreBlock + 16 * wv; j0 < min(len32, (blk + 1) * kKeyScoreBlock); j0 += 4 * 16) {
        // B operand: K_lr row of key n, ranks 4q .. 4q+3; the key's rotary entries of its dims
        const int jn = min(j0 + n, len - 1);
        const uint2 kl = 4 * q < R ? *reinterpret_cast<const uint2*>(Klr + (start + jn) * p.ld_klr + int64_t(a) * R + 4 * q)
                                   : make_uint2(0u, 0u);
        float4 cs[NPAIR], sn[NPAIR];
#pragma unroll
        for (int t = 0; t < NPAIR; ++t) {
            cs[t] = *reinterpret_cast<const float4*>(p.rope_cos + int64_t(jn) * (D / 2) + 16 * t + 4 * q);
            sn[t] = *reinterpret_cast<const float4*>(p.rope_sin + int64_t(jn) * (D / 2) + 16 * t + 4 * q);
        }
        for (int h = 0; h < nh; ++h) {
            const int g = g0 + h;
            // the rotated rank-r keys as fp16 A operands, tile t (dims 16t + 4q .. +3 of key n)
            uint2 ya[NDT];
            bool key_bad = false;
#pragma unroll
            for (int t = 0; t < NPAIR; ++t) {
                const uint2 blo = *reinterpret_cast<const uint2*>(&bkt[h][16 * t + n][4 * q]);
                const uint2 bhi = *reinterpret_cast<const uint2*>(&bkt[h][16 * (t + NPAIR) + n][4 * q]);
                const f32x4 ylo = mma16x16x16_bf16(blo, kl, f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 yhi = mma16x16x16_bf16(bhi, kl, f32x4{0.f, 0.f, 0.f, 0.f});
                const float cv[4] = {cs[t].x, cs[t].y, cs[t].z, cs[t].w}, sv[4] = {sn[t].x, sn[t].y, sn[t].z, sn[t].w};
                float lo[4], hi[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    lo[x] = ylo[x] * cv[x] - yhi[x] * sv[x];
                    hi[x] = yhi[x] * cv[x] + ylo[x] * sv[x];
                    key_bad = key_bad || !(fabsf(lo[x]) <= kF16Max) || !(fabsf(hi[x]) <= kF16Max);
                }
                ya[t] = make_uint2(pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3]));
                ya[t + NPAIR] = make_uint2(pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3]));
            }
            // B operand: query head g*G + n (columns >= G are zero), dims 16t + 4q .. +3, as fp16
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            bool head_bad = false;
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                uint2 qb = make_uint2(0u, 0u);
                if (n < p.G) {
                    const uint2 w = *reinterpret_cast<const uint2*>(Qb + (int64_t(g) * p.G + n) * D + 16 * t + 4 * q);
                    const float x0 = bf16_lo(w.x), x1 = bf16_hi(w.x), x2 = bf16_lo(w.y), x3 = bf16_hi(w.y);
                    head_bad = head_bad || !(fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))) <= kF16Max);
                    qb = make_uint2(pack_f16x2(x0, x1), pack_f16x2(x2, x3));
                }
                acc = mma16x16x16_f16(ya[t], qb, acc);
            }
            // lane (head n, group q) holds keys 4q .. 4q+3; NaN where the key part or the query left
            // the fp16 range (a key's dims sit in lanes n + 16q', a head's in lanes n + 16q')
            const uint64_t kb = __ballot(key_bad), hb = __ballot(head_bad);
            const uint32_t key_mask = uint32_t((kb | (kb >> 16) | (kb >> 32) | (kb >> 48)) & 0xffffu);
            const uint32_t head_mask = uint32_t((hb | (hb >> 16) | (hb >> 32) | (hb >> 48)) & 0xffffu);
            if (n < p.G) {
                float sv4[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const bool bad = ((key_mask >> (4 * q + x)) & 1u) || ((head_mask >> n) & 1u) || !(fabsf(acc[x]) <= kF16Max);
                    sv4[x] = bad ? __uint_as_float(0x7fc00000u) : acc[x];
                }
                uint16_t* dst = p.S + (int64_t(b) * p.n_q + int64_t(g) * p.G + n) * p.ks_stride + j0 + 4 * q;
                *reinterpret_cast<uint2*>(dst) = make_uint2(pack_f16x2(sv4[0], sv4[1]), pack_f16x2(sv4[2], sv4[3]));
            }
        }
    }
}

template <int D>
void launch_scores_d(const KeyScoreParams& p, hipStream_t stream) {
    const dim3 grid(unsigned((p.max_kv_len + kKeyScoreBlock - 1) / kKeyScoreBlock), unsigned(p.batch),
                    unsigned((p.n_kv + kHeads - 1) / kHeads));
    if (p.rank == 8) hipLaunchKernelGGL((key_scores_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((key_scores_kernel<D, 16>), grid, dim3(kThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_key_scores(const KeyScoreParams& p, hipStream_t stream) {
    if (p.d_head == 64) launch_scores_d<64>(p, stream);
    else launch_scores_d<128>(p, stream);
    return hipGetLastError();
}

hipError_t launch_key_expand(const KeyExpandParams& p, hipStream_t stream) {
    if (p.d_head == 64) launch_d<64>(p, stream);
    else launch_d<128>(p, stream);
    return hipGetLastError();
}

}  // namespace lra
