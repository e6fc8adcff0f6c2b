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
// Mapping: one workgroup = 4 waves = one 64-key tile of one KV head; wave w takes keys 16w..16w+15.
// For each pair of 16-dim tiles (dp, dp + d/32) the rank-r part comes out of two 16x16x16 bf16
// matrix-core steps Y^T = B_k^T K_lr^T (rank padded to 16 with zeros): lane (key n, group q) gets
// dims 16dp + 4q .. +3 of key n in both halves, which is exactly what the rotation pairs. The B_k
// slice is staged in LDS transposed ([dim][rank]) so each operand is one 8-byte read. The sum is
// taken in fp32 and rounded once to fp16; a tile that meets |value| > 65504 (or a NaN) sets its flag.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kThreads = 256;
constexpr int kRankPad = 16;

template <int D, int R>
__global__ __launch_bounds__(kThreads) void key_expand_kernel(KeyExpandParams p) {
    constexpr int NPAIR = D / 32;
    __shared__ uint16_t bkt[D][kRankPad + 4];   // B_k slice transposed, rows padded by 8 bytes

    const int tile = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int64_t kv_stride = int64_t(p.n_kv) * D;

    const uint16_t* __restrict__ Bk = static_cast<const uint16_t*>(p.Bk);
    for (int idx = tid; idx < D * kRankPad; idx += kThreads) {
        const int d = idx / kRankPad, r = idx - d * kRankPad;
        bkt[d][r] = r < R ? Bk[(int64_t(p.agent) * R + r) * kv_stride + int64_t(g) * D + d] : uint16_t(0);
    }

    // B operand: K_lr row of key n, ranks 4q .. 4q+3 (zero past the rank)
    const int64_t j = int64_t(tile) * kKeyTile + 16 * wv + n;
    const bool valid = j < p.n_rows;
    const int64_t jc = valid ? j : p.n_rows - 1;
    const uint16_t* __restrict__ Klr = static_cast<const uint16_t*>(p.Klr);
    const uint2 kl = 4 * q < R ? *reinterpret_cast<const uint2*>(Klr + jc * p.ld_klr + int64_t(p.agent) * R + 4 * q)
                               : make_uint2(0u, 0u);
    const uint16_t* __restrict__ krow = static_cast<const uint16_t*>(p.K) + jc * kv_stride + int64_t(g) * D;
    const float* __restrict__ crow = p.rope_cos + jc * (D / 2);
    const float* __restrict__ srow = p.rope_sin + jc * (D / 2);
    uint16_t* __restrict__ orow = static_cast<uint16_t*>(p.Ka) + jc * kv_stride + int64_t(g) * D;
    __syncthreads();

    bool out_of_range = false;   // |value| > 65504 or NaN (which compares false)
#pragma unroll
    for (int dp = 0; dp < NPAIR; ++dp) {
        const int c0 = 16 * dp + 4 * q;   // this lane's first dim of the low half
        const uint2 blo = *reinterpret_cast<const uint2*>(&bkt[16 * dp + n][4 * q]);
        const uint2 bhi = *reinterpret_cast<const uint2*>(&bkt[16 * (dp + NPAIR) + n][4 * q]);
        const f32x4 ylo = mma16x16x16_bf16(blo, kl, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 yhi = mma16x16x16_bf16(bhi, kl, f32x4{0.f, 0.f, 0.f, 0.f});
        const uint2 klo = *reinterpret_cast<const uint2*>(krow + c0);
        const uint2 khi = *reinterpret_cast<const uint2*>(krow + c0 + D / 2);
        const float4 c = *reinterpret_cast<const float4*>(crow + c0);
        const float4 s = *reinterpret_cast<const float4*>(srow + c0);
        const float cv[4] = {c.x, c.y, c.z, c.w}, sv[4] = {s.x, s.y, s.z, s.w};
        const uint32_t kw_lo[2] = {klo.x, klo.y}, kw_hi[2] = {khi.x, khi.y};
        uint32_t out_lo[2], out_hi[2];
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
            float lo[2], hi[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int x = 2 * w2 + e;
                const float kl0 = e ? bf16_hi(kw_lo[w2]) : bf16_lo(kw_lo[w2]);
                const float kh0 = e ? bf16_hi(kw_hi[w2]) : bf16_lo(kw_hi[w2]);
                lo[e] = kl0 + (ylo[x] * cv[x] - yhi[x] * sv[x]);
                hi[e] = kh0 + (yhi[x] * cv[x] + ylo[x] * sv[x]);
                out_of_range = out_of_range || !(fabsf(lo[e]) <= kF16Max) || !(fabsf(hi[e]) <= kF16Max);
            }
            out_lo[w2] = pack_f16x2(lo[0], lo[1]);
            out_hi[w2] = pack_f16x2(hi[0], hi[1]);
        }
        if (valid) {
            *reinterpret_cast<uint2*>(orow + c0) = make_uint2(out_lo[0], out_lo[1]);
            *reinterpret_cast<uint2*>(orow + c0 + D / 2) = make_uint2(out_hi[0], out_hi[1]);
        }
    }
    const int bad = valid && out_of_range;
    const int any_bad = __syncthreads_or(bad);
    if (tid == 0) p.flags[int64_t(tile) * p.n_kv + g] = any_bad;
}

template <int D>
void launch_d(const KeyExpandParams& p, hipStream_t stream) {
    const dim3 grid(unsigned((p.n_rows + kKeyTile - 1) / kKeyTile), unsigned(p.n_kv));
    if (p.rank == 8) hipLaunchKernelGGL((key_expand_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((key_expand_kernel<D, 16>), grid, dim3(kThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_key_expand(const KeyExpandParams& p, hipStream_t stream) {
    if (p.d_head == 64) launch_d<64>(p, stream);
    else launch_d<128>(p, stream);
    return hipGetLastError();
}

}  // namespace lra
