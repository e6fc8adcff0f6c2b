// Key expansion for LoRA on the key projection (the qkvo configuration) on gfx950.
//
// LRAgent page (limitations) and PReCache summary page (which adapt only q and v by default): when
// the key projection carries LoRA too, an agent's key is K_base + RoPE(K_lr B_k). The rotation
// sits between the up-projection and the dot product with the query, so the rank-r part cannot be
// folded behind the softmax the way the value side is; each key has to be expanded and rotated at
// its own position before the scores. A causal prefill stages every key once per workgroup (a pair
// of 128-row query pieces), so the expansion runs once per call in this pass and the attention
// kernel reads the result: Ka[j, g] = fp16(K_base[j, g] + RoPE_j(K_lr[j, agent] B_k[agent][:, g])).
//
// Rotation (rotate-half pairing): element i < d/2 pairs with i + d/2; with c = cos[j, i] and
// s = sin[j, i], (y_i, y_{i+d/2}) -> (y_i c - y_{i+d/2} s, y_{i+d/2} c + y_i s).
//
// Mapping: one workgroup = one 64-key tile of one KV head, 256 threads; a thread owns 8 consecutive
// dims i .. i+7 of the low half and their partners i+d/2 .. of one key (d/16 threads per key), so
// every K_base, table and output access is a 16-byte run and the threads of a key cover its row
// contiguously. The rank-r product (r = 8 or 16 multiply-adds per element) runs on the vector ALU
// from the key's K_lr row (one broadcast load) and the B_k slice staged in LDS. The sum is taken in
// fp32 and rounded once to fp16. Each (tile, KV head) records the largest |value| it produced (as
// fp32 bits; +inf for a NaN), which tells the attention whether the fp16 keys are in range and
// precise enough for its queries.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kThreads = 256;

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
    float vmax = 0.f;                            // largest |value| of this thread's keys
    bool nan_seen = false;
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
                vmax = fmaxf(vmax, fmaxf(fabsf(lo[e]), fabsf(hi[e])));
                nan_seen = nan_seen || lo[e] != lo[e] || hi[e] != hi[e];
            }
            ol[w] = pack_f16x2(lo[0], lo[1]);
            oh[w] = pack_f16x2(hi[0], hi[1]);
        }
        uint16_t* orow = static_cast<uint16_t*>(p.Ka) + j * kv_stride + int64_t(g) * D;
        *reinterpret_cast<uint4*>(orow + i0) = make_uint4(ol[0], ol[1], ol[2], ol[3]);
        *reinterpret_cast<uint4*>(orow + i0 + D / 2) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
    }
    __shared__ uint32_t tile_max;
    if (tid == 0) tile_max = 0u;
    __syncthreads();
    atomicMax(&tile_max, nan_seen ? 0x7f800000u : __float_as_uint(vmax));   // |v| >= 0: the bits order like the values
    __syncthreads();
    if (tid == 0) p.flags[int64_t(tile) * p.n_kv + g] = int32_t(tile_max);
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
