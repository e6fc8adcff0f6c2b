// Decode with LoRA on the key projection (the qkvo configuration) on gfx950: the rank-r part of
// every score.
//
// LRAgent page (limitations): with LoRA on the keys, request b's key t is
// K_base + RoPE_t(K_lr B_k), and the rotation between the up-projection and the dot product keeps
// the rank-r part from being moved behind the softmax. Its contribution to the score of query head
// h (KV head g) is
//     S[t, h] = q_h . RoPE_t(y_t),    y_t = K_lr[t, agent] B_k[agent][:, g*d .. g*d+d].
// With rotate-half pairing (element i < d/2 with i + d/2, cosine c_ti and sine s_ti) this is
//     S[t, h] = sum_{r, i} (K_lr[t, r] c_ti) P_h[r, i] + (K_lr[t, r] s_ti) M_h[r, i],
//     P_h[r, i] = B[r, i] q_h[i] + B[r, i + d/2] q_h[i + d/2],
//     M_h[r, i] = B[r, i] q_h[i + d/2] - B[r, i + d/2] q_h[i],
// (B = B_k[agent] restricted to KV head g), i.e. a dense product of per-key features
// F_t = K_lr[t, :] (x) [c_t, s_t] (d*r values) with per-head weights W_h = [P_h, M_h]. The weights
// depend on the request and head only, so one small pass computes them; the rotation then costs one
// packed fp16 multiply per pair of features instead of a rotation per key and KV head, and the
// reduction over d*r runs on 16x16x32 fp16 matrix-core steps.
//
// Mapping of the score pass: one workgroup = 4 waves = one 512-key block of one request and 16 or
// 32 query heads (the weights of those heads staged in LDS). A wave takes 16 keys at a time. Step s
// of the reduction covers 32 features: lane (key n, group q) builds its 8 = K_lr[t, r0 .. r0+7] x
// trig(ci) in registers (trig = cosine for ci < d/2, else sine), and reads the matching 8 weights
// of head n from LDS. The feature order k = ci * r + rr is shared by both operands; ci runs over a
// contiguous range per lane group. A small pass first repacks the rotary tables as fp16 in the
// lanes' order (per 16-key tile and group of 8 steps, 1 KB per wave): read in their natural layout,
// each load instruction touched 64 cache lines and those loads set the pass's time.
// Output lane (head n, group q) holds the scores of keys 4q .. 4q+3, stored as fp32.
//
// Range: the fp16 operands (weights, K_lr, rotary entries) hold magnitudes up to 65504. An operand
// beyond that becomes infinite and makes every score it enters non-finite; and an operand inside the
// range but large makes the fp16 rounding of the products (2^-11 relative) matter for the softmax.
// So a workgroup that produces a non-finite score, or a rank-r score part worth more than
// kSafeLogits in the exponent (scale * |S|; O(1) inputs give well under 1), sets its flag, and a
// second kernel recomputes exactly those workgroups' scores in fp32 from Q, K_lr, B_k and the fp32
// tables (rank-r up-projection, rotation, dot product, as in the expression above). Both kernels
// write every score of their workgroup, so the flags need no clearing between calls.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kThreads = 256;
constexpr float kSafeLogits = 16.f;

__device__ __forceinline__ bool key_score_request_ok(const KeyScoreParams& p, int64_t start, int32_t len, int32_t a) {
    // adapter-free and invalid requests need no scores (the decode adds none / writes NaN)
    return len > 0 && int64_t(len) <= p.max_kv_len && start >= 0 && start + int64_t(len) <= p.kv_rows && a >= 0 &&
           a < p.n_agents;
}

// W[b, h, ci*R + r] = P_h[r, ci] (ci < d/2) or M_h[r, ci - d/2], as fp16; one workgroup per
// (request, query head)
template <int D, int R>
__global__ __launch_bounds__(kThreads) void key_weights_kernel(KeyScoreParams p) {
    const int b = blockIdx.x, h = blockIdx.y;
    const int64_t start = p.kv_start[b];
    const int32_t len = p.kv_len[b], a = p.agent[b];
    if (!key_score_request_ok(p, start, len, a)) return;
    const int g = h / p.G;
    const int64_t kv_stride = int64_t(p.n_kv) * D;
    const uint16_t* __restrict__ Bk = static_cast<const uint16_t*>(p.Bk) + int64_t(a) * R * kv_stride + int64_t(g) * D;
    const uint16_t* __restrict__ qh = static_cast<const uint16_t*>(p.Q) + (int64_t(b) * p.n_q + h) * D;
    uint16_t* __restrict__ W = p.W + (int64_t(b) * p.n_q + h) * (D * R);
    for (int idx = threadIdx.x; idx < D * R; idx += kThreads) {
        const int ci = idx / R, r = idx - ci * R;
        const int i = ci < D / 2 ? ci : ci - D / 2;
        const float bl = bf16_to_f32(Bk[int64_t(r) * kv_stride + i]);
        const float bh = bf16_to_f32(Bk[int64_t(r) * kv_stride + i + D / 2]);
        const float ql = bf16_to_f32(qh[i]), qu = bf16_to_f32(qh[i + D / 2]);
        const float w = ci < D / 2 ? bl * ql + bh * qu : bl * qu - bh * ql;
        W[idx] = uint16_t(pack_f16x2(w, 0.f) & 0xffffu);
    }
}

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t x, uint32_t y) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, x) * __builtin_bit_cast(f16x2_t, y));
}

template <int D, int R, int HB>
__global__ __launch_bounds__(kThreads) void key_scores_kernel(KeyScoreParams p) {
    constexpr int KF = D * R;          // features per key
    constexpr int NS = KF / 32;        // reduction steps
    constexpr int SLOTS = 32 / R;      // rotary entries per step; R/8 lane groups share one
    constexpr int LDW = KF + 8;        // weight row in LDS (halves), padded by 16 bytes
    static_assert((SLOTS / 2) * NS == D / 2, "each lane group owns a contiguous run of one table");
    __shared__ uint16_t ws[HB * 16][LDW];

    // request fastest: the workgroups of one key block (the same rotary table rows) run together
    const int b = blockIdx.x, blk = blockIdx.y, h0 = blockIdx.z * (HB * 16);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int64_t start = p.kv_start[b];
    const int32_t len = p.kv_len[b], a = p.agent[b];
    const int32_t len32 = key_score_request_ok(p, start, len, a) ? (len + 31) / 32 * 32 : 0;   // keys the decode reads
    if (int64_t(blk) * kKeyScoreBlock >= len32) {   // workgroup-uniform
        if (tid == 0) p.flags[(int64_t(b) * gridDim.y + blk) * gridDim.z + blockIdx.z] = 0;
        return;
    }
    const int nhq = min(HB * 16, p.n_q - h0);
    bool nonfinite = false;   // some score of this workgroup is not finite or too large for fp16 rounding

    // this workgroup's head weights; rows past n_q are zero
    const uint16_t* __restrict__ Wg = p.W + (int64_t(b) * p.n_q + h0) * KF;
    for (int idx = tid; idx < HB * 16 * (KF / 8); idx += kThreads) {
        const int row = idx / (KF / 8), c = (idx - row * (KF / 8)) * 8;
        const uint4 v = row < nhq ? *reinterpret_cast<const uint4*>(Wg + int64_t(row) * KF + c) : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&ws[row][c]) = v;
    }
    __syncthreads();

    // lane group q: rotary slot (cosine for the first half of the slots), ranks r0 .. r0+7
    const int slot = q / (R / 8), r0 = 8 * (q % (R / 8));
    const int kbase = slot * NS * R + r0;   // feature of step s: kbase + s*R .. +7
    const bf16* __restrict__ Klr = static_cast<const bf16*>(p.Klr);
    const int jend = min(len32, (blk + 1) * kKeyScoreBlock);
    for (int j0 = blk * kKeyScoreBlock + 16 * wv; j0 < jend; j0 += 4 * 16) {
        const int jn = min(j0 + n, len - 1);   // later keys repeat the last row (masked by the decode)
        Vec<bf16, 8> lr;
        lr.load(Klr + (start + jn) * p.ld_klr + int64_t(a) * R + r0);
        uint32_t l16[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) l16[w] = pack_f16x2(bf16_lo(lr.w[w]), bf16_hi(lr.w[w]));
        // this tile's rotary entries, 8 steps per 16-byte load (the packed table's lane order)
        const uint4* __restrict__ tp = reinterpret_cast<const uint4*>(p.Tp) + int64_t(j0 / 16) * (NS / 8) * 64 + lane;

        f32x4 acc[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint4 tn0 = tp[0], tn1 = tp[min(1, NS / 8 - 1) * 64];   // loaded two groups of 8 steps ahead
#pragma unroll 2
        for (int s0 = 0; s0 < NS; s0 += 8) {
            const uint32_t th[4] = {tn0.x, tn0.y, tn0.z, tn0.w};
            tn0 = tn1;
            tn1 = tp[min(s0 / 8 + 2, NS / 8 - 1) * 64];   // the last groups reload the last (unused)
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = kbase + (s0 + u) * R;
                // the step's rotary entry in both halves
                const uint32_t t2 = __builtin_amdgcn_perm(th[u >> 1], th[u >> 1], (u & 1) ? 0x07060706u : 0x05040504u);
                H8 fa;
#pragma unroll
                for (int w = 0; w < 4; ++w) fa.w[w] = pk_mul_f16(l16[w], t2);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    const uint4 wb = *reinterpret_cast<const uint4*>(&ws[16 * hb + n][k]);
                    H8 fb;
                    fb.w[0] = wb.x; fb.w[1] = wb.y; fb.w[2] = wb.z; fb.w[3] = wb.w;
                    acc[hb] = mma16x16x32_f16(fa, fb, acc[hb]);
                }
            }
        }
        const int jk = j0 + 4 * q;   // this lane's first key
        if (jk >= len32) continue;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int hl = 16 * hb + n;
            if (hl < nhq) {
#pragma unroll
                for (int x = 0; x < 4; ++x) nonfinite = nonfinite || !(fabsf(acc[hb][x]) * p.scale <= kSafeLogits);
                float* dst = p.S + (int64_t(b) * p.n_q + h0 + hl) * p.ks_stride + jk;
                *reinterpret_cast<float4*>(dst) = make_float4(acc[hb][0], acc[hb][1], acc[hb][2], acc[hb][3]);
            }
        }
    }
    const int any_bad = __syncthreads_or(nonfinite);
    if (tid == 0) p.flags[(int64_t(b) * gridDim.y + blk) * gridDim.z + blockIdx.z] = any_bad;
}

// fp32 recomputation of the scores of a workgroup of key_scores_kernel that produced a non-finite
// value (an fp16 operand out of range): thread = (key, KV head) pair; it builds the key's rotated
// rank-r part y = RoPE_t(K_lr[t] B_k[:, g]) pair by pair (i, i + d/2) and adds its dot product with
// each query head of g in this workgroup's head range. Same grid and output as key_scores_kernel.
template <int D, int R, int HB>
__global__ __launch_bounds__(kThreads) void key_scores_exact_kernel(KeyScoreParams p) {
    const int b = blockIdx.x, blk = blockIdx.y, h0 = blockIdx.z * (HB * 16);
    if (p.flags[(int64_t(b) * gridDim.y + blk) * gridDim.z + blockIdx.z] == 0) return;   // workgroup-uniform
    const int64_t start = p.kv_start[b];
    const int32_t len = p.kv_len[b], a = p.agent[b];
    if (!key_score_request_ok(p, start, len, a)) return;
    const int len32 = (len + 31) / 32 * 32;
    const int nhq = min(HB * 16, p.n_q - h0);
    const int g0 = h0 / p.G, g1 = (h0 + nhq - 1) / p.G;   // KV heads of this head range
    const int n_g = g1 - g0 + 1;
    const int64_t kv_stride = int64_t(p.n_kv) * D;
    const bf16* __restrict__ Bk = static_cast<const bf16*>(p.Bk) + int64_t(a) * R * kv_stride;
    const bf16* __restrict__ Qb = static_cast<const bf16*>(p.Q) + int64_t(b) * p.n_q * D;
    const bf16* __restrict__ Klr = static_cast<const bf16*>(p.Klr);
    const int jbeg = blk * kKeyScoreBlock, jend = min(len32, (blk + 1) * kKeyScoreBlock);
    for (int idx = threadIdx.x; idx < (jend - jbeg) * n_g; idx += kThreads) {
        const int j = jbeg + idx / n_g;
        const int g = g0 + idx % n_g;
        const int jr = min(j, len - 1);   // later keys repeat the last row (masked by the decode)
        float klr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) klr[r] = bf16_to_f32(Klr[(start + jr) * p.ld_klr + int64_t(a) * R + r]);
        const int64_t trow = int64_t(jr) * (D / 2);
        const int ha = max(h0, g * p.G), hz = min(h0 + nhq, (g + 1) * p.G);   // query heads of g here (<= 8)
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < D / 2; ++i) {
            float ylo = 0.f, yhi = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                ylo = fmaf(klr[r], bf16_to_f32(Bk[int64_t(r) * kv_stride + int64_t(g) * D + i]), ylo);
                yhi = fmaf(klr[r], bf16_to_f32(Bk[int64_t(r) * kv_stride + int64_t(g) * D + i + D / 2]), yhi);
            }
            const float c = p.rope_cos[trow + i], sn = p.rope_sin[trow + i];
            const float rlo = ylo * c - yhi * sn, rhi = yhi * c + ylo * sn;
#pragma unroll
            for (int x = 0; x < 8; ++x)
                if (ha + x < hz)
                    acc[x] = fmaf(bf16_to_f32(Qb[int64_t(ha + x) * D + i]), rlo,
                                  fmaf(bf16_to_f32(Qb[int64_t(ha + x) * D + i + D / 2]), rhi, acc[x]));
        }
#pragma unroll
        for (int x = 0; x < 8; ++x)
            if (ha + x < hz) p.S[(int64_t(b) * p.n_q + ha + x) * p.ks_stride + j] = acc[x];
    }
}

// The rotary tables in the score kernel's lane order, as fp16: entry ((tile*(NS/8) + g)*64 + lane)
// holds, for key 16*tile + (lane & 15) and lane group q = lane >> 4, the 8 table values of steps
// 8g .. 8g+7 of that group's slot. A tile's group is then one contiguous 1 KB load per wave.
// Positions past the table's last row repeat it.
template <int D, int R>
__global__ __launch_bounds__(kThreads) void rope_pack_kernel(KeyScoreParams p) {
    constexpr int NS = D * R / 32, SLOTS = 32 / R;
    const int64_t e = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);   // (tile, group)
    const int64_t n_tiles = key_score_table_tiles(p.max_kv_len);
    if (e >= n_tiles * (NS / 8)) return;
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const int64_t tile = e / (NS / 8);
    const int g = int(e - tile * (NS / 8));
    const int slot = q / (R / 8);
    const int64_t j = min<int64_t>(tile * 16 + n, p.max_kv_len - 1);
    const float* row = (slot < SLOTS / 2 ? p.rope_cos : p.rope_sin) + j * (D / 2) + (slot % (SLOTS / 2)) * NS + 8 * g;
    const float4 a = *reinterpret_cast<const float4*>(row), b = *reinterpret_cast<const float4*>(row + 4);
    reinterpret_cast<uint4*>(p.Tp)[e * 64 + lane] =
        make_uint4(pack_f16x2(a.x, a.y), pack_f16x2(a.z, a.w), pack_f16x2(b.x, b.y), pack_f16x2(b.z, b.w));
}

template <int D, int R>
void launch_dr(const KeyScoreParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((key_weights_kernel<D, R>), dim3(unsigned(p.batch), unsigned(p.n_q)), dim3(kThreads), 0, stream, p);
    const int64_t n_pack = key_score_table_tiles(p.max_kv_len) * (D * R / 32 / 8);   // (tile, group) pairs, one wave each
    hipLaunchKernelGGL((rope_pack_kernel<D, R>), dim3(unsigned((n_pack + 3) / 4)), dim3(kThreads), 0, stream, p);
    constexpr int HB = D * R <= 1024 ? 2 : 1;   // weights of 16*HB heads in LDS (about 66 KB)
    static_assert(16 * HB == 32 || D * R > 1024, "key_score_heads");
    const dim3 grid(unsigned(p.batch), unsigned((p.max_kv_len + kKeyScoreBlock - 1) / kKeyScoreBlock),
                    unsigned((p.n_q + 16 * HB - 1) / (16 * HB)));
    hipLaunchKernelGGL((key_scores_kernel<D, R, HB>), grid, dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((key_scores_exact_kernel<D, R, HB>), grid, dim3(kThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_key_scores(const KeyScoreParams& p, hipStream_t stream) {
    if (p.d_head == 64) {
        if (p.rank == 8) launch_dr<64, 8>(p, stream);
        else launch_dr<64, 16>(p, stream);
    } else {
        if (p.rank == 8) launch_dr<128, 8>(p, stream);
        else launch_dr<128, 16>(p, stream);
    }
    return hipGetLastError();
}

}  // namespace lra
