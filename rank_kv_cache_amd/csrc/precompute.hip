// LR precompute for gfx950: V_lr[out_rows[t], k*r + j] = sum_c X[t, c] A_k[c, j].
//
// PReCache page, PreLRShared: every agent's down-projection is applied to the hidden states of a
// segment when it is first processed, so all N LR caches come out of one pass over X. The product
// is skinny (N*r = 24..48 columns) and X dominates the bytes, so the kernel streams X from HBM
// once with 128-bit loads and lets the matrix cores do the multiply-adds.
//
// The down-projections arrive stacked as At = [A_1^T; ...; A_N^T] ([N*r x d_model], the layout of
// the LoRA "A" weights), so both MFMA operands are contiguous 8-element runs along d_model:
//   A operand: lane (row n, slot q) <- X[row][k + 8q .. +7]
//   B operand: lane (col n, slot q) <- At[col][k + 8q .. +7]   (small, L2-resident)
// Grid (16-row tiles, reduction splits, column groups of <= 64). The 4 waves of a workgroup take
// interleaved 32-wide chunks of the workgroup's reduction range and are summed through LDS. With
// several splits each workgroup stores an fp32 partial, release-fences and counts its arrival; the
// last workgroup of a tile sums the partials in split order (deterministic), stores the rows and
// zeroes the counter for the next call.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kRows = 16;

template <typename T, int NT>
__global__ __launch_bounds__(256) void precompute_kernel(PrecomputeParams p) {
    constexpr int NRP = 16 * NT;
    __shared__ float red[4][kRows][NRP + 1];
    __shared__ int last_s;

    const int rt = blockIdx.x, ks = blockIdx.y, cg = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int c0 = cg * 64;
    const int ncol = min(p.NR - c0, NRP);
    const int kb = ks * p.kr;
    const int ke = min(kb + p.kr, p.d_model);
    const int nkc = (ke - kb) / 32;

    const T* __restrict__ Xp = static_cast<const T*>(p.X);
    const T* __restrict__ Ap = static_cast<const T*>(p.A);

    const int64_t xrow = int64_t(rt) * kRows + n;
    const bool xrow_ok = xrow < p.T;
    const T* xptr = Xp + (xrow_ok ? xrow : 0) * p.ldx + kb + 8 * q;
    const T* aptr[NT];
    bool acol_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = 16 * nt + n;
        acol_ok[nt] = c < ncol;
        aptr[nt] = Ap + int64_t(c0 + (acol_ok[nt] ? c : 0)) * p.d_model + kb + 8 * q;
    }

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = wv; kc < nkc; kc += 4) {
        Vec<T, 8> xf;
        if (xrow_ok) xf.load(xptr + 32 * kc);
        else xf.zero();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            Vec<T, 8> af;
            if (acol_ok[nt]) af.load(aptr[nt] + 32 * kc);
            else af.zero();
            acc[nt] = mma16x16x32(xf, af, acc[nt]);
        }
    }

    // lane holds C[row 4q+j][col 16nt+n]; sum the 4 waves
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wv][4 * q + j][16 * nt + n] = acc[nt][j];
    __syncthreads();

    const int64_t r0 = int64_t(rt) * kRows;
    const int nrows = int(min<int64_t>(kRows, p.T - r0));
    T* __restrict__ Op = static_cast<T*>(p.Vlr);
    if (p.ksplit == 1) {
        for (int idx = tid; idx < nrows * ncol; idx += 256) {
            const int rr = idx / ncol;
            const int c = idx - rr * ncol;
            const float v = red[0][rr][c] + red[1][rr][c] + red[2][rr][c] + red[3][rr][c];
            const int64_t orow = p.out_rows ? p.out_rows[r0 + rr] : r0 + rr;
            if (orow >= 0 && orow < p.vlr_rows) Op[orow * p.ld_vlr + c0 + c] = from_f32<T>(v);
        }
        return;
    }

    for (int idx = tid; idx < nrows * ncol; idx += 256) {
        const int rr = idx / ncol;
        const int c = idx - rr * ncol;
        const float v = red[0][rr][c] + red[1][rr][c] + red[2][rr][c] + red[3][rr][c];
        p.ws_part[(int64_t(ks) * p.T + r0 + rr) * p.NR + c0 + c] = v;
    }
    __threadfence();
    __syncthreads();
    uint32_t* counter = p.ws_count + int64_t(rt) * p.n_cg + cg;
    if (tid == 0) last_s = atomicAdd(counter, 1u) == uint32_t(p.ksplit - 1);
    __syncthreads();
    if (!last_s) return;
    __threadfence();
    for (int idx = tid; idx < nrows * ncol; idx += 256) {
        const int rr = idx / ncol;
        const int c = idx - rr * ncol;
        float sum = 0.f;
        for (int k = 0; k < p.ksplit; ++k) sum += p.ws_part[(int64_t(k) * p.T + r0 + rr) * p.NR + c0 + c];
        const int64_t orow = p.out_rows ? p.out_rows[r0 + rr] : r0 + rr;
        if (orow >= 0 && orow < p.vlr_rows) Op[orow * p.ld_vlr + c0 + c] = from_f32<T>(sum);
    }
    if (tid == 0) *counter = 0u;
}

template <typename T>
hipError_t launch_t(const PrecomputeParams& p, hipStream_t stream) {
    const int n_rt = int((p.T + kRows - 1) / kRows);
    const dim3 grid(n_rt, p.ksplit, p.n_cg);
    const int width = p.NR < 64 ? p.NR : 64;
    switch ((width + 15) / 16) {
        case 1: hipLaunchKernelGGL((precompute_kernel<T, 1>), grid, dim3(256), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((precompute_kernel<T, 2>), grid, dim3(256), 0, stream, p); break;
        case 3: hipLaunchKernelGGL((precompute_kernel<T, 3>), grid, dim3(256), 0, stream, p); break;
        default: hipLaunchKernelGGL((precompute_kernel<T, 4>), grid, dim3(256), 0, stream, p); break;
    }
    return hipGetLastError();
}

}  // namespace

PrecomputePlan plan_precompute(int64_t T, int d_model, int NR, bool /*bf16*/) {
    PrecomputePlan pl{};
    pl.n_rt = int((T + kRows - 1) / kRows);
    pl.n_cg = (NR + 63) / 64;
    const int64_t tiles = int64_t(pl.n_rt) * pl.n_cg;
    int ks = 1;
    for (;;) {
        const int kr = ((d_model + ks - 1) / ks + 31) / 32 * 32;
        if (tiles * ks >= 256 || kr <= 128 || ks >= 32) break;
        ks *= 2;
    }
    pl.kr = ((d_model + ks - 1) / ks + 31) / 32 * 32;
    pl.ksplit = (d_model + pl.kr - 1) / pl.kr;
    pl.count_bytes = size_t(tiles) * sizeof(uint32_t);
    pl.part_bytes = pl.ksplit > 1 ? size_t(pl.ksplit) * size_t(T) * size_t(NR) * sizeof(float) : 0;
    return pl;
}

hipError_t launch_precompute(const PrecomputeParams& p, hipStream_t stream) {
    return p.bf16 ? launch_t<bf16>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace lra
