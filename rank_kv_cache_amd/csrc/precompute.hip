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
// Grid (row tiles of 16 or 32 rows, reduction splits, column groups of <= 64); 8 waves per
// workgroup, each wave takes a contiguous eighth of the workgroup's reduction range and issues its
// loads in batches of 8 chunks (32 elements each) ahead of the multiplies. The waves are summed through LDS. With one split the
// workgroup writes the output rows; with several, each writes an fp32 partial and a second kernel
// sums the partials in split order (deterministic), converts and stores the rows. No workgroup
// waits on another: a device-scope fence per workgroup writes back and invalidates an XCD's L2.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kRows = 16;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBatch = 8;   // 32-element chunks whose loads a wave issues before multiplying

template <typename T, int NT, int MT>
__global__ __launch_bounds__(kThreads) void precompute_kernel(PrecomputeParams p) {
    constexpr int NRP = 16 * NT;
    constexpr int ROWS = kRows * MT;   // X rows of the workgroup: MT tiles of 16 share every A fragment
    __shared__ float red[kWaves][ROWS][NRP + 1];

    const int rt = blockIdx.x, ks = blockIdx.y, cg = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int c0 = cg * 64;
    const int ncol = min(p.NR - c0, NRP);
    // this workgroup's chunks [kc0, kc1) of 32 reduction elements, and this wave's share of them
    const int nkc_all = p.d_model / 32;
    const int kc0 = ks * (p.kr / 32);
    const int kc1 = min(kc0 + p.kr / 32, nkc_all);
    const int per_wave = (kc1 - kc0 + kWaves - 1) / kWaves;
    const int w0 = kc0 + wv * per_wave;
    const int w1 = min(w0 + per_wave, kc1);

    const T* __restrict__ Xp = static_cast<const T*>(p.X);
    const T* __restrict__ Ap = static_cast<const T*>(p.A);
    // rows past T and columns past ncol read a valid row / column; their outputs are never stored
    const T* xptr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t xrow = min<int64_t>(int64_t(rt) * ROWS + 16 * mt + n, p.T - 1);
        xptr[mt] = Xp + xrow * p.ldx + 8 * q;
    }
    const T* aptr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) aptr[nt] = Ap + int64_t(c0 + min(16 * nt + n, ncol - 1)) * p.d_model + 8 * q;

    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int b0 = w0; b0 < w1; b0 += kBatch) {
        Vec<T, 8> xf[kBatch][MT], af[kBatch][NT];
        // chunks past w1 re-read chunk w1 - 1 and are multiplied by zero
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int kc = min(b0 + u, w1 - 1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xf[u][mt].load(xptr[mt] + 32 * kc);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) af[u][nt].load(aptr[nt] + 32 * kc);
        }
        // keep the whole batch of loads in flight: the scheduler would otherwise sink each load to
        // its multiply to save registers
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (b0 + u >= w1) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) af[u][nt].zero();
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mma16x16x32(xf[u][mt], af[u][nt], acc[mt][nt]);
        }
    }

    // lane holds C[row 16mt+4q+j][col 16nt+n]; sum the waves
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wv][16 * mt + 4 * q + j][16 * nt + n] = acc[mt][nt][j];
    __syncthreads();

    const int64_t r0 = int64_t(rt) * ROWS;
    const int nrows = int(min<int64_t>(ROWS, p.T - r0));
    for (int idx = tid; idx < nrows * ncol; idx += kThreads) {
        const int rr = idx / ncol;
        const int c = idx - rr * ncol;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += red[w][rr][c];
        if (p.ksplit == 1) {
            const int64_t orow = p.out_rows ? p.out_rows[r0 + rr] : r0 + rr;
            if (orow >= 0 && orow < p.vlr_rows) static_cast<T*>(p.Vlr)[orow * p.ld_vlr + c0 + c] = from_f32<T>(v);
        } else {
            p.ws_part[(int64_t(ks) * p.T + r0 + rr) * p.NR + c0 + c] = v;
        }
    }
}

// Sum of the split partials in split order, then the row store (with the optional row map).
template <typename T>
__global__ __launch_bounds__(256) void precompute_reduce_kernel(PrecomputeParams p) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= p.T * p.NR) return;
    const int64_t t = idx / p.NR;
    const int c = int(idx - t * p.NR);
    // partials in split order, eight loads in flight at a time
    const int64_t stride = p.T * p.NR;
    const float* src = p.ws_part + idx;
    float v = 0.f;
    int k = 0;
    for (; k + 8 <= p.ksplit; k += 8) {
        float part[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) part[u] = src[(k + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += part[u];
    }
    for (; k < p.ksplit; ++k) v += src[k * stride];
    const int64_t orow = p.out_rows ? p.out_rows[t] : t;
    if (orow >= 0 && orow < p.vlr_rows) static_cast<T*>(p.Vlr)[orow * p.ld_vlr + c] = from_f32<T>(v);
}

template <typename T, int MT>
void launch_mt(const PrecomputeParams& p, hipStream_t stream) {
    const int n_rt = int((p.T + kRows * MT - 1) / (kRows * MT));
    const dim3 grid(n_rt, p.ksplit, p.n_cg);
    const int width = p.NR < 64 ? p.NR : 64;
    switch ((width + 15) / 16) {
        case 1: hipLaunchKernelGGL((precompute_kernel<T, 1, MT>), grid, dim3(kThreads), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((precompute_kernel<T, 2, MT>), grid, dim3(kThreads), 0, stream, p); break;
        case 3: hipLaunchKernelGGL((precompute_kernel<T, 3, MT>), grid, dim3(kThreads), 0, stream, p); break;
        default: hipLaunchKernelGGL((precompute_kernel<T, 4, MT>), grid, dim3(kThreads), 0, stream, p); break;
    }
}

template <typename T>
hipError_t launch_t(const PrecomputeParams& p, hipStream_t stream) {
    if (p.rows_per_wg == 2 * kRows) launch_mt<T, 2>(p, stream);
    else launch_mt<T, 1>(p, stream);
    if (p.ksplit > 1) {
        const int64_t n = p.T * p.NR;
        hipLaunchKernelGGL((precompute_reduce_kernel<T>), dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

PrecomputePlan plan_precompute(int64_t T, int d_model, int NR, bool /*bf16*/) {
    // Every workgroup reads the A fragments of its reduction range from L2 once per 16-row tile;
    // with many rows (>= 8192) a workgroup takes two tiles, so A costs half the L2 traffic. The
    // reduction is split until the grid reaches 256 workgroups (never below 256 elements per
    // workgroup, 32 per wave); a handful of rows (one new token per request) takes two splits.
    // Measured on MI355X: 2048 x 4096 rows run fastest with two splits (11.4 us against 13.6 with
    // one, 16 with four); 32 x 4096 rows with two (11.0 us; 11.4 with four to sixteen).
    PrecomputePlan pl{};
    pl.rows_per_wg = T >= 8192 ? 2 * kRows : kRows;
    pl.n_rt = int((T + pl.rows_per_wg - 1) / pl.rows_per_wg);
    pl.n_cg = (NR + 63) / 64;
    const int64_t tiles = int64_t(pl.n_rt) * pl.n_cg;
    int ks = 1;
    if (T <= 64) {
        ks = d_model >= 512 ? 2 : 1;
    } else {
        while (tiles * ks < 256 && d_model / (2 * ks) >= 256 && ks < 64) ks *= 2;
    }
    pl.kr = ((d_model + ks - 1) / ks + 31) / 32 * 32;
    pl.ksplit = (d_model + pl.kr - 1) / pl.kr;
    pl.part_bytes = pl.ksplit > 1 ? size_t(pl.ksplit) * size_t(T) * size_t(NR) * sizeof(float) : 0;
    return pl;
}

hipError_t launch_precompute(const PrecomputeParams& p, hipStream_t stream) {
    return p.bf16 ? launch_t<bf16>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace lra
