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
// One launch, no second pass: a workgroup of 16 waves (8 for 32 bf16 columns with d_model up to
// 4096, which need 256 registers per lane) owns a contiguous range of X rows (the rows are divided
// evenly, so every workgroup streams the same bytes) and one group of 16 or 32 output columns. Its
// waves split d_model 16 (8) ways; each wave holds the At fragments of its share in registers for
// the whole range (loaded once; for d_model beyond what fits they are reloaded per batch of chunks)
// and streams 16-row tiles of X: a tile's loads all go out at once, and each chunk of the next tile
// as soon as this tile's multiplies have read that chunk's registers, so the next tile is in flight
// while the partials are summed. The partial tiles are summed through LDS in a fixed order (deterministic)
// and stored with the optional row map. Workgroup w runs on XCD w % 8; the column groups of one row
// range get the same XCD and run side by side, so all but the first read X from L2, not HBM.
#include <algorithm>

#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

// WAVES: waves per workgroup, splitting d_model WAVES ways (16: 128 registers per lane; 8: 256).
// ARES: the wave's share of d_model is at most CB chunks, so its At fragments stay in registers for
// the whole row range; otherwise they are reloaded with each batch of CB chunks. NT: 16-column MFMA
// tiles per column group. With ARES each X chunk's registers are refilled with the next tile's chunk
// as soon as its multiplies have read them, when the registers allow it: one column tile at 16 waves,
// two at 8 waves (bf16: 16 chunks of A for two tiles, 128 registers, beside 16 chunks of X).
template <typename T, int CB, bool ARES, int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void precompute_kernel(PrecomputeParams p) {
    constexpr int kWaves = WAVES;
    constexpr int kThreads = 64 * WAVES;
    constexpr int NC = 16 * NT;   // columns of a group
    constexpr bool PREFETCH = ARES && (NT == 1 || WAVES == 8);
    // partial tiles, double-buffered: tile t sums from half t % 2, so one barrier per tile orders
    // both the partials before the sums and the sums before the next writes to that half
    __shared__ float red[2][kWaves][16][NC + 1];

    const int w = blockIdx.x, xcd = w & 7, rest = w >> 3;
    const int cg = rest % p.n_cg;
    const int rg = (rest / p.n_cg) * 8 + xcd;
    if (rg >= p.n_rg) return;
    const int64_t r0 = p.T * rg / p.n_rg, r1 = p.T * (rg + 1) / p.n_rg;   // this workgroup's X rows
    if (r0 >= r1) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, n = lane & 15, q = lane >> 4;
    const int c0 = cg * NC;
    const int ncol = min(p.NR - c0, NC);
    // this wave's chunks [kc0, kc1) of 32 reduction elements
    const int nch = p.d_model / 32;
    const int cpw = (nch + kWaves - 1) / kWaves;
    const int kc0 = min(wv * cpw, nch), kc1 = min(kc0 + cpw, nch);

    const T* __restrict__ Xp = static_cast<const T*>(p.X);
    // At fragments of chunks [b0, b0 + CB) (columns past ncol read a valid column, never stored;
    // chunks past kc1 are zero)
    Vec<T, 8> af[CB][NT];
    auto load_a = [&](int b0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const T* acol = static_cast<const T*>(p.A) + int64_t(c0 + min(16 * nt + n, ncol - 1)) * p.d_model + 8 * q;
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                if (b0 + u < kc1) af[u][nt].load(acol + 32 * (b0 + u));
                else af[u][nt].zero();
            }
        }
    };
    if constexpr (ARES) load_a(kc0);
    // X fragments of one 16-row tile; rows past r1 read row r1 - 1 (valid memory, never stored)
    Vec<T, 8> xf[CB];
    auto load_x = [&](int64_t rt, int b0) {
        const T* xrow = Xp + min<int64_t>(rt + n, r1 - 1) * p.ldx + 8 * q;
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            if (b0 + u < kc1) xf[u].load(xrow + 32 * (b0 + u));
            else xf[u].zero();
        }
    };
    if constexpr (PREFETCH) load_x(r0, kc0);

    int rb = 0;
    for (int64_t rt = r0; rt < r1; rt += 16) {
        f32x4 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (PREFETCH) {
            // chunk u's registers take the next tile's chunk u right after its multiplies, so the
            // next tile is in flight during this tile's reduction
            const bool more = rt + 16 < r1;
            const T* xnext = Xp + min<int64_t>(rt + 16 + n, r1 - 1) * p.ldx + 8 * q;
#pragma unroll
            for (int u = 0; u < CB; ++u) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = mma16x16x32(xf[u], af[u][nt], acc[nt]);
                if (more && kc0 + u < kc1) xf[u].load(xnext + 32 * (kc0 + u));
            }
        } else {
            for (int b0 = kc0; b0 < kc1; b0 += CB) {   // one batch when ARES
                if constexpr (!ARES) load_a(b0);
                load_x(rt, b0);
#pragma unroll
                for (int u = 0; u < CB; ++u)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[nt] = mma16x16x32(xf[u], af[u][nt], acc[nt]);
            }
        }

        // lane holds C[row 4q+j][col 16nt+n]; the 16 waves' partials are summed in wave order
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[rb][wv][4 * q + j][16 * nt + n] = acc[nt][j];
        __syncthreads();
        const int nrows = int(min<int64_t>(16, r1 - rt));
        for (int idx = tid; idx < nrows * ncol; idx += kThreads) {
            const int rr = idx / ncol;
            const int c = idx - rr * ncol;
            float v = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) v += red[rb][ww][rr][c];
            const int64_t orow = p.out_rows ? p.out_rows[rt + rr] : rt + rr;
            const int ka = (c0 + c) / p.rank;   // agent of output column c0 + c
            if (orow >= 0 && orow < p.vlr_rows)
                static_cast<T*>(p.Vlr)[orow * p.ld_vlr + ka * p.vlr_agent_stride + (c0 + c - ka * p.rank)] = from_f32<T>(v);
        }
        rb ^= 1;
    }
}

template <typename T, int CB>
void launch_t(const PrecomputeParams& p, hipStream_t stream) {
    const int64_t n_wg = (int64_t(p.n_rg) + 7) / 8 * 8 * p.n_cg;
    const int nch = p.d_model / 32;
    const int cpw16 = (nch + 15) / 16, cpw8 = (nch + 7) / 8;
    const dim3 grid{unsigned(n_wg)}, b16{1024u}, b8{512u};
    if (p.cols_per_group == 32) {
        // bf16 with d_model <= 4096: 8 waves, A resident for both column tiles, X prefetched
        if constexpr (sizeof(T) == 2) {
            if (cpw8 <= 2 * CB) {
                hipLaunchKernelGGL((precompute_kernel<T, 2 * CB, true, 2, 8>), grid, b8, 0, stream, p);
                return;
            }
        }
        if (cpw16 <= CB) hipLaunchKernelGGL((precompute_kernel<T, CB, true, 2, 16>), grid, b16, 0, stream, p);
        else hipLaunchKernelGGL((precompute_kernel<T, CB, false, 2, 16>), grid, b16, 0, stream, p);
    } else {
        if (cpw16 <= CB) hipLaunchKernelGGL((precompute_kernel<T, CB, true, 1, 16>), grid, b16, 0, stream, p);
        else hipLaunchKernelGGL((precompute_kernel<T, CB, false, 1, 16>), grid, b16, 0, stream, p);
    }
}

}  // namespace

PrecomputePlan plan_precompute(int64_t T, int d_model, int NR, bool bf16) {
    // Rows: about 16 per workgroup for a short X, and for a long one as many row ranges as give one
    // workgroup per CU (256 in all), each an equal share of the rows. Columns: groups of 16 for a
    // short X (more workgroups, the next tile prefetched); for a long X (4096 rows and more) groups
    // of 32, so each CU reads its X rows once: measured on MI355X, 2048 x 4096 -> 24 takes 10.2 us
    // with 16-column groups against 12.4 with 32, and 18432 x 4096 -> 24 takes 38 us against 41.
    PrecomputePlan pl{};
    pl.cols_per_group = (T >= 4096 && NR > 16) ? 32 : 16;
    pl.n_cg = (NR + pl.cols_per_group - 1) / pl.cols_per_group;
    const int64_t max_rg = std::max<int64_t>(1, 256 / pl.n_cg);
    pl.n_rg = int(std::max<int64_t>(1, std::min<int64_t>((T + 15) / 16, max_rg)));
    pl.chunks_per_wave = (d_model / 32 + 15) / 16;
    pl.cb = bf16 ? 8 : 4;
    return pl;
}

hipError_t launch_precompute(const PrecomputeParams& p, hipStream_t stream) {
    if (p.bf16) launch_t<bf16, 8>(p, stream);
    else launch_t<float, 4>(p, stream);
    return hipGetLastError();
}

}  // namespace lra
