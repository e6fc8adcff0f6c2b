// Value expansion for the expand-then-attend baseline on gfx950.
//
// LRAgent page, Flash-LoRA-Attention: without the reordering, an agent's full value cache
// V_a = V_base + V_lr B_a has to be built before attention reads it (one extra pass over the
// cache, written at full d_kv width per token); Flash-LoRA-Attention defers B_a behind the softmax
// instead. This pass builds V_a explicitly so that the two orders can be timed against each other
// on the same attention kernels (the attention then runs the adapter-free view over V_a):
//
//   V_out[dst_start[b] + t, g*d + c] = V_base[src_start[b] + t, g*d + c]
//                                      + sum_j V_lr[src_start[b] + t, a*r + j] * B_a[j, g*d + c]
//
// with a = agent[b]; the adapter-free agent (-1) copies V_base. The sum is taken in fp32 and rounded
// once to the element type (nearest, ties to even, for bf16).
//
// Mapping: one workgroup = a run of up to 256 rows of one request (a column block of 256 16-byte
// vectors when a row is wider than that); the run is shortened, down to 16 rows, until the grid
// holds about 2048 workgroups, so that a single request still spreads over the whole chip. A thread owns one fixed 16-byte vector of the row (8 bf16 or 4 fp32
// columns) and keeps the agent's B_a entries of those columns in fp32 registers for all its rows,
// so B is read once per workgroup. Each row costs one 16-byte V_base load, one broadcast load of
// the row's r V_lr entries and one 16-byte store; the loop keeps 8 rows (4 at rank 16) of loads in flight.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kThreads = 256;

template <typename T> __device__ __forceinline__ T nan_value();
template <> __device__ __forceinline__ float nan_value<float>() { return __uint_as_float(0x7fc00000u); }
template <> __device__ __forceinline__ bf16 nan_value<bf16>() { return bf16(0x7fc0); }

template <typename T, int R>
__global__ __launch_bounds__(kThreads) void value_expand_kernel(ValueExpandParams p) {
    constexpr int VEC = 16 / int(sizeof(T));
    constexpr int kUnroll = R == 8 ? 8 : 4;   // rows of loads in flight (register budget)
    const int tid = threadIdx.x;
    const int64_t chunk = blockIdx.x % p.n_chunks;
    const int b = int(blockIdx.x / p.n_chunks);
    const int ncv = p.row_elems / VEC;                  // 16-byte vectors per row
    // threads of one row, rows handled side by side, and this thread's vector / row slot
    const int tpr = ncv < kThreads ? ncv : kThreads;
    const int rpp = kThreads / tpr;
    const int cv = int(blockIdx.y) * kThreads + tid % tpr;
    const int rsub = tid / tpr;
    if (rsub >= rpp || cv >= ncv) return;

    const int32_t len = p.len[b];
    const int64_t src0 = p.src_start[b], dst0 = p.dst_start[b];
    const int32_t a = p.agent[b];
    const int64_t t0 = chunk * p.rows_per_wg;
    if (len <= 0 || t0 >= len || t0 >= p.max_len) return;
    // the destination range must lie inside V_out, else the request is skipped
    if (dst0 < 0 || dst0 > p.out_rows - len) return;
    const int64_t t1 = min(min<int64_t>(t0 + p.rows_per_wg, len), p.max_len);
    const int64_t col = int64_t(cv) * VEC;
    T* __restrict__ out = static_cast<T*>(p.Vout) + col;
    const bool valid = len <= p.max_len && src0 >= 0 && src0 <= p.kv_rows - len && a >= kAdapterFree && a < p.n_agents;
    if (!valid) {
        // an invalid source range or agent: NaN rows, nothing read
        for (int64_t t = t0 + rsub; t < t1; t += rpp) {
            T* o = out + (dst0 + t) * p.row_elems;
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = nan_value<T>();
        }
        return;
    }

    const T* __restrict__ vb = static_cast<const T*>(p.V) + src0 * p.row_elems + col;
    if (a == kAdapterFree) {
        for (int64_t t = t0 + rsub; t < t1; t += rpp)
            *reinterpret_cast<uint4*>(out + (dst0 + t) * p.row_elems) =
                *reinterpret_cast<const uint4*>(vb + t * p.row_elems);
        return;
    }

    // B_a[j, col .. col + VEC - 1] for j < R, fp32
    float bw[R][VEC];
    {
        const T* Bp = static_cast<const T*>(p.B) + int64_t(a) * R * p.row_elems + col;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            Vec<T, VEC> bv;
            bv.load(Bp + int64_t(j) * p.row_elems);
#pragma unroll
            for (int e = 0; e < VEC; ++e) bw[j][e] = bv.get(e);
        }
    }
    const T* __restrict__ lr = static_cast<const T*>(p.Vlr) + src0 * p.ld_vlr + int64_t(a) * R;

    for (int64_t tb = t0 + rsub; tb < t1; tb += int64_t(rpp) * kUnroll) {
        Vec<T, VEC> v[kUnroll];
        Vec<T, R> l[kUnroll];
        // rows past t1 re-read row t1 - 1 and are not stored
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t t = min(tb + int64_t(u) * rpp, t1 - 1);
            v[u].load(vb + t * p.row_elems);
            l[u].load(lr + t * p.ld_vlr);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t t = tb + int64_t(u) * rpp;
            if (t >= t1) break;
            float acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = v[u].get(e);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const float lj = l[u].get(j);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = fmaf(lj, bw[j][e], acc[e]);
            }
            T* o = out + (dst0 + t) * p.row_elems;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                          pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
            } else {
                *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
    }
}

template <typename T>
void launch_t(const ValueExpandParams& p, const dim3& grid, hipStream_t stream) {
    if (p.rank == 8) hipLaunchKernelGGL((value_expand_kernel<T, 8>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((value_expand_kernel<T, 16>), grid, dim3(kThreads), 0, stream, p);
}

}  // namespace

int value_expand_rows(int batch, int64_t max_len) {
    int rows = 256;
    while (rows > 16 && int64_t(batch) * ((max_len + rows - 1) / rows) < 2048) rows /= 2;
    return rows;
}

hipError_t launch_value_expand(const ValueExpandParams& p, hipStream_t stream) {
    const int vec = p.bf16 ? 8 : 4;
    const int ncv = p.row_elems / vec;
    const dim3 grid(unsigned(int64_t(p.batch) * p.n_chunks), unsigned((ncv + kThreads - 1) / kThreads));
    if (p.bf16) launch_t<bf16>(p, grid, stream);
    else launch_t<float>(p, grid, stream);
    return hipGetLastError();
}

}  // namespace lra
