// attn_fwd.hip -- launchers of the fused attention forward (the kernel is
// in attn_fwd_kernel.h) and the merge of split K/V partial results.
#include "attn_fwd_kernel.h"

namespace attn {
namespace {

template <typename TO, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws_o,
                                                    const float* __restrict__ ws_lse,
                                                    TO* __restrict__ o, float* __restrict__ lse,
                                                    int64_t rows, int nsplit, size_t split_o,
                                                    size_t split_lse) {
    constexpr int G = D / 4;   // 4-column groups per row
    const int64_t gid = (int64_t)wg_x() * 256 + tid_x();
    const int64_t row = gid / G;
    const int cg = (int)(gid - row * G);
    if (row >= rows) return;
    float m = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, ws_lse[sp * split_lse + row]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != -INFINITY) {
        for (int sp = 0; sp < nsplit; ++sp) {
            const float wgt = expf(ws_lse[sp * split_lse + row] - m);
            const f32x4 x = *(const f32x4*)(ws_o + sp * split_o + row * D + 4 * cg);
            wsum += wgt;
            acc[0] += wgt * x[0];
            acc[1] += wgt * x[1];
            acc[2] += wgt * x[2];
            acc[3] += wgt * x[3];
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const f32x4 y = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    store4<TO>(o + row * D + 4 * cg, y);
    if (cg == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

template <typename T, typename TO, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    if constexpr (sizeof(T) == 1) {
        hipLaunchKernelGGL((fwd_kernel<T, TO, D, CAUSAL, false, false>), dim3(a.total), dim3(NT), 0, stream, a);
    } else {
        if (a.drop.on)
            hipLaunchKernelGGL((fwd_kernel<T, TO, D, CAUSAL, true, false>), dim3(a.total), dim3(NT), 0, stream, a);
        else
            hipLaunchKernelGGL((fwd_kernel<T, TO, D, CAUSAL, false, false>), dim3(a.total), dim3(NT), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_t(const FwdArgs& a, int d, int causal, hipStream_t stream) {
    if (d == 64) return causal ? launch<T, TO, 64, true>(a, stream) : launch<T, TO, 64, false>(a, stream);
    return causal ? launch<T, TO, 128, true>(a, stream) : launch<T, TO, 128, false>(a, stream);
}

}  // namespace

int fwd_block_rows() { return BR; }

size_t fwd_split_workspace_bytes(int64_t BH, int64_t N, int64_t d, int nsplit) {
    return (size_t)nsplit * (size_t)BH * (size_t)N * (size_t)(d + 1) * 4;
}

template <typename TO, int D>
hipError_t launch_merge_t(const float* ws_o, const float* ws_lse, void* o, float* lse, int64_t rows,
                          int nsplit, size_t split_o, size_t split_lse, hipStream_t stream) {
    const int64_t threads = rows * (D / 4);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL((merge_kernel<TO, D>), dim3(grid), dim3(256), 0, stream, ws_o, ws_lse, (TO*)o,
                       lse, rows, nsplit, split_o, split_lse);
    return hipGetLastError();
}

hipError_t launch_fwd_merge(const float* ws_o, const float* ws_lse, void* o, float* lse, int64_t rows,
                            int nsplit, size_t split_o, size_t split_lse, int d, int dtype, bool out_f32,
                            hipStream_t stream) {
    if (out_f32)
        return d == 64 ? launch_merge_t<float, 64>(ws_o, ws_lse, o, lse, rows, nsplit, split_o, split_lse, stream)
                       : launch_merge_t<float, 128>(ws_o, ws_lse, o, lse, rows, nsplit, split_o, split_lse, stream);
    if (dtype == 1)
        return d == 64 ? launch_merge_t<__bf16, 64>(ws_o, ws_lse, o, lse, rows, nsplit, split_o, split_lse, stream)
                       : launch_merge_t<__bf16, 128>(ws_o, ws_lse, o, lse, rows, nsplit, split_o, split_lse, stream);
    return d == 64 ? launch_merge_t<_Float16, 64>(ws_o, ws_lse, o, lse, rows, nsplit, split_o, split_lse, stream)
                   : launch_merge_t<_Float16, 128>(ws_o, ws_lse, o, lse, rows, nsplit, split_o, split_lse, stream);
}

hipError_t launch_fwd_fp8(const FwdArgs& a, int out_dtype, int causal, hipStream_t stream) {
    if (out_dtype == 2)
        return causal ? launch<fp8e4m3, float, 128, true>(a, stream) : launch<fp8e4m3, float, 128, false>(a, stream);
    if (out_dtype == 1)
        return causal ? launch<fp8e4m3, __bf16, 128, true>(a, stream) : launch<fp8e4m3, __bf16, 128, false>(a, stream);
    return causal ? launch<fp8e4m3, _Float16, 128, true>(a, stream) : launch<fp8e4m3, _Float16, 128, false>(a, stream);
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, bool out_f32, int d, int causal, hipStream_t stream) {
    if (dtype == 1)
        return out_f32 ? launch_t<__bf16, float>(a, d, causal, stream)
                       : launch_t<__bf16, __bf16>(a, d, causal, stream);
    return out_f32 ? launch_t<_Float16, float>(a, d, causal, stream)
                   : launch_t<_Float16, _Float16>(a, d, causal, stream);
}

}  // namespace attn
