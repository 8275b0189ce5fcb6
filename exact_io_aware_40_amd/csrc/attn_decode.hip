// attn_decode.hip -- the fused attention forward for launches in which no
// two workgroups read the same K/V tile: one query block per (batch, head),
// as in a decode step against a key/value cache, whole or split into chunks
// (Flash-Decoding, "FlashAttention" explainer, "Common questions").  Every
// byte of K and V then crosses HBM once, and the tiles' copies into LDS are
// marked non-temporal so that they do not displace cached lines.  The kernel
// is the one every other launch uses (attn_fwd_kernel.h); outputs are the
// same bit for bit.  No dropout: a step with dropout takes the regular path.
#include "attn_fwd_kernel.h"

namespace attn {
namespace {

template <typename T, typename TO, int D, bool CAUSAL>
hipError_t launch_once(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_kernel<T, TO, D, CAUSAL, false, true>), dim3(a.total), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_once_t(const FwdArgs& a, int d, int causal, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_once<T, TO, 64, true>(a, stream) : launch_once<T, TO, 64, false>(a, stream);
    return causal ? launch_once<T, TO, 128, true>(a, stream) : launch_once<T, TO, 128, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_once(const FwdArgs& a, int dtype, bool out_f32, int d, int causal, hipStream_t stream) {
    if (dtype == 1)
        return out_f32 ? launch_once_t<__bf16, float>(a, d, causal, stream)
                       : launch_once_t<__bf16, __bf16>(a, d, causal, stream);
    return out_f32 ? launch_once_t<_Float16, float>(a, d, causal, stream)
                   : launch_once_t<_Float16, _Float16>(a, d, causal, stream);
}

hipError_t launch_fwd_fp8_once(const FwdArgs& a, int out_dtype, int causal, hipStream_t stream) {
    if (out_dtype == 2)
        return causal ? launch_once<fp8e4m3, float, 128, true>(a, stream)
                      : launch_once<fp8e4m3, float, 128, false>(a, stream);
    if (out_dtype == 1)
        return causal ? launch_once<fp8e4m3, __bf16, 128, true>(a, stream)
                      : launch_once<fp8e4m3, __bf16, 128, false>(a, stream);
    return causal ? launch_once<fp8e4m3, _Float16, 128, true>(a, stream)
                  : launch_once<fp8e4m3, _Float16, 128, false>(a, stream);
}

}  // namespace attn
