// attn_probe.hip -- the matrix cores' sustained rate on this device.
//
// A kernel's utilisation is stated against two ceilings: the published dense
// bf16 peak, and the rate a kernel doing nothing but products sustains on the
// same board at the clock the board holds under it (the pages rate attention
// kernels by the fraction of the hardware's peak they reach: "FlashAttention"
// explainer, Step 6, and the section "IO-optimal is not occupancy-optimal").
// The power a product draws depends on how its operand bits change, so the
// operands are pseudo-random bf16 values of either sign in [0.5, 2), like
// attention's Q, K, V and P, and consecutive products take different ones:
// every wave keeps four chains of v_mfma_f32_32x32x16_bf16, chain j of round
// step s multiplying A operand j by B operand (j + s) mod 4, four waves per
// workgroup and two workgroups per CU, so that only the matrix pipes limit
// the rate.
//
// The HBM read probe does the same for memory-bound kernels (a decode step
// reads its key/value cache once, and the pages measure such kernels by the
// bytes they move: "13% more FLOPs, 5.7x faster", "The takeaway that
// outlives the kernel"): it streams a buffer once with the kernels' own
// direct-to-LDS copies and keeps only a checksum, so HBM reads are all it
// costs.
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int PNT = 256;   // threads per workgroup: four waves, one per SIMD

// The operands' bits: a 32-bit mixing function of x (the finaliser of
// MurmurHash3), sign from bit 15, exponent 126 or 127 from bit 7, mantissa
// from bits 0..6.
__device__ __forceinline__ unsigned short probe_bits(unsigned x) {
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return (unsigned short)((x & 0x807Fu) | 0x3F00u | ((x >> 1) & 0x80u));
}

__global__ __launch_bounds__(PNT, 2) void mfma_probe_kernel(float* __restrict__ out, int rounds) {
    typedef Elem<__bf16>::v8 v8;
    const int tid = tid_x(), lane = tid & 63;
    // operand j of this lane: element e = bits of (64 (8 j + e) + lane)
    v8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[j][e] = __builtin_bit_cast(__bf16, probe_bits((unsigned)(64 * (8 * j + e) + lane)));
            b[j][e] = __builtin_bit_cast(__bf16, probe_bits((unsigned)(64 * (8 * (j + 4) + e) + lane)));
        }
    // Opaque to the compiler from here on, so it must hold the operands in
    // registers and cannot move any part of their hashing into the loop.
#pragma unroll
    for (int j = 0; j < 4; ++j) __asm__ volatile("" : "+v"(a[j]), "+v"(b[j]));
    f32x16 c[4] = {};
    for (int i = 0; i < rounds; ++i) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = Elem<__bf16>::mma(a[j], b[(j + s) & 3], c[j]);
    }
    // each lane's 64 accumulators summed and stored, so that every product
    // is kept
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) t += (c[0][r] + c[1][r]) + (c[2][r] + c[3][r]);
    out[(size_t)wg_x() * PNT + tid] = t;
}

// The buffer is cut into 1 KiB chunks (chunk c: the 16-byte granules 64 c
// .. 64 c + 63) and each workgroup takes a contiguous range of them, as each
// workgroup of a decode step streams its own part of the key/value cache:
// workgroup b of B gets chunks b C .. min((b + 1) C, chunks) - 1 with C =
// ceil(chunks / B), and its wave w the chunks w, w + 4, w + 8, ... of that
// range.  A wave copies eight chunks at a time into its own LDS slots with
// the forward's non-temporal direct-to-LDS copy, and lane l adds, modulo
// 2^32, the four words of granule 64 c + l of every chunk it copied; thread
// 64 (4 b + w) + l stores that sum.  A copy outside the workgroup's range is
// zero-length (it reads zeros, as does a partial chunk past the end).  Loads
// into registers instead (8 in flight, non-temporal, the best of 4, 8 and 16
// with and without the hint) streamed at 6.3-6.4 TB/s, and so did these
// copies when each wave's chunks were spread over the whole buffer.
constexpr int HBM_INFLIGHT = 8;

__global__ __launch_bounds__(PNT) void hbm_probe_kernel(const char* __restrict__ p, long long n16,
                                                       unsigned* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) i32x4 slot[HBM_INFLIGHT][PNT];   // 32 KiB
    const int tid = tid_x(), lane = tid & 63, w = tid >> 6;
    const long long nbytes = n16 * 16, nchunks = (n16 + 63) / 64, nwg = num_wg_x();
    const long long per = (nchunks + nwg - 1) / nwg;
    const long long cb = (long long)wg_x() * per;
    const long long ce = cb + per < nchunks ? cb + per : nchunks;
    const unsigned lbase = lds_addr(&slot[0][64 * w]);
    unsigned acc = 0;
    for (long long c0 = cb + w; c0 < ce; c0 += HBM_INFLIGHT * (PNT / 64)) {
#pragma unroll
        for (int u = 0; u < HBM_INFLIGHT; ++u) {
            const long long c = c0 + u * (PNT / 64);
            const long long rem = c < ce ? nbytes - c * 1024 : 0;
            const unsigned len = rem <= 0 ? 0u : (unsigned)(rem < 1024 ? rem : 1024);
            dma16_async_once(make_rsrc(p + (rem > 0 ? c * 1024 : 0), len), lbase + u * PNT * 16, 16 * lane);
        }
        wait_vmem();
#pragma unroll
        for (int u = 0; u < HBM_INFLIGHT; ++u) {
            const i32x4 x = slot[u][64 * w + lane];
            acc += ((unsigned)x[0] + (unsigned)x[1]) + ((unsigned)x[2] + (unsigned)x[3]);
        }
        // every LDS read of the slots completes before the next copies
        // overwrite them (lgkmcnt 0; vmcnt and expcnt left alone)
        __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    out[(size_t)wg_x() * PNT + tid] = acc;
}

}  // namespace

hipError_t launch_hbm_probe(const void* buf, long long n16, unsigned* out, int workgroups, hipStream_t stream) {
    hipLaunchKernelGGL(hbm_probe_kernel, dim3(workgroups), dim3(PNT), 0, stream, (const char*)buf, n16, out);
    return hipGetLastError();
}

hipError_t launch_mfma_probe(float* out, int workgroups, int rounds, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(PNT), 0, stream, out, rounds);
    return hipGetLastError();
}

}  // namespace attn
