// attn_std.hip -- materialised standard attention for gfx950: the baseline
// the pages measure the fused kernel against ("FlashAttention" explainer,
// Step 2 "Standard Attention"; "13% more FLOPs, 5.7x faster", introduction
// and section "The hierarchy attention keeps ignoring").
//
// Three kernels, each a full pass through HBM, as the explainer lists them:
//   scores   S = scale Q K^T          written in full (N x N fp32 per head)
//   softmax  P = softmax(S) per row   S read back, P written in full (N x N,
//                                     the input type), lse = m + ln l saved
//   pv       O = P V                  P read back
// The causal mask is applied by the softmax (masked probabilities are
// written as zeros); S is formed for every pair and P V runs over every key,
// so the traffic is that of the unfused computation whatever the mask.  Per
// head that is 4 N^2 elements of S and P traffic (S written and read, P
// written and read) against 4 N d of Q, K, V and O: the accounting of the
// explainer's Step 2, here with S in fp32 and P in 16 bits.
//
// The two products run on the matrix cores (v_mfma_f32_32x32x16_{bf16,f16},
// fp32 accumulate).  S is kept in fp32 so that the exponentials see the
// scores the fused kernel sees; P is normalised in fp32 and rounded once to
// the operand type of the second product.
#include <math.h>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int SB = 128;   // edge of the S tile of one scores workgroup
constexpr int PB = 128;   // query rows of one pv workgroup
constexpr int STD_NT = 256;

// S tile (i0 .. i0+127) x (j0 .. j0+127) of head bh: wave w forms the 64 x 64
// quadrant (w / 2, w % 2) as 2 x 2 products of 32 x 32, with Q rows as the A
// operand and K rows as the B operand (B[k][n] = K[n][k]: both operands hold
// eight consecutive d elements of one row per lane), read straight from HBM.
template <typename T, int D>
__global__ __launch_bounds__(STD_NT, 2) void std_scores_kernel(const T* __restrict__ q,
                                                               const T* __restrict__ k,
                                                               float* __restrict__ s, int N,
                                                               int nb, float scale) {
    typedef typename Elem<T>::v8 v8;
    constexpr int DK = D / 16;
    const int lane = tid_x() & 63, w = tid_x() >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    // consecutive logical tiles (the tiles of one head) share an XCD and its L2
    const unsigned L = (unsigned)xcd_remap(wg_x(), num_wg_x());
    const int jb = (int)(L % (unsigned)nb);
    const unsigned rest = L / (unsigned)nb;
    const int ib = (int)(rest % (unsigned)nb);
    const size_t bh = rest / (unsigned)nb;
    const int i0 = ib * SB + 64 * (w >> 1), j0 = jb * SB + 64 * (w & 1);
    const T* qh = q + bh * (size_t)N * D;
    const T* kh = k + bh * (size_t)N * D;

    v8 a[2][DK], b[2][DK];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int ri = i0 + 32 * x + l32, rj = j0 + 32 * x + l32;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
            v8 za = {}, zb = {};
            if (ri < N) za = *(const v8*)(qh + (size_t)ri * D + 16 * kk + 8 * h);
            if (rj < N) zb = *(const v8*)(kh + (size_t)rj * D + 16 * kk + 8 * h);
            a[x][kk] = za;
            b[x][kk] = zb;
        }
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = Elem<T>::mma(a[x][kk], b[y][kk], acc[x][y]);

    // accumulator element r of lane l is S[m][n], m = 8 (r / 4) + 4 (l / 32) + r % 4,
    // n = l % 32: each store writes 128 contiguous bytes per half wave
    float* sh = s + bh * (size_t)N * N;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int n = j0 + 32 * y + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = i0 + 32 * x + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < N && n < N) sh[(size_t)m * N + n] = scale * acc[x][y][r];
            }
        }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One wave per row of S (four rows per workgroup).  VEC: N is a multiple of
// four, so the row moves as 16-byte (S) and 8-byte (P) pieces; CH > 0: the
// row is held in registers, CH chunks of 256 elements (N <= 256 CH), and S
// is read once; CH = 0: the row is streamed twice (an online maximum and sum,
// then the probabilities), for rows too long for the registers.
template <typename T, int CH, bool VEC>
__global__ __launch_bounds__(STD_NT) void std_softmax_kernel(const float* __restrict__ s,
                                                             T* __restrict__ p,
                                                             float* __restrict__ lse,
                                                             size_t rows, int N, int causal) {
    const int lane = tid_x() & 63, w = tid_x() >> 6;
    const size_t row = (size_t)wg_x() * 4 + w;
    if (row >= rows) return;   // the whole wave leaves; the kernel has no barrier
    const int i = (int)(row % (unsigned)N);
    const int lim = causal ? i + 1 : N;   // keys 0 .. lim-1 are visible (lim >= 1)
    const float* sr = s + row * N;
    T* pr = p + row * N;

    auto load4 = [&](int j, float* x) __attribute__((always_inline)) {
        if (VEC && j + 3 < N) {
            const f32x4 v = *(const f32x4*)(sr + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = j + e < N ? sr[j + e] : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e >= lim) x[e] = -INFINITY;
    };
    auto store4 = [&](int j, const float* x, float inv) __attribute__((always_inline)) {
        if (VEC && j + 3 < N) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            t4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (T)(x[e] * inv);
            *(t4*)(pr + j) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < N) pr[j + e] = (T)(x[e] * inv);
        }
    };

    float m, l;
    if constexpr (CH > 0) {
        float x[CH][4];
        m = -INFINITY;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int j = 256 * c + 4 * lane;
            if (j < N) {
                load4(j, x[c]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[c][e] = -INFINITY;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, x[c][e]);
        }
        m = wave_max(m);
        l = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[c][e] = fast_exp2((x[c][e] - m) * kLog2e);
                l += x[c][e];
            }
        l = wave_sum(l);
        const float inv = 1.f / l;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int j = 256 * c + 4 * lane;
            if (j < N) store4(j, x[c], inv);
        }
    } else {
        // pass 1: a running maximum per lane with its sum rescaled as it moves
        m = -INFINITY;
        l = 0.f;
        for (int j = 4 * lane; j < N; j += 256) {
            float x[4];
            load4(j, x);
            const float mb = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            const float mn = fmaxf(m, mb);
            if (mn > -INFINITY) {
                l = l * fast_exp2((m - mn) * kLog2e);
#pragma unroll
                for (int e = 0; e < 4; ++e) l += fast_exp2((x[e] - mn) * kLog2e);
                m = mn;
            }
        }
        const float mw = wave_max(m);
        l = m > -INFINITY ? l * fast_exp2((m - mw) * kLog2e) : 0.f;
        m = mw;
        l = wave_sum(l);
        // pass 2: S read again, P written
        const float inv = 1.f / l;
        for (int j = 4 * lane; j < N; j += 256) {
            float x[4];
            load4(j, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = fast_exp2((x[e] - m) * kLog2e);
            store4(j, x, inv);
        }
    }
    if (lane == 0) lse[row] = m + __log2f(l) * kLn2;
}

// O rows i0 .. i0+127 of head bh: wave w owns 32 rows and all d columns.
// Per 32-key tile, V (32 keys x d) is staged through LDS transposed, so that
// the B operand (B[k = key][n = column]) is eight consecutive keys of one
// column per lane; the A operand is eight consecutive keys of one P row,
// read straight from HBM, as one 16-byte load when N is a multiple of 8
// (ALIGNED: every row then starts on a 16-byte boundary), else element by
// element.
template <typename T, typename TO, int D, bool ALIGNED>
__global__ __launch_bounds__(STD_NT) void std_pv_kernel(const T* __restrict__ p,
                                                        const T* __restrict__ v,
                                                        TO* __restrict__ o, int N, int nb) {
    typedef typename Elem<T>::v8 v8;
    constexpr int KT = 32;                 // keys per tile
    constexpr int VS = KT + 8;             // LDS row stride of the transposed tile (80 bytes)
    constexpr int DB = D / 32;             // output column blocks
    constexpr int G = KT * D / 8 / STD_NT; // 16-byte pieces of a tile per thread
    static_assert(G * STD_NT * 8 == KT * D, "the tile splits evenly over the workgroup");
    __shared__ __attribute__((aligned(16))) T vt[D * VS];

    const int tid = tid_x(), lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    // a head's query blocks share an XCD, so its V is read from HBM once
    const unsigned L = (unsigned)xcd_remap(wg_x(), num_wg_x());
    const int ib = (int)(L % (unsigned)nb);
    const size_t bh = L / (unsigned)nb;
    const int row = ib * PB + 32 * w + l32;
    const T* prow = p + bh * (size_t)N * N + (size_t)min(row, N - 1) * N;
    const T* vh = v + bh * (size_t)N * D;

    f32x16 acc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

    const int ntile = (N + KT - 1) / KT;
    for (int t = 0; t < ntile; ++t) {
        v8 pv[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int idx = tid + STD_NT * g;
            const int key = t * KT + idx / (D / 8);
            v8 z = {};
            if (key < N) z = *(const v8*)(vh + (size_t)key * D + 8 * (idx % (D / 8)));
            pv[g] = z;
        }
        v8 aop[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k0 = t * KT + 16 * ks + 8 * h;
            v8 z = {};
            if (row < N) {
                if (ALIGNED && k0 + 8 <= N) {
                    z = *(const v8*)(prow + k0);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (k0 + e < N) z[e] = prow[k0 + e];
                }
            }
            aop[ks] = z;
        }
        __syncthreads();   // every wave is done with the previous tile
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int idx = tid + STD_NT * g;
            const int key = idx / (D / 8), c0 = 8 * (idx % (D / 8));
#pragma unroll
            for (int e = 0; e < 8; ++e) vt[(c0 + e) * VS + key] = pv[g][e];
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int cb = 0; cb < DB; ++cb) {
                const v8 bop = *(const v8*)(vt + (32 * cb + l32) * VS + 16 * ks + 8 * h);
                acc[cb] = Elem<T>::mma(aop[ks], bop, acc[cb]);
            }
    }
    TO* oh = o + bh * (size_t)N * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = ib * PB + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m < N) oh[(size_t)m * D + 32 * cb + l32] = (TO)acc[cb][r];
        }
}

template <typename T>
hipError_t scores_t(const void* q, const void* k, float* s, int64_t BH, int N, int d, float scale,
                    hipStream_t st) {
    const int nb = (N + SB - 1) / SB;
    const dim3 grid((unsigned)(BH * nb * nb));
    if (d == 64)
        hipLaunchKernelGGL((std_scores_kernel<T, 64>), grid, dim3(STD_NT), 0, st, (const T*)q,
                           (const T*)k, s, N, nb, scale);
    else
        hipLaunchKernelGGL((std_scores_kernel<T, 128>), grid, dim3(STD_NT), 0, st, (const T*)q,
                           (const T*)k, s, N, nb, scale);
    return hipGetLastError();
}

template <typename T, int CH>
void softmax_launch(const float* s, void* p, float* lse, size_t rows, int N, int causal,
                    hipStream_t st) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (N % 4 == 0)
        hipLaunchKernelGGL((std_softmax_kernel<T, CH, true>), grid, dim3(STD_NT), 0, st, s, (T*)p,
                           lse, rows, N, causal);
    else
        hipLaunchKernelGGL((std_softmax_kernel<T, CH, false>), grid, dim3(STD_NT), 0, st, s, (T*)p,
                           lse, rows, N, causal);
}

template <typename T>
hipError_t softmax_t(const float* s, void* p, float* lse, int64_t BH, int N, int causal,
                     hipStream_t st) {
    const size_t rows = (size_t)BH * N;
    if (N <= 256) softmax_launch<T, 1>(s, p, lse, rows, N, causal, st);
    else if (N <= 1024) softmax_launch<T, 4>(s, p, lse, rows, N, causal, st);
    else if (N <= 4096) softmax_launch<T, 16>(s, p, lse, rows, N, causal, st);
    else softmax_launch<T, 0>(s, p, lse, rows, N, causal, st);
    return hipGetLastError();
}

template <typename T, typename TO, int D>
void pv_launch(const void* p, const void* v, void* o, int N, int nb, dim3 grid, hipStream_t st) {
    if (N % 8 == 0)
        hipLaunchKernelGGL((std_pv_kernel<T, TO, D, true>), grid, dim3(STD_NT), 0, st, (const T*)p,
                           (const T*)v, (TO*)o, N, nb);
    else
        hipLaunchKernelGGL((std_pv_kernel<T, TO, D, false>), grid, dim3(STD_NT), 0, st, (const T*)p,
                           (const T*)v, (TO*)o, N, nb);
}

template <typename T, typename TO>
hipError_t pv_t(const void* p, const void* v, void* o, int64_t BH, int N, int d, hipStream_t st) {
    const int nb = (N + PB - 1) / PB;
    const dim3 grid((unsigned)(BH * nb));
    if (d == 64) pv_launch<T, TO, 64>(p, v, o, N, nb, grid, st);
    else pv_launch<T, TO, 128>(p, v, o, N, nb, grid, st);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_std_scores(const void* q, const void* k, float* s, int64_t BH, int N, int d,
                             float scale, int dtype, hipStream_t stream) {
    return dtype == 1 ? scores_t<__bf16>(q, k, s, BH, N, d, scale, stream)
                      : scores_t<_Float16>(q, k, s, BH, N, d, scale, stream);
}

hipError_t launch_std_softmax(const float* s, void* p, float* lse, int64_t BH, int N, int causal,
                              int dtype, hipStream_t stream) {
    return dtype == 1 ? softmax_t<__bf16>(s, p, lse, BH, N, causal, stream)
                      : softmax_t<_Float16>(s, p, lse, BH, N, causal, stream);
}

hipError_t launch_std_pv(const void* p, const void* v, void* o, int64_t BH, int N, int d, int dtype,
                         bool out_f32, hipStream_t stream) {
    if (dtype == 1)
        return out_f32 ? pv_t<__bf16, float>(p, v, o, BH, N, d, stream)
                       : pv_t<__bf16, __bf16>(p, v, o, BH, N, d, stream);
    return out_f32 ? pv_t<_Float16, float>(p, v, o, BH, N, d, stream)
                   : pv_t<_Float16, _Float16>(p, v, o, BH, N, d, stream);
}

}  // namespace attn
