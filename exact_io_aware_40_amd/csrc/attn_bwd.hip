// attn_bwd.hip -- attention backward with recomputation for gfx950.
//
// The forward keeps only O and lse; here S and P are rebuilt tile by tile
// on chip from Q, K and lse ("13% more FLOPs, 5.7x faster", section "The
// backward pass: recompute instead of read"; explainer Step 5 "IO Savings").
// The gradient formulas are the chain rule through the row softmax:
//   P_ij = exp(s_ij - lse_i), D_i = dO_i . o_i, dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),
//   dq_i = scale sum_j dS_ij k_j, dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i P_ij dO_i.
//
// Two kernels, both deterministic (every output element is owned by one
// lane of one wave, no atomics):
//   dq_kernel   one workgroup per 128 query rows; streams K/V tiles.  It
//               also computes D_i for its rows and stores it in the
//               workspace for the second kernel.
//   dkdv_kernel one workgroup per 128 keys; streams Q/dO tiles.
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int NT = 256;         // 4 waves
constexpr int BQ = 128;         // dq_kernel: query rows per workgroup
constexpr int BKT = 64;         // dq_kernel: keys per K/V tile
constexpr int BK = 128;         // dkdv_kernel: keys per workgroup
constexpr int BQT = 64;         // dkdv_kernel: queries per Q/dO tile
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> __device__ __forceinline__ float to_f32(unsigned short x);
template <> __device__ __forceinline__ float to_f32<__bf16>(unsigned short x) {
    return __uint_as_float((unsigned)x << 16);
}
template <> __device__ __forceinline__ float to_f32<_Float16>(unsigned short x) {
    return (float)bit_cast<_Float16>(x);
}

// dot product of two 8-element rows held as raw 16-byte vectors
template <typename T> __device__ __forceinline__ float dot8(i32x4 a, i32x4 b) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned x = (unsigned)a[i], y = (unsigned)b[i];
        s = fmaf(to_f32<T>((unsigned short)(x & 0xffff)), to_f32<T>((unsigned short)(y & 0xffff)), s);
        s = fmaf(to_f32<T>((unsigned short)(x >> 16)), to_f32<T>((unsigned short)(y >> 16)), s);
    }
    return s;
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::v8 pack8(const f32x16& x, int q) {
    f32x4 lo = {x[8 * q + 0], x[8 * q + 1], x[8 * q + 2], x[8 * q + 3]};
    f32x4 hi = {x[8 * q + 4], x[8 * q + 5], x[8 * q + 6], x[8 * q + 7]};
    auto l4 = Elem<T>::cvt4(lo);
    auto h4 = Elem<T>::cvt4(hi);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Residual of pack8: x - (float)hi, rounded to T.  Used when T is fp16 to
// carry dS into the dQ and dK products as hi + lo, which keeps the rounding
// of dS to the operand type (relative 2^-11) out of those gradients; bf16
// operands keep the single rounding (their tolerance is 7.5x wider).
template <typename T>
__device__ __forceinline__ typename Elem<T>::v8 pack8_lo(const f32x16& x, int q,
                                                        typename Elem<T>::v8 hi) {
    f32x4 lo, hi4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = x[8 * q + e] - (float)hi[e];
        hi4[e] = x[8 * q + 4 + e] - (float)hi[4 + e];
    }
    auto l4 = Elem<T>::cvt4(lo);
    auto h4 = Elem<T>::cvt4(hi4);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename T> struct SplitDS { static constexpr bool value = false; };
template <> struct SplitDS<_Float16> { static constexpr bool value = true; };

// Store a 32-row x D accumulator set in "lane = row, 16 columns per block"
// layout (the C layout of a product whose n index is the row), times f.
template <typename TO, int D>
__device__ __forceinline__ void store_rows(TO* __restrict__ row_ptr, const f32x16* acc, float f, int h) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 x = {acc[cb][4 * g] * f, acc[cb][4 * g + 1] * f, acc[cb][4 * g + 2] * f,
                       acc[cb][4 * g + 3] * f};
            store4<TO>(row_ptr + 32 * cb + 8 * g + 4 * h, x);
        }
    }
}

// dO_i . o_i over the 8 columns at `off` (dO of type T, o of type TO)
template <typename T, typename TO> struct RowDot {
    static __device__ __forceinline__ float run(const T* g, const TO* o, size_t off) {
        return dot8<T>(*(const i32x4*)(g + off), *(const i32x4*)(o + off));
    }
};
template <typename T> struct RowDot<T, float> {
    static __device__ __forceinline__ float run(const T* g, const float* o, size_t off) {
        const i32x4 gx = *(const i32x4*)(g + off);
        const f32x4 o0 = *(const f32x4*)(o + off), o1 = *(const f32x4*)(o + off + 4);
        const float ov[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned x = (unsigned)gx[i];
            s = fmaf(to_f32<T>((unsigned short)(x & 0xffff)), ov[2 * i], s);
            s = fmaf(to_f32<T>((unsigned short)(x >> 16)), ov[2 * i + 1], s);
        }
        return s;
    }
};

// --------------------------------------------------------------------------
// dq_kernel
// --------------------------------------------------------------------------
template <typename T, typename TO, int D, bool CAUSAL>
__global__ __launch_bounds__(NT) void dq_kernel(BwdArgs a, int nqb, int total) {
    typedef typename Elem<T>::v8 v8;
    constexpr int GR = D / 8, RPP = NT / GR, LOADS = BKT / RPP;
    constexpr int KB = BKT / 32, DK = D / 16, DB = D / 32;

    __shared__ __attribute__((aligned(16))) char sK[BKT * D * 2];
    __shared__ __attribute__((aligned(16))) char sV[BKT * D * 2];

    const int N = a.N;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int s16 = lane & 15, grp = lane >> 4;

    const int L = xcd_remap(blockIdx.x, total);
    const int bh = L / nqb;
    int qb = L - bh * nqb;
    if (CAUSAL) qb = nqb - 1 - qb;
    const int q0 = qb * BQ;
    const size_t head = (size_t)bh * N * D;
    const T* __restrict__ Qh = (const T*)a.q + head;
    const T* __restrict__ Kh = (const T*)a.k + head;
    const T* __restrict__ Vh = (const T*)a.v + head;
    const TO* __restrict__ Oh = (const TO*)a.o + head;
    const T* __restrict__ Gh = (const T*)a.dO + head;

    const int qlo = q0 + 32 * w;
    const int qrow = qlo + l32;
    const bool live = qrow < N;

    // Q and dO fragments of this lane's row (B operands), and D_i
    i32x4 qf[DK], gf[DK];
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        i32x4 x = {0, 0, 0, 0}, g = {0, 0, 0, 0};
        if (live) {
            const size_t off = (size_t)qrow * D + 16 * kk + 8 * h;
            x = *(const i32x4*)(Qh + off);
            g = *(const i32x4*)(Gh + off);
            dpart += RowDot<T, TO>::run(Gh, Oh, off);
        }
        if (a.negate) x ^= (int)0x80008000;
        qf[kk] = x;
        gf[kk] = g;
    }
    const float delta = sum32(dpart);
    const float lse2 = live ? a.lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
    if (live && h == 0) a.delta[(size_t)bh * N + qrow] = delta;

    const int kend = CAUSAL ? min(N, q0 + BQ) : N;
    const int ntiles = (kend + BKT - 1) / BKT;

    const int g_col = tid % GR, g_row = tid / GR;
    i32x4 kreg[LOADS], vreg[LOADS];
    auto gload = [&](int j0) {
#pragma unroll
        for (int p = 0; p < LOADS; ++p) {
            const int row = j0 + g_row + p * RPP;
            i32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
            if (row < N) {
                kx = *(const i32x4*)(Kh + (size_t)row * D + g_col * 8);
                vx = *(const i32x4*)(Vh + (size_t)row * D + g_col * 8);
            }
            kreg[p] = kx;
            vreg[p] = vx;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int p = 0; p < LOADS; ++p) {
            const int row = g_row + p * RPP;
            *(i32x4*)(sK + t_off<D>(row, g_col)) = kreg[p];
            *(i32x4*)(sV + t_off<D>(row, g_col)) = vreg[p];
        }
    };

    const float c = a.c;
    f32x16 acc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

    gload(0);
    sstore();
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * BKT;
        if (t + 1 < ntiles) gload(j0 + BKT);

        int nb = KB;
        if (CAUSAL) {
            const int lim = qlo + 31 - j0;
            nb = lim < 0 ? 0 : min(KB, lim / 32 + 1);
        }
        nb = min(nb, (N - j0 + 31) / 32);
        const bool need_mask = (j0 + BKT > N) || (CAUSAL && j0 + BKT - 1 > qlo);

        constexpr bool SPLIT = SplitDS<T>::value;
        v8 dsb[KB][2], dsl[KB][2];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (b < nb) {
                f32x16 s, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[r] = 0.f;
                    dp[r] = 0.f;
                }
                const int krow = 32 * b + l32;
#pragma unroll
                for (int kk = 0; kk < DK; ++kk) {
                    const i32x4 kx = *(const i32x4*)(sK + t_off<D>(krow, 2 * kk + h));
                    s = Elem<T>::mma(bit_cast<v8>(kx), bit_cast<v8>(qf[kk]), s);
                }
#pragma unroll
                for (int kk = 0; kk < DK; ++kk) {
                    const i32x4 vx = *(const i32x4*)(sV + t_off<D>(krow, 2 * kk + h));
                    dp = Elem<T>::mma(bit_cast<v8>(vx), bit_cast<v8>(gf[kk]), dp);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(fmaf(s[r], c, -lse2));
                    if (need_mask) {
                        const int key = j0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
                        const bool ok = key < N && (!CAUSAL || key <= qrow);
                        p = ok ? p : 0.f;
                    }
                    s[r] = p * (dp[r] - delta);
                }
                dsb[b][0] = pack8<T>(s, 0);
                dsb[b][1] = pack8<T>(s, 1);
                if (SPLIT) {
                    dsl[b][0] = pack8_lo<T>(s, 0, dsb[b][0]);
                    dsl[b][1] = pack8_lo<T>(s, 1, dsb[b][1]);
                }
            }
        }
        // dQ^T += K^T dS^T (K^T through transposing reads of the K tile)
#pragma unroll
        for (int cb = 0; cb < DB; ++cb) {
            const int col = 32 * cb + 16 * (grp & 1) + 4 * (s16 & 3);
            const int gcol = col >> 3, within = (col & 7) * 2;
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                if (b < nb) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int row = 32 * b + 16 * q + 4 * h + (s16 >> 2);
                        const i16x4 lo = lds_read_tr16(sK, t_off<D>(row, gcol) + within);
                        const i16x4 hi = lds_read_tr16(sK, t_off<D>(row + 8, gcol) + within);
                        const v8 kt = join8<v8>(lo, hi);
                        acc[cb] = Elem<T>::mma(kt, dsb[b][q], acc[cb]);
                        if (SPLIT) acc[cb] = Elem<T>::mma(kt, dsl[b][q], acc[cb]);
                    }
                }
            }
        }
        if (t + 1 < ntiles) {
            __syncthreads();
            sstore();
            __syncthreads();
        }
    }
    if (live) store_rows<TO, D>((TO*)a.dq + head + (size_t)qrow * D, acc, a.scale, h);
}

// --------------------------------------------------------------------------
// dkdv_kernel
// --------------------------------------------------------------------------
template <typename T, typename TO, int D, bool CAUSAL>
__global__ __launch_bounds__(NT) void dkdv_kernel(BwdArgs a, int nkb, int total) {
    typedef typename Elem<T>::v8 v8;
    constexpr int GR = D / 8, RPP = NT / GR, LOADS = BQT / RPP;
    constexpr int QB = BQT / 32, DK = D / 16, DB = D / 32;

    __shared__ __attribute__((aligned(16))) char sQ[BQT * D * 2];
    __shared__ __attribute__((aligned(16))) char sG[BQT * D * 2];
    __shared__ __attribute__((aligned(16))) float sL[BQT];
    __shared__ __attribute__((aligned(16))) float sD[BQT];

    const int N = a.N;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int s16 = lane & 15, grp = lane >> 4;

    const int L = xcd_remap(blockIdx.x, total);
    const int bh = L / nkb;
    const int kblk = L - bh * nkb;     // ascending: most queries first under the mask
    const int kb0 = kblk * BK;
    const size_t head = (size_t)bh * N * D;
    const T* __restrict__ Qh = (const T*)a.q + head;
    const T* __restrict__ Kh = (const T*)a.k + head;
    const T* __restrict__ Vh = (const T*)a.v + head;
    const T* __restrict__ Gh = (const T*)a.dO + head;
    const float* __restrict__ lse_h = a.lse + (size_t)bh * N;
    const float* __restrict__ dl_h = a.delta + (size_t)bh * N;

    const int kw0 = kb0 + 32 * w;       // this wave's first key
    const int key = kw0 + l32;          // this lane's key
    const bool live = key < N;

    // K^T and V^T fragments of this lane's key (B operands)
    i32x4 kf[DK], vf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        i32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
        if (live) {
            const size_t off = (size_t)key * D + 16 * kk + 8 * h;
            x = *(const i32x4*)(Kh + off);
            y = *(const i32x4*)(Vh + off);
        }
        if (a.negate) x ^= (int)0x80008000;
        kf[kk] = x;
        vf[kk] = y;
    }

    const int t0 = CAUSAL ? kb0 / BQT : 0;
    const int ntiles = (N + BQT - 1) / BQT;

    const int g_col = tid % GR, g_row = tid / GR;
    i32x4 qreg[LOADS], greg[LOADS];
    float lreg = 0.f, dreg = 0.f;
    auto gload = [&](int i0) {
#pragma unroll
        for (int p = 0; p < LOADS; ++p) {
            const int row = i0 + g_row + p * RPP;
            i32x4 qx = {0, 0, 0, 0}, gx = {0, 0, 0, 0};
            if (row < N) {
                qx = *(const i32x4*)(Qh + (size_t)row * D + g_col * 8);
                gx = *(const i32x4*)(Gh + (size_t)row * D + g_col * 8);
            }
            qreg[p] = qx;
            greg[p] = gx;
        }
        if (tid < BQT) {
            const int row = i0 + tid;
            // rows past the end get lse = +inf, so their P is exactly 0
            lreg = row < N ? lse_h[row] * kLog2e : INFINITY;
            dreg = row < N ? dl_h[row] : 0.f;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int p = 0; p < LOADS; ++p) {
            const int row = g_row + p * RPP;
            *(i32x4*)(sQ + t_off<D>(row, g_col)) = qreg[p];
            *(i32x4*)(sG + t_off<D>(row, g_col)) = greg[p];
        }
        if (tid < BQT) {
            sL[tid] = lreg;
            sD[tid] = dreg;
        }
    };

    const float c = a.c;
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[cb][r] = 0.f;
            dv[cb][r] = 0.f;
        }

    if (t0 < ntiles) {
        gload(t0 * BQT);
        sstore();
    }
    __syncthreads();

    for (int t = t0; t < ntiles; ++t) {
        const int i0 = t * BQT;
        if (t + 1 < ntiles) gload(i0 + BQT);

#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int ib = i0 + 32 * qb;    // first query of this 32-row block
            // skip blocks with no query at or after any of this wave's keys
            const bool active = ib < N && (!CAUSAL || ib + 31 >= kw0);
            if (!active) continue;
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.f;
                dp[r] = 0.f;
            }
            const int qrow_l = 32 * qb + l32;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const i32x4 qx = *(const i32x4*)(sQ + t_off<D>(qrow_l, 2 * kk + h));
                s = Elem<T>::mma(bit_cast<v8>(qx), bit_cast<v8>(kf[kk]), s);
            }
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const i32x4 gx = *(const i32x4*)(sG + t_off<D>(qrow_l, 2 * kk + h));
                dp = Elem<T>::mma(bit_cast<v8>(gx), bit_cast<v8>(vf[kk]), dp);
            }
            // rows of this block held by the lane: 32qb + 8(r/4) + 4h + r%4
            const bool need_mask = CAUSAL && ib < kw0 + 31;
            f32x16 p;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int li = 32 * qb + 8 * rr + 4 * h;
                const f32x4 l4 = *(const f32x4*)(sL + li);
                const f32x4 d4 = *(const f32x4*)(sD + li);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rr + e;
                    float pv = fast_exp2(fmaf(s[r], c, -l4[e]));
                    if (need_mask) pv = (key <= i0 + li + e) ? pv : 0.f;
                    p[r] = pv;
                    s[r] = pv * (dp[r] - d4[e]);   // dS
                }
            }
            constexpr bool SPLIT = SplitDS<T>::value;
            const v8 pb0 = pack8<T>(p, 0), pb1 = pack8<T>(p, 1);
            const v8 db0 = pack8<T>(s, 0), db1 = pack8<T>(s, 1);
            v8 dl0 = db0, dl1 = db1;
            if (SPLIT) {
                dl0 = pack8_lo<T>(s, 0, db0);
                dl1 = pack8_lo<T>(s, 1, db1);
            }
            // dV^T += dO^T P,  dK^T += Q^T dS  (transposing reads of the tiles)
#pragma unroll
            for (int cb = 0; cb < DB; ++cb) {
                const int col = 32 * cb + 16 * (grp & 1) + 4 * (s16 & 3);
                const int gcol = col >> 3, within = (col & 7) * 2;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int row = 32 * qb + 16 * q + 4 * h + (s16 >> 2);
                    const i16x4 glo = lds_read_tr16(sG, t_off<D>(row, gcol) + within);
                    const i16x4 ghi = lds_read_tr16(sG, t_off<D>(row + 8, gcol) + within);
                    dv[cb] = Elem<T>::mma(join8<v8>(glo, ghi), q ? pb1 : pb0, dv[cb]);
                    const i16x4 qlo = lds_read_tr16(sQ, t_off<D>(row, gcol) + within);
                    const i16x4 qhi = lds_read_tr16(sQ, t_off<D>(row + 8, gcol) + within);
                    const v8 qt = join8<v8>(qlo, qhi);
                    dk[cb] = Elem<T>::mma(qt, q ? db1 : db0, dk[cb]);
                    if (SPLIT) dk[cb] = Elem<T>::mma(qt, q ? dl1 : dl0, dk[cb]);
                }
            }
        }
        if (t + 1 < ntiles) {
            __syncthreads();
            sstore();
            __syncthreads();
        }
    }
    if (live) {
        store_rows<TO, D>((TO*)a.dk + head + (size_t)key * D, dk, a.scale, h);
        store_rows<TO, D>((TO*)a.dv + head + (size_t)key * D, dv, 1.f, h);
    }
}

template <typename T, typename TO, int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
    const int nqb = (a.N + BQ - 1) / BQ;
    const int nkb = (a.N + BK - 1) / BK;
    const int tq = a.BH * nqb, tk = a.BH * nkb;
    hipLaunchKernelGGL((dq_kernel<T, TO, D, CAUSAL>), dim3(tq), dim3(NT), 0, stream, a, nqb, tq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dkdv_kernel<T, TO, D, CAUSAL>), dim3(tk), dim3(NT), 0, stream, a, nkb, tk);
    return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_t(const BwdArgs& a, int d, int causal, hipStream_t stream) {
    if (d == 64) return causal ? launch<T, TO, 64, true>(a, stream) : launch<T, TO, 64, false>(a, stream);
    return causal ? launch<T, TO, 128, true>(a, stream) : launch<T, TO, 128, false>(a, stream);
}

}  // namespace

size_t bwd_workspace_bytes(int64_t BH, int64_t N) {
    const size_t bytes = size_t(BH) * size_t(N) * sizeof(float);
    return (bytes + 255) & ~size_t(255);
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, bool out_f32, int d, int causal, hipStream_t stream) {
    if (dtype == 1)
        return out_f32 ? launch_t<__bf16, float>(a, d, causal, stream)
                       : launch_t<__bf16, __bf16>(a, d, causal, stream);
    return out_f32 ? launch_t<_Float16, float>(a, d, causal, stream)
                   : launch_t<_Float16, _Float16>(a, d, causal, stream);
}

}  // namespace attn
