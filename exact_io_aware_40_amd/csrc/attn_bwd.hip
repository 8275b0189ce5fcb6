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
//   dq_kernel   one workgroup per 128 query rows (under causal masking in
//               the forward's XCD head groups when B*H is a multiple of 8,
//               else per pair of a heavy and a light block of one head);
//               streams K/V tiles.  It also stores -D_i and lse_i log2(e) of its rows in
//               the workspace for the second kernel.
//   dkdv_kernel one workgroup per 128 keys (under causal masking per pair of
//               a heavy and a light block of one head); streams Q/dO tiles
//               together with their D and lse values.
// Tiles move global -> LDS with 16-byte direct copies into two stages
// (one barrier per tile); loads past the end of the sequence read zeros,
// which makes such rows contribute nothing (their dO, Q, lse and D are 0).
//
// Dropout (a separate instantiation) regenerates the forward's mask from the
// generator state: with W_ij = keep_ij r P_ij the weights applied to V
// (r = 256 / (256 - t)), dV_j = sum_i W_ij dO_i and dP_ij = keep_ij r
// dO_i . v_j, while D_i = dO_i . o_i is unchanged.  The kernels use
// D'_i = D_i / r, form dS / r = P (keep dP~ - D') with dP~ = dO_i . v_j, and
// apply r once to dQ, dK and dV.
#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int NT = 256;         // 4 waves
constexpr int BQ = 128;         // dq_kernel: query rows per workgroup
constexpr int BKT = 64;         // dq_kernel: keys per K/V tile
constexpr int BK = 128;         // dkdv_kernel: keys per workgroup
constexpr int NTK = 512;        // dkdv_kernel: 8 waves
constexpr int BQT = 64;         // dkdv_kernel: queries per Q/dO tile
constexpr int PADR = 64;        // workspace rows per head are padded to this
constexpr float kLog2e = 1.4426950408889634f;

template <int V> using IC = std::integral_constant<int, V>;

// lds_wait_upto<2 K>(a, b) for a K in 0..KMAX known only after unrolling.
template <int KMAX> struct WaitSel2 {
    static __device__ __forceinline__ void run(int k, i32x4& a, i32x4& b) {
        if (k >= KMAX) lds_wait_upto<2 * KMAX>(a, b);
        else WaitSel2<KMAX - 1>::run(k, a, b);
    }
};
template <> struct WaitSel2<0> {
    static __device__ __forceinline__ void run(int, i32x4& a, i32x4& b) { lds_wait_upto<0>(a, b); }
};
// lds_wait_upto<K>(a) for a K in 0..KMAX known only after unrolling.
template <int KMAX> struct WaitSel1 {
    static __device__ __forceinline__ void run(int k, i32x4& a) {
        if (k >= KMAX) lds_wait_upto<KMAX>(a);
        else WaitSel1<KMAX - 1>::run(k, a);
    }
};
template <> struct WaitSel1<0> {
    static __device__ __forceinline__ void run(int, i32x4& a) { lds_wait_upto<0>(a); }
};
// lds_wait_upto<2 K>(a, b) for two 8-byte results.
template <int KMAX> struct WaitSelT {
    static __device__ __forceinline__ void run(int k, i32x2& a, i32x2& b) {
        if (k >= KMAX) lds_wait_upto<2 * KMAX>(a, b);
        else WaitSelT<KMAX - 1>::run(k, a, b);
    }
};
template <> struct WaitSelT<0> {
    static __device__ __forceinline__ void run(int, i32x2& a, i32x2& b) { lds_wait_upto<0>(a, b); }
};

__host__ __device__ inline int padded_rows(int N) { return (N + PADR - 1) / PADR * PADR; }

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
// layout (the C layout of a product whose n index is the row), times f,
// straight from the registers (the dq kernel, at its register limit, keeps
// this form; the dk/dv kernel stages its rows through LDS).
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

// LDS slot source offsets for a [64][D] tile copied by 256 threads: copy p
// of this thread fills slot (p*4 + w)*64 + lane = tile row `row`, physical
// granule pg, which holds logical granule pg ^ key(row).
template <int D, int LOADS>
__device__ __forceinline__ void tile_sources(unsigned* src, int w, int lane) {
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
        const int slot = (p * 4 + w) * 64 + lane;
        const int row = slot / (D / 8), pg = slot % (D / 8);
        src[p] = (unsigned)(row * D * 2 + (pg ^ lds_key<D>(row)) * 16);
    }
}

// --------------------------------------------------------------------------
// dq_kernel: dQ for 128 query rows; K/V tiles stream past.
//   S^T = K Q^T, dP^T = V dO^T (keys x queries), P^T = 2^(S^T c - lse2),
//   dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// --------------------------------------------------------------------------
template <typename T, typename TO, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(NT, 2) void dq_kernel(BwdArgs a, int nqb, int total, int hgroup) {
    typedef typename Elem<T>::v8 v8;
    constexpr int ROWB = D * 2, TILE = BKT * ROWB, LOADS = TILE / (NT * 16);
    constexpr int KB = BKT / 32, DK = D / 16, DB = D / 32;
    constexpr bool SPLIT = SplitDS<T>::value;
    // SEED: every dP^T chain starts from -D_i (the lane's row) held in 16
    // registers for the whole kernel, so that it ends at dP - D and dS takes
    // one multiply.  Used where it measured faster: bf16, d = 128, causal
    // (at d = 128 the other types and the unmasked kernel spill with it; at
    // d = 64 the fp16 kernel ran 4% slower).  Elsewhere dS subtracts D.
    // Plain and dropout instantiations of one type, size and mask make the
    // same choice.
    constexpr bool SEED = D == 128 && CAUSAL && std::is_same_v<T, __bf16>;

    __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE];   // [stage][K | V]

    const int N = a.N, NP = padded_rows(N);
    const int tid = tid_x(), lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int s16 = lane & 15, grp = lane >> 4;

    const int L = xcd_remap(wg_x(), total);
    // Work: one query block of one (batch, head).  Under causal masking (the
    // dispatcher hands workgroup i to XCD i % 8, then to whichever of its
    // slots frees first):
    //  - hgroup > 0 (B*H a multiple of 8): XCD x takes the heads congruent to
    //    x modulo 8, hgroup heads at a time, each group's blocks heaviest
    //    first, so that the light blocks fill the slots the heavy ones free
    //    and only the last group's lightest blocks form the tail;
    //  - otherwise the pair of blocks nqb-1-p and p of one head, one after the
    //    other, so that every workgroup streams about as many K/V tiles as any
    //    other.
    // (wave-uniform: kept in scalar registers)
    int bh, qb_first, qb_second = 0, nitems = 1;
    if (CAUSAL && hgroup > 0) {
        const int i = wg_x(), x = i & 7, m = i >> 3;   // m-th workgroup of XCD x
        const int per = hgroup * nqb;                    // workgroups of one group
        const int g = m / per, rem = m - g * per;
        const int r = rem / hgroup, u = rem - r * hgroup;
        bh = 8 * (g * hgroup + u) + x;
        qb_first = nqb - 1 - r;
    } else if (CAUSAL) {
        const int npairs = (nqb + 1) >> 1;
        bh = L / npairs;
        const int p = L - bh * npairs;
        qb_first = nqb - 1 - p;
        qb_second = p;
        nitems = p != nqb - 1 - p ? 2 : 1;
    } else {
        bh = L / nqb;
        qb_first = L - bh * nqb;
    }
    bh = __builtin_amdgcn_readfirstlane(bh);
    qb_first = __builtin_amdgcn_readfirstlane(qb_first);
    qb_second = __builtin_amdgcn_readfirstlane(qb_second);
    nitems = __builtin_amdgcn_readfirstlane(nitems);
    // One query block; every tile step ends with a wait for this wave's
    // copies and a barrier, so a second block may refill the stages at once.
    // (called once or twice: one copy of the code per call, so that each is
    // allocated registers on its own)
    auto block = [&](const int qb) __attribute__((always_inline)) {
        const int q0 = qb * BQ;
        const size_t head = (size_t)bh * N * D;
        const T* __restrict__ Qh = (const T*)a.q + head;
        const T* __restrict__ Gh = (const T*)a.dO + head;
        const TO* __restrict__ Oh = (const TO*)a.o + head;
        const unsigned head_bytes = (unsigned)N * ROWB;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc((const T*)a.k + head, head_bytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const T*)a.v + head, head_bytes);

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
            qf[kk] = x;
            gf[kk] = g;
        }
        // D_i, divided by the keep factor under dropout
        const float delta = sum32(dpart) * (DROP ? 1.f / a.drop.scale : 1.f);
        const float lse2 = live ? a.lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
        // (the dropout instantiation, short of registers for the generator,
        // forms the same seed again before each chain instead of holding it)
        f32x16 ndseed = {};
        if constexpr (SEED && !DROP) {
    #pragma unroll
            for (int r = 0; r < 16; ++r) ndseed[r] = -delta;
        }
        if (live && h == 0) {
            a.ws[(size_t)bh * NP + qrow] = -delta;   // the dk/dv kernel starts its dP sums from it
            a.ws[((size_t)a.BH + bh) * NP + qrow] = lse2;
        }

        const int kend = CAUSAL ? min(N, q0 + BQ) : N;
        const int ntiles = (kend + BKT - 1) / BKT;

        unsigned src_off[LOADS];
        tile_sources<D, LOADS>(src_off, w, lane);
        auto issue = [&](auto stg, int t) {
            char* st = smem + decltype(stg)::value * 2 * TILE;
            const unsigned base = (unsigned)t * TILE;
    #pragma unroll
            for (int p = 0; p < LOADS; ++p) {
                dma16_async(krs, lds_addr(st + (p * 4 + w) * 1024), base + src_off[p]);
                dma16_async(vrs, lds_addr(st + TILE + (p * 4 + w) * 1024), base + src_off[p]);
            }
        };

        // K and V rows as A operands (16-byte reads, LDS byte addresses), K^T
        // through transposing reads
        unsigned roff[DK];
        const unsigned lbase = lds_addr(smem);
    #pragma unroll
        for (int kk = 0; kk < DK; ++kk) roff[kk] = lbase + t_off<D>(l32, 2 * kk + h);
        int toff[2][DB];
    #pragma unroll
        for (int cb = 0; cb < DB; ++cb) {
            const int col = 32 * cb + 16 * (grp & 1) + 4 * (s16 & 3);
            const int r0 = 4 * h + (s16 >> 2);
            toff[0][cb] = t_off<D>(r0, col >> 3) + (col & 7) * 2;
            toff[1][cb] = t_off<D>(r0 + 8, col >> 3) + (col & 7) * 2;
        }

        const float c = a.c;
        f32x16 acc[DB];
    #pragma unroll
        for (int cb = 0; cb < DB; ++cb)
    #pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

        auto tile = [&](auto stg, auto mask, int j0) {
            constexpr int STG = decltype(stg)::value;
            constexpr bool MASK = decltype(mask)::value;
            const char* sK = smem + STG * 2 * TILE;
            int nb = KB;
            if (MASK) {
                if (CAUSAL) {
                    const int lim = qlo + 31 - j0;
                    nb = lim < 0 ? 0 : min(KB, lim / 32 + 1);
                }
                nb = min(nb, (N - j0 + 31) / 32);
            }
            v8 dsb[KB][2], dsl[KB][2];
    #pragma unroll
            for (int b = 0; b < KB; ++b) {
                if (MASK && b >= nb) continue;
                f32x16 s, dp;
                // the row's generator call for this 32-key block: element r is
                // byte r % 4 of word r / 4
                unsigned ph[4];
                if (DROP) {
                    ph[0] = (unsigned)qrow;
                    ph[1] = (unsigned)(2 * ((j0 >> 5) + b) + h);
                    ph[2] = (unsigned)bh;
                    ph[3] = a.drop.offset;
    #pragma unroll
                    for (int n = 0; n < 10; ++n) philox_round(ph, a.drop.seed0, a.drop.seed1, n);
                }
                // S^T = K Q^T and dP^T = V dO^T alternate (step i is chain i % 2,
                // k-step i / 2); each step's K or V fragment is read DSD steps
                // ahead by inline assembly and waited for explicitly
                constexpr int NSD = 2 * DK, DSD = 3;
                i32x4 fr[DSD + 1];
                auto rd = [&](int i) __attribute__((always_inline)) {
                    fr[i % (DSD + 1)] = lds_read_b128_asm(roff[i >> 1], STG * 2 * TILE + (i & 1) * TILE + 32 * b * ROWB);
                };
    #pragma unroll
                for (int i = 0; i < DSD; ++i) rd(i);
    #pragma unroll
                for (int i = 0; i < NSD; ++i) {
                    WaitSel1<DSD - 1>::run(min(DSD - 1, NSD - 1 - i), fr[i % (DSD + 1)]);
                    const int kk = i >> 1;
                    if ((i & 1) == 0)
                        s = Elem<T>::mma(bit_cast<v8>(fr[i % (DSD + 1)]), bit_cast<v8>(qf[kk]), kk == 0 ? f32x16{} : s);
                    else {
                        f32x16 c0 = ndseed;
                        if constexpr (SEED && DROP) {
                            if (kk == 0) {
                                float nd = -delta;
                                __asm__ volatile("" : "+v"(nd));   // formed here, not held
    #pragma unroll
                                for (int r = 0; r < 16; ++r) c0[r] = nd;
                            }
                        }
                        dp = Elem<T>::mma(bit_cast<v8>(fr[i % (DSD + 1)]), bit_cast<v8>(gf[kk]), kk == 0 ? c0 : dp);
                    }
                    if (i + DSD < NSD) rd(i + DSD);
                }
    #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(fmaf(s[r], c, -lse2));
                    if (MASK) {
                        const int key = j0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
                        const bool ok = key < N && (!CAUSAL || key <= qrow);
                        p = ok ? p : 0.f;
                    }
                    const bool kp = !DROP || drop_keep(ph[r >> 2], r & 3, a.drop.t);
                    if constexpr (SEED) s[r] = p * (kp ? dp[r] : -delta);   // dp holds dP - D
                    else s[r] = p * ((kp ? dp[r] : 0.f) - delta);
                }
                dsb[b][0] = pack8<T>(s, 0);
                dsb[b][1] = pack8<T>(s, 1);
                if (SPLIT) {
                    dsl[b][0] = pack8_lo<T>(s, 0, dsb[b][0]);
                    dsl[b][1] = pack8_lo<T>(s, 1, dsb[b][1]);
                }
            }
            // dQ^T += K^T dS^T (a masked tile whose key blocks this wave all
            // sees takes the pipelined loop below)
            if (MASK && nb < KB) {
    #pragma unroll
                for (int cb = 0; cb < DB; ++cb) {
    #pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        if (b >= nb) continue;
    #pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int ro = (32 * b + 16 * q) * ROWB;
                            const v8 kt = join8<v8>(lds_read_tr16(sK, toff[0][cb] + ro),
                                                    lds_read_tr16(sK, toff[1][cb] + ro));
                            acc[cb] = Elem<T>::mma(kt, dsb[b][q], acc[cb]);
                            if (SPLIT) acc[cb] = Elem<T>::mma(kt, dsl[b][q], acc[cb]);
                        }
                    }
                }
            } else {
                // every key block: step i is column block i / (2 KB), key block
                // (i / 2) % KB, half i % 2; its two transposing reads are issued
                // DTR steps ahead by inline assembly and waited for explicitly
                constexpr int NTR = DB * KB * 2, DTR = 2;
                i32x2 ta[DTR + 1], tb[DTR + 1];
                const unsigned kl = lds_addr(smem);
                auto rdt = [&](int i) __attribute__((always_inline)) {
                    const int cb = i / (2 * KB), b = (i >> 1) % KB, q = i & 1;
                    const int imm = STG * 2 * TILE + (32 * b + 16 * q) * ROWB;
                    ta[i % (DTR + 1)] = lds_read_tr16_asm(kl + toff[0][cb], imm);
                    tb[i % (DTR + 1)] = lds_read_tr16_asm(kl + toff[1][cb], imm);
                };
    #pragma unroll
                for (int i = 0; i < DTR; ++i) rdt(i);
    #pragma unroll
                for (int i = 0; i < NTR; ++i) {
                    WaitSelT<DTR - 1>::run(min(DTR - 1, NTR - 1 - i), ta[i % (DTR + 1)], tb[i % (DTR + 1)]);
                    const int cb = i / (2 * KB), b = (i >> 1) % KB, q = i & 1;
                    const v8 kt = join8<v8>(bit_cast<i16x4>(ta[i % (DTR + 1)]), bit_cast<i16x4>(tb[i % (DTR + 1)]));
                    acc[cb] = Elem<T>::mma(kt, dsb[b][q], acc[cb]);
                    if (SPLIT) acc[cb] = Elem<T>::mma(kt, dsl[b][q], acc[cb]);
                    if (i + DTR < NTR) rdt(i + DTR);
                }
            }
        };

        auto step = [&](auto stg, int t) {
            constexpr int STG = decltype(stg)::value;
            if (t + 1 < ntiles) issue(IC<1 - STG>{}, t + 1);
            const int j0 = t * BKT;
            const bool need_mask = (j0 + BKT > N) || (CAUSAL && j0 + BKT - 1 > qlo);
            if (need_mask)
                tile(stg, std::true_type{}, j0);
            else
                tile(stg, std::false_type{}, j0);
            wait_vmem();
            __syncthreads();
        };

        issue(IC<0>{}, 0);
        wait_vmem();
        __syncthreads();
        int t = 0;
        for (; t + 1 < ntiles; t += 2) {
            step(IC<0>{}, t);
            step(IC<1>{}, t + 1);
        }
        if (t < ntiles) step(IC<0>{}, t);

        if (live) store_rows<TO, D>((TO*)a.dq + head + (size_t)qrow * D, acc, a.scale * (DROP ? a.drop.scale : 1.f), h);
    };
    block(qb_first);
    if (CAUSAL && nitems == 2) block(qb_second);
}

// --------------------------------------------------------------------------
// dkdv_kernel: dK, dV for 128 keys; Q/dO tiles of 64 queries stream past.
//   S = Q K^T, dP = dO V^T (queries x keys), P = 2^(S c - lse2),
//   dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
// Eight waves, two per SIMD: wave (kg, qh) owns keys 32 kg .. 32 kg + 31 of
// the block and query rows 32 qh .. 32 qh + 31 of every tile.  The block's
// K and V rows sit in LDS for the whole kernel; the two halves' partial dK
// and dV are added through LDS at the end.
// --------------------------------------------------------------------------
template <typename T, typename TO, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(NTK, 1) void dkdv_kernel(BwdArgs a, int nkb, int total) {
    typedef typename Elem<T>::v8 v8;
    constexpr int ROWB = D * 2;
    constexpr int TILE = BQT * ROWB;               // one Q or dO tile
    constexpr int KVB = BK * ROWB;                 // the K or V block
    constexpr int TLOADS = TILE / (NTK * 16), KLOADS = KVB / (NTK * 16);
    constexpr int DK = D / 16, DB = D / 32;
    constexpr int STAGE = 2 * TILE;                // Q tile, dO tile
    constexpr int KOFF = 2 * STAGE;                // K block, then V block
    constexpr int LOFF = KOFF + 2 * KVB;           // per stage: lse2[64], D[64]
    constexpr int MOFF = LOFF + 2 * 2 * BQT * 4;   // dropout: per wave 32 x 32 mask bytes
    constexpr int SMEM = MOFF + (DROP ? 8 * 1024 : 0);
    constexpr bool SPLIT = SplitDS<T>::value;
    static_assert(4 * 2 * DB * 16 * 64 * 4 <= SMEM, "reduction area must fit in LDS");
    static_assert(2 * STAGE <= 65536, "stage reads use 16-bit immediate offsets");

    // [stage 0: Q | dO][stage 1: Q | dO][K block][V block][lse2 | D per stage]
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int N = a.N, NP = padded_rows(N);
    const int tid = tid_x(), lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = w & 3, qh = w >> 2;
    const int l32 = lane & 31, h = lane >> 5;
    const int s16 = lane & 15, grp = lane >> 4;

    const int L = xcd_remap(wg_x(), total);
    // Work: one key block of one (batch, head); under causal masking the pair
    // of blocks p (most queries) and nkb-1-p of one head, one after the
    // other, so that every workgroup streams about as many Q/dO tiles as any
    // other (wave-uniform: kept in scalar registers)
    int bh, kb_first, kb_second = 0, nitems = 1;
    if (CAUSAL) {
        const int npairs = (nkb + 1) >> 1;
        bh = L / npairs;
        const int p = L - bh * npairs;
        kb_first = p;
        kb_second = nkb - 1 - p;
        nitems = p != nkb - 1 - p ? 2 : 1;
    } else {
        bh = L / nkb;
        kb_first = L - bh * nkb;
    }
    bh = __builtin_amdgcn_readfirstlane(bh);
    kb_first = __builtin_amdgcn_readfirstlane(kb_first);
    kb_second = __builtin_amdgcn_readfirstlane(kb_second);
    nitems = __builtin_amdgcn_readfirstlane(nitems);
    // One key block (called once or twice: one copy of the code per call, so
    // that each is allocated registers on its own).
    auto key_block = [&](const int kblk) __attribute__((always_inline)) {
        const int kb0 = kblk * BK;
        const size_t head = (size_t)bh * N * D;
        const unsigned head_bytes = (unsigned)N * ROWB;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc((const T*)a.k + head, head_bytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const T*)a.v + head, head_bytes);
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const T*)a.q + head, head_bytes);
        const __amdgpu_buffer_rsrc_t grs = make_rsrc((const T*)a.dO + head, head_bytes);
        const __amdgpu_buffer_rsrc_t drs = make_rsrc(a.ws + (size_t)bh * NP, (unsigned)N * 4);
        const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.ws + ((size_t)a.BH + bh) * NP, (unsigned)N * 4);

        const int kw0 = kb0 + 32 * kg;      // this wave's first key
        const int key = kw0 + l32;          // this lane's key

        // LDS slot s of a [rows][D] region holds row s / (D/8), physical granule
        // s % (D/8): the 16-byte piece at logical granule pg ^ key(row).
        auto src_of = [&](int slot) {
            const int row = slot / (D / 8), pg = slot % (D / 8);
            return (unsigned)(row * ROWB + (pg ^ lds_key<D>(row)) * 16);
        };
        // the block's K and V rows (rows past the end read as zeros)
    #pragma unroll
        for (int p = 0; p < KLOADS; ++p) {
            const int slot = (p * 8 + w) * 64 + lane;
            const unsigned off = (unsigned)kb0 * ROWB + src_of(slot);
            dma16_async(krs, lds_addr(smem + KOFF + (p * 8 + w) * 1024), off);
            dma16_async(vrs, lds_addr(smem + KOFF + KVB + (p * 8 + w) * 1024), off);
        }

        const int t0 = CAUSAL ? kb0 / BQT : 0;
        const int ntiles = (N + BQT - 1) / BQT;

        unsigned tsrc[TLOADS];
    #pragma unroll
        for (int p = 0; p < TLOADS; ++p) tsrc[p] = src_of((p * 8 + w) * 64 + lane);
        auto issue = [&](auto stg, int t) {
            constexpr int STG = decltype(stg)::value;
            char* st = smem + STG * STAGE;
            const unsigned base = (unsigned)t * TILE;
    #pragma unroll
            for (int p = 0; p < TLOADS; ++p) {
                dma16_async(qrs, lds_addr(st + (p * 8 + w) * 1024), base + tsrc[p]);
                dma16_async(grs, lds_addr(st + TILE + (p * 8 + w) * 1024), base + tsrc[p]);
            }
            // the tile's lse2 and D values: 64 floats each, 16 lanes of wave 0
            if (w == 0 && lane < BQT / 4) {
                const unsigned fo = (unsigned)(t * BQT + 4 * lane) * 4;
                dma16_async(lrs, lds_addr(smem + LOFF + STG * 2 * BQT * 4), fo);
                dma16_async(drs, lds_addr(smem + LOFF + STG * 2 * BQT * 4 + BQT * 4), fo);
            }
        };

        // Per-lane LDS offsets; every read below adds only a compile-time
        // immediate (stage, tensor, half tile) below 64 KiB.
        // LDS byte addresses of this lane's Q (dO) and K (V) operand reads: rows l32
        // (+ this wave's 32 rows) at granule 2kk + h; stage, tensor and V offsets
        // are added as immediates
        unsigned qaddr[DK], kaddr[DK];
        const unsigned lbase = lds_addr(smem);
    #pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
            const int o = t_off<D>(l32, 2 * kk + h);
            qaddr[kk] = lbase + o + 32 * qh * ROWB;
            kaddr[kk] = lbase + o + 32 * kg * ROWB + KOFF;
        }
        // transposing reads (LDS byte addresses): rows 32qh + 4h + s16/4 (+8)
        unsigned taddr[2][DB];
    #pragma unroll
        for (int cb = 0; cb < DB; ++cb) {
            const int col = 32 * cb + 16 * (grp & 1) + 4 * (s16 & 3);
            const int r0 = 4 * h + (s16 >> 2);
            taddr[0][cb] = lbase + t_off<D>(r0, col >> 3) + (col & 7) * 2 + 32 * qh * ROWB;
            taddr[1][cb] = lbase + t_off<D>(r0 + 8, col >> 3) + (col & 7) * 2 + 32 * qh * ROWB;
        }
        const int laddr = LOFF + (32 * qh + 4 * h) * 4;   // lse2 / D of this lane's rows

        const float c = a.c;   // signed exponent unit: no maximum is tracked here
        f32x16 dk[DB], dv[DB];
    #pragma unroll
        for (int cb = 0; cb < DB; ++cb)
    #pragma unroll
            for (int r = 0; r < 16; ++r) {
                dk[cb][r] = 0.f;
                dv[cb][r] = 0.f;
            }

        // This wave's 32 queries of a staged tile.  MASK: the block straddles
        // the causal diagonal of this wave's keys (only the first two tiles of a
        // key block can; they run before the main loop).
        auto block = [&](auto stg, auto mask, int i0) {
            constexpr int STG = decltype(stg)::value;
            constexpr bool MASK = decltype(mask)::value;
            // S = Q K^T and dP = dO V^T: the two chains alternate (step i is
            // chain i % 2, k-step i / 2), and each step's operand pair is read
            // DSD steps ahead by inline assembly, waited for explicitly
            constexpr int NSD = 2 * DK, DSD = 3;
            f32x16 s, dp;
            // the dP chain starts from -D of the lane's rows (the workspace holds
            // -D; -D' under dropout), so that it ends at dP - D; element r of the
            // accumulator is row 32 qh + 8(r/4) + 4h + r%4, as -D is laid out
            f32x16 dinit;
    #pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 nd = *(const f32x4*)(smem + laddr + STG * 2 * BQT * 4 + BQT * 4 + 32 * rr);
    #pragma unroll
                for (int e = 0; e < 4; ++e) dinit[4 * rr + e] = nd[e];
            }
            i32x4 fa[DSD + 1], fb[DSD + 1];
            auto rd = [&](int i) __attribute__((always_inline)) {
                const int kk = i >> 1, g = i & 1;
                fa[i % (DSD + 1)] = lds_read_b128_asm(qaddr[kk], STG * STAGE + g * TILE);
                fb[i % (DSD + 1)] = lds_read_b128_asm(kaddr[kk], g * KVB);
            };
    #pragma unroll
            for (int i = 0; i < DSD; ++i) rd(i);
    #pragma unroll
            for (int i = 0; i < NSD; ++i) {
                const int later = min(DSD - 1, NSD - 1 - i);   // pairs read after this one
                WaitSel2<DSD - 1>::run(later, fa[i % (DSD + 1)], fb[i % (DSD + 1)]);
                const int kk = i >> 1;
                if ((i & 1) == 0)
                    s = Elem<T>::mma(bit_cast<v8>(fa[i % (DSD + 1)]), bit_cast<v8>(fb[i % (DSD + 1)]), kk == 0 ? f32x16{} : s);
                else
                    dp = Elem<T>::mma(bit_cast<v8>(fa[i % (DSD + 1)]), bit_cast<v8>(fb[i % (DSD + 1)]), kk == 0 ? dinit : dp);
                if (i + DSD < NSD) rd(i + DSD);
            }
            // Dropout: this lane runs the generator call of row 32 qh + l32 and
            // lane half h, whose byte e % 4 of word e / 4 belongs to key
            // 8(e/4) + 4h + e%4 of the wave's 32; the bytes pass through the
            // wave's LDS area as [key][row], from which the lane reads, for its
            // key, rows 8(r/4) + 4h .. + 3 as one word per r/4.
            unsigned mw[4];
            if (DROP) {
                unsigned ph[4] = {(unsigned)(i0 + 32 * qh + l32), (unsigned)(2 * (kw0 >> 5) + h), (unsigned)bh,
                                  a.drop.offset};
    #pragma unroll
                for (int n = 0; n < 10; ++n) philox_round(ph, a.drop.seed0, a.drop.seed1, n);
                unsigned char* mt = (unsigned char*)smem + MOFF + w * 1024;
    #pragma unroll
                for (int g = 0; g < 4; ++g)
    #pragma unroll
                    for (int e = 0; e < 4; ++e) mt[(8 * g + 4 * h + e) * 32 + l32] = (unsigned char)(ph[g] >> (8 * e));
    #pragma unroll
                for (int g = 0; g < 4; ++g) mw[g] = *(const unsigned*)(mt + l32 * 32 + 8 * g + 4 * h);
            }
            // rows of this block held by the lane: 32 qh + 8(r/4) + 4h + r%4
            f32x16 p;
    #pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 l4 = *(const f32x4*)(smem + laddr + STG * 2 * BQT * 4 + 32 * rr);
                f32x4 nd4 = {};   // -D' (dropout)
                if (DROP) nd4 = *(const f32x4*)(smem + laddr + STG * 2 * BQT * 4 + BQT * 4 + 32 * rr);
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rr + e;
                    float pv = fast_exp2(fmaf(s[r], c, -l4[e]));
                    if (MASK) pv = (key <= i0 + 32 * qh + 8 * rr + 4 * h + e) ? pv : 0.f;
                    if (DROP) {
                        const bool kp = drop_keep(mw[rr], e, a.drop.t);
                        p[r] = kp ? pv : 0.f;                    // weights applied to dO (dV)
                        s[r] = pv * (kp ? dp[r] : nd4[e]);   // dS / r (dp holds dP~ - D')
                    } else {
                        p[r] = pv;
                        s[r] = pv * dp[r];   // dS (dp holds dP - D)
                    }
                }
            }
            const v8 pb0 = pack8<T>(p, 0), pb1 = pack8<T>(p, 1);
            const v8 db0 = pack8<T>(s, 0), db1 = pack8<T>(s, 1);
            v8 dl0 = db0, dl1 = db1;
            if (SPLIT) {
                dl0 = pack8_lo<T>(s, 0, db0);
                dl1 = pack8_lo<T>(s, 1, db1);
            }
            // dV^T += dO^T P,  dK^T += Q^T dS  (transposing reads of the tiles):
            // step i is column block i / 4, half (i / 2) % 2, dV for even i and dK
            // for odd i; its two reads are issued DTR steps ahead
            constexpr int NTR = 4 * DB, DTR = 3;
            i32x2 ta[DTR + 1], tb[DTR + 1];
            auto rdt = [&](int i) __attribute__((always_inline)) {
                const int cb = i >> 2, q = (i >> 1) & 1, isq = i & 1;
                const int imm = STG * STAGE + (isq ? 0 : TILE) + 16 * q * ROWB;
                ta[i % (DTR + 1)] = lds_read_tr16_asm(taddr[0][cb], imm);
                tb[i % (DTR + 1)] = lds_read_tr16_asm(taddr[1][cb], imm);
            };
    #pragma unroll
            for (int i = 0; i < DTR; ++i) rdt(i);
    #pragma unroll
            for (int i = 0; i < NTR; ++i) {
                WaitSelT<DTR - 1>::run(min(DTR - 1, NTR - 1 - i), ta[i % (DTR + 1)], tb[i % (DTR + 1)]);
                const int cb = i >> 2, q = (i >> 1) & 1;
                const v8 op = join8<v8>(bit_cast<i16x4>(ta[i % (DTR + 1)]), bit_cast<i16x4>(tb[i % (DTR + 1)]));
                if ((i & 1) == 0) {
                    dv[cb] = Elem<T>::mma(op, q ? pb1 : pb0, dv[cb]);
                } else {
                    dk[cb] = Elem<T>::mma(op, q ? db1 : db0, dk[cb]);
                    if (SPLIT) dk[cb] = Elem<T>::mma(op, q ? dl1 : dl0, dk[cb]);
                }
                if (i + DTR < NTR) rdt(i + DTR);
            }
        };

        auto step = [&](auto stg, auto mask, int t) {
            constexpr int STG = decltype(stg)::value;
            if (t + 1 < ntiles) issue(IC<1 - STG>{}, t + 1);
            const int i0 = t * BQT;
            const int ib = i0 + 32 * qh;        // first query of this wave's rows
            const bool skip = ib >= N || (CAUSAL && ib + 31 < kw0);   // every query before every key
            if (!skip) block(stg, mask, i0);
            wait_vmem();
            __syncthreads();
        };

        if (t0 < ntiles) issue(IC<0>{}, t0);
        wait_vmem();
        __syncthreads();
        int t = t0;
        if (CAUSAL) {
            // the key block spans queries kb0 .. kb0 + 127: tiles t0 and t0 + 1
            if (t < ntiles) step(IC<0>{}, std::true_type{}, t++);
            if (t < ntiles) step(IC<1>{}, std::true_type{}, t++);
        }
        for (; t + 1 < ntiles; t += 2) {
            step(IC<0>{}, std::false_type{}, t);
            step(IC<1>{}, std::false_type{}, t + 1);
        }
        if (t < ntiles) step(IC<0>{}, std::false_type{}, t);

        // the two query halves of each key group: qh = 1 hands its partial sums
        // to qh = 0 through LDS ([kg][accumulator quad][lane] of 16 bytes)
        f32x4* red = (f32x4*)smem + kg * (2 * DB * 4) * 64;
        if (qh == 1) {
    #pragma unroll
            for (int cb = 0; cb < DB; ++cb)
    #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    red[((cb * 4 + g) * 2 + 0) * 64 + lane] = {dk[cb][4 * g], dk[cb][4 * g + 1], dk[cb][4 * g + 2], dk[cb][4 * g + 3]};
                    red[((cb * 4 + g) * 2 + 1) * 64 + lane] = {dv[cb][4 * g], dv[cb][4 * g + 1], dv[cb][4 * g + 2], dv[cb][4 * g + 3]};
                }
        }
        __syncthreads();
        // (the whole wave takes part: the staged store below writes rows by
        // lane other than the lanes' own keys; rows past N are not written)
        if (qh == 0) {
    #pragma unroll
            for (int cb = 0; cb < DB; ++cb)
    #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 xk = red[((cb * 4 + g) * 2 + 0) * 64 + lane];
                    const f32x4 xv = red[((cb * 4 + g) * 2 + 1) * 64 + lane];
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dk[cb][4 * g + e] += xk[e];
                        dv[cb][4 * g + e] += xv[e];
                    }
                }
            const float rs = DROP ? a.drop.scale : 1.f;
            // dK and dV leave through LDS as whole rows, staged in this key
            // group's part of the reduction area (only this wave reads or
            // writes it after the barrier; its reads above complete first)
            char* const stg = (char*)red;
            store_rows_staged<TO, D>(stg, (TO*)a.dk + head + (size_t)kw0 * D, N - kw0, dk, a.scale * rs, lane);
            store_rows_staged<TO, D>(stg + 32 * D * (int)sizeof(TO), (TO*)a.dv + head + (size_t)kw0 * D,
                                     N - kw0, dv, rs, lane);
        }
    };
    key_block(kb_first);
    if (CAUSAL && nitems == 2) {
        __syncthreads();   // the last block's LDS reads (its reduction) are done
        key_block(kb_second);
    }
}

template <typename T, typename TO, int D, bool CAUSAL, bool DROP>
hipError_t launch(const BwdArgs& a, int which, hipStream_t stream) {
    if (which & 1) {
        const int nqb = (a.N + BQ - 1) / BQ;
        const int hg = xcd_head_group(a.BH, CAUSAL);
        // causal: every query block on its own (head groups) or pairs of them
        const int tq = hg ? a.BH * nqb : a.BH * (CAUSAL ? (nqb + 1) / 2 : nqb);
        hipLaunchKernelGGL((dq_kernel<T, TO, D, CAUSAL, DROP>), dim3(tq), dim3(NT), 0, stream, a, nqb, tq, hg);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (which & 2) {
        const int nkb = (a.N + BK - 1) / BK;
        const int tk = a.BH * (CAUSAL ? (nkb + 1) / 2 : nkb);   // causal: pairs of key blocks
        hipLaunchKernelGGL((dkdv_kernel<T, TO, D, CAUSAL, DROP>), dim3(tk), dim3(NTK), 0, stream, a, nkb, tk);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T, typename TO, int D, bool CAUSAL>
hipError_t launch_d(const BwdArgs& a, int which, hipStream_t stream) {
    return a.drop.on ? launch<T, TO, D, CAUSAL, true>(a, which, stream)
                     : launch<T, TO, D, CAUSAL, false>(a, which, stream);
}

template <typename T, typename TO>
hipError_t launch_t(const BwdArgs& a, int which, int d, int causal, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_d<T, TO, 64, true>(a, which, stream) : launch_d<T, TO, 64, false>(a, which, stream);
    return causal ? launch_d<T, TO, 128, true>(a, which, stream) : launch_d<T, TO, 128, false>(a, which, stream);
}

}  // namespace

size_t bwd_workspace_bytes(int64_t BH, int64_t N) {
    return size_t(2) * size_t(BH) * size_t(padded_rows(int(N))) * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs& a, int which, int dtype, bool out_f32, int d, int causal,
                      hipStream_t stream) {
    if (dtype == 1)
        return out_f32 ? launch_t<__bf16, float>(a, which, d, causal, stream)
                       : launch_t<__bf16, __bf16>(a, which, d, causal, stream);
    return out_f32 ? launch_t<_Float16, float>(a, which, d, causal, stream)
                   : launch_t<_Float16, _Float16>(a, which, d, causal, stream);
}

}  // namespace attn
