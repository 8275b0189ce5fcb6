// attn_fwd.hip -- fused attention forward for gfx950.
//
// One workgroup owns one block of BR = 128 query rows of one (batch, head);
// each of its four waves owns 32 of those rows for the whole kernel and
// writes their output once ("FlashAttention" explainer, Step 3 "Tiling":
// one Q block stays on chip while K/V tiles stream past, and each block's
// output is written once).  K/V tiles of BC = 64 keys go straight from
// global memory into one of two LDS stages (16-byte direct-to-LDS copies,
// coalesced, zero-filled past the end of the sequence by the buffer bounds
// check): tile t+1 is in flight while tile t is consumed, with one barrier
// per tile.  Two workgroups share a CU, so one wave's softmax can overlap
// another's matrix products.
//
// Per tile and wave (the pages' online softmax: "13% more FLOPs, 5.7x
// faster", sections "Softmax is the anti-tiling operation" and
// "FlashAttention's move: rescale the output, too"; explainer Step 4):
//   S^T = K Q^T         on the matrix cores (keys x queries, fp32)
//   mask                causal and ragged-tail tiles only
//   m_t = rowmax S               lanes own query rows; one cross-lane step
//   reference mc: the scaled running maximum, moved to m_t c only when
//                 that exceeds it by more than kTau binades (the first
//                 tile always moves it); alpha = 2^(mc_old - mc_new)
//   P = 2^(S c - mc),  c = |scale| log2(e);  l = alpha l + rowsum P
//   O^T = alpha O^T + V^T P^T    V^T read from the row-major tile with
//                                transposing LDS reads
// and after the last tile O = O^T / l (rounded once), lse = (mc + log2 l) ln 2.
// Any reference point gives the same O and lse (2^(x - m) = 2^(x - m')
// 2^(m' - m), the identity behind the pages' rescale); keeping it within
// kTau binades of the true maximum bounds P by 2^kTau, so nothing overflows,
// and lets most tiles skip the rescale of the accumulator.
// S and P exist only in registers; nothing of size N x N touches memory.
#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int BR = 128;   // query rows per workgroup
constexpr int BC = 64;    // keys per K/V tile
constexpr int NT = 256;   // threads per workgroup (4 waves)
// The exponent's reference point moves only when a row's maximum rises by
// more than kTau binades, so P <= 2^kTau and most tiles skip the rescale.
constexpr float kTau = 8.f;

template <int V> using IC = std::integral_constant<int, V>;

template <typename T, typename TO, int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void fwd_kernel(FwdArgs a) {
    typedef typename Elem<T>::v8 v8;
    constexpr int ROWB = D * 2;            // bytes per tile row
    constexpr int GR = D / 8;              // 16-byte granules per row
    constexpr int TILE = BC * ROWB;        // bytes of one K (or V) tile
    constexpr int LOADS = TILE / (NT * 16);  // copies per thread per tile and tensor
    constexpr int KB = BC / 32;            // 32-key blocks per tile
    constexpr int DK = D / 16;             // k-steps of the S product
    constexpr int DB = D / 32;             // 32-wide output column blocks

    // [stage][K | V][tile]
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];

    const int N = a.N;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
    const int l32 = lane & 31, h = lane >> 5;
    const int s16 = lane & 15, grp = lane >> 4;

    const int L = xcd_remap(blockIdx.x, a.total);
    const int bh = L / a.nqb;
    int qb = L - bh * a.nqb;
    if (CAUSAL) qb = a.nqb - 1 - qb;  // heaviest query blocks first
    const int q0 = qb * BR;
    const size_t head = (size_t)bh * N * D;
    const T* __restrict__ Qh = (const T*)a.q + head;
    const unsigned head_bytes = (unsigned)N * ROWB;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc((const T*)a.k + head, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const T*)a.v + head, head_bytes);

    // This lane's query row and its Q fragment (B operand of S^T = K Q^T).
    const int qlo = q0 + 32 * w;
    const int qrow = qlo + l32;
    i32x4 qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        i32x4 x = {0, 0, 0, 0};
        if (qrow < N) x = *(const i32x4*)(Qh + (size_t)qrow * D + 16 * kk + 8 * h);
        if (a.negate) x ^= (int)0x80008000;   // scale < 0: use -Q and |scale|
        qf[kk] = x;
    }

    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kend + BC - 1) / BC;

    // K and V tiles have separate double buffers: K runs one tile ahead of V,
    // because the products S = K Q^T for tile t+1 are issued while tile t's
    // exponents and P.V products run.  Copy p of this thread fills LDS slot
    // (p*4 + w)*64 + lane of a tile: row `row`, physical granule pg, which
    // holds logical granule pg ^ key(row) of that row (the t_off placement).
    unsigned src_off[LOADS];
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
        const int slot = (p * 4 + w) * 64 + lane;
        const int row = slot / GR, pg = slot % GR;
        src_off[p] = (unsigned)(row * ROWB + (pg ^ lds_key<D>(row)) * 16);
    }
    // smem: K slot 0, K slot 1, V slot 0, V slot 1.  Copies of tiles past
    // the end of the sequence read zeros and are never consumed.
    auto issue = [&](auto which, auto slot, int t) {
        char* st = smem + (decltype(which)::value * 2 + decltype(slot)::value) * TILE;
        const __amdgpu_buffer_rsrc_t rs = decltype(which)::value ? vrs : krs;
        const unsigned base = (unsigned)t * TILE;
#pragma unroll
        for (int p = 0; p < LOADS; ++p) dma16(rs, st + (p * 4 + w) * 1024, base + src_off[p]);
    };

    // Loop-invariant LDS offsets of this lane's operand reads; the block,
    // half-tile and slot parts are added as immediates (the swizzle key
    // depends on the row modulo 16 only).
    int koff[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) koff[kk] = t_off<D>(l32, 2 * kk + h);
    int voff[2][DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {
        const int col = 32 * cb + 16 * (grp & 1) + 4 * (s16 & 3);
        const int r0 = 4 * h + (s16 >> 2);
        voff[0][cb] = t_off<D>(r0, col >> 3) + (col & 7) * 2;
        voff[1][cb] = t_off<D>(r0 + 8, col >> 3) + (col & 7) * 2;
    }

    const float c = a.c;   // > 0 (the host maps a zero scale to the smallest normal unit)
    f32x16 oacc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    float mc_run = -INFINITY;   // exponent reference (scaled units) of this row
    // this lane's share of the row's normaliser, twice: the sum of P as
    // rounded for the P.V product (it normalises O, so O's weights sum to
    // one exactly as used) and the fp32 sum of P (it gives lse)
    float l_run = 0.f, lf_run = 0.f;

    // S^T = K Q^T for a whole tile (every 32-key block; blocks a wave cannot
    // see are masked to -inf afterwards and then contribute exactly zero).
    auto scores = [&](auto kslot, f32x16 (&s)[KB]) {
        const char* sK = smem + decltype(kslot)::value * TILE;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const i32x4 kx = *(const i32x4*)(sK + koff[kk] + 32 * b * ROWB);
                s[b] = Elem<T>::mma(bit_cast<v8>(kx), bit_cast<v8>(qf[kk]), kk == 0 ? f32x16{} : s[b]);
            }
    };

    // Mask tile j0's scores if needed, then move the row's reference when
    // its maximum rose by more than kTau binades; rescale l and O by the
    // factor (O already holds every earlier tile's P.V).
    auto rowmax_update = [&](f32x16 (&s)[KB], int j0) {
        const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qlo);
        if (need_mask) [[unlikely]] {
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
                    const bool ok = key < N && (!CAUSAL || key <= qrow);
                    s[b][r] = ok ? s[b][r] : -INFINITY;
                }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[b][r], s[b][r + 1]));
        const float tc = max32(mt) * c;
        const bool upd = tc > mc_run + kTau;
        const float mc = upd ? tc : mc_run;
        const float alpha = upd ? fast_exp2(mc_run - mc) : 1.f;
        mc_run = mc;
        l_run *= alpha;
        lf_run *= alpha;
        if (__ballot(upd) != 0) [[unlikely]] {
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        }
    };

    // P = 2^(S c - mc) for a tile whose reference is settled, packed to the
    // operand type, and O^T += V^T P^T.  B operand chunk (b, q) holds, at
    // k = 8h + e, the probability of key 32b + 16q + 8(e/4) + 4h + e%4; the
    // transposing reads fetch V at exactly those keys.
    auto exp_pv = [&](auto vslot, f32x16 (&s)[KB]) {
        const char* sV = smem + (2 + decltype(vslot)::value) * TILE;
        const float mc = mc_run;
        float lsum = 0.f, lfsum = 0.f;
        v8 pb[KB][2];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[b][r] = fast_exp2(fmaf(s[b][r], c, -mc));
                lfsum += s[b][r];
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const f32x4 lo = {s[b][8 * q + 0], s[b][8 * q + 1], s[b][8 * q + 2], s[b][8 * q + 3]};
                const f32x4 hi = {s[b][8 * q + 4], s[b][8 * q + 5], s[b][8 * q + 6], s[b][8 * q + 7]};
                const auto l4 = Elem<T>::cvt4(lo);
                const auto h4 = Elem<T>::cvt4(hi);
                pb[b][q] = __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
                lsum = Elem<T>::sum8(pb[b][q], lsum);
            }
        }
        l_run += lsum;
        lf_run += lfsum;
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int roff = (32 * b + 16 * q) * ROWB;
                    const i16x4 lo = lds_read_tr16(sV, voff[0][cb] + roff);
                    const i16x4 hi = lds_read_tr16(sV, voff[1][cb] + roff);
                    oacc[cb] = Elem<T>::mma(join8<v8>(lo, hi), pb[b][q], oacc[cb]);
                }
    };

    // Iteration t: K(t+2) and V(t+1) copies start; S for tile t+1 (its K
    // arrived one iteration ago) is issued while tile t's exponents and
    // P.V products run; then tile t+1's mask, row maximum and reference.
    // Invariant at the top: tile t's scores are in `cur`, K(t+1) and V(t)
    // are in LDS, and no wave still reads K(t)'s slot.
    auto step = [&](auto par, int t, f32x16 (&cur)[KB], f32x16 (&nxt)[KB]) {
        constexpr int P = decltype(par)::value;   // t % 2
        issue(IC<0>{}, IC<P>{}, t + 2);
        issue(IC<1>{}, IC<1 - P>{}, t + 1);
        scores(IC<1 - P>{}, nxt);
        exp_pv(IC<P>{}, cur);
        if (t + 1 < ntiles) rowmax_update(nxt, (t + 1) * BC);
        wait_vmem();
        __syncthreads();
    };

    f32x16 sA[KB], sB[KB];
    issue(IC<0>{}, IC<0>{}, 0);
    issue(IC<1>{}, IC<0>{}, 0);
    issue(IC<0>{}, IC<1>{}, 1);
    wait_vmem();
    __syncthreads();
    scores(IC<0>{}, sA);
    rowmax_update(sA, 0);
    __syncthreads();   // every wave is done with K(0)'s slot
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(IC<0>{}, t, sA, sB);
        step(IC<1>{}, t + 1, sB, sA);
    }
    if (t < ntiles) step(IC<0>{}, t, sA, sB);

    // epilogue: O = O^T / l, one rounding; lse = (mc + log2 l) ln 2
    const float l_tot = sum32(l_run);
    const float lf_tot = sum32(lf_run);
    const float inv = fast_rcp(l_tot);
    if (qrow < N) {
        TO* __restrict__ orow = (TO*)a.o + head + (size_t)qrow * D;
#pragma unroll
        for (int cb = 0; cb < DB; ++cb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x = {oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv,
                           oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv};
                store4<TO>(orow + 32 * cb + 8 * g + 4 * h, x);
            }
        }
        if (h == 0) a.lse[(size_t)bh * N + qrow] = (mc_run + fast_log2(lf_tot)) * 0.69314718055994531f;
    }
}

template <typename T, typename TO, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_kernel<T, TO, D, CAUSAL>), dim3(a.total), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_t(const FwdArgs& a, int d, int causal, hipStream_t stream) {
    if (d == 64) return causal ? launch<T, TO, 64, true>(a, stream) : launch<T, TO, 64, false>(a, stream);
    return causal ? launch<T, TO, 128, true>(a, stream) : launch<T, TO, 128, false>(a, stream);
}

}  // namespace

int fwd_block_rows() { return BR; }

hipError_t launch_fwd(const FwdArgs& a, int dtype, bool out_f32, int d, int causal, hipStream_t stream) {
    if (dtype == 1)
        return out_f32 ? launch_t<__bf16, float>(a, d, causal, stream)
                       : launch_t<__bf16, __bf16>(a, d, causal, stream);
    return out_f32 ? launch_t<_Float16, float>(a, d, causal, stream)
                   : launch_t<_Float16, _Float16>(a, d, causal, stream);
}

}  // namespace attn
