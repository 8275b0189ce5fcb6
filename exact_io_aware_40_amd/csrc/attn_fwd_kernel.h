// attn_fwd_kernel.h -- the fused attention forward kernel for gfx950.
// attn_decode.hip instantiates it for grids whose K/V tiles each have a
// single reader (ONCE: one query block per (batch, head), no dropout), with
// non-temporal K/V copies; attn_fwd.hip for every other launch.
//
// One workgroup owns BR = 128 query rows of one (batch, head) -- under causal
// masking with B*H not a multiple of 8, a pair of such blocks, one after the
// other (otherwise XCD head groups, below) -- and streams the K/V
// tiles those rows can see through LDS ("FlashAttention" explainer, Step 3
// "Tiling": a Q block stays on chip while K/V tiles stream past, and each
// block's output is written once).  Each of its four waves owns 32 of the
// rows for the whole block; two workgroups share a CU, so every SIMD runs
// two waves.  A tile holds 8 KiB of keys (32 keys at d = 128, 64 at d = 64).
//
// Per tile and wave (the pages' online softmax: sections "Softmax is the
// anti-tiling operation" and "FlashAttention's move: rescale the output,
// too"; explainer Step 4):
//   S^T = K Q^T         on the matrix cores (keys x queries, fp32)
//   mask                causal, ragged-tail and out-of-range tiles only
//   P = 2^(S c - mc),  c = |scale| log2(e), with the reference mc as it
//                 stands; l = alpha l + rowsum P
//   reference mc: the scaled running maximum, moved to m_t c, m_t = rowmax S
//                 (lanes own query rows; one cross-lane step), only when
//                 that exceeds it by more than kTau binades (32 for bf16
//                 operands, 15 for fp16; the first tile always moves it);
//                 alpha = 2^(mc_old - mc_new).  With 16-bit operands the
//                 row maximum is taken only for a tile in which some lane's
//                 sum of P exceeds 2^kTau (then P is formed again); every
//                 other tile leaves the reference where it is, since all
//                 its P are within 2^kTau.  8-bit: m_t first, then P.
//   O^T = alpha O^T + V^T P^T    V^T read from the row-major tile with
//                                transposing LDS reads
// and after the last tile O = O^T / l (rounded once), lse = (mc + log2 l) ln 2.
// Any reference point gives the same O and lse (2^(x - m) = 2^(x - m')
// 2^(m' - m), the identity behind the pages' rescale); keeping it within
// kTau binades of the true maximum bounds P by 2^kTau, so nothing overflows,
// and lets almost every tile skip the rescale of the accumulator.
// S and P exist only in registers; nothing of size N x N touches memory.
//
// Schedule.  Iteration t of a wave issues, interleaved: the softmax of tile
// t (vector ALU), cut into pieces; the products for S of tile t+1 and for
// P.V of tile t-1 (matrix cores), whose LDS operands are read four steps
// ahead; and the direct-to-LDS copies of K(t+4) and V(t+2) into rings of
// five buffers (all 160 KiB of LDS at two workgroups per CU), which lets one
// barrier serve two iterations.  The copies and the operand reads are written as inline
// assembly so that neither waits for the other (they never touch the same
// buffer), with explicit waits where the data is consumed.  Every wave
// walks every tile of its block: tiles past a wave's diagonal are masked
// entirely and contribute exactly zero.
//
// Split K/V (Flash-Decoding, explainer "Common questions"): a work item is one
// query block and one chunk of its tiles; the item writes its own softmax's
// normalised O (fp32) and lse to a workspace, and merge_kernel combines the
// chunks.  Queries and keys may differ in length (a decode step against a
// key/value cache): the queries are then the last positions of the sequence,
// and under the causal mask query row i sees keys 0 .. i + (Nk - Nq).
//
// Dropout (a separate instantiation): the pages fuse it into the kernel and
// keep only the generator state for the backward ("13% more FLOPs, 5.7x
// faster", "The backward pass: recompute instead of read"; explainer Step 3).
// A lane's 16 probabilities of a 32-key block are one Philox4x32-10 call
// (counter: its row, 2 x block + lane half, head, offset), whose ten rounds
// run as extra softmax pieces; dropped probabilities become zero in the P.V
// operand only, so l and lse stay those of the undropped softmax, and the
// epilogue scales O by 256 / (256 - t).
#pragma once

#include <float.h>

#include <type_traits>
#include <utility>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int QB = 1;             // 32-row query blocks per wave
constexpr int NW = 4;             // waves per workgroup
constexpr int BR = 32 * QB * NW;  // query rows per workgroup
constexpr int NT = 64 * NW;       // threads per workgroup
constexpr int OCC = 2;            // workgroups per CU
// keys per K/V tile: 8 KiB tiles
template <typename T, int D> constexpr int bc() { return 8192 / ((int)sizeof(T) * D); }
// LDS buffers for K tiles, and as many for V tiles, within a workgroup's
// share of the 160 KiB (five)
constexpr int RING = (160 * 1024 / OCC) / (2 * 8192);

// The exponent's reference point moves only when a row's maximum rises by
// more than kTau binades, so P <= 2^kTau and most tiles skip the rescale of
// the accumulator.  The bound keeps P representable in the operand type
// (fp16 holds up to 65504 < 2^16) and far below fp32's range for O and l.
// With 8-bit E4M3 probabilities (largest value 448) the reference is set
// kShift binades below the row maximum when it moves and moves once the
// maximum exceeds it by kTau = 8, so every P is at most 2^8 and the row's
// largest P, once its tile is in, at least 2^4: E4M3's normal range then
// covers P down to 2^-10 of the reference.
template <typename T> constexpr float kTau = 32.f;
template <> constexpr float kTau<_Float16> = 15.f;
template <> constexpr float kTau<fp8e4m3> = 8.f;
template <typename T> constexpr float kShift = 0.f;
template <> constexpr float kShift<fp8e4m3> = 4.f;
// 2^kTau (the bound of the 16-bit forward's lane-sum check)
template <typename T> constexpr float kBound = 4294967296.f;
template <> constexpr float kBound<_Float16> = 32768.f;

template <int V> using IC = std::integral_constant<int, V>;

// f(IC<0>), f(IC<1>), ... while f returns true.
template <typename F, int... I>
__device__ __forceinline__ bool for_ring(F& f, std::integer_sequence<int, I...>) {
    return (f(IC<I>{}) && ...);
}

// lds_wait_upto<3 K> for a K in 0..KMAX known only after unrolling.
template <int KMAX> struct WaitSel3 {
    static __device__ __forceinline__ void run(int k, i32x4& a, i32x2& b, i32x2& c) {
        if (k >= KMAX) lds_wait_upto<3 * KMAX>(a, b, c);
        else WaitSel3<KMAX - 1>::run(k, a, b, c);
    }
};
template <> struct WaitSel3<0> {
    static __device__ __forceinline__ void run(int, i32x4& a, i32x2& b, i32x2& c) { lds_wait_upto<0>(a, b, c); }
};
// lds_wait_upto<6 K> likewise (six reads per fragment)
template <int KMAX> struct WaitSel6 {
    static __device__ __forceinline__ void run(int k, i32x4& a, i32x4& b, i32x2& c, i32x2& d, i32x2& e,
                                               i32x2& f) {
        if (k >= KMAX) lds_wait_upto<6 * KMAX>(a, b, c, d, e, f);
        else WaitSel6<KMAX - 1>::run(k, a, b, c, d, e, f);
    }
};
template <> struct WaitSel6<0> {
    static __device__ __forceinline__ void run(int, i32x4& a, i32x4& b, i32x2& c, i32x2& d, i32x2& e,
                                               i32x2& f) {
        lds_wait_upto<0>(a, b, c, d, e, f);
    }
};

// An empty use of a register value: it must be computed at this point of
// the program (the compiler would otherwise sink work past later branches).
template <typename V> __device__ __forceinline__ void materialize(const V& x) {
    __asm__ volatile("" ::"v"(x));
}
// (a 32-byte operand as its two 16-byte halves)
__device__ __forceinline__ void materialize(const i32x8& x) {
    const i32x4 lo = __builtin_shufflevector(x, x, 0, 1, 2, 3);
    const i32x4 hi = __builtin_shufflevector(x, x, 4, 5, 6, 7);
    __asm__ volatile("" ::"v"(lo), "v"(hi));
}

template <typename T, typename TO, int D, bool CAUSAL, bool DROP, bool ONCE>
__global__ __launch_bounds__(NT, OCC) void fwd_kernel(FwdArgs a) {
    typedef typename Elem<T>::v8 v8;
    typedef typename Elem<T>::raw raw;
    constexpr bool F8 = sizeof(T) == 1;   // E4M3 operands (d = 128, no dropout)
    // 16-bit operands: whether the reference must move is read off each lane's
    // fp32 sum of the tile's P, formed with the current reference (see the
    // softmax pieces); 8-bit: from the tile's row maximum, computed first.
    constexpr bool LAZY = !F8;
    // The row normalisers.  O is divided by the sum of P as rounded for the
    // P.V product, so that O's weights sum to one exactly as used: P's
    // rounding (2^-11 relative for fp16, 2^-8 for bf16) would otherwise move
    // a row dominated by one key by that much of its V row, which reaches the
    // output bound (bf16: 2^-8 of a V element of 4 is 1.6e-2).  lse needs the
    // exact sum to 1e-3: fp16 takes the rounded sum for it too (2^-11
    // relative); bf16 keeps a second, fp32 sum of P for lse (OSUM); 8-bit
    // operands use the fp32 sum for both (their error bound accounts for
    // P's rounding, 2^-4 relative).
    constexpr bool RSUM = std::is_same_v<T, _Float16>;
    constexpr bool OSUM = std::is_same_v<T, __bf16>;
    static_assert(!F8 || (D == 128 && !DROP), "the 8-bit forward is instantiated for d = 128 only");
    constexpr int BC = bc<T, D>();
    static_assert(RING >= 4, "the pipeline needs four buffers per tensor");
    static_assert(RING <= 5, "the lead distances and the barrier rule are written for four or five buffers");
    constexpr int KLEAD = RING - 1;   // iteration t starts the copy of K(t + KLEAD) ...
    constexpr int VLEAD = RING - 3;   // ... and of V(t + VLEAD)
    constexpr int ROWB = D * (int)sizeof(T);   // bytes per tile row
    constexpr int LD = ROWB / 2;           // rows are placed as rows of LD 16-bit elements
    constexpr int GR = ROWB / 16;          // 16-byte granules per row
    constexpr int TILE = BC * ROWB;        // bytes of one K (or V) tile
    constexpr int LOADS = TILE / (NT * 16);  // 16-byte loads per thread per tile and tensor
    static_assert(LOADS * NT * 16 == TILE, "a tile splits evenly over the workgroup");
    constexpr int KS = Elem<T>::KSTEP;     // k of one product
    constexpr int KB = BC / 32;            // 32-key blocks per tile
    constexpr int DK = D / KS;             // k-steps of the S product
    constexpr int DB = D / 32;             // 32-wide output column blocks
    constexpr int VK = BC / KS;            // k-steps of the P.V product
    constexpr int NF = KB * DK;            // K fragments per tile (and as many V fragments)
    static_assert(NF == DB * VK, "");
    constexpr int NG = (int)sizeof(raw) / 16;   // 16-byte granules of one operand
    constexpr int NMM = 2 * QB * NF;       // products per iteration

    // K ring (RING tiles), then V ring (RING tiles)
    __shared__ __attribute__((aligned(1024))) char smem[2 * RING * TILE];

    const int N = a.N;                  // query rows per head
    const int Nk = a.Nk;                // keys per head
    const int coff = a.coff;            // causal: row i sees keys 0 .. i + coff
    const int tid = tid_x(), lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
    const int l32 = lane & 31, h = lane >> 5;
    const int s16 = lane & 15, grp = lane >> 4;

    // Work: one query block of one (batch, head).  Under causal masking the
    // blocks differ in length (block b sees b + 1 blocks of keys), so the grid
    // is ordered for the dispatcher, which hands workgroup i to XCD i % 8 and
    // then to whichever of that XCD's slots frees first:
    //  - hgroup > 0 (B*H a multiple of 8): XCD x takes the heads congruent to
    //    x modulo 8, hgroup heads at a time, and each group's blocks heaviest
    //    first; the light blocks of a group then fill the slots the heavy ones
    //    free, only the last group's lightest blocks form the kernel's tail,
    //    and an XCD streams the K/V of about hgroup heads at once (its L2);
    //  - otherwise one workgroup takes the pair of blocks nqb-1-p and p of one
    //    head, one after the other, so that every workgroup streams about as
    //    many tiles as any other.
    // (the divisions by run-time counts are vector code; their results are
    // the same in every lane and are moved to scalar registers, so that they
    // and everything derived from them take no vector registers in the loop)
    const int L = xcd_remap(wg_x(), a.total);
    int bh, qb_first, qb_second = 0, nitems = 1, split = 0;
    if (a.nsplit > 0) {
        // split K/V: one query block and one chunk of its tiles (heaviest
        // causal blocks first); the partial results are merged afterwards
        const int per = a.nqb * a.nsplit;
        bh = L / per;
        const int rem = L - bh * per;
        const int qbi = rem / a.nsplit;
        split = rem - qbi * a.nsplit;
        qb_first = CAUSAL ? a.nqb - 1 - qbi : qbi;
    } else if (CAUSAL && a.hgroup > 0) {
        const int i = wg_x(), x = i & 7, m = i >> 3;   // m-th workgroup of XCD x
        const int per = a.hgroup * a.nqb;                        // workgroups of one group
        const int g = m / per, rem = m - g * per;
        const int r = rem / a.hgroup, u = rem - r * a.hgroup;
        bh = 8 * (g * a.hgroup + u) + x;
        qb_first = a.nqb - 1 - r;
    } else if (CAUSAL) {
        const int npairs = (a.nqb + 1) >> 1;
        bh = L / npairs;
        const int p = L - bh * npairs;
        qb_first = a.nqb - 1 - p;
        qb_second = p;
        nitems = p != a.nqb - 1 - p ? 2 : 1;
    } else {
        bh = L / a.nqb;
        qb_first = L - bh * a.nqb;
    }
    bh = __builtin_amdgcn_readfirstlane(bh);
    qb_first = __builtin_amdgcn_readfirstlane(qb_first);
    qb_second = __builtin_amdgcn_readfirstlane(qb_second);
    nitems = __builtin_amdgcn_readfirstlane(nitems);
    split = __builtin_amdgcn_readfirstlane(split);
    for (int item = 0; item < nitems; ++item) {
        const int qb = item == 0 ? qb_first : qb_second;
        const int q0 = qb * BR;
        const size_t head = (size_t)bh * N * D;        // q and o of this head
        const size_t khead = (size_t)bh * Nk * D;      // k and v of this head
        const T* __restrict__ Qh = (const T*)a.q + head;
        const unsigned head_bytes = (unsigned)Nk * ROWB;
        const char* const kbase = (const char*)((const T*)a.k + khead);
        const char* const vbase = (const char*)((const T*)a.v + khead);

        // This lane's query rows and their Q fragments (B operands of S^T = K Q^T).
        const int qlo = q0 + 32 * QB * w;
        int qrow[QB];
        raw qf[QB][DK];
    #pragma unroll
        for (int r = 0; r < QB; ++r) {
            qrow[r] = qlo + 32 * r + l32;
    #pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                raw x = {};
                if (qrow[r] < N) x = *(const raw*)(Qh + (size_t)qrow[r] * D + KS * kk + (KS / 2) * h);
                if (a.negate) x ^= (int)Elem<T>::kSign;   // scale < 0: use -Q and |scale|
                qf[r][kk] = x;
            }
        }

        const int kend = CAUSAL ? max(0, min(Nk, q0 + BR + coff)) : Nk;
        const int ntiles = (kend + BC - 1) / BC;   // tiles the block's rows can see
        // The tiles of this work item, tb .. te-1: all of the block's, or one
        // chunk of them under split K/V (possibly none); keys from klim on are
        // masked.
        int tb = 0, te = ntiles;
        if (a.nsplit > 0) {
            const int chunk = (ntiles + a.nsplit - 1) / a.nsplit;
            tb = __builtin_amdgcn_readfirstlane(min(ntiles, split * chunk));
            te = __builtin_amdgcn_readfirstlane(min(ntiles, tb + chunk));
        }
        const int klim = min(kend, te * BC);

        // Copy p of this thread fills LDS slot (p*4 + w)*64 + lane of a tile:
        // row `row`, physical granule pg, which holds logical granule
        // pg ^ key(row) of that row (the t_off placement).
        unsigned src_off[LOADS];
    #pragma unroll
        for (int p = 0; p < LOADS; ++p) {
            const int slot = (p * NW + w) * 64 + lane;
            const int row = slot / GR, pg = slot % GR;
            src_off[p] = (unsigned)(row * ROWB + (pg ^ lds_key<LD>(row)) * 16);
        }
        // The copies of tile t go through a buffer descriptor whose base is the
        // tile's first byte and whose size is what is left of the head (none
        // past the end of the streamed range), formed in scalar registers: the
        // per-lane offsets stay fixed, and rows past the end of the sequence or
        // of the range read zeros and cost no memory traffic.
        const unsigned sbase = lds_addr(smem) + w * 1024;
        // ONCE: no other workgroup reads this workgroup's K/V tiles (one query
        // block per (batch, head): a decode step, split or not), so the copies
        // are marked non-temporal.
        auto issue = [&](const char* base, int t, int buf) __attribute__((always_inline)) {
            const bool in = t < te;
            const unsigned off = in ? (unsigned)t * TILE : 0u;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + off, in ? head_bytes - off : 0u);
    #pragma unroll
            for (int p = 0; p < LOADS; ++p) {
                if constexpr (ONCE) dma16_async_once(rs, sbase + buf * TILE + p * NW * 1024, src_off[p]);
                else dma16_async(rs, sbase + buf * TILE + p * NW * 1024, src_off[p]);
            }
        };
        // Loop-invariant LDS addresses of this lane's operand reads (those of V
        // include the V ring's base); the block, half-tile and buffer parts are
        // added as immediates (the swizzle key depends on the row modulo 16 only).
        // (K: row l32 of a 32-key block, the operand's granules of k-step kk)
        int koff[DK][NG];
    #pragma unroll
        for (int kk = 0; kk < DK; ++kk)
    #pragma unroll
            for (int gi = 0; gi < NG; ++gi)
                koff[kk][gi] = t_off<LD>(l32, (KS * kk + (KS / 2) * h) * (int)sizeof(T) / 16 + gi);
        int voff[2][DB];
    #pragma unroll
        for (int cb = 0; cb < DB; ++cb) {
            if constexpr (F8) {
                // 8-bit transposing reads: lane a of 16-lane group g (a % 16 =
                // 2 j + pi) addresses row 8 (j / 4) + 4 (g / 2) + j % 4 of a
                // 16-key group at columns 32 cb + 16 (g % 2) + 8 pi .. +7, so
                // that the lane at column m of the block receives the keys its
                // P operand holds (see product)
                const int jv = s16 >> 1, pv = lane & 1;
                const int rv = 8 * (jv >> 2) + 4 * (grp >> 1) + (jv & 3);
                voff[0][cb] = RING * TILE + t_off<LD>(rv, 2 * cb + (grp & 1)) + 8 * pv;
                voff[1][cb] = voff[0][cb];
            } else {
                const int col = 32 * cb + 16 * (grp & 1) + 4 * (s16 & 3);
                const int r0 = 4 * h + (s16 >> 2);
                voff[0][cb] = RING * TILE + t_off<D>(r0, col >> 3) + (col & 7) * 2;
                voff[1][cb] = RING * TILE + t_off<D>(r0 + 8, col >> 3) + (col & 7) * 2;
            }
        }

        const float c = a.c;   // > 0 (the host maps a zero scale to the smallest normal unit)
        f32x16 oacc[QB][DB];
    #pragma unroll
        for (int r = 0; r < QB; ++r)
    #pragma unroll
            for (int cb = 0; cb < DB; ++cb)
    #pragma unroll
                for (int e = 0; e < 16; ++e) oacc[r][cb][e] = 0.f;
        // per row: exponent reference (scaled units), and this lane's share of
        // the row's normaliser l
        float mc_run[QB], l_run[QB], lo_run[QB];   // lo_run: bf16's rounded sum (divides O)
        // (the reference starts at the lowest finite value: the first tile, whose
        // key 0 every row sees, always moves it, with alpha = 0)
    #pragma unroll
        for (int r = 0; r < QB; ++r) mc_run[r] = -FLT_MAX, l_run[r] = 0.f, lo_run[r] = 0.f;

        typedef f32x16 Scores[QB][KB];   // S^T of one tile, per row block and 32-key block
        typedef v8 Probs[QB][VK];        // P of one tile packed as B operands, per k-step

        // S^T = K Q^T for the tile in K buffer kb_, row blocks accumulated from
        // each K fragment in turn.
        auto s_frag = [&](int kbuf, int i, Scores& sn) __attribute__((always_inline)) {
            const int b = i % KB, kk = i / KB;
            raw kx;
            if constexpr (NG == 1) {
                kx = *(const i32x4*)(smem + kbuf * TILE + koff[kk][0] + 32 * b * ROWB);
            } else {
                const i32x4 lo = *(const i32x4*)(smem + kbuf * TILE + koff[kk][0] + 32 * b * ROWB);
                const i32x4 hi = *(const i32x4*)(smem + kbuf * TILE + koff[kk][1] + 32 * b * ROWB);
                kx = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
    #pragma unroll
            for (int r = 0; r < QB; ++r)
                sn[r][b] = Elem<T>::mma(bit_cast<v8>(kx), bit_cast<v8>(qf[r][kk]), kk == 0 ? f32x16{} : sn[r][b]);
        };
        // Scores of keys a row may not see (causal, past the end of the
        // sequence, or past the workgroup's range) become -inf.
        // Element e of block b holds key j0 + 4h + (32b + 8(e/4) + e%4), which is
        // visible when that key is below klim and (causal) at most the row: one
        // comparison of the constant part against a per-lane limit.
        auto apply_mask = [&](Scores& sc, int j0) __attribute__((always_inline)) {
    #pragma unroll
            for (int r = 0; r < QB; ++r) {
                const int lim = (CAUSAL ? min(klim - 1, qrow[r] + coff) : klim - 1) - j0 - 4 * h;
    #pragma unroll
                for (int b = 0; b < KB; ++b)
    #pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int kc = 32 * b + 8 * (e >> 2) + (e & 3);
                        sc[r][b][e] = kc <= lim ? sc[r][b][e] : -INFINITY;
                    }
            }
        };

        Scores sA, sB;
        Probs pA, pB;
    #pragma unroll
        for (int r = 0; r < QB; ++r)
    #pragma unroll
            for (int jj = 0; jj < VK; ++jj) pA[r][jj] = v8{};

        // An iteration runs in NF steps; step k reads K fragment k and V
        // fragment k and issues 2 QB products: per row block, one of S (for the
        // next tile) and one of P.V (for the previous tile).  Fragments are read
        // DIST steps ahead by inline assembly and waited for explicitly.  The
        // softmax of the current tile is cut into pieces, placed between the
        // products; scheduling fences keep every piece in its slot.
        constexpr int DIST = F8 ? 3 : QB == 1 ? 4 : 3;   // (8-bit: 6 reads per step, lgkmcnt <= 15)
        struct Frag16 {
            i32x4 k;
            i32x2 v0, v1;
        };
        struct Frag8 {
            i32x4 k, k1;
            i32x2 v0, v1, v2, v3;
        };
        typedef std::conditional_t<F8, Frag8, Frag16> Frag;
        const unsigned lbase = lds_addr(smem);
        unsigned kaddr[DK][NG];
    #pragma unroll
        for (int kk = 0; kk < DK; ++kk)
    #pragma unroll
            for (int gi = 0; gi < NG; ++gi) kaddr[kk][gi] = lbase + koff[kk][gi];
        unsigned vaddr[2][DB];
    #pragma unroll
        for (int cb = 0; cb < DB; ++cb) vaddr[0][cb] = lbase + voff[0][cb], vaddr[1][cb] = lbase + voff[1][cb];
        auto load_frag = [&](int kbuf, int vbuf, int k, Frag& f) __attribute__((always_inline)) {
            const int b = k % KB, kk = k / KB;
            f.k = lds_read_b128_asm(kaddr[kk][0], kbuf * TILE + 32 * b * ROWB);
            const int cb = k % DB, jj = k / DB;
            if constexpr (F8) {
                f.k1 = lds_read_b128_asm(kaddr[kk][1], kbuf * TILE + 32 * b * ROWB);
                const int roff = vbuf * TILE + 64 * jj * ROWB;
                f.v0 = lds_read_tr8_asm(vaddr[0][cb], roff);
                f.v1 = lds_read_tr8_asm(vaddr[0][cb], roff + 16 * ROWB);
                f.v2 = lds_read_tr8_asm(vaddr[0][cb], roff + 32 * ROWB);
                f.v3 = lds_read_tr8_asm(vaddr[0][cb], roff + 48 * ROWB);
            } else {
                const int bv = jj >> 1, q = jj & 1;
                const int roff = vbuf * TILE + (32 * bv + 16 * q) * ROWB;
                f.v0 = lds_read_tr16_asm(vaddr[0][cb], roff);
                f.v1 = lds_read_tr16_asm(vaddr[1][cb], roff);
            }
        };
        // product m of step k: row block r = m / 2, S for even m, P.V for odd m.
        // 16-bit: B operand jj = 2b + q of P holds, at k = 8h + e, the
        // probability of key 32b + 16q + 8(e/4) + 4h + e%4; 8-bit: B operand jj
        // holds as its element 16 b' + e (b' = 0, 1) the probability of key
        // 64 jj + 32 b' + 8(e/4) + 4h + e%4.  The transposing reads fetch V at
        // exactly those keys.
        auto product = [&](int k, int m, const Frag& f, Scores& sn, const Probs& pp) __attribute__((always_inline)) {
            const int r = m >> 1;
            if ((m & 1) == 0) {
                const int b = k % KB, kk = k / KB;
                raw kx;
                if constexpr (F8) kx = __builtin_shufflevector(f.k, f.k1, 0, 1, 2, 3, 4, 5, 6, 7);
                else kx = f.k;
                sn[r][b] = Elem<T>::mma(bit_cast<v8>(kx), bit_cast<v8>(qf[r][kk]), kk == 0 ? f32x16{} : sn[r][b]);
            } else {
                const int cb = k % DB, jj = k / DB;
                raw vx;
                if constexpr (F8) {
                    const i32x4 v01 = __builtin_shufflevector(f.v0, f.v1, 0, 1, 2, 3);
                    const i32x4 v23 = __builtin_shufflevector(f.v2, f.v3, 0, 1, 2, 3);
                    vx = __builtin_shufflevector(v01, v23, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {
                    vx = __builtin_shufflevector(f.v0, f.v1, 0, 1, 2, 3);
                }
                oacc[r][cb] = Elem<T>::mma(bit_cast<v8>(vx), pp[r][jj], oacc[r][cb]);
            }
        };

        // Softmax of one tile, as pieces p = 0 .. NP-1 (row block p % QB).
        // 8-bit operands: row maximum over 8 scores (2 KB pieces); the
        // reference and the wave's rescale flags (1); then the probabilities.
        // 16-bit operands: the probabilities only, formed with the reference
        // as it stands.  After the tile's products every lane compares its
        // share of the tile's l with 2^kTau: a lane at or below it has all its
        // P within the bound; a lane above it may hold a P above the bound or
        // an infinite one (the prologue sets the reference from tile 0, so
        // the first tile passes), and then the wave
        // takes the row maximum, moves the reference where that asks for it
        // and forms the tile's probabilities again.  A probability piece
        // forms two probabilities, their packed pair and their share of l
        // (fp32, or fp16 as rounded) (8 KB pieces).  The reference moves when the row maximum
        // rose by more than kTau binades; the factor for the older
        // accumulation, 2^(old - new), is formed only in the rare branch that
        // rescales O and l (also after the first tile, whose move from the
        // lowest finite value gives the factor 0 for an O and l that are
        // still zero).
        // Under dropout, the first 10 KB pieces of a row are the rounds of its
        // generator calls, one per 32-key block (tile j0 / 32 + b).
        constexpr int NPD = DROP ? 10 * KB : 0;
        constexpr int NP_ROW = NPD + (LAZY ? 8 * KB : 10 * KB + 1);
        constexpr int NP = QB * NP_ROW;
        float st_mt[QB], st_mold[QB], st_l[QB], st_lo[QB];
        constexpr int PWD = (int)sizeof(raw) / 4;   // words of one P operand
        unsigned pw[QB][VK][PWD];
        unsigned ph[QB][KB][4];   // generator state, then the call's four words
        int tile_j0 = 0;          // first key of the tile being normalised
        // probabilities q = 0 .. 8 KB - 1 of row block r: elements 2 (q % 8),
        // +1 of 32-key block q / 8, with the reference mc_run[r]
        auto probs = [&](int r, int q, const Scores& sc) __attribute__((always_inline)) {
            const int b = q / 8, e = 2 * (q % 8);
            const float x0 = fast_exp2(fmaf(sc[r][b][e], c, -mc_run[r]));
            const float x1 = fast_exp2(fmaf(sc[r][b][e + 1], c, -mc_run[r]));
            if constexpr (F8) {
                // bytes (16 (b % 2) + e) % 4, +1 of word 4 (b % 2) + e / 4 of P operand
                // b / 2; the row sum is that of the fp32 probabilities
                const int jj = b >> 1, wd = 4 * (b & 1) + (e >> 2);
                const bool hi = (e >> 1) & 1;
                if (q == 0) {
                    st_l[r] = x0 + x1;
                } else {
                    st_l[r] += x0;
                    st_l[r] += x1;
                }
                if (hi) {
                    pw[r][jj][wd] = Elem<T>::cvt2_into(x0, x1, pw[r][jj][wd], true);
                } else {
                    // the low pair is written into x1's own register, whose
                    // upper two bytes the hi call replaces: a zeroed word
                    // would cost a register move per word.  The empty asm
                    // takes the updated sum as input, so the sum reads x1
                    // before the conversion overwrites it and no copy is made
                    unsigned xb = __float_as_uint(x1);
                    __asm__("" : "+v"(xb) : "v"(st_l[r]));
                    pw[r][jj][wd] = Elem<T>::cvt2_into(x0, __uint_as_float(xb), xb, false);
                }
            } else {
                const unsigned pr = Elem<T>::cvt2(x0, x1);
                if constexpr (OSUM) st_lo[r] = Elem<T>::sum2(pr, q == 0 ? 0.f : st_lo[r]);
                if constexpr (RSUM) {
                    st_l[r] = Elem<T>::sum2(pr, q == 0 ? 0.f : st_l[r]);
                } else if (q == 0) {
                    st_l[r] = x0 + x1;
                } else {
                    st_l[r] += x0;
                    st_l[r] += x1;
                }
                if (DROP) {
                    // elements e, e + 1: bytes e % 4 and e % 4 + 1 of word e / 4
                    const unsigned wd = ph[r][b][e >> 2];
                    const bool k0 = drop_keep(wd, e & 3, a.drop.t), k1 = drop_keep(wd, (e & 3) + 1, a.drop.t);
                    pw[r][2 * b + e / 8][(e % 8) / 2] = Elem<T>::cvt2(k0 ? x0 : 0.f, k1 ? x1 : 0.f);
                } else {
                    pw[r][2 * b + e / 8][(e % 8) / 2] = pr;
                }
            }
        };
        // the tile's row maximum (over both lanes of the row), moved reference
        // and rescale flag of row block r
        auto move_ref = [&](int r, const Scores& sc) __attribute__((always_inline)) {
            float m = -INFINITY;
    #pragma unroll
            for (int b = 0; b < KB; ++b)
    #pragma unroll
                for (int e = 0; e < 16; e += 2) m = fmaxf(fmaxf(m, sc[r][b][e]), sc[r][b][e + 1]);
            const float tc = max32(m) * c;
            const bool upd = tc > mc_run[r] + kTau<T>;
            st_mold[r] = mc_run[r];
            float tnew = tc;
            if constexpr (kShift<T> != 0.f) tnew = tc - kShift<T>;
            mc_run[r] = upd ? tnew : mc_run[r];
            return upd;
        };
        auto piece = [&](int p, Scores& sc, uint64_t& upd_mask) __attribute__((always_inline)) {
            const int r = p % QB;
            if (DROP && p / QB < NPD) {
                const int b = (p / QB) / 10, n = (p / QB) % 10;
                if (n == 0) {
                    ph[r][b][0] = (unsigned)qrow[r];
                    ph[r][b][1] = (unsigned)(2 * (tile_j0 / 32 + b) + h);
                    ph[r][b][2] = (unsigned)bh;
                    ph[r][b][3] = a.drop.offset;
                }
                philox_round(ph[r][b], a.drop.seed0, a.drop.seed1, n);
                return;
            }
            const int sx = p / QB - NPD;
            if constexpr (LAZY) {
                probs(r, sx, sc);
            } else if (sx < 2 * KB) {
                // a chain of three-way maxima: 8 instructions per 16 scores
                const int b = sx >> 1, e0 = 8 * (sx & 1);
                const f32x16& x = sc[r][b];
                float m;
                if (sx == 0) {
                    m = fmaxf(fmaxf(x[e0], x[e0 + 1]), x[e0 + 2]);
                    m = fmaxf(fmaxf(m, x[e0 + 3]), x[e0 + 4]);
                    m = fmaxf(fmaxf(m, x[e0 + 5]), x[e0 + 6]);
                    m = fmaxf(m, x[e0 + 7]);
                } else {
                    m = st_mt[r];
    #pragma unroll
                    for (int e = 0; e < 8; e += 2) m = fmaxf(fmaxf(m, x[e0 + e]), x[e0 + e + 1]);
                }
                st_mt[r] = m;
            } else if (sx == 2 * KB) {
                const float tc = max32(st_mt[r]) * c;
                const bool upd = tc > mc_run[r] + kTau<T>;
                st_mold[r] = mc_run[r];
                float tnew = tc;
                if constexpr (kShift<T> != 0.f) tnew = tc - kShift<T>;
                mc_run[r] = upd ? tnew : mc_run[r];
                upd_mask |= __builtin_amdgcn_ballot_w64(upd);
            } else {
                probs(r, sx - 2 * KB - 1, sc);
            }
        };

        // Iteration t (t = 0 .. te-tb; tile numbers below are relative to tb):
        // copies of K(t+KLEAD) and V(t+VLEAD) start, into K buffer
        // (t+KLEAD)%RING and V buffer (t+VLEAD)%RING, which last held
        // K(t+KLEAD-RING) and V(t+VLEAD-RING), read in iteration t-2 at the
        // latest; softmax of tile t (scores in sc, P to pc), S of tile t+1 (to
        // sn, K buffer (t+1)%RING), P.V of tile t-1 (P in pp, V buffer
        // (t-1)%RING; for t = 0 both are zero).  With five buffers (KLEAD = 4,
        // VLEAD = 2) a barrier follows every odd iteration t: before it each
        // wave waits for all its copies but those of iteration t, so that
        // K(t+2), K(t+3), V(t) and V(t+1), which iterations t+1 and t+2 read,
        // are complete and visible; and every buffer those two iterations
        // overwrite was last read in iteration t or earlier.  One more barrier
        // follows iteration 0: iteration 1 refills K buffer 0, last read in the
        // prologue (S of tile 0), and a wave that skips its products (below)
        // would otherwise reach that copy while others still read K(0).  (With four
        // buffers, KLEAD = 3 and VLEAD = 1: a wait for all copies but those of
        // iterations t-1 and t, and a barrier, after every iteration.)  Tile
        // te-tb is all masked and its P is zero.
        constexpr int INFLIGHT = (KLEAD - 2) * 2 * LOADS;   // copies younger than those waited for
        static_assert(KLEAD - 2 == VLEAD, "K and V copies of one iteration are waited for together");
        static_assert(INFLIGHT < 64, "vmcnt is six bits");
        constexpr bool PAIRB = RING >= 5;   // a barrier every second iteration
        constexpr int WAIT_AT_BARRIER = PAIRB ? 2 * LOADS : INFLIGHT;
        auto iter = [&](auto J, int t, Scores& sc, Scores& sn, Probs& pp, Probs& pc) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;   // t modulo the unrolled group (RING or 2 RING)
            const int j0 = (tb + t) * BC;
            tile_j0 = j0;
            const bool need_mask = (j0 + BC > klim) || (CAUSAL && j0 + BC - 1 > qlo + coff);
            uint64_t upd_mask = 0;
            issue(kbase, tb + t + KLEAD, (j + KLEAD) % RING);
            issue(vbase, tb + t + VLEAD, RING + (j + VLEAD) % RING);
            // Under the causal mask the tiles past this wave's last row are
            // masked for all its rows.  Once tile t-1 is (and so t and t+1, and
            // every later tile), the iteration's products and softmax add
            // nothing; nor do they for a wave whose rows all lie past the end
            // of the queries (in a decode step most waves of a block).  They
            // are then skipped, with P = 0 and its sum 0 (the copies and the
            // barrier stay, for the other waves).
            const bool dead = (CAUSAL && j0 - BC > qlo + 32 * QB - 1 + coff) || qlo >= N;
            if (dead) [[unlikely]] {
    #pragma unroll
                for (int r = 0; r < QB; ++r) {
                    st_l[r] = 0.f;
                    st_lo[r] = 0.f;
    #pragma unroll
                    for (int jj = 0; jj < VK; ++jj)
    #pragma unroll
                        for (int wd = 0; wd < PWD; ++wd) pw[r][jj][wd] = 0u;
                }
            } else {
                if (need_mask) [[unlikely]] apply_mask(sc, j0);
                {
                    constexpr int kbuf = (j + 1) % RING, vbuf = (j + RING - 1) % RING;
                    constexpr int NS = 2 * QB;   // products per step
                    Frag f[DIST + 1];
    #pragma unroll
                    for (int k = 0; k < DIST; ++k) load_frag(kbuf, vbuf, k, f[k]);
    #pragma unroll
                    for (int k = 0; k < NF; ++k) {
                        Frag& cur = f[k % (DIST + 1)];
                        const int later = min(DIST - 1, NF - 1 - k);   // steps read after this one
                        if constexpr (F8) WaitSel6<DIST - 1>::run(later, cur.k, cur.k1, cur.v0, cur.v1, cur.v2, cur.v3);
                        else WaitSel3<DIST - 1>::run(later, cur.k, cur.v0, cur.v1);
                        __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                        for (int m = 0; m < NS; ++m) {
                            const int slot = k * NS + m;
                            product(k, m, cur, sn, pp);
                            if (m == 0 && k + DIST < NF) load_frag(kbuf, vbuf, k + DIST, f[(k + DIST) % (DIST + 1)]);
    #pragma unroll
                            for (int p = slot * NP / NMM; p < (slot + 1) * NP / NMM; ++p) piece(p, sc, upd_mask);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            }
            if constexpr (LAZY) {
                // a lane whose sum of P is at most 2^kTau has every P within the
                // bound; otherwise (a P above it or infinite) the wave moves the
                // reference where the row maximum asks for it and forms the
                // tile's probabilities again
                bool over = false;
    #pragma unroll
                for (int r = 0; r < QB; ++r) over |= st_l[r] > kBound<T>;
                upd_mask = __builtin_amdgcn_ballot_w64(over);
            }
            if (upd_mask != 0) [[unlikely]] {
    #pragma unroll
                for (int r = 0; r < QB; ++r) {
                    if constexpr (LAZY) {
                        move_ref(r, sc);
    #pragma unroll
                        for (int q = 0; q < 8 * KB; ++q) probs(r, q, sc);
                    }
                    const float alpha = fast_exp2(st_mold[r] - mc_run[r]);   // 1 for a row that stays
    #pragma unroll
                    for (int cb = 0; cb < DB; ++cb)
    #pragma unroll
                        for (int e = 0; e < 16; ++e) oacc[r][cb][e] *= alpha;
                    l_run[r] *= alpha;
                    lo_run[r] *= alpha;
                }
            }
    #pragma unroll
            for (int r = 0; r < QB; ++r) {
    #pragma unroll
                for (int jj = 0; jj < VK; ++jj) {
                    raw x;
    #pragma unroll
                    for (int wd = 0; wd < PWD; ++wd) x[wd] = (int)pw[r][jj][wd];
                    pc[r][jj] = bit_cast<v8>(x);
                    materialize(pc[r][jj]);
                }
            }
    #pragma unroll
            for (int r = 0; r < QB; ++r) {
                l_run[r] += st_l[r];
                if constexpr (OSUM) lo_run[r] += st_lo[r];
            }
            if (!PAIRB || j % 2 == 1) {
                wait_vmem_upto<WAIT_AT_BARRIER>();
                barrier_only();
            } else if (t == 0) {
                // iteration 1 refills K buffer 0, whose K(0) every wave reads
                // in the prologue: all waves must be past that first
                barrier_only();
            }
        };

        // Prologue: copies of K(0), K(1), then K(t+KLEAD) and V(t+VLEAD) in the
        // order iterations t = -VLEAD .. -1 would start them; V buffer RING-1
        // (read as "tile -1" with P = 0) cleared so that it holds finite values;
        // S of tile 0.
        issue(kbase, tb, 0);
        issue(kbase, tb + 1, 1);
    #pragma unroll
        for (int t = -VLEAD; t < 0; ++t) {
            issue(kbase, tb + t + KLEAD, t + KLEAD);
            issue(vbase, tb + t + VLEAD, RING + t + VLEAD);
        }
    #pragma unroll
        for (int p = 0; p < LOADS; ++p)
            *(i32x4*)(smem + (2 * RING - 1) * TILE + (p * NW + w) * 1024 + 16 * lane) = i32x4{0, 0, 0, 0};
        wait_vmem_upto<WAIT_AT_BARRIER>();   // Q and all but the copies of "iteration -1"
        __syncthreads();
    #pragma unroll
        for (int i = 0; i < NF; ++i) s_frag(0, i, sA);
        if constexpr (LAZY) {
            // the reference from tile 0's (masked) row maximum, so that its P
            // already stay within the bound and the first iteration needs no
            // second pass (iteration 0 masks the tile again, to the same values)
            const int j00 = tb * BC;
            if ((j00 + BC > klim) || (CAUSAL && j00 + BC - 1 > qlo + coff)) apply_mask(sA, j00);
    #pragma unroll
            for (int r = 0; r < QB; ++r) move_ref(r, sA);
        }

        // iterations in groups of RING, or 2 RING for an odd RING (buffer
        // indices and the barrier parity are constants); scores and
        // probabilities alternate between the A and B sets
        int t = 0;
        auto one = [&](auto J) __attribute__((always_inline)) {
            if constexpr (decltype(J)::value % 2 == 0) iter(J, t, sA, sB, pA, pB);
            else iter(J, t, sB, sA, pB, pA);
            return ++t <= te - tb;
        };
        while (for_ring(one, std::make_integer_sequence<int, RING % 2 ? 2 * RING : RING>{})) {
        }
        // no copy may still be writing LDS, and no wave still reads the rings:
        // the epilogue reuses their space
        wait_vmem();
        __syncthreads();

        // epilogue: O = O^T / l, one rounding; lse = (mc + log2 l) ln 2
    #pragma unroll
        for (int r = 0; r < QB; ++r) {
            // (8-bit: O is also scaled by V's descale)
            const float l_tot = sum32(l_run[r]);
            const float lo_tot = OSUM ? sum32(lo_run[r]) : l_tot;   // divides O
            // a row that sees no key of its chunk (split K/V only) gets O = 0 and
            // lse = -inf, which weigh nothing in the merge
            float inv = l_tot > 0.f ? fast_rcp(lo_tot) * (DROP ? a.drop.scale : 1.f) : 0.f;
            if constexpr (F8) inv *= a.oscale;
            // (the row index passes through an empty asm statement so that
            // its 64-bit offset is formed here, not kept live through the loop)
            int qr = qrow[r];
            __asm__ volatile("" : "+v"(qr));
            // O leaves through LDS as whole rows (a direct store from the
            // accumulators would write 64 rows x 8 bytes per instruction),
            // staged in this wave's own region of the idle rings
            store_rows_staged<TO, D>(smem + w * (32 * D * (int)sizeof(TO)),
                                     (TO*)a.o + (size_t)split * a.split_o + head + (size_t)(qlo + 32 * r) * D,
                                     N - (qlo + 32 * r), oacc[r], inv, lane);
            if (qr < N) {
                if (h == 0)
                    a.lse[(size_t)split * a.split_lse + (size_t)bh * N + qr] =
                        l_tot > 0.f ? (mc_run[r] + fast_log2(l_tot)) * 0.69314718055994531f : -INFINITY;
            }
        }
        // the next item reuses the LDS buffers (this wave's copies have
        // drained; the barrier waits for every other wave's reads)
        if (item + 1 < nitems) __syncthreads();
    }
}

// Merge of split K/V partials, one thread per 4 columns of a row: the
// pages' rescale rule for combining two partial softmaxes ("FlashAttention's
// move: rescale the output, too"; explainer "Common questions" on
// Flash-Decoding) in logsumexp form, over all chunks at once:
//   lse = log sum_s e^(lse_s),  O = sum_s e^(lse_s - lse) O_s,
// with each O_s already normalised by its own chunk's sum.  A chunk whose
// row saw no key has lse_s = -inf and weight 0.

}  // namespace
}  // namespace attn
