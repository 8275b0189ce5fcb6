// attn_launch.h -- internal interface between the C ABI (attn_api.cpp) and
// the kernel translation units.  Arguments reaching these functions have
// already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Dropout on the probabilities (inactive when `on` is 0): an element is kept
// when byte (j mod 4) of word ((j mod 32) / 8) of Philox4x32-10 with key
// (seed0, seed1) and counter (i, 2 (j / 32) + (j / 4) mod 2, bh, offset) is at
// least t; kept weights are scaled by `scale` = 256 / (256 - t).
struct DropArgs {
    int on;
    unsigned t;
    float scale;
    unsigned seed0, seed1, offset;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int N;        // query rows per (batch, head)
    int Nk;       // keys per (batch, head) (N for self-attention)
    int coff;     // causal offset Nk - N: query row i sees keys 0 .. i + coff
    int nqb;      // query blocks per (batch, head)
    int total;    // workgroups: B * H * nqb, or B * H * ceil(nqb / 2) under causal masking
    float c;      // |scale| * log2(e): exponent units of the kernel
    int negate;   // scale < 0: the kernel multiplies Q by -1 (exact)
    int nsplit;   // 0: whole query blocks; > 0: each block's K/V tiles in nsplit chunks,
                  // partial results (fp32 O, lse) to o / lse at chunk strides below
    size_t split_o;    // elements between the partial outputs of consecutive chunks
    size_t split_lse;  // elements between their partial lse
    DropArgs drop;
    float oscale;      // 8-bit inputs only: factor applied to O (V's descale)
    int hgroup;        // causal whole blocks, B*H a multiple of 8: heads per group in
                       // each XCD's heaviest-first order (total = B*H*nqb); 0: pairs
};

// Causal grids with B*H a multiple of 8 (0 otherwise): one workgroup per
// query block, and XCD x takes the heads congruent to x modulo 8 in groups of
// this many (the largest of 4, 3, 2, 1 that divides its B*H/8 heads), each
// group's blocks heaviest first.  The forward and the dq kernel use it.
inline int xcd_head_group(int64_t BH, int causal) {
    if (!causal || BH % 8 != 0) return 0;
    int hg = 4;
    while ((BH / 8) % hg != 0) --hg;
    return hg;
}

int fwd_block_rows();
hipError_t launch_fwd(const FwdArgs& a, int dtype, bool out_f32, int d, int causal, hipStream_t stream);
// 8-bit E4M3 q, k, v (d = 128, whole query blocks, no dropout); out_dtype:
// 0 fp16, 1 bf16, 2 fp32
hipError_t launch_fwd_fp8(const FwdArgs& a, int out_dtype, int causal, hipStream_t stream);
// The same launches for a grid with one query block per (batch, head) and no
// dropout (a.nqb == 1, !a.drop.on): no two workgroups read the same K/V tile,
// and the copies are marked non-temporal.  Same outputs bit for bit.
hipError_t launch_fwd_once(const FwdArgs& a, int dtype, bool out_f32, int d, int causal, hipStream_t stream);
hipError_t launch_fwd_fp8_once(const FwdArgs& a, int out_dtype, int causal, hipStream_t stream);

// Split K/V: workspace bytes for nsplit chunks (fp32 partial O and lse), and
// the merge of the partials into o (dtype, or fp32) and lse.
size_t fwd_split_workspace_bytes(int64_t BH, int64_t N, int64_t d, int nsplit);
hipError_t launch_fwd_merge(const float* ws_o, const float* ws_lse, void* o, float* lse, int64_t rows,
                            int nsplit, size_t split_o, size_t split_lse, int d, int dtype, bool out_f32,
                            hipStream_t stream);

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* ws;      // workspace: per head, D_i = dO_i . o_i then lse_i log2(e),
                    // each padded to NP = round_up(N, 64) floats: [2][B*H][NP]
    int N;
    int BH;
    float c;        // scale * log2(e) with its sign (magnitude at least FLT_MIN)
    float scale;    // the caller's scale (gradient factor)
    int negate;     // unused by the backward kernels
    DropArgs drop;  // the forward's dropout, regenerated here
};

size_t bwd_workspace_bytes(int64_t BH, int64_t N);
// The fixed per-GPU workspace of attn_bwd_noalloc: its size, and its device
// address on the current device (looked up on the first call per device).
constexpr size_t kBwdScratchBytes = size_t(16) << 20;
hipError_t bwd_scratch(void** ptr);
// which: 1 = dq kernel only, 2 = dk/dv kernel only, 3 = both in order
hipError_t launch_bwd(const BwdArgs& a, int which, int dtype, bool out_f32, int d, int causal,
                      hipStream_t stream);

// Materialised standard attention: S = scale Q K^T (fp32, [BH][N][N]),
// P = softmax(S) (dtype, masked entries 0) with lse, O = P V.
hipError_t launch_std_scores(const void* q, const void* k, float* s, int64_t BH, int N, int d,
                             float scale, int dtype, hipStream_t stream);
hipError_t launch_std_softmax(const float* s, void* p, float* lse, int64_t BH, int N, int causal,
                              int dtype, hipStream_t stream);
hipError_t launch_std_pv(const void* p, const void* v, void* o, int64_t BH, int N, int d, int dtype,
                         bool out_f32, hipStream_t stream);

// The matrix-core rate probe: `workgroups` workgroups of 256 threads, each
// wave running 16 x rounds bf16 32x32x16 products; out gets one float per thread.
hipError_t launch_mfma_probe(float* out, int workgroups, int rounds, hipStream_t stream);
hipError_t launch_hbm_probe(const void* buf, long long n16, unsigned* out, int workgroups, hipStream_t stream);

}  // namespace attn
