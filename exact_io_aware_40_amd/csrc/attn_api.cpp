// attn_api.cpp -- the C ABI declared in include/attn.h: argument
// validation, launch configuration and dispatch to the kernel instances.
// Validation runs before any HIP call, so every error path is reachable
// (and testable) without a GPU.
#include "attn.h"

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "attn_launch.h"

namespace {

constexpr int64_t kMaxHeadElems = int64_t(1) << 30;  // N * d per head
constexpr float kLog2e = 1.4426950408889634f;

// Exponent units of the kernels: |scale| log2(e), raised to the smallest
// normal float when it is smaller (a zero scale in particular).  For any
// finite score s, s * FLT_MIN rounds 2^(s c - m c) to exactly 1, so the
// weights of a zero scale come out uniform as they should, while a masked
// score (-inf) still gives -inf * c = -inf and weight 0.
float exponent_unit(float scale) { return fmaxf(fabsf(scale) * kLog2e, FLT_MIN); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range(const void* p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

// A grid with one query block per (batch, head) and no dropout reads every
// K/V tile in one workgroup only: those launches take the instantiation
// whose copies are marked non-temporal (same outputs).
hipError_t launch_forward(const attn::FwdArgs& a, int dtype, bool out_f32, int d, int causal, hipStream_t s) {
    return a.nqb == 1 && !a.drop.on ? attn::launch_fwd_once(a, dtype, out_f32, d, causal, s)
                                    : attn::launch_fwd(a, dtype, out_f32, d, causal, s);
}
hipError_t launch_forward_fp8(const attn::FwdArgs& a, int out_dtype, int causal, hipStream_t s) {
    return a.nqb == 1 ? attn::launch_fwd_fp8_once(a, out_dtype, causal, s)
                      : attn::launch_fwd_fp8(a, out_dtype, causal, s);
}

// Common checks of sizes, flags and scale.  Returns ATTN_OK or an error;
// sets *empty when there is nothing to compute.
int check_common(int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
                 int out_dtype, bool* empty) {
    *empty = false;
    if (B < 0 || H < 0 || N < 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (out_dtype != dtype && out_dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (B == 0 || H == 0 || N == 0) {
        *empty = true;
        return ATTN_OK;
    }
    if (N * d >= kMaxHeadElems) return ATTN_ERR_SHAPE;
    // total elements must index with 64-bit offsets and the grid must fit
    if (B > (int64_t(1) << 31) / H) return ATTN_ERR_SHAPE;
    const int64_t BH = B * H;
    if (BH > (int64_t(1) << 62) / (N * d)) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: B, H or N out of range";
        case ATTN_ERR_HEAD_DIM: return "ATTN_ERR_HEAD_DIM: d must be 64 or 128";
        case ATTN_ERR_DTYPE:
            return "ATTN_ERR_DTYPE: dtype must be ATTN_F16 or ATTN_BF16, out_dtype dtype or ATTN_F32";
        case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN: pointers must be 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing or too small";
        case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH: kernel launch failed";
        case ATTN_ERR_SCALE: return "ATTN_ERR_SCALE: scale must be finite (descale factors finite and > 0)";
        case ATTN_ERR_CAUSAL: return "ATTN_ERR_CAUSAL: causal must be 0 or 1";
        case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS: an output overlaps an input or another output";
        case ATTN_ERR_SPLIT: return "ATTN_ERR_SPLIT: nsplit must be in 1 .. ATTN_MAX_SPLIT";
        case ATTN_ERR_DROPOUT:
            return "ATTN_ERR_DROPOUT: dropout_p must be finite, >= 0 and round(256 dropout_p) <= 255";
        default: return "unknown attn status";
    }
}

}  // extern "C"

namespace {

// Dropout state from the caller's probability and generator state; ATTN_OK
// or ATTN_ERR_DROPOUT.  t = floor(256 p + 1/2) must be at most 255.
int drop_args(double p, uint64_t seed, uint32_t offset, attn::DropArgs* dr) {
    if (!isfinite(p) || p < 0.0) return ATTN_ERR_DROPOUT;
    const double t = floor(256.0 * p + 0.5);
    if (t > 255.0) return ATTN_ERR_DROPOUT;
    dr->on = 1;
    dr->t = unsigned(t);
    dr->scale = float(256.0 / (256.0 - t));
    dr->seed0 = uint32_t(seed);
    dr->seed1 = uint32_t(seed >> 32);
    dr->offset = offset;
    return ATTN_OK;
}

attn::DropArgs no_drop() {
    attn::DropArgs dr;
    dr.on = 0;
    dr.t = 0;
    dr.scale = 1.f;
    dr.seed0 = dr.seed1 = dr.offset = 0;
    return dr;
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
               int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, int out_dtype,
               const attn::DropArgs& drop, void* stream) {
    bool empty = false;
    int st = check_common(B, H, N, d, scale, causal, dtype, out_dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const size_t tbytes = size_t(BH * N * d) * 2;
    const size_t obytes = size_t(BH * N * d) * (out_dtype == ATTN_F32 ? 4 : 2);
    const Range ro = range(o, obytes), rl = range(lse, size_t(BH * N) * 4);
    const Range in[3] = {range(q, tbytes), range(k, tbytes), range(v, tbytes)};
    for (const Range& r : in)
        if (overlap(ro, r) || overlap(rl, r)) return ATTN_ERR_ALIAS;
    if (overlap(ro, rl)) return ATTN_ERR_ALIAS;

    attn::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.N = int(N);
    a.Nk = int(N);
    a.coff = 0;
    const int br = attn::fwd_block_rows();
    a.nqb = int((N + br - 1) / br);
    // causal: when B*H is a multiple of 8, one workgroup per query block in
    // each XCD's heaviest-first order over groups of heads; otherwise one per
    // pair of query blocks (a heavy and a light one)
    a.hgroup = attn::xcd_head_group(BH, causal);
    const int64_t total = a.hgroup ? BH * a.nqb : BH * (causal ? (a.nqb + 1) / 2 : a.nqb);
    if (total > 0x7fffffff) return ATTN_ERR_SHAPE;
    a.total = int(total);
    a.c = exponent_unit(scale);
    a.negate = scale < 0.f;
    a.nsplit = 0;
    a.split_o = 0;
    a.split_lse = 0;
    a.drop = drop;
    a.oscale = 1.f;
    hipError_t e = launch_forward(a, dtype, out_dtype == ATTN_F32, int(d), causal, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
             int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, int out_dtype,
             void* stream) {
    return fwd_common(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, out_dtype, no_drop(), stream);
}

int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t N, int64_t d, float scale, int causal, float dropout_p,
                     uint64_t seed, uint32_t offset, int dtype, int out_dtype, void* stream) {
    attn::DropArgs dr;
    const int st = drop_args(dropout_p, seed, offset, &dr);
    if (st != ATTN_OK) return st;
    return fwd_common(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, out_dtype, dr, stream);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                 int64_t H, int64_t N, int64_t d, float scale, float q_descale, float k_descale,
                 float v_descale, int causal, int out_dtype, void* stream) {
    if (B < 0 || H < 0 || N < 0) return ATTN_ERR_SHAPE;
    if (d != 128) return ATTN_ERR_HEAD_DIM;
    if (out_dtype != ATTN_F16 && out_dtype != ATTN_BF16 && out_dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
    const float qk = scale * q_descale * k_descale;   // the scores' scale
    if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale) ||
        !(q_descale > 0.f) || !(k_descale > 0.f) || !(v_descale > 0.f) || !isfinite(qk))
        return ATTN_ERR_SCALE;
    bool empty = false;
    const int st = check_common(B, H, N, d, qk, causal, ATTN_BF16, ATTN_BF16, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const size_t tbytes = size_t(BH * N * d);
    const size_t obytes = size_t(BH * N * d) * (out_dtype == ATTN_F32 ? 4 : 2);
    const Range ro = range(o, obytes), rl = range(lse, size_t(BH * N) * 4);
    const Range in[3] = {range(q, tbytes), range(k, tbytes), range(v, tbytes)};
    for (const Range& r : in)
        if (overlap(ro, r) || overlap(rl, r)) return ATTN_ERR_ALIAS;
    if (overlap(ro, rl)) return ATTN_ERR_ALIAS;

    attn::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.N = int(N);
    a.Nk = int(N);
    a.coff = 0;
    const int br = attn::fwd_block_rows();
    a.nqb = int((N + br - 1) / br);
    a.hgroup = 0;
    const int64_t total = BH * (causal ? (a.nqb + 1) / 2 : a.nqb);
    if (total > 0x7fffffff) return ATTN_ERR_SHAPE;
    a.total = int(total);
    a.c = exponent_unit(qk);
    a.negate = qk < 0.f;
    a.nsplit = 0;
    a.split_o = 0;
    a.split_lse = 0;
    a.drop = no_drop();
    a.oscale = v_descale;
    hipError_t e = launch_forward_fp8(a, out_dtype, causal, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_fwd_split_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int nsplit) {
    bool empty = false;
    if (check_common(B, H, N, d, 1.0f, 0, ATTN_BF16, ATTN_BF16, &empty) != ATTN_OK || empty) return 0;
    if (nsplit < 1 || nsplit > ATTN_MAX_SPLIT) return 0;
    return attn::fwd_split_workspace_bytes(B * H, N, d, nsplit);
}

}  // extern "C"

namespace {

// Split K/V forward of Nq query rows against Nk keys per head (Nq = Nk for
// attn_fwd_split): partials into the workspace, then the merge.
// Descale factors of 8-bit inputs (q, k, v); `on` false for 16-bit inputs.
struct Fp8Args {
    bool on;
    float qd, kd, vd;
};

int fwd_split_common(const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                     int64_t Nk, int64_t d, float scale, int causal, int dtype, int out_dtype,
                     int nsplit, void* stream, Fp8Args f8 = Fp8Args{false, 1.f, 1.f, 1.f}) {
    if (Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
    if (f8.on) {
        // 8-bit inputs: d = 128; the output type alone selects the merge's output
        if (B < 0 || H < 0) return ATTN_ERR_SHAPE;
        if (d != 128) return ATTN_ERR_HEAD_DIM;
        if (out_dtype != ATTN_F16 && out_dtype != ATTN_BF16 && out_dtype != ATTN_F32)
            return ATTN_ERR_DTYPE;
        if (!isfinite(scale) || !isfinite(f8.qd) || !isfinite(f8.kd) || !isfinite(f8.vd) ||
            !(f8.qd > 0.f) || !(f8.kd > 0.f) || !(f8.vd > 0.f) || !isfinite(scale * f8.qd * f8.kd))
            return ATTN_ERR_SCALE;
        scale = scale * f8.qd * f8.kd;
        dtype = out_dtype == ATTN_F32 ? ATTN_BF16 : out_dtype;
    }
    bool empty = false;
    int st = check_common(B, H, Nq > Nk ? Nq : Nk, d, scale, causal, dtype, out_dtype, &empty);
    if (st != ATTN_OK) return st;
    if (nsplit < 1 || nsplit > ATTN_MAX_SPLIT) return ATTN_ERR_SPLIT;
    if (empty || Nq == 0) return ATTN_OK;
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const size_t need = attn::fwd_split_workspace_bytes(BH, Nq, d, nsplit);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    const size_t esz = f8.on ? 1 : 2;   // bytes per input element
    const size_t qbytes = size_t(BH * Nq * d) * esz, kbytes = size_t(BH * Nk * d) * esz;
    const size_t obytes = size_t(BH * Nq * d) * (out_dtype == ATTN_F32 ? 4 : 2);
    const Range ro = range(o, obytes), rl = range(lse, size_t(BH * Nq) * 4), rw = range(workspace, need);
    const Range in[3] = {range(q, qbytes), range(k, kbytes), range(v, kbytes)};
    for (const Range& r : in)
        if (overlap(ro, r) || overlap(rl, r) || overlap(rw, r)) return ATTN_ERR_ALIAS;
    if (overlap(ro, rl) || overlap(ro, rw) || overlap(rl, rw)) return ATTN_ERR_ALIAS;

    attn::FwdArgs a;
    const size_t split_o = size_t(BH * Nq * d), split_lse = size_t(BH * Nq);
    float* ws_o = static_cast<float*>(workspace);
    float* ws_lse = ws_o + size_t(nsplit) * split_o;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = ws_o;
    a.lse = ws_lse;
    a.N = int(Nq);
    a.Nk = int(Nk);
    a.coff = int(Nk - Nq);
    const int br = attn::fwd_block_rows();
    a.nqb = int((Nq + br - 1) / br);
    const int64_t total = BH * a.nqb * nsplit;
    if (total > 0x7fffffff) return ATTN_ERR_SHAPE;
    a.total = int(total);
    a.c = exponent_unit(scale);
    a.negate = scale < 0.f;
    a.nsplit = nsplit;
    a.hgroup = 0;
    a.split_o = split_o;
    a.split_lse = split_lse;
    a.drop = no_drop();
    a.oscale = f8.on ? f8.vd : 1.f;
    // the partials are fp32 whatever the output type; the merge rounds once
    hipError_t e = f8.on ? launch_forward_fp8(a, ATTN_F32, causal, (hipStream_t)stream)
                         : launch_forward(a, dtype, true, int(d), causal, (hipStream_t)stream);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
    e = attn::launch_fwd_merge(ws_o, ws_lse, o, lse, BH * Nq, nsplit, split_o, split_lse, int(d), dtype,
                               out_dtype == ATTN_F32, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                   size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                   int causal, int dtype, int out_dtype, int nsplit, void* stream) {
    return fwd_split_common(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, N, d, scale, causal,
                            dtype, out_dtype, nsplit, stream);
}

int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                    float scale, int causal, int dtype, int out_dtype, int nsplit, void* stream) {
    return fwd_split_common(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale,
                            causal, dtype, out_dtype, nsplit, stream);
}

int attn_fwd_decode_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                        int64_t Nk, int64_t d, float scale, float q_descale, float k_descale,
                        float v_descale, int causal, int out_dtype, int nsplit, void* stream) {
    return fwd_split_common(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale, causal,
                            ATTN_BF16, out_dtype, nsplit, stream,
                            Fp8Args{true, q_descale, k_descale, v_descale});
}

size_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    bool empty = false;
    if (check_common(B, H, N, d, 1.0f, 0, dtype, dtype, &empty) != ATTN_OK || empty) return 0;
    return attn::bwd_workspace_bytes(B * H, N);
}

}  // extern "C"

namespace {

// Shared by attn_bwd (which = 3), attn_bwd_dq (1) and attn_bwd_dkdv (2).
// check_only: validate everything but the workspace and return (nothing is
// launched); *empty is then set when there is nothing to compute.
int bwd_common(int which, const void* q, const void* k, const void* v, const void* o,
               const void* dO, const float* lse, void* dq, void* dk, void* dv, const void* ws,
               size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
               int causal, int dtype, int out_dtype, const attn::DropArgs& drop, void* stream,
               bool check_only = false, bool* empty_out = nullptr) {
    bool empty = false;
    int st = check_common(B, H, N, d, scale, causal, dtype, out_dtype, &empty);
    if (empty_out) *empty_out = empty;
    if (st != ATTN_OK || empty) return st;
    const bool want_dq = which & 1, want_dkdv = which & 2;
    if (!q || !k || !v || !dO) return ATTN_ERR_NULL;
    if (want_dq && (!o || !lse || !dq)) return ATTN_ERR_NULL;
    if (want_dkdv && (!dk || !dv)) return ATTN_ERR_NULL;
    const void* ptrs[] = {q, k, v, dO, want_dq ? o : q, want_dq ? (const void*)lse : q,
                          want_dq ? dq : q, want_dkdv ? dk : q, want_dkdv ? dv : q};
    for (const void* p : ptrs)
        if (!aligned16(p)) return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const size_t need = attn::bwd_workspace_bytes(BH, N);
    if (check_only) {
        if (need > attn::kBwdScratchBytes) return ATTN_ERR_WORKSPACE;
    } else {
        if (!ws || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
        if (!aligned16(ws)) return ATTN_ERR_ALIGN;
    }
    if (BH > 0x7fffffff / ((N + 63) / 64)) return ATTN_ERR_SHAPE;

    // outputs may overlap neither the inputs nor each other
    const size_t tbytes = size_t(BH * N * d) * 2;
    const size_t obytes = size_t(BH * N * d) * (out_dtype == ATTN_F32 ? 4 : 2);
    Range outs[4];
    int no = 0;
    Range ins[7];
    int ni = 0;
    ins[ni++] = range(q, tbytes);
    ins[ni++] = range(k, tbytes);
    ins[ni++] = range(v, tbytes);
    ins[ni++] = range(dO, tbytes);
    if (want_dq) {
        ins[ni++] = range(o, obytes);
        ins[ni++] = range(lse, size_t(BH * N) * 4);
        outs[no++] = range(dq, obytes);
        if (!check_only) outs[no++] = range(ws, need);   // written by the dq half
    } else if (!check_only) {
        ins[ni++] = range(ws, need);                     // read by the dk/dv half
    }
    if (want_dkdv) {
        outs[no++] = range(dk, obytes);
        outs[no++] = range(dv, obytes);
    }
    for (int i = 0; i < no; ++i) {
        for (int r = 0; r < ni; ++r)
            if (overlap(outs[i], ins[r])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
    }
    if (check_only) return ATTN_OK;

    attn::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dO = dO;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.ws = static_cast<float*>(const_cast<void*>(ws));
    a.N = int(N);
    a.BH = int(BH);
    // the backward tracks no maximum, so it takes the exponent unit with the
    // scale's sign and uses q and k as they are
    a.c = scale < 0.f ? -exponent_unit(scale) : exponent_unit(scale);
    a.scale = scale;
    a.negate = scale < 0.f;
    a.drop = drop;
    hipError_t e = attn::launch_bwd(a, which, dtype, out_dtype == ATTN_F32, int(d), causal,
                                    (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
             int causal, int dtype, int out_dtype, void* stream) {
    return bwd_common(3, q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                      scale, causal, dtype, out_dtype, no_drop(), stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                     int64_t N, int64_t d, float scale, int causal, int dtype, int out_dtype,
                     void* stream) {
    // every argument is checked (and the workspace's size against the fixed
    // per-GPU scratch) before the first HIP call
    bool empty = false;
    int st = bwd_common(3, q, k, v, o, dO, lse, dq, dk, dv, nullptr, 0, B, H, N, d, scale, causal,
                        dtype, out_dtype, no_drop(), stream, true, &empty);
    if (st != ATTN_OK || empty) return st;
    void* ws = nullptr;
    if (attn::bwd_scratch(&ws) != hipSuccess) return ATTN_ERR_LAUNCH;
    return bwd_common(3, q, k, v, o, dO, lse, dq, dk, dv, ws, attn::kBwdScratchBytes, B, H, N, d,
                      scale, causal, dtype, out_dtype, no_drop(), stream);
}

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     int causal, float dropout_p, uint64_t seed, uint32_t offset, int dtype,
                     int out_dtype, void* stream) {
    attn::DropArgs dr;
    const int st = drop_args(dropout_p, seed, offset, &dr);
    if (st != ATTN_OK) return st;
    return bwd_common(3, q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                      scale, causal, dtype, out_dtype, dr, stream);
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* workspace, size_t workspace_bytes, int64_t B,
                int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
                int out_dtype, void* stream) {
    return bwd_common(1, q, k, v, o, dO, lse, dq, nullptr, nullptr, workspace, workspace_bytes, B,
                      H, N, d, scale, causal, dtype, out_dtype, no_drop(), stream);
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, void* dk,
                  void* dv, const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                  int64_t N, int64_t d, float scale, int causal, int dtype, int out_dtype,
                  void* stream) {
    return bwd_common(2, q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, workspace,
                      workspace_bytes, B, H, N, d, scale, causal, dtype, out_dtype, no_drop(), stream);
}

}  // extern "C"

namespace {

// Shapes the standard (materialised) passes accept: the common checks, N at
// most ATTN_STD_MAX_N, B * H * N * N elements addressable, and every grid
// within 2^31 - 1 workgroups.
int std_check(int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
              int out_dtype, bool* empty) {
    const int st = check_common(B, H, N, d, scale, causal, dtype, out_dtype, empty);
    if (st != ATTN_OK || *empty) return st;
    if (N > ATTN_STD_MAX_N) return ATTN_ERR_SHAPE;
    const int64_t BH = B * H;
    if (BH > (int64_t(1) << 62) / (N * N)) return ATTN_ERR_SHAPE;
    const int64_t nb = (N + 127) / 128;
    if (BH * nb * nb > 0x7fffffff || (BH * N + 3) / 4 > 0x7fffffff) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

size_t std_s_bytes(int64_t BH, int64_t N) { return (size_t(BH * N * N) * 4 + 255) & ~size_t(255); }

int std_scores(const void* q, const void* k, float* s, int64_t B, int64_t H, int64_t N, int64_t d,
               float scale, int dtype, void* stream) {
    bool empty = false;
    const int st = std_check(B, H, N, d, scale, 0, dtype, dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!q || !k || !s) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(s)) return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const size_t tbytes = size_t(BH * N * d) * 2;
    const Range rs = range(s, size_t(BH * N * N) * 4);
    if (overlap(rs, range(q, tbytes)) || overlap(rs, range(k, tbytes))) return ATTN_ERR_ALIAS;
    const hipError_t e = attn::launch_std_scores(q, k, s, BH, int(N), int(d), scale, dtype,
                                                 (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int std_softmax(const float* s, void* p, float* lse, int64_t B, int64_t H, int64_t N, int causal,
                int dtype, void* stream) {
    bool empty = false;
    const int st = std_check(B, H, N, 64, 1.f, causal, dtype, dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!s || !p || !lse) return ATTN_ERR_NULL;
    if (!aligned16(s) || !aligned16(p) || !aligned16(lse)) return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const Range rs = range(s, size_t(BH * N * N) * 4), rp = range(p, size_t(BH * N * N) * 2),
                rl = range(lse, size_t(BH * N) * 4);
    if (overlap(rp, rs) || overlap(rl, rs) || overlap(rp, rl)) return ATTN_ERR_ALIAS;
    const hipError_t e = attn::launch_std_softmax(s, p, lse, BH, int(N), causal, dtype,
                                                  (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int std_pv(const void* p, const void* v, void* o, int64_t B, int64_t H, int64_t N, int64_t d,
           int dtype, int out_dtype, void* stream) {
    bool empty = false;
    const int st = std_check(B, H, N, d, 1.f, 0, dtype, out_dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!p || !v || !o) return ATTN_ERR_NULL;
    if (!aligned16(p) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const Range ro = range(o, size_t(BH * N * d) * (out_dtype == ATTN_F32 ? 4 : 2));
    if (overlap(ro, range(p, size_t(BH * N * N) * 2)) || overlap(ro, range(v, size_t(BH * N * d) * 2)))
        return ATTN_ERR_ALIAS;
    const hipError_t e = attn::launch_std_pv(p, v, o, BH, int(N), int(d), dtype, out_dtype == ATTN_F32,
                                             (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t attn_std_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    bool empty = false;
    if (std_check(B, H, N, d, 1.f, 0, dtype, dtype, &empty) != ATTN_OK || empty) return 0;
    return std_s_bytes(B * H, N) + size_t(B * H * N * N) * 2;
}

int attn_std_scores(const void* q, const void* k, float* s, int64_t B, int64_t H, int64_t N,
                    int64_t d, float scale, int dtype, void* stream) {
    return std_scores(q, k, s, B, H, N, d, scale, dtype, stream);
}

int attn_std_softmax(const float* s, void* p, float* lse, int64_t B, int64_t H, int64_t N,
                     int causal, int dtype, void* stream) {
    return std_softmax(s, p, lse, B, H, N, causal, dtype, stream);
}

int attn_std_pv(const void* p, const void* v, void* o, int64_t B, int64_t H, int64_t N, int64_t d,
                int dtype, int out_dtype, void* stream) {
    return std_pv(p, v, o, B, H, N, d, dtype, out_dtype, stream);
}

int attn_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                 size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 int causal, int dtype, int out_dtype, void* stream) {
    bool empty = false;
    int st = std_check(B, H, N, d, scale, causal, dtype, out_dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_ALIGN;
    const int64_t BH = B * H;
    const size_t sb = std_s_bytes(BH, N), need = sb + size_t(BH * N * N) * 2;
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    const size_t tbytes = size_t(BH * N * d) * 2;
    const size_t obytes = size_t(BH * N * d) * (out_dtype == ATTN_F32 ? 4 : 2);
    const Range ro = range(o, obytes), rl = range(lse, size_t(BH * N) * 4), rw = range(workspace, need);
    const Range in[3] = {range(q, tbytes), range(k, tbytes), range(v, tbytes)};
    for (const Range& r : in)
        if (overlap(ro, r) || overlap(rl, r) || overlap(rw, r)) return ATTN_ERR_ALIAS;
    if (overlap(ro, rl) || overlap(ro, rw) || overlap(rl, rw)) return ATTN_ERR_ALIAS;
    float* s = static_cast<float*>(workspace);
    void* p = static_cast<char*>(workspace) + sb;
    if ((st = std_scores(q, k, s, B, H, N, d, scale, dtype, stream)) != ATTN_OK) return st;
    if ((st = std_softmax(s, p, lse, B, H, N, causal, dtype, stream)) != ATTN_OK) return st;
    return std_pv(p, v, o, B, H, N, d, dtype, out_dtype, stream);
}


int attn_probe_mfma(float* out, int64_t workgroups, int64_t rounds, void* stream) {
    if (workgroups < 1 || workgroups > (int64_t(1) << 20) || rounds < 1 || rounds > (int64_t(1) << 24))
        return ATTN_ERR_SHAPE;
    if (!out) return ATTN_ERR_NULL;
    if (!aligned16(out)) return ATTN_ERR_ALIGN;
    const hipError_t e = attn::launch_mfma_probe(out, int(workgroups), int(rounds), (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_probe_hbm(const void* buf, int64_t bytes, unsigned* out, int64_t workgroups, void* stream) {
    if (workgroups < 1 || workgroups > (int64_t(1) << 20) || bytes < 16 || bytes % 16 != 0 ||
        bytes > (int64_t(1) << 42))
        return ATTN_ERR_SHAPE;
    if (!buf || !out) return ATTN_ERR_NULL;
    if (!aligned16(buf) || !aligned16(out)) return ATTN_ERR_ALIGN;
    if (overlap(range(buf, size_t(bytes)), range(out, size_t(workgroups) * 256 * sizeof(unsigned))))
        return ATTN_ERR_ALIAS;
    const hipError_t e = attn::launch_hbm_probe(buf, (long long)(bytes / 16), out, int(workgroups),
                                                (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
