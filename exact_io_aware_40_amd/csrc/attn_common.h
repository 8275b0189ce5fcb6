// attn_common.h -- device-side building blocks shared by the forward and
// backward attention kernels for gfx950 (CDNA4, wave64).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_{bf16,f16},
// D[32x32] += A[32x16] * B[16x32], fp32 accumulate), for lane l of a wave:
//   A operand: 8 elements A[m = l%32][k = 8*(l/32) + e], e = 0..7
//   B operand: 8 elements B[k = 8*(l/32) + e][n = l%32]
//   C/D      : 16 floats  D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15
// A contraction may visit its k index in any order as long as A and B agree,
// which lets a probability tile produced in accumulator layout feed the next
// product as a B operand without any data movement.
//
// LDS transpose reads (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane t receives element (t % 4) of the 4-element vector addressed by lane
// (t / 4 + 4 j) as its element j.  Pointing the 16 lanes of a group at a 4x4
// arrangement of 4-element row pieces therefore delivers columns, which is
// how a row-major [key][d] tile is read as the k-contiguous operand of a
// product that contracts over keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes at `base`: loads past the end return 0.
// base and bytes must be the same for the whole wave; they are moved to
// scalar registers explicitly so that every load using the resource is a
// single instruction (a resource the compiler believes may differ between
// lanes costs a loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    const unsigned long long p = reinterpret_cast<unsigned long long>(base);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
    void* ub = reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}

// Work-item, workgroup and grid indices (x) read with the hardware
// builtins.  HIP's threadIdx, blockIdx and gridDim go through device-library
// functions that are not inlined under this build's floating-point flags:
// each use would be a call whose entry waits for every outstanding memory
// operation of the wave.
__device__ __forceinline__ int tid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int wg_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int num_wg_x() {
    return (int)(__builtin_amdgcn_grid_size_x() / __builtin_amdgcn_workgroup_size_x());
}

// Byte address in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's 16 bytes, read at
// byte offset `voff` of the buffer, land at lds_base + 16 l (lds_base must be
// the same for the whole wave).  Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, char* lds_base, unsigned voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// The same copy written as inline assembly.  The compiler then knows of no
// copy into LDS in flight, so it does not make LDS reads wait for it (it
// cannot tell which LDS bytes a copy writes, and before a transposing read it
// would wait for every outstanding copy); the caller orders the copies
// against the reads with wait_vmem_upto and barriers.  lds_base is an LDS
// byte address, the same for the whole wave.  M0 is written here; nothing
// else in the kernels that use this relies on it.
__device__ __forceinline__ void dma16_async(__amdgpu_buffer_rsrc_t rs, unsigned lds_base, unsigned voff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rs)
                     : "memory", "m0");
#pragma clang diagnostic pop
}

// dma16_async marked non-temporal, for data that no other workgroup reads
// (a decode step's key/value cache, streamed once): its lines are not kept
// in the caches at the expense of lines that others will read again.  For a
// one-pass read of the cache this streams 9-12% faster; for tiles that
// several workgroups read it is 9-12% slower.
__device__ __forceinline__ void dma16_async_once(__amdgpu_buffer_rsrc_t rs, unsigned lds_base, unsigned voff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rs)
                     : "memory", "m0");
#pragma clang diagnostic pop
}

// Wait until this wave's outstanding vector-memory operations (including
// direct-to-LDS copies) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector-memory operations are still in
// flight (they complete in issue order); expcnt and lgkmcnt are left alone.
template <int N> __device__ __forceinline__ void wait_vmem_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that does not wait for this wave's own memory operations
// (copies still in flight stay in flight); the empty asm statements keep the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_only() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Per-element-type pieces: operand vector types, the 32x32x16 product, and
// round-to-nearest-even conversion of four floats.
template <typename T> struct Elem;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <> struct Elem<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    typedef i32x4 raw;                          // an operand's bits
    static constexpr int KSTEP = 16;            // k of one product
    static constexpr unsigned kSign = 0x80008000u;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ v4 cvt4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
    // two floats rounded to nearest even and packed into one dword
    static __device__ __forceinline__ unsigned cvt2(float a, float b) {
        const f32x2 x = {a, b};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
    }
    // acc + both elements of a packed pair (fp32 accumulation)
    static __device__ __forceinline__ float sum2(unsigned pr, float acc) {
        const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr), one, acc, false);
    }
    // acc + x[0] + ... + x[7] of an 8-element operand (fp32 accumulation)
    static __device__ __forceinline__ float sum8(v8 x, float acc) {
        const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2 pr = {x[2 * i], x[2 * i + 1]};
            acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
        }
        return acc;
    }
};

template <> struct Elem<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    typedef i32x4 raw;
    static constexpr int KSTEP = 16;
    static constexpr unsigned kSign = 0x80008000u;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ v4 cvt4(f32x4 x) { return __builtin_convertvector(x, f16x4); }
    static __device__ __forceinline__ unsigned cvt2(float a, float b) {
        const f32x2 x = {a, b};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(x, f16x2));
    }
    static __device__ __forceinline__ float sum2(unsigned pr, float acc) {
        const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), one, acc, false);
    }
    static __device__ __forceinline__ float sum8(v8 x, float acc) {
        const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2 pr = {x[2 * i], x[2 * i + 1]};
            acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
        }
        return acc;
    }
};

// 8-bit E4M3 elements (the OCP format: sign, 4 exponent bits with bias 7, 3
// mantissa bits, no infinity; largest value 448), the format of gfx950's
// 8-bit conversions and of format selector 0 of its 8-bit products.
struct fp8e4m3 {
    unsigned char bits;
};
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <> struct Elem<fp8e4m3> {
    typedef i32x8 v8;   // 32 elements: one operand of the 32x32x64 product
    typedef i32x8 raw;
    static constexpr int KSTEP = 64;
    static constexpr unsigned kSign = 0x80808080u;
    // D[32x32] += A[32x64] * B[64x32] (v_mfma_f32_32x32x64_f8f6f4, both
    // operands E4M3, no block scales).  Lane l holds 32 elements of row l % 32
    // of A and of column l % 32 of B; which k an element stands for depends
    // only on l / 32 and its position, the same way for A and B, so a
    // contraction laid out consistently in both is exact whatever that map is.
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
    // a and b rounded to nearest even E4M3 (|a|, |b| <= 448), written to bytes
    // 0, 1 (hi false) or 2, 3 (hi true) of w; the other two bytes are kept
    static __device__ __forceinline__ unsigned cvt2_into(float a, float b, unsigned w, bool hi) {
        return hi ? (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, true)
                  : (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, false);
    }
};

template <typename V, typename U> __device__ __forceinline__ V bit_cast(U u) {
    static_assert(sizeof(V) == sizeof(U), "size mismatch");
    return __builtin_bit_cast(V, u);
}

// Value of x held by lane l ^ 32, combined symmetrically: the permlane32
// swap hands each lane the pair (x[l & 31], x[(l & 31) + 32]).
__device__ __forceinline__ f32x2 pair32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    f32x2 out;
    out[0] = __uint_as_float(r[0]);
    out[1] = __uint_as_float(r[1]);
    return out;
}
__device__ __forceinline__ float max32(float x) {
    f32x2 p = pair32(x);
    return fmaxf(p[0], p[1]);
}
__device__ __forceinline__ float sum32(float x) {
    f32x2 p = pair32(x);
    return p[0] + p[1];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 8-byte transposing LDS read at byte address `addr` of the LDS window.
__device__ __forceinline__ i16x4 lds_read_tr16(const char* base, int addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + addr));
}

// LDS reads written as inline assembly, for loops that also have
// direct-to-LDS copies in flight: the compiler cannot tell that a
// transposing read does not touch the copies' destination and would wait for
// every outstanding copy before it.  The compiler does not count these reads
// either, so their results may be used only after lds_wait_upto<n>(), with n
// the number of LDS reads issued after them.  `addr` is a byte address in
// LDS, `off` a constant below 65536 (it must fold to one after inlining).
__device__ __forceinline__ i32x4 lds_read_b128_asm(unsigned addr, int off) {
    i32x4 r;
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(off));
    return r;
}
__device__ __forceinline__ i32x2 lds_read_tr16_asm(unsigned addr, int off) {
    i32x2 r;
    __asm__ volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(off));
    return r;
}
// The 8-bit transposing read: within each group of 16 lanes, lane t receives
// byte (t % 8) of the 8-byte piece addressed by lane (t % 16) / 8 + 2 j of its
// group as its byte j, j = 0..7.
__device__ __forceinline__ i32x2 lds_read_tr8_asm(unsigned addr, int off) {
    i32x2 r;
    __asm__ volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(off));
    return r;
}
// Wait until at most N LDS operations of this wave are outstanding; the six
// registers passed are the results this makes safe to use (they are tied to
// the wait so that no use is scheduled above it).
template <int N>
__device__ __forceinline__ void lds_wait_upto(i32x4& a, i32x4& b, i32x2& c, i32x2& d, i32x2& e,
                                              i32x2& f) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
    __asm__ volatile("s_waitcnt lgkmcnt(%6)"
                     : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f)
                     : "i"(N));
}

// The same wait for one 16-byte result.
template <int N>
__device__ __forceinline__ void lds_wait_upto(i32x4& a) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
    __asm__ volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}

// The same wait for two 8-byte results.
template <int N>
__device__ __forceinline__ void lds_wait_upto(i32x2& a, i32x2& b) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
    __asm__ volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// The same wait for two 16-byte results.
template <int N>
__device__ __forceinline__ void lds_wait_upto(i32x4& a, i32x4& b) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
    __asm__ volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// The same wait for three results (one 16-byte and two 8-byte reads).
template <int N>
__device__ __forceinline__ void lds_wait_upto(i32x4& a, i32x2& b, i32x2& c) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
    __asm__ volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "i"(N));
}

// Two 4-element pieces -> one 8-element operand.
template <typename V8>
__device__ __forceinline__ V8 join8(i16x4 a, i16x4 b) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return bit_cast<V8>(v);
}

// LDS placement of 16-byte granule g of row r in a [rows][D] tile of 16-bit
// elements.  Tiles are read two ways: 16-byte reads of consecutive rows at
// one granule column (operands whose k index runs along d), and transposing
// 8-byte reads of 4 aligned consecutive rows by 2-4 adjacent granules
// (operands whose k index runs along the rows).  The row's granules are
// permuted by XOR with a key chosen so that the lanes the LDS serves
// together (256 bytes per clock, 64 banks) touch distinct banks in both
// patterns: for 128-byte rows two rows share a 256-byte line, so the key
// also depends on the row's half.
#ifndef ATTN_LDS_BANKS
#define ATTN_LDS_BANKS 64
#endif
template <int D> __device__ __forceinline__ int lds_key(int r) {
#if ATTN_LDS_BANKS == 64
    if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
#else
    return ((r & 3) << 1) | ((r >> 2) & 1);
#endif
}
template <int D> __device__ __forceinline__ int t_off(int r, int g) {
    return r * (D * 2) + ((g ^ lds_key<D>(r)) << 4);
}

// Output element stores: four fp32 values, rounded once to nearest even for
// a 16-bit output type, written as they are for an fp32 output.
template <typename TO> __device__ __forceinline__ void store4(TO* p, f32x4 x);
template <> __device__ __forceinline__ void store4<__bf16>(__bf16* p, f32x4 x) {
    *(bf16x4*)p = __builtin_convertvector(x, bf16x4);
}
template <> __device__ __forceinline__ void store4<_Float16>(_Float16* p, f32x4 x) {
    *(f16x4*)p = __builtin_convertvector(x, f16x4);
}
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 x) { *(f32x4*)p = x; }

// Store a wave's 32-row x D accumulator set, times f, through LDS.  In the
// layout of a product whose n index is the row (lane l holds row l % 32,
// four consecutive columns 32 cb + 8 g + 4 (l / 32) .. + 3 per quad g of
// block cb), a direct store writes 64 rows x 8 bytes per instruction.
// Instead the rounded rows go to `stage` (this wave's own 32 * D *
// sizeof(TO) bytes of LDS, 16-byte aligned; each row's 16-byte granules
// XOR-permuted by the row, so that the lanes' rows fall on distinct banks)
// and come back as 16-byte row pieces: each store instruction then writes
// 1 KiB (16-bit) of consecutive rows.  Rows base + r * D for r < rows_left
// are written (rows_left may be <= 0: nothing).  The caller makes sure no
// other wave uses `stage` meanwhile.
template <typename TO, int D>
__device__ __forceinline__ void store_rows_staged(char* stage, TO* __restrict__ base, int rows_left,
                                                  const f32x16* acc, float f, int lane) {
    constexpr int GPR = D * (int)sizeof(TO) / 16;   // 16-byte granules per row
    static_assert((GPR & (GPR - 1)) == 0 && 32 * GPR % 64 == 0, "");
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 x = {acc[cb][4 * g] * f, acc[cb][4 * g + 1] * f, acc[cb][4 * g + 2] * f,
                       acc[cb][4 * g + 3] * f};
            const int byte = (32 * cb + 8 * g + 4 * h) * (int)sizeof(TO);
            const int gi = (byte >> 4) ^ (l32 & (GPR - 1));
            store4<TO>((TO*)(stage + l32 * (GPR * 16) + gi * 16 + (byte & 15)), x);
        }
    }
#pragma unroll 1
    for (int i = 0; i < 32 * GPR / 64; ++i) {
        const int gi = i * 64 + lane, row = gi / GPR, col = gi % GPR;
        const i32x4 y = *(const i32x4*)(stage + row * (GPR * 16) + ((col ^ (row & (GPR - 1))) * 16));
        if (row < rows_left) *(i32x4*)((char*)(base + (size_t)row * D) + col * 16) = y;
    }
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011), the generator of the dropout mask.  A round
// maps the counter (c0, c1, c2, c3) under key (k0, k1) to
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); round n
// (0 .. 9) uses the key advanced n times by the Weyl constants W0, W1.
constexpr unsigned kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr unsigned kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;
__device__ __forceinline__ void philox_round(unsigned (&c)[4], unsigned k0, unsigned k1, int n) {
    const unsigned long long p0 = (unsigned long long)kPhiloxM0 * c[0];
    const unsigned long long p1 = (unsigned long long)kPhiloxM1 * c[2];
    const unsigned n0 = (unsigned)(p1 >> 32) ^ c[1] ^ (k0 + (unsigned)n * kPhiloxW0);
    const unsigned n2 = (unsigned)(p0 >> 32) ^ c[3] ^ (k1 + (unsigned)n * kPhiloxW1);
    c[1] = (unsigned)p1;
    c[3] = (unsigned)p0;
    c[0] = n0;
    c[2] = n2;
}
// Dropout keeps an element whose generator byte is at least the threshold t.
__device__ __forceinline__ bool drop_keep(unsigned word, int byte, unsigned t) {
    return ((word >> (8 * byte)) & 0xFFu) >= t;
}

// Workgroup id -> logical work item, so that consecutive logical items land
// on the same XCD.  The dispatcher hands workgroup ids to the 8 XCDs in
// round-robin order; XCD x receives logical items [base(x), base(x)+count(x)).
__device__ __forceinline__ int xcd_remap(int id, int total) {
    const int per = total >> 3, rem = total & 7, x = id & 7;
    return x * per + (x < rem ? x : rem) + (id >> 3);
}

}  // namespace attn
