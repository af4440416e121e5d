// Small device helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace octo {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulation.  Per lane l
// (n = l % 32, g = l / 32): A supplies row n and 8 of the 16 k values, B supplies
// column n and the same 8 k values, and the result holds column n, rows
// 8*(j/4) + 4*g + (j%4) for j = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void st16(bf16* p, bf16x8 v) {
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ bf16x4 ld8(const bf16* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ void st8(bf16* p, bf16x4 v) {
    *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ bf16x8 zero8() {
    return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// x as the sum of three bf16 values (the error is below 2^-24 |x|), in slots 0..2 of
// an MFMA operand; lanes of the upper half (k values 8..15) carry zeros.  The backward
// passes add a row's -LSE2 and -Delta to its scores through this one extra k-step.
__device__ __forceinline__ bf16x8 split3(float x, bool on) {
    x = on ? fmaxf(x, -1e30f) : 0.f;  // a padded row's -inf becomes a finite -1e30
    const bf16 h = (bf16)x;
    const float r1 = x - (float)h;
    const bf16 m = (bf16)r1;
    const bf16 l = (bf16)(r1 - (float)m);
    bf16x8 v = zero8();
    v[0] = h;
    v[1] = m;
    v[2] = l;
    return v;
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = 0.f;
    return z;
}

// Load through the constant address space: plan metadata is never written while a
// kernel runs, and with a wave-uniform address this becomes a scalar load (tracked
// by lgkmcnt, so it never waits behind the asynchronous LDS copies counted by vmcnt).
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return *(const __attribute__((address_space(4))) T*)(p);
#else
    return *p;
#endif
}
// The HIP vector structs are loaded as plain vectors: a struct load is split into
// scalar fields on the original (global) pointer, which would make it a vector-memory
// load and so a wait on every outstanding copy.
__device__ __forceinline__ int4 ld_const(const int4* p) {
    typedef __attribute__((ext_vector_type(4))) int i32x4;
    const i32x4 v = ld_const(reinterpret_cast<const i32x4*>(p));
    return make_int4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ int2 ld_const(const int2* p) {
    typedef __attribute__((ext_vector_type(2))) int i32x2;
    const i32x2 v = ld_const(reinterpret_cast<const i32x2*>(p));
    return make_int2(v[0], v[1]);
}

// Make the compiler wait here for a register loaded from memory (so later loops do not
// re-check it against outstanding asynchronous copies).
__device__ __forceinline__ void settle(const bf16x8& v) { asm volatile("" ::"v"(v)); }

// Wait for v and move it to accumulation registers: MFMA reads its A and B operands
// from either register file, and a loop-invariant operand kept there leaves the
// architectural registers free for staging LDS reads ahead of the MFMAs.
__device__ __forceinline__ void park(bf16x8& v) { asm volatile("" : "+a"(v)); }

// 2^x on the hardware exponential unit (exact 0 for -inf).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + the sum of the 8 bf16 values of v (v_dot2 against ones, two per instruction).
__device__ __forceinline__ float row_sum8(bf16x8 v, float acc) {
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, acc, false);
}

// ---------------------------------------------------------------- rotary embedding
//
// Rotate-half rotary embedding at a token's position (RopeFreq, kernels.h): feature
// pairs (x_i, x_{i+D/2}) turn by pos * theta_i.

// r^n for 0 <= n < 64 (binary powers; n is a compile-time constant plus a lane bit).
__device__ __forceinline__ double ipow64(double r, int n) {
    double out = 1.0, p = r;
#pragma unroll
    for (int b = 0; b < 6; ++b) {
        if ((n >> b) & 1) out *= p;
        p *= p;
    }
    return out;
}

// cos and sin of pair i's angle at position pos.  The angle in turns, pos * turn0 *
// ratio^i, is reduced in float64 to a fraction f of a turn in [-1/2, 1/2]; then f = q/4 +
// y/(2 pi) with q the nearest quarter turn and |y| <= pi/4, where the Taylor polynomials
// of sin y (to y^9/9!) and cos y (to y^10/10!) are within 2e-9; the quarter turns are
// applied exactly.  Straight-line code: no tables, no private memory.
__device__ __forceinline__ void rope_angle(int pos, const RopeFreq& f, int i, float& c,
                                           float& s) {
    const double t = (double)pos * (f.turn0 * ipow64(f.ratio, i));
    const float fr = (float)(t - rint(t));
    const float q = rintf(4.f * fr);
    const float y = (fr - 0.25f * q) * 6.283185307179586f;
    const float y2 = y * y;
    const float sy =
        y * (1.f + y2 * (-1.f / 6 + y2 * (1.f / 120 + y2 * (-1.f / 5040 + y2 * (1.f / 362880)))));
    const float cy =
        1.f + y2 * (-0.5f + y2 * (1.f / 24 + y2 * (-1.f / 720 + y2 * (1.f / 40320 +
                                                                       y2 * (-1.f / 3628800)))));
    const int qi = (int)q & 3;
    c = qi == 0 ? cy : qi == 1 ? -sy : qi == 2 ? -cy : sy;
    s = qi == 0 ? sy : qi == 1 ? cy : qi == 2 ? -sy : -cy;
}

// Turn the query operand of one lane in place: qf[ks][e] holds feature 16 ks + 8 g + e
// (the MFMA B-operand layout of one row), so the pair partner of ks < KS/2 is ks + KS/2
// in the same lane.  sign = +1 turns forward, -1 back.
template <int KS>
__device__ __forceinline__ void rope_operand(bf16x8 (&qf)[KS], int pos, const RopeFreq& rf,
                                             int g, float sign) {
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float c, s;
            rope_angle(pos, rf, 16 * ks + 8 * g + e, c, s);
            s *= sign;
            const float a = (float)qf[ks][e], b = (float)qf[ks + KS / 2][e];
            qf[ks][e] = (bf16)(a * c - b * s);
            qf[ks + KS / 2][e] = (bf16)(b * c + a * s);
        }
}

// Turn an accumulator tile in place: acc[db][j] holds feature 32 db + 8 (j / 4) + 4 g +
// j % 4 of the lane's column (the MFMA result layout of a D x 32 transposed tile), so
// the pair partner of db < DB/2 is db + DB/2 in the same lane.
template <int DB>
__device__ __forceinline__ void rope_accum(f32x16 (&acc)[DB], int pos, const RopeFreq& rf,
                                           int g, float sign) {
#pragma unroll
    for (int db = 0; db < DB / 2; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float c, s;
            rope_angle(pos, rf, 32 * db + 8 * (j >> 2) + 4 * g + (j & 3), c, s);
            s *= sign;
            const float a = acc[db][j], b = acc[db + DB / 2][j];
            acc[db][j] = a * c - b * s;
            acc[db + DB / 2][j] = b * c + a * s;
        }
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Map a block index onto (group, member) so that the `members` blocks of one group
// run on the same XCD (workgroups are dealt to the 8 XCDs round-robin by index) and
// groups keep their launch order.  Returns false for padding blocks.
__device__ __forceinline__ bool xcd_group(int bid, int members, int n_groups, int& group,
                                          int& member) {
    const int per = 8 * members;
    const int i8 = bid / per;
    const int rem = bid - i8 * per;
    group = i8 * 8 + (rem & 7);
    member = rem >> 3;
    return group < n_groups;
}

inline int xcd_grid(int n_groups, int members) { return (n_groups + 7) / 8 * 8 * members; }

// ---------------------------------------------------------------- LDS staging

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)(p);
}

// Asynchronous 16-byte copy global -> LDS (global_load_lds_dwordx4): lane i's 16 bytes
// land at LDS byte address lds_wave_base + 16 * i (M0); lds_wave_base must be the same
// for every lane of the wave.  Issued as inline assembly so the compiler neither
// inserts waits for it nor reorders LDS accesses around it: completion is tracked
// with explicit vmcnt waits, and the copy becomes visible to other waves after the
// issuing wave has waited and a barrier has passed.
__device__ __forceinline__ void dma16(const void* g, unsigned lds_wave_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_wave_base))
                 : "memory", "m0");
}

// The same copy from a wave-uniform base address plus a per-lane 32-bit byte offset:
// the per-lane part is computed once, the base on the scalar unit.
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff, unsigned lds_wave_base) {
    // The base is wave-uniform by contract; reading it through readfirstlane keeps it in
    // scalar registers even where the compiler computed it in vector registers.
    // (readfirstlane returns a signed int: widen through unsigned, never sign-extend.)
    const uint64_t b = reinterpret_cast<uint64_t>(sbase);
    const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
    const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
    const uint64_t sb = (hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_wave_base))
                 : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this wave's LDS (and scalar memory) operations have completed.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier without the implied memory fence of __syncthreads (which would
// drain every outstanding load, prefetches included).  LDS written by regular stores
// must be waited for (lgkmcnt) by the writer before it.  The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Transposed 8-byte LDS read (ds_read_b64_tr_b16).  In every group of 16 lanes,
// lane i receives element i % 4 of the 8-byte rows addressed by lanes 4j + i / 4,
// j = 0..3.  Addressing lane r at X[k0 + r / 4][c0 + 4 * (r % 4)] of a row-major
// 16-bit matrix therefore gives lane i the four values X[k0 + j][c0 + i].
__device__ __forceinline__ bf16x4 ld8_tr(const void* lds_addr) {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(lds_addr));
    return __builtin_bit_cast(bf16x4, v);
}

// LDS reads at a per-lane offset plus a constant (folded into the instruction's
// immediate offset once loops are unrolled).
__device__ __forceinline__ bf16x8 lds16(const unsigned char* smem, int lane_off, int imm) {
    return *reinterpret_cast<const bf16x8*>(smem + lane_off + imm);
}
__device__ __forceinline__ bf16x4 lds8_tr(const unsigned char* smem, int lane_off, int imm) {
    return ld8_tr(smem + lane_off + imm);
}

// 16-byte slot holding chunk `chunk` (8 elements) of row `row` in a row-major LDS tile
// of 16-bit elements with D columns, XOR-swizzled by a function of the row's low bits
// so that (a) 16 lanes reading the same chunk of 16 consecutive rows and (b) 16 lanes
// reading 4 chunks of 4 consecutive rows (the transposed reads) hit distinct banks.
template <int D>
__host__ __device__ constexpr int swz_key(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ swz_key<D>(row);
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {  // byte offset
    return row * (D * 2) + swz<D>(row, chunk) * 16;
}

}  // namespace octo
