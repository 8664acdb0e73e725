// ssd_device.hpp -- device-side helpers shared by the gfx950 kernels:
// bf16 <-> fp32 conversion, fast transcendental wrappers, 16x16 MFMA tile
// wrappers and the fragment layout they share.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16
// bf16 is the top half of an fp32 bit pattern.  Widening is exact (a shift);
// narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// ---------------------------------------------------------------- math
// exp2 on the hardware unit (v_exp_f32); inputs here are <= 0 or moderate.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// silu(v) = v * sigmoid(v) = v / (1 + 2^(-v log2 e)).
__device__ __forceinline__ float silu_f(float v) { return v * fast_rcp(1.0f + fast_exp2(-v * kLog2e)); }
// softplus(v) = max(v, 0) + log(1 + e^-|v|), with the accurate libm routines.
__device__ __forceinline__ float softplus_f(float v) { return fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v))); }

// ---------------------------------------------------------------- MFMA tiles
// All contractions are built from 16x16 output tiles.  Fragment layout, for
// lane l = 16*q + i (q = l / 16, i = l % 16):
//   * an operand fragment holds 4 consecutive K indices 4q..4q+3 of a 16-wide
//     K block, at row/column index i;
//   * an accumulator tile holds rows 4q..4q+3 of column i.
// Hence an accumulator tile is, unchanged, an operand fragment whose K index
// is the tile's row index.  A bf16 MFMA (16x16x32) consumes two K blocks at
// once: elements 0..3 of both operands carry block 0, elements 4..7 block 1;
// the fp32 MFMA (16x16x4) consumes one element per instruction.  Only the
// pairing of A and B elements matters for the sum over K, so this fixed
// assignment of K indices to (lane group, element) is valid for both.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct FragBF { uint32_t a, b; };   // 4 bf16: K = 4q+0,1 in a; 4q+2,3 in b

__device__ __forceinline__ f32x4 mma_bf16(f32x4 acc, FragBF a0, FragBF a1, FragBF b0, FragBF b1) {
    union { uint32_t u[4]; bf16x8 v; } A, B;
    A.u[0] = a0.a; A.u[1] = a0.b; A.u[2] = a1.a; A.u[3] = a1.b;
    B.u[0] = b0.a; B.u[1] = b0.b; B.u[2] = b1.a; B.u[3] = b1.b;
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.v, B.v, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_f32(f32x4 acc, float4 a, float4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ FragBF frag_from_f32(f32x4 v) {
    FragBF f;
    f.a = pack_bf16x2(v[0], v[1]);
    f.b = pack_bf16x2(v[2], v[3]);
    return f;
}

// ---------------------------------------------------------------- wave scan
// One step of an inclusive segmented scan across a wave64 with DPP moves:
// (value, segment-start flag, last segment start index).  Lanes whose source
// is outside the move (or whose row is masked off) combine with the identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ void segscan_step(float& v, int& f, int& s) {
    const float vu = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
    const int fu = __builtin_amdgcn_update_dpp(0, f, CTRL, ROWS, 0xF, false);
    const int su = __builtin_amdgcn_update_dpp(-1, s, CTRL, ROWS, 0xF, false);
    v = f ? v : v + vu;
    f = f | fu;
    s = max(s, su);
}
// v: per-lane value; f: 1 where a segment starts at this lane; s: lane index
// where f, else -1.  On return v is the sum from the lane's segment start (or
// lane 0) to the lane, s the last segment start at or before the lane (-1 if
// none).  Kogge-Stone within 16-lane rows (row_shr 1, 2, 4, 8), then the
// row_bcast 15 / 31 moves carry row totals across rows.
__device__ __forceinline__ void wave_segscan(float& v, int f, int& s) {
    segscan_step<0x111, 0xF>(v, f, s);
    segscan_step<0x112, 0xF>(v, f, s);
    segscan_step<0x114, 0xF>(v, f, s);
    segscan_step<0x118, 0xF>(v, f, s);
    segscan_step<0x142, 0xA>(v, f, s);
    segscan_step<0x143, 0xC>(v, f, s);
}

// ---------------------------------------------------------------- split operands
// fp32 operands of the split-product contractions are held in LDS as two
// bf16 planes, v = hi + lo + e with hi = bf16(v), lo = bf16(v - hi) (both
// rounded to nearest even, 8 significant bits each; v - hi is exact), so
// |v - hi| <= 2^-8 |v| and |e| <= 2^-16 |v|.  A matrix
// region of `cnt` fp32 slots keeps its byte size: the hi plane is its first
// cnt 16-bit elements, the lo plane the next cnt.  A product of two split
// operands is formed on the bf16 MFMA as lo*hi + hi*lo + hi*hi with fp32
// accumulation (the lo*lo term, at most 2^-16 of the product, is dropped):
// three 16x16x32 MFMAs replace the eight 16x16x4 fp32 ones for the same
// 32-wide K range, at most ~3 * 2^-16 relative error per product term.
struct Split4 { FragBF hi, lo; };      // 4 consecutive K elements of a fragment
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}
__device__ __forceinline__ Split4 split4(float a, float b, float c, float d) {
    Split4 r;
    split_pair(a, b, r.hi.a, r.lo.a);
    split_pair(c, d, r.hi.b, r.lo.b);
    return r;
}
__device__ __forceinline__ Split4 split_zero() { return {{0u, 0u}, {0u, 0u}}; }
// the 4 elements at index i (a multiple of 4) of a split region of cnt slots
__device__ __forceinline__ Split4 pld(const uint16_t* p, int cnt, int i) {
    const uint2 h = *reinterpret_cast<const uint2*>(p + i);
    const uint2 l = *reinterpret_cast<const uint2*>(p + cnt + i);
    return {{h.x, h.y}, {l.x, l.y}};
}
__device__ __forceinline__ void pst4(uint16_t* p, int cnt, int i, float a, float b, float c, float d) {
    const Split4 v = split4(a, b, c, d);
    *reinterpret_cast<uint2*>(p + i) = make_uint2(v.hi.a, v.hi.b);
    *reinterpret_cast<uint2*>(p + cnt + i) = make_uint2(v.lo.a, v.lo.b);
}
// two consecutive elements at index i (even)
__device__ __forceinline__ void pst2(uint16_t* p, int cnt, int i, float a, float b) {
    uint32_t hi, lo;
    split_pair(a, b, hi, lo);
    *reinterpret_cast<uint32_t*>(p + i) = hi;
    *reinterpret_cast<uint32_t*>(p + cnt + i) = lo;
}
__device__ __forceinline__ void pst1(uint16_t* p, int cnt, int i, float v) {
    const uint32_t hi = f32_to_bf16_bits(v);
    p[i] = (uint16_t)hi;
    p[cnt + i] = (uint16_t)f32_to_bf16_bits(v - __uint_as_float(hi << 16));
}
// the value at index i of a split region of cnt slots (hi + lo: exact in fp32)
__device__ __forceinline__ float sget(const uint16_t* p, int cnt, int i) {
    return bf16_to_f32(p[i]) + bf16_to_f32(p[cnt + i]);
}
// acc += A B over two 16-wide K blocks (a0/b0: block 0, a1/b1: block 1)
__device__ __forceinline__ f32x4 mma_split(f32x4 acc, const Split4& a0, const Split4& a1, const Split4& b0,
                                           const Split4& b1) {
    acc = mma_bf16(acc, a0.lo, a1.lo, b0.hi, b1.hi);
    acc = mma_bf16(acc, a0.hi, a1.hi, b0.lo, b1.lo);
    return mma_bf16(acc, a0.hi, a1.hi, b0.hi, b1.hi);
}

// Transposed reads of 16-bit tiles (ds_read_b64_tr_b16): in each 16-lane
// group, result lane j element e is element (j mod 4) of source lane 4e + j/4,
// so a lane (q, m) that addresses row 4q + m/4, column 4(m mod 4) of a tile
// receives column m, rows 4q..4q+3 -- the operand fragment of the transposed
// tile.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
#define SSD_LDS __attribute__((address_space(3)))

__device__ __forceinline__ FragBF tr_read(const unsigned char* lds_base, uint32_t byte_off) {
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSD_LDS v4i16_t*)(lds_base + byte_off));
    FragBF f;
    f.a = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
    f.b = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    return f;
}
__device__ __forceinline__ FragBF plain_read(const unsigned char* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return {v.x, v.y};
}
// Workgroup barrier for LDS traffic only: this wave's LDS operations are done,
// then s_barrier.  (A fence-based barrier would also wait for the copies in
// flight.)  The memory clobber keeps the compiler from moving accesses across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

}  // namespace ssd
