// common.hpp -- device helpers shared by the gfx950 kernels of libreplayssm.
//
// Checkpoint tile layout ("fragment order").  A (b, h) state is viewed as
// S^T[r][c]: r runs over the reduction axis of the read-out (Mamba-2 N, GDN
// d_k), c over the output axis (Mamba-2 P, GDN d_v).  The tile is cut into
// column strips of 16 (one wave each) and, inside a strip, into 16 x 16
// blocks along r.  Inside a block, lane l holds the four consecutive rows
// r = 4*(l/16) + 0..3 of column c = l%16 as one float4.  This is exactly the
// accumulator layout of v_mfma_f32_16x16x4_f32, so the fold's MFMA results
// line up with the registers the checkpoint was loaded into, and each lane's
// four values are one 128-bit load.  Blocks are stored lane-contiguous:
//   float4 index = ((tile * STRIPS + strip) * NB + block) * 64 + lane
// so every wave-wide load or store is one contiguous 1 KiB transaction.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace rs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---- scalar conversions -------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet): gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// e^x for the decay factors (x <= 0 in use): v_exp_f32 on x log2(e).  The
// product's rounding changes the result by a relative 2^-24 |x log2 e|, about
// 1e-6 for the decays of one window.
__device__ __forceinline__ float fexp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// A value every lane of the wave holds the same copy of, moved to a scalar
// register (index arithmetic on it then runs on the scalar unit).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read of a value no workgroup of the launch writes, at a wave-uniform address,
// through the constant address space: the compiler emits a scalar load, whose
// completion is counted apart from the vector loads, so waiting for it never
// waits for checkpoint loads issued before or after it.  (Reads only; data
// written by an earlier launch is visible, the scalar cache being invalidated
// at every dispatch.)
template <typename T>
__device__ __forceinline__ T uload(const T* p)
{
    return *(const __attribute__((address_space(4))) T*)p;
}

template <int IO>
__device__ __forceinline__ float ld_io(const void* p, size_t i) {
    if constexpr (IO == IO_F32) return static_cast<const float*>(p)[i];
    else return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int IO>
__device__ __forceinline__ void st_io(void* p, size_t i, float v) {
    if constexpr (IO == IO_F32) static_cast<float*>(p)[i] = v;
    else static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
}

// ---- wave-level helpers ---------------------------------------------------
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ---- DPP (data-parallel primitives) on gfx9: VALU lane permutes without LDS
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;      // lane i <-> 15-i within a row of 16
constexpr int DPP_ROW_HALF_MIRROR = 0x141; // lane i <-> 7-i within half a row
constexpr int DPP_ROW_BCAST15 = 0x142;     // lane 15 of a row -> the next row
constexpr int DPP_ROW_BCAST31 = 0x143;     // lane 31 -> rows 2 and 3

constexpr int DPP_ROW_SHR1 = 0x111;        // lane i <- lane i-1 within a row (0 at the row start)
constexpr int DPP_ROW_SHR2 = 0x112;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_SHR8 = 0x118;

// Inclusive prefix sum over lanes 0..31 (Hillis-Steele within each row of 16,
// then row 0's total carried into row 1).  Lanes 32..63 hold partial values.
__device__ __forceinline__ float scan32_inclusive(float v) {
    v += dpp_mov<DPP_ROW_SHR1>(v);
    v += dpp_mov<DPP_ROW_SHR2>(v);
    v += dpp_mov<DPP_ROW_SHR4>(v);
    v += dpp_mov<DPP_ROW_SHR8>(v);
    v += dpp_mov<0x142, 0xa>(v);            // row_bcast:15 into rows 1 and 3
    return v;
}

// Sum over the 4 lanes of each quad; every lane of the quad gets the sum.
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_mov<DPP_QUAD_XOR1>(v);
    v += dpp_mov<DPP_QUAD_XOR2>(v);
    return v;
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the whole wave, returned to every lane (wave-uniform): quads, half
// rows, rows by mirrors, then rows into lane 63 by the row broadcasts.
__device__ __forceinline__ float wave_sum_uniform(float v) {
    v = quad_sum(v);
    v += dpp_mov<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_mov<DPP_ROW_MIRROR>(v);
    v += dpp_mov<DPP_ROW_BCAST15, 0xa>(v);
    v += dpp_mov<DPP_ROW_BCAST31, 0xc>(v);
    return readlane(v, 63);
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32 or 64),
// returned to every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
    if constexpr (N == 1) return v;
    if constexpr (N == 2) return v + dpp_mov<DPP_QUAD_XOR1>(v);
    v = quad_sum(v);
    if constexpr (N >= 8) v += dpp_mov<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (N >= 16) v += dpp_mov<DPP_ROW_MIRROR>(v);
    if constexpr (N == 32) {
        v += dpp_mov<DPP_ROW_BCAST15, 0xa>(v);            // rows 1 and 3 hold their pair's sum
        const float lo = readlane(v, 31), hi = readlane(v, 63);
        v = (__lane_id() < 32) ? lo : hi;
    }
    if constexpr (N == 64) {
        v += dpp_mov<DPP_ROW_BCAST15, 0xa>(v);
        v += dpp_mov<DPP_ROW_BCAST31, 0xc>(v);
        v = readlane(v, 63);
    }
    return v;
}

// Across the four 16-lane rows of a wave, on gfx950's row-swap permutes (VALU,
// no LDS round trip): v_permlane16_swap with both operands v leaves rows
// (r0, r0, r2, r2) in one register and (r1, r1, r3, r3) in the other, so their
// sum holds r0 + r1 in rows 0-1 and r2 + r3 in rows 2-3; v_permlane32_swap does
// the same for the two halves.  Every lane ends with (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float row_pair_swap16(float v, float& other) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                     false, false);
    other = __builtin_bit_cast(float, (uint32_t)r[1]);
    return __builtin_bit_cast(float, (uint32_t)r[0]);
}
__device__ __forceinline__ float half_swap32(float v, float& other) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                     false, false);
    other = __builtin_bit_cast(float, (uint32_t)r[1]);
    return __builtin_bit_cast(float, (uint32_t)r[0]);
}

// Sum over the four lanes that share (lane % 16): lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float sum_over_row_groups(float v) {
    float o;
    const float a = row_pair_swap16(v, o);
    v = a + o;
    const float c = half_swap32(v, o);
    return c + o;
}

// Maximum over the same four lanes.
__device__ __forceinline__ float max_over_row_groups(float v) {
    float o;
    const float a = row_pair_swap16(v, o);
    v = fmaxf(a, o);
    const float c = half_swap32(v, o);
    return fmaxf(c, o);
}

// Order LDS accesses made by different lanes of the same wave (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup -> tile mapping.  Consecutive workgroups are dispatched round-robin
// over the 8 XCDs; remapping gives each XCD a contiguous range of tiles so that
// heads sharing group inputs (B/C, q/k) and neighbouring sequences share an L2.
__device__ __forceinline__ int xcd_tile_index() {
    const int n = (int)gridDim.x, i = (int)blockIdx.x;
    if ((n & 7) == 0) return (i & 7) * (n >> 3) + (i >> 3);
    return i;
}

// A (b, h) tile may be split over `nsplit` workgroups along its output axis;
// consecutive work items are the splits of one head, then the heads of one
// sequence.
struct TileIdx {
    int b, h, sp;
};

// Division by a divisor d that is the same for the whole launch, through a
// multiplier the host computes once (magic_div): q = floor(n m / 2^32) with
// m = floor(2^32 / d) + 1, exact whenever n d < 2^32; m = 0 stands for d = 1.
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994.)  One scalar multiply instead of a division sequence.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t m) { return m ? __umulhi(n, m) : n; }

// Small per-lane quotients: q = (n m) >> 20 with m = ceil(2^20 / d) (magic_div20),
// exact for n < 2^20 / d; with n < 4096 the 24-bit product fits 32 bits.
__device__ __forceinline__ int div_small(int n, int m20) { return (int)(__umul24((uint32_t)n, (uint32_t)m20) >> 20); }

__device__ __forceinline__ TileIdx tile_of(int item, int H, uint32_t mg_h, int nsplit, uint32_t mg_nsplit) {
    TileIdx t;
    const int bh = (int)div_magic((uint32_t)item, mg_nsplit);
    t.sp = item - bh * nsplit;
    t.b = (int)div_magic((uint32_t)bh, mg_h);
    t.h = bh - t.b * H;
    return t;
}

// An offset every lane of the wave holds the same value of, moved to scalar
// registers: a load or store at base + this offset + a per-lane offset then
// takes the scalar-base form (one VGPR for the lane's 32-bit offset) instead
// of a 64-bit VGPR address per access.
// This lane's index in its wave, computed afresh: a value the compiler cannot
// merge with an earlier threadIdx-based copy, so that copy need not stay live.
__device__ __forceinline__ int lane_id()
{
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ size_t wave_uniform(size_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((size_t)hi << 32) | lo;
}

// Lane `lane`'s 16 bytes of 1 KiB block `blk` of a strip whose first block
// starts at element `first` of `ck` (elements of type T, E per block).  Each run
// of four blocks gets its own wave-uniform base, so every access is a scalar
// base + the lane's 32-bit offset + an immediate below 4 KiB.
template <int E, class T>
__device__ __forceinline__ T* strip_block(T* ck, size_t first, int blk, int lane)
{
    return ck + wave_uniform(first + (size_t)(blk >> 2) * 4 * E) + (blk & 3) * E + lane * (E / 64);
}

__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 product, fp32 accumulation.  Operands: lane l holds row (A) or
// column (B) l%16 and eight k values; A and B lanes of one lane group must hold
// the same k values in the same order (which eight is the caller's choice: the
// sum over k does not depend on it).  Result: rows 4(l/16)..+3 of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x as hi + mid + lo, each a bf16 number rounded to nearest even from what the
// terms before it leave: 24 significant bits in all, so the three terms carry x
// up to a relative 2^-24 or so (each difference is exact in fp32).
__device__ __forceinline__ void split3_bf16(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo)
{
    hi = f32_to_bf16_bits(x);
    const float r1 = x - bf16_bits_to_f32((uint16_t)hi);
    mid = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32((uint16_t)mid);
    lo = f32_to_bf16_bits(r2);
}

// Eight bf16 codes (low halves of w0..w7) as one MFMA operand, w0 first.
__device__ __forceinline__ bf16x8 bf16x8_pack(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t w4,
                                              uint32_t w5, uint32_t w6, uint32_t w7)
{
    const u32x4 w = {w0 | (w1 << 16), w2 | (w3 << 16), w4 | (w5 << 16), w6 | (w7 << 16)};
    return __builtin_bit_cast(bf16x8, w);
}

// Eight fp32 values that are bf16 numbers (bf16 inputs widened, E4M3 values) as
// bf16: the upper half of each is its bf16 code, so the conversion is exact.
__device__ __forceinline__ bf16x8 bf16x8_exact(f32x4 lo, f32x4 hi)
{
    const u32x4 l = __builtin_bit_cast(u32x4, lo), h = __builtin_bit_cast(u32x4, hi);
    const u32x4 w = {(l.x >> 16) | (l.y & 0xffff0000u), (l.z >> 16) | (l.w & 0xffff0000u),
                     (h.x >> 16) | (h.y & 0xffff0000u), (h.z >> 16) | (h.w & 0xffff0000u)};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// EL consecutive floats of LDS to registers and back (16-byte accesses when EL
// is a multiple of 4; p then 16-byte aligned).
template <int EL>
__device__ __forceinline__ void lds_row_load(const float* p, float (&v)[EL]) {
    if constexpr (EL % 4 == 0) {
#pragma unroll
        for (int m = 0; m < EL; m += 4) {
            const f32x4 t = ld4(p + m);
            v[m] = t.x; v[m + 1] = t.y; v[m + 2] = t.z; v[m + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int m = 0; m < EL; ++m) v[m] = p[m];
    }
}
template <int EL>
__device__ __forceinline__ void lds_row_store(float* p, const float (&v)[EL]) {
    if constexpr (EL % 4 == 0) {
#pragma unroll
        for (int m = 0; m < EL; m += 4) st4(p + m, f32x4{v[m], v[m + 1], v[m + 2], v[m + 3]});
    } else {
#pragma unroll
        for (int m = 0; m < EL; ++m) p[m] = v[m];
    }
}

// Nontemporal 128-bit global load/store for the checkpoint stream.
__device__ __forceinline__ f32x4 ld4_stream(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st4_stream(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

}  // namespace rs
