// ckpt.hpp -- fragment-ordered checkpoint strips in fp32 or fp16 storage.
//
// A strip is the 16-column slice of a (b, h) tile that one wave owns: NB
// 16x16 blocks along the reduction axis, lane l holding rows 4(l/16)..+3 of
// column l%16 of every block (the v_mfma_f32_16x16x4_f32 accumulator layout,
// common.hpp).  Storage:
//   fp32  one 16-byte word per block and lane at float4 index
//         (strip*NB + nb)*64 + lane;
//   fp16  blocks 2p and 2p+1 share one 16-byte word per lane (4 halves each)
//         at 16-byte index (strip*NB/2 + p)*64 + lane; a one-block strip
//         (NB = 1) uses an 8-byte word per lane at index strip*64 + lane.
// Either way a wave moves a strip as contiguous 1 KiB rows of 128-bit words
// (512 B rows for NB = 1 in fp16).  Values are fp32 in registers; an fp16
// store rounds to nearest even.
#pragma once
#include "common.hpp"
#include "internal.hpp"
#include "rc.hpp"

namespace rs {

typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 h4_to_f32(u32x2 u) {
    return __builtin_convertvector(__builtin_bit_cast(h16x4, u), f32x4);
}
__device__ __forceinline__ u32x2 f32_to_h4(f32x4 v) {
    return __builtin_bit_cast(u32x2, __builtin_convertvector(v, h16x4));
}

// Issuing a strip's loads and decoding them are separate steps, so the wave
// keeps working (on LDS data) while the loads are in flight and waits only
// where the values are first needed.  The loaded words land in the state
// registers themselves (fp16: the word of blocks 2q and 2q+1 in s[2q]) and
// are decoded in place, so a step that may take either of two sources (the
// checkpoint or its read copy) holds one set of registers.
template <int NB, int CK>
__device__ __forceinline__ void ckpt_issue(const void* ck, size_t strip, int lane, f32x4 (&s)[NB])
{
    if constexpr (CK == CK_FP8) {
        uint32_t w[NB];
        rc_fp8_issue<NB>(static_cast<const uint8_t*>(ck), strip, lane, w);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb].x = __builtin_bit_cast(float, w[nb]);
    } else if constexpr (CK == CK_F32) {
        const float* p = static_cast<const float*>(ck);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb] = ld4_stream(strip_block<256>(p, strip * NB * 256, nb, lane));
    } else if constexpr (NB == 1) {
        const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(ck) + strip * 64 + lane);
        s[0] = __builtin_bit_cast(f32x4, u32x4{v.x, v.y, 0u, 0u});
    } else {
        const u32x4* p = static_cast<const u32x4*>(ck);
#pragma unroll
        for (int q = 0; q < NB / 2; ++q)
            s[2 * q] = __builtin_bit_cast(f32x4, __builtin_nontemporal_load(strip_block<64>(p, strip * (NB / 2) * 64, q, lane)));
    }
}

template <int NB, int CK>
__device__ __forceinline__ void ckpt_decode(f32x4 (&s)[NB])
{
    if constexpr (CK == CK_FP8) {
        uint32_t w[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float x = s[nb].x;                 // a vector component is bit-cast through a scalar
            w[nb] = __builtin_bit_cast(uint32_t, x);
        }
        rc_fp8_decode<NB>(w, s);
    } else if constexpr (CK == CK_F16) {
        if constexpr (NB == 1) {
            const u32x4 w = __builtin_bit_cast(u32x4, s[0]);
            s[0] = h4_to_f32(u32x2{w.x, w.y});
        } else {
#pragma unroll
            for (int q = 0; q < NB / 2; ++q) {
                const u32x4 w = __builtin_bit_cast(u32x4, s[2 * q]);
                s[2 * q] = h4_to_f32(u32x2{w.x, w.y});
                s[2 * q + 1] = h4_to_f32(u32x2{w.z, w.w});
            }
        }
    }
}

template <int NB, int CK>
__device__ __forceinline__ void ckpt_load(const void* ck, size_t strip, int lane, f32x4 (&s)[NB])
{
    if constexpr (CK == CK_FP8) {
        ckpt_issue<NB, CK>(ck, strip, lane, s);
        ckpt_decode<NB, CK>(s);
    } else if constexpr (CK == CK_F32) {
        const float* p = static_cast<const float*>(ck);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb] = ld4_stream(strip_block<256>(p, strip * NB * 256, nb, lane));
    } else if constexpr (NB == 1) {
        const u32x2* p = static_cast<const u32x2*>(ck) + strip * 64 + lane;
        s[0] = h4_to_f32(__builtin_nontemporal_load(p));
    } else {
        const u32x4* p = static_cast<const u32x4*>(ck);
#pragma unroll
        for (int q = 0; q < NB / 2; ++q) {
            const u32x4 w = __builtin_nontemporal_load(strip_block<64>(p, strip * (NB / 2) * 64, q, lane));
            s[2 * q] = h4_to_f32(u32x2{w.x, w.y});
            s[2 * q + 1] = h4_to_f32(u32x2{w.z, w.w});
        }
    }
}

template <int NB, int CK>
__device__ __forceinline__ void ckpt_store(void* ck, size_t strip, int lane, const f32x4 (&s)[NB])
{
    if constexpr (CK == CK_FP8) {
        rc_fp8_store<NB>(static_cast<uint8_t*>(ck), strip, lane, s);
    } else if constexpr (CK == CK_F32) {
        float* p = static_cast<float*>(ck);
        const int ln = lane_id();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) st4_stream(strip_block<256>(p, strip * NB * 256, nb, ln), s[nb]);
    } else if constexpr (NB == 1) {
        u32x2* p = static_cast<u32x2*>(ck) + strip * 64 + lane;
        __builtin_nontemporal_store(f32_to_h4(s[0]), p);
    } else {
        u32x4* p = static_cast<u32x4*>(ck);
        const int ln = lane_id();
#pragma unroll
        for (int q = 0; q < NB / 2; ++q) {
            const u32x2 lo = f32_to_h4(s[2 * q]), hi = f32_to_h4(s[2 * q + 1]);
            __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y}, strip_block<64>(p, strip * (NB / 2) * 64, q, ln));
        }
    }
}

// Dot product of a strip's checkpoint values with per-block read-out vectors
// (sum over nb of s[nb] . c[nb]), decoding the words ckpt_issue left in the
// registers on the fly (no decoded strip is formed; fp32 is used as loaded).
template <int NB, int CK>
__device__ __forceinline__ float ckpt_dot(const f32x4 (&s)[NB], const f32x4 (&c)[NB])
{
    float acc = 0.f;
    if constexpr (CK == CK_FP8) {
        acc = rc_dot<NB, RC_FP8>(s, c);
    } else if constexpr (CK == CK_F32) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc += dot4(s[nb], c[nb]);
    } else if constexpr (NB == 1) {
        const u32x4 w = __builtin_bit_cast(u32x4, s[0]);
        acc = dot4(h4_to_f32(u32x2{w.x, w.y}), c[0]);
    } else {
#pragma unroll
        for (int q = 0; q < NB / 2; ++q) {
            const u32x4 w = __builtin_bit_cast(u32x4, s[2 * q]);
            acc += dot4(h4_to_f32(u32x2{w.x, w.y}), c[2 * q]) + dot4(h4_to_f32(u32x2{w.z, w.w}), c[2 * q + 1]);
        }
    }
    return acc;
}

// Block jb of a strip as fp32, from the words ckpt_issue left in the registers
// (fp32 as loaded): lets a fold read the checkpoint twice without keeping a
// decoded copy of the strip.
template <int NB, int CK>
__device__ __forceinline__ f32x4 ckpt_block(const f32x4 (&s)[NB], int jb)
{
    if constexpr (CK == CK_FP8) {
        const uint32_t w = __builtin_bit_cast(uint32_t, s[jb].x);
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        return f32x4{lo[0], lo[1], hi[0], hi[1]};
    } else if constexpr (CK == CK_F16) {
        const u32x4 w = __builtin_bit_cast(u32x4, s[NB == 1 ? 0 : jb & ~1]);
        return (jb & 1) ? h4_to_f32(u32x2{w.z, w.w}) : h4_to_f32(u32x2{w.x, w.y});
    } else {
        return s[jb];
    }
}

// Registers -> the values the store will keep (identity for fp32).
template <int NB, int CK>
__device__ __forceinline__ void ckpt_round(f32x4 (&s)[NB])
{
    if constexpr (CK == CK_FP8) {
        rc_fp8_roundtrip<NB>(s);
    } else if constexpr (CK == CK_F16) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb] = h4_to_f32(f32_to_h4(s[nb]));
    }
}

// Element offset of the first of the 4 values of lane-block q, q = (strip*NB +
// nb)*64 + lane (the fp32 float4 index), in the storage of checkpoint dtype CK.
template <int CK>
__device__ __forceinline__ size_t ckpt_elem_offset(size_t q, int NB)
{
    if (CK == CK_FP8) {                             // bytes, in the FP8 read-copy layout
        const size_t lane = q & 63, sb = q >> 6;
        const size_t strip = sb / NB;
        const int nb = (int)(sb - strip * NB);
        const size_t bpl = 4 * (size_t)NB;
        if (bpl >= 16) return strip * 64 * bpl + (size_t)(nb / 4) * 1024 + lane * 16 + (nb % 4) * 4;
        return strip * 64 * bpl + lane * bpl + (size_t)nb * 4;
    }
    if (CK == CK_F32 || NB == 1) return q * 4;
    const size_t lane = q & 63, sb = q >> 6;       // sb = strip*NB + nb
    const size_t strip = sb / NB;
    const int nb = (int)(sb - strip * NB);
    return ((strip * (NB / 2) + nb / 2) * 64 + lane) * 8 + (nb & 1) * 4;
}

}  // namespace rs
