// rc.hpp -- the low-precision read copy of the checkpoint.
//
// The recurrence keeps its fp32 checkpoint; a copy in FP8 E4M3 or MXFP4 (E2M1
// elements, one E8M0 scale per 32 elements along the reduction axis) serves
// the reads of non-flush steps, and is refreshed whenever the checkpoint is
// written.  The fold never reads it, so its rounding error never enters the
// recurrence ([TR] "NVIDIA ve Dao AI Lab ...", section "Kuantizasyon
// hatasinin sinirlandirilmasi").  Formats: OCP Microscaling v1.0.
//
// Layout, per (tile, 16-column strip), in the lane order of the fp32
// fragment tiles (common.hpp): lane l holds, per 16x16 block nb, the four
// values of rows 4*(l/16)..+3 of column l%16.
//   FP8    4*NB bytes per lane; byte (nb%4)*4 + r of 16-byte chunk nb/4,
//          chunks stored [chunk][lane][16 B] (narrower tiles: [lane][4*NB B]).
//   MXFP4  2*NB bytes per lane; nibble (nb%8)*4 + r of 16-byte chunk nb/8,
//          low nibble first, chunks [chunk][lane][16 B] (narrower: [lane][2*NB B]).
//          The 32-element groups are block pairs (2s, 2s+1) of one column: the
//          8 values of each of the four lanes l%16 + 16*q.  Scales: byte
//          [tile][strip][l%16][s].
// Quantization rounds to nearest, ties to the even code, and saturates
// (FP8 at +-448, E2M1 at 6); the shared exponent is floor(log2(amax)) - 2,
// clamped to [-127, 127], and an all-zero group uses -127.
#pragma once
#include "common.hpp"

namespace rs {

// ---- FP8 E4M3 ------------------------------------------------------------
// gfx950's v_cvt_pk_fp8_f32 rounds to the nearest OCP E4M3 value (ties to
// even, subnormals included) but does not saturate here, so magnitudes of 448
// and above (infinities too) are clamped to 448 first.  It writes NaN as 0xff;
// the byte fix-up below makes every NaN the code 0x7f.
__device__ __forceinline__ float e4m3_sat(float x)
{
    return __builtin_fabsf(x) >= 448.f ? __builtin_copysignf(448.f, x) : x;
}

__device__ __forceinline__ uint32_t pack_e4m3(f32x4 v)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(v.x), e4m3_sat(v.y), 0, false);      // bytes 0, 1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(v.z), e4m3_sat(v.w), w, true);           // bytes 2, 3
    // bytes whose low seven bits are all ones are NaN: clear their sign bit (no carry
    // crosses a byte: each masked byte is at most 0x7f before the +1)
    const uint32_t t = (uint32_t)w & 0x7f7f7f7fu;
    return (uint32_t)w & ~((t + 0x01010101u) & 0x80808080u);
}

// ---- FP4 E2M1 and the E8M0 shared exponent --------------------------------
// Shared exponent X of a group with largest magnitude amax.  Default rule:
// floor(log2 amax) minus E2M1's largest exponent (2), so amax / 2^X lies in
// [4, 8) and the top of that range saturates at 6.  Non-clipping rule (ceil):
// one step more when amax / 2^X > 6, i.e. when amax's significand exceeds 1.5,
// which makes X the smallest exponent with amax <= 6 * 2^X.
__device__ __forceinline__ int mx_exponent(float amax, bool ceil)
{
    const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
    const uint32_t ebits = (bits >> 23) & 0xffu;
    if (ebits == 0) return -127;                                 // zero or subnormal amax
    const int X = (int)ebits - 127 - 2 + ((ceil && (bits & 0x7fffffu) > 0x400000u) ? 1 : 0);
    return X < -127 ? -127 : (X > 127 ? 127 : X);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t code)
{
    return code == 0 ? __builtin_bit_cast(float, 0x00400000u) : __builtin_bit_cast(float, code << 23);
}

// Eight E2M1 codes of v[k] / 2^X, v[0] in the low nibble.  gfx950's scaled
// conversion divides by the scale it is given, rounds to the nearest E2M1
// value with ties to even and saturates at 6; the scale is passed as the
// group's E8M0 value 2^X (2^-127 as the subnormal float for X = -127).
__device__ __forceinline__ uint32_t pack_e2m1(const float (&v)[8], int X)
{
    const float scale = e8m0_to_f32((uint32_t)(X + 127));
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
    return w;
}

// ---- tile addressing --------------------------------------------------------
template <int NB>
struct RcLayout {
    static constexpr int FP8_BYTES = 4 * NB;     // per lane per strip
    static constexpr int FP4_BYTES = 2 * NB;
};

// byte offset of lane `lane`'s data for chunk q of (tile, strip)
template <int BYTES_PER_LANE>
__device__ __forceinline__ size_t rc_offset(size_t strip_index, int q, int lane)
{
    if constexpr (BYTES_PER_LANE >= 16)
        return strip_index * (64 * BYTES_PER_LANE) + (size_t)q * 1024 + (size_t)lane * 16;
    else
        return strip_index * (64 * BYTES_PER_LANE) + (size_t)lane * BYTES_PER_LANE;
}

// ---- FP8: load + dequantize, quantize + store ---------------------------------
// Loads are issued into raw words and decoded where the values are needed, so
// the wave can work on other data while they are in flight.
template <int NB>
__device__ __forceinline__ void rc_fp8_issue(const uint8_t* base, size_t strip_index, int lane, uint32_t (&w)[NB])
{
    constexpr int BPL = 4 * NB;
    if constexpr (BPL >= 16) {
#pragma unroll
        for (int q = 0; q < NB / 4; ++q) {
            const u32x4 v = __builtin_nontemporal_load(strip_block<64>(reinterpret_cast<const u32x4*>(base), strip_index * 4 * BPL, q, lane));
            w[q * 4] = v.x; w[q * 4 + 1] = v.y; w[q * 4 + 2] = v.z; w[q * 4 + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            w[nb] = *reinterpret_cast<const uint32_t*>(base + rc_offset<BPL>(strip_index, 0, lane) + 4 * nb);
    }
}

template <int NB>
__device__ __forceinline__ void rc_fp8_decode(const uint32_t (&w)[NB], f32x4 (&s)[NB])
{
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[nb], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[nb], true);
        s[nb] = f32x4{lo[0], lo[1], hi[0], hi[1]};
    }
}

template <int NB>
__device__ __forceinline__ void rc_fp8_store(uint8_t* base, size_t strip_index, int lane, const f32x4 (&s)[NB])
{
    constexpr int BPL = 4 * NB;
    if constexpr (BPL >= 16) {
#pragma unroll
        for (int q = 0; q < NB / 4; ++q) {
            const u32x4 v = {pack_e4m3(s[q * 4]), pack_e4m3(s[q * 4 + 1]), pack_e4m3(s[q * 4 + 2]), pack_e4m3(s[q * 4 + 3])};
            __builtin_nontemporal_store(v, strip_block<64>(reinterpret_cast<u32x4*>(base), strip_index * 4 * BPL, q, lane_id()));
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<uint32_t*>(base + rc_offset<BPL>(strip_index, 0, lane) + 4 * nb) = pack_e4m3(s[nb]);
    }
}

// ---- MXFP4: load + dequantize, quantize + store --------------------------------
template <int NB>
__device__ __forceinline__ void rc_fp4_issue(const uint8_t* codes, const uint8_t* scales, size_t strip_index, int lane,
                                             uint32_t (&w)[NB / 2], uint32_t (&sc)[NB / 2])
{
    static_assert(NB % 2 == 0, "MXFP4 groups need block pairs");
    constexpr int BPL = 2 * NB;
    constexpr int NP = NB / 2;                       // groups (block pairs) per lane
    if constexpr (BPL >= 16) {
#pragma unroll
        for (int q = 0; q < NB / 8; ++q) {
            const u32x4 v = __builtin_nontemporal_load(strip_block<64>(reinterpret_cast<const u32x4*>(codes), strip_index * 4 * BPL, q, lane));
            w[q * 4] = v.x; w[q * 4 + 1] = v.y; w[q * 4 + 2] = v.z; w[q * 4 + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int p = 0; p < NP; ++p)
            w[p] = *reinterpret_cast<const uint32_t*>(codes + rc_offset<BPL>(strip_index, 0, lane) + 4 * p);
    }
    // the NP scale bytes of the lane's column are contiguous: one load
    const uint8_t* scp = scales + (strip_index * 16 + (lane & 15)) * NP;
    if constexpr (NP == 4) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(scp);
#pragma unroll
        for (int p = 0; p < NP; ++p) sc[p] = (v >> (8 * p)) & 0xffu;
    } else if constexpr (NP == 8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(scp);
#pragma unroll
        for (int p = 0; p < NP; ++p) sc[p] = ((p < 4 ? v.x : v.y) >> (8 * (p & 3))) & 0xffu;
    } else {
#pragma unroll
        for (int p = 0; p < NP; ++p) sc[p] = scp[p];
    }
}

template <int NB>
__device__ __forceinline__ void rc_fp4_decode(const uint32_t (&w)[NB / 2], const uint32_t (&sc)[NB / 2], f32x4 (&s)[NB])
{
#pragma unroll
    for (int p = 0; p < NB / 2; ++p) {
        const float scale = e8m0_to_f32(sc[p]);
        const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], scale, 0);
        const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], scale, 1);
        const auto b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], scale, 2);
        const auto b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], scale, 3);
        s[2 * p] = f32x4{b0[0], b0[1], b1[0], b1[1]};
        s[2 * p + 1] = f32x4{b2[0], b2[1], b3[0], b3[1]};
    }
}

template <int NB>
__device__ __forceinline__ void rc_fp4_store(uint8_t* codes, uint8_t* scales, size_t strip_index, int lane,
                                             const f32x4 (&s)[NB], bool ceil)
{
    static_assert(NB % 2 == 0, "MXFP4 groups need block pairs");
    constexpr int BPL = 2 * NB;
    constexpr int NP = NB / 2;
    uint32_t w[NP];
    uint32_t scw[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const f32x4 a = s[2 * p], b = s[2 * p + 1];
        float am = fmaxf(fmaxf(fmaxf(__builtin_fabsf(a.x), __builtin_fabsf(a.y)), fmaxf(__builtin_fabsf(a.z), __builtin_fabsf(a.w))),
                         fmaxf(fmaxf(__builtin_fabsf(b.x), __builtin_fabsf(b.y)), fmaxf(__builtin_fabsf(b.z), __builtin_fabsf(b.w))));
        am = max_over_row_groups(am);                // the group spans lanes l%16 + 16*q
        const int X = mx_exponent(am, ceil);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        w[p] = pack_e2m1(v, X);
        scw[p] = (uint32_t)(X + 127);
    }
    if constexpr (BPL >= 16) {
#pragma unroll
        for (int q = 0; q < NB / 8; ++q) {
            const u32x4 v = {w[q * 4], w[q * 4 + 1], w[q * 4 + 2], w[q * 4 + 3]};
            __builtin_nontemporal_store(v, strip_block<64>(reinterpret_cast<u32x4*>(codes), strip_index * 4 * BPL, q, lane_id()));
        }
    } else {
#pragma unroll
        for (int p = 0; p < NP; ++p)
            *reinterpret_cast<uint32_t*>(codes + rc_offset<BPL>(strip_index, 0, lane) + 4 * p) = w[p];
    }
    if (lane < 16) {
        uint8_t* sc = scales + (strip_index * 16 + lane) * NP;
#pragma unroll
        for (int p = 0; p < NP; ++p) sc[p] = (uint8_t)scw[p];
    }
}

// Round a strip's registers to the copy's grid (quantize, then dequantize),
// used when the checkpoint itself is kept at the copy's precision.
template <int NB>
__device__ __forceinline__ void rc_fp8_roundtrip(f32x4 (&s)[NB])
{
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const uint32_t w = pack_e4m3(s[nb]);
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        s[nb] = f32x4{lo[0], lo[1], hi[0], hi[1]};
    }
}

template <int NB>
__device__ __forceinline__ void rc_fp4_roundtrip(f32x4 (&s)[NB], bool ceil)
{
    static_assert(NB % 2 == 0, "MXFP4 groups need block pairs");
#pragma unroll
    for (int p = 0; p < NB / 2; ++p) {
        const f32x4 a = s[2 * p], b = s[2 * p + 1];
        float am = fmaxf(fmaxf(fmaxf(__builtin_fabsf(a.x), __builtin_fabsf(a.y)), fmaxf(__builtin_fabsf(a.z), __builtin_fabsf(a.w))),
                         fmaxf(fmaxf(__builtin_fabsf(b.x), __builtin_fabsf(b.y)), fmaxf(__builtin_fabsf(b.z), __builtin_fabsf(b.w))));
        am = max_over_row_groups(am);
        const int X = mx_exponent(am, ceil);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        const uint32_t word = pack_e2m1(v, X);
        const float scale = e8m0_to_f32((uint32_t)(X + 127));
        const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 0);
        const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 1);
        const auto b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 2);
        const auto b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 3);
        s[2 * p] = f32x4{b0[0], b0[1], b1[0], b1[1]};
        s[2 * p + 1] = f32x4{b2[0], b2[1], b3[0], b3[1]};
    }
}

template <int NB, int RC>
__device__ __forceinline__ void rc_roundtrip(f32x4 (&s)[NB], bool mx_ceil)
{
    if constexpr (RC == RC_FP8) rc_fp8_roundtrip<NB>(s);
    else if constexpr (RC == RC_MXFP4) rc_fp4_roundtrip<NB>(s, mx_ceil);
}

// Refresh the read copy of one strip from its fp32 registers.
template <int NB, int RC>
__device__ __forceinline__ void rc_store(uint8_t* codes, uint8_t* scales, size_t strip_index, int lane, const f32x4 (&s)[NB],
                                         bool mx_ceil)
{
    if constexpr (RC == RC_FP8) rc_fp8_store<NB>(codes, strip_index, lane, s);
    else if constexpr (RC == RC_MXFP4) rc_fp4_store<NB>(codes, scales, strip_index, lane, s, mx_ceil);
}

// Read-copy words of a strip, issued into the state registers (fp8: the word
// of block nb in s[nb].x; MXFP4: the codes of group p in s[2p].x and its
// scale in s[2p].y) and decoded in place where first needed.
template <int NB, int RC>
__device__ __forceinline__ void rc_issue(const uint8_t* codes, const uint8_t* scales, size_t strip_index, int lane,
                                         f32x4 (&s)[NB])
{
    if constexpr (RC == RC_FP8) {
        uint32_t w[NB];
        rc_fp8_issue<NB>(codes, strip_index, lane, w);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb].x = __builtin_bit_cast(float, w[nb]);
    } else if constexpr (RC == RC_MXFP4) {
        uint32_t w[NB / 2], sc[NB / 2];
        rc_fp4_issue<NB>(codes, scales, strip_index, lane, w, sc);
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
            s[2 * p].x = __builtin_bit_cast(float, w[p]);
            s[2 * p].y = __builtin_bit_cast(float, sc[p]);
        }
    }
}

template <int NB, int RC>
__device__ __forceinline__ void rc_decode(f32x4 (&s)[NB])
{
    if constexpr (RC == RC_FP8) {
        uint32_t w[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float x = s[nb].x;                 // bit_cast of a vector component goes through a scalar
            w[nb] = __builtin_bit_cast(uint32_t, x);
        }
        rc_fp8_decode<NB>(w, s);
    } else if constexpr (RC == RC_MXFP4) {
        uint32_t w[NB / 2], sc[NB / 2];
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
            const float x = s[2 * p].x, y = s[2 * p].y;   // via scalars (see above)
            w[p] = __builtin_bit_cast(uint32_t, x);
            sc[p] = __builtin_bit_cast(uint32_t, y);
        }
        rc_fp4_decode<NB>(w, sc, s);
    }
}

// Dot product of a strip's read-copy values with per-block read-out vectors:
// sum over nb of s[nb] . c[nb], the words decoded on the fly from the registers
// rc_issue filled (no decoded strip is formed).  MXFP4: the group scale, a power
// of two, multiplies the group's partial dot once.
template <int NB, int RC>
__device__ __forceinline__ float rc_dot(const f32x4 (&s)[NB], const f32x4 (&c)[NB])
{
    float acc = 0.f;
    if constexpr (RC == RC_FP8) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float x = s[nb].x;
            const uint32_t w = __builtin_bit_cast(uint32_t, x);
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
            acc += lo[0] * c[nb].x + lo[1] * c[nb].y + hi[0] * c[nb].z + hi[1] * c[nb].w;
        }
    } else if constexpr (RC == RC_MXFP4) {
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
            const float x = s[2 * p].x, y = s[2 * p].y;
            const uint32_t w = __builtin_bit_cast(uint32_t, x);
            const float scale = e8m0_to_f32(__builtin_bit_cast(uint32_t, y));
            const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 0);
            const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 1);
            const auto b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 2);
            const auto b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 3);
            const float g = b0[0] * c[2 * p].x + b0[1] * c[2 * p].y + b1[0] * c[2 * p].z + b1[1] * c[2 * p].w +
                            b2[0] * c[2 * p + 1].x + b2[1] * c[2 * p + 1].y + b3[0] * c[2 * p + 1].z +
                            b3[1] * c[2 * p + 1].w;
            acc += scale * g;
        }
    }
    return acc;
}

// A strip's low-precision words as loaded, kept compact (no decoded registers):
// FMT 0 the NB FP8 words (an FP8 read copy, or an FP8 checkpoint, which uses the
// same layout); FMT 1 the NB/2 MXFP4 code words followed by their NB/2 scales.
template <int NB, int FMT>
__device__ __forceinline__ void raw_issue(const uint8_t* codes, const uint8_t* scales, size_t strip_index, int lane,
                                          uint32_t (&w)[NB])
{
    if constexpr (FMT == 0) {
        rc_fp8_issue<NB>(codes, strip_index, lane, w);
    } else {
        uint32_t c[NB / 2], sc[NB / 2];
        rc_fp4_issue<NB>(codes, scales, strip_index, lane, c, sc);
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
            w[p] = c[p];
            w[NB / 2 + p] = sc[p];
        }
    }
}

// sum over nb of (strip block nb) . c[nb] from compact words (rc_dot's arithmetic)
template <int NB, int FMT>
__device__ __forceinline__ float raw_dot(const uint32_t (&w)[NB], const f32x4 (&c)[NB])
{
    float acc = 0.f;
    if constexpr (FMT == 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[nb], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[nb], true);
            acc += lo[0] * c[nb].x + lo[1] * c[nb].y + hi[0] * c[nb].z + hi[1] * c[nb].w;
        }
    } else {
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
            const float scale = e8m0_to_f32(w[NB / 2 + p]);
            const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.f, 0);
            const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.f, 1);
            const auto b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.f, 2);
            const auto b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.f, 3);
            const float g = b0[0] * c[2 * p].x + b0[1] * c[2 * p].y + b1[0] * c[2 * p].z + b1[1] * c[2 * p].w +
                            b2[0] * c[2 * p + 1].x + b2[1] * c[2 * p + 1].y + b3[0] * c[2 * p + 1].z +
                            b3[1] * c[2 * p + 1].w;
            acc += scale * g;
        }
    }
    return acc;
}

}  // namespace rs
