// conv.hip -- conventional fused decode, the in-run baseline.
//
// Ordinary decoding: per token and (b, h), load the state, decay and update
// it, read out the output, store the state ([DE] "ReplaySSM beschleunigt das
// Decoding ...", section "Wie es funktioniert" describes this step and why
// it is memory-bound).  The state is the plain logical tile [C][R] (Mamba-2
// [P][N], GDN [DV][DK]) in fp32, fp16 or FP8 E4M3; a low-precision state is
// updated in fp32 and rounded (RNE) after every token, and the token's output
// is read from the rounded values, the ones stored: the same order as a
// replayed step that folds (a conventional step is a replayed step with a
// one-entry buffer).  Every row evolves
// independently given the token, so a thread owns one 16-byte word of a row
// (4 fp32, 8 fp16 or 16 FP8 values): the lanes of a row are adjacent, loads and stores
// are 128-bit and contiguous across the row, and row dot products reduce with
// DPP.  UNR = 8 words per thread are loaded before any arithmetic.
//
// Speculative variant (the snapshot baseline): the state is read once, k
// draft tokens advance it in registers, and the state after draft j is
// written to snapshot j together with the draft's output; restoring copies
// snapshot a-1 into the state.
#include "ckpt.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace rs {

template <int IO>
__device__ __forceinline__ f32x4 ld4_io(const void* p, size_t i) {
    if constexpr (IO == IO_F32) return ld4(static_cast<const float*>(p) + i);
    else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return f32x4{bf16_bits_to_f32((uint16_t)(u.x & 0xffff)), bf16_bits_to_f32((uint16_t)(u.x >> 16)),
                     bf16_bits_to_f32((uint16_t)(u.y & 0xffff)), bf16_bits_to_f32((uint16_t)(u.y >> 16))};
    }
}

// A thread's share of a state row: VW groups of 4 consecutive values, one
// 16-byte word of storage (fp32: VW = 1; fp16: VW = 2).
template <int CK>
struct StateWord {
    static constexpr int VW = CK == CK_FP8 ? 4 : (CK == CK_F16 ? 2 : 1);
    static __device__ __forceinline__ void load(const void* base, size_t e, f32x4 (&v)[VW]) {
        if constexpr (CK == CK_F32) {
            v[0] = ld4_stream(static_cast<const float*>(base) + e);
        } else if constexpr (CK == CK_F16) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + e));
            v[0] = h4_to_f32(u32x2{w.x, w.y});
            v[1] = h4_to_f32(u32x2{w.z, w.w});
        } else {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(base) + e));
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(ww[i], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(ww[i], true);
                v[i] = f32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    }
    static __device__ __forceinline__ void store(void* base, size_t e, const f32x4 (&v)[VW]) {
        if constexpr (CK == CK_F32) {
            st4_stream(static_cast<float*>(base) + e, v[0]);
        } else if constexpr (CK == CK_F16) {
            const u32x2 lo = f32_to_h4(v[0]), hi = f32_to_h4(v[1]);
            __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y},
                                        reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + e));
        } else {
            __builtin_nontemporal_store(u32x4{pack_e4m3(v[0]), pack_e4m3(v[1]), pack_e4m3(v[2]), pack_e4m3(v[3])},
                                        reinterpret_cast<u32x4*>(static_cast<uint8_t*>(base) + e));
        }
    }
    static __device__ __forceinline__ void round(f32x4 (&v)[VW]) {
        if constexpr (CK == CK_F16) {
#pragma unroll
            for (int i = 0; i < VW; ++i) v[i] = h4_to_f32(f32_to_h4(v[i]));
        } else if constexpr (CK == CK_FP8) {
#pragma unroll
            for (int i = 0; i < VW; ++i) {
                const uint32_t w = pack_e4m3(v[i]);
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
                v[i] = f32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    }
};

constexpr int CONV_THREADS = 256;
// Row passes a thread holds at once: every storage width keeps 32 fp32 state
// values per thread in registers (fp32: 8 words of 4, fp16: 4 of 8, FP8: 2 of
// 16), which leaves room for seven waves per SIMD.
template <int CK>
constexpr int conv_unroll() { return CK == CK_FP8 ? 2 : (CK == CK_F16 ? 4 : 8); }

template <int R, int IO, int KIND, bool SPEC, int CK>
__global__ __launch_bounds__(CONV_THREADS) void conv_step_kernel(ConvArgs a)
{
    using SW = StateWord<CK>;
    constexpr int VW = SW::VW;
    constexpr int CONV_UNR = conv_unroll<CK>();
    constexpr int EPT = 4 * VW;              // state values per thread and row
    constexpr int NL = R / EPT;              // lanes per row (adjacent)
    constexpr int RP = CONV_THREADS / NL;    // rows per pass
    const int tile = xcd_tile_index();
    const int b = tile / a.H, h = tile - b * a.H;
    const int g = h / a.hpg;
    const int tid = threadIdx.x;
    const int q = tid % NL, r0 = tid / NL;
    const int C = a.C;
    const size_t tile_elems = (size_t)C * R;
    const size_t sB = (size_t)a.B;
    const void* src = SPEC ? a.S_in : a.S;
    const size_t t0 = (size_t)tile * tile_elems;
    const int passes = (C + RP - 1) / RP;

    for (int p0 = 0; p0 < passes; p0 += CONV_UNR) {
        f32x4 s[CONV_UNR][VW];
#pragma unroll
        for (int u = 0; u < CONV_UNR; ++u) {
            const int row = (p0 + u) * RP + r0;
#pragma unroll
            for (int i = 0; i < VW; ++i) s[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p0 + u < passes && row < C) SW::load(src, t0 + (size_t)row * R + EPT * q, s[u]);
        }
        for (int t = 0; t < a.T; ++t) {
            const size_t tb = (size_t)t * sB + b;
            const size_t vrow = (tb * a.G + g) * R + EPT * q;   // B/C (Mamba-2) or k/q (GDN) slice
            f32x4 v1[VW], v2[VW];
#pragma unroll
            for (int i = 0; i < VW; ++i) {
                v1[i] = ld4_io<IO>(a.in_r, vrow + 4 * i);
                v2[i] = ld4_io<IO>(a.in_q, vrow + 4 * i);
            }
            if constexpr (KIND == 0) {   // Mamba-2: v1 = B, v2 = C
                const float dt = ld_io<IO>(a.in_s0, tb * a.H + h);
                const float decay = expf(dt * a.A[h]);
                const float Dh = a.D[h];
#pragma unroll
                for (int u = 0; u < CONV_UNR; ++u) {
                    const int row = (p0 + u) * RP + r0;
                    if (p0 + u < passes) {           // uniform across the workgroup
                        const bool live = row < C;
                        const float x = live ? ld_io<IO>(a.in_c, (tb * a.H + h) * C + row) : 0.f;
#pragma unroll
                        for (int i = 0; i < VW; ++i) s[u][i] = decay * s[u][i] + (dt * x) * v1[i];
                        SW::round(s[u]);
                        float dot = 0.f;
#pragma unroll
                        for (int i = 0; i < VW; ++i) dot += dot4(s[u][i], v2[i]);
                        const float yv = group_sum<NL>(dot) + Dh * x;
                        if (live && q == 0) st_io<IO>(a.y, (tb * a.H + h) * C + row, yv);
                        if (SPEC && live)
                            SW::store(a.snaps, ((size_t)t * sB * a.H + tile) * tile_elems + (size_t)row * R + EPT * q, s[u]);
                    }
                }
            } else {                      // Gated DeltaNet: v1 = k, v2 = q
                const float al = static_cast<const float*>(a.in_s0)[tb * a.H + h];
                const float be = a.in_s1[tb * a.H + h];
#pragma unroll
                for (int u = 0; u < CONV_UNR; ++u) {
                    const int row = (p0 + u) * RP + r0;
                    if (p0 + u < passes) {
                        const bool live = row < C;
                        const float v = live ? ld_io<IO>(a.in_c, (tb * a.H + h) * C + row) : 0.f;
                        float sk = 0.f;
#pragma unroll
                        for (int i = 0; i < VW; ++i) sk += dot4(s[u][i], v1[i]);
                        sk = group_sum<NL>(sk);
                        const float w = be * (v - al * sk);
#pragma unroll
                        for (int i = 0; i < VW; ++i) s[u][i] = al * s[u][i] + w * v1[i];
                        SW::round(s[u]);
                        float ov = 0.f;
#pragma unroll
                        for (int i = 0; i < VW; ++i) ov += dot4(s[u][i], v2[i]);
                        ov = a.scale * group_sum<NL>(ov);
                        if (live && q == 0) st_io<IO>(a.y, (tb * a.H + h) * C + row, ov);
                        if (SPEC && live)
                            SW::store(a.snaps, ((size_t)t * sB * a.H + tile) * tile_elems + (size_t)row * R + EPT * q, s[u]);
                    }
                }
            }
        }
        if (!SPEC) {
#pragma unroll
            for (int u = 0; u < CONV_UNR; ++u) {
                const int row = (p0 + u) * RP + r0;
                if (p0 + u < passes && row < C) SW::store(a.S, t0 + (size_t)row * R + EPT * q, s[u]);
            }
        }
    }
}

template <int R, int IO, int CK>
static hipError_t conv_launch_r(const ConvArgs& a, hipStream_t s)
{
    const bool spec = a.snaps != nullptr;
    dim3 grid(a.B * a.H), block(CONV_THREADS);
    if (a.kind == 0) {
        if (spec) hipLaunchKernelGGL((conv_step_kernel<R, IO, 0, true, CK>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv_step_kernel<R, IO, 0, false, CK>), grid, block, 0, s, a);
    } else {
        if (spec) hipLaunchKernelGGL((conv_step_kernel<R, IO, 1, true, CK>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv_step_kernel<R, IO, 1, false, CK>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <int IO, int CK>
static hipError_t conv_launch_io(const ConvArgs& a, hipStream_t s)
{
    switch (a.R) {
        case 16: return conv_launch_r<16, IO, CK>(a, s);
        case 32: return conv_launch_r<32, IO, CK>(a, s);
        case 64: return conv_launch_r<64, IO, CK>(a, s);
        case 128: return conv_launch_r<128, IO, CK>(a, s);
        case 256: return conv_launch_r<256, IO, CK>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_conv_step(const ConvArgs& a, int io, int ck, hipStream_t s)
{
    if (ck == CK_FP8) return io == IO_BF16 ? conv_launch_io<IO_BF16, CK_FP8>(a, s) : conv_launch_io<IO_F32, CK_FP8>(a, s);
    if (ck == CK_F16) return io == IO_BF16 ? conv_launch_io<IO_BF16, CK_F16>(a, s) : conv_launch_io<IO_F32, CK_F16>(a, s);
    return io == IO_BF16 ? conv_launch_io<IO_BF16, CK_F32>(a, s) : conv_launch_io<IO_F32, CK_F32>(a, s);
}

// S[b][h] = snaps[a-1][b][h] for a = clamp(accepted[b], 0, k) >= 1 (a byte
// copy of one tile, 16 bytes per thread and step).
__global__ __launch_bounds__(256) void conv_restore_kernel(void* S, const void* snaps, const int32_t* accepted,
                                                           int B, int H, int k, size_t tile_bytes)
{
    const int tile = xcd_tile_index();
    const int b = tile / H;
    int acc = accepted[b];
    acc = acc < 0 ? 0 : (acc > k ? k : acc);
    if (acc == 0) return;
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(snaps) +
                                                      ((size_t)(acc - 1) * B * H + tile) * tile_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(S) + (size_t)tile * tile_bytes);
    for (size_t i = threadIdx.x; i < tile_bytes / 16; i += blockDim.x)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_conv_restore(void* S, const void* snaps, const int32_t* accepted, int B, size_t tile_bytes,
                               int H, int k, hipStream_t s)
{
    hipLaunchKernelGGL(conv_restore_kernel, dim3(B * H), dim3(256), 0, s, S, snaps, accepted, B, H, k, tile_bytes);
    return hipGetLastError();
}

}  // namespace rs
