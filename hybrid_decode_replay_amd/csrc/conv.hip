// conv.hip -- conventional fused decode, the in-run baseline.
//
// Ordinary decoding: per token and (b, h), load the state, decay and update
// it, read out the output, store the state ([DE] "ReplaySSM beschleunigt das
// Decoding ...", section "Wie es funktioniert" describes this step and why
// it is memory-bound).  The state is the plain logical fp32 tile [C][R]
// (Mamba-2 [P][N], GDN [DV][DK]).  Every row evolves independently given the
// token, so a thread owns one float4 of a row: the N/4 lanes of a row are
// adjacent, loads and stores are 128-bit and contiguous across the row, and
// row dot products reduce with lane shuffles.  UNR float4 loads per thread are
// issued before any arithmetic.
//
// Speculative variant (the snapshot baseline): the state is read once, k
// draft tokens advance it in registers, and the state after draft j is
// written to snapshot j together with the draft's output; restoring copies
// snapshot a-1 into the state.
#include "common.hpp"
#include "internal.hpp"

namespace rs {

template <int N4>
__device__ __forceinline__ float row_sum(float v) {
    return group_sum<N4>(v);     // the N4 adjacent lanes of a row, by DPP
}

template <int IO>
__device__ __forceinline__ f32x4 ld4_io(const void* p, size_t i) {
    if constexpr (IO == IO_F32) return ld4(static_cast<const float*>(p) + i);
    else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return f32x4{bf16_bits_to_f32((uint16_t)(u.x & 0xffff)), bf16_bits_to_f32((uint16_t)(u.x >> 16)),
                     bf16_bits_to_f32((uint16_t)(u.y & 0xffff)), bf16_bits_to_f32((uint16_t)(u.y >> 16))};
    }
}

constexpr int CONV_THREADS = 256;
constexpr int CONV_UNR = 8;

template <int N4, int IO, int KIND, bool SPEC>
__global__ __launch_bounds__(CONV_THREADS) void conv_step_kernel(ConvArgs a)
{
    constexpr int RP = CONV_THREADS / N4;   // rows per pass
    const int tile = xcd_tile_index();
    const int b = tile / a.H, h = tile - b * a.H;
    const int g = h / a.hpg;
    const int tid = threadIdx.x;
    const int q = tid % N4, r0 = tid / N4;
    const int C = a.C, R = N4 * 4;
    const size_t tile_elems = (size_t)C * R;
    const size_t sB = (size_t)a.B;
    const float* src = (SPEC ? a.S_in : a.S) + (size_t)tile * tile_elems;
    float* dst = a.S + (size_t)tile * tile_elems;
    const int passes = (C + RP - 1) / RP;

    for (int p0 = 0; p0 < passes; p0 += CONV_UNR) {
        f32x4 s[CONV_UNR];
#pragma unroll
        for (int u = 0; u < CONV_UNR; ++u) {
            const int row = (p0 + u) * RP + r0;
            s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p0 + u < passes && row < C) s[u] = ld4_stream(src + (size_t)row * R + 4 * q);
        }
        for (int t = 0; t < a.T; ++t) {
            const size_t tb = (size_t)t * sB + b;
            if constexpr (KIND == 0) {   // Mamba-2
                const float dt = ld_io<IO>(a.in_s0, tb * a.H + h);
                const float decay = expf(dt * a.A[h]);
                const f32x4 Bv = ld4_io<IO>(a.in_r, (tb * a.G + g) * R + 4 * q);
                const f32x4 Cv = ld4_io<IO>(a.in_q, (tb * a.G + g) * R + 4 * q);
                const float Dh = a.D[h];
#pragma unroll
                for (int u = 0; u < CONV_UNR; ++u) {
                    const int row = (p0 + u) * RP + r0;
                    if (p0 + u < passes) {           // uniform across the workgroup
                        const bool live = row < C;
                        const float x = live ? ld_io<IO>(a.in_c, (tb * a.H + h) * C + row) : 0.f;
                        s[u] = decay * s[u] + (dt * x) * Bv;
                        const float yv = row_sum<N4>(dot4(s[u], Cv)) + Dh * x;
                        if (live && q == 0) st_io<IO>(a.y, (tb * a.H + h) * C + row, yv);
                        if (SPEC && live)
                            st4_stream(a.snaps + ((size_t)t * sB * a.H + tile) * tile_elems + (size_t)row * R + 4 * q, s[u]);
                    }
                }
            } else {                      // Gated DeltaNet
                const float al = static_cast<const float*>(a.in_s0)[tb * a.H + h];
                const float be = a.in_s1[tb * a.H + h];
                const f32x4 kv = ld4_io<IO>(a.in_r, (tb * a.G + g) * R + 4 * q);
                const f32x4 qv = ld4_io<IO>(a.in_q, (tb * a.G + g) * R + 4 * q);
#pragma unroll
                for (int u = 0; u < CONV_UNR; ++u) {
                    const int row = (p0 + u) * RP + r0;
                    if (p0 + u < passes) {
                        const bool live = row < C;
                        const float v = live ? ld_io<IO>(a.in_c, (tb * a.H + h) * C + row) : 0.f;
                        const float sk = row_sum<N4>(dot4(s[u], kv));
                        s[u] = al * s[u] + (be * (v - al * sk)) * kv;
                        const float ov = a.scale * row_sum<N4>(dot4(s[u], qv));
                        if (live && q == 0) st_io<IO>(a.y, (tb * a.H + h) * C + row, ov);
                        if (SPEC && live)
                            st4_stream(a.snaps + ((size_t)t * sB * a.H + tile) * tile_elems + (size_t)row * R + 4 * q, s[u]);
                    }
                }
            }
        }
        if (!SPEC) {
#pragma unroll
            for (int u = 0; u < CONV_UNR; ++u) {
                const int row = (p0 + u) * RP + r0;
                if (p0 + u < passes && row < C) st4_stream(dst + (size_t)row * R + 4 * q, s[u]);
            }
        }
    }
}

template <int N4, int IO>
static hipError_t conv_launch_n4(const ConvArgs& a, hipStream_t s)
{
    const bool spec = a.snaps != nullptr;
    dim3 grid(a.B * a.H), block(CONV_THREADS);
    if (a.kind == 0) {
        if (spec) hipLaunchKernelGGL((conv_step_kernel<N4, IO, 0, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv_step_kernel<N4, IO, 0, false>), grid, block, 0, s, a);
    } else {
        if (spec) hipLaunchKernelGGL((conv_step_kernel<N4, IO, 1, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv_step_kernel<N4, IO, 1, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <int IO>
static hipError_t conv_launch_io(const ConvArgs& a, hipStream_t s)
{
    switch (a.R) {
        case 16: return conv_launch_n4<4, IO>(a, s);
        case 32: return conv_launch_n4<8, IO>(a, s);
        case 64: return conv_launch_n4<16, IO>(a, s);
        case 128: return conv_launch_n4<32, IO>(a, s);
        case 256: return conv_launch_n4<64, IO>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_conv_step(const ConvArgs& a, int io, hipStream_t s)
{
    return io == IO_BF16 ? conv_launch_io<IO_BF16>(a, s) : conv_launch_io<IO_F32>(a, s);
}

// S[b][h] = snaps[a-1][b][h] for a = clamp(accepted[b], 0, k) >= 1.
__global__ __launch_bounds__(256) void conv_restore_kernel(float* S, const float* snaps, const int32_t* accepted,
                                                           int B, int H, int k, size_t tile_elems)
{
    const int tile = xcd_tile_index();
    const int b = tile / H;
    int acc = accepted[b];
    acc = acc < 0 ? 0 : (acc > k ? k : acc);
    if (acc == 0) return;
    const float* src = snaps + ((size_t)(acc - 1) * B * H + tile) * tile_elems;
    float* dst = S + (size_t)tile * tile_elems;
    for (size_t i = threadIdx.x; i < tile_elems / 4; i += blockDim.x)
        st4_stream(dst + 4 * i, ld4_stream(src + 4 * i));
}

hipError_t launch_conv_restore(float* S, const float* snaps, const int32_t* accepted, int B, int tile_elems,
                               int H, int k, hipStream_t s)
{
    hipLaunchKernelGGL(conv_restore_kernel, dim3(B * H), dim3(256), 0, s, S, snaps, accepted, B, H, k,
                       (size_t)tile_elems);
    return hipGetLastError();
}

}  // namespace rs
