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

// ---- scalar conversions -------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
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

// Sum over the four lanes that share (lane % 16): lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float sum_over_row_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
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

__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Nontemporal 128-bit global load/store for the checkpoint stream.
__device__ __forceinline__ f32x4 ld4_stream(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st4_stream(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

}  // namespace rs
