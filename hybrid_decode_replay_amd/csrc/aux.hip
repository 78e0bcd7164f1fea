// aux.hip -- bookkeeping, layout conversion and measurement kernels.
#include "common.hpp"
#include "ckpt.hpp"
#include "internal.hpp"
#include "rc.hpp"

namespace rs {

// ---- bookkeeping ----------------------------------------------------------
// Book layout: int32 [2 copies][4 fields][B]; field 0 = len, 1 = pend, 2 = fc,
// 3 = lim (length of the current window).  Each launch that changes the
// bookkeeping reads copy `parity` and writes copy `parity ^ 1`, so every
// workgroup of a launch sees the same pre-launch values.

// Commit (accepted != null) or rollback (accepted == null): the accepted
// prefix advances the pointer, the rest of the drafts is dropped.
__global__ void book_commit_kernel(int32_t* book, uint32_t* err, int B, int parity, const int32_t* accepted)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int32_t* cur = book + (size_t)parity * 4 * B;
    int32_t* nxt = book + (size_t)(parity ^ 1) * 4 * B;
    const int pend = cur[B + b];
    const int a = accepted ? accepted[b] : 0;
    const int ac = a < 0 ? 0 : (a > pend ? pend : a);
    if (ac != a) atomicOr(err, REPLAY_COMMIT_CLAMPED_BIT);
    nxt[b] = cur[b] + ac;
    nxt[B + b] = 0;
    nxt[2 * B + b] = cur[2 * B + b];
    nxt[3 * B + b] = cur[3 * B + b];
}

// len = pend = fc = 0; lim = cap, or 1 + (b mod cap) for staggered flushes.
__global__ void book_reset_kernel(int32_t* book, uint32_t* err, int B, int parity, int cap, int stagger)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) {
        int32_t* cur = book + (size_t)parity * 4 * B;
        cur[b] = 0;
        cur[B + b] = 0;
        cur[2 * B + b] = 0;
        cur[3 * B + b] = stagger ? 1 + b % cap : cap;
    }
    if (b == 0) *err = 0u;
}

hipError_t launch_book_commit(int32_t* book, uint32_t* err, int B, int parity, const int32_t* accepted,
                              hipStream_t s)
{
    hipLaunchKernelGGL(book_commit_kernel, dim3((B + 255) / 256), dim3(256), 0, s, book, err, B, parity, accepted);
    return hipGetLastError();
}

hipError_t launch_book_reset(int32_t* book, uint32_t* err, int B, int parity, int cap, bool stagger, hipStream_t s)
{
    hipLaunchKernelGGL(book_reset_kernel, dim3((B + 255) / 256), dim3(256), 0, s, book, err, B, parity, cap,
                       stagger ? 1 : 0);
    return hipGetLastError();
}

// A sequence that (re)joins the batch: empty buffer, no drafts, a fresh window
// of cap entries.  Written into the current copy; the other copy is rewritten
// in full by the next launch that changes the bookkeeping.
__global__ void book_reset_slots_kernel(int32_t* book, int B, int parity, int cap, SlotMap m)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= m.n) return;
    const int b = m.slot[i];
    int32_t* cur = book + (size_t)parity * 4 * B;
    cur[b] = 0;
    cur[B + b] = 0;
    cur[2 * B + b] = 0;
    cur[3 * B + b] = cap;
}

hipError_t launch_book_reset_slots(int32_t* book, int B, int parity, int cap, const SlotMap& m, hipStream_t s)
{
    hipLaunchKernelGGL(book_reset_slots_kernel, dim3(1), dim3(SLOT_CHUNK), 0, s, book, B, parity, cap, m);
    return hipGetLastError();
}

// ---- zero fill (a kernel, not a memset, so it is safe under graph capture)
__global__ void fill_zero_kernel(uint4* p, size_t n16, uint8_t* tail, size_t ntail)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s)
{
    const size_t n16 = bytes / 16, ntail = bytes % 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n16,
                       (uint8_t*)p + n16 * 16, ntail);
    return hipGetLastError();
}

// ---- checkpoint layout conversion -----------------------------------------
// Logical tile [C][R] row-major (C = output axis, R = reduction axis) <->
// fragment order (common.hpp).  One thread per float4.
__device__ __forceinline__ size_t frag_to_logical(size_t q, int C, int R)
{
    const int NB = R >> 4;
    const size_t per_tile = (size_t)C * R / 4;
    const size_t tile = q / per_tile;
    size_t rem = q - tile * per_tile;
    const int lane = (int)(rem & 63);
    rem >>= 6;
    const int nb = (int)(rem % NB);
    const int strip = (int)(rem / NB);
    const int c = 16 * strip + (lane & 15);
    const int r = 16 * nb + 4 * (lane >> 4);
    return tile * (size_t)C * R + (size_t)c * R + r;
}

// One thread per lane-block q (4 consecutive values of a logical row), moved
// as one word W (16 bytes of fp32 or 8 bytes of fp16).
template <int CK, class W>
__global__ void tiles_to_logical_kernel(const W* ck, W* out, size_t n4, int C, int R)
{
    const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n4) return;
    out[frag_to_logical(q, C, R) / 4] = ck[ckpt_elem_offset<CK>(q, R >> 4) / 4];
}

// Lane-block q of the source tiles -> the same lane-block of the tile the slot
// map names.
__device__ __forceinline__ size_t map_block(size_t q, size_t per_tile, const SlotMap& m)
{
    if (m.n == 0) return q;
    const size_t ts = q / per_tile;
    const size_t i = ts / (size_t)m.H;
    const size_t td = (size_t)m.slot[i] * m.H + (ts - i * m.H);
    return td * per_tile + (q - ts * per_tile);
}

// One word W (4 values in the checkpoint dtype) per thread, same dtype on both sides.
template <int CK, class W>
__global__ void logical_to_tiles_kernel(const W* in, W* ck, size_t n4, int C, int R, SlotMap m)
{
    const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n4) return;
    const size_t qd = map_block(q, (size_t)C * R / 4, m);
    ck[ckpt_elem_offset<CK>(qd, R >> 4) / 4] = in[frag_to_logical(q, C, R) / 4];
}

// Four fp32 values per thread, rounded to the checkpoint dtype by the same
// conversions the fold's store uses (binary16 RNE; E4M3 RNE saturating at +-448,
// NaN to 0x7f).
template <int CK>
__global__ void logical_f32_to_tiles_kernel(const f32x4* in, void* ck, size_t n4, int C, int R, SlotMap m)
{
    const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n4) return;
    const f32x4 v = in[frag_to_logical(q, C, R) / 4];
    const size_t e = ckpt_elem_offset<CK>(map_block(q, (size_t)C * R / 4, m), R >> 4);
    if constexpr (CK == CK_F32) static_cast<f32x4*>(ck)[e / 4] = v;
    else if constexpr (CK == CK_F16) static_cast<u32x2*>(ck)[e / 4] = f32_to_h4(v);
    else static_cast<uint32_t*>(ck)[e / 4] = pack_e4m3(v);
}

hipError_t launch_tiles_to_logical(const void* ckpt, void* out, int tiles, int C, int R, int ck, hipStream_t s)
{
    const size_t n4 = (size_t)tiles * C * R / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
    if (ck == CK_FP8)
        hipLaunchKernelGGL((tiles_to_logical_kernel<CK_FP8, uint32_t>), grid, block, 0, s,
                           static_cast<const uint32_t*>(ckpt), static_cast<uint32_t*>(out), n4, C, R);
    else if (ck == CK_F16)
        hipLaunchKernelGGL((tiles_to_logical_kernel<CK_F16, u32x2>), grid, block, 0, s,
                           static_cast<const u32x2*>(ckpt), static_cast<u32x2*>(out), n4, C, R);
    else
        hipLaunchKernelGGL((tiles_to_logical_kernel<CK_F32, u32x4>), grid, block, 0, s,
                           static_cast<const u32x4*>(ckpt), static_cast<u32x4*>(out), n4, C, R);
    return hipGetLastError();
}

hipError_t launch_logical_to_tiles(const void* in, void* ckpt, int tiles, int C, int R, int ck, bool src_f32,
                                   const SlotMap& m, hipStream_t s)
{
    const size_t n4 = (size_t)tiles * C * R / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
    if (src_f32 && ck != CK_F32) {
        const f32x4* src = static_cast<const f32x4*>(in);
        if (ck == CK_FP8)
            hipLaunchKernelGGL((logical_f32_to_tiles_kernel<CK_FP8>), grid, block, 0, s, src, ckpt, n4, C, R, m);
        else
            hipLaunchKernelGGL((logical_f32_to_tiles_kernel<CK_F16>), grid, block, 0, s, src, ckpt, n4, C, R, m);
    } else if (ck == CK_FP8) {
        hipLaunchKernelGGL((logical_to_tiles_kernel<CK_FP8, uint32_t>), grid, block, 0, s,
                           static_cast<const uint32_t*>(in), static_cast<uint32_t*>(ckpt), n4, C, R, m);
    } else if (ck == CK_F16) {
        hipLaunchKernelGGL((logical_to_tiles_kernel<CK_F16, u32x2>), grid, block, 0, s,
                           static_cast<const u32x2*>(in), static_cast<u32x2*>(ckpt), n4, C, R, m);
    } else {
        hipLaunchKernelGGL((logical_to_tiles_kernel<CK_F32, u32x4>), grid, block, 0, s,
                           static_cast<const u32x4*>(in), static_cast<u32x4*>(ckpt), n4, C, R, m);
    }
    return hipGetLastError();
}

// ---- read copy: quantize the fragment-ordered checkpoint, export codes ---------
// One wave per (tile, 16-column strip), in the same lane order as the replay
// kernels, so the quantizer is the one the flush path uses.
template <int NB, int RC, int CK>
__global__ __launch_bounds__(256) void quantize_rc_kernel(void* ckpt, uint8_t* codes, uint8_t* scales,
                                                          size_t nstrips, int mode, int strips_per_tile, SlotMap m)
{
    const size_t src_strip = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (src_strip >= nstrips) return;              // whole waves leave together
    const size_t strip = map_block(src_strip, (size_t)strips_per_tile, m);
    f32x4 s[NB];
    ckpt_load<NB, CK>(ckpt, strip, lane, s);
    const bool mx_ceil = (mode & QMODE_MX_CEIL) != 0;
    rc_store<NB, RC>(codes, scales, strip, lane, s, mx_ceil);
    if (mode & QMODE_ROUND_CKPT) {                 // checkpoint kept at the copy's precision
        rc_roundtrip<NB, RC>(s, mx_ceil);
        ckpt_store<NB, CK>(ckpt, strip, lane, s);
    }
}

// Raw codes to logical order: codes_out [tiles][C][R] (one code per byte),
// scales_out [tiles][C][R/32] for MXFP4.
template <int NB, int RC>
__global__ __launch_bounds__(256) void rc_to_logical_kernel(const uint8_t* codes, const uint8_t* scales,
                                                            uint8_t* codes_out, uint8_t* scales_out, size_t nstrips, int C)
{
    constexpr int R = NB * 16;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t strip = gid / 64;
    const int lane = (int)(gid % 64);
    if (strip >= nstrips) return;
    const int strips = C / 16;
    const size_t tile = strip / strips;
    const int c = 16 * (int)(strip % strips) + (lane & 15);
    uint8_t* row = codes_out + (tile * C + c) * R;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint32_t code;
            if constexpr (RC == RC_FP8) {
                constexpr int BPL = 4 * NB;
                code = (BPL >= 16) ? codes[rc_offset<BPL>(strip, nb / 4, lane) + (nb % 4) * 4 + r]
                                   : codes[rc_offset<BPL>(strip, 0, lane) + 4 * nb + r];
            } else {
                constexpr int BPL = 2 * NB;
                const int n = (BPL >= 16 ? (nb % 8) : nb) * 4 + r;
                const uint8_t byte = codes[rc_offset<BPL>(strip, BPL >= 16 ? nb / 8 : 0, lane) + n / 2];
                code = (n & 1) ? (byte >> 4) : (byte & 0xfu);
            }
            row[16 * nb + 4 * (lane >> 4) + r] = (uint8_t)code;
        }
    }
    if constexpr (RC == RC_MXFP4) {
        if (lane < 16) {
            constexpr int NP = NB / 2;
            for (int p = 0; p < NP; ++p) scales_out[(tile * C + c) * NP + p] = scales[(strip * 16 + lane) * NP + p];
        }
    }
}

template <int RC, int CK>
static hipError_t rc_dispatch(bool quantize, void* ckpt, const uint8_t* codes_in, const uint8_t* scales_in,
                              uint8_t* codes, uint8_t* scales, int tiles, int C, int R, int mode,
                              const SlotMap& m, hipStream_t s)
{
    const size_t nstrips = (size_t)tiles * (C / 16);
    const int spt = C / 16;
    const dim3 grid((unsigned)((nstrips + 3) / 4)), block(256);
#define RS_RC_CASE(NBV)                                                                                  \
    case NBV * 16:                                                                                       \
        if (quantize) hipLaunchKernelGGL((quantize_rc_kernel<NBV, RC, CK>), grid, block, 0, s, ckpt, codes, scales,   \
                                         nstrips, mode, spt, m);                                  \
        else hipLaunchKernelGGL((rc_to_logical_kernel<NBV, RC>), grid, block, 0, s, codes_in, scales_in, codes, scales,    \
                                nstrips, C);                                                             \
        return hipGetLastError();
    switch (R) {
        case 16:
            if constexpr (RC == RC_FP8) {
                if (quantize) hipLaunchKernelGGL((quantize_rc_kernel<1, RC, CK>), grid, block, 0, s, ckpt, codes, scales,
                                                 nstrips, mode, spt, m);
                else hipLaunchKernelGGL((rc_to_logical_kernel<1, RC>), grid, block, 0, s, codes_in, scales_in, codes, scales,
                                        nstrips, C);
                return hipGetLastError();
            }
            return hipErrorInvalidValue;
        RS_RC_CASE(2)
        RS_RC_CASE(4)
        RS_RC_CASE(8)
        RS_RC_CASE(16)
    }
#undef RS_RC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_quantize_read_copy(void* ckpt, uint8_t* codes, uint8_t* scales, int tiles, int C, int R, int rc,
                                     int ck, bool round_ckpt, bool mx_ceil, const SlotMap& m, hipStream_t s)
{
    const int ceil_bit = (mx_ceil && rc == RC_MXFP4) ? QMODE_MX_CEIL : 0;
    const int mode = (round_ckpt ? QMODE_ROUND_CKPT : 0) | ceil_bit;
    if (ck == CK_FP8) {
        if (round_ckpt || rc != RC_MXFP4) return hipErrorInvalidValue;   // only an MXFP4 copy of an FP8 checkpoint
        return rc_dispatch<RC_MXFP4, CK_FP8>(true, ckpt, nullptr, nullptr, codes, scales, tiles, C, R, ceil_bit, m, s);
    }
    if (ck == CK_F16) {
        if (round_ckpt) return hipErrorInvalidValue;     // the quantized-checkpoint variant keeps fp32 storage
        if (rc == RC_FP8) return rc_dispatch<RC_FP8, CK_F16>(true, ckpt, nullptr, nullptr, codes, scales, tiles, C, R, 0, m, s);
        if (rc == RC_MXFP4)
            return rc_dispatch<RC_MXFP4, CK_F16>(true, ckpt, nullptr, nullptr, codes, scales, tiles, C, R, ceil_bit, m, s);
        return hipErrorInvalidValue;
    }
    if (rc == RC_FP8)
        return rc_dispatch<RC_FP8, CK_F32>(true, ckpt, nullptr, nullptr, codes, scales, tiles, C, R, mode, m, s);
    if (rc == RC_MXFP4)
        return rc_dispatch<RC_MXFP4, CK_F32>(true, ckpt, nullptr, nullptr, codes, scales, tiles, C, R, mode, m, s);
    return hipErrorInvalidValue;
}

hipError_t launch_read_copy_to_logical(const uint8_t* codes, const uint8_t* scales, uint8_t* codes_out,
                                       uint8_t* scales_out, int tiles, int C, int R, int rc, hipStream_t s)
{
    SlotMap all;
    all.n = 0;
    all.H = 1;
    if (rc == RC_FP8) return rc_dispatch<RC_FP8, CK_F32>(false, nullptr, codes, scales, codes_out, scales_out, tiles, C, R, 0, all, s);
    if (rc == RC_MXFP4) return rc_dispatch<RC_MXFP4, CK_F32>(false, nullptr, codes, scales, codes_out, scales_out, tiles, C, R, 0, all, s);
    return hipErrorInvalidValue;
}

// ---- streaming copy / read: bandwidth ceilings and byte-counter reference ----
// Same access pattern as the replay step kernels' checkpoint stream: one
// workgroup of four waves per 32 KiB tile, workgroups remapped so each XCD
// takes a contiguous range of tiles, every lane with eight 128-bit nontemporal
// loads in flight (each wave moves eight contiguous 1 KiB rows), issued before
// any of them is consumed.  A ragged tail (bytes not a multiple of 32 KiB) is
// handled by the last workgroup, 16 bytes per thread.
constexpr int STREAM_TILE_F4 = 2048;              // 32 KiB per workgroup

__global__ __launch_bounds__(256) void stream_copy_kernel(const f32x4* src, f32x4* dst, size_t n4)
{
    const size_t tile = (size_t)xcd_tile_index();
    const size_t base = tile * STREAM_TILE_F4 + (threadIdx.x >> 6) * 512 + (threadIdx.x & 63);
    if (base + 7 * 64 < n4 && (tile + 1) * STREAM_TILE_F4 <= n4) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(src + base + i * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(v[i], dst + base + i * 64);
        return;
    }
    for (size_t i = tile * STREAM_TILE_F4 + threadIdx.x; i < n4 && i < (tile + 1) * STREAM_TILE_F4; i += blockDim.x)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s)
{
    const size_t n4 = bytes / 16;
    size_t blocks = (n4 + STREAM_TILE_F4 - 1) / STREAM_TILE_F4;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const f32x4*)src, (f32x4*)dst, n4);
    return hipGetLastError();
}

// Read-only stream: the ceiling for checkpoint reads that write nothing back.
// The replay kernels' pattern: one 32 KiB tile per workgroup (eight 128-bit
// nontemporal loads in flight per lane, XCD-aware tile order), every loaded
// value summed so that no load is dead, and one plain store per workgroup of
// its tile's sum (a single shared accumulator would serialise 32768 atomics).
// The last workgroup takes the ragged tail.
__global__ __launch_bounds__(256) void stream_read_kernel(const f32x4* src, size_t n4, float* partials)
{
    __shared__ float part[4];
    const size_t t = (size_t)xcd_tile_index();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if ((t + 1) * STREAM_TILE_F4 <= n4) {
        const f32x4* p = src + t * STREAM_TILE_F4 + (threadIdx.x >> 6) * 512 + (threadIdx.x & 63);
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(p + i * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += v[i];
    } else {
        for (size_t i = t * STREAM_TILE_F4 + threadIdx.x; i < n4; i += blockDim.x)
            acc += __builtin_nontemporal_load(src + i);
    }
    const float v = wave_sum64(acc.x + acc.y + acc.z + acc.w);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) partials[t] = part[0] + part[1] + part[2] + part[3];
}

hipError_t launch_stream_read(const void* src, size_t bytes, float* partials, hipStream_t s)
{
    const size_t n4 = bytes / 16;
    size_t blocks = (n4 + STREAM_TILE_F4 - 1) / STREAM_TILE_F4;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const f32x4*)src, n4, partials);
    return hipGetLastError();
}

}  // namespace rs
