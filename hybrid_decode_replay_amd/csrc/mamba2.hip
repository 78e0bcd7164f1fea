// mamba2.hip -- replayed Mamba-2 decode step for gfx950 (CDNA4).
//
// One workgroup per (sequence b, head h); wave w owns the 16 output columns
// p in [16w, 16w+16) of the head and every state row n (see common.hpp for the
// fragment-ordered tile).  Per launch and sequence the virtual entry list is
// V = (committed buffer entries 0..len-1) ++ (T new tokens).  The first f
// entries are folded into the checkpoint (f = 0 on a non-flush step), the
// rest stay in the buffer and are replayed on top of the checkpoint for the
// outputs.  With l_i = dt_i A_h (pages: the checkpoint plus buffered inputs
// give the output and the recurrence is unrolled over the buffered window --
// [DE] "ReplaySSM beschleunigt das Decoding ...", section "Wie es
// funktioniert"; the filling step folds and writes the checkpoint once --
// [TR] "NVIDIA ve Dao AI Lab ...", section "ReplaySSM nasil calisir?"):
//
//   fold    S' = e^{sum_{i<f} l_i} S0 + sum_{i<f} e^{sum_{i<j<f} l_j} dt_i x_i B_i^T
//           a [P x f] . [f x N] contraction per head, on MFMA (f <= 16)
//   output  y_t = e^{L'} (S' C_t) + sum_{f<=j<=pos} e^{sum_{j<i<=pos} l_i} dt_j (B_j . C_t) x_j
//                 + D_h x_t,     L' = sum_{f<=i<=pos} l_i,  pos = len + t
//           (if the token itself was folded, pos < f: y_t = S' C_t + D_h x_t)
//
// Non-flush steps read the checkpoint once and write no state; the flush step
// writes it once.  Only exponentials of sums of l (all <= 0) are taken.
//
// Memory schedule per workgroup: the entry rows (x, B), the read-out rows C
// and dt are fetched as 16-byte chunks issued before the checkpoint stream,
// so they land while the 128-bit checkpoint loads are still in flight; one
// workgroup barrier publishes them in LDS.  Every wave then computes the
// replay coefficients it needs itself (lane-parallel dots and suffix sums),
// so a non-flush step has no second barrier.
#include "common.hpp"
#include "internal.hpp"

namespace rs {

template <int IO>
__device__ __forceinline__ void chunk_to_lds(float* dst, uint4 v)
{
    if constexpr (IO == IO_F32) {
        st4(dst, __builtin_bit_cast(f32x4, v));
    } else {
        st4(dst, f32x4{bf16_bits_to_f32((uint16_t)(v.x & 0xffff)), bf16_bits_to_f32((uint16_t)(v.x >> 16)),
                       bf16_bits_to_f32((uint16_t)(v.y & 0xffff)), bf16_bits_to_f32((uint16_t)(v.y >> 16))});
        st4(dst + 4, f32x4{bf16_bits_to_f32((uint16_t)(v.z & 0xffff)), bf16_bits_to_f32((uint16_t)(v.z >> 16)),
                           bf16_bits_to_f32((uint16_t)(v.w & 0xffff)), bf16_bits_to_f32((uint16_t)(v.w >> 16))});
    }
}

template <int IO>
__device__ __forceinline__ uint4 lds_to_chunk(const float* src)
{
    if constexpr (IO == IO_F32) {
        return __builtin_bit_cast(uint4, ld4(src));
    } else {
        const f32x4 a = ld4(src), b = ld4(src + 4);
        auto pk = [](float lo, float hi) {
            return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
        };
        return uint4{pk(a.x, a.y), pk(a.z, a.w), pk(b.x, b.y), pk(b.z, b.w)};
    }
}

template <int NB, int IO, int TMAX, bool MFMA_FOLD>
__global__ __launch_bounds__(1024) void mamba2_step_kernel(StepArgs a)
{
    extern __shared__ float lds[];
    constexpr int R = NB * 16;
    constexpr int ES = IO == IO_BF16 ? 2 : 4;   // bytes per io element
    constexpr int EPC = 16 / ES;                // elements per 16-byte chunk
    constexpr int RX = R / EPC;                 // chunks per B or C row
    constexpr int RS = R + 4;                   // padded LDS stride of B rows
    constexpr int PRE = 4;                      // chunks per thread fetched ahead of the checkpoint
    const int C = a.C, CX = C / EPC;
    const int tile = xcd_tile_index();
    const int b = tile / a.H, h = tile - b * a.H;
    const int g = h / a.hpg;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int w = tid >> 6, lane = tid & 63;
    const int col = 16 * w + (lane & 15);
    const int rq = 4 * (lane >> 4);
    const size_t sB = (size_t)a.B;

    // ---- bookkeeping: identical decision in every workgroup of sequence b
    const int32_t* bk = a.book + (size_t)a.parity * 3 * sB;
    const int len = min(max(bk[b], 0), a.cap);   // invariant 0 <= len <= cap; clamped so a
    const int fc = bk[2 * sB + b];                // corrupted word cannot index out of bounds
    const int T = a.T;
    int f;
    if (a.mode == MODE_DECODE) f = (len + 1 >= a.cap) ? min(len + 1, a.cap) : 0;
    else if (a.mode == MODE_FLUSH) f = len;
    else f = (len + T > a.cap) ? len : 0;
    const int V = len + T;
    const int bank = fc & 1;
    const int bank_new = (fc + (f > 0 ? 1 : 0)) & 1;

    if (h == 0 && tid == 0) {
        int32_t* nbk = a.book + (size_t)(a.parity ^ 1) * 3 * sB;
        nbk[b] = (a.mode == MODE_DECODE) ? len + 1 - f : (a.mode == MODE_FLUSH ? 0 : len - f);
        nbk[sB + b] = (a.mode == MODE_SPEC) ? T : 0;
        nbk[2 * sB + b] = fc + (f > 0 ? 1 : 0);
    }
    if (a.mode == MODE_FLUSH && f == 0) return;

    // ---- LDS partition (floats)
    const int Tr = T > 0 ? T : 1;
    float* xs = lds;                              // [vmax][C]  entry x rows
    float* bs = xs + (size_t)a.vmax * C;          // [vmax][RS] entry B rows
    float* cs = bs + (size_t)a.vmax * RS;         // [Tr][R]    read-out rows C_t
    float* ds = cs + (size_t)Tr * R;              // [vmax]     entry dt

    // ---- 1. entry and read-out chunks, issued ahead of the checkpoint stream
    const size_t hc = (size_t)b * a.H + h, gr = (size_t)b * a.G + g;
    const int nx = V * CX, nbr = V * RX, nch = nx + nbr + T * RX;
    auto chunk_src = [&](int ch) -> const uint4* {
        size_t e;
        const void* base;
        if (ch < nx) {
            const int j = ch / CX, o = ch - j * CX;
            if (j < len) { base = a.bufc; e = (size_t)bank * a.bank_c + (hc * a.cap + j) * C; }
            else { base = a.in_c; e = (((size_t)(j - len) * sB + b) * a.H + h) * C; }
            return reinterpret_cast<const uint4*>(static_cast<const char*>(base) + e * ES) + o;
        }
        ch -= nx;
        if (ch < nbr) {
            const int j = ch / RX, o = ch - j * RX;
            if (j < len) { base = a.bufr; e = (size_t)bank * a.bank_r + (gr * a.cap + j) * R; }
            else { base = a.in_r; e = (((size_t)(j - len) * sB + b) * a.G + g) * R; }
            return reinterpret_cast<const uint4*>(static_cast<const char*>(base) + e * ES) + o;
        }
        ch -= nbr;
        const int t = ch / RX, o = ch - t * RX;
        e = (((size_t)t * sB + b) * a.G + g) * R;
        return reinterpret_cast<const uint4*>(static_cast<const char*>(a.in_q) + e * ES) + o;
    };
    auto chunk_dst = [&](int ch) -> float* {
        if (ch < nx) { const int j = ch / CX; return xs + j * C + (ch - j * CX) * EPC; }
        ch -= nx;
        if (ch < nbr) { const int j = ch / RX; return bs + j * RS + (ch - j * RX) * EPC; }
        ch -= nbr;
        const int t = ch / RX;
        return cs + t * R + (ch - t * RX) * EPC;
    };
    uint4 pre[PRE];
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
        const int ch = tid + u * nthr;
        if (ch < nch) pre[u] = *chunk_src(ch);
    }
    // dt stays as raw bits until it is published, so its conversion does not make the
    // wave wait for the chunk loads before the checkpoint loads are issued
    uint32_t dtraw = 0, dtshift = 0;
    if (tid < V) {
        if (tid < len) {
            dtraw = reinterpret_cast<const uint32_t*>(a.bufs0)[(size_t)bank * a.bank_s + hc * a.cap + tid];
        } else if constexpr (IO == IO_F32) {
            dtraw = static_cast<const uint32_t*>(a.in_s0)[((size_t)(tid - len) * sB + b) * a.H + h];
        } else {
            dtraw = static_cast<const uint16_t*>(a.in_s0)[((size_t)(tid - len) * sB + b) * a.H + h];
            dtshift = 16;
        }
    }

    // ---- 2. checkpoint tile -> registers (one 128-bit load per 16x16 block)
    float* ckw = a.ckpt + (((size_t)tile * (C >> 4) + w) * NB * 64 + lane) * 4;
    f32x4 s[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = ld4_stream(ckw + (size_t)nb * 256);

    // ---- 3. publish the staged rows
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
        const int ch = tid + u * nthr;
        if (ch < nch) chunk_to_lds<IO>(chunk_dst(ch), pre[u]);
    }
    for (int ch = tid + PRE * nthr; ch < nch; ch += nthr) chunk_to_lds<IO>(chunk_dst(ch), *chunk_src(ch));
    if (tid < V) ds[tid] = __builtin_bit_cast(float, dtraw << dtshift);
    __syncthreads();

    const float Ah = a.A[h];

    // ---- 4. fold the first f entries into the checkpoint registers
    if (f > 0) {
        float Lf = 0.f;
        for (int i = 0; i < f; ++i) Lf += ds[i];
        const float decay = expf(Lf * Ah);
        if constexpr (MFMA_FOLD) {
            // D[n][p] += sum_i A[n][i] B[i][p] with A = B_i[n] (lane: n = l%16,
            // i = l/16) and B = e^{..} dt_i x_i[p] (lane: i = l/16, p = l%16).
            const int iq = lane >> 4;
            float bop[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int i = kb * 4 + iq;
                float v = 0.f;
                if (i < f) {
                    float suf = 0.f;
                    for (int j = i + 1; j < f; ++j) suf += ds[j];
                    v = expf(suf * Ah) * ds[i] * xs[i * C + col];
                }
                bop[kb] = v;
            }
            const int nkb = (f + 3) >> 2;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    if (kb < nkb) {
                        const int i = kb * 4 + iq;
                        const float av = (i < f) ? bs[i * RS + nb * 16 + (lane & 15)] : 0.f;
                        acc = mfma16x16x4(av, bop[kb], acc);
                    }
                }
                s[nb] = decay * s[nb] + acc;
            }
        } else {
            float wx[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float v = 0.f;
                if (i < f) {
                    float suf = 0.f;
                    for (int j = i + 1; j < f; ++j) suf += ds[j];
                    v = expf(suf * Ah) * ds[i] * xs[i * C + col];
                }
                wx[i] = v;
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (i < f) acc += wx[i] * ld4(bs + i * RS + nb * 16 + rq);
                s[nb] = decay * s[nb] + acc;
            }
        }
    }

    // ---- 5. outputs of the new tokens
    if (a.mode != MODE_FLUSH) {
        const float Dh = a.D[h];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {
                // checkpoint read-out (S' C_t)[col], reduced over the four row groups
                float gacc = 0.f;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) gacc += dot4(s[nb], ld4(cs + t * R + nb * 16 + rq));
                gacc = sum_over_row_groups(gacc);
                const int pos = len + t;
                float yv;
                if (pos < f) {
                    yv = gacc + Dh * xs[pos * C + col];
                } else {
                    // replay of entries f..pos: lane quad (jj = l/4) forms B_j . C_t and the
                    // decayed coefficient; output lanes gather the coefficients by shuffle
                    const int nr = pos - f + 1;
                    const int q = lane & 3;
                    float rep = 0.f;
                    for (int jj0 = 0; jj0 < nr; jj0 += 16) {
                        const int jj = jj0 + (lane >> 2), j = f + jj;
                        float dot = 0.f;
                        if (jj < nr) {
#pragma unroll
                            for (int i = 0; i < R / 16; ++i)
                                dot += dot4(ld4(bs + j * RS + 16 * i + 4 * q), ld4(cs + t * R + 16 * i + 4 * q));
                        }
                        dot += __shfl_xor(dot, 1, 64);
                        dot += __shfl_xor(dot, 2, 64);
                        float coef = 0.f;
                        if (jj < nr) {
                            float suf = 0.f;
                            for (int i = j + 1; i <= pos; ++i) suf += ds[i];
                            coef = expf(suf * Ah) * ds[j] * dot;
                        }
                        const int ne = min(16, nr - jj0);
                        for (int e = 0; e < ne; ++e)
                            rep += __shfl(coef, 4 * e, 64) * xs[(f + jj0 + e) * C + col];
                    }
                    float Lp = 0.f;
                    for (int i = f; i <= pos; ++i) Lp += ds[i];
                    yv = expf(Lp * Ah) * gacc + rep + Dh * xs[pos * C + col];
                }
                if (lane < 16) st_io<IO>(a.y, (((size_t)t * sB + b) * a.H + h) * C + col, yv);
            }
        }
    }

    // ---- 6. single checkpoint write on a folding step
    if (f > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) st4_stream(ckw + (size_t)nb * 256, s[nb]);
    }

    // ---- 7. append the unfolded new tokens to the buffer (slot = position - f)
    const int j0 = max(f, len);
    const int nnew = V - j0;
    if (nnew > 0) {
        char* bx = static_cast<char*>(a.bufc) + ((size_t)bank_new * a.bank_c + hc * a.cap * C) * ES;
        for (int i = tid; i < nnew * CX; i += nthr) {
            const int jj = i / CX, o = i - jj * CX, j = j0 + jj;
            reinterpret_cast<uint4*>(bx + (size_t)(j - f) * C * ES)[o] = lds_to_chunk<IO>(xs + j * C + o * EPC);
        }
        if (tid < nnew) a.bufs0[(size_t)bank_new * a.bank_s + hc * a.cap + (j0 + tid - f)] = ds[j0 + tid];
        if (h % a.hpg == 0) {
            char* bb = static_cast<char*>(a.bufr) + ((size_t)bank_new * a.bank_r + gr * a.cap * R) * ES;
            for (int i = tid; i < nnew * RX; i += nthr) {
                const int jj = i / RX, o = i - jj * RX, j = j0 + jj;
                reinterpret_cast<uint4*>(bb + (size_t)(j - f) * R * ES)[o] = lds_to_chunk<IO>(bs + j * RS + o * EPC);
            }
        }
    }
}

template <int NB, int IO, int TMAX, bool MF>
static hipError_t launch_nb(const StepArgs& a, hipStream_t s)
{
    const size_t Tr = a.T > 0 ? a.T : 1;
    const size_t R = NB * 16;
    const size_t lds = sizeof(float) * ((size_t)a.vmax * (a.C + R + 4) + Tr * R + (size_t)a.vmax);
    auto k = mamba2_step_kernel<NB, IO, TMAX, MF>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3(a.B * a.H), dim3(a.C * 4), lds, s, a);
    return hipGetLastError();
}

template <int IO, int TMAX, bool MF>
static hipError_t launch_io(const StepArgs& a, hipStream_t s)
{
    switch (a.R) {
        case 16: return launch_nb<1, IO, TMAX, MF>(a, s);
        case 32: return launch_nb<2, IO, TMAX, MF>(a, s);
        case 64: return launch_nb<4, IO, TMAX, MF>(a, s);
        case 128: return launch_nb<8, IO, TMAX, MF>(a, s);
        case 256: return launch_nb<16, IO, TMAX, MF>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int TMAX, bool MF>
static hipError_t launch_t(const StepArgs& a, int io, hipStream_t s)
{
    return io == IO_BF16 ? launch_io<IO_BF16, TMAX, MF>(a, s) : launch_io<IO_F32, TMAX, MF>(a, s);
}

hipError_t launch_mamba2_step(const StepArgs& a, int io, int rc, bool valu_fold, hipStream_t s)
{
    if (rc != RC_NONE) return hipErrorNotSupported;
    if (a.T <= 1) return valu_fold ? launch_t<1, false>(a, io, s) : launch_t<1, true>(a, io, s);
    if (a.T <= 4) return valu_fold ? launch_t<4, false>(a, io, s) : launch_t<4, true>(a, io, s);
    return valu_fold ? launch_t<16, false>(a, io, s) : launch_t<16, true>(a, io, s);
}

}  // namespace rs
