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
#include "common.hpp"
#include "internal.hpp"

namespace rs {

template <int NB, int IO, int TMAX, bool MFMA_FOLD>
__global__ __launch_bounds__(1024) void mamba2_step_kernel(StepArgs a)
{
    extern __shared__ float lds[];
    constexpr int R = NB * 16;
    const int C = a.C;
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
    const int fc = bk[2 * sB + b];                  // corrupted word cannot index out of bounds
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

    // ---- 1. checkpoint tile -> registers (one 128-bit load per block)
    float* ckw = a.ckpt + (((size_t)tile * (C >> 4) + w) * NB * 64 + lane) * 4;
    f32x4 s[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = ld4_stream(ckw + (size_t)nb * 256);

    // ---- 2. stage entries and read-out vectors in LDS
    const int Tr = T > 0 ? T : 1;
    float* xs = lds;                          // [vmax][C]
    float* bs = xs + (size_t)a.vmax * C;      // [vmax][R]
    float* ds = bs + (size_t)a.vmax * R;      // [vmax]
    float* cs = ds + ((a.vmax + 3) & ~3);     // [T][R] (16-byte aligned)
    float* gq = cs + (size_t)Tr * R;          // [vmax][T]
    const size_t hc = (size_t)b * a.H + h, gr = (size_t)b * a.G + g;
    for (int i = tid; i < V * C; i += nthr) {
        const int j = i / C, c = i - j * C;
        xs[i] = (j < len) ? ld_io<IO>(a.bufc, (size_t)bank * a.bank_c + ((hc * a.cap + j) * C + c))
                          : ld_io<IO>(a.in_c, (((size_t)(j - len) * sB + b) * a.H + h) * C + c);
    }
    for (int i = tid; i < V * R; i += nthr) {
        const int j = i / R, r = i - j * R;
        bs[i] = (j < len) ? ld_io<IO>(a.bufr, (size_t)bank * a.bank_r + ((gr * a.cap + j) * R + r))
                          : ld_io<IO>(a.in_r, (((size_t)(j - len) * sB + b) * a.G + g) * R + r);
    }
    for (int i = tid; i < T * R; i += nthr) {
        const int t = i / R, r = i - t * R;
        cs[i] = ld_io<IO>(a.in_q, (((size_t)t * sB + b) * a.G + g) * R + r);
    }
    for (int j = tid; j < V; j += nthr)
        ds[j] = (j < len) ? a.bufs0[(size_t)bank * a.bank_s + hc * a.cap + j]
                          : ld_io<IO>(a.in_s0, ((size_t)(j - len) * sB + b) * a.H + h);
    __syncthreads();

    const float Ah = a.A[h];

    // ---- 3. dots B_j . C_t for the entries replayed on top of the checkpoint
    const int nrem = V - f;
    const int waves = nthr >> 6;
    for (int d = w; d < nrem * T; d += waves) {
        const int jj = d / T, t = d - jj * T;
        const int j = f + jj;
        float acc = 0.f;
        if (j <= len + t)
            for (int r = lane; r < R; r += 64) acc += bs[j * R + r] * cs[t * R + r];
        acc = wave_sum64(acc);
        if (lane == 0) gq[j * Tr + t] = acc;
    }

    // ---- 4. fold the first f entries into the checkpoint registers
    if (f > 0) {
        float Lf = 0.f;
        for (int i = 0; i < f; ++i) Lf += ds[i] * Ah;
        const float decay = expf(Lf);
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
                    for (int j = i + 1; j < f; ++j) suf += ds[j] * Ah;
                    v = expf(suf) * ds[i] * xs[i * C + col];
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
                        const float av = (i < f) ? bs[i * R + nb * 16 + (lane & 15)] : 0.f;
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
                    for (int j = i + 1; j < f; ++j) suf += ds[j] * Ah;
                    v = expf(suf) * ds[i] * xs[i * C + col];
                }
                wx[i] = v;
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (i < f) acc += wx[i] * ld4(bs + i * R + nb * 16 + rq);
                s[nb] = decay * s[nb] + acc;
            }
        }
    }
    __syncthreads();   // gq complete

    // ---- 5. outputs of the new tokens
    if (a.mode != MODE_FLUSH) {
        float gacc[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) gacc[t] = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t < T) {
                    const f32x4 cv = ld4(cs + t * R + nb * 16 + rq);
                    gacc[t] += s[nb].x * cv.x + s[nb].y * cv.y + s[nb].z * cv.z + s[nb].w * cv.w;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            if (t < T) gacc[t] = sum_over_row_groups(gacc[t]);

        if (lane < 16) {
            const float Dh = a.D[h];
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t < T) {
                    const int pos = len + t;
                    float yv;
                    if (pos < f) {
                        yv = gacc[t] + Dh * xs[pos * C + col];
                    } else {
                        float suf = 0.f, rep = 0.f;
                        for (int j = pos; j >= f; --j) {
                            rep += expf(suf) * ds[j] * gq[j * Tr + t] * xs[j * C + col];
                            suf += ds[j] * Ah;
                        }
                        yv = expf(suf) * gacc[t] + rep + Dh * xs[pos * C + col];
                    }
                    st_io<IO>(a.y, (((size_t)t * sB + b) * a.H + h) * C + col, yv);
                }
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
        for (int i = tid; i < nnew * C; i += nthr) {
            const int jj = i / C, c = i - jj * C, j = j0 + jj;
            st_io<IO>(a.bufc, (size_t)bank_new * a.bank_c + ((hc * a.cap + (j - f)) * C + c), xs[j * C + c]);
        }
        for (int jj = tid; jj < nnew; jj += nthr)
            a.bufs0[(size_t)bank_new * a.bank_s + hc * a.cap + (j0 + jj - f)] = ds[j0 + jj];
        if (h % a.hpg == 0) {
            for (int i = tid; i < nnew * R; i += nthr) {
                const int jj = i / R, r = i - jj * R, j = j0 + jj;
                st_io<IO>(a.bufr, (size_t)bank_new * a.bank_r + ((gr * a.cap + (j - f)) * R + r), bs[j * R + r]);
            }
        }
    }
}

template <int NB, int IO, int TMAX, bool MF>
static hipError_t launch_nb(const StepArgs& a, hipStream_t s)
{
    const int Tr = a.T > 0 ? a.T : 1;
    const size_t vpad = ((size_t)a.vmax + 3) & ~(size_t)3;
    const size_t lds = sizeof(float) * ((size_t)a.vmax * (a.C + NB * 16 + Tr) + vpad + (size_t)Tr * NB * 16);
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
