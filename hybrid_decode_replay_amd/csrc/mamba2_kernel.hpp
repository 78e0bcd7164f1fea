// mamba2_kernel.hpp -- replayed Mamba-2 decode step for gfx950 (CDNA4).
// Included by one translation unit per checkpoint storage dtype.
//
// One workgroup per (sequence b, head h, column slice): the head's output
// columns are split over workgroups of at most four waves, and wave w owns 16
// output columns p and every state row n (see common.hpp for the
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
// writes it once.  Only exponentials of sums of l (all <= 0) are taken; a sum
// over an entry range is a difference of inclusive prefix sums of dt, formed
// once per launch by a wave scan while the entries are published.
//
// Memory schedule per workgroup: the entry rows (x, B), the read-out rows C
// and dt are fetched as 16-byte chunks issued before the checkpoint stream,
// so they land while the 128-bit checkpoint loads are still in flight; one
// workgroup barrier publishes them in LDS.  Every wave then computes the
// replay coefficients it needs itself (lane-parallel dots and suffix sums),
// so a non-flush step has no second barrier.
#pragma once
#include "common.hpp"
#include "internal.hpp"
#include "ckpt.hpp"
#include "rc.hpp"
#include "stage.hpp"

namespace rs {

// HT heads of one group per workgroup (HT = 1, 2 or 4; HT > 1 only with four
// waves).  The sequence's bookkeeping, the group's B and C rows and the entry
// staging are done once for the HT heads; the heads are then processed in turn,
// and head hh+1's checkpoint (or read-copy) loads are issued before head hh's
// arithmetic, so one head's stream overlaps the previous head's work.
// Workgroups per CU the register budget is set for: six single-head workgroups; four
// four-head ones, except with an FP8 checkpoint and an MXFP4 copy, where the fold's two
// encoders need more registers than four allow (at four the compiler spills the staged
// entry chunks of every step, and the step's scratch traffic depends on what ran before
// it; measured at batch 256: 29-40 % of peak spilling, 34 % at three without spills).
template <int HT, int NB, int RC, int CK>
constexpr int mamba2_wg_per_cu()
{
    if constexpr (HT == 1) return NB <= 8 ? 6 : 4;
    else if constexpr (NB > 8) return 2;
    else return CK == CK_FP8 && RC == RC_MXFP4 ? 3 : 4;
}

template <int NB, int IO, int TMAX, bool MFMA_FOLD, int RC, int CK, int HT>
__global__ __launch_bounds__(256, (mamba2_wg_per_cu<HT, NB, RC, CK>())) void mamba2_step_kernel(StepArgs a)
{
    extern __shared__ float lds[];
    constexpr int R = NB * 16;
    constexpr int RS = R + 4;                   // padded LDS stride of B rows
    constexpr int PRE = 4;                      // chunks per thread fetched ahead of the checkpoint
    constexpr int VM = (16 + TMAX + 3) & ~3;    // bound on the entry count cap + T, padded to 4
    constexpr int XS = 64;                      // LDS row stride of x rows (cw <= 64: four waves of 16)
    const int vx = a.vmax + 3;                  // x rows per head: entries, then three zero rows
    const int C = a.C;
    const TileIdx tix = tile_of(xcd_tile_index(), a.H / HT, a.mg_tiles, a.nsplit, a.mg_nsplit);
    const int b = tix.b, h0 = tix.h * HT;
    const int g = (int)div_magic((uint32_t)h0, a.mg_hpg);
    const int cw = a.cw, c0 = tix.sp * cw;           // this workgroup's output columns
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lc = 16 * w + (lane & 15);             // local output column
    const int col = c0 + lc;                          // global output column
    const int rq = 4 * (lane >> 4);
    const size_t sB = (size_t)a.B;

    // ---- the heads' A and D by scalar loads (a vector load issued after the
    // checkpoint loads could only be used once every one of them had landed)
    float Av[HT], Dv[HT];
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
        Av[hh] = uload(a.A + h0 + hh);
        Dv[hh] = uload(a.D + h0 + hh);
    }

    // ---- bookkeeping: identical decision in every workgroup of sequence b
    const StepPlan p = plan_step(a, b, h0 == 0 && tix.sp == 0 && tid == 0);
    if (p.skip || (a.mode == MODE_FLUSH && p.f == 0)) return;
    const int f = p.f, len = p.len, T = a.T;

    // ---- LDS partition (floats; the launch sizes cs for max(T, 1) rows)
    float* ds = lds;                              // [HT][VM]       entry dt (vmax <= VM)
    float* ps = ds + HT * VM;                     // [HT][VM]       inclusive prefix sums of dt
    float* xs = ps + HT * VM;                     // [HT][vx][XS]   entry x rows (own columns)
    float* bs = xs + (size_t)HT * vx * XS;        // [vmax][RS]     entry B rows
    float* cs = bs + (size_t)a.vmax * RS;         // [Tr][R]        read-out rows C_t
    float* cf = cs + (size_t)(T > 0 ? T : 1) * R; // [4][16]        per-wave replay coefficients
    float* gs = cf + 64;                          // [Tr][VM]       B_j . C_t (several tokens)

    StageGeom G;
    G.bufc = a.bufc; G.bufr = a.bufr; G.bufs0 = a.bufs0; G.bufs1 = nullptr;
    G.in_c = a.in_c; G.in_r = a.in_r; G.in_q = a.in_q; G.in_s0 = a.in_s0; G.in_s1 = nullptr;
    G.bank_c = a.bank_c; G.bank_r = a.bank_r; G.bank_s = a.bank_s;
    G.hc = (size_t)b * a.H + h0; G.gr = (size_t)b * a.G + g;
    G.b = b; G.h = h0; G.g = g; G.B = a.B; G.H = a.H; G.G = a.G; G.cap = a.cap; G.C = C;
    G.c0 = c0; G.cw = cw; G.m20_cx = a.m20_cx;
    G.ht = HT; G.xc_stride = vx * XS; G.xc_row = XS; G.sc_stride = VM;
    G.len = len; G.bank = p.bank; G.V = p.V; G.T = T;
    G.f = p.f; G.bank_new = p.bank_new; G.head_writer = tix.sp == 0; G.group_writer = tix.sp == 0 && h0 == g * a.hpg;
    G.xc = xs; G.xr = bs; G.xq = cs; G.s0 = ds; G.s1 = nullptr; G.p0 = ps;

    // ---- 1. entry and read-out chunks, issued ahead of the checkpoint stream
    const Stager<IO, R> stg(G);
    uint4 pre[PRE];
    ScalarRaw sr;
    stage_issue<IO, R, PRE, true>(stg, tid, nthr, pre, sr);

    // ---- 3. publish the staged rows; the three x rows after the last entry are
    // zeroed, so a replay pass of four entries may read past the last one (with a
    // zero coefficient) without touching stale values
    auto publish = [&]() {
        stage_publish<IO, R, PRE>(stg, tid, nthr, pre, sr);
        for (int i = tid; i < HT * 3 * (XS / 4); i += nthr) {
            const int hh = i / (3 * (XS / 4)), r = i - hh * (3 * (XS / 4));
            st4(xs + (size_t)hh * vx * XS + (size_t)(p.V + r / (XS / 4)) * XS + 4 * (r % (XS / 4)), f32x4{0.f, 0.f, 0.f, 0.f});
        }
        __syncthreads();
    };

    // B_j . C for the decode token: per group, so formed once for every head of the
    // workgroup (lane quad jj holds entry f + jj; one token has at most 16 unfolded
    // entries).  Several tokens form theirs per head below.
    auto token_dots = [&]() {
        float d = 0.f;
        const int nr = len - f + 1;
        if (a.mode != MODE_FLUSH && nr > 0) {
            const int jj = lane >> 2, j = f + jj, q = lane & 3;
            if (jj < nr) {
#pragma unroll
                for (int i = 0; i < R / 16; ++i)
                    d += dot4(ld4(bs + j * RS + 16 * i + 4 * q), ld4(cs + 16 * i + 4 * q));
            }
            d = quad_sum(d);
        }
        return d;
    };

    // Replay of the unfolded entries f..pos for one token (TMAX == 1): lane quad jj
    // forms entry f + jj's decayed coefficient into this wave's LDS row; every lane
    // then reads them four at a time (broadcast) against its column of the x rows
    // (fixed row stride: immediate offsets, no index math).  Returns the replay sum;
    // gdec receives the decay of the checkpoint term.
    auto replay1 = [&](const float* psh, const float* dsh, const float* xsh, float Ah, int pos, float dot1,
                       float& gdec) {
        float rep = 0.f;
        const int nr = pos - f + 1;
        const int jj = lane >> 2;
        float* cfw = cf + 16 * w;
        if ((lane & 3) == 0) {
            float c = 0.f;
            if (jj < nr) c = fexp((psh[pos] - psh[f + jj]) * Ah) * dsh[f + jj] * dot1;
            cfw[jj] = c;
        }
        wave_lds_sync();
        const float* xb = xsh + (size_t)f * XS + lc;
#pragma unroll
        for (int e4 = 0; e4 < 16; e4 += 4) {
            if (e4 < nr) {
                const f32x4 c4 = ld4(cfw + e4);
                rep += c4.x * xb[(e4 + 0) * XS] + c4.y * xb[(e4 + 1) * XS] + c4.z * xb[(e4 + 2) * XS] +
                       c4.w * xb[(e4 + 3) * XS];
            }
        }
        // the row is written again for the next head
        wave_lds_sync();
        gdec = fexp((psh[pos] - (f > 0 ? psh[f - 1] : 0.f)) * Ah);
        return rep;
    };

    // ---- 2'. a decode step that folds nothing and reads a read copy (FP8 or MXFP4
    // words) keeps every head's strip in flight at once: the words stay compact
    // until they are consumed by the read-out, so the loads of all HT heads fit the
    // register budget (2 KiB or less per head and wave would otherwise leave too few
    // bytes in flight to cover the memory latency).  Measured on the batch-256
    // layer: fp32 checkpoint with an FP8 copy 0.114 -> 0.100 ms per step, FP8
    // checkpoint with an MXFP4 copy 0.098 -> 0.082 ms; an FP8 checkpoint without a
    // copy gains nothing over the prefetching path below and keeps it.
    constexpr bool COMPACT = TMAX == 1 && HT > 1 && RC != RC_NONE;
    if constexpr (COMPACT) {
        if (a.mode != MODE_FLUSH && f == 0) {
            constexpr int FMT = RC == RC_MXFP4 ? 1 : 0;
            const uint8_t* words = a.rcopy;
            uint32_t raw[HT][NB];
#pragma unroll
            for (int hh = 0; hh < HT; ++hh)
                raw_issue<NB, FMT>(words, a.rscale, (size_t)(b * a.H + h0 + hh) * (C >> 4) + (c0 >> 4) + w, lane,
                                   raw[hh]);
            publish();
            const float dot1 = token_dots();
#pragma unroll
            for (int hh = 0; hh < HT; ++hh) {
                const int h = h0 + hh;
                const float* xsh = xs + (size_t)hh * vx * XS;
                const float Ah = Av[hh];
                float gdec;
                const float rep = replay1(ps + hh * VM, ds + hh * VM, xsh, Ah, len, dot1, gdec);
                f32x4 cvec[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) cvec[nb] = ld4(cs + nb * 16 + rq);
                const float gacc = sum_over_row_groups(raw_dot<NB, FMT>(raw[hh], cvec));
                const float yv = gdec * gacc + rep + Dv[hh] * xsh[len * XS + lc];
                if (lane < 16) st_io<IO>(a.y, ((size_t)b * a.H + h) * C + col, yv);
            }
            return;
        }
    }

    // ---- 2. checkpoint strip loads (128-bit, ckpt.hpp), decoded where first used;
    // a step that folds nothing reads the low-precision copy when there is one (in
    // the kernels with the compact path every such step took that path, and a flush
    // that folds nothing has returned: here f > 0)
    bool from_copy = false;
    if constexpr (RC != RC_NONE && !COMPACT) from_copy = (f == 0);
    auto issue = [&](int hh, f32x4 (&dst)[NB]) {
        const size_t strip = (size_t)(b * a.H + h0 + hh) * (C >> 4) + (c0 >> 4) + w;
        if (from_copy) {
            if constexpr (RC != RC_NONE) rc_issue<NB, RC>(a.rcopy, a.rscale, strip, lane, dst);
        } else {
            ckpt_issue<NB, CK>(a.ckpt, strip, lane, dst);
        }
    };
    // next head's strip in flight during the current head's arithmetic, except in
    // the kernels with the compact path: there this path only serves folding and
    // flush steps, and a single buffer keeps it within the register budget
    constexpr bool PREFETCH = HT > 1 && !COMPACT;
    f32x4 sbuf[PREFETCH ? 2 : 1][NB];
    issue(0, sbuf[0]);

    publish();
    // An fp16 checkpoint without a copy is decoded as soon as it is needed at all:
    // the shorter register life of the raw words keeps the kernel at more waves per
    // SIMD, which beats overlapping the replay terms with the loads.
    constexpr bool EARLY_DECODE = CK == CK_F16 && RC == RC_NONE;

    float dot1 = 0.f;
    if constexpr (TMAX == 1) dot1 = token_dots();
    // Several tokens: the dots B_j . C_t of the unfolded entries j = f .. len + t are
    // per group, so they are formed once for the workgroup (wave w: tokens w, w +
    // waves, ...; lane quad jj: entry f + jj) into an LDS table.
    if constexpr (TMAX > 1) {
        if (a.mode != MODE_FLUSH) {
            const int waves = nthr >> 6, q = lane & 3;
            for (int t = w; t < T; t += waves) {
                const int nr = len + t - f + 1;
                for (int jj0 = 0; jj0 < nr; jj0 += 16) {
                    const int jj = jj0 + (lane >> 2), j = f + jj;
                    float dot = 0.f;
                    if (jj < nr) {
#pragma unroll
                        for (int i = 0; i < R / 16; ++i)
                            dot += dot4(ld4(bs + j * RS + 16 * i + 4 * q), ld4(cs + t * R + 16 * i + 4 * q));
                    }
                    dot = quad_sum(dot);
                    if (q == 0 && jj < nr) gs[t * VM + j] = dot;
                }
            }
            __syncthreads();
        }
    }

#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
        f32x4 (&s)[NB] = sbuf[hh & (PREFETCH ? 1 : 0)];
        if constexpr (PREFETCH) {
            if (hh + 1 < HT) issue(hh + 1, sbuf[(hh + 1) & 1]);
        } else if constexpr (HT > 1) {
            if (hh > 0) issue(hh, s);
        }
        const int h = h0 + hh;
        const size_t strip_index = (size_t)(b * a.H + h) * (C >> 4) + (c0 >> 4) + w;
        const float* dsh = ds + hh * VM;
        const float* psh = ps + hh * VM;
        const float* xsh = xs + (size_t)hh * vx * XS;
        if constexpr (EARLY_DECODE) ckpt_decode<NB, CK>(s);

        const float Ah = Av[hh];

        // ---- 4. fold the first f entries into the checkpoint registers
        // sums of dt over an entry range come from the prefix sums: sum_{lo<=i<hi} = ps[hi-1] - ps[lo-1]
        // (with dt >= 0 and A_h <= 0 every exponent is <= 0 up to the rounding of that difference)
        if (f > 0) {
            if constexpr (!EARLY_DECODE) ckpt_decode<NB, CK>(s);
            const float pf = psh[f - 1];
            const float decay = fexp(pf * Ah);
            if constexpr (MFMA_FOLD) {
                // D[n][p] += sum_i A[n][i] B[i][p] with A = B_i[n] (lane: n = l%16,
                // i = l/16) and B = e^{..} dt_i x_i[p] (lane: i = l/16, p = l%16).
                const int iq = lane >> 4;
                float bop[4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int i = kb * 4 + iq;
                    bop[kb] = (i < f) ? fexp((pf - psh[i]) * Ah) * dsh[i] * xsh[i * XS + lc] : 0.f;
                }
                if constexpr (IO == IO_BF16 && HT > 1) {
                    // bf16 io (four-head kernels; the one-head kernels keep the fp32 product
                    // within their register budget, and their folds are bound by the
                    // checkpoint stream): the B entries are bf16 numbers, and each weight splits into
                    // three bf16 terms (hi + mid + lo, 24 bits), so two 16x16x32 bf16
                    // products per block replace four fp32 ones: exact products, fp32
                    // sums.  Lane group q holds entries 4 kb + q, in the k slots
                    // (hi of the four, mid of the four) and (lo of the four, zeros).
                    uint32_t wh[4], wm[4], wl[4];
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) split3_bf16(bop[kb], wh[kb], wm[kb], wl[kb]);
                    const bf16x8 b1 = bf16x8_pack(wh[0], wh[1], wh[2], wh[3], wm[0], wm[1], wm[2], wm[3]);
                    const bf16x8 b2 = bf16x8_pack(wl[0], wl[1], wl[2], wl[3], 0u, 0u, 0u, 0u);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        uint32_t av[4];
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            const int i = kb * 4 + iq;
                            av[kb] = (i < f) ? (__builtin_bit_cast(uint32_t, bs[i * RS + nb * 16 + (lane & 15)]) >> 16) : 0u;
                        }
                        f32x4 acc = mfma16x16x32bf16(bf16x8_pack(av[0], av[1], av[2], av[3], av[0], av[1], av[2], av[3]),
                                                     b1, f32x4{0.f, 0.f, 0.f, 0.f});
                        acc = mfma16x16x32bf16(bf16x8_pack(av[0], av[1], av[2], av[3], 0u, 0u, 0u, 0u), b2, acc);
                        s[nb] = decay * s[nb] + acc;
                    }
                } else {
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
                }
            } else {
                float wx[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    wx[i] = (i < f) ? fexp((pf - psh[i]) * Ah) * dsh[i] * xsh[i * XS + lc] : 0.f;
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

        // the folded state takes the checkpoint's storage precision at once (fp16:
        // RNE), so this step's outputs and the read copy see the stored values
        if (f > 0) ckpt_round<NB, CK>(s);
        // a checkpoint kept at the copy's precision is rounded as soon as it is folded
        if constexpr (RC != RC_NONE) {
            if (a.qckpt && f > 0) rc_roundtrip<NB, RC>(s, a.mxceil);
        }

        // ---- 5. single checkpoint write on a folding step (before the outputs, which
        // only read the folded values: the encoders' temporaries are dead by the time
        // the read-out rows are loaded)
        if (f > 0) {
            ckpt_store<NB, CK>(a.ckpt, strip_index, lane, s);
            if constexpr (RC != RC_NONE) rc_store<NB, RC>(a.rcopy, a.rscale, strip_index, lane, s, a.mxceil);
        }

        // ---- 6. outputs of the new tokens.  The replay terms of every token come
        // first: they need only LDS, so they run while the checkpoint loads are in
        // flight; then the checkpoint read-outs.
        if (a.mode != MODE_FLUSH) {
            const float Dh = Dv[hh];
            float rep[TMAX], gdec[TMAX];
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                rep[t] = 0.f;
                gdec[t] = 1.f;
                const int pos = len + t;
                if (t < T && pos >= f) {
                    if constexpr (TMAX == 1) {
                        rep[t] = replay1(psh, dsh, xsh, Ah, pos, dot1, gdec[t]);
                    } else {
                        // replay of entries f..pos: lane quad jj = l/4 forms B_j . C_t and the
                        // decayed coefficient; output lanes gather the coefficients by readlane
                        const int nr = pos - f + 1;
                        const float* xcol = xsh + lc;
                        const int pos_u = uni(pos), f_u = uni(f);
                        float r = 0.f;
                        for (int jj0 = 0; jj0 < nr; jj0 += 16) {
                            const int jj = jj0 + (lane >> 2), j = f + jj;
                            const float coef = (jj < nr) ? fexp((psh[pos] - psh[j]) * Ah) * dsh[j] * gs[t * VM + j] : 0.f;
                            // entries past pos carry a zero coefficient; their row is clamped to a
                            // staged one so the product stays finite (row offsets are scalar)
                            // four entries per pass, passes while entries remain (nr is uniform)
                            const int ne = uni(min(nr - jj0, 16));
#pragma unroll
                            for (int e4 = 0; e4 < 16; e4 += 4) {
                                if (e4 < ne) {
#pragma unroll
                                    for (int e = e4; e < e4 + 4; ++e)
                                        r += readlane(coef, 4 * e) * xcol[uni(min(f_u + jj0 + e, pos_u) * XS)];
                                }
                            }
                        }
                        rep[t] = r;
                        gdec[t] = fexp((psh[pos] - (f > 0 ? psh[f - 1] : 0.f)) * Ah);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t < T) {
                    const int pos = len + t;
                    const float xt = xsh[pos * XS + lc];
                    // checkpoint read-out (S' C_t)[col], reduced over the four row groups; one
                    // token reads raw words that were not folded straight into the dot product
                    float gacc = 0.f;
                    if constexpr (TMAX == 1 && !EARLY_DECODE) {
                        // C as the lanes' checkpoint rows need it (rows 4(l/16)..+3 of every block)
                        f32x4 cvec[NB];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) cvec[nb] = ld4(cs + nb * 16 + rq);
                        if (f == 0) {
                            gacc = from_copy ? rc_dot<NB, RC>(s, cvec) : ckpt_dot<NB, CK>(s, cvec);
                        } else {
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb) gacc += dot4(s[nb], cvec[nb]);
                        }
                    } else {
                        // the checkpoint values are needed from here on
                        if (!EARLY_DECODE && t == 0 && f == 0) {
                            if (from_copy) rc_decode<NB, RC>(s);
                            else ckpt_decode<NB, CK>(s);
                        }
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) gacc += dot4(s[nb], ld4(cs + t * R + nb * 16 + rq));
                    }
                    gacc = sum_over_row_groups(gacc);
                    const float yv = (pos >= f) ? gdec[t] * gacc + rep[t] + Dh * xt : gacc + Dh * xt;
                    if (lane < 16) st_io<IO>(a.y, (((size_t)t * sB + b) * a.H + h) * C + col, yv);
                }
            }
        }
    }
}

template <int NB, int IO, int TMAX, bool MF, int RC, int CK, int HT>
static hipError_t mamba2_launch_ht(const StepArgs& a, hipStream_t s)
{
    const size_t Tr = a.T > 0 ? a.T : 1;
    const size_t R = NB * 16;
    const size_t VM = (16 + TMAX + 3) & ~3;
    const size_t lds = sizeof(float) * (HT * ((size_t)a.vmax + 3) * 64 + (size_t)a.vmax * (R + 4) + Tr * R + 64 +
                                        (TMAX > 1 ? Tr * VM : 0) + 2 * HT * VM);
    auto k = mamba2_step_kernel<NB, IO, TMAX, MF, RC, CK, HT>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3(a.B * (a.H / HT) * a.nsplit), dim3(a.C / a.nsplit * 4), lds, s, a);
    return hipGetLastError();
}

// Heads per workgroup: a.ht (set by the host: 4 when four heads share a group and
// the workgroup has four waves, else 1).  The four-head form is built for state
// dimensions 64 and 128 and up to 4 new tokens per step; other launches use one head.
template <int NB, int IO, int TMAX, bool MF, int RC, int CK>
static hipError_t mamba2_launch_nb(const StepArgs& a, hipStream_t s)
{
    if constexpr ((NB == 4 || NB == 8) && TMAX <= 4 && MF) {
        if (a.ht == 4) return mamba2_launch_ht<NB, IO, TMAX, MF, RC, CK, 4>(a, s);
    }
    return mamba2_launch_ht<NB, IO, TMAX, MF, RC, CK, 1>(a, s);
}

template <int IO, int TMAX, bool MF, int RC, int CK>
static hipError_t mamba2_launch_io(const StepArgs& a, hipStream_t s)
{
    switch (a.R) {
        case 16:
            if constexpr (RC != RC_MXFP4) return mamba2_launch_nb<1, IO, TMAX, MF, RC, CK>(a, s);
            return hipErrorInvalidValue;     // MXFP4 groups need 32 rows
        case 32: return mamba2_launch_nb<2, IO, TMAX, MF, RC, CK>(a, s);
        case 64: return mamba2_launch_nb<4, IO, TMAX, MF, RC, CK>(a, s);
        case 128: return mamba2_launch_nb<8, IO, TMAX, MF, RC, CK>(a, s);
        case 256: return mamba2_launch_nb<16, IO, TMAX, MF, RC, CK>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int TMAX, bool MF, int RC, int CK>
static hipError_t mamba2_launch_t(const StepArgs& a, int io, hipStream_t s)
{
    return io == IO_BF16 ? mamba2_launch_io<IO_BF16, TMAX, MF, RC, CK>(a, s) : mamba2_launch_io<IO_F32, TMAX, MF, RC, CK>(a, s);
}

// Dispatch over the draft count (TMAX = 1, 4, 16), read copy and fold flavour
// for checkpoint storage CK; the MFMA fold is the product path, the vector
// fold a cross-check kept for fp32 checkpoints.
template <int TMAX, int CK>
static hipError_t mamba2_launch_tm(const StepArgs& a, int io, int rc, bool valu_fold, hipStream_t s)
{
    if (rc == RC_FP8) return mamba2_launch_t<TMAX, true, RC_FP8, CK>(a, io, s);
    if (rc == RC_MXFP4) return mamba2_launch_t<TMAX, true, RC_MXFP4, CK>(a, io, s);
    if constexpr (CK == CK_F32) {
        if (valu_fold) return mamba2_launch_t<TMAX, false, RC_NONE, CK>(a, io, s);
    }
    return mamba2_launch_t<TMAX, true, RC_NONE, CK>(a, io, s);
}

template <int CK>
static hipError_t mamba2_launch(const StepArgs& a, int io, int rc, bool valu_fold, hipStream_t s)
{
    if (a.T <= 1) return mamba2_launch_tm<1, CK>(a, io, rc, valu_fold, s);
    if (a.T <= 4) return mamba2_launch_tm<4, CK>(a, io, rc, valu_fold, s);
    return mamba2_launch_tm<16, CK>(a, io, rc, valu_fold, s);
}

}  // namespace rs
