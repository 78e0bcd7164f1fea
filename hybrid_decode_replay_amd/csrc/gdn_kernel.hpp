// gdn_kernel.hpp -- replayed Gated DeltaNet decode step for gfx950 (CDNA4).
// Included by one translation unit per checkpoint storage dtype.
//
// Layer: per head, S (d_v x d_k) evolves as S <- alpha S (I - beta k k^T) + beta v k^T
// and o = scale S q (gated delta rule).  The checkpoint tile is fragment-
// ordered (common.hpp) with the reduction axis r = d_k and the output axis
// c = d_v.  The value rows of a head are split over workgroups of at most
// four waves (d_v = 128: two workgroups of 64 rows) so that several
// workgroups share a CU; wave w owns 16 value rows.  Each slice recomputes the
// small per-head quantities (chains, Gram matrix, inverse) itself.
//
// Per launch and sequence the virtual entry list is the committed buffer
// entries followed by the T new tokens; the first f entries are folded into
// the checkpoint (the filling step, [TR] "NVIDIA ve Dao AI Lab ...", section
// "ReplaySSM nasil calisir?"), the rest are replayed on top of it for the
// outputs ([DE] "ReplaySSM beschleunigt das Decoding ...", section "Wie es
// funktioniert": output from the checkpoint plus the buffered inputs).
//
// Output of a token at position pos, by the adjoint chain: r = q; for
// i = pos down to f: c_i = beta_i (k_i . r), r <- alpha_i (r - c_i k_i); then
//     o = scale (S' r + sum_i c_i v_i).
// One checkpoint product per token; the chain needs only the buffered k, alpha,
// beta and costs O(d_k) per entry.  A chain runs on a row of 16 lanes (the
// dot k_i . r reduces inside the row), so it never waits on the checkpoint
// loads.  A single decode token runs its chain in every row of every wave,
// with no workgroup barrier; the drafts of a speculative append get one chain
// each, on separate rows, from the same checkpoint read (output-only
// evaluation, [TR] section "Durum trafigini azaltma ve rollback'in
// basitlestirilmesi").
//
// Fold of entries 0..f-1 in WY form (the intermediate state from small matrix
// products, same section), with P_i = alpha_0 ... alpha_i:
//     W   = K S0^T                       (f x d_v; MFMA, S0 straight from registers)
//     A_ij = beta_i (alpha_{j+1} ... alpha_i) (k_i . k_j)   for j < i
//     U   = (I + A)^{-1} diag(beta) (V - diag(P) W)      (16 x 16 inverse, then MFMA)
//     S'  = P_{f-1} S0 + sum_i (alpha_{i+1} ... alpha_{f-1}) u_i k_i^T   (MFMA)
// Decay factors are formed as products of the gates, never as quotients.
#pragma once
#include "common.hpp"
#include "internal.hpp"
#include "ckpt.hpp"
#include "rc.hpp"
#include "stage.hpp"

namespace rs {

// The lane index recomputed where it is used: the asm is opaque, so the compiler
// can neither merge it with another copy nor keep one copy live across the kernel
// (a value that cheap is better recomputed than held in a register or spilled).
__device__ __forceinline__ int lane_id_here()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Compile-time flag passed to the kernel's generic lambdas.
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Workgroups per CU the register budget is cut for (256 threads each).  The
// one-token two-strip kernels with bf16 io on fp16 and FP8 checkpoints, and on
// fp32 checkpoints with a copy, take five: a fifth wave per SIMD for the steps
// that fold nothing, in 96 VGPRs (their folds form each strip's W, and load each
// fp32 strip, when they fold it; with an MXFP4 copy the FP8 fold keeps one value
// in scratch).
template <int NB, int IO, int TMAX, int RC, int CK, int SPW>
constexpr int gdn_wg_per_cu()
{
    if constexpr (SPW == 1) return NB <= 8 ? 6 : 4;
    const bool five = IO == IO_BF16 && TMAX == 1 && NB <= 8 &&
                      (CK == CK_F16 || CK == CK_FP8 || (CK == CK_F32 && RC != RC_NONE));
    return five ? 5 : 4;
}

template <int NB, int IO, int TMAX, int RC, int CK, int SPW>
__global__ __launch_bounds__(256, (gdn_wg_per_cu<NB, IO, TMAX, RC, CK, SPW>())) void gdn_step_kernel(StepArgs a)
{
    extern __shared__ float lds[];
    constexpr int R = NB * 16;                  // d_k
    constexpr int RS = R + 4;
    constexpr int PRE = 4;
    constexpr int EL = R / 16;                  // chain elements per lane (one row of 16 lanes per chain)
    const int C = a.C;                          // d_v
    const TileIdx tix = tile_of(xcd_tile_index(), a.H, a.mg_tiles, a.nsplit, a.mg_nsplit);
    const int b = tix.b, h = tix.h, tile = b * a.H + h;
    const int g = (int)div_magic((uint32_t)h, a.mg_hpg);
    const int cw = a.cw, c0 = tix.sp * cw;           // this workgroup's output columns
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, waves = nthr >> 6;
    const int rq = 4 * (lane >> 4);
    const int l16 = lane & 15, lq = lane >> 4;
    const size_t sB = (size_t)a.B;
    // wave w owns the SPW strips w*SPW .. w*SPW+SPW-1 of the workgroup's columns
    const int lc0 = 16 * SPW * w + l16;              // local output column of strip 0

    const StepPlan p = plan_step(a, b, h == 0 && tix.sp == 0 && tid == 0);
    if (p.skip || (a.mode == MODE_FLUSH && p.f == 0)) return;
    const int f = p.f, len = p.len, V = p.V, T = a.T;
    const int Tr = T > 0 ? T : 1, vmax = a.vmax;

    // ---- LDS partition (floats)
    float* vs = lds;                          // [vmax][cw]  entry v rows (own columns)
    float* ks = vs + (size_t)vmax * cw;       // [vmax][RS]  entry k rows
    float* qs = ks + (size_t)vmax * RS;       // [Tr][R]     query rows
    float* rz = qs + (size_t)Tr * R;          // chain results r_0: [4][R] per wave (one token), [4][4][R]
                                              // per wave and token (up to four), or [Tr][R] per token
    float* al = rz + (size_t)(TMAX == 1 ? 4 : TMAX <= 4 ? 16 : Tr) * R;   // [vmax] alpha
    float* be = al + vmax;                    // [vmax]      beta
    float* cc = be + vmax;                    // [Tr][vmax]  chain coefficients c_i
    float* ti = cc + (size_t)Tr * vmax;       // [16][17]    (I + A)^{-1}
    float* tt = ti + 16 * 17;                 // [16][17]    gate products over entry ranges

    StageGeom G;
    G.bufc = a.bufc; G.bufr = a.bufr; G.bufs0 = a.bufs0; G.bufs1 = a.bufs1;
    G.in_c = a.in_c; G.in_r = a.in_r; G.in_q = a.in_q; G.in_s0 = a.in_s0; G.in_s1 = a.in_s1;
    G.bank_c = a.bank_c; G.bank_r = a.bank_r; G.bank_s = a.bank_s;
    G.hc = (size_t)b * a.H + h; G.gr = (size_t)b * a.G + g;
    G.b = b; G.h = h; G.g = g; G.B = a.B; G.H = a.H; G.G = a.G; G.cap = a.cap; G.C = C;
    G.c0 = c0; G.cw = cw; G.m20_cx = a.m20_cx;
    G.ht = 1; G.xc_stride = 0; G.xc_row = cw; G.sc_stride = 0;
    G.len = len; G.bank = p.bank; G.V = V; G.T = T;
    G.f = p.f; G.bank_new = p.bank_new; G.head_writer = tix.sp == 0; G.group_writer = tix.sp == 0 && h == g * a.hpg;
    G.xc = vs; G.xr = ks; G.xq = qs; G.s0 = al; G.s1 = be; G.p0 = nullptr;

    // ---- 1. entry chunks ahead of the checkpoint stream, 2. checkpoint strips
    const Stager<IO, R> stg(G);
    uint4 pre[PRE];
    ScalarRaw sr;
    stage_issue<IO, R, PRE, false>(stg, tid, nthr, pre, sr);
    // a step that folds nothing reads the low-precision copy when there is one
    // (loads issued now, decoded where the values are first used)
    const size_t strip0 = (size_t)tile * (C >> 4) + (c0 >> 4) + SPW * w;
    f32x4 s[SPW][NB];
    bool from_copy = false;
    if constexpr (RC != RC_NONE) from_copy = (f == 0);
    // One-token fold steps on an fp32 checkpoint with a copy load strip j > 0 when
    // they fold it, so one fp32 strip is held at a time (the steps that fold nothing
    // read only the copy's words).
    constexpr bool LATE = TMAX == 1 && SPW > 1 && CK == CK_F32 && RC != RC_NONE;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        if (from_copy) {
            if constexpr (RC != RC_NONE) rc_issue<NB, RC>(a.rcopy, a.rscale, strip0 + j, lane, s[j]);
        } else if (!LATE || j == 0) {
            ckpt_issue<NB, CK>(a.ckpt, strip0 + j, lane, s[j]);
        }
    }
    stage_publish<IO, R, PRE>(stg, tid, nthr, pre, sr);
    __syncthreads();

    // ---- 3. fold of the first f entries (WY form on MFMA), in two parts.
    // fold_front: wave 0 forms the gate products and (I + A)^{-1}; every wave forms
    // W = K S0^T for its first strip (one-token steps) or for all its strips; one
    // workgroup barrier.  fold_strip: strip j's
    // S' = P S0 + K^T U~ into `out`.  S0 is read as the registers hold it: decoded
    // fp32 (DEC), or the loaded words decoded block by block (fp16/FP8), so a fold
    // needs no decoded copy of the strips besides its result.
    auto s0_block = [&](auto dec, int j, int jb) -> f32x4 {
        if constexpr (decltype(dec)::value) return s[j][jb];
        else return ckpt_block<NB, CK>(s[j], jb);
    };
    // With bf16 io the entry keys are bf16 numbers, so the Gram matrix, W and the
    // update take the 16x16x32 bf16 product: exact products summed in fp32 like the
    // fp32 product's.  The other operand is a bf16 number (an FP8 checkpoint's
    // values) or split into two (fp16) or three (fp32) bf16 terms.  For key chunk m
    // (32 keys) lane group q holds keys 32m + 4q + 0..3 and 32m + 16 + 4q + 0..3,
    // the rows of checkpoint blocks 2m and 2m+1 it holds.
    constexpr bool BFK = IO == IO_BF16 && R % 32 == 0;
    // key chunk m of entry row l16 (zero past the folded entries)
    auto key_chunk = [&](int m) {
        const bool arow = l16 < f;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        return bf16x8_exact(arow ? ld4(ks + l16 * RS + 32 * m + rq) : z,
                            arow ? ld4(ks + l16 * RS + 32 * m + 16 + rq) : z);
    };
    // W[i][v] = (S0 k_i)[v] of strip j; lane result rows i = lq*4 + r, column lc0 + 16 j
    auto w_of = [&](auto dec, int j) __attribute__((always_inline)) -> f32x4 {
        f32x4 Wj = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BFK) {
#pragma unroll
            for (int m = 0; m < R / 32; ++m) {
                const bf16x8 km = key_chunk(m);
                const f32x4 sa = s0_block(dec, j, 2 * m), sb = s0_block(dec, j, 2 * m + 1);
                if constexpr (CK == CK_FP8) {
                    Wj = mfma16x16x32bf16(km, bf16x8_exact(sa, sb), Wj);
                } else {
                    // fp16 values are hi + mid exactly (11 bits); fp32 values take lo too
                    uint32_t h[8], md[8], lo[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        split3_bf16(sa[e], h[e], md[e], lo[e]);
                        split3_bf16(sb[e], h[4 + e], md[4 + e], lo[4 + e]);
                    }
                    Wj = mfma16x16x32bf16(km, bf16x8_pack(h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]), Wj);
                    Wj = mfma16x16x32bf16(km, bf16x8_pack(md[0], md[1], md[2], md[3], md[4], md[5], md[6], md[7]), Wj);
                    if constexpr (CK == CK_F32)
                        Wj = mfma16x16x32bf16(km, bf16x8_pack(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]),
                                              Wj);
                }
            }
        } else {
            const bool arow = l16 < f;
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                const f32x4 kv = arow ? ld4(ks + l16 * RS + jb * 16 + rq) : f32x4{0.f, 0.f, 0.f, 0.f};
                const f32x4 sv = s0_block(dec, j, jb);
                Wj = mfma16x16x4(kv.x, sv.x, Wj);
                Wj = mfma16x16x4(kv.y, sv.y, Wj);
                Wj = mfma16x16x4(kv.z, sv.z, Wj);
                Wj = mfma16x16x4(kv.w, sv.w, Wj);
            }
        }
        return Wj;
    };
    // fold_front forms W of every strip (all) or of strip 0 only while wave 0 works;
    // one-token steps form the other strips' W when they fold them, so no W is held
    // across another strip's fold.
    auto fold_front = [&](auto dec, auto all, f32x4 (&W)[SPW]) {
        const bool arow = l16 < f;
        if (w == 0) {
            // gate products tt[j][i] = alpha_{j+1} ... alpha_i (1 for i <= j), i, j < f:
            // lane j multiplies along i, every product formed as a product
            if (lane < 16) {
                float pr = 1.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (i > lane && i < f) pr *= al[i];
                    tt[lane * 17 + i] = pr;
                }
            }
            // Gram k_i . k_j on MFMA (lane result rows i = lq*4 + r, column j = l16)
            f32x4 gm = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BFK) {
#pragma unroll
                for (int m = 0; m < R / 32; ++m) {
                    const bf16x8 km = key_chunk(m);
                    gm = mfma16x16x32bf16(km, km, gm);
                }
            } else {
#pragma unroll
                for (int d = 0; d < R / 4; ++d) {
                    const float kv = arow ? ks[l16 * RS + 4 * d + lq] : 0.f;
                    gm = mfma16x16x4(kv, kv, gm);
                }
            }
            wave_lds_sync();
            // strictly lower triangle of A, written to ti as a scratch matrix
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = lq * 4 + r, jj = l16;
                const float v = (jj < i && i < f) ? be[i] * tt[jj * 17 + i] * gm[r] : 0.f;
                ti[i * 17 + jj] = v;
            }
            wave_lds_sync();
            // column c of (I + A)^{-1} by forward substitution (lanes 0..15)
            float tc[16];
            if (lane < 16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float acc = (i == lane) ? 1.f : 0.f;
#pragma unroll
                    for (int jj = 0; jj < i; ++jj) acc -= ti[i * 17 + jj] * tc[jj];
                    tc[i] = acc;
                }
            }
            // all reads of the scratch matrix are done before it is overwritten
            wave_lds_sync();
            if (lane < 16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) ti[i * 17 + lane] = tc[i];
            }
        }
#pragma unroll
        for (int j = 0; j < (decltype(all)::value ? SPW : 1); ++j) W[j] = w_of(dec, j);
        __syncthreads();
    };
    auto fold_strip = [&](auto dec, int j, const f32x4& Wj, f32x4 (&out)[NB]) {
        const float decay = al[0] * tt[f - 1];                       // P_{f-1}
        // rhs[i][v] = beta_i (v_i[v] - P_i W[i][v]) for i < f
        f32x4 rhs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = lq * 4 + r;
            float v = 0.f;
            if (i < f) v = be[i] * (vs[i * cw + 16 * (SPW * w + j) + (lane_id_here() & 15)] - (al[0] * tt[i]) * Wj[r]);
            rhs[r] = v;
        }
        // U = (I + A)^{-1} rhs, then scaled by the decay from entry i to the end of the fold
        f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) U = mfma16x16x4(ti[l16 * 17 + lq * 4 + r], rhs[r], U);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = lq * 4 + r;
            U[r] = (i < f) ? tt[i * 17 + f - 1] * U[r] : 0.f;         // alpha_{i+1} ... alpha_{f-1}
        }
        // S'^T[jk][v] = decay S0^T[jk][v] + sum_i K[i][jk] U~[i][v]
        if constexpr (BFK) {
            // the keys are bf16 numbers and U~ splits into three bf16 terms (hi + mid
            // + lo), so two 16x16x32 bf16 products per block replace four fp32 ones:
            // lane group q holds entries 4q..4q+3 twice, against (hi, mid) and (lo, 0)
            uint32_t uh[4], um[4], ul[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split3_bf16(U[r], uh[r], um[r], ul[r]);
            const bf16x8 b1 = bf16x8_pack(uh[0], uh[1], uh[2], uh[3], um[0], um[1], um[2], um[3]);
            const bf16x8 b2 = bf16x8_pack(ul[0], ul[1], ul[2], ul[3], 0u, 0u, 0u, 0u);
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                uint32_t kv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = lq * 4 + r;                        // rows past f are inside ks
                    const uint32_t raw = __builtin_bit_cast(uint32_t, ks[i * RS + jb * 16 + l16]);
                    kv[r] = (i < f) ? (raw >> 16) : 0u;
                }
                const bf16x8 ka = bf16x8_pack(kv[0], kv[1], kv[2], kv[3], kv[0], kv[1], kv[2], kv[3]);
                f32x4 acc = mfma16x16x32bf16(ka, b1, f32x4{0.f, 0.f, 0.f, 0.f});
                acc = mfma16x16x32bf16(ka, b2, acc);
                out[jb] = decay * s0_block(dec, j, jb) + acc;
            }
        } else {
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = lq * 4 + r;
                    const float kv = (i < f) ? ks[i * RS + jb * 16 + l16] : 0.f;
                    acc = mfma16x16x4(kv, U[r], acc);
                }
                out[jb] = decay * s0_block(dec, j, jb) + acc;
            }
        }
        // the folded state takes the checkpoint's storage precision at once (fp16:
        // RNE), so this step's outputs and the read copy see the stored values
        ckpt_round<NB, CK>(out);
        // a checkpoint kept at the copy's precision is rounded as soon as it is folded
        if constexpr (RC != RC_NONE) {
            if (a.qckpt) rc_roundtrip<NB, RC>(out, a.mxceil);
        }
    };

    // ---- 4./5. adjoint chains and outputs.  A chain runs on one row of 16 lanes:
    // lane j of the row holds elements EL*j .. EL*j+EL-1 of r (EL = d_k / 16), so
    // k_i . r reduces inside the row by DPP, with no cross-row step or readlane.
    // The gates are kept out of the vector update: with r = sig * rr and sig the
    // product of the gates of the entries already passed, c_i = sig beta_i (k_i . rr)
    // and rr <- rr - beta_i (k_i . rr) k_i, then sig <- alpha_i sig; r_0 = sig rr.
    const int rho = lane >> 4, j16 = lane & 15;
    if constexpr (TMAX == 1) {
        // One token.  Its chain needs only the published entries, so it runs first,
        // while the checkpoint loads land: every row of every wave runs it (no
        // workgroup barrier) and keeps the replay sums sum_i c_i v_i of its lanes'
        // columns; r_0 goes to a wave-private LDS row.  Then each strip is folded
        // (if this step folds), stored and read out in turn.
        float rep[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j) rep[j] = 0.f;
        float* rw = rz + (size_t)w * R;
        if (a.mode != MODE_FLUSH) {
            // With d_k >= 64 the chain is spread over the whole wave (lane l holds
            // elements EW*l .. EW*l+EW-1 of r, the dot reduced over the row and then the
            // four rows): a quarter of the per-entry multiply-adds of a 16-lane row,
            // for two more reduction steps.
            constexpr int EW = R >= 64 ? R / 64 : EL;
            constexpr int NL = R >= 64 ? 64 : 16;
            const int li = R >= 64 ? lane : j16;
            float r[EW];
            lds_row_load<EW>(qs + EW * li, r);
            float sig = 1.f;
            const float* vcol = vs + lc0;
            for (int i = len; i >= f; --i) {
                float kv[EW];
                lds_row_load<EW>(ks + i * RS + EW * li, kv);
                float part = 0.f;
#pragma unroll
                for (int m = 0; m < EW; ++m) part += kv[m] * r[m];
                part = group_sum<16>(part);
                if constexpr (NL == 64) part = sum_over_row_groups(part);
                const float bd = be[i] * part;
                const float cf = sig * bd;
#pragma unroll
                for (int j = 0; j < SPW; ++j) rep[j] += cf * vcol[i * cw + 16 * j];
#pragma unroll
                for (int m = 0; m < EW; ++m) r[m] -= bd * kv[m];
                sig *= al[i];
            }
#pragma unroll
            for (int m = 0; m < EW; ++m) r[m] *= sig;
            // r_0 of this wave -> wave-private LDS row
            if (NL == 64 || rho == 0) lds_row_store<EW>(rw + EW * li, r);
            wave_lds_sync();
        }
        auto emit = [&](int j, float gacc) {
            gacc = sum_over_row_groups(gacc);
            if (lane < 16) st_io<IO>(a.y, ((size_t)b * a.H + h) * C + c0 + lc0 + 16 * j, a.scale * (gacc + rep[j]));
        };
        if (f > 0) {
            f32x4 W[SPW];
            fold_front(BoolTag<false>{}, BoolTag<false>{}, W);
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                if (LATE && j > 0) ckpt_issue<NB, CK>(a.ckpt, strip0 + j, lane, s[j]);
                const f32x4 Wj = j == 0 ? W[0] : w_of(BoolTag<false>{}, j);
                auto finish = [&](f32x4 (&sn)[NB]) {
                    // single checkpoint write, then the read-out of the stored values
                    ckpt_store<NB, CK>(a.ckpt, strip0 + j, lane, sn);
                    if constexpr (RC != RC_NONE) rc_store<NB, RC>(a.rcopy, a.rscale, strip0 + j, lane, sn, a.mxceil);
                    if (a.mode != MODE_FLUSH) {
                        float gacc = 0.f;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) gacc += dot4(sn[nb], ld4(rw + nb * 16 + rq));
                        emit(j, gacc);
                    }
                };
                if constexpr (CK == CK_F32) {
                    fold_strip(BoolTag<true>{}, j, Wj, s[j]);        // in place: block jb is read before written
                    finish(s[j]);
                } else {
                    f32x4 sn[NB];
                    fold_strip(BoolTag<false>{}, j, Wj, sn);
                    finish(sn);
                }
            }
        } else if (a.mode != MODE_FLUSH) {
            // raw words that were not folded go straight into the dot product
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                f32x4 rv[NB];                 // r_0 as the lanes' checkpoint rows need it
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) rv[nb] = ld4(rw + nb * 16 + rq);
                emit(j, from_copy ? rc_dot<NB, RC>(s[j], rv) : ckpt_dot<NB, CK>(s[j], rv));
            }
        }
    } else if constexpr (TMAX <= 4) {
        // Up to four tokens: row rho of every wave runs token rho's chain itself (no
        // workgroup barrier), keeping that token's replay sums for the row's columns;
        // r_0 of each token goes to the wave's own LDS rows.  A lane (row rho, column
        // c) then owns the output of token rho at column c.  The chains need only the
        // published entries, so they run while the checkpoint loads land.
        float rep[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j) rep[j] = 0.f;
        float* rzw = rz + (size_t)w * 4 * R;
        if (a.mode != MODE_FLUSH) {
            if (rho < T) {
                float r[EL];
                lds_row_load<EL>(qs + rho * R + EL * j16, r);
                float sig = 1.f;
                const float* vcol = vs + lc0;
                for (int i = len + rho; i >= f; --i) {
                    float kv[EL];
                    lds_row_load<EL>(ks + i * RS + EL * j16, kv);
                    float part = 0.f;
#pragma unroll
                    for (int m = 0; m < EL; ++m) part += kv[m] * r[m];
                    const float bd = be[i] * group_sum<16>(part);
                    const float cf = sig * bd;
#pragma unroll
                    for (int j = 0; j < SPW; ++j) rep[j] += cf * vcol[i * cw + 16 * j];
#pragma unroll
                    for (int m = 0; m < EL; ++m) r[m] -= bd * kv[m];
                    sig *= al[i];
                }
#pragma unroll
                for (int m = 0; m < EL; ++m) r[m] *= sig;
                lds_row_store<EL>(rzw + rho * R + EL * j16, r);
            }
            wave_lds_sync();
        }
        if (f > 0) {
#pragma unroll
            for (int j = 0; j < SPW; ++j) ckpt_decode<NB, CK>(s[j]);
            f32x4 W[SPW];
            fold_front(BoolTag<true>{}, BoolTag<true>{}, W);
#pragma unroll
            for (int j = 0; j < SPW; ++j) fold_strip(BoolTag<true>{}, j, W[j], s[j]);
        }
        if (a.mode != MODE_FLUSH) {
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                if (f == 0) {
                    if (from_copy) rc_decode<NB, RC>(s[j]);
                    else ckpt_decode<NB, CK>(s[j]);
                }
                float mine = 0.f;
#pragma unroll
                for (int t = 0; t < TMAX; ++t) {
                    if (t < T) {
                        float gacc = 0.f;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) gacc += dot4(s[j][nb], ld4(rzw + t * R + nb * 16 + rq));
                        gacc = sum_over_row_groups(gacc);
                        if (rho == t) mine = gacc;
                    }
                }
                if (rho < T)
                    st_io<IO>(a.y, (((size_t)rho * sB + b) * a.H + h) * C + c0 + lc0 + 16 * j, a.scale * (mine + rep[j]));
            }
        }
        if (f > 0) {
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                ckpt_store<NB, CK>(a.ckpt, strip0 + j, lane, s[j]);
                if constexpr (RC != RC_NONE) rc_store<NB, RC>(a.rcopy, a.rscale, strip0 + j, lane, s[j], a.mxceil);
            }
        }
    } else {
        // Several tokens: the strips are decoded once, folded in place, read out by
        // every token, then stored.
        if (f > 0) {
#pragma unroll
            for (int j = 0; j < SPW; ++j) ckpt_decode<NB, CK>(s[j]);
            f32x4 W[SPW];
            fold_front(BoolTag<true>{}, BoolTag<true>{}, W);
#pragma unroll
            for (int j = 0; j < SPW; ++j) fold_strip(BoolTag<true>{}, j, W[j], s[j]);
        }
        if (a.mode != MODE_FLUSH) {
            // one chain per (wave, row) pair; coefficients and r_0 go through LDS to
            // the output lanes
            for (int t = w * 4 + rho; t < T; t += waves * 4) {
                const int pos = len + t;
                float r[EL];
                lds_row_load<EL>(qs + t * R + EL * j16, r);
                float sig = 1.f;
                for (int i = pos; i >= f; --i) {
                    float kv[EL];
                    lds_row_load<EL>(ks + i * RS + EL * j16, kv);
                    float part = 0.f;
#pragma unroll
                    for (int m = 0; m < EL; ++m) part += kv[m] * r[m];
                    const float bd = be[i] * group_sum<16>(part);
#pragma unroll
                    for (int m = 0; m < EL; ++m) r[m] -= bd * kv[m];
                    if (j16 == 0) cc[t * vmax + i] = sig * bd;
                    sig *= al[i];
                }
#pragma unroll
                for (int m = 0; m < EL; ++m) r[m] *= sig;
                lds_row_store<EL>(rz + t * R + EL * j16, r);
            }
            __syncthreads();

            // o_t = scale (S' r_0 + sum_i c_i v_i)
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                if (f == 0) {
                    if (from_copy) rc_decode<NB, RC>(s[j]);
                    else ckpt_decode<NB, CK>(s[j]);
                }
                const int lcj = lc0 + 16 * j;
#pragma unroll
                for (int t = 0; t < TMAX; ++t) {
                    if (t < T) {
                        float gacc = 0.f;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) gacc += dot4(s[j][nb], ld4(rz + t * R + nb * 16 + rq));
                        gacc = sum_over_row_groups(gacc);
                        const int pos = len + t;
                        float rep = 0.f;
                        for (int i = f; i <= pos; ++i) rep += cc[t * vmax + i] * vs[i * cw + lcj];
                        if (lane < 16)
                            st_io<IO>(a.y, (((size_t)t * sB + b) * a.H + h) * C + c0 + lcj, a.scale * (gacc + rep));
                    }
                }
            }
        }

        // ---- 6. single checkpoint write on a folding step
        if (f > 0) {
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                ckpt_store<NB, CK>(a.ckpt, strip0 + j, lane, s[j]);
                if constexpr (RC != RC_NONE) rc_store<NB, RC>(a.rcopy, a.rscale, strip0 + j, lane, s[j], a.mxceil);
            }
        }
    }
}

template <int NB, int IO, int TMAX, int RC, int CK, int SPW>
static hipError_t gdn_launch_spw(const StepArgs& a, hipStream_t s)
{
    const size_t Tr = a.T > 0 ? a.T : 1;
    const size_t R = NB * 16, vmax = a.vmax;
    const size_t rzr = TMAX == 1 ? 4 : TMAX <= 4 ? 16 : Tr;
    const size_t lds = sizeof(float) * (vmax * (a.C / a.nsplit + R + 4) + Tr * R + rzr * R + 2 * vmax +
                                        Tr * vmax + 2 * 16 * 17);
    auto k = gdn_step_kernel<NB, IO, TMAX, RC, CK, SPW>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3(a.B * a.H * a.nsplit), dim3(a.C / a.nsplit / SPW * 4), lds, s, a);
    return hipGetLastError();
}

template <int NB, int IO, int TMAX, int RC, int CK>
static hipError_t gdn_launch_nb(const StepArgs& a, hipStream_t s)
{
    if constexpr (NB == 8) {
        if (a.spw == 2) return gdn_launch_spw<NB, IO, TMAX, RC, CK, 2>(a, s);
    }
    if (a.spw != 1) return hipErrorInvalidValue;
    return gdn_launch_spw<NB, IO, TMAX, RC, CK, 1>(a, s);
}

template <int IO, int TMAX, int RC, int CK>
static hipError_t gdn_launch_io(const StepArgs& a, hipStream_t s)
{
    switch (a.R) {
        case 16:
            if constexpr (RC != RC_MXFP4) return gdn_launch_nb<1, IO, TMAX, RC, CK>(a, s);
            return hipErrorInvalidValue;     // MXFP4 groups need 32 rows
        case 32: return gdn_launch_nb<2, IO, TMAX, RC, CK>(a, s);
        case 64: return gdn_launch_nb<4, IO, TMAX, RC, CK>(a, s);
        case 128: return gdn_launch_nb<8, IO, TMAX, RC, CK>(a, s);
        case 256: return gdn_launch_nb<16, IO, TMAX, RC, CK>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int TMAX, int RC, int CK>
static hipError_t gdn_launch_t(const StepArgs& a, int io, hipStream_t s)
{
    return io == IO_BF16 ? gdn_launch_io<IO_BF16, TMAX, RC, CK>(a, s) : gdn_launch_io<IO_F32, TMAX, RC, CK>(a, s);
}

template <int TMAX, int CK>
static hipError_t gdn_launch_tm(const StepArgs& a, int io, int rc, hipStream_t s)
{
    if (rc == RC_FP8) return gdn_launch_t<TMAX, RC_FP8, CK>(a, io, s);
    if (rc == RC_MXFP4) return gdn_launch_t<TMAX, RC_MXFP4, CK>(a, io, s);
    return gdn_launch_t<TMAX, RC_NONE, CK>(a, io, s);
}

template <int CK>
static hipError_t gdn_launch(const StepArgs& a, int io, int rc, hipStream_t s)
{
    if (a.T <= 1) return gdn_launch_tm<1, CK>(a, io, rc, s);
    if (a.T <= 4) return gdn_launch_tm<4, CK>(a, io, rc, s);
    return gdn_launch_tm<16, CK>(a, io, rc, s);
}

}  // namespace rs
