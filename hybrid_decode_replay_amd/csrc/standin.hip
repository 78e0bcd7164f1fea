// standin.hip -- stand-in non-SSM layers of a hybrid model's decode step.
//
// A hybrid model interleaves its SSM layers with a few attention layers, and
// every mixer has dense input and output projections ([TR] "NVIDIA ve Dao AI
// Lab ...", section "ReplaySSM nasil calisir?"); the decode-step speedups the
// pages report are the SSM gain diluted by that rest of the model (section
// "Durum trafigini azaltma ve rollback'in basitlestirilmesi").  These two
// kernels are the rest, with random weights and synthetic caches, so that a
// model step can be timed with replayed and with conventional SSM layers:
//
//   linear     Y[M][N] = X[M][K] . W^T, W stored [N][K] (an output feature's
//              weights contiguous), bf16 in and out, fp32 accumulation on
//              v_mfma_f32_16x16x32_bf16.  At decode batch sizes the weights
//              are streamed once per step: HBM-bound on W.
//   attention  decode attention of one new query token per sequence over a
//              cache of L keys and values (grouped-query heads), bf16 in and
//              out, fp32 softmax; HBM-bound on the cache.
#include "common.hpp"
#include "internal.hpp"

namespace rs {

// ---- linear ------------------------------------------------------------------
// Workgroup: four waves in a 2 x 2 arrangement and an output tile of TM rows x 64
// columns (TM = 128 or 64); wave (wr, wc) owns TM/2 rows and 32 columns, i.e. BI x 2
// MFMA blocks of 16 x 16 (BI = TM / 32).  K advances in chunks of KC (64, 128 or
// 256: at decode batch sizes the launch is bound by the loads in flight, so the
// chunk is as deep as the registers allow): the chunk's X rows (TM x KC) and W rows
// (64 x KC) are copied to LDS once (coalesced 16-byte loads) and every wave reads
// its operands from there, so each X value is fetched from L2 once per workgroup
// and each weight once.  Two chunks are in flight
// while one is multiplied: chunk c+2's global loads are issued into the register
// set chunk c came through, and chunk c+1 (already in registers) is written to the
// other LDS buffer after chunk c's products; one barrier per chunk.  TM = 64 is
// taken when 128-row tiles would leave fewer than 512 workgroups (few output
// columns or a long K per workgroup).  Operand layout of the 16x16x32 MFMA: A lane
// l holds row l%16, k = 8(l/16)..+7; B lane l holds column l%16, the same k; the
// 16x16 result has rows 4(l/16)..+3 of column l%16.  LDS rows are KC + 8 bf16
// long (8 of padding), so consecutive rows of a fragment read start 4 banks apart.
// Rows past M and columns past N read row M-1 / column N-1 and are not stored.
constexpr int LIN_TN = 64;

template <int TM, int LIN_KC>
__global__ __launch_bounds__(256) void standin_linear_kernel(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M,
                                                             int K, int N)
{
    constexpr int LIN_PITCH = LIN_KC + 8;       // padded LDS row (bf16)
    constexpr int PR = LIN_KC / 8;              // 16-byte pieces per row and chunk
    constexpr int BI = TM / 32;                 // row blocks per wave
    constexpr int XU = TM * PR / 256;           // 16-byte X pieces per thread and chunk
    constexpr int WU = LIN_TN * PR / 256;       // 16-byte W pieces per thread and chunk
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][TM * LIN_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t wsh[2][LIN_TN * LIN_PITCH];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr = w >> 1, wc = w & 1;
    const int n0 = blockIdx.x * LIN_TN, m0 = blockIdx.y * TM;
    const int lr = lane & 15, kq = 8 * (lane >> 4);

    // X piece c = tid + 256 u: row c / 8, 16-byte piece c % 8; W piece likewise by column
    const uint16_t* xsrc[XU];
    int xdst[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int c = tid + 256 * u, row = c / PR, pc = c % PR;
        xsrc[u] = X + (size_t)min(m0 + row, M - 1) * K + 8 * pc;
        xdst[u] = row * LIN_PITCH + 8 * pc;
    }
    const uint16_t* wsrc[WU];
    int wdst[WU];
#pragma unroll
    for (int u = 0; u < WU; ++u) {
        const int c = tid + 256 * u, col = c / PR, pc = c % PR;
        wsrc[u] = W + (size_t)min(n0 + col, N - 1) * K + 8 * pc;
        wdst[u] = col * LIN_PITCH + 8 * pc;
    }
    struct Regs {
        u32x4 x[XU], w[WU];
    };
    Regs r0, r1;
    auto load_chunk = [&](Regs& r, int kc) {
        const int k0 = kc * LIN_KC;
#pragma unroll
        for (int u = 0; u < XU; ++u) r.x[u] = *reinterpret_cast<const u32x4*>(xsrc[u] + k0);
#pragma unroll
        for (int u = 0; u < WU; ++u) r.w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[u] + k0));
    };
    auto store_chunk = [&](const Regs& r, int buf) {
#pragma unroll
        for (int u = 0; u < XU; ++u) *reinterpret_cast<u32x4*>(&xs[buf][xdst[u]]) = r.x[u];
#pragma unroll
        for (int u = 0; u < WU; ++u) *reinterpret_cast<u32x4*>(&wsh[buf][wdst[u]]) = r.w[u];
    };

    f32x4 acc[BI][2];
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto multiply = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < LIN_KC / 32; ++ks) {
            bf16x8 a[BI], bb[2];
#pragma unroll
            for (int i = 0; i < BI; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(
                    &xs[buf][((TM / 2) * wr + 16 * i + lr) * LIN_PITCH + 32 * ks + kq]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bb[j] = *reinterpret_cast<const bf16x8*>(&wsh[buf][(32 * wc + 16 * j + lr) * LIN_PITCH + 32 * ks + kq]);
#pragma unroll
            for (int i = 0; i < BI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x32bf16(a[i], bb[j], acc[i][j]);
        }
    };

    // chunk c comes through register set c % 2 and LDS buffer c % 2
    const int nk = K / LIN_KC;
    load_chunk(r0, 0);
    if (nk > 1) load_chunk(r1, 1);
    store_chunk(r0, 0);
    __syncthreads();
    for (int kc = 0; kc < nk; kc += 2) {
        if (kc + 2 < nk) load_chunk(r0, kc + 2);
        multiply(0);
        if (kc + 1 < nk) store_chunk(r1, 1);
        __syncthreads();
        if (kc + 1 >= nk) break;
        if (kc + 3 < nk) load_chunk(r1, kc + 3);
        multiply(1);
        if (kc + 2 < nk) store_chunk(r0, 0);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 32 * wc + 16 * j + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + (TM / 2) * wr + 16 * i + 4 * (lane >> 4) + r;
                if (row < M && col < N) Y[(size_t)row * N + col] = f32_to_bf16_bits(acc[i][j][r]);
            }
        }
}

hipError_t launch_standin_linear(const void* X, const void* W, void* Y, int M, int K, int N, hipStream_t s)
{
    const auto x = static_cast<const uint16_t*>(X);
    const auto w = static_cast<const uint16_t*>(W);
    const auto y = static_cast<uint16_t*>(Y);
    const int cols = (N + LIN_TN - 1) / LIN_TN;
    // Chunk depth: the deepest the register budget allows for the tile, as K permits.
    // Measured at batch 256: 8192 -> 4096 projection 0.095 ms (64-deep chunks) ->
    // 0.059 (128) -> 0.049 ms (256); 4096 -> 18560 0.131 -> 0.123 ms (128).
    if ((long long)cols * ((M + 127) / 128) >= 512) {
        const dim3 grid(cols, (M + 127) / 128);
        if (K % 128 == 0) hipLaunchKernelGGL((standin_linear_kernel<128, 128>), grid, dim3(256), 0, s, x, w, y, M, K, N);
        else hipLaunchKernelGGL((standin_linear_kernel<128, 64>), grid, dim3(256), 0, s, x, w, y, M, K, N);
    } else {
        const dim3 grid(cols, (M + 63) / 64);
        if (K % 256 == 0) hipLaunchKernelGGL((standin_linear_kernel<64, 256>), grid, dim3(256), 0, s, x, w, y, M, K, N);
        else if (K % 128 == 0) hipLaunchKernelGGL((standin_linear_kernel<64, 128>), grid, dim3(256), 0, s, x, w, y, M, K, N);
        else hipLaunchKernelGGL((standin_linear_kernel<64, 64>), grid, dim3(256), 0, s, x, w, y, M, K, N);
    }
    return hipGetLastError();
}

// ---- attention ---------------------------------------------------------------
// One workgroup of four waves per (sequence, key/value head); the QPK query heads
// that share the key/value head are served together.  Wave w takes the 64-token
// chunks w, w+4, w+8, ... of the cache.  Inside a chunk a wave reads 4 tokens per
// instruction: lane l takes token 4u + l/16 and the 8 channels 8(l%16)..+7, so each
// load is four whole 256-byte rows (D = 128); dot products reduce over the 16 lanes
// of a row by DPP.  Online softmax per query head: the chunk's scores go through
// LDS, the wave takes their maximum and rescales its running sum and outputs.  At
// the end the 4 token groups of a wave and then the 4 waves are merged.
template <int D, int QPK>
__global__ __launch_bounds__(256) void standin_attention_kernel(const uint16_t* q, const uint16_t* Kc, const uint16_t* Vc,
                                                                uint16_t* o, int Hkv, int L, size_t q_stride,
                                                                float scale)
{
    static_assert(D == 128, "one 16-lane row of 8 channels each covers the head");
    __shared__ float qs[QPK][D];
    __shared__ float ps[4][64][QPK];
    __shared__ float wm[4][QPK], wl[4][QPK];
    __shared__ float wo[4][QPK][D];
    const int b = blockIdx.x / Hkv, kh = blockIdx.x - b * Hkv;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tg = lane >> 4, ch = 8 * (lane & 15);
    for (int i = tid; i < QPK * D; i += 256) {
        const int h = i / D, d = i - h * D;
        qs[h][d] = bf16_bits_to_f32(q[(size_t)b * q_stride + (size_t)(kh * QPK + h) * D + d]) * scale;
    }
    __syncthreads();
    float qv[QPK][8];
#pragma unroll
    for (int h = 0; h < QPK; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[h][e] = qs[h][ch + e];
    const size_t base = ((size_t)b * Hkv + kh) * L * D;
    const uint16_t* kp = Kc + base;
    const uint16_t* vp = Vc + base;
    float m[QPK], l[QPK], acc[QPK][8];
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    for (int c0 = 64 * w; c0 < L; c0 += 256) {
        const int nt = min(64, L - c0);
        // the chunk's keys and values, 4 tokens per load instruction, all issued up front
        u32x4 kw[16], vw[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = min(4 * u + tg, nt - 1);      // past the cache end: a valid row, never used
            kw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + (size_t)(c0 + t) * D + ch));
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = min(4 * u + tg, nt - 1);
            vw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + (size_t)(c0 + t) * D + ch));
        }
        // scores; the 16 lanes of a row hold the row's sum
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 4 * u + tg;
            float part[QPK];
#pragma unroll
            for (int h = 0; h < QPK; ++h) part[h] = 0.f;
            const uint32_t kk[4] = {kw[u].x, kw[u].y, kw[u].z, kw[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float k0 = bf16_bits_to_f32((uint16_t)(kk[e] & 0xffff));
                const float k1 = bf16_bits_to_f32((uint16_t)(kk[e] >> 16));
#pragma unroll
                for (int h = 0; h < QPK; ++h) part[h] += qv[h][2 * e] * k0 + qv[h][2 * e + 1] * k1;
            }
#pragma unroll
            for (int h = 0; h < QPK; ++h) part[h] = group_sum<16>(part[h]);
            if ((lane & 15) == 0) {
#pragma unroll
                for (int h = 0; h < QPK; ++h) ps[w][t][h] = t < nt ? part[h] : -INFINITY;
            }
        }
        wave_lds_sync();
        // chunk maximum per head (lane = token), new running maximum, probabilities
        float corr[QPK];
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            const float sv = ps[w][lane][h];
            float mx = sv;
#pragma unroll
            for (int o2 = 32; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
            const float mn = fmaxf(m[h], mx);
            corr[h] = __expf(m[h] - mn);
            const float p = lane < nt ? __expf(sv - mn) : 0.f;
            l[h] = l[h] * corr[h] + wave_sum64(p);
            m[h] = mn;
            ps[w][lane][h] = p;
        }
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < QPK; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= corr[h];
        // outputs: lane (token group tg, channels ch..ch+7) accumulates p * v (p = 0 past the end)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 4 * u + tg;
            const uint32_t vv[4] = {vw[u].x, vw[u].y, vw[u].z, vw[u].w};
#pragma unroll
            for (int h = 0; h < QPK; ++h) {
                const float p = ps[w][t][h];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[h][2 * e] += p * bf16_bits_to_f32((uint16_t)(vv[e] & 0xffff));
                    acc[h][2 * e + 1] += p * bf16_bits_to_f32((uint16_t)(vv[e] >> 16));
                }
            }
        }
        wave_lds_sync();
    }
    // merge the wave's 4 token groups (same running maximum), then the 4 waves
#pragma unroll
    for (int h = 0; h < QPK; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = sum_over_row_groups(acc[h][e]);
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < QPK; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) wo[w][h][ch + e] = acc[h][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            wm[w][h] = m[h];
            wl[w][h] = l[h];
        }
    }
    __syncthreads();
    for (int i = tid; i < QPK * D; i += 256) {
        const int h = i / D, d = i - h * D;
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, wm[v][h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float f = wm[v][h] == -INFINITY ? 0.f : __expf(wm[v][h] - mx);
            num += f * wo[v][h][d];
            den += f * wl[v][h];
        }
        o[((size_t)b * Hkv * QPK + (size_t)kh * QPK + h) * D + d] = f32_to_bf16_bits(num / den);
    }
}

hipError_t launch_standin_attention(const void* q, const void* Kc, const void* Vc, void* o, int B, int Hq, int Hkv,
                                    int D, int L, size_t q_stride, float scale, hipStream_t s)
{
    const int qpk = Hq / Hkv;
    const dim3 grid(B * Hkv), block(256);
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(Kc),
                           static_cast<const uint16_t*>(Vc), static_cast<uint16_t*>(o), Hkv, L, q_stride, scale);
    };
    if (D != 128) return hipErrorInvalidValue;
    switch (qpk) {
        case 1: args(standin_attention_kernel<128, 1>); break;
        case 2: args(standin_attention_kernel<128, 2>); break;
        case 4: args(standin_attention_kernel<128, 4>); break;
        case 8: args(standin_attention_kernel<128, 8>); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rs
