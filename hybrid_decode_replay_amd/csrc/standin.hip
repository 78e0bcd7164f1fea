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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16x16x32bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- linear ------------------------------------------------------------------
// Workgroup: four waves and an output tile of 64 rows x 32 columns (four 16-row
// by two 16-column MFMA blocks).  The waves split K: wave w takes the 128-wide
// k chunks w, w+4, w+8, ..., so every weight is read by one wave only, and the
// four partial tiles are summed through LDS at the end.  Operand layout of the
// 16x16x32 MFMA: A lane l holds row l%16, k = 8(l/16)..+7; B lane l holds column
// l%16, the same k; the 16x16 result has rows 4(l/16)..+3 of column l%16.  A
// chunk takes four 16-byte loads per operand block per lane; the next chunk's
// loads are issued before the current one is multiplied (two register sets).
// Rows past M read row M-1 and are not stored.
struct LinChunk {
    bf16x8 a[4][4], b[4][2];
};

__device__ __forceinline__ void lin_load(LinChunk& c, const uint16_t* const (&xrow)[4], const uint16_t* const (&wrow)[2],
                                         int k0)
{
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            c.b[u][j] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                                       reinterpret_cast<const u32x4*>(wrow[j] + k0 + 32 * u)));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            c.a[u][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xrow[i] + k0 + 32 * u));
    }
}

__device__ __forceinline__ void lin_mma(const LinChunk& c, f32x4 (&acc)[4][2])
{
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x32bf16(c.a[u][i], c.b[u][j], acc[i][j]);
}

__global__ __launch_bounds__(256) void standin_linear_kernel(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M,
                                                             int K, int N)
{
    __shared__ f32x4 red[3][4][2][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 64;
    const int lr = lane & 15, kq = 8 * (lane >> 4);
    const uint16_t* xrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xrow[i] = X + (size_t)min(m0 + 16 * i + lr, M - 1) * K + kq;
    const uint16_t* wrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) wrow[j] = W + (size_t)(n0 + 16 * j + lr) * K + kq;
    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nch = K / 128;
    LinChunk c0, c1;
    int c = w;
    if (c < nch) lin_load(c0, xrow, wrow, 128 * c);
    while (c < nch) {
        if (c + 4 < nch) lin_load(c1, xrow, wrow, 128 * (c + 4));
        lin_mma(c0, acc);
        c += 4;
        if (c >= nch) break;
        if (c + 4 < nch) lin_load(c0, xrow, wrow, 128 * (c + 4));
        lin_mma(c1, acc);
        c += 4;
    }
    if (w > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) red[w - 1][i][j][lane] = acc[i][j];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const f32x4 v = acc[i][j] + red[0][i][j][lane] + red[1][i][j][lane] + red[2][i][j][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 16 * i + 4 * (lane >> 4) + r;
                if (row < M) Y[(size_t)row * N + n0 + 16 * j + lr] = f32_to_bf16_bits(v[r]);
            }
        }
}

hipError_t launch_standin_linear(const void* X, const void* W, void* Y, int M, int K, int N, hipStream_t s)
{
    hipLaunchKernelGGL(standin_linear_kernel, dim3(N / 32, (M + 63) / 64), dim3(256), 0, s,
                       static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), static_cast<uint16_t*>(Y), M,
                       K, N);
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
