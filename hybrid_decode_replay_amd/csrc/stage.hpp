// stage.hpp -- entry staging shared by the replay step kernels.
//
// A launch works on a virtual entry list per sequence: the committed buffer
// entries 0..len-1 followed by the T new tokens.  Each entry has a per-head
// vector (Mamba-2 x, GDN v; C wide), a per-group vector (Mamba-2 B, GDN k;
// R wide) and one or two per-head scalars (Mamba-2 dt; GDN alpha, beta); each
// new token also has a per-group read-out vector (Mamba-2 C, GDN q).  The rows
// are fetched as 16-byte chunks.  stage_issue() puts the first PRE chunks of
// every thread in flight (call it before the checkpoint loads, so that
// consuming the chunks later waits only for them); stage_publish() converts
// them to fp32 in LDS and appends the new entries that stay unfolded to the
// buffer straight from the chunk registers (raw io bits; scalars as fp32).  The
// caller then needs one workgroup barrier.  The append writes slots the launch
// reads from no workgroup: slots >= len of the bank being read, or the other
// bank after a fold.
//
// A workgroup may serve ht consecutive heads h..h+ht-1 of one group: their
// per-head rows and scalars are staged side by side (xc_stride, sc_stride
// floats apart), the group's rows once.
#pragma once
#include "common.hpp"

namespace rs {

struct StageGeom {
    const void* bufc;    // per-head vectors, bank-strided
    const void* bufr;    // per-group vectors
    const float* bufs0;  // per-head scalar 0 (fp32)
    const float* bufs1;  // per-head scalar 1 (fp32) or null
    const void* in_c;
    const void* in_r;
    const void* in_q;
    const void* in_s0;   // io dtype (Mamba-2 dt) or fp32 (GDN alpha)
    const float* in_s1;
    size_t bank_c, bank_r, bank_s;
    size_t hc, gr;       // b*H + h (first head), b*G + g
    int b, h, g, B, H, G, cap, C, len, bank, V, T;
    int c0, cw;          // column slice [c0, c0 + cw) of the per-head vectors this workgroup owns
    int m20_cx;          // magic_div20 of the chunks per per-head row slice (cw / EPC)
    int ht;              // heads staged (h .. h + ht - 1, one group)
    int xc_stride;       // floats between consecutive heads' xc rows
    int xc_row;          // floats between consecutive entries' xc rows (>= cw)
    int sc_stride;       // floats between consecutive heads' scalars (s0, s1, p0)
    // append of the unfolded new entries j >= max(f, len) to bank bank_new at slot
    // j - f, made from the chunk registers as they are published
    int f, bank_new;
    bool head_writer;    // writes the per-head rows' own column slice and the scalars
    bool group_writer;   // writes the per-group rows
    float* xc;           // LDS [ht][vmax][xc_row]
    float* xr;           // LDS [vmax][R + 4]
    float* xq;           // LDS [T][R]
    float* s0;           // LDS [ht][sc_stride]
    float* s1;           // LDS [ht][sc_stride] or null
    float* p0;           // LDS [ht][sc_stride]: inclusive prefix sums of scalar 0, or null
};

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

template <int IO, int R>
struct Stager {
    static constexpr int ES = IO == IO_BF16 ? 2 : 4;
    static constexpr int EPC = 16 / ES;
    static constexpr int RX = R / EPC;
    static constexpr int RS = R + 4;

    const StageGeom& G;
    int CX, nxh, nx, nr, nch;

    __device__ explicit Stager(const StageGeom& g) : G(g) {
        CX = G.cw / EPC;
        nxh = G.V * CX;
        nx = G.ht * nxh;
        nr = G.V * RX;
        nch = nx + nr + G.T * RX;
    }

    // head of a per-head chunk: ht is 1 or at most 4, so compares replace a division
    __device__ int head_of(int ch) const {
        return G.ht == 1 ? 0 : (ch >= nxh) + (ch >= 2 * nxh) + (ch >= 3 * nxh);
    }

    // A chunk's place: kind 0 per-head row (head hh), 1 per-group row, 2 read-out
    // row; entry (or token) j, 16-byte offset o within the row slice.
    struct Ref {
        int kind, hh, j, o;
    };

    __device__ Ref ref(int ch) const {
        Ref c;
        if (ch < nx) {
            c.kind = 0;
            c.hh = head_of(ch);
            const int r = ch - c.hh * nxh;
            c.j = div_small(r, G.m20_cx);
            c.o = r - c.j * CX;
            return c;
        }
        ch -= nx;
        c.hh = 0;
        c.kind = ch < nr ? 1 : 2;
        if (ch >= nr) ch -= nr;
        c.j = ch / RX;
        c.o = ch - c.j * RX;
        return c;
    }

    __device__ const uint4* src(const Ref& c) const {
        size_t e;
        const void* base;
        if (c.kind == 0) {
            if (c.j < G.len) { base = G.bufc; e = (size_t)G.bank * G.bank_c + ((G.hc + c.hh) * G.cap + c.j) * G.C + G.c0; }
            else { base = G.in_c; e = (((size_t)(c.j - G.len) * G.B + G.b) * G.H + G.h + c.hh) * G.C + G.c0; }
        } else if (c.kind == 1) {
            if (c.j < G.len) { base = G.bufr; e = (size_t)G.bank * G.bank_r + (G.gr * G.cap + c.j) * R; }
            else { base = G.in_r; e = (((size_t)(c.j - G.len) * G.B + G.b) * G.G + G.g) * R; }
        } else {
            base = G.in_q;
            e = (((size_t)c.j * G.B + G.b) * G.G + G.g) * R;
        }
        return reinterpret_cast<const uint4*>(static_cast<const char*>(base) + e * ES) + c.o;
    }

    __device__ float* dst(const Ref& c) const {
        if (c.kind == 0) return G.xc + c.hh * G.xc_stride + c.j * G.xc_row + c.o * EPC;
        if (c.kind == 1) return G.xr + c.j * RS + c.o * EPC;
        return G.xq + c.j * R + c.o * EPC;
    }

    // Buffer slot a new entry's chunk is appended to, or null (an entry already in
    // the buffer, a folded one, a read-out row, or a row another workgroup writes).
    __device__ uint4* append_dst(const Ref& c) const {
        const int j0 = max(G.f, G.len);
        if (c.kind == 2 || c.j < j0) return nullptr;
        size_t e;
        void* base;
        if (c.kind == 0) {                  // every workgroup writes its own column slice
            base = const_cast<void*>(G.bufc);
            e = (size_t)G.bank_new * G.bank_c + ((G.hc + c.hh) * G.cap + (c.j - G.f)) * G.C + G.c0;
        } else {
            if (!G.group_writer) return nullptr;
            base = const_cast<void*>(G.bufr);
            e = (size_t)G.bank_new * G.bank_r + (G.gr * G.cap + (c.j - G.f)) * R;
        }
        return reinterpret_cast<uint4*>(static_cast<char*>(base) + e * ES) + c.o;
    }
};

// Raw bits of the per-entry scalars of one thread: head tid / 32, entry tid % 32
// (V <= 32).  They stay unconverted until published, so no conversion makes the
// wave wait for the chunk loads before the checkpoint loads are issued.
struct ScalarRaw {
    uint32_t s0 = 0, s0shift = 0, s1 = 0;
};

template <int IO, int R, int PRE, bool S0_IS_IO>
__device__ __forceinline__ void stage_issue(const Stager<IO, R>& st, int tid, int nthr, uint4 (&pre)[PRE], ScalarRaw& sr)
{
    const StageGeom& G = st.G;
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
        const int ch = tid + u * nthr;
        if (ch < st.nch) pre[u] = *st.src(st.ref(ch));
    }
    // Entry scalars: lanes below len read the buffer, the rest the current inputs
    // (present whenever tokens are appended; with none, V == len).  One load per
    // lane through a selected address: a branch per source would leave a register
    // written on one path and loaded on the other, and the wait that orders the two
    // would hold back the checkpoint loads behind every chunk issued above.
    const int sh = tid >> 5, sj = tid & 31;
    if (sh < G.ht && sj < G.V) {
        const bool buffered = sj < G.len;
        const size_t eb = (size_t)G.bank * G.bank_s + (G.hc + sh) * G.cap + sj;
        const size_t ei = ((size_t)max(sj - G.len, 0) * G.B + G.b) * G.H + G.h + sh;
        if constexpr (S0_IS_IO && IO == IO_BF16) {
            // with bf16 io every buffered value is a bf16 widened to fp32 (low half
            // zero), so its upper half is the bf16 code itself
            const uint16_t* p = buffered ? reinterpret_cast<const uint16_t*>(G.bufs0) + 2 * eb + 1
                                         : static_cast<const uint16_t*>(G.in_s0) + ei;
            sr.s0 = *p;
            sr.s0shift = 16;
        } else {
            const uint32_t* p = buffered ? reinterpret_cast<const uint32_t*>(G.bufs0) + eb
                                         : static_cast<const uint32_t*>(G.in_s0) + ei;
            sr.s0 = *p;
        }
        if (G.bufs1) {
            const uint32_t* p = buffered ? reinterpret_cast<const uint32_t*>(G.bufs1) + eb
                                         : reinterpret_cast<const uint32_t*>(G.in_s1) + ei;
            sr.s1 = *p;
        }
    }
}

template <int IO, int R, int PRE>
__device__ __forceinline__ void stage_publish(const Stager<IO, R>& st, int tid, int nthr, const uint4 (&pre)[PRE],
                                              const ScalarRaw& sr)
{
    const StageGeom& G = st.G;
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
        const int ch = tid + u * nthr;
        if (ch < st.nch) {
            const auto c = st.ref(ch);
            chunk_to_lds<IO>(st.dst(c), pre[u]);
            if (uint4* ap = st.append_dst(c)) *ap = pre[u];
        }
    }
    for (int ch = tid + PRE * nthr; ch < st.nch; ch += nthr) {
        const auto c = st.ref(ch);
        const uint4 v = *st.src(c);
        chunk_to_lds<IO>(st.dst(c), v);
        if (uint4* ap = st.append_dst(c)) *ap = v;
    }
    const int sh = tid >> 5, sj = tid & 31;
    const bool mine = sh < G.ht && sj < G.V;
    if (mine) {
        const float v0 = __builtin_bit_cast(float, sr.s0 << sr.s0shift), v1 = __builtin_bit_cast(float, sr.s1);
        G.s0[sh * G.sc_stride + sj] = v0;
        if (G.s1) G.s1[sh * G.sc_stride + sj] = v1;
        if (G.head_writer && sj >= max(G.f, G.len)) {      // append (buffered scalars are fp32)
            const size_t slot = (size_t)G.bank_new * G.bank_s + (G.hc + sh) * G.cap + (sj - G.f);
            const_cast<float*>(G.bufs0)[slot] = v0;
            if (G.bufs1) const_cast<float*>(G.bufs1)[slot] = v1;
        }
    }
    // entries are at most 32 (cap + T): one head's prefix sums per half wave (a
    // 32-lane scan runs in lanes 0..31 and, independently, in lanes 32..63)
    if (G.p0 && tid < 64 * ((G.ht + 1) >> 1)) {
        const float v = mine ? __builtin_bit_cast(float, sr.s0 << sr.s0shift) : 0.f;
        const float ps = scan32_inclusive(v);
        if (mine) G.p0[sh * G.sc_stride + sj] = ps;
    }
}

// Per-sequence decision shared by every workgroup of sequence b: how many
// leading entries of the virtual list are folded, and the bookkeeping update
// (written by one workgroup into the other copy).  A window holds lim entries
// (cap, or a shorter first window under staggered flushes):
//   decode  len == cap: forced fold of the committed entries first; then the
//           token is appended and a window that reaches lim folds.  With
//           cap == 1 both happen on one step (two folds, fc += 2).
//   flush   fold the len committed entries.
//   spec    len + T > cap: fold the committed prefix before the drafts.
// After a fold the window limit is cap.
// A sequence the step's active mask leaves out (decode and spec only) takes no
// part: nothing is appended, folded or written for it, and its bookkeeping is
// carried into the other copy unchanged (skip; the workgroup then returns).
struct StepPlan {
    int len, fc, f, V, bank, bank_new;
    bool skip;
};

// The current bookkeeping words of sequence b (len, fc, lim).
struct BookWords {
    int len, fc, lim;
};

// The words a step's plan depends on: the sequence's bookkeeping (the copy this
// launch reads; the launch writes only the other) and its active flag.  Scalar
// loads (uload): a kernel may issue its checkpoint loads before it waits for them.
struct PlanInputs {
    BookWords bw;
    bool active;
};

__device__ __forceinline__ BookWords book_words(const StepArgs& a, int b)
{
    const size_t sB = (size_t)a.B;
    const int32_t* bk = a.book + (size_t)a.parity * 4 * sB;
    return BookWords{uload(bk + b), uload(bk + 2 * sB + b), uload(bk + 3 * sB + b)};
}

__device__ __forceinline__ PlanInputs plan_inputs(const StepArgs& a, int b)
{
    PlanInputs q;
    q.bw = book_words(a, b);
    q.active = true;
    if (a.active != nullptr && a.mode != MODE_FLUSH) {
        // the aligned 32-bit word holding the flag byte: a scalar load reads whole
        // words, and an aligned word never spans two pages, so the bytes of it past
        // the end of the mask cannot fault (they are not used)
        const uintptr_t at = reinterpret_cast<uintptr_t>(a.active) + (uintptr_t)b;
        const uint32_t word = uload(reinterpret_cast<const uint32_t*>(at & ~(uintptr_t)3));
        q.active = ((word >> (8 * (at & 3))) & 0xffu) != 0;
    }
    return q;
}

__device__ __forceinline__ StepPlan plan_from(const StepArgs& a, int b, PlanInputs in, bool writer)
{
    const size_t sB = (size_t)a.B;
    const BookWords bw = in.bw;
    StepPlan p;
    p.len = min(max(bw.len, 0), a.cap);  // invariant 0 <= len <= cap; clamped so that a
    p.fc = bw.fc;                        // corrupted word cannot index out of bounds
    const int lim = min(max(bw.lim, 1), a.cap);
    p.skip = !in.active;
    if (p.skip) {
        if (writer) {
            int32_t* nbk = a.book + (size_t)(a.parity ^ 1) * 4 * sB;
            nbk[b] = p.len;
            nbk[sB + b] = 0;
            nbk[2 * sB + b] = p.fc;
            nbk[3 * sB + b] = lim;
        }
        p.f = 0;
        p.V = p.len;
        p.bank = p.bank_new = p.fc & 1;
        return p;
    }
    int folds;
    if (a.mode == MODE_DECODE) {
        if (p.len + 1 > a.cap) {          // forced: the buffer is full
            folds = a.cap == 1 ? 2 : 1;
            p.f = a.cap == 1 ? p.len + 1 : p.len;
        } else {
            folds = p.len + 1 >= lim ? 1 : 0;
            p.f = folds ? p.len + 1 : 0;
        }
    } else if (a.mode == MODE_FLUSH) {
        folds = p.len > 0 ? 1 : 0;
        p.f = p.len;
    } else {
        folds = p.len + a.T > a.cap ? 1 : 0;
        p.f = folds ? p.len : 0;
    }
    p.V = p.len + a.T;
    p.bank = p.fc & 1;
    p.bank_new = (p.fc + folds) & 1;
    if (writer) {
        int32_t* nbk = a.book + (size_t)(a.parity ^ 1) * 4 * sB;
        nbk[b] = (a.mode == MODE_SPEC) ? p.len - p.f : p.len + (a.mode == MODE_DECODE ? 1 : 0) - p.f;
        nbk[sB + b] = (a.mode == MODE_SPEC) ? a.T : 0;
        nbk[2 * sB + b] = p.fc + folds;
        nbk[3 * sB + b] = folds ? a.cap : lim;
    }
    return p;
}

__device__ __forceinline__ StepPlan plan_step(const StepArgs& a, int b, bool writer)
{
    return plan_from(a, b, plan_inputs(a, b), writer);
}

}  // namespace rs
