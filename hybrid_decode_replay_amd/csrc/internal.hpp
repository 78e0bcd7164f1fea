// internal.hpp -- kernel argument blocks and launchers (library-private).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rs {

enum : int { IO_F32 = 0, IO_BF16 = 1 };
enum : int { RC_NONE = 0, RC_FP8 = 1, RC_MXFP4 = 2 };
enum : int { MODE_DECODE = 0, MODE_FLUSH = 1, MODE_SPEC = 2 };
enum : int { CK_F32 = 0, CK_F16 = 1, CK_FP8 = 2 };   // recurrence checkpoint storage

// Device error word bits (mirror REPLAY_DEVERR_* of the public header).
constexpr uint32_t REPLAY_COMMIT_CLAMPED_BIT = 0x1u;

// The sequences a per-slot load writes, passed by value (kernel arguments), so
// the list a kernel sees is exactly the one the host validated: distinct slots
// in [0, B).  n == 0 means every tile in order (a whole-state load).  Source
// tile i*H + h (i-th listed sequence, head h) lands in tile slot[i]*H + h.
constexpr int SLOT_CHUNK = 256;
struct SlotMap {
    int n;
    int H;
    int32_t slot[SLOT_CHUNK];
};

// Arguments of the replay step kernels (decode, explicit flush, spec append).
// All buffer arrays hold two banks; the bank of a sequence is fc & 1 and a
// flush moves the sequence to the other bank, so the entries a fold reads are
// never overwritten by the same launch.
struct StepArgs {
    int B, H, G, hpg;        // batch, heads, groups, heads per group
    int C, R;                // output axis (P or DV), reduction axis (N or DK)
    int cap;                 // buffer capacity
    int parity;              // which bookkeeping copy is current
    int mode;                // MODE_DECODE / MODE_FLUSH / MODE_SPEC
    int T;                   // new tokens: 1 (decode), k (spec), 0 (flush)
    int vmax;                // LDS rows reserved for the virtual entry list
    int nsplit;              // workgroups per (b, h) tile, along the output axis
    int qckpt;               // nonzero: the checkpoint itself is kept at the copy's precision
    int mxceil;              // nonzero: MXFP4 groups take the non-clipping shared exponent
    int spw;                 // GDN: 16-column strips per wave (1 or 2)
    // launch-invariant divisions by multiplication (div_magic / div_small)
    int cw;                  // columns per workgroup, C / nsplit
    uint32_t mg_nsplit;      // magic_div(nsplit)
    uint32_t mg_tiles;       // magic_div(H / ht): heads served per sequence by the grid
    uint32_t mg_hpg;         // magic_div(hpg)
    int m20_cx;              // magic_div20(cw / elements per 16-byte chunk)
    float scale;             // GDN output scale
    void* ckpt;              // fragment-ordered tiles (fp32 or fp16, ckpt.hpp)
    uint8_t* rcopy;          // read-copy codes (or null)
    uint8_t* rscale;         // MXFP4 scales (or null)
    // buffer banks (element pointers; bank stride in elements)
    void* bufc;              // per-head entry vectors: Mamba-2 x [2][B][H][cap][P]; GDN v [2][B][H][cap][DV]
    void* bufr;              // per-group entry vectors: Mamba-2 B [2][B][G][cap][N]; GDN k [2][B][G][cap][DK]
    float* bufs0;            // per-head scalar: Mamba-2 dt; GDN alpha   [2][B][H][cap]
    float* bufs1;            // per-head scalar: GDN beta (null for Mamba-2)
    size_t bank_c, bank_r, bank_s;
    int32_t* book;           // [2][4][B]: len, pend, fc, lim (length of the current window)
    uint32_t* err;
    // token inputs [T][B][...]
    const void* in_c;        // Mamba-2 x ; GDN v
    const void* in_r;        // Mamba-2 B ; GDN k
    const void* in_q;        // Mamba-2 C ; GDN q
    const void* in_s0;       // Mamba-2 dt (io dtype) ; GDN alpha (fp32)
    const float* in_s1;      // GDN beta (fp32)
    const float* A;          // Mamba-2 A [H]
    const float* D;          // Mamba-2 D [H]
    void* y;                 // outputs [T][B][H][C]
    const uint8_t* active;   // [B] nonzero = the sequence takes part in the step (null = all)
    int ht;                  // heads per workgroup (Mamba-2: 1, 2 or 4; a divisor of hpg)
};

// One translation unit per checkpoint dtype (mamba2.hip / mamba2_f16.hip, ...).
hipError_t launch_mamba2_step_f32(const StepArgs& a, int io, int rc, bool valu_fold, hipStream_t s);
hipError_t launch_mamba2_step_f16(const StepArgs& a, int io, int rc, hipStream_t s);
hipError_t launch_gdn_step_f32(const StepArgs& a, int io, int rc, hipStream_t s);
hipError_t launch_gdn_step_f16(const StepArgs& a, int io, int rc, hipStream_t s);
hipError_t launch_mamba2_step_fp8(const StepArgs& a, int io, int rc, hipStream_t s);
hipError_t launch_gdn_step_fp8(const StepArgs& a, int io, int rc, hipStream_t s);

// Bookkeeping, layout conversion and helpers (aux.hip).
hipError_t launch_book_commit(int32_t* book, uint32_t* err, int B, int parity,
                              const int32_t* accepted, hipStream_t s);
hipError_t launch_book_reset(int32_t* book, uint32_t* err, int B, int parity, int cap, bool stagger, hipStream_t s);
// len = pend = fc = 0 and lim = cap for the listed sequences only (error word untouched).
hipError_t launch_book_reset_slots(int32_t* book, int B, int parity, int cap, const SlotMap& m, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_tiles_to_logical(const void* ckpt, void* out, int tiles, int C, int R, int ck, hipStream_t s);
// Logical source tiles (`tiles` of them, in the checkpoint dtype, or fp32 when
// src_f32 -- then rounded on the device to the checkpoint dtype: binary16 RNE,
// or E4M3 RNE saturating at +-448) into the fragment-ordered checkpoint, at the
// tiles `m` names.
hipError_t launch_logical_to_tiles(const void* in, void* ckpt, int tiles, int C, int R, int ck, bool src_f32,
                                   const SlotMap& m, hipStream_t s);
// Mode bits of the read-copy quantizer.
constexpr int QMODE_ROUND_CKPT = 0x1;   // round the checkpoint to the copy's grid too
constexpr int QMODE_MX_CEIL = 0x2;      // MXFP4: non-clipping shared exponent
hipError_t launch_quantize_read_copy(void* ckpt, uint8_t* codes, uint8_t* scales, int tiles,
                                     int C, int R, int rc, int ck, bool round_ckpt, bool mx_ceil, const SlotMap& m,
                                     hipStream_t s);
hipError_t launch_read_copy_to_logical(const uint8_t* codes, const uint8_t* scales, uint8_t* codes_out,
                                       uint8_t* scales_out, int tiles, int C, int R, int rc, hipStream_t s);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, float* partials, hipStream_t s);

// Conventional baselines (conv.hip).
struct ConvArgs {
    int kind, B, H, G, hpg, C, R, T;
    float scale;
    void* S;                 // logical [B][H][C][R] (fp32 or fp16)
    const void* S_in;        // spec: read-only source
    void* snaps;             // spec: [T][B][H][C][R]
    const void* in_c;
    const void* in_r;
    const void* in_q;
    const void* in_s0;
    const float* in_s1;
    const float* A;
    const float* D;
    void* y;
};
hipError_t launch_conv_step(const ConvArgs& a, int io, int ck, hipStream_t s);
// Stand-in non-SSM layers of a model step (standin.hip).
hipError_t launch_standin_linear(const void* X, const void* W, void* Y, int M, int K, int N, hipStream_t s);
hipError_t launch_standin_attention(const void* q, const void* Kc, const void* Vc, void* o, int B, int Hq, int Hkv,
                                    int D, int L, size_t q_stride, float scale, hipStream_t s);
hipError_t launch_conv_restore(void* S, const void* snaps, const int32_t* accepted, int B, size_t tile_bytes,
                               int H, int k, hipStream_t s);

}  // namespace rs
