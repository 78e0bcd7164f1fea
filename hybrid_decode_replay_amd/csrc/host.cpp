// host.cpp -- the C ABI (include/replayssm.h): validation, state layout,
// phase tracking, kernel selection and launch.  No call synchronizes.
#include "../../include/replayssm.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.hpp"

struct replay_state {
    replay_config cfg;
    uint8_t* mem;
    size_t bytes;
    replay_layout lay;
    int parity;   // bookkeeping copy that holds the current values
    int phase;    // 0 idle, 1 drafts pending
    replay_stack* stack = nullptr;   // set while bound to a stack (which then owns the bookkeeping)
    bool needs_load = false;         // a former stack member: its own bookkeeping is stale
};

// Layers of one model share one bookkeeping set (layer 0's region).  A model
// step runs every layer once, in order; `next` is the layer it expects.
struct replay_stack {
    std::vector<replay_state*> layers;
    int32_t* book;
    uint32_t* err;
    int parity = 0;
    int phase = 0;    // 0 idle, 1 drafts pending
    int next = 0;     // next layer of the current step (0 between steps)
    int step_mode = -1;
    int step_k = 0;
    const uint8_t* step_active = nullptr;   // the active mask every layer of the step uses
};

namespace {

thread_local std::string g_err;

replay_status fail(replay_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
replay_status fail(replay_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

replay_status ok()
{
    g_err.clear();
    return REPLAY_OK;
}

replay_status hip_check(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(REPLAY_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Clears an error an earlier, unrelated HIP call may have left behind, so that
// the hipGetLastError a launcher returns reports its own launch only.
hipError_t fresh() { return hipGetLastError(); }

// hip_check of a launch expression, after clearing any stale error (the comma
// operator sequences the clearing before the launch).
#define LAUNCH(expr, what) hip_check(((void)fresh(), (expr)), what)

rs::SlotMap all_tiles(int H)
{
    rs::SlotMap m;
    m.n = 0;
    m.H = H;
    return m;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int io_bytes(const replay_config* c) { return c->io_dtype == REPLAY_BF16 ? 2 : 4; }
int ckpt_bytes(const replay_config* c)
{
    return c->ckpt_dtype == REPLAY_F16 ? 2 : (c->ckpt_dtype == REPLAY_FP8_E4M3 ? 1 : 4);
}
int ck_kind(const replay_config* c)
{
    return c->ckpt_dtype == REPLAY_F16 ? rs::CK_F16 : (c->ckpt_dtype == REPLAY_FP8_E4M3 ? rs::CK_FP8 : rs::CK_F32);
}

replay_status check_config(const replay_config* c)
{
    if (!c) return fail(REPLAY_ERR_ARG, "config is NULL");
    if (c->abi_version != REPLAY_ABI_VERSION)
        return fail(REPLAY_ERR_ARG, "abi_version %d, library implements %d", c->abi_version, REPLAY_ABI_VERSION);
    if (c->kind != REPLAY_MAMBA2 && c->kind != REPLAY_GDN) return fail(REPLAY_ERR_ARG, "unknown kind %d", c->kind);
    if (c->batch < 1 || c->nheads < 1 || c->ngroups < 1)
        return fail(REPLAY_ERR_SHAPE, "batch, nheads and ngroups must be >= 1");
    if (c->nheads % c->ngroups != 0) return fail(REPLAY_ERR_SHAPE, "ngroups %d does not divide nheads %d", c->ngroups, c->nheads);
    if (c->head_dim < 16 || c->head_dim > 256 || c->head_dim % 16 != 0)
        return fail(REPLAY_ERR_SHAPE, "head_dim %d must be a multiple of 16 in [16, 256]", c->head_dim);
    const int R = c->state_dim;
    if (R != 16 && R != 32 && R != 64 && R != 128 && R != 256)
        return fail(REPLAY_ERR_SHAPE, "state_dim %d must be 16, 32, 64, 128 or 256", R);
    if (c->buf_cap < 1 || c->buf_cap > REPLAY_MAX_BUF)
        return fail(REPLAY_ERR_SHAPE, "buf_cap %d must be in [1, %d]", c->buf_cap, REPLAY_MAX_BUF);
    // the kernels split work item indices by multiplication (exact while index * divisor < 2^32)
    if ((long long)c->batch * c->nheads * (c->nheads > 256 ? c->nheads : 256) >= (1LL << 32))
        return fail(REPLAY_ERR_SHAPE, "batch * nheads * max(nheads, 256) must be below 2^32");
    if (c->io_dtype != REPLAY_F32 && c->io_dtype != REPLAY_BF16)
        return fail(REPLAY_ERR_DTYPE, "io_dtype must be REPLAY_F32 or REPLAY_BF16");
    if (c->ckpt_dtype != REPLAY_F32 && c->ckpt_dtype != REPLAY_F16 && c->ckpt_dtype != REPLAY_FP8_E4M3)
        return fail(REPLAY_ERR_DTYPE, "ckpt_dtype must be REPLAY_F32, REPLAY_F16 or REPLAY_FP8_E4M3");
    if (c->ckpt_dtype == REPLAY_FP8_E4M3 && c->read_copy == REPLAY_FP8_E4M3)
        return fail(REPLAY_ERR_UNSUPPORTED, "an FP8 checkpoint takes no FP8 read copy (it is one)");
    if (c->read_copy != REPLAY_NONE && c->read_copy != REPLAY_FP8_E4M3 && c->read_copy != REPLAY_MXFP4)
        return fail(REPLAY_ERR_DTYPE, "read_copy must be NONE, FP8_E4M3 or MXFP4");
    if (c->read_copy == REPLAY_MXFP4 && R % 32 != 0)
        return fail(REPLAY_ERR_SHAPE, "MXFP4 read copy needs state_dim divisible by 32");
    if (c->flags & ~(REPLAY_FLAG_VALU_FOLD | REPLAY_FLAG_QUANTIZED_CKPT | REPLAY_FLAG_STAGGER_FLUSH |
                     REPLAY_FLAG_MX_SCALE_CEIL))
        return fail(REPLAY_ERR_ARG, "unknown flags 0x%x", c->flags);
    if ((c->flags & REPLAY_FLAG_MX_SCALE_CEIL) && c->read_copy != REPLAY_MXFP4)
        return fail(REPLAY_ERR_ARG, "REPLAY_FLAG_MX_SCALE_CEIL applies to an MXFP4 read copy only");
    if ((c->flags & REPLAY_FLAG_QUANTIZED_CKPT) && c->read_copy == REPLAY_NONE)
        return fail(REPLAY_ERR_ARG, "REPLAY_FLAG_QUANTIZED_CKPT needs a read_copy format");
    if ((c->flags & REPLAY_FLAG_QUANTIZED_CKPT) && c->ckpt_dtype != REPLAY_F32)
        return fail(REPLAY_ERR_UNSUPPORTED, "REPLAY_FLAG_QUANTIZED_CKPT keeps an fp32 checkpoint");
    if ((c->flags & REPLAY_FLAG_VALU_FOLD) && (c->kind != REPLAY_MAMBA2 || c->ckpt_dtype != REPLAY_F32))
        return fail(REPLAY_ERR_UNSUPPORTED, "REPLAY_FLAG_VALU_FOLD is a Mamba-2 fp32-checkpoint cross-check");
    return ok();
}

void compute_layout(const replay_config* c, replay_layout* L)
{
    memset(L, 0, sizeof *L);
    const uint64_t B = c->batch, H = c->nheads, G = c->ngroups, C = c->head_dim, R = c->state_dim, cap = c->buf_cap;
    const uint64_t tiles = B * H, io = io_bytes(c);
    uint64_t off = 0;
    L->ckpt_off = off;
    L->ckpt_bytes = tiles * C * R * ckpt_bytes(c);
    off = align256(off + L->ckpt_bytes);
    if (c->read_copy == REPLAY_FP8_E4M3) L->rcopy_bytes = tiles * C * R;
    if (c->read_copy == REPLAY_MXFP4) {
        L->rcopy_bytes = tiles * C * R / 2;
        L->rscale_bytes = tiles * C * (R / 32);
    }
    L->rcopy_off = off;
    off = align256(off + L->rcopy_bytes);
    L->rscale_off = off;
    off = align256(off + L->rscale_bytes);
    L->buf_bytes[0] = 2 * B * H * cap * C * io;   // x (Mamba-2) / v (GDN)
    L->buf_bytes[1] = 2 * B * G * cap * R * io;   // B (Mamba-2) / k (GDN)
    L->buf_bytes[2] = 2 * B * H * cap * 4;        // dt (Mamba-2) / alpha (GDN), fp32
    L->buf_bytes[3] = c->kind == REPLAY_GDN ? 2 * B * H * cap * 4 : 0;  // beta
    for (int i = 0; i < 4; ++i) {
        L->buf_off[i] = off;
        off = align256(off + L->buf_bytes[i]);
    }
    L->book_off = off;
    L->book_bytes = 2 * 4 * B * 4;
    off = align256(off + L->book_bytes);
    L->err_off = off;
    off = align256(off + 4);
    L->total_bytes = off;
}

template <class T>
T* at(const replay_state* st, uint64_t off) { return reinterpret_cast<T*>(st->mem + off); }

int rc_kind(const replay_config* c)
{
    return c->read_copy == REPLAY_FP8_E4M3 ? rs::RC_FP8 : (c->read_copy == REPLAY_MXFP4 ? rs::RC_MXFP4 : rs::RC_NONE);
}

replay_status check_ptr(const void* p, const char* name)
{
    if (!p) return fail(REPLAY_ERR_ARG, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(REPLAY_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return REPLAY_OK;
}

replay_status check_inputs(const replay_config* c, const replay_inputs* in, bool need_tokens, bool need_D)
{
    if (!in) return fail(REPLAY_ERR_ARG, "inputs are NULL");
    replay_status s;
    if (c->kind == REPLAY_MAMBA2) {
        if ((s = check_ptr(in->A, "A")) != REPLAY_OK) return s;
        if (need_D && (s = check_ptr(in->D, "D")) != REPLAY_OK) return s;
        if (need_tokens) {
            if ((s = check_ptr(in->x, "x")) != REPLAY_OK) return s;
            if ((s = check_ptr(in->B, "B")) != REPLAY_OK) return s;
            if ((s = check_ptr(in->C, "C")) != REPLAY_OK) return s;
            if ((s = check_ptr(in->dt, "dt")) != REPLAY_OK) return s;
        }
    } else if (need_tokens) {
        if ((s = check_ptr(in->q, "q")) != REPLAY_OK) return s;
        if ((s = check_ptr(in->k, "k")) != REPLAY_OK) return s;
        if ((s = check_ptr(in->v, "v")) != REPLAY_OK) return s;
        if ((s = check_ptr(in->alpha, "alpha")) != REPLAY_OK) return s;
        if ((s = check_ptr(in->beta, "beta")) != REPLAY_OK) return s;
    }
    return REPLAY_OK;
}

// Mamba-2 heads per workgroup: the heads of a group share the staged B and C rows
// and the sequence's bookkeeping, and a workgroup that serves several of them
// streams one head's checkpoint while it computes the previous head's outputs.
// Used with four waves per workgroup when the group size allows it.
// An fp32 or fp16 checkpoint without a read copy streams enough bytes per head
// that six single-head workgroups per SIMD hide the fixed work better (measured
// on the batch-256 layer: fp32 0.182 vs 0.192 ms per step, fp16 0.108 vs
// 0.110 ms); the lighter streams gain from the shared staging (FP8 checkpoint
// 0.091 -> 0.077 ms, read copies 0.10-0.29 -> 0.07-0.11 ms).
int mamba2_heads_per_wg(const replay_config* c, int wpg)
{
    if (c->kind != REPLAY_MAMBA2 || wpg != 4) return 1;
    if (c->ckpt_dtype != REPLAY_FP8_E4M3 && c->read_copy == REPLAY_NONE) return 1;
    return (c->nheads / c->ngroups) % 4 == 0 ? 4 : 1;
}

// Multipliers for div_magic / div_small (the kernels' divisions by launch-invariant
// divisors): floor(2^32 / d) + 1, exact for quotients of n with n d < 2^32 (0 for
// d = 1); and ceil(2^20 / d), exact for n < 2^20 / d.
uint32_t magic_div(uint32_t d)
{
    return d <= 1 ? 0u : (uint32_t)((1ull << 32) / d + 1);
}

int magic_div20(int d)
{
    return (int)(((1u << 20) + (uint32_t)d - 1) / (uint32_t)d);
}

// GDN strips per wave.  Every wave of a head runs the head's adjoint chain and
// stages its entries, so a wave that owns two strips halves that work per head.
// Used where the value rows of a head fill whole workgroups of four waves with
// two strips each (d_v a multiple of 128), d_k = 128, and the step streams
// fewer bytes than an fp32 checkpoint (an fp16 or FP8 checkpoint or a read
// copy): there the fixed work per head bounds the step.  An fp32 stream keeps
// one strip per wave: six waves per SIMD keep more loads in flight than four
// (measured on the batch-256, 32-head layer: FP8 checkpoint 0.063 -> 0.054 ms
// per step with two strips; fp32 0.100 -> 0.119 ms).
int gdn_strips_per_wave(const replay_config* c)
{
    if (c->kind != REPLAY_GDN || c->state_dim != 128 || c->head_dim % 128 != 0) return 1;
    return c->ckpt_dtype == REPLAY_F32 && c->read_copy == REPLAY_NONE ? 1 : 2;
}

rs::StepArgs step_args(const replay_state* st, const replay_inputs* in, void* y, int mode, int T,
                       const uint8_t* active)
{
    const replay_config* c = &st->cfg;
    rs::StepArgs a;
    memset(&a, 0, sizeof a);
    a.B = c->batch;
    a.H = c->nheads;
    a.G = c->ngroups;
    a.hpg = c->nheads / c->ngroups;
    a.C = c->head_dim;
    a.R = c->state_dim;
    a.cap = c->buf_cap;
    a.parity = st->parity;
    a.mode = mode;
    a.T = T;
    a.vmax = mode == rs::MODE_DECODE ? c->buf_cap + 1 : (mode == rs::MODE_FLUSH ? c->buf_cap : c->buf_cap + T);
    a.scale = c->scale;
    // workgroups of at most 4 waves, each wave owning spw 16-column strips: the
    // largest divisor of the wave count that is <= 4 sets the waves per workgroup
    const int strips = c->head_dim / 16;
    a.spw = gdn_strips_per_wave(c);
    int wpg = 1;
    for (int d = 4; d >= 1; --d)
        if ((strips / a.spw) % d == 0) { wpg = d; break; }
    a.nsplit = strips / a.spw / wpg;
    a.ht = mamba2_heads_per_wg(c, wpg);
    a.cw = c->head_dim / a.nsplit;
    a.mg_nsplit = magic_div((uint32_t)a.nsplit);
    a.mg_tiles = magic_div((uint32_t)(c->nheads / a.ht));
    a.mg_hpg = magic_div((uint32_t)a.hpg);
    a.m20_cx = magic_div20(a.cw / (c->io_dtype == REPLAY_BF16 ? 8 : 4));
    a.qckpt = (c->flags & REPLAY_FLAG_QUANTIZED_CKPT) ? 1 : 0;
    a.mxceil = (c->flags & REPLAY_FLAG_MX_SCALE_CEIL) ? 1 : 0;
    const replay_layout& L = st->lay;
    a.ckpt = at<void>(st, L.ckpt_off);
    a.rcopy = L.rcopy_bytes ? at<uint8_t>(st, L.rcopy_off) : nullptr;
    a.rscale = L.rscale_bytes ? at<uint8_t>(st, L.rscale_off) : nullptr;
    a.bufc = at<void>(st, L.buf_off[0]);
    a.bufr = at<void>(st, L.buf_off[1]);
    a.bufs0 = at<float>(st, L.buf_off[2]);
    a.bufs1 = L.buf_bytes[3] ? at<float>(st, L.buf_off[3]) : nullptr;
    const uint64_t B = c->batch, H = c->nheads, G = c->ngroups, cap = c->buf_cap;
    a.bank_c = B * H * cap * c->head_dim;
    a.bank_r = B * G * cap * c->state_dim;
    a.bank_s = B * H * cap;
    a.book = at<int32_t>(st, L.book_off);
    a.err = at<uint32_t>(st, L.err_off);
    if (st->stack) {                      // every member follows the stack's one bookkeeping set
        a.book = st->stack->book;
        a.err = st->stack->err;
        a.parity = st->stack->parity;
    }
    if (c->kind == REPLAY_MAMBA2) {
        a.in_c = in->x;
        a.in_r = in->B;
        a.in_q = in->C;
        a.in_s0 = in->dt;
        a.A = in->A;
        a.D = in->D;
    } else {
        a.in_c = in->v;
        a.in_r = in->k;
        a.in_q = in->q;
        a.in_s0 = in->alpha;
        a.in_s1 = in->beta;
    }
    a.y = y;
    a.active = active;
    return a;
}

replay_status launch_step(replay_state* st, const replay_inputs* in, void* y, int mode, int T, void* stream,
                          const uint8_t* active = nullptr)
{
    const replay_config* c = &st->cfg;
    rs::StepArgs a = step_args(st, in, y, mode, T, active);
    (void)fresh();
    const int io = c->io_dtype == REPLAY_BF16 ? rs::IO_BF16 : rs::IO_F32;
    const int rc = rc_kind(c);
    hipError_t e;
    const hipStream_t hs = (hipStream_t)stream;
    const int ck = ck_kind(c);
    if (c->kind == REPLAY_MAMBA2)
        e = ck == rs::CK_F16   ? rs::launch_mamba2_step_f16(a, io, rc, hs)
            : ck == rs::CK_FP8 ? rs::launch_mamba2_step_fp8(a, io, rc, hs)
                               : rs::launch_mamba2_step_f32(a, io, rc, (c->flags & REPLAY_FLAG_VALU_FOLD) != 0, hs);
    else
        e = ck == rs::CK_F16   ? rs::launch_gdn_step_f16(a, io, rc, hs)
            : ck == rs::CK_FP8 ? rs::launch_gdn_step_fp8(a, io, rc, hs)
                               : rs::launch_gdn_step_f32(a, io, rc, hs);
    replay_status s = hip_check(e, "replay step launch");
    if (s == REPLAY_OK && !st->stack) st->parity ^= 1;
    return s;
}

}  // namespace

extern "C" {

int32_t replay_abi_version(void) { return REPLAY_ABI_VERSION; }

const char* replay_status_str(int32_t s)
{
    switch (s) {
        case REPLAY_OK: return "ok";
        case REPLAY_ERR_ARG: return "invalid argument";
        case REPLAY_ERR_SHAPE: return "unsupported or inconsistent shape";
        case REPLAY_ERR_DTYPE: return "unsupported dtype";
        case REPLAY_ERR_ALIGN: return "misaligned pointer or short region";
        case REPLAY_ERR_STATE: return "operation not allowed in the current phase";
        case REPLAY_ERR_CAPACITY: return "draft count outside [1, buf_cap]";
        case REPLAY_ERR_UNSUPPORTED: return "not supported by this build";
        case REPLAY_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* replay_last_error(void) { return g_err.c_str(); }

replay_status replay_config_check(const replay_config* cfg) { return check_config(cfg); }

size_t replay_state_bytes(const replay_config* cfg)
{
    if (check_config(cfg) != REPLAY_OK) return 0;
    replay_layout L;
    compute_layout(cfg, &L);
    return (size_t)L.total_bytes;
}

replay_status replay_state_alloc(const replay_config* cfg, void* dev_mem, size_t bytes, void* stream,
                                 replay_state** out)
{
    replay_status s = check_config(cfg);
    if (s != REPLAY_OK) return s;
    if (!out) return fail(REPLAY_ERR_ARG, "out is NULL");
    if (!dev_mem) return fail(REPLAY_ERR_ARG, "dev_mem is NULL");
    if (!aligned(dev_mem, 256)) return fail(REPLAY_ERR_ALIGN, "state region must be 256-byte aligned");
    replay_layout L;
    compute_layout(cfg, &L);
    if (bytes < L.total_bytes)
        return fail(REPLAY_ERR_ALIGN, "state region has %zu bytes, needs %llu", bytes, (unsigned long long)L.total_bytes);
    replay_state* st = new replay_state;
    st->cfg = *cfg;
    st->mem = static_cast<uint8_t*>(dev_mem);
    st->bytes = bytes;
    st->lay = L;
    st->parity = 0;
    st->phase = 0;
    s = LAUNCH(rs::launch_fill_zero(dev_mem, L.total_bytes, (hipStream_t)stream), "state initialisation");
    if (s == REPLAY_OK)
        s = LAUNCH(rs::launch_book_reset(at<int32_t>(st, L.book_off), at<uint32_t>(st, L.err_off), cfg->batch, 0,
                                            cfg->buf_cap, (cfg->flags & REPLAY_FLAG_STAGGER_FLUSH) != 0,
                                            (hipStream_t)stream),
                      "bookkeeping initialisation");
    if (s != REPLAY_OK) {
        delete st;
        return s;
    }
    *out = st;
    return ok();
}

replay_status replay_state_free(replay_state* st)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is bound to a stack: free the stack first");
    delete st;
    return ok();
}

replay_status replay_state_layout(const replay_state* st, replay_layout* out)
{
    if (!st || !out) return fail(REPLAY_ERR_ARG, "NULL argument");
    *out = st->lay;
    return ok();
}

int32_t replay_state_phase(const replay_state* st) { return st ? st->phase : -1; }

static replay_status load_impl(replay_state* st, const void* S, bool src_f32, void* stream);

replay_status replay_load_checkpoint(replay_state* st, const void* S, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: load through the stack");
    if (st->phase != 0) return fail(REPLAY_ERR_STATE, "load while drafts are pending");
    replay_status s = load_impl(st, S, false, stream);
    if (s == REPLAY_OK) st->needs_load = false;
    return s;
}

replay_status replay_load_checkpoint_f32(replay_state* st, const float* S, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: load through the stack");
    if (st->phase != 0) return fail(REPLAY_ERR_STATE, "load while drafts are pending");
    replay_status s = load_impl(st, S, true, stream);
    if (s == REPLAY_OK) st->needs_load = false;
    return s;
}

// Checkpoint tiles and read copy of the tiles `m` names (all of them for a
// whole-state load), from `ntiles` source tiles.
static replay_status load_tiles(replay_state* st, const void* S, bool src_f32, int ntiles, const rs::SlotMap& m,
                                hipStream_t hs)
{
    const replay_config* c = &st->cfg;
    replay_status s = LAUNCH(rs::launch_logical_to_tiles(S, at<void>(st, st->lay.ckpt_off), ntiles, c->head_dim,
                                                         c->state_dim, ck_kind(c), src_f32, m, hs),
                             "checkpoint load");
    if (s != REPLAY_OK || c->read_copy == REPLAY_NONE) return s;
    return LAUNCH(rs::launch_quantize_read_copy(at<void>(st, st->lay.ckpt_off), at<uint8_t>(st, st->lay.rcopy_off),
                                                st->lay.rscale_bytes ? at<uint8_t>(st, st->lay.rscale_off) : nullptr,
                                                ntiles, c->head_dim, c->state_dim, rc_kind(c), ck_kind(c),
                                                (c->flags & REPLAY_FLAG_QUANTIZED_CKPT) != 0,
                                                (c->flags & REPLAY_FLAG_MX_SCALE_CEIL) != 0, m, hs),
                  "read copy quantize");
}

// Checkpoint tiles and read copy of one state, then its bookkeeping (the
// stack's, for a member).
static replay_status load_impl(replay_state* st, const void* S, bool src_f32, void* stream)
{
    replay_status s = check_ptr(S, "S_logical");
    if (s != REPLAY_OK) return s;
    const replay_config* c = &st->cfg;
    hipStream_t hs = (hipStream_t)stream;
    s = load_tiles(st, S, src_f32, c->batch * c->nheads, all_tiles(c->nheads), hs);
    if (s != REPLAY_OK || st->stack) return s;
    return LAUNCH(rs::launch_book_reset(at<int32_t>(st, st->lay.book_off), at<uint32_t>(st, st->lay.err_off),
                                        c->batch, st->parity, c->buf_cap,
                                        (c->flags & REPLAY_FLAG_STAGGER_FLUSH) != 0, hs),
                  "bookkeeping reset");
}

// Host-side checks of a per-slot load's sequence list: 1 <= n <= B, every slot
// in [0, B), no slot twice.
static replay_status check_slots(int32_t n, const int32_t* slots, int B)
{
    if (n < 1 || n > B) return fail(REPLAY_ERR_ARG, "slot count %d outside [1, %d]", n, B);
    if (!slots) return fail(REPLAY_ERR_ARG, "slots is NULL");
    std::vector<char> seen((size_t)B, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t b = slots[i];
        if (b < 0 || b >= B) return fail(REPLAY_ERR_ARG, "slot %d outside [0, %d)", b, B);
        if (seen[(size_t)b]) return fail(REPLAY_ERR_ARG, "slot %d listed twice", b);
        seen[(size_t)b] = 1;
    }
    return REPLAY_OK;
}

// The listed sequences' checkpoints (fp32 source [n][H][rows][cols]) and read
// copies, in chunks of SLOT_CHUNK sequences per launch; then, unless the state
// is a stack member, their bookkeeping.
static replay_status load_slots_impl(replay_state* st, int32_t n, const int32_t* slots, const float* S, hipStream_t hs)
{
    const replay_config* c = &st->cfg;
    const size_t seq_floats = (size_t)c->nheads * c->head_dim * c->state_dim;
    for (int32_t i0 = 0; i0 < n; i0 += rs::SLOT_CHUNK) {
        rs::SlotMap m;
        m.n = n - i0 < rs::SLOT_CHUNK ? n - i0 : rs::SLOT_CHUNK;
        m.H = c->nheads;
        for (int i = 0; i < m.n; ++i) m.slot[i] = slots[i0 + i];
        replay_status s = load_tiles(st, S + (size_t)i0 * seq_floats, true, m.n * c->nheads, m, hs);
        if (s != REPLAY_OK) return s;
        if (!st->stack) {
            s = LAUNCH(rs::launch_book_reset_slots(at<int32_t>(st, st->lay.book_off), c->batch, st->parity,
                                                   c->buf_cap, m, hs),
                       "slot bookkeeping reset");
            if (s != REPLAY_OK) return s;
        }
    }
    return REPLAY_OK;
}

replay_status replay_load_slots(replay_state* st, int32_t n, const int32_t* slots, const float* S, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: load through the stack");
    if (st->needs_load) return fail(REPLAY_ERR_STATE, "a former stack member must be loaded first");
    if (st->phase != 0) return fail(REPLAY_ERR_STATE, "load while drafts are pending");
    replay_status s = check_slots(n, slots, st->cfg.batch);
    if (s != REPLAY_OK) return s;
    if ((s = check_ptr(S, "S_logical")) != REPLAY_OK) return s;
    if ((s = load_slots_impl(st, n, slots, S, (hipStream_t)stream)) != REPLAY_OK) return s;
    return ok();
}

replay_status replay_read_checkpoint(const replay_state* st, void* out, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    replay_status s = check_ptr(out, "S_out");
    if (s != REPLAY_OK) return s;
    const replay_config* c = &st->cfg;
    return LAUNCH(rs::launch_tiles_to_logical(at<void>(st, st->lay.ckpt_off), out, c->batch * c->nheads,
                                                 c->head_dim, c->state_dim, ck_kind(c), (hipStream_t)stream),
                     "checkpoint read");
}

replay_status replay_read_copy(const replay_state* st, uint8_t* codes_out, uint8_t* scales_out, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    const replay_config* c = &st->cfg;
    if (c->read_copy == REPLAY_NONE) return fail(REPLAY_ERR_STATE, "state has no read copy");
    if (!codes_out) return fail(REPLAY_ERR_ARG, "codes_out is NULL");
    if (c->read_copy == REPLAY_MXFP4 && !scales_out) return fail(REPLAY_ERR_ARG, "scales_out is NULL");
    return LAUNCH(rs::launch_read_copy_to_logical(at<uint8_t>(st, st->lay.rcopy_off),
                                                     st->lay.rscale_bytes ? at<uint8_t>(st, st->lay.rscale_off) : nullptr,
                                                     codes_out, scales_out, c->batch * c->nheads, c->head_dim,
                                                     c->state_dim, rc_kind(c), (hipStream_t)stream),
                     "read copy export");
}

static replay_status read_book_impl(const int32_t* book, const uint32_t* err, int B, int parity, int32_t* book_out,
                                    uint32_t* err_out, void* stream)
{
    if (!book_out) return fail(REPLAY_ERR_ARG, "book_out is NULL");
    const size_t n = (size_t)3 * B * sizeof(int32_t);
    hipStream_t hs = (hipStream_t)stream;
    replay_status s = LAUNCH(hipMemcpyAsync(book_out, book + (size_t)parity * 4 * B, n, hipMemcpyDeviceToDevice, hs),
                                "bookkeeping copy");
    if (s != REPLAY_OK || !err_out) return s;
    return LAUNCH(hipMemcpyAsync(err_out, err, 4, hipMemcpyDeviceToDevice, hs), "error word copy");
}

replay_status replay_read_book(const replay_state* st, int32_t* book_out, uint32_t* err_out, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: read the stack's bookkeeping");
    return read_book_impl(at<int32_t>(st, st->lay.book_off), at<uint32_t>(st, st->lay.err_off), st->cfg.batch,
                          st->parity, book_out, err_out, stream);
}

static replay_status decode_impl(replay_state* st, const replay_inputs* in, const uint8_t* active, void* y,
                                 void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: step it through the stack");
    if (st->needs_load) return fail(REPLAY_ERR_STATE, "a former stack member must be loaded first");
    if (st->phase != 0) return fail(REPLAY_ERR_STATE, "decode while drafts are pending");
    replay_status s = check_inputs(&st->cfg, in, true, true);
    if (s != REPLAY_OK) return s;
    if ((s = check_ptr(y, "y")) != REPLAY_OK) return s;
    return launch_step(st, in, y, rs::MODE_DECODE, 1, stream, active);
}

replay_status replay_decode_step(replay_state* st, const replay_inputs* in, void* y, void* stream)
{
    return decode_impl(st, in, nullptr, y, stream);
}

replay_status replay_decode_step_masked(replay_state* st, const replay_inputs* in, const uint8_t* active, void* y,
                                        void* stream)
{
    if (!active) return fail(REPLAY_ERR_ARG, "active is NULL");
    return decode_impl(st, in, active, y, stream);
}

replay_status replay_flush(replay_state* st, const replay_inputs* in, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: step it through the stack");
    if (st->needs_load) return fail(REPLAY_ERR_STATE, "a former stack member must be loaded first");
    if (st->phase != 0) return fail(REPLAY_ERR_STATE, "flush while drafts are pending");
    replay_inputs none;
    memset(&none, 0, sizeof none);
    if (!in) in = &none;
    if (st->cfg.kind == REPLAY_MAMBA2) {
        replay_status s = check_ptr(in->A, "A");
        if (s != REPLAY_OK) return s;
    }
    return launch_step(st, in, nullptr, rs::MODE_FLUSH, 0, stream);
}

static replay_status spec_impl(replay_state* st, int32_t k, const replay_inputs* drafts, const uint8_t* active,
                               void* y, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: step it through the stack");
    if (st->needs_load) return fail(REPLAY_ERR_STATE, "a former stack member must be loaded first");
    if (st->phase != 0) return fail(REPLAY_ERR_STATE, "spec_append while drafts are pending");
    if (k < 1 || k > st->cfg.buf_cap) return fail(REPLAY_ERR_CAPACITY, "k = %d outside [1, %d]", k, st->cfg.buf_cap);
    replay_status s = check_inputs(&st->cfg, drafts, true, true);
    if (s != REPLAY_OK) return s;
    if ((s = check_ptr(y, "y")) != REPLAY_OK) return s;
    s = launch_step(st, drafts, y, rs::MODE_SPEC, k, stream, active);
    if (s == REPLAY_OK) st->phase = 1;
    return s;
}

replay_status replay_spec_append(replay_state* st, int32_t k, const replay_inputs* drafts, void* y, void* stream)
{
    return spec_impl(st, k, drafts, nullptr, y, stream);
}

replay_status replay_spec_append_masked(replay_state* st, int32_t k, const replay_inputs* drafts,
                                        const uint8_t* active, void* y, void* stream)
{
    if (!active) return fail(REPLAY_ERR_ARG, "active is NULL");
    return spec_impl(st, k, drafts, active, y, stream);
}

static replay_status commit_impl(replay_state* st, const int32_t* accepted, void* stream)
{
    if (st->phase != 1) return fail(REPLAY_ERR_STATE, "no drafts pending");
    replay_status s = LAUNCH(rs::launch_book_commit(at<int32_t>(st, st->lay.book_off), at<uint32_t>(st, st->lay.err_off),
                                                       st->cfg.batch, st->parity, accepted, (hipStream_t)stream),
                                "commit");
    if (s == REPLAY_OK) {
        st->parity ^= 1;
        st->phase = 0;
    }
    return s;
}

replay_status replay_spec_commit(replay_state* st, const int32_t* accepted, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: step it through the stack");
    if (st->needs_load) return fail(REPLAY_ERR_STATE, "a former stack member must be loaded first");
    if (!accepted) return fail(REPLAY_ERR_ARG, "accepted is NULL");
    if (!aligned(accepted, 4)) return fail(REPLAY_ERR_ALIGN, "accepted is not 4-byte aligned");
    return commit_impl(st, accepted, stream);
}

replay_status replay_spec_rollback(replay_state* st, void* stream)
{
    if (!st) return fail(REPLAY_ERR_ARG, "state is NULL");
    if (st->stack) return fail(REPLAY_ERR_STATE, "the state is a stack member: step it through the stack");
    if (st->needs_load) return fail(REPLAY_ERR_STATE, "a former stack member must be loaded first");
    return commit_impl(st, nullptr, stream);
}

// ---- layer stacks: one bookkeeping set for every SSM layer of a model --------

static replay_status stack_check_step(const replay_stack* stk, int32_t layer, int mode, int k, const uint8_t* active)
{
    if (!stk) return fail(REPLAY_ERR_ARG, "stack is NULL");
    const int n = (int)stk->layers.size();
    if (layer < 0 || layer >= n) return fail(REPLAY_ERR_ARG, "layer %d outside [0, %d)", layer, n);
    if (layer != stk->next)
        return fail(REPLAY_ERR_STATE, "layer %d stepped out of order: the step expects layer %d", layer, stk->next);
    if (stk->next == 0 && stk->phase != 0) return fail(REPLAY_ERR_STATE, "drafts are pending");
    if (stk->next > 0 && (mode != stk->step_mode || k != stk->step_k))
        return fail(REPLAY_ERR_STATE, "every layer of a step runs the same operation with the same draft count");
    if (stk->next > 0 && active != stk->step_active)
        return fail(REPLAY_ERR_STATE, "every layer of a step uses the same active mask");
    return REPLAY_OK;
}

// A layer of the step ran: after the last one the shared bookkeeping copy
// written by the step becomes the current one.
static void stack_advance(replay_stack* stk, int mode, int k, const uint8_t* active)
{
    if (stk->next == 0) {
        stk->step_mode = mode;
        stk->step_k = k;
        stk->step_active = active;
    }
    if (++stk->next == (int)stk->layers.size()) {
        stk->next = 0;
        stk->parity ^= 1;
        stk->step_mode = -1;
        if (mode == rs::MODE_SPEC) stk->phase = 1;
    }
}

static replay_status stack_idle(const replay_stack* stk, const char* what)
{
    if (!stk) return fail(REPLAY_ERR_ARG, "stack is NULL");
    if (stk->next != 0) return fail(REPLAY_ERR_STATE, "%s in the middle of a step (layer %d is next)", what, stk->next);
    return REPLAY_OK;
}

static replay_status stack_reset_book(replay_stack* stk, void* stream)
{
    const replay_config* c = &stk->layers[0]->cfg;
    return LAUNCH(rs::launch_book_reset(stk->book, stk->err, c->batch, stk->parity, c->buf_cap,
                                           (c->flags & REPLAY_FLAG_STAGGER_FLUSH) != 0, (hipStream_t)stream),
                     "bookkeeping reset");
}

replay_status replay_stack_create(replay_state* const* layers, int32_t nlayers, void* stream, replay_stack** out)
{
    if (!out) return fail(REPLAY_ERR_ARG, "out is NULL");
    if (!layers || nlayers < 1) return fail(REPLAY_ERR_ARG, "a stack needs at least one layer");
    const replay_config* c0 = layers[0] ? &layers[0]->cfg : nullptr;
    for (int l = 0; l < nlayers; ++l) {
        const replay_state* st = layers[l];
        if (!st) return fail(REPLAY_ERR_ARG, "layer %d is NULL", l);
        for (int m = 0; m < l; ++m)
            if (layers[m] == st) return fail(REPLAY_ERR_ARG, "layer %d repeats layer %d", l, m);
        if (st->stack) return fail(REPLAY_ERR_STATE, "layer %d already belongs to a stack", l);
        if (st->phase != 0) return fail(REPLAY_ERR_STATE, "layer %d has pending drafts", l);
        const replay_config* c = &st->cfg;
        if (c->batch != c0->batch || c->buf_cap != c0->buf_cap)
            return fail(REPLAY_ERR_SHAPE, "layer %d: batch and buf_cap must match layer 0", l);
        if ((c->flags & REPLAY_FLAG_STAGGER_FLUSH) != (c0->flags & REPLAY_FLAG_STAGGER_FLUSH))
            return fail(REPLAY_ERR_ARG, "layer %d: REPLAY_FLAG_STAGGER_FLUSH must match layer 0", l);
    }
    replay_stack* stk = new replay_stack;
    stk->layers.assign(layers, layers + nlayers);
    stk->book = at<int32_t>(layers[0], layers[0]->lay.book_off);
    stk->err = at<uint32_t>(layers[0], layers[0]->lay.err_off);
    replay_status s = stack_reset_book(stk, stream);
    if (s != REPLAY_OK) {
        delete stk;
        return s;
    }
    for (replay_state* st : stk->layers) st->stack = stk;
    *out = stk;
    return ok();
}

replay_status replay_stack_free(replay_stack* stk)
{
    if (!stk) return fail(REPLAY_ERR_ARG, "stack is NULL");
    for (replay_state* st : stk->layers) {
        st->stack = nullptr;
        st->needs_load = true;
        st->phase = 0;
    }
    delete stk;
    return ok();
}

static replay_status stack_load_impl(replay_stack* stk, const void* const* S, bool src_f32, void* stream)
{
    replay_status s = stack_idle(stk, "load");
    if (s != REPLAY_OK) return s;
    if (stk->phase != 0) return fail(REPLAY_ERR_STATE, "load while drafts are pending");
    if (!S) return fail(REPLAY_ERR_ARG, "S_logical is NULL");
    for (size_t l = 0; l < stk->layers.size(); ++l)
        if ((s = check_ptr(S[l], "S_logical[layer]")) != REPLAY_OK) return s;
    for (size_t l = 0; l < stk->layers.size(); ++l)
        if ((s = load_impl(stk->layers[l], S[l], src_f32, stream)) != REPLAY_OK) return s;
    return stack_reset_book(stk, stream);
}

replay_status replay_stack_load(replay_stack* stk, const void* const* S, void* stream)
{
    return stack_load_impl(stk, S, false, stream);
}

replay_status replay_stack_load_f32(replay_stack* stk, const float* const* S, void* stream)
{
    return stack_load_impl(stk, reinterpret_cast<const void* const*>(S), true, stream);
}

replay_status replay_stack_load_slots(replay_stack* stk, int32_t n, const int32_t* slots, const float* const* S,
                                      void* stream)
{
    replay_status s = stack_idle(stk, "load");
    if (s != REPLAY_OK) return s;
    if (stk->phase != 0) return fail(REPLAY_ERR_STATE, "load while drafts are pending");
    const replay_config* c0 = &stk->layers[0]->cfg;
    if ((s = check_slots(n, slots, c0->batch)) != REPLAY_OK) return s;
    if (!S) return fail(REPLAY_ERR_ARG, "S_logical is NULL");
    for (size_t l = 0; l < stk->layers.size(); ++l)
        if ((s = check_ptr(S[l], "S_logical[layer]")) != REPLAY_OK) return s;
    hipStream_t hs = (hipStream_t)stream;
    for (size_t l = 0; l < stk->layers.size(); ++l)
        if ((s = load_slots_impl(stk->layers[l], n, slots, S[l], hs)) != REPLAY_OK) return s;
    for (int32_t i0 = 0; i0 < n; i0 += rs::SLOT_CHUNK) {
        rs::SlotMap m;
        m.n = n - i0 < rs::SLOT_CHUNK ? n - i0 : rs::SLOT_CHUNK;
        m.H = 1;
        for (int i = 0; i < m.n; ++i) m.slot[i] = slots[i0 + i];
        s = LAUNCH(rs::launch_book_reset_slots(stk->book, c0->batch, stk->parity, c0->buf_cap, m, hs),
                   "slot bookkeeping reset");
        if (s != REPLAY_OK) return s;
    }
    return ok();
}

static replay_status stack_decode_impl(replay_stack* stk, int32_t layer, const replay_inputs* in,
                                       const uint8_t* active, void* y, void* stream)
{
    replay_status s = stack_check_step(stk, layer, rs::MODE_DECODE, 1, active);
    if (s != REPLAY_OK) return s;
    replay_state* st = stk->layers[layer];
    if ((s = check_inputs(&st->cfg, in, true, true)) != REPLAY_OK) return s;
    if ((s = check_ptr(y, "y")) != REPLAY_OK) return s;
    if ((s = launch_step(st, in, y, rs::MODE_DECODE, 1, stream, active)) != REPLAY_OK) return s;
    stack_advance(stk, rs::MODE_DECODE, 1, active);
    return ok();
}

replay_status replay_stack_decode_layer(replay_stack* stk, int32_t layer, const replay_inputs* in, void* y,
                                        void* stream)
{
    return stack_decode_impl(stk, layer, in, nullptr, y, stream);
}

replay_status replay_stack_decode_layer_masked(replay_stack* stk, int32_t layer, const replay_inputs* in,
                                               const uint8_t* active, void* y, void* stream)
{
    if (!active) return fail(REPLAY_ERR_ARG, "active is NULL");
    return stack_decode_impl(stk, layer, in, active, y, stream);
}

static replay_status stack_spec_impl(replay_stack* stk, int32_t layer, int32_t k, const replay_inputs* drafts,
                                     const uint8_t* active, void* y, void* stream)
{
    replay_status s = stack_check_step(stk, layer, rs::MODE_SPEC, k, active);
    if (s != REPLAY_OK) return s;
    replay_state* st = stk->layers[layer];
    if (k < 1 || k > st->cfg.buf_cap) return fail(REPLAY_ERR_CAPACITY, "k = %d outside [1, %d]", k, st->cfg.buf_cap);
    if ((s = check_inputs(&st->cfg, drafts, true, true)) != REPLAY_OK) return s;
    if ((s = check_ptr(y, "y")) != REPLAY_OK) return s;
    if ((s = launch_step(st, drafts, y, rs::MODE_SPEC, k, stream, active)) != REPLAY_OK) return s;
    stack_advance(stk, rs::MODE_SPEC, k, active);
    return ok();
}

replay_status replay_stack_spec_layer(replay_stack* stk, int32_t layer, int32_t k, const replay_inputs* drafts,
                                      void* y, void* stream)
{
    return stack_spec_impl(stk, layer, k, drafts, nullptr, y, stream);
}

replay_status replay_stack_spec_layer_masked(replay_stack* stk, int32_t layer, int32_t k, const replay_inputs* drafts,
                                             const uint8_t* active, void* y, void* stream)
{
    if (!active) return fail(REPLAY_ERR_ARG, "active is NULL");
    return stack_spec_impl(stk, layer, k, drafts, active, y, stream);
}

replay_status replay_stack_flush(replay_stack* stk, const replay_inputs* const* in, void* stream)
{
    replay_status s = stack_idle(stk, "flush");
    if (s != REPLAY_OK) return s;
    if (stk->phase != 0) return fail(REPLAY_ERR_STATE, "flush while drafts are pending");
    replay_inputs none;
    memset(&none, 0, sizeof none);
    for (size_t l = 0; l < stk->layers.size(); ++l) {
        const replay_inputs* il = (in && in[l]) ? in[l] : &none;
        if (stk->layers[l]->cfg.kind == REPLAY_MAMBA2 && (s = check_ptr(il->A, "A")) != REPLAY_OK) return s;
    }
    for (size_t l = 0; l < stk->layers.size(); ++l) {
        const replay_inputs* il = (in && in[l]) ? in[l] : &none;
        if ((s = launch_step(stk->layers[l], il, nullptr, rs::MODE_FLUSH, 0, stream)) != REPLAY_OK) return s;
    }
    stk->parity ^= 1;
    return ok();
}

static replay_status stack_commit_impl(replay_stack* stk, const int32_t* accepted, void* stream)
{
    replay_status s = stack_idle(stk, "commit");
    if (s != REPLAY_OK) return s;
    if (stk->phase != 1) return fail(REPLAY_ERR_STATE, "no drafts pending");
    s = LAUNCH(rs::launch_book_commit(stk->book, stk->err, stk->layers[0]->cfg.batch, stk->parity, accepted,
                                         (hipStream_t)stream),
                  "commit");
    if (s == REPLAY_OK) {
        stk->parity ^= 1;
        stk->phase = 0;
    }
    return s;
}

replay_status replay_stack_commit(replay_stack* stk, const int32_t* accepted, void* stream)
{
    if (!accepted) return fail(REPLAY_ERR_ARG, "accepted is NULL");
    if (!aligned(accepted, 4)) return fail(REPLAY_ERR_ALIGN, "accepted is not 4-byte aligned");
    return stack_commit_impl(stk, accepted, stream);
}

replay_status replay_stack_rollback(replay_stack* stk, void* stream) { return stack_commit_impl(stk, nullptr, stream); }

replay_status replay_stack_read_book(const replay_stack* stk, int32_t* book_out, uint32_t* err_out, void* stream)
{
    if (!stk) return fail(REPLAY_ERR_ARG, "stack is NULL");
    return read_book_impl(stk->book, stk->err, stk->layers[0]->cfg.batch, stk->parity, book_out, err_out, stream);
}

int32_t replay_stack_layers(const replay_stack* stk) { return stk ? (int32_t)stk->layers.size() : -1; }
int32_t replay_stack_next_layer(const replay_stack* stk) { return stk ? stk->next : -1; }
int32_t replay_stack_phase(const replay_stack* stk) { return stk ? stk->phase : -1; }

static replay_status conv_common(const replay_config* cfg, rs::ConvArgs* a, const replay_inputs* in, void* y, int T)
{
    replay_config c = *cfg;
    // the baselines have no checkpoint/buffer: read-copy, flag and kind limits
    // of the replay kernels do not apply
    c.read_copy = REPLAY_NONE;
    c.flags = 0;
    const int kind = c.kind;
    c.kind = REPLAY_MAMBA2;
    replay_status s = check_config(&c);
    if (s != REPLAY_OK) return s;
    c.kind = kind;
    if ((s = check_inputs(&c, in, true, true)) != REPLAY_OK) return s;
    if ((s = check_ptr(y, "y")) != REPLAY_OK) return s;
    memset(a, 0, sizeof *a);
    a->kind = kind == REPLAY_GDN ? 1 : 0;
    a->B = c.batch;
    a->H = c.nheads;
    a->G = c.ngroups;
    a->hpg = c.nheads / c.ngroups;
    a->C = c.head_dim;
    a->R = c.state_dim;
    a->T = T;
    a->scale = c.scale;
    if (kind == REPLAY_MAMBA2) {
        a->in_c = in->x;
        a->in_r = in->B;
        a->in_q = in->C;
        a->in_s0 = in->dt;
        a->A = in->A;
        a->D = in->D;
    } else {
        a->in_c = in->v;
        a->in_r = in->k;
        a->in_q = in->q;
        a->in_s0 = in->alpha;
        a->in_s1 = in->beta;
    }
    a->y = y;
    return REPLAY_OK;
}

replay_status replay_conv_decode_step(const replay_config* cfg, void* S, const replay_inputs* in, void* y,
                                      void* stream)
{
    rs::ConvArgs a;
    replay_status s = conv_common(cfg, &a, in, y, 1);
    if (s != REPLAY_OK) return s;
    if ((s = check_ptr(S, "S")) != REPLAY_OK) return s;
    a.S = S;
    return LAUNCH(rs::launch_conv_step(a, cfg->io_dtype == REPLAY_BF16 ? rs::IO_BF16 : rs::IO_F32, ck_kind(cfg),
                                          (hipStream_t)stream),
                     "conventional decode");
}

replay_status replay_conv_spec_step(const replay_config* cfg, const void* S, void* snaps, int32_t k,
                                    const replay_inputs* drafts, void* y, void* stream)
{
    rs::ConvArgs a;
    replay_status s = conv_common(cfg, &a, drafts, y, k);
    if (s != REPLAY_OK) return s;
    if (k < 1 || k > REPLAY_MAX_BUF) return fail(REPLAY_ERR_CAPACITY, "k = %d outside [1, %d]", k, REPLAY_MAX_BUF);
    if ((s = check_ptr(S, "S")) != REPLAY_OK) return s;
    if ((s = check_ptr(snaps, "snaps")) != REPLAY_OK) return s;
    a.S_in = S;
    a.S = const_cast<void*>(S);
    a.snaps = snaps;
    return LAUNCH(rs::launch_conv_step(a, cfg->io_dtype == REPLAY_BF16 ? rs::IO_BF16 : rs::IO_F32, ck_kind(cfg),
                                          (hipStream_t)stream),
                     "conventional spec step");
}

replay_status replay_conv_spec_restore(const replay_config* cfg, void* S, const void* snaps, int32_t k,
                                       const int32_t* accepted, void* stream)
{
    if (!cfg) return fail(REPLAY_ERR_ARG, "config is NULL");
    replay_status s;
    if ((s = check_ptr(S, "S")) != REPLAY_OK) return s;
    if ((s = check_ptr(snaps, "snaps")) != REPLAY_OK) return s;
    if (!accepted) return fail(REPLAY_ERR_ARG, "accepted is NULL");
    if (k < 1 || k > REPLAY_MAX_BUF) return fail(REPLAY_ERR_CAPACITY, "k = %d outside [1, %d]", k, REPLAY_MAX_BUF);
    replay_config c = *cfg;
    c.kind = REPLAY_MAMBA2;
    c.read_copy = REPLAY_NONE;
    c.flags = 0;
    if ((s = check_config(&c)) != REPLAY_OK) return s;
    const size_t tile_bytes = (size_t)cfg->head_dim * cfg->state_dim * ckpt_bytes(cfg);
    return LAUNCH(rs::launch_conv_restore(S, snaps, accepted, cfg->batch, tile_bytes, cfg->nheads, k,
                                             (hipStream_t)stream),
                     "conventional restore");
}

replay_status replay_standin_linear(const void* X, const void* W, void* Y, int32_t M, int32_t K, int32_t N,
                                    void* stream)
{
    replay_status s;
    if ((s = check_ptr(X, "X")) != REPLAY_OK) return s;
    if ((s = check_ptr(W, "W")) != REPLAY_OK) return s;
    if ((s = check_ptr(Y, "Y")) != REPLAY_OK) return s;
    if (M < 1 || K < 64 || K % 64 != 0 || N < 1)
        return fail(REPLAY_ERR_SHAPE, "linear needs M >= 1, K a positive multiple of 64 and N >= 1 (M %d, K %d, N %d)",
                    M, K, N);
    if ((long long)(M + 63) / 64 > 65535) return fail(REPLAY_ERR_SHAPE, "M %d too large", M);
    return LAUNCH(rs::launch_standin_linear(X, W, Y, M, K, N, (hipStream_t)stream), "stand-in linear");
}

replay_status replay_standin_attention(const void* q, int64_t q_stride, const void* K, const void* V, void* o,
                                       int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t L, float scale,
                                       void* stream)
{
    replay_status s;
    if ((s = check_ptr(q, "q")) != REPLAY_OK) return s;
    if ((s = check_ptr(K, "K")) != REPLAY_OK) return s;
    if ((s = check_ptr(V, "V")) != REPLAY_OK) return s;
    if ((s = check_ptr(o, "o")) != REPLAY_OK) return s;
    if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || L < 1)
        return fail(REPLAY_ERR_SHAPE, "attention needs B, Hkv, L >= 1 and Hkv dividing Hq");
    const int qpk = Hq / Hkv;
    if (qpk != 1 && qpk != 2 && qpk != 4 && qpk != 8)
        return fail(REPLAY_ERR_UNSUPPORTED, "query heads per key/value head must be 1, 2, 4 or 8 (is %d)", qpk);
    if (D != 128) return fail(REPLAY_ERR_UNSUPPORTED, "head dimension %d (128 is built)", D);
    if (q_stride < (int64_t)Hq * D || q_stride % 8 != 0)
        return fail(REPLAY_ERR_ARG, "q_stride %lld must be >= Hq * D and a multiple of 8", (long long)q_stride);
    if ((long long)B * Hkv > (1LL << 31) - 1) return fail(REPLAY_ERR_SHAPE, "B * Hkv too large");
    return LAUNCH(rs::launch_standin_attention(q, K, V, o, B, Hq, Hkv, D, L, (size_t)q_stride, scale,
                                               (hipStream_t)stream),
                  "stand-in attention");
}

replay_status replay_stream_copy(void* dst, const void* src, size_t bytes, void* stream)
{
    replay_status s;
    if ((s = check_ptr(dst, "dst")) != REPLAY_OK) return s;
    if ((s = check_ptr(src, "src")) != REPLAY_OK) return s;
    if (bytes % 16) return fail(REPLAY_ERR_ALIGN, "bytes must be a multiple of 16");
    return LAUNCH(rs::launch_stream_copy(dst, src, bytes, (hipStream_t)stream), "stream copy");
}

replay_status replay_stream_read(const void* src, size_t bytes, float* partials, void* stream)
{
    replay_status s;
    if ((s = check_ptr(src, "src")) != REPLAY_OK) return s;
    if ((s = check_ptr(partials, "partials")) != REPLAY_OK) return s;
    if (bytes % 16) return fail(REPLAY_ERR_ALIGN, "bytes must be a multiple of 16");
    return LAUNCH(rs::launch_stream_read(src, bytes, partials, (hipStream_t)stream), "stream read");
}

}  // extern "C"
