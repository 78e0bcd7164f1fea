/*
 * replayssm.h -- C ABI of the MI355X (gfx950) replayed SSM decode library.
 *
 * The library keeps each sequence's SSM state as a checkpoint plus a buffer of
 * the most recent per-token inputs (capacity 1..16; 16 on the pages).  A
 * decode step that does not fill the buffer appends the token's inputs and
 * computes the output from the read-only checkpoint plus the buffered inputs,
 * writing no state; the step whose append fills the buffer folds the buffer
 * into the checkpoint and writes the checkpoint once.  Speculative drafts are
 * appended to the buffer, the accepted prefix advances the buffer pointer and
 * a rollback resets it.  Layers: Mamba-2 and Gated DeltaNet.
 *
 * Pages the operations follow:
 *   [DE] "ReplaySSM beschleunigt das Decoding von Hybridmodellen durch Caching
 *        der Eingaben statt des Zustands" -- sections "Was passiert ist" and
 *        "Wie es funktioniert" (checkpoint + input buffer, flush when full,
 *        pointer reset on rejected drafts).
 *   [TR] "NVIDIA ve Dao AI Lab, hibrit model cozumlemesini hizlandirmak icin
 *        ReplaySSM'i sundu" -- sections "ReplaySSM nasil calisir?" (16-entry
 *        buffer, non-flush and flush steps, outputs equal ordinary decoding up
 *        to rounding), "Durum trafigini azaltma ve rollback'in
 *        basitlestirilmesi" (one checkpoint write per window, drafts appended
 *        unverified, accepted prefix advances the pointer, output-only draft
 *        evaluation) and "Kuantizasyon hatasinin sinirlandirilmasi"
 *        (high-precision checkpoint for the recurrence, low-precision copy for
 *        reads).
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers unless stated otherwise.  The
 *     caller owns all device memory (the state region, inputs, outputs,
 *     baseline states and snapshots) and all streams; the library owns only
 *     the host-side handle.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream`; nothing synchronizes.
 *   - Host-side validation happens before anything is enqueued.  On a non-OK
 *     return nothing was enqueued and the state is unchanged; replay_last_error()
 *     then holds a message (thread-local).
 *   - REPLAY_ERR_HIP reports a launch error from the HIP runtime.
 *   - Device-side anomalies never trap: they set sticky bits in the state's
 *     device error word (replay_read_book).
 *   - Pointers to inputs, outputs and states must be 16-byte aligned; the
 *     state region must be 256-byte aligned.  Outputs must not alias inputs.
 *   - A handle must not be used from two streams without caller ordering.
 *
 * Tensor layouts (row-major, logical):
 *   Mamba-2  x [T][B][H][P], Bm and Cm [T][B][G][N], dt [T][B][H]
 *            (all in `io_dtype`), A and D [H] fp32, y [T][B][H][P] io_dtype,
 *            checkpoint (logical) [B][H][P][N] in `ckpt_dtype`.
 *   GDN      q and k [T][B][G][DK], v [T][B][H][DV] (io_dtype), alpha and
 *            beta [T][B][H] fp32, o [T][B][H][DV] io_dtype, checkpoint
 *            (logical) [B][H][DV][DK] in `ckpt_dtype`.
 *   T = 1 for a decode step, T = k for k speculative drafts.
 *   Head h reads B/C (Mamba-2) or q/k (GDN) of group h / (H / G).
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define REPLAY_ABI_VERSION 1
#define REPLAY_MAX_BUF 16

typedef enum {
    REPLAY_OK = 0,
    REPLAY_ERR_ARG = 1,         /* NULL pointer or bad scalar argument          */
    REPLAY_ERR_SHAPE = 2,       /* unsupported or inconsistent dimensions       */
    REPLAY_ERR_DTYPE = 3,       /* unsupported dtype combination                */
    REPLAY_ERR_ALIGN = 4,       /* pointer alignment or region size             */
    REPLAY_ERR_STATE = 5,       /* operation not allowed in the current phase   */
    REPLAY_ERR_CAPACITY = 6,    /* draft count outside [1, buf_cap]             */
    REPLAY_ERR_UNSUPPORTED = 7, /* valid request this build does not implement  */
    REPLAY_ERR_HIP = 8          /* HIP runtime error                            */
} replay_status;

typedef enum { REPLAY_MAMBA2 = 0, REPLAY_GDN = 1 } replay_kind;

typedef enum {
    REPLAY_NONE = 0,
    REPLAY_F32 = 1,
    REPLAY_F16 = 2,
    REPLAY_BF16 = 3,
    REPLAY_FP8_E4M3 = 4,    /* OCP FP8 E4M3 ("fn"), unscaled, RNE, saturating at +-448 */
    REPLAY_MXFP4 = 5        /* OCP MX FP4 E2M1, one E8M0 scale per 32 elements          */
} replay_dtype;

/* Recurrence checkpoint dtype.  REPLAY_F32, REPLAY_F16 (IEEE binary16) or
 * REPLAY_FP8_E4M3 (OCP E4M3, unscaled, RNE, saturating at +-448; the [TR]
 * page, section "Kuantizasyon hatasinin sinirlandirilmasi", pairs
 * low-precision reads with an FP16 or FP8 recurrence).  A fold decodes the
 * low-precision checkpoint to fp32, folds in fp32, rounds the result to the
 * checkpoint dtype (RNE) right away -- that step's outputs and the read copy
 * see the rounded values -- and writes it once.  Non-flush steps read half
 * (fp16) or a quarter (FP8) of the bytes of fp32.  An FP8 checkpoint takes no
 * read copy or an MXFP4 one (an FP8 copy would repeat the checkpoint:
 * REPLAY_ERR_UNSUPPORTED).  FP8 tiles use the read copy's strip layout. */

/* Device error word bits (sticky; cleared by replay_load_checkpoint). */
#define REPLAY_DEVERR_COMMIT_CLAMPED 0x1u  /* an accepted count was outside [0, pend] */

/* Configuration flags. */
#define REPLAY_FLAG_VALU_FOLD 0x1   /* Mamba-2, fp32 checkpoint: fold with vector FMAs instead
                                       of MFMA (cross-check) */
/* Keep the checkpoint itself at the read copy's precision (comparison variant:
 * a low-precision state inside the recurrence).  Needs read_copy != NONE and an
 * fp32 checkpoint.  The
 * checkpoint is rounded to the copy's grid at load and right after every fold
 * (before that step's outputs); the fp32 region then mirrors the copy exactly. */
#define REPLAY_FLAG_QUANTIZED_CKPT 0x2
/* Staggered flush phases: after a load, sequence b's first window ends after
 * 1 + (b mod buf_cap) decode tokens instead of buf_cap, so that in lockstep
 * decoding only about batch/buf_cap sequences fold on any one step and every
 * step costs about the same; later windows have buf_cap tokens.  An explicit
 * replay_flush ends the stagger for the sequences it folds.  Values do not
 * depend on when folds happen (up to rounding); only the flush schedule does. */
#define REPLAY_FLAG_STAGGER_FLUSH 0x4
/* MXFP4 read copy only (else REPLAY_ERR_ARG): give each 32-element group the
 * smallest shared exponent X with amax <= 6 * 2^X, so that no element saturates
 * (the default rule's X = floor(log2 amax) - 2, plus one when amax's
 * significand exceeds 1.5).  The default rule is the conversion of the OCP
 * Microscaling Formats specification; it clips amax / 2^X in (6, 8) to 6.
 * Same layout and cost; only the E8M0 values and the codes of such groups
 * differ. */
#define REPLAY_FLAG_MX_SCALE_CEIL 0x8

typedef struct {
    int32_t abi_version;  /* REPLAY_ABI_VERSION                                  */
    int32_t kind;         /* replay_kind                                         */
    int32_t batch;        /* B >= 1; B * H * max(H, 256) < 2^32 (REPLAY_ERR_SHAPE) */
    int32_t nheads;       /* H >= 1                                              */
    int32_t ngroups;      /* G >= 1, divides H (Mamba-2 B/C groups; GDN q/k heads)*/
    int32_t head_dim;     /* Mamba-2 P; GDN DV.  Multiple of 16, <= 256          */
    int32_t state_dim;    /* Mamba-2 N; GDN DK.  16, 32, 64, 128 or 256          */
    int32_t buf_cap;      /* buffer capacity, 1..16                              */
    int32_t ckpt_dtype;   /* REPLAY_F32 | REPLAY_F16 | REPLAY_FP8_E4M3 (recurrence checkpoint) */
    int32_t read_copy;    /* REPLAY_NONE | REPLAY_FP8_E4M3 | REPLAY_MXFP4        */
    int32_t io_dtype;     /* REPLAY_F32 | REPLAY_BF16 (token inputs and outputs) */
    int32_t flags;        /* REPLAY_FLAG_*                                       */
    float scale;          /* GDN output scale (o = scale * S q); ignored for Mamba-2 */
} replay_config;

/* Per-call inputs.  Unused fields must be NULL.  A and D (Mamba-2 layer
 * parameters, fp32 [H]) are needed by every call that computes values;
 * replay_flush needs only A. */
typedef struct {
    const void *x, *B, *C, *dt;     /* Mamba-2 token inputs (io_dtype)  */
    const float *A, *D;             /* Mamba-2 parameters               */
    const void *q, *k, *v;          /* GDN token inputs (io_dtype)      */
    const float *alpha, *beta;      /* GDN gates (fp32)                 */
} replay_inputs;

/* Byte offsets inside the caller's state region (for inspection/tests). */
typedef struct {
    uint64_t total_bytes;
    uint64_t ckpt_off, ckpt_bytes;     /* checkpoint, fragment-ordered tiles   */
    uint64_t rcopy_off, rcopy_bytes;   /* read copy element codes              */
    uint64_t rscale_off, rscale_bytes; /* MXFP4 E8M0 scales                    */
    uint64_t buf_off[4], buf_bytes[4]; /* buffer arrays, 2 banks each          */
    uint64_t book_off, book_bytes;     /* int32 [2][4][B]: len, pend, fc, window limit */
    uint64_t err_off;                  /* uint32 device error word             */
} replay_layout;

typedef struct replay_state replay_state; /* opaque host handle */

/* ---- library info ------------------------------------------------------ */
int32_t replay_abi_version(void);
const char *replay_status_str(int32_t status);
/* Message for the last non-OK return on this thread ("" if none). */
const char *replay_last_error(void);

/* ---- state lifetime ----------------------------------------------------- */
/* Validates a configuration without touching the GPU. */
replay_status replay_config_check(const replay_config *cfg);
/* Bytes of device memory a state needs (0 if the configuration is invalid). */
size_t replay_state_bytes(const replay_config *cfg);
/* Binds caller-owned device memory (>= replay_state_bytes, 256-byte aligned)
 * to a new handle and enqueues its initialisation: zero checkpoint, empty
 * buffer, len = pend = fc = 0, error word 0.  The memory stays owned by the
 * caller and must outlive the handle. */
replay_status replay_state_alloc(const replay_config *cfg, void *dev_mem, size_t bytes,
                                 void *stream, replay_state **out);
/* Frees the host handle only.  REPLAY_ERR_STATE while the state is bound to a
 * stack (free the stack first). */
replay_status replay_state_free(replay_state *st);
replay_status replay_state_layout(const replay_state *st, replay_layout *out);
/* Host-side phase: 0 = idle, 1 = drafts pending. */
int32_t replay_state_phase(const replay_state *st);

/* ---- checkpoint I/O ----------------------------------------------------- */
/* Logical checkpoints at the boundary are [B][H][rows][cols] arrays in the
 * state's ckpt_dtype (float, IEEE binary16 or E4M3 bytes), rows = P or DV,
 * cols = N or DK.
 * Loads a logical checkpoint (device), refreshes the read copy, empties the
 * buffer and resets len = pend = fc = 0 and the error word.  Not allowed
 * while drafts are pending. */
replay_status replay_load_checkpoint(replay_state *st, const void *S_logical, void *stream);
/* As replay_load_checkpoint, from an fp32 logical checkpoint [B][H][rows][cols]
 * (device) whatever the state's ckpt_dtype: the library rounds each value on
 * the device with the encoder its folds use -- IEEE binary16 round to nearest
 * even (overflow to +-inf) for REPLAY_F16; OCP E4M3 round to nearest even,
 * finite and infinite magnitudes beyond 448 saturated to +-448, NaN to 0x7f
 * for REPLAY_FP8_E4M3 ([TR] "Kuantizasyon hatasinin sinirlandirilmasi": FP16
 * or FP8 recurrence).  For an fp32 checkpoint it equals replay_load_checkpoint. */
replay_status replay_load_checkpoint_f32(replay_state *st, const float *S_logical, void *stream);
/* Per-sequence arrival: a prefill hands over the state of n sequences, which
 * (re)occupy batch slots slots[0..n-1] (HOST int32 array; distinct, each in
 * [0, B), 1 <= n <= B, else REPLAY_ERR_ARG).  S_logical (device fp32
 * [n][H][rows][cols], slot i's checkpoint at index i) is rounded to the
 * ckpt_dtype as in replay_load_checkpoint_f32 and becomes those sequences'
 * checkpoint; their read copy is refreshed, their buffer emptied and their
 * len = pend = fc = 0 with a full window of buf_cap entries (also under
 * REPLAY_FLAG_STAGGER_FLUSH: an arrival's window already starts at its own
 * time).  Every other sequence keeps its checkpoint, buffer and bookkeeping;
 * the error word is kept.  Not allowed while drafts are pending ([DE] "Warum
 * es wichtig ist": the gain comes from many concurrent sequences; [TR]
 * "ReplaySSM nasil calisir?": every sequence flushes its own buffer). */
replay_status replay_load_slots(replay_state *st, int32_t n, const int32_t *slots, const float *S_logical,
                                void *stream);
/* Writes the current checkpoint (not including buffered tokens) in logical
 * layout and ckpt_dtype to S_out (device). */
replay_status replay_read_checkpoint(const replay_state *st, void *S_out, void *stream);
/* Writes the read copy in logical element order: one byte per element
 * (FP8 code, or FP4 code in the low nibble) to codes_out [B][H][rows][cols],
 * and for MXFP4 the E8M0 scales to scales_out [B][H][rows][cols/32]
 * (may be NULL otherwise).  REPLAY_ERR_STATE if the state has no read copy. */
replay_status replay_read_copy(const replay_state *st, uint8_t *codes_out, uint8_t *scales_out,
                               void *stream);
/* Copies the bookkeeping to book_out (device int32 [3][B]: len, pend, fc) and,
 * if err_out is not NULL, the device error word to err_out (device uint32). */
replay_status replay_read_book(const replay_state *st, int32_t *book_out, uint32_t *err_out,
                               void *stream);

/* ---- the decode path ---------------------------------------------------- */
/* One decode token for every sequence.  Per sequence: if the buffer is
 * already full (possible after a commit), the buffer is folded first; the
 * token's inputs are appended; if that fills the buffer, the buffer is folded
 * into the checkpoint, which is written once, and the buffer is emptied.
 * Outputs y [1][B][H][P] (Mamba-2) or [1][B][H][DV] (GDN) in io_dtype.
 * Not allowed while drafts are pending. */
replay_status replay_decode_step(replay_state *st, const replay_inputs *in, void *y, void *stream);
/* replay_decode_step for the sequences whose active[b] (device uint8 [B]) is
 * nonzero.  A sequence with active[b] == 0 sits the step out: nothing is
 * appended to its buffer, nothing is folded or written for it, its rows of y
 * are left as they were and its len, fc and window are unchanged (departed or
 * idle slots of a serving batch).  The mask is read by the step's kernel on
 * `stream`. */
replay_status replay_decode_step_masked(replay_state *st, const replay_inputs *in, const uint8_t *active, void *y,
                                        void *stream);
/* Folds every non-empty buffer into its checkpoint (one write per sequence
 * that had entries); len = 0.  Uses only in->A (Mamba-2).  Not allowed while
 * drafts are pending. */
replay_status replay_flush(replay_state *st, const replay_inputs *in, void *stream);
/* Appends k draft tokens (inputs [k][B][...]) to every sequence's buffer
 * without verification and writes their outputs y [k][B][H][P or DV]; no
 * state is written unless a sequence's committed entries plus k exceed the
 * capacity, in which case its committed prefix is folded first.  Requires
 * 1 <= k <= buf_cap (else REPLAY_ERR_CAPACITY) and no pending drafts. */
replay_status replay_spec_append(replay_state *st, int32_t k, const replay_inputs *drafts,
                                 void *y, void *stream);
/* replay_spec_append for the sequences whose active[b] is nonzero (device
 * uint8 [B]); the others append no drafts (pend stays 0, so their accepted
 * count must be 0 at the commit), write no outputs and keep their buffer and
 * bookkeeping.  The drafts are pending for the whole state afterwards. */
replay_status replay_spec_append_masked(replay_state *st, int32_t k, const replay_inputs *drafts,
                                        const uint8_t *active, void *y, void *stream);
/* accepted: device int32 [B].  len += clamp(accepted[b], 0, pend); pend = 0.
 * A clamped value sets REPLAY_DEVERR_COMMIT_CLAMPED.  Moves no state bytes.
 * Requires pending drafts. */
replay_status replay_spec_commit(replay_state *st, const int32_t *accepted, void *stream);
/* Drops every pending draft (pointer reset; commit of 0). */
replay_status replay_spec_rollback(replay_state *st, void *stream);

/* ---- layer stacks --------------------------------------------------------
 * A hybrid model interleaves several SSM layers with a few attention layers
 * ([TR] "NVIDIA ve Dao AI Lab ...", section "ReplaySSM nasil calisir?"; the
 * decode-step speedups of section "Durum trafigini azaltma ve rollback'in
 * basitlestirilmesi" are measured on such models).  Every SSM layer of the model decodes the same
 * token positions of the same sequences, so the buffer bookkeeping (len, pend,
 * fc and the window limit per sequence) is one set for the whole model: a
 * stack keeps it once, every layer's step follows it, and a speculative commit
 * or rollback is one pointer update for all layers.
 *
 * Members are ordinary states (Mamba-2 and GDN may be mixed) with equal batch
 * and buf_cap and the same REPLAY_FLAG_STAGGER_FLUSH setting.  While bound to
 * a stack a member refuses its own load, decode, flush, spec, commit and
 * rollback calls (REPLAY_ERR_STATE); replay_read_checkpoint / replay_read_copy
 * still work on it.  A model step calls the layer entry points once per layer
 * in layer order (the caller computes layer l+1's inputs from layer l's
 * outputs in between); after the last layer the shared bookkeeping advances.
 * A call out of order, or a spec step whose k differs from the step's first
 * layer, returns REPLAY_ERR_STATE and launches nothing.
 */
typedef struct replay_stack replay_stack; /* opaque host handle */

/* Binds nlayers (>= 1) states into a stack, in layer order, and resets the
 * shared bookkeeping (len = pend = fc = 0, error word 0) on `stream`.  The
 * states must be idle and in no other stack.  The stack keeps the pointers; it
 * owns no device memory of its own (layer 0's bookkeeping region is the shared
 * one). */
replay_status replay_stack_create(replay_state *const *layers, int32_t nlayers, void *stream,
                                  replay_stack **out);
/* Unbinds the members and frees the handle.  A former member must be loaded
 * (replay_load_checkpoint) before it steps on its own again. */
replay_status replay_stack_free(replay_stack *stk);
/* Loads every layer's logical checkpoint (S_logical[l], device, in that
 * layer's ckpt_dtype), refreshes read copies and resets the shared
 * bookkeeping.  Not allowed mid-step or while drafts are pending. */
replay_status replay_stack_load(replay_stack *stk, const void *const *S_logical, void *stream);
/* As replay_stack_load from fp32 logical checkpoints, rounded by the library
 * (replay_load_checkpoint_f32). */
replay_status replay_stack_load_f32(replay_stack *stk, const float *const *S_logical, void *stream);
/* Per-sequence arrival for every layer (replay_load_slots): S_logical[l] is
 * layer l's device fp32 [n][H_l][rows_l][cols_l]; the shared bookkeeping of the
 * listed slots is reset once.  Not allowed mid-step or while drafts are
 * pending. */
replay_status replay_stack_load_slots(replay_stack *stk, int32_t n, const int32_t *slots,
                                      const float *const *S_logical, void *stream);
/* Layer `layer`'s decode step (as replay_decode_step).  Must be the next
 * layer of the current step. */
replay_status replay_stack_decode_layer(replay_stack *stk, int32_t layer, const replay_inputs *in,
                                        void *y, void *stream);
/* Layer `layer`'s spec append of k drafts (as replay_spec_append).  Every
 * layer of the step appends the same k; after the last layer the drafts are
 * pending for the whole stack. */
replay_status replay_stack_spec_layer(replay_stack *stk, int32_t layer, int32_t k,
                                      const replay_inputs *drafts, void *y, void *stream);
/* Masked variants (replay_decode_step_masked, replay_spec_append_masked):
 * every layer of one step must pass the same `active` pointer (else
 * REPLAY_ERR_STATE), and its contents must not change during the step. */
replay_status replay_stack_decode_layer_masked(replay_stack *stk, int32_t layer, const replay_inputs *in,
                                               const uint8_t *active, void *y, void *stream);
replay_status replay_stack_spec_layer_masked(replay_stack *stk, int32_t layer, int32_t k,
                                             const replay_inputs *drafts, const uint8_t *active, void *y,
                                             void *stream);
/* Folds every non-empty buffer of every layer (in[l] as for replay_flush;
 * in may be NULL for an all-GDN stack). */
replay_status replay_stack_flush(replay_stack *stk, const replay_inputs *const *in, void *stream);
/* One commit (accepted: device int32 [B]) or rollback for every layer. */
replay_status replay_stack_commit(replay_stack *stk, const int32_t *accepted, void *stream);
replay_status replay_stack_rollback(replay_stack *stk, void *stream);
/* The shared bookkeeping, as replay_read_book. */
replay_status replay_stack_read_book(const replay_stack *stk, int32_t *book_out, uint32_t *err_out,
                                     void *stream);
/* Number of layers; the layer the current step expects next (0 between
 * steps); 0 idle or 1 drafts pending.  -1 for a NULL handle. */
int32_t replay_stack_layers(const replay_stack *stk);
int32_t replay_stack_next_layer(const replay_stack *stk);
int32_t replay_stack_phase(const replay_stack *stk);

/* ---- in-run conventional baselines --------------------------------------
 * Ordinary decoding on a plain logical state [B][H][rows][cols] in the
 * config's ckpt_dtype (load, decay and update, output, store per token; a
 * low-precision state is updated in fp32, the output is read from that update
 * and the state is stored RNE), tuned like the replay kernels.  read_copy and flags
 * are ignored. */
replay_status replay_conv_decode_step(const replay_config *cfg, void *S, const replay_inputs *in,
                                      void *y, void *stream);
/* k draft steps from S (read once, not written); snapshot j (the state after
 * draft j) goes to snaps + j * B*H*rows*cols elements; outputs y [k][B][...]. */
replay_status replay_conv_spec_step(const replay_config *cfg, const void *S, void *snaps,
                                    int32_t k, const replay_inputs *drafts, void *y, void *stream);
/* S[b] = snaps[accepted[b] - 1][b] where 1 <= accepted[b] <= k; unchanged
 * otherwise.  accepted: device int32 [B]. */
replay_status replay_conv_spec_restore(const replay_config *cfg, void *S, const void *snaps,
                                       int32_t k, const int32_t *accepted, void *stream);

/* ---- stand-in non-SSM layers ----------------------------------------------
 * A hybrid model's decode step also runs its mixers' dense projections and a
 * few attention layers ([TR] "NVIDIA ve Dao AI Lab ...", section "ReplaySSM
 * nasil calisir?": SSM layers interleaved with attention layers); the pages'
 * decode-step speedups are the SSM gain diluted by them (section "Durum
 * trafigini azaltma ve rollback'in basitlestirilmesi").  These two calls are
 * that rest of a step, with caller-provided random weights and caches, so a
 * model step can be timed with replayed and with conventional SSM layers.
 * Both are plain definitions (no buffer or checkpoint): */
/* Y[m][n] = sum_k X[m][k] W[n][k]: X [M][K], W [N][K] (one output feature's
 * weights contiguous), Y [M][N]; all bf16, row-major, fp32 accumulation, Y
 * rounded to nearest even.  Needs K a positive multiple of 64 and M, N >= 1
 * (else REPLAY_ERR_SHAPE). */
replay_status replay_standin_linear(const void *X, const void *W, void *Y, int32_t M, int32_t K, int32_t N,
                                    void *stream);
/* Decode attention of one query token per sequence: for sequence b and query
 * head h (key/value head g = h / (Hq / Hkv)),
 *   o[b][h] = sum_t softmax_t(scale * q[b][h] . K[b][g][t]) V[b][g][t]
 * over the L cached tokens.  q row b starts at q + b * q_stride elements (its
 * Hq heads of D values contiguous), K and V are [B][Hkv][L][D], o is
 * [B][Hq][D]; all bf16, fp32 softmax and accumulation.  D must be 128 and
 * Hq / Hkv one of 1, 2, 4, 8 (else REPLAY_ERR_UNSUPPORTED). */
replay_status replay_standin_attention(const void *q, int64_t q_stride, const void *K, const void *V, void *o,
                                       int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t L, float scale,
                                       void *stream);

/* ---- measurement helpers ------------------------------------------------ */
/* Streaming copy of `bytes` (multiple of 16) from src to dst: the in-run
 * bandwidth ceiling and the reference for hardware byte counters. */
replay_status replay_stream_copy(void *dst, const void *src, size_t bytes, void *stream);
/* Streaming read of `bytes` (multiple of 16, else REPLAY_ERR_ALIGN) of fp32
 * values from src, in the replay kernels' access pattern (one 32 KiB tile per
 * workgroup, 128-bit nontemporal loads): the read-only bandwidth ceiling that
 * non-flush steps are measured against.  partials (device, caller-owned,
 * max(1, ceil(bytes / 32768)) floats) receives the sum of each 32 KiB tile's
 * values, the last tile ragged; every entry is overwritten. */
replay_status replay_stream_read(const void *src, size_t bytes, float *partials, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* REPLAYSSM_H */
