/*
 * r2l_scan.h -- C ABI of the MI355X (gfx950) selective-scan library libr2l_scan.so.
 *
 * The library runs the hot path of the Bifocal dLLM / R2LM method and of its
 * block-diffusion companion:
 *
 *  - r2l_scan: the right-to-left (R2L) stream. "Bifocal Diffusion Language
 *    Models" (gist.science nl and fr technical summaries, section 2
 *    "Methodology") describes a sidecar that reverses the backbone's hidden
 *    states, runs a Mamba selective scan over them and reverses the result
 *    back, producing a residual correction Delta^R2L that a learnable scalar s
 *    (initialised at zero, so that the model starts out identical to the
 *    causal backbone) adds to the hidden states. During denoising the scan
 *    covers the generation block only. The reversal is folded into the index
 *    math here: nothing is flipped in memory.
 *  - prefix_scan_state: the forward-only Mamba boundary state after each
 *    prefix ("Training Hybrid Block Diffusion Language Models with Partial
 *    Bidirectionality", nl summary, "Methodology" item 1: completed prefix
 *    blocks are cached as forward-only boundary states that depend on the
 *    clean prefix alone).
 *  - block_commit_state: the same cache advanced over a committed block (same
 *    passage and item 3: the cache is built by scanning the clean prefix, and
 *    finished blocks become prefix).
 *
 * The recurrence (the pages name "selective scan (Mamba)" without writing it
 * out; this is the Mamba-1 reading, with zero-order hold for A and an Euler
 * step for B). For each sequence, channel d < D and state n < N, visiting the
 * tokens right to left (r2l_scan) or left to right (the other two):
 *
 *     Delta_t = delta_softplus ? log(1 + exp(dt[t,d])) : dt[t,d]
 *     h_n     = exp(Delta_t * A[d,n]) * h_n + Delta_t * Bm[t,n] * x[t,d]
 *     y_t     = sum_n Cm[t,n] * h_n + Dskip[d] * x[t,d]
 *     out[t,d] = res == NULL ? y_t : (s == 0 ? res[t,d] : res[t,d] + s * y_t)
 *
 * h starts from h_in (or zero) before the first visited token; h_out receives
 * the state after the last visited token. All arithmetic is fp32 (state, Delta,
 * exponentials, sums) whatever the storage type of the inputs.
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 *  Layout   Token-major, the last dimension contiguous. x, dt, res and out are
 *           [tokens, D] with a token stride in elements (>= D); Bm and Cm are
 *           [tokens, N] with a token stride (>= N), shared by all channels.
 *           In the dense layout each of them also has a batch stride, so a
 *           slice [:, a:b] of a [batch, L, .] tensor is taken as it is;
 *           A is [D, N] fp32 contiguous; Dskip is [D] fp32; h_in / h_out are
 *           [batch, D, N] fp32 contiguous.
 *  Batches  Dense: batch sequences of seqlen tokens each, sequence b owning
 *           rows b*seqlen .. (b+1)*seqlen-1. Ragged: cu_seqlens (device memory,
 *           int32 [batch+1], cu_seqlens[0] = 0, non-decreasing) gives each
 *           sequence's rows; total_tokens (host) must equal cu_seqlens[batch]
 *           and max_seqlen (host) must bound every length. Length-0 sequences
 *           are legal: they write no rows and h_out = h_in (or zero). The
 *           ragged fields are taken on trust (they live on the device); the
 *           library only checks them when the environment variable
 *           R2L_CHECK_SEQLENS=1 is set, at the price of a synchronous copy.
 *  Memory   Every pointer except `a` itself is device memory. The caller owns
 *           every buffer; the library allocates nothing, keeps no state
 *           between calls and is safe to call from several host threads.
 *           (Exceptions, each described where it is declared: the GEMM
 *           context the sidecar block's caller creates and passes in, and
 *           r2l_scan_noalloc's scratch array.)
 *  Streams  `stream` is a hipStream_t (NULL: the null stream). Work is queued
 *           on it and the call returns without waiting.
 *  Aliasing out may be exactly x and/or exactly res (same base pointer and
 *           strides): the in-place hook update. h_out may be exactly h_in. Any
 *           other overlap between an output and any other buffer returns
 *           R2L_ERR_ALIAS. Overlap is judged on the address span each tensor's
 *           strides reach, so interleaved layouts count as overlapping.
 *  Alignment Element alignment for x, dt, Bm, Cm, res, out; 16 bytes for A,
 *           h_in and h_out; 4 bytes for Dskip.
 *  Errors   Every argument is checked on the host before anything is queued;
 *           on error nothing is launched and nothing is written.
 *           r2l_last_error() then describes the first failed check. Faults
 *           inside kernels surface at the caller's next synchronisation.
 *  NaN/Inf  Propagate; nothing is trapped. With s == 0 the output is the
 *           residual bit for bit, whatever y holds.
 *  s == 0   (with res given) No readout runs: out receives a copy of res (no
 *           launch at all when out is res itself), and the state is still
 *           scanned when h_out is given (bit-identical to the state of the
 *           same call with s != 0).
 */
#ifndef R2L_SCAN_H_
#define R2L_SCAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define R2L_ABI_VERSION 8

/* exported from libr2l_scan.so (everything else in it is hidden) */
#if defined(__GNUC__)
#define R2L_API __attribute__((visibility("default")))
#else
#define R2L_API
#endif

typedef int32_t r2l_status;
#define R2L_OK 0
#define R2L_ERR_INVALID_ARG (-1) /* a required pointer is NULL, a size or stride is out of range */
#define R2L_ERR_UNSUPPORTED (-2) /* dtype or state size N not built (N must be 16) */
#define R2L_ERR_ALIAS (-3)       /* an output overlaps another buffer other than as allowed */
#define R2L_ERR_MISALIGNED (-4)  /* a pointer breaks the alignment rules above */
#define R2L_ERR_WORKSPACE (-5)   /* workspace missing or smaller than r2l_workspace_size */
#define R2L_ERR_HIP (-6)         /* the HIP runtime refused a launch or a query */

/* element type of x, dt, Bm, Cm, res and out */
#define R2L_DTYPE_F32 0
#define R2L_DTYPE_BF16 1

/* operation codes for r2l_workspace_size */
#define R2L_OP_SCAN 0
#define R2L_OP_PREFIX 1
#define R2L_OP_COMMIT 2
#define R2L_OP_BIDIR 3
#define R2L_OP_SAVE 4          /* r2l_scan_save */
#define R2L_OP_PREFIX_SAVE 5   /* prefix_scan_save */

typedef struct r2l_scan_args {
    /* ---- shape ---- */
    int64_t batch;              /* sequences, >= 0 */
    int64_t seqlen;             /* dense: tokens per sequence, >= 0 (ignored when ragged) */
    const int32_t *cu_seqlens;  /* ragged: device int32 [batch+1]; NULL selects dense */
    int64_t total_tokens;       /* ragged: cu_seqlens[batch], known on the host */
    int64_t max_seqlen;         /* ragged: an upper bound of every sequence length */
    int64_t dim;                /* D, channels, >= 1 */
    int32_t dstate;             /* N, state size; 16 is built */
    int32_t dtype;              /* R2L_DTYPE_* of x, dt, Bm, Cm, res, out */

    /* ---- inputs ----
     * Each token-major tensor has a token stride and, for the dense layout, a
     * batch stride (elements between sequence b and b+1; 0 = seqlen * token
     * stride, i.e. packed). Ragged layouts ignore the batch strides. */
    const void *x;   int64_t x_stride;  int64_t x_batch_stride;  /* [tokens, D] scan input (hidden states) */
    const void *dt;  int64_t dt_stride; int64_t dt_batch_stride; /* [tokens, D] step input before softplus */
    const void *Bm;  int64_t Bm_stride; int64_t Bm_batch_stride; /* [tokens, N] input matrix rows */
    const void *Cm;  int64_t Cm_stride; int64_t Cm_batch_stride; /* [tokens, N] readout rows (unused by state-only calls) */
    const float *A;                      /* [D, N] state matrix (diagonal per channel), fp32 */
    const float *Dskip;                  /* [D] skip weights, fp32, or NULL for zero */
    int32_t delta_softplus;              /* 1: Delta = softplus(dt); 0: Delta = dt */

    /* ---- planning hints (0 = let the library choose) ----
     * chunk_tokens  > 0: split every sequence into chunks of this many tokens
     *               and join them with the carry pass (needs workspace);
     *               < 0: never split; 0: split when the shape needs it.
     * state_split   1, 2 or 4 lanes share one channel's N states; 0: choose.
     * Results differ between plans by rounding only. */
    int32_t chunk_tokens;
    int32_t state_split;

    /* ---- state ---- */
    const float *h_in;                   /* [batch, D, N] initial state, or NULL for zero */
    float *h_out;                        /* [batch, D, N] final state, or NULL */

    /* ---- output ---- */
    const void *res; int64_t res_stride; int64_t res_batch_stride; /* [tokens, D] residual base, or NULL */
    float s;                                                       /* residual gate */
    void *out; int64_t out_stride; int64_t out_batch_stride;       /* [tokens, D] */

    /* ---- scratch for chunked plans ---- */
    void *workspace;                     /* device, 256-byte aligned, or NULL */
    size_t workspace_bytes;
} r2l_scan_args;

/*
 * r2l_scan -- the R2L stream over each sequence (the generation block during
 * denoising, the whole prompt at prefill). Tokens are visited right to left
 * starting from h_in (NULL: zero state at the right edge), y is read out at
 * every token and out receives y or the gated residual at the token's own
 * position. Required: x, dt, Bm, Cm, A, out. Optional: Dskip, h_in, h_out,
 * res. h_out receives the state after the leftmost token.
 * Source: "Bifocal Diffusion Language Models", section 2 (reverse, scan,
 * reverse back, residual through s; scan over generation tokens only), and
 * "Training Hybrid Block Diffusion ...", "Methodology" item 1 (reverse scan
 * limited to the active block).
 */
R2L_API r2l_status r2l_scan(const r2l_scan_args *a, void *stream);

/*
 * r2l_scan_noalloc -- r2l_scan for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, checks and results as r2l_scan, except:
 *  - the workspace fields are ignored: a chunked plan's carry data goes to a
 *    scratch array of R2L_NOALLOC_SCRATCH_BYTES that the library holds in
 *    device memory on each GPU it runs on, for the life of the process (its
 *    address is looked up on the first call on each device);
 *  - a plan needing more scratch than that returns R2L_ERR_WORKSPACE and
 *    launches nothing (r2l_workspace_size with R2L_OP_SCAN tells the need);
 *  - the optional R2L_CHECK_SEQLENS copy is not made.
 * Nothing is allocated, by the library or by any routine it calls. Every
 * word of scratch a launch reads was written earlier in the same call, so
 * nothing is cleared between calls. All calls on one GPU share its scratch:
 * calls on one stream are ordered, but calls that may overlap on one GPU (other
 * streams, other host threads) race on it and must not be made.
 */
#define R2L_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
R2L_API r2l_status r2l_scan_noalloc(const r2l_scan_args *a, void *stream);

/*
 * prefix_scan_state -- the forward-only boundary state of each prefix: tokens
 * visited left to right from h_in (NULL: zero), h_out = the state after the
 * last token. If out is given, y (or the gated residual) is also written,
 * which is the forward continuation of a block resumed from a cached state;
 * Cm is then required. At least one of h_out and out is required.
 * Source: "Training Hybrid Block Diffusion ...", "Methodology" items 1-2
 * (forward-only boundary states; a timestep-free prefix operator followed by
 * the active-block continuation).
 */
R2L_API r2l_status prefix_scan_state(const r2l_scan_args *a, void *stream);

/*
 * block_commit_state -- advance cached boundary states over committed blocks,
 * in place: h_out holds the state before the call and receives the state
 * after each sequence's block. h_in must be NULL or equal to h_out. out is an
 * optional forward readout over the block (then Cm is required).
 * Source: "Training Hybrid Block Diffusion ...", "Methodology" items 1 and 3
 * (the cache is built by scanning the clean prefix; completed blocks join it).
 */
R2L_API r2l_status block_commit_state(const r2l_scan_args *a, void *stream);

/*
 * r2l_workspace_size -- bytes of workspace that the plan for operation `op`
 * (R2L_OP_*) with these arguments needs; 0 when the plan does not chunk (and,
 * for R2L_OP_BIDIR, runs no readout).
 * Only the shape fields and the planning hints are read. Returns R2L_OK and
 * writes *bytes, or an error status.
 */
R2L_API r2l_status r2l_workspace_size(int32_t op, const r2l_scan_args *a, size_t *bytes);

/*
 * Gradients of r2l_scan, for training the R2L stream (the pages train the
 * sidecar jointly with the backbone, or, plug-in, only the sidecar and s).
 * The forward call is described by the same r2l_scan_args (x, dt, Bm, Cm, A,
 * Dskip, h_in, res, s, delta_softplus, layout; out, h_out, state_split and the
 * workspace fields are not read). chunk_tokens is the planning hint of the
 * backward's forward state pass (rounded up to a multiple of 8 tokens; the
 * same meaning of > 0, < 0 and 0 as above). With a residual,
 * dL/dy = s * dout; without, dL/dy = dout. A separate residual's gradient is
 * dout itself and is not written; when the residual is x, dx includes dout.
 *
 * Layout: dout, dx, ddt are token-major like x (element strides, batch
 * strides in the dense layout, 0 = contiguous) in the storage type of x;
 * every other gradient is fp32 and contiguous: dBm, dCm [tokens, dstate]
 * with tokens packed (dense: row b * seqlen + l), dA [dim, dstate],
 * dDskip [dim], dh_in [batch, dim, dstate], ds [1]. dh_out (dL/dh_out) is
 * optional. Every output may be NULL (not computed); ds needs a residual.
 * Outputs may not overlap each other or any input.
 */
typedef struct r2l_grad_args {
    const void *dout;   int64_t dout_stride, dout_batch_stride;   /* dL/dout, required */
    const float *dh_out;                                        /* [batch, dim, dstate] or NULL */
    void *dx;           int64_t dx_stride, dx_batch_stride;
    void *ddt;          int64_t ddt_stride, ddt_batch_stride;
    float *dBm;
    float *dCm;
    float *dA;
    float *dDskip;
    float *dh_in;
    float *ds;
    void *workspace;                  /* device memory, 256-byte aligned */
    size_t workspace_bytes;           /* at least r2l_backward_workspace_size() */
} r2l_grad_args;

/*
 * r2l_scan_backward -- the gradients of r2l_scan at `fwd` for dL/dout (and
 * dL/dh_out): the adjoint of the reverse scan, visiting the tokens of each
 * sequence left to right. Every sum (over channels for dBm and dCm, over
 * tokens and sequences for dA, dDskip and ds) is taken in a fixed order, so
 * repeated calls give the same bits. All arithmetic is fp32.
 * Source: "Bifocal Diffusion Language Models", section 2 (the R2L stream,
 * its residual through s, and its training).
 */
R2L_API r2l_status r2l_scan_backward(const r2l_scan_args *fwd, const r2l_grad_args *grad,
                                     void *stream);

/*
 * prefix_scan_backward -- the same for the forward-direction scan with readout
 * (prefix_scan_state with Cm and out: the left-to-right stream of the L2R
 * ablation), visiting the tokens of each sequence right to left. dh_out is the
 * gradient of its final state. Same arguments, layouts and guarantees.
 * Source: "Bifocal Diffusion Language Models", section 4 (the L2R-Mamba
 * ablation trains the same sidecar scanning left to right).
 */
R2L_API r2l_status prefix_scan_backward(const r2l_scan_args *fwd, const r2l_grad_args *grad,
                                        void *stream);

/* Bytes of workspace r2l_scan_backward or prefix_scan_backward needs for these
 * arguments (only shape fields and which outputs are wanted are read). */
R2L_API r2l_status r2l_backward_workspace_size(const r2l_scan_args *fwd,
                                               const r2l_grad_args *grad, size_t *bytes);

/*
 * Saving the forward states for the backward (training the R2L stream: the
 * forward runs anyway, so the backward need not scan the states again).
 *
 * r2l_scan_save -- r2l_scan with the same arguments and results, which also
 * stores the state entering every 8th visited position of each sequence (its
 * "checkpoints") at ckpt: fp32, rows = (tokens / 8 + batch + 1) of
 * dim * dstate floats, the row of visited position p (a multiple of 8) of
 * sequence b being r = (packed start of b + p) / 8 + b; a row holds dstate/4
 * planes of [dim][4]: state n of channel d at ((r * dstate/4 + n/4) * dim + d)
 * * 4 + n % 4 (so that stores and loads by consecutive channels are
 * contiguous); ckpt_bytes of at
 * least r2l_checkpoint_size(). ckpt is an output (16-byte aligned, overlapping
 * no other buffer of the call); state_split must be 0 or 1. The workspace
 * is sized by r2l_workspace_size with R2L_OP_SAVE (the plan may chunk
 * differently from r2l_scan's). The states are
 * those of the readout (with s == 0 and a residual, where r2l_scan runs no
 * readout, one more state-only scan stores them). A chunked plan may cut
 * sequences at other points than r2l_scan's (whole groups of 8 tokens);
 * results differ from r2l_scan's by rounding only, and are bit-identical to
 * them when the plan does not chunk.
 * Source: "Bifocal Diffusion Language Models", section 2 (the R2L stream is
 * trained with the backbone or alone).
 */
R2L_API r2l_status r2l_scan_save(const r2l_scan_args *a, float *ckpt, size_t ckpt_bytes,
                                 void *stream);

/* Bytes of the checkpoints of a call with these arguments (0 with no token). */
R2L_API r2l_status r2l_checkpoint_size(const r2l_scan_args *a, size_t *bytes);

/*
 * r2l_scan_backward_saved -- r2l_scan_backward whose states come from the
 * checkpoints that r2l_scan_save stored for the same forward arguments
 * (ckpt: input, ckpt_bytes >= r2l_checkpoint_size()). It runs no forward state
 * pass; its workspace needs no checkpoint area (r2l_backward_workspace_size
 * still suffices). Same gradients, layouts and guarantees as
 * r2l_scan_backward (bit-identical to it when neither plan chunks).
 */
R2L_API r2l_status r2l_scan_backward_saved(const r2l_scan_args *fwd, const r2l_grad_args *grad,
                                           const float *ckpt, size_t ckpt_bytes, void *stream);

/*
 * prefix_scan_save / prefix_scan_backward_saved -- the same pair for the
 * left-to-right stream (prefix_scan_state with a readout, and
 * prefix_scan_backward): visited positions count from each sequence's first
 * token; the rows, sizes (r2l_checkpoint_size), checks and guarantees are those
 * above; the workspace of the saving call is sized with R2L_OP_PREFIX_SAVE.
 * Source: "Bifocal Diffusion Language Models", section 4 (the ablation that
 * trains a left-to-right stream in place of the right-to-left one).
 */
R2L_API r2l_status prefix_scan_save(const r2l_scan_args *a, float *ckpt, size_t ckpt_bytes,
                                    void *stream);
R2L_API r2l_status prefix_scan_backward_saved(const r2l_scan_args *fwd, const r2l_grad_args *grad,
                                              const float *ckpt, size_t ckpt_bytes, void *stream);

/*
 * bidir_scan -- the bidirectional full-window scan: over each whole sequence,
 * the forward scan of x (left to right from h_in, the parameters of `a`) plus
 * the reverse scan of the same x (right to left from zero, the parameters of
 * `rev`), their readouts added:
 *     y_t   = y_t(forward) + y_t(reverse)
 *     out   = res == NULL ? y : (s == 0 ? res : res + s * y)
 * h_out (optional) receives the forward direction's final state. Each
 * direction's readout includes its own Dskip * x term.
 * Source: "Training Hybrid Block Diffusion Language Models with Partial
 * Bidirectionality", nl summary, problem statement (the earlier hybrids,
 * DiffuMamba among them, run bidirectional Mamba scans over the whole
 * denoising window, which is what prevents exact caching); "Bifocal Diffusion
 * Language Models", section 4 (the streams of either direction in the
 * ablations). How the two directions combine is not on the pages: adding the
 * two readouts, each direction with its own parameters, is the reading taken.
 *
 * rev: the reverse direction's dt, Bm, Cm (same layout rules and dtype as in
 * `a`), A and Dskip. rev == NULL, or a NULL pointer in it, shares the forward
 * direction's tensor (with the forward's strides); a reverse direction without
 * a skip term needs an explicit zero Dskip. Everything else (shape, x, res, s,
 * out, h_in, h_out, delta_softplus, chunk_tokens) comes from `a`; state_split
 * must be 0 or 1 (one lane per channel).
 * Required: x, dt, Bm, Cm, A, out. The workspace (r2l_workspace_size with
 * R2L_OP_BIDIR) holds the reverse readout as fp32 [tokens, D] rows plus the
 * chunked plans' carry data; it is needed whenever the readout runs. With
 * s == 0 (and res) no readout runs, as in the other entry points: out is res
 * bit for bit and only the forward state is scanned when h_out is given.
 * out may be exactly x and/or res; any other overlap with an input of either
 * direction is R2L_ERR_ALIAS.
 */
typedef struct r2l_dir_args {
    const void *dt;  int64_t dt_stride; int64_t dt_batch_stride;
    const void *Bm;  int64_t Bm_stride; int64_t Bm_batch_stride;
    const void *Cm;  int64_t Cm_stride; int64_t Cm_batch_stride;
    const float *A;
    const float *Dskip;
} r2l_dir_args;

R2L_API r2l_status bidir_scan(const r2l_scan_args *a, const r2l_dir_args *rev, void *stream);

/*
 * r2l_sidecar_forward -- the sidecar block around the R2L scan, as a hook:
 * out = hidden + s * sidecar(hidden). The pages name a Mamba SSM sidecar run
 * over the reversed sequence ("Bifocal Diffusion Language Models", section 2)
 * and give none of its internals; this is the plain Mamba block, whose
 * left-to-right form run on the reversed sequence reads, in the original
 * order (per sequence; weights stored [out, in] as in a linear layer):
 *     [x | z] = hidden W_in^T                        (d_model -> 2 d_inner)
 *     u_t     = SiLU(conv_b + sum_{j<K} conv_w[:, K-1-j] * x_{t+j})
 *               (the causal depthwise conv of the reversed sequence; zero
 *               past each sequence's last token)
 *     [r | B | C] = u W_x^T                          (d_inner -> dt_rank + 2 N)
 *     y       = the R2L scan of u with dt = r W_dt^T + dt_bias (softplus
 *               applied), B, C, A, Dskip, from a zero state
 *     out     = hidden + s * (y * SiLU(z)) W_out^T
 * With s == 0, out is hidden bit for bit and nothing else runs.
 *
 * Storage: hidden, out and W_in, W_x, W_dt, W_out in `dtype`; conv_w [d_inner,
 * d_conv], conv_b [d_inner], dt_bias [d_inner], A [d_inner, dstate] and
 * Dskip [d_inner] fp32 (conv_b, dt_bias, Dskip may be NULL: zero). Every
 * intermediate (x|z, u, r|B|C, r W_dt^T, the gated y) is stored in `dtype` in
 * the workspace, as a model in that dtype stores its activations; the GEMMs
 * and the scan accumulate in fp32. Tokens are packed rows of hidden and out
 * (row stride in elements, >= d_model): dense sequence b owns rows
 * b*seqlen .. (b+1)*seqlen-1, ragged ones follow cu_seqlens. Weights are
 * contiguous. out may be exactly hidden; any other overlap is R2L_ERR_ALIAS.
 * d_conv is 1..4, dstate 16; d_model, d_inner and dt_rank are multiples of 8
 * and the rows of hidden and out start on 16-byte boundaries (the GEMMs'
 * operands). The four projections run as hipBLASLt GEMMs through `gemm`, a
 * context the caller creates (r2l_gemm_context_create) on the device of the
 * call and keeps for as long as it calls: it holds the hipBLASLt handle and
 * the algorithm chosen for each GEMM shape (the library's first choice, or
 * what r2l_sidecar_tune found); the GEMMs' scratch is part of the workspace
 * (r2l_sidecar_workspace_size). Required unless s == 0.
 */
/* Opaque: one device's hipBLASLt handle and per-shape algorithm choices. */
typedef struct r2l_gemm_context_s *r2l_gemm_context;

/*
 * r2l_gemm_context_create -- a GEMM context for the current device, written to
 * *ctx (NULL on failure). It allocates host memory and the hipBLASLt handle's
 * resources; the caller owns it and releases it with r2l_gemm_context_destroy.
 * Calls on several host threads may share one context (its plan table is
 * locked); a context is only valid on the device it was created on.
 * Errors: R2L_ERR_INVALID_ARG (ctx NULL), R2L_ERR_HIP (no device, or the
 * library refused a handle).
 */
R2L_API r2l_status r2l_gemm_context_create(r2l_gemm_context *ctx);

/*
 * r2l_gemm_context_destroy -- releases a context made by
 * r2l_gemm_context_create (on its own device, whichever is current). No call
 * that uses it may still be queued. NULL, or a handle that is not a live
 * context the library can recognise, is R2L_ERR_INVALID_ARG; destroying a
 * context twice is undefined.
 */
R2L_API r2l_status r2l_gemm_context_destroy(r2l_gemm_context ctx);

typedef struct r2l_sidecar_args {
    int64_t batch;
    int64_t seqlen;             /* dense */
    const int32_t *cu_seqlens;  /* ragged, device [batch+1], or NULL */
    int64_t total_tokens;       /* ragged */
    int64_t max_seqlen;         /* ragged */
    int64_t d_model;
    int64_t d_inner;
    int32_t dstate;
    int32_t dt_rank;
    int32_t d_conv;
    int32_t dtype;              /* R2L_DTYPE_* */
    const void *hidden; int64_t hidden_stride;
    const void *W_in;           /* [2 d_inner, d_model] */
    const float *conv_w;        /* [d_inner, d_conv] */
    const float *conv_b;        /* [d_inner] or NULL */
    const void *W_x;            /* [dt_rank + 2 dstate, d_inner] */
    const void *W_dt;           /* [d_inner, dt_rank] */
    const float *dt_bias;       /* [d_inner] or NULL */
    const float *A;             /* [d_inner, dstate] */
    const float *Dskip;         /* [d_inner] or NULL */
    const void *W_out;          /* [d_model, d_inner] */
    float s;
    void *out; int64_t out_stride;
    void *workspace;            /* device, 256-byte aligned */
    size_t workspace_bytes;
    r2l_gemm_context gemm;      /* the caller's GEMM context (required unless s == 0) */
} r2l_sidecar_args;

R2L_API r2l_status r2l_sidecar_forward(const r2l_sidecar_args *a, void *stream);

/*
 * r2l_sidecar_tune -- for the four projections of a call with these
 * arguments, times hipBLASLt's candidate algorithms on `stream` and keeps the
 * fastest (the library's first choice unless another is at least 5% faster)
 * in the call's GEMM context, for every later r2l_sidecar_forward with the
 * same shapes and that context. Call it once before serving or graph capture: it
 * synchronizes the stream, and it overwrites the workspace (never hidden or
 * out, except that when the out-projection's rows do not fit the workspace's
 * in-projection rows it is timed in out itself, or, when out is hidden, not
 * tuned). The same checks as r2l_sidecar_forward; s == 0 does nothing.
 */
R2L_API r2l_status r2l_sidecar_tune(const r2l_sidecar_args *a, void *stream);

/* Bytes of workspace r2l_sidecar_forward needs for these arguments (shape
 * fields and s only). */
R2L_API r2l_status r2l_sidecar_workspace_size(const r2l_sidecar_args *a, size_t *bytes);

/* Short static description of a status code. */
R2L_API const char *r2l_status_string(r2l_status status);

/* Description of the last error returned on the calling host thread ("" if none). */
R2L_API const char *r2l_last_error(void);

/* R2L_ABI_VERSION of the library. */
R2L_API int32_t r2l_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* R2L_SCAN_H_ */
