/*
 * m2ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 mixer hot path.
 *
 * The compute entry points are the steps that the Zamba2 article ("Transformers 中 Zamba2
 * 混合架构模型解析", §三 "Mamba2 Mixer") places between the mixer's input projection and
 * its output projection:
 *
 *   m2_conv1d_fwd    causal depthwise conv1d of width mamba_d_conv, then SiLU,
 *                    over a prompt (groups = conv_dim; §五: use_conv_bias)
 *   m2_ssd_scan_fwd  the selective state-space scan over a prompt, computed in
 *                    chunks (§三: intra-chunk + inter-chunk scan, chunk_size)
 *   m2_ssd_step      the single-token recurrent update used when a cached state
 *                    exists and the new sequence length is 1 (§三); it also
 *                    advances the cached conv state (§三: the cache holds each
 *                    layer's conv state and recurrent state)
 *   m2_mixer_prefill_fwd  the conv and the scan of a prompt in one pass, without
 *                    writing the conv output (§五: use_mem_eff_path)
 *   m2_gated_rmsnorm the gated group RMSNorm applied to the scan's output (§三)
 *   m2_ssd_scan_bwd  the backward of the scan: the gradients a training step of the stateful
 *                    mixer needs (§三)
 *
 * A batch of prompts of different lengths (the recurrent mask of §2.3) is given either
 * right-padded (seq_lens on m2_conv1d_fwd / m2_ssd_scan_fwd / m2_mixer_prefill_fwd /
 * m2_ssd_scan_bwd) or packed back to back (m2_conv1d_fwd_packed / m2_ssd_scan_fwd_packed /
 * m2_mixer_prefill_fwd_packed / m2_ssd_scan_bwd_packed with cu_seqlens offsets).
 *
 * The recurrence, per batch element b and head h, for t = 0..L-1:
 *     dt_t = softplus(dt_raw_t + dt_bias[h])        (then clamped to [dt_min, dt_max])
 *     S_t  = exp(dt_t * A[h]) * S_{t-1} + dt_t * x_t (outer) B_t     S is headdim x d_state, fp32
 *     y_t  = S_t . C_t + D[h] * x_t
 * with S_{-1} = state_in (zero if NULL); head h reads group g(h) = h / (nheads / n_groups).
 *
 * Conventions
 *   - Every pointer argument except `stream` is DEVICE memory owned by the caller.
 *     The library allocates nothing and never synchronises: each call only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the default stream) and returns.
 *     It keeps no state between calls beyond a cached record of each device's compute
 *     units and XCDs and one static scratch array per device (m2_ssd_scan_fwd_noalloc).
 *     Calls are thread-safe, except that calls of m2_ssd_scan_fwd_noalloc that may
 *     overlap on one GPU share its scratch array.
 *   - Activations (xBC, x, B, C, dt, y, conv ring) are stored in dims.io (bf16 or
 *     fp32); fp32 accumulation everywhere.  Parameters (conv w/bias, dt_bias, A, D)
 *     and the SSM state are always fp32.
 *   - Strides are in ELEMENTS.  A "token stride" is the distance between tokens t
 *     and t+1 of one sequence; the batch stride is seqlen * token stride.
 *   - Errors: arguments are validated on the host before anything is enqueued; a
 *     nonzero m2_status means nothing was launched, except M2_ERR_LAUNCH (the
 *     runtime refused a launch).  NaN/Inf in the data are propagated, not reported.
 *     Not checked: A <= 0 and finiteness of the inputs.
 *   - Device pointers must be 16-byte aligned and strides multiples of 16 bytes /
 *     element size where noted; otherwise M2_ERR_UNSUPPORTED.
 */
#ifndef M2SSD_H
#define M2SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define M2SSD_ABI_VERSION 8

typedef enum {
    M2_OK = 0,
    M2_ERR_NULL = 1,         /* a required pointer is NULL */
    M2_ERR_SHAPE = 2,        /* non-positive or inconsistent sizes, stride below row width */
    M2_ERR_DTYPE = 3,        /* dims.io is not a supported storage type */
    M2_ERR_ALIAS = 4,        /* an output overlaps an input it must not overlap */
    M2_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the size its query reports */
    M2_ERR_UNSUPPORTED = 6,  /* valid but not built: headdim/d_state/alignment outside the kernels' set */
    M2_ERR_LAUNCH = 7,       /* the HIP runtime reported an error at launch */
    M2_ERR_TOO_LARGE = 8     /* the call needs more scratch than the library's static buffer holds */
} m2_status;

/* Bytes of the static device scratch buffer behind m2_ssd_scan_fwd_noalloc (one per GPU). */
#define M2_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum { M2_F32 = 0, M2_BF16 = 1 } m2_dtype;

/* Mixer dimensions (the Zamba2 configuration names of article §五 in brackets).
 * Derived: d_inner = expand * d_model, nheads = d_inner / headdim,
 *          conv_dim = d_inner + 2 * n_groups * d_state.                        */
typedef struct {
    int64_t batch;       /* sequences */
    int64_t seqlen;      /* tokens per sequence (ignored by m2_ssd_step) */
    int32_t d_model;     /* [hidden_size] */
    int32_t expand;      /* [mamba_expand] */
    int32_t headdim;     /* [mamba_headdim]  P */
    int32_t d_state;     /* [mamba_d_state]  N */
    int32_t n_groups;    /* [mamba_ngroups]  G, must divide nheads */
    int32_t d_conv;      /* [mamba_d_conv]   W, 2..4 */
    int32_t chunk_size;  /* [chunk_size]     a hint: 16, 32 or 64 are used where built (64 not
                          * for fp32); any other value, 0 included, means the library's choice */
    int32_t io;          /* m2_dtype of the activations */
} m2_dims;

/* Causal depthwise conv1d + SiLU over a prompt.
 *   out[b,t,c] = SiLU(bias[c] + sum_{k<W} w[c,k] * x[b, t-(W-1)+k, c]),  SiLU(v) = v / (1 + e^-v)
 * xbc      [batch, seqlen, conv_dim] io, token stride xbc_tok_stride (>= conv_dim);
 *          channel order x (d_inner) | B (n_groups*d_state) | C (n_groups*d_state)
 * w        [conv_dim, W] fp32;  bias [conv_dim] fp32 or NULL (no bias)
 * ring_in  [batch, W, conv_dim] io or NULL (zero history): the conv state of the tokens
 *          before t = 0, as a ring at phase ring_in_step: the token j places before
 *          t = 0 (j = 1..W-1) is in slot (ring_in_step - j) mod W
 * ring_out [batch, W, conv_dim] io or NULL: receives the last W tokens as a ring at
 *          phase 0 (slot j = token seqlen-W+j, taken from ring_in when negative);
 *          must not overlap ring_in or xbc
 * out      [batch, seqlen, conv_dim] io, token stride out_tok_stride; must not overlap xbc
 * seq_lens [batch] int32 on the device, or NULL (every sequence is seqlen tokens long): a
 *          right-padded batch, in which sequence b holds only its first seq_lens[b] tokens
 *          (the recurrent mask of the Zamba2 page, §2.3, for padding at the end).  Values
 *          are clamped to [0, seqlen].  out at later positions is left as it was, and
 *          ring_out holds the W tokens before seq_lens[b].  Must not overlap an output.
 * seqlen may be 0 (then only ring_out is written, as a copy of the history). */
m2_status m2_conv1d_fwd(const m2_dims* dims,
                        const void* xbc, int64_t xbc_tok_stride,
                        const float* w, const float* bias,
                        const void* ring_in, int64_t ring_in_step,
                        void* ring_out,
                        void* out, int64_t out_tok_stride,
                        const int32_t* seq_lens,
                        void* stream);

/* Packed batch (sequences back to back, no padding): the same as m2_conv1d_fwd for dims.batch
 * sequences that lie one after another in one token-major array of total_tokens rows.
 * cu_seqlens [batch+1] int32 on the device: sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1
 *          (cu_seqlens[0] = 0, non-decreasing, cu_seqlens[batch] = total_tokens).  On the device
 *          the offsets are clamped to [0, total_tokens] and a sequence is cut at dims.seqlen tokens,
 *          so dims.seqlen is the longest sequence (rows past the cut are left as they were).
 *          Must not overlap an output.
 * xbc, out [total_tokens, conv_dim] io with token strides as in m2_conv1d_fwd;
 * ring_in, ring_out [batch, W, conv_dim] io or NULL, one ring per sequence, as in m2_conv1d_fwd. */
m2_status m2_conv1d_fwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                               const void* xbc, int64_t xbc_tok_stride,
                               const float* w, const float* bias,
                               const void* ring_in, int64_t ring_in_step,
                               void* ring_out,
                               void* out, int64_t out_tok_stride,
                               void* stream);

/* Workspace bytes m2_ssd_scan_fwd needs for these dims (0 if none). */
size_t m2_ssd_scan_workspace(const m2_dims* dims);

/* Chunked selective state-space scan over a prompt (the recurrence above for t = 0..seqlen-1).
 * x        [batch, seqlen, nheads, headdim] io, token stride x_tok_stride (>= d_inner)
 * B, C     [batch, seqlen, n_groups, d_state] io, token stride bc_tok_stride (>= n_groups*d_state)
 * dt       [batch, seqlen, nheads] io (raw, before bias and softplus), token stride dt_tok_stride
 * dt_bias, A [nheads] fp32;  D [nheads] fp32 or NULL (no skip term)
 * dt_min, dt_max  clamp of dt after softplus; pass 0 and +INFINITY for none
 * state_in  [batch, nheads, headdim, d_state] fp32 or NULL (zero initial state)
 * state_out [batch, nheads, headdim, d_state] fp32 or NULL; must not overlap state_in
 * y        [batch, seqlen, nheads*headdim] io, token stride y_tok_stride; must not overlap
 *          x, B, C or dt
 * workspace device scratch of at least m2_ssd_scan_workspace(dims) bytes (NULL if 0), any
 *          alignment; its contents on entry do not matter.  Calls that may run at the same
 *          time (other streams) need separate workspaces.
 * seq_lens [batch] int32 on the device, or NULL (every sequence is seqlen tokens long): a
 *          right-padded batch as in m2_conv1d_fwd.  Sequence b consumes only its first
 *          seq_lens[b] tokens (clamped to [0, seqlen]): y at later positions is left as it
 *          was, and state_out is the state after its last token (state_in, or zero, for an
 *          empty one).  Must not overlap an output or the workspace.
 * x/B/C may be strided views into one conv1d output (token stride conv_dim).
 * x, B, C and y must start on 16-byte boundaries and their token strides be multiples of 16
 * bytes (else M2_ERR_UNSUPPORTED); dt has no alignment requirement. */
m2_status m2_ssd_scan_fwd(const m2_dims* dims,
                          const void* x, int64_t x_tok_stride,
                          const void* B, const void* C, int64_t bc_tok_stride,
                          const void* dt, int64_t dt_tok_stride,
                          const float* dt_bias, const float* A, const float* D,
                          float dt_min, float dt_max,
                          const float* state_in, float* state_out,
                          void* y, int64_t y_tok_stride,
                          void* workspace, size_t workspace_bytes,
                          const int32_t* seq_lens,
                          void* stream);

/* Workspace bytes m2_ssd_scan_fwd_packed needs for dims (dims.seqlen the longest sequence) and
 * total_tokens rows (0 if none, or if the arguments are invalid).  The packed scan sizes its
 * segments from the total, so this can differ from m2_ssd_scan_workspace(dims): the segment length
 * is picked on the device from the lengths in cu_seqlens, and the workspace covers the shortest
 * one any lengths adding up to total_tokens could call for. */
size_t m2_ssd_scan_workspace_packed(const m2_dims* dims, int64_t total_tokens);

/* Packed batch: the same as m2_ssd_scan_fwd for dims.batch sequences back to back in arrays of
 * total_tokens rows (x [total_tokens, nheads, headdim], B/C [total_tokens, n_groups, d_state],
 * dt [total_tokens, nheads], y [total_tokens, nheads*headdim], with token strides and alignment as
 * in m2_ssd_scan_fwd).  cu_seqlens as in m2_conv1d_fwd_packed; dims.seqlen is the longest
 * sequence; workspace holds at least m2_ssd_scan_workspace_packed(dims, total_tokens) bytes.
 * Each sequence starts from its own state_in[b] (or zero) and returns state_out[b], the
 * state after its last token.  Sequences never see one another's tokens. */
m2_status m2_ssd_scan_fwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                                 const void* x, int64_t x_tok_stride,
                                 const void* B, const void* C, int64_t bc_tok_stride,
                                 const void* dt, int64_t dt_tok_stride,
                                 const float* dt_bias, const float* A, const float* D,
                                 float dt_min, float dt_max,
                                 const float* state_in, float* state_out,
                                 void* y, int64_t y_tok_stride,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Workspace bytes m2_mixer_prefill_fwd needs for these dims (0 when the fused path is not built for
 * them: then it returns M2_ERR_UNSUPPORTED). */
size_t m2_mixer_prefill_workspace(const m2_dims* dims);

/* The prompt path in one pass: conv1d + SiLU of the raw conv input, then the scan, with the conv
 * output never written to memory (article §五: use_mem_eff_path, the fused conv1d + scan path).
 * Results are those of m2_conv1d_fwd followed by m2_ssd_scan_fwd on its x | B | C split, except that
 * the x channels enter the state update at fp32 instead of rounded to the storage type:
 *   y, state_out  as m2_ssd_scan_fwd;  ring_out as m2_conv1d_fwd (the last W raw tokens).
 * xbc      [batch, seqlen, conv_dim] raw conv input (x | B | C), token stride xbc_tok_stride
 * conv_w, conv_b, ring_in, ring_in_step, ring_out   as in m2_conv1d_fwd
 * dt, dt_bias, A, D, dt_min, dt_max, state_in, state_out, y, seq_lens   as in m2_ssd_scan_fwd
 * workspace device scratch of at least m2_mixer_prefill_workspace(dims) bytes, any alignment
 *          (it holds the conv output of the B and C channels and the scan's segment records)
 * Built for bf16 activations, headdim 64, d_state 64 (the Zamba2-2.7B mixer shape), nheads /
 * n_groups a multiple of 4, chunk_size taken as a hint (32 tokens are used).  Other shapes, and dt
 * views not on a 4-byte boundary or with an odd token stride, return M2_ERR_UNSUPPORTED: use the
 * two entry points.  xbc and y as the scan's x and y (16-byte aligned rows); outputs must not
 * overlap inputs, each other or the workspace. */
m2_status m2_mixer_prefill_fwd(const m2_dims* dims,
                               const void* xbc, int64_t xbc_tok_stride,
                               const float* conv_w, const float* conv_b,
                               const void* ring_in, int64_t ring_in_step,
                               void* ring_out,
                               const void* dt, int64_t dt_tok_stride,
                               const float* dt_bias, const float* A, const float* D,
                               float dt_min, float dt_max,
                               const float* state_in, float* state_out,
                               void* y, int64_t y_tok_stride,
                               void* workspace, size_t workspace_bytes,
                               const int32_t* seq_lens,
                               void* stream);

/* Workspace bytes m2_mixer_prefill_fwd_packed needs for dims (dims.seqlen the longest sequence) and
 * total_tokens rows (0 when the fused path is not built for these dims, or if the arguments are
 * invalid).  It sizes the scan's segments from the total, as m2_ssd_scan_workspace_packed does. */
size_t m2_mixer_prefill_workspace_packed(const m2_dims* dims, int64_t total_tokens);

/* Packed batch: the same as m2_mixer_prefill_fwd for dims.batch sequences back to back in arrays of
 * total_tokens rows (xbc [total_tokens, conv_dim], dt [total_tokens, nheads], y [total_tokens,
 * nheads*headdim], with token strides and alignment as in m2_mixer_prefill_fwd).  cu_seqlens as in
 * m2_conv1d_fwd_packed; dims.seqlen is the longest sequence; workspace holds at least
 * m2_mixer_prefill_workspace_packed(dims, total_tokens) bytes.  Each sequence starts from its own
 * conv history ring_in[b] and state_in[b] (or zeros) and returns ring_out[b] and state_out[b], as
 * m2_conv1d_fwd_packed and m2_ssd_scan_fwd_packed do.  Sequences never see one another's tokens. */
m2_status m2_mixer_prefill_fwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                                      const void* xbc, int64_t xbc_tok_stride,
                                      const float* conv_w, const float* conv_b,
                                      const void* ring_in, int64_t ring_in_step,
                                      void* ring_out,
                                      const void* dt, int64_t dt_tok_stride,
                                      const float* dt_bias, const float* A, const float* D,
                                      float dt_min, float dt_max,
                                      const float* state_in, float* state_out,
                                      void* y, int64_t y_tok_stride,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/* m2_ssd_scan_fwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The
 * workspace m2_ssd_scan_workspace(dims) reports comes from a static device array of
 * M2_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process ends;
 * its address is looked up once per device on the first call there.  Arguments, results and
 * errors are those of m2_ssd_scan_fwd, plus M2_ERR_TOO_LARGE (nothing launched) when the call
 * needs more than M2_STATIC_SCRATCH_BYTES (the Zamba2-2.7B mixer shape needs about 50 MB for one
 * 32768-token sequence).  No call allocates or frees memory.  Every call on one GPU uses the same
 * array: calls that may overlap on one GPU (other streams, other threads without ordering) race
 * and must not be made; calls ordered on one stream are safe. */
m2_status m2_ssd_scan_fwd_noalloc(const m2_dims* dims,
                                  const void* x, int64_t x_tok_stride,
                                  const void* B, const void* C, int64_t bc_tok_stride,
                                  const void* dt, int64_t dt_tok_stride,
                                  const float* dt_bias, const float* A, const float* D,
                                  float dt_min, float dt_max,
                                  const float* state_in, float* state_out,
                                  void* y, int64_t y_tok_stride,
                                  const int32_t* seq_lens,
                                  void* stream);

/* One decode token for every sequence, fused: conv window (W-1 cached tokens + the new
 * one) -> SiLU -> split x | B | C -> dt -> state update -> output.
 * xbc_tok  [batch, conv_dim] io, batch stride xbc_stride (>= conv_dim)
 * dt_tok   [batch, nheads] io (raw), batch stride dt_stride (>= nheads)
 * w, bias  conv parameters as in m2_conv1d_fwd;  dt_bias, A, D, dt_min, dt_max as in the scan
 * ring     [batch, W, conv_dim] io, IN PLACE: a ring at phase `step` (after a prefill that
 *          wrote ring_out, step counts the decode tokens since, from 0).  The new token
 *          is written into slot step mod W, the slot that just left the window.
 * state    [batch, nheads, headdim, d_state] fp32, IN PLACE
 * y        [batch, nheads*headdim] io; must not overlap the other arguments
 * step >= 0.  dims.seqlen is ignored. */
m2_status m2_ssd_step(const m2_dims* dims,
                      const void* xbc_tok, int64_t xbc_stride,
                      const void* dt_tok, int64_t dt_stride,
                      const float* w, const float* bias,
                      const float* dt_bias, const float* A, const float* D,
                      float dt_min, float dt_max,
                      void* ring, int64_t step,
                      float* state, void* y,
                      void* stream);

/* Gated group RMSNorm after the scan (article §三: group RMSNorm times SiLU of the gate z
 * over intermediate_size, in groups; §五: eps = rms_norm_eps, 1e-5 in Zamba2):
 *   norm_before_gate = 0:  g = y * SiLU(z),  out = g / sqrt(mean_group(g^2) + eps) * w
 *   norm_before_gate = 1:  out = y / sqrt(mean_group(y^2) + eps) * w * SiLU(z)
 * Each row holds d_inner channels, normalised in groups of group_size consecutive channels
 * (Zamba2's norm uses d_inner / n_groups).
 * ntok     rows: batch * seqlen after a prompt scan, batch after a decode step (0: no-op)
 * y, z     [ntok, d_inner] io, row strides y_tok_stride, z_tok_stride (>= d_inner)
 * w        [d_inner] fp32
 * out      [ntok, d_inner] io, row stride out_tok_stride; may be y itself (same stride), but
 *          must not otherwise overlap y, and must not overlap z
 * group_size must divide d_inner and be a multiple of 16 bytes / element size, at most
 * 8192 (bf16) or 4096 (fp32) channels; y, z, out, w and all strides 16-byte aligned
 * (else M2_ERR_UNSUPPORTED). */
m2_status m2_gated_rmsnorm(int64_t ntok, int32_t d_inner, int32_t group_size, int32_t io,
                           const void* y, int64_t y_tok_stride,
                           const void* z, int64_t z_tok_stride,
                           const float* w, float eps, int32_t norm_before_gate,
                           void* out, int64_t out_tok_stride,
                           void* stream);

/* A plain device-to-device copy of `bytes` (a multiple of 16; dst and src 16-byte aligned and not
 * overlapping): not part of the mixer, but the attainable read + write bandwidth of the device,
 * measured with a streaming kernel of this library, which the benchmark reports beside the HBM
 * peak as the reference for the kernels' bandwidth fractions. */
m2_status m2_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Workspace bytes m2_ssd_scan_bwd needs for these dims (0 when the backward is not built for them:
 * then it returns M2_ERR_UNSUPPORTED). */
size_t m2_ssd_scan_bwd_workspace(const m2_dims* dims);

/* Backward of m2_ssd_scan_fwd (article §三: the Mamba2 mixer's chunked scan on the training path of
 * the stateful model): the gradients of
 *     L = sum_{b,t} dy_t . y_t + <dstate_out, state_out>
 * with respect to every input of the scan, for y and state_out as m2_ssd_scan_fwd computes them
 * from the same arguments.  Built for bf16 activations at headdim 64 and d_state 64 (the
 * Zamba2-2.7B mixer shape), any batch, seqlen and n_groups dividing nheads; chunk_size is ignored
 * (chunks of 64 tokens).  Other dims return M2_ERR_UNSUPPORTED.  Right-padded batches take
 * seq_lens; packed batches take m2_ssd_scan_bwd_packed.
 * Inputs as m2_ssd_scan_fwd (x, B, C, raw dt, dt_bias, A, D or NULL, dt_min, dt_max, state_in or
 * NULL), plus
 *   dy         [batch, seqlen, nheads*headdim] io, token stride dy_tok_stride: dL/dy
 *   dstate_out [batch, nheads, headdim, d_state] fp32 or NULL (zero): dL/dstate_out
 * Outputs (written, not accumulated):
 *   dx         [batch, seqlen, nheads*headdim] io, token stride dx_tok_stride
 *   dB, dC     [batch, seqlen, n_groups*d_state] io, token stride dbc_tok_stride: summed over the
 *              heads of each group
 *   ddt        [batch, seqlen, nheads] io, token stride ddt_tok_stride: dL/d(raw dt), zero where the
 *              clamp holds dt at dt_min or dt_max
 *   ddt_bias, dA, dD  [nheads] fp32, summed over the batch and the tokens (dD also when D is NULL)
 *   dstate_in  [batch, nheads, headdim, d_state] fp32 or NULL: dL/dstate_in
 * workspace: at least m2_ssd_scan_bwd_workspace(dims) bytes, any alignment, contents on entry
 * irrelevant; calls that may run at the same time need separate workspaces.
 * seq_lens   [batch] int32 on the device, or NULL (every sequence is seqlen tokens): a right-padded
 *            batch as in m2_ssd_scan_fwd.  Sequence b consumes only its first seq_lens[b] tokens
 *            (clamped to [0, seqlen]), dstate_out is the adjoint of the state after the last of them,
 *            and dx, dB, dC and ddt at later positions are left as they were; padded tokens add
 *            nothing to ddt_bias, dA and dD.  4-byte aligned; must not overlap an output.
 * x, B, C, dy, dx, dB and dC must start on 16-byte boundaries with token strides that are multiples
 * of 16 bytes (else M2_ERR_UNSUPPORTED).  No output may overlap an input, another output or the
 * workspace (M2_ERR_ALIAS); overlap is judged on each array's byte range from its first to its last
 * element, so dB and dC interleaved in one buffer count as overlapping: pass separate arrays. */
m2_status m2_ssd_scan_bwd(const m2_dims* dims,
                          const void* x, int64_t x_tok_stride,
                          const void* B, const void* C, int64_t bc_tok_stride,
                          const void* dt, int64_t dt_tok_stride,
                          const float* dt_bias, const float* A, const float* D,
                          float dt_min, float dt_max,
                          const float* state_in,
                          const void* dy, int64_t dy_tok_stride,
                          const float* dstate_out,
                          void* dx, int64_t dx_tok_stride,
                          void* dB, void* dC, int64_t dbc_tok_stride,
                          void* ddt, int64_t ddt_tok_stride,
                          float* ddt_bias, float* dA, float* dD,
                          float* dstate_in,
                          void* workspace, size_t workspace_bytes,
                          const int32_t* seq_lens,
                          void* stream);

/* Packed batch: the same as m2_ssd_scan_bwd for dims.batch sequences back to back in arrays of
 * total_tokens rows (x, dy, dx [total_tokens, nheads*headdim]; B, C, dB, dC [total_tokens,
 * n_groups*d_state]; dt, ddt [total_tokens, nheads]; token strides and alignment as in
 * m2_ssd_scan_bwd), the backward of m2_ssd_scan_fwd_packed on the same arguments.  cu_seqlens as
 * in m2_conv1d_fwd_packed (each offset clamped to [0, total_tokens], a sequence's end to at least
 * its start and its length to dims.seqlen); dims.seqlen is the longest sequence; workspace holds
 * at least m2_ssd_scan_bwd_workspace(dims) bytes.  Sequence b starts from state_in[b] (or zero),
 * dstate_out[b] is the adjoint of its state after its last token and dstate_in[b] receives the
 * adjoint of state_in[b]; rows that no sequence covers are left as they were.  Sequences never
 * see one another's tokens. */
m2_status m2_ssd_scan_bwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                                 const void* x, int64_t x_tok_stride,
                                 const void* B, const void* C, int64_t bc_tok_stride,
                                 const void* dt, int64_t dt_tok_stride,
                                 const float* dt_bias, const float* A, const float* D,
                                 float dt_min, float dt_max,
                                 const float* state_in,
                                 const void* dy, int64_t dy_tok_stride,
                                 const float* dstate_out,
                                 void* dx, int64_t dx_tok_stride,
                                 void* dB, void* dC, int64_t dbc_tok_stride,
                                 void* ddt, int64_t ddt_tok_stride,
                                 float* ddt_bias, float* dA, float* dD,
                                 float* dstate_in,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Static text for a status code. */
const char* m2_status_str(m2_status status);

/* M2SSD_ABI_VERSION of the built library. */
int m2_abi_version(void);

/* Name of the HIP runtime error behind the calling thread's most recent M2_ERR_LAUNCH
 * ("hipSuccess" if none).  Static text. */
const char* m2_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* M2SSD_H */
