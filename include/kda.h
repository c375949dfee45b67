/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library: the
 * chunked prefill, the decode step and the prefill's backward pass.
 *
 * The operation (per batch row b and head h; one state per head):
 *
 *   S <- h0                                     d_k x d_v, fp32
 *   for each token t:
 *     S <- Diag(exp(g_t)) S                     decay every key channel first
 *     S <- S + beta_t k_t (v_t - S^T k_t)^T     recall with the incoming key,
 *                                               then write only the difference
 *     o_t = scale * S^T q_t                     read after the write
 *   hT <- S
 *
 * Sources: "Kimi K3 Architecture Explained: How the World's Largest Open
 * Source AI Model Works", section 3 "Kimi Delta Attention (KDA)" (the
 * decay -> erase -> write order and DeltaNet's difference write); the Kimi K3
 * paper digest on devpress.csdn.net, section 2.1 (1) (delta-rule recursion
 * with a per-channel forget gate on a fixed-size state; gate bounded below by
 * g_min = -5 with 16-token chunks so that in-chunk reciprocal factors stay in
 * bf16 range) and section 2.4 (1) (the FlashKDA kernel overlaps intra-chunk
 * parallel work with inter-chunk state propagation).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers on the calling thread's current
 *    HIP device, owned by the caller.  The library allocates no device
 *    memory at run time.  It holds two fixed device arrays per device, which
 *    come with the loaded library: 512 KB of progress reports that pace the
 *    prefill's work-groups (no result depends on them) and the 32 MiB
 *    workspace of kda_chunk_fwd_kcp_noalloc.  Besides these it keeps only
 *    cached device properties.  Calls are thread-safe, except that
 *    kda_chunk_fwd_kcp_noalloc calls overlapping on one device race.
 *  - Every call is asynchronous and ordered on `stream` (a hipStream_t passed
 *    as void*; NULL = the null stream).  The library never synchronises.
 *  - Layouts are dense, row-major, token-major:
 *        q, k, g  [B, T, H, Dk]      v, o  [B, T, H, Dv]      beta [B, T, H]
 *        states   [B, H, Dk, Dv]     (row index = key channel)
 *    q, k, v are stored in `in_dtype`; g, beta, states and o are fp32.
 *  - g is the log-decay, expected in [-5, 0] (the bounded gate above); values
 *    outside are not clamped, but g < -5 may underflow the in-chunk factors.
 *  - scale <= 0 selects Dk^-1/2.
 *  - Supported shapes: Dk == Dv in {16, 128}.  Indices are 64-bit, so T and
 *    B*T*H are limited by device memory only; a prefill with B*H above
 *    2^25 - 1 (B*n_seg*H for the segmented one) or a decode step with B*H
 *    above 2^31 - 1 exceeds one launch's grid and is KDA_ERR_UNSUPPORTED.
 *  - Argument errors are detected before anything is launched and return
 *    KDA_ERR_INVALID_ARGUMENT or KDA_ERR_UNSUPPORTED; kda_last_error() then
 *    describes the problem.  A failed launch returns KDA_ERR_LAUNCH.  No C++
 *    exception crosses this interface.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, overlap */
    KDA_ERR_UNSUPPORTED = 2,      /* valid request this build does not implement */
    KDA_ERR_LAUNCH = 3,           /* the HIP runtime rejected a launch */
    KDA_ERR_DEVICE = 4            /* no usable device / unsupported architecture */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* How the forget gate is given to kda_chunk_fwd_qknorm. */
typedef enum kda_gate {
    KDA_GATE_LOG_DECAY = 0,  /* g itself, fp32 (as kda_chunk_fwd) */
    KDA_GATE_LOGIT_F32 = 1,  /* fp32 logits x, g = g_min sigmoid(x) (as kda_chunk_fwd_gate) */
    KDA_GATE_LOGIT_BF16 = 2  /* bf16 logits x, likewise */
} kda_gate;

/*
 * kda_chunk_fwd -- chunked prefill over a whole sequence, with an optional
 * initial state (prefix reuse: the digest's section 2.4 (4) keeps sparse KDA
 * state checkpoints so that cached prefixes can be resumed).
 *
 *   q, k   [B, T, H, Dk]  in_dtype   queries and keys (any norm; callers
 *                                    usually L2-normalise them)
 *   v      [B, T, H, Dv]  in_dtype   values
 *   g      [B, T, H, Dk]  fp32       per-channel log-decay
 *   beta   [B, T, H]      fp32       write strength
 *   h0     [B, H, Dk, Dv] fp32       initial state, or NULL for zeros
 *   o      [B, T, H, Dv]  fp32       output, written (must not overlap any input)
 *   hT     [B, H, Dk, Dv] fp32       final state, written; NULL = not wanted.
 *                                    hT == h0 (exact alias) is allowed: the
 *                                    state is then updated in place.
 *
 * T need not be a multiple of the 16-token chunk; T == 0 copies h0 (or zeros)
 * to hT.  B, H, Dk, Dv must be positive; T >= 0.  All pointers 16-byte aligned.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *h0,
                         float *o, float *hT,
                         int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                         kda_dtype in_dtype, float scale, void *stream);

/*
 * kda_chunk_fwd_ckpt -- kda_chunk_fwd that also writes the state every
 * ckpt_every tokens: the sparse KDA state checkpoints of the Kimi K3 paper
 * digest (devpress.csdn.net), section 2.4 (4), from which a cached prefix can
 * be resumed.
 *
 *   ckpt        [n_ckpt, B, H, Dk, Dv] fp32, written, n_ckpt = T / ckpt_every
 *               rounded down.  Checkpoint i is the state after the first
 *               (i + 1) * ckpt_every tokens, laid out like h0, so any one of
 *               them can be passed back as h0 to continue from that token.
 *               It must not overlap any other argument.  NULL = no
 *               checkpoints (the call is then exactly kda_chunk_fwd).
 *   ckpt_every  tokens between checkpoints, a positive multiple of the
 *               16-token chunk; ignored when ckpt is NULL.
 *   o           as for kda_chunk_fwd, or NULL when ckpt is given: then only
 *               the checkpoints and hT are written, by a pass that skips the
 *               output's work (q, its scaled operand and the products that
 *               form o); the states are bit-identical to those of a call with
 *               o.  A NULL o without ckpt (and T > 0) is
 *               KDA_ERR_INVALID_ARGUMENT.
 *
 * All other arguments, the layouts and the errors are those of kda_chunk_fwd;
 * a ckpt_every that is not a positive multiple of 16 is
 * KDA_ERR_INVALID_ARGUMENT.
 */
kda_status kda_chunk_fwd_ckpt(const void *q, const void *k, const void *v,
                              const float *g, const float *beta, const float *h0,
                              float *o, float *hT, float *ckpt, int64_t ckpt_every,
                              int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                              kda_dtype in_dtype, float scale, void *stream);

/*
 * kda_chunk_fwd_gate -- kda_chunk_fwd with the forget gate given as its
 * logit, turned into the log-decay inside the kernel (the gate prologue fused
 * into the prefill):
 *
 *   g = g_min * sigmoid(x) = g_min / (1 + exp(-x))   per key channel,
 *
 * the bounded scaled-sigmoid gate with floor g_min of the Kimi K3 paper digest
 * (devpress.csdn.net), section 2.1 (1).  Saves the separate pass that would
 * write g, and with bf16 logits halves the gate's bytes.
 *
 *   x          [B, T, H, Dk] in gate_dtype (KDA_F32 or KDA_BF16): gate logits
 *   gate_dtype storage type of x
 *   g_min      floor of the gate, finite and -5 <= g_min < 0 (the bound the
 *              chunk form needs); anything else is KDA_ERR_INVALID_ARGUMENT
 *
 * All other arguments, the layouts and the errors are those of kda_chunk_fwd
 * (x takes the place and the alignment and overlap rules of g).
 */
kda_status kda_chunk_fwd_gate(const void *q, const void *k, const void *v,
                              const void *x, kda_dtype gate_dtype, float g_min,
                              const float *beta, const float *h0,
                              float *o, float *hT,
                              int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                              kda_dtype in_dtype, float scale, void *stream);

/*
 * kda_chunk_fwd_qknorm -- the prefill with the q/k normalisation fused in
 * front of it: every query and key vector (per batch row, token and head) is
 * used as
 *
 *   x / max(||x||_2, eps)
 *
 * formed in fp32 from the stored values inside the kernel, so the raw
 * projections go in unchanged and no normalised copy is written.  The pages
 * name no normalisation; the erase-then-write with the incoming key
 * ("Kimi K3 Architecture Explained", section 3) removes the recalled value
 * exactly only for a unit key, which is why delta-rule layers feed unit keys
 * (and queries).
 *
 *   g, gate    the gate as kda_chunk_fwd's g (KDA_GATE_LOG_DECAY; g_min is
 *              then ignored) or as kda_chunk_fwd_gate's logits x (the two
 *              KDA_GATE_LOGIT kinds, with g_min as there)
 *   eps        the floor, finite and 1e-18 <= eps <= 1e18, else
 *              KDA_ERR_INVALID_ARGUMENT (a zero vector stays zero)
 *
 * All other arguments, the layouts and the errors are those of kda_chunk_fwd
 * (g takes the place of kda_chunk_fwd's g or kda_chunk_fwd_gate's x).
 */
kda_status kda_chunk_fwd_qknorm(const void *q, const void *k, const void *v,
                                const void *g, kda_gate gate, float g_min, float eps,
                                const float *beta, const float *h0,
                                float *o, float *hT,
                                int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                kda_dtype in_dtype, float scale, void *stream);

/*
 * kda_chunk_fwd_kcp -- kda_chunk_fwd computed as n_seg segments in parallel:
 * the state-transition split of KDA context parallelism (KCP) in the Kimi K3
 * paper digest (devpress.csdn.net), section 2.4 (1), on one device.  Over a
 * segment p the recurrence is affine in its incoming state,
 *
 *   S_out = M_p S_in + B_p,
 *
 * with B_p the segment's final state from a zero state and M_p its final
 * state from the identity with zero values (the transition matrix, Dk x Dk).
 * All segments run side by side from a zero state and from the identity, a
 * scan over the P maps gives every segment's incoming state (and hT), and all
 * segments run again from those states to write o.  This fills the device
 * when B * H alone gives too few work-groups (one long sequence), at the cost
 * of about three passes over the inputs instead of one.
 *
 *   n_seg     number of segments, >= 1; T must be a multiple of n_seg, else
 *             KDA_ERR_INVALID_ARGUMENT.  n_seg == 1 (or T == 0) is exactly
 *             kda_chunk_fwd, and ws is then not used.  A segment length that
 *             is a multiple of 16 keeps the chunks of the single pass.
 *   ws        device workspace of at least kda_chunk_fwd_kcp_ws_bytes(...)
 *             bytes, 16-byte aligned, owned by the caller, overwritten, and
 *             not overlapping any other argument.  Needs Dk == Dv.
 *   ws_bytes  its size in bytes.
 *
 * All other arguments, the layouts and the errors are those of kda_chunk_fwd
 * (hT == h0 stays allowed).  The results equal kda_chunk_fwd's up to the
 * rounding of the different summation order.
 */
kda_status kda_chunk_fwd_kcp(const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *h0,
                             float *o, float *hT, int64_t n_seg,
                             void *ws, uint64_t ws_bytes,
                             int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                             kda_dtype in_dtype, float scale, void *stream);

/*
 * kda_chunk_fwd_kcp_ws_bytes -- bytes of workspace kda_chunk_fwd_kcp needs:
 * three fp32 state sets of [B * n_seg, H, Dk, Dv] (the transitions, the
 * zero-start states and the incoming states).  0 when n_seg <= 1 or the sizes
 * are invalid (non-positive, T not a multiple of n_seg, or 64-bit overflow).
 */
uint64_t kda_chunk_fwd_kcp_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t n_seg);

/*
 * kda_chunk_fwd_kcp_noalloc -- kda_chunk_fwd_kcp for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and results, with
 * the workspace taken from a fixed array the library keeps on each device
 * (kda_chunk_fwd_kcp_noalloc_max_bytes() bytes, 32 MiB, held until the process
 * ends) instead of a `ws` argument.  The call allocates nothing.
 *
 *   - A request whose workspace (kda_chunk_fwd_kcp_ws_bytes(...)) exceeds the
 *     array is KDA_ERR_UNSUPPORTED: 3 * B * n_seg * H * Dk * Dv * 4 bytes
 *     must fit, e.g. B * n_seg * H <= 170 at Dk = Dv = 128.
 *   - Every call on one device uses that device's one array, so calls that
 *     overlap in time on one device (other streams, other threads) race and
 *     give wrong results; calls ordered on one stream are safe.  Nothing in the
 *     array needs to start at zero: each call writes all it reads.
 *   - The array's address is looked up once per device, on the first call
 *     made while that device is current.
 *
 * All other arguments, the layouts and the errors are those of
 * kda_chunk_fwd_kcp.
 */
kda_status kda_chunk_fwd_kcp_noalloc(const void *q, const void *k, const void *v,
                                     const float *g, const float *beta, const float *h0,
                                     float *o, float *hT, int64_t n_seg,
                                     int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                     kda_dtype in_dtype, float scale, void *stream);

/* Size in bytes of kda_chunk_fwd_kcp_noalloc's fixed workspace array. */
uint64_t kda_chunk_fwd_kcp_noalloc_max_bytes(void);

/*
 * kda_chunk_bwd -- gradients of kda_chunk_fwd (training; the FlashKDA kernel
 * of the Kimi K3 paper digest, devpress.csdn.net, section 2.4 (1), serves
 * training as well as prefill).  For a loss L with dO = dL/do and
 * dhT = dL/dhT, it returns dL/d of every input: the reverse-mode adjoint of
 * the recurrence at the top of this file, run from the last token to the
 * first (with S'_t = Diag(exp g_t) S_{t-1}, r_t = S'_t^T k_t and
 * e_t = beta_t (v_t - r_t); dS is dL/dS_t):
 *
 *   dS += scale q_t do_t^T        dq_t = scale S_t do_t
 *   de  = dS^T k_t                dk_t = dS e_t + S'_t dr,   dr = -beta_t de
 *   dbeta_t = de . (v_t - r_t)    dv_t = beta_t de
 *   dg_t = rowsum((dS + k_t dr^T) .* S'_t)
 *   dS  = Diag(exp g_t) (dS + k_t dr^T)          dh0 = dS after token 0
 *
 *   q, k, v, g, beta, h0   as for kda_chunk_fwd (h0 NULL = zeros)
 *   dO     [B, T, H, Dv] fp32   upstream gradient of o
 *   dhT    [B, H, Dk, Dv] fp32  upstream gradient of the final state, or NULL (zero)
 *   dq, dk, dg [B, T, H, Dk] fp32, dv [B, T, H, Dv] fp32, dbeta [B, T, H] fp32: written
 *   dh0    [B, H, Dk, Dv] fp32, written, or NULL (not wanted)
 *   ws     device workspace of at least kda_chunk_bwd_ws_bytes(...) bytes,
 *          16-byte aligned, owned by the caller, overwritten.  It holds the
 *          forward state after every 16 tokens (written here by the prefill
 *          kernels) and per-slice partial sums.
 *
 * The outputs must not overlap each other, the inputs or ws.  Results are
 * deterministic (fixed summation order).  All other rules, the
 * layouts and the errors are those of kda_chunk_fwd; T == 0 writes dh0 = dhT
 * (or zeros).
 *
 * With bf16 inputs at Dk = 128 the gradient is computed in the 16-token chunk
 * form on the fp32 matrix cores (the same values up to rounding; dg, formed
 * from pieces that partly cancel, carries the largest error, about 1e-3 of
 * its rms); fp32 inputs, and Dk = 16, take the token-by-token form above.
 */
kda_status kda_chunk_bwd(const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *h0,
                         const float *dO, const float *dhT,
                         float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dh0,
                         void *ws, uint64_t ws_bytes,
                         int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                         kda_dtype in_dtype, float scale, void *stream);

/*
 * kda_chunk_bwd_ws_bytes -- bytes of workspace kda_chunk_bwd needs:
 * floor(T / 16) states of [B, H, Dk, Dv] fp32 plus, per column slice (4
 * slices at Dk = 128, 1 at Dk = 16), (3 Dk + 1) B T H fp32 partial sums
 * rounded up to a multiple of 4.
 * 0 for unsupported or invalid sizes (Dk != Dv, Dk not 16 or 128, or 64-bit
 * overflow).
 */
uint64_t kda_chunk_bwd_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv);

/*
 * kda_decode_step -- one new token per sequence (recurrent decoding, the case
 * behind the 4x decoding speed-up at 1M tokens quoted in "Kimi K3
 * Architecture Explained", section 3): the recurrence above with T = 1,
 * updating the state IN PLACE.
 *
 *   q, k   [B, H, Dk]  in_dtype     v [B, H, Dv] in_dtype
 *   g      [B, H, Dk]  fp32         beta [B, H] fp32
 *   state  [B, H, Dk, Dv] fp32      read, then overwritten with the new state
 *   o      [B, H, Dv]  fp32         written (must not overlap anything else)
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, float *o,
                           int64_t B, int64_t H, int64_t Dk, int64_t Dv,
                           kda_dtype in_dtype, float scale, void *stream);

/*
 * kda_decode_step_qknorm -- kda_decode_step with q and k normalised as in
 * kda_chunk_fwd_qknorm (x / max(||x||_2, eps), in fp32, inside the kernel).
 * eps: finite, 1e-18 <= eps <= 1e18, else KDA_ERR_INVALID_ARGUMENT.  All
 * other arguments, the layouts and the errors are those of kda_decode_step.
 */
kda_status kda_decode_step_qknorm(const void *q, const void *k, const void *v,
                                  const float *g, const float *beta,
                                  float *state, float *o,
                                  int64_t B, int64_t H, int64_t Dk, int64_t Dv,
                                  kda_dtype in_dtype, float scale, float eps, void *stream);

/* Human-readable name of a status code (static string). */
const char *kda_status_string(kda_status s);

/* Description of the last error returned on the calling thread ("" if none). */
const char *kda_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
