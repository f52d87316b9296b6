/*
 * fa2.h -- C ABI of libfa2.so: exact attention forward (FlashAttention-2
 * schedule) and flash-decoding on AMD Instinct MI355X (gfx950).
 *
 * Callers need no HIP header: device pointers are plain `void*`, the stream
 * is an opaque `void*` holding a hipStream_t (NULL = the default stream).
 *
 * Conventions for every entry point
 *   Ownership  The caller allocates, owns and frees every buffer (device
 *              memory).  The library never allocates, frees or synchronises;
 *              its only global state is a once-filled, thread-safe cache of
 *              device properties.
 *   Launch     Work is enqueued on `stream` and the call returns at once.
 *              Results are valid after the stream is synchronised.  Calls on
 *              one stream run in order; apart from a pending timing request
 *              (fa2_time_next_launch, per host thread) the library keeps no
 *              state between calls, so calls on different streams may overlap
 *              when their output buffers do not (attn_fwd_noalloc aside).
 *   Layouts    Contiguous row-major, innermost dimension last.  Element type
 *              of q/k/v/o is `dtype`; lse and decode partials are float32.
 *   Alignment  Every pointer must be 16-byte aligned (128-bit loads/stores).
 *   Errors     Arguments are checked before anything is enqueued; a rejected
 *              call enqueues nothing.  A failed launch is reported as
 *              FA2_ERR_LAUNCH.  The library never aborts the process.
 *   Limits     One (b,h) slice of q, k or v must be smaller than 2 GiB, and
 *              B*H must be at most 65535 (attn_fwd, attn_fwd_ws, attn_bwd,
 *              attn_decode_split); attn_bwd also needs
 *              B*H*ceil(max(Nq,Nk) / W) < 2^24 with W = 128 (D = 64) or 64
 *              (D = 128).  Requests beyond these return FA2_ERR_UNSUPPORTED.
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA2_F32 = 0,  /* IEEE binary32 */
    FA2_F16 = 1,  /* IEEE binary16 */
    FA2_BF16 = 2  /* bfloat16 */
} fa2_dtype;

typedef enum {
    FA2_OK = 0,
    FA2_ERR_NULL = 1,        /* a required pointer is NULL */
    FA2_ERR_SHAPE = 2,       /* a size is negative or zero where it must be positive */
    FA2_ERR_UNSUPPORTED = 3, /* valid request this build does not implement (D, dtype,
                                causal with Nq != Nk, a non-finite scale, a slice of
                                2 GiB or more, B*H > 65535, the backward's grid limit) */
    FA2_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    FA2_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch */
    FA2_ERR_DEVICE = 6       /* no usable gfx950 device, or a device query failed */
} fa2_status;

/*
 * attn_fwd -- exact attention forward for [B,H,N,D] tensors.
 *
 * Computes, for every batch b, head h and query row i,
 *     s_ij   = scale * <q[b,h,i,:], k[b,h,j,:]>           for live keys j
 *     o[b,h,i,:] = sum_j exp(s_ij - m_i) v[b,h,j,:] / sum_j exp(s_ij - m_i)
 *     lse[b,h,i] = m_i + ln(sum_j exp(s_ij - m_i)),  m_i = max_j s_ij
 * ("Flash attention, f32": opening paragraph and section Online softmax;
 *  "Flash Attention" (aarnphm.xyz): sections Deriving the online softmax and
 *  FlashAttention 2 -- the log-sum-exp per row; "06: Fused attention":
 *  attn_fwd, causal masking and the per-row L).  Each workgroup walks K/V in
 *  blocks with a running max, running denominator and an unnormalised
 *  accumulator, so the Nq x Nk score matrix is never stored.
 *
 *   q    [B,H,Nq,D] dtype      k, v [B,H,Nk,D] dtype      o [B,H,Nq,D] dtype
 *   lse  [B,H,Nq] float32, natural log of the scaled scores; may be NULL.
 *   causal  0: every key is live.  1: key j is live for query i only when
 *           j <= i (top-left aligned); requires Nq == Nk.
 *   scale   multiplies q.k before the softmax (for example 1/sqrt(D)); any
 *           finite value (0 gives equal weights over the live keys, a
 *           negative scale favours the least similar keys); a NaN or
 *           infinite scale returns FA2_ERR_UNSUPPORTED.
 *   Arithmetic: float32 softmax state and accumulation.  f16/bf16 inputs run
 *   both products on MFMA with P rounded to the input dtype; float32 inputs
 *   run both products on float32 MFMA (no reduced-precision rounding).
 *   o is rounded to nearest-even into dtype.
 *   Supported: D == 64 or 128 with dtype F32, F16 or BF16; B, H >= 0 with
 *   B*H <= 65535; Nq >= 0 (zero-size outputs enqueue nothing); Nk >= 1;
 *   ragged Nq/Nk are masked in the tail.
 */
fa2_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int Nq, int Nk, int D, float scale, int causal,
                    fa2_dtype dtype, void *stream);

/*
 * attn_fwd_ws -- attn_fwd with a caller-provided device workspace.
 *
 * Same result and arguments as attn_fwd.  When there are too few query tiles
 * to fill the device (few heads, short sequences), a workspace of at least
 * attn_fwd_workspace_size() bytes lets the library split the keys of each
 * query tile into chunks, compute one unnormalised partial (O_s, m_s, l_s)
 * per row and chunk and merge them with the flash-decoding combine ("Flash
 * decoding": Overview of the algorithm -- the split is the same, applied to
 * many query rows; "Flash Attention": the (m, l) monoid).  With a NULL or
 * smaller workspace it runs exactly as attn_fwd.  The two paths may differ in
 * the last bits (the sums are grouped differently), each within the bounds
 * stated for attn_fwd.
 *   Where the keys of each tile are split in exactly two chunks (f16 and
 *   bf16, causal or not; and the float32 split of unmasked D = 64 shapes
 *   with few 32-row query tiles), there is no combine launch: the tile's two
 *   workgroups meet at the end with no wait.  Each publishes its partial
 *   state, then swaps a 64-bit value drawn for this call into the tile's
 *   handshake word in the workspace; the one that gets the value back merges
 *   the two states in chunk order (so the result does not depend on which
 *   one finished last), writes o and lse, and resets the word.
 *   workspace  device memory, 16-byte aligned, owned by the caller.  Its
 *              contents on entry do not matter: the handshake words are read
 *              before they are written, but only a word that already holds
 *              this call's value (odd; a counter with a random start,
 *              scrambled by the SplitMix64 finaliser) would count, and every
 *              call leaves them 0.  On return the rest is unspecified.
 *              Calls that share one workspace must not overlap in time.
 */
fa2_status attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int H, int Nq, int Nk, int D, float scale, int causal,
                       fa2_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_fwd_noalloc -- attn_fwd_ws for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Nothing is allocated or freed by the call.
 *
 * Same arguments and result as attn_fwd (the caller passes the inputs and
 * the outputs o and lse); the workspace that attn_fwd_ws would take from the
 * caller is the library's own device array of FA2_NOALLOC_SCRATCH_BYTES
 * bytes, one per device, which every device the library is loaded on holds
 * until the process ends.
 *   Errors   A shape whose workspace (attn_fwd_workspace_size) exceeds
 *            FA2_NOALLOC_SCRATCH_BYTES returns FA2_ERR_UNSUPPORTED (on a
 *            256-CU MI355X: head-dimension-128 shapes whose key split fills
 *            every workgroup slot, and unmasked float32 head-dimension-64
 *            shapes of 1986 or more 32-row query tiles that would split their
 *            keys in two); use attn_fwd_ws for those.  FA2_ERR_DEVICE if the
 *            array's device address cannot be obtained.
 *   Races    All attn_fwd_noalloc calls on one device share its array, which
 *            keeps the last call's contents: calls that can overlap in time on
 *            one device (different streams, or different host threads) race.
 *            Serialise them, e.g. issue them on one stream.  The array's
 *            contents on entry do not change the result (see attn_fwd_ws:
 *            the only words read before they are written are handshake
 *            words, compared with a value drawn for each call).
 */
#define FA2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa2_status attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int H, int Nq, int Nk, int D, float scale, int causal,
                            fa2_dtype dtype, void *stream);

/*
 * attn_fwd_workspace_size -- bytes of workspace attn_fwd_ws would use for
 * this shape on the current device (0: it would not split, or the shape is
 * not supported).  If the device cannot be queried it assumes 256 compute
 * units.
 */
size_t attn_fwd_workspace_size(int B, int H, int Nq, int Nk, int D, int causal, fa2_dtype dtype);

/*
 * attn_bwd -- exact attention backward: gradients of attn_fwd's o with
 * respect to q, k and v, given the upstream gradient dout.
 *
 * With P_ij = exp(s_ij - lse_i) the probabilities of the forward (s_ij as in
 * attn_fwd, 0 for keys that are not live) and
 *     delta[b,h,i] = sum_d dout[b,h,i,d] o[b,h,i,d]
 *     dS_ij = P_ij (dout_i . v_j - delta_i)
 *     dv_j = sum_i P_ij dout_i,  dq_i = scale sum_j dS_ij k_j,
 *     dk_j = scale sum_i dS_ij q_i
 * ("Flash Attention" (aarnphm.xyz): section IO complexity, the backward
 * pass -- only O and the log-sum-exp are kept, P is recomputed block by
 * block; "06: Fused attention": the backward kernels, the pre-pass for
 * delta, the dK/dV pass over query blocks and the dQ pass over key blocks).
 * No Nq x Nk matrix is stored.
 *
 *   q, o, dout  [B,H,Nq,D] dtype      k, v [B,H,Nk,D] dtype
 *   lse         [B,H,Nq] float32, natural log, as written by attn_fwd for
 *               the same q, k, scale and causal flag
 *   dq [B,H,Nq,D], dk, dv [B,H,Nk,D] dtype: outputs, rounded to nearest-even
 *   delta       [B,H,Nq] float32: output (the library fills it and then
 *               reads it; its contents on entry are ignored)
 *   causal, scale  as in attn_fwd (causal requires Nq == Nk)
 *   Arithmetic: the products per block run on MFMA with float32
 *   accumulation.  F16/BF16: P and dS are rounded to dtype before the two
 *   products that consume them (as P is in attn_fwd); delta, P and dS are
 *   formed in float32.  F32: float32 MFMA operands, nothing is rounded to a
 *   narrower type.  With Nq == 0, dk and dv are set to zero.  The results do
 *   not depend on timing (no atomics): equal inputs give equal bits.
 *   Supported: D == 64 or 128 with F32, F16 or BF16; B, H >= 0 with
 *   B*H <= 65535, Nq >= 0 (B*H == 0 enqueues nothing); Nk >= 1;
 *   B*H*ceil(max(Nq,Nk) / W) < 2^24 with W = 128 (D = 64) or 64 (D = 128).
 */
fa2_status attn_bwd(const void *q, const void *k, const void *v, const void *o,
                    const void *dout, const float *lse, void *dq, void *dk, void *dv,
                    float *delta, int B, int H, int Nq, int Nk, int D, float scale,
                    int causal, fa2_dtype dtype, void *stream);

/*
 * attn_decode_split -- flash-decoding, phase 1: unnormalised partials.
 *
 * One query row per (b,h) attends all N keys of its slice, with the keys cut
 * into n_splits contiguous splits ("Flash decoding": Overview of the
 * algorithm, and its split kernel).  Split s covers keys
 * [s*S, min((s+1)*S, N)) with S = ceil(N / n_splits), and stores
 *     m_part[b,h,s] = max_j s_j                 (s_j = scale * <q[b,h,:], k[b,h,j,:]>)
 *     l_part[b,h,s] = sum_j exp(s_j - m_part)
 *     o_part[b,h,s,:] = sum_j exp(s_j - m_part) v[b,h,j,:]   (not divided by l)
 * in natural-log units of the scaled scores.  A split with no keys (when
 * n_splits > N) stores m = -inf, l = 0, o = 0.
 *
 *   q [B,H,D] dtype;  k, v [B,H,N,D] dtype
 *   o_part [B,H,n_splits,D] float32;  m_part, l_part [B,H,n_splits] float32
 *   Supported: D in {64, 128}; dtype F16, BF16, F32; N >= 1; n_splits >= 1;
 *   B*H <= 65535; any finite scale (otherwise FA2_ERR_UNSUPPORTED); B*H == 0
 *   enqueues nothing.
 */
fa2_status attn_decode_split(const void *q, const void *k, const void *v,
                             float *o_part, float *m_part, float *l_part,
                             int B, int H, int N, int D, float scale, int n_splits,
                             fa2_dtype dtype, void *stream);

/*
 * attn_decode_combine -- flash-decoding, phase 2: merge the partials.
 *
 *     m_g = max_s m_s,   l_g = sum_s exp(m_s - m_g) l_s,
 *     o[b,h,:] = sum_s exp(m_s - m_g) o_s / l_g
 * ("Flash decoding": Overview of the algorithm, combine equations, and its
 * combine kernel -- one workgroup per (batch, head)).  Splits with
 * m_s = -inf carry no keys and get weight 0.
 *
 *   o_part [B,H,n_splits,D], m_part, l_part [B,H,n_splits] float32 (as written
 *   by attn_decode_split);  o [B,H,D] dtype, rounded to nearest-even.
 *   Alignment: o_part and o 16 bytes (the general rule); m_part and l_part
 *   only need 4.
 *   Supported: D in {64, 128}; dtype F16, BF16, F32; n_splits >= 1.
 */
fa2_status attn_decode_combine(const float *o_part, const float *m_part, const float *l_part,
                               void *o, int B, int H, int D, int n_splits,
                               fa2_dtype dtype, void *stream);

/*
 * attn_decode_default_splits -- split count for attn_decode_split that fills
 * the current device ("Flash decoding": many blocks each reading a chunk of
 * the cache is what lets the read use the memory bandwidth).  Picks the
 * count so that B*H*n_splits workgroups cover the device's compute units in
 * whole waves of residency, with at least 256 keys per split.  Returns a value
 * >= 1; if the device cannot be queried it assumes 256 compute units.
 */
int attn_decode_default_splits(int B, int H, int N, int D);

/*
 * fa2_time_next_launch -- measurement aid: the next kernel that the calling
 * host thread enqueues through this library (through any entry point)
 * records `start_event` when it starts and `stop_event` when it ends, from
 * the kernel's own dispatch (hipExtLaunchKernel), so that their elapsed time
 * is that kernel's execution alone, without the queue's gap before it or the
 * marker packets of separately recorded events.  Both are hipEvent_t handles
 * created with timing enabled, or NULL (NULL, NULL cancels a pending
 * request).  The request is used by exactly one launch: an entry point that
 * enqueues several kernels (a key-split forward and its combine, the
 * backward's three passes) times the first.  Never fails (FA2_OK).
 */
fa2_status fa2_time_next_launch(void *start_event, void *stop_event);

/* Human-readable name of a status code (static storage, never NULL). */
const char *fa2_status_string(fa2_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
