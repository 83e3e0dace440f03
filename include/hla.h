/*
 * hla.h -- C ABI of the MI355X (gfx950) library for masked second-order
 * Higher-order Linear Attention (HLA).
 *
 * Sources.  "Higher-order Linear Attention" (Zhang, Qin, Gu), as summarised
 * on three web pages:
 *   [SUM]  paperlayer.ai section-by-section summary;
 *   [EXP]  gist.science explainer, "Technische Zusammenfassung";
 *   [SKL]  skillmd.com skill page "Scale Attention to Long Contexts via
 *          Linear-Time Matrix Interactions" (its listings are NOT followed:
 *          they use a softmax feature map and a token-count normaliser that
 *          the other pages do not have).
 *
 * What the library computes, per head h with decay g = gamma[h] and ridge
 * lambda, for tokens t = 0..n-1 (all accumulation in fp32):
 *   S_t = g S_{t-1} + k_t k_t^T            key second moment, d x d
 *   C_t = g C_{t-1} + q_t v_t^T            query-value accumulator, d x dv
 *   m_t = g m_{t-1} + q_t                  query mass, d
 *   G_t = g^2 G_{t-1} + g k_t (k_t^T C_{t-1})   cross summary, d x dv
 *   h_t = g^2 h_{t-1} + g k_t (k_t . m_{t-1})   cross summary, d
 *   num_t = q_t^T ((S_t + lambda I) C_t - G_t)
 *   den_t = q_t^T ((S_t + lambda I) m_t - h_t)
 *   out_t = num_t (default) or num_t / den_t (normalize = 1)
 * [EXP] "Methodik" item 1 (prefix summaries S, C, m; cross summaries G, h
 * that remove the future terms of the naive product S C; output
 * q^T(S C - G); ratio with a masked denominator); [SUM] sec. 3.1 (mask keeps
 * j <= t), sec. 4.3 (fixed decay as an attenuation factor), sec. 5.1 (ridge
 * lambda I, unnormalised output by default).  Equivalently
 *   num_t = sum_{j<=t} sum_{i<=j} g^(2t-i-j) (q_t.k_i)(k_i.q_j) v_j
 *           + lambda sum_{j<=t} g^(t-j) (q_t.q_j) v_j.
 * No epsilon is added to the denominator; a zero denominator gives IEEE
 * inf/NaN in the ratio.  NaN/Inf inputs propagate.
 *
 * Conventions shared by every entry point.
 *   - Device pointers are plain HIP device addresses, 16-byte aligned.
 *     Tensors are contiguous, row-major.  The state index of batch b,
 *     head h is b*H + h.
 *   - The caller owns all memory.  The library allocates and frees nothing
 *     and keeps no state between calls beyond its loaded code and the
 *     static scratch of hla_forward_chunked_noalloc.
 *   - Calls are asynchronous on `stream` (0 = the null stream) and never
 *     synchronise.  Validation is host-only and happens before anything is
 *     enqueued; on any error nothing is enqueued and no output is touched.
 *   - Errors are returned as hla_status; hla_last_error() gives a
 *     thread-local detail string for the last failing call on that thread.
 *     A launch failure reported by the HIP runtime is HLA_ERR_DEVICE.
 *   - All entry points are thread-safe; calls that share output, state or
 *     workspace memory must be ordered on one stream by the caller.
 */
#ifndef HLA_H_
#define HLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t only */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HLA_OK = 0,
    HLA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad gamma/ridge, aliasing */
    HLA_ERR_UNSUPPORTED = 2,      /* a size or width the library has no kernel for   */
    HLA_ERR_ALIGNMENT = 3,        /* a device pointer not 16-byte aligned             */
    HLA_ERR_WORKSPACE = 4,        /* workspace missing or smaller than required       */
    HLA_ERR_DEVICE = 5            /* the HIP runtime reported a launch error          */
} hla_status;

typedef enum { HLA_F32 = 0, HLA_BF16 = 1 } hla_dtype;

/* A segment summary for BH = B*H heads ([SUM] sec. 4.2: the masked state
 * tuple (S, C, m, G, h); rho is the segment's attenuation g^len, [SUM]
 * sec. 4.3).  All fp32 device arrays, contiguous:
 *   S [BH,d,d] (symmetric), C [BH,d,dv], m [BH,d], G [BH,d,dv], h [BH,d],
 *   rho [BH] (may be NULL: read as 1, not written). */
typedef struct {
    float *S;
    float *C;
    float *m;
    float *G;
    float *h;
    float *rho;
} hla_state;

typedef struct {
    int32_t B, H;        /* batch and heads, >= 1                                 */
    int32_t n;           /* tokens per head, >= 0 (decode: must be 1)             */
    int32_t d, dv;       /* key/query width and value width, each 16, 32, 64, 128 */
    int32_t chunk;       /* chunk width w: 16, 32, 64 or 128; 0 = default: w = d  */
    hla_dtype dtype;     /* element type of q, k, v                               */
    const float *gamma;  /* HOST array [H] of decays in (0, 1]; NULL = no decay   */
    float ridge;         /* lambda >= 0                                           */
    int32_t normalize;   /* 0: out = numerator; 1: out = numerator / denominator  */
} hla_params;

/* Bytes of device workspace hla_forward_chunked needs for these params
 * (0 for an invalid p).  Its first 8192 bytes are a control block that the
 * library keeps valid from call to call (32-bit words: 2 = launches of the
 * one-launch kernels, 3 = waits that hit the spin limit, 4 = that limit in
 * polls (0 = the built-in 4M; -1 = give up at once in the d = 128 kernel and
 * after one poll in the d = 64 kernel; the only word a caller may set, e.g.
 * to test the give-up path), 64 = finished-workgroup counter, 65 = launch
 * epoch, 66 = segment ticket).  Then come the flags of the one-launch
 * kernels, each tagged with the epoch of the launch that set it, in a region
 * of their own whose place and size depend on p alone, and then the data of
 * whichever path a call takes (per-chunk or per-segment partial summaries),
 * which never reaches the flags.  Zero-fill the workspace once before its
 * first use and write nothing else in it afterwards; it then serves any
 * number of calls with the same params (with or without states and den, in
 * any order).  Zero-fill it again before calls with other params: their data
 * may cover where this call's flags were.
 *
 * The one-launch kernels (bf16 with every decay >= 0.75: d = dv = 64, chunk
 * 64, every option and state; d = dv = 128 without ridge, den or ratio, with
 * an initial or final state when each head is one segment or B*H times
 * the segments per head is at most 256) hand partial sums between workgroups of one launch when a head is cut into
 * several segments: a segment waits for the sums of the earlier segments of
 * its head.  Both kernels then hand segments out by ticket, in increasing
 * order, so a segment only ever waits on segments that running workgroups
 * hold, whatever other streams run: every wait ends.  The sums travel as
 * device-coherent accesses.  A wait that still exceeds a fixed spin limit
 * (about 4M polls, seconds) gives up and adds one to word 3, and the carry
 * it waited for is made NaN: every output that depends on it (that
 * segment's and the later segments' of the head) is then NaN, never a wrong
 * number.
 *
 * Short sequences (n <= 256, d and dv in {16, 32}, fp32 or bf16, any decays,
 * no ridge, den, normalisation or states) take neither the chunks nor the
 * flags: the masked numerator is the sum of (q_t . k_i)(k_i . q_j) v_j over
 * i <= j <= t, decayed by g^(2t - i - j) (the equivalent form above: [SUM] sec. 3.1 and
 * 4.3), computed as two
 * direct causal maps, U_j = sum over i <= j of g^(j-i) (q_j . k_i) k_i and
 * out_t = sum over j <= t of g^(2(t-j)) (q_t . U_j) v_j, in fp32, with U
 * (B*H*n*d floats) kept in the workspace's data.  The chunk setting does not
 * change their result. */
size_t hla_forward_workspace_size(const hla_params *p);

/* Chunk-parallel masked forward ([SUM] sec. 4 and 5: token deltas feed an
 * exclusive scan inside each chunk, each token forms its inclusive state and
 * output, and chunk summaries are scanned with the same operator to give
 * carry-ins; the result equals the serial recurrence above up to fp32
 * rounding order).
 *   q, k  [B,H,n,d], v [B,H,n,dv] in p->dtype      (inputs, not modified)
 *   out   [B,H,n,dv] fp32                           (output)
 *   den   [B,H,n] fp32 or NULL                      (output: den_t)
 *   init  NULL = zero state, else the state at position -1 (all of S, C, m,
 *         G, h set; rho optional and only used to form final_state->rho)
 *   final_state  NULL, or receives the state after token n-1, with
 *         rho = (init rho or 1) * g^n.  The scan carries X = S C - G and
 *         y = S m - h and returns G = S C - X, h = S m - y, so G and h are
 *         accurate relative to the size of S C and S m (fp32 rounding on
 *         the chunked fp32 path, about 1e-5 of it on the one-launch bf16
 *         kernels, whose products split fp32 operands into bf16 pairs), not
 *         to their own: after one token G is exactly zero, and the value
 *         returned is a rounding residue of S C.
 *   workspace    device memory of at least hla_forward_workspace_size(p)
 *         bytes (may be NULL when that size is 0).
 * out and den must not overlap q, k, v, init or the workspace; init and
 * final_state must not overlap.  With n = 0 only final_state is written. */
hla_status hla_forward_chunked(const hla_params *p, const void *q, const void *k,
                               const void *v, float *out, float *den,
                               const hla_state *init, hla_state *final_state,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Bytes of the static scratch behind hla_forward_chunked_noalloc. */
#define HLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* hla_forward_chunked without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, computation, outputs and
 * errors as hla_forward_chunked, minus workspace and workspace_bytes: the
 * workspace is a static device array of HLA_NOALLOC_SCRATCH_BYTES owned by
 * the library, one per GPU it runs on, held until the process ends.  The
 * call allocates nothing; its first call on a device looks up that device's
 * copy of the array.  The array keeps 4 MiB for the one-launch kernels'
 * flags at a fixed place, so calls with any params, in any order, find their
 * flags outside every other call's data.  A call whose kernel path needs
 * more than that (the one-launch paths need 0.5 MB of flags and 14 MB of
 * data at B4 H8 n2048 d64, 2.1 MB and 54 MB at B8 H8 n4096 d64; the generic
 * path with an initial or final state needs about 2.2 KB of data per
 * head-token at d = dv = 64) fails with HLA_ERR_WORKSPACE before anything is
 * enqueued.  Every call on a GPU shares that GPU's array, which keeps the
 * previous call's contents (a control block that each call leaves valid for
 * the next, and flags that only ever hold launch epochs; nothing needs
 * clearing): calls that overlap in
 * time on one GPU (two streams or two host threads) race and must not be
 * made; calls ordered on one stream are fine, captured into a HIP graph
 * too. */
hla_status hla_forward_chunked_noalloc(const hla_params *p, const void *q, const void *k,
                                       const void *v, float *out, float *den,
                                       const hla_state *init, hla_state *final_state,
                                       hipStream_t stream);

/* Bytes of device workspace hla_backward_chunked needs for these params (0
 * for an invalid p).  Unlike the forward's, it holds no control block: its
 * contents need no initialisation and are overwritten by every call. */
size_t hla_backward_workspace_size(const hla_params *p);

/* Gradients of the chunked forward: with L = sum_t <out_t, dout_t>, writes
 * dq = dL/dq, dk = dL/dk, dv = dL/dv for every option of p (decay per head,
 * ridge, normalize), from the zero state or from `init`, and on request the
 * gradient with respect to that initial state; a gradient flowing into the
 * final state (`dfinal`) may be added to L.  [SUM] sec. 4 and 5 (the scan
 * trains chunk-parallel; the state at a segment boundary is what sequence
 * shards hand on, so its gradient is what they hand back).  The gradient is
 * itself a masked second-order scan, run from the last token to the first:
 * with Gb_j = sum_{t>=j} g^(2(t-j)) q_t dnum_t^T (and its den column),
 * w_j = Gb_j v_j and T_i = sum_{j>=i} g^(j-i) (w_j q_j^T + q_j w_j^T),
 *   dq_t = X_t dnum_t + S_t w_t (+ ridge terms),  dk_i = T_i k_i,
 *   dv_j = Gb_j^T S_j q_j (+ ridge terms),
 * where X = S C - G is the forward's corrected carry; for the ratio
 * dnum = dout/den and the den column carries -(dout . out)/den.  The forward
 * is recomputed inside the call (its out and den are not inputs).
 *   q, k  [B,H,n,d], v [B,H,n,dv] in p->dtype       (inputs, not modified)
 *   init  NULL = zero state, else the state at position -1 (all of S, C, m,
 *         G, h set; as for hla_forward_chunked)
 *   dout  [B,H,n,dv] fp32                            (input)
 *   dq, dk [B,H,n,d], dv [B,H,n,dv] fp32             (outputs)
 *   dfinal NULL = none, else all of S, C, m, G, h set (fp32, shaped as a
 *         state; rho not read): L gains sum over the parts of <final part,
 *         dfinal part>, the gradient a later segment hands back.  It enters
 *         the reverse scan as its carries one token past the last, so every
 *         decay must be >= 1e-6 (HLA_ERR_UNSUPPORTED otherwise).  With n = 0
 *         it passes straight to dinit.
 *   dinit NULL = not formed, else all of S, C, m, G, h set (fp32, shaped as
 *         a state): receives dL/d(init) (of the zero state when init is
 *         NULL); its rho, if set, receives 0 (rho reaches no output).  Each
 *         entry of S counts as its own variable, the read-out of token t
 *         being (S_t q_t)^T C_t; with Gb_0 and Cb_0 (Cb: powers g^(t-j)) at
 *         token 0 and [C | m], [G | h] of init widened by the den column,
 *           dS = g^2 [C|m] Gb_0^T + sum_j g^(j+1) q_j w_j^T,
 *           d[C|m] = g^2 S Gb_0 + lambda g Cb_0,   d[G|h] = -g^2 Gb_0,
 *         plus, with dfinal, g^n (dS_f + [C|m]_n d[G|h]_f^T) in dS and
 *         g^n (d[C|m]_f + S_n d[G|h]_f) in d[C|m] (Gb_0 already holds the
 *         g^(2n) X_n part).  For n = 0 it is dfinal, or zero.
 *   workspace  device memory of at least hla_backward_workspace_size(p)
 *         bytes, 256-byte aligned (may be NULL when n = 0).
 * Outputs must not overlap each other, the inputs or the workspace.  With the
 * ratio, a zero denominator gives IEEE inf/NaN gradients. */
hla_status hla_backward_chunked(const hla_params *p, const void *q, const void *k,
                                const void *v, const hla_state *init, const float *dout,
                                float *dq, float *dk, float *dv, const hla_state *dfinal,
                                hla_state *dinit, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* One streaming decode step ([SUM] sec. 1 and 2: constant-size state,
 * O(d^2 + d dv) work per token): applies token (q, k, v) to `state` in place
 * and writes its output.  p->n must be 1.
 *   q, k [B,H,d], v [B,H,dv] in p->dtype
 *   state  in/out, all of S, C, m, G, h set; S must be symmetric (as the
 *          method produces it); rho, if set, is multiplied by g
 *   out    [B,H,dv] fp32; den [B,H] fp32 or NULL
 * Each of S, C, G is read once and written once. */
hla_status hla_decode_step(const hla_params *p, const void *q, const void *k,
                           const void *v, hla_state *state, float *out, float *den,
                           hipStream_t stream);

/* The decode state with the key moment shared by groups of query heads and
 * stored packed ([SUM] sec. 5.2: multi-query sharing reduces the state from
 * O(h d^2) to O(d^2 + h d dv); packed symmetric storage of S cuts
 * bandwidth).  For B batches, H query heads and kv_heads groups (H a
 * multiple of kv_heads; group j holds query heads j*R .. j*R + R - 1,
 * R = H / kv_heads), fp32 device arrays:
 *   S   [B*kv_heads, d*(d+1)/2]  the group's key moment, packed: the 32 x 32
 *       tiles (I, J), I <= J, in row-major tile order, an off-diagonal tile
 *       whole (1024 floats, row-major), a diagonal tile as its upper
 *       triangle (528 floats, row r holding columns r..31);
 *   C, G [B*H, d, dv], m, h [B*H, d]  per query head, as in hla_state;
 *   rho [B*kv_heads] or NULL. */
typedef struct {
    float *S;
    float *C;
    float *m;
    float *G;
    float *h;
    float *rho;
} hla_mq_state;

/* One decode step ([SUM] sec. 1, 2 and 5.2) for query heads that share keys
 * and values in groups (grouped / multi-query attention): the update and
 * output of hla_decode_step for every query head, with one key moment S per
 * group, read from and written to packed storage.
 *   p          B, H (query heads), d in {32, 64, 128}, dv, dtype, gamma
 *              (per query head, equal within a group), ridge, normalize;
 *              n must be 1
 *   q          [B,H,d];  k [B,kv_heads,d];  v [B,kv_heads,dv]  (p->dtype)
 *   state      in/out, updated in place (hla_mq_state)
 *   out        [B,H,dv] fp32;  den [B,H] fp32 or NULL
 * With one query head per group (kv_heads = H) this is the unshared step on
 * packed storage: each of S (packed), C, G read once and written once.
 * With groups of several heads the group's S is read by each of its heads
 * and then updated once. */
hla_status hla_decode_step_mq(const hla_params *p, int32_t kv_heads, const void *q, const void *k,
                              const void *v, hla_mq_state *state, float *out, float *den,
                              hipStream_t stream);

/* Converts `count` symmetric d x d key moments (d in {32, 64, 128}) between
 * full storage ([count,d,d], as in hla_state) and the packed storage of
 * hla_mq_state ([count, d*(d+1)/2]): pack reads the upper triangle of each
 * full matrix; unpack writes both triangles.  src and dst must not overlap. */
hla_status hla_key_moment_pack(int32_t count, int32_t d, const float *S_full, float *S_packed,
                               hipStream_t stream);
hla_status hla_key_moment_unpack(int32_t count, int32_t d, const float *S_packed, float *S_full,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * The asymmetric variant (AHLA) and third order.
 *
 * AHLA ([SUM] sec. 6, 6.1-6.3; [EXP] "Methodik" item 2): the masked
 * left-cascaded product Q (K^T Q)(K^T V), per head with decay g:
 *   num_t = sum_{j<=t} sum_{i<=j} g^(t-i) (q_t . k_j)(q_j . k_i) v_i
 *   den_t = the same with every v_i = 1;   out_t = num_t or num_t / den_t
 * Streaming summaries, each decayed by g per token:
 *   P_t = g P + k v^T,  m_t = g m + k,  E_t = g E + k (P_t^T q)^T,
 *   n_t = g n + (q . m_t) k;   num_t = E_t^T q_t,  den_t = q_t . n_t.
 *
 * Third order ([SUM] sec. 7, 7.1-7.3; [EXP] "Methodik" item 3): A A^T A V
 * with A = Q K^T, masked at every factor, no decay (the pages state its scan
 * for g = 1):
 *   num_t = sum_{j<=t} sum_{i<=j} sum_{l<=j} (q_t . k_i)(k_i . q_j)(q_j . k_l) v_l
 * Streaming state: S_t = S + k k^T, P_t = P + k v^T, m_t = m + k,
 *   F_t = F + (S_t q)(P_t^T q)^T,  Fd_t = Fd + (q . m_t)(S_t q);
 *   num_t = F_t^T q_t,  den_t = q_t . Fd_t.
 *
 * Both take hla_params with ridge = 0 (the pages define no ridge for them;
 * HLA_ERR_UNSUPPORTED otherwise); third order takes gamma NULL or all 1.
 * Arguments, layouts, aliasing rules and errors are those of
 * hla_forward_chunked and hla_decode_step, with these states (fp32 device
 * arrays, BH = B*H entries): */
typedef struct {
    float *P;    /* [BH,d,dv] */
    float *m;    /* [BH,d]    */
    float *E;    /* [BH,d,dv] */
    float *n;    /* [BH,d]    */
    float *rho;  /* [BH] or NULL: g^len of the covered segment (NULL read as 1) */
} hla_ahla_state;

typedef struct {
    float *S;    /* [BH,d,d] (symmetric) */
    float *P;    /* [BH,d,dv] */
    float *m;    /* [BH,d]    */
    float *F;    /* [BH,d,dv] */
    float *Fd;   /* [BH,d]    */
} hla_third_state;

/* Workspace bytes of the AHLA / third-order forward; 0 for an invalid p.
 * As for hla_forward_chunked: its first 8 KB are a control block, the flags
 * that follow are tagged with the launch epoch kept there (both kept valid
 * from call to call: a call never clears them), and no path's data reaches
 * the flags; zero-fill the workspace once before its first use, write
 * nothing in it afterwards, and zero-fill it again before calls with other
 * params or of the other order.  bf16 calls with d = dv = 64, chunk 64, every decay >= 0.75,
 * no denominator, ratio or state run one-launch kernels (AHLA as first-order
 * attention applied twice, third order as second-order HLA over first-order
 * attention values); every other call runs the chunked fp32 kernels. */
size_t hla_ahla_workspace_size(const hla_params *p);
size_t hla_third_workspace_size(const hla_params *p);

/* Chunk-parallel forward (sec. 6.2 / 7.3: an exclusive scan of chunk
 * summaries gives each chunk its carry-in, the result equals the serial
 * recurrence up to fp32 rounding order).  init NULL = zero state;
 * final_state NULL = not returned (AHLA rho = (init rho or 1) * g^n). */
hla_status hla_ahla_forward(const hla_params *p, const void *q, const void *k, const void *v,
                            float *out, float *den, const hla_ahla_state *init,
                            hla_ahla_state *final_state, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);
hla_status hla_third_forward(const hla_params *p, const void *q, const void *k, const void *v,
                             float *out, float *den, const hla_third_state *init,
                             hla_third_state *final_state, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* One streaming step per state (sec. 6.3 / 7.2), state updated in place;
 * q, k [B,H,d], v [B,H,dv]; out [B,H,dv]; den [B,H] or NULL.  Each state
 * matrix is read once and written once. */
hla_status hla_ahla_decode_step(const hla_params *p, const void *q, const void *k, const void *v,
                                hla_ahla_state *state, float *out, float *den, hipStream_t stream);
hla_status hla_third_decode_step(const hla_params *p, const void *q, const void *k, const void *v,
                                 hla_third_state *state, float *out, float *den, hipStream_t stream);

/* Masked semidirect-product composition of `count` segment pairs, earlier
 * segment a then later segment b ([SUM] sec. 4.2; [EXP] "Assoziative
 * Operatoren", cross term S_B C_A):
 *   S = rho_b S_a + S_b       C = rho_b C_a + C_b       m = rho_b m_a + m_b
 *   G = rho_b^2 G_a + G_b + rho_b S_b C_a
 *   h = rho_b^2 h_a + h_b + rho_b S_b m_a            rho = rho_a rho_b
 * All three states hold `count` entries of width d x dv (d, dv in
 * {16,32,64,128}); result must not overlap either input. */
hla_status hla_state_compose(int32_t count, int32_t d, int32_t dv,
                             const hla_state *earlier, const hla_state *later,
                             hla_state *result, hipStream_t stream);

/* Static name of a status code. */
const char *hla_status_string(hla_status s);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char *hla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HLA_H_ */
