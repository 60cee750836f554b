/*
 * vwl.h -- speculative verification and logit fusion over vocabulary-wide
 * logit rows, on AMD Instinct MI355X (gfx950).
 *
 * Entry points, one per method (plus the AsymSpec ablation variants):
 *
 *   asym_verify   AsymSpec ("AsymSpec: Context-Asymmetric Speculative
 *                 Decoding for Agentic LLMs" reading notes, section 4.1
 *                 "contrastive delta-fusion" and section 4.2 "CDA gate").
 *   e2sci_verify  E2-SCI ("E2-SCI: Elastic Edge-Cloud Speculative Decoding
 *                 via Credit Inertia" notes, key design 3 "online adaptive
 *                 verification").
 *   rapid_verify  RAPID ("RAPID: Long-Context Inference with
 *                 Retrieval-Augmented Speculative Decoding" notes, key
 *                 designs 2 "retrieval-augmented target distribution",
 *                 3 "tail protection" and 4 "adjusted residual sampling",
 *                 with the rejection-sampling loop of its overall framework).
 *
 * Conventions shared by every call:
 *   - Every data pointer is a DEVICE pointer on the current HIP device.  The
 *     caller allocates and owns every buffer; the library never allocates,
 *     frees or synchronises.  Every call is asynchronous on `stream`.
 *   - Logit tensors are contiguous, row-major [B][P][V] (P positions per
 *     request), in the dtype given, with 16-byte-aligned base pointers; any
 *     V >= 1 is accepted (rows that do not start on a 16-byte boundary are
 *     peeled).  Index arrays are int32 and uniforms fp32 (4-byte aligned),
 *     flags uint8.  A misaligned pointer returns VWL_ERR_ALIGN.
 *   - Host-side argument checks run synchronously and return a status; a
 *     failed launch returns VWL_ERR_HIP (from hipGetLastError).
 *   - Device-side data faults cannot be reported synchronously; they get
 *     defined behaviour and set bits in *dev_err when dev_err is non-null
 *     (the kernels OR bits in; the caller clears it):
 *       VWL_DEVERR_DRAFT    a draft id outside [0, V): that draft is rejected
 *       VWL_DEVERR_UNIFORM  a uniform outside [0, 1) or NaN: clamped into [0, 1)
 *       VWL_DEVERR_TIMEOUT  a workgroup waited more than ~2 s for the others
 *                           of its row (only possible when the device is
 *                           starved); outputs of that call are undefined and
 *                           the workspace must be reset with vwl_workspace_reset
 *   - Workspace: 256-byte-aligned device memory of at least the size the
 *     matching *_workspace_bytes query returns for the same shape (the size
 *     depends on the shape and dtype only, not on the device).  It must be
 *     zero-filled before its first use (vwl_workspace_reset does that); every
 *     completed call leaves every counter, flag and exchange word that a
 *     later call reads before writing back at zero (the rest holds values a
 *     later call overwrites before reading them).  Two calls that share one
 *     workspace must be ordered (same stream, or synchronised).
 *   - Results are bitwise deterministic for identical inputs, shape and device.
 */
#ifndef VWL_H
#define VWL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VWL_OK = 0,
    VWL_ERR_NULL = 1,      /* a required pointer is null */
    VWL_ERR_SHAPE = 2,     /* B, K/G or V out of range, or sizes overflow */
    VWL_ERR_DTYPE = 3,     /* unknown dtype */
    VWL_ERR_PARAM = 4,     /* beta, gamma, eta or T out of range */
    VWL_ERR_WORKSPACE = 5, /* workspace smaller than the query returns */
    VWL_ERR_HIP = 6,       /* a HIP runtime call or kernel launch failed */
    VWL_ERR_ALIGN = 7,     /* a pointer is not aligned as documented */
    VWL_ERR_SCRATCH = 8,   /* asym_verify_noalloc: the shape needs more than its static scratch */
    VWL_STATUS_INT_MIN_ = -2147483647 - 1, /* not codes: they give the enum the range of an int */
    VWL_STATUS_INT_MAX_ = 2147483647
} vwl_status;

/* Logit storage.  Every enum of this header spans the whole int range, so
 * any int a C caller passes is a value of the type (an unknown one is
 * refused with a status, never undefined behaviour). */
typedef enum {
    VWL_F32 = 0,
    VWL_BF16 = 1,
    VWL_DTYPE_INT_MIN_ = -2147483647 - 1,
    VWL_DTYPE_INT_MAX_ = 2147483647
} vwl_dtype;

#define VWL_DEVERR_DRAFT 1
#define VWL_DEVERR_UNIFORM 2
#define VWL_DEVERR_TIMEOUT 4
#define VWL_DEVERR_MAP 8     /* a vocabulary-alignment entry outside [-1, Vd): treated as unpaired */

#define VWL_MAX_K 63 /* drafts per request, both methods */

/* Human-readable name of a status code (static storage); any int is
 * accepted, values that are no vwl_status give "unknown vwl_status". */
const char *vwl_status_string(int status);

/* Library version as an integer: major*10000 + minor*100 + patch. */
int vwl_version(void);

/* Zero-fill `bytes` of workspace on `stream` with a fill kernel (no memset
 * node, so it may be captured into a graph).  Returns VWL_ERR_NULL for a null
 * pointer with bytes > 0. */
vwl_status vwl_workspace_reset(void *workspace, size_t bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * AsymSpec verification (AsymSpec notes, sections 4.1-4.2)
 *
 * For request b and position i in [0, K] (row r = b*(K+1) + i):
 *   L_x      = log sum_v exp(x_v)           for x in {a_i, b_i, t_i}
 *   D_i      = JSD(softmax(a_i) || softmax(b_i)), natural log, in [0, ln 2]
 *   geff_i   = gamma * exp(-D_i)            (section 4.2, the CDA threshold)
 *   fused_i  = lowest v maximising t_v + beta*(a_v - b_v)   (section 4.1)
 *   for i < K, with d = draft[b][i]:
 *   accept_i = softmax(t_i)[d] > geff_i * softmax(b_i)[d]   (section 4.2),
 *              evaluated as (t_d - L_t) - (b_d - L_b) > log(gamma) - D_i
 *   accept_len[b] = first i < K with accept_i == 0, else K
 *   token[b]      = fused[b][accept_len[b]]  (the delta-fusion token at the
 *                   first rejection; the bonus row K when all are accepted)
 *
 * Inputs:
 *   a, b, t   [B][K+1][V] logits of dtype `dt`: drafter on the full context,
 *             drafter on the compressed context, verifier on the compressed
 *             context.  Row i of request b holds position i.
 *   draft     [B][K] int32 draft ids (may be null when K == 0).
 *   B >= 1, 0 <= K <= VWL_MAX_K, V >= 1; B*(K+1)*V must fit in int64.
 *   beta      finite (any sign); gamma finite and >= 0.
 * Outputs (all required; written in full by every successful call):
 *   D, gamma_eff  [B][K+1] fp32
 *   accept        [B][K]   uint8 (may be null when K == 0)
 *   fused         [B][K+1] int32
 *   accept_len, token  [B] int32
 *   dev_err       [1] int32, nullable; bits are OR-ed in.
 * Precision: per-lane fp32 arithmetic on the widened logits, fp64 for every
 *   combine across lanes and workgroups and for the row scalars.
 * --------------------------------------------------------------------------- */
size_t vwl_asym_workspace_bytes(int B, int K, int V, vwl_dtype dt);

vwl_status asym_verify(const void *a, const void *b, const void *t,
                       const int32_t *draft,
                       int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                       float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                       int32_t *accept_len, int32_t *token, int32_t *dev_err,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * asym_verify without a workspace argument, for callers that cannot allocate
 * device memory or hand the library any: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.
 *
 * Same inputs, outputs, results (bit for bit) and errors as asym_verify; the
 * workspace is a static device array of VWL_NOALLOC_SCRATCH_BYTES per device,
 * held until the process ends.  The call allocates and frees nothing.  The
 * first call on a device looks up the array's address and zero-fills it with
 * a fill kernel on `stream`; every completed call leaves its counters at zero
 * again.  A shape whose vwl_asym_workspace_bytes exceeds the scratch returns
 * VWL_ERR_SCRATCH (at V = 151936 the scratch holds 2,781 bf16 or 1,403 fp32
 * rows B*(K+1); the large B = 256, K = 4 bf16 batch needs 7.7 MB).
 * All calls on one device share its scratch: two calls that may overlap on a
 * device (different streams without ordering, or different host threads)
 * race, and their results are undefined.  Order them.
 * --------------------------------------------------------------------------- */
#define VWL_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

vwl_status asym_verify_noalloc(const void *a, const void *b, const void *t,
                               const int32_t *draft,
                               int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                               float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                               int32_t *accept_len, int32_t *token, int32_t *dev_err,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * AsymSpec variants: the mechanism ablation of the AsymSpec notes
 * (experiments, and the counterfactual reasoning of its analysis) replaces
 * the fusion source and drops the CDA gate.
 *
 *   delta  VWL_DELTA_A_MINUS_B  delta = a - b, the context gain (section 4.1;
 *                               asym_verify)
 *          VWL_DELTA_A          delta = a, the raw full-context logits
 *          VWL_DELTA_T_MINUS_B  delta = t - b, the two-model difference of
 *                               speculative contrastive decoding
 *          fused_i = lowest v maximising t_v + beta*delta_v
 *   gate   VWL_GATE_CDA    threshold gamma*exp(-D_i) (section 4.2; asym_verify)
 *          VWL_GATE_FIXED  threshold gamma: accept_i = softmax(t_i)[d] >
 *                          gamma*softmax(b_i)[d]; D is not computed (D[r] is
 *                          written as NaN) and gamma_eff[r] = gamma
 *
 * Everything else (inputs, outputs, layouts, workspace, errors) is as for
 * asym_verify, which equals asym_verify_variant(..., VWL_DELTA_A_MINUS_B,
 * VWL_GATE_CDA, ...).  `a` may be null, and is never read, with
 * VWL_GATE_FIXED and VWL_DELTA_T_MINUS_B.  An unknown enum value returns
 * VWL_ERR_PARAM.
 * --------------------------------------------------------------------------- */
typedef enum {
    VWL_DELTA_A_MINUS_B = 0,
    VWL_DELTA_A = 1,
    VWL_DELTA_T_MINUS_B = 2,
    VWL_DELTA_INT_MIN_ = -2147483647 - 1,
    VWL_DELTA_INT_MAX_ = 2147483647
} vwl_delta_source;
typedef enum { VWL_GATE_CDA = 0, VWL_GATE_FIXED = 1, VWL_GATE_INT_MIN_ = -2147483647 - 1, VWL_GATE_INT_MAX_ = 2147483647 } vwl_gate;

vwl_status asym_verify_variant(const void *a, const void *b, const void *t,
                               const int32_t *draft,
                               int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                               vwl_delta_source delta, vwl_gate gate,
                               float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                               int32_t *accept_len, int32_t *token, int32_t *dev_err,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * AsymSpec across model families (AsymSpec notes, the analysis of why
 * cross-family pairs work at a discount): the drafter's context gain lives
 * on the drafter's vocabulary and reaches the verifier through a vocabulary
 * alignment (string-identical tokens plus paired special tokens), with
 * generation restricted to the paired tokens.
 *
 *   a, b   [B][K+1][Vd] drafter logits (full and compressed context)
 *   t      [B][K+1][Vt] verifier logits, its own vocabulary
 *   vmap   [Vt] int32 device array: the drafter id paired with verifier
 *          token v, or -1 (an entry outside [-1, Vd) is treated as -1 and
 *          sets VWL_DEVERR_MAP)
 *   draft  [B][K] int32 drafts as VERIFIER ids
 * Per row: L_a, L_b over Vd, L_t over Vt; D = JSD(softmax(a) || softmax(b))
 * on the drafter vocabulary; gamma_eff = gamma*exp(-D);
 *   fused_i  = lowest verifier id v with vmap[v] >= 0 maximising
 *              t_v + beta*(a[vmap v] - b[vmap v])  (-1 when nothing is paired)
 *   accept_i = softmax(t_i)[d] > gamma_eff * softmax(b_i)[vmap d]; a draft
 *              without a pair is rejected (a draft outside [0, Vt) also sets
 *              VWL_DEVERR_DRAFT)
 * accept_len, token as asym_verify.  Outputs, dtype rules and errors as
 * asym_verify; Vt >= 1; the workspace comes from
 * vwl_asym_xfam_workspace_bytes.  With Vt = Vd and the identity alignment
 * the results equal asym_verify's.  When every row is made of whole 16-byte
 * vectors (Vd and Vt times the element size multiples of 16) a staged
 * verifier pass reads a, b and t contiguously; other vocabulary sizes take a
 * pass that gathers a and b through vmap.  Both give the same results up to
 * the fp64 summation order of L_t.
 * --------------------------------------------------------------------------- */
size_t vwl_asym_xfam_workspace_bytes(int B, int K, int Vd, int Vt, vwl_dtype dt);

vwl_status asym_verify_xfam(const void *a, const void *b, int Vd, const void *t, int Vt,
                            const int32_t *vmap, const int32_t *draft,
                            int B, int K, vwl_dtype dt, float beta, float gamma,
                            float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                            int32_t *accept_len, int32_t *token, int32_t *dev_err,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * AsymSpec from hidden states (the step before the pass on the AsymSpec
 * pages: the LM heads turn hidden states into logits).  The heads' products
 * are formed on the matrix cores with the row statistics in their epilogue,
 * and t is never written.  The JSD needs a and b again once their
 * log-sum-exps are known: with a workspace of
 * vwl_asym_lmhead_workspace_bytes the drafter's logit pairs (a, b) are
 * written once to it, as fp32, and streamed back; with one of at least
 * vwl_asym_lmhead_workspace_min_bytes (but less) a and b are formed again
 * instead (the same bits), so no logit is ever written to memory:
 *   a = h_a W_d^T, b = h_b W_d^T (the drafter's head, full and compressed
 *   context), t = h_t W_t^T (the verifier's head); then everything as
 *   asym_verify (delta = a - b, the CDA gate).
 * Inputs, all bf16, row-major, 16-byte aligned:
 *   h_a, h_b  [B][K+1][Hd]; h_t [B][K+1][Ht]; W_d [V][Hd]; W_t [V][Ht]
 *   (one row of a head per vocabulary entry); Hd and Ht multiples of 64
 *   (else VWL_ERR_SHAPE); draft [B][K] int32.
 * Outputs as asym_verify.  Precision: each logit is an fp32 sum of exact
 *   bf16 products (MFMA accumulation), so within Hd (or Ht) * 2^-24 *
 *   sum_k |h_k w_k| of its value; the draft's logits in the test are fp64
 *   dot products; statistics as asym_verify.
 * Workspace: vwl_asym_lmhead_workspace_bytes (shape only; about
 * 8 * B * (K+1) * V bytes, the stored pairs, plus the per-row records and
 * partials) for the stored pairs, at least
 * vwl_asym_lmhead_workspace_min_bytes (the records and partials) for the
 * path that forms a and b twice; smaller: VWL_ERR_WORKSPACE.  Zero-filled
 * before first use; left zero-filled where it must be.  Both sizes are 0 for
 * an invalid shape.
 * --------------------------------------------------------------------------- */
size_t vwl_asym_lmhead_workspace_bytes(int B, int K, int V, int Hd, int Ht);
size_t vwl_asym_lmhead_workspace_min_bytes(int B, int K, int V, int Hd, int Ht);

vwl_status asym_verify_lmhead(const void *h_a, const void *h_b, const void *W_d,
                              const void *h_t, const void *W_t, const int32_t *draft,
                              int B, int K, int V, int Hd, int Ht, float beta, float gamma,
                              float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                              int32_t *accept_len, int32_t *token, int32_t *dev_err,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * E2-SCI adaptive JSD acceptance ("E2-SCI: Elastic Edge-Cloud Speculative
 * Decoding via Credit Inertia" notes, key design 3 "online adaptive
 * verification", with the credit state of key design 1)
 *
 * One window of W drafts per request b, verified against the window's
 * threshold T_in[b]; then the caller-owned credit state moves on:
 *   D_i      = JSD(softmax(y_i) || softmax(z_i)), natural log, in [0, ln 2]
 *   accept_i = D_i <= T_in[b]     (a divergence above the threshold rejects)
 *   accept_len[b] = first i with accept_i == 0, else W
 *   r_hat[b] := (1 - ewma) * r_hat[b] + ewma * accept_len[b] / W
 *   T_prop    = max(T_min, min(T_base + alpha * omega[b] * (r_hat[b] - tau_credit), T_max))
 * then the stabilisers the same passage names (hysteresis, a minimum refresh
 * interval, a fall-back to a conservative threshold when the acceptance
 * drops below delta; the page gives no rule, this is the library's reading),
 * in this order, with p_acc = accept_len[b] / W:
 *   p_acc < delta                       -> T_out = T_safe, age := 0
 *   else age[b] + 1 < min_refresh       -> T_out = T_in,   age := age + 1
 *   else |T_prop - T_in| > hysteresis   -> T_out = T_prop, age := 0
 *   else                                -> T_out = T_in,   age := age + 1
 * (age saturates at INT32_MAX).  Zero-initialised stabiliser fields switch
 * them off: T_out is then T_prop.  The page's EWMA decay is 0.3; the other
 * constants are the caller's (the page gives none).  omega is the adaptive
 * weight of the page's predictor, which needs trained weights and stays with
 * the caller.
 *
 * Inputs:
 *   y, z      [B][W][V] drafter and target logits of dtype `dt`, 16-byte
 *             aligned; W >= 1 draft positions per request, W <= VWL_MAX_K+1.
 *   T_in, omega  [B] fp32 device arrays.
 *   r_hat     [B] fp32 device array, read and updated in place.
 *   age       [B] int32 device array, read and updated in place: windows
 *             the request's current threshold has been in effect before this
 *             one (0 when the threshold was just set).  May be null when
 *             min_refresh <= 1 (every window may refresh; no count is kept).
 *   params    host pointer; every constant finite, T_min <= T_max,
 *             0 <= ewma <= 1, hysteresis >= 0, min_refresh >= 0, and
 *             T_min <= T_safe <= T_max when delta > 0, else VWL_ERR_PARAM;
 *             min_refresh > 1 with a null age is VWL_ERR_NULL.
 * Outputs: D [B][W] fp32, accept [B][W] uint8, accept_len [B] int32,
 *   T_out [B] fp32 (may alias T_in: each row reads its threshold before the
 *   request's last row writes the next one), dev_err nullable.
 * Workspace: vwl_e2sci_workspace_bytes, with the same rules as the others.
 * Precision: as asym_verify (fp32 lanes, fp64 combines); the decision
 *   D <= T and the state update are taken in fp64.
 * --------------------------------------------------------------------------- */
typedef struct {
    float alpha;      /* gain of the credit term */
    float tau_credit; /* neutral credit level */
    float T_base;     /* base threshold */
    float T_min;      /* lower safety bound */
    float T_max;      /* upper safety bound */
    float ewma;       /* EWMA decay of the credit state (0.3 on the page) */
    float hysteresis; /* dead band: a smaller threshold change is not made */
    int32_t min_refresh; /* windows a threshold stays in effect at least */
    float delta;      /* acceptance floor of the safety check (0: off) */
    float T_safe;     /* conservative threshold of the safety check */
} vwl_e2sci_params;

size_t vwl_e2sci_workspace_bytes(int B, int W, int V, vwl_dtype dt);

vwl_status e2sci_verify(const void *y, const void *z, int B, int W, int V, vwl_dtype dt,
                        const float *T_in, const float *omega, float *r_hat, int32_t *age,
                        const vwl_e2sci_params *params,
                        float *D, uint8_t *accept, int32_t *accept_len, float *T_out,
                        int32_t *dev_err, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Launch plan of e2sci_verify (same fields as vwl_plan_info; [5] = B*W). */
vwl_status vwl_e2sci_plan_info(int B, int W, int V, vwl_dtype dt, int64_t out[6]);

/* Largest vocabulary a RAPID call accepts (2^21 logits per row). */
#define VWL_RAPID_MAX_V 2097152

/* ---------------------------------------------------------------------------
 * RAPID verification (RAPID notes, key designs 2-4)
 *
 * For request b and position i in [0, G] (G drafts, the page's "gamma"):
 *   p = softmax(z_i / T), q = softmax(y_i / T)
 *   zhat = z_i + eta*T*(q - p)                       (design 2)
 *   phat_raw = softmax(zhat / T)
 *   phat_v = p_v where phat_raw_v < 0.1 * max phat_raw, else phat_raw_v
 *            (design 3; no renormalisation afterwards)
 *   for i < G, with x = draft[b][i] and u = u_accept[b][i]:
 *   accept_i = u * q(x) < phat(x)     (rejection sampling against phat)
 *   n = accept_len[b] = first i < G with accept_i == 0, else G
 *   token[b]: if n < G, the residual r = max(p - phat, p - q, 0) of row n
 *             (design 4), S = sum r, token = smallest k with
 *             sum_{v<=k} r_v > u_sample[b][n] * S; when S == 0, or when
 *             n == G (all drafts accepted), the same inverse-CDF rule on p
 *             of row n with u_sample[b][n].
 *
 * Inputs:
 *   z, y      [B][G+1][V] target and RAG-drafter logits of dtype `dt`.
 *   draft     [B][G] int32 (may be null when G == 0).
 *   u_accept  [B][G] fp32 in [0,1) (may be null when G == 0);
 *   u_sample  [B][G+1] fp32 in [0,1).
 *   B >= 1, 0 <= G <= VWL_MAX_K, 1 <= V <= VWL_RAPID_MAX_V; eta finite and
 *   >= 0; T finite and > 0.  Otherwise VWL_ERR_SHAPE / VWL_ERR_PARAM.
 * Outputs:
 *   accept     [B][G] uint8 (may be null when G == 0)
 *   accept_len, token  [B] int32 (required)
 *   p_hat_draft, q_draft  [B][G] fp32, nullable: phat(x_i) and q(x_i)
 *   emit_dist  [B][V] fp32, nullable: the normalised distribution the token
 *              was drawn from (r/S, or p of row n)
 *   dev_err    [1] int32, nullable.
 * Precision: fp32 element arithmetic with fp64 sums for the row statistics;
 *   the emitting row's residual, its sums and the inverse CDF in fp64.
 * --------------------------------------------------------------------------- */
size_t vwl_rapid_workspace_bytes(int B, int G, int V, vwl_dtype dt);

vwl_status rapid_verify(const void *z, const void *y, const int32_t *draft,
                        const float *u_accept, const float *u_sample,
                        int B, int G, int V, vwl_dtype dt, float eta, float T,
                        uint8_t *accept, int32_t *accept_len, int32_t *token,
                        float *p_hat_draft, float *q_draft, float *emit_dist,
                        int32_t *dev_err, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Launch-plan inspection (host only; no device memory is touched).
 * Fills `out` with: [0] workgroups per row (team size), [1] 16-byte vectors
 * per thread per tensor, [2] teams, [3] grid size, [4] threads per
 * workgroup, [5] rows.  Returns VWL_OK or an argument status.
 * mode 0 = AsymSpec, 1 = RAPID (G in place of K).
 * --------------------------------------------------------------------------- */
vwl_status vwl_plan_info(int mode, int B, int K, int V, vwl_dtype dt, int64_t out[6]);

/* The same for one AsymSpec variant (the plan depends on the variant's
 * register use); vwl_plan_info(0, ...) is the VWL_DELTA_A_MINUS_B,
 * VWL_GATE_CDA plan. */
vwl_status vwl_asym_plan_info(int B, int K, int V, vwl_dtype dt, vwl_delta_source delta, vwl_gate gate,
                              int64_t out[6]);

/* Host-only argument check of asym_verify / rapid_verify: the same checks,
 * in the same order, without launching anything.  Lets a caller (or a test
 * on a machine without a GPU) validate arguments; `workspace_bytes` is
 * compared against `needed_bytes` instead of querying the device. */
vwl_status vwl_asym_check(const void *a, const void *b, const void *t, const int32_t *draft,
                          int B, int K, int V, int dt, float beta, float gamma,
                          const void *D, const void *gamma_eff, const void *accept,
                          const void *fused, const void *accept_len, const void *token,
                          const void *workspace, size_t workspace_bytes, size_t needed_bytes);

vwl_status vwl_rapid_check(const void *z, const void *y, const int32_t *draft,
                           const float *u_accept, const float *u_sample,
                           int B, int G, int V, int dt, float eta, float T,
                           const void *accept, const void *accept_len, const void *token,
                           const void *workspace, size_t workspace_bytes, size_t needed_bytes);

/* Tuning hook: pin the vectors-per-thread choice (1, 2, 4 or 8; 0 = automatic)
 * and cap the number of teams (0 = no cap) of one mode (0 = AsymSpec,
 * 1 = RAPID) for later calls in this process.  Results do not depend on the
 * plan except through the documented fp32 summation order of the partials. */
vwl_status vwl_set_plan_override(int mode, int nv, int max_teams);

/* Tuning and test hook of asym_verify_xfam, process-wide for later calls:
 * general = 1 forces the general verifier pass (a and b gathered through
 * vmap, used anyway when a row is not made of 16-byte aligned vectors);
 * segs in 1..16 pins the staged pass's number of drafter segments per row.
 * 0 restores the automatic choice; other values give VWL_ERR_PARAM.  The
 * results do not depend on either choice except through the fp64 summation
 * order of the verifier's softmax partials. */
vwl_status vwl_set_xfam_override(int general, int segs);

/* Profiling hook: while `hip_event` (a hipEvent_t) is non-null, every
 * asym_verify / rapid_verify call records it on the call's stream right after
 * enqueuing the row kernel and before the kernels that follow it, so a caller
 * that records an event of its own just before the call can time the row
 * kernel alone with hipEventElapsedTime.  Process-wide; pass NULL to stop.
 * The event stays owned by the caller and must outlive the calls that use it.
 * A failed record is returned by that call as VWL_ERR_HIP. */
vwl_status vwl_set_phase_event(void *hip_event);

#ifdef __cplusplus
}
#endif
#endif /* VWL_H */
