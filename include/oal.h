/*
 * oal.h -- C ABI of liboal.so: causal OAL attention on AMD Instinct MI355X (gfx950).
 *
 * The method is Outlier-Aware Attention Linearization, from "Not All Dimensions
 * Are Equal: Outlier-Aware Attention Linearization with Grouped Quadratic
 * Kernels" (Sun, Wu, Wang, Hu; arXiv 2610.13674), cited below as [OAL].
 *
 *   kernel      kappa(q, k) = eps + s_bar^T L L^T s_bar,  s_bar = [1, s_1 .. s_G],
 *               s_g = sum_{r in group g} q_r k_r / sqrt(d_h)       ([OAL] §4.3, Eq. 7)
 *   output      y_i = sum_{j<=i} kappa(q_i, k_j) v_j / sum_{j<=i} kappa(q_i, k_j)
 *   evaluation  prefix states H0 = sum [v;1], H1_r = sum k_r [v;1],
 *               H2_rt = sum k_r k_t [v;1] and the readout of [OAL] Eq. 5-6,
 *               which equals the direct sum exactly ([OAL] App. D, Eq. 25).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, except the
 *     opaque oal_state, which the library owns from oal_state_alloc to
 *     oal_state_free.  Tensors are dense, row-major and contiguous.
 *   - Every call is enqueued on `stream` and returns without synchronising.
 *     Argument errors are detected on the host before anything is launched and
 *     return OAL_ERR_INVALID_ARG / OAL_ERR_UNSUPPORTED; a failed launch returns
 *     OAL_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation.  No C++ exception crosses this boundary.
 *   - oal_prefill and oal_decode_step never allocate device memory.
 *   - A state must not be used from two streams at once.
 *   - Supported shapes: d_h = d_v = 64; n_q_heads % n_kv_heads == 0, query head h
 *     reading KV head h / (n_q_heads / n_kv_heads) (grouped-query sharing of the
 *     KV states, [OAL] App. D); 1 <= G_h <= g_max <= 6 groups per query head.
 *   - After a failing call, oal_last_error() returns a message for this thread.
 */
#ifndef OAL_H
#define OAL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OAL_OK = 0,
  OAL_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent shapes           */
  OAL_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement (d_h!=64) */
  OAL_ERR_OUT_OF_MEMORY = 3, /* oal_state_alloc could not allocate                     */
  OAL_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed             */
} oal_status;

typedef enum { OAL_F32 = 0, OAL_BF16 = 1 } oal_dtype;

typedef struct oal_state oal_state; /* opaque; device memory owned by the library */

/* Layout of the coefficient buffer written by oal_expand_coeffs: one record of
 * OAL_COEF_WORDS 32-bit words per query head, record h at word h*OAL_COEF_WORDS.
 * Word offsets inside a record (float unless noted):                              */
#define OAL_COEF_A      0     /* a = eps + M_00                                       */
#define OAL_COEF_EPS    1     /* eps                                                  */
#define OAL_COEF_NG     2     /* int32: G_h                                           */
#define OAL_COEF_BP     16    /* [64]  b'_r = b_r / sqrt(d_h) = 2 M_{0,g(r)} / sqrt(d_h) */
#define OAL_COEF_GMAP   80    /* [64]  int32 g(r) in 1..G_h                           */
#define OAL_COEF_M      144   /* [7][7] M = L L^T (rows/cols >= G_h+1 are zero)        */
#define OAL_COEF_L      208   /* [7][7] L with the upper triangle zeroed              */
#define OAL_COEF_ELL    272   /* [7][64] ell_p[r] = L_{g(r),p} / sqrt(d_h)             */
#define OAL_COEF_CM     720   /* [64][64] C_rt / d_h = M_{g(r),g(t)} / d_h             */
#define OAL_COEF_CP     4816  /* [2080] c'_rt = m_rt C_rt / d_h over pairs r <= t in   */
                              /* row-major order; m = 1 if r == t else 2               */
#define OAL_COEF_MG     6896  /* [7][64] M_{gamma,g(t)} / d_h, gamma = 0..6            */
#define OAL_COEF_GPACK  7344  /* [8]   uint32: g(r) packed 4 bits per r, r = 8 i .. 8 i + 7
                                 in word i, low nibble first                          */
#define OAL_COEF_WORDS  7424

/* Bytes of the coefficient buffer for n_q_heads heads (d_h must be 64, g_max <= 6). */
size_t oal_coeffs_bytes(int n_q_heads, int d_h, int g_max);

/* Coefficient expansion, [OAL] §4.3 ("set M = L L^T; a = eps + M_00,
 * b_r = 2 M_{0,g(r)}, C_rt = M_{g(r),g(t)}") and Algorithm 1, causal-evaluation
 * step 5.  The expanded coefficients put the grouped kernel in the dimension-wise
 * form of [OAL] Eq. 3, which the readout of Eq. 6 evaluates.
 *   n_groups  device int32 [n_q_heads], G_h in 1..g_max
 *   group_map device int32 [n_q_heads][d_h], values 1..G_h (any partition, groups
 *             need not be contiguous); out-of-range labels are clamped to 1..G_h
 *   L         device float [n_q_heads][g_max+1][g_max+1]; only the lower triangle
 *             of the leading (G_h+1)x(G_h+1) block is read
 *   eps       > 0
 *   coeffs    device output, oal_coeffs_bytes() bytes, layout above            */
oal_status oal_expand_coeffs(int n_q_heads, int d_h, int g_max, const int32_t* n_groups,
                             const int32_t* group_map, const float* L, float eps,
                             void* coeffs, hipStream_t stream);

/* Dimension-specific coefficients: the general kernel of [OAL] §4.1, Eq. 3,
 *   kappa_dim(q, k) = a + sum_r b_r x_r + sum_{r,t} C_rt x_r x_t,  x_r = q_r k_r / sqrt(d_h),
 * with arbitrary a, b_r and C_rt per query head (no group structure; the grouped
 * kernel of oal_expand_coeffs is the special case a = eps + M_00,
 * b_r = 2 M_{0,g(r)}, C_rt = M_{g(r),g(t)}).
 *   a   device float [n_q_heads]
 *   b   device float [n_q_heads][d_h]
 *   C   device float [n_q_heads][d_h][d_h], row-major; only (C + C^T) / 2 enters
 *       kappa_dim, and the record stores that symmetric part
 *   coeffs  device output, oal_coeffs_bytes(n_q_heads, d_h, 1) bytes; the record
 *       has NG = 0, EPS = 0, A = a, BP, CM and CP filled and the group fields zero.
 * Such a record is read by oal_prefill_dim and oal_decode_step.  oal_prefill's
 * readouts evaluate grouped records only and return NaN outputs for it: the
 * record lives in device memory, and telling its kind on the host would take a
 * device-to-host copy and a synchronisation inside every prefill call (the
 * Python binding refuses, on the host, a buffer that oal_dim_coeffs filled).
 * kappa_dim must stay positive on the inputs for the outputs to be meaningful
 * (e.g. [[a, b^T/2], [b/2, C]] positive definite); nothing checks this. */
oal_status oal_dim_coeffs(int n_q_heads, int d_h, const float* a, const float* b, const float* C,
                          void* coeffs, hipStream_t stream);

/* Allocate a zeroed prefix state (H0 = H1 = H2 = 0, [OAL] Algorithm 1 step 5) for
 * batch x n_kv_heads sequences.  The state is fp32 and its device layout is private
 * (use oal_state_export to read it).  Size: batch*n_kv_heads*65*2176*4 bytes. */
oal_status oal_state_alloc(int batch, int n_kv_heads, int d_h, int d_v, oal_state** out);
/* Zero a state again (enqueued on stream). */
oal_status oal_state_reset(oal_state* state, hipStream_t stream);
/* Release a state (synchronises the device first).  NULL is accepted. */
oal_status oal_state_free(oal_state* state);
/* Copy src into dst (same shape), enqueued on stream. */
oal_status oal_state_copy(oal_state* dst, const oal_state* src, hipStream_t stream);
/* Bytes of device memory the state holds. */
size_t oal_state_bytes(const oal_state* state);
/* Number of tokens absorbed into the state so far (host-side counter kept by the
 * library: prefill adds seq_len, a decode step adds 1, reset sets 0). */
int64_t oal_state_tokens(const oal_state* state);
/* Export the state in canonical packed order ([OAL] Eq. 5; packed-symmetric rows,
 * App. D): dst is device float [batch][n_kv_heads][2145][65]; row 0 = H0,
 * rows 1..64 = H1_r, then one row per pair r <= t of H2 in row-major pair order;
 * column 64 is the all-ones (denominator) channel. */
oal_status oal_state_export(const oal_state* state, float* dst, hipStream_t stream);

/* Device workspace oal_prefill needs for these sizes: the per-chunk prefix states
 * read by the readout (with_output != 0) and the scratch of the state builder.
 * With with_output == 0 the size covers a call with y == NULL (state only).
 * chunk = 0 selects the default (128).  Returns 0 when no workspace is needed or
 * the arguments are unsupported. */
size_t oal_prefill_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                                   int d_h, int d_v, int chunk, oal_dtype in_dtype,
                                   int with_output);

/* Causal prefill over seq_len tokens: [OAL] Algorithm 1 steps 6-12 evaluated in
 * chunks (the paper's backend works on 128-token blocks, [OAL] App. E).
 *   q   [batch][n_q_heads][seq_len][d_h];  k, v [batch][n_kv_heads][seq_len][d_h/d_v]
 *       in in_dtype (fp32 or bf16).  q may be NULL when y is NULL.
 *   coeffs  written by oal_expand_coeffs for n_q_heads heads (a record of
 *           oal_dim_coeffs gives NaN outputs here: use oal_prefill_dim)
 *   chunk   0 (= 128), 64, 128 or 256
 *   state   NULL: the sequence starts empty.  Otherwise the prefix it holds is
 *           read first and, on return, it holds the state after the seq_len
 *           tokens have been appended.
 *   y       [batch][n_q_heads][seq_len][d_v] in out_dtype, or NULL to only
 *           advance the state (then state must not be NULL).
 *   workspace  >= oal_prefill_workspace_bytes(..., with_output = y != NULL) bytes of
 *           device memory, 256-byte aligned; may be NULL when that size is 0.
 * seq_len == 0 is a valid no-op. */
oal_status oal_prefill(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h, int d_v,
                       oal_dtype in_dtype, const void* q, const void* k, const void* v,
                       const void* coeffs, int chunk, oal_state* state, void* y,
                       oal_dtype out_dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* oal_prefill for a sequence that starts empty ([OAL] Algorithm 1 step 5, then
 * steps 6-12), into state: the state's contents on entry are ignored (taken as
 * zero) and replaced by the state after the seq_len tokens; its token count
 * becomes seq_len.  With bf16 inputs the state is only written, never read or
 * cleared first (oal_state_reset followed by oal_prefill clears it and reads the
 * zeros back).  state must not be NULL (OAL_ERR_INVALID_ARG); seq_len == 0 leaves
 * it zero.  Other arguments and errors as oal_prefill. */
oal_status oal_prefill_fresh(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h, int d_v,
                             oal_dtype in_dtype, const void* q, const void* k, const void* v,
                             const void* coeffs, int chunk, oal_state* state, void* y,
                             oal_dtype out_dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ---- allocation-free prefill ----------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): oal_prefill with the
 * same arguments except the workspace, which comes from a static device array of
 * OAL_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds on every GPU it runs
 * on until the process ends.  The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine); its first call on a device looks the array's
 * address up.  Sizes whose workspace (oal_prefill_workspace_bytes) exceeds the
 * array return OAL_ERR_UNSUPPORTED before any HIP call; other errors are those of
 * oal_prefill.  Every call on a GPU shares that GPU's array, so calls that overlap
 * on one GPU (concurrent streams, or host threads) race and must be serialised by
 * the caller; nothing in the array needs to start at zero. */
#define OAL_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
size_t oal_prefill_noalloc_scratch_bytes(void);
oal_status oal_prefill_noalloc(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                               int d_v, oal_dtype in_dtype, const void* q, const void* k,
                               const void* v, const void* coeffs, int chunk, oal_state* state,
                               void* y, oal_dtype out_dtype, hipStream_t stream);

/* Device workspace oal_prefill_dim needs (same conventions as
 * oal_prefill_workspace_bytes; the size does not depend on the input dtype). */
size_t oal_prefill_dim_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                                       int d_h, int d_v, int chunk, int with_output);

/* Causal prefill for any coefficient record, including the dimension-specific ones
 * of oal_dim_coeffs: the same chunked evaluation of [OAL] Algorithm 1 (Eq. 5-6)
 * with the same arguments, state semantics and errors as oal_prefill, but every
 * kernel value inside a chunk is a + sum_r b'_r p_r + sum_{r<=t} c'_rt p_r p_t
 * (p_r = q_r k_r) from the record's expanded coefficients.  It runs on the vector
 * ALUs in fp32 for fp32 and bf16 inputs alike (slower than oal_prefill's matrix
 * core path for grouped records); workspace >= oal_prefill_dim_workspace_bytes(). */
oal_status oal_prefill_dim(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                           int d_v, oal_dtype in_dtype, const void* q, const void* k,
                           const void* v, const void* coeffs, int chunk, oal_state* state,
                           void* y, oal_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* One decode step: [OAL] Algorithm 1 loop body (steps 7-10) for one new token per
 * sequence: u = [v; 1]; H0 += u; H1_r += k_r u; H2_rt += k_r k_t u; then the
 * readout of Eq. 6 for every query head of the KV group (inclusive of the new
 * token).  q [batch][n_q_heads][d_h], k [batch][n_kv_heads][d_h],
 * v [batch][n_kv_heads][d_v] in in_dtype; y [batch][n_q_heads][d_v] in out_dtype;
 * state in/out.  coeffs may come from oal_expand_coeffs or oal_dim_coeffs (the
 * readout uses only the expanded a, b', c'). */
oal_status oal_decode_step(int batch, int n_q_heads, int n_kv_heads, int d_h, int d_v,
                           oal_dtype in_dtype, const void* q, const void* k, const void* v,
                           const void* coeffs, oal_state* state, void* y, oal_dtype out_dtype,
                           hipStream_t stream);

/* Device workspace oal_prefill_backward needs: the per-chunk prefix and suffix
 * states (2 x batch x n_kv_heads x ceil(seq_len/chunk) x 565,760 B), the rows
 * g_i and alpha_ij of every chunk, and the per-chunk coefficient sums.  chunk 0
 * selects 128; returns 0 for unsupported arguments or seq_len == 0. */
size_t oal_prefill_backward_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                                            int d_h, int d_v, int chunk);

/* Backward of a prefill that starts from an empty state (oal_prefill with a
 * fresh state, or oal_prefill_dim): for the loss sum_i dy_i . y_i, the gradients
 * with respect to q, k, v and the kernel's dimension-wise coefficients.  It
 * differentiates the causal sum of [OAL] Eq. 5-7 (exact, like the forward):
 * with g_i = [dy_i / den_i ; -(dy_i . y_i) / den_i] and alpha_ij = g_i . [v_j; 1],
 *   dv_j = sum_{i>=j} kappa_ij dy_i / den_i,   dq_i = sum_{j<=i} alpha_ij d kappa_ij / d q_i,
 *   dk_j = sum_{i>=j} alpha_ij d kappa_ij / d k_j,  and for [OAL] Eq. 3's a, b_r, C_rt:
 *   da = sum alpha_ij, db_r = sum alpha_ij x_r, dC_rt = sum alpha_ij x_r x_t
 * (x = q_i o k_j / sqrt(d_h)); sums over i include every query head that shares
 * the KV head.  Linear in seq_len: the parts outside a row's chunk go through
 * prefix and suffix states, the chunk itself pair by pair; fp32 on the vector
 * ALUs.
 *   q, k, v, coeffs as for oal_prefill (fp32 or bf16 inputs; any record kind)
 *   dy      device float [batch][n_q_heads][seq_len][d_v]
 *   chunk   0 (= 128), 64 or 128
 *   dq      device float out [batch][n_q_heads][seq_len][d_h]
 *   dk, dv  device float out [batch][n_kv_heads][seq_len][d_h / d_v]
 *   da, db, dC  device float out [n_q_heads], [n_q_heads][d_h], [n_q_heads][d_h][d_h]
 *           (dC symmetric, summed over the batch), or all three NULL to skip them
 *   workspace  >= oal_prefill_backward_workspace_bytes() bytes, 256-byte aligned
 * seq_len == 0 writes zero coefficient gradients (when requested) and nothing
 * else.  Allocates nothing. */
oal_status oal_prefill_backward(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                                int d_v, oal_dtype in_dtype, const void* q, const void* k,
                                const void* v, const void* coeffs, const float* dy, int chunk,
                                float* dq, float* dk, float* dv, float* da, float* db, float* dC,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gradient with respect to L of the grouped kernel ([OAL] §4.3, M = L L^T,
 * a = eps + M_00, b_r = 2 M_{0,g(r)}, C_rt = M_{g(r),g(t)}) from the gradients
 * (da, db, dC) with respect to the dimension-wise coefficients: dM_00 = da,
 * dM_{0,g} = dM_{g,0} = sum_{r in g} db_r, dM_{g,h} = sum_{r in g, t in h} dC_rt,
 * dL = (dM + dM^T) L.  Same n_groups / group_map / L conventions (and clamping)
 * as oal_expand_coeffs; dL [n_q_heads][g_max+1][g_max+1] holds the lower
 * triangle of the leading (G_h+1) block and zero elsewhere. */
oal_status oal_coeffs_backward(int n_q_heads, int d_h, int g_max, const int32_t* n_groups,
                               const int32_t* group_map, const float* L, const float* da,
                               const float* db, const float* dC, float* dL, hipStream_t stream);

/* ---- dimension grouping ([OAL] §3.1 Eq. 2; App. B Eq. 16-19) -------------- */

/* Contribution scores of Eq. 2: for prompt p and query head h,
 *   chi_prompt[p][h][r] = mean over the causal pairs j <= i of the prompt of
 *                         |q_ir k_jr| / sqrt(d_h)     (k from the head's KV head),
 * and chi[h][r] = the equal-weight mean over the prompts (chi may be NULL).
 *   q [n_q_heads][total_tokens][d_h], k [n_kv_heads][total_tokens][d_h] (fp32 or
 *   bf16): the prompts concatenated; prompt p is tokens offsets[p] ..
 *   offsets[p+1]-1 (offsets: device int32 [n_prompts+1], non-decreasing; values
 *   are clamped into 0..total_tokens, an empty prompt scores 0).  Linear in the
 *   tokens (the pair sum is sum_i |q_ir| sum_{j<=i} |k_jr|), double accumulation. */
oal_status oal_contribution_scores(int n_q_heads, int n_kv_heads, int n_prompts, int total_tokens,
                                  int d_h, oal_dtype in_dtype, const void* q, const void* k,
                                  const int32_t* offsets, float* chi_prompt, float* chi,
                                  hipStream_t stream);

/* Bootstrap tail-cut grouping of App. B from the per-prompt scores: per head the
 * dimensions are ordered by increasing chi (stable), candidate cuts are
 * k = max(1, d_h - ceil(alpha d_h)) .. d_h - 1, rho_k = chi_{pi_{k+1}} /
 * max(chi_{pi_k}, eps) (Eq. 16), S_k = the fraction of the n_boot replicates with
 * min over the upper side >= tau max(max over the lower side, eps) of the
 * replicate's mean scores in that fixed order (Eq. 17-18); cuts with rho_k >= tau
 * and S_k >= gamma are kept and, below g_min groups, unused candidates are added
 * by descending (S_k, rho_k) (ties: smaller k first); labels per Eq. 19 (group 1
 * = the low-contribution bulk).  The pages use alpha 0.25 / 0.5, tau 1.5,
 * gamma 0.9 / 0.5, g_min 2, 1000 replicates of 40 prompts.
 *   chi_prompt [n_prompts][n_q_heads][d_h] (from oal_contribution_scores),
 *   n_prompts <= 256; boot_idx: device int32 [n_boot][n_prompts], the prompt
 *   indices of every replicate, drawn with replacement by the caller (clamped to
 *   0..n_prompts-1);
 *   group_map [n_q_heads][d_h] (labels 1..G), n_groups [n_q_heads] int32 out;
 *   support, gap [n_q_heads][d_h] float out (S_k, rho_k at the candidate k, 0
 *   elsewhere), or NULL.  G is not capped: oal_expand_coeffs accepts G <= 6.
 * Decisions are taken in double precision; deterministic. */
oal_status oal_bootstrap_grouping(int n_q_heads, int n_prompts, int d_h, const float* chi_prompt,
                                  int n_boot, const int32_t* boot_idx, float alpha, float tau,
                                  float gamma, int g_min, float eps, int32_t* group_map,
                                  int32_t* n_groups, float* support, float* gap,
                                  hipStream_t stream);

/* ---- calibration of L by output matching ([OAL] App. B, Eq. 20) ------------ */

/* Workspace of oal_calib_grad for n_pos sampled positions (0 if invalid). */
size_t oal_calib_workspace_bytes(int n_q_heads, int n_pos);

/* Loss and gradient of one calibration update for one sequence: per query head
 * h, loss_h = (1 / (2 n_pos)) sum_{i in positions} ||y_i - y_ref_i||^2 (Eq. 20
 * restricted to the sampled causal positions) with y the OAL output of the
 * grouped kernel (L, g, eps as for oal_expand_coeffs), and dL_h its gradient with
 * respect to L (lower triangle of the leading (G_h+1) block; zero elsewhere).
 * The sampled rows are evaluated directly (each row's causal sum over its keys),
 * not through a prefill.
 *   q [n_q_heads][seq_len][d_h], k, v [n_kv_heads][seq_len][d_h / d_v]: one
 *   sequence, fp32 or bf16; y_ref [n_q_heads][seq_len][d_v] fp32 (the softmax
 *   output, e.g. from oal_softmax_attention); positions: device int32 [n_pos],
 *   distinct, in 0..seq_len-1 (a position outside contributes nothing);
 *   dL [n_q_heads][g_max+1][g_max+1], loss [n_q_heads] device fp32 out;
 *   workspace >= oal_calib_workspace_bytes(), 256-byte aligned.  Deterministic. */
oal_status oal_calib_grad(int n_q_heads, int n_kv_heads, int seq_len, int d_h, int d_v,
                          oal_dtype in_dtype, const void* q, const void* k, const void* v,
                          const float* y_ref, const int32_t* positions, int n_pos, int g_max,
                          const int32_t* n_groups, const int32_t* group_map, const float* L,
                          float eps, float* dL, float* loss, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* One Adam update of L in place (Kingma and Ba, Algorithm 1; the calibration of
 * [OAL] App. B uses Adam at lr 0.02 with the gradient norm clipped at 10): per
 * head, the gradient dL is scaled to Euclidean norm <= clip_norm over the
 * parameter entries (lower triangle of the leading (G_h+1) block), then
 * m = beta1 m + (1 - beta1) g, v = beta2 v + (1 - beta2) g^2 and
 * L -= lr (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps) on those
 * entries; other entries are untouched.  L, dL, m, v: device fp32
 * [n_q_heads][g_max+1][g_max+1] (m, v start at zero); step is 1-based. */
oal_status oal_adam_step(int n_q_heads, int g_max, const int32_t* n_groups, float* L,
                         const float* dL, float* m, float* v, int step, float lr, float beta1,
                         float beta2, float eps, float clip_norm, hipStream_t stream);

/* The learned global quadratic embedded into the grouped form ([OAL] App. D,
 * Eq. 23: eps + [1 s] M_g [1 s]^T with s = q . k / sqrt(d_h); M_00 = m00,
 * M_{0g} = M_{g0} = m01, M_{gh} = m11 for every group), the start of a grouped
 * calibration from a calibrated global kernel.  L_global: device fp32
 * [n_q_heads][g_ld][g_ld], of which the lower triangle of the leading 2 x 2 block
 * is M_g's factor (a G = 1 calibration's L, g_ld = its g_max + 1); L: device fp32
 * out [n_q_heads][g_max+1][g_max+1], rows 1..G_h = (l10, l11, 0, ..), row 0 =
 * (l00, 0, ..), l00 = sqrt(m00), l10 = m01 / l00, l11 = sqrt(max(m11 - l10^2, 0)). */
oal_status oal_embed_global(int n_q_heads, int g_max, const int32_t* n_groups, int g_ld,
                            const float* L_global, float* L, hipStream_t stream);

/* Per query head, the mean over batch, positions and channels of (y - y_ref)^2
 * for y, y_ref [batch][n_q_heads][seq_len][d_v] fp32: the validation error of the
 * calibration (and the MSE of [OAL] App. C, Eq. 21, per head). */
oal_status oal_output_mse(int batch, int n_q_heads, int seq_len, int d_v, const float* y,
                          const float* y_ref, float* mse, hipStream_t stream);

/* Exact causal softmax attention, the reference OAL approximates ([OAL] §3:
 * y_i = sum_{j<=i} exp(s_ij) v_j / sum_{j<=i} exp(s_ij), s_ij = q_i . k_j / sqrt(d_h),
 * query head h reading KV head h / (n_q_heads / n_kv_heads)); used for the
 * frozen-attention fidelity metrics of [OAL] App. C (Eqs. 21-22).
 *   q [batch][n_q_heads][seq_len][d_h], k, v [batch][n_kv_heads][seq_len][d_h/d_v]
 *   in bf16 (in_dtype must be OAL_BF16: other types return OAL_ERR_UNSUPPORTED);
 *   y [batch][n_q_heads][seq_len][d_v] in out_dtype.  d_h = d_v = 64.
 * seq_len == 0 is a valid no-op.  Allocates nothing. */
oal_status oal_softmax_attention(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                                 int d_v, oal_dtype in_dtype, const void* q, const void* k,
                                 const void* v, void* y, oal_dtype out_dtype, hipStream_t stream);

/* Per-kernel timing (a tracing aid, off by default).  While enabled, the library
 * records a pair of HIP events on the launch stream around every kernel it
 * launches.  oal_profile_query waits for the pending events of the named kernel
 * ("k_decode", "k_readout_vec", ...; NULL = all kernels) and returns their total
 * duration and launch count since the last reset.  oal_profile_filter restricts
 * the events to the kernel of that name (NULL: every kernel again), so that one
 * kernel can be timed inside a sequence of launches without widening the gaps
 * between the others.  Host-global, not thread-safe against concurrent launches
 * from several threads. */
oal_status oal_profile_enable(int enable);
oal_status oal_profile_filter(const char* kernel);
oal_status oal_profile_reset(void);
oal_status oal_profile_query(const char* kernel, double* total_ms, int64_t* launches);

const char* oal_status_string(oal_status status);
const char* oal_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OAL_H */
