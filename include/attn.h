/*
 * attn.h - C ABI of the MI355X (gfx950) causal RoPE attention library, libattn.so.
 *
 * The operation (forward and backward) is causal self-attention with rotary
 * position embedding applied to the query and key projections, as the pages
 * describe it: a prediction may depend only on earlier positions, and RoPE is
 * applied to the projections to encode relative positions ("Tiny Hackable CUDA",
 * section 3, causal attention paragraph); the engine uses a hand-written
 * FlashAttention with RoPE, and its analytic gradients (RoPE included) are
 * checked against centred differences in double precision ("Show HN: NanoEuler",
 * paragraph 2). Head shapes follow the GPT-2-small specification of 12 heads and
 * width 768 (NanoEuler article on techinfos.ro, "Arhitectură și tehnologii
 * folosite"), so D = 64; D = 128 is also supported.
 *
 * Definitions used by every entry point (readings where the pages are silent):
 *   theta_i   = base^(-2i/D), i = 0 .. D/2-1, D = head dimension
 *   R_t x     rotates each adjacent pair (x[2i], x[2i+1]) by the angle t*theta_i:
 *             (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos); positions start at 0
 *   S[t,u]    = (1/sqrt(D)) <R_t q_t, R_u k_u>, kept for u <= t, -inf for u > t
 *   P         = row softmax of S;  o_t = sum_u P[t,u] v_u   (v is not rotated)
 *   lse_t     = natural log of sum_{u<=t} exp(S[t,u])
 *   backward  = gradients of L = sum(o * dO) with respect to the un-rotated
 *               q, k and v (the RoPE backward is part of the operation).
 *
 * Conventions common to all calls:
 *   - Every tensor pointer is a DEVICE pointer, 16-byte aligned; tensors are
 *     contiguous row-major [B, H, T, D] with D innermost (the *_packed entry
 *     points take the model-native layouts they describe instead); lse and the
 *     backward workspace hold [B, H, T] fp32; cos/sin tables are [T, D/2] fp32.
 *   - dtype is ATTN_BF16 (bf16 storage, fp32 accumulation; rotated q/k and dS
 *     are carried in fp16 inside the kernels), ATTN_F16 (the same kernels with
 *     fp16 storage, so P, V and dO are fp16 operands too) or ATTN_F32 (fp32
 *     everywhere); it applies to q, k, v, o, dO, dq, dk and dv. "The 16-bit
 *     path" below means ATTN_BF16 and ATTN_F16.
 *   - D in {64, 128}; T >= 1; B*H >= 1; B*H*T*D < 2^31. The scale is fixed at
 *     1/sqrt(D). There is no dropout, bias, padding mask or grouped-query sharing.
 *   - The caller owns all memory. The library never allocates, frees or
 *     synchronises; work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and the call returns before the GPU finishes.
 *   - No output may overlap an input or another output (checked on the byte
 *     ranges each call touches); outputs are overwritten, not accumulated.
 *   - Every failure is reported by the return value. Arguments are validated
 *     before anything is launched; nothing aborts and no exception crosses the
 *     ABI. ATTN_ERR_HIP means a launch failed; attn_last_hip_error() then gives
 *     the hipError_t value (per calling thread).
 */
#ifndef CAUSAL_ROPE_ATTN_H
#define CAUSAL_ROPE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_dtype { ATTN_BF16 = 0, ATTN_F32 = 1, ATTN_F16 = 2 };

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,       /* a required pointer is NULL                         */
    ATTN_ERR_SHAPE = 2,      /* B, H, T or D outside the supported range           */
    ATTN_ERR_DTYPE = 3,      /* unknown dtype                                      */
    ATTN_ERR_ALIGN = 4,      /* a tensor pointer is not 16-byte aligned            */
    ATTN_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required         */
    ATTN_ERR_HIP = 6,        /* a HIP launch failed (see attn_last_hip_error)      */
    ATTN_ERR_ALIAS = 7,      /* an output's bytes overlap an input's or an output's */
    ATTN_ERR_VALUE = 8,      /* a scalar argument (e.g. the RoPE base) is invalid   */
    ATTN_ERR_SAVED = 9,      /* the saved rotated q/k buffer is too small           */
    ATTN_ERR_SCRATCH = 10    /* too large for the static scratch of a no-alloc call */
};

/*
 * attn_rope_tables - fill the RoPE tables cos_tab[t*(D/2) + i] = cos(t*theta_i)
 * and sin_tab[t*(D/2) + i] = sin(t*theta_i) for t < T, i < D/2.
 * The angle t*theta_i and its cosine/sine are evaluated in double precision on
 * the GPU and rounded once to fp32. Position encoding per "Tiny Hackable CUDA",
 * section 3 (RoPE on the projections, relative positions); base must be > 1
 * (10000 for the model the pages describe). D must be even, 2 <= D <= 1024.
 * Tables depend only on (T, D, base): build once, reuse for every call.
 */
int attn_rope_tables(float* cos_tab, float* sin_tab, int T, int D, double base,
                     void* stream);

/*
 * attn_fwd - forward pass. Reads the pre-RoPE q, k and v, and writes
 * o = softmax(S) v and lse (natural log-sum-exp of each row's scaled, masked
 * scores; kept for the backward). FlashAttention-style: the T x T score matrix
 * is never stored ("Show HN: NanoEuler", paragraph 2). RoPE is applied on load
 * ("Tiny Hackable CUDA", section 3: RoPE on the query and key projections): on
 * the 16-bit path each query row is rotated (and multiplied by log2(e)/sqrt(D))
 * in fp32 once, in registers, and every key tile is rotated in fp32 on its way
 * into on-chip memory; both are rounded once to fp16 for the score products.
 *   q, k, v   [B,H,T,D] dtype, inputs (q, k not rotated)
 *   cos_tab, sin_tab  [T,D/2] fp32 from attn_rope_tables (or equal values)
 *   o         [B,H,T,D] dtype, output
 *   lse       [B,H,T] fp32, output
 */
int attn_fwd(const void* q, const void* k, const void* v,
             const float* cos_tab, const float* sin_tab,
             void* o, float* lse,
             int B, int H, int T, int D, int dtype, void* stream);

/*
 * attn_saved_bytes - size of the "saved" buffer of attn_fwd_save and
 * attn_bwd_saved: for the 16-bit path the rotated q times log2(e)/sqrt(D),
 * then the rotated k, each [B,H,T,D] fp16 (4*B*H*T*D bytes, rounded up to 256);
 * 0 for ATTN_F32, whose kernels rotate on load. Returns 0 for arguments the
 * other calls would reject.
 */
size_t attn_saved_bytes(int B, int H, int T, int D, int dtype);

/*
 * attn_fwd_save - attn_fwd that also hands the rotated q and k to the
 * backward, for a training step: the rotation pass (attn_rotate_qk) writes
 * c * R_t q_t (c = log2(e)/sqrt(D)) and R_t k_t, fp16, into `saved`
 * ([2][B,H,T,D] fp16, at least attn_saved_bytes() bytes), and the forward
 * (attn_fwd_rotated) reads them from there; o and lse are bitwise those of
 * attn_fwd (both form the same rotated values and feed them to the same
 * arithmetic). Pass the buffer to attn_bwd_saved with the same q and k, and
 * the backward skips their rotation. The backward needs the rotated values
 * anyway, so one pass that serves both is cheaper than the on-load rotation
 * writing them out. ATTN_F32: `saved` is ignored and may be NULL.
 */
int attn_fwd_save(const void* q, const void* k, const void* v,
                  const float* cos_tab, const float* sin_tab,
                  void* o, float* lse, void* saved, size_t saved_bytes,
                  int B, int H, int T, int D, int dtype, void* stream);

/*
 * attn_bwd_workspace_bytes - device workspace of attn_bwd, rounded up to 256:
 * the per-row entries of the pre-pass, that is -lse_t * log2 e then -delta_t
 * for every row on the 16-bit path (8*B*H*T bytes, rounded up to 256), or
 * delta_t alone for ATTN_F32 (4*B*H*T), where delta_t = sum_d dO[t,d] o[t,d];
 * then, on the 16-bit path, room for the rotated q and k (attn_saved_bytes()).
 * attn_bwd_saved, attn_bwd_prep and attn_bwd_grads use only the per-row part,
 * and accept a workspace of that size. Returns 0 for arguments attn_bwd would
 * reject.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int T, int D, int dtype);

/*
 * attn_bwd - backward pass: the analytic gradients of L = sum(o * dO) with
 * respect to the pre-RoPE q, k and v ("Show HN: NanoEuler", paragraph 2: every
 * analytic gradient, RoPE's included, is checked against centred differences).
 * Recompute-based: P is rebuilt from q, k and lse; nothing of size T x T is
 * stored. Two launches on `stream`: the pre-pass (attn_bwd_prep), which on the
 * 16-bit path also rotates this call's q and k into the workspace (bitwise the
 * values attn_fwd's on-load rotation forms), then the gradient kernel
 * (attn_bwd_grads) reading them there.
 *   q, k, v, o, dO  [B,H,T,D] dtype, inputs (o and lse from attn_fwd)
 *   lse             [B,H,T] fp32, input
 *   dq, dk, dv      [B,H,T,D] dtype, outputs (overwritten)
 *   workspace       device buffer of at least attn_bwd_workspace_bytes()
 * The 16-bit path rounds dS = P (dP - delta) to fp16 for the dq/dk products, so
 * |dS| must stay below 65504 (true whenever |dO_t|*|v_u| < 32752 in L2 norm).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dO, const float* lse,
             const float* cos_tab, const float* sin_tab,
             void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int B, int H, int T, int D, int dtype, void* stream);

/*
 * attn_bwd_saved - attn_bwd without the rotation pass: the 16-bit kernels take
 * the rotated q and k from `saved`, which must be what attn_fwd_save (or
 * attn_rotate_qk) wrote for these q and k - a buffer left over from other
 * inputs gives wrong gradients. q and k are not read on the 16-bit path (they
 * may be NULL there); ATTN_F32 reads q and k and ignores `saved`. The workspace
 * needs only the per-row part of attn_bwd_workspace_bytes(). Otherwise as
 * attn_bwd.
 */
int attn_bwd_saved(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse,
                   const float* cos_tab, const float* sin_tab,
                   const void* saved, size_t saved_bytes,
                   void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int T, int D, int dtype, void* stream);

/*
 * The stages, for callers that schedule them separately (and to time each):
 *
 * attn_rotate_qk - RoPE once ("Tiny Hackable CUDA", section 3): writes
 * c * R_t q_t, c = log2(e)/sqrt(D), then R_t k_t into `saved` ([2][B,H,T,D]
 * fp16), each value rotated (and scaled) in fp32 and rounded once to fp16 -
 * bitwise the values the on-load rotation of attn_fwd forms. The factor c makes a score product
 * come out as S*log2(e), ready for base-2 exponentials. fp16's 11-bit
 * significand keeps the score products accurate where the softmax is sharp,
 * and bounds |c R_t q_t| and |R_t k_t| by 65504. ATTN_F32: does nothing.
 */
int attn_rotate_qk(const void* q, const void* k, const float* cos_tab, const float* sin_tab,
                   void* saved, size_t saved_bytes, int B, int H, int T, int D, int dtype,
                   void* stream);

/*
 * attn_fwd_rotated - the forward from rotated q and k already in `saved`
 * (attn_rotate_qk) and from v: the same o and lse as attn_fwd. 16-bit path
 * only (ATTN_F32 gets ATTN_ERR_DTYPE).
 */
int attn_fwd_rotated(const void* saved, size_t saved_bytes, const void* v, void* o, float* lse,
                     int B, int H, int T, int D, int dtype, void* stream);

/*
 * attn_bwd_prep - the per-row pre-pass of the recompute-based backward:
 * delta_t = sum_d dO[t,d] o[t,d] (equal to sum_u P[t,u] dP[t,u], the softmax
 * Jacobian term) and, for the 16-bit path, lse_t * log2 e, written to the
 * per-row part of the workspace (see attn_bwd_workspace_bytes). o, dO
 * [B,H,T,D] dtype and lse [B,H,T] fp32 are inputs. With q and k (16-bit path;
 * NULL for both skips it) the same pass also writes their rotation - the values
 * attn_rotate_qk writes - into the rest of the workspace, which must then hold
 * attn_bwd_workspace_bytes(); cos_tab and sin_tab are read only then.
 */
int attn_bwd_prep(const void* q, const void* k, const void* o, const void* dO, const float* lse,
                  const float* cos_tab, const float* sin_tab,
                  void* workspace, size_t workspace_bytes,
                  int B, int H, int T, int D, int dtype, void* stream);

/*
 * attn_bwd_grads - writes dq, dk (w.r.t. the pre-RoPE q and k) and dv. Reads
 * the workspace entries of attn_bwd_prep, which must have been enqueued before
 * it on the same stream (or completed) for the same o, dO and lse. The 16-bit
 * path takes the rotated q and k from `saved` (as attn_bwd_saved) or, when
 * `saved` is NULL, from the workspace, where attn_bwd_prep wrote them (then the
 * workspace holds attn_bwd_workspace_bytes()); q and k are not read there and
 * may be NULL. ATTN_F32 reads q and k. dq and dk/dv come from one launch.
 * attn_bwd is attn_bwd_prep with q, k followed by this call with saved NULL.
 */
int attn_bwd_grads(const void* q, const void* k, const void* v,
                   const void* dO, const float* lse,
                   const float* cos_tab, const float* sin_tab,
                   const void* saved, size_t saved_bytes,
                   void* dq, void* dk, void* dv,
                   const void* workspace, size_t workspace_bytes,
                   int B, int H, int T, int D, int dtype, void* stream);

/*
 * Model-native layouts. In the model the pages describe, attention sits between
 * two projections: the query, key and value projections (RoPE is applied to the
 * first two) feed it, and its output feeds the output projection ("Tiny Hackable
 * CUDA", section 3, causal attention paragraph; the engine runs those
 * projections as cuBLAS matrix products, "Show HN: NanoEuler", paragraph 2). A
 * fused QKV projection of a [B*T, C] activation, C = H*D, produces one
 * [B, T, 3, H, D] tensor (q, k, v slots of each token's row), and the output
 * projection consumes o as [B, T, H*D]. These two entry points read and write
 * those layouts directly, so no permute copies are needed on either side; the
 * arithmetic, kernels and results are those of attn_fwd / attn_bwd (bitwise
 * equal for the same values).
 *
 * 16-bit path only (ATTN_BF16, ATTN_F16; ATTN_F32 gets ATTN_ERR_DTYPE); the
 * packed tensor must hold fewer than 2^31 elements (3*B*H*T*D < 2^31) and a
 * token row of it fewer than 2^23 (3*H*D < 2^23); otherwise ATTN_ERR_SHAPE.
 * lse, the saved buffer and the workspace keep their [B, H, T] / [2][B, H, T, D]
 * layouts and sizes (attn_saved_bytes, attn_bwd_workspace_bytes).
 */

/*
 * attn_fwd_packed - forward pass from the packed projection output.
 *   qkv       [B, T, 3, H, D] dtype, input: qkv[b,t,0,h,:] is q of head h at
 *             position t, [.., 1, ..] is k, [.., 2, ..] is v (pre-RoPE)
 *   cos_tab, sin_tab  [T, D/2] fp32 from attn_rope_tables
 *   o         [B, T, H, D] dtype (= [B, T, H*D]), output
 *   lse       [B, H, T] fp32, output
 *   saved     NULL, or a device buffer of attn_saved_bytes() that receives the
 *             rotated q and k (as attn_fwd_save)
 * Without saved: one launch of the forward kernel with RoPE on load (as
 * attn_fwd); with it: the rotation pass, then the forward from its output (as
 * attn_fwd_save).
 */
int attn_fwd_packed(const void* qkv, const float* cos_tab, const float* sin_tab,
                    void* o, float* lse, void* saved, size_t saved_bytes,
                    int B, int H, int T, int D, int dtype, void* stream);

/*
 * attn_bwd_packed - backward pass in the same layouts: gradients of
 * L = sum(o * dO) with respect to the pre-RoPE q, k and v, written into one
 * [B, T, 3, H, D] tensor, ready for the QKV projection's backward.
 *   qkv       [B, T, 3, H, D] dtype, the forward's input (v is read from it)
 *   o, dO     [B, T, H, D] dtype, inputs (o and lse from attn_fwd_packed)
 *   lse       [B, H, T] fp32, input
 *   saved     the buffer attn_fwd_packed filled for this qkv, or NULL: then
 *             the rotated q and k are formed again, in the workspace
 *   dqkv      [B, T, 3, H, D] dtype, output (overwritten): dq, dk, dv slots
 *   workspace device buffer of at least attn_bwd_workspace_bytes() (the
 *             per-row part suffices when saved is given)
 * Enqueues the pre-pass (which, without saved, also rotates q and k into the
 * workspace) and the gradient kernel; the |dS| bound of attn_bwd applies.
 */
int attn_bwd_packed(const void* qkv, const void* o, const void* dO, const float* lse,
                    const float* cos_tab, const float* sin_tab,
                    const void* saved, size_t saved_bytes, void* dqkv,
                    void* workspace, size_t workspace_bytes,
                    int B, int H, int T, int D, int dtype, void* stream);

/*
 * Decode over a key/value cache. The pages' model generates text one token at
 * a time, and the token at position pos may attend only to positions
 * 0 .. pos ("Tiny Hackable CUDA", section 3, causal attention paragraph). A
 * generation step therefore scores one new query against the keys of all
 * earlier tokens; keeping those keys (already rotated by their own positions)
 * and values in a cache makes a step cost O(pos) instead of a full forward.
 * The result of attn_decode at position pos is, by definition, row pos of
 * attn_fwd over positions 0 .. pos.
 *
 * 16-bit path only (ATTN_BF16, ATTN_F16; ATTN_F32 gets ATTN_ERR_DTYPE). Every
 * sequence of the batch is at the same position. The RoPE tables passed to
 * these calls must hold at least Tmax rows (attn_rope_tables with T = Tmax).
 *
 * Cache layout (one device buffer of attn_kv_cache_bytes()): the rotated keys
 * R_u k_u as fp16 [B, H, Tmax, D] (rotated in fp32, rounded once; the same
 * values the forward's rotation pass produces for k), then the values as
 * [B, H, Tmax, D] dtype. Rows at positions not yet appended are not read.
 */

/* attn_kv_cache_bytes - 4*B*H*Tmax*D rounded up to 256 (0 for rejected arguments). */
size_t attn_kv_cache_bytes(int B, int H, int Tmax, int D, int dtype);

/*
 * attn_kv_append - write n tokens into the cache at positions pos0 .. pos0+n-1
 * (n = 1 for a generation step, n = prompt length for a prefill).
 *   k, v      [B, H, n, D] dtype, the pre-RoPE key and value projections of
 *             those tokens
 *   cache     the cache buffer (cache_bytes >= attn_kv_cache_bytes(), else
 *             ATTN_ERR_WORKSPACE); 0 <= pos0, pos0 + n <= Tmax (ATTN_ERR_SHAPE)
 */
int attn_kv_append(const void* k, const void* v, const float* cos_tab, const float* sin_tab,
                   void* cache, size_t cache_bytes, int pos0, int n,
                   int B, int H, int Tmax, int D, int dtype, void* stream);

/*
 * attn_decode_workspace_bytes - partial results of attn_decode for any
 * pos < Tmax: B*H*ceil(Tmax/64)*(D+4) fp32, rounded up to 256.
 */
size_t attn_decode_workspace_bytes(int B, int H, int Tmax, int D, int dtype);

/*
 * attn_decode - one generation step at position pos (0 <= pos < Tmax, else
 * ATTN_ERR_SHAPE), over cache rows 0 .. pos (appended before, on this stream
 * or completed).
 *   q         [B, H, D] dtype, the pre-RoPE query of the new token (rotated
 *             here by position pos)
 *   o         [B, H, D] dtype, output: softmax over u <= pos of
 *             (1/sqrt(D)) <R_pos q, R_u k_u>, applied to v
 *   lse       [B, H] fp32, output: natural log-sum-exp of those scores
 *   workspace at least attn_decode_workspace_bytes()
 */
int attn_decode(const void* q, const void* cache, size_t cache_bytes,
                const float* cos_tab, const float* sin_tab, void* o, float* lse,
                void* workspace, size_t workspace_bytes, int pos,
                int B, int H, int Tmax, int D, int dtype, void* stream);

/*
 * The per-layer kernels next to attention. The pages list RMSNorm and SwiGLU
 * among the engine's hand-written CUDA kernels ("Show HN: NanoEuler",
 * paragraph 2); each layer is causal attention plus a feed-forward network of
 * two linear transforms with a Swish activation, both wrapped in residual
 * connections ("Tiny Hackable CUDA", section 3). They give no formulas; the
 * readings implemented here:
 *   h = x + r                      (the residual stream, stored in dtype)
 *   y = h * rstd * g,  rstd = 1 / sqrt(mean over the C features of h^2 + eps)
 *   swiglu(u) = silu(a) * b for u = [a | b] (the fused gate/up projection),
 *   silu(a) = a * sigmoid(a)
 * 16-bit path only (ATTN_BF16, ATTN_F16; ATTN_F32 gets ATTN_ERR_DTYPE); every
 * tensor is row-major with rows of C (or 2F / F) elements, fp32 arithmetic.
 */

/*
 * attn_rmsnorm_fwd - residual add + RMSNorm of N rows of C features
 * (C a multiple of 256, 256 <= C <= 4096; N*C < 2^31).
 *   x         [N, C] dtype, input
 *   res       [N, C] dtype, residual added to x (NULL: h = x)
 *   g         [C] dtype, per-feature gain
 *   eps       > 0 (ATTN_ERR_VALUE otherwise); 1e-5 for the model read here
 *   h         [N, C] dtype, output x + res as stored (NULL: not written)
 *   y         [N, C] dtype, output
 *   rstd      [N] fp32, output (kept for the backward)
 */
int attn_rmsnorm_fwd(const void* x, const void* res, const void* g, float eps,
                     void* h, void* y, float* rstd, int N, int C, int dtype, void* stream);

/* attn_rmsnorm_bwd_workspace_bytes - P * C fp32, rounded up to 256, with P = min(ceil(N/w),
 * 4096/w) partial column sums, w = 16 for C <= 768 and 4 above. 0 for invalid arguments. */
size_t attn_rmsnorm_bwd_workspace_bytes(int N, int C, int dtype);

/*
 * attn_rmsnorm_bwd - gradients of L = sum(y * dy) + sum(h * dres):
 *   dh = rstd * (g*dy - h^ * mean(h^ * g * dy)) + dres, h^ = h * rstd,
 * the gradient of x and of res alike; dg = sum over rows of dy * h^ (a fixed
 * reduction order: deterministic).
 *   h, g, rstd  the forward's h (or x when it had no residual), gain and rstd
 *   dy          [N, C] dtype;  dres [N, C] dtype or NULL (zero)
 *   dh          [N, C] dtype, output;  dg [C] fp32, output
 *   workspace   at least attn_rmsnorm_bwd_workspace_bytes()
 */
int attn_rmsnorm_bwd(const void* h, const void* g, const float* rstd, const void* dy,
                     const void* dres, void* dh, float* dg, void* workspace,
                     size_t workspace_bytes, int N, int C, int dtype, void* stream);

/*
 * attn_swiglu_fwd - out = silu(a) * b for each row u = [a | b] of the fused
 * gate/up projection. u [N, 2F] dtype, out [N, F] dtype; F a multiple of 8,
 * 2*N*F < 2^31.
 */
int attn_swiglu_fwd(const void* u, void* out, int N, int F, int dtype, void* stream);

/*
 * attn_swiglu_bwd - du = [da | db], [N, 2F] dtype, for upstream dout [N, F]:
 * da = dout * b * s * (1 + a * (1 - s)), db = dout * silu(a), s = sigmoid(a).
 */
int attn_swiglu_bwd(const void* u, const void* dout, void* du, int N, int F, int dtype,
                    void* stream);

/*
 * attn_decode_step - a whole generation step in one launch: attn_kv_append of
 * the new token at position pos (k_new, v_new [B, H, D] dtype, pre-RoPE k),
 * then attn_decode at pos, with the same results. The new key and value are
 * used directly by the step and written into cache row pos. Arguments and
 * rules as attn_decode, plus k_new and v_new; the cache is an output here.
 */
int attn_decode_step(const void* q, const void* k_new, const void* v_new, void* cache,
                     size_t cache_bytes, const float* cos_tab, const float* sin_tab,
                     void* o, float* lse, void* workspace, size_t workspace_bytes, int pos,
                     int B, int H, int Tmax, int D, int dtype, void* stream);

/*
 * attn_bwd_saved_noalloc - attn_bwd_saved for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and bitwise the same dq, dk, dv, with the
 * pre-pass's per-row entries in a device array the library owns instead of a
 * caller workspace. Nothing is allocated or freed here. The array holds
 * attn_noalloc_scratch_bytes() (4 MiB) on each GPU, enough for B*H*T up to
 * 524288 rows on the 16-bit path (1048576 for ATTN_F32); larger problems get
 * ATTN_ERR_SCRATCH before any launch. Every call on a GPU uses that GPU's one
 * copy, so calls that overlap on one GPU (other streams or threads) race.
 * `stream` must belong to the current device (else ATTN_ERR_VALUE).
 */
int attn_bwd_saved_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse,
                           const float* cos_tab, const float* sin_tab,
                           const void* saved, size_t saved_bytes,
                           void* dq, void* dk, void* dv,
                           int B, int H, int T, int D, int dtype, void* stream);

/* attn_noalloc_scratch_bytes - bytes of that array on each GPU (4 MiB). */
size_t attn_noalloc_scratch_bytes(void);

/* attn_status_string - static, human-readable name of a status code. */
const char* attn_status_string(int status);

/* attn_last_hip_error - hipError_t of the calling thread's last ATTN_ERR_HIP (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_ROPE_ATTN_H */
