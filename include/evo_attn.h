/*
 * evo_attn.h -- C ABI of libevoattn.so: the Evoformer's biased, gated
 * attention on AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  For every attention line (batch b, row r),
 * head h, query q and key k:
 *
 *     s[q,k] = <Q[q], K[k]> / sqrt(C) + bias[b,h,q,k] + (keep[k] ? 0 : -inf)
 *     Out[q] = sigmoid(G[q]) * sum_k softmax_k(s[q,:])[k] * V[k]
 *
 * This is triangle attention as described in "Evoformer: the memory wall ZeRO
 * cannot move" (DeepSpeed course), section "The three operations" (the third
 * residue k of the triangle is chosen by attention; the logits are
 * O(N_res^3 * n_heads), section "Where the memory goes"), and the MSA row
 * attention with pair bias of the same trunk.  The forward and backward never
 * store the logits: they are tiled through on-chip memory with an online
 * softmax, the approach of EvoFlash-3D in "MegaFold: Efficient Training of
 * Next-Generation 3D Attention Protein Models on Cross-Platform GPUs",
 * section "Methodologie", item 1, including its additively broadcast pair
 * bias (one [H, N, N] bias shared by every row of a batch).
 *
 * Conventions shared by every entry point:
 *  - Pointers are device memory owned by the caller (except where stated).
 *    The library never allocates, frees or keeps a pointer after returning;
 *    the one exception is the fixed static scratch of evo_attn_fwd_noalloc.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns at once.  Inputs must stay valid and unchanged, and
 *    outputs untouched, until the stream has passed the work.
 *  - Tensors are dense, row-major (C order), with 16-byte aligned bases.
 *    "[B,R,N,H,C]" means element (b,r,n,h,c) sits at
 *    ((((b*R + r)*N + n)*H + h)*C + c).
 *  - dtype EVO_BF16: activations, weights, bias and outputs are bfloat16;
 *    products accumulate in fp32.  EVO_FP32: everything fp32.
 *  - Every argument is validated before any work is enqueued.  On error the
 *    call returns a non-zero evo_status_t, enqueues nothing, leaves outputs
 *    untouched and records a message readable with evo_last_error() on the
 *    calling thread.  No entry point prints, aborts or throws.
 *  - Supported head dimension: C = 32.  N, R, B and H are arbitrary (N >= 1);
 *    ragged tiles are handled in the kernels.
 *  - Calls on one stream are ordered; calls on different streams that share
 *    output buffers race (the library takes no locks).
 */
#ifndef EVO_ATTN_H
#define EVO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EVO_OK = 0,
  EVO_EINVAL = 1,      /* bad argument: NULL, size <= 0, inconsistent option */
  EVO_ENOTSUP = 2,     /* valid but unsupported: head dim, dtype, alignment  */
  EVO_EWORKSPACE = 3,  /* workspace missing or smaller than required         */
  EVO_EHIP = 4,        /* the HIP runtime reported an error on launch        */
  EVO_EINTERNAL = 5
} evo_status_t;

typedef enum { EVO_FP32 = 0, EVO_BF16 = 1 } evo_dtype_t;

/* Version of this header's ABI (incremented on incompatible change). */
int evo_abi_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on that thread. */
const char* evo_last_error(void);

/*
 * evo_attn_fwd -- forward of biased gated attention.
 *
 *   q, k, v   [B,R,N,H,C] dtype.  Rows r are independent attention lines
 *             (MSA sequences, or rows/columns of the pair representation).
 *   gate      [B,R,N,H,C] dtype, pre-sigmoid g; NULL = no gating.
 *   key_mask  [B,mask_rows,N] uint8, nonzero = keep the key, 0 = the key's
 *             logit is -inf in every query; mask_rows is 1 (shared by all rows
 *             of a batch) or R (one mask per row).  NULL = no mask
 *             (mask_rows ignored).
 *   bias      [B,H,N,N] dtype, bias[b,h,q,k] added to the logits of every row
 *             of batch b; NULL = no bias.
 *   out       [B,R,N,H,C] dtype.
 *   lse       [B,R,H,N] fp32, natural-log log-sum-exp of each query's logits
 *             (needed by evo_attn_bwd); NULL = not written.
 *   workspace device scratch of evo_attn_fwd_workspace_bytes(...) bytes,
 *             16-byte aligned, owned by the caller; required when bias or
 *             key_mask is given, ignored otherwise.  It holds the bias in the
 *             kernel's tile order with the shared mask and the tile padding
 *             folded in as -inf: fp32 for EVO_FP32, fp16 for EVO_BF16 (which
 *             holds every bf16 value of magnitude 2^-14 .. 65504 exactly;
 *             finite bias values beyond +-65504 are clamped to it).  Contents
 *             on entry are ignored.
 *
 * A query whose keys are all masked gets Out = 0 and lse = -inf.
 */
evo_status_t evo_attn_fwd(evo_dtype_t dtype, int64_t B, int64_t R, int64_t N,
                          int64_t H, int64_t C, const void* q, const void* k,
                          const void* v, const void* gate,
                          const uint8_t* key_mask, int64_t mask_rows,
                          const void* bias, void* out, float* lse,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * evo_attn_fwd_noalloc -- evo_attn_fwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and errors as evo_attn_fwd, minus workspace/workspace_bytes.
 *
 * The prepared bias lives in a static scratch array of 16 MiB inside the
 * library (one per GPU, held until the process ends; its device address is
 * looked up once per device on the first call there).  A problem whose
 * evo_attn_fwd_workspace_bytes(...) exceeds 16 MiB is rejected with
 * EVO_ENOTSUP before anything is enqueued (e.g. bf16 with H * N^2 above
 * 8 Mi elements: H = 4 up to N ~ 1448).  The call allocates nothing.  Every
 * call on one GPU uses the same scratch: calls that may overlap on one GPU
 * (different streams without ordering) race and must not be issued.  The
 * scratch needs no clearing: each call writes every element it reads.
 */
evo_status_t evo_attn_fwd_noalloc(evo_dtype_t dtype, int64_t B, int64_t R,
                                  int64_t N, int64_t H, int64_t C, const void* q,
                                  const void* k, const void* v, const void* gate,
                                  const uint8_t* key_mask, int64_t mask_rows,
                                  const void* bias, void* out, float* lse,
                                  void* stream);

/*
 * evo_probe_issue_rate -- a measurement helper, not part of the attention
 * path: launches 256 * waves_per_simd workgroups of 256 threads that each
 * run `iters` iterations of 8 independent instructions of one kind (0:
 * v_exp_f32, 1: v_fma_f32, 2: v_mfma_f32_16x16x32_bf16) and write one
 * float per thread to `out` (device, 256 * 256 * waves_per_simd floats,
 * caller-owned).  Timing the launch gives that instruction's issue interval
 * per SIMD, from which the benchmark derives the softmax's ceiling on the
 * matrix-core fraction.  waves_per_simd in 1..8, iters >= 1.
 */
evo_status_t evo_probe_issue_rate(int kind, int waves_per_simd, int iters, float* out,
                                  void* stream);

/* Bytes of device workspace evo_attn_fwd needs when a bias or mask is given
 * (O(B * H * N^2); 0 on a problem evo_attn_fwd would reject). */
size_t evo_attn_fwd_workspace_bytes(evo_dtype_t dtype, int64_t B, int64_t R,
                                    int64_t N, int64_t H, int64_t C);

/* Bytes of device workspace evo_attn_bwd needs for this problem (0 on a
 * problem evo_attn_bwd would reject). */
size_t evo_attn_bwd_workspace_bytes(evo_dtype_t dtype, int64_t B, int64_t R,
                                    int64_t N, int64_t H, int64_t C);

/*
 * evo_attn_bwd -- backward of evo_attn_fwd (same q, k, v, gate, key_mask,
 * mask_rows, bias), recomputing the logits tile by tile from `lse`.
 *
 *   out       [B,R,N,H,C] dtype, the forward output.
 *   lse       [B,R,H,N] fp32 from evo_attn_fwd.
 *   dout      [B,R,N,H,C] dtype, gradient of the loss with respect to out.
 *   dq,dk,dv  [B,R,N,H,C] dtype, written (not accumulated).
 *   dgate     [B,R,N,H,C] dtype, gradient w.r.t. the pre-sigmoid gate;
 *             must be NULL iff gate is NULL.
 *   dbias     [B,H,N,N] fp32: the sum over the R rows of each batch of the
 *             logit gradients, written (not accumulated); NULL = skipped.
 *   workspace device scratch of evo_attn_bwd_workspace_bytes(...) bytes,
 *             16-byte aligned, owned by the caller; its contents on entry are
 *             ignored and on return are unspecified.
 *
 * Memory beyond inputs and outputs is O(R*H*N*C + H*N^2): the [N,N] logit
 * blocks of each row are never stored.
 */
evo_status_t evo_attn_bwd(evo_dtype_t dtype, int64_t B, int64_t R, int64_t N,
                          int64_t H, int64_t C, const void* q, const void* k,
                          const void* v, const void* gate,
                          const uint8_t* key_mask, int64_t mask_rows,
                          const void* bias, const void* out, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          void* dgate, float* dbias, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * tri_attn_project -- first half of a triangle-attention module: LayerNorm
 * of the pair representation fused with the Q, K, V, gate and pair-bias
 * projections (the normalised N x N tensor is never written; the fusion of
 * "MegaFold...", section "Methodologie", item 3 "EvoFusion").
 *
 *   z          [N,N,CZ] dtype, the pair representation; CZ a multiple of
 *              32, at most 256; H*C at most 256; N at most 46340 (N*N
 *              positions are indexed in 32 bits); otherwise EVO_ENOTSUP.
 *   ln_w,ln_b  [CZ] dtype, LayerNorm weight and bias; ln_eps > 0.
 *              LayerNorm uses the population variance, statistics in fp32.
 *   w_q,w_k,w_v,w_g  [H*C, CZ] dtype in [out, in] layout (as
 *              torch.nn.Linear.weight): y = x . W^T, x a row vector.
 *   b_g        [H*C] dtype, gate bias; NULL = zero.
 *   w_bias     [H, CZ] dtype, pair-bias projection ([out, in]).
 *   ending     0 = starting node: line i holds z[i,:], so q[0,i,j] is the
 *              projection of z[i,j] and bias[0,h,j,k] comes from z[j,k].
 *              1 = ending node: line j holds column z[:,j], so q[0,j,i] is
 *              the projection of z[i,j] and bias[0,h,i,k] comes from z[k,i].
 *   q,k,v,g    [1,N,N,H,C] dtype outputs (B = 1, R = N lines).
 *   bias       [1,H,N,N] dtype output.
 */
evo_status_t tri_attn_project(evo_dtype_t dtype, int64_t N, int64_t CZ,
                              int64_t H, int64_t C, int ending, const void* z,
                              const void* ln_w, const void* ln_b, float ln_eps,
                              const void* w_q, const void* w_k,
                              const void* w_v, const void* w_g,
                              const void* b_g, const void* w_bias, void* q,
                              void* k, void* v, void* g, void* bias,
                              void* stream);

/*
 * tri_attn_out_project -- last step of the module: out = O . w_o + b_o,
 * written back in z layout.
 *
 *   o     [1,N,N,H,C] dtype (line layout, as produced by evo_attn_fwd on the
 *         tensors of tri_attn_project).
 *   w_o   [CZ, H*C] dtype in [out, in] layout: out = O . w_o^T + b_o;
 *         b_o [CZ] dtype or NULL = zero.
 *   out   [N,N,CZ] dtype; for the ending node, line j / place i is written to
 *         out[i,j].
 */
evo_status_t tri_attn_out_project(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                  int64_t H, int64_t C, int ending,
                                  const void* o, const void* w_o,
                                  const void* b_o, void* out, void* stream);

/* Bytes of device workspace tri_attn_module_fwd needs (0 if it would
 * reject the sizes). */
size_t tri_attn_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                int64_t H, int64_t C);

/*
 * tri_attn_module_fwd -- whole triangle-attention module forward:
 * tri_attn_project, evo_attn_fwd over the N lines with the projected pair
 * bias and the residue mask applied to keys, then tri_attn_out_project.
 *
 *   residue_mask  [N] uint8, nonzero = keep residue k as a key in every
 *                 line; NULL = no mask.  Masked residues still get outputs as
 *                 queries.
 *   out           [N,N,CZ] dtype, the module's update (no residual add).
 *   workspace     caller-owned device scratch of tri_attn_workspace_bytes(...)
 *                 bytes (holds the projected Q, K, V, gate, bias, the
 *                 attention output and the forward's prepared bias;
 *                 O(N^2 * H * C)).
 * Other arguments as in tri_attn_project / tri_attn_out_project.
 */
evo_status_t tri_attn_module_fwd(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                 int64_t H, int64_t C, int ending,
                                 const void* z, const uint8_t* residue_mask,
                                 const void* ln_w, const void* ln_b,
                                 float ln_eps, const void* w_q,
                                 const void* w_k, const void* w_v,
                                 const void* w_g, const void* b_g,
                                 const void* w_bias, const void* w_o,
                                 const void* b_o, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Backward of the triangle-attention module.
 *
 * The pages train with the fused kernels in both directions ("MegaFold:
 * Efficient Training of Next-Generation 3D Attention Protein Models on
 * Cross-Platform GPUs", section "Methodologie", items 1 and 3) but print no
 * formula for the backward; these calls compute the chain rule of the
 * forward defined by tri_attn_project, evo_attn_fwd and tri_attn_out_project.
 * Input gradients are in the working dtype; parameter gradients are fp32,
 * summed over every pair position, and overwrite their buffers.  The results
 * are deterministic (no atomics; sums in a fixed order).
 *
 * Sizes: as for the forward, and in addition CZ <= 128 and H*C <= 128
 * (otherwise EVO_ENOTSUP).  Pointers: caller-owned device memory, 16-byte
 * aligned (EVO_ENOTSUP otherwise), NULL only where stated (EVO_EINVAL).
 * The calls enqueue on `stream` and return at once.
 */

/* Bytes of device workspace tri_attn_out_project_bwd and
 * tri_attn_project_bwd need (0 if they would reject the sizes). */
size_t tri_attn_proj_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N,
                                         int64_t CZ, int64_t H, int64_t C);

/*
 * tri_attn_out_project_bwd -- backward of tri_attn_out_project.
 *
 *   o      [1,N,N,H,C] dtype, the forward's input (line layout).
 *   w_o    [CZ, H*C] dtype ([out, in]).
 *   dout   [N,N,CZ] dtype, gradient of the output (z layout).
 *   d_o    [1,N,N,H,C] dtype out: dout (line order) . w_o.
 *   dw_o   [CZ, H*C] fp32 out: sum over positions of dout^T o.
 *   db_o   [CZ] fp32 out: sum over positions of dout.
 *   workspace  tri_attn_proj_bwd_workspace_bytes(...) bytes.
 */
evo_status_t tri_attn_out_project_bwd(evo_dtype_t dtype, int64_t N,
                                      int64_t CZ, int64_t H, int64_t C,
                                      int ending, const void* o,
                                      const void* w_o, const void* dout,
                                      void* d_o, float* dw_o, float* db_o,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * tri_attn_project_bwd -- backward of tri_attn_project (LayerNorm and the
 * Q, K, V, gate and pair-bias projections), fused like the forward: the
 * normalised pair representation is recomputed from z and never stored.
 *
 *   z, ln_w, ln_b, ln_eps, w_q, w_k, w_v, w_g, w_bias, ending: as given to
 *              tri_attn_project.
 *   dq,dk,dv,dg  [1,N,N,H,C] dtype: gradients of q, k, v and of the
 *              pre-sigmoid gate g (as evo_attn_bwd returns them).
 *   dbias      [1,H,N,N] fp32: gradient of the projected pair bias.
 *   dz         [N,N,CZ] dtype out: gradient of z.
 *   dln_w, dln_b  [CZ] fp32 out.
 *   dw_q,dw_k,dw_v,dw_g  [H*C, CZ] fp32 out; db_g [H*C] fp32 out (the gate
 *              bias; its gradient is the sum of dg).
 *   dw_bias    [H, CZ] fp32 out.
 *   workspace  tri_attn_proj_bwd_workspace_bytes(...) bytes.
 */
evo_status_t tri_attn_project_bwd(
    evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t H, int64_t C, int ending,
    const void* z, const void* ln_w, const void* ln_b, float ln_eps,
    const void* w_q, const void* w_k, const void* w_v, const void* w_g,
    const void* w_bias, const void* dq, const void* dk, const void* dv,
    const void* dg, const float* dbias, void* dz, float* dln_w, float* dln_b,
    float* dw_q, float* dw_k, float* dw_v, float* dw_g, float* db_g,
    float* dw_bias, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace tri_attn_module_bwd needs (0 if it would reject
 * the sizes): the recomputed activations and their gradients, O(N^2 * H *
 * C). */
size_t tri_attn_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                    int64_t H, int64_t C);

/*
 * tri_attn_module_bwd -- gradients of the whole module forward
 * (tri_attn_module_fwd) with respect to z and every parameter, given the
 * gradient of its output.  The forward's activations are recomputed from z
 * (tri_attn_project, evo_attn_fwd with the log-sum-exp), then
 * tri_attn_out_project_bwd, evo_attn_bwd (residue mask on keys, pair-bias
 * gradient summed over lines) and tri_attn_project_bwd run in turn.
 *
 *   z, residue_mask, ln_w, ln_b, ln_eps, w_q, w_k, w_v, w_g, b_g, w_bias,
 *   w_o, ending: as given to tri_attn_module_fwd (b_o does not enter the
 *              gradients).
 *   dout       [N,N,CZ] dtype: gradient of the module's output.
 *   dz ... dw_bias: as in tri_attn_project_bwd; dw_o, db_o: as in
 *              tri_attn_out_project_bwd.
 *   workspace  tri_attn_bwd_workspace_bytes(...) bytes.
 */
evo_status_t tri_attn_module_bwd(
    evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t H, int64_t C, int ending,
    const void* z, const uint8_t* residue_mask, const void* ln_w,
    const void* ln_b, float ln_eps, const void* w_q, const void* w_k,
    const void* w_v, const void* w_g, const void* b_g, const void* w_bias,
    const void* w_o, const void* dout, void* dz, float* dln_w, float* dln_b,
    float* dw_q, float* dw_k, float* dw_v, float* dw_g, float* db_g,
    float* dw_bias, float* dw_o, float* db_o, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * Triangular multiplicative update ("Evoformer: the memory wall ZeRO cannot
 * move", section "The three operations"): edge (i, j) of the pair
 * representation is updated from every third residue k as the sum over k of
 * a_ik * b_jk, channel by channel.  a and b are projections of the
 * layer-normalised pair representation (the normalisation and projection of
 * tri_attn_project); the update is projected back to CZ channels:
 *   x = LN(z),  a = x . w_a^T,  b = x . w_b^T                 (C channels)
 *   outgoing:  t[i,j,c] = sum_k keep[k] a[i,k,c] b[j,k,c]
 *   incoming:  t[i,j,c] = sum_k keep[k] a[k,i,c] b[k,j,c]
 *   out[i,j]   = t[i,j] . w_o^T + b_o
 * The sum over k is a dense per-channel matrix product (C products of
 * N x N by N x N) on the matrix cores, fp32 accumulation.
 *
 *   z          [N,N,CZ] dtype; N at most 46340; CZ and C multiples of 32, at
 *              most 128 (EVO_ENOTSUP otherwise).
 *   residue_mask  [N] uint8, nonzero = keep residue k as a third residue;
 *              NULL = keep all.
 *   ln_w, ln_b [CZ] dtype; ln_eps > 0 (population variance, fp32 statistics).
 *   w_a, w_b   [C, CZ] dtype ([out, in]); w_o [CZ, C] dtype; b_o [CZ] dtype
 *              or NULL = zero.
 *   outgoing   1 = outgoing edges (i,k), (j,k); 0 = incoming (k,i), (k,j).
 *   out        [N,N,CZ] dtype, the update (no residual add).
 *   workspace  tri_mul_workspace_bytes(...) bytes, caller-owned (a and b
 *              channel-major with padded rows, and t; O(N^2 * C)).
 * Pointers: device memory, 16-byte aligned.  Enqueued on `stream`.
 */
size_t tri_mul_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                               int64_t C);
evo_status_t tri_mul_fwd(evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t C,
                         int outgoing, const void* z,
                         const uint8_t* residue_mask, const void* ln_w,
                         const void* ln_b, float ln_eps, const void* w_a,
                         const void* w_b, const void* w_o, const void* b_o,
                         void* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * tri_mul_bwd -- gradients of tri_mul_fwd for training.  The pages print no
 * backward for the update (it is part of the trained trunk, "Evoformer: the
 * memory wall ZeRO cannot move", section "The three operations"); this is
 * the chain rule of the forward.  Per channel, with A_c[i,k] = a[i,k,c]
 * (outgoing; a[k,i,c] incoming), B_c likewise and dT = dout . w_o:
 *   dA_c = (dT_c . B_c) * keep[k],   dB_c = (dT_c^T . A_c) * keep[k],
 *   dz   = LayerNorm backward of (da . w_a + db . w_b),
 *   dw_a = sum over positions of da^T LN(z), dw_b likewise,
 *   dw_o = sum over positions of dout^T t,   db_o = sum of dout,
 *   dln_w, dln_b the LayerNorm parameter gradients.
 * The activations (a, b, t) are recomputed from z; the two products per
 * channel run on the matrix cores; sums over positions are deterministic
 * (fixed order, no atomics).
 *
 *   N, CZ, C, outgoing, z, residue_mask, ln_w, ln_b, ln_eps, w_a, w_b, w_o
 *              as tri_mul_fwd (b_o is not needed).
 *   dout       [N,N,CZ] dtype: the upstream gradient.
 *   dz         [N,N,CZ] dtype (written).
 *   dln_w, dln_b [CZ] fp32; dw_a, dw_b [C, CZ] fp32; dw_o [CZ, C] fp32;
 *              db_o [CZ] fp32 (written, not accumulated).
 *   workspace  tri_mul_bwd_workspace_bytes(...) bytes, caller-owned: the
 *              operands and their transposes, t, dT and the products, and
 *              the reduction partials (about 6 C N^2 + 3 C N^2 elements of
 *              dtype; 1.4 GB in bf16 at N = 768, C = 128).
 * Sizes outside tri_mul_fwd's limits: EVO_ENOTSUP; null required pointers
 * or a short workspace: EVO_EINVAL.  Pointers: device memory, 16-byte
 * aligned.  Enqueued on `stream`.
 */
size_t tri_mul_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                   int64_t C);
evo_status_t tri_mul_bwd(evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t C,
                         int outgoing, const void* z,
                         const uint8_t* residue_mask, const void* ln_w,
                         const void* ln_b, float ln_eps, const void* w_a,
                         const void* w_b, const void* w_o, const void* dout,
                         void* dz, float* dln_w, float* dln_b, float* dw_a,
                         float* dw_b, float* dw_o, float* db_o, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * pair_transition_fwd -- LayerNorm + linear + SwiGLU transition of the pair
 * representation, fused (EvoFusion, "MegaFold: Efficient Training of
 * Next-Generation 3D Attention Protein Models on Cross-Platform GPUs",
 * section "Methodologie", item 3: no N x N intermediate is written between
 * the normalisation, the projections and the activation).  Per position:
 *   x = LN(z),  h = silu(x . w_a^T) * (x . w_b^T),  out = h . w_o^T
 * with silu(u) = u * sigmoid(u); no bias vectors; fp32 accumulation.
 *
 *   z          [N,N,CZ] dtype; N at most 46340; CZ a multiple of 32, at most
 *              128 (EVO_ENOTSUP otherwise).
 *   ln_w, ln_b [CZ] dtype; ln_eps > 0 (population variance, fp32 statistics).
 *   w_a, w_b   [HID, CZ] dtype ([out, in]); HID a multiple of 64, at most
 *              4096 (EVO_ENOTSUP otherwise).
 *   w_o        [CZ, HID] dtype.
 *   out        [N,N,CZ] dtype.
 *   workspace  pair_transition_workspace_bytes(...) bytes, caller-owned: the
 *              weights rearranged once per call for the fused kernel
 *              (O(HID * CZ), independent of N).
 * Pointers: device memory, 16-byte aligned.  Enqueued on `stream`.
 */
size_t pair_transition_workspace_bytes(evo_dtype_t dtype, int64_t N,
                                       int64_t CZ, int64_t HID);
evo_status_t pair_transition_fwd(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                 int64_t HID, const void* z, const void* ln_w,
                                 const void* ln_b, float ln_eps,
                                 const void* w_a, const void* w_b,
                                 const void* w_o, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * pair_transition_bwd -- gradients of pair_transition_fwd for training
 * (EvoFusion targets the activation memory of LayerNorm, projections and
 * SwiGLU: "MegaFold: Efficient Training of Next-Generation 3D Attention
 * Protein Models on Cross-Platform GPUs", section "Methodologie", item 3).
 * The chain rule of the forward, with silu'(u) = sigmoid(u) (1 + u (1 -
 * sigmoid(u))):
 *   dh = dout . w_o,  du = dh * v * silu'(u),  dv = dh * silu(u),
 *   dz = LayerNorm backward of du . w_a + dv . w_b,
 *   dw_a = sum over positions of du^T x, dw_b likewise with dv,
 *   dw_o = sum of dout^T h,  dln_w, dln_b the LayerNorm parameter gradients.
 * Activations are recomputed from z; sums over positions are deterministic
 * (fixed order, no atomics).
 *
 *   z, ln_w, ln_b, ln_eps, w_a, w_b, w_o  as pair_transition_fwd; HID a
 *              multiple of 128 (EVO_ENOTSUP otherwise).
 *   dout       [N,N,CZ] dtype: the upstream gradient.
 *   dz         [N,N,CZ] dtype (written).
 *   dln_w, dln_b [CZ] fp32; dw_a, dw_b [HID, CZ] fp32; dw_o [CZ, HID] fp32
 *              (written, not accumulated).
 *   workspace  pair_transition_bwd_workspace_bytes(...) bytes, caller-owned:
 *              the prepared weights, du, dv and h for the weight reductions
 *              (3 N^2 HID elements of dtype) and the reduction partials.
 * Pointers: device memory, 16-byte aligned.  Enqueued on `stream`.
 */
size_t pair_transition_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N,
                                           int64_t CZ, int64_t HID);
evo_status_t pair_transition_bwd(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                 int64_t HID, const void* z, const void* ln_w,
                                 const void* ln_b, float ln_eps,
                                 const void* w_a, const void* w_b,
                                 const void* w_o, const void* dout, void* dz,
                                 float* dln_w, float* dln_b, float* dw_a,
                                 float* dw_b, float* dw_o, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * outer_product_mean_fwd -- the MSA-to-pair bridge ("Evoformer: the memory
 * wall ZeRO cannot move", section "The three operations": the mean over all
 * sequences of the outer product of MSA columns i and j).  The pages give no
 * formula; this entry point computes
 *   x = LN(m),  a = x . w_a^T,  b = x . w_b^T               (c channels)
 *   o[i,j,c,d] = (1/S) sum_s a[s,i,c] b[s,j,d]
 *   out[i,j]   = flatten(o[i,j]) . w_o^T + b_o              (d fastest)
 * with fp32 accumulation; the product sum_s a b is rounded to dtype once
 * before the output projection.
 *
 *   m          [S,N,CM] dtype (sequence, residue, channel); S >= 1, N >= 1,
 *              S*N below 2^31; CM a multiple of 32, at most 256.
 *   ln_w, ln_b [CM] dtype; ln_eps > 0 (population variance, fp32 statistics).
 *   w_a, w_b   [C, CM] dtype ([out, in]); C a multiple of 32, at most 128.
 *   w_o        [CZ, C*C] dtype; CZ a multiple of 32, at most 128.
 *   b_o        [CZ] dtype, or null for no bias.
 *   out        [N,N,CZ] dtype.
 *   workspace  outer_product_mean_workspace_bytes(...) bytes, caller-owned:
 *              the two projections [N*C, S] and the product [N*C, N*C]
 *              (O(N^2 C^2); 1.2 GB in bf16 at N = 768, C = 32).
 * Sizes outside these limits: EVO_ENOTSUP; non-positive sizes, null required
 * pointers or a short workspace: EVO_EINVAL.  Pointers: device memory,
 * 16-byte aligned.  Enqueued on `stream`.
 */
size_t outer_product_mean_workspace_bytes(evo_dtype_t dtype, int64_t S,
                                          int64_t N, int64_t CM, int64_t C,
                                          int64_t CZ);
evo_status_t outer_product_mean_fwd(evo_dtype_t dtype, int64_t S, int64_t N,
                                    int64_t CM, int64_t C, int64_t CZ,
                                    const void* m, const void* ln_w,
                                    const void* ln_b, float ln_eps,
                                    const void* w_a, const void* w_b,
                                    const void* w_o, const void* b_o,
                                    void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * outer_product_mean_bwd -- gradients of outer_product_mean_fwd for
 * training.  The pages print no backward (the bridge is part of the trained
 * trunk, "Evoformer: the memory wall ZeRO cannot move", section "The three
 * operations"); this is the chain rule of the forward.  With
 * P[i,j,c,d] = sum_s a[s,i,c] b[s,j,d] and dO = (dout . w_o) / S per pair:
 *   da[s,i,c] = sum_{j,d} dO[i,j,c,d] b[s,j,d],
 *   db[s,j,d] = sum_{i,c} dO[i,j,c,d] a[s,i,c],
 *   dm   = LayerNorm backward of (da . w_a + db . w_b),
 *   dw_a = sum over (s, i) of da^T LN(m), dw_b likewise,
 *   dw_o = sum over pairs of dout^T flatten(P) / S,  db_o = sum of dout,
 *   dln_w, dln_b the LayerNorm parameter gradients.
 * a, b and P are recomputed from m; the three large contractions run on the
 * matrix cores; sums over positions are deterministic (fixed order, no
 * atomics).
 *
 *   S, N, CM, C, CZ, m, ln_w, ln_b, ln_eps, w_a, w_b, w_o  as
 *              outer_product_mean_fwd (b_o is not needed); CM at most 128,
 *              or 256 (EVO_ENOTSUP otherwise).
 *   dout       [N,N,CZ] dtype: the upstream gradient.
 *   dm         [S,N,CM] dtype (written).
 *   dln_w, dln_b [CM] fp32; dw_a, dw_b [C, CM] fp32; dw_o [CZ, C*C] fp32;
 *              db_o [CZ] fp32 (written, not accumulated).
 *   workspace  outer_product_mean_bwd_workspace_bytes(...) bytes,
 *              caller-owned: the operands in both orientations, P (then
 *              dP), P by pair rows (then dP transposed), dA, dB in both
 *              layouts and the reduction partials (about 2 (N C)^2 elements
 *              of dtype; 2.5 GB in bf16 at N = 768, C = 32).
 * Sizes outside these limits: EVO_ENOTSUP; null required pointers or a
 * short workspace: EVO_EINVAL.  Pointers: device memory, 16-byte aligned.
 * Enqueued on `stream`.
 */
size_t outer_product_mean_bwd_workspace_bytes(evo_dtype_t dtype, int64_t S,
                                              int64_t N, int64_t CM, int64_t C,
                                              int64_t CZ);
evo_status_t outer_product_mean_bwd(evo_dtype_t dtype, int64_t S, int64_t N,
                                    int64_t CM, int64_t C, int64_t CZ,
                                    const void* m, const void* ln_w,
                                    const void* ln_b, float ln_eps,
                                    const void* w_a, const void* w_b,
                                    const void* w_o, const void* dout, void* dm,
                                    float* dln_w, float* dln_b, float* dw_a,
                                    float* dw_b, float* dw_o, float* db_o,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EVO_ATTN_H */
