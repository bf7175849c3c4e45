/*
 * vsa.h -- C ABI of libvsa.so: the forward pass of Video Sparse Attention
 * (VSA) on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [VSA-ROCm]  "VSA: Accelerating Video Diffusion Inference with Sparse
 *               Attention on AMD GPUs" (AMD ROCm blog).
 *   [VSA-arXiv] "VSA: Faster Video Diffusion with Trainable Sparse Attention"
 *               (arXiv 2505.13389), Abstract.
 *
 * The forward pass, per attention layer and per (batch, head):
 *   1. vsa_permute      raster (t,h,w) tokens -> cube-major order
 *   2. vsa_pool         cube mean-pool -> Qc, Kc, Vc
 *   3. vsa_coarse_topk  coarse cube attention O_c + Top-K key cubes (LUT)
 *   4. vsa_sparse_attn_fwd  fine attention over the listed cubes, combined
 *                       with O_c through the gates
 *   5. vsa_unpermute    cube-major -> raster order
 * and, for training a layer end to end, the backward of each step:
 *   vsa_combine_bwd, vsa_sparse_attn_bwd, vsa_coarse_bwd and
 *   vsa_pool_unpermute_bwd (the index list held fixed); a training forward
 *   keeps O_f (step 4 without gates) and forms the output with vsa_combine.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, row-major, caller-allocated device buffers.  Raster
 *   token tensors are [batch, heads, N, head_dim] with N = T*H*W and raster
 *   token index (t*H + h)*W + w.  The cube grid is (ceil(T/ct), ceil(H/ch),
 *   ceil(W/cw)) with Nc cubes: a grid that does not divide into cubes is
 *   padded up to whole cubes ([VSA-ROCm] shows no other handling; reading:
 *   padded positions hold no token).  Cube-major token tensors are [batch,
 *   heads, Np, head_dim] with Np = Nc*vol rows; position p = c*vol + l, where
 *   cube c runs over the cube grid in the problem's cube order (raster by
 *   default, or along a 3D Hilbert curve) and l in raster order over
 *   (ct, ch, cw) inside the cube.  Padded positions hold zeros after a
 *   reorder, are never attended as keys, are left out of the cube means, and
 *   have no raster row (their cube-major outputs are unspecified).  Cube
 *   tensors are [batch, heads, Nc, head_dim].  When the grid divides, Np = N.
 * - The library never allocates, frees or synchronises.  Every call only
 *   queues work on `stream` (a hipStream_t; NULL is the default stream) and
 *   returns.  Calls are stateless and re-entrant; two calls may run
 *   concurrently on different streams if their outputs do not overlap.
 * - Arguments are checked on the host before anything is queued.  On an
 *   error nothing is launched and no output is touched.  The library cannot
 *   see buffer sizes: the caller guarantees each buffer holds the stated
 *   number of elements.  A launch failure returns VSA_ERR_HIP; faults inside
 *   a kernel surface at the caller's next synchronisation.
 * - The softmax scale is fixed at 1/sqrt(head_dim), as in the scaled
 *   dot-product attention of [VSA-ROCm] §The Attention Bottleneck in Video
 *   Diffusion.
 */
#ifndef VSA_H_
#define VSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem statement: token grid, cube edge lengths, heads and head size
 * ([VSA-ROCm] §Two-Stage Architecture, Stage 1, and §Appendix - Tensor
 * Specifications). */
typedef struct vsa_problem {
  int32_t batch;
  int32_t heads;
  int32_t T, H, W;      /* token grid */
  int32_t ct, ch, cw;   /* cube edges (a grid that does not divide is padded) */
  int32_t head_dim;     /* 64 or 128 */
  int32_t heads_kv;     /* key/value heads (grouped heads, the nhead_k of the
                           CK interface in [VSA-ROCm]); 0 means heads.  Must
                           divide heads: query head h uses key/value head
                           h / (heads / heads_kv).  K, V, Kc, Vc and their
                           gradients have heads_kv heads; everything else
                           has heads.  The single-tensor reorders and pools
                           work on p->heads heads: for a grouped K or V pass a
                           problem whose heads is heads_kv. */
  int32_t cube_order;   /* VSA_CUBES_RASTER or VSA_CUBES_HILBERT: the order
                           of the cubes in every cube-major tensor, in the
                           LUT and in the cube tensors ([VSA-ROCm]
                           §Two-Stage Architecture, Pre-stage: a 3D
                           space-filling curve; the raster order of the cube
                           grid is the default reading, the Hilbert order
                           keeps consecutive cubes adjacent in 3D). */
  int32_t head_dim_v;   /* value head size (the hdim_v of the CK interface in
                           [VSA-ROCm]); 0 means head_dim.  64 or 128.  V, Vc,
                           O_c, the gates and the attention output are this
                           wide; Q, K, Qc and Kc are head_dim wide, and the
                           softmax scale stays 1/sqrt(head_dim).  The
                           single-tensor reorders and pools work on
                           p->head_dim: for V pass a problem whose head_dim
                           is head_dim_v.  In the backward, O, dO, dV, dVc,
                           dO_c and the gate gradients are head_dim_v wide
                           as well. */
  const int32_t* cube_coords;  /* device array of Nc packed cube coordinates
                           written by vsa_cube_table for this problem and
                           copied to the device by the caller.  Required
                           (VSA_ERR_NULL otherwise) by every device entry
                           point when cube_order is VSA_CUBES_HILBERT;
                           ignored for VSA_CUBES_RASTER.  A table that was
                           not written for this problem gives unspecified
                           results, but kernels skip entries that lie outside
                           the cube grid, so it never causes an
                           out-of-bounds access. */
} vsa_problem;

/* Cube orders.  VSA_CUBES_HILBERT: the cubes follow the 3D Hilbert curve
 * of Skilling's transform ("Programming the Hilbert curve", AIP Conference
 * Proceedings 707, 2004) over the smallest power-of-two cube covering the
 * cube grid, t taking the first bit of each level; cells outside the grid
 * are skipped.  Each side of the cube grid must be at most 1024 cubes
 * (VSA_ERR_UNSUPPORTED otherwise). */
enum { VSA_CUBES_RASTER = 0, VSA_CUBES_HILBERT = 1 };

/* Element type of token tensors. */
enum { VSA_BF16 = 0, VSA_F32 = 1 };

/* Status codes. */
enum {
  VSA_OK = 0,
  VSA_ERR_NULL = -1,        /* a required pointer is NULL (or gate_c without oc) */
  VSA_ERR_SHAPE = -2,       /* a size <= 0, heads_kv not dividing heads, or sizes overflow */
  VSA_ERR_TOPK = -3,        /* top_k / max_kv_blocks outside [1, Nc] */
  VSA_ERR_UNSUPPORTED = -4, /* head_dim, dtype or cube volume the library does not handle */
  VSA_ERR_HIP = -5,         /* the HIP runtime refused a launch */
  VSA_ERR_LUT = -6,         /* reserved for LUT validation results */
  VSA_ERR_WORKSPACE = -7    /* workspace_bytes below what the workspace query reports */
};

/* Reorder raster tokens into cube-major order:
 *   x_cube[b, h, p, :] = x_raster[b, h, pi(p), :]
 * where pi(p) is the raster index of cube-major position p.  This is the
 * pre-stage token reordering of [VSA-ROCm] §Two-Stage Architecture: every run
 * of vol = ct*ch*cw consecutive positions is one spatio-temporal cube.
 * x_raster, x_cube: [batch, heads, N, head_dim] of `dtype` (VSA_BF16 or
 * VSA_F32).  Bit copy: the result is exact.  Buffers must not overlap. */
int vsa_permute(const vsa_problem* p, int32_t dtype, const void* x_raster,
                void* x_cube, void* stream);

/* Inverse of vsa_permute: x_raster[b, h, pi(p), :] = x_cube[b, h, p, :].
 * Hands the output back in the model's token order.  Same layouts and rules
 * as vsa_permute. */
int vsa_unpermute(const vsa_problem* p, int32_t dtype, const void* x_cube,
                  void* x_raster, void* stream);

/* Cube mean-pool ([VSA-ROCm] §Two-Stage Architecture, Stage 1):
 *   xc[b, h, c, :] = (1/n_c) * sum over the n_c real positions l of cube c
 *                    of x_cube[b, h, c*vol + l, :]   (n_c = vol unless padded)
 * x_cube: [batch, heads, N, head_dim] of `dtype`, cube-major.
 * xc:     [batch, heads, Nc, head_dim] float32, accumulated in float32 in a
 *         fixed order (deterministic). */
int vsa_pool(const vsa_problem* p, int32_t dtype, const void* x_cube,
             float* xc, void* stream);

/* vsa_permute followed by vsa_pool in one pass over the tokens
 * ([VSA-ROCm] §Two-Stage Architecture: the pre-stage reordering and the
 * Stage 1 cube pooling; every token is read once):
 *   x_cube[b, h, p, :] = x_raster[b, h, pi(p), :]
 *   xc[b, h, c, :]     = (1/vol) * sum_{l < vol} x_cube[b, h, c*vol + l, :]
 * Same layouts and rules as vsa_permute and vsa_pool; x_cube and xc hold
 * exactly the bits the two separate calls produce.  x_cube may be NULL:
 * then only xc is written, read straight from the raster rows (the same
 * bits), for a fine stage that gathers its cube tiles from raster order
 * (vsa_sparse_attn_fwd_gather). */
int vsa_permute_pool(const vsa_problem* p, int32_t dtype, const void* x_raster,
                     void* x_cube, float* xc, void* stream);

/* Coarse stage ([VSA-ROCm] §Two-Stage Architecture, Stage 1, and
 * §Generating Sparsity Patterns; [VSA-arXiv] Abstract).  Per (b, h) and query
 * cube i, with S[i, j] = <qc[i], kc[j]> / sqrt(head_dim) over all Nc cubes:
 *   kv_block_idx[b, h, i, 0:top_k] = the top_k cubes j with the largest
 *       S[i, j], ties to the lower j, stored in ascending j;
 *   valid_block_num[b, h, i] = top_k;
 *   oc[b, h, i, :] = sum_j softmax_j(S[i, :]) * vc[j, :]   (if oc != NULL).
 * qc, kc, vc, oc: [batch, heads, Nc, head_dim] float32 (vc may be NULL when
 * oc is NULL).  kv_block_idx: [batch, heads, Nc, top_k] int32 (row stride
 * top_k).  valid_block_num: [batch, heads, Nc] int32.  Scores and the
 * selection are computed in float32.  Nc up to 4096. */
int vsa_coarse_topk(const vsa_problem* p, int32_t top_k, const float* qc,
                    const float* kc, const float* vc, int32_t* kv_block_idx,
                    int32_t* valid_block_num, float* oc, void* stream);

/* Fine block-sparse attention with the gated combination
 * ([VSA-ROCm] §Two-Stage Architecture Stage 2, §Block-Sparse Encoding,
 * §Kernel Architecture, §Sparse Traversal; [VSA-arXiv] Abstract).
 * For query cube i of (b, h) and n = valid_block_num[b, h, i], the keys are
 * the tokens of cubes kv_block_idx[b, h, i, 0..n-1] (each listed entry
 * attended once per listing), and for every query token p of cube i:
 *   O_f[p] = sum_q softmax_q(<q_p, k_q> / sqrt(head_dim)) v_q
 *   out[p] = g_f[p] * O_f[p] + g_c[p] * oc[b, h, i]         (bf16, RNE)
 *   lse[p] = log(sum_q exp(<q_p, k_q> / sqrt(head_dim)))   (natural log)
 * gate_f == NULL means g_f = 1; gate_c == NULL means g_c = 0 (then oc may be
 * NULL).  A row with n == 0 gives O_f = 0 and lse = -inf.
 * q, k, v, out, gate_c, gate_f: [batch, heads, N, head_dim] bf16 cube-major.
 * kv_block_idx: [batch, heads, Nc, max_kv_blocks] int32; each of the first
 *   n entries of a row must lie in [0, Nc) (not checked here; see
 *   vsa_check_lut).  valid_block_num: [batch, heads, Nc] int32, each in
 *   [0, max_kv_blocks].
 * oc: [batch, heads, Nc, head_dim] float32; lse: [batch, heads, N] float32,
 *   cube-major, or NULL.
 * Requires cube volume 64, head_dim 64 or 128, Nc <= 65534, and a LUT row
 * length whose per-row schedule fits in on-chip memory (28 * max_kv_blocks +
 * Nc / 4 bytes <= 32 KiB, about max_kv_blocks <= 1130 at Nc = 4096);
 * otherwise VSA_ERR_UNSUPPORTED.  out must not alias an input. */
int vsa_sparse_attn_fwd(const vsa_problem* p, const void* q, const void* k,
                        const void* v, const int32_t* kv_block_idx,
                        const int32_t* valid_block_num, int32_t max_kv_blocks,
                        const float* oc, const void* gate_c,
                        const void* gate_f, void* out, float* lse,
                        void* stream);

/* vsa_sparse_attn_fwd followed by vsa_unpermute of out (and of lse) in one
 * pass ([VSA-ROCm] §Two-Stage Architecture: the output is handed back in
 * the model's token order): q, k, v, kv_block_idx, valid_block_num and oc
 * as for vsa_sparse_attn_fwd (cube-major); gate_c, gate_f and out are
 * [batch, heads, N, head_dim] bf16 and lse [batch, heads, N] float32 in
 * raster (t, h, w) token order.  out[b, h, pi(p), :] holds exactly the bits
 * vsa_sparse_attn_fwd writes to its out[b, h, p, :] when given the
 * cube-major gates.  Same requirements and errors as vsa_sparse_attn_fwd. */
int vsa_sparse_attn_fwd_raster(const vsa_problem* p, const void* q,
                               const void* k, const void* v,
                               const int32_t* kv_block_idx,
                               const int32_t* valid_block_num,
                               int32_t max_kv_blocks, const float* oc,
                               const void* gate_c, const void* gate_f,
                               void* out, float* lse, void* stream);

/* vsa_permute of q, k and v followed by vsa_sparse_attn_fwd_raster, with
 * the reorder done by the fine kernel's own tile loads ([VSA-ROCm]
 * §Two-Stage Architecture: the pre-stage reordering groups each cube's
 * tokens together; here the kernel fetches every 64-token key, value and
 * query cube straight from the raster rows, one run of 4 tokens along w per
 * 1 KiB load, instead of reading a reordered copy).
 * q: [batch, heads, N, head_dim] bf16, k, v: [batch, heads_kv, N, head_dim]
 * bf16, all in raster (t, h, w) token order; kv_block_idx, valid_block_num
 * and oc as for vsa_sparse_attn_fwd (cube-major, per cube); gate_c, gate_f,
 * out and lse in raster order as for vsa_sparse_attn_fwd_raster.  out and
 * lse hold exactly the bits vsa_sparse_attn_fwd_raster writes when given
 * vsa_permute of q, k and v.  Requires head_dim = head_dim_v = 128, cubes 4
 * tokens wide (cw = 4; cube volume 64), a grid that divides into cubes and
 * the schedule limit of vsa_sparse_attn_fwd; otherwise VSA_ERR_UNSUPPORTED.
 * Every LUT row length runs the pair-of-cubes kernel (the quad kernel, which
 * vsa_sparse_attn_fwd uses for rows listing at least half of the cubes,
 * does not gather).  out must not alias an input. */
int vsa_sparse_attn_fwd_gather(const vsa_problem* p, const void* q,
                               const void* k, const void* v,
                               const int32_t* kv_block_idx,
                               const int32_t* valid_block_num,
                               int32_t max_kv_blocks, const float* oc,
                               const void* gate_c, const void* gate_f,
                               void* out, float* lse, void* stream);

/* The model's own token layout ([VSA-ROCm] §Two-Stage Architecture: the
 * pre-stage reordering reads the sequence as the DiT produces it, and the
 * output is handed back in the model's order).  These take the raster-side
 * token tensors as [batch, N, heads, head_dim] (token-major, heads
 * interleaved, what a DiT's projections produce) instead of [batch, heads,
 * N, head_dim]; everything else is as for the entry point named in each.
 * Cube-major tensors keep the [batch, heads, N, head_dim] layout. */

/* vsa_permute with x_bnhd [batch, N, heads, head_dim]. */
int vsa_permute_bnhd(const vsa_problem* p, int32_t dtype, const void* x_bnhd,
                     void* x_cube, void* stream);

/* vsa_permute_pool with x_bnhd [batch, N, heads, head_dim]. */
int vsa_permute_pool_bnhd(const vsa_problem* p, int32_t dtype,
                          const void* x_bnhd, void* x_cube, float* xc,
                          void* stream);

/* vsa_sparse_attn_fwd_raster with gate_c, gate_f and out as [batch, N,
 * heads, head_dim] bf16 (raster token order); lse stays [batch, heads, N]
 * float32 in raster order.  out holds exactly the bits of the raster entry
 * point's out, transposed. */
int vsa_sparse_attn_fwd_bnhd(const vsa_problem* p, const void* q,
                             const void* k, const void* v,
                             const int32_t* kv_block_idx,
                             const int32_t* valid_block_num,
                             int32_t max_kv_blocks, const float* oc,
                             const void* gate_c, const void* gate_f,
                             void* out, float* lse, void* stream);

/* vsa_pool_unpermute_bwd with dx_bnhd [batch, N, heads, head_dim] float32. */
int vsa_pool_unpermute_bwd_bnhd(const vsa_problem* p, const float* dx_cube,
                                const float* dxc, float* dx_bnhd,
                                void* stream);

/* Device-side LUT validator (optional, asynchronous).  Writes to
 * *bad_rows (one device int32) the number of LUT rows whose count is
 * outside [0, max_kv_blocks] or which list a cube outside [0, Nc).
 * Read it after synchronising the stream; 0 means the LUT is safe to pass
 * to vsa_sparse_attn_fwd ([VSA-ROCm] §Block-Sparse Encoding). */
int vsa_check_lut(const vsa_problem* p, const int32_t* kv_block_idx,
                  const int32_t* valid_block_num, int32_t max_kv_blocks,
                  int32_t* bad_rows, void* stream);

/* Block relation matrix -> index list ([VSA-ROCm] §Comparison with Jenga,
 * "Sparse Encoding in CK Tile", and §Block-Sparse Encoding): turns the M x M
 * one-hot encoding a block-mask method keeps into the LUT the fine kernel
 * consumes, so such patterns (e.g. a union of importance, condition and
 * adjacency masks, with a different count per row) run on
 * vsa_sparse_attn_fwd unchanged.
 * mask: [batch, heads, Nc, Nc] uint8 on the device, nonzero = query cube i
 *   attends key cube j.
 * kv_block_idx: [batch, heads, Nc, max_kv_blocks] int32: the j of each row
 *   with mask != 0, ascending; entries past the row's count are not written.
 * valid_block_num: [batch, heads, Nc] int32 = min(row count, max_kv_blocks).
 * overflow_rows: one device int32, set to the number of rows with more than
 *   max_kv_blocks selected cubes (those keep their first max_kv_blocks).
 * max_kv_blocks in [1, Nc], else VSA_ERR_TOPK. */
int vsa_mask_to_lut(const vsa_problem* p, const uint8_t* mask,
                    int32_t max_kv_blocks, int32_t* kv_block_idx,
                    int32_t* valid_block_num, int32_t* overflow_rows,
                    void* stream);

/* Workspace of vsa_sparse_attn_bwd, in bytes, for this problem and LUT row
 * length (host only, no device work).  Same argument checks and errors as
 * vsa_sparse_attn_bwd. */
int vsa_sparse_attn_bwd_workspace_size(const vsa_problem* p,
                                       int32_t max_kv_blocks, size_t* bytes);

/* Backward of the fine attention O_f of vsa_sparse_attn_fwd
 * ([VSA-arXiv] Abstract: the sparse attention is trained end to end;
 * [VSA-ROCm] §Two-Stage Architecture Stage 2 and §Block-Sparse Encoding for
 * the function differentiated).  For query cube i with listed key tokens R,
 * scale = 1/sqrt(head_dim), P = exp(scale * Q_i K_R^T - lse_i) and
 * Drow = rowsum(dO_i * O_i):
 *   dP = dO_i V_R^T,  dS = P * (dP - Drow),
 *   dq_i = scale * dS K_R,  dk_R += scale * dS^T Q_i,  dv_R += P^T dO_i,
 * summed over every listing (a cube listed twice contributes twice); tokens of
 * cubes no row lists get dk = dv = 0, rows with count 0 get dq = 0.
 * q, k, v, kv_block_idx, valid_block_num, max_kv_blocks: exactly as passed to
 *   vsa_sparse_attn_fwd (cube-major; every listed entry in [0, Nc)).
 * o:   [batch, heads, N, head_dim_v] bf16, cube-major: O_f, i.e. the out of
 *      vsa_sparse_attn_fwd called with gate_c == NULL and gate_f == NULL.
 * lse: [batch, heads, N] float32, cube-major: the lse of that call.
 * d_o: [batch, heads, N, head_dim_v] bf16, cube-major: the gradient of the loss
 *      with respect to O_f (the gates' own chain rule, elementwise, is the
 *      caller's).
 * dq, dk, dv: [batch, heads, N, head_dim] float32 (dv head_dim_v wide),
 *      cube-major, fully written
 *      (no accumulation into prior contents); the products run on bf16 MFMA
 *      with float32 accumulation, P and dS rounded to bf16 as operands.
 * workspace: device memory of workspace_bytes >= the size
 *      vsa_sparse_attn_bwd_workspace_size reports, else VSA_ERR_WORKSPACE;
 *      its contents on entry do not matter and are clobbered.
 * Deterministic: no atomics touch dq, dk or dv; repeated calls give the same
 * bits.  Requires cube volume 64, head_dim 64 or 128 and Nc <= 8192, else
 * VSA_ERR_UNSUPPORTED; max_kv_blocks outside [1, Nc] is VSA_ERR_TOPK.
 * Outputs must not alias inputs or the workspace. */
int vsa_sparse_attn_bwd(const vsa_problem* p, const void* q, const void* k,
                        const void* v, const int32_t* kv_block_idx,
                        const int32_t* valid_block_num, int32_t max_kv_blocks,
                        const void* o, const float* lse, const void* d_o,
                        float* dq, float* dk, float* dv, void* workspace,
                        size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * backward as vsa_sparse_attn_bwd with the same arguments except the
 * workspace, which is a fixed device array of VSA_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, kept until the process ends.  Calls on
 * one GPU share that array: two calls that overlap in time on the same GPU
 * (different streams, or host threads without ordering) race and give
 * unspecified results; calls queued on one stream are ordered and safe.
 * Problems whose workspace (vsa_sparse_attn_bwd_workspace_size) exceeds
 * VSA_NOALLOC_SCRATCH_BYTES return VSA_ERR_WORKSPACE and launch nothing.
 * Allocates nothing: no hipMalloc, hipFree or allocating library call (the
 * array's device address is looked up once per GPU with
 * hipGetSymbolAddress, on the first call there).  Outputs are bit-identical
 * to vsa_sparse_attn_bwd's. */
#define VSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int vsa_sparse_attn_bwd_noalloc(const vsa_problem* p, const void* q, const void* k,
                                const void* v, const int32_t* kv_block_idx,
                                const int32_t* valid_block_num, int32_t max_kv_blocks,
                                const void* o, const float* lse, const void* d_o,
                                float* dq, float* dk, float* dv, void* stream);

/* The gated combination as a pass of its own ([VSA-ROCm] §Two-Stage
 * Architecture: the output combines the coarse and fine outputs through
 * gates), for callers that keep the fine output O_f itself, such as a
 * training forward (run vsa_sparse_attn_fwd without gates for O_f and its
 * LSE, then this call for the layer's output):
 *   out[b, h, pi(p), :] = g_f[b, h, pi(p), :] * o_f[b, h, p, :]
 *                         + g_c[b, h, pi(p), :] * oc[b, h, c(p), :]
 * formed in float32 (the product with g_f, then one fused multiply-add with
 * g_c, as in vsa_sparse_attn_fwd's epilogue) and rounded to bf16 once.
 * Because o_f is already bf16 this differs from the fused epilogue by that
 * one rounding of O_f.  gate_f == NULL means g_f = 1; gate_c == NULL means
 * g_c = 0 (oc may then be NULL); without gates this is vsa_unpermute of o_f.
 * o_f:  [batch, heads, Np, head_dim_v] bf16, cube-major (padded positions
 *       are not read); oc: [batch, heads, Nc, head_dim_v] float32.
 * gate_c, gate_f, out: [batch, heads, N, head_dim_v] bf16, raster order.
 * Errors: VSA_ERR_NULL (o_f or out NULL, or gate_c without oc), the
 * vsa_problem checks; nothing is written then. */
int vsa_combine(const vsa_problem* p, const void* o_f, const float* oc,
                const void* gate_c, const void* gate_f, void* out, void* stream);

/* Backward of the gated combination ([VSA-ROCm] §Two-Stage Architecture:
 * gates between the coarse and fine outputs; [VSA-arXiv] Abstract: trained
 * end to end).  For out[p] = g_f[p] * O_f[p] + g_c[p] * oc[c(p)], c(p) the cube
 * of token p, and the upstream gradient dout:
 *   d_of[p]     = g_f[p] * dout[p]                   (bf16, RNE)
 *   d_oc[c]     = sum over the cube's tokens of g_c * dout   (float32,
 *                 fixed summation order; 0 when gate_c == NULL)
 *   d_gate_f[p] = dout[p] * O_f[p],  d_gate_c[p] = dout[p] * oc[c(p)]  (float32)
 * gate_f == NULL means g_f = 1 (then o_f and d_gate_f may be NULL);
 * gate_c == NULL means g_c = 0 (then oc and d_gate_c may be NULL).
 * dout, o_f, gate_c, gate_f, d_of: [batch, heads, N, head_dim_v] bf16;
 * d_gate_c, d_gate_f: same shape float32; oc, d_oc: [batch, heads, Nc,
 * head_dim_v] float32.  All token tensors cube-major (vsa_permute them). */
int vsa_combine_bwd(const vsa_problem* p, const void* dout, const void* o_f,
                    const float* oc, const void* gate_c, const void* gate_f,
                    void* d_of, float* d_oc, float* d_gate_c, float* d_gate_f,
                    void* stream);

/* Workspace of vsa_coarse_bwd in bytes (2 * batch * heads * Nc^2 * 4: the
 * coarse probabilities P and dS).  Host only; Nc > 4096 gives
 * VSA_ERR_UNSUPPORTED. */
int vsa_coarse_bwd_workspace_size(const vsa_problem* p, size_t* bytes);

/* Backward of the coarse attention ([VSA-ROCm] §Two-Stage Architecture,
 * Stage 1; [VSA-arXiv] Abstract).  With S = qc kc^T / sqrt(head_dim) over all
 * cubes, P = softmax(S) (recomputed), Dc = rowsum(d_oc * oc):
 *   dvc = P^T d_oc,  dS = P * (d_oc vc^T - Dc),
 *   dqc = dS kc / sqrt(head_dim),  dkc = dS^T qc / sqrt(head_dim).
 * qc, kc, vc, oc (the forward's O_c), d_oc, dqc, dkc, dvc: [batch, heads, Nc,
 * head_dim] float32 (vc, oc, d_oc and dvc head_dim_v wide), computed in
 * float32.  workspace of workspace_bytes >=
 * vsa_coarse_bwd_workspace_size, else VSA_ERR_WORKSPACE; clobbered.
 * Nc <= 4096. */
int vsa_coarse_bwd(const vsa_problem* p, const float* qc, const float* kc,
                   const float* vc, const float* oc, const float* d_oc,
                   float* dqc, float* dkc, float* dvc, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Backward of the reorder and the cube pool ([VSA-ROCm] §Two-Stage
 * Architecture: pre-stage reordering and Stage 1 mean-pooling): the gradient
 * of the raster input collects the cube-major gradient of its token plus,
 * through the mean, 1/vol of its cube's pooled gradient:
 *   dx_raster[b, h, pi(p), :] = dx_cube[b, h, p, :] + dxc[b, h, c(p), :] / vol
 * dx_cube, dx_raster: [batch, heads, N, head_dim] float32; dxc: [batch,
 * heads, Nc, head_dim] float32 or NULL (then a plain float32 unpermute).
 * Buffers must not overlap. */
int vsa_pool_unpermute_bwd(const vsa_problem* p, const float* dx_cube,
                           const float* dxc, float* dx_raster, void* stream);

/* Host helper: perm_host[p] = pi(p) for p < Np (the order vsa_permute
 * applies, in p->cube_order), -1 at padded positions.  perm_host is a host
 * array of Np int32.  No device work; cube_coords is not read. */
int vsa_perm_index(const vsa_problem* p, int32_t* perm_host);

/* Host helper: coords_host[c] = (ct_c << 20) | (ch_c << 10) | cw_c, the
 * grid coordinates of the c-th cube in p->cube_order, for c < Nc.  Copy
 * the array to the device and pass it as p->cube_coords.  coords_host is a
 * host array of Nc int32.  Each side of the cube grid must be at most 1024
 * cubes (VSA_ERR_UNSUPPORTED).  No device work, no allocation. */
int vsa_cube_table(const vsa_problem* p, int32_t* coords_host);

/* Host helper for measurement: the compute-unit count and peak shader clock
 * (kHz) HIP reports for `device`, and the dense bf16 matrix-core peak they
 * imply, cu_count * clock * 4096 flop per clock per CU (four SIMDs, each
 * retiring one 32x32x16 bf16 product of 32768 flop every 32 clocks), in
 * TFLOP/s.  Any output pointer may be NULL.  VSA_ERR_HIP when the device
 * cannot be queried; no device work, no allocation. */
int vsa_device_peak(int32_t device, int32_t* cu_count, int32_t* clock_khz,
                    double* bf16_tflops);

/* Static description of a status code (never NULL). */
const char* vsa_status_str(int status);

/* ABI version of this header: (major << 16) | minor. */
int vsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H_ */
