/*
 * svg.h -- C ABI of libsvg: the per-layer hot path of Sparse VideoGen's
 * spatial/temporal sparse 3D attention on one MI355X (gfx950).
 *
 * Sources cited below:
 *   [svg-authors] "Sparse VideoGen: Accelerating Video Diffusion Transformers with
 *                 Spatial-Temporal Sparsity", the authors' article (dtcms.com repost,
 *                 wzjs/233309).
 *   [svg-jqzx]    机器之心's ICML 2025 article on Sparse VideoGen (xinfinite.net repost,
 *                 t/topic/12021).
 *   [svg2-gist]   "Sparse VideoGen2: Accelerate Video Generation with Sparse Attention
 *                 via Semantic-Aware Permutation", explainer at gist.science (2505.18875).
 *   [adaspa]      "Training-free and Adaptive Sparse Attention for Efficient Long Video
 *                 Generation", the arxivdaily page of arXiv 2502.21079 (its abstract).
 *
 * Conventions shared by every call
 * --------------------------------
 * Geometry.  A latent video is F frames of an HH x WW token grid: P = HH*WW tokens per
 *   frame and S = F*P tokens.  Frame-major order (the model's) indexes token (f, y, x) as
 *   t = f*P + y*WW + x.  Token-major order indexes it as u = p*F + f with p = y*WW + x.
 * Tensors.  Q, K, V and outputs are [B][H][S][D] arrays, row-major, D contiguous, bf16
 *   (2-byte bfloat16) unless a call says otherwise.  D must be 64 or 128.
 * Memory.  Every tensor pointer is a DEVICE pointer owned by the caller and must be
 *   16-byte aligned.  The library allocates no device memory; calls that need scratch
 *   memory take a caller-owned workspace `ws` of at least svg_workspace_bytes(...) bytes.
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues
 *   work on it and returns; none synchronises the host.  Head kinds and errors written by
 *   svg_profile_heads stay on the device and are read there by later calls.
 * Errors.  Calls return svg_status: 0 on success, a negative code on failure.  Arguments
 *   are checked on the host before anything is enqueued; a failed check enqueues nothing.
 *   svg_last_error() gives a message for the calling thread's most recent failure.
 * Kinds.  One uint8 per (b, h) in [B*H] device arrays: SVG_SPATIAL, SVG_TEMPORAL or
 *   SVG_DENSE.  Kernels treat any other value as SVG_DENSE (a superset of both masks).
 * Thread safety.  The library keeps no state between calls except the per-thread error
 *   message; calls on different streams may run concurrently.
 */
#ifndef SVG_H
#define SVG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t svg_status;
#define SVG_OK               0
#define SVG_ERR_INVALID     (-1)   /* a null pointer, bad size, bad window, misaligned pointer ... */
#define SVG_ERR_UNSUPPORTED (-2)   /* a valid request the library does not implement (e.g. D not in {64,128}) */
#define SVG_ERR_HIP         (-3)   /* the HIP runtime reported an error while enqueueing */
#define SVG_ERR_WORKSPACE   (-4)   /* ws is NULL or smaller than svg_workspace_bytes() */

/* Head kinds ([svg-authors] Spatial Head / Temporal Head). */
#define SVG_SPATIAL  0
#define SVG_TEMPORAL 1
#define SVG_DENSE    2

/* Workspace-size queries. */
#define SVG_OP_PROFILE     1
#define SVG_OP_SPARSE_ATTN 2
#define SVG_OP_LAYER       3
#define SVG_OP_KMEANS      4   /* n = cluster count C */
#define SVG_OP_CLUSTER_ATTN 5  /* n = query cluster count Cq */
#define SVG_OP_BLOCK_ATTN  6   /* n unused */

/* Blocks of the block-sparse path: query rows x keys. */
#define SVG_BLOCK_Q 256
#define SVG_BLOCK_K 64

typedef struct {
    int32_t B, H;       /* batch, heads */
    int32_t F, HH, WW;  /* frames, token-grid rows, token-grid columns: S = F*HH*WW */
    int32_t D;          /* head dim, 64 or 128 */
} svg_geom;

typedef struct {
    int32_t frames;     /* w_f >= 0: a spatial head attends frames f-w_f .. f+w_f (clipped) */
    int32_t positions;  /* w_p >= 0: a temporal head attends in-frame positions p-w_p .. p+w_p
                           (flattened p = y*WW + x, clipped) in every frame */
} svg_windows;

/*
 * svg_qknorm_rope -- fused QK-RMSNorm and 3D rotary embedding of Q and K.
 * [svg-authors] closing section and [svg-jqzx] end of the layout section name both
 * operations as a cost the method optimises; neither page defines them.  Computed here:
 *   y[c] = x[c] / sqrt(mean_c' x[c']^2 + eps) * w[c]              (over the D channels of a row)
 *   then channel pairs (2j, 2j+1) of the slice of width n that holds them rotate by
 *   theta = pos * rope_base^(-2j/n):  (a, b) -> (a cos - b sin, a sin + b cos),
 *   where the head dim is split into slices [0, dt) | [dt, dt+dh) | [dt+dh, D) whose pos
 *   is the token's frame f, grid row y and grid column x respectively.
 * q, k:            bf16 [B][H][S][D] frame-major inputs.
 * q_out, k_out:    bf16 [B][H][S][D] outputs; may equal q / k (in place).
 * wq, wk:          fp32 [D] device arrays, shared by all heads.
 * eps > 0, rope_base > 0; dt, dh, dw >= 0, even, dt + dh + dw == D (svg_rope_split gives the
 *   split used by default).
 * The rotation tables are built on the device, once per workgroup, from rope_base alone: each
 *   inverse frequency rope_base^(-2j/n) is an fp64 power, each angle pos * freq is formed in
 *   fp64 and reduced to [-pi, pi], and its cosine and sine are taken in fp32 (within about one
 *   fp32 ulp).  The caller therefore passes no cos/sin tables.
 * Arithmetic in fp32, round-to-nearest-even on store.  V is not touched.
 */
svg_status svg_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                           const float* wq, const float* wk, float eps, float rope_base,
                           int32_t dt, int32_t dh, int32_t dw, svg_geom g, void* stream);

/*
 * svg_profile_heads -- online choice of each head's sparsity pattern.
 * [svg-jqzx] dynamic adaptive sparsity strategy, steps 1-3, and [svg-authors] Online
 * Profiling Strategy: for a small random sample of query rows, attention is computed with
 * the spatial mask, the temporal mask and no mask; each head keeps the mask whose result
 * is closest to the unmasked one.  Computed here, per (b, h):
 *   mse_x = mean over the n_q sampled rows and D channels of (O_x - O_dense)^2,  x in {sp, tp}
 *   kind  = SVG_SPATIAL if mse_sp <= mse_tp (both as stored fp32) else SVG_TEMPORAL.
 * q, k, v:   bf16 [B][H][S][D] frame-major.
 * q_idx:     int32 [n_q] device array of frame-major rows in [0, S), one sample for all
 *            heads; 1 <= n_q <= S.  Out-of-range entries are clamped into [0, S).
 * w:         the two candidate masks' windows.   scale > 0: softmax scale (1/sqrt(D) usual).
 * mse_out:   fp32 [B*H][2] device array (spatial, temporal).
 * kind_out:  uint8 [B*H] device array.
 * ws:        >= svg_workspace_bytes(SVG_OP_PROFILE, &g, n_q) bytes of device memory.
 * One head of K or V must stay under 4 GB (S * D * 2 bytes), else SVG_ERR_UNSUPPORTED.
 */
svg_status svg_profile_heads(const void* q, const void* k, const void* v, const int32_t* q_idx, int32_t n_q,
                             svg_geom g, svg_windows w, float scale, float* mse_out, uint8_t* kind_out,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * svg_permute / svg_unpermute -- the hardware-efficient layout transformation.
 * [svg-authors] Layout Transformation and [svg-jqzx] layout section: Q, K and V are
 * reordered along the sequence so that the tokens of one location (all frames) are
 * adjacent, by transposing the frame x location grid; the output is restored afterwards.
 *   svg_permute:   dst[b][h][u] = src[b][h][pi(u)],     pi(u)     = (u mod F)*P + u div F
 *   svg_unpermute: dst[b][h][t] = src[b][h][pi^-1(t)],  pi^-1(t)  = (t mod P)*F + t div P
 * Rows of D elements of elem_bytes (2 = bf16, 4 = fp32) are copied bit for bit.
 * Only heads with kind[b*H+h] == select are written; kind == NULL selects every head.
 * src and dst must not overlap.
 */
svg_status svg_permute(const void* src, void* dst, int32_t elem_bytes, const uint8_t* kind, int32_t select,
                       svg_geom g, void* stream);
svg_status svg_unpermute(const void* src, void* dst, int32_t elem_bytes, const uint8_t* kind, int32_t select,
                         svg_geom g, void* stream);

/*
 * svg_build_block_mask -- which bm x bn tiles of each head's score matrix hold at least one
 * allowed (query, key) pair, in the head's working layout (token-major for temporal heads,
 * frame-major otherwise).  This is the schedule svg_sparse_attn follows; it is exported for
 * inspection.  Patterns: [svg-authors] Spatial Head (blocks around the diagonal) and
 * Temporal Head (slash lines, contiguous after the layout transformation).
 * mask_out: uint8 [B*H][ceil(S/bm)][ceil(S/bn)] device array; 1 = tile computed.
 * bm, bn >= 1 (a tile may exceed the sequence; it is then clipped).
 */
svg_status svg_build_block_mask(const uint8_t* kind, svg_geom g, svg_windows w, int32_t bm, int32_t bn,
                                uint8_t* mask_out, void* stream);

/*
 * svg_sparse_attn -- block-sparse attention, each head under the mask of its kind.
 * [svg-authors] Layout Transformation / [svg-jqzx] kernel section: the sparse kernel only
 * computes the tiles the pattern needs.  Per head, in its working layout:
 *   O = softmax(scale * Q K^T  restricted to the head's token mask) V
 * Spatial and dense heads read q, k, v (frame-major) and write o.  Temporal heads work in
 * token-major order, in one of two ways:
 *   - qt, kt, vt, ot all non-NULL: they read qt, kt, vt (token-major, e.g. from svg_permute)
 *     and write ot (token-major; restore with svg_unpermute);
 *   - qt, kt, vt, ot all NULL (fused layout transformation): they read q, k, v and write o,
 *     frame-major, and the kernel applies the permutation as it loads and stores rows.
 *     Results are bit-identical to the first way followed by svg_unpermute.
 * Tiles outside the mask are skipped; inside boundary tiles the exact token mask is
 * applied.  bf16 inputs, fp32 accumulation, bf16 output.
 * q, k, v, o, qt, kt, vt, ot: bf16 [B][H][S][D]; a mix of NULL and non-NULL token-major
 * pointers is SVG_ERR_INVALID when kind is given (they are ignored when kind is NULL).
 * kind: uint8 [B*H] device array (NULL = every head dense).
 * ws:   >= svg_workspace_bytes(SVG_OP_SPARSE_ATTN, &g, 0) bytes: the order in which heads
 *       are processed and the counters workgroups take band items from; two calls in
 *       flight at once must not share it.
 * S*D*2 bytes (one head) must be below 4 GB, else SVG_ERR_UNSUPPORTED (also svg_dense_attn).
 */
svg_status svg_sparse_attn(const void* q, const void* k, const void* v,
                           const void* qt, const void* kt, const void* vt,
                           const uint8_t* kind, svg_geom g, svg_windows w, float scale,
                           void* o, void* ot, void* ws, size_t ws_bytes, void* stream);

/*
 * svg_dense_attn -- unmasked attention with the same kernel: the profiling reference of
 * [svg-jqzx] step 2 and the attention of the dense early steps in [svg-authors]' other
 * optimisations.  bf16 [B][H][S][D] in and out, frame-major.
 */
svg_status svg_dense_attn(const void* q, const void* k, const void* v, svg_geom g, float scale, void* o,
                          void* stream);

/*
 * svg_layer -- one attention layer of a denoising step in one call: the per-layer pipeline
 * of [svg-authors] (QK-Norm and RoPE, online profiling, sparse attention with the layout
 * transformation) and its schedule of dense attention in the early steps ([svg-authors]
 * other optimisations).  Enqueued in order on `stream`:
 *   1. when wq or wk is given: svg_qknorm_rope of q, k into qn, kn (slice widths dt, dh, dw);
 *      profiling and attention then read qn, kn.  Otherwise they read q, k, and qn, kn,
 *      eps, rope_base and dt, dh, dw are ignored.
 *   2. dense != 0: svg_dense_attn into o; q_idx, n_q, w, mse_out and kind_out are ignored.
 *      dense == 0: svg_profile_heads (kinds into kind_out, errors into mse_out), then
 *      svg_sparse_attn with the fused layout transformation into o.
 * Arguments, layouts and limits are those of the calls named above; every stage is checked
 * before any is enqueued.  o: bf16 [B][H][S][D] frame-major.
 * ws: >= svg_workspace_bytes(SVG_OP_LAYER, &g, n_q) bytes (profiling and attention share it).
 */
svg_status svg_layer(const void* q, const void* k, const void* v, const float* wq, const float* wk, float eps,
                     float rope_base, int32_t dt, int32_t dh, int32_t dw, void* qn, void* kn,
                     const int32_t* q_idx, int32_t n_q, svg_geom g, svg_windows w, float scale, int32_t dense,
                     void* o, float* mse_out, uint8_t* kind_out, void* ws, size_t ws_bytes, void* stream);

/*
 * svg_layer_noalloc -- svg_layer for callers that cannot allocate device memory or hand in a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, kernels and results as svg_layer, without ws and
 * ws_bytes: the scratch memory lives in a static device array of
 * SVG_LAYER_NOALLOC_SCRATCH_BYTES, one copy per device, held until the process ends; its
 * address is looked up once per device (with that device current) on the first call there.
 * The call allocates nothing.
 * Requests whose svg_workspace_bytes(SVG_OP_LAYER, &g, n_q) exceeds that size return
 * SVG_ERR_WORKSPACE before anything is enqueued.  `stream` must belong to the current device
 * (SVG_ERR_INVALID otherwise).  Every call on one device shares that device's scratch and
 * leaves its contents behind: calls that may overlap on one device (different streams, or
 * host threads) race and must be serialised by the caller.
 */
#define SVG_LAYER_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
svg_status svg_layer_noalloc(const void* q, const void* k, const void* v, const float* wq, const float* wk,
                             float eps, float rope_base, int32_t dt, int32_t dh, int32_t dw, void* qn, void* kn,
                             const int32_t* q_idx, int32_t n_q, svg_geom g, svg_windows w, float scale,
                             int32_t dense, void* o, float* mse_out, uint8_t* kind_out, void* stream);

/*
 * svg_dense_step -- the step schedule of [svg-authors] other optimisations: the first
 * dense_fraction of the n_steps denoising steps run dense attention, the rest sparse.
 * Step s (0-based) runs dense iff s < dense_fraction * n_steps, i.e. the first
 * ceil(dense_fraction * n_steps) steps.  Returns 1 (dense) or 0 (sparse);
 * SVG_ERR_INVALID unless 0 <= step < n_steps and 0 <= dense_fraction <= 1.
 */
int32_t svg_dense_step(int32_t step, int32_t n_steps, float dense_fraction);

/*
 * ---------------------------------------------------------------------------------------
 * Semantic clustering path ([svg2-gist] technical summary, section 2: A semantic-aware
 * permutation, B centroid-based top-p selection, C centroid cache and a kernel for
 * variable-size blocks).  Per (b, h): cluster the Q rows into Cq clusters and the K rows
 * into Ck clusters (svg_kmeans, twice), pick per query cluster the key clusters that carry
 * the top-p share of its estimated attention (svg_centroid_topp), and attend each query to
 * exactly the keys of its selected clusters (svg_cluster_attn).
 * ---------------------------------------------------------------------------------------
 */

/*
 * svg_kmeans -- `iters` Lloyd iterations on the rows of x (section 2A): every row goes to the
 * nearest centroid (squared Euclidean distance to the centroid rounded to bf16, evaluated as
 * bf16 products with fp32 accumulation; ties to the lowest index), then every centroid moves to
 * the fp64 mean of its rows, rounded to fp32; an empty cluster keeps its centroid.
 *
 * x:          bf16 [B][H][S][D] (Q or K), read only.
 * C:          clusters per (b, h), 1 <= C <= min(S, 4096).   iters: 1 .. 1000.
 * init_idx:   int32 [C] token indices or NULL.  Given: a cold start -- centroid c of every
 *             (b, h) starts as the row at token init_idx[c] (indices are clamped into [0, S)).
 *             NULL: start from the centroids passed in (the previous denoising step's, the
 *             cache of section 2C).
 * centroids:  fp32 [B*H][C][D], in (unless init_idx) and out: the centroids of the last update.
 * labels:     int32 [B*H][S] out: cluster of each token at the last assignment (so every
 *             centroid is the mean of the rows labelled with it).
 * perm:       int32 [B*H][S] out: the tokens sorted by cluster, stably (clusters in index
 *             order, tokens in order inside a cluster) -- the permutation of section 2A.
 * offsets:    int32 [B*H][C+1] out: cluster c holds perm[offsets[c] .. offsets[c+1]).
 * ws:         >= svg_workspace_bytes(SVG_OP_KMEANS, &g, C) bytes.
 */
svg_status svg_kmeans(const void* x, svg_geom g, int32_t C, int32_t iters, const int32_t* init_idx,
                      float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * svg_centroid_topp -- centroid-based top-p selection (section 2B), in fp64.  For query
 * cluster i and key cluster j with n_j > 0 keys, s_ij = scale * cq_i . ck_j and the estimated
 * share of i's attention on j is w_ij = n_j exp(s_ij) / sum_j' n_j' exp(s_ij') (a centroid
 * stands for all n_j keys of its cluster; empty clusters get 0).  Per query cluster, key
 * clusters are taken in decreasing w (ties: lower index first) until the taken shares sum to
 * at least p; clusters of share 0 are never taken.
 *
 * cq, ck:     fp32 [B*H][Cq][D], [B*H][Ck][D] (svg_kmeans centroids of Q and of K).
 * k_offsets:  int32 [B*H][Ck+1] from svg_kmeans of K (cluster sizes n_j).
 * Cq:         1 .. S.   Ck: 1 .. min(S, 1024).   p: (0, 1].   scale > 0.
 * sel:        uint8 [B*H][Cq][Ck] out: 1 for a selected key cluster.  Every query cluster
 *             selects at least one non-empty key cluster.
 */
svg_status svg_centroid_topp(const float* cq, const float* ck, const int32_t* k_offsets, svg_geom g, int32_t Cq,
                             int32_t Ck, float scale, float p, uint8_t* sel, void* stream);

/*
 * svg_cluster_attn -- attention over the selected clusters (sections 2A and 2C): every query
 * token attends exactly to the keys of the key clusters selected for its query cluster,
 * softmax(scale q k^T) v with bf16 products, fp32 accumulation and online softmax (the
 * weights rounded to bf16 for the value product).  The queries of one cluster are computed
 * together as dense tiles of up to 256 rows; their keys are gathered row by row from the key
 * list (the sorted tokens of the selected key clusters), so no tile is padded with keys of
 * unselected clusters.
 *
 * q, k, v:    bf16 [B][H][S][D] frame-major (the model's order), read only.
 * q_perm, q_offsets, k_perm, k_offsets: svg_kmeans outputs for Q (Cq clusters) and K (Ck).
 * sel:        uint8 [B*H][Cq][Ck] from svg_centroid_topp.
 * Cq:         1 .. min(S, 32767).   Ck: 1 .. min(S, 1024).   S <= 65535 * 256.
 * o:          bf16 [B][H][S][D] out, in the original token order.  A query cluster whose
 *             selected clusters hold no key leaves its rows unwritten (svg_centroid_topp never
 *             produces one).
 * ws:         >= svg_workspace_bytes(SVG_OP_CLUSTER_ATTN, &g, Cq) bytes (the key lists:
 *             B*H*Cq*S int32, plus work items).
 */
svg_status svg_cluster_attn(const void* q, const void* k, const void* v, const int32_t* q_perm,
                            const int32_t* q_offsets, const int32_t* k_perm, const int32_t* k_offsets,
                            const uint8_t* sel, svg_geom g, int32_t Cq, int32_t Ck, float scale, void* o, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * ---------------------------------------------------------------------------------------
 * Head-adaptive block-sparse path with an LSE-cached block search ([adaspa] abstract: a
 * blockified sparse pattern; a search that uses the log-sum-exp of attention rows cached from
 * earlier denoising steps; head-adaptive block-sparse attention).  Blocks are SVG_BLOCK_Q
 * query rows by SVG_BLOCK_K keys in token order, the last ones clipped at S:
 * nqb = ceil(S / 256) query blocks and nkb = ceil(S / 64) key blocks, nkb <= 4096.
 * ---------------------------------------------------------------------------------------
 */

/*
 * svg_dense_attn_lse -- svg_dense_attn that also writes every row's natural-log log-sum-exp
 * LSE_q = log sum_k exp(scale q.k) (from the kernel's running max and the row sum of its bf16
 * weights): the normaliser a later step's block search reuses.
 * lse: fp32 [B*H][S] out.
 */
svg_status svg_dense_attn_lse(const void* q, const void* k, const void* v, svg_geom g, float scale, void* o,
                              float* lse, void* stream);

/*
 * svg_block_mass -- the attention mass of every block under a cached normaliser:
 * mass[i][j] = sum over rows q of query block i and keys k of key block j of
 * exp(scale q.k - lse[q]) (bf16 products, fp32 accumulation, exponentials and sums).  With the
 * lse of the same q and k, a block row sums to its row count.
 * q, k: bf16 [B][H][S][D].  lse: fp32 [B*H][S] (from svg_dense_attn_lse of an earlier step).
 * mass: fp32 [B*H][nqb][nkb] out.
 */
svg_status svg_block_mass(const void* q, const void* k, const float* lse, svg_geom g, float scale, float* mass,
                          void* stream);

/*
 * svg_block_select -- the head-adaptive choice: per (b, h) and query block, key blocks in
 * decreasing mass (ties: lower block first) until their mass reaches coverage times the
 * block row's total mass (fp64 prefix sums of the fp32 masses); blocks of zero mass are never
 * chosen.  coverage: (0, 1].  sel: uint8 [B*H][nqb][nkb] out, 1 = chosen.
 */
svg_status svg_block_select(const float* mass, svg_geom g, float coverage, uint8_t* sel, void* stream);

/*
 * svg_block_sparse_attn -- attention of every query to exactly the keys of the key blocks
 * chosen for its query block (any uint8 [B*H][nqb][nkb] block mask), with the keys of the
 * chosen blocks gathered into the attention kernel's 64-key tiles.  A query block with no
 * chosen block leaves its rows unwritten.
 * o: bf16 [B][H][S][D] out.  ws: >= svg_workspace_bytes(SVG_OP_BLOCK_ATTN, &g, 0) bytes.
 */
svg_status svg_block_sparse_attn(const void* q, const void* k, const void* v, const uint8_t* sel, svg_geom g,
                                 float scale, void* o, void* ws, size_t ws_bytes, void* stream);

/* The default widths of the frame / grid-row / grid-column slices of the head dim for RoPE:
 * dt = D - 4*floor(D/6), dh = dw = 2*floor(D/6) (44/42/42 at D = 128, 24/20/20 at D = 64), the
 * near-even split into three even slices.  SVG_ERR_INVALID for D < 6 or odd D, or NULL outputs. */
svg_status svg_rope_split(int32_t D, int32_t* dt, int32_t* dh, int32_t* dw);

/* The default softmax scale 1/sqrt(D) (0 for D <= 0). */
float svg_default_scale(int32_t D);

/* Bytes of workspace a call needs (0 for an invalid request); n is the sample size n_q for
 * SVG_OP_PROFILE and SVG_OP_LAYER, the cluster count for SVG_OP_KMEANS and SVG_OP_CLUSTER_ATTN. */
size_t svg_workspace_bytes(int32_t op, const svg_geom* g, int32_t n);

/* Query-block x key-block tile of svg_sparse_attn / svg_dense_attn. */
void svg_tile_shape(int32_t* bm, int32_t* bn);

/* Static description of a status code. */
const char* svg_status_string(svg_status s);

/* Message of the calling thread's last failed call ("" if none). */
const char* svg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SVG_H */
