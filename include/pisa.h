/*
 * pisa.h -- C ABI of libpisa: piecewise block-sparse ("exact-or-approximate")
 * attention for diffusion-transformer self-attention on AMD Instinct MI355X
 * (gfx950), with keep-or-drop block-sparse attention as a mode flag.
 *
 * Method: "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
 * Transformers" (technical summary, gist.science), section 2 "Methodology":
 * the KV blocks of query block i are split into an exact set S_i and the rest
 * U_i; the output is o_t = N_t / D_t where the exact blocks contribute
 * e^{q k} terms, every block of U_i contributes a zeroth-order block Taylor
 * term alpha_{t,j} * sum_n v_{j,n} with alpha_{t,j} = e^{q kbar_j}, and one
 * global first-order correction q_t Hbar sum_{j in U_i} alpha_{t,j} is added.
 * Keep-or-drop: block-sparse attention notes (dpshk.com), section 3.3,
 * O_i = softmax(Q_i K_{S_i}^T / sqrt(d)) V_{S_i}.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors are dense, row-major and contiguous: Q, K, V, O are [b, h, L, d].
 *   Q, K, V and O share one element type (pisa_shape.dtype).  Statistics are
 *   always float32.
 * - Sequences are split into blocks of `block` consecutive tokens; query blocks
 *   and KV blocks have the same size.  L must be a multiple of `block` (pad on
 *   the caller's side, per modality, as the block-sparse notes do in section
 *   4.1); the library rejects ragged blocks rather than bias centroids with pad
 *   tokens.  nb = L / block.
 * - Supported: head_dim in {64, 128}; block in {64, 128}; nb <= 2048;
 *   batch*heads*nb < 2^31; batch*heads < 2^27 (PISA_ERR_SHAPE otherwise).
 * - Every pointer argument except `stream` is a DEVICE pointer owned by the
 *   caller; the library never allocates or frees device memory.  Its only
 *   device memory of its own is the static workspace array of
 *   pisa_precompute_noalloc (one per GPU, from module load until the process
 *   ends), and its only global state the per-device addresses of that array.
 *   `stream` is a hipStream_t (NULL = the
 *   legacy default stream).  Calls are asynchronous on that stream: results are
 *   valid once the stream reaches them.
 * - Every call validates its arguments on the host first and returns an error
 *   code without launching anything when they are wrong.  A failed launch
 *   returns PISA_ERR_HIP; pisa_last_error() then names the HIP error.  No C++
 *   exception crosses the ABI.
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PISA_VERSION 103 /* major * 100 + minor; 1.01 adds pisa_route_attention, 1.02
                            pisa_precompute_noalloc and pisa_attention_split, 1.03 the
                            form argument of pisa_route_attention */

typedef enum {
  PISA_OK = 0,
  PISA_ERR_NULL = 1,        /* a required pointer is NULL */
  PISA_ERR_SHAPE = 2,       /* L % block != 0, unsupported head_dim/block, sizes <= 0 or too large */
  PISA_ERR_ARG = 3,         /* k or kmax out of range, unknown mode, non-finite scale/lambda */
  PISA_ERR_DTYPE = 4,       /* unknown element type */
  PISA_ERR_WORKSPACE = 5,   /* workspace smaller than pisa_workspace_size() */
  PISA_ERR_HIP = 6          /* a HIP launch or runtime call failed */
} pisa_status;

typedef enum {
  PISA_DTYPE_BF16 = 0,      /* bfloat16 storage, float32 accumulation, bf16 MFMA */
  PISA_DTYPE_FP32 = 1       /* float32 storage and arithmetic throughout */
} pisa_dtype;

typedef enum {
  PISA_MODE_APPROX = 0,     /* PISA: exact S_i + zeroth-order U_i + global first-order correction */
  PISA_MODE_DROP = 1,       /* keep-or-drop block-sparse attention over S_i only */
  PISA_MODE_ZEROTH = 2,     /* exact S_i + zeroth-order U_i, no first-order term */
  PISA_MODE_FIRST = 3       /* exact S_i + zeroth-order U_i + a first-order term per U_i block,
                               alpha_{t,j} (q H_j): the expansion that the global Hbar stands
                               in for (PISA summary, section 2, "Core algorithm": the mixed
                               order avoids these per-block terms because each needs its own
                               d x d matrix) */
} pisa_mode;

/* How pisa_route_attention runs (the selection and the output are the same
 * bit for bit in every form). */
typedef enum {
  PISA_ROUTE_AUTO = 0,         /* IN_KERNEL when idx is NULL or when the call's work items fit
                                  one round of resident workgroups; TWO_LAUNCH otherwise     */
  PISA_ROUTE_IN_KERNEL = 1,    /* each attention workgroup routes its own query block(s)    */
  PISA_ROUTE_TWO_LAUNCH = 2    /* the route kernel writes idx, then the attention kernel reads
                                  it (idx required)                                          */
} pisa_route_form;

typedef enum {
  PISA_NORM_FROBENIUS = 0,  /* M_j = ||H_j - Hbar||_F (entrywise 2-norm)                    */
  PISA_NORM_SPECTRAL = 1    /* M_j = largest singular value of H_j - Hbar                  */
} pisa_norm;

typedef struct {
  int32_t batch;            /* b */
  int32_t heads;            /* h */
  int32_t seq_len;          /* L, multiple of block */
  int32_t head_dim;         /* d: 64 or 128 (keys and values share it) */
  int32_t block;            /* B: 64 or 128 */
  int32_t dtype;            /* pisa_dtype of Q, K, V, O */
  const int32_t* seq_lens;  /* NULLABLE device int32 [batch]: valid length of each sequence in
                               its padded [L] buffer (values clamped to [0, L]).  Tokens at or
                               beyond it are not part of the sequence: the statistics count the
                               n_j = clip(len - j*block, 0, block) valid tokens of block j
                               (centroid = their mean, Hbar = mean over non-empty blocks, M_j
                               = 0 for empty blocks), routing never picks an empty block and
                               pads a row with -1 when fewer than k blocks remain (an empty
                               query block gets an all -1 row), attention skips padding keys,
                               weighs an unselected block by n_j, and writes 0 to the rows of
                               padding queries.  Padding contents are never read into a
                               result.  (Block-sparse notes, sections 4.1 and 8.2: sequences
                               are padded to a block multiple and batches to a common length.)
                               NULL: every sequence has length L.                          */
} pisa_shape;

/* Block statistics, all float32 device arrays owned by the caller. */
typedef struct {
  float* centroid;          /* [b,h,nb,d]   kbar_j = mean of block j's keys                  */
  float* vsum;              /* [b,h,nb,d]   sigma_j = sum of block j's values                */
  float* H;                 /* [b,h,nb,d,d] H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n}, row =
                                            key dim, column = value dim.  NULLABLE: written
                                            only when non-NULL                               */
  float* Hbar;              /* [b,h,d,d]    mean of H_j over the nb blocks of (b,h)          */
  float* M;                 /* [b,h,nb]     M_j = ||H_j - Hbar||_F                           */
  void* packed;             /* NULLABLE, bf16 inputs only: pisa_packed_size() bytes holding
                               bfloat16 copies that the attention kernel streams:
                                 centroid [b,h,nbp,d] | vsum [b,h,nbp,d] | Hbar^T [b,h,d,d]
                               (nbp = nb rounded up to a multiple of block, padding rows 0;
                               Hbar^T row = value dim).  Written by pisa_precompute when
                               non-NULL; read by pisa_attention (PISA mode) when non-NULL,
                               which otherwise converts the fp32 statistics itself.         */
  void* Ht;                 /* NULLABLE, bf16 inputs only: bfloat16 [b,h,nb,d,d] holding H_j^T
                               (row = value dim, column = key dim), b*h*nb*d*d*2 bytes.
                               Written by pisa_precompute when non-NULL; required by
                               PISA_MODE_FIRST with bf16 inputs (fp32 inputs read H).       */
  int32_t m_norm;           /* INPUT to pisa_precompute: pisa_norm used for M_j (the PISA
                               summary, "Covariance-aware routing", writes ||.||_2 of a
                               matrix; FROBENIUS is the default reading).  SPECTRAL with
                               bf16 inputs needs H (it is computed from the stored H_j).    */
} pisa_stats;

/* Version of the library (PISA_VERSION at build time). */
int32_t pisa_version(void);

/* Static text for a status code; never NULL. */
const char* pisa_status_string(int32_t status);

/* Text of the most recent PISA_ERR_* raised on the calling thread (validation
 * message or HIP error string); "" if none.  Thread-local, never NULL. */
const char* pisa_last_error(void);

/* Bytes of device workspace pisa_precompute needs for this shape (0 if the
 * shape is invalid).  The workspace holds deterministic partial sums of H_j:
 * for bf16 inputs one d x d fp32 sum per workgroup range of 4 to 24
 * consecutive blocks of one head (about one round of workgroups on MI355X)
 * plus a copy of Hbar per head in the MFMA fragment order, for fp32 inputs
 * one d x d fp32 matrix per block. */
size_t pisa_workspace_size(const pisa_shape* shape);

/* Bytes of the optional bf16 statistics pack (pisa_stats.packed) for this
 * shape: b*h*(2*nbp*d + d*d)*2 for bf16 inputs, 0 for fp32 or invalid shapes. */
size_t pisa_packed_size(const pisa_shape* shape);

/*
 * pisa_precompute -- block statistics (PISA summary, section 2: "Core
 * algorithm" defines kbar_j, the value sums, H_j and Hbar; "Covariance-aware
 * routing" defines M_j = ||H_j - Hbar||_2, read here as the Frobenius norm;
 * "Hardware implementation" places this computation before the attention).
 *
 *   K, V       [b,h,L,d] of shape->dtype (device, read only)
 *   out        centroid, vsum, Hbar, M required; H, packed and Ht optional (see
 *              pisa_stats; Ht must be NULL for fp32 inputs); out->m_norm selects
 *              the norm of M_j (SPECTRAL: 24 Lanczos steps on (H_j - Hbar)^T
 *              (H_j - Hbar) per block, then the largest eigenvalue of the
 *              tridiagonal by Sturm multisection in fp64)
 *   workspace  device scratch of at least pisa_workspace_size(shape) bytes,
 *              caller-owned; contents on entry are ignored
 *
 * Two streaming passes over K and V (M_j needs the global Hbar); Hbar is
 * reduced in a fixed order, so results are bitwise reproducible.
 */
pisa_status pisa_precompute(const pisa_shape* shape, const void* K, const void* V,
                            const pisa_stats* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * pisa_precompute_noalloc -- pisa_precompute for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results (bit for bit), with the
 * workspace taken from a static device array of the library instead of a
 * caller buffer.  The call itself allocates nothing.
 *
 *   K, V, out  as for pisa_precompute (the caller still owns the inputs and
 *              every output buffer)
 *
 * The static array holds PISA_NOALLOC_SCRATCH_BYTES bytes; each GPU the
 * library runs on holds its own copy until the process ends.  Shapes whose
 * pisa_workspace_size() exceeds it return PISA_ERR_WORKSPACE before anything
 * is launched (use pisa_precompute then).  Run with the device of `stream`
 * current.  Every call on one GPU uses that GPU's array, so calls that overlap
 * on one GPU (different streams, or several host threads) race; calls on one
 * stream are ordered and safe.  Nothing in the array needs clearing between
 * calls: each call overwrites the part it reads.
 */
#define PISA_NOALLOC_SCRATCH_BYTES (64u << 20)
pisa_status pisa_precompute_noalloc(const pisa_shape* shape, const void* K, const void* V,
                                    const pisa_stats* out, void* stream);

/*
 * pisa_route -- covariance-aware top-k routing (PISA summary, section 2,
 * "Covariance-aware routing": the block score combines the attention score
 * with M_j).  Score of query block i and KV block j, computed in float64:
 *
 *     score_ij = scale * qbar_i . kbar_j + lambda * M_j,
 *     qbar_i   = mean of the `block` queries of block i.
 *
 * qbar_i is exact (an fp64 sum of the bf16 or fp32 queries); the dot product
 * is one chain of fp64 FMAs over d in a fixed order, and scale * dot +
 * lambda * M_j one more FMA.  pisa_route_attention computes the same chain,
 * so both select the same blocks.  S_i = the k highest scores; ties go to the
 * lower j.
 *
 *   Q         [b,h,L,d] of shape->dtype (device)
 *   centroid  [b,h,nb,d] float32, M [b,h,nb] float32 (from pisa_precompute)
 *   k         1 <= k <= nb
 *   scale     softmax scale (1/sqrt(d) for standard attention), finite
 *   lambda    weight of M_j, finite
 *   idx       out: int32 [b,h,nb,k], each row strictly ascending
 */
pisa_status pisa_route(const pisa_shape* shape, const void* Q, const float* centroid,
                       const float* M, int32_t k, double scale, double lambda, int32_t* idx,
                       void* stream);

/*
 * pisa_attention -- one fused kernel per query block (PISA summary, section 2,
 * "Hardware implementation": stage 1 exact attention over the selected blocks,
 * stage 2 zeroth-order sweep over the other blocks' centroids and value sums,
 * stage 3 the global first-order correction, all inside one online softmax).
 *
 *   Q, K, V   [b,h,L,d] of shape->dtype (device)
 *   idx       int32 [b,h,nb,kmax]: block ids of S_i; entries < 0 are padding
 *             and are skipped wherever they appear, ids >= nb are skipped, and
 *             an id repeated in a row counts once (S_i is a set).  The exact
 *             blocks are attended in ascending block order, whatever the order
 *             of the row.  Rows may be fully padded (S_i empty).
 *   kmax      row length of idx, 1 <= kmax <= nb
 *   stats     centroid, vsum, Hbar (and packed, when non-NULL) read in APPROX;
 *             centroid, vsum (and packed) in ZEROTH; centroid, vsum, packed and Ht
 *             (bf16) or H (fp32) in FIRST; may be NULL in DROP.  M is not read.
 *   mode      pisa_mode
 *   scale     softmax scale applied to every q_t (exact logits, alpha and the
 *             correction), finite
 *   O         out: [b,h,L,d] of shape->dtype (device)
 *
 * APPROX: o_t = N_t / D_t with, for q = scale * q_t,
 *   N_t = sum_{S_i,n} e^{q k} v + sum_{U_i} e^{q kbar_j} sigma_j + (q Hbar) sum_{U_i} e^{q kbar_j}
 *   D_t = sum_{S_i,n} e^{q k}   + block * sum_{U_i} e^{q kbar_j}
 * (the first-order term adds nothing to D_t: block deviations sum to zero).
 * ZEROTH: the same without the (q Hbar) term.  FIRST: the (q Hbar) term
 * replaced by sum_{U_i} e^{q kbar_j} (q H_j).
 * DROP: softmax over the keys of S_i only; o_t = 0 when S_i is empty.
 */
pisa_status pisa_attention(const pisa_shape* shape, const void* Q, const void* K,
                           const void* V, const int32_t* idx, int32_t kmax,
                           const pisa_stats* stats, int32_t mode, float scale, void* O,
                           void* stream);

/*
 * pisa_attention_split -- pisa_attention with long exact lists split over
 * several workgroups (bf16).  A fixed block mask can give some query blocks
 * far more exact blocks than others (the block-sparse notes' multimodal mask,
 * section 4.2: text rows attend to every block, image rows to a window); one
 * workgroup per query block would then wait on its heaviest rows.  Here a
 * work item (the query block, or the pair of neighbouring query blocks, that
 * one workgroup of pisa_attention takes) whose exact list holds more than
 * max_blocks blocks runs as up to min(32, ceil(min(nb, 2*kmax) / max_blocks))
 * parts on separate workgroups, each over a contiguous share of the exact
 * blocks (the
 * first part also takes the zeroth-order sweep and the correction); the parts
 * leave unnormalised softmax states (acc, running max, denominator) in the
 * workspace and a second kernel merges them:
 *     o = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p.
 * The extra parts of all items are dispatched before the first parts, so the
 * heavy items' parts start first and apart from each other.  The result is
 * pisa_attention's up to the order of floating-point sums (items that run as
 * one part give it bit for bit).
 *
 *   Q, K, V, idx, kmax, stats, scale, O   as for pisa_attention (bf16 only)
 *   mode        PISA_MODE_APPROX, PISA_MODE_DROP or PISA_MODE_ZEROTH
 *   max_blocks  >= 1: most exact blocks of one part
 *   workspace   device scratch of at least
 *               pisa_attention_split_workspace_size(shape, kmax, max_blocks)
 *               bytes, caller-owned; contents on entry are ignored
 *
 * Errors as pisa_attention, and PISA_ERR_DTYPE for fp32 inputs, PISA_ERR_ARG
 * for PISA_MODE_FIRST or max_blocks < 1, PISA_ERR_WORKSPACE for a workspace
 * that is too small.
 */
size_t pisa_attention_split_workspace_size(const pisa_shape* shape, int32_t kmax, int32_t max_blocks);
pisa_status pisa_attention_split(const pisa_shape* shape, const void* Q, const void* K,
                                 const void* V, const int32_t* idx, int32_t kmax,
                                 const pisa_stats* stats, int32_t mode, float scale,
                                 int32_t max_blocks, void* O, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * pisa_route_attention -- routing and attention in one call (PISA summary,
 * section 2, "Covariance-aware routing" for the selection and "Hardware
 * implementation" for the stages).  In the in-kernel form each attention
 * workgroup routes its own query block(s) exactly as pisa_route does (same
 * fp64 pooled query, scores and top-k, so the selection is identical bit for
 * bit) and then runs the attention of pisa_attention on that selection: no
 * idx round trip through memory and no separate routing launch.  The
 * two-launch form runs pisa_route into idx, then pisa_attention on it.  Both
 * give the same selection and the same O bit for bit.  In-kernel routing wins
 * when the call's work items (one per query block, or per pair of query
 * blocks with 64-token blocks) fit one round of resident workgroups: the
 * separate launch and its pass over Q are then a large share of a short call.
 * Over several rounds every workgroup scoring all nb centroids for one query
 * block costs more than the route kernel, which scores eight query blocks per
 * workgroup, so PISA_ROUTE_AUTO switches to two launches there (it needs idx
 * to hold the selection between them).
 *
 *   Q, K, V   [b,h,L,d] bf16 (device)
 *   stats     centroid and M (routing), plus what pisa_attention reads in `mode`
 *   k         blocks per query block, 1 <= k <= nb
 *   lambda    weight of M_j, finite
 *   mode      PISA_MODE_APPROX, PISA_MODE_DROP or PISA_MODE_ZEROTH
 *   scale     the routing score uses it as given (float64); the attention uses
 *             (float)scale, as pisa_attention with that value
 *   idx       NULLABLE out: int32 [b,h,nb,k], the selection, as pisa_route
 *             writes it (ascending, -1 after fewer than k candidates);
 *             required for PISA_ROUTE_TWO_LAUNCH
 *   O         out: [b,h,L,d] bf16 (device)
 *   form      pisa_route_form
 *
 * Errors as pisa_route and pisa_attention, and: PISA_ERR_DTYPE for fp32
 * inputs, PISA_ERR_ARG for PISA_MODE_FIRST or an unknown form, PISA_ERR_NULL
 * for PISA_ROUTE_TWO_LAUNCH without idx, PISA_ERR_SHAPE when the in-kernel
 * form would run with nb above what the kernel's LDS holds for the score rows
 * (d = 128: nb <= 2048 with 128-token blocks, nb <= 1920 with 64-token blocks;
 * d = 64: nb <= 2048 and 960); PISA_ROUTE_AUTO with idx takes two launches
 * there instead.
 */
pisa_status pisa_route_attention(const pisa_shape* shape, const void* Q, const void* K,
                                 const void* V, const pisa_stats* stats, int32_t k, double lambda,
                                 int32_t mode, double scale, int32_t* idx, void* O, int32_t form,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
