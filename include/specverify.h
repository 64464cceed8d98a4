/*
 * libspecverify -- the verification step of speculative decoding on MI355X
 * (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * The operation (chain form) is the acceptance stage of one speculative
 * decoding round: Leviathan et al.'s Algorithm 1 as restated in "LLM
 * speculative decoding close-reading notes 02", section 4 (the full
 * algorithm with uniforms r_i), and in the CMU 15-779 lecture 17 notes,
 * sections 2.3-2.4.  For each request b, with p_i = softmax(target_i / T)
 * and q_i = softmax(draft_i / T) (one temperature for both, close-reading
 * notes section 3):
 *   for i = 0 .. gamma-1: accept draft token x_i iff u[b][i] <= tau_i,
 *       tau_i = 1 if q_i(x_i) <= p_i(x_i) else p_i(x_i) / q_i(x_i);
 *       at the first rejection emit a token drawn from the residual
 *       max(0, p_i - q_i) (normalised) with u[b][gamma], and stop;
 *   if all gamma drafts are accepted, emit a bonus token drawn from
 *       p_gamma with u[b][gamma].
 * Greedy requests (T == 0) accept iff x_i == argmax p_i and emit the argmax
 * at the first mismatch, or argmax p_gamma after gamma matches
 * (close-reading notes section 10).
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers (HIP device memory), row-major
 *    and contiguous, owned by the caller.  The library never allocates or
 *    frees memory on a call.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t, NULL = the
 *    default stream).  The return code reports only what the host can see
 *    before launching: NULL pointers, unsupported shapes, dtype, workspace
 *    size/alignment, misaligned pointers and launch failures.  Outputs are
 *    valid once the stream has been synchronised.
 *  - Bad data inside an otherwise valid call (a draft or node token outside
 *    [0, V), a temperature that is negative, NaN, infinite or positive but
 *    below the smallest normal float (1.17549435e-38), a sampling
 *    request whose uniforms are not all in [0, 1), a malformed parent array,
 *    a tree deeper than max_depth, draft_logits == NULL for a sampling
 *    request) marks that request invalid: its accepted count is -1 and all
 *    its output tokens are -1.  Other requests are unaffected.
 *  - Every wait of one workgroup for another is bounded.  A wait that gives
 *    up (which only a dispatch order the hardware does not use, or
 *    SV_HOOK_SPIN_LIMIT, can cause) makes that request's accepted count
 *    SV_GAVE_UP (-2); its output tokens are then unspecified, and the
 *    workspace may hold stale words: zero it (sv_workspace_clear, or for
 *    spec_verify_chain_noalloc a call with B == 0) before the next call that
 *    uses it.  Other requests keep exact results.
 *  - Logits must be finite or -inf (masked); each row needs at least one
 *    finite entry.  NaN / +inf logits give unspecified tokens.
 *  - Inverse-CDF draws: with weights w_k in vocabulary order, C_k their
 *    running sum and W = C_{V-1}, the token is the smallest k with
 *    C_k > u * W (zero-weight tokens are never drawn).  Argmax ties go to
 *    the lowest index.
 *  - Workspace: a device buffer of at least the size returned by the
 *    matching *_workspace_bytes query, 256-byte aligned.  It must be
 *    zero-filled before its first use (e.g. allocate it zeroed, or call
 *    sv_workspace_clear); every call that completes leaves it zero-filled
 *    again.  One workspace serves one call at a time: calls that may overlap
 *    (different streams) need different workspaces.
 *  - The library is stateless and reentrant; it draws no random numbers.
 *    All randomness is the caller's uniforms (close-reading notes section
 *    11.3: deterministic, per-request random streams).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,        /* a required pointer is NULL */
  SV_ERR_SHAPE = 2,       /* B, gamma, V, N or max_depth outside the limits below */
  SV_ERR_DTYPE = 3,       /* dtype is not one of sv_dtype */
  SV_ERR_WORKSPACE = 4,   /* workspace too small or not 256-byte aligned */
  SV_ERR_ALIGN = 5,       /* a logit pointer is not aligned to its element size */
  SV_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed */
  SV_ERR_SCRATCH = 7      /* spec_verify_chain_noalloc: the shape needs more than SV_CHAIN_SCRATCH_BYTES */
} sv_status;

typedef enum {
  SV_BF16 = 0,            /* logits are bfloat16 (raw 16-bit patterns) */
  SV_F32 = 1              /* logits are IEEE float32 */
} sv_dtype;

/* Accepted count of a request whose bounded wait gave up. */
#define SV_GAVE_UP (-2)

/* Limits checked on the host (SV_ERR_SHAPE otherwise). */
#define SV_MAX_GAMMA 32
#define SV_MAX_BATCH 16384   /* requests per chain call */
#define SV_MAX_VOCAB (1 << 24)
#define SV_MAX_TREE_NODES 1024
#define SV_MAX_TREE_DEPTH 64
#define SV_MAX_TOPK 128          /* top_k of a sampling request in spec_verify_chain_topk */
#define SV_TOPK_MAX_KEPT 256     /* logits a filtered row may keep (k plus ties at the k-th value) */

/* Text for a status code (static storage; never NULL). */
SV_API const char* sv_status_string(int status);

/* Library version as "major.minor.patch" (static storage). */
SV_API const char* sv_version(void);

/*
 * Zero-fill `bytes` of a workspace on `hip_stream` with a fill kernel (safe
 * under stream capture).  Only needed after an aborted call or for a new
 * buffer that was not allocated zeroed.
 */
SV_API int sv_workspace_clear(void* workspace, size_t bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Chain verification.
 *
 * target_logits    [B][gamma+1][V]  dtype   target rows p_1 .. p_{gamma+1}
 * draft_logits     [B][gamma][V]    dtype   draft rows q_1 .. q_gamma; may be
 *                                           NULL if every request is greedy
 * draft_tokens     [B][gamma]       int32   x_1 .. x_gamma (may be NULL if gamma == 0)
 * uniforms         [B][gamma+1]     float   u[b][i], i < gamma: accept test of
 *                                           draft i; u[b][gamma]: the final
 *                                           draw (residual or bonus).  Read
 *                                           only for sampling requests.
 * temperature      [B]              float   T > 0 sampling, T == 0 greedy
 * out_tokens       [B][gamma+1]     int32   emitted tokens x_1..x_n, then the
 *                                           resampled/bonus/argmax token; the
 *                                           rest is -1
 * out_num_accepted [B]              int32   n in [0, gamma] (n + 1 tokens are
 *                                           emitted; the caller rolls back
 *                                           gamma - n cached positions), -1
 *                                           (invalid request) or SV_GAVE_UP
 * Limits: 0 <= B <= SV_MAX_BATCH (B == 0 is a no-op), 0 <= gamma <= SV_MAX_GAMMA,
 *         1 <= V <= SV_MAX_VOCAB.
 * Returns an sv_status.
 * ---------------------------------------------------------------------- */
SV_API size_t sv_chain_workspace_bytes(int B, int gamma, int V, int dtype);

SV_API int spec_verify_chain(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, int B, int gamma, int V, int dtype,
                      int32_t* out_tokens, int32_t* out_num_accepted,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Chain verification that allocates nothing and takes no workspace.
 *
 * For callers that cannot allocate device memory or size a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Arguments, results and error behaviour are those of
 * spec_verify_chain, which this call runs with the same kernels; the
 * workspace is instead a static device array of SV_CHAIN_SCRATCH_BYTES that
 * the library keeps on each GPU it runs on until the process ends.  The
 * first call on a GPU zero-fills that array with a fill kernel on
 * `hip_stream`; every call that completes leaves it zero again.
 * A shape whose workspace (sv_chain_workspace_bytes) exceeds
 * SV_CHAIN_SCRATCH_BYTES returns SV_ERR_SCRATCH without launching anything.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams without ordering between them) race and give
 * unspecified results.  A call with B == 0 launches only the zero-fill of
 * the array on `hip_stream`: that is how to reset it after a call that did
 * not complete (a bounded wait that gave up, which only a dispatch order the
 * hardware does not use can cause; its requests report -1).
 * ---------------------------------------------------------------------- */
#define SV_CHAIN_SCRATCH_BYTES (8u << 20)

SV_API int spec_verify_chain_noalloc(const void* target_logits, const void* draft_logits,
                              const int32_t* draft_tokens, const float* uniforms,
                              const float* temperature, int B, int gamma, int V, int dtype,
                              int32_t* out_tokens, int32_t* out_num_accepted, void* hip_stream);

/* ------------------------------------------------------------------------
 * Chain verification under a general consistent filter: top-k and/or top-p
 * over the whole vocabulary (close-reading notes 02, section 5.4: a decoding
 * rule applied alike to p and q keeps the method exact for the filtered
 * target).
 *
 * Every target and draft row of a sampling request is cut alike before the
 * temperature softmax, and the logits below its cut count as -inf:
 *  - top-k: the cut is the row's min(k, V)-th largest logit (every logit
 *    equal to it stays);
 *  - top-p: over what top-k kept (the whole row without top-k), with r the
 *    temperature softmax of those logits, the cut rises to the largest kept
 *    logit v whose mass, the sum of r over the kept logits >= v, reaches p.
 * p' and q' are the softmax of the cut rows; the test, the residual draw
 * from norm(max(0, p' - q')) and the bonus draw from p' are those of
 * spec_verify_chain, so the draft tokens must come from the cut q'.  A draft
 * token below its draft row's cut has q' = 0 and is accepted.  Greedy
 * requests (T == 0) ignore both filters.  Unlike spec_verify_chain_topk, no
 * limit applies to k or to the number of logits a row keeps.
 *
 * The arguments are spec_verify_chain's, plus
 * top_k   [B]  int32  optional (NULL: no top-k): k >= 1 of each request;
 *                     k >= V keeps the whole row
 * top_p   [B]  float  optional (NULL: no top-p): p in (0, 1]; 1 cuts nothing
 * and draft_logits is required whenever gamma > 0.  A sampling request with
 * k < 1 or p outside (0, 1] is invalid (count -1, tokens -1).
 * Precision: bf16 rows are cut exactly: their values are counted once and
 * every distinct value's mass is count * 2^((v - max) / T) in fp64.  fp32
 * rows take fp32 exponentials per logit on the scale of the row maximum,
 * summed in fp64, so an fp32 cut can differ from an exact one only where p
 * lies within about 1e-7 of the mass at the cut.  Work: one launch finds the
 * cuts of all rows of the sampling requests (bf16: one read of each row;
 * fp32: one read from HBM, then one pass from the caches per further digit
 * of each search), then the chain launch of spec_verify_chain with the cuts
 * applied wherever a row is read; a bf16 search also leaves each cut row's
 * maximum and kept mass (fp64), so the chain launch does not read those rows
 * again except where a draw needs them.  Rows are searched in groups of at most
 * 1024 (B times 2 gamma + 1 rows in all); a group of bf16 rows also holds
 * at most 256 MiB of counts (about 272 KiB per row at V = 128256).  The
 * workspace comes from sv_chain_filtered_workspace_bytes (spec_verify_chain's
 * plus that search area), zero-filled before the first call and left
 * zero-filled by every call.  Returns an sv_status.
 * ---------------------------------------------------------------------- */
SV_API size_t sv_chain_filtered_workspace_bytes(int B, int gamma, int V, int dtype);

SV_API int spec_verify_chain_filtered(const void* target_logits, const void* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms,
                               const float* temperature, const int32_t* top_k, const float* top_p,
                               int B, int gamma, int V, int dtype, int32_t* out_tokens,
                               int32_t* out_num_accepted, void* workspace, size_t workspace_bytes,
                               void* hip_stream);

/* ------------------------------------------------------------------------
 * Chain verification with a scheduling hint (close-reading notes 02,
 * section 4, as spec_verify_chain).
 *
 * sampling_hint  [B]  uint8, HOST memory, or NULL: nonzero where the caller
 *                     expects request b to sample (temperature[b] > 0).
 * The hint changes only the order in which the work is laid out on the GPU:
 * the requests hinted to sample stream first, their draws then run while the
 * other requests' rows stream.  Results are those of spec_verify_chain for
 * any hint (a wrong hint costs time, not correctness); the kernel still takes
 * every request's mode from its temperature.  The hint is read on the host
 * during the call and may be freed when it returns.  It is used for batches of
 * at most SV_HINT_MAX_BATCH requests and ignored otherwise (as is NULL).
 * Everything else as spec_verify_chain (same workspace query).
 * ---------------------------------------------------------------------- */
#define SV_HINT_MAX_BATCH 256

SV_API int spec_verify_chain_hinted(const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* uniforms,
                             const float* temperature, const uint8_t* sampling_hint, int B, int gamma,
                             int V, int dtype, int32_t* out_tokens, int32_t* out_num_accepted,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Chain verification under a consistent top-k filter.
 *
 * Every target and draft row of a sampling request is filtered alike before
 * the temperature softmax: the logits >= the row's min(k, V)-th largest
 * value are kept (so every logit equal to that value stays; a row may keep
 * more than k) and the rest count as -inf.  p' and q' are the softmax of the
 * filtered rows; the test, the residual draw from norm(max(0, p' - q')) and
 * the bonus draw from p' are those of spec_verify_chain.  Applying the same
 * rule to both sides keeps the method exact for the filtered target (the
 * close-reading notes 02, section 5.4), so the draft tokens must have been
 * drawn from the filtered q'.  A draft token below its draft row's threshold
 * has q' = 0 and is accepted (tau = 1 when q' <= p'), as in the unfiltered
 * call.  Greedy requests (T == 0) ignore top_k: the argmax is always kept.
 *
 * The arguments are spec_verify_chain's, plus
 * top_k            [B]   int32   k of each request, 1 <= k <= SV_MAX_TOPK for
 *                                a sampling request (k >= V keeps the whole
 *                                row, which then must fit the kept limit)
 * top_p            [B]   float   optional (NULL: no top-p): p in (0, 1] of each
 *                                request.  After the top-k filter, every row
 *                                is filtered again, alike on both sides: its
 *                                threshold rises to the largest kept logit v
 *                                whose mass -- the temperature softmax over
 *                                the kept logits, summed over those >= v --
 *                                reaches p, and the logits >= v stay.  p = 1
 *                                keeps the top-k set.
 * and draft_logits is required whenever gamma > 0.  A sampling request is
 * invalid (count -1, tokens -1) if its k is outside [1, SV_MAX_TOPK], its p
 * (when given) outside (0, 1], or any of its rows keeps more than
 * SV_TOPK_MAX_KEPT logits after the top-k filter; the other invalid
 * inputs are those of spec_verify_chain.  Logits are finite or -inf.
 * Work: one workgroup per row read finds the row's threshold and kept
 * logits (a sampling row is visited twice, the second visit mostly through
 * the caches, and more often only when more than 512 logits reach the first
 * bound); the test and the draws then touch only the kept logits.
 * Limits as spec_verify_chain.  Returns an sv_status.
 * ---------------------------------------------------------------------- */
SV_API size_t sv_chain_topk_workspace_bytes(int B, int gamma, int V, int dtype);

SV_API int spec_verify_chain_topk(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, const int32_t* top_k, const float* top_p,
                      int B, int gamma, int V,
                      int dtype, int32_t* out_tokens, int32_t* out_num_accepted,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Ragged chain verification: a draft length per request in one call, and the
 * acceptance probability of every test taken.
 *
 * The arrays keep spec_verify_chain's layout, padded to gamma (the longest
 * round).  Request b drafts g = gammas[b] tokens: it is exactly the round of
 * g drafts -- tests on draft_tokens[b][0..g-1] with uniforms[b][0..g-1]
 * against target and draft rows 0..g-1, then the residual draw or the bonus
 * draw from target row g, with uniforms[b][g].  Nothing past g is read (rows,
 * tokens or uniforms); out_tokens[b] holds n + 1 tokens then -1 up to
 * gamma + 1 entries.  A length outside [0, gamma] makes the request invalid.
 * The rows past a request's length are skipped by the streaming, so a batch
 * of short rounds reads only its own rows.
 *
 * gammas           [B]         int32  g of each request, in [0, gamma];
 *                                     NULL means every request drafts gamma
 * out_accept_prob  [B][gamma]  float  optional (NULL): tau of each test taken,
 *                                     i.e. positions 0..n (the rejected one
 *                                     included), -1 for the rest.  tau =
 *                                     min(1, p(x)/q(x)) for sampling, 1 or 0
 *                                     (draft == argmax) for greedy.  Over
 *                                     x ~ q, tau averages to sum_k min(p, q):
 *                                     the mean of a round's taus is an
 *                                     unbiased acceptance-rate estimate for
 *                                     choosing the next round's length
 *                                     (lecture 17 notes, section 2.3).
 * Everything else as spec_verify_chain (same workspace query); draft_logits
 * is required when gamma > 0.
 * ---------------------------------------------------------------------- */
SV_API int spec_verify_chain_ragged(const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* uniforms,
                             const float* temperature, const int32_t* gammas, int B, int gamma,
                             int V, int dtype, int32_t* out_tokens, int32_t* out_num_accepted,
                             float* out_accept_prob, void* workspace, size_t workspace_bytes,
                             void* hip_stream);

/* ------------------------------------------------------------------------
 * Token-tree verification (CMU 15-779 lecture 17 notes, section 4.4
 * VerifyGreedy for T == 0 and section 4.5 naive sampling for T > 0).
 *
 * Each request holds a token tree of N nodes linearised depth-first
 * (ancestors first, section 4.3); node 0 is the root, the last verified
 * token.  From the root: pick c = argmax p_n (greedy) or draw c from p_n with
 * u[b][n] (naive sampling); if a child of n carries c (children in index
 * order, the lowest index wins on duplicate tokens) accept that child and
 * continue from it, otherwise emit c and stop.  At a leaf c is the extra
 * token.
 *
 * target_logits  [B][N][V]  dtype  one target row per node
 * node_tokens    [B][N]     int32  token of each node (entry 0 ignored)
 * parents        [B][N]     int32  parents[b][0] == -1, 0 <= parents[b][i] < i
 * uniforms       [B][N]     float  u[b][n] for the draw at node n (sampling only)
 * temperature    [B]        float  0 greedy descent, > 0 naive sampling
 * max_depth                        every node's depth must be <= max_depth
 * out_tokens     [B][max_depth+1] int32  accepted node tokens, then the extra
 *                                        token; -1 padded
 * out_path_nodes [B][max_depth+1] int32  accepted node ids (their positions in
 *                                        the linearised KV cache); -1 padded
 * out_num_accepted [B]            int32  number of accepted nodes, -1 (invalid) or SV_GAVE_UP
 * Limits: B >= 0, 1 <= N <= SV_MAX_TREE_NODES, 1 <= V <= SV_MAX_VOCAB,
 *         0 <= max_depth <= SV_MAX_TREE_DEPTH.
 * ---------------------------------------------------------------------- */
SV_API size_t sv_tree_workspace_bytes(int B, int N, int V, int dtype);

SV_API int spec_verify_tree(const void* target_logits, const int32_t* node_tokens,
                     const int32_t* parents, const float* uniforms,
                     const float* temperature, int B, int N, int V, int max_depth,
                     int dtype, int32_t* out_tokens, int32_t* out_path_nodes,
                     int32_t* out_num_accepted, void* workspace,
                     size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Token-tree verification by multi-step speculative sampling, MSS (CMU
 * 15-779 lecture 17 notes, section 4.5: VerifyStochastic, unbiased when the
 * children are sampled without replacement and q_j is renormalised, and
 * exercises 6-7; section 4.4 VerifyGreedy for T == 0).
 *
 * Node n's children were drawn without replacement from
 * q_n = softmax(draft_logits[b][n] / T).  At node n, with p_n =
 * softmax(target_logits[b][n] / T) and the residual r = p_n: the children are
 * tested in index order, skipping a child whose token an earlier sibling
 * already carries.  Child j (token x) is tested against q_j = q_n without the
 * tokens tested before, renormalised: accept iff accept_uniforms[b][j] <= tau,
 * tau = 1 if q_j(x) <= r(x) else r(x)/q_j(x).  An accepted child becomes the
 * next node.  A rejection sets r = norm(max(0, r - q_j)).  If every child is
 * rejected, or n has none, the node emits a token drawn from r (p_n for a
 * leaf) with draw_uniforms[b][n] and the descent stops.  Two degenerate cases
 * only arise through rounding or impossible draws.  A rejection that leaves r
 * without mass draws from p_n instead.  Once the tested tokens hold all of
 * q_n's mass, later children are not tested.  T == 0 is greedy descent, as in
 * spec_verify_tree; draft logits and uniforms are then not read.
 *
 * target_logits   [B][N][V]  dtype  target row of each node
 * draft_logits    [B][N][V]  dtype  draft row of each node (rows of leaves are
 *                                   never read)
 * node_tokens     [B][N]     int32  as spec_verify_tree
 * parents         [B][N]     int32  as spec_verify_tree
 * accept_uniforms [B][N]     float  entry j: the test of node j (entry 0 unused)
 * draw_uniforms   [B][N]     float  entry n: the draw when the descent stops at n
 * temperature     [B]        float  0 greedy, > 0 MSS
 * out_tokens, out_path_nodes, out_num_accepted: as spec_verify_tree.
 * A request is invalid (-1) if any node has more than 64 children, or, for
 * a sampling request, if accept_uniforms[b][1..N-1] or draw_uniforms[b] leave
 * [0, 1).
 * Limits: as spec_verify_tree, and V <= 524288 with B * (ceil(V / 2048) + 1)
 * <= 2^20 (SV_ERR_SHAPE otherwise; the workspace query then returns 0).
 * ---------------------------------------------------------------------- */
SV_API size_t sv_tree_mss_workspace_bytes(int B, int N, int V, int dtype);

SV_API int spec_verify_tree_mss(const void* target_logits, const void* draft_logits,
                         const int32_t* node_tokens, const int32_t* parents,
                         const float* accept_uniforms, const float* draw_uniforms,
                         const float* temperature, int B, int N, int V, int max_depth,
                         int dtype, int32_t* out_tokens, int32_t* out_path_nodes,
                         int32_t* out_num_accepted, void* workspace,
                         size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Tree attention mask and depth positions: the inputs of the one forward
 * pass that scores a whole token tree (CMU 15-779 lecture 17 notes, section
 * 4.3: a depth-first linearised tree, a topology-aware causal mask under
 * which each node sees only itself and its ancestors, and positions by
 * depth; exercise 5).
 *
 * parents        [B][N]        int32   parents[b][0] == -1, 0 <= parents[b][i] < i
 *                                      (any order with parents first; depth-first
 *                                      is the one the verifier's KV layout uses)
 * out_mask       [B][N][words] uint64  words = ceil(N / 64); bit (j % 64) of word
 *                                      j / 64 of row i is 1 iff node j is node i
 *                                      or one of its ancestors (the root
 *                                      included).  Byte for byte this is each
 *                                      row's bits packed little-endian, bit j of
 *                                      the row at byte j / 8, bit j % 8.  The
 *                                      verified prefix before the root is
 *                                      visible to every row and not included.
 * out_depth      [B][N]        int32   edges from the root (root 0); the position
 *                                      id of node i is the root's position plus
 *                                      out_depth[b][i]
 * out_tree_depth [B]           int32   deepest node's depth; may be NULL
 * A request whose parent array is malformed, or with a node deeper than
 * max_depth, gets all-zero rows and -1 depths (and tree depth -1).
 * Limits: B >= 0 (B == 0 is a no-op), 1 <= N <= SV_MAX_TREE_NODES,
 *         0 <= max_depth <= SV_MAX_TREE_DEPTH; out_mask 8-byte aligned
 *         (SV_ERR_ALIGN otherwise).  No workspace.
 * ---------------------------------------------------------------------- */
SV_API int spec_tree_mask(const int32_t* parents, int B, int N, int max_depth,
                   uint64_t* out_mask, int32_t* out_depth, int32_t* out_tree_depth,
                   void* hip_stream);

/* ------------------------------------------------------------------------
 * Debug probabilities for every draft position i < gamma, whether or not
 * verification would reach it:
 *   p_at_draft[b][i]    = p_i(x_i)
 *   q_at_draft[b][i]    = q_i(x_i)
 *   residual_mass[b][i] = sum_k max(0, p_i(k) - q_i(k)) = 1 - sum_k min(p_i, q_i)
 *                         (close-reading notes section 5.1; lecture 17 notes
 *                         section 2.3, acceptance rate = 1 - this)
 *   target_lse[b][i]    = log sum_k exp(target_i(k) / T), i <= gamma (optional, may be NULL)
 *   draft_lse[b][i]     = log sum_k exp(draft_i(k) / T), i < gamma  (optional, may be NULL)
 * Requests with T == 0 or an invalid T produce NaN; a token outside [0, V)
 * gives NaN p/q at that position.  Arrays are float32, [B][gamma] unless
 * stated.  Limits as for spec_verify_chain.
 * ---------------------------------------------------------------------- */
SV_API size_t sv_probs_workspace_bytes(int B, int gamma, int V, int dtype);

SV_API int spec_probs_debug(const void* target_logits, const void* draft_logits,
                     const int32_t* draft_tokens, const float* temperature,
                     int B, int gamma, int V, int dtype,
                     float* p_at_draft, float* q_at_draft, float* residual_mass,
                     float* target_lse, float* draft_lse,
                     void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Kernel timing, for benchmarks.  While a timing session is open, every
 * kernel the library launches carries a pair of HIP events attached to its
 * dispatch (hipExtLaunchKernel), so the recorded time is the kernel's own
 * execution with no extra packets on the stream.
 *
 * sv_timing_begin(capacity)  creates `capacity` event pairs and opens a
 *     session (host call; not while the stream is being captured).  Launches
 *     beyond the capacity run untimed.  SV_ERR_SHAPE if capacity is not in
 *     [1, 1 << 20], SV_ERR_HIP if event creation fails.
 * sv_timing_end(total_ms, launches, n)  waits for every recorded launch,
 *     ADDS each kernel's summed milliseconds and launch count into
 *     total_ms[k] / launches[k] for k < n (indexed by sv_kernel; either
 *     array may be NULL), destroys the events and closes the session.
 *     Returns SV_ERR_HIP if an event could not be read.
 * One session at a time per process; calls from several host threads during
 * a session are recorded in launch order.
 * ---------------------------------------------------------------------- */
typedef enum {
  SV_K_CHAIN_VERIFY = 0,      /* chain: row statistics, accept tests and draws in one launch */
  SV_K_CHAIN_STREAM = 1,      /* chain, very large shapes: row statistics in a launch of their own */
  SV_K_CHAIN_DECIDE = 2,      /* chain, very large shapes: accept tests in a launch of their own */
  SV_K_CHAIN_UNITS = 3,       /* chain, very large shapes: draw sums and draws in a launch of their own */
  SV_K_TREE_INIT = 4,
  SV_K_TREE_NODE_PASS = 5,
  SV_K_TREE_CHOOSE = 6,
  SV_K_PROBS_ROW_STATS = 7,
  SV_K_PROBS_RESIDUAL = 8,
  SV_K_PROBS_FINALIZE = 9,
  SV_K_WORKSPACE_CLEAR = 10,
  SV_K_TREE_VERIFY = 11,      /* tree: every depth step of every request in one launch */
  SV_K_TREE_MASK = 12,        /* tree attention mask and depth positions */
  SV_K_TREE_MSS = 13,         /* tree: multi-step speculative sampling, one launch */
  SV_K_TOPK_ROWS = 14,        /* chain under top-k: each row's max, threshold and kept logits */
  SV_K_TOPK_DECIDE = 15,      /* chain under top-k: accept tests and draws over the kept logits */
  SV_K_FILTER_ROWS = 16,      /* filtered chain: the top-k / top-p cut of every sampling row */
  SV_K_COUNT = 17
} sv_kernel;

/* Name of a kernel id (static storage; "unknown" outside [0, SV_K_COUNT)). */
SV_API const char* sv_kernel_name(int kernel);

SV_API int sv_timing_begin(int capacity);

SV_API int sv_timing_end(double* total_ms, int* launches, int n);

/* ------------------------------------------------------------------------
 * Test controls.  For tests only: they force paths that ordinary inputs of a
 * test's size never take -- the multi-launch forms that very large shapes
 * use, and give-ups of the bounded waits (SV_GAVE_UP) with every kernel still
 * running to its end.  A control is process-wide and read by every later
 * call on any thread; value 0 restores the default.  Production code never
 * sets one.  Returns SV_ERR_SHAPE for an unknown control or a negative value.
 * ---------------------------------------------------------------------- */
typedef enum {
  SV_HOOK_CHAIN_GRID_CAP = 0, /* > 0: chain calls use the three-launch form, grids capped at this many workgroups */
  SV_HOOK_CHAIN_SPLIT = 1,    /* != 0: chain calls use the three-launch form */
  SV_HOOK_TREE_SPLIT = 2,     /* != 0: spec_verify_tree uses its launch-per-step form */
  SV_HOOK_SPIN_LIMIT = 3,     /* > 0: each bounded wait of the chain and tree kernels gives up after this many polls */
  SV_HOOK_TREE_ALL_NODES = 4, /* != 0: spec_verify_tree reduces every node's row first, then descends (the
                                 all-nodes design, lecture 17 notes section 4.3, kept to be measured against
                                 path descent); sv_tree_workspace_bytes then sizes its B*N*chunks partials */
  SV_HOOK_COUNT = 5
} sv_hook;

SV_API int sv_set_test_hook(int hook, long long value);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
