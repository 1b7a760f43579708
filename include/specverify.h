/* libspecverify -- speculative-decoding verification on AMD Instinct MI355X (gfx950).
 *
 * The library implements the acceptance step of speculative decoding: given the
 * target model's logits at the verified positions and the draft's logits (or a
 * candidate tree), it finds the longest acceptable draft prefix and emits one
 * more token from the target.
 *
 * Sources (web pages; sections named as on the pages):
 *  [S-SD]  "Accelerating Sonar through speculation", section "Spekulatives Decoding":
 *          each candidate prefix is scored, the longest one above the acceptance
 *          threshold is kept, and a draft of n tokens yields up to n+1 tokens;
 *          phases "Akzeptanz" and "Zielgenerierung": the target logits at the first
 *          mismatch, or after the last draft, are sampled for one more token.
 *  [S-ZE]  same page, section "Ziel-Entwurf": the sampler finds the accepted length
 *          by comparing the full draft and target distributions, then samples the
 *          target's extra logits row.
 *  [S-MTP] same page, section "MTP": all schemes share sampling and logit
 *          processing; section "MTP-Zeitplan für ein einzelnes Token": the target
 *          verifies 2*D tokens for a decode batch of D (k = 1).
 *  [S-INF] same page, section "Inferenz mit spekulativem Decoding": the accepted
 *          count sets the next sequence length; the library never synchronises
 *          with the host, so results stay on the device.
 *  [S-MTPZ] section "MTP-Zeitplan für ein einzelnes Token", further: after the
 *          acceptance a kernel inserts the next target token into the target's input
 *          tokens shifted one place left (section "MTP": the draft's token buffer is
 *          shifted one place left against the target's hidden states), so that no
 *          CPU-GPU synchronisation follows.
 *  [M-3]   "Speculative-Decoding, LLM推理的加速 / Medusa 方法阅读", section 三
 *          (Attention Tree): tree nodes get logits from one pass; the sampler's token
 *          at the root is looked up among level-1 candidates and followed level by
 *          level while a child matches. The tree is flattened into one sequence whose
 *          attention mask lets a token see only itself and its ancestors, as a causal
 *          mask does along a chain.
 *  [M-4]   same page, section 四 (optimized tree construction): with per-head, per-rank
 *          accuracies a_k^(i) taken as independent, a node's contribution to the
 *          expected accepted length is the product of the accuracies on its path;
 *          for a node budget, nodes are added greedily, largest contribution first.
 * The acceptance rule is the one of the method the Sonar page cites (Leviathan et
 * al.) but does not print: accept draft token x at position i iff
 * u_i < p_t,i(x) / p_d,i(x); after the first rejection at L, draw from
 * max(0, p_t,L - p_d,L) renormalised; if all k drafts pass, draw from p_t,k.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers unless stated otherwise; the caller
 *    owns every buffer. The library allocates nothing, frees nothing and keeps no
 *    pointer after returning.
 *  - Logits are row-major with contiguous rows of V elements in the stated dtype.
 *    Rows whose start is 16-byte aligned take the vector path; other rows are
 *    handled element by element (correct, slower).
 *  - softmax at temperature T: p(v) = exp(x_v / T) / sum_w exp(x_w / T). Greedy
 *    mode ignores T and the uniforms and uses argmax (largest value, lowest index
 *    on ties, NaN entries never chosen).
 *  - Inverse CDF draw with uniform u over weights w: the smallest v whose
 *    cumulative weight exceeds u * sum(w).
 *  - Calls only enqueue work on `stream` and never synchronise; outputs are valid
 *    once the stream reaches that point. Concurrent calls need distinct workspaces.
 *  - Workspace: device memory of at least the size the *_workspace function
 *    returns, 256-byte aligned, zero-filled before its first use (for instance with
 *    spec_workspace_clear). The waves of one launch pass results to each other
 *    through records and atomic arrival counters in it; every call tags its
 *    records with a fresh value, each record is cleared by the wave that reads it
 *    last and each counter by the wave that completes it, so a call that ends
 *    without SV_ERR_INTERNAL leaves the workspace all zeros again, ready for any
 *    entry point and shape. One workspace serves one launch at a time; after
 *    SV_ERR_INTERNAL, clear it again before reuse.
 *  - Errors detectable on the host return a non-zero status before anything is
 *    enqueued. Data errors seen on the device set bits in err_flags (if given) and
 *    give that sequence accept_len = -1 and -1 tokens:
 *      bit0 SV_ERR_TOKEN   a draft or candidate token outside [0, V)
 *      bit1 SV_ERR_ROW     a row with no entry above -inf, or (stochastic) a
 *                          non-finite softmax normaliser (NaN or +inf logits)
 *      bit2 SV_ERR_TREE    parent[0] != -1, parent[i] outside [0, i), or a node
 *                          deeper than max_depth
 *      bit3 SV_ERR_INTERNAL a wait between workgroups of the launch gave up (after
 *                          0.25 s, see spec_set_wait_limit: only if the GPU did
 *                          not run the launch's workgroups in dispatch order, or a
 *                          concurrent call shared the workspace); outputs are not
 *                          valid, and a wait that gave up can also leave other
 *                          sequences of that launch unwritten (in a stochastic
 *                          linear launch of many sequences, possibly with no bit
 *                          set anywhere: a caller that must detect this fills
 *                          accept_len with a sentinel before the call)
 *      bit4 SV_ERR_CAPACITY  (commit) the history buffer cannot take the new tokens
 *      bit5 SV_ERR_UNVERIFIED (commit) the sequence's verification reported an error
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sv_stream_t; /* the same type as hipStream_t; NULL = default stream */

/* The enums below are int-sized in both languages. In C++ they get int as their
 * fixed underlying type, so that any int a C caller passes (an unknown mode or
 * dtype, which the calls reject) is a valid value rather than undefined behaviour. */
#ifdef __cplusplus
#define SV_ENUM_INT : int
#else
#define SV_ENUM_INT
#endif

typedef enum SV_ENUM_INT {
  SV_OK = 0,
  SV_EINVAL = 1,      /* bad size, NULL required pointer, bad temperature or mode */
  SV_EDTYPE = 2,      /* unknown dtype */
  SV_EWORKSPACE = 3,  /* workspace NULL, misaligned or too small */
  SV_EHIP = 4,        /* a HIP launch failed */
  SV_ELIMIT = 5       /* shape beyond a documented limit */
} sv_status;

typedef enum SV_ENUM_INT { SV_GREEDY = 0, SV_STOCHASTIC = 1 } sv_mode;
typedef enum SV_ENUM_INT { SV_F32 = 0, SV_BF16 = 1, SV_F16 = 2 } sv_dtype;

enum { SV_ERR_TOKEN = 1, SV_ERR_ROW = 2, SV_ERR_TREE = 4, SV_ERR_INTERNAL = 8,
       SV_ERR_CAPACITY = 16, SV_ERR_UNVERIFIED = 32 };

/* Limits: k <= SV_MAX_K drafts per sequence; n_nodes <= SV_MAX_TREE_NODES; a row
 * holds at most SV_MAX_ROW_BYTES of logits (V <= 1048576 for bf16/fp16, 524288 for
 * fp32). Larger shapes return SV_ELIMIT. */
enum { SV_MAX_K = 31, SV_MAX_TREE_NODES = 16384, SV_MAX_ROW_BYTES = 2097152 };

/* ---------------------------------------------------------------- linear drafts
 * [S-SD], [S-ZE], [S-MTP]. B sequences, k draft tokens each (k = 0 is plain
 * sampling from target row 0).
 *   target_logits  [B][k+1][V]  target logits at the k draft positions and after them
 *   draft_logits   [B][k][V]    draft logits; read in SV_STOCHASTIC only (may be NULL in greedy)
 *   draft_tokens   [B][k]       int32 draft tokens (may be NULL when k = 0)
 *   uniforms       [B][k+1]     float in [0,1): u[b][i<k] decides draft i, u[b][k] is the
 *                               final draw; SV_STOCHASTIC only (may be NULL in greedy)
 * Outputs:
 *   accept_len     [B]          L in [0,k], or -1 on a data error
 *   out_tokens     [B][k+1]     the L accepted drafts, then the target's token, then -1
 *   p_target, p_draft [B][k]    optional (NULL to skip), SV_STOCHASTIC only: p_t,i(x_i) and
 *                               p_d,i(x_i) for every i < k (NaN on a data error)
 *   err_flags      [B]          optional data-error bits (see above)
 * Greedy mode accepts x_i iff x_i = argmax(target row i) and emits argmax(target row L).
 * One kernel launch; every logit row is read once, and in SV_STOCHASTIC rows t_L and
 * d_L of sequences that rejected a draft (L < k) are read a second time for the
 * residual draw ([S-ZE]).
 */
size_t spec_verify_linear_workspace(int64_t B, int64_t k, int64_t V, sv_dtype dtype, sv_mode mode);

sv_status spec_verify_linear(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                             sv_dtype dtype, const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* uniforms,
                             int32_t* accept_len, int32_t* out_tokens, float* p_target,
                             float* p_draft, int32_t* err_flags, void* workspace,
                             size_t workspace_bytes, sv_stream_t stream);

/* ---------------------------------------------------------------- candidate trees
 * [M-3]; "Accelerating Sonar through speculation", section "EAGLE" (keep the longest
 * suitable candidate sequence and append one target token).
 *   n_nodes        nodes per tree including the root (node 0)
 *   parent         [n_nodes] shared by all trees when parent_batch_stride = 0, else
 *                  parent + b * parent_batch_stride; parent[0] = -1, 0 <= parent[i] < i
 *   cand_tokens    [B][n_nodes] int32 candidate token of each node (entry 0 ignored)
 *   target_logits  [B][n_nodes][V] target logits at every node
 *   uniforms       [B][n_nodes] one draw per node; SV_STOCHASTIC only
 *   max_depth      caller's bound on the tree depth; sizes path_nodes / out_tokens
 * Each node n gets token y_n: argmax of its row (greedy) or the inverse-CDF draw
 * from softmax(row / T) with u[b][n] (stochastic). Node i is accepted iff its parent
 * is accepted and cand_i = y_parent(i); the root always is. The accepted node of
 * greatest depth (lowest index on ties) ends the path.
 * Outputs:
 *   accept_len     [B]                 depth of that node, or -1 on a data error
 *   path_nodes     [B][max_depth]      its path from level 1 down, then -1
 *   out_tokens     [B][max_depth + 1]  the path's candidate tokens, then y of the last
 *                                      node, then -1
 *   err_flags      [B]                 optional data-error bits
 */
size_t spec_verify_tree_workspace(int64_t B, int64_t n_nodes, int64_t V, sv_dtype dtype,
                                  sv_mode mode);

sv_status spec_verify_tree(sv_mode mode, float temperature, int64_t B, int64_t n_nodes, int64_t V,
                           sv_dtype dtype, const int32_t* parent, int64_t parent_batch_stride,
                           const int32_t* cand_tokens, const void* target_logits,
                           const float* uniforms, int64_t max_depth, int32_t* accept_len,
                           int32_t* path_nodes, int32_t* out_tokens, int32_t* err_flags,
                           void* workspace, size_t workspace_bytes, sv_stream_t stream);

/* ---------------------------------------------------------------- typical acceptance (trees)
 * Named by the workload description of the full Medusa tree, NOT defined on the source
 * pages: the rule below is this library's reading, and its constants are the caller's.
 * Same arguments and outputs as spec_verify_tree (stochastic, at temperature T, same
 * workspace size), plus epsilon, delta >= 0. With p_n = softmax(row n / T) and H_n its
 * entropy in nats, node i passes iff p_parent(i)(cand_i) > min(epsilon, delta * exp(-H_parent(i)));
 * node i is accepted iff it passes and its parent is accepted (the root always is).
 * The deepest accepted node (lowest index on ties) ends the path; the final token is the
 * inverse-CDF draw from p_last with u[b][last]. Two kernel launches.
 */
sv_status spec_verify_tree_typical(float temperature, double epsilon, double delta, int64_t B,
                                   int64_t n_nodes, int64_t V, sv_dtype dtype, const int32_t* parent,
                                   int64_t parent_batch_stride, const int32_t* cand_tokens,
                                   const void* target_logits, const float* uniforms, int64_t max_depth,
                                   int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                                   int32_t* err_flags, void* workspace, size_t workspace_bytes,
                                   sv_stream_t stream);

/* ---------------------------------------------------------------- row statistics
 * [S-SD], [M-3]. The target's logits over the vocabulary define the next token's
 * distribution (Sonar page, section "Spekulatives Decoding"); the Medusa page,
 * section 三, turns a node's logits into that distribution by a softmax before the
 * sampler takes its token. This is that reduction on its own -- the streaming row
 * softmax the verifier is built on, exposed for diagnostics:
 * for rows x[rows][V], row_max = max_v x_v, row_lse = log sum_v exp(x_v / T),
 * row_argmax = lowest index of the maximum (-1 and SV_ERR_ROW if no entry exceeds
 * -inf). Any output pointer may be NULL. row_lse is NaN when the normaliser is not
 * finite (SV_ERR_ROW).
 */
size_t spec_row_stats_workspace(int64_t rows, int64_t V, sv_dtype dtype);

sv_status spec_row_stats(sv_dtype dtype, float temperature, int64_t rows, int64_t V,
                         const void* x, float* row_max, float* row_lse, int32_t* row_argmax,
                         int32_t* err_flags, void* workspace, size_t workspace_bytes,
                         sv_stream_t stream);

/* ---------------------------------------------------------------- commit (after verification)
 * [S-MTPZ], [S-INF]. Applies the outcome of spec_verify_linear on the device, with no
 * host synchronisation, for B sequences with k drafts:
 *   accept_len [B], out_tokens [B][k+1]   the outputs of spec_verify_linear
 *   draft_tokens [B][k]                   the drafts verified (needed for `shifted`)
 *   seq_len    [B]            in/out: tokens in each sequence; grows by L+1
 *   history    [B][capacity]  in/out: each sequence's tokens; out_tokens[b][0..L] are
 *                             written at positions seq_len[b] .. seq_len[b]+L (may be NULL
 *                             with capacity 0: lengths, shifted and next_token only)
 *   shifted    [B][k+1]       optional out: the draft's input tokens for its pass over the
 *                             verified positions, the target's inputs shifted one place left:
 *                             position j holds the token that follows position j, i.e.
 *                             out_tokens[b][j] (= x_j) for j < L, the target's token
 *                             y = out_tokens[b][L] at j = L; positions after
 *                             L hold x_j (their results are to be discarded) and position k
 *                             holds y
 *   next_token [B]            optional out: y, the first input of the next step
 *   err_flags  [B]            optional out: SV_ERR_UNVERIFIED (accept_len outside [0, k]),
 *                             SV_ERR_CAPACITY (seq_len + L + 1 > capacity); such a sequence
 *                             keeps its length and history, and gets -1 in shifted and
 *                             next_token
 * One kernel launch, one wave per sequence.
 */
sv_status spec_commit_linear(int64_t B, int64_t k, const int32_t* accept_len, const int32_t* out_tokens,
                             const int32_t* draft_tokens, int32_t* seq_len, int32_t* history,
                             int64_t capacity, int32_t* shifted, int32_t* next_token,
                             int32_t* err_flags, sv_stream_t stream);

/* Verification and commit in one launch: spec_verify_linear's arguments and outputs,
 * then the commit of spec_commit_linear (seq_len, history, capacity, shifted,
 * next_token as there) applied by the wave that writes the sequence's outputs, with
 * no second launch. err_flags carries the verification's bits and SV_ERR_CAPACITY;
 * with SV_ERR_CAPACITY alone the verification outputs are valid and nothing is
 * committed. Same workspace as spec_verify_linear.
 */
sv_status spec_verify_linear_commit(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                                    sv_dtype dtype, const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* uniforms,
                                    int32_t* accept_len, int32_t* out_tokens, float* p_target,
                                    float* p_draft, int32_t* err_flags, int32_t* seq_len,
                                    int32_t* history, int64_t capacity, int32_t* shifted,
                                    int32_t* next_token, void* workspace, size_t workspace_bytes,
                                    sv_stream_t stream);

/* ---------------------------------------------------------------- sampler
 * [S-MTP] (sampling shared by every scheme), [S-ZE]. One token per row of
 * logits[rows][V]: argmax (SV_GREEDY: largest value, lowest index on ties) or the
 * inverse-CDF draw from softmax(row / T) with uniforms[row] (SV_STOCHASTIC): the
 * smallest v whose cumulative probability exceeds u. tokens[rows] out (-1 with
 * SV_ERR_ROW if the row has no usable entry); err_flags[rows] optional. The same row
 * reduction and draw as the verifier's; one kernel launch.
 */
size_t spec_sample_workspace(int64_t rows, int64_t V, sv_dtype dtype);

sv_status spec_sample(sv_mode mode, float temperature, int64_t rows, int64_t V, sv_dtype dtype,
                      const void* logits, const float* uniforms, int32_t* tokens, int32_t* err_flags,
                      void* workspace, size_t workspace_bytes, sv_stream_t stream);

/* ---------------------------------------------------------------- tree attention mask
 * [M-3]. For n_trees trees of n_nodes (parent arrays as for spec_verify_tree):
 * mask[t][i][w] (uint32 words, W = ceil(n_nodes / 32) per row) has bit (j mod 32) of
 * word j / 32 set iff node j is node i or one of its ancestors. err_flags[t] optional
 * (zeroed, then SV_ERR_TREE if the parent array is invalid; the mask of such a tree is
 * unspecified). One kernel launch (two with err_flags); one wave per row.
 */
sv_status spec_tree_mask(int64_t n_trees, int64_t n_nodes, const int32_t* parent,
                         int64_t parent_batch_stride, uint32_t* mask, int32_t* err_flags,
                         sv_stream_t stream);

/* ---------------------------------------------------------------- greedy sparse tree (host)
 * [M-4]. HOST pointers; runs on the CPU (a one-off construction, no device work).
 *   accuracy [K][S]   a_k^(i) at accuracy[(k-1)*S + (i-1)]: accuracy of the rank-i
 *                     candidate of head k (tree depth k), each in [0, 1]
 *   budget            candidate nodes wanted (the root is extra)
 * Nodes are added one at a time, each time the candidate whose path product of
 * accuracies is largest (ties: smaller depth, then the earlier-added parent, then the
 * smaller rank), starting from the root's children; a node's children become
 * candidates when it is added. Output (n = returned count, root included, at most
 * budget + 1; fewer if the full tree of depth K is smaller): parent[n] in breadth-first
 * order (by depth, then parent, then rank; parent[0] = -1, parent[i] < i), depth[n] and
 * rank[n] optional (root: 0, 0), expected_len optional: the sum of the path products
 * (the expected accepted length of the tree). Returns n, or -SV_EINVAL / -SV_ELIMIT.
 */
int64_t spec_tree_build_greedy(int64_t K, int64_t S, const double* accuracy, int64_t budget,
                               int32_t* parent, int32_t* depth, int32_t* rank, double* expected_len);

/* Zero-fill `bytes` of a 16-byte aligned workspace on `stream` with a fill kernel (no host sync). */
sv_status spec_workspace_clear(void* workspace, size_t bytes, sv_stream_t stream);

/* ---------------------------------------------------------------- plain read (measurement aid)
 * Not a step of the method: reads a_bytes of device buffer a and b_bytes of b (a
 * verification's target and draft logits, say) with nothing else done, in the
 * streaming waves' pattern (one wave per 8 KiB chunk, eight 16-byte loads per lane
 * issued together), so that a benchmark can time what reading those bytes costs by
 * itself on this GPU. Each wave stores its chunk's largest 32-bit word to
 * sink[wave] (a's chunks first); a trailing part of a buffer shorter than 16 bytes
 * is not read. a and b (either may be null with size 0) must be 16-byte aligned;
 * sink holds at least ceil(a_bytes / 8192) + ceil(b_bytes / 8192) words.
 * SV_EINVAL for a null or misaligned buffer of nonzero size or a short sink,
 * SV_ELIMIT past the launch's wave limit; enqueues only.
 */
sv_status spec_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink,
                          size_t sink_words, sv_stream_t stream);

/* ---------------------------------------------------------------- wait limit (test hook)
 * How long, in seconds of the GPU's constant 100 MHz clock, any wait between the
 * waves of one launch may last before it gives up and reports SV_ERR_INTERNAL
 * (bit3 above), on the current device: default 0.25, at most 60; 0 lets every
 * wait give up after its second unsuccessful poll. For tests of the give-up path:
 * set it between calls, never while this library's kernels run on the device, and
 * clear the workspace of a call that gave up before its next use. A synchronous
 * copy to the device; SV_EINVAL outside [0, 60] (or NaN), SV_EHIP if the copy fails.
 */
sv_status spec_set_wait_limit(double seconds);

/* ---------------------------------------------------------------- linear drafts, no allocation
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, outputs
 * and results as spec_verify_linear, without the workspace: the kernels use a
 * scratch array of SV_MAX_STATIC_WORKSPACE bytes that the library holds on each
 * GPU it runs on until the process ends (its device address is looked up once per
 * device, on the first call there). Each call zero-fills the part of that array it
 * uses with a fill kernel on `stream` (no memset node) and then launches the
 * verification there: two launches, no allocation, no host synchronisation.
 * Shapes whose workspace (spec_verify_linear_workspace) exceeds the array return
 * SV_ELIMIT before anything is launched; SV_EHIP if the array's address cannot be
 * obtained. All calls on one GPU share its array: calls that overlap on one GPU
 * (on different streams, or from different host threads) race and must not be
 * issued.
 */
enum { SV_MAX_STATIC_WORKSPACE = 8 * 1024 * 1024 };

sv_status spec_verify_linear_static(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                                    sv_dtype dtype, const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* uniforms,
                                    int32_t* accept_len, int32_t* out_tokens, float* p_target,
                                    float* p_draft, int32_t* err_flags, sv_stream_t stream);

/* Static description of a status code. */
const char* spec_verify_status_string(sv_status status);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
