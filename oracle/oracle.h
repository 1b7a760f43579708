/* Reference oracle for speculative-decoding verification -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, single-threaded C++17 in double precision. Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never does, and the two share no code.
 *
 * What it follows (pages: "Accelerating Sonar through speculation", original
 * German page and its Chinese / Hindi translations; "Speculative-Decoding, LLM推理的加速 /
 * Medusa 方法阅读"):
 *  - the longest acceptable draft prefix plus one extra target token: a draft of
 *    n tokens yields up to n+1 tokens (Sonar page, section "Spekulatives Decoding");
 *  - acceptance decided by comparing the full draft and target distributions, and
 *    the logits after the accepted prefix sampled for one more token (Sonar page,
 *    section "Ziel-Entwurf"; section "Spekulatives Decoding", phases "Akzeptanz"
 *    and "Zielgenerierung"). The page cites Leviathan et al. for the rule but does
 *    not print it; the rule used is that method's: accept draft token x at
 *    position i iff u_i < p_t,i(x) / p_d,i(x); on the first rejection at position
 *    L, sample from the residual max(0, p_t,L - p_d,L) renormalised; if every
 *    draft is accepted, sample from p_t,k;
 *  - the Medusa tree walk: sample (or take the argmax of) the root's logits,
 *    look for a level-1 candidate holding that token, follow it level by level
 *    until no child matches (Medusa page, section 三 "Attention Tree");
 *  - the expected accepted length E[L] = sum over tree nodes of the product of
 *    per-level accuracies along the node's path (Medusa page, section 四).
 *
 * Parity pins: every function here is pinned by CPU tests (closed forms,
 * library routines, brute force, chi-square losslessness, the pages' counts);
 * see the test files under tests/ that start with test_oracle_.
 */
#ifndef SV_ORACLE_H
#define SV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype: 0 fp32, 1 bf16, 2 fp16. mode: 0 greedy, 1 stochastic. */

/* Row statistics at temperature T over rows x[rows][V]:
 * m = max_v x_v, lse = log sum_v exp(x_v / T) = m/T + log sum_v exp((x_v - m)/T),
 * argmax = lowest index of the largest value (NaN entries never chosen).
 * flags[r]: bit1 if no entry exceeds -inf or the sum is not finite. */
int orc_row_stats(int dtype, double T, int64_t rows, int64_t V, const void* x,
                  double* m, double* lse, int32_t* argmax, int32_t* flags);

/* Inverse CDF over non-negative weights w[0..n): S = sum w, C_v = prefix sums in
 * ascending order; returns min{v : C_v > u*S}, or the last v with w_v > 0 when
 * rounding leaves none; -1 if S is not a positive finite number.
 * lo/hi (optional) receive C_{y-1}/S and C_y/S. */
int64_t orc_invcdf(const double* w, int64_t n, double u, double* lo, double* hi);

/* Linear verification for B sequences (see header comment). Outputs:
 *  accept_len[B] in [0,k] (-1 on a data error), out_tokens[B][k+1] (-1 padded),
 *  p_target/p_draft[B][k] (optional, NaN on error), err_flags[B]
 *  (bit0 token out of range, bit1 non-finite row), near_tie[B], n_eval[B].
 * Evaluated draws (n_eval) are the ones the result depends on: the accept tests
 *  of positions 0..L (0..k-1 when L = k) and the final draw, so min(L+1, k) + 1;
 *  0 for greedy and for a sequence with a data error.
 * near_tie bits: 1 if an evaluated accept test has |u_i - min(1, q_i)| < tie_eps
 *  (it can change L and so every output), 2 if the final draw has u_k within
 *  tie_eps of either edge of the bin it selected (it can change only the final
 *  token). Returns 0, or -1 on bad arguments. */
int orc_verify_linear(int mode, double T, int64_t B, int64_t k, int64_t V, int dtype,
                      const void* target, const void* draft, const int32_t* draft_tokens,
                      const float* uniforms, double tie_eps,
                      int32_t* accept_len, int32_t* out_tokens, double* p_target,
                      double* p_draft, int32_t* err_flags, int32_t* near_tie, int32_t* n_eval);

/* Tree verification for B trees of n_nodes (node 0 = root). parent[n_nodes] is
 * shared when parent_stride == 0, else [B][n_nodes]. Outputs: accept_len[B],
 * path_nodes[B][max_depth], out_tokens[B][max_depth+1], err_flags[B]
 * (bit0 candidate out of range, bit1 non-finite row, bit2 invalid tree or depth
 * above max_depth), near_tie[B], n_eval[B], and optional node_token[B][n_nodes]
 * (the per-node argmax / sampled token). Stochastic: the evaluated draws are
 * those at accepted nodes (each decides which of the node's children match); a
 * near tie (u within tie_eps of an edge of its bin) sets bit 1 at a node with
 * children (it can change the path) and bit 2 at a leaf (only the final token).
 * Greedy: n_eval = near_tie = 0. */
int orc_verify_tree(int mode, double T, int64_t B, int64_t n_nodes, int64_t V, int dtype,
                    const int32_t* parent, int64_t parent_stride, const int32_t* cand,
                    const void* logits, const float* uniforms, int64_t max_depth, double tie_eps,
                    int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                    int32_t* err_flags, int32_t* near_tie, int32_t* n_eval, int32_t* node_token);

/* E[L] of a candidate tree under independent per-level accuracies:
 * sum over non-root nodes of prod_{edges on the path} acc[(depth-1)*S + rank-1],
 * rank in 1..S (Medusa page, section 四, items 2-4). */
double orc_expected_accept_len(int64_t n_nodes, const int32_t* parent, const int32_t* rank,
                               int64_t S, const double* acc);

/* Commit of a linear verification (Sonar page, section "MTP-Zeitplan für ein
 * einzelnes Token": the target's input tokens shifted one place left, the next
 * target token inserted at its place; section "Inferenz mit spekulativem
 * Decoding": the accepted count sets the next length). For each sequence with
 * L = accept_len[b] in [0, k] and len + L + 1 <= capacity (history NULL: no
 * capacity check): history[b][len + j] = out_tokens[b][j] for j <= L, len += L + 1;
 * shifted[b][j] = y (= out_tokens[b][L]) for j = L and j = k, else drafts[b][j];
 * next_token[b] = y. Otherwise err 32 (L outside [0, k]) or 16 (capacity), nothing
 * committed, shifted row and next_token -1. */
int orc_commit_linear(int64_t B, int64_t k, const int32_t* accept_len, const int32_t* out_tokens,
                      const int32_t* drafts, int32_t* seq_len, int32_t* history, int64_t capacity,
                      int32_t* shifted, int32_t* next_token, int32_t* err_flags);

/* One token per row of x[rows][V]: greedy = argmax (lowest index), stochastic =
 * invcdf(softmax(x / T), u[row]) (Sonar page, sections "MTP" and "Ziel-Entwurf":
 * sampling shared by all schemes). tokens -1 and err bit1 for a row without a usable
 * entry; near_tie[row] (optional) 2 if u lies within tie_eps of an edge of the drawn
 * bin (the token is a final draw), else 0. */
int orc_sample(int mode, double T, int64_t rows, int64_t V, int dtype, const void* x,
               const float* uniforms, double tie_eps, int32_t* tokens, int32_t* err_flags,
               int32_t* near_tie);

/* Tree attention mask (Medusa page, section 三): dense[i][j] = 1 iff node j is node i
 * or an ancestor of it, built row by row as the parent's row plus node i itself.
 * Returns 0, or -1 if the parent array is invalid (parent[0] != -1 or parent[i]
 * outside [0, i)). */
int orc_tree_mask(int64_t n_nodes, const int32_t* parent, uint8_t* dense);

/* Greedy sparse tree (Medusa page, section 四): starting from the root, repeatedly
 * add the candidate node with the largest product of accuracies along its path
 * (acc[(depth-1)*S + rank-1]); ties by smaller depth, then the earlier-added parent,
 * then smaller rank; the children of an added node (up to depth K) become
 * candidates. Stops after `budget` nodes or when no candidate is left. Nodes are
 * numbered in breadth-first order (children in rank order). Returns the node count
 * n (root included); parent/depth/rank[n]; *expected_len = sum of the added nodes'
 * products in node order. */
int64_t orc_tree_build_greedy(int64_t K, int64_t S, const double* acc, int64_t budget,
                              int32_t* parent, int32_t* depth, int32_t* rank, double* expected_len);

/* Typical acceptance on candidate trees (named by the workload description, NOT
 * defined on the pages: a reading, parity unpinned by the pages). With p_n =
 * softmax(row n / T) and H_n = -sum_v p_n(v) ln p_n(v) (its entropy, nats), node
 * i >= 1 passes iff p_parent(cand_i) > min(epsilon, delta * exp(-H_parent)); it is
 * accepted iff it passes and its parent is accepted (the root always is); the
 * deepest accepted node (lowest index on ties) ends the path, and the final token is
 * invcdf(p_best, u[b][best]). near_tie[b]: bit 1 if a decisive pass test (one of a
 * child of an accepted node) lies within tie_eps (relative) of its threshold, bit 2 if
 * the final draw lies within tie_eps of a bin edge. n_eval[b]: decisive tests plus the
 * final draw. Errors as for orc_verify_tree. */
int orc_verify_tree_typical(double T, double epsilon, double delta, int64_t B, int64_t n_nodes,
                            int64_t V, int dtype, const int32_t* parent, int64_t parent_stride,
                            const int32_t* cand, const void* logits, const float* uniforms,
                            int64_t max_depth, double tie_eps, int32_t* accept_len,
                            int32_t* path_nodes, int32_t* out_tokens, int32_t* err_flags,
                            int32_t* near_tie, int32_t* n_eval);

/* Planted-mistake switch for negative-control tests only (0 = off). */
void orc_set_mutation(int which);

#ifdef __cplusplus
}
#endif
#endif
