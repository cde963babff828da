/*
 * more_route.h -- C ABI of the MI355X (gfx950) fused MoE router library
 * (libmore_route.so).
 *
 * Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
 * routing" (Wong, Goel, Boix-Adsera).
 *   - §2: the standard router g(x) = softmax(TopK(R x)) and the low-rank
 *     router, where R is replaced by the product of a rank-r down-projection
 *     and an up-projection.
 *   - App. F, eq. (5): logits of all tokens and experts; App. F.1,
 *     Algorithm 1: one fused pass that never writes the N x M logits and
 *     returns the top-k values and indices; Fig. 12: gate weights are a
 *     softmax over the k selected logits.
 *   - App. F.2.1, eq. (6) and eq. (8): the full softmax over all M experts,
 *     built with a running maximum and a running normaliser across expert
 *     tiles (online log-sum-exp).
 *
 * Convention.  R1 is the h x r down-projection and R2 the r x M
 * up-projection, both row-major, so token x (a row of X) has logits
 * l = (x R1) R2 + b.  (The paper writes the factors the other way round:
 * its down-projection is our R1 transposed and its up-projection our R2
 * transposed.)  The full-rank router takes W (h x M, row-major): l = x W + b.
 *
 * Common rules for every routing call:
 *   Pointers.  X, R1, R2, W, bias and every output are DEVICE pointers
 *   (hipMalloc'd or torch CUDA tensors) on the current HIP device.  All
 *   tensors are dense row-major and 16-byte aligned.  Ownership stays with
 *   the caller; the library allocates and frees nothing and keeps no state
 *   between calls, so calls on different streams may run concurrently as long
 *   as their outputs and workspaces do not overlap.
 *   Asynchrony.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *   legacy default stream) and the call returns without synchronising.
 *   Outputs are valid once the stream reaches that point.
 *   Errors.  Arguments are validated on the host before any HIP call; a
 *   failed check returns its code and enqueues nothing.  MORE_ERR_HIP means a
 *   kernel launch was rejected; faults during execution surface at the
 *   caller's next synchronisation, not here.
 *   Contract.  1 <= k <= min(M, 32); N >= 0 (N = 0 is a no-op); h, M >= 1;
 *   h % 8 == 0; for the low-rank router r % 16 == 0 and r <= 128.  Inputs
 *   must be finite: non-finite inputs give undefined results.
 *   Outputs.  Per token the k experts are listed by logit descending; equal
 *   logits are listed by expert index ascending, and when equal logits
 *   straddle the k-th place the lower indices are selected.  topk_idx is
 *   int32 (N x k); topk_gate, topk_logit (N x k) and lse (N) are fp32.  The
 *   logits are computed with fp32 accumulation of exact bf16 (or fp32)
 *   products; the down-projection result enters the second product as a
 *   bf16 hi+lo pair, i.e. at about 16 significant bits.
 *   Gates.  MORE_GATE_TOPK_SOFTMAX: g_j = exp(l_j - l_1) / sum over the k
 *   selected of exp(l_i - l_1).  MORE_GATE_FULL_SOFTMAX: g_j = exp(l_j - lse)
 *   with lse = log sum over all M experts of exp(l) (not renormalised).
 *   Workspace.  Device scratch owned by the caller, at least
 *   more_route_workspace_bytes(...) bytes for the same arguments, 256-byte
 *   aligned.  It carries the per-call packed weights, then (low rank, bf16,
 *   r <= 64) token scratch sized by N: the rank-r intermediate z of every
 *   32-token block (4 bytes per token and rank) for the two-kernel path.  A
 *   workspace without room for that scratch is still valid; the routing call
 *   then takes a one-kernel path.  Its contents need no initialisation and
 *   are garbage afterwards.  Two calls in flight must not share a workspace.
 */
#ifndef MORE_ROUTE_H
#define MORE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MORE_ABI_VERSION 1
#define MORE_MAX_K 32
#define MORE_MAX_R 128

typedef enum {
    MORE_OK = 0,
    MORE_ERR_NULL_ARG = 1,    /* a required pointer is NULL                      */
    MORE_ERR_BAD_SHAPE = 2,   /* N < 0, h < 1, M < 1, r < 1, or size overflow    */
    MORE_ERR_BAD_K = 3,       /* k < 1, k > M or k > MORE_MAX_K                 */
    MORE_ERR_BAD_DTYPE = 4,   /* unknown more_dtype                              */
    MORE_ERR_BAD_GATE = 5,    /* unknown more_gate                               */
    MORE_ERR_WORKSPACE = 6,   /* workspace NULL/too small/misaligned             */
    MORE_ERR_UNSUPPORTED = 7, /* outside the envelope: h % 8, r % 16, r > 128    */
    MORE_ERR_HIP = 8,         /* a HIP launch or query failed                    */
    MORE_ERR_ALIGNMENT = 9,   /* a tensor pointer is not 16-byte aligned         */
    MORE_ERR_STALLED = 10,    /* a kernel's bounded wait gave up: outputs invalid */
    MORE_ERR_SCRATCH_LIMIT = 11 /* needs more than the library's static scratch   */
} more_status;

typedef enum {
    MORE_DT_BF16 = 0, /* X, R1, R2 (or W) stored as bf16 */
    MORE_DT_F32 = 1   /* X, R1, R2 (or W) stored as fp32 */
} more_dtype;

typedef enum {
    MORE_GATE_TOPK_SOFTMAX = 0, /* softmax over the k selected logits (Fig. 12)      */
    MORE_GATE_FULL_SOFTMAX = 1  /* full-softmax probability via online LSE (eq. 6/8) */
} more_gate;

/*
 * Fused low-rank router + top-k + gates (App. F.1 Algorithm 1; gates per
 * Fig. 12 or eq. (6)).  One pass over X: z = x R1 stays on chip, the experts
 * are swept in tiles of z R2 + b with a streaming top-k, and only the
 * N x k results reach memory.
 *   dt          storage type of X, R1 and R2.
 *   X           N x h.          R1  h x r.          R2  r x M.
 *   bias        M fp32, or NULL for no bias.  The biased logit drives both
 *               selection and gates.
 *   k, gate     as above.
 *   topk_idx    N x k int32 (required).   topk_gate  N x k fp32 (required).
 *   topk_logit  N x k fp32 or NULL.       lse        N fp32 or NULL; written
 *               only in FULL_SOFTMAX mode.
 *   workspace   see above; size from more_route_workspace_bytes(0, ...).
 *   stream      hipStream_t or NULL.
 */
more_status more_route_lowrank(more_dtype dt, const void* X, int64_t N, int64_t h, const void* R1,
                               int64_t r, const void* R2, int64_t M, const float* bias, int32_t k,
                               more_gate gate, int32_t* topk_idx, float* topk_gate,
                               float* topk_logit, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Split form of more_route_lowrank for static weights: more_lowrank_pack
 * writes the sweep order and the MFMA-ordered copies of R1, R2 and the bias
 * into `workspace` (size from more_route_workspace_bytes(0, ...)); after it,
 * more_lowrank_route_packed routes any number of token batches against that
 * workspace without touching R1, R2 or the bias again.  The two calls must
 * agree on dt, h, r and M (and on whether a bias was given); the library
 * cannot check this because the packed data lives on the device.
 * more_route_lowrank(...) is exactly more_lowrank_pack followed by
 * more_lowrank_route_packed on the same stream.  more_lowrank_route_packed
 * only reads the packed part of the workspace; it overwrites the token
 * scratch behind it (used when workspace_bytes covers N tokens).
 */
more_status more_lowrank_pack(more_dtype dt, const void* R1, int64_t h, int64_t r, const void* R2,
                              int64_t M, const float* bias, void* workspace, size_t workspace_bytes,
                              void* stream);
more_status more_lowrank_route_packed(more_dtype dt, const void* X, int64_t N, int64_t h, int64_t r,
                                      int64_t M, int32_t k, more_gate gate, int32_t* topk_idx,
                                      float* topk_gate, float* topk_logit, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training forward with balancing statistics (App. F.2.1, Algorithm 2: a
 * first sweep with the running top-k and the running maximum / normaliser of
 * eq. (8), then a second sweep that recomputes every logit tile and adds the
 * full-softmax probabilities into per-expert column sums; eq. (7) and (9);
 * App. G.1 for the entropy).  Against weights packed by more_lowrank_pack:
 *   topk_idx, topk_gate, topk_logit  as for more_lowrank_route_packed.
 *   lse        N fp32 (required): log sum over all M experts of exp(l), in
 *              both gate modes (the training forward's normaliser m + log Z).
 *   psum       M fp32 (required): psum_i = sum over the N tokens of
 *              P_{n,i} = exp(l_{n,i} - lse_n), the biased logits' softmax.
 *   counts     M int32 (required): how many of the N k selected slots went to
 *              each expert (a bincount of topk_idx).
 *   stats      2 fp32 (required): stats[0] = L_bal = M sum_i f_i p_i with
 *              f_i = counts_i / (N k) and p_i = psum_i / N (the Switch loss,
 *              eq. 9); stats[1] = H_norm = -sum_a q_a log q_a / log M with
 *              q_a = counts_a / (N k) (1 for M = 1).
 *   workspace  at least more_balance_workspace_bytes(...) bytes: the packed
 *              weights, then the token scratch and the per-slot partial sums
 *              (overwritten).
 * Envelope: the shapes whose routing runs as the projection + routing
 * kernel pair: bf16, k <= 8, M <= 65536, and R1 small enough to stay in the
 * projection kernel's LDS (h <= 4608 for r = 16, h <= 2048 for r = 32,
 * h <= 768 for r = 48 or 64); other shapes return
 * MORE_ERR_UNSUPPORTED (more_balance_workspace_bytes returns 0 for them).  psum, counts and stats are written in a fixed
 * summation order (the same inputs give the same bits).  N = 0 is a no-op.
 */
more_status more_lowrank_balance_packed(more_dtype dt, const void* X, int64_t N, int64_t h, int64_t r,
                                        int64_t M, int32_t k, more_gate gate, int32_t* topk_idx,
                                        float* topk_gate, float* topk_logit, float* lse, float* psum,
                                        int32_t* counts, float* stats, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of more_lowrank_balance_packed for these arguments (0 where
 * it would return MORE_ERR_UNSUPPORTED or reject the shape).  Pure host
 * function, no HIP call.
 */
size_t more_balance_workspace_bytes(more_dtype dt, int64_t N, int64_t h, int64_t r, int64_t M, int32_t k);

/*
 * Expert dispatch after the router (App. E, Fig. 9: "sort + count", the
 * (N, k) selected indices become N k indices sorted by expert + offsets).
 *   topk_idx       N x k int32 expert indices, each in [0, M) (the router's
 *                  topk_idx).  Entries outside [0, M) give an unspecified
 *                  order but no access outside the outputs.
 *   sorted_expert  N k int32: the experts in non-decreasing order.
 *   sorted_slot    N k int32: slot s = n k + j of each entry (token n = s / k,
 *                  its j-th choice); within one expert the slots increase
 *                  (stable), so the result is unique.
 *   offsets        M + 1 int32: expert e owns positions offsets[e] ..
 *                  offsets[e+1] - 1; offsets[M] = N k.
 *   workspace      at least more_dispatch_workspace_bytes(N, k, M) bytes,
 *                  256-byte aligned (per-block digit counts, about 2 bytes
 *                  per entry at M >= 4096; for M > 4096 one extra N k key +
 *                  slot buffer), overwritten.
 * Contract: N k < 2^31 - 1, 1 <= k <= M <= 2^24.  N = 0 is a no-op.  Integer
 * work only: the result is exact and deterministic.
 */
more_status more_dispatch_sort(const int32_t* topk_idx, int64_t N, int32_t k, int64_t M, int32_t* sorted_expert,
                               int32_t* sorted_slot, int32_t* offsets, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Workspace bytes of more_dispatch_sort (0 for arguments it rejects).  Pure
 * host function, no HIP call. */
size_t more_dispatch_workspace_bytes(int64_t N, int32_t k, int64_t M);

/*
 * more_dispatch_sort for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks and results as more_dispatch_sort,
 * without the workspace.  Its scratch (the per-block digit counts and the
 * key + slot buffer of the multi-pass sort) is a static 32 MiB device array
 * of the library, one per GPU, held until the process ends; no call here
 * allocates or frees memory.  A call whose more_dispatch_workspace_bytes(N,
 * k, M) exceeds 32 MiB (N k above about 16.7 million entries for M <= 4096,
 * 3.3 million for M > 4096) returns MORE_ERR_SCRATCH_LIMIT and enqueues
 * nothing.  Every call on one
 * GPU uses that GPU's one array and leaves it overwritten: calls that may
 * overlap on one GPU (different streams, or threads without ordering) race
 * and must be serialised by the caller.  MORE_ERR_HIP if the array's device
 * address cannot be obtained.
 */
more_status more_dispatch_sort_noalloc(const int32_t* topk_idx, int64_t N, int32_t k, int64_t M,
                                       int32_t* sorted_expert, int32_t* sorted_slot, int32_t* offsets,
                                       void* stream);

/*
 * Backward pass of the low-rank router with recompute (App. F.2.2, eq. (10)-
 * (12), Algorithm 3).  With the forward's selection held fixed, it returns the
 * gradients of F = sum_{n,j} tvbar[n,j] l[n, idx[n,j]] + sum_i pbar_i psum_i:
 *   g_n = sum_i pbar_i P_{n,i}, P = exp(l - lse),
 *   ybar_{n,e} = P_{n,e} (pbar_e - g_n) + tvbar[n,j] where idx[n,j] = e,
 *   X_grad = (ybar R2^T) R1^T, R1_grad = X^T (ybar R2^T), R2_grad = z^T ybar,
 *   bias_grad = sum over tokens of ybar   (z = X R1).
 * Against weights packed by more_lowrank_pack (same R1, R2, bias):
 *   X, R1, R2       the forward's inputs (bf16; R1 h x r, R2 r x M).
 *   topk_idx        N x k int32: the forward's selection.
 *   topk_logit_grad N x k fp32: gradient on the selected logits (tvbar).
 *   psum_grad       M fp32 or NULL (zero): gradient on psum (pbar; for the
 *                   Switch loss of eq. (9), pbar_i = (M / N) f_i).
 *   lse             N fp32: the forward's log-sum-exp (balancing call).
 *   X_grad          N x h bf16 (required).  R1_grad h x r, R2_grad r x M
 *                   fp32 (required).  bias_grad M fp32 or NULL.
 *   workspace       at least more_backward_workspace_bytes(...) bytes: the
 *                   packed weights, then the token scratch and the backward's
 *                   intermediates (overwritten).
 * Envelope: bf16, r in {16, 32}, h % 32 == 0, k <= 32, M <= 16384 and R1
 * small enough for the projection kernel's LDS; other shapes return
 * MORE_ERR_UNSUPPORTED.  Sums over tokens run in a fixed order (the same
 * inputs give the same bits).  N = 0 is a no-op.
 */
more_status more_lowrank_backward_packed(more_dtype dt, const void* X, int64_t N, int64_t h, const void* R1,
                                         int64_t r, const void* R2, int64_t M, int32_t k, const int32_t* topk_idx,
                                         const float* topk_logit_grad, const float* psum_grad, const float* lse,
                                         void* X_grad, float* R1_grad, float* R2_grad, float* bias_grad,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of more_lowrank_backward_packed (0 outside its envelope).
 * Pure host function, no HIP call. */
size_t more_backward_workspace_bytes(more_dtype dt, int64_t N, int64_t h, int64_t r, int64_t M, int32_t k);

/*
 * Top-k over expert shards: merges per-shard candidate lists into the
 * token's top k and gates (App. E.3: a hierarchical top-k over shards of the
 * experts; gates as Fig. 12 or eq. (6) with the normaliser of eq. (8)).
 * The M experts are cut into G = ceil(M / shard_width) shards of
 * shard_width consecutive experts (the last may be shorter); shard g covers
 * experts g * shard_width ..  Each shard routes every token over its own
 * experts (more_route_lowrank / more_lowrank_route_packed with that shard's
 * columns of R2 and entries of the bias, or more_route_fullrank) and hands
 * over its topk_logit and topk_idx (shard-local indices) and, for
 * MORE_GATE_FULL_SOFTMAX, its lse.
 *   cand_logit  G x N x k fp32: shard g's logits, each row ordered by
 *               (logit desc, index asc) as the routing calls write them.
 *   cand_idx    G x N x k int32: shard-local expert indices.
 *   shard_lse   G x N fp32 (MORE_GATE_FULL_SOFTMAX) or NULL (TOPK).
 *   topk_idx, topk_gate (N x k, required), topk_logit (N x k, NULL to skip),
 *   lse (N, full-softmax gates only, NULL to skip): as for more_route_lowrank;
 *   global expert indices, ordered by (logit desc, index asc).
 * Requires 1 <= k <= MORE_MAX_K, k <= shard_width and at least k experts in
 * the last shard (else MORE_ERR_BAD_K).  The caller owns every buffer; the
 * call allocates nothing and enqueues one kernel on `stream`.  N = 0 is a
 * no-op.
 */
more_status more_topk_merge(int64_t N, int64_t M, int64_t shard_width, int32_t k, more_gate gate,
                            const float* cand_logit, const int32_t* cand_idx, const float* shard_lse,
                            int32_t* topk_idx, float* topk_gate, float* topk_logit, float* lse, void* stream);

/*
 * Fused standard (full-rank) router + top-k + gates: the same selection and
 * gates with l = x W + b (§2 standard router; App. H.3 Fig. 20 fuses it the
 * same way, reloading weight tiles instead of a rank-r intermediate).
 *   W  h x M.  Other arguments as for more_route_lowrank.
 *   workspace  size from more_route_workspace_bytes(1, ...): W and the bias
 *              are repacked into it on every call (overwritten).
 * bf16 with k <= 8 and h % 64 == 0 runs an LDS-tiled MFMA sweep (256 tokens
 * per workgroup, 256-expert slabs); other shapes and fp32 run a plain
 * one-wave-per-32-tokens kernel.  Both give the same selection rule.
 */
more_status more_route_fullrank(more_dtype dt, const void* X, int64_t N, int64_t h, const void* W,
                                int64_t M, const float* bias, int32_t k, more_gate gate,
                                int32_t* topk_idx, float* topk_gate, float* topk_logit, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes needed by a routing call with these arguments (fullrank = 0
 * for more_route_lowrank, 1 for more_route_fullrank; r is ignored for full
 * rank; has_bias != 0 when a bias pointer will be passed).  Returns 0 for
 * arguments the call would reject.  Pure host function, no HIP call.
 */
size_t more_route_workspace_bytes(int fullrank, more_dtype dt, int64_t N, int64_t h, int64_t r,
                                  int64_t M, int32_t k, more_gate gate, int has_bias);

/*
 * Testing aid: restrict the kernel forms the low-rank routing calls may take
 * to a comma-separated subset of "split,ring,pc,lock,stream" (the plain kernel,
 * which fits every shape, always remains; an empty subset such as "none"
 * leaves only it).  NULL or "" allows every form again.  Every form computes
 * the same selection and gates; this only lets tests check each of them on
 * shapes a faster one would take.  The environment variable MORE_ROUTE_PATHS
 * sets the initial subset, read once at the first routing call.  Process-wide;
 * not to be called while routing calls are being enqueued on other threads.
 */
void more_set_route_paths(const char* names);

/*
 * Outcome of the routing calls enqueued so far on a workspace.  The persistent
 * routing kernels hand work between their waves through bounded waits; a wait
 * that gives up (a protocol failure, never expected) makes every wave of that
 * launch exit normally and records the failure in a status word at offset 0 of
 * the workspace, which more_lowrank_pack clears.  This call synchronises
 * `stream`, reads the word and clears it: MORE_OK, or MORE_ERR_STALLED when
 * some routing, balancing or backward call on this workspace since the last
 * check (or the last pack) returned invalid outputs.  MORE_ERR_NULL_ARG /
 * MORE_ERR_WORKSPACE for a NULL or misaligned workspace, MORE_ERR_HIP if the
 * synchronisation or a copy fails.  Host function.
 */
more_status more_route_status(void* workspace, void* stream);

/*
 * Testing aid: polls before a bounded wait gives up (<= 0 restores the
 * default, 4194304).  Process-wide; a tiny value makes the waits give up from
 * the host side so that the error path can be exercised without a failure on
 * the device (every kernel still exits normally).
 */
void more_set_spin_limit(int polls);

/* Static string for a status code (never NULL). */
const char* more_status_str(more_status s);

/* MORE_ABI_VERSION of the built library. */
int more_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MORE_ROUTE_H */
