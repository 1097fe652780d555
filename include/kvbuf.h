/*
 * kvbuf.h -- KVBuffer linear-attention decode for AMD Instinct MI355X (gfx950).
 *
 * The method (KVBuffer: IO-aware Serving for Linear Attention, Zou and Zhong,
 * arXiv 2605.19049; pith.science page, abstract and Figures 1-3):
 * a request's linear-attention state S (d_k x d_v per head) is not rewritten at
 * every decoded token.  Instead the request keeps its most recent keys and
 * values in a paged buffer; a token's output is computed from the state plus
 * the buffered keys and values, and the buffered tokens are folded into the
 * state in one batched update once the buffer holds m of them.  The same
 * buffer verifies n draft tokens of speculative decoding in one call without
 * temporary states, and serves short requests from the buffer alone, without
 * ever creating a state.
 *
 * Update rules (the pages name none; these are the ones this library serves),
 * for a token with key k, value v, log-gate g and step size beta:
 *   KVBUF_RULE_LINEAR  S <- S + k v^T
 *   KVBUF_RULE_GATED   S <- exp(g) S + k v^T
 *   KVBUF_RULE_DELTA   S <- exp(g) (I - beta k k^T) S + beta k v^T
 *   KVBUF_RULE_CHANNEL S <- diag(exp(g)) S + k v^T, one log-gate per key channel
 *                      (the diagonal decay of the gated linear attention and
 *                      matrix-state RNN works in the page's reference list)
 * and the token's output is o = S^T (scale q), read after the token's own update.
 *
 * Everything is asynchronous on the caller's HIP stream.  The library
 * allocates no memory and holds no mutable global state: the caller owns every
 * buffer below (for example as PyTorch tensors).  Argument validation happens
 * on the host before anything is enqueued, so a call that returns an error
 * has changed nothing.  Metadata that lives on the device (occupancy, block
 * ids, state slots, accepted counts) is checked by the kernels: a (request,
 * head) tile whose metadata is out of range is skipped (no memory outside the
 * pools is touched) and a bit is set in the optional device error word.
 *
 * Concurrency: calls on one stream are ordered; two calls that overlap in time
 * (different streams) must not touch the same requests, blocks or state slots.
 */
#ifndef KVBUF_H
#define KVBUF_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVBUF_ABI_VERSION 5

typedef enum kvbuf_status {
    KVBUF_OK = 0,
    KVBUF_EINVAL = -1,       /* null pointer, negative size, inconsistent layout */
    KVBUF_EUNSUPPORTED = -2, /* head dims / dtype / rule / mode not provided */
    KVBUF_ECAPACITY = -3,    /* m not a multiple of block_size, buffer too small */
    KVBUF_EHIP = -4          /* the HIP runtime refused the launch */
} kvbuf_status;

typedef enum kvbuf_rule {
    KVBUF_RULE_LINEAR = 0,
    KVBUF_RULE_GATED = 1,
    KVBUF_RULE_DELTA = 2,
    /* One log-gate per key channel (log-gates are decays: a buffer's gates
     * should not sum past about 80 in any channel, where exp(sum) leaves the
     * fp32 range).  Served by every entry point. */
    KVBUF_RULE_CHANNEL = 3
} kvbuf_rule;

typedef enum kvbuf_dtype {
    KVBUF_BF16 = 0,
    KVBUF_F32 = 1
} kvbuf_dtype;

/* Element type of the outputs (`out` of kvbuf_decode, kvbuf_direct,
 * kvbuf_verify, kvbuf_verify_tree and kvbuf_verify_recurrent).  The sums are
 * formed in fp32 either way; KVBUF_OUT_BF16 rounds each output to the
 * nearest bf16 (ties to even) when it is stored.  Zero, the value of a
 * zero-initialised layout, is fp32. */
typedef enum kvbuf_out_dtype {
    KVBUF_OUT_F32 = 0,
    KVBUF_OUT_BF16 = 1
} kvbuf_out_dtype;

typedef enum kvbuf_flush_policy {
    /* kvbuf_decode and kvbuf_commit fold a request's buffer into its state in
     * the same call as soon as it holds m tokens (kvbuf_commit and, for the
     * usual m, kvbuf_decode in the same kernel; a decode whose m exceeds what
     * its kernel stages enqueues a fold launch right after it). */
    KVBUF_FLUSH_EAGER = 0,
    /* they only append; the caller folds with kvbuf_flush. */
    KVBUF_FLUSH_DEFERRED = 1
} kvbuf_flush_policy;

/* Bits of the device error word (kvbuf_batch.error). */
#define KVBUF_DEVERR_BLOCK 1u    /* a block id outside [0, num_blocks) */
#define KVBUF_DEVERR_SLOT 2u     /* a state slot >= num_state_slots, or none where one is required */
#define KVBUF_DEVERR_OVERFLOW 4u /* occupancy < 0, or appending would exceed the buffer capacity */
#define KVBUF_DEVERR_ACCEPT 8u   /* accepted[b] outside [0, n] */
#define KVBUF_DEVERR_META 16u    /* a request's head copies disagree with its row (kvbuf_check),
                                    or kvbuf_admit was given an index outside [0, B) */

/* Shapes and policy.  Host struct, read during the call only. */
typedef struct kvbuf_layout {
    int32_t num_heads;       /* H */
    int32_t d_k;             /* key/query head dim; d_k == d_v, one of 16, 64, 128 */
    int32_t d_v;             /* value head dim */
    int32_t m;               /* tokens folded per flush; 0 = recurrent mode (no buffer) */
    int32_t block_size;      /* tokens per pool block; m must be a multiple of it */
    int32_t blocks_per_req;  /* table row length, <= 64 entries; capacity = block_size * blocks_per_req,
                                m <= capacity <= 512 positions */
    int32_t num_blocks;      /* blocks in the pool */
    int32_t num_state_slots; /* slots in the state pool */
    int32_t rule;            /* kvbuf_rule */
    int32_t io_dtype;        /* kvbuf_dtype of q, k, v inputs and of the pool's key plane
                                (and of its value plane for the linear and gated rules) */
    int32_t flush;           /* kvbuf_flush_policy */
    float scale;             /* queries are multiplied by it (1.0 = none) */
    int32_t out_dtype;       /* kvbuf_out_dtype of every `out` argument */
} kvbuf_layout;

/* Device memory pools (caller-owned, row-major):
 *   state [num_state_slots][H][d_k][d_v]   fp32
 *   key   [num_blocks][H][block_size][d_k] io_dtype
 *   value [num_blocks][H][block_size][d_v] io_dtype for the linear and gated rules;
 *         fp32 for the delta rule, where it holds each token's pseudo-value
 *         u = beta (v - exp(g) S_prev^T k), so that S = exp(g) S_prev + k u^T
 *   gate  [num_blocks][H][block_size]      fp32 log-gates (NULL for the linear rule);
 *         [num_blocks][H][block_size][d_k] for the per-channel rule
 * In recurrent mode (m = 0) only `state` is used. */
typedef struct kvbuf_pools {
    float* state;
    void* key;
    void* value;
    float* gate;
} kvbuf_pools;

/* The batch: B requests.  All arrays are int32 in device memory, caller-owned.
 *   state_slot  [B]                  slot in the state pool; -1 = no state (the
 *                                    request is served from its buffer alone and
 *                                    never folds).  Never written.
 *   block_table [B][blocks_per_req]  each request's pool block ids, in buffer
 *                                    order: buffer position p is in block
 *                                    block_table[b][p / block_size], offset
 *                                    p % block_size.  A fold moves the
 *                                    m / block_size leading blocks to the back.
 *   occupancy   [B]                  tokens buffered since the last fold
 *   error       [1] or NULL          KVBUF_DEVERR_* bits are OR-ed into it
 *   tile_meta   [B][H][1 + blocks_per_req]  the library's working copies: for
 *                                    every (request, head), its occupancy and
 *                                    table row.
 * block_table and occupancy are the caller's view: the library keeps them
 * current in stream order (after every call they hold each request's row and
 * occupancy), and the caller writes them only to admit a request -- then calls
 * kvbuf_admit for it before any other call that touches it.  The kernels of a
 * call read and advance tile_meta, whose copy of (b, h) only the workgroup
 * serving that head touches, so a call needs no synchronisation across
 * workgroups; head 0's workgroup writes the request's new values to
 * block_table and occupancy.  A tile whose metadata fails a device check is
 * skipped and its copy left unchanged (the request's heads may then disagree:
 * kvbuf_check reports it). */
typedef struct kvbuf_batch {
    int32_t size;
    int32_t* state_slot;
    int32_t* block_table;
    int32_t* occupancy;
    int32_t* error;
    int32_t* tile_meta;
} kvbuf_batch;

/*
 * kvbuf_admit -- copy requests' block_table rows and occupancies into their
 * per-head working copies (tile_meta), for requests the caller has just given
 * blocks (a new request, one whose blocks changed, one promoted to a state)
 * (pith.science page, Figure 1 caption: each request owns its buffer blocks).
 * requests: [count] int32 request indices in device memory, or NULL for all
 * B requests (count ignored).  An index outside [0, B) sets KVBUF_DEVERR_META.
 * Requires m > 0.
 */
kvbuf_status kvbuf_admit(const kvbuf_layout* layout, const kvbuf_batch* batch, const int32_t* requests,
                         int32_t count, hipStream_t stream);

/*
 * kvbuf_check -- set KVBUF_DEVERR_META in the error word (required) if any
 * request's per-head copies disagree with its block_table row or occupancy
 * (after a device error skipped some of its heads).  Reads only.
 */
kvbuf_status kvbuf_check(const kvbuf_layout* layout, const kvbuf_batch* batch, hipStream_t stream);

/*
 * kvbuf_decode -- one decode step for every request of the batch.
 * (pith.science page, Figure 1 caption: decode reads the state and the
 * request's buffer blocks side by side; a full buffer is folded into the
 * state, which goes back to its slot.  Figure 3 caption: a buffer of size
 * m = 0 is the recurrent baseline.)
 *
 * Inputs  q, k [B][H][d_k] and v [B][H][d_v] in io_dtype; g [B][H] fp32
 *         log-gates (rules GATED, DELTA; [B][H][d_k] for CHANNEL; NULL for
 *         LINEAR); beta [B][H] fp32 (DELTA; else NULL).
 * Output  out [B][H][d_v] (layout->out_dtype), o = S_t^T (scale q) with S_t the state after
 *         this token.
 * m > 0:  appends the token at buffer position occupancy[b] and advances
 *         the occupancy.  A request with a state slot computes its output from the
 *         state at its last fold plus the buffer; one without (slot -1) from
 *         the buffer alone.  With KVBUF_FLUSH_EAGER a request with a state
 *         whose buffer reaches m folds in the same call (see
 *         KVBUF_FLUSH_EAGER).
 * m = 0:  recurrent: reads, updates and writes back every request's state.
 */
kvbuf_status kvbuf_decode(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, void* out,
                          hipStream_t stream);

/*
 * kvbuf_flush -- fold the first m buffered tokens of every request that has a
 * state slot and at least m buffered tokens into its state, write the state
 * back, rotate its block table and lower its occupancy by m.  Other requests
 * are left untouched.  (Figure 1 caption and abstract: the state changes
 * once per buffer, in one batched update.)  No-op when m = 0.
 */
kvbuf_status kvbuf_flush(const kvbuf_layout* layout, const kvbuf_pools* pools,
                         const kvbuf_batch* batch, hipStream_t stream);

/*
 * kvbuf_verify -- parallel verification of n draft tokens per request
 * (Figure 2 caption: the drafts' keys and values are buffered and verified
 * together, without a temporary state per draft).
 * Inputs  q, k [B][n][H][d_k], v [B][n][H][d_v] (io_dtype); g, beta [B][n][H]
 *         (g [B][n][H][d_k] for the per-channel rule).
 * Output  out [B][n][H][d_v] (layout->out_dtype): draft d attends to the state, the buffer and
 *         drafts 0..d (causal within the drafts).
 * The drafts are written at buffer positions occupancy .. occupancy+n-1; the
 * occupancy does not change.  Requires m > 0 and 1 <= n <= 8.
 */
kvbuf_status kvbuf_verify(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, int32_t n, const void* q,
                          const void* k, const void* v, const float* g,
                          const float* beta, void* out, hipStream_t stream);

/*
 * kvbuf_commit -- keep the first accepted[b] (0..n) drafts of the preceding
 * kvbuf_verify: the occupancy advances over them; rejected drafts stay behind
 * as dead data.  With KVBUF_FLUSH_EAGER a request with a state whose buffer
 * reaches m folds its first m tokens in the same kernel.
 * accepted: [B] int32, device memory.
 */
kvbuf_status kvbuf_commit(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, int32_t n, const int32_t* accepted,
                          hipStream_t stream);

/*
 * kvbuf_verify_tree -- verification of n draft tokens that form a tree (the
 * page's reference list includes tree speculative decoding for state-space
 * models): parent [B][n] int32, device memory, parent[b][d] in {-1, 0 .. d-1};
 * -1 makes draft d follow the buffer directly.  Draft d attends to the state,
 * the buffer, its ancestors and itself, with the gates accumulated along that
 * path -- the output a serial decode of its root-to-node path would give.
 * Drafts are written at buffer positions occupancy + d as with kvbuf_verify;
 * the occupancy does not change.  A chain (parent[d] = d - 1) is kvbuf_verify.
 * Requires m > 0 and 1 <= n <= 8.  A parent outside
 * its range sets KVBUF_DEVERR_ACCEPT and skips the tile.
 */
kvbuf_status kvbuf_verify_tree(const kvbuf_layout* layout, const kvbuf_pools* pools,
                               const kvbuf_batch* batch, int32_t n, const int32_t* parent,
                               const void* q, const void* k, const void* v, const float* g,
                               const float* beta, void* out, hipStream_t stream);

/*
 * kvbuf_commit_tree -- keep the drafts on the path from the root to leaf[b]
 * ([B] int32, device memory; -1 keeps none) of the preceding
 * kvbuf_verify_tree with the same parent array: they move to consecutive
 * buffer positions after the buffered tokens (other drafts stay behind as
 * dead data) and the occupancy advances over them; with KVBUF_FLUSH_EAGER a
 * request whose buffer reaches m folds in the same kernel.
 */
kvbuf_status kvbuf_commit_tree(const kvbuf_layout* layout, const kvbuf_pools* pools,
                               const kvbuf_batch* batch, int32_t n, const int32_t* parent,
                               const int32_t* leaf, hipStream_t stream);

/*
 * kvbuf_verify_recurrent -- the verification that kvbuf_verify replaces
 * (Figure 2 caption: a system with only a state pool verifies drafts with the
 * recurrent form and keeps a temporary state for every draft).  Recurrent
 * mode only (m = 0).  For every request, drafts 0..n-1 are applied one at a
 * time to a copy of its state: draft d's output goes to out [B][n][H][d_v]
 * (layout->out_dtype) and the state after draft d to temp [n][B][H][d_k][d_v] fp32
 * (caller-owned device memory, n states per request).  The state pool is not
 * modified.  Inputs as kvbuf_verify.  Requires 1 <= n <= 8; a request
 * without a valid state slot sets KVBUF_DEVERR_SLOT and is skipped.
 */
kvbuf_status kvbuf_verify_recurrent(const kvbuf_layout* layout, const kvbuf_pools* pools,
                                    const kvbuf_batch* batch, int32_t n, const void* q,
                                    const void* k, const void* v, const float* g,
                                    const float* beta, void* out, float* temp,
                                    hipStream_t stream);

/*
 * kvbuf_commit_recurrent -- completes kvbuf_verify_recurrent: a request with
 * accepted[b] = a > 0 takes temp[a-1] as its state (Figure 2 caption: the
 * request's state is replaced by the temporary state of its last accepted
 * draft); a = 0 leaves it unchanged.  accepted: [B] int32, device memory;
 * a value outside [0, n] sets KVBUF_DEVERR_ACCEPT and skips the request.
 */
kvbuf_status kvbuf_commit_recurrent(const kvbuf_layout* layout, const kvbuf_pools* pools,
                                    const kvbuf_batch* batch, int32_t n,
                                    const int32_t* accepted, const float* temp,
                                    hipStream_t stream);

/*
 * kvbuf_direct -- decode from the buffer alone for every request, whatever its
 * state slot (abstract: a short request never gets a state; its buffer alone
 * yields its outputs).
 * Same arguments as kvbuf_decode; the state pool is never read or written and
 * no request folds.  Requires m > 0.
 */
kvbuf_status kvbuf_direct(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, void* out,
                          hipStream_t stream);

/*
 * kvbuf_materialize -- write every request's current effective state (its
 * state at the last fold, or zero without a slot, with all buffered tokens
 * applied) to states [B][H][d_k][d_v] fp32.  Reads only; pools, tables and
 * occupancies are unchanged.  For checkpointing, migration and checks.
 */
kvbuf_status kvbuf_materialize(const kvbuf_layout* layout, const kvbuf_pools* pools,
                               const kvbuf_batch* batch, float* states, hipStream_t stream);

/* Static description of a status code. */
const char* kvbuf_strerror(kvbuf_status status);

/* KVBUF_ABI_VERSION of the built library. */
int32_t kvbuf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVBUF_H */
