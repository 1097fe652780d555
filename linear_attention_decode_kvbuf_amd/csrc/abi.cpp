// The C ABI of libkvbuf: argument validation on the host, then one kernel
// launch on the caller's stream (two for an eager decode whose m exceeds what
// the decode kernel folds itself).  No allocation, no synchronisation, no
// global mutable state.
#include <hip/hip_runtime.h>

#include "kvbuf.h"
#include "kvbuf_internal.hpp"

using kvbuf::TileParams;

namespace {

kvbuf_status check_layout(const kvbuf_layout* L, bool need_buffer) {
    if (!L) return KVBUF_EINVAL;
    if (L->num_heads <= 0 || L->d_k <= 0 || L->d_v <= 0 || L->m < 0) return KVBUF_EINVAL;
    if (L->num_state_slots < 0 || L->num_blocks < 0) return KVBUF_EINVAL;
    if (L->rule < KVBUF_RULE_LINEAR || L->rule > KVBUF_RULE_CHANNEL) return KVBUF_EUNSUPPORTED;
    if (L->io_dtype != KVBUF_BF16 && L->io_dtype != KVBUF_F32) return KVBUF_EUNSUPPORTED;
    if (L->flush != KVBUF_FLUSH_EAGER && L->flush != KVBUF_FLUSH_DEFERRED) return KVBUF_EINVAL;
    if (L->d_k != L->d_v || !kvbuf::supported_dim(L->d_k)) return KVBUF_EUNSUPPORTED;
    if (!(L->scale == L->scale)) return KVBUF_EINVAL;  // NaN scale
    if (L->out_dtype != KVBUF_OUT_F32 && L->out_dtype != KVBUF_OUT_BF16) return KVBUF_EINVAL;
    if (need_buffer && L->m == 0) return KVBUF_EUNSUPPORTED;
    if (L->m > 0) {
        if (L->block_size <= 0 || L->blocks_per_req <= 0 || L->num_blocks <= 0) return KVBUF_EINVAL;
        if (L->blocks_per_req > kvbuf::kMaxTableRow) return KVBUF_ECAPACITY;
        if (L->m % L->block_size != 0) return KVBUF_ECAPACITY;
        if (static_cast<long long>(L->block_size) * L->blocks_per_req < L->m) return KVBUF_ECAPACITY;
        if (static_cast<long long>(L->block_size) * L->blocks_per_req > kvbuf::kMaxCapacity) return KVBUF_ECAPACITY;
        // pool rows (block, head, slot) are indexed with 32-bit integers
        if (static_cast<long long>(L->num_blocks) * L->num_heads * L->block_size > 0x7fffffffLL)
            return KVBUF_ECAPACITY;
    }
    return KVBUF_OK;
}

kvbuf_status check_batch(const kvbuf_layout* L, const kvbuf_batch* B) {
    if (!B) return KVBUF_EINVAL;
    if (B->size < 0) return KVBUF_EINVAL;
    if (B->size == 0) return KVBUF_OK;
    if (!B->state_slot) return KVBUF_EINVAL;
    if (L->m == 0) return KVBUF_OK;  // recurrent mode: no buffer metadata
    if (!B->block_table || !B->occupancy || !B->tile_meta) return KVBUF_EINVAL;
    return KVBUF_OK;
}

// Grid size B * H must fit one launch dimension.
kvbuf_status check_grid(const kvbuf_layout* L, const kvbuf_batch* B) {
    if (static_cast<long long>(B->size) * L->num_heads > 0x7fffffffLL) return KVBUF_EINVAL;
    return KVBUF_OK;
}

kvbuf_status check_pools(const kvbuf_layout* L, const kvbuf_pools* P, bool need_state) {
    if (!P) return KVBUF_EINVAL;
    if (need_state && (!P->state || L->num_state_slots <= 0)) return KVBUF_EINVAL;
    if (L->m > 0) {
        if (!P->key || !P->value) return KVBUF_EINVAL;
        if (L->rule != KVBUF_RULE_LINEAR && !P->gate) return KVBUF_EINVAL;
    }
    return KVBUF_OK;
}

kvbuf_status check_tokens(const kvbuf_layout* L, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const void* out) {
    if (!q || !k || !v || !out) return KVBUF_EINVAL;
    if (L->rule != KVBUF_RULE_LINEAR && !g) return KVBUF_EINVAL;
    if (L->rule == KVBUF_RULE_DELTA && !beta) return KVBUF_EINVAL;
    return KVBUF_OK;
}

TileParams make_params(const kvbuf_layout* L, const kvbuf_pools* P, const kvbuf_batch* B) {
    TileParams t{};
    t.batch = B->size;
    t.H = L->num_heads;
    t.block_size = L->block_size;
    t.blocks_per_req = L->blocks_per_req;
    t.m = L->m;
    t.num_blocks = L->num_blocks;
    t.num_slots = L->num_state_slots;
    t.fuse = L->flush == KVBUF_FLUSH_EAGER;
    t.scale = L->scale;
    t.out_bf16 = L->out_dtype == KVBUF_OUT_BF16;
    t.state = P->state;
    t.key = P->key;
    t.value = P->value;
    t.gate = P->gate;
    t.slot = B->state_slot;
    t.table = B->block_table;
    t.occ = B->occupancy;
    t.tmeta = B->tile_meta;
    t.err = B->error;
    return t;
}

// Tokens staged in LDS per fold round for folds of up to `count` tokens.
int32_t fold_chunk(int count) { return count < kvbuf::kFoldChunk ? (count > 0 ? count : 1) : kvbuf::kFoldChunk; }

kvbuf_status from_hip(hipError_t e) { return e == hipSuccess ? KVBUF_OK : KVBUF_EHIP; }

#define KVBUF_TRY(x)                       \
    do {                                   \
        kvbuf_status st_ = (x);            \
        if (st_ != KVBUF_OK) return st_;   \
    } while (0)

kvbuf_status chunk_call(const kvbuf_layout* layout, const kvbuf_pools* pools,
                        const kvbuf_batch* batch, int mode, int n, const void* q,
                        const void* k, const void* v, const float* g, const float* beta,
                        void* out, hipStream_t stream, const int32_t* parent = nullptr) {
    const bool direct = mode == kvbuf::MODE_DIRECT;
    KVBUF_TRY(check_layout(layout, mode != kvbuf::MODE_DECODE));
    KVBUF_TRY(check_batch(layout, batch));
    KVBUF_TRY(check_pools(layout, pools, !direct));
    if (batch->size == 0) return KVBUF_OK;
    KVBUF_TRY(check_tokens(layout, q, k, v, g, beta, out));
    KVBUF_TRY(check_grid(layout, batch));
    if (mode == kvbuf::MODE_VERIFY) {
        if (n < 1 || n > kvbuf::kMaxDrafts) return KVBUF_EUNSUPPORTED;
        if (n > layout->block_size * layout->blocks_per_req) return KVBUF_ECAPACITY;
    }
    if (direct) {  // every rule, any capacity: the one-wave-per-tile kernel
        TileParams t = make_params(layout, pools, batch);
        t.mode = mode;
        t.n = 1;
        t.q = q;
        t.k = k;
        t.v = v;
        t.g = g;
        t.beta = beta;
        t.out = out;
        return from_hip(kvbuf::launch_direct(t, layout->rule, layout->d_k, layout->io_dtype, batch->size, stream));
    }
    TileParams t = make_params(layout, pools, batch);
    t.mode = mode;
    t.n = n;
    t.parent = parent;
    // A decode under the eager policy folds inside the decode kernel when the
    // m tokens fit its first staging pass; otherwise a fold launch follows it.
    const bool eager_decode = mode == kvbuf::MODE_DECODE && t.fuse && layout->m > 0;
    const bool fused = eager_decode &&
                       layout->m <= kvbuf::chunk_fold_limit(layout->rule, layout->d_k, layout->io_dtype, n,
                                                            layout->block_size * layout->blocks_per_req, layout->m,
                                                            static_cast<int64_t>(batch->size) * layout->num_heads);
    t.fold_chunk = fused ? layout->m : 0;
    t.q = q;
    t.k = k;
    t.v = v;
    t.g = g;
    t.beta = beta;
    t.out = out;
    if (layout->m == 0)
        return from_hip(kvbuf::launch_recurrent(t, layout->rule, layout->d_k, layout->io_dtype,
                                                batch->size, stream));
    hipError_t e = kvbuf::launch_chunk(t, layout->rule, layout->d_k, layout->io_dtype, batch->size, stream);
    if (e == hipSuccess && eager_decode && !fused) {
        t.mode = kvbuf::MODE_FLUSH;
        t.fold_chunk = fold_chunk(layout->m);
        t.sparse = 1;
        e = kvbuf::launch_fold(t, layout->rule, layout->d_k, layout->io_dtype, batch->size, stream);
    }
    return from_hip(e);
}

}  // namespace

extern "C" {

kvbuf_status kvbuf_decode(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, void* out,
                          hipStream_t stream) {
    return chunk_call(layout, pools, batch, kvbuf::MODE_DECODE, 1, q, k, v, g, beta, out, stream);
}

kvbuf_status kvbuf_direct(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, void* out,
                          hipStream_t stream) {
    return chunk_call(layout, pools, batch, kvbuf::MODE_DIRECT, 1, q, k, v, g, beta, out, stream);
}

kvbuf_status kvbuf_verify(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, int32_t n, const void* q,
                          const void* k, const void* v, const float* g,
                          const float* beta, void* out, hipStream_t stream) {
    return chunk_call(layout, pools, batch, kvbuf::MODE_VERIFY, n, q, k, v, g, beta, out, stream);
}

kvbuf_status kvbuf_flush(const kvbuf_layout* layout, const kvbuf_pools* pools,
                         const kvbuf_batch* batch, hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, false));
    KVBUF_TRY(check_batch(layout, batch));
    KVBUF_TRY(check_pools(layout, pools, true));
    if (batch->size == 0 || layout->m == 0) return KVBUF_OK;
    KVBUF_TRY(check_grid(layout, batch));
    TileParams t = make_params(layout, pools, batch);
    t.mode = kvbuf::MODE_FLUSH;
    t.fold_chunk = fold_chunk(layout->m);
    return from_hip(kvbuf::launch_fold(t, layout->rule, layout->d_k, layout->io_dtype, batch->size, stream));
}

kvbuf_status kvbuf_commit(const kvbuf_layout* layout, const kvbuf_pools* pools,
                          const kvbuf_batch* batch, int32_t n, const int32_t* accepted,
                          hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, true));
    KVBUF_TRY(check_batch(layout, batch));
    KVBUF_TRY(check_pools(layout, pools, true));
    if (batch->size == 0) return KVBUF_OK;
    if (!accepted) return KVBUF_EINVAL;
    if (n < 0 || n > kvbuf::kMaxDrafts) return KVBUF_EUNSUPPORTED;
    KVBUF_TRY(check_grid(layout, batch));
    TileParams t = make_params(layout, pools, batch);
    t.mode = kvbuf::MODE_COMMIT;
    t.n = n;
    t.fold_chunk = fold_chunk(layout->m);
    t.accepted = accepted;
    return from_hip(kvbuf::launch_fold(t, layout->rule, layout->d_k, layout->io_dtype, batch->size, stream));
}

kvbuf_status kvbuf_verify_tree(const kvbuf_layout* layout, const kvbuf_pools* pools,
                               const kvbuf_batch* batch, int32_t n, const int32_t* parent,
                               const void* q, const void* k, const void* v, const float* g,
                               const float* beta, void* out, hipStream_t stream) {
    if (!parent) return KVBUF_EINVAL;
    return chunk_call(layout, pools, batch, kvbuf::MODE_VERIFY, n, q, k, v, g, beta, out, stream, parent);
}

kvbuf_status kvbuf_commit_tree(const kvbuf_layout* layout, const kvbuf_pools* pools,
                               const kvbuf_batch* batch, int32_t n, const int32_t* parent,
                               const int32_t* leaf, hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, true));
    KVBUF_TRY(check_batch(layout, batch));
    KVBUF_TRY(check_pools(layout, pools, true));
    if (batch->size == 0) return KVBUF_OK;
    if (!parent || !leaf) return KVBUF_EINVAL;
    if (n < 1 || n > kvbuf::kMaxDrafts) return KVBUF_EUNSUPPORTED;
    KVBUF_TRY(check_grid(layout, batch));
    TileParams t = make_params(layout, pools, batch);
    t.mode = kvbuf::MODE_COMMIT;
    t.n = n;
    t.fold_chunk = fold_chunk(layout->m);
    t.parent = parent;
    t.leaf = leaf;
    return from_hip(kvbuf::launch_fold(t, layout->rule, layout->d_k, layout->io_dtype, batch->size, stream));
}

kvbuf_status kvbuf_verify_recurrent(const kvbuf_layout* layout, const kvbuf_pools* pools,
                                    const kvbuf_batch* batch, int32_t n, const void* q,
                                    const void* k, const void* v, const float* g,
                                    const float* beta, void* out, float* temp,
                                    hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, false));
    if (layout->m != 0) return KVBUF_EUNSUPPORTED;  // the baseline has no buffer
    KVBUF_TRY(check_batch(layout, batch));
    KVBUF_TRY(check_pools(layout, pools, true));
    if (batch->size == 0) return KVBUF_OK;
    KVBUF_TRY(check_tokens(layout, q, k, v, g, beta, out));
    if (!temp) return KVBUF_EINVAL;
    if (n < 1 || n > kvbuf::kMaxDrafts) return KVBUF_EUNSUPPORTED;
    KVBUF_TRY(check_grid(layout, batch));
    TileParams t = make_params(layout, pools, batch);
    t.mode = kvbuf::MODE_VERIFY;
    t.n = n;
    t.q = q;
    t.k = k;
    t.v = v;
    t.g = g;
    t.beta = beta;
    t.out = out;
    return from_hip(kvbuf::launch_verify_recurrent(t, layout->rule, layout->d_k, layout->io_dtype, temp, stream));
}

kvbuf_status kvbuf_commit_recurrent(const kvbuf_layout* layout, const kvbuf_pools* pools,
                                    const kvbuf_batch* batch, int32_t n,
                                    const int32_t* accepted, const float* temp,
                                    hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, false));
    if (layout->m != 0) return KVBUF_EUNSUPPORTED;
    KVBUF_TRY(check_batch(layout, batch));
    KVBUF_TRY(check_pools(layout, pools, true));
    if (batch->size == 0) return KVBUF_OK;
    if (!accepted || !temp) return KVBUF_EINVAL;
    if (n < 1 || n > kvbuf::kMaxDrafts) return KVBUF_EUNSUPPORTED;
    KVBUF_TRY(check_grid(layout, batch));
    TileParams t = make_params(layout, pools, batch);
    t.mode = kvbuf::MODE_COMMIT;
    t.n = n;
    t.accepted = accepted;
    return from_hip(kvbuf::launch_commit_recurrent(t, layout->d_k, temp, stream));
}

kvbuf_status kvbuf_materialize(const kvbuf_layout* layout, const kvbuf_pools* pools,
                               const kvbuf_batch* batch, float* states, hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, true));
    KVBUF_TRY(check_batch(layout, batch));
    KVBUF_TRY(check_pools(layout, pools, false));
    if (batch->size == 0) return KVBUF_OK;
    if (!states) return KVBUF_EINVAL;
    KVBUF_TRY(check_grid(layout, batch));
    TileParams t = make_params(layout, pools, batch);
    t.mode = kvbuf::MODE_MATERIALIZE;
    t.fold_chunk = fold_chunk(layout->block_size * layout->blocks_per_req);
    t.states_out = states;
    return from_hip(kvbuf::launch_fold(t, layout->rule, layout->d_k, layout->io_dtype,
                                       batch->size, stream));
}

kvbuf_status kvbuf_admit(const kvbuf_layout* layout, const kvbuf_batch* batch, const int32_t* requests,
                         int32_t count, hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, true));
    KVBUF_TRY(check_batch(layout, batch));
    if (batch->size == 0) return KVBUF_OK;
    if (requests && count < 0) return KVBUF_EINVAL;
    const int n = requests ? count : batch->size;
    if (n == 0) return KVBUF_OK;
    KVBUF_TRY(check_grid(layout, batch));
    kvbuf_pools none{};
    TileParams t = make_params(layout, &none, batch);
    return from_hip(kvbuf::launch_admit(t, requests, n, stream));
}

kvbuf_status kvbuf_check(const kvbuf_layout* layout, const kvbuf_batch* batch, hipStream_t stream) {
    KVBUF_TRY(check_layout(layout, true));
    KVBUF_TRY(check_batch(layout, batch));
    if (batch->size == 0) return KVBUF_OK;
    if (!batch->error) return KVBUF_EINVAL;
    KVBUF_TRY(check_grid(layout, batch));
    kvbuf_pools none{};
    TileParams t = make_params(layout, &none, batch);
    return from_hip(kvbuf::launch_check(t, stream));
}

const char* kvbuf_strerror(kvbuf_status status) {
    switch (status) {
        case KVBUF_OK: return "success";
        case KVBUF_EINVAL: return "invalid argument (null pointer, negative size or inconsistent layout)";
        case KVBUF_EUNSUPPORTED: return "unsupported head dims, dtype, rule or mode";
        case KVBUF_ECAPACITY: return "buffer capacity: m must be a multiple of block_size and fit the table";
        case KVBUF_EHIP: return "HIP runtime error at launch";
    }
    return "unknown kvbuf status";
}

int32_t kvbuf_abi_version(void) { return KVBUF_ABI_VERSION; }

}  // extern "C"
