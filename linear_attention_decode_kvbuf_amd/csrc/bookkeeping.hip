// Per-request bookkeeping after a decode, direct decode, flush or commit
// launch: advance the occupancy over the tokens the launch appended or kept,
// and after a fold move the m / block_size leading table entries to the back
// and lower the occupancy by m (KVBuffer: IO-aware Serving for Linear
// Attention, pith.science page, Figure 1 caption: the buffer is partitioned
// into blocks owned by the request; once the state has absorbed the buffered
// tokens their blocks are free for the next ones).
//
// It runs as its own small launch after the compute launch in stream order,
// so every workgroup of that launch has finished with the request's
// metadata: no atomics and no workspace are needed.  It repeats the compute
// kernel's checks and fold decision exactly, so a request the compute kernel
// skipped (bad metadata) is left unchanged.  One wave per request; lane j
// owns table entry j (a row has at most 64 entries), so the rotation is one
// cross-lane move: every lane reads before any lane writes.
#include "device_common.hpp"

namespace kvbuf {
namespace {

constexpr int kAdvanceWaves = 4;  // requests per workgroup

__global__ __launch_bounds__(64 * kAdvanceWaves) void advance_kernel(TileParams P) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kAdvanceWaves + (threadIdx.x >> 6);
    if (b >= P.batch) return;
    const int bs = P.block_size;
    const int bpr = P.blocks_per_req;
    const int cap = bs * bpr;
    const bool direct = P.mode == MODE_DIRECT;
    // every load is issued before any result is used: one round trip
    int32_t* row = P.table + static_cast<size_t>(b) * bpr;
    const int p = P.occ[b];
    const int slot = direct ? -1 : P.slot[b];
    const int a = P.mode == MODE_COMMIT ? P.accepted[b] : 0;
    const int blk = lane < bpr ? row[lane] : 0;
    const bool has_state = slot >= 0;

    int pn = p;           // occupancy after this launch's appends / kept drafts
    bool fold = false;
    int checked = 0;      // buffer positions whose blocks the compute kernel checked
    bool bad = p < 0 || p > cap || slot >= P.num_slots;  // (then p + n cannot overflow)
    if (P.mode == MODE_DECODE || P.mode == MODE_DIRECT) {
        pn = p + P.n;
        checked = pn;
        fold = P.fold_chunk > 0 && has_state && pn >= P.m;
    } else {  // MODE_FLUSH or MODE_COMMIT
        if (P.mode == MODE_COMMIT) {
            bad = bad || a < 0 || a > P.n;
            pn = p + a;
        }
        fold = has_state && P.m > 0 && pn >= P.m && (P.mode == MODE_FLUSH || P.fuse);
        checked = fold ? P.m : 0;
    }
    bad = bad || pn > cap;
    if (bad) return;
    const int nblk = (checked + bs - 1) / bs;
    if (__ballot(lane < nblk && (blk < 0 || blk >= P.num_blocks)) != 0) return;
    if (fold) {
        const int k = P.m / bs;  // blocks consumed by the fold move to the back
        const int src = lane + k < bpr ? lane + k : lane + k - bpr;
        const int moved = __shfl(blk, src);
        if (lane < bpr) row[lane] = moved;
        pn -= P.m;
    }
    if (lane == 0) P.occ[b] = pn;
}

}  // namespace

hipError_t launch_advance(const TileParams& p, hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>((p.batch + kAdvanceWaves - 1) / kAdvanceWaves);
    advance_kernel<<<dim3(blocks), dim3(64 * kAdvanceWaves), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace kvbuf
