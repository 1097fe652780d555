// Per-request buffer metadata and the per-tile copies the kernels work on.
//
// The caller keeps one occupancy [B] and one block-table row [B][bpr] per
// request (KVBuffer: IO-aware Serving for Linear Attention, pith.science
// page, Figure 1 caption: a request owns its buffer blocks and one state
// slot).  The kernels of a call read and advance a copy per (request, head)
// -- each tile's workgroup owns its copy, so a call needs no synchronisation
// across workgroups -- and head 0's workgroup writes the request's new values
// back to the per-request arrays.  kvbuf_admit copies the per-request values
// into the copies (after the caller has written a new request's row and
// occupancy); kvbuf_check compares them.
#include "device_common.hpp"

namespace kvbuf {
namespace {

// One thread per (listed request, head): the request's occupancy and table
// row into that head's record.  A listed index outside [0, B) is reported.
__global__ __launch_bounds__(256) void admit_kernel(TileParams P, const int32_t* req, int count) {
    const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= static_cast<long long>(count) * P.H) return;
    const int k = static_cast<int>(t / P.H);
    const int h = static_cast<int>(t - static_cast<long long>(k) * P.H);
    const int b = req ? req[k] : k;
    if (b < 0 || b >= P.batch) {
        if (h == 0 && P.err) atomicOr(reinterpret_cast<unsigned*>(P.err), KVBUF_DEVERR_META);
        return;
    }
    const int bpr = P.blocks_per_req;
    int32_t* rec = tile_meta(P, b, h);
    rec[0] = P.occ[b];
    for (int i = 0; i < bpr; ++i) rec[1 + i] = P.table[static_cast<size_t>(b) * bpr + i];
}

// One thread per tile: its record against the request's values.
__global__ __launch_bounds__(256) void check_kernel(TileParams P) {
    const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= static_cast<long long>(P.batch) * P.H) return;
    const int b = static_cast<int>(t / P.H);
    const int h = static_cast<int>(t - static_cast<long long>(b) * P.H);
    const int bpr = P.blocks_per_req;
    const int32_t* rec = tile_meta(P, b, h);
    bool same = rec[0] == P.occ[b];
    for (int i = 0; i < bpr; ++i) same = same && rec[1 + i] == P.table[static_cast<size_t>(b) * bpr + i];
    if (!same && P.err) atomicOr(reinterpret_cast<unsigned*>(P.err), KVBUF_DEVERR_META);
}

}  // namespace

hipError_t launch_admit(const TileParams& p, const int32_t* requests, int count, hipStream_t s) {
    const long long n = static_cast<long long>(count) * p.H;
    admit_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(p, requests, count);
    return hipGetLastError();
}

hipError_t launch_check(const TileParams& p, hipStream_t s) {
    const long long n = static_cast<long long>(p.batch) * p.H;
    check_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace kvbuf
