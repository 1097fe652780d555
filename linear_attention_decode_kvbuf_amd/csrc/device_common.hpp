// Device-side building blocks shared by the kvbuf kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbuf_internal.hpp"

namespace kvbuf {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;  // bfloat16 kept as its raw bits

// ---------------------------------------------------------------------------
// Tile geometry.  One workgroup owns one (request, head) tile: a d_k x d_v
// fp32 state read as rows of d_v floats.  A thread owns 4 consecutive columns
// (one 128-bit load per row) of RPT rows; TPR threads cover a row, RG row
// groups split the rows.  Row j of a thread is r = rg + RG * j, so the two row
// groups of a wave read two adjacent rows: every load instruction of a wave
// covers a contiguous 2 * d_v * 4 bytes.
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct Geo {
    static constexpr int NT = DV >= 128 ? 256 : (DV >= 64 ? 128 : 64);
    static constexpr int TPR = DV / 4;
    static constexpr int RG = NT / TPR;
    static constexpr int RPT = DK / RG;
    static_assert(TPR * RG == NT && RG * RPT == DK, "tile geometry");
    // Dot products (q . k over d_k) use groups of 16 lanes; each lane owns E
    // consecutive elements.
    static constexpr int DOT_LANES = 16;
    static constexpr int E = DK / DOT_LANES;
    static constexpr int GROUPS = NT / DOT_LANES;
};

// Tokens folded per LDS staging round.
constexpr int kFoldChunk = 32;

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const bf16_bits* p) { return bf2f(*p); }

// Four consecutive elements as fp32.
__device__ __forceinline__ f4 load4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 load4(const bf16_bits* p) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    f4 r;
    r.x = __uint_as_float(u.x << 16);
    r.y = __uint_as_float(u.x & 0xffff0000u);
    r.z = __uint_as_float(u.y << 16);
    r.w = __uint_as_float(u.y & 0xffff0000u);
    return r;
}

// E consecutive elements as fp32 (E = 1, 4 or 8).
template <int E>
__device__ __forceinline__ void loadE(const float* p, float (&o)[E]) {
    if constexpr (E == 1) {
        o[0] = p[0];
    } else {
#pragma unroll
        for (int i = 0; i < E; i += 4) {
            f4 x = load4(p + i);
            o[i] = x.x; o[i + 1] = x.y; o[i + 2] = x.z; o[i + 3] = x.w;
        }
    }
}
template <int E>
__device__ __forceinline__ void loadE(const bf16_bits* p, float (&o)[E]) {
    if constexpr (E == 1) {
        o[0] = load1(p);
    } else if constexpr (E == 4) {
        f4 x = load4(p);
        o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    } else {
        static_assert(E == 8, "dot lane width");
        uint4 u = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

// Sum over the 16 lanes of a dot group (butterfly through lane shuffles).
__device__ __forceinline__ float group16_sum(float x) {
    x += __shfl_xor(x, 8, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 1, 16);
    return x;
}

// Inclusive prefix sum of the log-gates of buffer positions 0 .. T-1 into
// bl[0 .. T-1] (LDS), done by wave 0 in 64-wide segments.  gate_at(i) returns
// the log-gate of position i.  Callers synchronise afterwards.
template <typename GateAt>
__device__ __forceinline__ void gate_prefix(float* bl, int T, GateAt gate_at) {
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    float carry = 0.0f;
    for (int base = 0; base < T; base += 64) {
        const int i = base + lane;
        float x = i < T ? gate_at(i) : 0.0f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        x += carry;
        if (i < T) bl[i] = x;
        carry = __shfl(x, 63, 64);
    }
}

// Positions of the buffer and of this call's new tokens for one tile.
// Position i < p lives in the pool; position p + d is new token d of this call
// (inputs laid out [B][n][H][d]).  XIO is the value plane's element type.
template <int DK, int DV, typename IO, typename XIO>
struct TileTokens {
    const IO* kpool;
    const XIO* xpool;
    const float* gpool;
    const int32_t* row;  // LDS copy of the request's table row
    int bs, H, h, p;
    const IO* kin;        // key of new token 0; new token d at kin + d * in_stride_k
    const IO* vin;
    const float* gin;     // gate of new token 0; new token d at gin + d * H
    size_t in_stride_k, in_stride_v;

    __device__ __forceinline__ size_t slot_index(int i) const {
        const int blk = row[i / bs];
        return (static_cast<size_t>(blk) * H + h) * bs + (i % bs);
    }
    __device__ __forceinline__ const IO* key(int i) const {
        return i < p ? kpool + slot_index(i) * DK : kin + (i - p) * in_stride_k;
    }
    // Buffered value (or delta-rule pseudo-value) of a pool position.
    __device__ __forceinline__ const XIO* pooled_value(int i) const { return xpool + slot_index(i) * DV; }
    __device__ __forceinline__ const IO* new_value(int d) const { return vin + d * in_stride_v; }
    __device__ __forceinline__ float gate(int i) const {
        return i < p ? gpool[slot_index(i)] : gin[(i - p) * H];
    }
};

// Orders this workgroup's reads of the request's metadata before the
// request's bookkeeping update, which the last of its H workgroups applies:
// the occupancy becomes new_occ and, when rotate > 0, the table row moves its
// first `rotate` entries to the back.  Every thread of the workgroup calls it;
// it must be the last thing the workgroup does with the metadata.
__device__ __forceinline__ void finish_request(const TileParams& P, int b, int new_occ, int rotate) {
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const int t = atomicAdd(&P.ticket[b], 1);
        s_last = (t == P.H - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const int bpr = P.blocks_per_req;
    int32_t* row = P.table + static_cast<size_t>(b) * bpr;
    int val = 0;
    const bool mine = rotate > 0 && static_cast<int>(threadIdx.x) < bpr;
    if (mine) val = __atomic_load_n(&row[(threadIdx.x + rotate) % bpr], __ATOMIC_RELAXED);
    __syncthreads();
    if (mine) row[threadIdx.x] = val;
    if (threadIdx.x == 0) {
        P.occ[b] = new_occ;
        P.ticket[b] = 0;
    }
}

__device__ __forceinline__ void report(const TileParams& P, unsigned bits) {
    if (bits && P.err && threadIdx.x == 0) atomicOr(reinterpret_cast<unsigned*>(P.err), bits);
}

// Checks the request's buffer positions [0, end) against the pool and copies
// the table row to LDS.  Returns KVBUF_DEVERR_* bits (0 = usable).
__device__ __forceinline__ unsigned load_row(const TileParams& P, int b, int end, int32_t* s_row) {
    const int bpr = P.blocks_per_req;
    const int cap = P.block_size * bpr;
    if (end < 0 || end > cap) return KVBUF_DEVERR_OVERFLOW;
    const int nblk = (end + P.block_size - 1) / P.block_size;
    unsigned bad = 0;
    for (int j = 0; j < nblk; ++j) {
        const int blk = P.table[static_cast<size_t>(b) * bpr + j];
        if (blk < 0 || blk >= P.num_blocks) bad |= KVBUF_DEVERR_BLOCK;
        if (threadIdx.x == 0) s_row[j] = blk;
    }
    return bad;
}

}  // namespace kvbuf
