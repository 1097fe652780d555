// Device-side building blocks shared by the kvbuf kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbuf_internal.hpp"

namespace kvbuf {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;  // bfloat16 kept as its raw bits

// ---------------------------------------------------------------------------
// Workgroup layout.  One workgroup owns one (request, head) tile: a d_k x d_v
// fp32 state read as rows of d_v floats.
//
// The first NT threads ("state waves") hold the tile in registers: a thread
// owns 4 consecutive columns (one 128-bit load per row) of RPT consecutive
// rows r = rg * RPT + j; TPR threads cover a row and RG row groups split the
// rows.  Every load instruction of a wave covers whole 512-byte rows, and a
// thread's rows are 512 bytes apart, so its RPT loads need only two base
// addresses (the immediate offset reaches 4 KiB).
//
// One more wave ("token wave", 64 lanes) does everything that depends on the
// individual tokens: staging queries, gate prefix sums, q . k scores, the
// weighted sum of buffered values, fold staging and the appends.  The wave's
// memory counter is private, so the state waves' 16 outstanding loads are
// never waited on before they are needed: they stay in flight while the token
// wave works, and the two sides meet at one barrier.
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct Geo {
    static constexpr int NT = DV >= 128 ? 256 : (DV >= 64 ? 128 : 64);  // state threads
    static constexpr int NTOK = 64;                                     // token wave
    static constexpr int NTHREADS = NT + NTOK;
    static constexpr int TPR = DV / 4;
    static constexpr int RG = NT / TPR;
    static constexpr int RPT = DK / RG;
    static_assert(TPR * RG == NT && RG * RPT == DK, "tile geometry");
    // Dot products (q . k over d_k) use groups of 16 lanes of the token wave;
    // each lane owns E consecutive elements.
    static constexpr int DOT_LANES = 16;
    static constexpr int E = DK / DOT_LANES;
    static constexpr int GROUPS = NTOK / DOT_LANES;
    // Value columns per token-wave lane in the buffer sums.
    static constexpr int CPL = DV >= 64 ? DV / 64 : 1;
};

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

// A lane's share of one token row when 16 lanes split the row: E consecutive
// elements of type T kept as raw bits, so that a batch of loads can be
// issued before any of them is waited on.
template <typename T, int E>
struct RawChunk {
    static constexpr int BYTES = E * static_cast<int>(sizeof(T));
    static constexpr int WORDS = BYTES >= 4 ? BYTES / 4 : 1;
    uint32_t w[WORDS];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < WORDS; ++i) w[i] = 0u;
    }
    __device__ __forceinline__ void load(const T* p) {
        if constexpr (BYTES >= 16) {
#pragma unroll
            for (int i = 0; i < WORDS; i += 4) {
                const uint4 u = reinterpret_cast<const uint4*>(p)[i / 4];
                w[i] = u.x; w[i + 1] = u.y; w[i + 2] = u.z; w[i + 3] = u.w;
            }
        } else if constexpr (BYTES == 8) {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            w[0] = u.x; w[1] = u.y;
        } else if constexpr (BYTES == 4) {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        } else {
            w[0] = *reinterpret_cast<const uint16_t*>(p);
        }
    }
    __device__ __forceinline__ void store(T* p) const {
        if constexpr (BYTES >= 16) {
#pragma unroll
            for (int i = 0; i < WORDS; i += 4)
                reinterpret_cast<uint4*>(p)[i / 4] = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
        } else if constexpr (BYTES == 8) {
            *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        } else if constexpr (BYTES == 4) {
            *reinterpret_cast<uint32_t*>(p) = w[0];
        } else {
            *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(w[0]);
        }
    }
    __device__ __forceinline__ void to_float(float (&o)[E]) const {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < E; ++i) o[i] = __uint_as_float(w[i]);
        } else if constexpr (E == 1) {
            o[0] = __uint_as_float(w[0] << 16);
        } else {
#pragma unroll
            for (int i = 0; i < E / 2; ++i) {
                o[2 * i] = __uint_as_float(w[i] << 16);
                o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    }
};

// Sum over the 16 lanes of a dot group (butterfly through lane shuffles).
__device__ __forceinline__ float group16_sum(float x) {
    x += __shfl_xor(x, 8, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 1, 16);
    return x;
}

// Inclusive prefix sum of the log-gates of buffer positions 0 .. T-1 into
// bl[0 .. T-1] (LDS), by one wave (lane = 0..63) in 64-wide segments.
// gate_at(i) returns the log-gate of position i.
template <typename GateAt>
__device__ __forceinline__ void gate_prefix(float* bl, int T, int lane, GateAt gate_at) {
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

// Token wave: copies the keys and values of positions i0 .. i0+cnt-1 of the
// tile to LDS as fp32 rows (fk: d_k per row, fx: d_v per row).  Sixteen lanes
// share a row (one 16-byte load each for bf16 rows of 128), four rows per
// round, and the loads of two rounds are issued before any is used, so a
// round trip to HBM is paid once per 8 rows.  Values of positions >= tok.p
// come from `un` (delta-rule pseudo-values already in LDS) when given, else
// from this call's inputs.
template <int DK, int DV, typename IO, typename XIO>
__device__ __forceinline__ void stage_rows(const TileTokens<DK, DV, IO, XIO>& tok, int i0, int cnt,
                                           float* fk, float* fx, const float* un, int lane) {
    constexpr int E = DK / 16, EV = DV / 16, NB = 2;
    const int gl = lane >> 4, cl = lane & 15;
    for (int b0 = 0; b0 < cnt; b0 += 4 * NB) {
        RawChunk<IO, E> kr[NB];
        RawChunk<XIO, EV> xr[NB];
#pragma unroll
        for (int rr = 0; rr < NB; ++rr) {
            const int ii = b0 + 4 * rr + gl;
            const int i = i0 + ii;
            kr[rr].zero();
            xr[rr].zero();
            if (ii < cnt) {
                kr[rr].load(tok.key(i) + cl * E);
                if (i < tok.p) {
                    xr[rr].load(tok.pooled_value(i) + cl * EV);
                } else if constexpr (std::is_same<XIO, IO>::value) {
                    if (!un) xr[rr].load(tok.new_value(i - tok.p) + cl * EV);
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < NB; ++rr) {
            const int ii = b0 + 4 * rr + gl;
            const int i = i0 + ii;
            if (ii < cnt) {
                float kf[E], xf[EV];
                kr[rr].to_float(kf);
                xr[rr].to_float(xf);
                if (i >= tok.p && un) {
#pragma unroll
                    for (int e = 0; e < EV; ++e) xf[e] = un[(i - tok.p) * DV + cl * EV + e];
                }
#pragma unroll
                for (int e = 0; e < E; ++e) fk[ii * DK + cl * E + e] = kf[e];
#pragma unroll
                for (int e = 0; e < EV; ++e) fx[ii * DV + cl * EV + e] = xf[e];
            }
        }
    }
}

// Workgroups are numbered head-major: workgroup w serves request w % B and
// head w / B.  The H workgroups of one request are therefore dispatched B
// apart instead of back to back, so their per-request ticket atomics (one
// counter per request) do not queue up on one address at the same moment.
struct TileIndex {
    int b, h;
};
__device__ __forceinline__ TileIndex tile_index(const TileParams& P) {
    const int w = blockIdx.x;
    const int h = w / P.batch;
    return TileIndex{w - h * P.batch, h};
}

// Per-request bookkeeping.  All H workgroups of a request read its occupancy,
// state slot and table row; the last of them to finish with those values
// (found with a per-request ticket counter) applies the update: the occupancy
// becomes new_occ and, when rotate > 0, the first `rotate` table entries move
// to the back; then it clears the ticket.
//
// take_ticket is called by one thread after a barrier that follows every
// read of the metadata by every wave of the workgroup, so those reads have
// completed; nothing in the kernel reads the metadata afterwards (the table
// row used later is an LDS copy).  No memory fence is needed -- an agent-scope
// fence would write back the XCD's whole L2 for every workgroup -- because
// the bookkeeping stores only have to be visible to the next kernel, which the
// kernel boundary guarantees.  The ticket's round trip overlaps the rest of
// the workgroup's work; its result is read after a later barrier.
__device__ __forceinline__ int take_ticket(const TileParams& P, int b) {
    return atomicAdd(&P.ticket[b], 1) == P.H - 1;
}

// Every thread of the workgroup calls this last; `last` is take_ticket's
// result (as seen after a barrier).
__device__ __forceinline__ void apply_bookkeeping(const TileParams& P, int b, bool last, int new_occ,
                                                  int rotate) {
    if (!last) return;
    const int bpr = P.blocks_per_req;
    int32_t* row = P.table + static_cast<size_t>(b) * bpr;
    int val = 0;
    const bool mine = rotate > 0 && static_cast<int>(threadIdx.x) < bpr;
    if (mine) val = row[(threadIdx.x + rotate) % bpr];
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

// One wave (lane = 0..63) copies the request's whole table row to LDS with a
// single vector load -- it does not wait for the occupancy, so the row and
// the occupancy arrive in the same round trip -- and checks the block ids
// that cover buffer positions [0, end).  Returns KVBUF_DEVERR_* bits, the
// same in every lane (0 = usable).
__device__ __forceinline__ unsigned stage_row(const TileParams& P, int b, int end, int32_t* s_row, int lane) {
    const int bpr = P.blocks_per_req;  // <= 64 (host-checked)
    int blk = 0;
    if (lane < bpr) {
        blk = P.table[static_cast<size_t>(b) * bpr + lane];
        s_row[lane] = blk;
    }
    const int cap = P.block_size * bpr;
    if (end < 0 || end > cap) return KVBUF_DEVERR_OVERFLOW;
    const int nblk = (end + P.block_size - 1) / P.block_size;
    const bool badblk = lane < nblk && (blk < 0 || blk >= P.num_blocks);
    return __ballot(badblk) ? KVBUF_DEVERR_BLOCK : 0u;
}

}  // namespace kvbuf
