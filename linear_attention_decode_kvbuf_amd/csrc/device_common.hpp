// Device-side building blocks shared by the kvbuf kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbuf_internal.hpp"

namespace kvbuf {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;  // bfloat16 kept as its raw bits

// Word 3 of a raw (untyped) buffer resource on gfx9-family GPUs, and the
// cache-policy bits of a non-temporal access.
constexpr int kBufferFlags = 0x00020000;
constexpr int kCachePolicyNT = 2;

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
// An element kept as loaded, converted where it is used.  The bf16 widening
// is written as one instruction of inline assembly so that the optimizer
// cannot move it next to the load (a conditional load joined with a
// constant otherwise has the shift folded into its branch, which then waits
// for the load, and with it for everything the wave issued before it).
__device__ __forceinline__ float as_float(float x) { return x; }
__device__ __forceinline__ float as_float(bf16_bits x) {
    const uint32_t v = x;
    float f;
    asm("v_lshlrev_b32 %0, 16, %1" : "=v"(f) : "v"(v));
    return f;
}

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
    // element i as fp32 (i a compile-time index after unrolling)
    __device__ __forceinline__ float at(int i) const {
        if constexpr (sizeof(T) == 4) return __uint_as_float(w[i]);
        else if constexpr (E == 1) return __uint_as_float(w[0] << 16);
        else return (i & 1) ? __uint_as_float(w[i / 2] & 0xffff0000u) : __uint_as_float(w[i / 2] << 16);
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

// q . k over one 16-lane share of a row, from raw chunks (bf16 pairs through
// the packed bf16 dot instruction: the products are exact in fp32).
template <typename T, int E>
__device__ __forceinline__ float chunk_dot(const RawChunk<T, E>& a, const RawChunk<T, E>& b) {
    float acc = 0.f;
    if constexpr (sizeof(T) == 2 && E >= 2) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int w = 0; w < RawChunk<T, E>::WORDS; ++w)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a.w[w]), __builtin_bit_cast(bf2, b.w[w]),
                                                  acc, false);
    } else {
        float x[E], y[E];
        a.to_float(x);
        b.to_float(y);
#pragma unroll
        for (int e = 0; e < E; ++e) acc += x[e] * y[e];
    }
    return acc;
}

// Issues the RPT 128-bit loads of a thread's share of a d_k x d_v fp32
// state tile (rows rg*RPT .. rg*RPT+RPT-1, columns c0 .. c0+3) as buffer
// loads through a range-checked resource.  A request without a state passes
// present = false: the range is empty and every load returns zeros without
// touching memory.  The loads are unconditional instructions either way, so
// the compiler's memory-counter bookkeeping stays exact for loads issued
// before them (a branch around them would make it wait for everything).
// Non-temporal: a tile is not read again before it is evicted.
template <int RPT, int DK, int DV>
__device__ __forceinline__ void load_tile(f4 (&s)[RPT], const float* tile, bool present, int rg, int c0) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(tile), 0, present ? DK * DV * static_cast<int>(sizeof(float)) : 0, kBufferFlags);
    const int v = (rg * RPT * DV + c0) * static_cast<int>(sizeof(float));
#pragma unroll
    for (int j = 0; j < RPT; ++j)
        s[j] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, v, j * DV * 4, kCachePolicyNT));
}

// DPP lane permutation of a float within each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a dot group (one DPP row): swap neighbours, swap
// pairs, mirror within 8, mirror within 16 -- every lane ends with the sum.
// DPP needs no lane-index registers, unlike a shuffle through LDS permute.
__device__ __forceinline__ float group16_sum(float x) {
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);  // row_half_mirror
    x += dpp_f<0x140>(x);  // row_mirror
    return x;
}

// e^x through the hardware base-2 exponential.  The arguments here are sums
// of log-gates (|x| below about 10), where the relative error stays under
// 1e-6.
__device__ __forceinline__ float exp_gate(float x) { return __expf(x); }

// Output element i of a call: fp32, or rounded to the nearest bf16 (ties to
// even) when the layout asks for bf16 outputs.
__device__ __forceinline__ void store_out(const TileParams& P, size_t i, float v) {
    if (P.out_bf16) static_cast<__bf16*>(P.out)[i] = static_cast<__bf16>(v);
    else static_cast<float*>(P.out)[i] = v;
}

// Inclusive prefix sum of the log-gates of buffer positions 0 .. T-1 into
// bl[0 .. T-1] (LDS), by one wave (lane = 0..63) in 64-wide segments.
// gate_at(i) returns the log-gate of position i (cheap: from LDS).
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

// The same when gate_at reads device memory: the gates of every segment are
// requested before the first is summed (one round trip for a buffer of any
// length; T <= kMaxCapacity; eight registers per lane).  All eight loads are
// issued whatever T, with no branch between them -- segments past the end
// read position T - 1 again and count as zeros -- since loads under a branch
// each end with a wait for the counter to drain.
template <typename GateAt>
__device__ __forceinline__ void gate_prefix_loads(float* bl, int T, int lane, GateAt gate_at) {
    constexpr int KS = kMaxCapacity / 64;
    if (T <= 0) return;
    float g[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) g[k] = gate_at(min(64 * k + lane, T - 1));
    float carry = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        if (64 * k < T) {
            const int i = 64 * k + lane;
            float x = i < T ? g[k] : 0.0f;
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
}

// Positions of the buffer and of this call's new tokens for one tile.
// Position i < p lives in the pool at row pos[i] (a row = one token of one
// head; pos is the LDS table stage_row builds); position p + d is new token d
// of this call (inputs laid out [B][n][H][d]).  XIO is the value plane's
// element type.
template <int DK, int DV, typename IO, typename XIO>
struct TileTokens {
    const IO* kpool;
    const XIO* xpool;
    const float* gpool;
    const uint32_t* pos;  // pool row of each buffer position (LDS)
    int H, p;
    const IO* kin;        // key of new token 0; new token d at kin + d * in_stride_k
    const IO* vin;
    const float* gin;     // gate of new token 0; new token d at gin + d * H
    size_t in_stride_k, in_stride_v;

    __device__ __forceinline__ size_t slot_index(int i) const { return pos[i]; }
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

// One direct-to-LDS copy instruction: lane L's 16 bytes at src land at LDS
// byte window + 16 L (window uniform across the wave, 16-byte aligned).  It
// is written as inline assembly so that the compiler does not track it.  A
// tracked copy makes the compiler wait for every outstanding load of the
// wave -- a whole state tile, say -- before the next LDS read that might
// alias the copied bytes, and at a loop head or a branch join it assumes the
// worst; here the LDS rows a copy fills are read only after an explicit wait
// on the wave's copies (s_waitcnt vmcnt) and, by other waves, after a
// barrier.  Instructions the compiler does not count only lengthen its own
// vmcnt waits, never shorten them.  The copy writes no register.  It sets
// m0, which the compiler may not treat as clobbered (it warns so); the
// compiler's own code for these kernels never uses m0 (none in their
// generated assembly outside these copies), so nothing it holds there is
// lost.
__device__ __forceinline__ uint32_t lds_byte_address(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}
__device__ __forceinline__ void lds_dma16(const void* src, void* window) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_byte_address(window));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0) : "memory", "m0");
}

// Direct-to-LDS copy of `rows` rows of RB bytes (RB a multiple of 16, at
// most 1 KiB) by one wave: row i is read from src(i) and lands at dst + i RB.
// One instruction carries 1 KiB, 16 bytes per lane: lane L writes dst + 16 L
// of its window, holding bytes 16 (L mod RB/16) .. of row L / (RB/16).  dst
// must be 16-byte aligned.  src may use wave shuffles: every lane calls it.
template <int RB, typename SrcOf>
__device__ __forceinline__ void lds_copy_rows(char* dst, int rows, SrcOf src, int lane) {
    static_assert(RB % 16 == 0 && RB <= 1024, "whole 16-byte lanes of a 1 KiB copy");
    constexpr int LPR = RB / 16;   // lanes per row
    constexpr int RPI = 64 / LPR;  // rows per instruction
    const int rr = lane / LPR;
    const int off = (lane % LPR) * 16;
    for (int r0 = 0; r0 < rows; r0 += RPI) {
        const int row = r0 + rr;
        const char* a = src(row < rows ? row : r0) + off;
        if (row < rows) lds_dma16(a, dst + r0 * RB);
    }
}

// The copies count on the wave's vector-memory counter and land in LDS
// asynchronously; the compiler does not reliably order LDS reads of the rows
// after them, so the wave waits for the counter to drain (vmcnt(0) in the
// gfx9 encoding) and keeps the scheduler from moving anything across.
__device__ __forceinline__ void wait_lds_copies() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroups are numbered head-major: workgroup w serves request w % B and
// head w / B, so consecutive workgroups stream different requests' state
// slots and buffer blocks.
struct TileIndex {
    int b, h;
};
__device__ __forceinline__ TileIndex tile_index(const TileParams& P) {
    const int w = blockIdx.x;
    const int h = w / P.batch;
    return TileIndex{w - h * P.batch, h};
}

__device__ __forceinline__ void report(const TileParams& P, unsigned bits) {
    if (bits && P.err && threadIdx.x == 0) atomicOr(reinterpret_cast<unsigned*>(P.err), bits);
}

// Buffer metadata: the caller sees one occupancy [B] and one table row
// [B][blocks_per_req] per request; the kernels read and advance per-tile
// copies, a record [B][H][1 + blocks_per_req] (occupancy, then the row) per
// (request, head).  The workgroup serving tile (b, h) is the only one that
// reads or writes its record, so it updates it in place once it is done
// reading it -- with no atomics, fences or second launch; within a workgroup
// one wave does the reads and the update, so program order alone separates
// them.  The workgroup of head 0 also writes the request's new values to the
// per-request arrays, which no kernel reads during a call (kvbuf_admit copies
// them into the records; kvbuf_check compares them).
__device__ __forceinline__ int32_t* tile_meta(const TileParams& P, int b, int h) {
    return P.tmeta + (static_cast<size_t>(b) * P.H + h) * (1 + P.blocks_per_req);
}
__device__ __forceinline__ int load_occupancy(const TileParams& P, int b, int h) { return tile_meta(P, b, h)[0]; }

// The tile's occupancy <- v (one lane), and the request's if h = 0.
__device__ __forceinline__ void store_occupancy(const TileParams& P, int b, int h, int v) {
    tile_meta(P, b, h)[0] = v;
    if (h == 0) P.occ[b] = v;
}

// By the wave that read the metadata (lane = 0..63, all active; blk = table
// entry `lane` as read, see load_table_row): occupancy <- p_new and, when
// k > 0, the first k table entries move to the back (the blocks a fold
// consumed), rotated in registers -- re-reading the row would put a round
// trip at the end of the wave's chain.
__device__ __forceinline__ void update_meta(const TileParams& P, int b, int h, int p_new, int k, int lane,
                                            int blk) {
    int32_t* rec = tile_meta(P, b, h);
    const int bpr = P.blocks_per_req;
    if (k > 0) {
        const int src = lane + k < bpr ? lane + k : lane + k - bpr;
        const int v = __shfl(blk, src & 63, 64);
        if (lane < bpr) {
            rec[1 + lane] = v;
            if (h == 0) P.table[static_cast<size_t>(b) * bpr + lane] = v;
        }
    }
    if (lane == 0) store_occupancy(P, b, h, p_new);
}

// One wave (lane = 0..63) reads the tile's whole table row with a single
// vector load (load_table_row: lane i gets entry i) -- it does not wait for
// the occupancy, so the row and the occupancy arrive in the same round trip --
// and stage_row_from writes, for every buffer position i < capacity, its pool
// row (block * H + h) * block_size + i mod block_size to pos[i] in LDS, so
// that later address arithmetic is one lookup.  (The host bounds num_blocks *
// H * block_size below 2^31.)  It checks the block ids covering positions
// [0, end) and returns KVBUF_DEVERR_* bits, the same in every lane (0 =
// usable).
__device__ __forceinline__ unsigned stage_row_from(const TileParams& P, int h, int end, uint32_t* pos, int lane,
                                                   int blk) {
    const int bpr = P.blocks_per_req;
    const int bs = P.block_size;
    const int cap = bs * bpr;
    // A lane permute reads zero from an inactive source lane, so every pass
    // runs with all 64 lanes active (a uniform trip count, the source index
    // clamped into the row) and only the store is guarded: a loop over
    // i < cap would leave the lanes past the end of the last partial pass
    // inactive while the lanes before them fetch block ids from them.
    for (int base = 0; base < cap; base += 64) {
        const int i = base + lane;
        const int q = min(i / bs, bpr - 1);
        const uint32_t bi = static_cast<uint32_t>(__shfl(blk, q, 64));
        if (i < cap)
            pos[i] = (bi * static_cast<uint32_t>(P.H) + static_cast<uint32_t>(h)) * static_cast<uint32_t>(bs) +
                     static_cast<uint32_t>(i - q * bs);
    }
    if (end < 0 || end > cap) return KVBUF_DEVERR_OVERFLOW;
    const int nblk = (end + bs - 1) / bs;
    const bool badblk = lane < nblk && (blk < 0 || blk >= P.num_blocks);
    return __ballot(badblk) ? KVBUF_DEVERR_BLOCK : 0u;
}
__device__ __forceinline__ int load_table_row(const TileParams& P, int b, int h, int lane) {
    const int bpr = P.blocks_per_req;  // <= 64 (host-checked)
    return lane < bpr ? tile_meta(P, b, h)[1 + lane] : 0;
}

}  // namespace kvbuf
