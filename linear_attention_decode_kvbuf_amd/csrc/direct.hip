// Buffer-only decode (kvbuf_direct): one wave per (request, head) tile.
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page,
// abstract: a short request never gets a state; its buffer alone yields its
// outputs; Figure 5 caption: the buffer-only form is compared with the
// recurrent and chunkwise forms over context lengths).  With no state the
// output of the new token t = p (b_i the cumulative log-gate of position i):
//   o_t = sum_{i<=t} e^{b_t - b_i} scale (q_t . k_i) x_i
// with x_i = v_i (linear, gated rules) or, for the delta rule, the stored
// pseudo-value u_i of a buffered position and for the new token
//   u_t = beta_t (v_t - sum_{i<t} e^{b_t - b_i} (k_t . k_i) u_i).
// With one log-gate per key channel the decay is a vector acting on the key
// channels: q_t . k_i becomes sum_r q_t[r] k_i[r] e^{B_t[r] - B_i[r]}.
//
// A tile without a state moves only its buffered rows (up to 772 bytes per
// position at d = 128), so the work is latency-bound unless many tiles are in
// flight.  Each wave serves one tile on its own -- no workgroup barrier, a
// few dozen registers -- so a compute unit keeps several times more tiles in
// flight than a one-workgroup-per-tile kernel:
//  * lane l owns key channels and value columns C l .. C l + C - 1 (C = d/64;
//    one of them at d <= 64), so a buffered row is one coalesced load per
//    plane;
//  * rows stream through registers in batches of 8 positions, the next
//    batch requested before the current one is used;
//  * the 8 dot products of a batch are summed over the wave with one
//    transposing reduction (10 lane exchanges instead of 48);
//  * scalar gates: the cumulative log-gates of all positions (one load per
//    lane per 64 positions, a wave scan) give every position's weight, kept
//    in the wave's LDS; per-channel gates: each lane keeps the suffix sums of
//    its own channels while the positions are visited from the newest back.
#include "device_common.hpp"

namespace kvbuf {
namespace {

constexpr int kDirectWaves = 4;  // tiles (waves) per workgroup
constexpr int kDirectBatch = 8;  // buffered positions per load batch

// Sums x[0..7] over the 64 lanes of the wave; every lane returns the total of
// x[(lane >> 3) & 7].  Each exchange halves the values a lane keeps (it adds
// its partner's partials of the values it keeps and sends those it drops),
// then the 8 lanes that share bits 5..3 sum what they hold.
__device__ __forceinline__ float reduce8(const float (&x)[8], int lane) {
    const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
    float y[4], z[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = (h5 ? x[k + 4] : x[k]) + __shfl_xor(h5 ? x[k] : x[k + 4], 32, 64);
#pragma unroll
    for (int k = 0; k < 2; ++k) z[k] = (h4 ? y[k + 2] : y[k]) + __shfl_xor(h4 ? y[k] : y[k + 2], 16, 64);
    // lane i and lane 15 - i of a row of 16 differ in bit 3
    float s = (h3 ? z[1] : z[0]) + dpp_f<0x140>(h3 ? z[0] : z[1]);
    s += dpp_f<0xB1>(s);   // quad_perm [1,0,3,2]
    s += dpp_f<0x4E>(s);   // quad_perm [2,3,0,1]
    s += dpp_f<0x141>(s);  // row_half_mirror: the 8 lanes of a half-row
    return s;
}

// Sum over the 64 lanes, in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    x += __shfl_xor(x, 32, 64);
    x += __shfl_xor(x, 16, 64);
    x += dpp_f<0x140>(x);  // row_mirror
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    return x;
}

// Scalar log-gates: wl[i] = e^{b_p - b_i} for the buffer positions i < p of
// a tile, b the cumulative log-gate from position 0 and position p the new
// token (log-gate gnew).  The gates are requested together (one per lane per
// 64 positions), summed by a wave scan, and the weights left in the wave's
// LDS.  blk: table entry `lane` of the tile (block ids checked); all 64 lanes.
__device__ __forceinline__ void scalar_weights(const TileParams& P, int h, int p, int blk, float gnew, float* wl,
                                               int lane) {
    constexpr int KS = kMaxCapacity / 64;
    const int bs = P.block_size, bpr = P.blocks_per_req, H = P.H;
    float gs[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int i = lane + 64 * k;
        gs[k] = 0.f;
        if (64 * k < p + 1) {
            // every lane takes part in the permute (it reads zero from an inactive lane)
            const int q = min(i / bs, bpr - 1);
            const uint32_t bi = static_cast<uint32_t>(__shfl(blk, q, 64));
            const size_t row = (static_cast<size_t>(bi) * H + h) * bs + (i - q * bs);
            if (i < p) gs[k] = P.gate[row];
            else if (i == p) gs[k] = gnew;
        }
    }
    float carry = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        if (64 * k < p + 1) {
            float x = gs[k];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            x += carry;
            gs[k] = x;  // b_i, i = lane + 64 k
            carry = __shfl(x, 63, 64);
        }
    }
    // b_p: position p lives in lane p % 64 of segment p / 64
    float bt = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
        if (k == p / 64) bt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs[k]), p % 64));
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int i = lane + 64 * k;
        if (i < p) wl[i] = exp_gate(bt - gs[k]);
    }
    __builtin_amdgcn_wave_barrier();
}

template <int RULE, int D, typename IO>
__global__ __launch_bounds__(64 * kDirectWaves) void direct_kernel(TileParams P) {
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool CH = RULE == KVBUF_RULE_CHANNEL;
    constexpr bool SGATE = RULE == KVBUF_RULE_GATED || DELTA;  // one log-gate per token
    constexpr int C = D >= 64 ? D / 64 : 1;                    // channels / columns per lane
    constexpr int NB = kDirectBatch;
    using XIO = typename std::conditional<DELTA, float, IO>::type;

    extern __shared__ float lds[];  // per wave: cap weights e^{b_t - b_i} (scalar gates)
    const int lane = threadIdx.x & 63;
    // the wave index is the same in every lane: said so, everything derived
    // from it (tile, rows, buffer resources) stays in scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = blockIdx.x * kDirectWaves + wv;
    if (tile >= P.batch * P.H) return;  // whole waves
    const int h = tile / P.batch;
    const int b = tile - h * P.batch;
    const int bs = P.block_size, bpr = P.blocks_per_req, cap = bs * bpr;
    float* wl = lds + wv * cap;
    const bool live = lane * C < D;  // lanes owning channels (all at d >= 64)
    const int c0 = lane * C;

    // ---- metadata and this call's token: one round trip ----------------------
    const int p_raw = load_occupancy(P, b, h);
    const int blk = load_table_row(P, b, h, lane);
    const size_t in_row = static_cast<size_t>(b) * P.H + h;
    RawChunk<IO, C> qv, kt, vt;
    qv.zero();
    kt.zero();
    vt.zero();
    float gch[C];
#pragma unroll
    for (int c = 0; c < C; ++c) gch[c] = 0.f;
    if (live) {
        qv.load(static_cast<const IO*>(P.q) + in_row * D + c0);
        kt.load(static_cast<const IO*>(P.k) + in_row * D + c0);
        vt.load(static_cast<const IO*>(P.v) + in_row * D + c0);
        if constexpr (CH) {
#pragma unroll
            for (int c = 0; c < C; ++c) gch[c] = P.g[in_row * D + c0 + c];
        }
    }
    float gnew = 0.f, beta = 0.f;
    if constexpr (SGATE) gnew = P.g[in_row];
    if constexpr (DELTA) beta = P.beta[in_row];

    const int p = __builtin_amdgcn_readfirstlane(p_raw);
    unsigned bad = (p < 0 || p >= cap) ? KVBUF_DEVERR_OVERFLOW : 0u;
    if (!bad) {
        const int nblk = p / bs + 1;  // blocks holding positions 0 .. p
        if (__ballot(lane < nblk && (blk < 0 || blk >= P.num_blocks))) bad |= KVBUF_DEVERR_BLOCK;
    }
    if (bad) {
        if (lane == 0 && P.err) atomicOr(reinterpret_cast<unsigned*>(P.err), bad);
        return;  // the tile is skipped and its metadata left unchanged
    }
    const int H = P.H;
    // pool row of buffer position i (i the same in every lane)
    auto row_of = [&](int i) -> size_t {
        const int q = i / bs;
        const uint32_t bi = static_cast<uint32_t>(__builtin_amdgcn_readlane(blk, q));
        return (static_cast<size_t>(bi) * H + h) * bs + (i - q * bs);
    };
    const IO* kpool = static_cast<const IO*>(P.key);
    const XIO* xpool = static_cast<const XIO*>(P.value);

    // ---- batches of buffered rows, the next one in flight while one is used -----
    RawChunk<IO, C> ka[NB], kb2[NB];
    RawChunk<XIO, C> xa[NB], xb2[NB];
    RawChunk<float, C> ga[CH ? NB : 1], gb2[CH ? NB : 1];
    const int nbat = (p + NB - 1) / NB;
    // the per-channel rule visits the batches from the newest back
    auto batch_base = [&](int r) { return CH ? (nbat - 1 - r) * NB : r * NB; };
    // Loads only for positions that exist: a range-checked buffer load that
    // reads nothing still costs a round trip (measured: launches with short
    // buffers took 3-4 us longer when every batch issued all its loads).
    auto issue = [&](int r, RawChunk<IO, C>(&kk)[NB], RawChunk<XIO, C>(&xx)[NB],
                     RawChunk<float, C>(&gg)[CH ? NB : 1]) {
        const int i0 = batch_base(r);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            kk[j].zero();
            xx[j].zero();
            if constexpr (CH) gg[j].zero();
            const int i = i0 + j;
            if (r < nbat && i < p) {  // the same in every lane
                const size_t row = row_of(i);
                if (live) {
                    kk[j].load(kpool + row * D + c0);
                    xx[j].load(xpool + row * D + c0);
                    if constexpr (CH) gg[j].load(P.gate + row * D + c0);
                }
            }
        }
    };
    issue(0, ka, xa, ga);

    // ---- scalar gates: weights e^{b_t - b_i} of every position ---------------------
    if constexpr (SGATE) scalar_weights(P, h, p, blk, gnew, wl, lane);

    // ---- the buffered positions -------------------------------------------------
    float acc[C], acck[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = acck[c] = 0.f;
    float suf[C];  // per-channel rule: B_t - B_i of the position being visited
#pragma unroll
    for (int c = 0; c < C; ++c) suf[c] = gch[c];  // i = t - 1: the gates after it = g_t
    float qf[C], ktf[C];
    qv.to_float(qf);
    kt.to_float(ktf);
#pragma unroll
    for (int c = 0; c < C; ++c) qf[c] *= P.scale;

    auto consume = [&](int r, const RawChunk<IO, C>(&kk)[NB], const RawChunk<XIO, C>(&xx)[NB],
                       const RawChunk<float, C>(&gg)[CH ? NB : 1]) {
        const int i0 = batch_base(r);
        float dq[NB], dk[NB];
        if constexpr (CH) {
            // positions from the newest back: decay e^{B_t - B_i} per channel
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) {
                const int j = NB - 1 - jj;
                float kf[C], gf[C];
                kk[j].to_float(kf);
                gg[j].to_float(gf);
                float s = 0.f;
                const bool in = i0 + j < p;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    s += qf[c] * kf[c] * exp_gate(suf[c]);
                    if (in) suf[c] += gf[c];
                }
                dq[j] = s;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float kf[C];
                kk[j].to_float(kf);
                float s = 0.f, sk = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    s += qf[c] * kf[c];
                    if constexpr (DELTA) sk += ktf[c] * kf[c];
                }
                dq[j] = s;
                dk[j] = sk;
            }
        }
        const float sq = reduce8(dq, lane);
        float skr = 0.f;
        if constexpr (DELTA) skr = reduce8(dk, lane);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (i0 + j < p) {
                const float w = SGATE ? wl[i0 + j] : 1.0f;
                const float cq = w * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq), 8 * j));
                float xf[C];
                xx[j].to_float(xf);
#pragma unroll
                for (int c = 0; c < C; ++c) acc[c] += cq * xf[c];
                if constexpr (DELTA) {
                    const float ck = w * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(skr), 8 * j));
#pragma unroll
                    for (int c = 0; c < C; ++c) acck[c] += ck * xf[c];
                }
            }
        }
    };
    for (int r = 0; r < nbat; r += 2) {
        issue(r + 1, kb2, xb2, gb2);
        consume(r, ka, xa, ga);
        if (r + 1 < nbat) {
            issue(r + 2, ka, xa, ga);
            consume(r + 1, kb2, xb2, gb2);
        }
    }

    // ---- the new token: its own term, the pseudo-value, the output -----------------
    const float qk = wave_sum([&] {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) s += qf[c] * ktf[c];
        return s;
    }());
    float vf[C], x[C];
    vt.to_float(vf);
#pragma unroll
    for (int c = 0; c < C; ++c) x[c] = DELTA ? beta * (vf[c] - acck[c]) : vf[c];
    const size_t out_row = in_row * D + c0;
    const size_t arow = row_of(p);
    if (live) {
#pragma unroll
        for (int c = 0; c < C; ++c) store_out(P, out_row + c, acc[c] + qk * x[c]);
        // appends: key, value (delta rule: its pseudo-value), gate
        kt.store(static_cast<IO*>(P.key) + arow * D + c0);
        if constexpr (DELTA) {
#pragma unroll
            for (int c = 0; c < C; ++c) static_cast<float*>(P.value)[arow * D + c0 + c] = x[c];
        } else {
            vt.store(static_cast<IO*>(P.value) + arow * D + c0);
        }
        if constexpr (CH) {
#pragma unroll
            for (int c = 0; c < C; ++c) P.gate[arow * D + c0 + c] = gch[c];
        }
    }
    if constexpr (SGATE) {
        if (lane == 0) P.gate[arow] = gnew;
    }
    if (lane == 0) store_occupancy(P, b, h, p + 1);
}

// The linear, gated and delta rules: 16 lanes per buffered row.  Lane l
// serves row slot l / 16 and holds elements E (l % 16) .. + E - 1 of its row
// (E = d / 16), so one 16-byte load per lane brings four rows of 128 bf16
// keys, the dot products of a row are summed within its 16 lanes by DPP (no
// broadcast), and each lane accumulates its E value columns for the rows of
// its slot; the four slots are summed once, at the end.  A batch of NB
// positions is NB / 4 such loads per plane (the delta rule's fp32
// pseudo-value rows take twice the registers of a bf16 row: smaller batches
// there keep more waves resident).
template <int RULE, int D, typename IO, int NB>
__global__ __launch_bounds__(64 * kDirectWaves) void direct_rows_kernel(TileParams P) {
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool SGATE = RULE != KVBUF_RULE_LINEAR;
    static_assert(RULE != KVBUF_RULE_CHANNEL, "per-channel gates: direct_kernel");
    constexpr int E = D / 16;
    constexpr int NS = NB / 4;  // loads per plane per batch
    using XIO = typename std::conditional<DELTA, float, IO>::type;

    extern __shared__ float lds[];  // per wave: cap weights e^{b_t - b_i}
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = blockIdx.x * kDirectWaves + wv;
    if (tile >= P.batch * P.H) return;  // whole waves
    const int h = tile / P.batch;
    const int b = tile - h * P.batch;
    const int bs = P.block_size, bpr = P.blocks_per_req, cap = bs * bpr;
    float* wl = lds + wv * cap;
    const int rs = lane >> 4;  // row slot
    const int cl = lane & 15;  // 1/16 of a row

    // ---- metadata and this call's token (every slot holds the same chunks) ------
    const int p_raw = load_occupancy(P, b, h);
    const int blk = load_table_row(P, b, h, lane);
    const size_t in_row = static_cast<size_t>(b) * P.H + h;
    RawChunk<IO, E> qc, kt, vt;
    qc.load(static_cast<const IO*>(P.q) + in_row * D + cl * E);
    kt.load(static_cast<const IO*>(P.k) + in_row * D + cl * E);
    vt.load(static_cast<const IO*>(P.v) + in_row * D + cl * E);
    float gnew = 0.f, beta = 0.f;
    if constexpr (SGATE) gnew = P.g[in_row];
    if constexpr (DELTA) beta = P.beta[in_row];

    const int p = __builtin_amdgcn_readfirstlane(p_raw);
    unsigned bad = (p < 0 || p >= cap) ? KVBUF_DEVERR_OVERFLOW : 0u;
    if (!bad) {
        const int nblk = p / bs + 1;  // blocks holding positions 0 .. p
        if (__ballot(lane < nblk && (blk < 0 || blk >= P.num_blocks))) bad |= KVBUF_DEVERR_BLOCK;
    }
    if (bad) {
        if (lane == 0 && P.err) atomicOr(reinterpret_cast<unsigned*>(P.err), bad);
        return;  // the tile is skipped and its metadata left unchanged
    }
    const int H = P.H;
    const IO* kpool = static_cast<const IO*>(P.key);
    const XIO* xpool = static_cast<const XIO*>(P.value);

    // ---- batches of buffered rows, the next one in flight while one is used -----
    RawChunk<IO, E> ka[NS], kb2[NS];
    RawChunk<XIO, E> xa[NS], xb2[NS];
    const int nbat = (p + NB - 1) / NB;
    // loads only for positions that exist (a range-checked load that reads
    // nothing still costs a round trip)
    auto issue = [&](int r, RawChunk<IO, E>(&kk)[NS], RawChunk<XIO, E>(&xx)[NS]) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            kk[u].zero();
            xx[u].zero();
            const int i = r * NB + 4 * u + rs;  // this lane's position
            // every lane takes part in the permute; clamped into the row
            const int q = min(i / bs, bpr - 1);
            const uint32_t bi = static_cast<uint32_t>(__shfl(blk, q, 64));
            const size_t row = (static_cast<size_t>(bi) * H + h) * bs + (i - q * bs);
            if (r < nbat && i < p) {
                kk[u].load(kpool + row * D + cl * E);
                xx[u].load(xpool + row * D + cl * E);
            }
        }
    };
    issue(0, ka, xa);
    if constexpr (SGATE) scalar_weights(P, h, p, blk, gnew, wl, lane);

    float acc[E], acck[DELTA ? E : 1];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int e = 0; e < (DELTA ? E : 1); ++e) acck[e] = 0.f;
    auto consume = [&](int r, const RawChunk<IO, E>(&kk)[NS], const RawChunk<XIO, E>(&xx)[NS]) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int i = r * NB + 4 * u + rs;
            const bool in = i < p;
            const float w = in ? (SGATE ? wl[i] : 1.0f) : 0.0f;
            const float cq = w * P.scale * group16_sum(chunk_dot(qc, kk[u]));
            float ck = 0.f;
            if constexpr (DELTA) ck = w * group16_sum(chunk_dot(kt, kk[u]));
            float xf[E];
            xx[u].to_float(xf);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                acc[e] += cq * xf[e];
                if constexpr (DELTA) acck[e] += ck * xf[e];
            }
        }
    };
    for (int r = 0; r < nbat; r += 2) {
        issue(r + 1, kb2, xb2);
        consume(r, ka, xa);
        if (r + 1 < nbat) {
            issue(r + 2, ka, xa);
            consume(r + 1, kb2, xb2);
        }
    }
    // the four row slots
#pragma unroll
    for (int e = 0; e < E; ++e) {
        acc[e] += __shfl_xor(acc[e], 16, 64);
        acc[e] += __shfl_xor(acc[e], 32, 64);
        if constexpr (DELTA) {
            acck[e] += __shfl_xor(acck[e], 16, 64);
            acck[e] += __shfl_xor(acck[e], 32, 64);
        }
    }

    // ---- the new token: its own term, the pseudo-value, the output -----------------
    const float qk = P.scale * group16_sum(chunk_dot(qc, kt));
    float vf[E], x[E];
    vt.to_float(vf);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = DELTA ? beta * (vf[e] - acck[e]) : vf[e];
    const int qa = p / bs;
    const uint32_t ba = static_cast<uint32_t>(__builtin_amdgcn_readlane(blk, qa));
    const size_t arow = (static_cast<size_t>(ba) * H + h) * bs + (p - qa * bs);
    if (rs == 0) {
        const size_t o = in_row * D + cl * E;
#pragma unroll
        for (int e = 0; e < E; ++e) store_out(P, o + e, acc[e] + qk * x[e]);
        // appends: key, value (delta rule: its pseudo-value), gate
        kt.store(static_cast<IO*>(P.key) + arow * D + cl * E);
        if constexpr (DELTA) {
#pragma unroll
            for (int e = 0; e < E; ++e) static_cast<float*>(P.value)[arow * D + cl * E + e] = x[e];
        } else {
            vt.store(static_cast<IO*>(P.value) + arow * D + cl * E);
        }
    }
    if constexpr (SGATE) {
        if (lane == 0) P.gate[arow] = gnew;
    }
    if (lane == 0) store_occupancy(P, b, h, p + 1);
}

template <int RULE, int D, typename IO>
hipError_t launch_direct_t(const TileParams& p, int batch, hipStream_t s) {
    const int tiles = batch * p.H;
    const unsigned grid = static_cast<unsigned>((tiles + kDirectWaves - 1) / kDirectWaves);
    const bool sgate = RULE == KVBUF_RULE_GATED || RULE == KVBUF_RULE_DELTA;
    const size_t lds = sgate ? sizeof(float) * kDirectWaves * p.block_size * p.blocks_per_req : 0;
    if constexpr (RULE == KVBUF_RULE_CHANNEL)
        direct_kernel<RULE, D, IO><<<dim3(grid), dim3(64 * kDirectWaves), lds, s>>>(p);
    else
        direct_rows_kernel<RULE, D, IO, RULE == KVBUF_RULE_DELTA ? 4 : kDirectBatch>
            <<<dim3(grid), dim3(64 * kDirectWaves), lds, s>>>(p);
    return hipGetLastError();
}

template <int RULE, typename IO>
hipError_t launch_direct_d(const TileParams& p, int d, int batch, hipStream_t s) {
    switch (d) {
        case 16: return launch_direct_t<RULE, 16, IO>(p, batch, s);
        case 64: return launch_direct_t<RULE, 64, IO>(p, batch, s);
        default: return launch_direct_t<RULE, 128, IO>(p, batch, s);
    }
}

template <typename IO>
hipError_t launch_direct_r(const TileParams& p, int rule, int d, int batch, hipStream_t s) {
    switch (rule) {
        case KVBUF_RULE_LINEAR: return launch_direct_d<KVBUF_RULE_LINEAR, IO>(p, d, batch, s);
        case KVBUF_RULE_GATED: return launch_direct_d<KVBUF_RULE_GATED, IO>(p, d, batch, s);
        case KVBUF_RULE_CHANNEL: return launch_direct_d<KVBUF_RULE_CHANNEL, IO>(p, d, batch, s);
        default: return launch_direct_d<KVBUF_RULE_DELTA, IO>(p, d, batch, s);
    }
}

}  // namespace

hipError_t launch_direct(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s) {
    return io == KVBUF_BF16 ? launch_direct_r<bf16_bits>(p, rule, d, batch, s)
                            : launch_direct_r<float>(p, rule, d, batch, s);
}

}  // namespace kvbuf
