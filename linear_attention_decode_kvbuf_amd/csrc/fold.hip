// Deferred batched state update ("flush"), commit of accepted drafts, and
// materialisation of the effective state.
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page):
//  * Figure 1 caption -- a full buffer is folded into the state on the
//    device, and the new state replaces the old one in its slot;
//  * abstract -- the state changes once per buffer, in one batched update,
//    not once per token;
//  * Figure 2 caption -- of the verified drafts, the request keeps the
//    accepted ones.
//
// Folding positions 0 .. T-1 (cumulative log-gates b_i since the last fold)
// into the state S0 at the last fold:
//   S <- e^{b_{T-1}} S0 + sum_{i<T} e^{b_{T-1} - b_i} k_i x_i^T
// a rank-T update of the d_k x d_v tile (x_i = v_i, or the delta rule's
// pseudo-value u_i).  With one log-gate per key channel the decays are
// vectors and act on rows: row r of S0 is scaled by e^{B_{T-1}[r]} and k_i[r]
// by e^{B_{T-1}[r] - B_i[r]} (B the per-channel cumulative log-gate).
//
// One workgroup per (request, head): the state waves put the 64 KiB tile in
// flight while the token wave forms the decay weights and stages the keys and
// values in LDS (rounds of up to 32 tokens); the state waves apply the update
// from registers and write the tile back.  The update costs 2 T flops per 8
// bytes of state traffic: short folds (T <= 16) run on the vector ALUs, longer
// ones on the matrix cores, whose fp32 operands enter as exact bf16 terms --
// every workgroup of a launch runs the same phases in step, so the arithmetic
// of a round adds to the time unless it is short.
#include "device_common.hpp"

namespace kvbuf {
namespace {

// LDS: pool row of each buffer position, cumulative log-gates, the weight
// of every position (raw staging), nb staging buffers of fc tokens (keys,
// values and -- fp32 staging -- weights), the state weight e^{b_{T-1}} (per
// key channel for the per-channel rule: DK of them).  Keys and values are
// staged as fp32 (kb = xb = 4) or, for the matrix-core folds, raw: as stored
// in the pool (kb, xb = element bytes), by direct-to-LDS copies.  The
// matrix-core folds reuse the staging area, once the last round is applied,
// to turn the update into whole rows (64 rows of 128 floats at a time), so
// it spans at least kFoldConvFloats.
constexpr int kFoldConvFloats = 64 * 128;
__host__ __device__ inline int fold_stage_floats(int DK, int DV, int fc, int kb, int xb, bool raw) {
    return (fc * (DK * kb + DV * xb)) / 4 + (raw ? 0 : ((fc + 3) & ~3));
}
__host__ __device__ inline int fold_stage_area(int stage_floats, int nb, bool mf) {
    const int a = nb * stage_floats;
    return (mf && a < kFoldConvFloats) ? kFoldConvFloats : a;
}
__host__ __device__ inline int fold_lds_floats(int DK, int DV, int cap, int stage_area, bool ch) {
    return 2 * ((cap + 3) & ~3) + ((cap + 31) & ~31) + stage_area + (ch ? DK : 4);
}
// raw multi-round folds of bf16 rows keep this many staging buffers: the
// copies of round r + 2 are in flight while round r is applied
constexpr int kFoldRing = 3;

// A barrier for LDS only: after the metadata, and between ring rounds.  At a
// __syncthreads() the compiler may make a wave drain its vector-memory
// counter first (it did after the metadata), which would wait for stores and
// for the direct-to-LDS copies of later rounds; here each wave only completes
// its LDS accesses (lgkmcnt(0)) before the barrier, and between rounds the
// token wave has already waited for the round that is read next.  The signal
// fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Copies rows src[k] -> dst[k], k < a (U 16-byte units per row) with one
// wave: all loads first (at most four per lane, held in named registers),
// then the stores in the same order.
template <int U>
__device__ __forceinline__ void move_rows(char* plane, const uint32_t* src, const uint32_t* dst, int a,
                                          int lane) {
    constexpr int N = (kMaxDrafts * U + 63) / 64;
    static_assert(N <= 4, "rows of at most 512 bytes");
    auto at = [&](const uint32_t* rows, int r) {
        const int u = lane + 64 * r;
        return reinterpret_cast<uint4*>(plane + (static_cast<size_t>(rows[u / U]) * U + u % U) * 16);
    };
    auto live = [&](int r) { return (lane + 64 * r) / U < a; };
    uint4 v0{}, v1{}, v2{}, v3{};
    if (live(0)) v0 = *at(src, 0);
    if (N > 1 && live(1)) v1 = *at(src, 1);
    if (N > 2 && live(2)) v2 = *at(src, 2);
    if (N > 3 && live(3)) v3 = *at(src, 3);
    if (live(0)) *at(dst, 0) = v0;
    if (N > 1 && live(1)) *at(dst, 1) = v1;
    if (N > 2 && live(2)) *at(dst, 2) = v2;
    if (N > 3 && live(3)) *at(dst, 3) = v3;
}

// Long folds on the matrix cores (bf16 MFMA, fp32 accumulate).  An fp32 value
// x enters as three bf16 terms, hi = bf16(x), mid = bf16(x - hi),
// lo = bf16(x - hi - mid), whose sum carries x to about 2^-27 of its size;
// products of bf16 terms are exact in fp32.
typedef short mf_s4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t mf_pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
}
__device__ __forceinline__ float mf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float mf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// four values exactly representable in bf16
__device__ __forceinline__ mf_s4 mf_exact(const float (&x)[4]) {
    return __builtin_bit_cast(mf_s4, make_uint2(mf_pack2(x[0], x[1]), mf_pack2(x[2], x[3])));
}
__device__ __forceinline__ void mf_split3(const float (&x)[4], mf_s4& h, mf_s4& m, mf_s4& l) {
    float r[4];
    const uint32_t h01 = mf_pack2(x[0], x[1]), h23 = mf_pack2(x[2], x[3]);
    r[0] = x[0] - mf_lo(h01); r[1] = x[1] - mf_hi(h01); r[2] = x[2] - mf_lo(h23); r[3] = x[3] - mf_hi(h23);
    const uint32_t m01 = mf_pack2(r[0], r[1]), m23 = mf_pack2(r[2], r[3]);
    r[0] -= mf_lo(m01); r[1] -= mf_hi(m01); r[2] -= mf_lo(m23); r[3] -= mf_hi(m23);
    h = __builtin_bit_cast(mf_s4, make_uint2(h01, h23));
    m = __builtin_bit_cast(mf_s4, make_uint2(m01, m23));
    l = __builtin_bit_cast(mf_s4, make_uint2(mf_pack2(r[0], r[1]), mf_pack2(r[2], r[3])));
}
__device__ __forceinline__ f4 mf_mac(mf_s4 a, mf_s4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// bf16 rows of 128 (256 bytes) staged for the 16 x 16 x 32 products.
// v_mfma_f32_16x16x32_bf16 takes, in lane l (group G = l / 16, t = l % 16),
// A[t][8G + i] and B[8G + i][t] for i < 8 and returns D[4G + j][t], j < 4;
// ds_read_b64_tr_b16 gives lane t of a 16-lane group element j of source lane
// 4j + t / 4, word t % 4.  So when the 16 lanes of group G point at rows
// 8G + t / 4 (+ 4), columns c0 + 4 (t % 4) of a row-major tile, lane t
// receives column c0 + t of rows 8G .. 8G + 3 (+ 4): the K-major operand
// that the product wants, from rows as they were copied.  The 16-byte chunk
// cc of row r sits at slot 16 r + (cc ^ f(r)), f(r) = 2 ((r & 3) | (((r >> 3)
// & 1) << 2)), which spreads the 16 rows that one such read touches over all
// LDS banks.
typedef short tr_s4 __attribute__((ext_vector_type(4)));
typedef __bf16 mf_b8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ int tr_swz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }
template <typename SrcOf>
__device__ __forceinline__ void lds_copy_swz(char* dst, int rows, SrcOf src, int lane) {
    for (int r0 = 0; r0 < rows; r0 += 4) {
        const int r = r0 + (lane >> 4);
        const char* a = src(r < rows ? r : r0) + 16 * ((lane & 15) ^ tr_swz(r));
        if (r < rows) lds_dma16(a, dst + r0 * 256);
    }
}
// fp32 rows of 128 (512 bytes, the delta rule's pseudo-values), read one
// word per lane: chunk cc of row r at slot 32 r + (cc ^ 4 ((r >> 3) & 3)), so
// that the four rows 8G + i (G < 4) of one read land in different banks.
template <typename SrcOf>
__device__ __forceinline__ void lds_copy_swz32(char* dst, int rows, SrcOf src, int lane) {
    for (int r0 = 0; r0 < rows; r0 += 2) {
        const int r = r0 + (lane >> 5);
        const char* a = src(r < rows ? r : r0) + 16 * ((lane & 31) ^ (4 * ((r >> 3) & 3)));
        if (r < rows) lds_dma16(a, dst + r0 * 512);
    }
}
// LDS byte address of a pointer into the workgroup's LDS, and reads at one
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}
__device__ __forceinline__ tr_s4 tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr_s4*)(p));
}
__device__ __forceinline__ tr_s4 tr_read(uint32_t a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr_s4*)(uintptr_t)(a));
}
__device__ __forceinline__ float lds_f32(uint32_t a) {
    return *(__attribute__((address_space(3))) const float*)(uintptr_t)(a);
}
__device__ __forceinline__ mf_b8 tr_join(tr_s4 a, tr_s4 b) {
    typedef short s8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(mf_b8, s8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
}
__device__ __forceinline__ f4 mf_mac32(mf_b8 a, mf_b8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// MULTI: the fold may take more than one staging round (then the token wave
// stages round r+1 while the state waves apply round r).  Without it every
// position is staged before the state loads are issued, which keeps the
// token wave's registers out of the tile's live range.
// TREE: a commit of a root-to-leaf path of tree drafts.
// W4: four waves, wave 0 taking the token wave's part as well (rows staged as
// stored, not a tree commit).  A workgroup of five waves is placed on a CU
// only while every SIMD has room for two of its waves, which left the fold at
// two workgroups per CU where its registers allow three (measured); with four
// waves the registers and LDS decide.
template <int RULE, int DK, int DV, typename IO, bool MULTI, bool TREE, bool MFT, bool W4 = false>
__device__ __forceinline__ void fold_tile(const TileParams& P, int b, int h, int tid) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RPT = G::RPT;
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool CH = RULE == KVBUF_RULE_CHANNEL;
    constexpr bool SGATE = RULE == KVBUF_RULE_GATED || DELTA;  // one scalar gate per token
    constexpr int CPL = (DK + 63) / 64;                        // key channels per token-wave lane
    using XIO = typename std::conditional<DELTA, float, IO>::type;
    // Folds that may exceed 16 positions (MFT, d = 128): the rank-T update
    // runs on the matrix cores (shorter ones are cheaper on the vector ALUs).
    // The tile is then held in the MFMA accumulator layout -- 16 x 16 blocks
    // of S^T, wave w owning rows 32w .. 32w+31: lane l holds row
    // 32w + 16 rb + l % 16, columns 16 cb + 4 (l / 16) .. +3 of block (rb, cb)
    // in s[8 rb + cb] -- and block (rb, cb) of S^T gains sum_k x_k[c] (w_k
    // k_k[r]) as A (x rows, M = columns) times B (weighted keys, N = rows) over
    // K-chunks of 16 positions (one round) or 32 (several rounds, TR below).
    constexpr bool MF = MFT && DK == 128 && DV == 128;
    constexpr bool XEXACT = std::is_same<XIO, bf16_bits>::value;  // values exact in bf16
    // ... and their rows are staged as loaded, by direct-to-LDS copies (one
    // round trip per staging round; the per-channel rule keeps fp32 rows,
    // whose keys carry per-channel decays)
    constexpr bool RAW = MF && !CH;
    // Multi-round folds of bf16 rows keep three staging buffers, the copies of
    // round r + 2 in flight while round r is applied (three buffers of fp32
    // rows would cost a workgroup per CU); four-wave workgroups keep two, the
    // copies of round r + 1 in flight (measured: a fourth workgroup per CU
    // outweighs the deeper ring, 289 against 300 us at m = 128).
    constexpr bool RING = RAW && MULTI && sizeof(XIO) == 2;
    // multi-round folds of bf16 keys: 16 x 16 x 32 products on transposing
    // LDS reads (their wider operands cost a wave per SIMD, which a single
    // round does not win back).  bf16 values enter as they are and the
    // weighted keys as three terms; the delta rule's fp32 pseudo-values carry
    // the weight and enter as three terms against the keys as they are.
    constexpr bool TR = RAW && MULTI && sizeof(IO) == 2;
    // ... and then each state wave holds 32 columns of the tile (all rows),
    // so that it splits only its own columns of the pseudo-values
    constexpr bool COLS = TR && !XEXACT;
    constexpr int NBUF = (RING && !W4) ? kFoldRing : 2;
    static_assert(!W4 || (!CH && (MF || !MULTI)), "four waves: not the per-channel rule");

    extern __shared__ __attribute__((aligned(16))) float lds[];  // 16-byte rows for the LDS copies
    __shared__ unsigned s_bad;
    __shared__ int s_T, s_fold;
    // the metadata update, stored by the token wave at the end of the tile:
    // whether there is one, the new occupancy, the table entries rotated, and
    // the table row as read
    __shared__ int s_upd, s_pnew, s_rot;
    __shared__ int s_blk[kMaxTableRow];
    // tree commit: pool rows of the k-th kept draft before (src) and after
    // (dst) its move to buffer position p + k
    __shared__ uint32_t s_src[TREE ? kMaxDrafts : 1], s_dst[TREE ? kMaxDrafts : 1];

    // the wave with the token part (metadata, copies, gates, weights) and the
    // waves holding the tile
    const bool token_wave = W4 ? tid < 64 : tid >= NT;
    const bool state_wave = W4 || tid < NT;
    const int lane = W4 ? tid : tid - NT;
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * 4;
    const int cap = P.block_size * P.blocks_per_req;
    const bool materialize = P.mode == MODE_MATERIALIZE;

    // The token wave reads the tile's metadata, checks it, and -- being its
    // only reader -- advances it in place (flush, commit) before the barrier.
    const int slot = P.slot[b];
    const bool has_state = slot >= 0;
    constexpr bool tree = TREE;
    int a = 0;        // drafts kept
    int a_moves = 0;  // tree commit: kept drafts whose rows move
    if (token_wave) {
        // occupancy, table row, accepted count / parents and leaf: all
        // requested before any is used (one round trip)
        const int p = load_occupancy(P, b, h);
        const int blk = load_table_row(P, b, h, lane);
        unsigned bad = 0;
        uint32_t path = 0;  // tree commit: bit d set = draft d is kept
        if (!tree && P.mode == MODE_COMMIT) {
            a = P.accepted[b];
            if (a < 0 || a > P.n) bad |= KVBUF_DEVERR_ACCEPT;
        } else if (tree) {
            // the path from the root to the leaf, walked up through the parents
            const int n = P.n;
            const int leaf = P.leaf[b];
            const int par = lane < n ? P.parent[static_cast<size_t>(b) * n + lane] : -1;
            if (__ballot(lane < n && (par < -1 || par >= lane)) || leaf < -1 || leaf >= n)
                bad |= KVBUF_DEVERR_ACCEPT;
            int cur = bad ? -1 : leaf;
            for (int step = 0; step < n; ++step) {
                if (cur >= 0) path |= 1u << cur;
                const int up = __shfl(par, cur >= 0 ? cur : 0, 64);
                cur = (cur > 0 && up < cur) ? up : -1;
            }
            a = __popc(path);
            if (p + n > cap) bad |= KVBUF_DEVERR_OVERFLOW;  // the drafts sit at p .. p + n - 1
        }
        const int pn = (p < 0 || p > cap) ? -1 : p + a;  // occupancy after the kept drafts
        if (pn < 0 || pn > cap) bad |= KVBUF_DEVERR_OVERFLOW;
        if (slot >= P.num_slots) bad |= KVBUF_DEVERR_SLOT;
        const bool fold0 = !materialize && has_state && P.m > 0 && pn >= P.m &&
                           (P.mode == MODE_FLUSH || P.fuse);
        const int T0 = materialize ? p : (fold0 ? P.m : 0);  // positions applied
        uint32_t* pos = reinterpret_cast<uint32_t*>(lds);
        bad |= stage_row_from(P, h, (tree && pn >= 0) ? max(T0, p + P.n) : T0, pos, lane, blk);
        if (tree && !bad) {
            // kept draft d (rank k on the path) moves from position p + d to
            // p + k: the fold below reads it from its draft row, and its rows
            // are copied once the fold's reads are done (drafts already in
            // place, d = k, are not copied)
            const bool kept = lane < P.n && ((path >> lane) & 1u);
            const int k = kept ? __popc(path & ((1u << lane) - 1u)) : 0;
            const bool moves = kept && k != lane;
            const uint64_t mv = __ballot(moves);
            const int slot_k = moves ? __popc(static_cast<uint32_t>(mv) & ((1u << lane) - 1u)) : 0;
            uint32_t src = 0, dst = 0;
            if (kept) {
                src = pos[p + lane];
                dst = pos[p + k];
            }
            __builtin_amdgcn_wave_barrier();
            if (kept) pos[p + k] = src;
            if (moves) {
                s_src[slot_k] = src;
                s_dst[slot_k] = dst;
            }
            a_moves = __popcll(mv);
        }
        if (lane == 0) {
            s_bad = bad;
            s_T = T0;
            s_fold = fold0 ? 1 : 0;
            s_upd = !bad && !materialize && (fold0 || a != 0);
            s_pnew = fold0 ? pn - P.m : pn;
            s_rot = fold0 ? P.m / P.block_size : 0;
        }
        s_blk[lane] = blk;
    }
    // The position table, s_T, s_fold and s_bad are complete.  The token
    // wave's metadata stores need not be: nothing in this workgroup reads
    // them back, so the barrier waits for LDS accesses only.
    ring_barrier();
    if (s_bad) {
        report(P, s_bad);
        return;
    }
    const bool fold = s_fold != 0;
    const int T = s_T;
    // Token wave: the metadata stores are issued last, so that no wait on
    // them stands between the metadata and the first copies, or before a
    // barrier the state waves take.
    auto meta = [&]() __attribute__((always_inline)) {
        if (s_upd) update_meta(P, b, h, s_pnew, s_rot, lane, s_blk[lane]);
    };

    // Token wave, tree commit: copy the kept drafts' key, value and gate rows
    // to their new positions.  Every load is issued before the first store and
    // a row's destination is never the source of a later row (kept draft k
    // comes from position p + d with d >= k), so no row is overwritten before
    // it is read.
    auto move_kept = [&]() __attribute__((always_inline)) {
        const int nm = a_moves;
        if (nm == 0) return;
        move_rows<DK * sizeof(IO) / 16>(static_cast<char*>(P.key), s_src, s_dst, nm, lane);
        move_rows<DV * sizeof(XIO) / 16>(static_cast<char*>(P.value), s_src, s_dst, nm, lane);
        if constexpr (CH) {
            move_rows<DK * 4 / 16>(reinterpret_cast<char*>(P.gate), s_src, s_dst, nm, lane);
        } else if constexpr (SGATE) {
            const float gk = lane < nm ? P.gate[s_src[lane]] : 0.0f;
            if (lane < nm) P.gate[s_dst[lane]] = gk;
        }
    };
    if (!materialize && !fold) {  // no state change for this tile
        if (token_wave) {
            if (tree) move_kept();
            meta();
        }
        return;
    }

    // multi-round raw folds always take the full raw chunk (the launcher)
    const int fc = RING ? kRawFoldChunk : P.fold_chunk;
    const int cap4 = (cap + 3) & ~3;
    float* bl = lds + cap4;
    float* fwa = bl + cap4;  // raw staging: the weight of every position (0 up to a multiple of 32)
    float* stage0 = fwa + ((cap + 31) & ~31);
    constexpr int KB = RAW ? static_cast<int>(sizeof(IO)) : 4, XB = RAW ? static_cast<int>(sizeof(XIO)) : 4;
    const int srows = TR ? 32 : fc;  // rows of a staging buffer (TR: a whole product chunk)
    const int stage_floats = fold_stage_floats(DK, DV, srows, KB, XB, RAW);
    float* e0p = stage0 + fold_stage_area(stage_floats, NBUF, MF);

    TileTokens<DK, DV, IO, XIO> tok;
    tok.kpool = static_cast<const IO*>(P.key);
    tok.xpool = static_cast<const XIO*>(P.value);
    tok.gpool = P.gate;
    tok.pos = reinterpret_cast<const uint32_t*>(lds);
    tok.H = P.H;
    tok.p = cap;  // every position read here is in the pool

    // Per-channel rule: the token wave holds, for its key channels
    // ch = lane + 64 c, the running sum of the gates of the positions staged
    // so far (prefix) and their total over all T positions (e0p[ch]).
    float prefix[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) prefix[c] = 0.0f;

    // Token wave: stage round r (tokens r*fc ..) into buffer r % NBUF.  Raw
    // rows are only issued here: stage() waits for them, a ring fold
    // (ring_wait) counts them.
    // Four-wave folds other than tree commits: wave 1 forms the decay weights
    // while wave 0 requests the rows (and, vector-ALU folds, its share of the
    // tile).  A wave's loads retire in order, so gate loads issued behind the
    // copies or the tile waited for them; on a wave of their own they are
    // formed during that round trip (measured: m = 32 folds 204 -> 199 us
    // gated, 209 -> 206 us delta rule; m = 64 gated 210 -> 207 us).  The
    // delta rule's fp32 rows keep one round ahead: requesting its first two
    // rounds together took m = 64 from 265 to 270 us.  A one-round tree
    // commit moves its kept rows after the barrier that ends the weights'
    // reads of their gates; a multi-round one keeps the weights on wave 0.
    constexpr bool GW = W4 && !(TREE && MULTI);
    const bool gate_wave = GW ? (tid >> 6) == 1 : token_wave;
    const int glane = GW ? tid - 64 : lane;
    auto issue = [&](int r) {
        char* fk = reinterpret_cast<char*>(stage0 + (r % NBUF) * stage_floats);
        char* fx = fk + srows * DK * KB;
        const int i0 = r * fc;
        const int cnt = min(fc, T - i0);
        auto key_row = [&](int ii) { return reinterpret_cast<const char*>(tok.key(i0 + ii)); };
        auto value_row = [&](int ii) { return reinterpret_cast<const char*>(tok.pooled_value(i0 + ii)); };
        if constexpr (TR) {
            constexpr int XC = DV * XB / 16;  // 16-byte chunks of a value row
            lds_copy_swz(fk, cnt, key_row, lane);
            if constexpr (XB == 2) lds_copy_swz(fx, cnt, value_row, lane);
            else lds_copy_swz32(fx, cnt, value_row, lane);
            // rows past the end of a short round read as zeros
            for (int q = cnt * 16 + lane; q < 32 * 16; q += 64)
                reinterpret_cast<uint4*>(fk)[q] = make_uint4(0u, 0u, 0u, 0u);
            for (int q = cnt * XC + lane; q < 32 * XC; q += 64)
                reinterpret_cast<uint4*>(fx)[q] = make_uint4(0u, 0u, 0u, 0u);
        } else {
            lds_copy_rows<DK * KB>(fk, cnt, key_row, lane);
            lds_copy_rows<DV * XB>(fx, cnt, value_row, lane);
        }
    };
    // Per-channel rule: this lane's channels of the log-gates of positions
    // i0 .. i0 + n - 1 (n <= 8; zero past n), all requested before any is used.
    auto gate_chunk = [&](int i0, int n, float (&gv)[CPL][8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t row = u < n ? static_cast<size_t>(tok.pos[i0 + u]) * DK : 0;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = lane + 64 * c;
                gv[c][u] = (u < n && ch < DK) ? P.gate[row + ch] : 0.0f;
            }
        }
    };
    auto stage = [&](int r) {
        float* fk = stage0 + (r % NBUF) * stage_floats;
        float* fx = fk + srows * DK * KB / 4;
        float* fw = fx + srows * DV * XB / 4;
        const int i0 = r * fc;
        const int cnt = min(fc, T - i0);
        if constexpr (RAW) {
            issue(r);
            wait_lds_copies();
            return;
        } else {
            stage_rows(tok, i0, cnt, fk, fx, nullptr, lane);
        }
        if constexpr (CH) {
            // k_i[ch] e^{B_{T-1}[ch] - B_i[ch]}, positions in order; the gates
            // of 8 positions are requested before any is used
            for (int ii0 = 0; ii0 < cnt; ii0 += 8) {
                float gv[CPL][8];
                gate_chunk(i0 + ii0, min(8, cnt - ii0), gv);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int ii = ii0 + u;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const int ch = lane + 64 * c;
                        if (ch < DK && ii < cnt) {
                            prefix[c] += gv[c][u];
                            fk[ii * DK + ch] *= exp_gate(e0p[ch] - prefix[c]);
                        }
                    }
                }
            }
            for (int ii = lane; ii < cnt; ii += 64) fw[ii] = 1.0f;
        } else if constexpr (!GW) {  // (GW: wave 1 writes them)
            for (int ii = lane; ii < cnt; ii += 64)
                fw[ii] = SGATE ? exp_gate(bl[T - 1] - bl[i0 + ii]) : 1.0f;
        }
    };
    // Ring: wait until the copies of round r have landed while those of round
    // r + 1 (if issued) may still be in flight.  The copies retire in order;
    // a full round is a known number of copy instructions, a short (last)
    // round waits for everything.
    auto ring_wait = [&](int r) {
        constexpr int RPIK = 64 / (DK * KB / 16), RPIX = 64 / (DV * XB / 16);
        constexpr int FULL = (kRawFoldChunk + RPIK - 1) / RPIK + (kRawFoldChunk + RPIX - 1) / RPIX;
        static_assert(FULL < 64, "vmcnt holds six bits");
        if ((r + 2) * fc <= T)
            __builtin_amdgcn_s_waitcnt((FULL & 15) | ((FULL >> 4) << 14) | 0x0F70);
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_sched_barrier(0);
    };

    f4 s[RPT];
    const int mw = tid >> 6, ml = tid & 63;  // MF: wave and lane
    const float* tile = has_state ? P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV : P.state;
    // Four waves, vector-ALU fold (commits): a chain commit's wave 0 requests
    // its share of the tile before it stages the rows, both in flight
    // together.  A tree commit's wave 0 requests it with the other waves,
    // after the path walk and the staging, which keeps its registers at five
    // waves per SIMD (five workgroups per CU instead of four; measured, tree
    // commits 30.4 / 35.4 / 42.8 / 50.5 -> 28.1 / 32.8 / 39.4 / 46.9 us at
    // n = 1 / 2 / 4 / 8; chain commits gained at n <= 4 and lost 2.6% at n = 8,
    // where half the tiles fold and wait for wave 0's later share).
    constexpr bool W4_EARLY_TILE = W4 && !MF && !TREE;
    if (token_wave) {
        if constexpr (W4_EARLY_TILE) load_tile<RPT, DK, DV>(s, tile, has_state, rg, c0);
        if constexpr (RAW) {
            // The first rounds' copies need only the position table: requested
            // before the gates, both are in flight in the same round trip.
            // Nothing else is outstanding on the wave's counter here (the
            // metadata stores come last), so the ring waits' counts hold.
            if (T > 0) issue(0);
            if (RING && T > fc) issue(1);
        }
    }
    if (gate_wave) {
        if constexpr (SGATE) gate_prefix_loads(bl, T, glane, [&](int i) { return tok.gate(i); });
        if constexpr (CH) {
            // total log-gate of each key channel over the T positions, summed
            // in order
            float tot[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) tot[c] = 0.0f;
            for (int i0 = 0; i0 < T; i0 += 8) {
                float gv[CPL][8];
                gate_chunk(i0, min(8, T - i0), gv);
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) tot[c] += gv[c][u];  // zero past the end
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                if (lane + 64 * c < DK) e0p[lane + 64 * c] = tot[c];
        } else {
            if (glane == 0) *e0p = (SGATE && T > 0) ? exp_gate(bl[T - 1]) : 1.0f;
        }
        if constexpr (RAW) {
            for (int i = glane; i < ((T + 31) & ~31); i += 64)
                fwa[i] = i >= T ? 0.0f : SGATE ? exp_gate(bl[T - 1] - bl[i]) : 1.0f;
        } else if constexpr (GW) {
            // the one staging round's weights (four-wave vector-ALU folds
            // take at most 16 positions)
            static_assert(!GW || MF || !MULTI, "one round");
            float* fw0 = stage0 + srows * DK * KB / 4 + srows * DV * XB / 4;
            for (int i = glane; i < T; i += 64) fw0[i] = SGATE ? exp_gate(bl[T - 1] - bl[i]) : 1.0f;
        }
    }
    if (token_wave) {
        if constexpr (RING) {
            ring_wait(0);
        } else if constexpr (RAW) {
            if (T > 0) wait_lds_copies();  // round 0, requested above
        } else {
            if (T > 0) stage(0);
        }
        if (tree && !MULTI && !GW) move_kept();  // the fold's rows are staged
    }
    if (state_wave) {
        if constexpr (MF) {
            // the matrix cores accumulate the update alone, from zero; the
            // state is read after the last round, in whole rows
            static_assert(RPT == 16, "16 blocks of 16 x 16 per wave");
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        } else if (!(W4_EARLY_TILE && token_wave)) {
            load_tile<RPT, DK, DV>(s, tile, has_state, rg, c0);
        }
    }
    if constexpr (RING || GW) ring_barrier();  // round 0 has landed
    else __syncthreads();
    // (GW: every gate the weights read has been read)
    if (GW && tree && !MULTI && token_wave) move_kept();
    if (state_wave) {
        if constexpr (MF) {
        } else if constexpr (CH) {
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] *= exp_gate(e0p[rg * RPT + j]);
        } else {
            const float e0 = *e0p;
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] *= e0;
        }
    }
    auto apply = [&](int r) {
        const float* fk = stage0 + (r % NBUF) * stage_floats;
        const float* fx = fk + srows * DK * KB / 4;
        const float* fw = RAW ? fwa + r * fc : fx + srows * DV * XB / 4;
        const int cnt = min(fc, T - r * fc);
        if constexpr (TR) {
            // lane ml: group G, row-in-group t; its read address inside a
            // chunk of 32 rows for column block cbx (16 columns) and half h
            const int G = ml >> 4, t = ml & 15;
            const int f2 = (t >> 2) | ((G & 1) << 2);  // tr_swz of the row, halved
            const int lane_off = (8 * G + (t >> 2)) * 256 + 16 * ((t & 3) >> 1) + 8 * (t & 1);
            auto at = [&](const float* buf, int kb, int h, int cbx) {
                return reinterpret_cast<const char*>(buf) + kb * 256 + h * 1024 + lane_off + 32 * (cbx ^ f2);
            };
            // The same as an LDS address, formed so that the compiler does not
            // keep the eight column offsets in registers: staging buffers sit
            // at multiples of 512 bytes from the first, so the swizzle is an
            // XOR of the offset bits that select the 32-byte column pair.
            const uint32_t base0 = lds_addr(stage0);
            auto rel = [&](const float* buf) { return static_cast<uint32_t>((buf - stage0) * 4); };
            auto at_x = [&](const float* buf, int kb, int h, int cbx) {
                return base0 + ((rel(buf) + kb * 256 + h * 1024 + lane_off + 32 * f2) ^ static_cast<uint32_t>(32 * cbx));
            };
            for (int kb = 0; kb < cnt; kb += 32) {
                if constexpr (COLS) {
                    // A: w_p u_p[c] in three terms, for this wave's columns
                    // c = 32 mw + 16 cb + t, read one word per lane from the
                    // swizzled fp32 rows; B: k_p[n] as stored, n = 16 rb + t
                    // (read again for the second column block: holding all
                    // eight would cost a wave per SIMD)
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) {
                        const uint32_t xr = base0 + ((rel(fx) + (kb + 8 * G) * 512 + 64 * G + 4 * t) ^
                                                     static_cast<uint32_t>(64 * (2 * mw + cb)));
                        const f4 w0 = *reinterpret_cast<const f4*>(fw + kb + 8 * G);
                        const f4 w1 = *reinterpret_cast<const f4*>(fw + kb + 8 * G + 4);
                        float v0[4], v1[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            v0[i] = w0[i] * lds_f32(xr + i * 512);
                            v1[i] = w1[i] * lds_f32(xr + (i + 4) * 512);
                        }
                        mf_s4 h0, m0, o0, h1, m1, o1;
                        mf_split3(v0, h0, m0, o0);
                        mf_split3(v1, h1, m1, o1);
                        const mf_b8 ah = tr_join(h0, h1), am = tr_join(m0, m1), ao = tr_join(o0, o1);
                        auto keys = [&](int rb) {
                            return tr_join(tr_read(at_x(fk, kb, 0, rb)), tr_read(at_x(fk, kb, 1, rb)));
                        };
                        // one row block's keys at a time: the scheduling
                        // barriers keep the compiler from hoisting all eight
                        // (registers); other waves cover the read latency
#pragma unroll
                        for (int rb = 0; rb < 8; ++rb) {
                            const mf_b8 kr = keys(rb);
                            f4 d = s[2 * rb + cb];
                            d = mf_mac32(ah, kr, d);
                            d = mf_mac32(am, kr, d);
                            d = mf_mac32(ao, kr, d);
                            s[2 * rb + cb] = d;
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        asm volatile("" ::: "memory");  // the key reads are not merged across column blocks
                    }
                    continue;
                }
                // B: w_p k_p[n] for positions kb + 8G + i, rows n = 32 mw + 16 rb + t
                const f4 w0 = *reinterpret_cast<const f4*>(fw + kb + 8 * G);
                const f4 w1 = *reinterpret_cast<const f4*>(fw + kb + 8 * G + 4);
                mf_b8 bh[2], bm[2], bo[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const tr_s4 k0 = tr_read(at(fk, kb, 0, 2 * mw + rb));
                    const tr_s4 k1 = tr_read(at(fk, kb, 1, 2 * mw + rb));
                    float v0[4], v1[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v0[i] = w0[i] * __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(k0[i])) << 16);
                        v1[i] = w1[i] * __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(k1[i])) << 16);
                    }
                    mf_s4 h0, m0, o0, h1, m1, o1;
                    mf_split3(v0, h0, m0, o0);
                    mf_split3(v1, h1, m1, o1);
                    bh[rb] = tr_join(h0, h1);
                    bm[rb] = tr_join(m0, m1);
                    bo[rb] = tr_join(o0, o1);
                }
                // A: x_p[c], columns c = 16 cb + t; each block takes its
                // three products in the order hi, mid, lo
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) {
                    const mf_b8 a = tr_join(tr_read(at(fx, kb, 0, cb)), tr_read(at(fx, kb, 1, cb)));
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        f4 d = s[8 * rb + cb];
                        d = mf_mac32(a, bh[rb], d);
                        d = mf_mac32(a, bm[rb], d);
                        d = mf_mac32(a, bo[rb], d);
                        s[8 * rb + cb] = d;
                    }
                }
            }
            return;
        }
        if constexpr (MF) {
            const int g = ml >> 4, nn = ml & 15;
            for (int k0 = 0; k0 < cnt; k0 += 16) {
                // B: weighted keys w_p k_p[r], positions k0 + 4g + i, row r of block rb
                mf_s4 bh[2], bm[2], bo[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int pp = k0 + 4 * g + i;
                        const int at = pp * DK + 32 * mw + 16 * rb + nn;
                        const float kv = RAW ? load1(reinterpret_cast<const IO*>(fk) + at) : fk[at];
                        v[i] = pp < cnt ? fw[pp] * kv : 0.0f;
                    }
                    mf_split3(v, bh[rb], bm[rb], bo[rb]);
                }
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) {
                    // A: values x_p[c], column c = 16 cb + nn
                    float x[4];
                    mf_s4 xb;  // raw bf16 rows: the bits themselves
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int pp = k0 + 4 * g + i;
                        const int at = pp * DV + 16 * cb + nn;
                        if constexpr (RAW && XEXACT) {
                            xb[i] = pp < cnt ? static_cast<short>(reinterpret_cast<const bf16_bits*>(fx)[at]) : 0;
                        } else if constexpr (RAW) {
                            x[i] = pp < cnt ? load1(reinterpret_cast<const XIO*>(fx) + at) : 0.0f;
                        } else {
                            x[i] = pp < cnt ? fx[at] : 0.0f;
                        }
                    }
                    if constexpr (XEXACT) {
                        const mf_s4 a = RAW ? xb : mf_exact(x);
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb) {
                            f4 d = s[8 * rb + cb];
                            d = mf_mac(a, bh[rb], d);
                            d = mf_mac(a, bm[rb], d);
                            d = mf_mac(a, bo[rb], d);
                            s[8 * rb + cb] = d;
                        }
                    } else {
                        mf_s4 ah, am, ao;
                        mf_split3(x, ah, am, ao);
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb) {
                            f4 d = s[8 * rb + cb];
                            d = mf_mac(ah, bh[rb], d);
                            d = mf_mac(ah, bm[rb], d);
                            d = mf_mac(am, bh[rb], d);
                            d = mf_mac(ah, bo[rb], d);
                            d = mf_mac(ao, bh[rb], d);
                            d = mf_mac(am, bm[rb], d);
                            s[8 * rb + cb] = d;
                        }
                    }
                }
            }
            return;
        }
        for (int ii = 0; ii < cnt; ++ii) {
            const f4 x = *reinterpret_cast<const f4*>(fx + ii * DV + c0);
            const float w = fw[ii];
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] += (w * fk[ii * DK + rg * RPT + j]) * x;
        }
    };
    if constexpr (!MULTI) {
        if (state_wave && T > 0) apply(0);
    } else {
        const int rounds = (T + fc - 1) / fc;
        for (int r = 0; r < rounds; ++r) {
            if constexpr (W4) {
                // wave 0 requests a later round, applies its share of this one,
                // then waits for the next round's copies
                if (token_wave) {
                    // buffer (r + 1) % 2 was last read by round r - 1 (the
                    // ring's round 1 was requested with round 0)
                    if (r >= (RING ? 1 : 0) && r + 1 < rounds) issue(r + 1);
                }
                apply(r);
                // no later round is in flight: the wait is for everything
                if (token_wave && r + 1 < rounds) wait_lds_copies();
            } else if (token_wave) {
                if constexpr (RING) {
                    // buffer (r + 2) % 3 was last read by round r - 1
                    if (r + 2 < rounds) issue(r + 2);
                    if (r + 1 < rounds) ring_wait(r + 1);
                } else {
                    if (r + 1 < rounds) stage(r + 1);
                }
            } else {
                apply(r);
            }
            if constexpr (RING || GW) ring_barrier();
            else __syncthreads();
        }
        if (tree && token_wave) move_kept();  // every round is staged
    }
    float* dst = materialize ? P.states_out + (static_cast<size_t>(b) * P.H + h) * DK * DV
                             : P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
    if constexpr (!MF) {
        if (state_wave) {
#pragma unroll
            for (int j = 0; j < RPT; ++j)
                __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(dst + (rg * RPT + j) * DV + c0));
        }
    } else {
        // Matrix-core folds: the update is held in the accumulator layout, in
        // which one instruction covers 64-byte pieces of 16 rows; read and
        // written that way the state streams at about four fifths of the rate of
        // whole rows (measured).  So the state is read here in whole rows -- one
        // instruction covers two rows of 512 bytes -- and the update is turned
        // into the same layout through LDS (the staging area, free once every
        // wave has applied the last round), in two passes of 64 rows.  Wave mw
        // ends with the rows strip(p) .. strip(p) + 15 of pass p, lane l holding
        // columns 4 (l % 32) .. + 3 of row strip(p) + 2 i + l / 32 in vector i.
        // The 16-byte piece c of LDS row R sits at slot c ^ (R % 16), so that
        // the 16 rows of an accumulator block fall in distinct banks.
        if constexpr (!MULTI) ring_barrier();  // (a multi-round fold ended its last round with one)
        // lane indices from an opaque copy of the thread index: the
        // addresses below are formed here, not hoisted above the rounds and
        // held (or spilled) across them
        int et = tid;
        asm volatile("" : "+v"(et));
        const int mw = et >> 6, ml = et & 63;
        const int half = ml >> 5, cc = ml & 31;
        auto strip = [&](int p) { return COLS ? 64 * p + 16 * mw : 32 * mw + 16 * p; };
        char* conv = reinterpret_cast<char*>(stage0);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(tile), 0, has_state ? DK * DV * static_cast<int>(sizeof(float)) : 0, kBufferFlags);
        // the state rows of pass p; every wave issues them, the token wave's
        // past the end of the resource (the range check drops them: they
        // read zeros and touch no memory), so that the registers that receive
        // them are not held across a branch
        const int past = state_wave ? 0 : DK * DV * static_cast<int>(sizeof(float));
        auto load_rows = [&](int p, f4 (&st)[8]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = strip(p) + 2 * i + half;
                st[i] = __builtin_bit_cast(
                    f4, __builtin_amdgcn_raw_buffer_load_b128(rs, past + (row * DV + 4 * cc) * 4, 0, kCachePolicyNT));
            }
        };
        // accumulator vectors 8p .. 8p + 7 into LDS: rows 16 (jj / 2) + l % 16
        // of the pass, columns 32 mw + 16 (jj % 2) + 4 (l / 16) (COLS), or
        // rows strip(p) + l % 16, columns 16 jj + 4 (l / 16)
        auto put = [&](int p) {
            const int r = ml & 15, G = ml >> 4;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int R = COLS ? 16 * (jj >> 1) + r : 16 * mw + r;
                const int c = COLS ? 8 * mw + 4 * (jj & 1) + G : 4 * jj + G;
                *reinterpret_cast<f4*>(conv + R * 512 + ((c ^ r) << 4)) = s[8 * p + jj];
            }
        };
        const float e0 = CH ? 1.0f : *e0p;
        auto finish = [&](int p, const f4 (&st)[8]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int rr = 2 * i + half;
                const f4 d = *reinterpret_cast<const f4*>(conv + (16 * mw + rr) * 512 + ((cc ^ rr) << 4));
                const int row = strip(p) + rr;
                const float e = CH ? exp_gate(e0p[row]) : e0;
                __builtin_nontemporal_store(st[i] * e + d, reinterpret_cast<f4*>(dst + row * DV + 4 * cc));
                if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // four rows at a time (registers)
            }
        };
        // COLS: a pass reads rows that other waves' columns make up;
        // otherwise each wave reads back only its own rows
        auto sync = [&]() {
            if constexpr (COLS) ring_barrier();
            else __builtin_amdgcn_s_waitcnt(0xC07F);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        };
        // the state loads are issued once the first pass's accumulators are
        // in LDS (their registers are free then)
        f4 st0[8], st1[8];
        if (state_wave) put(0);
        __builtin_amdgcn_sched_barrier(0);
        load_rows(0, st0);
        load_rows(1, st1);
        // Both passes' rows are waited for before the first store, by every
        // wave (the token wave's are the dropped ones): stores and loads share
        // the counter, and a count taken behind the first pass's stores would
        // make the second pass wait for them too.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        sync();
        if (state_wave) finish(0, st0);
        sync();  // the second pass overwrites what the first read
        if (state_wave) put(1);
        sync();
        if (state_wave) finish(1, st1);
    }
    if (token_wave) meta();
}

// One workgroup per tile (W4: of four waves).
template <int RULE, int DK, int DV, typename IO, bool MULTI, bool TREE, bool MFT, bool W4 = false>
__global__ __launch_bounds__((W4 ? Geo<DK, DV>::NT : Geo<DK, DV>::NTHREADS))
__attribute__((amdgpu_waves_per_eu((W4 && TREE && !MFT) ? 5 : ((RULE == KVBUF_RULE_DELTA && MULTI) || W4 ? 4 : 1))))
void fold_kernel(TileParams P) {
    const TileIndex ti = tile_index(P);
    fold_tile<RULE, DK, DV, IO, MULTI, TREE, MFT, W4>(P, ti.b, ti.h, threadIdx.x);
}

// The flush that follows a decode launch whose eager fold does not fit the
// decode kernel: at any step only the tiles whose buffer just filled have
// work.  A workgroup takes kSparseTiles consecutive tiles, reads their slots
// and occupancies in one round trip, and runs the flush of a tile only if it
// is full (or its metadata is out of range, to report it); the flush of any
// other tile changes nothing.  Launching a workgroup per tile instead costs a
// dispatch, a metadata round trip and a barrier for every tile at every step.
constexpr int kSparseTiles = 8;
template <int RULE, int DK, int DV, typename IO, bool MULTI, bool MFT>
__global__ __launch_bounds__((Geo<DK, DV>::NTHREADS))
__attribute__((amdgpu_waves_per_eu(MULTI ? 4 : 1))) void fold_sparse_kernel(TileParams P) {
    constexpr int NT = Geo<DK, DV>::NT;
    __shared__ uint32_t s_mask;
    const int ntiles = P.batch * P.H;
    const int first = blockIdx.x * kSparseTiles;
    if (threadIdx.x >= NT) {
        const int lane = threadIdx.x - NT;
        const int t = first + lane;
        bool need = false;
        if (lane < kSparseTiles && t < ntiles) {
            const int h = t / P.batch;
            const int b = t - h * P.batch;
            const int slot = P.slot[b];
            const int p = load_occupancy(P, b, h);
            const int cap = P.block_size * P.blocks_per_req;
            need = p < 0 || p > cap || slot >= P.num_slots || (slot >= 0 && p >= P.m);
        }
        const uint64_t m = __ballot(need);
        if (lane == 0) s_mask = static_cast<uint32_t>(m);
    }
    __syncthreads();
    uint32_t mask = s_mask;
    bool later = false;
    while (mask != 0u) {
        const int k = __builtin_ctz(mask);
        mask &= mask - 1u;
        if (later) __syncthreads();  // the previous tile's LDS has been consumed
        later = true;
        const int t = first + k;
        const int h = t / P.batch;
        // the thread index is made opaque to the compiler in each
        // iteration, so that it does not keep every lane-derived value of the
        // tile code live across the loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        fold_tile<RULE, DK, DV, IO, MULTI, false, MFT>(P, t - h * P.batch, h, tid);
    }
}

template <int RULE, int D, typename IO>
hipError_t launch_fold_t(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    const int cap = p.block_size * p.blocks_per_req;
    const int most = p.mode == MODE_MATERIALIZE ? cap : p.m;  // most positions one tile applies
    const dim3 grid(static_cast<unsigned>(batch) * p.H), block(G::NTHREADS);
    const bool tree = p.leaf != nullptr;
    const bool mf = most > 16;
    // the matrix-core instances (d = 128) stage pool rows as stored, except
    // under the per-channel rule
    constexpr bool CH = RULE == KVBUF_RULE_CHANNEL;
    const bool raw = mf && D == 128 && !CH;
    const int kb = raw ? static_cast<int>(sizeof(IO)) : 4;
    const int xb = raw && RULE != KVBUF_RULE_DELTA ? static_cast<int>(sizeof(IO)) : 4;
    TileParams q = p;
    q.fold_chunk = std::min(most, raw ? kRawFoldChunk : kFoldChunk);
    // multi-round folds always exceed 16 positions (the chunk is at least 16 then)
    const bool multi = most > q.fold_chunk;
    const bool tr = raw && multi && kb == 2;  // staged in whole chunks of 32 rows
    // rows staged as stored (d = 128, not per-channel): four-wave workgroups,
    // whose rings keep two staging buffers
    const bool w4 = raw && D == 128 && !q.sparse;
    const bool ring = raw && multi && xb == 2;
    const int nbuf = ring && !w4 ? kFoldRing : 2;
    const size_t lds = sizeof(float) * fold_lds_floats(D, D, cap,
                                                       fold_stage_area(fold_stage_floats(D, D, tr ? 32 : q.fold_chunk,
                                                                                         kb, xb, raw),
                                                                       nbuf, mf && D == 128),
                                                       CH);
    const dim3 block4(G::NT);
    if (q.sparse) {  // a flush after a decode launch (never a tree commit)
        const dim3 sgrid((static_cast<unsigned>(batch) * q.H + kSparseTiles - 1) / kSparseTiles);
        if (multi) fold_sparse_kernel<RULE, D, D, IO, true, true><<<sgrid, block, lds, s>>>(q);
        else if (mf) fold_sparse_kernel<RULE, D, D, IO, false, true><<<sgrid, block, lds, s>>>(q);
        else fold_sparse_kernel<RULE, D, D, IO, false, false><<<sgrid, block, lds, s>>>(q);
        return hipGetLastError();
    }
    constexpr bool W4_OK = D == 128 && !CH;  // instances with a four-wave form
    if (multi) {
        if (w4) {
            if constexpr (W4_OK) {
                if (tree) fold_kernel<RULE, D, D, IO, true, true, true, true><<<grid, block4, lds, s>>>(q);
                else fold_kernel<RULE, D, D, IO, true, false, true, true><<<grid, block4, lds, s>>>(q);
            }
        } else if (tree) fold_kernel<RULE, D, D, IO, true, true, true><<<grid, block, lds, s>>>(q);
        else fold_kernel<RULE, D, D, IO, true, false, true><<<grid, block, lds, s>>>(q);
    } else if (mf) {
        if (w4) {
            if constexpr (W4_OK) {
                if (tree) fold_kernel<RULE, D, D, IO, false, true, true, true><<<grid, block4, lds, s>>>(q);
                else fold_kernel<RULE, D, D, IO, false, false, true, true><<<grid, block4, lds, s>>>(q);
            }
        } else if (tree) fold_kernel<RULE, D, D, IO, false, true, true><<<grid, block, lds, s>>>(q);
        else fold_kernel<RULE, D, D, IO, false, false, true><<<grid, block, lds, s>>>(q);
    } else {
        // vector-ALU folds (at most 16 positions, one round) of d = 128: a
        // commit runs four waves (most of its tiles only advance their
        // metadata, and more workgroups per CU hide that chain: 66 -> 62 us at
        // eight drafts); a flush, whose every tile streams its state, stays on
        // five (four measured 3% slower)
        if (D == 128 && !CH && q.mode == MODE_COMMIT) {
            if constexpr (W4_OK) {
                if (tree) fold_kernel<RULE, D, D, IO, false, true, false, true><<<grid, block4, lds, s>>>(q);
                else fold_kernel<RULE, D, D, IO, false, false, false, true><<<grid, block4, lds, s>>>(q);
            }
        } else if (tree) fold_kernel<RULE, D, D, IO, false, true, false><<<grid, block, lds, s>>>(q);
        else fold_kernel<RULE, D, D, IO, false, false, false><<<grid, block, lds, s>>>(q);
    }
    return hipGetLastError();
}

template <int RULE, typename IO>
hipError_t launch_fold_d(const TileParams& p, int d, int batch, hipStream_t s) {
    switch (d) {
        case 16: return launch_fold_t<RULE, 16, IO>(p, batch, s);
        case 64: return launch_fold_t<RULE, 64, IO>(p, batch, s);
        default: return launch_fold_t<RULE, 128, IO>(p, batch, s);
    }
}

template <typename IO>
hipError_t launch_fold_r(const TileParams& p, int rule, int d, int batch, hipStream_t s) {
    switch (rule) {
        case KVBUF_RULE_LINEAR: return launch_fold_d<KVBUF_RULE_LINEAR, IO>(p, d, batch, s);
        case KVBUF_RULE_GATED: return launch_fold_d<KVBUF_RULE_GATED, IO>(p, d, batch, s);
        case KVBUF_RULE_CHANNEL: return launch_fold_d<KVBUF_RULE_CHANNEL, IO>(p, d, batch, s);
        default: return launch_fold_d<KVBUF_RULE_DELTA, IO>(p, d, batch, s);
    }
}

}  // namespace

hipError_t launch_fold(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s) {
    return io == KVBUF_BF16 ? launch_fold_r<bf16_bits>(p, rule, d, batch, s)
                            : launch_fold_r<float>(p, rule, d, batch, s);
}

}  // namespace kvbuf
